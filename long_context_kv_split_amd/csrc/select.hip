// Static draft-KV selection on gfx950: StreamingLLM window and SnapKV.
//
// MagicDec (deep notes on papercache.org, §4.4, §5.2, Appendix A.1) drafts
// with a static compressed KV cache built once at prefill, chosen by
// StreamingLLM (sink + recent tokens) or SnapKV (observation-window attention
// votes). SnapKV runs in three kernels:
//   1. snap_stats:  per (sequence, KV head, chunk of keys) the online max and
//      sum of exp2 of every window row's scaled scores (causal over the last
//      W keys), S^T = K Q^T on 16x16x32 bf16 MFMA, persistent waves over
//      (sequence, KV head, 16-key step) with K streamed through an LDS ring;
//   2. snap_votes:  merge the chunk statistics into each row's log2
//      normaliser, recompute the scores of the prefix keys as S = Q K^T (each
//      lane holds four window rows of one key), normalise, and sum over the
//      rows in-lane and across the four lane groups; votes are staged in LDS
//      and stored 512 keys at a time;
//   3. snap_topk:   one 1024-thread block per (sequence, KV head): clipped
//      max-pool of the votes into registers, the (budget - W)-th largest
//      pooled value found bit by bit from the top (non-negative floats order
//      as their bit patterns; each bit is one ballot count over the block;
//      the low bits are searched only among the keys in the threshold's
//      band, gathered in LDS), then an order-preserving write of every value
//      above that threshold
//      and of the lowest positions among the ties, from one block scan of
//      per-wave counts; the window positions are appended (ascending).
//      Prefixes longer than 64 Ki keys and pool kernels wider than 129 use a
//      variant that keeps the pooled values in the workspace and selects with
//      a 4-pass 8-bit radix.
//
// Top-K attention (the dynamic draft of §4.4: per query head, the budget
// positions with the largest q.k, searched again at every draft step) reuses
// the pieces in four kernels: topk_tau scores a sample of 1024 positions per
// row and takes a threshold that the budget-th largest key exceeds except
// with negligible probability; topk_scores streams K like the SnapKV passes
// and writes only the keys at or above it (order-preserving 32-bit keys with
// their positions, staged in LDS); topk_rows_small selects the budget largest
// candidates of a row in registers with the same bit-by-bit search (from bit
// 31); topk_rows_full takes the rows it could not (too many candidates, or
// too few when the threshold was too high: then it recomputes the whole row),
// so the sample changes the speed and never the result.
#include "sd_device.h"
#include "sd_host.h"
#include "sd_sched.h"

#include <algorithm>

using namespace sdk;

namespace {

constexpr int kStepTokens = 16;
constexpr int kTopkThreads = 1024;
constexpr int kMaxPoolHalf = 64;  // register top-K: pool kernels up to 129
// Register top-K: after the bits from 22 up (sign, exponent and the top
// mantissa bit of the pooled votes) the search goes on among the keys that
// share them with the threshold: about 1000 of 32736 at the 32k-context
// workload; up to kBandCap of them are gathered in LDS.
constexpr int kBandCut = 22;
constexpr int kBandCap = 2048;

// ---------------------------------------------------------------- StreamingLLM
__global__ __launch_bounds__(256) void streaming_select_kernel(const int32_t *kv_lens, int sink,
                                                               int recent, int32_t *idx,
                                                               int32_t *sel_lens) {
  const int b = blockIdx.x;
  const int L = max(0, kv_lens[b]);
  const int n_sink = min(sink, L);
  const int start_recent = max(sink, L - recent);
  const int n_recent = max(0, L - start_recent);
  const int n = n_sink + n_recent;
  const int cap = sink + recent;
  for (int t = threadIdx.x; t < cap; t += blockDim.x) {
    int v = -1;
    if (t < n_sink)
      v = t;
    else if (t < n)
      v = start_recent + (t - n_sink);
    idx[(size_t)b * cap + t] = v;
  }
  if (threadIdx.x == 0) sel_lens[b] = n;
}

// ---------------------------------------------------------------- SnapKV
struct SnapParams {
  const void *k_pages;
  const int32_t *page_table;
  const int32_t *kv_lens;
  const void *q_obs;  // [B, W, Hq, D]
  Sched sc;           // persistent schedule over (sequence, KV head, 16-key step)
  float *stats;       // [slots, rows, 2]  per-segment (m, l), log2 domain
  float *votes;       // [B*Hkv, vote_stride]
  float *pooled;      // [B*Hkv, vote_stride]
  int32_t *idx;       // [B, Hkv, budget]
  int32_t *sel_lens;  // [B]
  int32_t W, Hq, Hkv, G, rows;
  int32_t num_pages, page_size, max_pages;
  int32_t len_cap, vote_stride;
  int32_t pool_kernel, budget;  // budget: the largest budget and the width of an idx row
  const int32_t *budgets;       // [B] per-sequence budgets, or null (every sequence uses `budget`)
  const float *obs_lse;         // [B, W, Hq] window normalisers (natural log) given by the caller, or null
  float *lse_out;               // [B, W, Hq] window normalisers written by snap_lse_kernel
  float scale_log2;
  // top-K attention
  uint32_t *keys;      // [B*Hq, key_stride] candidate order keys of q.k (per scoring segment)
  int32_t *cand_pos;   // [B*Hq, key_stride] their positions
  uint32_t *tau;       // [B*Hq] candidate threshold per row
  int32_t *counts;     // [slots, G] candidates per scoring segment and head
  int32_t *deferred;   // [1 + B*Hq]: count, then the rows left to the full selection kernel
  int32_t key_stride;  // a multiple of 16
  int32_t head_dim;
};

constexpr int kRing = 4;       // 16-key K steps per wave in LDS: 3 loading while one is scored
constexpr int kWinSteps = 64;  // steps per row-id window (lane i holds the first row of step i)
constexpr int kStageSteps = 32;  // votes staged in LDS and stored every 32 steps
typedef __attribute__((ext_vector_type(2))) float f32x2;
constexpr float kHeadroom = 8.f;  // log2 slack of the lazily moved row max in the stats pass

// Two 16-byte LDS reads at byte_off and byte_off + gap (gap an immediate
// offset), untracked by the compiler like the word accesses below; they
// return with their data.
template <int GAP>
__device__ __forceinline__ void lds_read_b128_pair_t(const char *lds, int byte_off, u32x4 &lo, u32x4 &hi) {
  const uint32_t addr = (uint32_t)(size_t)((const __attribute__((address_space(3))) char *)lds + byte_off);
#if __HIP_DEVICE_COMPILE__
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:%3\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(lo), "=&v"(hi)
               : "v"(addr), "n"(GAP)
               : "memory");
#endif
}

// LDS word access the compiler does not track (so it adds no wait for the
// asynchronous ring loads); the read returns with its data.
__device__ __forceinline__ void lds_write_f32(const char *lds, int byte_off, float v) {
  const uint32_t addr = (uint32_t)(size_t)((const __attribute__((address_space(3))) char *)lds + byte_off);
#if __HIP_DEVICE_COMPILE__
  asm volatile("ds_write_b32 %0, %1" ::"v"(addr), "v"(v) : "memory");
#endif
}

// Budget of sequence b (device-side per-sequence values are clamped into
// [W + 1, budget]).
__device__ __forceinline__ int seq_budget(const SnapParams &a, int b) {
  return a.budgets ? clampi(a.budgets[b], a.W + 1, a.budget) : a.budget;
}

// Keys scored for sequence b: every cached key when the sequence is longer
// than its budget (shorter ones keep everything and are not scored).
__device__ __forceinline__ int snap_steps(const SnapParams &a, int b) {
  const int L = clampi(a.kv_lens[b], 0, a.len_cap);
  return L > seq_budget(a, b) ? (L + kStepTokens - 1) / kStepTokens : 0;
}

__global__ __launch_bounds__(kPlanThreads) void snap_plan_kernel(SnapParams a) {
  sched_plan(a.sc, [&](int b) { return snap_steps(a, b); });
}

// K of one unit's consecutive 16-key steps streamed through a per-wave LDS
// ring by asynchronous global->LDS loads, so loads in flight hold no
// registers. Step s lands in slot s % kRing as 16 token rows; 16-byte chunk j
// of token t is stored at chunk position j ^ (t mod chunks-per-row), so the
// MFMA operand reads (16 tokens x one chunk) fall in distinct banks.
//
// Waits are explicit: every step issues the same number of loads (prefetches
// past the segment re-load its last step into a slot no longer read), so
// "at most (kRing-1)*kInsts newer operations outstanding" means the step has
// landed; any other memory operation only makes that wait stricter. The ring
// is read with inline ds_read blocks that end in their own lgkmcnt wait, which
// keeps the compiler from adding its own vmcnt(0) before LDS reads (it cannot
// tell which slot an asynchronous load writes).
//
// Row ids come in 64-step windows: lane i of rows_a / rows_b holds the first
// row of step wb + i / wb + 64 + i, and the page-table entries of the window
// after those are copied into LDS one window ahead, so sliding the window
// never waits on a load issued in the same iteration.
template <int D>
struct KStream {
  static constexpr int kRowChunks = D * 2 / 16;  // 16-byte chunks per token row
  static constexpr int kStepChunks = kStepTokens * kRowChunks;
  static constexpr int kInsts = kStepChunks / 64;  // loads per lane and step
  static constexpr int kLdsBytes = kRing * kStepChunks * 16 + kWinSteps * 4;
  lds_u32x4 *ring;                                 // [kRing][kStepChunks]
  __attribute__((address_space(3))) int32_t *entries;  // [kWinSteps] page-table entries
  const char *kp;
  const int32_t *pt;  // page-table row of the sequence
  int Hkv, kvh, P, num_pages, last;
  int lane_off[kInsts];  // byte offset of this lane's chunk inside a step
  int wb, rows_a, rows_b;
  int s0 = 0;       // first position of the segment
  StepWalk walk;    // positions s0 + v, v < walk.n, read step s0 + walk(v)

  __device__ KStream(const SnapParams &a, int b, int kvh_, int last_step, char *lds)
      : ring((lds_u32x4 *)(__attribute__((address_space(3))) char *)lds),
        entries((__attribute__((address_space(3))) int32_t *)(
            (__attribute__((address_space(3))) char *)lds + kRing * kStepChunks * 16)),
        kp(reinterpret_cast<const char *>(a.k_pages)), pt(a.page_table + (size_t)b * a.max_pages),
        Hkv(a.Hkv), kvh(kvh_), P(a.page_size), num_pages(a.num_pages), last(last_step) {
#pragma unroll
    for (int c = 0; c < kInsts; ++c) {
      const int idx = c * 64 + lane_id();
      const int t = idx / kRowChunks, p = idx % kRowChunks;
      lane_off[c] = (t * kRowChunks + (p ^ (t & (kRowChunks - 1)))) * 16;
    }
  }
  // Step read at position s (the identity unless permute() was called).
  __device__ int step_at(int s) const { return s0 + walk(min(s, last) - s0); }
  __device__ const int32_t *entry_ptr(int s) const { return pt + step_at(s) * kStepTokens / P; }
  // First token row of the step at position s (16 keys never straddle a
  // page: P % 16 == 0).
  __device__ int row_from(int entry, int s) const {
    const int pos = step_at(s) * kStepTokens;
    return (clampi(entry, 0, num_pages - 1) * Hkv + kvh) * P + pos % P;
  }
  // Read positions s_begin .. s_begin + n - 1 in a permuted order (before
  // begin(s_begin); for passes whose result does not depend on the order).
  __device__ void permute(int n, uint32_t hash) { walk = StepWalk(n >= kWalkMinSteps ? n : 0, hash); }
  // Copy the page-table entries of window steps w0 + lane into LDS.
  __device__ void fetch_entries(int w0) {
    lds_dma4(entry_ptr(w0 + lane_id()), entries);
  }
  __device__ int read_entry() const {
    int e = 0;
    const uint32_t addr = (uint32_t)(size_t)(entries + lane_id());
#if __HIP_DEVICE_COMPILE__  // VGPR asm constraints exist only for the device target
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(e) : "v"(addr) : "memory");
#endif
    return e;
  }
  __device__ void issue(int s, int slot) {
    const int d = s - wb;
    const int row = d < kWinSteps ? __builtin_amdgcn_readlane(rows_a, d)
                                  : __builtin_amdgcn_readlane(rows_b, d - kWinSteps);
    const char *src = kp + (size_t)row * D * 2;
#pragma unroll
    for (int c = 0; c < kInsts; ++c)
      lds_dma16(src + lane_off[c], ring + slot * kStepChunks + c * 64);
  }
  __device__ void begin(int s_begin) {
    const int lane = lane_id();
    s0 = s_begin;
    wb = s_begin;
    rows_a = row_from(*entry_ptr(wb + lane), wb + lane);
    rows_b = row_from(*entry_ptr(wb + kWinSteps + lane), wb + kWinSteps + lane);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // entries LDS of a previous segment is free
    fetch_entries(wb + 2 * kWinSteps);
#pragma unroll
    for (int i = 0; i < kRing - 1; ++i) issue(min(s_begin + i, last), (s_begin + i) % kRing);
  }
  // Before scoring step s: slide the row window, start loading step
  // s + kRing - 1 into the slot step s - 1 used, and wait for step s.
  __device__ void advance(int s) {
    if (s - wb == kWinSteps) {
      const int lane = lane_id();
      wb += kWinSteps;
      rows_a = rows_b;
      // entries of this window were requested 64 steps ago: at least kRing-1
      // steps' loads were issued after them and waited for since
      rows_b = row_from(read_entry(), wb + kWinSteps + lane);
      fetch_entries(wb + 2 * kWinSteps);
    }
    issue(min(s + kRing - 1, last), (s + kRing - 1) % kRing);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kRing - 1) * kInsts) : "memory");
  }
  // MFMA A operand of step s: token r, head-dim chunk 4*kk + g.
  __device__ void operand(int s, u32x4 (&k)[D / 32]) const {
    const int lane = lane_id(), g = lane >> 4, r = lane & 15;
    const lds_u32x4 *rowp = ring + (s % kRing) * kStepChunks + r * kRowChunks;
    uint32_t ad[D / 32];
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) ad[kk] = (uint32_t)(size_t)(rowp + ((4 * kk + g) ^ (r & (kRowChunks - 1))));
#if __HIP_DEVICE_COMPILE__  // VGPR asm constraints exist only for the device target
    if constexpr (D == 128) {
      asm volatile(
          "ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3])
          : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
          : "memory");
    } else {
      static_assert(D == 64, "head_dim 64 or 128");
      asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                   : "=&v"(k[0]), "=&v"(k[1])
                   : "v"(ad[0]), "v"(ad[1])
                   : "memory");
    }
#endif
  }
  // Loads still writing LDS must land before the wave's LDS is released.
  __device__ static void drain() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
};

template <int D, int NB>
__device__ __forceinline__ void snap_load_q(const SnapParams &a, int b, int kvh, u32x4 (&q)[NB][D / 32]) {
  const int lane = lane_id();
  const int g = lane >> 4, r = lane & 15;
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
    const int R = rb * 16 + r;  // row R = w * G + hl
    const bool live = R < a.rows;
    const int w = live ? R / a.G : 0, hl = live ? R % a.G : 0;
    const char *qb = reinterpret_cast<const char *>(a.q_obs) +
                     ((((size_t)b * a.W + w) * a.Hq + (size_t)kvh * a.G + hl) * D) * 2;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (live) v = *reinterpret_cast<const u32x4 *>(qb + (32 * kk + 8 * g) * 2);
      q[rb][kk] = v;
    }
  }
}

template <int D, int NB>
__device__ __forceinline__ f32x4 snap_scores(const u32x4 (&k)[D / 32], const u32x4 (&q)[NB][D / 32], int rb) {
  f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) sc = mfma_16x16x32_bf16(k[kk], q[rb][kk], sc);
  return sc;
}

__device__ __forceinline__ void merge_ml(float &m, float &l, float m2, float l2) {
  const float M = fmaxf(m, m2);
  if (M == kNegInf) return;
  l = (m == kNegInf ? 0.f : l * __builtin_amdgcn_exp2f(m - M)) +
      (m2 == kNegInf ? 0.f : l2 * __builtin_amdgcn_exp2f(m2 - M));
  m = M;
}

// (m, l) merged over the four 16-lane rows (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ void rows4_merge(float &m, float &l) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(l), __float_as_uint(l), false, false);
  m = __uint_as_float(a[0]);
  l = __uint_as_float(b[0]);
  merge_ml(m, l, __uint_as_float(a[1]), __uint_as_float(b[1]));
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  auto d = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l), false, false);
  m = __uint_as_float(c[0]);
  l = __uint_as_float(d[0]);
  merge_ml(m, l, __uint_as_float(c[1]), __uint_as_float(d[1]));
}

// Pass 1: per segment of a unit, each window row's (max, sum of exp2) of its
// scaled scores over the segment's keys, causal over the last W keys.
template <int D, int NB>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void snap_stats_kernel(SnapParams a) {
  __shared__ __attribute__((aligned(16))) char lds[KStream<D>::kLdsBytes];
  const int lane = lane_id();
  const int g = lane >> 4, r = lane & 15;
  sched_for_each_segment(a.sc, blockIdx.x, [&](int b, int kvh, int s_begin, int s_end, size_t slot) {
    s_begin = __builtin_amdgcn_readfirstlane(s_begin);
    s_end = __builtin_amdgcn_readfirstlane(s_end);
    const int L = __builtin_amdgcn_readfirstlane(clampi(a.kv_lens[b], 0, a.len_cap));
    u32x4 q[NB][D / 32];
    snap_load_q<D, NB>(a, b, kvh, q);
    float m[NB], l[NB];
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) {
      m[rb] = kNegInf;
      l[rb] = 0.f;
    }
    const int lim_min = L - a.W;  // keys up to here are seen by every window row
    const float c = a.scale_log2;
    // Unmasked steps: the row max moves lazily. Exponents are taken against
    // the current m; only when some lane's exponent exceeds kHeadroom (sums of
    // up to 2^kHeadroom per key stay exact enough in fp32) does the wave rebase
    // those lanes on their exact running max, in a rare uniform branch.
    auto plain_step = [&](const u32x4 (&k)[D / 32]) {
#pragma unroll
      for (int rb = 0; rb < NB; ++rb) {
        const f32x4 sc = snap_scores<D, NB>(k, q, rb);
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = fmaf(sc[e], c, -m[rb]);
        const float xm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        if (__builtin_expect(__ballot(xm > kHeadroom) != 0, 0)) {
          if (xm > kHeadroom) {  // also the first key of a lane (m = -inf gives +inf)
            const float pm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])) * c;
            l[rb] = (m[rb] == kNegInf) ? 0.f : l[rb] * __builtin_amdgcn_exp2f(m[rb] - pm);
            m[rb] = pm;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = fmaf(sc[e], c, -pm);
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) l[rb] += __builtin_amdgcn_exp2f(x[e]);
      }
    };
    auto masked_step = [&](const u32x4 (&k)[D / 32], int s) {
      const int tok0 = s * kStepTokens;
#pragma unroll
      for (int rb = 0; rb < NB; ++rb) {
        const f32x4 sc = snap_scores<D, NB>(k, q, rb);
        float p[4];
        const int R = rb * 16 + r;
        const int lim = R < a.rows ? L - a.W + R / a.G : L - 1;  // last key row R sees
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = tok0 + 4 * g + e > lim ? kNegInf : sc[e] * c;
        const float pm = fmaxf(fmaxf(p[0], p[1]), fmaxf(p[2], p[3]));
        if (pm > m[rb]) {
          l[rb] = (m[rb] == kNegInf) ? 0.f : l[rb] * __builtin_amdgcn_exp2f(m[rb] - pm);
          m[rb] = pm;
        }
        if (m[rb] != kNegInf) {
#pragma unroll
          for (int e = 0; e < 4; ++e) l[rb] += __builtin_amdgcn_exp2f(p[e] - m[rb]);
        }
      }
    };
    const int first_masked = lim_min >= 0 ? (lim_min + 1) / kStepTokens : 0;
    const int plain_end = max(s_begin, min(s_end, first_masked));
    KStream<D> ks(a, b, kvh, s_end - 1, lds);
    ks.permute(plain_end - s_begin, segment_hash(b, kvh, s_begin));  // sums do not depend on the order
    ks.begin(s_begin);
    for (int s = s_begin; s < plain_end; ++s) {
      ks.advance(s);
      u32x4 k[D / 32];
      ks.operand(s, k);
      plain_step(k);
    }
    for (int s = plain_end; s < s_end; ++s) {
      ks.advance(s);
      u32x4 k[D / 32];
      ks.operand(s, k);
      masked_step(k, s);
    }
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) {
      float mm = m[rb], ll = l[rb];
      rows4_merge(mm, ll);
      const int R = rb * 16 + r;
      if (g == 0 && R < a.rows) {
        a.stats[(slot * a.rows + R) * 2 + 0] = mm;
        a.stats[(slot * a.rows + R) * 2 + 1] = ll;
      }
    }
  });
  KStream<D>::drain();
}

// Merge the pass-1 statistics of unit u over its segments: lane (g, r) ends
// with (max, sum) of row 16 rb + r in log2 units. The unit's slots (many when
// a few units are spread over all waves) are split among the four lanes of
// each row, lane group g taking slots s0 + g, s0 + g + 4, ..., with the loads
// of kMergeBatch slots per lane issued together (addresses clamped, values
// masked), then merged across the groups; every caller merges in the same
// order.
template <int NB>
__device__ __forceinline__ void snap_merge_unit(const SnapParams &a, int u, float (&mm)[NB], float (&ll)[NB]) {
  constexpr int kMergeBatch = 4;
  const int lane = lane_id();
  const int g = lane >> 4, r = lane & 15;
  const int s0 = a.sc.slot_base[u], n_slots = a.sc.slot_base[u + 1] - s0;
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
    mm[rb] = kNegInf;
    ll[rb] = 0.f;
  }
  for (int base = 0; base < n_slots; base += 4 * kMergeBatch) {
    f32x2 v[kMergeBatch][NB];
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      const int s = s0 + min(base + 4 * i + g, n_slots - 1);
#pragma unroll
      for (int rb = 0; rb < NB; ++rb) {
        const int R = min(rb * 16 + r, a.rows - 1);
        v[i][rb] = *reinterpret_cast<const f32x2 *>(a.stats + ((size_t)s * a.rows + R) * 2);
      }
    }
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      if (base + 4 * i + g < n_slots) {
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) merge_ml(mm[rb], ll[rb], v[i][rb].x, v[i][rb].y);
      }
    }
  }
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) rows4_merge(mm[rb], ll[rb]);
}

// The window normalisers alone: one wave per unit merges its pass-1
// statistics and writes lse[b, w, h] = ln 2 * (max + log2 sum) of row
// R = w * G + hl (h = kvh * G + hl), -inf for a row that sees no key.
template <int NB>
__global__ __launch_bounds__(64) void snap_lse_kernel(SnapParams a) {
  const int u = blockIdx.x;
  const int b = u / a.Hkv, kvh = u % a.Hkv;
  const int lane = lane_id();
  const int g = lane >> 4, r = lane & 15;
  float mm[NB], ll[NB];
  snap_merge_unit<NB>(a, u, mm, ll);
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
    const int R = rb * 16 + r;
    if (g == 0 && R < a.rows)
      a.lse_out[((size_t)b * a.W + R / a.G) * a.Hq + (size_t)kvh * a.G + R % a.G] =
          ll[rb] > 0.f ? (mm[rb] + __log2f(ll[rb])) * kLn2 : kNegInf;
  }
}

// Pass 2: votes of the prefix keys [0, L - W): merge the unit's pass-1
// statistics into each row's log2 normaliser, recompute the scores, and sum
// the normalised weights over the window rows of the group.
template <int D, int NB>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void snap_votes_kernel(SnapParams a) {
  // K stream, then the votes of up to kStageSteps steps (16 floats per step).
  // Stores share the in-order load counter with the K stream, so a store
  // stalls the stream until it is acknowledged: votes leave in batches of
  // 512 keys (8 stores) every kStageSteps steps.
  constexpr int kStageOff = KStream<D>::kLdsBytes;
  __shared__ __attribute__((aligned(16))) char lds[kStageOff + kStageSteps * kStepTokens * 4];
  const int lane = lane_id();
  const int g = lane >> 4, r = lane & 15;
  sched_for_each_segment(a.sc, blockIdx.x, [&](int b, int kvh, int s_begin, int s_end_all, size_t) {
    s_begin = __builtin_amdgcn_readfirstlane(s_begin);
    const int L = __builtin_amdgcn_readfirstlane(clampi(a.kv_lens[b], 0, a.len_cap));
    const int npre = L - a.W;
    const int s_end = __builtin_amdgcn_readfirstlane(min(s_end_all, (npre + kStepTokens - 1) / kStepTokens));
    if (s_begin >= s_end) return;
    const int u = b * a.Hkv + kvh;
    // Scores are computed as S = Q K^T (window rows on M, keys on N): lane
    // (g, r) holds rows 16*rb + 4g + e of key r, so a key's vote is an in-lane
    // sum over (rb, e) plus a sum over the four lane groups. off[rb][e]: max +
    // log2(sum) of that row (+inf for padding rows: p = 0).
    float off[NB][4];
    if (a.obs_lse != nullptr) {
      // normalisers given: row R = w * G + hl is (b, w, kvh * G + hl) of obs_lse
#pragma unroll
      for (int rb = 0; rb < NB; ++rb) {
        const int R = rb * 16 + r;
        float o = __builtin_inff();
        if (R < a.rows) {
          const float x = a.obs_lse[((size_t)b * a.W + R / a.G) * a.Hq + (size_t)kvh * a.G + R % a.G];
          if (x > kNegInf) o = x * kLog2e;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) off[rb][e] = __shfl(o, 4 * g + e, 64);
      }
    } else {
      float mm[NB], ll[NB];
      snap_merge_unit<NB>(a, u, mm, ll);
#pragma unroll
      for (int rb = 0; rb < NB; ++rb) {
        const bool live = rb * 16 + r < a.rows;
        const float o = (live && ll[rb] > 0.f) ? mm[rb] + __log2f(ll[rb]) : __builtin_inff();  // row 16 rb + r
#pragma unroll
        for (int e = 0; e < 4; ++e) off[rb][e] = __shfl(o, 4 * g + e, 64);
      }
    }
    u32x4 q[NB][D / 32];
    snap_load_q<D, NB>(a, b, kvh, q);
    const float c = a.scale_log2;
    float *vrow = a.votes + (size_t)u * a.vote_stride;
    const int t_hi = min(s_end * kStepTokens, npre);
    KStream<D> ks(a, b, kvh, s_end - 1, lds);
    ks.begin(s_begin);
    // Staged steps [w0, s] of the current batch to global memory.
    // Lane l stores staged votes 4l..4l+3 and 256+4l..256+4l+3 of the batch
    // as 16-byte stores (the row stride is a multiple of 4 floats). The
    // nontemporal policy streams them past the caches: with plain stores the
    // pass measured about 5% slower.
    auto flush = [&](int w0, int s) {
      const int n = (s - w0 + 1) * kStepTokens;
      u32x4 v[2];
      lds_read_b128_pair_t<1024>(lds, kStageOff + 16 * lane, v[0], v[1]);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int j = 256 * c + 4 * lane;
        const int tok = w0 * kStepTokens + j;
        if (j + 3 < n && tok + 3 < t_hi) {
          __builtin_nontemporal_store(v[c], reinterpret_cast<u32x4 *>(vrow + tok));
        } else {
          const uint32_t e4[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (j + e < n && tok + e < t_hi) vrow[tok + e] = __uint_as_float(e4[e]);
        }
      }
    };
    for (int s = s_begin; s < s_end; ++s) {
      ks.advance(s);
      u32x4 k[D / 32];
      ks.operand(s, k);
      float acc = 0.f;
#pragma unroll
      for (int rb = 0; rb < NB; ++rb) {
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) sc = mfma_16x16x32_bf16(q[rb][kk], k[kk], sc);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc += __builtin_amdgcn_exp2f(fmaf(sc[e], c, -off[rb][e]));
      }
      // sum over the four lane groups: every lane (g, r) ends with key r's vote
      auto a16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc), __float_as_uint(acc), false, false);
      const float acc2 = __uint_as_float(a16[0]) + __uint_as_float(a16[1]);
      auto a32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc2), __float_as_uint(acc2), false, false);
      const float w = __uint_as_float(a32[0]) + __uint_as_float(a32[1]);
      const int k_in = (s - s_begin) % kStageSteps;
      if (g == 0) lds_write_f32(lds, kStageOff + (k_in * kStepTokens + r) * 4, w);
      if (k_in == kStageSteps - 1 || s == s_end - 1) flush(s - k_in, s);
    }
  });
  KStream<D>::drain();
}

// Block-wide exclusive scan of one uint32 per thread (1024 threads); returns the
// exclusive prefix and writes the block total to *total.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *lds_waves,
                                                         uint32_t *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) lds_waves[wave] = x;
  __syncthreads();
  if (wave == 0) {
    uint32_t w = lane < kTopkThreads / 64 ? lds_waves[lane] : 0u;
    uint32_t ws = w;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const uint32_t y = __shfl_up(ws, o, 64);
      if (lane >= o) ws += y;
    }
    if (lane < kTopkThreads / 64) lds_waves[16 + lane] = ws - w;  // exclusive wave offsets
    if (lane == kTopkThreads / 64 - 1) lds_waves[32] = ws;
  }
  __syncthreads();
  const uint32_t res = lds_waves[16 + wave] + x - v;
  *total = lds_waves[32];
  __syncthreads();
  return res;
}

// Sum over the wave (lane 0 holds the total): DPP within rows of 16, then
// the row totals.
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false);
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
         __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

// Block-wide exclusive scan of one uint64 per thread (WAVES waves).
template <int WAVES>
__device__ __forceinline__ uint64_t block_exclusive_scan_u64(uint64_t v, uint64_t *lds_waves) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) lds_waves[wave] = x;
  __syncthreads();
  uint64_t before = 0;
#pragma unroll
  for (int w = 0; w < WAVES; ++w)
    if (w < wave) before += lds_waves[w];
  __syncthreads();
  return before + x - v;
}

// Top-K of the pooled votes with the pooled values held in registers: thread
// t of THREADS holds positions t + THREADS*i, i < VPT, so (i, wave, lane)
// order is position order. The threshold key T is the largest key with at
// least `keep` keys >= T, built greedily from the top bit down, one block
// count per bit (counting several candidate bits per barrier measured slower:
// the compares, not the barriers, dominate). The output slot of a kept position is (#keys > T before it) +
// min(#keys == T before it, need), need = keep - #keys > T: every key above T
// and the lowest-position ties.
// Shared memory of the register top-K.
template <int THREADS, int VPT>
struct TopkLds {
  static constexpr int kWaves = THREADS / 64;
  static_assert(VPT * kWaves <= THREADS, "one scan entry per thread");
  uint32_t cnt[2][kWaves];
  uint64_t pre[VPT * kWaves];
  uint64_t scan_waves[kWaves];
};

// Keys whose bits above CUT equal those of the threshold found so far (the
// band the remaining bits are searched in), gathered in LDS: at most CAP.
template <int CAP>
struct TopkBand {
  uint32_t keys[CAP];
  uint32_t count;
};

// Writes out[0, keep) = the positions j < n with the `keep` largest keys, ties
// to the lower position, ascending; 0 < keep <= n. key[i] is the key of
// position threadIdx.x + THREADS * i and 0 past n (a zero is never counted
// above a candidate, which has a bit set); bits above TOP_BIT are clear. The keep-th largest key T is found bit by bit from the
// top (each bit one ballot count over the block); then every key above T and
// the lowest-positioned keys equal to T are written in position order from one
// block scan of per-wave counts.
struct PosIdentity {
  __device__ int operator()(int, int j) const { return j; }
};

// One bit of the threshold search: T | (1 << bit) is kept when at least `keep`
// keys are >= it, counting `extra` (the same on every thread) plus the block's
// keys in k[]. The count buffer of a bit is rewritten two bits later, after
// the next bit's barrier.
template <int THREADS, int N, int VPT>
__device__ __forceinline__ uint32_t search_bit(const uint32_t (&k)[N], int bit, uint32_t T, uint32_t extra,
                                               uint32_t keep, TopkLds<THREADS, VPT> &sm) {
  constexpr int kWaves = THREADS / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t cand = T | (1u << bit);
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) c += k[i] >= cand ? 1u : 0u;
  c = wave_sum_u32(c);
  if (lane == 0) sm.cnt[bit & 1][wave] = c;
  __syncthreads();
  uint32_t total = extra;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) total += sm.cnt[bit & 1][w];
  return total >= keep ? cand : T;
}

// pos(i, j): the value written for the key in register i of position j.
// With CUT > 0 the bits below CUT are searched only among the keys whose bits
// from CUT up equal the threshold's (gathered in `band` when they fit, else
// the search goes on over all keys): keys above that band are >= every
// remaining candidate and keys below it are < all of them, so the counts, and
// the threshold, are the same as over all keys.
template <int THREADS, int VPT, int TOP_BIT, class PosFn = PosIdentity, int CUT = 0, int CAP = 1>
__device__ __forceinline__ void select_top_keys(const uint32_t (&key)[VPT], int n, uint32_t keep, int32_t *out,
                                                TopkLds<THREADS, VPT> &sm, PosFn pos = PosFn(),
                                                TopkBand<CAP> *band = nullptr) {
  constexpr int kWaves = THREADS / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t T = 0;
  int bit = TOP_BIT;
  for (; bit >= CUT; --bit) T = search_bit<THREADS>(key, bit, T, 0u, keep, sm);
  if constexpr (CUT > 0) {
    static_assert(CAP % THREADS == 0, "band slots per thread");
    constexpr int kPer = CAP / THREADS;
    const uint32_t hi = T >> CUT;
    if (tid == 0) band->count = 0u;
    __syncthreads();
    // Band members: counted per wave, one LDS reservation per wave, then
    // placed by a second pass over the same ballots. Zero keys (every key
    // past n, and any zero value) are left out: a zero is never >= a
    // candidate, and never above the band.
    uint32_t above = 0, mine = 0;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      above += (key[i] >> CUT) > hi ? 1u : 0u;
      mine += ((key[i] >> CUT) == hi && key[i] != 0u) ? 1u : 0u;
    }
    const uint32_t wave_cnt = wave_sum_u32(mine);
    uint32_t base = 0u;
    if (lane == 0 && wave_cnt > 0u) base = atomicAdd(&band->count, wave_cnt);
    base = __builtin_amdgcn_readfirstlane(base);
    if (wave_cnt > 0u) {
      const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const bool in = (key[i] >> CUT) == hi && key[i] != 0u;
        const uint64_t m = __ballot(in);
        const uint32_t slot = base + (uint32_t)__popcll(m & below);
        if (in && slot < (uint32_t)CAP) band->keys[slot] = key[i];
        base += (uint32_t)__popcll(m);
      }
    }
    above = wave_sum_u32(above);
    if (lane == 0) sm.cnt[0][wave] = above;  // both count buffers are free here
    __syncthreads();
    uint32_t n_above = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) n_above += sm.cnt[0][w];
    const uint32_t n_band = band->count;
    __syncthreads();  // cnt[0] and the band are read before they are reused
    if (n_band <= (uint32_t)CAP) {
      uint32_t bk[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const uint32_t slot = (uint32_t)(tid + THREADS * j);
        bk[j] = slot < n_band ? band->keys[slot] : 0u;  // a zero is never >= a candidate
      }
      for (; bit >= 0; --bit) T = search_bit<THREADS>(bk, bit, T, n_above, keep, sm);
    } else {
      for (; bit >= 0; --bit) T = search_bit<THREADS>(key, bit, T, 0u, keep, sm);
    }
  }

  // Per (i, wave): keys above T (low word) and equal to T (high word).
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const bool valid = tid + THREADS * i < n;
    const uint64_t gm = __ballot(key[i] > T);  // a zero past n is never above T
    const uint64_t em = __ballot(valid && key[i] == T);
    if (lane == 0) sm.pre[i * kWaves + wave] = (uint64_t)__popcll(gm) | ((uint64_t)__popcll(em) << 32);
  }
  __syncthreads();
  const uint64_t mine = tid < VPT * kWaves ? sm.pre[tid] : 0ull;
  const uint64_t ex = block_exclusive_scan_u64<kWaves>(mine, sm.scan_waves);
  if (tid == THREADS - 1) sm.scan_waves[0] = ex + mine;  // totals
  if (tid < VPT * kWaves) sm.pre[tid] = ex;
  __syncthreads();
  const uint32_t need = keep - (uint32_t)sm.scan_waves[0];
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int j = tid + THREADS * i;
    const bool valid = j < n;
    const bool gt = key[i] > T, eq = valid && key[i] == T;
    const uint64_t gm = __ballot(gt);
    const uint64_t em = __ballot(eq);
    const uint64_t p = sm.pre[i * kWaves + wave];
    const uint32_t gt_before = (uint32_t)p + (uint32_t)__popcll(gm & below);
    const uint32_t eq_before = (uint32_t)(p >> 32) + (uint32_t)__popcll(em & below);
    if (gt)
      out[gt_before + min(eq_before, need)] = pos(i, j);
    else if (eq && eq_before < need)
      out[gt_before + eq_before] = pos(i, j);
  }
}

// Up to 32 values per thread the kernel fits 64 VGPRs, so two 1024-thread
// blocks share a CU and one block's count-and-barrier chain overlaps the
// other's compares (measured about 20% faster than one block per CU).
template <int THREADS, int VPT>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(VPT <= 32 ? 8 : 4))) void snap_topk_kernel(SnapParams a) {
  __shared__ TopkLds<THREADS, VPT> sm;
  __shared__ TopkBand<kBandCap> band;
  __shared__ float pool_lds[2][THREADS + 2 * kMaxPoolHalf];
  const int tid = threadIdx.x;
  const int kvh = blockIdx.x % a.Hkv, b = blockIdx.x / a.Hkv;
  const int L = clampi(a.kv_lens[b], 0, a.len_cap);
  int32_t *out = a.idx + ((size_t)b * a.Hkv + kvh) * a.budget;
  const int budget = seq_budget(a, b);
  if (kvh == 0 && tid == 0) a.sel_lens[b] = min(L, budget);
  if (L <= budget) {
    for (int t = tid; t < a.budget; t += THREADS) out[t] = t < L ? t : -1;
    return;
  }
  const int npre = L - a.W;  // <= THREADS * VPT and pool_kernel / 2 <= kMaxPoolHalf (host)
  const uint32_t keep = (uint32_t)(budget - a.W);
  const float *votes = a.votes + ((size_t)b * a.Hkv + kvh) * a.vote_stride;
  const int half = a.pool_kernel / 2;

  // Clipped max-pool. Raw votes of position tid + THREADS*i go to key[i] (0
  // past the prefix: votes are >= 0, so zero padding equals clipping); tile i
  // sits in LDS at offset kMaxPoolHalf with `half` halo values on each side
  // (the left halo from the previous tile's buffer, the right one from
  // key[i + 1]), and key[i] becomes the pooled value.
  uint32_t key[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int j = tid + THREADS * i;
    key[i] = j < npre ? __float_as_uint(votes[j]) : 0u;
  }
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    float *cur = pool_lds[i & 1];
    const float *prev = pool_lds[(i + 1) & 1];
    cur[kMaxPoolHalf + tid] = __uint_as_float(key[i]);
    if (tid < half) {
      cur[kMaxPoolHalf - half + tid] = i > 0 ? prev[kMaxPoolHalf + THREADS - half + tid] : 0.f;
      cur[kMaxPoolHalf + THREADS + tid] = i + 1 < VPT ? __uint_as_float(key[i + 1 < VPT ? i + 1 : i]) : 0.f;
    }
    __syncthreads();
    const float *w = cur + kMaxPoolHalf + tid;
    float v = w[0];
    if (half <= 3) {  // short windows: all reads issued together
      float x[6];
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        x[2 * t] = w[-(t + 1)];
        x[2 * t + 1] = w[t + 1];
      }
#pragma unroll
      for (int t = 0; t < 3; ++t)
        if (t < half) v = fmaxf(v, fmaxf(x[2 * t], x[2 * t + 1]));
    } else {
      for (int t = 1; t <= half; ++t) v = fmaxf(v, fmaxf(w[-t], w[t]));
    }
    key[i] = tid + THREADS * i < npre ? __float_as_uint(v) : 0u;
  }

  // Votes are sums of exponentials (>= +0), so bit 31 is clear.
  select_top_keys<THREADS, VPT, 30, PosIdentity, kBandCut, kBandCap>(key, npre, keep, out, sm, PosIdentity(),
                                                                     &band);
  for (int w = tid; w < a.W; w += THREADS) out[keep + w] = npre + w;
  for (int t = budget + tid; t < a.budget; t += THREADS) out[t] = -1;  // row past this budget
}

// Long prefixes: pooled values in the workspace, 4-pass 8-bit radix select.
// Writes out[0, keep) = the positions j < n with the `keep` largest keys,
// ties to the lower position, ascending; 0 < keep <= n; key(j) reads the key
// of position j from global memory. A 4-pass 8-bit radix select over an LDS
// histogram finds the keep-th largest key; an order-preserving compaction
// (two block scans per 1024 positions) writes every key above it and the
// lowest-positioned ties. One block of kTopkThreads threads.
template <class KeyFn>
__device__ __forceinline__ void select_top_keys_global(KeyFn key, int n, int keep, int32_t *out) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t scan_tmp[40];
  __shared__ uint32_t sel_digit, sel_above;
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = 0;
  uint32_t k_rem = (uint32_t)keep;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    for (int j = tid; j < n; j += kTopkThreads) {
      const uint32_t k = key(j);
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane owns bins 4*lane .. 4*lane+3; count of keys in bins above each
      uint32_t c[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) c[e] = hist[4 * tid + e];
      const uint32_t mine = c[0] + c[1] + c[2] + c[3];
      uint32_t incl = mine;  // inclusive suffix sum over lanes >= tid
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_down(incl, o, 64);
        if (tid + o < 64) incl += y;
      }
      uint32_t above = incl - mine;  // keys in bins of higher lanes
#pragma unroll
      for (int e = 3; e >= 0; --e) {
        if (above < k_rem && above + c[e] >= k_rem) {
          sel_digit = 4 * tid + e;
          sel_above = above;
        }
        above += c[e];
      }
    }
    __syncthreads();
    prefix |= sel_digit << shift;
    mask |= 255u << shift;
    k_rem -= sel_above;
    __syncthreads();
  }
  const uint32_t thr = prefix;  // the keep-th largest key
  const uint32_t need_eq = k_rem;  // how many keys equal to thr are taken

  uint32_t eq_carry = 0, out_carry = 0;
  for (int base = 0; base < n; base += kTopkThreads) {
    const int j = base + tid;
    const bool valid = j < n;
    const uint32_t k = valid ? key(j) : 0u;
    const bool gt = valid && k > thr;
    const bool eq = valid && k == thr;
    uint32_t eq_total;
    const uint32_t eq_rank = block_exclusive_scan(eq ? 1u : 0u, scan_tmp, &eq_total) + eq_carry;
    const bool take = gt || (eq && eq_rank < need_eq);
    uint32_t take_total;
    const uint32_t pos = block_exclusive_scan(take ? 1u : 0u, scan_tmp, &take_total) + out_carry;
    if (take && pos < (uint32_t)keep) out[pos] = j;
    eq_carry += eq_total;
    out_carry += take_total;
  }
}

__global__ __launch_bounds__(kTopkThreads) void snap_topk_global_kernel(SnapParams a) {
  const int tid = threadIdx.x;
  const int kvh = blockIdx.x % a.Hkv, b = blockIdx.x / a.Hkv;
  const int L = clampi(a.kv_lens[b], 0, a.len_cap);
  int32_t *out = a.idx + ((size_t)b * a.Hkv + kvh) * a.budget;
  const int budget = seq_budget(a, b);
  if (kvh == 0 && tid == 0) a.sel_lens[b] = min(L, budget);
  if (L <= budget) {
    for (int t = tid; t < a.budget; t += kTopkThreads) out[t] = t < L ? t : -1;
    return;
  }
  const int npre = L - a.W;
  const int keep = budget - a.W;
  const float *votes = a.votes + ((size_t)b * a.Hkv + kvh) * a.vote_stride;
  float *pooled = a.pooled + ((size_t)b * a.Hkv + kvh) * a.vote_stride;
  const int half = a.pool_kernel / 2;

  for (int j = tid; j < npre; j += kTopkThreads) {
    const int lo = max(0, j - half), hi = min(npre - 1, j + half);
    float v = votes[lo];
    for (int t = lo + 1; t <= hi; ++t) v = fmaxf(v, votes[t]);
    pooled[j] = v;
  }
  __threadfence_block();
  __syncthreads();
  // pooled votes are >= +0: their bit patterns order like the values
  select_top_keys_global([&](int j) { return __float_as_uint(pooled[j]); }, npre, keep, out);
  for (int w = tid; w < a.W; w += kTopkThreads) out[keep + w] = npre + w;
  for (int t = budget + tid; t < a.budget; t += kTopkThreads) out[t] = -1;  // row past this budget
}

// ---------------------------------------------------------------- top-K attention
// Order key of a score: a larger float gets a larger unsigned key; -0 and +0
// share the key of +0.
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  u = u == 0x80000000u ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kTauWords = 4096;      // sampled keys per unit (all heads)
constexpr int kTauThreads = 1024;
constexpr int kSmallThreads = 256;   // selection of rows with few candidates
constexpr int kSmallVpt = 24;
constexpr int kSmallSegs = 512;
constexpr int kStageEntries = 256;   // staged candidates per wave in the scoring pass
constexpr int kRowsThreads = 1024;
constexpr int kCandVpt = 8;          // candidates per thread in the selection (8192 per row)
constexpr int kCandVptBig = 32;      // the same for large budgets (32768 per row)
constexpr int kMaxSegs = 4096;       // scoring segments per unit the selection gathers from LDS

// Sampled position i < n_s of a sequence of length L: every position when
// n_s = L; otherwise n_s / 16 runs of 16 consecutive positions (one step, one
// page block) at evenly spread steps, all below L.
__device__ __forceinline__ int sample_pos(int i, int L, int n_s) {
  if (n_s >= L) return i;
  const int runs = n_s / kStepTokens, full_steps = L / kStepTokens;  // full_steps >= runs since L > n_s
  return (int)((int64_t)(i / kStepTokens) * full_steps / runs) * kStepTokens + i % kStepTokens;
}

// Threshold per (sequence, query head): the t-th largest score key of n_s
// sampled positions (sample_pos), with t chosen so that at least `budget`
// keys of the whole row lie at or above it unless the sample is far from
// representative: t = n_s * budget / L (the expected number of samples among
// the budget largest keys) plus five standard deviations of that count plus
// 8, a binomial tail of about 1e-8 per row for independent scores. Keys at or
// above the threshold are the row's candidates; a row with fewer than
// `budget` candidates is recomputed in full by the selection kernel, so the
// threshold only affects speed, never the result. One block of
// 16 waves per (sequence, KV head): each wave scores at most kBatch steps of
// 16 samples, with all their loads in flight at once.
template <int D>
__global__ __launch_bounds__(kTauThreads) void topk_tau_kernel(SnapParams a) {
  __shared__ uint32_t sk[kTauWords];
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int kvh = blockIdx.x % a.Hkv, b = blockIdx.x / a.Hkv;
  if (blockIdx.x == 0 && threadIdx.x == 0) a.deferred[0] = 0;  // the selection kernels run after this one
  const int L = clampi(a.kv_lens[b], 0, a.len_cap);
  if (L <= a.budget) return;
  const int cap = min(1024, kTauWords / a.G / kStepTokens * kStepTokens);  // samples per head, >= 256
  const int n_s = min(L, cap);
  u32x4 q[1][D / 32];
  snap_load_q<D, 1>(a, b, kvh, q);
  const char *kp = reinterpret_cast<const char *>(a.k_pages);
  const int32_t *pt = a.page_table + (size_t)b * a.max_pages;
  constexpr int kBatch = 4;  // steps of 16 samples whose loads are issued together
  constexpr int kWaves = kTauThreads / 64;
  const int n_steps = (n_s + kStepTokens - 1) / kStepTokens;
  // wave w scores steps w, w + kWaves, ...
  for (int s0 = wave; s0 < n_steps; s0 += kBatch * kWaves) {
    u32x4 k[kBatch][D / 32];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = min((s0 + j * kWaves) * kStepTokens + r, n_s - 1);
      const int pos = sample_pos(i, L, n_s);
      const int page = clampi(pt[pos / a.page_size], 0, a.num_pages - 1);
      const char *kb = kp + ((size_t)(page * a.Hkv + kvh) * a.page_size + pos % a.page_size) * D * 2;
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk)
        k[j][kk] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kb + (32 * kk + 8 * g) * 2));
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int st = s0 + j * kWaves;
      if (st >= n_steps) break;
      const f32x4 sc = snap_scores<D, 1>(k[j], q, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = st * kStepTokens + 4 * g + e;
        if (r < a.G && i < n_s) sk[r * cap + i] = order_key(sc[e]);
      }
    }
  }
  __syncthreads();
  const float expect = (float)a.budget * (float)n_s / (float)L;
  const int t = n_s == L ? a.budget : min(n_s, (int)ceilf(expect + 5.f * sqrtf(expect) + 8.f));
  for (int h = wave; h < a.G; h += kWaves) {
    uint32_t v[16];  // cap / 64 <= 16 keys per lane
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int idx = lane + 64 * i;
      v[i] = idx < n_s ? sk[h * cap + idx] : 0u;
    }
    uint32_t T = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = T | (1u << bit);
      uint32_t c = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) c += v[i] >= cand ? 1u : 0u;
      if (wave_sum_u32(c) >= (uint32_t)t) T = cand;
    }
    if (lane == 0) a.tau[(size_t)b * a.Hq + (size_t)kvh * a.G + h] = T;
  }
}

// LDS accesses the compiler does not track (no wait added for the
// asynchronous ring loads); reads return with their data.
__device__ __forceinline__ void lds_write_b64(const char *lds, int byte_off, uint32_t x, uint32_t y) {
  const uint32_t addr = (uint32_t)(size_t)((const __attribute__((address_space(3))) char *)lds + byte_off);
  u32x2 v = {x, y};
#if __HIP_DEVICE_COMPILE__
  asm volatile("ds_write_b64 %0, %1" ::"v"(addr), "v"(v) : "memory");
#endif
}
__device__ __forceinline__ void lds_read_4xb64(const char *lds, int byte_off, int stride, u32x2 (&v)[4]) {
  const uint32_t a0 = (uint32_t)(size_t)((const __attribute__((address_space(3))) char *)lds + byte_off);
  const uint32_t a1 = a0 + stride, a2 = a0 + 2 * stride, a3 = a0 + 3 * stride;
#if __HIP_DEVICE_COMPILE__
  asm volatile(
      "ds_read_b64 %0, %4\n\tds_read_b64 %1, %5\n\tds_read_b64 %2, %6\n\tds_read_b64 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
      : "memory");
#endif
}

// Scores <q_h, k_j> of the G query heads of each KV head over the unit's keys
// (sequences longer than the budget only). Keys at or above the row's
// threshold are candidates: each segment writes its candidates, in position
// order, as (key, position) at the start of its own key range of the row
// (keys[row][s_begin*16 + c], cand_pos likewise) and their number to
// counts[slot*G + h]. Lane (g, r) holds keys 4g..4g+3 of a step for head r;
// a candidate's place among the step's candidates of its head comes from four
// ballots. Stores share the in-order memory counter with the K stream, so
// candidates are staged in LDS (kStageEntries / G per head) and leave in
// batches.
template <int D>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void topk_scores_kernel(SnapParams a) {
  constexpr int kStageOff = KStream<D>::kLdsBytes;
  __shared__ __attribute__((aligned(16))) char lds[kStageOff + kStageEntries * 8];
  const int lane = lane_id();
  const int g = lane >> 4, r = lane & 15;
  const int cap_h = kStageEntries / a.G;  // staged entries per head (G <= 16: >= 16, one step's worth)
  const uint64_t head_lanes = 0x0001000100010001ull << r;          // lanes (0..3, r)
  const uint64_t lower_lanes = head_lanes & ((1ull << (16 * g)) - 1ull);  // lanes (g' < g, r)
  sched_for_each_segment(a.sc, blockIdx.x, [&](int b, int kvh, int s_begin, int s_end, size_t slot) {
    s_begin = __builtin_amdgcn_readfirstlane(s_begin);
    s_end = __builtin_amdgcn_readfirstlane(s_end);
    u32x4 q[1][D / 32];
    snap_load_q<D, 1>(a, b, kvh, q);  // rows = G (one query row per head)
    const size_t row0 = (size_t)b * a.Hq + (size_t)kvh * a.G;
    const uint32_t tau = r < a.G ? a.tau[row0 + r] : 0u;
    const int L = clampi(a.kv_lens[b], 0, a.len_cap);  // positions past L are never candidates
    int staged = 0, written = 0;  // of head r (the same in every lane of that head)
    // Write the staged entries of every head after the ones already written:
    // lane l moves stage slots l, l+64, l+128, l+192.
    auto flush = [&]() {
      u32x2 v[4];
      lds_read_4xb64(lds, kStageOff + 8 * lane, 64 * 8, v);
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const int slot_i = lane + 64 * k4;
        const int h = slot_i / cap_h, i = slot_i % cap_h;
        const int hs = min(h, a.G - 1);
        const int n_h = __shfl(staged, hs, 64), w_h = __shfl(written, hs, 64);
        if (h < a.G && i < n_h) {
          const size_t at = (row0 + h) * a.key_stride + (size_t)s_begin * kStepTokens + w_h + i;
          a.keys[at] = v[k4].x;
          a.cand_pos[at] = (int32_t)v[k4].y;
        }
      }
      written += staged;
      staged = 0;
    };
    KStream<D> ks(a, b, kvh, s_end - 1, lds);
    ks.begin(s_begin);
    for (int s = s_begin; s < s_end; ++s) {
      ks.advance(s);
      u32x4 k[D / 32];
      ks.operand(s, k);
      const f32x4 sc = snap_scores<D, 1>(k, q, 0);
      uint32_t key[4];
      bool pass[4];
      uint64_t m[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        key[e] = order_key(sc[e]);
        pass[e] = r < a.G && key[e] >= tau && s * kStepTokens + 4 * g + e < L;
        m[e] = __ballot(pass[e]);
      }
      if ((m[0] | m[1] | m[2] | m[3]) == 0ull) continue;  // no candidate in this step (the common case)
      if (__ballot(staged + kStepTokens > cap_h) != 0ull) flush();
      int before = 0, total = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        before += __popcll(m[e] & lower_lanes);
        total += __popcll(m[e] & head_lanes);
      }
      int at = staged + before;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (pass[e]) {
          lds_write_b64(lds, kStageOff + (r * cap_h + at) * 8, key[e], (uint32_t)(s * kStepTokens + 4 * g + e));
          ++at;
        }
      }
      staged += total;
    }
    flush();
    if (g == 0 && r < a.G) a.counts[slot * a.G + r] = written;
  });
  KStream<D>::drain();
}

// Segments of the unit (sequence b, KV head kvh) in the scoring schedule:
// waves w_lo..w_hi each own a run of its steps.
struct UnitSegs {
  int64_t T, W, A, w_lo, w_hi;
  __device__ UnitSegs(const SnapParams &a, int b, int kvh, int n) {
    T = (int64_t)a.Hkv * a.sc.seq_prefix[a.sc.B];
    W = sched_working_waves(a.sc, T);
    A = (int64_t)a.Hkv * a.sc.seq_prefix[b] + (int64_t)kvh * n;
    sched_unit_waves(A, n, T, W, w_lo, w_hi);
  }
  __device__ int count() const { return (int)(w_hi - w_lo + 1); }
  // first key (within the unit) of segment i
  __device__ int key0(int i) const {
    const int64_t w = w_lo + i;
    return (int)(max(A, (w * T + W - 1) / W) - A) * kStepTokens;
  }
};

// Per (sequence, query head) with at most kSmallThreads * kSmallVpt
// candidates (the common case): gather the row's candidates from its unit's
// scoring segments and select the budget largest, ties to the lower position,
// ascending, in one block of four waves. Other rows are marked for
// topk_rows_full_kernel.
__global__ __launch_bounds__(kSmallThreads) void topk_rows_small_kernel(SnapParams a) {
  __shared__ TopkLds<kSmallThreads, kSmallVpt> sm;
  __shared__ int32_t seg_off[kSmallSegs + 1];
  __shared__ int32_t seg_key0[kSmallSegs];
  __shared__ uint64_t scan_w[kSmallThreads / 64];
  __shared__ uint64_t total_sh;
  const int tid = threadIdx.x;
  const int h = blockIdx.x % a.Hq, b = blockIdx.x / a.Hq;
  const size_t row = (size_t)b * a.Hq + h;
  const int L = clampi(a.kv_lens[b], 0, a.len_cap);
  int32_t *out = a.idx + row * a.budget;
  if (L <= a.budget) {
    if (h == 0 && tid == 0) a.sel_lens[b] = L;
    for (int t = tid; t < a.budget; t += kSmallThreads) out[t] = t < L ? t : -1;
    return;
  }
  const int kvh = h / a.G, hl = h % a.G;
  const int u = b * a.Hkv + kvh;
  const UnitSegs us(a, b, kvh, (L + kStepTokens - 1) / kStepTokens);
  const int nseg = us.count();
  int E = -1;
  if (nseg <= kSmallSegs) {
    uint64_t carry = 0;
    for (int base = 0; base < nseg; base += kSmallThreads) {
      const int sgi = base + tid;
      uint64_t cnt = 0;
      if (sgi < nseg) {
        seg_key0[sgi] = us.key0(sgi);
        cnt = (uint64_t)a.counts[((size_t)a.sc.slot_base[u] + sgi) * a.G + hl];
      }
      const uint64_t ex = block_exclusive_scan_u64<kSmallThreads / 64>(cnt, scan_w);
      if (sgi < nseg) seg_off[sgi] = (int)(carry + ex);
      if (tid == kSmallThreads - 1) total_sh = ex + cnt;
      __syncthreads();
      carry += total_sh;
      __syncthreads();
    }
    if (tid == 0) seg_off[nseg] = (int)carry;
    __syncthreads();
    E = (int)carry;
  }
  const bool here = E >= a.budget && E <= kSmallThreads * kSmallVpt;
  if (!here) {
    if (tid == 0) a.deferred[1 + atomicAdd(a.deferred, 1)] = (int32_t)row;
    return;
  }
  if (h == 0 && tid == 0) a.sel_lens[b] = a.budget;
  const uint32_t *krow = a.keys + row * a.key_stride;
  const int32_t *prow = a.cand_pos + row * a.key_stride;
  uint32_t key[kSmallVpt];
  int32_t pos[kSmallVpt];
#pragma unroll
  for (int i = 0; i < kSmallVpt; ++i) {
    const int e = tid + kSmallThreads * i;
    key[i] = 0u;  // candidate keys are >= their threshold > 0: zero padding is never counted
    pos[i] = 0;
    if (e < E) {
      int lo = 0, hi = nseg - 1;  // last segment with seg_off <= e
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (seg_off[mid] <= e)
          lo = mid;
        else
          hi = mid - 1;
      }
      const int at = seg_key0[lo] + (e - seg_off[lo]);
      key[i] = krow[at];
      pos[i] = prow[at];
    }
  }
  select_top_keys<kSmallThreads, kSmallVpt, 31>(key, E, (uint32_t)a.budget, out, sm,
                                                [&](int i, int) { return pos[i]; });
}

// The rows topk_rows_small_kernel left: the budget largest keys of the row,
// ties to the lower position, ascending. The row's candidates are gathered
// from the scoring segments of its unit (the segment boundaries follow from
// the schedule tables), and the budget largest are selected among them in
// registers. A row with fewer candidates than the budget (threshold above the
// budget-th key), more than kRowsThreads * kCandVptBig candidates, or more than
// kMaxSegs segments is recomputed in full: every score again with the
// scoring pass's MFMA arithmetic, written over the row's key array, and
// selected with the radix select.
template <int D>
__device__ void topk_row_full(const SnapParams &a, int b, int h) {
  __shared__ TopkLds<kRowsThreads, kCandVpt> sm;
  __shared__ TopkLds<kRowsThreads, kCandVptBig> sm_big;
  __shared__ int32_t seg_off[kMaxSegs + 1];
  __shared__ int32_t seg_key0[kMaxSegs];
  __shared__ uint32_t scan_tmp[40];
  const int tid = threadIdx.x;
  const size_t row = (size_t)b * a.Hq + h;
  const int L = clampi(a.kv_lens[b], 0, a.len_cap);
  int32_t *out = a.idx + row * a.budget;
  if (h == 0 && tid == 0) a.sel_lens[b] = min(L, a.budget);
  const int kvh = h / a.G, hl = h % a.G;
  uint32_t *krow = a.keys + row * a.key_stride;
  const int32_t *prow = a.cand_pos + row * a.key_stride;

  const int u = b * a.Hkv + kvh;
  const UnitSegs us(a, b, kvh, (L + kStepTokens - 1) / kStepTokens);
  const int nseg = us.count();
  int E = 0;
  if (nseg <= kMaxSegs) {
    uint32_t carry = 0;
    for (int base = 0; base < nseg; base += kRowsThreads) {
      const int sgi = base + tid;
      uint32_t cnt = 0;
      if (sgi < nseg) {
        seg_key0[sgi] = us.key0(sgi);
        cnt = (uint32_t)a.counts[((size_t)a.sc.slot_base[u] + sgi) * a.G + hl];
      }
      uint32_t tot;
      const uint32_t ex = block_exclusive_scan(cnt, scan_tmp, &tot);
      if (sgi < nseg) seg_off[sgi] = (int)(carry + ex);
      carry += tot;
    }
    if (tid == 0) seg_off[nseg] = (int)carry;
    __syncthreads();
    E = (int)carry;
  }
  // Candidate e (in position order) sits at the start of its segment's key range.
  auto gather = [&](int e, uint32_t &key, int32_t &pos) {
    int lo = 0, hi = nseg - 1;  // last segment with seg_off <= e
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (seg_off[mid] <= e)
        lo = mid;
      else
        hi = mid - 1;
    }
    const int at = seg_key0[lo] + (e - seg_off[lo]);
    key = krow[at];
    pos = prow[at];
  };
  // candidate keys are >= their threshold > 0, so zero padding is never counted
  if (nseg <= kMaxSegs && E >= a.budget && E <= kRowsThreads * kCandVpt) {
    uint32_t key[kCandVpt];
    int32_t pos[kCandVpt];
#pragma unroll
    for (int i = 0; i < kCandVpt; ++i) {
      key[i] = 0u;
      pos[i] = 0;
      if (tid + kRowsThreads * i < E) gather(tid + kRowsThreads * i, key[i], pos[i]);
    }
    select_top_keys<kRowsThreads, kCandVpt, 31>(key, E, (uint32_t)a.budget, out, sm,
                                                [&](int i, int) { return pos[i]; });
    return;
  }
  if (nseg <= kMaxSegs && E >= a.budget && E <= kRowsThreads * kCandVptBig) {
    uint32_t key[kCandVptBig];
    int32_t pos[kCandVptBig];
#pragma unroll
    for (int i = 0; i < kCandVptBig; ++i) {
      key[i] = 0u;
      pos[i] = 0;
      if (tid + kRowsThreads * i < E) gather(tid + kRowsThreads * i, key[i], pos[i]);
    }
    select_top_keys<kRowsThreads, kCandVptBig, 31>(key, E, (uint32_t)a.budget, out, sm_big,
                                                   [&](int i, int) { return pos[i]; });
    return;
  }

  // Full recomputation of the row with the scoring pass's arithmetic: wave w
  // of the block scores steps w, w + 16, ... (16 keys each, kBatch steps'
  // loads in flight) for the G heads of the unit and keeps head hl's keys.
  constexpr int kWaves = kRowsThreads / 64;
  constexpr int kBatch = 4;
  const int lane = lane_id(), wave = tid >> 6;
  const int g = lane >> 4, r = lane & 15;
  u32x4 q[1][D / 32];
  snap_load_q<D, 1>(a, b, kvh, q);
  const char *kp = reinterpret_cast<const char *>(a.k_pages);
  const int32_t *pt = a.page_table + (size_t)b * a.max_pages;
  const int n_steps = (L + kStepTokens - 1) / kStepTokens;
  for (int s0 = wave; s0 < n_steps; s0 += kBatch * kWaves) {
    u32x4 k[kBatch][D / 32];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int pos = min((s0 + j * kWaves) * kStepTokens + r, L - 1);
      const int page = clampi(pt[pos / a.page_size], 0, a.num_pages - 1);
      const char *kb = kp + ((size_t)(page * a.Hkv + kvh) * a.page_size + pos % a.page_size) * D * 2;
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk)
        k[j][kk] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kb + (32 * kk + 8 * g) * 2));
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int st = s0 + j * kWaves;
      if (st >= n_steps) break;
      const f32x4 sc = snap_scores<D, 1>(k[j], q, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pos = st * kStepTokens + 4 * g + e;
        if (r == hl && pos < L) krow[pos] = order_key(sc[e]);
      }
    }
  }
  __threadfence_block();
  __syncthreads();
  select_top_keys_global([&](int j) { return krow[j]; }, L, a.budget, out);
}

// One block per deferred row, in turn.
template <int D>
__global__ __launch_bounds__(kRowsThreads) void topk_rows_full_kernel(SnapParams a) {
  for (int k = blockIdx.x; k < a.deferred[0]; k += gridDim.x) {
    const int row_id = a.deferred[1 + k];
    topk_row_full<D>(a, row_id / a.Hq, row_id % a.Hq);
    __syncthreads();  // LDS of this row is reused by the next
  }
}

struct SnapLayout {
  int vote_stride;
  size_t stats_off, votes_off, pooled_off, bytes;
};

SnapLayout snap_layout(int64_t B, int64_t Hkv, int64_t rows, int64_t max_len) {
  SnapLayout l;
  l.vote_stride = (int)(sdh::ceil_div(std::max<int64_t>(1, max_len), 4) * 4);  // 16-byte aligned rows
  l.stats_off = sdh::sched_table_bytes(B, Hkv);
  l.votes_off = l.stats_off + sdh::align_up((size_t)sdh::sched_max_slots(B, Hkv) * rows * 2 * 4);
  l.pooled_off = l.votes_off + sdh::align_up((size_t)B * Hkv * l.vote_stride * 4);
  l.bytes = l.pooled_off + sdh::align_up((size_t)B * Hkv * l.vote_stride * 4);
  return l;
}

// Register top-K with the fewest values per thread that cover the prefix.
void launch_topk_reg(SnapParams &a, unsigned blocks, int64_t npre_cap, hipStream_t st) {
  constexpr int TH = kTopkThreads;
  if (npre_cap <= 8 * TH)
    snap_topk_kernel<TH, 8><<<blocks, TH, 0, st>>>(a);
  else if (npre_cap <= 16 * TH)
    snap_topk_kernel<TH, 16><<<blocks, TH, 0, st>>>(a);
  else if (npre_cap <= 32 * TH)
    snap_topk_kernel<TH, 32><<<blocks, TH, 0, st>>>(a);
  else
    snap_topk_kernel<TH, 64><<<blocks, TH, 0, st>>>(a);
}

// What a SnapKV call computes: the whole selection; the window normalisers
// alone (pass 1 and a merge); or the selection from normalisers the caller
// gives (pass 2 and the top-K, no pass 1).
enum class SnapMode { kSelect, kWindowLse, kSelectFromLse };

template <int D, int NB>
void launch_snap_passes(SnapParams &a, SnapMode mode, hipStream_t st) {
  static int cache[sdh::kMaxDevices] = {};  // resident waves of this instantiation per device
  a.sc.waves = sdh::resident_waves(reinterpret_cast<const void *>(snap_stats_kernel<D, NB>), 2 * kSimdsPerCU,
                                   cache);
  snap_plan_kernel<<<1, kPlanThreads, 0, st>>>(a);
  if (mode != SnapMode::kSelectFromLse) snap_stats_kernel<D, NB><<<(unsigned)a.sc.waves, 64, 0, st>>>(a);
  if (mode == SnapMode::kWindowLse)
    snap_lse_kernel<NB><<<(unsigned)(a.sc.B * a.Hkv), 64, 0, st>>>(a);
  else
    snap_votes_kernel<D, NB><<<(unsigned)a.sc.waves, 64, 0, st>>>(a);
}

template <int D>
sd_status launch_snap(SnapParams &a, int B, SnapMode mode, hipStream_t st) {
  switch ((a.rows + 15) / 16) {
    case 1: launch_snap_passes<D, 1>(a, mode, st); break;
    case 2: launch_snap_passes<D, 2>(a, mode, st); break;
    case 3: launch_snap_passes<D, 3>(a, mode, st); break;
    case 4: launch_snap_passes<D, 4>(a, mode, st); break;
    case 5: launch_snap_passes<D, 5>(a, mode, st); break;
    case 6: launch_snap_passes<D, 6>(a, mode, st); break;
    case 7: launch_snap_passes<D, 7>(a, mode, st); break;
    case 8: launch_snap_passes<D, 8>(a, mode, st); break;
    default: return SD_ERR_UNSUPPORTED;
  }
  if (mode == SnapMode::kWindowLse) return sdh::launch_status();
  const unsigned blocks = (unsigned)(B * a.Hkv);
  const int64_t npre_cap = (int64_t)a.len_cap - a.W;
  if (a.pool_kernel / 2 > kMaxPoolHalf || npre_cap > (int64_t)kTopkThreads * 64)
    snap_topk_global_kernel<<<blocks, kTopkThreads, 0, st>>>(a);
  else
    launch_topk_reg(a, blocks, npre_cap, st);
  return sdh::launch_status();
}

}  // namespace

extern "C" sd_status sd_streaming_select(const int32_t *kv_lens, int32_t batch, int32_t sink,
                                         int32_t recent, int32_t *idx, int32_t *sel_lens,
                                         void *stream) {
  SD_REQUIRE(kv_lens != nullptr && idx != nullptr && sel_lens != nullptr, SD_ERR_INVALID_ARG);
  SD_REQUIRE(batch > 0 && sink >= 0 && recent >= 0 && (int64_t)sink + recent > 0, SD_ERR_INVALID_ARG);
  SD_REQUIRE((int64_t)sink + recent < ((int64_t)1 << 30), SD_ERR_UNSUPPORTED);  // int32 row offsets
  streaming_select_kernel<<<(unsigned)batch, 256, 0, sdh::as_stream(stream)>>>(kv_lens, sink, recent,
                                                                              idx, sel_lens);
  return sdh::launch_status();
}

extern "C" size_t sd_snapkv_select_workspace_size(int32_t batch, int32_t window,
                                                  int32_t num_q_heads, int32_t num_kv_heads,
                                                  int32_t max_kv_len) {
  if (batch <= 0 || window <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_kv_len < 0 ||
      num_q_heads % num_kv_heads != 0)
    return 0;
  const int rows = num_q_heads / num_kv_heads * window;
  return snap_layout(batch, num_kv_heads, rows, max_kv_len).bytes;
}

namespace {

sd_status snapkv_impl(SnapMode mode, const sd_kv_cache *kv, const void *q_obs, const float *obs_lse,
                      int32_t batch, int32_t window, int32_t num_q_heads, int32_t pool_kernel,
                      const int32_t *budgets, int32_t budget, int32_t max_kv_len, float softmax_scale,
                      int32_t *idx, int32_t *sel_lens, float *lse_out, void *workspace,
                      size_t workspace_bytes, void *stream) {
  sd_status s = sdh::check_kv(kv, false);
  if (s != SD_OK) return s;
  SD_REQUIRE(q_obs != nullptr, SD_ERR_INVALID_ARG);
  if (mode == SnapMode::kWindowLse) {
    SD_REQUIRE(lse_out != nullptr, SD_ERR_INVALID_ARG);
  } else {
    SD_REQUIRE(idx != nullptr && sel_lens != nullptr, SD_ERR_INVALID_ARG);
    SD_REQUIRE(mode != SnapMode::kSelectFromLse || obs_lse != nullptr, SD_ERR_INVALID_ARG);
    SD_REQUIRE(budget > window, SD_ERR_INVALID_ARG);
    SD_REQUIRE(pool_kernel >= 1 && (pool_kernel & 1) == 1, SD_ERR_INVALID_ARG);
  }
  SD_REQUIRE(sdh::aligned16(q_obs), SD_ERR_INVALID_ARG);
  SD_REQUIRE(batch > 0 && window >= 1 && num_q_heads > 0, SD_ERR_INVALID_ARG);
  SD_REQUIRE(num_q_heads % kv->num_kv_heads == 0, SD_ERR_INVALID_ARG);
  SD_REQUIRE(max_kv_len >= 0 && (int64_t)max_kv_len <= (int64_t)kv->max_pages * kv->page_size,
             SD_ERR_INVALID_ARG);
  // the scaled scores (and the stats pass's lazily rebased row maxima) are
  // meaningful only for a finite positive scale
  SD_REQUIRE(softmax_scale > 0.f && softmax_scale * kLog2e < __builtin_inff(), SD_ERR_INVALID_ARG);
  SD_REQUIRE(kv->dtype == SD_BF16, SD_ERR_UNSUPPORTED);
  const int G = num_q_heads / kv->num_kv_heads;
  SD_REQUIRE((int64_t)G * window <= 128, SD_ERR_UNSUPPORTED);
  const int rows = G * window;
  const SnapLayout lay = snap_layout(batch, kv->num_kv_heads, rows, max_kv_len);
  SD_REQUIRE(workspace != nullptr && workspace_bytes >= lay.bytes, SD_ERR_WORKSPACE);
  SD_REQUIRE((int64_t)batch * kv->num_kv_heads + kMaxWaves < ((int64_t)1 << 30), SD_ERR_UNSUPPORTED);
  // the schedule keeps per-sequence step prefix sums in int32
  SD_REQUIRE((int64_t)batch * sdh::ceil_div(max_kv_len, 16) < ((int64_t)1 << 31), SD_ERR_UNSUPPORTED);

  SnapParams a{};
  a.k_pages = kv->k_pages;
  a.page_table = kv->page_table;
  a.kv_lens = kv->kv_lens;
  a.q_obs = q_obs;
  char *ws = reinterpret_cast<char *>(workspace);
  sdh::sched_bind(a.sc, ws, batch, kv->num_kv_heads);
  a.stats = reinterpret_cast<float *>(ws + lay.stats_off);
  a.votes = reinterpret_cast<float *>(ws + lay.votes_off);
  a.pooled = reinterpret_cast<float *>(ws + lay.pooled_off);
  a.idx = idx;
  a.sel_lens = sel_lens;
  a.W = window;
  a.Hq = num_q_heads;
  a.Hkv = kv->num_kv_heads;
  a.G = G;
  a.rows = rows;
  a.num_pages = kv->num_pages;
  a.page_size = kv->page_size;
  a.max_pages = kv->max_pages;
  a.len_cap = max_kv_len;
  a.vote_stride = lay.vote_stride;
  a.pool_kernel = pool_kernel;
  a.budget = budget;
  a.budgets = budgets;
  a.obs_lse = mode == SnapMode::kSelectFromLse ? obs_lse : nullptr;
  a.lse_out = lse_out;
  a.scale_log2 = softmax_scale * kLog2e;
  hipStream_t st = sdh::as_stream(stream);
  if (kv->head_dim == 128) return launch_snap<128>(a, batch, mode, st);
  return launch_snap<64>(a, batch, mode, st);
}

}  // namespace

extern "C" sd_status sd_snapkv_select(const sd_kv_cache *kv, const void *q_obs, int32_t batch,
                                      int32_t window, int32_t num_q_heads, int32_t pool_kernel,
                                      int32_t budget, int32_t max_kv_len, float softmax_scale,
                                      int32_t *idx, int32_t *sel_lens, void *workspace,
                                      size_t workspace_bytes, void *stream) {
  return snapkv_impl(SnapMode::kSelect, kv, q_obs, nullptr, batch, window, num_q_heads, pool_kernel, nullptr,
                     budget, max_kv_len, softmax_scale, idx, sel_lens, nullptr, workspace, workspace_bytes,
                     stream);
}

extern "C" sd_status sd_snapkv_window_lse(const sd_kv_cache *kv, const void *q_obs, int32_t batch,
                                          int32_t window, int32_t num_q_heads, int32_t max_kv_len,
                                          float softmax_scale, float *lse, void *workspace,
                                          size_t workspace_bytes, void *stream) {
  // budget 0: every sequence with a key is scored
  return snapkv_impl(SnapMode::kWindowLse, kv, q_obs, nullptr, batch, window, num_q_heads, 1, nullptr, 0,
                     max_kv_len, softmax_scale, nullptr, nullptr, lse, workspace, workspace_bytes, stream);
}

extern "C" sd_status sd_snapkv_select_lse(const sd_kv_cache *kv, const void *q_obs, const float *obs_lse,
                                          int32_t batch, int32_t window, int32_t num_q_heads,
                                          int32_t pool_kernel, int32_t budget, int32_t max_kv_len,
                                          float softmax_scale, int32_t *idx, int32_t *sel_lens,
                                          void *workspace, size_t workspace_bytes, void *stream) {
  return snapkv_impl(SnapMode::kSelectFromLse, kv, q_obs, obs_lse, batch, window, num_q_heads, pool_kernel,
                     nullptr, budget, max_kv_len, softmax_scale, idx, sel_lens, nullptr, workspace,
                     workspace_bytes, stream);
}

extern "C" sd_status sd_snapkv_select_budgets(const sd_kv_cache *kv, const void *q_obs, int32_t batch,
                                              int32_t window, int32_t num_q_heads, int32_t pool_kernel,
                                              const int32_t *budgets, int32_t max_budget,
                                              int32_t max_kv_len, float softmax_scale, int32_t *idx,
                                              int32_t *sel_lens, void *workspace, size_t workspace_bytes,
                                              void *stream) {
  SD_REQUIRE(budgets != nullptr, SD_ERR_INVALID_ARG);
  return snapkv_impl(SnapMode::kSelect, kv, q_obs, nullptr, batch, window, num_q_heads, pool_kernel, budgets,
                     max_budget, max_kv_len, softmax_scale, idx, sel_lens, nullptr, workspace, workspace_bytes,
                     stream);
}

namespace {

struct TopkLayout {
  size_t tau_off, def_off, counts_off, keys_off, pos_off, bytes;
  int key_stride;
};

TopkLayout topk_layout(int64_t B, int64_t Hq, int64_t Hkv, int64_t max_len) {
  TopkLayout l;
  l.key_stride = (int)(sdh::ceil_div(std::max<int64_t>(1, max_len), 16) * 16);
  const size_t row_bytes = sdh::align_up((size_t)B * Hq * l.key_stride * 4);
  l.tau_off = sdh::sched_table_bytes(B, Hkv);
  l.def_off = l.tau_off + sdh::align_up((size_t)B * Hq * 4);
  l.counts_off = l.def_off + sdh::align_up((size_t)(B * Hq + 1) * 4);
  l.keys_off = l.counts_off + sdh::align_up((size_t)sdh::sched_max_slots(B, Hkv) * (Hq / Hkv) * 4);
  l.pos_off = l.keys_off + row_bytes;
  l.bytes = l.pos_off + row_bytes;
  return l;
}

template <int D>
void launch_topk_attn_select(SnapParams &a, int B, hipStream_t st) {
  static int cache[sdh::kMaxDevices] = {};  // resident waves of the scoring kernel per device
  a.sc.waves = sdh::resident_waves(reinterpret_cast<const void *>(topk_scores_kernel<D>), 2 * kSimdsPerCU, cache);
  snap_plan_kernel<<<1, kPlanThreads, 0, st>>>(a);
  topk_tau_kernel<D><<<(unsigned)(B * a.Hkv), kTauThreads, 0, st>>>(a);
  topk_scores_kernel<D><<<(unsigned)a.sc.waves, 64, 0, st>>>(a);
  topk_rows_small_kernel<<<(unsigned)(B * a.Hq), kSmallThreads, 0, st>>>(a);
  topk_rows_full_kernel<D><<<(unsigned)std::min<int64_t>((int64_t)B * a.Hq, 2 * kNumCUs), kRowsThreads, 0, st>>>(a);
}

}  // namespace

extern "C" size_t sd_topk_select_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                                int32_t max_kv_len) {
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_kv_len < 0 || num_q_heads % num_kv_heads != 0)
    return 0;
  return topk_layout(batch, num_q_heads, num_kv_heads, max_kv_len).bytes;
}

extern "C" sd_status sd_topk_select(const sd_kv_cache *kv, const void *q, int32_t batch, int32_t num_q_heads,
                                    int32_t budget, int32_t max_kv_len, int32_t *idx, int32_t *sel_lens,
                                    void *workspace, size_t workspace_bytes, void *stream) {
  sd_status s = sdh::check_kv(kv, false);
  if (s != SD_OK) return s;
  SD_REQUIRE(q != nullptr && idx != nullptr && sel_lens != nullptr, SD_ERR_INVALID_ARG);
  SD_REQUIRE(sdh::aligned16(q), SD_ERR_INVALID_ARG);
  SD_REQUIRE(batch > 0 && num_q_heads > 0 && budget > 0, SD_ERR_INVALID_ARG);
  SD_REQUIRE(num_q_heads % kv->num_kv_heads == 0, SD_ERR_INVALID_ARG);
  SD_REQUIRE(max_kv_len >= 0 && (int64_t)max_kv_len <= (int64_t)kv->max_pages * kv->page_size,
             SD_ERR_INVALID_ARG);
  SD_REQUIRE(kv->dtype == SD_BF16, SD_ERR_UNSUPPORTED);
  const int G = num_q_heads / kv->num_kv_heads;
  SD_REQUIRE(G <= 16, SD_ERR_UNSUPPORTED);
  SD_REQUIRE((int64_t)batch * kv->num_kv_heads + kMaxWaves < ((int64_t)1 << 30), SD_ERR_UNSUPPORTED);
  SD_REQUIRE((int64_t)batch * num_q_heads < ((int64_t)1 << 31), SD_ERR_UNSUPPORTED);
  // the schedule keeps per-sequence step prefix sums in int32
  SD_REQUIRE((int64_t)batch * sdh::ceil_div(max_kv_len, 16) < ((int64_t)1 << 31), SD_ERR_UNSUPPORTED);
  const TopkLayout lay = topk_layout(batch, num_q_heads, kv->num_kv_heads, max_kv_len);
  SD_REQUIRE(workspace != nullptr && workspace_bytes >= lay.bytes, SD_ERR_WORKSPACE);

  SnapParams a{};
  a.k_pages = kv->k_pages;
  a.page_table = kv->page_table;
  a.kv_lens = kv->kv_lens;
  a.q_obs = q;  // [B, 1, Hq, D]: one query row per head
  char *ws = reinterpret_cast<char *>(workspace);
  sdh::sched_bind(a.sc, ws, batch, kv->num_kv_heads);
  a.keys = reinterpret_cast<uint32_t *>(ws + lay.keys_off);
  a.cand_pos = reinterpret_cast<int32_t *>(ws + lay.pos_off);
  a.tau = reinterpret_cast<uint32_t *>(ws + lay.tau_off);
  a.counts = reinterpret_cast<int32_t *>(ws + lay.counts_off);
  a.deferred = reinterpret_cast<int32_t *>(ws + lay.def_off);
  a.key_stride = lay.key_stride;
  a.head_dim = kv->head_dim;
  a.idx = idx;
  a.sel_lens = sel_lens;
  a.W = 1;
  a.Hq = num_q_heads;
  a.Hkv = kv->num_kv_heads;
  a.G = G;
  a.rows = G;
  a.num_pages = kv->num_pages;
  a.page_size = kv->page_size;
  a.max_pages = kv->max_pages;
  a.len_cap = max_kv_len;
  a.budget = budget;  // scored only when L > budget (snap_steps)
  a.budgets = nullptr;
  a.pool_kernel = 1;
  a.scale_log2 = 1.f;
  hipStream_t st = sdh::as_stream(stream);
  if (kv->head_dim == 128)
    launch_topk_attn_select<128>(a, batch, st);
  else
    launch_topk_attn_select<64>(a, batch, st);
  return sdh::launch_status();
}
