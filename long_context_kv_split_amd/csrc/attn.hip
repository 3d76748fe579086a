// Paged GQA attention for the verify pass and the sparse draft pass, gfx950.
//
// MagicDec (deep notes on papercache.org, §3.2) observes that at long context
// both verification and drafting are bound by loading the KV cache; the verify
// pass reads all of it for gamma+1 causal queries per sequence, the draft pass
// (§3.3, §4.1) reads only K selected tokens. One kernel template serves both:
// a "step" is 16 cached tokens, taken from consecutive positions of one page
// (verify) or from 16 entries of a selection list (draft).
//
// Schedule (persistent split-KV): the launch has exactly as many waves as the
// chip keeps resident for the instantiation. Each wave scans the device
// lengths itself (no plan launch) and takes the w-th equal share of the
// flattened (sequence, KV head, step) space, so the work is balanced to one
// step whatever the length mix, and writes one (m, l, o) partial per unit
// segment it covers into a slot table of at most waves + units entries. The
// assignment depends only on shapes and lengths, so results are bitwise
// reproducible. Verify waves take the unmasked steps of a segment in a
// permuted order (StepWalk), which reads pages laid out in order as fast as
// shuffled ones. A combine kernel merges each unit's partials by log-sum-exp;
// the call is two launches. Small calls (every unit in one round of the chip,
// at most 1024 tokens each, one 16-row tile) run one workgroup per unit
// instead, its waves merging in LDS: one launch.
//
// Per step a wave computes S^T = K Q^T with 16x16x32 bf16 MFMA (tokens on M,
// the G*n_q query rows of the KV head on N, padded to NB tiles of 16), applies
// the mask and an online softmax in the log2 domain, and accumulates
// O^T += V^T P^T with 16x16x16 bf16 MFMA. The accumulator layout of the first
// product is exactly the B-operand layout of the second, so P never leaves
// registers. V^T is formed from plain 16-byte row loads: lane (g, r) loads
// d-range [DPL*r, DPL*r+DPL) of tokens 4g..4g+3 and builds the A operand of
// d-tile dt from element dt of those four rows (v_perm), which assigns
// head-dim index DPL*m + dt to MFMA row m. float32 caches use the same
// structure with 16x16x4 f32 MFMA.
//
// A draft with one index set per query head (top-K attention, §4.4 of the
// notes) cannot share K/V loads across the group, so its units are (sequence,
// query head) with one query row each (G = 1), reading pool head h / G.
#include "sd_device.h"
#include "sd_host.h"
#include "sd_sched.h"

#include <algorithm>
#include <type_traits>

using namespace sdk;

namespace {

constexpr int kStepTokens = 16;
// Row-id table of a sub-chunk in LDS (8 KB): verify keeps one base row per
// step (the 16 tokens of a step are consecutive slots of one page), so a
// sub-chunk is up to 2048 steps; the draft keeps one row per token, 128 steps.
constexpr int kTableInts = 2048;
template <bool SPARSE>
constexpr int chunk_steps() {
  return SPARSE ? kTableInts / kStepTokens : kTableInts;
}
constexpr int kResolveBatch = 16;  // independent table lookups per lane in flight

struct AttnParams {
  const void *k_pages;
  const void *v_pages;
  const int32_t *page_table;
  const int32_t *lens;  // kv_lens (verify) or sel_lens (draft)
  const int32_t *idx;   // draft: [B, idx_heads, max_sel]
  const void *q;        // [B, n_q, Hq, D]
  Sched sc;             // schedule: wave count and the per-sequence step prefix (written by wave 0)
  float *part_o;        // [slots, rows, D]
  float *part_ml;       // [slots, rows, 2]
  // Units are (sequence, head) pairs: the KV heads (Hkv = pool heads, G query
  // heads each), or, for a draft with one index set per query head, the query
  // heads (Hkv = Hq, G = 1) reading pool head h / unit_div.
  int32_t B, n_q, Hq, Hkv, G, rows;
  int32_t pool_heads, unit_div;
  int32_t num_pages, page_size, max_pages;
  int32_t idx_heads, max_sel;
  int32_t len_cap;  // upper clamp of lens
  // draft only: positions [tail_begin[b], kv_lens[b]) read after the selection
  const int32_t *tail_begin;  // [B] or null (no tail)
  const int32_t *kv_lens;     // the cache's lengths (end of the tail)
  int32_t tail_cap;           // upper clamp of a tail's length
  float scale_log2;
};

// Tokens read for sequence b: the clamped length, plus the draft's tail.
__device__ __forceinline__ int tail_len(const AttnParams &a, int b) {
  return a.tail_begin ? clampi(a.kv_lens[b] - a.tail_begin[b], 0, a.tail_cap) : 0;
}
__device__ __forceinline__ int attn_len(const AttnParams &a, int b) {
  return clampi(a.lens[b], 0, a.len_cap) + tail_len(a, b);
}

template <typename T>
struct EltInfo;
template <>
struct EltInfo<__bf16> {
  static constexpr int bytes = 2;
};
template <>
struct EltInfo<float> {
  static constexpr int bytes = 4;
};

template <typename T, int D>
struct StepRegs {
  static constexpr int kBytesPerLane = D * EltInfo<T>::bytes / 4;  // per operand
  static constexpr int kVec = kBytesPerLane / 16;                   // u32x4 per operand
  static constexpr int kVDwords = D * EltInfo<T>::bytes / 64;       // dwords per V row slice
  u32x4 k[kVec];
  uint32_t v[4][kVDwords];
};

template <int N>
__device__ __forceinline__ void load_dwords(uint32_t (&dst)[N], const char *p) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p + 16 * i));
      dst[4 * i + 0] = t.x;
      dst[4 * i + 1] = t.y;
      dst[4 * i + 2] = t.z;
      dst[4 * i + 3] = t.w;
    }
  } else {
    static_assert(N == 2, "unsupported V slice");
    u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
    dst[0] = t.x;
    dst[1] = t.y;
  }
}

// Fill the sub-chunk's row table, rows (page * pool_heads + pkvh) * P + slot
// through the page table: for verify the first row of each of steps
// [sc_begin, sc_begin + n_steps); for the draft the row of each token of
// those steps (entry t of the selection, then the tail in order). Lookups go
// out kResolveBatch per lane before any is waited for, so a sub-chunk costs
// one or two memory round trips instead of one per token.
template <bool SPARSE>
__device__ __forceinline__ void resolve_rows(const AttnParams &a, int b, int pkvh, int sc_begin, int n_steps,
                                             int len, int sel, const int32_t *idx_row, int *rows) {
  const int lane = lane_id();
  const int32_t *pt = a.page_table + (size_t)b * a.max_pages;
  const int P = a.page_size;
  if constexpr (!SPARSE) {
    for (int k0 = 0; k0 < n_steps; k0 += 64 * kResolveBatch) {
      int e[kResolveBatch];
#pragma unroll
      for (int i = 0; i < kResolveBatch; ++i) {
        const int k = min(k0 + 64 * i + lane, n_steps - 1);
        e[i] = pt[clampi((sc_begin + k) * kStepTokens / P, 0, a.max_pages - 1)];
      }
#pragma unroll
      for (int i = 0; i < kResolveBatch; ++i) {
        const int k = k0 + 64 * i + lane;
        if (k < n_steps)
          rows[k] = (clampi(e[i], 0, a.num_pages - 1) * a.pool_heads + pkvh) * P + (sc_begin + k) * kStepTokens % P;
      }
    }
  } else {
    const int n_tok = n_steps * kStepTokens;
    const int t_base = sc_begin * kStepTokens;
    const int tail0 = a.tail_begin ? a.tail_begin[b] : 0;
    const int last_sel = max(sel - 1, 0);
    const int pos_cap = a.max_pages * P - 1;
    for (int t0 = 0; t0 < n_tok; t0 += 64 * kResolveBatch) {
      int pos[kResolveBatch];
#pragma unroll
      for (int i = 0; i < kResolveBatch; ++i) {
        const int t = clampi(t_base + t0 + 64 * i + lane, 0, len - 1);
        const int from_idx = idx_row[min(t, last_sel)];
        pos[i] = clampi(t < sel ? from_idx : tail0 + (t - sel), 0, pos_cap);
      }
      int e[kResolveBatch];
#pragma unroll
      for (int i = 0; i < kResolveBatch; ++i) e[i] = pt[pos[i] / P];
#pragma unroll
      for (int i = 0; i < kResolveBatch; ++i) {
        const int tt = t0 + 64 * i + lane;
        if (tt < n_tok) rows[tt] = (clampi(e[i], 0, a.num_pages - 1) * a.pool_heads + pkvh) * P + pos[i] % P;
      }
    }
  }
}

// Issue the K and V loads of one 16-token step whose row ids sit in LDS at
// rows[0..15]: K of token r for this lane's MFMA A operand, V of tokens
// 4g..4g+3 (the four ids are one 16-byte LDS read). K/V are streamed once per
// call, so the loads carry the nontemporal hint (measured: about 5% more read
// bandwidth than plain loads on this access pattern).
template <typename T, int D, bool SPARSE>
__device__ __forceinline__ void load_step(const AttnParams &a, const int *rows, StepRegs<T, D> &R) {
  constexpr int EB = EltInfo<T>::bytes;
  constexpr int DPL = D / 16;
  const int lane = lane_id();
  const int g = lane >> 4, r = lane & 15;
  int rowK;
  int4 rowV;
  if constexpr (SPARSE) {
    rowK = rows[r];
    rowV = *reinterpret_cast<const int4 *>(rows + 4 * g);
  } else {  // one page: the step's rows are base .. base + 15
    const int base = __builtin_amdgcn_readfirstlane(rows[0]);
    rowK = base + r;
    rowV = int4{base + 4 * g, base + 4 * g + 1, base + 4 * g + 2, base + 4 * g + 3};
  }
  const char *kb = reinterpret_cast<const char *>(a.k_pages) + (size_t)rowK * D * EB;
  if constexpr (EB == 2) {
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      R.k[kk] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kb + (32 * kk + 8 * g) * EB));
  } else {
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
      R.k[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kb + ((D / 4) * g + 4 * c) * EB));
  }
  const int rv[4] = {rowV.x, rowV.y, rowV.z, rowV.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const char *vb = reinterpret_cast<const char *>(a.v_pages) + ((size_t)rv[j] * D + DPL * r) * EB;
    load_dwords(R.v[j], vb);
  }
}

// max / sum over the four lanes l, l^16, l^32, l^48 (the four 16-lane rows)
__device__ __forceinline__ float rows4_max(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Per-wave state of the online softmax and the output accumulators.
template <typename T, int D, int NB>
struct AttnState {
  static constexpr int DPL = D / 16;
  static constexpr int QV = StepRegs<T, D>::kVec;
  u32x4 q[NB][QV];
  int lim[NB];
  f32x4 o[NB][DPL];
  float m[NB], l[NB];
};

// One 16-token step: scores, mask, online softmax, P V.
// MASK = false is only used for steps whose every token is visible to every
// query row (no causal limit, no tail of the sequence inside the step).
template <typename T, int D, int NB, bool SPARSE, bool MASK>
__device__ __forceinline__ void compute_step(const AttnParams &a, AttnState<T, D, NB> &st,
                                             StepRegs<T, D> &cur, int s, int len) {
  constexpr int EB = EltInfo<T>::bytes;
  constexpr int DPL = D / 16;
  constexpr int QV = StepRegs<T, D>::kVec;
  const int g = lane_id() >> 4;
  const int tok0 = s * kStepTokens;

  if constexpr (MASK) {  // zero V rows of tokens no row may see (they can hold NaN)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (tok0 + 4 * g + j >= len)
#pragma unroll
        for (int w = 0; w < StepRegs<T, D>::kVDwords; ++w) cur.v[j][w] = 0u;
  }

#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (EB == 2) {
#pragma unroll
      for (int c = 0; c < QV; ++c) sc = mfma_16x16x32_bf16(cur.k[c], st.q[rb][c], sc);
    } else {
      // (__uint_as_float, not __builtin_bit_cast: the latter applied to an
      // ext-vector element miscompiles to the first element with this clang)
#pragma unroll
      for (int c = 0; c < QV; ++c) {
        sc = mfma_16x16x4_f32(__uint_as_float(cur.k[c].x), __uint_as_float(st.q[rb][c].x), sc);
        sc = mfma_16x16x4_f32(__uint_as_float(cur.k[c].y), __uint_as_float(st.q[rb][c].y), sc);
        sc = mfma_16x16x4_f32(__uint_as_float(cur.k[c].z), __uint_as_float(st.q[rb][c].z), sc);
        sc = mfma_16x16x4_f32(__uint_as_float(cur.k[c].w), __uint_as_float(st.q[rb][c].w), sc);
      }
    }
    float p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = sc[e] * a.scale_log2;
    if constexpr (MASK) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (tok0 + 4 * g + e > st.lim[rb]) p[e] = kNegInf;
    }
    const float mx = rows4_max(fmaxf(fmaxf(p[0], p[1]), fmaxf(p[2], p[3])));
    const float m_new = fmaxf(st.m[rb], mx);
    if (__ballot(m_new > st.m[rb]) != 0) {
      const float alpha = (m_new == st.m[rb]) ? 1.f : __builtin_amdgcn_exp2f(st.m[rb] - m_new);
      st.l[rb] *= alpha;
#pragma unroll
      for (int dt = 0; dt < DPL; ++dt) st.o[rb][dt] *= alpha;
      st.m[rb] = m_new;
    }
    const float mu = (st.m[rb] == kNegInf) ? 0.f : st.m[rb];
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = __builtin_amdgcn_exp2f(p[e] - mu);
    st.l[rb] += (p[0] + p[1]) + (p[2] + p[3]);

    if constexpr (EB == 2) {
      const u32x2 pb = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
#pragma unroll
      for (int dt = 0; dt < DPL; ++dt) {
        const bool hi = dt & 1;
        const u32x2 av = {pick_halves(cur.v[0][dt / 2], cur.v[1][dt / 2], hi),
                          pick_halves(cur.v[2][dt / 2], cur.v[3][dt / 2], hi)};
        st.o[rb][dt] = mfma_16x16x16_bf16(av, pb, st.o[rb][dt]);
      }
    } else {
#pragma unroll
      for (int dt = 0; dt < DPL; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          st.o[rb][dt] = mfma_16x16x4_f32(__uint_as_float(cur.v[j][dt]), p[j], st.o[rb][dt]);
    }
  }
}

// Buffers in flight and occupancy per instantiation: bf16 with up to two row
// tiles keeps three steps of K/V in registers at two waves per SIMD; three row
// tiles keep two steps at two waves; larger tiles or fp32 run one wave.
template <typename T, int NB>
struct AttnTuning {
  static constexpr bool kBf16 = EltInfo<T>::bytes == 2;
  static constexpr int kBufs = (kBf16 && NB <= 2) ? 3 : 2;
  static constexpr int kWavesPerEU = (kBf16 && NB <= 3) ? 2 : 1;
};


__device__ __forceinline__ int unit_steps(const AttnParams &a, int b) {
  return (attn_len(a, b) + kStepTokens - 1) / kStepTokens;
}

// Each wave of a split kernel finds its own unit segments (no plan kernel);
// wave 0 also writes the per-sequence step prefix the combine reads.
template <class F>
__device__ __forceinline__ void attn_for_each_segment(const AttnParams &a, F &&f) {
  sched_inline_for_each_segment(a.B, a.Hkv, a.sc.waves, blockIdx.x, [&](int b) { return unit_steps(a, b); },
                                blockIdx.x == 0 ? a.sc.seq_prefix : nullptr, f);
}

template <typename T, int D, int NB, bool SPARSE>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(AttnTuning<T, NB>::kWavesPerEU)))
void attn_split_kernel(AttnParams a) {
  constexpr int EB = EltInfo<T>::bytes;
  constexpr int DPL = D / 16;
  constexpr int QV = StepRegs<T, D>::kVec;
  constexpr int NBUF = AttnTuning<T, NB>::kBufs;
  __shared__ __attribute__((aligned(16))) int rows_lds[kTableInts];
  const int lane = lane_id();
  const int g = lane >> 4, r = lane & 15;

  attn_for_each_segment(a, [&](int b, int kvh, int s_begin, int s_end, size_t slot) {
    const int len = attn_len(a, b);
    const int sel = clampi(a.lens[b], 0, a.len_cap);  // draft: entries of idx read before the tail
    const int pkvh = kvh / a.unit_div;                // pool head of the unit
    const int32_t *idx_row = nullptr;
    if constexpr (SPARSE)
      idx_row = a.idx + ((size_t)b * a.idx_heads + (a.idx_heads > 1 ? kvh : 0)) * a.max_sel;

    AttnState<T, D, NB> st;
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) {
      const int R = rb * 16 + r;
      int i = 0, hl = 0;
      const bool live = R < a.rows;
      if (live) {
        i = R / a.G;
        hl = R % a.G;
      }
      st.lim[rb] = SPARSE ? len - 1 : (live ? len - a.n_q + i : len - 1);
      const char *qb = reinterpret_cast<const char *>(a.q) +
                       ((((size_t)b * a.n_q + i) * a.Hq + (size_t)kvh * a.G + hl) * D) * EB;
#pragma unroll
      for (int c = 0; c < QV; ++c) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (live) {
          if constexpr (EB == 2)
            v = *reinterpret_cast<const u32x4 *>(qb + (32 * c + 8 * g) * EB);
          else
            v = *reinterpret_cast<const u32x4 *>(qb + ((D / 4) * g + 4 * c) * EB);
        }
        st.q[rb][c] = v;
      }
      st.m[rb] = kNegInf;
      st.l[rb] = 0.f;
#pragma unroll
      for (int dt = 0; dt < DPL; ++dt) st.o[rb][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int lim_min = SPARSE ? len - 1 : len - a.n_q;  // smallest limit of any real row

    // The segment is processed in sub-chunks of at most chunk_steps steps:
    // the row ids of a sub-chunk are resolved into LDS first, so that no K/V
    // load of the main loop waits on a dependent vector load.
    constexpr int kChunk = chunk_steps<SPARSE>();
    for (int sc_begin = s_begin; sc_begin < s_end; sc_begin += kChunk) {
      const int sc_end = min(s_end, sc_begin + kChunk);
      __syncthreads();  // the previous sub-chunk's table reads are done
      resolve_rows<SPARSE>(a, b, pkvh, sc_begin, sc_end - sc_begin, len, sel, idx_row, rows_lds);
      __syncthreads();
      // Main loop: groups of NBUF steps that need no mask, with a ring of NBUF
      // step buffers unrolled so every buffer has a fixed role and the loop
      // body is straight-line code (exact wait counts, NBUF-1 steps in flight).
      // Loads past the sub-chunk end repeat its last step (in bounds, cached).
      const int last = sc_end - sc_begin - 1;
      const int first_masked = lim_min >= 0 ? (lim_min + 1) / kStepTokens : 0;
      const int n_plain = max(0, min(sc_end, first_masked) - sc_begin);
      const int n_groups = n_plain / NBUF;
      auto rows_of = [&](int k) { return rows_lds + min(k, last) * (SPARSE ? kStepTokens : 1); };
      StepRegs<T, D> buf[NBUF];
      if (n_groups > 0) {
#pragma unroll
        for (int k = 0; k < NBUF - 1; ++k) load_step<T, D, SPARSE>(a, rows_of(k), buf[k]);
        for (int k0 = 0; k0 < n_groups * NBUF; k0 += NBUF) {
#pragma unroll
          for (int j = 0; j < NBUF; ++j) {
            load_step<T, D, SPARSE>(a, rows_of(k0 + j + NBUF - 1), buf[(j + NBUF - 1) % NBUF]);
            compute_step<T, D, NB, SPARSE, false>(a, st, buf[j], sc_begin + k0 + j, len);
          }
        }
      }
      // Tail: the remaining steps, one at a time, with the mask.
      for (int k = n_groups * NBUF; k <= last; ++k) {
        load_step<T, D, SPARSE>(a, rows_of(k), buf[0]);
        compute_step<T, D, NB, SPARSE, true>(a, st, buf[0], sc_begin + k, len);
      }
    }

    // Partial of this segment: unnormalised o (relative to m), (m, l) in log2 units.
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) {
      const int R = rb * 16 + r;
      const float l = rows4_sum(st.l[rb]);
      if (R < a.rows) {
        float *dst = a.part_o + (slot * a.rows + R) * D + 4 * DPL * g;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float vals[DPL];
#pragma unroll
          for (int dt = 0; dt < DPL; ++dt) vals[dt] = st.o[rb][dt][e];
#pragma unroll
          for (int v4 = 0; v4 < DPL; v4 += 4)
            *reinterpret_cast<f32x4 *>(dst + DPL * e + v4) =
                f32x4{vals[v4], vals[v4 + 1], vals[v4 + 2], vals[v4 + 3]};
        }
        if (g == 0) {
          a.part_ml[(slot * a.rows + R) * 2 + 0] = st.m[rb];
          a.part_ml[(slot * a.rows + R) * 2 + 1] = l;
        }
      }
    }
  });
}

// ---------------------------------------------------------------------------
// bf16 caches with head_dim 128: K and V streamed through a per-wave LDS ring.
//
// Every 16-token step is copied global -> LDS by asynchronous 16-byte copies
// (4 per lane for K, 4 for V), so loads in flight hold no registers and the
// wave decides its own waits: each step issues the same 8 copies, and
// "at most (kStreamRing - 1) * 8 newer vector-memory operations outstanding"
// means the step has landed (any other memory operation only makes that
// stricter). The ring is read with inline ds_read blocks that end in their
// own LDS wait, so the compiler adds no wait of its own for the copies.
// LDS layout of a step: K as 16 rows of 16 chunks with chunk c of token t at
// position c ^ t (the MFMA operand reads, 16 tokens x one chunk, fall in
// distinct banks), then V as 16 plain rows (the V^T operand reads four whole
// rows per instruction).
// Row ids: verify keeps the first row of each step (its 16 tokens share a
// page) in a 64-step register window, lane i holding step wb + i, read with
// readlane; the page-table entries of the window after next are copied into
// LDS one window early, so sliding the window never waits on a load issued in
// the same iteration. The draft resolves a sub-chunk of steps into an LDS
// table first, stored so that lane (g, r) finds the rows of tokens g, g + 4,
// g + 8, g + 12 (the tokens of its four copies) in one 16-byte read.
// Steps per wave in the LDS ring, and with it the resident waves: a deeper
// ring keeps more bytes in flight per wave but leaves room for fewer waves
// per CU. Four steps (four waves per CU, one per SIMD) for every tile count:
// e.g. the 8k-context batch 0.186 against 0.207 ms with two steps, the 70B
// shape 0.709 against 0.766 ms. Two tiles (20 query rows at gamma = 4) ran
// best with two steps (eight waves per CU) while waves walked their pages in
// order; with the permuted walk four steps are faster (2.49 against
// 2.53-2.54 ms at B = 128, 32k).
template <int NB>
constexpr int stream_ring() {
  return 4;
}
constexpr int kStreamChunks = 256;   // 16-byte chunks per 16-token step of one tensor (d = 128, bf16)
constexpr int kStreamWin = 64;       // steps per row window (verify)
constexpr int kSparseSubSteps = 48;  // draft row table: 48 steps x 16 tokens x 4 B = 3 KB

template <bool SPARSE, int RING>
struct StreamLayout {
  static constexpr int kRingBytes = RING * 2 * kStreamChunks * 16;
  static constexpr int kTableBytes = SPARSE ? kSparseSubSteps * kStepTokens * 4 : kStreamWin * 4;
  static constexpr int kBytes = kRingBytes + kTableBytes;
};

__device__ __forceinline__ int lds_read_i32(const lds_char *p) {
  int v = 0;
#if __HIP_DEVICE_COMPILE__
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"((uint32_t)(size_t)p) : "memory");
#endif
  return v;
}
__device__ __forceinline__ int4 lds_read_i32x4(const lds_char *p) {
  u32x4 v = {0u, 0u, 0u, 0u};
#if __HIP_DEVICE_COMPILE__
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"((uint32_t)(size_t)p) : "memory");
#endif
  return int4{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
}
__device__ __forceinline__ void lds_write_i32(lds_char *p, int v) {
#if __HIP_DEVICE_COMPILE__
  asm volatile("ds_write_b32 %0, %1" ::"v"((uint32_t)(size_t)p), "v"(v) : "memory");
#endif
}

// Operands of one step from ring slot `sl`: K chunk 4 kk + g of token r
// (MFMA A operand of S^T = K Q^T) and V d-range [8r, 8r + 8) of tokens
// 4g .. 4g + 3 (rows of the V^T operand).
__device__ __forceinline__ void stream_operands(const lds_u32x4 *ring, int sl, StepRegs<__bf16, 128> &cur) {
  const int lane = lane_id(), g = lane >> 4, r = lane & 15;
  const lds_u32x4 *kb = ring + sl * 2 * kStreamChunks;
  const lds_u32x4 *vb = kb + kStreamChunks;
  uint32_t ad[8];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) ad[kk] = (uint32_t)(size_t)(kb + r * 16 + ((4 * kk + g) ^ r));
#pragma unroll
  for (int j = 0; j < 4; ++j) ad[4 + j] = (uint32_t)(size_t)(vb + (4 * g + j) * 16 + r);
  u32x4 v[4];
#if __HIP_DEVICE_COMPILE__
  asm volatile(
      "ds_read_b128 %0, %8\n\tds_read_b128 %1, %9\n\tds_read_b128 %2, %10\n\tds_read_b128 %3, %11\n\t"
      "ds_read_b128 %4, %12\n\tds_read_b128 %5, %13\n\tds_read_b128 %6, %14\n\tds_read_b128 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(cur.k[0]), "=&v"(cur.k[1]), "=&v"(cur.k[2]), "=&v"(cur.k[3]), "=&v"(v[0]), "=&v"(v[1]),
        "=&v"(v[2]), "=&v"(v[3])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7])
      : "memory");
#endif
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    cur.v[j][0] = v[j].x;
    cur.v[j][1] = v[j].y;
    cur.v[j][2] = v[j].z;
    cur.v[j][3] = v[j].w;
  }
}

// One segment [s_begin, s_end) of unit (b, kvh) through this wave's LDS ring
// of RING steps at `lds` (Lay::kBytes): st ends holding the segment's (m, l, o).
template <int NB, bool SPARSE, int RING>
__device__ __forceinline__ void stream_segment(const AttnParams &a, lds_char *lds, int b, int kvh, int s_begin,
                                               int s_end, AttnState<__bf16, 128, NB> &st) {
  constexpr int D = 128;
  constexpr int QV = StepRegs<__bf16, D>::kVec;
  constexpr int DPL = D / 16;
  constexpr int kStreamRing = RING;
  using Lay = StreamLayout<SPARSE, kStreamRing>;
  lds_u32x4 *ring = (lds_u32x4 *)lds;
  lds_char *table = lds + Lay::kRingBytes;
  const int lane = lane_id();
  const int g = lane >> 4, r = lane & 15;
  const char *kp = reinterpret_cast<const char *>(a.k_pages);
  const char *vp = reinterpret_cast<const char *>(a.v_pages);
  s_begin = __builtin_amdgcn_readfirstlane(s_begin);
  s_end = __builtin_amdgcn_readfirstlane(s_end);
  const int len = __builtin_amdgcn_readfirstlane(attn_len(a, b));
  const int sel = clampi(a.lens[b], 0, a.len_cap);
  const int pkvh = kvh / a.unit_div;
  const int32_t *idx_row = nullptr;
  if constexpr (SPARSE)
    idx_row = a.idx + ((size_t)b * a.idx_heads + (a.idx_heads > 1 ? kvh : 0)) * a.max_sel;

#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
    const int R = rb * 16 + r;
    int i = 0, hl = 0;
    const bool live = R < a.rows;
    if (live) {
      i = R / a.G;
      hl = R % a.G;
    }
    st.lim[rb] = SPARSE ? len - 1 : (live ? len - a.n_q + i : len - 1);
    const char *qb = reinterpret_cast<const char *>(a.q) +
                     ((((size_t)b * a.n_q + i) * a.Hq + (size_t)kvh * a.G + hl) * D) * 2;
#pragma unroll
    for (int c = 0; c < QV; ++c) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (live) v = *reinterpret_cast<const u32x4 *>(qb + (32 * c + 8 * g) * 2);
      st.q[rb][c] = v;
    }
    st.m[rb] = kNegInf;
    st.l[rb] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DPL; ++dt) st.o[rb][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int lim_min = SPARSE ? len - 1 : len - a.n_q;  // smallest limit of any real row
  const int first_masked = lim_min >= 0 ? (lim_min + 1) / kStepTokens : 0;

  // this lane's chunk of copy i: token 4i + g, chunk position r (K: global chunk r ^ t)
  auto issue_rows = [&](int4 rows4, int sl) {
    lds_u32x4 *kd = ring + sl * 2 * kStreamChunks;
    const int rw[4] = {rows4.x, rows4.y, rows4.z, rows4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * i + g;
      lds_dma16(kp + (size_t)rw[i] * (D * 2) + ((r ^ t) & 15) * 16, kd + i * 64);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_dma16(vp + (size_t)rw[i] * (D * 2) + r * 16, kd + kStreamChunks + i * 64);
  };
  // the step's rows are base .. base + 15 (wave-uniform base): per-lane byte
  // offsets of the eight copies relative to row `base`
  auto issue_base = [&](int base, int sl) {
    lds_u32x4 *kd = ring + sl * 2 * kStreamChunks;
    const char *kb = kp + (size_t)base * (D * 2);
    const char *vb = vp + (size_t)base * (D * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * i + g;
      lds_dma16(kb + t * (D * 2) + ((r ^ t) & 15) * 16, kd + i * 64);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_dma16(vb + (4 * i + g) * (D * 2) + r * 16, kd + kStreamChunks + i * 64);
  };
  // one step: start the copies of step `ahead`, wait for step s, compute it
  auto step = [&](auto masked, int s, int sl, auto &&start_ahead) {
    start_ahead();
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kStreamRing - 1) * 8) : "memory");
    StepRegs<__bf16, D> cur;
    stream_operands(ring, sl, cur);
    compute_step<__bf16, D, NB, SPARSE, decltype(masked)::value>(a, st, cur, s, len);
  };
  using Plain = std::integral_constant<bool, false>;
  using Masked = std::integral_constant<bool, true>;

  if constexpr (!SPARSE) {
    // ------------------------------------------------------------- verify
    // The unmasked steps [s_begin, plain_end) are taken in a permuted order
    // (StepWalk) when there are at least kWalkMinSteps of them, the masked
    // steps follow in order. Loop indices below are positions v; phys(v) is
    // the step.
    const int32_t *pt = a.page_table + (size_t)b * a.max_pages;
    const int P = a.page_size;
    const int n_tot = s_end - s_begin;  // >= 1
    const int n_plain = max(0, min(s_end, first_masked) - s_begin);
    const StepWalk walk(n_plain >= kWalkMinSteps ? n_plain : 0, segment_hash(b, kvh, s_begin));
    auto phys = [&](int v) { return s_begin + walk(min(v, n_tot - 1)); };
    auto entry_ptr = [&](int v) { return pt + clampi(phys(v) * kStepTokens / P, 0, a.max_pages - 1); };
    auto row_from = [&](int entry, int v) {
      return (clampi(entry, 0, a.num_pages - 1) * a.pool_heads + pkvh) * P + phys(v) * kStepTokens % P;
    };
    int wb = 0;
    int rows_a = row_from(*entry_ptr(wb + lane), wb + lane);
    int rows_b = row_from(*entry_ptr(wb + kStreamWin + lane), wb + kStreamWin + lane);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the table of a previous segment is free
    lds_dma4(entry_ptr(wb + 2 * kStreamWin + lane), (__attribute__((address_space(3))) void *)table);
    auto base_of = [&](int v) {
      const int d = v - wb;
      return d < kStreamWin ? __builtin_amdgcn_readlane(rows_a, d) : __builtin_amdgcn_readlane(rows_b, d - kStreamWin);
    };
    auto issue_step = [&](int v, int sl) { issue_base(base_of(min(v, n_tot - 1)), sl); };
    auto ahead = [&](int v) {
      return [&, v] {
        if (v - wb == kStreamWin) {
          // entries of this window were requested kStreamWin steps ago and
          // waited for since (every step waits for its own copies)
          wb += kStreamWin;
          rows_a = rows_b;
          rows_b = row_from(lds_read_i32(table + 4 * lane), wb + kStreamWin + lane);
          lds_dma4(entry_ptr(wb + 2 * kStreamWin + lane), (__attribute__((address_space(3))) void *)table);
        }
        issue_step(v + kStreamRing - 1, (v + kStreamRing - 1) % kStreamRing);
      };
    };
#pragma unroll
    for (int i = 0; i < kStreamRing - 1; ++i) issue_step(i, i);
    for (int v = 0; v < n_plain; ++v) step(Plain{}, phys(v), v % kStreamRing, ahead(v));
    for (int v = n_plain; v < n_tot; ++v) step(Masked{}, s_begin + v, v % kStreamRing, ahead(v));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // copies into the ring or table have landed
  } else {
    // -------------------------------------------------------------- draft
    const int32_t *pt = a.page_table + (size_t)b * a.max_pages;
    const int P = a.page_size;
    const int tail0 = a.tail_begin ? a.tail_begin[b] : 0;
    const int last_sel = max(sel - 1, 0);
    const int pos_cap = a.max_pages * P - 1;
    for (int sc_begin = s_begin; sc_begin < s_end; sc_begin += kSparseSubSteps) {
      const int sc_end = min(s_end, sc_begin + kSparseSubSteps);
      const int n_tok = (sc_end - sc_begin) * kStepTokens;
      // rows of the sub-chunk's tokens; token t of step k at table entry
      // 16k + 4 (t % 4) + t / 4, so lane g reads tokens g, g+4, g+8, g+12 at 16k + 4g
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // previous copies have landed
      for (int t0 = 0; t0 < n_tok; t0 += 64 * kResolveBatch) {
        int pos[kResolveBatch];
#pragma unroll
        for (int i = 0; i < kResolveBatch; ++i) {
          const int t = clampi(sc_begin * kStepTokens + t0 + 64 * i + lane, 0, len - 1);
          const int from_idx = idx_row[min(t, last_sel)];
          pos[i] = clampi(t < sel ? from_idx : tail0 + (t - sel), 0, pos_cap);
        }
        int e[kResolveBatch];
#pragma unroll
        for (int i = 0; i < kResolveBatch; ++i) e[i] = pt[pos[i] / P];
#pragma unroll
        for (int i = 0; i < kResolveBatch; ++i) {
          const int tt = t0 + 64 * i + lane;
          if (tt < n_tok) {
            const int k = tt / kStepTokens, t = tt % kStepTokens;
            lds_write_i32(table + 4 * (k * kStepTokens + 4 * (t % 4) + t / 4),
                          (clampi(e[i], 0, a.num_pages - 1) * a.pool_heads + pkvh) * P + pos[i] % P);
          }
        }
      }
      const int last_k = sc_end - sc_begin - 1;
      auto issue_step = [&](int k, int sl) {
        issue_rows(lds_read_i32x4(table + 4 * (min(k, last_k) * kStepTokens + 4 * g)), sl);
      };
      auto ahead = [&](int k) { return [&, k] { issue_step(k + kStreamRing - 1, (k + kStreamRing - 1) % kStreamRing); }; };
#pragma unroll
      for (int i = 0; i < kStreamRing - 1; ++i) issue_step(i, i % kStreamRing);
      const int plain_end = max(0, min(last_k + 1, first_masked - sc_begin));
      for (int k = 0; k < plain_end; ++k) step(Plain{}, sc_begin + k, k % kStreamRing, ahead(k));
      for (int k = plain_end; k <= last_k; ++k) step(Masked{}, sc_begin + k, k % kStreamRing, ahead(k));
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
  }
}

template <int NB, bool SPARSE, int RING>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(NB <= 3 ? 2 : 1)))
void attn_stream_kernel(AttnParams a) {
  constexpr int D = 128;
  constexpr int DPL = D / 16;
  using Lay = StreamLayout<SPARSE, RING>;
  __shared__ __attribute__((aligned(16))) char lds_raw[Lay::kBytes];
  const int g = lane_id() >> 4, r = lane_id() & 15;

  attn_for_each_segment(a, [&](int b, int kvh, int s_begin, int s_end, size_t slot) {
    AttnState<__bf16, D, NB> st;
    stream_segment<NB, SPARSE, RING>(a, (lds_char *)lds_raw, b, kvh, s_begin, s_end, st);

    // Partial of this segment: unnormalised o (relative to m), (m, l) in log2 units.
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) {
      const int R = rb * 16 + r;
      const float l = rows4_sum(st.l[rb]);
      if (R < a.rows) {
        float *dst = a.part_o + (slot * a.rows + R) * D + 4 * DPL * g;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float vals[DPL];
#pragma unroll
          for (int dt = 0; dt < DPL; ++dt) vals[dt] = st.o[rb][dt][e];
#pragma unroll
          for (int v4 = 0; v4 < DPL; v4 += 4)
            *reinterpret_cast<f32x4 *>(dst + DPL * e + v4) =
                f32x4{vals[v4], vals[v4 + 1], vals[v4 + 2], vals[v4 + 3]};
        }
        if (g == 0) {
          a.part_ml[(slot * a.rows + R) * 2 + 0] = st.m[rb];
          a.part_ml[(slot * a.rows + R) * 2 + 1] = l;
        }
      }
    }
  });
}

// Small calls (every unit fits one round of the chip and is short): one
// workgroup per unit, its kUnitWaves waves splitting the unit's steps evenly.
// Each wave leaves its segment's (m, l, o) in its own LDS region; the waves
// then merge them by log-sum-exp and write the output. One launch, no length
// scan across the batch and no partials in global memory. One 16-row tile.
constexpr int kUnitWaves = 4;
constexpr int kUnitMaxSteps = 64;  // steps per unit that the unit kernel takes

template <bool SPARSE>
__global__ __launch_bounds__(64 * kUnitWaves) void attn_unit_kernel(AttnParams a, void *out, float *lse) {
  constexpr int NB = 1, D = 128, DPL = D / 16;
  using Lay = StreamLayout<SPARSE, stream_ring<NB>()>;
  static_assert(16 * (D + 2) * 4 <= Lay::kBytes, "a wave's partial fits its LDS region");
  __shared__ __attribute__((aligned(16))) char lds_raw[kUnitWaves * Lay::kBytes];
  const int wv = threadIdx.x >> 6, lane = lane_id();
  const int g = lane >> 4, r = lane & 15;
  const int u = blockIdx.x;
  const int b = u / a.Hkv, kvh = u % a.Hkv;
  const int n = unit_steps(a, b);
  const int s0 = n * wv / kUnitWaves, s1 = n * (wv + 1) / kUnitWaves;
  lds_char *mine = (lds_char *)lds_raw + wv * Lay::kBytes;
  AttnState<__bf16, D, NB> st;
  if (s0 < s1) {
    stream_segment<NB, SPARSE, stream_ring<NB>()>(a, mine, b, kvh, s0, s1, st);
  } else {
    st.m[0] = kNegInf;
    st.l[0] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DPL; ++dt) st.o[0][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // this wave's partial into its region: row R's o at R * D (the layout of
  // the global partials), (m, l) after the 16 rows
  float *po = reinterpret_cast<float *>(lds_raw + wv * Lay::kBytes);
  const float l = rows4_sum(st.l[0]);
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int dt = 0; dt < DPL; ++dt) po[r * D + 4 * DPL * g + DPL * e + dt] = st.o[0][dt][e];
  if (g == 0) {
    po[16 * D + 2 * r] = st.m[0];
    po[16 * D + 2 * r + 1] = l;
  }
  __syncthreads();
  // wave wv merges rows 4 wv .. 4 wv + 3: 16 lanes per row, 8 elements each
  const int R = 4 * wv + g, sub = r;
  if (R >= a.rows) return;
  float M = kNegInf;
#pragma unroll
  for (int k = 0; k < kUnitWaves; ++k) M = fmaxf(M, reinterpret_cast<const float *>(lds_raw + k * Lay::kBytes)[16 * D + 2 * R]);
  float o[DPL] = {};
  float L = 0.f;
  if (M != kNegInf) {
#pragma unroll
    for (int k = 0; k < kUnitWaves; ++k) {
      const float *pk = reinterpret_cast<const float *>(lds_raw + k * Lay::kBytes);
      const float mk = pk[16 * D + 2 * R];
      const float w = mk == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mk - M);
      L += w * pk[16 * D + 2 * R + 1];
#pragma unroll
      for (int j = 0; j < DPL; ++j) o[j] += w * pk[R * D + DPL * sub + j];
    }
  }
  const int i = R / a.G, hl = R % a.G;
  const size_t orow = (((size_t)b * a.n_q + i) * a.Hq + (size_t)kvh * a.G + hl);
  const bool empty = !(L > 0.f);
  const float inv = empty ? 0.f : 1.f / L;
  uint32_t pk[DPL / 2];
#pragma unroll
  for (int k = 0; k < DPL / 2; ++k) pk[k] = pack_bf16x2(o[2 * k] * inv, o[2 * k + 1] * inv);
  *reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(out) + orow * D + sub * DPL) =
      u32x4{pk[0], pk[1], pk[2], pk[3]};
  if (lse != nullptr && sub == 0) lse[orow] = empty ? kNegInf : (M + __log2f(L)) * kLn2;
}

// Merge each unit's partials by log-sum-exp. One wave takes four output
// rows (b, kvh, 4 q .. 4 q + 3) of a unit, 16 lanes per row, each lane D / 16
// elements of o: lane j of a row's group holds the (m, l) of the unit's slot
// j0 + j, so the slots' statistics arrive in one round trip, and the o
// partials of four slots are loaded together before they are summed (slot
// order, each slot's weight taken from the lane that holds it).
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnParams a, void *out, float *lse,
                                                           int total_groups) {
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wave >= total_groups) return;
  const int lane = lane_id();
  const int gl = lane >> 4, sub = lane & 15;
  const int row_groups = (a.rows + 3) / 4;
  const int u = wave / row_groups;
  const int R = (wave % row_groups) * 4 + gl;
  const bool live = R < a.rows;
  const int Rc = live ? R : a.rows - 1;  // padding lanes repeat the last row, write nothing
  const int kvh = u % a.Hkv;
  const int b = u / a.Hkv;
  int s0, s1;
  sched_inline_unit_slots(a.sc.seq_prefix, a.B, a.Hkv, a.sc.waves, b, kvh, s0, s1);
  const int ns = s1 - s0;

  float M = kNegInf;
  for (int j0 = 0; j0 < ns; j0 += 16)
    if (j0 + sub < ns) M = fmaxf(M, a.part_ml[((size_t)(s0 + j0 + sub) * a.rows + Rc) * 2]);
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
  constexpr int PER = D / 16;  // elements of o per lane
  float o[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) o[k] = 0.f;
  float L = 0.f;
  if (M != kNegInf) {
    for (int j0 = 0; j0 < ns; j0 += 16) {
      float w = 0.f;
      if (j0 + sub < ns) {
        const size_t base = (size_t)(s0 + j0 + sub) * a.rows + Rc;
        const float mc = a.part_ml[base * 2];
        w = mc == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mc - M);
        L += w * a.part_ml[base * 2 + 1];
      }
      const int cnt = min(16, ns - j0);
      for (int k0 = 0; k0 < cnt; k0 += 4) {
        f32x4 v[4][PER / 4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const size_t base = (size_t)(s0 + j0 + min(k0 + q, cnt - 1)) * a.rows + Rc;
#pragma unroll
          for (int c = 0; c < PER / 4; ++c)
            v[q][c] = *reinterpret_cast<const f32x4 *>(a.part_o + base * D + sub * PER + 4 * c);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float wq = __shfl(w, 16 * gl + k0 + q, 64);
          if (k0 + q < cnt) {
#pragma unroll
            for (int c = 0; c < PER / 4; ++c)
#pragma unroll
              for (int e = 0; e < 4; ++e) o[4 * c + e] += wq * v[q][c][e];
          }
        }
      }
    }
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) L += __shfl_xor(L, m, 64);
  if (!live) return;
  const int i = R / a.G, hl = R % a.G;
  const size_t orow = (((size_t)b * a.n_q + i) * a.Hq + (size_t)kvh * a.G + hl);
  const bool empty = !(L > 0.f);
  const float inv = empty ? 0.f : 1.f / L;
  if constexpr (EltInfo<T>::bytes == 2) {
    uint32_t pk[PER / 2];
#pragma unroll
    for (int k = 0; k < PER / 2; ++k) pk[k] = pack_bf16x2(o[2 * k] * inv, o[2 * k + 1] * inv);
    uint16_t *dst = reinterpret_cast<uint16_t *>(out) + orow * D + sub * PER;
    if constexpr (PER == 8)
      *reinterpret_cast<u32x4 *>(dst) = u32x4{pk[0], pk[1], pk[2], pk[3]};
    else
      *reinterpret_cast<u32x2 *>(dst) = u32x2{pk[0], pk[1]};
  } else {
    float *dst = reinterpret_cast<float *>(out) + orow * D + sub * PER;
#pragma unroll
    for (int c = 0; c < PER / 4; ++c)
      *reinterpret_cast<f32x4 *>(dst + 4 * c) = f32x4{o[4 * c] * inv, o[4 * c + 1] * inv, o[4 * c + 2] * inv,
                                                      o[4 * c + 3] * inv};
  }
  if (lse != nullptr && sub == 0) lse[orow] = empty ? kNegInf : (M + __log2f(L)) * kLn2;
}

// Workspace: prefix tables, then the partial slots. Sized for the largest
// launch (kMaxWaves) so that the size depends on shapes only.
struct WsLayout {
  size_t ml_off, o_off, bytes;
};

WsLayout ws_layout(int64_t B, int64_t Hkv, int64_t rows, int64_t D) {
  WsLayout l;
  const int64_t slots = sdh::sched_max_slots(B, Hkv);
  l.ml_off = sdh::sched_table_bytes(B, Hkv);
  l.o_off = l.ml_off + sdh::align_up((size_t)slots * rows * 2 * 4);
  l.bytes = l.o_off + sdh::align_up((size_t)slots * rows * D * 4);
  return l;
}

template <typename T, int D, int NB, bool SPARSE>
sd_status launch_nb(AttnParams &a, void *out, float *lse, hipStream_t st) {
  // bf16 with head_dim 128 streams K/V through the LDS ring; fp32 caches and
  // head_dim 64 use the register ring
  constexpr bool kStream = EltInfo<T>::bytes == 2 && D == 128;
  constexpr int kRing = stream_ring<NB>();
  const void *kernel = kStream ? reinterpret_cast<const void *>(attn_stream_kernel<NB, SPARSE, kRing>)
                               : reinterpret_cast<const void *>(attn_split_kernel<T, D, NB, SPARSE>);
  if constexpr (kStream && NB == 1) {
    // every unit in one round of the chip, each short: one workgroup per unit
    const int64_t units = (int64_t)a.B * a.Hkv;
    if (units <= kNumCUs && (int64_t)a.len_cap + a.tail_cap <= (int64_t)kUnitMaxSteps * kStepTokens) {
      attn_unit_kernel<SPARSE><<<(unsigned)units, 64 * kUnitWaves, 0, st>>>(a, out, lse);
      return sdh::launch_status();
    }
  }
  static int cache[sdh::kMaxDevices] = {};  // resident waves of this instantiation per device
  a.sc.waves = sdh::resident_waves(kernel, kSimdsPerCU * AttnTuning<T, NB>::kWavesPerEU, cache);
  if constexpr (kStream && NB == 1 && SPARSE) {
    // Drafts with more units than the four-step ring has resident waves (the
    // ragged batch's 2048 units and more) run with two-step rings: twice the
    // waves fit, one unit each where the four-step grid would give a wave
    // two. One tile at four steps stays for the rest (1024 units of the
    // 32k batch: every wave one unit either way).
    const int64_t units = (int64_t)a.B * a.Hkv;
    if (units > a.sc.waves) {
      static int cache2[sdh::kMaxDevices] = {};
      a.sc.waves = sdh::resident_waves(reinterpret_cast<const void *>(attn_stream_kernel<1, true, 2>),
                                       kSimdsPerCU * AttnTuning<T, NB>::kWavesPerEU, cache2);
      attn_stream_kernel<1, true, 2><<<(unsigned)a.sc.waves, 64, 0, st>>>(a);
    } else {
      attn_stream_kernel<1, true, kRing><<<(unsigned)a.sc.waves, 64, 0, st>>>(a);
    }
  } else if constexpr (kStream)
    attn_stream_kernel<NB, SPARSE, kRing><<<(unsigned)a.sc.waves, 64, 0, st>>>(a);
  else
    attn_split_kernel<T, D, NB, SPARSE><<<(unsigned)a.sc.waves, 64, 0, st>>>(a);
  const int total_groups = a.B * a.Hkv * ((a.rows + 3) / 4);
  attn_combine_kernel<T, D><<<(total_groups + 3) / 4, 256, 0, st>>>(a, out, lse, total_groups);
  return sdh::launch_status();
}

template <typename T, int D, bool SPARSE>
sd_status launch_attn(AttnParams &a, void *out, float *lse, hipStream_t st) {
  switch ((a.rows + 15) / 16) {
    case 1: return launch_nb<T, D, 1, SPARSE>(a, out, lse, st);
    case 2: return launch_nb<T, D, 2, SPARSE>(a, out, lse, st);
    case 3: return launch_nb<T, D, 3, SPARSE>(a, out, lse, st);
    case 4: return launch_nb<T, D, 4, SPARSE>(a, out, lse, st);
    default: return SD_ERR_UNSUPPORTED;
  }
}

template <bool SPARSE>
sd_status run_attn(AttnParams &a, int D, int dtype, void *out, float *lse, hipStream_t st) {
  if (dtype == SD_BF16) {
    if (D == 128) return launch_attn<__bf16, 128, SPARSE>(a, out, lse, st);
    return launch_attn<__bf16, 64, SPARSE>(a, out, lse, st);
  }
  if (D == 128) return launch_attn<float, 128, SPARSE>(a, out, lse, st);
  return launch_attn<float, 64, SPARSE>(a, out, lse, st);
}

sd_status common_checks(const sd_kv_cache *kv, const void *q, int32_t batch, int32_t n_q,
                        int32_t num_q_heads, float softmax_scale, void *out) {
  sd_status s = sdh::check_kv(kv, true);
  if (s != SD_OK) return s;
  SD_REQUIRE(q != nullptr && out != nullptr, SD_ERR_INVALID_ARG);
  SD_REQUIRE(sdh::aligned16(q) && sdh::aligned16(out), SD_ERR_INVALID_ARG);
  SD_REQUIRE(batch > 0 && n_q > 0 && num_q_heads > 0, SD_ERR_INVALID_ARG);
  SD_REQUIRE(num_q_heads % kv->num_kv_heads == 0, SD_ERR_INVALID_ARG);
  SD_REQUIRE((int64_t)(num_q_heads / kv->num_kv_heads) * n_q <= 64, SD_ERR_UNSUPPORTED);
  SD_REQUIRE(softmax_scale > 0.f && softmax_scale * kLog2e < __builtin_inff(), SD_ERR_INVALID_ARG);
  SD_REQUIRE((int64_t)batch * kv->num_kv_heads + kMaxWaves < ((int64_t)1 << 30), SD_ERR_UNSUPPORTED);
  return SD_OK;
}

// per_query_head: one unit per (sequence, query head) instead of per KV head.
void fill_common(AttnParams &a, const sd_kv_cache *kv, const void *q, int32_t batch, int32_t n_q,
                 int32_t num_q_heads, float softmax_scale, void *workspace, const WsLayout &l,
                 bool per_query_head) {
  char *ws = reinterpret_cast<char *>(workspace);
  const int G = num_q_heads / kv->num_kv_heads;
  a.k_pages = kv->k_pages;
  a.v_pages = kv->v_pages;
  a.page_table = kv->page_table;
  a.q = q;
  a.B = batch;
  a.n_q = n_q;
  a.Hq = num_q_heads;
  a.Hkv = per_query_head ? num_q_heads : kv->num_kv_heads;
  a.G = per_query_head ? 1 : G;
  a.rows = a.G * n_q;
  a.pool_heads = kv->num_kv_heads;
  a.unit_div = per_query_head ? G : 1;
  sdh::sched_bind(a.sc, ws, batch, a.Hkv);
  a.part_ml = reinterpret_cast<float *>(ws + l.ml_off);
  a.part_o = reinterpret_cast<float *>(ws + l.o_off);
  a.num_pages = kv->num_pages;
  a.page_size = kv->page_size;
  a.max_pages = kv->max_pages;
  a.scale_log2 = softmax_scale * kLog2e;
}

}  // namespace

extern "C" size_t sd_verify_attn_workspace_size(int32_t batch, int32_t n_q, int32_t num_q_heads,
                                                int32_t num_kv_heads, int32_t head_dim,
                                                int32_t max_kv_len) {
  if (batch <= 0 || n_q <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_kv_len < 0 || num_q_heads % num_kv_heads != 0)
    return 0;
  return ws_layout(batch, num_kv_heads, num_q_heads / num_kv_heads * n_q, head_dim).bytes;
}

extern "C" sd_status sd_verify_attn(const sd_kv_cache *kv, const void *q, int32_t batch, int32_t n_q,
                                    int32_t num_q_heads, int32_t max_kv_len, float softmax_scale,
                                    void *out, float *lse, void *workspace, size_t workspace_bytes,
                                    void *stream) {
  sd_status s = common_checks(kv, q, batch, n_q, num_q_heads, softmax_scale, out);
  if (s != SD_OK) return s;
  SD_REQUIRE(max_kv_len >= 0 && (int64_t)max_kv_len <= (int64_t)kv->max_pages * kv->page_size,
             SD_ERR_INVALID_ARG);
  // the schedule keeps per-sequence step prefix sums in int32
  SD_REQUIRE((int64_t)batch * sdh::ceil_div(max_kv_len, 16) < ((int64_t)1 << 31), SD_ERR_UNSUPPORTED);
  const WsLayout l = ws_layout(batch, kv->num_kv_heads, num_q_heads / kv->num_kv_heads * n_q, kv->head_dim);
  SD_REQUIRE(workspace != nullptr && workspace_bytes >= l.bytes, SD_ERR_WORKSPACE);
  AttnParams a{};
  fill_common(a, kv, q, batch, n_q, num_q_heads, softmax_scale, workspace, l, false);
  a.lens = kv->kv_lens;
  a.idx = nullptr;
  a.idx_heads = 1;
  a.max_sel = 0;
  a.len_cap = max_kv_len;
  return run_attn<false>(a, kv->head_dim, kv->dtype, out, lse, sdh::as_stream(stream));
}

extern "C" size_t sd_draft_attn_sparse_workspace_size(int32_t batch, int32_t n_q,
                                                      int32_t num_q_heads, int32_t num_kv_heads,
                                                      int32_t head_dim, int32_t max_sel) {
  // enough for units per KV head and, with idx_heads = num_q_heads, per query head
  const size_t per_kv = sd_verify_attn_workspace_size(batch, n_q, num_q_heads, num_kv_heads, head_dim, max_sel);
  if (per_kv == 0) return 0;
  return std::max(per_kv, ws_layout(batch, num_q_heads, n_q, head_dim).bytes);
}

namespace {

sd_status draft_impl(const sd_kv_cache *kv, const void *q, int32_t batch, int32_t n_q, int32_t num_q_heads,
                     const int32_t *idx, const int32_t *sel_lens, int32_t idx_heads, int32_t max_sel,
                     const int32_t *tail_begin, int32_t max_tail, float softmax_scale, void *out, float *lse,
                     void *workspace, size_t workspace_bytes, void *stream) {
  sd_status s = common_checks(kv, q, batch, n_q, num_q_heads, softmax_scale, out);
  if (s != SD_OK) return s;
  SD_REQUIRE(idx != nullptr && sel_lens != nullptr, SD_ERR_INVALID_ARG);
  SD_REQUIRE(idx_heads == 1 || idx_heads == kv->num_kv_heads || idx_heads == num_q_heads, SD_ERR_INVALID_ARG);
  SD_REQUIRE(max_sel > 0 && max_tail >= 0, SD_ERR_INVALID_ARG);
  SD_REQUIRE((int64_t)max_tail <= (int64_t)kv->max_pages * kv->page_size, SD_ERR_INVALID_ARG);
  SD_REQUIRE((int64_t)batch * sdh::ceil_div((int64_t)max_sel + max_tail, 16) < ((int64_t)1 << 31),
             SD_ERR_UNSUPPORTED);
  // one index set per query head (top-K attention): units per query head
  const bool per_query_head = idx_heads == num_q_heads && num_q_heads != kv->num_kv_heads;
  SD_REQUIRE((int64_t)batch * num_q_heads + kMaxWaves < ((int64_t)1 << 30), SD_ERR_UNSUPPORTED);
  const WsLayout l = per_query_head
                         ? ws_layout(batch, num_q_heads, n_q, kv->head_dim)
                         : ws_layout(batch, kv->num_kv_heads, num_q_heads / kv->num_kv_heads * n_q, kv->head_dim);
  SD_REQUIRE(workspace != nullptr && workspace_bytes >= l.bytes, SD_ERR_WORKSPACE);
  AttnParams a{};
  fill_common(a, kv, q, batch, n_q, num_q_heads, softmax_scale, workspace, l, per_query_head);
  a.lens = sel_lens;
  a.idx = idx;
  a.idx_heads = idx_heads;
  a.max_sel = max_sel;
  a.len_cap = max_sel;
  a.tail_begin = tail_begin;
  a.kv_lens = kv->kv_lens;
  a.tail_cap = max_tail;
  return run_attn<true>(a, kv->head_dim, kv->dtype, out, lse, sdh::as_stream(stream));
}

}  // namespace

extern "C" sd_status sd_draft_attn_sparse(const sd_kv_cache *kv, const void *q, int32_t batch,
                                          int32_t n_q, int32_t num_q_heads, const int32_t *idx,
                                          const int32_t *sel_lens, int32_t idx_heads,
                                          int32_t max_sel, float softmax_scale, void *out,
                                          float *lse, void *workspace, size_t workspace_bytes,
                                          void *stream) {
  return draft_impl(kv, q, batch, n_q, num_q_heads, idx, sel_lens, idx_heads, max_sel, nullptr, 0,
                    softmax_scale, out, lse, workspace, workspace_bytes, stream);
}

extern "C" sd_status sd_draft_attn_sparse_tail(const sd_kv_cache *kv, const void *q, int32_t batch,
                                               int32_t n_q, int32_t num_q_heads, const int32_t *idx,
                                               const int32_t *sel_lens, int32_t idx_heads,
                                               int32_t max_sel, const int32_t *tail_begin,
                                               int32_t max_tail, float softmax_scale, void *out,
                                               float *lse, void *workspace, size_t workspace_bytes,
                                               void *stream) {
  SD_REQUIRE(tail_begin != nullptr, SD_ERR_INVALID_ARG);
  return draft_impl(kv, q, batch, n_q, num_q_heads, idx, sel_lens, idx_heads, max_sel, tail_begin, max_tail,
                    softmax_scale, out, lse, workspace, workspace_bytes, stream);
}
