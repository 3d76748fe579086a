// Persistent, balanced split of a batch of (sequence, KV head) units over the
// resident waves of one kernel launch. Used by the attention kernels and the
// SnapKV scoring passes.
//
// Each unit u = b*Hkv + kvh owns n_b steps (n_b depends on the sequence only)
// and the units are flattened b-major into [0, T), T = Hkv * sum_b n_b. With W
// working waves, wave w owns the steps {t : floor(t*W/T) == w}, a contiguous
// range of length floor(T/W) or ceil(T/W): balanced to one step whatever the
// length mix, and fixed by the shapes and lengths alone (deterministic).
// Because W <= T, every wave in [floor(A*W/T), floor((A+n-1)*W/T)] of a unit
// with steps [A, A+n) owns at least one of them, so the unit's partial results
// occupy a dense run of slots starting at slot_base[u]; the slot table has at
// most W + units entries.
#pragma once

#include "sd_device.h"
#include "sd_host.h"

namespace sdk {

constexpr int kNumCUs = 256;  // MI355X
constexpr int kSimdsPerCU = 4;
constexpr int kMaxWaves = kNumCUs * kSimdsPerCU * 8;  // bound used to size slot tables
constexpr int kPlanThreads = 1024;
constexpr int kMinStepsPerWave = 8;  // a partial covers at least 8 steps when there is work

struct Sched {
  int32_t *seq_prefix;  // [B + 1]: steps of the sequences before b
  int32_t *slot_base;   // [B * Hkv + 1]: first partial slot of each unit
  int32_t B, Hkv, waves;
};

// Waves that get work: at most the launched waves and never more than
// T / kMinStepsPerWave (so W <= T).
__device__ __forceinline__ int64_t sched_working_waves(const Sched &s, int64_t T) {
  return max<int64_t>(1, min<int64_t>(s.waves, (T + kMinStepsPerWave - 1) / kMinStepsPerWave));
}

// First and last wave (inclusive) owning steps of a unit with steps [A, A+n), n >= 1.
__device__ __forceinline__ void sched_unit_waves(int64_t A, int64_t n, int64_t T, int64_t W,
                                                 int64_t &lo, int64_t &hi) {
  lo = A * W / T;
  hi = (A + n - 1) * W / T;
}

// Block-wide exclusive scan (kPlanThreads threads) with a carried offset.
__device__ __forceinline__ int64_t sched_block_scan(int64_t v, int64_t *lds, int64_t &carry) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int64_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) lds[wave] = x;
  __syncthreads();
  int64_t before = carry;
  for (int w = 0; w < wave; ++w) before += lds[w];
  int64_t total = 0;
  for (int w = 0; w < kPlanThreads / 64; ++w) total += lds[w];
  __syncthreads();
  carry += total;
  return before + x - v;
}

// Plan body for a one-block kernel of kPlanThreads threads. steps(b) = n_b.
template <class StepsFn>
__device__ __forceinline__ void sched_plan(const Sched &s, StepsFn steps) {
  __shared__ int64_t lds[kPlanThreads / 64];
  int64_t carry = 0;
  for (int base = 0; base < s.B; base += kPlanThreads) {
    const int b = base + threadIdx.x;
    const int64_t n = b < s.B ? (int64_t)steps(b) : 0;
    const int64_t ex = sched_block_scan(n, lds, carry);
    if (b < s.B) s.seq_prefix[b] = (int32_t)ex;
  }
  if (threadIdx.x == 0) s.seq_prefix[s.B] = (int32_t)carry;
  __syncthreads();
  const int64_t T = (int64_t)s.Hkv * carry;
  const int64_t W = sched_working_waves(s, T);
  const int U = s.B * s.Hkv;
  int64_t slots = 0;
  for (int base = 0; base < U; base += kPlanThreads) {
    const int u = base + threadIdx.x;
    int64_t cnt = 0;
    if (u < U) {
      const int b = u / s.Hkv, kvh = u % s.Hkv;
      const int64_t n = s.seq_prefix[b + 1] - s.seq_prefix[b];
      if (n > 0) {
        const int64_t A = (int64_t)s.Hkv * s.seq_prefix[b] + (int64_t)kvh * n;
        int64_t lo, hi;
        sched_unit_waves(A, n, T, W, lo, hi);
        cnt = hi - lo + 1;
      }
    }
    const int64_t ex = sched_block_scan(cnt, lds, slots);
    if (u < U) s.slot_base[u] = (int32_t)ex;
  }
  if (threadIdx.x == 0) s.slot_base[U] = (int32_t)slots;
}

// Largest b in [0, B) with seq_prefix[b] <= q (64-way search, one load per round).
__device__ __forceinline__ int sched_find_seq(const Sched &s, int64_t q) {
  int lo = 0, hi = s.B;
  while (hi - lo > 1) {
    const int step = (hi - lo + 63) / 64;
    const int i = lo + lane_id() * step;
    const bool ok = i < hi && (int64_t)s.seq_prefix[i] <= q;
    const int cnt = __popcll(__ballot(ok));
    const int nlo = lo + (cnt - 1) * step;
    hi = min(hi, nlo + step);
    lo = nlo;
  }
  return lo;
}

// Visit the unit segments of wave w (blockIdx.x of a one-wave block):
// f(b, kvh, s_begin, s_end, slot) with steps [s_begin, s_end) of unit
// (b, kvh) and the partial slot of this segment. Returns without calling f
// when the wave has no work.
template <class F>
__device__ __forceinline__ void sched_for_each_segment(const Sched &s, int64_t w, F &&f) {
  const int64_t T = (int64_t)s.Hkv * s.seq_prefix[s.B];
  if (T == 0) return;
  const int64_t W = sched_working_waves(s, T);
  if (w >= W) return;
  const int64_t t_begin = (w * T + W - 1) / W;
  const int64_t t_end = ((w + 1) * T + W - 1) / W;
  if (t_begin >= t_end) return;
  int b = sched_find_seq(s, t_begin / s.Hkv);
  int64_t t = t_begin;
  while (t < t_end) {
    const int n_b = s.seq_prefix[b + 1] - s.seq_prefix[b];
    const int64_t base_b = (int64_t)s.Hkv * s.seq_prefix[b];
    if (n_b == 0 || t >= base_b + (int64_t)s.Hkv * n_b) {  // next sequence with steps
      ++b;
      continue;
    }
    const int kvh = (int)((t - base_b) / n_b);
    const int64_t A_u = base_b + (int64_t)kvh * n_b;
    const int64_t seg_end = min(t_end, A_u + n_b);
    int64_t w_lo, w_hi;
    sched_unit_waves(A_u, n_b, T, W, w_lo, w_hi);
    const size_t slot = (size_t)s.slot_base[b * s.Hkv + kvh] + (size_t)(w - w_lo);
    f(b, kvh, (int)(t - A_u), (int)(seg_end - A_u), slot);
    t = seg_end;
  }
}

// Inclusive wave scan of int64 values (lane order).
__device__ __forceinline__ int64_t wave_incl_scan_i64(int64_t x) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

__device__ __forceinline__ int64_t readlane_i64(int64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, l);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)v >> 32), l);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// The same partition as sched_for_each_segment without a plan kernel: wave
// w scans the per-sequence step counts 64 at a time, first for the total T,
// then up to the end of its own range, and visits f(b, kvh, s_begin, s_end,
// slot) for each unit segment it owns. A unit's partials go to slots
// w + u (u = b * Hkv + kvh) for the waves w in [lo(u), hi(u)] that own its
// steps: consecutive units' wave ranges share at most one wave, so these
// runs never overlap, and every slot is below W + U. When prefix_out is set
// (one wave of the launch), it receives the exclusive step prefix per
// sequence and the total at [B] for the combine.
template <class StepsFn, class F>
__device__ __forceinline__ void sched_inline_for_each_segment(int B, int Hkv, int waves, int64_t w, StepsFn steps,
                                                              int32_t *prefix_out, F &&f) {
  const int lane = lane_id();
  int64_t carry = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    const int64_t n = b < B ? (int64_t)steps(b) : 0;
    const int64_t incl = wave_incl_scan_i64(n);
    if (prefix_out != nullptr && b < B) prefix_out[b] = (int32_t)(carry + incl - n);
    carry += readlane_i64(incl, 63);
  }
  if (prefix_out != nullptr && lane == 0) prefix_out[B] = (int32_t)carry;
  const int64_t T = (int64_t)Hkv * carry;
  if (T == 0) return;
  const int64_t W = max<int64_t>(1, min<int64_t>(waves, (T + kMinStepsPerWave - 1) / kMinStepsPerWave));
  if (w >= W) return;
  const int64_t t_begin = (w * T + W - 1) / W;
  const int64_t t_end = ((w + 1) * T + W - 1) / W;
  if (t_begin >= t_end) return;
  carry = 0;
  for (int b0 = 0; b0 < B && (int64_t)Hkv * carry < t_end; b0 += 64) {
    const int b = b0 + lane;
    const int64_t n = b < B ? (int64_t)steps(b) : 0;
    const int64_t incl = wave_incl_scan_i64(n);
    const int64_t base = (int64_t)Hkv * (carry + incl - n), end = (int64_t)Hkv * (carry + incl);
    uint64_t hit = __ballot(b < B && n > 0 && end > t_begin && base < t_end);
    while (hit != 0) {
      const int j = (int)__builtin_ctzll(hit);
      hit &= hit - 1;
      const int bb = b0 + j;
      const int64_t nb = readlane_i64(n, j);
      const int64_t base_b = readlane_i64(base, j);
      for (int kvh = (int)max<int64_t>(0, (t_begin - base_b) / nb); kvh < Hkv; ++kvh) {
        const int64_t A = base_b + (int64_t)kvh * nb;
        if (A >= t_end) break;
        const int64_t sb = max(t_begin, A), se = min(t_end, A + nb);
        if (sb < se) f(bb, kvh, (int)(sb - A), (int)(se - A), (size_t)(w + (int64_t)bb * Hkv + kvh));
      }
    }
    carry += readlane_i64(incl, 63);
  }
}

// Partial slots [s0, s1) of unit (b, kvh) under sched_inline_for_each_segment,
// from the per-sequence prefix it wrote (empty when the unit has no steps).
__device__ __forceinline__ void sched_inline_unit_slots(const int32_t *prefix, int B, int Hkv, int waves, int b,
                                                        int kvh, int &s0, int &s1) {
  const int64_t T = (int64_t)Hkv * prefix[B];
  const int64_t n = prefix[b + 1] - prefix[b];
  s0 = s1 = 0;
  if (T == 0 || n == 0) return;
  const int64_t W = max<int64_t>(1, min<int64_t>(waves, (T + kMinStepsPerWave - 1) / kMinStepsPerWave));
  const int64_t A = (int64_t)Hkv * prefix[b] + (int64_t)kvh * n;
  int64_t lo, hi;
  sched_unit_waves(A, n, T, W, lo, hi);
  const int64_t u = (int64_t)b * Hkv + kvh;
  s0 = (int)(lo + u);
  s1 = (int)(hi + u + 1);
}

}  // namespace sdk

namespace sdh {

// Bytes of the two schedule tables (each 256-byte aligned).
inline size_t sched_table_bytes(int64_t B, int64_t Hkv) {
  return align_up((size_t)(B + 1) * 4) + align_up((size_t)(B * Hkv + 1) * 4);
}

inline int64_t sched_max_slots(int64_t B, int64_t Hkv) { return sdk::kMaxWaves + B * Hkv; }

inline void sched_bind(sdk::Sched &s, void *tables, int32_t B, int32_t Hkv) {
  char *p = reinterpret_cast<char *>(tables);
  s.seq_prefix = reinterpret_cast<int32_t *>(p);
  s.slot_base = reinterpret_cast<int32_t *>(p + align_up((size_t)(B + 1) * 4));
  s.B = B;
  s.Hkv = Hkv;
}

constexpr int kMaxDevices = 64;  // devices with a cached occupancy entry

// Resident one-wave blocks of `kernel` on the current device, queried once per
// kernel and device and kept in cache[device] (cache has kMaxDevices entries;
// devices past that are queried every call). A failed query falls back to
// `fallback_per_cu` per CU. The count only sets the launch size and the
// split-KV schedule; a device always gets the same count, so results stay
// reproducible, and the workspace is sized for kMaxWaves whatever it is.
inline int resident_waves(const void *kernel, int fallback_per_cu, int *cache) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    dev = -1;
  }
  int *slot = dev >= 0 && dev < kMaxDevices ? cache + dev : nullptr;
  int w = slot ? __atomic_load_n(slot, __ATOMIC_RELAXED) : 0;
  if (w > 0) return w;
  int per_cu = 0, cus = 0;
  if (dev < 0 || hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 64, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      per_cu <= 0 || cus <= 0) {
    (void)hipGetLastError();
    per_cu = fallback_per_cu;
    cus = sdk::kNumCUs;
  }
  w = per_cu * cus < sdk::kMaxWaves ? per_cu * cus : sdk::kMaxWaves;
  if (slot) __atomic_store_n(slot, w, __ATOMIC_RELAXED);  // a race stores the same value
  return w;
}

}  // namespace sdh
