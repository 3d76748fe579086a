// Modified rejection sampling for one speculative round, gfx950.
//
// "Wann beschleunigt spekulatives Decoding das LLM-Serving?" (slavadubrov.com,
// verification-round section): accept the drafts left to right with both
// distributions, correct from the residual target distribution at the first
// rejection, or draw a bonus token from the target when all are accepted.
//
// Four kernels; the logits are streamed once, plus the one or two rows the
// residual needs:
//   accept_stats:    one block per (row, vocab chunk) of the 2*gamma+1 rows of
//                    every sequence: chunk max of z/t and the sum of exp(z/t -
//                    max) (fp32 exponentials, fp64 sums; each thread keeps its
//                    own running max, merged once at the end);
//   accept_decide:   one wave per sequence: lanes merge the chunk statistics of
//                    each row into log-normalisers (fp64) in parallel, lane i
//                    evaluates p_i(x_i), q_i(x_i) and the test
//                    u_i q_i(x_i) < p_i(x_i) (fp64); the accepted count n is
//                    the first failing lane;
//   accept_residual: one block per (sequence, vocab chunk): residual weights
//                    max(0, p_n - q_n) (or p_gamma) of the chunk, summed per
//                    2048-entry wave segment in fp64;
//   accept_sample:   one wave per sequence walks the segment sums to the one
//                    holding u*Z and finds the token there with wave prefix
//                    sums (fp64) over the segment loaded into registers.
#include "sd_device.h"
#include "sd_host.h"

#include <algorithm>

using namespace sdk;

namespace {

constexpr int kAccThreads = 256;
constexpr int kPerThread = 32;
constexpr int kChunk = kAccThreads * kPerThread;  // vocab entries per block
constexpr int kSegsPerChunk = kAccThreads / 64;   // wave segments of 64 * kPerThread entries
constexpr int kSeg = 64 * kPerThread;
constexpr int kMaxGamma = 64;                     // one decide lane per draft position
constexpr double kLog2eD = 1.4426950408889634;

struct AccParams {
  const float *zt;  // [B, gamma+1, V]
  const float *zd;  // [B, gamma, V]
  const int32_t *tokens;
  const float *u_accept;
  const float *u_sample;
  int32_t *n_accepted;
  int32_t *out_tokens;
  double *stats;      // [B, 2*gamma+1, n_chunks, 2]  (max, sum)
  double *dec;        // [B, 4]: n, log-normaliser of the p row, of the q row, unused
  double *seg_z;      // [B, n_chunks * kSegsPerChunk] residual mass per wave segment
  int32_t *seg_last;  // [B, n_chunks * kSegsPerChunk] last index with mass (-1)
  int32_t B, gamma, V, n_chunks;
  float inv_temp;
  double inv_temp_d;
};

__device__ __forceinline__ const float *row_ptr(const AccParams &a, int b, int k) {
  // k <= gamma: target row k; else draft row k - gamma - 1
  if (k <= a.gamma) return a.zt + ((size_t)b * (a.gamma + 1) + k) * a.V;
  return a.zd + ((size_t)b * a.gamma + (k - a.gamma - 1)) * a.V;
}

// Merge (m, s) pairs: s is relative to m; m = -inf means empty.
__device__ __forceinline__ void merge_ms(float &m, double &s, float m2, double s2) {
  const float M = fmaxf(m, m2);
  if (M == kNegInf) return;
  s = (m == kNegInf ? 0.0 : s * (double)__builtin_amdgcn_exp2f((m - M) * kLog2e)) +
      (m2 == kNegInf ? 0.0 : s2 * (double)__builtin_amdgcn_exp2f((m2 - M) * kLog2e));
  m = M;
}

// VEC = 4: 16-byte loads (rows 16-byte aligned), else 4-byte loads.
template <int VEC>
__device__ __forceinline__ void load_chunk(const float *z, int t0, int V, float inv_temp,
                                           float (&x)[kPerThread]) {
  if constexpr (VEC == 4) {
#pragma unroll
    for (int e = 0; e < kPerThread / 4; ++e) {
      const int t = t0 + (e * kAccThreads + (int)threadIdx.x) * 4;
      if (t + 3 < V) {
        const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(z + t));
#pragma unroll
        for (int j = 0; j < 4; ++j) x[4 * e + j] = v[j] * inv_temp;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) x[4 * e + j] = t + j < V ? z[t + j] * inv_temp : kNegInf;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const int t = t0 + e * kAccThreads + (int)threadIdx.x;
      x[e] = t < V ? z[t] * inv_temp : kNegInf;
    }
  }
}

template <int VEC>
__global__ __launch_bounds__(kAccThreads) void accept_stats_kernel(AccParams a) {
  __shared__ float lds_m[kAccThreads / 64];
  __shared__ double lds_s[kAccThreads / 64];
  const int c = blockIdx.x;
  const int rowid = blockIdx.y;  // b * (2*gamma+1) + k
  const int nrow = 2 * a.gamma + 1;
  const int b = rowid / nrow, k = rowid % nrow;
  const float *z = row_ptr(a, b, k);
  float x[kPerThread];
  load_chunk<VEC>(z, c * kChunk, a.V, a.inv_temp, x);
  float m = kNegInf;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) m = fmaxf(m, x[e]);
  double s = 0.0;
  if (m != kNegInf) {
    double s4[4] = {0.0, 0.0, 0.0, 0.0};  // four independent fp64 chains
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) s4[e & 3] += (double)__builtin_amdgcn_exp2f((x[e] - m) * kLog2e);
    s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) merge_ms(m, s, __shfl_xor(m, o, 64), __shfl_xor(s, o, 64));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    lds_m[wave] = m;
    lds_s[wave] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kAccThreads / 64; ++w) merge_ms(m, s, lds_m[w], lds_s[w]);
    double *st = a.stats + (((size_t)b * nrow + k) * a.n_chunks + c) * 2;
    st[0] = (double)m;
    st[1] = s;
  }
}

// Log of the softmax normaliser of row k (max of z/t plus log of the sum).
__device__ __forceinline__ double row_lse(const AccParams &a, int b, int k) {
  const int nrow = 2 * a.gamma + 1;
  const double *st = a.stats + ((size_t)b * nrow + k) * a.n_chunks * 2;
  double M = -__builtin_inf();
  for (int c = 0; c < a.n_chunks; ++c) M = fmax(M, st[2 * c]);
  double l = 0.0;
  for (int c = 0; c < a.n_chunks; ++c)
    if (st[2 * c] != -__builtin_inf()) l += st[2 * c + 1] * exp(st[2 * c] - M);
  return M + log(l);
}

// One wave per sequence.
__global__ __launch_bounds__(64) void accept_decide_kernel(AccParams a) {
  __shared__ double lse[2 * kMaxGamma + 1];
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int g = a.gamma;
  for (int k = lane; k < 2 * g + 1; k += 64) lse[k] = row_lse(a, b, k);
  __syncthreads();
  bool acc = false;  // lanes at or past gamma count as rejections (they stop the scan)
  if (lane < g) {
    const int x = clampi(a.tokens[(size_t)b * g + lane], 0, a.V - 1);
    const double p = exp((double)row_ptr(a, b, lane)[x] * a.inv_temp_d - lse[lane]);
    const double q = exp((double)row_ptr(a, b, g + 1 + lane)[x] * a.inv_temp_d - lse[g + 1 + lane]);
    acc = (double)a.u_accept[(size_t)b * g + lane] * q < p;
  }
  const uint64_t rej = ~__ballot(acc);
  const int n = min(g, rej != 0 ? (int)__builtin_ctzll(rej) : 64);
  if (lane == 0) {
    a.dec[(size_t)b * 4 + 0] = (double)n;
    a.dec[(size_t)b * 4 + 1] = lse[n];
    a.dec[(size_t)b * 4 + 2] = n < g ? lse[g + 1 + n] : 0.0;
    a.n_accepted[b] = n;
  }
  // accepted drafts and the -1 padding; slot n gets the sampled token later
  for (int t = lane; t <= g; t += 64) {
    if (t < n)
      a.out_tokens[(size_t)b * (g + 1) + t] = clampi(a.tokens[(size_t)b * g + t], 0, a.V - 1);
    else if (t > n)
      a.out_tokens[(size_t)b * (g + 1) + t] = -1;
  }
}

__device__ __forceinline__ double wave_incl_scan_f64(double v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  return v;
}

template <typename X>
__device__ __forceinline__ X prior_load(const X *p) {
  return *p;  // written by an earlier kernel on the same stream
}

template <int VEC>
__global__ __launch_bounds__(kAccThreads) void accept_residual_kernel(AccParams a) {
  const int c = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = a.gamma;
  const int n = (int)a.dec[(size_t)b * 4 + 0];
  const bool residual = n < g;
  const double cp = a.dec[(size_t)b * 4 + 1];
  const double cq = a.dec[(size_t)b * 4 + 2];
  const float *zp = row_ptr(a, b, n);
  const float *zq = residual ? row_ptr(a, b, g + 1 + n) : nullptr;
  // p(t) = exp(z_t/T - lse): the offset stays fp64 so that the p and q
  // normalisers carry no systematic fp32 rounding (it would not cancel in
  // p - q); only the final exponential is fp32.
  auto prob = [&](const float *z, double off, int t) -> float {
    return __builtin_amdgcn_exp2f((float)(((double)z[t] * a.inv_temp_d - off) * kLog2eD));
  };
  auto weight = [&](int t, bool target_only) -> float {
    const float p = prob(zp, cp, t);
    if (!residual || target_only) return p;
    return fmaxf(0.f, p - prob(zq, cq, t));
  };

  // Wave segment: entries seg0 + e*64 + lane, e < kPerThread (coalesced, and
  // consecutive in (e, lane) order).
  const int nseg = a.n_chunks * kSegsPerChunk;
  const int seg = c * kSegsPerChunk + wave;
  const int seg0 = seg * kSeg;
  double part = 0.0;
  int last = -1;
  if constexpr (VEC == 4) {
    // lane owns 4 consecutive entries per step: seg0 + e*256 + 4*lane + j
#pragma unroll 4
    for (int e = 0; e < kPerThread / 4; ++e) {
      const int t = seg0 + e * 256 + 4 * lane;
      float w[4];
      if (t + 3 < a.V) {
        const f32x4 pv = *reinterpret_cast<const f32x4 *>(zp + t);
        f32x4 qv = {0.f, 0.f, 0.f, 0.f};
        if (residual) qv = *reinterpret_cast<const f32x4 *>(zq + t);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p = __builtin_amdgcn_exp2f((float)(((double)pv[j] * a.inv_temp_d - cp) * kLog2eD));
          const float q = residual ? __builtin_amdgcn_exp2f((float)(((double)qv[j] * a.inv_temp_d - cq) * kLog2eD)) : 0.f;
          w[j] = residual ? fmaxf(0.f, p - q) : p;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = t + j < a.V ? weight(t + j, false) : 0.f;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        part += (double)w[j];
        if (w[j] > 0.f) last = t + j;
      }
    }
  } else {
#pragma unroll 8
    for (int e = 0; e < kPerThread; ++e) {
      const int t = seg0 + e * 64 + lane;
      if (t < a.V) {
        const float w = weight(t, false);
        part += (double)w;
        if (w > 0.f) last = t;
      }
    }
  }
  part = wave_sum_f64(part);
  for (int o = 32; o >= 1; o >>= 1) last = max(last, __shfl_xor(last, o, 64));
  if (lane == 0) {
    a.seg_z[(size_t)b * nseg + seg] = part;
    a.seg_last[(size_t)b * nseg + seg] = last;
  }
}

// One wave per sequence: segment sums -> segment holding u*Z -> token.
template <int VEC>
__global__ __launch_bounds__(64) void accept_sample_kernel(AccParams a) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int g = a.gamma;
  const int n = (int)a.dec[(size_t)b * 4 + 0];
  const bool residual = n < g;
  const double cp = a.dec[(size_t)b * 4 + 1];
  const double cq = a.dec[(size_t)b * 4 + 2];
  const float *zp = row_ptr(a, b, n);
  const float *zq = residual ? row_ptr(a, b, g + 1 + n) : nullptr;
  auto prob = [&](const float *z, double off, int t) -> float {
    return __builtin_amdgcn_exp2f((float)(((double)z[t] * a.inv_temp_d - off) * kLog2eD));
  };
  auto weight = [&](int t, bool target_only) -> float {
    const float p = prob(zp, cp, t);
    if (!residual || target_only) return p;
    return fmaxf(0.f, p - prob(zq, cq, t));
  };
  const int nseg = a.n_chunks * kSegsPerChunk;
  const double *zs = a.seg_z + (size_t)b * nseg;
  const int32_t *ls = a.seg_last + (size_t)b * nseg;
  int glast = -1;
  for (int k = lane; k < nseg; k += 64) glast = max(glast, prior_load(ls + k));
  for (int o = 32; o >= 1; o >>= 1) glast = max(glast, __shfl_xor(glast, o, 64));
  // Segment prefix sums, 64 segments per wave scan; the same scan (same
  // summation order) gives Z and then locates the segment holding u*Z.
  auto seg_scan = [&](int k0, double carry, double &incl, double &excl) {
    const double z = k0 + lane < nseg ? prior_load(zs + k0 + lane) : 0.0;
    incl = wave_incl_scan_f64(z) + carry;
    const double up = __shfl_up(incl, 1, 64);
    excl = lane == 0 ? carry : up;
  };
  double Z = 0.0;
  for (int k0 = 0; k0 < nseg; k0 += 64) {
    double incl, excl;
    seg_scan(k0, Z, incl, excl);
    Z = __shfl(incl, 63, 64);
  }
  const double v = (double)a.u_sample[(size_t)b * (g + 1) + n];
  const bool target_only = glast < 0;  // no residual mass at all (p_n == q_n): draw from p_n
  int k_first = -1, k_end = nseg;
  double before = 0.0, thr;
  if (target_only) {
    double tot = 0.0;
    for (int k = 0; k < nseg; ++k) {
      double ps = 0.0;
      for (int e = 0; e < kPerThread; ++e) {
        const int t = k * kSeg + e * 64 + lane;
        if (t < a.V) ps += (double)weight(t, true);
      }
      tot += wave_sum_f64(ps);
    }
    thr = v * tot;
    k_first = 0;
  } else {
    thr = v * Z;
    double carry = 0.0;
    for (int k0 = 0; k0 < nseg && k_first < 0; k0 += 64) {
      double incl, excl;
      seg_scan(k0, carry, incl, excl);
      const uint64_t hit = __ballot(k0 + lane < nseg && incl > thr);
      if (hit != 0) {
        const int j = (int)__builtin_ctzll(hit);
        k_first = k0 + j;
        before = __shfl(excl, j, 64);
      }
      carry = __shfl(incl, 63, 64);
    }
    k_end = k_first + 1;
  }
  int y = -1;
  if (k_first >= 0 && !target_only) {
    // The crossing segment: all its weights are loaded at once (lane owns the
    // same entries as in the summing pass), then scanned in order in registers.
    constexpr int J = VEC;                 // consecutive entries per lane per group
    constexpr int NG = kPerThread / J;     // groups of 64*J entries
    const int base = k_first * kSeg;
    float w[kPerThread];
#pragma unroll
    for (int eg = 0; eg < NG; ++eg)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int t = base + eg * 64 * J + J * lane + j;
        w[eg * J + j] = t < a.V ? weight(t, false) : 0.f;
      }
    for (int eg = 0; eg < NG && y < 0; ++eg) {
      double local[J];
      double run = 0.0;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        run += (double)w[eg * J + j];
        local[j] = run;
      }
      const double incl = wave_incl_scan_f64(run);
      const double excl = before + (incl - run);
      int hit_j = J;
#pragma unroll
      for (int j = J - 1; j >= 0; --j)
        if (w[eg * J + j] > 0.f && excl + local[j] > thr) hit_j = j;
      const uint64_t hit = __ballot(hit_j < J);
      if (hit != 0) {
        const int l = (int)__builtin_ctzll(hit);
        y = base + eg * 64 * J + J * l + __shfl(hit_j, l, 64);
      }
      before += __shfl(incl, 63, 64);
    }
    // rounding left no crossing inside the chosen segment: its last token with mass
    if (y < 0) y = prior_load(ls + k_first);
  } else if (k_first >= 0) {
    for (int k = k_first; k < k_end && y < 0; ++k) {
      for (int e = 0; e < kPerThread && y < 0; ++e) {
        const int t = k * kSeg + e * 64 + lane;
        const float wt = t < a.V ? weight(t, true) : 0.f;
        const double cum = before + wave_incl_scan_f64((double)wt);
        const uint64_t hit = __ballot(wt > 0.f && cum > thr);
        if (hit != 0) y = k * kSeg + e * 64 + (int)__builtin_ctzll(hit);
        before = __shfl(cum, 63, 64);
      }
    }
  }
  if (y < 0) y = target_only ? a.V - 1 : glast;
  if (lane == 0) a.out_tokens[(size_t)b * (g + 1) + n] = max(0, y);
}

struct AccPlan {
  int n_chunks;
  size_t stats_bytes, dec_bytes, segz_bytes, seglast_bytes, ws_bytes;
};

AccPlan plan_accept(int64_t B, int64_t gamma, int64_t V) {
  AccPlan p;
  p.n_chunks = (int)sdh::ceil_div(V, kChunk);
  const int64_t nseg = (int64_t)p.n_chunks * kSegsPerChunk;
  p.stats_bytes = sdh::align_up((size_t)B * (2 * gamma + 1) * p.n_chunks * 2 * 8);
  p.dec_bytes = sdh::align_up((size_t)B * 4 * 8);
  p.segz_bytes = sdh::align_up((size_t)B * nseg * 8);
  p.seglast_bytes = sdh::align_up((size_t)B * nseg * 4);
  p.ws_bytes = p.stats_bytes + p.dec_bytes + p.segz_bytes + p.seglast_bytes;
  return p;
}

}  // namespace

extern "C" size_t sd_spec_accept_workspace_size(int32_t batch, int32_t gamma, int32_t vocab) {
  if (batch <= 0 || gamma < 0 || vocab <= 0) return 0;
  return plan_accept(batch, gamma, vocab).ws_bytes;
}

namespace {

// Host checks shared by both acceptance entry points (no HIP call).
sd_status check_accept(const float *target_logits, const float *draft_logits, const int32_t *draft_tokens,
                       const float *u_accept, const float *u_sample, int32_t batch, int32_t gamma,
                       int32_t vocab, float temperature, int32_t *n_accepted, int32_t *out_tokens) {
  SD_REQUIRE(batch > 0 && gamma >= 0 && vocab > 0, SD_ERR_INVALID_ARG);
  SD_REQUIRE(gamma <= kMaxGamma, SD_ERR_UNSUPPORTED);
  SD_REQUIRE(target_logits != nullptr && u_sample != nullptr && n_accepted != nullptr &&
                 out_tokens != nullptr,
             SD_ERR_INVALID_ARG);
  SD_REQUIRE(gamma == 0 || (draft_logits != nullptr && draft_tokens != nullptr && u_accept != nullptr),
             SD_ERR_INVALID_ARG);
  SD_REQUIRE(temperature > 0.f && temperature < __builtin_inff(), SD_ERR_INVALID_ARG);
  SD_REQUIRE((int64_t)batch * (gamma + 1) * vocab < ((int64_t)1 << 40), SD_ERR_UNSUPPORTED);
  SD_REQUIRE(vocab < (1 << 30), SD_ERR_UNSUPPORTED);
  SD_REQUIRE((int64_t)batch * (2 * gamma + 1) < ((int64_t)1 << 31), SD_ERR_UNSUPPORTED);  // grid rows
  return SD_OK;
}

// Enqueue the four kernels with `workspace` (at least plan_accept's ws_bytes).
sd_status launch_accept(const float *target_logits, const float *draft_logits, const int32_t *draft_tokens,
                        const float *u_accept, const float *u_sample, int32_t batch, int32_t gamma,
                        int32_t vocab, float temperature, int32_t *n_accepted, int32_t *out_tokens,
                        const AccPlan &p, void *workspace, hipStream_t st) {
  AccParams a{};
  a.zt = target_logits;
  a.zd = draft_logits;
  a.tokens = draft_tokens;
  a.u_accept = u_accept;
  a.u_sample = u_sample;
  a.n_accepted = n_accepted;
  a.out_tokens = out_tokens;
  char *ws = reinterpret_cast<char *>(workspace);
  size_t off = 0;
  a.stats = reinterpret_cast<double *>(ws + off);
  off += p.stats_bytes;
  a.dec = reinterpret_cast<double *>(ws + off);
  off += p.dec_bytes;
  a.seg_z = reinterpret_cast<double *>(ws + off);
  off += p.segz_bytes;
  a.seg_last = reinterpret_cast<int32_t *>(ws + off);
  a.B = batch;
  a.gamma = gamma;
  a.V = vocab;
  a.n_chunks = p.n_chunks;
  a.inv_temp = 1.f / temperature;
  a.inv_temp_d = 1.0 / (double)temperature;
  // 16-byte loads need every row 16-byte aligned
  const bool vec = vocab % 4 == 0 && reinterpret_cast<uintptr_t>(target_logits) % 16 == 0 &&
                   (gamma == 0 || reinterpret_cast<uintptr_t>(draft_logits) % 16 == 0);
  const dim3 g_stats((unsigned)p.n_chunks, (unsigned)(batch * (2 * gamma + 1)));
  const dim3 g_res((unsigned)p.n_chunks, (unsigned)batch);
  if (vec)
    accept_stats_kernel<4><<<g_stats, kAccThreads, 0, st>>>(a);
  else
    accept_stats_kernel<1><<<g_stats, kAccThreads, 0, st>>>(a);
  accept_decide_kernel<<<(unsigned)batch, 64, 0, st>>>(a);
  if (vec) {
    accept_residual_kernel<4><<<g_res, kAccThreads, 0, st>>>(a);
    accept_sample_kernel<4><<<(unsigned)batch, 64, 0, st>>>(a);
  } else {
    accept_residual_kernel<1><<<g_res, kAccThreads, 0, st>>>(a);
    accept_sample_kernel<1><<<(unsigned)batch, 64, 0, st>>>(a);
  }
  return sdh::launch_status();
}

// Scratch of sd_spec_accept_noalloc: a fixed array in the library's device
// memory, one copy per GPU, held until the process ends. Host code never uses
// this name as an address: the device address comes from hipGetSymbolAddress
// and is kept per device in scratch_addr.
static __device__ __align__(256) unsigned char scratch[SD_SPEC_ACCEPT_SCRATCH_BYTES];

constexpr int kScratchDevices = 64;
void *scratch_addr[kScratchDevices];  // device address of `scratch` per device, set on first use

// Device address of `scratch` on `dev` (the current device): looked up once
// per device; a race stores the same address.
sd_status scratch_for(int dev, void **ptr) {
  SD_REQUIRE(dev >= 0 && dev < kScratchDevices, SD_ERR_UNSUPPORTED);
  void *p = __atomic_load_n(&scratch_addr[dev], __ATOMIC_ACQUIRE);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return SD_ERR_HIP;
    }
    __atomic_store_n(&scratch_addr[dev], p, __ATOMIC_RELEASE);
  }
  *ptr = p;
  return SD_OK;
}

}  // namespace

extern "C" sd_status sd_spec_accept(const float *target_logits, const float *draft_logits,
                                    const int32_t *draft_tokens, const float *u_accept,
                                    const float *u_sample, int32_t batch, int32_t gamma,
                                    int32_t vocab, float temperature, int32_t *n_accepted,
                                    int32_t *out_tokens, void *workspace, size_t workspace_bytes,
                                    void *stream) {
  sd_status s = check_accept(target_logits, draft_logits, draft_tokens, u_accept, u_sample, batch, gamma,
                             vocab, temperature, n_accepted, out_tokens);
  if (s != SD_OK) return s;
  AccPlan p = plan_accept(batch, gamma, vocab);
  SD_REQUIRE(workspace != nullptr && workspace_bytes >= p.ws_bytes, SD_ERR_WORKSPACE);
  return launch_accept(target_logits, draft_logits, draft_tokens, u_accept, u_sample, batch, gamma, vocab,
                       temperature, n_accepted, out_tokens, p, workspace, sdh::as_stream(stream));
}

extern "C" sd_status sd_spec_accept_noalloc(const float *target_logits, const float *draft_logits,
                                            const int32_t *draft_tokens, const float *u_accept,
                                            const float *u_sample, int32_t batch, int32_t gamma,
                                            int32_t vocab, float temperature, int32_t *n_accepted,
                                            int32_t *out_tokens, void *stream) {
  sd_status s = check_accept(target_logits, draft_logits, draft_tokens, u_accept, u_sample, batch, gamma,
                             vocab, temperature, n_accepted, out_tokens);
  if (s != SD_OK) return s;
  AccPlan p = plan_accept(batch, gamma, vocab);
  SD_REQUIRE(p.ws_bytes <= SD_SPEC_ACCEPT_SCRATCH_BYTES, SD_ERR_UNSUPPORTED);
  hipStream_t st = sdh::as_stream(stream);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return SD_ERR_HIP;
  }
  if (st != nullptr) {
    // the scratch address is per device: the stream must be the current device's
    int sdev = -1;
    if (hipStreamGetDevice(st, &sdev) != hipSuccess) {
      (void)hipGetLastError();
      return SD_ERR_HIP;
    }
    SD_REQUIRE(sdev == dev, SD_ERR_INVALID_ARG);
  }
  void *ws = nullptr;
  s = scratch_for(dev, &ws);
  if (s != SD_OK) return s;
  return launch_accept(target_logits, draft_logits, draft_tokens, u_accept, u_sample, batch, gamma, vocab,
                       temperature, n_accepted, out_tokens, p, ws, st);
}
