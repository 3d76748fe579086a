// Modified rejection sampling for one speculative round, gfx950.
//
// "Wann beschleunigt spekulatives Decoding das LLM-Serving?" (slavadubrov.com,
// verification-round section): accept the drafts left to right with both
// distributions, correct from the residual target distribution at the first
// rejection, or draw a bonus token from the target when all are accepted.
//
// Two kernels, both streaming the fp32 logits once:
//   accept_stats:  one block per (row, vocab chunk) of the 2*gamma+1 rows of
//     every sequence: chunk max of z/t and sum of exp(z/t - max) (fp32 exp,
//     fp64 accumulation);
//   accept_sample: one block per (sequence, vocab chunk). Every block merges
//     the chunk statistics into per-row log-normalisers (fp64), replays the
//     accept tests (fp64) to find n, then sums the residual weights of its
//     chunk (fp64). The last block of a sequence to finish (device-scope
//     counter) walks the chunk totals, rescans the chunk where the cumulative
//     weight crosses u*Z with an fp64 block prefix sum, and writes the tokens.
#include "sd_device.h"
#include "sd_host.h"

#include <algorithm>

using namespace sdk;

namespace {

constexpr int kAccThreads = 256;
constexpr int kPerThread = 32;
constexpr int kChunk = kAccThreads * kPerThread;  // vocab entries per block
constexpr int kMaxGamma = 64;

struct AccParams {
  const float *zt;  // [B, gamma+1, V]
  const float *zd;  // [B, gamma, V]
  const int32_t *tokens;
  const float *u_accept;
  const float *u_sample;
  int32_t *n_accepted;
  int32_t *out_tokens;
  double *stats;      // [B, 2*gamma+1, n_chunks, 2]  (max, sum)
  double *chunk_z;    // [B, n_chunks]
  int32_t *chunk_last;  // [B, n_chunks] last index with positive weight (-1)
  uint32_t *counter;  // [B]
  int32_t B, gamma, V, n_chunks;
  float inv_temp;
  double inv_temp_d;
};

__device__ __forceinline__ const float *row_ptr(const AccParams &a, int b, int k) {
  // k <= gamma: target row k; else draft row k - gamma - 1
  if (k <= a.gamma) return a.zt + ((size_t)b * (a.gamma + 1) + k) * a.V;
  return a.zd + ((size_t)b * a.gamma + (k - a.gamma - 1)) * a.V;
}

__device__ __forceinline__ double block_sum_f64(double v, double *lds) {
  v = wave_sum_f64(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < kAccThreads / 64; ++w) t += lds[w];
  __syncthreads();
  return t;
}

__device__ __forceinline__ float block_max_f32(float v, float *lds) {
  v = wave_max_f32(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  float t = lds[0];
#pragma unroll
  for (int w = 1; w < kAccThreads / 64; ++w) t = fmaxf(t, lds[w]);
  __syncthreads();
  return t;
}

__global__ __launch_bounds__(kAccThreads) void accept_stats_kernel(AccParams a) {
  __shared__ double lds_d[kAccThreads / 64];
  __shared__ float lds_f[kAccThreads / 64];
  const int c = blockIdx.x;
  const int rowid = blockIdx.y;  // b * (2*gamma+1) + k
  const int nrow = 2 * a.gamma + 1;
  const int b = rowid / nrow, k = rowid % nrow;
  const float *z = row_ptr(a, b, k);
  const int t0 = c * kChunk;
  float x[kPerThread];
  float mx = kNegInf;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const int t = t0 + e * kAccThreads + threadIdx.x;
    x[e] = t < a.V ? z[t] * a.inv_temp : kNegInf;
    mx = fmaxf(mx, x[e]);
  }
  mx = block_max_f32(mx, lds_f);
  double s = 0.0;
  if (mx != kNegInf) {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) s += (double)__builtin_amdgcn_exp2f((x[e] - mx) * kLog2e);
  }
  s = block_sum_f64(s, lds_d);
  if (threadIdx.x == 0) {
    double *st = a.stats + (((size_t)b * nrow + k) * a.n_chunks + c) * 2;
    st[0] = (double)mx;
    st[1] = s;
    if (c == 0 && k == 0) a.counter[b] = 0u;
  }
}

// Per-row (max, log of the normaliser relative to max), float64.
__device__ __forceinline__ void row_norm(const AccParams &a, int b, int k, double &M, double &logl) {
  const int nrow = 2 * a.gamma + 1;
  const double *st = a.stats + ((size_t)b * nrow + k) * a.n_chunks * 2;
  M = -__builtin_inf();
  for (int c = 0; c < a.n_chunks; ++c) M = fmax(M, st[2 * c]);
  double l = 0.0;
  for (int c = 0; c < a.n_chunks; ++c)
    if (st[2 * c] != -__builtin_inf()) l += st[2 * c + 1] * exp(st[2 * c] - M);
  logl = log(l);
}

__global__ __launch_bounds__(kAccThreads) void accept_sample_kernel(AccParams a) {
  __shared__ double s_rowM[2 * kMaxGamma + 1], s_rowL[2 * kMaxGamma + 1];
  __shared__ int s_n;
  __shared__ double lds_d[kAccThreads / 64];
  __shared__ double s_scan[kAccThreads];
  __shared__ int s_last, s_pick;
  __shared__ bool s_is_last;
  const int c = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int g = a.gamma;

  // 1. per-row log-normalisers (one thread per row), then the accept tests
  //    (thread 0, float64) and the residual rows.
  if (tid < 2 * g + 1) row_norm(a, b, tid, s_rowM[tid], s_rowL[tid]);
  __syncthreads();
  if (tid == 0) {
    int n = 0;
    for (int i = 0; i < g; ++i) {
      const int x = clampi(a.tokens[(size_t)b * g + i], 0, a.V - 1);
      const double zp = (double)row_ptr(a, b, i)[x] * a.inv_temp_d;
      const double zq = (double)row_ptr(a, b, g + 1 + i)[x] * a.inv_temp_d;
      const double p = exp(zp - s_rowM[i] - s_rowL[i]);
      const double q = exp(zq - s_rowM[g + 1 + i] - s_rowL[g + 1 + i]);
      const double u = (double)a.u_accept[(size_t)b * g + i];
      if (u * q < p)
        ++n;
      else
        break;
    }
    s_n = n;
  }
  __syncthreads();
  const int n = s_n;
  const bool residual = n < g;
  const float *zp = row_ptr(a, b, n);
  const float *zq = residual ? row_ptr(a, b, g + 1 + n) : nullptr;
  // p(t) = exp(z_t/T - M - log l): the offset M + log l stays in float64 so the
  // normalisers of p and q carry no systematic float32 rounding (it would not
  // cancel in p - q); only the final exponential is float32.
  const double cp = s_rowM[n] + s_rowL[n];
  const double cq = residual ? s_rowM[g + 1 + n] + s_rowL[g + 1 + n] : 0.0;
  constexpr double kLog2eD = 1.4426950408889634;
  auto prob = [&](const float *z, double c, int t) -> float {
    return __builtin_amdgcn_exp2f((float)(((double)z[t] * a.inv_temp_d - c) * kLog2eD));
  };
  auto weight = [&](int t) -> float {
    const float p = prob(zp, cp, t);
    if (!residual) return p;
    return fmaxf(0.f, p - prob(zq, cq, t));
  };

  // 2. this chunk's residual mass and last index with mass (order-free, so
  //    read with coalesced strided loads).
  double part = 0.0;
  int last = -1;
  for (int e = 0; e < kPerThread; ++e) {
    const int t = c * kChunk + e * kAccThreads + tid;
    if (t < a.V) {
      const float w = weight(t);
      part += (double)w;
      if (w > 0.f) last = t;
    }
  }
  const double zc = block_sum_f64(part, lds_d);
  if (tid == 0) s_last = -1;
  __syncthreads();
  if (last >= 0) atomicMax(&s_last, last);
  __syncthreads();
  if (tid == 0) {
    a.chunk_z[(size_t)b * a.n_chunks + c] = zc;
    a.chunk_last[(size_t)b * a.n_chunks + c] = s_last;
    __threadfence();
    const uint32_t done = atomicAdd(&a.counter[b], 1u);
    s_is_last = (done == (uint32_t)a.n_chunks - 1);
  }
  __syncthreads();
  if (!s_is_last) return;
  __threadfence();

  // 3. last block of this sequence: locate the chunk where the CDF crosses v*Z.
  __shared__ double s_before, s_thr;
  __shared__ int s_chunk, s_global_last;
  if (tid == 0) {
    double Z = 0.0;
    int glast = -1;
    for (int k = 0; k < a.n_chunks; ++k) {
      Z += __hip_atomic_load(&a.chunk_z[(size_t)b * a.n_chunks + k], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      glast = max(glast, __hip_atomic_load(&a.chunk_last[(size_t)b * a.n_chunks + k],
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    }
    s_global_last = glast;
    s_chunk = -1;
    if (Z > 0.0) {
      const double thr = (double)a.u_sample[(size_t)b * (g + 1) + n] * Z;
      double before = 0.0;
      for (int k = 0; k < a.n_chunks; ++k) {
        const double zk = __hip_atomic_load(&a.chunk_z[(size_t)b * a.n_chunks + k],
                                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (before + zk > thr) {
          s_chunk = k;
          break;
        }
        before += zk;
      }
      s_before = before;
      s_thr = thr;
    }
  }
  __syncthreads();
  int y = -1;
  if (s_chunk >= 0 || s_global_last < 0) {
    // Residual mass vanished (p_n == q_n): fall back to p_n over the whole row,
    // else rescan only the crossing chunk.
    const bool fallback = s_global_last < 0;
    const int c_lo = fallback ? 0 : s_chunk;
    const int c_hi = fallback ? a.n_chunks : s_chunk + 1;
    double before = fallback ? 0.0 : s_before;
    double thr = s_thr;
    if (fallback) {
      double tot = 0.0;
      for (int k = 0; k < a.n_chunks; ++k) {
        double pt = 0.0;
        for (int e = 0; e < kPerThread; ++e) {
          const int t = k * kChunk + e * kAccThreads + tid;
          if (t < a.V) pt += (double)prob(zp, cp, t);
        }
        tot += block_sum_f64(pt, lds_d);
      }
      thr = (double)a.u_sample[(size_t)b * (g + 1) + n] * tot;
    }
    if (tid == 0) s_pick = 0x7fffffff;  // smallest crossing token found
    __syncthreads();
    for (int k = c_lo; k < c_hi; ++k) {
      float w[kPerThread];
      double mine = 0.0;
      for (int e = 0; e < kPerThread; ++e) {
        const int t = k * kChunk + tid * kPerThread + e;
        float v = 0.f;
        if (t < a.V) {
          v = fallback ? prob(zp, cp, t) : weight(t);
        }
        w[e] = v;
        mine += (double)v;
      }
      // exclusive prefix of per-thread totals, in thread order
      s_scan[tid] = mine;
      __syncthreads();
      if (tid == 0) {
        double run = 0.0;
        for (int u = 0; u < kAccThreads; ++u) {
          const double v = s_scan[u];
          s_scan[u] = run;
          run += v;
        }
      }
      __syncthreads();
      double cum = before + s_scan[tid];
      for (int e = 0; e < kPerThread; ++e) {
        cum += (double)w[e];
        const int t = k * kChunk + tid * kPerThread + e;
        if (w[e] > 0.f && cum > thr) {
          atomicMin(&s_pick, t);
          break;
        }
      }
      __syncthreads();
      if (s_pick != 0x7fffffff) break;
      if (tid == kAccThreads - 1) s_scan[0] = cum;  // running total for the next chunk
      __syncthreads();
      before = s_scan[0];
      __syncthreads();
    }
    y = s_pick;
    if (y == 0x7fffffff) y = -1;
  }
  if (tid == 0) {
    // Rounding left no crossing inside the chosen chunk: its last token with mass.
    if (y < 0 && s_chunk >= 0)
      y = __hip_atomic_load(&a.chunk_last[(size_t)b * a.n_chunks + s_chunk], __ATOMIC_RELAXED,
                            __HIP_MEMORY_SCOPE_AGENT);
    if (y < 0) y = s_global_last;
    if (y < 0) y = 0;
    a.n_accepted[b] = n;
    int32_t *o = a.out_tokens + (size_t)b * (g + 1);
    for (int i = 0; i <= g; ++i) o[i] = i < n ? clampi(a.tokens[(size_t)b * g + i], 0, a.V - 1) : (i == n ? y : -1);
    a.counter[b] = 0u;
  }
}

struct AccPlan {
  int n_chunks;
  size_t stats_bytes, z_bytes, last_bytes, counter_bytes, ws_bytes;
};

AccPlan plan_accept(int64_t B, int64_t gamma, int64_t V) {
  AccPlan p;
  p.n_chunks = (int)sdh::ceil_div(V, kChunk);
  p.stats_bytes = sdh::align_up((size_t)B * (2 * gamma + 1) * p.n_chunks * 2 * 8);
  p.z_bytes = sdh::align_up((size_t)B * p.n_chunks * 8);
  p.last_bytes = sdh::align_up((size_t)B * p.n_chunks * 4);
  p.counter_bytes = sdh::align_up((size_t)B * 4);
  p.ws_bytes = p.stats_bytes + p.z_bytes + p.last_bytes + p.counter_bytes;
  return p;
}

}  // namespace

extern "C" size_t sd_spec_accept_workspace_size(int32_t batch, int32_t gamma, int32_t vocab) {
  if (batch <= 0 || gamma < 0 || vocab <= 0) return 0;
  return plan_accept(batch, gamma, vocab).ws_bytes;
}

extern "C" sd_status sd_spec_accept(const float *target_logits, const float *draft_logits,
                                    const int32_t *draft_tokens, const float *u_accept,
                                    const float *u_sample, int32_t batch, int32_t gamma,
                                    int32_t vocab, float temperature, int32_t *n_accepted,
                                    int32_t *out_tokens, void *workspace, size_t workspace_bytes,
                                    void *stream) {
  SD_REQUIRE(batch > 0 && gamma >= 0 && vocab > 0, SD_ERR_INVALID_ARG);
  SD_REQUIRE(gamma <= kMaxGamma, SD_ERR_UNSUPPORTED);
  SD_REQUIRE(target_logits != nullptr && u_sample != nullptr && n_accepted != nullptr &&
                 out_tokens != nullptr,
             SD_ERR_INVALID_ARG);
  SD_REQUIRE(gamma == 0 || (draft_logits != nullptr && draft_tokens != nullptr && u_accept != nullptr),
             SD_ERR_INVALID_ARG);
  SD_REQUIRE(temperature > 0.f && temperature < __builtin_inff(), SD_ERR_INVALID_ARG);
  SD_REQUIRE((int64_t)batch * (gamma + 1) * vocab < ((int64_t)1 << 40), SD_ERR_UNSUPPORTED);
  AccPlan p = plan_accept(batch, gamma, vocab);
  SD_REQUIRE(workspace != nullptr && workspace_bytes >= p.ws_bytes, SD_ERR_WORKSPACE);

  AccParams a{};
  a.zt = target_logits;
  a.zd = draft_logits;
  a.tokens = draft_tokens;
  a.u_accept = u_accept;
  a.u_sample = u_sample;
  a.n_accepted = n_accepted;
  a.out_tokens = out_tokens;
  char *ws = reinterpret_cast<char *>(workspace);
  a.stats = reinterpret_cast<double *>(ws);
  a.chunk_z = reinterpret_cast<double *>(ws + p.stats_bytes);
  a.chunk_last = reinterpret_cast<int32_t *>(ws + p.stats_bytes + p.z_bytes);
  a.counter = reinterpret_cast<uint32_t *>(ws + p.stats_bytes + p.z_bytes + p.last_bytes);
  a.B = batch;
  a.gamma = gamma;
  a.V = vocab;
  a.n_chunks = p.n_chunks;
  a.inv_temp = 1.f / temperature;
  a.inv_temp_d = 1.0 / (double)temperature;
  hipStream_t st = sdh::as_stream(stream);
  accept_stats_kernel<<<dim3((unsigned)p.n_chunks, (unsigned)(batch * (2 * gamma + 1))), kAccThreads, 0,
                        st>>>(a);
  accept_sample_kernel<<<dim3((unsigned)p.n_chunks, (unsigned)batch), kAccThreads, 0, st>>>(a);
  return sdh::launch_status();
}

