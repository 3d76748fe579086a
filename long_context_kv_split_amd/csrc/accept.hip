// Modified rejection sampling for one speculative round, gfx950.
//
// "Wann beschleunigt spekulatives Decoding das LLM-Serving?" (slavadubrov.com,
// verification-round section): accept the drafts left to right with both
// distributions, correct from the residual target distribution at the first
// rejection, or draw a bonus token from the target when all are accepted.
//
// Two kernels; the logits are streamed once, plus the one or two rows the
// draw needs:
//   accept_stats:  one block per (row, vocab chunk) of the 2*gamma+1 rows of
//                  every sequence: chunk max of z/t and the sum of exp(z/t -
//                  max) (fp32 exponentials, fp64 sums; each thread keeps its
//                  own running max, merged once at the end);
//   accept_finish: one 1024-thread block per sequence: its waves merge the
//                  chunk statistics of each row into log-normalisers (fp64),
//                  wave 0 evaluates u_i q_i(x_i) < p_i(x_i) for every draft
//                  (fp64; n = the first failure), then the block streams the
//                  drawn row pair once, residual weights max(0, p_n - q_n) (or
//                  p_gamma) summed per (slot, wave) piece in vocabulary order
//                  into LDS (fp64), scans the piece sums for the one holding
//                  u*Z, and the wave owning that piece rescans it for the
//                  token.
#include "sd_device.h"
#include "sd_host.h"

#include <algorithm>

using namespace sdk;

namespace {

constexpr int kAccThreads = 256;
constexpr int kPerThread = 32;
constexpr int kChunk = kAccThreads * kPerThread;  // vocab entries per block
constexpr int kMaxGamma = 64;                     // one decide lane per draft position

struct AccParams {
  const float *zt;  // [B, gamma+1, V]
  const float *zd;  // [B, gamma, V]
  const int32_t *tokens;
  const float *u_accept;
  const float *u_sample;
  int32_t *n_accepted;
  int32_t *out_tokens;
  double *stats;      // [B, 2*gamma+1, n_chunks, 2]  (max, sum)
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

// VEC = 4: 16-byte loads (rows 16-byte aligned, V a multiple of 4), else
// 4-byte loads. Addresses past the row are clamped onto its last entries and
// the values masked, so every load is issued unconditionally and all of a
// thread's loads are in flight together.
template <int VEC>
__device__ __forceinline__ void load_chunk(const float *z, int t0, int V, float inv_temp,
                                           float (&x)[kPerThread]) {
  if constexpr (VEC == 4) {
    f32x4 v[kPerThread / 4];
#pragma unroll
    for (int e = 0; e < kPerThread / 4; ++e) {
      const int t = t0 + (e * kAccThreads + (int)threadIdx.x) * 4;
      v[e] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(z + min(t, V - 4)));
    }
#pragma unroll
    for (int e = 0; e < kPerThread / 4; ++e) {
      const int t = t0 + (e * kAccThreads + (int)threadIdx.x) * 4;
#pragma unroll
      for (int j = 0; j < 4; ++j) x[4 * e + j] = t + j < V ? v[e][j] * inv_temp : kNegInf;
    }
  } else {
    float v[kPerThread];
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) v[e] = z[min(t0 + e * kAccThreads + (int)threadIdx.x, V - 1)];
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const int t = t0 + e * kAccThreads + (int)threadIdx.x;
      x[e] = t < V ? v[e] * inv_temp : kNegInf;
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

__device__ __forceinline__ double wave_incl_scan_f64(double v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  return v;
}

__device__ __forceinline__ double wave_max_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ int wave_max_i32(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}

// The finishing kernel: one 1024-thread block per sequence. The drawn row is
// cut into slots of G * kFinSpan entries (G = 1 up to a million entries), and
// slot k into one piece of G * kWaveSpan consecutive entries per wave: wave
// wv owns [k G kFinSpan + wv G kWaveSpan, + G kWaveSpan), which it reads in G
// iterations of kWaveSpan entries (lane l four consecutive ones). Pieces
// ordered by (slot, wave) are therefore in vocabulary order, and their sums
// fit in LDS. Entries past the row read as zero weight.
constexpr int kFinThreads = 1024;
constexpr int kFinWaves = kFinThreads / 64;
constexpr int kFinEnt = 4;                       // consecutive entries per lane and iteration
constexpr int kWaveSpan = 64 * kFinEnt;          // 256
constexpr int kFinSpan = kFinThreads * kFinEnt;  // 4096
constexpr int kFinSlots = 256;                   // slots per wave held in LDS
constexpr int kFinUnroll = 4;                    // iterations per pipelined batch of loads

// Weights of entries t..t+3 (t a multiple of 4) of the drawn row:
// max(0, p - q) (RESID) or p, p(t) = exp(z_t / T - lse). The fp64 normaliser
// enters as an fp32 pair (hi + lo = lse to about 2^-48 relative), so it
// carries no systematic fp32 rounding (that would scale p and q by different
// constants, an error that does not cancel in p - q); the exponent itself is
// formed in fp32 with one fused multiply-add, rounded per token like the
// final exponential.
// Loads are unconditional (clamped into the row, masked afterwards).
template <int VEC, bool RESID>
__device__ __forceinline__ void draw_load(const AccParams &a, const float *zp, const float *zq, int t,
                                          float (&zpv)[kFinEnt], float (&zqv)[kFinEnt]) {
  if constexpr (VEC == 4) {
    const int tc = min(t, a.V - 4);
    const f32x4 pv = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(zp + tc));
#pragma unroll
    for (int j = 0; j < 4; ++j) zpv[j] = pv[j];
    if constexpr (RESID) {
      const f32x4 qv = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(zq + tc));
#pragma unroll
      for (int j = 0; j < 4; ++j) zqv[j] = qv[j];
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tc = min(t + j, a.V - 1);
      zpv[j] = zp[tc];
      if constexpr (RESID) zqv[j] = zq[tc];
    }
  }
}

// First entry of lane `lane` of wave wv in iteration e (G iterations per slot).
__device__ __forceinline__ int fin_entry(int e, int G, int wv, int lane) {
  const int k = e / G;
  return k * G * kFinSpan + wv * G * kWaveSpan + (e - k * G) * kWaveSpan + kFinEnt * lane;
}

struct Offset {
  float hi, lo;
};
__device__ __forceinline__ Offset split_offset(double c) {
  const float hi = (float)c;
  return Offset{hi, (float)(c - (double)hi)};
}

template <bool RESID>
__device__ __forceinline__ void draw_weights(const AccParams &a, Offset cp, Offset cq, int t,
                                             const float (&zpv)[kFinEnt], const float (&zqv)[kFinEnt],
                                             float (&w)[kFinEnt]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float p = __builtin_amdgcn_exp2f((fmaf(zpv[j], a.inv_temp, -cp.hi) - cp.lo) * kLog2e);
    float r = p;
    if constexpr (RESID)
      r = fmaxf(0.f, p - __builtin_amdgcn_exp2f((fmaf(zqv[j], a.inv_temp, -cq.hi) - cq.lo) * kLog2e));
    w[j] = t + j < a.V ? r : 0.f;
  }
}

// One sweep over the drawn row: the (slot, wave) piece sums into seg, and the
// last entry with mass of this thread. Software-pipelined: the loads of the
// next kFinUnroll iterations are in flight while the current ones are
// summed (two register buffers used alternately; loads past the row are
// clamped into it and their results dropped).
template <int VEC, bool RESID>
__device__ __forceinline__ int draw_sweep(const AccParams &a, const float *zp, const float *zq, Offset cp,
                                          Offset cq, int iters, int G, double *seg) {
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  int last = -1;
  double gsum = 0.0;
  struct Buf {
    float p[kFinUnroll][kFinEnt], q[kFinUnroll][kFinEnt];
  };
  auto fetch = [&](int e0, Buf &bf) {
#pragma unroll
    for (int u = 0; u < kFinUnroll; ++u) draw_load<VEC, RESID>(a, zp, zq, fin_entry(e0 + u, G, wv, lane), bf.p[u], bf.q[u]);
  };
  auto consume = [&](int e0, const Buf &bf) {
#pragma unroll
    for (int u = 0; u < kFinUnroll; ++u) {
      const int e = e0 + u;
      if (e < iters) {
        const int t = fin_entry(e, G, wv, lane);
        float w[kFinEnt];
        draw_weights<RESID>(a, cp, cq, t, bf.p[u], bf.q[u], w);
        double s = 0.0;
#pragma unroll
        for (int j = 0; j < kFinEnt; ++j) {
          s += (double)w[j];
          if (w[j] > 0.f) last = t + j;
        }
        gsum += wave_sum_f64(s);
        if ((e + 1) % G == 0) {
          if (lane == 0) seg[(e / G) * kFinWaves + wv] = gsum;
          gsum = 0.0;
        }
      }
    }
  };
  Buf A, B;
  fetch(0, A);
  for (int e0 = 0; e0 < iters; e0 += 2 * kFinUnroll) {
    fetch(min(e0 + kFinUnroll, iters), B);
    consume(e0, A);
    if (e0 + kFinUnroll >= iters) break;
    fetch(min(e0 + 2 * kFinUnroll, iters), A);
    consume(e0 + kFinUnroll, B);
  }
  return last;
}

// The owning wave's rescan of piece (slot, wave): the first token with mass
// whose cumulative weight exceeds thr, or -1; *seg_last gets the piece's last
// token with mass.
template <int VEC, bool RESID>
__device__ __forceinline__ int draw_rescan(const AccParams &a, const float *zp, const float *zq, Offset cp,
                                           Offset cq, int e_begin, int e_end, int G, double before, double thr,
                                           int *seg_last) {
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  int y = -1, sl = -1;
  for (int e = e_begin; e < e_end && y < 0; ++e) {
    const int t = fin_entry(e, G, wv, lane);
    float zpv[kFinEnt], zqv[kFinEnt], w[kFinEnt];
    draw_load<VEC, RESID>(a, zp, zq, t, zpv, zqv);
    draw_weights<RESID>(a, cp, cq, t, zpv, zqv, w);
    double loc[kFinEnt], r = 0.0;
#pragma unroll
    for (int j = 0; j < kFinEnt; ++j) {
      r += (double)w[j];
      loc[j] = r;
      if (w[j] > 0.f) sl = t + j;
    }
    const double inc = wave_incl_scan_f64(r);
    const double exc = before + (inc - r);
    int hj = kFinEnt;
#pragma unroll
    for (int j = kFinEnt - 1; j >= 0; --j)
      if (w[j] > 0.f && exc + loc[j] > thr) hj = j;
    const uint64_t h = __ballot(hj < kFinEnt);
    if (h != 0) {
      const int l = (int)__builtin_ctzll(h);
      y = fin_entry(e, G, wv, l) + __shfl(hj, l, 64);
    }
    before += __shfl(inc, 63, 64);
  }
  *seg_last = wave_max_i32(sl);
  return y;
}

template <int VEC>
__global__ __launch_bounds__(kFinThreads) void accept_finish_kernel(AccParams a) {
  __shared__ double seg[kFinSlots * kFinWaves];  // (slot, wave) weight sums, vocabulary order
  __shared__ double lse[2 * kMaxGamma + 1];
  __shared__ double scan_w[kFinWaves];
  __shared__ int last_w[kFinWaves];
  __shared__ int hit_w[kFinWaves];
  __shared__ int n_s;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = a.gamma, nrow = 2 * g + 1;

  // Draft tokens and their logits depend on the inputs only: wave 0 fetches
  // them first, so their loads overlap the normalisers' merge below.
  int x = 0;
  float zpx = 0.f, zqx = 0.f;
  if (wv == 0 && lane < g) {
    x = clampi(a.tokens[(size_t)b * g + lane], 0, a.V - 1);
    zpx = row_ptr(a, b, lane)[x];
    zqx = row_ptr(a, b, g + 1 + lane)[x];
  }

  // 1. Row normalisers: one wave per row merges the row's chunk statistics
  //    (max of the chunk maxima, then the rescaled sum).
  for (int k = wv; k < nrow; k += kFinWaves) {
    const double *st = a.stats + ((size_t)b * nrow + k) * a.n_chunks * 2;
    double M = -__builtin_inf();
    for (int c = lane; c < a.n_chunks; c += 64) M = fmax(M, st[2 * c]);
    M = wave_max_f64(M);
    double l = 0.0;
    for (int c = lane; c < a.n_chunks; c += 64)
      if (st[2 * c] != -__builtin_inf()) l += st[2 * c + 1] * exp(st[2 * c] - M);
    l = wave_sum_f64(l);
    if (lane == 0) lse[k] = M + log(l);
  }
  __syncthreads();

  // 2. Accept tests: lane i of wave 0 evaluates u_i q_i(x_i) < p_i(x_i) (fp64);
  //    n is the first failing lane. Accepted drafts and the -1 padding are
  //    written here, the drawn token at the end.
  if (wv == 0) {
    bool acc = false;  // lanes at or past gamma count as rejections (they stop the scan)
    if (lane < g) {
      const double p = exp((double)zpx * a.inv_temp_d - lse[lane]);
      const double q = exp((double)zqx * a.inv_temp_d - lse[g + 1 + lane]);
      acc = (double)a.u_accept[(size_t)b * g + lane] * q < p;
    }
    const uint64_t rej = ~__ballot(acc);
    const int n = min(g, rej != 0 ? (int)__builtin_ctzll(rej) : 64);
    if (lane == 0) {
      n_s = n;
      a.n_accepted[b] = n;
    }
    for (int t = lane; t <= g; t += 64) {
      if (t < n)
        a.out_tokens[(size_t)b * (g + 1) + t] = clampi(a.tokens[(size_t)b * g + t], 0, a.V - 1);
      else if (t > n)
        a.out_tokens[(size_t)b * (g + 1) + t] = -1;
    }
  }
  __syncthreads();
  const int n = n_s;
  const float *zp = row_ptr(a, b, n);
  const float *zq = n < g ? row_ptr(a, b, g + 1 + n) : zp;
  const Offset cp = split_offset(lse[n]);
  const Offset cq = split_offset(n < g ? lse[g + 1 + n] : 0.0);
  const int row_iters = (a.V + kFinSpan - 1) / kFinSpan;
  const int G = (row_iters + kFinSlots - 1) / kFinSlots;  // iterations per slot
  const int nslots = (row_iters + G - 1) / G;
  const int iters = nslots * G;  // whole slots; entries past the row weigh zero
  const int npieces = nslots * kFinWaves;

  // 3. One sweep over the drawn row: (slot, wave) sums in LDS, and the last
  //    entry with mass. The residual of a row pair with no mass at all
  //    (p_n == q_n) is replaced by p_n, as the pages' reading prescribes.
  bool residual = n < g;
  int glast = -1;
  for (int pass = 0; pass < 2; ++pass) {
    int last = residual ? draw_sweep<VEC, true>(a, zp, zq, cp, cq, iters, G, seg)
                        : draw_sweep<VEC, false>(a, zp, zq, cp, cq, iters, G, seg);
    last = wave_max_i32(last);
    if (lane == 0) last_w[wv] = last;
    __syncthreads();
    glast = -1;
    for (int w2 = 0; w2 < kFinWaves; ++w2) glast = max(glast, last_w[w2]);
    __syncthreads();
    if (glast >= 0 || !residual) break;
    residual = false;  // no residual mass anywhere: draw from p_n
  }

  // 4. Scan of the piece sums (fp64, vocabulary order): thread i takes
  //    pieces 4i .. 4i+3; the first piece whose inclusive sum exceeds u*Z
  //    holds the token.
  constexpr int kPer = kFinSlots * kFinWaves / kFinThreads;  // 4
  double ps[kPer], run = 0.0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = kPer * tid + j;
    run += i < npieces ? seg[i] : 0.0;
    ps[j] = run;
  }
  const double incl = wave_incl_scan_f64(run);
  if (lane == 63) scan_w[wv] = incl;
  __syncthreads();
  double before_w = 0.0, Z = 0.0;
  for (int w2 = 0; w2 < kFinWaves; ++w2) {
    if (w2 < wv) before_w += scan_w[w2];
    Z += scan_w[w2];
  }
  const double excl_t = before_w + incl - run;  // sum of the pieces before 4*tid
  const double v = (double)a.u_sample[(size_t)b * (g + 1) + n];
  const double thr = v * Z;
  int hit = kPer;
#pragma unroll
  for (int j = kPer - 1; j >= 0; --j)
    if (kPer * tid + j < npieces && excl_t + ps[j] > thr) hit = j;
  const uint64_t hb = __ballot(hit < kPer);
  if (lane == 0) hit_w[wv] = hb != 0 ? (64 * wv + (int)__builtin_ctzll(hb)) : 0x7fffffff;
  __syncthreads();
  int first_t = 0x7fffffff;
  for (int w2 = 0; w2 < kFinWaves; ++w2) first_t = min(first_t, hit_w[w2]);
  int y = -1;
  if (first_t != 0x7fffffff) {
    // the thread that found the first crossing publishes its piece and the
    // sum of the pieces before it
    __shared__ int piece_s;
    __shared__ double before_s;
    if (tid == first_t) {
      piece_s = kPer * tid + hit;
      before_s = excl_t + (hit > 0 ? ps[hit - 1] : 0.0);
    }
    __syncthreads();
    const int piece = piece_s;
    const int slot = piece / kFinWaves, pw = piece % kFinWaves;
    if (wv == pw) {
      // the owning wave reloads its entries of the slot's iterations and
      // scans them in vocabulary order
      const int e_end = (slot + 1) * G;
      int seg_last = -1;
      y = residual ? draw_rescan<VEC, true>(a, zp, zq, cp, cq, slot * G, e_end, G, before_s, thr, &seg_last)
                   : draw_rescan<VEC, false>(a, zp, zq, cp, cq, slot * G, e_end, G, before_s, thr, &seg_last);
      // rounding left no crossing inside the piece: its last token with mass
      if (y < 0) y = seg_last;
      if (y < 0) y = glast;
      if (lane == 0) a.out_tokens[(size_t)b * (g + 1) + n] = max(0, y);
    }
  } else if (tid == 0) {
    // rounding left v*Z at or above the total: the last token with mass
    a.out_tokens[(size_t)b * (g + 1) + n] = max(0, glast);
  }
}

struct AccPlan {
  int n_chunks;
  size_t ws_bytes;  // the chunk statistics
};

AccPlan plan_accept(int64_t B, int64_t gamma, int64_t V) {
  AccPlan p;
  p.n_chunks = (int)sdh::ceil_div(V, kChunk);
  p.ws_bytes = sdh::align_up((size_t)B * (2 * gamma + 1) * p.n_chunks * 2 * 8);
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
  a.stats = reinterpret_cast<double *>(workspace);
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
  if (vec) {
    accept_stats_kernel<4><<<g_stats, kAccThreads, 0, st>>>(a);
    accept_finish_kernel<4><<<(unsigned)batch, kFinThreads, 0, st>>>(a);
  } else {
    accept_stats_kernel<1><<<g_stats, kAccThreads, 0, st>>>(a);
    accept_finish_kernel<1><<<(unsigned)batch, kFinThreads, 0, st>>>(a);
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
