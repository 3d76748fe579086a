// Modified rejection sampling for one speculative round, gfx950.
//
// "Wann beschleunigt spekulatives Decoding das LLM-Serving?" (slavadubrov.com,
// verification-round section): accept the drafts left to right with both
// distributions, correct from the residual target distribution at the first
// rejection, or draw a bonus token from the target when all are accepted.
//
// Three kernels; the logits are streamed once, plus the one or two rows the
// draw needs:
//   accept_stats:    one block per (draft position, vocab chunk) of every
//                    sequence, reading the chunk of p_i and of q_i together
//                    (p_gamma alone): per row the chunk max of z/t and the sum
//                    of exp(z/t - max) (fp32 exponentials, fp64 sums), and for
//                    the pair the sum of p weights times expm1((zq - zp)/t),
//                    from which the difference of the two normalisers comes out
//                    to full relative accuracy when q is close to p;
//   accept_residual: one block per (sequence, slice of the vocabulary): the
//                    block merges the sequence's chunk statistics into row
//                    log-normalisers (fp64), evaluates u_i q_i(x_i) < p_i(x_i)
//                    for every draft (fp64; n = the first failure), forms the
//                    drawn pair's normaliser gap from the cross sums, and sums
//                    the weights of the drawn row pair over its slice, per
//                    1024-entry piece, in fp64: max(0, p_n - q_n) (as
//                    p (1 - q/p)) and p_n, or p_gamma. Several blocks per
//                    sequence spread the drawn row over the CUs (one CU
//                    streams a row at a few tens of GB/s);
//   accept_draw:     one block per sequence scans the piece sums in vocabulary
//                    order for the piece holding u*Z and rescans that piece for
//                    the token.
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
  double *cross;      // [B, gamma, n_chunks]: sum of p_i weights (relative to the chunk max) x expm1(d)
  double *pieces;     // [B, 2, npieces]: weight sums per piece, residual (0) and p_n (1)
  double *seq_lse;    // [B, 2]: the drawn row's normaliser lse_p and lse_q - lse_p (residual draws)
  int32_t *seq_n;     // [B]: accepted drafts
  int32_t B, gamma, V, n_chunks;
  int32_t npieces, pps;  // pieces per row, pieces per residual slice
  float inv_temp;
  double inv_temp_d;
};

__device__ __forceinline__ const float *row_ptr(const AccParams &a, int b, int k) {
  // k <= gamma: target row k; else draft row k - gamma - 1
  if (k <= a.gamma) return a.zt + ((size_t)b * (a.gamma + 1) + k) * a.V;
  return a.zd + ((size_t)b * a.gamma + (k - a.gamma - 1)) * a.V;
}

// expm1(d) for |d| < 1/8: its Taylor series to degree 5 (relative error
// below 5e-8, under fp32's own rounding).
__device__ __forceinline__ float expm1_small(float d) {
  return d * fmaf(d, fmaf(d, fmaf(d, fmaf(d, 1.f / 120.f, 1.f / 24.f), 1.f / 6.f), 0.5f), 1.f);
}

// Raw logits of one row's chunk (entries past the row clamped onto its last
// ones; the caller masks them).
template <int VEC>
__device__ __forceinline__ void load_raw(const float *z, int t0, int V, float (&v)[kPerThread]) {
  if constexpr (VEC == 4) {
    f32x4 w[kPerThread / 4];
#pragma unroll
    for (int e = 0; e < kPerThread / 4; ++e) {
      const int t = t0 + (e * kAccThreads + (int)threadIdx.x) * 4;
      w[e] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(z + min(t, V - 4)));
    }
#pragma unroll
    for (int e = 0; e < kPerThread / 4; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j) v[4 * e + j] = w[e][j];
  } else {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) v[e] = z[min(t0 + e * kAccThreads + (int)threadIdx.x, V - 1)];
  }
}

// Wave max of x, then the wave's sum of exp(x - max) (fp64 over pairs summed
// in fp32); m = -inf for a wave with no entry.
__device__ __forceinline__ void wave_max_sum(const float (&x)[kPerThread], float &m, double &s) {
  m = kNegInf;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) m = fmaxf(m, x[e]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  s = 0.0;
  if (m != kNegInf) {
    double s2[2] = {0.0, 0.0};  // pairs of weights summed in fp32, then in fp64
#pragma unroll
    for (int e = 0; e < kPerThread; e += 2)
      s2[(e >> 1) & 1] += (double)(__builtin_amdgcn_exp2f((x[e] - m) * kLog2e) +
                                   __builtin_amdgcn_exp2f((x[e + 1] - m) * kLog2e));
    s = s2[0] + s2[1];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
}

// One block per (sequence, draft position i, chunk): rows p_i and q_i of the
// chunk (i < gamma), or p_gamma alone. Per row the chunk's max of z/t (exact,
// float) and the sum of exp(z/t - max) (wave max first, fp32 exponentials
// added in pairs in fp32, then in fp64; the waves' sums merged by thread 0).
// For a pair also
//   T = sum_t exp(zp_t/t - M_p) expm1(d_t),  d_t = (zq_t - zp_t)/t,
// with the same p weights as the p sum: summed over the chunks with weight
// exp(M_p - lse_p) it is E_p[exp(d)] - 1 = exp(lse_q - lse_p) - 1, so the
// normalisers' difference is known to the relative accuracy of T, not to the
// absolute accuracy of either normaliser. d_t is formed from the raw logits
// (their difference is exact when they are close). Where the p weight
// underflows, the entry adds its q weight exp(zq_t/t - M_p) instead (the same
// quantity, w expm1(d) = exp(zq/t - M_p) - w with w = 0; its |d| is large, so
// the term is formed as that difference); where a wave's p
// entries are all -inf and its q entries are not, T is +inf, and so is the
// chunk's if every p entry is -inf: the relative form does not exist there
// and the plain difference of the normalisers is used.
template <int VEC, bool PAIR>
__device__ __forceinline__ void stats_chunk(const AccParams &a, int b, int i, int c) {
  __shared__ float lds_m[2][kAccThreads / 64];
  __shared__ double lds_s[3][kAccThreads / 64];
  const int nrow = 2 * a.gamma + 1;
  const int t0 = c * kChunk;
  float zp[kPerThread], zq[kPerThread];
  load_raw<VEC>(row_ptr(a, b, i), t0, a.V, zp);
  if constexpr (PAIR) load_raw<VEC>(row_ptr(a, b, a.gamma + 1 + i), t0, a.V, zq);
  float xp[kPerThread], xq[kPerThread];
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const int t = VEC == 4 ? t0 + ((e / 4) * kAccThreads + (int)threadIdx.x) * 4 + e % 4
                           : t0 + e * kAccThreads + (int)threadIdx.x;
    xp[e] = t < a.V ? zp[e] * a.inv_temp : kNegInf;
    if constexpr (PAIR) xq[e] = t < a.V ? zq[e] * a.inv_temp : kNegInf;
  }
  float mp, mq = kNegInf;
  double sp, sq = 0.0, tx = 0.0;
  if constexpr (!PAIR) {
    wave_max_sum(xp, mp, sp);
  } else {
    mp = kNegInf;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      mp = fmaxf(mp, xp[e]);
      mq = fmaxf(mq, xq[e]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      mp = fmaxf(mp, __shfl_xor(mp, o, 64));
      mq = fmaxf(mq, __shfl_xor(mq, o, 64));
    }
    sp = 0.0;
    if (mp != kNegInf) {
      // q weight relative to mp = wq * exp(mq - mp) (inf where q lies far above p)
      const float qp = mq == kNegInf ? 0.f : __builtin_amdgcn_exp2f((mq - mp) * kLog2e);
      // an entry's term of T: wp expm1(d) = wq qp - wp. Below |d| = 1/8 it is
      // wp times expm1(d) from its Taylor series; above, the difference loses
      // at most a factor ~10 of fp32's precision. With wp = 0 (p's weight
      // underflows) it is q's weight alone.
      auto term = [&](int e, float wp, float wq) {
        const float d = (zq[e] - zp[e]) * a.inv_temp;
        return fabsf(d) < 0.125f ? wp * expm1_small(d) : fmaf(wq, qp, -wp);
      };
      // two entries summed in fp32 per fp64 addition: the pair sums of the
      // weights are exact to ~6e-8 relative, less than each weight's own
      // error; a pair of T terms that cancels loses absolute accuracy of
      // ~6e-8 of its terms only, which moves the normalisers' gap by far
      // less than it moves the residual weights
      double s2[2] = {0.0, 0.0}, q2[2] = {0.0, 0.0}, t2[2] = {0.0, 0.0};
#pragma unroll
      for (int e = 0; e < kPerThread; e += 2) {
        const float wp0 = __builtin_amdgcn_exp2f((xp[e] - mp) * kLog2e);
        const float wq0 = __builtin_amdgcn_exp2f((xq[e] - mq) * kLog2e);
        const float wp1 = __builtin_amdgcn_exp2f((xp[e + 1] - mp) * kLog2e);
        const float wq1 = __builtin_amdgcn_exp2f((xq[e + 1] - mq) * kLog2e);
        s2[(e >> 1) & 1] += (double)(wp0 + wp1);
        q2[(e >> 1) & 1] += (double)(wq0 + wq1);
        t2[(e >> 1) & 1] += (double)(term(e, wp0, wq0) + term(e + 1, wp1, wq1));
      }
      sp = s2[0] + s2[1];
      sq = q2[0] + q2[1];
      tx = t2[0] + t2[1];
    } else if (mq != kNegInf) {
      double q2[2] = {0.0, 0.0};
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) q2[e & 1] += (double)__builtin_amdgcn_exp2f((xq[e] - mq) * kLog2e);
      sq = q2[0] + q2[1];
      tx = __builtin_inf();  // q mass where p has none
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      sp += __shfl_xor(sp, o, 64);
      sq += __shfl_xor(sq, o, 64);
      tx += __shfl_xor(tx, o, 64);
    }
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    lds_m[0][wave] = mp;
    lds_s[0][wave] = sp;
    lds_m[1][wave] = mq;
    lds_s[1][wave] = sq;
    lds_s[2][wave] = tx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    // the block max of each row, then every wave's sums rescaled to it (T
    // with the p factors)
    float Mp = kNegInf, Mq = kNegInf;
    for (int w = 0; w < kAccThreads / 64; ++w) {
      Mp = fmaxf(Mp, lds_m[0][w]);
      Mq = fmaxf(Mq, lds_m[1][w]);
    }
    double Sp = 0.0, Sq = 0.0, Tx = 0.0;
    for (int w = 0; w < kAccThreads / 64; ++w) {
      if (lds_m[0][w] != kNegInf) {
        const double f = (double)__builtin_amdgcn_exp2f((lds_m[0][w] - Mp) * kLog2e);
        Sp += lds_s[0][w] * f;
        Tx += lds_s[2][w] * f;
      } else if (lds_s[2][w] != 0.0) {
        Tx = __builtin_inf();
      }
      if (PAIR && lds_m[1][w] != kNegInf)
        Sq += lds_s[1][w] * (double)__builtin_amdgcn_exp2f((lds_m[1][w] - Mq) * kLog2e);
    }
    double *st = a.stats + (((size_t)b * nrow + i) * a.n_chunks + c) * 2;
    st[0] = (double)Mp;
    st[1] = Sp;
    if constexpr (PAIR) {
      double *sq_ = a.stats + (((size_t)b * nrow + a.gamma + 1 + i) * a.n_chunks + c) * 2;
      sq_[0] = (double)Mq;
      sq_[1] = Sq;
      a.cross[((size_t)b * a.gamma + i) * a.n_chunks + c] = Tx;
    }
  }
}

template <int VEC>
__global__ __launch_bounds__(kAccThreads) void accept_stats_kernel(AccParams a) {
  const int c = blockIdx.x;
  const int b = blockIdx.y / (a.gamma + 1), i = blockIdx.y % (a.gamma + 1);
  if (i < a.gamma)
    stats_chunk<VEC, true>(a, b, i, c);
  else
    stats_chunk<VEC, false>(a, b, i, c);
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

__device__ __forceinline__ int wave_max_i32(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}

// Residual and draw kernels. The drawn row (the residual max(0, p_n - q_n)
// after a rejection, p_gamma when every draft is accepted) is cut into pieces
// of kPiece consecutive entries; lane l of the wave that owns a piece reads
// entries 256 j + 4 l .. 256 j + 4 l + 3 of it (j = 0..3), so each of its
// loads is one contiguous 1 KB row segment across the wave. Entries past the
// row weigh zero.
constexpr int kResThreads = 256;
constexpr int kResWaves = kResThreads / 64;
constexpr int kPieceLoads = 4;                // 16-byte loads per lane, row and piece
constexpr int kPiece = 64 * 4 * kPieceLoads;  // 1024 entries
constexpr int kTargetBlocks = 1024;           // residual blocks per call (sequences x slices)
constexpr int kDrawThreads = 256;
constexpr int kDrawPer = 4;  // piece sums per thread and round of the draw's scan

struct Offset {
  float hi, lo;
};
__device__ __forceinline__ Offset split_offset(double c) {
  const float hi = (float)c;
  return Offset{hi, (float)(c - (double)hi)};
}

// Weights of the entries t .. t+3 (t = piece base + 256 j + 4 lane):
// p = exp(z_t / T - lse_p), and max(0, p - q) (RESID). The fp64 normaliser
// enters as an fp32 pair (hi + lo = lse to about 2^-48 relative), so it
// carries no systematic fp32 rounding; the exponent itself is formed in fp32,
// rounded per token like the final exponential. The residual is not formed
// as the difference of two rounded probabilities: where q is close to p that
// difference loses most of its digits, and the draw then lands on other
// tokens than the exact residual's. It is p (1 - q/p) = -p expm1(e) with
// e = ln(q/p) = (zq - zp) / T - (lse_q - lse_p), whose logit difference is
// exact when the two logits are close and whose normaliser difference enters
// as an fp32 pair as well, so r keeps the relative accuracy of p. Loads are
// unconditional (clamped into the row, masked afterwards).
template <int VEC, bool RESID>
__device__ __forceinline__ void piece_load(const AccParams &a, const float *zp, const float *zq, int t,
                                           float (&zpv)[4], float (&zqv)[4]) {
  if constexpr (VEC == 4) {
    const int tc = min(t, a.V - 4);
    const f32x4 pv = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(zp + tc));
#pragma unroll
    for (int e = 0; e < 4; ++e) zpv[e] = pv[e];
    if constexpr (RESID) {
      const f32x4 qv = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(zq + tc));
#pragma unroll
      for (int e = 0; e < 4; ++e) zqv[e] = qv[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int tc = min(t + e, a.V - 1);
      zpv[e] = zp[tc];
      if constexpr (RESID) zqv[e] = zq[tc];
    }
  }
}

// p weights (pw) and, with RESID, residual weights (rw) of entries t .. t+3.
// cp: lse_p; cd: lse_q - lse_p (both as fp32 pairs).
template <bool RESID>
__device__ __forceinline__ void piece_weights(const AccParams &a, Offset cp, Offset cd, int t,
                                              const float (&zpv)[4], const float (&zqv)[4], float (&pw)[4],
                                              float (&rw)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float p = __builtin_amdgcn_exp2f((fmaf(zpv[e], a.inv_temp, -cp.hi) - cp.lo) * kLog2e);
    float r = p;
    if constexpr (RESID) {
      // ln(q/p); NaN (both logits -inf) and e >= 0 (q >= p) give no residual;
      // expm1 from its series below 1/8, else exp - 1 (no cancellation there)
      const float lr = fmaf(zqv[e] - zpv[e], a.inv_temp, -cd.hi) - cd.lo;
      const float em1 = fabsf(lr) < 0.125f ? expm1_small(lr) : __builtin_amdgcn_exp2f(lr * kLog2e) - 1.f;
      r = lr < 0.f ? -p * em1 : 0.f;
    }
    const bool in = t + e < a.V;
    pw[e] = in ? p : 0.f;
    rw[e] = in ? r : 0.f;
  }
}

// Row normalisers of sequence b into lse[0 .. 2 gamma] (max of the chunk
// maxima, then the rescaled sum, fp64). Each row is merged by a group of L
// lanes (L = the chunk count rounded up to a power of two, at most 64), so a
// wave merges 64 / L rows at once: the rows' loads go out together and the
// group reductions are log2(L) steps.
template <int WAVES>
__device__ __forceinline__ void row_normalisers(const AccParams &a, int b, double *lse) {
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int nrow = 2 * a.gamma + 1;
  int L = 1;
  while (L < a.n_chunks && L < 64) L <<= 1;
  const int rpw = 64 / L, sub = lane & (L - 1);
  for (int k0 = wv * rpw; k0 < nrow; k0 += WAVES * rpw) {
    const int k = k0 + lane / L;
    const double *st = a.stats + ((size_t)b * nrow + min(k, nrow - 1)) * a.n_chunks * 2;
    double M = -__builtin_inf();
    for (int c = sub; c < a.n_chunks; c += L) M = fmax(M, st[2 * c]);
    for (int m = 1; m < L; m <<= 1) M = fmax(M, __shfl_xor(M, m, 64));
    double l = 0.0;
    for (int c = sub; c < a.n_chunks; c += L)
      if (st[2 * c] != -__builtin_inf()) l += st[2 * c + 1] * exp(st[2 * c] - M);
    for (int m = 1; m < L; m <<= 1) l += __shfl_xor(l, m, 64);
    if (k < nrow && sub == 0) lse[k] = M + log(l);
  }
}

// lse_q_i - lse_p_i for draft position i (one wave; the result in every
// lane): log1p(S) with S = sum over the chunks of exp(M_p - lse_p) T
// (= E_p[exp(d)] - 1), which keeps the relative accuracy of T; where S is not
// in (-1/2, 2^1000) (far-apart or degenerate distributions, where the plain
// difference loses nothing that matters) the plain difference.
__device__ __forceinline__ double normaliser_gap(const AccParams &a, int b, int i, const double *lse) {
  const int lane = lane_id();
  const int nrow = 2 * a.gamma + 1;
  const double *st = a.stats + ((size_t)b * nrow + i) * a.n_chunks * 2;
  const double *cr = a.cross + ((size_t)b * a.gamma + i) * a.n_chunks;
  const double lp = lse[i];
  double S = 0.0;
  for (int c = lane; c < a.n_chunks; c += 64) {
    if (st[2 * c] != -__builtin_inf())
      S += cr[c] * exp(st[2 * c] - lp);
    else if (cr[c] != 0.0)
      S = __builtin_inf();  // q mass in a chunk where p has none
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) S += __shfl_xor(S, m, 64);
  return S > -0.5 && S < 0x1p1000 ? log1p(S) : lse[a.gamma + 1 + i] - lp;
}

// Pieces [p0, p1) of the drawn row, one wave per piece: the fp64 sum of the
// p weights of each piece into a.pieces (kind 1) and, with RESID, of the
// residual weights (kind 0).
template <int VEC, bool RESID>
__device__ __forceinline__ void residual_pieces(const AccParams &a, int b, const float *zp, const float *zq,
                                                Offset cp, Offset cd, int p0, int p1) {
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  double *pr = a.pieces + ((size_t)b * 2 + 0) * a.npieces;
  double *pp = a.pieces + ((size_t)b * 2 + 1) * a.npieces;
  for (int p = p0 + wv; p < p1; p += kResWaves) {
    const int t0 = p * kPiece + 4 * lane;
    float zpv[kPieceLoads][4], zqv[kPieceLoads][4];
#pragma unroll
    for (int j = 0; j < kPieceLoads; ++j) piece_load<VEC, RESID>(a, zp, zq, t0 + 256 * j, zpv[j], zqv[j]);
    double sp = 0.0, sr = 0.0;
#pragma unroll
    for (int j = 0; j < kPieceLoads; ++j) {
      float pw[4], rw[4];
      piece_weights<RESID>(a, cp, cd, t0 + 256 * j, zpv[j], zqv[j], pw, rw);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sp += (double)pw[e];
        if constexpr (RESID) sr += (double)rw[e];
      }
    }
    // two independent wave sums, interleaved
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      sp += __shfl_xor(sp, m, 64);
      if constexpr (RESID) sr += __shfl_xor(sr, m, 64);
    }
    if (lane == 0) {
      pp[p] = sp;
      if constexpr (RESID) pr[p] = sr;
    }
  }
}

// Residual kernel: block (s, b) recomputes sequence b's row normalisers and
// accept decisions (a few hundred statistics, cheaper than a launch between
// them), then sums the weights of slice s of the drawn row. Slice 0 writes
// n, the accepted drafts, the -1 padding and the drawn pair's normalisers.
template <int VEC>
__global__ __launch_bounds__(kResThreads) void accept_residual_kernel(AccParams a) {
  __shared__ double lse[2 * kMaxGamma + 1];
  __shared__ double gap_s;  // lse_q_n - lse_p_n of the drawn pair
  __shared__ int n_s;
  const int b = blockIdx.x, s = blockIdx.y;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int g = a.gamma;

  // Draft tokens and their logits depend on the inputs only: wave 0 fetches
  // them first, so their loads overlap the normalisers' merge below.
  int x = 0;
  float zpx = 0.f, zqx = 0.f;
  if (wv == 0 && lane < g) {
    x = clampi(a.tokens[(size_t)b * g + lane], 0, a.V - 1);
    zpx = row_ptr(a, b, lane)[x];
    zqx = row_ptr(a, b, g + 1 + lane)[x];
  }
  row_normalisers<kResWaves>(a, b, lse);
  __syncthreads();

  // Accept tests: lane i of wave 0 evaluates u_i q_i(x_i) < p_i(x_i) (fp64);
  // n is the first failing lane.
  if (wv == 0) {
    bool acc = false;  // lanes at or past gamma count as rejections (they stop the scan)
    if (lane < g) {
      const double p = exp((double)zpx * a.inv_temp_d - lse[lane]);
      const double q = exp((double)zqx * a.inv_temp_d - lse[g + 1 + lane]);
      acc = (double)a.u_accept[(size_t)b * g + lane] * q < p;
    }
    const uint64_t rej = ~__ballot(acc);
    const int n = min(g, rej != 0 ? (int)__builtin_ctzll(rej) : 64);
    const double gap = n < g ? normaliser_gap(a, b, n, lse) : 0.0;
    if (lane == 0) {
      n_s = n;
      gap_s = gap;
    }
    if (s == 0) {
      if (lane == 0) {
        a.n_accepted[b] = n;
        a.seq_n[b] = n;
        a.seq_lse[2 * (size_t)b] = lse[n];
        a.seq_lse[2 * (size_t)b + 1] = gap;
      }
      for (int t = lane; t <= g; t += 64) {
        if (t < n)
          a.out_tokens[(size_t)b * (g + 1) + t] = clampi(a.tokens[(size_t)b * g + t], 0, a.V - 1);
        else if (t > n)
          a.out_tokens[(size_t)b * (g + 1) + t] = -1;
      }
    }
  }
  __syncthreads();
  const int n = n_s;
  const float *zp = row_ptr(a, b, n);
  const float *zq = n < g ? row_ptr(a, b, g + 1 + n) : zp;
  const Offset cp = split_offset(lse[n]);
  const Offset cd = split_offset(gap_s);
  const int p0 = s * a.pps, p1 = min(p0 + a.pps, a.npieces);
  if (n < g)
    residual_pieces<VEC, true>(a, b, zp, zq, cp, cd, p0, p1);
  else
    residual_pieces<VEC, false>(a, b, zp, zq, cp, cd, p0, p1);
}

// Block sums (fp64, any order) of two values per thread.
__device__ __forceinline__ void block_sum2_f64(double &x, double &y, double (*lds_w)[2]) {
  const int lane = lane_id(), wv = threadIdx.x >> 6;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    x += __shfl_xor(x, m, 64);
    y += __shfl_xor(y, m, 64);
  }
  if (lane == 0) {
    lds_w[wv][0] = x;
    lds_w[wv][1] = y;
  }
  __syncthreads();
  x = y = 0.0;
  for (int w = 0; w < kDrawThreads / 64; ++w) {
    x += lds_w[w][0];
    y += lds_w[w][1];
  }
  __syncthreads();
}

// One wave's scan of piece p in vocabulary order: the first entry with mass
// whose cumulative weight (from `before`) exceeds thr, or -1; *last gets the
// piece's last entry with mass (-1 if none).
template <int VEC, bool RESID>
__device__ __forceinline__ int piece_rescan(const AccParams &a, const float *zp, const float *zq, Offset cp,
                                            Offset cd, int p, double before, double thr, int *last) {
  const int lane = lane_id();
  int y = -1, sl = -1;
  const int t0 = p * kPiece + 4 * lane;
  float zpv[kPieceLoads][4], zqv[kPieceLoads][4];
#pragma unroll
  for (int j = 0; j < kPieceLoads; ++j) piece_load<VEC, RESID>(a, zp, zq, t0 + 256 * j, zpv[j], zqv[j]);
#pragma unroll
  for (int j = 0; j < kPieceLoads; ++j) {
    const int t = t0 + 256 * j;
    float pw[4], rw[4];
    piece_weights<RESID>(a, cp, cd, t, zpv[j], zqv[j], pw, rw);
    double loc[4], r = 0.0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r += (double)rw[e];
      loc[e] = r;
      if (rw[e] > 0.f) sl = t + e;
    }
    const double inc = wave_incl_scan_f64(r);
    const double exc = before + (inc - r);
    int hj = 4;
#pragma unroll
    for (int e = 3; e >= 0; --e)
      if (rw[e] > 0.f && exc + loc[e] > thr) hj = e;
    const uint64_t h = __ballot(hj < 4);
    if (y < 0 && h != 0) {
      const int l = (int)__builtin_ctzll(h);
      y = p * kPiece + 256 * j + 4 * l + __shfl(hj, l, 64);
    }
    before += __shfl(inc, 63, 64);
  }
  *last = wave_max_i32(sl);
  return y;
}

// Draw kernel: one block per sequence. The residual's piece sums (or p_n's,
// when n = gamma or the residual has no mass at all, the pages' reading for
// p_n = q_n) give Z; a block scan in vocabulary order finds the first piece
// whose inclusive sum exceeds u Z, and wave 0 rescans that piece for the
// token. Rounding that leaves no crossing falls back to the last entry with
// mass (of the piece, else of the row). Up to kDrawThreads * kDrawPer pieces
// (vocabularies up to a million entries) the piece sums are loaded once and
// kept in registers.
template <int VEC>
__global__ __launch_bounds__(kDrawThreads) void accept_draw_kernel(AccParams a) {
  constexpr int kRound = kDrawThreads * kDrawPer;
  __shared__ double lds_w[kDrawThreads / 64][2];
  __shared__ double scan_w[kDrawThreads / 64];
  __shared__ int hit_w[kDrawThreads / 64];
  __shared__ int piece_s, lastp_s;
  __shared__ double before_s;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = a.gamma;
  const int n = clampi(a.seq_n[b], 0, g);
  const bool two = n < g;  // residual piece sums were written
  const double *pr = a.pieces + ((size_t)b * 2 + 0) * a.npieces;
  const double *pp = a.pieces + ((size_t)b * 2 + 1) * a.npieces;
  const int np = a.npieces;
  const bool inreg = np <= kRound;
  double vr[kDrawPer], vp[kDrawPer];
  double Zr = 0.0, Zp = 0.0;
#pragma unroll
  for (int j = 0; j < kDrawPer; ++j) {
    const int i = kDrawPer * tid + j;
    vr[j] = inreg && two && i < np ? pr[i] : 0.0;
    vp[j] = inreg && i < np ? pp[i] : 0.0;
    Zr += vr[j];
    Zp += vp[j];
  }
  if (!inreg) {
    for (int i = tid; i < np; i += kDrawThreads) {
      if (two) Zr += pr[i];
      Zp += pp[i];
    }
  }
  block_sum2_f64(Zr, Zp, lds_w);
  const bool resid = two && Zr > 0.0;
  const double *ps = resid ? pr : pp;
  const double Z = resid ? Zr : Zp;
  const double thr = (double)a.u_sample[(size_t)b * (g + 1) + n] * Z;

  // first piece with inclusive sum > thr, and the last piece with mass
  if (tid == 0) {
    piece_s = -1;
    lastp_s = -1;
  }
  __syncthreads();
  double run = 0.0;  // sum of the pieces before this round
  for (int base = 0; base < np; base += kRound) {
    double v[kDrawPer], loc = 0.0;
    int lastp = -1;
#pragma unroll
    for (int j = 0; j < kDrawPer; ++j) {
      const int i = base + kDrawPer * tid + j;
      v[j] = inreg ? (resid ? vr[j] : vp[j]) : (i < np ? ps[i] : 0.0);
      loc += v[j];
      if (v[j] > 0.0) lastp = i;
    }
    lastp = wave_max_i32(lastp);
    const double incl = wave_incl_scan_f64(loc);
    if (lane == 63) scan_w[wv] = incl;
    __syncthreads();
    double before_w = 0.0, tot = 0.0;
    for (int w2 = 0; w2 < kDrawThreads / 64; ++w2) {
      if (w2 < wv) before_w += scan_w[w2];
      tot += scan_w[w2];
    }
    double c = run + before_w + incl - loc;  // sum of the pieces before this thread's first
    int hit = -1;
    double hit_before = 0.0;
#pragma unroll
    for (int j = 0; j < kDrawPer; ++j) {
      if (hit < 0 && v[j] > 0.0 && c + v[j] > thr) {
        hit = j;
        hit_before = c;
      }
      c += v[j];
    }
    const uint64_t hb = __ballot(hit >= 0);
    if (lane == 0) hit_w[wv] = hb != 0 ? 64 * wv + (int)__builtin_ctzll(hb) : 0x7fffffff;
    if (lane == 0 && lastp >= 0) atomicMax(&lastp_s, lastp);
    __syncthreads();
    int first = 0x7fffffff;
    for (int w2 = 0; w2 < kDrawThreads / 64; ++w2) first = min(first, hit_w[w2]);
    if (first != 0x7fffffff && tid == first && piece_s < 0) {
      piece_s = base + kDrawPer * tid + hit;
      before_s = hit_before;
    }
    __syncthreads();
    if (piece_s >= 0) break;
    run += tot;
  }
  if (wv != 0) return;
  const float *zp = row_ptr(a, b, n);
  const float *zq = n < g ? row_ptr(a, b, g + 1 + n) : zp;
  const Offset cp = split_offset(a.seq_lse[2 * (size_t)b]);
  const Offset cd = split_offset(a.seq_lse[2 * (size_t)b + 1]);
  int y = -1, last = -1;
  const int piece = piece_s >= 0 ? piece_s : lastp_s;  // no crossing: the last piece with mass
  if (piece >= 0) {
    const double before = piece_s >= 0 ? before_s : 0.0;
    const double t = piece_s >= 0 ? thr : __builtin_inf();
    y = resid ? piece_rescan<VEC, true>(a, zp, zq, cp, cd, piece, before, t, &last)
              : piece_rescan<VEC, false>(a, zp, zq, cp, cd, piece, before, t, &last);
    if (y < 0) y = last;
  }
  if (lane == 0) a.out_tokens[(size_t)b * (g + 1) + n] = max(0, y);
}

struct AccPlan {
  int n_chunks;
  int npieces, pps, slices;  // pieces per row, per residual slice, slices per sequence
  size_t cross_off, pieces_off, lse_off, n_off;
  size_t ws_bytes;  // chunk statistics, cross sums, piece sums, the drawn row's normalisers, n
};

AccPlan plan_accept(int64_t B, int64_t gamma, int64_t V) {
  AccPlan p;
  p.n_chunks = (int)sdh::ceil_div(V, kChunk);
  p.npieces = (int)sdh::ceil_div(V, kPiece);
  // enough residual blocks to spread each sequence's drawn row over several CUs
  const int64_t want = std::max<int64_t>(1, sdh::ceil_div((int64_t)kTargetBlocks, B));
  const int64_t sl = std::min<int64_t>(p.npieces, want);
  p.pps = (int)sdh::ceil_div(p.npieces, sl);
  p.slices = (int)sdh::ceil_div(p.npieces, p.pps);
  p.cross_off = sdh::align_up((size_t)B * (2 * gamma + 1) * p.n_chunks * 2 * 8);
  p.pieces_off = p.cross_off + sdh::align_up((size_t)B * gamma * p.n_chunks * 8);
  p.lse_off = p.pieces_off + sdh::align_up((size_t)B * 2 * p.npieces * 8);
  p.n_off = p.lse_off + sdh::align_up((size_t)B * 2 * 8);
  p.ws_bytes = p.n_off + sdh::align_up((size_t)B * 4);
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

// Enqueue the three kernels with `workspace` (at least plan_accept's ws_bytes).
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
  a.stats = reinterpret_cast<double *>(ws);
  a.cross = reinterpret_cast<double *>(ws + p.cross_off);
  a.pieces = reinterpret_cast<double *>(ws + p.pieces_off);
  a.seq_lse = reinterpret_cast<double *>(ws + p.lse_off);
  a.seq_n = reinterpret_cast<int32_t *>(ws + p.n_off);
  a.B = batch;
  a.gamma = gamma;
  a.V = vocab;
  a.n_chunks = p.n_chunks;
  a.npieces = p.npieces;
  a.pps = p.pps;
  a.inv_temp = 1.f / temperature;
  a.inv_temp_d = 1.0 / (double)temperature;
  // 16-byte loads need every row 16-byte aligned
  const bool vec = vocab % 4 == 0 && reinterpret_cast<uintptr_t>(target_logits) % 16 == 0 &&
                   (gamma == 0 || reinterpret_cast<uintptr_t>(draft_logits) % 16 == 0);
  const dim3 g_stats((unsigned)p.n_chunks, (unsigned)(batch * (gamma + 1)));
  const dim3 g_res((unsigned)batch, (unsigned)p.slices);
  if (vec) {
    accept_stats_kernel<4><<<g_stats, kAccThreads, 0, st>>>(a);
    accept_residual_kernel<4><<<g_res, kResThreads, 0, st>>>(a);
    accept_draw_kernel<4><<<(unsigned)batch, kDrawThreads, 0, st>>>(a);
  } else {
    accept_stats_kernel<1><<<g_stats, kAccThreads, 0, st>>>(a);
    accept_residual_kernel<1><<<g_res, kResThreads, 0, st>>>(a);
    accept_draw_kernel<1><<<(unsigned)batch, kDrawThreads, 0, st>>>(a);
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
