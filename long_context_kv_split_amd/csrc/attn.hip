// Paged GQA attention for the verify pass and the sparse draft pass, gfx950.
//
// MagicDec (deep notes on papercache.org, §3.2) observes that at long context
// both verification and drafting are bound by loading the KV cache; the verify
// pass reads all of it for gamma+1 causal queries per sequence, the draft pass
// (§3.3, §4.1) reads only K selected tokens. One kernel template serves both:
// a "step" is 16 cached tokens, taken from consecutive positions of one page
// (verify) or from 16 entries of a selection list (draft).
//
// Work split (split-KV): one wavefront per (sequence, KV head, chunk of
// steps). The G*n_q query rows that share the KV head are padded to NB tiles
// of 16 rows. Per step the wave computes S^T = K Q^T with 16x16x32 bf16 MFMA
// (tokens on M, query rows on N), applies the mask and an online softmax in
// the log2 domain, and accumulates O^T += V^T P^T with 16x16x16 bf16 MFMA.
// The accumulator layout of the first product is exactly the B-operand layout
// of the second, so P never leaves registers. V^T is formed from plain 16-byte
// row loads: lane (g, r) loads d-range [DPL*r, DPL*r+DPL) of tokens 4g..4g+3 and
// builds the A operand of d-tile dt from element dt of those four rows
// (v_perm), which assigns head-dim index DPL*m + dt to MFMA row m.
// A combine kernel merges the per-chunk (m, l, o) partials by log-sum-exp.
// float32 caches use the same structure with 16x16x4 f32 MFMA.
#include "sd_device.h"
#include "sd_host.h"

#include <algorithm>

using namespace sdk;

namespace {

constexpr int kStepTokens = 16;
constexpr int kTargetWaves = 16384;

struct AttnParams {
  const void *k_pages;
  const void *v_pages;
  const int32_t *page_table;
  const int32_t *lens;  // kv_lens (verify) or sel_lens (draft)
  const int32_t *idx;   // draft: [B, idx_heads, max_sel]
  const void *q;        // [B, n_q, Hq, D]
  float *part_o;        // [B*Hkv*max_chunks, rows, D]
  float *part_ml;       // [B*Hkv*max_chunks, rows, 2]
  int32_t n_q, Hq, Hkv, G, rows;
  int32_t num_pages, page_size, max_pages;
  int32_t idx_heads, max_sel;
  int32_t len_cap;  // upper clamp of lens
  int32_t chunk_steps, max_chunks;
  float scale_log2;
};

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
      u32x4 t = *reinterpret_cast<const u32x4 *>(p + 16 * i);
      dst[4 * i + 0] = t.x;
      dst[4 * i + 1] = t.y;
      dst[4 * i + 2] = t.z;
      dst[4 * i + 3] = t.w;
    }
  } else {
    static_assert(N == 2, "unsupported V slice");
    u32x2 t = *reinterpret_cast<const u32x2 *>(p);
    dst[0] = t.x;
    dst[1] = t.y;
  }
}

// Row index (page*Hkv + kvh)*P + slot of the cached token this lane's K load
// and the four V loads use, for step s.
template <bool SPARSE>
__device__ __forceinline__ int token_row(const AttnParams &a, int b, int kvh, int s, int len,
                                         const int32_t *idx_row, int t_in_step) {
  int pos;
  if constexpr (SPARSE) {
    int t = clampi(s * kStepTokens + t_in_step, 0, len - 1);
    pos = clampi(idx_row[t], 0, a.max_pages * a.page_size - 1);
  } else {
    pos = s * kStepTokens + t_in_step;
  }
  int page = a.page_table[(size_t)b * a.max_pages + pos / a.page_size];
  page = clampi(page, 0, a.num_pages - 1);
  return (page * a.Hkv + kvh) * a.page_size + pos % a.page_size;
}

template <typename T, int D, bool SPARSE>
__device__ __forceinline__ void load_step(const AttnParams &a, int b, int kvh, int s, int len,
                                          const int32_t *idx_row, StepRegs<T, D> &R) {
  constexpr int EB = EltInfo<T>::bytes;
  constexpr int DPL = D / 16;
  const int lane = lane_id();
  const int g = lane >> 4, r = lane & 15;
  // K: token r of the step; V: tokens 4g..4g+3 (their row ids come from the
  // lanes that computed them).
  int rowK = token_row<SPARSE>(a, b, kvh, s, len, idx_row, r);
  const char *kb = reinterpret_cast<const char *>(a.k_pages) + (size_t)rowK * D * EB;
  if constexpr (EB == 2) {
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      R.k[kk] = *reinterpret_cast<const u32x4 *>(kb + (32 * kk + 8 * g) * EB);
  } else {
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
      R.k[c] = *reinterpret_cast<const u32x4 *>(kb + ((D / 4) * g + 4 * c) * EB);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int rowV = __shfl(rowK, 4 * g + j, 64);
    const char *vb = reinterpret_cast<const char *>(a.v_pages) + ((size_t)rowV * D + DPL * r) * EB;
    load_dwords(R.v[j], vb);
  }
}

template <typename T, int D, int NB, bool SPARSE>
__global__ __launch_bounds__(64) void attn_split_kernel(AttnParams a) {
  constexpr int EB = EltInfo<T>::bytes;
  constexpr int DPL = D / 16;  // head-dim values per lane per token row of V
  const int lane = lane_id();
  const int g = lane >> 4, r = lane & 15;

  int unit = blockIdx.x;
  const int chunk = unit % a.max_chunks;
  unit /= a.max_chunks;
  const int kvh = unit % a.Hkv;
  const int b = unit / a.Hkv;
  const int len = clampi(a.lens[b], 0, a.len_cap);
  const int n_steps = (len + kStepTokens - 1) / kStepTokens;
  const int s_begin = chunk * a.chunk_steps;
  if (s_begin >= n_steps) return;
  const int s_end = min(n_steps, s_begin + a.chunk_steps);
  const int32_t *idx_row = nullptr;
  if constexpr (SPARSE)
    idx_row = a.idx + ((size_t)b * a.idx_heads + (a.idx_heads > 1 ? kvh : 0)) * a.max_sel;

  // Query operands and each row's last visible position.
  constexpr int QV = StepRegs<T, D>::kVec;
  u32x4 qreg[NB][QV];
  int lim[NB];
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
    const int R = rb * 16 + r;
    int i = 0, hl = 0;
    bool live = R < a.rows;
    if (live) {
      i = R / a.G;
      hl = R % a.G;
    }
    lim[rb] = SPARSE ? len - 1 : (live ? len - a.n_q + i : len - 1);
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
      qreg[rb][c] = v;
    }
  }
  const int lim_min = SPARSE ? len - 1 : len - a.n_q;  // smallest limit of any real row

  f32x4 acc_o[NB][DPL];
  float m_run[NB], l_run[NB];
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
    m_run[rb] = kNegInf;
    l_run[rb] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DPL; ++dt) acc_o[rb][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  StepRegs<T, D> cur, nxt;
  load_step<T, D, SPARSE>(a, b, kvh, s_begin, len, idx_row, cur);

  for (int s = s_begin; s < s_end; ++s) {
    if (s + 1 < s_end) load_step<T, D, SPARSE>(a, b, kvh, s + 1, len, idx_row, nxt);
    const int tok0 = s * kStepTokens;
    const bool boundary = tok0 + kStepTokens - 1 > lim_min;

    if (boundary) {  // zero V rows of tokens no row may see (they can hold NaN)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (tok0 + 4 * g + j >= len)
#pragma unroll
          for (int w = 0; w < StepRegs<T, D>::kVDwords; ++w) cur.v[j][w] = 0u;
    }

    // V^T operands, shared by all row tiles.
    constexpr int NA = (EB == 2) ? DPL : DPL * 4;
    uint32_t va[NA][EB == 2 ? 2 : 1];
    if constexpr (EB == 2) {
#pragma unroll
      for (int dt = 0; dt < DPL; ++dt) {
        const bool hi = dt & 1;
        va[dt][0] = pick_halves(cur.v[0][dt / 2], cur.v[1][dt / 2], hi);
        va[dt][1] = pick_halves(cur.v[2][dt / 2], cur.v[3][dt / 2], hi);
      }
    }

#pragma unroll
    for (int rb = 0; rb < NB; ++rb) {
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (EB == 2) {
#pragma unroll
        for (int c = 0; c < QV; ++c) sc = mfma_16x16x32_bf16(cur.k[c], qreg[rb][c], sc);
      } else {
        // (__uint_as_float, not __builtin_bit_cast: the latter applied to an
        // ext-vector element miscompiles to the first element with this clang)
#pragma unroll
        for (int c = 0; c < QV; ++c) {
          sc = mfma_16x16x4_f32(__uint_as_float(cur.k[c].x),
                                __uint_as_float(qreg[rb][c].x), sc);
          sc = mfma_16x16x4_f32(__uint_as_float(cur.k[c].y),
                                __uint_as_float(qreg[rb][c].y), sc);
          sc = mfma_16x16x4_f32(__uint_as_float(cur.k[c].z),
                                __uint_as_float(qreg[rb][c].z), sc);
          sc = mfma_16x16x4_f32(__uint_as_float(cur.k[c].w),
                                __uint_as_float(qreg[rb][c].w), sc);
        }
      }
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = sc[e] * a.scale_log2;
      if (boundary) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (tok0 + 4 * g + e > lim[rb]) p[e] = kNegInf;
      }
      float mx = fmaxf(fmaxf(p[0], p[1]), fmaxf(p[2], p[3]));
      mx = wave_max_xor(mx, 16);
      mx = wave_max_xor(mx, 32);
      const float m_new = fmaxf(m_run[rb], mx);
      if (__ballot(m_new > m_run[rb]) != 0) {
        const float alpha = (m_new == m_run[rb]) ? 1.f : __builtin_amdgcn_exp2f(m_run[rb] - m_new);
        l_run[rb] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DPL; ++dt) acc_o[rb][dt] *= alpha;
        m_run[rb] = m_new;
      }
      const float mu = (m_run[rb] == kNegInf) ? 0.f : m_run[rb];
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = __builtin_amdgcn_exp2f(p[e] - mu);
      l_run[rb] += (p[0] + p[1]) + (p[2] + p[3]);

      if constexpr (EB == 2) {
        u32x2 pb = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
#pragma unroll
        for (int dt = 0; dt < DPL; ++dt) {
          u32x2 av = {va[dt][0], va[dt][1]};
          acc_o[rb][dt] = mfma_16x16x16_bf16(av, pb, acc_o[rb][dt]);
        }
      } else {
#pragma unroll
        for (int dt = 0; dt < DPL; ++dt)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc_o[rb][dt] = mfma_16x16x4_f32(__uint_as_float(cur.v[j][dt]), p[j],
                                             acc_o[rb][dt]);
      }
    }
    if (s + 1 < s_end) cur = nxt;
  }

  // Partials: unnormalised o (relative to m), and (m, l) in the log2 domain.
  const size_t uc = ((size_t)b * a.Hkv + kvh) * a.max_chunks + chunk;
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
    const int R = rb * 16 + r;
    float l = l_run[rb];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (R < a.rows) {
      float *dst = a.part_o + (uc * a.rows + R) * D + 4 * DPL * g;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float vals[DPL];
#pragma unroll
        for (int dt = 0; dt < DPL; ++dt) vals[dt] = acc_o[rb][dt][e];
#pragma unroll
        for (int w = 0; w < DPL; w += 4)
          *reinterpret_cast<f32x4 *>(dst + DPL * e + w) =
              f32x4{vals[w], vals[w + 1], vals[w + 2], vals[w + 3]};
      }
      if (g == 0) {
        a.part_ml[(uc * a.rows + R) * 2 + 0] = m_run[rb];
        a.part_ml[(uc * a.rows + R) * 2 + 1] = l;
      }
    }
  }
}

// One wave per output row (b, kvh, R): merge chunk partials by log-sum-exp.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnParams a, void *out, float *lse,
                                                           int total_rows) {
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wave >= total_rows) return;
  const int lane = lane_id();
  const int R = wave % a.rows;
  const int bk = wave / a.rows;
  const int kvh = bk % a.Hkv;
  const int b = bk / a.Hkv;
  const int len = clampi(a.lens[b], 0, a.len_cap);
  const int n_steps = (len + kStepTokens - 1) / kStepTokens;
  const int n_chunks = min(a.max_chunks, (n_steps + a.chunk_steps - 1) / a.chunk_steps);
  const size_t uc0 = ((size_t)b * a.Hkv + kvh) * a.max_chunks;

  float M = kNegInf;
  for (int c = 0; c < n_chunks; ++c) M = fmaxf(M, a.part_ml[((uc0 + c) * a.rows + R) * 2]);
  constexpr int PER = D / 64;
  float o[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) o[k] = 0.f;
  float L = 0.f;
  if (M != kNegInf) {
    for (int c = 0; c < n_chunks; ++c) {
      const size_t base = (uc0 + c) * a.rows + R;
      const float mc = a.part_ml[base * 2];
      if (mc == kNegInf) continue;
      const float w = __builtin_amdgcn_exp2f(mc - M);
      L += w * a.part_ml[base * 2 + 1];
#pragma unroll
      for (int k = 0; k < PER; ++k) o[k] += w * a.part_o[base * D + lane * PER + k];
    }
  }
  const int i = R / a.G, hl = R % a.G;
  const size_t orow = (((size_t)b * a.n_q + i) * a.Hq + (size_t)kvh * a.G + hl);
  const bool empty = !(L > 0.f);
  const float inv = empty ? 0.f : 1.f / L;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const float v = o[k] * inv;
    if constexpr (EltInfo<T>::bytes == 2)
      reinterpret_cast<uint16_t *>(out)[orow * D + lane * PER + k] = (uint16_t)f32_to_bf16_bits(v);
    else
      reinterpret_cast<float *>(out)[orow * D + lane * PER + k] = v;
  }
  if (lse != nullptr && lane == 0) lse[orow] = empty ? kNegInf : (M + __log2f(L)) * kLn2;
}

struct SplitPlan {
  int chunk_steps;
  int max_chunks;
  size_t o_bytes, ml_bytes, ws_bytes;
};

SplitPlan plan_split(int64_t B, int64_t Hkv, int64_t rows, int64_t D, int64_t max_len) {
  SplitPlan p;
  const int64_t steps = std::max<int64_t>(1, sdh::ceil_div(max_len, kStepTokens));
  const int64_t units = B * Hkv;
  int64_t cs = sdh::ceil_div(steps * units, kTargetWaves);
  cs = std::max<int64_t>(cs, std::max<int64_t>(8, 2 * rows));
  cs = std::min<int64_t>(cs, steps);
  p.chunk_steps = (int)cs;
  p.max_chunks = (int)sdh::ceil_div(steps, cs);
  const int64_t slots = units * p.max_chunks * rows;
  p.o_bytes = sdh::align_up((size_t)slots * D * 4);
  p.ml_bytes = sdh::align_up((size_t)slots * 2 * 4);
  p.ws_bytes = p.o_bytes + p.ml_bytes;
  return p;
}

template <typename T, int D, bool SPARSE>
sd_status launch_attn(AttnParams &a, int B, int NB, void *out, float *lse, hipStream_t st) {
  const unsigned grid = (unsigned)((size_t)B * a.Hkv * a.max_chunks);
  switch (NB) {
    case 1: attn_split_kernel<T, D, 1, SPARSE><<<grid, 64, 0, st>>>(a); break;
    case 2: attn_split_kernel<T, D, 2, SPARSE><<<grid, 64, 0, st>>>(a); break;
    case 3: attn_split_kernel<T, D, 3, SPARSE><<<grid, 64, 0, st>>>(a); break;
    case 4: attn_split_kernel<T, D, 4, SPARSE><<<grid, 64, 0, st>>>(a); break;
    default: return SD_ERR_UNSUPPORTED;
  }
  const int total_rows = B * a.Hkv * a.rows;
  attn_combine_kernel<T, D><<<(total_rows + 3) / 4, 256, 0, st>>>(a, out, lse, total_rows);
  return sdh::launch_status();
}

template <bool SPARSE>
sd_status run_attn(AttnParams &a, int B, int D, int dtype, void *out, float *lse, hipStream_t st) {
  const int NB = (a.rows + 15) / 16;
  if (dtype == SD_BF16) {
    if (D == 128) return launch_attn<__bf16, 128, SPARSE>(a, B, NB, out, lse, st);
    return launch_attn<__bf16, 64, SPARSE>(a, B, NB, out, lse, st);
  }
  if (D == 128) return launch_attn<float, 128, SPARSE>(a, B, NB, out, lse, st);
  return launch_attn<float, 64, SPARSE>(a, B, NB, out, lse, st);
}

sd_status common_checks(const sd_kv_cache *kv, const void *q, int32_t batch, int32_t n_q,
                        int32_t num_q_heads, void *out) {
  sd_status s = sdh::check_kv(kv, true);
  if (s != SD_OK) return s;
  SD_REQUIRE(q != nullptr && out != nullptr, SD_ERR_INVALID_ARG);
  SD_REQUIRE(batch > 0 && n_q > 0 && num_q_heads > 0, SD_ERR_INVALID_ARG);
  SD_REQUIRE(num_q_heads % kv->num_kv_heads == 0, SD_ERR_INVALID_ARG);
  SD_REQUIRE((int64_t)(num_q_heads / kv->num_kv_heads) * n_q <= 64, SD_ERR_UNSUPPORTED);
  return SD_OK;
}

}  // namespace

extern "C" size_t sd_verify_attn_workspace_size(int32_t batch, int32_t n_q, int32_t num_q_heads,
                                                int32_t num_kv_heads, int32_t head_dim,
                                                int32_t max_kv_len) {
  if (batch <= 0 || n_q <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_kv_len < 0 || num_q_heads % num_kv_heads != 0)
    return 0;
  const int rows = num_q_heads / num_kv_heads * n_q;
  return plan_split(batch, num_kv_heads, rows, head_dim, max_kv_len).ws_bytes;
}

extern "C" sd_status sd_verify_attn(const sd_kv_cache *kv, const void *q, int32_t batch, int32_t n_q,
                                    int32_t num_q_heads, int32_t max_kv_len, float softmax_scale,
                                    void *out, float *lse, void *workspace, size_t workspace_bytes,
                                    void *stream) {
  sd_status s = common_checks(kv, q, batch, n_q, num_q_heads, out);
  if (s != SD_OK) return s;
  SD_REQUIRE(max_kv_len >= 0 && (int64_t)max_kv_len <= (int64_t)kv->max_pages * kv->page_size,
             SD_ERR_INVALID_ARG);
  SD_REQUIRE(softmax_scale == softmax_scale, SD_ERR_INVALID_ARG);
  const int G = num_q_heads / kv->num_kv_heads;
  const int rows = G * n_q;
  SplitPlan p = plan_split(batch, kv->num_kv_heads, rows, kv->head_dim, max_kv_len);
  SD_REQUIRE(workspace != nullptr && workspace_bytes >= p.ws_bytes, SD_ERR_WORKSPACE);

  AttnParams a{};
  a.k_pages = kv->k_pages;
  a.v_pages = kv->v_pages;
  a.page_table = kv->page_table;
  a.lens = kv->kv_lens;
  a.idx = nullptr;
  a.q = q;
  a.part_o = reinterpret_cast<float *>(workspace);
  a.part_ml = reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) + p.o_bytes);
  a.n_q = n_q;
  a.Hq = num_q_heads;
  a.Hkv = kv->num_kv_heads;
  a.G = G;
  a.rows = rows;
  a.num_pages = kv->num_pages;
  a.page_size = kv->page_size;
  a.max_pages = kv->max_pages;
  a.idx_heads = 1;
  a.max_sel = 0;
  a.len_cap = max_kv_len;
  a.chunk_steps = p.chunk_steps;
  a.max_chunks = p.max_chunks;
  a.scale_log2 = softmax_scale * kLog2e;
  return run_attn<false>(a, batch, kv->head_dim, kv->dtype, out, lse, sdh::as_stream(stream));
}

extern "C" size_t sd_draft_attn_sparse_workspace_size(int32_t batch, int32_t n_q,
                                                      int32_t num_q_heads, int32_t num_kv_heads,
                                                      int32_t head_dim, int32_t max_sel) {
  return sd_verify_attn_workspace_size(batch, n_q, num_q_heads, num_kv_heads, head_dim, max_sel);
}

extern "C" sd_status sd_draft_attn_sparse(const sd_kv_cache *kv, const void *q, int32_t batch,
                                          int32_t n_q, int32_t num_q_heads, const int32_t *idx,
                                          const int32_t *sel_lens, int32_t idx_heads,
                                          int32_t max_sel, float softmax_scale, void *out,
                                          float *lse, void *workspace, size_t workspace_bytes,
                                          void *stream) {
  sd_status s = common_checks(kv, q, batch, n_q, num_q_heads, out);
  if (s != SD_OK) return s;
  SD_REQUIRE(idx != nullptr && sel_lens != nullptr, SD_ERR_INVALID_ARG);
  SD_REQUIRE(idx_heads == 1 || idx_heads == kv->num_kv_heads, SD_ERR_INVALID_ARG);
  SD_REQUIRE(max_sel > 0, SD_ERR_INVALID_ARG);
  SD_REQUIRE(softmax_scale == softmax_scale, SD_ERR_INVALID_ARG);
  const int G = num_q_heads / kv->num_kv_heads;
  const int rows = G * n_q;
  SplitPlan p = plan_split(batch, kv->num_kv_heads, rows, kv->head_dim, max_sel);
  SD_REQUIRE(workspace != nullptr && workspace_bytes >= p.ws_bytes, SD_ERR_WORKSPACE);

  AttnParams a{};
  a.k_pages = kv->k_pages;
  a.v_pages = kv->v_pages;
  a.page_table = kv->page_table;
  a.lens = sel_lens;
  a.idx = idx;
  a.q = q;
  a.part_o = reinterpret_cast<float *>(workspace);
  a.part_ml = reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) + p.o_bytes);
  a.n_q = n_q;
  a.Hq = num_q_heads;
  a.Hkv = kv->num_kv_heads;
  a.G = G;
  a.rows = rows;
  a.num_pages = kv->num_pages;
  a.page_size = kv->page_size;
  a.max_pages = kv->max_pages;
  a.idx_heads = idx_heads;
  a.max_sel = max_sel;
  a.len_cap = max_sel;
  a.chunk_steps = p.chunk_steps;
  a.max_chunks = p.max_chunks;
  a.scale_log2 = softmax_scale * kLog2e;
  return run_attn<true>(a, batch, kv->head_dim, kv->dtype, out, lse, sdh::as_stream(stream));
}
