// Cache bookkeeping of a self-speculative round on gfx950: append new tokens'
// K/V to the paged cache and move the per-sequence lengths.
//
// MagicDec (deep notes on papercache.org, §3.1-§3.3, §4.1): the draft proposes
// gamma tokens one at a time over the compressed cache, the target scores the
// candidate positions in one batched pass over the full cache, and a prefix of
// the drafts is kept. New tokens' K/V go to the end of each sequence (position
// kv_lens[b] + j, page page_table[b][pos / P], slot pos % P); after acceptance
// the length drops the rejected drafts (kv_len - gamma + n). The draft's
// compressed cache can also be copied out once, as a cache of its own whose
// dense decode is the draft over the selection (kv_compact).
#include "sd_device.h"
#include "sd_host.h"

using namespace sdk;

namespace {

constexpr int kAppendThreads = 256;

// One thread per 16-byte chunk of a new row. Rows whose position lies past
// the page table are not written; page ids are clamped into the pool.
__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(
    char *k_pages, char *v_pages, const char *k_new, const char *v_new, const int32_t *page_table,
    const int32_t *kv_lens, int64_t n_chunks, int32_t n_new, int32_t Hkv, int32_t row_chunks,
    int32_t page_size, int32_t max_pages, int32_t num_pages) {
  const int64_t c = (int64_t)blockIdx.x * kAppendThreads + threadIdx.x;
  if (c >= n_chunks) return;
  const int64_t row = c / row_chunks;  // (b, j, kvh) of k_new [B, n_new, Hkv, D]
  const int ch = (int)(c % row_chunks);
  const int kvh = (int)(row % Hkv);
  const int64_t bj = row / Hkv;
  const int j = (int)(bj % n_new);
  const int b = (int)(bj / n_new);
  const int64_t pos = (int64_t)max(0, kv_lens[b]) + j;
  if (pos >= (int64_t)max_pages * page_size) return;
  const int page = clampi(page_table[(size_t)b * max_pages + pos / page_size], 0, num_pages - 1);
  const int64_t dst = ((int64_t)(page * Hkv + kvh) * page_size + pos % page_size) * row_chunks + ch;
  reinterpret_cast<u32x4 *>(k_pages)[dst] = reinterpret_cast<const u32x4 *>(k_new)[c];
  reinterpret_cast<u32x4 *>(v_pages)[dst] = reinterpret_cast<const u32x4 *>(v_new)[c];
}

// One thread per 16-byte chunk of a compact-cache row, ordered as the output
// is laid out: (sequence b, output page j, KV head h, slot, chunk) with the
// chunk fastest, so a workgroup writes whole 4 KB (page, head) blocks and
// only the reads are gathered. List entry t = j P + slot; entries past the
// sequence's selection are not written; positions, page ids and lengths are
// clamped into range.
__global__ __launch_bounds__(kAppendThreads) void kv_compact_kernel(
    char *k_out, char *v_out, const char *k_pages, const char *v_pages, const int32_t *page_table,
    const int32_t *idx, const int32_t *sel_lens, int64_t n_chunks, int32_t max_sel, int32_t idx_heads,
    int32_t pages_per_seq, int32_t used_pages, int32_t Hkv, int32_t row_chunks, int32_t page_size,
    int32_t max_pages, int32_t num_pages) {
  const int64_t c = (int64_t)blockIdx.x * kAppendThreads + threadIdx.x;
  if (c >= n_chunks) return;
  const int ch = (int)(c % row_chunks);
  const int64_t row = c / row_chunks;
  const int slot = (int)(row % page_size);
  const int64_t ph = row / page_size;
  const int h = (int)(ph % Hkv);
  const int64_t bj = ph / Hkv;
  const int j = (int)(bj % used_pages);
  const int b = (int)(bj / used_pages);
  const int t = j * page_size + slot;
  if (t >= clampi(sel_lens[b], 0, max_sel)) return;
  const int pos = clampi(idx[((size_t)b * idx_heads + (idx_heads > 1 ? h : 0)) * max_sel + t], 0,
                         max_pages * page_size - 1);
  const int page = clampi(page_table[(size_t)b * max_pages + pos / page_size], 0, num_pages - 1);
  const int64_t src = ((int64_t)(page * Hkv + h) * page_size + pos % page_size) * row_chunks + ch;
  const int64_t dst = ((((int64_t)b * pages_per_seq + j) * Hkv + h) * page_size + slot) * row_chunks + ch;
  const u32x4 kv_k = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(k_pages) + src);
  const u32x4 kv_v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(v_pages) + src);
  reinterpret_cast<u32x4 *>(k_out)[dst] = kv_k;
  reinterpret_cast<u32x4 *>(v_out)[dst] = kv_v;
}

__global__ __launch_bounds__(256) void kv_advance_kernel(int32_t *kv_lens, const int32_t *n_accepted,
                                                         int32_t batch, int32_t add) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= batch) return;
  const int n = n_accepted ? n_accepted[b] : 0;
  kv_lens[b] = max(0, kv_lens[b] + add + n);
}

}  // namespace

extern "C" sd_status sd_kv_append(const sd_kv_cache *kv, const void *k_new, const void *v_new,
                                  int32_t batch, int32_t n_new, void *stream) {
  sd_status s = sdh::check_kv(kv, true);
  if (s != SD_OK) return s;
  SD_REQUIRE(k_new != nullptr && v_new != nullptr, SD_ERR_INVALID_ARG);
  SD_REQUIRE(sdh::aligned16(k_new) && sdh::aligned16(v_new), SD_ERR_INVALID_ARG);
  SD_REQUIRE(batch > 0 && n_new >= 0, SD_ERR_INVALID_ARG);
  if (n_new == 0) return SD_OK;
  const int row_chunks = kv->head_dim * sdh::dtype_bytes(kv->dtype) / 16;
  const int64_t n_chunks = (int64_t)batch * n_new * kv->num_kv_heads * row_chunks;
  SD_REQUIRE(n_chunks / kAppendThreads < ((int64_t)1 << 31), SD_ERR_UNSUPPORTED);
  kv_append_kernel<<<(unsigned)((n_chunks + kAppendThreads - 1) / kAppendThreads), kAppendThreads, 0,
                     sdh::as_stream(stream)>>>(
      // the pools are the cache's own storage: this call is the one that writes them
      const_cast<char *>(reinterpret_cast<const char *>(kv->k_pages)),
      const_cast<char *>(reinterpret_cast<const char *>(kv->v_pages)), reinterpret_cast<const char *>(k_new),
      reinterpret_cast<const char *>(v_new), kv->page_table, kv->kv_lens, n_chunks, n_new, kv->num_kv_heads,
      row_chunks, kv->page_size, kv->max_pages, kv->num_pages);
  return sdh::launch_status();
}

extern "C" sd_status sd_kv_advance(int32_t *kv_lens, const int32_t *n_accepted, int32_t batch, int32_t add,
                                   void *stream) {
  SD_REQUIRE(kv_lens != nullptr && batch > 0, SD_ERR_INVALID_ARG);
  kv_advance_kernel<<<(unsigned)((batch + 255) / 256), 256, 0, sdh::as_stream(stream)>>>(kv_lens, n_accepted,
                                                                                         batch, add);
  return sdh::launch_status();
}

extern "C" sd_status sd_kv_compact(const sd_kv_cache *kv, const int32_t *idx, const int32_t *sel_lens,
                                   int32_t batch, int32_t idx_heads, int32_t max_sel, int32_t pages_per_seq,
                                   void *k_out, void *v_out, void *stream) {
  sd_status s = sdh::check_kv(kv, true);
  if (s != SD_OK) return s;
  SD_REQUIRE(idx != nullptr && sel_lens != nullptr && k_out != nullptr && v_out != nullptr, SD_ERR_INVALID_ARG);
  SD_REQUIRE(sdh::aligned16(k_out) && sdh::aligned16(v_out), SD_ERR_INVALID_ARG);
  SD_REQUIRE(batch > 0 && max_sel >= 1, SD_ERR_INVALID_ARG);
  SD_REQUIRE(idx_heads == 1 || idx_heads == kv->num_kv_heads, SD_ERR_INVALID_ARG);
  SD_REQUIRE(pages_per_seq >= sdh::ceil_div(max_sel, kv->page_size), SD_ERR_INVALID_ARG);
  // the compact pool must itself be addressable as a cache
  SD_REQUIRE((int64_t)batch * pages_per_seq * kv->num_kv_heads * kv->page_size < ((int64_t)1 << 31),
             SD_ERR_UNSUPPORTED);
  const int row_chunks = kv->head_dim * sdh::dtype_bytes(kv->dtype) / 16;
  const int used_pages = sdh::ceil_div(max_sel, kv->page_size);  // output pages a selection can fill
  const int64_t n_chunks = (int64_t)batch * used_pages * kv->num_kv_heads * kv->page_size * row_chunks;
  SD_REQUIRE(n_chunks / kAppendThreads < ((int64_t)1 << 31), SD_ERR_UNSUPPORTED);
  kv_compact_kernel<<<(unsigned)((n_chunks + kAppendThreads - 1) / kAppendThreads), kAppendThreads, 0,
                      sdh::as_stream(stream)>>>(
      reinterpret_cast<char *>(k_out), reinterpret_cast<char *>(v_out), reinterpret_cast<const char *>(kv->k_pages),
      reinterpret_cast<const char *>(kv->v_pages), kv->page_table, idx, sel_lens, n_chunks, max_sel, idx_heads,
      pages_per_seq, used_pages, kv->num_kv_heads, row_chunks, kv->page_size, kv->max_pages, kv->num_pages);
  return sdh::launch_status();
}
