// Host-side helpers shared by the entry points: argument checks, workspace
// carving and launch-error mapping. Every check here runs before any HIP call.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sd.h"

namespace sdh {

#define SD_REQUIRE(cond, code) \
  do {                         \
    if (!(cond)) return (code);\
  } while (0)

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

inline size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline sd_status launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? SD_OK : SD_ERR_HIP;
}

inline int dtype_bytes(int32_t dtype) { return dtype == SD_BF16 ? 2 : (dtype == SD_F32 ? 4 : 0); }

// The kernels move K, V and query rows in 16-byte pieces.
inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Checks common to every call that reads the paged cache.
inline sd_status check_kv(const sd_kv_cache *kv, bool need_v) {
  SD_REQUIRE(kv != nullptr, SD_ERR_INVALID_ARG);
  SD_REQUIRE(kv->k_pages != nullptr && kv->page_table != nullptr && kv->kv_lens != nullptr,
             SD_ERR_INVALID_ARG);
  SD_REQUIRE(!need_v || kv->v_pages != nullptr, SD_ERR_INVALID_ARG);
  SD_REQUIRE(aligned16(kv->k_pages) && (!need_v || aligned16(kv->v_pages)), SD_ERR_INVALID_ARG);
  SD_REQUIRE(kv->num_pages > 0 && kv->page_size > 0 && kv->max_pages > 0 && kv->num_kv_heads > 0 &&
                 kv->head_dim > 0,
             SD_ERR_INVALID_ARG);
  SD_REQUIRE(kv->dtype == SD_BF16 || kv->dtype == SD_F32, SD_ERR_UNSUPPORTED);
  SD_REQUIRE(kv->page_size % 16 == 0, SD_ERR_UNSUPPORTED);
  SD_REQUIRE(kv->head_dim == 64 || kv->head_dim == 128, SD_ERR_UNSUPPORTED);
  SD_REQUIRE((int64_t)kv->num_pages * kv->num_kv_heads * kv->page_size < (int64_t)1 << 31,
             SD_ERR_UNSUPPORTED);
  SD_REQUIRE((int64_t)kv->max_pages * kv->page_size < (int64_t)1 << 30, SD_ERR_UNSUPPORTED);
  return SD_OK;
}

}  // namespace sdh
