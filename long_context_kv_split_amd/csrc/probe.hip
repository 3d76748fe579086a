// Streaming-read probe: the attainable HBM read bandwidth of this chip.
//
// MagicDec (deep notes on papercache.org, §3.2) argues that at long context
// verification and drafting are bound by loading the KV cache, so the ceiling
// every attention kernel here is measured against is the read bandwidth HBM can
// actually deliver, next to the nominal figure. This kernel measures that
// ceiling: every wave streams one contiguous slice of the buffer with 16-byte
// vector loads, eight per lane in flight (8 KB per wave and round, each load
// one contiguous 1 KB request), with the nontemporal hint as the attention
// kernels use it, or without it. The launch size is the caller's choice (the
// best size depends on the access pattern, so a measurement sweeps it). The
// 32-bit words are summed modulo 2^32 so the loads cannot be dropped; each
// wave adds its sum to the caller's counter with one vector atomic (integer
// addition, so the result does not depend on the order).
#include "sd_device.h"
#include "sd_host.h"
#include "sd_sched.h"

using namespace sdk;

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;  // 16-byte loads in flight per lane
constexpr int kMaxProbeBlocks = 65536;

template <bool NT>
__device__ __forceinline__ u32x4 probe_load(const u32x4 *p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

template <bool NT>
__global__ __launch_bounds__(kProbeThreads) void hbm_read_probe_kernel(const u32x4 *buf, int64_t n16,
                                                                       uint32_t *checksum) {
  constexpr int kWavesPerBlock = kProbeThreads / 64;
  const int64_t waves = (int64_t)gridDim.x * kWavesPerBlock;
  const int64_t w = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / 64;
  const int lane = lane_id();
  // wave w reads chunks [b0, b1): an equal contiguous slice (empty past the end)
  const int64_t seg = (n16 + waves - 1) / waves;
  const int64_t b0 = w * seg;
  const int64_t b1 = b0 + seg < n16 ? b0 + seg : n16;
  uint32_t acc = 0;
  int64_t i = b0;
  // full rounds: all 64 * kProbeUnroll chunks of the round lie inside the slice
  for (; i + 64 * kProbeUnroll <= b1; i += 64 * kProbeUnroll) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int k = 0; k < kProbeUnroll; ++k) v[k] = probe_load<NT>(buf + i + k * 64 + lane);
#pragma unroll
    for (int k = 0; k < kProbeUnroll; ++k) acc += v[k].x + v[k].y + v[k].z + v[k].w;
  }
  // rest of the slice, one guarded load at a time
  for (int64_t j = i + lane; j < b1; j += 64) {
    const u32x4 v = probe_load<NT>(buf + j);
    acc += v.x + v.y + v.z + v.w;
  }
  for (int m = 32; m >= 1; m >>= 1) acc += (uint32_t)__shfl_xor((int)acc, m, 64);
  if (lane == 0) atomicAdd(checksum, acc);
}

template <bool NT>
sd_status launch_probe(const void *buf, int64_t n16, int blocks, uint32_t *checksum, hipStream_t st) {
  if (blocks == 0) {
    // resident 256-thread blocks of this instantiation, queried once per device
    static int cache[sdh::kMaxDevices] = {};
    int dev = 0, per_cu = 0, cus = 0;
    const bool have_dev = hipGetDevice(&dev) == hipSuccess && dev >= 0;
    int *slot = have_dev && dev < sdh::kMaxDevices ? cache + dev : nullptr;
    blocks = slot ? __atomic_load_n(slot, __ATOMIC_RELAXED) : 0;
    if (blocks <= 0) {
      if (!have_dev ||
          hipOccupancyMaxActiveBlocksPerMultiprocessor(
              &per_cu, reinterpret_cast<const void *>(hbm_read_probe_kernel<NT>), kProbeThreads, 0) !=
              hipSuccess ||
          hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
          per_cu <= 0 || cus <= 0) {
        (void)hipGetLastError();
        per_cu = 4;
        cus = kNumCUs;
      }
      blocks = per_cu * cus;
      if (slot) __atomic_store_n(slot, blocks, __ATOMIC_RELAXED);
    }
  }
  hbm_read_probe_kernel<NT><<<(unsigned)blocks, kProbeThreads, 0, st>>>(reinterpret_cast<const u32x4 *>(buf),
                                                                         n16, checksum);
  return sdh::launch_status();
}

}  // namespace

extern "C" sd_status sd_hbm_read_probe(const void *buf, size_t bytes, int32_t nontemporal, int32_t blocks,
                                       uint32_t *checksum, void *stream) {
  SD_REQUIRE(buf != nullptr && checksum != nullptr, SD_ERR_INVALID_ARG);
  SD_REQUIRE(bytes > 0 && bytes % 16 == 0, SD_ERR_INVALID_ARG);
  SD_REQUIRE(reinterpret_cast<uintptr_t>(buf) % 16 == 0, SD_ERR_INVALID_ARG);
  SD_REQUIRE(reinterpret_cast<uintptr_t>(checksum) % 4 == 0, SD_ERR_INVALID_ARG);
  SD_REQUIRE(nontemporal == 0 || nontemporal == 1, SD_ERR_INVALID_ARG);
  SD_REQUIRE(blocks >= 0 && blocks <= kMaxProbeBlocks, SD_ERR_INVALID_ARG);
  SD_REQUIRE(bytes / 16 < ((uint64_t)1 << 40), SD_ERR_UNSUPPORTED);
  const int64_t n16 = (int64_t)(bytes / 16);
  hipStream_t st = sdh::as_stream(stream);
  return nontemporal ? launch_probe<true>(buf, n16, blocks, checksum, st)
                     : launch_probe<false>(buf, n16, blocks, checksum, st);
}
