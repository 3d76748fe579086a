// Device helpers for the gfx950 kernels: vector types, MFMA wrappers,
// bf16 packing and wave-level reductions. Only the HIP library includes this.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdk {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short short4v;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// 16x16x32 bf16 MFMA: lane l supplies A[m = l%16][8 k-values] and
// B[8 k-values][n = l%16]; both operands use the same lane->k assignment, so
// any consistent split of the reduction axis over lanes is valid.
__device__ __forceinline__ f32x4 mfma_16x16x32_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 16x16x16 bf16 MFMA: lane l supplies A[m = l%16][k = 4(l/16) .. +3] and
// B[k = 4(l/16) .. +3][n = l%16] (element e of the packed pair-of-dwords is k = 4(l/16)+e).
__device__ __forceinline__ f32x4 mfma_16x16x16_bf16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4v, a),
                                                   __builtin_bit_cast(short4v, b), c, 0, 0, 0);
}

// 16x16x4 f32 MFMA: lane l supplies A[m = l%16][k = l/16] and B[k = l/16][n = l%16].
__device__ __forceinline__ f32x4 mfma_16x16x4_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// In all three, the accumulator of lane l holds C[m = 4(l/16) + e][n = l%16], e = 0..3.

// Round-to-nearest-even float -> bf16 bits (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Pack two floats as bf16 (lo in bits 0-15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Two 16-bit halves taken from two dwords: the low halves (hi_half=false) or
// the high halves (hi_half=true); x supplies bits 0-15 of the result, y 16-31.
__device__ __forceinline__ uint32_t pick_halves(uint32_t x, uint32_t y, bool hi_half) {
  return __builtin_amdgcn_perm(y, x, hi_half ? 0x07060302u : 0x05040100u);
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// A well-mixed 32-bit hash of a stream segment (wave-uniform inputs).
__device__ __forceinline__ uint32_t segment_hash(int b, int kvh, int s_begin) {
  uint32_t h = (uint32_t)b * 0x9E3779B1u ^ (uint32_t)kvh * 0x85EBCA77u ^ (uint32_t)s_begin * 0xC2B2AE3Du;
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 13;
  return h;
}

// A permuted walk over n steps: position v reads step (A v + rot) mod n, A a
// small prime that does not divide n (so the map is a bijection) and rot a
// hash of the segment. Consecutive reads of a wave land A steps apart and
// waves start at unrelated offsets: walking a sequence's pages in order puts
// a wave's successive 4 KB blocks at one fixed stride, and pages laid out in
// order then read measurably slower than shuffled ones.
// Segments shorter than this walk in order: on the 8k-context batch (128
// steps per wave) the permuted walk measured 1-2% slower.
constexpr int kWalkMinSteps = 256;

struct StepWalk {
  int n;
  uint32_t A, rot;
  __device__ StepWalk() : n(0), A(1u), rot(0u) {}
  __device__ StepWalk(int n_, uint32_t hash)
      : n(n_), A(n_ % 37 ? 37u : n_ % 41 ? 41u : n_ % 43 ? 43u : 1u), rot(n_ > 1 ? hash % (uint32_t)n_ : 0u) {}
  // step of position v (positions >= n are not permuted)
  __device__ int operator()(int v) const {
    if (v >= n) return v;
    if (n < (1 << 25)) return (int)(((uint32_t)v * A + rot) % (uint32_t)n);  // v A + rot < 2^32
    return (int)(((uint64_t)v * A + rot) % (uint32_t)n);
  }
};

typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) char lds_char;

// Asynchronous copies of 16 or 4 bytes per lane from global memory to LDS at
// dst + lane * size (dst is wave-uniform). They hold no registers while in
// flight and count in the vector-memory counter like any load. The builtin
// exists only for the device target; a host pass that sees it drops the
// kernels that use it. The 16-byte copies stream the KV cache and carry the
// nontemporal cache policy (bit 1 of the policy operand).
__device__ __forceinline__ void lds_dma16(const void *src, __attribute__((address_space(3))) void *dst) {
#if __HIP_DEVICE_COMPILE__
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 2);
#endif
}
__device__ __forceinline__ void lds_dma4(const void *src, __attribute__((address_space(3))) void *dst) {
#if __HIP_DEVICE_COMPILE__
  __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
#endif
}

}  // namespace sdk
