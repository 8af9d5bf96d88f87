// qk_device.h - device helpers shared by the gfx950 kernels of libqk.so.
//
// Block geometry of the GGUF formats (candle formats page, "块结构" field table):
//   Q8_0  34 B: d f16 @0, qs int8[32] @2
//   Q4_0  18 B: d f16 @0, qs u8[16] @2 (byte j: element j low nibble, j+16 high)
//   Q4_K 144 B: d f16 @0, dmin f16 @2, scales u8[12] @4, qs u8[128] @16
//   Q6_K 210 B: ql u8[128] @0, qh u8[64] @128, scales int8[16] @192, d f16 @208
//   Q8_K 292 B: d f32 @0, qs int8[256] @4, bsums int16[16] @260
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qk {

constexpr int kQ8_0Bytes = 34;
constexpr int kQ4_0Bytes = 18;
constexpr int kQ4_KBytes = 144;
constexpr int kQ6_KBytes = 210;
constexpr int kQ8_KBytes = 292;

// Four int8 x int8 products added into a 32-bit accumulator (v_dot4c_i32_i8).
__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int acc) {
  return __builtin_amdgcn_sdot4(static_cast<int>(a), static_cast<int>(b), acc, false);
}

// binary16 bits -> f32 (v_cvt_f32_f16, exact).
__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  _Float16 h;
  uint16_t b = static_cast<uint16_t>(bits16);
  __builtin_memcpy(&h, &b, 2);
  return static_cast<float>(h);
}

// f32 -> binary16 bits, round to nearest even, subnormals kept, overflow to inf
// (v_cvt_f16_f32 with the kernel's default rounding and f16 denormal modes).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 h = static_cast<_Float16>(f);
  uint16_t b;
  __builtin_memcpy(&b, &h, 2);
  return b;
}

// Loads of block fields that are only 2-byte aligned (34-, 18- and 210-byte
// blocks).  The compiler emits single dword/dwordx4 accesses for these: the HSA
// runtime runs the GPU with unaligned memory access enabled.
template <typename T>
__device__ __forceinline__ T load_u2(const uint8_t* p) {
  const uint16_t* p2 = reinterpret_cast<const uint16_t*>(__builtin_assume_aligned(p, 2));
  T v;
  __builtin_memcpy(&v, p2, sizeof(T));
  return v;
}

template <typename T>
__device__ __forceinline__ void store_u2(uint8_t* p, const T& v) {
  uint16_t* p2 = reinterpret_cast<uint16_t*>(__builtin_assume_aligned(p, 2));
  __builtin_memcpy(p2, &v, sizeof(T));
}

// Cross-lane sums inside groups of 4 lanes (DPP quad_perm, exact int32 adds).
__device__ __forceinline__ int quad_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
  return v;
}

// Sum over the 64 lanes of a wavefront (every lane receives the total).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

}  // namespace qk
