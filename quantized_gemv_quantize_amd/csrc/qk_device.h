// qk_device.h - device helpers shared by the gfx950 kernels of libqk.so.
//
// Block geometry of the GGUF formats (candle formats page, "块结构" field table):
//   Q8_0  34 B: d f16 @0, qs int8[32] @2
//   Q4_0  18 B: d f16 @0, qs u8[16] @2 (byte j: element j low nibble, j+16 high)
//   Q4_1  20 B: d f16 @0, m f16 @2, qs u8[16] @4 (nibbles as Q4_0)
//   Q5_0  22 B: d f16 @0, qh u32 @2 (bit e: bit 4 of element e), qs u8[16] @6
//   Q5_1  24 B: d f16 @0, m f16 @2, qh u32 @4, qs u8[16] @8 (GGUF order)
//   Q4_K 144 B: d f16 @0, dmin f16 @2, scales u8[12] @4, qs u8[128] @16
//   Q5_K 176 B: d f16 @0, dmin f16 @2, scales u8[12] @4 (as Q4_K), qh u8[32] @16,
//               qs u8[128] @48 (the pages give the size and field roles; the
//               order and bit arrangement are GGUF's)
//   Q6_K 210 B: ql u8[128] @0, qh u8[64] @128, scales int8[16] @192, d f16 @208
//   Q8_K 292 B: d f32 @0, qs int8[256] @4, bsums int16[16] @260
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qk {

constexpr int kQ8_0Bytes = 34;
constexpr int kQ4_0Bytes = 18;
constexpr int kQ4_1Bytes = 20;
constexpr int kQ5_0Bytes = 22;
constexpr int kQ5_1Bytes = 24;
constexpr int kQ8_1Bytes = 36;
constexpr int kQ2_KBytes = 84;
constexpr int kQ3_KBytes = 110;
constexpr int kQ4_KBytes = 144;
constexpr int kQ5_KBytes = 176;
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
// (v_cvt_f16_f32 with the kernel's default rounding and f16 denormal modes).  The
// argument is an f32 value already rounded: the empty asm hides how it was computed,
// because the backend otherwise merges a product feeding this conversion into one
// mixed-precision multiply (v_fma_mix) rounded once to f16, a different value near
// f16 ties.
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  asm volatile("" : "+v"(f));
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

// Index of the wavefront inside its workgroup, as a wave-uniform (scalar) value so
// that row base addresses live in SGPRs and loads take a 32-bit lane offset.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
}

// Cross-lane sums inside groups of 4 lanes (DPP quad_perm, exact int32 adds).
__device__ __forceinline__ int quad_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
  return v;
}

// a * b + c for |a|, |b| < 2^23 (v_mad_i32_i24, full rate).
__device__ __forceinline__ int mad24(int a, int b, int c) { return __mul24(a, b) + c; }

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes of a wavefront, returned in every lane: DPP sums inside
// each row of 16 lanes (quad swaps, half-row and row mirrors), then the four row
// totals are read from lanes 15, 31, 47 and 63.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror: sum of 8
  v += dpp_f<0x140>(v);  // row_mirror: sum of 16 in every lane of the row
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 15)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 47)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Sum over groups of 8 lanes (returned in every lane of the group, exact int32).
__device__ __forceinline__ int sum8(int v) {
  v = quad_sum(v);
  return v + __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
}

// Largest value over groups of 8 lanes (returned in every lane of the group).
__device__ __forceinline__ float max8(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2,3,0,1]
  return fmaxf(v, dpp_f<0x141>(v));  // row_half_mirror
}

// Largest value over the 64 lanes of a wavefront, returned in every lane.
__device__ __forceinline__ float wave_max(float v) {
  v = max8(v);
  v = fmaxf(v, dpp_f<0x140>(v));  // row_mirror: max of 16
  return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 15)),
                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31))),
               fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 47)),
                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63))));
}

// ---------------------------------------------------------------------------
// Activation quantization (codeloopback Example 2's rule; candle BlockQ8K layout),
// shared by the quantize kernels and the GEMV that quantizes its own x.

// roundf, halves away from zero; NaN -> 0; saturated to int8.
__device__ __forceinline__ int code_q8(float v) {
  if (v != v) return 0;
  float r = roundf(v);
  r = fminf(fmaxf(r, -128.0f), 127.0f);
  return static_cast<int>(r);
}

__device__ __forceinline__ uint32_t pack4(int c0, int c1, int c2, int c3) {
  return (static_cast<uint32_t>(c0) & 0xFFu) | ((static_cast<uint32_t>(c1) & 0xFFu) << 8) |
         ((static_cast<uint32_t>(c2) & 0xFFu) << 16) | ((static_cast<uint32_t>(c3) & 0xFFu) << 24);
}

// Largest |x| of 4 values folded from 0, so NaN never wins (fmaxf returns the
// other operand) and an all-NaN block gives 0, as the sequential definition does.
__device__ __forceinline__ float abs_max4(float4 v) {
  return fmaxf(fmaxf(fmaxf(fmaxf(0.0f, fabsf(v.x)), fabsf(v.y)), fabsf(v.z)), fabsf(v.w));
}

// One Q8_K block by one wavefront, lane l holding elements 4l .. 4l+3 in v: d = amax
// / 127 (f32), codes roundf(x / d) via id = 1 / d (0 when d is 0), the 16 int16 code
// sums, written at ob (global memory or LDS: d @0, codes @4, bsums @260).
__device__ __forceinline__ void q8K_block(float4 v, int lane, uint8_t* ob) {
  const float amax = wave_max(abs_max4(v));
  const float d = amax / 127.0f;
  const float id = (d != 0.0f) ? 1.0f / d : 0.0f;
  const int c0 = code_q8(v.x * id), c1 = code_q8(v.y * id);
  const int c2 = code_q8(v.z * id), c3 = code_q8(v.w * id);
  *reinterpret_cast<uint32_t*>(ob + 4 + lane * 4) = pack4(c0, c1, c2, c3);
  const int s16 = quad_sum(c0 + c1 + c2 + c3);  // 16 codes = 4 lanes
  if ((lane & 3) == 0) {
    *reinterpret_cast<int16_t*>(ob + 260 + 2 * (lane >> 2)) = static_cast<int16_t>(s16);
  }
  if (lane == 0) *reinterpret_cast<float*>(ob) = d;
}

}  // namespace qk
