// qk_quantize.hip - activation quantization kernels (Q8_0 and Q8_K) for gfx950.
//
// Definition (codeloopback "Building Q8_0 and Q4_0 Like ggml", Example 2; candle
// formats page, BlockQ8_0::from_float and the "一些边界值" edge table):
//   amax = largest |x| of the block, NaN ignored;
//   d    = amax / 127 (correctly rounded f32 division);
//   id   = 1 / d, or 0 when d is 0;
//   code = roundf(x * id): halves away from zero, NaN -> 0, saturated to int8.
// Q8_0 keeps d as f16 (RNE, subnormals kept, overflow -> inf) before 32 codes.
// Q8_K (candle BlockQ8K) keeps d as f32, then 256 codes, then 16 int16 bsums,
// each the sum of 16 consecutive codes.  The pages give no scale rule of its own
// for Q8_K; the Q8_0 rule is applied over its 256 elements.
//
// Blocks of consecutive activation columns are contiguous, so ncols columns of n
// elements are quantized as one run of ncols * n / block blocks.
#include "qk_device.h"
#include "qk_internal.h"

namespace qk {
namespace {

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

// 8 lanes per 32-element block, 4 consecutive elements per lane.
__global__ __launch_bounds__(256) void quantize_q8_0_kernel(const float* __restrict__ x,
                                                            uint8_t* __restrict__ xq,
                                                            int64_t nblocks) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t b = t >> 3;
  const int part = threadIdx.x & 7;
  const bool valid = b < nblocks;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (valid) v = *reinterpret_cast<const float4*>(x + b * 32 + part * 4);
  const float amax = max8(abs_max4(v));  // the 8 lanes of this block
  const float d = amax / 127.0f;
  const float id = (d != 0.0f) ? 1.0f / d : 0.0f;
  if (!valid) return;
  const uint32_t packed =
      pack4(code_q8(v.x * id), code_q8(v.y * id), code_q8(v.z * id), code_q8(v.w * id));
  uint8_t* ob = xq + b * kQ8_0Bytes;
  store_u2(ob + 2 + part * 4, packed);
  if (part == 0) *reinterpret_cast<uint16_t*>(ob) = f32_to_f16_bits(d);
}

// One wavefront per 256-element block, 4 consecutive elements per lane.
__global__ __launch_bounds__(256) void quantize_q8_K_kernel(const float* __restrict__ x,
                                                            uint8_t* __restrict__ xq,
                                                            int64_t nblocks) {
  const int lane = threadIdx.x & 63;
  const int64_t b = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (b >= nblocks) return;  // whole wavefront leaves together
  const float4 v = *reinterpret_cast<const float4*>(x + b * 256 + lane * 4);
  const float amax = wave_max(abs_max4(v));
  const float d = amax / 127.0f;
  const float id = (d != 0.0f) ? 1.0f / d : 0.0f;
  const int c0 = code_q8(v.x * id), c1 = code_q8(v.y * id);
  const int c2 = code_q8(v.z * id), c3 = code_q8(v.w * id);
  uint8_t* ob = xq + b * kQ8_KBytes;
  *reinterpret_cast<uint32_t*>(ob + 4 + lane * 4) = pack4(c0, c1, c2, c3);
  const int s16 = quad_sum(c0 + c1 + c2 + c3);  // 16 codes = 4 lanes
  if ((lane & 3) == 0) {
    *reinterpret_cast<int16_t*>(ob + 260 + 2 * (lane >> 2)) = static_cast<int16_t>(s16);
  }
  if (lane == 0) *reinterpret_cast<float*>(ob) = d;
}

}  // namespace

hipError_t launch_quantize(int act_type, const float* x, uint8_t* xq, int64_t nblocks,
                           hipStream_t s) {
  if (nblocks <= 0) return hipSuccess;
  if (act_type == kQ8_0) {
    const int64_t threads = nblocks * 8;
    const unsigned grid = static_cast<unsigned>((threads + 255) / 256);
    quantize_q8_0_kernel<<<grid, 256, 0, s>>>(x, xq, nblocks);
  } else {
    const unsigned grid = static_cast<unsigned>((nblocks + 3) / 4);
    quantize_q8_K_kernel<<<grid, 256, 0, s>>>(x, xq, nblocks);
  }
  return hipGetLastError();
}

}  // namespace qk
