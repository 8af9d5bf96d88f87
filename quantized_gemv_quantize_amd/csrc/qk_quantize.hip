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
//
// The weight quantizers Q4_0, Q4_1 and Q5_0 (quantize_row_*_ref) follow below.
#include <float.h>
#include <limits.h>

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

// ---------------------------------------------------------------------------
// Weight quantizers Q4_0, Q4_1, Q5_0 (codeloopback Examples 5, 7, 8).  8 lanes per
// 32-element block, lane p holding elements 4p .. 4p+3.  The sequential reference
// scans elements in order and replaces its candidate only on a strictly better
// value, so every reduction below keeps (value, index) and prefers the lower index
// on ties (this decides signed zeros and equal magnitudes exactly as the scan).

// The 8 lanes of a block exchange through ds_bpermute (width 8).
template <typename T>
__device__ __forceinline__ T xor8(T v, int m) {
  return __shfl_xor(v, m, 8);
}

struct Pick {
  float key;  // compared value (|x| for the signed max, x for min / max)
  float val;  // value kept (x)
  int idx;    // element index, 32 when the lane has no candidate
};

// better(a, b): a beats b under comparison C (a strict improvement, or equal with
// a lower index).
template <bool kMax>
__device__ __forceinline__ bool better(const Pick& a, const Pick& b) {
  const bool strictly = kMax ? (a.key > b.key) : (a.key < b.key);
  return strictly || (a.key == b.key && a.idx < b.idx);
}

template <bool kMax>
__device__ __forceinline__ Pick reduce8(Pick p) {
#pragma unroll
  for (int m = 1; m < 8; m <<= 1) {
    Pick o;
    o.key = xor8(p.key, m);
    o.val = xor8(p.val, m);
    o.idx = xor8(p.idx, m);
    if (better<kMax>(o, p)) p = o;
  }
  return p;
}

constexpr int kFmtQ4_0 = 0, kFmtQ4_1 = 1, kFmtQ5_0 = 2;

// Float to int the way the codes' definition converts: truncation toward zero,
// saturating at the int32 limits, NaN -> 0.  Inside 0..31.5 it is a plain
// truncation; infinities only arise when 1/d overflows (a scale below 2^-128).
__device__ __forceinline__ int trunc_sat(float f) {
  if (f != f) return 0;
  if (f >= 2147483648.0f) return INT_MAX;
  if (f <= -2147483648.0f) return INT_MIN;
  return static_cast<int>(f);
}

template <int FMT>
__global__ __launch_bounds__(256) void quantize_row_kernel(const float* __restrict__ x,
                                                           uint8_t* __restrict__ dst,
                                                           int64_t nblocks) {
#pragma clang fp contract(off)
  constexpr int kBytes = (FMT == kFmtQ4_0) ? kQ4_0Bytes : (FMT == kFmtQ4_1) ? kQ4_1Bytes : kQ5_0Bytes;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t b = t >> 3;  // the 8 lanes of a block are all in or all out of range
  const int part = threadIdx.x & 7;
  const bool valid = b < nblocks;
  float4 v4 = make_float4(0.f, 0.f, 0.f, 0.f);
  if (valid) v4 = *reinterpret_cast<const float4*>(x + b * 32 + part * 4);
  const float v[4] = {v4.x, v4.y, v4.z, v4.w};

  float d, id, mn = 0.0f;
  if constexpr (FMT == kFmtQ4_1) {
    // min and max, each the first occurrence of its value (reference: strict < / >)
    Pick lo{FLT_MAX, FLT_MAX, 32}, hi{-FLT_MAX, -FLT_MAX, 32};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (v[i] < lo.key) lo = Pick{v[i], v[i], 4 * part + i};
      if (v[i] > hi.key) hi = Pick{v[i], v[i], 4 * part + i};
    }
    lo = reduce8<false>(lo);
    hi = reduce8<true>(hi);
    mn = lo.val;
    d = (hi.val - mn) / 15.0f;
  } else {
    // the first element of largest magnitude, with its sign
    Pick m{0.0f, 0.0f, 32};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (m.key < fabsf(v[i])) m = Pick{fabsf(v[i]), v[i], 4 * part + i};
    }
    m = reduce8<true>(m);
    d = m.val / ((FMT == kFmtQ4_0) ? -8.0f : -16.0f);
  }
  id = (d != 0.0f) ? 1.0f / d : 0.0f;

  int c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float f;
    if constexpr (FMT == kFmtQ4_0) f = v[i] * id + 8.5f;
    else if constexpr (FMT == kFmtQ4_1) f = (v[i] - mn) * id + 0.5f;
    else f = v[i] * id + 16.5f;
    c[i] = min(trunc_sat(f), (FMT == kFmtQ5_0) ? 31 : 15);
  }
  const uint32_t nib = (c[0] & 15) | ((c[1] & 15) << 8) | ((c[2] & 15) << 16) |
                       (static_cast<uint32_t>(c[3] & 15) << 24);
  const uint32_t upper = xor8(nib, 4);  // elements 16 + 4p .. (lanes p < 4)
  uint32_t qh = 0;
  if constexpr (FMT == kFmtQ5_0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) qh |= ((static_cast<uint32_t>(c[i]) >> 4) & 1u) << (4 * part + i);
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) qh |= xor8(qh, m);
  }
  if (!valid) return;
  uint8_t* ob = dst + b * kBytes;
  constexpr int kQs = (FMT == kFmtQ4_0) ? 2 : (FMT == kFmtQ4_1) ? 4 : 6;
  if (part < 4) store_u2(ob + kQs + 4 * part, nib | (upper << 4));
  if (part == 0) {
    store_u2(ob, f32_to_f16_bits(d));
    if constexpr (FMT == kFmtQ4_1) store_u2(ob + 2, f32_to_f16_bits(mn));
    if constexpr (FMT == kFmtQ5_0) store_u2(ob + 2, qh);
  }
}

}  // namespace

hipError_t launch_quantize_row(int type, const float* x, uint8_t* dst, int64_t nblocks,
                               hipStream_t s) {
  if (nblocks <= 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>((nblocks * 8 + 255) / 256);
  switch (type) {
    case kQ8_0: quantize_q8_0_kernel<<<grid, 256, 0, s>>>(x, dst, nblocks); break;
    case kQ4_0: quantize_row_kernel<kFmtQ4_0><<<grid, 256, 0, s>>>(x, dst, nblocks); break;
    case kQ4_1: quantize_row_kernel<kFmtQ4_1><<<grid, 256, 0, s>>>(x, dst, nblocks); break;
    case kQ5_0: quantize_row_kernel<kFmtQ5_0><<<grid, 256, 0, s>>>(x, dst, nblocks); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

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
