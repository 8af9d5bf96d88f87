// qk_quantize.hip - activation quantization kernels (Q8_0, Q8_1 and Q8_K) for gfx950.
//
// Definition (codeloopback "Building Q8_0 and Q4_0 Like ggml", Example 2; candle
// formats page, BlockQ8_0::from_float and the "一些边界值" edge table):
//   amax = largest |x| of the block, NaN ignored;
//   d    = amax / 127 (correctly rounded f32 division);
//   id   = 1 / d, or 0 when d is 0;
//   code = roundf(x * id): halves away from zero, NaN -> 0, saturated to int8.
// Q8_0 keeps d as f16 (RNE, subnormals kept, overflow -> inf) before 32 codes.
// Q8_1 (the activation block candle's VecDotType table pairs with Q4_1 and Q5_1;
// its layout is not printed, so this is a reading): f16 d, then f16 s = d * sum of
// the block's codes (the sum the weight minimum's term needs), then 32 codes.
// Q8_K (candle BlockQ8K) keeps d as f32, then 256 codes, then 16 int16 bsums,
// each the sum of 16 consecutive codes.  The pages give no scale rule of its own
// for Q8_K; the Q8_0 rule is applied over its 256 elements.
//
// Blocks of consecutive activation columns are contiguous, so ncols columns of n
// elements are quantized as one run of ncols * n / block blocks.
//
// The weight quantizers Q4_0, Q4_1 and Q5_0 (quantize_row_*_ref) follow below.
#include <float.h>
#include <hip/hip_ext.h>
#include <limits.h>

#include "qk_device.h"
#include "qk_internal.h"

namespace qk {
namespace {

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

// Q8_1: the Q8_0 block with s = f16(d * sum of the 32 codes) after d (d unrounded
// f32 in that product; a NaN product, from an infinite d, stored as 0x7E00), codes at
// byte 4.  8 lanes per block as Q8_0.
__global__ __launch_bounds__(256) void quantize_q8_1_kernel(const float* __restrict__ x,
                                                            uint8_t* __restrict__ xq,
                                                            int64_t nblocks) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t b = t >> 3;
  const int part = threadIdx.x & 7;
  const bool valid = b < nblocks;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (valid) v = *reinterpret_cast<const float4*>(x + b * 32 + part * 4);
  const float amax = max8(abs_max4(v));
  const float d = amax / 127.0f;
  const float id = (d != 0.0f) ? 1.0f / d : 0.0f;
  const int c0 = code_q8(v.x * id), c1 = code_q8(v.y * id);
  const int c2 = code_q8(v.z * id), c3 = code_q8(v.w * id);
  const int sum = sum8(c0 + c1 + c2 + c3);  // every lane of the block takes part
  if (!valid) return;
  uint8_t* ob = xq + b * kQ8_1Bytes;
  *reinterpret_cast<uint32_t*>(ob + 4 + part * 4) = pack4(c0, c1, c2, c3);
  if (part == 0) {
    // an infinite d (a block holding an infinity) has every code 0: the NaN product
    // is stored as the quiet NaN 0x7E00
    const float p = static_cast<float>(sum) * d;
    const uint32_t s_bits = (p != p) ? 0x7E00u : static_cast<uint32_t>(f32_to_f16_bits(p));
    *reinterpret_cast<uint32_t*>(ob) = static_cast<uint32_t>(f32_to_f16_bits(d)) | (s_bits << 16);
  }
}

// One wavefront per 256-element block, 4 consecutive elements per lane.
__global__ __launch_bounds__(256) void quantize_q8_K_kernel(const float* __restrict__ x,
                                                            uint8_t* __restrict__ xq,
                                                            int64_t nblocks) {
  const int lane = threadIdx.x & 63;
  const int64_t b = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (b >= nblocks) return;  // whole wavefront leaves together
  const float4 v = *reinterpret_cast<const float4*>(x + b * 256 + lane * 4);
  q8K_block(v, lane, xq + b * kQ8_KBytes);
}

// ---------------------------------------------------------------------------
// Weight quantizers Q4_0, Q4_1, Q5_0 (codeloopback Examples 5, 7, 8).  8 lanes per
// 32-element block.  The sequential reference scans elements in order and replaces
// its candidate only on a strictly better value, so every reduction below keeps
// (value, index) and prefers the lower index on ties (this decides signed zeros and
// equal magnitudes exactly as the scan).
//
// Lane p of a block holds elements e0(p) .. e0(p) + 3 with e0 = 4p for p < 4 and
// 44 - 4p for p >= 4 (lanes 4..7 hold 28, 24, 20, 16): byte k of the packed nibbles
// pairs element k with element k + 16, and with this order the lane holding the
// upper half of lane p's bytes is lane 7 - p, which the DPP half-row mirror reaches.
// All exchanges are DPP moves inside the 8 lanes (quad swaps, then the mirror).
// Each group of 8 lanes quantizes kRowUnroll blocks, the loads of all of them
// issued first; the blocks of one load instruction are consecutive.
constexpr int kRowUnroll = 4;  // 4 measured best (8: slower)

__device__ __forceinline__ int lane_e0(int part) { return part < 4 ? 4 * part : 44 - 4 * part; }

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

struct Pick {
  float key;  // compared value (|x| for the signed max, x for min / max)
  float val;  // value kept (x)
  int idx;    // element index
};

// better(a, b): a beats b under comparison C (a strict improvement, or equal with
// a lower index).
template <bool kMax>
__device__ __forceinline__ bool better(const Pick& a, const Pick& b) {
  const bool strictly = kMax ? (a.key > b.key) : (a.key < b.key);
  return strictly || (a.key == b.key && a.idx < b.idx);
}

template <bool kMax, int CTRL>
__device__ __forceinline__ Pick pick_step(Pick p) {
  Pick o;
  o.key = __int_as_float(dpp_i<CTRL>(__float_as_int(p.key)));
  o.val = __int_as_float(dpp_i<CTRL>(__float_as_int(p.val)));
  o.idx = dpp_i<CTRL>(p.idx);
  return better<kMax>(o, p) ? o : p;
}

// Best of the 8 lanes of a block, in every lane: quad swaps [1,0,3,2] and
// [2,3,0,1], then the half-row mirror joins the two quads.
template <bool kMax>
__device__ __forceinline__ Pick reduce8(Pick p) {
  p = pick_step<kMax, 0xB1>(p);
  p = pick_step<kMax, 0x4E>(p);
  return pick_step<kMax, 0x141>(p);
}

__device__ __forceinline__ uint32_t or8(uint32_t v) {
  v |= static_cast<uint32_t>(dpp_i<0xB1>(static_cast<int>(v)));
  v |= static_cast<uint32_t>(dpp_i<0x4E>(static_cast<int>(v)));
  return v | static_cast<uint32_t>(dpp_i<0x141>(static_cast<int>(v)));
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
__device__ __forceinline__ void quantize_block(float4 v4, int part, bool valid, uint8_t* ob) {
#pragma clang fp contract(off)
  const float v[4] = {v4.x, v4.y, v4.z, v4.w};
  const int e0 = lane_e0(part);
  float d, id, mn = 0.0f;
  if constexpr (FMT == kFmtQ4_1) {
    // min and max, each the first occurrence of its value (strict < / >)
    Pick lo{v[0], v[0], e0}, hi{v[0], v[0], e0};
#pragma unroll
    for (int i = 1; i < 4; ++i) {
      if (v[i] < lo.key) lo = Pick{v[i], v[i], e0 + i};
      if (v[i] > hi.key) hi = Pick{v[i], v[i], e0 + i};
    }
    lo = reduce8<false>(lo);
    hi = reduce8<true>(hi);
    mn = lo.val;
    d = (hi.val - mn) / 15.0f;
  } else {
    // the first element of largest magnitude, with its sign (from 0: an all-zero
    // block keeps max = 0)
    Pick m{0.0f, 0.0f, 32};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (m.key < fabsf(v[i])) m = Pick{fabsf(v[i]), v[i], e0 + i};
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
  const uint32_t upper = static_cast<uint32_t>(dpp_i<0x141>(static_cast<int>(nib)));  // lane 7 - p
  uint32_t qh = 0;
  if constexpr (FMT == kFmtQ5_0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) qh |= ((static_cast<uint32_t>(c[i]) >> 4) & 1u) << (e0 + i);
    qh = or8(qh);
  }
  if (!valid) return;
  constexpr int kQs = (FMT == kFmtQ4_0) ? 2 : (FMT == kFmtQ4_1) ? 4 : 6;
  if (part < 4) store_u2(ob + kQs + 4 * part, nib | (upper << 4));
  if (part == 0) {
    store_u2(ob, f32_to_f16_bits(d));
    if constexpr (FMT == kFmtQ4_1) store_u2(ob + 2, f32_to_f16_bits(mn));
    if constexpr (FMT == kFmtQ5_0) store_u2(ob + 2, qh);
  }
}

template <int FMT>
__global__ __launch_bounds__(256) void quantize_row_kernel(const float* __restrict__ x,
                                                           uint8_t* __restrict__ dst,
                                                           int64_t nblocks) {
  constexpr int kBytes = (FMT == kFmtQ4_0) ? kQ4_0Bytes : (FMT == kFmtQ4_1) ? kQ4_1Bytes : kQ5_0Bytes;
  const int lane = threadIdx.x & 63;
  const int part = lane & 7, grp = lane >> 3;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) >> 6;
  const int64_t base = wave * (8 * kRowUnroll) + grp;  // block of unroll step 0
  float4 v[kRowUnroll];
#pragma unroll
  for (int u = 0; u < kRowUnroll; ++u) {
    const int64_t b = base + 8 * u;
    v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (b < nblocks) v[u] = *reinterpret_cast<const float4*>(x + b * 32 + lane_e0(part));
  }
#pragma unroll
  for (int u = 0; u < kRowUnroll; ++u) {
    const int64_t b = base + 8 * u;
    // every lane takes part in the exchanges; only whole blocks in range store
    quantize_block<FMT>(v[u], part, b < nblocks, dst + b * kBytes);
  }
}

}  // namespace

hipError_t launch_quantize_row(int type, const float* x, uint8_t* dst, int64_t nblocks,
                               hipStream_t s) {
  if (nblocks <= 0) return hipSuccess;
  // Q8_0: 8 lanes per block; the others: 4 wavefronts per workgroup, 8 * kRowUnroll
  // blocks per wavefront
  unsigned grid = 0;
  if (!launch_grid(type == kQ8_0 ? (nblocks * 8 + 255) / 256 : (nblocks + 32 * kRowUnroll - 1) / (32 * kRowUnroll),
                   256, &grid))
    return hipErrorInvalidConfiguration;
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
                           hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (nblocks <= 0) return hipSuccess;
  // Q8_0, Q8_1: 8 lanes per block; Q8_K: one wavefront per block
  const bool q8K = act_type == kQ8_K;
  unsigned grid = 0;
  if (!launch_grid(q8K ? (nblocks + 3) / 4 : (nblocks * 8 + 255) / 256, 256, &grid))
    return hipErrorInvalidConfiguration;
  auto* kernel = q8K ? quantize_q8_K_kernel : act_type == kQ8_1 ? quantize_q8_1_kernel : quantize_q8_0_kernel;
  if (e0 != nullptr || e1 != nullptr) {
    hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(256), 0, s, e0, e1, 0, x, xq, nblocks);
  } else {
    kernel<<<grid, 256, 0, s>>>(x, xq, nblocks);
  }
  return hipGetLastError();
}

}  // namespace qk
