// qk_dequant.hip - DequantizeRow kernels (block -> f32) for gfx950.
//
// Values (rml "Dequantization"; candle formats page, block table; codeloopback
// Example 6 for Q4_0's nibble order):
//   Q8_0  d * q
//   Q4_0  d * (q - 8); byte j: element j in the low nibble, element j+16 in the high
//   Q4_1  q * d + m, nibbles as Q4_0 (codeloopback Example 7)
//   Q5_0  d * (q - 16), low nibbles as Q4_0, bit 4 from qh (codeloopback Example 8)
//   Q5_1  q * d + m, q as Q5_0's code (the _1 block adds an f16 min to the _0 one)
//   Q4_K  d * sc_j * q - dmin * m_j for 32-element sub-block j (scales per
//         get_scale_min_k4, rml element-200 trace)
//   Q5_K  the same with a 5-bit q: element 64c + p takes bit 2c + (p >= 32) of
//         qh[p % 32] as bit 4 (GGUF arrangement; the pages give the field roles)
//   Q6_K  d * sc_j * (q - 32) for 16-element sub-block j; q = 4 bits from ql and
//         2 bits from qh in the GGUF arrangement (the pages give only the roles)
//   Q2_K  d * sc_j * q - dmin * m_j, Q3_K d * (sc_j - 32) * (q - 4), 16-element j
//         (GGUF arrangement; the pages give only the sizes)
// Each product is exact in f32 (at most 23 significant bits), so the order of
// multiplication and any FMA contraction leave the result unchanged.
//
// Each lane produces 4 consecutive floats and stores them as one float4, so a
// wavefront writes contiguous spans (the f32 output is 4-7x the bytes read).
#include "qk_device.h"
#include "qk_internal.h"

namespace qk {
namespace {

constexpr uint32_t kLo4 = 0x0F0F0F0Fu;

// The f32 output is written once and not read back by this kernel: non-temporal
// stores (32000 x 4096 Q6_K: 121.9 against 127.7 us with ordinary stores).
typedef float f4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_f4(float* p, float4 o) {
  __builtin_nontemporal_store(f4v{o.x, o.y, o.z, o.w}, reinterpret_cast<f4v*>(p));
}

__device__ __forceinline__ float4 scale_bytes_signed(uint32_t q, float scale, int offset) {
  return make_float4(scale * static_cast<float>(static_cast<int>(q & 0xFF) - offset),
                     scale * static_cast<float>(static_cast<int>((q >> 8) & 0xFF) - offset),
                     scale * static_cast<float>(static_cast<int>((q >> 16) & 0xFF) - offset),
                     scale * static_cast<float>(static_cast<int>(q >> 24) - offset));
}

// Q8_0: 8 lanes per block.
__global__ __launch_bounds__(256) void dequant_q8_0_kernel(const uint8_t* __restrict__ src,
                                                           float* __restrict__ dst,
                                                           int64_t nblocks) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t b = t >> 3;
  if (b >= nblocks) return;
  const int part = threadIdx.x & 7;
  const uint8_t* blk = src + b * kQ8_0Bytes;
  const float d = f16_to_f32(*reinterpret_cast<const uint16_t*>(blk));
  const uint32_t q = load_u2<uint32_t>(blk + 2 + 4 * part);
  float4 o;
  o.x = d * static_cast<float>(static_cast<int8_t>(q & 0xFF));
  o.y = d * static_cast<float>(static_cast<int8_t>((q >> 8) & 0xFF));
  o.z = d * static_cast<float>(static_cast<int8_t>((q >> 16) & 0xFF));
  o.w = d * static_cast<float>(static_cast<int8_t>(q >> 24));
  store_f4(dst + b * 32 + 4 * part, o);
}

// Q4_0: 8 lanes per block; lanes 0-3 take low nibbles (elements 0-15), lanes 4-7
// the high nibbles (elements 16-31) of the same 16 bytes.
__global__ __launch_bounds__(256) void dequant_q4_0_kernel(const uint8_t* __restrict__ src,
                                                           float* __restrict__ dst,
                                                           int64_t nblocks) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t b = t >> 3;
  if (b >= nblocks) return;
  const int part = threadIdx.x & 7;
  const uint8_t* blk = src + b * kQ4_0Bytes;
  const float d = f16_to_f32(*reinterpret_cast<const uint16_t*>(blk));
  const uint32_t w = load_u2<uint32_t>(blk + 2 + 4 * (part & 3));
  const uint32_t q = (part < 4) ? (w & kLo4) : ((w >> 4) & kLo4);
  store_f4(dst + b * 32 + 4 * part, scale_bytes_signed(q, d, 8));
}

// Q4_1: as Q4_0 with the codes unsigned and a min added: value = q * d + m (the
// product is exact, so fused or not the one rounding is the addition).
__global__ __launch_bounds__(256) void dequant_q4_1_kernel(const uint8_t* __restrict__ src,
                                                           float* __restrict__ dst,
                                                           int64_t nblocks) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t b = t >> 3;
  if (b >= nblocks) return;
  const int part = threadIdx.x & 7;
  const uint8_t* blk = src + b * kQ4_1Bytes;
  const uint32_t dm = *reinterpret_cast<const uint32_t*>(blk);  // 4-byte aligned: d, m
  const float d = f16_to_f32(dm & 0xFFFF), m = f16_to_f32(dm >> 16);
  const uint32_t w = *reinterpret_cast<const uint32_t*>(blk + 4 + 4 * (part & 3));
  const uint32_t q = (part < 4) ? (w & kLo4) : ((w >> 4) & kLo4);
  float4 o;
  o.x = static_cast<float>(q & 0xFF) * d + m;
  o.y = static_cast<float>((q >> 8) & 0xFF) * d + m;
  o.z = static_cast<float>((q >> 16) & 0xFF) * d + m;
  o.w = static_cast<float>(q >> 24) * d + m;
  store_f4(dst + b * 32 + 4 * part, o);
}

// Q5_0: the Q4_0 nibbles plus bit e of qh as bit 4 of element e; value d * (q - 16).
// Lane part holds elements 4 part .. 4 part + 3 (nibbles of bytes 4 (part & 3) ..,
// low for part < 4, high otherwise), whose fifth bits are qh bits 4 part .. + 3.
__global__ __launch_bounds__(256) void dequant_q5_0_kernel(const uint8_t* __restrict__ src,
                                                           float* __restrict__ dst,
                                                           int64_t nblocks) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t b = t >> 3;
  if (b >= nblocks) return;
  const int part = threadIdx.x & 7;
  const uint8_t* blk = src + b * kQ5_0Bytes;
  const float d = f16_to_f32(*reinterpret_cast<const uint16_t*>(blk));
  const uint32_t qh = load_u2<uint32_t>(blk + 2);
  const uint32_t w = load_u2<uint32_t>(blk + 6 + 4 * (part & 3));
  const uint32_t lo = (part < 4) ? (w & kLo4) : ((w >> 4) & kLo4);
  // four bits -> bit 4 of four bytes: multiplying by 0x204081 copies bit i to bit 8i
  const uint32_t fifth = ((((qh >> (4 * part)) & 0xF) * 0x00204081u) & 0x01010101u) << 4;
  store_f4(dst + b * 32 + 4 * part, scale_bytes_signed(lo | fifth, d, 16));
}

// Q5_1: Q5_0's codes (unsigned) with Q4_1's value q * d + m; d, m, qh in the first 8
// bytes (4-byte aligned: 24-byte blocks from a 16-byte aligned base).
__global__ __launch_bounds__(256) void dequant_q5_1_kernel(const uint8_t* __restrict__ src,
                                                           float* __restrict__ dst,
                                                           int64_t nblocks) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t b = t >> 3;
  if (b >= nblocks) return;
  const int part = threadIdx.x & 7;
  const uint8_t* blk = src + b * kQ5_1Bytes;
  const uint2 dmq = *reinterpret_cast<const uint2*>(blk);  // d, m, qh
  const float d = f16_to_f32(dmq.x & 0xFFFF), m = f16_to_f32(dmq.x >> 16);
  const uint32_t w = *reinterpret_cast<const uint32_t*>(blk + 8 + 4 * (part & 3));
  const uint32_t lo = (part < 4) ? (w & kLo4) : ((w >> 4) & kLo4);
  const uint32_t q = lo | (((((dmq.y >> (4 * part)) & 0xF) * 0x00204081u) & 0x01010101u) << 4);
  float4 o;
  o.x = static_cast<float>(q & 0xFF) * d + m;
  o.y = static_cast<float>((q >> 8) & 0xFF) * d + m;
  o.z = static_cast<float>((q >> 16) & 0xFF) * d + m;
  o.w = static_cast<float>(q >> 24) * d + m;
  store_f4(dst + b * 32 + 4 * part, o);
}

// Q4_K, Q5_K and Q6_K: one wavefront per kSB consecutive superblocks, lane l -> elements
// 4l..4l+3 of each; every load of the kSB superblocks is issued before the first
// store, and fewer, longer wavefronts keep the dispatcher out of the way.
constexpr int kSB = 4;

struct Q4KPart {
  uint4 h;      // d, dmin, scales[12]
  uint32_t w;   // the 4 qs bytes holding this lane's 4 nibbles
  uint32_t qh;  // Q5_K: the 4 qh bytes holding this lane's fifth bits
};

// Q5 selects Q5_K (176-byte superblocks: qh[32] at byte 16, qs at byte 48).
template <int Q5>
__global__ __launch_bounds__(256) void dequant_q4_K_kernel(const uint8_t* __restrict__ src,
                                                           float* __restrict__ dst,
                                                           int64_t nblocks) {
  const int lane = threadIdx.x & 63;
  const int64_t b0 = (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * kSB;
  if (b0 >= nblocks) return;
  const int e0 = 4 * lane;
  const int j = e0 >> 5;   // sub-block
  const int c = e0 >> 6;   // 64-element chunk
  const int p = e0 & 63;   // position in the chunk
  constexpr int kBytes = Q5 ? kQ5_KBytes : kQ4_KBytes, kQs = Q5 ? 48 : 16;
  Q4KPart v[kSB];
#pragma unroll
  for (int k = 0; k < kSB; ++k) {
    const uint8_t* blk = src + min(b0 + k, nblocks - 1) * kBytes;
    v[k].h = *reinterpret_cast<const uint4*>(blk);
    v[k].w = *reinterpret_cast<const uint32_t*>(blk + kQs + 32 * c + (p & 31));
    v[k].qh = Q5 ? *reinterpret_cast<const uint32_t*>(blk + 16 + (p & 31)) : 0u;
  }
#pragma unroll
  for (int k = 0; k < kSB; ++k) {
    if (b0 + k >= nblocks) break;  // uniform over the wavefront
    const uint4 h = v[k].h;
    const float d = f16_to_f32(h.x & 0xFFFF);
    const float dmin = f16_to_f32(h.x >> 16);
    // get_scale_min_k4: sub-blocks 0-3 use the low 6 bits of bytes j and j+4; 4-7
    // take the low / high nibble of byte j+4 and the top 2 bits of bytes j-4 / j.
    const uint32_t s0 = h.y, s1 = h.z, s2 = h.w;
    const uint32_t scw = (j < 4) ? (s0 & 0x3F3F3F3Fu) : ((s2 & kLo4) | ((s0 >> 2) & 0x30303030u));
    const uint32_t mw = (j < 4) ? (s1 & 0x3F3F3F3Fu) : (((s2 >> 4) & kLo4) | ((s1 >> 2) & 0x30303030u));
    const int sh = 8 * (j & 3);
    const float sc = static_cast<float>((scw >> sh) & 0xFF);
    const float mn = static_cast<float>((mw >> sh) & 0xFF);
    uint32_t q = (p < 32) ? (v[k].w & kLo4) : ((v[k].w >> 4) & kLo4);
    if constexpr (Q5 != 0) q |= ((v[k].qh >> (2 * c + (p >= 32 ? 1 : 0))) & 0x01010101u) << 4;
    const float dsc = d * sc;
    const float dm = dmin * mn;
    float4 o;
    o.x = dsc * static_cast<float>(q & 0xFF) - dm;
    o.y = dsc * static_cast<float>((q >> 8) & 0xFF) - dm;
    o.z = dsc * static_cast<float>((q >> 16) & 0xFF) - dm;
    o.w = dsc * static_cast<float>(q >> 24) - dm;
    store_f4(dst + (b0 + k) * 256 + e0, o);
  }
}

// Q6_K: element e: half h = e/128, r = e%128, group g = r/32, l = r%32; low 4 bits
// are nibble (g < 2 ? low : high) of ql[64h + l + 32(g&1)], high 2 bits are
// (qh[32h + l] >> 2g) & 3.
struct Q6KPart {
  uint32_t wl, wh;  // ql and qh bytes of this lane's 4 elements
  uint32_t dw;      // the f16 d (bytes 208-209)
  int sc;           // the int8 scale of this lane's 16-element sub-block
};

__global__ __launch_bounds__(256) void dequant_q6_K_kernel(const uint8_t* __restrict__ src,
                                                           float* __restrict__ dst,
                                                           int64_t nblocks) {
  const int lane = threadIdx.x & 63;
  const int64_t b0 = (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * kSB;
  if (b0 >= nblocks) return;
  const int e0 = 4 * lane;
  const int h = e0 >> 7, r = e0 & 127, g = r >> 5, l = r & 31;
  Q6KPart v[kSB];
#pragma unroll
  for (int k = 0; k < kSB; ++k) {
    const uint8_t* blk = src + min(b0 + k, nblocks - 1) * kQ6_KBytes;
    v[k].wl = load_u2<uint32_t>(blk + 64 * h + l + 32 * (g & 1));
    v[k].wh = load_u2<uint32_t>(blk + 128 + 32 * h + l);
    v[k].dw = *reinterpret_cast<const uint16_t*>(blk + 208);
    v[k].sc = static_cast<int8_t>(blk[192 + (e0 >> 4)]);
  }
#pragma unroll
  for (int k = 0; k < kSB; ++k) {
    if (b0 + k >= nblocks) break;  // uniform over the wavefront
    const uint32_t lo = (g < 2) ? (v[k].wl & kLo4) : ((v[k].wl >> 4) & kLo4);
    const uint32_t q = lo | (((v[k].wh >> (2 * g)) & 0x03030303u) << 4);
    const float d = f16_to_f32(v[k].dw);
    store_f4(dst + (b0 + k) * 256 + e0, scale_bytes_signed(q, d * static_cast<float>(v[k].sc), 32));
  }
}

// Q2_K and Q3_K (GGUF arrangement; the pages give their sizes only): lane takes 4
// consecutive elements e0 .. e0 + 3 of one 16-element sub-block j = e0 / 16, half
// h = e0 / 128, group g = (e0 % 128) / 32, l = e0 % 32: 2 code bits at bits 2g of
// qs[32h + l .. +3].  Q2_K (84 B): d * (scales[j] & 15) * q - dmin * (scales[j] >> 4),
// d, dmin at bytes 80, 82.  Q3_K (110 B, 2-byte aligned): bit 2 of the code from
// bit 4h + g of hmask[l], value d * (scale_j - 32) * (code - 4), scale_j's low 4 bits
// from byte j (j < 8) or the high nibble of byte j - 8, its high 2 bits from bits
// 2(j/4) of byte 8 + j % 4 of scales[12] at 96; d at byte 108.
struct Q23Part {
  uint32_t q, m;  // code bytes (qs) and, for Q3_K, hmask bytes of this lane's 4 elements
  uint32_t d;     // Q2_K: d | dmin << 16; Q3_K: d
  uint32_t sc;    // Q2_K: scales[j]; Q3_K: the unsigned 6-bit scale of sub-block j
};

template <int Q3>
__global__ __launch_bounds__(256) void dequant_q23_K_kernel(const uint8_t* __restrict__ src,
                                                            float* __restrict__ dst,
                                                            int64_t nblocks) {
  const int lane = threadIdx.x & 63;
  const int64_t b0 = (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * kSB;
  if (b0 >= nblocks) return;
  const int e0 = 4 * lane;
  const int j = e0 >> 4, h = e0 >> 7, g = (e0 & 127) >> 5, l = e0 & 31;
  constexpr int kBytes = Q3 ? kQ3_KBytes : kQ2_KBytes;
  Q23Part v[kSB];
#pragma unroll
  for (int k = 0; k < kSB; ++k) {
    const uint8_t* blk = src + min(b0 + k, nblocks - 1) * kBytes;
    if constexpr (Q3 != 0) {
      v[k].q = load_u2<uint32_t>(blk + 32 + 32 * h + l);
      v[k].m = load_u2<uint32_t>(blk + l);
      v[k].d = *reinterpret_cast<const uint16_t*>(blk + 108);
      const int low4 = (j < 8) ? (blk[96 + j] & 15) : (blk[96 + j - 8] >> 4);
      v[k].sc = static_cast<uint32_t>(low4 | (((blk[104 + (j & 3)] >> (2 * (j >> 2))) & 3) << 4));
    } else {
      v[k].q = *reinterpret_cast<const uint32_t*>(blk + 16 + 32 * h + l);
      v[k].m = 0u;
      v[k].d = *reinterpret_cast<const uint32_t*>(blk + 80);
      v[k].sc = blk[j];
    }
  }
#pragma unroll
  for (int k = 0; k < kSB; ++k) {
    if (b0 + k >= nblocks) break;  // uniform over the wavefront
    uint32_t q = (v[k].q >> (2 * g)) & 0x03030303u;
    float4 o;
    if constexpr (Q3 != 0) {
      q |= ((v[k].m >> (4 * h + g)) & 0x01010101u) << 2;
      o = scale_bytes_signed(q, f16_to_f32(v[k].d) * static_cast<float>(static_cast<int>(v[k].sc) - 32), 4);
    } else {
      const float dsc = f16_to_f32(v[k].d & 0xFFFF) * static_cast<float>(v[k].sc & 15);
      const float dm = f16_to_f32(v[k].d >> 16) * static_cast<float>(v[k].sc >> 4);
      o.x = dsc * static_cast<float>(q & 0xFF) - dm;
      o.y = dsc * static_cast<float>((q >> 8) & 0xFF) - dm;
      o.z = dsc * static_cast<float>((q >> 16) & 0xFF) - dm;
      o.w = dsc * static_cast<float>(q >> 24) - dm;
    }
    store_f4(dst + (b0 + k) * 256 + e0, o);
  }
}

}  // namespace

hipError_t launch_dequantize(int type, const uint8_t* src, float* dst, int64_t nblocks,
                             hipStream_t s) {
  if (nblocks <= 0) return hipSuccess;
  // 32-element formats: 8 lanes per block; K-quants: kSB superblocks per wavefront
  const bool small = type == kQ8_0 || type == kQ4_0 || type == kQ4_1 || type == kQ5_0 || type == kQ5_1;
  unsigned grid = 0;
  if (!launch_grid(small ? (nblocks * 8 + 255) / 256 : (nblocks + 4 * kSB - 1) / (4 * kSB), 256, &grid))
    return hipErrorInvalidConfiguration;
  switch (type) {
    case kQ8_0: dequant_q8_0_kernel<<<grid, 256, 0, s>>>(src, dst, nblocks); break;
    case kQ4_0: dequant_q4_0_kernel<<<grid, 256, 0, s>>>(src, dst, nblocks); break;
    case kQ4_1: dequant_q4_1_kernel<<<grid, 256, 0, s>>>(src, dst, nblocks); break;
    case kQ5_0: dequant_q5_0_kernel<<<grid, 256, 0, s>>>(src, dst, nblocks); break;
    case kQ5_1: dequant_q5_1_kernel<<<grid, 256, 0, s>>>(src, dst, nblocks); break;
    case kQ4_K: dequant_q4_K_kernel<0><<<grid, 256, 0, s>>>(src, dst, nblocks); break;
    case kQ5_K: dequant_q4_K_kernel<1><<<grid, 256, 0, s>>>(src, dst, nblocks); break;
    case kQ6_K: dequant_q6_K_kernel<<<grid, 256, 0, s>>>(src, dst, nblocks); break;
    case kQ2_K: dequant_q23_K_kernel<0><<<grid, 256, 0, s>>>(src, dst, nblocks); break;
    case kQ3_K: dequant_q23_K_kernel<1><<<grid, 256, 0, s>>>(src, dst, nblocks); break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qk
