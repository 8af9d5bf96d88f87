// qk_gemv.hip - batch-1 GEMV kernels y = W x for gfx950, one per weight format.
//
// Method (rml "Quantized dot products" and "Kernels and references"; codeloopback
// Examples 10 and 11; candle formats page, VecDotType and BlockQ8K): x has been
// quantized once into int8 blocks aligned with W's blocks; for each (row, block)
// the products of codes are summed exactly in int32 (v_dot4 over packed bytes),
// the K-quant sub-block scales are applied as int32 multiply-adds, and only the
// block step uses floats:
//   Q8_0, Q4_0, Q5_0  c = s * (d_w * d_x)  (Q5_0: codeloopback Example 8's 5-bit
//               codes, bit 4 from qh, paired with Q8_0 per candle's VecDotType)
//   Q4_K, Q5_K  c = (d_x * d) * S_q - (d_x * dmin) * S_m,
//               S_q = sum_j sc_j s_j, S_m = sum_j m_j (bsum_2j + bsum_2j+1)
//               (Q5_K: the same with 5-bit codes, bit 4 from qh)
//   Q6_K        c = (d_x * d) * S,  S = sum_j sc_j sum_e (q_e - 32) a_e
//   Q4_1, Q5_1  against Q8_1: c = s * (d_w * d_x) + m_w * s_x, s = sum code a
//   Q2_K        as Q4_K over 16-element sub-blocks (2-bit codes, 4-bit scale / min)
//   Q3_K        c = (d_x * d) * S,  S = sum_j (sc_j - 32) sum_e (q_e - 4) a_e
// y[row] is the f32 sum of c over the row's blocks.
//
// Mapping on the GPU (all kernels):
//  - one wavefront per output row; its lanes cover a span of consecutive blocks
//    (Q2_K .. Q6_K: 4 lanes per 256-element superblock, 16 superblocks per pass;
//    Q8_0, Q4_0, Q5_0, Q4_1, Q5_1: 1 lane per 32-element block, 64 blocks per pass);
//  - rows of one or two passes keep the activation blocks a lane needs in
//    registers, loaded once per wavefront and reused over grid-strided rows;
//  - longer rows share the activation row through LDS: every lane issues the
//    global loads of up to UNR passes of its row first, then the workgroup copies
//    the paired activation row into LDS (Q8_K: the 292-byte blocks as they are;
//    Q8_0: codes at a padded 48-byte stride, scales converted to f32), so the HBM
//    stream is in flight while the activations are copied;
//  - lanes of one superblock combine their int32 partial sums with DPP (exact),
//    then one lane applies the float step; the row total is a wavefront sum.
#include <hip/hip_ext.h>

#include <atomic>

#include "qk_device.h"
#include "qk_internal.h"


namespace qk {
namespace {

constexpr uint32_t kLo4 = 0x0F0F0F0Fu;
constexpr uint32_t kHi2 = 0x30303030u;
constexpr uint32_t kOnes = 0x01010101u;

// Q5_0 codes of four elements: their low nibbles (one per byte) plus bit 4 taken
// from four consecutive qh bits starting at `shift` (multiplying the 4-bit field by
// 0x204081 copies bit i to bit 8i).
__device__ __forceinline__ uint32_t q5_codes(uint32_t nibbles, uint32_t qh, int shift) {
  return nibbles | (((((qh >> shift) & 0xFu) * 0x00204081u) & kOnes) << 4);
}


__host__ __device__ constexpr int64_t align16(int64_t v) { return (v + 15) & ~int64_t(15); }

// ---------------------------------------------------------------------------
// LDS layout of a Q8_0 activation row (for Q8_0 and Q4_0 weights): 32 codes per
// block at a 48-byte stride (lanes of a pass read consecutive blocks), then d
// (f32) per block.
struct LayoutQ80 {
  static constexpr int kStride = 48;
  int64_t off_d, bytes;
  __host__ __device__ explicit LayoutQ80(int64_t nb) {
    off_d = nb * kStride;
    bytes = align16(off_d + 4 * nb);
  }
};

// Staging of one Q8_0 activation row into LDS.
//
// The row is split into 16-byte pieces of codes (one dwordx4 load and one
// ds_write_b128 each) and small units (the block scale and the bsums).  Staging
// runs in two phases so that its global loads are issued before the weight loads:
// `load` fills registers, `place` writes LDS after the weight loads are in
// flight; because the load counter retires in order, `place` then waits for the
// older activation loads only.  Every index is clamped to the last unit, so all
// lanes issue the same loads without branches (a clamped lane rewrites the value
// the last unit already holds).  Units beyond kPieces / kSmall per thread (rows
// longer than 16 K elements) are copied by a plain loop afterwards.
constexpr int kPieces = 4;
constexpr int kSmall = 2;

struct StagedQ80 {
  uint4 piece[kPieces];
  uint16_t small[kSmall];
};

__device__ __forceinline__ int sext16_lo(uint32_t v) { return static_cast<int16_t>(v & 0xFFFF); }
// Signed 16-bit half `hi` (0 or 1) and signed byte at bit `off` of v, one v_bfe_i32 each.
__device__ __forceinline__ int sbfe16(uint32_t v, int hi) { return static_cast<int>(__builtin_amdgcn_sbfe(v, 16 * hi, 16)); }
__device__ __forceinline__ int sbfe8(uint32_t v, int off) { return static_cast<int>(__builtin_amdgcn_sbfe(v, off, 8)); }
__device__ __forceinline__ int sext16_hi(uint32_t v) { return static_cast<int16_t>(v >> 16); }

// Q8_0 block i (34 bytes): pieces 0, 1 = codes at 2 and 18; small unit = f16 d at 0.
// LDS: piece p -> 48 i + 16 p; d -> off_d + 4 i as f32.
template <int NT>
__device__ __forceinline__ void stage_load_q80(StagedQ80& st, const uint8_t* __restrict__ xq, int nb) {
  const int np = nb * 2;
#pragma unroll
  for (int i = 0; i < kPieces; ++i) {
    const int u = min(static_cast<int>(threadIdx.x) + i * NT, np - 1);
    st.piece[i] = load_u2<uint4>(xq + static_cast<uint32_t>((u >> 1) * kQ8_0Bytes + 2 + 16 * (u & 1)));
  }
#pragma unroll
  for (int i = 0; i < kSmall; ++i) {
    const int u = min(static_cast<int>(threadIdx.x) + i * NT, nb - 1);
    st.small[i] = *reinterpret_cast<const uint16_t*>(xq + static_cast<uint32_t>(u * kQ8_0Bytes));
  }
}

template <int NT>
__device__ __forceinline__ void stage_place_q80(uint8_t* lds, const LayoutQ80& L, const StagedQ80& st,
                                                const uint8_t* __restrict__ xq, int nb) {
  const int np = nb * 2;
  float* dA = reinterpret_cast<float*>(lds + L.off_d);
#pragma unroll
  for (int i = 0; i < kPieces; ++i) {
    const int u = min(static_cast<int>(threadIdx.x) + i * NT, np - 1);
    *reinterpret_cast<uint4*>(lds + (u >> 1) * LayoutQ80::kStride + 16 * (u & 1)) = st.piece[i];
  }
#pragma unroll
  for (int i = 0; i < kSmall; ++i) {
    const int u = min(static_cast<int>(threadIdx.x) + i * NT, nb - 1);
    dA[u] = f16_to_f32(st.small[i]);
  }
  for (int u = static_cast<int>(threadIdx.x) + kPieces * NT; u < np; u += NT) {
    *reinterpret_cast<uint4*>(lds + (u >> 1) * LayoutQ80::kStride + 16 * (u & 1)) =
        load_u2<uint4>(xq + (u >> 1) * kQ8_0Bytes + 2 + 16 * (u & 1));
  }
  for (int u = static_cast<int>(threadIdx.x) + kSmall * NT; u < nb; u += NT) {
    dA[u] = f16_to_f32(*reinterpret_cast<const uint16_t*>(xq + u * kQ8_0Bytes));
  }
}

// Keeps the backend scheduler from interleaving the activation and weight loads.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// The code bytes of a 32-element block (4 or 8 dwords) start 2 or 6 bytes into
// the block, and blocks of 18, 22 or 34 bytes are only 2-byte aligned, so a field
// starts 0 or 2 bytes past a dword boundary.  It is read with dword-aligned loads:
// N dwords from the boundary at or below its start and, for a shifted field, its
// last two bytes (a 16-bit load; every byte read lies inside the field), then
// realigned in registers with v_alignbit once the loads have landed.  Measured on
// the 4096 x 11008 Q4_0 GEMV: 7-12 % faster than 16-byte loads at 2-byte alignment.
template <int N>
struct ShiftedField {
  uint32_t w[N];
  uint32_t tail;  // the field's last two bytes when shifted (unused otherwise)
  uint32_t sh;    // 0 or 16: bit offset of the field in w[0]
};

template <int N>
__device__ __forceinline__ ShiftedField<N> load_field(const uint8_t* p) {
  static_assert(N % 4 == 0, "whole 16-byte loads");
  ShiftedField<N> f;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  const uint8_t* base = reinterpret_cast<const uint8_t*>(a & ~uintptr_t(3));
  f.sh = static_cast<uint32_t>(a & 2) * 8;
#pragma unroll
  for (int k = 0; k < N / 4; ++k) {
    uint4 v;
    __builtin_memcpy(&v, __builtin_assume_aligned(base + 16 * k, 4), 16);
    f.w[4 * k] = v.x;
    f.w[4 * k + 1] = v.y;
    f.w[4 * k + 2] = v.z;
    f.w[4 * k + 3] = v.w;
  }
  f.tail = *reinterpret_cast<const uint16_t*>(base + (f.sh ? 4 * N : 4 * N - 4));
  return f;
}

template <int N>
__device__ __forceinline__ void align_field(const ShiftedField<N>& f, uint32_t (&out)[N]) {
#pragma unroll
  for (int j = 0; j < N - 1; ++j) out[j] = __builtin_amdgcn_alignbit(f.w[j + 1], f.w[j], f.sh);
  out[N - 1] = __builtin_amdgcn_alignbit(f.tail, f.w[N - 1], f.sh);
}

template <typename T>
__device__ __forceinline__ T load_a4(const uint8_t* p) {  // 4-byte aligned field
  const uint32_t* p4 = reinterpret_cast<const uint32_t*>(__builtin_assume_aligned(p, 4));
  T v;
  __builtin_memcpy(&v, p4, sizeof(T));
  return v;
}

// S_q and S_m partials of chunk c (sub-blocks 2c, 2c+1) from its two sub-block
// code sums slo, shi and activation sums asum: get_scale_min_k4 for all four
// sub-blocks of a group at once: sub-blocks 0-3 take the low 6 bits of scale bytes
// 0-3 / 4-7; sub-blocks 4-7 take the low / high nibble of bytes 8-11 and the top 2
// bits of bytes 0-3 / 4-7.  hi_mask is all ones for chunks 2 and 3 (sub-blocks
// 4-7), zero otherwise, so the scale words are selected with bit operations
// instead of a divergent branch; sh = 16 (c & 1) picks the byte pair.
__device__ __forceinline__ int2 q4K_scale_mins(int slo, int shi, const uint4& h, int2 asum,
                                               uint32_t hi_mask, int sh) {
  const uint32_t sc_a = h.y & 0x3F3F3F3Fu;
  const uint32_t m_a = h.z & 0x3F3F3F3Fu;
  const uint32_t sc_b = (h.w & kLo4) | ((h.y >> 2) & kHi2);
  const uint32_t m_b = ((h.w >> 4) & kLo4) | ((h.z >> 2) & kHi2);
  const uint32_t scw = (sc_b & hi_mask) | (sc_a & ~hi_mask);
  const uint32_t mw = (m_b & hi_mask) | (m_a & ~hi_mask);
  const int sc_lo = __builtin_amdgcn_ubfe(scw, sh, 8), sc_hi = __builtin_amdgcn_ubfe(scw, sh + 8, 8);
  const int m_lo = __builtin_amdgcn_ubfe(mw, sh, 8), m_hi = __builtin_amdgcn_ubfe(mw, sh + 8, 8);
  return make_int2(mad24(sc_lo, slo, __mul24(sc_hi, shi)), mad24(m_lo, asum.x, __mul24(m_hi, asum.y)));
}

// Exact integer part of one Q4_K superblock for chunk c (sub-blocks 2c, 2c+1):
// returns this lane's S_q and S_m partial sums (before the quad reduction).
__device__ __forceinline__ int2 q4K_chunk(const uint4& q0, const uint4& q1, const uint4& h,
                                          const uint4& a0, const uint4& a1, const uint4& a2,
                                          const uint4& a3, int2 asum, uint32_t hi_mask, int sh) {
  int slo = 0, shi = 0;
  slo = dot4(q0.x & kLo4, a0.x, slo);
  slo = dot4(q0.y & kLo4, a0.y, slo);
  slo = dot4(q0.z & kLo4, a0.z, slo);
  slo = dot4(q0.w & kLo4, a0.w, slo);
  slo = dot4(q1.x & kLo4, a1.x, slo);
  slo = dot4(q1.y & kLo4, a1.y, slo);
  slo = dot4(q1.z & kLo4, a1.z, slo);
  slo = dot4(q1.w & kLo4, a1.w, slo);
  shi = dot4((q0.x >> 4) & kLo4, a2.x, shi);
  shi = dot4((q0.y >> 4) & kLo4, a2.y, shi);
  shi = dot4((q0.z >> 4) & kLo4, a2.z, shi);
  shi = dot4((q0.w >> 4) & kLo4, a2.w, shi);
  shi = dot4((q1.x >> 4) & kLo4, a3.x, shi);
  shi = dot4((q1.y >> 4) & kLo4, a3.y, shi);
  shi = dot4((q1.z >> 4) & kLo4, a3.z, shi);
  shi = dot4((q1.w >> 4) & kLo4, a3.w, shi);
  return q4K_scale_mins(slo, shi, h, asum, hi_mask, sh);
}

// Q5_K chunk c: the Q4_K nibbles plus, for element 64c + p, bit 2c (p < 32) or
// 2c + 1 (p >= 32) of qh byte p % 32 as bit 4.  qh0 / qh1 are qh bytes 0-15 /
// 16-31 after rot_q5 (each word rotated right by 2c - 4), so bits 4 and 5 of each
// byte are this chunk's two fifth bits.  Codes stay below 32, so the signed dot is
// exact.
__device__ __forceinline__ int2 q5K_chunk(const uint4& q0, const uint4& q1, const uint4& qh0,
                                          const uint4& qh1, const uint4& h, const uint4& a0,
                                          const uint4& a1, const uint4& a2, const uint4& a3,
                                          int2 asum, uint32_t hi_mask, int sh) {
  const uint32_t ql[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
  const uint32_t qh[8] = {qh0.x, qh0.y, qh0.z, qh0.w, qh1.x, qh1.y, qh1.z, qh1.w};
  const uint32_t al[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
  const uint32_t ah[8] = {a2.x, a2.y, a2.z, a2.w, a3.x, a3.y, a3.z, a3.w};
  int slo = 0, shi = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t lo = (ql[k] & kLo4) | (qh[k] & 0x10101010u);
    const uint32_t hi = ((ql[k] >> 4) & kLo4) | ((qh[k] >> 1) & 0x10101010u);
    slo = dot4(lo, al[k], slo);
    shi = dot4(hi, ah[k], shi);
  }
  return q4K_scale_mins(slo, shi, h, asum, hi_mask, sh);
}



// Image staging of a Q8_K activation row: the row's bytes are copied to LDS
// unchanged (16-byte chunks: one dwordx4 load and one ds_write_b128 each), so the
// copy needs almost no index arithmetic; readers address the image directly
// (block b at 292 b: d at +0, codes at +4, bsums at +260; 4-byte aligned fields).
// As with the other staging, loads go out before the weight loads, and chunk
// indices are clamped so every lane issues the same loads.
constexpr int kImgChunks = 4;

struct ImageQ8K {
  uint4 v[kImgChunks];
  uint32_t tail;
};

template <int NT>
__device__ __forceinline__ void image_load_q8K(ImageQ8K& st, const uint8_t* __restrict__ xq, int nb) {
  const int bytes = nb * kQ8_KBytes;
  const int nch = bytes >> 4;
#pragma unroll
  for (int i = 0; i < kImgChunks; ++i) {
    const int k = min(static_cast<int>(threadIdx.x) + i * NT, nch - 1);
    st.v[i] = load_a4<uint4>(xq + static_cast<uint32_t>(16 * k));
  }
  // the last (bytes mod 16) / 4 dwords
  const int ntail = (bytes & 15) >> 2;
  const int t = min(static_cast<int>(threadIdx.x), max(ntail - 1, 0));
  st.tail = ntail ? *reinterpret_cast<const uint32_t*>(xq + static_cast<uint32_t>(16 * nch + 4 * t)) : 0u;
}

template <int NT>
__device__ __forceinline__ void image_place_q8K(uint8_t* lds, const ImageQ8K& st,
                                                const uint8_t* __restrict__ xq, int nb) {
  const int bytes = nb * kQ8_KBytes;
  const int nch = bytes >> 4;
#pragma unroll
  for (int i = 0; i < kImgChunks; ++i) {
    const int k = min(static_cast<int>(threadIdx.x) + i * NT, nch - 1);
    *reinterpret_cast<uint4*>(lds + 16 * k) = st.v[i];
  }
  const int ntail = (bytes & 15) >> 2;
  if (static_cast<int>(threadIdx.x) < ntail) {
    *reinterpret_cast<uint32_t*>(lds + 16 * nch + 4 * threadIdx.x) = st.tail;
  }
  for (int k = static_cast<int>(threadIdx.x) + kImgChunks * NT; k < nch; k += NT) {
    *reinterpret_cast<uint4*>(lds + 16 * k) = load_a4<uint4>(xq + static_cast<uint32_t>(16 * k));
  }
}

template <typename T>
__device__ __forceinline__ T lds_a4(const uint8_t* p) {  // 4-byte aligned LDS field
  const uint32_t* p4 = reinterpret_cast<const uint32_t*>(__builtin_assume_aligned(p, 4));
  T v;
  __builtin_memcpy(&v, p4, sizeof(T));
  return v;
}

// Lane K's value in every lane of its group of 4 (DPP quad_perm [K,K,K,K]).
template <int K>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), K * 0x55, 0xF, 0xF, false));
}
// DPP quad_perm with the control word P: lane i of each quad takes lane (P >> 2i) & 3.
template <int P>
__device__ __forceinline__ uint32_t quad_perm(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), P, 0xF, 0xF, false));
}

// The four lanes of a quad hold one K-quant superblock, and each needs all of its
// 16-byte header (d, dmin, scales) and, for Q5_K, all 32 qh bytes.  In the LDS kernel
// below lane c loads only header dword c and qh bytes 16 + 8c .. 23 + 8c, and the
// rest comes from the other lanes by DPP: four loads of the same bytes per quad cost
// address-unit time, a broadcast one VALU instruction.  (4096 x 14336 Q5_K: 8.91 ->
// 8.55-8.60 us, Q4_K 7.48-7.49 -> 7.35-7.39, 4096 x 11008 Q4_K 6.21-6.27 -> 6.17-6.18.
// The register-resident row-walking kernels measured 2-3 % slower with the same
// change, the gate / up pair kernel of Q5_K 13 % slower, and keep full loads.)
// Callers keep all four lanes of a quad active wherever these run.
__device__ __forceinline__ uint32_t load_head(const uint8_t* p, int c) {
  return *reinterpret_cast<const uint32_t*>(p + 4 * c);
}
__device__ __forceinline__ uint4 head_of(uint32_t w) {
  return make_uint4(quad_bcast<0>(w), quad_bcast<1>(w), quad_bcast<2>(w), quad_bcast<3>(w));
}
__device__ __forceinline__ uint2 load_qh(const uint8_t* p, int c) {
  return *reinterpret_cast<const uint2*>(p + 16 + 8 * c);
}
__device__ __forceinline__ uint4 qh_lo(uint2 v) {  // qh bytes 0 .. 15
  return make_uint4(quad_bcast<0>(v.x), quad_bcast<0>(v.y), quad_bcast<1>(v.x), quad_bcast<1>(v.y));
}
__device__ __forceinline__ uint4 qh_hi(uint2 v) {  // qh bytes 16 .. 31
  return make_uint4(quad_bcast<2>(v.x), quad_bcast<2>(v.y), quad_bcast<3>(v.x), quad_bcast<3>(v.y));
}

// ---------------------------------------------------------------------------
// Q4_K x Q8_K.  Lane (u = lane >> 2, c = lane & 3) of pass `it` handles 64-element
// chunk c of superblock it*16 + u: qs[32c .. 32c+31] hold sub-block 2c in their low
// nibbles and sub-block 2c+1 in their high nibbles.  Q5 selects Q5_K: 176-byte
// superblocks whose qs start at byte 48, and every lane also loads the 32 qh bytes
// (bytes 16-47) for the fifth bits of its chunk.
template <int Q5>
struct KQuant4 {
  static constexpr int kBytes = Q5 ? kQ5_KBytes : kQ4_KBytes;
  static constexpr int kQs = Q5 ? 48 : 16;
};

// The qh words of Q5_K chunk c rotated right by 2c - 4 (mod 32): bit 2c of every
// byte lands on bit 4 of the same byte and bit 2c + 1 on bit 5 (the bits that wrap
// around stay below bit 4 of byte 0).
__device__ __forceinline__ uint4 rot_q5(const uint4& v, int c) {
  const uint32_t r = static_cast<uint32_t>(2 * c - 4) & 31u;
  return make_uint4(__builtin_amdgcn_alignbit(v.x, v.x, r), __builtin_amdgcn_alignbit(v.y, v.y, r),
                    __builtin_amdgcn_alignbit(v.z, v.z, r), __builtin_amdgcn_alignbit(v.w, v.w, r));
}

template <int NW, int UNR, bool SUMS, int Q5 = 0>
__global__ __launch_bounds__(NW * 64) void gemv_q4_K_kernel(
    const uint8_t* __restrict__ W, int n_out, int nb, const uint8_t* __restrict__ xq,
    float* __restrict__ y, int32_t* __restrict__ sums) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * NW + wave_id();
  const int c = lane & 3, u = lane >> 2;
  const bool row_ok = row < n_out;
  using F = KQuant4<Q5>;
  const size_t rb = static_cast<size_t>(nb) * F::kBytes;
  const uint8_t* wrow = W + static_cast<size_t>(row_ok ? row : n_out - 1) * rb;
  const int passes = (nb + 15) >> 4;

  uint32_t H[UNR];
  uint4 Q0[UNR], Q1[UNR];
  uint2 QH[Q5 ? UNR : 1];
  // Unconditional loads (superblock index clamped): the same number of loads in
  // every lane lets the compiler wait for pass j's data only.
  auto issue = [&](int p0) {
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
      const int sb = min((p0 + j) * 16 + u, nb - 1);
      const uint8_t* p = wrow + static_cast<uint32_t>(sb * F::kBytes);
      H[j] = load_head(p, c);
      Q0[j] = *reinterpret_cast<const uint4*>(p + F::kQs + 32 * c);
      Q1[j] = *reinterpret_cast<const uint4*>(p + F::kQs + 16 + 32 * c);
      if constexpr (Q5 != 0) {
        QH[j] = load_qh(p, c);
      }
    }
  };
  ImageQ8K st;
  image_load_q8K<NW * 64>(st, xq, nb);
  sched_fence();
  issue(0);
  sched_fence();
  image_place_q8K<NW * 64>(lds, st, xq, nb);
  __syncthreads();

  const int sh = (c & 1) * 16;   // byte pair of this chunk's two sub-blocks
  const uint32_t hi_mask = (c & 2) ? 0xFFFFFFFFu : 0u;
  float acc = 0.0f;

  for (int p0 = 0; p0 < passes; p0 += UNR) {
    if (p0 > 0) issue(p0);
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
      const int sb = (p0 + j) * 16 + u;
      if (!row_ok || sb >= nb) continue;  // uniform over the 4 lanes of a superblock
      const uint8_t* blk = lds + sb * kQ8_KBytes;
      const uint8_t* ap = blk + 4 + 64 * c;
      const uint4 a0 = lds_a4<uint4>(ap);
      const uint4 a1 = lds_a4<uint4>(ap + 16);
      const uint4 a2 = lds_a4<uint4>(ap + 32);
      const uint4 a3 = lds_a4<uint4>(ap + 48);
      const uint2 bsw = lds_a4<uint2>(blk + 260 + 8 * c);  // bsums 4c .. 4c+3
      const int2 asum = make_int2(sext16_lo(bsw.x) + sext16_hi(bsw.x), sext16_lo(bsw.y) + sext16_hi(bsw.y));
      const float dx = lds_a4<float>(blk);
      const uint4 h = head_of(H[j]);
      int2 part;
      if constexpr (Q5 != 0) {
        part = q5K_chunk(Q0[j], Q1[j], rot_q5(qh_lo(QH[j]), c), rot_q5(qh_hi(QH[j]), c), h, a0, a1, a2, a3, asum,
                         hi_mask, sh);
      } else {
        part = q4K_chunk(Q0[j], Q1[j], h, a0, a1, a2, a3, asum, hi_mask, sh);
      }
      const int sq = quad_sum(part.x);
      const int sm = quad_sum(part.y);
      const float cb = (dx * f16_to_f32(h.x & 0xFFFF)) * static_cast<float>(sq) -
                       (dx * f16_to_f32(h.x >> 16)) * static_cast<float>(sm);
      acc += (c == 0) ? cb : 0.0f;
      if (c == 0) {
        if constexpr (SUMS) {
          int32_t* o = sums + (static_cast<size_t>(row) * nb + sb) * 2;
          o[0] = sq;
          o[1] = sm;
        }
      }
    }
  }
  if (row_ok) {
    const float total = wave_sum(acc);
    if (lane == 0 && y != nullptr) y[row] = total;
  }
}

// ---------------------------------------------------------------------------
// Q2_K and Q3_K x Q8_K (GGUF arrangement; the pages give only their sizes and that
// they are K-quants paired with Q8K).  Sub-blocks of 16 elements; element
// e = 128h + 32g + l has its 2 low code bits at bits 2g of qs[32h + l].
//   Q2_K (84 B: scales[16] @0, qs @16, d @80, dmin @82): code 0..3, scales[j] =
//        scale | min << 4;  c = (d_x d) S_q - (d_x dmin) S_m with
//        S_q = sum_j sc_j sum q a, S_m = sum_j m_j bsum_j (one Q8_K bsum per sub-block).
//   Q3_K (110 B: hmask @0, qs @32, scales[12] @96, d @108): bit 2 of the code is bit
//        4h + g of hmask[l]; value (code - 4) (scale_j - 32), the 6-bit scale split
//        into a low nibble (byte j, or the high nibble of byte j - 8) and 2 high bits
//        (bits 2(j/4) of byte 8 + j % 4);  c = (d_x d) S,
//        S = sum_j (scale_j - 32) (sum code a - 4 bsum_j), codes taken unsigned 0..7.
// Lane (u = lane >> 2, c = lane & 3) of a pass takes superblock 16 pass + u.
//  - Q2_K: elements 64c .. 64c + 63 (sub-blocks 4c .. 4c + 3, half h = c >> 1, shift
//    groups 2 (c & 1) and 2 (c & 1) + 1), from the 32 qs bytes of half h, the 4 scale
//    bytes of its sub-blocks and d / dmin: 84-byte blocks keep every field 4-byte
//    aligned.
//  - Q3_K: qs bytes 16c .. 16c + 15 (half h = c >> 1, l = 16 (c & 1) + i), which in
//    shift group g hold elements 128h + 32g + 16 (c & 1) + i, sub-block 8h + 2g +
//    (c & 1); with the 16 hmask bytes of its l range each qs and hmask byte goes
//    through the address unit once or twice per superblock instead of four times
//    (measured on 4096 x 11008: 7.6 against 9.3 us with the Q2_K mapping, which in
//    turn is faster for Q2_K: 5.1 against 5.6 us).  The blocks are only 2-byte
//    aligned: the fields are read as 4-byte aligned dwords and shifted into place
//    (q23_load).
template <int Q3>
struct KQuant23 {
  static constexpr int kBytes = Q3 ? kQ3_KBytes : kQ2_KBytes;
  static constexpr int kQs = Q3 ? 32 : 16;
};

struct Q23Loads {
  uint4 q0;       // Q2_K: qs bytes 16c .. 16c + 15; Q3_K: the aligned words at or below qs bytes 16c ..
  uint4 m;        // Q3_K: the 4-byte aligned words at or below hmask bytes 16 (c & 1) ..
  uint2 sc;       // Q2_K: sc.x = scales[4c .. 4c + 3]; Q3_K: sc.x = aligned scale word c
  uint32_t sc2;   // Q3_K: shift of the aligned words (0 or 16 bits)
  uint32_t d;     // Q2_K: d | dmin << 16; Q3_K: d
};

template <int Q3>
__device__ __forceinline__ void q23_load(Q23Loads& v, const uint8_t* p, int c) {
  using F = KQuant23<Q3>;
  if constexpr (Q3 != 0) {
    // Every field starts a multiple of 4 bytes into the 110-byte block, and the block
    // itself is only 2-byte aligned.  Loads at 2-byte aligned addresses take a slow
    // path (Q3_K 4096 x 11008 with the products removed: 5.67 us, 4.62 with the same
    // loads 4-byte aligned), so each lane reads 4-byte aligned words from pa, the
    // aligned address at or just below the block (sh = 0 or 16 bits of shift), and
    // q23_chunk shifts them into place.  The lane loads its 16 qs bytes and its 16
    // hmask bytes as dwordx4 from pa, plus dword c of the 16 bytes at pa + 96 (the
    // scales); the word after each dwordx4 and the other scale words come from the
    // other lanes of the quad, which hold the same block.  All words lie inside the
    // block, except that a block at 2 mod 4 also reads the 2 bytes before it (the
    // previous block's; the first block of W is 16-byte aligned) and that with sh = 0
    // lane 3 re-reads scale word 2 (its word 3 would end past the block).
    const uint32_t sh = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p) & 2u) * 8u;
    const uint8_t* pa = p - (sh >> 3);
    v.q0 = load_a4<uint4>(pa + F::kQs + 16 * c);
    v.m = load_a4<uint4>(pa + 16 * (c & 1));
    v.sc.x = load_a4<uint32_t>(pa + 96 + 4 * ((sh == 0 && c == 3) ? 2 : c));
    v.sc2 = sh;
    v.d = *reinterpret_cast<const uint16_t*>(p + 108);
  } else {
    v.q0 = load_a4<uint4>(p + F::kQs + 16 * c);  // qs bytes 16c .. 16c + 15
    v.sc.x = load_a4<uint32_t>(p + 4 * c);
    v.d = load_a4<uint32_t>(p + 80);
  }
}

// This lane's exact integer partials of one superblock: Q2_K (S_q, S_m), Q3_K (S, 0).
template <int Q3>
__device__ __forceinline__ int2 q23_chunk(const Q23Loads& v, const uint8_t* ablk, int c) {
  const int h = c >> 1, lh = c & 1;
  int sq = 0, sm = 0;
  if constexpr (Q3 != 0) {
    const uint4 bsv = lds_a4<uint4>(ablk + 260 + 16 * h);  // bsums 8h .. 8h + 7
    const uint32_t bw[4] = {bsv.x, bsv.y, bsv.z, bsv.w};
    // the block's fields from the 4-byte aligned words of q23_load: the scale words
    // from the quad's four lanes, the word after this lane's qs bytes from lane c + 1
    // (lane 3: scale word 0), the word after its hmask bytes from lane c + 1 (hmask
    // bytes 16 ..) or lane 0 (qs bytes 0 ..)
    const uint32_t sh = v.sc2;
    const uint32_t w0 = quad_bcast<0>(v.sc.x), w1 = quad_bcast<1>(v.sc.x);
    const uint32_t w2 = quad_bcast<2>(v.sc.x), w3 = quad_bcast<3>(v.sc.x);
    const uint32_t qnext = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v.q0.x), 0xF9, 0xF, 0xF, false));  // [1,2,3,3]
    const uint32_t qn = (c == 3) ? w0 : qnext;
    const uint32_t mn = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>((c & 1) ? v.m.x : v.q0.x), 0x31, 0xF, 0xF, false));  // [1,0,3,0]
    const uint32_t qw[4] = {__builtin_amdgcn_alignbit(v.q0.y, v.q0.x, sh), __builtin_amdgcn_alignbit(v.q0.z, v.q0.y, sh),
                            __builtin_amdgcn_alignbit(v.q0.w, v.q0.z, sh), __builtin_amdgcn_alignbit(qn, v.q0.w, sh)};
    const uint4 mraw = make_uint4(__builtin_amdgcn_alignbit(v.m.y, v.m.x, sh), __builtin_amdgcn_alignbit(v.m.z, v.m.y, sh),
                                  __builtin_amdgcn_alignbit(v.m.w, v.m.z, sh), __builtin_amdgcn_alignbit(mn, v.m.w, sh));
    const uint2 scw = make_uint2(__builtin_amdgcn_alignbit(w1, w0, sh), __builtin_amdgcn_alignbit(w2, w1, sh));
    const uint32_t sc2w = __builtin_amdgcn_alignbit(w3, w2, sh);
    // Bit 2 of the code of shift group g is bit 4h + g of the hmask byte: rotating
    // each hmask word right by 4h - 2 (mod 32) puts bit 4h + g of every byte at bit
    // g + 2 of the same byte (the bits that wrap around land below bit 2 of byte 0,
    // which no group reads).
    const uint32_t rot = h ? 2u : 30u;
    const uint32_t mq[4] = {__builtin_amdgcn_alignbit(mraw.x, mraw.x, rot), __builtin_amdgcn_alignbit(mraw.y, mraw.y, rot),
                            __builtin_amdgcn_alignbit(mraw.z, mraw.z, rot), __builtin_amdgcn_alignbit(mraw.w, mraw.w, rot)};
    // 6-bit scales of sub-blocks j = 8h + 2g + lh, g = 0 .. 3: the low 4 bits are
    // nibble h of scale byte 2g + lh, the high 2 bits are bits 4h + 2 (g >> 1) of
    // scale byte 8 + 2 (g & 1) + lh.  s01 holds the scales of g = 0, 1 in bytes lh and
    // 2 + lh, s23 those of g = 2, 3, each with its bit 5 flipped (the xor flips the
    // upper bit of both 2-bit fields of every byte): a 6-bit s with bit 5 flipped,
    // read as a signed 6-bit field, is s - 32.
    const uint32_t hs = (sc2w >> (4 * h)) ^ 0x0A0A0A0Au;
    const uint32_t s01 = ((scw.x >> (4 * h)) & kLo4) | ((hs & 0x03030303u) << 4);
    const uint32_t s23 = ((scw.y >> (4 * h)) & kLo4) | (((hs >> 2) & 0x03030303u) << 4);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint4 a = lds_a4<uint4>(ablk + 4 + 128 * h + 32 * g + 16 * lh);
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        w[k] = ((qw[k] >> (2 * g)) & 0x03030303u) | ((mq[k] >> g) & 0x04040404u);
      }
      const int bs = static_cast<int>(__builtin_amdgcn_sbfe(bw[g], 16 * lh, 16));  // bsum of sub-block 8h + 2g + lh
      int t = __mul24(bs, -4);  // sum (code - 4) a, the codes taken unsigned
      t = dot4(w[0], a.x, t);
      t = dot4(w[1], a.y, t);
      t = dot4(w[2], a.z, t);
      t = dot4(w[3], a.w, t);
      const int scale = static_cast<int>(__builtin_amdgcn_sbfe(g < 2 ? s01 : s23, 8 * (lh + 2 * (g & 1)), 6));
      sq = mad24(scale, t, sq);  // (scale_j - 32) t_j
    }
  } else {
    const uint8_t* ap = ablk + 4 + 64 * c;
    const uint4 a[4] = {lds_a4<uint4>(ap), lds_a4<uint4>(ap + 16), lds_a4<uint4>(ap + 32), lds_a4<uint4>(ap + 48)};
    const uint2 bsw = lds_a4<uint2>(ablk + 260 + 8 * c);  // bsums 4c .. 4c+3
    const int bs[4] = {sext16_lo(bsw.x), sext16_hi(bsw.x), sext16_lo(bsw.y), sext16_hi(bsw.y)};
    const int g0 = 2 * lh;
    // The lane's half takes qs bytes 32h .. 32h + 31, loaded by lanes 2h and 2h + 1 of
    // the quad (one 16-byte load per lane instead of two; DPP quad_perm [0,0,2,2] and
    // [1,1,3,3]): 11008 x 4096 5.46 -> 5.31 us, 4096 x 14336 6.26-6.39 -> 6.05,
    // 4096 x 11008 unchanged at 5.16.
    const uint4 qa = make_uint4(quad_perm<0xA0>(v.q0.x), quad_perm<0xA0>(v.q0.y), quad_perm<0xA0>(v.q0.z),
                                quad_perm<0xA0>(v.q0.w));
    const uint4 qb = make_uint4(quad_perm<0xF5>(v.q0.x), quad_perm<0xF5>(v.q0.y), quad_perm<0xF5>(v.q0.z),
                                quad_perm<0xF5>(v.q0.w));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint4 q = (k & 1) ? qb : qa;  // bytes l = 16 (k & 1) .. + 15
      const int sh = 2 * (g0 + (k >> 1));
      int s = 0;
      s = dot4((q.x >> sh) & 0x03030303u, a[k].x, s);
      s = dot4((q.y >> sh) & 0x03030303u, a[k].y, s);
      s = dot4((q.z >> sh) & 0x03030303u, a[k].z, s);
      s = dot4((q.w >> sh) & 0x03030303u, a[k].w, s);
      const int scb = static_cast<int>((v.sc.x >> (8 * k)) & 0xFFu);  // scales[4c + k]
      sq = mad24(scb & 15, s, sq);
      sm = mad24(scb >> 4, bs[k], sm);
    }
  }
  return make_int2(sq, sm);
}

template <int NW, int UNR, bool SUMS, int Q3>
__global__ __launch_bounds__(NW * 64) void gemv_q23_K_kernel(
    const uint8_t* __restrict__ W, int n_out, int nb, const uint8_t* __restrict__ xq,
    float* __restrict__ y, int32_t* __restrict__ sums) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * NW + wave_id();
  const int c = lane & 3, u = lane >> 2;
  const bool row_ok = row < n_out;
  using F = KQuant23<Q3>;
  const size_t rb = static_cast<size_t>(nb) * F::kBytes;
  const uint8_t* wrow = W + static_cast<size_t>(row_ok ? row : n_out - 1) * rb;
  const int passes = (nb + 15) >> 4;

  Q23Loads V[UNR];
  auto issue = [&](int p0) {
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
      const int sb = min((p0 + j) * 16 + u, nb - 1);
      q23_load<Q3>(V[j], wrow + static_cast<uint32_t>(sb * F::kBytes), c);
    }
  };
  ImageQ8K st;
  image_load_q8K<NW * 64>(st, xq, nb);
  sched_fence();
  issue(0);
  sched_fence();
  image_place_q8K<NW * 64>(lds, st, xq, nb);
  __syncthreads();

  float acc = 0.0f;
  for (int p0 = 0; p0 < passes; p0 += UNR) {
    if (p0 > 0) issue(p0);
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
      const int sb = (p0 + j) * 16 + u;
      if (!row_ok || sb >= nb) continue;  // uniform over the 4 lanes of a superblock
      const uint8_t* ablk = lds + sb * kQ8_KBytes;
      const int2 part = q23_chunk<Q3>(V[j], ablk, c);
      const int sq = quad_sum(part.x);
      const float dx = lds_a4<float>(ablk);
      float cb;
      if constexpr (Q3 != 0) {
        cb = (dx * f16_to_f32(V[j].d)) * static_cast<float>(sq);
      } else {
        const int sm = quad_sum(part.y);
        cb = (dx * f16_to_f32(V[j].d & 0xFFFF)) * static_cast<float>(sq) -
             (dx * f16_to_f32(V[j].d >> 16)) * static_cast<float>(sm);
        if constexpr (SUMS) {
          if (c == 0) sums[(static_cast<size_t>(row) * nb + sb) * 2 + 1] = sm;
        }
      }
      acc += (c == 0) ? cb : 0.0f;
      if constexpr (SUMS) {
        if (c == 0) sums[(static_cast<size_t>(row) * nb + sb) * (Q3 ? 1 : 2)] = sq;
      }
    }
  }
  if (row_ok) {
    const float total = wave_sum(acc);
    if (lane == 0 && y != nullptr) y[row] = total;
  }
}

// ---------------------------------------------------------------------------
// Q4_K / Q5_K x Q8_K for NC = 2..4 activation columns (a small batch): the LDS
// kernel above with each weight superblock loaded and unpacked once and its codes
// multiplied against every column's activations, the NC Q8_K rows staged one after
// another in LDS (images `img` bytes apart).  W is read once per call instead of
// once per column.  The integer sums and float steps per column are the
// one-column kernel's, in the same order.
template <int Q5>
__device__ __forceinline__ void kq_codes(const uint4& q0, const uint4& q1, const uint4& qh0, const uint4& qh1,
                                         uint32_t (&lo)[8], uint32_t (&hi)[8]) {
  const uint32_t ql[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
  const uint32_t qh[8] = {qh0.x, qh0.y, qh0.z, qh0.w, qh1.x, qh1.y, qh1.z, qh1.w};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    lo[k] = ql[k] & kLo4;
    hi[k] = (ql[k] >> 4) & kLo4;
    if constexpr (Q5 != 0) {  // qh after rot_q5: fifth bits at bits 4 and 5
      lo[k] |= qh[k] & 0x10101010u;
      hi[k] |= (qh[k] >> 1) & 0x10101010u;
    }
  }
}

template <int NW, int UNR, int NC, bool SUMS, int Q5>
__global__ __launch_bounds__(NW * 64) void gemv_q4_K_cols(
    const uint8_t* __restrict__ W, int n_out, int nb, const uint8_t* __restrict__ xq,
    float* __restrict__ y, int32_t* __restrict__ sums) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * NW + wave_id();
  const int c = lane & 3, u = lane >> 2;
  const bool row_ok = row < n_out;
  using F = KQuant4<Q5>;
  const size_t rb = static_cast<size_t>(nb) * F::kBytes;
  const uint8_t* wrow = W + static_cast<size_t>(row_ok ? row : n_out - 1) * rb;
  const int passes = (nb + 15) >> 4;
  const int xrow = nb * kQ8_KBytes;          // bytes of one column's Q8_K row
  const int img = (xrow + 15) & ~15;         // its LDS image, 16-byte aligned

  uint4 H[UNR], Q0[UNR], Q1[UNR], QH0[Q5 ? UNR : 1], QH1[Q5 ? UNR : 1];
  auto issue = [&](int p0) {
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
      const int sb = min((p0 + j) * 16 + u, nb - 1);
      const uint8_t* p = wrow + static_cast<uint32_t>(sb * F::kBytes);
      H[j] = *reinterpret_cast<const uint4*>(p);
      Q0[j] = *reinterpret_cast<const uint4*>(p + F::kQs + 32 * c);
      Q1[j] = *reinterpret_cast<const uint4*>(p + F::kQs + 16 + 32 * c);
      if constexpr (Q5 != 0) {
        QH0[j] = *reinterpret_cast<const uint4*>(p + 16);
        QH1[j] = *reinterpret_cast<const uint4*>(p + 32);
      }
    }
  };
  ImageQ8K st;
  image_load_q8K<NW * 64>(st, xq, nb);
  sched_fence();
  issue(0);
  sched_fence();
  image_place_q8K<NW * 64>(lds, st, xq, nb);
#pragma unroll
  for (int col = 1; col < NC; ++col) {
    const uint8_t* xc = xq + static_cast<uint32_t>(col * xrow);
    ImageQ8K sc;
    image_load_q8K<NW * 64>(sc, xc, nb);
    image_place_q8K<NW * 64>(lds + col * img, sc, xc, nb);
  }
  __syncthreads();

  const int sh = (c & 1) * 16;
  const uint32_t hi_mask = (c & 2) ? 0xFFFFFFFFu : 0u;
  float acc[NC];
#pragma unroll
  for (int col = 0; col < NC; ++col) acc[col] = 0.0f;

  for (int p0 = 0; p0 < passes; p0 += UNR) {
    if (p0 > 0) issue(p0);
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
      const int sb = (p0 + j) * 16 + u;
      if (!row_ok || sb >= nb) continue;  // uniform over the 4 lanes of a superblock
      uint32_t lo[8], hi[8];
      if constexpr (Q5 != 0) {
        kq_codes<1>(Q0[j], Q1[j], rot_q5(QH0[j], c), rot_q5(QH1[j], c), lo, hi);
      } else {
        kq_codes<0>(Q0[j], Q1[j], Q0[j], Q1[j], lo, hi);
      }
      const uint4 h = H[j];
      const float d = f16_to_f32(h.x & 0xFFFF), dmin = f16_to_f32(h.x >> 16);
#pragma unroll
      for (int col = 0; col < NC; ++col) {
        const uint8_t* blk = lds + col * img + sb * kQ8_KBytes;
        const uint8_t* ap = blk + 4 + 64 * c;
        const uint4 a0 = lds_a4<uint4>(ap);
        const uint4 a1 = lds_a4<uint4>(ap + 16);
        const uint4 a2 = lds_a4<uint4>(ap + 32);
        const uint4 a3 = lds_a4<uint4>(ap + 48);
        const uint2 bsw = lds_a4<uint2>(blk + 260 + 8 * c);
        const int2 asum = make_int2(sext16_lo(bsw.x) + sext16_hi(bsw.x), sext16_lo(bsw.y) + sext16_hi(bsw.y));
        const float dx = lds_a4<float>(blk);
        const uint32_t al[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        const uint32_t ah[8] = {a2.x, a2.y, a2.z, a2.w, a3.x, a3.y, a3.z, a3.w};
        int slo = 0, shi = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          slo = dot4(lo[k], al[k], slo);
          shi = dot4(hi[k], ah[k], shi);
        }
        const int2 part = q4K_scale_mins(slo, shi, h, asum, hi_mask, sh);
        const int sq = quad_sum(part.x);
        const int sm = quad_sum(part.y);
        const float cb = (dx * d) * static_cast<float>(sq) - (dx * dmin) * static_cast<float>(sm);
        acc[col] += (c == 0) ? cb : 0.0f;
        if constexpr (SUMS) {
          if (c == 0) {
            int32_t* o = sums + ((static_cast<size_t>(col) * n_out + row) * nb + sb) * 2;
            o[0] = sq;
            o[1] = sm;
          }
        }
      }
    }
  }
  if (row_ok) {
#pragma unroll
    for (int col = 0; col < NC; ++col) {
      const float total = wave_sum(acc[col]);
      if (lane == 0 && y != nullptr) y[static_cast<size_t>(col) * n_out + row] = total;
    }
  }
}

// Codes of one dword of each Q6_K group: low nibbles from the ql words a (groups 0
// and 2: low / high nibbles) and b (groups 1 and 3), the high 2 bits of group g at
// bits 2g of each qh byte of h.  h masked to the fields of groups 0 and 2 (bits 0-1,
// 4-5), and shifted right by 2 and masked to those of groups 1 and 3, lets a single
// bit-field insert take each code's bits 0-3 from the nibble word and bits 4-7 from
// the field word: the bits a shift carries in from the neighbouring byte all land in
// the half the insert discards.
// (The compiler folds a written-out (x & m) | (y & ~m) back into shifts and masks
// here, because it knows y's zero bits, so the insert is written as v_bfi_b32.)
struct Q6Codes {
  uint32_t q0, q1, q2, q3;
};
__device__ __forceinline__ uint32_t bit_insert(uint32_t mask, uint32_t x, uint32_t y) {  // (x & mask) | (y & ~mask)
  uint32_t r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(mask), "v"(x), "v"(y));
  return r;
}
__device__ __forceinline__ Q6Codes q6_codes(uint32_t a, uint32_t b, uint32_t h) {
  const uint32_t h02 = h & 0x33333333u, h13 = (h >> 2) & 0x33333333u;
  Q6Codes r;
  r.q0 = bit_insert(kLo4, a, h02 << 4);
  r.q1 = bit_insert(kLo4, b, h13 << 4);
  r.q2 = bit_insert(kLo4, a >> 4, h02);
  r.q3 = bit_insert(kLo4, b >> 4, h13);
  return r;
}

// ---------------------------------------------------------------------------
// Q6_K x Q8_K.  Lane (u = lane >> 2, p = lane & 3 -> half h = p >> 1, k = p & 1) of
// pass `it` handles, in superblock it*16 + u, positions l in [16k, 16k+16) of half
// h for all four groups g: elements 128h + 32g + l, sub-blocks 8h + 2g + k.
template <int NW, int UNR, bool SUMS>
__global__ __launch_bounds__(NW * 64) void gemv_q6_K_kernel(
    const uint8_t* __restrict__ W, int n_out, int nb, const uint8_t* __restrict__ xq,
    float* __restrict__ y, int32_t* __restrict__ sums) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * NW + wave_id();
  const int pos = lane & 3, u = lane >> 2;
  const int hh = pos >> 1, kk = pos & 1;
  const bool row_ok = row < n_out;
  const size_t rb = static_cast<size_t>(nb) * kQ6_KBytes;
  const uint8_t* wrow = W + static_cast<size_t>(row_ok ? row : n_out - 1) * rb;
  const int passes = (nb + 15) >> 4;

  uint4 A[UNR], B[UNR], QH[UNR];
  uint2 SC[UNR];
  uint32_t D[UNR];
  auto issue = [&](int p0) {
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
      const int sb = min((p0 + j) * 16 + u, nb - 1);
      const uint8_t* p = wrow + static_cast<uint32_t>(sb * kQ6_KBytes);
      A[j] = load_u2<uint4>(p + 64 * hh + 16 * kk);
      B[j] = load_u2<uint4>(p + 64 * hh + 32 + 16 * kk);
      QH[j] = load_u2<uint4>(p + 128 + 32 * hh + 16 * kk);
      SC[j] = load_u2<uint2>(p + 192 + 8 * hh);
      D[j] = *reinterpret_cast<const uint16_t*>(p + 208);
    }
  };
  ImageQ8K st;
  image_load_q8K<NW * 64>(st, xq, nb);
  sched_fence();
  issue(0);
  sched_fence();
  image_place_q8K<NW * 64>(lds, st, xq, nb);
  __syncthreads();

  float acc = 0.0f;

  for (int p0 = 0; p0 < passes; p0 += UNR) {
    if (p0 > 0) issue(p0);
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
      const int sb = (p0 + j) * 16 + u;
      if (!row_ok || sb >= nb) continue;
      const uint8_t* blk = lds + sb * kQ8_KBytes;
      uint4 a[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) a[g] = lds_a4<uint4>(blk + 4 + 128 * hh + 32 * g + 16 * kk);
      const uint4 bw = lds_a4<uint4>(blk + 260 + 16 * hh);  // bsums 8h .. 8h+7
      // q is stored as 0..63: each sub-block's sum (q - 32) a starts at -32 bsum
      const int4 bs = make_int4(__mul24(sbfe16(bw.x, kk), -32), __mul24(sbfe16(bw.y, kk), -32),
                                __mul24(sbfe16(bw.z, kk), -32), __mul24(sbfe16(bw.w, kk), -32));
      const float dx = lds_a4<float>(blk);
      const uint32_t al[4] = {A[j].x, A[j].y, A[j].z, A[j].w};
      const uint32_t bl[4] = {B[j].x, B[j].y, B[j].z, B[j].w};
      const uint32_t hl[4] = {QH[j].x, QH[j].y, QH[j].z, QH[j].w};
      const uint32_t a0[4] = {a[0].x, a[0].y, a[0].z, a[0].w};
      const uint32_t a1[4] = {a[1].x, a[1].y, a[1].z, a[1].w};
      const uint32_t a2[4] = {a[2].x, a[2].y, a[2].z, a[2].w};
      const uint32_t a3[4] = {a[3].x, a[3].y, a[3].z, a[3].w};
      int s0 = bs.x, s1 = bs.y, s2 = bs.z, s3 = bs.w;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const Q6Codes q = q6_codes(al[i], bl[i], hl[i]);
        s0 = dot4(q.q0, a0[i], s0);
        s1 = dot4(q.q1, a1[i], s1);
        s2 = dot4(q.q2, a2[i], s2);
        s3 = dot4(q.q3, a3[i], s3);
      }
      // sub-block scales sc[8h + 2g + k] = byte (2g + k) of the 8 bytes at 192 + 8h
      const int sc0 = sbfe8(SC[j].x, 8 * kk), sc1 = sbfe8(SC[j].x, 16 + 8 * kk);
      const int sc2 = sbfe8(SC[j].y, 8 * kk), sc3 = sbfe8(SC[j].y, 16 + 8 * kk);
      const int part = mad24(sc0, s0, mad24(sc1, s1, mad24(sc2, s2, __mul24(sc3, s3))));
      const int S = quad_sum(part);
      if (pos == 0) {
        const float d = f16_to_f32(D[j]);
        acc += (dx * d) * static_cast<float>(S);
        if constexpr (SUMS) sums[static_cast<size_t>(row) * nb + sb] = S;
      }
    }
  }
  if (row_ok) {
    const float total = wave_sum(acc);
    if (lane == 0 && y != nullptr) y[row] = total;
  }
}

// ---------------------------------------------------------------------------
// Q6_K x Q8_K for NC = 2..4 activation columns: the kernel above with each
// superblock's 6-bit codes and signed scales built once and dotted against every
// column's Q8_K row, the rows staged one after another in LDS (`img` bytes
// apart) as in gemv_q4_K_cols.  Integer sums and float steps per column are the
// one-column kernel's, in the same order.
template <int NW, int UNR, int NC, bool SUMS>
__global__ __launch_bounds__(NW * 64) void gemv_q6_K_cols(
    const uint8_t* __restrict__ W, int n_out, int nb, const uint8_t* __restrict__ xq,
    float* __restrict__ y, int32_t* __restrict__ sums) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * NW + wave_id();
  const int pos = lane & 3, u = lane >> 2;
  const int hh = pos >> 1, kk = pos & 1;
  const bool row_ok = row < n_out;
  const size_t rb = static_cast<size_t>(nb) * kQ6_KBytes;
  const uint8_t* wrow = W + static_cast<size_t>(row_ok ? row : n_out - 1) * rb;
  const int passes = (nb + 15) >> 4;
  const int xrow = nb * kQ8_KBytes;
  const int img = (xrow + 15) & ~15;

  uint4 A[UNR], B[UNR], QH[UNR];
  uint2 SC[UNR];
  uint32_t D[UNR];
  auto issue = [&](int p0) {
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
      const int sb = min((p0 + j) * 16 + u, nb - 1);
      const uint8_t* p = wrow + static_cast<uint32_t>(sb * kQ6_KBytes);
      A[j] = load_u2<uint4>(p + 64 * hh + 16 * kk);
      B[j] = load_u2<uint4>(p + 64 * hh + 32 + 16 * kk);
      QH[j] = load_u2<uint4>(p + 128 + 32 * hh + 16 * kk);
      SC[j] = load_u2<uint2>(p + 192 + 8 * hh);
      D[j] = *reinterpret_cast<const uint16_t*>(p + 208);
    }
  };
  ImageQ8K st;
  image_load_q8K<NW * 64>(st, xq, nb);
  sched_fence();
  issue(0);
  sched_fence();
  image_place_q8K<NW * 64>(lds, st, xq, nb);
#pragma unroll
  for (int col = 1; col < NC; ++col) {
    const uint8_t* xc = xq + static_cast<uint32_t>(col * xrow);
    ImageQ8K sc;
    image_load_q8K<NW * 64>(sc, xc, nb);
    image_place_q8K<NW * 64>(lds + col * img, sc, xc, nb);
  }
  __syncthreads();

  float acc[NC];
#pragma unroll
  for (int col = 0; col < NC; ++col) acc[col] = 0.0f;

  for (int p0 = 0; p0 < passes; p0 += UNR) {
    if (p0 > 0) issue(p0);
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
      const int sb = (p0 + j) * 16 + u;
      if (!row_ok || sb >= nb) continue;
      const uint32_t al[4] = {A[j].x, A[j].y, A[j].z, A[j].w};
      const uint32_t bl[4] = {B[j].x, B[j].y, B[j].z, B[j].w};
      const uint32_t hl[4] = {QH[j].x, QH[j].y, QH[j].z, QH[j].w};
      uint32_t q[4][4];  // q[g][i]: codes of group g, dword i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const Q6Codes c6 = q6_codes(al[i], bl[i], hl[i]);
        q[0][i] = c6.q0;
        q[1][i] = c6.q1;
        q[2][i] = c6.q2;
        q[3][i] = c6.q3;
      }
      const int sc0 = static_cast<int8_t>((SC[j].x >> (8 * kk)) & 0xFF);
      const int sc1 = static_cast<int8_t>((SC[j].x >> (16 + 8 * kk)) & 0xFF);
      const int sc2 = static_cast<int8_t>((SC[j].y >> (8 * kk)) & 0xFF);
      const int sc3 = static_cast<int8_t>((SC[j].y >> (16 + 8 * kk)) & 0xFF);
      const float d = f16_to_f32(D[j]);
#pragma unroll
      for (int col = 0; col < NC; ++col) {
        const uint8_t* blk = lds + col * img + sb * kQ8_KBytes;
        int sg[4] = {0, 0, 0, 0};
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint4 a = lds_a4<uint4>(blk + 4 + 128 * hh + 32 * g + 16 * kk);
          sg[g] = dot4(q[g][0], a.x, sg[g]);
          sg[g] = dot4(q[g][1], a.y, sg[g]);
          sg[g] = dot4(q[g][2], a.z, sg[g]);
          sg[g] = dot4(q[g][3], a.w, sg[g]);
        }
        const uint4 bw = lds_a4<uint4>(blk + 260 + 16 * hh);  // bsums 8h .. 8h+7
        const int b0 = 32 * (kk ? sext16_hi(bw.x) : sext16_lo(bw.x));
        const int b1 = 32 * (kk ? sext16_hi(bw.y) : sext16_lo(bw.y));
        const int b2 = 32 * (kk ? sext16_hi(bw.z) : sext16_lo(bw.z));
        const int b3 = 32 * (kk ? sext16_hi(bw.w) : sext16_lo(bw.w));
        const float dx = lds_a4<float>(blk);
        const int part = mad24(sc0, sg[0] - b0, mad24(sc1, sg[1] - b1, mad24(sc2, sg[2] - b2, __mul24(sc3, sg[3] - b3))));
        const int S = quad_sum(part);
        if (pos == 0) {
          acc[col] += (dx * d) * static_cast<float>(S);
          if constexpr (SUMS) sums[(static_cast<size_t>(col) * n_out + row) * nb + sb] = S;
        }
      }
    }
  }
  if (row_ok) {
#pragma unroll
    for (int col = 0; col < NC; ++col) {
      const float total = wave_sum(acc[col]);
      if (lane == 0 && y != nullptr) y[static_cast<size_t>(col) * n_out + row] = total;
    }
  }
}

// ---------------------------------------------------------------------------
// Q8_0 x Q8_0 and Q4_0 x Q8_0: lane b of pass `it` handles block it*64 + lane.
template <int NW, int UNR, bool SUMS>
__global__ __launch_bounds__(NW * 64) void gemv_q8_0_kernel(
    const uint8_t* __restrict__ W, int n_out, int nb, const uint8_t* __restrict__ xq,
    float* __restrict__ y, int32_t* __restrict__ sums) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * NW + wave_id();
  const bool row_ok = row < n_out;
  const size_t rb = static_cast<size_t>(nb) * kQ8_0Bytes;
  const uint8_t* wrow = W + static_cast<size_t>(row_ok ? row : n_out - 1) * rb;
  const int passes = (nb + 63) >> 6;

  ShiftedField<8> QS[UNR];
  uint32_t D[UNR];
  auto issue = [&](int p0) {
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
      const int b = min((p0 + j) * 64 + lane, nb - 1);
      const uint8_t* p = wrow + static_cast<uint32_t>(b * kQ8_0Bytes);
      D[j] = *reinterpret_cast<const uint16_t*>(p);
      QS[j] = load_field<8>(p + 2);
    }
  };
  const LayoutQ80 L(nb);
  StagedQ80 st;
  stage_load_q80<NW * 64>(st, xq, nb);
  sched_fence();
  issue(0);
  sched_fence();
  stage_place_q80<NW * 64>(lds, L, st, xq, nb);
  __syncthreads();

  const float* dA = reinterpret_cast<const float*>(lds + L.off_d);
  float acc = 0.0f;
  for (int p0 = 0; p0 < passes; p0 += UNR) {
    if (p0 > 0) issue(p0);
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
      const int b = (p0 + j) * 64 + lane;
      if (!row_ok || b >= nb) continue;
      const uint4 a0 = *reinterpret_cast<const uint4*>(lds + b * LayoutQ80::kStride);
      const uint4 a1 = *reinterpret_cast<const uint4*>(lds + b * LayoutQ80::kStride + 16);
      uint32_t q[8];
      align_field(QS[j], q);
      int s = 0;
      s = dot4(q[0], a0.x, s);
      s = dot4(q[1], a0.y, s);
      s = dot4(q[2], a0.z, s);
      s = dot4(q[3], a0.w, s);
      s = dot4(q[4], a1.x, s);
      s = dot4(q[5], a1.y, s);
      s = dot4(q[6], a1.z, s);
      s = dot4(q[7], a1.w, s);
      acc += static_cast<float>(s) * (f16_to_f32(D[j]) * dA[b]);
      if constexpr (SUMS) sums[static_cast<size_t>(row) * nb + b] = s;
    }
  }
  if (row_ok) {
    const float total = wave_sum(acc);
    if (lane == 0 && y != nullptr) y[row] = total;
  }
}

template <int NW, int UNR, bool Q5, bool SUMS>
__global__ __launch_bounds__(NW * 64) void gemv_q4_0_kernel(
    const uint8_t* __restrict__ W, int n_out, int nb, const uint8_t* __restrict__ xq,
    float* __restrict__ y, int32_t* __restrict__ sums) {
  constexpr int kWB = Q5 ? kQ5_0Bytes : kQ4_0Bytes;
  constexpr int kQs = Q5 ? 6 : 2;         // offset of the 16 nibble bytes
  constexpr int kBias = Q5 ? 16 : 8;      // stored code = value + bias
  extern __shared__ __align__(16) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * NW + wave_id();
  const bool row_ok = row < n_out;
  const size_t rb = static_cast<size_t>(nb) * kWB;
  const uint8_t* wrow = W + static_cast<size_t>(row_ok ? row : n_out - 1) * rb;
  const int passes = (nb + 63) >> 6;

  ShiftedField<4> QS[UNR];
  uint32_t D[UNR], QH[UNR];
  auto issue = [&](int p0) {
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
      const int b = min((p0 + j) * 64 + lane, nb - 1);
      const uint8_t* p = wrow + static_cast<uint32_t>(b * kWB);
      D[j] = *reinterpret_cast<const uint16_t*>(p);
      if constexpr (Q5) QH[j] = load_u2<uint32_t>(p + 2);
      QS[j] = load_field<4>(p + kQs);
    }
  };
  const LayoutQ80 L(nb);
  StagedQ80 st;
  stage_load_q80<NW * 64>(st, xq, nb);
  sched_fence();
  issue(0);
  sched_fence();
  stage_place_q80<NW * 64>(lds, L, st, xq, nb);
  __syncthreads();

  const float* dA = reinterpret_cast<const float*>(lds + L.off_d);
  float acc = 0.0f;
  for (int p0 = 0; p0 < passes; p0 += UNR) {
    if (p0 > 0) issue(p0);
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
      const int b = (p0 + j) * 64 + lane;
      if (!row_ok || b >= nb) continue;
      const uint4 a0 = *reinterpret_cast<const uint4*>(lds + b * LayoutQ80::kStride);       // elements 0-15
      const uint4 a1 = *reinterpret_cast<const uint4*>(lds + b * LayoutQ80::kStride + 16);  // 16-31
      uint32_t qw[4];
      align_field(QS[j], qw);
      const uint4 q = make_uint4(qw[0], qw[1], qw[2], qw[3]);
      uint32_t lo[4] = {q.x & kLo4, q.y & kLo4, q.z & kLo4, q.w & kLo4};
      uint32_t hi[4] = {(q.x >> 4) & kLo4, (q.y >> 4) & kLo4, (q.z >> 4) & kLo4, (q.w >> 4) & kLo4};
      if constexpr (Q5) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          lo[k] = q5_codes(lo[k], QH[j], 4 * k);
          hi[k] = q5_codes(hi[k], QH[j], 16 + 4 * k);
        }
      }
      int s = 0, sa = 0;
      s = dot4(lo[0], a0.x, s);
      s = dot4(lo[1], a0.y, s);
      s = dot4(lo[2], a0.z, s);
      s = dot4(lo[3], a0.w, s);
      s = dot4(hi[0], a1.x, s);
      s = dot4(hi[1], a1.y, s);
      s = dot4(hi[2], a1.z, s);
      s = dot4(hi[3], a1.w, s);
      sa = dot4(kOnes, a0.x, sa);
      sa = dot4(kOnes, a0.y, sa);
      sa = dot4(kOnes, a0.z, sa);
      sa = dot4(kOnes, a0.w, sa);
      sa = dot4(kOnes, a1.x, sa);
      sa = dot4(kOnes, a1.y, sa);
      sa = dot4(kOnes, a1.z, sa);
      sa = dot4(kOnes, a1.w, sa);
      s -= kBias * sa;  // codes are stored as value + bias
      acc += static_cast<float>(s) * (f16_to_f32(D[j]) * dA[b]);
      if constexpr (SUMS) sums[static_cast<size_t>(row) * nb + b] = s;
    }
  }
  if (row_ok) {
    const float total = wave_sum(acc);
    if (lane == 0 && y != nullptr) y[row] = total;
  }
}

// ---------------------------------------------------------------------------
// Q4_1 and Q5_1 x Q8_1 (candle formats page, VecDotType table: the _1 weight types
// pair with BlockQ8_1).  Weight value = code * d_w + m_w with unsigned codes, the
// activation d_x * a, so a block contributes
//   c = s * (d_w * d_x) + m_w * s_x,   s = sum code * a (exact int32),
// with s_x the Q8_1 block's stored f16 d_x * sum a.  Blocks of 20 / 24 bytes keep
// every field 4-byte aligned (Q4_1: d, m, qs[16] at 4; Q5_1: d, m, qh at 4, qs at
// 8), so each lane loads its block with one dword and one dwordx4 (plus the qh dword).
// The Q8_1 row is staged into LDS as the Q8_0 row is: codes at a 48-byte stride,
// then d_x and s_x as f32 per block.
struct LayoutQ81 {
  static constexpr int kStride = 48;
  int64_t off_d, off_s, bytes;
  __host__ __device__ explicit LayoutQ81(int64_t nb) {
    off_d = nb * kStride;
    off_s = off_d + 4 * nb;
    bytes = align16(off_s + 4 * nb);
  }
};

struct StagedQ81 {
  uint4 piece[kPieces];
  uint32_t small[kSmall];  // d | s << 16
};

// Q8_1 block i (36 bytes): pieces 0, 1 = codes at 4 and 20; small unit = d, s at 0.
template <int NT>
__device__ __forceinline__ void stage_load_q81(StagedQ81& st, const uint8_t* __restrict__ xq, int nb) {
  const int np = nb * 2;
#pragma unroll
  for (int i = 0; i < kPieces; ++i) {
    const int u = min(static_cast<int>(threadIdx.x) + i * NT, np - 1);
    st.piece[i] = load_a4<uint4>(xq + static_cast<uint32_t>((u >> 1) * kQ8_1Bytes + 4 + 16 * (u & 1)));
  }
#pragma unroll
  for (int i = 0; i < kSmall; ++i) {
    const int u = min(static_cast<int>(threadIdx.x) + i * NT, nb - 1);
    st.small[i] = load_a4<uint32_t>(xq + static_cast<uint32_t>(u * kQ8_1Bytes));
  }
}

template <int NT>
__device__ __forceinline__ void stage_place_q81(uint8_t* lds, const LayoutQ81& L, const StagedQ81& st,
                                                const uint8_t* __restrict__ xq, int nb) {
  const int np = nb * 2;
  float* dA = reinterpret_cast<float*>(lds + L.off_d);
  float* sA = reinterpret_cast<float*>(lds + L.off_s);
#pragma unroll
  for (int i = 0; i < kPieces; ++i) {
    const int u = min(static_cast<int>(threadIdx.x) + i * NT, np - 1);
    *reinterpret_cast<uint4*>(lds + (u >> 1) * LayoutQ81::kStride + 16 * (u & 1)) = st.piece[i];
  }
#pragma unroll
  for (int i = 0; i < kSmall; ++i) {
    const int u = min(static_cast<int>(threadIdx.x) + i * NT, nb - 1);
    dA[u] = f16_to_f32(st.small[i] & 0xFFFFu);
    sA[u] = f16_to_f32(st.small[i] >> 16);
  }
  for (int u = static_cast<int>(threadIdx.x) + kPieces * NT; u < np; u += NT) {
    *reinterpret_cast<uint4*>(lds + (u >> 1) * LayoutQ81::kStride + 16 * (u & 1)) =
        load_a4<uint4>(xq + (u >> 1) * kQ8_1Bytes + 4 + 16 * (u & 1));
  }
  for (int u = static_cast<int>(threadIdx.x) + kSmall * NT; u < nb; u += NT) {
    const uint32_t ds = load_a4<uint32_t>(xq + u * kQ8_1Bytes);
    dA[u] = f16_to_f32(ds & 0xFFFFu);
    sA[u] = f16_to_f32(ds >> 16);
  }
}

template <int NW, int UNR, bool Q5, bool SUMS>
__global__ __launch_bounds__(NW * 64) void gemv_q4_1_kernel(
    const uint8_t* __restrict__ W, int n_out, int nb, const uint8_t* __restrict__ xq,
    float* __restrict__ y, int32_t* __restrict__ sums) {
  constexpr int kWB = Q5 ? kQ5_1Bytes : kQ4_1Bytes;
  constexpr int kQs = Q5 ? 8 : 4;  // offset of the 16 nibble bytes
  extern __shared__ __align__(16) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * NW + wave_id();
  const bool row_ok = row < n_out;
  const size_t rb = static_cast<size_t>(nb) * kWB;
  const uint8_t* wrow = W + static_cast<size_t>(row_ok ? row : n_out - 1) * rb;
  const int passes = (nb + 63) >> 6;

  uint4 QS[UNR];
  uint32_t DM[UNR], QH[UNR];
  auto issue = [&](int p0) {
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
      const int b = min((p0 + j) * 64 + lane, nb - 1);
      const uint8_t* p = wrow + static_cast<uint32_t>(b * kWB);
      DM[j] = load_a4<uint32_t>(p);
      if constexpr (Q5) QH[j] = load_a4<uint32_t>(p + 4);
      QS[j] = load_a4<uint4>(p + kQs);
    }
  };
  const LayoutQ81 L(nb);
  StagedQ81 st;
  stage_load_q81<NW * 64>(st, xq, nb);
  sched_fence();
  issue(0);
  sched_fence();
  stage_place_q81<NW * 64>(lds, L, st, xq, nb);
  __syncthreads();

  const float* dA = reinterpret_cast<const float*>(lds + L.off_d);
  const float* sA = reinterpret_cast<const float*>(lds + L.off_s);
  float acc = 0.0f;
  for (int p0 = 0; p0 < passes; p0 += UNR) {
    if (p0 > 0) issue(p0);
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
      const int b = (p0 + j) * 64 + lane;
      if (!row_ok || b >= nb) continue;
      const uint4 a0 = *reinterpret_cast<const uint4*>(lds + b * LayoutQ81::kStride);       // elements 0-15
      const uint4 a1 = *reinterpret_cast<const uint4*>(lds + b * LayoutQ81::kStride + 16);  // 16-31
      const uint4 q = QS[j];
      uint32_t lo[4] = {q.x & kLo4, q.y & kLo4, q.z & kLo4, q.w & kLo4};
      uint32_t hi[4] = {(q.x >> 4) & kLo4, (q.y >> 4) & kLo4, (q.z >> 4) & kLo4, (q.w >> 4) & kLo4};
      if constexpr (Q5) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          lo[k] = q5_codes(lo[k], QH[j], 4 * k);
          hi[k] = q5_codes(hi[k], QH[j], 16 + 4 * k);
        }
      }
      int sv = 0;  // codes are at most 31: the signed byte dot is exact
      sv = dot4(lo[0], a0.x, sv);
      sv = dot4(lo[1], a0.y, sv);
      sv = dot4(lo[2], a0.z, sv);
      sv = dot4(lo[3], a0.w, sv);
      sv = dot4(hi[0], a1.x, sv);
      sv = dot4(hi[1], a1.y, sv);
      sv = dot4(hi[2], a1.z, sv);
      sv = dot4(hi[3], a1.w, sv);
      const float dw = f16_to_f32(DM[j] & 0xFFFFu), mw = f16_to_f32(DM[j] >> 16);
      acc += static_cast<float>(sv) * (dw * dA[b]) + mw * sA[b];
      if constexpr (SUMS) sums[static_cast<size_t>(row) * nb + b] = sv;
    }
  }
  if (row_ok) {
    const float total = wave_sum(acc);
    if (lane == 0 && y != nullptr) y[row] = total;
  }
}

// ---------------------------------------------------------------------------
// Q8_0, Q4_0 and Q5_0 x Q8_0 for NC = 2..4 activation columns: the LDS kernels
// above with the NC Q8_0 rows staged one after another (LayoutQ80 regions
// `L.bytes` apart) and each weight block loaded once.  The lane turns its block's
// codes into signed bytes once (Q4_0 / Q5_0: the stored value + bias minus the
// bias, per byte without borrows since every byte is at least 0x80 after the OR),
// then takes 8 dot4 per column: s = sum (q - bias) a, the same integer as the
// one-column kernels' sum q a - bias sum a.  FMT: 0 Q8_0, 1 Q4_0, 2 Q5_0.
template <int NW, int UNR, int NC, int FMT, bool SUMS>
__global__ __launch_bounds__(NW * 64) void gemv_q80_cols(
    const uint8_t* __restrict__ W, int n_out, int nb, const uint8_t* __restrict__ xq,
    float* __restrict__ y, int32_t* __restrict__ sums) {
  constexpr int kWB = FMT == 0 ? kQ8_0Bytes : FMT == 1 ? kQ4_0Bytes : kQ5_0Bytes;
  constexpr int kQs = FMT == 2 ? 6 : 2;             // offset of the code bytes
  constexpr uint32_t kBias4 = FMT == 2 ? 0x10101010u : 0x08080808u;
  constexpr int kN = FMT == 0 ? 8 : 4;              // dwords of code bytes
  extern __shared__ __align__(16) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * NW + wave_id();
  const bool row_ok = row < n_out;
  const size_t rb = static_cast<size_t>(nb) * kWB;
  const uint8_t* wrow = W + static_cast<size_t>(row_ok ? row : n_out - 1) * rb;
  const int passes = (nb + 63) >> 6;
  const int xrow = nb * kQ8_0Bytes;

  ShiftedField<kN> QS[UNR];
  uint32_t D[UNR], QH[UNR];
  auto issue = [&](int p0) {
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
      const int b = min((p0 + j) * 64 + lane, nb - 1);
      const uint8_t* p = wrow + static_cast<uint32_t>(b * kWB);
      D[j] = *reinterpret_cast<const uint16_t*>(p);
      if constexpr (FMT == 2) QH[j] = load_u2<uint32_t>(p + 2);
      QS[j] = load_field<kN>(p + kQs);
    }
  };
  const LayoutQ80 L(nb);
  StagedQ80 st;
  stage_load_q80<NW * 64>(st, xq, nb);
  sched_fence();
  issue(0);
  sched_fence();
  stage_place_q80<NW * 64>(lds, L, st, xq, nb);
#pragma unroll
  for (int col = 1; col < NC; ++col) {
    const uint8_t* xc = xq + static_cast<uint32_t>(col * xrow);
    StagedQ80 sc;
    stage_load_q80<NW * 64>(sc, xc, nb);
    stage_place_q80<NW * 64>(lds + col * L.bytes, L, sc, xc, nb);
  }
  __syncthreads();

  float acc[NC];
#pragma unroll
  for (int col = 0; col < NC; ++col) acc[col] = 0.0f;
  for (int p0 = 0; p0 < passes; p0 += UNR) {
    if (p0 > 0) issue(p0);
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
      const int b = (p0 + j) * 64 + lane;
      if (!row_ok || b >= nb) continue;
      uint32_t q[8];  // signed codes of elements 4i .. 4i+3
      if constexpr (FMT == 0) {
        align_field(QS[j], q);
      } else {
        uint32_t w[4];
        align_field(QS[j], w);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint32_t lo = w[k] & kLo4, hi = (w[k] >> 4) & kLo4;
          if constexpr (FMT == 2) {
            lo = q5_codes(lo, QH[j], 4 * k);
            hi = q5_codes(hi, QH[j], 16 + 4 * k);
          }
          q[k] = ((lo | 0x80808080u) - kBias4) ^ 0x80808080u;
          q[4 + k] = ((hi | 0x80808080u) - kBias4) ^ 0x80808080u;
        }
      }
      const float d = f16_to_f32(D[j]);
#pragma unroll
      for (int col = 0; col < NC; ++col) {
        const uint8_t* base = lds + col * L.bytes;
        const uint4 a0 = *reinterpret_cast<const uint4*>(base + b * LayoutQ80::kStride);
        const uint4 a1 = *reinterpret_cast<const uint4*>(base + b * LayoutQ80::kStride + 16);
        const float dx = reinterpret_cast<const float*>(base + L.off_d)[b];
        int sv = 0;
        sv = dot4(q[0], a0.x, sv);
        sv = dot4(q[1], a0.y, sv);
        sv = dot4(q[2], a0.z, sv);
        sv = dot4(q[3], a0.w, sv);
        sv = dot4(q[4], a1.x, sv);
        sv = dot4(q[5], a1.y, sv);
        sv = dot4(q[6], a1.z, sv);
        sv = dot4(q[7], a1.w, sv);
        acc[col] += static_cast<float>(sv) * (d * dx);
        if constexpr (SUMS) sums[(static_cast<size_t>(col) * n_out + row) * nb + b] = sv;
      }
    }
  }
  if (row_ok) {
#pragma unroll
    for (int col = 0; col < NC; ++col) {
      const float total = wave_sum(acc[col]);
      if (lane == 0 && y != nullptr) y[static_cast<size_t>(col) * n_out + row] = total;
    }
  }
}

// ---------------------------------------------------------------------------
// Register-resident activations.  Each lane loads, once per wavefront, the
// activation codes, sums and scale of the blocks it covers in every pass of a
// row, then the wavefront walks its rows (RPW at a time, strided by the grid)
// reusing those registers: no LDS, no workgroup barrier.
template <int NW, int NP, int RPW, bool SUMS, int Q5 = 0>
__global__ __launch_bounds__(NW * 64) void gemv_q4_K_reg(
    const uint8_t* __restrict__ W, int n_out, int nb, const uint8_t* __restrict__ xq,
    float* __restrict__ y, int32_t* __restrict__ sums) {
  const int lane = threadIdx.x & 63;
  const int c = lane & 3, u = lane >> 2;
  const uint32_t hi_mask = (c & 2) ? 0xFFFFFFFFu : 0u;
  const int sh = (c & 1) * 16;
  const int wave = blockIdx.x * NW + wave_id();
  const int nwaves = gridDim.x * NW;
  using F = KQuant4<Q5>;
  const size_t rb = static_cast<size_t>(nb) * F::kBytes;

  uint4 A[NP][4];
  int2 S2[NP];
  float DX[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const uint8_t* a = xq + static_cast<uint32_t>(min(p * 16 + u, nb - 1) * kQ8_KBytes);
    DX[p] = *reinterpret_cast<const float*>(a);
#pragma unroll
    for (int i = 0; i < 4; ++i) A[p][i] = load_a4<uint4>(a + 4 + 64 * c + 16 * i);
    const uint2 bs = load_a4<uint2>(a + 260 + 8 * c);
    S2[p] = make_int2(sext16_lo(bs.x) + sext16_hi(bs.x), sext16_lo(bs.y) + sext16_hi(bs.y));
  }

  for (int r0 = wave * RPW; r0 < n_out; r0 += nwaves * RPW) {
    uint4 H[RPW][NP], Q0[RPW][NP], Q1[RPW][NP], QH0[RPW][Q5 ? NP : 1], QH1[RPW][Q5 ? NP : 1];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const uint8_t* wrow = W + static_cast<size_t>(min(r0 + r, n_out - 1)) * rb;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const uint8_t* q = wrow + static_cast<uint32_t>(min(p * 16 + u, nb - 1) * F::kBytes);
        H[r][p] = *reinterpret_cast<const uint4*>(q);
        Q0[r][p] = *reinterpret_cast<const uint4*>(q + F::kQs + 32 * c);
        Q1[r][p] = *reinterpret_cast<const uint4*>(q + F::kQs + 16 + 32 * c);
        if constexpr (Q5 != 0) {
          QH0[r][p] = *reinterpret_cast<const uint4*>(q + 16);
          QH1[r][p] = *reinterpret_cast<const uint4*>(q + 32);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int row = r0 + r;
      if (row >= n_out) break;  // uniform over the wavefront
      float acc = 0.0f;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int sb = p * 16 + u;
        if (sb >= nb) continue;  // uniform over the 4 lanes of a superblock
        int2 part;
        if constexpr (Q5 != 0) {
          part = q5K_chunk(Q0[r][p], Q1[r][p], rot_q5(QH0[r][p], c), rot_q5(QH1[r][p], c), H[r][p],
                           A[p][0], A[p][1], A[p][2], A[p][3], S2[p], hi_mask, sh);
        } else {
          part = q4K_chunk(Q0[r][p], Q1[r][p], H[r][p], A[p][0], A[p][1], A[p][2], A[p][3], S2[p], hi_mask,
                           sh);
        }
        const int sq = quad_sum(part.x);
        const int sm = quad_sum(part.y);
        const uint32_t dd = H[r][p].x;
        const float cb = (DX[p] * f16_to_f32(dd & 0xFFFF)) * static_cast<float>(sq) -
                         (DX[p] * f16_to_f32(dd >> 16)) * static_cast<float>(sm);
        acc += (c == 0) ? cb : 0.0f;
        if (c == 0) {
          if constexpr (SUMS) {
            int32_t* o = sums + (static_cast<size_t>(row) * nb + sb) * 2;
            o[0] = sq;
            o[1] = sm;
          }
        }
      }
      const float total = wave_sum(acc);
      if (lane == 0 && y != nullptr) y[row] = total;
    }
  }
}

// ---------------------------------------------------------------------------
// Two Q4_K matrices (or, with the Q5 flag, two Q5_K matrices) over one activation
// row: the gate and up projections of an FFN layer.  The wavefront that owns row r
// computes it in both W1 and W2 from
// the same activation operands (candle formats page, "实测：一次点积": vec_dot_4
// takes one activation row against four weight rows with the activation loaded
// once; here one row of each matrix), then writes y1[r] and y2[r], or the gated activation
// silu(y1[r]) * y2[r] = y1 / (1 + e^-y1) * y2 that the down projection consumes.
// blockIdx.y is the activation column.
constexpr int kEpiPair = 0, kEpiSwiglu = 1;

template <int EPI>
__device__ __forceinline__ void pair_out(float* out, int n_out, int row, float g, float u) {
  if constexpr (EPI == kEpiSwiglu) {
    out[row] = g / (1.0f + expf(-g)) * u;
  } else {
    out[row] = g;
    out[n_out + row] = u;
  }
}

// Rows of one or two passes: activations in registers (as gemv_q4_K_reg), rows
// grid-strided.
template <int NW, int NP, int EPI, int Q5 = 0>
__global__ __launch_bounds__(NW * 64) void gemv_q4_K_pair_reg(
    const uint8_t* __restrict__ W1, const uint8_t* __restrict__ W2, int n_out, int nb,
    const uint8_t* __restrict__ xq, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int c = lane & 3, u = lane >> 2;
  const uint32_t hi_mask = (c & 2) ? 0xFFFFFFFFu : 0u;
  const int sh = (c & 1) * 16;
  const int wave = blockIdx.x * NW + wave_id();
  const int nwaves = gridDim.x * NW;
  using F = KQuant4<Q5>;
  const size_t rb = static_cast<size_t>(nb) * F::kBytes;
  xq += static_cast<size_t>(blockIdx.y) * nb * kQ8_KBytes;
  out += static_cast<size_t>(blockIdx.y) * (EPI == kEpiSwiglu ? 1 : 2) * n_out;

  uint4 A[NP][4];
  int2 S2[NP];
  float DX[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const uint8_t* a = xq + static_cast<uint32_t>(min(p * 16 + u, nb - 1) * kQ8_KBytes);
    DX[p] = *reinterpret_cast<const float*>(a);
#pragma unroll
    for (int i = 0; i < 4; ++i) A[p][i] = load_a4<uint4>(a + 4 + 64 * c + 16 * i);
    const uint2 bs = load_a4<uint2>(a + 260 + 8 * c);
    S2[p] = make_int2(sext16_lo(bs.x) + sext16_hi(bs.x), sext16_lo(bs.y) + sext16_hi(bs.y));
  }

  for (int row = wave; row < n_out; row += nwaves) {
    uint4 H[2][NP], Q0[2][NP], Q1[2][NP], QH0[2][Q5 ? NP : 1], QH1[2][Q5 ? NP : 1];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint8_t* wrow = (m ? W2 : W1) + static_cast<size_t>(row) * rb;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const uint8_t* q = wrow + static_cast<uint32_t>(min(p * 16 + u, nb - 1) * F::kBytes);
        H[m][p] = *reinterpret_cast<const uint4*>(q);
        Q0[m][p] = *reinterpret_cast<const uint4*>(q + F::kQs + 32 * c);
        Q1[m][p] = *reinterpret_cast<const uint4*>(q + F::kQs + 16 + 32 * c);
        if constexpr (Q5 != 0) {
          QH0[m][p] = *reinterpret_cast<const uint4*>(q + 16);
          QH1[m][p] = *reinterpret_cast<const uint4*>(q + 32);
        }
      }
    }
    float acc[2] = {0.0f, 0.0f};
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        if (p * 16 + u >= nb) continue;  // uniform over the 4 lanes of a superblock
        int2 part;
        if constexpr (Q5 != 0) {
          part = q5K_chunk(Q0[m][p], Q1[m][p], rot_q5(QH0[m][p], c), rot_q5(QH1[m][p], c), H[m][p],
                           A[p][0], A[p][1], A[p][2], A[p][3], S2[p], hi_mask, sh);
        } else {
          part = q4K_chunk(Q0[m][p], Q1[m][p], H[m][p], A[p][0], A[p][1], A[p][2], A[p][3], S2[p], hi_mask,
                           sh);
        }
        const int sq = quad_sum(part.x);
        const int sm = quad_sum(part.y);
        const uint32_t dd = H[m][p].x;
        const float cb = (DX[p] * f16_to_f32(dd & 0xFFFF)) * static_cast<float>(sq) -
                         (DX[p] * f16_to_f32(dd >> 16)) * static_cast<float>(sm);
        acc[m] += (c == 0) ? cb : 0.0f;
      }
    }
    const float g = wave_sum(acc[0]);
    const float v = wave_sum(acc[1]);
    if (lane == 0) pair_out<EPI>(out, n_out, row, g, v);
  }
}

// Longer rows: the activation row staged in LDS once per workgroup (as
// gemv_q4_K_kernel), one row of each matrix per wavefront.
template <int NW, int UNR, int EPI, int Q5 = 0>
__global__ __launch_bounds__(NW * 64) void gemv_q4_K_pair_kernel(
    const uint8_t* __restrict__ W1, const uint8_t* __restrict__ W2, int n_out, int nb,
    const uint8_t* __restrict__ xq, float* __restrict__ out) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * NW + wave_id();
  const int c = lane & 3, u = lane >> 2;
  const bool row_ok = row < n_out;
  using F = KQuant4<Q5>;
  const size_t rb = static_cast<size_t>(nb) * F::kBytes;
  const size_t roff = static_cast<size_t>(row_ok ? row : n_out - 1) * rb;
  const int passes = (nb + 15) >> 4;
  xq += static_cast<size_t>(blockIdx.y) * nb * kQ8_KBytes;
  out += static_cast<size_t>(blockIdx.y) * (EPI == kEpiSwiglu ? 1 : 2) * n_out;

  uint4 H[2][UNR], Q0[2][UNR], Q1[2][UNR], QH0[2][Q5 ? UNR : 1], QH1[2][Q5 ? UNR : 1];
  auto issue = [&](int p0) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint8_t* wrow = (m ? W2 : W1) + roff;
#pragma unroll
      for (int j = 0; j < UNR; ++j) {
        const int sb = min((p0 + j) * 16 + u, nb - 1);
        const uint8_t* p = wrow + static_cast<uint32_t>(sb * F::kBytes);
        H[m][j] = *reinterpret_cast<const uint4*>(p);
        Q0[m][j] = *reinterpret_cast<const uint4*>(p + F::kQs + 32 * c);
        Q1[m][j] = *reinterpret_cast<const uint4*>(p + F::kQs + 16 + 32 * c);
        if constexpr (Q5 != 0) {
          QH0[m][j] = *reinterpret_cast<const uint4*>(p + 16);
          QH1[m][j] = *reinterpret_cast<const uint4*>(p + 32);
        }
      }
    }
  };
  ImageQ8K st;
  image_load_q8K<NW * 64>(st, xq, nb);
  sched_fence();
  issue(0);
  sched_fence();
  image_place_q8K<NW * 64>(lds, st, xq, nb);
  __syncthreads();

  const int sh = (c & 1) * 16;
  const uint32_t hi_mask = (c & 2) ? 0xFFFFFFFFu : 0u;
  float acc[2] = {0.0f, 0.0f};
  for (int p0 = 0; p0 < passes; p0 += UNR) {
    if (p0 > 0) issue(p0);
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
      const int sb = (p0 + j) * 16 + u;
      if (!row_ok || sb >= nb) continue;  // uniform over the 4 lanes of a superblock
      const uint8_t* blk = lds + sb * kQ8_KBytes;
      const uint8_t* ap = blk + 4 + 64 * c;
      const uint4 a0 = lds_a4<uint4>(ap);
      const uint4 a1 = lds_a4<uint4>(ap + 16);
      const uint4 a2 = lds_a4<uint4>(ap + 32);
      const uint4 a3 = lds_a4<uint4>(ap + 48);
      const uint2 bsw = lds_a4<uint2>(blk + 260 + 8 * c);
      const int2 asum = make_int2(sext16_lo(bsw.x) + sext16_hi(bsw.x), sext16_lo(bsw.y) + sext16_hi(bsw.y));
      const float dx = lds_a4<float>(blk);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const uint4 h = H[m][j];
        int2 part;
        if constexpr (Q5 != 0) {
          part = q5K_chunk(Q0[m][j], Q1[m][j], rot_q5(QH0[m][j], c), rot_q5(QH1[m][j], c), h, a0, a1, a2,
                           a3, asum, hi_mask, sh);
        } else {
          part = q4K_chunk(Q0[m][j], Q1[m][j], h, a0, a1, a2, a3, asum, hi_mask, sh);
        }
        const int sq = quad_sum(part.x);
        const int sm = quad_sum(part.y);
        const float cb = (dx * f16_to_f32(h.x & 0xFFFF)) * static_cast<float>(sq) -
                         (dx * f16_to_f32(h.x >> 16)) * static_cast<float>(sm);
        acc[m] += (c == 0) ? cb : 0.0f;
      }
    }
  }
  if (row_ok) {
    const float g = wave_sum(acc[0]);
    const float v = wave_sum(acc[1]);
    if (lane == 0) pair_out<EPI>(out, n_out, row, g, v);
  }
}

// Q6_K x Q8_K, register-resident activations.  Lane (u, p = h*2 + k) of pass P
// covers l in [16k, 16k+16) of half h of superblock P*16 + u for the four groups
// g: activation pieces 8h + 2g + k, 16-element sub-blocks 8h + 2g + k.
template <int NW, int NP, bool SUMS>
__global__ __launch_bounds__(NW * 64) void gemv_q6_K_reg(
    const uint8_t* __restrict__ W, int n_out, int nb, const uint8_t* __restrict__ xq,
    float* __restrict__ y, int32_t* __restrict__ sums) {
  const int lane = threadIdx.x & 63;
  const int pos = lane & 3, u = lane >> 2;
  const int hh = pos >> 1, kk = pos & 1;
  const int wave = blockIdx.x * NW + wave_id();
  const int nwaves = gridDim.x * NW;
  const size_t rb = static_cast<size_t>(nb) * kQ6_KBytes;

  uint4 A[NP][4];
  int4 BS[NP];  // 32 * bsum of sub-blocks 8h + 2g + k, g = 0..3
  float DX[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const uint8_t* a = xq + static_cast<uint32_t>(min(p * 16 + u, nb - 1) * kQ8_KBytes);
    DX[p] = *reinterpret_cast<const float*>(a);
#pragma unroll
    for (int g = 0; g < 4; ++g) A[p][g] = load_a4<uint4>(a + 4 + 128 * hh + 32 * g + 16 * kk);
    const uint4 b = load_a4<uint4>(a + 260 + 16 * hh);  // bsums 8h .. 8h+7
    const uint32_t w[4] = {b.x, b.y, b.z, b.w};
    int v[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) v[g] = 32 * (kk ? sext16_hi(w[g]) : sext16_lo(w[g]));
    BS[p] = make_int4(v[0], v[1], v[2], v[3]);
  }

  for (int row = wave; row < n_out; row += nwaves) {
    const uint8_t* wrow = W + static_cast<size_t>(row) * rb;
    uint4 QA[NP], QB[NP], QH[NP];
    uint2 SC[NP];
    uint32_t D[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const uint8_t* q = wrow + static_cast<uint32_t>(min(p * 16 + u, nb - 1) * kQ6_KBytes);
      QA[p] = load_u2<uint4>(q + 64 * hh + 16 * kk);
      QB[p] = load_u2<uint4>(q + 64 * hh + 32 + 16 * kk);
      QH[p] = load_u2<uint4>(q + 128 + 32 * hh + 16 * kk);
      SC[p] = load_u2<uint2>(q + 192 + 8 * hh);
      D[p] = *reinterpret_cast<const uint16_t*>(q + 208);
    }
    float acc = 0.0f;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int sb = p * 16 + u;
      if (sb >= nb) continue;
      const uint32_t al[4] = {QA[p].x, QA[p].y, QA[p].z, QA[p].w};
      const uint32_t bl[4] = {QB[p].x, QB[p].y, QB[p].z, QB[p].w};
      const uint32_t hl[4] = {QH[p].x, QH[p].y, QH[p].z, QH[p].w};
      int s0 = 0, s1 = 0, s2 = 0, s3 = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t a0 = i == 0 ? A[p][0].x : i == 1 ? A[p][0].y : i == 2 ? A[p][0].z : A[p][0].w;
        const uint32_t a1 = i == 0 ? A[p][1].x : i == 1 ? A[p][1].y : i == 2 ? A[p][1].z : A[p][1].w;
        const uint32_t a2 = i == 0 ? A[p][2].x : i == 1 ? A[p][2].y : i == 2 ? A[p][2].z : A[p][2].w;
        const uint32_t a3 = i == 0 ? A[p][3].x : i == 1 ? A[p][3].y : i == 2 ? A[p][3].z : A[p][3].w;
        const Q6Codes q = q6_codes(al[i], bl[i], hl[i]);
        s0 = dot4(q.q0, a0, s0);
        s1 = dot4(q.q1, a1, s1);
        s2 = dot4(q.q2, a2, s2);
        s3 = dot4(q.q3, a3, s3);
      }
      const int sc0 = static_cast<int8_t>((SC[p].x >> (8 * kk)) & 0xFF);
      const int sc1 = static_cast<int8_t>((SC[p].x >> (16 + 8 * kk)) & 0xFF);
      const int sc2 = static_cast<int8_t>((SC[p].y >> (8 * kk)) & 0xFF);
      const int sc3 = static_cast<int8_t>((SC[p].y >> (16 + 8 * kk)) & 0xFF);
      const int part = mad24(sc0, s0 - BS[p].x, mad24(sc1, s1 - BS[p].y,
                             mad24(sc2, s2 - BS[p].z, __mul24(sc3, s3 - BS[p].w))));
      const int S = quad_sum(part);
      const float cb = (DX[p] * f16_to_f32(D[p])) * static_cast<float>(S);
      acc += (pos == 0) ? cb : 0.0f;
      if constexpr (SUMS) {
        if (pos == 0) sums[static_cast<size_t>(row) * nb + sb] = S;
      }
    }
    const float total = wave_sum(acc);
    if (lane == 0 && y != nullptr) y[row] = total;
  }
}

// Q8_0 x Q8_0 and Q4_0 x Q8_0, register-resident activations: lane b of pass P
// holds the 32 codes, d and (for Q4_0) the code sum of activation block P*64 + b.
constexpr int kFmtQ8_0 = 0, kFmtQ4_0 = 1, kFmtQ5_0 = 2;

template <int NW, int NP, int FMT, bool SUMS>
__global__ __launch_bounds__(NW * 64) void gemv_q80_reg(
    const uint8_t* __restrict__ W, int n_out, int nb, const uint8_t* __restrict__ xq,
    float* __restrict__ y, int32_t* __restrict__ sums) {
  constexpr bool Q4 = FMT != kFmtQ8_0;  // nibble formats (Q4_0, Q5_0)
  constexpr bool Q5 = FMT == kFmtQ5_0;
  constexpr int kWB = (FMT == kFmtQ4_0) ? kQ4_0Bytes : Q5 ? kQ5_0Bytes : kQ8_0Bytes;
  constexpr int kQs = Q5 ? 6 : 2;
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * NW + wave_id();
  const int nwaves = gridDim.x * NW;
  const size_t rb = static_cast<size_t>(nb) * kWB;

  uint4 A0[NP], A1[NP];
  float DX[NP];
  int ASUM[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const uint8_t* a = xq + static_cast<uint32_t>(min(p * 64 + lane, nb - 1) * kQ8_0Bytes);
    DX[p] = f16_to_f32(*reinterpret_cast<const uint16_t*>(a));
    A0[p] = load_u2<uint4>(a + 2);
    A1[p] = load_u2<uint4>(a + 18);
    int sa = 0;
    if constexpr (Q4) {
      sa = dot4(kOnes, A0[p].x, sa);
      sa = dot4(kOnes, A0[p].y, sa);
      sa = dot4(kOnes, A0[p].z, sa);
      sa = dot4(kOnes, A0[p].w, sa);
      sa = dot4(kOnes, A1[p].x, sa);
      sa = dot4(kOnes, A1[p].y, sa);
      sa = dot4(kOnes, A1[p].z, sa);
      sa = dot4(kOnes, A1[p].w, sa);
    }
    ASUM[p] = (Q5 ? 16 : 8) * sa;  // codes are stored as value + bias
  }

  for (int row = wave; row < n_out; row += nwaves) {
    const uint8_t* wrow = W + static_cast<size_t>(row) * rb;
    uint4 Q0[NP], Q1[NP];
    uint32_t D[NP], QH[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const uint8_t* q = wrow + static_cast<uint32_t>(min(p * 64 + lane, nb - 1) * kWB);
      D[p] = *reinterpret_cast<const uint16_t*>(q);
      if constexpr (Q5) QH[p] = load_u2<uint32_t>(q + 2);
      Q0[p] = load_u2<uint4>(q + kQs);
      if constexpr (!Q4) Q1[p] = load_u2<uint4>(q + 18);
    }
    float acc = 0.0f;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int b = p * 64 + lane;
      if (b >= nb) continue;
      int s = 0;
      if constexpr (Q4) {
        const uint4 q = Q0[p];
        uint32_t lo[4] = {q.x & kLo4, q.y & kLo4, q.z & kLo4, q.w & kLo4};
        uint32_t hi[4] = {(q.x >> 4) & kLo4, (q.y >> 4) & kLo4, (q.z >> 4) & kLo4, (q.w >> 4) & kLo4};
        if constexpr (Q5) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            lo[k] = q5_codes(lo[k], QH[p], 4 * k);
            hi[k] = q5_codes(hi[k], QH[p], 16 + 4 * k);
          }
        }
        s = dot4(lo[0], A0[p].x, s);
        s = dot4(lo[1], A0[p].y, s);
        s = dot4(lo[2], A0[p].z, s);
        s = dot4(lo[3], A0[p].w, s);
        s = dot4(hi[0], A1[p].x, s);
        s = dot4(hi[1], A1[p].y, s);
        s = dot4(hi[2], A1[p].z, s);
        s = dot4(hi[3], A1[p].w, s);
        s -= ASUM[p];  // codes are stored as value + bias
      } else {
        s = dot4(Q0[p].x, A0[p].x, s);
        s = dot4(Q0[p].y, A0[p].y, s);
        s = dot4(Q0[p].z, A0[p].z, s);
        s = dot4(Q0[p].w, A0[p].w, s);
        s = dot4(Q1[p].x, A1[p].x, s);
        s = dot4(Q1[p].y, A1[p].y, s);
        s = dot4(Q1[p].z, A1[p].z, s);
        s = dot4(Q1[p].w, A1[p].w, s);
      }
      acc += static_cast<float>(s) * (f16_to_f32(D[p]) * DX[p]);
      if constexpr (SUMS) sums[static_cast<size_t>(row) * nb + b] = s;
    }
    const float total = wave_sum(acc);
    if (lane == 0 && y != nullptr) y[row] = total;
  }
}

// Dynamic LDS above 64 KB has to be allowed for the kernel on the current device;
// set on every such launch (the library keeps no per-device state).
template <typename K>
hipError_t allow_lds(K kernel, int64_t lds_bytes) {
  if (lds_bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             static_cast<int>(lds_bytes));
}

template <int NW, typename K>
hipError_t launch(K kernel, int64_t n_out, int64_t lds_bytes, hipStream_t s, hipEvent_t e0,
                  hipEvent_t e1, const uint8_t* W, int nb, const uint8_t* xq, float* y,
                  int32_t* sums) {
  unsigned grid = 0;
  if (!launch_grid((n_out + NW - 1) / NW, NW * 64, &grid)) return hipErrorInvalidConfiguration;
  const hipError_t attr = allow_lds(kernel, lds_bytes);
  if (attr != hipSuccess) return attr;
  const int n = static_cast<int>(n_out);
  if (e0 != nullptr || e1 != nullptr) {
    hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(NW * 64), static_cast<uint32_t>(lds_bytes),
                          s, e0, e1, 0, W, n, nb, xq, y, sums);
  } else {
    kernel<<<grid, NW * 64, lds_bytes, s>>>(W, n, nb, xq, y, sums);
  }
  return hipGetLastError();
}

template <int NW, typename K>
hipError_t launch_rows(K kernel, int64_t n_out, int rpw, int max_waves, hipStream_t s,
                       hipEvent_t e0, hipEvent_t e1, const uint8_t* W, int nb, const uint8_t* xq,
                       float* y, int32_t* sums) {
  const int64_t groups = (n_out + rpw - 1) / rpw;
  const int64_t waves = groups < max_waves ? groups : max_waves;
  unsigned grid = 0;
  if (!launch_grid((waves + NW - 1) / NW, NW * 64, &grid)) return hipErrorInvalidConfiguration;
  const int n = static_cast<int>(n_out);
  if (e0 != nullptr || e1 != nullptr) {
    hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(NW * 64), 0, s, e0, e1, 0, W, n, nb, xq, y, sums);
  } else {
    kernel<<<grid, NW * 64, 0, s>>>(W, n, nb, xq, y, sums);
  }
  return hipGetLastError();
}

}  // namespace

int64_t gemv_lds_bytes(int w_type, int64_t n_in) {
  switch (w_type) {
    case kQ2_K:
    case kQ3_K:
    case kQ4_K:
    case kQ5_K:
    case kQ6_K: return align16(n_in / 256 * kQ8_KBytes);
    case kQ8_0:
    case kQ4_0:
    case kQ5_0: return LayoutQ80(n_in / 32).bytes;
    case kQ4_1:
    case kQ5_1: return LayoutQ81(n_in / 32).bytes;
    default: return -1;
  }
}

// Wavefronts (rows) per workgroup of the LDS-staged GEMV launches: 4 for the
// K-quant and _1 kernels (8 and 2 were slower on every 4096 x 11008 shape, e.g. Q4_K
// decode, Q5_K 7.69 / 9.32 against 7.20 us), 8 for the Q8_0 / Q4_0 / Q5_0 kernels,
// whose staging (the per-block layout and, for Q4_0 / Q5_0, the activation sums) is
// then shared by twice the rows: Q4_0 4096 x 11008 8.43 -> 8.03 us, 8192 x 8192
// 11.12 -> 10.1, 14336 x 4096 11.08 -> 10.18, Q8_0 4096 x 11008 11.02 -> 10.69, Q5_0
// 14336 x 4096 12.71 -> 11.99, 4096 x 4096 Q4_0 4.60 -> 4.43.  The same holds for their
// multi-column kernel (Q4_0 4096 x 11008 at 3 columns 15.4 -> 12.8 us, at 2 11.6 -> 10.6,
// Q8_0 4096 x 4096 at 4 columns 9.4 -> 8.7), while the K-quant multi-column kernels were
// slower with 8 (Q4_K 4096 x 11008 at 2 columns 8.42 -> 9.0, Q6_K 12.1 -> 13.1).
constexpr int kWaves = 4;
constexpr int kWaves32 = 8;

// Compute units of the current device (256 on MI355X), queried once per device.
int cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);  // threads that race here store the same value
  }
  return n;
}

// The register-resident kernels walk the rows with a grid of exactly three
// 4-wavefront workgroups per compute unit (3072 wavefronts on MI355X).  Measured
// on the 32000 x 4096 Q6_K output head (launch-recorded events): 18.9 us at three
// workgroups per CU and at two, 21.4 at four, 20.6 at six, 29.4 at one; counts
// that do not divide evenly over the CUs were slow (2.5 per CU 21.7, 1.5 per CU
// 23.4).  On 11008 x 4096 Q4_K: 5.65-5.74 us at three per CU, 5.74-6.01 at four,
// 6.5-6.6 at two.
int max_row_waves() { return 3 * 4 * cu_count(); }

bool gemv_cols_fits(int w_type, int64_t n_in, int64_t ncols) {
  if (ncols < 2 || ncols > kGemvMaxCols) return false;
  if (w_type == kQ8_0 || w_type == kQ4_0 || w_type == kQ5_0) return ncols * LayoutQ80(n_in / 32).bytes <= kColsLdsBytes;
  if (w_type != kQ4_K && w_type != kQ5_K && w_type != kQ6_K) return false;
  return ncols * align16(n_in / 256 * kQ8_KBytes) <= kColsLdsBytes;
}

namespace {
// FMT: 0 Q8_0, 1 Q4_0, 2 Q5_0.
template <int NC, bool S, int FMT>
hipError_t launch_q80_cols_nc(const uint8_t* W, int64_t n_out, int nb, const uint8_t* xq, float* y,
                              int32_t* sums, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const int64_t lds = NC * LayoutQ80(nb).bytes;
  const int passes = (nb + 63) / 64;
  if (passes == 1) return launch<kWaves32>(gemv_q80_cols<kWaves32, 1, NC, FMT, S>, n_out, lds, s, e0, e1, W, nb, xq, y, sums);
  if (passes == 2) return launch<kWaves32>(gemv_q80_cols<kWaves32, 2, NC, FMT, S>, n_out, lds, s, e0, e1, W, nb, xq, y, sums);
  return launch<kWaves32>(gemv_q80_cols<kWaves32, 4, NC, FMT, S>, n_out, lds, s, e0, e1, W, nb, xq, y, sums);
}
template <bool S, int FMT>
hipError_t launch_q80_cols_s(const uint8_t* W, int64_t n_out, int nb, const uint8_t* xq, int64_t ncols, float* y,
                             int32_t* sums, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (ncols == 2) return launch_q80_cols_nc<2, S, FMT>(W, n_out, nb, xq, y, sums, s, e0, e1);
  if (ncols == 3) return launch_q80_cols_nc<3, S, FMT>(W, n_out, nb, xq, y, sums, s, e0, e1);
  return launch_q80_cols_nc<4, S, FMT>(W, n_out, nb, xq, y, sums, s, e0, e1);
}

// FMT: 0 Q4_K, 1 Q5_K, 2 Q6_K.
template <int NC, bool S, int FMT>
hipError_t launch_cols_nc(const uint8_t* W, int64_t n_out, int nb, const uint8_t* xq, float* y, int32_t* sums,
                          hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const int64_t lds = NC * align16(static_cast<int64_t>(nb) * kQ8_KBytes);
  const int passes = (nb + 15) / 16;
  if constexpr (FMT == 2) {
    if (passes == 1) return launch<kWaves>(gemv_q6_K_cols<kWaves, 1, NC, S>, n_out, lds, s, e0, e1, W, nb, xq, y, sums);
    if (passes == 2) return launch<kWaves>(gemv_q6_K_cols<kWaves, 2, NC, S>, n_out, lds, s, e0, e1, W, nb, xq, y, sums);
    return launch<kWaves>(gemv_q6_K_cols<kWaves, 3, NC, S>, n_out, lds, s, e0, e1, W, nb, xq, y, sums);
  } else {
    if (passes == 1) return launch<kWaves>(gemv_q4_K_cols<kWaves, 1, NC, S, FMT>, n_out, lds, s, e0, e1, W, nb, xq, y, sums);
    if (passes == 2) return launch<kWaves>(gemv_q4_K_cols<kWaves, 2, NC, S, FMT>, n_out, lds, s, e0, e1, W, nb, xq, y, sums);
    return launch<kWaves>(gemv_q4_K_cols<kWaves, 3, NC, S, FMT>, n_out, lds, s, e0, e1, W, nb, xq, y, sums);
  }
}
template <bool S, int FMT>
hipError_t launch_cols_s(const uint8_t* W, int64_t n_out, int nb, const uint8_t* xq, int64_t ncols, float* y,
                         int32_t* sums, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (ncols == 2) return launch_cols_nc<2, S, FMT>(W, n_out, nb, xq, y, sums, s, e0, e1);
  if (ncols == 3) return launch_cols_nc<3, S, FMT>(W, n_out, nb, xq, y, sums, s, e0, e1);
  return launch_cols_nc<4, S, FMT>(W, n_out, nb, xq, y, sums, s, e0, e1);
}
}  // namespace

hipError_t launch_gemv_cols(int w_type, const uint8_t* W, int64_t n_out, int64_t n_in, const uint8_t* xq,
                            int64_t ncols, float* y, int32_t* sums, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (!gemv_cols_fits(w_type, n_in, ncols)) return hipErrorInvalidValue;
  if (n_out <= 0) return hipSuccess;
  const bool S = sums != nullptr;
  if (w_type == kQ8_0 || w_type == kQ4_0 || w_type == kQ5_0) {
    const int nb32 = static_cast<int>(n_in / 32);
    const int f = w_type == kQ8_0 ? 0 : w_type == kQ4_0 ? 1 : 2;
    if (f == 0) return S ? launch_q80_cols_s<true, 0>(W, n_out, nb32, xq, ncols, y, sums, s, e0, e1)
                         : launch_q80_cols_s<false, 0>(W, n_out, nb32, xq, ncols, y, sums, s, e0, e1);
    if (f == 1) return S ? launch_q80_cols_s<true, 1>(W, n_out, nb32, xq, ncols, y, sums, s, e0, e1)
                         : launch_q80_cols_s<false, 1>(W, n_out, nb32, xq, ncols, y, sums, s, e0, e1);
    return S ? launch_q80_cols_s<true, 2>(W, n_out, nb32, xq, ncols, y, sums, s, e0, e1)
             : launch_q80_cols_s<false, 2>(W, n_out, nb32, xq, ncols, y, sums, s, e0, e1);
  }
  const int nb = static_cast<int>(n_in / 256);
  if (w_type == kQ5_K) {
    return S ? launch_cols_s<true, 1>(W, n_out, nb, xq, ncols, y, sums, s, e0, e1)
             : launch_cols_s<false, 1>(W, n_out, nb, xq, ncols, y, sums, s, e0, e1);
  }
  if (w_type == kQ6_K) {
    return S ? launch_cols_s<true, 2>(W, n_out, nb, xq, ncols, y, sums, s, e0, e1)
             : launch_cols_s<false, 2>(W, n_out, nb, xq, ncols, y, sums, s, e0, e1);
  }
  return S ? launch_cols_s<true, 0>(W, n_out, nb, xq, ncols, y, sums, s, e0, e1)
           : launch_cols_s<false, 0>(W, n_out, nb, xq, ncols, y, sums, s, e0, e1);
}

hipError_t launch_gemv(int w_type, const uint8_t* W, int64_t n_out, int64_t n_in,
                       const uint8_t* xq, float* y, int32_t* sums, hipStream_t s,
                       hipEvent_t e0, hipEvent_t e1) {
  if (n_out <= 0) return hipSuccess;
  const int64_t lds = gemv_lds_bytes(w_type, n_in);
  const bool S = sums != nullptr;
#define QK_ROWS(kern) launch_rows<4>(kern, n_out, 1, max_row_waves(), s, e0, e1, W, nb, xq, y, sums)
#define QK_LDS(kern) launch<kWaves>(kern, n_out, lds, s, e0, e1, W, nb, xq, y, sums)
#define QK_LDS8(kern) launch<kWaves32>(kern, n_out, lds, s, e0, e1, W, nb, xq, y, sums)
  switch (w_type) {
    case kQ4_K: {
      const int nb = static_cast<int>(n_in / 256);
      const int passes = (nb + 15) / 16;
      if (passes == 1) return S ? QK_ROWS((gemv_q4_K_reg<4, 1, 1, true>)) : QK_ROWS((gemv_q4_K_reg<4, 1, 1, false>));
      if (passes == 2) return S ? QK_ROWS((gemv_q4_K_reg<4, 2, 1, true>)) : QK_ROWS((gemv_q4_K_reg<4, 2, 1, false>));
      if (passes == 3) return S ? QK_LDS((gemv_q4_K_kernel<kWaves, 3, true>)) : QK_LDS((gemv_q4_K_kernel<kWaves, 3, false>));
      return S ? QK_LDS((gemv_q4_K_kernel<kWaves, 4, true>)) : QK_LDS((gemv_q4_K_kernel<kWaves, 4, false>));
    }
    case kQ5_K: {
      const int nb = static_cast<int>(n_in / 256);
      const int passes = (nb + 15) / 16;
      if (passes == 1) return S ? QK_ROWS((gemv_q4_K_reg<4, 1, 1, true, 1>)) : QK_ROWS((gemv_q4_K_reg<4, 1, 1, false, 1>));
      if (passes == 2) return S ? QK_ROWS((gemv_q4_K_reg<4, 2, 1, true, 1>)) : QK_ROWS((gemv_q4_K_reg<4, 2, 1, false, 1>));
      if (passes == 3) return S ? QK_LDS((gemv_q4_K_kernel<kWaves, 3, true, 1>)) : QK_LDS((gemv_q4_K_kernel<kWaves, 3, false, 1>));
      return S ? QK_LDS((gemv_q4_K_kernel<kWaves, 4, true, 1>)) : QK_LDS((gemv_q4_K_kernel<kWaves, 4, false, 1>));
    }
    case kQ6_K: {
      const int nb = static_cast<int>(n_in / 256);
      const int passes = (nb + 15) / 16;
      if (passes == 1) return S ? QK_ROWS((gemv_q6_K_reg<4, 1, true>)) : QK_ROWS((gemv_q6_K_reg<4, 1, false>));
      if (passes == 2) return S ? QK_ROWS((gemv_q6_K_reg<4, 2, true>)) : QK_ROWS((gemv_q6_K_reg<4, 2, false>));
      if (passes == 3) return S ? QK_LDS((gemv_q6_K_kernel<kWaves, 3, true>)) : QK_LDS((gemv_q6_K_kernel<kWaves, 3, false>));
      return S ? QK_LDS((gemv_q6_K_kernel<kWaves, 4, true>)) : QK_LDS((gemv_q6_K_kernel<kWaves, 4, false>));
    }
    case kQ8_0: {
      const int nb = static_cast<int>(n_in / 32);
      const int passes = (nb + 63) / 64;
      if (passes == 1) return S ? QK_ROWS((gemv_q80_reg<4, 1, kFmtQ8_0, true>)) : QK_ROWS((gemv_q80_reg<4, 1, kFmtQ8_0, false>));
      if (passes == 2) return S ? QK_LDS8((gemv_q8_0_kernel<kWaves32, 2, true>)) : QK_LDS8((gemv_q8_0_kernel<kWaves32, 2, false>));
      if (passes <= 4) return S ? QK_LDS8((gemv_q8_0_kernel<kWaves32, 4, true>)) : QK_LDS8((gemv_q8_0_kernel<kWaves32, 4, false>));
      return S ? QK_LDS8((gemv_q8_0_kernel<kWaves32, 6, true>)) : QK_LDS8((gemv_q8_0_kernel<kWaves32, 6, false>));
    }
    case kQ4_0: {
      // 32-element formats keep all of a row's passes of weight loads in flight up
      // to six passes (rows of 10240 and 11008): at 4096 x 11008, six in flight
      // rather than eight measured Q4_0 9.1 -> 8.7 us, Q5_0 10.5 -> 9.7,
      // Q4_1 7.1 -> 6.6 and Q5_1 8.3 -> 7.5.
      const int nb = static_cast<int>(n_in / 32);
      const int passes = (nb + 63) / 64;
      if (passes == 1) return S ? QK_ROWS((gemv_q80_reg<4, 1, kFmtQ4_0, true>)) : QK_ROWS((gemv_q80_reg<4, 1, kFmtQ4_0, false>));
      if (passes == 2) return S ? QK_LDS8((gemv_q4_0_kernel<kWaves32, 2, false, true>)) : QK_LDS8((gemv_q4_0_kernel<kWaves32, 2, false, false>));
      if (passes <= 4) return S ? QK_LDS8((gemv_q4_0_kernel<kWaves32, 4, false, true>)) : QK_LDS8((gemv_q4_0_kernel<kWaves32, 4, false, false>));
      if (passes <= 6) return S ? QK_LDS8((gemv_q4_0_kernel<kWaves32, 6, false, true>)) : QK_LDS8((gemv_q4_0_kernel<kWaves32, 6, false, false>));
      return S ? QK_LDS8((gemv_q4_0_kernel<kWaves32, 8, false, true>)) : QK_LDS8((gemv_q4_0_kernel<kWaves32, 8, false, false>));
    }
    case kQ5_0: {
      const int nb = static_cast<int>(n_in / 32);
      const int passes = (nb + 63) / 64;
      if (passes == 1) return S ? QK_ROWS((gemv_q80_reg<4, 1, kFmtQ5_0, true>)) : QK_ROWS((gemv_q80_reg<4, 1, kFmtQ5_0, false>));
      if (passes == 2) return S ? QK_LDS8((gemv_q4_0_kernel<kWaves32, 2, true, true>)) : QK_LDS8((gemv_q4_0_kernel<kWaves32, 2, true, false>));
      if (passes <= 4) return S ? QK_LDS8((gemv_q4_0_kernel<kWaves32, 4, true, true>)) : QK_LDS8((gemv_q4_0_kernel<kWaves32, 4, true, false>));
      if (passes <= 6) return S ? QK_LDS8((gemv_q4_0_kernel<kWaves32, 6, true, true>)) : QK_LDS8((gemv_q4_0_kernel<kWaves32, 6, true, false>));
      return S ? QK_LDS8((gemv_q4_0_kernel<kWaves32, 8, true, true>)) : QK_LDS8((gemv_q4_0_kernel<kWaves32, 8, true, false>));
    }
    case kQ2_K:
    case kQ3_K: {
      const int nb = static_cast<int>(n_in / 256);
      const int passes = (nb + 15) / 16;
      if (w_type == kQ2_K) {
        if (passes == 1) return S ? QK_LDS((gemv_q23_K_kernel<kWaves, 1, true, 0>)) : QK_LDS((gemv_q23_K_kernel<kWaves, 1, false, 0>));
        if (passes == 2) return S ? QK_LDS((gemv_q23_K_kernel<kWaves, 2, true, 0>)) : QK_LDS((gemv_q23_K_kernel<kWaves, 2, false, 0>));
        if (passes == 3) return S ? QK_LDS((gemv_q23_K_kernel<kWaves, 3, true, 0>)) : QK_LDS((gemv_q23_K_kernel<kWaves, 3, false, 0>));
        return S ? QK_LDS((gemv_q23_K_kernel<kWaves, 4, true, 0>)) : QK_LDS((gemv_q23_K_kernel<kWaves, 4, false, 0>));
      }
      if (passes == 1) return S ? QK_LDS((gemv_q23_K_kernel<kWaves, 1, true, 1>)) : QK_LDS((gemv_q23_K_kernel<kWaves, 1, false, 1>));
      if (passes == 2) return S ? QK_LDS((gemv_q23_K_kernel<kWaves, 2, true, 1>)) : QK_LDS((gemv_q23_K_kernel<kWaves, 2, false, 1>));
      if (passes == 3) return S ? QK_LDS((gemv_q23_K_kernel<kWaves, 3, true, 1>)) : QK_LDS((gemv_q23_K_kernel<kWaves, 3, false, 1>));
      return S ? QK_LDS((gemv_q23_K_kernel<kWaves, 4, true, 1>)) : QK_LDS((gemv_q23_K_kernel<kWaves, 4, false, 1>));
    }
    case kQ4_1:
    case kQ5_1: {
      const int nb = static_cast<int>(n_in / 32);
      const int passes = (nb + 63) / 64;
      if (w_type == kQ4_1) {
        if (passes == 1) return S ? QK_LDS((gemv_q4_1_kernel<kWaves, 1, false, true>)) : QK_LDS((gemv_q4_1_kernel<kWaves, 1, false, false>));
        if (passes == 2) return S ? QK_LDS((gemv_q4_1_kernel<kWaves, 2, false, true>)) : QK_LDS((gemv_q4_1_kernel<kWaves, 2, false, false>));
        if (passes <= 4) return S ? QK_LDS((gemv_q4_1_kernel<kWaves, 4, false, true>)) : QK_LDS((gemv_q4_1_kernel<kWaves, 4, false, false>));
        if (passes <= 6) return S ? QK_LDS((gemv_q4_1_kernel<kWaves, 6, false, true>)) : QK_LDS((gemv_q4_1_kernel<kWaves, 6, false, false>));
        return S ? QK_LDS((gemv_q4_1_kernel<kWaves, 8, false, true>)) : QK_LDS((gemv_q4_1_kernel<kWaves, 8, false, false>));
      }
      if (passes == 1) return S ? QK_LDS((gemv_q4_1_kernel<kWaves, 1, true, true>)) : QK_LDS((gemv_q4_1_kernel<kWaves, 1, true, false>));
      if (passes == 2) return S ? QK_LDS((gemv_q4_1_kernel<kWaves, 2, true, true>)) : QK_LDS((gemv_q4_1_kernel<kWaves, 2, true, false>));
      if (passes <= 4) return S ? QK_LDS((gemv_q4_1_kernel<kWaves, 4, true, true>)) : QK_LDS((gemv_q4_1_kernel<kWaves, 4, true, false>));
      if (passes <= 6) return S ? QK_LDS((gemv_q4_1_kernel<kWaves, 6, true, true>)) : QK_LDS((gemv_q4_1_kernel<kWaves, 6, true, false>));
      return S ? QK_LDS((gemv_q4_1_kernel<kWaves, 8, true, true>)) : QK_LDS((gemv_q4_1_kernel<kWaves, 8, true, false>));
    }
    default:
      return hipErrorInvalidValue;
  }
#undef QK_ROWS
#undef QK_LDS
#undef QK_LDS8
}

// One launch, with the caller's start / stop events recorded by the launch itself
// when either is non-null (HIP extended launch).
template <typename K, typename... Args>
void launch_ev(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s, hipEvent_t e0, hipEvent_t e1,
               Args... args) {
  if (e0 != nullptr || e1 != nullptr) {
    hipExtLaunchKernelGGL(kernel, grid, block, static_cast<uint32_t>(lds), s, e0, e1, 0, args...);
  } else {
    kernel<<<grid, block, lds, s>>>(args...);
  }
}

template <int EPI, int Q5>
hipError_t launch_pair_epi(const uint8_t* W1, const uint8_t* W2, int64_t n_out, int64_t n_in,
                           const uint8_t* xq, int64_t ncols, float* out, hipStream_t s, hipEvent_t e0,
                           hipEvent_t e1) {
  const int nb = static_cast<int>(n_in / 256);
  const int n = static_cast<int>(n_out);
  const int passes = (nb + 15) / 16;
  if (passes <= 2) {
    // a wavefront has two rows' loads in flight: two 4-wavefront workgroups per CU
    // (2048 wavefronts measured best on the 11008 x 4096 gate / up pair; 4096 and
    // 8192 slower)
    const int64_t pair_waves = 2 * 4 * cu_count();
    const int64_t waves = n_out < pair_waves ? n_out : pair_waves;
    const dim3 grid(static_cast<unsigned>((waves + 3) / 4), static_cast<unsigned>(ncols));
    if (passes == 1) launch_ev(gemv_q4_K_pair_reg<4, 1, EPI, Q5>, grid, dim3(256), 0, s, e0, e1, W1, W2, n, nb, xq, out);
    else launch_ev(gemv_q4_K_pair_reg<4, 2, EPI, Q5>, grid, dim3(256), 0, s, e0, e1, W1, W2, n, nb, xq, out);
  } else {
    unsigned gx = 0;
    if (!launch_grid((n_out + kWaves - 1) / kWaves, kWaves * 64, &gx)) return hipErrorInvalidConfiguration;
    const dim3 grid(gx, static_cast<unsigned>(ncols));
    const int64_t lds = gemv_lds_bytes(kQ4_K, n_in);
    const hipError_t attr = allow_lds(gemv_q4_K_pair_kernel<kWaves, 3, EPI, Q5>, lds);
    if (attr != hipSuccess) return attr;
    launch_ev(gemv_q4_K_pair_kernel<kWaves, 3, EPI, Q5>, grid, dim3(kWaves * 64), static_cast<size_t>(lds), s, e0, e1,
              W1, W2, n, nb, xq, out);
  }
  return hipGetLastError();
}

hipError_t launch_gemv_pair(int w_type, const uint8_t* W1, const uint8_t* W2, int64_t n_out, int64_t n_in,
                            const uint8_t* xq, int64_t ncols, int swiglu, float* out, hipStream_t s,
                            hipEvent_t e0, hipEvent_t e1) {
  if (n_out <= 0 || ncols <= 0) return hipSuccess;
  if (w_type == kQ5_K) {
    return swiglu ? launch_pair_epi<kEpiSwiglu, 1>(W1, W2, n_out, n_in, xq, ncols, out, s, e0, e1)
                  : launch_pair_epi<kEpiPair, 1>(W1, W2, n_out, n_in, xq, ncols, out, s, e0, e1);
  }
  if (w_type != kQ4_K) return hipErrorInvalidValue;
  return swiglu ? launch_pair_epi<kEpiSwiglu, 0>(W1, W2, n_out, n_in, xq, ncols, out, s, e0, e1)
                : launch_pair_epi<kEpiPair, 0>(W1, W2, n_out, n_in, xq, ncols, out, s, e0, e1);
}

}  // namespace qk
