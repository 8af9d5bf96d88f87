// qk_gemm.hip - batched Q4_K x Q8_K product (2..64 activation columns per launch)
// on the gfx950 matrix cores.
//
// Same method as the GEMV (rml "Quantized dot products"; candle formats page,
// BlockQ4K / BlockQ8K): for every (token t, row r, superblock b) the exact int32
//   S_q = sum_j sc_j * s_j,  s_j = sum_{e in sub-block j} q_e a_e   (32 elements)
//   S_m = sum_j m_j * B_j,   B_j = sum_{e in j} a_e = bsum_{2j} + bsum_{2j+1}
// (candle 块结构: BlockQ8K carries the 16-element code sums so that the min term needs
// no pass over the codes), and y[t][r] accumulates dx * (d * S_q - dmin * S_m) in f32.
// With many tokens the code products are a dense contraction, so they run on MFMA:
//   - S_q: v_mfma_i32_16x16x64_i8 with the 6-bit scale folded into the weight
//     operand, split as sc = 8 * (sc >> 3) + (sc & 7): the bytes q * (sc & 7) and
//     q * (sc >> 3) are at most 105, so both are int8 operands and S_q = 8 * Q_hi +
//     Q_lo, where Q_hi and Q_lo accumulate over the superblock inside the matrix core
//     (exact int32).  Two MFMAs per 64 elements and 16 x 16 tile.
//   - S_m: one v_mfma_f32_16x16x32_bf16 per superblock and tile from the bsums.  B_j
//     lies in [-4064, 4064]; it is split as B_j = 64 * Bh + Bl with Bl = B_j & 63, and
//     64 * Bh (a multiple of 64 below 2^13) and Bl (below 64) are exact bf16 values,
//     as is m_j <= 63.  The 16 products m_j * (64 Bh_j) and m_j * Bl_j are exact in f32
//     and so is every partial sum (|S_m| < 2^21 < 2^24), so the f32 result is S_m
//     exactly.
// Operand layout (checked on the hardware): A = activations, lane l holds token
// l % 16 and k-slot group g = l / 16 (16 bytes, or 8 bf16); B = weights, lane l
// holds row l % 16 and the same k-slot group; D[token][row] lands in lane row +
// 16 * (token / 4), element token % 4, so the four outputs of a lane share one
// weight row and its scales.  Lane group g of a row holds qs bytes 16g .. 16g+15
// (chunk g / 2) and 64 + 16g .. 64 + 16g + 15 (chunk 2 + g / 2); their low and high
// nibbles are four runs of 16 consecutive elements, one sub-block each: with
// c = g / 2 and p = 16 (g % 2), MFMA i = 0, 1, 2, 3 takes elements 64c + p, 64c + 32
// + p, 64(c + 2) + p and 64(c + 2) + 32 + p onwards (sub-blocks 2c, 2c + 1, 2c + 4,
// 2c + 5), so each operand carries one scale factor and its activation bytes are
// 16 consecutive codes of the Q8_K block.
//
// Data movement.  A workgroup owns R rows (R a multiple of 8, chosen so that about
// one workgroup runs per CU) and all tokens.  Its compute wavefronts (RT 16-row
// tiles x KS, each of the KS taking a contiguous range of every chunk's
// superblocks) stream their own rows' 144-byte superblocks from HBM into
// registers, P superblocks in flight.  The loads are coalesced: four consecutive
// lanes read one row's 16-byte header (a dword each) and 2 x 64 contiguous qs
// bytes, so a quad of lanes touches one cache line per instruction; ds_bpermute
// then moves each row's bytes to the four lanes of the MFMA layout (loading lane
// 4r + g -> MFMA lane 16g + r).  No weight byte is stored in LDS.
// Four staging wavefronts copy the activations into LDS in chunks of KC
// superblocks x all tokens (two buffers, one chunk ahead), token-major with a
// 272-byte stride (coalesced 16-byte writes, and the MFMA's 16-byte reads of 8
// consecutive tokens fall in distinct banks), each (superblock, 16-token tile)
// followed by the bf16 digits of B_j for the S_m MFMA and the 16 scales dx.  They
// issue no weight loads, so their in-order memory counter never waits behind the
// weight stream; both roles meet only at the chunk barriers.  The K-split partial
// sums of an output are added in LDS at the end, in split order.
#include <hip/hip_ext.h>

#include <type_traits>

#include "qk_device.h"
#include "qk_internal.h"

namespace qk {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));  // register-friendly 16 bytes
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr uint32_t kLo4 = 0x0F0F0F0Fu;
constexpr uint32_t kHi2 = 0x30303030u;

// LDS image of one (superblock, 16-token tile).
constexpr int kTokStride = 272;              // 256 codes + 16: conflict-free operand reads
constexpr int kDigOff = 16 * kTokStride;     // digits: lanes 0-15 64 * Bh_j, lanes 16-31 Bl_j (8 bf16)
constexpr int kDxOff = kDigOff + 512;        // 16 f32 scales dx
constexpr int kBT = kDxOff + 64;             // 4928 bytes
constexpr int kZeroBytes = 512;              // the digit operand of lanes 32..63 (all zero)
constexpr int kTokImg = 304;                 // one token's Q8_K block in a wavefront's LDS region

// 16 bytes at a 4-byte aligned global address (Q8_K codes start 4 bytes into the block)
__device__ __forceinline__ u4 load_a4x4(const uint8_t* p) {
  const uint32_t* p4 = reinterpret_cast<const uint32_t*>(__builtin_assume_aligned(p, 4));
  u4 v;
  __builtin_memcpy(&v, p4, 16);
  return v;
}
// Each byte of x times the small factor held in both halves of s2 (packed 16-bit
// multiply): every product stays below 256 (codes <= 15, factor <= 7), so no byte
// carries into its neighbour.
__device__ __forceinline__ int mul_bytes(uint32_t x, uint32_t s2) {
  return static_cast<int>(
      __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, x) * __builtin_bit_cast(u16x2, s2)));
}
// bf16 bits of a float that bf16 holds exactly (its low 16 bits are zero).
__device__ __forceinline__ uint32_t bf16_hi(float f) { return __float_as_uint(f) >> 16; }
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Launch shape: NT 16-token tiles, RT 16-row tiles per workgroup, KS compute
// wavefronts per row tile splitting the superblocks, P superblocks of weights in
// flight per compute wavefront; SW staging wavefronts copy the activations in
// chunks of KC superblocks (at most 16 / NT: two chunks fill the LDS).
template <int NT_, int RT_, int KS_, int P_, int SW_ = 4, int KC_ = 16 / NT_>
struct Cfg {
  static constexpr int NT = NT_, RT = RT_, KS = KS_, P = P_, SW = SW_;
  static constexpr int KC = KC_;                // superblocks per LDS chunk
  static constexpr int QC = KC / KS;            // superblocks per wavefront and chunk
  static constexpr int B = P > QC ? P : QC;     // superblocks per loop iteration
  static constexpr int kCW = RT * KS;           // compute wavefronts
  static constexpr int kWaves = kCW + SW;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kST = 64 * SW;           // staging threads
  static constexpr int kChunk = KC * NT * kBT;  // 78,848 bytes for KC = 16 / NT
  static constexpr int kLds = kZeroBytes + 2 * kChunk;
  static constexpr int kPieces = KC * NT * 256;  // 16-byte code pieces per chunk
  static constexpr int kPPT = kPieces / kST;
  static constexpr int kPairs = KC * NT * 16;    // (superblock, token) pairs per chunk
  static constexpr int kRedBytes = (KS - 1) * RT * NT * 4 * 64 * 4;
  static_assert(KC % KS == 0 && QC >= 1, "whole superblocks per wavefront and chunk");
  static_assert(B % QC == 0 && B % P == 0, "whole chunks and whole weight rings per iteration");
  static_assert(kST == 256 && kPieces % kST == 0, "piece k of a staging thread is image k");
  static_assert(kPairs <= kST, "at most one (superblock, token) pair per staging thread");
  static_assert(kRedBytes <= 2 * kChunk, "the K-split reduction fits the chunk buffers");
  static_assert(kLds <= 160 * 1024, "one workgroup's LDS fits a CU");
};

// One chunk's activation bytes in flight, per thread.
template <class C>
struct Stage {
  u4 code[C::kPPT];
  u4 bs0, bs1;  // the 16 bsums of this thread's (superblock, token) pair
  float dx;
};

// What each staging thread copies, fixed for the whole kernel.  Piece k of staging
// thread i (i = 0 .. 255) is piece j = i % 16 of token n = (i / 16) % 16 of image k
// (image = (superblock, tile) pair, k = sb * NT + t), so the image and the
// superblock part of the address are compile-time / wave-uniform and only the
// token part is per lane.  Superblocks past the row end are clamped to the last
// one (valid memory, never used).
template <class C>
struct StageMap {
  uint32_t src[C::kPPT];  // token * xrow + 4 + 16 j (per lane)
  uint32_t dst;           // n * kTokStride + 16 j; image k adds k * kBT
  uint32_t psrc;          // the thread's (superblock, token) pair
  int psb;
  uint32_t pimg;          // LDS offset of the pair's (superblock, tile) image
  int ptok;               // the pair's token inside its tile

  __device__ __forceinline__ StageMap(int sid, int ncols, uint32_t xrow) {
    const int n = (sid >> 4) & 15, j = sid & 15;
#pragma unroll
    for (int k = 0; k < C::kPPT; ++k) {
      const int tok = min(16 * (k % C::NT) + n, ncols - 1);
      src[k] = static_cast<uint32_t>(tok) * xrow + 4 + 16 * j;
    }
    dst = n * kTokStride + 16 * j;
    const int tok = sid % (16 * C::NT);
    psrc = static_cast<uint32_t>(min(tok, ncols - 1)) * xrow;
    psb = sid / (16 * C::NT);
    pimg = (psb * C::NT + tok / 16) * kBT;
    ptok = tok % 16;
  }
};

template <class C>
__device__ __forceinline__ void stage_load(Stage<C>& st, const StageMap<C>& m, const uint8_t* __restrict__ xq,
                                           int nb, int b0) {
#pragma unroll
  for (int k = 0; k < C::kPPT; ++k) {
    const uint8_t* base = xq + static_cast<uint32_t>(min(b0 + k / C::NT, nb - 1)) * kQ8_KBytes;  // scalar
    st.code[k] = load_a4x4(base + m.src[k]);
  }
  const uint8_t* p = xq + m.psrc + static_cast<uint32_t>(min(b0 + m.psb, nb - 1)) * kQ8_KBytes;
  st.dx = *reinterpret_cast<const float*>(p);
  st.bs0 = load_a4x4(p + 260);
  st.bs1 = load_a4x4(p + 276);
}

template <class C>
__device__ __forceinline__ void stage_store(const Stage<C>& st, const StageMap<C>& m, uint8_t* buf) {
#pragma unroll
  for (int k = 0; k < C::kPPT; ++k) *reinterpret_cast<u4*>(buf + m.dst + k * kBT) = st.code[k];
  {
    // B_j = bsum_{2j} + bsum_{2j+1}, split into the bf16 digits 64 * Bh_j and Bl_j
    const uint32_t w[8] = {st.bs0[0], st.bs0[1], st.bs0[2], st.bs0[3],
                           st.bs1[0], st.bs1[1], st.bs1[2], st.bs1[3]};
    float hi[8], lo[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int B = static_cast<int>(static_cast<int16_t>(w[j] & 0xFFFFu)) + (static_cast<int>(w[j]) >> 16);
      const int bl = B & 63;
      hi[j] = static_cast<float>(B - bl);
      lo[j] = static_cast<float>(bl);
    }
    u4 h4, l4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h4[e] = pack_bf16(hi[2 * e], hi[2 * e + 1]);
      l4[e] = pack_bf16(lo[2 * e], lo[2 * e + 1]);
    }
    if (m.psb >= C::KC) return;  // smaller chunks: more staging threads than pairs
    uint8_t* img = buf + m.pimg;
    *reinterpret_cast<u4*>(img + kDigOff + m.ptok * 16) = h4;        // lanes 0-15
    *reinterpret_cast<u4*>(img + kDigOff + 256 + m.ptok * 16) = l4;  // lanes 16-31
    *reinterpret_cast<float*>(img + kDxOff + m.ptok * 4) = st.dx;
  }
}

// The four scaled weight operand pairs, d, dmin and the bf16 mins of one superblock
// for the lane's row and k-slot group g (sub-blocks 2c, 2c + 1, 2c + 4, 2c + 5 with
// c = g / 2; sel0 / sel1 pick byte 2c / 2c + 1 of a scale word into both 16-bit
// halves).
struct WOps {
  v4i lo[4], hi[4];
  bf16x8 m;
  float d, dmin;
};

__device__ __forceinline__ WOps build_wops(const u4& h, const u4& qa, const u4& qb, uint32_t sel0,
                                           uint32_t sel1) {
  WOps o;
  // 6-bit scales and mins of the 8 sub-blocks (get_scale_min_k4 on whole words)
  const uint32_t sc_a = h[1] & 0x3F3F3F3Fu, m_a = h[2] & 0x3F3F3F3Fu;
  const uint32_t sc_b = (h[3] & kLo4) | ((h[1] >> 2) & kHi2);
  const uint32_t m_b = ((h[3] >> 4) & kLo4) | ((h[2] >> 2) & kHi2);
  const uint32_t l3a = sc_a & 0x07070707u, h3a = (sc_a >> 3) & 0x07070707u;
  const uint32_t l3b = sc_b & 0x07070707u, h3b = (sc_b >> 3) & 0x07070707u;
  const uint32_t s_l[4] = {__builtin_amdgcn_perm(l3a, l3a, sel0), __builtin_amdgcn_perm(l3a, l3a, sel1),
                           __builtin_amdgcn_perm(l3b, l3b, sel0), __builtin_amdgcn_perm(l3b, l3b, sel1)};
  const uint32_t s_h[4] = {__builtin_amdgcn_perm(h3a, h3a, sel0), __builtin_amdgcn_perm(h3a, h3a, sel1),
                           __builtin_amdgcn_perm(h3b, h3b, sel0), __builtin_amdgcn_perm(h3b, h3b, sel1)};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t q4[4] = {qa[e] & kLo4, (qa[e] >> 4) & kLo4, qb[e] & kLo4, (qb[e] >> 4) & kLo4};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o.lo[i][e] = mul_bytes(q4[i], s_l[i]);
      o.hi[i][e] = mul_bytes(q4[i], s_h[i]);
    }
  }
  u4 mw;
  mw[0] = pack_bf16(static_cast<float>(m_a & 0xFF), static_cast<float>((m_a >> 8) & 0xFF));
  mw[1] = pack_bf16(static_cast<float>((m_a >> 16) & 0xFF), static_cast<float>(m_a >> 24));
  mw[2] = pack_bf16(static_cast<float>(m_b & 0xFF), static_cast<float>((m_b >> 8) & 0xFF));
  mw[3] = pack_bf16(static_cast<float>((m_b >> 16) & 0xFF), static_cast<float>(m_b >> 24));
  o.m = __builtin_bit_cast(bf16x8, mw);
  o.d = f16_to_f32(h[0] & 0xFFFFu);
  o.dmin = f16_to_f32(h[0] >> 16);
  return o;
}

// One superblock of weights as loaded (coalesced layout): lane 4r + q holds header
// dword q and qs bytes 16q .. 16q+15 and 64 + 16q .. 64 + 16q + 15 of row r.
struct WRaw {
  uint32_t hd;
  u4 qa, qb;
};

__device__ __forceinline__ uint32_t from_lane(int byte_addr, uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(byte_addr, static_cast<int>(v)));
}

template <class C, bool SUMS>
__global__ __launch_bounds__(C::kThreads) void gemm_q4_K_mfma(const uint8_t* __restrict__ W, int n_out, int nb,
                                                              const uint8_t* __restrict__ xq, int ncols,
                                                              int rows_wg, float* __restrict__ y,
                                                              int32_t* __restrict__ sums) {
  constexpr int NT = C::NT, KC = C::KC, KS = C::KS, QC = C::QC, P = C::P, B = C::B;
  extern __shared__ __align__(16) uint8_t lds[];
  uint8_t* const zero = lds;
  uint8_t* const buf0 = lds + kZeroBytes;
  uint8_t* const buf1 = buf0 + C::kChunk;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int n = lane & 15;  // weight row in the tile; token in the A operand
  const int g = lane >> 4;  // k-slot group; the lane's outputs are tokens 4g .. 4g+3
  const int w = wave_id();
  const uint32_t wrow = static_cast<uint32_t>(nb) * kQ4_KBytes;
  const uint32_t xrow = static_cast<uint32_t>(nb) * kQ8_KBytes;
  const int nchunk = (nb + KC - 1) / KC;
  const int qpad = (nchunk * QC + B - 1) / B * B;  // whole loop iterations
  const int nbarrier = qpad / QC;                  // chunk ends of the compute loop

  if (w >= C::kCW) {
    // Staging wavefronts: they issue no weight loads, so their waits cover only the
    // activation bytes.  Chunk 0 goes to buffer 0 before the first barrier; after
    // barrier c (the compute wavefronts are then on chunk c) chunk c + 1 goes to
    // the other buffer, whose last reader was chunk c - 1.  The barrier count
    // matches the compute wavefronts' (chunk ends, then the K-split reduction).
    const int sid = tid - 64 * C::kCW;
    const StageMap<C> map(sid, ncols, xrow);
    Stage<C> st;
    stage_load<C>(st, map, xq, nb, 0);
    if (sid < kZeroBytes / 16) *reinterpret_cast<u4*>(zero + sid * 16) = u4{0u, 0u, 0u, 0u};
    stage_store<C>(st, map, buf0);
    __syncthreads();
    for (int c = 0; c < nbarrier; ++c) {
      stage_load<C>(st, map, xq, nb, (c + 1) * KC);
      stage_store<C>(st, map, (c & 1) ? buf0 : buf1);
      __syncthreads();
    }
    if constexpr (!SUMS && KS > 1) __syncthreads();
    return;
  }

  const int rt = w % C::RT;  // row tile
  const int ks = w / C::RT;  // K split
  const int row0 = blockIdx.x * rows_wg;
  const int row_end = min(row0 + rows_wg, n_out);
  const int row = row0 + 16 * rt + n;
  // Weights: the workgroup's rows start at a wave-uniform address; the loading
  // layout's lane 4r + q reads row r of the tile (rows past the workgroup's end
  // read its last row: valid memory, never stored) at a 32-bit lane offset.
  const uint8_t* const Wwg = W + static_cast<size_t>(row0) * wrow;
  const uint32_t lw_hd = static_cast<uint32_t>(min(16 * rt + (lane >> 2), row_end - row0 - 1)) * wrow + 4 * (lane & 3);
  const uint32_t lw_qs = lw_hd + 12 * (lane & 3) + 16;  // qs bytes 16 q .. 16 q + 15
  // MFMA lane (n, g) takes row n's bytes from loading lane 4n + g; the header from
  // lanes 4n .. 4n + 3
  const int src_lane = 4 * (4 * n + g);
  const int src_hdr = 16 * n;
  const uint32_t sel0 = 0x0C000C00u + 0x00010001u * static_cast<uint32_t>(g & 2);
  const uint32_t sel1 = sel0 + 0x00010001u;
  // LDS: the wavefront multiplies superblocks ks * QC .. ks * QC + QC - 1 of each
  // chunk.  A operand of lane (token n, g): codes 64c + 16 (g % 2) + {0, 32, 128,
  // 160} of the token's row, c = g / 2; the digit operand of lanes 32..63 is the
  // zero area.
  const uint32_t wave_img = static_cast<uint32_t>(ks * QC * NT * kBT);
  const uint32_t a_lane = wave_img + n * kTokStride + 64 * (g >> 1) + 16 * (g & 1);
  const uint32_t dig_lane = wave_img + kDigOff + lane * 16;
  const uint32_t zero_lane = static_cast<uint32_t>(lane - 32) * 16;
  const uint32_t dx_lane = wave_img + kDxOff + g * 16;

  // the wavefront's superblock sequence: in chunk c, b = c * KC + ks * QC + j
  auto sb_of = [&](int q) { return (q / QC) * KC + ks * QC + (q % QC); };

  // a ring of P weight slots (superblocks past the row end are clamped; their
  // products get zero scales)
  WRaw ring[P];
  auto wload = [&](WRaw& r, int q) {
    const uint8_t* base = Wwg + static_cast<uint32_t>(min(sb_of(q), nb - 1)) * kQ4_KBytes;  // scalar
    r.hd = *reinterpret_cast<const uint32_t*>(base + lw_hd);
    r.qa = *reinterpret_cast<const u4*>(base + lw_qs);
    r.qb = *reinterpret_cast<const u4*>(base + lw_qs + 64);
  };

  // At most two superblocks of weights are requested before the first barrier (the
  // staging wavefronts' activation reads then meet a shorter queue), the rest of
  // the ring right after it.
  constexpr int kEarly = P < 2 ? P : 2;
#pragma unroll
  for (int s = 0; s < kEarly; ++s) wload(ring[s], s);
  __syncthreads();
#pragma unroll
  for (int s = kEarly; s < P; ++s) wload(ring[s], s);

  float acc[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[t][e] = 0.0f;

  // multiply the wavefront's superblock jj of the chunk in `cur` (superblock b)
  auto multiply = [&](const WOps& o, const uint8_t* cur, int jj, int b) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int img = (jj * NT + t) * kBT;
      v4i ql = {0, 0, 0, 0}, qh = {0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const v4i a = *reinterpret_cast<const v4i*>(cur + a_lane + img + 32 * (i & 1) + 128 * (i >> 1));
        ql = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, o.lo[i], ql, 0, 0, 0);
        qh = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, o.hi[i], qh, 0, 0, 0);
      }
      const bf16x8 dg = *reinterpret_cast<const bf16x8*>(g < 2 ? cur + dig_lane + img : zero + zero_lane);
      const v4f sm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dg, o.m, v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
      const v4f dx = *reinterpret_cast<const v4f*>(cur + dx_lane + img);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int sq = (qh[e] << 3) + ql[e];  // sc = 8 * (sc >> 3) + (sc & 7)
        const float v = fmaf(-o.dmin, sm[e], o.d * static_cast<float>(sq));
        acc[t][e] = fmaf(dx[e], v, acc[t][e]);
        if constexpr (SUMS) {
          const int tk = 16 * t + 4 * g + e;
          if (b < nb && row < row_end && tk < ncols) {
            int32_t* out = sums + ((static_cast<size_t>(tk) * n_out + row) * nb + b) * 2;
            out[0] = sq;
            out[1] = static_cast<int>(sm[e]);
          }
        }
      }
    }
  };

  // B superblocks per iteration; the slot of step j is j % P.  `more` is false on
  // the last iteration, which requests no weights past the wavefront's sequence.
  auto iteration = [&](int q0, auto more) {
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int q = q0 + j;
      const int cc = q / QC, jj = j % QC;  // q0 is a multiple of QC
      const int b = cc * KC + ks * QC + jj;
      WRaw& r = ring[j % P];
      u4 h, qa, qb;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        h[k] = from_lane(src_hdr + 4 * k, r.hd);
        qa[k] = from_lane(src_lane, r.qa[k]);
        qb[k] = from_lane(src_lane, r.qb[k]);
      }
      if (decltype(more)::value || j < B - P) wload(r, q + P);
      WOps o = build_wops(h, qa, qb, sel0, sel1);
      if (b < nb) multiply(o, (cc & 1) ? buf1 : buf0, jj, b);
      if (jj == QC - 1) __syncthreads();  // end of chunk cc: chunk cc + 1 is staged
    }
  };
  int q0 = 0;
  for (; q0 + B < qpad; q0 += B) iteration(q0, std::true_type{});
  iteration(q0, std::false_type{});

  if constexpr (!SUMS) {
    if constexpr (KS > 1) {
      // K-split wavefronts 1 .. KS-1 hand their partial sums to wavefront 0 of the
      // row tile, which adds them in split order
      float* red = reinterpret_cast<float*>(buf0);
      if (ks > 0) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) red[((((ks - 1) * C::RT + rt) * NT + t) * 4 + e) * 64 + lane] = acc[t][e];
      }
      __syncthreads();
      if (ks > 0) return;
#pragma unroll
      for (int k = 1; k < KS; ++k)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[t][e] += red[((((k - 1) * C::RT + rt) * NT + t) * 4 + e) * 64 + lane];
    }
    if (row < row_end) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int tk = 16 * t + 4 * g + e;
          if (tk < ncols) y[static_cast<size_t>(tk) * n_out + row] = acc[t][e];
        }
    }
  }
}

// ---------------------------------------------------------------------------
// Up to 16 tokens and rows of at most 16 superblocks (n_in <= 4096): the tokens'
// activation blocks for the whole row fit one workgroup's LDS (16 images of
// kBT bytes, 79 KB), so they are staged once, by the compute wavefronts
// themselves, and every wavefront puts all of its weight loads in flight at
// kernel start, as the one-column GEMV does.  A workgroup of RT x KS wavefronts
// owns RT 16-row tiles; wavefront (rt, ks) multiplies superblocks ks * QS ..
// ks * QS + QS - 1 of tile rt, and the KS partial sums of an output are added in
// LDS at the end, in split order.  Each thread issues its activation loads
// before its weight loads; the load counter retires in order, so storing the
// activations to LDS waits for those loads only.  The products and the float
// step are the kernel above's.
template <int RT, int KS, bool SUMS>
__global__ __launch_bounds__(64 * RT * KS) void gemm_q4_K_res(const uint8_t* __restrict__ W, int n_out, int nb,
                                                              const uint8_t* __restrict__ xq, int ncols,
                                                              int rows_wg, float* __restrict__ y,
                                                              int32_t* __restrict__ sums) {
  constexpr int NTH = 64 * RT * KS;
  constexpr int QS = (16 + KS - 1) / KS;       // superblocks per wavefront
  constexpr int kPPT = (4096 + NTH - 1) / NTH;  // 16-byte code pieces per thread (16 x 16 x 16)
  extern __shared__ __align__(16) uint8_t lds[];
  uint8_t* const zero = lds;
  uint8_t* const img0 = lds + kZeroBytes;       // superblock b's image at img0 + b * kBT

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int w = wave_id();
  const int rt = w % RT, ks = w / RT;
  const uint32_t wrow = static_cast<uint32_t>(nb) * kQ4_KBytes;
  const uint32_t xrow = static_cast<uint32_t>(nb) * kQ8_KBytes;
  const int row0 = blockIdx.x * rows_wg;
  const int row_end = min(row0 + rows_wg, n_out);
  const int row = row0 + 16 * rt + n;

  // activation loads: piece p = (superblock p / 256, token (p / 16) % 16, 16-byte
  // piece p % 16); one (superblock, token) pair of bsums and scale per thread of
  // the first 256.  Indices past the row's pieces or the call's tokens are clamped
  // (the clamped thread stores what the last one stores).
  const int npieces = nb * 256, npairs = nb * 16;
  u4 code[kPPT];
#pragma unroll
  for (int k = 0; k < kPPT; ++k) {
    const int pc = min(tid + k * NTH, npieces - 1);
    const int sb = pc >> 8, tok = min((pc >> 4) & 15, ncols - 1);
    code[k] = load_a4x4(xq + static_cast<uint32_t>(tok) * xrow + static_cast<uint32_t>(sb) * kQ8_KBytes + 4 +
                        16 * (pc & 15));
  }
  const bool pair_thread = tid < 256;  // whole wavefronts
  const int pp = min(tid, npairs - 1);
  const int psb = pp >> 4, ptok = pp & 15;
  u4 bs0 = u4{0u, 0u, 0u, 0u}, bs1 = u4{0u, 0u, 0u, 0u};
  float pdx = 0.0f;
  if (pair_thread) {
    const uint8_t* p = xq + static_cast<uint32_t>(min(ptok, ncols - 1)) * xrow + static_cast<uint32_t>(psb) * kQ8_KBytes;
    pdx = *reinterpret_cast<const float*>(p);
    bs0 = load_a4x4(p + 260);
    bs1 = load_a4x4(p + 276);
  }
  __builtin_amdgcn_sched_barrier(0);

  // all of this wavefront's weights (coalesced layout, as the kernel above)
  const uint8_t* const Wwg = W + static_cast<size_t>(row0) * wrow;
  const uint32_t lw_hd = static_cast<uint32_t>(min(16 * rt + (lane >> 2), row_end - row0 - 1)) * wrow + 4 * (lane & 3);
  const uint32_t lw_qs = lw_hd + 12 * (lane & 3) + 16;
  WRaw ring[QS];
#pragma unroll
  for (int i = 0; i < QS; ++i) {
    const uint8_t* base = Wwg + static_cast<uint32_t>(min(ks * QS + i, nb - 1)) * kQ4_KBytes;
    ring[i].hd = *reinterpret_cast<const uint32_t*>(base + lw_hd);
    ring[i].qa = *reinterpret_cast<const u4*>(base + lw_qs);
    ring[i].qb = *reinterpret_cast<const u4*>(base + lw_qs + 64);
  }
  __builtin_amdgcn_sched_barrier(0);

  // activations into LDS
#pragma unroll
  for (int k = 0; k < kPPT; ++k) {
    const int pc = min(tid + k * NTH, npieces - 1);
    *reinterpret_cast<u4*>(img0 + (pc >> 8) * kBT + ((pc >> 4) & 15) * kTokStride + 16 * (pc & 15)) = code[k];
  }
  if (pair_thread) {
    // B_j = bsum_{2j} + bsum_{2j+1}, split into the bf16 digits 64 * Bh_j and Bl_j
    const uint32_t wd[8] = {bs0[0], bs0[1], bs0[2], bs0[3], bs1[0], bs1[1], bs1[2], bs1[3]};
    float hi[8], lo[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int Bj = static_cast<int>(static_cast<int16_t>(wd[j] & 0xFFFFu)) + (static_cast<int>(wd[j]) >> 16);
      const int bl = Bj & 63;
      hi[j] = static_cast<float>(Bj - bl);
      lo[j] = static_cast<float>(bl);
    }
    u4 h4, l4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h4[e] = pack_bf16(hi[2 * e], hi[2 * e + 1]);
      l4[e] = pack_bf16(lo[2 * e], lo[2 * e + 1]);
    }
    uint8_t* img = img0 + psb * kBT;
    *reinterpret_cast<u4*>(img + kDigOff + ptok * 16) = h4;
    *reinterpret_cast<u4*>(img + kDigOff + 256 + ptok * 16) = l4;
    *reinterpret_cast<float*>(img + kDxOff + ptok * 4) = pdx;
  }
  if (tid < kZeroBytes / 16) *reinterpret_cast<u4*>(zero + tid * 16) = u4{0u, 0u, 0u, 0u};
  __syncthreads();

  // The lane indices of the weights' ds_bpermute are defined after the barrier (an
  // empty asm), so the compiler cannot hoist the permutes, and the waits for the
  // weight loads that they need, above it: the barrier waits for the activations
  // only.
  int src_lane = 4 * (4 * n + g);
  int src_hdr = 16 * n;
  asm volatile("" : "+v"(src_lane), "+v"(src_hdr));
  const uint32_t sel0 = 0x0C000C00u + 0x00010001u * static_cast<uint32_t>(g & 2);
  const uint32_t sel1 = sel0 + 0x00010001u;
  const uint32_t a_lane = n * kTokStride + 64 * (g >> 1) + 16 * (g & 1);
  const uint32_t dig_lane = kDigOff + lane * 16;
  const uint32_t zero_lane = static_cast<uint32_t>(lane - 32) * 16;
  const uint32_t dx_lane = kDxOff + g * 16;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < QS; ++i) {
    const int b = ks * QS + i;
    const WRaw& r = ring[i];
    u4 h, qa, qb;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      h[k] = from_lane(src_hdr + 4 * k, r.hd);
      qa[k] = from_lane(src_lane, r.qa[k]);
      qb[k] = from_lane(src_lane, r.qb[k]);
    }
    if (b >= nb) continue;  // wave-uniform
    const WOps o = build_wops(h, qa, qb, sel0, sel1);
    const uint8_t* cur = img0 + b * kBT;
    v4i ql = {0, 0, 0, 0}, qh = {0, 0, 0, 0};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const v4i a = *reinterpret_cast<const v4i*>(cur + a_lane + 32 * (m & 1) + 128 * (m >> 1));
      ql = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, o.lo[m], ql, 0, 0, 0);
      qh = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, o.hi[m], qh, 0, 0, 0);
    }
    const bf16x8 dg = *reinterpret_cast<const bf16x8*>(g < 2 ? cur + dig_lane : zero + zero_lane);
    const v4f sm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dg, o.m, v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
    const v4f dx = *reinterpret_cast<const v4f*>(cur + dx_lane);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int sq = (qh[e] << 3) + ql[e];  // sc = 8 * (sc >> 3) + (sc & 7)
      const float v = fmaf(-o.dmin, sm[e], o.d * static_cast<float>(sq));
      acc[e] = fmaf(dx[e], v, acc[e]);
      if constexpr (SUMS) {
        const int tk = 4 * g + e;
        if (row < row_end && tk < ncols) {
          int32_t* out = sums + ((static_cast<size_t>(tk) * n_out + row) * nb + b) * 2;
          out[0] = sq;
          out[1] = static_cast<int>(sm[e]);
        }
      }
    }
  }

  if constexpr (!SUMS) {
    if constexpr (KS > 1) {
      __syncthreads();  // every wavefront is done with the images
      float* red = reinterpret_cast<float*>(lds);
      if (ks > 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) red[(((ks - 1) * RT + rt) * 4 + e) * 64 + lane] = acc[e];
      }
      __syncthreads();
      if (ks > 0) return;
#pragma unroll
      for (int k = 1; k < KS; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += red[(((k - 1) * RT + rt) * 4 + e) * 64 + lane];
    }
    if (row < row_end) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tk = 4 * g + e;
        if (tk < ncols) y[static_cast<size_t>(tk) * n_out + row] = acc[e];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Up to 16 tokens, rows of at most 16 superblocks, tall matrices: wavefront k of a
// 16-wavefront workgroup owns superblock k of the workgroup's RT row tiles.  It
// loads that superblock's activation blocks of the 16 tokens (contiguous 16-byte
// pieces, through its own LDS region into the MFMA operand layout), then the
// weights of all RT row tiles, so every weight byte is requested at kernel start
// and no product waits for a workgroup barrier.  Each lane's RT x 4 products d_x (d S_q - dmin S_m)
// go to LDS once; after the one barrier each thread adds one output's partials in
// superblock order.  The products are the kernels' above.
template <int RT, bool SUMS>
__global__ __launch_bounds__(1024) void gemm_q4_K_col(const uint8_t* __restrict__ W, int n_out, int nb,
                                                      const uint8_t* __restrict__ xq, int ncols, int rows_wg,
                                                      float* __restrict__ y, int32_t* __restrict__ sums) {
  constexpr int kOut = RT * 256;  // outputs of a workgroup: RT tiles x 16 rows x 16 tokens
  extern __shared__ __align__(16) uint8_t lds[];
  float* const red = reinterpret_cast<float*>(lds);  // [superblock][RT][4][64]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int b = wave_id();        // this wavefront's superblock (no products when b >= nb)
  const int bc = min(b, nb - 1);  // valid memory for the loads
  const uint32_t wrow = static_cast<uint32_t>(nb) * kQ4_KBytes;
  const uint32_t xrow = static_cast<uint32_t>(nb) * kQ8_KBytes;
  const int row0 = blockIdx.x * rows_wg;
  const int row_end = min(row0 + rows_wg, n_out);

  // activations: the wavefront copies the 16 tokens' blocks of superblock bc into its
  // own LDS region (tokens past the call's are clamped), each token's 292 bytes at a
  // 304-byte stride shifted by 12, so that the codes (block bytes 4..259) and both
  // halves of the bsums start 16-byte aligned.  Piece j = 1..18 of token t is block
  // bytes 16j - 12 .. 16j + 3, copied with one 16-byte load; consecutive lanes take
  // consecutive pieces of one token, so a load instruction reads a few whole
  // 288-byte runs instead of a 32-byte run per token and lane group.  Dword 0 (the
  // scale dx) goes separately.  Only this wavefront writes and reads the region.
  const uint8_t* const xb = xq + static_cast<uint32_t>(bc) * kQ8_KBytes;  // scalar
  uint8_t* const img = lds + (SUMS ? 0 : nb * kOut * 4) + b * (16 * kTokImg);
  u4 piece[5];
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    const int pc = min(lane + 64 * k, 16 * 18 - 1);
    const int t = pc / 18, j = 1 + pc % 18;
    piece[k] = load_a4x4(xb + static_cast<uint32_t>(min(t, ncols - 1)) * xrow + 16 * j - 12);
  }
  const float dxt = *reinterpret_cast<const float*>(xb + static_cast<uint32_t>(min(n, ncols - 1)) * xrow);
  __builtin_amdgcn_sched_barrier(0);

  // weights of superblock bc, coalesced: lane 4r + q of row tile rt reads header
  // dword q and qs bytes 16q .. 16q + 15 and 64 + 16q .. of row 16 rt + r (rows past
  // the workgroup's end read its last row: valid memory, never stored)
  const uint8_t* const Wb = W + static_cast<size_t>(row0) * wrow + static_cast<uint32_t>(bc) * kQ4_KBytes;
  WRaw wr[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const uint32_t hd = static_cast<uint32_t>(min(16 * rt + (lane >> 2), row_end - row0 - 1)) * wrow + 4 * (lane & 3);
    const uint32_t qs = hd + 12 * (lane & 3) + 16;
    wr[rt].hd = *reinterpret_cast<const uint32_t*>(Wb + hd);
    wr[rt].qa = *reinterpret_cast<const u4*>(Wb + qs);
    wr[rt].qb = *reinterpret_cast<const u4*>(Wb + qs + 64);
  }
  __builtin_amdgcn_sched_barrier(0);

  // the activation pieces into the region (the waits cover the activation loads only:
  // the load counter retires in order), then this lane's operands out of it: the A
  // pieces of token n (codes 64c + 16 (g % 2) + {0, 32, 128, 160} onwards, c = g / 2),
  // its bsums, and dx of tokens 4g .. 4g + 3
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    const int pc = min(lane + 64 * k, 16 * 18 - 1);
    *reinterpret_cast<u4*>(img + (pc / 18) * kTokImg + 16 * (1 + pc % 18)) = piece[k];
  }
  *reinterpret_cast<float*>(img + n * kTokImg + 12) = dxt;  // the 4 lanes of a token store the same value
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  const uint8_t* const timg = img + n * kTokImg;
  v4i a[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    a[i] = *reinterpret_cast<const v4i*>(timg + 16 + 64 * (g >> 1) + 16 * (g & 1) + 32 * (i & 1) + 128 * (i >> 1));
  const u4 bs0 = *reinterpret_cast<const u4*>(timg + 272), bs1 = *reinterpret_cast<const u4*>(timg + 288);
  float dxv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) dxv[e] = *reinterpret_cast<const float*>(img + (4 * g + e) * kTokImg + 12);

  // bf16 digits of B_j = bsum_{2j} + bsum_{2j+1}: lanes 0-15 64 * Bh_j, lanes 16-31
  // Bl_j, lanes 32-63 zero (the k-slots that carry no products)
  bf16x8 dg;
  {
    const uint32_t wd[8] = {bs0[0], bs0[1], bs0[2], bs0[3], bs1[0], bs1[1], bs1[2], bs1[3]};
    float dv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int Bj = static_cast<int>(static_cast<int16_t>(wd[j] & 0xFFFFu)) + (static_cast<int>(wd[j]) >> 16);
      const int bl = Bj & 63;
      dv[j] = g == 0 ? static_cast<float>(Bj - bl) : (g == 1 ? static_cast<float>(bl) : 0.0f);
    }
    u4 d4;
#pragma unroll
    for (int e = 0; e < 4; ++e) d4[e] = pack_bf16(dv[2 * e], dv[2 * e + 1]);
    dg = __builtin_bit_cast(bf16x8, d4);
  }

  const int src_lane = 4 * (4 * n + g);
  const int src_hdr = 16 * n;
  const uint32_t sel0 = 0x0C000C00u + 0x00010001u * static_cast<uint32_t>(g & 2);
  const uint32_t sel1 = sel0 + 0x00010001u;
  float part[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    u4 h, qa, qb;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      h[k] = from_lane(src_hdr + 4 * k, wr[rt].hd);
      qa[k] = from_lane(src_lane, wr[rt].qa[k]);
      qb[k] = from_lane(src_lane, wr[rt].qb[k]);
    }
    const WOps o = build_wops(h, qa, qb, sel0, sel1);
    v4i ql = {0, 0, 0, 0}, qh = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ql = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], o.lo[i], ql, 0, 0, 0);
      qh = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], o.hi[i], qh, 0, 0, 0);
    }
    const v4f sm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dg, o.m, v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
    const int row = row0 + 16 * rt + n;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int sq = (qh[e] << 3) + ql[e];  // sc = 8 * (sc >> 3) + (sc & 7)
      part[rt][e] = dxv[e] * fmaf(-o.dmin, sm[e], o.d * static_cast<float>(sq));
      if constexpr (SUMS) {
        const int tk = 4 * g + e;
        if (b < nb && row < row_end && tk < ncols) {
          int32_t* out = sums + ((static_cast<size_t>(tk) * n_out + row) * nb + b) * 2;
          out[0] = sq;
          out[1] = static_cast<int>(sm[e]);
        }
      }
    }
  }

  if constexpr (!SUMS) {
    if (b < nb) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[b * kOut + (rt * 4 + e) * 64 + lane] = part[rt][e];
    }
    __syncthreads();
    for (int t = tid; t < kOut; t += 1024) {
      float s = red[t];
      for (int k = 1; k < nb; ++k) s += red[k * kOut + t];
      const int l = t & 63;
      const int row = row0 + 16 * (t >> 8) + (l & 15), tk = 4 * (l >> 4) + ((t >> 6) & 3);
      if (row < row_end && tk < ncols) y[static_cast<size_t>(tk) * n_out + row] = s;
    }
  }
}

template <int RT, bool SUMS>
hipError_t launch_col_kernel(const uint8_t* W, int n_out, int nb, const uint8_t* xq, int ncols, int rows_wg,
                             float* y, int32_t* sums, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  auto k = gemm_q4_K_col<RT, SUMS>;
  unsigned grid = 0;
  if (!launch_grid((static_cast<int64_t>(n_out) + rows_wg - 1) / rows_wg, 1024, &grid))
    return hipErrorInvalidConfiguration;
  // the partial sums, then each wavefront's 16 activation blocks
  const size_t lds = (SUMS ? 0 : static_cast<size_t>(nb) * RT * 256 * 4) + 16 * 16 * kTokImg;
  if (lds > 65536) {
    const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                                hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (attr != hipSuccess) return attr;
  }
  if (e0 != nullptr || e1 != nullptr) {
    hipExtLaunchKernelGGL(k, dim3(grid), dim3(1024), lds, s, e0, e1, 0, W, n_out, nb, xq, ncols, rows_wg, y, sums);
  } else {
    k<<<grid, 1024, lds, s>>>(W, n_out, nb, xq, ncols, rows_wg, y, sums);
  }
  return hipGetLastError();
}

template <int RT>
hipError_t launch_col(const uint8_t* W, int n_out, int nb, const uint8_t* xq, int ncols, int rows_wg, float* y,
                      int32_t* sums, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (sums != nullptr) return launch_col_kernel<RT, true>(W, n_out, nb, xq, ncols, rows_wg, y, sums, s, e0, e1);
  return launch_col_kernel<RT, false>(W, n_out, nb, xq, ncols, rows_wg, y, sums, s, e0, e1);
}

template <int RT, int KS, bool SUMS>
hipError_t launch_res_kernel(const uint8_t* W, int n_out, int nb, const uint8_t* xq, int ncols, float* y,
                             int32_t* sums, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  auto k = gemm_q4_K_res<RT, KS, SUMS>;
  constexpr int rows_wg = 16 * RT;
  unsigned grid = 0;
  if (!launch_grid((static_cast<int64_t>(n_out) + rows_wg - 1) / rows_wg, 64 * RT * KS, &grid))
    return hipErrorInvalidConfiguration;
  // the images of nb superblocks, and room for the K-split partial sums that
  // replace them at the end (more than the images when nb is small)
  constexpr size_t kRed = static_cast<size_t>(KS - 1) * RT * 4 * 64 * 4;
  const size_t images = kZeroBytes + static_cast<size_t>(nb) * kBT;
  const size_t lds = images > kRed ? images : kRed;
  if (lds > 65536) {
    const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                                hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (attr != hipSuccess) return attr;
  }
  if (e0 != nullptr || e1 != nullptr) {
    hipExtLaunchKernelGGL(k, dim3(grid), dim3(64 * RT * KS), lds, s, e0, e1, 0, W, n_out, nb, xq, ncols, rows_wg,
                          y, sums);
  } else {
    k<<<grid, 64 * RT * KS, lds, s>>>(W, n_out, nb, xq, ncols, rows_wg, y, sums);
  }
  return hipGetLastError();
}

template <int RT, int KS>
hipError_t launch_res(const uint8_t* W, int n_out, int nb, const uint8_t* xq, int ncols, float* y, int32_t* sums,
                      hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (sums != nullptr) return launch_res_kernel<RT, KS, true>(W, n_out, nb, xq, ncols, y, sums, s, e0, e1);
  return launch_res_kernel<RT, KS, false>(W, n_out, nb, xq, ncols, y, sums, s, e0, e1);
}

template <class C, bool SUMS>
hipError_t launch_kernel(const uint8_t* W, int n_out, int nb, const uint8_t* xq, int ncols, int rows_wg, float* y,
                         int32_t* sums, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  auto k = gemm_q4_K_mfma<C, SUMS>;
  unsigned grid = 0;
  if (!launch_grid((static_cast<int64_t>(n_out) + rows_wg - 1) / rows_wg, C::kThreads, &grid))
    return hipErrorInvalidConfiguration;
  constexpr size_t lds = C::kLds;
  // above the default dynamic LDS limit: raise it for this kernel on the current
  // device (set on every launch: the library keeps no per-device state)
  const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (attr != hipSuccess) return attr;
  if (e0 != nullptr || e1 != nullptr) {
    hipExtLaunchKernelGGL(k, dim3(grid), dim3(C::kThreads), lds, s, e0, e1, 0, W, n_out, nb, xq, ncols, rows_wg, y,
                          sums);
  } else {
    k<<<grid, C::kThreads, lds, s>>>(W, n_out, nb, xq, ncols, rows_wg, y, sums);
  }
  return hipGetLastError();
}

template <class C>
hipError_t launch_cfg(const uint8_t* W, int n_out, int nb, const uint8_t* xq, int ncols, int rows_wg, float* y,
                      int32_t* sums, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (sums != nullptr) return launch_kernel<C, true>(W, n_out, nb, xq, ncols, rows_wg, y, sums, s, e0, e1);
  return launch_kernel<C, false>(W, n_out, nb, xq, ncols, rows_wg, y, sums, s, e0, e1);
}

template <int NT, int KS1, int KS2, int KS4, int P, int KC24 = 16 / NT>
hipError_t launch_nt(int rt, const uint8_t* W, int n_out, int nb, const uint8_t* xq, int ncols, int rows_wg,
                     float* y, int32_t* sums, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (rt == 1) return launch_cfg<Cfg<NT, 1, KS1, P>>(W, n_out, nb, xq, ncols, rows_wg, y, sums, s, e0, e1);
  if (rt == 2) return launch_cfg<Cfg<NT, 2, KS2, P, 4, KC24>>(W, n_out, nb, xq, ncols, rows_wg, y, sums, s, e0, e1);
  return launch_cfg<Cfg<NT, 4, KS4, P, 4, KC24>>(W, n_out, nb, xq, ncols, rows_wg, y, sums, s, e0, e1);
}

}  // namespace

hipError_t launch_gemm_q4K(const uint8_t* W, int64_t n_out, int64_t n_in, const uint8_t* xq,
                           int64_t ncols, float* y, int32_t* sums, hipStream_t s, hipEvent_t e0,
                           hipEvent_t e1) {
  if (ncols < 1 || ncols > kGemmMaxCols) return hipErrorInvalidValue;
  const int nb = static_cast<int>(n_in / 256);
  const int n = static_cast<int>(n_out), nc = static_cast<int>(ncols);
  // Rows per workgroup: a multiple of 8 that spreads the rows over about 256
  // workgroups (one per CU: 14336 rows -> 56, 4096 -> 16), at most 64; the row
  // tiles of a workgroup cover them (a last tile may hold fewer than 16 rows).
  const int64_t r0 = 8 * ((n_out + 2047) / 2048);
  const int rt = r0 <= 16 ? 1 : (r0 <= 32 ? 2 : 4);
  const int rows_wg = static_cast<int>(r0 < 16 * rt ? r0 : 16 * rt);
  // 8 compute wavefronts per workgroup (4 for 32 or more tokens on one row tile),
  // splitting each row tile's superblocks, plus 4 staging wavefronts; 2 (up to 16
  // tokens) or 4 superblocks of weights in flight per compute wavefront (measured
  // on 14336 x 4096: 16 tokens 11.8 us with 2 against 12.6 with 4 and 13.5 with 8;
  // 64 tokens 20.7 us with 4 against 22.1 with 2 and 22.6 with 8).  Up to 16
  // tokens on two or four row tiles the activations go in chunks of 4 superblocks,
  // so the products start after a quarter of the staging (14336 x 4096: 11.1
  // against 11.7 us with whole 16-superblock chunks; 2-superblock chunks 12.9);
  // one row tile keeps 16-superblock chunks and 8 K-split wavefronts (4096 x 11008:
  // 12.2 against 13.8 us)
  // Up to 16 tokens on short matrices (under 400 16-row tiles, rows of at most 16
  // superblocks): the LDS-resident kernel, one row tile per workgroup split over
  // 16 K-split wavefronts (4096 x 4096 at 16 / 8 columns: 6.9 / 5.4 against 7.6 /
  // 6.0 us).  On taller matrices its products, all after the one staging barrier,
  // no longer hide under the weight stream (14336 x 4096 at 16 columns: 14.3
  // against 11.1 us with 4 row tiles per workgroup), and the kernel below wins.
  if (nc <= 16 && nb <= 16 && (n_out + 15) / 16 < 400)
    return launch_res<1, 16>(W, n, nb, xq, nc, y, sums, s, e0, e1);
  // Up to 16 tokens on taller matrices with rows of at most 16 superblocks: one
  // superblock per wavefront, no staging barrier (14336 / 11008 / 8192 x 4096 at 16
  // columns: 10.3 / 8.9 / 7.2 against 11.2 / 10.7 / 8.5 us with the chunked kernel
  // below; loading each lane's operand pieces from global memory directly, 10.7 / 9.4
  // / 7.8 us, its many 32-byte requests stalling the address unit; staging the
  // activations in LDS for the whole workgroup, with the one barrier that needs,
  // 13.3 us on 14336 x 4096).
  if (nc <= 16 && nb <= 16 && rt > 1) {
    const int tiles = (rows_wg + 15) / 16;  // 2, 3 or 4
    if (tiles == 2) return launch_col<2>(W, n, nb, xq, nc, rows_wg, y, sums, s, e0, e1);
    if (tiles == 3) return launch_col<3>(W, n, nb, xq, nc, rows_wg, y, sums, s, e0, e1);
    return launch_col<4>(W, n, nb, xq, nc, rows_wg, y, sums, s, e0, e1);
  }
  if (nc <= 16) return launch_nt<1, 8, 4, 2, 2, 4>(rt, W, n, nb, xq, nc, rows_wg, y, sums, s, e0, e1);
  if (nc <= 32) return launch_nt<2, 8, 4, 2, 4>(rt, W, n, nb, xq, nc, rows_wg, y, sums, s, e0, e1);
  return launch_nt<4, 4, 4, 2, 4>(rt, W, n, nb, xq, nc, rows_wg, y, sums, s, e0, e1);
}

}  // namespace qk
