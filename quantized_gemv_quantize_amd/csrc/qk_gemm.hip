// qk_gemm.hip - batched Q4_K x Q8_K product (2..64 activation columns per launch)
// on the gfx950 int8 matrix cores.
//
// Same method as the GEMV (rml "Quantized dot products"; candle formats page,
// BlockQ4K / BlockQ8K): for every (token t, row r, superblock b) the exact int32
//   S_q = sum_j sc_j * s_j,  s_j = sum_{e in sub-block j} q_e a_e   (32 elements)
//   S_m = sum_j m_j * sum_{e in j} a_e
// and y[t][r] accumulates (dx * d) * S_q - (dx * dmin) * S_m in f32.  With many
// tokens the code products are a dense contraction, so they run on MFMA:
//   - s_j for a 16-token x 16-row tile is one v_mfma_i32_16x16x32_i8 (K = one
//     sub-block); each lane then adds sc_j * s_j with v_mad_i32_i24 (exact);
//   - S_m is a K = 256 int8 contraction of the activations with m_j repeated over
//     sub-block j (m_j <= 63 fits int8): four v_mfma_i32_16x16x64_i8 per tile.
// Operand layout (checked on the hardware): A = activations, lane l holds token
// l % 16 and k-slot group l / 16; B = weights, lane l holds row l % 16 and the same
// k-slot group; D[token][row] lands in lane row + 16 * (token / 4), element
// token % 4, so the four outputs of a lane share one weight row and its scales.
// k-slot group g of sub-block 2c is elements 64c + 8g .. +7 (low nibbles of
// qs[32c + 8g .. +7]); of sub-block 2c+1 it is elements 64c + 32 + 8g .. +7 (high
// nibbles of the same bytes).  For the K = 64 instruction the same byte of A and
// of B always meets the same k slot, so any consistent grouping gives the sum.
//
// Data movement: a workgroup (4 wavefronts) owns 32 rows and all columns.  Per
// stage it copies KSP superblocks of those rows (whole 144-byte blocks) and of
// every activation column (256 codes + d) from HBM / L2 into LDS with contiguous
// 16-byte loads, double-buffered so the next stage's loads are in flight while
// the current one is multiplied.  Wavefront w takes row tile w & 1; the other bit
// selects either its token tiles or (KSP = 2, 16 columns) its superblock of the
// stage, the two superblock halves being added in LDS at the end.
// LDS row strides are odd multiples of 16 bytes, so the 16 rows (tokens) a
// wavefront reads at one offset fall in distinct banks.
#include <hip/hip_ext.h>

#include "qk_device.h"
#include "qk_internal.h"

namespace qk {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));  // register-friendly 16 bytes

constexpr uint32_t kLo4 = 0x0F0F0F0Fu;
constexpr uint32_t kHi2 = 0x30303030u;
constexpr int kRows = 32;       // rows per workgroup (two 16-row tiles)
constexpr int kAStride = 272;   // LDS bytes per staged activation column (256 codes + pad)

__device__ __forceinline__ long as_long(uint2 v) {
  long r;
  __builtin_memcpy(&r, &v, 8);
  return r;
}
__device__ __forceinline__ v4i as_v4i(uint2 lo, uint2 hi) {
  v4i r;
  r[0] = static_cast<int>(lo.x);
  r[1] = static_cast<int>(lo.y);
  r[2] = static_cast<int>(hi.x);
  r[3] = static_cast<int>(hi.y);
  return r;
}
// 16 bytes at a 4-byte aligned global address (Q8_K codes start 4 bytes into the block)
__device__ __forceinline__ u4 load_a4x4(const uint8_t* p) {
  const uint32_t* p4 = reinterpret_cast<const uint32_t*>(__builtin_assume_aligned(p, 4));
  u4 v;
  __builtin_memcpy(&v, p4, 16);
  return v;
}

// Stage geometry: KSP superblocks of kRows weight rows and of 16 * NT columns.
template <int NT, int KSP>
struct Stage {
  static constexpr int kTok = 16 * NT;
  static constexpr int kWStride = (KSP == 1) ? 144 : 304;  // bytes per row: KSP * 144, padded
  static constexpr int kWBytes = kRows * kWStride;
  static constexpr int kABytes = KSP * kTok * kAStride;
  static constexpr int kDBytes = KSP * kTok * 4;
  static constexpr int kBytes = kWBytes + kABytes + kDBytes;
  static constexpr int kWPieces = kRows * KSP * 9;                       // 16-byte pieces
  static constexpr int kWPerThread = (kWPieces + 255) / 256;
  static constexpr int kAPerThread = KSP * kTok * 16 / 256;             // exact
};

template <int NT, int KSP>
struct Prefetch {
  u4 w[Stage<NT, KSP>::kWPerThread];
  u4 a[Stage<NT, KSP>::kAPerThread];
  float dx;
};

// Global -> registers for the stage starting at superblock b.
template <int NT, int KSP>
__device__ __forceinline__ Prefetch<NT, KSP> stage_load(const uint8_t* __restrict__ W,
                                           size_t wrow, int row0, int n_out, int nb,
                                           const uint8_t* __restrict__ xq, uint32_t xrow, int ncols,
                                           int b) {
  using S = Stage<NT, KSP>;
  const int tid = threadIdx.x;
  Prefetch<NT, KSP> pf;
#pragma unroll
  for (int k = 0; k < S::kWPerThread; ++k) {
    // pieces past the stage, or of a superblock past the row end, load a valid
    // block of the same row instead (never read from LDS)
    const int p = min(tid + 256 * k, S::kWPieces - 1);
    const int row = p / (9 * KSP), rem = p % (9 * KSP);
    const int sb = min(b + rem / 9, nb - 1);
    const size_t off = static_cast<size_t>(min(row0 + row, n_out - 1)) * wrow +
                       static_cast<size_t>(sb) * kQ4_KBytes + (rem % 9) * 16;
    pf.w[k] = *reinterpret_cast<const u4*>(W + off);
  }
#pragma unroll
  for (int k = 0; k < S::kAPerThread; ++k) {
    const int p = tid + 256 * k;
    const int piece = p & 15, col = (p >> 4) % S::kTok, kk = (p >> 4) / S::kTok;
    const uint32_t off = static_cast<uint32_t>(min(col, ncols - 1)) * xrow +
                         static_cast<uint32_t>(min(b + kk, nb - 1) * kQ8_KBytes) + 4 + piece * 16;
    pf.a[k] = load_a4x4(xq + off);
  }
  {
    const int t = min(tid, KSP * S::kTok - 1);
    const int col = t % S::kTok, kk = t / S::kTok;
    const uint32_t off = static_cast<uint32_t>(min(col, ncols - 1)) * xrow +
                         static_cast<uint32_t>(min(b + kk, nb - 1) * kQ8_KBytes);
    pf.dx = *reinterpret_cast<const float*>(xq + off);
  }
  return pf;
}

// Registers -> LDS stage buffer.
template <int NT, int KSP>
__device__ __forceinline__ void stage_store(const Prefetch<NT, KSP>& pf, uint8_t* lds) {
  using S = Stage<NT, KSP>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < S::kWPerThread; ++k) {
    const int p = tid + 256 * k;
    if (p < S::kWPieces) {
      const int row = p / (9 * KSP), rem = p % (9 * KSP);
      *reinterpret_cast<u4*>(lds + row * S::kWStride + rem * 16) = pf.w[k];
    }
  }
#pragma unroll
  for (int k = 0; k < S::kAPerThread; ++k) {
    const int p = tid + 256 * k;
    const int piece = p & 15, colk = p >> 4;  // colk = kk * kTok + col
    *reinterpret_cast<u4*>(lds + S::kWBytes + colk * kAStride + piece * 16) = pf.a[k];
  }
  if (tid < KSP * S::kTok) *reinterpret_cast<float*>(lds + S::kWBytes + S::kABytes + tid * 4) = pf.dx;
}

// NT = 16-column tiles in the launch, TW = tiles per wavefront, KSP = superblocks
// per stage (one per wavefront pair).  Supported: (1,1,2), (2,1,1), (4,2,1).
template <int NT, int TW, int KSP, bool SUMS>
__global__ __launch_bounds__(256) void gemm_q4_K_mfma(const uint8_t* __restrict__ W, int n_out,
                                                      int nb, const uint8_t* __restrict__ xq,
                                                      int ncols, float* __restrict__ y,
                                                      int32_t* __restrict__ sums) {
  static_assert(KSP * (NT / TW) == 2, "four wavefronts: two row tiles x two slices");
  using S = Stage<NT, KSP>;
  extern __shared__ __align__(16) uint8_t lds[];

  const int lane = threadIdx.x & 63;
  const int n = lane & 15;  // weight row in the tile; token in the A operand
  const int g = lane >> 4;  // k-slot group; the lane's outputs are tokens 4g .. 4g+3
  const int w = wave_id();
  const int rt = w & 1;                       // row tile
  const int kh = (KSP == 2) ? (w >> 1) : 0;   // superblock of the stage
  const int tg = (KSP == 2) ? 0 : (w >> 1);   // token-tile group
  const int row0 = blockIdx.x * kRows;
  const int row = row0 + 16 * rt + n;
  const size_t wrow = static_cast<size_t>(nb) * kQ4_KBytes;
  const uint32_t xrow = static_cast<uint32_t>(nb) * kQ8_KBytes;

  float acc[TW][4];
#pragma unroll
  for (int t = 0; t < TW; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[t][i] = 0.0f;

  const int nstage = (nb + KSP - 1) / KSP;
  Prefetch<NT, KSP> pf = stage_load<NT, KSP>(W, wrow, row0, n_out, nb, xq, xrow, ncols, 0);
  stage_store<NT, KSP>(pf, lds);
  __syncthreads();

  for (int s = 0; s < nstage; ++s) {
    uint8_t* cur = lds + (s & 1) * S::kBytes;
    if (s + 1 < nstage) pf = stage_load<NT, KSP>(W, wrow, row0, n_out, nb, xq, xrow, ncols, (s + 1) * KSP);
    const int b = s * KSP + kh;
    if (b < nb) {
      const uint8_t* wl = cur + (16 * rt + n) * S::kWStride + kh * 144;
      const uint4 h = *reinterpret_cast<const uint4*>(wl);
      // 6-bit scales and mins of the 8 sub-blocks (get_scale_min_k4)
      const uint32_t sc_a = h.y & 0x3F3F3F3Fu, m_a = h.z & 0x3F3F3F3Fu;
      const uint32_t sc_b = (h.w & kLo4) | ((h.y >> 2) & kHi2);
      const uint32_t m_b = ((h.w >> 4) & kLo4) | ((h.z >> 2) & kHi2);
      int sc[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sc[j] = __builtin_amdgcn_ubfe(sc_a, 8 * j, 8);
        sc[j + 4] = __builtin_amdgcn_ubfe(sc_b, 8 * j, 8);
      }
      uint2 lo[4], hi[4];
      v4i mB[4];  // m_{2c} in bytes 0..7, m_{2c+1} in bytes 8..15
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint2 q = *reinterpret_cast<const uint2*>(wl + 16 + 32 * c + 8 * g);
        lo[c] = make_uint2(q.x & kLo4, q.y & kLo4);
        hi[c] = make_uint2((q.x >> 4) & kLo4, (q.y >> 4) & kLo4);
        const uint32_t mw = (c < 2) ? m_a : m_b;
        const uint32_t m0 = __builtin_amdgcn_ubfe(mw, 16 * (c & 1), 8) * 0x01010101u;
        const uint32_t m1 = __builtin_amdgcn_ubfe(mw, 16 * (c & 1) + 8, 8) * 0x01010101u;
        mB[c][0] = static_cast<int>(m0);
        mB[c][1] = static_cast<int>(m0);
        mB[c][2] = static_cast<int>(m1);
        mB[c][3] = static_cast<int>(m1);
      }
      const float d = f16_to_f32(h.x & 0xFFFF);
      const float dmin = f16_to_f32(h.x >> 16);

#pragma unroll
      for (int t = 0; t < TW; ++t) {
        const int tt = tg * TW + t;  // token tile
        const uint8_t* al = cur + S::kWBytes + (kh * S::kTok + 16 * tt + n) * kAStride;
        const float4 dx4 = *reinterpret_cast<const float4*>(cur + S::kWBytes + S::kABytes +
                                                            (kh * S::kTok + 16 * tt + 4 * g) * 4);
        const float dx[4] = {dx4.x, dx4.y, dx4.z, dx4.w};
        v4i sq = {0, 0, 0, 0};
        v4i sm = {0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint2 alo = *reinterpret_cast<const uint2*>(al + 64 * c + 8 * g);
          const uint2 ahi = *reinterpret_cast<const uint2*>(al + 64 * c + 32 + 8 * g);
          const v4i z = {0, 0, 0, 0};
          const v4i s0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(as_long(alo), as_long(lo[c]), z, 0, 0, 0);
          const v4i s1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(as_long(ahi), as_long(hi[c]), z, 0, 0, 0);
          sm = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_v4i(alo, ahi), mB[c], sm, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) sq[i] = mad24(sc[2 * c], s0[i], mad24(sc[2 * c + 1], s1[i], sq[i]));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[t][i] += (dx[i] * d) * static_cast<float>(sq[i]) - (dx[i] * dmin) * static_cast<float>(sm[i]);
          if constexpr (SUMS) {
            const int tk = 16 * tt + 4 * g + i;
            if (row < n_out && tk < ncols) {
              int32_t* o = sums + ((static_cast<size_t>(tk) * n_out + row) * nb + b) * 2;
              o[0] = sq[i];
              o[1] = sm[i];
            }
          }
        }
      }
    }
    if (s + 1 < nstage) stage_store<NT, KSP>(pf, lds + ((s + 1) & 1) * S::kBytes);
    __syncthreads();
  }

  if constexpr (!SUMS) {
    float* red = reinterpret_cast<float*>(lds);
    if constexpr (KSP == 2) {
      // superblock halves: wavefronts 2, 3 hand their sums to wavefronts 0, 1
      if (kh == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) red[(rt * 4 + i) * 64 + lane] = acc[0][i];
      }
      __syncthreads();
      if (kh == 1) return;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[0][i] += red[(rt * 4 + i) * 64 + lane];
    }
    if (row < n_out) {
#pragma unroll
      for (int t = 0; t < TW; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tk = 16 * (tg * TW + t) + 4 * g + i;
          if (tk < ncols) y[static_cast<size_t>(tk) * n_out + row] = acc[t][i];
        }
    }
  }
}

template <int NT, int TW, int KSP>
hipError_t launch_cfg(const uint8_t* W, int n_out, int nb, const uint8_t* xq, int ncols, float* y,
                      int32_t* sums, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const unsigned grid = static_cast<unsigned>((n_out + kRows - 1) / kRows);
  const size_t lds = 2 * Stage<NT, KSP>::kBytes;
  if (sums != nullptr) {
    auto k = gemm_q4_K_mfma<NT, TW, KSP, true>;
    if (e0 != nullptr || e1 != nullptr) {
      hipExtLaunchKernelGGL(k, dim3(grid), dim3(256), lds, s, e0, e1, 0, W, n_out, nb, xq, ncols, y, sums);
    } else {
      k<<<grid, 256, lds, s>>>(W, n_out, nb, xq, ncols, y, sums);
    }
  } else {
    auto k = gemm_q4_K_mfma<NT, TW, KSP, false>;
    if (e0 != nullptr || e1 != nullptr) {
      hipExtLaunchKernelGGL(k, dim3(grid), dim3(256), lds, s, e0, e1, 0, W, n_out, nb, xq, ncols, y, sums);
    } else {
      k<<<grid, 256, lds, s>>>(W, n_out, nb, xq, ncols, y, sums);
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_q4K(const uint8_t* W, int64_t n_out, int64_t n_in, const uint8_t* xq,
                           int64_t ncols, float* y, int32_t* sums, hipStream_t s, hipEvent_t e0,
                           hipEvent_t e1) {
  const int nb = static_cast<int>(n_in / 256);
  const int n = static_cast<int>(n_out), nc = static_cast<int>(ncols);
  if (nc <= 16) return launch_cfg<1, 1, 2>(W, n, nb, xq, nc, y, sums, s, e0, e1);
  if (nc <= 32) return launch_cfg<2, 1, 1>(W, n, nb, xq, nc, y, sums, s, e0, e1);
  if (nc <= 64) return launch_cfg<4, 2, 1>(W, n, nb, xq, nc, y, sums, s, e0, e1);
  return hipErrorInvalidValue;
}

}  // namespace qk
