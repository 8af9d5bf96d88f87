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
// Work split: a workgroup of 4 wavefronts owns R 16-row tiles; wavefront w takes
// superblocks w, w + 4, ...  The activation registers of a superblock are reused
// for all R row tiles; the weights are read from HBM exactly once.  The four
// partial sums of each output are added in LDS at the end.
#include <hip/hip_ext.h>

#include "qk_device.h"
#include "qk_internal.h"

namespace qk {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr uint32_t kLo4 = 0x0F0F0F0Fu;
constexpr uint32_t kHi2 = 0x30303030u;
constexpr int kSplit = 4;  // wavefronts per workgroup, each a slice of the superblocks

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
template <typename T>
__device__ __forceinline__ T ld4(const uint8_t* p) {  // field with 4-byte alignment
  const uint32_t* p4 = reinterpret_cast<const uint32_t*>(__builtin_assume_aligned(p, 4));
  T v;
  __builtin_memcpy(&v, p4, sizeof(T));
  return v;
}

// The part of one Q4_K superblock that lane (row n, group g) needs: the 16-byte
// header (d, dmin, 12 scale bytes) and 8 qs bytes of each 64-element chunk.
struct WPart {
  uint4 h;
  uint2 q[4];
};

__device__ __forceinline__ WPart load_wpart(const uint8_t* blk, int g) {
  WPart v;
  v.h = *reinterpret_cast<const uint4*>(blk);
#pragma unroll
  for (int c = 0; c < 4; ++c) v.q[c] = *reinterpret_cast<const uint2*>(blk + 16 + 32 * c + 8 * g);
  return v;
}

template <int NT, int R, bool SUMS>
__global__ __launch_bounds__(256) void gemm_q4_K_mfma(const uint8_t* __restrict__ W, int n_out,
                                                      int nb, const uint8_t* __restrict__ xq,
                                                      int ncols, float* __restrict__ y,
                                                      int32_t* __restrict__ sums) {
  constexpr int K = R * NT * 4;  // outputs per lane
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;  // weight row in the tile; token in the A operand
  const int g = lane >> 4;  // k-slot group; the lane's outputs are tokens 4g .. 4g+3
  const int w = wave_id();
  const int row0 = blockIdx.x * (16 * R);
  const size_t wrow = static_cast<size_t>(nb) * kQ4_KBytes;
  const uint32_t xrow = static_cast<uint32_t>(nb) * kQ8_KBytes;  // bytes per activation column

  const uint8_t* wr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) wr[r] = W + static_cast<size_t>(min(row0 + 16 * r + n, n_out - 1)) * wrow;
  uint32_t xa[NT];     // A operand column of this lane, per token tile
  uint32_t xd[NT][4];  // columns of the lane's four outputs, per token tile
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    xa[t] = static_cast<uint32_t>(min(16 * t + n, ncols - 1)) * xrow;
#pragma unroll
    for (int i = 0; i < 4; ++i) xd[t][i] = static_cast<uint32_t>(min(16 * t + 4 * g + i, ncols - 1)) * xrow;
  }

  float acc[R][NT][4];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[r][t][i] = 0.0f;

  for (int b = w; b < nb; b += kSplit) {
    WPart wp[R];
#pragma unroll
    for (int r = 0; r < R; ++r) wp[r] = load_wpart(wr[r] + static_cast<uint32_t>(b * kQ4_KBytes), g);
    const uint8_t* xb = xq + static_cast<uint32_t>(b * kQ8_KBytes);
    uint2 alo[NT][4], ahi[NT][4];
    float dx[NT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        alo[t][c] = ld4<uint2>(xb + xa[t] + 4 + 64 * c + 8 * g);
        ahi[t][c] = ld4<uint2>(xb + xa[t] + 4 + 64 * c + 32 + 8 * g);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) dx[t][i] = ld4<float>(xb + xd[t][i]);
    }

#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint4 h = wp[r].h;
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
        const uint2 q = wp[r].q[c];
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
      for (int t = 0; t < NT; ++t) {
        v4i sq = {0, 0, 0, 0};
        v4i sm = {0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const v4i z = {0, 0, 0, 0};
          const v4i s0 =
              __builtin_amdgcn_mfma_i32_16x16x32_i8(as_long(alo[t][c]), as_long(lo[c]), z, 0, 0, 0);
          const v4i s1 =
              __builtin_amdgcn_mfma_i32_16x16x32_i8(as_long(ahi[t][c]), as_long(hi[c]), z, 0, 0, 0);
          sm = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_v4i(alo[t][c], ahi[t][c]), mB[c], sm, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) sq[i] = mad24(sc[2 * c], s0[i], mad24(sc[2 * c + 1], s1[i], sq[i]));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[r][t][i] += (dx[t][i] * d) * static_cast<float>(sq[i]) -
                          (dx[t][i] * dmin) * static_cast<float>(sm[i]);
          if constexpr (SUMS) {
            const int row = row0 + 16 * r + n, tk = 16 * t + 4 * g + i;
            if (row < n_out && tk < ncols) {
              int32_t* o = sums + ((static_cast<size_t>(tk) * n_out + row) * nb + b) * 2;
              o[0] = sq[i];
              o[1] = sm[i];
            }
          }
        }
      }
    }
  }

  if constexpr (!SUMS) {
    // add the kSplit partial sums of every output, then store
    __shared__ float red[kSplit][K][64];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[w][(r * NT + t) * 4 + i][lane] = acc[r][t][i];
    __syncthreads();
    for (int k = w; k < K; k += kSplit) {
      float s = red[0][k][lane];
#pragma unroll
      for (int v = 1; v < kSplit; ++v) s += red[v][k][lane];
      const int r = k / (4 * NT), t = (k / 4) % NT, i = k % 4;
      const int row = row0 + 16 * r + n, tk = 16 * t + 4 * g + i;
      if (row < n_out && tk < ncols) y[static_cast<size_t>(tk) * n_out + row] = s;
    }
  }
}

template <int NT, int R, bool SUMS>
hipError_t launch_mfma(const uint8_t* W, int n_out, int nb, const uint8_t* xq, int ncols, float* y,
                       int32_t* sums, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const unsigned grid = static_cast<unsigned>((n_out + 16 * R - 1) / (16 * R));
  if (e0 != nullptr || e1 != nullptr) {
    hipExtLaunchKernelGGL(gemm_q4_K_mfma<NT, R, SUMS>, dim3(grid), dim3(64 * kSplit), 0, s, e0, e1, 0,
                          W, n_out, nb, xq, ncols, y, sums);
  } else {
    gemm_q4_K_mfma<NT, R, SUMS><<<grid, 64 * kSplit, 0, s>>>(W, n_out, nb, xq, ncols, y, sums);
  }
  return hipGetLastError();
}

template <int NT>
hipError_t launch_nt(const uint8_t* W, int n_out, int nb, const uint8_t* xq, int ncols, float* y,
                     int32_t* sums, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  constexpr int R = 2;
  if (sums != nullptr) return launch_mfma<NT, R, true>(W, n_out, nb, xq, ncols, y, sums, s, e0, e1);
  return launch_mfma<NT, R, false>(W, n_out, nb, xq, ncols, y, sums, s, e0, e1);
}

}  // namespace

hipError_t launch_gemm_q4K(const uint8_t* W, int64_t n_out, int64_t n_in, const uint8_t* xq,
                           int64_t ncols, float* y, int32_t* sums, hipStream_t s, hipEvent_t e0,
                           hipEvent_t e1) {
  const int nb = static_cast<int>(n_in / 256);
  const int n = static_cast<int>(n_out), nc = static_cast<int>(ncols);
  switch ((nc + 15) / 16) {
    case 1: return launch_nt<1>(W, n, nb, xq, nc, y, sums, s, e0, e1);
    case 2: return launch_nt<2>(W, n, nb, xq, nc, y, sums, s, e0, e1);
    case 3: return launch_nt<3>(W, n, nb, xq, nc, y, sums, s, e0, e1);
    case 4: return launch_nt<4>(W, n, nb, xq, nc, y, sums, s, e0, e1);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qk
