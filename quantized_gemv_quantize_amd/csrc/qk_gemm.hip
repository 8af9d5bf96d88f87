// qk_gemm.hip - batched Q4_K x Q8_K product (2..64 activation columns per launch)
// on the gfx950 int8 matrix cores.
//
// Same method as the GEMV (rml "Quantized dot products"; candle formats page,
// BlockQ4K / BlockQ8K): for every (token t, row r, superblock b) the exact int32
//   S_q = sum_j sc_j * s_j,  s_j = sum_{e in sub-block j} q_e a_e   (32 elements)
//   S_m = sum_j m_j * sum_{e in j} a_e
// and y[t][r] accumulates (dx * d) * S_q - (dx * dmin) * S_m in f32.  With many tokens
// the code products are a dense contraction, so they run on MFMA
// (v_mfma_i32_16x16x64_i8, K = one 64-element chunk = two sub-blocks):
//   - the 6-bit scale goes into the weight operand, split as sc = 8 * (sc >> 3) +
//     (sc & 7): the bytes q * (sc & 7) and q * (sc >> 3) are at most 105, so both
//     are int8 operands, and S_q = 8 * Q_hi + Q_lo where Q_hi, Q_lo accumulate
//     over the superblock's four chunks inside the matrix core (exact int32);
//   - S_m is the same contraction against m_j repeated over sub-block j (m <= 63).
// Three MFMAs per chunk and tile, no per-sub-block integer work on the VALU.
// Operand layout (checked on the hardware): A = activations, lane l holds token
// l % 16 and k-slot group l / 16; B = weights, lane l holds row l % 16 and the same
// k-slot group; D[token][row] lands in lane row + 16 * (token / 4), element
// token % 4, so the four outputs of a lane share one weight row and its scales.
// In chunk c, lane group g holds bytes 0-7 = elements 64c + 8g .. +7 of sub-block
// 2c (low nibbles of qs[32c + 8g .. +7]) and bytes 8-15 = elements 64c + 32 + 8g
// .. +7 of sub-block 2c+1 (high nibbles of the same bytes).  The same byte of A and
// of B always meets the same k slot, so this grouping gives the full sum.
//
// Data movement: a workgroup owns RT 16-row tiles and all columns.  Per stage it
// copies KSP superblocks of those rows (whole 144-byte blocks) and of every
// activation column (256 codes + d) from HBM / L2 into LDS with contiguous 16-byte
// loads; the loads run two stages ahead of the multiply and each stage is written
// to LDS one stage ahead of its use (two buffers).  The workgroup has
// RT x (NT / TW) x KSP wavefronts: a row tile, a group of TW token tiles and one
// superblock of the stage each; the KSP partial sums of an output are added in
// LDS at the end, always in the same order.  A wavefront that holds all token
// tiles (TW = NT) builds each scaled weight operand once per superblock.  LDS row strides are 8 bytes more
// than a multiple of 16, so the 16 rows (tokens) that a wavefront reads at one
// offset fall in different bank pairs.
#include <hip/hip_ext.h>

#include "qk_device.h"
#include "qk_internal.h"

namespace qk {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));  // register-friendly 16 bytes
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kLo4 = 0x0F0F0F0Fu;
constexpr uint32_t kHi2 = 0x30303030u;
constexpr int kAStride = 264;   // LDS bytes per staged activation column (256 codes + pad)

__device__ __forceinline__ v4i as_v4i(uint2 lo, uint2 hi) {
  v4i r;
  r[0] = static_cast<int>(lo.x);
  r[1] = static_cast<int>(lo.y);
  r[2] = static_cast<int>(hi.x);
  r[3] = static_cast<int>(hi.y);
  return r;
}
// Byte j of x in both 16-bit halves (v_perm_b32; selector 12 gives a zero byte).
__device__ __forceinline__ uint32_t bcast16(uint32_t x, uint32_t j) {
  return __builtin_amdgcn_perm(x, x, j * 0x00010001u + 0x0C000C00u);
}
// Each byte of x times the small factor s held in both halves of s2 (packed 16-bit
// multiply): every product stays below 256 (codes <= 15, factor <= 7), so no
// byte carries into its neighbour.
__device__ __forceinline__ uint32_t mul_bytes(uint32_t x, uint32_t s2) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, x) * __builtin_bit_cast(u16x2, s2));
}
// 16 bytes to / from LDS at an 8-byte aligned address (rows padded to 8 bytes).
__device__ __forceinline__ void lds_store16(uint8_t* p, u4 v) {
  uint2* q = reinterpret_cast<uint2*>(__builtin_assume_aligned(p, 8));
  q[0] = make_uint2(v[0], v[1]);
  q[1] = make_uint2(v[2], v[3]);
}
__device__ __forceinline__ uint4 lds_load16(const uint8_t* p) {
  const uint2* q = reinterpret_cast<const uint2*>(__builtin_assume_aligned(p, 8));
  const uint2 a = q[0], b = q[1];
  return make_uint4(a.x, a.y, b.x, b.y);
}
// 16 bytes at a 4-byte aligned global address (Q8_K codes start 4 bytes into the block)
__device__ __forceinline__ u4 load_a4x4(const uint8_t* p) {
  const uint32_t* p4 = reinterpret_cast<const uint32_t*>(__builtin_assume_aligned(p, 4));
  u4 v;
  __builtin_memcpy(&v, p4, 16);
  return v;
}

// Launch shape and stage geometry: NT 16-column tiles, TW tiles per wavefront,
// KSP superblocks per stage, RT 16-row tiles per workgroup.
template <int NT_, int TW_, int KSP_, int RT_ = 2>
struct Cfg {
  static constexpr int NT = NT_, TW = TW_, KSP = KSP_, RT = RT_;
  static constexpr int kRows = 16 * RT;                // rows per workgroup
  static constexpr int kTG = NT / TW;                  // token-tile groups
  static constexpr int kWaves = RT * kTG * KSP;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kTok = 16 * NT;
  static constexpr int kWStride = KSP * kQ4_KBytes + 8;  // bytes per staged weight row
  static constexpr int kWBytes = kRows * kWStride;
  static constexpr int kABytes = KSP * kTok * kAStride;
  static constexpr int kDBytes = KSP * kTok * 4;
  static constexpr int kBytes = kWBytes + kABytes + kDBytes;  // one stage buffer
  static constexpr int kWPieces = kRows * KSP * 9;            // 16-byte pieces
  static constexpr int kWPerThread = (kWPieces + kThreads - 1) / kThreads;
  static constexpr int kAPieces = KSP * kTok * 16;
  static constexpr int kAPerThread = kAPieces / kThreads;
  static constexpr int kRedBytes = (KSP - 1) * RT * kTG * TW * 4 * 64 * 4;  // partial sums
  static_assert(NT % TW == 0, "token tiles split evenly over wavefronts");
  static_assert(kAPieces % kThreads == 0, "activation pieces split evenly");
  static_assert(KSP * kTok <= kThreads, "one thread per staged scale");
  static_assert(kBytes % 16 == 0, "stage buffers stay 16-byte aligned");
  static_assert(kRedBytes <= 2 * kBytes, "the final reduction fits the stage buffers");
};

template <class C>
struct Prefetch {
  u4 w[C::kWPerThread];
  u4 a[C::kAPerThread];
  float dx;
};

// What each thread copies in every stage, fixed for the whole kernel: the byte
// offsets of its pieces relative to the stage's first superblock, and where they
// go in the LDS stage buffer.  A stage starting at superblock b adds b * 144 (W)
// or b * 292 (activations).  Pieces of superblocks past the row end (the last
// stage when KSP does not divide the superblock count, and the stages the
// straight-line loop runs past the end) re-read the row's last superblock; they
// are never used.
template <class C>
struct StageMap {
  size_t wsrc[C::kWPerThread];     // row * row_bytes + sub * 144 + piece * 16
  int wsub[C::kWPerThread];        // superblock of the stage the piece belongs to
  int wdst[C::kWPerThread];        // LDS offset, -1 for threads without a piece
  uint32_t asrc[C::kAPerThread];   // column * xrow + sub * 292 + 4 + piece * 16
  int asub[C::kAPerThread];
  uint32_t dsrc;
  int dsub;

  __device__ __forceinline__ StageMap(int row0, int n_out, size_t wrow, int ncols, uint32_t xrow) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int k = 0; k < C::kWPerThread; ++k) {
      const int p0 = tid + C::kThreads * k;
      const int p = min(p0, C::kWPieces - 1);
      const int row = p / (9 * C::KSP), rem = p % (9 * C::KSP);
      wsrc[k] = static_cast<size_t>(min(row0 + row, n_out - 1)) * wrow + rem * 16;
      wsub[k] = rem / 9;
      wdst[k] = (p0 < C::kWPieces) ? row * C::kWStride + rem * 16 : -1;
    }
#pragma unroll
    for (int k = 0; k < C::kAPerThread; ++k) {
      const int p = tid + C::kThreads * k;
      const int piece = p & 15, col = (p >> 4) % C::kTok, kk = (p >> 4) / C::kTok;
      asrc[k] = static_cast<uint32_t>(min(col, ncols - 1)) * xrow + kk * kQ8_KBytes + 4 + piece * 16;
      asub[k] = kk;
    }
    const int t = min(tid, C::KSP * C::kTok - 1);
    dsrc = static_cast<uint32_t>(min(t % C::kTok, ncols - 1)) * xrow + (t / C::kTok) * kQ8_KBytes;
    dsub = t / C::kTok;
  }
};

// Global -> registers for the stage starting at superblock b.  Offsets only
// grow: a piece of a superblock past the row end steps back after b's offset is
// added, never below its own row's start.
template <class C>
__device__ __forceinline__ Prefetch<C> stage_load(const StageMap<C>& m, const uint8_t* __restrict__ W,
                                                  const uint8_t* __restrict__ xq, int nb, int b) {
  const int last = nb - 1 - b;  // last superblock of this stage inside the row (>= 0)
  Prefetch<C> pf;
#pragma unroll
  for (int k = 0; k < C::kWPerThread; ++k) {
    const size_t back = static_cast<size_t>(max(m.wsub[k] - last, 0)) * kQ4_KBytes;
    pf.w[k] = *reinterpret_cast<const u4*>(W + (m.wsrc[k] + static_cast<size_t>(b) * kQ4_KBytes - back));
  }
#pragma unroll
  for (int k = 0; k < C::kAPerThread; ++k) {
    const uint32_t back = static_cast<uint32_t>(max(m.asub[k] - last, 0)) * kQ8_KBytes;
    pf.a[k] = load_a4x4(xq + (m.asrc[k] + static_cast<uint32_t>(b * kQ8_KBytes) - back));
  }
  {
    const uint32_t back = static_cast<uint32_t>(max(m.dsub - last, 0)) * kQ8_KBytes;
    pf.dx = *reinterpret_cast<const float*>(xq + (m.dsrc + static_cast<uint32_t>(b * kQ8_KBytes) - back));
  }
  return pf;
}

// Registers -> LDS stage buffer.
template <class C>
__device__ __forceinline__ void stage_store(const StageMap<C>& m, const Prefetch<C>& pf, uint8_t* lds) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < C::kWPerThread; ++k) {
    if (m.wdst[k] >= 0) lds_store16(lds + m.wdst[k], pf.w[k]);
  }
#pragma unroll
  for (int k = 0; k < C::kAPerThread; ++k) {
    const int p = tid + C::kThreads * k;
    const int piece = p & 15, colk = p >> 4;  // colk = sub * kTok + col
    lds_store16(lds + C::kWBytes + colk * kAStride + piece * 16, pf.a[k]);
  }
  if (tid < C::KSP * C::kTok) *reinterpret_cast<float*>(lds + C::kWBytes + C::kABytes + tid * 4) = pf.dx;
}

template <class C, bool SUMS>
__global__ __launch_bounds__(C::kThreads) void gemm_q4_K_mfma(const uint8_t* __restrict__ W, int n_out,
                                                              int nb, const uint8_t* __restrict__ xq,
                                                              int ncols, float* __restrict__ y,
                                                              int32_t* __restrict__ sums) {
  constexpr int TW = C::TW, KSP = C::KSP;
  extern __shared__ __align__(16) uint8_t lds[];

  const int lane = threadIdx.x & 63;
  const int n = lane & 15;  // weight row in the tile; token in the A operand
  const int g = lane >> 4;  // k-slot group; the lane's outputs are tokens 4g .. 4g+3
  const int w = wave_id();
  const int rt = w % C::RT;               // row tile
  const int tg = (w / C::RT) % C::kTG;   // token-tile group
  const int kh = (w / C::RT) / C::kTG;   // superblock of the stage
  const int row0 = blockIdx.x * C::kRows;
  const int row = row0 + 16 * rt + n;
  const size_t wrow = static_cast<size_t>(nb) * kQ4_KBytes;
  const uint32_t xrow = static_cast<uint32_t>(nb) * kQ8_KBytes;

  float acc[TW][4];
#pragma unroll
  for (int t = 0; t < TW; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[t][i] = 0.0f;

  // multiply the stage in LDS buffer `cur` (stage index s)
  auto compute = [&](const uint8_t* cur, int s) {
    const int b = s * KSP + kh;
    if (b >= nb) return;
    const uint8_t* wl = cur + (16 * rt + n) * C::kWStride + kh * kQ4_KBytes;
    const uint4 h = lds_load16(wl);
    // 6-bit scales and mins of the 8 sub-blocks (get_scale_min_k4)
    const uint32_t sc_a = h.y & 0x3F3F3F3Fu, m_a = h.z & 0x3F3F3F3Fu;
    const uint32_t sc_b = (h.w & kLo4) | ((h.y >> 2) & kHi2);
    const uint32_t m_b = ((h.w >> 4) & kLo4) | ((h.z >> 2) & kHi2);
    // B operands per 64-element chunk c (bytes 0-7: sub-block 2c, low nibbles;
    // bytes 8-15: sub-block 2c+1, high nibbles): the codes times the low three
    // and the high three bits of the sub-block's scale, and the min repeated.
    const uint32_t l3a = sc_a & 0x07070707u, h3a = (sc_a >> 3) & 0x07070707u;
    const uint32_t l3b = sc_b & 0x07070707u, h3b = (sc_b >> 3) & 0x07070707u;
    v4i bl[4], bh[4], mB[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint2 q = *reinterpret_cast<const uint2*>(wl + 16 + 32 * c + 8 * g);
      const uint32_t lo0 = q.x & kLo4, lo1 = q.y & kLo4;
      const uint32_t hi0 = (q.x >> 4) & kLo4, hi1 = (q.y >> 4) & kLo4;
      const uint32_t l3 = (c < 2) ? l3a : l3b, h3 = (c < 2) ? h3a : h3b;
      const uint32_t j0 = 2 * (c & 1), j1 = j0 + 1;  // byte of sub-blocks 2c, 2c+1
      const uint32_t sl0 = bcast16(l3, j0), sl1 = bcast16(l3, j1);
      const uint32_t sh0 = bcast16(h3, j0), sh1 = bcast16(h3, j1);
      bl[c][0] = static_cast<int>(mul_bytes(lo0, sl0));
      bl[c][1] = static_cast<int>(mul_bytes(lo1, sl0));
      bl[c][2] = static_cast<int>(mul_bytes(hi0, sl1));
      bl[c][3] = static_cast<int>(mul_bytes(hi1, sl1));
      bh[c][0] = static_cast<int>(mul_bytes(lo0, sh0));
      bh[c][1] = static_cast<int>(mul_bytes(lo1, sh0));
      bh[c][2] = static_cast<int>(mul_bytes(hi0, sh1));
      bh[c][3] = static_cast<int>(mul_bytes(hi1, sh1));
      const uint32_t mw = (c < 2) ? m_a : m_b;
      const uint32_t m0 = __builtin_amdgcn_perm(mw, mw, 0x01010101u * j0);
      const uint32_t m1 = __builtin_amdgcn_perm(mw, mw, 0x01010101u * j1);
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
      const uint8_t* al = cur + C::kWBytes + (kh * C::kTok + 16 * tt + n) * kAStride;
      const float4 dx4 = *reinterpret_cast<const float4*>(cur + C::kWBytes + C::kABytes +
                                                          (kh * C::kTok + 16 * tt + 4 * g) * 4);
      const float dx[4] = {dx4.x, dx4.y, dx4.z, dx4.w};
      v4i ql = {0, 0, 0, 0}, qh = {0, 0, 0, 0}, sm = {0, 0, 0, 0};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint2 alo = *reinterpret_cast<const uint2*>(al + 64 * c + 8 * g);
        const uint2 ahi = *reinterpret_cast<const uint2*>(al + 64 * c + 32 + 8 * g);
        const v4i a = as_v4i(alo, ahi);
        ql = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bl[c], ql, 0, 0, 0);
        qh = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bh[c], qh, 0, 0, 0);
        sm = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, mB[c], sm, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int sq = (qh[i] << 3) + ql[i];  // sc = 8 * (sc >> 3) + (sc & 7)
        acc[t][i] += (dx[i] * d) * static_cast<float>(sq) - (dx[i] * dmin) * static_cast<float>(sm[i]);
        if constexpr (SUMS) {
          const int tk = 16 * tt + 4 * g + i;
          if (row < n_out && tk < ncols) {
            int32_t* o = sums + ((static_cast<size_t>(tk) * n_out + row) * nb + b) * 2;
            o[0] = sq;
            o[1] = sm[i];
          }
        }
      }
    }
  };

  // Global loads run two stages ahead of the multiply: two register sets
  // alternate (the loop is unrolled by two so each set has a fixed name), and
  // each stage is written to LDS one stage ahead of its use.  The body is
  // straight-line: loads of stages past the end re-read the row's last superblock
  // (stage_load clamps) and those stages multiply nothing, so no load sits under a
  // condition and the compiler's wait counts cover only the older register set.
  const int nstage = (nb + KSP - 1) / KSP;
  const int nstage2 = (nstage + 1) & ~1;
  const StageMap<C> map(row0, n_out, wrow, ncols, xrow);
  uint8_t* even = lds;               // stages 0, 2, 4, ...
  uint8_t* odd = lds + C::kBytes;    // stages 1, 3, 5, ...
  Prefetch<C> pa = stage_load<C>(map, W, xq, nb, 0);
  Prefetch<C> pb = stage_load<C>(map, W, xq, nb, KSP);
  stage_store<C>(map, pa, even);
  __syncthreads();
  for (int s = 0; s < nstage2; s += 2) {
    pa = stage_load<C>(map, W, xq, nb, (s + 2) * KSP);
    compute(even, s);
    stage_store<C>(map, pb, odd);
    __syncthreads();
    pb = stage_load<C>(map, W, xq, nb, (s + 3) * KSP);
    compute(odd, s + 1);
    stage_store<C>(map, pa, even);
    __syncthreads();
  }

  if constexpr (!SUMS) {
    if constexpr (KSP > 1) {
      // wavefronts of superblocks 1 .. KSP-1 hand their partial sums to those of
      // superblock 0, which add them in superblock order
      float* red = reinterpret_cast<float*>(lds);
      const int slot = (rt * C::kTG + tg) * TW;
      constexpr int kPer = C::RT * C::kTG * TW;  // slots per superblock of the stage
      if (kh > 0) {
#pragma unroll
        for (int t = 0; t < TW; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) red[(((kh - 1) * kPer + slot + t) * 4 + i) * 64 + lane] = acc[t][i];
      }
      __syncthreads();
      if (kh > 0) return;
#pragma unroll
      for (int k = 1; k < KSP; ++k)
#pragma unroll
        for (int t = 0; t < TW; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[t][i] += red[(((k - 1) * kPer + slot + t) * 4 + i) * 64 + lane];
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

template <class C, bool SUMS>
hipError_t launch_kernel(const uint8_t* W, int n_out, int nb, const uint8_t* xq, int ncols, float* y,
                         int32_t* sums, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  auto k = gemm_q4_K_mfma<C, SUMS>;
  unsigned grid = 0;
  if (!launch_grid((static_cast<int64_t>(n_out) + C::kRows - 1) / C::kRows, C::kThreads, &grid))
    return hipErrorInvalidConfiguration;
  constexpr size_t lds = 2 * C::kBytes;
  if constexpr (lds > 65536) {
    // above the default dynamic LDS limit: raise it for this kernel on the current
    // device (set on every launch: the library keeps no per-device state)
    const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                                hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (attr != hipSuccess) return attr;
  }
  if (e0 != nullptr || e1 != nullptr) {
    hipExtLaunchKernelGGL(k, dim3(grid), dim3(C::kThreads), lds, s, e0, e1, 0, W, n_out, nb, xq, ncols, y,
                          sums);
  } else {
    k<<<grid, C::kThreads, lds, s>>>(W, n_out, nb, xq, ncols, y, sums);
  }
  return hipGetLastError();
}

template <class C>
hipError_t launch_cfg(const uint8_t* W, int n_out, int nb, const uint8_t* xq, int ncols, float* y,
                      int32_t* sums, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (sums != nullptr) return launch_kernel<C, true>(W, n_out, nb, xq, ncols, y, sums, s, e0, e1);
  return launch_kernel<C, false>(W, n_out, nb, xq, ncols, y, sums, s, e0, e1);
}

}  // namespace

hipError_t launch_gemm_q4K(const uint8_t* W, int64_t n_out, int64_t n_in, const uint8_t* xq,
                           int64_t ncols, float* y, int32_t* sums, hipStream_t s, hipEvent_t e0,
                           hipEvent_t e1) {
  const int nb = static_cast<int>(n_in / 256);
  const int n = static_cast<int>(n_out), nc = static_cast<int>(ncols);
  // 64-row workgroups (RT = 4) share each staged activation tile over four row
  // tiles, measured best on 14336 x 4096 (graph replay: 16 columns 12.2 us, two row
  // tiles 13.3; 32 columns 16.3 us, Cfg<2,1,1> with two row tiles 19.3; 64 columns
  // 22.6 us, Cfg<4,2,1> 27.8).  Few rows leave most CUs idle at 64 rows per
  // workgroup (4096 rows: 64 workgroups for 256 CUs), so matrices with at most 128
  // (16 columns) or 64 (32, 64 columns) such groups use 16-row workgroups with four
  // superblocks per stage instead (launch-recorded events: 4096 x 11008 at 16 / 32 /
  // 64 columns 25.9 / 35.9 / 52.4 -> 15.7 / 21.4 / 33.6 us; 4096 x 4096 13.0 / 16.9 /
  // 23.8 -> 9.1 / 11.5 / 16.8 us; at 11008 or more rows the 64-row shapes stay
  // faster).  Shapes of 16 wavefronts that need more than 128 registers spill and
  // are slower.
  const int64_t groups64 = (n_out + 63) / 64;
  if (nc <= 16) {
    if (groups64 <= 128) return launch_cfg<Cfg<1, 1, 4, 1>>(W, n, nb, xq, nc, y, sums, s, e0, e1);
    return launch_cfg<Cfg<1, 1, 2, 4>>(W, n, nb, xq, nc, y, sums, s, e0, e1);
  }
  if (nc <= 32) {
    if (groups64 <= 64) return launch_cfg<Cfg<2, 1, 4, 1>>(W, n, nb, xq, nc, y, sums, s, e0, e1);
    return launch_cfg<Cfg<2, 1, 2, 4>>(W, n, nb, xq, nc, y, sums, s, e0, e1);
  }
  if (nc <= 64) {
    if (groups64 <= 64) return launch_cfg<Cfg<4, 2, 4, 1>>(W, n, nb, xq, nc, y, sums, s, e0, e1);
    return launch_cfg<Cfg<4, 4, 2, 4>>(W, n, nb, xq, nc, y, sums, s, e0, e1);
  }
  return hipErrorInvalidValue;
}

}  // namespace qk
