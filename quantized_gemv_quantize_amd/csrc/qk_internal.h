// qk_internal.h - launchers between the C ABI (qk_capi.hip) and the kernels.
// Arguments reaching a launcher have been validated by the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qk {

enum WType : int { kQ4_0 = 2, kQ4_1 = 3, kQ5_0 = 6, kQ5_1 = 7, kQ8_0 = 8, kQ8_1 = 9, kQ2_K = 10, kQ3_K = 11, kQ4_K = 12, kQ5_K = 13, kQ6_K = 14, kQ8_K = 15 };

// The work-items of one launch are counted in 32 bits (the dispatch packet's grid
// size).  Launchers size their grids through launch_grid and refuse a larger launch
// with hipErrorInvalidConfiguration, which the C ABI reports as QK_E_LIMIT.
constexpr int64_t kMaxLaunchItems = 0xFFFFFFFFll;
inline bool launch_grid(int64_t blocks, int threads_per_block, unsigned* grid) {
  if (blocks < 0 || blocks > kMaxLaunchItems / threads_per_block) return false;
  *grid = static_cast<unsigned>(blocks);
  return true;
}

// Activation quantization of `nblocks` consecutive blocks (any number of columns
// laid end to end: blocks of consecutive columns are contiguous).  Non-null events
// are recorded by the launch itself (start / end of the kernel).
hipError_t launch_quantize(int act_type, const float* x, uint8_t* xq, int64_t nblocks,
                           hipStream_t s, hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);

// Weight quantization (quantize_row_*_ref) of `nblocks` 32-element blocks of
// type Q8_0, Q4_0, Q4_1 or Q5_0.
hipError_t launch_quantize_row(int type, const float* x, uint8_t* dst, int64_t nblocks,
                               hipStream_t s);

// One GEMV over one activation column.  `sums` non-null selects the variant that
// stores the per-block integers (and `y` may be null).  ev_start / ev_stop, when
// non-null, are recorded by the kernel launch itself.
hipError_t launch_gemv(int w_type, const uint8_t* W, int64_t n_out, int64_t n_in,
                       const uint8_t* xq, float* y, int32_t* sums, hipStream_t s,
                       hipEvent_t ev_start, hipEvent_t ev_stop);

// Q8_0 / Q4_0 / Q5_0 x Q8_0 and Q4_K / Q5_K / Q6_K x Q8_K over 2..kGemvMaxCols
// activation columns with the weights read once (the one-column kernels' integer
// sums per column; the columns' activation rows are staged together in LDS).
// gemv_cols_fits says whether a shape qualifies.
constexpr int64_t kGemvMaxCols = 4;
bool gemv_cols_fits(int w_type, int64_t n_in, int64_t ncols);
hipError_t launch_gemv_cols(int w_type, const uint8_t* W, int64_t n_out, int64_t n_in, const uint8_t* xq,
                            int64_t ncols, float* y, int32_t* sums, hipStream_t s, hipEvent_t ev_start,
                            hipEvent_t ev_stop);

// Q4_K x Q8_K over 2..64 activation columns at once (int8 MFMA).  xq holds ncols
// consecutive Q8_K rows, y is [ncols][n_out], sums (when non-null) is
// [ncols][n_out][n_in / 256][2].
hipError_t launch_gemm_q4K(const uint8_t* W, int64_t n_out, int64_t n_in, const uint8_t* xq,
                           int64_t ncols, float* y, int32_t* sums, hipStream_t s,
                           hipEvent_t ev_start, hipEvent_t ev_stop);
constexpr int64_t kGemmMaxCols = 64;

// Bytes of dynamic LDS a GEMV over rows of n_in elements needs.
int64_t gemv_lds_bytes(int w_type, int64_t n_in);

// Q4_K W1 and W2 over the same Q8_K activation columns (ncols <= 65535): out is
// [ncols][2][n_out] (y1 then y2) or, with swiglu, [ncols][n_out] silu(y1) * y2.
// ev_start / ev_stop as launch_gemv (one launch).
hipError_t launch_gemv_pair(int w_type, const uint8_t* W1, const uint8_t* W2, int64_t n_out, int64_t n_in,
                            const uint8_t* xq, int64_t ncols, int swiglu, float* out, hipStream_t s,
                            hipEvent_t ev_start, hipEvent_t ev_stop);
// LDS one workgroup may address on gfx950: all 160 KB of a CU (the device reports
// it as sharedMemPerBlock).  The longest activation row a one-column GEMV stages;
// launches above 64 KB opt in per kernel (hipFuncAttributeMaxDynamicSharedMemorySize).
constexpr int64_t kMaxLdsBytes = 163840;
// LDS budget of the multi-column GEMV kernels' column groups: at most 64 KB, so
// that two 4-wavefront workgroups still share a CU; longer groups run fewer columns
// per launch (the measured trade-off of those kernels).
constexpr int64_t kColsLdsBytes = 65536;

hipError_t launch_dequantize(int type, const uint8_t* src, float* dst, int64_t nblocks,
                             hipStream_t s);

// Read-stream probe over `bytes` (a multiple of 16) bytes: one XOR word per group
// of kb kilobytes (kb in 1, 2, 4, 8, 16) into out; grid_blocks > 0 launches a
// persistent grid of that many 4-wavefront workgroups, 0 one wavefront per group;
// nontemporal selects streaming loads.  ev_start / ev_stop as launch_gemv.
bool read_probe_kb_ok(int kb);
hipError_t launch_read_probe(const uint8_t* src, int64_t bytes, uint32_t* out, int kb, int64_t grid_blocks,
                             int nontemporal, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop);

}  // namespace qk
