// qk_capi.hip - the C ABI of libqk.so (declared in include/qk.h).
//
// Host-side validation of types, pairing, shapes, pointers and alignment, then
// asynchronous launches on the caller's stream.  No allocation, no state.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qk.h"
#include "qk_internal.h"

namespace {

// Weight formats with a GEMV (a paired activation type).
bool is_weight(int t) {
  return t == QK_TYPE_Q4_0 || t == QK_TYPE_Q5_0 || t == QK_TYPE_Q8_0 || t == QK_TYPE_Q4_1 ||
         t == QK_TYPE_Q5_1 || t == QK_TYPE_Q2_K || t == QK_TYPE_Q3_K || t == QK_TYPE_Q4_K ||
         t == QK_TYPE_Q5_K || t == QK_TYPE_Q6_K;
}
// Weight formats qk_dequantize_row expands (every GEMV weight format).
bool is_dequant(int t) { return is_weight(t); }
// Weight formats qk_quantize_row writes.
bool is_quant_row(int t) {
  return t == QK_TYPE_Q8_0 || t == QK_TYPE_Q4_0 || t == QK_TYPE_Q4_1 || t == QK_TYPE_Q5_0;
}
bool is_act(int t) { return t == QK_TYPE_Q8_0 || t == QK_TYPE_Q8_1 || t == QK_TYPE_Q8_K; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A launch beyond the 32-bit work-item count (refused by the launchers before
// anything is enqueued) is a size limit; any other runtime error is QK_E_DEVICE.
int status_of(hipError_t e) {
  if (e == hipSuccess) return QK_OK;
  return e == hipErrorInvalidConfiguration ? QK_E_LIMIT : QK_E_DEVICE;
}

// Common checks of a GEMV call; `out` is y or sums.
int check_gemv(int w_type, const void* W, int64_t n_out, int64_t n_in, const void* xq,
               int64_t ncols, const void* out) {
  if (!is_weight(w_type)) return QK_E_TYPE;
  if (n_out < 0 || ncols < 0 || n_in <= 0 || n_in % qk_block_elems(w_type) != 0) return QK_E_SHAPE;
  if (n_out > INT32_MAX) return QK_E_SHAPE;
  if (n_in > qk_max_n_in(w_type)) return QK_E_LIMIT;
  if (n_out == 0 || ncols == 0) return QK_OK;
  if (W == nullptr || xq == nullptr || out == nullptr) return QK_E_NULL;
  if (!aligned16(W) || !aligned16(xq) || !aligned16(out)) return QK_E_ALIGN;
  return QK_OK;
}

int gemv_impl(int w_type, const void* W, int64_t n_out, int64_t n_in, const void* xq,
              int64_t ncols, float* y, int32_t* sums, void* stream, void* ev0, void* ev1) {
  const void* out = y ? static_cast<const void*>(y) : static_cast<const void*>(sums);
  const int rc = check_gemv(w_type, W, n_out, n_in, xq, ncols, out);
  if (rc != QK_OK || n_out == 0 || ncols == 0) return rc;
  const int at = qk_act_type(w_type);
  const int64_t xrow = qk_row_bytes(at, n_in);
  const int64_t nb = n_in / qk_block_elems(w_type);
  const int k = (w_type == QK_TYPE_Q2_K || w_type == QK_TYPE_Q4_K || w_type == QK_TYPE_Q5_K) ? 2 : 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Small batches read W once with the multi-column GEMV kernel: Q4_K at 2 columns,
  // and at 3 when the matrix has at most 8192 rows (beyond, and from 4 columns, the
  // matrix-core kernel is faster: 14336 x 4096 at 3 columns 13.7 against 15.9 us);
  // every other format, which has no matrix-core path, in groups of up to 4 columns.
  const bool small_q4K = w_type == QK_TYPE_Q4_K && (ncols == 2 || (ncols == 3 && n_out <= 8192));
  int64_t group = qk::kGemvMaxCols;  // columns per launch: as many as the LDS holds
  while (group > 1 && !qk::gemv_cols_fits(w_type, n_in, group)) --group;
  const bool gemv_only = w_type != QK_TYPE_Q4_K;  // formats with no matrix-core path
  if ((small_q4K || (gemv_only && ncols > 1)) && group > 1) {
    // as few launches as the group size allows, their sizes balanced (4 columns that
    // take at most 3 per launch run as 2 + 2, not 3 + 1: Q4_0 4096 x 11008 21.6
    // against 22.8 us)
    const int64_t launches = (ncols + group - 1) / group;
    for (int64_t c = 0, i = 0; c < ncols; c += ncols / launches + (i < ncols % launches), ++i) {
      const int64_t nc = ncols / launches + (i < ncols % launches ? 1 : 0);
      const uint8_t* xc = static_cast<const uint8_t*>(xq) + c * xrow;
      float* yc = y ? y + c * n_out : nullptr;
      int32_t* sc = sums ? sums + c * n_out * nb * k : nullptr;
      hipEvent_t e0 = (c == 0) ? static_cast<hipEvent_t>(ev0) : nullptr;
      hipEvent_t e1 = (c + nc == ncols) ? static_cast<hipEvent_t>(ev1) : nullptr;
      const hipError_t e =
          nc == 1 ? qk::launch_gemv(w_type, static_cast<const uint8_t*>(W), n_out, n_in, xc, yc, sc, s, e0, e1)
                  : qk::launch_gemv_cols(w_type, static_cast<const uint8_t*>(W), n_out, n_in, xc, nc, yc, sc, s, e0, e1);
      if (e != hipSuccess) return status_of(e);
    }
    return QK_OK;
  }
  if (w_type == QK_TYPE_Q4_K && ncols > 1) {
    // several columns: one pass over W per group of up to 64 columns (matrix cores)
    for (int64_t c = 0; c < ncols; c += qk::kGemmMaxCols) {
      const int64_t nc = (ncols - c < qk::kGemmMaxCols) ? ncols - c : qk::kGemmMaxCols;
      const uint8_t* xc = static_cast<const uint8_t*>(xq) + c * xrow;
      float* yc = y ? y + c * n_out : nullptr;
      int32_t* sc = sums ? sums + c * n_out * nb * k : nullptr;
      hipEvent_t e0 = (c == 0) ? static_cast<hipEvent_t>(ev0) : nullptr;
      hipEvent_t e1 = (c + nc == ncols) ? static_cast<hipEvent_t>(ev1) : nullptr;
      const hipError_t e = qk::launch_gemm_q4K(static_cast<const uint8_t*>(W), n_out, n_in, xc, nc,
                                               yc, sc, s, e0, e1);
      if (e != hipSuccess) return status_of(e);
    }
    return QK_OK;
  }
  for (int64_t c = 0; c < ncols; ++c) {
    const uint8_t* xc = static_cast<const uint8_t*>(xq) + c * xrow;
    float* yc = y ? y + c * n_out : nullptr;
    int32_t* sc = sums ? sums + c * n_out * nb * k : nullptr;
    hipEvent_t e0 = (c == 0) ? static_cast<hipEvent_t>(ev0) : nullptr;
    hipEvent_t e1 = (c == ncols - 1) ? static_cast<hipEvent_t>(ev1) : nullptr;
    const hipError_t e = qk::launch_gemv(w_type, static_cast<const uint8_t*>(W), n_out, n_in, xc,
                                         yc, sc, s, e0, e1);
    if (e != hipSuccess) return status_of(e);
  }
  return QK_OK;
}

}  // namespace

extern "C" {

int64_t qk_block_elems(int type) {
  switch (type) {
    case QK_TYPE_Q4_0:
    case QK_TYPE_Q4_1:
    case QK_TYPE_Q5_0:
    case QK_TYPE_Q5_1:
    case QK_TYPE_Q8_0:
    case QK_TYPE_Q8_1: return 32;
    case QK_TYPE_Q2_K:
    case QK_TYPE_Q3_K:
    case QK_TYPE_Q4_K:
    case QK_TYPE_Q5_K:
    case QK_TYPE_Q6_K:
    case QK_TYPE_Q8_K: return 256;
    default: return 0;
  }
}

int64_t qk_block_bytes(int type) {
  switch (type) {
    case QK_TYPE_Q4_0: return 18;
    case QK_TYPE_Q4_1: return 20;
    case QK_TYPE_Q5_0: return 22;
    case QK_TYPE_Q5_1: return 24;
    case QK_TYPE_Q8_0: return 34;
    case QK_TYPE_Q8_1: return 36;
    case QK_TYPE_Q2_K: return 84;
    case QK_TYPE_Q3_K: return 110;
    case QK_TYPE_Q4_K: return 144;
    case QK_TYPE_Q5_K: return 176;
    case QK_TYPE_Q6_K: return 210;
    case QK_TYPE_Q8_K: return 292;
    default: return 0;
  }
}

int64_t qk_row_bytes(int type, int64_t n) {
  const int64_t be = qk_block_elems(type);
  if (be == 0 || n < 0 || n % be != 0) return 0;
  return n / be * qk_block_bytes(type);
}

int qk_act_type(int weight_type) {
  switch (weight_type) {
    case QK_TYPE_Q4_0:
    case QK_TYPE_Q5_0:
    case QK_TYPE_Q8_0: return QK_TYPE_Q8_0;
    case QK_TYPE_Q4_1:
    case QK_TYPE_Q5_1: return QK_TYPE_Q8_1;
    case QK_TYPE_Q2_K:
    case QK_TYPE_Q3_K:
    case QK_TYPE_Q4_K:
    case QK_TYPE_Q5_K:
    case QK_TYPE_Q6_K: return QK_TYPE_Q8_K;
    default: return -1;
  }
}

const char* qk_status_str(int status) {
  switch (status) {
    case QK_OK: return "ok";
    case QK_E_TYPE: return "unknown type, or a type this call does not take";
    case QK_E_PAIR: return "the activation type is not the one the weight type pairs with";
    case QK_E_SHAPE: return "shape is not whole blocks, or a count is negative";
    case QK_E_ALIGN: return "a base pointer is not 16-byte aligned";
    case QK_E_NULL: return "a required pointer is NULL";
    case QK_E_DEVICE: return "HIP runtime error while enqueueing";
    case QK_E_LIMIT: return "a size beyond the kernels' limits (LDS budget, columns, one launch)";
    case QK_E_ARG: return "an argument outside its documented set of values";
    default: return "unknown status";
  }
}

int64_t qk_max_n_in(int weight_type) {
  if (!is_weight(weight_type)) return 0;
  const int64_t be = qk_block_elems(weight_type);
  int64_t best = 0;
  // largest whole-block n_in whose LDS layout fits (monotone in n_in)
  int64_t lo = 1, hi = (int64_t(1) << 20) / be;
  while (lo <= hi) {
    const int64_t mid = (lo + hi) / 2;
    if (qk::gemv_lds_bytes(weight_type, mid * be) <= qk::kMaxLdsBytes) {
      best = mid * be;
      lo = mid + 1;
    } else {
      hi = mid - 1;
    }
  }
  return best;
}

int qk_quantize_act_timed(int act_type, const float* x, void* xq, int64_t n, int64_t ncols,
                          void* stream, void* ev_start, void* ev_stop) {
  if (!is_act(act_type)) return QK_E_TYPE;
  const int64_t be = qk_block_elems(act_type);
  if (n <= 0 || n % be != 0 || ncols < 0) return QK_E_SHAPE;
  if (ncols == 0) return QK_OK;
  if (x == nullptr || xq == nullptr) return QK_E_NULL;
  if (!aligned16(x) || !aligned16(xq)) return QK_E_ALIGN;
  const int64_t nblocks = n / be * ncols;
  return status_of(qk::launch_quantize(act_type, x, static_cast<uint8_t*>(xq), nblocks,
                                       static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(ev_start),
                                       static_cast<hipEvent_t>(ev_stop)));
}

int qk_quantize_act(int act_type, const float* x, void* xq, int64_t n, int64_t ncols,
                    void* stream) {
  return qk_quantize_act_timed(act_type, x, xq, n, ncols, stream, nullptr, nullptr);
}

int qk_quantize_row(int type, const float* x, void* dst, int64_t n, void* stream) {
  if (!is_quant_row(type)) return QK_E_TYPE;
  if (n < 0 || n % 32 != 0) return QK_E_SHAPE;
  if (n == 0) return QK_OK;
  if (x == nullptr || dst == nullptr) return QK_E_NULL;
  if (!aligned16(x) || !aligned16(dst)) return QK_E_ALIGN;
  return status_of(qk::launch_quantize_row(type, x, static_cast<uint8_t*>(dst), n / 32,
                                           static_cast<hipStream_t>(stream)));
}

int qk_gemv(int w_type, const void* W, int64_t n_out, int64_t n_in, const void* xq,
            int64_t ncols, float* y, void* stream) {
  return gemv_impl(w_type, W, n_out, n_in, xq, ncols, y, nullptr, stream, nullptr, nullptr);
}

int qk_gemv_typed(int w_type, int act_type, const void* W, int64_t n_out, int64_t n_in,
                  const void* xq, int64_t ncols, float* y, void* stream) {
  if (!is_weight(w_type) || !is_act(act_type)) return QK_E_TYPE;
  if (act_type != qk_act_type(w_type)) return QK_E_PAIR;
  return gemv_impl(w_type, W, n_out, n_in, xq, ncols, y, nullptr, stream, nullptr, nullptr);
}

int qk_gemv_timed(int w_type, const void* W, int64_t n_out, int64_t n_in, const void* xq,
                  int64_t ncols, float* y, void* stream, void* ev_start, void* ev_stop) {
  return gemv_impl(w_type, W, n_out, n_in, xq, ncols, y, nullptr, stream, ev_start, ev_stop);
}

int qk_gemv_pair_timed(int w_type, const void* W1, const void* W2, int64_t n_out, int64_t n_in,
                       const void* xq, int64_t ncols, int epilogue, float* out, void* stream,
                       void* ev_start, void* ev_stop) {
  if (w_type != QK_TYPE_Q4_K && w_type != QK_TYPE_Q5_K) return QK_E_TYPE;
  if (epilogue != QK_EPI_NONE && epilogue != QK_EPI_SWIGLU) return QK_E_ARG;
  int rc = check_gemv(w_type, W1, n_out, n_in, xq, ncols, out);
  if (rc != QK_OK) return rc;
  if (ncols > 65535) return QK_E_LIMIT;
  if (n_out == 0 || ncols == 0) return QK_OK;
  if (W2 == nullptr) return QK_E_NULL;
  if (!aligned16(W2)) return QK_E_ALIGN;
  return status_of(qk::launch_gemv_pair(w_type, static_cast<const uint8_t*>(W1), static_cast<const uint8_t*>(W2),
                                        n_out, n_in, static_cast<const uint8_t*>(xq), ncols,
                                        epilogue == QK_EPI_SWIGLU, out, static_cast<hipStream_t>(stream),
                                        static_cast<hipEvent_t>(ev_start),
                                        static_cast<hipEvent_t>(ev_stop)));
}

int qk_gemv_pair(int w_type, const void* W1, const void* W2, int64_t n_out, int64_t n_in,
                 const void* xq, int64_t ncols, int epilogue, float* out, void* stream) {
  return qk_gemv_pair_timed(w_type, W1, W2, n_out, n_in, xq, ncols, epilogue, out, stream, nullptr,
                            nullptr);
}

int qk_gemv_block_sums(int w_type, const void* W, int64_t n_out, int64_t n_in,
                       const void* xq, int64_t ncols, int32_t* sums, void* stream) {
  if (sums == nullptr && is_weight(w_type) && n_out > 0 && ncols > 0) return QK_E_NULL;
  return gemv_impl(w_type, W, n_out, n_in, xq, ncols, nullptr, sums, stream, nullptr, nullptr);
}

int qk_dequantize_row(int type, const void* src, float* dst, int64_t n, void* stream) {
  if (!is_dequant(type)) return QK_E_TYPE;
  const int64_t be = qk_block_elems(type);
  if (n < 0 || n % be != 0) return QK_E_SHAPE;
  if (n == 0) return QK_OK;
  if (src == nullptr || dst == nullptr) return QK_E_NULL;
  if (!aligned16(src) || !aligned16(dst)) return QK_E_ALIGN;
  return status_of(qk::launch_dequantize(type, static_cast<const uint8_t*>(src), dst, n / be,
                                         static_cast<hipStream_t>(stream)));
}

int qk_read_probe_ex(const void* src, int64_t bytes, uint32_t* out, int kb_per_wave, int64_t grid_blocks,
                     int nontemporal, void* stream, void* ev_start, void* ev_stop) {
  if (!qk::read_probe_kb_ok(kb_per_wave) || grid_blocks < 0 || (nontemporal != 0 && nontemporal != 1))
    return QK_E_ARG;
  if (bytes <= 0 || bytes % 16 != 0) return QK_E_SHAPE;
  if (src == nullptr || out == nullptr) return QK_E_NULL;
  if (!aligned16(src) || !aligned16(out)) return QK_E_ALIGN;
  return status_of(qk::launch_read_probe(static_cast<const uint8_t*>(src), bytes, out, kb_per_wave, grid_blocks,
                                         nontemporal, static_cast<hipStream_t>(stream),
                                         static_cast<hipEvent_t>(ev_start), static_cast<hipEvent_t>(ev_stop)));
}

int qk_read_probe(const void* src, int64_t bytes, uint32_t* out, void* stream, void* ev_start,
                  void* ev_stop) {
  return qk_read_probe_ex(src, bytes, out, 2, 0, 0, stream, ev_start, ev_stop);
}

}  // extern "C"
