// abi_check - the C ABI of libqk.so used from a plain host program (no Python, no
// torch): device memory from the HIP runtime, every call through include/qk.h, and
// every result checked against the CPU oracle (oracle/qk_oracle.h, test
// infrastructure) on the same inputs.
//
// Bars: activation blocks, per-block int32 sums, dequantized values and weight
// blocks bit-exact; y within 1e-5 * L per output, L the oracle's sum of the absolute
// float terms of the block steps (orc_gemv's l1).
// Inputs: splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", 2014) drives random block bytes, f16 scales drawn uniformly in the
// workloads' ranges, and activations uniform in [-2, 2).
// Exit status 0 when every check passes; the first failures are printed.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "qk.h"
#include "qk_oracle.h"

namespace {

uint64_t g_state = 0x5eed0001ull;
uint64_t next_u64() {  // splitmix64
  uint64_t z = (g_state += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}
double uniform01() { return static_cast<double>(next_u64() >> 11) * (1.0 / 9007199254740992.0); }

int g_failures = 0;
void fail(const char* what) {
  if (++g_failures <= 20) std::printf("FAIL %s\n", what);
}
#define HIPCHECK(x)                                                              \
  do {                                                                           \
    hipError_t e_ = (x);                                                         \
    if (e_ != hipSuccess) {                                                      \
      std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 2;                                                                  \
    }                                                                            \
  } while (0)

template <typename T>
struct Dev {
  T* p = nullptr;
  explicit Dev(size_t n) {
    if (hipMalloc(reinterpret_cast<void**>(&p), n * sizeof(T) + 16) != hipSuccess) p = nullptr;
  }
  ~Dev() {
    if (p) (void)hipFree(p);
  }
};

void put_f16(uint8_t* dst, double lo, double hi) {
  const uint16_t h = orc_f32_to_f16(static_cast<float>(lo + (hi - lo) * uniform01()));
  std::memcpy(dst, &h, 2);
}

// Random weight blocks of a type: uniform bytes, then valid f16 scale fields.
std::vector<uint8_t> weights(int type, int64_t n_out, int64_t n_in) {
  const int64_t bb = qk_block_bytes(type), nb = n_out * (n_in / qk_block_elems(type));
  std::vector<uint8_t> w(static_cast<size_t>(bb * nb));
  for (auto& b : w) b = static_cast<uint8_t>(next_u64() >> 56);
  for (int64_t i = 0; i < nb; ++i) {
    uint8_t* blk = w.data() + i * bb;
    if (type == QK_TYPE_Q4_K || type == QK_TYPE_Q5_K) {
      put_f16(blk, 1e-4, 1e-3);
      put_f16(blk + 2, 1e-4, 1e-3);
    } else if (type == QK_TYPE_Q6_K) {
      put_f16(blk + 208, 1e-4, 1e-3);
    } else if (type == QK_TYPE_Q2_K) {
      put_f16(blk + 80, 1e-4, 1e-3);
      put_f16(blk + 82, 1e-4, 1e-3);
    } else if (type == QK_TYPE_Q3_K) {
      put_f16(blk + 108, 1e-4, 1e-3);
    } else if (type == QK_TYPE_Q4_1 || type == QK_TYPE_Q5_1) {
      put_f16(blk, 1e-3, 4e-3);
      put_f16(blk + 2, -0.03, -0.005);
    } else {
      put_f16(blk, 1e-3, 4e-3);
    }
  }
  return w;
}

int check_type(int type, int64_t n_out, int64_t n_in, int64_t ncols) {
  char what[160];
  const int at = qk_act_type(type);
  const int64_t wbytes = n_out * qk_row_bytes(type, n_in), xbytes = ncols * qk_row_bytes(at, n_in);
  std::vector<uint8_t> W = weights(type, n_out, n_in);
  std::vector<float> x(static_cast<size_t>(n_in * ncols));
  for (auto& v : x) v = static_cast<float>(4.0 * uniform01() - 2.0);

  Dev<uint8_t> dW(wbytes), dxq(xbytes);
  Dev<float> dx(x.size()), dy(n_out * ncols), dy2(n_out * ncols), dd(n_out * n_in);
  const int64_t k = orc_sums_per_block(type), nb = n_in / qk_block_elems(type);
  Dev<int32_t> ds(ncols * n_out * nb * k);
  if (!dW.p || !dxq.p || !dx.p || !dy.p || !dy2.p || !dd.p || !ds.p) return 2;
  HIPCHECK(hipMemcpy(dW.p, W.data(), wbytes, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(dx.p, x.data(), x.size() * 4, hipMemcpyHostToDevice));

  int rc = qk_quantize_act(at, dx.p, dxq.p, n_in, ncols, nullptr);
  if (rc == QK_OK) rc = qk_gemv(type, dW.p, n_out, n_in, dxq.p, ncols, dy.p, nullptr);
  if (rc == QK_OK) rc = qk_gemv_typed(type, at, dW.p, n_out, n_in, dxq.p, ncols, dy2.p, nullptr);
  if (rc == QK_OK) rc = qk_gemv_block_sums(type, dW.p, n_out, n_in, dxq.p, ncols, ds.p, nullptr);
  if (rc == QK_OK) rc = qk_dequantize_row(type, dW.p, dd.p, n_out * n_in, nullptr);
  // an activation type the weight type does not pair with: refused before any launch
  const int wrong = at == QK_TYPE_Q8_K ? QK_TYPE_Q8_0 : QK_TYPE_Q8_K;
  if (qk_gemv_typed(type, wrong, dW.p, n_out, n_in, dxq.p, ncols, dy2.p, nullptr) != QK_E_PAIR) {
    std::snprintf(what, sizeof what, "type %d: a mismatched activation type was not refused", type);
    fail(what);
  }
  if (rc != QK_OK) {
    std::snprintf(what, sizeof what, "type %d: status %d (%s)", type, rc, qk_status_str(rc));
    fail(what);
    return 0;
  }
  HIPCHECK(hipDeviceSynchronize());
  std::vector<uint8_t> xq(static_cast<size_t>(xbytes));
  std::vector<float> y(static_cast<size_t>(n_out * ncols)), deq(static_cast<size_t>(n_out * n_in));
  std::vector<int32_t> sums(static_cast<size_t>(ncols * n_out * nb * k));
  HIPCHECK(hipMemcpy(xq.data(), dxq.p, xbytes, hipMemcpyDeviceToHost));
  HIPCHECK(hipMemcpy(y.data(), dy.p, y.size() * 4, hipMemcpyDeviceToHost));
  {
    std::vector<float> y2(y.size());
    HIPCHECK(hipMemcpy(y2.data(), dy2.p, y2.size() * 4, hipMemcpyDeviceToHost));
    if (std::memcmp(y.data(), y2.data(), y.size() * 4) != 0) {
      std::snprintf(what, sizeof what, "type %d: qk_gemv_typed differs from qk_gemv", type);
      fail(what);
    }
  }
  HIPCHECK(hipMemcpy(deq.data(), dd.p, deq.size() * 4, hipMemcpyDeviceToHost));
  HIPCHECK(hipMemcpy(sums.data(), ds.p, sums.size() * 4, hipMemcpyDeviceToHost));

  // activation blocks
  std::vector<uint8_t> xq_o(static_cast<size_t>(xbytes));
  const int qrc = at == QK_TYPE_Q8_0   ? orc_quantize_q8_0(x.data(), xq_o.data(), n_in * ncols)
                  : at == QK_TYPE_Q8_1 ? orc_quantize_q8_1(x.data(), xq_o.data(), n_in * ncols)
                                       : orc_quantize_q8_K(x.data(), xq_o.data(), n_in * ncols);
  if (qrc != ORC_OK || std::memcmp(xq.data(), xq_o.data(), xq.size()) != 0) {
    std::snprintf(what, sizeof what, "type %d: activation blocks differ from the oracle", type);
    fail(what);
  }
  // per-block int32 sums and y
  const int64_t rbytes = qk_row_bytes(type, n_in), xrow = qk_row_bytes(at, n_in);
  std::vector<int32_t> s_o(static_cast<size_t>(nb * k));
  for (int64_t c = 0; c < ncols; ++c)
    for (int64_t r = 0; r < n_out; ++r) {
      if (orc_block_sums(type, W.data() + r * rbytes, xq_o.data() + c * xrow, n_in, s_o.data()) != ORC_OK ||
          std::memcmp(s_o.data(), sums.data() + (c * n_out + r) * nb * k, s_o.size() * 4) != 0) {
        std::snprintf(what, sizeof what, "type %d: block sums differ (column %lld, row %lld)", type,
                      static_cast<long long>(c), static_cast<long long>(r));
        fail(what);
      }
    }
  std::vector<float> y_o(y.size());
  std::vector<double> l1(y.size());
  if (orc_gemv(type, W.data(), n_out, n_in, xq_o.data(), ncols, y_o.data(), l1.data()) != ORC_OK) fail("oracle gemv");
  for (size_t i = 0; i < y.size(); ++i)
    if (std::fabs(static_cast<double>(y[i]) - static_cast<double>(y_o[i])) > 1e-5 * l1[i]) {
      std::snprintf(what, sizeof what, "type %d: y[%zu] = %.9g, oracle %.9g, bound %.3g", type, i, y[i], y_o[i],
                    1e-5 * l1[i]);
      fail(what);
    }
  // dequantized values
  std::vector<float> deq_o(deq.size());
  if (orc_dequantize(type, W.data(), deq_o.data(), n_out * n_in) != ORC_OK ||
      std::memcmp(deq.data(), deq_o.data(), deq.size() * 4) != 0) {
    std::snprintf(what, sizeof what, "type %d: dequantized values differ", type);
    fail(what);
  }
  return 0;
}

int check_quantize_row(int type, int64_t n) {
  char what[96];
  std::vector<float> w(static_cast<size_t>(n));
  for (auto& v : w) v = static_cast<float>(0.04 * uniform01() - 0.02);
  const int64_t bytes = qk_row_bytes(type, n);
  Dev<float> dw(n);
  Dev<uint8_t> dq(bytes);
  if (!dw.p || !dq.p) return 2;
  HIPCHECK(hipMemcpy(dw.p, w.data(), n * 4, hipMemcpyHostToDevice));
  const int rc = qk_quantize_row(type, dw.p, dq.p, n, nullptr);
  if (rc != QK_OK) {
    std::snprintf(what, sizeof what, "quantize_row %d: status %d", type, rc);
    fail(what);
    return 0;
  }
  HIPCHECK(hipDeviceSynchronize());
  std::vector<uint8_t> q(static_cast<size_t>(bytes)), q_o(static_cast<size_t>(bytes));
  HIPCHECK(hipMemcpy(q.data(), dq.p, bytes, hipMemcpyDeviceToHost));
  const int orc = type == QK_TYPE_Q8_0 ? orc_quantize_q8_0(w.data(), q_o.data(), n)
                  : type == QK_TYPE_Q4_0 ? orc_quantize_q4_0(w.data(), q_o.data(), n)
                  : type == QK_TYPE_Q4_1 ? orc_quantize_q4_1(w.data(), q_o.data(), n)
                                         : orc_quantize_q5_0(w.data(), q_o.data(), n);
  if (orc != ORC_OK || q != q_o) {
    std::snprintf(what, sizeof what, "quantize_row %d: blocks differ from the oracle", type);
    fail(what);
  }
  return 0;
}

}  // namespace

int main() {
  int dev_count = 0;
  if (hipGetDeviceCount(&dev_count) != hipSuccess || dev_count == 0) {
    std::printf("no GPU visible\n");
    return 2;
  }
  const int types[] = {QK_TYPE_Q8_0, QK_TYPE_Q4_0, QK_TYPE_Q5_0, QK_TYPE_Q4_1, QK_TYPE_Q5_1,
                       QK_TYPE_Q2_K, QK_TYPE_Q3_K, QK_TYPE_Q4_K, QK_TYPE_Q5_K, QK_TYPE_Q6_K};
  for (int t : types) {
    // one column (GEMV kernels) and three (Q4_K: the matrix-core path), ragged rows,
    // rows of two passes and of three (the LDS-staged kernels)
    const int64_t shapes[][3] = {{37, 2304, 1}, {37, 2304, 3}, {9, 11008, 1}};
    for (const auto& sh : shapes)
      if (int r = check_type(t, sh[0], sh[1], sh[2])) return r;
  }
  const int qtypes[] = {QK_TYPE_Q8_0, QK_TYPE_Q4_0, QK_TYPE_Q4_1, QK_TYPE_Q5_0};
  for (int t : qtypes)
    if (int r = check_quantize_row(t, 32 * 1001)) return r;
  if (g_failures) {
    std::printf("abi_check: %d failures\n", g_failures);
    return 1;
  }
  std::printf("abi_check ok: quantize_act, gemv, gemv_block_sums, dequantize_row for Q8_0, Q4_0, Q5_0, "
              "Q4_K, Q5_K, Q6_K and quantize_row for Q8_0, Q4_0, Q4_1, Q5_0 match the oracle\n");
  return 0;
}
