/*
 * qk.h - C ABI of libqk.so, the MI355X (gfx950) block-quantized GEMV library.
 *
 * The library computes y = W x where W is stored row-major as whole ggml blocks
 * (Q8_0, Q4_0, Q5_0, Q4_1, Q5_1, Q2_K, Q3_K, Q4_K, Q5_K or Q6_K, byte-exact GGUF layouts) and x is
 * quantized once per call into int8 activation blocks (Q8_0, Q8_1 or Q8_K) aligned
 * with W's blocks.  Every
 * product inside a block is an exact int32 sum; only the block scales are float.
 * Sources (page title, section):
 *   "Quantization" (rml): type table, DequantizeRow, VecDot and its pairing.
 *   "Quantization" (sipllm): dequantize_row(t, src, dst, n), matmul_quant layout.
 *   "Building Q8_0 and Q4_0 Like ggml" (codeloopback): Q8_0/Q4_0 bytes, Examples 1-11.
 *   "量化格式" (candle formats): type table, BlockQ4K/Q6K/Q8K fields, VecDotType.
 * Q5_1, Q5_K and Q6_K: the pages give their size and the role of each field, not
 * which bit belongs to which element; Q2_K and Q3_K: the pages give their size only.
 * For all five the GGUF arrangement is implemented (stated below at
 * qk_dequantize_row).  Q8_1: the pages name it as the activation block of
 * the _1 types without its layout; the reading is stated at qk_quantize_act.
 *
 * Conventions shared by every call:
 *  - Types are ggml's ids, as a GGUF tensor record stores them.
 *  - All buffers are device memory owned by the caller (for example torch tensors);
 *    the library allocates nothing and keeps no state between calls.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *    asynchronously on it; a QK_OK return means it was enqueued.
 *  - Arguments are checked on the host before anything is enqueued; on any error
 *    nothing is launched and no buffer is touched.
 *  - Base pointers must be 16-byte aligned (QK_E_ALIGN otherwise).  Rows inside W
 *    need not be: a Q6_K row of 11008 elements is 9030 bytes.
 */
#ifndef QK_H
#define QK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ggml type ids of the formats on the path. */
#define QK_TYPE_Q4_0 2
#define QK_TYPE_Q4_1 3
#define QK_TYPE_Q5_0 6
#define QK_TYPE_Q5_1 7
#define QK_TYPE_Q8_0 8
#define QK_TYPE_Q8_1 9
#define QK_TYPE_Q2_K 10
#define QK_TYPE_Q3_K 11
#define QK_TYPE_Q4_K 12
#define QK_TYPE_Q5_K 13
#define QK_TYPE_Q6_K 14
#define QK_TYPE_Q8_K 15

/* Status codes returned by every call that can fail. */
#define QK_OK 0
#define QK_E_TYPE 1   /* unknown type id, or a type the call does not take */
#define QK_E_PAIR 2   /* the activation type is not the one the weight type pairs with */
#define QK_E_SHAPE 3  /* n not a positive multiple of the block size, or a negative count */
#define QK_E_ALIGN 4  /* a base pointer is not 16-byte aligned */
#define QK_E_NULL 5   /* a required pointer is NULL */
#define QK_E_DEVICE 6 /* the HIP runtime reported an error while enqueueing */
#define QK_E_LIMIT 7  /* the activation row does not fit the kernels' LDS budget, more
                         activation columns than a call takes, or more work than one
                         kernel launch addresses (2^32 - 1 work-items) */
#define QK_E_ARG 8    /* an argument outside its documented set of values */

/* Epilogues of qk_gemv_pair. */
#define QK_EPI_NONE 0
#define QK_EPI_SWIGLU 1

/* Elements per block (32 or 256) and bytes per block (Q4_0 18, Q4_1 20, Q5_0 22,
 * Q5_1 24, Q8_0 34, Q8_1 36, Q2_K 84, Q3_K 110, Q4_K 144, Q5_K 176, Q6_K 210, Q8_K 292) of a type, 0 for an
 * unknown id.  Geometry from the candle formats page, "GgmlDType" table (Q8_1's 36
 * bytes are the reading stated at qk_quantize_act). */
int64_t qk_block_elems(int type);
int64_t qk_block_bytes(int type);

/* Bytes of n elements of a type: n / block_elems * block_bytes, rows being whole
 * blocks with nothing between them (codeloopback Example 9; sipllm type_nbytes).
 * 0 when the type is unknown or n is negative or not a multiple of the block size. */
int64_t qk_row_bytes(int type, int64_t n);

/* Activation type a weight type is multiplied against (candle "VecDotType" table;
 * codeloopback Example 11): Q4_0, Q5_0, Q8_0 -> Q8_0; Q4_1, Q5_1 -> Q8_1; Q2_K, Q3_K,
 * Q4_K, Q5_K, Q6_K -> Q8_K; -1 otherwise (including the activation-only Q8_1 and Q8_K). */
int qk_act_type(int weight_type);

/* Human-readable text of a status code (static storage, never NULL). */
const char* qk_status_str(int status);

/* Largest n_in a GEMV accepts for a weight type (the paired activation row is held
 * in LDS); 0 for an unknown or non-weight type. */
int64_t qk_max_n_in(int weight_type);

/*
 * qk_quantize_act - quantize float activations into int8 blocks, once per call.
 *   act_type  QK_TYPE_Q8_0, QK_TYPE_Q8_1 or QK_TYPE_Q8_K (else QK_E_TYPE).
 *   x         f32 [ncols][n], row-major, device.
 *   xq        out: [ncols][n / block] blocks, ncols * qk_row_bytes(act_type, n) bytes.
 *   n         elements per column, a positive multiple of the block size.
 *   ncols     number of columns (tokens), >= 0; 0 enqueues nothing.
 * Per block (codeloopback Example 2; candle BlockQ8_0::from_float): amax = largest
 * |x| (NaN ignored); d = amax / 127 (correctly rounded f32); id = 1/d, or 0 when d
 * is 0; code = roundf(x * id), halves away from zero, NaN -> 0, saturated to int8.
 * Q8_0 stores d as f16 (round to nearest even, subnormals kept, overflow -> inf)
 * then 32 codes (34 bytes).  Q8_K stores d as f32, 256 codes and 16 int16 bsums,
 * each the sum of 16 consecutive codes (292 bytes; candle BlockQ8K).  Q8_1 (36 bytes;
 * candle names BlockQ8_1 as the activation block of Q4_1 and Q5_1 without printing
 * it, so this layout is a reading): f16 d, f16 s = (sum of the 32 codes) * d with the
 * unrounded f32 d, rounded to f16, then the 32 codes as Q8_0's.
 * Results are bit-exact to that definition.
 */
int qk_quantize_act(int act_type, const float* x, void* xq, int64_t n, int64_t ncols,
                    void* stream);

/* qk_quantize_act_timed - qk_quantize_act whose kernel launch records ev_start and
 * ev_stop itself (hipEvent_t, either may be NULL), as qk_gemv_timed: timing every
 * kernel of a step the same way keeps the per-kernel durations comparable.
 * Arguments and errors otherwise as qk_quantize_act. */
int qk_quantize_act_timed(int act_type, const float* x, void* xq, int64_t n, int64_t ncols,
                          void* stream, void* ev_start, void* ev_stop);

/*
 * qk_quantize_row - quantize f32 weights into GGUF blocks (quantize_row_*_ref).
 *   type      QK_TYPE_Q8_0, Q4_0, Q4_1 or Q5_0 (else QK_E_TYPE).
 *   x         f32 [n], device, 16-byte aligned.
 *   dst       out: n / 32 blocks (qk_row_bytes(type, n) bytes), device.
 *   n         >= 0, a multiple of 32; 0 enqueues nothing.
 * Per 32-element block (codeloopback Examples 2, 5, 7, 8; every float operation
 * rounded on its own, never fused):
 *   Q8_0  as qk_quantize_act.
 *   Q4_0  max = the first element of largest |x|; d = max / -8; id = 1/d (0 when
 *         d is 0); code = min(15, trunc(x * id + 8.5)); f16 d, then 16 bytes whose
 *         low nibble is element j and high nibble element j + 16.
 *   Q4_1  d = (max - min) / 15; code = min(15, trunc((x - min) * id + 0.5)); f16 d,
 *         f16 min, then the nibbles as Q4_0 (codes use the unrounded d and min).
 *   Q5_0  max as Q4_0; d = max / -16; code = min(31, trunc(x * id + 16.5)); f16 d,
 *         a 32-bit word whose bit e is bit 4 of code e, then the low 4 bits as Q4_0.
 * trunc is the (int) cast of the listings in those examples: toward zero,
 * saturating at the int32 limits, NaN -> 0; the stored bits are its low 4 (or 5).
 * It departs from plain truncation only when 1/d overflows to infinity, which
 * happens for blocks whose scale is below 2^-128.  Inputs must be finite; the
 * bytes are identical to that definition.
 */
int qk_quantize_row(int type, const float* x, void* dst, int64_t n, void* stream);

/*
 * qk_gemv - y = W x for quantized W and already-quantized activations.
 *   w_type    QK_TYPE_Q8_0, Q4_0, Q5_0, Q4_1, Q5_1, Q2_K, Q3_K, Q4_K, Q5_K or Q6_K
 *             (else QK_E_TYPE).
 *   W         n_out rows of qk_row_bytes(w_type, n_in) bytes, contiguous, row-major
 *             (sipllm matmul_quant layout), device.
 *   n_out     output rows, >= 0.
 *   n_in      elements per row, a positive multiple of the block size,
 *             <= qk_max_n_in(w_type) (else QK_E_LIMIT).
 *   xq        ncols activation rows from qk_quantize_act(qk_act_type(w_type), ...).
 *   ncols     number of activation columns (tokens), >= 0.
 *   y         out: f32 [ncols][n_out], device.
 * For every (row, block): the exact int32 sums of code products (VecDot, rml
 * "Quantized dot products"; the Q4_K / Q5_K min term taken from the activation bsums), then
 * one f32 step with the block scales; y is the f32 sum of those steps.  Q4_1 and Q5_1:
 * s * (d_w * d_x) + m_w * s_x, with s_x the Q8_1 block's f16 sum field.  Q2_K as
 * Q4_K over 16-element sub-blocks; Q3_K as Q6_K with codes - 4 and scales - 32.  The
 * summation order differs from a sequential loop, so y matches a sequential f32
 * evaluation to within rounding, not bit for bit.  Several columns: Q4_K at 2
 * columns (3 up to 8192 rows), Q8_0, Q4_0, Q5_0, Q5_K and Q6_K in groups of up to 4 columns run a GEMV
 * kernel that reads W once for all its columns (each column's arithmetic as the
 * one-column kernel's); Q4_K otherwise runs on the int8 matrix cores, up to 64
 * columns per launch (same per-block integers, y equal to within rounding); every
 * other case, and rows too long for the shared activation buffer, runs the
 * one-column kernels per column.
 * Errors: QK_E_TYPE; QK_E_SHAPE (n_in not whole blocks, a negative count, or
 * n_out above INT32_MAX); QK_E_LIMIT (n_in above qk_max_n_in, or a launch beyond
 * 2^32 - 1 work-items); QK_E_NULL / QK_E_ALIGN for W, xq, y; QK_E_DEVICE.
 */
int qk_gemv(int w_type, const void* W, int64_t n_out, int64_t n_in, const void* xq,
            int64_t ncols, float* y, void* stream);

/*
 * qk_gemv_typed - qk_gemv with the activation blocks' type stated by the caller.
 * Each weight format is multiplied against one activation format whose blocks line
 * up with its own, and an unpaired combination has no dot product (rml "Quantized
 * dot products"; candle "VecDotType" table).
 *   act_type  the type xq was quantized to; must equal qk_act_type(w_type).
 *   other arguments as qk_gemv.
 * Errors: QK_E_TYPE when w_type is not a weight type or act_type not an activation
 * type; QK_E_PAIR when act_type is not qk_act_type(w_type); then as qk_gemv.  The
 * checks run on the host before anything is enqueued.
 */
int qk_gemv_typed(int w_type, int act_type, const void* W, int64_t n_out, int64_t n_in,
                  const void* xq, int64_t ncols, float* y, void* stream);

/*
 * qk_dequantize_row - expand n elements (whole blocks) of a weight type to f32.
 *   type      QK_TYPE_Q8_0, Q4_0, Q4_1, Q5_0, Q5_1, Q2_K, Q3_K, Q4_K, Q5_K or Q6_K
 *             (Q8_1 and Q8_K are activation-only formats and are refused with
 *             QK_E_TYPE, as sipllm's dequantize_row refuses them).
 *   src       n / block blocks, device.  A whole matrix is n = n_out * n_in.
 *   dst       out: f32 [n], device.
 *   n         >= 0, a multiple of the block size; 0 enqueues nothing.
 * Values (rml DequantizeRow; candle block table; codeloopback Examples 7, 8): Q8_0
 * d*q; Q4_0 d*(q-8); Q4_1 and Q5_1 q*d + m; Q5_0 d*(q-16); Q2_K, Q4_K and Q5_K
 * d*sc_j*q - dmin*m_j; Q3_K d*(sc_j-32)*(q-4); Q6_K d*sc_j*(q-32).  Each product is
 * exact in f32 (at most one rounding, in the final addition of Q4_1, Q5_1, Q2_K, Q4_K
 * and Q5_K), so the result
 * is bit-exact.
 * Q5_1 (24 B): d f16 @0, m f16 @2, qh u32 @4, qs[16] @8 (the _1 types add an f16 min
 * to the _0 block; the order is GGUF's); code as Q5_0's, unsigned 0..31.
 * Q5_K (176 B): d f16 @0, dmin f16 @2, scales[12] @4 packed as Q4_K's, qh[32] @16,
 * qs[128] @48; element e = 64c + p: low 4 bits as Q4_K's (qs[32c + p % 32], low
 * nibble for p < 32, else high), bit 4 = bit 2c + (p >= 32) of qh[p % 32].
 * Q2_K (84 B): scales[16] @0 (sub-block j of 16 elements: scale = low nibble, min =
 * high nibble), qs[64] @16, d f16 @80, dmin f16 @82; element e, h = e / 128,
 * r = e % 128, g = r / 32, l = r % 32: code (qs[32h + l] >> 2g) & 3.
 * Q3_K (110 B): hmask[32] @0, qs[64] @32, scales[12] @96, d f16 @108; element e (h,
 * g, l as Q2_K): low 2 bits (qs[32h + l] >> 2g) & 3, bit 2 = bit 4h + g of hmask[l];
 * sub-block j's 6-bit scale: low 4 bits the low nibble of scales[j] (j < 8) or the
 * high nibble of scales[j - 8], high 2 bits (scales[8 + j % 4] >> 2(j / 4)) & 3.
 * Q6_K (210 B): ql[128] @0, qh[64] @128, int8 scales[16] @192, d f16 @208; element
 * e, h = e / 128, r = e % 128, g = r / 32, l = r % 32: low 4 bits the low (g < 2)
 * or high nibble of ql[64h + l + 32 (g & 1)], high 2 bits (qh[32h + l] >> 2g) & 3.
 */
int qk_dequantize_row(int type, const void* src, float* dst, int64_t n, void* stream);

/*
 * qk_gemv_block_sums - the same GEMV kernels, storing the per-block integers they
 * compute instead of y.  For checking exactness; not needed to use the library.
 *   sums      out: int32 [ncols][n_out][n_in / block][k]; k = 2 for Q2_K, Q4_K, Q5_K (the scale
 *             sum S_q = sum_j sc_j s_j and the min sum S_m = sum_j m_j sum(a_j)),
 *             k = 1 otherwise (Q8_0, Q4_0, Q5_0, Q4_1, Q5_1: the block's code-product sum; Q3_K, Q6_K:
 *             S = sum_j sc_j sum (q - 32) a).
 * Other arguments and errors as qk_gemv.
 */
int qk_gemv_block_sums(int w_type, const void* W, int64_t n_out, int64_t n_in,
                       const void* xq, int64_t ncols, int32_t* sums, void* stream);

/*
 * qk_gemv_timed - qk_gemv whose kernel launches carry two hipEvent_t that record
 * the start of the first and the end of the last GEMV kernel themselves (HIP's
 * extended launch), for measuring kernel duration without enqueue gaps.  Either
 * event may be NULL.  Arguments and errors otherwise as qk_gemv.
 */
int qk_gemv_timed(int w_type, const void* W, int64_t n_out, int64_t n_in, const void* xq,
                  int64_t ncols, float* y, void* stream, void* ev_start, void* ev_stop);

/*
 * qk_gemv_pair - the gate and up projections of an FFN layer in one launch: two
 * GEMVs of the same shape over the same activation columns, y1 = W1 x and
 * y2 = W2 x.  Each row is computed in both matrices from one load of the
 * activation operands (candle formats page, "实测：一次点积": vec_dot_4, one
 * activation row against several weight rows with the activation loaded once).
 *   w_type    QK_TYPE_Q4_K or QK_TYPE_Q5_K (else QK_E_TYPE); x blocks are Q8_K.
 *   W1, W2    n_out rows of qk_row_bytes(w_type, n_in) bytes each, device.
 *   n_out, n_in, xq, ncols   as qk_gemv; ncols <= 65535 (else QK_E_LIMIT).
 *   epilogue  QK_EPI_NONE: out is f32 [ncols][2][n_out], y1 then y2 per column.
 *             QK_EPI_SWIGLU: out is f32 [ncols][n_out], silu(y1) * y2 with
 *             silu(v) = v / (1 + e^-v) in f32: the gated activation that the down
 *             projection of the layer consumes (the pages stop at the products;
 *             this is the SwiGLU form of the 7B-shape layers).
 *             Any other value: QK_E_ARG.
 * Every column runs the one-column GEMV kernels' arithmetic (same integer sums,
 * float steps and summation order), so with ncols = 1 QK_EPI_NONE returns what
 * qk_gemv returns bit for bit; with more Q4_K columns qk_gemv uses the matrix cores
 * and the two agree to within rounding.  Errors otherwise as qk_gemv.
 */
int qk_gemv_pair(int w_type, const void* W1, const void* W2, int64_t n_out, int64_t n_in,
                 const void* xq, int64_t ncols, int epilogue, float* out, void* stream);

/* qk_gemv_pair_timed - qk_gemv_pair whose single kernel launch records ev_start and
 * ev_stop itself, as qk_gemv_timed.  Arguments and errors otherwise as qk_gemv_pair. */
int qk_gemv_pair_timed(int w_type, const void* W1, const void* W2, int64_t n_out, int64_t n_in,
                       const void* xq, int64_t ncols, int epilogue, float* out, void* stream,
                       void* ev_start, void* ev_stop);

/*
 * qk_read_probe - measurement probe, not part of the method: a kernel that only
 * reads `bytes` bytes of device memory, timed like the GEMV, gives the HBM read
 * bandwidth one launch of that size reaches on the machine (start-up and drain
 * included).  A GEMV's weight bandwidth is reported against it as well as against
 * the vendor peak.
 *   src       device buffer, 16-byte aligned, `bytes` readable bytes.
 *   bytes     > 0 and a multiple of 16 (else QK_E_SHAPE).
 *   out       device uint32 [ceil(bytes / 2048)], 16-byte aligned: word g is the
 *             XOR of the 32-bit little-endian words of bytes [2048 g, 2048 g + 2048)
 *             (the last group only up to `bytes`), so a test can check the read.
 *   stream, ev_start, ev_stop   as qk_gemv_timed (either event may be NULL).
 * QK_E_NULL for a NULL src or out, QK_E_ALIGN for a misaligned one.
 */
int qk_read_probe(const void* src, int64_t bytes, uint32_t* out, void* stream, void* ev_start,
                  void* ev_stop);

/*
 * qk_read_probe_ex - qk_read_probe with its load pattern as arguments, so a sweep
 * can look for the fastest way one launch reads a given number of bytes.
 *   kb_per_wave   1, 2, 4, 8 or 16: each wavefront reads one group of that many
 *                 kilobytes (kb_per_wave 16-byte loads per lane, all issued before
 *                 any use); out word g is the XOR of the 32-bit words of group g,
 *                 out holds ceil(bytes / (1024 kb_per_wave)) words.
 *   grid_blocks   0: one wavefront per group (qk_read_probe); > 0: a persistent grid
 *                 of that many 256-thread workgroups (at most one per four groups)
 *                 whose wavefronts stride over the groups.
 *   nontemporal   0: plain loads; 1: non-temporal (streaming) loads.
 * QK_E_ARG for any other kb_per_wave, a negative grid_blocks or another
 * nontemporal value; otherwise as qk_read_probe (qk_read_probe is this call with
 * 2, 0, 0).
 */
int qk_read_probe_ex(const void* src, int64_t bytes, uint32_t* out, int kb_per_wave, int64_t grid_blocks,
                     int nontemporal, void* stream, void* ev_start, void* ev_stop);

#ifdef __cplusplus
}
#endif
#endif
