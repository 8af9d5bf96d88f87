/*
 * qk_oracle.h - plain scalar CPU oracle for ggml block-quantized GEMV.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this code: only tests, the smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no code, header or constant with the HIP library; it keeps
 * its own copy of the block layouts on purpose.
 *
 * Every routine is written element by element, in the order the pages define
 * the formats, not for speed.  Sources (page title, then section):
 *   [rml]     "Quantization" (rayaq.ca/rml/quantization)
 *   [sipllm]  "Quantization" (ankit1057.github.io/sipllm-docs)
 *   [cl]      "Building Q8_0 and Q4_0 Like ggml" (codeloopback.dev), Examples 1-14
 *   [candle]  "量化格式" (rustineverything.app/docs/candle/06-quantized/formats)
 *
 * Parity status per function (what pins it is listed in tests/test_oracle_pins.py):
 *   f16 conversion, quantize_q8_0, quantize_q4_0, dequantize Q8_0/Q4_0,
 *   vec_dot Q8_0xQ8_0 and Q4_0xQ8_0: pinned by printed bytes and values.
 *   dequantize Q4_K: pinned by the [rml] element-200 trace and [candle]
 *   get_scale_min_k4 prose, plus brute force.
 *   vec_dot Q4_KxQ8_K / Q6_KxQ8_K: pinned by brute force against the dequant
 *   definitions and by the bsums identity.
 *   quantize_q8_K: the pages give its layout, and for its scale rule only the
 *   round-trip statistics of [candle] "往返误差"; the rule taken is the Q8_0 one
 *   over 256 elements, pinned by those statistics and by invariants.
 *   Q6_K ql/qh bit arrangement: parity unpinned (the pages give only the field
 *   roles); the GGUF arrangement is assumed.
 *   dequantize Q5_1: the pages give its size (24 bytes) and that the _1 types add
 *   an f16 min to the _0 layout; the field order (d, m, qh, qs) is GGUF's.  With no
 *   fifth bit set it reduces to the pinned Q4_1 decoder; dequantize only, as Q4_1.
 *   Q5_K field order and fifth-bit arrangement: parity unpinned (the pages give
 *   its size and that it shares Q4K's d, dmin and 6-bit scales and mins); the
 *   GGUF arrangement is assumed.  With every fifth bit clear it reduces to the
 *   pinned Q4_K decoder; vec_dot Q5_KxQ8_K is pinned by brute force against its
 *   dequant definition, as the other K-quants are.
 *   quantize / dequantize Q4_1 and Q5_0, vec_dot Q5_0xQ8_0: pinned by the [cl]
 *   Example 7, 8, 12 and 14 printed values and bytes, plus brute force.
 *   quantize_q8_1 and vec_dot Q4_1xQ8_1 / Q5_1xQ8_1: [candle] names BlockQ8_1 as
 *   the activation format of the _1 types (VecDotType table) without printing its
 *   layout.  The reading taken: d f16 @0, s f16 @2, 32 int8 codes @4 (36 bytes);
 *   d and the codes follow the Q8_0 rule, s = f16(d * sum of codes) with the
 *   unrounded f32 d, the sum the weight minimum's term needs (as BlockQ8K's bsums
 *   serve Q4K's min term).  Codes and d are pinned by the printed Q8_0 bytes; s by
 *   a hand-worked block; the dot product by f64 brute force over the pinned Q4_1
 *   decoder within the bound of s's f16 rounding, and its integer sum exactly.
 *   Q2_K and Q3_K: parity unpinned.  The pages give their size (84 and 110 bytes
 *   per 256 elements, [candle] GgmlDType table), that they are K-quants (16-element
 *   sub-blocks with small integer scales times the f16 d, [rml] summary) and that
 *   dequantize_row handles them ([sipllm] Per-format dequant), not their field
 *   order or bit arrangement; the GGUF arrangement is assumed (stated at the
 *   decoders).  Pinned: sizes, structure any arrangement of those fields has (each
 *   code bit moves one element, each scale field one 16-element sub-block), and the
 *   dot products by f64 brute force against the dequantizer.
 */
#ifndef QK_ORACLE_H
#define QK_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* GGUF type ids (ggml's numbering, which is what a GGUF tensor record stores). */
#define ORC_Q4_0 2
#define ORC_Q4_1 3
#define ORC_Q5_0 6
#define ORC_Q5_1 7
#define ORC_Q8_0 8
#define ORC_Q8_1 9
#define ORC_Q2_K 10
#define ORC_Q3_K 11
#define ORC_Q4_K 12
#define ORC_Q5_K 13
#define ORC_Q6_K 14
#define ORC_Q8_K 15

/* Return codes. */
#define ORC_OK 0
#define ORC_BAD_TYPE (-1)
#define ORC_BAD_SHAPE (-2)
#define ORC_BAD_PAIR (-3)
#define ORC_INCONSISTENT (-4) /* two independent routes to one integer disagreed */

int64_t orc_block_elems(int type);
int64_t orc_block_bytes(int type);
int64_t orc_row_bytes(int type, int64_t n);
int orc_act_type(int weight_type);

float orc_f16_to_f32(uint16_t h);
uint16_t orc_f32_to_f16(float f);

int orc_quantize_q8_0(const float* x, uint8_t* out, int64_t n);
int orc_quantize_q8_K(const float* x, uint8_t* out, int64_t n);
int orc_quantize_q4_0(const float* x, uint8_t* out, int64_t n);
int orc_quantize_q4_1(const float* x, uint8_t* out, int64_t n);
int orc_quantize_q5_0(const float* x, uint8_t* out, int64_t n);
int orc_quantize_q8_1(const float* x, uint8_t* out, int64_t n);

int orc_dequantize(int type, const uint8_t* src, float* dst, int64_t n);

int64_t orc_sums_per_block(int weight_type);
int orc_block_sums(int weight_type, const uint8_t* w, const uint8_t* xq, int64_t n,
                   int32_t* sums);
int orc_vec_dot(int weight_type, const uint8_t* w, const uint8_t* xq, int64_t n,
                float* out, double* l1);
int orc_gemv(int weight_type, const uint8_t* W, int64_t n_out, int64_t n_in,
             const uint8_t* xq, int64_t ncols, float* y, double* l1);
int orc_gemv_block_sums(int weight_type, const uint8_t* W, int64_t n_out, int64_t n_in,
                        const uint8_t* xq, int64_t ncols, int32_t* sums);
int orc_swiglu(const float* g, const float* u, int64_t n, double* h);

#ifdef __cplusplus
}
#endif
#endif
