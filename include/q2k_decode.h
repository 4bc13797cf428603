/*
 * q2k_decode.h - C ABI of the MI355X (gfx950) Q2_K quantised decode library
 * (libq2kdecode.so).
 *
 * The operations are the single-token (m <= 8) decode path of a 2-bit
 * k-quant model as the metrale engine pages describe it:
 *   - q8_1 quantisation of bf16 activation rows   (moe_v41/init.rs: the
 *     kquant_q8_1_rows_bf16 kernel and kquant_q8_1_rows_bytes sizing;
 *     attn_v41/decode.rs, q_kv_projections: one quantisation for two matrices)
 *   - the Q2_K x q8_1 matrix-vector product, single / shared-input pair /
 *     expert-id batch (kquant_mmvq_q2_k_w, mmvq_q2k_pair_w,
 *     kquant_mmvq_q2_k_experts_w*)
 *   - fused bf16 SwiGLU + q8_1 re-quantisation (kquant_swiglu_q8_1_rows_bf16)
 *   - engram Q2_K row gather + dequantisation to bf16 (engram_v41.rs,
 *     EngramV41::rows_from_q2k and its dequant_q2_k_to_bf16 launch)
 *   - the engram gate (engram_v41/apply.rs, the engram_v41_gate launch;
 *     engram_v41.rs module doc, step 4)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers named *_dev, and every tensor argument, are DEVICE pointers on the
 * current HIP device; `bases` in q2k_mmvq_experts is a HOST array of device
 * pointers. `stream` is a hipStream_t passed as void* (NULL = the null
 * stream). The caller owns every buffer and the stream. The library never
 * allocates, frees or synchronises: each call only enqueues kernels on
 * `stream` and returns, so every call may be captured in a HIP graph.
 *
 * Every argument check runs on the host before any HIP call, in release
 * builds too. Return values: Q2K_OK (0) or a negative Q2K_E* code;
 * q2k_last_error() then gives a message (thread-local, valid until the next
 * failing call on that thread). Data errors that only the device can see
 * (an expert id or a table row id out of range) write NaN into the affected
 * output rows and store 1 into *err_flag_dev when that pointer is non-NULL;
 * the flag is never cleared by the library.
 *
 * Q2_K weights are GGUF Q2_K super-blocks, unchanged: 84 bytes per 256
 * weights (engram_v41.rs, const ENGRAM_ROW_BYTES and the
 * EngramLayerWeights::wkv_q2k doc), laid out scales[16] (low nibble = scale,
 * high nibble = min), qs[64] (2-bit quants; element 128h+32j+l is bits
 * 2j..2j+1 of qs[32h+l], sub-block 8h+2j+(l>=16)), fp16 d, fp16 dmin. A
 * matrix [n, k] is n rows of k/256 consecutive blocks (row-major, no
 * padding); its base must be 4-byte aligned.
 *
 * q8_1 activation rows use this library's own layout, sized by
 * q8_1_rows_bytes(): per row of k values, k int8 quants, then k/32 f32 block
 * scales, then k/16 int16 sums of each 16 quants. Treat it as opaque.
 */
#ifndef Q2K_DECODE_H
#define Q2K_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define Q2K_API __attribute__((visibility("default")))
#else
#define Q2K_API
#endif

#define Q2K_ABI_VERSION 5

#define Q2K_OK 0
#define Q2K_EINVAL (-1)   /* NULL pointer, or pointers that must not overlap do */
#define Q2K_ESHAPE (-2)   /* k % 256 != 0, m outside 1..8, n <= 0, hc outside 1..4, ... */
#define Q2K_ESPACE (-3)   /* an output or workspace is smaller than required */
#define Q2K_EALIGN (-4)   /* a pointer or stride is not aligned as documented */
#define Q2K_ELAUNCH (-5)  /* the HIP launch itself failed (hipGetLastError) */
#define Q2K_EDEVICE (-6)  /* no usable HIP device for the query the call needs */

/* Largest token count of the product entry points (the pages take the
 * Q2_K route for m <= 8 only: attn_v41/decode.rs, q_kv_projections). */
#define Q2K_MAX_M 8

/* Version of this ABI (Q2K_ABI_VERSION). */
Q2K_API int32_t q2k_abi_version(void);

/* Message for the last non-zero return on the calling thread ("" if none). */
Q2K_API const char* q2k_last_error(void);

/* Bytes of `m` q8_1 rows of `k` values (cf. kquant_q8_1_rows_bytes in
 * moe_v41/init.rs): m * k * 5 / 4. Returns 0 when m < 1 or k is not a
 * positive multiple of 256. */
Q2K_API size_t q8_1_rows_bytes(int32_t m, int32_t k);

/* q8_1 quantisation of bf16 rows (kquant_q8_1_rows_bf16, moe_v41/init.rs;
 * used once per input in attn_v41/decode.rs q_kv_projections).
 *   x_bf16_dev : bf16 [m, k], row i at x + i * x_row_stride elements;
 *                16-byte aligned base, x_row_stride % 8 == 0, >= k.
 *   xq_dev     : output, q8_1_rows_bytes(m, k) bytes (xq_bytes must be at
 *                least that), 16-byte aligned.
 *   m >= 1 rows, k % 256 == 0.
 * Per 32-wide block: amax = max|x|, d = amax/127 (correctly rounded f32
 * division), q = round-half-away(x/d) in -127..127 (0 when amax == 0). */
Q2K_API int32_t q8_1_rows(const void* x_bf16_dev, int64_t x_row_stride, void* xq_dev,
                  size_t xq_bytes, int32_t m, int32_t k, void* stream);

/* Q2_K x q8_1 product, one matrix (kquant_mmvq_q2_k_w, moe_v41/init.rs;
 * the engram wkv projection of engram_v41/apply.rs).
 *   w_dev  : Q2_K [n, k], 4-byte aligned.
 *   xq_dev : q8_1 rows [m, k] from q8_1_rows, 16-byte aligned.
 *   y_dev  : f32 [m, n] (row t at y + t*n), 4-byte aligned; must not
 *            overlap w or xq.
 *   1 <= m <= 8, n >= 1, k % 256 == 0.
 * y[t][r] = sum over the row's blocks b and q8 blocks c of
 *           d8[t][c] * (d_b * I - dmin_b * M), I and M exact int32 sums,
 * evaluated in one fixed order that every product kernel of this library
 * follows, so that all of them (and every entry point that computes this
 * product: pair, expert, grouped, fused and mmq forms) return the same bits:
 *   - per half block (super-block b, half h, q8 blocks c = 8b+4h+j, j=0..3):
 *     fI = ((d8_0*I_0 + d8_1*I_1) + d8_2*I_2) + d8_3*I_3 in fp64, one fma per
 *     term starting from +0 (each product is exact), fM likewise with M, and
 *     v = RN(d_b*fI) - RN(dmin_b*fM);
 *   - per half h, a pairwise tree over b = 0..NBP-1 (NBP = k/256 rounded up
 *     to a power of two; leaves past the row are +0), neighbours first;
 *   - y = f32(T_0 + T_1), rounded once.
 * The pages fix no order; this one keeps the result within ~2^-50 relative
 * of the exact sum and independent of the launch shape. */
Q2K_API int32_t q2k_mmvq(const void* w_dev, const void* xq_dev, float* y_dev,
                 int32_t n, int32_t k, int32_t m, void* stream);

/* q8_1_rows and then q2k_mmvq in one call, with the same bytes in xq and
 * the same bits in y as the two calls (attn_v41/decode.rs and moe_v41/init.rs
 * quantise an input once and then run its products; here the quantisation
 * can live inside the product). For rows of 1024..8192 values on the
 * packed-dot run kernel (at least 2048 row steps x tokens) it is one
 * launch: each workgroup quantises the bf16 row of its token into LDS while
 * its first weight loads are in flight (with 2..8 tokens each workgroup
 * takes one token), and one workgroup per token writes its q8_1 row to xq;
 * otherwise (fewer row steps, the matrix cores) a q8_1 launch runs ahead of
 * the product.
 *   w_dev, y_dev, n, k, m : as in q2k_mmvq (m in 1..8).
 *   x_bf16_dev, x_row_stride : as in q8_1_rows.
 *   xq_dev, xq_bytes : output, the q8_1 rows (q8_1_rows_bytes(m, k)),
 *                      16-byte aligned, overlapping no input.
 * Errors: those of q8_1_rows and q2k_mmvq; y may not overlap w, x or xq. */
Q2K_API int32_t q8_1_q2k_mmvq(const void* w_dev, const void* x_bf16_dev, int64_t x_row_stride,
                              void* xq_dev, size_t xq_bytes, float* y_dev, int32_t n, int32_t k,
                              int32_t m, void* stream);

/* Two Q2_K matrices that read the same q8_1 rows, in one launch
 * (mmvq_q2k_pair_w via kquant_mmvq_pair_w, attn_v41/decode.rs
 * q_kv_projections: wq_a and wkv). ya_dev f32 [m, na], yb_dev f32 [m, nb];
 * each as in q2k_mmvq; the two outputs must not overlap. */
Q2K_API int32_t q2k_mmvq_pair(const void* wa_dev, float* ya_dev, int32_t na,
                      const void* wb_dev, float* yb_dev, int32_t nb,
                      const void* xq_dev, int32_t k, int32_t m, void* stream);

/* q8_1_rows and then q2k_mmvq_pair in one call (attn_v41/decode.rs
 * q_kv_projections quantises the input once for wq_a and wkv), with the same
 * bytes in xq and bits in ya, yb as the two calls. Where the pair takes the
 * packed-dot run kernel (at least 2048 row steps x tokens, rows of
 * 1024..8192 values) it is one launch, the quantisation inside the product
 * as in q8_1_q2k_mmvq; otherwise a q8_1 launch runs ahead of the pair.
 *   wa_dev .. nb, k, m : as in q2k_mmvq_pair.
 *   x_bf16_dev, x_row_stride : bf16 [m, k] as in q8_1_rows.
 *   xq_dev, xq_bytes : output, q8_1_rows_bytes(m, k) bytes, 16-byte aligned.
 * Errors: those of q8_1_rows and q2k_mmvq_pair; xq may not overlap x or the
 * matrices, nor an output overlap x. */
Q2K_API int32_t q8_1_q2k_mmvq_pair(const void* wa_dev, float* ya_dev, int32_t na,
                                   const void* wb_dev, float* yb_dev, int32_t nb,
                                   const void* x_bf16_dev, int64_t x_row_stride, void* xq_dev,
                                   size_t xq_bytes, int32_t k, int32_t m, void* stream);

/* Expert-id batch (kquant_mmvq_q2_k_experts_w*, moe_v41/init.rs: gate and
 * up run as one batch of 2*ne matrices, up read at gate_out + ne*inter).
 *   bases      : HOST array of n_bases (1..4) device pointers; base j holds
 *                n_experts Q2_K matrices [n, k], expert e at
 *                bases[j] + e * expert_stride_bytes (stride >= n*k/256*84,
 *                multiple of 4).
 *   ids_dev    : int32 [n_ids] expert ids (device); 1 <= n_ids <= 64.
 *   xq_dev     : x_per_id == 0: q8_1 rows [m, k] shared by every matrix;
 *                x_per_id == 1: q8_1 rows [n_ids * m, k], id i reads rows
 *                i*m .. i*m+m-1.
 *   y_dev      : f32 [n_bases, n_ids, m, n], in id-list order.
 *   err_flag_dev : nullable int32; an id outside [0, n_experts) NaN-fills
 *                its outputs and stores 1 here.
 * Only the selected experts' matrices are read. */
Q2K_API int32_t q2k_mmvq_experts(const void* const* bases, int32_t n_bases,
                         int64_t expert_stride_bytes, int32_t n_experts,
                         const int32_t* ids_dev, int32_t n_ids,
                         const void* xq_dev, int32_t x_per_id, float* y_dev,
                         int32_t n, int32_t k, int32_t m,
                         int32_t* err_flag_dev, void* stream);

/* q8_1_rows of one shared input and then q2k_mmvq_experts on it
 * (x_per_id = 0: the gate/up form of moe_v41/init.rs), in one call with the
 * same bytes in xq and bits in y as the two calls. For one token on the
 * run kernel it is one launch (each workgroup quantises x into LDS while
 * its first weight loads are in flight; workgroup 0 writes xq); otherwise a
 * q8_1 launch runs ahead of the product.
 *   bases .. n_ids, y_dev, n, k, m, err_flag_dev : as in q2k_mmvq_experts.
 *   x_bf16_dev, x_row_stride : bf16 [m, k] as in q8_1_rows.
 *   xq_dev, xq_bytes : output, q8_1_rows_bytes(m, k) bytes, 16-byte aligned.
 * Errors: those of q8_1_rows and q2k_mmvq_experts; x, xq, y, ids and the
 * expert sets may not overlap. */
Q2K_API int32_t q8_1_q2k_mmvq_experts(const void* const* bases, int32_t n_bases,
                                      int64_t expert_stride_bytes, int32_t n_experts,
                                      const int32_t* ids_dev, int32_t n_ids,
                                      const void* x_bf16_dev, int64_t x_row_stride, void* xq_dev,
                                      size_t xq_bytes, float* y_dev, int32_t n, int32_t k,
                                      int32_t m, int32_t* err_flag_dev, void* stream);

/* q8_1_q2k_mmvq_experts on the gate and up sets of one token followed by
 * swiglu_q8_1_rows of its two result sets (moe_v41/init.rs: the gate/up
 * product, then kquant_swiglu_q8_1_rows_bf16 ahead of the down product),
 * in one call with the same bits in y and bytes in xq, h and hq as those
 * calls in sequence. For rows of 2048 to 8192 values and n a multiple of 64
 * on the run kernel it is one launch: each workgroup takes 64 rows of one
 * id in both sets (its waves 32 consecutive rows each) and, after its
 * product, forms their bf16 SwiGLU and the two q8_1 blocks of h in its
 * epilogue. Otherwise the SwiGLU launch follows the product.
 *   bases[0], bases[1] : the gate and up expert sets, as in q2k_mmvq_experts.
 *   expert_stride_bytes, n_experts, ids_dev, n_ids, err_flag_dev : as there.
 *   x_bf16_dev : bf16 [1, k], 16-byte aligned; xq_dev, xq_bytes : output,
 *                its q8_1 row (q8_1_rows_bytes(1, k)), 16-byte aligned.
 *   y_dev      : output, f32 [2, n_ids, n] (gate rows, then up rows).
 *   h_bf16_dev : nullable output, bf16 [n_ids, n], 16-byte aligned.
 *   hq_dev, hq_bytes : output, the q8_1 rows of h (q8_1_rows_bytes(n_ids, n)),
 *                16-byte aligned: the input of the down product
 *                (q2k_mmvq_experts with x_per_id = 1).
 *   n % 256 == 0 (h is a q8_1 row of n values), k % 256 == 0.
 * Errors: those of q8_1_q2k_mmvq_experts and swiglu_q8_1_rows; no output
 * may overlap another buffer of the call. */
Q2K_API int32_t q8_1_q2k_mmvq_experts_swiglu(const void* const* bases, int64_t expert_stride_bytes,
                                             int32_t n_experts, const int32_t* ids_dev,
                                             int32_t n_ids, const void* x_bf16_dev, void* xq_dev,
                                             size_t xq_bytes, float* y_dev, void* h_bf16_dev,
                                             void* hq_dev, size_t hq_bytes, int32_t n, int32_t k,
                                             int32_t* err_flag_dev, void* stream);

/* swiglu_q8_1_rows of gate and up rows and then the down product on them
 * (q2k_mmvq_experts with x_per_id = 1, one token), in one call with the
 * same bytes in hq and bits in y as the two calls (moe_v41/init.rs:
 * kquant_swiglu_q8_1_rows_bf16 between the gate/up and down products). For
 * rows of at most 2048 values on the run kernel, with every workgroup
 * inside one id's waves, it is one launch: each workgroup forms its id's
 * bf16 SwiGLU and q8_1 row in LDS while its first weight loads are in
 * flight; the workgroup holding the id's first wave writes that row to hq.
 * Otherwise a SwiGLU launch runs ahead of the product.
 *   bases .. n_ids, y_dev, n, k, err_flag_dev : as in q2k_mmvq_experts
 *                (y f32 [n_bases, n_ids, n]).
 *   g_dev, u_dev : f32 [n_ids, k] gate and up rows (row i for the i-th id),
 *                  16-byte aligned.
 *   hq_dev, hq_bytes : output, the q8_1 rows of h (q8_1_rows_bytes(n_ids, k)),
 *                  16-byte aligned.
 * Errors: those of swiglu_q8_1_rows and q2k_mmvq_experts; hq may not
 * overlap g, u, ids or the expert sets, nor y overlap g or u. */
Q2K_API int32_t swiglu_q2k_mmvq_experts(const void* const* bases, int32_t n_bases,
                                        int64_t expert_stride_bytes, int32_t n_experts,
                                        const int32_t* ids_dev, int32_t n_ids, const float* g_dev,
                                        const float* u_dev, void* hq_dev, size_t hq_bytes,
                                        float* y_dev, int32_t n, int32_t k,
                                        int32_t* err_flag_dev, void* stream);

/* Q2_K x q8_1 product for any number of tokens (prefill, batched verify):
 * the pages' route past 8 tokens (moe_v41/init.rs, MoeV41::new: the
 * metrale_q2_k_mmq128_{nc,wc} kernels and the mmq activation buffers sized
 * beside the q8_1 rows). The same sum as q2k_mmvq for each token,
 * y[t][r] = sum over the row of d8 * (d*I - dmin*M), with the same exact
 * int32 block sums and the same fp64 value per half block, in one of two
 * fixed orders:
 *   m <= 16: the q2k_mmvq kernels on groups of 8 tokens (the pairwise tree
 *            stated at q2k_mmvq; the same bits as q2k_mmvq per group);
 *   m >= 17: the tile kernel (matrix cores, 32 tokens x 64 rows per
 *            workgroup, any row length), whose half-block values are added
 *            to one running fp64 sum in row order, (b, h) = (0,0), (0,1),
 *            (1,0), ..., then rounded to f32.
 *   w_dev  : Q2_K [n, k]; xq_dev : q8_1 rows [m, k]; y_dev : f32 [m, n].
 *   1 <= m <= Q2K_MMQ_MAX_M, k % 256 == 0, m * n <= 2^31; errors as
 *   q2k_mmvq. */
#define Q2K_MMQ_MAX_M 4096
Q2K_API int32_t q2k_mmq(const void* w_dev, const void* xq_dev, float* y_dev, int32_t n,
                        int32_t k, int32_t m, void* stream);

/* Grouped-input product: the Q2_K route of the attention output projection
 * wo_a (attn_v41/decode.rs, the grouped wo_a step of the decode body, taken
 * when wo_a is Q2_K and m <= 8), where output row g*o_rank + r is the dot of
 * wo_a's row with the g-th column slice o_g of the attention output.
 *   w_dev          : Q2_K [groups * rows_per_group, k]; rows g*R .. g*R+R-1
 *                    (R = rows_per_group) belong to group g.
 *   xq_dev         : q8_1 rows [m, groups * k] (q8_1_rows of the whole input
 *                    rows); group g reads elements g*k .. g*k+k-1 of each.
 *   y_dev          : f32 [m, groups * R] (token-major):
 *                    y[t][g*R + r] = sum_e W[g*R + r][e] * x[t][g*k + e].
 *   groups >= 1, rows_per_group >= 1, k % 256 == 0, 1 <= m <= Q2K_MAX_M,
 *   groups * R, groups * k < 2^31. Q2K_ESHAPE otherwise; Q2K_EINVAL for
 *   null pointers or y overlapping w or xq; Q2K_EALIGN as q2k_mmvq. */
Q2K_API int32_t q2k_mmvq_grouped(const void* w_dev, const void* xq_dev, float* y_dev,
                         int32_t groups, int32_t rows_per_group, int32_t k, int32_t m,
                         void* stream);

/* Q2_K weights times bf16 activations: the single-token engram projection
 * read off the raw Q2_K blocks (engram_v41/apply.rs, the
 * engram_v41_wkv_q2k_gemv launch; engram_v41.rs, EngramLayerWeights::wkv_q2k:
 * bit for bit the bf16 GEMV over the bf16 expansion of the blocks).
 *   w_dev        : Q2_K [n, k].
 *   x_bf16_dev   : bf16 [m, k], row stride x_row_stride elements (a multiple
 *                  of 8, >= k), 16-byte aligned. Not quantised.
 *   y_dev        : f32 [m, n].
 * y[t][r] = f32_rne(sum_e bf16(W[r][e]) * x[t][e]) where bf16(W) is the
 * expansion q2k_dequant_rows produces (f32 d*sc*q - dmin*m, one rounding,
 * then bf16 to nearest-even); the bf16 products are exact and are summed in
 * fp64, so the result is the correctly rounded dot product of the expansion
 * for any order (to ~2^-53 of the sum). 1 <= m <= Q2K_MAX_M, k % 256 == 0.
 * Errors as q2k_mmvq (plus Q2K_ESHAPE for a stride < k, Q2K_EALIGN for x). */
Q2K_API int32_t q2k_gemv_bf16(const void* w_dev, const void* x_bf16_dev, int64_t x_row_stride,
                         float* y_dev, int32_t n, int32_t k, int32_t m, void* stream);

/* Fused bf16 SwiGLU and q8_1 re-quantisation
 * (kquant_swiglu_q8_1_rows_bf16, moe_v41/init.rs).
 *   g_dev, u_dev : f32 [rows, k] contiguous (gate and up outputs).
 *   h_bf16_dev   : nullable bf16 [rows, k]; receives h when non-NULL.
 *   hq_dev       : q8_1 rows [rows, k], hq_bytes >= q8_1_rows_bytes(rows, k).
 * h = bf16_rne(silu(g) * u) with silu(g) = g / (1 + exp(-g)) in f32, then
 * hq = q8_1 of h exactly as q8_1_rows would quantise it. */
Q2K_API int32_t swiglu_q8_1_rows(const float* g_dev, const float* u_dev, void* h_bf16_dev,
                         void* hq_dev, size_t hq_bytes, int32_t rows, int32_t k,
                         void* stream);

/* Engram row gather and dequantisation to bf16 (engram_v41.rs,
 * EngramV41::rows_from_q2k, dequant_q2_k_to_bf16): one Q2_K block per
 * 256-wide row.
 *   table_dev    : n_table_rows Q2_K blocks (84 bytes each), 4-byte aligned.
 *   ids_dev      : nullable int64 [n_rows]; NULL reads rows 0..n_rows-1.
 *   out_bf16_dev : bf16 [n_rows, 256].
 *   err_flag_dev : nullable; an id outside [0, n_table_rows) NaN-fills its
 *                  row and stores 1 here.
 * out = bf16_rne(d*sc*q - dmin*m) with the value formed in f32. */
Q2K_API int32_t q2k_dequant_rows(const void* table_dev, int64_t n_table_rows,
                         const int64_t* ids_dev, int32_t n_rows, void* out_bf16_dev,
                         int32_t* err_flag_dev, void* stream);

/* Engram rows gathered, dequantised and quantised to q8_1 in one launch:
 * q2k_dequant_rows followed by q8_1_rows on its output viewed as one row of
 * 256 * n_rows values (the engram step feeds the gathered rows to the wkv
 * projection as one [1, 256 * n_rows] activation: engram_v41/apply.rs,
 * apply; engram_v41.rs module doc steps 2 and 3), with the same bits as
 * those two calls.
 *   table_dev, ids_dev, n_rows, err_flag_dev : as q2k_dequant_rows
 *                  (1 <= n_rows <= 2^20).
 *   out_bf16_dev : nullable bf16 [n_rows, 256], 16-byte aligned; receives
 *                  the dequantised rows when non-NULL.
 *   xq_dev       : one q8_1 row of width 256 * n_rows, 16-byte aligned,
 *                  xq_bytes >= q8_1_rows_bytes(1, 256 * n_rows).
 * Errors: Q2K_EINVAL (null table or xq, outputs overlapping the table or
 * each other), Q2K_ESHAPE, Q2K_ESPACE (xq too small, or contiguous rows past
 * the table), Q2K_EALIGN. */
Q2K_API int32_t q2k_dequant_rows_q8_1(const void* table_dev, int64_t n_table_rows,
                         const int64_t* ids_dev, int32_t n_rows, void* out_bf16_dev,
                         void* xq_dev, size_t xq_bytes, int32_t* err_flag_dev, void* stream);

/* Engram gate, in place on the f32 stream (engram_v41/apply.rs: grid
 * [T, hc], arguments streams, kv, qk, dim, hc, eps; engram_v41.rs module doc
 * step 4).
 *   h_dev  : f32 [t, hc, dim], updated in place.
 *   kv_dev : f32 [t, (hc+1)*dim]: the keys of streams 0..hc-1, then the one
 *            shared value; must not overlap h.
 *   qk_dev : f32 [hc, dim], the product q_weight * k_weight.
 *   1 <= hc <= 4, dim >= 1, t >= 1.
 * For each (t, j): s = sum(qk*h*k) / (rms(h)*rms(k)*sqrt(dim)) with
 * rms(x) = sqrt(mean(x^2) + eps); g = sigmoid(sign(s)*sqrt|s|);
 * h += g * value. */
Q2K_API int32_t engram_gate(float* h_dev, const float* kv_dev, const float* qk_dev,
                    int32_t t, int32_t hc, int32_t dim, float eps, void* stream);

/* Engram n-gram hash: the row ids each hashed layer gathers (engram_v41.rs,
 * EngramHasher::hash and EngramHasher::layer_row_ids; the tables are
 * EngramHashTables). The pages run it on the host; here it runs on the
 * device next to the table.
 *   token_map_dev    : int64 [vocab] compressed id per token id, -1 = unmapped.
 *   multipliers_dev  : int64 [n_layers, max_ngram].
 *   primes_dev       : int64 [n_layers, max_ngram - 1, n_heads], each > 0.
 *   offsets_dev      : int64 [n_layers, (max_ngram - 1) * n_heads].
 *   cache_dev        : int64 [cache_len], the sequence's compressed ids by
 *                      position (the hasher state). Positions < start_pos are
 *                      read; positions start_pos .. start_pos+seqlen-1 are
 *                      written. Zero it for a new sequence.
 *   ids_dev          : int32 [seqlen] token ids at positions start_pos.. .
 *   out_dev          : int64 [n_layers][seqlen][cols], cols = (max_ngram-1) *
 *                      n_heads: layer l's ids are one contiguous [seqlen, cols]
 *                      array (token-major, as layer_row_ids orders them), ready
 *                      for q2k_dequant_rows.
 * Row id (s, l, (i-1)*n_heads + h) for position p = start_pos + s: window
 * tokens tok[j] = compressed id of position p - j (position 0 when p < j),
 * pad_id from the first j with p < j or an unmapped id on; rolling =
 * tok[0]*mult[l][0], then rolling ^= tok[i]*mult[l][i] (64-bit wrapping);
 * id = (rolling mod primes[l][i-1][h], in [0, prime)) + offsets[l][col].
 * A token id outside [0, vocab) (the pages refuse the call) or a prime <= 0
 * writes -1 for every row id whose window reads it and stores 1 into the
 * nullable *err_flag_dev. Q2K_ESHAPE: vocab < 1, n_layers outside 1..64,
 * max_ngram outside 2..8, n_heads outside 1..64, seqlen < 1, positions past
 * cache_len; Q2K_EINVAL: null pointers, out or cache overlapping an input;
 * Q2K_EALIGN: 64-bit arrays not 8-byte aligned, ids not 4-byte aligned. */
Q2K_API int32_t engram_hash(const int64_t* token_map_dev, int64_t vocab,
                         const int64_t* multipliers_dev, const int64_t* primes_dev,
                         const int64_t* offsets_dev, int32_t n_layers, int32_t max_ngram,
                         int32_t n_heads, int64_t pad_id, int64_t* cache_dev, int64_t cache_len,
                         const int32_t* ids_dev, int32_t seqlen, int64_t start_pos,
                         int64_t* out_dev, int32_t* err_flag_dev, void* stream);

/* One decode token through the engram row path in one launch: engram_hash
 * for this token (position pos, ids = token_dev[0]) restricted to hashed
 * layer `layer`, then q2k_dequant_rows_q8_1 of that layer's row ids
 * (engram_v41.rs EngramHasher::hash / layer_row_ids, then
 * EngramV41::rows_from_q2k and the projection's q8_1 input). The same ids,
 * cache update (cache[pos] = the token's compressed id), rows, q8_1 bytes
 * and error flag as those two calls.
 *   token_map_dev .. cache_len : as in engram_hash.
 *   token_dev : int32 [1], the token at position pos (0 <= pos < cache_len).
 *   layer : the hashed layer whose row ids are gathered, 0..n_layers-1.
 *   table_dev, n_table_rows : as in q2k_dequant_rows_q8_1.
 *   ids_out_dev : nullable int64 [cols] (cols = (max_ngram-1)*n_heads <= 32).
 *   rows_out_dev : nullable bf16 [cols, 256], 16-byte aligned.
 *   xq_dev, xq_bytes : output, q8_1_rows_bytes(1, 256*cols), 16-byte aligned.
 * Errors: those of the two calls; cols > 32 is Q2K_ESHAPE; the outputs may
 * not overlap each other, the cache or an input. */
Q2K_API int32_t engram_rows_q8_1(const int64_t* token_map_dev, int64_t vocab,
                                 const int64_t* multipliers_dev, const int64_t* primes_dev,
                                 const int64_t* offsets_dev, int32_t n_layers, int32_t max_ngram,
                                 int32_t n_heads, int64_t pad_id, int64_t* cache_dev,
                                 int64_t cache_len, const int32_t* token_dev, int64_t pos,
                                 int32_t layer, const void* table_dev, int64_t n_table_rows,
                                 int64_t* ids_out_dev, void* rows_out_dev, void* xq_dev,
                                 size_t xq_bytes, int32_t* err_flag_dev, void* stream);

/* One decode token through the whole engram layer step (engram_v41.rs module
 * doc steps 1-4; engram_v41/apply.rs, EngramV41::apply with one token and
 * the Q2_K projection): the token's row ids of hashed layer `layer`
 * (engram_hash), the gather, dequantisation and q8_1 of those rows viewed as
 * one row (q2k_dequant_rows_q8_1), the wkv projection of that row (q2k_mmvq,
 * m = 1) into kv, and the gate on h (engram_gate). The same bits in h, the
 * cache and the error flag as engram_rows_q8_1 + q2k_mmvq + engram_gate.
 * When the projection takes the run kernel (at least 2048 row steps) the
 * first three stages are one launch: every workgroup of the product forms
 * the q8_1 row in its prologue while its first weight loads are in flight;
 * then the gate launch.
 *   token_map_dev .. layer : as in engram_rows_q8_1 (cols = (max_ngram-1) *
 *                  n_heads <= 32 row ids, so the projection's input width is
 *                  k = 256 * cols).
 *   table_dev, n_table_rows : as in q2k_dequant_rows.
 *   wkv_dev      : Q2_K [(hc+1)*dim, 256*cols].
 *   qk_dev, h_dev, hc, dim, eps : as in engram_gate with t = 1 (h updated in
 *                  place).
 *   workspace_dev, workspace_bytes : device memory the step may overwrite
 *                  (the pages keep kv in a workspace of EngramV41: its kv
 *                  buffer): kv f32 [(hc+1)*dim] then the q8_1 row, at least
 *                  engram_step_workspace_bytes(max_ngram, n_heads, hc, dim)
 *                  bytes, 256-byte aligned; its contents after the call are
 *                  kv (rounded up to 256 bytes) and the q8_1 row.
 *   err_flag_dev : nullable, as in engram_rows_q8_1.
 * Errors: Q2K_EINVAL (null pointers; h, the cache or the workspace
 * overlapping each other or an input), Q2K_ESHAPE (as the calls it
 * replaces), Q2K_ESPACE (workspace too small), Q2K_EALIGN. */
Q2K_API size_t engram_step_workspace_bytes(int32_t max_ngram, int32_t n_heads, int32_t hc,
                                           int32_t dim);
Q2K_API int32_t engram_step(const int64_t* token_map_dev, int64_t vocab,
                            const int64_t* multipliers_dev, const int64_t* primes_dev,
                            const int64_t* offsets_dev, int32_t n_layers, int32_t max_ngram,
                            int32_t n_heads, int64_t pad_id, int64_t* cache_dev, int64_t cache_len,
                            const int32_t* token_dev, int64_t pos, int32_t layer,
                            const void* table_dev, int64_t n_table_rows, const void* wkv_dev,
                            const float* qk_dev, float* h_dev, int32_t hc, int32_t dim, float eps,
                            void* workspace_dev, size_t workspace_bytes, int32_t* err_flag_dev,
                            void* stream);

/* engram_step without the workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same launches and the same bits as
 * engram_step, with kv and the q8_1 row kept in a device array of the
 * library (Q2K_ENGRAM_SCRATCH_BYTES, one per GPU, held until the process
 * ends; its address is looked up once per device). Calls no allocator.
 * Limit: engram_step_workspace_bytes(max_ngram, n_heads, hc, dim) <=
 * Q2K_ENGRAM_SCRATCH_BYTES (hc + 1 = 5 streams of dim 8192 with 32 row
 * ids fit), else Q2K_ESPACE before any launch. Every call on one GPU uses
 * the same array and overwrites what it reads (kv and the q8_1 row are
 * written whole before they are read), so nothing needs clearing between
 * calls; calls that overlap on one GPU (other streams, other threads) race.
 * Arguments and other errors as engram_step; Q2K_EDEVICE when the array's
 * device address cannot be looked up. */
#define Q2K_ENGRAM_SCRATCH_BYTES (176 * 1024)
Q2K_API int32_t engram_step_noalloc(const int64_t* token_map_dev, int64_t vocab,
                                    const int64_t* multipliers_dev, const int64_t* primes_dev,
                                    const int64_t* offsets_dev, int32_t n_layers,
                                    int32_t max_ngram, int32_t n_heads, int64_t pad_id,
                                    int64_t* cache_dev, int64_t cache_len,
                                    const int32_t* token_dev, int64_t pos, int32_t layer,
                                    const void* table_dev, int64_t n_table_rows,
                                    const void* wkv_dev, const float* qk_dev, float* h_dev,
                                    int32_t hc, int32_t dim, float eps, int32_t* err_flag_dev,
                                    void* stream);

/* Which kernel runs the Q2_K x q8_1 products (q2k_mmvq, its pair, expert
 * and grouped forms, q2k_mmq up to 16 tokens and q2k_block_dots),
 * process-wide. Every kernel forms the same exact int32 block sums and
 * follows the fixed summation order stated at q2k_mmvq, so every choice
 * returns the same bits: the choice changes speed only. (q2k_mmq from 17
 * tokens always runs its tile kernel and order.)
 *   Q2K_KERNEL_AUTO (the default): a cost model measured on MI355X picks
 *     the matrix-core kernel (2..8 tokens; rows of 4, 8, 16 or 28
 *     super-blocks) or the packed-dot kernels (tokens split over waves);
 *   Q2K_KERNEL_MATRIX_CORES: the matrix-core kernel wherever it applies;
 *   Q2K_KERNEL_PACKED_DOTS: never the matrix-core kernel (9..16 tokens
 *     then run as groups of 8 on the packed-dot kernels).
 * Returns the previous choice, or Q2K_EINVAL for an unknown one. Launches
 * already enqueued are unaffected; a thread that launches while another
 * changes the choice gets either kernel (the same bits). */
#define Q2K_KERNEL_AUTO 0
#define Q2K_KERNEL_MATRIX_CORES 1
#define Q2K_KERNEL_PACKED_DOTS 2
Q2K_API int32_t q2k_set_product_kernel(int32_t choice);

/* The kernel a single-matrix q2k_mmvq, q2k_block_dots or q2k_mmq of this
 * shape runs under the current choice: Q2K_KERNEL_MATRIX_CORES or
 * Q2K_KERNEL_PACKED_DOTS (always the matrix cores from 17 tokens, where the
 * choice does not apply); Q2K_ESHAPE for n < 1, k not a positive multiple
 * of 256 or m outside 1..Q2K_MMQ_MAX_M. Host only, no device call. */
Q2K_API int32_t q2k_product_kernel(int32_t n, int32_t k, int32_t m);

/* Integer stage of the product of m tokens (q2k_mmvq, and q2k_mmq past 8
 * tokens), exported for exact checking: out_dev int32 [m, n, k/32, 2]
 * receives, per token t, row r and q8 block c, I = sum sc*q*xq and
 * M = sum m*xq over the block's 32 values, as formed by the kernel the
 * product takes for this shape (q2k_product_kernel): the matrix-core
 * kernels' own v_mfma_i32_16x16x64_i8 (up to 16 tokens) or
 * v_mfma_i32_16x16x32_i8 (from 17) outputs, or the packed-dot kernels'
 * v_dot4 sums (the device function every packed-dot product kernel uses).
 * 1 <= m <= Q2K_MMQ_MAX_M, m * n * k/32 * 2 <= 2^31; out may not overlap
 * w or xq; other arguments and errors as in q2k_mmvq. */
Q2K_API int32_t q2k_block_dots(const void* w_dev, const void* xq_dev, int32_t* out_dev,
                       int32_t n, int32_t k, int32_t m, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* Q2K_DECODE_H */
