/*
 * bpg.h -- C ABI of the MI355X (gfx950) Hadamard-rotated W4A4 prompt GEMM.
 *
 * The method ("509 tokens a second of prompt: the Hadamard route ships",
 * sections "Why prompts are a matrix-unit problem" and "The rotation"; and
 * "Qwen3.8-27B at 45.7 tok/s: DFlash2 in 1bit serve, and 4-bit activations
 * with a Hadamard rotation", section "Prompt processing: 4-bit activations,
 * rotated first"):
 *   - every 32-value block of the activations is rotated by a 32-point
 *     Walsh-Hadamard transform and rounded to 4-bit codes sharing one scale;
 *   - the weights are Q4_0 (4-bit code u meaning u-8, one fp16 scale per 32)
 *     that were rotated the same way once, offline, so x.w = (Hx).(Hw);
 *   - the product runs on integer matrix instructions; the kernel reads the
 *     Q4_0 nibbles bit for bit, flipping each code's top bit to get u-8 in
 *     two's complement.
 * The MoE variant ("Where the engine is going: HRX and the NPU", section
 * "4-bit activations reach the MoE experts") runs the same route over the
 * expert matmuls.  The 8-bit activation route is the pages' "exact 8-bit"
 * comparison path.
 *
 * Numerics fixed by this library (the pages are silent on them):
 *   - rotation: Sylvester-order H32, butterfly stages h = 1,2,4,8,16 in fp32
 *     (lower index a+b, upper a-b), then times fp32(1/sqrt(32)); no FMA;
 *   - scale d = amax/7 (8-bit: amax/127), IEEE fp32 division; code
 *     q = clamp(rint(v/d), -8, 7) (8-bit: +-127), ties to even; a block with
 *     d = 0 (all zero, or amax/7 underflowing to 0) has codes 0;
 *   - block dot products are exact int32; the output is
 *     y[m][n] = sum_b da[m][b] * dw[n][b] * S[m][n][b], accumulated in fp32
 *     in a fixed order per shape (bit-identical from run to run).
 *
 * Conventions for every call:
 *   - returns bpg_status; BPG_OK on success.  No call allocates device memory,
 *     keeps a pointer after returning, or logs;
 *   - all argument and stamp checks run on the host, before any HIP call, so
 *     every error except BPG_ERR_DEVICE / BPG_ERR_LAUNCH is reported without
 *     touching a GPU;
 *   - device calls are asynchronous on `stream` (a hipStream_t; NULL = the
 *     null stream); execution faults surface at the caller's synchronisation;
 *   - the caller owns every buffer; device pointers must be 16-byte aligned;
 *     when the row count is 0, activation, code, scale and output pointers
 *     may be NULL (nothing is read or written);
 *   - K (input channels) is a multiple of 32, N (output channels) a multiple
 *     of 32; M (tokens) may be 0 (the call is then a no-op after its checks);
 *   - inputs are finite and below 2^120 in magnitude (every sum of the
 *     rotation, up to 128 values, then stays finite); NaN or Inf input, or a
 *     rotation that overflows, gives unspecified codes.
 */
#ifndef BPG_H
#define BPG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BPG_OK = 0,
    BPG_ERR_NULL = 1,   /* a required pointer is NULL */
    BPG_ERR_SHAPE = 2,  /* a size is negative, K or N not a multiple of 32, ld too small, ... */
    BPG_ERR_ALIGN = 3,  /* a device pointer or leading dimension breaks the alignment rule */
    BPG_ERR_DTYPE = 4,  /* unknown dtype or source kind, or act_bits not 4 or 8 */
    BPG_ERR_STAMP = 5,  /* weight descriptor not made by this library's packers, wrong
                           version or layout, an image of the other route (rotated
                           vs unrotated), or sizes that disagree */
    BPG_ERR_BUFFER = 6, /* destination buffer too small */
    BPG_ERR_DEVICE = 7, /* the current device is not a gfx950 GPU */
    BPG_ERR_LAUNCH = 8  /* the kernel launch failed (hipGetLastError after enqueue) */
} bpg_status;

/* Source of rotate_pack_weights and pack_weights_unrotated. */
typedef enum {
    BPG_SRC_F32 = 0,           /* unrotated float weights [E][N][K], fp32 */
    BPG_SRC_BF16 = 1,          /* unrotated float weights [E][N][K], bf16 bits */
    BPG_SRC_Q4_0_ROTATED = 2,  /* Q4_0 blocks [E][N][K/32] x 18 B of weights already
                                  rotated by H32 (a rotated file's tensors);
                                  rotate_pack_weights only */
    BPG_SRC_Q4_0 = 3           /* plain (unrotated) Q4_0 blocks, same layout;
                                  pack_weights_unrotated only */
} bpg_src_kind;

/* Activation dtype of quantize_act_h32. */
typedef enum { BPG_X_F32 = 0, BPG_X_BF16 = 1 } bpg_x_dtype;

#define BPG_WEIGHTS_MAGIC 0x57475042u /* "BPGW" little-endian */
#define BPG_WEIGHTS_VERSION 1u
#define BPG_LAYOUT_GROUP4 3u

/*
 * Stamp of a packed weight image (the analogue of the rotated file's stamp:
 * a GEMM refuses an image whose stamp is missing or does not say rotated).
 *
 * Device image, layout BPG_LAYOUT_GROUP4, for E experts (1 if dense),
 * B = K/32 blocks per row, G = ceil(B/4) groups of four blocks and T = N/32
 * column tiles of 32 columns: one 2304-byte block per (expert, tile, group),
 * in that order ([E][T][G]), holding
 *   bytes 0..2047:     uint32 [4 slots s][32 columns c][4 blocks q]: dword s
 *                      (bytes 4s..4s+3) of the 16 Q4_0 nibble bytes of column
 *                      32t+c, block 4G+q (byte j: element j in the low nibble,
 *                      element j+16 in the high nibble; code u means u-8);
 *   bytes 2048..2303:  fp16 [16][2][4 blocks q]: the block scale of column
 *                      c = 16h + c16 at [c16][h][q].
 * Blocks past B (when B is not a multiple of 4) hold codes 0x88 (value 0)
 * and scale 0.  One 16-byte read at (s, c) holds slot s of column c for four
 * consecutive blocks; one at scale row c16 holds the four scales of columns
 * c16 and 16 + c16.  Total bytes = E*T*G*2304 (= E*N*K*18/32, as for Q4_0,
 * when K is a multiple of 128).  scales_offset is 2048: the offset of a
 * group's scales inside its block.
 */
typedef struct {
    uint32_t magic;        /* BPG_WEIGHTS_MAGIC */
    uint32_t version;      /* BPG_WEIGHTS_VERSION */
    uint32_t rotation;     /* 32: every block rotated by H32 (rotate_pack_weights);
                              0: unrotated (pack_weights_unrotated);
                              64, 128: spans rotated by H64, H128
                              (rotate_pack_weights_rot) */
    uint32_t layout;       /* BPG_LAYOUT_GROUP4 */
    int64_t n;             /* output channels per expert */
    int64_t k;             /* input channels */
    int64_t num_experts;   /* 1 for a dense weight */
    uint64_t bytes;        /* size of the image */
    uint64_t scales_offset;/* 2048: offset of a group's scales in its block */
} bpg_weights_desc;

/* Human-readable name of a status (static string). */
const char *bpg_status_str(bpg_status s);

/* Size in bytes of the packed image for the given shape; 0 if the shape is invalid. */
size_t rotate_pack_weights_bytes(int64_t n, int64_t k, int64_t num_experts);

/*
 * Offline weight preparation, on the CPU, synchronous
 * ("509 tokens a second of prompt: the Hadamard route ships", section
 * "Making the file is part of the engine": the tool rotates the projections,
 * quantizes to Q4_0 and stamps the file).
 *
 *   src       host pointer; layout given by `kind` (see bpg_src_kind)
 *   n, k      per-expert output and input channels (both multiples of 32)
 *   num_experts  >= 1
 *   dst_host  host buffer of at least rotate_pack_weights_bytes(n, k, E) bytes;
 *             receives the device image, to be copied to the GPU as-is
 *   desc_out  receives the stamp
 *
 * Float sources are rotated per 32-block in fp64 (same butterfly order, times
 * fp64 1/sqrt(32)) and quantized to Q4_0: dw = fp16(amax/7), u = clamp(
 * rint(w'/dw), -8, 7) + 8 with the fp16-rounded dw.  Q4_0 sources are only
 * re-laid out; plain BPG_SRC_Q4_0 is refused (DTYPE).  Errors: NULL, SHAPE,
 * DTYPE, BUFFER.
 */
bpg_status rotate_pack_weights(const void *src, bpg_src_kind kind, int64_t n, int64_t k,
                               int64_t num_experts, void *dst_host, size_t dst_bytes,
                               bpg_weights_desc *desc_out);

/*
 * FWHT-32 fused into per-block activation quantization, on the GPU
 * ("509 tokens a second of prompt: the Hadamard route ships", section
 * "The rotation": the rotation runs inside the step that quantizes
 * activations; blocks of 32 values share one scale).
 *
 *   x        device, [m][ldx] elements of `dt` (fp32, or bf16 bits); ldx >= k,
 *            ldx % 4 == 0
 *   act_bits 4: codes [m][k/2] bytes, each block's 16 bytes holding element j
 *            in the low nibble and element j+16 in the high nibble of byte j
 *            (4-bit two's complement, the Q4_0 pairing);
 *            8: codes [m][k] int8 in natural element order
 *   scales   device, [m][k/32] fp32
 * Errors: NULL, SHAPE, ALIGN, DTYPE, DEVICE, LAUNCH.
 */
bpg_status quantize_act_h32(const void *x, bpg_x_dtype dt, int64_t m, int64_t k, int64_t ldx,
                            int act_bits, void *codes, float *scales, void *stream);

/*
 * The unrotated W4A4 route ("Qwen3.8-27B at 45.7 tok/s: DFlash2 in 1bit serve,
 * and 4-bit activations with a Hadamard rotation", section "Prompt processing:
 * 4-bit activations, rotated first": plain Q4_0 weights read bit for bit and
 * activations rounded to 4 bits with no rotation; faster to set up, larger
 * error).  The same kernels run on an image and codes made without H32.
 *
 * pack_weights_unrotated: as rotate_pack_weights, but float sources are
 * quantized to Q4_0 without rotation and BPG_SRC_Q4_0 blocks are only
 * re-laid out; the stamp says rotation 0.  BPG_SRC_Q4_0_ROTATED is refused
 * (DTYPE).  Errors: NULL, SHAPE, DTYPE, BUFFER.
 *
 * quantize_act_unrotated: as quantize_act_h32 with the rotation left out
 * (amax, scale and codes of the raw 32-value blocks, same code layouts).
 * Errors: NULL, SHAPE, ALIGN, DTYPE, DEVICE, LAUNCH.
 *
 * w4a4_gemm_unrotated: as w4a4_gemm, for codes from quantize_act_unrotated
 * and an image stamped rotation 0 (a rotated image gives STAMP, and
 * w4a4_gemm refuses an unrotated one the same way).
 * Errors: NULL, SHAPE, ALIGN, DTYPE, STAMP, DEVICE, LAUNCH.
 */
bpg_status pack_weights_unrotated(const void *src, bpg_src_kind kind, int64_t n, int64_t k,
                                  int64_t num_experts, void *dst_host, size_t dst_bytes,
                                  bpg_weights_desc *desc_out);
bpg_status quantize_act_unrotated(const void *x, bpg_x_dtype dt, int64_t m, int64_t k,
                                  int64_t ldx, int act_bits, void *codes, float *scales,
                                  void *stream);
bpg_status w4a4_gemm_unrotated(const void *codes, const float *scales, int act_bits, int64_t m,
                               const bpg_weights_desc *w, const void *w_dev, float *y,
                               int64_t ldy, void *stream);

/*
 * Rotations longer than 32 ("Qwen3.8-27B at 45.7 tok/s: DFlash2 in 1bit
 * serve, and 4-bit activations with a Hadamard rotation", section "What's
 * next": rotations larger than 32, which spread outliers further).  The span
 * of the rotation is `rotation` = 32, 64 or 128 values (Sylvester order,
 * butterflies h = 1 .. rotation/2 in the 32-point route's order and sign
 * convention, then times 1/sqrt(rotation): fp32(1/sqrt 32), 1/8 or half of
 * fp32(1/sqrt 32) on the GPU, the fp64 value offline); the 32-value scale
 * blocks, the codes and the image layout are unchanged.  K must be a multiple
 * of the span.  With rotation = 32 these are exactly rotate_pack_weights,
 * quantize_act_h32 and w4a4_gemm.
 *
 * rotate_pack_weights_rot: float sources are rotated per span in fp64 and
 * quantized to Q4_0; BPG_SRC_Q4_0_ROTATED blocks (rotated with this span) are
 * only re-laid out; the stamp records the span.  Errors: NULL, SHAPE (also
 * for a span other than 32, 64, 128), DTYPE, BUFFER.
 * quantize_act_rot: as quantize_act_h32 with the given span.
 * Errors: NULL, SHAPE, ALIGN, DTYPE, DEVICE, LAUNCH.
 * w4a4_gemm_rot: as w4a4_gemm for codes made with the given span; the image's
 * stamp must record the same span (else STAMP).
 * Errors: NULL, SHAPE, ALIGN, DTYPE, STAMP, DEVICE, LAUNCH.
 */
bpg_status rotate_pack_weights_rot(const void *src, bpg_src_kind kind, int64_t n, int64_t k,
                                   int64_t num_experts, int rotation, void *dst_host,
                                   size_t dst_bytes, bpg_weights_desc *desc_out);
bpg_status quantize_act_rot(const void *x, bpg_x_dtype dt, int64_t m, int64_t k, int64_t ldx,
                            int act_bits, int rotation, void *codes, float *scales, void *stream);
bpg_status w4a4_gemm_rot(const void *codes, const float *scales, int act_bits, int rotation,
                         int64_t m, const bpg_weights_desc *w, const void *w_dev, float *y,
                         int64_t ldy, void *stream);

/*
 * Dense W4A4 (or W4A8) product y = x . W^T from codes, on the GPU
 * ("509 tokens a second of prompt: the Hadamard route ships", section
 * "Why prompts are a matrix-unit problem").
 *
 *   codes, scales  device, as written by quantize_act_h32 for m rows and k = w->k
 *   act_bits       4 or 8, as given to quantize_act_h32
 *   w, w_dev       stamp (host) and device copy of the image; w->num_experts == 1
 *   y              device, [m][ldy] fp32, ldy >= w->n, ldy % 4 == 0; overwritten
 * Errors: NULL, SHAPE, ALIGN, DTYPE, STAMP, DEVICE, LAUNCH.
 */
bpg_status w4a4_gemm(const void *codes, const float *scales, int act_bits, int64_t m,
                     const bpg_weights_desc *w, const void *w_dev, float *y, int64_t ldy,
                     void *stream);

/*
 * Grouped (MoE) product over ragged expert row ranges, on the GPU
 * ("Where the engine is going: HRX and the NPU", section "4-bit activations
 * reach the MoE experts").  Rows of `codes` are sorted by expert: expert e
 * owns rows [offsets[e], offsets[e+1]) and multiplies them by its weights.
 *
 *   total_rows          rows of codes/scales/y
 *   expert_offsets_dev  device, int32 [E+1], non-decreasing, offsets[0] >= 0,
 *                       offsets[E] <= total_rows, E = w->num_experts.  Not
 *                       read on the host (no synchronisation).  Values that
 *                       break the rule give unspecified rows of y, but every
 *                       access stays inside [0, total_rows).
 *   y                   device, [total_rows][ldy] fp32; rows outside every
 *                       expert's range are left untouched
 * Errors: NULL, SHAPE, ALIGN, DTYPE, STAMP, DEVICE, LAUNCH.
 */
bpg_status w4a4_grouped_gemm(const void *codes, const float *scales, int act_bits,
                             int64_t total_rows, const int32_t *expert_offsets_dev,
                             const bpg_weights_desc *w, const void *w_dev, float *y,
                             int64_t ldy, void *stream);

/*
 * bf16 output.  The pages accumulate the product in fp32 and say nothing of
 * the type the result is stored in ("509 tokens a second of prompt: the
 * Hadamard route ships", section "Why prompts are a matrix-unit problem");
 * these variants compute exactly as w4a4_gemm / w4a4_grouped_gemm and round
 * each fp32 result to bf16 (round to nearest even) at the store, halving the
 * output bytes.  Every element equals bf16_rne of the fp32 variant's result.
 *
 *   y    device, [m or total_rows][ldy] bf16 (uint16 bit patterns),
 *        ldy >= w->n, ldy % 8 == 0 (16-byte aligned rows); overwritten
 *        (grouped: rows outside every expert's range untouched)
 * Other arguments, limits and errors as w4a4_gemm / w4a4_grouped_gemm.
 */
bpg_status w4a4_gemm_bf16(const void *codes, const float *scales, int act_bits, int64_t m,
                          const bpg_weights_desc *w, const void *w_dev, uint16_t *y,
                          int64_t ldy, void *stream);
bpg_status w4a4_grouped_gemm_bf16(const void *codes, const float *scales, int act_bits,
                                  int64_t total_rows, const int32_t *expert_offsets_dev,
                                  const bpg_weights_desc *w, const void *w_dev, uint16_t *y,
                                  int64_t ldy, void *stream);

/*
 * The expert layer around the grouped product ("Where the engine is going: HRX
 * and the NPU", section "4-bit activations reach the MoE experts": the route
 * covers the expert matmuls; the pages give no detail of the layer around
 * them, so the steps below are this library's reading).  A layer of T tokens,
 * each routed to topk experts (entry t*topk + j), runs as
 *   moe_route_sort -> quantize_act_h32 (T token rows, once)
 *   -> w4a4_grouped_gemm_gather (gate and up projections, rows gathered by
 *      token) -> swiglu_quantize_h32 -> w4a4_grouped_gemm (down projection)
 *   -> moe_combine.
 *
 * moe_route_sort: sorts the entries by expert, stably (entry order inside an
 * expert), on the GPU (one workgroup per expert, each reading every entry).
 *   expert_of_dev   device, int32 [tokens*topk]; ids outside [0, experts) are
 *                   clamped (unspecified grouping, in-bounds accesses)
 *   offsets_dev     device, int32 [experts+1]: expert e owns sorted rows
 *                   [offsets[e], offsets[e+1])
 *   row_token_dev   device, int32 [tokens*topk]: the token of each sorted row
 *   slot_of_dev     device, int32 [tokens*topk]: the sorted row of each entry
 * Limits: experts <= 512, tokens*topk <= 2^20.  Pointers 4-byte aligned.
 * Errors: NULL, SHAPE, ALIGN, DEVICE, LAUNCH.
 */
bpg_status moe_route_sort(const int32_t *expert_of_dev, int64_t tokens, int64_t topk,
                          int64_t experts, int32_t *offsets_dev, int32_t *row_token_dev,
                          int32_t *slot_of_dev, void *stream);

/*
 * w4a4_grouped_gemm_gather: as w4a4_grouped_gemm, but sorted row r reads
 * activation row row_ids_dev[r] (clamped to [0, src_rows)) of codes and
 * scales, which hold src_rows rows (e.g. the tokens, quantized once); y has
 * total_rows rows in sorted order.  src_rows * (bytes per code row) < 2^31.
 * row_ids_dev is device int32 [total_rows], 4-byte aligned.
 * Errors: NULL, SHAPE, ALIGN, DTYPE, STAMP, DEVICE, LAUNCH.
 */
bpg_status w4a4_grouped_gemm_gather(const void *codes, const float *scales, int act_bits,
                                    int64_t src_rows, const int32_t *row_ids_dev,
                                    int64_t total_rows, const int32_t *expert_offsets_dev,
                                    const bpg_weights_desc *w, const void *w_dev, float *y,
                                    int64_t ldy, void *stream);

/*
 * swiglu_quantize_h32: the down projection's input.  gu is device fp32
 * [rows][ldgu] with the gate projection in columns [0, inter) and the up
 * projection in [inter, 2*inter) (ldgu >= 2*inter, ldgu % 4 == 0).
 * h = silu(gate) * up in fp32, with silu(g) = g / (1 + e^-g) (IEEE division)
 * and e^x computed in fp32 as: x clamped to [-87, 88]; n = rint(x * fp32(log2 e));
 * r = (x - n * 0.693145751953125) - n * fp32(ln 2 - 0.693145751953125);
 * p = Horner form of the degree-6 Taylor polynomial of e^r with coefficients
 * fp32(1/720), fp32(1/120), fp32(1/24), fp32(1/6), 0.5, 1, 1; e^x = p * 2^n;
 * every step one fp32 operation, no FMA.  Then h is rotated and quantized
 * exactly as quantize_act_h32 does (codes [rows][inter/2] or [rows][inter],
 * scales [rows][inter/32]).
 * Errors: NULL, SHAPE, ALIGN, DTYPE, DEVICE, LAUNCH.
 */
bpg_status swiglu_quantize_h32(const float *gu, int64_t rows, int64_t inter, int64_t ldgu,
                               int act_bits, void *codes, float *scales, void *stream);

/*
 * moe_combine: y[t][c] = sum over j = 0..topk-1, in that order, of
 * weights[t*topk + j] * dn[slot_of[t*topk + j]][c]; the accumulator starts at
 * 0 and every step is one fp32 fma.  dn is device fp32 [rows][lddn] (sorted
 * rows; slot values are clamped to [0, rows)); y is device fp32
 * [tokens][ldy], overwritten.  hidden % 4 == 0, lddn and ldy >= hidden and
 * multiples of 4; dn and y 16-byte aligned, slot_of and weights 4-byte.
 * Errors: NULL, SHAPE, ALIGN, DEVICE, LAUNCH.
 */
bpg_status moe_combine(const float *dn, int64_t lddn, int64_t rows, const int32_t *slot_of_dev,
                       const float *weights_dev, int64_t tokens, int64_t topk, int64_t hidden,
                       float *y, int64_t ldy, void *stream);

/*
 * Parity and debug: the exact int32 block dot products
 * S[m][n][b] = sum_i q_a[m][32b+i] * (u[n][32b+i] - 8) ("509 tokens a second
 * of prompt: the Hadamard route ships", section "Why prompts are a
 * matrix-unit problem": the product is integer matrix work over Q4_0 codes),
 * for rows [m0, m1) and columns [n0, n1) of expert `expert` (0 for a dense
 * image).  This call always runs one kernel: the tiled kernel's 32 x 32
 * matrix-instruction main loop (one v_mfma_i32_32x32x32_i8 per tile and
 * block, the operand widening shared with every product kernel), writing S
 * instead of applying the scales.  The kernels w4a4_gemm and
 * w4a4_grouped_gemm route to (see w4a4_gemm_kernel_name) do not write S;
 * their block sums are shown exact through their outputs: with power-of-two
 * scales every step of the fp32 epilogue is exact, and with the activation
 * scales of all blocks but one set to 0 the output is dw * S of that block.
 *
 *   scales  not read (may be NULL)
 *   sums    device, int32 [(m1-m0)][(n1-n0)][k/32]
 *   expert  in [0, w->num_experts)
 * Errors: NULL, SHAPE, ALIGN, DTYPE, STAMP, DEVICE, LAUNCH.
 */
bpg_status w4a4_gemm_blocksums(const void *codes, const float *scales, int act_bits, int64_t m,
                               const bpg_weights_desc *w, const void *w_dev, int64_t expert,
                               int64_t m0, int64_t m1, int64_t n0, int64_t n1, int32_t *sums,
                               void *stream);

/*
 * Routing queries, host only (no GPU call): the name of the kernel that
 * w4a4_gemm (and its _bf16, _unrotated and _rot forms) with these arguments
 * launches, and the same for w4a4_grouped_gemm (src_rows = 0) or
 * w4a4_grouped_gemm_gather (src_rows = the activation rows it reads).  The
 * kernel is chosen from the shape and the code width alone, so the answer is
 * what the product call runs: "weight-stream", "wide 64x160",
 * "strip 32x128", "tiled BMxBN", "expert-slot" or "grouped 32xBN"; "none"
 * when there are no rows.  NULL for an invalid stamp or act_bits (static
 * strings; the caller frees nothing).
 */
const char *w4a4_gemm_kernel_name(int act_bits, int64_t m, const bpg_weights_desc *w);
const char *w4a4_grouped_gemm_kernel_name(int act_bits, int64_t total_rows, int64_t src_rows,
                                          const bpg_weights_desc *w);

#ifdef __cplusplus
}
#endif

#endif /* BPG_H */
