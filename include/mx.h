/*
 * mx.h -- C ABI of libmx: block-scaled 4-bit floating-point quantization
 * (MXFP4, NVFP4; also the wider MX elements MXFP8 and MXFP6) and the matrix
 * products that consume it, for AMD gfx950.
 *
 * Formats (sources are the web pages this library implements):
 *   E2M1 element: 1 sign, 2 exponent (bias 1), 1 mantissa bit; states
 *     {0, 0.5, 1, 1.5, 2, 3, 4, 6} and their negatives, zero signed
 *     ("NVFP4 Architecture: Microscaling & 4-Bit LLMs on Blackwell", section
 *     "1. The E2M1 Floating-Point Format", table "The Complete Discrete State
 *     Mapping of E2M1").
 *   MXFP4: 32-element blocks, one E8M0 scale byte per block, S = 2^(E-127)
 *     ("How Microscaling FP4 (MXFP4) Halves Memory Bandwidth", section "The
 *     Microscaling Breakthrough: 32-Element Blocks"; "NVFP4 Architecture",
 *     section "2. Micro-Block Exponent Scaling: E8M0 Format").
 *   NVFP4: 16-element blocks ("NVIDIA NVFP4 quantization", section "The Physics
 *     of NVFP4"), one FP8 E4M3 scale byte per block and one fp32 scale per
 *     tensor (dual-level scaling, "NVFP4 Architecture", section "1. The
 *     Dual-Level Mathematical Formulation").
 *   MXFP8 / MXFP6: the same 32-element blocks and E8M0 scales with 8-bit
 *     (E4M3 bias 7, largest 448; E5M2 bias 15, largest 57344) or 6-bit (E2M3
 *     bias 1, largest 7.5; E3M2 bias 3, largest 28) elements (the MX family
 *     of the "MXFP4" card, section "Core Facts": MXFP8/MXFP4 scaled GEMM; the
 *     exponent/mantissa trade-off of "How Microscaling FP4 (MXFP4)...",
 *     section "The Representation Dilemma").
 *
 *   Emulation variants ("NVFP4 Architecture", section "1. The Dual-Level
 *     Mathematical Formulation", equation S_block with S_global, and section
 *     "End-to-End Implementation", whose emulation uses 16-element blocks
 *     with power-of-two scales and zero-pads to whole blocks):
 *     MX_FMT_MXFP4_K16 = E2M1 in 16-element blocks with E8M0 scales and an
 *     optional fp32 tensor scale g (global_scale; NULL = 1):
 *     S_block = 2^ceil(log2(m / (6 g))); MX_FMT_FP4_TENSOR = the naive
 *     baseline (section "The Problem", figure "The Outlier Distortion in
 *     Coarse-Grained FP4"): one fp32 scale s = fp32(max(max|x|, 1e-8) / 6)
 *     for the whole tensor in global_scale, no block scales.
 *
 * Memory layout of a quantized [rows, cols] tensor (blocks run along cols):
 *   codes  uint8 [rows, cols*b/8] for b-bit elements (b = 4, 6 or 8), rows
 *          packed back to back; element i of a row occupies bits
 *          [b*i, b*i + b) of the row read as one little-endian bit string
 *          (4-bit: element 2j in the low nibble of byte j, 2j+1 in the high
 *          nibble; 8-bit: one byte per element).
 *   scales uint8 [rows, cols/k], row pitch cols/k bytes (k = 32 or 16).
 *   E8M0-scaled formats (MXFP4, MXFP8, MXFP6, MXFP4_K16) accept any cols:
 *   each row is stored zero-padded to P = ceil(cols/k)*k elements (codes
 *   [rows, P*b/8], scales [rows, P/k]); the padding quantizes to +0.
 *   MX_FMT_FP4_TENSOR: codes [rows, cols/2] (cols even), scales unused (may
 *   be NULL), global_scale fp32[1].
 *   global_scale  fp32[1] (NVFP4 only).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or keeps them.  Scalars are passed by value.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *     default stream).  Results are visible after the caller synchronizes.
 *   - Arguments are validated on the host before any HIP call; an invalid call
 *     returns a negative mx_status and enqueues nothing.  A failed launch
 *     returns MX_ERR_HIP.  Faults inside kernels surface at the caller's sync.
 *   - Device pointers must be 16-byte aligned; leading dimensions are in
 *     elements and must keep every row 16-byte aligned.
 *   - The library has no global state (except the static device scratch of
 *     mx_quantize_noalloc) and is thread-safe; calls on one stream run in
 *     order.
 */
#ifndef MX_H_
#define MX_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mx_status {
  MX_OK = 0,
  MX_ERR_NULL = -1,         /* a required pointer is NULL */
  MX_ERR_SHAPE = -2,        /* negative or inconsistent sizes / leading dims */
  MX_ERR_ALIGN = -3,        /* pointer or row not 16-byte aligned */
  MX_ERR_DTYPE = -4,        /* unknown or unsupported element type */
  MX_ERR_UNSUPPORTED = -5,  /* valid but not provided (e.g. cols % k != 0) */
  MX_ERR_HIP = -6,          /* a HIP launch failed */
  MX_ERR_WORKSPACE = -7,    /* workspace missing or too small */
  MX_ERR_FORMAT = -8        /* unknown format or mismatched operand formats */
} mx_status;

enum {
  MX_FMT_MXFP4 = 0,       /* E2M1 elements, 32-element blocks, E8M0 scales */
  MX_FMT_NVFP4 = 1,       /* E2M1, 16-element blocks, E4M3 scales, fp32 tensor scale */
  MX_FMT_MXFP8_E4M3 = 2,  /* 8-bit E4M3 elements, 32-element blocks, E8M0 scales */
  MX_FMT_MXFP8_E5M2 = 3,  /* 8-bit E5M2 */
  MX_FMT_MXFP6_E2M3 = 4,  /* 6-bit E2M3 */
  MX_FMT_MXFP6_E3M2 = 5,  /* 6-bit E3M2 */
  MX_FMT_MXFP4_K16 = 6,   /* E2M1, 16-element blocks, E8M0 scales, optional fp32 tensor scale */
  MX_FMT_FP4_TENSOR = 7   /* E2M1 with one fp32 scale for the whole tensor (naive baseline) */
};
enum { MX_DT_F32 = 0, MX_DT_BF16 = 1 };

/* mx_quantize flags */
enum {
  MX_QUANT_DEFAULT = 0,
  /* NVFP4: use *global_scale as given (a calibrated, static per-tensor scale)
     instead of computing it from the tensor's max |x|. */
  MX_QUANT_STATIC_GLOBAL = 1,
  /* E8M0-scaled formats: the OCP exponent rule e = floor(log2 max|x|) -
     floor(log2 Emax) instead of the pages' smallest e with max|x| <= Emax*2^e;
     elements beyond Emax then saturate to +-Emax. */
  MX_QUANT_SCALE_FLOOR = 2
};

/* mx_gemm_args.flags */
enum {
  /* MX pairs with an FP8 or FP6 operand: use the block-scaled FP8/FP6/FP4
     matrix cores (faster; products truncated, see mx_gemm) instead of the
     exact route.  Ignored for MXFP4 x MXFP4, whose products those matrix
     cores form exactly. */
  MX_GEMM_F8F6F4_MATRIX_CORES = 1,
  /* Dynamic MXFP4 A: quantize and multiply in one persistent kernel instead
     of a quantize launch followed by the GEMM (see mx_gemm). */
  MX_GEMM_FUSED_QUANTIZE = 2
};
/* Bits 4-7 of mx_gemm_args.flags: the element format a dynamic A is
   quantized to (MX_FMT_MXFP4, MX_FMT_MXFP8_* or MX_FMT_MXFP6_*); without it
   A takes the format of B. */
#define MX_GEMM_DYNAMIC_A_FORMAT(fmt) ((int32_t)(((fmt) + 1) << 4))

/* mx_workspace_bytes operations */
enum { MX_OP_QUANTIZE = 0, MX_OP_GEMM = 1, MX_OP_MOE_ROUTE = 2 };

typedef struct mx_tensor {
  int32_t fmt;            /* MX_FMT_* */
  int32_t reserved;       /* must be 0 */
  int64_t rows, cols;     /* logical shape; cols is the blocked (K) axis */
  uint8_t *codes;         /* device [rows, cols*b/8] (b = element bits) */
  uint8_t *scales;        /* device [rows, cols/k] */
  float *global_scale;    /* device fp32[1]; NVFP4 only, NULL for MXFP4 */
} mx_tensor;

/*
 * mx_quantize -- quantize a row-major [out->rows, out->cols] fp32/bf16 tensor.
 *
 * MXFP4 ("NVFP4 Architecture", section "1. The Dual-Level Mathematical
 * Formulation", equations S_block and q_i, with S_global = 1, and the pages'
 * PyTorch emulation): per 32-element block, m = max|x|;
 * e = max(-29, smallest integer with m <= 6*2^e) (the emulation's
 * max >= 1e-8 guard); scale byte e + 127; each element takes the E2M1 state
 * nearest to x/2^e, half-way cases to the even code, sign copied from x.
 * NVFP4: g = fp32(max|x| / 2688) over the whole tensor (1 if the tensor is 0),
 * or *global_scale with MX_QUANT_STATIC_GLOBAL; per 16-element block the E4M3
 * byte nearest to m/(6g) (ties to even, saturating at 448); elements take the
 * E2M1 state nearest to x/(s*g), saturating at +-6.  The computed g is written
 * to *out->global_scale.
 * MXFP4_K16: as MXFP4 with 16-element blocks and, when out->global_scale is
 * not NULL, g = *global_scale (set by the caller): e = smallest integer with
 * max(m, 1e-8) <= 6*g*2^e, elements the state nearest to x/(g*2^e) (g must
 * keep every e in [-127, 127]).  MX_FMT_FP4_TENSOR: s = fp32(max(max|x|,
 * 1e-8)/6) written to *out->global_scale, elements the state nearest to x/s
 * (saturating at 6); needs a workspace like dynamic NVFP4.  Flag
 * MX_QUANT_SCALE_FLOOR selects the OCP exponent rule for the E8M0-scaled
 * formats (not with a MXFP4_K16 tensor scale).  Rows whose length is not a
 * multiple of the block are zero-padded (layout above).  These variant paths
 * (MXFP4_K16, FP4_TENSOR, the floor rule, rows of any length) read x element
 * by element: any ld_x >= cols is accepted (x aligned to its element size).
 * MXFP8 / MXFP6: as MXFP4 with the element format's largest value Emax in
 * place of 6: e = smallest integer with max(m, fp32(1e-8)) <= Emax*2^e, scale
 * byte e + 127, each element the code nearest to x/2^e (ties to the even
 * code; the rule keeps |x|/2^e <= Emax, so nothing saturates and no NaN or
 * infinity code is produced).
 *   x          device, x_dtype (MX_DT_F32 / MX_DT_BF16), row pitch ld_x elems
 *   out        descriptor of the destination (device buffers caller-owned)
 *   workspace  device scratch of mx_workspace_bytes(MX_OP_QUANTIZE, out)
 *              bytes (0 for MXFP4 and for NVFP4 with MX_QUANT_STATIC_GLOBAL)
 * Requires cols % k == 0 (else MX_ERR_UNSUPPORTED).  rows == 0 is a no-op.
 * Inputs must be finite.
 */
int mx_quantize(const void *x, int32_t x_dtype, int64_t ld_x, const mx_tensor *out,
                int32_t flags, void *workspace, size_t workspace_bytes, void *stream);

/*
 * mx_quantize_noalloc -- mx_quantize without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * layouts, results and errors as mx_quantize; the dynamic NVFP4 and
 * FP4_TENSOR paths keep their per-workgroup partial maxima in a static
 * device array of 16 KiB inside the library (one per device, held until the
 * process ends) instead of a caller workspace, and the call allocates and
 * frees nothing.  Every call on one device shares that device's array, so
 * calls that overlap on one device (different streams or threads) race;
 * calls ordered on one stream do not.  Nothing in the array needs clearing:
 * every call writes each partial it reads.  A call whose scratch need
 * exceeds the array (never, for the sizes mx_quantize accepts) returns
 * MX_ERR_WORKSPACE.
 */
int mx_quantize_noalloc(const void *x, int32_t x_dtype, int64_t ld_x, const mx_tensor *out, int32_t flags,
                        void *stream);

/*
 * mx_dequantize -- x_hat = q * S_block * S_global ("NVFP4 Architecture",
 * section "1. The Dual-Level Mathematical Formulation", reconstruction
 * equation).  MXFP4, MXFP8, MXFP6: q * 2^(E-127) (exact in fp32 for every
 * scale the quantizer emits; otherwise rounded to nearest fp32); MXFP4_K16:
 * fp32(q * 2^(E-127) * g); FP4_TENSOR: fp32(q * s).  Only the first cols
 * elements of a padded row are written, and for those variant formats (and
 * rows of any length) any ld_y >= cols is accepted.  NVFP4:
 * fp32(fp32(q * s) * g).  bf16 output is the round-to-nearest-even of that
 * fp32 value.  y is device [in->rows, in->cols] with row pitch ld_y elements.
 */
int mx_dequantize(const mx_tensor *in, void *y, int32_t y_dtype, int64_t ld_y, void *stream);

/*
 * mx_gemm -- C[M, N] = A[M, K] . B[N, K]^T in native W4A4
 * (Y = X . W, "NVFP4 Architecture", section "1. The Dual-Level Mathematical
 * Formulation"; the block-scaled dot product with fp32 accumulation of
 * section "2. Hardware-Managed Tensor Core Dot-Products").
 *   MXFP4 x MXFP4: C = sum_b 2^(eA+eB) sum_{k in b} qA qB, fp32 accumulate.
 *   NVFP4 x NVFP4: C = gA gB sum_b sA sB sum_{k in b} qA qB.
 * Grouped form (groups >= 1): b holds `groups` stacked [N, K] matrices
 * (b->rows == groups * N); rows [off[g], off[g+1]) of A and C use matrix g.
 * `group_offsets` is a device int32 array of groups + 1 non-decreasing
 * entries with off[0] = 0 and off[groups] = M (entries are clamped to [0, M]
 * on the device, so malformed offsets cannot index out of bounds).
 * Dynamic activation quantization: pass a == NULL and a_raw (bf16/fp32
 * [M, K], pitch lda_raw elements, K % 32 == 0); A is quantized once (as
 * mx_quantize would) to the format of B, or to the MX format that
 * MX_GEMM_DYNAMIC_A_FORMAT(fmt) in flags names (e.g. MXFP8 E4M3 activations
 * against MXFP4 weights), into a_codes_out [M, K*b/8] / a_scales_out
 * [M, K/32] if given, else into the workspace, then multiplied: a quantize
 * launch, then the GEMM.  Not for NVFP4 B (MX_ERR_UNSUPPORTED); a format
 * outside the five MX formats, or one given while a != NULL, is
 * MX_ERR_FORMAT.
 * With flags MX_GEMM_FUSED_QUANTIZE (MXFP4 A and B, K % 512 == 0, lda_raw < 2^24, a
 * 256-CU device; otherwise the two launches run) one persistent kernel does
 * both, XCD by XCD: each XCD's workgroups quantize the rows of their share
 * of the output tiles, then multiply them, the last round of tiles split
 * along K.  Codes and scale bytes are identical either way; C agrees within
 * the fp32 summation-order tolerance (split tiles add K parts in a fixed
 * order, so repeated calls give identical C).  The workspace then also holds
 * the fused kernel's counters and partial tiles (mx_workspace_bytes), also
 * when a_codes_out/a_scales_out are given.  On MI355X the fused kernel is
 * not faster: a workgroup needs 157 KiB of LDS, one per CU, so the
 * memory-bound quantization cannot run beside the matrix-core work and
 * costs its full time in either form.
 * MXFP4 x MXFP4 and NVFP4 x NVFP4 with K % 256 == 0 (outside the fused
 * kernel): one workgroup per CU takes a 256 x 256 output tile, so when the
 * tile count T is not a multiple of the device's CU count the last T mod CUs
 * tiles would run alone; they are cut into up to 4 K parts instead, whose
 * fp32 partial tiles a second launch adds in part order (then times gA gB
 * for NVFP4; repeated calls give identical C; it agrees with the unsplit
 * kernel within the fp32 summation-order tolerance).
 * The partials live in the workspace after the quantized A (if any), which
 * mx_workspace_bytes then includes (up to CUs x 256 KiB, none for a dense
 * product that fills whole rounds); a workspace too small for them runs the
 * unsplit kernel.
 * c_dtype is MX_DT_F32 or MX_DT_BF16 (round-to-nearest-even), row pitch ldc.
 * Requires K % 32 == 0 (MXFP4) or K % 16 == 0 (NVFP4).
 * MX element pairs beyond MXFP4 x MXFP4 (A and B each MXFP4, MXFP8 E4M3/E5M2
 * or MXFP6 E2M3/E3M2, mixed pairs allowed, e.g. FP8 activations x FP4
 * weights): C = sum_b 2^(eA+eB) sum_{k in b} qA qB with fp32 accumulation,
 * every product exact (the codes are expanded to bf16 values q * 2^e for the
 * bf16 matrix cores, exact while each lies in [2^-126, 2^128), as for every
 * tensor the quantizer writes from inputs below 2^127 in magnitude; scale
 * bytes 0 and 255, which the quantizer never writes, are taken as 1 and 254).
 * With flags MX_GEMM_F8F6F4_MATRIX_CORES the pair runs on the block-scaled
 * FP8/FP6/FP4 matrix cores instead, about three times as fast, which
 * truncate each product of a group of 8 consecutive K to 13
 * bits below the largest product of the group (measured on gfx950): per
 * output the error grows by at most 8 * 2^(L_g - 12) per group g, L_g the
 * binary exponent of that largest product.  These pairs take the grouped
 * form and a dynamic A too; padded K % 128 == 0 and K <= 2^22 (else
 * MX_ERR_UNSUPPORTED).  NVFP4 pairs only with NVFP4 (else MX_ERR_FORMAT) and
 * has no grouped form (MX_ERR_UNSUPPORTED).  Pre-quantized MX operands
 * with K % 32 != 0 (zero-padded rows) multiply over the padded length, which
 * gives the same product.  MXFP4_K16 and FP4_TENSOR operands are not
 * provided (MX_ERR_UNSUPPORTED: their scales do not map onto the matrix
 * cores' 32-element blocks).
 */
typedef struct mx_gemm_args {
  int64_t M, N, K;
  const mx_tensor *a;            /* quantized A [M, K], or NULL (dynamic)   */
  const void *a_raw;             /* dynamic path: unquantized A            */
  int32_t a_raw_dtype;           /* MX_DT_F32 / MX_DT_BF16                  */
  int32_t groups;                /* 0: dense; >= 1: grouped                 */
  int64_t lda_raw;               /* elements                                */
  const mx_tensor *b;            /* [N, K] or [groups*N, K]                 */
  const int32_t *group_offsets;  /* device int32 [groups + 1] (grouped)     */
  void *c;                       /* device [M, N]                           */
  int32_t c_dtype;
  int32_t flags;                 /* MX_GEMM_* bits, or 0                    */
  int64_t ldc;                   /* elements                                */
  uint8_t *a_codes_out;          /* optional [M, K*b/8] (dynamic path)      */
  uint8_t *a_scales_out;         /* optional [M, K/32] (dynamic path)       */
  void *workspace;
  size_t workspace_bytes;
} mx_gemm_args;

int mx_gemm(const mx_gemm_args *args, void *stream);

/*
 * mx_gemv -- W4A16 decode product y[M, N] = x[M, K] . W_hat[N, K]^T with bf16
 * activations and MXFP4 weights dequantized in registers: weights stay
 * compressed in memory, the arithmetic is 16-bit x dequantized weight with
 * fp32 accumulation ("Extreme Quantization and Precision Engineering", section
 * "Key points", W4A16).  Every weight is expanded on chip to the exact bf16
 * value q * 2^e, so each product is exact and only the fp32 summation order
 * varies.  Which unit takes the products (MXFP4 weights):
 *   M <= 3, or any M when K % 256 != 0: the vector ALU (v_dot2_f32_bf16);
 *     no matrix cores;
 *   4 <= M <= 16 with K % 256 == 0: the bf16 matrix cores
 *     (v_mfma_f32_16x16x32_bf16, activation rows zero-padded to 16), because
 *     one dot2 per weight pair and activation row makes the vector ALU, not
 *     the weight stream, the bound from M = 4 on.
 * MXFP8 (E4M3 / E5M2) and MXFP6 (E2M3 / E3M2) weights (W8A16, W6A16) are
 * expanded the same way (exact: at most 4 significant bits, in bf16's normal
 * range for every tensor the quantizer writes) and take the same two routes:
 * the vector ALU for M <= 3 or K % 256 != 0, the bf16 matrix cores for
 * 4 <= M <= 16 with K % 256 == 0.  A scale byte 0 gives a zero block.
 * 1 <= M <= 16; x bf16 [M, K] pitch ld_x; y bf16 [M, N] pitch ld_y.
 * Requires K % 32 == 0.
 */
int mx_gemv(const void *x, int32_t x_dtype, int64_t M, int64_t ld_x, const mx_tensor *w,
            void *y, int32_t y_dtype, int64_t ld_y, void *stream);

/*
 * Routed mixture-of-experts layers around the grouped GEMM.  Expert weights
 * are where block-scaled FP4 pays most ("NVFP4 Architecture", section
 * "Strategic Recommendations: Adopting NVFP4 in 2026"); grouped GEMM and TopK
 * belong to an MXFP4 serving stack ("MXFP4" card, section "Core Facts").
 * A layer with top-k routing runs
 *   mx_moe_route      (token, slot) pairs -> expert-sorted rows
 *   mx_quantize_rows  the routed tokens' activations, in that order, to MXFP4
 *   mx_gemm           grouped W4A4 over offsets[] (groups = experts)
 *   mx_moe_combine    out[t] = sum_s weight[t, s] * y[dest_row[t, s]]
 *
 * mx_moe_route -- stable counting sort of the pairs by expert.
 *   topk_ids   device int32 [tokens, topk], expert of pair (t, s)
 *   offsets    device int32 [experts + 1] out: offsets[g] = number of pairs
 *              with a valid expert id below g (offsets[experts] = all valid)
 *   dest_row   device int32 [tokens * topk] out: row of pair (t, s) in the
 *              sorted order; -1 for an id outside [0, experts) (such pairs
 *              are dropped)
 *   src_token  device int32 [tokens * topk] out: token of sorted row r for
 *              r < offsets[experts] (entries beyond are not written)
 *   workspace  device, >= mx_workspace_bytes(MX_OP_MOE_ROUTE, &experts) bytes
 *              (per-chunk counts: 4 * max(1, 65536 / experts) * experts
 *              bytes, at most 256 KiB)
 * Pairs of one expert keep their flat order t * topk + s, so the result is
 * unique.  Three launches, each linear in the pairs plus the chunk counts:
 * counts per chunk of consecutive pairs, one prefix over them (expert by
 * expert), and one wave per chunk that gives its pairs their rows in order.
 * 1 <= topk, 1 <= experts <= 65536, tokens * topk < 2^31.
 */
int mx_moe_route(const int32_t *topk_ids, int64_t tokens, int32_t topk, int32_t experts,
                 int32_t *offsets, int32_t *dest_row, int32_t *src_token,
                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * mx_quantize_rows -- MXFP4 quantization (exactly as mx_quantize) of gathered
 * rows: output row r is input row row_index[r] of x (device int32
 * [out->rows]); an index outside [0, x_rows) gives an all-zero row (scale
 * byte 98, +0 codes).  x is [x_rows, out->cols] with pitch ld_x elements.
 */
int mx_quantize_rows(const void *x, int32_t x_dtype, int64_t ld_x, int64_t x_rows,
                     const int32_t *row_index, const mx_tensor *out, void *stream);

/*
 * mx_moe_combine -- out[t, n] = sum_{s < topk} weights[t, s] * y[dest_row[t, s], n]
 * with fp32 accumulation in slot order (fused multiply-add); a pair whose row
 * is outside [0, y_rows) adds nothing.  y is [y_rows, N] (f32 or bf16, pitch
 * ld_y), out is [tokens, N] (f32 or bf16 round-to-nearest-even, pitch
 * ld_out), weights device fp32 [tokens, topk].  Requires N % 8 == 0.
 */
int mx_moe_combine(const void *y, int32_t y_dtype, int64_t ld_y, int64_t y_rows,
                   const int32_t *dest_row, const float *weights, int64_t tokens, int32_t topk,
                   int64_t N, void *out, int32_t out_dtype, int64_t ld_out, void *stream);

/*
 * mx_rmsnorm_quantize -- RMSNorm fused with the FP4 quantization of its
 * output, so the normalized activations never round-trip through HBM
 * (dynamic re-quantization is the overhead "NVFP4 Architecture" names in
 * section "The Problem"; RMSNorm belongs to an MXFP4 serving stack, "MXFP4"
 * card, section "Core Facts").  Per row of x (bf16 [out->rows, out->cols],
 * pitch ld_x):
 *   s   = fp32 sum of x_k^2: thread t of 256 adds the squares of the
 *         32-element chunks t, t+256, ... in element order, then the 256
 *         partials are added as a pairwise tree over thread index (per 64,
 *         then (w0 + w1) + (w2 + w3));
 *   r   = fp32(1 / sqrt(s / K + eps)) evaluated in fp64;
 *   y_k = fp32(fp32(x_k * r) * gamma_k)   (gamma fp32 or bf16 [K]);
 * and y is quantized exactly as mx_quantize quantizes fp32 input: MXFP4
 * (flags 0) or NVFP4 with the caller's per-tensor scale *out->global_scale
 * (flags MX_QUANT_STATIC_GLOBAL: no tensor-wide max pass).
 * Requires K % 32 == 0 and K <= 32768 (else MX_ERR_UNSUPPORTED) and eps > 0
 * (so an all-zero row stays finite; else MX_ERR_SHAPE).
 */
int mx_rmsnorm_quantize(const void *x, int32_t x_dtype, int64_t ld_x, const void *gamma,
                        int32_t gamma_dtype, float eps, const mx_tensor *out, int32_t flags,
                        void *stream);

/* Scratch bytes that op needs: desc is an mx_tensor* (MX_OP_QUANTIZE, with
   flags as in mx_quantize), an mx_gemm_args* (MX_OP_GEMM) or a pointer to
   the int32 expert count (MX_OP_MOE_ROUTE). */
size_t mx_workspace_bytes(int32_t op, const void *desc, int32_t flags);

/* Static, never-NULL description of a status code. */
const char *mx_status_string(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
int mx_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MX_H_ */
