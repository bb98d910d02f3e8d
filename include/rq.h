/*
 * rq.h -- C ABI of librq: matrix products that read group-wise quantized
 * RWKV-7 projection weights directly, on AMD MI355X (gfx950).
 *
 * What is computed.  A weight matrix W[N][K] (N outputs, K inputs) is stored
 * quantized; a product computes y[m][n] = sum_k x[m][k] * W_hat[n][k] where
 * W_hat is the dequantized weight, without ever writing W_hat out.  This is
 * the "no dequantization" inference of the RWKV-7 Quantization Toolkit page
 * (Key Design) and the int4 GEMV / small-M GEMM family of the
 * "RWKV-7 G1 1.5B -- int4 GPTQ for rwkv-sglang" model card (summary:
 * decode at batch <= 32; "Format & loading": group-wise symmetric int4 with a
 * .qweight code tensor and a .scale tensor, fp16 activations).
 *
 * Conventions shared by every entry point
 *   - Every buffer pointer is a DEVICE pointer on the current HIP device,
 *     except the rq_qweight descriptor itself and the size_t outputs of
 *     rq_qweight_bytes, which live in host memory.  The caller allocates and
 *     frees every buffer it passes; the library keeps no pointer to them
 *     after returning.
 *   - Workspace: the products (rq_gemv_*, rq_gemm_small_m, rq_fused_rkv,
 *     rq_gemm_w4, rq_gemm_fp8, rq_gemm_int8, rq_gemm_int8_acc) may cut K
 *     across workgroups and add the partial sums afterwards.  The partial
 *     sums live in a device buffer the CALLER owns and passes as
 *     (workspace, workspace_bytes): 16-byte aligned, disjoint from the call's
 *     inputs and outputs (RQ_ERR_ALIGN, RQ_ERR_ALIAS).  Its first 64 KiB hold
 *     the arrival counters through which the weight-streaming products
 *     (rq_gemv_*, rq_gemm_small_m, rq_fused_rkv) let the last workgroup of
 *     each tile group split into up to four K slices add the partial sums,
 *     in the same launch (more slices are added by a second kernel): the
 *     caller ZERO-FILLS them once, before the buffer's first use (e.g. one
 *     hipMemset of the whole buffer after allocating it), and every call
 *     leaves them at zero when it completes.  Bytes past the first 64 KiB
 *     hold nothing between calls.  rq_workspace_bytes() is the size that
 *     admits every product's fastest launch shape; with a smaller buffer (64
 *     KiB or less counts as none), or workspace == NULL (workspace_bytes is
 *     then ignored), the planner keeps to the shapes that fit, down to no K
 *     split at all.  The launch shape is a function of the arguments alone
 *     (shapes, formats, whether a workspace is given and its size), never of
 *     earlier calls.  No product call allocates device memory.  Calls that
 *     may run at the same time (on different streams, or graph replays on
 *     different streams) need distinct workspaces.
 *   - fp16 values are IEEE binary16 bit patterns (uint16_t).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued on it; product calls return without synchronizing.
 *   - Return value: RQ_OK (0) or a negative rq_status.  On a validation error
 *     nothing is launched and no output is touched.  A failed launch returns
 *     RQ_ERR_HIP.  Faults inside a kernel surface at the caller's next
 *     synchronization.  No C++ exception crosses the ABI.
 *   - Alignment: every device pointer must be 16-byte aligned (RQ_ERR_ALIGN);
 *     leading dimensions of fp16 activation arrays (ldx) are multiples of 8
 *     elements.  Outputs may not overlap any input (RQ_ERR_ALIAS).
 *   - Shapes: n >= 0 and m >= 0 (zero = nothing to do, RQ_OK, but pointers must
 *     still be valid), k >= 1, n and k below 2^31, and the per-format rules of
 *     rq_qweight.
 *   - Determinism: the same inputs and workspace size on the same device
 *     give bit-identical outputs (fixed reduction order, no floating-point
 *     atomics).  Different entry points over the same weights (a fused call
 *     and three single calls), or different workspace sizes, may split K
 *     differently and then differ within the fp32 summation tolerance.
 *   - Thread safety: the library keeps no state between calls; calls on
 *     different streams may run concurrently given distinct workspaces.
 */
#ifndef RQ_H
#define RQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RQ_ABI_VERSION 5

enum rq_status {
  RQ_OK = 0,
  RQ_ERR_NULL = -1,      /* a required pointer is NULL                         */
  RQ_ERR_SHAPE = -2,     /* bad n, m, k, ld, or k not a multiple of the group  */
  RQ_ERR_ALIGN = -3,     /* pointer or leading dimension misaligned            */
  RQ_ERR_FORMAT = -4,    /* unknown format/group, or wrong entry for format    */
  RQ_ERR_NONFINITE = -5, /* NaN or Inf in quantizer input                      */
  RQ_ERR_RANGE = -6,     /* a scale overflows its storage type                 */
  RQ_ERR_HIP = -7,       /* a HIP runtime call failed                          */
  RQ_ERR_ALIAS = -8,     /* an output overlaps an input                        */
  RQ_ERR_SCRATCH = -9,   /* too large for rq_gemm_small_m_noalloc's scratch    */
  RQ_ERR_DEGENERATE = -10 /* rq_proxy: every weight equal (no gap to normalise) */
};

/*
 * Weight formats.  Layouts are row-major over W[N][K]; "group" runs along K
 * inside one row.
 *
 * RQ_W8_SYM, RQ_W4_SYM (group 16, 32 or 64; k % group == 0)
 *   Symmetric round-to-nearest codes with one fp16 scale per (row, group):
 *   Q = 127 (int8) or 7 (int4), s = fp16(absmax / Q), q = clamp(RNE(w/s), -Q, Q),
 *   W_hat = q * s.  Model card, "Format & loading" (GROUP=64 symmetric int4)
 *   and accuracy warning (int8 w8g64 tier); rwkv-quant news article, section
 *   "Dois presets e seis tamanhos" (8-bit symmetric projections, group 16).
 *     codes : int8 [n][k]                          (W8)
 *             uint8 [n][k/2], u = q + 8 in 4-bit words (W4): see "int4
 *             code words" below
 *     scales: fp16 [n][k/group]
 * RQ_W4_ASYM_SB256 (group must be 32; k % 256 == 0)
 *   Asymmetric 4-bit codes in superblocks of 256 = 8 groups of 32 (news
 *   article, "Dois presets e seis tamanhos": 4-bit asymmetric superblocks,
 *   group 32).  Per group j: S_j = d * sc_j, M_j = dmin * mc_j,
 *   W_hat = S_j * q - M_j with q in 0..15.
 *     codes : uint8 [n][k/2] (q in 4-bit words: see "int4 code words")
 *     scales: fp16 d    [n][k/256]
 *     mins  : fp16 dmin [n][k/256]
 *     sub   : uint8 [n][k/256][12]: 96-bit little-endian stream, sc_j at bit
 *             6j and mc_j at bit 48 + 6j (6-bit codes)
 * RQ_FP8_E4M3_CH, RQ_I8_CH (group ignored; k % 16 == 0; the MFMA GEMMs need
 *   k % 128 == 0)
 *   One fp32 scale per output row: s_n = fp32(absmax_n / 448) with OCP e4m3fn
 *   codes (saturating RNE), or fp32(absmax_n / 127) with int8 codes in
 *   -127..127 (RWKV-7 Quantization Toolkit, Key Design: FP8 weights on FP8
 *   tensor cores, INT8 through int8 x int8 dot products).
 *     codes : uint8 (e4m3fn) or int8 [n][k];  scales: fp32 [n]
 * RQ_F16 (group ignored; k % 8 == 0)
 *   Unquantized fp16 weights, used for the output head, which the toolkit
 *   keeps in FP16 (Key Design) and the model card keeps full precision.
 *     codes : fp16 [n][k];  scales, mins, sub: unused
 * RQ_W6_SYM, RQ_W5_SYM (group 32 or 64; k % 128 == 0)
 *   The 6- and 5-bit widths of the news article's presets ("Dois presets e
 *   seis tamanhos": channel-mix weights at 6 bits; channel-mix key and head at
 *   5 bits).  The article gives the widths only; these are the symmetric rule
 *   above with Q = 31 / 15.  Codes are offset binary u = q + 32 / q + 16 in two
 *   planes:
 *     codes : uint8 [n][k/2], the low nibbles u & 15 as int4 code words
 *     sub   : the high bits u >> 4 per 8-k word w, with e = hi(8w + 2i) and
 *             o = hi(8w + 2i + 1), i = 0..3:
 *             W6: uint16 [n][k/8], bits 4i..4i+1 = e, 4i+2..4i+3 = o;
 *             W5: uint8  [n][k/8], bit i = e, bit 4 + i = o
 *     scales: fp16 [n][k/group];  mins: unused
 * RQ_BF16 (group ignored; k % 32 == 0)
 *   bfloat16 weights (news article, "Onde o 2.9B quebra": the first block's
 *   output projection kept in bf16).  The quantizer rounds fp32 to nearest,
 *   ties to even; a weight past the largest finite bf16 is RQ_ERR_RANGE.
 *     codes : bf16 [n][k];  scales, mins, sub: unused
 *
 * int4 code words (RQ_W4_SYM, RQ_W4_ASYM_SB256).  The pages fix no nibble
 * order; each run of 8 consecutive k of a row is one little-endian 32-bit
 * word whose bits 4i..4i+3 hold k = 2i and bits 16+4i..16+4i+3 hold
 * k = 2i + 1 (i = 0..3), i.e. bytes [u0|u2<<4, u4|u6<<4, u1|u3<<4, u5|u7<<4].
 * Even k fill the low half-word and odd k the high one, so a pair (2i,
 * 2i + 1) decodes with one mask into the two halves of a packed fp16 pair.
 *
 * For quantizers, a zero scale (all-zero group, or a scale that rounds to
 * zero) gives all-zero codes.
 */
enum rq_format {
  RQ_W8_SYM = 1,
  RQ_W4_SYM = 2,
  RQ_W4_ASYM_SB256 = 3,
  RQ_FP8_E4M3_CH = 4,
  RQ_I8_CH = 5,
  RQ_F16 = 6,
  RQ_W5_SYM = 7,
  RQ_W6_SYM = 8,
  RQ_BF16 = 9
};

/* Host-side descriptor of one quantized weight; the four buffers are device
 * pointers laid out as described for the format (unused ones may be NULL). */
typedef struct rq_qweight {
  int32_t format;
  int32_t group;
  int64_t n;
  int64_t k;
  void *codes;
  void *scales;
  void *mins;
  void *sub;
} rq_qweight;

/* ABI version of the loaded library (RQ_ABI_VERSION). */
int rq_abi_version(void);

/* Static text for a status code (never NULL). */
const char *rq_status_str(int status);

/* Size in bytes of the workspace that admits every product's fastest launch
 * shape (see Workspace above).  Host-only. */
size_t rq_workspace_bytes(void);

/* Byte sizes of the four buffers of a (format, group, n, k) weight.  Any of
 * the output pointers may be NULL.  Host-only; launches nothing.
 * Errors: RQ_ERR_FORMAT, RQ_ERR_SHAPE. */
int rq_qweight_bytes(int format, int group, int64_t n, int64_t k, size_t *codes_bytes,
                     size_t *scales_bytes, size_t *mins_bytes, size_t *sub_bytes);

/* Round-to-nearest quantization of fp32 weights w[n][k] (device, contiguous)
 * into the format, group, n and k named by *out (the group-wise codes plus
 * scales of the model card's "Format & loading" -- a .qweight code tensor and
 * a .scale tensor -- and the formats listed above with their pages), whose buffers the caller has
 * allocated with rq_qweight_bytes sizes.  Every quotient is an IEEE fp64
 * division followed by one rounding to the target grid, so the codes and
 * scales are exactly those of the format's definition.  Synchronizes `stream`
 * (it reads back a status word); allocates and frees 4 bytes of device memory
 * per call.  Errors: validation codes, RQ_ERR_NONFINITE (NaN/Inf in w),
 * RQ_ERR_RANGE (a scale overflows fp16/fp32); after those two the output
 * buffers hold unspecified bytes.  RQ_F16 converts to fp16 (RNE). */
int rq_quantize_rtn(const float *w, const rq_qweight *out, void *stream);

/* Activation-weighted quantization (rwkv-quant news article, section "Dois
 * presets e seis tamanhos": group scales and offsets chosen by a search
 * weighted by E[x^2] of each input channel).  act_sq[k] (device fp32,
 * 16-byte aligned, finite and >= 0) is that mean square per input channel.
 * For each group, 16 candidates shrink the RTN scale (symmetric formats: the
 * fp16 scale absmax/Q times 1 - t/32, t = 0..15) or both ends of the RTN
 * range (RQ_W4_ASYM_SB256: lo and hi times 1 - t/32, scored with the
 * unquantized scale and offset) and are scored by sum a_k (w_k - w_hat_k)^2
 * in fp64; the smallest t within a factor 1 + 2^-40 of the lowest score is
 * kept (step 0 is RTN, so an all-zero act_sq gives rq_quantize_rtn's bytes).
 * Superblock weights then take the RTN superblock step with the chosen group
 * parameters.  Formats: RQ_W8_SYM, RQ_W4_SYM, RQ_W6_SYM, RQ_W5_SYM,
 * RQ_W4_ASYM_SB256, else RQ_ERR_FORMAT.  Synchronization, allocation and errors as rq_quantize_rtn;
 * a NaN, Inf or negative act_sq entry gives RQ_ERR_NONFINITE.  act_sq may
 * not overlap an output buffer (RQ_ERR_ALIAS). */
int rq_quantize_aw(const float *w, const float *act_sq, const rq_qweight *out, void *stream);

/* M = 1 products y[n] = sum_k x[k] * W_hat[n][k], fp32 accumulation, fp16
 * output (RNE): the int4 GEMV of the model card's summary (decode reads the
 * packed codes and scales directly, no dequantized copy: RWKV-7 Quantization
 * Toolkit, Key Design), and its int8 tier (model card, accuracy warning:
 * w8g64).  x: fp16 [k]; y: fp16 [n].  Each entry point accepts exactly
 * its format and group (RQ_ERR_FORMAT otherwise):
 *   w4gG: RQ_W4_SYM, group G;  w8gG: RQ_W8_SYM, group G;
 *   w4sb256: RQ_W4_ASYM_SB256;  f16: RQ_F16. */
int rq_gemv_w4g16(const uint16_t *x, const rq_qweight *w, uint16_t *y, void *workspace,
                  size_t workspace_bytes, void *stream);
int rq_gemv_w4g32(const uint16_t *x, const rq_qweight *w, uint16_t *y, void *workspace,
                  size_t workspace_bytes, void *stream);
int rq_gemv_w4g64(const uint16_t *x, const rq_qweight *w, uint16_t *y, void *workspace,
                  size_t workspace_bytes, void *stream);
int rq_gemv_w8g16(const uint16_t *x, const rq_qweight *w, uint16_t *y, void *workspace,
                  size_t workspace_bytes, void *stream);
int rq_gemv_w8g32(const uint16_t *x, const rq_qweight *w, uint16_t *y, void *workspace,
                  size_t workspace_bytes, void *stream);
int rq_gemv_w8g64(const uint16_t *x, const rq_qweight *w, uint16_t *y, void *workspace,
                  size_t workspace_bytes, void *stream);
int rq_gemv_w4sb256(const uint16_t *x, const rq_qweight *w, uint16_t *y, void *workspace,
                    size_t workspace_bytes, void *stream);
int rq_gemv_f16(const uint16_t *x, const rq_qweight *w, uint16_t *y, void *workspace,
                size_t workspace_bytes, void *stream);

/* Small-M products for decode batches 1 <= m <= 32 (model card, summary:
 * batch sizes up to 32).  x: fp16 [m][ldx], ldx >= k, ldx % 8 == 0;
 * y: fp16 [m][ldy], ldy >= n.  Accepts RQ_W8_SYM, RQ_W4_SYM,
 * RQ_W4_ASYM_SB256, RQ_F16, RQ_W6_SYM, RQ_W5_SYM and RQ_BF16.  The weights
 * are read once per call.
 * Errors: RQ_ERR_SHAPE for m outside 0..32.  RQ_W6_SYM, RQ_W5_SYM and
 * RQ_BF16 have one kernel, whose activation slice must fit LDS; they also
 * return RQ_ERR_SHAPE when one weight buffer or the activation span
 * m * ldx * 2 reaches 2^31 bytes, or when K cut into 16 slices still leaves
 * a slice too large: with chunks of C = 128 k (RQ_W6_SYM, RQ_W5_SYM) or 32 k
 * (RQ_BF16) and c = ceil(k / 16 / C) chunks per slice, (m + 1) * (c * C + 8)
 * above 40960 (k above 18432 at m = 32, 36864 at m = 16) or c above 128
 * (256 for RQ_BF16 at m <= 2).  Cutting K needs a workspace of enough bytes (see
 * Workspace); without one, (m + 1) * (k + 8) must stay within 40960, or
 * 76800 for 128 or more row tiles (192 to 256 row tiles also stream k up to
 * 8192 at m > 16 and 16384 at m = 4..8).  Other formats take any shape. */
int rq_gemm_small_m(const uint16_t *x, int64_t m, int64_t ldx, const rq_qweight *w,
                    uint16_t *y, int64_t ldy, void *workspace, size_t workspace_bytes, void *stream);

/* The launch rq_gemm_small_m would make for weight w, m rows of x with row
 * stride ldx and a workspace of workspace_bytes (0: none), described
 * without launching (the same planner; host only, no GPU call, nothing is
 * read through w's buffer pointers).  For callers that size workspaces, pick
 * batch sizes or check a launch shape ahead of graph capture.
 * kernel: RQ_PLAN_NONE when nothing would be launched (m == 0 or n == 0);
 *   RQ_PLAN_STREAMING: one workgroup per group of tiles per K slice, the
 *   activation slice copied once into LDS; RQ_PLAN_TWO_RANGES: the same on
 *   8-row tiles that each cover K as two halves (int4 groups, m <= 8);
 *   RQ_PLAN_STREAMED_X: each wave streams its own chunks of x; RQ_PLAN_PHASED:
 *   x, codes and scales moved through LDS in phases of 512 k (int4 groups,
 *   m > 16, or m >= 9 in place of a split into more than four slices or
 *   where four row tiles per workgroup need no split);
 *   RQ_PLAN_FIRST: the one-tile-per-workgroup kernel.
 * split > 1: K is cut into split slices of chunks_per_slice chunks (128 k
 * for 4-, 5-, 6-bit codes and SB256, 64 k for int8, 32 k for fp16/bf16), the
 * counters and partial tiles take the first workspace_bytes of the workspace;
 * the last workgroup of each tile group adds them in the same launch for
 * split <= 4 (at most 16384 tile groups), a second kernel for more slices.  lds_bytes: dynamic LDS of the main launch; threads: per
 * workgroup.  Errors as rq_gemm_small_m's validation (the buffer pointers
 * must be valid descriptors but are not dereferenced; ldx as for x there),
 * RQ_ERR_SHAPE when no launch shape exists, RQ_ERR_NULL for a null out. */
enum {
  RQ_PLAN_NONE = 0,
  RQ_PLAN_STREAMING = 1,
  RQ_PLAN_TWO_RANGES = 2,
  RQ_PLAN_STREAMED_X = 3,
  RQ_PLAN_PHASED = 4,
  RQ_PLAN_FIRST = 5
};
typedef struct rq_plan {
  int32_t kernel;              /* RQ_PLAN_* */
  int32_t split;               /* K slices */
  int32_t chunks_per_slice;
  int32_t chunks_per_wave;     /* streaming kernels; 0 otherwise */
  int32_t waves_per_tile;      /* streaming kernels; 0 otherwise */
  int32_t tiles_per_workgroup;
  int32_t workgroups;          /* of the main launch */
  int32_t threads;             /* per workgroup */
  int64_t lds_bytes;
  int64_t workspace_bytes;
} rq_plan;
int rq_plan_small_m(const rq_qweight *w, int64_t m, int64_t ldx, size_t workspace_bytes, rq_plan *out);

/* rq_gemm_small_m for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, formats and results as
 * rq_gemm_small_m given a workspace of rq_workspace_bytes() (the same launch
 * shape, so the same bits).  Its K-split partial sums use a static device
 * array of 8 MiB per GPU (after 64 KiB of split counters, zero when the
 * library is loaded and left at zero by every call), owned by the library and
 * held until the process ends; a call allocates nothing.  Limit: 16 * ceil(n / 16) * t * 1024 bytes
 * must fit in 8 MiB, t = 1 for m <= 16 and 2 above (n <= 4096 at any m,
 * n <= 8192 at m <= 16); larger calls return RQ_ERR_SCRATCH.  Every call on
 * a GPU shares that GPU's array: calls that overlap in time on one GPU
 * (different streams, or graph replays running concurrently) race. */
int rq_gemm_small_m_noalloc(const uint16_t *x, int64_t m, int64_t ldx, const rq_qweight *w,
                            uint16_t *y, int64_t ldy, void *stream);

/* Prefill products on int4 codes for any number of rows m (the tensor-core
 * GEMM member of the int4 family in the model card's summary), on MFMA:
 * y[m][n] = fp16(sum_k x[m][k] * w[n][k]) with fp32 accumulation.  RQ_W4_SYM
 * (group 16, 32 or 64; k % 128 == 0): the weight is dequantized to fp16 in
 * registers, w = fp16(q * s), at most 2^-11 of the weight off (one rounding);
 * RQ_W4_ASYM_SB256: per 32-group, S_j * sum(x u) - M_j * sum(x) with both sums
 * on MFMA and S_j, M_j applied in fp32, nothing rounded below fp32.  Other formats:
 * RQ_ERR_FORMAT.  x: fp16 [m][ldx], ldx >= k, ldx % 8 == 0; y: fp16
 * [m][ldy], ldy >= n.  The weights are read once per tile row of 64 or 128
 * activation rows; meant for m from about 64 up (rq_gemm_small_m covers
 * m <= 32).  Any m >= 0. */
int rq_gemm_w4(const uint16_t *x, int64_t m, int64_t ldx, const rq_qweight *w, uint16_t *y,
               int64_t ldy, void *workspace, size_t workspace_bytes, void *stream);

/* The R, K and V projections in one launch (RWKV-7 Quantization Toolkit,
 * Key Design: "R/K/V projections computed in a single kernel launch").
 * Three independent small-M products with a shared m, ldx and ldy; the three
 * weights must have the same format, group and k (their n may differ).
 * xr, xk, xv may be the same pointer (a shared input); the outputs may not
 * overlap each other or any input. */
int rq_fused_rkv(const uint16_t *xr, const uint16_t *xk, const uint16_t *xv, int64_t m,
                 int64_t ldx, const rq_qweight *wr, const rq_qweight *wk, const rq_qweight *wv,
                 uint16_t *yr, uint16_t *yk, uint16_t *yv, int64_t ldy, void *workspace,
                 size_t workspace_bytes, void *stream);

/* Per-token dynamic activation quantization for the W8A8 / FP8 GEMMs (both
 * operands of the toolkit's int8 x int8 and fp8 x fp8 products are
 * quantized): for each row m of x (fp16 [m][ldx]), s_x[m] = fp32(absmax/448)
 * with e4m3fn codes (format RQ_FP8_E4M3_CH) or fp32(absmax/127) with int8
 * codes in -127..127 (RQ_I8_CH), quotients in fp64.  xq: [m][k] bytes,
 * contiguous; sx: fp32 [m].  k % 16 == 0. */
int rq_quantize_act(const uint16_t *x, int64_t m, int64_t k, int64_t ldx, int format, void *xq,
                    float *sx, void *stream);

/* FP8 x FP8 GEMM on MFMA: y[m][n] = fp16(s_x[m] * s_w[n] * sum_k dec(xq[m][k]) *
 * dec(wq[n][k])) with fp32 accumulation (toolkit, Key Design and
 * Architecture: FP8 GEMM with shape-aware tile configurations).  xq: e4m3fn
 * [m][k]; w: RQ_FP8_E4M3_CH with k % 128 == 0; y: fp16 [m][ldy], ldy >= n.
 * Any m >= 0. */
int rq_gemm_fp8(const uint8_t *xq, const float *sx, int64_t m, const rq_qweight *w, uint16_t *y,
                int64_t ldy, void *workspace, size_t workspace_bytes, void *stream);

/* INT8 x INT8 GEMM on MFMA with exact int32 accumulation ("INT8 via DP4A" on
 * the toolkit page): y[m][n] = fp16(float(acc) * s_x[m] * s_w[n]).
 * w: RQ_I8_CH with k % 128 == 0 and k <= 131072 (|acc| < 2^31). */
int rq_gemm_int8(const int8_t *xq, const float *sx, int64_t m, const rq_qweight *w, uint16_t *y,
                 int64_t ldy, void *workspace, size_t workspace_bytes, void *stream);

/* The int32 accumulators of rq_gemm_int8 (acc: int32 [m][n], contiguous),
 * for bit-exact checking of the integer contraction. */
int rq_gemm_int8_acc(const int8_t *xq, int64_t m, const rq_qweight *w, int32_t *acc,
                     void *workspace, size_t workspace_bytes, void *stream);

/* Measurement aid: reads `bytes` of device memory at buf (16-byte aligned,
 * bytes % 16 == 0) with 16-byte non-temporal loads spread over every compute
 * unit and stores nothing but, at most, one word to *sink (device, 4-byte
 * aligned).  A read-only stream: what the memory system delivers to a kernel
 * that does nothing else, the ceiling the weight-streaming products are
 * measured against beside the 8 TB/s peak.  Errors: RQ_ERR_NULL,
 * RQ_ERR_ALIGN, RQ_ERR_SHAPE. */
int rq_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);

/* RWKVQuant's weights-only coarse-to-fine proxy of one weight tensor (RWKVQuant:
 * Quantizing the RWKV Family with Proxy Guided Hybrid of Scalar and Vector
 * Quantization -- Abstract on the index page; machine-review page,
 * pith_extraction.key_machinery): the `count` fp32 weights at w (HOST memory,
 * any order; the tensor is flattened) are sorted, their n = count - 1 adjacent
 * gaps divided by the mean gap (g), and
 *   *pc = P_c = H(uniform gaps) - H(gaps) = log n - H(g / sum g)   (nats)
 *   *pf = P_f = sum_{k=2..K} v[k-2] * |M_k|,  M_k = mean((g - mean g)^k)
 * with v = NULL meaning v_k = 1/k!.  moments (may be NULL) receives M_2..M_K
 * (K - 1 doubles).  The pages route a layer to scalar quantization only when
 * P_c < tau_c and P_f < tau_f (tau_c = 1.54, tau_f = 30 reported for RWKV-7);
 * they leave the gap normalisation, the entropy's base and binning, K and v_k
 * open, and the values here follow the readings stated above.  Runs on the
 * calling thread, O(count log count) for the sort, allocates a host copy of
 * the weights.  Errors: RQ_ERR_NULL (w, pc or pf), RQ_ERR_SHAPE (count < 3,
 * K < 2 or K > RQ_PROXY_MAX_K), RQ_ERR_NONFINITE, RQ_ERR_DEGENERATE. */
#define RQ_PROXY_MAX_K 16
int rq_proxy(const float *w, int64_t count, int K, const double *v, double *pc, double *pf,
             double *moments);

/* Test aid: the library's own fp64 -> fp16 (kind 0, uint16 out), fp64 ->
 * fp32 (kind 1, uint32 out) and fp64 -> e4m3fn (kind 2, uint8 out)
 * round-to-nearest-even conversions, run on the host over `count` values of
 * host arrays.  These are the conversions the quantizer kernels use.
 * Errors: RQ_ERR_NULL, RQ_ERR_SHAPE (count < 0), RQ_ERR_FORMAT (kind). */
int rq_host_convert(int kind, const double *in, void *out, int64_t count);

#ifdef __cplusplus
}
#endif

#endif /* RQ_H */
