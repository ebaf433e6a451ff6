/*
 * hq.h -- C ABI of the MI355X (gfx950) block-scaled low-precision GEMM library.
 *
 * The operations follow the HALOps "GEMM" API page (sections group_wise_quant,
 * dense_gemm, batch_gemm, group_contiguous_gemm, group_masked_gemm,
 * fused_swiglu_quant), the flashrt/fp4-gemm kernel page (NVFP4 A4W4 GEMM with
 * BF16 output; unsupported calls fail before launch, output never silently
 * undefined; calls usable under graph capture) and cuDNN FE "Grouped GEMM +
 * dGLU (SM100)" (Step 1: the grouped GEMM over cumulative group offsets; the
 * Data Types table; at most 1024 experts; 16-byte aligned tensors).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - All tensor pointers are DEVICE pointers (memory of the current HIP
 *    device).  The caller allocates and owns every buffer, the FP32
 *    workspace of a K-split GEMM included (hq_dense_gemm_ws,
 *    hq_batch_gemm_ws; the flashrt/fp4-gemm page's large-M tier, whose
 *    workspace is caller-owned, allocated before graph capture and passed on
 *    every replay).  The library allocates no memory, keeps no pointer after
 *    a call returns and never synchronises the host.  Work is enqueued on
 *    `stream` (a hipStream_t; NULL = the null stream) and is stream-ordered
 *    with no memset nodes, so a call may be captured into a graph.
 *  - BF16 values are passed as their uint16_t bit patterns.
 *  - Quantised operands are K-major and row-major:
 *        MXFP8: codes uint8 [rows, K]      (E4M3 "fn")
 *        MXFP4: codes uint8 [rows, K/2]    (E2M1, element 2j in the low nibble
 *                                           of byte j, element 2j+1 high)
 *        NVFP4: codes uint8 [rows, K/2]    (E2M1, same packing)
 *    Scale factors are uint8, plain row-major [rows, K/gs]:
 *        MXFP8, MXFP4: gs = 32, UE8M0 (byte b means 2^(b-127))
 *        NVFP4:        gs = 16, UE4M3 (E4M3 bit pattern, sign clear)
 *    NVFP4 additionally carries one FP32 global scale per tensor; a GEMM takes
 *    alpha = g_A * g_B.
 *  - Inputs are const; outputs are written in place and only at valid rows.
 *  - Every call validates its arguments on the host BEFORE any device work.
 *    On error nothing is launched and no output byte is written; the status
 *    is returned and hq_last_error() describes it.
 *  - Counts and offsets that live in device memory cannot be validated by the
 *    host.  Kernels clamp them: a masked count to [0, max_m_per_group]; a
 *    group end to [previous end, m_total].
 *  - Size limits: k > 0, k % 32 == 0; n % 8 == 0; h % 32 == 0;
 *    1 <= num_groups <= 1024; row counts < 2^31; m == 0 or n == 0 is a no-op.
 *    Pointers to x, a, b, q and out must be 16-byte aligned.
 */
#ifndef HQ_H_
#define HQ_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Quantisation recipe ("w8a8-mxfp8", "w4a4-mxfp4", "w4a4-nvfp4" on the
 * HALOps page). */
typedef enum {
  HQ_MXFP8 = 0,
  HQ_MXFP4 = 1,
  HQ_NVFP4 = 2
} hq_mode;

typedef int32_t hq_status;

#define HQ_OK 0
#define HQ_ERR_NULL (-1)   /* a required pointer is NULL                    */
#define HQ_ERR_SHAPE (-2)  /* invalid dimensions                            */
#define HQ_ERR_ALIGN (-3)  /* a tensor pointer is not 16-byte aligned       */
#define HQ_ERR_MODE (-4)   /* mode or option combination not allowed        */
#define HQ_ERR_DEVICE (-5) /* current device is not gfx950 / HIP error      */
#define HQ_ERR_LAUNCH (-6) /* a kernel launch failed                        */

/* OR'ed into the mode of hq_dense_gemm, hq_batch_gemm, hq_group_contiguous_gemm,
 * hq_group_contiguous_gemm_ptr_array and hq_group_masked_gemm: out holds IEEE
 * binary16 (FP16) values, each rounded to nearest even from the FP32 result
 * (+ bias, x alpha; Inf beyond 65504), instead of BF16 (the flashrt/fp4-gemm
 * page's *_fp16 GEMMs).  bias stays BF16. */
#define HQ_OUT_FP16 0x100

/* hq_group_wise_quant flags */
#define HQ_GS_INPUT 1u /* NVFP4: read the global scale from *global_scale   */
#define HQ_IN_FP16 2u  /* x holds IEEE binary16 (FP16) patterns, not BF16  */

/* Thread-local description of the last error of this thread ("" if none). */
const char* hq_last_error(void);

/*
 * Group-wise quantisation of BF16 or FP16 rows (HALOps "GEMM" page,
 * group_wise_quant section; here always with the plain row-major scale
 * layout).
 *
 *   x   [m, k] BF16, or FP16 with flags & HQ_IN_FP16   (input)
 *   q   [m, k] (MXFP8) or [m, k/2] (FP4)    (output codes)
 *   sf  [m, k/gs]                           (output scales)
 *
 * MX modes: per row and 32-group, s = clamp(floor(log2 amax) - emax, -127,
 * 127) with emax = 8 (E4M3) or 2 (E2M1); sf = s + 127; code = nearest element
 * of x / 2^s, ties to even, saturating to +-448 / +-6, sign kept (also for
 * zero).  global_scale must be NULL and flags 0 or HQ_IN_FP16.
 *
 * NVFP4: g = amax(x) / 2688 in FP32 (1 if amax == 0), or *global_scale when
 * flags & HQ_GS_INPUT.  Per 16-group: sf = UE4M3(amax_b / (6 g)), then
 * code = E2M1(x / (decode(sf) * g)), each division an IEEE FP32 operation
 * rounded to nearest even (code = +-0 when decode(sf) * g == 0).
 * global_scale (device float[1]) is required: read when HQ_GS_INPUT is set,
 * otherwise computed and written (the call then enqueues an amax pass, which
 * uses the start of q as scratch before the codes overwrite it: x, q, sf and
 * global_scale must not overlap).
 * Inputs convert exactly to FP32 (both formats); the rules above then apply
 * to those values.
 */
hq_status hq_group_wise_quant(void* stream, int32_t mode, const uint16_t* x,
                              int64_t m, int64_t k, uint8_t* q, uint8_t* sf,
                              float* global_scale, uint32_t flags);

/*
 * Dense scaled GEMM (HALOps "GEMM" page, dense_gemm section):
 *   out[m, n] = bf16( alpha * sum_k deq(a)[m, k] * deq(b)[n, k] + bias[n] )
 *   a [m, K'] + sfa [m, k/gs];  b [n, K'] + sfb [n, k/gs];  out [m, n] BF16.
 * bias [n] (BF16) is accepted only in MXFP8 mode (else must be NULL).
 * alpha (device float[1]) is required in NVFP4 mode and rejected otherwise.
 * Accumulation is FP32 on the matrix cores; the output is rounded once to
 * BF16 (nearest even).  cu_limit > 0 caps the compute units used (<= 0: all).
 * Every K step of a tile runs in one workgroup (no K split, no workspace);
 * hq_dense_gemm_ws is the same call with a caller-owned workspace that lets
 * K be split where the tiles cannot fill the chip.
 */
hq_status hq_dense_gemm(void* stream, int32_t mode, const uint8_t* a,
                        const uint8_t* sfa, const uint8_t* b,
                        const uint8_t* sfb, const uint16_t* bias,
                        const float* alpha, uint16_t* out, int64_t m,
                        int64_t n, int64_t k, int32_t cu_limit);

/*
 * hq_dense_gemm with a caller-owned FP32 workspace (the flashrt/fp4-gemm
 * page's large-M tier: the workspace is allocated by the caller, before any
 * graph capture, and passed on every call).  hq_gemm_workspace_size gives
 * the bytes this shape uses; when workspace_bytes holds them the call may
 * split K.  The first 16 KB of the workspace hold 64-bit flag words of the
 * stream-K form; the FP32 partials of every form follow them.
 *  - when the output tiles cannot fill half of the compute units and K is
 *    long (at least 8 K steps of 128 bytes per row), K is cut into 2..8
 *    contiguous slices: each slice's FP32 partial products go to the
 *    workspace (slices * m * n floats), a second kernel adds the slices in
 *    order and applies bias / alpha, then rounds once to BF16.  Taken where
 *    the matrix time saved outweighs the partial planes' memory traffic;
 *  - when the tiles fill whole rounds of the compute units and leave a last
 *    round at most half full, and K is long (at least 48 MXFP8, 40 MXFP4 or
 *    12 NVFP4 steps), the last round's tiles -- whole 256-column tiles of the
 *    last 1024 rows or fewer -- are computed the same way, after the others,
 *    with slices * rows * columns floats of that rectangle;
 *  - stream-K: when the tiles make one round of more than a third of the
 *    compute units and the matrix time saved pays for the hand-off (long K,
 *    or NVFP4), the K steps of all tiles are dealt out in equal runs, one
 *    per workgroup (in 8 groups -- every eighth workgroup, one XCD's share
 *    under the round-robin dispatch -- each taking an eighth of the tiles),
 *    and each tile's pieces hand their FP32 partial tiles to its last
 *    piece, which writes the output (two 256 KB partial tiles per
 *    workgroup).  A piece waits only for workgroups of lower index,
 *    dispatched before it (in index order), which hand their partial on
 *    before they wait for
 *    anything, so the waits end whether or not the launch's workgroups are
 *    all resident at once; a wait that still finds no partial after about a
 *    second (a fault elsewhere) gives up and sets the last flag word instead
 *    of hanging.
 * With a NULL workspace, or fewer bytes than the shape uses, the call runs
 * unsplit (as hq_dense_gemm).  A split changes the FP32 summation order, not
 * the result's contract.  The workspace is scratch: its contents before the
 * call do not change the result (the stream-K flags carry a value of the
 * call's own and are cleared by the call), and two calls in flight at once
 * (on two streams) need two workspaces.  It must be 16-byte aligned
 * (HQ_ERR_NULL for a NULL workspace with workspace_bytes > 0).
 */
hq_status hq_dense_gemm_ws(void* stream, int32_t mode, const uint8_t* a,
                           const uint8_t* sfa, const uint8_t* b,
                           const uint8_t* sfb, const uint16_t* bias,
                           const float* alpha, uint16_t* out, int64_t m,
                           int64_t n, int64_t k, int32_t cu_limit,
                           void* workspace, uint64_t workspace_bytes);

/*
 * hq_dense_gemm_ws for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * K-split workspace is the library's own scratch array of HQ_SCRATCH_BYTES
 * per GPU (a static device array, resolved once per device on first use and
 * held until the process ends); the call allocates nothing.  Same arguments,
 * result and split plan as hq_dense_gemm_ws given a workspace of
 * HQ_SCRATCH_BYTES.  A shape whose K-split plan needs more than
 * HQ_SCRATCH_BYTES (hq_gemm_workspace_size) is refused with HQ_ERR_SHAPE
 * before any launch; a stream-K plan that does not fit is not taken (the
 * call runs unsplit).
 * Every call on one GPU uses the same scratch: calls that may overlap on a
 * GPU (several streams, several host threads) race and must be serialised
 * by the caller; a call's scratch contents are meaningless afterwards.
 */
#define HQ_SCRATCH_BYTES (32u << 20)
hq_status hq_dense_gemm_scratch(void* stream, int32_t mode, const uint8_t* a,
                                const uint8_t* sfa, const uint8_t* b,
                                const uint8_t* sfb, const uint16_t* bias,
                                const float* alpha, uint16_t* out, int64_t m,
                                int64_t n, int64_t k, int32_t cu_limit);

/*
 * Workspace bytes that hq_dense_gemm_ws (batch == 1) or hq_batch_gemm_ws
 * (batch items of m x n) uses for this shape, mode and cu_limit on the
 * current device, written to *bytes; 0 when the shape never splits.  A host
 * query (device properties only): nothing is launched.  Shape and mode
 * errors as for the GEMM calls; HQ_ERR_DEVICE off gfx950.
 */
hq_status hq_gemm_workspace_size(int32_t mode, int64_t batch, int64_t m,
                                 int64_t n, int64_t k, int32_t cu_limit,
                                 uint64_t* bytes);

/*
 * Batch GEMM (HALOps "GEMM" page, batch_gemm section): for every batch item
 * b, out[b] = a[b] * w[b]^T, with bias[b] / alpha[b].
 *   a [batch, m, K'], sfa [batch, m, k/gs], b [batch, n, K'],
 *   sfb [batch, n, k/gs], bias [batch, n], alpha [batch], out [batch, m, n].
 */
hq_status hq_batch_gemm(void* stream, int32_t mode, const uint8_t* a,
                        const uint8_t* sfa, const uint8_t* b,
                        const uint8_t* sfb, const uint16_t* bias,
                        const float* alpha, uint16_t* out, int64_t batch,
                        int64_t m, int64_t n, int64_t k, int32_t cu_limit);

/* hq_batch_gemm with a caller-owned workspace: the K split of
 * hq_dense_gemm_ws (its first form: few tiles, long K) over all batch items,
 * slices * batch * m * n floats; same workspace rules. */
hq_status hq_batch_gemm_ws(void* stream, int32_t mode, const uint8_t* a,
                           const uint8_t* sfa, const uint8_t* b,
                           const uint8_t* sfb, const uint16_t* bias,
                           const float* alpha, uint16_t* out, int64_t batch,
                           int64_t m, int64_t n, int64_t k, int32_t cu_limit,
                           void* workspace, uint64_t workspace_bytes);

/*
 * Grouped-contiguous GEMM (HALOps "GEMM" page, group_contiguous_gemm section;
 * cuDNN FE "Grouped GEMM + dGLU (SM100)", Step 1): group g owns rows
 * [group_end[g-1], group_end[g]) of a (group_end[-1] = 0) and uses
 * b[g] / sfb[g] / bias[g] / alpha[g].
 *   a [m_total, K'], sfa [m_total, k/gs], b [num_groups, n, K'],
 *   sfb [num_groups, n, k/gs], group_end [num_groups] int32 (device,
 *   cumulative ends, non-decreasing), bias [num_groups, n],
 *   alpha [num_groups], out [m_total, n].
 * Any group size (including 0) is allowed.  Rows at or beyond the last end
 * are not written.  A row map of sorted per-row expert ids converts to
 * group_end[g] = number of rows with id <= g.
 */
hq_status hq_group_contiguous_gemm(void* stream, int32_t mode,
                                   const uint8_t* a, const uint8_t* sfa,
                                   const uint8_t* b, const uint8_t* sfb,
                                   const int32_t* group_end,
                                   int32_t num_groups, const uint16_t* bias,
                                   const float* alpha, uint16_t* out,
                                   int64_t m_total, int64_t n, int64_t k,
                                   int32_t cu_limit);

/*
 * Grouped-contiguous GEMM with discrete expert weights (cuDNN FE "Grouped GEMM
 * + dGLU (SM100)" page, the discrete b_ptrs form of its B operand): as
 * hq_group_contiguous_gemm, but group g's weights live in their own
 * allocations.
 *   b_ptrs [num_groups], sfb_ptrs [num_groups]: device arrays of 64-bit
 *   device addresses; b_ptrs[g] points to group g's [n, K'] codes and
 *   sfb_ptrs[g] to its [n, k/gs] scales (row-major, as b[g] / sfb[g] of
 *   hq_group_contiguous_gemm).  Every code address must be 16-byte aligned
 *   and every scale address 16-byte aligned (device data: not checked).
 *   Other arguments and the result as for hq_group_contiguous_gemm; the
 *   arrays and what they point to are read on the stream, so they must stay
 *   alive and unchanged until the call's work has run.
 */
hq_status hq_group_contiguous_gemm_ptr_array(void* stream, int32_t mode,
                                             const uint8_t* a, const uint8_t* sfa,
                                             const uint64_t* b_ptrs,
                                             const uint64_t* sfb_ptrs,
                                             const int32_t* group_end,
                                             int32_t num_groups, const uint16_t* bias,
                                             const float* alpha, uint16_t* out,
                                             int64_t m_total, int64_t n, int64_t k,
                                             int32_t cu_limit);

/*
 * Grouped-contiguous gate|up GEMM with the SwiGLU + re-quantisation applied in
 * its epilogue (HALOps "GEMM" page, group_contiguous_gemm and
 * fused_swiglu_quant sections; the flashrt/fp4-gemm page's fused GEMM
 * epilogues).  The result is that of hq_group_contiguous_gemm into a BF16
 * [m_total, 2h] x = [gate | up] followed by hq_fused_swiglu_quant(MXFP8,
 * group_end, valid) on x -- the same codes and scales, bit for bit (x's BF16
 * rounding included) -- without writing or reading x.
 *   mode must be HQ_MXFP8.  a [m_total, k], sfa [m_total, k/32],
 *   b [num_groups, 2h, k] (rows [0, h) gate, [h, 2h) up), sfb
 *   [num_groups, 2h, k/32], group_end [num_groups] int32 (device, as for
 *   hq_group_contiguous_gemm), valid (optional, device int32 [num_groups]:
 *   only the first min(valid[g], size) rows of group g are written),
 *   bias (optional) [num_groups, 2h] BF16, q [m_total, h] E4M3 codes,
 *   sf [m_total, h/32] UE8M0, y_debug (optional, device float [m_total, h]):
 *   the FP32 y of the written rows.
 *   h % 128 == 0 (h <= 2^20); k % 128 == 0 and k >= 256 (the tiled kernel's
 *   K step and two steps); (h + 256) * k < 2^31; sfa / sfb 4-byte aligned.
 * Rows not written keep their contents.  No workspace is used.
 */
hq_status hq_group_contiguous_gemm_swiglu_quant(void* stream, int32_t mode,
                                                const uint8_t* a, const uint8_t* sfa,
                                                const uint8_t* b, const uint8_t* sfb,
                                                const int32_t* group_end,
                                                int32_t num_groups, const int32_t* valid,
                                                const uint16_t* bias, uint8_t* q,
                                                uint8_t* sf, float* y_debug,
                                                int64_t m_total, int64_t h, int64_t k,
                                                int32_t cu_limit);

/*
 * Backward block-scaled grouped GEMM with the dSwiGLU epilogue (cuDNN FE
 * "Grouped GEMM + dGLU (SM100)": the compact-gradient equation
 * R_g = alpha_g^2 A_g B_g^T, X_g = beta_g C_g; Step 1, the block-scaled
 * grouped GEMM; Step 2, the dGLU epilogue for dSwiGLU).  For every row m of
 * group g (rows [group_end[g-1], group_end[g]), as hq_group_contiguous_gemm)
 * and R column n = 32 j + t, with input = X[m, 64 j + t],
 * gate = X[m, 64 j + 32 + t], s = sigmoid(gate), swish = gate s:
 *   d[m, 64 j + t]      = R[m, n] prob[m] swish
 *   d[m, 64 j + 32 + t] = R[m, n] prob[m] input s (1 + gate (1 - s))
 *   dprob[m]           += sum over n of swish input R[m, n]
 * in FP32, d rounded once to BF16.
 *   mode HQ_MXFP8 or HQ_MXFP4; a [m_total, K'], sfa [m_total, k/32] (the
 *   upstream gradient, quantised); b [num_groups, n, K'], sfb
 *   [num_groups, n, k/32] (each expert's weights, K-major);
 *   group_end [num_groups] int32 (device, cumulative ends);
 *   c [m_total, 2n] BF16: the forward activations, alternating 32-column
 *   blocks of the input and the gate half (input block first);
 *   alpha, beta [num_groups] FP32 (optional: NULL means 1);
 *   prob [m_total] FP32 routing probabilities; dprob [m_total] FP32,
 *   accumulated (+=; zero it for a plain gradient; the adds of one row come
 *   from several workgroups, so their FP32 order is not fixed);
 *   d [m_total, 2n] BF16 output.
 * n % 32 == 0, n * 1024 < 2^31; k a multiple of the tiled K step (128 MXFP8,
 * 256 MXFP4), at least two steps; a, b, c, d 16-byte aligned; sfa, sfb, prob,
 * dprob 4-byte aligned.  Rows at or past the last end are not written (d
 * nor dprob).  No workspace is used.
 */
hq_status hq_group_contiguous_gemm_dswiglu(void* stream, int32_t mode,
                                           const uint8_t* a, const uint8_t* sfa,
                                           const uint8_t* b, const uint8_t* sfb,
                                           const int32_t* group_end,
                                           int32_t num_groups, const uint16_t* c,
                                           const float* alpha, const float* beta,
                                           const float* prob, float* dprob,
                                           uint16_t* d, int64_t m_total, int64_t n,
                                           int64_t k, int32_t cu_limit);

/*
 * hq_group_contiguous_gemm_dswiglu with a row-quantised D (the same page's
 * optional output quantisation, Step 3, read with this library's MXFP8
 * rule): instead of BF16 d, every row's 32-column blocks of D (one input or
 * gate block each) are quantised from their BF16 values exactly as
 * hq_group_wise_quant(HQ_MXFP8) quantises BF16 rows -- per block a UE8M0
 * scale s = clamp(floor(log2 amax) - 8, -127, 127) and E4M3 codes of
 * D / 2^s (nearest even, saturating).  So dq / dsf equal hq_group_wise_quant
 * applied to the d of hq_group_contiguous_gemm_dswiglu.  (The page's own FP8
 * recipe, a normalisation constant times the block amax times a reciprocal
 * maximum with 128x4 scale atoms, is not implemented.)
 *   dq [m_total, 2n] u8 E4M3 codes (16-byte aligned); dsf [m_total, 2n / 32]
 *   u8 UE8M0 scales; every other argument as hq_group_contiguous_gemm_dswiglu.
 * Rows at or past the last end are not written (dq, dsf nor dprob).  No
 * workspace is used.
 */
hq_status hq_group_contiguous_gemm_dswiglu_quant(void* stream, int32_t mode,
                                                 const uint8_t* a, const uint8_t* sfa,
                                                 const uint8_t* b, const uint8_t* sfb,
                                                 const int32_t* group_end,
                                                 int32_t num_groups, const uint16_t* c,
                                                 const float* alpha, const float* beta,
                                                 const float* prob, float* dprob,
                                                 uint8_t* dq, uint8_t* dsf,
                                                 int64_t m_total, int64_t n, int64_t k,
                                                 int32_t cu_limit);

/*
 * Grouped-masked GEMM (HALOps "GEMM" page, group_masked_gemm section): expert
 * e owns the slot of rows [e * max_m, (e + 1) * max_m); only its first
 * min(masked_m[e], max_m) rows are computed and written (padded rows are
 * neither read into a valid output nor written).
 *   a [num_groups * max_m, K'], sfa [num_groups * max_m, k/gs],
 *   b [num_groups, n, K'], sfb [num_groups, n, k/gs],
 *   masked_m [num_groups] int32 (device), bias [num_groups, n],
 *   alpha [num_groups], out [num_groups * max_m, n].  max_m > 0.
 */
hq_status hq_group_masked_gemm(void* stream, int32_t mode, const uint8_t* a,
                               const uint8_t* sfa, const uint8_t* b,
                               const uint8_t* sfb, const int32_t* masked_m,
                               int32_t num_groups, int64_t max_m_per_group,
                               const uint16_t* bias, const float* alpha,
                               uint16_t* out, int64_t n, int64_t k,
                               int32_t cu_limit);

/*
 * Fused SwiGLU + re-quantisation (HALOps "GEMM" page, fused_swiglu_quant
 * section): x [rows, 2h] BF16 is [gate | up]; y = up * gate / (1 + exp(-gate))
 * in FP32 (no intermediate BF16 rounding), then y is quantised group-wise in
 * `mode` exactly as hq_group_wise_quant does (NVFP4: the global scale is read
 * from *global_scale, which is then required).
 *   q [rows, h] (MXFP8) or [rows, h/2]; sf [rows, h/gs].
 * Row selection: if group_end (device int32 [num_groups]) is given, group g
 * spans [group_end[g-1], group_end[g]); otherwise group g spans
 * [g * slot_rows, (g + 1) * slot_rows).  If valid (device int32
 * [num_groups]) is given only the first min(valid[g], size) rows of each
 * group are processed, otherwise all of them.  Other rows are not written.
 * y_debug (optional, device float [rows, h]) receives the FP32 y of the
 * processed rows: the codes are then exactly the quantisation of y_debug.
 */
hq_status hq_fused_swiglu_quant(void* stream, int32_t mode, const uint16_t* x,
                                int64_t rows, int64_t h, int32_t num_groups,
                                const int32_t* group_end, int64_t slot_rows,
                                const int32_t* valid, uint8_t* q, uint8_t* sf,
                                const float* global_scale, float* y_debug);

/*
 * Token permute into the masked-GEMM layout (HALOps "GEMM" page,
 * prefill_permute_to_masked_gemm section).  For every (token t, slot j)
 * whose expert id e = topk_ids[t, j] lies in [0, num_experts), the token's
 * row is copied to the next free row r of expert e's slot:
 *   permute_x[e * max_token_num + r]  = x[t]          (row_bytes bytes)
 *   out_scale[e, r, :]                = per-32 scales of token t
 *   indice_map[t, j]                  = r
 * and token_nums[e] ends as the number of rows written to expert e.
 *   x           [num_tokens, row_bytes] (FP8 codes, BF16 values or packed
 *               FP4 codes: copied bit for bit; row_bytes % 16 == 0)
 *   scale       HQ_SCALE_BROADCAST: int32 [num_tokens, hidden/512], byte b
 *               (little-endian) of word w = scale of the 128-group 4w + b,
 *               given to its four 32-groups (hidden % 512 == 0);
 *               HQ_SCALE_DIRECT: uint8 [num_tokens, hidden/32] per-32 bytes
 *               (hidden % 128 == 0)
 *   topk_ids    int64 [num_tokens, topk], 1 <= topk <= 64; ids outside
 *               [0, num_experts) (e.g. -1) are unassigned: map -1
 *   permute_x   [num_experts * max_token_num, row_bytes]; rows past an
 *               expert's count are not written
 *   out_scale   uint8 [num_experts, max_token_num, hidden/32], plain
 *               row-major (the scale layout the masked GEMM takes)
 *   indice_map  int32 [num_tokens, topk];  token_nums  int32 [num_experts]
 * max_token_num must be a positive multiple of 128.  Pairs beyond
 * max_token_num for one expert are dropped (map -1; the section's kernel
 * would write past the slot).  The order of rows inside an expert is not
 * fixed (it follows atomic arrival); the set of rows, their contents, the
 * counts and the map's consistency are.  x, permute_x 16-byte aligned;
 * scale, out_scale 4-byte aligned.
 */
#define HQ_SCALE_BROADCAST 0
#define HQ_SCALE_DIRECT 1
hq_status hq_prefill_permute_to_masked_gemm(void* stream, const uint8_t* x, int64_t num_tokens,
                                            int64_t row_bytes, int64_t hidden, const void* scale,
                                            int32_t scale_mode, const int64_t* topk_ids,
                                            int32_t topk, int32_t num_experts,
                                            int64_t max_token_num, uint8_t* permute_x,
                                            uint8_t* out_scale, int32_t* indice_map,
                                            int32_t* token_nums);

#ifdef __cplusplus
}
#endif

#endif /* HQ_H_ */
