/*
 * qgemm.h -- C ABI of libqgemm.so: the batched prefill projection matmul over
 * GGUF Q4_K / Q6_K weights on AMD Instinct MI355X (gfx950).
 *
 * Operation.  y[M x N] = x[M x K] . W[N x K]^T where W stays in its GGUF
 * super-blocks and x is a whole prompt's activation rows.  The weights are
 * decoded to small integers on the GPU, every activation row is quantised to
 * int8 per 32 consecutive values (one fp32 scale d = amax/127 and the int32 sum
 * of the codes per block), the contraction is int8 x int8 -> int32 on the
 * matrix cores, and each weight sub-block's scale and min are applied to the
 * int32 partial in fp32.  This is the fused "decode super-blocks in registers,
 * int8 tensor-core GEMM" design of sparkinfer PR #464 ("fused Q4K/Q6K->int8
 * dequant ...", section "Summary") and the "row-batched fused Q4_K x int8
 * kernel" branch of the design question in aprender issue #5475 ("Qwen3.5 on
 * CPU prefills one token at a time", section "Ask"); the activation block is
 * the q8_1-style per-32 block that issue #4220 ("CRUX parity spike ...",
 * technique 5) names for the quantised-activation GEMV.  The LM-head entry is
 * the "LM head on the last token only" of aprender issue #5305 (sub-ticket
 * #4313).
 *
 * Block layouts (public GGUF K-quant format; little-endian, binary16 scales):
 *   Q4_K: 144 bytes per 256 values -- d, dmin, 12 bytes of packed 6-bit
 *         sub-block scales/mins (8 sub-blocks of 32), 128 bytes of 4-bit codes;
 *         w = d*sc*q - dmin*m.
 *   Q6_K: 210 bytes per 256 values -- ql[128], qh[64], 16 int8 scales (16
 *         sub-blocks of 16), d; w = d*sc*(q6 - 32).
 *   Q5_K: 176 bytes per 256 values -- the 16-byte Q4_K header, qh[32] (bit v/32
 *         of qh[v % 32] is the fifth bit of value v), 128 bytes of low nibbles
 *         placed as Q4_K's codes; w = d*sc*q5 - dmin*m, q5 in [0, 31].  The
 *         format aprender issue #5305's decode-GEMV ticket #5221 finds slowest;
 *         it runs through the Q4_K kernels (tiled, small-grid, skinny) with the
 *         fifth bit or-ed into the codes.
 *   Q8_0: 34 bytes per 32 values -- d, then 32 int8 codes; w = d*q (named on
 *         aprender issue #5475's page among the formats its CPU path runs row
 *         by row).  K is still a multiple of 256 (a row is K/32 blocks).  The
 *         codes go to the matrix core as they are, with d as the block scale
 *         and no min term; the skinny kernel takes it for M <= 8.
 * The per-256 entry points take Q4_K only and the fp16-branch ones Q4_K /
 * Q6_K (QG_EFMT for Q5_K and Q8_0).
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers owned by the caller.  The library
 *     allocates nothing, keeps no pointer after returning and has no mutable
 *     global state.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is only enqueued; return value 0 means "enqueued".  The caller
 *     synchronises.  Calls on different streams may run concurrently if they
 *     use different workspaces.
 *   - Errors are negative return codes (see QG_E*); on error nothing is
 *     launched, except QG_ELAUNCH, which reports a launch failure after the
 *     fact.  No C++ exception crosses this boundary.
 *   - Non-finite activations or weight scales are a precondition violation;
 *     the results are then unspecified.
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* weight formats */
enum { QG_Q4_K = 0, QG_Q6_K = 1, QG_Q5_K = 2, QG_Q8_0 = 3 };
/* activation element types: IEEE binary32, or bfloat16 (raw 16-bit patterns) */
enum { QG_F32 = 0, QG_BF16 = 1 };
/* kernel path selection for qgemm_prefill_ex */
enum { QG_PATH_AUTO = 0, QG_PATH_TILED = 1, QG_PATH_SKINNY = 2 };
/* return codes */
enum {
    QG_OK = 0,
    QG_EINVAL = -1,     /* null pointer, M/N/K < 1, K % 256 != 0, size overflow, bad path */
    QG_EFMT = -2,       /* fmt not QG_Q4_K / QG_Q5_K / QG_Q6_K / QG_Q8_0, or not one the entry point takes */
    QG_EDTYPE = -3,     /* x_dtype not QG_F32 / QG_BF16 */
    QG_EWORKSPACE = -4, /* workspace NULL, smaller than qgemm_workspace_bytes, or not 256-B aligned */
    QG_EALIGN = -5,     /* q_weights not 16-B aligned, x not aligned to 16 B, y not 16-B aligned */
    QG_ELAUNCH = -6,    /* the HIP runtime reported a launch error */
    QG_EDEVICE = -7,    /* the current device is not a gfx950 GPU */
    QG_ENOSCRATCH = -8  /* qgemm_prefill_noalloc: the problem's workspace exceeds the static scratch */
};

/* Largest skinny-path batch.  Under QG_PATH_AUTO, Q6_K and Q8_0 problems with
 * M <= QG_SKINNY_MAX_M rows go to the bandwidth-bound skinny kernel, and Q4_K
 * and Q5_K problems with M <= m(N, K) rows: m = 8 for N <= 1024; for K <= 1024,
 * 4 when N <= 4096 and 2 above; otherwise 6 when N <= 12288 and 4 above.  Larger
 * M go to the tiled matrix-core kernels (the small-grid one for M <= 8). */
#define QG_SKINNY_MAX_M 8

/* Workspace bytes needed by qgemm_prefill / qgemm_lm_head for M activation rows
 * of length K (int8 codes, per-block fp32 scales and scaled block sums).
 * Rows are padded to a multiple of 256: the tiled kernels read whole row tiles
 * (up to 128 rows) of the scale arrays, and a problem of any M, M <= 8
 * included, may be sent down the tiled path (QG_PATH_TILED), while the
 * workspace is sized before the path is known.  For one row at K = 4096 the
 * padding costs 1.6 MB of workspace, against the LM head's 511 MB of weights.
 * Returns 0 when M < 1, K < 1, K % 256 != 0 or the size overflows. */
size_t qgemm_workspace_bytes(int64_t M, int64_t K);

/* y[m][n] = sum_k x[m][k] * W[n][k] under the method's quantisation.
 *   q_weights : GGUF tensor data of a 2-D weight with K contiguous: row n holds
 *               K/256 consecutive blocks starting at byte n*(K/256)*bytes_per_block.
 *               Must be 16-byte aligned.
 *   fmt       : QG_Q4_K, QG_Q6_K, QG_Q5_K or QG_Q8_0 (block layouts above).
 *   x         : activations [M][K] row-major, element type x_dtype, 16-byte aligned.
 *   M, N, K   : M, N >= 1; K >= 256 and K % 256 == 0.
 *   y         : output [M][N] fp32 row-major (leading dimension N), overwritten.
 *               Must be 16-byte aligned.
 *   workspace : device scratch of at least qgemm_workspace_bytes(M, K) bytes,
 *               256-byte aligned; its contents are scratch on entry and exit.
 *   stream    : hipStream_t (NULL = default stream).
 * Dispatch: the skinny kernel for M <= QG_SKINNY_MAX_M (Q6_K, Q8_0) or M <= m(N, K)
 * (Q4_K, Q5_K; m as given at QG_SKINNY_MAX_M), otherwise the tiled kernels. */
int qgemm_prefill(const void *q_weights, int fmt, const void *x, int x_dtype, int64_t M,
                  int64_t N, int64_t K, float *y, void *workspace, size_t workspace_bytes,
                  void *stream);

/* qgemm_prefill with an explicit kernel path (QG_PATH_AUTO / _TILED / _SKINNY).
 * QG_PATH_SKINNY requires M <= QG_SKINNY_MAX_M (else QG_EINVAL).  Both paths
 * compute the same quantities; they differ only in fp32 summation order. */
int qgemm_prefill_ex(const void *q_weights, int fmt, const void *x, int x_dtype, int64_t M,
                     int64_t N, int64_t K, float *y, void *workspace, size_t workspace_bytes,
                     void *stream, int path);

/* LM head on the last token only: qgemm_prefill with M = 1.  x_row points at the
 * one activation row [K]; y receives [N] logits. */
int qgemm_lm_head(const void *q_weights, int fmt, const void *x_row, int x_dtype, int64_t N,
                  int64_t K, float *y, void *workspace, size_t workspace_bytes, void *stream);

/* The two halves of qgemm_prefill, for callers that feed one activation matrix
 * to several projections (the fused QKV and gate/up projections of a layer
 * read the same hidden rows): quantise once, then run one GEMM per weight.
 *
 * qgemm_quantize_workspace: quantise x [M][K] into `workspace` (layout private
 * to the library, sized by qgemm_workspace_bytes(M, K)).
 * qgemm_gemm_quantized: y = x . W^T from a workspace filled by
 * qgemm_quantize_workspace with the same M and K (and not modified since);
 * path as in qgemm_prefill_ex.  Argument rules and codes as qgemm_prefill. */
int qgemm_quantize_workspace(const void *x, int x_dtype, int64_t M, int64_t K, void *workspace,
                             size_t workspace_bytes, void *stream);
int qgemm_gemm_quantized(const void *q_weights, int fmt, const void *workspace,
                         size_t workspace_bytes, int64_t M, int64_t N, int64_t K, float *y,
                         void *stream, int path);

/* Name of the GPU kernel qgemm_gemm_quantized would launch for this problem
 * and path, as a profiler lists it (template arguments included); for
 * benchmarks and profiles.  The string stays valid until the next call from
 * the same thread.  NULL when the arguments would be rejected.  Launches
 * nothing and needs no GPU. */
const char *qgemm_kernel_name(int fmt, int64_t M, int64_t N, int64_t K, int path);

/* Static message for a return code (never NULL). */
const char *qgemm_strerror(int code);

/* ---- test hooks: the comparison points for bit-exact parity ---- */

/* Activation quantiser alone: q [M][K] int8, d [M][K/32] fp32, S [M][K/32] int32
 * (row-major).  d = amax/127 (IEEE division), codes rint(x * (1/d)) ties to even
 * clamped to [-127, 127], code 0 where x == 0, S = sum of the block's codes;
 * an all-zero block gives d = 0.  K % 32 == 0 is required here. */
int qgemm_quantize_act(const void *x, int x_dtype, int64_t M, int64_t K, int8_t *q, float *d,
                       int32_t *S, void *stream);

/* Decoded weights w [N][K] fp32, each the correctly rounded fp32 value of
 * d*sc*q - dmin*m (Q4_K; Q5_K with q5), d*sc*(q6 - 32) (Q6_K) or d*q (Q8_0). */
int qgemm_dequant(const void *q_weights, int fmt, int64_t N, int64_t K, float *w, void *stream);

/* Per-block int32 partials computed by the tiled kernel's own decode and matrix
 * instructions: Q4_K out[m][n][b] = sum_{t<32} q[n][32b+t] * qx[m][32b+t]
 * (K/32 per pair, q in 0..15; Q5_K the same with q5 in 0..31; Q8_0 with the
 * int8 codes); Q6_K out[m][n][s] = sum_{t<16} (q6[n][16s+t] - 32)
 * * qx[m][16s+t] (K/16 per pair).  qx is int8 [M][K]; out has M*N*K/32 (Q4_K,
 * Q5_K, Q8_0) or M*N*K/16 (Q6_K) elements.  Meant for small shapes. */
int qgemm_block_partials(const void *q_weights, int fmt, const int8_t *qx, int64_t M, int64_t N,
                         int64_t K, int32_t *out, void *stream);

/* ---- per-256 activation scales (Q4_K) ----
 *
 * The activation block the same issue pairs with Q4_K ("Q4_K x Q8_K", aprender
 * issue #5475, section "Ask", item 1): one fp32 scale per 256-value super-block
 * instead of per 32 values, with the code sums kept per 32-value sub-block.
 * The quantiser takes the steps of qgemm_quantize_act over each super-block
 * (d = amax/127, codes rint(x * (1/d)) ties to even clamped to [-127, 127],
 * code 0 where x == 0); the GEMM computes
 *   y[m][n] = sum_sb dx[sb] * sum_j ( d*sc[j]*I[j] - dmin*m[j]*S[j] )
 * with exact int32 sub-block partials I[j] -- a different (coarser) activation
 * encoding than the per-32 entry points, not their result.  Q4_K only
 * (QG_EFMT otherwise).  The workspace is sized by qgemm_workspace_bytes; its
 * layout is the per-32 one with every 32-value block holding its super-block's
 * scale, which lets the tiled kernels combine a super-block's eight partials
 * in integers and apply the fp32 scales once per super-block. */

/* Quantise x [M][K] per 256 values into `workspace` (argument rules and codes
 * as qgemm_quantize_workspace). */
int qgemm_quantize_workspace_a256(const void *x, int x_dtype, int64_t M, int64_t K,
                                  void *workspace, size_t workspace_bytes, void *stream);
/* y = x . W^T from a workspace filled by qgemm_quantize_workspace_a256 with the
 * same M and K (argument rules and codes as qgemm_gemm_quantized, path AUTO). */
int qgemm_gemm_quantized_a256(const void *q_weights, int fmt, const void *workspace,
                              size_t workspace_bytes, int64_t M, int64_t N, int64_t K, float *y,
                              void *stream);
/* The two above in one call (argument rules and codes as qgemm_prefill). */
int qgemm_prefill_a256(const void *q_weights, int fmt, const void *x, int x_dtype, int64_t M,
                       int64_t N, int64_t K, float *y, void *workspace, size_t workspace_bytes,
                       void *stream);
/* Name of the GEMM kernel qgemm_gemm_quantized_a256 launches, or NULL. */
const char *qgemm_kernel_name_a256(int fmt, int64_t M, int64_t N, int64_t K);
/* Test hook: the per-256 quantiser alone.  q [M][K] int8, d [M][K/256] fp32,
 * S [M][K/32] int32 (sub-block code sums); K % 256 == 0. */
int qgemm_quantize_act_a256(const void *x, int x_dtype, int64_t M, int64_t K, int8_t *q, float *d,
                            int32_t *S, void *stream);

/* ---- the other design branch: dequantise to binary16, float matrix-core GEMM ----
 *
 * aprender issue #5475 ("apr serve / apr run: Qwen3.5 on CPU prefills one token
 * at a time ..."), section "Ask", item 1, names two kernels for the batched
 * quantised matmul: dequantise a weight tile and call a float GEMM, or the
 * row-batched fused Q4_K x int8 kernel above.  These entry points are the first
 * branch, built to measure it beside the second; they compute a different
 * (fp16-rounded) result, not the int8 method's.  Each step rounds once, to
 * nearest even:
 *   x16 = f16(x)  (x as its fp32 value; bf16 widens exactly)
 *   per sub-block j: dsc = f16(d*sc[j]), dmn = f16(dmin*m[j]); w16 = f16(dsc*q - dmn)
 *   y[m][n] = sum_k x16[m][k] * w16[n][k], accumulated in fp32 on the matrix cores.
 * For Q6_K: dsc = f16(d*sc[s]) per 16-value sub-block, w16 = f16(dsc*(q6 - 32)).
 * Activations of magnitude 65520 and above become infinite in binary16, and
 * weights whose d*sc or dmin*m reach 65520 are outside the domain (results
 * unspecified). */

/* Workspace bytes for qgemm_prefill_deq_f16: the binary16 copy of x (M*K*2,
 * rounded up to 256).  0 when M < 1, K < 256, K % 256 != 0 or on overflow. */
size_t qgemm_deq_f16_workspace_bytes(int64_t M, int64_t K);

/* y[m][n] = sum_k x16[m][k] * w16[n][k] as above.  Arguments, alignment,
 * ownership and error codes as qgemm_prefill, with workspace sized by
 * qgemm_deq_f16_workspace_bytes.  Two launches: x -> binary16 into the
 * workspace, then the GEMM, which dequantises each weight tile in registers. */
int qgemm_prefill_deq_f16(const void *q_weights, int fmt, const void *x, int x_dtype, int64_t M,
                          int64_t N, int64_t K, float *y, void *workspace, size_t workspace_bytes,
                          void *stream);

/* Name of the GEMM kernel qgemm_prefill_deq_f16 launches (as a profiler lists
 * it), or NULL for arguments it would reject.  Needs no GPU. */
const char *qgemm_deq_f16_kernel_name(int fmt, int64_t M, int64_t N, int64_t K);

/* Test hooks of this branch.  qgemm_to_f16: x [M][K] -> binary16 bits x16 [M][K]
 * (K % 8 == 0; x and x16 16-byte aligned).  qgemm_dequant_f16: every weight of
 * W [N][K] as binary16 bits w16 [N][K] (16-byte aligned), through the GEMM's own
 * decoders.  A zero weight may be returned as -0. */
int qgemm_to_f16(const void *x, int x_dtype, int64_t M, int64_t K, uint16_t *x16, void *stream);
int qgemm_dequant_f16(const void *q_weights, int fmt, int64_t N, int64_t K, uint16_t *w16,
                      void *stream);

/* ---- fusions either side of the GEMM ----
 *
 * aprender issue #4220 ("CRUX parity spike: apr serve vs ollama"), table of the
 * techniques llama.cpp uses that apr lacks: technique 2 counts a layer's
 * per-token launches, its norms and its swiglu among them; technique 6 is the
 * norm fused with the multiply by its weight.  sparkinfer PR #464, section
 * "Summary": the cost removed is the projection path's scratch written and
 * read back.  Here the norm is fused into the activation quantiser (the
 * normalised row never reaches memory) and SwiGLU into the gate+up GEMM's
 * epilogue (the fp32 gate and up outputs never reach memory; h is written as
 * bfloat16, 2 bytes per value against 8 for the two fp32 outputs). */

/* RMSNorm of each row of x [M][K] with the fp32 weight g [K] and epsilon eps,
 * then the per-32 quantiser of qgemm_quantize_workspace, into `workspace`
 * (sized by qgemm_workspace_bytes(M, K)); qgemm_gemm_quantized and
 * qgemm_gemm_quantized_swiglu take the workspace as from that function.
 * Numerics (the standard RMSNorm; the pages print no formula):
 *   ss = sum_k x_k^2 in binary64 (each square exact), r = f32(1/sqrt(ss/K + eps))
 *   with binary64 steps, xn_k = f32(f32(x_k * r) * g_k), then the quantiser on xn.
 * The order of the binary64 sum is the kernel's; another order can change r
 * only where r lies within a few binary64 units of an fp32 rounding boundary.
 * Rules: 256 <= K <= 32768, K % 256 == 0; 1 <= M <= 2^31 - 1; eps finite and
 * >= 0 (QG_EINVAL otherwise); x and g 16-byte aligned (QG_EALIGN); other
 * arguments and codes as qgemm_quantize_workspace. */
int qgemm_rmsnorm_quantize_workspace(const void *x, int x_dtype, const float *g, float eps, int64_t M,
                                     int64_t K, void *workspace, size_t workspace_bytes, void *stream);
/* Test hook: the same into the layout of qgemm_quantize_act (q [M][K] int8,
 * d [M][K/32] fp32, S [M][K/32] int32). */
int qgemm_rmsnorm_quantize_act(const void *x, int x_dtype, const float *g, float eps, int64_t M,
                               int64_t K, int8_t *q, float *d, int32_t *S, void *stream);

/* SwiGLU over a gate+up projection.  q_weights holds 2F weight rows of length
 * K: the gate rows (0..F-1), then the up rows (F..2F-1), i.e. the two GGUF
 * tensors stacked.  With y = x . W^T under the method's quantisation ([M][2F]):
 *   h[m][f] = bf16( silu(y[m][f]) * y[m][F + f] ),  silu(z) = z / (1 + e^-z),
 * in fp32 from the fp32 GEMM result, rounded once to bfloat16 (nearest even).
 * h is bfloat16 bits [M][F], 16-byte aligned.  Q4_K, Q5_K and Q8_0 problems
 * on the tiled kernels run as ONE kernel (the gate and up columns of an output
 * tile are computed by paired waves and combined in LDS); decode-sized batches
 * (the skinny path), small grids and Q6_K weights run the plain GEMM into the
 * workspace, then a SwiGLU kernel. */

/* Workspace bytes for the SwiGLU entry points: the quantised activations and,
 * where the problem does not run fused, the fp32 [M][2F] GEMM output.  0 for a
 * bad format, M, F < 1, K < 256, K % 256 != 0 or on overflow. */
size_t qgemm_swiglu_workspace_bytes(int fmt, int64_t M, int64_t F, int64_t K);
/* h from a workspace filled by qgemm_quantize_workspace or
 * qgemm_rmsnorm_quantize_workspace with the same M and K (argument rules and
 * codes as qgemm_gemm_quantized with N = 2F, path AUTO; workspace sized by
 * qgemm_swiglu_workspace_bytes). */
int qgemm_gemm_quantized_swiglu(const void *q_weights, int fmt, const void *workspace,
                                size_t workspace_bytes, int64_t M, int64_t F, int64_t K, uint16_t *h,
                                void *stream);
/* Quantise x, then qgemm_gemm_quantized_swiglu (rules as qgemm_prefill). */
int qgemm_prefill_swiglu(const void *q_weights, int fmt, const void *x, int x_dtype, int64_t M, int64_t F,
                         int64_t K, uint16_t *h, void *workspace, size_t workspace_bytes, void *stream);
/* Name of the kernel the SwiGLU entry points launch for the GEMM (the fused
 * kernel, or the plain GEMM kernel that precedes the SwiGLU kernel), or NULL. */
const char *qgemm_kernel_name_swiglu(int fmt, int64_t M, int64_t F, int64_t K);
/* The SwiGLU step alone: h [M][F] from the fp32 gate+up output y [M][2F] (y
 * and h 16-byte aligned; M * F <= 2^38). */
int qgemm_swiglu(const float *y, int64_t M, int64_t F, uint16_t *h, void *stream);

/* ---- no allocation ----
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * qgemm_prefill_noalloc computes exactly what qgemm_prefill computes (same
 * kernels, same result bit for bit) with the workspace taken from a static
 * device array of QG_NOALLOC_SCRATCH_BYTES inside the library instead of a
 * caller buffer, so it takes no workspace argument and allocates nothing.
 *   - Limit: problems with qgemm_workspace_bytes(M, K) > QG_NOALLOC_SCRATCH_BYTES
 *     are refused with QG_ENOSCRATCH before any launch (16 MiB holds e.g.
 *     M = 2048 rows at K = 4096, or M = 512 at K = 16384).
 *   - Every GPU the library runs on holds its own copy of the array (device
 *     memory reserved with the library's code on that device) until the
 *     process ends.  Its device address is looked up on the first call on
 *     each device (make that first call outside graph capture).
 *   - All calls on one GPU share that GPU's array: calls that may overlap on
 *     one GPU (different streams, different host threads) race and must be
 *     serialised by the caller.  Nothing in the array needs clearing; it is
 *     rewritten by each call before it is read.
 *   - Arguments, alignment, ownership and the other error codes as
 *     qgemm_prefill (QG_PATH_AUTO). */
#define QG_NOALLOC_SCRATCH_BYTES (16ll << 20)
int qgemm_prefill_noalloc(const void *q_weights, int fmt, const void *x, int x_dtype, int64_t M,
                          int64_t N, int64_t K, float *y, void *stream);

/* ---- diagnostics ---- */

/* Shader clock under int8 matrix-core load, for benchmark receipts (the int8
 * peak is quoted at the top clock; sustained matrix-core load runs lower).
 * Launches one kernel on `stream` that keeps every SIMD of the current device
 * busy with independent int8 32x32x32 MFMA chains (four waves per SIMD, four
 * MFMAs per iteration, `iters` iterations) and writes to ticks[0..2] (device
 * memory, 8-byte aligned, 3 x uint64): the shader-clock ticks and the 100 MHz
 * reference-clock ticks that one wave counted over its loop, and a checksum of
 * the MFMA results.  Shader clock in MHz = 100 * ticks[0] / ticks[1].
 * iters in 1 .. 2^24 (QG_EINVAL otherwise).
 *
 * Path tracing: with QGEMM_TRACE=1 in the environment, every accepted GEMM call
 * (plain, per-256, SwiGLU, fp16 branch) writes one line to stderr naming the
 * entry point, format, M, N, K, the path taken and the kernel launched. */
int qgemm_sclk_probe(uint64_t *ticks, int iters, void *stream);

/* Read floor, for benchmark receipts of the bandwidth-bound kernels: launches
 * one kernel on `stream` that reads every byte of src[0 .. bytes) once
 * (16-byte loads, grid-stride over eight 256-thread workgroups per CU) and
 * writes nothing.  Its time is the floor that any one launch reading the same
 * bytes can reach, ramp-up and tail included (a decode GEMV is quoted against
 * it).  src: device memory, 16-byte aligned (QG_EALIGN otherwise), not
 * modified; bytes: a multiple of 16, >= 0 (QG_EINVAL otherwise; 0 launches
 * nothing); src may be NULL only when bytes = 0. */
int qgemm_read_probe(const void *src, int64_t bytes, void *stream);

/* Planted delay, the falsifier of a benchmark's per-kernel timing rows (the
 * bench check of aprender issue #3598, "EPIC E2 0.73: Verbs Are Fast", prior
 * body, row 1: a delay planted in one kernel must move that kernel's row and
 * the step total, and nothing else).  kernel = QG_PLANT_QUANTIZE: from the
 * next call on, every launch of the per-32 activation quantiser that writes
 * a GEMM workspace (qgemm_quantize_workspace, and the quantiser half of
 * qgemm_prefill / qgemm_prefill_ex) has one wave of its first workgroup sleep
 * `sleeps` times 64 shader clocks (s_sleep 1 in a loop of `sleeps`
 * iterations) before it starts; the output is unchanged.  sleeps = 0 removes
 * the delay.  sleeps in 0 .. QG_PLANT_MAX_SLEEPS, an unknown kernel:
 * QG_EINVAL.  The setting is process-wide, host-side state (no launch, no
 * device needed); set it only while no other thread is timing or launching. */
#define QG_PLANT_QUANTIZE 1
#define QG_PLANT_MAX_SLEEPS 1000000
int qgemm_test_plant_delay(int kernel, int sleeps);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_H */
