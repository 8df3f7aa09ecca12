/*
 * flash_attn.h - C ABI of the fused exact-attention library for AMD MI355X
 * (gfx950).
 *
 * What is computed (sources are the web pages the method is described on):
 *
 *   O = softmax(scale * Q K^T) V          per (batch, head)
 *
 * the scaled dot-product attention of "优化的注意力实现 (FlashAttention)"
 * (apxml course page, section "标准注意力中的内存带宽瓶颈") and of the CMU
 * 15-442/642 notes "Transformer、注意力机制与优化" (section "数学公式"), with
 * Q, K, V in R^{N x d}.  The forward pass is one fused, tiled kernel that
 * keeps a running row maximum m and row sum l (same notes, section
 * "安全 Softmax 与在线 Softmax") so the N x N score matrix never reaches
 * device memory; it stores O and, per row, LSE = m + ln l, the single
 * statistic the FlashAttention-2 forward keeps for the backward pass
 * ("FlashAttention 系列技术详解", section "具体优化策略").  The backward pass
 * recomputes the scores from LSE ("FlashAttention 的基本原理", section 2.4).
 * The CMU notes (section "为什么前向和反向的并行化策略不同") accumulate dQ
 * across key blocks with atomic adds; on MI355X those fp32 atomics are the
 * bottleneck, so here dQ has its own pass over query blocks (recomputing S
 * and dP for its rows) and every result, dQ included, is deterministic.
 *
 * Conventions shared by every entry point
 *  - Tensors are dense, row-major [B, H, N, d]: element (b, h, n, c) is at
 *    ((b * H + h) * N + n) * d + c.  Q, K, V, O, dO, dQ, dK, dV are bf16
 *    (passed as raw pointers to 16-bit storage); LSE is float32 [B, H, N].
 *  - Queries and keys have the same length N.  Causal masking lets query i
 *    see key j iff j <= i (the apxml example's tril(diagonal=0) mask).
 *  - softmax_scale multiplies Q K^T before masking and softmax; it must be
 *    finite and > 0 (the pages' scale is 1/sqrt(d)).
 *  - LSE is the natural-log log-sum-exp of the scaled, masked scores.
 *  - Supported head dims: d = 64 and d = 128.  Any N >= 1 (ragged tails are
 *    masked).  B, H >= 1.  B = 0, H = 0 or N = 0 is an empty problem: the
 *    call returns FA_OK at once and touches no pointer.
 *  - Every device pointer must be 16-byte aligned (LSE: 4-byte).
 *  - Ownership: the caller allocates and frees every buffer, including the
 *    backward workspace.  The library never allocates, frees or keeps device
 *    memory and holds no mutable global state; calls on different streams
 *    may run concurrently.
 *  - Outputs are fully overwritten and must not overlap any input or each
 *    other (FA_ERR_ALIASING).
 *  - Errors: arguments are validated synchronously, before any HIP call, and
 *    an error leaves every buffer untouched.  Work is enqueued on `stream`
 *    (a hipStream_t; NULL means the null stream) and runs asynchronously;
 *    FA_ERR_HIP reports a failed launch (hipGetLastError after enqueueing).
 *    Faults during execution surface at the caller's next synchronisation.
 *  - There is no fallback path: an unsupported argument is an error.
 */
#ifndef FLASH_ATTN_MI355X_H
#define FLASH_ATTN_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL_POINTER = 1,        /* a required pointer is NULL */
  FA_ERR_BAD_SHAPE = 2,           /* B, H or N negative, or sizes overflow */
  FA_ERR_UNSUPPORTED_HEAD_DIM = 3,/* d is not 64 or 128 */
  FA_ERR_MISALIGNED = 4,          /* a pointer breaks the alignment rule */
  FA_ERR_BAD_SCALE = 5,           /* softmax_scale is NaN, Inf or <= 0 */
  FA_ERR_WORKSPACE_TOO_SMALL = 6, /* workspace_bytes below the required size */
  FA_ERR_HIP = 7,                 /* the HIP runtime rejected a launch */
  FA_ERR_ALIASING = 8,            /* an output overlaps an input or output */
  FA_ERR_BAD_SPLITS = 9,          /* num_splits outside 1..128 (split-KV forward) */
  FA_ERR_BAD_DESCALE = 10,        /* an FP8 descale factor is NaN, Inf or <= 0 */
  FA_ERR_BAD_DROPOUT = 11,        /* dropout_p is NaN, < 0 or rounds to 1 (see below) */
  FA_ERR_SCRATCH_TOO_SMALL = 12   /* problem needs more than the library's static scratch */
};

/*
 * Forward pass.
 *   q, k, v : in,  bf16 [B, H, N, d]
 *   o       : out, bf16 [B, H, N, d]   O = softmax(scale * Q K^T (masked)) V
 *   lse     : out, fp32 [B, H, N]      LSE = m + ln l of each query row
 *   causal  : 0 = full attention, non-zero = causal mask
 * Follows the FlashAttention-2 outline of the CMU notes (section
 * "FlashAttention-2 算法"): one query block per workgroup, K/V blocks
 * streamed through on-chip memory, running (m, l, O) in registers, one
 * division by l at the end.  Deterministic: identical inputs give
 * bit-identical O and LSE.
 */
int flash_attn_fwd(const void* q, const void* k, const void* v,
                   void* o, float* lse,
                   int64_t B, int64_t H, int64_t N, int64_t d,
                   int causal, float softmax_scale, void* stream);

/*
 * Split-KV forward: the same O and LSE as flash_attn_fwd, computed with the
 * key tiles of every query block cut into num_splits contiguous ranges, one
 * workgroup per (head, query block, range), followed by a merge kernel.
 * This is the combine step of Flash-Decoding (CMU notes, section
 * "Flash-Decoding": the per-block statistics (m, l) merge associatively and
 * commutatively, section "安全 Softmax 与在线 Softmax"): each range yields
 * an unnormalised partial output with its own running max m_s and row sum
 * l_s, and per row
 *   M = max_s m_s,  L = sum_s 2^(m_s - M) l_s,
 *   O = sum_s 2^(m_s - M) O_s / L,  LSE = (M + log2 L) ln 2
 * (m in log2 units of the scaled scores).  It fills the GPU when
 * B * H * ceil(N_q / 256) is small.  Results agree with flash_attn_fwd to
 * rounding (not bitwise: the sums are grouped differently).
 * The queries and the keys may differ in number, as in the decode step of
 * the CMU notes (section "生成式 LLM 推理"): one new query, or a short block
 * of them, against every cached key and value, which is the case Flash-
 * Decoding splits the keys for.  The apxml example's interface gives the
 * query and key/value tensors their own sequence lengths the same way.
 *   q, o       : bf16 [B, H, N_q, d];  lse : fp32 [B, H, N_q]
 *   k, v       : bf16 [B, H, N_kv, d]
 *   causal     : requires N_q == N_kv (FA_ERR_BAD_SHAPE otherwise); with
 *                N_q != N_kv every query sees every key
 *   N_kv       : >= 1 when B * H * N_q > 0 (FA_ERR_BAD_SHAPE otherwise)
 *   softmax_scale : as flash_attn_fwd
 *   workspace  : device memory of at least
 *                flash_attn_fwd_splitkv_workspace_bytes(B, H, N_q, d,
 *                num_splits) bytes, 16-byte aligned, caller-owned, no
 *                initialisation; it must not overlap any other argument
 *   num_splits : 1 .. 128 key ranges per query block (ranges with no key a
 *                query sees contribute nothing); FA_ERR_BAD_SPLITS otherwise
 * Two launches on `stream`.  Deterministic.
 */
int flash_attn_fwd_splitkv(const void* q, const void* k, const void* v,
                           void* o, float* lse,
                           void* workspace, size_t workspace_bytes,
                           int64_t B, int64_t H, int64_t N_q, int64_t N_kv, int64_t d,
                           int causal, float softmax_scale, int64_t num_splits,
                           void* stream);

/*
 * Bytes of workspace flash_attn_fwd_splitkv needs for N_q queries per
 * head: fp32 partial outputs [num_splits, B*H, N_q, d], then the fp32
 * running max and row sum [num_splits, B*H, N_q] each, every section
 * rounded up to 256 bytes (the key length does not enter).  Returns 0 for an
 * empty problem and for invalid sizes or num_splits.
 */
size_t flash_attn_fwd_splitkv_workspace_bytes(int64_t B, int64_t H, int64_t N_q, int64_t d,
                                              int64_t num_splits);

/*
 * FP8 forward: the attention of flash_attn_fwd over Q, K, V given as OCP FP8
 * E4M3 ("E4M3FN": sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities, S.1111.111 = NaN), one byte per element, each tensor with one
 * float32 dequantisation factor: the real input is descale * e4m3(code).
 * Low-precision FP8 matrix products are the FlashAttention-3 change listed
 * in "FlashAttention 系列技术详解" (section on FlashAttention-3).
 *   q, k, v    : in,  E4M3 codes [B, H, N, d] (uint8 storage)
 *   o          : out, bf16 [B, H, N, d]
 *                O = softmax(softmax_scale * dq * dk * Q K^T (masked)) * dv V
 *   lse        : out, fp32 [B, H, N], natural log, of those scaled scores
 *   descale_q, descale_k, descale_v : dq, dk, dv; finite and > 0
 *                (FA_ERR_BAD_DESCALE otherwise)
 *   causal, softmax_scale, stream   : as flash_attn_fwd
 * Both products run on the FP8 matrix cores with fp32 accumulation.  Q K^T
 * is exact products summed in fp32; the probabilities are rounded to E4M3
 * (relative error <= 2^-4, values below 2^-14 of the row max may round to
 * 0) before the product with V, so O is accurate to about that rounding;
 * the row sums, and hence LSE, use the unrounded fp32 probabilities.
 * Inputs must hold no NaN codes.  Same shapes, alignment (16 bytes for q, k,
 * v, o), ownership and error rules as flash_attn_fwd.  Deterministic.
 */
int flash_attn_fwd_fp8(const void* q, const void* k, const void* v,
                       void* o, float* lse,
                       int64_t B, int64_t H, int64_t N, int64_t d,
                       int causal, float softmax_scale,
                       float descale_q, float descale_k, float descale_v,
                       void* stream);

/*
 * FP8 quantisation for flash_attn_fwd_fp8, with optional incoherent
 * processing ("FlashAttention 系列技术详解", FlashAttention-3 section: the
 * queries and keys are multiplied by a random orthogonal matrix, a Hadamard
 * transform, to spread large entries and lower the quantisation error).
 *   x         : in,  bf16 [rows, d] (e.g. Q or K as [B*H*N, d])
 *   codes     : out, E4M3 [rows, d]: codes of y / descale, nearest even
 *   descale   : out, device fp32 scalar: amax|y| / 448 (1 if y is all zero)
 *   workspace : device memory of at least FA_QUANT_WORKSPACE_BYTES bytes,
 *               16-byte aligned, no initialisation (partial maxima)
 *   signs     : device fp32 [d] of +1 / -1, or NULL.  With signs,
 *               y = x M, M = diag(signs) H_d / sqrt(d) (H_d the Sylvester
 *               Hadamard matrix); apply the same signs to Q and K (then
 *               Q M (K M)^T = Q K^T) and pass V with NULL.  Without, y = x.
 *   d         : 64 or 128
 * x, codes, signs and workspace need 16-byte alignment, descale 4 bytes;
 * codes, descale and workspace must not overlap x, signs or each other.
 * x must be finite.  rows = 0 is a no-op.  Two launches on `stream`.
 * Deterministic.
 */
#define FA_QUANT_WORKSPACE_BYTES 4096
int flash_attn_quantize_fp8(const void* x, void* codes, float* descale,
                            void* workspace, size_t workspace_bytes,
                            int64_t rows, int64_t d, const float* signs, void* stream);

/*
 * Dropout on the attention probabilities.  "FlashAttention 的基本原理" (section
 * 2.4) notes that the backward algorithm also covers dropout, and the apxml
 * example applies it to the attention weights after the softmax.  With it,
 *   O = (P o Z * s) V,   P = softmax(scale * Q K^T (masked)),
 * where the keep mask Z is drawn, not passed: element (b, h, i, j) (query i,
 * key j) is kept iff byte (j mod 16) of Philox4x32-10 (Salmon et al.,
 * "Parallel random numbers: as easy as 1, 2, 3", SC 2011) with
 *   counter = (floor(j / 16), i, b * H + h, offset),
 *   key     = (seed mod 2^32, floor(seed / 2^32))
 * (bytes numbered little-endian through the four output words) is >= t,
 * t = floor(256 * dropout_p + 1/2), and s = 256 / (256 - t).  dropout_p must
 * be >= 0 with t <= 255 (FA_ERR_BAD_DROPOUT otherwise); t = 0 keeps every
 * element.  LSE is that of the scores (dropout does not change the softmax
 * statistics).  The same (seed, offset) must be passed to the backward.
 *   all other arguments : as flash_attn_fwd
 * Deterministic.
 */
int flash_attn_fwd_dropout(const void* q, const void* k, const void* v,
                           void* o, float* lse,
                           int64_t B, int64_t H, int64_t N, int64_t d,
                           int causal, float softmax_scale,
                           float dropout_p, uint64_t seed, uint32_t offset,
                           void* stream);

/*
 * Backward of flash_attn_fwd_dropout: dV = (P o Z s)^T dO, dP = (dO V^T) o Z s,
 * dS = P o (dP - D) with D_i = sum_c dO_ic O_ic, dQ = scale dS K,
 * dK = scale dS^T Q, the mask Z redrawn from the same (seed, offset).
 *   o, lse : the outputs of flash_attn_fwd_dropout with the same arguments
 *   all other arguments : as flash_attn_bwd and flash_attn_fwd_dropout
 * Three launches (row pass, key-block pass, query-block pass).  Deterministic.
 */
int flash_attn_bwd_dropout(const void* q, const void* k, const void* v,
                           const void* o, const float* lse, const void* dout,
                           void* dq, void* dk, void* dv,
                           void* workspace, size_t workspace_bytes,
                           int64_t B, int64_t H, int64_t N, int64_t d,
                           int causal, float softmax_scale,
                           float dropout_p, uint64_t seed, uint32_t offset,
                           void* stream);

/*
 * Bytes of device workspace flash_attn_bwd needs for this shape: two fp32
 * row vectors [B*H, Npad] (the rowsum(dO o O) term D, stored negated, and
 * LSE in base 2; Npad is N rounded up to a multiple of 64), each rounded up
 * to 256 bytes.
 * Returns 0 for an empty problem and for invalid sizes.
 * The two vectors are the per-row statistics the backward pass works from:
 * the stored sum of exponentials it recomputes the probabilities with
 * ("FlashAttention 系列技术详解", section "反向传播步骤"; the FlashAttention-2
 * forward keeps only that one statistic, section "具体优化策略"), and the
 * per-row softmax-gradient term of "FlashAttention 的基本原理" (section 2.4).
 * The caller owns the memory so that the library never allocates.
 */
size_t flash_attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d);

/*
 * Backward pass (recompute from LSE).
 *   q, k, v, o : in, bf16 [B, H, N, d]  (o and lse from flash_attn_fwd with
 *                the same q, k, v, causal and softmax_scale)
 *   lse        : in, fp32 [B, H, N]
 *   dout       : in, bf16 [B, H, N, d]  gradient of the loss w.r.t. O
 *   dq, dk, dv : out, bf16 [B, H, N, d]
 *   workspace  : device memory of at least
 *                flash_attn_bwd_workspace_bytes(B, H, N, d) bytes, 16-byte
 *                aligned, no initialisation needed, caller-owned; it must
 *                not overlap any other argument.
 * Three launches on `stream`: a row pass (D_i = sum_c dO_ic O_ic and LSE in
 * base 2 into the workspace), a pass over key blocks (dK, dV accumulated in
 * registers per key block) and a pass over query blocks (dQ accumulated in
 * registers per query block).  No atomics: the results are deterministic.
 */
int flash_attn_bwd(const void* q, const void* k, const void* v,
                   const void* o, const float* lse, const void* dout,
                   void* dq, void* dk, void* dv,
                   void* workspace, size_t workspace_bytes,
                   int64_t B, int64_t H, int64_t N, int64_t d,
                   int causal, float softmax_scale, void* stream);

/*
 * Backward pass that allocates nothing, for callers that cannot allocate or
 * pass device memory: code under stream capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, kernels and results as
 * flash_attn_bwd (bit-identical outputs), minus the workspace: the row
 * vectors live in a device buffer the library itself holds, one static copy
 * of FA_BWD_NOALLOC_SCRATCH_BYTES per device for the life of the process.
 *   FA_ERR_SCRATCH_TOO_SMALL if flash_attn_bwd_workspace_bytes(B, H, N, d)
 *   exceeds FA_BWD_NOALLOC_SCRATCH_BYTES (B * H * Npad > 2^20 rows), before
 *   any HIP call.
 * The first call on a device looks up that device's buffer address (a HIP
 * call with the device current, nothing allocated); a failed lookup is
 * FA_ERR_HIP.  No hipMalloc, hipFree or memset is ever issued.  Every call on
 * one device uses the same buffer and overwrites it (nothing in it needs to
 * start at zero): calls that overlap in time on one device, for example on
 * two streams, race and must not be issued.
 */
#define FA_BWD_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int flash_attn_bwd_noalloc(const void* q, const void* k, const void* v,
                           const void* o, const float* lse, const void* dout,
                           void* dq, void* dk, void* dv,
                           int64_t B, int64_t H, int64_t N, int64_t d,
                           int causal, float softmax_scale, void* stream);

/*
 * The three stages of flash_attn_bwd as separate calls, one kernel launch
 * each, for callers that want to time a stage or put other work between
 * stages.  Enqueued in this order on one stream, with the same shapes and
 * workspace, they are exactly flash_attn_bwd.  Each validates only the
 * pointers it uses (the same rules as flash_attn_bwd); the workspace
 * carries the state from one stage to the next.
 *
 * flash_attn_bwd_preprocess: -D_i = -sum_c dO_ic O_ic and LSE * log2(e)
 *   into the workspace.  Reads o, lse, dout.
 * flash_attn_bwd_kv_blocks: the pass over key blocks.  Reads q, k, v, dout
 *   and the workspace; writes dk, dv.
 * flash_attn_bwd_q_blocks: the pass over query blocks.  Reads q, k, v, dout
 *   and the workspace; writes dq.  The two passes are independent of each
 *   other and may run in either order (or on two streams) after the
 *   preprocess stage.
 */
int flash_attn_bwd_preprocess(const void* o, const float* lse, const void* dout,
                              void* workspace, size_t workspace_bytes,
                              int64_t B, int64_t H, int64_t N, int64_t d, void* stream);

int flash_attn_bwd_kv_blocks(const void* q, const void* k, const void* v,
                             const void* dout, void* dk, void* dv,
                             void* workspace, size_t workspace_bytes,
                             int64_t B, int64_t H, int64_t N, int64_t d,
                             int causal, float softmax_scale, void* stream);

int flash_attn_bwd_q_blocks(const void* q, const void* k, const void* v,
                            const void* dout, void* dq,
                            void* workspace, size_t workspace_bytes,
                            int64_t B, int64_t H, int64_t N, int64_t d,
                            int causal, float softmax_scale, void* stream);

/*
 * Static, human-readable text for a status code ("unknown status" if none).
 * An unsupported configuration is reported, never rerouted: the apxml
 * example ("优化的注意力实现 (FlashAttention)") catches the RuntimeError of
 * an optimised attention kernel that fails or does not support its inputs
 * and falls back, on the caller's side, to the plain implementation.  The
 * library returns the status and this text and leaves any fallback to the
 * caller.
 */
const char* flash_attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FLASH_ATTN_MI355X_H */
