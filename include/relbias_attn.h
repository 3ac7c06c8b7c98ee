/*
 * relbias_attn.h - C ABI of the relative-position-bias attention library (MI355X, gfx950).
 *
 * The operation (both entry points): causal softmax attention whose logits
 * carry an additive bias that depends on the query-key distance
 *     delta = pos(query) - pos(key),
 *     s = scale * <q, k> + beta(h, query, delta),   o = softmax(s) @ v,
 * with keys visible iff 0 <= delta and (window == 0 or delta < window), and
 * beta = 0 for delta >= bias_range ("Learned Relative-Position Bias",
 * section "Standard Relative Bias (T5-style)" for the scaled content term plus
 * a distance bias, section "Inkling's Input-Dependent Version (Conceptual)"
 * for the 512 / 1024 ranges and the content-only tail; "Thinking Machines
 * dropped RoPE", steps 1-5, for the input-dependent bias and the hard zero
 * outside the range).  The bias is added after `scale`, it is not scaled.
 *
 * Optional context-length temperature (temp_len > 0): the logit of a query that
 * sees n keys becomes tau(n) * s with
 *     tau(n) = 1 for n <= temp_len,   tau(n) = ln(n) / ln(temp_len) beyond,
 * a factor on the q.k term and the bias alike ("Thinking Machines dropped RoPE",
 * section "The temperature scale is dependent on context length": global layers
 * scale the queries and the position bias by a factor that is flat up to 128k
 * visible keys and grows logarithmically after; that page prints no formula, the
 * log-ratio above is the plain log-n form it names).  n counts the visible keys:
 * pos + 1, capped at window when window > 0.  temp_len = 131072 gives the 128k
 * threshold; temp_len = 0 turns the temperature off.
 *
 * Bias modes:
 *   RBA_BIAS_NONE   beta = 0 (content only).
 *   RBA_BIAS_TABLE  beta = table[h, delta]: a learned per-head table indexed by
 *                   distance, T5 style ("Thinking Machines dropped RoPE",
 *                   section "Option 3: position as a bias to the attention").
 *   RBA_BIAS_RPROJ  beta = sum_{f<R} r[token, h, f] * E[h, f, delta]: the query
 *                   token's coefficients (output of the fourth projection,
 *                   "Inkling 975B MoE architecture deep dive", section "No RoPE?
 *                   No Problem?") weighting a bank of R learned distance curves
 *                   ("Thinking Machines dropped RoPE", steps 1-3).
 *   RBA_BIAS_RPROJ_SHARED
 *                   beta = sum_{f<R} r[token, h, f] * E[f, delta]: as RBA_BIAS_RPROJ
 *                   with one bank of R curves used by every head of the layer, the
 *                   form that essay's step 2 describes (one set of learned distance
 *                   functions for all heads and tokens); E is [R, bias_range].
 *
 * Conventions shared by every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     allocates nothing, keeps no state other than a thread-local error
 *     message, and may be called from several threads.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL = the
 *     default stream) and is asynchronous: outputs are valid once the stream
 *     has reached the call.  Nothing synchronises.
 *   - Tensors are dense and row-major with the last index innermost, as in
 *     the shapes below.  q, k, v, o (and the caches) must be 16-byte aligned.
 *   - GQA: query head h reads kv head h / (Hq / Hkv); Hq must be a multiple
 *     of Hkv.
 *   - Return value: RBA_OK, or an error code with nothing launched
 *     (RBA_EINVAL: invalid argument; RBA_ENOTSUP: valid but outside the
 *     supported set).  RBA_EHIP reports a HIP error seen at launch time.
 *     relbias_attn_last_error() gives the message of the calling thread's
 *     last non-OK status.
 *   - Supported set: dtype RBA_BF16 with D in {64, 128}; dtype RBA_F32 with
 *     D in {32, 64, 128}; 1 <= R <= 16; bias_range <= 1048576.
 *   - Empty problems (B == 0 or S == 0) return RBA_OK and launch nothing.
 */
#ifndef RELBIAS_ATTN_H
#define RELBIAS_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { RBA_OK = 0, RBA_EINVAL = 1, RBA_ENOTSUP = 2, RBA_EHIP = 3 } rba_status_t;
typedef enum { RBA_F32 = 0, RBA_BF16 = 1 } rba_dtype_t;
typedef enum {
  RBA_BIAS_NONE = 0,
  RBA_BIAS_TABLE = 1,
  RBA_BIAS_RPROJ = 2,
  RBA_BIAS_RPROJ_SHARED = 3
} rba_bias_mode_t;

/*
 * Prefill: every token of B sequences of length S attends to its own
 * sequence; query i and key j sit at positions i and j.
 *
 *   dtype       RBA_BF16 or RBA_F32: element type of q, k, v, o and r.
 *   q           [B, S, Hq, D]
 *   k, v        [B, S, Hkv, D]
 *   o           [B, S, Hq, D]  (written)
 *   lse         [B, Hq, S] fp32 natural-log sum-exp of each row (written), or NULL.
 *   window      0 = full causal; else key j is visible to query i iff 0 <= i-j < window.
 *   bias_range  bias applied iff 0 <= i-j < bias_range (ignored for RBA_BIAS_NONE).
 *   mode        rba_bias_mode_t.
 *   table       RBA_BIAS_TABLE: [Hq, bias_range] fp32; else ignored (may be NULL).
 *   r           RBA_BIAS_RPROJ(_SHARED): [B, S, Hq, R] of dtype; else ignored.
 *   E           RBA_BIAS_RPROJ: [Hq, R, bias_range] fp32; RBA_BIAS_RPROJ_SHARED:
 *               [R, bias_range] fp32; else ignored.
 *   R           RBA_BIAS_RPROJ(_SHARED): number of curves, 1..16.
 *   scale       multiplier of q.k (typically 1/sqrt(D)); the bias is not scaled.
 *   temp_len    0 (no temperature) or >= 2: the visible-key count beyond which the
 *               context-length temperature grows (see above); 1 or negative: RBA_EINVAL.
 *   workspace   device scratch of at least relbias_attn_fwd_workspace_size(...) bytes,
 *               16-byte aligned, owned by the caller; contents on entry are ignored and
 *               are undefined on return.  NULL is allowed when that size is 0.  A call
 *               reads and writes it on `stream` only: calls that overlap in time need
 *               distinct workspaces.  Too small or misaligned: RBA_EINVAL.
 *   workspace_bytes  its size in bytes.
 *   stream      hipStream_t.
 */
int relbias_attn_fwd(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int S, int Hq, int Hkv, int D, int window, int bias_range, int mode,
                     const float* table, const void* r, const float* E, int R, float scale,
                     int temp_len, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace relbias_attn_fwd needs for these arguments (0: none).
 * With the input-dependent bias (head_dim 128, Hq/Hkv a multiple of 4, bias_range a
 * multiple of 4) the bf16 prefill converts E once per call into a bf16, distance-major
 * copy there: heads * (bias_range + 129) * EF * 2 bytes rounded up to 256, with EF = 8
 * for R <= 8 and 16 above, heads = Hq (RBA_BIAS_RPROJ) or 1 (RBA_BIAS_RPROJ_SHARED).
 * Pure host function; arguments that relbias_attn_fwd would reject give 0.
 */
size_t relbias_attn_fwd_workspace_size(int dtype, int B, int S, int Hq, int Hkv, int D,
                                       int window, int bias_range, int mode, int R,
                                       float scale);

/*
 * Bytes of device workspace relbias_attn_decode needs for these sizes
 * (0 when a single pass writes the output directly).  Pure host function.
 */
size_t relbias_attn_decode_workspace_size(int B, int Hq, int Hkv, int D, int kv_len, int window);

/*
 * Single-token decode against a contiguous KV cache (one new query per sequence).
 * The cache already holds the new token's own key/value at row kv_len-1; the
 * query sits at position kv_len-1 and key row j at position j (rows >= kv_len
 * are not read).  Attention, window and bias are as in relbias_attn_fwd.
 *
 *   q           [B, Hq, D]
 *   k_cache     [B, L_max, Hkv, D]; v_cache the same.  1 <= kv_len <= L_max.
 *   o           [B, Hq, D] (written); lse [B, Hq] fp32 or NULL.
 *   r           RBA_BIAS_RPROJ(_SHARED): [B, Hq, R] of dtype (coefficients of the new token).
 *   table, E, R, scale, temp_len: as in relbias_attn_fwd (the query sees
 *               min(kv_len, window) keys with a window, kv_len without).
 *   workspace   device scratch of at least relbias_attn_decode_workspace_size(...)
 *               bytes (may be NULL when that size is 0); contents on entry are
 *               ignored.  Calls that share one workspace must be ordered on one stream.
 *   Supported: dtype RBA_BF16 with D in {64, 128}, and dtype RBA_F32 with D in {32, 64, 128}.
 */
int relbias_attn_decode(int dtype, const void* q, const void* k_cache, const void* v_cache,
                        void* o, float* lse, int B, int L_max, int kv_len, int Hq, int Hkv, int D,
                        int window, int bias_range, int mode, const float* table, const void* r,
                        const float* E, int R, float scale, int temp_len, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * Size of the fixed per-GPU scratch of relbias_attn_decode_noalloc (16 MiB).
 */
#define RBA_DECODE_NOALLOC_SCRATCH_BYTES (16 * 1024 * 1024)

/*
 * relbias_attn_decode without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments (minus workspace and workspace_bytes), same kernels and the same results as
 * relbias_attn_decode; bf16 only (RBA_ENOTSUP for RBA_F32).
 *
 * The split partials live in a fixed device array inside the library, one copy per GPU of
 * RBA_DECODE_NOALLOC_SCRATCH_BYTES, held until the process ends; this call allocates nothing
 * (no hipMalloc, no allocating library routine).  Sizes whose
 * relbias_attn_decode_workspace_size(...) exceeds RBA_DECODE_NOALLOC_SCRATCH_BYTES return
 * RBA_ENOTSUP before anything is launched.  The stream must belong to the current device
 * (RBA_EINVAL otherwise).  Every call on one GPU shares that GPU's array and the array keeps the
 * last call's contents (nothing there needs to start at zero): calls that overlap on one GPU
 * (on different streams, or from several host threads) race and give wrong results; order them
 * on one stream.
 */
int relbias_attn_decode_noalloc(int dtype, const void* q, const void* k_cache, const void* v_cache,
                                void* o, float* lse, int B, int L_max, int kv_len, int Hq, int Hkv,
                                int D, int window, int bias_range, int mode, const float* table,
                                const void* r, const float* E, int R, float scale, int temp_len,
                                void* stream);

/*
 * Bytes of device workspace relbias_attn_decode_paged needs (0 when none): the
 * launch is sized for max_kv_len, so this is the contiguous size at that length.
 */
size_t relbias_attn_decode_paged_workspace_size(int B, int Hq, int Hkv, int D, int max_kv_len,
                                                int window);

/*
 * Single-token decode against a paged KV cache with a cache length per sequence,
 * two of the shapes a fused-bias attention kernel has to cover ("Thinking Machines
 * dropped RoPE", the paragraphs on the kernel cost of the bias, which list paged
 * KV and variable sequence lengths among them).  Per sequence b it computes exactly
 * what relbias_attn_decode computes with kv_len = kv_lens[b] over the logical
 * cache whose row j is row (j % page_size) of page block_table[b][j / page_size].
 *
 *   q           [B, Hq, D]; o [B, Hq, D] (written); lse [B, Hq] fp32 or NULL.
 *   k_pages     [num_pages, page_size, Hkv, D] of dtype: the pool of key pages;
 *               v_pages the same for values.  Pages may be shared or in any order.
 *   block_table DEVICE int32 [B, max_pages]: page of each sequence's logical page.
 *   kv_lens     DEVICE int32 [B]: cache length of each sequence, 1..max_kv_len;
 *               the query sits at position kv_lens[b] - 1.
 *   max_kv_len  host upper bound of every kv_lens[b] (sizes the launch);
 *               1 <= max_kv_len <= max_pages * page_size.
 *   page_size   rows per page, a multiple of 16.
 *   window, bias_range, mode, table, r ([B, Hq, R]), E, R, scale, temp_len: as in
 *               relbias_attn_decode (the temperature follows each kv_lens[b]).
 *   workspace   at least relbias_attn_decode_paged_workspace_size(...) bytes
 *               (may be NULL when that size is 0).
 * The device values are not validated: lengths are clamped to [0, max_kv_len] and
 * page indices to [0, num_pages), so wrong values give wrong results but no
 * access outside the given buffers; kv_lens[b] = 0 leaves o[b] undefined.
 * Supported: dtype RBA_BF16 with D in {64, 128} (RBA_ENOTSUP otherwise).
 */
int relbias_attn_decode_paged(int dtype, const void* q, const void* k_pages, const void* v_pages,
                              const int* block_table, const int* kv_lens, void* o, float* lse,
                              int B, int num_pages, int page_size, int max_pages, int max_kv_len,
                              int Hq, int Hkv, int D, int window, int bias_range, int mode,
                              const float* table, const void* r, const float* E, int R,
                              float scale, int temp_len, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * MXFP4 quantisation of bf16 rows, the FP4 KV cache format of relbias_attn_decode_fp4.  The
 * pages list an FP4 KV cache among Inkling's KV-cache compression methods and MXFP4 among its
 * FP4 formats ("models/inkling" (archdiff), the component diagram: KV-cache compression and
 * FP8-to-FP4 training); the format is the OCP Microscaling one: each block of 32 consecutive
 * elements of a row shares the scale 2^(s - 127) stored as one byte s (E8M0), each element is
 * a 4-bit E2M1 code (bit 3 the sign; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6).  Rounding: the
 * block exponent is floor(log2(max |x|)) - 2, clamped to [-126, 127]; x / 2^exponent goes to
 * the nearest magnitude, ties to the even code, saturating at 6; the sign bit is set iff
 * x < 0; an all-zero block gets scale byte 0 and zero codes.  NaN inputs are not supported.
 *
 *   x       [rows, D] bf16, 16-byte aligned; D a multiple of 32.
 *   codes   [rows, D / 2] bytes (written): element 2j in the low nibble of byte j, element
 *           2j + 1 in the high nibble; 16-byte aligned.
 *   scales  [rows, D / 32] bytes (written).
 * A KV cache [B, L, Hkv, D] is rows = B * L * Hkv rows of D.
 */
int relbias_attn_kv_quantize_fp4(const void* x, void* codes, void* scales, long long rows, int D,
                                 void* stream);

/*
 * relbias_attn_decode over MXFP4 caches: the same computation, with K and V read from
 * k_codes [B, L_max, Hkv, D / 2] + k_scales [B, L_max, Hkv, D / 32] (and the same for V) in
 * the layout relbias_attn_kv_quantize_fp4 writes; each element is code value * 2^(s - 127)
 * (scale byte 0 reads as 0).  q is bf16 [B, Hq, D]; every other argument (workspace size
 * included) as in relbias_attn_decode with dtype RBA_BF16.  Supported: D = 64 or 128 and
 * Hq / Hkv <= 32 (RBA_ENOTSUP otherwise).
 */
int relbias_attn_decode_fp4(const void* q, const void* k_codes, const void* k_scales,
                            const void* v_codes, const void* v_scales, void* o, float* lse, int B,
                            int L_max, int kv_len, int Hq, int Hkv, int D, int window,
                            int bias_range, int mode, const float* table, const void* r,
                            const float* E, int R, float scale, int temp_len, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * relbias_attn_decode_paged over MXFP4 page pools: the paged cache shapes the pages list for a
 * fused-bias kernel ("Thinking Machines dropped RoPE", the paragraphs on the kernel cost of the
 * bias: paged KV, variable sequence lengths) with the FP4 KV-cache compression of
 * relbias_attn_decode_fp4 ("models/inkling" (archdiff), the component diagram).  Per sequence b
 * it computes exactly what relbias_attn_decode_fp4 computes with kv_len = kv_lens[b] over the
 * logical cache whose row j is row (j % page_size) of page block_table[b][j / page_size].
 *
 *   k_codes     [num_pages, page_size, Hkv, D / 2] MXFP4 codes, k_scales [num_pages,
 *               page_size, Hkv, D / 32] E8M0 scale bytes, in the layout
 *               relbias_attn_kv_quantize_fp4 writes (and the same for V); codes 16-byte aligned.
 *   q, o, lse, block_table, kv_lens, num_pages, page_size, max_pages, max_kv_len, window,
 *               bias_range, mode, table, r, E, R, scale, temp_len, workspace: as in
 *               relbias_attn_decode_paged (dtype RBA_BF16), with the same clamping of the
 *               device values and the same workspace size.
 * Supported: D = 64 or 128 and Hq / Hkv <= 32 (RBA_ENOTSUP otherwise).
 */
int relbias_attn_decode_fp4_paged(const void* q, const void* k_codes, const void* k_scales,
                                  const void* v_codes, const void* v_scales,
                                  const int* block_table, const int* kv_lens, void* o, float* lse,
                                  int B, int num_pages, int page_size, int max_pages,
                                  int max_kv_len, int Hq, int Hkv, int D, int window,
                                  int bias_range, int mode, const float* table, const void* r,
                                  const float* E, int R, float scale, int temp_len,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace relbias_attn_bwd needs: one fp32 per (batch, row, query head),
 * rounded up to 256 bytes, and for the input-dependent modes the bank E converted to bf16 high
 * and low parts (per bank head (Hq, or 1 when shared): bias_range + 129 distances of 32 bf16
 * values each); independent of S beyond the first term.  Pure host function.
 */
size_t relbias_attn_bwd_workspace_size(int B, int S, int Hq, int mode, int bias_range);

/*
 * Backward of relbias_attn_fwd: gradients of a scalar loss given its gradient dout on o.
 * The bias is a learned part of the layer ("Thinking Machines dropped RoPE": the bank of
 * distance curves and the coefficient projection are trained with the model; "Learned
 * Relative-Position Bias", section "Standard Relative Bias (T5-style)": the table is a
 * learned parameter), so the call also returns the gradient of the bias parameters.
 * With P the forward's softmax and tau the temperature (1 when temp_len = 0):
 *   dP = dout v^T,  dS = P * (dP - rowsum(dout * o)),  dZ = tau * dS,
 *   dq = scale dZ k,  dk = scale dZ^T q,  dv = P^T dout  (kv heads sum their query heads),
 *   at in-band pairs the bias gradient is dZ, reduced to dtable[h, d] (sum along the
 *   diagonal at distance d), or to dr[token, h, f] = sum_j dZ E[h, f, delta] and
 *   dE[h, f, d] = sum over tokens of r[token, h, f] dZ at distance d (summed over heads
 *   for RBA_BIAS_RPROJ_SHARED).
 *
 *   dtype       RBA_BF16 (D in {64, 128}; MFMA kernels) or RBA_F32 (D in {32, 64, 128};
 *               vector-ALU kernels, fp32 throughout); every tensor below of that dtype
 *               unless stated.  The bf16 kernels stage the bias parameters in LDS, which
 *               bounds bias_range: table up to 14016 distances (D = 128) or 17088 (D = 64);
 *               r.E up to 3456 with R = 8 and 1664 with R = 16 at D = 128 (4992 and 2432 at
 *               D = 64; more for smaller R); past that the call returns RBA_ENOTSUP.  The fp32
 *               kernels read the bias parameters from global memory and have no such bound.
 *   q, k, v, window, bias_range, mode, table, r, E, R, scale, temp_len, shapes:
 *               exactly as passed to relbias_attn_fwd.
 *   o           [B, S, Hq, D]: the forward's output.
 *   lse         [B, Hq, S] fp32: the forward's log-sum-exp (required).
 *   dout        [B, S, Hq, D]: gradient of the loss on o.
 *   dq          [B, S, Hq, D] (written); dk, dv [B, S, Hkv, D] (written).
 *   dtable      RBA_BIAS_TABLE: [Hq, bias_range] fp32 (written); else ignored.
 *   dr          RBA_BIAS_RPROJ(_SHARED): [B, S, Hq, R] of dtype (written); else ignored.
 *   dE          RBA_BIAS_RPROJ: [Hq, R, bias_range] fp32; RBA_BIAS_RPROJ_SHARED:
 *               [R, bias_range] fp32 (written); else ignored.
 *   workspace   device scratch of at least relbias_attn_bwd_workspace_size(B, S, Hq, mode,
 *               bias_range) bytes, 16-byte aligned; contents on entry are ignored.  Calls that share one workspace,
 *               dtable or dE must be ordered on one stream.
 * dtable and dE are summed with fp32 atomics, so their last bits may differ between runs;
 * dq, dk, dv and dr are deterministic.
 */
int relbias_attn_bwd(int dtype, const void* q, const void* k, const void* v, const void* o,
                     const float* lse, const void* dout, void* dq, void* dk, void* dv,
                     float* dtable, void* dr, float* dE, int B, int S, int Hq, int Hkv, int D,
                     int window, int bias_range, int mode, const float* table, const void* r,
                     const float* E, int R, float scale, int temp_len, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Message for the calling thread's last non-OK status ("" if none).  The pointer
 * stays valid until the next call on the same thread. */
const char* relbias_attn_last_error(void);

/* Library version string, e.g. "relbias_attn 0.1 gfx950". */
const char* relbias_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RELBIAS_ATTN_H */
