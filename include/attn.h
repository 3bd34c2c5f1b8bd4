/*
 * attn.h -- C ABI of the MI355X (gfx950) fused attention-forward library.
 *
 * One operation: the forward pass of multi-head scaled-dot-product attention,
 *   O = softmax(Q K^T * scale + mask) V          per (sequence, head),
 * the definition of mlqm.cn/news/343191 chapter 1, fused into one kernel as
 * the chain "Q K^T -> scale -> mask -> softmax -> P V" of the same page's
 * §3.1, computed tile by tile with the online softmax of
 * jianying88.com/news/49672 §3 (running row maximum m_i and exponential sum
 * l_i), so the S x S score matrix never reaches device memory.
 *
 * All tensor pointers are DEVICE pointers owned by the caller. The library
 * allocates no memory, keeps no mutable global state and never synchronizes
 * the stream (except attn_check_cu_seqlens), so it is reentrant and
 * thread-safe. Work is enqueued on `stream` (a hipStream_t; NULL = the
 * default stream).
 */
#ifndef SDPA08_ATTN_H
#define SDPA08_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and out. */
enum {
  ATTN_DTYPE_FP16 = 0, /* IEEE binary16 */
  ATTN_DTYPE_BF16 = 1  /* bfloat16 */
};

/* Status codes. Argument errors are returned before any HIP call is made. */
enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = -1,        /* a required pointer is NULL */
  ATTN_ERR_SHAPE = -2,       /* B, H or S out of range, or sizes overflow */
  ATTN_ERR_DTYPE = -3,       /* dtype is not ATTN_DTYPE_FP16 / ATTN_DTYPE_BF16 */
  ATTN_ERR_SCALE = -4,       /* scale is NaN or infinite */
  ATTN_ERR_UNSUPPORTED = -5, /* head dimension D is not 64 or 128 */
  ATTN_ERR_LAUNCH = -6,      /* the HIP runtime reported an error at launch */
  ATTN_ERR_SEQLENS = -7,     /* cu_seqlens failed validation (debug check) */
  ATTN_ERR_ALIGN = -8,       /* a tensor pointer is not 16-byte aligned */
  ATTN_ERR_WORKSPACE = -9,   /* attn_decode / attn_bwd: workspace NULL or too small */
  ATTN_ERR_SCRATCH = -10     /* attn_decode_noalloc: explicit split count beyond its scratch */
};

/*
 * attn_fwd -- fused attention forward.
 *
 * Padded mode (cu_seqlens == NULL):
 *   q, k, v, out : contiguous (B, S, H, D) arrays of `dtype`
 *                  (the (batch, seq, head, dim) layout of
 *                  jianying88.com/news/49672 §4.2).
 *   lse          : contiguous (B, H, S) float32, or NULL (not written).
 * Packed mode (cu_seqlens != NULL), the variable-length interface of
 * lnrk.cn/news/11729 §1 with separate q, k, v tensors:
 *   B            : number of sequences; S: total token count T.
 *   q, k, v, out : contiguous (T, H, D) arrays of `dtype`.
 *   cu_seqlens   : int32 DEVICE array of B+1 prefix offsets, cu_seqlens[0]=0,
 *                  non-decreasing, cu_seqlens[B]=T (zero-length sequences
 *                  allowed). Its contents are a precondition; with the
 *                  environment variable ATTN_DEBUG=1 set when the library
 *                  first checks it, every packed call validates them first
 *                  (this synchronizes the stream).
 *   lse          : contiguous (H, T) float32, or NULL.
 *
 * Semantics: self-attention (query and key lengths equal, same head count
 * for Q and K/V). Scores s_ij = scale * <q_i, k_j> accumulate in fp32 from
 * fp16/bf16 operands; with causal != 0 key j is visible to query i iff j <= i
 * (indices local to the sequence; mlqm.cn/news/343191 §3.1). Packed
 * sequences never attend to each other. lse[i] = ln(sum_j exp(s_ij)) over the
 * visible keys (natural log, fp32). out is rounded to nearest-even.
 *   D     : 64 or 128, else ATTN_ERR_UNSUPPORTED.
 *   scale : any finite float (0 gives uniform attention; negative allowed);
 *           callers usually pass 1/sqrt(D).
 *   B, H, S : 1 <= H <= 65535, B >= 1 (padded) or >= 0 (packed), S >= 0;
 *           B*H*S*D must fit in int64 and the grid in 2^31-1 workgroups.
 *           S == 0 (or B == 0 in packed mode) is a valid no-op.
 * q, k, v, out must be 16-byte aligned (lse: 4-byte aligned), else
 * ATTN_ERR_ALIGN. out/lse must not overlap q, k, v or each other.
 *
 * Errors: ATTN_ERR_* argument codes are returned synchronously with nothing
 * enqueued; ATTN_ERR_LAUNCH if the launch fails (hipGetLastError).
 *
 * The library picks 128- or 256-row query tiles per workgroup from the
 * problem size (attn_fwd_tuned fixes the choice).
 */
int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
             int B, int H, int S, int D, int causal, float scale, int dtype,
             const int32_t* cu_seqlens, void* stream);

/*
 * attn_fwd_tuned -- attn_fwd with its launch shape fixed by the caller (for
 * tuning sweeps and for tests that must reach every kernel instance).
 *
 * Same arguments, layouts, semantics and errors as attn_fwd, plus:
 *   tile_rows  : query rows per workgroup, 128 or 256; 0 lets the library
 *                choose as attn_fwd does. Anything else: ATTN_ERR_UNSUPPORTED.
 *   key_split  : 1: one wave per 32 query rows walks all of the tile's keys;
 *                2: two groups of waves share the rows and take alternate key
 *                blocks, their partial results merged at the end (128-row
 *                tiles only); 0 lets the library choose. Other values, or 2
 *                with 256-row tiles: ATTN_ERR_UNSUPPORTED.
 *   head_group : how many (batch, head) pairs one XCD interleaves the query
 *                tiles of (clamped to B*H, or H when packed); 0 lets the
 *                library choose. Negative: ATTN_ERR_SHAPE.
 * Results do not depend on head_group. 128- and 256-row tiles without a key
 * split are bitwise identical (both walk 64-key tiles with the same per-row
 * arithmetic); the key split adds two partial sums, so it agrees with them to
 * rounding.
 */
int attn_fwd_tuned(const void* q, const void* k, const void* v, void* out, float* lse,
                   int B, int H, int S, int D, int causal, float scale, int dtype,
                   const int32_t* cu_seqlens, int tile_rows, int key_split, int head_group,
                   void* stream);

/*
 * attn_fwd_ext -- attn_fwd with the mask and bias variants.
 *
 * Same arguments, layouts and errors as attn_fwd, plus:
 *   window       : sliding-window width in keys, >= 0 (0: no window). Query
 *                  row i (local index) then sees keys j with i-window < j <= i
 *                  (causal) or |i-j| < window (non-causal): the sliding-window
 *                  attention of lnrk.cn/news/11729 §2.5.
 *   n_global     : >= 0. The first n_global query rows of every sequence see
 *                  every key of it (the "global tokens" of the same section,
 *                  whose listing gives the first queries full attention).
 *   alibi_slopes : NULL, or a DEVICE float32 array of H slopes (4-byte
 *                  aligned): score_ij gets -slope_h * |i - j| added after
 *                  scaling -- the ALiBi linear bias named in
 *                  jianying88.com/news/49672 §5.1.
 * window < 0 or n_global < 0 -> ATTN_ERR_SHAPE. With window == n_global == 0
 * and alibi_slopes == NULL the result equals attn_fwd's.
 */
int attn_fwd_ext(const void* q, const void* k, const void* v, void* out, float* lse,
                 int B, int H, int S, int D, int causal, float scale, int dtype,
                 const int32_t* cu_seqlens, int window, int n_global,
                 const float* alibi_slopes, void* stream);

/*
 * attn_fwd_ext_tuned -- attn_fwd_ext with its launch shape fixed by the caller
 * (for tests that must reach every kernel instance, and for sweeps).
 *
 * Same arguments, layouts, semantics and errors as attn_fwd_ext, plus:
 *   tile_rows  : 0 lets the library choose as attn_fwd_ext does; 128 runs the
 *                4-wave mask-variant kernel; 256 runs the 8-wave ping-pong
 *                kernel, which takes the ALiBi bias alone: it needs D == 128,
 *                window == n_global == 0 and alibi_slopes != NULL. Anything
 *                else: ATTN_ERR_UNSUPPORTED.
 *   head_group : as in attn_fwd_tuned (0: the library's choice; negative:
 *                ATTN_ERR_SHAPE).
 * The two kernels agree to rounding (they sum a row's keys in the same order
 * but take the running maximum at different steps).
 */
int attn_fwd_ext_tuned(const void* q, const void* k, const void* v, void* out, float* lse,
                       int B, int H, int S, int D, int causal, float scale, int dtype,
                       const int32_t* cu_seqlens, int window, int n_global,
                       const float* alibi_slopes, int tile_rows, int head_group, void* stream);

/*
 * attn_fwd_fp8 -- attn_fwd on FP8 inputs.
 *
 * jianying88.com/news/49672 §3 mentions FP8 attention (less memory, a small
 * speed gain); this is that variant for D = 128: q, k, v hold OCP E4M3 codes
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; 448 the largest
 * finite value), one byte per element, in attn_fwd's layouts; each tensor
 * carries one float scale, so the operation is
 *   out = softmax(scale * (descale_q Q)(descale_k K)^T + mask) (descale_v V).
 * out is written in `out_dtype` (ATTN_DTYPE_BF16 or ATTN_DTYPE_FP16), lse in
 * fp32 as attn_fwd. Both products run on the 8-bit matrix core with fp32
 * accumulation; the probabilities are rounded to E4M3 (after scaling by
 * 2^4) for the P V product, so O carries up to 2^-4 relative error per term
 * of its weighted sum (the LSE does not: it sums the fp32 probabilities).
 * D other than 128 -> ATTN_ERR_UNSUPPORTED; a non-finite descale or scale
 * product -> ATTN_ERR_SCALE. Other arguments and errors as attn_fwd.
 */
int attn_fwd_fp8(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                 int H, int S, int D, int causal, float scale, float descale_q, float descale_k,
                 float descale_v, int out_dtype, const int32_t* cu_seqlens, void* stream);

/*
 * attn_decode -- attention of a few new query rows against a KV cache.
 *
 * The decode step of autoregressive generation: the cache holds keys and
 * values of earlier tokens in the [batch, heads, seq_len, head_dim] layout of
 * lnrk.cn/news/11729 §2.2 (which notes that it grows by one row per
 * generated token); the new rows attend to it with the definition of
 * mlqm.cn/news/343191 chapter 1.
 *   q         : contiguous (B, Sq, H, D) array of `dtype` (Sq new rows per sequence).
 *   k_cache,
 *   v_cache   : contiguous (B, H, S_max, D) arrays of `dtype`.
 *   seqlens_k : int32 DEVICE array of B valid cache lengths, or NULL (all
 *               S_max). Values are clamped to [0, S_max]; rows past a
 *               sequence's length are never read.
 *   out       : contiguous (B, Sq, H, D) array of `dtype`.
 *   lse       : contiguous (B, H, Sq) float32 (natural log), or NULL.
 * Query row i of sequence b sits at position L_b - Sq + i. Without causality
 * it sees all L_b valid rows; with causal != 0 it sees rows j <= L_b - Sq + i.
 * A row that sees none (L_b == 0, or L_b < Sq under causality) gets out = 0
 * and lse = -inf.
 *   D : 64 or 128.  scale : any finite float.  B, Sq, S_max >= 0, H >= 1;
 *   S_max * D * 2 bytes must stay below 4 GiB - 1 MiB.
 *   num_splits : 0 picks the split count from the shapes; n > 0 asks for at
 *               most n splits of the cache rows per query row (capped at 256).
 *   workspace  : DEVICE memory of at least attn_decode_workspace_size(...)
 *               bytes for the same B, H, Sq, S_max, D and num_splits,
 *               16-byte aligned, owned by the caller and used as scratch
 *               (partial results of the splits) until the stream reaches the
 *               end of the call. May be NULL when that size is 0 (one split).
 * Two kernels run on `stream` when there is more than one split (per-split
 * partial results, then their log-sum-exp merge), one otherwise. Errors as
 * attn_fwd, plus ATTN_ERR_WORKSPACE.
 */
size_t attn_decode_workspace_size(int B, int H, int Sq, int S_max, int D, int num_splits);

int attn_decode(const void* q, const void* k_cache, const void* v_cache,
                const int32_t* seqlens_k, void* out, float* lse, int B, int H, int Sq,
                int S_max, int D, int causal, float scale, int dtype, int num_splits,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_noalloc -- attn_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, and harnesses
 * that forbid hipMalloc. It takes no workspace; the split partials live in a
 * fixed array of the library, 16 MiB per GPU, which each GPU that runs this
 * call holds until the process ends. The call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine); its first call on a device looks up
 * that device's array address once (hipGetSymbolAddress).
 *
 * Arguments, layouts, semantics and results as attn_decode, without
 * workspace / workspace_bytes. num_splits = 0 chooses the split count as
 * attn_decode does and, when the partials of that choice would not fit in
 * the array ((D + 1) * 4 bytes per split per query row), uses the largest
 * count that fits (a single split needs none); an explicit num_splits whose
 * partials do not fit returns ATTN_ERR_SCRATCH with nothing enqueued.
 * Nothing in the array needs clearing: every call writes each partial it
 * later reads. Calls on one GPU share its array, so calls that can overlap on
 * one GPU (different streams, or another thread between enqueue and
 * completion) race and give wrong results: order them on one stream.
 */
int attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* seqlens_k, void* out, float* lse, int B, int H, int Sq,
                        int S_max, int D, int causal, float scale, int dtype, int num_splits,
                        void* stream);

/*
 * attn_bwd -- gradients of attn_fwd with respect to q, k and v.
 *
 * The backward(grad_output) step that mlqm.cn/news/343191 §3.3 reserves for
 * the fused operation: given the forward's inputs, its output `out` and its
 * log-sum-exp `lse`, and the gradient `dout` of a loss with respect to out,
 *   dv = P^T dout,  dS = P * (dout v^T - rowsum(dout * out)),
 *   dq = scale * dS k,  dk = scale * dS^T q,
 * per (sequence, head), with P recomputed from q, k and lse tile by tile
 * (it never reaches memory). Masks and layouts are attn_fwd's (padded
 * (B, S, H, D) or packed (T, H, D) with cu_seqlens; lse (B, H, S) or (H, T),
 * REQUIRED here). dout, dq, dk, dv have q's layout and dtype; dq, dk, dv are
 * written (rounded to nearest even) and must not overlap the inputs.
 *   workspace : DEVICE memory of attn_bwd_workspace_size(B, H, S, packed)
 *               bytes (two fp32 per row and head), 16-byte aligned, owned by
 *               the caller, used until the stream passes the call.
 * Kernels on `stream`: dq (which also fills the workspace with
 * rowsum(dout * out) and lse * log2(e)), then dk and dv (two launches for
 * D = 128, one for D = 64). No atomics: results are
 * deterministic. Errors as attn_fwd, plus ATTN_ERR_NULL for a missing lse,
 * dout, dq, dk or dv and ATTN_ERR_WORKSPACE.
 */
size_t attn_bwd_workspace_size(int B, int H, int S, int packed);

int attn_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, int B, int H, int S, int D,
             int causal, float scale, int dtype, const int32_t* cu_seqlens, void* workspace,
             size_t workspace_bytes, void* stream);

/* Human-readable text of a status code (static storage; never NULL). */
const char* attn_strerror(int status);

/*
 * attn_check_cu_seqlens -- debug validator of packed-mode offsets.
 * Copies cu_seqlens (B+1 int32, device) to the host on `stream`,
 * synchronizes it and checks cu[0] == 0, cu non-decreasing, cu[B] == T.
 * Returns ATTN_OK, ATTN_ERR_SEQLENS, ATTN_ERR_NULL / ATTN_ERR_SHAPE for bad
 * arguments, or ATTN_ERR_LAUNCH if the copy fails.
 */
int attn_check_cu_seqlens(const int32_t* cu_seqlens, int B, int T, void* stream);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int attn_version(void);

/*
 * The hipError_t of the most recent kernel launch (or device look-up) of
 * any attn_* call on the calling thread: 0 after a successful launch, the
 * runtime's code after one that returned ATTN_ERR_LAUNCH. Launches first clear
 * an error that an earlier runtime call of the thread left pending, so the
 * code is the launch's own.
 */
int attn_last_hip_error(void);

/*
 * Measurement support (not part of the attention path): enqueues on `stream`
 * waves on every CU that record, for CU slot s (s = 128 * XCD + the CU's
 * HW_ID bits [14:8]: shader engine, array and CU), the CU's shader-clock
 * counter (cycles of its shader clock; the counter stops while the CU is
 * clock-gated) in dst[2s] and the 100 MHz real-time counter in dst[2s + 1].
 * dst is DEVICE memory for 2048 uint64_t, 8-byte aligned (else ATTN_ERR_NULL
 * / ATTN_ERR_ALIGN); slots of absent CUs are left as they were. Counters of
 * different CUs do not share an origin: compare two samples per slot. Over a
 * busy region between them, (dst'[2s] - dst[2s]) / (dst'[2s+1] - dst[2s+1]) *
 * 100 MHz is that CU's average shader clock. A kernel can start on CUs the
 * previous kernel of the stream has released while that kernel still runs,
 * so a sample meant to follow earlier work must be enqueued after a barrier
 * (an event record) on the stream.
 */
int attn_clock_sample(uint64_t* dst, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SDPA08_ATTN_H */
