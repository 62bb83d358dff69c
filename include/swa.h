/*
 * swa.h - C ABI of the MI355X (gfx950) sliding-window attention library.
 *
 * The operation: causal softmax attention in which query t attends the first
 * s tokens (attention sinks) and its r most recent tokens including itself,
 * each key once,
 *     U(t) = { i <= t : i < s or i >= t - r + 1 },   |U(t)| = min(t+1, s+r),
 *     O_t  = sum_{i in U(t)} softmax_i(scale * q_t . k_i) v_i .
 * Sources: the SWA formula and the fixed first s = 4 sink tokens in the
 * "带 Sink 的滑动窗口注意力" section of the hyper.ai summary of arXiv
 * 2608.28444; the sink + recent cache composition (eq:attn-fixed-streaming),
 * the rolling buffer (eq:attn-fixed-rolling), chunked prefill and RoPE
 * re-positioning inside the cache on the t6page page "滑窗与固定稀疏";
 * softmax attention, eq.(1) of section 2.1 of the Blurry Window Attention
 * page (arXiv 2606.09862).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers to contiguous row-major arrays
 *    whose base address is 16-byte aligned.  Element type is desc->dtype
 *    (fp32 or bf16); the output has the input's type.  The caller owns every
 *    buffer (inputs, outputs, caches, workspaces); the library never
 *    allocates, frees or synchronises.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue
 *    kernels on it and return; device-side results are ready after the
 *    caller synchronises the stream.
 *  - Return value: SWA_OK (0) or a negative status.  Arguments are validated
 *    on the host before any HIP call; a rejected call enqueues nothing and
 *    leaves a message in swa_last_error() (per calling thread).
 *  - GQA: q-head h reads kv-head h / (Hq / Hkv) (contiguous groups).
 *  - Rolling cache layout [B, Hkv, s + r, d]: token p lives in slot p when
 *    p < s, else in slot s + (p mod r) (the sink slots in front of an r-slot
 *    rolling buffer written at p mod r).  Tokens below s go only to their
 *    sink slot.
 */
#ifndef SWA_H_
#define SWA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SWA_ABI_VERSION 1

enum swa_status {
    SWA_OK = 0,
    SWA_ERR_INVALID_ARG = -1,  /* null pointer, bad size, misalignment, workspace too small */
    SWA_ERR_UNSUPPORTED = -2,  /* valid but not built: d not in {64, 128}, unknown dtype */
    SWA_ERR_HIP = -3           /* a HIP launch or runtime call failed */
};

enum swa_dtype { SWA_F32 = 0, SWA_BF16 = 1 };

typedef struct swa_desc {
    int32_t B;          /* batch (sequences), >= 1 */
    int32_t Hq;         /* query heads, >= 1 */
    int32_t Hkv;        /* key/value heads, >= 1, divides Hq */
    int32_t d;          /* head dimension: 64 or 128 */
    int32_t s;          /* sink tokens, >= 0 */
    int32_t r;          /* recent tokens including the query's own, >= 1 */
    int32_t dtype;      /* enum swa_dtype */
    float scale;        /* score scale, > 0 (usually 1/sqrt(d)) */
    float rope_base;    /* 0: no rotary embedding; > 0: RoPE base (bf16 only) */
} swa_desc;

/*
 * Bytes of device workspace swa_prefill needs for these arguments: 0 (the
 * prefill kernels use none; kept so callers can size a workspace
 * generically).
 */
size_t swa_prefill_workspace_bytes(const swa_desc* desc, int64_t L);

/*
 * RoPE re-positioning (the StreamingLLM paragraph after
 * eq:attn-fixed-streaming on the t6page page "滑窗与固定稀疏"): for query t
 * the keys of U(t), in temporal order, sit at positions 0 .. |U(t)|-1 and the
 * query at |U(t)|-1.  Rotary scores depend only on the difference of the two
 * positions, so a window key i sits at its true distance t - i and sink j
 * at min(t, s+r-1) - j.  The library therefore takes every key rotated ONCE
 * at its own token's position (with rope_base > 0, the keys given to
 * swa_prefill, stored by swa_cache_append and read by swa_decode /
 * swa_decode_step are such keys) and turns the query itself: to t for
 * window keys, to min(t, s+r-1) for sinks.  Queries are given unrotated.
 *
 * swa_rope_keys rotates n key rows per (batch, kv-head) (k, k_rot:
 * [B, Hkv, n, d], bf16; row i is the token at position pos0 + i) to their
 * positions: dimension j pairs with j + d/2 and the pair turns by
 * position * rope_base^(-2j/d) (fp64 angle, fp32 rotation, bf16 result).
 * k_rot may equal k (in place).  Errors: SWA_ERR_INVALID_ARG (rope_base not
 * > 0, null/misaligned pointer, n < 1, pos0 < 0), SWA_ERR_UNSUPPORTED (d,
 * dtype other than bf16), SWA_ERR_HIP.
 */
int swa_rope_keys(const swa_desc* desc, const void* k, int64_t n, int64_t pos0, void* k_rot, void* stream);

/*
 * Banded flash-style prefill of L query rows.
 *   q, o: [B, Hq, L, d];  k, v: [B, Hkv, L, d]  (the chunk's own tokens).
 * Plain prefill: k_cache = v_cache = NULL and pos0 = 0; row i is position i.
 * Chunked prefill: rows are positions pos0 .. pos0+L-1, and k_cache/v_cache
 * ([B, Hkv, s + r, d], the rolling cache) hold tokens 0 .. pos0-1 written by
 * swa_cache_append; the cache is read, not written (append the chunk after
 * this call, on the same stream).  pos0 > 0 requires a cache.
 * RoPE (desc->rope_base > 0, see swa_rope_keys): k and the cache's keys are
 * rotated at their tokens' positions, q is not; the kernel rotates each
 * query to t for the window and to min(t, s+r-1) for the sinks.  workspace
 * may be NULL (swa_prefill_workspace_bytes() is 0).
 * Errors: SWA_ERR_INVALID_ARG (null or misaligned pointer, L < 1, pos0 < 0,
 * pos0 > 0 without a cache, workspace too small, s < 0, r < 1, Hq % Hkv,
 * scale <= 0), SWA_ERR_UNSUPPORTED (d, dtype, RoPE with fp32), SWA_ERR_HIP.
 */
int swa_prefill(const swa_desc* desc, const void* q, const void* k, const void* v, void* o, int64_t L,
                const void* k_cache, const void* v_cache, int64_t pos0,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Write tokens pos0 .. pos0+n-1 (k_new, v_new: [B, Hkv, n, d]) into the
 * rolling cache (k_cache, v_cache: [B, Hkv, s + r, d]) at their slots.  When
 * n > r several tokens of the call map to one recent slot; only the last of
 * them (the one that survives in a token-by-token append) is written, so
 * every slot has one writer.  Bytes are copied unchanged.
 * Errors: SWA_ERR_INVALID_ARG (null/misaligned pointer, n < 1, pos0 < 0,
 * bad shape fields), SWA_ERR_UNSUPPORTED (d, dtype), SWA_ERR_HIP.
 */
int swa_cache_append(const swa_desc* desc, const void* k_new, const void* v_new, int64_t n, int64_t pos0,
                     void* k_cache, void* v_cache, void* stream);

/*
 * One chunk of the streaming prefill with the append fused in: the rows of
 * swa_prefill over (k_cache, v_cache) + the chunk (chunked prefill on the
 * t6page page), and, in the same launch, the cache after appending the
 * chunk (swa_cache_append's result) written to a second cache pair
 * (k_next, v_next, [B, Hkv, s + r, d]); k_cache / v_cache are only read.
 * The call needs every rolling slot that holds a token afterwards to come
 * from the chunk: L >= r, or pos0 <= s.  Then k_next / v_next receive the
 * chunk's surviving tokens at their slots and the sink slots below pos0
 * from the cache; slots that hold no token after the call are not written.
 * Alternating two cache pairs, chunk by chunk, gives the rows and caches of
 * swa_prefill + swa_cache_append without the separate copy launch.
 * bf16 only; the cache pairs must not overlap (k_next != k_cache, ...).
 * Errors: those of swa_prefill, SWA_ERR_INVALID_ARG for L < r with
 * pos0 > s, a null or misaligned next cache, or next == current,
 * SWA_ERR_UNSUPPORTED for fp32.
 */
int swa_prefill_append(const swa_desc* desc, const void* q, const void* k, const void* v, void* o, int64_t L,
                       const void* k_cache, const void* v_cache, int64_t pos0, void* k_next, void* v_next,
                       void* stream);

/*
 * Dilated sliding window (prefill, no cache, no RoPE): query t attends the
 * sinks 0 .. min(s, t+1)-1 and the r positions t, t - dilation, ...,
 * t - (r-1) dilation that are >= s (the glossary entry on dilated SWA and
 * the Longformer section of the t6page page "滑窗与固定稀疏": attended
 * positions skip dilation-1 tokens, the number of keys is unchanged).
 * Layouts as for swa_prefill.  dilation = 1 is swa_prefill without a cache.
 * Otherwise the rows of each residue class mod dilation from position s on
 * form an ordinary window over the sinks; they are read and written in
 * place (row stride dilation * d), every class in one launch, after one
 * launch for the s sink rows.  No workspace: workspace may be NULL, and
 * swa_prefill_dilated_workspace_bytes() returns 0 (kept for callers that
 * size one).  Errors: those of swa_prefill, SWA_ERR_INVALID_ARG for
 * dilation < 1 or > 65536, SWA_ERR_UNSUPPORTED with RoPE.
 */
size_t swa_prefill_dilated_workspace_bytes(const swa_desc* desc, int64_t L, int32_t dilation);
int swa_prefill_dilated(const swa_desc* desc, int32_t dilation, const void* q, const void* k, const void* v, void* o,
                        int64_t L, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Task-bound global tokens on the sliding window with sinks (the Longformer
 * section and the glossary entry on global tokens of the t6page page
 * "滑窗与固定稀疏": a few tokens, chosen by the task, see the whole sequence
 * and are seen by all of it), in causal form.  globals: ng HOST positions
 * (0 <= ng <= SWA_MAX_GLOBALS), strictly increasing, each in 0 .. L-1.  A row
 * t in globals attends every key 0 .. t; any other row attends U(t) plus the
 * global positions g <= t, each key once (a global among the sinks or inside
 * the window adds nothing).  Layouts as for swa_prefill without a cache;
 * bf16, no RoPE, up to 16 q-heads per kv-head.  ng = 0 is swa_prefill.
 * Gathers the global keys and values into one 64-key block, runs the banded
 * prefill with that block as one more key tile (each row keeps the globals
 * outside its key set), then computes the global rows as dense causal rows,
 * 16 / (Hq/Hkv) of them per decode launch.  Workspace:
 * swa_prefill_global_workspace_bytes(desc, L, ng) bytes (the gathered keys
 * and values, one byte per position, the dense rows' split partials).
 * Errors: those of swa_prefill, SWA_ERR_INVALID_ARG for bad globals or a
 * short workspace, SWA_ERR_UNSUPPORTED for fp32, RoPE or wide GQA groups.
 */
#define SWA_MAX_GLOBALS 64
size_t swa_prefill_global_workspace_bytes(const swa_desc* desc, int64_t L, int32_t ng);
int swa_prefill_global(const swa_desc* desc, const void* q, const void* k, const void* v, void* o, int64_t L,
                       const int32_t* globals, int32_t ng, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Split-K decode.  Bytes of workspace swa_decode needs for n_split splits of
 * the s + r slots (0 = the library's choice for this shape):
 * B * Hq * n_split * (d + 2) * 4 bytes, or 0 for one split (the split
 * kernel then writes o itself and workspace may be NULL).
 */
size_t swa_decode_workspace_bytes(const swa_desc* desc, int32_t n_split);

/*
 * One decode step: the query q ([B, Hq, d]) of the token at position T-1
 * attends the cache ([B, Hkv, s + r, d]) holding tokens 0 .. T-1 (append the
 * token first), i.e. U(T-1).  Slot order does not matter to softmax
 * attention over a set, so slots are read in physical order.  Writes
 * o ([B, Hq, d]).  n_split: 0 = the library's choice, else 1 .. 64.
 * With rope_base > 0 (up to 8 q-heads per kv-head) the cache holds keys
 * rotated at their tokens' positions (see swa_rope_keys) and q is given
 * unrotated; it is turned to T-1 for the window slots and to
 * min(T-1, s+r-1) for the sink slots (the StreamingLLM re-positioning).
 * Errors: SWA_ERR_INVALID_ARG (null/misaligned pointer, T < 1, workspace too
 * small, n_split out of range), SWA_ERR_UNSUPPORTED (d, dtype other than
 * bf16), SWA_ERR_HIP.
 */
int swa_decode(const swa_desc* desc, const void* q, const void* k_cache, const void* v_cache, int64_t T,
               void* o, int32_t n_split, void* workspace, size_t workspace_bytes, void* stream);

/*
 * One generation step in one launch: appends token T-1 (k_new, v_new:
 * [B, Hkv, d], the same bytes swa_cache_append would take with n = 1,
 * pos0 = T-1) to the cache and decodes its query q over the cache holding
 * tokens 0 .. T-1.  The result and the cache afterwards equal those of
 * swa_cache_append followed by swa_decode (the token is read from k_new /
 * v_new, and written to its slot, in the same kernel); workspace as for
 * swa_decode.  With rope_base > 0, k_new is rotated at position T-1.  Errors: those of swa_decode, and SWA_ERR_INVALID_ARG for a
 * null or misaligned k_new / v_new.
 */
int swa_decode_step(const swa_desc* desc, const void* q, const void* k_new, const void* v_new, void* k_cache,
                    void* v_cache, int64_t T, void* o, int32_t n_split, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * swa_decode_step without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, kernels, results and errors as swa_decode_step; with more than
 * one split the per-split partial results go to a static device array of
 * SWA_NOALLOC_SCRATCH_BYTES bytes that the library holds on each GPU it runs
 * on until the process ends (the array of the device current at the call).
 * Calls whose partials need more (B * Hq * n_split * (d + 2) * 4 bytes) are
 * rejected with SWA_ERR_INVALID_ARG before anything is enqueued.  All calls
 * on one GPU share that array and it keeps the last call's contents: calls
 * that overlap on one GPU (other streams, other threads) race on it, so
 * order them on one stream.  No hipMalloc, hipFree or allocating library
 * routine is called.
 */
#define SWA_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int swa_decode_step_noalloc(const swa_desc* desc, const void* q, const void* k_new, const void* v_new,
                            void* k_cache, void* v_cache, int64_t T, void* o, int32_t n_split, void* stream);

/*
 * Backward of swa_prefill without a cache or RoPE (training): the gradients
 * of the rows O with respect to q, k and v for an upstream gradient dout.
 * The rows are softmax over U(t) of scale * q_t . k_i weighting v_i (the
 * hyper.ai summary's section on sliding-window attention with sinks,
 * eq:attn-fixed-streaming on the t6page page); the gradient is that
 * definition's derivative:
 *   dV_i = sum_t P_ti dout_t,  dS_ti = P_ti (dout_t . v_i - dout_t . o_t),
 *   dQ_t = scale sum_i dS_ti k_i,  dK_i = scale sum_t dS_ti q_t,
 * over the pairs with i in U(t), dK and dV summed over the q-heads of each
 * kv-head.  o is the forward output the caller holds (it enters
 * dout_t . o_t; pass swa_prefill's output).  P is recomputed from q and k.
 * Inputs bf16 (desc->dtype = SWA_BF16): q, o, dout [B, Hq, L, d]; k, v
 * [B, Hkv, L, d].  Outputs fp32, caller-owned, fully overwritten: dq
 * [B, Hq, L, d]; dk, dv [B, Hkv, L, d].  Workspace: at least
 * swa_backward_workspace_bytes() bytes (per-row log-sum-exp and
 * dout . o, then partial dK and dV sums of the key tiles whose queries are
 * split into segments), 16-byte aligned.  No atomics: the partial sums are
 * added in a fixed order, so repeated calls give identical gradients.
 * Errors: SWA_ERR_INVALID_ARG (null or misaligned pointer, L < 1, short
 * workspace, shape fields), SWA_ERR_UNSUPPORTED (d, fp32 inputs, RoPE),
 * SWA_ERR_HIP.
 */
size_t swa_backward_workspace_bytes(const swa_desc* desc, int64_t L);
int swa_backward(const swa_desc* desc, const void* q, const void* k, const void* v, const void* o, const void* dout,
                 float* dq, float* dk, float* dv, int64_t L, void* workspace, size_t workspace_bytes, void* stream);

/* The split count swa_decode uses for n_split = 0. */
int32_t swa_decode_default_splits(const swa_desc* desc);

/* Static text for a status code. */
const char* swa_status_str(int status);

/* Message of the last failed call on this thread ("" if none). */
const char* swa_last_error(void);

/* SWA_ABI_VERSION of the loaded library. */
int swa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SWA_H_ */
