/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention (KDA) core.
 *
 * The operation (per sequence n, per head h, tokens t in order):
 *
 *   S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T
 *   o_t = scale * S_t^T q_t
 *
 * with S a d_k x d_v fp32 state whose rows are key channels, exp(g_t) a
 * per-key-channel retention, beta_t a scalar write strength, and the readout
 * taken after the token's own write.  Sources: "Understanding Kimi K3's
 * attention" (dhruvpendharkar.github.io) -- symbol table, state-update and
 * readout equations, and the g_min = -5 bound on the log-decay; "KDA: the
 * memory matrix" (kimi-k3-course.pages.dev, lesson 2) -- the three per-token
 * operations and the read-after-write rule; "Inside Kimi K3" (flozi.net),
 * section "Sequence mixing" -- chunkwise prefill with state passed between
 * chunks, a causal intra-chunk matrix that includes its diagonal, 16-token
 * tiles whose cumulative log-decay stays above -80, and KDA state restored at
 * a token boundary for prefix reuse.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers, row-major and contiguous.
 *     q, k, v, g, o and the state buffers must be 16-byte aligned (the
 *     kernels use 16-byte vector accesses); beta and cu_seqlens need only
 *     their natural 4-byte alignment.  The caller owns every buffer; the library
 *     allocates no device memory and keeps no mutable global state (except
 *     the one flag word of the KDA_VALIDATE check below).
 *   - Element offsets are 64-bit; token counts up to 2^31 - 1 per call.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *     asynchronous on it; a KDA_OK return means the work was launched.
 *   - Every argument is validated on the host before any HIP call, so an
 *     error return has touched no device memory.  Errors are returned, never
 *     printed or raised; nothing aborts.
 *   - Device-side preconditions: g in [-5, 0] (the chunked kernels rely on
 *     a 16-token cumulative log-decay >= -80), beta in [0, 1], finite inputs,
 *     and cu_seqlens non-decreasing from 0 to total_tokens.  By default they
 *     are not checked: a violation changes the numbers, never the memory the
 *     kernels touch (sequence bounds read from cu_seqlens are clamped to
 *     [0, total_tokens] on the device).  When the environment variable
 *     KDA_VALIDATE is "1" at the time of a call, kda_prefill and
 *     kda_decode_step first read g, beta and cu_seqlens on the device, wait
 *     for the stream, and return KDA_ERR_DOMAIN without launching the
 *     computation if one of them is violated (NaN in g or beta counts as a
 *     violation).  That mode blocks the calling thread, cannot be used under
 *     graph capture, and uses one __device__ flag word per GPU, so two calls
 *     validating on one GPU at the same time may report each other's
 *     violation.
 *   - qkv_dtype selects the dtype of q, k, v and o: KDA_DTYPE_BF16 (bf16
 *     storage, bf16 MFMA products with fp32 accumulation, fp32 state) or
 *     KDA_DTYPE_F32 (fp32 throughout, fp32 MFMA).  g, beta and the state are
 *     always fp32.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 4

typedef enum {
    KDA_DTYPE_F32 = 0,
    KDA_DTYPE_BF16 = 1
} kda_dtype;

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL_POINTER = 1, /* a required pointer is NULL                       */
    KDA_ERR_BAD_SHAPE = 2,    /* negative / inconsistent sizes                     */
    KDA_ERR_UNSUPPORTED = 3,  /* valid but not built: (dtype, d_k, d_v, chunk)     */
    KDA_ERR_MISALIGNED = 4,   /* a pointer breaks the alignment rule above         */
    KDA_ERR_WORKSPACE = 5,    /* workspace smaller than kda_prefill_workspace_bytes */
    KDA_ERR_HIP = 6,          /* the HIP runtime reported an error at launch       */
    KDA_ERR_DOMAIN = 7,       /* g, beta or cu_seqlens break the preconditions;    */
                              /* returned only when KDA_VALIDATE=1                 */
    KDA_ERR_SCRATCH = 8       /* kda_prefill_ex_noalloc: the call needs more than  */
                              /* kda_noalloc_scratch_bytes() of workspace          */
} kda_status;

/* KDA_ABI_VERSION of the built library. */
int32_t kda_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *kda_status_string(int32_t status);

/* 1 if (qkv_dtype, d_k, d_v, chunk_size) has a built prefill kernel, else 0.
 * chunk_size 0 asks for the library default (16 for both dtypes). */
int32_t kda_prefill_supported(int32_t qkv_dtype, int32_t d_k, int32_t d_v,
                              int32_t chunk_size);

/* 1 if (qkv_dtype, d_k, d_v) has a built decode kernel, else 0. */
int32_t kda_decode_supported(int32_t qkv_dtype, int32_t d_k, int32_t d_v);

/*
 * Bytes of device workspace kda_prefill needs for these sizes (0 = none;
 * then workspace may be NULL).  Returns 0 as well for unsupported or invalid
 * sizes, which kda_prefill itself rejects.  The figure is for a dense batch
 * (cu_seqlens NULL) on the current device; a call with cu_seqlens needs no
 * workspace.  The only user is the sequence-segment scan (see
 * kda_prefill_desc.segments), which the library picks for dense batches with
 * few (sequence, head) recurrences per compute unit: about (G - 1) * 128 KiB
 * per (sequence, head) for G segments per sequence (32 MiB for one
 * 1,048,576-token sequence of 16 heads on 256 compute units, G = 17).
 */
size_t kda_prefill_workspace_bytes(int32_t num_seqs, int64_t total_tokens,
                                   int32_t num_heads, int32_t d_k, int32_t d_v,
                                   int32_t qkv_dtype, int32_t chunk_size);

/*
 * kda_prefill -- the whole recurrence over a packed batch of sequences,
 * computed chunkwise: inside a chunk the tokens are processed in parallel
 * (cumulative log-decay per chunk, the causal intra-chunk matrix including
 * its diagonal, and the triangular solve of I + strictly-lower A), and the
 * state is passed from chunk to chunk ("Inside Kimi K3", flozi.net, section
 * "Sequence mixing"; "Hybrid Attention", kimi-k3.adriaflores.com, section
 * "But isn't a recurrent update sequential?").  The result equals the
 * token-by-token recurrence up to rounding.
 *
 *   num_seqs      N >= 0 sequences.
 *   total_tokens  T_total >= 0 tokens over all sequences.
 *   num_heads     H >= 1;  d_k, d_v: head dims (see kda_prefill_supported).
 *                 16 token rows of all heads must stay below 2^31 bytes in
 *                 fp32 (H * max(d_k, d_v) * 64 <= INT32_MAX: H <= 262,143 at
 *                 d = 128), else KDA_ERR_UNSUPPORTED (the kernels address a
 *                 chunk's rows with 32-bit offsets); T_total <= INT32_MAX.
 *   qkv_dtype     kda_dtype of q, k, v and o.
 *   chunk_size    tokens per chunk (16, 32 or 64), or 0 for the default.
 *   scale         readout scale; 1.0f gives o_t = S_t^T q_t exactly.
 *   q, k          [T_total, H, d_k]  qkv_dtype
 *   v             [T_total, H, d_v]  qkv_dtype
 *   g             [T_total, H, d_k]  fp32 log-decay (alpha = exp(g))
 *   beta          [T_total, H]       fp32
 *   initial_state [N, H, d_k, d_v]   fp32, or NULL for zeros
 *   cu_seqlens    [N + 1] int32 device array of sequence offsets (cu[0] = 0,
 *                 cu[N] = T_total), or NULL for N equal-length sequences of
 *                 T_total / N tokens (T_total must then divide by N).
 *                 Empty sequences are allowed: their final state is their
 *                 initial state and they produce no outputs.
 *   o             [T_total, H, d_v]  qkv_dtype, written.  Must not overlap
 *                 an input; o equal to an input pointer is rejected with
 *                 KDA_ERR_BAD_SHAPE (partial overlap is not detected).
 *   final_state   [N, H, d_k, d_v]   fp32, written, or NULL to skip.  May be
 *                 the same pointer as initial_state (in-place carry).
 *   workspace     device buffer of workspace_bytes (may be NULL when the
 *                 workspace query returns 0).
 *
 * Errors: KDA_ERR_NULL_POINTER, KDA_ERR_BAD_SHAPE, KDA_ERR_UNSUPPORTED,
 * KDA_ERR_MISALIGNED, KDA_ERR_WORKSPACE, KDA_ERR_HIP, and KDA_ERR_DOMAIN
 * (only under KDA_VALIDATE=1).  N = 0 or T_total = 0
 * with N > 0 is valid: final_state receives the initial state (or zeros).
 */
kda_status kda_prefill(int32_t num_seqs, int64_t total_tokens,
                       int32_t num_heads, int32_t d_k, int32_t d_v,
                       int32_t qkv_dtype, int32_t chunk_size, float scale,
                       const void *q, const void *k, const void *v,
                       const float *g, const float *beta,
                       const float *initial_state, const int32_t *cu_seqlens,
                       void *o, float *final_state,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_prefill_ex -- the prefill entry points in one call, with the kernel
 * plan explicit: for measurements and tests that compare kernels, and for
 * callers that want to fix the plan.  kda_prefill, kda_prefill_fused and
 * kda_prefill_checkpointed are this call with a zero plan (the library's
 * choice, which depends only on the sizes and the device's compute-unit
 * count).  No plan changes what is computed; kernels and slab widths change
 * the rounding order at most (results stay deterministic for a given plan;
 * slab widths of one kernel are bitwise identical).
 *
 * Sequence-segment scan.  A dense batch whose (sequence, head) recurrences
 * are too few to fill the device is cut into G segments per sequence.  The
 * state update is affine in the state ("Understanding Kimi K3's attention",
 * state-update equation), so each segment g is one map S_end = M_g S_start +
 * B_g.  Three launches: the maps of segments 1 .. G-2 are computed in
 * parallel, M_g and B_g of one segment by one workgroup (M_g from the
 * identity with v = 0, B_g from zero), beside segment 0, which runs from the
 * initial state with its outputs and leaves its end state; a short combine
 * chains start(g + 1) = M_g start(g) + B_g in fp32; segments 1 .. G-1 run
 * again from their start states with outputs.  This is the pages' state
 * passing between chunks ("Inside Kimi K3", section "Sequence mixing")
 * applied between segments, in parallel over segments instead of one chain.
 */
#define KDA_KERNEL_AUTO 0          /* the library's choice                          */
#define KDA_KERNEL_PIPELINED 1     /* wave-specialised pipeline: bf16, d = 128, chunk 16 */
#define KDA_KERNEL_CHUNK_STAGED 2  /* one chunk at a time by all waves: every built
                                      (dtype, d, chunk)                              */

typedef struct {
    int32_t num_seqs;             /* as kda_prefill                                   */
    int64_t total_tokens;
    int32_t num_heads;
    int32_t d_k;
    int32_t d_v;
    int32_t qkv_dtype;
    int32_t chunk_size;           /* 16, 32, 64 or 0 (default 16)                     */
    float scale;
    int32_t fused;                /* 1: kda_prefill_fused semantics (raw q, k; z and   */
                                  /*    a_log instead of g), else 0                   */
    int32_t checkpoint_interval;  /* 0: none; else as kda_prefill_checkpointed        */
    int64_t checkpoint_capacity;
    int32_t kernel;               /* KDA_KERNEL_*                                     */
    int32_t slab_columns;         /* value columns per workgroup: 0 = library choice,  */
                                  /* else one the kernel is built with (pipelined:    */
                                  /* 16, 32, 64, 128; chunk-staged d = 128: 32, 64,   */
                                  /* 128 by chunk)                                    */
    int32_t segments;             /* segment scan: 0 = library choice, 1 = off,        */
                                  /* 2 .. 256 = segments per sequence (dense batches,  */
                                  /* pipelined kernel, no fused gate or checkpoints,  */
                                  /* at least `segments` chunks per sequence)          */
} kda_prefill_desc;

typedef struct {
    const void *q, *k, *v;        /* as kda_prefill (fused: raw q and k)              */
    const float *g;               /* NULL when fused                                  */
    const void *z;                /* fused only: decay logits                          */
    const float *a_log;           /* fused only                                       */
    const float *beta;
    const float *initial_state;
    const int32_t *cu_seqlens;
    void *o;
    float *final_state;
    float *checkpoints;           /* with checkpoint_interval > 0                      */
} kda_prefill_tensors;

/* Workspace bytes of kda_prefill_ex for this description, for a dense batch
 * (cu_seqlens NULL) on the current device; 0 for invalid or unsupported
 * descriptions and whenever no segment scan runs. */
size_t kda_prefill_ex_workspace_bytes(const kda_prefill_desc *desc);

/* Errors as the flat entry points; KDA_ERR_NULL_POINTER for a NULL desc or
 * tensors; KDA_ERR_UNSUPPORTED for a kernel, slab width or segment count
 * that is not built or not applicable to the call (e.g. segments >= 2 with
 * cu_seqlens); KDA_ERR_BAD_SHAPE for negative plan fields or a workspace
 * equal to a tensor pointer. */
kda_status kda_prefill_ex(const kda_prefill_desc *desc, const kda_prefill_tensors *tensors, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * kda_prefill_ex_noalloc -- kda_prefill_ex for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): it takes no workspace and allocates nothing.  The
 * workspace the call needs (the segment scan's maps, kda_prefill_ex_
 * workspace_bytes) comes from one static device buffer of
 * kda_noalloc_scratch_bytes() bytes (64 MiB) that the library holds on every
 * GPU it runs on until the process ends.  Calls that need no workspace (packed
 * batches, direct chains) run as kda_prefill_ex; a call that needs more than
 * the buffer returns KDA_ERR_SCRATCH before any HIP call (the library's own
 * plans need at most 128 KiB per (sequence, head) per compute unit of the
 * device: 32 MiB on 256 compute units).  The buffer keeps the last call's
 * contents and every call on one GPU shares it: calls that overlap on one
 * GPU (other streams, other host threads) race on it and must be serialised
 * by the caller.  Results are bitwise those of kda_prefill_ex with the same
 * description.  Errors as kda_prefill_ex, plus KDA_ERR_SCRATCH.
 */
size_t kda_noalloc_scratch_bytes(void);
kda_status kda_prefill_ex_noalloc(const kda_prefill_desc *desc, const kda_prefill_tensors *tensors, void *stream);

/*
 * kda_prefill_checkpointed -- kda_prefill that also emits the state at every
 * checkpoint_interval tokens of each sequence, for restoring the KDA state at
 * a token boundary when a prompt prefix is reused ("Inside Kimi K3",
 * flozi.net, section "Sequence mixing": prefix caching must restore the
 * state at a token boundary).  All arguments shared with kda_prefill mean
 * the same and are validated the same way; in addition:
 *
 *   checkpoint_interval  tokens between checkpoints, >= 1 and a multiple of
 *                        the chunk size in use (chunk_size, or 16 for 0).
 *   checkpoints          [checkpoint_capacity, H, d_k, d_v] fp32 device
 *                        buffer, 16-byte aligned, written; may be NULL only
 *                        when checkpoint_capacity is 0.
 *   checkpoint_capacity  slots in checkpoints; must be at least
 *                        floor(total_tokens / checkpoint_interval), which
 *                        is never less than the number of checkpoints.
 *
 * Sequence n (tokens cu[n] .. cu[n+1]-1, length L_n) has floor(L_n /
 * checkpoint_interval) checkpoints.  Its checkpoint j (0-based) is the state
 * after its first (j + 1) * checkpoint_interval tokens, starting from its
 * initial state, and is stored in slot  sum_{m < n} floor(L_m / interval) + j.
 * Slots past the last checkpoint are not written.  A sequence whose length
 * is a multiple of the interval has its final state as its last checkpoint.
 * The buffer must not be an input or output pointer of the call (equal
 * pointers are rejected with KDA_ERR_BAD_SHAPE).
 *
 * Errors as for kda_prefill; KDA_ERR_BAD_SHAPE also for an interval that is
 * not a positive multiple of the chunk or a capacity below the bound above,
 * KDA_ERR_NULL_POINTER for a NULL buffer with capacity > 0.
 */
kda_status kda_prefill_checkpointed(int32_t num_seqs, int64_t total_tokens,
                                    int32_t num_heads, int32_t d_k, int32_t d_v,
                                    int32_t qkv_dtype, int32_t chunk_size,
                                    float scale, const void *q, const void *k,
                                    const void *v, const float *g,
                                    const float *beta,
                                    const float *initial_state,
                                    const int32_t *cu_seqlens, void *o,
                                    float *final_state,
                                    int32_t checkpoint_interval,
                                    float *checkpoints,
                                    int64_t checkpoint_capacity,
                                    void *workspace, size_t workspace_bytes,
                                    void *stream);

/* 1 if (qkv_dtype, d_k, d_v, chunk_size) has a built kda_prefill_fused
 * kernel, else 0 (chunk_size 0 = the default, 16). */
int32_t kda_prefill_fused_supported(int32_t qkv_dtype, int32_t d_k, int32_t d_v,
                                    int32_t chunk_size);

/*
 * kda_prefill_fused -- kda_prefill with the decay gate and the L2
 * normalisation of queries and keys computed inside the kernel, so that the
 * gate logits and the raw projections are read once and no normalised copy
 * or fp32 g is written beforehand.  The pages define q_t and k_t as
 * L2-normalised vectors (symbol table) and the log-decay as
 * g_t = g_min Sigmoid(e^{A_h} z_t) with g_min = -5 and a per-head log-scale
 * A_h ("Understanding Kimi K3's attention", gate equation).  Arguments as for
 * kda_prefill, except:
 *
 *   q, k    [T_total, H, d_k] qkv_dtype, NOT normalised: each (token, head)
 *           vector is divided by its L2 norm in the kernel (a zero vector
 *           stays zero).
 *   z       [T_total, H, d_k] qkv_dtype, the decay logits (16-byte aligned).
 *   a_log   [H] fp32, A_h of each head.
 *   (no g)  g = -5 / (1 + exp(-exp(a_log[h]) z)) per channel, in (-5, 0).
 *
 * Built for bf16 with d_k = d_v = 128 and chunk 16 (or 0); other
 * combinations return KDA_ERR_UNSUPPORTED.  z and a_log may be NULL only
 * when total_tokens is 0.  Under KDA_VALIDATE=1 only beta and cu_seqlens are
 * checked (every z gives a g inside the bound).
 */
kda_status kda_prefill_fused(int32_t num_seqs, int64_t total_tokens,
                             int32_t num_heads, int32_t d_k, int32_t d_v,
                             int32_t qkv_dtype, int32_t chunk_size, float scale,
                             const void *q, const void *k, const void *v,
                             const void *z, const float *a_log,
                             const float *beta, const float *initial_state,
                             const int32_t *cu_seqlens, void *o,
                             float *final_state, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * kda_decode_step -- one new token per sequence, state updated in place
 * (serving needs a dedicated decode kernel: "Kimi K3.1 and the Road From
 * Softmax Attention to KDA", neuralmasteryai.com, section 8; constant cost
 * per token: "KDA: the memory matrix", lesson 2).  Per (n, h):
 *   S <- Diag(exp g) S;  a = S^T k;  S <- S + beta k (v - a)^T;  o = scale S^T q
 * streaming each fp32 state through HBM once (read once, written once).
 *
 *   num_seqs  N >= 0;  num_heads H >= 1;  d_k, d_v: see kda_decode_supported.
 *   q, k      [N, H, d_k] qkv_dtype;  v [N, H, d_v] qkv_dtype
 *   g         [N, H, d_k] fp32;       beta [N, H] fp32
 *   state     [N, H, d_k, d_v] fp32, read and overwritten in place
 *   o         [N, H, d_v] qkv_dtype, written; must not overlap state or an
 *             input (equal pointers are rejected with KDA_ERR_BAD_SHAPE)
 *
 * Errors as for kda_prefill.  N = 0 is a valid no-op.
 */
kda_status kda_decode_step(int32_t num_seqs, int32_t num_heads, int32_t d_k,
                           int32_t d_v, int32_t qkv_dtype, float scale,
                           const void *q, const void *k, const void *v,
                           const float *g, const float *beta, float *state,
                           void *o, void *stream);

/* 1 if (qkv_dtype, d_v) has a built kda_output_gate kernel, else 0. */
int32_t kda_output_gate_supported(int32_t qkv_dtype, int32_t d_v);

/*
 * kda_output_gate -- the gated output of a KDA layer before its output
 * projection ("Understanding Kimi K3's attention", output equation:
 * Sigmoid(W_g x_t) times RMSNorm of the ungated readout o~_t; W_g x_t is
 * computed upstream and passed as `gate`, W_o stays outside).  Per (token,
 * head) row of d_v channels:
 *
 *   y = Sigmoid(gate) * o / sqrt(mean over the row of o^2 + eps) * weight
 *
 *   total_tokens, num_heads  rows = total_tokens * num_heads
 *   d_v         channels per row (see kda_output_gate_supported: 16, 32, 64
 *               or 128)
 *   qkv_dtype   dtype of o, gate and y (KDA_DTYPE_BF16 or KDA_DTYPE_F32);
 *               arithmetic in fp32, y rounded to nearest even for bf16
 *   eps         >= 0, added to the mean square (the pages give no value)
 *   o, gate     [total_tokens, H, d_v] device buffers, 16-byte aligned
 *   weight      [d_v] fp32, the per-channel RMSNorm weight, shared by heads
 *   y           [total_tokens, H, d_v], written; may be the same buffer as
 *               o or as gate (each element is read before it is written),
 *               must not overlap them otherwise
 *
 * Errors: KDA_ERR_BAD_SHAPE (sizes, eps negative, NaN or huge, y == weight),
 * KDA_ERR_UNSUPPORTED, KDA_ERR_NULL_POINTER, KDA_ERR_MISALIGNED, KDA_ERR_HIP.
 * total_tokens = 0 is a valid no-op.
 */
kda_status kda_output_gate(int64_t total_tokens, int32_t num_heads,
                           int32_t d_v, int32_t qkv_dtype, float eps,
                           const void *o, const void *gate,
                           const float *weight, void *y, void *stream);

/*
 * kda_prefill_output_gated -- kda_prefill followed by the gated output of the
 * layer, y = Sigmoid(gate) * RMSNorm(o) * weight ("Understanding Kimi K3's
 * attention", output equation; the readout o is that of kda_prefill), with y
 * returned in place of o.  Where one workgroup holds a whole head (bf16,
 * d = 128, the library's whole-head slab: batches with more (sequence, head)
 * units than half the compute units), the gate is applied before the store
 * and o never reaches memory: the o tiles go through LDS to two waves of the
 * workgroup, each of which forms every row's sum of squares and stores half
 * of y.  Otherwise o is written to y and
 * kda_output_gate runs over it in place.  The norm is taken over the o values
 * as rounded to qkv_dtype, as a separate pass would read them.
 *
 * Arguments as kda_prefill (o replaced by y), plus:
 *   gate    [T_total, H, d_v] qkv_dtype, 16-byte aligned: the gate logits
 *           (W_g x_t, computed upstream).  y may be the same buffer as gate.
 *   weight  [d_v] fp32: the RMSNorm weight, shared by the heads.
 *   eps     >= 0, added to the mean square.
 *   y       [T_total, H, d_v] qkv_dtype, written.
 * Supported where kda_prefill and kda_output_gate both are.  Errors as
 * kda_prefill and kda_output_gate.
 */
kda_status kda_prefill_output_gated(int32_t num_seqs, int64_t total_tokens, int32_t num_heads, int32_t d_k,
                                    int32_t d_v, int32_t qkv_dtype, int32_t chunk_size, float scale,
                                    const void *q, const void *k, const void *v, const float *g,
                                    const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                                    const void *gate, const float *weight, float eps, void *y,
                                    float *final_state, void *workspace, size_t workspace_bytes, void *stream);

/* 1 if kda_prefill_backward is built for (qkv_dtype, d_k, d_v): bf16 with
 * d_k = d_v = 128. */
int32_t kda_prefill_backward_supported(int32_t qkv_dtype, int32_t d_k,
                                       int32_t d_v);

/* Bytes of device workspace kda_prefill_backward needs (0 for unsupported
 * arguments), three parts each rounded up to 256 bytes: the state after every
 * 16 tokens of each sequence (floor(total_tokens / 16) * num_heads * d_k *
 * d_v, rounded to bf16: the reverse pass uses the states only as bf16 matrix
 * operands), per half of the value columns the partial key-side gradients (2 *
 * total_tokens * num_heads * (3 * d_k + 1) fp32), and the initial states
 * rounded to bf16 (num_seqs * num_heads * d_k * d_v). */
size_t kda_prefill_backward_workspace_bytes(int32_t num_seqs,
                                            int64_t total_tokens,
                                            int32_t num_heads, int32_t d_k,
                                            int32_t d_v, int32_t qkv_dtype);

/*
 * kda_prefill_backward -- gradients of kda_prefill for training ("Hybrid
 * Attention", kimi-k3.adriaflores.com, section "But isn't a recurrent update
 * sequential?": the chunked form's outputs and gradients are checked against
 * the token recurrence).  For a scalar loss with gradient d_o with respect to
 * o and d_final_state with respect to the final states, it returns the
 * gradients with respect to q, k, v, g, beta and the initial states.
 *
 * Computed in three launches on `stream` (four with initial states): the
 * forward recurrence again (the kernel of kda_prefill, chunk 16, without its
 * output), keeping the state at every 16-token boundary in the workspace; the
 * initial states
 * rounded into the same form; the reverse pass, two workgroups per
 * (sequence, head), one per half of the value columns, walking the chunks
 * last to first; and the sum of the two halves' key-side partials.
 *
 * Arguments shared with kda_prefill (num_seqs, total_tokens, num_heads, d_k,
 * d_v, qkv_dtype, scale, q, k, v, g, beta, initial_state, cu_seqlens) mean
 * the same and follow the same rules; qkv_dtype must be KDA_DTYPE_BF16 and
 * d_k = d_v = 128 (kda_prefill_backward_supported).  In addition, device
 * memory, 16-byte aligned unless noted:
 *   d_o              [T_total, H, d_v] bf16, read: gradient with respect to o.
 *   d_final_state    [N, H, d_k, d_v] fp32 or NULL (zeros), read.
 *   dq, dk           [T_total, H, d_k] bf16, written.
 *   dv               [T_total, H, d_v] bf16, written.
 *   dg               [T_total, H, d_k] fp32, written.
 *   dbeta            [T_total, H] fp32 (4-byte aligned), written.
 *   d_initial_state  [N, H, d_k, d_v] fp32 or NULL (not returned), written.
 *   workspace        at least kda_prefill_backward_workspace_bytes, owned by
 *                    the caller, contents undefined afterwards.
 * Outputs must not alias inputs or each other.  Errors as kda_prefill
 * (KDA_ERR_WORKSPACE for a short workspace); with KDA_VALIDATE=1, g, beta
 * and cu_seqlens are checked as there.  Results are deterministic.
 */
kda_status kda_prefill_backward(int32_t num_seqs, int64_t total_tokens,
                                int32_t num_heads, int32_t d_k, int32_t d_v,
                                int32_t qkv_dtype, float scale, const void *q,
                                const void *k, const void *v, const float *g,
                                const float *beta, const float *initial_state,
                                const int32_t *cu_seqlens, const void *d_o,
                                const float *d_final_state, void *dq, void *dk,
                                void *dv, float *dg, float *dbeta,
                                float *d_initial_state, void *workspace,
                                size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
