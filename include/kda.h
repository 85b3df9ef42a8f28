/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention (KDA) core.
 *
 * What is computed: "Kimi K3 Technical Report: Open Frontier Intelligence",
 * §2.1.1 (Kimi Delta Attention).  Per head, with state S in R^{d_k x d_v}:
 *
 *   eq. (1)   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *             o_t = S_t^T (scale * q_t)                (eq. (1) itself has scale = 1)
 *   eq. (5)   g_t = g_min * Sigmoid(exp(A_h) * z_t),  alpha_t = exp(g_t)
 *
 * kda_chunk_fwd evaluates eq. (1) over whole sequences in the chunkwise-parallel
 * form of eqs. (3)-(4) (chunk size 64, 16-token sub-tiles); kda_recurrent_step
 * applies eq. (1) to one token per sequence with the state updated in place
 * (§5.4.2, "KDA" paragraph: the decode state is updated in place every step);
 * kda_recurrent_replay runs a speculative-decoding window (replayed accepted
 * tokens plus new tokens) in one pass over the in-place state (same paragraph).
 * Each entry point can also apply the layer's input prologue (eq. (2)) and
 * output epilogue (eq. (6)) inside its kernels; see kda_layer_fusion_t.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller; all tensors are
 *     dense, row-major (last index fastest) and 16-byte aligned.  The library
 *     allocates no device memory and keeps no state between calls (apart from
 *     the fixed workspace array of kda_chunk_fwd_noalloc, below).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream).
 *     No call synchronises the device or copies data to the host.
 *   - Validation happens before anything is enqueued; on error nothing is
 *     launched and no output is touched.  A launch failure returns
 *     KDA_ERROR_HIP; faults during execution surface at the caller's next
 *     synchronisation, as usual for HIP.  kda_last_error_message() returns a
 *     thread-local description of the last failure on the calling thread.
 *   - Decay input `g`: when A_log is NULL it holds log-decays g in [g_min, 0]
 *     (values outside are clamped to that range, which the range argument of
 *     eq. (5) needs); when A_log is non-NULL it holds decay logits z and the
 *     eq. (5) gate is applied inside the kernels in fp32.
 *   - Preconditions not checked on the device: q and k rows have L2 norm <= 1
 *     (eq. (2) normalises them), beta in [0, 1], cu_seqlens non-decreasing
 *     from 0 to T.  Offsets that break the last one give wrong results but no
 *     access outside the caller's tensors or the workspace: each sequence is
 *     clamped into tokens [0, T] (a decreasing pair is an empty sequence) and
 *     the chunk count saturates at the workspace's capacity.
 *   - The library is thread-safe; calls that share output buffers race.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define KDA_API __attribute__((visibility("default")))
#else
#define KDA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_F32 = 0,   /* float32 q, k, v, g, beta, o */
    KDA_BF16 = 1   /* bfloat16 q, k, v, g, beta, o (fp32 state and accumulation) */
} kda_dtype_t;

typedef enum {
    KDA_SUCCESS = 0,
    KDA_ERROR_INVALID_VALUE = 1,   /* null pointer, bad size, misalignment, bad flag */
    KDA_ERROR_NOT_SUPPORTED = 2,   /* head dims outside {64, 128}, g_min outside [-5, 0) */
    KDA_ERROR_WORKSPACE = 3,       /* workspace missing or smaller than required */
    KDA_ERROR_HIP = 4              /* a HIP runtime call or kernel launch failed */
} kda_status_t;

/*
 * Optional fusion of the layer around the recurrence ("Kimi K3 Technical
 * Report", §2.1.1 eqs. (2) and (6); §5.4.2 describes the decode kernel as one
 * fused loop over short convolution, input normalisation, gating, the
 * recurrence and output normalisation).  The dense projections (W x products,
 * the low-rank decay projection and W_o) stay with the caller.
 *
 * Prologue (eq. (2)), on when conv_width >= 1.  Then q, k, v hold the
 * projections W_q x, W_k x, W_v x BEFORE the convolution and beta holds the
 * logits W_beta x; per head and token the kernels form
 *   q = L2Norm(Swish(ShortConv(W_q x))),  k likewise,  v = Swish(ShortConv(W_v x)),
 *   beta = Sigmoid(W_beta x),
 * with Swish(x) = x Sigmoid(x) (§2.3.2) and L2Norm(y) = y / sqrt(sum y^2 + qk_norm_eps)
 * over the head's Dk channels.  ShortConv is a causal depthwise convolution over
 * time with no bias: channel c of token t is
 *   sum_{i < W} conv_weight[h][c][i] * x[t - (W - 1) + i][c],
 * the W - 1 positions before a sequence's first token read from conv_state.
 * Channels per head: Dk query channels, then Dk key channels, then Dv value
 * channels (C = 2*Dk + Dv).  g (log-decays or logits z, with A_log) is used
 * as without the prologue.
 *   conv_weight : [H, C, W] float32, 16-byte aligned.
 *   conv_state  : [N, H, W - 1, C] elements of the call's dtype: the
 *                 pre-activations of the W - 1 tokens before the first one
 *                 (oldest first).
 *     kda_chunk_fwd:        read only; NULL = zeros (fresh sequences).
 *     kda_recurrent_step / kda_recurrent_replay: required when W > 1; read and
 *                 overwritten IN PLACE at the commit point with the W - 1
 *                 pre-activations before it (replayed tokens included; left
 *                 untouched when nothing is committed), like the state.
 *   conv_state_out : kda_chunk_fwd only (NULL elsewhere): [N, H, W - 1, C],
 *                 each sequence's last W - 1 pre-activations (older rows
 *                 from conv_state when a sequence is shorter), or NULL.  It
 *                 must not overlap conv_state.
 *   conv_checkpoints : kda_chunk_fwd only, with checkpoints set: [N, slots, H,
 *                 W - 1, C]; slot j receives the convolution state at the
 *                 position of checkpoint slot j (what resuming from that
 *                 checkpoint needs as conv_state), or NULL.
 * Epilogue (eq. (6) without W_o), on when gate is non-NULL: o receives
 *   y = Sigmoid(gate) * o_norm_weight[h] * o~ / sqrt(mean(o~^2) + o_norm_eps)
 * per head and token (mean over the Dv channels of the recurrence output o~).
 *   gate          : logits W_g x, shaped like o, in the call's dtype.
 *   o_norm_weight : [H, Dv] float32, required with gate.
 * Both epsilons must be >= 0; with an epsilon of 0, a sum (or mean) of squares
 * below 2^-126 is taken as 2^-126 (so a zero vector stays zero).  A NULL fusion
 * pointer (or conv_width = 0 and gate = NULL) leaves every entry point exactly
 * as documented above it.
 */
typedef struct {
    int32_t conv_width;            /* W in 1..4, or 0: no prologue */
    const float *conv_weight;
    void *conv_state;
    void *conv_state_out;
    void *conv_checkpoints;
    float qk_norm_eps;
    const void *gate;              /* NULL: no epilogue */
    const float *o_norm_weight;
    float o_norm_eps;
} kda_layer_fusion_t;

/* Chunk size of the chunkwise-parallel form and its sub-tile size. */
#define KDA_CHUNK 64
#define KDA_SUBTILE 16

/*
 * Prefill / training forward over whole sequences (chunkwise-parallel form,
 * §2.1.1 eqs. (3)-(4); inter-chunk state hand-off derived from eq. (1)).
 *
 * Shapes (row-major):
 *   q, k, g : [B, T, H, Dk]     v, o : [B, T, H, Dv]     beta : [B, T, H]
 *   A_log   : [H] float32, or NULL (see "Decay input" above)
 *   cu_seqlens : [N+1] int32 token offsets of N packed sequences, or NULL.
 *                When set, B must be 1 and sequence s covers tokens
 *                [cu_seqlens[s], cu_seqlens[s+1]) of the T tokens; chunks restart
 *                at every sequence start.  When NULL, the B rows are the N = B
 *                sequences, each T tokens long.
 *   initial_state : [N, H, Dk, Dv] float32 entering states, or NULL for zeros.
 *                   Read only; it may alias final_state (in-place resume).
 *   final_state   : [N, H, Dk, Dv] float32 states after each sequence's last
 *                   token, or NULL if not wanted.
 * Dk, Dv in {64, 128}.  T may be 0 (then final_state = initial_state).
 * The workspace (device memory, >= kda_chunk_fwd_workspace_size bytes,
 * 256-byte aligned) holds the packed-sequence chunk table and per-chunk
 * intermediates; its contents on entry are ignored and on exit are
 * unspecified.  With bf16 inputs, Dk = 128, no layer prologue and 128 or more
 * (sequence, head) pairs the per-chunk intermediates stay on chip and the
 * workspace holds the chunk table only (none for a batch of equal-length
 * sequences).
 *
 * State checkpoints ("Kimi K3 Technical Report", §5.4.1: the KDA state is
 * persisted at hash-block-aligned prefix positions so that a later request
 * sharing the prefix resumes from it):
 *   checkpoints : [N, checkpoint_slots, H, Dk, Dv] float32, or NULL for none.
 *   Slot j of sequence s receives the state after the first
 *   (j + 1) * checkpoint_every * KDA_CHUNK tokens of s, for every j with that
 *   position strictly inside the sequence and j < checkpoint_slots; other
 *   slots are not written.  (The state after the last token is final_state.)
 *   Resuming = passing a slot as initial_state for the remaining tokens.
 *   checkpoint_every >= 1 and checkpoint_slots >= 1 are required when
 *   checkpoints is set; both are ignored otherwise.  The buffer is owned by
 *   the caller, must be 16-byte aligned and must not overlap any other
 *   argument; its size is not checked (the library holds no shapes of it).
 */
typedef struct {
    int32_t B, T, H, Dk, Dv;
    int32_t dtype;                 /* kda_dtype_t */
    const void *q, *k, *v, *g, *beta;
    const float *A_log;
    float g_min;                   /* lower bound of the log-decay, in [-5, 0); the pages use -5 */
    float scale;                   /* query scale; 1.0 reproduces eq. (1) */
    const int32_t *cu_seqlens;
    int32_t N;                     /* number of sequences when cu_seqlens is set (else ignored) */
    const float *initial_state;
    void *o;
    float *final_state;
    void *workspace;
    size_t workspace_bytes;
    float *checkpoints;            /* optional prefix-state checkpoints, see above */
    int32_t checkpoint_every;      /* chunks of KDA_CHUNK tokens between checkpoints */
    int32_t checkpoint_slots;      /* capacity per sequence */
    const kda_layer_fusion_t *fusion;   /* optional prologue / epilogue, or NULL */
} kda_chunk_fwd_args_t;

/* Workspace bytes kda_chunk_fwd needs for these shapes (pointers are not
 * read).  Depends on B, T, H, Dk, Dv, dtype and on whether cu_seqlens is set
 * (and N); the layer prologue and epilogue need none. */
KDA_API kda_status_t kda_chunk_fwd_workspace_size(const kda_chunk_fwd_args_t *args, size_t *bytes);

KDA_API kda_status_t kda_chunk_fwd(const kda_chunk_fwd_args_t *args, void *stream);

/*
 * kda_chunk_fwd without a caller-provided workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  It computes exactly what kda_chunk_fwd
 * computes, with the same kernels, and calls no allocating routine: its
 * workspace is a fixed array of KDA_NOALLOC_WORKSPACE_BYTES in device memory
 * that every device the library runs on holds from module load until the
 * process ends.  args->workspace must be NULL and args->workspace_bytes 0.
 * Shapes whose kda_chunk_fwd_workspace_size exceeds the array are rejected
 * with KDA_ERROR_WORKSPACE before anything is enqueued (at bf16 and
 * Dk = Dv = 128 with fewer than 128 (sequence, head) pairs the array holds
 * 897 chunk blocks of 64 tokens x 1 head, e.g. B = 1, T = 7168 tokens at
 * H = 8; with 128 pairs or more it needs only the chunk table).  The array used
 * is the copy on the device that is current when the call is made, which must
 * be the stream's device.  Every call on one device uses the same array, so
 * calls that overlap on a device (on different streams, or from different
 * threads without ordering) race; calls ordered on one stream do not.  The
 * array's contents on entry are ignored: every value a call uses from it is
 * written earlier in the same call, so nothing needs clearing between calls.
 */
#define KDA_NOALLOC_WORKSPACE_BYTES (64u << 20)
KDA_API kda_status_t kda_chunk_fwd_noalloc(const kda_chunk_fwd_args_t *args, void *stream);

/*
 * One decode step for N independent sequences (one token each), eq. (1):
 *   q, k, g : [N, H, Dk]    v, o : [N, H, Dv]    beta : [N, H]
 *   state   : [N, H, Dk, Dv] float32, read and overwritten IN PLACE with S_t.
 * Dk, Dv in {64, 128}; A_log / g as for kda_chunk_fwd.  N = 0 is a no-op;
 * N*H above 2^30 - 1 returns KDA_ERROR_NOT_SUPPORTED.  The state must not
 * alias q/k/v/g/beta/o.  All pointers are device memory owned by the caller;
 * the call allocates nothing and is asynchronous on `stream`.
 */
typedef struct {
    int32_t N, H, Dk, Dv;
    int32_t dtype;                 /* kda_dtype_t */
    const void *q, *k, *v, *g, *beta;
    const float *A_log;
    float g_min;
    float scale;
    float *state;
    void *o;
    const kda_layer_fusion_t *fusion;   /* optional prologue / epilogue, or NULL */
} kda_step_args_t;

KDA_API kda_status_t kda_recurrent_step(const kda_step_args_t *args, void *stream);

/*
 * Speculative-decoding step with replay ("Kimi K3 Technical Report", §5.4.2,
 * "KDA" paragraph).  With multi-token drafts the in-place state cannot be
 * rolled back once it has moved past a rejected draft, and keeping a state
 * snapshot per draft position multiplies the state traffic.  The state after
 * any accepted draft prefix is fixed by the drafts' projected inputs, which are
 * much smaller, so the caller keeps those and this call rebuilds the accepted
 * state on chip: for each sequence s and head h, in ONE pass over the state,
 *   1. replay: the first n_replay[s] tokens of the cached window (k_r, v_r,
 *      g_r, beta_r; their outputs were produced by an earlier call) go through
 *      eq. (1) with no output;
 *   2. new window: tokens 0 .. T_new-1 (q, k, v, g, beta) go through eq. (1)
 *      and o[s, t] receives each token's output;
 *   3. the state written back is the one after the replayed tokens and the
 *      first n_commit tokens of the new window (typically 1: the bonus token
 *      is certain, the drafts behind it are not); if that count is 0 the state
 *      is left untouched.
 * With T_replay = 0 and n_commit = T_new this is T_new decode steps in one
 * pass; with n_commit = 0 it only verifies.
 *   k_r, g_r : [N, T_replay, H, Dk]   v_r : [N, T_replay, H, Dv]   beta_r : [N, T_replay, H]
 *   q, k, g  : [N, T_new, H, Dk]      v, o : [N, T_new, H, Dv]    beta : [N, T_new, H]
 *   n_replay : [N] int32 on the device, or NULL (= T_replay for every sequence);
 *              values are clamped to [0, T_replay] on the device
 *   state    : [N, H, Dk, Dv] float32, in place
 * Requirements: N >= 0, H >= 1, T_replay >= 0, T_new >= 0, 0 <= n_commit <=
 * T_new; the replay tensors may be NULL when T_replay = 0 and the new-window
 * tensors when T_new = 0.  Dk, Dv, dtype, A_log / g and alignment as for
 * kda_recurrent_step; the state must not alias any other argument.
 * With the fused prologue the replayed window also needs its query
 * projections, q_r : [N, T_replay, H, Dk] (the query convolution runs through
 * the replayed tokens); q_r is ignored otherwise.
 */
typedef struct {
    int32_t N, H, Dk, Dv;
    int32_t dtype;                 /* kda_dtype_t */
    int32_t T_replay, T_new, n_commit;
    const void *k_r, *v_r, *g_r, *beta_r;
    const int32_t *n_replay;
    const void *q, *k, *v, *g, *beta;
    const float *A_log;
    float g_min;
    float scale;
    float *state;
    void *o;
    const void *q_r;                    /* replayed query projections (fused prologue only) */
    const kda_layer_fusion_t *fusion;   /* optional prologue / epilogue, or NULL */
} kda_replay_args_t;

KDA_API kda_status_t kda_recurrent_replay(const kda_replay_args_t *args, void *stream);

/* Static description of a status code. */
KDA_API const char *kda_status_string(kda_status_t status);

/* Thread-local detail of the last failure on this thread ("" if none). */
KDA_API const char *kda_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
