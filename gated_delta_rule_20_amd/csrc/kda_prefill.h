// kda_prefill.h -- host-side interface of the chunkwise-parallel KDA kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// Layer prologue / epilogue fused around the recurrence (kda_layer_fusion_t).
struct FusionParams {
    int conv_w;                         // ShortConv width W (1..4), 0: no prologue
    const float *conv_weight;           // [H, 2*Dk + Dv, W]
    void *conv_state;                   // [N, H, W-1, 2*Dk + Dv] element type T, or null
    void *conv_state_out;               // prefill: [N, H, W-1, 2*Dk + Dv] or null
    void *conv_ckpt;                    // prefill: [N, ckpt_slots, H, W-1, 2*Dk + Dv] or null
    float qk_eps;
    const void *gate;                   // logits shaped like o, or null: no epilogue
    const float *o_weight;              // [H, Dv]
    float o_eps;
};

// Everything the three prefill kernels need, passed by value.
struct PrefillParams {
    const void *q, *k, *v, *g, *beta;   // [rows, H, D] token-major, element type T
    const float *A_log;                 // [H] or null (g holds log-decays)
    float g_min, scale;
    const int32_t *cu;                  // [N+1] packed-sequence offsets (varlen) or null
    int N, T, H;                        // N sequences; T = tokens per sequence when !varlen
    int varlen;
    const float *h0;                    // [N, H, Dk, Dv] or null
    float *hT;                          // [N, H, Dk, Dv] or null
    void *o;                            // [rows, H, Dv]
    int32_t *chunk_off;                 // [N+1] (varlen; workspace)
    int32_t *order;                     // [N]   (varlen; workspace)
    int32_t *span;                      // [N][2] clamped (first token, length) (varlen; workspace)
    char *blocks;                       // [H][n_chunks_cap] per-chunk blocks (workspace)
    int n_chunks_cap;
    float *ckpt;                        // [N, ckpt_slots, H, Dk, Dv] or null
    int ckpt_every, ckpt_slots;         // chunks between checkpoints, slots per sequence
    FusionParams f;
};

// With this many (sequence, head) pairs or more the chain stage runs per pair:
// inside the intra-chunk kernel (pair mode, no chunk blocks in the workspace)
// for bf16 with d_k = 128 and no layer prologue, else on the wide chain kernel.
constexpr long MANY_PAIRS = 128;
inline bool pair_mode(int bf16, int Dk, long npairs, int prologue)
{
    return bf16 && Dk == 128 && !prologue && npairs >= MANY_PAIRS;
}

// Bytes of one (head, chunk) workspace block; 0 if the combination is unsupported.
size_t block_bytes(int bf16, int Dk, int Dv);

// Bytes of the chunk table at the front of the workspace (0 when !varlen).
inline size_t table_bytes(int varlen, int N)
{
    return varlen ? ((size_t)(4 * N + 1) * sizeof(int32_t) + 255) / 256 * 256 : 0;
}

// Enqueue the full prefill on `stream`.  The caller has validated arguments
// and carved the workspace into p.chunk_off / p.order / p.span / p.blocks.
hipError_t launch_chunk_fwd(int bf16, int Dk, int Dv, const PrefillParams &p, hipStream_t stream);

// Speculative-decoding step with replay (one pass over the in-place state).
struct ReplayParams {
    int N, H, T_replay, T_new, n_commit;
    const void *k_r, *v_r, *g_r, *beta_r;   // cached window [N, T_replay, H, D]
    const int32_t *n_replay;                // [N] or null (= T_replay)
    const void *q, *k, *v, *g, *beta;       // new window [N, T_new, H, D]
    const float *A_log;
    float g_min, scale;
    float *state;                           // [N, H, Dk, Dv]
    void *o;                                // [N, T_new, H, Dv]
    const void *q_r;                        // [N, T_replay, H, Dk] (prologue only)
    FusionParams f;
};

hipError_t launch_recurrent_replay(int bf16, int Dk, int Dv, const ReplayParams &p, hipStream_t stream);


}  // namespace kda
