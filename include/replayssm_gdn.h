/*
 * replayssm_gdn.h: C ABI of the ReplaySSM decode hot path for one Gated
 * DeltaNet (GDN) layer, hand-written HIP kernels for MI355X (gfx950), in
 * libreplayssm.so beside the Mamba-2 entry points of replayssm.h (whose
 * element types, return codes, status bits, limits and replayssm_last_error()
 * it shares).
 *
 * Method: NVIDIA Developer blog "ReplaySSM: Rethinking State Storage for Faster
 * Hybrid-Model Decoding".  Section "Why SSM layers can become a decoding
 * bottleneck" states that GDN's update, delta-rule correction included, keeps
 * Mamba-2's decay-plus-rank-1 structure, so the checkpoint-plus-buffer state of
 * section "How ReplaySSM represents the state" applies; section "Benefit 2"
 * says GDN can use output-only evaluation.  The GDN recurrence is the gated
 * delta rule (Yang, Kautz and Hatamizadeh, "Gated Delta Networks", ICLR 2025),
 * per sequence b and value head h reading key head kh = h / (nv/nk):
 *
 *   S_t = S_{t-1} alpha_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t
 *
 * with S (dv x dk) and alpha_t = exp(g_t).  Expanded, S_t = alpha_t S_{t-1} +
 * u_t k_t^T with the corrected value u_t = beta_t (v_t - alpha_t S_{t-1} k_t).
 * A record is therefore (k_t, u_t, g_t): the library computes u_t when the
 * token arrives, from the checkpoint and the records before it, and stores it.
 * With the window's records numbered from the last flush and
 * G(c, m) = exp(sum_{c<i<=m} g_i), a query at window position m computes
 *
 *   u_m = beta_m (v_m - [G(-1, m) (S_s k_m) + sum_{c<m} G(c, m) (k_c . k_m) u_c])
 *   o_m = G(-1, m) (S_s q_m) + sum_{c<=m} G(c, m) (k_c . q_m) u_c
 *
 * reading the checkpoint S_s once for both products, and a flush folds
 * S_s <- G(-1, n-1) S_s + sum_{c<n} G(c, n-1) u_c k_c^T and writes it once.
 * This equals stepping the recurrence token by token, up to rounding.
 *
 * Conventions: as in replayssm.h (device pointers, caller-owned buffers, no
 * allocation or synchronisation, work on `stream`, negative return codes with
 * the message in replayssm_last_error(), data errors found by a kernel set
 * bits in *status, leave the state untouched and write NaN outputs).
 * Compiled shapes: dk = 16 with dv % 16 == 0, and dk = 128 with dv % 64 == 0;
 * nv % nk == 0.  Each value head's state is split into dv/16 (dk = 16) or
 * dv/64 (dk = 128) row blocks of 16 x 16 or 64 x 128 elements, each with its
 * own copy of the ring pointer; a workgroup serves one block (two with an FP16
 * checkpoint, dk = 128 and dv % 128 == 0).
 * Token, record and state pointers must be 16-byte aligned.
 */
#ifndef REPLAYSSM_GDN_H
#define REPLAYSSM_GDN_H

#include <stddef.h>
#include <stdint.h>

#include "replayssm.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int32_t batch;
    int32_t nv, nk;      /* value heads, key heads (nv % nk == 0) */
    int32_t dk, dv;      /* key / value head dimension */
    int32_t window;      /* L: a call that starts with >= L committed records flushes first */
    int32_t max_drafts;  /* T_max */
    int32_t in_dtype;    /* RSSM_F32 or RSSM_BF16: tokens q, k, v and the k records */
    int32_t ckpt_dtype;  /* RSSM_F32 (0): FP32 checkpoint.  RSSM_F16: half-precision recurrence
                            checkpoint (blog section "Benefit 3": a half-precision recurrence state
                            stays close to FP32 when its writes round stochastically): every call
                            widens the fp16 checkpoint to fp32
                            registers; a flush folds there and writes fp16 with stochastic rounding
                            (random words as for the Mamba-2 FP16 checkpoint in replayssm.h: Philox4x32-10,
                            element 4v+e takes word e at counter (v low, v high, 0, 0) under the key
                            sr_seed, v the 4-element vector index over [batch][nv][dv][dk]); the
                            flushing call's outputs and records come from the fp32 registers.
                            gdn_conventional_* need RSSM_F32. */
} gdn_config;

/* Number of row blocks (workgroups) per value head: dv/16 for dk = 16, dv/64 for dk = 128. */
int gdn_row_blocks(const gdn_config *cfg);

/*
 * Per-layer GDN decode state; cap = window + 2*max_drafts - 1 record slots
 * per sequence, used as a ring (record c of the window in slot (start + c) % cap).
 */
typedef struct {
    void *ckpt;       /* [batch][nv][dv][dk] checkpoint S_s: fp32, or fp16 bits with RSSM_F16 */
    void *buf_k;      /* [batch][nk][cap][dk] in_dtype: keys of the records */
    float *buf_u;     /* [batch][nv][cap][dv] fp32: corrected values u of the records */
    float *buf_g;     /* [batch][nv][cap] fp32: log decays g of the records */
    int32_t *meta;    /* [batch][nv][row_blocks][2] = {ring start, committed length}: one copy per
                         workgroup, all copies of a sequence equal (initialise them together);
                         a copy disagreeing with the sequence's first one sets RSSM_STATUS_META */
    int32_t *status;  /* sticky RSSM_STATUS_* bits, or NULL */
} gdn_state;

/* T tokens per sequence: q, k [batch][T][nk][dk] and v [batch][T][nv][dv] in in_dtype
   (q and k as the layer hands them over: normalised and scaled); g (log decay, <= 0)
   and beta [batch][T][nv] fp32. */
typedef struct {
    const void *q, *k, *v;
    const float *g, *beta;
    int32_t T;
    uint64_t sr_seed;   /* RSSM_F16 checkpoint: key of the stochastic rounding of a flush this call
                           performs (vary it per call, e.g. a step counter); ignored for RSSM_F32 */
} gdn_tokens;

/* Byte sizes of ckpt, buf_k, buf_u, buf_g, meta (in that order) for cfg. */
#define GDN_NUM_BUFS 5
int gdn_sizes(const gdn_config *cfg, size_t bytes[GDN_NUM_BUFS]);

/* One decode token per sequence (T == 1): flush first if the buffer holds >= L
   committed records, compute u and o, append the record, commit it.
   o: [batch][1][nv][dv] fp32. */
int gdn_decode_step(const gdn_config *cfg, const gdn_state *st, const gdn_tokens *tok, float *o,
                    void *stream);

/* Outputs of T draft tokens (1 <= T <= max_drafts; draft q sees the committed records
   and drafts 0..q): flush first if >= L committed records, append the drafts' records
   beyond the committed length, leave the length unchanged (blog section "Benefit 2":
   rollback is a pointer move).  o: [batch][T][nv][dv] fp32. */
int gdn_verify_drafts(const gdn_config *cfg, const gdn_state *st, const gdn_tokens *tok, float *o,
                      void *stream);

/* gdn_commit of the previous round (accepted_prev, T_prev) fused into this round's
   gdn_verify_drafts: one launch per speculative round.  Equivalent, bit for bit, to
   gdn_commit(cfg, st, accepted_prev, T_prev) followed by gdn_verify_drafts(cfg, st, tok, o);
   an accepted count outside 0..T_prev sets RSSM_STATUS_ACCEPT, leaves that sequence alone and
   writes NaN to its outputs. */
int gdn_commit_verify(const gdn_config *cfg, const gdn_state *st, const int32_t *accepted_prev,
                      int32_t T_prev, const gdn_tokens *tok, float *o, void *stream);

/* Commit accepted[b] (device int32 [batch], 0..T) of the last T drafts: the committed
   length grows by accepted[b]; nothing else moves.  An accepted count outside 0..T (or
   past the ring) sets RSSM_STATUS_ACCEPT and leaves that sequence alone. */
int gdn_commit(const gdn_config *cfg, const gdn_state *st, const int32_t *accepted, int32_t T,
               void *stream);

/* Fold every sequence's committed records into its checkpoint (those with none are
   left alone); sr_seed keys the stochastic rounding of an RSSM_F16 checkpoint. */
int gdn_flush(const gdn_config *cfg, const gdn_state *st, uint64_t sr_seed, void *stream);

/* Conventional GDN step (the in-library baseline; blog section "Why SSM layers can become a
   decoding bottleneck": every token loads, updates and stores the full state): per token,
   S k, u = beta (v - alpha S k), S <- alpha S + u k^T, o = S q.
   states: [batch][nslots][nv][dv][dk] fp32.
   nslots == 1: tok->T must be 1 and the state is updated in place; slot may be NULL.
   nslots > 1 (speculative verification with one state snapshot per draft, blog section
     "Rollback for speculative decoding"): slot[b] (device int32 [batch]) names the current
     state; draft q's state is written to slot (slot[b] + 1 + q) % nslots, 1 <= T < nslots,
     T <= RSSM_MAX_DRAFTS.  A slot index out of range sets RSSM_STATUS_SLOT, writes NaN
     outputs and leaves that sequence alone.
   o: [batch][T][nv][dv] fp32. */
int gdn_conventional_update(const gdn_config *cfg, float *states, int32_t nslots, const int32_t *slot,
                            int32_t *status, const gdn_tokens *tok, float *o, void *stream);

/* Baseline commit after a snapshot verification: slot[b] = (slot[b] + accepted[b]) % nslots,
   0 <= accepted[b] <= T (else RSSM_STATUS_ACCEPT and the sequence is left alone). */
int gdn_conventional_commit(const gdn_config *cfg, int32_t *slot, int32_t nslots, const int32_t *accepted,
                            int32_t T, int32_t *status, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* REPLAYSSM_GDN_H */
