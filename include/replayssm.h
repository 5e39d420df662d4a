/*
 * replayssm.h: C ABI of the ReplaySSM decode hot path for one Mamba-2 layer,
 * hand-written HIP kernels for MI355X (gfx950).
 *
 * Method: NVIDIA Developer blog "ReplaySSM: Rethinking State Storage for Faster
 * Hybrid-Model Decoding".  Each sequence's SSM state is kept as an FP32
 * checkpoint H_s plus a buffer of the input records (x_k, B_k, dt_k) that came
 * after it (section "How ReplaySSM represents the state").  Per sequence b and
 * head h, with g = h / (nheads/ngroups), a_k = dt_k * A[h], and the records of
 * the current window numbered from the last flush:
 *
 *   y_q = exp(sum_{k<=m} a_k) * (H_s C_q)
 *         + sum_{k<=m} dt_k exp(sum_{k<i<=m} a_i) (B_k . C_q) x_k + D[h] x_q
 *
 * where m is the window position of query q.  This equals the conventional
 * recurrence H <- exp(dt A) H + dt x B^T, y = H C + D x stepped token by token
 * (section "Why SSM layers can become a decoding bottleneck"), up to rounding.
 *
 * Conventions for every entry point:
 *   - All pointers except the config/struct pointers themselves are DEVICE
 *     pointers.  The caller allocates and owns every buffer; the library
 *     allocates nothing, keeps no state between calls, and never synchronises
 *     the stream.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream).
 *   - Return value: RSSM_OK or a negative RSSM_ERR_* code; the message is in
 *     replayssm_last_error() (per calling thread).  On an error nothing is
 *     enqueued.
 *   - Errors a kernel finds in the data (a ring pointer out of range, a head's
 *     copy of it disagreeing with the sequence's first copy, a call whose
 *     committed records plus its tokens would not fit the ring, an accepted
 *     count out of range) OR a bit into *status (when status is not NULL; every
 *     workgroup that finds one reports it), leave the state of the heads
 *     concerned untouched and write NaN to their outputs; the other heads and
 *     sequences proceed unaffected.
 *   - batch == 0: only the config is checked and nothing is enqueued.
 *   - Calls that share buffers must be ordered on one stream.
 *   - Tile shapes compiled in: (headdim, dstate) = (16, 16), (64, 64),
 *     (64, 128), (128, 128).  nheads % ngroups == 0.  Pointers to tiles,
 *     records and bf16/fp32 token arrays must be 16-byte aligned.
 *   - Limits: 1 <= window <= RSSM_MAX_WINDOW, 1 <= max_drafts <= RSSM_MAX_DRAFTS.
 */
#ifndef REPLAYSSM_H
#define REPLAYSSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. */
#define RSSM_F32 0
#define RSSM_BF16 1
#define RSSM_FP8_E4M3 2 /* OCP e4m3fn: max 448, no infinities */
#define RSSM_NONE 3
#define RSSM_MXFP4 4    /* OCP MX FP4: E2M1 codes, one E8M0 scale per 32 consecutive dstate elements */
#define RSSM_MXFP8 5    /* MX FP8: e4m3fn codes, one E8M0 scale per 32 consecutive dstate elements,
                           chosen so that no element saturates (smallest X with max |v| / X <= 448) */
#define RSSM_F16 6      /* IEEE binary16 (the checkpoint, written with stochastic rounding) */

/* Return codes. */
#define RSSM_OK 0
#define RSSM_ERR_NULL (-1)   /* a required pointer is NULL */
#define RSSM_ERR_SHAPE (-2)  /* unsupported shape, limit or alignment */
#define RSSM_ERR_DTYPE (-3)  /* unsupported element type combination */
#define RSSM_ERR_DRAFTS (-4) /* token count T out of range for this call */
#define RSSM_ERR_HIP (-5)    /* the HIP runtime refused the launch */

/* Sticky device status bits, OR-ed into *status. */
#define RSSM_STATUS_META 1u   /* {start, len} out of range or copies disagree: heads skipped */
#define RSSM_STATUS_ACCEPT 2u /* accepted count outside 0..T: sequence skipped */
#define RSSM_STATUS_SLOT 4u   /* conventional: slot index out of range */

/* replayssm_flush flags. */
#define RSSM_FLUSH_FORCE_CAST 1 /* also rewrite the read copy of sequences with nothing to fold */

#define RSSM_MAX_DRAFTS 8
#define RSSM_MAX_WINDOW 64

typedef struct {
    int32_t batch, nheads, headdim, dstate, ngroups;
    int32_t window;     /* L: a call that starts with >= L committed records flushes first */
    int32_t max_drafts; /* T_max: largest T passed to replayssm_verify_drafts */
    int32_t in_dtype;   /* RSSM_F32 or RSSM_BF16: tokens x, B, C and the x/B records */
    int32_t read_copy;  /* RSSM_NONE, RSSM_BF16, RSSM_FP8_E4M3, RSSM_MXFP4 or RSSM_MXFP8 (the MX modes
                           need dstate % 32 == 0) */
    int32_t ckpt_dtype; /* RSSM_F32 (0): FP32 checkpoint.  RSSM_F16: half-precision recurrence
                           checkpoint (blog section "Benefit 3": a half-precision recurrence state
                           stays close to FP32 when its writes round stochastically): each flush
                           computes the new state in fp32
                           registers, writes it to fp16 with stochastic rounding (see
                           rssm_params.sr_seed) and casts the read copy from the same registers;
                           non-flush calls read the fp16 checkpoint itself when read_copy is
                           RSSM_NONE.  With RSSM_F16, read_copy must be RSSM_NONE or RSSM_MXFP4
                           (else RSSM_ERR_DTYPE).  The conventional entry points need RSSM_F32. */
} rssm_config;

/*
 * Per-layer decode state.  cap = window + 2*max_drafts - 1 record slots per
 * sequence, used as a ring: record k of the window lives in slot
 * (start + k) % cap.  Every head keeps its own copy of the ring pointer
 * {start, len}; all copies of a sequence hold the same values (initialise them
 * together; the library keeps them equal).  A workgroup then writes only the
 * copies of the heads it owns and never waits on another workgroup; it also
 * reads the sequence's first copy and reports RSSM_STATUS_META when that copy
 * holds neither its own pair nor the pair it is about to write.  Each copy is
 * read and written as one 8-byte word (meta must be 8-byte aligned).
 */
typedef struct {
    void *ckpt;         /* [batch][nheads][headdim][dstate] checkpoint H_s: fp32, or fp16 bits with
                           ckpt_dtype == RSSM_F16 */
    void *ckpt_read;    /* same layout in read_copy's type; NULL iff read_copy == RSSM_NONE.
                           MXFP4: [batch][nheads][headdim][dstate/2] bytes, two E2M1 codes per
                           byte, the lower column in the low nibble; MXFP8: one e4m3 byte per
                           element */
    void *ckpt_scale;   /* e4m3: [batch][nheads] fp32, one scale per tile; MXFP4 and MXFP8:
                           [batch][nheads][headdim][dstate/32] E8M0 bytes, one per block of 32
                           columns (scale 2^(e-127); e = 255 marks a block holding a NaN);
                           NULL for the other modes */
    void *buf_x;        /* [batch][nheads][cap][headdim] in_dtype */
    void *buf_B;        /* [batch][ngroups][cap][dstate] in_dtype */
    float *buf_dt;      /* [batch][nheads][cap] fp32 (after softplus) */
    int32_t *meta;      /* [batch][nheads][2] = {ring start, committed length}, 0 <= start < cap */
    int32_t *status;    /* one int32 of sticky RSSM_STATUS_* bits, or NULL */
} rssm_state;

/* T consecutive tokens per sequence (decode: T == 1). */
typedef struct {
    const void *x;    /* [batch][T][nheads][headdim] in_dtype */
    const void *B;    /* [batch][T][ngroups][dstate] in_dtype */
    const void *C;    /* [batch][T][ngroups][dstate] in_dtype */
    const float *dt;  /* [batch][T][nheads] fp32 (after softplus) */
    int32_t T;
} rssm_tokens;

typedef struct {
    const float *A;   /* [nheads], negative */
    const float *D;   /* [nheads] skip */
    uint64_t sr_seed; /* RSSM_F16 checkpoint only: key of this call's rounding.  A flush rounds
                         checkpoint element 4v + e (row-major over the whole array) away from zero
                         iff its distance above the fp16 value below it, in units of their
                         spacing and taken to 13 bits, plus the low 13 bits of word e of
                         Philox4x32-10 (Salmon et al., SC 2011) at counter (v low 32 bits, v high
                         32 bits, 0, 0) under key (sr_seed low, sr_seed high) reaches 2^13.  Pass a
                         new value on every call (a step counter will do), or flushes reuse the
                         same random words; |v| >= 65504 saturates, NaN stays NaN. */
} rssm_params;

/* Buffers of rssm_state, in the order of replayssm_sizes(). */
#define RSSM_BUF_CKPT 0
#define RSSM_BUF_CKPT_READ 1
#define RSSM_BUF_CKPT_SCALE 2
#define RSSM_BUF_X 3
#define RSSM_BUF_B 4
#define RSSM_BUF_DT 5
#define RSSM_BUF_META 6
#define RSSM_NUM_BUFS 7

/* Host only.  Ring capacity cap = window + 2*max_drafts - 1 (or an error code). */
int replayssm_capacity(const rssm_config *cfg);

/* Host only.  Bytes of each rssm_state buffer (0 for buffers the config does
 * not use).  Returns RSSM_OK or an error code; validates the config. */
int replayssm_sizes(const rssm_config *cfg, size_t bytes[RSSM_NUM_BUFS]);

/*
 * One decode token per sequence (tokens->T == 1).
 * Blog section "How ReplaySSM represents the state": a non-flush step appends
 * the token's record and computes y from the checkpoint and the buffer without
 * storing any state; once L records are committed the buffered inputs are
 * folded into the checkpoint, written once, and the buffer restarts.  Here the
 * flush happens at the start of the call that finds len >= L, then that call
 * continues as a non-flush step on the new checkpoint.
 * Effect per sequence: (flush if len >= L), y[b][0] = output of the token,
 * record appended at slot (start + len) % cap, len += 1.
 * y: [batch][1][nheads][headdim] fp32.  With a read copy, non-flush calls read
 * the copy instead of the FP32 checkpoint (blog section "Benefit 3").
 */
int replayssm_decode_step(const rssm_config *cfg, const rssm_state *st, const rssm_params *p,
                          const rssm_tokens *tok, float *y, void *stream);

/*
 * Fold every sequence's committed records into its checkpoint (sequences with
 * len == 0 are left alone), write the FP32 checkpoint and its read copy, and
 * empty the buffer (start += len, len = 0).  Blog sections "How ReplaySSM
 * represents the state" (the flush) and "Benefit 3" (the flush casts the new
 * checkpoint into both precisions independently).  flags:
 * RSSM_FLUSH_FORCE_CAST also recasts the read copy of sequences with len == 0;
 * use it once to create the read copy of an initial checkpoint.
 */
int replayssm_flush(const rssm_config *cfg, const rssm_state *st, const rssm_params *p,
                    int32_t flags, void *stream);

/*
 * Speculative verification of T drafts per sequence, 1 <= T <= max_drafts.
 * Blog section "Benefit 2: Simplify rollback and speed up verification": the
 * records of all T drafts are appended past the buffer pointer and the T
 * outputs are evaluated output-only from the checkpoint (read once for all T
 * queries) and the buffer; no state is written unless the call starts with
 * len >= L, in which case the committed records (never the drafts) are folded
 * first.  len is unchanged; replayssm_commit then advances it.
 * y: [batch][T][nheads][headdim] fp32; draft q sees records 0..len-1 and
 * drafts 0..q.
 */
int replayssm_verify_drafts(const rssm_config *cfg, const rssm_state *st, const rssm_params *p,
                            const rssm_tokens *tok, float *y, void *stream);

/*
 * Commit the accepted prefix of the last verification: len += accepted[b]
 * (device array [batch], 0 <= accepted[b] <= T).  Rollback is this pointer
 * move alone; draft records past the pointer are ignored and overwritten by
 * the next append (blog section "Benefit 2").
 */
int replayssm_commit(const rssm_config *cfg, const rssm_state *st, const int32_t *accepted,
                     int32_t T, void *stream);

/*
 * replayssm_commit(accepted_prev, T_prev) followed by
 * replayssm_verify_drafts(tok), in one launch: each head's workgroup advances
 * its own copy of the ring pointer by accepted_prev[b] before it verifies the
 * new drafts, so a speculative round costs one launch instead of two.  Same
 * results, bit for bit, as the two calls (blog section "Benefit 2": rollback
 * is only the pointer move).  An accepted count outside 0..T_prev sets
 * RSSM_STATUS_ACCEPT, writes NaN outputs and leaves that sequence's state
 * untouched.
 */
int replayssm_commit_verify(const rssm_config *cfg, const rssm_state *st, const rssm_params *p,
                            const int32_t *accepted_prev, int32_t T_prev, const rssm_tokens *tok,
                            float *y, void *stream);

/*
 * Baseline: the conventional Mamba-2 decode step, which loads the full state,
 * decays it, adds the rank-1 update, reads the output and stores the state
 * (blog section "Why SSM layers can become a decoding bottleneck"), and its
 * speculative variant that stores one state snapshot per draft (blog section
 * "Rollback for speculative decoding").
 *   states [batch][nslots][nheads][headdim][dstate] fp32.
 *   nslots == 1: tok->T must be 1 and the state is updated in place; `slot`
 *     may be NULL.
 *   nslots > 1: slot[b] (device, [batch]) names the current state; draft q's
 *     state is written to slot (slot[b] + 1 + q) % nslots, 1 <= T < nslots.
 *     The current slot is read once and never written.
 * y: [batch][T][nheads][headdim] fp32.  Uses cfg's shape and in_dtype only.
 */
int conventional_state_update(const rssm_config *cfg, float *states, int32_t nslots,
                              const int32_t *slot, int32_t *status, const rssm_params *p,
                              const rssm_tokens *tok, float *y, void *stream);

/* Baseline commit: slot[b] = (slot[b] + accepted[b]) % nslots, 0 <= accepted[b] <= T. */
int conventional_commit(const rssm_config *cfg, int32_t *slot, int32_t nslots,
                        const int32_t *accepted, int32_t T, int32_t *status, void *stream);

/* Message of the last failed call on this thread ("" if none). */
const char *replayssm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* REPLAYSSM_H */
