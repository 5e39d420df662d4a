// C ABI of libreplayssm: argument checks, dispatch and launches on the
// caller's stream.  Declarations and semantics: include/replayssm.h.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/replayssm.h"
#include "../../include/replayssm_gdn.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr size_t kMaxLds = 64 * 1024;

// Shape, type and limit checks shared by every entry point.
int check_config(const rssm_config* c, bool need_window) {
    if (!c) return fail(RSSM_ERR_NULL, "config is NULL");
    if (c->batch < 0) return fail(RSSM_ERR_SHAPE, "batch %d < 0", c->batch);
    if (c->nheads <= 0 || c->ngroups <= 0 || c->nheads % c->ngroups != 0)
        return fail(RSSM_ERR_SHAPE, "nheads %d must be a positive multiple of ngroups %d", c->nheads,
                    c->ngroups);
    if (!rssm::shape_supported(c->headdim, c->dstate))
        return fail(RSSM_ERR_SHAPE,
                    "(headdim, dstate) = (%d, %d) not compiled; supported: (16,16) (64,64) (64,128) (128,128)",
                    c->headdim, c->dstate);
    if ((long long)c->batch * c->nheads > INT_MAX)
        return fail(RSSM_ERR_SHAPE, "batch * nheads too large");
    if (c->in_dtype != RSSM_F32 && c->in_dtype != RSSM_BF16)
        return fail(RSSM_ERR_DTYPE, "in_dtype must be RSSM_F32 or RSSM_BF16");
    if (need_window) {
        if (c->window < 1 || c->window > RSSM_MAX_WINDOW)
            return fail(RSSM_ERR_SHAPE, "window %d outside 1..%d", c->window, RSSM_MAX_WINDOW);
        if (c->max_drafts < 1 || c->max_drafts > RSSM_MAX_DRAFTS)
            return fail(RSSM_ERR_SHAPE, "max_drafts %d outside 1..%d", c->max_drafts, RSSM_MAX_DRAFTS);
        if (c->read_copy != RSSM_NONE && c->read_copy != RSSM_BF16 && c->read_copy != RSSM_FP8_E4M3 &&
            c->read_copy != RSSM_MXFP4 && c->read_copy != RSSM_MXFP8)
            return fail(RSSM_ERR_DTYPE,
                        "read_copy must be RSSM_NONE, RSSM_BF16, RSSM_FP8_E4M3, RSSM_MXFP4 or RSSM_MXFP8");
        if (c->ckpt_dtype != RSSM_F32 && c->ckpt_dtype != RSSM_F16)
            return fail(RSSM_ERR_DTYPE, "ckpt_dtype must be RSSM_F32 or RSSM_F16");
        if (c->ckpt_dtype == RSSM_F16 && c->read_copy != RSSM_NONE && c->read_copy != RSSM_MXFP4)
            return fail(RSSM_ERR_DTYPE,
                        "an RSSM_F16 checkpoint is read directly (RSSM_NONE) or through an RSSM_MXFP4 copy");
        if ((c->read_copy == RSSM_MXFP4 || c->read_copy == RSSM_MXFP8) && c->dstate % 32 != 0)
            return fail(RSSM_ERR_SHAPE, "the MX read copies need dstate %% 32 == 0 (blocks of 32 columns), got %d",
                        c->dstate);
        const int cap = c->window + 2 * c->max_drafts - 1;
        if (rssm::replay_lds_bytes(c->headdim, c->dstate, cap, c->max_drafts, c->in_dtype == RSSM_BF16 ? 2 : 4) >
            kMaxLds)
            return fail(RSSM_ERR_SHAPE, "window/max_drafts need more than 64 KiB of LDS");
    }
    return RSSM_OK;
}

int read_mode(const rssm_config* c) {
    if (c->ckpt_dtype == RSSM_F16 && c->read_copy == RSSM_NONE) return rssm::READ_F16;
    return c->read_copy == RSSM_BF16       ? rssm::READ_BF16
           : c->read_copy == RSSM_FP8_E4M3 ? rssm::READ_E4M3
           : c->read_copy == RSSM_MXFP4    ? rssm::READ_MXFP4
           : c->read_copy == RSSM_MXFP8    ? rssm::READ_MXFP8
                                            : rssm::READ_F32;
}

int check_state(const rssm_config* c, const rssm_state* s) {
    if (!s) return fail(RSSM_ERR_NULL, "state is NULL");
    if (!s->ckpt || !s->buf_x || !s->buf_B || !s->buf_dt || !s->meta)
        return fail(RSSM_ERR_NULL, "state: ckpt, buf_x, buf_B, buf_dt and meta are required");
    if ((c->read_copy == RSSM_NONE) != (s->ckpt_read == nullptr))
        return fail(RSSM_ERR_NULL, "state: ckpt_read must be set iff read_copy != RSSM_NONE");
    if ((c->read_copy == RSSM_FP8_E4M3 || c->read_copy == RSSM_MXFP4 || c->read_copy == RSSM_MXFP8) !=
        (s->ckpt_scale != nullptr))
        return fail(RSSM_ERR_NULL,
                    "state: ckpt_scale must be set iff read_copy is RSSM_FP8_E4M3, RSSM_MXFP4 or RSSM_MXFP8");
    if (!aligned(s->ckpt, 16) || !aligned(s->buf_x, 16) || !aligned(s->buf_B, 16) ||
        (s->ckpt_read && !aligned(s->ckpt_read, 16)))
        return fail(RSSM_ERR_SHAPE, "state: ckpt, ckpt_read, buf_x and buf_B must be 16-byte aligned");
    if (!aligned(s->buf_dt, 4) || !aligned(s->meta, 8) ||
        (s->ckpt_scale && !aligned(s->ckpt_scale, 4)) || (s->status && !aligned(s->status, 4)))
        return fail(RSSM_ERR_SHAPE, "state: misaligned scalar buffer");
    return RSSM_OK;
}

int check_tokens(const rssm_tokens* t, const rssm_params* p, const float* y, int tmin, int tmax) {
    if (!t || !p) return fail(RSSM_ERR_NULL, "tokens or params is NULL");
    if (!t->x || !t->B || !t->C || !t->dt || !p->A || !p->D || !y)
        return fail(RSSM_ERR_NULL, "tokens x, B, C, dt, params A, D and y are required");
    if (t->T < tmin || t->T > tmax)
        return fail(RSSM_ERR_DRAFTS, "T = %d outside %d..%d", t->T, tmin, tmax);
    if (!aligned(t->x, 16) || !aligned(t->B, 16) || !aligned(t->C, 16) || !aligned(t->dt, 4) ||
        !aligned(y, 4) || !aligned(p->A, 4) || !aligned(p->D, 4))
        return fail(RSSM_ERR_SHAPE, "tokens x, B, C must be 16-byte aligned");
    return RSSM_OK;
}

// log2 of a positive power of two, else -1.
int log2_exact(int v) {
    if (v <= 0 || (v & (v - 1)) != 0) return -1;
    int l = 0;
    while ((1 << l) < v) ++l;
    return l;
}

rssm::ReplayArgs replay_args(const rssm_config* c, const rssm_state* s, const rssm_params* p) {
    rssm::ReplayArgs a;
    std::memset(&a, 0, sizeof a);
    a.ckpt = static_cast<float*>(s->ckpt);
    a.ckpt16 = c->ckpt_dtype == RSSM_F16;
    a.ckpt_read = s->ckpt_read;
    a.ckpt_scale = static_cast<float*>(s->ckpt_scale);
    a.buf_x = s->buf_x;
    a.buf_B = s->buf_B;
    a.buf_dt = s->buf_dt;
    a.meta = s->meta;
    a.status = s->status;
    a.A = p ? p->A : nullptr;
    a.D = p ? p->D : nullptr;
    a.sr_seed = p ? p->sr_seed : 0;
    a.batch = c->batch;
    a.nheads = c->nheads;
    a.ngroups = c->ngroups;
    a.L = c->window;
    a.cap = c->window + 2 * c->max_drafts - 1;
    a.nheads_log2 = log2_exact(c->nheads);
    a.hpg_log2 = c->ngroups > 0 && c->nheads % c->ngroups == 0 ? log2_exact(c->nheads / c->ngroups) : -1;
    return a;
}

int launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(RSSM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    g_err[0] = '\0';
    return RSSM_OK;
}

int run_replay(const rssm_config* c, const rssm_state* s, const rssm_params* p, const rssm_tokens* t,
               float* y, int mode, int flags, void* stream, const char* what,
               const int32_t* accepted_prev = nullptr, int32_t T_prev = 0) {
    rssm::ReplayArgs a = replay_args(c, s, p);
    a.accepted_prev = accepted_prev;
    a.T_prev = T_prev;
    if (t) {
        a.x = t->x;
        a.B = t->B;
        a.C = t->C;
        a.dt = t->dt;
        a.T = t->T;
    }
    a.y = y;
    a.mode = mode;
    a.flags = flags;
    if (c->batch == 0) return RSSM_OK;
    const int in_type = c->in_dtype == RSSM_BF16 ? rssm::IN_BF16 : rssm::IN_F32;
    return launched(rssm::launch_replay(a, c->headdim, c->dstate, in_type, read_mode(c),
                                        static_cast<hipStream_t>(stream)),
                    what);
}


// ---- Gated DeltaNet layer --------------------------------------------------

int gdn_check_config(const gdn_config* c) {
    if (!c) return fail(RSSM_ERR_NULL, "config is NULL");
    if (c->batch < 0) return fail(RSSM_ERR_SHAPE, "batch %d < 0", c->batch);
    if (c->nv <= 0 || c->nk <= 0 || c->nv % c->nk != 0)
        return fail(RSSM_ERR_SHAPE, "nv %d must be a positive multiple of nk %d", c->nv, c->nk);
    if (!rssm::gdn_shape_supported(c->dk, c->dv))
        return fail(RSSM_ERR_SHAPE, "(dk, dv) = (%d, %d) not compiled; supported: dk 16 with dv %% 16 == 0, "
                    "dk 128 with dv %% 64 == 0", c->dk, c->dv);
    if ((long long)c->batch * c->nv * (c->dv / rssm::gdn_rows(c->dk)) > INT_MAX)
        return fail(RSSM_ERR_SHAPE, "batch * nv * row blocks too large");
    if (c->in_dtype != RSSM_F32 && c->in_dtype != RSSM_BF16)
        return fail(RSSM_ERR_DTYPE, "in_dtype must be RSSM_F32 or RSSM_BF16");
    if (c->ckpt_dtype != RSSM_F32 && c->ckpt_dtype != RSSM_F16)
        return fail(RSSM_ERR_DTYPE, "ckpt_dtype must be RSSM_F32 or RSSM_F16");
    if (c->window < 1 || c->window > RSSM_MAX_WINDOW)
        return fail(RSSM_ERR_SHAPE, "window %d outside 1..%d", c->window, RSSM_MAX_WINDOW);
    if (c->max_drafts < 1 || c->max_drafts > RSSM_MAX_DRAFTS)
        return fail(RSSM_ERR_SHAPE, "max_drafts %d outside 1..%d", c->max_drafts, RSSM_MAX_DRAFTS);
    if (rssm::gdn_lds_bytes(c->dk, c->window + 2 * c->max_drafts - 1, c->max_drafts) > kMaxLds)
        return fail(RSSM_ERR_SHAPE, "window/max_drafts need more than 64 KiB of LDS");
    return RSSM_OK;
}

int gdn_check_state(const gdn_state* s) {
    if (!s) return fail(RSSM_ERR_NULL, "state is NULL");
    if (!s->ckpt || !s->buf_k || !s->buf_u || !s->buf_g || !s->meta)
        return fail(RSSM_ERR_NULL, "state: ckpt, buf_k, buf_u, buf_g and meta are required");
    if (!aligned(s->ckpt, 16) || !aligned(s->buf_k, 16) || !aligned(s->buf_u, 16))
        return fail(RSSM_ERR_SHAPE, "state: ckpt, buf_k and buf_u must be 16-byte aligned");
    if (!aligned(s->buf_g, 4) || !aligned(s->meta, 8) || (s->status && !aligned(s->status, 4)))
        return fail(RSSM_ERR_SHAPE, "state: misaligned scalar buffer");
    return RSSM_OK;
}

int gdn_check_tokens(const gdn_tokens* t, const float* o, int tmin, int tmax) {
    if (!t) return fail(RSSM_ERR_NULL, "tokens is NULL");
    if (!t->q || !t->k || !t->v || !t->g || !t->beta || !o)
        return fail(RSSM_ERR_NULL, "tokens q, k, v, g, beta and o are required");
    if (t->T < tmin || t->T > tmax) return fail(RSSM_ERR_DRAFTS, "T = %d outside %d..%d", t->T, tmin, tmax);
    if (!aligned(t->q, 16) || !aligned(t->k, 16) || !aligned(t->v, 16))
        return fail(RSSM_ERR_SHAPE, "tokens q, k, v must be 16-byte aligned");
    if (!aligned(t->g, 4) || !aligned(t->beta, 4) || !aligned(o, 4))
        return fail(RSSM_ERR_SHAPE, "misaligned g, beta or o");
    return RSSM_OK;
}

rssm::GdnArgs gdn_args(const gdn_config* c, const gdn_state* s, const gdn_tokens* t, float* o, int mode) {
    rssm::GdnArgs a;
    std::memset(&a, 0, sizeof a);
    if (s) {
        a.ckpt = static_cast<float*>(s->ckpt);
        a.buf_k = s->buf_k;
        a.buf_u = s->buf_u;
        a.buf_g = s->buf_g;
        a.meta = s->meta;
        a.status = s->status;
    }
    if (t) {
        a.q = t->q;
        a.k = t->k;
        a.v = t->v;
        a.g = t->g;
        a.beta = t->beta;
        a.T = t->T;
        a.sr_seed = t->sr_seed;
    }
    a.o = o;
    a.batch = c->batch;
    a.nv = c->nv;
    a.nk = c->nk;
    a.dv = c->dv;
    a.parts = c->dv / rssm::gdn_rows(c->dk);
    a.L = c->window;
    a.cap = c->window + 2 * c->max_drafts - 1;
    a.mode = mode;
    a.ckpt16 = c->ckpt_dtype == RSSM_F16;
    a.parts_log2 = log2_exact(a.parts);
    a.nv_log2 = log2_exact(c->nv);
    a.hpk_log2 = c->nk > 0 && c->nv % c->nk == 0 ? log2_exact(c->nv / c->nk) : -1;
    return a;
}

int run_gdn(const gdn_config* c, const gdn_state* s, const gdn_tokens* t, float* o, int mode, void* stream,
            const char* what) {
    const rssm::GdnArgs a = gdn_args(c, s, t, o, mode);
    return launched(rssm::launch_gdn_replay(a, c->dk, c->in_dtype == RSSM_BF16 ? rssm::IN_BF16 : rssm::IN_F32,
                                            static_cast<hipStream_t>(stream)),
                    what);
}

}  // namespace

extern "C" {

int replayssm_capacity(const rssm_config* cfg) {
    const int rc = check_config(cfg, true);
    if (rc) return rc;
    return cfg->window + 2 * cfg->max_drafts - 1;
}

int replayssm_sizes(const rssm_config* c, size_t bytes[RSSM_NUM_BUFS]) {
    const int rc = check_config(c, true);
    if (rc) return rc;
    if (!bytes) return fail(RSSM_ERR_NULL, "bytes is NULL");
    const size_t tiles = (size_t)c->batch * c->nheads;
    const size_t tile = (size_t)c->headdim * c->dstate;
    const size_t cap = (size_t)(c->window + 2 * c->max_drafts - 1);
    const size_t in_bytes = c->in_dtype == RSSM_BF16 ? 2 : 4;
    bytes[RSSM_BUF_CKPT] = tiles * tile * (c->ckpt_dtype == RSSM_F16 ? 2 : 4);
    bytes[RSSM_BUF_CKPT_READ] = c->read_copy == RSSM_BF16       ? tiles * tile * 2
                                : c->read_copy == RSSM_FP8_E4M3 ? tiles * tile
                                : c->read_copy == RSSM_MXFP8    ? tiles * tile
                                : c->read_copy == RSSM_MXFP4    ? tiles * tile / 2
                                                                : 0;
    bytes[RSSM_BUF_CKPT_SCALE] = c->read_copy == RSSM_FP8_E4M3 ? tiles * 4
                                 : c->read_copy == RSSM_MXFP4  ? tiles * tile / 32
                                 : c->read_copy == RSSM_MXFP8  ? tiles * tile / 32
                                                               : 0;
    bytes[RSSM_BUF_X] = tiles * cap * c->headdim * in_bytes;
    bytes[RSSM_BUF_B] = (size_t)c->batch * c->ngroups * cap * c->dstate * in_bytes;
    bytes[RSSM_BUF_DT] = tiles * cap * 4;
    bytes[RSSM_BUF_META] = tiles * 2 * 4;
    g_err[0] = '\0';
    return RSSM_OK;
}

int replayssm_decode_step(const rssm_config* cfg, const rssm_state* st, const rssm_params* p,
                          const rssm_tokens* tok, float* y, void* stream) {
    int rc = check_config(cfg, true);
    if (rc) return rc;
    if (cfg->batch == 0) return RSSM_OK;
    rc = check_state(cfg, st);
    if (!rc) rc = check_tokens(tok, p, y, 1, 1);
    if (rc) return rc;
    return run_replay(cfg, st, p, tok, y, rssm::MODE_DECODE, 0, stream, "replayssm_decode_step");
}

int replayssm_flush(const rssm_config* cfg, const rssm_state* st, const rssm_params* p, int32_t flags,
                    void* stream) {
    int rc = check_config(cfg, true);
    if (rc) return rc;
    if (flags & ~RSSM_FLUSH_FORCE_CAST) return fail(RSSM_ERR_SHAPE, "unknown flush flags 0x%x", flags);
    if (cfg->batch == 0) return RSSM_OK;
    rc = check_state(cfg, st);
    if (rc) return rc;
    if (!p || !p->A || !p->D) return fail(RSSM_ERR_NULL, "params A and D are required");
    return run_replay(cfg, st, p, nullptr, nullptr, rssm::MODE_FLUSH, flags, stream, "replayssm_flush");
}

int replayssm_verify_drafts(const rssm_config* cfg, const rssm_state* st, const rssm_params* p,
                            const rssm_tokens* tok, float* y, void* stream) {
    int rc = check_config(cfg, true);
    if (rc) return rc;
    if (cfg->batch == 0) return RSSM_OK;
    rc = check_state(cfg, st);
    if (!rc) rc = check_tokens(tok, p, y, 1, cfg->max_drafts);
    if (rc) return rc;
    return run_replay(cfg, st, p, tok, y, rssm::MODE_VERIFY, 0, stream, "replayssm_verify_drafts");
}

int replayssm_commit_verify(const rssm_config* cfg, const rssm_state* st, const rssm_params* p,
                            const int32_t* accepted_prev, int32_t T_prev, const rssm_tokens* tok, float* y,
                            void* stream) {
    int rc = check_config(cfg, true);
    if (rc) return rc;
    if (T_prev < 1 || T_prev > cfg->max_drafts)
        return fail(RSSM_ERR_DRAFTS, "T_prev = %d outside 1..%d", T_prev, cfg->max_drafts);
    if (cfg->batch == 0) return RSSM_OK;
    if (!accepted_prev) return fail(RSSM_ERR_NULL, "accepted_prev is required");
    if (!aligned(accepted_prev, 4)) return fail(RSSM_ERR_SHAPE, "misaligned accepted_prev");
    rc = check_state(cfg, st);
    if (!rc) rc = check_tokens(tok, p, y, 1, cfg->max_drafts);
    if (rc) return rc;
    return run_replay(cfg, st, p, tok, y, rssm::MODE_VERIFY, 0, stream, "replayssm_commit_verify",
                      accepted_prev, T_prev);
}

int replayssm_commit(const rssm_config* cfg, const rssm_state* st, const int32_t* accepted, int32_t T,
                     void* stream) {
    int rc = check_config(cfg, true);
    if (rc) return rc;
    if (T < 1 || T > cfg->max_drafts) return fail(RSSM_ERR_DRAFTS, "T = %d outside 1..%d", T, cfg->max_drafts);
    if (cfg->batch == 0) return RSSM_OK;
    if (!st || !st->meta || !accepted) return fail(RSSM_ERR_NULL, "state meta and accepted are required");
    if (!aligned(st->meta, 8) || !aligned(accepted, 4) || (st->status && !aligned(st->status, 4)))
        return fail(RSSM_ERR_SHAPE, "misaligned meta, accepted or status");
    rssm::CommitArgs a;
    std::memset(&a, 0, sizeof a);
    a.meta = st->meta;
    a.accepted = accepted;
    a.status = st->status;
    a.batch = cfg->batch;
    a.nheads = cfg->nheads;
    a.T = T;
    a.cap = cfg->window + 2 * cfg->max_drafts - 1;
    return launched(rssm::launch_replay_commit(a, static_cast<hipStream_t>(stream)), "replayssm_commit");
}

int conventional_state_update(const rssm_config* cfg, float* states, int32_t nslots, const int32_t* slot,
                              int32_t* status, const rssm_params* p, const rssm_tokens* tok, float* y,
                              void* stream) {
    int rc = check_config(cfg, false);
    if (rc) return rc;
    if (cfg->ckpt_dtype != RSSM_F32) return fail(RSSM_ERR_DTYPE, "the conventional state is fp32 (ckpt_dtype RSSM_F32)");
    if (cfg->batch == 0) return RSSM_OK;
    if (!states) return fail(RSSM_ERR_NULL, "states is NULL");
    if (!aligned(states, 16)) return fail(RSSM_ERR_SHAPE, "states must be 16-byte aligned");
    if (nslots < 1) return fail(RSSM_ERR_SHAPE, "nslots %d < 1", nslots);
    if (nslots > 1 && !slot) return fail(RSSM_ERR_NULL, "slot is required when nslots > 1");
    const int tmax = nslots == 1 ? 1 : (nslots - 1 < RSSM_MAX_DRAFTS ? nslots - 1 : RSSM_MAX_DRAFTS);
    rc = check_tokens(tok, p, y, 1, tmax);
    if (rc) return rc;
    if (rssm::conventional_lds_bytes(cfg->headdim, cfg->dstate, tok->T) > kMaxLds)
        return fail(RSSM_ERR_SHAPE, "T too large for LDS");
    if (slot && !aligned(slot, 4)) return fail(RSSM_ERR_SHAPE, "misaligned slot");
    rssm::ConvArgs a;
    std::memset(&a, 0, sizeof a);
    a.states = states;
    a.slot = slot;
    a.status = status;
    a.x = tok->x;
    a.B = tok->B;
    a.C = tok->C;
    a.dt = tok->dt;
    a.A = p->A;
    a.D = p->D;
    a.y = y;
    a.batch = cfg->batch;
    a.nheads = cfg->nheads;
    a.ngroups = cfg->ngroups;
    a.nslots = nslots;
    a.T = tok->T;
    const int in_type = cfg->in_dtype == RSSM_BF16 ? rssm::IN_BF16 : rssm::IN_F32;
    return launched(rssm::launch_conventional(a, cfg->headdim, cfg->dstate, in_type,
                                              static_cast<hipStream_t>(stream)),
                    "conventional_state_update");
}

int conventional_commit(const rssm_config* cfg, int32_t* slot, int32_t nslots, const int32_t* accepted,
                        int32_t T, int32_t* status, void* stream) {
    if (!cfg) return fail(RSSM_ERR_NULL, "config is NULL");
    if (cfg->batch < 0) return fail(RSSM_ERR_SHAPE, "batch %d < 0", cfg->batch);
    if (nslots < 2) return fail(RSSM_ERR_SHAPE, "nslots %d < 2", nslots);
    if (T < 1 || T >= nslots) return fail(RSSM_ERR_DRAFTS, "T = %d outside 1..%d", T, nslots - 1);
    if (cfg->batch == 0) return RSSM_OK;
    if (!slot || !accepted) return fail(RSSM_ERR_NULL, "slot and accepted are required");
    if (!aligned(slot, 4) || !aligned(accepted, 4) || (status && !aligned(status, 4)))
        return fail(RSSM_ERR_SHAPE, "misaligned slot, accepted or status");
    rssm::CommitArgs a;
    std::memset(&a, 0, sizeof a);
    a.slot = slot;
    a.accepted = accepted;
    a.status = status;
    a.batch = cfg->batch;
    a.T = T;
    a.nslots = nslots;
    return launched(rssm::launch_conventional_commit(a, static_cast<hipStream_t>(stream)),
                    "conventional_commit");
}

int gdn_row_blocks(const gdn_config* cfg) {
    const int rc = gdn_check_config(cfg);
    if (rc) return rc;
    return cfg->dv / rssm::gdn_rows(cfg->dk);
}

int gdn_sizes(const gdn_config* c, size_t bytes[GDN_NUM_BUFS]) {
    const int rc = gdn_check_config(c);
    if (rc) return rc;
    if (!bytes) return fail(RSSM_ERR_NULL, "bytes is NULL");
    const size_t cap = (size_t)(c->window + 2 * c->max_drafts - 1);
    const size_t in_bytes = c->in_dtype == RSSM_BF16 ? 2 : 4;
    const size_t heads = (size_t)c->batch * c->nv;
    bytes[0] = heads * c->dv * c->dk * (c->ckpt_dtype == RSSM_F16 ? 2 : 4);
    bytes[1] = (size_t)c->batch * c->nk * cap * c->dk * in_bytes;
    bytes[2] = heads * cap * c->dv * 4;
    bytes[3] = heads * cap * 4;
    bytes[4] = heads * (c->dv / rssm::gdn_rows(c->dk)) * 2 * 4;
    g_err[0] = '\0';
    return RSSM_OK;
}

int gdn_decode_step(const gdn_config* cfg, const gdn_state* st, const gdn_tokens* tok, float* o, void* stream) {
    int rc = gdn_check_config(cfg);
    if (rc) return rc;
    if (cfg->batch == 0) return RSSM_OK;
    rc = gdn_check_state(st);
    if (!rc) rc = gdn_check_tokens(tok, o, 1, 1);
    if (rc) return rc;
    return run_gdn(cfg, st, tok, o, rssm::MODE_DECODE, stream, "gdn_decode_step");
}

int gdn_verify_drafts(const gdn_config* cfg, const gdn_state* st, const gdn_tokens* tok, float* o, void* stream) {
    int rc = gdn_check_config(cfg);
    if (rc) return rc;
    if (cfg->batch == 0) return RSSM_OK;
    rc = gdn_check_state(st);
    if (!rc) rc = gdn_check_tokens(tok, o, 1, cfg->max_drafts);
    if (rc) return rc;
    return run_gdn(cfg, st, tok, o, rssm::MODE_VERIFY, stream, "gdn_verify_drafts");
}

int gdn_commit_verify(const gdn_config* cfg, const gdn_state* st, const int32_t* accepted_prev, int32_t T_prev,
                      const gdn_tokens* tok, float* o, void* stream) {
    int rc = gdn_check_config(cfg);
    if (rc) return rc;
    if (T_prev < 1 || T_prev > cfg->max_drafts)
        return fail(RSSM_ERR_DRAFTS, "T_prev = %d outside 1..%d", T_prev, cfg->max_drafts);
    if (cfg->batch == 0) return RSSM_OK;
    if (!accepted_prev) return fail(RSSM_ERR_NULL, "accepted_prev is required");
    if (!aligned(accepted_prev, 4)) return fail(RSSM_ERR_SHAPE, "misaligned accepted_prev");
    rc = gdn_check_state(st);
    if (!rc) rc = gdn_check_tokens(tok, o, 1, cfg->max_drafts);
    if (rc) return rc;
    rssm::GdnArgs a = gdn_args(cfg, st, tok, o, rssm::MODE_VERIFY);
    a.accepted_prev = accepted_prev;
    a.T_prev = T_prev;
    return launched(rssm::launch_gdn_replay(a, cfg->dk, cfg->in_dtype == RSSM_BF16 ? rssm::IN_BF16 : rssm::IN_F32,
                                            static_cast<hipStream_t>(stream)),
                    "gdn_commit_verify");
}

int gdn_flush(const gdn_config* cfg, const gdn_state* st, uint64_t sr_seed, void* stream) {
    int rc = gdn_check_config(cfg);
    if (rc) return rc;
    if (cfg->batch == 0) return RSSM_OK;
    rc = gdn_check_state(st);
    if (rc) return rc;
    rssm::GdnArgs a = gdn_args(cfg, st, nullptr, nullptr, rssm::MODE_FLUSH);
    a.sr_seed = sr_seed;
    return launched(rssm::launch_gdn_replay(a, cfg->dk, cfg->in_dtype == RSSM_BF16 ? rssm::IN_BF16 : rssm::IN_F32,
                                            static_cast<hipStream_t>(stream)),
                    "gdn_flush");
}

int gdn_commit(const gdn_config* cfg, const gdn_state* st, const int32_t* accepted, int32_t T, void* stream) {
    int rc = gdn_check_config(cfg);
    if (rc) return rc;
    if (T < 1 || T > cfg->max_drafts) return fail(RSSM_ERR_DRAFTS, "T = %d outside 1..%d", T, cfg->max_drafts);
    if (cfg->batch == 0) return RSSM_OK;
    if (!st || !st->meta || !accepted) return fail(RSSM_ERR_NULL, "state meta and accepted are required");
    if (!aligned(st->meta, 8) || !aligned(accepted, 4) || (st->status && !aligned(st->status, 4)))
        return fail(RSSM_ERR_SHAPE, "misaligned meta, accepted or status");
    rssm::CommitArgs a;
    std::memset(&a, 0, sizeof a);
    a.meta = st->meta;
    a.accepted = accepted;
    a.status = st->status;
    a.batch = cfg->batch;
    a.nheads = cfg->nv * (cfg->dv / rssm::gdn_rows(cfg->dk));   // one pointer copy per workgroup
    a.T = T;
    a.cap = cfg->window + 2 * cfg->max_drafts - 1;
    return launched(rssm::launch_replay_commit(a, static_cast<hipStream_t>(stream)), "gdn_commit");
}

int gdn_conventional_update(const gdn_config* cfg, float* states, int32_t nslots, const int32_t* slot,
                            int32_t* status, const gdn_tokens* tok, float* o, void* stream) {
    int rc = gdn_check_config(cfg);
    if (rc) return rc;
    if (cfg->ckpt_dtype != RSSM_F32) return fail(RSSM_ERR_DTYPE, "the conventional GDN state is fp32 (ckpt_dtype RSSM_F32)");
    if (cfg->batch == 0) return RSSM_OK;
    if (!states) return fail(RSSM_ERR_NULL, "states is NULL");
    if (!aligned(states, 16)) return fail(RSSM_ERR_SHAPE, "states must be 16-byte aligned");
    if (nslots < 1) return fail(RSSM_ERR_SHAPE, "nslots %d < 1", nslots);
    if (nslots > 1 && !slot) return fail(RSSM_ERR_NULL, "slot is required when nslots > 1");
    if ((slot && !aligned(slot, 4)) || (status && !aligned(status, 4)))
        return fail(RSSM_ERR_SHAPE, "misaligned slot or status");
    const int tmax = nslots == 1 ? 1 : (nslots - 1 < RSSM_MAX_DRAFTS ? nslots - 1 : RSSM_MAX_DRAFTS);
    rc = gdn_check_tokens(tok, o, 1, tmax);
    if (rc) return rc;
    gdn_state s;
    std::memset(&s, 0, sizeof s);
    s.ckpt = states;
    s.status = status;
    rssm::GdnArgs a = gdn_args(cfg, &s, tok, o, rssm::MODE_DECODE);
    a.nslots = nslots;
    a.slot = nslots > 1 ? slot : nullptr;
    return launched(rssm::launch_gdn_conventional(a, cfg->dk, cfg->in_dtype == RSSM_BF16 ? rssm::IN_BF16 : rssm::IN_F32,
                                                  static_cast<hipStream_t>(stream)),
                    "gdn_conventional_update");
}

int gdn_conventional_commit(const gdn_config* cfg, int32_t* slot, int32_t nslots, const int32_t* accepted,
                            int32_t T, int32_t* status, void* stream) {
    if (!cfg) return fail(RSSM_ERR_NULL, "config is NULL");
    if (cfg->batch < 0) return fail(RSSM_ERR_SHAPE, "batch %d < 0", cfg->batch);
    if (nslots < 2) return fail(RSSM_ERR_SHAPE, "nslots %d < 2", nslots);
    if (T < 1 || T >= nslots) return fail(RSSM_ERR_DRAFTS, "T = %d outside 1..%d", T, nslots - 1);
    if (cfg->batch == 0) return RSSM_OK;
    if (!slot || !accepted) return fail(RSSM_ERR_NULL, "slot and accepted are required");
    if (!aligned(slot, 4) || !aligned(accepted, 4) || (status && !aligned(status, 4)))
        return fail(RSSM_ERR_SHAPE, "misaligned slot, accepted or status");
    rssm::CommitArgs a;
    std::memset(&a, 0, sizeof a);
    a.slot = slot;
    a.accepted = accepted;
    a.status = status;
    a.batch = cfg->batch;
    a.T = T;
    a.nslots = nslots;
    return launched(rssm::launch_conventional_commit(a, static_cast<hipStream_t>(stream)), "gdn_conventional_commit");
}

const char* replayssm_last_error(void) { return g_err; }

}  // extern "C"
