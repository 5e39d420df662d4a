"""fp64 CPU oracle of the Gated DeltaNet (GDN) decode recurrence.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg use this module; the library never does.  It shares no code
with the HIP path.

The ReplaySSM page (NVIDIA Developer blog "ReplaySSM: Rethinking State Storage
for Faster Hybrid-Model Decoding", section "Why SSM layers can become a decoding
bottleneck") names GDN as one of the SSM layers the method covers and states
that its update, which corrects the decay-plus-rank-1 step with the delta rule,
keeps that step's structure.  The page prints no GDN formula; the
definition used here is the gated delta rule of Yang, Kautz and Hatamizadeh,
"Gated Delta Networks: Improving Mamba2 with Delta Rule" (ICLR 2025), per
sequence b and value head h (key head kh(h)):

    S_t = S_{t-1} (alpha_t (I - beta_t k_t k_t^T)) + beta_t v_t k_t^T     (dv x dk)
    o_t = S_t q_t

with alpha_t = exp(g_t) (g is the log decay, <= 0) and beta_t in (0, 1).

Readings taken where the page is silent:
  - q and k arrive after the layer's normalisation and scaling (projections,
    short convolutions, L2 norms and the 1/sqrt(dk) factor are outside the
    decode step), v after its projection; g and beta after their gates;
  - value heads map to key heads in contiguous blocks: kh = h // (nv/nk);
  - the output of token t reads the state that already includes token t;
  - there is no skip term.

`conventional` is the definition, written as the matrix product of the
formula (S_{t-1} times the dk x dk transition matrix).  `Replay` is an
independent fp64 form of the page's checkpoint-plus-buffer representation
for this layer (the reading of that statement): expanding the
product gives S_t = alpha_t S_{t-1} + u_t k_t^T with the corrected value
u_t = beta_t (v_t - alpha_t S_{t-1} k_t), so a record holds (k_t, u_t, g_t),
a flush folds the records exactly as for Mamba-2 and a non-flush step needs
S_{t-1} k_t, which the checkpoint and the records give without forming a
state (section "Benefit 2", output-only evaluation, which the page says GDN
can use as well).
"""
from __future__ import annotations

import numpy as np


def key_head(h: int, nv: int, nk: int) -> int:
    """Key head read by value head h (contiguous blocks of nv/nk value heads)."""
    return h // (nv // nk)


def _kmap(nv: int, nk: int) -> np.ndarray:
    return np.array([key_head(h, nv, nk) for h in range(nv)])


def conventional(S0, q, k, v, g, beta, nsteps=None):
    """Step the gated delta rule over `steps` tokens in fp64.

    S0 [batch][nv][dv][dk]; q, k [steps][batch][nk][dk]; v [steps][batch][nv][dv];
    g, beta [steps][batch][nv]; nsteps [batch] (tokens applied to sequence b)
    or None for all.  Returns (S [batch][nv][dv][dk],
    o [steps][batch][nv][dv]); o of a token beyond nsteps[b] is NaN.
    """
    S = np.array(S0, dtype=np.float64, copy=True)
    steps, batch, nk, dk = np.shape(k)
    nv = np.shape(v)[2]
    if nv % nk:
        raise ValueError("nv must be a multiple of nk")
    km = _kmap(nv, nk)
    n = np.full(batch, steps) if nsteps is None else np.asarray(nsteps)
    o = np.full((steps, batch, nv, np.shape(v)[3]), np.nan)
    eye = np.eye(dk)
    for t in range(steps):
        act = np.nonzero(t < n)[0]
        if act.size == 0:
            continue
        kt = np.asarray(k[t], np.float64)[act][:, km]          # [b][nv][dk]
        qt = np.asarray(q[t], np.float64)[act][:, km]
        vt = np.asarray(v[t], np.float64)[act]                 # [b][nv][dv]
        alpha = np.exp(np.asarray(g[t], np.float64)[act])      # [b][nv]
        bt = np.asarray(beta[t], np.float64)[act]
        # transition matrix alpha (I - beta k k^T), dk x dk per (sequence, head)
        M = alpha[..., None, None] * (eye - bt[..., None, None] * kt[..., :, None] * kt[..., None, :])
        S[act] = np.matmul(S[act], M) + bt[..., None, None] * vt[..., :, None] * kt[..., None, :]
        o[t, act] = np.matmul(S[act], qt[..., :, None])[..., 0]
    return S, o


class Replay:
    """Checkpoint plus record buffer of one GDN layer, in fp64 (replay form).

    ckpt [batch][nv][dv][dk]; per sequence a list of records (k [nv][dk]
    gathered per value head, u [nv][dv], g [nv]) since the last fold.
    """

    def __init__(self, S0, nv: int, nk: int):
        self.ckpt = np.array(S0, dtype=np.float64, copy=True)
        self.nv, self.nk = nv, nk
        self.km = _kmap(nv, nk)
        self.records = [[] for _ in range(self.ckpt.shape[0])]

    def _applied(self, b, recs, vec):
        """S_end . vec [nv][dk] for the state S_end after the records `recs`:
        S_end = exp(sum g) ckpt + sum_c exp(sum_{i > c} g_i) u_c k_c^T, applied
        term by term without forming S_end."""
        G = np.zeros(self.nv)                     # sum of g over records after c
        acc = np.zeros((self.nv, self.ckpt.shape[2]))
        for kc, uc, gc in reversed(recs):
            acc += np.exp(G)[:, None] * np.sum(kc * vec, axis=-1)[:, None] * uc
            G = G + gc
        acc += np.exp(G)[:, None] * np.einsum("hij,hj->hi", self.ckpt[b], vec)
        return acc

    def _token(self, b, recs, q, k, v, g, beta):
        """Output and record of one token after the records `recs` of sequence b."""
        kk = np.asarray(k, np.float64)[self.km]
        qq = np.asarray(q, np.float64)[self.km]
        g = np.asarray(g, np.float64)
        # alpha_t S_{t-1} k_t from the checkpoint and the records
        Sk = np.exp(g)[:, None] * self._applied(b, recs, kk)
        u = np.asarray(beta, np.float64)[:, None] * (np.asarray(v, np.float64) - Sk)
        rec = (kk, u, g)
        return self._applied(b, recs + [rec], qq), rec

    def step(self, b, q, k, v, g, beta):
        """Decode one token of sequence b (q, k [nk][dk]; v [nv][dv]; g, beta
        [nv]) and append its record; returns o [nv][dv]."""
        o, rec = self._token(b, self.records[b], q, k, v, g, beta)
        self.records[b].append(rec)
        return o

    def verify(self, b, drafts):
        """Outputs of the drafts (a list of (q, k, v, g, beta)) of sequence b,
        each seeing the committed records and the drafts before it; nothing is
        committed.  Returns (outputs, draft records)."""
        recs, outs, new = list(self.records[b]), [], []
        for d in drafts:
            o, rec = self._token(b, recs, *d)
            recs.append(rec)
            new.append(rec)
            outs.append(o)
        return outs, new

    def commit(self, b, draft_records, a: int):
        """Keep the first a draft records of sequence b (pointer advance)."""
        self.records[b].extend(draft_records[:a])

    def fold(self, b):
        """Fold sequence b's records into its checkpoint and clear them."""
        G = np.zeros(self.nv)
        add = np.zeros_like(self.ckpt[b])
        for kc, uc, gc in reversed(self.records[b]):
            add += np.exp(G)[:, None, None] * uc[:, :, None] * kc[:, None, :]
            G = G + gc
        self.ckpt[b] = np.exp(G)[:, None, None] * self.ckpt[b] + add
        self.records[b] = []


def replay_decode(S0, q, k, v, g, beta, window: int):
    """Decode every token through the replay form with flush-at-start.

    A token that finds `window` committed records folds them first (as the
    library does).  Returns (checkpoint after folding what is left,
    o [steps][batch][nv][dv])."""
    steps, batch, nk, dk = np.shape(k)
    nv = np.shape(v)[2]
    r = Replay(S0, nv, nk)
    o = np.zeros((steps, batch, nv, np.shape(v)[3]))
    for t in range(steps):
        for b in range(batch):
            if len(r.records[b]) >= window:
                r.fold(b)
            o[t, b] = r.step(b, q[t][b], k[t][b], v[t][b], g[t][b], beta[t][b])
    for b in range(batch):
        r.fold(b)
    return r.ckpt, o
