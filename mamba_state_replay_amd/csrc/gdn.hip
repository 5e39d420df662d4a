// Gated DeltaNet (GDN) layer in ReplaySSM form on gfx950: the decode / verify /
// flush kernels over an FP32 (or FP16, stochastically rounded) checkpoint plus
// corrected-value records, and the conventional GDN step (the in-library
// baseline, with one state snapshot per draft for verification).
//
// Method: NVIDIA Developer blog "ReplaySSM: Rethinking State Storage for Faster
// Hybrid-Model Decoding".  Its section "Why SSM layers can become a decoding
// bottleneck" states that GDN's update, delta-rule correction included, has
// the decay-plus-rank-1 structure of Mamba-2's, so the checkpoint-plus-buffer state (section "How
// ReplaySSM represents the state") and output-only evaluation (section
// "Benefit 2") carry over.  The gated delta rule (Yang, Kautz and Hatamizadeh,
// "Gated Delta Networks", ICLR 2025), S_t = S_{t-1} alpha_t (I - beta_t k_t k_t^T)
// + beta_t v_t k_t^T, o_t = S_t q_t, expands to S_t = alpha_t S_{t-1} + u_t k_t^T
// with u_t = beta_t (v_t - alpha_t S_{t-1} k_t).  A record is (k, u, g = log
// alpha); u is formed when its token arrives, from the checkpoint (one more
// product with the streamed tile) and the records before it.
//
// Row i of u_t needs only row i of S_{t-1}, so the rows of a value head's state
// are independent: a head's dv x dk state is split into blocks of ROWS rows,
// one workgroup each, streaming one ROWS x DK fp32 tile (64 x 128 = 32 KiB)
// with the thread layout of TileGeo (8 lanes per row, 16-byte loads).  An FP16
// checkpoint with dk = 128 and dv a multiple of 128 has its own kernel
// (gdn_replay_f16_wide_kernel) that serves two row blocks per workgroup, so a
// workgroup still streams 32 KiB.
//
// One call of gdn_replay_kernel, workgroup = (sequence b, value head h, row block p):
//  1. read the workgroup's ring pointer {start, n}; decide the flush (n >= L,
//     or n > 0 in flush mode);
//  2. load the committed records (keys, this block's u rows, g) and the call's
//     tokens (q, k, this block's v rows, g, beta), issue the tile's loads behind
//     them, and stage the records and tokens in LDS (keys widened to fp32); the
//     first block of the key head's first value head appends the tokens' keys
//     to the key ring;
//  3. flush: fold the records into the tile registers (rank-n update), store
//     the tile once, move the pointer past the folded records;
//  4. one 8-lane group per (query, window position) pair forms the segment
//     decay and the key-key and key-query scores;
//  5. per query, in order, each thread forms its rows' share of S_s k_q and
//     S_s q_q from the registers, scaled by the query's checkpoint decay, adds
//     the committed records' terms (records split over the row's lanes); the
//     row's lanes reduce and each adds the earlier drafts' terms and forms
//     u_q, then o_q; one lane per row writes o and appends u;
//  6. write the ring pointer (decode commits its token).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace rssm {

namespace {

template <int DK>
struct GdnGeo;
template <>
struct GdnGeo<16> { static constexpr int ROWS = 16, NT = 64; };
template <>
struct GdnGeo<128> { static constexpr int ROWS = 64, NT = 256; };

// LDS plan in floats.  Committed records use window positions 0 .. n-1; the
// call's tokens (queries) sit at n .. n+T-1 after any flush.
struct GdnLds {
    int K, KQ, QQ, U, US, V, G, GQ, BE, CK, CQ, DD, WF, UD, total;
};

// kbytes: bytes per element of the committed records' keys in LDS (they stay
// in the input type: 2 for bf16, 4 for fp32).
__host__ __device__ inline GdnLds gdn_plan(int DK, int ROWS, int cap, int T, int kbytes = 4) {
    GdnLds l;
    int o = 0;
    l.US = ROWS + 4;                // u row stride: lanes reading different records hit different banks
    l.K = o;  o += (cap * DK * kbytes + 15) / 16 * 4;   // committed records' keys, input type
    l.KQ = o; o += T * DK;          // tokens' keys
    l.QQ = o; o += T * DK;          // tokens' queries
    l.U = o;  o += cap * l.US;      // committed records' u, this block's rows
    l.V = o;  o += T * ROWS;        // tokens' v, this block's rows
    l.G = o;  o += cap;             // committed records' g
    l.GQ = o; o += T;               // tokens' g
    l.BE = o; o += T;               // tokens' beta
    l.CK = o; o += T * cap;         // ck[q][c] = exp(sum_{c<i<=m_q} g_i) (key_c . k_q), c < m_q
    l.CQ = o; o += T * cap;         // cq[q][c] = exp(sum_{c<i<=m_q} g_i) (key_c . q_q), c <= m_q
    l.DD = o; o += T + 1;           // dd[q] = exp(sum_{i<=m_q} g_i); [T]: the flush's checkpoint decay
    l.WF = o; o += cap;             // flush weights exp(sum_{c<i<n} g_i)
    l.UD = o; o += T * ROWS;        // the tokens' u
    l.total = (o + 3) & ~3;
    return l;
}

// A workgroup's place: wg = (b nv + h) span + part, span parts per (sequence,
// value head), and the head's key head kh = h / (nv / nk); by shifts where
// span, nv and nv / nk are powers of two (the host passes their logarithms,
// span_log2 < 0 where it is not), else by divisions.
struct GdnIdx {
    int part, bh, b, h, kh;
    bool key_writer;   // the first value head of its key head
};
__device__ __forceinline__ GdnIdx gdn_index(const GdnArgs& a, int wg, int span, int span_log2) {
    GdnIdx x;
    if (span_log2 >= 0 && a.nv_log2 >= 0 && a.hpk_log2 >= 0) {
        x.part = wg & (span - 1);
        x.bh = wg >> span_log2;
        x.b = x.bh >> a.nv_log2;
        x.h = x.bh & ((1 << a.nv_log2) - 1);
        x.kh = x.h >> a.hpk_log2;
        x.key_writer = (x.h & ((1 << a.hpk_log2) - 1)) == 0;
    } else {
        const int hpk = a.nv / a.nk;
        x.part = wg % span;
        x.bh = wg / span;
        x.b = x.bh / a.nv;
        x.h = x.bh - x.b * a.nv;
        x.kh = x.h / hpk;
        x.key_writer = x.h == x.kh * hpk;
    }
    return x;
}

// One input-type element (fp32, or bf16 bits) as fp32.
__device__ __forceinline__ float in_to_f32(float v) { return v; }
__device__ __forceinline__ float in_to_f32(uint16_t v) { return bf16_to_f32(v); }

// Four consecutive key elements starting at element e of an LDS array held in
// the input type, as fp32.
template <typename InT>
__device__ __forceinline__ float4 key4(const float* base, int e) {
    if constexpr (sizeof(InT) == 4) {
        return *reinterpret_cast<const float4*>(base + e);
    } else {
        const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + e);
        return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                           __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u));
    }
}

__device__ __forceinline__ float dot4(const v4f a, const float4 b) {
    float s = a[0] * b.x;
    s = fmaf(a[1], b.y, s);
    s = fmaf(a[2], b.z, s);
    return fmaf(a[3], b.w, s);
}

// Step 2 of a call, shared by the replay kernels: the staging list of a
// workgroup that serves ROWS value rows starting at row r0 of head h.  Vector
// i of the list is a 16-byte vector of a committed record's key, of the
// records' u rows, of a token's key or query, or of the tokens' v rows; `job`
// names its source, its LDS destination, whether it is widened from InT (else
// copied as fp32) and where a token key is appended to the key ring (or null).
// `issue` loads the first JOBS vectors of each thread into registers, so the
// kernel can issue the tile's loads behind them; `finish` stores them (and
// loads and stores the rest of a long window).  The log decays g (records) and
// g, beta (tokens) are scalars: `load_g` / `store_g`.
// KEYS_F32: the committed records' keys are widened to fp32 in LDS (else kept
// in the input type).
template <int DK, int ROWS, int NT, typename InT, bool KEYS_F32 = false>
struct GdnStage {
    static constexpr int EPV = InTraits<InT>::EPV;   // input elements per 16-byte vector
    static constexpr int KV = DK / EPV;              // vectors per key / query
    static constexpr int RV = ROWS / EPV;            // vectors per block of v rows
    static constexpr int UV = ROWS / 4;              // fp32 vectors per block of u rows
    static constexpr int JOBS = 2;

    const GdnArgs& a;
    float* smem;
    const GdnLds& Ls;
    const InT* kring;        // this key head's key ring
    const float* uring;      // this head's u ring, at row r0
    int b, h, kh, bh, r0, cap, T, start, n, np, qstart;
    bool append_k;
    int nkv, nuv, ntk, total;

    __device__ GdnStage(const GdnArgs& a_, float* smem_, const GdnLds& Ls_, int b_, int h_, int kh_, int r0_,
                        int T_, int start_, int n_, int np_, int qstart_, bool append_k_)
        : a(a_), smem(smem_), Ls(Ls_), b(b_), h(h_), kh(kh_), bh(b_ * a_.nv + h_), r0(r0_), cap(a_.cap), T(T_),
          start(start_), n(n_), np(np_), qstart(qstart_), append_k(append_k_) {
        kring = static_cast<const InT*>(a.buf_k) + (size_t)(b * a.nk + kh) * cap * DK;
        uring = a.buf_u + (size_t)bh * cap * a.dv + r0;
        nkv = n * KV;
        nuv = n * UV;
        ntk = T * KV;
        total = nkv + nuv + 2 * ntk + T * RV;
    }

    __device__ __forceinline__ int slot_of(int c) const {   // (start + c) mod cap, c < cap
        const int s = start + c;
        return s >= cap ? s - cap : s;
    }

    __device__ __forceinline__ void job(int i, const uint4*& src, float*& dst, bool& widen, uint4*& app) const {
        app = nullptr;
        widen = true;
        if (i < nkv) {
            const int c = i / KV, e = i - c * KV;
            src = reinterpret_cast<const uint4*>(kring + (size_t)slot_of(c) * DK) + e;
            if constexpr (KEYS_F32) {
                dst = smem + Ls.K + c * DK + e * EPV;
            } else {
                dst = reinterpret_cast<float*>(reinterpret_cast<InT*>(smem + Ls.K) + c * DK + e * EPV);
                widen = false;                           // kept in the input type
            }
            return;
        }
        i -= nkv;
        if (i < nuv) {
            const int c = i / UV, e = i - c * UV;
            src = reinterpret_cast<const uint4*>(uring + (size_t)slot_of(c) * a.dv) + e;
            dst = smem + Ls.U + c * Ls.US + 4 * e;
            widen = false;
            return;
        }
        i -= nuv;
        if (i < 2 * ntk) {
            const bool isq = i >= ntk;
            const int r = isq ? i - ntk : i;
            const int q = r / KV, e = r - q * KV;
            src = reinterpret_cast<const uint4*>(static_cast<const InT*>(isq ? a.q : a.k) +
                                                 ((size_t)(b * T + q) * a.nk + kh) * DK) + e;
            dst = smem + (isq ? Ls.QQ : Ls.KQ) + q * DK + e * EPV;
            if (!isq && append_k) {
                int slot = qstart + np + q;
                slot -= slot >= cap ? cap : 0;
                app = reinterpret_cast<uint4*>(static_cast<InT*>(a.buf_k) +
                                               ((size_t)(b * a.nk + kh) * cap + slot) * DK) + e;
            }
            return;
        }
        i -= 2 * ntk;
        const int q = i / RV, e = i - q * RV;
        src = reinterpret_cast<const uint4*>(static_cast<const InT*>(a.v) +
                                             ((size_t)(b * T + q) * a.nv + h) * a.dv + r0) + e;
        dst = smem + Ls.V + q * ROWS + e * EPV;
    }

    __device__ __forceinline__ static void put(float* dst, bool widen, uint4* app, const uint4 v) {
        if (app) *app = v;
        if (widen) {
            widen16<InT>(v, dst);
        } else {
            *reinterpret_cast<uint4*>(dst) = v;
        }
    }

    __device__ __forceinline__ void issue(uint4 (&jv)[JOBS], int tid) const {
#pragma unroll
        for (int j = 0; j < JOBS; ++j) {
            const int i = tid + j * NT;
            if (i < total) {
                const uint4* src;
                float* dst;
                bool widen;
                uint4* app;
                job(i, src, dst, widen, app);
                jv[j] = *src;
            }
        }
    }

    __device__ __forceinline__ void finish(const uint4 (&jv)[JOBS], int tid) const {
#pragma unroll
        for (int j = 0; j < JOBS; ++j) {
            const int i = tid + j * NT;
            if (i < total) {
                const uint4* src;
                float* dst;
                bool widen;
                uint4* app;
                job(i, src, dst, widen, app);
                put(dst, widen, app, jv[j]);
            }
        }
        for (int i = tid + JOBS * NT; i < total; i += NT) {   // windows longer than JOBS vectors a thread
            const uint4* src;
            float* dst;
            bool widen;
            uint4* app;
            job(i, src, dst, widen, app);
            put(dst, widen, app, *src);
        }
    }

    __device__ __forceinline__ void load_g(int tid, float& gv, float& gq, float& bq) const {
        gv = gq = bq = 0.0f;
        if (tid < n) gv = a.buf_g[(size_t)bh * cap + slot_of(tid)];
        if (tid < T) {
            const size_t ti = (size_t)(b * T + tid) * a.nv + h;
            gq = a.g[ti];
            bq = a.beta[ti];
        }
    }

    __device__ __forceinline__ void store_g(int tid, float gv, float gq, float bq) const {
        if (tid < n) smem[Ls.G + tid] = gv;
        for (int i = tid + NT; i < n; i += NT) smem[Ls.G + i] = a.buf_g[(size_t)bh * cap + slot_of(i)];
        if (tid < T) {
            smem[Ls.GQ + tid] = gq;
            smem[Ls.BE + tid] = bq;
        }
    }
};

// Step 4 of a call: one 8-lane group per (query q, window position c <= m_q =
// np + q) forms the segment decay exp(sum_{c<i<=m_q} g_i) and the key-key and
// key-query scores (k_c . k_q, k_c . q_q), which give ck[q][c] (c < m_q) and
// cq[q][c]; then dd[q] = exp(sum_{i<=m_q} g_i).  Window positions below np are
// committed records (K, G), the others the call's tokens (KQ, GQ).
template <int DK, int NT, typename InT>
__device__ __forceinline__ void gdn_coefficients(float* smem, const GdnLds& Ls, int np, int T, int cap, int tid) {
    const int m = np + T;                             // window positions of the call
    const int grp = tid / 8, gl = tid % 8;
    for (int idx = grp; idx < T * m; idx += NT / 8) {
        const int q = idx / m, c = idx % m;
        const int mq = np + q;
        if (c > mq) continue;                         // the whole group skips together
        const float* kq = smem + Ls.KQ + q * DK;
        const float* qq = smem + Ls.QQ + q * DK;
        float sk = 0.0f, sq = 0.0f, seg = 0.0f;
        // lane gl takes the 4-element chunks gl, gl + 8, ... (16-byte reads; the
        // group's lanes read consecutive chunks; not unrolled, so that only one
        // chunk's values are live beside the tile's registers)
#pragma unroll 1
        for (int j4 = gl; j4 < DK / 4; j4 += 8) {
            const float4 kv = c < np ? key4<InT>(smem + Ls.K, c * DK + 4 * j4)   // committed key, input type
                                     : *reinterpret_cast<const float4*>(smem + Ls.KQ + (c - np) * DK + 4 * j4);
            const float4 a = *reinterpret_cast<const float4*>(kq + 4 * j4);
            const float4 bq = *reinterpret_cast<const float4*>(qq + 4 * j4);
            sk = fmaf(kv.x, a.x, sk);
            sk = fmaf(kv.y, a.y, sk);
            sk = fmaf(kv.z, a.z, sk);
            sk = fmaf(kv.w, a.w, sk);
            sq = fmaf(kv.x, bq.x, sq);
            sq = fmaf(kv.y, bq.y, sq);
            sq = fmaf(kv.z, bq.z, sq);
            sq = fmaf(kv.w, bq.w, sq);
        }
        for (int i = c + 1 + gl; i <= mq; i += 8) seg += i < np ? smem[Ls.G + i] : smem[Ls.GQ + i - np];
        sk = group_sum<8>(sk);
        sq = group_sum<8>(sq);
        seg = group_sum<8>(seg);
        if (gl == 0) {
            const float w = __expf(seg);
            smem[Ls.CK + q * cap + c] = c < mq ? w * sk : 0.0f;
            smem[Ls.CQ + q * cap + c] = w * sq;
        }
    }
    for (int q = tid; q < T; q += NT) {
        float s = 0.0f;
        for (int i = 0; i <= np + q; ++i) s += i < np ? smem[Ls.G + i] : smem[Ls.GQ + i - np];
        smem[Ls.DD + q] = __expf(s);
    }
}

// F16: the checkpoint is fp16 (widened to fp32 registers after the loads, and
// written with stochastic rounding by a flush).
template <int DK, typename InT, bool F16>
__global__ __launch_bounds__(GdnGeo<DK>::NT, 7) void gdn_replay_kernel(const GdnArgs a) {
    constexpr int ROWS = GdnGeo<DK>::ROWS;
    constexpr int NT = GdnGeo<DK>::NT;
    using Geo = TileGeo<ROWS, DK, NT, 4>;
    constexpr int W = Geo::W;
    extern __shared__ float smem[];

    const int tid = threadIdx.x;
    const int wg = xcd_remap(blockIdx.x, gridDim.x);   // = (b * nv + h) * parts + p
    const GdnIdx ix = gdn_index(a, wg, a.parts, a.parts_log2);
    const int p = ix.part, bh = ix.bh, b = ix.b, h = ix.h, kh = ix.kh;
    const int cap = a.cap;
    const int T = a.mode == MODE_FLUSH ? 0 : a.T;
    const GdnLds Ls = gdn_plan(DK, ROWS, cap, T, sizeof(InT));

    // 1. ring pointer (every thread reads the workgroup's copy, checked against
    // the sequence's first copy), the fused commit of the previous verification
    // if any (len += accepted_prev[b]), and the flush decision
    const RingPtr own = load_ring_ptr(a.meta, wg);
    const size_t ref_copy = (size_t)b * a.nv * a.parts;
    const RingPtr ref = load_ring_ptr(a.meta, ref_copy);
    const int acc_prev = a.accepted_prev ? a.accepted_prev[b] : 0;
    // the loads in flight together (the reference is needed only after the
    // flush decision; issued after it the latencies would add up)
    asm volatile("" ::"s"(own.start), "s"(own.n), "s"(ref.start), "s"(ref.n), "s"(acc_prev));
    const int start = own.start;
    const int n_stored = own.n;
    const bool acc_ok = !a.accepted_prev ||
                        (acc_prev >= 0 && acc_prev <= a.T_prev && n_stored >= 0 && n_stored + acc_prev <= cap);
    const int n = n_stored + acc_prev;
    const bool fold = a.mode == MODE_FLUSH ? n > 0 : n >= a.L;
    const int np = fold ? 0 : n;                          // committed records seen by the queries
    // the pointer this call leaves (the drafts of a folding call go to the T
    // slots after the n folded ones, so n + T must fit the ring whether or not
    // the call folds)
    const int wrapped = start + n >= cap ? start + n - cap : start + n;   // start + n < 2 cap when valid
    const RingPtr after{fold ? wrapped : start, np + (a.mode == MODE_DECODE ? T : 0)};
    const bool agree = (size_t)wg == ref_copy || ring_ptr_agrees(ref, own, after);
    const bool valid = acc_ok && agree && start >= 0 && start < cap && n >= 0 && n + T <= cap;
    if (!valid) {
        if (tid == 0 && a.status) atomicOr(a.status, (int)(acc_ok ? kStatusMeta : kStatusAccept));
        for (int i = tid; i < T * ROWS; i += NT)
            a.o[((size_t)(b * T + i / ROWS) * a.nv + h) * a.dv + p * ROWS + i % ROWS] = __builtin_nanf("");
        return;
    }
    if (!fold && T == 0) return;                          // flush call with nothing to fold
    int qstart = start + n;                               // ring start after the flush
    qstart -= qstart >= cap ? cap : 0;
    if (!fold) qstart = start;

    // 2. staging: the records' and tokens' 16-byte vectors are loaded into
    // registers first, the tile's loads are issued behind them, and the staged
    // vectors are stored to LDS while the tile is still in flight (loads
    // complete in order, so waiting for a staged vector never waits for the tile).
    const GdnStage<DK, ROWS, NT, InT> stage(a, smem, Ls, b, h, kh, p * ROWS, T, start, n, np, qstart,
                                            ix.key_writer && p == 0);
    uint4 jv[stage.JOBS];
    stage.issue(jv, tid);
    float gv, gq, bq;
    stage.load_g(tid, gv, gq, bq);

    const size_t tile_off = ((size_t)bh * a.dv + p * ROWS) * DK;   // first element of the tile
    float* const tile_p = a.ckpt + tile_off;
    uint16_t* const tile16 = reinterpret_cast<uint16_t*>(a.ckpt) + tile_off;
    v4f raw[Geo::NV];
    v2u raw16[F16 ? Geo::NV : 1];
    if constexpr (F16) {
#pragma unroll
        for (int s = 0; s < Geo::NV; ++s)
            raw16[s] = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(tile16) + Geo::vec(tid, s));
    } else {
#pragma unroll
        for (int s = 0; s < Geo::NV; ++s)
            raw[s] = __builtin_bit_cast(v4f, __builtin_nontemporal_load(reinterpret_cast<const v4u*>(tile_p) +
                                                                        Geo::vec(tid, s)));
    }

    stage.finish(jv, tid);
    stage.store_g(tid, gv, gq, bq);
    __syncthreads();
    if constexpr (F16) {
#pragma unroll
        for (int s = 0; s < Geo::NV; ++s) {
            const uint32_t w0 = raw16[s][0], w1 = raw16[s][1];
            raw[s] = v4f{f16lo_to_f32(w0), f16hi_to_f32(w0), f16lo_to_f32(w1), f16hi_to_f32(w1)};
        }
    }

    const int row0 = Geo::row0(tid);
    const int lane = tid % W;

    // 3. flush: S <- exp(sum g) S + sum_c exp(sum_{c<i<n} g_i) u_c k_c^T, stored once
    if (fold) {
        for (int c = tid; c < n; c += NT) {
            float sg = 0.0f;
            for (int i = c + 1; i < n; ++i) sg += smem[Ls.G + i];
            smem[Ls.WF + c] = __expf(sg);
        }
        if (tid == NT - 1) {
            float sg = 0.0f;
            for (int i = 0; i < n; ++i) sg += smem[Ls.G + i];
            smem[Ls.DD + T] = __expf(sg);
        }
        __syncthreads();
        const float gf = smem[Ls.DD + T];
#pragma unroll
        for (int s = 0; s < Geo::NV; ++s) raw[s] *= gf;
        for (int c = 0; c < n; ++c) {
            float cf[Geo::NI];
            const float wc = smem[Ls.WF + c];
#pragma unroll
            for (int r = 0; r < Geo::NI; ++r) cf[r] = wc * smem[Ls.U + c * Ls.US + row0 + r];
#pragma unroll
            for (int k = 0; k < Geo::VPL; ++k) {
                const float4 kc = key4<InT>(smem + Ls.K, c * DK + 4 * (lane + W * k));
#pragma unroll
                for (int r = 0; r < Geo::NI; ++r) {
                    v4f& x = raw[r * Geo::VPL + k];
                    x[0] = fmaf(cf[r], kc.x, x[0]);
                    x[1] = fmaf(cf[r], kc.y, x[1]);
                    x[2] = fmaf(cf[r], kc.z, x[2]);
                    x[3] = fmaf(cf[r], kc.w, x[3]);
                }
            }
        }
        if constexpr (F16) {
            // (tile_off / 4: vector index of the tile's first element)
            store_f16_sr<Geo>(reinterpret_cast<uint64_t*>(tile16), tile_off / 4, raw, a.sr_seed, tid);
        } else {
#pragma unroll
            for (int s = 0; s < Geo::NV; ++s)
                __builtin_nontemporal_store(__builtin_bit_cast(v4u, raw[s]),
                                            reinterpret_cast<v4u*>(tile_p) + Geo::vec(tid, s));
        }
        if (T == 0) {
            if (tid == 0) store_ring_ptr(a.meta, wg, after);
            return;
        }
    }

    // 4. coefficients: one 8-lane group per (query q, window position c <= np + q)
    gdn_coefficients<DK, NT, InT>(smem, Ls, np, T, cap, tid);
    __syncthreads();

    // 5. per query, in order: the rows' share of S_s k_q and S_s q_q from the
    // registers (scaled by the query's checkpoint decay) plus the committed
    // records' terms (records split over the row's lanes), reduced over the
    // row's lanes; then, on every lane of the row, the earlier drafts' terms,
    // u_q and o_q.  The drafts' u rows are kept in LDS (each lane reads back
    // what it wrote).
    float* const uring_w = a.buf_u + (size_t)bh * cap * a.dv + p * ROWS;
    for (int q = 0; q < T; ++q) {
        float pk[Geo::NI], pq[Geo::NI];
#pragma unroll
        for (int r = 0; r < Geo::NI; ++r) {
            pk[r] = 0.0f;
            pq[r] = 0.0f;
        }
#pragma unroll
        for (int k = 0; k < Geo::VPL; ++k) {
            const int vc = lane + W * k;
            const float4 k4 = *reinterpret_cast<const float4*>(smem + Ls.KQ + q * DK + 4 * vc);
            const float4 q4 = *reinterpret_cast<const float4*>(smem + Ls.QQ + q * DK + 4 * vc);
#pragma unroll
            for (int r = 0; r < Geo::NI; ++r) {
                pk[r] += dot4(raw[r * Geo::VPL + k], k4);
                pq[r] += dot4(raw[r * Geo::VPL + k], q4);
            }
        }
        const float d = smem[Ls.DD + q];
#pragma unroll
        for (int r = 0; r < Geo::NI; ++r) {
            pk[r] *= d;
            pq[r] *= d;
        }
        for (int c = lane; c < np; c += W) {
            const float ck = smem[Ls.CK + q * cap + c];
            const float cq = smem[Ls.CQ + q * cap + c];
#pragma unroll
            for (int r = 0; r < Geo::NI; ++r) {
                const float u = smem[Ls.U + c * Ls.US + row0 + r];
                pk[r] = fmaf(ck, u, pk[r]);
                pq[r] = fmaf(cq, u, pq[r]);
            }
        }
        int slot = qstart + np + q;
        slot -= slot >= cap ? cap : 0;
        const float bet = smem[Ls.BE + q];
        const float cself = smem[Ls.CQ + q * cap + np + q];
        // One transposed reduction of the 2 NI sums over the row's W lanes
        // (halving stages, as the Mamba-2 kernel reduces its rows): lane j of
        // the group ends with the full sum of value idx(j), where values
        // 0 .. NI-1 are S k of the thread's rows and NI .. 2 NI-1 their S q.
        // A lane holding S k of a row and the lane holding S q of the same row
        // differ in bit 0: the first forms u, passes it to the second, which
        // forms o.
        constexpr int NV2 = 2 * Geo::NI;
        static_assert(NV2 <= W, "transposed reduction needs 2 NI <= W");
        float red[16];
#pragma unroll
        for (int r = 0; r < Geo::NI; ++r) {
            red[r] = pk[r];
            red[Geo::NI + r] = pq[r];
        }
        int idx;
        float acc = transpose_reduce<NV2, W>(red, lane, idx);
        const bool is_k = idx < Geo::NI;
        const int row = row0 + (is_k ? idx : idx - Geo::NI);
        for (int dd = 0; dd < q; ++dd)
            acc = fmaf(smem[(is_k ? Ls.CK : Ls.CQ) + q * cap + np + dd], smem[Ls.UD + dd * ROWS + row], acc);
        const float u = bet * (smem[Ls.V + q * ROWS + row] - acc);     // meaningful where is_k
        const float u_row = xor_shfl<1>(u);                            // the S q lane gets its row's u
        const float o = fmaf(cself, u_row, acc);                       // meaningful where !is_k
        if ((lane & (W - 1)) < NV2) {                                  // lanes holding distinct values
            if (is_k) {
                if (q + 1 < T) smem[Ls.UD + q * ROWS + row] = u;
                uring_w[(size_t)slot * a.dv + row] = u;
            } else {
                a.o[((size_t)(b * T + q) * a.nv + h) * a.dv + p * ROWS + row] = o;
            }
        }
    }
    if (p == 0 && tid < T) {
        int slot = qstart + np + tid;
        slot -= slot >= cap ? cap : 0;
        a.buf_g[(size_t)bh * cap + slot] = smem[Ls.GQ + tid];
    }

    // 6. ring pointer: verify leaves the length, decode commits its token
    if (tid == 0) store_ring_ptr(a.meta, wg, after);
}

// FP16 checkpoint, one workgroup per 128 value rows (two 64-row blocks) of a
// head with dk = 128.  The fp16 tile of 128 rows is 32 KiB, the register
// footprint of one 64-row FP32 tile, so a workgroup streams as many bytes as
// the FP32 kernel's instead of half of them.  The tile stays packed in
// registers (TileGeo<128, 128, 256, 2>: 4 rows per thread, two 8-element
// vectors per row) and is widened where it is read.  The steps are those of
// gdn_replay_kernel with these differences: a flush folds one row at a time in
// fp32, writes it with stochastic rounding and forms that row's query products
// from the fp32 values; the products are reduced per row and staged in LDS,
// and one thread per row then walks the queries in order (u_q, o_q).
template <typename InT>
__global__ __launch_bounds__(256, 7) void gdn_replay_f16_wide_kernel(const GdnArgs a) {
    constexpr int DK = 128, ROWS = 128, NT = 256;
    using Geo = TileGeo<ROWS, DK, NT, 2>;
    static_assert(Geo::NI == 4 && Geo::VPL == 2 && Geo::W == 8 && Geo::NV == 8, "fp16 wide tile layout");
    constexpr int W = Geo::W;
    extern __shared__ float smem[];

    const int tid = threadIdx.x;
    const int wg = xcd_remap(blockIdx.x, gridDim.x);   // = (b * nv + h) * (parts / 2) + pw
    const int pairs = a.parts / 2;
    const GdnIdx ix = gdn_index(a, wg, pairs, a.parts_log2 >= 1 ? a.parts_log2 - 1 : -1);
    const int pw = ix.part, bh = ix.bh, b = ix.b, h = ix.h, kh = ix.kh;
    const int cap = a.cap;
    const int T = a.mode == MODE_FLUSH ? 0 : a.T;
    const GdnLds Ls = gdn_plan(DK, ROWS, cap, T, 4);   // keys widened to fp32: the row-by-row fold reads each one per row
    const int PK = Ls.total, PQ = Ls.total + T * ROWS;     // reduced products [q][row]
    const int m0 = bh * a.parts + 2 * pw;                  // the pointer copies of the two row blocks

    // 1. ring pointer (the copies of both row blocks are equal, and agree with
    // the sequence's first copy), the fused commit if any, and the flush decision
    const RingPtr own = load_ring_ptr(a.meta, m0);
    const size_t ref_copy = (size_t)b * a.nv * a.parts;
    const RingPtr ref = load_ring_ptr(a.meta, ref_copy);
    const int acc_prev = a.accepted_prev ? a.accepted_prev[b] : 0;
    // the loads in flight together (the reference is needed only after the
    // flush decision; issued after it the latencies would add up)
    asm volatile("" ::"s"(own.start), "s"(own.n), "s"(ref.start), "s"(ref.n), "s"(acc_prev));
    const int start = own.start;
    const int n_stored = own.n;
    const bool acc_ok = !a.accepted_prev ||
                        (acc_prev >= 0 && acc_prev <= a.T_prev && n_stored >= 0 && n_stored + acc_prev <= cap);
    const int n = n_stored + acc_prev;
    const bool fold = a.mode == MODE_FLUSH ? n > 0 : n >= a.L;
    const int np = fold ? 0 : n;
    const int wrapped = start + n >= cap ? start + n - cap : start + n;   // start + n < 2 cap when valid
    const RingPtr after{fold ? wrapped : start, np + (a.mode == MODE_DECODE ? T : 0)};
    const bool agree = load_ring_ptr(a.meta, m0 + 1) == own &&
                       ((size_t)m0 == ref_copy || ring_ptr_agrees(ref, own, after));
    const bool valid = acc_ok && agree && start >= 0 && start < cap && n >= 0 && n + T <= cap;
    if (!valid) {
        if (tid == 0 && a.status) atomicOr(a.status, (int)(acc_ok ? kStatusMeta : kStatusAccept));
        for (int i = tid; i < T * ROWS; i += NT)
            a.o[((size_t)(b * T + i / ROWS) * a.nv + h) * a.dv + pw * ROWS + i % ROWS] = __builtin_nanf("");
        return;
    }
    if (!fold && T == 0) return;
    // Two bodies, with and without the flush: the registers that the flush's
    // fold and rounding hold then do not shape the non-flush path's allocation.
    auto run = [&](auto fold_tag) {
        constexpr bool fold = decltype(fold_tag)::value;
        int qstart = start + n;
        qstart -= qstart >= cap ? cap : 0;
        if (!fold) qstart = start;

        // 2. staging (as in gdn_replay_kernel, for 128 rows)
        const GdnStage<DK, ROWS, NT, InT, true> stage(a, smem, Ls, b, h, kh, pw * ROWS, T, start, n, np, qstart,
                                                ix.key_writer && pw == 0);
        uint4 jv[stage.JOBS];
        stage.issue(jv, tid);
        float gv, gq, bq;
        stage.load_g(tid, gv, gq, bq);

        const size_t tile_off = ((size_t)bh * a.dv + pw * ROWS) * DK;
        uint16_t* const tile16 = reinterpret_cast<uint16_t*>(a.ckpt) + tile_off;
        v4u raw[Geo::NV];                                       // 8 fp16 values per vector
    #pragma unroll
        for (int s = 0; s < Geo::NV; ++s)
            raw[s] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(tile16) + Geo::vec(tid, s));

        stage.finish(jv, tid);
        stage.store_g(tid, gv, gq, bq);
        __syncthreads();

        const int row0 = Geo::row0(tid);
        const int lane = tid % W;
        // the 16 values of row r of this thread's share, widened: columns (lane + 8k) * 8 + e
        auto widen_row = [&](int r, float (&f)[16]) {
    #pragma unroll
            for (int k = 0; k < 2; ++k) {
                const v4u w = raw[r * Geo::VPL + k];
    #pragma unroll
                for (int e = 0; e < 4; ++e) {
                    f[8 * k + 2 * e] = f16lo_to_f32(w[e]);
                    f[8 * k + 2 * e + 1] = f16hi_to_f32(w[e]);
                }
            }
        };
        auto dot_row = [&](const float (&f)[16], const float* x) {
            float acc = 0.0f;
    #pragma unroll
            for (int k = 0; k < 2; ++k) {
                const float4 x0 = *reinterpret_cast<const float4*>(x + (lane + W * k) * 8);
                const float4 x1 = *reinterpret_cast<const float4*>(x + (lane + W * k) * 8 + 4);
                acc = fmaf(f[8 * k], x0.x, acc);
                acc = fmaf(f[8 * k + 1], x0.y, acc);
                acc = fmaf(f[8 * k + 2], x0.z, acc);
                acc = fmaf(f[8 * k + 3], x0.w, acc);
                acc = fmaf(f[8 * k + 4], x1.x, acc);
                acc = fmaf(f[8 * k + 5], x1.y, acc);
                acc = fmaf(f[8 * k + 6], x1.z, acc);
                acc = fmaf(f[8 * k + 7], x1.w, acc);
            }
            return acc;
        };

        if (fold) {
            // 3. flush weights, then per row: fold in fp32, write with stochastic rounding
            for (int c = tid; c < n; c += NT) {
                float sg = 0.0f;
                for (int i = c + 1; i < n; ++i) sg += smem[Ls.G + i];
                smem[Ls.WF + c] = __expf(sg);
            }
            if (tid == NT - 1) {
                float sg = 0.0f;
                for (int i = 0; i < n; ++i) sg += smem[Ls.G + i];
                smem[Ls.DD + T] = __expf(sg);
            }
        }
        // 4. coefficients
        gdn_coefficients<DK, NT, float>(smem, Ls, np, T, cap, tid);
        __syncthreads();

        // 5. per row of this thread: the query products (from the fp32 fold on a
        // flush call, else from the widened fp16 checkpoint) plus the committed
        // records' terms, reduced over the row's lanes and staged in LDS
        const float gf = fold ? smem[Ls.DD + T] : 1.0f;
    #pragma unroll
        for (int r = 0; r < Geo::NI; ++r) {
            const int row = row0 + r;
            float f[16];
            widen_row(r, f);
            if (fold) {
    #pragma unroll
                for (int e = 0; e < 16; ++e) f[e] *= gf;
                for (int c = 0; c < n; ++c) {
                    const float cf = smem[Ls.WF + c] * smem[Ls.U + c * Ls.US + row];
    #pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        const float4 k0 = key4<float>(smem + Ls.K, c * DK + (lane + W * k) * 8);
                        const float4 k1 = key4<float>(smem + Ls.K, c * DK + (lane + W * k) * 8 + 4);
                        f[8 * k] = fmaf(cf, k0.x, f[8 * k]);
                        f[8 * k + 1] = fmaf(cf, k0.y, f[8 * k + 1]);
                        f[8 * k + 2] = fmaf(cf, k0.z, f[8 * k + 2]);
                        f[8 * k + 3] = fmaf(cf, k0.w, f[8 * k + 3]);
                        f[8 * k + 4] = fmaf(cf, k1.x, f[8 * k + 4]);
                        f[8 * k + 5] = fmaf(cf, k1.y, f[8 * k + 5]);
                        f[8 * k + 6] = fmaf(cf, k1.z, f[8 * k + 6]);
                        f[8 * k + 7] = fmaf(cf, k1.w, f[8 * k + 7]);
                    }
                }
                // fp32 vectors v0, v0 + 1 (k = 0) and v0 + 16, v0 + 17 (k = 1): two
                // generator calls, each shared by a vector and the one 16 after it
                const uint64_t v0 = (tile_off + (size_t)row * DK + (size_t)lane * 8) / 4;
                uint2 a0, a1, b0, b1;
                f32x8_to_f16x8_sr(v4f{f[0], f[1], f[2], f[3]}, v4f{f[8], f[9], f[10], f[11]}, v0, a.sr_seed, a0, a1);
                __builtin_amdgcn_sched_barrier(0);   // one call's random words live at a time
                f32x8_to_f16x8_sr(v4f{f[4], f[5], f[6], f[7]}, v4f{f[12], f[13], f[14], f[15]}, v0 + 1, a.sr_seed, b0,
                                  b1);
                __builtin_nontemporal_store(v4u{a0.x, a0.y, b0.x, b0.y},
                                            reinterpret_cast<v4u*>(tile16) + Geo::vec(tid, r * Geo::VPL));
                __builtin_nontemporal_store(v4u{a1.x, a1.y, b1.x, b1.y},
                                            reinterpret_cast<v4u*>(tile16) + Geo::vec(tid, r * Geo::VPL + 1));
            }
            for (int q = 0; q < T; ++q) {
                const float d = smem[Ls.DD + q];
                float pk = d * dot_row(f, smem + Ls.KQ + q * DK);
                float pq = d * dot_row(f, smem + Ls.QQ + q * DK);
                for (int c = lane; c < np; c += W) {
                    const float u = smem[Ls.U + c * Ls.US + row];
                    pk = fmaf(smem[Ls.CK + q * cap + c], u, pk);
                    pq = fmaf(smem[Ls.CQ + q * cap + c], u, pq);
                }
                pk = group_sum<W>(pk);
                pq = group_sum<W>(pq);
                if (lane == 0) {
                    smem[PK + q * ROWS + row] = pk;
                    smem[PQ + q * ROWS + row] = pq;
                }
            }
        }
        if (T == 0) {
            if (tid < 2) store_ring_ptr(a.meta, m0 + tid, after);
            return;
        }
        __syncthreads();

        // 6. one thread per row walks the queries in order: u_q, then o_q
        if (tid < ROWS) {
            const int row = tid;
            float* const uring_w = a.buf_u + (size_t)bh * cap * a.dv + pw * ROWS + row;
            for (int q = 0; q < T; ++q) {
                float sk = smem[PK + q * ROWS + row];
                float o = smem[PQ + q * ROWS + row];
                for (int dd = 0; dd < q; ++dd) {
                    const float ud = smem[Ls.UD + dd * ROWS + row];
                    sk = fmaf(smem[Ls.CK + q * cap + np + dd], ud, sk);
                    o = fmaf(smem[Ls.CQ + q * cap + np + dd], ud, o);
                }
                const float u = smem[Ls.BE + q] * (smem[Ls.V + q * ROWS + row] - sk);
                o = fmaf(smem[Ls.CQ + q * cap + np + q], u, o);
                smem[Ls.UD + q * ROWS + row] = u;
                a.o[((size_t)(b * T + q) * a.nv + h) * a.dv + pw * ROWS + row] = o;
                int slot = qstart + np + q;
                slot -= slot >= cap ? cap : 0;
                uring_w[(size_t)slot * a.dv] = u;
            }
        }
        if (pw == 0 && tid >= ROWS && tid < ROWS + T) {
            const int q = tid - ROWS;
            int slot = qstart + np + q;
            slot -= slot >= cap ? cap : 0;
            a.buf_g[(size_t)bh * cap + slot] = smem[Ls.GQ + q];
        }
        // 7. ring pointers of both row blocks
        if (tid < 2) store_ring_ptr(a.meta, m0 + tid, after);
    };
    if (fold)
        run(std::true_type{});
    else
        run(std::false_type{});
}

// Conventional GDN step (the in-library baseline): read the tile, then per
// token S k, u = beta (v - alpha S k), S <- alpha S + u k^T, o = S q, store.
// With nslots > 1 (speculative verification with one snapshot per draft, blog
// section "Rollback for speculative decoding") the current slot is read once
// and draft q's state is written to slot (slot + 1 + q) % nslots.
template <int DK, typename InT>
__global__ __launch_bounds__(GdnGeo<DK>::NT, 8) void gdn_conventional_kernel(const GdnArgs a) {
    constexpr int ROWS = GdnGeo<DK>::ROWS;
    constexpr int NT = GdnGeo<DK>::NT;
    using Geo = TileGeo<ROWS, DK, NT, 4>;
    constexpr int W = Geo::W;
    constexpr int EPV = InTraits<InT>::EPV;
    constexpr int KV = DK / EPV;
    constexpr int RV = ROWS / EPV;
    extern __shared__ float smem[];
    const int T = a.T;
    float* const kk = smem;                     // [T][DK]
    float* const qq = smem + T * DK;            // [T][DK]
    float* const vv = smem + 2 * T * DK;        // [T][ROWS]
    float* const gb = vv + T * ROWS;            // [T][2]: g, beta

    const int tid = threadIdx.x;
    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    const GdnIdx ix = gdn_index(a, wg, a.parts, a.parts_log2);
    const int p = ix.part, bh = ix.bh, b = ix.b, h = ix.h, kh = ix.kh;
    const int nslots = a.nslots;
    const int s0 = nslots > 1 ? a.slot[b] : 0;
    if (s0 < 0 || s0 >= nslots) {
        if (tid == 0 && h == 0 && p == 0 && a.status) atomicOr(a.status, (int)kStatusSlot);
        for (int i = tid; i < T * ROWS; i += NT)
            a.o[((size_t)(b * T + i / ROWS) * a.nv + h) * a.dv + p * ROWS + i % ROWS] = __builtin_nanf("");
        return;
    }
    const size_t per_slot = (size_t)a.nv * a.dv * DK;
    float* const seq = a.ckpt + (size_t)b * nslots * per_slot + ((size_t)h * a.dv + p * ROWS) * DK;

    v4f raw[Geo::NV];
    {
        const v4u* src = reinterpret_cast<const v4u*>(seq + s0 * per_slot);
#pragma unroll
        for (int s = 0; s < Geo::NV; ++s)
            raw[s] = __builtin_bit_cast(v4f, __builtin_nontemporal_load(src + Geo::vec(tid, s)));
    }
    for (int i = tid; i < T * (2 * KV + RV); i += NT) {
        const int q = i / (2 * KV + RV);
        const int r = i - q * (2 * KV + RV);
        if (r < 2 * KV) {
            const bool isq = r >= KV;
            const int e = isq ? r - KV : r;
            const InT* src = static_cast<const InT*>(isq ? a.q : a.k) + ((size_t)(b * T + q) * a.nk + kh) * DK;
            widen16<InT>(reinterpret_cast<const uint4*>(src)[e], (isq ? qq : kk) + q * DK + e * EPV);
        } else {
            const int e = r - 2 * KV;
            const InT* src = static_cast<const InT*>(a.v) + ((size_t)(b * T + q) * a.nv + h) * a.dv + p * ROWS;
            widen16<InT>(reinterpret_cast<const uint4*>(src)[e], vv + q * ROWS + e * EPV);
        }
    }
    if (tid < T) {
        const size_t ti = (size_t)(b * T + tid) * a.nv + h;
        gb[2 * tid] = a.g[ti];
        gb[2 * tid + 1] = a.beta[ti];
    }
    __syncthreads();
    const int row0 = Geo::row0(tid);
    const int lane = tid % W;

    for (int q = 0; q < T; ++q) {
        const float alpha = __expf(gb[2 * q]);
        const float beta = gb[2 * q + 1];
        const float* kq = kk + q * DK;
        const float* qv = qq + q * DK;
        float sk[Geo::NI];
#pragma unroll
        for (int r = 0; r < Geo::NI; ++r) sk[r] = 0.0f;
#pragma unroll
        for (int s = 0; s < Geo::NV; ++s) {
            const int vc = lane + W * (s % Geo::VPL);
            sk[s / Geo::VPL] += dot4(raw[s], *reinterpret_cast<const float4*>(kq + 4 * vc));
        }
        float u[Geo::NI];
#pragma unroll
        for (int r = 0; r < Geo::NI; ++r) u[r] = beta * (vv[q * ROWS + row0 + r] - alpha * group_sum<W>(sk[r]));
        float o[Geo::NI];
#pragma unroll
        for (int r = 0; r < Geo::NI; ++r) o[r] = 0.0f;
#pragma unroll
        for (int s = 0; s < Geo::NV; ++s) {
            const int r = s / Geo::VPL;
            const int vc = lane + W * (s % Geo::VPL);
            const float4 k4 = *reinterpret_cast<const float4*>(kq + 4 * vc);
            v4f x = raw[s];
            x[0] = fmaf(alpha, x[0], u[r] * k4.x);
            x[1] = fmaf(alpha, x[1], u[r] * k4.y);
            x[2] = fmaf(alpha, x[2], u[r] * k4.z);
            x[3] = fmaf(alpha, x[3], u[r] * k4.w);
            raw[s] = x;
            o[r] += dot4(x, *reinterpret_cast<const float4*>(qv + 4 * vc));
        }
        int dst = s0;
        if (nslots > 1) {
            dst = s0 + 1 + q;
            dst -= dst >= nslots ? nslots : 0;
        }
        v4u* const out = reinterpret_cast<v4u*>(seq + dst * per_slot);
#pragma unroll
        for (int s = 0; s < Geo::NV; ++s)
            __builtin_nontemporal_store(__builtin_bit_cast(v4u, raw[s]), out + Geo::vec(tid, s));
#pragma unroll
        for (int r = 0; r < Geo::NI; ++r) o[r] = group_sum<W>(o[r]);
        if (lane == 0) {
#pragma unroll
            for (int r = 0; r < Geo::NI; ++r)
                a.o[((size_t)(b * T + q) * a.nv + h) * a.dv + p * ROWS + row0 + r] = o[r];
        }
    }
}

template <int DK, typename InT>
hipError_t launch_replay_t(const GdnArgs& a, hipStream_t stream) {
    constexpr int ROWS = GdnGeo<DK>::ROWS, NT = GdnGeo<DK>::NT;
    const int T = a.mode == MODE_FLUSH ? 0 : a.T;
    const size_t lds = (size_t)gdn_plan(DK, ROWS, a.cap, T, sizeof(InT)).total * 4;
    const int nwg = a.batch * a.nv * a.parts;
    if constexpr (DK == 128) {
        const size_t lds2 = ((size_t)gdn_plan(DK, 128, a.cap, T, 4).total + 2 * (size_t)T * 128) * 4;
        if (a.ckpt16 && a.parts % 2 == 0 && lds2 <= 64 * 1024) {   // 128 rows per workgroup
            hipLaunchKernelGGL((gdn_replay_f16_wide_kernel<InT>), dim3(nwg / 2), dim3(256), lds2, stream, a);
            return hipGetLastError();
        }
    }
    if (a.ckpt16)
        hipLaunchKernelGGL((gdn_replay_kernel<DK, InT, true>), dim3(nwg), dim3(NT), lds, stream, a);
    else
        hipLaunchKernelGGL((gdn_replay_kernel<DK, InT, false>), dim3(nwg), dim3(NT), lds, stream, a);
    return hipGetLastError();
}

template <int DK, typename InT>
hipError_t launch_conv_t(const GdnArgs& a, hipStream_t stream) {
    constexpr int ROWS = GdnGeo<DK>::ROWS, NT = GdnGeo<DK>::NT;
    const size_t lds = (size_t)a.T * (2 * DK + ROWS + 2) * 4;
    const int nwg = a.batch * a.nv * a.parts;
    hipLaunchKernelGGL((gdn_conventional_kernel<DK, InT>), dim3(nwg), dim3(NT), lds, stream, a);
    return hipGetLastError();
}

}  // namespace

bool gdn_shape_supported(int dk, int dv) {
    return (dk == 16 && dv > 0 && dv % 16 == 0) || (dk == 128 && dv > 0 && dv % 64 == 0);
}

int gdn_rows(int dk) { return dk == 16 ? GdnGeo<16>::ROWS : GdnGeo<128>::ROWS; }

// LDS of the 64-row (or 16-row) replay kernel with fp32 keys: an upper bound
// for every replay kernel the library picks for these sizes (bf16 keys take
// less; the 128-row FP16 kernel is used only where its plan fits 64 KiB).
size_t gdn_lds_bytes(int dk, int cap, int T) {
    return (size_t)gdn_plan(dk, gdn_rows(dk), cap, T).total * 4;
}

hipError_t launch_gdn_replay(const GdnArgs& a, int dk, int in_type, hipStream_t stream) {
    if (dk == 16) return in_type == IN_BF16 ? launch_replay_t<16, uint16_t>(a, stream) : launch_replay_t<16, float>(a, stream);
    return in_type == IN_BF16 ? launch_replay_t<128, uint16_t>(a, stream) : launch_replay_t<128, float>(a, stream);
}

hipError_t launch_gdn_conventional(const GdnArgs& a, int dk, int in_type, hipStream_t stream) {
    if (dk == 16) return in_type == IN_BF16 ? launch_conv_t<16, uint16_t>(a, stream) : launch_conv_t<16, float>(a, stream);
    return in_type == IN_BF16 ? launch_conv_t<128, uint16_t>(a, stream) : launch_conv_t<128, float>(a, stream);
}

}  // namespace rssm
