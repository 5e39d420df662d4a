// ReplaySSM decode / verify / flush kernel for one Mamba-2 layer (gfx950).
//
// Method: NVIDIA Developer blog "ReplaySSM: Rethinking State Storage for
// Faster Hybrid-Model Decoding".  The state of (sequence b, head h) is an FP32
// checkpoint tile H_s (HD x DS) plus the records (x_k, B_k, dt_k) appended
// since the last flush (section "How ReplaySSM represents the state").
//
// One workgroup per (b, h) tile.  Per call:
//   1. read {start, n} of sequence b; the call flushes first when n >= L
//      (decode/verify) or n > 0 (flush), and issues the 16-byte loads of the
//      tile it needs (FP32 checkpoint, or the low-precision read copy on a
//      non-flush call) right away, behind the small record loads, so the tile
//      streams in while the rest of the setup runs;
//   2. stage the n records and the T query tokens in LDS as fp32 and append
//      the queries' records to the ring (x and dt by every head, B by the
//      first head of the group);
//   3. per (query, record) pair, one 8-lane group forms the coefficient
//      co[q][c] = dt_c exp(sum_{c<i<=m_q} a_i) (B_c . C_q) (+ D_h when c is
//      the query's own record), splitting both the segment sum (never ratios
//      of exponentials) and the score over its lanes; the same groups form
//      the flush weights dt_c exp(sum_{c<i<n} a_i);
//   4. flush: H = exp(sum a) H_s + sum_k dt_k exp(sum_{k<i<n} a_i) x_k B_k^T,
//      the rank-n update applied to the tile in registers, written once, with
//      the read copy cast from the same registers (section "Benefit 3": the
//      copy is never read back into the recurrence);
//   5. per query, every thread forms its share of d_q (H C_q)[i] plus its
//      share of sum_c co[q][c] x_c[i] for each of its rows (section "Benefit
//      2": the checkpoint is read once for all queries; output-only
//      evaluation: no intermediate state is formed), and one reduction over
//      the W lanes of each row gives y_q[i];
//   6. write the head's new ring pointer.  Every head keeps its own copy of
//      {start, n} (all copies of a sequence are equal), read and written only
//      by the workgroup that owns the head, so no workgroup waits on another.
#include "common.h"
#include "kernels.h"

namespace rssm {

namespace {

// LDS plan in floats.  x rows are padded to XS = HD + 4 floats so that the
// lanes of a row group, each reading a different record's x rows in step 5,
// fall on different banks.
struct Lds {
    int X, XS, K, Cq, DT, AA, CO, DQ, WF, RED, total;
};

__host__ __device__ inline Lds lds_plan(int HD, int DS, int cap, int T) {
    Lds l;
    int o = 0;
    l.XS = HD + 4;
    l.X = o;  o += cap * l.XS; // x of records then queries, window order
    l.K = o;  o += cap * DS;   // B of records then queries
    l.Cq = o; o += T * DS;     // C of the queries
    l.DT = o; o += cap;        // dt, window order
    l.AA = o; o += cap;        // a = dt * A
    l.CO = o; o += T * cap;    // co[q][c] = dt_c exp(sum_{c<i<=m_q} a_i) (B_c . C_q) [+ D at c = m_q]
    l.DQ = o; o += T + 1;      // d_q = exp(sum_{first<=i<=m_q} a_i); [T] = flush decay
    l.WF = o; o += cap;        // flush weights dt_c exp(sum_{c<i<n} a_i)
    l.RED = o; o += 16;        // cross-wave reductions
    l.total = (o + 3) & ~3;
    return l;
}

// This thread's share of a tile held as raw 16-byte vectors (issued in step
// 1, consumed in steps 4 and 5): NV vectors of the tile's element size EB,
// laid out as TileGeo describes, in one register array sized for the FP32
// tile so the FP32 and read-copy paths share it.
template <int HD, int DS, int NT>
struct TileRegs {
    static constexpr int NMAX = TileGeo<HD, DS, NT, 4>::NV;
    v4u raw[NMAX];

    template <int EB>
    __device__ __forceinline__ void load(const void* tile, int tid) {
        using G = TileGeo<HD, DS, NT, EB>;
        static_assert(G::NV <= NMAX, "copy tile needs more vectors than the FP32 tile");
        if (tid >= G::ACTIVE) return;
        const v4u* base = reinterpret_cast<const v4u*>(tile);
#pragma unroll
        for (int s = 0; s < G::NV; ++s) raw[s] = __builtin_nontemporal_load(base + G::vec(tid, s));
    }

    // v[r] += (vector k of row r) . ck for each of the thread's NI rows; ck
    // holds the EPV columns of C under that vector.  Low-precision words are
    // widened one at a time, next to their use, so such a row never occupies
    // a full set of fp32 registers.
    template <int EB>
    __device__ __forceinline__ void dot_vec(int k, const float* ck, float* v) const {
        using G = TileGeo<HD, DS, NT, EB>;
#pragma unroll
        for (int r = 0; r < G::NI; ++r) {
            const v4u rv = raw[r * G::VPL + k];
            const uint32_t w[4] = {rv.x, rv.y, rv.z, rv.w};
            float acc = v[r];
            if constexpr (EB == 4) {
#pragma unroll
                for (int e = 0; e < 4; ++e) acc = fmaf(__uint_as_float(w[e]), ck[e], acc);
            } else if constexpr (EB == 2) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    uint32_t we = w[e];
                    asm volatile("" : "+v"(we));   // keep the widening inside the query loop
                    acc = fmaf(__uint_as_float(we << 16), ck[2 * e], acc);
                    acc = fmaf(__uint_as_float(we & 0xFFFF0000u), ck[2 * e + 1], acc);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    uint32_t we = w[e];
                    asm volatile("" : "+v"(we));   // decode next to its use, per query
                    float f[4];
                    e4m3x4_to_f32(we, f);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc = fmaf(f[i], ck[4 * e + i], acc);
                }
            }
            v[r] = acc;
        }
    }

    // All NMAX vectors as fp32 (FP32 tile only).
    __device__ __forceinline__ void widen(float (&f)[NMAX][4]) const {
#pragma unroll
        for (int s = 0; s < NMAX; ++s)
#pragma unroll
            for (int e = 0; e < 4; ++e) f[s][e] = __uint_as_float(raw[s][e]);
    }

    __device__ __forceinline__ void set(const float (&f)[NMAX][4]) {
#pragma unroll
        for (int s = 0; s < NMAX; ++s)
            raw[s] = v4u{__float_as_uint(f[s][0]), __float_as_uint(f[s][1]), __float_as_uint(f[s][2]),
                         __float_as_uint(f[s][3])};
    }
};

struct Window {
    int n, first, T, cap;
};

// Where staged vector v comes from and goes: the x rows of the window, then
// its B rows, then the queries' C rows.  Rows c < n are committed records read
// from the ring; rows c >= n are query tokens, whose x and B are also appended
// to the ring at slot (start + c) % cap.
struct StageMap {
    const void* bx;   // this head's x ring
    const void* bB;   // this group's B ring
    const void* xt;   // query tokens
    const void* Bt;
    const void* Ct;
    int start, n, cap, T, b, h, g, nheads, ngroups, nx, nb;
    int ldsX, ldsXS, ldsK, ldsC;
    bool append_x, append_B;
};

struct StageJob {
    const uint4* src;
    uint4* app;   // ring destination of a query's record, or null
    int dst;      // LDS offset (floats)
};

template <int HD, int DS, typename InT>
__device__ __forceinline__ StageJob stage_job(const StageMap& m, int v) {
    constexpr int EPVIN = InTraits<InT>::EPV;
    constexpr int VR = HD / EPVIN;
    constexpr int VS = DS / EPVIN;
    const uint4* bx = reinterpret_cast<const uint4*>(m.bx);
    const uint4* bB = reinterpret_cast<const uint4*>(m.bB);
    StageJob j;
    j.app = nullptr;
    if (v < m.nx) {
        const int c = v / VR, cv = v - c * VR;
        const uint4* ring = bx + (size_t)((m.start + c) % m.cap) * VR + cv;
        if (c < m.n) {
            j.src = ring;
        } else {
            j.src = reinterpret_cast<const uint4*>(m.xt) +
                    ((size_t)(m.b * m.T + c - m.n) * m.nheads + m.h) * VR + cv;
            if (m.append_x) j.app = const_cast<uint4*>(ring);
        }
        j.dst = m.ldsX + c * m.ldsXS + cv * EPVIN;
    } else if (v < m.nx + m.nb) {
        const int u = v - m.nx;
        const int c = u / VS, cv = u - c * VS;
        const uint4* ring = bB + (size_t)((m.start + c) % m.cap) * VS + cv;
        if (c < m.n) {
            j.src = ring;
        } else {
            j.src = reinterpret_cast<const uint4*>(m.Bt) +
                    ((size_t)(m.b * m.T + c - m.n) * m.ngroups + m.g) * VS + cv;
            if (m.append_B) j.app = const_cast<uint4*>(ring);
        }
        j.dst = m.ldsK + c * DS + cv * EPVIN;
    } else {
        const int u = v - m.nx - m.nb;
        const int q = u / VS, cv = u - q * VS;
        j.src = reinterpret_cast<const uint4*>(m.Ct) + ((size_t)(m.b * m.T + q) * m.ngroups + m.g) * VS + cv;
        j.dst = m.ldsC + q * DS + cv * EPVIN;
    }
    return j;
}

// Step 5 for one tile held in registers with element size EB.  For query q
// the thread forms, for each of its NI rows, d_q * (its columns' share of
// H C_q) plus its share of the record terms: lane j of a row group takes the
// records c = first + j, first + j + W, ... and adds co[q][c] x_c[row] (the
// D x_q term rides on co[q][m_q]).  One transposed reduction over the row's
// W lanes then leaves y_q[row] on one lane, which stores it.
template <int HD, int DS, int NT, int EB>
__device__ __forceinline__ void queries_and_outputs(const TileRegs<HD, DS, NT>& t, const float* lds,
                                                    const Lds& L, const Window& w, float scale,
                                                    float* y_head, size_t y_qstride, int tid) {
    using G = TileGeo<HD, DS, NT, EB>;
    const int j = tid % G::W;
    const int row0 = G::row0(tid);
    const int lane = tid & 63;
    for (int q = 0; q < w.T; ++q) {
        float v[16];
#pragma unroll
        for (int r = 0; r < G::NI; ++r) v[r] = 0.f;
#pragma unroll
        for (int k = 0; k < G::VPL; ++k) {
            float c[G::EPV];
#pragma unroll
            for (int e = 0; e < G::EPV; e += 4) {
                const float4 cv =
                    *reinterpret_cast<const float4*>(lds + L.Cq + q * DS + (j + G::W * k) * G::EPV + e);
                c[e] = cv.x;
                c[e + 1] = cv.y;
                c[e + 2] = cv.z;
                c[e + 3] = cv.w;
            }
            t.template dot_vec<EB>(k, c, v);
        }
        const float dq = lds[L.DQ + q] * scale;
#pragma unroll
        for (int r = 0; r < G::NI; ++r) v[r] *= dq;
        const int m = w.n + q;
        for (int cc = w.first + j; cc <= m; cc += G::W) {
            const float co = lds[L.CO + q * w.cap + cc];
            const float* xr = lds + L.X + cc * L.XS + row0;
            if constexpr (G::NI % 4 == 0) {
#pragma unroll
                for (int r = 0; r < G::NI; r += 4) {
                    const float4 xv = *reinterpret_cast<const float4*>(xr + r);
                    v[r] = fmaf(co, xv.x, v[r]);
                    v[r + 1] = fmaf(co, xv.y, v[r + 1]);
                    v[r + 2] = fmaf(co, xv.z, v[r + 2]);
                    v[r + 3] = fmaf(co, xv.w, v[r + 3]);
                }
            } else if constexpr (G::NI == 2) {
                const float2 xv = *reinterpret_cast<const float2*>(xr);
                v[0] = fmaf(co, xv.x, v[0]);
                v[1] = fmaf(co, xv.y, v[1]);
            } else {
                v[0] = fmaf(co, xr[0], v[0]);
            }
        }
        int idx;
        const float u = transpose_reduce<G::NI, G::W>(v, lane, idx);
        if ((lane % G::W) < G::NI) y_head[q * y_qstride + row0 + idx] = u;
    }
}

template <int HD, int DS, int NT, typename InT, int RM>
__global__ __launch_bounds__(NT, 8) void replay_kernel(const ReplayArgs a) {
    extern __shared__ float lds[];
    using G32 = TileGeo<HD, DS, NT, 4>;
    constexpr int EBC = RM == READ_BF16 ? 2 : 1;     // element size of the read copy
    constexpr int EPVIN = InTraits<InT>::EPV;
    constexpr int VR = HD / EPVIN;                   // 16-byte vectors per x row
    constexpr int VS = DS / EPVIN;                   // 16-byte vectors per B/C row
    constexpr int NW = NT / 64;
    constexpr int JOBS = 2;                          // staged vectors per thread issued up front

    const int nwg = a.batch * a.nheads;
    const int wg = xcd_remap(blockIdx.x, nwg);
    const int b = wg / a.nheads;
    const int h = wg - b * a.nheads;
    const int hpg = a.nheads / a.ngroups;
    const int g = h / hpg;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int cap = a.cap;
    const int T = a.T;
    const size_t tile = (size_t)b * a.nheads + h;

    const int start = a.meta[2 * tile];
    const int n_stored = a.meta[2 * tile + 1];
    // Fused commit of the previous verification: len += accepted_prev[b].
    int acc_prev = 0;
    bool acc_ok = true;
    if (a.accepted_prev) {
        acc_prev = a.accepted_prev[b];
        acc_ok = acc_prev >= 0 && acc_prev <= a.T_prev && n_stored >= 0 && n_stored + acc_prev <= cap;
    }
    const int n = n_stored + acc_prev;

    if (!(acc_ok && start >= 0 && start < cap && n >= 0 && n + T <= cap)) {
        if (tid == 0 && h == 0 && a.status) atomicOr(a.status, (int)(acc_ok ? kStatusMeta : kStatusAccept));
        for (int o = tid; o < T * HD; o += NT) {
            const int q = o / HD, i = o - q * HD;
            a.y[((size_t)(b * T + q) * a.nheads + h) * HD + i] = __builtin_nanf("");
        }
        return;
    }

    const bool flush_call = a.mode == MODE_FLUSH;
    const bool cast_only = flush_call && n == 0 && (a.flags & kFlushForceCast) && RM != READ_F32;
    const bool fold = flush_call ? (n > 0 || cast_only) : (n >= a.L);
    if (flush_call && !fold) return;
    const int first = fold ? n : 0;  // first window index of the outputs
    const bool append = !flush_call;
    const int rows = n + T;          // window rows staged in LDS
    const float Ah = a.A[h];
    const float Dh = a.D[h];

    const Lds L = lds_plan(HD, DS, cap, T);

    // ---- 1/2. record loads, then the tile stream, then LDS staging --------------
    const InT* bx = reinterpret_cast<const InT*>(a.buf_x) + tile * cap * HD;
    const InT* bB = reinterpret_cast<const InT*>(a.buf_B) + ((size_t)b * a.ngroups + g) * cap * DS;
    const InT* xt = reinterpret_cast<const InT*>(a.x);
    const InT* Bt = reinterpret_cast<const InT*>(a.B);
    const InT* Ct = reinterpret_cast<const InT*>(a.C);
    const bool writer = (h % hpg) == 0;
    const int nx = rows * VR, nb = rows * VS, nc = T * VS;
    const int nv = nx + nb + nc;

    const StageMap sm{bx, bB, xt, Bt, Ct, start, n, cap, T, b, h, g, a.nheads, a.ngroups,
                      nx, nb, L.X, L.XS, L.K, L.Cq, append, append && writer};
    uint4 jv[JOBS];
#pragma unroll
    for (int j = 0; j < JOBS; ++j) {
        const int v = tid + j * NT;
        if (v < nv) jv[j] = *stage_job<HD, DS, InT>(sm, v).src;
    }
    float dtv = 0.f;
    float* bdt = a.buf_dt + tile * cap;
    if (tid < rows) {
        const int slot = (start + tid) % cap;
        dtv = tid < n ? bdt[slot] : a.dt[(size_t)(b * T + (tid - n)) * a.nheads + h];
    }

    // The tile this call streams: FP32 when it flushes or has no read copy.
    TileRegs<HD, DS, NT> treg;
    if (fold || RM == READ_F32) {
        treg.template load<4>(a.ckpt + tile * HD * DS, tid);
    } else {
        treg.template load<EBC>(reinterpret_cast<const uint8_t*>(a.ckpt_read) + tile * HD * DS * EBC, tid);
    }

#pragma unroll
    for (int j = 0; j < JOBS; ++j) {
        const int v = tid + j * NT;
        if (v < nv) {
            const StageJob jb = stage_job<HD, DS, InT>(sm, v);
            if (jb.app) *jb.app = jv[j];
            widen16<InT>(jv[j], lds + jb.dst);
        }
    }
    for (int v = tid + JOBS * NT; v < nv; v += NT) {   // windows too long for JOBS vectors a thread
        const StageJob jb = stage_job<HD, DS, InT>(sm, v);
        const uint4 val = *jb.src;
        if (jb.app) *jb.app = val;
        widen16<InT>(val, lds + jb.dst);
    }
    if (tid < rows) {
        if (append && tid >= n) bdt[(start + tid) % cap] = dtv;
        lds[L.DT + tid] = dtv;
        lds[L.AA + tid] = dtv * Ah;
    }
    for (int c = tid + NT; c < rows; c += NT) {   // windows longer than the workgroup
        const int slot = (start + c) % cap;
        float d;
        if (c < n) {
            d = bdt[slot];
        } else {
            d = a.dt[(size_t)(b * T + (c - n)) * a.nheads + h];
            if (append) bdt[slot] = d;
        }
        lds[L.DT + c] = d;
        lds[L.AA + c] = d * Ah;
    }
    __syncthreads();

    // ---- 3. coefficients: one 8-lane group per (query, record) pair ---------------
    // Pairs (q, c), c = first .. m_q, give co[q][c]; when the call folds, the n
    // pairs (T, c), c < n, give the flush weights.  The group's lanes split the
    // segment sum of a over (c, m] and the score B_c . C_q, and reduce both.
    {
        constexpr int NG = NT / 8;
        const int sub = tid & 7;
        const int per0 = n - first + 1;                      // pairs of query 0
        const int nflush = fold ? n : 0;
        const int npairs = nflush + T * per0 + T * (T - 1) / 2;
        for (int p = tid >> 3; p < npairs; p += NG) {
            int q, c;
            if (p < nflush) {
                q = T;
                c = p;
            } else {
                int r = p - nflush;
                q = 0;
                while (r >= per0 + q) r -= per0 + q++;
                c = first + r;
            }
            const int m = q < T ? n + q : n - 1;             // last record the weight spans
            float seg = 0.f;
            for (int i = c + 1 + sub; i <= m; i += 8) seg += lds[L.AA + i];
            float sc = 0.f;
            if (q < T) {
                for (int j4 = sub; j4 < DS / 4; j4 += 8) {
                    const float4 kb = *reinterpret_cast<const float4*>(lds + L.K + c * DS + 4 * j4);
                    const float4 cq = *reinterpret_cast<const float4*>(lds + L.Cq + q * DS + 4 * j4);
                    sc = fmaf(kb.x, cq.x, sc);
                    sc = fmaf(kb.y, cq.y, sc);
                    sc = fmaf(kb.z, cq.z, sc);
                    sc = fmaf(kb.w, cq.w, sc);
                }
                sc = group_sum<8>(sc);
            }
            seg = group_sum<8>(seg);
            if (sub == 0) {
                const float wgt = lds[L.DT + c] * expf(seg);
                if (q < T) {
                    lds[L.CO + q * cap + c] = fmaf(wgt, sc, c == m ? Dh : 0.f);
                    if (c == first) lds[L.DQ + q] = expf(seg + lds[L.AA + c]);
                } else {
                    lds[L.WF + c] = wgt;
                    if (c == 0) lds[L.DQ + T] = expf(seg + lds[L.AA + 0]);
                }
            }
        }
    }
    __syncthreads();

    // ---- 4/5. flush in registers, then queries and outputs --------------------------
    const Window win{n, first, T, cap};
    float* y_head = a.y ? a.y + ((size_t)b * T * a.nheads + h) * HD : nullptr;
    const size_t y_qstride = (size_t)a.nheads * HD;
    if (fold) {
        float f[G32::NV][4];
        const bool active = tid < G32::ACTIVE;
        const int j = tid % G32::W;
        const int row0 = G32::row0(tid);
        float* ck = a.ckpt + tile * HD * DS;
        float amax = 0.f;
        if (active) {
            treg.widen(f);
            if (n > 0) {
                const float df = lds[L.DQ + T];
#pragma unroll
                for (int s = 0; s < G32::NV; ++s)
#pragma unroll
                    for (int e = 0; e < 4; ++e) f[s][e] *= df;
                for (int c = 0; c < n; ++c) {
                    const float wf = lds[L.WF + c];
                    float xs[G32::NI];
#pragma unroll
                    for (int r = 0; r < G32::NI; ++r) xs[r] = lds[L.X + c * L.XS + row0 + r] * wf;
#pragma unroll
                    for (int k = 0; k < G32::VPL; ++k) {
                        const float4 kb = *reinterpret_cast<const float4*>(lds + L.K + c * DS + (j + G32::W * k) * 4);
#pragma unroll
                        for (int r = 0; r < G32::NI; ++r) {
                            float* fv = f[r * G32::VPL + k];
                            fv[0] = fmaf(xs[r], kb.x, fv[0]);
                            fv[1] = fmaf(xs[r], kb.y, fv[1]);
                            fv[2] = fmaf(xs[r], kb.z, fv[2]);
                            fv[3] = fmaf(xs[r], kb.w, fv[3]);
                        }
                    }
                }
                v4f* out = reinterpret_cast<v4f*>(ck);
#pragma unroll
                for (int s = 0; s < G32::NV; ++s) {
                    const v4f val = {f[s][0], f[s][1], f[s][2], f[s][3]};
                    __builtin_nontemporal_store(val, out + G32::vec(tid, s));
                }
            }
            if constexpr (RM == READ_BF16) {
                uint2* out = reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.ckpt_read) + tile * HD * DS);
#pragma unroll
                for (int s = 0; s < G32::NV; ++s)
                    out[G32::vec(tid, s)] =
                        make_uint2(f32x2_to_bf16x2(f[s][0], f[s][1]), f32x2_to_bf16x2(f[s][2], f[s][3]));
            }
            if constexpr (RM == READ_E4M3) {
#pragma unroll
                for (int s = 0; s < G32::NV; ++s)
#pragma unroll
                    for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fabsf(f[s][e]));
            }
        }
        if constexpr (RM == READ_E4M3) {
            amax = group_max<64>(amax);
            if (lane == 0) lds[L.RED + wave] = amax;
            __syncthreads();
            amax = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) amax = fmaxf(amax, lds[L.RED + w]);
            const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
            const float inv = 1.0f / sc;
            if (active) {
                uint32_t* out = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(a.ckpt_read) + tile * HD * DS);
#pragma unroll
                for (int s = 0; s < G32::NV; ++s)
                    out[G32::vec(tid, s)] = f32x4_to_e4m3(f[s][0] * inv, f[s][1] * inv, f[s][2] * inv, f[s][3] * inv);
            }
            if (tid == 0) a.ckpt_scale[tile] = sc;
        }
        if (active && T > 0) {
            treg.set(f);
            queries_and_outputs<HD, DS, NT, 4>(treg, lds, L, win, 1.0f, y_head, y_qstride, tid);
        }
    } else if constexpr (RM == READ_F32) {
        if (tid < G32::ACTIVE)
            queries_and_outputs<HD, DS, NT, 4>(treg, lds, L, win, 1.0f, y_head, y_qstride, tid);
    } else {
        if (tid < TileGeo<HD, DS, NT, EBC>::ACTIVE) {
            const float sc = RM == READ_E4M3 ? a.ckpt_scale[tile] : 1.0f;
            queries_and_outputs<HD, DS, NT, EBC>(treg, lds, L, win, sc, y_head, y_qstride, tid);
        }
    }

    // ---- 6. advance this head's ring pointer -----------------------------------------
    const int new_start = fold && n > 0 ? (start + n) % cap : start;
    const int new_n = (fold ? 0 : n) + (a.mode == MODE_DECODE ? 1 : 0);
    if ((new_start != start || new_n != n_stored) && tid == 0) {
        a.meta[2 * tile] = new_start;
        a.meta[2 * tile + 1] = new_n;
    }
}

template <int HD, int DS, typename InT, int RM>
hipError_t launch_one(const ReplayArgs& a, hipStream_t stream) {
    constexpr int NT = ShapeNT<HD, DS>::NT;
    const int nwg = a.batch * a.nheads;
    const size_t lds = (size_t)lds_plan(HD, DS, a.cap, a.T).total * sizeof(float);
    hipLaunchKernelGGL((replay_kernel<HD, DS, NT, InT, RM>), dim3(nwg), dim3(NT), lds, stream, a);
    return hipGetLastError();
}

template <int HD, int DS>
hipError_t launch_shape(const ReplayArgs& a, int in_type, int read_mode, hipStream_t stream) {
    if (in_type == IN_F32) {
        switch (read_mode) {
            case READ_F32: return launch_one<HD, DS, float, READ_F32>(a, stream);
            case READ_BF16: return launch_one<HD, DS, float, READ_BF16>(a, stream);
            case READ_E4M3: return launch_one<HD, DS, float, READ_E4M3>(a, stream);
        }
    } else {
        switch (read_mode) {
            case READ_F32: return launch_one<HD, DS, uint16_t, READ_F32>(a, stream);
            case READ_BF16: return launch_one<HD, DS, uint16_t, READ_BF16>(a, stream);
            case READ_E4M3: return launch_one<HD, DS, uint16_t, READ_E4M3>(a, stream);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace

size_t replay_lds_bytes(int hd, int ds, int cap, int T, int /*in_bytes: records are widened to fp32*/) {
    return (size_t)lds_plan(hd, ds, cap, T).total * sizeof(float);
}

bool shape_supported(int hd, int ds) {
    return (hd == 16 && ds == 16) || (hd == 64 && ds == 64) || (hd == 64 && ds == 128) ||
           (hd == 128 && ds == 128);
}

hipError_t launch_replay(const ReplayArgs& a, int hd, int ds, int in_type, int read_mode,
                         hipStream_t stream) {
    if (hd == 16 && ds == 16) return launch_shape<16, 16>(a, in_type, read_mode, stream);
    if (hd == 64 && ds == 64) return launch_shape<64, 64>(a, in_type, read_mode, stream);
    if (hd == 64 && ds == 128) return launch_shape<64, 128>(a, in_type, read_mode, stream);
    if (hd == 128 && ds == 128) return launch_shape<128, 128>(a, in_type, read_mode, stream);
    return hipErrorInvalidValue;
}

}  // namespace rssm
