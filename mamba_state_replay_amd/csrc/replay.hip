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
//   3. decay weights w[q][c] = dt_c exp(sum_{c<i<=m_q} a_i) (one thread per
//      (query, record) pair, segment sums, never ratios of exponentials) and
//      the group scores s[q][c] = B_c . C_q (one wave per pair);
//   4. flush: H = exp(sum a) H_s + sum_k dt_k exp(sum_{k<i<n} a_i) x_k B_k^T,
//      the rank-n update applied to the tile in registers, written once, with
//      the read copy cast from the same registers (section "Benefit 3": the
//      copy is never read back into the recurrence);
//   5. per query, u_q = H C_q from the same registers (section "Benefit 2":
//      the checkpoint is read once for all queries), reduced across the lanes
//      of each row; the lane that ends up with row i's sum writes
//      y_q[i] = d_q u_q[i] + sum_{c<=m} w[q][c] s[q][c] x_c[i] + D x_q[i]
//      (output-only evaluation: no intermediate state is formed);
//   6. write the head's new ring pointer.  Every head keeps its own copy of
//      {start, n} (all copies of a sequence are equal), read and written only
//      by the workgroup that owns the head, so no workgroup waits on another.
#include "common.h"
#include "kernels.h"

namespace rssm {

namespace {

// LDS plan in floats.
struct Lds {
    int X, K, Cq, DT, AA, W, S, DQ, WF, RED, total;
};

__host__ __device__ inline Lds lds_plan(int HD, int DS, int cap, int T) {
    Lds l;
    int o = 0;
    l.X = o;  o += cap * HD;   // x of records then queries, window order
    l.K = o;  o += cap * DS;   // B of records then queries
    l.Cq = o; o += T * DS;     // C of the queries
    l.DT = o; o += cap;        // dt, window order
    l.AA = o; o += cap;        // a = dt * A
    l.W = o;  o += T * cap;    // w[q][c] = dt_c exp(sum_{c<i<=m_q} a_i)
    l.S = o;  o += T * cap;    // s[q][c] = B_c . C_q
    l.DQ = o; o += T + 1;      // d_q = exp(sum_{first<=i<=m_q} a_i); [T] = flush decay
    l.WF = o; o += cap;        // flush weights dt_c exp(sum_{c<i<n} a_i)
    l.RED = o; o += 16;        // cross-wave reductions
    l.total = (o + 3) & ~3;
    return l;
}

// This thread's share of a tile held as raw 16-byte vectors (issued in step
// 1, consumed in step 4): NI vectors of the tile's element size EB, in one
// register array sized for the FP32 tile so the FP32 and read-copy paths
// share it.  widen() gives fp32 rows: f[s][e] is element (row0 + s,
// colv*EPV + e) of the thread's rows.
template <int HD, int DS, int NT>
struct TileRegs {
    static constexpr int NMAX = TileGeo<HD, DS, NT, 4>::NI;
    v4u raw[NMAX];

    template <int EB>
    __device__ __forceinline__ void load(const void* tile, int tid) {
        using G = TileGeo<HD, DS, NT, EB>;
        static_assert(G::NI <= NMAX, "copy tile needs more vectors than the FP32 tile");
        if (tid >= G::ACTIVE) return;
        const int colv = tid % G::LPR;
        const int row0 = (tid / G::LPR) * G::NI;
        const v4u* base = reinterpret_cast<const v4u*>(tile);
#pragma unroll
        for (int s = 0; s < G::NI; ++s)
            raw[s] = __builtin_nontemporal_load(base + (size_t)(row0 + s) * G::LPR + colv);
    }

    // Row s of this thread's share, widened to fp32 (16 / EB values).
    template <int EB>
    __device__ __forceinline__ void widen_row(int s, float* f) const {
        const uint32_t w[4] = {raw[s].x, raw[s].y, raw[s].z, raw[s].w};
        if constexpr (EB == 4) {
#pragma unroll
            for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(w[e]);
        } else if constexpr (EB == 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[2 * e] = __uint_as_float(w[e] << 16);
                f[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) e4m3x4_to_f32(w[e], f + 4 * e);
        }
    }

    // sum_e row_s[e] * c[e] over this thread's 16 / EB columns of row s; c
    // points at those columns of C in LDS.  Widens and multiplies one 32-bit
    // word at a time so a low-precision row never occupies 16 fp32 registers.
    template <int EB>
    __device__ __forceinline__ float dot_row(int s, const float* c) const {
        const uint32_t w[4] = {raw[s].x, raw[s].y, raw[s].z, raw[s].w};
        float acc = 0.f;
        if constexpr (EB == 4) {
            const float4 cv = *reinterpret_cast<const float4*>(c);
            acc = fmaf(__uint_as_float(w[0]), cv.x, acc);
            acc = fmaf(__uint_as_float(w[1]), cv.y, acc);
            acc = fmaf(__uint_as_float(w[2]), cv.z, acc);
            acc = fmaf(__uint_as_float(w[3]), cv.w, acc);
        } else if constexpr (EB == 2) {
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
                uint32_t w0 = w[e], w1 = w[e + 1];
                // keep the widening next to its use (not hoisted out of the query loop)
                asm volatile("" : "+v"(w0), "+v"(w1));
                const float4 cv = *reinterpret_cast<const float4*>(c + 2 * e);
                acc = fmaf(__uint_as_float(w0 << 16), cv.x, acc);
                acc = fmaf(__uint_as_float(w0 & 0xFFFF0000u), cv.y, acc);
                acc = fmaf(__uint_as_float(w1 << 16), cv.z, acc);
                acc = fmaf(__uint_as_float(w1 & 0xFFFF0000u), cv.w, acc);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint32_t we = w[e];
                asm volatile("" : "+v"(we));   // decode next to its use, per query
                const float4 cv = *reinterpret_cast<const float4*>(c + 4 * e);
                float f[4];
                e4m3x4_to_f32(we, f);
                acc = fmaf(f[0], cv.x, acc);
                acc = fmaf(f[1], cv.y, acc);
                acc = fmaf(f[2], cv.z, acc);
                acc = fmaf(f[3], cv.w, acc);
            }
        }
        return acc;
    }

    // All NMAX rows as fp32 (FP32 tile only).
    __device__ __forceinline__ void widen(float (&f)[NMAX][4]) const {
#pragma unroll
        for (int s = 0; s < NMAX; ++s) widen_row<4>(s, f[s]);
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
    int ldsX, ldsK, ldsC;
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
        j.dst = m.ldsX + c * HD + cv * EPVIN;
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

// Step 5 for one tile held in registers with element size EB: for every
// query, reduce u_q over the lanes of each row, then the lane holding row i's
// sum writes y_q[i].  Rows are widened to fp32 one at a time, inside the query
// loop, so a low-precision tile never needs a full fp32 copy in registers.
template <int HD, int DS, int NT, int EB>
__device__ __forceinline__ void queries_and_outputs(const TileRegs<HD, DS, NT>& t, const float* lds,
                                                    const Lds& L, const Window& w, float scale, float Dh,
                                                    float* y_head, size_t y_qstride, int tid) {
    using G = TileGeo<HD, DS, NT, EB>;
    const int colv = tid % G::LPR;
    const int row0 = (tid / G::LPR) * G::NI;
    const int lane = tid & 63;
    for (int q = 0; q < w.T; ++q) {
        const float* c = lds + L.Cq + q * DS + colv * G::EPV;
        float v[16];
#pragma unroll
        for (int s = 0; s < G::NI; ++s) v[s] = t.template dot_row<EB>(s, c);
        int idx;
        const float u = transpose_reduce<G::NI, G::LPR>(v, lane, idx);
        if ((lane % G::LPR) < G::NI) {
            const int row = row0 + idx;
            const int m = w.n + q;
            float acc = lds[L.DQ + q] * (u * scale);
#pragma unroll 4
            for (int cc = w.first; cc <= m; ++cc)
                acc = fmaf(lds[L.W + q * w.cap + cc] * lds[L.S + q * w.cap + cc], lds[L.X + cc * HD + row], acc);
            acc = fmaf(Dh, lds[L.X + m * HD + row], acc);
            y_head[q * y_qstride + row] = acc;
        }
    }
}

template <int HD, int DS, int NT, typename InT, int RM>
__global__ __launch_bounds__(NT, 2048 / NT) void replay_kernel(const ReplayArgs a) {
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
                      nx, nb, L.X, L.K, L.Cq, append, append && writer};
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

    // ---- 3. decay weights and scores ------------------------------------------------
    for (int p = tid; p < (T + 1) * cap; p += NT) {
        const int q = p / cap, c = p - q * cap;
        if (q < T) {
            const int m = n + q;
            if (c >= first && c <= m) {
                float s = 0.f;
#pragma unroll 4
                for (int i = c + 1; i <= m; ++i) s += lds[L.AA + i];
                lds[L.W + q * cap + c] = lds[L.DT + c] * expf(s);
                if (c == first) lds[L.DQ + q] = expf(s + lds[L.AA + c]);
            }
        } else if (fold && c < n) {
            float s = 0.f;
#pragma unroll 4
            for (int i = c + 1; i < n; ++i) s += lds[L.AA + i];
            lds[L.WF + c] = lds[L.DT + c] * expf(s);
            if (c == 0) lds[L.DQ + T] = expf(s + lds[L.AA + 0]);
        }
    }
    for (int q = 0; q < T; ++q) {
        for (int c = first + wave; c <= n + q; c += NW) {
            float p = 0.f;
            for (int j = lane; j < DS; j += 64) p = fmaf(lds[L.K + c * DS + j], lds[L.Cq + q * DS + j], p);
            p = group_sum<64>(p);
            if (lane == 0) lds[L.S + q * cap + c] = p;
        }
    }
    __syncthreads();

    // ---- 4/5. flush in registers, then queries and outputs --------------------------
    const Window win{n, first, T, cap};
    float* y_head = a.y ? a.y + ((size_t)b * T * a.nheads + h) * HD : nullptr;
    const size_t y_qstride = (size_t)a.nheads * HD;
    if (fold) {
        float f[G32::NI][4];
        const bool active = tid < G32::ACTIVE;
        const int colv = tid % G32::LPR;
        const int row0 = (tid / G32::LPR) * G32::NI;
        float* ck = a.ckpt + tile * HD * DS;
        float amax = 0.f;
        if (active) {
            treg.widen(f);
            if (n > 0) {
                const float df = lds[L.DQ + T];
#pragma unroll
                for (int s = 0; s < G32::NI; ++s)
#pragma unroll
                    for (int e = 0; e < 4; ++e) f[s][e] *= df;
                for (int c = 0; c < n; ++c) {
                    const float wf = lds[L.WF + c];
                    const float4 kb = *reinterpret_cast<const float4*>(lds + L.K + c * DS + colv * 4);
                    float xs[G32::NI];
#pragma unroll
                    for (int s = 0; s < G32::NI; ++s) xs[s] = lds[L.X + c * HD + row0 + s] * wf;
#pragma unroll
                    for (int s = 0; s < G32::NI; ++s) {
                        f[s][0] = fmaf(xs[s], kb.x, f[s][0]);
                        f[s][1] = fmaf(xs[s], kb.y, f[s][1]);
                        f[s][2] = fmaf(xs[s], kb.z, f[s][2]);
                        f[s][3] = fmaf(xs[s], kb.w, f[s][3]);
                    }
                }
                v4f* out = reinterpret_cast<v4f*>(ck);
#pragma unroll
                for (int s = 0; s < G32::NI; ++s) {
                    const v4f val = {f[s][0], f[s][1], f[s][2], f[s][3]};
                    __builtin_nontemporal_store(val, out + (size_t)(row0 + s) * G32::LPR + colv);
                }
            }
            if constexpr (RM == READ_BF16) {
                uint2* out = reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.ckpt_read) + tile * HD * DS);
#pragma unroll
                for (int s = 0; s < G32::NI; ++s) {
                    out[(size_t)(row0 + s) * G32::LPR + colv] =
                        make_uint2(f32x2_to_bf16x2(f[s][0], f[s][1]), f32x2_to_bf16x2(f[s][2], f[s][3]));
                }
            }
            if constexpr (RM == READ_E4M3) {
#pragma unroll
                for (int s = 0; s < G32::NI; ++s)
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
                for (int s = 0; s < G32::NI; ++s) {
                    out[(size_t)(row0 + s) * G32::LPR + colv] =
                        f32x4_to_e4m3(f[s][0] * inv, f[s][1] * inv, f[s][2] * inv, f[s][3] * inv);
                }
            }
            if (tid == 0) a.ckpt_scale[tile] = sc;
        }
        if (active && T > 0) {
            treg.set(f);
            queries_and_outputs<HD, DS, NT, 4>(treg, lds, L, win, 1.0f, Dh, y_head, y_qstride, tid);
        }
    } else if constexpr (RM == READ_F32) {
        if (tid < G32::ACTIVE)
            queries_and_outputs<HD, DS, NT, 4>(treg, lds, L, win, 1.0f, Dh, y_head, y_qstride, tid);
    } else {
        if (tid < TileGeo<HD, DS, NT, EBC>::ACTIVE) {
            const float sc = RM == READ_E4M3 ? a.ckpt_scale[tile] : 1.0f;
            queries_and_outputs<HD, DS, NT, EBC>(treg, lds, L, win, sc, Dh, y_head, y_qstride, tid);
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
