// Kernel templates and launch helpers of the ReplaySSM decode / verify /
// flush kernel (gfx950), shared by the translation units that instantiate
// them (replay.hip: FP32 checkpoint; replay_f16.hip: FP16 checkpoint).  The
// method and the steps of a call are described at the top of replay.hip.
#pragma once

#include "common.h"
#include "kernels.h"

namespace rssm {

namespace {

// LDS plan in floats for a workgroup serving HPW heads of one group.  The x
// and B rows keep the input element type (xbytes = 4 for fp32, 2 for bf16;
// they are widened where they are read), which keeps a workgroup's LDS small
// enough for 8 workgroups per CU at up to 8 drafts; x rows are padded to XS
// elements, a row stride of 4 banks mod 32, so that the lanes of a row group,
// each reading a different record's x in step 5, fall on different banks.
// Per-head arrays are indexed [head][...]; B rows are the group's and shared
// by the heads; the queries' C rows are widened to fp32.
struct Lds {
    int X, XS, K, SC, Cq, Cb, DT, AA, CO, DQ, WF, RED, total;
};

constexpr int kRedSlots = 64;   // cross-wave reduction slots: [head][wave]

// mxbytes: the MX scale bytes of one head's tile (HD * DS / 32), staged for
// the copy-reading calls of the MX modes; 0 otherwise.
__host__ __device__ inline Lds lds_plan(int HD, int DS, int cap, int T, int HPW, int xbytes, int mxbytes = 0) {
    Lds l;
    int o = 0;
    l.XS = xbytes == 4 ? HD + 4 : HD + 8;           // elements; 16-byte aligned rows
    l.X = o;  o += HPW * cap * l.XS * xbytes / 4;    // x of records then queries, window order, per head
    l.K = o;  o += cap * DS * xbytes / 4;   // B of records then queries (input type)
    l.SC = o; o += HPW * mxbytes / 4;       // MX scale bytes of the heads' tiles
    l.Cq = o; o += T * DS;           // C of the queries
    l.Cb = o; o += xbytes == 2 ? T * DS / 2 : 0;   // bf16 inputs: C of the queries as bf16 pairs too
    l.DT = o; o += HPW * cap;        // dt, window order, per head
    l.AA = o; o += HPW * cap;        // a = dt * A, per head
    l.CO = o; o += HPW * T * cap;    // co[h][q][c] = dt_c exp(sum_{c<i<=m_q} a_i) (B_c . C_q) [+ D at c = m_q]
    l.DQ = o; o += HPW * (T + 1);    // d[h][q] = exp(sum_{first<=i<=m_q} a_i); [h][T] = flush decay
    l.WF = o; o += HPW * cap;        // flush weights dt_c exp(sum_{c<i<n} a_i), per head
    l.RED = o; o += kRedSlots;       // cross-wave reductions
    l.total = (o + 3) & ~3;
    return l;
}

// One head's view of the per-head LDS arrays.
struct HeadView {
    int X, DT, AA, CO, DQ, WF;
};

// X is the head's x block in floats; its rows hold elements of type InT.
template <typename InT>
__device__ __forceinline__ HeadView head_view(const Lds& L, int hh, int cap, int T) {
    return HeadView{L.X + hh * cap * L.XS * (int)sizeof(InT) / 4, L.DT + hh * cap, L.AA + hh * cap,
                    L.CO + hh * T * cap, L.DQ + hh * (T + 1), L.WF + hh * cap};
}

// x_c[row0 .. row0 + N - 1] of one head as fp32, from a row of InT elements.
template <typename InT, int N>
__device__ __forceinline__ void load_x(const float* lds, int xblock, int elem, float (&out)[N]) {
    if constexpr (sizeof(InT) == 4) {
        const float* p = lds + xblock + elem;
        if constexpr (N % 4 == 0) {
#pragma unroll
            for (int r = 0; r < N; r += 4) {
                const float4 v = *reinterpret_cast<const float4*>(p + r);
                out[r] = v.x;
                out[r + 1] = v.y;
                out[r + 2] = v.z;
                out[r + 3] = v.w;
            }
        } else if constexpr (N == 2) {
            const float2 v = *reinterpret_cast<const float2*>(p);
            out[0] = v.x;
            out[1] = v.y;
        } else {
#pragma unroll
            for (int r = 0; r < N; ++r) out[r] = p[r];
        }
    } else {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(lds + xblock) + elem;
        if constexpr (N % 2 == 0) {
#pragma unroll
            for (int r = 0; r < N; r += 2) {
                const uint32_t w = *reinterpret_cast<const uint32_t*>(p + r);
                out[r] = __uint_as_float(w << 16);
                out[r + 1] = __uint_as_float(w & 0xFFFF0000u);
            }
        } else {
#pragma unroll
            for (int r = 0; r < N; ++r) out[r] = bf16_to_f32(p[r]);
        }
    }
}

// This thread's share of a tile held as raw 16-byte vectors (issued in step
// 1, consumed in steps 4 and 5): NV vectors of the tile's element size EB,
// laid out as TileGeo describes, in one register array sized for the FP32
// tile so the FP32 and read-copy paths share it.
template <int HD, int DS, int NT>
struct TileRegs {
    static constexpr int NMAX = TileGeo<HD, DS, NT, 4>::NV;
    v4f raw[NMAX];   // fp32 values, or the bits of bf16 / e4m3 codes

    // Load one tile of element size EB into vectors off .. off + NV - 1.
    template <int EB, int OFF = 0>
    __device__ __forceinline__ void load(const void* tile, int tid) {
        using G = TileGeo<HD, DS, NT, EB>;
        static_assert(OFF + G::NV <= NMAX, "tiles need more vectors than the FP32 tile");
        if (G::ACTIVE < NT && tid >= G::ACTIVE) return;
        const v4u* base = reinterpret_cast<const v4u*>(tile);
#pragma unroll
        for (int s = 0; s < G::NV; ++s)
            raw[OFF + s] = __builtin_bit_cast(v4f, __builtin_nontemporal_load(base + G::vec(tid, s)));
    }

    // v[r] += (row r of this thread's share) . C for each of its NI rows.  cq
    // points at C in LDS; the thread's columns are (j + W k) * EPV + e.  The
    // product runs over chunks of 4 columns: one float4 of C, then for every row
    // the 4 tile values under it (an fp32 quarter-vector, two bf16 words or
    // one e4m3 word, widened next to its use), so few values are live at once.
    //
    // DOT2 (bf16 inputs, 1- and 2-byte copy tiles): cb points at C as bf16
    // pairs; a bf16 copy word is already a pair, and an e4m3 word becomes two
    // pairs by gfx950's fp8 -> bf16 converter (exact, scale 1: the copy's scale
    // is applied to the sum), so each pair of columns is one v_dot2c_f32_bf16
    // (the products of two bf16 values are exact in fp32) instead of a widening
    // step and two FMAs.
    template <int EB, int OFF = 0, bool F16 = false, bool DOT2 = false>
    __device__ __forceinline__ void dot(const float* cq, const uint32_t* cb, int j, float* v) const {
        using G = TileGeo<HD, DS, NT, EB>;
        if constexpr (DOT2) {
            static_assert((EB == 2 && !F16) || EB == 1, "pairs of bf16 or e4m3 codes");
#pragma unroll
            for (int k = 0; k < G::VPL; ++k) {
                const uint4* cp = reinterpret_cast<const uint4*>(cb + (j + G::W * k) * G::EPV / 2);
#pragma unroll
                for (int h = 0; h < G::EPV / 8; ++h) {            // 8 columns (4 C pairs) at a time
                    const uint4 c = cp[h];
                    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
                    for (int r = 0; r < G::NI; ++r) {
                        const v4u rv = __builtin_bit_cast(v4u, raw[OFF + r * G::VPL + k]);
                        const uint32_t tw[4] = {rv.x, rv.y, rv.z, rv.w};
                        float acc = v[r];
                        if constexpr (EB == 2) {
#pragma unroll
                            for (int w = 0; w < 4; ++w) acc = dot2_bf16(tw[w], cw[w], acc);
                        } else {
#pragma unroll
                            for (int w = 0; w < 2; ++w) {
                                uint32_t code = tw[2 * h + w];
                                asm volatile("" : "+v"(code));          // decode inside the query loop
                                acc = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(code, 1.0f, false), cw[2 * w], acc);
                                acc = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(code, 1.0f, true), cw[2 * w + 1], acc);
                            }
                        }
                        v[r] = acc;
                    }
                }
            }
            return;
        }
#pragma unroll
        for (int k = 0; k < G::VPL; ++k) {
#pragma unroll
            for (int ch = 0; ch < G::EPV / 4; ++ch) {
                const float4 c = *reinterpret_cast<const float4*>(cq + (j + G::W * k) * G::EPV + 4 * ch);
#pragma unroll
                for (int r = 0; r < G::NI; ++r) {
                    const v4f rf = raw[OFF + r * G::VPL + k];
                    const v4u rv = __builtin_bit_cast(v4u, rf);
                    float f[4];
                    if constexpr (EB == 4) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) f[e] = rf[e];
                    } else if constexpr (EB == 2) {
                        uint32_t w0 = rv[2 * ch], w1 = rv[2 * ch + 1];
                        asm volatile("" : "+v"(w0), "+v"(w1));   // widen inside the query loop
                        if constexpr (F16) {                      // fp16 checkpoint
                            f[0] = f16lo_to_f32(w0);
                            f[1] = f16hi_to_f32(w0);
                            f[2] = f16lo_to_f32(w1);
                            f[3] = f16hi_to_f32(w1);
                        } else {                                  // bf16 copy
                            f[0] = __uint_as_float(w0 << 16);
                            f[1] = __uint_as_float(w0 & 0xFFFF0000u);
                            f[2] = __uint_as_float(w1 << 16);
                            f[3] = __uint_as_float(w1 & 0xFFFF0000u);
                        }
                    } else {
                        uint32_t w = rv[ch];
                        asm volatile("" : "+v"(w));              // decode inside the query loop
                        e4m3x4_to_f32(w, f);
                    }
                    float acc = v[r];
                    acc = fmaf(f[0], c.x, acc);
                    acc = fmaf(f[1], c.y, acc);
                    acc = fmaf(f[2], c.z, acc);
                    acc = fmaf(f[3], c.w, acc);
                    v[r] = acc;
                }
            }
        }
    }
};

struct Window {
    int n, first, T, cap;
};

// Where staged vector v comes from and goes: the x rows of the window of
// each head, then the group's B rows, then the queries' C rows, then (MX
// copies, calls that read the copy) the heads' scale bytes.  Rows c < n
// are committed records read from the ring; rows c >= n are query tokens,
// whose x and B are also appended to the ring at slot (start + c) % cap.
struct StageMap {
    const void* bx;   // the first head's x ring (heads follow at cap * HD elements)
    const void* bB;   // this group's B ring
    const void* xt;   // query tokens
    const void* Bt;
    const void* Ct;
    int start, n, cap, T, b, h, g, nheads, ngroups, nx, nb, rows;
    int ldsX, ldsXS, ldsK, ldsC;
    bool append_x, append_B;
    const void* sc;   // MX scale bytes of the workgroup's heads (contiguous), staged after the C rows
    int nc, ldsSC;
};

struct StageJob {
    const uint4* src;
    uint4* app;   // ring destination of a query's record, or null
    int dst;      // LDS offset in bytes
    bool wide;    // widen to fp32 (B and C rows) or keep the input type (x rows)
};

// (start + c) mod cap for 0 <= start < cap and 0 <= c < cap (a window never
// exceeds the ring), without a division.
__device__ __forceinline__ int ring_slot(int start, int c, int cap) {
    const int s = start + c;
    return s >= cap ? s - cap : s;
}

// v / span for 0 <= v < HPW * span, without a division (HPW <= 4).
template <int HPW>
__device__ __forceinline__ int block_of(int v, int span) {
    int k = 0;
#pragma unroll
    for (int i = 1; i < HPW; ++i) k += v >= i * span ? 1 : 0;
    return k;
}

template <int HD, int DS, typename InT, int HPW>
__device__ __forceinline__ StageJob stage_job(const StageMap& m, int v) {
    constexpr int EPVIN = InTraits<InT>::EPV;
    constexpr int VR = HD / EPVIN;
    constexpr int VS = DS / EPVIN;
    const uint4* bx = reinterpret_cast<const uint4*>(m.bx);
    const uint4* bB = reinterpret_cast<const uint4*>(m.bB);
    StageJob j;
    j.app = nullptr;
    if (v < m.nx) {
        const int hh = block_of<HPW>(v, m.rows * VR);
        const int u = v - hh * m.rows * VR;
        const int c = u / VR, cv = u - c * VR;
        const uint4* ring = bx + ((size_t)hh * m.cap + ring_slot(m.start, c, m.cap)) * VR + cv;
        if (c < m.n) {
            j.src = ring;
        } else {
            j.src = reinterpret_cast<const uint4*>(m.xt) +
                    ((size_t)(m.b * m.T + c - m.n) * m.nheads + m.h + hh) * VR + cv;
            if (m.append_x) j.app = const_cast<uint4*>(ring);
        }
        j.dst = m.ldsX * 4 + ((hh * m.cap + c) * m.ldsXS + cv * EPVIN) * (int)sizeof(InT);
        j.wide = false;
    } else if (v < m.nx + m.nb) {
        const int u = v - m.nx;
        const int c = u / VS, cv = u - c * VS;
        const uint4* ring = bB + (size_t)ring_slot(m.start, c, m.cap) * VS + cv;
        if (c < m.n) {
            j.src = ring;
        } else {
            j.src = reinterpret_cast<const uint4*>(m.Bt) +
                    ((size_t)(m.b * m.T + c - m.n) * m.ngroups + m.g) * VS + cv;
            if (m.append_B) j.app = const_cast<uint4*>(ring);
        }
        j.dst = m.ldsK * 4 + (c * DS + cv * EPVIN) * (int)sizeof(InT);
        j.wide = false;
    } else if (v < m.nx + m.nb + m.nc) {
        const int u = v - m.nx - m.nb;
        const int q = u / VS, cv = u - q * VS;
        j.src = reinterpret_cast<const uint4*>(m.Ct) + ((size_t)(m.b * m.T + q) * m.ngroups + m.g) * VS + cv;
        j.dst = (m.ldsC + q * DS + cv * EPVIN) * 4;
        j.wide = true;
    } else {
        const int u = v - m.nx - m.nb - m.nc;
        j.src = reinterpret_cast<const uint4*>(m.sc) + u;
        j.dst = m.ldsSC * 4 + u * 16;
        j.wide = false;
    }
    return j;
}

// A C vector (jb.wide) of bf16 inputs is stored widened at Cq and as it came
// (bf16 pairs) at the same element offset in Cb.
template <typename InT>
__device__ __forceinline__ void stage_store(float* lds, const StageJob& jb, const uint4 v, const Lds& L) {
    char* d = reinterpret_cast<char*>(lds) + jb.dst;
    if (sizeof(InT) == 4 || !jb.wide) {
        *reinterpret_cast<uint4*>(d) = v;
    } else {
        widen16<InT>(v, reinterpret_cast<float*>(d));
        *reinterpret_cast<uint4*>(reinterpret_cast<char*>(lds) + L.Cb * 4 + (jb.dst - L.Cq * 4) / 2) = v;
    }
}

// B_c[col .. col + 3] as fp32 from the B rows in LDS (input type).
template <typename InT, int DS>
__device__ __forceinline__ float4 load_b4(const float* lds, int K, int c, int col) {
    if constexpr (sizeof(InT) == 4) {
        return *reinterpret_cast<const float4*>(lds + K + c * DS + col);
    } else {
        const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(lds + K) + c * DS + col);
        return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                           __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u));
    }
}

// Step 5 for one head's tile held in registers (vectors OFF ..) with element
// size EB.  For query q the thread forms, for each of its NI rows, d_q * (its
// columns' share of H C_q) plus its share of the record terms: lane j of a
// row group takes the records c = first + j, first + j + W, ... and adds
// co[q][c] x_c[row] (the D x_q term rides on co[q][m_q]).  One transposed
// reduction over the row's W lanes then leaves y_q[row] on one lane, which
// stores it.  rs[r] scales the tile's share of row r (the read copy's scale:
// one per tile, or per block of 32 columns for the MX copies).
template <int HD, int DS, int NT, typename InT, int EB, int OFF = 0, bool F16 = false>
__device__ __forceinline__ void queries_and_outputs(const TileRegs<HD, DS, NT>& t, const float* lds,
                                                    const Lds& L, const HeadView& hv, const Window& w,
                                                    const float* rs, float* y_head, size_t y_qstride, int tid) {
    using G = TileGeo<HD, DS, NT, EB>;
    const int j = tid % G::W;
    const int row0 = G::row0(tid);
    const int lane = tid & 63;
    for (int q = 0; q < w.T; ++q) {
        float v[16];
#pragma unroll
        for (int r = 0; r < G::NI; ++r) v[r] = 0.f;
        constexpr bool DOT2 = InTraits<InT>::EPV == 8 && (EB == 1 || (EB == 2 && !F16));
        t.template dot<EB, OFF, F16, DOT2>(lds + L.Cq + q * DS,
                                           reinterpret_cast<const uint32_t*>(lds + L.Cb) + q * DS / 2, j, v);
        const float dq = lds[hv.DQ + q];
#pragma unroll
        for (int r = 0; r < G::NI; ++r) v[r] *= dq * rs[r];
        const int m = w.n + q;
        for (int cc = w.first + j; cc <= m; cc += G::W) {
            const float co = lds[hv.CO + q * w.cap + cc];
            float xv[G::NI];
            load_x<InT, G::NI>(lds, hv.X, cc * L.XS + row0, xv);
#pragma unroll
            for (int r = 0; r < G::NI; ++r) v[r] = fmaf(co, xv[r], v[r]);
        }
        int idx;
        const float u = transpose_reduce<G::NI, G::W>(v, lane, idx);
        if ((lane % G::W) < G::NI) y_head[q * y_qstride + row0 + idx] = u;
    }
}

// The E8M0 scale byte of the block that row r of the thread's share of head
// hh's copy tile lies in (from the scale bytes staged in LDS).
template <int HD, int DS, int NT, int EBC>
__device__ __forceinline__ uint32_t mx_scale_byte(const float* lds, const Lds& L, int hh, int r, int tid) {
    using GC = TileGeo<HD, DS, NT, EBC>;
    const int blk = GC::vec(tid, r * GC::VPL) * GC::EPV / 32;
    return reinterpret_cast<const uint8_t*>(lds + L.SC)[hh * (HD * DS / 32) + blk];
}

// The read-copy tiles of HPW heads, each over the whole workgroup in its own
// vectors of the register array: step 5 for every head.  Row scales: the
// head's tile scale (scales[HH], or 1 without one), or with MX the E8M0 scale
// of the block each of the thread's rows holds.
template <int HD, int DS, int NT, typename InT, int EBC, int HPW, bool MX, bool F16, int HH = 0>
__device__ __forceinline__ void copy_queries(const TileRegs<HD, DS, NT>& t, const float* lds, const Lds& L,
                                             const Window& w, const float* scales, float* y0,
                                             size_t y_qstride, int tid) {
    if constexpr (HH < HPW) {
        using GC = TileGeo<HD, DS, NT, EBC>;
        const HeadView hv = head_view<InT>(L, HH, w.cap, w.T);
        float rs[GC::NI];
#pragma unroll
        for (int r = 0; r < GC::NI; ++r)
            rs[r] = MX ? e8m0_to_f32(mx_scale_byte<HD, DS, NT, EBC>(lds, L, HH, r, tid)) : scales ? scales[HH] : 1.0f;
        if (tid < GC::ACTIVE)
            queries_and_outputs<HD, DS, NT, InT, EBC, HH * GC::NV, F16>(t, lds, L, hv, w, rs,
                                                                  y0 ? y0 + HH * HD : nullptr, y_qstride, tid);
        copy_queries<HD, DS, NT, InT, EBC, HPW, MX, F16, HH + 1>(t, lds, L, w, scales, y0, y_qstride, tid);
    }
}

// The read-copy tiles of HPW heads (consecutive, tile_bytes apart) into the
// register array, head hh in vectors hh * NV ..
template <int HD, int DS, int NT, int EB, int HPW, int HH = 0>
__device__ __forceinline__ void load_heads(TileRegs<HD, DS, NT>& t, const uint8_t* cp, size_t tile_bytes, int tid) {
    if constexpr (HH < HPW) {
        t.template load<EB, HH * TileGeo<HD, DS, NT, EB>::NV>(cp + HH * tile_bytes, tid);
        load_heads<HD, DS, NT, EB, HPW, HH + 1>(t, cp, tile_bytes, tid);
    }
}

// Step 5 for HPW heads' MXFP4 tiles (one 32-column block per thread and
// head, in vector hh of the register array), head after head so that only one
// head's sums and addresses are live.  gfx950's fp4 converter decodes two
// codes per instruction and applies the block's E8M0 scale (its operand must
// be a power of two: the converter takes only the exponent of that operand,
// so d_q is applied to the sum afterwards).  A block whose scale byte is 255
// (NaN) gives its row a NaN.  The decode is repeated per query rather than
// kept decoded in registers across queries.  Each sum then gets its record
// terms and is reduced over the W lanes of its row.
template <int HD, int DS, int NT, typename InT, int HPW>
__device__ __forceinline__ void mx_queries(const TileRegs<HD, DS, NT>& t, const float* lds, const Lds& L,
                                           const Window& w, float* y0, size_t y_qstride, int tid) {
    using G = TileGeo<HD, DS, NT, 0>;
    static_assert(G::NV == 1 && G::NI == 1, "one block per thread and head");
    typedef float f2 __attribute__((ext_vector_type(2)));
    const int j = tid % G::W;
    const int row = G::row0(tid);
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
        const HeadView hv = head_view<InT>(L, hh, w.cap, w.T);
        const uint32_t e = mx_scale_byte<HD, DS, NT, 0>(lds, L, hh, 0, tid);
        const v4u words = __builtin_bit_cast(v4u, t.raw[hh]);
        const float bs = e == 255u ? 1.0f : e8m0_to_f32(e);
        for (int q = 0; q < w.T; ++q) {
            float sq = bs;
            asm volatile("" : "+v"(sq));     // decode per query, not hoisted into registers
            float acc = 0.f;
            if constexpr (InTraits<InT>::EPV == 8) {
                // bf16 inputs: the converter writes two codes as a bf16 pair (times the
                // block scale, exact), and one v_dot2c_f32_bf16 takes the pair with
                // the matching pair of C (bf16 as staged)
                const uint4* cp = reinterpret_cast<const uint4*>(reinterpret_cast<const uint32_t*>(lds + L.Cb) +
                                                                 q * DS / 2 + j * 16);
                const uint32_t cwd[4] = {words.x, words.y, words.z, words.w};
#pragma unroll
                for (int wq = 0; wq < 4; ++wq) {                  // code word wq: columns 8 wq .. 8 wq + 7
                    const uint4 c = cp[wq];
                    acc = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cwd[wq], sq, 0), c.x, acc);
                    acc = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cwd[wq], sq, 1), c.y, acc);
                    acc = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cwd[wq], sq, 2), c.z, acc);
                    acc = dot2_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cwd[wq], sq, 3), c.w, acc);
                }
            } else {
                const float* cq = lds + L.Cq + q * DS + j * 32;
#pragma unroll
                for (int ch = 0; ch < 8; ++ch) {
                    const float4 c = *reinterpret_cast<const float4*>(cq + 4 * ch);
                    f2 lo, hi;
                    if (ch % 2 == 0) {
                        lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(words[ch / 2], sq, 0);
                        hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(words[ch / 2], sq, 1);
                    } else {
                        lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(words[ch / 2], sq, 2);
                        hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(words[ch / 2], sq, 3);
                    }
                    acc = fmaf(lo[0], c.x, acc);
                    acc = fmaf(lo[1], c.y, acc);
                    acc = fmaf(hi[0], c.z, acc);
                    acc = fmaf(hi[1], c.w, acc);
                    if (ch % 2 == 1) __builtin_amdgcn_sched_barrier(0);   // two chunks of C live at a time
                }
            }
            acc = e == 255u ? __builtin_nanf("") : acc * lds[hv.DQ + q];
            const int m = w.n + q;
            for (int cc = w.first + j; cc <= m; cc += G::W) {
                float xv[1];
                load_x<InT, 1>(lds, hv.X, cc * L.XS + row, xv);
                acc = fmaf(lds[hv.CO + q * w.cap + cc], xv[0], acc);
            }
            acc = group_sum<G::W>(acc);
            if (j == 0 && y0) y0[hh * HD + q * y_qstride + row] = acc;
        }
    }
}

// The FP32 registers of checkpoint tile `tile`: an fp32 checkpoint (CK = 4)
// as stored, an FP16 one (CK = 2) read 8 bytes per fp32 vector position and
// widened (exactly).
template <int HD, int DS, int NT, int CK>
__device__ __forceinline__ void load_ckpt(TileRegs<HD, DS, NT>& t, const void* ckpt, size_t tile, int tid) {
    using G32 = TileGeo<HD, DS, NT, 4>;
    if constexpr (CK == 4) {
        t.template load<4>(static_cast<const float*>(ckpt) + tile * HD * DS, tid);
    } else {
        if (G32::ACTIVE < NT && tid >= G32::ACTIVE) return;
        const v2u* base = static_cast<const v2u*>(ckpt) + tile * (HD * DS / 4);
#pragma unroll
        for (int s = 0; s < G32::NV; ++s) {                 // the fp16 bits in the vector's first half
            const v2u w = __builtin_nontemporal_load(base + G32::vec(tid, s));
            t.raw[s].x = __uint_as_float(w.x);
            t.raw[s].y = __uint_as_float(w.y);
        }
#pragma unroll
        for (int s = 0; s < G32::NV; ++s) {                 // widened in place
            const uint32_t w0 = __float_as_uint(t.raw[s].x), w1 = __float_as_uint(t.raw[s].y);
            t.raw[s] = v4f{f16lo_to_f32(w0), f16hi_to_f32(w0), f16lo_to_f32(w1), f16hi_to_f32(w1)};
        }
    }
}

// Write the folded tile f back: fp32 as is, or FP16 with stochastic rounding
// (random draws keyed by the call's seed and the vectors' indices in the whole
// checkpoint).
template <int HD, int DS, int NT, int CK>
__device__ __forceinline__ void store_ckpt(void* ckpt, size_t tile, const v4f* f, uint64_t seed, int tid) {
    using G32 = TileGeo<HD, DS, NT, 4>;
    if constexpr (CK == 4) {
        v4f* out = static_cast<v4f*>(ckpt) + tile * (HD * DS / 4);
#pragma unroll
        for (int s = 0; s < G32::NV; ++s) __builtin_nontemporal_store(f[s], out + G32::vec(tid, s));
    } else {
        store_f16_sr<G32>(static_cast<uint64_t*>(ckpt) + tile * (HD * DS / 4), tile * (HD * DS / 4), f, seed, tid);
    }
}

// Small batches: the launch is bound by its chain of dependent loads (ring
// pointer, then the records it locates, then the tile), not by bytes.  The
// eager variant (FP32 reads, one head per workgroup) issues, before the ring
// pointer has arrived, the loads of every slot of the head's and group's
// rings, of the call's tokens, of dt and of the FP32 tile; once the pointer
// is known each thread routes its vectors to their window rows in LDS (a ring
// slot s holds window position (s - start) mod cap, used if below n) and
// appends the tokens' records.  It reads cap instead of n records, which
// costs nothing where latency, not bandwidth, sets the time.
constexpr int kEagerJobs = 4;   // 16-byte vectors per thread

template <int NT>
struct EagerRegs {
    uint4 v[kEagerJobs];
    float dt;
};

// Vectors of the eager list: x ring (cap x VR), B ring (cap x VS), then the
// tokens' x (T x VR), B and C (T x VS each).
__host__ __device__ inline int eager_count(int cap, int T, int VR, int VS) {
    return cap * (VR + VS) + T * (VR + 2 * VS);
}

// Where a workgroup's call stands once its ring pointers are checked.
struct WgCtx {
    size_t tile0;           // tile of the first head
    int b, h0, g, hpg;      // sequence, first head, group, heads per group
    int start, n_stored, n; // ring start, records stored, records counted (with a fused commit)
    bool flush_call;
};

// Steps 1-6 of a decode / verify / flush call for one workgroup; FOLD: the call
// folds its window into the checkpoint (and rewrites the read copy); CK: the
// checkpoint's element bytes (4: FP32; 2: FP16 written with stochastic rounding).
template <int HD, int DS, int NT, typename InT, int RM, int HPW, int CK, bool FOLD, bool EAGER>
__device__ __forceinline__ void replay_body(const ReplayArgs& a, const WgCtx& ctx, float* lds,
                                            TileRegs<HD, DS, NT>& treg, const EagerRegs<NT>& er) {
    using G32 = TileGeo<HD, DS, NT, 4>;
    // read-tile element bytes (0: fp4); READ_F16 reads the FP16 checkpoint itself
    constexpr int EBC = RM == READ_MXFP4 ? 0 : (RM == READ_BF16 || RM == READ_F16) ? 2 : 1;
    static_assert(CK == 4 || CK == 2, "checkpoint element bytes");
    static_assert(CK == 2 ? (RM == READ_F16 || RM == READ_MXFP4) : RM != READ_F16,
                  "an FP16 checkpoint is read directly or through an MXFP4 copy");
    using GC = TileGeo<HD, DS, NT, EBC>;
    constexpr size_t CB = EBC ? (size_t)HD * DS * EBC : (size_t)HD * DS / 2;   // read-copy tile bytes
    constexpr int EPVIN = InTraits<InT>::EPV;
    constexpr int VR = HD / EPVIN;                   // 16-byte vectors per x row
    constexpr int VS = DS / EPVIN;                   // 16-byte vectors per B/C row
    constexpr int NW = NT / 64;
    // staged vectors per thread issued up front: 4 on the non-folding calls of the
    // 4-head MX workgroups (whose windows of x rows for four heads exceed two
    // vectors a thread from about half a window on), 2 elsewhere (more spill)
    constexpr int JOBS = !FOLD && HPW >= 4 && (RM == READ_MXFP4 || RM == READ_MXFP8) ? 4 : 2;
    static_assert(HPW == 1 || (RM != READ_F32 && HPW * GC::NV <= G32::NV && GC::ACTIVE == NT),
                  "several heads per workgroup only for read copies that fill the register array");
    static_assert(HPW * NW <= kRedSlots, "reduction slots");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int cap = a.cap;
    const int T = a.T;
    const size_t tile0 = ctx.tile0;
    const int b = ctx.b, h0 = ctx.h0, g = ctx.g, hpg = ctx.hpg;
    const int start = ctx.start, n_stored = ctx.n_stored, n = ctx.n;
    const bool flush_call = ctx.flush_call;
    constexpr bool fold = FOLD;
    const int first = fold ? n : 0;  // first window index of the outputs
    const bool append = !flush_call;
    const int rows = n + T;          // window rows staged in LDS

    constexpr bool MX = RM == READ_MXFP4 || RM == READ_MXFP8;
    constexpr int MXB = MX ? HD * DS / 32 : 0;       // MX scale bytes per head tile
    const Lds L = lds_plan(HD, DS, cap, T, HPW, sizeof(InT), MXB);
    float Ah[HPW], Dh[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
        Ah[hh] = a.A[h0 + hh];
        Dh[hh] = a.D[h0 + hh];
    }

    // ---- 1/2. record loads, then the tile stream, then LDS staging --------------
    const InT* bx = reinterpret_cast<const InT*>(a.buf_x) + tile0 * cap * HD;
    const InT* bB = reinterpret_cast<const InT*>(a.buf_B) + ((size_t)b * a.ngroups + g) * cap * DS;
    const InT* xt = reinterpret_cast<const InT*>(a.x);
    const InT* Bt = reinterpret_cast<const InT*>(a.B);
    const InT* Ct = reinterpret_cast<const InT*>(a.C);
    const bool writer = h0 == g * hpg;             // the group's first head
    const int nx = HPW * rows * VR, nb = rows * VS, nc = T * VS;
    const int ns = fold ? 0 : HPW * MXB / 16;        // the copy's scale bytes, 16 per vector
    const int nv = nx + nb + nc + ns;

    const StageMap sm{bx, bB, xt, Bt, Ct, start, n, cap, T, b, h0, g, a.nheads, a.ngroups,
                      nx, nb, rows, L.X, L.XS, L.K, L.Cq, append, append && writer,
                      reinterpret_cast<const uint8_t*>(a.ckpt_scale) + tile0 * MXB, nc, L.SC};
  if constexpr (EAGER) {
    static_assert(RM == READ_F32 && CK == 4 && HPW == 1, "eager loads: FP32 reads, one head");
    // route the preloaded vectors (see EagerRegs) to their window rows
    const int nring = cap * (VR + VS);
    const int ne = eager_count(cap, T, VR, VS);
    uint4* xring = reinterpret_cast<uint4*>(const_cast<InT*>(bx));
    uint4* Bring = reinterpret_cast<uint4*>(const_cast<InT*>(bB));
#pragma unroll
    for (int j = 0; j < kEagerJobs; ++j) {
        const int v = tid + j * NT;
        if (v >= ne) continue;
        int dst = -1;
        bool wide = false;
        uint4* app = nullptr;
        if (v < cap * VR) {                                     // x ring slot s
            const int s = v / VR, cv = v - s * VR;
            const int c = s - start < 0 ? s - start + cap : s - start;
            if (c < n) dst = L.X * 4 + (c * L.XS + cv * EPVIN) * (int)sizeof(InT);
        } else if (v < nring) {                                 // B ring slot s
            const int u = v - cap * VR;
            const int s = u / VS, cv = u - s * VS;
            const int c = s - start < 0 ? s - start + cap : s - start;
            if (c < n) dst = L.K * 4 + (c * DS + cv * EPVIN) * (int)sizeof(InT);
        } else if (v < nring + T * VR) {                        // x of query q
            const int u = v - nring;
            const int q = u / VR, cv = u - q * VR;
            dst = L.X * 4 + ((n + q) * L.XS + cv * EPVIN) * (int)sizeof(InT);
            if (append) app = xring + ring_slot(start, n + q, cap) * VR + cv;
        } else if (v < nring + T * (VR + VS)) {                 // B of query q
            const int u = v - nring - T * VR;
            const int q = u / VS, cv = u - q * VS;
            dst = L.K * 4 + ((n + q) * DS + cv * EPVIN) * (int)sizeof(InT);
            if (append && writer) app = Bring + ring_slot(start, n + q, cap) * VS + cv;
        } else {                                                // C of query q
            const int u = v - nring - T * (VR + VS);
            const int q = u / VS, cv = u - q * VS;
            dst = (L.Cq + q * DS + cv * EPVIN) * 4;
            wide = true;
        }
        if (app) *app = er.v[j];
        if (dst >= 0) stage_store<InT>(lds, StageJob{nullptr, nullptr, dst, wide}, er.v[j], L);
    }
    if (tid < cap + T) {
        float* const bdt = a.buf_dt + tile0 * cap;
        const float d = er.dt;
        int c;                                                  // window row, or past them
        if (tid < cap) {                                        // ring slot tid: a committed record?
            c = tid - start < 0 ? tid - start + cap : tid - start;
            c = c < n ? c : rows;
        } else {                                                // the token of query tid - cap
            c = n + tid - cap;
            if (append) bdt[ring_slot(start, c, cap)] = d;
        }
        if (c < rows) {
            lds[L.DT + c] = d;
            lds[L.AA + c] = d * Ah[0];
        }
    }
  } else {
    uint4 jv[JOBS];
#pragma unroll
    for (int j = 0; j < JOBS; ++j) {
        const int v = tid + j * NT;
        if (v < nv) jv[j] = *stage_job<HD, DS, InT, HPW>(sm, v).src;
    }
    // dt of (head hh, window row c) for t = hh * rows + c: from the ring for
    // committed records, from the tokens (and appended to the ring) for queries.
    float* const bdt0 = a.buf_dt + tile0 * cap;
    float dtv = 0.f;
    if (tid < HPW * rows) {
        const int hh = block_of<HPW>(tid, rows), c = tid - hh * rows;
        dtv = c < n ? bdt0[hh * cap + ring_slot(start, c, cap)]
                    : a.dt[(size_t)(b * T + (c - n)) * a.nheads + h0 + hh];
    }

    // The tile this call streams: FP32 when it flushes or has no read copy,
    // else the read copies of the workgroup's heads.  A flushing call with
    // several heads starts the first head's FP32 tile here and streams the
    // others in step 4.
    if constexpr (FOLD) {
        load_ckpt<HD, DS, NT, CK>(treg, a.ckpt, tile0, tid);
    } else if constexpr (RM == READ_F32) {
        treg.template load<4>(a.ckpt + tile0 * HD * DS, tid);
    } else {
        const void* src = RM == READ_F16 ? static_cast<const void*>(a.ckpt) : a.ckpt_read;
        load_heads<HD, DS, NT, EBC, HPW>(treg, static_cast<const uint8_t*>(src) + tile0 * CB, CB, tid);
    }

#pragma unroll
    for (int j = 0; j < JOBS; ++j) {
        const int v = tid + j * NT;
        if (v < nv) {
            const StageJob jb = stage_job<HD, DS, InT, HPW>(sm, v);
            if (jb.app) *jb.app = jv[j];
            stage_store<InT>(lds, jb, jv[j], L);
        }
    }
    for (int v = tid + JOBS * NT; v < nv; v += NT) {   // windows too long for JOBS vectors a thread
        const StageJob jb = stage_job<HD, DS, InT, HPW>(sm, v);
        const uint4 val = *jb.src;
        if (jb.app) *jb.app = val;
        stage_store<InT>(lds, jb, val, L);
    }
    for (int t = tid; t < HPW * rows; t += NT) {
        const int hh = block_of<HPW>(t, rows), c = t - hh * rows;
        float d = dtv;
        if (t >= NT)                                        // windows longer than the workgroup
            d = c < n ? bdt0[hh * cap + ring_slot(start, c, cap)]
                      : a.dt[(size_t)(b * T + (c - n)) * a.nheads + h0 + hh];
        if (append && c >= n) bdt0[hh * cap + ring_slot(start, c, cap)] = d;
        float ah = Ah[0];
#pragma unroll
        for (int k = 1; k < HPW; ++k) ah = hh == k ? Ah[k] : ah;
        lds[L.DT + hh * cap + c] = d;
        lds[L.AA + hh * cap + c] = d * ah;
    }
  }
    __syncthreads();

    // ---- 3. coefficients: one 8-lane group per (query, record) pair ---------------
    // Pairs (q, c), c = first .. m_q, give co[h][q][c] for every head h of the
    // workgroup (the score B_c . C_q is the group's, formed once); when the
    // call folds, the n pairs (T, c), c < n, give the flush weights.  The
    // group's lanes split the score and each head's segment sum of a over
    // (c, m], and reduce them.
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
            float sc = 0.f;
            if (q < T) {
                // (fp32 FMAs: v_dot2c_f32_bf16 on the bf16 B and C rows measured slower here)
                for (int j4 = sub; j4 < DS / 4; j4 += 8) {
                    const float4 kb = load_b4<InT, DS>(lds, L.K, c, 4 * j4);
                    const float4 cq = *reinterpret_cast<const float4*>(lds + L.Cq + q * DS + 4 * j4);
                    sc = fmaf(kb.x, cq.x, sc);
                    sc = fmaf(kb.y, cq.y, sc);
                    sc = fmaf(kb.z, cq.z, sc);
                    sc = fmaf(kb.w, cq.w, sc);
                }
                sc = group_sum<8>(sc);
            }
#pragma unroll
            for (int hh = 0; hh < HPW; ++hh) {
                const HeadView hv = head_view<InT>(L, hh, cap, T);
                float seg = 0.f;
                for (int i = c + 1 + sub; i <= m; i += 8) seg += lds[hv.AA + i];
                seg = group_sum<8>(seg);
                if (sub == 0) {
                    const float wgt = lds[hv.DT + c] * expf(seg);
                    if (q < T) {
                        lds[hv.CO + q * cap + c] = fmaf(wgt, sc, c == m ? Dh[hh] : 0.f);
                        if (c == first) lds[hv.DQ + q] = expf(seg + lds[hv.AA + c]);
                    } else {
                        lds[hv.WF + c] = wgt;
                        if (c == 0) lds[hv.DQ + T] = expf(seg + lds[hv.AA + 0]);
                    }
                }
            }
        }
    }
    __syncthreads();

    // ---- 4/5. flush in registers, then queries and outputs --------------------------
    const Window win{n, first, T, cap};
    const float kOnes[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};   // FP32 tile: no row scales
    float* y0 = a.y ? a.y + ((size_t)b * T * a.nheads + h0) * HD : nullptr;
    const size_t y_qstride = (size_t)a.nheads * HD;
    if (fold) {
        const bool active = tid < G32::ACTIVE;
        const int j = tid % G32::W;
        const int row0 = G32::row0(tid);
#pragma unroll 1
        for (int hh = 0; hh < HPW; ++hh) {                   // one head's FP32 tile at a time
            const HeadView hv = head_view<InT>(L, hh, cap, T);
            const size_t tile = tile0 + hh;
            if (HPW > 1 && hh > 0) load_ckpt<HD, DS, NT, CK>(treg, a.ckpt, tile, tid);
            v4f* f = treg.raw;                                // the tile, updated in place
            float amax = 0.f;
            if (active) {
                if (n > 0) {
                    const float df = lds[hv.DQ + T];
#pragma unroll
                    for (int s = 0; s < G32::NV; ++s) f[s] *= df;
                    for (int c = 0; c < n; ++c) {
                        const float wf = lds[hv.WF + c];
                        float xs[G32::NI];
                        load_x<InT, G32::NI>(lds, hv.X, c * L.XS + row0, xs);
#pragma unroll
                        for (int r = 0; r < G32::NI; ++r) xs[r] *= wf;
#pragma unroll
                        for (int k = 0; k < G32::VPL; ++k) {
                            const float4 kb =
                                load_b4<InT, DS>(lds, L.K, c, (j + G32::W * k) * 4);
#pragma unroll
                            for (int r = 0; r < G32::NI; ++r) {
                                v4f& fv = f[r * G32::VPL + k];
                                fv.x = fmaf(xs[r], kb.x, fv.x);
                                fv.y = fmaf(xs[r], kb.y, fv.y);
                                fv.z = fmaf(xs[r], kb.z, fv.z);
                                fv.w = fmaf(xs[r], kb.w, fv.w);
                            }
                        }
                    }
                    store_ckpt<HD, DS, NT, CK>(a.ckpt, tile, f, a.sr_seed, tid);
                }
                if constexpr (RM == READ_BF16) {
                    uint2* out =
                        reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.ckpt_read) + tile * HD * DS);
#pragma unroll
                    for (int s = 0; s < G32::NV; ++s)
                        out[G32::vec(tid, s)] =
                            make_uint2(f32x2_to_bf16x2(f[s].x, f[s].y), f32x2_to_bf16x2(f[s].z, f[s].w));
                }
                if constexpr (RM == READ_E4M3) {
#pragma unroll
                    for (int s = 0; s < G32::NV; ++s)
#pragma unroll
                        for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fabsf(f[s][e]));
                }
                if constexpr (MX) {
                    // Block k of row r (32 columns) is vector k of that row on the 8
                    // lanes of the row group: its largest magnitude and NaN flag are
                    // reduced over those lanes, then each lane encodes its 4 values
                    // (v / X, nearest even) into 16 bits (E2M1, saturating at 6) or
                    // 32 bits (e4m3; the MXFP8 scale leaves nothing to saturate).
                    uint8_t* out = reinterpret_cast<uint8_t*>(a.ckpt_read) + tile * CB;
                    uint8_t* sc_out = reinterpret_cast<uint8_t*>(a.ckpt_scale) + tile * (HD * DS / 32);
                    const int jr = tid % G32::W;
                    // largest |v| of each block as fp32 bits: a NaN (bits above those of
                    // infinity) wins the unsigned maximum, so one reduction also finds NaNs
                    uint32_t mb[G32::NV];
#pragma unroll
                    for (int s = 0; s < G32::NV; ++s) {
                        const v4u u = __builtin_bit_cast(v4u, f[s]) & 0x7FFFFFFFu;
                        mb[s] = max(max(u.x, u.y), max(u.z, u.w));
                    }
#pragma unroll
                    for (int s = 0; s < G32::NV; ++s) mb[s] = group_umax<G32::W>(mb[s]);
                    // vector s of a thread is block s % VPL of its row s / VPL; the
                    // scale bytes of a row's DS / 32 blocks are adjacent, and lane 0 of
                    // the row group stores them in one write per row
                    static_assert(G32::VPL * 32 == DS && (G32::VPL == 2 || G32::VPL == 4), "blocks per row");
                    uint32_t packed[G32::NI] = {};
#pragma unroll
                    for (int s = 0; s < G32::NV; ++s) {
                        const bool nan = mb[s] > 0x7F800000u;
                        const v4f fv = f[s];
                        uint32_t e;
                        if constexpr (RM == READ_MXFP4) {
                            e = mx_block_scale(__uint_as_float(mb[s]), nan);
                            const float X = e == 255u ? 1.0f : e8m0_to_f32(e);
                            uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, fv.x, fv.y, X, 0);
                            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, fv.z, fv.w, X, 1);
                            reinterpret_cast<uint16_t*>(out)[G32::vec(tid, s)] = (uint16_t)w;   // 4 columns = 2 bytes
                        } else {
                            e = mx8_block_scale(__uint_as_float(mb[s]), nan);
                            const float inv = e == 255u ? 1.0f : e8m0_to_f32(254u - e);        // 1 / X, exact
                            reinterpret_cast<uint32_t*>(out)[G32::vec(tid, s)] =
                                f32x4_to_e4m3(fv.x * inv, fv.y * inv, fv.z * inv, fv.w * inv);
                        }
                        packed[s / G32::VPL] |= e << (8 * (s % G32::VPL));
                    }
                    if (jr == 0) {
#pragma unroll
                        for (int r = 0; r < G32::NI; ++r) {
                            uint8_t* dst = sc_out + G32::vec(tid, r * G32::VPL) / 8;   // 8 fp32 vectors per block
                            if constexpr (G32::VPL == 4)
                                *reinterpret_cast<uint32_t*>(dst) = packed[r];
                            else
                                *reinterpret_cast<uint16_t*>(dst) = (uint16_t)packed[r];
                        }
                    }
                }
            }
            if constexpr (RM == READ_E4M3) {
                amax = group_max<64>(amax);
                if (lane == 0) lds[L.RED + hh * NW + wave] = amax;
                __syncthreads();
                amax = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) amax = fmaxf(amax, lds[L.RED + hh * NW + w]);
                const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
                const float inv = 1.0f / sc;
                if (active) {
                    uint32_t* out =
                        reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(a.ckpt_read) + tile * HD * DS);
#pragma unroll
                    for (int s = 0; s < G32::NV; ++s)
                        out[G32::vec(tid, s)] = f32x4_to_e4m3(f[s].x * inv, f[s].y * inv, f[s].z * inv, f[s].w * inv);
                }
                if (tid == 0) a.ckpt_scale[tile] = sc;
            }
            if (active && T > 0)
                queries_and_outputs<HD, DS, NT, InT, 4>(treg, lds, L, hv, win, kOnes, y0 ? y0 + hh * HD : nullptr,
                                                        y_qstride, tid);
        }
    } else if constexpr (RM == READ_F32) {
        if (tid < G32::ACTIVE)
            queries_and_outputs<HD, DS, NT, InT, 4>(treg, lds, L, head_view<InT>(L, 0, cap, T), win, kOnes, y0,
                                                    y_qstride, tid);
    } else if constexpr (RM == READ_MXFP4) {
        mx_queries<HD, DS, NT, InT, HPW>(treg, lds, L, win, y0, y_qstride, tid);
    } else {
        float scales[HPW];
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) scales[hh] = RM == READ_E4M3 ? a.ckpt_scale[tile0 + hh] : 1.0f;
        copy_queries<HD, DS, NT, InT, EBC, HPW, MX, RM == READ_F16>(treg, lds, L, win, scales, y0, y_qstride, tid);
    }

    // ---- 6. advance the heads' ring pointers -----------------------------------------
    // (the pair the prologue checked the reference copy against)
    const int wrapped = start + n >= cap ? start + n - cap : start + n;
    const RingPtr after{fold && n > 0 ? wrapped : start, (fold ? 0 : n) + (a.mode == MODE_DECODE ? 1 : 0)};
    if (!(after == RingPtr{start, n_stored}) && tid < HPW) store_ring_ptr(a.meta, tile0 + tid, after);
}

// Waves per SIMD: 8 (64 VGPRs), except for the MXFP4 kernels, whose flush
// encodes and whose query loop decodes several heads' blocks: with bf16
// inputs (codes decoded to bf16 pairs) 7 over an FP32 checkpoint and 6 over
// an FP16 one; with fp32 inputs (codes decoded to fp32) 5.  Fewer would spill.
template <int RM, typename InT, int CK>
constexpr int replay_waves() {
    return RM == READ_MXFP8 ? 7 : RM != READ_MXFP4 ? 8 : InTraits<InT>::EPV != 8 ? 5 : CK == 4 ? 7 : 6;
}

template <int HD, int DS, int NT, typename InT, int RM, int HPW, int CK, bool EAGER>
__global__ __launch_bounds__(NT, (EAGER ? 2 : replay_waves<RM, InT, CK>())) void replay_kernel(const ReplayArgs a) {
    extern __shared__ float lds[];

    const int chunks = a.nheads / HPW;
    const int nwg = a.batch * chunks;
    const int wg = xcd_remap(blockIdx.x, nwg);
    // sequence, first head of this workgroup, heads per group and group: by
    // shifts where the head counts are powers of two, else by divisions
    constexpr int LH = HPW == 4 ? 2 : HPW == 2 ? 1 : 0;
    int b, h0, hpg, g;
    if (a.nheads_log2 >= LH && a.hpg_log2 >= 0) {
        const int cl = a.nheads_log2 - LH;
        b = wg >> cl;
        h0 = (wg - (b << cl)) * HPW;
        hpg = 1 << a.hpg_log2;
        g = h0 >> a.hpg_log2;
    } else {
        b = wg / chunks;
        h0 = (wg - b * chunks) * HPW;
        hpg = a.nheads / a.ngroups;
        g = h0 / hpg;
    }
    const int tid = threadIdx.x;
    const int cap = a.cap;
    const int T = a.T;
    const size_t tile0 = (size_t)b * a.nheads + h0;

    TileRegs<HD, DS, NT> treg;
    EagerRegs<NT> er;
    if constexpr (EAGER) {
        // every slot of the rings, the tokens, dt and the FP32 tile, before the pointer
        constexpr int EPVIN = InTraits<InT>::EPV;
        constexpr int VR = HD / EPVIN, VS = DS / EPVIN;
        const int ne = eager_count(cap, T, VR, VS), nring = cap * (VR + VS);
        const uint4* xring = reinterpret_cast<const uint4*>(static_cast<const InT*>(a.buf_x) + tile0 * cap * HD);
        const uint4* Bring =
            reinterpret_cast<const uint4*>(static_cast<const InT*>(a.buf_B) + ((size_t)b * a.ngroups + g) * cap * DS);
#pragma unroll
        for (int j = 0; j < kEagerJobs; ++j) {
            const int v = tid + j * NT;
            if (v >= ne) continue;
            const uint4* src;
            if (v < cap * VR) {
                src = xring + v;
            } else if (v < nring) {
                src = Bring + (v - cap * VR);
            } else if (v < nring + T * VR) {
                const int u = v - nring, q = u / VR;
                src = reinterpret_cast<const uint4*>(a.x) + ((size_t)(b * T + q) * a.nheads + h0) * VR + (u - q * VR);
            } else if (v < nring + T * (VR + VS)) {
                const int u = v - nring - T * VR, q = u / VS;
                src = reinterpret_cast<const uint4*>(a.B) + ((size_t)(b * T + q) * a.ngroups + g) * VS + (u - q * VS);
            } else {
                const int u = v - nring - T * (VR + VS), q = u / VS;
                src = reinterpret_cast<const uint4*>(a.C) + ((size_t)(b * T + q) * a.ngroups + g) * VS + (u - q * VS);
            }
            er.v[j] = *src;
        }
        er.dt = tid < cap ? a.buf_dt[tile0 * cap + tid]
                          : tid < cap + T ? a.dt[(size_t)(b * T + tid - cap) * a.nheads + h0] : 0.f;
        treg.template load<4>(a.ckpt + tile0 * HD * DS, tid);
    }

    // Every head keeps its own copy of the ring pointer; those of a workgroup's
    // heads must agree with each other and with the copy of the sequence's
    // first head (read as it stands before or after this launch rewrites it).
    RingPtr cp[HPW];                                  // the copies of the workgroup's heads
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) cp[hh] = load_ring_ptr(a.meta, tile0 + hh);
    const RingPtr own = cp[0];
    const RingPtr ref = load_ring_ptr(a.meta, (size_t)b * a.nheads);
    // fused commit of the previous verification: len += accepted_prev[b]
    const int acc_prev = a.accepted_prev ? a.accepted_prev[b] : 0;
    // every load in flight together: the reference is needed only after the
    // flush decision, and issued after it the latencies would add up
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) asm volatile("" ::"s"(cp[hh].start), "s"(cp[hh].n));
    asm volatile("" ::"s"(ref.start), "s"(ref.n), "s"(acc_prev));
    const int start = own.start;
    const int n_stored = own.n;
    bool same = true;
#pragma unroll
    for (int hh = 1; hh < HPW; ++hh) same = same && cp[hh] == own;
    const bool acc_ok = !a.accepted_prev ||
                        (acc_prev >= 0 && acc_prev <= a.T_prev && n_stored >= 0 && n_stored + acc_prev <= cap);
    const int n = n_stored + acc_prev;
    const bool flush_call = a.mode == MODE_FLUSH;
    const bool cast_only = flush_call && n == 0 && (a.flags & kFlushForceCast) && RM != READ_F32 && RM != READ_F16;
    const bool fold = flush_call ? (n > 0 || cast_only) : (n >= a.L);
    // the pointer this call leaves: past the folded records, and the decode token committed
    // (start + n < 2 cap for every pointer that passes the checks below)
    const int wrapped = start + n >= cap ? start + n - cap : start + n;
    const RingPtr after{fold && n > 0 ? wrapped : start, (fold ? 0 : n) + (a.mode == MODE_DECODE ? 1 : 0)};
    const bool agree = h0 == 0 || ring_ptr_agrees(ref, own, after);

    if (!(same && agree && acc_ok && start >= 0 && start < cap && n >= 0 && n + T <= cap)) {
        if (tid == 0 && a.status) atomicOr(a.status, (int)(acc_ok ? kStatusMeta : kStatusAccept));
        for (int o = tid; o < HPW * T * HD; o += NT) {
            const int hh = o / (T * HD), r = o - hh * T * HD;
            const int q = r / HD, i = r - q * HD;
            a.y[((size_t)(b * T + q) * a.nheads + h0 + hh) * HD + i] = __builtin_nanf("");
        }
        return;
    }

    if (flush_call && !fold) return;
    // One body per case, so that the registers of the FP32 tile a flush holds
    // are not kept live across the read-copy path.
    const WgCtx ctx{tile0, b, h0, g, hpg, start, n_stored, n, flush_call};
    if (fold)
        replay_body<HD, DS, NT, InT, RM, HPW, CK, true, EAGER>(a, ctx, lds, treg, er);
    else
        replay_body<HD, DS, NT, InT, RM, HPW, CK, false, EAGER>(a, ctx, lds, treg, er);
}

// MX scale bytes per head tile staged in LDS by the MX read modes.
constexpr int mx_bytes(int hd, int ds, int read_mode) {
    return read_mode == READ_MXFP4 || read_mode == READ_MXFP8 ? hd * ds / 32 : 0;
}

inline int threads_for(int hd, int ds) {
    if (hd == 16 && ds == 16) return ShapeNT<16, 16>::NT;
    if (hd == 64 && ds == 64) return ShapeNT<64, 64>::NT;
    if (hd == 64 && ds == 128) return ShapeNT<64, 128>::NT;
    return ShapeNT<128, 128>::NT;
}

// Heads per workgroup: the read-copy modes serve several heads of one group
// per workgroup (so each streams as many bytes as one FP32 tile and the heads
// share the group's B/C staging and scores) when the heads of a group split
// evenly and the workgroup's LDS stays within 64 KiB; flush-only calls and
// the FP32 mode use one head.
inline int heads_per_wg(int hd, int ds, int nheads, int ngroups, int cap, int T, int read_mode, int mode,
                        int xbytes) {
    // (the launchers fall back to fewer heads where a shape's copy tile does not
    // leave room in the register array for this many)
    if (read_mode == READ_F32 || mode == MODE_FLUSH || hd == 16) return 1;
    const int want = read_mode == READ_BF16 || read_mode == READ_F16 ? 2 : 4;
    const int hpg = nheads / ngroups;
    for (int hpw = want; hpw > 1; hpw /= 2)
        if (hpg % hpw == 0 && (size_t)lds_plan(hd, ds, cap, T, hpw, xbytes, mx_bytes(hd, ds, read_mode)).total *
                                      sizeof(float) <= 65536 &&
            hpw * (threads_for(hd, ds) / 64) <= kRedSlots)
            return hpw;
    return 1;
}

template <int HD, int DS, typename InT, int RM, int HPW, int CK>
hipError_t launch_one(const ReplayArgs& a, hipStream_t stream) {
    constexpr int NT = ShapeNT<HD, DS>::NT;
    const int nwg = a.batch * (a.nheads / HPW);
    const size_t lds =
        (size_t)lds_plan(HD, DS, a.cap, a.T, HPW, sizeof(InT), mx_bytes(HD, DS, RM)).total * sizeof(float);
    if constexpr (RM == READ_F32 && CK == 4 && HPW == 1) {
        // small batches (fewer workgroups than two per compute unit): the eager variant,
        // with twice the threads (each holding half the tile registers and half the
        // staged vectors), where its vectors fit kEagerJobs per thread
        constexpr int EPVIN = InTraits<InT>::EPV;
        if (nwg <= 512 && eager_count(a.cap, a.T, HD / EPVIN, DS / EPVIN) <= kEagerJobs * 2 * NT &&
            a.cap + a.T <= 2 * NT && a.mode != MODE_FLUSH) {
            hipLaunchKernelGGL((replay_kernel<HD, DS, 2 * NT, InT, RM, HPW, CK, true>), dim3(nwg), dim3(2 * NT), lds,
                               stream, a);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((replay_kernel<HD, DS, NT, InT, RM, HPW, CK, false>), dim3(nwg), dim3(NT), lds, stream, a);
    return hipGetLastError();
}


// Read-copy launch with hpw heads per workgroup; the multi-head kernels are
// compiled only where a copy tile leaves room for them (not 16 x 16).
template <int HD, int DS, int RM, int HPW>
constexpr bool multi_head_fits() {
    using GC = TileGeo<HD, DS, ShapeNT<HD, DS>::NT, RM == READ_BF16 || RM == READ_F16 ? 2 : RM == READ_MXFP4 ? 0 : 1>;
    return HD != 16 && HPW * GC::NV <= TileGeo<HD, DS, ShapeNT<HD, DS>::NT, 4>::NV &&
           GC::ACTIVE == ShapeNT<HD, DS>::NT;
}

template <int HD, int DS, typename InT, int RM, int CK>
hipError_t launch_copy(const ReplayArgs& a, int hpw, hipStream_t stream) {
    if constexpr (RM != READ_BF16 && RM != READ_F16 && multi_head_fits<HD, DS, RM, 4>())
        if (hpw >= 4) return launch_one<HD, DS, InT, RM, 4, CK>(a, stream);
    if constexpr (multi_head_fits<HD, DS, RM, 2>())
        if (hpw >= 2) return launch_one<HD, DS, InT, RM, 2, CK>(a, stream);
    return launch_one<HD, DS, InT, RM, 1, CK>(a, stream);
}

// CK: checkpoint element bytes.  An FP32 checkpoint is read as is or through
// any copy; an FP16 one directly (READ_F16) or through an MXFP4 copy (with the
// per-tile e4m3 or the MXFP8 copy its flush does not fit 64 VGPRs).
template <int HD, int DS, typename InT, int CK>
hipError_t launch_type(const ReplayArgs& a, int read_mode, int hpw, hipStream_t stream) {
    switch (read_mode) {
        case READ_F32:
            if constexpr (CK == 4) return launch_one<HD, DS, InT, READ_F32, 1, CK>(a, stream);
            return hipErrorInvalidValue;
        case READ_BF16:
            if constexpr (CK == 4) return launch_copy<HD, DS, InT, READ_BF16, CK>(a, hpw, stream);
            return hipErrorInvalidValue;
        case READ_F16:
            if constexpr (CK == 2) return launch_copy<HD, DS, InT, READ_F16, CK>(a, hpw, stream);
            return hipErrorInvalidValue;
        case READ_E4M3:
            if constexpr (CK == 4) return launch_copy<HD, DS, InT, READ_E4M3, CK>(a, hpw, stream);
            return hipErrorInvalidValue;
        case READ_MXFP4:
            if constexpr (DS % 32 == 0) return launch_copy<HD, DS, InT, READ_MXFP4, CK>(a, hpw, stream);
            return hipErrorInvalidValue;
        case READ_MXFP8:
            if constexpr (CK == 4 && DS % 32 == 0) return launch_copy<HD, DS, InT, READ_MXFP8, CK>(a, hpw, stream);
            return hipErrorInvalidValue;
    }
    return hipErrorInvalidValue;
}

template <int HD, int DS, int CK>
hipError_t launch_shape(const ReplayArgs& a, int in_type, int read_mode, hipStream_t stream) {
    const int hpw = heads_per_wg(HD, DS, a.nheads, a.ngroups, a.cap, a.T, read_mode, a.mode,
                                 in_type == IN_F32 ? 4 : 2);
    if (in_type == IN_F32) return launch_type<HD, DS, float, CK>(a, read_mode, hpw, stream);
    return launch_type<HD, DS, uint16_t, CK>(a, read_mode, hpw, stream);
}

// Every compiled shape for checkpoint element bytes CK.
template <int CK>
hipError_t launch_ck(const ReplayArgs& a, int hd, int ds, int in_type, int read_mode, hipStream_t stream) {
    if (hd == 16 && ds == 16) return launch_shape<16, 16, CK>(a, in_type, read_mode, stream);
    if (hd == 64 && ds == 64) return launch_shape<64, 64, CK>(a, in_type, read_mode, stream);
    if (hd == 64 && ds == 128) return launch_shape<64, 128, CK>(a, in_type, read_mode, stream);
    if (hd == 128 && ds == 128) return launch_shape<128, 128, CK>(a, in_type, read_mode, stream);
    return hipErrorInvalidValue;
}

}  // namespace
}  // namespace rssm
