// ReplaySSM decode / verify / flush kernel for one Mamba-2 layer (gfx950).
//
// Method: NVIDIA Developer blog "ReplaySSM: Rethinking State Storage for
// Faster Hybrid-Model Decoding".  The state of (sequence b, head h) is an FP32
// checkpoint tile H_s (HD x DS) plus the records (x_k, B_k, dt_k) appended
// since the last flush (section "How ReplaySSM represents the state").
//
// One workgroup per (b, h) tile.  Per call:
//   1. read {start, n} of sequence b; flush first when n >= L (decode/verify)
//      or n > 0 (flush);
//   2. stage the n records and the T query tokens in LDS as fp32, and append
//      the tokens' records to the ring (x and dt by every head, B by the first
//      head of the group);
//   3. decays and weights by backward segment sums (one thread per query), and
//      the group scores s[q][c] = B_c . C_q (one wave per pair);
//   4. stream the tile once with 16-byte loads into registers:
//        flush: H = exp(sum a) H_s + sum_k dt_k exp(sum_{k<i<n} a_i) x_k B_k^T
//               (rank-n update in registers), write it once, cast the read
//               copy (section "Benefit 3": both precisions from the same
//               registers; the copy is never read back into the recurrence);
//        then u_q[i] = sum_j H[i,j] C_q[j] for all T queries from the same
//        registers (section "Benefit 2": the checkpoint is used once for all
//        queries);
//   5. y_q = d_q u_q + sum_{c<=m} w[q][c] s[q][c] x_c + D x_q (output-only
//      evaluation; no intermediate state is formed);
//   6. the last workgroup of the sequence to finish advances {start, n}.
#include "common.h"
#include "kernels.h"

namespace rssm {

namespace {

// LDS plan in floats.
struct Lds {
    int X, K, Cq, DT, W, S, DQ, WF, U, RED, total;
};

__host__ __device__ inline Lds lds_plan(int HD, int DS, int cap, int T) {
    Lds l;
    int o = 0;
    l.X = o;  o += cap * HD;   // x of records then queries, window order
    l.K = o;  o += cap * DS;   // B of records then queries
    l.Cq = o; o += T * DS;     // C of the queries
    l.DT = o; o += cap;        // dt, window order
    l.W = o;  o += T * cap;    // w[q][c] = dt_c exp(sum_{c<i<=m_q} a_i)
    l.S = o;  o += T * cap;    // s[q][c] = B_c . C_q
    l.DQ = o; o += T + 1;      // d_q = exp(sum_{first<=i<=m_q} a_i); [T] = flush decay
    l.WF = o; o += cap;        // flush weights dt_c exp(sum_{c<i<n} a_i)
    l.U = o;  o += T * HD;     // u_q[i] = (H C_q)[i]
    l.RED = o; o += 16;        // cross-wave reductions
    l.total = o;
    return l;
}

// Load this thread's NI rows of a tile stored with element size EB and widen
// them to fp32: f[s][e] is element (row0 + s, colv*EPV + e).
template <int HD, int DS, int NT, int EB>
__device__ __forceinline__ void load_tile(const void* tile, int tid,
                                          float (&f)[TileGeo<HD, DS, NT, EB>::NI]
                                                    [TileGeo<HD, DS, NT, EB>::EPV]) {
    using G = TileGeo<HD, DS, NT, EB>;
    const int colv = tid % G::LPR;
    const int row0 = (tid / G::LPR) * G::NI;
    const v4u* base = reinterpret_cast<const v4u*>(tile);
    v4u raw[G::NI];
#pragma unroll
    for (int s = 0; s < G::NI; ++s)
        raw[s] = __builtin_nontemporal_load(base + (size_t)(row0 + s) * G::LPR + colv);
#pragma unroll
    for (int s = 0; s < G::NI; ++s) {
        const uint32_t w[4] = {raw[s].x, raw[s].y, raw[s].z, raw[s].w};
        if constexpr (EB == 4) {
#pragma unroll
            for (int e = 0; e < 4; ++e) f[s][e] = __uint_as_float(w[e]);
        } else if constexpr (EB == 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[s][2 * e] = __uint_as_float(w[e] << 16);
                f[s][2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) e4m3x4_to_f32(w[e], &f[s][4 * e]);
        }
    }
}

// u_q[row] = scale * sum_j f[row][j] C_q[j] for every query, reduced across
// the LPR lanes of each row group and written to LDS.
template <int HD, int DS, int NT, int EB>
__device__ __forceinline__ void tile_queries(const float (&f)[TileGeo<HD, DS, NT, EB>::NI]
                                                            [TileGeo<HD, DS, NT, EB>::EPV],
                                             const float* lds, float* ldsU, int cq, int T,
                                             int tid, float scale) {
    using G = TileGeo<HD, DS, NT, EB>;
    const int colv = tid % G::LPR;
    const int row0 = (tid / G::LPR) * G::NI;
    const int lane = tid & 63;
    for (int q = 0; q < T; ++q) {
        float c[G::EPV];
        const float4* cp = reinterpret_cast<const float4*>(lds + cq + q * DS + colv * G::EPV);
#pragma unroll
        for (int e = 0; e < G::EPV / 4; ++e) {
            const float4 t = cp[e];
            c[4 * e] = t.x; c[4 * e + 1] = t.y; c[4 * e + 2] = t.z; c[4 * e + 3] = t.w;
        }
        float v[16];
#pragma unroll
        for (int s = 0; s < G::NI; ++s) {
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < G::EPV; ++e) acc = fmaf(f[s][e], c[e], acc);
            v[s] = acc;
        }
        int idx;
        const float u = transpose_reduce<G::NI, G::LPR>(v, lane, idx);
        if ((lane % G::LPR) < G::NI) ldsU[q * HD + row0 + idx] = u * scale;
    }
}

template <int HD, int DS, int NT, typename InT, int RM>
__global__ __launch_bounds__(NT) void replay_kernel(const ReplayArgs a) {
    extern __shared__ float lds[];
    using G32 = TileGeo<HD, DS, NT, 4>;
    constexpr int EPVIN = InTraits<InT>::EPV;
    constexpr int NW = NT / 64;

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

    const int start = a.meta[2 * b];
    const int n = a.meta[2 * b + 1];

    if (!(start >= 0 && start < cap && n >= 0 && n + T <= cap)) {
        if (tid == 0 && h == 0 && a.status) atomicOr(a.status, (int)kStatusMeta);
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

    const Lds L = lds_plan(HD, DS, cap, T);

    // ---- 2. stage records and queries; append the queries' records -------------
    {
        const InT* bx = reinterpret_cast<const InT*>(a.buf_x) + tile * cap * HD;
        const InT* xt = reinterpret_cast<const InT*>(a.x);
        constexpr int VR = HD / EPVIN;
        for (int v = tid; v < (n + T) * VR; v += NT) {
            const int c = v / VR, cv = v - c * VR;
            const int slot = (start + c) % cap;
            uint4 val;
            if (c < n) {
                val = *(reinterpret_cast<const uint4*>(bx + (size_t)slot * HD) + cv);
            } else {
                const int q = c - n;
                val = *(reinterpret_cast<const uint4*>(xt + ((size_t)(b * T + q) * a.nheads + h) * HD) + cv);
                if (append)
                    *(reinterpret_cast<uint4*>(const_cast<InT*>(bx) + (size_t)slot * HD) + cv) = val;
            }
            widen16<InT>(val, lds + L.X + c * HD + cv * EPVIN);
        }
        const InT* bB = reinterpret_cast<const InT*>(a.buf_B) + ((size_t)b * a.ngroups + g) * cap * DS;
        const InT* Bt = reinterpret_cast<const InT*>(a.B);
        const InT* Ct = reinterpret_cast<const InT*>(a.C);
        const bool writer = (h % hpg) == 0;
        constexpr int VS = DS / EPVIN;
        for (int v = tid; v < (n + T) * VS; v += NT) {
            const int c = v / VS, cv = v - c * VS;
            const int slot = (start + c) % cap;
            uint4 val;
            if (c < n) {
                val = *(reinterpret_cast<const uint4*>(bB + (size_t)slot * DS) + cv);
            } else {
                const int q = c - n;
                const size_t off = ((size_t)(b * T + q) * a.ngroups + g) * DS;
                val = *(reinterpret_cast<const uint4*>(Bt + off) + cv);
                if (append && writer)
                    *(reinterpret_cast<uint4*>(const_cast<InT*>(bB) + (size_t)slot * DS) + cv) = val;
                const uint4 cval = *(reinterpret_cast<const uint4*>(Ct + off) + cv);
                widen16<InT>(cval, lds + L.Cq + q * DS + cv * EPVIN);
            }
            widen16<InT>(val, lds + L.K + c * DS + cv * EPVIN);
        }
        float* bdt = a.buf_dt + tile * cap;
        for (int c = tid; c < n + T; c += NT) {
            const int slot = (start + c) % cap;
            float d;
            if (c < n) {
                d = bdt[slot];
            } else {
                d = a.dt[(size_t)(b * T + (c - n)) * a.nheads + h];
                if (append) bdt[slot] = d;
            }
            lds[L.DT + c] = d;
        }
    }
    __syncthreads();

    // ---- 3. decays, weights and scores ------------------------------------------
    const float Ah = a.A[h];
    if (tid < T) {
        // window positions first..m of query q; backward segment sums
        const int q = tid, m = n + q;
        float cum = 0.f;
        for (int c = m; c >= first; --c) {
            const float d = lds[L.DT + c];
            lds[L.W + q * cap + c] = d * expf(cum);
            cum += d * Ah;
        }
        lds[L.DQ + q] = expf(cum);
    }
    if (fold && tid == NT - 1) {
        float cum = 0.f;
        for (int c = n - 1; c >= 0; --c) {
            const float d = lds[L.DT + c];
            lds[L.WF + c] = d * expf(cum);
            cum += d * Ah;
        }
        lds[L.DQ + T] = expf(cum);
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

    // ---- 4. stream the tile --------------------------------------------------------
    if (fold) {
        float f[G32::NI][4];
        const bool active = tid < G32::ACTIVE;
        const int colv = tid % G32::LPR;
        const int row0 = (tid / G32::LPR) * G32::NI;
        float* ck = a.ckpt + tile * HD * DS;
        float amax = 0.f;
        if (active) {
            load_tile<HD, DS, NT, 4>(ck, tid, f);
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
                    const uint32_t lo = f32_to_bf16(f[s][0]) | (f32_to_bf16(f[s][1]) << 16);
                    const uint32_t hi = f32_to_bf16(f[s][2]) | (f32_to_bf16(f[s][3]) << 16);
                    out[(size_t)(row0 + s) * G32::LPR + colv] = make_uint2(lo, hi);
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
                    const uint32_t w = f32_to_e4m3(f[s][0] * inv) | (f32_to_e4m3(f[s][1] * inv) << 8) |
                                       (f32_to_e4m3(f[s][2] * inv) << 16) | (f32_to_e4m3(f[s][3] * inv) << 24);
                    out[(size_t)(row0 + s) * G32::LPR + colv] = w;
                }
            }
            if (tid == 0) a.ckpt_scale[tile] = sc;
        }
        if (active && T > 0) tile_queries<HD, DS, NT, 4>(f, lds, lds + L.U, L.Cq, T, tid, 1.0f);
    } else if constexpr (RM == READ_F32) {
        float f[G32::NI][4];
        if (tid < G32::ACTIVE) {
            load_tile<HD, DS, NT, 4>(a.ckpt + tile * HD * DS, tid, f);
            tile_queries<HD, DS, NT, 4>(f, lds, lds + L.U, L.Cq, T, tid, 1.0f);
        }
    } else if constexpr (RM == READ_BF16) {
        using G = TileGeo<HD, DS, NT, 2>;
        float f[G::NI][G::EPV];
        if (tid < G::ACTIVE) {
            load_tile<HD, DS, NT, 2>(reinterpret_cast<const uint16_t*>(a.ckpt_read) + tile * HD * DS, tid, f);
            tile_queries<HD, DS, NT, 2>(f, lds, lds + L.U, L.Cq, T, tid, 1.0f);
        }
    } else {
        using G = TileGeo<HD, DS, NT, 1>;
        float f[G::NI][G::EPV];
        if (tid < G::ACTIVE) {
            const float sc = a.ckpt_scale[tile];
            load_tile<HD, DS, NT, 1>(reinterpret_cast<const uint8_t*>(a.ckpt_read) + tile * HD * DS, tid, f);
            tile_queries<HD, DS, NT, 1>(f, lds, lds + L.U, L.Cq, T, tid, sc);
        }
    }
    __syncthreads();

    // ---- 5. outputs ------------------------------------------------------------------
    const float Dh = a.D[h];
    for (int o = tid; o < T * HD; o += NT) {
        const int q = o / HD, i = o - q * HD;
        const int m = n + q;
        float acc = lds[L.DQ + q] * lds[L.U + q * HD + i];
        for (int c = first; c <= m; ++c)
            acc = fmaf(lds[L.W + q * cap + c] * lds[L.S + q * cap + c], lds[L.X + c * HD + i], acc);
        acc = fmaf(Dh, lds[L.X + m * HD + i], acc);
        a.y[((size_t)(b * T + q) * a.nheads + h) * HD + i] = acc;
    }

    // ---- 6. advance the sequence's ring pointer (last workgroup of b) ----------------
    const int new_start = fold && n > 0 ? (start + n) % cap : start;
    const int new_n = (fold ? 0 : n) + (a.mode == MODE_DECODE ? 1 : 0);
    if ((new_start != start || new_n != n) && tid == 0) {
        const int old = atomicAdd(a.arrive + b, 1);
        if (old == a.nheads - 1) {
            a.arrive[b] = 0;
            a.meta[2 * b] = new_start;
            a.meta[2 * b + 1] = new_n;
        }
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

size_t replay_lds_bytes(int hd, int ds, int cap, int T) {
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
