// Conventional Mamba-2 decode step, the in-library baseline (gfx950).
//
// NVIDIA Developer blog "ReplaySSM: Rethinking State Storage for Faster
// Hybrid-Model Decoding", section "Why SSM layers can become a decoding
// bottleneck": every step loads the state from HBM, decays it, adds the
// rank-1 update, reads the output with C and stores the state back.  With T
// drafts (section "Rollback for speculative decoding") the state is read once
// and one snapshot is written per draft, so that any accepted prefix can be
// picked afterwards.
//
// One workgroup per (sequence, head) tile, the same streaming layout as the
// replay kernel (TileGeo): each thread holds NI rows x VPL 16-byte vectors of
// the tile in registers, updates them in place for every token, writes them
// out, and reduces the output rows across the W lanes of each row.
#include "common.h"
#include "kernels.h"

namespace rssm {

namespace {

struct ConvLds {
    int X, B, C, DEC, DTS, U, total;
};

__host__ __device__ inline ConvLds conv_plan(int HD, int DS, int T) {
    ConvLds l;
    int o = 0;
    l.X = o;   o += T * HD;
    l.B = o;   o += T * DS;
    l.C = o;   o += T * DS;
    l.DEC = o; o += T;      // exp(dt_q A)
    l.DTS = o; o += T;      // dt_q
    l.U = o;   o += T * HD;
    o = (o + 3) & ~3;
    l.total = o;
    return l;
}

template <int HD, int DS, int NT, typename InT>
__global__ __launch_bounds__(NT) void conventional_kernel(const ConvArgs a) {
    extern __shared__ float lds[];
    using G = TileGeo<HD, DS, NT, 4>;
    constexpr int EPVIN = InTraits<InT>::EPV;

    const int nwg = a.batch * a.nheads;
    const int wg = xcd_remap(blockIdx.x, nwg);
    const int b = wg / a.nheads;
    const int h = wg - b * a.nheads;
    const int g = h / (a.nheads / a.ngroups);
    const int tid = threadIdx.x;
    const int T = a.T;
    const int nslots = a.nslots;

    const int s0 = nslots > 1 ? a.slot[b] : 0;
    if (s0 < 0 || s0 >= nslots) {
        if (tid == 0 && h == 0 && a.status) atomicOr(a.status, (int)kStatusSlot);
        for (int o = tid; o < T * HD; o += NT) {
            const int q = o / HD, i = o - q * HD;
            a.y[((size_t)(b * T + q) * a.nheads + h) * HD + i] = __builtin_nanf("");
        }
        return;
    }
    const size_t tile_elems = (size_t)HD * DS;
    auto state_ptr = [&](int slot) {
        return a.states + (((size_t)b * nslots + slot) * a.nheads + h) * tile_elems;
    };

    // Issue the tile loads first; the token staging below overlaps them.
    const int j = tid % G::W;
    const int row0 = G::row0(tid);
    const bool active = tid < G::ACTIVE;
    v4f f[G::NV];
    if (active) {
        const v4f* src = reinterpret_cast<const v4f*>(state_ptr(s0));
#pragma unroll
        for (int s = 0; s < G::NV; ++s) f[s] = __builtin_nontemporal_load(src + G::vec(tid, s));
    }

    const ConvLds L = conv_plan(HD, DS, T);
    {
        const InT* xt = reinterpret_cast<const InT*>(a.x);
        constexpr int VR = HD / EPVIN;
        for (int v = tid; v < T * VR; v += NT) {
            const int q = v / VR, cv = v - q * VR;
            const uint4 val = *(reinterpret_cast<const uint4*>(xt + ((size_t)(b * T + q) * a.nheads + h) * HD) + cv);
            widen16<InT>(val, lds + L.X + q * HD + cv * EPVIN);
        }
        const InT* Bt = reinterpret_cast<const InT*>(a.B);
        const InT* Ct = reinterpret_cast<const InT*>(a.C);
        constexpr int VS = DS / EPVIN;
        for (int v = tid; v < T * VS; v += NT) {
            const int q = v / VS, cv = v - q * VS;
            const size_t off = ((size_t)(b * T + q) * a.ngroups + g) * DS;
            widen16<InT>(*(reinterpret_cast<const uint4*>(Bt + off) + cv), lds + L.B + q * DS + cv * EPVIN);
            widen16<InT>(*(reinterpret_cast<const uint4*>(Ct + off) + cv), lds + L.C + q * DS + cv * EPVIN);
        }
        if (tid < T) {
            const float d = a.dt[(size_t)(b * T + tid) * a.nheads + h];
            lds[L.DTS + tid] = d;
            lds[L.DEC + tid] = expf(d * a.A[h]);
        }
    }
    __syncthreads();

    if (active) {
        const int lane = tid & 63;
        for (int q = 0; q < T; ++q) {
            const float dec = lds[L.DEC + q];
            const float dtq = lds[L.DTS + q];
            float v[16];
#pragma unroll
            for (int r = 0; r < G::NI; ++r) v[r] = 0.f;
#pragma unroll
            for (int k = 0; k < G::VPL; ++k) {
                const int col = (j + G::W * k) * 4;
                const float4 bv = *reinterpret_cast<const float4*>(lds + L.B + q * DS + col);
                const float4 cv = *reinterpret_cast<const float4*>(lds + L.C + q * DS + col);
#pragma unroll
                for (int r = 0; r < G::NI; ++r) {
                    const float xs = dtq * lds[L.X + q * HD + row0 + r];
                    v4f& fv = f[r * G::VPL + k];
                    fv.x = fmaf(dec, fv.x, xs * bv.x);
                    fv.y = fmaf(dec, fv.y, xs * bv.y);
                    fv.z = fmaf(dec, fv.z, xs * bv.z);
                    fv.w = fmaf(dec, fv.w, xs * bv.w);
                    v[r] = fmaf(fv.x, cv.x, fmaf(fv.y, cv.y, fmaf(fv.z, cv.z, fmaf(fv.w, cv.w, v[r]))));
                }
            }
            const int dst = nslots == 1 ? 0 : (s0 + 1 + q) % nslots;
            v4f* out = reinterpret_cast<v4f*>(state_ptr(dst));
#pragma unroll
            for (int s = 0; s < G::NV; ++s) __builtin_nontemporal_store(f[s], out + G::vec(tid, s));
            int idx;
            const float u = transpose_reduce<G::NI, G::W>(v, lane, idx);
            if ((lane % G::W) < G::NI) lds[L.U + q * HD + row0 + idx] = u;
        }
    }
    __syncthreads();

    const float Dh = a.D[h];
    for (int o = tid; o < T * HD; o += NT) {
        const int q = o / HD, i = o - q * HD;
        a.y[((size_t)(b * T + q) * a.nheads + h) * HD + i] =
            fmaf(Dh, lds[L.X + q * HD + i], lds[L.U + q * HD + i]);
    }
}

template <int HD, int DS>
hipError_t conv_shape(const ConvArgs& a, int in_type, hipStream_t stream) {
    constexpr int NT = ShapeNT<HD, DS>::NT;
    const size_t lds = (size_t)conv_plan(HD, DS, a.T).total * sizeof(float);
    const int nwg = a.batch * a.nheads;
    if (in_type == IN_F32)
        hipLaunchKernelGGL((conventional_kernel<HD, DS, NT, float>), dim3(nwg), dim3(NT), lds, stream, a);
    else
        hipLaunchKernelGGL((conventional_kernel<HD, DS, NT, uint16_t>), dim3(nwg), dim3(NT), lds, stream, a);
    return hipGetLastError();
}

// Commit kernels.  Replay: one thread per (sequence, head) copy of the ring
// pointer (nheads = copies per sequence), each checked against the sequence's
// first copy as that copy stands before or after its own thread commits;
// conventional: one thread per sequence.
__global__ void replay_commit_kernel(const CommitArgs a) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= a.batch * a.nheads) return;
    const int b = t / a.nheads;
    const int acc = a.accepted[b];
    const RingPtr own = load_ring_ptr(a.meta, t);
    const RingPtr after{own.start, own.n + acc};
    if (t != b * a.nheads && !ring_ptr_agrees(load_ring_ptr(a.meta, (size_t)b * a.nheads), own, after)) {
        if (a.status) atomicOr(a.status, (int)kStatusMeta);
        return;
    }
    if (acc < 0 || acc > a.T || own.n < 0 || own.n + acc > a.cap) {
        if (a.status) atomicOr(a.status, (int)kStatusAccept);
        return;
    }
    store_ring_ptr(a.meta, t, after);
}

__global__ void conventional_commit_kernel(const CommitArgs a) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= a.batch) return;
    const int acc = a.accepted[b];
    const int s = a.slot[b];
    if (acc < 0 || acc > a.T || s < 0 || s >= a.nslots) {
        if (a.status) atomicOr(a.status, (int)kStatusAccept);
        return;
    }
    a.slot[b] = (s + acc) % a.nslots;
}

}  // namespace

size_t conventional_lds_bytes(int hd, int ds, int T) {
    return (size_t)conv_plan(hd, ds, T).total * sizeof(float);
}

hipError_t launch_conventional(const ConvArgs& a, int hd, int ds, int in_type, hipStream_t stream) {
    if (hd == 16 && ds == 16) return conv_shape<16, 16>(a, in_type, stream);
    if (hd == 64 && ds == 64) return conv_shape<64, 64>(a, in_type, stream);
    if (hd == 64 && ds == 128) return conv_shape<64, 128>(a, in_type, stream);
    if (hd == 128 && ds == 128) return conv_shape<128, 128>(a, in_type, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_replay_commit(const CommitArgs& a, hipStream_t stream) {
    const int n = a.batch * a.nheads;
    hipLaunchKernelGGL(replay_commit_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_conventional_commit(const CommitArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(conventional_commit_kernel, dim3((a.batch + 255) / 256), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace rssm
