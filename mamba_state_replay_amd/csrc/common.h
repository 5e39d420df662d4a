// Device helpers shared by the ReplaySSM kernels: tile geometry, number
// formats and wave-level reductions for gfx950 (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rssm {

// Native 16-byte vector types (usable with the nontemporal builtins).
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Tile geometry.
//
// A (sequence, head) tile is HD rows x DS columns, row-major, streamed by a
// workgroup of NT threads with 16-byte vector loads.  A row of VPR vectors is
// shared by W consecutive lanes (W = 8 where the row has 8 or more vectors):
// lane j of the row group holds vector columns j, j + W, j + 2W, ... (VPL of
// them), and the group holds NI consecutive rows.  Thread t's vector s is
//     row (t / W) * NI + s / VPL,  vector column t % W + W * (s % VPL),
// so each load instruction (fixed s) of a wave reads whole 128-byte lines,
// and a row's dot product needs a reduction over only W lanes.  EB is the
// element size of the tile's storage type (4 fp32, 2 bf16, 1 e4m3, 0 for
// 4-bit codes, 32 to a vector).
// ---------------------------------------------------------------------------
template <int HD, int DS, int NT, int EB>
struct TileGeo {
    static constexpr int EPV = EB == 0 ? 32 : 16 / EB;   // elements per 16-byte vector (EB 0: fp4)
    static constexpr int VPR = DS / EPV;                 // vectors per row
    static constexpr int W = VPR < 8 ? VPR : 8;          // lanes per row
    static constexpr int VPL = VPR / W;                  // vectors per lane per row
    static constexpr int TV = HD * VPR;                  // vectors per tile
    static constexpr int NV = TV >= NT ? TV / NT : 1;    // vectors per thread
    static constexpr int ACTIVE = TV >= NT ? NT : TV;    // threads that own data
    static constexpr int NI = NV / VPL;                  // rows per thread
    static_assert(DS % EPV == 0 && VPR % W == 0, "row must be whole vectors split evenly over W lanes");
    static_assert((W & (W - 1)) == 0 && W >= 1 && W <= 8, "lanes per row: power of two <= 8");
    static_assert(NI >= 1 && NI * VPL == NV && NV <= 8, "thread share: whole rows, at most 8 vectors");
    static_assert(NI <= W, "transposed reduction needs NI <= W");
    static_assert(ACTIVE * NV == TV, "tile must split evenly over the workgroup");

    __device__ static __forceinline__ int row0(int t) { return (t / W) * NI; }
    // Offset of thread t's vector s from the tile base, in 16-byte vectors.
    __device__ static __forceinline__ int vec(int t, int s) {
        return (row0(t) + s / VPL) * VPR + (t % W) + W * (s % VPL);
    }
};

// ---------------------------------------------------------------------------
// Number formats.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Two fp32 -> two bf16 (low half = a), round to nearest even, with gfx950's
// packed converter (v_cvt_pk_bf16_f32); NaN stays NaN.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Four fp32 -> four OCP e4m3fn codes (low byte = a), round to nearest even,
// saturating: magnitudes above 448 (the largest finite e4m3fn value) are
// clamped to +-448 by a compare and select, which leaves a NaN a NaN (a med3
// clamp would return a bound for it), then converted by gfx950's fp8
// converter.
__device__ __forceinline__ float sat448(float v) {
    return fabsf(v) > 448.0f ? copysignf(448.0f, v) : v;
}

__device__ __forceinline__ uint32_t f32x4_to_e4m3(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(c), sat448(d), w, true);
    return (uint32_t)w;
}

// Four e4m3 codes (bytes of w, low byte first) -> fp32, with the hardware
// converter (gfx950 reads OCP e4m3fn).
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float out[4]) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    out[0] = lo[0];
    out[1] = lo[1];
    out[2] = hi[0];
    out[3] = hi[1];
}

// Two bf16 values packed in a word (low half first), as the operand type of
// gfx950's bf16 dot instruction.  The word goes through a copy: bit-casting an
// element of an ext_vector_type vector straight to the pair type was seen to
// compile to the vector's first element for every index.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t u) {
    bf16x2_t r;
    __builtin_memcpy(&r, &u, 4);
    return r;
}

// c + a.lo * b.lo + a.hi * b.hi with v_dot2c_f32_bf16 (the products of two
// bf16 values are exact in fp32).
__device__ __forceinline__ float dot2_bf16(bf16x2_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, as_bf16x2(b), c, false);
}
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return dot2_bf16(as_bf16x2(a), b, c);
}

// MX block scale (E8M0 byte e: 2^(e - 127), e = 255 NaN) as fp32.
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
    return e == 255u ? __builtin_nanf("") : e == 0u ? __uint_as_float(0x00400000u) : __uint_as_float(e << 23);
}

// E8M0 scale of an MXFP4 block with largest magnitude amax (fp32 bits): the
// block's largest exponent minus 2 (the largest E2M1 exponent), clamped to
// 1 .. 254 so that the scale is a normal fp32 number; 255 if the block holds
// a NaN.
__device__ __forceinline__ uint32_t mx_block_scale(float amax, bool has_nan) {
    const int biased = (int)((__float_as_uint(amax) >> 23) & 0xFF);
    const int e = biased - 2 < 1 ? 1 : biased - 2 > 254 ? 254 : biased - 2;
    return has_nan ? 255u : (uint32_t)e;
}

// E8M0 scale of an MXFP8 (e4m3) block with largest magnitude amax: the
// smallest power of two X with amax / X <= 448, so that no element saturates
// (amax = m 2^E needs X = 2^(E - 8), or 2^(E - 7) when m > 1.75), clamped to
// 1 .. 254; 255 if the block holds a NaN.  An infinite amax gets the scale of
// the largest finite fp32 value.
__device__ __forceinline__ uint32_t mx8_block_scale(float amax, bool has_nan) {
    const uint32_t bits = __float_as_uint(amax);
    const int e0 = (int)((bits >> 23) & 0xFF) - 8 + ((bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    const int e = e0 < 1 ? 1 : e0 > 254 ? 254 : e0;
    return has_nan ? 255u : (uint32_t)e;
}

// ---------------------------------------------------------------------------
// Cross-lane exchange within 32-lane halves: DPP quad permutes for xor 1 and
// xor 2, ds_swizzle (bit-mask mode) for xor 4, 8 and 16.
// ---------------------------------------------------------------------------
template <int MASK>
__device__ __forceinline__ float xor_shfl(float v) {
    const int iv = __float_as_int(v);
    int r;
    if constexpr (MASK == 1) {
        r = __builtin_amdgcn_mov_dpp(iv, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
    } else if constexpr (MASK == 2) {
        r = __builtin_amdgcn_mov_dpp(iv, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
    } else if constexpr (MASK == 4 || MASK == 8 || MASK == 16) {
        r = __builtin_amdgcn_ds_swizzle(iv, (MASK << 10) | 0x1F);
    } else {
        static_assert(MASK == 32, "unsupported lane mask");
        r = __shfl_xor(iv, 32);
    }
    return __int_as_float(r);
}

template <int MASK>
__device__ __forceinline__ float xor_max(float v) {
    return fmaxf(v, xor_shfl<MASK>(v));
}

// Sum v over groups of W consecutive lanes (W a power of two <= 64); every
// lane of a group gets the group's sum.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (W >= 2) v += xor_shfl<1>(v);
    if constexpr (W >= 4) v += xor_shfl<2>(v);
    if constexpr (W >= 8) v += xor_shfl<4>(v);
    if constexpr (W >= 16) v += xor_shfl<8>(v);
    if constexpr (W >= 32) v += xor_shfl<16>(v);
    if constexpr (W >= 64) v += xor_shfl<32>(v);
    return v;
}

// Unsigned maximum over groups of W consecutive lanes (W <= 32).
template <int W>
__device__ __forceinline__ uint32_t group_umax(uint32_t v) {
    if constexpr (W >= 2) v = max(v, __float_as_uint(xor_shfl<1>(__uint_as_float(v))));
    if constexpr (W >= 4) v = max(v, __float_as_uint(xor_shfl<2>(__uint_as_float(v))));
    if constexpr (W >= 8) v = max(v, __float_as_uint(xor_shfl<4>(__uint_as_float(v))));
    if constexpr (W >= 16) v = max(v, __float_as_uint(xor_shfl<8>(__uint_as_float(v))));
    if constexpr (W >= 32) v = max(v, __float_as_uint(xor_shfl<16>(__uint_as_float(v))));
    return v;
}

template <int W>
__device__ __forceinline__ float group_max(float v) {
    if constexpr (W >= 2) v = xor_max<1>(v);
    if constexpr (W >= 4) v = xor_max<2>(v);
    if constexpr (W >= 8) v = xor_max<4>(v);
    if constexpr (W >= 16) v = xor_max<8>(v);
    if constexpr (W >= 32) v = xor_max<16>(v);
    if constexpr (W >= 64) v = xor_max<32>(v);
    return v;
}

// One halving stage of the transposed reduction: lanes whose MASK bit is set
// end with the sums of the upper half of their N values with their partner's,
// the others with the sums of the lower half.  For the DPP masks (1, 2) the
// exchange folds into the add, so both halves are summed and one is kept; for
// the others each lane sends the half it gives away.
template <int MASK, int N>
__device__ __forceinline__ void halve(float (&v)[16], bool upper) {
    constexpr int H = N / 2;
#pragma unroll
    for (int i = 0; i < H; ++i) {
        if constexpr (MASK <= 2) {
            const float lo = v[i] + xor_shfl<MASK>(v[i]);
            const float hi = v[i + H] + xor_shfl<MASK>(v[i + H]);
            v[i] = upper ? hi : lo;
        } else {
            const float keep = upper ? v[i + H] : v[i];
            const float send = upper ? v[i] : v[i + H];
            v[i] = keep + xor_shfl<MASK>(send);
        }
    }
}

// Reduce N values per lane over groups of W consecutive lanes (N <= W, both
// powers of two) with log2(N) halving stages followed by log2(W/N) plain
// butterfly stages.  Returns the sum of value index `idx` over the group;
// lanes with (lane % W) < N hold distinct indices (idx is then lane % W read
// with its bits reversed into the stage order below).
template <int N, int W>
__device__ __forceinline__ float transpose_reduce(float (&v)[16], int lane, int& idx) {
    static_assert(N <= W, "need at least as many lanes as values");
    idx = 0;
    if constexpr (N >= 2) { const bool u = lane & 1; halve<1, N>(v, u); idx += u ? N / 2 : 0; }
    if constexpr (N >= 4) { const bool u = lane & 2; halve<2, N / 2>(v, u); idx += u ? N / 4 : 0; }
    if constexpr (N >= 8) { const bool u = lane & 4; halve<4, N / 4>(v, u); idx += u ? N / 8 : 0; }
    if constexpr (N >= 16) { const bool u = lane & 8; halve<8, N / 8>(v, u); idx += u ? N / 16 : 0; }
    float s = v[0];
    if constexpr (W > N) {
        if constexpr (N <= 1 && W >= 2) s += xor_shfl<1>(s);
        if constexpr (N <= 2 && W >= 4) s += xor_shfl<2>(s);
        if constexpr (N <= 4 && W >= 8) s += xor_shfl<4>(s);
        if constexpr (N <= 8 && W >= 16) s += xor_shfl<8>(s);
        if constexpr (N <= 16 && W >= 32) s += xor_shfl<16>(s);
    }
    return s;
}

// ---------------------------------------------------------------------------
// Ring pointers.  A sequence keeps several copies of its pointer {start, n}
// (one per head, or per workgroup), each read and rewritten only by its owner.
// A copy is one aligned 64-bit word (start in the low half), loaded and stored
// as a single 8-byte access (an s_load_dwordx2 / global_store_dwordx2: the
// memory system performs an aligned 8-byte access whole), so another workgroup
// that reads it while its owner rewrites it sees either the old pair or the new
// one, never a mix of the two.  The loads are plain so that the compiler keeps
// them on the scalar unit, ahead of the tile loads that wait for them.
// ---------------------------------------------------------------------------
struct RingPtr {
    int start, n;
    __device__ __forceinline__ bool operator==(const RingPtr& o) const { return start == o.start && n == o.n; }
};

__device__ __forceinline__ RingPtr load_ring_ptr(const int32_t* meta, size_t copy) {
    const uint64_t w = reinterpret_cast<const uint64_t*>(meta)[copy];
    return RingPtr{(int)(uint32_t)w, (int)(uint32_t)(w >> 32)};
}

__device__ __forceinline__ void store_ring_ptr(int32_t* meta, size_t copy, RingPtr p) {
    reinterpret_cast<uint64_t*>(meta)[copy] = (uint64_t)(uint32_t)p.start | ((uint64_t)(uint32_t)p.n << 32);
}

// Whether a workgroup's copy agrees with the sequence's reference copy (the
// first one), which its owner may rewrite during the same launch: the
// reference must hold the pair this copy holds now or the pair it will hold
// after the call (own_new), which the owner of the reference computes alike.
__device__ __forceinline__ bool ring_ptr_agrees(RingPtr ref, RingPtr own, RingPtr own_new) {
    return ref == own || ref == own_new;
}

// Remap the linear workgroup id so that each of the 8 XCDs (which receive
// workgroups round-robin) processes one contiguous block of tiles; the heads
// of a group then share B/C records through that XCD's L2.
__device__ __forceinline__ int xcd_remap(int wg, int nwg) {
    if ((nwg & 7) != 0) return wg;
    return (wg & 7) * (nwg >> 3) + (wg >> 3);
}

}  // namespace rssm

namespace rssm {

// Threads per workgroup for each compiled tile shape: every thread of the
// large shapes owns 128 bytes of the FP32 tile (8 16-byte vectors).
template <int HD, int DS>
struct ShapeNT;
template <>
struct ShapeNT<16, 16> { static constexpr int NT = 64; };
template <>
struct ShapeNT<64, 64> { static constexpr int NT = 128; };
template <>
struct ShapeNT<64, 128> { static constexpr int NT = 256; };
template <>
struct ShapeNT<128, 128> { static constexpr int NT = 512; };

// Token / record element type: fp32, or bf16 carried as its 16-bit pattern.
template <typename InT>
struct InTraits;
template <>
struct InTraits<float> { static constexpr int EPV = 4; };
template <>
struct InTraits<uint16_t> { static constexpr int EPV = 8; };

// Widen one 16-byte vector of InT elements to fp32.
template <typename InT>
__device__ __forceinline__ void widen16(const uint4 v, float* out) {
    if constexpr (InTraits<InT>::EPV == 4) {
        out[0] = __uint_as_float(v.x);
        out[1] = __uint_as_float(v.y);
        out[2] = __uint_as_float(v.z);
        out[3] = __uint_as_float(v.w);
    } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = __uint_as_float(w[i] << 16);
            out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    }
}


// ---- FP16 checkpoint with stochastic rounding ---------------------------------------

// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): ten rounds of two 32 x 32 -> 64-bit products
// mixing a 128-bit counter under a 64-bit key that is bumped by the Weyl
// constants between rounds; 4 x 32 random bits per (counter, key).
struct U32x4 {
    uint32_t x, y, z, w;
};

__device__ __forceinline__ U32x4 philox4x32_10(U32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        // each 32 x 32 -> 64-bit product as one 64-bit multiply (one v_mad_u64_u32
        // instead of separate low and high multiplies: measured 27% faster)
        const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
        c = U32x4{(uint32_t)(p1 >> 32) ^ c.y ^ k0, (uint32_t)p1, (uint32_t)(p0 >> 32) ^ c.w ^ k1, (uint32_t)p0};
    }
    return c;
}

// fp32 -> fp16 with stochastic rounding: |v| goes to the fp16 value above it
// with probability equal to its distance from the fp16 value below it, in
// units of their spacing, decided by a 13-bit random residue r13: away from
// zero iff distance * 2^13 + r13 >= 2^13 (in the fp16 normal range the
// distance is exactly the 13 fp32 mantissa bits below the fp16 ones; below
// 2^-14 it is the distance truncated to 13 bits).  |v| >= 65504 and
// infinities give +-65504; a NaN stays a NaN.
//
// gfx950's converter v_cvt_sr_f16_f32 rounds away from zero iff the dropped
// fraction of |v| (in units of the fp16 spacing) plus its 32-bit random
// operand / 2^32 reaches 1; with r13 in the operand's top 13 bits and zeros
// below, that is the rule above (checked bit for bit against a software
// implementation of the rule over the normal, subnormal and underflow ranges
// and every special value, and by the library's rounding test).  Where the
// rule saturates the converter gives an infinity (inputs from 65504 up that
// round up, larger ones, infinities): an infinite half becomes +-65504 by
// subtracting one from its bits; a NaN stays a NaN.
//
// Two values to one word of fp16 bits (a in the low half), residues in the low
// 13 bits of ra and rb.
__device__ __forceinline__ uint32_t f32x2_to_f16x2_sr(float a, float b, uint32_t ra, uint32_t rb) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    f16x2 w = {0, 0};
    w = __builtin_amdgcn_cvt_sr_f16_f32(w, a, ra << 19, false);
    w = __builtin_amdgcn_cvt_sr_f16_f32(w, b, rb << 19, true);
    const uint32_t u = __builtin_bit_cast(uint32_t, w);
    const uint32_t lo = (u & 0x7FFFu) == 0x7C00u ? 1u : 0u;
    const uint32_t hi = (u & 0x7FFF0000u) == 0x7C000000u ? 0x10000u : 0u;
    return u - lo - hi;
}

// Random draws of the checkpoint's 4-element vectors (vector index vi,
// row-major over the whole [batch][nheads][headdim][dstate] array): vectors vi
// and vi + 16 of each aligned block of 32 share the Philox4x32-10 call at
// counter (u low, u high, 0, 0), u = 16 (vi / 32) + vi % 16, under the key
// (seed low, seed high); column e of the lower vector takes the low 16 bits
// of word e, the upper vector the high 16 bits.  One call serves 8 values.
__device__ __forceinline__ U32x4 sr_words(uint64_t vi, uint64_t seed) {
    const uint64_t u = (vi >> 5) * 16 + (vi & 15);
    return philox4x32_10(U32x4{(uint32_t)u, (uint32_t)(u >> 32), 0u, 0u}, (uint32_t)seed, (uint32_t)(seed >> 32));
}

__device__ __forceinline__ uint2 f32x4_sr_with(const v4f f, const U32x4 r, int shift) {
    return make_uint2(f32x2_to_f16x2_sr(f.x, f.y, r.x >> shift, r.y >> shift),
                      f32x2_to_f16x2_sr(f.z, f.w, r.z >> shift, r.w >> shift));
}

// One vector to fp16 with stochastic rounding (the half of its call that the
// partner vector uses is dropped).
__device__ __forceinline__ uint2 f32x4_to_f16x4_sr(const v4f f, uint64_t vi, uint64_t seed) {
    return f32x4_sr_with(f, sr_words(vi, seed), (vi & 16) ? 16 : 0);
}

// Vectors vi (vi % 32 < 16) and vi + 16 from one call.
__device__ __forceinline__ void f32x8_to_f16x8_sr(const v4f lo, const v4f hi, uint64_t vi, uint64_t seed,
                                                  uint2& out_lo, uint2& out_hi) {
    const U32x4 r = sr_words(vi, seed);
    out_lo = f32x4_sr_with(lo, r, 0);
    out_hi = f32x4_sr_with(hi, r, 16);
}

// A thread's share of a tile in the TileGeo layout G (vector s at G::vec(t, s),
// tile vectors from index base in the whole checkpoint) written as fp16 with
// stochastic rounding.  Where rows hold 32 vectors (VPL = 4) or 16 (VPL = 2,
// an even number of rows per thread), the thread's vectors s and s + 2 lie 16
// apart in one aligned block of 32 (vector columns j + 8 k and j + 8 k + 16,
// or the same column of an even row and of the next) and share a generator
// call.
template <typename G>
__device__ __forceinline__ void store_f16_sr(uint64_t* out, uint64_t base, const v4f* f, uint64_t seed, int tid) {
    constexpr bool PAIRS = G::W == 8 && ((G::VPR == 32 && G::VPL == 4) || (G::VPR == 16 && G::VPL == 2 && G::NI % 2 == 0));
    if constexpr (PAIRS) {
#pragma unroll
        for (int s = 0; s < G::NV; ++s) {
            if (s & 2) continue;
            uint2 lo, hi;
            f32x8_to_f16x8_sr(f[s], f[s + 2], base + G::vec(tid, s), seed, lo, hi);
            __builtin_nontemporal_store((uint64_t)lo.x | (uint64_t)lo.y << 32, out + G::vec(tid, s));
            __builtin_nontemporal_store((uint64_t)hi.x | (uint64_t)hi.y << 32, out + G::vec(tid, s + 2));
            __builtin_amdgcn_sched_barrier(0);   // one call's random words live at a time
        }
    } else {
#pragma unroll
        for (int s = 0; s < G::NV; ++s) {
            const uint2 h = f32x4_to_f16x4_sr(f[s], base + G::vec(tid, s), seed);
            __builtin_nontemporal_store((uint64_t)h.x | (uint64_t)h.y << 32, out + G::vec(tid, s));
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// fp16 bits (low / high half of a word) to fp32, exact.
__device__ __forceinline__ float f16lo_to_f32(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16hi_to_f32(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

}  // namespace rssm
