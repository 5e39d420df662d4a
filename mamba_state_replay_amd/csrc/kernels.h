// Host-side launch interface between api.cpp (argument checks) and the
// kernel files.  Internal to the library; not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rssm {

enum Mode : int32_t { MODE_DECODE = 0, MODE_VERIFY = 1, MODE_FLUSH = 2 };
enum InType : int32_t { IN_F32 = 0, IN_BF16 = 1 };
// READ_F16: the FP16 checkpoint read directly (no copy).
enum ReadMode : int32_t { READ_F32 = 0, READ_BF16 = 1, READ_E4M3 = 2, READ_MXFP4 = 3, READ_MXFP8 = 4, READ_F16 = 5 };

constexpr uint32_t kStatusMeta = 1u;
constexpr uint32_t kStatusAccept = 2u;
constexpr uint32_t kStatusSlot = 4u;
constexpr int32_t kFlushForceCast = 1;

struct ReplayArgs {
    float* ckpt;        // fp32, or fp16 bits when ckpt16
    void* ckpt_read;
    float* ckpt_scale;
    void* buf_x;
    void* buf_B;
    float* buf_dt;
    int32_t* meta;      // [batch][nheads][2]
    int32_t* status;
    const void* x;
    const void* B;
    const void* C;
    const float* dt;
    const float* A;
    const float* D;
    float* y;
    const int32_t* accepted_prev;   // fused commit of the previous verification, or null
    int32_t batch, nheads, ngroups;
    int32_t L, cap, T, T_prev;
    int32_t mode, flags;
    int32_t ckpt16;     // the checkpoint is FP16, written with stochastic rounding
    int32_t nheads_log2, hpg_log2;   // log2 of nheads and of nheads / ngroups where they are
                                     // powers of two (else -1): the kernel then shifts, not divides
    uint64_t sr_seed;   // key of the rounding's random words for this call
};

struct ConvArgs {
    float* states;
    const int32_t* slot;
    int32_t* status;
    const void* x;
    const void* B;
    const void* C;
    const float* dt;
    const float* A;
    const float* D;
    float* y;
    int32_t batch, nheads, ngroups, nslots, T;
};

struct CommitArgs {
    int32_t* meta;      // replay: [batch][nheads][2]
    int32_t* slot;      // conventional: [batch]
    const int32_t* accepted;
    int32_t* status;
    int32_t batch, nheads, T, cap, nslots;
};

// Dynamic LDS bytes of the replay kernel for a shape, ring capacity and T.
size_t replay_lds_bytes(int hd, int ds, int cap, int T, int in_bytes);
size_t conventional_lds_bytes(int hd, int ds, int T);

// Each returns hipSuccess or the launch error; -1 cast to hipError_t never
// happens because api.cpp only passes shapes that replay_shape_supported accepts.
bool shape_supported(int hd, int ds);
hipError_t launch_replay(const ReplayArgs& a, int hd, int ds, int in_type, int read_mode,
                         hipStream_t stream);
hipError_t launch_replay_f16(const ReplayArgs& a, int hd, int ds, int in_type, int read_mode, hipStream_t stream);
hipError_t launch_conventional(const ConvArgs& a, int hd, int ds, int in_type, hipStream_t stream);
hipError_t launch_replay_commit(const CommitArgs& a, hipStream_t stream);
hipError_t launch_conventional_commit(const CommitArgs& a, hipStream_t stream);

// Gated DeltaNet layer (gdn.hip): one workgroup per (sequence, value head,
// row block of ROWS value rows).
struct GdnArgs {
    float* ckpt;        // [batch][nv][dv][dk] fp32, or fp16 bits (ckpt16); or the conventional states
    void* buf_k;        // [batch][nk][cap][dk] input type
    float* buf_u;       // [batch][nv][cap][dv]
    float* buf_g;       // [batch][nv][cap]
    int32_t* meta;      // [batch][nv][parts][2]
    int32_t* status;
    const void* q;      // [batch][T][nk][dk]
    const void* k;
    const void* v;      // [batch][T][nv][dv]
    const float* g;     // [batch][T][nv]
    const float* beta;
    float* o;           // [batch][T][nv][dv]
    const int32_t* accepted_prev;   // fused commit of the previous verification, or null
    int32_t T_prev;
    const int32_t* slot;   // conventional with snapshots: current slot per sequence, or null
    int32_t nslots;        // conventional: state slots per sequence (1: in place)
    int32_t batch, nv, nk, dv, parts;
    int32_t L, cap, T, mode;
    int32_t ckpt16;     // FP16 checkpoint written with stochastic rounding
    int32_t parts_log2, nv_log2, hpk_log2;   // log2 of parts, nv and nv / nk where they are powers
                                             // of two (else -1): the kernels then shift, not divide
    uint64_t sr_seed;
};

bool gdn_shape_supported(int dk, int dv);
int gdn_rows(int dk);   // value rows per workgroup
size_t gdn_lds_bytes(int dk, int cap, int T);
hipError_t launch_gdn_replay(const GdnArgs& a, int dk, int in_type, hipStream_t stream);   // a.ckpt16 selects the FP16 kernel
hipError_t launch_gdn_conventional(const GdnArgs& a, int dk, int in_type, hipStream_t stream);

}  // namespace rssm
