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
#include "replay_impl.h"

namespace rssm {

size_t replay_lds_bytes(int hd, int ds, int cap, int T, int in_bytes) {
    // one head per workgroup, with room for MX scale bytes (an upper bound for every read mode)
    return (size_t)lds_plan(hd, ds, cap, T, 1, in_bytes, hd * ds / 32).total * sizeof(float);
}

bool shape_supported(int hd, int ds) {
    return (hd == 16 && ds == 16) || (hd == 64 && ds == 64) || (hd == 64 && ds == 128) ||
           (hd == 128 && ds == 128);
}

hipError_t launch_replay(const ReplayArgs& a, int hd, int ds, int in_type, int read_mode,
                         hipStream_t stream) {
    if (a.ckpt16) return launch_replay_f16(a, hd, ds, in_type, read_mode, stream);
    return launch_ck<4>(a, hd, ds, in_type, read_mode, stream);
}

}  // namespace rssm
