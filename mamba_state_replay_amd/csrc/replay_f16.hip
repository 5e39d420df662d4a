// The ReplaySSM kernel instantiated for an FP16 checkpoint written with
// stochastic rounding (kernel templates in replay_impl.h; a translation unit
// of its own so the two checkpoint types compile in parallel).
#include "replay_impl.h"

namespace rssm {

hipError_t launch_replay_f16(const ReplayArgs& a, int hd, int ds, int in_type, int read_mode, hipStream_t stream) {
    return launch_ck<2>(a, hd, ds, in_type, read_mode, stream);
}

}  // namespace rssm
