// fwd_f32_large.hip -- instantiates the forward launchers ((batch, seqlen) layout) for: float N=32, float N=64 (padded)
#include "kernels.hpp"

namespace ssm {
template int launch_fwd_flags<float, 32, true, false>(const FwdArgs<float>&, int64_t, bool,
                                                  bool, hipStream_t);
template int launch_fwd_flags<float, 64, false, false>(const FwdArgs<float>&, int64_t, bool,
                                                  bool, hipStream_t);
}  // namespace ssm
