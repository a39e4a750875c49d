// fwd_f32_small.hip -- instantiates the forward launchers ((batch, seqlen) layout) for: float N=4, float N=8, float N=4 (padded), float N=16 (padded)
#include "kernels.hpp"

namespace ssm {
template int launch_fwd_flags<float, 4, true, false>(const FwdArgs<float>&, int64_t, bool,
                                                  bool, hipStream_t);
template int launch_fwd_flags<float, 8, true, false>(const FwdArgs<float>&, int64_t, bool,
                                                  bool, hipStream_t);
template int launch_fwd_flags<float, 4, false, false>(const FwdArgs<float>&, int64_t, bool,
                                                  bool, hipStream_t);
template int launch_fwd_flags<float, 16, false, false>(const FwdArgs<float>&, int64_t, bool,
                                                  bool, hipStream_t);
}  // namespace ssm
