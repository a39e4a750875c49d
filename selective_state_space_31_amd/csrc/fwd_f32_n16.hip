// fwd_f32_n16.hip -- instantiates the forward launchers ((batch, seqlen) layout) for: float N=16
#include "kernels.hpp"

namespace ssm {
template int launch_fwd_flags<float, 16, true, false>(const FwdArgs<float>&, int64_t, bool,
                                                  bool, hipStream_t);
}  // namespace ssm
