// fwd_vl_f32_small.hip -- instantiates the forward launchers (packed variable-length sequences) for: float N=4, float N=8, float N=4 (padded), float N=16 (padded)
#include "kernels.hpp"

namespace ssm {
template int launch_fwd_flags<float, 4, true, true>(const FwdArgs<float>&, int64_t, bool,
                                                  bool, hipStream_t);
template int launch_fwd_flags<float, 8, true, true>(const FwdArgs<float>&, int64_t, bool,
                                                  bool, hipStream_t);
template int launch_fwd_flags<float, 4, false, true>(const FwdArgs<float>&, int64_t, bool,
                                                  bool, hipStream_t);
template int launch_fwd_flags<float, 16, false, true>(const FwdArgs<float>&, int64_t, bool,
                                                  bool, hipStream_t);
}  // namespace ssm
