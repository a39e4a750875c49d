// fwd_bf16_large.hip -- instantiates the forward launchers ((batch, seqlen) layout) for: bf16_t N=32, bf16_t N=64 (padded)
#include "kernels.hpp"

namespace ssm {
template int launch_fwd_flags<bf16_t, 32, true, false>(const FwdArgs<bf16_t>&, int64_t, bool,
                                                  bool, hipStream_t);
template int launch_fwd_flags<bf16_t, 64, false, false>(const FwdArgs<bf16_t>&, int64_t, bool,
                                                  bool, hipStream_t);
}  // namespace ssm
