// fwd_vl_bf16_small.hip -- instantiates the forward launchers (packed variable-length sequences) for: bf16_t N=4, bf16_t N=8, bf16_t N=4 (padded), bf16_t N=16 (padded)
#include "kernels.hpp"

namespace ssm {
template int launch_fwd_flags<bf16_t, 4, true, true>(const FwdArgs<bf16_t>&, int64_t, bool,
                                                  bool, hipStream_t);
template int launch_fwd_flags<bf16_t, 8, true, true>(const FwdArgs<bf16_t>&, int64_t, bool,
                                                  bool, hipStream_t);
template int launch_fwd_flags<bf16_t, 4, false, true>(const FwdArgs<bf16_t>&, int64_t, bool,
                                                  bool, hipStream_t);
template int launch_fwd_flags<bf16_t, 16, false, true>(const FwdArgs<bf16_t>&, int64_t, bool,
                                                  bool, hipStream_t);
}  // namespace ssm
