// fwd_vl_bf16_n16.hip -- instantiates the forward launchers (packed variable-length sequences) for: bf16_t N=16
#include "kernels.hpp"

namespace ssm {
template int launch_fwd_flags<bf16_t, 16, true, true>(const FwdArgs<bf16_t>&, int64_t, bool,
                                                  bool, hipStream_t);
}  // namespace ssm
