// fwd_bf16_n16.hip -- instantiates the forward launchers ((batch, seqlen) layout) for: bf16_t N=16; also the backward's recomputation of the chunk-entering states (exact widths)
#include "kernels.hpp"

namespace ssm {
template int launch_fwd_flags<bf16_t, 16, true, false>(const FwdArgs<bf16_t>&, int64_t, bool,
                                                  bool, hipStream_t);
template int launch_fwd_states<bf16_t, 16, true>(const FwdArgs<bf16_t>&, int64_t, bool, hipStream_t);
}  // namespace ssm
