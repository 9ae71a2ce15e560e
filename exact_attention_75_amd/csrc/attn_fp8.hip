// attn_fp8.hip -- placeholder until the fp8 kernels land.
#include "kernels.h"
namespace attn {
int fwd_fp8_block_m() { return 128; }
hipError_t launch_fwd_fp8(const Fp8FwdParams&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_prepass(const PrepassParams&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace attn
