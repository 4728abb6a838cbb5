// The non-causal 8-wave forward instantiation (the dense long-sequence case),
// compiled on its own so that build.py can give it the machine scheduler that
// suits it: LLVM's iterative ILP strategy measured 2 % faster on this kernel
// (7.44 vs 7.60 ms on the 8 x 32 x 8192 x 128 workload) and 3 % slower on the
// causal one, which stays in attn_fwd_bf16.hip with the default scheduler.
// Only this file instantiates kernel<D, false, 8, 64>.
#define ATTN_FWD_BF16_NO_DEFAULT_LAUNCHER
#include "attn_fwd_bf16.hip"

namespace attn {

hipError_t launch_fwd_bf16_dense8(const FwdArgs &a, hipStream_t s) {
    if (a.d == 128) return fwd_bf16::launch<128, false, 8, 64>(a, s);
    return fwd_bf16::launch<64, false, 8, 64>(a, s);
}

}  // namespace attn
