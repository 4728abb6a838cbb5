// The persistent forward instantiations (persistent_kernel, every head dim,
// causal and not), compiled on their own so that build.py can give them the
// machine scheduler that suits them: LLVM's max-memory-clause strategy
// measured 0.9-1.1 % faster on the causal 1 x 32 x 32768 x 128 workload and
// 0.5 % on 4 x 32 x 2048 x 128, neutral on the dense 8 x 32 x 8192 x 128 one,
// and 1-1.5 % slower on the per-block causal kernels, which stay in
// attn_fwd_bf16.hip with the default scheduler.
#define ATTN_FWD_BF16_NO_DEFAULT_LAUNCHER
#include "attn_fwd_bf16.hip"

namespace attn {

bool launch_fwd_bf16_persistent(const FwdArgs &a, hipStream_t s, hipError_t &err) {
    using namespace fwd_bf16;
    if (a.d == 128) return a.causal ? launch_persistent<128, true>(a, s, err) : launch_persistent<128, false>(a, s, err);
    return a.causal ? launch_persistent<64, true>(a, s, err) : launch_persistent<64, false>(a, s, err);
}

}  // namespace attn
