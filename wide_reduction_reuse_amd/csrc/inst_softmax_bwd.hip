// Kernel instantiations for Softmax-logits backward (fp32 and bf16).
#include "instantiate.hpp"

namespace credit {

void register_softmax_bwd_kernels(std::vector<KernelEntry> &out)
{
    register_op_dtype<kSoftmaxBwd, float, 0>(out);
    register_op_dtype<kSoftmaxBwd, bf16_t, 1>(out);
}

}  // namespace credit
