// Kernel instantiations for the softmax operator (fp32 and bf16).
#include "instantiate.hpp"

namespace credit {

void register_softmax_kernels(std::vector<KernelEntry> &out)
{
    register_op_dtype<kSoftmax, float, 0>(out);
    register_op_dtype<kSoftmax, bf16_t, 1>(out);
}

}  // namespace credit
