// Kernel instantiations for the rmsnorm operator (fp32 and bf16).
#include "instantiate.hpp"

namespace credit {

void register_rmsnorm_kernels(std::vector<KernelEntry> &out)
{
    register_op_dtype<kRmsNorm, float, 0>(out);
    register_op_dtype<kRmsNorm, bf16_t, 1>(out);
}

}  // namespace credit
