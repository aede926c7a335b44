// Kernel instantiations for the layernorm operator (fp32 and bf16).
#include "instantiate.hpp"

namespace credit {

void register_layernorm_kernels(std::vector<KernelEntry> &out)
{
    register_op_dtype<kLayerNorm, float, 0>(out);
    register_op_dtype<kLayerNorm, bf16_t, 1>(out);
}

}  // namespace credit
