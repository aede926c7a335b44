// Kernel instantiations for LayerNorm backward (row part) (fp32 and bf16).
#include "instantiate.hpp"

namespace credit {

void register_layernorm_bwd_kernels(std::vector<KernelEntry> &out)
{
    register_op_dtype<kLayerNormBwd, float, 0>(out);
    register_op_dtype<kLayerNormBwd, bf16_t, 1>(out);
}

}  // namespace credit
