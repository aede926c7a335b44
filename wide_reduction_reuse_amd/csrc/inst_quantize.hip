// Kernel instantiations for int8 quantization (fp32 and bf16).
#include "instantiate.hpp"

namespace credit {

void register_quantize_kernels(std::vector<KernelEntry> &out)
{
    register_op_dtype<kQuantInt8, float, 0>(out);
    register_op_dtype<kQuantInt8, bf16_t, 1>(out);
}

}  // namespace credit
