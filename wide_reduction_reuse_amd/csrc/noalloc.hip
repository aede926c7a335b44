// credit_run_plan_static: credit_run_plan for callers that cannot allocate
// device memory (code under graph capture, tight serving loops).  The only
// device memory the library ever allocates is a split-row exchange scratch;
// this entry point uses the file-scope array `scratch` below instead, one
// copy per GPU, which the module's loader places and zero-fills (the
// protocol's initial state) and which lives until the process ends.
//
// Host code never passes `scratch` itself to the device: in host code the
// name is a host-side stand-in.  The array's address on a device comes from
// hipGetSymbolAddress, taken once per device on the entry point's first call
// there (with that device current), and only that address is used.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "api_internal.hpp"
#include "args.hpp"
#include "credit.h"

namespace credit {
namespace {

static_assert(kScratchBytes % 8 == 0, "the scratch is a whole number of 64-bit words");

// The split-row scratch of this entry point: a SplitCtl, then kSlotWords
// exchange words (kScratchBytes, 1 MiB + 640 bytes), on every GPU.
static __device__ __align__(256) uint64_t scratch[kScratchBytes / 8];

std::mutex g_static_mu;
std::map<int, SplitCtl *> g_static_ptr;  // device -> address of `scratch` there

// The current device's copy of `scratch`, its address taken on first use.
credit_status_t static_scratch(SplitCtl **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return CREDIT_ERR_HIP;
    }
    std::lock_guard<std::mutex> lk(g_static_mu);
    auto it = g_static_ptr.find(dev);
    if (it != g_static_ptr.end()) {
        *out = it->second;
        return CREDIT_OK;
    }
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
        (void)hipGetLastError();
        return CREDIT_ERR_HIP;
    }
    *out = g_static_ptr[dev] = static_cast<SplitCtl *>(ptr);
    return CREDIT_OK;
}

}  // namespace

SplitCtl *static_scratch_if_set_up()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::lock_guard<std::mutex> lk(g_static_mu);
    auto it = g_static_ptr.find(dev);
    return it == g_static_ptr.end() ? nullptr : it->second;
}

}  // namespace credit

extern "C" credit_status_t credit_run_plan_static(credit_op_t op, const credit_operands_t *ops, int64_t rows,
                                                  int64_t cols, float eps, credit_dtype_t dt,
                                                  const credit_plan_t *plan, void *stream)
{
    if (plan == nullptr || ops == nullptr)
        return CREDIT_ERR_INVALID_ARG;
    bool noop = false;
    credit_status_t st = credit::validate_operands(op, *ops, rows, cols, eps, dt, &noop);
    if (st != CREDIT_OK || noop)
        return st;
    credit::SplitCtl *ctl = nullptr;
    st = credit::static_scratch(&ctl);
    if (st != CREDIT_OK)
        return st;
    return credit::run_plan_on_scratch(op, *ops, rows, cols, eps, dt, *plan, stream, ctl);
}
