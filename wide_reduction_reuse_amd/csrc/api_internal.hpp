// Internal interface between the C ABI translation units of libcredit.so.
#pragma once

#include "args.hpp"
#include "credit.h"

namespace credit {

// credit_run_plan with the split-row exchange on the scratch at `ctl`
// (kScratchBytes of device memory of the current device, in the layout of
// args.hpp) instead of the stream's own, which is then neither allocated nor
// used.  Same validation and errors as credit_run_plan.
credit_status_t run_plan_on_scratch(credit_op_t op, const credit_operands_t &ops, int64_t rows, int64_t cols,
                                    float eps, credit_dtype_t dt, const credit_plan_t &plan, void *stream,
                                    SplitCtl *ctl);

// The argument validation of the operator entry points (credit_run_plan's):
// CREDIT_OK with *noop set when rows == 0.
credit_status_t validate_operands(credit_op_t op, const credit_operands_t &ops, int64_t rows, int64_t cols,
                                  float eps, credit_dtype_t dt, bool *noop);

// The static scratch of the current device (credit_run_plan_static), or null
// if that entry point has not set it up on this device.
SplitCtl *static_scratch_if_set_up();

}  // namespace credit
