// Online cost/benefit controller for a batch of requests, for gfx950
// (MI355X): one thread per request (Strata prompt-lookup page, section 5;
// the step itself is in pld_control_step.h, shared with the lookup scan's
// emit when a draft call also runs the controller).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pld_control_step.h"
#include "pld_kernels.h"

namespace pld {

namespace {

__global__ __launch_bounds__(256) void pld_control_kernel(ControlArgs a)
{
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= a.batch)
        return;
    double *row = a.state + b * kCtlWords;
    CtlState st = ctl_load(row);
    const ControlResult res =
        control_step(a, st, a.accepted[b], a.round_time[b], a.lookup_len[b], a.lookup_match[b]);
    ctl_store(row, st);
    control_write(a, b, res);
}

}  // namespace

hipError_t launch_control(const ControlArgs &a, hipStream_t s)
{
    if (a.batch <= 0)
        return hipSuccess;
    const unsigned blocks = (unsigned)((a.batch + 255) / 256);
    hipLaunchKernelGGL(pld_control_kernel, dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace pld
