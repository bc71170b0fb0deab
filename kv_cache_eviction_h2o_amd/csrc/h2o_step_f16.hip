// FMA decode-step kernels with _Float16 cumulative scores (see h2o_step.h).
#include "h2o_step.h"

namespace h2o {

hipError_t launch_step_f16(const StepArgs& a, bool llds, size_t dyn, hipStream_t st)
{
    return launch_step_scored<_Float16>(a, llds, dyn, st);
}

}  // namespace h2o
