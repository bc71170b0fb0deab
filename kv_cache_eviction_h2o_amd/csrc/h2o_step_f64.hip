// FMA decode-step kernels with double cumulative scores (see h2o_step.h).
#include "h2o_step.h"

namespace h2o {

hipError_t launch_step_f64(const StepArgs& a, bool llds, size_t dyn, hipStream_t st)
{
    return launch_step_scored<double>(a, llds, dyn, st);
}

}  // namespace h2o
