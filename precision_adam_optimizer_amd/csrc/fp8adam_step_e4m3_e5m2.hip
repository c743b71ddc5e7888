// fp8adam_step_e4m3_e5m2.hip -- instantiates the step kernels for m in E4M3 and v in E5M2
// (one translation unit per format pair, so the library builds in parallel).
#include "fp8adam_engine.h"

namespace fp8adam_engine {

template int run_step_f<0, 1>(fp8adam_ctx*, const StepConsts&, int64_t, hipStream_t);

}  // namespace fp8adam_engine
