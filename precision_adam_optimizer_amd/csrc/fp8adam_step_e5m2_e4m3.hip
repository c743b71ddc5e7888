// fp8adam_step_e5m2_e4m3.hip -- instantiates the step kernels for m in E5M2 and v in E4M3
// (one translation unit per format pair, so the library builds in parallel).
#include "fp8adam_engine.h"

namespace fp8adam_engine {

template int run_step_f<1, 0>(fp8adam_ctx*, const StepConsts&, int64_t, hipStream_t);

}  // namespace fp8adam_engine
