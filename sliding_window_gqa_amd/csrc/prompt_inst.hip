// One instantiation of the prompt kernels with P in WA_INST_NP bf16 parts: at head dim 128 the
// 128-pair kernel (prompt_impl.h), at head dim 256 the quarter-tile kernel of dense prompts
// (prompt_quarter.h) and the row-group kernel of block-sparse prompts (prompt_sparse.h); with
// WA_INST_POST also the merge and check kernels at that head dim.
// The build compiles this file once per variant the launcher in prompt.hip calls, so that
// they compile in parallel.
#include "prompt_sparse.h"

#if !defined(WA_INST_D) || !defined(WA_INST_NP) || !defined(WA_INST_POST)
#error "prompt_inst.hip is compiled with -DWA_INST_D=.. -DWA_INST_NP=.. -DWA_INST_POST=0|1"
#endif

#define WA_CAT3(a, b, c) a##b##_##c
#define WA_MAIN(d, np) WA_CAT3(launch_prompt_main_, d, np)
#define WA_CAT2(a, b) a##b
#define WA_POST(d) WA_CAT2(launch_prompt_post_, d)

namespace wa {

#if WA_INST_D == 128
hipError_t WA_MAIN(WA_INST_D, WA_INST_NP)(const PromptArgs& b, int nblk, unsigned grid, hipStream_t s) {
    return launch_main<WA_INST_D, WA_INST_NP>(b, nblk, grid, s);
}
#endif

#if WA_INST_D == 256
#define WA_QUARTER(np) WA_CAT2(launch_prompt_quarter_, np)
#define WA_ROWS(np) WA_CAT2(launch_prompt_rows_, np)
hipError_t WA_QUARTER(WA_INST_NP)(const PromptArgs& b, hipStream_t s) { return launch_quarter<WA_INST_NP>(b, s); }
hipError_t WA_ROWS(WA_INST_NP)(const PromptArgs& b, hipStream_t s) { return launch_rows<WA_INST_NP>(b, s); }
#endif

#if WA_INST_POST
hipError_t WA_POST(WA_INST_D)(const PromptArgs& a, hipStream_t s) { return launch_post<WA_INST_D>(a, s); }
#endif

}  // namespace wa
