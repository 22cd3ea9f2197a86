// Launcher of the prompt form (wa_prompt, wa_prompt_sparse): grid shape, dispatch order and
// the kernel variant for the head dim and the number of bf16 parts of P. The kernels and
// their design are in prompt_impl.h (128 pairs a workgroup: prompts at d = 128),
// prompt_quarter.h (dense prompts at d = 256) and prompt_sparse.h (block-sparse prompts at
// d = 256); prompt_inst.hip instantiates them.
#include "wa_common.h"

namespace wa {

hipError_t launch_prompt_main_128_1(const PromptArgs&, int, unsigned, hipStream_t);
hipError_t launch_prompt_main_128_2(const PromptArgs&, int, unsigned, hipStream_t);
hipError_t launch_prompt_main_128_3(const PromptArgs&, int, unsigned, hipStream_t);
hipError_t launch_prompt_quarter_1(const PromptArgs&, hipStream_t);
hipError_t launch_prompt_quarter_2(const PromptArgs&, hipStream_t);
hipError_t launch_prompt_quarter_3(const PromptArgs&, hipStream_t);
hipError_t launch_prompt_rows_1(const PromptArgs&, hipStream_t);
hipError_t launch_prompt_rows_2(const PromptArgs&, hipStream_t);
hipError_t launch_prompt_rows_3(const PromptArgs&, hipStream_t);
hipError_t launch_prompt_post_128(const PromptArgs&, hipStream_t);
hipError_t launch_prompt_post_256(const PromptArgs&, hipStream_t);

hipError_t launch_prompt(const PromptArgs& a, hipStream_t s) {
    const int D = a.d;
    if (D == 256 && !a.bm) {
        // dense prompts at d = 256: every row finished inside one workgroup of the
        // quarter-tile kernel (windowed or not), non-finite re-runs included
        PromptArgs b = a;
        b.nchunk = 1;
        return a.p_parts == 3 ? launch_prompt_quarter_3(b, s)
             : a.p_parts == 2 ? launch_prompt_quarter_2(b, s)
                              : launch_prompt_quarter_1(b, s);
    }
    if (D == 256) {
        // block-sparse prompts at d = 256: row groups over 4096-key segments at absolute
        // positions, then the ordered merge of the segments' partials
        PromptArgs b = a;
        b.chunk_keys = kSparseSeg;
        b.nchunk = b.Cp = sparse_segments(a.window, a.p0, a.n);
        const hipError_t e = a.p_parts == 3 ? launch_prompt_rows_3(b, s)
                           : a.p_parts == 2 ? launch_prompt_rows_2(b, s)
                                            : launch_prompt_rows_1(b, s);
        if (e != hipSuccess) return e;
        return launch_prompt_post_256(b, s);
    }
    // d = 128: the 128-pair kernel, then the merge of a split prompt's chunk partials (or the
    // check of an unsplit one)
    const int G = a.hq / a.hkv;
    const int nblk = (int)(((int64_t)a.n * G + kPromptPairs - 1) / kPromptPairs);
    const unsigned grid = (unsigned)(nblk * a.hkv * a.nchunk);
    const hipError_t e = a.p_parts == 3 ? launch_prompt_main_128_3(a, nblk, grid, s)
                       : a.p_parts == 2 ? launch_prompt_main_128_2(a, nblk, grid, s)
                                        : launch_prompt_main_128_1(a, nblk, grid, s);
    if (e != hipSuccess) return e;
    return launch_prompt_post_128(a, s);
}

}  // namespace wa
