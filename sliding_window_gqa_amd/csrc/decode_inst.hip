// One instantiation of the decode chunk kernel (decode_impl.h): head dim WA_INST_D, up to
// WA_INST_G query heads per key head, whole rows if WA_INST_WHOLE. The build compiles this
// file once per variant the launcher in decode.hip calls, so that they compile in parallel.
#include "decode_impl.h"

#if !defined(WA_INST_D) || !defined(WA_INST_G) || !defined(WA_INST_WHOLE)
#error "decode_inst.hip is compiled with -DWA_INST_D=.. -DWA_INST_G=.. -DWA_INST_WHOLE=0|1"
#endif

#define WA_CAT4(a, b, c, d) a##b##c##_##d
#define WA_NAME(kind, d, g) WA_CAT4(launch_decode_, kind, d, g)
#if WA_INST_WHOLE
#define WA_FN WA_NAME(whole_, WA_INST_D, WA_INST_G)
#else
#define WA_FN WA_NAME(kernel_, WA_INST_D, WA_INST_G)
#endif

namespace wa {

hipError_t WA_FN(const DecodeArgs& a, unsigned grid, hipStream_t s) {
    return launch_chunk_kernel<WA_INST_D, WA_INST_G, WA_INST_WHOLE != 0>(a, grid, s);
}

}  // namespace wa
