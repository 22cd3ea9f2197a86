// Instantiations of the decode chunk kernel (decode_impl.h): head dim WA_INST_D, up to
// WA_INST_G query heads per key head; whole rows (8-key load units) if WA_INST_WHOLE, else the
// chunk-partial kernel with 8-key load units (large grids) and with whole-run units (32 keys at
// d = 256 up to four query heads a key head, else 16) for small grids.
// The build compiles this file once per variant the launcher in decode.hip calls, so that they
// compile in parallel.
#include "decode_impl.h"

#if !defined(WA_INST_D) || !defined(WA_INST_G) || !defined(WA_INST_WHOLE)
#error "decode_inst.hip is compiled with -DWA_INST_D=.. -DWA_INST_G=.. -DWA_INST_WHOLE=0|1"
#endif

#define WA_CAT4(a, b, c, d) a##b##c##_##d
#define WA_NAME(kind, d, g) WA_CAT4(launch_decode_, kind, d, g)
namespace wa {

#if WA_INST_WHOLE
hipError_t WA_NAME(whole_, WA_INST_D, WA_INST_G)(const DecodeArgs& a, unsigned grid, hipStream_t s) {
    return launch_chunk_kernel<WA_INST_D, WA_INST_G, true, 8>(a, grid, s);
}
#else
// (beyond four query heads a key head the tree works on 16-key units, so both load 16 keys)
hipError_t WA_NAME(kernel_, WA_INST_D, WA_INST_G)(const DecodeArgs& a, unsigned grid, hipStream_t s) {
    return launch_chunk_kernel<WA_INST_D, WA_INST_G, false, (WA_INST_G <= 4 ? 8 : 16)>(a, grid, s);
}
hipError_t WA_NAME(small_, WA_INST_D, WA_INST_G)(const DecodeArgs& a, unsigned grid, hipStream_t s) {
    return launch_chunk_kernel<WA_INST_D, WA_INST_G, false, (WA_INST_D == 256 && WA_INST_G <= 4 ? 32 : 16)>(a, grid, s);
}
#endif

}  // namespace wa
