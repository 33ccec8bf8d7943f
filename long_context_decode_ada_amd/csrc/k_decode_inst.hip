// k_decode_inst.hip -- one (head dimension, group size, query precision)
// family of the decode kernels (k_decode.h), built once per family with
// SKA_INST_D, SKA_INST_G and SKA_INST_QF set, so that the families compile in
// parallel.
#include "k_decode.h"

#if !defined(SKA_INST_D) || !defined(SKA_INST_G) || !defined(SKA_INST_QF)
#error "build with -DSKA_INST_D=<64|128> -DSKA_INST_G=<1|2|4> -DSKA_INST_QF=<0|1>"
#endif

namespace ska {
template hipError_t launch_dg<SKA_INST_D, SKA_INST_G, (SKA_INST_QF != 0)>(const DecodeArgs &, int, dim3, hipStream_t);
}  // namespace ska
