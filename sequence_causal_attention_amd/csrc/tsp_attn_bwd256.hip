// tsp_attn_bwd256.hip -- the dh-256 backward kernels. A unit of its own because the
// key-stationary kernel's 256 accumulator values per lane fill the arch VGPRs: here MFMA
// results stay in the accumulation registers (the compiler's default form), while the
// other head dims are built with MFMA results in arch VGPRs.
#include "bwd_config.h"

template void tsp_bwd_launch<256>(const tsp::TspBwdParams&, int64_t, hipStream_t);
