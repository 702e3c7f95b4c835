// FP8 (e4m3) Skiparse-2D attention forward: not built yet.
#include "internal.h"

namespace skiparse {

hipError_t launch_attn_fp8(AttnArgs, int, int, hipStream_t) { return hipErrorNotSupported; }

}  // namespace skiparse
