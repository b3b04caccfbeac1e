// la_kernels.h -- entry points of the kernel translation units, called by the
// C-ABI front end after it has validated the arguments and laid out the
// workspace.
#pragma once

#include "la_common.h"

namespace la {

// Float32 vector-ALU path: every dtype / D / mode / feature map.
hipError_t generic_run(const Args &a, int bf16, int bwd, int causal, int phi, hipStream_t s);

}  // namespace la
