// Host-side helpers of the C ABI shared between its source files.
#pragma once
#include "../../include/wc.h"

namespace wc {

// Argument checks of wc_forward (problem, pointers) without the workspace: WC_OK when the
// call would proceed to the workspace check.  Touches no HIP API.
wc_status forward_check(const wc_problem* p, const void* Q, const void* K, const void* V,
                        const float* u_forced, const void* O, const int32_t* pivots,
                        const int32_t* rank, const uint32_t* flags);

}  // namespace wc
