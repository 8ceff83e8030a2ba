// Host-side helpers shared by the C ABI's source files.
#pragma once
#include "csa2.h"

namespace csa2 {

// Records a formatted message for csa2_last_error() on this thread and returns st.
csa2_status api_fail(csa2_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace csa2
