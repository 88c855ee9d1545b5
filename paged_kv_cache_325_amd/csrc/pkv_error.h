// The calling thread's last-error message, shared by every translation unit
// of the C ABI (pkv_last_error() returns it).  Host code only.
#pragma once

#include "pkv.h"

namespace pkv {

// Records a printf-style message for pkv_last_error() and returns st.
pkv_status fail(pkv_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

const char* last_error();

}  // namespace pkv
