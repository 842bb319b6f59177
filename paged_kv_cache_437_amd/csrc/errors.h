// Last-error text of the C ABI (internal): one thread-local message per thread,
// read back by pkv_last_error.
#pragma once

#include "../../include/pkv.h"

namespace pkv {

// Sets the calling thread's last-error text (printf format) and returns st.
pkv_status report_error(pkv_status st, const char* fmt, ...)
    __attribute__((format(printf, 2, 3)));
// Clears it and returns PKV_OK.
pkv_status report_ok();

}  // namespace pkv
