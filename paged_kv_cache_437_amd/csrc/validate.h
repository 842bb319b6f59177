// The PKV_DEBUG switch of the data-plane calls (internal; the checks themselves are the
// pkv_validate_* calls of include/pkv.h).
#pragma once

namespace pkv {

// True while debug checks are on: every data-plane call then checks its metadata
// arrays on the device (pkv_validate_*) before launching anything, and returns the
// violation instead of launching.  Initially on when the environment variable
// PKV_DEBUG is set to anything but "" or "0"; pkv_debug_enable changes it.
bool debug_checks_on();

}  // namespace pkv
