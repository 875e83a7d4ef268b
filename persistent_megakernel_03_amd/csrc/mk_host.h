// mk_host.h -- host-side helpers shared by the library's translation units.
#pragma once

#include "../../include/mk.h"

namespace mk {

// Set the calling thread's mk_last_error() message (printf-style) and return st.
mk_status host_fail(mk_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace mk
