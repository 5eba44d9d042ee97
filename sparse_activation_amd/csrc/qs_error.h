// Thread-local error text behind qs_last_error() (internal).
#pragma once

#include "../../include/qs.h"

namespace qs {
// Records `msg` as the calling thread's last error text and returns `st`.
qs_status set_error(qs_status st, const char* msg);
}  // namespace qs
