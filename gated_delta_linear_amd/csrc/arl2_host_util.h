// Helpers shared by the library's host files (not part of the C interface): the calling
// thread's last-error text that arl2_last_error() returns, and argument checks.
#pragma once

#include "../../include/arl2.h"

namespace arl2host {

// Records a formatted detail as the calling thread's last error and returns st.
arl2_status fail(arl2_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
const char* last_error();
bool aligned16(const void* p);
// ARL2_DEBUG_SYNC=1: synchronise after every launch so that a kernel fault names its call.
bool debug_sync();
// Every rule on a layer configuration that does not need the device (sizes, dtypes, access).
arl2_status check_config(const arl2_config& c);
// The current HIP device, if there is one and it is a gfx950 (else NO_DEVICE / UNSUPPORTED / HIP).
arl2_status current_gfx950(int* dev);

}  // namespace arl2host
