// Debug mode of the entry points (not installed): with LYNX_DEBUG set in the
// environment, a call that queued work waits for its stream before returning.
#pragma once

#include <hip/hip_runtime.h>

#include "lynx.h"

namespace lynx {

// Returns `st` unchanged unless it is LYNX_OK and LYNX_DEBUG is set to
// anything but "" or "0" (read on every call).  Then it waits for `stream`
// and returns LYNX_ERR_DEVICE if the wait reports an error (a kernel fault
// of this call or of earlier work on the stream).  A stream that is being
// captured into a graph, or whose capture state cannot be queried, is not
// waited for.
lynx_status debug_sync(lynx_status st, hipStream_t stream);

}  // namespace lynx
