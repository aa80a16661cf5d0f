// attn_host.h - host-side helpers shared by the library's translation units.
#ifndef ATTN_HOST_H
#define ATTN_HOST_H

#include <stddef.h>

#include "attn_fwd.h"

namespace attn_host {

// Clears the calling thread's error text (every entry point starts with it).
void clear_error();
// Records printf-style error text for attn_last_error() and returns s.
attn_status_t fail(attn_status_t s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Whether the byte ranges [a, a+na) and [b, b+nb) intersect.
bool overlaps(const void* a, size_t na, const void* b, size_t nb);

// XCDs and compute units of the current device (cached per device). Workgroups are
// dealt round-robin to the XCDs, so the kernels map workgroup slot v to XCD
// v % xcds. {8, 256} (an MI355X) if the runtime cannot tell; any value is correct,
// only the L2 locality of the tile order depends on it.
struct DeviceShape {
  int xcds;
  int cus;
};
DeviceShape device_shape();

}  // namespace attn_host

#endif
