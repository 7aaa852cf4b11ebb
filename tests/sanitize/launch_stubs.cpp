// Stand-ins for the two kernel launchers in the host-only sanitizer build of
// the planner and the C ABI layer (tests/test_sanitize.py). That build runs the
// CPU tests only, which never reach a launch; if one did, the call fails with
// hipErrorInvalidValue (1) instead of touching a device.
#include "pod_internal.h"

namespace pod {

int launch_pod_grid(const Params&, int, int, void*, void*) { return 1; }

int static_scratch(int, void**) { return 1; }

int launch_merge_states(const void*, const float*, const void*, const float*, void*, float*, int64_t,
                        int, int, const float*, void*) {
  return 1;
}

}  // namespace pod
