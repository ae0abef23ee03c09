// Instantiation of the prefill routing kernel for bf16 queries, head dim 64.
#include "route_impl.h"

namespace dash {
hipError_t launch_route_bf16_64(const RouteParams& p, int b, hipStream_t s) {
    return launch_route_d<uint16_t, 64>(p, b, s);
}
}  // namespace dash
