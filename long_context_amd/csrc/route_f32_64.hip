// Instantiation of the prefill routing kernel for f32 queries, head dim 64.
#include "route_impl.h"

namespace dash {
hipError_t launch_route_f32_64(const RouteParams& p, int b, hipStream_t s) {
    return launch_route_d<float, 64>(p, b, s);
}
}  // namespace dash
