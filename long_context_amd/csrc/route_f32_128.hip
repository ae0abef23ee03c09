// Instantiation of the prefill routing kernel for f32 queries, head dim 128.
#include "route_impl.h"

namespace dash {
hipError_t launch_route_f32_128(const RouteParams& p, int b, hipStream_t s) {
    return launch_route_d<float, 128>(p, b, s);
}
}  // namespace dash
