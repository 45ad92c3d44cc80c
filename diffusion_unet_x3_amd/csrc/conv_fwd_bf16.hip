#include "common.hpp"
#include "launch.hpp"
namespace conv3x3 {
bool launch_fwd_bf16(const Plan&, bool, const uint16_t*, const uint16_t*, const float*, float*,
                     int, int, int, int, int, hipStream_t) { return false; }
}
