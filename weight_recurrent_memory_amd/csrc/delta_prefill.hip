// Delta-rule prefill (work in progress: kernels land in the next change).
#include "kernels.hpp"
namespace la {
size_t delta_ws_floats(int HT, int dk, int dv, const LaPlan& plan) {
    return (size_t)HT * plan.G * ((size_t)dk * (dk + dv) + (size_t)dk * dv);
}
hipError_t launch_delta_forward(const void*, const void*, const void*, const void*, const float*, void*,
                                float*, int, int, int, int, int, const LaPlan&, float*, hipStream_t) {
    return hipErrorNotSupported;
}
}  // namespace la
