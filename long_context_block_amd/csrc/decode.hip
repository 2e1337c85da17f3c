// Fused decode step (placeholder until the fused kernel lands).
#include "common.hpp"
#include "internal.hpp"
namespace pisa {
hipError_t launch_decode(const DecodeArgs&, const void*, const void*, const void*, void*, void*, float*, float*, void*,
                         int*, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace pisa
