// Temporary: entry points not yet implemented report an error.
#include "sas_internal.h"
namespace sas {
hipError_t launch_fwd_f32(const void*, const void*, const void*, const void*, const void*,
                          const float*, void*, float*, const Dims&, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_bwd_f32(const void*, const void*, const void*, const void*, const void*,
                          const float*, const void*, const void*, const float*, void*, void*,
                          void*, void*, void*, float*, char*, const BwdWs&, const Dims&,
                          hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace sas
