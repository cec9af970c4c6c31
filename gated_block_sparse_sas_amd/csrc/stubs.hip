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
size_t sparse_workspace(const Dims&, int) { return 0; }
hipError_t launch_sparse(const void*, const void*, const void*, const int*, const float*, void*,
                         float*, char*, size_t, int, const Dims&, bool, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace sas
