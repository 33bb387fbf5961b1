// bf16 MFMA split-KV latent decode for gfx950 (placeholder: no shape is
// specialised yet, so the host falls back to the portable kernel).
#include "internal.h"

namespace mlra {

bool decode_mfma_supported(const Geom&) { return false; }
int decode_mfma_items_per_cu(const Geom&) { return 1; }
hipError_t launch_decode_mfma(const Geom&, const void*, const void*, const void*,
                              const Workspace&, int, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace mlra
