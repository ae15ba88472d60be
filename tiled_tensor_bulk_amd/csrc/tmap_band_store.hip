// The band-schedule kernels of rank-2 sweeps (store); see tmap_band.h.
#include "tmap_band.h"

namespace tmap {
int launch_band_store(int stages, const KArgs &a, void *stream) {
    return launch_band_mode<kStore>(stages, a, stream);
}
}  // namespace tmap
