// The band-schedule kernels of rank-2 sweeps (load); see tmap_band.h.
#include "tmap_band.h"

namespace tmap {
int launch_band_load(int stages, const KArgs &a, void *stream) {
    return launch_band_mode<kLoad>(stages, a, stream);
}
}  // namespace tmap
