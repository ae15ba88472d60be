// The band-schedule kernels of rank-2 sweeps (roundtrip); see tmap_band.h.
#include "tmap_band.h"

namespace tmap {
int launch_band_roundtrip(int stages, const KArgs &a, void *stream) {
    return launch_band_mode<kRoundtrip>(stages, a, stream);
}
}  // namespace tmap
