// The corner kernels (boxes at explicit corners, one wave per box, the
// drained image held in registers) of direction roundtrip; see tmap_corner.h.
#include "tmap_corner.h"

namespace tmap {
int launch_corner_roundtrip(int nslot, int dims, const KArgs &a, void *stream) {
    return dims == 2 ? launch_corner_mode<kRoundtrip, 2>(nslot, a, stream) : launch_corner_mode<kRoundtrip, 5>(nslot, a, stream);
}
}  // namespace tmap
