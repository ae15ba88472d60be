// The corner kernels (boxes at explicit corners, one wave per box, the
// drained image held in registers) of direction store; see tmap_corner.h.
#include "tmap_corner.h"

namespace tmap {
int launch_corner_store(int nslot, int dims, const KArgs &a, void *stream) {
    return dims == 2 ? launch_corner_mode<kStore, 2>(nslot, a, stream) : launch_corner_mode<kStore, 5>(nslot, a, stream);
}
}  // namespace tmap
