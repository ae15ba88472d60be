// The corner kernels in 4-byte lanes (boxes at explicit corners, one wave per
// box, unswizzled 4- or 8-byte elements) of direction load; see tmap_corner4.h.
#include "tmap_corner4.h"

namespace tmap {
int launch_corner4_load(int nslot, int dims, const KArgs &a, void *stream) {
    return dims == 2 ? launch_corner4_mode<kLoad, 2>(nslot, a, stream) : launch_corner4_mode<kLoad, 5>(nslot, a, stream);
}
}  // namespace tmap
