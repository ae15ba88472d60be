// tmap_store_r5.hip -- instantiates the store variants of the copy kernel
// that walk 5 dimensions.
#include "tmap_copy.h"

namespace tmap {
int launch_store_r5(int stages, int nslot, const KArgs &a, void *stream) {
    return launch_mode<kStore, 5>(stages, nslot, a, stream);
}
}  // namespace tmap
