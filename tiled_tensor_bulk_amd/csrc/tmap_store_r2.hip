// tmap_store_r2.hip -- instantiates the store variants of the copy kernel
// that walk 2 dimensions.
#include "tmap_copy.h"

namespace tmap {
int launch_store_r2(int stages, int nslot, const KArgs &a, void *stream) {
    return launch_mode<kStore, 2>(stages, nslot, a, stream);
}
}  // namespace tmap
