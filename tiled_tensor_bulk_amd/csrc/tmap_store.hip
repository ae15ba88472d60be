// tmap_store.hip -- instantiates the store variants of the copy kernel.
#include "tmap_copy.h"

namespace tmap {
int launch_store(int stages, int nslot, const KArgs &a, void *stream) {
    return launch_mode<kStore>(stages, nslot, a, stream);
}
}  // namespace tmap
