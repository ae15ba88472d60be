// tmap_load_r5.hip -- instantiates the load variants of the copy kernel
// that walk 5 dimensions.
#include "tmap_copy.h"

namespace tmap {
int launch_load_r5(int stages, int nslot, const KArgs &a, void *stream) {
    return launch_mode<kLoad, 5>(stages, nslot, a, stream);
}
}  // namespace tmap
