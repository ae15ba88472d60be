// tmap_load_r2.hip -- instantiates the load variants of the copy kernel
// that walk 2 dimensions.
#include "tmap_copy.h"

namespace tmap {
int launch_load_r2(int stages, int nslot, const KArgs &a, void *stream) {
    return launch_mode<kLoad, 2>(stages, nslot, a, stream);
}
}  // namespace tmap
