// tmap_load.hip -- instantiates the load variants of the copy kernel.
#include "tmap_copy.h"

namespace tmap {
int launch_load(int stages, int nslot, const KArgs &a, void *stream) {
    return launch_mode<kLoad>(stages, nslot, a, stream);
}
}  // namespace tmap
