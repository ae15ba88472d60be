// tmap_roundtrip_r2.hip -- instantiates the roundtrip variants of the copy kernel
// that walk 2 dimensions.
#include "tmap_copy.h"

namespace tmap {
int launch_roundtrip_r2(int stages, int nslot, const KArgs &a, void *stream) {
    return launch_mode<kRoundtrip, 2>(stages, nslot, a, stream);
}
}  // namespace tmap
