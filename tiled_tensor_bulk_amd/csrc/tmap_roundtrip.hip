// tmap_roundtrip.hip -- instantiates the roundtrip variants of the copy kernel.
#include "tmap_copy.h"

namespace tmap {
int launch_roundtrip(int stages, int nslot, const KArgs &a, void *stream) {
    return launch_mode<kRoundtrip>(stages, nslot, a, stream);
}
}  // namespace tmap
