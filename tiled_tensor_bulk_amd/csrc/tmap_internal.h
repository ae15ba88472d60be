// tmap_internal.h -- private layout of the 128-byte tensor map and of the
// kernel argument block.  Shared by the host half (tmap_host.cpp) and the
// device half (tmap_kernels.hip) of libtmap only.
#pragma once

#include <stdint.h>

#include "../../include/tmap.h"

namespace tmap {

constexpr int kMaxRank = 5;
constexpr uint32_t kMagic = 0x544D4150u;  // "TMAP"

// The decoded form of tmap_t.  Exactly 128 bytes so it can be copied into and
// out of the opaque words, and handed to kernels by value (kernel arguments
// are loaded into scalar registers).  Unused dimensions (d >= rank) hold
// dims = 1, box = 1, stride = 0, so kernels treat every map as rank 5.
struct MapImpl {
    uint64_t base;                // device address of element (0,...,0)
    uint64_t dims[kMaxRank];      // elements, innermost first
    uint64_t strides[kMaxRank];   // bytes; strides[0] == elem_size
    uint16_t box[kMaxRank];       // box extents, innermost first
    uint8_t elem_size;            // 1, 2, 4, 8
    uint8_t rank;                 // 1..5
    uint8_t swz_b, swz_m, swz_s;  // XOR swizzle
    uint8_t dtype;                // tmap_dtype
    uint32_t box_bytes;           // product(box) * elem_size
    uint32_t span;                // box[0]*es + sum_{d>0} (box[d]-1)*strides[d]  (< 2^31)
    uint32_t magic;               // kMagic once encoded
    uint32_t reserved[3];
};
static_assert(sizeof(MapImpl) == 128, "tensor map must be 128 bytes");
static_assert(sizeof(tmap_t) == 128, "tmap_t must be 128 bytes");

enum Mode : int { kLoad = 0, kStore = 1, kRoundtrip = 2 };

constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kThreads = 64 * kWaves;     // 256 lanes
constexpr int kBlockBytes = 1024;         // one wave-wide 16-byte-per-lane LDS write

// Everything a copy kernel needs, passed by value.
struct KArgs {
    MapImpl src;                  // load / round trip: the source map
    MapImpl dst;                  // store / round trip: the destination map
    const int32_t *coords;        // [n][rank] corners, or nullptr for a sweep
    uint8_t *packed;              // load: output images; store: input images
    uint32_t *status;             // device status word (bit 0: readiness wait expired)
    int64_t n_tiles;
    uint32_t sweep_tiles[kMaxRank];  // ceil(dims/box) per dimension of the swept map
    uint32_t step_digits[kMaxRank];  // the tile step of one workgroup (grid, or 1 when
                                     // contiguous) as mixed-radix digits over sweep_tiles
    uint32_t n_chunks;            // box_bytes / 16
    uint32_t row_chunks;          // box[0]*es / 16
    uint32_t k_el;                // elements per 16-byte chunk (16 / es)
    uint32_t elemwise;            // 1 when the swizzle moves data inside 16-byte chunks
    uint32_t grid;                // workgroups launched
    uint32_t flags;               // TMAP_FLAG_*
    uint32_t spin_limit;          // readiness-wait polls before giving up
};

}  // namespace tmap

// Launch one copy-kernel variant (stages in 1..4, nslot in {1,2,4,8,16}:
// 16-byte chunks per lane per tile).  Each direction's variants live in their
// own translation unit (tmap_load.hip, tmap_store.hip, tmap_roundtrip.hip).
// Return a hipError_t as int (0 on success).
namespace tmap {
int launch_load(int stages, int nslot, const KArgs &a, void *stream);
int launch_store(int stages, int nslot, const KArgs &a, void *stream);
int launch_roundtrip(int stages, int nslot, const KArgs &a, void *stream);

// LDS bytes one workgroup of a variant uses: the ring plus the barrier words.
inline uint32_t variant_lds_bytes(int stages, int nslot) {
    return (uint32_t)stages * (uint32_t)nslot * kWaves * kBlockBytes + 64u;
}
}  // namespace tmap
