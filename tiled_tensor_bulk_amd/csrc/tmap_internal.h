// tmap_internal.h -- private layout of the 128-byte tensor map and of the
// kernel argument block.  Shared by the host half (tmap_host.cpp) and the
// device half (tmap_copy.h) of libtmap only.
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

// The kernel's form of a tensor map: the fields the copy reads, with 32-bit
// dims and 16-bit box extents so that it stays small in scalar registers.
struct KMap {
    uint64_t base;
    uint64_t strides[kMaxRank];   // bytes; strides[0] == elem_size; 0 for unused dims
    uint32_t dims[kMaxRank];      // <= 2^31; 1 for unused dims
    int32_t lim[kMaxRank];        // dims - box: a corner c is inside in dim d iff 0 <= c <= lim
    uint32_t span;                // num_records of a buffer resource rebased to a corner
    uint32_t box_bytes;
    uint16_t box[kMaxRank];       // 1 for unused dims
    uint8_t elem_size, rank, swz_b, swz_m, swz_s, pad_[3];
    uint32_t pad2_[3];
};
static_assert(sizeof(KMap) == 128, "KMap layout");

inline KMap kernel_map(const MapImpl &m) {
    KMap k{};
    k.base = m.base;
    for (int d = 0; d < kMaxRank; ++d) {
        k.strides[d] = m.strides[d];
        k.dims[d] = (uint32_t)m.dims[d];
        k.lim[d] = (int32_t)((int64_t)m.dims[d] - (int64_t)m.box[d]);
        k.box[d] = m.box[d];
    }
    k.span = m.span;
    k.box_bytes = m.box_bytes;
    k.elem_size = m.elem_size;
    k.rank = m.rank;
    k.swz_b = m.swz_b;
    k.swz_m = m.swz_m;
    k.swz_s = m.swz_s;
    return k;
}

// Everything a copy kernel needs, passed by value.
struct KArgs {
    KMap src;                     // load / round trip: the source map
    KMap dst;                     // store / round trip: the destination map
    const int32_t *coords;        // [n][rank] corners, or nullptr for a sweep
    uint8_t *packed;              // load: output images; store: input images
    uint32_t *status;             // device status word (bit 0: readiness wait expired)
    int64_t n_tiles;
    uint32_t sweep_tiles[kMaxRank];  // ceil(dims/box) per dimension of the swept map
    // A workgroup walks tiles t0, t0+1, .. in groups of (group_mask+1); from
    // the last tile of a group it jumps by big_step.  Both steps are also
    // given as mixed-radix digits over sweep_tiles for the carry-add cursor.
    uint32_t step_digits[kMaxRank];  // digits of 1
    uint32_t big_digits[kMaxRank];   // digits of big_step
    int64_t big_step;                // grid*group - group + 1
    uint32_t group;                  // tiles per group (power of two); 0 = contiguous runs
    uint32_t group_mask;             // group - 1, or 0xFFFFFFFF for contiguous runs
    // n_tiles / (grid*group) and n_tiles % (grid*group) (contiguous runs: by
    // grid): the same for every workgroup, so divided once on the host
    int64_t deal_q, deal_r;
    uint32_t n_chunks;            // box_bytes / 16
    uint32_t row_chunks;          // box[0]*es / 16
    uint32_t k_el;                // elements per 16-byte chunk (16 / es)
    uint32_t lk_el;               // log2(k_el)
    // A chunk's box indices without a division: n / d == mulhi(n, magic(d))
    // for every n < 2^16 and 2 <= d <= 2^16, with magic(d) = ceil(2^32 / d);
    // magic 0 stands for d == 1.  Chunk indices stay below 4096 (64 KiB boxes).
    uint32_t rc_magic;               // magic(row_chunks)
    uint32_t box_magic[kMaxRank];    // magic(box[d]) of the swept map (a round trip's maps share the box)
    // 1 when, in both maps, every corner whose box touches the tensor lies
    // within 2 GiB of the base, so that corner offsets can be summed in 32
    // bits (explicit-corner kernels)
    uint32_t off32;
    uint32_t elemwise;            // 1 when the swizzle moves data inside 16-byte chunks
    uint32_t grid;                // workgroups launched
    uint32_t regions;             // interleaved streams the groups are dealt as (1: none)
    uint32_t flags;               // TMAP_FLAG_*
    uint32_t spin_limit;          // readiness-wait polls before giving up
    uint32_t add_f32;             // round trip: add `addend` to every fp32 element before storing
    float addend;
    // Band schedule (sweeps of boxes with narrow rows).  A unit is the same
    // band of box rows (the band height) taken from band_g boxes that are
    // neighbours in dimension 0, 16 KiB in all; a stage holds one unit, each
    // box's band as the contiguous piece of that box's LDS image it is.  The
    // cursor then walks units: sweep_tiles/n_tiles count units, ubox is a
    // unit's extent (band_g*box0, band height, box2, ..) and the maps' lim is
    // dims - ubox.  band_g == 0: one whole box per stage, ubox == box.
    uint32_t band_g;              // boxes per unit
    uint32_t band_lnb;            // log2(bands per box)
    uint32_t band_lbc;            // log2(16-byte chunks in one box's band)
    uint32_t band_lbe;            // log2(elements in one box's band)
    uint32_t band_bytes;          // bytes of one box's band
    uint32_t tiles[kMaxRank];     // ceil(dims/box) per dimension of the swept map
    uint32_t ubox[kMaxRank];      // extent of a unit per dimension
    // Explicit corners in 4-byte lanes (tmap_corner4.h): log2 of the 4-byte
    // words in a box row (2..6), log2 of the element size (0..3) and the
    // rows of a box (<= 64).
    uint32_t c4_dshift;
    uint32_t c4_esz;
    uint32_t c4_rows;
    // ... and of a swizzle that moves words within rows: the byte-offset
    // bit its XOR lands on (tb), the bit it takes its key from (sb), and
    // the key's mask (2^B - 1, B <= 4)
    uint32_t c4_tb;
    uint32_t c4_sb;
    uint32_t c4_smask;
};

constexpr int kBandSlots = 4;             // a band stage is 4 slots per lane: 16 KiB
constexpr uint32_t kBandChunks = kBandSlots * kWaves * 64;  // 16-byte chunks in a band stage

}  // namespace tmap

// Launch one copy-kernel variant (stages: see launch_mode; nslot in {1,2,4,8,16}:
// 16-byte chunks per lane per tile; dims 2 for maps of rank <= 2, else 5).
// Each direction and dims class has its own translation unit
// (tmap_{load,store,roundtrip}_r{2,5}.hip).  Return a hipError_t as int.
namespace tmap {
int launch_load_r2(int stages, int nslot, const KArgs &a, void *stream);
int launch_store_r2(int stages, int nslot, const KArgs &a, void *stream);
int launch_roundtrip_r2(int stages, int nslot, const KArgs &a, void *stream);
int launch_load_r5(int stages, int nslot, const KArgs &a, void *stream);
int launch_store_r5(int stages, int nslot, const KArgs &a, void *stream);
int launch_roundtrip_r5(int stages, int nslot, const KArgs &a, void *stream);

// The band schedule of sweeps over maps of rank <= 2 whose dimension-0 rows
// are whole 16-byte chunks: the lean band kernels (tmap_band.h), stages 1..4,
// one translation unit per direction (tmap_band_{load,store,roundtrip}.hip).
int launch_band_load(int stages, const KArgs &a, void *stream);
int launch_band_store(int stages, const KArgs &a, void *stream);
int launch_band_roundtrip(int stages, const KArgs &a, void *stream);

// The no-allocation entry point's status word (tmap_noalloc.hip): its device
// address on the current device, looked up on the first call there
// (noalloc_scratch), or nullptr for a device it was never looked up on
// (noalloc_status).
tmap_status noalloc_scratch(uint32_t **out);
uint32_t *noalloc_status(int dev);
// Record a failure's status and detail text for tmap_last_error_detail().
tmap_status record_failure(tmap_status st, const char *detail);

// Boxes at explicit corners, one wave per box with one stage, boxes of at
// most 8 KiB, swizzles that move whole chunks: the corner kernels
// (tmap_corner.h), nslot 1..8, dims 2 for maps of rank <= 2 else 5, one
// translation unit per direction (tmap_corner_{load,store,roundtrip}.hip).
int launch_corner_load(int nslot, int dims, const KArgs &a, void *stream);
int launch_corner_store(int nslot, int dims, const KArgs &a, void *stream);
int launch_corner_roundtrip(int nslot, int dims, const KArgs &a, void *stream);

// The corner kernels in 4-byte lanes (tmap_corner4.h): maps whose box rows
// are a power of two from 16 to 256 bytes, boxes of at most 64 rows and 8 KiB,
// unswizzled or with a swizzle that moves whole words within rows; nslot 1..8 KiB of stage per wave, dims
// as above, one translation unit per direction
// (tmap_corner4_{load,store,roundtrip}.hip).
int launch_corner4_load(int nslot, int dims, const KArgs &a, void *stream);
int launch_corner4_store(int nslot, int dims, const KArgs &a, void *stream);
int launch_corner4_roundtrip(int nslot, int dims, const KArgs &a, void *stream);

// LDS bytes one workgroup of a variant uses: the ring plus the barrier words.
inline uint32_t variant_lds_bytes(int stages, int nslot) {
    return (uint32_t)stages * (uint32_t)nslot * kWaves * kBlockBytes + 64u;
}

// Waves per workgroup of the wave-per-box variant.  Boxes of 8 KiB and more
// run one wave per workgroup: a CU's LDS then holds as many one-box rings as
// fit (nineteen of 8 KiB) instead of whole groups of four, whose barrier
// words push a fifth group of four 8 KiB rings past the 160 KiB (measured on
// 10^5 scattered 8 KiB boxes: load +3%, round trip +9%).  Smaller boxes keep
// four waves to a workgroup, as the number of workgroups a CU holds is
// limited too.
constexpr int wave_group(int nslot) { return nslot >= 8 ? 1 : kWaves; }

// The same for the wave-per-box variant: one ring of one-box stages per wave.
inline uint32_t wave_lds_bytes(int stages, int nslot) {
    const uint32_t wg = (uint32_t)wave_group(nslot);
    return wg * (uint32_t)stages * (uint32_t)nslot * kBlockBytes + wg * 32u + 4u;
}

// LDS the corner kernels reserve per workgroup beyond their stages and
// barrier words: the load of 8 KiB boxes takes 11 KiB in all, which keeps
// fourteen such workgroups on a CU instead of eighteen (measured on MI355X
// over 10^5 scattered 8 KiB fp32 boxes, before such boxes moved to the
// 4-byte lanes: 0.707 -> 0.730 of peak; sixteen 0.725, thirteen
// 0.68-0.72).  The stores and round trips lose with fewer.
inline uint32_t corner_lds_reserve(int mode, int nslot) {
    return (mode == kLoad && nslot == 8) ? 11264u - (8u * kBlockBytes + 8u) : 0u;
}

// LDS bytes one workgroup of the corner kernels takes.
inline uint32_t corner_lds_bytes(int mode, int nslot) {
    const uint32_t wg = (uint32_t)wave_group(nslot);
    return wg * (uint32_t)nslot * kBlockBytes + wg * 8u + corner_lds_reserve(mode, nslot);
}

// The same for the corner kernels in 4-byte lanes, which reserve nothing
// (up to 5 KiB more per workgroup moved the 10^5 scattered 8 KiB fp32 boxes
// by under 1% in every direction).
inline uint32_t corner4_lds_reserve(int mode, int nslot) {
    (void)mode;
    (void)nslot;
    return 0u;
}
inline uint32_t corner4_lds_bytes(int mode, int nslot) {
    const uint32_t wg = (uint32_t)wave_group(nslot);
    return wg * (uint32_t)nslot * kBlockBytes + wg * 8u + corner4_lds_reserve(mode, nslot);
}
}  // namespace tmap
