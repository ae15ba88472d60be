// tmap_host.cpp -- host half of libtmap: tensor-map encode and validation,
// queries, the gfx950 device gate, launch selection and the status word.
//
// Encode follows "Day 76: The Tensor Memory Accelerator (TMA)", sections
// "The address arithmetic moves into a descriptor" and "Pitfalls": the map is
// validated and packed once on the host, every rule is checked, and a single
// failed rule fails the whole call with INVALID_VALUE.

#include <hip/hip_runtime_api.h>

#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>

#include "tmap_internal.h"

using tmap::MapImpl;

namespace {

thread_local std::string g_detail;

tmap_status fail(tmap_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
tmap_status fail(tmap_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_detail = buf;
    return st;
}

tmap_status ok() {
    g_detail.clear();
    return TMAP_SUCCESS;
}

int elem_size_of(tmap_dtype t) {
    switch (t) {
        case TMAP_U8: case TMAP_I8: return 1;
        case TMAP_U16: case TMAP_F16: case TMAP_BF16: return 2;
        case TMAP_U32: case TMAP_I32: case TMAP_F32: return 4;
        case TMAP_U64: case TMAP_F64: return 8;
    }
    return 0;
}

bool decode(const tmap_t *map, MapImpl &m) {
    if (!map) return false;
    std::memcpy(&m, map, sizeof m);
    return m.magic == tmap::kMagic;
}

// ------------------------------------------------------------------ device
// The status words kernels set when a bounded readiness wait expires: one
// per stream that has launched on the device, so that a timeout is reported
// to the stream whose copy it was.  Word 0 is shared by the streams beyond
// the first kStatusSlots - 1.
constexpr uint32_t kStatusSlots = 256;

struct DeviceState {
    bool probed = false;
    bool supported = false;
    int cus = 0;
    uint32_t lds_per_cu = 0;
    uint32_t *status = nullptr;  // kStatusSlots words, allocated on first launch
    std::unordered_map<void *, uint32_t> slot_of;  // stream -> its word
};
std::mutex g_dev_mu;
DeviceState g_dev[64];

// Arch gate: the copy kernels are built for gfx950 only.  The check happens
// before any allocation or launch ("Day 76", "Checks for the first run": the
// capability gate is a branch taken before anything is allocated).
// need_status: also allocate the status word (launches; a plan query does not).
tmap_status device_for_launch(DeviceState **out, bool need_status = true) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return fail(TMAP_ERROR_UNSUPPORTED_DEVICE, "no HIP device is available");
    }
    std::lock_guard<std::mutex> lk(g_dev_mu);
    DeviceState &d = g_dev[dev];
    if (!d.probed) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess) {
            (void)hipGetLastError();
            return fail(TMAP_ERROR_UNSUPPORTED_DEVICE, "cannot query HIP device %d", dev);
        }
        d.probed = true;
        d.supported = std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
        d.cus = p.multiProcessorCount;
        d.lds_per_cu = (uint32_t)p.maxSharedMemoryPerMultiProcessor;
        if (d.lds_per_cu == 0) d.lds_per_cu = 160 * 1024;
    }
    if (!d.supported)
        return fail(TMAP_ERROR_UNSUPPORTED_DEVICE, "device %d is not gfx950", dev);
    if (need_status && !d.status) {
        void *p = nullptr;
        const size_t bytes = kStatusSlots * sizeof(uint32_t);
        if (hipMalloc(&p, bytes) != hipSuccess || hipMemset(p, 0, bytes) != hipSuccess ||
            hipDeviceSynchronize() != hipSuccess) {
            (void)hipGetLastError();
            if (p) (void)hipFree(p);
            return fail(TMAP_ERROR_LAUNCH, "cannot allocate the status words");
        }
        d.status = (uint32_t *)p;
    }
    *out = &d;
    return TMAP_SUCCESS;
}

// The status word of `stream` on device d: its own while fewer than
// kStatusSlots - 1 streams have launched there, else the shared word 0.
uint32_t status_slot(DeviceState &d, void *stream) {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    auto it = d.slot_of.find(stream);
    if (it != d.slot_of.end()) return it->second;
    const uint32_t slot = d.slot_of.size() + 1 < kStatusSlots ? (uint32_t)d.slot_of.size() + 1 : 0u;
    d.slot_of.emplace(stream, slot);
    return slot;
}

int64_t sweep_count(const MapImpl &m) {
    int64_t n = 1;
    for (int d = 0; d < m.rank; ++d) n *= (int64_t)((m.dims[d] + m.box[d] - 1) / m.box[d]);
    return n;
}

struct Plan {
    int nslot, stages;            // stages: the launch code of launch_mode
    uint32_t grid;                // walkers the tiles are dealt to
    uint32_t group;
    uint32_t regions;
    uint32_t lds;                 // bytes per workgroup
    uint32_t band_g, band_rows;   // band schedule (0: whole boxes)
    bool lean;                    // the band schedule runs the lean rank-2 band kernels
    bool corner;                  // wave per box with one stage runs the corner kernels
    bool corner4;                 // ... in 4-byte lanes (tmap_corner4.h)
};

uint32_t log2u(uint32_t v) {
    uint32_t l = 0;
    while ((1u << l) < v) ++l;
    return l;
}

// Bytes a unit of g boxes, `rows` rows tall, reaches from its corner in
// kernel map k.
uint64_t band_span(const tmap::KMap &k, uint32_t g, uint32_t rows) {
    return (uint64_t)g * k.box[0] * k.elem_size + (uint64_t)(rows - 1) * k.strides[1];
}

// Whether a launch runs on the band schedule, and its boxes per unit (g),
// bands per box (nb) and rows per band.  It applies to sweeps whose boxes
// have rows of 64 to 512 bytes and whose dimension-1 extent is a power-of-two
// multiple of the band height (boxes of rank 2, or with extent 1 above
// dimension 1), when the swizzle maps each band of a box onto itself and a
// row of the sweep holds at least one full unit.  A unit is one 16 KiB
// stage: g = 16 KiB / (rows * box row bytes) boxes side by side.  By default
// it is taken only for tensors spanning at least kBandMinSpan bytes: it buys
// DRAM page locality, which a tensor that fits in the 256 MB last-level
// cache (MALL) does not need, while its smaller units cost latency there.
constexpr uint64_t kBandMinSpan = 256ull << 20;

// Default band heights, measured on MI355X over the 2 GiB u8, 1 GiB fp32 and
// ragged bf16 sweeps.  The band kernel of rank-2 sweeps (tmap_band.h): round
// trips 8-row bands (units 2 KiB wide), loads and stores 16-row bands (units
// 1 KiB wide for 128-byte box rows); the generic ring: round trips 2-row
// bands of units 8 KiB wide (with 3 stages and 4 units per workgroup, see
// plan_launch), loads and stores 8-row bands (0.5-1.8% faster than 16).
// Where that height does not fit the box or the sweep, the next taller one
// that does is taken.
constexpr uint32_t kBandRowsRoundtrip = 2;
constexpr uint32_t kBandRowsLoadStore = 8;
constexpr uint32_t kLeanRowsRoundtrip = 8;
constexpr uint32_t kLeanRowsLoadStore = 16;

// A band-kernel round trip between tensors whose row pitch is not a power of
// two takes 2-row bands dealt as two interleaved streams instead.  Measured
// on MI355X (3 stages x 2 units; fraction of 8 TB/s): the ragged bf16 sweep
// (pitch 32640) 0.796-0.801 at three placements of the destination against
// 0.68-0.76 in 8-row bands; pitches 33024 and 40960: 0.793 and 0.763
// against 0.793 and 0.746; 49152: 0.746 against 0.752.  With power-of-two
// pitches 8-row bands in one stream stay best (2 GiB u8: 0.818 against
// 0.813, 1 GiB fp32: 0.827 against 0.811, pitch 32768: 0.817 against 0.808).
constexpr uint32_t kLeanRowsRoundtripSpread = 2;

// The accelerator complex dies (XCDs) of an MI355X: each has its own L2, and
// the dispatcher hands consecutive workgroups to them in turn.
constexpr uint32_t kXcds = 8;

// Whether every tensor a round trip streams has a power-of-two row pitch
// (the byte stride of dimension 1).
bool pow2_pitches(const tmap::KArgs &a) {
    for (const tmap::KMap *k : {&a.src, &a.dst}) {
        const uint64_t p = k->strides[1];
        if (k->rank >= 2 && (p & (p - 1))) return false;
    }
    return true;
}

// The checks that depend on the band height; nullptr when `rows` fits,
// else the reason.  rc: 16-byte chunks per box row.
const char *band_height_misfit(const MapImpl &m, const tmap::KArgs &a, uint32_t rc, uint32_t rows, uint32_t &g,
                               uint32_t &nb) {
    if (!rows || (rows & (rows - 1))) return "band_rows must be a power of two";
    if (rows * rc > tmap::kBandChunks) return "a band of band_rows box rows exceeds a 16 KiB stage";
    g = tmap::kBandChunks / (rows * rc);
    if (m.box[1] % rows) return "band_rows must divide the box's dimension-1 extent";
    nb = m.box[1] / rows;
    if (nb & (nb - 1)) return "the box's dimension-1 extent must be band_rows times a power of two";
    // the swizzle only changes element-offset bits [m, m+b), so it maps each
    // band onto itself when a band is a whole number of 2^(m+b) blocks
    if (m.swz_b && ((uint64_t)rows * m.box[0]) % (1ull << (m.swz_m + m.swz_b)))
        return "the swizzle does not map a band of band_rows rows onto itself";
    if (a.tiles[0] < g) return "a row of the sweep holds fewer boxes than a unit of band_rows rows";
    // a unit's buffer records, like a box's, stay below the out-of-range offset
    if (band_span(a.src, g, rows) >= 0x80000000ull || band_span(a.dst, g, rows) >= 0x80000000ull)
        return "a unit reaches 2 GiB or more from its corner";
    return nullptr;
}

// Whether the maps of a copy suit the band kernel of rank-2 sweeps
// (tmap_band.h): both have rank <= 2, or are batches of such planes, and
// every tensor side's dimension-0 row is a whole number of 16-byte chunks,
// so that the tensor's edge never cuts a chunk (the generic ring's element
// path is then never needed).
bool band_lean_maps(int mode, const tmap::KArgs &a) {
    // rank 2, or a batch of planes: rank 3 with boxes of extent 1 in
    // dimension 2 (the kernel's third cursor digit walks the planes)
    auto planes = [](const tmap::KMap &k) { return k.rank <= 2 || (k.rank == 3 && k.box[2] == 1); };
    if (!planes(a.src) || !planes(a.dst)) return false;
    auto whole = [](const tmap::KMap &k) { return ((uint64_t)k.dims[0] * k.elem_size) % 16u == 0; };
    if (mode != tmap::kStore && !whole(a.src)) return false;
    if (mode != tmap::kLoad && !whole(a.dst)) return false;
    return true;
}

// Whether a tensor's span (outermost dim times its stride) is below the
// size from which the band pays for DRAM page locality: it then stays in
// the last-level cache.
bool resident_span(const MapImpl &m) { return m.dims[m.rank - 1] * m.strides[m.rank - 1] < kBandMinSpan; }

// want_rows: the band height asked for, 0 for the default of the direction
// (lean: the maps suit the band kernel, whose defaults differ).  An explicit
// height that does not fit leaves *why set and returns false; without one
// the schedule falls back to whole boxes silently.
bool band_fits(const MapImpl &m, const tmap::KArgs &a, bool roundtrip, uint32_t flags, uint32_t want_rows,
               uint32_t &g, uint32_t &nb, uint32_t &rows, const char **why = nullptr, bool lean = false) {
    if (a.coords || a.elemwise) return false;
    if (flags & (TMAP_FLAG_THREAD_COPY | TMAP_FLAG_PRODUCER_WAVE | TMAP_FLAG_WAVE_PER_BOX)) return false;
    // whole boxes: on the band kernel, units of whole boxes (bands as tall
    // as the box, so a stage holds each of its boxes' whole swizzled
    // images); the generic ring otherwise
    const bool whole = flags & TMAP_FLAG_WHOLE_BOX;
    if (whole && !lean) return false;
    if (m.rank < 2) return false;
    // a tensor that fits in the last-level cache takes the band only on the
    // band kernel (or when TMAP_FLAG_BAND asks for it), and then in the
    // tallest bands that fit: there the per-unit work, not DRAM page
    // locality, decides (measured on MI355X over the 30 MB fp16 strips
    // workload: 0.835 of peak in 32-row bands against 0.70 through registers
    // and 0.60 for whole boxes on the generic ring)
    const bool resident = !(flags & TMAP_FLAG_BAND) && resident_span(m);
    if (resident && !lean) return false;
    for (int d = 2; d < tmap::kMaxRank; ++d)
        if (m.box[d] != 1) return false;
    const uint32_t rc = (uint32_t)m.box[0] * m.elem_size / 16u;  // 16-byte chunks per box row
    if (rc < 4 || rc > 32 || (rc & (rc - 1))) return false;
    if (whole) {
        rows = m.box[1];
        return !band_height_misfit(m, a, rc, rows, g, nb);
    }
    if (want_rows) {
        rows = want_rows;
        const char *w = band_height_misfit(m, a, rc, rows, g, nb);
        if (w && why) *why = w;
        return w == nullptr;
    }
    if (resident) {
        for (rows = 1u << 8; rows >= 1; rows /= 2)
            if (rows <= m.box[1] && !band_height_misfit(m, a, rc, rows, g, nb)) return true;
        return false;
    }
    const uint32_t first =
        lean ? (roundtrip ? (pow2_pitches(a) ? kLeanRowsRoundtrip : kLeanRowsRoundtripSpread) : kLeanRowsLoadStore)
             : (roundtrip ? kBandRowsRoundtrip : kBandRowsLoadStore);
    for (rows = first; rows <= m.box[1]; rows *= 2)
        if (!band_height_misfit(m, a, rc, rows, g, nb)) return true;
    // the band kernel's defaults are tall: a shorter box takes the tallest
    // height below them that fits
    if (lean)
        for (rows = first / 2; rows >= 1; rows /= 2)
            if (!band_height_misfit(m, a, rc, rows, g, nb)) return true;
    return false;
}

// Re-point the launch at units of the band schedule.
void band_setup(const MapImpl &m, tmap::KArgs &a, uint32_t g, uint32_t nb, uint32_t rows) {
    const uint32_t bc = rows * a.row_chunks;
    a.band_g = g;
    a.band_lnb = log2u(nb);
    a.band_lbc = log2u(bc);
    a.band_lbe = log2u(rows * (uint32_t)m.box[0]);
    a.band_bytes = bc * 16u;
    int64_t units = 1;
    for (int d = 0; d < tmap::kMaxRank; ++d) {
        a.sweep_tiles[d] = d == 0 ? (a.tiles[0] + g - 1) / g : (d == 1 ? a.tiles[1] * nb : a.tiles[d]);
        a.ubox[d] = d == 0 ? g * m.box[0] : (d == 1 ? rows : m.box[d]);
        units *= a.sweep_tiles[d];
    }
    a.n_tiles = units;
    a.n_chunks = tmap::kBandSlots * tmap::kWaves * 64u;
    for (tmap::KMap *k : {&a.src, &a.dst}) {
        for (int d = 0; d < tmap::kMaxRank; ++d) k->lim[d] = (int32_t)((int64_t)k->dims[d] - (int64_t)a.ubox[d]);
        k->span = (uint32_t)band_span(*k, g, rows);
    }
}

// Every flag bit the header defines; a caller's other bits are rejected
// rather than ignored, so that a misspelt or future flag does not run as a
// different copy.
constexpr uint32_t kKnownFlags = TMAP_FLAG_CONTIGUOUS | TMAP_FLAG_NONTEMPORAL | TMAP_FLAG_THREAD_COPY |
                                 TMAP_FLAG_PRODUCER_WAVE | TMAP_FLAG_WHOLE_BOX | TMAP_FLAG_BAND |
                                 TMAP_FLAG_WAVE_PER_BOX | TMAP_FLAG_CACHED_PACKED | TMAP_FLAG_INJECT_BUDGET_MISMATCH |
                                 TMAP_FLAG_DEBUG_POISON;

// lean: the band schedule runs the band kernel of rank-2 sweeps.
// elemwise: the swizzle moves data inside 16-byte chunks.
tmap_status plan_launch(int mode, const MapImpl &m, int64_t n_tiles, const tmap_launch_opts *opts,
                        const DeviceState &dev, bool band, bool lean, bool corners, bool elemwise, Plan &pl) {
    const uint32_t flags0 = opts ? opts->flags : 0u;
    const uint32_t per_wave_pass = tmap::kWaves * tmap::kBlockBytes;  // bytes one slot per lane covers
    const uint32_t need = (m.box_bytes + per_wave_pass - 1) / per_wave_pass;
    int nslot = 1;
    while ((uint32_t)nslot < need) nslot *= 2;
    if (nslot > 16) return fail(TMAP_ERROR_INVALID_VALUE, "box of %u bytes is too large", m.box_bytes);
    if (band) nslot = tmap::kBandSlots;  // a stage is one 16 KiB unit
    // default ring depth: 2; explicit corners (boxes scattered over the
    // tensor, many of them cut by its edges): 1, as each box's edge work
    // leaves little to overlap and the smaller footprint fits more
    // workgroups (measured best on MI355X)
    int stages = (opts && opts->stages) ? (int)opts->stages : (corners ? 1 : 2);
    // band sweeps on the generic ring (maps the band kernel does not take,
    // such as batches of planes that do not fold into one matrix): round
    // trips 2 stages over 4 units per workgroup, loads and stores 1 stage
    // over 2 units (measured on MI355X over batches of 32 planes that do not
    // fold, u8 1000 rows in 128 x 128 boxes, bf16 1000 rows and fp32 500
    // rows in 64 x 64 boxes, fraction of 8 TB/s: round trips 0.685 / 0.765
    // / 0.766 against 0.662 / 0.657 / 0.658 with 3 stages, loads 0.798 /
    // 0.782 / 0.791 against 0.652 / 0.649 / 0.641 with 1 unit, stores 0.782
    // / 0.781 / 0.770 against 0.745 / 0.753 / 0.750)
    if (band && mode == tmap::kRoundtrip && !(opts && opts->stages)) stages = 2;
    // the band kernel: 3 stages in every direction, of which its two units
    // (below) use two; the third stage's LDS holds a CU to three workgroups.
    // Measured on MI355X with 5 warm-up and 20 timed launches after an idle
    // gap, 2 GiB u8 round trip: 0.816-0.818 of peak at 3 stages x 2 units,
    // 0.812-0.815 at 2 x 2 (four workgroups a CU), 0.756-0.764 at 3 x 4.
    // A tensor that stays in the last-level cache takes 2 stages (fp16
    // strips: 0.835 against 0.78 at 3)
    if (lean && !(opts && opts->stages)) stages = (resident_span(m) && !(flags0 & TMAP_FLAG_BAND)) ? 2 : 3;
    // whole 16 KiB boxes (one to a unit) in a round trip on the band kernel:
    // 4 stages x 4 units in one stream (measured on MI355X, fraction of 8
    // TB/s, against 3 x 2 in two streams: 2 GiB u8 0.738 / 0.705, 1 GiB fp32
    // +1.0f 0.774 / 0.755; ragged bf16's 8 KiB boxes keep 3 x 2, two streams)
    const bool whole16 = lean && (flags0 & TMAP_FLAG_WHOLE_BOX) && mode == tmap::kRoundtrip &&
                         m.box_bytes == 16384u && !resident_span(m);
    if (whole16 && !(opts && opts->stages)) stages = 4;
    if (stages < 1 || stages > 4)
        return fail(TMAP_ERROR_INVALID_VALUE, "stages must be 1..4 (got %d)", stages);
    const uint32_t flags = opts ? opts->flags : 0u;
    const bool thread_copy = flags & TMAP_FLAG_THREAD_COPY;
    const bool producer_wave = flags & TMAP_FLAG_PRODUCER_WAVE;
    bool wave_box = flags & TMAP_FLAG_WAVE_PER_BOX;
    if ((int)thread_copy + (int)producer_wave + (int)wave_box > 1)
        return fail(TMAP_ERROR_INVALID_VALUE, "thread-copy, producer-wave and wave-per-box modes exclude each other");
    if (wave_box && (flags & TMAP_FLAG_WHOLE_BOX))
        return fail(TMAP_ERROR_INVALID_VALUE, "TMAP_FLAG_WAVE_PER_BOX and TMAP_FLAG_WHOLE_BOX exclude each other");
    // explicit corners of boxes up to 8 KiB run wave-per-box by default: one
    // wave per box does each box's scalar address and bounds work once and
    // keeps four boxes in flight per workgroup (measured on MI355X over 10^5
    // scattered 8 KiB boxes: round trip +28%, store +12%, load +2%)
    if (corners && !band && m.box_bytes <= 8192u && !(opts && opts->stages > 2) &&
        !(flags & (TMAP_FLAG_THREAD_COPY | TMAP_FLAG_PRODUCER_WAVE | TMAP_FLAG_WHOLE_BOX)))
        wave_box = true;
    // sweeps the band kernel does not take (maps of rank 3 and more, and
    // others) with boxes of up to 8 KiB and a swizzle that moves whole
    // chunks run on the corner kernels too, one stage, their corners walked
    // by the kernels' cursor (measured on MI355X, padded 5-D fp32 tensor
    // tiled by three shapes of 8 KiB box, in 4-byte lanes, one stream,
    // fraction of 8 TB/s against the shared ring: round trips 0.45 / 0.53 /
    // 0.45 against 0.23 / 0.17 / 0.22, loads 0.65 / 0.76 / 0.66 against
    // 0.38 / 0.31 / 0.38, stores 0.63 / 0.69 / 0.63 against 0.47 / 0.40 /
    // 0.47)
    const bool sweep_corner = !corners && !band && !elemwise && m.box_bytes <= 8192u &&
                              !(opts && opts->stages > 1) &&
                              !(flags & (TMAP_FLAG_THREAD_COPY | TMAP_FLAG_PRODUCER_WAVE | TMAP_FLAG_WHOLE_BOX));
    if (sweep_corner) {
        wave_box = true;
        stages = 1;
    }
    // the other sweeps of whole boxes on the cooperative ring (boxes over
    // 8 KiB, swizzles that move elements inside chunks, TMAP_FLAG_WHOLE_BOX
    // where the band kernel does not apply): one stage, which fits twice the
    // workgroups on a CU (measured on MI355X, padded 5-D fp32 tensor swept
    // by 16 and 32 KiB boxes, fraction of 8 TB/s: loads 0.615 / 0.589
    // against 0.485 / 0.448 with two stages, round trips 0.274 / 0.273
    // against 0.248 / 0.201, stores 0.565 / 0.540 against 0.562 / 0.520;
    // 8 KiB whole boxes: load 0.462 against 0.381; 8 KiB boxes under a
    // swizzle of 4-byte granules: load 0.196 against 0.172)
    if (!(opts && opts->stages) && !corners && !band && !sweep_corner &&
        !(flags & (TMAP_FLAG_THREAD_COPY | TMAP_FLAG_PRODUCER_WAVE | TMAP_FLAG_WAVE_PER_BOX)))
        stages = 1;
    if (opts && (opts->flags & TMAP_FLAG_BAND) && (opts->flags & TMAP_FLAG_WHOLE_BOX))
        return fail(TMAP_ERROR_INVALID_VALUE, "TMAP_FLAG_BAND and TMAP_FLAG_WHOLE_BOX exclude each other");
    if (thread_copy) stages = 1;  // one LDS stage; the next tile waits in registers
    if (producer_wave) {
        if (nslot > 8)
            return fail(TMAP_ERROR_INVALID_VALUE, "producer-wave mode needs boxes of at most 32 KiB");
        if (stages < 2) stages = 2;
    }
    if (wave_box) {
        // a stage is one box of one wave: nslot KiB (16-byte slots per lane)
        nslot = 1;
        while ((uint32_t)nslot * tmap::kBlockBytes < m.box_bytes) nslot *= 2;
        if (nslot > 16)
            return fail(TMAP_ERROR_INVALID_VALUE, "wave-per-box mode needs boxes of at most 16 KiB");
        if (stages > 2) return fail(TMAP_ERROR_INVALID_VALUE, "wave-per-box mode takes 1 or 2 stages");
    }
    const uint32_t lds = wave_box ? tmap::wave_lds_bytes(stages, nslot) : tmap::variant_lds_bytes(stages, nslot);
    if (lds > dev.lds_per_cu || (!wave_box && nslot == 16 && stages > 2))
        return fail(TMAP_ERROR_INVALID_VALUE, "%d stages of %u bytes do not fit in LDS", stages,
                    (unsigned)(nslot * (wave_box ? tmap::kBlockBytes : per_wave_pass)));
    // group: consecutive tiles (units on the band schedule) a workgroup takes
    // in a row.  Whole boxes: enough boxes side by side to cover 512 bytes of
    // a row, so that a workgroup's tiles in flight read and write neighbouring
    // row segments, and at least 2; units: 4 for a round trip and 1 for a
    // load or store; explicit corners: 8 (measured best on MI355X).
    uint32_t group = (opts && opts->group) ? opts->group : 0;
    if (group && (group > 64 || (group & (group - 1))))
        return fail(TMAP_ERROR_INVALID_VALUE, "group must be a power of two <= 64 (got %u)", group);
    // the band kernel: 2 units a workgroup in every direction (its setup is
    // a few shifts, so short-lived workgroups cost little; measured on the
    // 2 GiB u8, 1 GiB fp32 and ragged bf16 sweeps, 4 units lose 3-8%)
    if (!group && whole16) group = 4u;
    if (!group && lean) group = 2u;
    if (!group && band) group = mode == tmap::kRoundtrip ? 4u : 2u;
    if (band && !lean && mode != tmap::kRoundtrip && !(opts && opts->stages)) stages = 1;
    // explicit corners and the sweeps that run like them: 8 tiles to a
    // walker; a wave-per-box store takes 4.  Where each wave is a workgroup
    // of its own, the wave kernel's stores take 2 and its loads 4 (measured
    // best on MI355X over 10^5 scattered 8 KiB boxes: store 0.539 -> 0.557
    // of peak, load 0.625 -> 0.669 with the packed side's non-temporal hints)
    if (!group && (corners || sweep_corner)) {
        // the corner kernels (one stage, whole-chunk swizzles): about 4 KiB
        // of boxes to a wave, in every direction: one box from 4 KiB up, two
        // of 2 KiB, four of 1 KiB.  Measured on MI355X over the padded 5-D
        // tensor, fraction of 8 TB/s, sweeps and 10^5 random corners: 8 KiB
        // boxes in 4-byte lanes, one box against 2 and 4: load 0.743 / 0.740
        // / 0.735, store 0.674 / 0.667 / 0.659, round trip 0.427 / 0.428 /
        // 0.422 (random); in 16-byte lanes, stores of sweeps 0.583 / 0.544 /
        // 0.504 and of random corners 0.551 / 0.534 / 0.528; 4 KiB boxes, one
        // against the 8 (stores 4) that four-wave workgroups took before:
        // sweeps' round trips 0.605 against 0.404 in 4-byte lanes and 0.419
        // against 0.305 in 16-byte lanes, loads 0.757 against 0.633, random
        // corners 1-8% faster; 2 KiB boxes, two against 1 and 8 (stores 4):
        // sweeps' round trips 0.539 against 0.443 and 0.443, random loads
        // 0.677 against 0.620 and 0.590; 1 KiB boxes, four against 2 and 1:
        // sweeps' round trips 0.354 / 0.314 / 0.247, loads 0.442 / 0.389 /
        // 0.305, random round trips 0.246 / 0.235 / 0.198
        const bool corner = wave_box && stages == 1 && !elemwise && nslot <= 8;
        if (corner) {
            group = 1;
            while (group < 64 && 2 * group * m.box_bytes <= 4096u) group *= 2;
        }
        else if (wave_box && tmap::wave_group(nslot) == 1)
            group = mode == tmap::kStore ? 2u : (mode == tmap::kLoad ? 4u : 8u);
        else
            group = (wave_box && mode == tmap::kStore) ? 4u : 8u;
    }
    // a workgroup that takes one band unit has nothing to overlap in its ring
    if (band && group == 1 && !(opts && opts->stages)) stages = 1;
    if (!group) {
        const uint32_t row = (uint32_t)m.box[0] * m.elem_size;
        group = 2;  // at least two, so that the ring overlaps a fill with a drain
        while (group < 8 && group * row < 512u) group *= 2;
    }
    // default grid: one workgroup per group.  The dispatcher then starts
    // workgroups in tile order as others finish, so the tiles in flight at
    // any moment cover a narrow stretch of the tensor (a few rows of tiles),
    // which HBM serves faster than the spread-out mix that persistent
    // workgroups drift into.  Contiguous runs keep a persistent grid: twice
    // the workgroups that fit in a CU's LDS at once (at most 16 per CU).  In
    // wave-per-box mode the grid counts waves, each walking its own groups,
    // four to a workgroup.
    const bool contiguous = opts && (opts->flags & TMAP_FLAG_CONTIGUOUS);
    const int64_t useful = contiguous ? n_tiles : (n_tiles + group - 1) / group;
    uint32_t grid = (opts && opts->grid_wgs) ? opts->grid_wgs : 0;
    if (!grid && contiguous) {
        uint32_t per_cu = 2 * (dev.lds_per_cu / lds);
        if (per_cu > 16) per_cu = 16;
        if (per_cu < 1) per_cu = 1;
        grid = (uint32_t)dev.cus * per_cu * (wave_box ? (uint32_t)tmap::wave_group(nslot) : 1u);
    }
    // producer-wave mode: a persistent grid of 8 workgroups per CU measured
    // best (each runs a producer wave ahead of four consumer waves, which
    // needs several tiles per workgroup to pay off)
    if (!grid && producer_wave) grid = 8u * (uint32_t)dev.cus;
    if (!grid) grid = (uint32_t)std::min<int64_t>(useful, 1 << 30);
    if ((int64_t)grid > useful) grid = (uint32_t)useful;
    // regions: band-schedule loads and stores deal their units as two
    // interleaved streams (measured on MI355X over three workloads and three
    // placements of the packed buffer: never more than 1% slower than one
    // stream, up to 6% faster); round trips and whole boxes keep one (two
    // cost the 2 GiB round trip about 1%)
    uint32_t regions = (opts && opts->regions) ? opts->regions : 0u;
    if (regions > 64) return fail(TMAP_ERROR_INVALID_VALUE, "regions must be 1..64 (got %u)", regions);
    if (!regions) regions = (band && mode != tmap::kRoundtrip && !(lean && resident_span(m) && !(flags0 & TMAP_FLAG_BAND)))
                                ? 2u
                                : 1u;
    pl.lds = lds;
    pl.nslot = nslot;
    pl.stages = thread_copy ? 0
                : (producer_wave ? 10 + stages : (band ? 20 + stages : (wave_box ? 30 + stages : stages)));
    pl.grid = grid;
    pl.group = group;
    pl.regions = regions;
    return TMAP_SUCCESS;
}

// A sweep whose boxes have extent 1 in a dimension d >= 2, over planes that
// are dense in dimension d - 1 (strides[d] == dims[d-1] * strides[d-1]) and
// a whole number of boxes tall there (dims[d-1] % box[d-1] == 0), is the
// same sweep with dimension d folded into d - 1: a batch of matrices swept
// by 2-D boxes is one taller matrix.  The tiles come in the same order, each
// covering the same elements with the same bounds, so every image and every
// stored byte is unchanged; the folded maps can take the kernels of lower
// ranks (the band kernel takes rank 2).  A round trip's destination folds
// with the source, with the same plane height, or neither folds.
void fold_sweep(MapImpl &m, MapImpl *m2) {
    auto foldable = [](const MapImpl &x, int d) {
        return x.box[d] == 1 && x.dims[d - 1] % x.box[d - 1] == 0 &&
               x.strides[d] == x.dims[d - 1] * x.strides[d - 1] && x.dims[d - 1] * x.dims[d] < (1ull << 31);
    };
    for (int d = 2; d < m.rank;) {
        if (!foldable(m, d) || (m2 && (!foldable(*m2, d) || m2->dims[d - 1] != m.dims[d - 1]))) {
            ++d;
            continue;
        }
        for (MapImpl *x : {&m, m2}) {
            if (!x) continue;
            x->dims[d - 1] *= x->dims[d];
            for (int k = d; k + 1 < x->rank; ++k) {
                x->dims[k] = x->dims[k + 1];
                x->strides[k] = x->strides[k + 1];
                x->box[k] = x->box[k + 1];
            }
            const int last = x->rank - 1;
            x->dims[last] = 1;
            x->strides[last] = 0;
            x->box[last] = 1;
            x->rank = (uint8_t)last;
        }
    }
}

tmap_status check_coords_and_count(const MapImpl &swept, const int32_t *coords, int64_t n_tiles) {
    if (n_tiles < 0) return fail(TMAP_ERROR_INVALID_VALUE, "n_tiles is negative");
    if (!coords && n_tiles != sweep_count(swept))
        return fail(TMAP_ERROR_INVALID_VALUE, "a sweep (coords == NULL) needs n_tiles == %lld, got %lld",
                    (long long)sweep_count(swept), (long long)n_tiles);
    if (coords && ((uintptr_t)coords & 3u))
        return fail(TMAP_ERROR_INVALID_VALUE, "coords must be 4-byte aligned");
    return TMAP_SUCCESS;
}

// ceil(2^32 / d) for 2 <= d <= 2^16, 0 for d == 1: the multiplier that
// divides any n < 2^16 by d with one high multiply (the rounding error of
// the multiplier, below n / 2^32 < 1 / d, never carries past the next
// integer).
uint32_t div_magic(uint32_t d) {
    return d <= 1 ? 0u : (uint32_t)((((uint64_t)1 << 32) + d - 1) / d);
}

// Whether every corner of a box that touches the tensor of map m (corner
// coordinates in (-box, dims) per dimension) is less than 2 GiB from the
// base: then sum_d |c_d| * stride_d < sum_d (dims_d + box_d) * stride_d < 2^31.
// A map with no rank (the unused side of a load or store) qualifies.
bool small_offsets(const tmap::KMap &m) {
    uint64_t s = 0;
    for (int d = 0; d < tmap::kMaxRank; ++d) {
        if (m.strides[d] >= ((uint64_t)1 << 31)) return false;
        s += ((uint64_t)m.dims[d] + m.box[d]) * m.strides[d];
        if (s >= ((uint64_t)1 << 31)) return false;
    }
    return true;
}

// Whether the corner kernels can run in 4-byte lanes (tmap_corner4.h): the
// swept map (a round trip's destination has its box, element size and
// swizzle) has box rows of a power of two from 16 to 256 bytes and at most
// 64 rows to a box.  Then a lane's column is the same in every slot, and
// only a word of 1- or 2-byte elements that the tensor's dimension-0 edge
// cuts needs its elements moved one by one.  A swizzle qualifies when it
// moves whole words within rows (granules of 4 bytes or more: its XOR's
// target bits from bit 2 of the byte offset up to below the row's size)
// with a key of at most 4 bits.  Granules of 4 and 8 bytes, which the other
// kernels move element by element, are whole words here.
bool corner4_fits(int mode, const tmap::KArgs &a) {
    const tmap::KMap &m = mode == tmap::kStore ? a.dst : a.src;
    const uint32_t row = (uint32_t)m.box[0] * m.elem_size;
    if (row < 16u || row > 256u || (row & (row - 1u))) return false;
    if (m.box_bytes / row > 64u) return false;
    if (m.swz_b == 0) return true;
    const uint32_t tb = m.swz_m + log2u(m.elem_size);
    return tb >= 2u && m.swz_b <= 4u && tb + m.swz_b <= log2u(row);
}

void fill_common(tmap::KArgs &a, const MapImpl &swept, const int32_t *coords, int64_t n_tiles) {
    a.coords = coords;
    a.n_tiles = n_tiles;
    for (int d = 0; d < tmap::kMaxRank; ++d) {
        a.tiles[d] = (uint32_t)((swept.dims[d] + swept.box[d] - 1) / swept.box[d]);
        a.sweep_tiles[d] = a.tiles[d];
        a.ubox[d] = swept.box[d];
    }
    a.n_chunks = swept.box_bytes / 16u;
    a.row_chunks = (uint32_t)swept.box[0] * swept.elem_size / 16u;
    a.k_el = 16u / swept.elem_size;
    a.lk_el = log2u(a.k_el);
    a.rc_magic = div_magic(a.row_chunks);
    for (int d = 0; d < tmap::kMaxRank; ++d) a.box_magic[d] = div_magic(swept.box[d]);
    // The direct-to-LDS path moves whole 16-byte chunks; a swizzle that
    // permutes elements inside a chunk needs the element path for every chunk.
    a.elemwise = (swept.swz_b > 0 && ((1u << swept.swz_m) * swept.elem_size) < 16u) ? 1u : 0u;
}

// Choose the schedule of a copy (band or whole boxes, variant, ring, deal)
// and complete the kernel arguments for it, short of the status word.
tmap_status prepare(int mode, const MapImpl &swept, tmap::KArgs &a, const tmap_launch_opts *opts,
                    const DeviceState &dev, Plan &pl) {
    if (opts && (opts->flags & ~kKnownFlags))
        return fail(TMAP_ERROR_INVALID_VALUE, "unknown flag bits 0x%x", opts->flags & ~kKnownFlags);
    uint32_t g = 0, nb = 0, rows = 0;
    const char *why = nullptr;
    const bool lean_maps = band_lean_maps(mode, a);
    const bool band = band_fits(swept, a, mode == tmap::kRoundtrip, opts ? opts->flags : 0u,
                                opts ? opts->band_rows : 0u, g, nb, rows, &why, lean_maps);
    if (why) return fail(TMAP_ERROR_INVALID_VALUE, "%s", why);
    if (band) band_setup(swept, a, g, nb, rows);
    const bool lean = band && lean_maps;
    const bool c4 = !band && corner4_fits(mode, a);
    tmap_status st =
        plan_launch(mode, swept, a.n_tiles, opts, dev, band, lean, a.coords != nullptr, a.elemwise != 0 && !c4, pl);
    if (st != TMAP_SUCCESS) return st;
    pl.band_g = band ? g : 0u;
    pl.band_rows = band ? rows : 0u;
    pl.lean = lean;
    // the spread round trip of tensors without a power-of-two pitch (see
    // kLeanRowsRoundtripSpread): two interleaved streams
    const bool resident = resident_span(swept) && !(opts && (opts->flags & TMAP_FLAG_BAND));
    if (lean && mode == tmap::kRoundtrip && !(opts && opts->regions) && !resident && !pow2_pitches(a))
        pl.regions = 2u;
    // whole boxes on the band kernel: two interleaved streams in every
    // direction (measured on MI355X, 3 stages x 2 units, fraction of 8 TB/s:
    // round trips 0.705 / 0.761 / 0.785 on the 2 GiB u8, 1 GiB fp32 and
    // ragged bf16 sweeps against 0.699 / 0.755 / 0.697 on the generic ring;
    // loads 0.721 / 0.755 / 0.782)
    if (lean && (opts && (opts->flags & TMAP_FLAG_WHOLE_BOX)) && !opts->regions && !resident &&
        !(mode == tmap::kRoundtrip && swept.box_bytes == 16384u))
        pl.regions = 2u;
    // one wave per box with one stage, boxes of at most 8 KiB and a swizzle
    // that moves whole chunks, at explicit corners or over a sweep: the
    // corner kernels, which hold each drained box in registers while the
    // next one loads
    pl.corner = pl.stages == 31 && pl.nslot <= 8 && (!a.elemwise || c4);
    // ... in 4-byte lanes where the maps allow it: no element-by-element
    // patching of chunks the tensor's edge cuts, and a row's offset worked
    // out once per box instead of once per chunk (measured on MI355X over
    // 10^5 scattered 8 KiB fp32 boxes, fraction of 8 TB/s: round trip 0.351
    // -> 0.427, store 0.637 -> 0.674, load 0.733 -> 0.743)
    pl.corner4 = pl.corner && c4;
    // Where each wave is a workgroup of its own (8 KiB boxes), the corner
    // kernels deal the waves as one interleaved stream per XCD, and where a
    // four-wave workgroup's waves take one box at a time (4 KiB boxes), as
    // one per XCD and wave slot: the
    // dispatcher hands workgroups to the XCDs in turn, so workgroups b and
    // b + 8 share an L2 and get neighbouring boxes, and the cache lines that
    // neighbouring boxes share (box rows that do not start on a line) are
    // fetched into one L2 instead of two.  Measured on MI355X, sweeps of the
    // padded 5-D fp32 tensor by three 8 KiB box shapes, fraction of 8 TB/s:
    // round trips 0.732 / 0.736 / 0.729 against 0.447 / 0.528 / 0.450 with
    // one stream, loads 0.871 / 0.886 / 0.879 against 0.621 / 0.716 / 0.629,
    // stores 0.706 / 0.721 / 0.708 against 0.624 / 0.692 / 0.633; the same
    // sweep's corners as a list alike; 10^5 random corners 0.8-1.9% faster.
    // 4 KiB boxes dealt as 32 streams: sweeps' loads 0.877 against 0.757 in
    // 4-byte lanes and 0.697 against 0.641 in 16-byte lanes, round trips
    // 0.637 against 0.606, random corners within 0.5%.  Walkers that take
    // several boxes at a time (smaller boxes) keep one stream: 32 streams
    // cost 2 KiB boxes 1-7%.
    if (pl.corner && !(opts && opts->regions)) {
        const uint32_t wg = (uint32_t)tmap::wave_group(pl.nslot);
        if (wg == 1)
            pl.regions = kXcds;
        else if (pl.group == 1)
            pl.regions = kXcds * wg;
    }
    if (pl.corner4) {
        const uint32_t row = (uint32_t)swept.box[0] * swept.elem_size;
        a.c4_dshift = log2u(row / 4u);
        a.c4_esz = log2u(swept.elem_size);
        a.c4_tb = swept.swz_m + a.c4_esz;
        a.c4_sb = swept.swz_m + swept.swz_s + a.c4_esz;
        a.c4_smask = (1u << swept.swz_b) - 1u;
        a.c4_rows = swept.box_bytes / row;
        pl.lds = tmap::corner4_lds_bytes(mode, pl.nslot);
    } else if (pl.corner) {
        pl.lds = tmap::corner_lds_bytes(mode, pl.nslot);
    }
    a.grid = pl.grid;
    a.regions = pl.regions;
    a.flags = opts ? opts->flags : 0u;
    // A sweep of a tensor larger than the last-level cache streams it once:
    // non-temporal hints on the tensor side too (measured on MI355X over the
    // 2 GiB u8 round trip: 0.744 of peak without them, 0.815 with them).
    if (!a.coords && swept.dims[swept.rank - 1] * swept.strides[swept.rank - 1] >= kBandMinSpan)
        a.flags |= TMAP_FLAG_NONTEMPORAL;
    // each workgroup advances through the tiles by +1 inside a group and by
    // big_step between groups; kernels add the steps' digits with carries
    // instead of dividing per tile
    const bool contiguous = (a.flags & TMAP_FLAG_CONTIGUOUS) != 0;
    a.group = contiguous ? 0u : pl.group;
    a.group_mask = contiguous ? 0xFFFFFFFFu : pl.group - 1u;
    a.big_step = contiguous ? 1 : (int64_t)pl.grid * pl.group - pl.group + 1;
    const int64_t deal = contiguous ? (int64_t)pl.grid : (int64_t)pl.grid * pl.group;
    a.deal_q = a.n_tiles / deal;
    a.deal_r = a.n_tiles % deal;
    uint64_t s1 = 1, sb = (uint64_t)a.big_step;
    for (int d = 0; d < tmap::kMaxRank; ++d) {
        a.step_digits[d] = (uint32_t)(s1 % a.sweep_tiles[d]);
        s1 /= a.sweep_tiles[d];
        a.big_digits[d] = (uint32_t)(sb % a.sweep_tiles[d]);
        sb /= a.sweep_tiles[d];
    }
    a.spin_limit = (opts && opts->spin_limit) ? opts->spin_limit : (1u << 22);
    return TMAP_SUCCESS;
}

// noalloc: the kernels set the no-allocation entry point's static status
// word (tmap_noalloc.hip) instead of the device's library-allocated one,
// which is then neither allocated nor touched.
tmap_status run(int mode, const MapImpl &swept, tmap::KArgs &a, const tmap_launch_opts *opts,
                void *stream, bool noalloc = false) {
    DeviceState *dev = nullptr;
    tmap_status st = device_for_launch(&dev, !noalloc);
    if (st != TMAP_SUCCESS) return st;
    Plan pl;
    st = prepare(mode, swept, a, opts, *dev, pl);
    if (st != TMAP_SUCCESS) return st;
    if (!noalloc) a.status = dev->status + status_slot(*dev, stream);
    if (noalloc) {
        st = tmap::noalloc_scratch(&a.status);
        if (st != TMAP_SUCCESS) return st;
    }
    // maps of rank <= 2 run the variants that only walk two dimensions
    const bool r2 = a.src.rank <= 2 && a.dst.rank <= 2;
    int rc = (int)hipErrorInvalidValue;
    if (pl.corner) {
        const int dims = r2 ? 2 : 5;
        a.off32 = small_offsets(a.src) && small_offsets(a.dst) ? 1u : 0u;
        if (pl.corner4)
            rc = mode == tmap::kLoad    ? tmap::launch_corner4_load(pl.nslot, dims, a, stream)
                 : mode == tmap::kStore ? tmap::launch_corner4_store(pl.nslot, dims, a, stream)
                                        : tmap::launch_corner4_roundtrip(pl.nslot, dims, a, stream);
        else
            rc = mode == tmap::kLoad    ? tmap::launch_corner_load(pl.nslot, dims, a, stream)
                 : mode == tmap::kStore ? tmap::launch_corner_store(pl.nslot, dims, a, stream)
                                        : tmap::launch_corner_roundtrip(pl.nslot, dims, a, stream);
        if (rc != 0) {
            (void)hipGetLastError();
            return fail(TMAP_ERROR_LAUNCH, "kernel launch failed: %s", hipGetErrorString((hipError_t)rc));
        }
        return ok();
    }
    if (pl.lean) {
        const int st = pl.stages - 20;  // band launch codes are 20 + stages
        rc = mode == tmap::kLoad    ? tmap::launch_band_load(st, a, stream)
             : mode == tmap::kStore ? tmap::launch_band_store(st, a, stream)
                                    : tmap::launch_band_roundtrip(st, a, stream);
        if (rc != 0) {
            (void)hipGetLastError();
            return fail(TMAP_ERROR_LAUNCH, "kernel launch failed: %s", hipGetErrorString((hipError_t)rc));
        }
        return ok();
    }
    switch (mode) {
        case tmap::kLoad:
            rc = r2 ? tmap::launch_load_r2(pl.stages, pl.nslot, a, stream)
                    : tmap::launch_load_r5(pl.stages, pl.nslot, a, stream);
            break;
        case tmap::kStore:
            rc = r2 ? tmap::launch_store_r2(pl.stages, pl.nslot, a, stream)
                    : tmap::launch_store_r5(pl.stages, pl.nslot, a, stream);
            break;
        case tmap::kRoundtrip:
            rc = r2 ? tmap::launch_roundtrip_r2(pl.stages, pl.nslot, a, stream)
                    : tmap::launch_roundtrip_r5(pl.stages, pl.nslot, a, stream);
            break;
        default: break;
    }
    if (rc != 0) {
        (void)hipGetLastError();
        return fail(TMAP_ERROR_LAUNCH, "kernel launch failed: %s", hipGetErrorString((hipError_t)rc));
    }
    return ok();
}

// A map of 8-byte elements over a contiguous byte range for the bulk copy:
// rank 1 (dims0 elements, boxes of box0) or rank 2 (rows of dims0 elements
// at a pitch of dims0 * 8 bytes, boxes of box0 x box1).
MapImpl bulk_map(uint64_t base, int rank, uint64_t dims0, uint64_t dims1, uint32_t box0, uint32_t box1) {
    MapImpl m;
    std::memset(&m, 0, sizeof m);
    m.base = base;
    for (int d = 0; d < tmap::kMaxRank; ++d) {
        m.dims[d] = d == 0 ? dims0 : (d == 1 ? dims1 : 1);
        m.box[d] = (uint16_t)(d == 0 ? box0 : (d == 1 ? box1 : 1));
        m.strides[d] = d == 0 ? 8u : (d == 1 && rank > 1 ? dims0 * 8u : 0u);
    }
    m.elem_size = 8;
    m.rank = (uint8_t)rank;
    m.dtype = TMAP_U64;
    m.box_bytes = box0 * box1 * 8u;
    m.span = (uint32_t)(box0 * 8u + (uint64_t)(box1 - 1) * m.strides[1]);
    m.magic = tmap::kMagic;
    return m;
}

tmap_status bulk_launch(const MapImpl &m, const MapImpl &md, const tmap_launch_opts *opts, void *stream) {
    tmap::KArgs a;
    std::memset(&a, 0, sizeof a);
    a.src = tmap::kernel_map(m);
    a.dst = tmap::kernel_map(md);
    fill_common(a, m, nullptr, sweep_count(m));
    return run(tmap::kRoundtrip, m, a, opts, stream);
}

}  // namespace

extern "C" {

const char *tmap_status_string(tmap_status s) {
    switch (s) {
        case TMAP_SUCCESS: return "TMAP_SUCCESS";
        case TMAP_ERROR_INVALID_VALUE: return "TMAP_ERROR_INVALID_VALUE";
        case TMAP_ERROR_UNSUPPORTED_DEVICE: return "TMAP_ERROR_UNSUPPORTED_DEVICE";
        case TMAP_ERROR_LAUNCH: return "TMAP_ERROR_LAUNCH";
        case TMAP_ERROR_TIMEOUT: return "TMAP_ERROR_TIMEOUT";
    }
    return "TMAP_ERROR_UNKNOWN";
}

const char *tmap_last_error_detail(void) { return g_detail.c_str(); }

tmap_status tmap_encode(tmap_t *map, tmap_dtype dtype, uint32_t rank, void *global_address,
                        const uint64_t *global_dim, const uint64_t *global_strides,
                        const uint32_t *box_dim, const uint32_t *element_strides,
                        tmap_swizzle swizzle) {
    if (!map) return fail(TMAP_ERROR_INVALID_VALUE, "map is NULL");
    // the pages' rules
    if (rank < 1 || rank > (uint32_t)tmap::kMaxRank)
        return fail(TMAP_ERROR_INVALID_VALUE, "rank %u is outside 1..5", rank);
    if (!global_dim || !box_dim || (rank > 1 && !global_strides))
        return fail(TMAP_ERROR_INVALID_VALUE, "dims, strides or box array is NULL");
    for (uint32_t d = 0; d < rank; ++d)
        if (box_dim[d] > 256u)
            return fail(TMAP_ERROR_INVALID_VALUE, "box dim %u is %u, above 256", d, box_dim[d]);
    for (uint32_t d = 1; d < rank; ++d)
        if (global_strides[d - 1] % 16u)
            return fail(TMAP_ERROR_INVALID_VALUE, "stride of dim %u (%llu bytes) is not a multiple of 16", d,
                        (unsigned long long)global_strides[d - 1]);
    const uint64_t base = (uint64_t)(uintptr_t)global_address;
    if (base % 16u)
        return fail(TMAP_ERROR_INVALID_VALUE, "global address 0x%llx is not 16-byte aligned",
                    (unsigned long long)base);
    // this library's rules
    if (base == 0) return fail(TMAP_ERROR_INVALID_VALUE, "global address is NULL");
    const int es = elem_size_of(dtype);
    if (!es) return fail(TMAP_ERROR_INVALID_VALUE, "unknown dtype %d", (int)dtype);
    for (uint32_t d = 0; d < rank; ++d)
        if (global_dim[d] < 1 || global_dim[d] > (1ull << 31))
            return fail(TMAP_ERROR_INVALID_VALUE, "dim %u (%llu) is outside [1, 2^31]", d,
                        (unsigned long long)global_dim[d]);
    for (uint32_t d = 0; d < rank; ++d)
        if (box_dim[d] < 1) return fail(TMAP_ERROR_INVALID_VALUE, "box dim %u is 0", d);
    for (uint32_t d = 1; d < rank; ++d)
        if (global_strides[d - 1] == 0 || global_strides[d - 1] >= (1ull << 40))
            return fail(TMAP_ERROR_INVALID_VALUE, "stride of dim %u is 0 or not below 2^40", d);
    if (element_strides)
        for (uint32_t d = 0; d < rank; ++d)
            if (element_strides[d] != 1u)
                return fail(TMAP_ERROR_INVALID_VALUE, "element stride of dim %u is %u; only 1 is supported", d,
                            element_strides[d]);
    if (((uint64_t)box_dim[0] * (uint64_t)es) % 16u)
        return fail(TMAP_ERROR_INVALID_VALUE, "box row of %llu bytes is not a whole number of 16-byte chunks",
                    (unsigned long long)box_dim[0] * es);
    uint64_t n_el = 1;
    for (uint32_t d = 0; d < rank; ++d) n_el *= box_dim[d];
    if (n_el * (uint64_t)es > 65536u)
        return fail(TMAP_ERROR_INVALID_VALUE, "box of %llu bytes is above 64 KiB",
                    (unsigned long long)(n_el * es));
    const uint32_t b = swizzle.b, m = swizzle.m, s = swizzle.s;
    if (b > 8 || m > 16 || s > 16)
        return fail(TMAP_ERROR_INVALID_VALUE, "swizzle (%u,%u,%u) is out of range", b, m, s);
    if (b > 0 && s < b)
        return fail(TMAP_ERROR_INVALID_VALUE, "swizzle shift %u is below its bit count %u", s, b);
    if (b > 0 && (n_el % (1ull << (m + b))) != 0)
        return fail(TMAP_ERROR_INVALID_VALUE, "box of %llu elements is not a multiple of the swizzle period 2^%u",
                    (unsigned long long)n_el, m + b);
    uint64_t span = (uint64_t)box_dim[0] * es;
    for (uint32_t d = 1; d < rank; ++d) span += (uint64_t)(box_dim[d] - 1) * global_strides[d - 1];
    if (span >= (1ull << 31))
        return fail(TMAP_ERROR_INVALID_VALUE, "box footprint of %llu bytes is not below 2 GiB",
                    (unsigned long long)span);

    MapImpl mi;
    std::memset(&mi, 0, sizeof mi);
    mi.base = base;
    for (int d = 0; d < tmap::kMaxRank; ++d) {
        const bool used = (uint32_t)d < rank;
        mi.dims[d] = used ? global_dim[d] : 1;
        mi.strides[d] = !used ? 0 : (d == 0 ? (uint64_t)es : global_strides[d - 1]);
        mi.box[d] = (uint16_t)(used ? box_dim[d] : 1);
    }
    mi.elem_size = (uint8_t)es;
    mi.rank = (uint8_t)rank;
    mi.swz_b = (uint8_t)b;
    mi.swz_m = (uint8_t)m;
    mi.swz_s = (uint8_t)s;
    mi.dtype = (uint8_t)dtype;
    mi.box_bytes = (uint32_t)(n_el * es);
    mi.span = (uint32_t)span;
    mi.magic = tmap::kMagic;
    std::memcpy(map, &mi, sizeof mi);
    return ok();
}

uint64_t tmap_box_bytes(const tmap_t *map) {
    MapImpl m;
    return decode(map, m) ? m.box_bytes : 0;
}

int64_t tmap_sweep_tiles(const tmap_t *map) {
    MapImpl m;
    return decode(map, m) ? sweep_count(m) : -1;
}

uint32_t tmap_band_boxes(const tmap_t *src, const tmap_t *dst, const int32_t *coords,
                         const tmap_launch_opts *opts) {
    MapImpl s, d;
    if (!decode(src, s)) return 0;
    if (dst && !decode(dst, d)) return 0;
    if (opts && (opts->flags & ~kKnownFlags)) return 0;  // the launch would reject them
    if (opts && (opts->flags & TMAP_FLAG_BAND) && (opts->flags & TMAP_FLAG_WHOLE_BOX)) return 0;
    tmap::KArgs a;
    std::memset(&a, 0, sizeof a);
    a.src = tmap::kernel_map(s);
    a.dst = dst ? tmap::kernel_map(d) : a.src;
    fill_common(a, s, coords, 0);
    uint32_t g = 0, nb = 0, rows = 0;
    // a load and a store take the same band (the swept map is either side)
    const bool lean = band_lean_maps(dst ? (int)tmap::kRoundtrip : (int)tmap::kLoad, a);
    return band_fits(s, a, dst != nullptr, opts ? opts->flags : 0u, opts ? opts->band_rows : 0u, g, nb, rows,
                     nullptr, lean)
               ? g
               : 0u;
}

tmap_status tmap_query(const tmap_t *map, tmap_info *out) {
    MapImpl m;
    if (!out || !decode(map, m)) return fail(TMAP_ERROR_INVALID_VALUE, "map is NULL or not encoded");
    std::memset(out, 0, sizeof *out);
    out->global_address = m.base;
    for (int d = 0; d < tmap::kMaxRank; ++d) {
        out->dims[d] = d < m.rank ? m.dims[d] : 0;
        out->strides[d] = d < m.rank ? m.strides[d] : 0;
        out->box[d] = d < m.rank ? m.box[d] : 0;
    }
    out->rank = m.rank;
    out->elem_size = m.elem_size;
    out->dtype = m.dtype;
    out->swizzle.b = m.swz_b;
    out->swizzle.m = m.swz_m;
    out->swizzle.s = m.swz_s;
    return ok();
}

tmap_status tmap_inbounds_elems(const tmap_t *map, const int32_t *host_coords, int64_t n_tiles,
                                uint64_t *out_elems) {
    MapImpl m;
    if (!out_elems || !decode(map, m)) return fail(TMAP_ERROR_INVALID_VALUE, "map is NULL or not encoded");
    tmap_status st = check_coords_and_count(m, host_coords, n_tiles);
    if (st != TMAP_SUCCESS) return st;
    // per tile: product over dimensions of the overlap of [c, c+box) with [0, dim)
    uint64_t total = 0;
    int64_t nt[tmap::kMaxRank];
    for (int d = 0; d < tmap::kMaxRank; ++d) nt[d] = (int64_t)((m.dims[d] + m.box[d] - 1) / m.box[d]);
    for (int64_t t = 0; t < n_tiles; ++t) {
        uint64_t prod = 1;
        int64_t rest = t;
        for (int d = 0; d < tmap::kMaxRank; ++d) {
            int64_t c;
            if (host_coords) {
                c = d < m.rank ? host_coords[t * m.rank + d] : 0;
            } else {
                c = (rest % nt[d]) * (int64_t)m.box[d];
                rest /= nt[d];
            }
            int64_t lo = c < 0 ? 0 : c;
            int64_t hi = c + (int64_t)m.box[d];
            if (hi > (int64_t)m.dims[d]) hi = (int64_t)m.dims[d];
            prod *= hi > lo ? (uint64_t)(hi - lo) : 0u;
        }
        total += prod;
    }
    *out_elems = total;
    return ok();
}

tmap_status tmap_load_tiles(const tmap_t *src, const int32_t *coords, int64_t n_tiles, void *packed_out,
                            const tmap_launch_opts *opts, void *hip_stream) {
    MapImpl s;
    if (!decode(src, s)) return fail(TMAP_ERROR_INVALID_VALUE, "src map is NULL or not encoded");
    tmap_status st = check_coords_and_count(s, coords, n_tiles);
    if (st != TMAP_SUCCESS) return st;
    if (!packed_out || ((uintptr_t)packed_out & 15u))
        return fail(TMAP_ERROR_INVALID_VALUE, "packed_out is NULL or not 16-byte aligned");
    if (n_tiles == 0) return ok();
    if (!coords) fold_sweep(s, nullptr);
    tmap::KArgs a;
    std::memset(&a, 0, sizeof a);
    a.src = tmap::kernel_map(s);
    a.dst = a.src;
    a.packed = (uint8_t *)packed_out;
    fill_common(a, s, coords, n_tiles);
    return run(tmap::kLoad, s, a, opts, hip_stream);
}

tmap_status tmap_store_tiles(const tmap_t *dst, const int32_t *coords, int64_t n_tiles, const void *packed_in,
                             const tmap_launch_opts *opts, void *hip_stream) {
    MapImpl d;
    if (!decode(dst, d)) return fail(TMAP_ERROR_INVALID_VALUE, "dst map is NULL or not encoded");
    tmap_status st = check_coords_and_count(d, coords, n_tiles);
    if (st != TMAP_SUCCESS) return st;
    if (!packed_in || ((uintptr_t)packed_in & 15u))
        return fail(TMAP_ERROR_INVALID_VALUE, "packed_in is NULL or not 16-byte aligned");
    if (n_tiles == 0) return ok();
    if (!coords) fold_sweep(d, nullptr);
    tmap::KArgs a;
    std::memset(&a, 0, sizeof a);
    a.src = tmap::kernel_map(d);
    a.dst = a.src;
    a.packed = (uint8_t *)const_cast<void *>(packed_in);
    fill_common(a, d, coords, n_tiles);
    return run(tmap::kStore, d, a, opts, hip_stream);
}

static tmap_status roundtrip_impl(const tmap_t *src, const tmap_t *dst, const int32_t *coords, int64_t n_tiles,
                                  bool add, float addend, const tmap_launch_opts *opts, void *hip_stream,
                                  bool noalloc = false);

tmap_status tmap_roundtrip(const tmap_t *src, const tmap_t *dst, const int32_t *coords, int64_t n_tiles,
                           const tmap_launch_opts *opts, void *hip_stream) {
    return roundtrip_impl(src, dst, coords, n_tiles, false, 0.0f, opts, hip_stream);
}

tmap_status tmap_roundtrip_add_f32(const tmap_t *src, const tmap_t *dst, const int32_t *coords, int64_t n_tiles,
                                   float addend, const tmap_launch_opts *opts, void *hip_stream) {
    MapImpl s, d;
    if (decode(src, s) && decode(dst, d) && (s.dtype != TMAP_F32 || d.dtype != TMAP_F32))
        return fail(TMAP_ERROR_INVALID_VALUE, "the fp32 update needs TMAP_F32 maps");
    return roundtrip_impl(src, dst, coords, n_tiles, true, addend, opts, hip_stream);
}

tmap_status tmap_bulk_copy(void *dst, const void *src, uint64_t bytes, const tmap_launch_opts *opts,
                           void *hip_stream) {
    if (bytes == 0) return ok();
    if (!dst || !src || ((uintptr_t)dst & 15u) || ((uintptr_t)src & 15u))
        return fail(TMAP_ERROR_INVALID_VALUE, "src and dst must be non-NULL and 16-byte aligned");
    if (bytes % 16u) return fail(TMAP_ERROR_INVALID_VALUE, "bytes (%llu) must be a multiple of 16",
                                 (unsigned long long)bytes);
    const uint64_t lo_d = (uint64_t)(uintptr_t)dst, lo_s = (uint64_t)(uintptr_t)src;
    if (lo_d < lo_s + bytes && lo_s < lo_d + bytes)
        return fail(TMAP_ERROR_INVALID_VALUE, "src and dst ranges overlap");
    uint64_t done = 0;
    // Ranges of 16 MiB and more: the whole 64 KiB rows as a 2-D tensor of
    // 8-byte elements, 8192 to a row, in 16 x 128 boxes (16 KiB), which
    // takes the band schedule like a sweep of that size (a unit is two rows
    // of 8 KiB; measured on MI355X over 2 GiB: 0.76 of peak as 16 KiB tiles
    // in address order, 0.81 as bands; over 16 / 32 / 64 / 128 MiB, 0.531
    // / 0.678 / 0.750 / 0.795 against 0.407 / 0.560 / 0.679 / 0.750 as
    // tiles; 200 MiB 0.655 against 0.660).  At most 2^31 rows a launch.
    constexpr uint64_t kBulkBandMin = 16ull << 20;
    if (bytes >= kBulkBandMin) {
        const uint64_t kRow = 65536, kMaxRows = 1ull << 31;
        while (bytes - done >= kRow) {
            const uint64_t rows = std::min<uint64_t>((bytes - done) / kRow, kMaxRows);
            MapImpl m = bulk_map(lo_s + done, 2, kRow / 8u, rows, 16u, 128u);
            MapImpl md = m;
            md.base = lo_d + done;
            tmap_status st = bulk_launch(m, md, opts, hip_stream);
            if (st != TMAP_SUCCESS) return st;
            done += rows * kRow;
        }
    }
    // The rest: a rank-1 map of 8-byte elements with 16 KiB boxes over each
    // side; ranges above 16 GiB go in several launches so that dims stay
    // within 2^31.
    const uint64_t kBox = 2048, kMaxElems = 1ull << 31;
    while (done < bytes) {
        const uint64_t elems = std::min<uint64_t>((bytes - done) / 8u, kMaxElems);
        MapImpl m = bulk_map(lo_s + done, 1, elems, 1, (uint32_t)kBox, 1);
        MapImpl md = m;
        md.base = lo_d + done;
        tmap_status st = bulk_launch(m, md, opts, hip_stream);
        if (st != TMAP_SUCCESS) return st;
        done += elems * 8u;
    }
    return ok();
}

static tmap_status roundtrip_impl(const tmap_t *src, const tmap_t *dst, const int32_t *coords, int64_t n_tiles,
                                  bool add, float addend, const tmap_launch_opts *opts, void *hip_stream,
                                  bool noalloc) {
    MapImpl s, d;
    if (!decode(src, s)) return fail(TMAP_ERROR_INVALID_VALUE, "src map is NULL or not encoded");
    if (!decode(dst, d)) return fail(TMAP_ERROR_INVALID_VALUE, "dst map is NULL or not encoded");
    // The tile is read back with the layout it was written in: the two maps
    // must agree on element size, rank, box and swizzle ("TMA -- the async
    // bulk copy engine", "The descriptor records the layout, including the
    // swizzle": a swizzle mismatch reads scrambled bytes).
    const bool same_swizzle = s.swz_b == d.swz_b && (s.swz_b == 0 || (s.swz_m == d.swz_m && s.swz_s == d.swz_s));
    if (s.elem_size != d.elem_size || s.rank != d.rank || !same_swizzle ||
        std::memcmp(s.box, d.box, sizeof s.box) != 0)
        return fail(TMAP_ERROR_INVALID_VALUE,
                    "src and dst maps differ in element size, rank, box or swizzle");
    tmap_status st = check_coords_and_count(s, coords, n_tiles);
    if (st != TMAP_SUCCESS) return st;
    if (n_tiles == 0) return ok();
    if (!coords) fold_sweep(s, &d);
    tmap::KArgs a;
    std::memset(&a, 0, sizeof a);
    a.src = tmap::kernel_map(s);
    a.dst = tmap::kernel_map(d);
    a.packed = nullptr;
    a.add_f32 = add ? 1u : 0u;
    a.addend = addend;
    fill_common(a, s, coords, n_tiles);
    return run(tmap::kRoundtrip, s, a, opts, hip_stream, noalloc);
}

tmap_status tmap_roundtrip_noalloc(const tmap_t *src, const tmap_t *dst, const int32_t *coords, int64_t n_tiles,
                                   const tmap_launch_opts *opts, void *hip_stream) {
    return roundtrip_impl(src, dst, coords, n_tiles, false, 0.0f, opts, hip_stream, true);
}

}  // extern "C"

tmap_status tmap::record_failure(tmap_status st, const char *detail) {
    return fail(st, "%s", detail);
}

extern "C" {

tmap_status tmap_plan_launch(tmap_direction direction, const tmap_t *swept, const tmap_t *dst,
                             const int32_t *coords, int64_t n_tiles, const tmap_launch_opts *opts,
                             tmap_plan *out) {
    if (!out) return fail(TMAP_ERROR_INVALID_VALUE, "out is NULL");
    if (direction != TMAP_DIR_LOAD && direction != TMAP_DIR_STORE && direction != TMAP_DIR_ROUNDTRIP)
        return fail(TMAP_ERROR_INVALID_VALUE, "direction must be TMAP_DIR_LOAD, _STORE or _ROUNDTRIP");
    MapImpl s, d;
    if (!decode(swept, s)) return fail(TMAP_ERROR_INVALID_VALUE, "swept map is NULL or not encoded");
    d = s;
    if (direction == TMAP_DIR_ROUNDTRIP) {
        if (!decode(dst, d)) return fail(TMAP_ERROR_INVALID_VALUE, "dst map is NULL or not encoded");
        const bool same_swizzle =
            s.swz_b == d.swz_b && (s.swz_b == 0 || (s.swz_m == d.swz_m && s.swz_s == d.swz_s));
        if (s.elem_size != d.elem_size || s.rank != d.rank || !same_swizzle ||
            std::memcmp(s.box, d.box, sizeof s.box) != 0)
            return fail(TMAP_ERROR_INVALID_VALUE, "src and dst maps differ in element size, rank, box or swizzle");
    }
    tmap_status st = check_coords_and_count(s, coords, n_tiles);
    if (st != TMAP_SUCCESS) return st;
    std::memset(out, 0, sizeof *out);
    if (n_tiles == 0) return ok();  // nothing would be launched
    if (!coords) {
        fold_sweep(s, direction == TMAP_DIR_ROUNDTRIP ? &d : nullptr);
        if (direction != TMAP_DIR_ROUNDTRIP) d = s;
    }
    DeviceState *dev = nullptr;
    st = device_for_launch(&dev, false);
    if (st != TMAP_SUCCESS) return st;
    tmap::KArgs a;
    std::memset(&a, 0, sizeof a);
    a.src = tmap::kernel_map(s);
    a.dst = tmap::kernel_map(d);
    fill_common(a, s, coords, n_tiles);
    Plan pl;
    st = prepare((int)direction, s, a, opts, *dev, pl);
    if (st != TMAP_SUCCESS) return st;
    const int code = pl.stages;
    out->variant = code == 0 ? TMAP_VARIANT_THREAD_COPY
                   : pl.corner4 ? TMAP_VARIANT_CORNER4
                   : pl.corner ? TMAP_VARIANT_CORNER
                   : code > 30 ? TMAP_VARIANT_WAVE_PER_BOX
                   : (code > 10 && code < 20) ? TMAP_VARIANT_PRODUCER_WAVE
                   : pl.lean ? TMAP_VARIANT_BAND
                   : TMAP_VARIANT_RING;
    out->band_boxes = pl.band_g;
    out->band_rows = pl.band_rows;
    out->stages = code == 0 ? 1u : (uint32_t)(code % 10);
    out->slots = (uint32_t)pl.nslot;
    out->group = a.group;
    out->walkers = pl.grid;
    const uint32_t wg = (out->variant == TMAP_VARIANT_WAVE_PER_BOX || out->variant == TMAP_VARIANT_CORNER ||
                         out->variant == TMAP_VARIANT_CORNER4)
                            ? (uint32_t)tmap::wave_group(pl.nslot)
                            : 1u;
    out->workgroups = (pl.grid + wg - 1) / wg;
    out->regions = pl.regions;
    out->lds_bytes = pl.lds;
    out->units = a.n_tiles;
    return ok();
}

tmap_status tmap_sync_status(void *hip_stream) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return fail(TMAP_ERROR_UNSUPPORTED_DEVICE, "no HIP device is available");
    }
    if (hipStreamSynchronize((hipStream_t)hip_stream) != hipSuccess) {
        const hipError_t e = hipGetLastError();
        return fail(TMAP_ERROR_LAUNCH, "stream error: %s", hipGetErrorString(e));
    }
    // this stream's word of the library's table (none if it never launched
    // a copy on this device) and the no-allocation entry point's word
    uint32_t *words[2] = {nullptr, tmap::noalloc_status(dev)};
    {
        std::lock_guard<std::mutex> lk(g_dev_mu);
        const DeviceState &d = g_dev[dev];
        const auto it = d.slot_of.find(hip_stream);
        if (d.status && it != d.slot_of.end()) words[0] = d.status + it->second;
    }
    uint32_t any = 0;
    for (uint32_t *word : words) {
        if (!word) continue;
        uint32_t v = 0;
        if (hipMemcpy(&v, word, 4, hipMemcpyDeviceToHost) != hipSuccess) {
            const hipError_t e = hipGetLastError();
            return fail(TMAP_ERROR_LAUNCH, "cannot read the status word: %s", hipGetErrorString(e));
        }
        if (v) {
            (void)hipMemset(word, 0, 4);
            (void)hipDeviceSynchronize();
            any |= v;
        }
    }
    if (any) return fail(TMAP_ERROR_TIMEOUT, "a readiness wait expired (status 0x%x)", any);
    return ok();
}

}  // extern "C"
