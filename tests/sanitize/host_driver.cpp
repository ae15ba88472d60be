// host_driver.cpp -- drives the host half of libtmap (tmap_host.cpp, linked
// in directly with the kernel launchers stubbed out) under AddressSanitizer
// and UndefinedBehaviorSanitizer on a machine without a GPU: tmap_encode on
// arbitrary and on valid parameters, every query on each accepted map, the
// band-schedule and launch-plan queries with random options, and every copy
// entry point, which must stop at an argument error or at the device gate.
// Exit status 0 when every call returned one of its documented codes.
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <vector>

#include "../../tiled_tensor_bulk_amd/csrc/tmap_internal.h"

// The launchers live in the device translation units; with no GPU the
// device gate stops every copy before they would be reached.
namespace tmap {
int launch_load_r2(int, int, const KArgs &, void *) { return 1; }
int launch_store_r2(int, int, const KArgs &, void *) { return 1; }
int launch_roundtrip_r2(int, int, const KArgs &, void *) { return 1; }
int launch_load_r5(int, int, const KArgs &, void *) { return 1; }
int launch_store_r5(int, int, const KArgs &, void *) { return 1; }
int launch_roundtrip_r5(int, int, const KArgs &, void *) { return 1; }
int launch_band_load(int, const KArgs &, void *) { return 1; }
int launch_band_store(int, const KArgs &, void *) { return 1; }
int launch_band_roundtrip(int, const KArgs &, void *) { return 1; }
int launch_corner_load(int, int, const KArgs &, void *) { return 1; }
int launch_corner_store(int, int, const KArgs &, void *) { return 1; }
int launch_corner_roundtrip(int, int, const KArgs &, void *) { return 1; }
int launch_corner4_load(int, int, const KArgs &, void *) { return 1; }
int launch_corner4_store(int, int, const KArgs &, void *) { return 1; }
int launch_corner4_roundtrip(int, int, const KArgs &, void *) { return 1; }
uint32_t *noalloc_status(int) { return nullptr; }
tmap_status noalloc_scratch(uint32_t **) { return TMAP_ERROR_LAUNCH; }
}  // namespace tmap

static uint64_t g_state = 0xD1B54A32D192ED03ull;
static uint64_t rnd() {
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    return g_state * 0x2545F4914F6CDD1Dull;
}
static int64_t range(int64_t lo, int64_t hi) { return lo + (int64_t)(rnd() % (uint64_t)(hi - lo + 1)); }

static int bad = 0;
static void expect(bool ok, const char *what) {
    if (!ok && bad++ < 20) std::fprintf(stderr, "unexpected result: %s (%s)\n", what, tmap_last_error_detail());
}

static tmap_launch_opts random_opts() {
    tmap_launch_opts o;
    std::memset(&o, 0, sizeof o);
    o.stages = (uint32_t)range(0, 6);
    o.grid_wgs = (uint32_t)(rnd() & 1 ? 0 : range(1, 100000));
    o.flags = (uint32_t)(rnd() & 0x3FF);
    o.spin_limit = (uint32_t)range(0, 10);
    o.group = (uint32_t)range(0, 130);
    o.regions = (uint32_t)range(0, 70);
    o.band_rows = (uint32_t)range(0, 300);
    return o;
}

int main() {
    int accepted = 0, valid_maps = 0;
    // arbitrary parameters: every call either packs a map or is rejected
    for (int i = 0; i < 200000; ++i) {
        uint64_t dims[6], strides[6];
        uint32_t box[6], es[6];
        for (int d = 0; d < 6; ++d) {
            dims[d] = rnd() >> (rnd() % 64);
            strides[d] = rnd() >> (rnd() % 64);
            box[d] = (uint32_t)(rnd() >> (rnd() % 32 + 32));
            es[d] = (uint32_t)range(0, 2);
        }
        tmap_t m;
        std::memset(&m, 0xAB, sizeof m);
        tmap_swizzle sw = {(uint8_t)range(0, 12), (uint8_t)range(0, 20), (uint8_t)range(0, 20)};
        const tmap_status st =
            tmap_encode(&m, (tmap_dtype)range(-1, 11), (uint32_t)range(0, 7), (void *)(uintptr_t)(rnd() >> (rnd() % 64)),
                        dims, strides, box, (rnd() & 1) ? es : nullptr, sw);
        expect(st == TMAP_SUCCESS || st == TMAP_ERROR_INVALID_VALUE, "encode");
        accepted += st == TMAP_SUCCESS;
    }
    expect(tmap_encode(nullptr, TMAP_U8, 2, (void *)0x1000, nullptr, nullptr, nullptr, nullptr, {0, 0, 0}) ==
               TMAP_ERROR_INVALID_VALUE, "encode NULL");
    // valid maps: queries, schedule queries and copies (stopped at the gate)
    for (int i = 0; i < 20000; ++i) {
        const uint32_t rank = (uint32_t)range(1, 5);
        const int es_log = (int)range(0, 3), es = 1 << es_log;
        const tmap_dtype dt = es == 1 ? TMAP_U8 : es == 2 ? TMAP_F16 : es == 4 ? TMAP_F32 : TMAP_F64;
        uint64_t dims[5], strides[4];
        uint32_t box[5];
        for (uint32_t d = 0; d < rank; ++d) {
            dims[d] = (uint64_t)range(1, d == 0 ? 5000 : 300);
            box[d] = (uint32_t)range(1, d < 2 ? 256 : 4);
        }
        box[0] = (uint32_t)((box[0] * es + 15) / 16 * 16 / es);  // whole 16-byte chunks, still <= 256
        uint64_t s = (dims[0] * es + 15) / 16 * 16;
        for (uint32_t d = 1; d < rank; ++d) {
            strides[d - 1] = s;
            s *= dims[d];
        }
        tmap_swizzle sw = {0, 0, 0};
        if (rnd() & 1) sw = {(uint8_t)range(1, 3), (uint8_t)range(0, 4), (uint8_t)range(3, 5)};
        tmap_t m;
        if (tmap_encode(&m, dt, rank, (void *)0x7F0000000000ull, dims, strides, box, nullptr, sw) != TMAP_SUCCESS)
            continue;
        ++valid_maps;
        expect(tmap_box_bytes(&m) > 0, "box bytes");
        const int64_t sweep = tmap_sweep_tiles(&m);
        expect(sweep >= 1, "sweep tiles");
        tmap_info info;
        expect(tmap_query(&m, &info) == TMAP_SUCCESS && info.rank == rank, "query");
        const int64_t n = range(0, 40);
        std::vector<int32_t> coords((size_t)(n * rank) + 1);
        for (int64_t t = 0; t < n; ++t)
            for (uint32_t d = 0; d < rank; ++d)
                coords[(size_t)(t * rank + d)] = (int32_t)range(-(int64_t)box[d] - 3, (int64_t)dims[d] + 3);
        uint64_t inb = 0;
        expect(tmap_inbounds_elems(&m, coords.data(), n, &inb) == TMAP_SUCCESS, "inbounds");
        if (sweep < 100000) expect(tmap_inbounds_elems(&m, nullptr, sweep, &inb) == TMAP_SUCCESS, "inbounds sweep");
        tmap_launch_opts o = random_opts();
        (void)tmap_band_boxes(&m, (rnd() & 1) ? &m : nullptr, (rnd() & 1) ? coords.data() : nullptr, &o);
        (void)tmap_band_boxes(&m, nullptr, nullptr, nullptr);
        tmap_plan plan;
        const tmap_direction dir = (tmap_direction)range(0, 3);
        const tmap_status ps = tmap_plan_launch(dir, &m, &m, (rnd() & 1) ? coords.data() : nullptr,
                                                (rnd() & 1) ? sweep : n, (rnd() & 1) ? &o : nullptr, &plan);
        expect(ps == TMAP_SUCCESS || ps == TMAP_ERROR_INVALID_VALUE || ps == TMAP_ERROR_UNSUPPORTED_DEVICE,
               "plan");
        void *packed = (void *)0x7E0000000000ull;
        const tmap_status ls = tmap_load_tiles(&m, n ? coords.data() : nullptr, n ? n : sweep, packed, &o, nullptr);
        const tmap_status ss = tmap_store_tiles(&m, nullptr, sweep, packed, &o, nullptr);
        const tmap_status rs = tmap_roundtrip(&m, &m, coords.data(), n, &o, nullptr);
        for (tmap_status x : {ls, ss, rs})
            expect(x == TMAP_SUCCESS || x == TMAP_ERROR_INVALID_VALUE || x == TMAP_ERROR_UNSUPPORTED_DEVICE, "copy");
        if (es == 4) {
            const tmap_status as = tmap_roundtrip_add_f32(&m, &m, coords.data(), n, 1.0f, &o, nullptr);
            expect(as == TMAP_SUCCESS || as == TMAP_ERROR_INVALID_VALUE || as == TMAP_ERROR_UNSUPPORTED_DEVICE,
                   "add");
        }
    }
    for (int i = 0; i < 1000; ++i) {
        const uint64_t bytes = rnd() >> (rnd() % 64);
        const tmap_status bs = tmap_bulk_copy((void *)(uintptr_t)(rnd() >> (rnd() % 64)),
                                              (void *)(uintptr_t)(rnd() >> (rnd() % 64)), bytes, nullptr, nullptr);
        expect(bs == TMAP_SUCCESS || bs == TMAP_ERROR_INVALID_VALUE || bs == TMAP_ERROR_UNSUPPORTED_DEVICE, "bulk");
    }
    for (int s = -2; s < 8; ++s) expect(tmap_status_string((tmap_status)s) != nullptr, "status string");
    expect(tmap_sync_status(nullptr) == TMAP_ERROR_UNSUPPORTED_DEVICE || tmap_sync_status(nullptr) == TMAP_SUCCESS,
           "sync");
    std::printf("host driver: %d arbitrary encodes accepted, %d valid maps exercised, %d unexpected results\n",
                accepted, valid_maps, bad);
    return (bad == 0 && valid_maps > 1000) ? 0 : 1;
}
