/*
 * A plain C99 client of libtmap: it includes only include/tmap.h, links the
 * built shared library, and uses the host-side calls the way a C program
 * would -- encode (the rules of "Day 76: The Tensor Memory Accelerator
 * (TMA)", "Pitfalls"), queries, the in-bounds count and the error
 * reporting.  No device memory is touched: a map only records its base
 * address, so any 16-byte-aligned value serves.  Copies are not launched
 * here (they need a GPU).  Prints "abi client ok" and exits 0 when every
 * check holds; otherwise names the first failed check and exits 1.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "tmap.h"

static int failed = 0;

/* The plan's variant codes are part of the ABI: a C99 compile-time check
 * that they keep their values. */
typedef char variant_codes_keep_their_values[(TMAP_VARIANT_RING == 0 && TMAP_VARIANT_THREAD_COPY == 1 &&
                                              TMAP_VARIANT_PRODUCER_WAVE == 2 && TMAP_VARIANT_WAVE_PER_BOX == 3 &&
                                              TMAP_VARIANT_BAND == 4 && TMAP_VARIANT_CORNER == 5 &&
                                              TMAP_VARIANT_CORNER4 == 6)
                                                 ? 1
                                                 : -1];

#define CHECK(cond)                                                        \
    do {                                                                   \
        if (!(cond)) {                                                     \
            printf("check failed (line %d): %s\n", __LINE__, #cond);       \
            failed = 1;                                                    \
            return;                                                        \
        }                                                                  \
    } while (0)

/* 2 GiB of u8, 65536 bytes wide, 128 x 128 boxes, 128-byte swizzle. */
static void encode_and_query(void) {
    tmap_t map;
    tmap_info info;
    const uint64_t dims[2] = {65536u, 32768u};
    const uint64_t strides[1] = {65536u};
    const uint32_t box[2] = {128u, 128u};
    const tmap_swizzle swz = {3, 4, 3};
    void *base = (void *)(uintptr_t)0x100000u;

    CHECK(tmap_encode(&map, TMAP_U8, 2, base, dims, strides, box, NULL, swz) == TMAP_SUCCESS);
    CHECK(strcmp(tmap_last_error_detail(), "") == 0);
    CHECK(tmap_box_bytes(&map) == 16384u);
    CHECK(tmap_sweep_tiles(&map) == 512 * 256);
    CHECK(tmap_query(&map, &info) == TMAP_SUCCESS);
    CHECK(info.global_address == (uint64_t)(uintptr_t)base);
    CHECK(info.rank == 2 && info.elem_size == 1 && info.dtype == TMAP_U8);
    CHECK(info.dims[0] == 65536u && info.dims[1] == 32768u);
    CHECK(info.strides[0] == 1u && info.strides[1] == 65536u);
    CHECK(info.box[0] == 128u && info.box[1] == 128u);
    CHECK(info.swizzle.b == 3 && info.swizzle.m == 4 && info.swizzle.s == 3);
}

/* A rule violation returns INVALID_VALUE, explains itself and leaves the
 * map as it was. */
static void rejected_encodes(void) {
    tmap_t map, before;
    const uint64_t dims[2] = {1000u, 100u};
    const uint64_t strides[1] = {1024u};
    const uint64_t bad_strides[1] = {1000u};   /* not a multiple of 16 */
    const uint32_t box[2] = {64u, 16u};
    const uint32_t big_box[2] = {257u, 16u};   /* box extent above 256 */
    const tmap_swizzle none = {0, 0, 0};
    void *base = (void *)(uintptr_t)0x2000u;
    void *misaligned = (void *)(uintptr_t)0x2008u;

    memset(&map, 0xA5, sizeof map);
    memcpy(&before, &map, sizeof map);
    CHECK(tmap_encode(&map, TMAP_F32, 2, base, dims, strides, big_box, NULL, none) == TMAP_ERROR_INVALID_VALUE);
    CHECK(strlen(tmap_last_error_detail()) > 0);
    CHECK(memcmp(&map, &before, sizeof map) == 0);
    CHECK(tmap_encode(&map, TMAP_F32, 2, base, dims, bad_strides, box, NULL, none) == TMAP_ERROR_INVALID_VALUE);
    CHECK(tmap_encode(&map, TMAP_F32, 2, misaligned, dims, strides, box, NULL, none) == TMAP_ERROR_INVALID_VALUE);
    CHECK(tmap_encode(&map, TMAP_F32, 6, base, dims, strides, box, NULL, none) == TMAP_ERROR_INVALID_VALUE);
    CHECK(memcmp(&map, &before, sizeof map) == 0);
    CHECK(tmap_sweep_tiles(&map) == -1);
}

/* In-bounds elements of explicit corners, counted per dimension by hand:
 * a 64 x 16 box over a 100 x 70 fp16 tensor. */
static void inbounds_count(void) {
    tmap_t map;
    const uint64_t dims[2] = {100u, 70u};
    const uint64_t strides[1] = {208u};
    const uint32_t box[2] = {64u, 16u};
    const tmap_swizzle none = {0, 0, 0};
    const int32_t corners[4][2] = {
        {0, 0},      /* inside: 64 * 16        */
        {-10, -3},   /* 54 * 13                */
        {50, 60},    /* 50 * 10                */
        {100, 0},    /* past the end in x: 0   */
    };
    uint64_t n = 0;

    CHECK(tmap_encode(&map, TMAP_F16, 2, (void *)(uintptr_t)0x4000u, dims, strides, box, NULL, none) ==
          TMAP_SUCCESS);
    CHECK(tmap_inbounds_elems(&map, &corners[0][0], 4, &n) == TMAP_SUCCESS);
    CHECK(n == 64u * 16u + 54u * 13u + 50u * 10u);
    /* the full sweep covers every element exactly once */
    CHECK(tmap_inbounds_elems(&map, NULL, tmap_sweep_tiles(&map), &n) == TMAP_SUCCESS);
    CHECK(n == 100u * 70u);
    CHECK(tmap_inbounds_elems(&map, NULL, 3, &n) == TMAP_ERROR_INVALID_VALUE);
}

static void status_strings(void) {
    CHECK(strcmp(tmap_status_string(TMAP_SUCCESS), "TMAP_SUCCESS") == 0);
    CHECK(strcmp(tmap_status_string(TMAP_ERROR_INVALID_VALUE), "TMAP_ERROR_INVALID_VALUE") == 0);
    CHECK(strcmp(tmap_status_string(TMAP_ERROR_TIMEOUT), "TMAP_ERROR_TIMEOUT") == 0);
}

/* The launch options and plan are plain C structs a caller fills field by
 * field; the schedule query on the host needs no device. */
static void options_from_c(void) {
    tmap_t map;
    tmap_launch_opts opts;
    const uint64_t dims[2] = {65536u, 32768u};
    const uint64_t strides[1] = {65536u};
    const uint32_t box[2] = {128u, 128u};
    const tmap_swizzle swz = {3, 4, 3};

    CHECK(tmap_encode(&map, TMAP_U8, 2, (void *)(uintptr_t)0x100000u, dims, strides, box, NULL, swz) ==
          TMAP_SUCCESS);
    memset(&opts, 0, sizeof opts);
    opts.flags = TMAP_FLAG_WHOLE_BOX; /* on the band kernel: one 16 KiB box per unit */
    CHECK(tmap_band_boxes(&map, &map, NULL, &opts) == 1u);
    opts.flags = TMAP_FLAG_WHOLE_BOX | TMAP_FLAG_BAND; /* exclusive: the launch would reject them */
    CHECK(tmap_band_boxes(&map, &map, NULL, &opts) == 0u);
    opts.flags = TMAP_FLAG_BAND;
    opts.band_rows = 16;
    CHECK(tmap_band_boxes(&map, NULL, NULL, &opts) == 8u);
}

int main(void) {
    encode_and_query();
    rejected_encodes();
    inbounds_count();
    status_strings();
    options_from_c();
    if (failed) return 1;
    printf("abi client ok\n");
    return 0;
}
