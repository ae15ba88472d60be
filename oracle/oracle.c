/*
 * oracle.c -- plain, slow, single-threaded CPU oracle for the descriptor-driven
 * tiled bulk copy (tensor map + box copy global <-> on-chip tile, XOR swizzle,
 * out-of-bounds zero fill, clipped store).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or load
 * this file: only the test-suite, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or constant with the HIP
 * library; it has its own map struct, its own validator and its own swizzle.
 *
 * Every function computes the plain definition element by element, in the order
 * the pages describe it.  Sources (page title, section):
 *   [TMA-L04]  "TMA -- the async bulk copy engine" (modern_gpu lesson 04)
 *   [GPU-TMA]  "GPU TMA" blog (aicassindra)
 *   [DAY76]    "Day 76: The Tensor Memory Accelerator (TMA)"
 *   [CUTE-TMA] "Understanding TMA loads in CuTe DSL"
 *
 * Readings taken where the pages leave a step open (each also listed in the
 * design notes): swizzle is the XOR bit-field swizzle (B,M,S) applied to
 * tile-local element offsets; out-of-bounds elements read as zero bytes;
 * coordinates are signed and name the box corner, innermost dimension first;
 * a store never writes an out-of-bounds element; tiles are applied in
 * increasing index order (last writer wins).
 *
 * Pins: every function here is checked by the not-GPU tests against values the
 * pages print, closed forms, invariants and an independent array formulation.
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>

#define OR_MAX_RANK 5

/* The oracle's own description of a tensor map.  Dimension 0 is the
 * innermost (contiguous) one; stride[0] is the element size and is implied.
 * [DAY76 "The address arithmetic moves into a descriptor": element type,
 * rank, base, dims, byte strides, box shape; code comment in "An exact round
 * trip": rank 2 has one stride because the innermost dimension is contiguous] */
typedef struct {
    int32_t es;                     /* element size in bytes: 1, 2, 4 or 8        */
    int32_t rank;                   /* 1..5                                        */
    uint64_t dims[OR_MAX_RANK];     /* elements per dimension, innermost first      */
    uint64_t stride[OR_MAX_RANK];   /* bytes; stride[0] == es                       */
    uint32_t box[OR_MAX_RANK];      /* box extent per dimension, innermost first    */
    int32_t swz_b, swz_m, swz_s;    /* XOR swizzle (B bits, base M, shift S)        */
} oracle_map;

/* ---------------------------------------------------------------- validator */
/* Reject codes.  1..4 are the rules the pages state [DAY76 "The address
 * arithmetic moves into a descriptor" and "Pitfalls": box dims at most 256,
 * global strides multiples of 16 bytes, base 16-byte aligned, rank at most 5;
 * one failed rule fails the whole call].  The rest are this library's own
 * rules, needed so that every accepted map has a well-defined result. */
enum {
    OR_OK = 0,
    OR_RANK = 1,          /* rank outside [1,5]                               */
    OR_BOX_MAX = 2,       /* some box dim > 256                               */
    OR_STRIDE_16 = 3,     /* some global stride not a multiple of 16 bytes   */
    OR_BASE_16 = 4,       /* base address not 16-byte aligned                */
    OR_BASE_NULL = 5,     /* base address is 0                               */
    OR_ES = 6,            /* element size not 1, 2, 4 or 8                   */
    OR_DIM_RANGE = 7,     /* some dim outside [1, 2^31] (int32 coordinates)  */
    OR_BOX_ZERO = 8,      /* some box dim is 0                               */
    OR_STRIDE_RANGE = 9,  /* some stride 0 or >= 2^40                        */
    OR_ESTRIDE = 10,      /* some element stride != 1                        */
    OR_ROW_16 = 11,       /* box row (box[0]*es) not a multiple of 16 bytes  */
    OR_BOX_BYTES = 12,    /* box bytes > 65536                               */
    OR_SWZ_RANGE = 13,    /* B > 8, M > 16 or S > 16                         */
    OR_SWZ_SHIFT = 14,    /* B > 0 and S < B (not an involution)            */
    OR_SWZ_TILE = 15,     /* B > 0 and box elements not a multiple of 2^(M+B) */
    OR_SPAN = 16          /* box byte footprint >= 2^31                      */
};

int oracle_validate(int32_t es, int32_t rank, uint64_t base,
                    const uint64_t *dims, const uint64_t *strides_1,
                    const uint32_t *box, const uint32_t *estrides,
                    int32_t b, int32_t m, int32_t s)
{
    int d;
    uint64_t n_elems = 1, span;
    if (rank < 1 || rank > OR_MAX_RANK) return OR_RANK;
    for (d = 0; d < rank; ++d)
        if (box[d] > 256u) return OR_BOX_MAX;
    for (d = 1; d < rank; ++d)
        if (strides_1[d - 1] % 16u != 0) return OR_STRIDE_16;
    if (base % 16u != 0) return OR_BASE_16;
    if (base == 0) return OR_BASE_NULL;
    if (!(es == 1 || es == 2 || es == 4 || es == 8)) return OR_ES;
    for (d = 0; d < rank; ++d)
        if (dims[d] < 1 || dims[d] > (1ull << 31)) return OR_DIM_RANGE;
    for (d = 0; d < rank; ++d)
        if (box[d] < 1) return OR_BOX_ZERO;
    for (d = 1; d < rank; ++d)
        if (strides_1[d - 1] == 0 || strides_1[d - 1] >= (1ull << 40)) return OR_STRIDE_RANGE;
    if (estrides)
        for (d = 0; d < rank; ++d)
            if (estrides[d] != 1u) return OR_ESTRIDE;
    if (((uint64_t)box[0] * (uint64_t)es) % 16u != 0) return OR_ROW_16;
    for (d = 0; d < rank; ++d) n_elems *= box[d];
    if (n_elems * (uint64_t)es > 65536u) return OR_BOX_BYTES;
    if (b < 0 || b > 8 || m < 0 || m > 16 || s < 0 || s > 16) return OR_SWZ_RANGE;
    if (b > 0 && s < b) return OR_SWZ_SHIFT;
    if (b > 0 && (n_elems % (1ull << (m + b))) != 0) return OR_SWZ_TILE;
    /* bytes from the box corner to one past its last element */
    span = (uint64_t)box[0] * (uint64_t)es;
    for (d = 1; d < rank; ++d) span += (uint64_t)(box[d] - 1) * strides_1[d - 1];
    if (span >= (1ull << 31)) return OR_SPAN;
    return OR_OK;
}

/* ------------------------------------------------------------------ swizzle */
/* A swizzle permutes tile-local layout offsets; with zero swizzle bits it is
 * the identity [CUTE-TMA "Describe the memory layout first": make_swizzle and
 * make_composed_layout].  Reading taken: the (B,M,S) XOR bit-field swizzle on
 * element offsets: the B bits that start at bit M+S are XORed into the B bits
 * that start at bit M. */
uint64_t oracle_swizzle(uint64_t e, int32_t b, int32_t m, int32_t s)
{
    uint64_t field;
    if (b == 0) return e;
    field = (e >> (uint64_t)(m + s)) & ((1ull << (uint64_t)b) - 1ull);
    return e ^ (field << (uint64_t)m);
}

/* ------------------------------------------------------------- tile counts */
/* Number of boxes a full sweep covers: per dimension the ceiling of dim/box
 * (boxes that hang past the end are kept and zero-filled), multiplied over
 * dimensions [CUTE-TMA "The work assigned to each block": 132 row strips x 7
 * column tiles = 924 loads for a 64x256 box].  Reading taken: ragged edges
 * round up. */
int64_t oracle_sweep_count(const oracle_map *mp)
{
    int d;
    int64_t n = 1;
    for (d = 0; d < mp->rank; ++d)
        n *= (int64_t)((mp->dims[d] + mp->box[d] - 1) / mp->box[d]);
    return n;
}

/* Box corner of sweep tile t: t is split by mixed radix over the per-dimension
 * tile counts with the innermost tile index varying fastest, and each tile index
 * is scaled by the box extent [CUTE-TMA "Construct the copy atom and coordinate
 * tensor": tile (1,2) has element origin (64,512); block b owns rows
 * [64b,64b+64) and walks column tiles j in order, so t = 7b + j]. */
void oracle_sweep_coords(const oracle_map *mp, int64_t t, int32_t *coords)
{
    int d;
    for (d = 0; d < mp->rank; ++d) {
        int64_t nt = (int64_t)((mp->dims[d] + mp->box[d] - 1) / mp->box[d]);
        coords[d] = (int32_t)((t % nt) * (int64_t)mp->box[d]);
        t /= nt;
    }
}

static void tile_corner(const oracle_map *mp, const int32_t *coords, int64_t t,
                        int32_t *c)
{
    int d;
    if (coords) {
        for (d = 0; d < mp->rank; ++d) c[d] = coords[t * mp->rank + d];
    } else {
        oracle_sweep_coords(mp, t, c);
    }
}

static uint64_t box_elems(const oracle_map *mp)
{
    int d;
    uint64_t n = 1;
    for (d = 0; d < mp->rank; ++d) n *= mp->box[d];
    return n;
}

/* Global position of box element e of the box whose corner is c: split e by
 * mixed radix over the box extents (innermost fastest) and add the corner.
 * Returns 1 when every coordinate lies in [0, dims) and then sets *off to the
 * byte offset sum g_d * stride_d from the base [GPU-TMA "The architecture":
 * the descriptor holds base, dims and strides; DAY76: corner coordinates are
 * element offsets, innermost first]. */
static int element_position(const oracle_map *mp, const int32_t *c, uint64_t e,
                            uint64_t *off)
{
    int d;
    int inb = 1;
    uint64_t rest = e, o = 0;
    for (d = 0; d < mp->rank; ++d) {
        int64_t i = (int64_t)(rest % mp->box[d]);
        int64_t g = (int64_t)c[d] + i;
        rest /= mp->box[d];
        if (g < 0 || (uint64_t)g >= mp->dims[d]) inb = 0;
        else o += (uint64_t)g * mp->stride[d];
    }
    *off = o;
    return inb;
}

/* ------------------------------------------------------------------- load */
/* Load one box into a tile image: every box element is read from the global
 * tensor, or is zero when any coordinate is out of bounds, and lands at its
 * swizzled offset in the tile [TMA-L04 "What the issuing thread actually
 * does" and "The descriptor records the layout, including the swizzle": the
 * engine walks the box and the bytes are permuted as they land; GPU-TMA "Why
 * architecture matters here": out-of-bounds elements are zero-filled]. */
static int load_one_tile(const oracle_map *mp, const uint8_t *src, uint64_t src_len,
                         const int32_t *c, uint8_t *tile)
{
    uint64_t n = box_elems(mp), e, off;
    const uint64_t es = (uint64_t)mp->es;
    for (e = 0; e < n; ++e) {
        uint8_t *dst = tile + oracle_swizzle(e, mp->swz_b, mp->swz_m, mp->swz_s) * es;
        if (element_position(mp, c, e, &off)) {
            if (off + es > src_len) return -1; /* map describes bytes outside the buffer */
            memcpy(dst, src + off, es);
        } else {
            memset(dst, 0, es);
        }
    }
    return 0;
}

/* Store one tile image back: box element e is taken from its swizzled offset
 * in the tile and written to the global tensor only when it is in bounds;
 * out-of-bounds elements are never written [GPU-TMA "End-to-end flow": the
 * store is the same mechanism in reverse; DAY76 "Exercise" and "Solution":
 * the shared-to-global direction with the same shape arguments].  Reading
 * taken: clipped, no byte outside the tensor's bounds is touched. */
static int store_one_tile(const oracle_map *mp, uint8_t *dstb, uint64_t dst_len,
                          const int32_t *c, const uint8_t *tile)
{
    uint64_t n = box_elems(mp), e, off;
    const uint64_t es = (uint64_t)mp->es;
    for (e = 0; e < n; ++e) {
        if (element_position(mp, c, e, &off)) {
            if (off + es > dst_len) return -1;
            memcpy(dstb + off,
                   tile + oracle_swizzle(e, mp->swz_b, mp->swz_m, mp->swz_s) * es, es);
        }
    }
    return 0;
}

/* Bytes in one tile image [DAY76 "The address arithmetic moves into a
 * descriptor": a 64x64 float box is a 16384-byte transfer]. */
uint64_t oracle_box_bytes(const oracle_map *mp)
{
    return box_elems(mp) * (uint64_t)mp->es;
}

/* Load n boxes; tile t's image goes to packed[t*box_bytes ...].  coords is
 * [n][rank] (innermost first) or NULL for a full sweep (then n must equal the
 * sweep count).  Returns 0, or -1 when the map reaches outside src_len. */
int oracle_load_tiles(const oracle_map *mp, const uint8_t *src, uint64_t src_len,
                      const int32_t *coords, int64_t n, uint8_t *packed)
{
    int64_t t;
    int32_t c[OR_MAX_RANK];
    uint64_t bb = oracle_box_bytes(mp);
    for (t = 0; t < n; ++t) {
        tile_corner(mp, coords, t, c);
        if (load_one_tile(mp, src, src_len, c, packed + (uint64_t)t * bb)) return -1;
    }
    return 0;
}

/* Store n tile images from packed back into dst, in increasing t. */
int oracle_store_tiles(const oracle_map *mp, uint8_t *dst, uint64_t dst_len,
                       const int32_t *coords, int64_t n, const uint8_t *packed)
{
    int64_t t;
    int32_t c[OR_MAX_RANK];
    uint64_t bb = oracle_box_bytes(mp);
    for (t = 0; t < n; ++t) {
        tile_corner(mp, coords, t, c);
        if (store_one_tile(mp, dst, dst_len, c, packed + (uint64_t)t * bb)) return -1;
    }
    return 0;
}

/* Round trip: for each tile, load the box from src into a tile image, then
 * store that image through the dst map at the same corner [DAY76 "An exact
 * round trip" with the symmetric write-back of "Exercise"].  The two maps
 * share element size, rank, box and swizzle; their dims and strides may
 * differ.  tile_scratch must hold box_bytes. */
int oracle_roundtrip(const oracle_map *src_map, const uint8_t *src, uint64_t src_len,
                     const oracle_map *dst_map, uint8_t *dst, uint64_t dst_len,
                     const int32_t *coords, int64_t n, uint8_t *tile_scratch)
{
    int64_t t;
    int32_t c[OR_MAX_RANK];
    for (t = 0; t < n; ++t) {
        tile_corner(src_map, coords, t, c);
        if (load_one_tile(src_map, src, src_len, c, tile_scratch)) return -1;
        if (store_one_tile(dst_map, dst, dst_len, c, tile_scratch)) return -1;
    }
    return 0;
}

/* Fused round trip with an fp32 update in on-chip memory: each tile is
 * loaded, every element of the tile image gets + addend in single precision,
 * and the image is stored through dst [DAY76 "An exact round trip": one load
 * per block, +1.0f per element in shared memory, the tile written back; and
 * "Solution": the +1.0f becomes a shared-memory update between the load and
 * the store].  Both maps must have 4-byte elements. */
int oracle_roundtrip_add_f32(const oracle_map *src_map, const uint8_t *src, uint64_t src_len,
                             const oracle_map *dst_map, uint8_t *dst, uint64_t dst_len,
                             const int32_t *coords, int64_t n, float addend, uint8_t *tile_scratch)
{
    int64_t t;
    int32_t c[OR_MAX_RANK];
    uint64_t e, nb = box_elems(src_map);
    if (src_map->es != 4 || dst_map->es != 4) return -1;
    for (t = 0; t < n; ++t) {
        tile_corner(src_map, coords, t, c);
        if (load_one_tile(src_map, src, src_len, c, tile_scratch)) return -1;
        for (e = 0; e < nb; ++e) {
            float f;
            memcpy(&f, tile_scratch + e * 4u, 4);
            f = f + addend;
            memcpy(tile_scratch + e * 4u, &f, 4);
        }
        if (store_one_tile(dst_map, dst, dst_len, c, tile_scratch)) return -1;
    }
    return 0;
}

/* Raw one-dimensional bulk copy of a contiguous byte range [TMA-L04 "The real
 * toolchain": the plain bulk copy moves a contiguous byte range, with no
 * tensor map and no swizzle]. */
void oracle_bulk_copy(uint8_t *dst, const uint8_t *src, uint64_t bytes)
{
    uint64_t i;
    for (i = 0; i < bytes; ++i) dst[i] = src[i];
}

/* Count of in-bounds box elements over n tiles (the bytes a copy must read or
 * write, divided by es). */
uint64_t oracle_inb_elems(const oracle_map *mp, const int32_t *coords, int64_t n)
{
    int64_t t;
    int32_t c[OR_MAX_RANK];
    uint64_t e, total = 0, off, nb = box_elems(mp);
    for (t = 0; t < n; ++t) {
        tile_corner(mp, coords, t, c);
        for (e = 0; e < nb; ++e) total += (uint64_t)element_position(mp, c, e, &off);
    }
    return total;
}
