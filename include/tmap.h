/*
 * tmap.h -- C ABI of libtmap: descriptor-driven tiled bulk copy between HBM
 * and LDS on AMD Instinct MI355X (gfx950).
 *
 * A tensor map describes a strided tensor of up to five dimensions and the
 * box (tile) to cut from it; a copy moves whole boxes at given corners
 * between global memory and an on-chip LDS tile, permutes the bytes with an
 * XOR swizzle as they land, fills out-of-bounds elements with zeros, and
 * stores back with out-of-bounds elements clipped.  The operations follow
 * these pages (cited by title and section):
 *   "TMA -- the async bulk copy engine" (modern_gpu lesson 04)
 *   "GPU TMA" (aicassindra blog)
 *   "Day 76: The Tensor Memory Accelerator (TMA)"
 *   "Understanding TMA loads in CuTe DSL"
 *
 * Conventions for every call:
 *   - Dimensions, box extents and coordinates are innermost (contiguous)
 *     dimension first ("Day 76", "Pitfalls": x, then y).
 *   - Coordinates are int32 element offsets of the box corner and may be
 *     negative or past the end; elements outside [0, dim) read as zero and
 *     are never written.
 *   - Pointers named "device" are HIP device pointers; "host" pointers are
 *     ordinary CPU memory.  The library never takes ownership: a map borrows
 *     its tensor's address, and the caller keeps tensors, coordinate arrays
 *     and packed buffers alive until the stream work has completed.
 *   - The copy calls enqueue on the given HIP stream (NULL = the default
 *     stream) and return without waiting.  Argument errors are reported
 *     synchronously, before anything is launched; a failed call launches
 *     nothing.  n_tiles == 0 is a successful no-op.
 *   - No call allocates device memory per call.  One 1 KiB table of status
 *     words per device (a word for each stream that launches a copy there)
 *     is allocated on first use and kept until process exit.
 *   - The copy calls can be captured into a HIP graph and replayed: once the
 *     device's status words exist (after any earlier launch on it), a launch
 *     only enqueues kernels, with no allocation, copy or memset.
 */
#ifndef TMAP_H
#define TMAP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 128 opaque bytes, sixteen 64-bit words, 64-byte aligned
 * ("Day 76", "The address arithmetic moves into a descriptor": the map is
 * built once on the host and handed to the kernel by value, which treats it
 * as opaque).  Filled only by tmap_encode. */
typedef struct __attribute__((aligned(64))) tmap_t {
    uint64_t opaque[16];
} tmap_t;

typedef enum tmap_status {
    TMAP_SUCCESS = 0,
    TMAP_ERROR_INVALID_VALUE = 1,      /* a rule or argument check failed            */
    TMAP_ERROR_UNSUPPORTED_DEVICE = 2, /* no gfx950 device current                   */
    TMAP_ERROR_LAUNCH = 3,             /* the HIP runtime refused a launch           */
    TMAP_ERROR_TIMEOUT = 4             /* a kernel's bounded readiness wait expired  */
} tmap_status;

/* Only the element size matters to the copy; bytes move verbatim. */
typedef enum tmap_dtype {
    TMAP_U8 = 0, TMAP_I8 = 1, TMAP_U16 = 2, TMAP_F16 = 3, TMAP_BF16 = 4,
    TMAP_U32 = 5, TMAP_I32 = 6, TMAP_F32 = 7, TMAP_U64 = 8, TMAP_F64 = 9
} tmap_dtype;

/* XOR swizzle on tile-local element offsets: the b bits starting at bit m+s
 * are XORed into the b bits starting at bit m.  b == 0 is the identity
 * ("Understanding TMA loads in CuTe DSL", "Describe the memory layout
 * first": make_swizzle(0,4,3) leaves offsets unchanged).  The 128-byte
 * swizzle of a box with 128-byte rows is (3, log2(16/elem_size), 3). */
typedef struct tmap_swizzle {
    uint8_t b, m, s;
} tmap_swizzle;

/* Launch options; pass NULL for the defaults.  Any field left 0 takes its
 * default. */
typedef struct tmap_launch_opts {
    uint32_t stages;      /* LDS ring depth 1..4 (default 2; 1 with explicit corners, for
                             sweeps of whole boxes (on the corner kernels, see
                             TMAP_FLAG_WAVE_PER_BOX, or on the cooperative ring) and
                             when each workgroup takes a single band unit, and for
                             loads and stores on the band schedule outside the band
                             kernel; 3 for every direction of the band kernel,
                             TMAP_VARIANT_BAND, except 4 for round trips of whole
                             16 KiB boxes there)                                         */
    uint32_t grid_wgs;    /* workgroups launched; fewer than there are groups makes each
                             take several (default: one workgroup per group; with
                             TMAP_FLAG_CONTIGUOUS, twice what fits in LDS per CU; in
                             producer-wave mode, 8 per CU)                               */
    uint32_t flags;       /* TMAP_FLAG_* bits; any other bit is TMAP_ERROR_INVALID_VALUE   */
    uint32_t spin_limit;  /* readiness-wait polls before TMAP_ERROR_TIMEOUT (default 2^22) */
    uint32_t group;       /* tiles (band units) dealt to a workgroup at a time, a power of
                             two <= 64 (default: enough boxes side by side to span 512
                             bytes of a row, at least 2 and at most 8; band units: 2 on
                             the band kernel (4 for round trips of whole 16 KiB boxes),
                             else 4 for a round trip and 2 for a load
                             or store; on the corner kernels, TMAP_VARIANT_CORNER and
                             TMAP_VARIANT_CORNER4: about 4 KiB of boxes, 1 for boxes of
                             4 KiB and more, 2 of 2 KiB, 4 of 1 KiB; other explicit
                             corners: 8, for a wave-per-box
                             store 4, and with boxes of 8 KiB and more 4 for a
                             wave-per-box load, 2 for a store and 8 for a round trip) */
    uint32_t regions;     /* 1..64: deal the groups to the grid as that many interleaved
                             streams, each sweeping an equal contiguous stretch of the
                             tiles (workgroup i takes stretch i mod regions; in
                             wave-per-box mode and on the corner kernels, wave i), so
                             that the tiles in flight lie in that many places of the
                             tensor instead of one.  How the addresses in flight fall
                             on the HBM channels and the L2 caches decides which is
                             faster (default on the corner kernels, TMAP_VARIANT_CORNER
                             and TMAP_VARIANT_CORNER4: 8 where a workgroup is one wave
                             (boxes of 8 KiB), 32 where its four waves take one box at a
                             time (4 KiB boxes), so that the workgroups on one of the
                             GPU's 8 XCDs, which share an L2, take neighbouring tiles;
                             else 1; 2 for loads and stores on the band schedule, for
                             band-kernel round trips of tensors whose row pitch is not
                             a power of two, and for whole boxes on the band kernel
                             except round trips of 16 KiB boxes; else 1)               */
    uint32_t band_rows;   /* band schedule: box rows per band, a power of two.  A unit is
                             then 16 KiB / (band_rows * box row bytes) boxes side by
                             side.  Default on the band kernel: 8 for a round trip (2
                             where a tensor's row pitch, the byte stride of dimension
                             1, is not a power of two), 16 for a load or store;
                             elsewhere 2 for a round trip (units 8 KiB wide with
                             128-byte box rows), 8 for a load or store; or the next
                             taller height that fits.  An explicit height that does not fit
                             the box, the swizzle or the sweep (see below) is
                             TMAP_ERROR_INVALID_VALUE where the band schedule applies,
                             and ignored elsewhere                                       */
} tmap_launch_opts;

/* Band schedule.  A sweep (coords == NULL) of boxes whose rows hold 64 to
 * 512 bytes, whose dimension-1 extent is the band height times a power of
 * two and whose higher extents are 1 runs on it when the tensor spans at
 * least 256 MiB (dims[rank-1] * strides[rank-1]), or when TMAP_FLAG_BAND
 * asks for it, or when its maps suit the band kernel (TMAP_VARIANT_BAND:
 * rank <= 2, dimension-0 rows of whole 16-byte chunks); unless
 * TMAP_FLAG_WHOLE_BOX (on the band kernel: units of whole boxes),
 * thread-copy, producer-wave or wave-per-box mode is asked for.  A smaller tensor stays in the last-level cache, where DRAM
 * page locality gains nothing: on the band kernel it then takes the tallest
 * band that fits (often one whole box), 2 stages and one region, and other
 * maps keep whole boxes.  A stage then holds the same band of band_rows rows of the
 * neighbouring boxes that together fill 16 KiB (a "unit"), each box's band
 * being the contiguous piece of that box's swizzled LDS image that it
 * always is.  The swizzle must map each band onto itself (band_rows * box[0]
 * a multiple of 2^(m+b): the swizzle only changes element-offset bits
 * [m, m+b)), and a row of the sweep must hold a whole unit.  Every box's
 * image is unchanged; the tensor is read and written in wide, short pieces
 * (2 rows of 8 KiB, or 8 rows of 2 KiB, by default), which HBM serves faster
 * than narrow rows of tall boxes.  A stage's byte record counts the unit's
 * 16 KiB.  In a round trip, where no image leaves the workgroup, every band
 * is staged in the arrangement of a box's first band. */

/* Tile order: tile index t runs innermost-fastest over the sweep (or over the
 * coords array).  By default the tiles are dealt in groups of `group`
 * consecutive indices, group after group round-robin over the workgroups, so
 * that a workgroup's tiles in flight are neighbours in memory.  With this
 * flag each workgroup instead takes one contiguous run of tiles. */
#define TMAP_FLAG_CONTIGUOUS 0x1u
/* Non-temporal hints on the tensor side of a copy: the loads of a load, the
 * stores of a store, both of a round trip.  They pay when the tensor is
 * larger than the 256 MB last-level cache, and sweeps (coords == NULL) of
 * tensors spanning 256 MiB or more (dims[rank-1] * strides[rank-1]) get
 * them without the flag; on smaller tensors, and on the scattered,
 * partial-line accesses of explicit corners, they cost. */
#define TMAP_FLAG_NONTEMPORAL 0x2u
/* Keep the packed images cached.  By default the packed side of a load or
 * store (the images it writes or reads, each touched once per call) carries
 * non-temporal hints, so that streaming them does not evict the tensor from
 * the caches; a caller that reads the images again right away can keep them
 * with this flag. */
#define TMAP_FLAG_CACHED_PACKED 0x80u
/* Thread-copy mode: the lanes load each box into registers and write it into
 * a single LDS stage themselves, publishing it with a workgroup barrier,
 * instead of direct-to-LDS loads counted by the per-stage byte record
 * ("TMA -- the async bulk copy engine", "Interactive": thread-copy mode).
 * Same results; an A/B baseline.  `stages` is ignored. */
#define TMAP_FLAG_THREAD_COPY 0x4u
/* Producer-wave mode: one wave of a 5-wave workgroup issues every load of a
 * box under a single arrive+expect of its bytes; four consumer waves wait on
 * the stage's byte count, drain it and release it through a second per-stage
 * record ("GPU TMA", "Warp specialization").  Same results.  Needs boxes of
 * at most 32 KiB; `stages` 1 is taken as 2. */
#define TMAP_FLAG_PRODUCER_WAVE 0x8u
/* Wave-per-box mode: each wave walks its own tiles through its own ring of
 * one-box stages (stages 1 or 2), issuing all of a box's direct-to-LDS loads
 * under one arrive+expect of its bytes on its own stage record, and draining
 * the box itself once the record's phase flips.
 * The per-box address and bounds work is done once per box instead of once
 * per wave, and no workgroup barrier is needed.  Same results.  Needs boxes
 * of at most 16 KiB; grid_wgs then counts waves, which run four to a
 * workgroup for boxes under 8 KiB and one to a workgroup for larger boxes
 * (as many one-box rings as fit in a CU's LDS).  Excludes the thread-copy
 * and producer-wave modes, TMAP_FLAG_WHOLE_BOX and the band schedule.  The
 * default for explicit corners of boxes up to 8 KiB (unless stages > 2), and
 * for sweeps of such boxes that the band schedule does not take, on the
 * corner kernels, TMAP_VARIANT_CORNER and TMAP_VARIANT_CORNER4 (unless
 * stages > 1 or the swizzle moves data inside 16-byte chunks). */
#define TMAP_FLAG_WAVE_PER_BOX 0x40u
/* One whole box per stage, even where the band schedule or wave-per-box
 * mode would be the default (for A/B runs, and for a consumer that needs a
 * box's full LDS image at once).  Sweeps whose maps suit the band kernel
 * (TMAP_VARIANT_BAND) with boxes of at most 16 KiB run there, in units of
 * the whole boxes that fill 16 KiB (band_rows = box[1]), 3 stages x 2
 * units, two interleaved streams; other copies run the cooperative ring,
 * the workgroup's four waves sharing each stage. */
#define TMAP_FLAG_WHOLE_BOX 0x10u
/* The band schedule wherever its shape rules allow, whatever the tensor's
 * size.  Excludes TMAP_FLAG_WHOLE_BOX. */
#define TMAP_FLAG_BAND 0x20u
/* Test hook: every wave announces 16 bytes more than it delivers, so a
 * stage never becomes ready and the bounded wait must end the kernel with
 * TMAP_ERROR_TIMEOUT ("Day 76", "Pitfalls": a byte budget that does not match
 * the bytes delivered decouples the wait from the data). */
#define TMAP_FLAG_INJECT_BUDGET_MISMATCH 0x100u
/* Debug aid: before the loads of each stage are issued, the stage is filled
 * with the pattern 0xDEADBEEF, so that a consumer reading it before its byte
 * count completes would copy the pattern out rather than stale bytes of an
 * earlier tile.  Same results as without it when the accounting is right;
 * slower.  Not for the thread-copy mode (it writes the stage itself). */
#define TMAP_FLAG_DEBUG_POISON 0x200u

/*
 * tmap_encode -- validate and pack a tensor map.
 * ("Day 76", "The address arithmetic moves into a descriptor" and
 * "Pitfalls"; "GPU TMA", "The architecture: every piece explained";
 * "TMA -- the async bulk copy engine", "The real toolchain".)
 *
 *   map             out: written only on success
 *   dtype           element type (element size 1, 2, 4 or 8 bytes)
 *   rank            1..5
 *   global_address  device address of element (0,..,0); 16-byte aligned
 *   global_dim      host [rank] elements per dimension, each in [1, 2^31]
 *                   (coordinates are int32)
 *   global_strides  host [rank-1] byte strides of dimensions 1..rank-1,
 *                   multiples of 16, in (0, 2^40); dimension 0 is contiguous
 *   box_dim         host [rank] box extents, each in [1, 256]
 *   element_strides host [rank], all 1, or NULL
 *   swizzle         see tmap_swizzle
 *
 * Rules: the pages' four (box <= 256, strides multiple of 16 bytes, base
 * 16-byte aligned, rank <= 5) plus this library's own: non-NULL base,
 * dims and strides in range, unit element strides, box rows a whole number
 * of 16-byte chunks, at most 64 KiB per box, the box's byte footprint
 * (box[0]*elem + sum (box[d]-1)*stride[d]) below 2 GiB, and for b > 0:
 * b <= 8, m <= 16, s <= 16, s >= b and the box element count a multiple of
 * 2^(m+b).  Any violated rule returns TMAP_ERROR_INVALID_VALUE and leaves
 * *map unmodified; tmap_last_error_detail() names the rule.  Host-only: no
 * GPU is needed.
 */
tmap_status tmap_encode(tmap_t *map, tmap_dtype dtype, uint32_t rank, void *global_address,
                        const uint64_t *global_dim, const uint64_t *global_strides,
                        const uint32_t *box_dim, const uint32_t *element_strides,
                        tmap_swizzle swizzle);

/*
 * tmap_load_tiles -- copy n_tiles boxes from the map's tensor into LDS and
 * write each tile's LDS image to packed_out.
 * ("TMA -- the async bulk copy engine", "What the issuing thread actually
 * does", "The descriptor records the layout, including the swizzle" and
 * "Load completion"; "Day 76", "The address arithmetic moves into a
 * descriptor"; "Understanding TMA loads in CuTe DSL", "The work assigned to
 * each block" and "Issue the load and wait for its phase".)
 *
 *   src        encoded map of the source tensor
 *   coords     device int32 [n_tiles][rank] box corners, or NULL for a full
 *              sweep in which case n_tiles must equal tmap_sweep_tiles(src)
 *              (tile t: innermost tile index fastest)
 *   n_tiles    >= 0
 *   packed_out device, n_tiles * tmap_box_bytes(src) bytes, 16-byte aligned;
 *              tile t's image starts at t * box_bytes; box element e sits at
 *              byte swizzle(e) * elem_size of its image; out-of-bounds
 *              elements are zero
 *   opts       NULL or launch options
 *   hip_stream hipStream_t to enqueue on (NULL = default stream)
 *
 * Each box lands in an LDS stage whose readiness is a per-stage byte count:
 * the stage is read only after all box_bytes (zero-filled bytes included)
 * have arrived, and the count's phase parity flips once per fill.
 */
tmap_status tmap_load_tiles(const tmap_t *src, const int32_t *coords, int64_t n_tiles,
                            void *packed_out, const tmap_launch_opts *opts, void *hip_stream);

/*
 * tmap_store_tiles -- the reverse direction: copy each tile image from
 * packed_in into LDS and store its in-bounds elements to the map's tensor;
 * out-of-bounds elements are never written.
 * ("GPU TMA", "End-to-end flow": the store is the same mechanism in
 * reverse; "Day 76", "Exercise" and "Solution"; "TMA -- the async bulk copy
 * engine", "Store completion".)
 *
 *   dst        encoded map of the destination tensor
 *   coords     device int32 [n_tiles][rank], or NULL for a full sweep
 *   packed_in  device, n_tiles * tmap_box_bytes(dst) bytes, 16-byte aligned,
 *              laid out as tmap_load_tiles writes it
 *   Overlapping boxes that write different bytes to one element leave that
 *   element with one of them (which one is unspecified).
 */
tmap_status tmap_store_tiles(const tmap_t *dst, const int32_t *coords, int64_t n_tiles,
                             const void *packed_in, const tmap_launch_opts *opts,
                             void *hip_stream);

/*
 * tmap_roundtrip -- for each tile: load the box from src into LDS (swizzled,
 * zero-filled) and store it through dst at the same corner (clipped).
 * ("Day 76", "An exact round trip" with the symmetric write-back of
 * "Exercise".)  src and dst must have equal element size, rank, box and
 * swizzle; their dims and strides may differ.  Otherwise as above.
 */
tmap_status tmap_roundtrip(const tmap_t *src, const tmap_t *dst, const int32_t *coords,
                           int64_t n_tiles, const tmap_launch_opts *opts, void *hip_stream);

/*
 * tmap_roundtrip_noalloc -- tmap_roundtrip for callers that cannot allocate
 * device memory: code being captured into a HIP graph on its first launch,
 * serving loops and harnesses that forbid hipMalloc.  Same arguments,
 * checks, schedule and results as tmap_roundtrip; it never allocates or
 * frees device memory, on its first call included.
 *
 * The copy kernels need one 4-byte status word beyond their inputs and
 * outputs, which they set when a bounded readiness wait expires.  Here it is
 * a static device array of the library (4 bytes per device, kept until the
 * process ends) instead of the per-stream words tmap_roundtrip allocates on
 * first use;
 * its need does not grow with the input, so no input size is refused for it.
 * The device address of the array is looked up once per device, on the
 * first call there (a gfx950 device must be current, else
 * TMAP_ERROR_UNSUPPORTED_DEVICE).  Every call on a device shares that
 * device's word: a timeout stays recorded until tmap_sync_status reads and
 * clears it, and calls that overlap on one device (on several streams) race
 * for it, so a timeout cannot be told apart by stream.
 */
tmap_status tmap_roundtrip_noalloc(const tmap_t *src, const tmap_t *dst, const int32_t *coords,
                                   int64_t n_tiles, const tmap_launch_opts *opts, void *hip_stream);

/*
 * tmap_roundtrip_add_f32 -- the round trip with an fp32 update of the tile in
 * on-chip memory: each box is loaded into LDS, every element gets + addend
 * (IEEE single precision, round to nearest even) between the LDS read and the
 * store, and the in-bounds elements are stored through dst.
 * ("Day 76", "An exact round trip": +1.0f per element in shared memory, a
 * bit-exact host check; "Solution": the +1.0f is a shared-memory update
 * between the load and the store.)  Both maps must be TMAP_F32 and agree as
 * for tmap_roundtrip.  NaN inputs give NaN outputs; their payload bits are the
 * hardware's.
 */
tmap_status tmap_roundtrip_add_f32(const tmap_t *src, const tmap_t *dst, const int32_t *coords,
                                   int64_t n_tiles, float addend, const tmap_launch_opts *opts,
                                   void *hip_stream);

/*
 * tmap_bulk_copy -- raw one-dimensional bulk copy of `bytes` contiguous bytes
 * from src to dst through the same LDS ring, with no tensor map and no
 * swizzle ("TMA -- the async bulk copy engine", "The real toolchain": the
 * plain bulk copy moves a contiguous byte range).  src and dst are device
 * pointers, 16-byte aligned, not overlapping; bytes is a multiple of 16
 * (bytes == 0 is a no-op).  From 16 MiB the whole 64 KiB rows are moved as
 * a 2-D sweep of 16 KiB boxes, 128 rows of 128 bytes, on the band schedule
 * described at tmap_launch_opts (HBM serves short, wide bands faster than
 * one long stream of tiles); the rest, and smaller ranges, are moved in
 * 16 KiB tiles of the range, ranges above 16 GiB in several launches.  All
 * launches go on hip_stream.
 */
tmap_status tmap_bulk_copy(void *dst, const void *src, uint64_t bytes, const tmap_launch_opts *opts,
                           void *hip_stream);

/* Bytes of one tile image: product of the box extents times the element
 * size ("Day 76", "An exact round trip": a 64x64 fp32 tile is 16384 bytes,
 * the byte count its barrier expects).  0 for a map never encoded. */
uint64_t tmap_box_bytes(const tmap_t *map);

/* Tiles in a full sweep: product over dimensions of ceil(dim / box), the
 * count a copy with coords == NULL must be given.  ("Understanding TMA loads
 * in CuTe DSL", "The work assigned to each block": the 8448 x 1792 fp16
 * matrix in 64 x 256 boxes is 132 strips of 7 tiles, 924 tile loads; a
 * ragged last tile in a dimension counts as a whole one, its overhang
 * zero-filled as "GPU TMA", "Why architecture matters here" describes.)
 * -1 for a map never encoded. */
int64_t tmap_sweep_tiles(const tmap_t *map);

/* Host-side count of in-bounds box elements over n_tiles corners (host
 * int32 [n_tiles][rank], or NULL for the full sweep): the elements a copy
 * must read or write, since out-of-bounds elements are zero-filled rather
 * than read, and never stored ("GPU TMA", "Why architecture matters here").
 * The copies' algorithmic byte counts are built from it.  Writes
 * *out_elems; TMAP_ERROR_INVALID_VALUE on bad arguments (the checks of the
 * copy calls for n_tiles and corners). */
tmap_status tmap_inbounds_elems(const tmap_t *map, const int32_t *host_coords,
                                int64_t n_tiles, uint64_t *out_elems);

/* Schedule a copy would take (host only, no device needed): the boxes per
 * stage on the band schedule described at tmap_launch_opts (with
 * TMAP_FLAG_WHOLE_BOX on the band kernel, the whole boxes that fill a
 * 16 KiB unit), or 0 when every stage of the generic ring holds one whole
 * box.  (A stage is what "TMA -- the async bulk copy
 * engine", "Why this only pays off inside a pipeline" calls a pipeline
 * stage: one byte-counted buffer of the ring.)  src is the swept map of a load or round trip
 * (of a store: the destination map), dst the round trip's destination map or
 * NULL for a load or store; coords is non-NULL for explicit corners (any non-NULL pointer: it is
 * not read); opts are the launch options the copy would get (NULL: the
 * defaults).  0 for a map never encoded, and for a band_rows or flag bits
 * the launch would reject. */
uint32_t tmap_band_boxes(const tmap_t *src, const tmap_t *dst, const int32_t *coords,
                         const tmap_launch_opts *opts);

/* The schedule a copy would run with: variant, band, ring depth, deal of
 * the tiles to workgroups ("Understanding TMA loads in CuTe DSL", "The work
 * assigned to each block": which tiles each block walks, in what order).
 * No device memory is touched and nothing is launched (the plan depends on
 * the current device's CU count and LDS size, so a gfx950 device must be
 * current, else TMAP_ERROR_UNSUPPORTED_DEVICE).  Arguments as for the copy call of that
 * direction: `swept` is the source map of a load or round trip and the
 * destination map of a store, `dst` the round trip's destination map (NULL
 * otherwise), `coords` non-NULL for explicit corners (not read), `n_tiles`
 * checked as the copy checks it.  Errors are those the copy call would
 * report before launching.  n_tiles == 0 gives an all-zero plan. */
typedef enum tmap_direction { TMAP_DIR_LOAD = 0, TMAP_DIR_STORE = 1, TMAP_DIR_ROUNDTRIP = 2 } tmap_direction;
typedef enum tmap_variant {
    TMAP_VARIANT_RING = 0,          /* workgroup-shared ring of stages (whole boxes or band units) */
    TMAP_VARIANT_THREAD_COPY = 1,   /* TMAP_FLAG_THREAD_COPY                                       */
    TMAP_VARIANT_PRODUCER_WAVE = 2, /* TMAP_FLAG_PRODUCER_WAVE                                     */
    TMAP_VARIANT_WAVE_PER_BOX = 3,  /* TMAP_FLAG_WAVE_PER_BOX, or its default                      */
    TMAP_VARIANT_BAND = 4,          /* band schedule of a sweep whose maps have rank <= 2 and whose
                                       dimension-0 rows are whole 16-byte chunks: the band ring
                                       with per-slot offsets fixed per kernel.  Also batches of
                                       such planes: maps of rank 3 with boxes of extent 1 in
                                       dimension 2, walked plane by plane, and sweeps of higher
                                       rank over dense planes a whole number of boxes tall,
                                       which are the same sweep over one taller matrix          */
    TMAP_VARIANT_CORNER = 5,        /* wave per box with one stage, boxes of at most 8 KiB and a
                                       swizzle that moves whole chunks, at explicit corners or
                                       over a sweep the band schedule does not take: each wave
                                       holds a drained box in registers while the next one
                                       loads                                                   */
    TMAP_VARIANT_CORNER4 = 6        /* the same boxes in 4-byte lanes, for maps with box rows of a
                                       power of two from 16 to 256 bytes, at most 64 rows to a
                                       box, and no swizzle or one that moves whole words (4-byte
                                       granules or larger) within rows: the hardware's bounds
                                       check clips every lane, and only words of 1- or 2-byte
                                       elements that the tensor's edge cuts move element by
                                       element.  Also
                                       sweeps of such maps that the band schedule does not take
                                       (maps of rank 3 and more, among others)                */
} tmap_variant;
typedef struct tmap_plan {
    uint32_t variant;     /* tmap_variant                                                  */
    uint32_t band_boxes;  /* boxes per stage on the band schedule, 0 for one box per stage */
    uint32_t band_rows;   /* box rows per band, 0 without the band schedule                */
    uint32_t stages;      /* LDS ring depth                                                */
    uint32_t slots;       /* 16-byte slots per lane and stage                              */
    uint32_t group;       /* tiles (band units) a walker takes in a row; 0: one contiguous
                             run per walker (TMAP_FLAG_CONTIGUOUS)                         */
    uint32_t walkers;     /* tile sequences: workgroups, or waves in wave-per-box mode     */
    uint32_t workgroups;  /* workgroups launched                                           */
    uint32_t regions;     /* interleaved streams the groups are dealt as                   */
    uint32_t lds_bytes;   /* LDS per workgroup                                             */
    int64_t units;        /* tiles, or band units, dealt to the walkers                    */
} tmap_plan;
tmap_status tmap_plan_launch(tmap_direction direction, const tmap_t *swept, const tmap_t *dst,
                             const int32_t *coords, int64_t n_tiles, const tmap_launch_opts *opts,
                             tmap_plan *out);

/* Decoded fields of an encoded map (for inspection and tests): what "GPU
 * TMA", "The architecture: every piece explained" lists a tensor descriptor
 * as recording -- base address, rank, per-dimension size and stride, tile
 * shape -- plus the element size and the swizzle.  TMAP_ERROR_INVALID_VALUE
 * for a NULL or never encoded map or a NULL out. */
typedef struct tmap_info {
    uint64_t global_address;
    uint64_t dims[5];
    uint64_t strides[5];   /* bytes; strides[0] is the element size */
    uint32_t box[5];
    uint32_t rank;
    uint32_t elem_size;
    uint32_t dtype;
    tmap_swizzle swizzle;
} tmap_info;
tmap_status tmap_query(const tmap_t *map, tmap_info *out);

/* Static text for a status code ("TMAP_ERROR_INVALID_VALUE" and so on; the
 * names follow the driver results the pages quote, "Day 76", "Pitfalls":
 * a failed encode rule gives INVALID_VALUE).  Never NULL. */
const char *tmap_status_string(tmap_status status);

/* Thread-local text describing the last failure of a call on this thread
 * (the rule that failed, the argument that was wrong); "" after success.
 * An addition: the encode of "Day 76", "Pitfalls" reports a failed rule
 * only as INVALID_VALUE, with no word on which rule it was. */
const char *tmap_last_error_detail(void);

/* Wait for hip_stream, then read and clear the status words that kernels
 * set when a bounded readiness wait expires: the current device's word for
 * this stream, and the one word of tmap_roundtrip_noalloc on the device.
 * Returns TMAP_SUCCESS or TMAP_ERROR_TIMEOUT (or TMAP_ERROR_LAUNCH if the
 * stream reports an error).  Each stream that launches copies on a device
 * gets a word of its own there (the first 255 streams; later ones share a
 * word), so a timeout is reported to the stream whose copy it was, and a
 * copy still running on another stream cannot set the word being read and
 * cleared.  tmap_roundtrip_noalloc's word is shared by every stream of the
 * device: its timeouts are reported to whichever stream checks first, and
 * one recorded by a copy on another stream between this call's read and
 * clear goes unreported.
 * ("TMA -- the async bulk copy engine", "Load completion -- the mbarrier and
 * the byte budget": a wait on a byte budget that never completes must end;
 * here it ends the kernel and is reported here.) */
tmap_status tmap_sync_status(void *hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* TMAP_H */
