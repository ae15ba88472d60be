// tmap_copy.h -- gfx950 kernel template of the descriptor-driven tiled bulk copy.
// Included by one small .hip file per (copy direction, dimension count), which
// instantiates the variants of that direction.
//
// One kernel template serves the three directions (load to packed images,
// store from packed images, round trip).  Each workgroup (4 waves) walks its
// share of the tiles (by default one group of neighbouring tiles) through a
// ring of S LDS stages -- or, in wave-per-box mode, each wave walks its own
// share through its own ring of one-box stages (four such waves to a
// workgroup for boxes under 8 KiB, one for larger boxes):
//
//   fill    every lane issues one 16-byte direct-to-LDS buffer load per slot
//           it owns (buffer_load_dwordx4 ... lds).  The tensor map sits in
//           scalar registers; per tile only the buffer resource is rebased to
//           the box corner, and each lane reuses the in-box byte offsets it
//           computed once at kernel start.  Chunks that are out of bounds get
//           the offset 0x80000000, past num_records, so the hardware writes
//           zeros into LDS ("GPU TMA", "Why architecture matters here":
//           out-of-bounds elements are zero-filled by the copy itself).
//           The swizzle is applied as the bytes land: lane slot p receives
//           the logical chunk swizzle(p), because a direct-to-LDS load writes
//           lane l's 16 bytes at M0 + 16*l and the XOR swizzle is its own
//           inverse ("TMA -- the async bulk copy engine", "The descriptor
//           records the layout, including the swizzle").
//   land    the wave waits for its own loads (vmcnt), patches chunks that are
//           only partly inside the tensor element by element, and reports
//           the bytes it delivered to the stage's barrier record.
//   ready   a stage is ready when every wave has announced its byte budget and
//           the outstanding byte count is back to zero; the record's phase bit
//           then flips and consumers wait on that parity ("TMA -- the async
//           bulk copy engine", "Load completion -- the mbarrier and the byte
//           budget"; "Understanding TMA loads in CuTe DSL", "Issue the load
//           and wait for its phase").  Consumers read slots another wave
//           loaded, so the byte count, not the wave's own vmcnt, is what
//           makes the stage safe to read.
//   consume load: copy the LDS image out linearly; store / round trip: read
//           each logical chunk back from its swizzled slot and store it,
//           clipped to the destination's bounds.
//   release one s_barrier per tile: no wave refills a stage before every
//           wave finished reading it ("TMA -- the async bulk copy engine",
//           "Why this only pays off inside a pipeline"); a wave that owns
//           its stages only waits for its own reads.
//
// The tile loop is unrolled by S.  The direct-to-LDS loads are issued from
// assembly and each stage waits for exactly its own loads (a vmcnt that
// leaves the later stages' loads and the earlier drains' stores in flight),
// so a stage drains while the next ones fill.  On the band schedule (sweeps
// of boxes with narrow rows) a stage holds the same band of rows of several
// neighbouring boxes instead of one box.  R is the number of dimensions the
// scalar tile arithmetic walks: 2 for maps of rank <= 2, else 5.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "tmap_internal.h"

namespace tmap {
namespace {

typedef __attribute__((address_space(3))) void lds_void_t;

typedef __attribute__((ext_vector_type(4))) int i32x4;

constexpr uint32_t kOob = 0x80000000u;       // offset past every num_records
constexpr int kRsrcWord3 = 0x00020000;       // raw buffer, gfx9 family
constexpr uint64_t kArrive = 1ull << 32;     // one arrival in a barrier record
constexpr uint64_t kPhase = 1ull << 63;      // phase bit of a barrier record
constexpr uint32_t kWaitLgkm = 0xC07F;       // s_waitcnt lgkmcnt(0) only

enum Cls : uint32_t { kZero = 0, kFull = 1, kPart = 2 };

// A buffer range as the direct-to-LDS loads take it: base address and
// number of bytes in range.
struct Src {
    uint64_t base;
    uint32_t nrec;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(uint64_t addr, uint32_t nrec) {
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(addr), 0, (int)nrec, kRsrcWord3);
}

// ---------------------------------------------------------------- LDS DMA
// One wave-wide direct-to-LDS load: lane l's 16 bytes at voff land at LDS
// address lds + 16*l.  Issued from assembly so that the compiler does not
// guard later LDS accesses against it: lacking alias information it would
// put vmcnt(0) before every LDS access after it (the barrier records, the
// consumer's reads), draining the next stage's loads and with them the
// ring's overlap.  The ring waits for its loads itself (wait_vmcnt), and the
// "memory" clobber keeps the compiler's own LDS accesses on their side of it.
// (M0 takes the LDS address and is restored afterwards, since the compiler
// reserves it; the nops cover the M0 -> LDS-DMA hazard and an SGPR just
// written by a VALU.)
__device__ __forceinline__ void dma_lds(uint64_t base, uint32_t nrec, const uint8_t *lds, uint32_t voff, bool nt) {
    // the buffer descriptor and the LDS address are uniform per wave; say so
    // explicitly so they are held in SGPRs
    const i32x4 d = {__builtin_amdgcn_readfirstlane((int)(uint32_t)base),
                     __builtin_amdgcn_readfirstlane((int)((uint32_t)(base >> 32) & 0xFFFFu)),
                     __builtin_amdgcn_readfirstlane((int)nrec), kRsrcWord3};
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)(lds_void_t *)lds);
    uint32_t saved;
    if (nt)
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 4\n\t"
            "buffer_load_dwordx4 %2, %3, 0 offen nt lds\n\ts_nop 0\n\ts_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(m0), "v"(voff), "s"(d)
            : "memory");
    else
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 4\n\t"
            "buffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_nop 0\n\ts_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(m0), "v"(voff), "s"(d)
            : "memory");
}

// The same load with the cache hint fixed at compile time (no branch around
// it) and the LDS destination given as an LDS address.
template <bool NT>
__device__ __forceinline__ void dma_lds_hint(uint64_t base, uint32_t nrec, uint32_t lds_addr, uint32_t voff) {
    const i32x4 d = {__builtin_amdgcn_readfirstlane((int)(uint32_t)base),
                     __builtin_amdgcn_readfirstlane((int)((uint32_t)(base >> 32) & 0xFFFFu)),
                     __builtin_amdgcn_readfirstlane((int)nrec), kRsrcWord3};
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((int)lds_addr);
    uint32_t saved;
    if constexpr (NT)
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 4\n\t"
            "buffer_load_dwordx4 %2, %3, 0 offen nt lds\n\ts_nop 0\n\ts_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(m0), "v"(voff), "s"(d)
            : "memory");
    else
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 4\n\t"
            "buffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_nop 0\n\ts_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(m0), "v"(voff), "s"(d)
            : "memory");
}

// The same in 4-byte lanes: lane l's 4 bytes at voff land at LDS address
// lds_addr + 4*l (zeros when voff is past nrec).
template <bool NT>
__device__ __forceinline__ void dma_lds_dword(uint64_t base, uint32_t nrec, uint32_t lds_addr, uint32_t voff) {
    const i32x4 d = {__builtin_amdgcn_readfirstlane((int)(uint32_t)base),
                     __builtin_amdgcn_readfirstlane((int)((uint32_t)(base >> 32) & 0xFFFFu)),
                     __builtin_amdgcn_readfirstlane((int)nrec), kRsrcWord3};
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((int)lds_addr);
    uint32_t saved;
    if constexpr (NT)
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 4\n\t"
            "buffer_load_dword %2, %3, 0 offen nt lds\n\ts_nop 0\n\ts_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(m0), "v"(voff), "s"(d)
            : "memory");
    else
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 4\n\t"
            "buffer_load_dword %2, %3, 0 offen lds\n\ts_nop 0\n\ts_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(m0), "v"(voff), "s"(d)
            : "memory");
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (expcnt and lgkmcnt untouched).  The counter counts loads (direct-to-LDS
// ones included) and stores alike and retires them in issue order, so after
// issuing k more operations behind a stage's loads, vmcnt(k) guarantees that
// the stage's loads have landed while those k may still be in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    constexpr int n = N > 63 ? 63 : N;
    __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | 0x70 | 0xF00);
    asm volatile("" ::: "memory");
}

// Debug aid (TMAP_FLAG_DEBUG_POISON): fill `blocks` consecutive 1 KiB blocks
// of LDS from `lds`, this lane's 16 bytes of each, with a recognisable
// pattern, and wait for the writes, before direct-to-LDS loads refill them.
// A consumer that read the blocks before the byte count allowed would then
// copy the pattern into its output, where a comparison with the oracle
// finds it, instead of stale bytes of an earlier tile.
constexpr int kPoison = (int)0xDEADBEEFu;

__device__ __forceinline__ void poison_blocks(uint8_t *lds, int blocks, int stride_blocks, uint32_t lane) {
    const i32x4 v = {kPoison, kPoison, kPoison, kPoison};
    for (int j = 0; j < blocks; ++j) *(i32x4 *)(lds + (size_t)j * stride_blocks * kBlockBytes + lane * 16u) = v;
    __builtin_amdgcn_s_waitcnt(kWaitLgkm);
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t swizzle(uint32_t e, uint32_t b, uint32_t m, uint32_t s) {
    return b ? e ^ (((e >> (m + s)) & ((1u << b) - 1u)) << m) : e;
}

// ---------------------------------------------------------------- tile cursor
// Position of a workgroup in its tile sequence.  In a sweep the tile index
// is held as mixed-radix digits over the per-dimension tile counts (innermost
// fastest) and advanced by the workgroup's step with carries, so no tile ever
// costs a division; with explicit corners it is a plain index.
template <int R>
struct Cursor {
    int64_t t;        // tile index
    uint32_t k;       // position in this workgroup's sequence
    uint32_t dig[R];  // sweep: tile index per dimension
};

template <int R>
__device__ __forceinline__ void cursor_init(const KArgs &a, int64_t t, Cursor<R> &cur) {
    cur.t = t;
    cur.k = 0;
    if ((uint64_t)t >> 32 == 0) {
        // the usual case: 32-bit divisions (64-bit ones are long sequences)
        uint32_t rest = (uint32_t)t;
#pragma unroll
        for (int d = 0; d < R; ++d) {
            const uint32_t nt = a.sweep_tiles[d];
            const uint32_t q = rest / nt;
            cur.dig[d] = rest - q * nt;
            rest = q;
        }
        return;
    }
    uint64_t rest = (uint64_t)t;
#pragma unroll
    for (int d = 0; d < R; ++d) {
        const uint64_t nt = a.sweep_tiles[d];
        const uint64_t q = rest / nt;
        cur.dig[d] = (uint32_t)(rest - q * nt);
        rest = q;
    }
}

// Next tile: +1 inside a group, big_step from the last tile of a group.
template <int R>
__device__ __forceinline__ void cursor_advance(const KArgs &a, Cursor<R> &cur) {
    const bool big = (cur.k & a.group_mask) == a.group_mask;
    cur.k += 1;
    cur.t += big ? a.big_step : 1;
    if (a.coords) return;
    uint32_t carry = 0;
#pragma unroll
    for (int d = 0; d < R; ++d) {
        const uint32_t v = cur.dig[d] + (big ? a.big_digits[d] : a.step_digits[d]) + carry;
        carry = v >= a.sweep_tiles[d] ? 1u : 0u;
        cur.dig[d] = carry ? v - a.sweep_tiles[d] : v;
    }
}

// Box corner of the cursor's tile (innermost first).
template <int R>
__device__ __forceinline__ void cursor_corner(const KArgs &a, const KMap &swept, const Cursor<R> &cur,
                                              int32_t c[R]) {
    if (a.coords) {
        // Corners are read through the constant address space: uniform
        // scalar loads (lgkmcnt), so they never wait behind the ring's
        // direct-to-LDS loads (vmcnt).
        typedef const __attribute__((address_space(4))) int32_t const_i32;
        const int r = swept.rank;
        const_i32 *p = (const_i32 *)(a.coords) + cur.t * r;
#pragma unroll
        for (int d = 0; d < R; ++d) c[d] = d < r ? p[d] : 0;
    } else {
#pragma unroll
        for (int d = 0; d < R; ++d) c[d] = (int32_t)(cur.dig[d] * (uint32_t)swept.box[d]);
    }
}

// Byte offset of the box corner from the base, and whether the whole box lies
// inside the tensor (0 <= c <= dims - box in every dimension).
struct Place {
    int64_t off;
    bool interior;
};

template <int R>
__device__ __forceinline__ Place place(const KMap &m, const int32_t c[R]) {
    Place p;
    p.off = 0;
    p.interior = true;
#pragma unroll
    for (int d = 0; d < R; ++d) {
        p.off += (int64_t)c[d] * (int64_t)m.strides[d];
        p.interior = p.interior & (c[d] >= 0) & (c[d] <= m.lim[d]);
    }
    return p;
}

// Per dimension, the window [lo, hi) of box indices inside the tensor.
template <int R>
struct Win {
    uint32_t lo[R];
    uint32_t hi[R];
};

// ext: the extent of the region at corner c per dimension (a box, or a unit
// of the band schedule).
template <int R, typename E>
__device__ __forceinline__ Win<R> window_ext(const KMap &m, const int32_t c[R], const E *ext) {
    Win<R> w;
#pragma unroll
    for (int d = 0; d < R; ++d) {
        const int64_t cd = c[d];
        const int64_t b = ext[d];
        int64_t lo = -cd;
        lo = lo < 0 ? 0 : (lo > b ? b : lo);
        int64_t hi = (int64_t)m.dims[d] - cd;
        hi = hi < lo ? lo : (hi > b ? b : hi);
        w.lo[d] = (uint32_t)lo;
        w.hi[d] = (uint32_t)hi;
    }
    return w;
}

template <int R>
__device__ __forceinline__ Win<R> window(const KMap &m, const int32_t c[R]) {
    return window_ext<R>(m, c, m.box);
}

// Packed box indices of a chunk: w0 = x0 | i1 << 16, w1 = i2 | i3 << 8 | i4 << 16,
// x0 being the first element index of the chunk in dimension 0.
template <int R>
__device__ __forceinline__ uint32_t classify(uint32_t w0, uint32_t w1, const Win<R> &w, uint32_t k_el) {
    const uint32_t x0 = w0 & 0xFFFFu;
    bool row_in = (w0 >> 16) - w.lo[1] < w.hi[1] - w.lo[1];
    if constexpr (R > 2) {
        const uint32_t i2 = w1 & 0xFFu, i3 = (w1 >> 8) & 0xFFu, i4 = w1 >> 16;
        row_in = row_in & (i2 - w.lo[2] < w.hi[2] - w.lo[2]) & (i3 - w.lo[3] < w.hi[3] - w.lo[3]) &
                 (i4 - w.lo[4] < w.hi[4] - w.lo[4]);
    }
    const bool full0 = (x0 >= w.lo[0]) & (x0 + k_el <= w.hi[0]);
    const bool any0 = (x0 < w.hi[0]) & (x0 + k_el > w.lo[0]);
    return !row_in ? kZero : (full0 ? kFull : (any0 ? kPart : kZero));
}

// Box indices of tile-local element e (innermost fastest).
template <int R>
__device__ __forceinline__ void unravel(uint32_t e, const KMap &m, uint32_t i[R]) {
#pragma unroll
    for (int d = 0; d < R; ++d) {
        const uint32_t b = m.box[d];
        const uint32_t q = e / b;
        i[d] = e - q * b;
        e = q;
    }
}

template <int R>
__device__ __forceinline__ bool inside(const uint32_t i[R], const Win<R> &w) {
    bool ok = true;
#pragma unroll
    for (int d = 0; d < R; ++d) ok = ok & (i[d] - w.lo[d] < w.hi[d] - w.lo[d]);
    return ok;
}

template <int R>
__device__ __forceinline__ uint32_t inbox_offset(const uint32_t i[R], const KMap &m) {
    uint64_t o = 0;
#pragma unroll
    for (int d = 0; d < R; ++d) o += (uint64_t)i[d] * m.strides[d];
    return (uint32_t)o;
}

// ---------------------------------------------------------------- cache hints
// Packed images are streamed once per call (written by a load, read by a
// store), so their side of a copy gets non-temporal hints unless
// TMAP_FLAG_CACHED_PACKED keeps them cached; the tensor side gets them with
// TMAP_FLAG_NONTEMPORAL (worth it only when the tensor exceeds the last-level
// cache).  Measured on MI355X: 10^5 scattered 8 KiB boxes of a 103 MB tensor,
// load 0.46 -> 0.62 and store 0.56 -> 0.62 of peak with the packed side
// hinted, and both lower with the tensor side hinted too.
template <int MODE>
__host__ __device__ __forceinline__ bool nontemporal_loads(uint32_t flags) {
    return MODE == kStore ? !(flags & TMAP_FLAG_CACHED_PACKED) : (flags & TMAP_FLAG_NONTEMPORAL) != 0;
}
template <int MODE>
__host__ __device__ __forceinline__ bool nontemporal_stores(uint32_t flags) {
    return MODE == kLoad ? !(flags & TMAP_FLAG_CACHED_PACKED) : (flags & TMAP_FLAG_NONTEMPORAL) != 0;
}

// ---------------------------------------------------------------- barrier record
// One 8-byte LDS word per stage: bits 0..31 outstanding bytes, bits 32..62
// arrivals, bit 63 phase.  The operation that leaves (all waves arrived, zero
// bytes outstanding) resets the counts and flips the phase.
// `arrivals` is the number of arrivals a phase needs.
__device__ __forceinline__ void bar_update(uint64_t *bar, uint64_t delta, uint32_t arrivals = kWaves) {
    const uint64_t old = __hip_atomic_fetch_add(bar, delta, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const uint64_t now = old + delta;
    if ((now & ~kPhase) == ((uint64_t)arrivals << 32))
        __hip_atomic_fetch_add(bar, kPhase - ((uint64_t)arrivals << 32), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
}

// arrive + expect_tx(bytes).  With bytes > 0 this can never complete the
// phase (this wave's own bytes are still outstanding), so it needs no result.
__device__ __forceinline__ void bar_arrive_expect(uint64_t *bar, uint32_t bytes, uint32_t lane,
                                                  uint32_t arrivals = kWaves) {
    if (lane == 0) {
        if (bytes)
            __hip_atomic_fetch_add(bar, kArrive + bytes, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        else
            bar_update(bar, kArrive, arrivals);
    }
}

// complete_tx(bytes): the wave's own loads into the stage have landed
__device__ __forceinline__ void bar_complete(uint64_t *bar, uint32_t bytes, uint32_t lane,
                                             uint32_t arrivals = kWaves) {
    if (lane == 0 && bytes) bar_update(bar, (uint64_t)0 - (uint64_t)bytes, arrivals);
}

// A plain arrival (no bytes), e.g. a consumer releasing a stage.
__device__ __forceinline__ void bar_arrive(uint64_t *bar, uint32_t lane, uint32_t arrivals) {
    if (lane == 0) bar_update(bar, kArrive, arrivals);
}

// Wait until the phase with parity `parity` has completed; false on timeout.
__device__ __forceinline__ bool bar_wait(uint64_t *bar, uint32_t parity, uint32_t limit) {
    for (uint32_t polls = 0;; ++polls) {
        const uint64_t v = __hip_atomic_load(bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if ((uint32_t)(v >> 63) != parity) return true;
        if (polls >= limit) return false;
        __builtin_amdgcn_s_sleep(1);
    }
}

// ---------------------------------------------------------------- element path
// Load the elements of LDS slot p one by one (used for chunks that straddle a
// dimension-0 edge, and for every chunk when the swizzle permutes bytes inside
// a 16-byte chunk).  Out-of-bounds elements read the out-of-range offset and
// land as zero.
template <int R>
__device__ __forceinline__ void load_slot_elements(uint8_t *stage, uint32_t p, const KArgs &a, const KMap &m,
                                                   const Win<R> &w, __amdgpu_buffer_rsrc_t r) {
    const uint32_t es = m.elem_size, k = a.k_el;
    for (uint32_t j = 0; j < k; ++j) {
        const uint32_t s = p * k + j;
        uint32_t i[R];
        unravel<R>(swizzle(s, m.swz_b, m.swz_m, m.swz_s), m, i);
        const uint32_t off = inside<R>(i, w) ? inbox_offset<R>(i, m) : kOob;
        uint8_t *dst = stage + (size_t)s * es;
        if (es == 1) {
            *dst = __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
        } else if (es == 2) {
            *(uint16_t *)dst = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
        } else if (es == 4) {
            *(uint32_t *)dst = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
        } else {
            auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
            *(decltype(v) *)dst = v;
        }
    }
}

// Store the in-bounds elements held in LDS slot p one by one.
template <int R>
__device__ __forceinline__ void store_slot_elements(const uint8_t *stage, uint32_t p, const KArgs &a,
                                                    const KMap &m, const Win<R> &w, __amdgpu_buffer_rsrc_t r,
                                                    bool add) {
    const uint32_t es = m.elem_size, k = a.k_el;
    for (uint32_t j = 0; j < k; ++j) {
        const uint32_t s = p * k + j;
        uint32_t i[R];
        unravel<R>(swizzle(s, m.swz_b, m.swz_m, m.swz_s), m, i);
        if (!inside<R>(i, w)) continue;
        const uint32_t off = inbox_offset<R>(i, m);
        const uint8_t *src = stage + (size_t)s * es;
        if (es == 1) {
            __builtin_amdgcn_raw_buffer_store_b8(*src, r, off, 0, 0);
        } else if (es == 2) {
            __builtin_amdgcn_raw_buffer_store_b16(*(const uint16_t *)src, r, off, 0, 0);
        } else if (es == 4) {
            uint32_t v = *(const uint32_t *)src;
            if (add) v = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, v) + a.addend);
            __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0);
        } else {
            typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
            __builtin_amdgcn_raw_buffer_store_b64(*(const u32x2 *)src, r, off, 0, 0);
        }
    }
}

// Partial chunk of a swizzle whose granule is at least 16 bytes: the slot
// holds the k = 16/ES consecutive dimension-0 elements x0 .. x0+k-1 of one box
// row that lies inside the tensor, starting at in-box byte offset `off`;
// element j is inside iff lo0 <= x0+j < hi0.  Loads land in the slot (the
// out-of-range ones as zero); stores write only the inside elements.
template <int ES>
__device__ __forceinline__ void load_chunk_edge(uint8_t *slot, uint32_t off, uint32_t x0, uint32_t lo0,
                                                uint32_t hi0, __amdgpu_buffer_rsrc_t r) {
    constexpr int K = 16 / ES;
#pragma unroll 4
    for (int j = 0; j < K; ++j) {
        const uint32_t voff = (x0 + j - lo0 < hi0 - lo0) ? off + j * ES : kOob;
        if constexpr (ES == 1) {
            slot[j] = __builtin_amdgcn_raw_buffer_load_b8(r, voff, 0, 0);
        } else if constexpr (ES == 2) {
            ((uint16_t *)slot)[j] = __builtin_amdgcn_raw_buffer_load_b16(r, voff, 0, 0);
        } else if constexpr (ES == 4) {
            ((uint32_t *)slot)[j] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0);
        } else {
            auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0);
            ((decltype(v) *)slot)[j] = v;
        }
    }
}

template <int ES>
__device__ __forceinline__ void store_chunk_edge(const uint8_t *slot, uint32_t off, uint32_t x0, uint32_t lo0,
                                                 uint32_t hi0, __amdgpu_buffer_rsrc_t r, bool add, float addend) {
    constexpr int K = 16 / ES;
#pragma unroll 4
    for (int j = 0; j < K; ++j) {
        if (x0 + j - lo0 >= hi0 - lo0) continue;
        if constexpr (ES == 1) {
            __builtin_amdgcn_raw_buffer_store_b8(slot[j], r, off + j, 0, 0);
        } else if constexpr (ES == 2) {
            __builtin_amdgcn_raw_buffer_store_b16(((const uint16_t *)slot)[j], r, off + j * 2, 0, 0);
        } else if constexpr (ES == 4) {
            uint32_t v = ((const uint32_t *)slot)[j];
            if (add) v = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, v) + addend);
            __builtin_amdgcn_raw_buffer_store_b32(v, r, off + j * 4, 0, 0);
        } else {
            typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
            __builtin_amdgcn_raw_buffer_store_b64(((const u32x2 *)slot)[j], r, off + j * 8, 0, 0);
        }
    }
}

__device__ __forceinline__ void load_chunk_edge_es(uint32_t es, uint8_t *slot, uint32_t off, uint32_t x0,
                                                   uint32_t lo0, uint32_t hi0, __amdgpu_buffer_rsrc_t r) {
    switch (es) {
        case 1: load_chunk_edge<1>(slot, off, x0, lo0, hi0, r); break;
        case 2: load_chunk_edge<2>(slot, off, x0, lo0, hi0, r); break;
        case 4: load_chunk_edge<4>(slot, off, x0, lo0, hi0, r); break;
        default: load_chunk_edge<8>(slot, off, x0, lo0, hi0, r); break;
    }
}

__device__ __forceinline__ void store_chunk_edge_es(uint32_t es, const uint8_t *slot, uint32_t off, uint32_t x0,
                                                    uint32_t lo0, uint32_t hi0, __amdgpu_buffer_rsrc_t r, bool add,
                                                    float addend) {
    switch (es) {
        case 1: store_chunk_edge<1>(slot, off, x0, lo0, hi0, r, false, 0.f); break;
        case 2: store_chunk_edge<2>(slot, off, x0, lo0, hi0, r, false, 0.f); break;
        case 4: store_chunk_edge<4>(slot, off, x0, lo0, hi0, r, add, addend); break;
        default: store_chunk_edge<8>(slot, off, x0, lo0, hi0, r, false, 0.f); break;
    }
}

// The kernel arguments, read again from the argument segment where this is
// called: the compiler cannot tell the address from the one it loaded
// before, so it keeps no register copy of the fields read through it alive
// across a loop.  For slow paths that need fields the hot loop does not.
// The kernels take one argument, the KArgs, at the start of the segment.
__device__ __forceinline__ const KArgs &reread(const KArgs &) {
    typedef const __attribute__((address_space(4))) uint8_t const_u8;
    const_u8 *p = (const_u8 *)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(p));
    return *(const KArgs *)(const uint8_t *)p;
}

// n / d for n < 2^16, given magic = ceil(2^32 / d), or 0 for d == 1.
__device__ __forceinline__ uint32_t div_small(uint32_t n, uint32_t magic) {
    return magic ? __umulhi(n, magic) : n;
}

// In-box byte offset (in map m) and packed indices of logical chunk q.
// The offset wraps modulo 2^32 like every in-box offset (box footprints
// stay below 2 GiB), so the 32-bit products suffice.
template <int R>
__device__ __forceinline__ void chunk_info_of(const KArgs &a, uint32_t q, const KMap &m, uint32_t &off,
                                              uint32_t &w0, uint32_t &w1) {
    const uint32_t row = div_small(q, a.rc_magic);
    const uint32_t x0 = (q - row * a.row_chunks) << a.lk_el;
    uint32_t i[kMaxRank] = {x0, 0, 0, 0, 0};
    uint32_t rest = row;
#pragma unroll
    for (int d = 1; d < R; ++d) {
        const uint32_t qq = div_small(rest, a.box_magic[d]);
        i[d] = rest - qq * m.box[d];
        rest = qq;
    }
    uint32_t o = 0;
#pragma unroll
    for (int d = 0; d < R; ++d) o += i[d] * (uint32_t)m.strides[d];
    off = o;
    w0 = x0 | (i[1] << 16);
    w1 = i[2] | (i[3] << 8) | (i[4] << 16);
}

// Logical chunk held by LDS slot p (the swizzle is its own inverse).
__device__ __forceinline__ uint32_t logical_chunk_of(const KArgs &a, uint32_t p, const KMap &m) {
    return swizzle(p << a.lk_el, m.swz_b, m.swz_m, m.swz_s) >> a.lk_el;
}

// ---------------------------------------------------------------- the kernel
// BAND: the stage holds one unit of the band schedule (see KArgs) instead of
// one box.  W: waves that share a stage (and a tile sequence) -- the whole
// 4-wave workgroup, or 1 in wave-per-box mode, where every wave of the
// workgroup walks its own tiles through its own ring.
template <int MODE, int S, int NSLOT, int R, bool BAND = false, int W = kWaves, int WG = kWaves>
struct Copier {
    static_assert(W == kWaves || W == 1, "a stage is shared by the workgroup or owned by one wave");
    static_assert(!BAND || NSLOT == kBandSlots, "a band stage is 16 KiB");
    const KArgs &a;
    uint32_t lane, wave, my_bytes, parity;
    uint32_t edge;  // bit X: the tile in stage X needs the element path when it lands
    int64_t cnt;
    bool nt, nts;  // non-temporal hints on this copy's loads / stores
    uint64_t *bars;
    uint32_t *abort_flag;
    Cursor<R> fcur;  // next tile to fill
    Cursor<R> ccur;  // next tile to land and consume
    // Corners are read once, one fill ahead (explicit corners cost a scalar
    // memory round trip each), and kept per stage for landing and draining.
    int32_t fc[R];     // corner of the tile under the fill cursor
    int32_t sc[S][R];  // corner of the tile in each stage
    int64_t nfill;     // tiles this workgroup has filled
    // producer slots (the slots this lane fills) and consumer slots (the slots
    // this lane drains: those the next wave filled)
    uint32_t pslot[NSLOT], poff[NSLOT], pw0[NSLOT], pw1[NSLOT];
    uint32_t cslot[NSLOT], coff[NSLOT], cw0[NSLOT], cw1[NSLOT];

    __device__ __forceinline__ Copier(const KArgs &args, uint64_t *b, uint32_t *ab) : a(args), bars(b), abort_flag(ab) {}

    __device__ __forceinline__ const KMap &swept() const { return MODE == kStore ? a.dst : a.src; }

    __device__ __forceinline__ void chunk_info(uint32_t q, const KMap &m, uint32_t &off, uint32_t &w0,
                                               uint32_t &w1) const {
        chunk_info_of<R>(a, q, m, off, w0, w1);
    }

    __device__ __forceinline__ uint32_t logical_chunk(uint32_t p, const KMap &m) const {
        return logical_chunk_of(a, p, m);
    }

    // Region offset and packed indices of the chunk in stage slot p.  In the
    // band schedule, slot p is chunk l = p mod (band chunks) of the band of
    // the unit's box g = p / (band chunks); the swizzle maps every band of a
    // box onto itself, so l's logical chunk is found as in band 0 (the
    // packed side corrects for the band, see band_xor) and the box's place
    // in the unit is added in dimension 0.
    __device__ __forceinline__ void slot_info(uint32_t p, const KMap &m, uint32_t &off, uint32_t &w0,
                                              uint32_t &w1) const {
        if constexpr (BAND) {
            const uint32_t g = p >> a.band_lbc;
            chunk_info(logical_chunk(p & ((1u << a.band_lbc) - 1u), m), m, off, w0, w1);
            const uint32_t x = g * (uint32_t)m.box[0];
            off += x * m.elem_size;
            w0 += x;  // dimension-0 index field: below 2^16
        } else {
            chunk_info(logical_chunk(p, m), m, off, w0, w1);
        }
    }

    // Band j of a box is swizzled like band 0 but for one extra XOR: the
    // swizzle changes only element-offset bits [m, m+b), so with a band of
    // 2^lbe elements (a multiple of 2^(m+b)) the offset j*2^lbe + l goes to
    // j*2^lbe + (swizzle(l) ^ x_j), x_j = swizzle(j*2^lbe) ^ j*2^lbe.  The
    // stage's slots follow band 0's arrangement, so a load writes slot p to
    // image position p ^ x_j of its box's band and a store reads it from
    // there.  Returns x_j in bytes (a multiple of 16: the swizzle moves whole
    // chunks on the direct-to-LDS path); 0 without the band schedule.
    __device__ __forceinline__ uint32_t band_xor(const Cursor<R> &cur) const {
        if constexpr (BAND) {
            const KMap &m = swept();
            const uint32_t jb = (cur.dig[1] & ((1u << a.band_lnb) - 1u)) << a.band_lbe;
            return (swizzle(jb, m.swz_b, m.swz_m, m.swz_s) ^ jb) * m.elem_size;
        } else {
            return 0u;
        }
    }

    // Offset of slot p's chunk in the packed images, from the unit's base.
    __device__ __forceinline__ uint32_t slot_packed(uint32_t p, uint32_t bb) const {
        if constexpr (BAND)
            return (p >> a.band_lbc) * bb + (p & ((1u << a.band_lbc) - 1u)) * 16u;
        else
            return p * 16u;
    }

    // Corner of the region (box or unit) under cursor cur.
    __device__ __forceinline__ void corner(const Cursor<R> &cur, int32_t c[R]) const {
        if constexpr (BAND) {
#pragma unroll
            for (int d = 0; d < R; ++d) c[d] = (int32_t)(cur.dig[d] * a.ubox[d]);
        } else {
            cursor_corner<R>(a, swept(), cur, c);
        }
    }

    // Boxes of the unit under cur that exist (the last unit of a row of the
    // sweep can reach past its last box); 1 without the band schedule.
    __device__ __forceinline__ uint32_t unit_boxes(const Cursor<R> &cur) const {
        if constexpr (BAND) {
            const uint32_t left = a.tiles[0] - cur.dig[0] * a.band_g;
            return left < a.band_g ? left : a.band_g;
        } else {
            return 1u;
        }
    }

    // Buffer resource over the packed images of the region under cur: the
    // box's image, or the unit's bands (records end after the last existing
    // box's band, so chunks of missing boxes read zero and are not written).
    __device__ __forceinline__ Src packed_src(const Cursor<R> &cur, uint32_t bb) const {
        if constexpr (BAND) {
            uint64_t t = 0;
#pragma unroll
            for (int d = R - 1; d >= 1; --d) t = t * a.tiles[d] + (d == 1 ? (cur.dig[1] >> a.band_lnb) : cur.dig[d]);
            t = t * a.tiles[0] + (uint64_t)cur.dig[0] * a.band_g;
            const uint32_t j = cur.dig[1] & ((1u << a.band_lnb) - 1u);
            return Src{(uint64_t)a.packed + t * bb + (uint64_t)j * a.band_bytes,
                       (unit_boxes(cur) - 1u) * bb + a.band_bytes};
        } else {
            return Src{(uint64_t)a.packed + (uint64_t)cur.t * bb, bb};
        }
    }

    __device__ __forceinline__ __amdgpu_buffer_rsrc_t packed_rsrc(const Cursor<R> &cur, uint32_t bb) const {
        const Src p = packed_src(cur, bb);
        return make_rsrc(p.base, p.nrec);
    }
    // Whether the region at corner c lies inside map m: the whole box, or the
    // first `boxes` boxes of a unit (a short last unit of a row is inside
    // when its existing boxes are).
    __device__ __forceinline__ bool inside_map(const KMap &m, const int32_t c[R], const Place &pl,
                                               uint32_t boxes) const {
        if constexpr (BAND) {
            bool in = (c[0] >= 0) & ((int64_t)c[0] + (int64_t)boxes * m.box[0] <= (int64_t)m.dims[0]);
#pragma unroll
            for (int d = 1; d < R; ++d) in = in & (c[d] >= 0) & (c[d] <= m.lim[d]);
            return in;
        } else {
            return pl.interior;
        }
    }

    // Whether stage slot p belongs to one of the first `boxes` boxes of the
    // unit (always, for whole boxes).
    __device__ __forceinline__ bool slot_present(uint32_t p, uint32_t boxes) const {
        if constexpr (BAND)
            return (p >> a.band_lbc) < boxes;
        else
            return true;
    }

    // Whether window w cuts through a 16-byte chunk in dimension 0: only
    // then does some chunk hold elements both inside and outside the tensor
    // and need the element path.  Chunks start at multiples of k_el, so that
    // is when a bound of a non-empty window is not such a multiple.
    __device__ __forceinline__ bool splits_chunks(const Win<R> &w) const {
        bool rows = true;
#pragma unroll
        for (int d = 1; d < R; ++d) rows = rows & (w.lo[d] < w.hi[d]);
        return rows & (w.lo[0] < w.hi[0]) & (((w.lo[0] | w.hi[0]) & (a.k_el - 1u)) != 0u);
    }

    // Window of the region at corner c in map m, limited to the first `boxes`
    // boxes of a unit.
    __device__ __forceinline__ Win<R> win(const KMap &m, const int32_t c[R], uint32_t boxes) const {
        if constexpr (BAND) {
            Win<R> w = window_ext<R>(m, c, a.ubox);
            const uint32_t cap = boxes * (uint32_t)m.box[0];
            w.hi[0] = w.hi[0] < cap ? w.hi[0] : cap;
            w.lo[0] = w.lo[0] < w.hi[0] ? w.lo[0] : w.hi[0];
            return w;
        } else {
            return window<R>(m, c);
        }
    }

    // vwave >= 0 makes this lane act as wave vwave of a 4-wave workgroup
    // (the consumers of the producer-wave variant use it).
    __device__ __forceinline__ void setup(int vwave = -1) {
        lane = threadIdx.x & 63u;
        const uint32_t hw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave in the workgroup
        wave = vwave >= 0 ? (uint32_t)vwave : (W == 1 ? 0u : hw);
        nt = nontemporal_loads<MODE>(a.flags);
        nts = nontemporal_stores<MODE>(a.flags);
        parity = 0;
        edge = 0;
        // the tile sequences are dealt to a.grid walkers: the workgroups, or
        // in wave-per-box mode the waves (wave w of workgroup b, of WG waves
        // each, is walker WG*b + w; walkers past a.grid in the last
        // workgroup take no tiles).
        // Walker index -> place in the deal: with R regions the first
        // R*(grid/R) walkers are dealt as R interleaved streams, walker i
        // taking the next place of stretch i mod R (a permutation of
        // 0..grid-1, so every place is still taken once)
        int64_t g = W == 1 ? (int64_t)blockIdx.x * WG + hw : (int64_t)blockIdx.x;
        const bool walker = g < (int64_t)a.grid;
        if (a.regions > 1) {
            const uint32_t per = a.grid / a.regions;
            if ((uint32_t)g < per * a.regions) g = (int64_t)((uint32_t)g % a.regions) * per + (uint32_t)g / a.regions;
        }
        int64_t t0;
        if (a.group == 0) {
            // one contiguous run per workgroup
            const int64_t base = a.deal_q, rem = a.deal_r;
            cnt = base + (g < rem ? 1 : 0);
            t0 = g * base + (g < rem ? g : rem);
        } else {
            // groups of Q consecutive tiles, dealt round-robin: workgroup g
            // takes tiles [g*Q, g*Q+Q) of every round of grid*Q tiles
            const int64_t Q = a.group;
            int64_t last = a.deal_r - g * Q;
            last = last < 0 ? 0 : (last > Q ? Q : last);
            cnt = a.deal_q * Q + last;
            t0 = g * Q;
        }
        if (!walker) cnt = 0;
        cursor_init<R>(a, t0, fcur);
        ccur = fcur;
        nfill = 0;
        if (cnt > 0) corner(fcur, fc);
        my_bytes = 0;
        const uint32_t cw = (wave + 1) % W;
#pragma unroll
        for (int j = 0; j < NSLOT; ++j) {
            const uint32_t pb = (uint32_t)(j * W) + wave;
            const int32_t valid = (int32_t)a.n_chunks - (int32_t)(pb * 64u);
            my_bytes += 16u * (uint32_t)(valid <= 0 ? 0 : (valid >= 64 ? 64 : valid));
            pslot[j] = pb * 64u + lane;
            cslot[j] = ((uint32_t)(j * W) + cw) * 64u + lane;
            poff[j] = pw0[j] = pw1[j] = 0;
            coff[j] = cw0[j] = cw1[j] = 0;
            // the packed side of a copy reads / writes the slots' image
            // offsets; the tensor side their region offsets
            if (MODE == kStore) poff[j] = slot_packed(pslot[j], a.dst.box_bytes);
            if (MODE == kLoad) coff[j] = slot_packed(cslot[j], a.src.box_bytes);
            if (!a.elemwise) {
                if (MODE != kStore && pslot[j] < a.n_chunks) slot_info(pslot[j], a.src, poff[j], pw0[j], pw1[j]);
                if (MODE != kLoad && cslot[j] < a.n_chunks) slot_info(cslot[j], a.dst, coff[j], cw0[j], cw1[j]);
                // a wave that drains its own slots in a round trip (whose
                // maps share box and swizzle) finds the same box indices on
                // both sides: hold them once
                if (W == 1 && MODE == kRoundtrip) {
                    cw0[j] = pw0[j];
                    cw1[j] = pw1[j];
                }
            }
        }
    }

    template <typename T>
    __device__ __forceinline__ void dma(const Src &src, T *stage, int j, uint32_t voff) const {
        dma_lds(src.base, src.nrec, stage + (j * W + wave) * kBlockBytes, voff, nt);
    }

    // Issue the loads of the tile under the fill cursor into stage XF, then
    // move the cursor on.
    template <int XF>
    __device__ __forceinline__ void fill(uint8_t *stage, uint64_t *bar) {
        const uint32_t budget = my_bytes + ((a.flags & TMAP_FLAG_INJECT_BUDGET_MISMATCH) ? 16u : 0u);
        if (a.flags & TMAP_FLAG_DEBUG_POISON) poison_blocks(stage + wave * kBlockBytes, NSLOT, W, lane);
        bar_arrive_expect(bar, budget, lane, W);
        int32_t c[R];
#pragma unroll
        for (int d = 0; d < R; ++d) c[d] = sc[XF][d] = fc[d];
        if (MODE == kStore) {
            const Src r = packed_src(fcur, a.dst.box_bytes);
            const uint32_t x = band_xor(fcur);
#pragma unroll
            for (int j = 0; j < NSLOT; ++j) dma(r, stage, j, pslot[j] < a.n_chunks ? (poff[j] ^ x) : kOob);
        } else {
            const Place pl = place<R>(a.src, c);
            const Src r{a.src.base + (uint64_t)pl.off, a.src.span};
            const uint32_t boxes = unit_boxes(fcur);
            const bool fast = inside_map(a.src, c, pl, boxes) && !a.elemwise;
            // edge bit: the tile needs the element path when it lands
            bool patch = false;
            if (fast) {
#pragma unroll
                for (int j = 0; j < NSLOT; ++j)
                    dma(r, stage, j, pslot[j] < a.n_chunks && slot_present(pslot[j], boxes) ? poff[j] : kOob);
            } else {
                // the source is the swept map: boxes past its last one lie
                // outside it anyway
                const Win<R> w = win(a.src, c, a.band_g);
#pragma unroll
                for (int j = 0; j < NSLOT; ++j) {
                    const bool full = !a.elemwise && pslot[j] < a.n_chunks &&
                                      classify<R>(pw0[j], pw1[j], w, a.k_el) == kFull;
                    dma(r, stage, j, full ? poff[j] : kOob);
                }
                patch = a.elemwise || splits_chunks(w);
            }
            edge = patch ? (edge | (1u << XF)) : (edge & ~(1u << XF));
        }
        cursor_advance<R>(a, fcur);
        // read the next fill's corner now, while this tile's loads fly (never
        // past this workgroup's last tile: an explicit-corner array ends there)
        if (++nfill < cnt) corner(fcur, fc);
    }

    // Wait for this wave's loads of the tile at corner c into stage X, patch
    // its partial chunks, then report the delivered bytes.  `later`: the
    // S-1 tiles after it have been filled (their NSLOT loads each may stay in
    // flight).  `drained`: the S-1 tiles before it have also been drained
    // since it was filled; every drain issues at least NSLOT 16-byte stores
    // (drain16), so those may stay in flight as well and the landing never
    // waits for a store.
    template <int X>
    __device__ __forceinline__ void land(uint8_t *stage, uint64_t *bar, const int32_t c[R], bool later,
                                         bool drained) const {
        if (later && drained)
            wait_vmcnt<2 * (S - 1) * NSLOT>();
        else if (later)
            wait_vmcnt<(S - 1) * NSLOT>();
        else
            wait_vmcnt<0>();
        if (MODE != kStore && ((edge >> X) & 1u)) patch_edge(stage, c);
        __builtin_amdgcn_s_waitcnt(kWaitLgkm);
        asm volatile("" ::: "memory");
        bar_complete(bar, my_bytes, lane, W);
    }

    // Edge tile at corner c: fill in the partial chunks of this lane's
    // producer slots element by element.  Slow path, kept out of the unrolled
    // slot arrays: each slot's chunk is recomputed.
    __device__ __forceinline__ void patch_edge(uint8_t *stage, const int32_t c[R]) const {
        const Place pl = place<R>(a.src, c);
        const Win<R> w = win(a.src, c, a.band_g);
        const __amdgpu_buffer_rsrc_t r = make_rsrc(a.src.base + (uint64_t)pl.off, a.src.span);
#pragma unroll 1
        for (int j = 0; j < NSLOT; ++j) {
            const uint32_t p = ((uint32_t)(j * W) + wave) * 64u + lane;
            if (p >= a.n_chunks) continue;
            if (a.elemwise) {
                load_slot_elements<R>(stage, p, a, a.src, w, r);
                continue;
            }
            uint32_t off, w0, w1;
            slot_info(p, a.src, off, w0, w1);
            if (classify<R>(w0, w1, w, a.k_el) == kPart)
                load_chunk_edge_es(a.src.elem_size, stage + p * 16u, off, w0 & 0xFFFFu, w.lo[0], w.hi[0], r);
        }
    }

    template <typename Rs>
    __device__ __forceinline__ void store16(const i32x4 &v, Rs r, uint32_t off) const {
        if (nts)
            __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 2);
        else
            __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
    }

    // The tile update of the fused round trip: + addend on each fp32 element
    // read back from the stage ("Day 76", "Solution").
    __device__ __forceinline__ i32x4 update(i32x4 v) const {
        if (MODE == kRoundtrip && a.add_f32) {
            typedef __attribute__((ext_vector_type(4))) float f32x4;
            f32x4 f = __builtin_bit_cast(f32x4, v);
            f = f + a.addend;
            v = __builtin_bit_cast(i32x4, f);
        }
        return v;
    }

    // Store slot chunk v at offset off when `on`.  With a ring of several
    // stages every drain issues the store regardless, sending the chunks
    // with nothing to write to the out-of-range offset (the hardware drops
    // them), so that land() can count on NSLOT stores per drain; with one
    // stage nothing counts on them and they are skipped.
    template <typename Rs>
    __device__ __forceinline__ void drain16(const i32x4 &v, Rs r, uint32_t off, bool on) const {
        if constexpr (S > 1)
            store16(v, r, on ? off : kOob);
        else if (on)
            store16(v, r, off);
    }

    // Read the region (box or unit) under cursor cur, at corner c, out of
    // `stage`.
    __device__ __forceinline__ void consume(uint8_t *stage, const int32_t c[R], const Cursor<R> &cur) const {
        if (MODE == kLoad) {
            const __amdgpu_buffer_rsrc_t r = packed_rsrc(cur, a.src.box_bytes);
            const uint32_t x = band_xor(cur);
#pragma unroll
            for (int j = 0; j < NSLOT; ++j) {
                const i32x4 v = *(const i32x4 *)(stage + cslot[j] * 16u);
                drain16(v, r, coff[j] ^ x, cslot[j] < a.n_chunks);
            }
        } else {
            const Place pl = place<R>(a.dst, c);
            const __amdgpu_buffer_rsrc_t r = make_rsrc(a.dst.base + (uint64_t)pl.off, a.dst.span);
            // a round trip's destination can be larger than the swept
            // source: only the unit's existing boxes are stored
            const uint32_t boxes = unit_boxes(cur);
            if (inside_map(a.dst, c, pl, boxes) && !a.elemwise) {
#pragma unroll
                for (int j = 0; j < NSLOT; ++j) {
                    const bool on = cslot[j] < a.n_chunks && slot_present(cslot[j], boxes);
                    const i32x4 v = update(*(const i32x4 *)(stage + cslot[j] * 16u));
                    drain16(v, r, coff[j], on);
                }
            } else {
                const Win<R> w = win(a.dst, c, boxes);
                // whole chunks (none when the swizzle moves elements inside
                // chunks: the element path below stores everything then)
#pragma unroll
                for (int j = 0; j < NSLOT; ++j) {
                    const bool on = !a.elemwise && cslot[j] < a.n_chunks &&
                                    classify<R>(cw0[j], cw1[j], w, a.k_el) == kFull;
                    const i32x4 v = update(*(const i32x4 *)(stage + cslot[j] * 16u));
                    drain16(v, r, coff[j], on);
                }
                // slow path, kept out of the unrolled slot arrays: recompute
                // each slot's chunk, store the inside elements of partial ones
                if (!a.elemwise && !splits_chunks(w)) return;
                const uint32_t cw = (wave + 1) % W;
#pragma unroll 1
                for (int j = 0; j < NSLOT; ++j) {
                    const uint32_t p = ((uint32_t)(j * W) + cw) * 64u + lane;
                    if (p >= a.n_chunks) continue;
                    if (a.elemwise) {
                        store_slot_elements<R>(stage, p, a, a.dst, w, r, MODE == kRoundtrip && a.add_f32);
                        continue;
                    }
                    uint32_t off, w0, w1;
                    slot_info(p, a.dst, off, w0, w1);
                    if (classify<R>(w0, w1, w, a.k_el) == kPart)
                        store_chunk_edge_es(a.dst.elem_size, stage + p * 16u, off, w0 & 0xFFFFu, w.lo[0], w.hi[0], r,
                                            MODE == kRoundtrip && a.add_f32, a.addend);
                }
            }
        }
    }

    // One step of a one-stage ring whose drain is held in registers (a
    // load of a wave that owns its stage): land tile k, read its image out
    // of the stage into `held`, refill the stage with tile k+1, and only then
    // store the image.  The stores of tile k are thus issued after the loads
    // of tile k+1, and the next landing waits for those loads alone
    // (vmcnt(NSLOT) leaves tile k's NSLOT stores in flight), where an
    // ordinary one-stage step would also wait for the previous stores.
    __device__ __forceinline__ bool step_held(uint8_t *st, int64_t k, i32x4 (&held)[NSLOT]) {
        static_assert(MODE == kLoad && S == 1 && W == 1, "a one-stage load ring of one wave");
        if (k >= cnt) return false;
        if (__hip_atomic_load(abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) return false;
        int32_t c[R];
#pragma unroll
        for (int d = 0; d < R; ++d) c[d] = sc[0][d];
        // after tile k's loads this wave issued tile k-1's NSLOT stores
        if (k > 0)
            wait_vmcnt<NSLOT>();
        else
            wait_vmcnt<0>();
        if ((edge & 1u) != 0u) patch_edge(st, c);
        __builtin_amdgcn_s_waitcnt(kWaitLgkm);
        asm volatile("" ::: "memory");
        bar_complete(&bars[0], my_bytes, lane, W);
        const bool ok = bar_wait(&bars[0], parity & 1u, a.spin_limit);
        parity ^= 1u;
        asm volatile("" ::: "memory");
        if (!ok) {
            if (lane == 0) {
                __hip_atomic_store(abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                __hip_atomic_fetch_or(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            return false;
        }
#pragma unroll
        for (int j = 0; j < NSLOT; ++j) held[j] = *(const i32x4 *)(st + cslot[j] * 16u);
        // the stage is free once these reads have completed
        __builtin_amdgcn_s_waitcnt(kWaitLgkm);
        asm volatile("" ::: "memory");
        const __amdgpu_buffer_rsrc_t r = packed_rsrc(ccur, a.src.box_bytes);
        if (k + 1 < cnt) fill<0>(st, &bars[0]);
#pragma unroll
        for (int j = 0; j < NSLOT; ++j) store16(held[j], r, cslot[j] < a.n_chunks ? coff[j] : kOob);
        cursor_advance<R>(a, ccur);
        return true;
    }

    // One ring step for tile k held in stage X; `fillst` is the stage that
    // tile k+S-1 goes to (the one tile k-1 just left).  False ends the loop.
    template <int X>
    __device__ __forceinline__ bool step(uint8_t *st, uint8_t *fillst, int64_t k) {
        if (k >= cnt) return false;
        // this wave's reads of the stage about to be refilled are done; with
        // a shared stage, every wave's (a wave that owns its stage read it
        // itself, so its own wait is enough)
        __builtin_amdgcn_s_waitcnt(kWaitLgkm);
        if constexpr (W > 1) __builtin_amdgcn_s_barrier();
        if (__hip_atomic_load(abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) return false;
        constexpr int XF = (X + S - 1) % S;
        // the tile's corner, recorded when it was filled (with one stage the
        // fill of this step is tile k itself, so read it after the fill)
        int32_t c[R];
        if (S > 1 && MODE != kStore && ((edge >> X) & 1u)) {
            // An edge tile's element loads must be waited for (vmcnt); landing
            // it before the next fill keeps that wait off the fill's loads.
#pragma unroll
            for (int d = 0; d < R; ++d) c[d] = sc[X][d];
            land<X>(st, &bars[X], c, false, false);
            if (k + S - 1 < cnt) fill<XF>(fillst, &bars[XF]);
        } else {
            const bool later = k + S - 1 < cnt;
            if (later) fill<XF>(fillst, &bars[XF]);
#pragma unroll
            for (int d = 0; d < R; ++d) c[d] = sc[X][d];
            // tile k was filled S-1 steps ago (or in the prologue), and the
            // steps since then each drained a tile after filling
            land<X>(st, &bars[X], c, later && S > 1, k >= S - 1);
        }
        const bool ok = bar_wait(&bars[X], (parity >> X) & 1u, a.spin_limit);
        parity ^= 1u << X;
        asm volatile("" ::: "memory");
        if (ok) {
            consume(st, c, ccur);
        } else if (lane == 0) {
            __hip_atomic_store(abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            __hip_atomic_fetch_or(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        cursor_advance<R>(a, ccur);
        return true;
    }
};

template <int MODE, int S, int NSLOT, int R, bool BAND = false>
__global__ __launch_bounds__(kThreads) void copy_kernel(const KArgs a) {
    constexpr uint32_t SB = NSLOT * kWaves * kBlockBytes;
    __shared__ __attribute__((aligned(1024))) uint8_t st0[SB];
    __shared__ __attribute__((aligned(1024))) uint8_t st1[S > 1 ? SB : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t st2[S > 2 ? SB : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t st3[S > 3 ? SB : 16];
    __shared__ uint64_t bars[4];
    __shared__ uint32_t abort_flag;

    Copier<MODE, S, NSLOT, R, BAND> cp(a, bars, &abort_flag);
    if (threadIdx.x == 0) {
        for (int i = 0; i < 4; ++i) bars[i] = 0;
        abort_flag = 0;
    }
    cp.setup();
    __syncthreads();
    if (cp.cnt <= 0) return;

    // prologue: tiles 0..S-2 go to stages 0..S-2
    if constexpr (S > 1) cp.template fill<0>(st0, &bars[0]);
    if constexpr (S > 2) if (1 < cp.cnt) cp.template fill<1>(st1, &bars[1]);
    if constexpr (S > 3) if (2 < cp.cnt) cp.template fill<2>(st2, &bars[2]);

    for (int64_t kb = 0; kb < cp.cnt; kb += S) {
        if constexpr (S == 1) {
            if (!cp.template step<0>(st0, st0, kb)) break;
        } else if constexpr (S == 2) {
            if (!cp.template step<0>(st0, st1, kb)) break;
            if (!cp.template step<1>(st1, st0, kb + 1)) break;
        } else if constexpr (S == 3) {
            if (!cp.template step<0>(st0, st2, kb)) break;
            if (!cp.template step<1>(st1, st0, kb + 1)) break;
            if (!cp.template step<2>(st2, st1, kb + 2)) break;
        } else {
            if (!cp.template step<0>(st0, st3, kb)) break;
            if (!cp.template step<1>(st1, st0, kb + 1)) break;
            if (!cp.template step<2>(st2, st1, kb + 2)) break;
            if (!cp.template step<3>(st3, st2, kb + 3)) break;
        }
    }
    // nothing may still be writing LDS or memory when the wave ends
    __builtin_amdgcn_s_waitcnt(0);
}

// ---------------------------------------------------------------- wave-per-box variant
// Every wave of the workgroup walks its own tile sequence through its own
// ring of S stages of one box each (NSLOT KiB): it issues all of a box's
// direct-to-LDS loads, arrives on its own stage record with the box's bytes,
// completes them once its loads have landed and drains the box after the
// record's phase flips -- the same byte-count protocol with one arrival per
// phase, and no workgroup barrier.  The per-box scalar work (corner,
// address, bounds) is done once per box instead of once per wave.  A
// workgroup is wave_group(NSLOT) such waves: four for boxes under 8 KiB, one
// for larger ones.
template <int MODE, int S, int NSLOT, int R>
__global__ __launch_bounds__(64 * wave_group(NSLOT)) void wave_kernel(const KArgs a) {
    constexpr int WG = wave_group(NSLOT);
    constexpr uint32_t SB = NSLOT * kBlockBytes;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[WG * S * SB];
    __shared__ uint64_t bars[WG * 4];
    __shared__ uint32_t abort_flag;

    const uint32_t hw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    Copier<MODE, S, NSLOT, R, false, 1, WG> cp(a, bars + 4 * hw, &abort_flag);
    if (threadIdx.x == 0) {
        for (int i = 0; i < WG * 4; ++i) bars[i] = 0;
        abort_flag = 0;
    }
    cp.setup();
    __syncthreads();
    if (cp.cnt <= 0) return;
    uint8_t *st0 = ring + hw * (S * SB);
    uint8_t *st1 = st0 + (S > 1 ? SB : 0);
    uint8_t *st2 = st0 + (S > 2 ? 2 * SB : 0);
    uint8_t *st3 = st0 + (S > 3 ? 3 * SB : 0);

    if constexpr (MODE == kLoad && S == 1) {
        // one stage, its drain held in registers while the next tile loads
        i32x4 held[NSLOT];
        cp.template fill<0>(st0, &cp.bars[0]);
        for (int64_t k = 0; k < cp.cnt; ++k)
            if (!cp.step_held(st0, k, held)) break;
        __builtin_amdgcn_s_waitcnt(0);
        return;
    }
    if constexpr (S > 1) cp.template fill<0>(st0, &cp.bars[0]);
    if constexpr (S > 2) if (1 < cp.cnt) cp.template fill<1>(st1, &cp.bars[1]);
    if constexpr (S > 3) if (2 < cp.cnt) cp.template fill<2>(st2, &cp.bars[2]);

    for (int64_t kb = 0; kb < cp.cnt; kb += S) {
        if constexpr (S == 1) {
            if (!cp.template step<0>(st0, st0, kb)) break;
        } else if constexpr (S == 2) {
            if (!cp.template step<0>(st0, st1, kb)) break;
            if (!cp.template step<1>(st1, st0, kb + 1)) break;
        } else if constexpr (S == 3) {
            if (!cp.template step<0>(st0, st2, kb)) break;
            if (!cp.template step<1>(st1, st0, kb + 1)) break;
            if (!cp.template step<2>(st2, st1, kb + 2)) break;
        } else {
            if (!cp.template step<0>(st0, st3, kb)) break;
            if (!cp.template step<1>(st1, st0, kb + 1)) break;
            if (!cp.template step<2>(st2, st1, kb + 2)) break;
            if (!cp.template step<3>(st3, st2, kb + 3)) break;
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
}

// ---------------------------------------------------------------- thread-copy variant
// The register path the pages contrast with the copy engine ("TMA -- the
// async bulk copy engine", "Interactive": thread-copy mode, the threads drive
// the copy lane by lane; "Day 76", the diagram's first band: every thread
// computes its addresses and moves the data through registers).  Each lane
// loads its chunks into VGPRs (the next tile's loads are in flight while the
// current tile is handled), writes them into the single LDS stage itself, and
// a plain workgroup barrier is then enough to publish the tile, because the
// writes were the threads' own.  Same tile order, bounds, zero fill, swizzle
// and clipped stores as the staged kernel; used as its A/B baseline.
template <int MODE, int NSLOT, int R>
struct ThreadCopier : Copier<MODE, 1, NSLOT, R> {
    using Base = Copier<MODE, 1, NSLOT, R>;
    using Base::a;
    using Base::ccur;
    using Base::cnt;
    using Base::fcur;
    using Base::nt;
    using Base::poff;
    using Base::pslot;
    using Base::pw0;
    using Base::pw1;

    __device__ __forceinline__ ThreadCopier(const KArgs &args, uint64_t *b, uint32_t *ab) : Base(args, b, ab) {}

    __device__ __forceinline__ i32x4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) const {
        return nt ? __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2)
                  : __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    }

    // Start the register loads of the fill cursor's tile; true for an edge tile.
    __device__ __forceinline__ bool issue(i32x4 (&v)[NSLOT]) {
        bool edge = false;
        if (MODE == kStore) {
            const uint64_t bb = a.dst.box_bytes;
            const __amdgpu_buffer_rsrc_t r = make_rsrc((uint64_t)a.packed + (uint64_t)fcur.t * bb, (uint32_t)bb);
#pragma unroll
            for (int j = 0; j < NSLOT; ++j) v[j] = ld16(r, pslot[j] < a.n_chunks ? pslot[j] * 16u : kOob);
        } else {
            int32_t c[R];
            cursor_corner<R>(a, a.src, fcur, c);
            const Place pl = place<R>(a.src, c);
            const __amdgpu_buffer_rsrc_t r = make_rsrc(a.src.base + (uint64_t)pl.off, a.src.span);
            edge = !(pl.interior && !a.elemwise);
            if (!edge) {
#pragma unroll
                for (int j = 0; j < NSLOT; ++j) v[j] = ld16(r, pslot[j] < a.n_chunks ? poff[j] : kOob);
            } else {
                const Win<R> w = window<R>(a.src, c);
#pragma unroll
                for (int j = 0; j < NSLOT; ++j) {
                    const bool full = !a.elemwise && pslot[j] < a.n_chunks &&
                                      classify<R>(pw0[j], pw1[j], w, a.k_el) == kFull;
                    v[j] = ld16(r, full ? poff[j] : kOob);
                }
            }
        }
        cursor_advance<R>(a, fcur);
        return edge;
    }

    // One tile: write `cur` into the stage, publish it with a barrier, drain it.
    __device__ __forceinline__ bool tile(uint8_t *stage, i32x4 (&cur)[NSLOT], bool cur_edge, i32x4 (&nxt)[NSLOT],
                                         bool &nxt_edge, int64_t k) {
        if (k >= cnt) return false;
        if (k + 1 < cnt) nxt_edge = issue(nxt);
        __builtin_amdgcn_s_waitcnt(kWaitLgkm);
        __builtin_amdgcn_s_barrier();  // every wave is done reading the previous tile
        int32_t c[R];
        cursor_corner<R>(a, this->swept(), ccur, c);
#pragma unroll
        for (int j = 0; j < NSLOT; ++j)
            if (pslot[j] < a.n_chunks) *(i32x4 *)(stage + pslot[j] * 16u) = cur[j];
        if (MODE != kStore && cur_edge) this->patch_edge(stage, c);
        __builtin_amdgcn_s_waitcnt(kWaitLgkm);
        __builtin_amdgcn_s_barrier();  // the tile is complete in LDS
        asm volatile("" ::: "memory");
        this->consume(stage, c, ccur);
        cursor_advance<R>(a, ccur);
        return true;
    }
};

template <int MODE, int NSLOT, int R>
__global__ __launch_bounds__(kThreads) void thread_kernel(const KArgs a) {
    constexpr uint32_t SB = NSLOT * kWaves * kBlockBytes;
    __shared__ __attribute__((aligned(1024))) uint8_t stage[SB];
    __shared__ uint64_t bars[4];
    __shared__ uint32_t abort_flag;
    ThreadCopier<MODE, NSLOT, R> cp(a, bars, &abort_flag);
    cp.setup();
    __syncthreads();
    if (cp.cnt <= 0) return;
    i32x4 va[NSLOT], vb[NSLOT];
    bool ea = cp.issue(va), eb = false;
    for (int64_t k = 0; k < cp.cnt; k += 2) {  // ping-pong, so no register copies
        if (!cp.tile(stage, va, ea, vb, eb, k)) break;
        if (!cp.tile(stage, vb, eb, va, ea, k + 1)) break;
    }
    __builtin_amdgcn_s_waitcnt(0);
}

// ---------------------------------------------------------------- producer-wave variant
// A dedicated issuing wave ("GPU TMA", "Warp specialization": producer warps
// issue the copies, consumer warps work on the tiles that are ready; "TMA --
// the async bulk copy engine", "Why this only pays off inside a pipeline").
// Wave 0 issues every direct-to-LDS load of a box under one arrive+expect of
// the whole box_bytes and completes it once its loads have landed; waves 1..4
// wait on the stage's full parity, drain it exactly like the cooperative
// kernel's consumers, and arrive on the stage's empty record, which the
// producer waits on before it refills the stage.  No workgroup barrier per
// tile.
constexpr int kWsConsumers = 4;
constexpr int kWsThreads = 64 * (kWsConsumers + 1);

template <int MODE, int S, int NSLOT, int R>
struct WsProducer {
    static constexpr int NP = NSLOT * kWsConsumers;  // 16-byte slots per producer lane per tile
    const KArgs &a;
    uint64_t *full, *empty;
    uint32_t *abort_flag;
    uint32_t lane, eparity, edge;
    int64_t cnt;
    bool nt;
    Cursor<R> fcur;
    uint32_t poff[NP], pw0[NP], pw1[NP];

    __device__ __forceinline__ WsProducer(const KArgs &args, uint64_t *f, uint64_t *e, uint32_t *ab, int64_t n,
                                          int64_t t0)
        : a(args), full(f), empty(e), abort_flag(ab), cnt(n) {
        lane = threadIdx.x & 63u;
        eparity = 0;
        edge = 0;
        nt = nontemporal_loads<MODE>(a.flags);
        cursor_init<R>(a, t0, fcur);
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const uint32_t p = (uint32_t)j * 64u + lane;
            poff[j] = pw0[j] = pw1[j] = 0;
            if (MODE != kStore && !a.elemwise && p < a.n_chunks)
                chunk_info_of<R>(a, logical_chunk_of(a, p, a.src), a.src, poff[j], pw0[j], pw1[j]);
        }
    }

    __device__ __forceinline__ void dma(const Src &src, uint8_t *stage, int j, uint32_t voff) const {
        dma_lds(src.base, src.nrec, stage + j * kBlockBytes, voff, nt);
    }

    // Arm stage X's full record with the box's bytes and issue all its loads.
    template <int X>
    __device__ __forceinline__ void fill(uint8_t *stage) {
        const uint32_t bb = a.src.box_bytes;
        const uint32_t budget = bb + ((a.flags & TMAP_FLAG_INJECT_BUDGET_MISMATCH) ? 16u : 0u);
        if (a.flags & TMAP_FLAG_DEBUG_POISON) poison_blocks(stage, NP, 1, lane);
        bar_arrive_expect(&full[X], budget, lane, 1);
        if (MODE == kStore) {
            const uint64_t dbb = a.dst.box_bytes;
            const Src r{(uint64_t)a.packed + (uint64_t)fcur.t * dbb, (uint32_t)dbb};
#pragma unroll
            for (int j = 0; j < NP; ++j) {
                const uint32_t p = (uint32_t)j * 64u + lane;
                dma(r, stage, j, p < a.n_chunks ? p * 16u : kOob);
            }
        } else {
            int32_t c[R];
            cursor_corner<R>(a, a.src, fcur, c);
            const Place pl = place<R>(a.src, c);
            const Src r{a.src.base + (uint64_t)pl.off, a.src.span};
            const bool fast = pl.interior && !a.elemwise;
            edge = fast ? (edge & ~(1u << X)) : (edge | (1u << X));
            if (fast) {
#pragma unroll
                for (int j = 0; j < NP; ++j) dma(r, stage, j, (uint32_t)j * 64u + lane < a.n_chunks ? poff[j] : kOob);
            } else {
                const Win<R> w = window<R>(a.src, c);
#pragma unroll
                for (int j = 0; j < NP; ++j) {
                    const bool full_chunk = !a.elemwise && (uint32_t)j * 64u + lane < a.n_chunks &&
                                            classify<R>(pw0[j], pw1[j], w, a.k_el) == kFull;
                    dma(r, stage, j, full_chunk ? poff[j] : kOob);
                }
            }
        }
        cursor_advance<R>(a, fcur);
    }

    // Wait for the loads of the tile at corner c into stage X, patch its
    // partial chunks and complete the stage's byte budget.  `later`: the S-1
    // tiles after it have been filled.
    template <int X>
    __device__ __forceinline__ void land(uint8_t *stage, const int32_t c[R], bool later) const {
        if (later)
            wait_vmcnt<(S - 1) * NP>();
        else
            wait_vmcnt<0>();
        if (MODE != kStore && ((edge >> X) & 1u)) {
            const Place pl = place<R>(a.src, c);
            const Win<R> w = window<R>(a.src, c);
            const __amdgpu_buffer_rsrc_t r = make_rsrc(a.src.base + (uint64_t)pl.off, a.src.span);
#pragma unroll 1
            for (int j = 0; j < NP; ++j) {
                const uint32_t p = (uint32_t)j * 64u + lane;
                if (p >= a.n_chunks) continue;
                if (a.elemwise) {
                    load_slot_elements<R>(stage, p, a, a.src, w, r);
                    continue;
                }
                uint32_t off, w0, w1;
                chunk_info_of<R>(a, logical_chunk_of(a, p, a.src), a.src, off, w0, w1);
                if (classify<R>(w0, w1, w, a.k_el) == kPart)
                    load_chunk_edge_es(a.src.elem_size, stage + p * 16u, off, w0 & 0xFFFFu, w.lo[0], w.hi[0], r);
            }
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm);
        asm volatile("" ::: "memory");
        bar_complete(&full[X], a.src.box_bytes, lane, 1);
    }

    __device__ __forceinline__ bool aborted() const {
        return __hip_atomic_load(abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0;
    }

    __device__ __forceinline__ void fail() const {
        if (lane == 0) {
            __hip_atomic_store(abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            __hip_atomic_fetch_or(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    // Tile i sits in stage X: land it, then (once the consumers released the
    // stage) refill the stage with tile i+S.  False ends the loop.
    template <int X>
    __device__ __forceinline__ bool step(uint8_t *st, Cursor<R> &lcur, int64_t i) {
        if (i >= cnt || aborted()) return false;
        int32_t c[R];
        cursor_corner<R>(a, MODE == kStore ? a.dst : a.src, lcur, c);
        land<X>(st, c, i + S - 1 < cnt);
        cursor_advance<R>(a, lcur);
        if (i + S < cnt) {
            if (!bar_wait(&empty[X], (eparity >> X) & 1u, a.spin_limit)) {
                fail();
                return false;
            }
            eparity ^= 1u << X;
            asm volatile("" ::: "memory");
            fill<X>(st);
        }
        return true;
    }
};

template <int MODE, int S, int NSLOT, int R>
__global__ __launch_bounds__(kWsThreads) void ws_kernel(const KArgs a) {
    constexpr uint32_t SB = NSLOT * kWsConsumers * kBlockBytes;
    __shared__ __attribute__((aligned(1024))) uint8_t st0[SB];
    __shared__ __attribute__((aligned(1024))) uint8_t st1[S > 1 ? SB : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t st2[S > 2 ? SB : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t st3[S > 3 ? SB : 16];
    __shared__ uint64_t full[4], empty[4];
    __shared__ uint32_t abort_flag;

    if (threadIdx.x == 0) {
        for (int i = 0; i < 4; ++i) full[i] = empty[i] = 0;
        abort_flag = 0;
    }
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // the consumers' view: consumer cw = wave-1 drains the slots of the
    // cooperative kernel's consumer cw, i.e. acts as its wave (cw+3) % 4
    Copier<MODE, S, NSLOT, R> cons(a, full, &abort_flag);
    cons.setup(wave == 0 ? 0 : (int)((wave - 1 + kWsConsumers - 1) % kWsConsumers));
    __syncthreads();
    if (cons.cnt <= 0) return;

    if (wave == 0) {
        WsProducer<MODE, S, NSLOT, R> pr(a, full, empty, &abort_flag, cons.cnt, cons.fcur.t);
        Cursor<R> lcur = pr.fcur;
        pr.template fill<0>(st0);
        if constexpr (S > 1) if (1 < pr.cnt) pr.template fill<1>(st1);
        if constexpr (S > 2) if (2 < pr.cnt) pr.template fill<2>(st2);
        if constexpr (S > 3) if (3 < pr.cnt) pr.template fill<3>(st3);
        for (int64_t kb = 0; kb < pr.cnt; kb += S) {
            if (!pr.template step<0>(st0, lcur, kb)) break;
            if constexpr (S > 1) if (!pr.template step<1>(st1, lcur, kb + 1)) break;
            if constexpr (S > 2) if (!pr.template step<2>(st2, lcur, kb + 2)) break;
            if constexpr (S > 3) if (!pr.template step<3>(st3, lcur, kb + 3)) break;
        }
    } else {
        uint32_t fparity = 0;
        auto consume = [&](auto xc, uint8_t *st, int64_t i) -> bool {
            constexpr int X = decltype(xc)::value;
            if (i >= cons.cnt) return false;
            if (__hip_atomic_load(&abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) return false;
            if (!bar_wait(&full[X], (fparity >> X) & 1u, a.spin_limit)) {
                if (cons.lane == 0) {
                    __hip_atomic_store(&abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                    __hip_atomic_fetch_or(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                return false;
            }
            fparity ^= 1u << X;
            asm volatile("" ::: "memory");
            int32_t c[R];
            cursor_corner<R>(a, cons.swept(), cons.ccur, c);
            cons.consume(st, c, cons.ccur);
            __builtin_amdgcn_s_waitcnt(kWaitLgkm);  // this wave's reads of the stage are done
            bar_arrive(&empty[X], cons.lane, kWsConsumers);
            cursor_advance<R>(a, cons.ccur);
            return true;
        };
        for (int64_t kb = 0; kb < cons.cnt; kb += S) {
            if (!consume(std::integral_constant<int, 0>{}, st0, kb)) break;
            if constexpr (S > 1) if (!consume(std::integral_constant<int, 1>{}, st1, kb + 1)) break;
            if constexpr (S > 2) if (!consume(std::integral_constant<int, 2>{}, st2, kb + 2)) break;
            if constexpr (S > 3) if (!consume(std::integral_constant<int, 3>{}, st3, kb + 3)) break;
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
}

typedef void (*KernelFn)(const KArgs);

template <int MODE, int S, int R>
KernelFn pick_nslot(int nslot) {
    switch (nslot) {
        case 1: return copy_kernel<MODE, S, 1, R>;
        case 2: return copy_kernel<MODE, S, 2, R>;
        case 4: return copy_kernel<MODE, S, 4, R>;
        case 8: return copy_kernel<MODE, S, 8, R>;
        case 16:
            if constexpr (S <= 2) return copy_kernel<MODE, S, 16, R>;
            return nullptr;
        default: return nullptr;
    }
}

template <int MODE, int R>
KernelFn pick_thread(int nslot) {
    switch (nslot) {
        case 1: return thread_kernel<MODE, 1, R>;
        case 2: return thread_kernel<MODE, 2, R>;
        case 4: return thread_kernel<MODE, 4, R>;
        case 8: return thread_kernel<MODE, 8, R>;
        case 16: return thread_kernel<MODE, 16, R>;
        default: return nullptr;
    }
}

template <int MODE, int S, int R>
KernelFn pick_wave(int nslot) {
    switch (nslot) {
        case 1: return wave_kernel<MODE, S, 1, R>;
        case 2: return wave_kernel<MODE, S, 2, R>;
        case 4: return wave_kernel<MODE, S, 4, R>;
        case 8: return wave_kernel<MODE, S, 8, R>;
        case 16: return wave_kernel<MODE, S, 16, R>;
        default: return nullptr;
    }
}

template <int MODE, int S, int R>
KernelFn pick_ws(int nslot) {
    switch (nslot) {
        case 1: return ws_kernel<MODE, S, 1, R>;
        case 2: return ws_kernel<MODE, S, 2, R>;
        case 4: return ws_kernel<MODE, S, 4, R>;
        case 8: return ws_kernel<MODE, S, 8, R>;
        default: return nullptr;
    }
}

// Launch the (MODE, stages, nslot, R) variant; stages == 0 is the
// thread-copy variant, stages 12..14 the producer-wave variant with 2..4
// stages, stages 21..24 the ring with 1..4 stages on the band schedule
// (nslot is then 4) and stages 31..32 the wave-per-box variant with 1..2
// stages of nslot KiB per wave.  hipError_t as int.
template <int MODE, int R>
int launch_mode(int stages, int nslot, const KArgs &a, void *stream) {
    KernelFn fn = nullptr;
    int threads = kThreads;
    uint32_t blocks = a.grid;
    switch (stages) {
        case 0: fn = pick_thread<MODE, R>(nslot); break;
        case 12: fn = pick_ws<MODE, 2, R>(nslot); threads = kWsThreads; break;
        case 13: fn = pick_ws<MODE, 3, R>(nslot); threads = kWsThreads; break;
        case 14: fn = pick_ws<MODE, 4, R>(nslot); threads = kWsThreads; break;
        case 1: fn = pick_nslot<MODE, 1, R>(nslot); break;
        case 2: fn = pick_nslot<MODE, 2, R>(nslot); break;
        case 3: fn = pick_nslot<MODE, 3, R>(nslot); break;
        case 4: fn = pick_nslot<MODE, 4, R>(nslot); break;
        case 21: fn = copy_kernel<MODE, 1, kBandSlots, R, true>; break;
        case 22: fn = copy_kernel<MODE, 2, kBandSlots, R, true>; break;
        case 23: fn = copy_kernel<MODE, 3, kBandSlots, R, true>; break;
        case 24: fn = copy_kernel<MODE, 4, kBandSlots, R, true>; break;
        // a.grid counts waves here: wave_group(nslot) to a workgroup
        case 31:
        case 32:
            fn = stages == 31 ? pick_wave<MODE, 1, R>(nslot) : pick_wave<MODE, 2, R>(nslot);
            threads = 64 * wave_group(nslot);
            blocks = (a.grid + wave_group(nslot) - 1) / wave_group(nslot);
            break;
        default: break;
    }
    if (!fn) return (int)hipErrorInvalidValue;
    KArgs copy = a;
    void *args[] = {&copy};
    return (int)hipLaunchKernel((const void *)fn, dim3(blocks), dim3(threads), args, 0, (hipStream_t)stream);
}

}  // namespace
}  // namespace tmap
