// tmap_corner4.h -- boxes at explicit corners in 4-byte lanes: the corner
// path for maps whose box rows are a power of two from 16 to 256 bytes, in
// boxes of at most 64 rows and 8 KiB, unswizzled or with a swizzle that moves
// whole 16-byte chunks within rows.
//
// The 16-byte lanes of the corner kernel (tmap_corner.h) can straddle the
// tensor's dimension-0 edge, and each chunk cut that way is patched element
// by element.  A 4-byte lane of 4- or 8-byte elements never holds part of an
// inside element and part of an outside one, so every lane is wholly in or
// out, and the hardware does all of the clipping: a load past num_records
// lands zeros ("GPU TMA", "Why architecture matters here": the copy itself
// zero-fills out-of-bounds elements) and a store past it is dropped.  With
// 1- or 2-byte elements the edge can cut a word; only the lanes of the
// columns it cuts (at most one at each edge of the row) then move their
// inside elements one by one, in a pass a wave takes only when one of its
// lanes needs it.  The image a wave lands is the same as in 16-byte lanes:
// slot i of lane l is the box's 4-byte word 64 i + l, at LDS stage + 256 i
// + 4 l.
//
// A box row is 4 * 2^dshift bytes, so a slot's 64 lanes cover 64 / 2^dshift
// whole rows and a lane's column (its word in the row) is the same in every
// slot.  Per box, lane l works out row l's in-box byte offset in one pass
// (mixed radix over box[1..]) and tests the row against the box's window; a
// row outside gets the out-of-range offset.  Each slot then fetches its
// row's value from the lane that holds it (ds_bpermute) and adds its
// column's offset with a saturating add, so that an out-of-range row or
// column stays out of range.  Per box that is one pass of row arithmetic
// for the whole wave, then two instructions per slot (without a swizzle).
//
// A swizzle whose XOR lands inside a row (its target bits below the row's
// size) leaves every word in its row and moves it within the row: the word
// at column x of row r holds the logical column x ^ key(r) ^ key(x), the
// keys being the swizzle's source bits of the row and of the column.  The
// slot fetching the row's entry then also gets the row's key (kept in the
// entry's low 4 bits: in-box row offsets are multiples of 16), forms its
// logical column and looks its range test up in a column table (one entry
// per logical column, a lane each), with a second ds_bpermute.
//
// Each wave walks its own share of the tiles through its own one-box stage
// and 8-byte byte record, as the corner kernel does.  The tiles are explicit
// corners, or those of a sweep (maps of rank 3 and more, and others the band
// kernel does not take), whose corners the carry-add cursor walks:
//
//   fill    arrive on the record with the box's byte budget and issue one
//           4-byte direct-to-LDS load per slot from the tensor (a store: one
//           16-byte load per slot from the packed image);
//   land    wait for the loads (vmcnt), complete the budget, wait for the
//           record's phase ("TMA -- the async bulk copy engine", "Load
//           completion -- the mbarrier and the byte budget");
//   drain   a load copies the image to its packed slot in 16-byte lanes; a
//           store or round trip reads its 4-byte slots back and stores each
//           through the destination map, whose out-of-range slots are
//           dropped.

#pragma once

#include "tmap_corner.h"

namespace tmap {
namespace {

// Column entries: the byte offset of a word in its row when every element of
// the word lies inside the window in dimension 0, kOob when none does, and
// kOob | 1 when the window cuts the word (1- and 2-byte elements only).
constexpr uint32_t kCut = kOob | 1u;

// One side of the copy (the map a box is loaded from or stored to) for one
// box, as this lane holds it.
//   row  the row table entry for row `lane`: the row's in-box byte offset
//        (with a swizzle, | its swizzle key in bits 0..3), or kOob when the
//        row lies outside the tensor or past the box's rows;
//   col  without a swizzle, this lane's column entry; with one, the column
//        table entry of logical column lane % (words per row);
//   xb   this lane's column byte (with a swizzle, XOR its own bits' key).
struct C4Side {
    uint32_t row, col, xb;
};

template <int R, bool SWZ>
__device__ __forceinline__ C4Side c4_side(const KArgs &A, const KMap &m, const Win<R> &w, uint32_t lane) {
    C4Side s;
    uint32_t r = lane, ro = 0;
    bool in = lane < A.c4_rows;
#pragma unroll
    for (int d = 1; d < R; ++d) {
        const uint32_t q = div_small(r, A.box_magic[d]);
        const uint32_t id = r - q * (uint32_t)m.box[d];
        r = q;
        in = in & (id - w.lo[d] < w.hi[d] - w.lo[d]);
        ro += id * (uint32_t)m.strides[d];
    }
    if constexpr (SWZ) ro |= ((lane << (A.c4_dshift + 2u)) >> A.c4_sb) & A.c4_smask;
    s.row = in ? ro : kOob;
    const uint32_t xb = (lane & ((1u << A.c4_dshift) - 1u)) * 4u;
    const uint32_t e0 = xb >> A.c4_esz, e1 = (xb + 3u) >> A.c4_esz;  // the word's first and last element
    const bool full = (e0 >= w.lo[0]) && (e1 < w.hi[0]);
    const bool any = (e0 < w.hi[0]) && (e1 >= w.lo[0]) && (w.lo[0] < w.hi[0]);
    s.col = full ? xb : (any ? kCut : kOob);
    s.xb = SWZ ? xb ^ (((xb >> A.c4_sb) & A.c4_smask) << A.c4_tb) : xb;
    return s;
}

// One slot of this lane: the row table entry of its row (raddr: the lane
// holding it, times 4), its logical column byte and that column's entry.
struct C4Slot {
    uint32_t row, xl, col;
};

template <bool SWZ>
__device__ __forceinline__ C4Slot c4_slot(const KArgs &A, const C4Side &s, uint32_t raddr) {
    C4Slot q;
    q.row = (uint32_t)__builtin_amdgcn_ds_bpermute((int)raddr, (int)s.row);
    if constexpr (SWZ) {
        q.xl = s.xb ^ ((q.row & 15u) << A.c4_tb);
        q.col = (uint32_t)__builtin_amdgcn_ds_bpermute((int)q.xl, (int)s.col);
        q.row &= ~15u;
    } else {
        q.xl = s.xb;
        q.col = s.col;
    }
    return q;
}

// The slot's byte offset from the box corner, or >= kOob when its row or
// column lies outside (the saturating add keeps kOob + anything >= kOob).
__device__ __forceinline__ uint32_t c4_off(const C4Slot &q) {
    return __builtin_elementwise_add_sat(q.row, q.col & ~1u);
}

// Every slot's offset (off[i] for slot i).  With a swizzle each slot takes
// two table fetches, and each offset is pinned where it is formed: left
// alone, the compiler would sink the final add to the stores and hold both
// fetched entries of every slot until then (131 VGPRs for a store, three
// waves to a SIMD).
template <int NI, bool SWZ>
__device__ __forceinline__ void c4_offsets(const KArgs &A, const C4Side &s, uint32_t ra, uint32_t rstep,
                                           uint32_t (&off)[NI]) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        off[i] = c4_off(c4_slot<SWZ>(A, s, ra + (uint32_t)i * rstep));
        if constexpr (SWZ) asm volatile("" : "+v"(off[i]));
    }
}

// Whether the window cuts the slot's word inside a row that is inside.
__device__ __forceinline__ bool c4_cut(const C4Slot &q) { return (q.col == kCut) & (q.row < kOob); }

// The cut word at byte offset row + xl: its elements of ES bytes inside the
// window [lo0, hi0), loaded one by one, the others zero (what the
// out-of-range load landed for the whole word).
template <int ES>
__device__ __forceinline__ uint32_t c4_cut_word(__amdgpu_buffer_rsrc_t r, uint32_t row, uint32_t xl, uint32_t lo0,
                                                uint32_t hi0) {
    uint32_t w = 0;
#pragma unroll
    for (uint32_t b = 0; b < 4u; b += ES) {
        if (((xl + b) / ES) - lo0 >= hi0 - lo0) continue;
        const uint32_t v = ES == 1 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, row + xl + b, 0, 0)
                                   : (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, row + xl + b, 0, 0);
        w |= v << (8u * b);
    }
    return w;
}

// The landed stage's cut words, rewritten whole with their inside elements.
// In batches of 8 slots, so that a batch's loads are in flight together;
// every lane takes part in the table fetches, which read other lanes.
template <int NI, int ES, bool SWZ>
__device__ __forceinline__ void c4_patch_cut(const KArgs &A, uint8_t *stage, uint32_t lane, const C4Side &s,
                                             uint32_t ra, uint32_t rstep, __amdgpu_buffer_rsrc_t r, uint32_t lo0,
                                             uint32_t hi0) {
    constexpr int B = NI < 8 ? NI : 8;
#pragma unroll 1
    for (int i0 = 0; i0 < NI; i0 += B) {
        C4Slot q[B];
        uint32_t w[B];
#pragma unroll
        for (int j = 0; j < B; ++j) q[j] = c4_slot<SWZ>(A, s, ra + (uint32_t)(i0 + j) * rstep);
#pragma unroll
        for (int j = 0; j < B; ++j) w[j] = c4_cut(q[j]) ? c4_cut_word<ES>(r, q[j].row, q[j].xl, lo0, hi0) : 0u;
#pragma unroll
        for (int j = 0; j < B; ++j)
            if (c4_cut(q[j])) *(uint32_t *)(stage + ((uint32_t)(i0 + j) * 64u + lane) * 4u) = w[j];
    }
}

// The stage's cut words stored through the destination: only their
// elements inside the window [lo0, hi0), one by one.  Batches of 8 slots as
// above (the words are read again from the stage: 1- and 2-byte elements
// take no +addend).
template <int NI, int ES, bool SWZ, bool NT>
__device__ __forceinline__ void c4_store_cut(const KArgs &A, const uint8_t *stage, uint32_t lane, const C4Side &s,
                                             uint32_t ra, uint32_t rstep, __amdgpu_buffer_rsrc_t r, uint32_t lo0,
                                             uint32_t hi0) {
    constexpr int B = NI < 8 ? NI : 8;
#pragma unroll 1
    for (int i0 = 0; i0 < NI; i0 += B) {
        C4Slot q[B];
        uint32_t w[B];
#pragma unroll
        for (int j = 0; j < B; ++j) {
            q[j] = c4_slot<SWZ>(A, s, ra + (uint32_t)(i0 + j) * rstep);
            w[j] = *(const uint32_t *)(stage + ((uint32_t)(i0 + j) * 64u + lane) * 4u);
        }
#pragma unroll
        for (int j = 0; j < B; ++j) {
            if (!c4_cut(q[j])) continue;
#pragma unroll
            for (uint32_t b = 0; b < 4u; b += ES) {
                if (((q[j].xl + b) / ES) - lo0 >= hi0 - lo0) continue;
                const uint32_t o = q[j].row + q[j].xl + b;
                if constexpr (ES == 1)
                    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(w[j] >> (8u * b)), r, o, 0, NT ? 2 : 0);
                else
                    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(w[j] >> (8u * b)), r, o, 0, NT ? 2 : 0);
            }
        }
    }
}

template <bool NT>
__device__ __forceinline__ void c4_store4(uint32_t v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (NT)
        __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 2);
    else
        __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0);
}

template <bool NT>
__device__ __forceinline__ void c4_store16(const i32x4 &v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (NT)
        __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 2);
    else
        __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}

// SAME: a round trip whose destination map has the source's dims and
// strides (only its base differs): the stores reuse the loads' offsets.
// SWZ: the maps' swizzle moves words within rows (see above).
// `a` must stay the kernel's only argument: reread() finds it at the start
// of the argument segment.
template <int MODE, int NSLOT, int R, bool NTL, bool NTS, bool ADD, bool SAME, bool SWZ>
__global__ __launch_bounds__(64 * wave_group(NSLOT)) void corner4_kernel(const KArgs a) {
    static_assert(!SAME || MODE == kRoundtrip, "a load or store has one tensor map");
    constexpr int WG = wave_group(NSLOT);
    constexpr uint32_t SB = NSLOT * kBlockBytes;
    constexpr int NI = NSLOT * 4;  // 4-byte slots per lane
    __shared__ __attribute__((aligned(1024))) uint8_t ring[WG * SB];
    __shared__ uint64_t bars[WG];

    const uint32_t hw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = threadIdx.x & 63u;
    uint64_t *bar = &bars[hw];
    if (lane == 0) *bar = 0;
    int64_t cnt, t;
    corner_deal(a, (int64_t)blockIdx.x * WG + hw, cnt, t);
    // each wave owns its record and stage: its own LDS write is ordered
    // before its own atomics on it
    __builtin_amdgcn_s_waitcnt(kWaitLgkm);
    if (cnt <= 0) return;
    uint8_t *stage = ring + hw * SB;
    const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void_t *)stage;
    const KMap &sw = MODE == kStore ? a.dst : a.src;
    // this lane's row among a slot's rows as a ds_bpermute address, and the
    // address step from one slot to the next (rows per slot, times 4)
    const uint32_t raddr = (lane >> a.c4_dshift) * 4u;
    const uint32_t rstep = (64u >> a.c4_dshift) * 4u;
    const uint32_t bytes = sw.box_bytes;
    const uint32_t budget = bytes + ((a.flags & TMAP_FLAG_INJECT_BUDGET_MISMATCH) ? 16u : 0u);
    uint32_t parity = 0;
    // the wave's tiles: explicit corners are read per tile; a sweep walks
    // its tiles' digits with the carry-add cursor, divided out once here
    Cursor<R> cur;
    if (a.coords) {
        cur.t = t;
        cur.k = 0;
    } else {
        cursor_init<R>(a, t, cur);
    }

    for (int64_t n = 0; n < cnt; ++n) {
        int32_t c[R];
        cursor_corner<R>(a, sw, cur, c);
        // the slots' row-fetch addresses are formed per box, not held across
        // the loop in NI registers
        uint32_t ra = raddr;
        asm volatile("" : "+v"(ra));
        if (a.flags & TMAP_FLAG_DEBUG_POISON) poison_blocks(stage, NSLOT, 1, lane);
        bar_arrive_expect(bar, budget, lane, 1);
        // destination offsets of the slots, held until the drain, and the
        // tables of the two sides for the cut words
        uint32_t off[NI];
        C4Side ss = {kOob, kOob, 0u}, ds = {kOob, kOob, 0u};
        if constexpr (MODE == kStore) {
            const uint64_t base = (uint64_t)a.packed + (uint64_t)cur.t * bytes;
#pragma unroll
            for (int j = 0; j < NSLOT; ++j) {
                const uint32_t p = (uint32_t)j * 64u + lane;
                dma_lds_hint<NTL>(base, bytes, m0 + (uint32_t)j * kBlockBytes, p < a.n_chunks ? p * 16u : kOob);
            }
        } else {
            const Win<R> w = corner_window<R>(a.src, c);
            ss = c4_side<R, SWZ>(a, a.src, w, lane);
            const uint64_t base = a.src.base + (uint64_t)corner_offset<R>(a, a.src, c);
            // every slot's offset first, so that the table fetches overlap,
            // then the loads
            uint32_t so[NI];
            c4_offsets<NI, SWZ>(a, ss, ra, rstep, so);
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                dma_lds_dword<NTL>(base, a.src.span, m0 + (uint32_t)i * 256u, so[i]);
                if constexpr (SAME) off[i] = so[i];
            }
        }
        if constexpr (MODE == kStore || (MODE == kRoundtrip && !SAME)) {
            // while the loads fly: the destination's offsets (a round trip
            // between two maps reads the destination's fields again, as both
            // maps' fields would not fit in scalar registers)
            const KArgs &A = MODE == kRoundtrip ? reread(a) : a;
            const Win<R> w = corner_window<R>(A.dst, c);
            ds = c4_side<R, SWZ>(A, A.dst, w, lane);
            c4_offsets<NI, SWZ>(A, ds, ra, rstep, off);
        } else if constexpr (SAME) {
            ds = ss;
        }

        // land: every slot's load has written the stage (zeros past the
        // tensor); the cut words' inside elements; then the record's byte
        // count and phase
        wait_vmcnt<0>();
        if constexpr (MODE != kStore) {
            // a wave with a cut column (1- and 2-byte elements only)
            if (__builtin_amdgcn_ballot_w64(ss.col == kCut)) {
                const KArgs &A = reread(a);
                const Win<R> w = corner_window<R>(A.src, c);
                const __amdgpu_buffer_rsrc_t r =
                    make_rsrc(A.src.base + (uint64_t)corner_offset<R>(A, A.src, c), A.src.span);
                if (A.c4_esz == 0)
                    c4_patch_cut<NI, 1, SWZ>(A, stage, lane, ss, ra, rstep, r, w.lo[0], w.hi[0]);
                else
                    c4_patch_cut<NI, 2, SWZ>(A, stage, lane, ss, ra, rstep, r, w.lo[0], w.hi[0]);
            }
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm);
        asm volatile("" ::: "memory");
        bar_complete(bar, bytes, lane, 1);
        const bool ok = bar_wait(bar, parity, a.spin_limit);
        parity ^= 1u;
        asm volatile("" ::: "memory");
        if (!ok) {
            if (lane == 0) __hip_atomic_fetch_or(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }

        // drain
        if constexpr (MODE == kLoad) {
            i32x4 v[NSLOT];
#pragma unroll
            for (int j = 0; j < NSLOT; ++j) v[j] = *(const i32x4 *)(stage + ((uint32_t)j * 64u + lane) * 16u);
            const __amdgpu_buffer_rsrc_t r = make_rsrc((uint64_t)a.packed + (uint64_t)cur.t * bytes, bytes);
#pragma unroll
            for (int j = 0; j < NSLOT; ++j) {
                const uint32_t p = (uint32_t)j * 64u + lane;
                c4_store16<NTS>(v[j], r, p < a.n_chunks ? p * 16u : kOob);
            }
        } else {
            uint32_t v[NI];
#pragma unroll
            for (int i = 0; i < NI; ++i) v[i] = *(const uint32_t *)(stage + ((uint32_t)i * 64u + lane) * 4u);
            if constexpr (ADD) {
                // the tile update of the fused round trip (fp32 elements)
#pragma unroll
                for (int i = 0; i < NI; ++i)
                    v[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, v[i]) + a.addend);
            }
            const KArgs &A = (MODE == kRoundtrip && !SAME) ? reread(a) : a;
            const KMap &dm = SAME ? A.src : A.dst;
            const __amdgpu_buffer_rsrc_t r =
                make_rsrc(A.dst.base + (uint64_t)corner_offset<R>(A, dm, c), dm.span);
#pragma unroll
            for (int i = 0; i < NI; ++i) c4_store4<NTS>(v[i], r, off[i]);
            if (__builtin_amdgcn_ballot_w64(ds.col == kCut)) {
                // the words the destination's window cuts, element by element
                const Win<R> w = corner_window<R>(dm, c);
                if (A.c4_esz == 0)
                    c4_store_cut<NI, 1, SWZ, NTS>(A, stage, lane, ds, ra, rstep, r, w.lo[0], w.hi[0]);
                else
                    c4_store_cut<NI, 2, SWZ, NTS>(A, stage, lane, ds, ra, rstep, r, w.lo[0], w.hi[0]);
            }
        }
        // the stage is free once these reads have completed
        __builtin_amdgcn_s_waitcnt(kWaitLgkm);
        asm volatile("" ::: "memory");
        cursor_advance<R>(a, cur);
    }
    // nothing may still be writing LDS or memory when the wave ends
    __builtin_amdgcn_s_waitcnt(0);
}

template <int MODE, int NSLOT, int R, bool ADD, bool SAME, bool SWZ>
KernelFn pick_corner4_hints(bool ntl, bool nts) {
    if constexpr (MODE == kRoundtrip) {
        // both sides are the tensor's: one hint for both
        (void)nts;
        return ntl ? corner4_kernel<MODE, NSLOT, R, true, true, ADD, SAME, SWZ>
                   : corner4_kernel<MODE, NSLOT, R, false, false, ADD, SAME, SWZ>;
    } else {
        if (ntl)
            return nts ? corner4_kernel<MODE, NSLOT, R, true, true, ADD, SAME, SWZ>
                       : corner4_kernel<MODE, NSLOT, R, true, false, ADD, SAME, SWZ>;
        return nts ? corner4_kernel<MODE, NSLOT, R, false, true, ADD, SAME, SWZ>
                   : corner4_kernel<MODE, NSLOT, R, false, false, ADD, SAME, SWZ>;
    }
}

template <int MODE, int R, bool ADD, bool SAME, bool SWZ>
KernelFn pick_corner4_slots(int nslot, bool ntl, bool nts) {
    switch (nslot) {
        case 1: return pick_corner4_hints<MODE, 1, R, ADD, SAME, SWZ>(ntl, nts);
        case 2: return pick_corner4_hints<MODE, 2, R, ADD, SAME, SWZ>(ntl, nts);
        case 4: return pick_corner4_hints<MODE, 4, R, ADD, SAME, SWZ>(ntl, nts);
        case 8: return pick_corner4_hints<MODE, 8, R, ADD, SAME, SWZ>(ntl, nts);
        default: return nullptr;
    }
}

template <int MODE, int R, bool ADD, bool SAME = false>
KernelFn pick_corner4(int nslot, bool swz, bool ntl, bool nts) {
    return swz ? pick_corner4_slots<MODE, R, ADD, SAME, true>(nslot, ntl, nts)
               : pick_corner4_slots<MODE, R, ADD, SAME, false>(nslot, ntl, nts);
}

// Launch the 4-byte-lane corner kernel of direction MODE over a.grid waves
// (wave_group to a workgroup).  hipError_t as int.
template <int MODE, int R>
int launch_corner4_mode(int nslot, const KArgs &a, void *stream) {
    const bool ntl = nontemporal_loads<MODE>(a.flags), nts = nontemporal_stores<MODE>(a.flags);
    const bool swz = (MODE == kStore ? a.dst : a.src).swz_b != 0;
    KernelFn fn = nullptr;
    if constexpr (MODE == kRoundtrip) {
        if (same_shape(a.src, a.dst))
            fn = a.add_f32 ? pick_corner4<MODE, R, true, true>(nslot, swz, ntl, nts)
                           : pick_corner4<MODE, R, false, true>(nslot, swz, ntl, nts);
        else
            fn = a.add_f32 ? pick_corner4<MODE, R, true>(nslot, swz, ntl, nts)
                           : pick_corner4<MODE, R, false>(nslot, swz, ntl, nts);
    } else {
        fn = pick_corner4<MODE, R, false>(nslot, swz, ntl, nts);
    }
    if (!fn) return (int)hipErrorInvalidValue;
    const uint32_t wg = (uint32_t)wave_group(nslot);
    KArgs copy = a;
    void *args[] = {&copy};
    return (int)hipLaunchKernel((const void *)fn, dim3((a.grid + wg - 1) / wg), dim3(64 * wg), args,
                                corner4_lds_reserve(MODE, nslot), (hipStream_t)stream);
}

}  // namespace
}  // namespace tmap
