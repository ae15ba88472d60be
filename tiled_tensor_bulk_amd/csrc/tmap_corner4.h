// tmap_corner4.h -- boxes at explicit corners in 4-byte lanes: the corner
// path for unswizzled maps whose box rows are a power of two from 16 to 256
// bytes, in boxes of at most 64 rows and 8 KiB.
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
// for the whole wave, then two instructions per slot.
//
// Each wave walks its own share of the corners through its own one-box
// stage and 8-byte byte record, as the corner kernel does:
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

// Row `lane` of a box at the corner whose window is w: its in-box byte
// offset in map m, or kOob when the row lies outside the tensor or past the
// box's rows.  In-box offsets are below the map's span (< 2 GiB).
template <int R>
__device__ __forceinline__ uint32_t c4_row(const KArgs &A, const KMap &m, const Win<R> &w, uint32_t lane) {
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
    return in ? ro : kOob;
}

// This lane's column against the window in dimension 0: v, the byte offset
// of its word in the row when every element of the word lies inside, else
// kOob; cut, whether the window takes some of the word's elements but not
// all (1- and 2-byte elements only).
struct C4Col {
    uint32_t v;
    bool cut;
};

template <int R>
__device__ __forceinline__ C4Col c4_col(const KArgs &A, const Win<R> &w, uint32_t lane) {
    const uint32_t xb = (lane & ((1u << A.c4_dshift) - 1u)) * 4u;
    const uint32_t e0 = xb >> A.c4_esz, e1 = (xb + 3u) >> A.c4_esz;  // the word's first and last element
    const bool full = (e0 >= w.lo[0]) && (e1 < w.hi[0]);
    const bool any = (e0 < w.hi[0]) && (e1 >= w.lo[0]) && (w.lo[0] < w.hi[0]);
    return {full ? xb : kOob, any && !full};
}

// The cut word at byte offset row + xb: its elements of ES bytes inside the
// window [lo0, hi0), loaded one by one, the others zero (what the
// out-of-range load landed for the whole word).
template <int ES>
__device__ __forceinline__ uint32_t c4_cut_word(__amdgpu_buffer_rsrc_t r, uint32_t row, uint32_t xb, uint32_t lo0,
                                                uint32_t hi0) {
    uint32_t w = 0;
#pragma unroll
    for (uint32_t b = 0; b < 4u; b += ES) {
        if (((xb + b) / ES) - lo0 >= hi0 - lo0) continue;
        const uint32_t v = ES == 1 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, row + xb + b, 0, 0)
                                   : (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, row + xb + b, 0, 0);
        w |= v << (8u * b);
    }
    return w;
}

// The landed stage's cut words (slots whose row is inside, lanes whose
// column the window cuts), rewritten whole with their inside elements.  In
// batches of 8 slots, so that a batch's loads are in flight together; every
// lane takes part in the row fetches, which read other lanes.
template <int NI, int ES>
__device__ __forceinline__ void c4_patch_cut(uint8_t *stage, uint32_t lane, bool cut, uint32_t rowv, uint32_t ra,
                                             uint32_t rstep, __amdgpu_buffer_rsrc_t r, uint32_t xb, uint32_t lo0,
                                             uint32_t hi0) {
    constexpr int B = NI < 8 ? NI : 8;
#pragma unroll 1
    for (int i0 = 0; i0 < NI; i0 += B) {
        uint32_t row[B], w[B];
#pragma unroll
        for (int j = 0; j < B; ++j)
            row[j] = (uint32_t)__builtin_amdgcn_ds_bpermute((int)(ra + (uint32_t)(i0 + j) * rstep), (int)rowv);
#pragma unroll
        for (int j = 0; j < B; ++j) w[j] = (cut && row[j] != kOob) ? c4_cut_word<ES>(r, row[j], xb, lo0, hi0) : 0u;
#pragma unroll
        for (int j = 0; j < B; ++j)
            if (cut && row[j] != kOob) *(uint32_t *)(stage + ((uint32_t)(i0 + j) * 64u + lane) * 4u) = w[j];
    }
}

// The stage's cut words stored through the destination: only their
// elements inside the window [lo0, hi0), one by one.  Batches of 8 slots as
// above (the words are read again from the stage: 1- and 2-byte elements
// take no +addend).
template <int NI, int ES, bool NT>
__device__ __forceinline__ void c4_store_cut(const uint8_t *stage, uint32_t lane, bool cut, uint32_t rowv, uint32_t ra,
                                             uint32_t rstep, __amdgpu_buffer_rsrc_t r, uint32_t xb, uint32_t lo0,
                                             uint32_t hi0) {
    constexpr int B = NI < 8 ? NI : 8;
#pragma unroll 1
    for (int i0 = 0; i0 < NI; i0 += B) {
        uint32_t row[B], w[B];
#pragma unroll
        for (int j = 0; j < B; ++j) {
            row[j] = (uint32_t)__builtin_amdgcn_ds_bpermute((int)(ra + (uint32_t)(i0 + j) * rstep), (int)rowv);
            w[j] = *(const uint32_t *)(stage + ((uint32_t)(i0 + j) * 64u + lane) * 4u);
        }
#pragma unroll
        for (int j = 0; j < B; ++j) {
            if (!cut || row[j] == kOob) continue;
#pragma unroll
            for (uint32_t b = 0; b < 4u; b += ES) {
                if (((xb + b) / ES) - lo0 >= hi0 - lo0) continue;
                if constexpr (ES == 1)
                    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(w[j] >> (8u * b)), r, row[j] + xb + b, 0, NT ? 2 : 0);
                else
                    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(w[j] >> (8u * b)), r, row[j] + xb + b, 0,
                                                          NT ? 2 : 0);
            }
        }
    }
}

// Slot i's offset: its row's value, fetched from the lane that holds it,
// plus the column.  The saturating add keeps kOob + anything >= kOob.
__device__ __forceinline__ uint32_t c4_slot(uint32_t rowv, uint32_t colv, uint32_t raddr) {
    const uint32_t r = (uint32_t)__builtin_amdgcn_ds_bpermute((int)raddr, (int)rowv);
    return __builtin_elementwise_add_sat(r, colv);
}

// Corner of tile t: uniform scalar loads through the constant address space.
template <int R>
__device__ __forceinline__ void c4_corner(const KArgs &A, const KMap &swept, int64_t t, int32_t (&c)[R]) {
    typedef const __attribute__((address_space(4))) int32_t const_i32;
    const int r = swept.rank;
    const_i32 *p = (const_i32 *)(A.coords) + t * r;
#pragma unroll
    for (int d = 0; d < R; ++d) c[d] = d < r ? p[d] : 0;
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
// `a` must stay the kernel's only argument: reread() finds it at the start
// of the argument segment.
template <int MODE, int NSLOT, int R, bool NTL, bool NTS, bool ADD, bool SAME>
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
    uint32_t parity = 0, k = 0;

    for (int64_t n = 0; n < cnt; ++n) {
        int32_t c[R];
        c4_corner<R>(a, sw, t, c);
        // the slots' row-fetch addresses are formed per box, not held across
        // the loop in NI registers
        uint32_t ra = raddr;
        asm volatile("" : "+v"(ra));
        if (a.flags & TMAP_FLAG_DEBUG_POISON) poison_blocks(stage, NSLOT, 1, lane);
        bar_arrive_expect(bar, budget, lane, 1);
        // destination offsets of the slots, held until the drain, and the
        // row tables and columns of the two sides for the cut words
        uint32_t off[NI];
        uint32_t srow = kOob, drow = kOob;
        C4Col scol = {kOob, false}, dcol = {kOob, false};
        if constexpr (MODE == kStore) {
            const uint64_t base = (uint64_t)a.packed + (uint64_t)t * bytes;
#pragma unroll
            for (int j = 0; j < NSLOT; ++j) {
                const uint32_t p = (uint32_t)j * 64u + lane;
                dma_lds_hint<NTL>(base, bytes, m0 + (uint32_t)j * kBlockBytes, p < a.n_chunks ? p * 16u : kOob);
            }
        } else {
            const Win<R> w = corner_window<R>(a.src, c);
            srow = c4_row<R>(a, a.src, w, lane);
            scol = c4_col<R>(a, w, lane);
            const uint64_t base = a.src.base + (uint64_t)corner_offset<R>(a, a.src, c);
            // every slot's offset first, so that the row fetches overlap,
            // then the loads
            uint32_t so[NI];
#pragma unroll
            for (int i = 0; i < NI; ++i) so[i] = c4_slot(srow, scol.v, ra + (uint32_t)i * rstep);
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
            drow = c4_row<R>(A, A.dst, w, lane);
            dcol = c4_col<R>(A, w, lane);
#pragma unroll
            for (int i = 0; i < NI; ++i) off[i] = c4_slot(drow, dcol.v, ra + (uint32_t)i * rstep);
        } else if constexpr (SAME) {
            drow = srow;
            dcol = scol;
        }

        // land: every slot's load has written the stage (zeros past the
        // tensor); the cut words' inside elements; then the record's byte
        // count and phase
        wait_vmcnt<0>();
        if constexpr (MODE != kStore) {
            if (__builtin_amdgcn_ballot_w64(scol.cut)) {
                const KArgs &A = reread(a);
                const Win<R> w = corner_window<R>(A.src, c);
                const __amdgpu_buffer_rsrc_t r =
                    make_rsrc(A.src.base + (uint64_t)corner_offset<R>(A, A.src, c), A.src.span);
                const uint32_t xb = (lane & ((1u << A.c4_dshift) - 1u)) * 4u;
                if (A.c4_esz == 0)
                    c4_patch_cut<NI, 1>(stage, lane, scol.cut, srow, ra, rstep, r, xb, w.lo[0], w.hi[0]);
                else
                    c4_patch_cut<NI, 2>(stage, lane, scol.cut, srow, ra, rstep, r, xb, w.lo[0], w.hi[0]);
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
            const __amdgpu_buffer_rsrc_t r = make_rsrc((uint64_t)a.packed + (uint64_t)t * bytes, bytes);
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
            if (__builtin_amdgcn_ballot_w64(dcol.cut)) {
                // the words the destination's window cuts, element by element
                const Win<R> w = corner_window<R>(dm, c);
                const uint32_t xb = (lane & ((1u << A.c4_dshift) - 1u)) * 4u;
                if (A.c4_esz == 0)
                    c4_store_cut<NI, 1, NTS>(stage, lane, dcol.cut, drow, ra, rstep, r, xb, w.lo[0], w.hi[0]);
                else
                    c4_store_cut<NI, 2, NTS>(stage, lane, dcol.cut, drow, ra, rstep, r, xb, w.lo[0], w.hi[0]);
            }
        }
        // the stage is free once these reads have completed
        __builtin_amdgcn_s_waitcnt(kWaitLgkm);
        asm volatile("" ::: "memory");
        const bool big = (k & a.group_mask) == a.group_mask;
        k += 1;
        t += big ? a.big_step : 1;
    }
    // nothing may still be writing LDS or memory when the wave ends
    __builtin_amdgcn_s_waitcnt(0);
}

template <int MODE, int NSLOT, int R, bool ADD, bool SAME>
KernelFn pick_corner4_hints(bool ntl, bool nts) {
    if constexpr (MODE == kRoundtrip) {
        // both sides are the tensor's: one hint for both
        (void)nts;
        return ntl ? corner4_kernel<MODE, NSLOT, R, true, true, ADD, SAME>
                   : corner4_kernel<MODE, NSLOT, R, false, false, ADD, SAME>;
    } else {
        if (ntl)
            return nts ? corner4_kernel<MODE, NSLOT, R, true, true, ADD, SAME>
                       : corner4_kernel<MODE, NSLOT, R, true, false, ADD, SAME>;
        return nts ? corner4_kernel<MODE, NSLOT, R, false, true, ADD, SAME>
                   : corner4_kernel<MODE, NSLOT, R, false, false, ADD, SAME>;
    }
}

template <int MODE, int R, bool ADD, bool SAME = false>
KernelFn pick_corner4(int nslot, bool ntl, bool nts) {
    switch (nslot) {
        case 1: return pick_corner4_hints<MODE, 1, R, ADD, SAME>(ntl, nts);
        case 2: return pick_corner4_hints<MODE, 2, R, ADD, SAME>(ntl, nts);
        case 4: return pick_corner4_hints<MODE, 4, R, ADD, SAME>(ntl, nts);
        case 8: return pick_corner4_hints<MODE, 8, R, ADD, SAME>(ntl, nts);
        default: return nullptr;
    }
}

// Launch the 4-byte-lane corner kernel of direction MODE over a.grid waves
// (wave_group to a workgroup).  hipError_t as int.
template <int MODE, int R>
int launch_corner4_mode(int nslot, const KArgs &a, void *stream) {
    const bool ntl = nontemporal_loads<MODE>(a.flags), nts = nontemporal_stores<MODE>(a.flags);
    KernelFn fn = nullptr;
    if constexpr (MODE == kRoundtrip) {
        if (same_shape(a.src, a.dst))
            fn = a.add_f32 ? pick_corner4<MODE, R, true, true>(nslot, ntl, nts)
                           : pick_corner4<MODE, R, false, true>(nslot, ntl, nts);
        else
            fn = a.add_f32 ? pick_corner4<MODE, R, true>(nslot, ntl, nts)
                           : pick_corner4<MODE, R, false>(nslot, ntl, nts);
    } else {
        fn = pick_corner4<MODE, R, false>(nslot, ntl, nts);
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
