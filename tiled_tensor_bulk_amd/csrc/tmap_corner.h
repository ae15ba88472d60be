// tmap_corner.h -- the copy of boxes at explicit corners, or over a sweep,
// one wave per box, written for the fewest instructions per box; a wave that
// takes several boxes keeps one loading while it stores the one before.
//
// Each wave walks its own share of the corners (or of the sweep's boxes,
// with the carry-add cursor of the other kernels) through one LDS stage of
// one box (NSLOT KiB, NSLOT <= 8) and its own 8-byte barrier record:
//
//   fill    take the corner (scalar loads from the corner list, or the
//           cursor's digits times the box), rebase the buffer resource to it,
//           and issue one 16-byte direct-to-LDS load per slot: slot p takes
//           the logical chunk swizzle(p), so the swizzle is applied as the
//           bytes land ("TMA -- the async bulk copy engine", "The descriptor
//           records the layout, including the swizzle").  A box wholly
//           inside the tensor uses the per-slot offsets as they are; an edge
//           box sends the chunks that are not wholly inside to the
//           out-of-range offset, which lands as zeros ("GPU TMA", "Why
//           architecture matters here"), and patches the chunks the tensor's
//           dimension-0 edge cuts through element by element when they land.
//   land    wait for the box's loads (vmcnt), complete the wave's byte budget
//           on the stage record and wait for its phase ("TMA -- the async
//           bulk copy engine", "Load completion -- the mbarrier and the byte
//           budget"; "Understanding TMA loads in CuTe DSL", "Issue the load
//           and wait for its phase").
//   hold    read the box's image out of the stage into registers; the stage
//           is then free, and the next box's loads are issued into it.
//   drain   store the held image: a load writes it to the packed images; a
//           store or round trip stores each logical chunk through the
//           destination map, clipped to its bounds.  Chunks the destination's
//           edge cuts through are stored element by element from the stage,
//           before it is refilled.
//
// So a box's stores are issued after the next box's loads, and the next
// landing waits for those loads alone (vmcnt leaves the stores in flight).
// Per-slot
// quantities (box indices, in-box offsets in both maps) are computed once per
// kernel; per box only the scalar corner, base addresses and bounds change,
// and an edge box costs a few vector compares per slot.

#pragma once

#include "tmap_copy.h"

namespace tmap {
namespace {

// The tiles of walker g (a wave), dealt as the other variants deal them to
// their walkers: groups of a.group consecutive tiles, round robin, as
// a.regions interleaved streams.  cnt tiles from t0 (none for a wave past
// the grid).
__device__ __forceinline__ void corner_deal(const KArgs &a, int64_t g, int64_t &cnt, int64_t &t0) {
    const bool walker = g < (int64_t)a.grid;
    if (a.regions > 1) {
        const uint32_t per = a.grid / a.regions;
        if ((uint32_t)g < per * a.regions) g = (int64_t)((uint32_t)g % a.regions) * per + (uint32_t)g / a.regions;
    }
    if (a.group == 0) {
        cnt = a.deal_q + (g < a.deal_r ? 1 : 0);
        t0 = g * a.deal_q + (g < a.deal_r ? g : a.deal_r);
    } else {
        const int64_t Q = a.group;
        int64_t last = a.deal_r - g * Q;
        last = last < 0 ? 0 : (last > Q ? Q : last);
        cnt = a.deal_q * Q + last;
        t0 = g * Q;
    }
    if (!walker) cnt = 0;
}

// Byte offset of a box corner from the map's base.  With small offsets (the
// host has checked that every corner whose box touches the tensor is less
// than 2 GiB from the base in every direction) the sum is taken in 32 bits:
// a box that does not touch the tensor gets a meaningless offset, but none
// of its chunks is read or written.
template <int R>
__device__ __forceinline__ int64_t corner_offset(const KArgs &A, const KMap &m, const int32_t (&c)[R]) {
    if (A.off32) {
        uint32_t o = 0;
#pragma unroll
        for (int d = 0; d < R; ++d) o += (uint32_t)c[d] * (uint32_t)m.strides[d];
        return (int64_t)(int32_t)o;
    }
    int64_t o = 0;
#pragma unroll
    for (int d = 0; d < R; ++d) o += (int64_t)c[d] * (int64_t)m.strides[d];
    return o;
}

// Whether the box at corner c lies wholly inside the tensor.
template <int R>
__device__ __forceinline__ bool corner_inside(const KMap &m, const int32_t (&c)[R]) {
    bool in = true;
#pragma unroll
    for (int d = 0; d < R; ++d) in = in & (c[d] >= 0) & (c[d] <= m.lim[d]);
    return in;
}

// Per dimension, the window [lo, hi) of box indices inside the tensor, in
// 32-bit scalar arithmetic: dims <= 2^31 and box extents <= 256, so every
// difference taken below fits (a corner below -box or past dims gives an
// empty window).
template <int R>
__device__ __forceinline__ Win<R> corner_window(const KMap &m, const int32_t (&c)[R]) {
    Win<R> w;
#pragma unroll
    for (int d = 0; d < R; ++d) {
        const int32_t cd = c[d];
        const uint32_t b = m.box[d];
        const uint32_t lo = cd >= 0 ? 0u : (cd <= -(int32_t)b ? b : 0u - (uint32_t)cd);
        const int32_t lim = (int32_t)(m.dims[d] - b);           // dims - box, negative if the box is larger
        const int32_t hr = (int32_t)(m.dims[d] - (uint32_t)cd);  // dims - c when c > lim: below box
        w.lo[d] = lo;
        w.hi[d] = cd <= lim ? b : (hr < (int32_t)lo ? lo : (uint32_t)hr);
    }
    return w;
}

// SAME: a round trip whose destination map has the source's dims and strides
// (only its base differs), so the drain takes the source map's offsets,
// interior test and windows.
//
// Across the loop a wave holds its tile positions, the corners of the box
// in the stage and of the next one, and per-slot vectors.  The map fields
// stay in scalar registers where one map serves both sides; a round trip
// between two maps reads them again in each phase (scalar loads that hit
// the constant cache), as both would not fit, and every slow path does.
template <int MODE, int NSLOT, int R, bool NTL, bool NTS, bool ADD, bool SAME = false>
struct CornerCopier {
    static_assert(NSLOT <= 8, "the held image takes 4 VGPRs per slot");
    static_assert(!SAME || MODE == kRoundtrip, "a load or store has one tensor map");
    const KArgs &a;
    uint32_t lane, parity;
    int64_t cnt;
    // the box to fill next: a tile index, the position in this wave's
    // sequence and, over a sweep, the tile's digits; the box to drain needs
    // only its tile index and position (for its packed image)
    Cursor<R> fcur;
    int64_t ct;
    uint32_t ck;
    int32_t fc[R];  // corner of the box under the fill cursor, read one fill ahead
    int32_t sc[R];  // corner of the box in the stage
    bool edge;      // the box in the stage needs its cut chunks patched
    bool behind;    // exactly NSLOT stores (one drain) were issued after the stage's loads
    // per slot: the logical chunk's box indices (x0 | i1 << 16, i2 | i3 << 8
    // | i4 << 16) and its in-box byte offsets in the source and destination
    // maps (for a load the destination side is the slot's image offset, for
    // a store the source side is).  A slot past the box has the out-of-range
    // offsets and indices no window contains, so no test is needed per box.
    uint32_t w0[NSLOT], w1[NSLOT], soff[NSLOT], doff[NSLOT];
    uint64_t *bar;

    __device__ __forceinline__ CornerCopier(const KArgs &args, uint64_t *b) : a(args), bar(b) {}

    __device__ __forceinline__ static const KMap &swept(const KArgs &A) { return MODE == kStore ? A.dst : A.src; }

    // The arguments fill and drain read.  With one map (a load, a store, a
    // round trip between maps of the same shape) they stay in scalar
    // registers, some spilled to vector lanes, and the loads and stores
    // issue without waiting for an argument read: measured faster than
    // reading them again (10^5 scattered 8 KiB boxes: store 0.622 -> 0.633
    // of peak, round trip 0.355 -> 0.366).  A round trip between two
    // different maps reads them again each time: both would not fit.
    __device__ __forceinline__ const KArgs &side_args() const { return (MODE != kRoundtrip || SAME) ? a : reread(a); }

    // The destination's dims, strides and span (its base is always A.dst's).
    __device__ __forceinline__ static const KMap &dst_shape(const KArgs &A) { return SAME ? A.src : A.dst; }

    __device__ __forceinline__ void setup(uint32_t hw, uint32_t wg) {
        lane = threadIdx.x & 63u;
        parity = 0;
        edge = false;
        behind = false;
        int64_t t0;
        corner_deal(a, (int64_t)blockIdx.x * wg + hw, cnt, t0);
        ct = t0;
        ck = 0;
        if (a.coords) {
            fcur.t = t0;
            fcur.k = 0;
        } else {
            cursor_init<R>(a, t0, fcur);
        }
        const KMap &sw = swept(a);
#pragma unroll
        for (int j = 0; j < NSLOT; ++j) {
            const uint32_t p = (uint32_t)j * 64u + lane;
            w0[j] = w1[j] = 0xFFFFFFFFu;
            soff[j] = doff[j] = kOob;
            if (p < a.n_chunks) {
                uint32_t off;
                chunk_info_of<R>(a, logical_chunk_of(a, p, sw), sw, off, w0[j], w1[j]);
                if (MODE == kLoad) {
                    soff[j] = off;
                    doff[j] = p * 16u;
                } else if (MODE == kStore) {
                    soff[j] = p * 16u;
                    doff[j] = off;
                } else {
                    soff[j] = off;
                    // the destination has the same box and swizzle, maybe other strides
                    uint32_t o2 = off, u0, u1;
                    if (!SAME) chunk_info_of<R>(a, logical_chunk_of(a, p, a.dst), a.dst, o2, u0, u1);
                    doff[j] = o2;
                }
            }
        }
        if (cnt > 0) cursor_corner<R>(a, sw, fcur, fc);
    }

    // Next tile of the drain's sequence: +1 inside a group, big_step after
    // its last.
    __device__ __forceinline__ static void advance(const KArgs &A, int64_t &t, uint32_t &k) {
        const bool big = (k & A.group_mask) == A.group_mask;
        k += 1;
        t += big ? A.big_step : 1;
    }

    // slot j's direct-to-LDS load: lane l's 16 bytes at voff land at m0 + j KiB + 16 l
    __device__ __forceinline__ static void dma(uint64_t base, uint32_t nrec, uint32_t m0, int j, uint32_t voff) {
        dma_lds_hint<NTL>(base, nrec, m0 + (uint32_t)j * kBlockBytes, voff);
    }

    // Issue the loads of the box under the fill cursor into the stage.
    __device__ __forceinline__ void fill(uint8_t *stage, int64_t nfill) {
        const KArgs &A = side_args();
#pragma unroll
        for (int d = 0; d < R; ++d) sc[d] = fc[d];
        if (a.flags & TMAP_FLAG_DEBUG_POISON) poison_blocks(stage, NSLOT, 1, lane);
        const uint32_t budget = a.src.box_bytes + ((a.flags & TMAP_FLAG_INJECT_BUDGET_MISMATCH) ? 16u : 0u);
        bar_arrive_expect(bar, budget, lane, 1);
        const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void_t *)stage;
        if (MODE == kStore) {
            // the packed images' fields stay in registers: the loads issue
            // without waiting for an argument read
            const uint64_t base = (uint64_t)a.packed + (uint64_t)fcur.t * a.dst.box_bytes;
#pragma unroll
            for (int j = 0; j < NSLOT; ++j) dma(base, a.dst.box_bytes, m0, j, soff[j]);
            edge = false;
        } else {
            const uint64_t base = A.src.base + (uint64_t)corner_offset<R>(A, A.src, sc);
            if (corner_inside<R>(A.src, sc)) {
#pragma unroll
                for (int j = 0; j < NSLOT; ++j) dma(base, A.src.span, m0, j, soff[j]);
                edge = false;
            } else {
                const Win<R> w = corner_window<R>(A.src, sc);
#pragma unroll
                for (int j = 0; j < NSLOT; ++j)
                    dma(base, A.src.span, m0, j, classify<R>(w0[j], w1[j], w, A.k_el) == kFull ? soff[j] : kOob);
                edge = cuts_chunks(A, w);
            }
        }
        cursor_advance<R>(a, fcur);
        // take the next corner now, while this box's loads fly (never past
        // this wave's last tile: an explicit-corner array ends there)
        if (nfill + 1 < cnt) cursor_corner<R>(A, swept(A), fcur, fc);
    }

    // Whether window w cuts through a 16-byte chunk in dimension 0.
    __device__ __forceinline__ static bool cuts_chunks(const KArgs &A, const Win<R> &w) {
        bool rows = true;
#pragma unroll
        for (int d = 1; d < R; ++d) rows = rows & (w.lo[d] < w.hi[d]);
        return rows & (w.lo[0] < w.hi[0]) & (((w.lo[0] | w.hi[0]) & (A.k_el - 1u)) != 0u);
    }

    // Land the box in the stage: wait for its loads, patch its cut chunks,
    // complete the byte budget, wait for the phase.  False on a timeout.
    __device__ __forceinline__ bool land(uint8_t *stage) {
        // after this box's loads the wave issued the previous box's drain;
        // when that was NSLOT plain stores they may stay in flight (the
        // counter retires operations in issue order)
        if (behind)
            wait_vmcnt<NSLOT>();
        else
            wait_vmcnt<0>();
        if (MODE != kStore && edge) {
            // slow path, kept out of the unrolled slot arrays: each slot's
            // chunk is recomputed
            const KArgs &A = reread(a);
            const Win<R> w = corner_window<R>(A.src, sc);
            const __amdgpu_buffer_rsrc_t r =
                make_rsrc(A.src.base + (uint64_t)corner_offset<R>(A, A.src, sc), A.src.span);
#pragma unroll 1
            for (int j = 0; j < NSLOT; ++j) {
                const uint32_t p = (uint32_t)j * 64u + lane;
                if (p >= A.n_chunks) continue;
                uint32_t off, u0, u1;
                chunk_info_of<R>(A, logical_chunk_of(A, p, A.src), A.src, off, u0, u1);
                if (classify<R>(u0, u1, w, A.k_el) == kPart)
                    load_chunk_edge_es(A.src.elem_size, stage + p * 16u, off, u0 & 0xFFFFu, w.lo[0], w.hi[0], r);
            }
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm);
        asm volatile("" ::: "memory");
        bar_complete(bar, a.src.box_bytes, lane, 1);
        const bool ok = bar_wait(bar, parity, a.spin_limit);
        parity ^= 1u;
        asm volatile("" ::: "memory");
        return ok;
    }

    template <typename Rs>
    __device__ __forceinline__ static void store16(const i32x4 &v, Rs r, uint32_t off) {
        if constexpr (NTS)
            __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 2);
        else
            __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
    }

    // Chunks of the box in the stage that the destination's dimension-0
    // edge cuts through: store their inside elements, read from the stage,
    // before the stage is refilled (so these stores precede the next box's
    // loads and the next landing need not count them).  Slow path, kept out
    // of the unrolled slot arrays.
    __device__ __forceinline__ void drain_cut_chunks(const uint8_t *stage, const int32_t (&c)[R]) const {
        if (MODE == kLoad) return;
        const KArgs &A = side_args();
        const KMap &dm = dst_shape(A);
        if (corner_inside<R>(dm, c)) return;
        const Win<R> w = corner_window<R>(dm, c);
        if (!cuts_chunks(A, w)) return;
        const __amdgpu_buffer_rsrc_t r = make_rsrc(A.dst.base + (uint64_t)corner_offset<R>(A, dm, c), dm.span);
#pragma unroll 1
        for (int j = 0; j < NSLOT; ++j) {
            const uint32_t p = (uint32_t)j * 64u + lane;
            if (p >= A.n_chunks) continue;
            uint32_t off, u0, u1;
            chunk_info_of<R>(A, logical_chunk_of(A, p, dm), dm, off, u0, u1);
            if (classify<R>(u0, u1, w, A.k_el) == kPart)
                store_chunk_edge_es(A.dst.elem_size, stage + p * 16u, off, u0 & 0xFFFFu, w.lo[0], w.hi[0], r, ADD,
                                    A.addend);
        }
    }

    // Store the whole chunks of the held image of the box under the drain
    // cursor: always NSLOT stores per lane, chunks with nothing to write
    // going to the out-of-range offset, so that the next landing can count
    // them.
    __device__ __forceinline__ void drain(i32x4 (&v)[NSLOT], const int32_t (&c)[R], bool after_fill) {
        // the next landing may leave these NSLOT stores in flight when they
        // are the only operations issued after its loads
        behind = after_fill;
        const KArgs &A = side_args();
        if (MODE == kLoad) {
            const __amdgpu_buffer_rsrc_t r =
                make_rsrc((uint64_t)A.packed + (uint64_t)ct * A.src.box_bytes, A.src.box_bytes);
#pragma unroll
            for (int j = 0; j < NSLOT; ++j) store16(v[j], r, doff[j]);
            advance(a, ct, ck);
            return;
        }
        if constexpr (ADD) {
            // the tile update of the fused round trip, in the held registers
            typedef __attribute__((ext_vector_type(4))) float f32x4;
#pragma unroll
            for (int j = 0; j < NSLOT; ++j) v[j] = __builtin_bit_cast(i32x4, __builtin_bit_cast(f32x4, v[j]) + A.addend);
        }
        const KMap &dm = dst_shape(A);
        const __amdgpu_buffer_rsrc_t r = make_rsrc(A.dst.base + (uint64_t)corner_offset<R>(A, dm, c), dm.span);
        if (corner_inside<R>(dm, c)) {
#pragma unroll
            for (int j = 0; j < NSLOT; ++j) store16(v[j], r, doff[j]);
        } else {
            const Win<R> w = corner_window<R>(dm, c);
#pragma unroll
            for (int j = 0; j < NSLOT; ++j)
                store16(v[j], r, classify<R>(w0[j], w1[j], w, A.k_el) == kFull ? doff[j] : kOob);
        }
        advance(a, ct, ck);
    }
};

// `a` must stay the kernel's only argument: reread() finds it at the start
// of the argument segment.
template <int MODE, int NSLOT, int R, bool NTL, bool NTS, bool ADD, bool SAME>
__global__ __launch_bounds__(64 * wave_group(NSLOT)) void corner_kernel(const KArgs a) {
    constexpr int WG = wave_group(NSLOT);
    constexpr uint32_t SB = NSLOT * kBlockBytes;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[WG * SB];
    __shared__ uint64_t bars[WG];

    const uint32_t hw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    CornerCopier<MODE, NSLOT, R, NTL, NTS, ADD, SAME> cp(a, &bars[hw]);
    if ((threadIdx.x & 63u) == 0) bars[hw] = 0;
    cp.setup(hw, WG);
    // each wave owns its record and stage: its own LDS write is ordered
    // before its own atomics on it
    __builtin_amdgcn_s_waitcnt(kWaitLgkm);
    if (cp.cnt <= 0) return;
    uint8_t *stage = ring + hw * SB;

    i32x4 held[NSLOT];
    cp.fill(stage, 0);
    for (int64_t k = 0; k < cp.cnt; ++k) {
        // the per-slot box indices are unpacked where they are tested, not
        // once before the loop: unpacked, they would take four times the
        // vector registers for the whole loop
#pragma unroll
        for (int j = 0; j < NSLOT; ++j) asm volatile("" : "+v"(cp.w0[j]), "+v"(cp.w1[j]));
        if (!cp.land(stage)) {
            if (cp.lane == 0) __hip_atomic_fetch_or(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        // the box's corner, kept before the next fill replaces it
        int32_t c[R];
#pragma unroll
        for (int d = 0; d < R; ++d) c[d] = cp.sc[d];
#pragma unroll
        for (int j = 0; j < NSLOT; ++j) held[j] = *(const i32x4 *)(stage + ((uint32_t)j * 64u + cp.lane) * 16u);
        cp.drain_cut_chunks(stage, c);
        // the stage is free once these reads have completed
        __builtin_amdgcn_s_waitcnt(kWaitLgkm);
        asm volatile("" ::: "memory");
        const bool more = k + 1 < cp.cnt;
        if (more) cp.fill(stage, k + 1);
        cp.drain(held, c, more);
    }
    // nothing may still be writing LDS or memory when the wave ends
    __builtin_amdgcn_s_waitcnt(0);
}

template <int MODE, int NSLOT, int R, bool ADD, bool SAME>
KernelFn pick_corner_hints(bool ntl, bool nts) {
    if (ntl)
        return nts ? corner_kernel<MODE, NSLOT, R, true, true, ADD, SAME>
                   : corner_kernel<MODE, NSLOT, R, true, false, ADD, SAME>;
    return nts ? corner_kernel<MODE, NSLOT, R, false, true, ADD, SAME>
               : corner_kernel<MODE, NSLOT, R, false, false, ADD, SAME>;
}

template <int MODE, int R, bool ADD, bool SAME = false>
KernelFn pick_corner(int nslot, bool ntl, bool nts) {
    switch (nslot) {
        case 1: return pick_corner_hints<MODE, 1, R, ADD, SAME>(ntl, nts);
        case 2: return pick_corner_hints<MODE, 2, R, ADD, SAME>(ntl, nts);
        case 4: return pick_corner_hints<MODE, 4, R, ADD, SAME>(ntl, nts);
        case 8: return pick_corner_hints<MODE, 8, R, ADD, SAME>(ntl, nts);
        default: return nullptr;
    }
}

// Whether a round trip's destination map has the source's dims, strides and
// span (only the base differs).
inline bool same_shape(const KMap &s, const KMap &d) {
    for (int k = 0; k < kMaxRank; ++k)
        if (s.dims[k] != d.dims[k] || s.strides[k] != d.strides[k]) return false;
    return s.span == d.span;
}

// Launch the corner kernel of direction MODE over a.grid waves (wave_group
// to a workgroup).  hipError_t as int.
template <int MODE, int R>
int launch_corner_mode(int nslot, const KArgs &a, void *stream) {
    const bool ntl = nontemporal_loads<MODE>(a.flags), nts = nontemporal_stores<MODE>(a.flags);
    KernelFn fn = nullptr;
    if constexpr (MODE == kRoundtrip) {
        // the same-shape round trip has its own instances for maps of rank
        // > 2, where the two maps' fields would not fit in scalar registers
        if (R > 2 && same_shape(a.src, a.dst))
            fn = a.add_f32 ? pick_corner<MODE, R, true, true>(nslot, ntl, nts)
                           : pick_corner<MODE, R, false, true>(nslot, ntl, nts);
        else
            fn = a.add_f32 ? pick_corner<MODE, R, true>(nslot, ntl, nts) : pick_corner<MODE, R, false>(nslot, ntl, nts);
    } else {
        fn = pick_corner<MODE, R, false>(nslot, ntl, nts);
    }
    if (!fn) return (int)hipErrorInvalidValue;
    const uint32_t wg = (uint32_t)wave_group(nslot);
    KArgs copy = a;
    void *args[] = {&copy};
    // the reserve is allocated as dynamic LDS the kernel does not touch
    return (int)hipLaunchKernel((const void *)fn, dim3((a.grid + wg - 1) / wg), dim3(64 * wg), args,
                                corner_lds_reserve(MODE, nslot), (hipStream_t)stream);
}

}  // namespace
}  // namespace tmap
