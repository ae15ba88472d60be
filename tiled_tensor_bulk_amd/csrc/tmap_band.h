// tmap_band.h -- the band-schedule copy for maps of rank <= 2 (and batches
// of such planes: rank 3 with boxes of extent 1 in dimension 2), written for
// the fewest instructions per byte.
//
// A sweep of boxes with rows of 64..512 bytes runs on the band schedule: a
// 16 KiB stage holds one "unit", the same band of H rows of the G boxes that
// are neighbours in dimension 0 (G * H * row bytes = 16 KiB), each box's band
// being the contiguous piece of that box's swizzled LDS image it always is.
// For maps of rank <= 2 whose rows are whole 16-byte chunks (so no chunk is
// ever cut by the tensor's dimension-0 edge), and batches of such planes
// walked plane after plane, this kernel replaces the generic ring of
// tmap_copy.h on that schedule.  Same steps, same results:
//
//   fill    every lane issues one 16-byte direct-to-LDS buffer load per slot
//           it owns (4 slots: 16 KiB over 256 lanes); slot p receives the
//           logical chunk swizzle(p) of its box's band, so the swizzle is
//           applied as the bytes land ("TMA -- the async bulk copy engine",
//           "The descriptor records the layout, including the swizzle").
//           Chunks outside the tensor get the out-of-range offset and land as
//           zeros ("GPU TMA", "Why architecture matters here").
//   land    the wave waits for its own loads (an exact vmcnt that leaves the
//           later fills and the earlier drains in flight) and completes its
//           byte budget on the stage's record ("TMA -- the async bulk copy
//           engine", "Load completion -- the mbarrier and the byte budget").
//   ready   consumers wait for the record's phase to flip ("Understanding TMA
//           loads in CuTe DSL", "Issue the load and wait for its phase"); a
//           consumer reads the slots the next wave filled, so only the byte
//           count makes the read safe.
//   consume load: the stage's slots go to the packed images; store / round
//           trip: each logical chunk is stored through the destination map,
//           clipped to its bounds.
//   release one s_barrier per unit before its stage is refilled.
//
// What makes it lean: every per-slot quantity (in-unit offsets on both
// sides, the chunk's column and row for the bounds test) is computed once
// per kernel from shifts and masks, as box rows, band heights and boxes per
// unit are powers of two; per unit only the scalar base addresses and two
// scalar limits change, and an edge unit costs two vector compares per slot;
// the cache hints are template parameters, so no branch sits between the
// loads; one asm block issues a unit's four loads.

#pragma once

#include "tmap_copy.h"

namespace tmap {
namespace {

constexpr uint32_t kUnitBytes = kBandSlots * kWaves * kBlockBytes;  // one 16 KiB stage
constexpr uint32_t kUnitWaveStep = kWaves * kBlockBytes;           // LDS bytes between a lane's slots

// The four direct-to-LDS loads of a wave's slots of one unit: slot jj of the
// wave lands in the 1 KiB block at m0 + jj * 4 KiB, lane l's 16 bytes at
// +16*l, read from voff[jj] of the buffer (base, nrec).  Issued as one asm
// block for the reasons given at dma_lds; M0 is restored at the end.
template <bool NT>
__device__ __forceinline__ void dma4(uint64_t base, uint32_t nrec, uint32_t m0, const uint32_t (&voff)[kBandSlots]) {
    const i32x4 d = {__builtin_amdgcn_readfirstlane((int)(uint32_t)base),
                     __builtin_amdgcn_readfirstlane((int)((uint32_t)(base >> 32) & 0xFFFFu)),
                     __builtin_amdgcn_readfirstlane((int)nrec), kRsrcWord3};
    const uint32_t a0 = __builtin_amdgcn_readfirstlane((int)m0);
    const uint32_t a1 = a0 + kUnitWaveStep, a2 = a0 + 2 * kUnitWaveStep, a3 = a0 + 3 * kUnitWaveStep;
    uint32_t saved;
    if constexpr (NT)
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %1\n\ts_nop 4\n\tbuffer_load_dwordx4 %5, %9, 0 offen nt lds\n\ts_nop 0\n\t"
            "s_mov_b32 m0, %2\n\ts_nop 4\n\tbuffer_load_dwordx4 %6, %9, 0 offen nt lds\n\ts_nop 0\n\t"
            "s_mov_b32 m0, %3\n\ts_nop 4\n\tbuffer_load_dwordx4 %7, %9, 0 offen nt lds\n\ts_nop 0\n\t"
            "s_mov_b32 m0, %4\n\ts_nop 4\n\tbuffer_load_dwordx4 %8, %9, 0 offen nt lds\n\ts_nop 0\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(a0), "s"(a1), "s"(a2), "s"(a3), "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(d)
            : "memory");
    else
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %1\n\ts_nop 4\n\tbuffer_load_dwordx4 %5, %9, 0 offen lds\n\ts_nop 0\n\t"
            "s_mov_b32 m0, %2\n\ts_nop 4\n\tbuffer_load_dwordx4 %6, %9, 0 offen lds\n\ts_nop 0\n\t"
            "s_mov_b32 m0, %3\n\ts_nop 4\n\tbuffer_load_dwordx4 %7, %9, 0 offen lds\n\ts_nop 0\n\t"
            "s_mov_b32 m0, %4\n\ts_nop 4\n\tbuffer_load_dwordx4 %8, %9, 0 offen lds\n\ts_nop 0\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(a0), "s"(a1), "s"(a2), "s"(a3), "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(d)
            : "memory");
}

// vmcnt(n) for a wave-uniform n that is a multiple of 4 in [0, 8(S-1)]
// (s_waitcnt takes an immediate); rounds down, which only waits longer.
template <int S>
__device__ __forceinline__ void wait_vmcnt_upto(uint32_t n) {
    switch (n >> 2) {
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<4>(); break;
        case 2: wait_vmcnt<8>(); break;
        case 3: wait_vmcnt<12>(); break;
        case 4: wait_vmcnt<16>(); break;
        case 5: wait_vmcnt<20>(); break;
        default: wait_vmcnt<(S > 3 ? 24 : (S > 2 ? 16 : 8))>(); break;
    }
}

// Geometry of one slot of a unit (p = stage slot 0..1023): its box g in the
// unit, its chunk l in that box's band, and where the logical chunk
// swizzle(l) sits in the band: row r and 16-byte column cc of the box.
struct SlotGeom {
    uint32_t g, l, r, cc;
};

__device__ __forceinline__ SlotGeom slot_geom(uint32_t p, uint32_t lbc, uint32_t lrc, uint32_t lk, const KMap &m) {
    SlotGeom s;
    s.g = p >> lbc;
    s.l = p & ((1u << lbc) - 1u);
    // the swizzle moves whole chunks here (its granule is >= 16 bytes)
    const uint32_t lc = swizzle(s.l << lk, m.swz_b, m.swz_m, m.swz_s) >> lk;
    s.r = lc >> lrc;
    s.cc = lc & ((1u << lrc) - 1u);
    return s;
}

// One side of a unit: where its region starts and which of its chunks lie
// inside the map (scalar; the same for every lane).
// Whether a slot's chunk (column | row << 16 within the unit) lies inside a
// side whose first xl columns and rl rows lie inside its map.
__device__ __forceinline__ bool slot_inside(uint32_t xy, int32_t xl, int32_t rl) {
    return ((int32_t)(xy & 0xFFFFu) < xl) & ((int32_t)(xy >> 16) < rl);
}

struct Side {
    uint64_t base;  // first byte of the unit's region
    uint32_t nrec;  // buffer records from there
    int32_t xl;     // 16-byte columns of the unit that lie inside the map (clamped to [0, unit width])
    int32_t rl;     // rows of the band that lie inside the map (clamped to [0, H])
    bool inside;    // every chunk of the unit lies inside
};

template <int MODE, int S, bool NTL, bool NTS, bool ADD>
struct BandCopier {
    const KArgs &a;
    uint32_t lane, wave, parity;
    // shapes (log2): 16-byte chunks per box row, per box band; band rows; boxes per unit
    uint32_t lrc, lbc, lh, lg, lk;
    int64_t cnt;
    Cursor<3> fcur, ccur;
    // producer slots (filled by this lane): source offsets in the unit, and
    // column | row << 16 for the bounds test (packed offsets for a store)
    uint32_t poff[kBandSlots], pxy[kBandSlots];
    // consumer slots (the slots the next wave filled): destination offsets
    // and column | row << 16 (packed offsets for a load)
    uint32_t coff[kBandSlots], cxy[kBandSlots];
    uint64_t *bars;

    __device__ __forceinline__ BandCopier(const KArgs &args, uint64_t *b) : a(args), bars(b) {}

    __device__ __forceinline__ const KMap &swept() const { return MODE == kStore ? a.dst : a.src; }

    __device__ __forceinline__ void setup() {
        lane = threadIdx.x & 63u;
        wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        parity = 0;
        const KMap &sw = swept();
        lrc = __builtin_ctz(a.row_chunks);
        lbc = a.band_lbc;
        lh = __builtin_ctz(a.ubox[1]);
        lg = __builtin_ctz(a.band_g);
        lk = 4u - __builtin_ctz((uint32_t)sw.elem_size);
        // the deal: groups of a.group consecutive units, round robin over the
        // workgroups, optionally as a.regions interleaved streams (as the
        // generic ring deals them)
        int64_t g = blockIdx.x;
        if (a.regions > 1) {
            const uint32_t per = a.grid / a.regions;
            if ((uint32_t)g < per * a.regions) g = (int64_t)((uint32_t)g % a.regions) * per + (uint32_t)g / a.regions;
        }
        int64_t t0;
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
        if (g >= (int64_t)a.grid) cnt = 0;
        cursor_init<3>(a, t0, fcur);
        ccur = fcur;
        const uint32_t cw = (wave + 1u) & (kWaves - 1u);
        const uint32_t bb = sw.box_bytes;
#pragma unroll
        for (int jj = 0; jj < kBandSlots; ++jj) {
            const SlotGeom ps = slot_geom(((uint32_t)(jj * kWaves) + wave) * 64u + lane, lbc, lrc, lk, sw);
            const SlotGeom cs = slot_geom(((uint32_t)(jj * kWaves) + cw) * 64u + lane, lbc, lrc, lk, sw);
            const uint32_t rb = 16u << lrc;
            if (MODE == kStore) {
                poff[jj] = ps.g * bb + ps.l * 16u;
                pxy[jj] = 0;
            } else {
                poff[jj] = (uint32_t)((uint64_t)ps.r * a.src.strides[1]) + ps.g * rb + ps.cc * 16u;
                pxy[jj] = ((ps.g << lrc) + ps.cc) | (ps.r << 16);
            }
            if (MODE == kLoad) {
                coff[jj] = cs.g * bb + cs.l * 16u;
                cxy[jj] = 0;
            } else {
                coff[jj] = (uint32_t)((uint64_t)cs.r * a.dst.strides[1]) + cs.g * rb + cs.cc * 16u;
                cxy[jj] = ((cs.g << lrc) + cs.cc) | (cs.r << 16);
            }
        }
    }

    // The tensor side of the unit under cur in map m; `boxes` caps the
    // columns at the unit's existing boxes (a round trip's destination may
    // reach past the swept source's last box).
    __device__ __forceinline__ Side tensor_side(const KMap &m, const Cursor<3> &cur, uint32_t boxes) const {
        Side s;
        const uint32_t ux = cur.dig[0], v = cur.dig[1], z = cur.dig[2];
        const uint32_t width = boxes << lrc;  // 16-byte columns of the unit's existing boxes
        const uint32_t x0 = ux << (lg + lrc), y0 = v << lh, h = 1u << lh;
        // a map of rank 3 is a batch of planes (boxes of extent 1 in
        // dimension 2): the third digit is the plane; rank 2 keeps it 0
        s.base = m.base + (uint64_t)z * m.strides[2] + (uint64_t)y0 * m.strides[1] + ((uint64_t)x0 << 4);
        s.nrec = m.span;
        // 16-byte columns and rows of the map (dims[0] * elem_size is a
        // multiple of 16, checked on the host; both fit 31 bits, and so do
        // x0 and y0, which stay within a unit of the sweep's end)
        const uint32_t xc = m.dims[0] >> lk, yc = m.dims[1];
        const uint32_t xl = x0 >= xc ? 0u : (xc - x0 < width ? xc - x0 : width);
        // rows past the plane's height, or a plane past a round trip's
        // destination, hold nothing
        const uint32_t rl = (y0 >= yc || z >= m.dims[2]) ? 0u : (yc - y0 < h ? yc - y0 : h);
        s.xl = (int32_t)xl;
        s.rl = (int32_t)rl;
        s.inside = xl == (a.band_g << lrc) && rl == h;
        return s;
    }

    // Boxes of the unit under cur that exist (the last unit of a row of the
    // sweep can reach past the row's last box).
    __device__ __forceinline__ uint32_t unit_boxes(const Cursor<3> &cur) const {
        const uint32_t left = a.tiles[0] - (cur.dig[0] << lg);
        return left < a.band_g ? left : a.band_g;
    }

    // The packed side: the unit's bands in the images of its boxes.  Records
    // end after the last existing box's band.
    __device__ __forceinline__ Side packed_side(const Cursor<3> &cur, uint32_t boxes) const {
        const KMap &sw = swept();
        const uint32_t lnb = a.band_lnb;
        const uint64_t t = ((uint64_t)cur.dig[2] * a.tiles[1] + (cur.dig[1] >> lnb)) * a.tiles[0] +
                           ((uint64_t)cur.dig[0] << lg);
        const uint32_t j = cur.dig[1] & ((1u << lnb) - 1u);
        Side s;
        s.base = (uint64_t)a.packed + t * sw.box_bytes + (uint64_t)j * a.band_bytes;
        s.nrec = (boxes - 1u) * sw.box_bytes + a.band_bytes;
        s.xl = s.rl = 0;
        s.inside = true;
        return s;
    }

    // Band j of a box is staged in band 0's arrangement: its image position
    // is the slot's position XOR x_j (bytes) -- see the band schedule notes
    // at tmap_launch_opts.
    __device__ __forceinline__ uint32_t band_xor(const Cursor<3> &cur) const {
        const KMap &sw = swept();
        const uint32_t jb = (cur.dig[1] & ((1u << a.band_lnb) - 1u)) << a.band_lbe;
        return (swizzle(jb, sw.swz_b, sw.swz_m, sw.swz_s) ^ jb) * sw.elem_size;
    }

    // arrive + expect the wave's 4 KiB (+16 under the budget-mismatch test
    // hook) on stage X, issue its four loads of the unit under the fill
    // cursor, move the cursor on
    template <int X>
    __device__ __forceinline__ void fill(uint8_t *ring) {
        uint8_t *stage = ring + X * kUnitBytes;
        if (a.flags & TMAP_FLAG_DEBUG_POISON) poison_blocks(stage + wave * kBlockBytes, kBandSlots, kWaves, lane);
        const uint32_t budget = kBandSlots * kBlockBytes + ((a.flags & TMAP_FLAG_INJECT_BUDGET_MISMATCH) ? 16u : 0u);
        bar_arrive_expect(&bars[X], budget, lane, kWaves);
        const uint32_t boxes = unit_boxes(fcur);
        uint32_t v[kBandSlots];
        Side s;
        if (MODE == kStore) {
            s = packed_side(fcur, boxes);
            const uint32_t x = band_xor(fcur);
#pragma unroll
            for (int jj = 0; jj < kBandSlots; ++jj) v[jj] = poff[jj] ^ x;
        } else {
            s = tensor_side(a.src, fcur, a.band_g);
            if (s.inside) {
#pragma unroll
                for (int jj = 0; jj < kBandSlots; ++jj) v[jj] = poff[jj];
            } else {
#pragma unroll
                for (int jj = 0; jj < kBandSlots; ++jj)
                    v[jj] = slot_inside(pxy[jj], s.xl, s.rl) ? poff[jj] : kOob;
            }
        }
        dma4<NTL>(s.base, s.nrec, (uint32_t)(uintptr_t)(lds_void_t *)(stage + wave * kBlockBytes), v);
        cursor_advance<3>(a, fcur);
    }

    template <typename Rs>
    __device__ __forceinline__ void store16(const i32x4 &v, Rs r, uint32_t off) const {
        if constexpr (NTS)
            __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 2);
        else
            __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
    }

    // Drain stage X (the unit under the consume cursor): always four stores
    // per lane, chunks with nothing to write going to the out-of-range
    // offset, so that the landing waits can count them.
    template <int X>
    __device__ __forceinline__ void consume(uint8_t *ring) {
        const uint8_t *stage = ring + X * kUnitBytes;
        i32x4 v[kBandSlots];
#pragma unroll
        for (int jj = 0; jj < kBandSlots; ++jj) {
            const uint32_t q = ((uint32_t)(jj * kWaves) + ((wave + 1u) & (kWaves - 1u))) * 64u + lane;
            v[jj] = *(const i32x4 *)(stage + q * 16u);
        }
        const uint32_t boxes = unit_boxes(ccur);
        if (MODE == kLoad) {
            const Side s = packed_side(ccur, boxes);
            const __amdgpu_buffer_rsrc_t r = make_rsrc(s.base, s.nrec);
            const uint32_t x = band_xor(ccur);
#pragma unroll
            for (int jj = 0; jj < kBandSlots; ++jj) store16(v[jj], r, coff[jj] ^ x);
        } else {
            const Side s = tensor_side(a.dst, ccur, boxes);
            const __amdgpu_buffer_rsrc_t r = make_rsrc(s.base, s.nrec);
            if constexpr (ADD) {
                typedef __attribute__((ext_vector_type(4))) float f32x4;
#pragma unroll
                for (int jj = 0; jj < kBandSlots; ++jj)
                    v[jj] = __builtin_bit_cast(i32x4, __builtin_bit_cast(f32x4, v[jj]) + a.addend);
            }
            if (s.inside) {
#pragma unroll
                for (int jj = 0; jj < kBandSlots; ++jj) store16(v[jj], r, coff[jj]);
            } else {
#pragma unroll
                for (int jj = 0; jj < kBandSlots; ++jj)
                    store16(v[jj], r, slot_inside(cxy[jj], s.xl, s.rl) ? coff[jj] : kOob);
            }
        }
        cursor_advance<3>(a, ccur);
    }

    // One step: unit k sits in stage X; the unit k+S-1 goes into the stage
    // unit k-1 left.  False ends the walk (done, or the wait timed out).
    template <int X>
    __device__ __forceinline__ bool step(uint8_t *ring, int64_t k) {
        if (k >= cnt) return false;
        // every wave has finished reading the stage about to be refilled
        __builtin_amdgcn_s_waitcnt(kWaitLgkm);
        __builtin_amdgcn_s_barrier();
        constexpr int XF = (X + S - 1) % S;
        const int64_t ahead = cnt - 1 - k;
        if (ahead >= S - 1) fill<XF>(ring);
        // operations this wave issued after unit k's loads: the fills of the
        // units after it (up to S-1) and the drains of the units before it
        // since its fill (up to S-1), four each; the counter retires them in
        // issue order, so those may stay in flight
        const uint32_t later = (uint32_t)(ahead < S - 1 ? ahead : S - 1);
        const uint32_t before = (uint32_t)(k < S - 1 ? k : S - 1);
        wait_vmcnt_upto<S>(4u * (later + before));
        __builtin_amdgcn_s_waitcnt(kWaitLgkm);
        asm volatile("" ::: "memory");
        bar_complete(&bars[X], kBandSlots * kBlockBytes, lane, kWaves);
        const bool ok = bar_wait(&bars[X], (parity >> X) & 1u, a.spin_limit);
        parity ^= 1u << X;
        asm volatile("" ::: "memory");
        if (!ok) {
            if (lane == 0) __hip_atomic_fetch_or(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
        consume<X>(ring);
        return true;
    }
};

template <int MODE, int S, bool NTL, bool NTS, bool ADD>
__global__ __launch_bounds__(kThreads) void band_kernel(const KArgs a) {
    __shared__ __attribute__((aligned(1024))) uint8_t ring[S * kUnitBytes];
    __shared__ uint64_t bars[S];

    BandCopier<MODE, S, NTL, NTS, ADD> cp(a, bars);
    if (threadIdx.x < (uint32_t)S) bars[threadIdx.x] = 0;
    cp.setup();
    __syncthreads();
    if (cp.cnt <= 0) return;

    // prologue: units 0..S-2 go to stages 0..S-2
    if constexpr (S > 1) cp.template fill<0>(ring);
    if constexpr (S > 2) if (1 < cp.cnt) cp.template fill<1>(ring);
    if constexpr (S > 3) if (2 < cp.cnt) cp.template fill<2>(ring);

    for (int64_t kb = 0; kb < cp.cnt; kb += S) {
        if (!cp.template step<0>(ring, kb)) break;
        if constexpr (S > 1) if (!cp.template step<1>(ring, kb + 1)) break;
        if constexpr (S > 2) if (!cp.template step<2>(ring, kb + 2)) break;
        if constexpr (S > 3) if (!cp.template step<3>(ring, kb + 3)) break;
    }
    // nothing may still be writing LDS or memory when the wave ends
    __builtin_amdgcn_s_waitcnt(0);
}

template <int MODE, int S, bool ADD>
KernelFn pick_band_hints(bool ntl, bool nts) {
    if (ntl) return nts ? band_kernel<MODE, S, true, true, ADD> : band_kernel<MODE, S, true, false, ADD>;
    return nts ? band_kernel<MODE, S, false, true, ADD> : band_kernel<MODE, S, false, false, ADD>;
}

template <int MODE, bool ADD>
KernelFn pick_band(int stages, bool ntl, bool nts) {
    switch (stages) {
        case 1: return pick_band_hints<MODE, 1, ADD>(ntl, nts);
        case 2: return pick_band_hints<MODE, 2, ADD>(ntl, nts);
        case 3: return pick_band_hints<MODE, 3, ADD>(ntl, nts);
        case 4: return pick_band_hints<MODE, 4, ADD>(ntl, nts);
        default: return nullptr;
    }
}

// Launch the band kernel of direction MODE with `stages` stages (1..4) over
// a.grid workgroups; the cache hints follow the flags as in the generic
// ring.  hipError_t as int.
template <int MODE>
int launch_band_mode(int stages, const KArgs &a, void *stream) {
    const bool ntl = nontemporal_loads<MODE>(a.flags), nts = nontemporal_stores<MODE>(a.flags);
    KernelFn fn = nullptr;
    if constexpr (MODE == kRoundtrip)
        fn = a.add_f32 ? pick_band<MODE, true>(stages, ntl, nts) : pick_band<MODE, false>(stages, ntl, nts);
    else
        fn = pick_band<MODE, false>(stages, ntl, nts);
    if (!fn) return (int)hipErrorInvalidValue;
    KArgs copy = a;
    void *args[] = {&copy};
    return (int)hipLaunchKernel((const void *)fn, dim3(a.grid), dim3(kThreads), args, 0, (hipStream_t)stream);
}

}  // namespace
}  // namespace tmap
