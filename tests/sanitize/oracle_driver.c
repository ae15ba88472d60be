/*
 * oracle_driver.c -- drives the CPU oracle (included whole, one translation
 * unit) over seeded random maps under AddressSanitizer and
 * UndefinedBehaviorSanitizer: the validator on arbitrary parameters, and on
 * every map it accepts the loads, stores, round trips, +addend round trips,
 * sweeps and in-bounds counts, with buffers sized exactly to the tensor
 * footprint and the packed images, so any read or write outside them trips
 * the sanitizer.  Also checks that a round trip equals a store of the loaded
 * images.  Exit status 0 when everything holds.
 */
#include <stdio.h>
#include <stdlib.h>

#include "../../oracle/oracle.c"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t rnd(void)
{
    /* xorshift64* */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return rng_state * 0x2545F4914F6CDD1Dull;
}
static int64_t range(int64_t lo, int64_t hi) { return lo + (int64_t)(rnd() % (uint64_t)(hi - lo + 1)); }

/* Bytes from element (0,..,0) to one past the last in-bounds element. */
static uint64_t footprint(const oracle_map *m)
{
    uint64_t f = m->dims[0] * (uint64_t)m->es;
    int d;
    for (d = 1; d < m->rank; ++d) f += (m->dims[d] - 1) * m->stride[d];
    return f;
}

static int garbage_validator_calls(int n)
{
    int i, d, accepted = 0;
    for (i = 0; i < n; ++i) {
        uint64_t dims[5], strides[4];
        uint32_t box[5], es_[5];
        int32_t rank = (int32_t)range(-1, 7);
        for (d = 0; d < 5; ++d) {
            dims[d] = rnd() >> (rnd() % 64);
            box[d] = (uint32_t)(rnd() >> (rnd() % 32 + 32));
            es_[d] = (uint32_t)range(0, 2);
        }
        for (d = 0; d < 4; ++d) strides[d] = rnd() >> (rnd() % 64);
        accepted += oracle_validate((int32_t)range(-1, 9), rank, rnd() >> (rnd() % 64), dims, strides, box,
                                    (rnd() & 1) ? es_ : NULL, (int32_t)range(-2, 10), (int32_t)range(-2, 18),
                                    (int32_t)range(-2, 18)) == OR_OK;
    }
    return accepted;
}

static int exercise_map(void)
{
    oracle_map m;
    uint64_t strides1[4];
    int32_t *coords;
    uint8_t *src, *dst, *dst2, *packed, *scratch;
    uint64_t fp, bb, row;
    int64_t n, t, ns;
    int d, rc;
    memset(&m, 0, sizeof m);
    m.es = 1 << range(0, 3);
    m.rank = (int32_t)range(1, 5);
    for (d = 0; d < m.rank; ++d) {
        m.dims[d] = (uint64_t)range(1, d == 0 ? 70 : 9);
        m.box[d] = (uint32_t)range(1, d == 0 ? 40 : 5);
    }
    m.box[0] = (uint32_t)((m.box[0] * m.es + 15) / 16 * 16 / m.es);  /* rows of whole 16-byte chunks */
    row = (m.dims[0] * (uint64_t)m.es + 15) / 16 * 16 + 16 * (uint64_t)range(0, 2);
    m.stride[0] = (uint64_t)m.es;
    for (d = 1; d < m.rank; ++d) {
        m.stride[d] = d == 1 ? row : m.stride[d - 1] * m.dims[d - 1] + 16 * (uint64_t)range(0, 1);
        strides1[d - 1] = m.stride[d];
    }
    m.swz_b = (int32_t)range(0, 3);
    m.swz_m = (int32_t)range(0, 4);
    m.swz_s = (int32_t)range(m.swz_b, 5);
    if (oracle_validate(m.es, m.rank, 0x1000, m.dims, strides1, m.box, NULL, m.swz_b, m.swz_m, m.swz_s) != OR_OK) {
        m.swz_b = m.swz_m = m.swz_s = 0;
        if (oracle_validate(m.es, m.rank, 0x1000, m.dims, strides1, m.box, NULL, 0, 0, 0) != OR_OK) return 0;
    }
    fp = footprint(&m);
    bb = oracle_box_bytes(&m);
    n = range(1, 24);
    coords = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n * m.rank));
    for (t = 0; t < n; ++t)
        for (d = 0; d < m.rank; ++d)
            coords[t * m.rank + d] = (int32_t)range(-(int64_t)m.box[d] - 2, (int64_t)m.dims[d] + 2);
    src = (uint8_t *)malloc(fp);
    dst = (uint8_t *)malloc(fp);
    dst2 = (uint8_t *)malloc(fp);
    packed = (uint8_t *)malloc((size_t)(bb * (uint64_t)n));
    scratch = (uint8_t *)malloc(bb);
    for (t = 0; t < (int64_t)fp; ++t) src[t] = (uint8_t)rnd();
    for (t = 0; t < (int64_t)fp; ++t) dst[t] = dst2[t] = (uint8_t)rnd();
    rc = oracle_load_tiles(&m, src, fp, coords, n, packed);
    rc |= oracle_store_tiles(&m, dst, fp, coords, n, packed);
    rc |= oracle_roundtrip(&m, src, fp, &m, dst2, fp, coords, n, scratch);
    if (rc) { fprintf(stderr, "oracle call failed\n"); return -1; }
    if (memcmp(dst, dst2, fp) != 0) { fprintf(stderr, "round trip != store(load)\n"); return -1; }
    if (m.es == 4) rc |= oracle_roundtrip_add_f32(&m, src, fp, &m, dst2, fp, coords, n, 1.0f, scratch);
    (void)oracle_inb_elems(&m, coords, n);
    ns = oracle_sweep_count(&m);
    if (ns <= 64) {
        int32_t c[OR_MAX_RANK];
        uint8_t *sp = (uint8_t *)malloc((size_t)(bb * (uint64_t)ns));
        for (t = 0; t < ns; ++t) oracle_sweep_coords(&m, t, c);
        rc |= oracle_load_tiles(&m, src, fp, NULL, ns, sp);
        rc |= oracle_store_tiles(&m, dst, fp, NULL, ns, sp);
        (void)oracle_inb_elems(&m, NULL, ns);
        free(sp);
    }
    oracle_bulk_copy(dst, src, fp);
    free(coords); free(src); free(dst); free(dst2); free(packed); free(scratch);
    return rc ? -1 : 1;
}

int main(void)
{
    int i, maps = 0;
    int accepted = garbage_validator_calls(100000);
    for (i = 0; i < 1500; ++i) {
        int r = exercise_map();
        if (r < 0) return 1;
        maps += r;
    }
    printf("oracle driver: %d garbage encodes accepted, %d maps exercised\n", accepted, maps);
    return maps > 500 ? 0 : 1;
}
