/*
 * Driver for the sanitizer run of the CPU oracle (TEST INFRASTRUCTURE): built
 * together with oracle/ibp_oracle.c under -fsanitize=address,undefined by
 * tests/test_sanitizers.py, it runs every oracle function on small seeded
 * inputs with exactly sized heap buffers (so any read or write past a buffer
 * is reported), checks the round trip, and exits 0.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int64_t orc_cutoff(double threshold, uint64_t n);
uint32_t orc_num_chunks(uint32_t tensor_bytes, uint32_t chunk_bytes);
int orc_build_metadata(const uint8_t *rows, uint64_t row_stride, const int64_t *sample_ids,
                       uint64_t n_samples, uint32_t tensor_bytes, double threshold,
                       uint8_t *mask, uint8_t *bitval, uint64_t *ones);
int orc_compress(const uint8_t *rows, uint64_t row_stride, uint64_t n_rows, uint64_t first_tensor,
                 uint32_t tensor_bytes, uint32_t chunk_bytes, const uint8_t *mask,
                 const uint8_t *bitval, uint8_t *store, uint64_t slot_bytes, uint32_t *part_bits,
                 uint32_t *lengths);
int orc_compact(const uint8_t *store, uint64_t slot_bytes, const uint32_t *lengths,
                uint64_t n_tensors, uint64_t *offsets, uint8_t *cache);
int orc_compact_aligned(const uint8_t *store, uint64_t slot_bytes, const uint32_t *lengths,
                        uint64_t n_tensors, uint32_t align, uint64_t *offsets, uint8_t *cache);
int orc_cache_index(const uint32_t *part_bits, uint64_t n_bits, uint64_t *index);
int orc_gather_decompress(const uint8_t *store, uint64_t slot_bytes, const uint64_t *offsets,
                          const uint32_t *part_bits, uint64_t n_tensors, const int64_t *ids,
                          uint64_t n_ids, uint32_t tensor_bytes, uint32_t chunk_bytes,
                          const uint8_t *mask, const uint8_t *bitval, uint8_t *out);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next32(void)
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (uint32_t)(rng >> 16);
}

static void *xmalloc(size_t n)
{
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

/* one case: n tensors of B bytes (B % 4 == 0), chunks of C bytes */
static int run_case(uint32_t B, uint32_t C, uint32_t n, double T)
{
    const uint32_t W = B / 4, nc = orc_num_chunks(B, C);
    const uint64_t S = (B + 127) / 128 * 128;
    uint8_t *rows = xmalloc((size_t)n * B);
    for (uint32_t t = 0; t < n; t++)
        for (uint32_t w = 0; w < W; w++) {
            uint32_t x = next32();
            if (next32() % 8)          /* mostly fixed high bits: some invariance */
                x = (x & 0x00FFFFFFu) | 0x3C000000u;
            memcpy(rows + (size_t)t * B + 4 * w, &x, 4);
        }
    uint8_t *mask = xmalloc(B), *bitval = xmalloc(B);
    uint64_t *ones = xmalloc((size_t)8 * B * sizeof(uint64_t));
    int64_t *sid = xmalloc((size_t)(n / 2 + 1) * sizeof(int64_t));
    for (uint32_t i = 0; i < n / 2 + 1; i++)
        sid[i] = (int64_t)(next32() % n);
    if (orc_build_metadata(rows, B, sid, n / 2 + 1, B, T, mask, bitval, ones))
        return 1;
    if (orc_build_metadata(rows, B, NULL, n, B, T, mask, bitval, ones))
        return 1;
    uint8_t *store = xmalloc((size_t)n * S);
    const uint64_t nbits = (uint64_t)n * nc;
    uint32_t *part = xmalloc((size_t)((nbits + 31) / 32) * 4);
    uint32_t *lens = xmalloc((size_t)n * 4);
    memset(part, 0, (size_t)((nbits + 31) / 32) * 4);
    if (orc_compress(rows, B, n, 0, B, C, mask, bitval, store, S, part, lens))
        return 1;
    uint64_t *off = xmalloc((size_t)(n + 1) * 8), *offa = xmalloc((size_t)(n + 1) * 8);
    if (orc_compact(NULL, S, lens, n, off, NULL) || orc_compact_aligned(NULL, S, lens, n, 128, offa, NULL))
        return 1;
    uint8_t *cache = xmalloc((size_t)off[n]), *cachea = xmalloc((size_t)offa[n]);
    if (orc_compact(store, S, lens, n, off, cache) ||
        orc_compact_aligned(store, S, lens, n, 128, offa, cachea))
        return 1;
    uint64_t *index = xmalloc((size_t)((nbits + 31) / 32) * 8);
    if (orc_cache_index(part, nbits, index))
        return 1;
    const uint32_t m = 3 * n + 5;
    int64_t *ids = xmalloc((size_t)m * 8);
    for (uint32_t i = 0; i < m; i++)
        ids[i] = (int64_t)(next32() % (n + 4)) - 2;   /* some invalid */
    uint8_t *out = xmalloc((size_t)m * B);
    const uint8_t *src[3] = {store, cache, cachea};
    const uint64_t *offs[3] = {NULL, off, offa};
    for (int k = 0; k < 3; k++) {
        if (orc_gather_decompress(src[k], S, offs[k], part, n, ids, m, B, C, mask, bitval, out))
            return 1;
        for (uint32_t i = 0; i < m; i++) {
            const int64_t t = ids[i];
            const int ok = t >= 0 && t < (int64_t)n;
            for (uint32_t b = 0; b < B; b++) {
                const uint8_t want = ok ? rows[(size_t)t * B + b] : 0;
                if (out[(size_t)i * B + b] != want) {
                    fprintf(stderr, "round trip differs: B=%u C=%u layout %d row %u\n", B, C, k, i);
                    return 1;
                }
            }
        }
    }
    free(rows); free(mask); free(bitval); free(ones); free(sid); free(store); free(part);
    free(lens); free(off); free(offa); free(cache); free(cachea); free(index); free(ids);
    free(out);
    return 0;
}

int main(void)
{
    static const uint32_t shapes[][3] = {
        {4, 256, 9}, {12, 4, 17}, {36, 16, 33}, {260, 256, 21}, {512, 1024, 40},
        {1028, 256, 13}, {5732, 1024, 7}, {16384, 256, 3},
    };
    for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; i++)
        for (int k = 0; k < 3; k++) {
            const double T = k == 0 ? 0.5 : (k == 1 ? 0.9 : 1.0);
            if (run_case(shapes[i][0], shapes[i][1], shapes[i][2], T)) {
                fprintf(stderr, "case %zu failed\n", i);
                return 1;
            }
        }
    if (orc_cutoff(0.99, 4096) != 4056)
        return 1;
    printf("oracle sanitizer run ok\n");
    return 0;
}
