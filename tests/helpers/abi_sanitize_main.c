/*
 * Driver for the sanitizer run of the C ABI's host code (TEST
 * INFRASTRUCTURE): linked with api.hip built with host-side ASan/UBSan by
 * tests/test_sanitizers.py.  Calls every entry point with arguments each
 * check must reject (expecting the documented status and a message), then
 * valid calls that enqueue nothing, which must report IBP_ERR_HIP when no GPU
 * is visible.  Never dereferences the fake addresses it passes.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ibp.h"

static int fails = 0;

static void expect(int got, int want, const char *what)
{
    const char *msg = ibp_last_error();
    if (got != want || (want < 0 && (!msg || !msg[0]))) {
        fprintf(stderr, "%s: status %d, expected %d (%s)\n", what, got, want, msg ? msg : "");
        fails++;
    }
}

int main(int argc, char **argv)
{
    const int no_device = argc > 1 && strcmp(argv[1], "no-device") == 0;
    void *P = (void *)(uintptr_t)(1u << 20);  /* aligned, never dereferenced */
    uint32_t *Pu = (uint32_t *)P;
    uint64_t *Pq = (uint64_t *)P;
    const int64_t *Pi = (const int64_t *)P;
    void *odd = (void *)((uintptr_t)P + 2);
    uint64_t seg[4] = {0, 2, 2, 5};
    uint64_t row[2] = {0, 1}, cnt[2] = {1, 1};

    expect(ibp_num_chunks(5732, 1024), 6, "num_chunks");
    expect(ibp_num_chunks(6, 256), IBP_ERR_SIZE, "num_chunks size");
    expect(ibp_build_metadata(NULL, 512, NULL, 10, 512, 0.99, Pu, Pu, Pu, NULL), IBP_ERR_NULL, "meta null");
    expect(ibp_build_metadata(P, 512, NULL, 10, 512, 1.5, Pu, Pu, Pu, NULL), IBP_ERR_THRESHOLD, "meta T");
    expect(ibp_build_metadata(odd, 512, NULL, 10, 512, 0.99, Pu, Pu, Pu, NULL), IBP_ERR_ALIGN, "meta align");
    expect(ibp_build_metadata_noalloc(P, 1u << 20, NULL, 10, 16388, 0.99, Pu, Pu, NULL), IBP_ERR_SIZE, "noalloc size");
    expect(ibp_build_metadata_noalloc(P, 512, NULL, 0, 512, 0.99, Pu, Pu, NULL), IBP_ERR_SIZE, "noalloc n");
    expect(ibp_compress(P, 512, 10, 5, 10, 512, 256, Pu, Pu, P, 512, Pu, Pu, NULL), IBP_ERR_SIZE, "compress range");
    expect(ibp_compress(P, 512, 10, 0, 10, 512, 100, Pu, Pu, P, 512, Pu, Pu, NULL), IBP_ERR_CHUNK, "compress chunk");
    expect(ibp_compress_segments(P, 512, row, row, cnt, 0, 10, 512, 256, Pu, Pu, P, 512, Pu, Pu, NULL), IBP_ERR_SIZE, "compress seg n");
    expect(ibp_compress_segments(P, 512, row, row, cnt, 2, 1, 512, 256, Pu, Pu, P, 512, Pu, Pu, NULL), IBP_ERR_SIZE, "compress seg range");
    expect(ibp_compact_offsets(NULL, 10, Pq, NULL), IBP_ERR_NULL, "offsets null");
    expect(ibp_compact_offsets_aligned(Pu, 10, 96, Pq, NULL), IBP_ERR_ALIGN, "aligned 96");
    expect(ibp_cache_index(Pu, 1ull << 32, Pq, NULL), IBP_ERR_SIZE, "index n");
    expect(ibp_compact(P, 500, 10, Pq, P, 100, NULL), IBP_ERR_SIZE, "compact slot");
    expect(ibp_gather_decompress(P, 5119, 512, NULL, Pu, 10, Pi, 4, 512, 256, Pu, Pu, P, NULL), IBP_ERR_SIZE, "gather store");
    expect(ibp_gather_decompress_ex(P, 5120, 512, Pq, Pu, 10, Pi, 4, 512, 256, Pu, Pu, P, 1u, NULL), IBP_ERR_FLAGS, "gather route cache");
    expect(ibp_gather_decompress_segments(P, 5120, 512, NULL, Pu, 10, Pi, seg, 0, 512, 256, Pu, Pu, P, 0, NULL), IBP_ERR_SIZE, "seg n");
    seg[2] = 1;
    expect(ibp_gather_decompress_segments(P, 5120, 512, NULL, Pu, 10, Pi, seg, 3, 512, 256, Pu, Pu, P, 0, NULL), IBP_ERR_SIZE, "seg decreasing");
    expect(ibp_gather_decompress_indexed(P, 4096, 128, Pq, 10, Pi, 4, 768, 1024, Pu, Pu, P, NULL), IBP_ERR_SIZE, "indexed size");
    expect(ibp_gather_decompress_indexed(P, 4096, 128, Pq, 10, Pi, 4, 512, 256, Pu, Pu, P, NULL), IBP_ERR_CHUNK, "indexed chunks");
    expect(ibp_cache_offsets(Pu, NULL, 10, Pq, NULL), IBP_ERR_NULL, "cache offsets");
    expect(ibp_cache_fill(P, 500, Pu, 10, Pq, P, 100, NULL), IBP_ERR_SIZE, "cache fill");
    expect(ibp_gather_decompress_hybrid(P, 5120, 512, NULL, 100, Pq, Pu, 10, Pi, 4, 512, 256, Pu, Pu, P, NULL), IBP_ERR_NULL, "hybrid");
    expect(ibp_raw_gather(odd, 512, 10, Pi, 4, 512, P, 0, NULL), IBP_ERR_ALIGN, "raw align");
    expect(ibp_stream_read(P, 100, 0, Pu, NULL), IBP_ERR_SIZE, "stream size");
    void *hp = P;
    expect(ibp_host_alloc(0, 0, &hp), IBP_ERR_SIZE, "host alloc 0");
    expect(ibp_host_alloc(64, 9, &hp), IBP_ERR_FLAGS, "host alloc flags");
    expect(ibp_host_free(NULL), IBP_OK, "host free null");
    if (no_device) {
        /* valid calls that would enqueue nothing: the HIP runtime reports no device */
        expect(ibp_gather_decompress(P, 5120, 512, NULL, Pu, 10, Pi, 0, 512, 256, Pu, Pu, P, NULL), IBP_ERR_HIP, "gather no device");
        expect(ibp_raw_gather(P, 512, 10, Pi, 0, 512, P, 0, NULL), IBP_ERR_HIP, "raw no device");
        expect(ibp_stream_read(P, 0, 0, Pu, NULL), IBP_ERR_HIP, "stream no device");
        expect(ibp_build_metadata_noalloc(P, 512, NULL, 10, 512, 0.99, Pu, Pu, NULL), IBP_ERR_HIP, "noalloc no device");
    }
    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    printf("abi sanitizer run ok\n");
    return 0;
}
