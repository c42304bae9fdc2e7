/*
 * ibp_oracle.c -- plain, slow CPU oracle for Invariant Bit Packing (IBP).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or helper
 * with the HIP library under host_transfer_amd/csrc, and it does not know that
 * library exists.
 *
 * Every step is written as single-bit loops over the definition, with OpenMP
 * only over independent rows (or independent bit positions for the metadata
 * build).  No intrinsics, no word tricks, no blocking.
 *
 * Sources (the pages are web text about one paper, "Reducing the GPU Memory
 * Bottleneck with Lossless Compression for ML -- Extended"):
 *   [G-EN]  gist.science English explainer, "Technical Summary" part
 *   [JH]    juhe.plus Chinese review of the same paper
 *
 * Readings taken where the pages are silent (each one is listed in the design
 * notes of the repository):
 *   - bit i of a B-byte tensor is bit (i mod 8) of byte (i div 8): LSB-first,
 *     so on a little-endian host it is bit (i mod 32) of 32-bit word (i div 32);
 *     Mask and Bitval are B-byte strings addressed the same way;
 *   - "invariant across a high percentage T" means the majority value of the
 *     bit reaches the cutoff m = ceil(T * n) computed in IEEE binary64, with
 *     0.5 <= T <= 1; the invariant value is 1 only on a strict majority of ones;
 *   - chunk c of a tensor is bytes [c*C, min((c+1)*C, B)); one chunk when C >= B;
 *   - a chunk participates only if every Mask bit in it matches Bitval AND it
 *     holds at least one Mask bit (otherwise packing saves nothing);
 *   - the participation bits live in a separate bitmap, bit (t*n_c + c) in
 *     32-bit words LSB-first, not inside the payload;
 *   - the payload is the chunks' bit streams back to back with no padding:
 *     stream bit j is bit (j mod 8) of byte (j div 8); the last byte is
 *     zero-filled; the payload length is ceil(bits / 8) bytes.
 *
 * Return values: 0 on success, -1 on an argument the definitions exclude.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_API __attribute__((visibility("default")))

static unsigned get_bit(const uint8_t *p, uint64_t i)
{
    return (p[i / 8] >> (i % 8)) & 1u;
}

static void put_bit(uint8_t *p, uint64_t i, unsigned v)
{
    uint8_t m = (uint8_t)(1u << (i % 8));
    if (v)
        p[i / 8] = (uint8_t)(p[i / 8] | m);
    else
        p[i / 8] = (uint8_t)(p[i / 8] & (uint8_t)~m);
}

static unsigned get_map_bit(const uint32_t *map, uint64_t j)
{
    return (map[j / 32] >> (j % 32)) & 1u;
}

static void put_map_bit(uint32_t *map, uint64_t j, unsigned v)
{
    uint32_t m = 1u << (j % 32);
    if (v)
        map[j / 32] |= m;
    else
        map[j / 32] &= ~m;
}

ORC_API int orc_version(void) { return 1; }

/* Cutoff m of the threshold rule ([G-EN] Core Algorithm, Preprocessing): a
 * bit position is invariant when at least m of the n sampled tensors agree. */
ORC_API int64_t orc_cutoff(double threshold, uint64_t n)
{
    return (int64_t)ceil(threshold * (double)n);
}

/* Number of chunks of a B-byte tensor cut into C-byte chunks. */
ORC_API uint32_t orc_num_chunks(uint32_t tensor_bytes, uint32_t chunk_bytes)
{
    return (tensor_bytes + chunk_bytes - 1) / chunk_bytes;
}

/*
 * Metadata generation ([G-EN] Core Algorithm, Preprocessing; [JH] paragraph
 * on the Mask and Bitval metadata).  For every bit position i:
 *   n1 = number of sampled tensors with bit i set, n0 = n - n1,
 *   Mask[i]   = max(n0, n1) >= m,
 *   Bitval[i] = Mask[i] and n1 > n0.
 * rows: tensor r starts at rows + r*row_stride.  sample_ids: the n sampled
 * tensor indices, or NULL for tensors 0..n-1.  ones (optional): n1 per bit.
 */
ORC_API int orc_build_metadata(const uint8_t *rows, uint64_t row_stride,
                               const int64_t *sample_ids, uint64_t n_samples,
                               uint32_t tensor_bytes, double threshold,
                               uint8_t *mask, uint8_t *bitval, uint64_t *ones)
{
    if (!rows || !mask || !bitval || n_samples == 0 || tensor_bytes == 0)
        return -1;
    if (!(threshold >= 0.5 && threshold <= 1.0))
        return -1;
    const int64_t m = orc_cutoff(threshold, n_samples);

    /* one byte of the metadata per iteration, so no two threads share a byte */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t byte = 0; byte < (int64_t)tensor_bytes; byte++) {
        for (uint64_t b = 0; b < 8; b++) {
            const uint64_t i = (uint64_t)byte * 8 + b;
            uint64_t n1 = 0;
            for (uint64_t s = 0; s < n_samples; s++) {
                const uint64_t r = sample_ids ? (uint64_t)sample_ids[s] : s;
                n1 += get_bit(rows + r * row_stride, i);
            }
            const uint64_t n0 = n_samples - n1;
            const uint64_t top = n1 > n0 ? n1 : n0;
            const unsigned inv = (int64_t)top >= m;
            put_bit(mask, i, inv);
            put_bit(bitval, i, inv && n1 > n0);
            if (ones)
                ones[i] = n1;
        }
    }
    return 0;
}

/*
 * Compression ([G-EN] Core Algorithm, Compression; System Integration, PCIe
 * transfer compression).  Row i of `rows` is tensor t = first_tensor + i.
 * For every chunk c of t:
 *   K_c  = number of bits in c whose Mask bit is 0,
 *   P    = (every Mask bit of c equals its Bitval bit) and K_c < bits in c,
 *   emit = the bits whose Mask bit is 0, in ascending order, if P;
 *          every bit of c, in ascending order, otherwise.
 * The emitted streams of all chunks are concatenated and written to the slot
 * of t at store + t*slot_bytes (in-place fixed-size buffers); bytes
 * [0, tensor_bytes) of the slot are cleared first.  P goes to bit t*n_c + c
 * of part_bits; the payload length in bytes goes to lengths[i] if given.
 */
ORC_API int orc_compress(const uint8_t *rows, uint64_t row_stride,
                         uint64_t n_rows, uint64_t first_tensor,
                         uint32_t tensor_bytes, uint32_t chunk_bytes,
                         const uint8_t *mask, const uint8_t *bitval,
                         uint8_t *store, uint64_t slot_bytes,
                         uint32_t *part_bits, uint32_t *lengths)
{
    if (!rows || !mask || !bitval || !store || !part_bits)
        return -1;
    if (tensor_bytes == 0 || chunk_bytes == 0 || slot_bytes < tensor_bytes)
        return -1;
    const uint64_t n_c = orc_num_chunks(tensor_bytes, chunk_bytes);
    uint8_t *flags = calloc(n_rows * n_c + 1, 1);
    if (!flags)
        return -1;

#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n_rows; i++) {
        const uint8_t *x = rows + (uint64_t)i * row_stride;
        uint8_t *out = store + (first_tensor + (uint64_t)i) * slot_bytes;
        memset(out, 0, tensor_bytes);
        uint64_t cursor = 0;
        for (uint64_t c = 0; c < n_c; c++) {
            const uint64_t lo = c * chunk_bytes * 8;
            uint64_t hi = (c + 1) * chunk_bytes * 8;
            if (hi > (uint64_t)tensor_bytes * 8)
                hi = (uint64_t)tensor_bytes * 8;
            uint64_t k = 0;
            unsigned match = 1;
            for (uint64_t b = lo; b < hi; b++) {
                if (get_bit(mask, b)) {
                    if (get_bit(x, b) != get_bit(bitval, b))
                        match = 0;
                } else {
                    k++;
                }
            }
            const unsigned p = match && k < hi - lo;
            for (uint64_t b = lo; b < hi; b++) {
                if (!p || !get_bit(mask, b))
                    put_bit(out, cursor++, get_bit(x, b));
            }
            flags[(uint64_t)i * n_c + c] = (uint8_t)p;
        }
        if (lengths)
            lengths[i] = (uint32_t)((cursor + 7) / 8);
    }

    for (uint64_t i = 0; i < n_rows; i++)
        for (uint64_t c = 0; c < n_c; c++)
            put_map_bit(part_bits, (first_tensor + i) * n_c + c, flags[i * n_c + c]);
    free(flags);
    return 0;
}

/*
 * Compacted cache layout for compressed tensors kept in GPU memory ([G-EN]
 * System Integration, cache compression): entry t starts at offsets[t],
 * offsets[0] = 0 and offsets[t+1] = offsets[t] + lengths[t] rounded up to a
 * multiple of 16.  If `cache` is given, entry t receives the lengths[t]
 * payload bytes of slot t followed by zero bytes up to the next entry.
 */
ORC_API int orc_compact(const uint8_t *store, uint64_t slot_bytes,
                        const uint32_t *lengths, uint64_t n_tensors,
                        uint64_t *offsets, uint8_t *cache)
{
    if (!lengths || !offsets)
        return -1;
    offsets[0] = 0;
    for (uint64_t t = 0; t < n_tensors; t++)
        offsets[t + 1] = offsets[t] + (((uint64_t)lengths[t] + 15) / 16) * 16;
    if (cache) {
        if (!store)
            return -1;
        for (uint64_t t = 0; t < n_tensors; t++) {
            uint64_t e = offsets[t + 1] - offsets[t];
            memset(cache + offsets[t], 0, e);
            memcpy(cache + offsets[t], store + t * slot_bytes, lengths[t]);
        }
    }
    return 0;
}

/*
 * The same compacted layout with every entry rounded up to a multiple of
 * `align` bytes instead of 16: offsets[t+1] = offsets[t] + lengths[t] rounded
 * up to a multiple of align (align >= 1).  With align = 128 each entry starts
 * at a multiple of 128 bytes.  If `cache` is given, entry t receives the
 * lengths[t] payload bytes of slot t followed by zero bytes up to the next
 * entry.
 */
ORC_API int orc_compact_aligned(const uint8_t *store, uint64_t slot_bytes,
                                const uint32_t *lengths, uint64_t n_tensors,
                                uint32_t align, uint64_t *offsets, uint8_t *cache)
{
    if (!lengths || !offsets || align == 0)
        return -1;
    offsets[0] = 0;
    for (uint64_t t = 0; t < n_tensors; t++) {
        uint64_t size = 0;
        while (size < lengths[t])
            size += align;
        offsets[t + 1] = offsets[t] + size;
    }
    if (cache) {
        if (!store)
            return -1;
        for (uint64_t t = 0; t < n_tensors; t++) {
            uint64_t e = offsets[t + 1] - offsets[t];
            memset(cache + offsets[t], 0, e);
            memcpy(cache + offsets[t], store + t * slot_bytes, lengths[t]);
        }
    }
    return 0;
}

/*
 * Rank index of a participation bitmap of n_bits bits: for each 32-bit word
 * w, index[w] = (number of set bits among bitmap bits 0 .. 32w-1) * 2^32 +
 * (word w with every bit at or past n_bits cleared).  Counted one bit at a
 * time.
 */
ORC_API int orc_cache_index(const uint32_t *part_bits, uint64_t n_bits, uint64_t *index)
{
    if (!part_bits || !index)
        return -1;
    uint64_t before = 0;
    for (uint64_t w = 0; w * 32 < n_bits; w++) {
        uint64_t word = 0;
        for (unsigned b = 0; b < 32; b++) {
            const uint64_t j = w * 32 + b;
            if (j < n_bits && get_map_bit(part_bits, j))
                word |= (uint64_t)1 << b;
        }
        index[w] = (before << 32) | word;
        for (unsigned b = 0; b < 32; b++)
            before += (word >> b) & 1;
    }
    return 0;
}

/*
 * Gather + decompress ([G-EN] Core Algorithm, Decompression).  Output row r
 * is tensor t = ids[r]: walking the chunks in order with one cursor into the
 * payload of t, a participating chunk takes Bitval at its Mask positions and
 * the next payload bit everywhere else; a chunk that does not participate
 * takes the next payload bit at every position.  The payload of t is at
 * store + offsets[t] when offsets is given (compacted cache), else at
 * store + t*slot_bytes (in-place slots).  An id outside [0, n_tensors)
 * yields a row of zero bytes.
 */
ORC_API int orc_gather_decompress(const uint8_t *store, uint64_t slot_bytes,
                                  const uint64_t *offsets,
                                  const uint32_t *part_bits, uint64_t n_tensors,
                                  const int64_t *ids, uint64_t n_ids,
                                  uint32_t tensor_bytes, uint32_t chunk_bytes,
                                  const uint8_t *mask, const uint8_t *bitval,
                                  uint8_t *out)
{
    if (!store || !part_bits || !ids || !mask || !bitval || !out)
        return -1;
    if (tensor_bytes == 0 || chunk_bytes == 0)
        return -1;
    const uint64_t n_c = orc_num_chunks(tensor_bytes, chunk_bytes);

#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < (int64_t)n_ids; r++) {
        uint8_t *y = out + (uint64_t)r * tensor_bytes;
        memset(y, 0, tensor_bytes);
        const int64_t t = ids[r];
        if (t < 0 || (uint64_t)t >= n_tensors)
            continue;
        const uint8_t *src = offsets ? store + offsets[t] : store + (uint64_t)t * slot_bytes;
        uint64_t cursor = 0;
        for (uint64_t c = 0; c < n_c; c++) {
            const unsigned p = get_map_bit(part_bits, (uint64_t)t * n_c + c);
            const uint64_t lo = c * chunk_bytes * 8;
            uint64_t hi = (c + 1) * chunk_bytes * 8;
            if (hi > (uint64_t)tensor_bytes * 8)
                hi = (uint64_t)tensor_bytes * 8;
            for (uint64_t b = lo; b < hi; b++) {
                unsigned v;
                if (p && get_bit(mask, b))
                    v = get_bit(bitval, b);
                else
                    v = get_bit(src, cursor++);
                put_bit(y, b, v);
            }
        }
    }
    return 0;
}
