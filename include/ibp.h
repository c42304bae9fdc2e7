/*
 * ibp.h -- C ABI of libibp.so: Invariant Bit Packing (IBP) on AMD Instinct
 * MI355X (gfx950).  Batched gather + decompress of IBP-compressed fixed-size
 * tensors into dense device buffers, plus the two off-critical-path steps
 * that produce the compressed form (metadata build, compression) and the
 * compaction into a GPU-resident compressed cache.
 *
 * The method is the one described on web pages about the paper "Reducing the
 * GPU Memory Bottleneck with Lossless Compression for ML -- Extended"
 * (Kamath, Krishnamurthy, Canini, Peter).  Citations below name the page and
 * the part of it:
 *   [G-EN]  gist.science English explainer, "Technical Summary": Core
 *           Algorithm (Preprocessing, Compression, Decompression) and System
 *           Integration (cache compression, PCIe transfer compression);
 *   [JH]    juhe.plus Chinese review of the same paper (its paragraphs on the
 *           Mask/Bitval metadata, on warp-per-tensor decompression, on
 *           128 B-aligned GPU-initiated transfers and on sampling).
 *
 * ---------------------------------------------------------------- FORMAT
 * The pages fix no byte format; this library fixes the following one.
 *   tensor     B bytes (B % 4 == 0, 4 <= B <= IBP_MAX_TENSOR_BYTES); bit i is
 *              bit (i % 8) of byte (i / 8), i.e. bit (i % 32) of the
 *              little-endian 32-bit word i / 32.  W = B / 4 words.
 *   Mask       W words; bit i set = position i is invariant.
 *   Bitval     W words; the invariant value of each Mask position, 0 elsewhere.
 *   chunk      C bytes, C in {256, 1024, 4096} (the chunk sizes the pages
 *              evaluate, [JH] Figure 7 discussion); chunk c of a tensor is
 *              bytes [c*C, min((c+1)*C, B)); n_c = ceil(B / C) <= 64.
 *   P[t][c]    participation of chunk c of tensor t: 1 iff every Mask bit of
 *              the chunk equals its Bitval bit and the chunk holds at least one
 *              Mask bit (otherwise packing it would save nothing).
 *   bitmap     P[t][c] is bit (t*n_c + c) of a uint32 array, LSB first.  It
 *              lives in GPU memory, apart from the payloads ([G-EN] System
 *              Integration: a GPU-memory bitmask says which tensors are
 *              compressed; here one bit per chunk, so a tensor is compressed
 *              iff any of its bits is set).
 *   payload    chunk streams back to back, no padding: a participating chunk
 *              contributes its non-Mask bits in ascending position, another
 *              chunk all its bits; stream bit j is bit (j % 8) of byte j / 8;
 *              unused bits of the last byte are 0.  len_t = ceil(bits / 8)
 *              <= B bytes.
 *   slot store the payload of tensor t starts at store + t*slot_bytes
 *              (in-place fixed-size buffers, [G-EN] System Integration, PCIe
 *              transfer compression); slot bytes [len_t, slot_bytes) are
 *              don't-care (the compressor writes zeros up to the next 16 B).
 *   cache      compacted layout: payload of t at cache + offsets[t],
 *              offsets[0] = 0, offsets[t+1] = offsets[t] + roundup(len_t, A)
 *              with entry alignment A = 16 (ibp_compact_offsets) or a power
 *              of two up to 4096 (ibp_compact_offsets_aligned; A = 128 puts
 *              each entry on the fewest 128 B lines its length allows)
 *              ([G-EN] System Integration, cache compression).
 *   index      for a cache of one-chunk tensors: one uint64 per 32 tensors,
 *              index[w] = (participating tensors in bitmap words < w) << 32
 *              | bitmap word w.  Every entry then has one of two sizes, so
 *              its offset follows from the index word alone
 *              (ibp_gather_decompress_indexed).
 *
 * -------------------------------------------------------------- CONVENTIONS
 *   - Every function returns IBP_OK (0) or a negative ibp_status.  Arguments
 *     are validated synchronously before anything is enqueued; on failure
 *     nothing is enqueued and ibp_last_error() describes why (thread-local).
 *     Nothing throws across this interface.
 *   - GPU work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream) of the current HIP device; results are valid once the stream
 *     has been synchronized.  A HIP launch failure returns IBP_ERR_HIP.
 *   - The caller owns every buffer and keeps it alive until the stream has
 *     finished with it.  "device" buffers are GPU memory; "host-mapped" means
 *     pinned host memory from ibp_host_alloc (the GPU reads and writes it
 *     directly over PCIe).  The library keeps no allocation between calls.
 *   - Pointer alignment: rows and word arrays 4 B; store, cache and out 16 B.
 *   - Output is deterministic: the same inputs give the same bytes.
 */
#ifndef IBP_H
#define IBP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    IBP_OK = 0,
    IBP_ERR_NULL = -1,       /* a required pointer is NULL                     */
    IBP_ERR_SIZE = -2,       /* a size, count or stride is out of range         */
    IBP_ERR_CHUNK = -3,      /* chunk_bytes not in {256, 1024, 4096}            */
    IBP_ERR_THRESHOLD = -4,  /* threshold not in [0.5, 1] (or NaN)             */
    IBP_ERR_ALIGN = -5,      /* a pointer or stride breaks its alignment rule   */
    IBP_ERR_HIP = -6,        /* the HIP runtime reported an error               */
    IBP_ERR_FLAGS = -7       /* unknown flag bits                               */
} ibp_status;

#define IBP_VERSION 1
#define IBP_MAX_TENSOR_BYTES 16384u
#define IBP_MAX_CHUNKS 64u

/* Library version (IBP_VERSION). */
int ibp_version(void);

/* Message of the last failing call on this thread ("" if none). */
const char *ibp_last_error(void);

/* n_c = ceil(tensor_bytes / chunk_bytes), or a negative ibp_status if the
 * pair is not accepted by the other calls. */
int ibp_num_chunks(uint32_t tensor_bytes, uint32_t chunk_bytes);

/*
 * ibp_build_metadata -- [G-EN] Core Algorithm, Preprocessing; [JH] paragraph
 * on Mask/Bitval and paragraph on sampling 1/5/10 % of the data.
 * Over the n_samples sampled tensors, counts per bit position i the number n1
 * of tensors with bit i set (n0 = n_samples - n1), then writes
 *     Mask[i]   = max(n0, n1) >= m,   m = ceil(threshold * n_samples)
 *     Bitval[i] = Mask[i] && n1 > n0
 * m is computed on the host in IEEE binary64.
 *   rows         tensor r at rows + r*row_stride (device or host-mapped).
 *   sample_ids   device int64[n_samples] of tensor indices, or NULL for
 *                tensors 0..n_samples-1.  Precondition: each id < the number
 *                of tensors behind `rows` (not checked on the GPU).
 *   threshold    T in [0.5, 1].
 *   mask, bitval device uint32[tensor_bytes / 4] outputs.
 *   counts       device uint32[8 * tensor_bytes] workspace; on completion it
 *                holds n1 of every bit position i at counts[i].
 * Errors: NULL pointer, tensor_bytes out of range or not % 4, n_samples == 0
 * or > 2^32 - 1, row_stride < tensor_bytes or not % 4, bad threshold.
 */
int ibp_build_metadata(const void *rows, uint64_t row_stride,
                       const int64_t *sample_ids, uint64_t n_samples,
                       uint32_t tensor_bytes, double threshold,
                       uint32_t *mask, uint32_t *bitval, uint32_t *counts,
                       void *stream);

/*
 * ibp_build_metadata_noalloc -- ibp_build_metadata without the counts
 * workspace, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, meaning, Mask and Bitval as ibp_build_metadata.  The per-bit
 * counters live in a fixed array of 8 * IBP_NOALLOC_MAX_TENSOR_BYTES uint32
 * (512 KiB) inside the library, one per GPU, held until the process ends;
 * the call allocates nothing (no hipMalloc, no hipFree) and clears the
 * counters it uses with a kernel before counting.  Every call on one GPU
 * uses that GPU's array: calls that overlap on one GPU (on different streams,
 * or from different threads) race and give wrong Mask/Bitval.
 * Errors: as ibp_build_metadata; tensor_bytes > IBP_NOALLOC_MAX_TENSOR_BYTES
 * (IBP_ERR_SIZE); IBP_ERR_HIP if the array's device address cannot be found.
 */
#define IBP_NOALLOC_MAX_TENSOR_BYTES 16384u
int ibp_build_metadata_noalloc(const void *rows, uint64_t row_stride,
                               const int64_t *sample_ids, uint64_t n_samples,
                               uint32_t tensor_bytes, double threshold,
                               uint32_t *mask, uint32_t *bitval, void *stream);

/*
 * ibp_compress -- [G-EN] Core Algorithm, Compression; System Integration,
 * PCIe transfer compression (in-place fixed-size buffers, GPU bitmask); the
 * GPU writes the store directly, also when it is host-mapped.
 * Compresses rows 0..n_rows-1 as tensors t = first_tensor + i of a store of
 * n_tensors slots: writes the payload of t to its slot (bytes
 * [0, roundup(len_t, 16)) of the slot; zeros after len_t), sets/clears bits
 * t*n_c + c of part_bits, and writes len_t to lengths[t] if lengths != NULL.
 * Other tensors' slots, bits and lengths are untouched.
 *   rows        row i at rows + i*row_stride (device or host-mapped).
 *   mask,bitval device uint32[tensor_bytes / 4] (from ibp_build_metadata).
 *   store       device or host-mapped, n_tensors*slot_bytes bytes, 16 B aligned.
 *   slot_bytes  >= tensor_bytes, % 16 == 0 (128 recommended for host stores).
 *   part_bits   device uint32[ceil(n_tensors*n_c / 32)].
 *   lengths     device uint32[n_tensors] or NULL.
 * Calls that write the same tensors, or run concurrently on one store, race.
 * Errors: NULL pointer, sizes, first_tensor + n_rows > n_tensors, alignment.
 */
int ibp_compress(const void *rows, uint64_t row_stride, uint64_t n_rows,
                 uint64_t first_tensor, uint64_t n_tensors,
                 uint32_t tensor_bytes, uint32_t chunk_bytes,
                 const uint32_t *mask, const uint32_t *bitval,
                 void *store, uint64_t slot_bytes,
                 uint32_t *part_bits, uint32_t *lengths, void *stream);

/* Most segments one segmented call takes (ibp_compress_segments,
 * ibp_gather_decompress_segments). */
#define IBP_MAX_SEGMENTS 256u

/*
 * ibp_compress_segments -- several ibp_compress calls of one tensor shape in
 * one launch, each segment with its own Mask and Bitval (compress-on-write of
 * one decode token's new K/V rows for every (layer, K|V) pair, [JH] LLM
 * paragraph).  Segment k compresses rows seg_row[k] + i of `rows` (at
 * rows + (seg_row[k] + i) * row_stride) as tensors seg_first[k] + i,
 * i < seg_count[k], with the Mask words at masks + k*W and the Bitval words
 * at bitvals + k*W (W = tensor_bytes / 4).  Store, bitmap, lengths and slot
 * layout as in ibp_compress.  Same bytes as one ibp_compress call per segment.
 *   seg_row, seg_first, seg_count  HOST uint64[n_segments]; seg_count[k] <
 *               2^32 and seg_first[k] + seg_count[k] <= n_tensors.  Empty
 *               segments are allowed.  Segments that share a tensor race.
 *   n_segments  1 .. IBP_MAX_SEGMENTS.
 *   masks, bitvals  device uint32[n_segments * W] each.
 * Errors: as ibp_compress; n_segments out of range or a segment past
 * n_tensors (IBP_ERR_SIZE).
 */
int ibp_compress_segments(const void *rows, uint64_t row_stride,
                          const uint64_t *seg_row, const uint64_t *seg_first,
                          const uint64_t *seg_count, uint32_t n_segments,
                          uint64_t n_tensors, uint32_t tensor_bytes,
                          uint32_t chunk_bytes, const uint32_t *masks,
                          const uint32_t *bitvals, void *store, uint64_t slot_bytes,
                          uint32_t *part_bits, uint32_t *lengths, void *stream);

/*
 * ibp_compact_offsets -- [G-EN] System Integration, cache compression.
 * offsets[0] = 0, offsets[t+1] = offsets[t] + roundup(lengths[t], 16) for
 * t < n_tensors (so offsets[n_tensors] is the cache size in bytes).
 *   lengths  device uint32[n_tensors];  offsets  device uint64[n_tensors + 1].
 */
int ibp_compact_offsets(const uint32_t *lengths, uint64_t n_tensors,
                        uint64_t *offsets, void *stream);

/*
 * ibp_compact_offsets_aligned -- as ibp_compact_offsets with each entry
 * rounded up to entry_align bytes: offsets[t+1] = offsets[t] +
 * roundup(lengths[t], entry_align).  With entry_align = 128 every entry starts
 * on a 128 B line, so a payload of len bytes occupies ceil(len / 128) lines,
 * the fewest its length allows (the GPU reads HBM in whole 128 B lines; with
 * 16 B alignment a payload crosses one line more on average).  Fill the cache
 * with ibp_cache_fill (it copies each payload, rounded up to 16 B; the bytes
 * after it, up to the next entry, are left as they were).
 *   entry_align  a power of two in [16, 4096] (IBP_ERR_ALIGN otherwise).
 *   lengths  device uint32[n_tensors];  offsets  device uint64[n_tensors + 1].
 */
int ibp_compact_offsets_aligned(const uint32_t *lengths, uint64_t n_tensors,
                                uint32_t entry_align, uint64_t *offsets, void *stream);

/*
 * ibp_cache_index -- rank index of a participation bitmap, for one-chunk
 * tensors (chunk_bytes >= tensor_bytes, so bit t of part_bits is tensor t):
 *     index[w] = (number of set bits of part_bits[0 .. w-1]) << 32
 *                | part_bits[w]          for w < ceil(n_tensors / 32),
 * with bits t >= n_tensors of the last word cleared.  A tensor's entry in a
 * cache compacted with ibp_compact_offsets_aligned follows from it (see
 * ibp_gather_decompress_indexed), so a gather reads one 8-byte index word
 * per 32 tensors instead of one 8-byte offset per tensor.
 *   part_bits  device uint32[ceil(n_tensors / 32)];  index  device
 *   uint64[ceil(n_tensors / 32)].  n_tensors < 2^32 (IBP_ERR_SIZE).
 */
int ibp_cache_index(const uint32_t *part_bits, uint64_t n_tensors, uint64_t *index,
                    void *stream);

/*
 * ibp_compact -- copies entry t (offsets[t+1] - offsets[t] bytes from the
 * start of slot t) to cache + offsets[t] for every t < n_tensors.  Entries
 * that would end past cache_bytes are not copied.
 *   store  device or host-mapped slots (as written by ibp_compress).
 *   cache  device, cache_bytes bytes, 16 B aligned.
 */
int ibp_compact(const void *store, uint64_t slot_bytes, uint64_t n_tensors,
                const uint64_t *offsets, void *cache, uint64_t cache_bytes,
                void *stream);

/*
 * ibp_gather_decompress -- [G-EN] Core Algorithm, Decompression; [JH]
 * paragraphs on warp-per-tensor decompression with chunk offsets from a scan
 * inside the warp, and on 128 B-aligned GPU-initiated reads of host memory
 * overlapped with decoding.
 * out row r (tensor_bytes bytes at out + r*tensor_bytes) = the decompressed
 * tensor ids[r]: participating chunks take Bitval at Mask positions and the
 * next payload bits elsewhere; other chunks take payload bits everywhere.
 *   store        payloads: slots (offsets == NULL; store holds
 *                n_tensors*slot_bytes bytes, host-mapped or device) or a
 *                compacted cache (offsets != NULL; device uint64 offsets as
 *                from ibp_compact_offsets; an IBP_NOT_CACHED entry yields a
 *                row of zero bytes).
 *   store_bytes  readable bytes at store.  Reads never go past it (a corrupt
 *                bitmap or offset yields wrong rows, never an access fault).
 *   part_bits    device bitmap of the n_tensors tensors.
 *   ids          device int64[n_ids]; repeats allowed.  An id outside
 *                [0, n_tensors) yields a row of zero bytes.
 *   mask,bitval  device uint32[tensor_bytes / 4].
 *   out          device, n_ids*tensor_bytes bytes, 16 B aligned.
 * Errors: NULL pointer, sizes (store_bytes < n_tensors*slot_bytes in slot
 * mode), chunk size, alignment.
 */
int ibp_gather_decompress(const void *store, uint64_t store_bytes,
                          uint64_t slot_bytes, const uint64_t *offsets,
                          const uint32_t *part_bits, uint64_t n_tensors,
                          const int64_t *ids, uint64_t n_ids,
                          uint32_t tensor_bytes, uint32_t chunk_bytes,
                          const uint32_t *mask, const uint32_t *bitval,
                          void *out, void *stream);

/* ibp_gather_decompress with flags (0 = ibp_gather_decompress).
 *   IBP_GATHER_ROUTE_XCD  slot mode only (offsets == NULL), n_ids < 2^32.
 *     Each row is decoded on the XCD (the GPU's eight dies, each with its own
 *     L2 cache) chosen by a hash of its tensor index, so a tensor that the
 *     batch repeats is read over the host link (or from HBM) once per launch
 *     instead of once per XCD.  Same output.  For batches with repeated ids
 *     (Zipf embedding or feature lookups); batches without repeats are as
 *     fast or faster without it, because rows then spread less evenly.
 * Errors: as ibp_gather_decompress; unknown flags, routing with an offset
 * table (IBP_ERR_FLAGS); routing with n_ids >= 2^32 (IBP_ERR_SIZE). */
#define IBP_GATHER_ROUTE_XCD 1u
int ibp_gather_decompress_ex(const void *store, uint64_t store_bytes,
                             uint64_t slot_bytes, const uint64_t *offsets,
                             const uint32_t *part_bits, uint64_t n_tensors,
                             const int64_t *ids, uint64_t n_ids,
                             uint32_t tensor_bytes, uint32_t chunk_bytes,
                             const uint32_t *mask, const uint32_t *bitval,
                             void *out, unsigned flags, void *stream);

/*
 * ibp_gather_decompress_segments -- several gathers of one tensor shape in
 * one launch, each segment with its own Mask and Bitval ([JH] LLM paragraph:
 * one Mask per (layer, K|V) pair, from that pair's prompt K/V; a decode step
 * fetches every pair).  Segment k gathers ids[seg_ids[k] .. seg_ids[k+1])
 * into out rows seg_ids[k] .. seg_ids[k+1]-1, decoded with the Mask words at
 * masks + k*W and the Bitval words at bitvals + k*W (W = tensor_bytes / 4).
 * The segments share the store or cache, the bitmap and n_tensors, as in
 * ibp_gather_decompress (store, store_bytes, slot_bytes, offsets, part_bits,
 * n_tensors: same meaning).  Same rows as one ibp_gather_decompress call
 * per segment; the launch's fixed cost is paid once for all segments (also
 * for many embedding tables with one Mask each: [JH] DLRM paragraph).
 *   seg_ids     HOST uint64[n_segments + 1], seg_ids[0] = 0, non-decreasing;
 *               n_ids = seg_ids[n_segments].  Empty segments are allowed.
 *   n_segments  1 .. IBP_MAX_SEGMENTS.
 *   ids         device int64[n_ids];  out  device, n_ids*tensor_bytes bytes.
 *   masks, bitvals  device uint32[n_segments * W] each.
 *   flags       0 or IBP_GATHER_ROUTE_XCD (as ibp_gather_decompress_ex, each
 *               segment's rows routed by tensor index; slot mode only).
 * Errors: as ibp_gather_decompress; n_segments out of range, seg_ids[0] != 0
 * or decreasing (IBP_ERR_SIZE); as ibp_gather_decompress_ex for flags.
 */
int ibp_gather_decompress_segments(const void *store, uint64_t store_bytes,
                                   uint64_t slot_bytes, const uint64_t *offsets,
                                   const uint32_t *part_bits, uint64_t n_tensors,
                                   const int64_t *ids, const uint64_t *seg_ids,
                                   uint32_t n_segments, uint32_t tensor_bytes,
                                   uint32_t chunk_bytes, const uint32_t *masks,
                                   const uint32_t *bitvals, void *out, unsigned flags,
                                   void *stream);

/*
 * ibp_gather_decompress_indexed -- ibp_gather_decompress from a compacted
 * cache of one-chunk tensors, with entries found through the rank index
 * instead of an offset table ([G-EN] System Integration, cache compression;
 * Core Algorithm, Decompression).  The cache must hold every tensor, compacted
 * with ibp_compact_offsets_aligned(entry_align) from the lengths ibp_compress
 * wrote with this Mask: a one-chunk tensor's payload is ceil(K / 8) bytes
 * when it participates (K = bits not set in the Mask) and tensor_bytes
 * otherwise, so with s_p = roundup(ceil(K / 8), entry_align) and
 * s_r = roundup(tensor_bytes, entry_align) entry t starts at
 *     t * s_r - r1(t) * (s_r - s_p),   r1(t) = participating tensors before t.
 * Same rows as ibp_gather_decompress with the matching offset table.
 *   cache        device, cache_bytes bytes, 16 B aligned, below address 2^48.
 *                Reads never go past cache_bytes (an entry that would, and an
 *                id outside [0, n_tensors), yield a row of zero bytes).
 *   entry_align  the alignment the cache was compacted with.
 *   index        device, from ibp_cache_index; n_tensors < 2^32.
 *   tensor_bytes 256, 512 or 1024 (IBP_ERR_SIZE otherwise); chunk_bytes >=
 *                tensor_bytes (IBP_ERR_CHUNK otherwise).
 *   ids, mask, bitval, out  as ibp_gather_decompress.
 */
int ibp_gather_decompress_indexed(const void *cache, uint64_t cache_bytes,
                                  uint32_t entry_align, const uint64_t *index,
                                  uint64_t n_tensors, const int64_t *ids, uint64_t n_ids,
                                  uint32_t tensor_bytes, uint32_t chunk_bytes,
                                  const uint32_t *mask, const uint32_t *bitval, void *out,
                                  void *stream);

/* ------------------------------------------------------ cache + store together
 * [G-EN] System Integration uses both placements at once: a compressed
 * software cache in GPU memory for hot tensors, and compressed in-place
 * buffers in CPU memory for the rest ([JH] Figure 8 paragraph: cache plus
 * PCIe traffic compression gives the largest GNN speedups).  A partial cache
 * is described by an offset table with one entry per tensor; IBP_NOT_CACHED
 * marks a tensor that is only in the in-place store. */
#define IBP_NOT_CACHED UINT64_MAX

/*
 * ibp_cache_offsets -- cache_offsets[t] = running sum of roundup(lengths[u],
 * 16) over the selected u < t if select[t] != 0, else IBP_NOT_CACHED;
 * cache_offsets[n_tensors] = the cache size in bytes.
 *   lengths  device uint32[n_tensors];  select  device uint32[n_tensors];
 *   cache_offsets  device uint64[n_tensors + 1].
 */
int ibp_cache_offsets(const uint32_t *lengths, const uint32_t *select, uint64_t n_tensors,
                      uint64_t *cache_offsets, void *stream);

/*
 * ibp_cache_fill -- copies the payload of every cached tensor (roundup(len,
 * 16) bytes from the start of its slot) to cache + cache_offsets[t].  Entries
 * that would end past cache_bytes are not copied.
 *   store  in-place slots (device or host-mapped);  cache  device, 16 B aligned.
 */
int ibp_cache_fill(const void *store, uint64_t slot_bytes, const uint32_t *lengths,
                   uint64_t n_tensors, const uint64_t *cache_offsets, void *cache,
                   uint64_t cache_bytes, void *stream);

/*
 * ibp_gather_decompress_hybrid -- as ibp_gather_decompress, in one launch,
 * with each tensor read from the cache when cache_offsets[t] !=
 * IBP_NOT_CACHED (HBM) and from its slot of `store` otherwise (typically
 * host-mapped).  Every read stays inside [store, store + store_bytes) or
 * [cache, cache + cache_bytes).
 * Errors: as ibp_gather_decompress; store, cache and cache_offsets required.
 */
int ibp_gather_decompress_hybrid(const void *store, uint64_t store_bytes, uint64_t slot_bytes,
                                 const void *cache, uint64_t cache_bytes,
                                 const uint64_t *cache_offsets, const uint32_t *part_bits,
                                 uint64_t n_tensors, const int64_t *ids, uint64_t n_ids,
                                 uint32_t tensor_bytes, uint32_t chunk_bytes,
                                 const uint32_t *mask, const uint32_t *bitval, void *out,
                                 void *stream);

/* ------------------------------------------------------------ host memory
 * Pinned host memory that the GPU reads and writes directly (zero-copy),
 * [G-EN] Core Algorithm, Compression (zero-copy access to CPU memory).
 *   IBP_HOST_DEFAULT      mapped, portable; coherence per HIP's default
 *   IBP_HOST_COHERENT     + fine-grained (coherent) memory
 *   IBP_HOST_NONCOHERENT  + coarse-grained (non-coherent) memory
 * ibp_host_free releases memory from ibp_host_alloc (NULL is accepted). */
#define IBP_HOST_DEFAULT 0u
#define IBP_HOST_COHERENT 1u
#define IBP_HOST_NONCOHERENT 2u
int ibp_host_alloc(uint64_t bytes, unsigned flags, void **ptr);
int ibp_host_free(void *ptr);

/* ------------------------------------------------------------ measurement
 * Baselines the pages compare against ([JH] Table 1 and Figure 5
 * discussions): an uncompressed GPU-initiated gather of the same rows, a
 * streaming read that measures the link or HBM read rate, and a streaming
 * copy that measures the HBM read + write rate. */

/* out row r = row_bytes bytes at src + ids[r]*row_stride.  Ids outside
 * [0, n_rows) give zero rows.  src device or host-mapped; row_bytes,
 * row_stride, src and out multiples of 4.  When all four are multiples of 16
 * the rows move in 16 B units (aligned transfers), else in 4 B units (the
 * unaligned GPU copy the pages compare against).
 * flags: 0, or IBP_RAW_ROUTE_XCD: each row is copied by a wave on the XCD
 * chosen by a hash of its id, as ibp_gather_decompress_ex does with
 * IBP_GATHER_ROUTE_XCD (repeated ids then share one XCD's L2); same output;
 * requires n_ids < 2^32.  Errors: NULL pointers, sizes (including
 * n_rows*row_stride or n_ids*row_bytes past 2^64), alignment, unknown flags,
 * n_ids too large for routing. */
#define IBP_RAW_ROUTE_XCD 1u
int ibp_raw_gather(const void *src, uint64_t row_stride, uint64_t n_rows,
                   const int64_t *ids, uint64_t n_ids, uint32_t row_bytes,
                   void *out, unsigned flags, void *stream);

/* Reads bytes (a multiple of 16) at src with 16 B loads spread over the whole
 * GPU.  sink: device uint32[1]; written only if the XOR of all data equals
 * `never` (so the reads cannot be optimised away).  src 16 B aligned. */
int ibp_stream_read(const void *src, uint64_t bytes, uint32_t never,
                    uint32_t *sink, void *stream);

/* Copies bytes (a multiple of 16) from src to dst with 16 B loads and
 * streaming 16 B stores spread over the whole GPU: in HBM, the read + write
 * rate a gather's traffic is compared against.  src and dst device or
 * host-mapped, 16 B aligned, not overlapping.  Errors: NULL pointers, bytes
 * not a multiple of 16, alignment, overlap. */
int ibp_stream_copy(const void *src, void *dst, uint64_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* IBP_H */
