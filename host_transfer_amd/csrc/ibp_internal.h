// ibp_internal.h -- launch interface between the C ABI (api.hip) and the
// kernel files.  Host-side only; every launcher validates nothing (the C ABI
// has done it) and returns the HIP error of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ibp {

// Geometry shared by the compressor and the decompressor.
struct Geometry {
  uint32_t tensor_bytes, chunk_bytes;
  uint32_t W, n_c, wpc_log2, last_bits;
  uint32_t group;   // threads per tensor
  uint32_t J;       // words per thread
  uint32_t groups;  // groups per workgroup
};

Geometry make_geometry(uint32_t tensor_bytes, uint32_t chunk_bytes);

struct DeviceInfo {
  int device;
  int cus;
  size_t lds_per_block;
};
hipError_t device_info(DeviceInfo* info);

hipError_t launch_fill_u32(uint32_t* p, uint64_t n, uint32_t value, hipStream_t s);

hipError_t launch_build_metadata(const uint8_t* rows, uint64_t row_stride, const int64_t* ids,
                                 uint64_t n, uint32_t tensor_bytes, uint64_t cutoff,
                                 uint32_t* mask, uint32_t* bitval, uint32_t* counts,
                                 hipStream_t s);

hipError_t launch_compress(const Geometry& g, const uint8_t* rows, uint64_t row_stride,
                           uint64_t n_rows, uint64_t first, const uint32_t* mask,
                           const uint32_t* bitval, uint8_t* store, uint64_t slot_bytes,
                           uint32_t* part_bits, uint32_t* lengths, hipStream_t s);

hipError_t launch_compact_offsets(const uint32_t* lengths, uint64_t n, uint32_t align,
                                  uint64_t* offsets, hipStream_t s);

hipError_t launch_cache_index(const uint32_t* part_bits, uint64_t n_bits, uint64_t* index,
                              hipStream_t s);

// One-chunk tensors of 64, 128 or 256 words from a compacted HBM cache
// (gather_cache.hip): entries found through the offset table + bitmap, or
// through the rank index (entry alignment `entry_align`).
bool cache_kernel_fits(const Geometry& g);

hipError_t launch_gather_cache_table(const Geometry& g, const uint8_t* cache, uint64_t cache_bytes,
                                     const uint64_t* offsets, const uint32_t* part_bits,
                                     uint64_t n_tensors, const int64_t* ids, uint64_t n_ids,
                                     const uint32_t* mask, const uint32_t* bitval, uint32_t* out,
                                     hipStream_t s);

hipError_t launch_gather_cache_index(const Geometry& g, const uint8_t* cache, uint64_t cache_bytes,
                                     uint32_t entry_align, const uint64_t* index,
                                     uint64_t n_tensors, const int64_t* ids, uint64_t n_ids,
                                     const uint32_t* mask, const uint32_t* bitval, uint32_t* out,
                                     hipStream_t s);

hipError_t launch_compact(const uint8_t* store, uint64_t slot_bytes, uint64_t n,
                          const uint64_t* offsets, uint8_t* cache, uint64_t cache_bytes,
                          hipStream_t s);

// store: in-place slots (or null); offsets + cache: compacted cache entries
// (kNotCached marks a tensor that is read from its slot instead).
// Most segments one ibp_gather_decompress_segments call takes (IBP_MAX_SEGMENTS).
constexpr uint32_t kMaxSegments = 256;

hipError_t launch_compress_segments(const Geometry& g, const uint8_t* rows, uint64_t row_stride,
                                    const uint64_t* seg_row, const uint64_t* seg_first,
                                    const uint64_t* seg_count, uint32_t n_seg,
                                    const uint32_t* masks, const uint32_t* bitvals,
                                    uint8_t* store, uint64_t slot_bytes, uint32_t* part_bits,
                                    uint32_t* lengths, hipStream_t s);

hipError_t launch_gather_segments(const Geometry& g, const uint8_t* store, uint64_t store_bytes,
                                  uint64_t slot_bytes, const uint64_t* offsets,
                                  const uint8_t* cache, uint64_t cache_bytes,
                                  const uint32_t* part_bits, uint64_t n_tensors,
                                  const int64_t* ids, const uint64_t* seg_off, uint32_t n_seg,
                                  const uint32_t* masks, const uint32_t* bitvals, uint32_t* out,
                                  bool route, hipStream_t s);

hipError_t launch_gather(const Geometry& g, const uint8_t* store, uint64_t store_bytes,
                         uint64_t slot_bytes, const uint64_t* offsets, const uint8_t* cache,
                         uint64_t cache_bytes, const uint32_t* part_bits, uint64_t n_tensors,
                         const int64_t* ids, uint64_t n_ids, const uint32_t* mask,
                         const uint32_t* bitval, uint32_t* out, bool route, hipStream_t s);

hipError_t launch_cache_offsets(const uint32_t* lengths, const uint32_t* select, uint64_t n,
                                uint64_t* offsets, hipStream_t s);

hipError_t launch_cache_fill(const uint8_t* store, uint64_t slot_bytes, const uint32_t* lengths,
                             uint64_t n, const uint64_t* offsets, uint8_t* cache,
                             uint64_t cache_bytes, hipStream_t s);

hipError_t launch_raw_gather(const uint8_t* src, uint64_t row_stride, uint64_t n_rows,
                             const int64_t* ids, uint64_t n_ids, uint32_t row_bytes, uint8_t* out,
                             bool route, hipStream_t s);

hipError_t launch_stream_copy(const uint8_t* src, uint8_t* dst, uint64_t bytes, hipStream_t s);
hipError_t launch_stream_read(const uint8_t* src, uint64_t bytes, uint32_t never, uint32_t* sink,
                              hipStream_t s);

}  // namespace ibp
