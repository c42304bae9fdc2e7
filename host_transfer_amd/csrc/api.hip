// api.hip -- the extern "C" entry points of libibp.so (include/ibp.h).
// Validates every argument before any HIP call, then hands over to the
// launchers of the kernel files.  Errors are reported through the return code
// and a thread-local message; nothing throws across the ABI.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <mutex>

#include "ibp.h"
#include "ibp_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return IBP_OK;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(IBP_ERR_HIP, "%s: HIP error %d (%s)", where, (int)e, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Confirms a usable current device before anything is launched.
int require_device(const char* where) {
  ibp::DeviceInfo di;
  hipError_t e = ibp::device_info(&di);
  if (e != hipSuccess) return hip_fail(e, where);
  return IBP_OK;
}

int check_tensor(uint32_t tensor_bytes) {
  if (tensor_bytes == 0 || tensor_bytes % 4 != 0 || tensor_bytes > IBP_MAX_TENSOR_BYTES)
    return fail(IBP_ERR_SIZE, "tensor_bytes %u must be a multiple of 4 in [4, %u]", tensor_bytes,
                IBP_MAX_TENSOR_BYTES);
  return IBP_OK;
}

int check_chunk(uint32_t chunk_bytes) {
  if (chunk_bytes != 256 && chunk_bytes != 1024 && chunk_bytes != 4096)
    return fail(IBP_ERR_CHUNK, "chunk_bytes %u must be 256, 1024 or 4096", chunk_bytes);
  return IBP_OK;
}

// Entry alignment of a compacted cache: a power of two in [16, 4096].
bool valid_align(uint32_t a) { return a >= 16 && a <= 4096 && (a & (a - 1)) == 0; }

// Bitmap words for n tensors of n_c chunks, or 0 on overflow.
uint64_t bitmap_bits(uint64_t n_tensors, uint32_t n_c) {
  if (n_tensors > (UINT64_MAX - 31) / n_c) return 0;
  return n_tensors * n_c;
}

struct DevCache {
  std::once_flag once;
  ibp::DeviceInfo info;
  hipError_t err;
};
constexpr int kMaxDevices = 64;
DevCache g_dev[kMaxDevices];

}  // namespace

// Per-bit-position counters of ibp_build_metadata_noalloc: one uint32 per bit
// of the largest tensor that call accepts.  Every GPU holds its own copy.  In
// host code the name stands for a host-side placeholder, never a device
// address: host code uses only the address hipGetSymbolAddress returns for
// the current device (scratch_address below).
static __device__ __align__(256) uint32_t scratch[8u * IBP_NOALLOC_MAX_TENSOR_BYTES];

namespace {

struct ScratchAddr {
  std::once_flag once;
  uint32_t* ptr;
  hipError_t err;
};
ScratchAddr g_scratch[kMaxDevices];

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
hipError_t scratch_address(uint32_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  ScratchAddr& s = g_scratch[dev];
  std::call_once(s.once, [&] {
    void* p = nullptr;
    s.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    s.ptr = s.err == hipSuccess ? (uint32_t*)p : nullptr;
    if (s.err == hipSuccess && !s.ptr) s.err = hipErrorInvalidSymbol;
  });
  *out = s.ptr;
  return s.err;
}

}  // namespace

namespace ibp {

hipError_t device_info(DeviceInfo* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  DevCache& c = g_dev[dev];
  std::call_once(c.once, [&] {
    c.info.device = dev;
    c.err = hipDeviceGetAttribute(&c.info.cus, hipDeviceAttributeMultiprocessorCount, dev);
    int lds = 0;
    if (c.err == hipSuccess)
      c.err = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    c.info.lds_per_block = (size_t)lds;
  });
  *out = c.info;
  return c.err;
}

#ifndef IBP_MAX_WORDS_PER_THREAD
#define IBP_MAX_WORDS_PER_THREAD 6  // 1..6: registers per word bound J (see k_gather_decompress)
#endif

Geometry make_geometry(uint32_t tensor_bytes, uint32_t chunk_bytes) {
  Geometry g;
  g.tensor_bytes = tensor_bytes;
  g.chunk_bytes = chunk_bytes;
  g.W = tensor_bytes / 4;
  g.n_c = (tensor_bytes + chunk_bytes - 1) / chunk_bytes;
  g.wpc_log2 = 0;
  while ((1u << g.wpc_log2) < chunk_bytes / 4) ++g.wpc_log2;
  g.last_bits = 8u * (tensor_bytes - (g.n_c - 1) * chunk_bytes);
  // smallest group (threads per tensor) that keeps <= 6 words per thread, so
  // the per-word registers fit without spilling (and a payload of at most
  // B <= 24*G bytes fits in two 16 B registers per thread)
  g.group = 64;
  while (g.group * IBP_MAX_WORDS_PER_THREAD < g.W) g.group *= 2;
  g.J = (g.W + g.group - 1) / g.group;
  g.groups = g.group == 64 ? 4 : 1;
  return g;
}

}  // namespace ibp

namespace {

// Argument checks shared by the two metadata entry points (counts aside).
int check_metadata_args(const char* name, const void* rows, uint64_t row_stride,
                        const int64_t* sample_ids, uint64_t n_samples, uint32_t tensor_bytes,
                        double threshold, const uint32_t* mask, const uint32_t* bitval) {
  if (!rows || !mask || !bitval)
    return fail(IBP_ERR_NULL, "%s: rows, mask and bitval are required", name);
  int r = check_tensor(tensor_bytes);
  if (r) return r;
  if (n_samples == 0 || n_samples > 0xFFFFFFFFull)
    return fail(IBP_ERR_SIZE, "%s: n_samples %llu must be in [1, 2^32-1]", name,
                (unsigned long long)n_samples);
  if (row_stride < tensor_bytes || row_stride % 4 != 0)
    return fail(IBP_ERR_SIZE, "%s: row_stride %llu must be >= tensor_bytes and %% 4", name,
                (unsigned long long)row_stride);
  if (!(threshold >= 0.5 && threshold <= 1.0))
    return fail(IBP_ERR_THRESHOLD, "%s: threshold must be in [0.5, 1]", name);
  if (!aligned(rows, 4) || !aligned(mask, 4) || !aligned(bitval, 4) ||
      (sample_ids && !aligned(sample_ids, 8)))
    return fail(IBP_ERR_ALIGN, "%s: misaligned pointer", name);
  return IBP_OK;
}

// Checks the arguments, then counts into `counts` (device, 8 * tensor_bytes
// words, cleared by the launch) and thresholds.
int build_metadata_into(const char* name, const void* rows, uint64_t row_stride,
                        const int64_t* sample_ids, uint64_t n_samples, uint32_t tensor_bytes,
                        double threshold, uint32_t* mask, uint32_t* bitval, uint32_t* counts,
                        void* stream) {
  int r = check_metadata_args(name, rows, row_stride, sample_ids, n_samples, tensor_bytes,
                              threshold, mask, bitval);
  if (r) return r;
  // cutoff m = ceil(T * n) in binary64
  const uint64_t cutoff = (uint64_t)ceil(threshold * (double)n_samples);
  if ((r = require_device(name))) return r;
  hipError_t e = ibp::launch_build_metadata((const uint8_t*)rows, row_stride, sample_ids,
                                            n_samples, tensor_bytes, cutoff, mask, bitval, counts,
                                            (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, name);
  return ok();
}

}  // namespace

extern "C" {

int ibp_version(void) { return IBP_VERSION; }

const char* ibp_last_error(void) { return g_err; }

int ibp_num_chunks(uint32_t tensor_bytes, uint32_t chunk_bytes) {
  int r = check_tensor(tensor_bytes);
  if (r) return r;
  if ((r = check_chunk(chunk_bytes))) return r;
  ok();
  return (int)((tensor_bytes + chunk_bytes - 1) / chunk_bytes);
}

int ibp_build_metadata(const void* rows, uint64_t row_stride, const int64_t* sample_ids,
                       uint64_t n_samples, uint32_t tensor_bytes, double threshold,
                       uint32_t* mask, uint32_t* bitval, uint32_t* counts, void* stream) {
  const char* name = "ibp_build_metadata";
  if (!counts) return fail(IBP_ERR_NULL, "%s: counts is required", name);
  if (!aligned(counts, 4)) return fail(IBP_ERR_ALIGN, "%s: misaligned pointer", name);
  return build_metadata_into(name, rows, row_stride, sample_ids, n_samples, tensor_bytes,
                             threshold, mask, bitval, counts, stream);
}

int ibp_build_metadata_noalloc(const void* rows, uint64_t row_stride, const int64_t* sample_ids,
                               uint64_t n_samples, uint32_t tensor_bytes, double threshold,
                               uint32_t* mask, uint32_t* bitval, void* stream) {
  const char* name = "ibp_build_metadata_noalloc";
  static_assert(IBP_NOALLOC_MAX_TENSOR_BYTES <= IBP_MAX_TENSOR_BYTES, "scratch size");
  if (tensor_bytes > IBP_NOALLOC_MAX_TENSOR_BYTES)
    return fail(IBP_ERR_SIZE, "%s: tensor_bytes %u exceeds the %u the fixed counter array holds",
                name, tensor_bytes, IBP_NOALLOC_MAX_TENSOR_BYTES);
  int r = check_metadata_args(name, rows, row_stride, sample_ids, n_samples, tensor_bytes,
                              threshold, mask, bitval);
  if (r) return r;
  if ((r = require_device(name))) return r;
  uint32_t* counts = nullptr;
  hipError_t e = scratch_address(&counts);
  if (e != hipSuccess) return hip_fail(e, "ibp_build_metadata_noalloc: device address of the counters");
  return build_metadata_into(name, rows, row_stride, sample_ids, n_samples, tensor_bytes,
                             threshold, mask, bitval, counts, stream);
}

int ibp_compress(const void* rows, uint64_t row_stride, uint64_t n_rows, uint64_t first_tensor,
                 uint64_t n_tensors, uint32_t tensor_bytes, uint32_t chunk_bytes,
                 const uint32_t* mask, const uint32_t* bitval, void* store, uint64_t slot_bytes,
                 uint32_t* part_bits, uint32_t* lengths, void* stream) {
  if (!rows || !mask || !bitval || !store || !part_bits)
    return fail(IBP_ERR_NULL, "ibp_compress: rows, mask, bitval, store and part_bits are required");
  int r = check_tensor(tensor_bytes);
  if (r) return r;
  if ((r = check_chunk(chunk_bytes))) return r;
  if (first_tensor > n_tensors || n_rows > n_tensors - first_tensor)
    return fail(IBP_ERR_SIZE, "ibp_compress: first_tensor + n_rows exceeds n_tensors");
  if (row_stride < tensor_bytes || row_stride % 4 != 0)
    return fail(IBP_ERR_SIZE, "ibp_compress: row_stride must be >= tensor_bytes and %% 4");
  if (slot_bytes < tensor_bytes || slot_bytes % 16 != 0)
    return fail(IBP_ERR_SIZE, "ibp_compress: slot_bytes must be >= tensor_bytes and %% 16");
  const uint32_t n_c = (tensor_bytes + chunk_bytes - 1) / chunk_bytes;
  if (n_tensors && (!bitmap_bits(n_tensors, n_c) || n_tensors > UINT64_MAX / slot_bytes))
    return fail(IBP_ERR_SIZE, "ibp_compress: n_tensors too large");
  if (!aligned(rows, 4) || !aligned(mask, 4) || !aligned(bitval, 4) || !aligned(store, 16) ||
      !aligned(part_bits, 4) || (lengths && !aligned(lengths, 4)))
    return fail(IBP_ERR_ALIGN, "ibp_compress: misaligned pointer");
  if ((r = require_device("ibp_compress"))) return r;
  const ibp::Geometry g = ibp::make_geometry(tensor_bytes, chunk_bytes);
  hipError_t e = ibp::launch_compress(g, (const uint8_t*)rows, row_stride, n_rows, first_tensor,
                                      mask, bitval, (uint8_t*)store, slot_bytes, part_bits,
                                      lengths, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "ibp_compress");
  return ok();
}

int ibp_compress_segments(const void* rows, uint64_t row_stride, const uint64_t* seg_row,
                          const uint64_t* seg_first, const uint64_t* seg_count,
                          uint32_t n_segments, uint64_t n_tensors, uint32_t tensor_bytes,
                          uint32_t chunk_bytes, const uint32_t* masks, const uint32_t* bitvals,
                          void* store, uint64_t slot_bytes, uint32_t* part_bits,
                          uint32_t* lengths, void* stream) {
  const char* name = "ibp_compress_segments";
  if (n_segments == 0 || n_segments > IBP_MAX_SEGMENTS)
    return fail(IBP_ERR_SIZE, "%s: n_segments %u must be in [1, %u]", name, n_segments,
                IBP_MAX_SEGMENTS);
  if (!rows || !seg_row || !seg_first || !seg_count || !masks || !bitvals || !store || !part_bits)
    return fail(IBP_ERR_NULL, "%s: a required pointer is null", name);
  int r = check_tensor(tensor_bytes);
  if (r) return r;
  if ((r = check_chunk(chunk_bytes))) return r;
  if (row_stride < tensor_bytes || row_stride % 4 != 0)
    return fail(IBP_ERR_SIZE, "%s: row_stride must be >= tensor_bytes and %% 4", name);
  for (uint32_t k = 0; k < n_segments; ++k) {
    if (seg_count[k] > 0xFFFFFFFFull || seg_first[k] > n_tensors ||
        seg_count[k] > n_tensors - seg_first[k])
      return fail(IBP_ERR_SIZE, "%s: segment %u exceeds n_tensors", name, k);
    if (seg_row[k] > UINT64_MAX / row_stride - seg_count[k])
      return fail(IBP_ERR_SIZE, "%s: segment %u: rows past 2^64 bytes", name, k);
  }
  if (slot_bytes < tensor_bytes || slot_bytes % 16 != 0)
    return fail(IBP_ERR_SIZE, "%s: slot_bytes must be >= tensor_bytes and %% 16", name);
  const uint32_t n_c = (tensor_bytes + chunk_bytes - 1) / chunk_bytes;
  if (n_tensors && (!bitmap_bits(n_tensors, n_c) || n_tensors > UINT64_MAX / slot_bytes))
    return fail(IBP_ERR_SIZE, "%s: n_tensors too large", name);
  if (!aligned(rows, 4) || !aligned(masks, 4) || !aligned(bitvals, 4) || !aligned(store, 16) ||
      !aligned(part_bits, 4) || (lengths && !aligned(lengths, 4)))
    return fail(IBP_ERR_ALIGN, "%s: misaligned pointer", name);
  if ((r = require_device(name))) return r;
  const ibp::Geometry g = ibp::make_geometry(tensor_bytes, chunk_bytes);
  hipError_t e = ibp::launch_compress_segments(g, (const uint8_t*)rows, row_stride, seg_row,
                                               seg_first, seg_count, n_segments, masks, bitvals,
                                               (uint8_t*)store, slot_bytes, part_bits, lengths,
                                               (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, name);
  return ok();
}

int ibp_compact_offsets(const uint32_t* lengths, uint64_t n_tensors, uint64_t* offsets,
                        void* stream) {
  if (!lengths || !offsets)
    return fail(IBP_ERR_NULL, "ibp_compact_offsets: lengths and offsets are required");
  if (!aligned(lengths, 4) || !aligned(offsets, 8))
    return fail(IBP_ERR_ALIGN, "ibp_compact_offsets: misaligned pointer");
  int r;
  if ((r = require_device("ibp_compact_offsets"))) return r;
  hipError_t e = ibp::launch_compact_offsets(lengths, n_tensors, 16u, offsets, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "ibp_compact_offsets");
  return ok();
}

int ibp_compact_offsets_aligned(const uint32_t* lengths, uint64_t n_tensors, uint32_t entry_align,
                                uint64_t* offsets, void* stream) {
  const char* name = "ibp_compact_offsets_aligned";
  if (!lengths || !offsets) return fail(IBP_ERR_NULL, "%s: lengths and offsets are required", name);
  if (!valid_align(entry_align))
    return fail(IBP_ERR_ALIGN, "%s: entry_align %u must be a power of two in [16, 4096]", name,
                entry_align);
  if (!aligned(lengths, 4) || !aligned(offsets, 8))
    return fail(IBP_ERR_ALIGN, "%s: misaligned pointer", name);
  int r;
  if ((r = require_device(name))) return r;
  hipError_t e = ibp::launch_compact_offsets(lengths, n_tensors, entry_align, offsets,
                                             (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, name);
  return ok();
}

int ibp_cache_index(const uint32_t* part_bits, uint64_t n_tensors, uint64_t* index, void* stream) {
  const char* name = "ibp_cache_index";
  if (!part_bits || !index) return fail(IBP_ERR_NULL, "%s: part_bits and index are required", name);
  if (n_tensors >= (1ull << 32))
    return fail(IBP_ERR_SIZE, "%s: n_tensors must be below 2^32", name);
  if (!aligned(part_bits, 4) || !aligned(index, 8))
    return fail(IBP_ERR_ALIGN, "%s: misaligned pointer", name);
  int r;
  if ((r = require_device(name))) return r;
  hipError_t e = ibp::launch_cache_index(part_bits, n_tensors, index, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, name);
  return ok();
}

int ibp_gather_decompress_indexed(const void* cache, uint64_t cache_bytes, uint32_t entry_align,
                                  const uint64_t* index, uint64_t n_tensors, const int64_t* ids,
                                  uint64_t n_ids, uint32_t tensor_bytes, uint32_t chunk_bytes,
                                  const uint32_t* mask, const uint32_t* bitval, void* out,
                                  void* stream) {
  const char* name = "ibp_gather_decompress_indexed";
  if (!cache || !index || !ids || !mask || !bitval || !out)
    return fail(IBP_ERR_NULL, "%s: cache, index, ids, mask, bitval and out are required", name);
  int r = check_tensor(tensor_bytes);
  if (r) return r;
  if ((r = check_chunk(chunk_bytes))) return r;
  if (chunk_bytes < tensor_bytes)
    return fail(IBP_ERR_CHUNK, "%s: tensors must be one chunk (chunk_bytes >= tensor_bytes)", name);
  if (tensor_bytes != 256 && tensor_bytes != 512 && tensor_bytes != 1024)
    return fail(IBP_ERR_SIZE, "%s: tensor_bytes %u: 256, 512 or 1024 bytes", name, tensor_bytes);
  if (!valid_align(entry_align))
    return fail(IBP_ERR_ALIGN, "%s: entry_align %u must be a power of two in [16, 4096]", name,
                entry_align);
  if (n_tensors >= (1ull << 32))
    return fail(IBP_ERR_SIZE, "%s: n_tensors must be below 2^32", name);
  if (n_ids > UINT64_MAX / tensor_bytes) return fail(IBP_ERR_SIZE, "%s: n_ids too large", name);
  if ((uint64_t)(uintptr_t)cache >= (1ull << 48) || cache_bytes > (1ull << 48) - (uintptr_t)cache)
    return fail(IBP_ERR_SIZE, "%s: the cache must lie below 2^48 (a device address)", name);
  if (!aligned(cache, 16) || !aligned(out, 16) || !aligned(ids, 8) || !aligned(index, 8) ||
      !aligned(mask, 4) || !aligned(bitval, 4))
    return fail(IBP_ERR_ALIGN, "%s: misaligned pointer", name);
  if ((r = require_device(name))) return r;
  const ibp::Geometry g = ibp::make_geometry(tensor_bytes, chunk_bytes);
  hipError_t e = ibp::launch_gather_cache_index(g, (const uint8_t*)cache, cache_bytes, entry_align,
                                                index, n_tensors, ids, n_ids, mask, bitval,
                                                (uint32_t*)out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, name);
  return ok();
}

int ibp_compact(const void* store, uint64_t slot_bytes, uint64_t n_tensors,
                const uint64_t* offsets, void* cache, uint64_t cache_bytes, void* stream) {
  if (!store || !offsets || !cache)
    return fail(IBP_ERR_NULL, "ibp_compact: store, offsets and cache are required");
  if (slot_bytes == 0 || slot_bytes % 16 != 0)
    return fail(IBP_ERR_SIZE, "ibp_compact: slot_bytes must be a positive multiple of 16");
  if (n_tensors > UINT64_MAX / slot_bytes)
    return fail(IBP_ERR_SIZE, "ibp_compact: n_tensors too large");
  if (!aligned(store, 16) || !aligned(cache, 16) || !aligned(offsets, 8))
    return fail(IBP_ERR_ALIGN, "ibp_compact: misaligned pointer");
  int r;
  if ((r = require_device("ibp_compact"))) return r;
  hipError_t e = ibp::launch_compact((const uint8_t*)store, slot_bytes, n_tensors, offsets,
                                     (uint8_t*)cache, cache_bytes, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "ibp_compact");
  return ok();
}

int ibp_gather_decompress(const void* store, uint64_t store_bytes, uint64_t slot_bytes,
                          const uint64_t* offsets, const uint32_t* part_bits, uint64_t n_tensors,
                          const int64_t* ids, uint64_t n_ids, uint32_t tensor_bytes,
                          uint32_t chunk_bytes, const uint32_t* mask, const uint32_t* bitval,
                          void* out, void* stream) {
  return ibp_gather_decompress_ex(store, store_bytes, slot_bytes, offsets, part_bits, n_tensors,
                                  ids, n_ids, tensor_bytes, chunk_bytes, mask, bitval, out, 0u,
                                  stream);
}

int ibp_gather_decompress_ex(const void* store, uint64_t store_bytes, uint64_t slot_bytes,
                             const uint64_t* offsets, const uint32_t* part_bits,
                             uint64_t n_tensors, const int64_t* ids, uint64_t n_ids,
                             uint32_t tensor_bytes, uint32_t chunk_bytes, const uint32_t* mask,
                             const uint32_t* bitval, void* out, unsigned flags, void* stream) {
  if (flags & ~IBP_GATHER_ROUTE_XCD)
    return fail(IBP_ERR_FLAGS, "ibp_gather_decompress: unknown flags");
  const bool route = (flags & IBP_GATHER_ROUTE_XCD) != 0;
  if (route && offsets)
    return fail(IBP_ERR_FLAGS, "ibp_gather_decompress: routing applies to slot mode (no offsets)");
  if (route && n_ids >= (1ull << 32))
    return fail(IBP_ERR_SIZE, "ibp_gather_decompress: routing needs n_ids < 2^32");
  if (!store || !part_bits || !ids || !mask || !bitval || !out)
    return fail(IBP_ERR_NULL,
                "ibp_gather_decompress: store, part_bits, ids, mask, bitval and out are required");
  int r = check_tensor(tensor_bytes);
  if (r) return r;
  if ((r = check_chunk(chunk_bytes))) return r;
  const uint32_t n_c = (tensor_bytes + chunk_bytes - 1) / chunk_bytes;
  if (n_tensors && !bitmap_bits(n_tensors, n_c))
    return fail(IBP_ERR_SIZE, "ibp_gather_decompress: n_tensors too large");
  if (!offsets) {
    if (slot_bytes < tensor_bytes || slot_bytes % 16 != 0)
      return fail(IBP_ERR_SIZE,
                  "ibp_gather_decompress: slot_bytes must be >= tensor_bytes and %% 16");
    if (n_tensors > UINT64_MAX / slot_bytes || store_bytes < n_tensors * slot_bytes)
      return fail(IBP_ERR_SIZE, "ibp_gather_decompress: store_bytes < n_tensors * slot_bytes");
  }
  if (n_ids > UINT64_MAX / tensor_bytes)
    return fail(IBP_ERR_SIZE, "ibp_gather_decompress: n_ids too large");
  if (!aligned(store, 16) || !aligned(out, 16) || !aligned(ids, 8) || !aligned(mask, 4) ||
      !aligned(bitval, 4) || !aligned(part_bits, 4) || (offsets && !aligned(offsets, 8)))
    return fail(IBP_ERR_ALIGN, "ibp_gather_decompress: misaligned pointer");
  if ((r = require_device("ibp_gather_decompress"))) return r;
  const ibp::Geometry g = ibp::make_geometry(tensor_bytes, chunk_bytes);
  // slot mode: store holds the slots; cache mode: store is the compacted cache
  hipError_t e = offsets
      ? ibp::launch_gather(g, nullptr, 0, 0, offsets, (const uint8_t*)store, store_bytes,
                           part_bits, n_tensors, ids, n_ids, mask, bitval, (uint32_t*)out, false,
                           (hipStream_t)stream)
      : ibp::launch_gather(g, (const uint8_t*)store, store_bytes, slot_bytes, nullptr, nullptr, 0,
                           part_bits, n_tensors, ids, n_ids, mask, bitval, (uint32_t*)out, route,
                           (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "ibp_gather_decompress");
  return ok();
}

int ibp_gather_decompress_segments(const void* store, uint64_t store_bytes, uint64_t slot_bytes,
                                   const uint64_t* offsets, const uint32_t* part_bits,
                                   uint64_t n_tensors, const int64_t* ids,
                                   const uint64_t* seg_ids, uint32_t n_segments,
                                   uint32_t tensor_bytes, uint32_t chunk_bytes,
                                   const uint32_t* masks, const uint32_t* bitvals, void* out,
                                   unsigned flags, void* stream) {
  static_assert(ibp::kMaxSegments == IBP_MAX_SEGMENTS, "segment limit");
  const char* name = "ibp_gather_decompress_segments";
  if (flags & ~IBP_GATHER_ROUTE_XCD) return fail(IBP_ERR_FLAGS, "%s: unknown flags", name);
  const bool route = (flags & IBP_GATHER_ROUTE_XCD) != 0;
  if (route && offsets)
    return fail(IBP_ERR_FLAGS, "%s: routing applies to slot mode (no offsets)", name);
  if (!store || !part_bits || !ids || !seg_ids || !masks || !bitvals || !out)
    return fail(IBP_ERR_NULL, "%s: a required pointer is null", name);
  if (n_segments == 0 || n_segments > IBP_MAX_SEGMENTS)
    return fail(IBP_ERR_SIZE, "%s: n_segments %u must be in [1, %u]", name, n_segments,
                IBP_MAX_SEGMENTS);
  if (seg_ids[0] != 0) return fail(IBP_ERR_SIZE, "%s: seg_ids[0] must be 0", name);
  for (uint32_t k = 0; k < n_segments; ++k)
    if (seg_ids[k + 1] < seg_ids[k])
      return fail(IBP_ERR_SIZE, "%s: seg_ids must not decrease (segment %u)", name, k);
  const uint64_t n_ids = seg_ids[n_segments];
  int r = check_tensor(tensor_bytes);
  if (r) return r;
  if ((r = check_chunk(chunk_bytes))) return r;
  const uint32_t n_c = (tensor_bytes + chunk_bytes - 1) / chunk_bytes;
  if (n_tensors && !bitmap_bits(n_tensors, n_c))
    return fail(IBP_ERR_SIZE, "%s: n_tensors too large", name);
  if (!offsets) {
    if (slot_bytes < tensor_bytes || slot_bytes % 16 != 0)
      return fail(IBP_ERR_SIZE, "%s: slot_bytes must be >= tensor_bytes and %% 16", name);
    if (n_tensors > UINT64_MAX / slot_bytes || store_bytes < n_tensors * slot_bytes)
      return fail(IBP_ERR_SIZE, "%s: store_bytes < n_tensors * slot_bytes", name);
  }
  if (n_ids > UINT64_MAX / tensor_bytes) return fail(IBP_ERR_SIZE, "%s: n_ids too large", name);
  if (route && n_ids >= (1ull << 32))
    return fail(IBP_ERR_SIZE, "%s: routing needs n_ids < 2^32", name);
  if (!aligned(store, 16) || !aligned(out, 16) || !aligned(ids, 8) || !aligned(masks, 4) ||
      !aligned(bitvals, 4) || !aligned(part_bits, 4) || (offsets && !aligned(offsets, 8)))
    return fail(IBP_ERR_ALIGN, "%s: misaligned pointer", name);
  if ((r = require_device(name))) return r;
  const ibp::Geometry g = ibp::make_geometry(tensor_bytes, chunk_bytes);
  hipError_t e = offsets
      ? ibp::launch_gather_segments(g, nullptr, 0, 0, offsets, (const uint8_t*)store, store_bytes,
                                    part_bits, n_tensors, ids, seg_ids, n_segments, masks,
                                    bitvals, (uint32_t*)out, false, (hipStream_t)stream)
      : ibp::launch_gather_segments(g, (const uint8_t*)store, store_bytes, slot_bytes, nullptr,
                                    nullptr, 0, part_bits, n_tensors, ids, seg_ids, n_segments,
                                    masks, bitvals, (uint32_t*)out, route, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, name);
  return ok();
}

int ibp_cache_offsets(const uint32_t* lengths, const uint32_t* select, uint64_t n_tensors,
                      uint64_t* cache_offsets, void* stream) {
  if (!lengths || !select || !cache_offsets)
    return fail(IBP_ERR_NULL, "ibp_cache_offsets: lengths, select and cache_offsets are required");
  if (!aligned(lengths, 4) || !aligned(select, 4) || !aligned(cache_offsets, 8))
    return fail(IBP_ERR_ALIGN, "ibp_cache_offsets: misaligned pointer");
  int r;
  if ((r = require_device("ibp_cache_offsets"))) return r;
  hipError_t e = ibp::launch_cache_offsets(lengths, select, n_tensors, cache_offsets,
                                           (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "ibp_cache_offsets");
  return ok();
}

int ibp_cache_fill(const void* store, uint64_t slot_bytes, const uint32_t* lengths,
                   uint64_t n_tensors, const uint64_t* cache_offsets, void* cache,
                   uint64_t cache_bytes, void* stream) {
  if (!store || !lengths || !cache_offsets || !cache)
    return fail(IBP_ERR_NULL, "ibp_cache_fill: store, lengths, cache_offsets and cache are required");
  if (slot_bytes == 0 || slot_bytes % 16 != 0 || n_tensors > UINT64_MAX / slot_bytes)
    return fail(IBP_ERR_SIZE, "ibp_cache_fill: slot_bytes must be a positive multiple of 16");
  if (!aligned(store, 16) || !aligned(cache, 16) || !aligned(lengths, 4) ||
      !aligned(cache_offsets, 8))
    return fail(IBP_ERR_ALIGN, "ibp_cache_fill: misaligned pointer");
  int r;
  if ((r = require_device("ibp_cache_fill"))) return r;
  hipError_t e = ibp::launch_cache_fill((const uint8_t*)store, slot_bytes, lengths, n_tensors,
                                        cache_offsets, (uint8_t*)cache, cache_bytes,
                                        (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "ibp_cache_fill");
  return ok();
}

int ibp_gather_decompress_hybrid(const void* store, uint64_t store_bytes, uint64_t slot_bytes,
                                 const void* cache, uint64_t cache_bytes,
                                 const uint64_t* cache_offsets, const uint32_t* part_bits,
                                 uint64_t n_tensors, const int64_t* ids, uint64_t n_ids,
                                 uint32_t tensor_bytes, uint32_t chunk_bytes,
                                 const uint32_t* mask, const uint32_t* bitval, void* out,
                                 void* stream) {
  if (!store || !cache || !cache_offsets || !part_bits || !ids || !mask || !bitval || !out)
    return fail(IBP_ERR_NULL, "ibp_gather_decompress_hybrid: a required pointer is null");
  int r = check_tensor(tensor_bytes);
  if (r) return r;
  if ((r = check_chunk(chunk_bytes))) return r;
  const uint32_t n_c = (tensor_bytes + chunk_bytes - 1) / chunk_bytes;
  if (n_tensors && !bitmap_bits(n_tensors, n_c))
    return fail(IBP_ERR_SIZE, "ibp_gather_decompress_hybrid: n_tensors too large");
  if (slot_bytes < tensor_bytes || slot_bytes % 16 != 0)
    return fail(IBP_ERR_SIZE,
                "ibp_gather_decompress_hybrid: slot_bytes must be >= tensor_bytes and %% 16");
  if (n_tensors > UINT64_MAX / slot_bytes || store_bytes < n_tensors * slot_bytes)
    return fail(IBP_ERR_SIZE, "ibp_gather_decompress_hybrid: store_bytes < n_tensors * slot_bytes");
  if (n_ids > UINT64_MAX / tensor_bytes)
    return fail(IBP_ERR_SIZE, "ibp_gather_decompress_hybrid: n_ids too large");
  if (!aligned(store, 16) || !aligned(cache, 16) || !aligned(out, 16) || !aligned(ids, 8) ||
      !aligned(mask, 4) || !aligned(bitval, 4) || !aligned(part_bits, 4) ||
      !aligned(cache_offsets, 8))
    return fail(IBP_ERR_ALIGN, "ibp_gather_decompress_hybrid: misaligned pointer");
  if ((r = require_device("ibp_gather_decompress_hybrid"))) return r;
  const ibp::Geometry g = ibp::make_geometry(tensor_bytes, chunk_bytes);
  hipError_t e = ibp::launch_gather(g, (const uint8_t*)store, store_bytes, slot_bytes,
                                    cache_offsets, (const uint8_t*)cache, cache_bytes, part_bits,
                                    n_tensors, ids, n_ids, mask, bitval, (uint32_t*)out, false,
                                    (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "ibp_gather_decompress_hybrid");
  return ok();
}

int ibp_host_alloc(uint64_t bytes, unsigned flags, void** ptr) {
  if (!ptr) return fail(IBP_ERR_NULL, "ibp_host_alloc: ptr is required");
  *ptr = nullptr;
  if (bytes == 0) return fail(IBP_ERR_SIZE, "ibp_host_alloc: bytes must be > 0");
  if (flags > IBP_HOST_NONCOHERENT) return fail(IBP_ERR_FLAGS, "ibp_host_alloc: unknown flags");
  unsigned hf = hipHostMallocMapped | hipHostMallocPortable;
  if (flags == IBP_HOST_COHERENT) hf |= hipHostMallocCoherent;
  if (flags == IBP_HOST_NONCOHERENT) hf |= hipHostMallocNonCoherent;
  hipError_t e = hipHostMalloc(ptr, (size_t)bytes, hf);
  if (e != hipSuccess) {
    *ptr = nullptr;
    return hip_fail(e, "ibp_host_alloc");
  }
  return ok();
}

int ibp_host_free(void* ptr) {
  if (!ptr) return ok();
  hipError_t e = hipHostFree(ptr);
  if (e != hipSuccess) return hip_fail(e, "ibp_host_free");
  return ok();
}

int ibp_raw_gather(const void* src, uint64_t row_stride, uint64_t n_rows, const int64_t* ids,
                   uint64_t n_ids, uint32_t row_bytes, void* out, unsigned flags, void* stream) {
  if (!src || !ids || !out) return fail(IBP_ERR_NULL, "ibp_raw_gather: src, ids and out are required");
  if (row_bytes == 0 || row_bytes % 4 != 0 || row_stride < row_bytes || row_stride % 4 != 0)
    return fail(IBP_ERR_SIZE, "ibp_raw_gather: row_bytes %% 4, row_stride >= row_bytes and %% 4");
  if (n_rows > UINT64_MAX / row_stride || n_ids > UINT64_MAX / row_bytes)
    return fail(IBP_ERR_SIZE, "ibp_raw_gather: n_rows * row_stride or n_ids * row_bytes overflows");
  if (!aligned(src, 4) || !aligned(out, 4) || !aligned(ids, 8))
    return fail(IBP_ERR_ALIGN, "ibp_raw_gather: misaligned pointer");
  if (flags & ~IBP_RAW_ROUTE_XCD) return fail(IBP_ERR_FLAGS, "ibp_raw_gather: unknown flags");
  const bool route = (flags & IBP_RAW_ROUTE_XCD) != 0;
  if (route && n_ids >= (1ull << 32))
    return fail(IBP_ERR_SIZE, "ibp_raw_gather: routing needs n_ids < 2^32");
  int r;
  if ((r = require_device("ibp_raw_gather"))) return r;
  hipError_t e = ibp::launch_raw_gather((const uint8_t*)src, row_stride, n_rows, ids, n_ids,
                                        row_bytes, (uint8_t*)out, route, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "ibp_raw_gather");
  return ok();
}

int ibp_stream_read(const void* src, uint64_t bytes, uint32_t never, uint32_t* sink,
                    void* stream) {
  if (!src || !sink) return fail(IBP_ERR_NULL, "ibp_stream_read: src and sink are required");
  if (bytes % 16 != 0) return fail(IBP_ERR_SIZE, "ibp_stream_read: bytes must be %% 16");
  if (!aligned(src, 16) || !aligned(sink, 4))
    return fail(IBP_ERR_ALIGN, "ibp_stream_read: misaligned pointer");
  int r;
  if ((r = require_device("ibp_stream_read"))) return r;
  hipError_t e = ibp::launch_stream_read((const uint8_t*)src, bytes, never, sink,
                                         (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "ibp_stream_read");
  return ok();
}

int ibp_stream_copy(const void* src, void* dst, uint64_t bytes, void* stream) {
  if (!src || !dst) return fail(IBP_ERR_NULL, "ibp_stream_copy: src and dst are required");
  if (bytes % 16 != 0) return fail(IBP_ERR_SIZE, "ibp_stream_copy: bytes must be %% 16");
  if (!aligned(src, 16) || !aligned(dst, 16))
    return fail(IBP_ERR_ALIGN, "ibp_stream_copy: misaligned pointer");
  const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
  if (bytes && s0 < d0 + bytes && d0 < s0 + bytes)
    return fail(IBP_ERR_SIZE, "ibp_stream_copy: src and dst overlap");
  int r;
  if ((r = require_device("ibp_stream_copy"))) return r;
  hipError_t e = ibp::launch_stream_copy((const uint8_t*)src, (uint8_t*)dst, bytes,
                                         (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "ibp_stream_copy");
  return ok();
}

}  // extern "C"
