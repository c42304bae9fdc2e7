// probe.hip -- measurement baselines ([JH] Table 1 and Figure 5 discussions):
//   k_raw_gather   uncompressed GPU-initiated gather of the same rows (what
//                  the compressed gather is compared against);
//   k_stream_read  streaming 16 B loads over a buffer (host-mapped: the rate
//                  of GPU-initiated reads over the host link; device: HBM);
//   k_stream_copy  a 16 B-per-lane copy (in HBM: the read + write rate a
//                  gather is compared against).
#include "ibp_internal.h"
#include "ibp_device.h"

namespace ibp {

// 2^lanes_log2 lanes per output row (up to a whole wave; several rows per
// wave when rows are short and the batch is large).  16 B units when rows, stride and buffers are all
// 16 B aligned ("aligned" transfers), else 4 B units (rows packed at any 4 B
// stride: the unaligned zero-copy baseline).
__global__ __launch_bounds__(256) void k_raw_gather(const uint8_t* __restrict__ src,
                                                     uint64_t row_stride, uint64_t n_rows,
                                                     const int64_t* __restrict__ ids,
                                                     uint64_t n_ids, uint32_t row_bytes,
                                                     uint8_t* __restrict__ out, bool wide,
                                                     uint32_t lanes_log2) {
  const uint32_t lane = lane_id();
  const uint32_t lanes = 1u << lanes_log2;
  const uint32_t sub = lane >> lanes_log2, q0 = lane & (lanes - 1);
  const uint32_t rows_per_wave = kWave >> lanes_log2;
  const uint64_t wave = (uint64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const uint64_t waves = (uint64_t)gridDim.x * (blockDim.x / kWave);
  for (uint64_t r = wave * rows_per_wave + sub; r < n_ids + sub; r += waves * rows_per_wave) {
    if (r >= n_ids) continue;
    const int64_t id = ids[r];
    const bool valid = id >= 0 && (uint64_t)id < n_rows;
    const uint8_t* s = src + (valid ? (uint64_t)id * row_stride : 0);
    uint8_t* d = out + r * row_bytes;
    // streaming stores, as the gather kernels write their rows
    if (wide) {
      typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
      for (uint32_t q = q0; q < row_bytes / 16; q += lanes) {
        const u32x4 v = valid ? ((const u32x4*)s)[q] : u32x4{0u, 0u, 0u, 0u};
        __builtin_nontemporal_store(v, (u32x4*)d + q);
      }
    } else {
      for (uint32_t q = q0; q < row_bytes / 4; q += lanes)
        __builtin_nontemporal_store(valid ? ((const uint32_t*)s)[q] : 0u, (uint32_t*)d + q);
    }
  }
}

// The same copy with every row routed to the XCD its id hashes to: the waves
// of XCD x split the batch into equal segments, and each wave copies the rows
// of its segment whose id hashes to x (the grid is a multiple of 8).
__global__ __launch_bounds__(256) void k_raw_gather_routed(const uint8_t* __restrict__ src,
                                                            uint64_t row_stride, uint64_t n_rows,
                                                            const int64_t* __restrict__ ids,
                                                            uint64_t n_ids, uint32_t row_bytes,
                                                            uint8_t* __restrict__ out, bool wide,
                                                            uint32_t lanes_log2) {
  __shared__ uint32_t s_rows[4][kWave];
  __shared__ int64_t s_ids[4][kWave];
  const uint32_t lane = lane_id();
  const uint32_t wave = uniform(threadIdx.x / kWave);
  const uint32_t wpb = blockDim.x / kWave;
  const uint32_t lanes = 1u << lanes_log2;
  const uint32_t sub = lane >> lanes_log2, q0 = lane & (lanes - 1);
  const uint32_t rows_per_wave = kWave >> lanes_log2;
  const uint32_t xcd = blockIdx.x % kXcds;
  const uint64_t wc = (uint64_t)(gridDim.x / kXcds) * wpb;
  const uint64_t wk = (uint64_t)(blockIdx.x / kXcds) * wpb + wave;
  const uint64_t seg = (n_ids + wc - 1) / wc;
  const uint64_t s0 = min(wk * seg, n_ids), s1 = min(s0 + seg, n_ids);
  for (uint64_t base = s0; base < s1; base += kWave) {
    const uint64_t r = base + lane;
    const bool in = r < s1;
    const int64_t rid = ids[in ? r : s1 - 1];
    const bool mine = in && xcd_of_tensor(rid) == xcd;
    const uint64_t bal = __ballot(mine);
    const uint32_t before = (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
    if (mine) {
      s_rows[wave][before] = (uint32_t)r;
      s_ids[wave][before] = rid;
    }
    const uint32_t n = (uint32_t)__popcll(bal);
    wave_sync();
    for (uint32_t k0 = 0; k0 < n; k0 += rows_per_wave) {
      const uint32_t k = k0 + sub;
      if (k >= n) continue;
      const uint64_t row = s_rows[wave][k];
      const int64_t id = s_ids[wave][k];
      const bool valid = id >= 0 && (uint64_t)id < n_rows;
      const uint8_t* sp = src + (valid ? (uint64_t)id * row_stride : 0);
      uint8_t* d = out + row * row_bytes;
      if (wide) {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        for (uint32_t q = q0; q < row_bytes / 16; q += lanes) {
          const u32x4 v = valid ? ((const u32x4*)sp)[q] : u32x4{0u, 0u, 0u, 0u};
          __builtin_nontemporal_store(v, (u32x4*)d + q);
        }
      } else {
        for (uint32_t q = q0; q < row_bytes / 4; q += lanes)
          __builtin_nontemporal_store(valid ? ((const uint32_t*)sp)[q] : 0u, (uint32_t*)d + q);
      }
    }
    wave_sync();
  }
}

__global__ __launch_bounds__(256) void k_stream_read(const uint4* __restrict__ src, uint64_t n16,
                                                      uint32_t never, uint32_t* __restrict__ sink) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  // one load per step: four strided loads per step read HBM 12 % slower (more
  // DRAM pages open at once) and the host link no faster
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == never) sink[0] = acc;
}

hipError_t launch_raw_gather(const uint8_t* src, uint64_t row_stride, uint64_t n_rows,
                             const int64_t* ids, uint64_t n_ids, uint32_t row_bytes, uint8_t* out,
                             bool route, hipStream_t s) {
  if (n_ids == 0) return hipSuccess;
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  const bool wide = ((row_bytes | row_stride | (uintptr_t)src | (uintptr_t)out) & 15u) == 0;
  const uint32_t units = row_bytes / (wide ? 16 : 4);
  uint32_t lanes_log2 = 0;
  while ((1u << lanes_log2) < units && (1u << lanes_log2) < (uint32_t)kWave) ++lanes_log2;
  if (route) {
    // about one window of ids per wave, eight XCD classes of blocks
    const uint64_t want = (n_ids + 4ull * kWave - 1) / (4ull * kWave) * kXcds;
    const uint64_t cap = (uint64_t)di.cus * 8;
    uint64_t blocks = want < cap ? want : cap;
    blocks = blocks < kXcds ? kXcds : blocks / kXcds * kXcds;
    hipLaunchKernelGGL(k_raw_gather_routed, dim3((uint32_t)blocks), dim3(256), 0, s, src,
                       row_stride, n_rows, ids, n_ids, row_bytes, out, wide, lanes_log2);
    return hipGetLastError();
  }
  // several rows per wave only while the batch still fills every CU with
  // waves (a wave per row keeps more requests in flight on small batches)
  while (lanes_log2 < 6 && n_ids / (kWave >> lanes_log2) < (uint64_t)di.cus * 32) ++lanes_log2;
  const uint64_t rows_per_block = 4ull * (kWave >> lanes_log2);
  const uint64_t want = (n_ids + rows_per_block - 1) / rows_per_block;
  const uint64_t cap = (uint64_t)di.cus * 8;
  hipLaunchKernelGGL(k_raw_gather, dim3((uint32_t)(want < cap ? want : cap)), dim3(256), 0, s,
                     src, row_stride, n_rows, ids, n_ids, row_bytes, out, wide, lanes_log2);
  return hipGetLastError();
}

// dst[i] = src[i], 16 B per lane with streaming stores: the copy rate that
// a gather's reads and writes are compared against.
__global__ __launch_bounds__(256) void k_stream_copy(const uint4* __restrict__ src,
                                                      uint4* __restrict__ dst, uint64_t n16) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const uint4 a = src[i];
    const u32x4 v = {a.x, a.y, a.z, a.w};
    __builtin_nontemporal_store(v, (u32x4*)dst + i);
  }
}

hipError_t launch_stream_read(const uint8_t* src, uint64_t bytes, uint32_t never, uint32_t* sink,
                              hipStream_t s) {
  const uint64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  const uint64_t want = (n16 + 255) / 256;
  const uint64_t cap = (uint64_t)di.cus * 8;
  hipLaunchKernelGGL(k_stream_read, dim3((uint32_t)(want < cap ? want : cap)), dim3(256), 0, s,
                     (const uint4*)src, n16, never, sink);
  return hipGetLastError();
}

hipError_t launch_stream_copy(const uint8_t* src, uint8_t* dst, uint64_t bytes, hipStream_t s) {
  const uint64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  // four workgroups per CU: in HBM a copy moved 5.6 TB/s (read + write) at
  // three or four, 4.6-4.8 at eight or sixteen (fewer rows written at once)
  const uint64_t want = (n16 + 255) / 256;
  const uint64_t cap = (uint64_t)di.cus * 4;
  hipLaunchKernelGGL(k_stream_copy, dim3((uint32_t)(want < cap ? want : cap)), dim3(256), 0, s,
                     (const uint4*)src, (uint4*)dst, n16);
  return hipGetLastError();
}

}  // namespace ibp
