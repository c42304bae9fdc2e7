// meta.hip -- Mask/Bitval metadata build (off the critical path).
//
// [G-EN] Core Algorithm, Preprocessing: over a set of tensors (a sample is
// enough, [JH] sampling paragraph), find the bit positions whose value agrees
// across at least a fraction T of them, and record them (Mask) with their
// value (Bitval).  Two kernels:
//   k_meta_count      per bit position, the number of sampled tensors with
//                     that bit set.  Lane l of a wave owns word w (coalesced
//                     loads across lanes), keeps 32 counters in registers over
//                     a slab of sampled rows, then adds them to the global
//                     counters with atomics.
//   k_meta_threshold  one thread per word applies the cutoff m (computed on
//                     the host in binary64) to its 32 counters.
#include "ibp_internal.h"
#include "ibp_device.h"

namespace ibp {

__global__ __launch_bounds__(256) void k_fill_u32(uint32_t* __restrict__ p, uint64_t n,
                                                   uint32_t value) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    p[i] = value;
}

hipError_t launch_fill_u32(uint32_t* p, uint64_t n, uint32_t value, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const uint64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(k_fill_u32, dim3((uint32_t)(blocks < 4096 ? blocks : 4096)), dim3(256), 0,
                     s, p, n, value);
  return hipGetLastError();
}

// grid: word_groups * slabs blocks of 64 threads; block b handles words
// [64*(b % word_groups), +64) of sampled rows [per_slab*(b / word_groups), +per_slab).
__global__ __launch_bounds__(64) void k_meta_count(const uint8_t* __restrict__ rows,
                                                    uint64_t row_stride,
                                                    const int64_t* __restrict__ ids, uint64_t n,
                                                    uint32_t W, uint32_t word_groups,
                                                    uint64_t per_slab,
                                                    uint32_t* __restrict__ counts) {
  const uint32_t wg = blockIdx.x % word_groups;
  const uint64_t slab = blockIdx.x / word_groups;
  const uint32_t w = wg * kWave + threadIdx.x;
  const uint64_t s0 = slab * per_slab;
  const uint64_t s1 = min(n, s0 + per_slab);
  if (w >= W) return;
  uint32_t cnt[32];
#pragma unroll
  for (int b = 0; b < 32; ++b) cnt[b] = 0;
  for (uint64_t s = s0; s < s1; ++s) {
    const uint64_t r = ids ? (uint64_t)ids[s] : s;
    const uint32_t x = *(const uint32_t*)(rows + r * row_stride + 4ull * w);
#pragma unroll
    for (int b = 0; b < 32; ++b) cnt[b] += (x >> b) & 1u;
  }
#pragma unroll
  for (int b = 0; b < 32; ++b)
    if (cnt[b]) atomicAdd(counts + 32ull * w + b, cnt[b]);
}

__global__ __launch_bounds__(256) void k_meta_threshold(const uint32_t* __restrict__ counts,
                                                         uint32_t W, uint64_t n, uint64_t cutoff,
                                                         uint32_t* __restrict__ mask,
                                                         uint32_t* __restrict__ bitval) {
  const uint32_t w = blockIdx.x * blockDim.x + threadIdx.x;
  if (w >= W) return;
  uint32_t m = 0, v = 0;
  for (int b = 0; b < 32; ++b) {
    const uint64_t n1 = counts[32ull * w + b];
    const uint64_t n0 = n - n1;
    const bool inv = (n1 > n0 ? n1 : n0) >= cutoff;
    m |= (uint32_t)inv << b;
    v |= (uint32_t)(inv && n1 > n0) << b;
  }
  mask[w] = m;
  bitval[w] = v;
}

hipError_t launch_build_metadata(const uint8_t* rows, uint64_t row_stride, const int64_t* ids,
                                 uint64_t n, uint32_t tensor_bytes, uint64_t cutoff,
                                 uint32_t* mask, uint32_t* bitval, uint32_t* counts,
                                 hipStream_t s) {
  const uint32_t W = tensor_bytes / 4;
  hipError_t e = launch_fill_u32(counts, 32ull * W, 0u, s);
  if (e != hipSuccess) return e;
  DeviceInfo di;
  e = device_info(&di);
  if (e != hipSuccess) return e;
  const uint32_t word_groups = (W + kWave - 1) / kWave;
  // enough waves to fill the GPU, but at least 64 rows per wave so the
  // counter flush (32 atomics per lane) stays small next to the loads
  const uint64_t target_waves = (uint64_t)di.cus * 32;
  uint64_t slabs = target_waves / word_groups;
  if (slabs < 1) slabs = 1;
  if (slabs > (n + 63) / 64) slabs = (n + 63) / 64;
  const uint64_t per_slab = (n + slabs - 1) / slabs;
  slabs = (n + per_slab - 1) / per_slab;
  hipLaunchKernelGGL(k_meta_count, dim3((uint32_t)(slabs * word_groups)), dim3(kWave), 0, s, rows,
                     row_stride, ids, n, W, word_groups, per_slab, counts);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_meta_threshold, dim3((W + 255) / 256), dim3(256), 0, s, counts, W, n,
                     cutoff, mask, bitval);
  return hipGetLastError();
}

}  // namespace ibp
