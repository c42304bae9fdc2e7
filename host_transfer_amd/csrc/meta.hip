// meta.hip -- Mask/Bitval metadata build (off the critical path).
//
// [G-EN] Core Algorithm, Preprocessing: over a set of tensors (a sample is
// enough, [JH] sampling paragraph), find the bit positions whose value agrees
// across at least a fraction T of them, and record them (Mask) with their
// value (Bitval).  Two kernels:
//   k_meta_count      per bit position, the number of sampled tensors with
//                     that bit set.  Lane l of a wave owns word w (coalesced
//                     loads across lanes) and counts over a slab of sampled
//                     rows with carry-save adders (see the kernel); a
//                     workgroup's four waves sum in LDS, then add to the
//                     global counters with atomics.
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

// Carry-save adder on 32 independent bit positions: h:l = a + b + c per
// position (l the sum bit, h the carry).
__device__ __forceinline__ void csa(uint32_t& h, uint32_t& l, uint32_t a, uint32_t b,
                                    uint32_t c) {
  const uint32_t u = a ^ b;
  h = (a & b) | (u & c);
  l = u ^ c;
}

constexpr uint32_t kMetaWaves = 4;  // waves per workgroup, all on the same 64 words

// grid: word_groups * slabs workgroups of 4 waves; workgroup b handles words
// [64*(b % word_groups), +64) of sampled rows [per_slab*(b / word_groups),
// +per_slab), wave k a quarter of those rows.  Lane l counts the ones of each
// bit position of word 64*(b % word_groups) + l (coalesced loads across
// lanes).  Positional population count: sixteen rows at a time go through a
// tree of carry-save adders (the Harley-Seal scheme; H. S. Warren, "Hacker's
// Delight", 2nd ed., section 5-1), which leaves per bit position a sum in
// the bit planes ones/twos/fours/eights and one "sixteens" carry word; only
// that word is added into the 32 counters.  About 9 operations per row and
// word instead of 64.  The workgroup's four waves add their counts in LDS,
// and the workgroup adds the totals to the global counters with atomics.
// kIds: rows are picked by sample ids (else rows 0..n-1).  A template
// parameter rather than a test per row, so the sixteen loads of a group are
// issued together instead of each one waiting behind a branch.
template <bool kIds>
__global__ __launch_bounds__(256) void k_meta_count(const uint8_t* __restrict__ rows,
                                                     uint64_t row_stride,
                                                     const int64_t* __restrict__ ids, uint64_t n,
                                                     uint32_t W, uint32_t word_groups,
                                                     uint64_t per_slab,
                                                     uint32_t* __restrict__ counts) {
  __shared__ uint32_t s_cnt[32 * kWave];  // [bit][lane]
  const uint32_t wg = blockIdx.x % word_groups;
  const uint64_t slab = blockIdx.x / word_groups;
  const uint32_t lane = threadIdx.x % kWave;
  const uint32_t wave = threadIdx.x / kWave;
  const uint32_t w = wg * kWave + lane;
  const bool active = w < W;
  const uint32_t wl = active ? w : W - 1u;  // clamped: every lane loads
  for (uint32_t i = threadIdx.x; i < 32 * kWave; i += blockDim.x) s_cnt[i] = 0;
  // this wave's rows of the slab
  const uint64_t s0 = min(n, slab * per_slab), s1 = min(n, s0 + per_slab);
  const uint64_t per_wave = (s1 - s0 + kMetaWaves - 1) / kMetaWaves;
  const uint64_t r0 = min(s1, s0 + wave * per_wave), r1 = min(s1, r0 + per_wave);
  const uint8_t* base = rows + 4ull * wl;
  uint32_t cnt[32];
#pragma unroll
  for (int b = 0; b < 32; ++b) cnt[b] = 0;
  uint32_t ones = 0, twos = 0, fours = 0, eights = 0;
  uint64_t s = r0;
  for (; s + 16 <= r1; s += 16) {
    uint64_t r[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) r[i] = kIds ? (uint64_t)ids[s + i] : s + i;
    uint32_t x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = *(const uint32_t*)(base + r[i] * row_stride);
    uint32_t twosA, twosB, foursA, foursB, eightsA, eightsB, sixteens;
    csa(twosA, ones, ones, x[0], x[1]);
    csa(twosB, ones, ones, x[2], x[3]);
    csa(foursA, twos, twos, twosA, twosB);
    csa(twosA, ones, ones, x[4], x[5]);
    csa(twosB, ones, ones, x[6], x[7]);
    csa(foursB, twos, twos, twosA, twosB);
    csa(eightsA, fours, fours, foursA, foursB);
    csa(twosA, ones, ones, x[8], x[9]);
    csa(twosB, ones, ones, x[10], x[11]);
    csa(foursA, twos, twos, twosA, twosB);
    csa(twosA, ones, ones, x[12], x[13]);
    csa(twosB, ones, ones, x[14], x[15]);
    csa(foursB, twos, twos, twosA, twosB);
    csa(eightsB, fours, fours, foursA, foursB);
    csa(sixteens, eights, eights, eightsA, eightsB);
#pragma unroll
    for (int b = 0; b < 32; ++b) cnt[b] += (sixteens >> b) & 1u;  // in units of 16
  }
  // fewer than 16 rows left: add them one at a time through the planes
  for (; s < r1; ++s) {
    const uint64_t r = kIds ? (uint64_t)ids[s] : s;
    uint32_t c = *(const uint32_t*)(base + r * row_stride);
    uint32_t t = ones & c;
    ones ^= c;
    c = t;
    t = twos & c;
    twos ^= c;
    c = t;
    t = fours & c;
    fours ^= c;
    c = t;
    t = eights & c;
    eights ^= c;
#pragma unroll
    for (int b = 0; b < 32; ++b) cnt[b] += (t >> b) & 1u;
  }
  __syncthreads();  // s_cnt cleared
  if (active) {
#pragma unroll
    for (int b = 0; b < 32; ++b) {
      const uint32_t v = 16u * cnt[b] + 8u * ((eights >> b) & 1u) + 4u * ((fours >> b) & 1u) +
                         2u * ((twos >> b) & 1u) + ((ones >> b) & 1u);
      if (v) atomicAdd(&s_cnt[b * kWave + lane], v);
    }
  }
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < 32 * kWave; i += blockDim.x) {
    const uint32_t b = i / kWave, l = i % kWave;
    const uint32_t ww = wg * kWave + l;
    const uint32_t v = s_cnt[i];
    if (ww < W && v) atomicAdd(counts + 32ull * ww + b, v);
  }
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
  // about 16 waves per CU, but at least 64 rows per wave (four groups of 16)
  // so the counter flush stays small next to the loads
  const uint64_t target_blocks = (uint64_t)di.cus * 16 / kMetaWaves;
  uint64_t slabs = target_blocks / word_groups;
  if (slabs < 1) slabs = 1;
  const uint64_t min_rows = 64ull * kMetaWaves;
  if (slabs > (n + min_rows - 1) / min_rows) slabs = (n + min_rows - 1) / min_rows;
  const uint64_t per_slab = (n + slabs - 1) / slabs;
  slabs = (n + per_slab - 1) / per_slab;
  if (ids)
    hipLaunchKernelGGL(k_meta_count<true>, dim3((uint32_t)(slabs * word_groups)),
                       dim3(kWave * kMetaWaves), 0, s, rows, row_stride, ids, n, W, word_groups,
                       per_slab, counts);
  else
    hipLaunchKernelGGL(k_meta_count<false>, dim3((uint32_t)(slabs * word_groups)),
                       dim3(kWave * kMetaWaves), 0, s, rows, row_stride, ids, n, W, word_groups,
                       per_slab, counts);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_meta_threshold, dim3((W + 255) / 256), dim3(256), 0, s, counts, W, n,
                     cutoff, mask, bitval);
  return hipGetLastError();
}

}  // namespace ibp
