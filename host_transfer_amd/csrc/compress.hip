// compress.hip -- IBP compression and compaction (off the critical path).
//
// [G-EN] Core Algorithm, Compression: chunk by chunk, the invariant positions
// are checked against Bitval; a matching chunk drops them and closes the gaps,
// a chunk that does not match (or would not shrink) is kept whole, and its
// participation bit records which.  The GPU writes the result straight into
// the (possibly host-mapped) store.  [G-EN] System Integration: in-place
// fixed-size slots and a GPU-memory bitmask; cache compression keeps the
// compressed tensors packed in GPU memory (ibp_compact).
//
// One group of G threads per tensor, with the same word ownership and
// registers as the decompressor (ibp_plan.h):
//   1. each thread loads its words (coalesced) and flags its chunk in LDS if
//      a Mask bit differs from Bitval;
//   2. the first wave decides P per chunk (lane c owns chunk c), scans the
//      chunk sizes into bit offsets, and updates the bitmap bits of the
//      tensor (atomic AND/OR, so neighbouring tensors sharing a bitmap word
//      can be compressed concurrently);
//   3. each thread packs its words and ORs them into an LDS buffer at their
//      bit offsets (LDS atomics; a word can straddle two buffer words);
//   4. the group writes the buffer to the slot in 16 B stores and clears it.
#include "ibp_internal.h"
#include "ibp_plan.h"

namespace ibp {

struct CompressArgs {
  const uint8_t* rows;
  uint64_t row_stride;
  uint64_t n_rows;
  uint64_t first;
  const uint32_t* mask;
  const uint32_t* bitval;
  uint8_t* store;
  uint64_t slot_bytes;
  uint32_t* part_bits;
  uint32_t* lengths;
  Shape sh;
  uint32_t groups;
  uint32_t pbuf_bytes;
};

struct CompressLds {
  uint32_t pref, kc, wsum, group0, group_stride;
  __host__ __device__ CompressLds(uint32_t W, uint32_t pbuf_bytes) {
    pref = 0;
    kc = ((4u * (W + 1)) + 15u) & ~15u;
    wsum = kc + 256;
    group0 = wsum + 64;
    // header, chunk offsets, chunk mismatch flags, payload buffer
    group_stride = (uint32_t)sizeof(GroupHdr) + 256 + 256 + pbuf_bytes;
  }
  __host__ __device__ uint32_t total(uint32_t groups) const { return group0 + groups * group_stride; }
};

// The body of the compress kernel for workgroup `block` of `blocks` (the
// whole grid, or the workgroups of one segment of k_compress_seg).
template <int J>
__device__ __forceinline__ void compress_body(const CompressArgs& a, uint32_t block,
                                              uint32_t blocks) {
  extern __shared__ __align__(16) uint8_t smem[];
  const CompressLds L(a.sh.W, a.pbuf_bytes);
  uint32_t* s_pref = (uint32_t*)(smem + L.pref);
  uint32_t* s_kc = (uint32_t*)(smem + L.kc);
  uint32_t* s_wsum = (uint32_t*)(smem + L.wsum);

  const uint32_t G = a.sh.group;
  const uint32_t g = threadIdx.x / G;
  const uint32_t gl = threadIdx.x - g * G;
  uint8_t* gbase = smem + L.group0 + g * L.group_stride;
  GroupHdr* hdr = (GroupHdr*)gbase;
  uint32_t* s_obuf = (uint32_t*)(gbase + sizeof(GroupHdr));
  uint32_t* s_fail = (uint32_t*)(gbase + sizeof(GroupHdr) + 256);
  uint8_t* pbuf = gbase + sizeof(GroupHdr) + 512;
  uint32_t* pb32 = (uint32_t*)pbuf;
  uint4* pb128 = (uint4*)pbuf;

  // clean buffer and flags before the first tensor
  for (uint32_t q = gl; q < a.pbuf_bytes / 16; q += G) pb128[q] = make_uint4(0, 0, 0, 0);
  if (gl < kWave) s_fail[gl] = 0;

  WordRegs<J> R;
  PlanRun run;
  load_plan_run(a.mask, a.sh, run);
  load_plan_fetch<J>(a.mask, a.bitval, a.sh, gl, R);
  load_plan_counts(run, a.sh, s_pref, s_kc, s_wsum);
  load_plan_words<J>(a.sh, s_pref, gl, R);

  const bool single = G == kWave;
  const uint32_t W = a.sh.W, n_c = a.sh.n_c;
  const uint64_t step = (uint64_t)blocks * a.groups;
  for (uint64_t row = (uint64_t)block * a.groups + g; row < a.n_rows; row += step) {
    const uint64_t t = a.first + row;
    const uint32_t* x32 = (const uint32_t*)(a.rows + row * a.row_stride);

    // 1. load words, flag mismatching chunks
    uint32_t x[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint32_t w = gl + G * j;
      x[j] = w < W ? x32[w] : 0u;
      if (w < W && ((x[j] ^ R.bitval[j]) & R.mask[j]) != 0u) s_fail[w >> a.sh.wpc_log2] = 1u;
    }
    group_sync(single);

    // 2. participation, offsets, length, bitmap (first wave)
    if (gl < kWave) {
      uint32_t size = 0;
      bool p = false;
      if (gl < n_c) {
        const uint32_t bits = chunk_bits(a.sh, gl);
        p = s_fail[gl] == 0u && s_kc[gl] < bits;
        size = p ? s_kc[gl] : bits;
        s_fail[gl] = 0u;
        const uint64_t bit = t * n_c + gl;
        const uint32_t b = 1u << (bit & 31);
        if (p)
          atomicOr(a.part_bits + (bit >> 5), b);
        else
          atomicAnd(a.part_bits + (bit >> 5), ~b);
      }
      const uint32_t incl = wave_inclusive_sum(size);
      if (gl < n_c) s_obuf[gl] = incl - size;
      const uint64_t pm = __ballot(p);
      const uint32_t total = __shfl(incl, kWave - 1, kWave);
      if (gl == 0) {
        hdr->pmask = pm;
        hdr->len = (total + 7u) >> 3;
      }
    }
    group_sync(single);
    const uint64_t pmask = hdr->pmask;
    const uint32_t len = hdr->len;

    // 3. pack and deposit at the bit offsets
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint32_t w = gl + G * j;
      if (w < W) {
        const uint32_t c = w >> a.sh.wpc_log2;
        const bool p = (pmask >> c) & 1u;
        const uint32_t off = s_obuf[c] + (p ? (R.info[j] & 0xFFFFu) : (R.info[j] >> 16));
        const uint32_t v = p ? pack_bits(x[j], ~R.mask[j], R.mv[j]) : x[j];
        const uint32_t sh = off & 31u;
        const uint32_t lo = v << sh;
        const uint32_t hi = sh ? (v >> (32u - sh)) : 0u;
        if (lo) atomicOr(pb32 + (off >> 5), lo);
        if (hi) atomicOr(pb32 + (off >> 5) + 1, hi);
      }
    }
    group_sync(single);

    // 4. buffer -> slot (16 B units up to the payload's end), then clear it
    uint4* dst = (uint4*)(a.store + t * a.slot_bytes);
    const uint32_t n16 = (len + 15u) >> 4;
    for (uint32_t q = gl; q < n16; q += G) {
      dst[q] = pb128[q];
      pb128[q] = make_uint4(0, 0, 0, 0);
    }
    if (gl == 0 && a.lengths) a.lengths[t] = len;
    group_sync(single);
  }
}

template <int J>
__global__ __launch_bounds__(1024) void k_compress(CompressArgs a) {
  compress_body<J>(a, blockIdx.x, gridDim.x);
}

// Several compress calls of one tensor shape in one launch, each segment with
// its own Mask/Bitval (compress-on-write of one decode token's K/V rows for
// every (layer, K|V) pair).  Segment k compresses rows row0[k] + i of `rows`
// as tensors first[k] + i, i < count[k].  Workgroup b serves segment
// b / per_seg as workgroup b % per_seg of per_seg.
constexpr uint32_t kCompressSegs = 128;  // segments per launch (kernel-argument space)

struct CompressSegTable {
  uint64_t row0[kCompressSegs];
  uint64_t first[kCompressSegs];
  uint32_t count[kCompressSegs];
  uint32_t per_seg;
};

template <int J>
__global__ __launch_bounds__(1024) void k_compress_seg(CompressArgs a, CompressSegTable t) {
  const uint32_t seg = blockIdx.x / t.per_seg;  // < segments of this launch
  if (t.count[seg] == 0) return;                // the whole workgroup, before any barrier
  CompressArgs b = a;
  b.rows = a.rows + t.row0[seg] * a.row_stride;
  b.n_rows = t.count[seg];
  b.first = t.first[seg];
  b.mask = a.mask + (uint64_t)seg * a.sh.W;
  b.bitval = a.bitval + (uint64_t)seg * a.sh.W;
  compress_body<J>(b, blockIdx.x % t.per_seg, t.per_seg);
}

template <int J>
static hipError_t launch_j(const Geometry& g, const CompressArgs& a, hipStream_t s) {
  const CompressLds L(g.W, a.pbuf_bytes);
  const uint32_t lds = L.total(g.groups);
  const uint32_t threads = g.group * g.groups;
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_compress<J>, threads, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  const uint64_t want = (a.n_rows + g.groups - 1) / g.groups;
  const uint64_t cap = (uint64_t)per_cu * (uint64_t)di.cus;
  const uint32_t blocks = (uint32_t)(want < cap ? want : cap);
  hipLaunchKernelGGL(k_compress<J>, dim3(blocks), dim3(threads), lds, s, a);
  return hipGetLastError();
}

template <int J>
static hipError_t launch_j_seg(const Geometry& g, const CompressArgs& a, CompressSegTable& t,
                               uint32_t n_seg, uint64_t max_rows, hipStream_t s) {
  const CompressLds L(g.W, a.pbuf_bytes);
  const uint32_t lds = L.total(g.groups);
  const uint32_t threads = g.group * g.groups;
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_compress_seg<J>, threads, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  const uint64_t cap = (uint64_t)per_cu * (uint64_t)di.cus;
  uint64_t per = cap / n_seg;
  const uint64_t need = (max_rows + g.groups - 1) / g.groups;
  if (per > need) per = need;
  if (per < 1) per = 1;
  t.per_seg = (uint32_t)per;
  hipLaunchKernelGGL(k_compress_seg<J>, dim3((uint32_t)(per * n_seg)), dim3(threads), lds, s, a,
                     t);
  return hipGetLastError();
}

hipError_t launch_compress_segments(const Geometry& g, const uint8_t* rows, uint64_t row_stride,
                                    const uint64_t* seg_row, const uint64_t* seg_first,
                                    const uint64_t* seg_count, uint32_t n_seg,
                                    const uint32_t* masks, const uint32_t* bitvals,
                                    uint8_t* store, uint64_t slot_bytes, uint32_t* part_bits,
                                    uint32_t* lengths, hipStream_t s) {
  CompressArgs a;
  a.rows = rows;
  a.row_stride = row_stride;
  a.n_rows = 0;
  a.first = 0;
  a.store = store;
  a.slot_bytes = slot_bytes;
  a.part_bits = part_bits;
  a.lengths = lengths;
  a.sh = Shape{g.W, g.n_c, g.wpc_log2, g.last_bits, g.group};
  a.groups = g.groups;
  a.pbuf_bytes = ((g.tensor_bytes + 15u) & ~15u) + 16u;
  for (uint32_t k0 = 0; k0 < n_seg; k0 += kCompressSegs) {
    const uint32_t n = n_seg - k0 < kCompressSegs ? n_seg - k0 : kCompressSegs;
    CompressSegTable t;
    uint64_t max_rows = 0;
    for (uint32_t k = 0; k < n; ++k) {
      t.row0[k] = seg_row[k0 + k];
      t.first[k] = seg_first[k0 + k];
      t.count[k] = (uint32_t)seg_count[k0 + k];
      if (seg_count[k0 + k] > max_rows) max_rows = seg_count[k0 + k];
    }
    t.per_seg = 1;
    if (max_rows == 0) continue;
    a.mask = masks + (uint64_t)k0 * g.W;
    a.bitval = bitvals + (uint64_t)k0 * g.W;
    hipError_t e;
    switch (g.J) {
      case 1: e = launch_j_seg<1>(g, a, t, n, max_rows, s); break;
      case 2: e = launch_j_seg<2>(g, a, t, n, max_rows, s); break;
      case 3: e = launch_j_seg<3>(g, a, t, n, max_rows, s); break;
      case 4: e = launch_j_seg<4>(g, a, t, n, max_rows, s); break;
      case 5: e = launch_j_seg<5>(g, a, t, n, max_rows, s); break;
      case 6: e = launch_j_seg<6>(g, a, t, n, max_rows, s); break;
      default: e = hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_compress(const Geometry& g, const uint8_t* rows, uint64_t row_stride,
                           uint64_t n_rows, uint64_t first, const uint32_t* mask,
                           const uint32_t* bitval, uint8_t* store, uint64_t slot_bytes,
                           uint32_t* part_bits, uint32_t* lengths, hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  CompressArgs a;
  a.rows = rows;
  a.row_stride = row_stride;
  a.n_rows = n_rows;
  a.first = first;
  a.mask = mask;
  a.bitval = bitval;
  a.store = store;
  a.slot_bytes = slot_bytes;
  a.part_bits = part_bits;
  a.lengths = lengths;
  a.sh = Shape{g.W, g.n_c, g.wpc_log2, g.last_bits, g.group};
  a.groups = g.groups;
  a.pbuf_bytes = ((g.tensor_bytes + 15u) & ~15u) + 16u;
  switch (g.J) {
    case 1: return launch_j<1>(g, a, s);
    case 2: return launch_j<2>(g, a, s);
    case 3: return launch_j<3>(g, a, s);
    case 4: return launch_j<4>(g, a, s);
    case 5: return launch_j<5>(g, a, s);
    case 6: return launch_j<6>(g, a, s);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------- compaction

// offsets[t] = sum of roundup(lengths[u], align) over the selected u < t;
// offsets[n] = total.  select: null (every tensor) or a flag per tensor; with
// `mark`, an unselected tensor's entry is kNotCachedEntry.  One workgroup
// walks the array in tiles of 4 x 1024 entries (off the critical path: a few
// milliseconds for millions of tensors).  align: a power of two, 16..4096.
constexpr uint64_t kNotCachedEntry = ~0ull;

__global__ __launch_bounds__(1024) void k_compact_offsets(const uint32_t* __restrict__ lengths,
                                                           const uint32_t* __restrict__ select,
                                                           uint64_t n, uint32_t align,
                                                           uint64_t* __restrict__ offsets,
                                                           bool mark) {
  __shared__ uint32_t s_wsum[16];
  const uint32_t tid = threadIdx.x;
  const uint32_t am = align - 1u;
  uint64_t carry = 0;
  for (uint64_t base = 0; base < n; base += 4096) {
    uint32_t v[4];
    bool sel[4];
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint64_t t = base + 4u * tid + i;
      sel[i] = t < n && (select == nullptr || select[t] != 0u);
      v[i] = sel[i] ? ((lengths[t] + am) & ~am) : 0u;
      local += v[i];
    }
    uint32_t tot;
    const uint32_t incl = block_inclusive_sum(local, s_wsum, &tot);
    uint64_t o = carry + (incl - local);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint64_t t = base + 4u * tid + i;
      if (t < n) offsets[t] = (mark && !sel[i]) ? kNotCachedEntry : o;
      o += v[i];
    }
    carry += tot;
  }
  if (tid == 0) offsets[n] = carry;
}

// index[w] = (participating chunks in bitmap words 0..w-1) << 32 |
// part_bits[w], for w < ceil(n_bits / 32); bits at or past n_bits are
// cleared.  One workgroup, tiles of 4 x 1024 words.  The count is exact
// while n_bits < 2^32.
__global__ __launch_bounds__(1024) void k_cache_index(const uint32_t* __restrict__ part_bits,
                                                       uint64_t n_bits,
                                                       uint64_t* __restrict__ index) {
  __shared__ uint32_t s_wsum[16];
  const uint32_t tid = threadIdx.x;
  const uint64_t n_words = (n_bits + 31u) / 32u;
  uint32_t carry = 0;
  for (uint64_t base = 0; base < n_words; base += 4096) {
    uint32_t wv[4];
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint64_t w = base + 4u * tid + i;
      uint32_t x = w < n_words ? part_bits[w] : 0u;
      if (w + 1u == n_words && (n_bits & 31u)) x &= (1u << (n_bits & 31u)) - 1u;
      wv[i] = x;
      local += (uint32_t)__popc(x);
    }
    uint32_t tot;
    const uint32_t incl = block_inclusive_sum(local, s_wsum, &tot);
    uint32_t r = carry + (incl - local);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint64_t w = base + 4u * tid + i;
      if (w < n_words) index[w] = ((uint64_t)r << 32) | wv[i];
      r += (uint32_t)__popc(wv[i]);
    }
    carry += tot;
  }
}

// One wave per cached tensor: copies its payload (rounded up to 16 B) from
// its slot to cache + offsets[t].  Entries that would end past cache_bytes or
// read past the slot are skipped.
__global__ __launch_bounds__(256) void k_cache_fill(const uint8_t* __restrict__ store,
                                                     uint64_t slot_bytes,
                                                     const uint32_t* __restrict__ lengths,
                                                     uint64_t n, const uint64_t* __restrict__ offsets,
                                                     uint8_t* __restrict__ cache,
                                                     uint64_t cache_bytes) {
  const uint32_t lane = lane_id();
  const uint64_t wave = (uint64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const uint64_t waves = (uint64_t)gridDim.x * (blockDim.x / kWave);
  for (uint64_t t = wave; t < n; t += waves) {
    const uint64_t o = offsets[t];
    const uint64_t size = ((uint64_t)lengths[t] + 15u) & ~15ull;
    if (o == kNotCachedEntry || (o & 15u) != 0 || size > slot_bytes || o > cache_bytes ||
        size > cache_bytes - o)
      continue;
    const uint4* src = (const uint4*)(store + t * slot_bytes);
    uint4* dst = (uint4*)(cache + o);
    for (uint32_t q = lane; q < (uint32_t)(size >> 4); q += kWave) dst[q] = src[q];
  }
}

// One wave per entry: copies offsets[t+1] - offsets[t] bytes from slot t.
__global__ __launch_bounds__(256) void k_compact_copy(const uint8_t* __restrict__ store,
                                                       uint64_t slot_bytes, uint64_t n,
                                                       const uint64_t* __restrict__ offsets,
                                                       uint8_t* __restrict__ cache,
                                                       uint64_t cache_bytes) {
  const uint32_t lane = lane_id();
  const uint64_t wave = (uint64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const uint64_t waves = (uint64_t)gridDim.x * (blockDim.x / kWave);
  for (uint64_t t = wave; t < n; t += waves) {
    const uint64_t o0 = offsets[t], o1 = offsets[t + 1];
    if (o1 < o0 || o1 > cache_bytes || ((o0 | o1) & 15u) != 0 || o1 - o0 > slot_bytes) continue;
    const uint4* src = (const uint4*)(store + t * slot_bytes);
    uint4* dst = (uint4*)(cache + o0);
    const uint32_t n16 = (uint32_t)((o1 - o0) >> 4);
    for (uint32_t q = lane; q < n16; q += kWave) dst[q] = src[q];
  }
}

hipError_t launch_compact_offsets(const uint32_t* lengths, uint64_t n, uint32_t align,
                                  uint64_t* offsets, hipStream_t s) {
  hipLaunchKernelGGL(k_compact_offsets, dim3(1), dim3(1024), 0, s, lengths,
                     (const uint32_t*)nullptr, n, align, offsets, false);
  return hipGetLastError();
}

hipError_t launch_cache_index(const uint32_t* part_bits, uint64_t n_bits, uint64_t* index,
                              hipStream_t s) {
  if (n_bits == 0) return hipSuccess;
  hipLaunchKernelGGL(k_cache_index, dim3(1), dim3(1024), 0, s, part_bits, n_bits, index);
  return hipGetLastError();
}

hipError_t launch_cache_offsets(const uint32_t* lengths, const uint32_t* select, uint64_t n,
                                uint64_t* offsets, hipStream_t s) {
  hipLaunchKernelGGL(k_compact_offsets, dim3(1), dim3(1024), 0, s, lengths, select, n, 16u,
                     offsets, true);
  return hipGetLastError();
}

hipError_t launch_cache_fill(const uint8_t* store, uint64_t slot_bytes, const uint32_t* lengths,
                             uint64_t n, const uint64_t* offsets, uint8_t* cache,
                             uint64_t cache_bytes, hipStream_t s) {
  if (n == 0) return hipSuccess;
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  const uint64_t want = (n + 3) / 4;
  const uint64_t cap = (uint64_t)di.cus * 8;
  hipLaunchKernelGGL(k_cache_fill, dim3((uint32_t)(want < cap ? want : cap)), dim3(256), 0, s,
                     store, slot_bytes, lengths, n, offsets, cache, cache_bytes);
  return hipGetLastError();
}

hipError_t launch_compact(const uint8_t* store, uint64_t slot_bytes, uint64_t n,
                          const uint64_t* offsets, uint8_t* cache, uint64_t cache_bytes,
                          hipStream_t s) {
  if (n == 0) return hipSuccess;
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  const uint64_t want = (n + 3) / 4;
  const uint64_t cap = (uint64_t)di.cus * 8;
  hipLaunchKernelGGL(k_compact_copy, dim3((uint32_t)(want < cap ? want : cap)), dim3(256), 0, s,
                     store, slot_bytes, n, offsets, cache, cache_bytes);
  return hipGetLastError();
}

}  // namespace ibp
