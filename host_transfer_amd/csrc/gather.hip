// gather.hip -- batched gather + decompress of IBP tensors (the critical path).
//
// [G-EN] Core Algorithm, Decompression: one warp per tensor, the compressed
// segment staged in shared memory, a warp scan for each thread's chunk start,
// then every thread re-inserts the invariant bits on its own.  [JH]
// decompression paragraph: one thread per chunk, no cross-warp
// synchronisation; transfer paragraph: GPU-initiated 128 B-aligned reads of
// host memory.  On gfx950 a group of G = 64..512 threads (one or more wave64s)
// handles one tensor:
//   1. the first wave reads the chunk participation bits (lane c owns chunk
//      c, n_c <= 64), a wave scan gives each chunk's bit offset in the payload
//      and the payload length;
//   2. the group copies the payload (16 B per lane, whole 16 B units from a
//      16 B-aligned start, so every 128 B line of it is read once) from the
//      host-mapped slot or the HBM cache into LDS;
//   3. each thread decodes its own words: a 64-bit window of the payload at the
//      word's bit offset (two LDS words and v_alignbit), unpack with the
//      word's move masks, insert Bitval; raw chunks take the window as is;
//   4. coalesced 4 B stores of the dense row (consecutive lanes, consecutive
//      words).
// Latency is hidden by occupancy: many groups per CU each wait on their own
// payload while others decode.
#include "ibp_internal.h"
#include "ibp_plan.h"

namespace ibp {

struct GatherArgs {
  const uint8_t* store;
  uint64_t store_bytes;
  uint64_t slot_bytes;
  const uint64_t* offsets;
  const uint32_t* part_bits;
  uint64_t n_tensors;
  const int64_t* ids;
  uint64_t n_ids;
  const uint32_t* mask;
  const uint32_t* bitval;
  uint32_t* out;
  Shape sh;
  uint32_t groups;      // groups per workgroup
  uint32_t pbuf_bytes;  // LDS payload buffer per group
};

// LDS layout, in bytes from the start of dynamic shared memory.
struct GatherLds {
  uint32_t pref, kc, wsum, group0, group_stride;
  __host__ __device__ static uint32_t align16(uint32_t x) { return (x + 15u) & ~15u; }
  __host__ __device__ GatherLds(uint32_t W, uint32_t pbuf_bytes) {
    pref = 0;
    kc = align16(4u * (W + 1));
    wsum = kc + 256;
    group0 = wsum + 64;
    group_stride = (uint32_t)sizeof(GroupHdr) + 256 + pbuf_bytes;
  }
  __host__ __device__ uint32_t total(uint32_t groups) const { return group0 + groups * group_stride; }
};

template <int J>
__global__ __launch_bounds__(1024) void k_gather_decompress(GatherArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const GatherLds L(a.sh.W, a.pbuf_bytes);
  uint32_t* s_pref = (uint32_t*)(smem + L.pref);
  uint32_t* s_kc = (uint32_t*)(smem + L.kc);
  uint32_t* s_wsum = (uint32_t*)(smem + L.wsum);

  const uint32_t G = a.sh.group;
  const uint32_t g = threadIdx.x / G;
  const uint32_t gl = threadIdx.x - g * G;
  uint8_t* gbase = smem + L.group0 + g * L.group_stride;
  GroupHdr* hdr = (GroupHdr*)gbase;
  uint32_t* s_obuf = (uint32_t*)(gbase + sizeof(GroupHdr));
  uint8_t* pbuf = gbase + sizeof(GroupHdr) + 256;
  const uint32_t* pb32 = (const uint32_t*)pbuf;

  WordRegs<J> R;
  load_plan<J>(a.mask, a.bitval, a.sh, s_pref, s_kc, s_wsum, gl, R);

  const bool single = G == kWave;
  const uint32_t W = a.sh.W, n_c = a.sh.n_c;
  const uint64_t step = (uint64_t)gridDim.x * a.groups;
  for (uint64_t row = (uint64_t)blockIdx.x * a.groups + g; row < a.n_ids; row += step) {
    // 1. participation bits, chunk offsets and payload length (first wave)
    if (gl < kWave) {
      const int64_t id = a.ids[row];
      const bool valid = id >= 0 && (uint64_t)id < a.n_tensors;
      uint32_t size = 0;
      bool p = false;
      if (valid && gl < n_c) {
        const uint64_t bit = (uint64_t)id * n_c + gl;
        p = (a.part_bits[bit >> 5] >> (bit & 31)) & 1u;
        size = p ? s_kc[gl] : chunk_bits(a.sh, gl);
      }
      const uint32_t incl = wave_inclusive_sum(size);
      if (gl < n_c) s_obuf[gl] = incl - size;
      const uint64_t pm = __ballot(p);
      const uint32_t total = __shfl(incl, kWave - 1, kWave);
      if (gl == 0) {
        hdr->pmask = pm;
        hdr->valid = valid;
        hdr->len = (total + 7u) >> 3;
        hdr->base = !valid ? 0 : (a.offsets ? a.offsets[id] : (uint64_t)id * a.slot_bytes);
      }
    }
    group_sync(single);
    const uint64_t pmask = hdr->pmask;
    const bool valid = hdr->valid != 0;
    const uint32_t len = hdr->len;
    const uint64_t base = hdr->base;

    // 2. payload -> LDS, whole 16 B units, never past store_bytes
    if (valid) {
      const uint64_t avail = base < a.store_bytes ? (a.store_bytes - base) & ~15ull : 0ull;
      const uint32_t want = (len + 15u) & ~15u;
      const uint32_t n16 = (uint32_t)(min((uint64_t)want, avail) >> 4);
      const uint4* src = (const uint4*)(a.store + base);
      uint4* dst = (uint4*)pbuf;
      for (uint32_t q = gl; q < n16; q += G) dst[q] = src[q];
    }
    group_sync(single);

    // 3 + 4. decode the thread's words and store them
    uint32_t* orow = a.out + row * W;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint32_t w = gl + G * j;
      if (w < W) {
        const uint32_t c = w >> a.sh.wpc_log2;
        const bool p = (pmask >> c) & 1u;
        const uint32_t off = s_obuf[c] + (p ? (R.info[j] & 0xFFFFu) : (R.info[j] >> 16));
        const uint32_t d0 = pb32[off >> 5];
        const uint32_t d1 = pb32[(off >> 5) + 1];
        const uint32_t x = __builtin_amdgcn_alignbit(d1, d0, off & 31u);
        const uint32_t y = bfi(R.mask[j], R.bitval[j], unpack_bits(x, R.mv[j]));
        orow[w] = valid ? (p ? y : x) : 0u;
      }
    }
    group_sync(single);
  }
}

template <int J>
static hipError_t launch_j(const Geometry& g, const GatherArgs& a, hipStream_t s) {
  const GatherLds L(g.W, a.pbuf_bytes);
  const uint32_t lds = L.total(g.groups);
  const uint32_t threads = g.group * g.groups;
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_gather_decompress<J>, threads, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  const uint64_t want = (a.n_ids + g.groups - 1) / g.groups;
  const uint64_t cap = (uint64_t)per_cu * (uint64_t)di.cus;
  const uint32_t blocks = (uint32_t)(want < cap ? want : cap);
  hipLaunchKernelGGL(k_gather_decompress<J>, dim3(blocks), dim3(threads), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_gather(const Geometry& g, const uint8_t* store, uint64_t store_bytes,
                         uint64_t slot_bytes, const uint64_t* offsets, const uint32_t* part_bits,
                         uint64_t n_tensors, const int64_t* ids, uint64_t n_ids,
                         const uint32_t* mask, const uint32_t* bitval, uint32_t* out,
                         hipStream_t s) {
  if (n_ids == 0) return hipSuccess;
  GatherArgs a;
  a.store = store;
  a.store_bytes = store_bytes;
  a.slot_bytes = slot_bytes;
  a.offsets = offsets;
  a.part_bits = part_bits;
  a.n_tensors = n_tensors;
  a.ids = ids;
  a.n_ids = n_ids;
  a.mask = mask;
  a.bitval = bitval;
  a.out = out;
  a.sh = Shape{g.W, g.n_c, g.wpc_log2, g.last_bits, g.group};
  a.groups = g.groups;
  // payload rounded to 16 B, plus one word read past the end by the window
  a.pbuf_bytes = ((g.tensor_bytes + 15u) & ~15u) + 16u;
  switch (g.J) {
    case 1: return launch_j<1>(g, a, s);
    case 2: return launch_j<2>(g, a, s);
    case 3: return launch_j<3>(g, a, s);
    case 4: return launch_j<4>(g, a, s);
    case 5: return launch_j<5>(g, a, s);
    case 6: return launch_j<6>(g, a, s);
    case 7: return launch_j<7>(g, a, s);
    case 8: return launch_j<8>(g, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ibp
