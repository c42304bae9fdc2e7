// gather.hip -- batched gather + decompress of IBP tensors (the critical path).
//
// [G-EN] Core Algorithm, Decompression: one warp per tensor, the compressed
// segment staged in shared memory, a warp scan for each thread's chunk start,
// then every thread re-inserts the invariant bits on its own, with fetches
// overlapped with decoding.  [JH] decompression paragraph: one thread per
// chunk, no cross-warp synchronisation; transfer paragraph: GPU-initiated
// 128 B-aligned reads of host memory.  On gfx950 a group of G = 64..512
// threads (one or more wave64s) handles one tensor at a time:
//   1. the first wave reads the tensor's id and participation bits (lane c
//      owns chunk c, n_c <= 64); a wave scan gives each chunk's bit offset in
//      the payload and the payload length;
//   2. the group loads the payload (whole 16 B units from a 16 B-aligned
//      start, so every 128 B line is read once) from the host-mapped slot or
//      the HBM cache into registers, then LDS;
//   3. each thread decodes its own words: a 64-bit window of the payload at
//      the word's bit offset (two LDS words and v_alignbit), unpack with the
//      word's move masks, insert Bitval; raw chunks take the window as is;
//   4. coalesced 4 B stores of the dense row (consecutive lanes, consecutive
//      words).
// Software pipeline per group: while tensor i is decoded, the payload loads of
// tensor i+1 are in flight, and while tensor i's payload arrives the first
// wave fetches and scans the id and participation bits of tensor i+1.  A
// payload is at most B <= 24*G bytes (at most 6 words per thread), so it
// fits in two 16 B registers per thread.  Workgroup barriers only wait for
// LDS traffic, so global loads stay in flight across them.
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
  uint32_t lpr;         // tile kernel: lanes per tensor in the load phase
};

// LDS layout, in bytes from the start of dynamic shared memory.  Per group:
// two headers and two chunk-offset tables (current and next tensor), one
// payload buffer.
struct GatherLds {
  uint32_t pref, kc, wsum, group0, group_stride;
  __host__ __device__ static uint32_t align16(uint32_t x) { return (x + 15u) & ~15u; }
  __host__ __device__ GatherLds(uint32_t W, uint32_t pbuf_bytes) {
    pref = 0;
    kc = align16(4u * (W + 1));
    wsum = kc + 256;
    group0 = wsum + 64;
    group_stride = 2u * (uint32_t)sizeof(GroupHdr) + 2u * 256u + pbuf_bytes;
  }
  __host__ __device__ uint32_t total(uint32_t groups) const { return group0 + groups * group_stride; }
};

// What the first wave knows about one tensor before its payload is read.
struct RowMeta {
  uint64_t base;  // payload offset in the store
  uint32_t bits;  // participation word holding this lane's chunk bit (shifted)
  bool valid;
};

__device__ __forceinline__ int64_t load_id(const GatherArgs& a, uint64_t row) {
  return row < a.n_ids ? a.ids[row] : -1;
}

// Participation word and payload offset of tensor `id` (lane c: chunk c).
__device__ __forceinline__ RowMeta load_meta(const GatherArgs& a, int64_t id, uint32_t lane) {
  RowMeta m;
  m.valid = id >= 0 && (uint64_t)id < a.n_tensors;
  m.bits = 0;
  m.base = 0;
  if (m.valid) {
    if (lane < a.sh.n_c) {
      const uint64_t bit = (uint64_t)id * a.sh.n_c + lane;
      m.bits = a.part_bits[bit >> 5] >> (bit & 31);
    }
    m.base = a.offsets ? a.offsets[id] : (uint64_t)id * a.slot_bytes;
  }
  return m;
}

// Participation, chunk offsets and payload length of one tensor (first wave).
__device__ __forceinline__ void scan_row(const GatherArgs& a, const RowMeta& m, uint32_t lane,
                                         const uint32_t* s_kc, GroupHdr* hdr, uint32_t* obuf) {
  const bool p = m.valid && lane < a.sh.n_c && (m.bits & 1u);
  const uint32_t size = !m.valid || lane >= a.sh.n_c ? 0u : (p ? s_kc[lane] : chunk_bits(a.sh, lane));
  const uint32_t incl = wave_inclusive_sum(size);
  if (lane < a.sh.n_c) obuf[lane] = incl - size;
  const uint64_t pm = __ballot(p);
  const uint32_t total = __shfl(incl, kWave - 1, kWave);
  if (lane == 0) {
    hdr->pmask = pm;
    hdr->valid = m.valid;
    hdr->len = (total + 7u) >> 3;
    hdr->base = m.base;
  }
}

// Number of 16 B payload units to read: the payload rounded up to 16 B,
// never past store_bytes.
__device__ __forceinline__ uint32_t payload_units(const GatherArgs& a, const GroupHdr& h) {
  if (!h.valid) return 0;
  const uint64_t avail = h.base < a.store_bytes ? (a.store_bytes - h.base) & ~15ull : 0ull;
  const uint32_t want = (h.len + 15u) & ~15u;
  return (uint32_t)(min((uint64_t)want, avail) >> 4);
}

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
  GroupHdr* hdrs = (GroupHdr*)gbase;                                   // [2]
  uint32_t* obufs = (uint32_t*)(gbase + 2 * sizeof(GroupHdr));         // [2][64]
  uint8_t* pbuf = gbase + 2 * sizeof(GroupHdr) + 512;
  const uint32_t* pb32 = (const uint32_t*)pbuf;
  uint4* pb128 = (uint4*)pbuf;

  const bool single = G == kWave;
  const bool first_wave = gl < kWave;
  const uint32_t W = a.sh.W;
  const uint64_t step = (uint64_t)gridDim.x * a.groups;
  const uint64_t row0 = (uint64_t)blockIdx.x * a.groups + g;

  // Metadata runs ahead of the payloads so that no wait for it also waits
  // for a payload still in flight (vector loads retire in issue order):
  // ids three tensors ahead, participation words and offsets two ahead, the
  // scan one ahead.
  int64_t id_a = -1, id_b = -1;
  if (first_wave) {
    id_a = load_id(a, row0);
    id_b = load_id(a, row0 + step);
  }

  WordRegs<J> R;
  load_plan<J>(a.mask, a.bitval, a.sh, s_pref, s_kc, s_wsum, gl, R);

  if (row0 >= a.n_ids) return;  // uniform per group; no workgroup barrier follows for it
  RowMeta meta_next;             // tensor row+step (first wave)
  int64_t id_next2 = -1;         // tensor row+2*step (first wave)
  if (first_wave) {
    const RowMeta m0 = load_meta(a, id_a, gl);
    meta_next = load_meta(a, id_b, gl);
    id_next2 = load_id(a, row0 + 2 * step);
    scan_row(a, m0, gl, s_kc, &hdrs[0], obufs);
  }
  group_sync(single);

  // payload registers of the tensor in flight
  uint4 v0 = make_uint4(0, 0, 0, 0), v1 = v0;
  {
    const GroupHdr h = hdrs[0];
    const uint32_t n16 = payload_units(a, h);
    const uint4* src = (const uint4*)(a.store + h.base);
    if (gl < n16) v0 = src[gl];
    if (gl + G < n16) v1 = src[gl + G];
  }

  uint32_t cur = 0;
  for (uint64_t row = row0; row < a.n_ids; row += step, cur ^= 1u) {
    const bool has_next = row + step < a.n_ids;
    // 1. scan of the next tensor (its metadata was loaded an iteration ago)
    if (first_wave && has_next) scan_row(a, meta_next, gl, s_kc, &hdrs[cur ^ 1u], obufs + 64u * (cur ^ 1u));
    // 2. this payload -> LDS
    const GroupHdr h = hdrs[cur];
    {
      const uint32_t n16 = payload_units(a, h);
      if (gl < n16) pb128[gl] = v0;
      if (gl + G < n16) pb128[gl + G] = v1;
    }
    group_sync(single);
    // 3. metadata two and three tensors ahead, then the next payload, all
    //    before this tensor is decoded
    if (first_wave) {
      meta_next = load_meta(a, id_next2, gl);
      id_next2 = load_id(a, row + 3 * step);
    }
    if (has_next) {
      const GroupHdr hn = hdrs[cur ^ 1u];
      const uint32_t n16 = payload_units(a, hn);
      const uint4* src = (const uint4*)(a.store + hn.base);
      if (gl < n16) v0 = src[gl];
      if (gl + G < n16) v1 = src[gl + G];
    }
    // 4. decode this tensor's words and store them.  With chunks of at least
    //    64 words, the 64 words a wave handles for one j lie in one chunk, so
    //    the chunk, its participation and its offset are wave-uniform.
    const uint32_t* obuf = obufs + 64u * cur;
    uint32_t* orow = a.out + row * W;
    const uint32_t wave_w0 = uniform(gl) & ~(kWave - 1u);
    if (!uniform(h.valid)) {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const uint32_t w = gl + G * j;
        if (w < W) orow[w] = 0u;
      }
    } else {
      const uint32_t pmask_lo = uniform((uint32_t)h.pmask), pmask_hi = uniform((uint32_t)(h.pmask >> 32));
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const uint32_t w = gl + G * j;
        const uint32_t c = (wave_w0 + G * j) >> a.sh.wpc_log2;  // uniform
        if (c >= a.sh.n_c) continue;                            // whole wave past the end
        const uint32_t o = uniform(obuf[c]);
        const bool p = ((c < 32 ? pmask_lo >> c : pmask_hi >> (c - 32)) & 1u) != 0u;
        uint32_t v;
        if (p) {
          v = window32(pb32, o + (R.info[j] & 0xFFFFu));
          v = bfi_op(R.mask[j], R.bitval[j], unpack_stages(v, R.mv[j], R.stages[j]));
        } else {
          v = window32(pb32, o + (R.info[j] >> 16));
        }
        if (w < W) orow[w] = v;
      }
    }
    group_sync(single);
  }
}

// ---------------------------------------------------------------------------
// Tile kernel for small tensors (B <= 1 KB, so n_c <= 4 and W <= 256).
//
// With a whole group per small tensor, the per-tensor work (id, bitmap, scan,
// header, barriers) costs as many instructions as decoding it, and too few
// bytes are in flight per wave to cover HBM latency.  Here one wave takes T
// tensors at a time:
//   1. lane i < T computes tensor i's header (id, participation bits, chunk
//      offsets, payload length, offset) in one pass, so one wave instruction
//      serves T tensors;
//   2. the T payloads are loaded with all lanes busy: LPR = 64/RPI lanes per
//      tensor (RPI = 2 tensors per load instruction when a payload is at most
//      32 units of 16 B, else 1), every load issued before any is used;
//   3. lane l decodes words l + 64j of each of the T tensors, with the same
//      per-word registers for all of them (J = W/64 words per lane);
//   4. coalesced 4 B stores, 256 B per wave instruction.
// Waves are independent: only wave-level synchronisation inside the loop.

struct TileHdr {
  uint64_t base;
  uint32_t len;
  uint32_t pmask;
  uint32_t valid;
  uint32_t off[3];  // bit offsets of chunks 1..3 (chunk 0 starts at 0)
};

// Per-lane (lane i < T) metadata of tensor i of a tile, loaded ahead of use.
struct TileMeta {
  uint64_t base;
  uint32_t w0, w1;  // bitmap words holding the tensor's chunk bits
  uint32_t sh;      // bit position of chunk 0 in w0
  bool valid;
};

__device__ __forceinline__ TileMeta load_tile_meta(const GatherArgs& a, int64_t id) {
  TileMeta m;
  m.valid = id >= 0 && (uint64_t)id < a.n_tensors;
  m.base = 0;
  m.w0 = m.w1 = m.sh = 0;
  if (m.valid) {
    const uint64_t bit = (uint64_t)id * a.sh.n_c;
    m.sh = bit & 31;
    m.w0 = a.part_bits[bit >> 5];
    if (m.sh + a.sh.n_c > 32) m.w1 = a.part_bits[(bit >> 5) + 1];
    m.base = a.offsets ? a.offsets[id] : (uint64_t)id * a.slot_bytes;
  }
  return m;
}

__device__ __forceinline__ TileHdr make_tile_hdr(const GatherArgs& a, const TileMeta& m,
                                                 const uint32_t* s_kc) {
  TileHdr h;
  h.valid = m.valid;
  h.base = m.base;
  h.len = 0;
  h.pmask = 0;
  h.off[0] = h.off[1] = h.off[2] = 0;
  if (m.valid) {
    const uint32_t n_c = a.sh.n_c;
    const uint64_t word = (uint64_t)m.w0 | ((uint64_t)m.w1 << 32);
    const uint32_t pm = (uint32_t)(word >> m.sh) & ((1u << n_c) - 1u);
    uint32_t o = 0, offs[4];
#pragma unroll
    for (uint32_t c = 0; c < 4; ++c) {  // n_c <= 4; chunks past n_c add nothing
      offs[c] = o;
      if (c < n_c) o += ((pm >> c) & 1u) ? s_kc[c] : chunk_bits(a.sh, c);
    }
    h.off[0] = offs[1];
    h.off[1] = offs[2];
    h.off[2] = offs[3];
    h.pmask = pm;
    h.len = (o + 7u) >> 3;
  }
  return h;
}

template <int J, int T>
__global__ __launch_bounds__(256) void k_gather_tile(GatherArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const GatherLds L(a.sh.W, a.pbuf_bytes);  // pref/kc/wsum as the group kernel
  uint32_t* s_pref = (uint32_t*)(smem + L.pref);
  uint32_t* s_kc = (uint32_t*)(smem + L.kc);
  uint32_t* s_wsum = (uint32_t*)(smem + L.wsum);
  const uint32_t wave = threadIdx.x / kWave;
  const uint32_t lane = threadIdx.x % kWave;
  uint8_t* wbase = smem + L.group0 + wave * (2 * T * (uint32_t)sizeof(TileHdr) + T * a.pbuf_bytes);
  TileHdr* hdrs = (TileHdr*)wbase;  // [2][T]
  uint8_t* pbufs = wbase + 2 * T * sizeof(TileHdr);

  const uint32_t W = a.sh.W;
  const uint32_t lpr = a.lpr;  // lanes per tensor in the load phase
  const uint32_t rpi = kWave / lpr;
  const uint64_t n_tiles = (a.n_ids + T - 1) / T;
  const uint64_t waves = (uint64_t)gridDim.x * (blockDim.x / kWave);
  const uint64_t tile0 = (uint64_t)blockIdx.x * (blockDim.x / kWave) + wave;
  const bool meta_lane = lane < (uint32_t)T;
  auto row_id = [&](uint64_t tile) -> int64_t {
    const uint64_t row = tile * T + lane;
    return (meta_lane && tile < n_tiles && row < a.n_ids) ? a.ids[row] : -1;
  };

  // Tile metadata runs ahead of the payloads (vector loads retire in issue
  // order): ids three tiles ahead, bitmap words and offsets two ahead, the
  // headers one ahead.
  const int64_t id_a = row_id(tile0), id_b = row_id(tile0 + waves);

  WordRegs<J> R;
  load_plan<J>(a.mask, a.bitval, a.sh, s_pref, s_kc, s_wsum, lane, R);
  if (tile0 >= n_tiles) return;  // per wave; no workgroup barrier follows

  TileMeta meta_next = load_tile_meta(a, id_b);
  {
    const TileMeta m0 = load_tile_meta(a, id_a);
    if (meta_lane) hdrs[lane] = make_tile_hdr(a, m0, s_kc);
  }
  int64_t id_next2 = row_id(tile0 + 2 * waves);
  wave_sync();

  uint4 v[T];
  uint32_t n16s[T];
  auto issue_loads = [&](const TileHdr* hdr) {
#pragma unroll
    for (int k = 0; k < T; ++k) {
      n16s[k] = 0;
      v[k] = make_uint4(0, 0, 0, 0);
      if ((uint32_t)k * rpi >= (uint32_t)T) continue;
      const uint32_t i = k * rpi + lane / lpr;
      const uint32_t u = lane % lpr;
      const TileHdr& h = hdr[i];
      uint32_t n16 = 0;
      if (h.valid) {
        const uint64_t avail = h.base < a.store_bytes ? (a.store_bytes - h.base) & ~15ull : 0ull;
        n16 = (uint32_t)(min((uint64_t)((h.len + 15u) & ~15u), avail) >> 4);
      }
      n16s[k] = n16;
      if (u < n16) v[k] = ((const uint4*)(a.store + h.base))[u];
    }
  };
  issue_loads(hdrs);

  uint32_t cur = 0;
  for (uint64_t tile = tile0; tile < n_tiles; tile += waves, cur ^= 1u) {
    const bool has_next = tile + waves < n_tiles;
    TileHdr* hcur = hdrs + cur * T;
    TileHdr* hnext = hdrs + (cur ^ 1u) * T;
    // a. this tile's payloads -> LDS
#pragma unroll
    for (int k = 0; k < T; ++k) {
      if ((uint32_t)k * rpi >= (uint32_t)T) continue;
      const uint32_t i = k * rpi + lane / lpr;
      const uint32_t u = lane % lpr;
      if (u < n16s[k]) ((uint4*)(pbufs + i * a.pbuf_bytes))[u] = v[k];
    }
    // b. next tile's headers (metadata loaded an iteration ago)
    if (has_next && meta_lane) hnext[lane] = make_tile_hdr(a, meta_next, s_kc);
    wave_sync();
    // c. metadata two and three tiles ahead, d. next tile's payload loads
    meta_next = load_tile_meta(a, id_next2);
    id_next2 = row_id(tile + 3 * waves);
    if (has_next) issue_loads(hnext);
    // e. decode this tile and store it.  Chunks hold at least 64 words, so
    //    the 64 words lane l handles for one j lie in one chunk: chunk,
    //    participation and offset are wave-uniform.
    const uint64_t row0 = tile * T;
    for (int i = 0; i < T; ++i) {
      const uint64_t row = row0 + i;
      if (row >= a.n_ids) break;
      const TileHdr* hp = hcur + i;
      uint32_t* orow = a.out + row * W;
      if (!uniform(hp->valid)) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
          const uint32_t w = lane + kWave * j;
          if (w < W) orow[w] = 0u;
        }
        continue;
      }
      const uint32_t pm = uniform(hp->pmask);
      const uint32_t o1 = uniform(hp->off[0]), o2 = uniform(hp->off[1]), o3 = uniform(hp->off[2]);
      const uint32_t* pb32 = (const uint32_t*)(pbufs + i * a.pbuf_bytes);
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const uint32_t w = lane + kWave * j;
        const uint32_t c = (kWave * j) >> a.sh.wpc_log2;  // uniform
        const uint32_t o = c == 0 ? 0u : c == 1 ? o1 : c == 2 ? o2 : o3;
        uint32_t v;
        if ((pm >> c) & 1u) {
          v = window32(pb32, o + (R.info[j] & 0xFFFFu));
          v = bfi_op(R.mask[j], R.bitval[j], unpack_stages(v, R.mv[j], R.stages[j]));
        } else {
          v = window32(pb32, o + (R.info[j] >> 16));
        }
        if (w < W) orow[w] = v;
      }
    }
    wave_sync();
  }
}

template <int J, int T>
static hipError_t launch_tile(const Geometry& g, GatherArgs a, hipStream_t s) {
  // lanes per tensor in the load phase: the payload's 16 B units, rounded up
  // to a power of two, at most 64
  const uint32_t units = ((g.tensor_bytes + 15u) & ~15u) / 16u;
  uint32_t lpr = 64;
  while (lpr / 2 >= units && lpr > 16) lpr /= 2;
  a.lpr = lpr;
  a.sh.group = kWave;  // lane l owns words l + 64j
  const uint32_t waves = 4;
  const GatherLds L(g.W, a.pbuf_bytes);
  const uint32_t lds = L.group0 + waves * (2 * T * (uint32_t)sizeof(TileHdr) + T * a.pbuf_bytes);
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_gather_tile<J, T>, waves * 64, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  const uint64_t tiles = (a.n_ids + T - 1) / T;
  const uint64_t want = (tiles + waves - 1) / waves;
  const uint64_t cap = (uint64_t)per_cu * (uint64_t)di.cus;
  const uint32_t blocks = (uint32_t)(want < cap ? want : cap);
  hipLaunchKernelGGL((k_gather_tile<J, T>), dim3(blocks), dim3(waves * 64), lds, s, a);
  return hipGetLastError();
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
  a.lpr = 0;
  if (g.W <= 4 * (uint32_t)kWave) {
    // small tensors: tile kernel, lane l owns words l + 64j
    const uint32_t J = (g.W + kWave - 1) / kWave;
    const bool t8 = g.tensor_bytes <= 512;
    switch (J * 2 + (t8 ? 1 : 0)) {
      case 3: return launch_tile<1, 8>(g, a, s);
      case 5: return launch_tile<2, 8>(g, a, s);
      case 6: return launch_tile<3, 4>(g, a, s);
      case 8: return launch_tile<4, 4>(g, a, s);
      default: return hipErrorInvalidValue;
    }
  }
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

}  // namespace ibp
