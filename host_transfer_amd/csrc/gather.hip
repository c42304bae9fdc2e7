// gather.hip -- batched gather + decompress of IBP tensors (the critical path).
//
// [G-EN] Core Algorithm, Decompression: one warp per tensor, the compressed
// segment staged in shared memory, a warp scan for each thread's chunk start,
// then every thread re-inserts the invariant bits on its own, with fetches
// overlapped with decoding.  [JH] decompression paragraph: one thread per
// chunk, no cross-warp synchronisation; transfer paragraph: GPU-initiated
// 128 B-aligned reads of host memory.
//
// On gfx950 there are two kernels, chosen by the tensor size W (words):
//
// k_gather_decompress (W > 256): a group of G = 64..1024 threads (one or more
// wave64s, G the smallest with W <= 6 G) handles one tensor at a time:
//   1. the first wave reads the tensor's participation bits (lane c owns
//      chunk c, n_c <= 64); a wave scan gives each chunk's bit offset in the
//      payload and the payload length;
//   2. the group loads the payload (whole 16 B units from a 16 B-aligned
//      start, so every 128 B line is read once) from the host-mapped slot or
//      the HBM cache into registers, then LDS;
//   3. each thread decodes its own words: a 64-bit window of the payload at
//      the word's bit offset (two LDS words and v_alignbit), unpack with the
//      word's move masks, insert Bitval; raw chunks take the window as is;
//   4. coalesced streaming stores of the dense row.
// Software pipeline per group: while tensor i is decoded, the payload loads of
// tensor i+1 are in flight, and the ids and participation words of tensors
// i+2 and i+3 are loaded ahead.  A payload is at most B <= 24*G bytes, so it
// fits in two 16 B registers per thread.  Workgroup barriers only wait for
// LDS traffic, so global loads stay in flight across them.
//
// k_gather_tile (W <= 256): one wave decodes a tile of T small tensors at a
// time (see its comment), with the same pipeline across tiles.
// k_gather_direct: short batches of such tensors held in an HBM cache, read
// in place without staging (see its comment).
// One-chunk tensors of 64, 128 or 256 words held in an HBM cache take
// k_gather_cache (gather_cache.hip) instead.
//
// Both have a routed variant (k_gather_decompress_routed, k_gather_tile_routed)
// that sends every row to the XCD its tensor hashes to, for batches that
// repeat ids (see k_gather_tile_routed).
#include "ibp_internal.h"
#include "ibp_plan.h"

namespace ibp {

// Where payloads are read from.  A tensor whose offset-table entry is not
// kNotCached is read from the compacted cache at that offset; any other
// tensor from its slot of the in-place store.  Slot mode: no offset table;
// cache mode: no store; hybrid: both.
struct GatherArgs {
  const uint8_t* store;     // in-place store (slot t at t*slot_bytes), or null
  uint64_t store_bytes;
  uint64_t slot_bytes;
  const uint64_t* offsets;  // cache entry per tensor, or null
  const uint8_t* cache;     // compacted cache, or null
  uint64_t cache_bytes;
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
  uint32_t route;       // route ids to XCDs (slot mode only)
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

// 16 zero bytes in device memory: lanes with nothing to load read this
// instead of skipping the load, so every wave issues the same number of
// vector memory operations on every path and the compiler's in-order wait
// counts stay exact (a skipped load would force waits for everything in
// flight, stores and prefetches included).
__device__ __align__(16) uint4 g_zero16 = {0u, 0u, 0u, 0u};

constexpr uint64_t kNotCached = ~0ull;

// Output rows are written once and not read again by the kernel: streaming
// (non-temporal) stores keep them from displacing the payloads, offsets and
// bitmap words that repeated ids read again.
__device__ __forceinline__ void store_out(uint32_t* p, uint32_t v) {
  __builtin_nontemporal_store(v, p);
}


// Address of tensor t's payload and the bytes readable from there (0 when it
// has no source).  One unconditional load of the offset table entry.
struct Source {
  uint64_t addr;
  uint64_t avail;
  bool ok;
};

// Marks the stage flags as redefined at the top of every loop iteration, so
// the compiler tests their bits in place (one scalar register per word
// position) rather than hoisting one 64-bit lane mask per stage out of the
// loop, which overflows the scalar registers into spills.
template <int J>
__device__ __forceinline__ void keep_stage_flags(WordRegs<J>& R) {
#pragma unroll
  for (int j = 0; j < J; ++j) asm volatile("" : "+s"(R.stages[j]));
}

// The same for the shape fields: the few scalar instructions that derive
// per-chunk values from them are cheaper inside the loop than the registers
// (and spills) that hoisting every derived value costs.
__device__ __forceinline__ void keep_shape(GatherArgs& a) {
  asm volatile("" : "+s"(a.sh.n_c), "+s"(a.sh.wpc_log2), "+s"(a.sh.last_bits));
}

// The offset-table entry of tensor t as loaded (zero without a table; the
// load is unconditional, see g_zero16).  It is resolved by source_of one
// pipeline step later, so no wait for it sits in front of the loads issued
// after it.
__device__ __forceinline__ uint64_t load_offset(const GatherArgs& a, uint64_t t) {
  return load_global(a.offsets ? a.offsets + t : (const uint64_t*)&g_zero16);
}

// Where tensor t's payload is: its cache entry when the table has one, else
// its slot; avail bounds every read there.
__device__ __forceinline__ Source source_of(const GatherArgs& a, uint64_t t, uint64_t o) {
  const bool hit = a.offsets != nullptr && o != kNotCached;
  const uint64_t so = t * a.slot_bytes;
  const uint64_t at = hit ? o : so;
  const uint64_t lim = hit ? a.cache_bytes : a.store_bytes;
  Source r;
  r.addr = hit ? (uint64_t)a.cache + o : (uint64_t)a.store + so;
  r.avail = at < lim ? (lim - at) & ~15ull : 0ull;
  r.ok = hit || a.store != nullptr;
  return r;
}

// One tensor's metadata as loaded, before its payload is read (consumed by
// scan_row one pipeline step later).
struct RowMeta {
  uint64_t t;     // tensor index (0 for an invalid id)
  uint64_t o;     // offset-table entry
  uint32_t word;  // participation word holding this lane's chunk bit
  uint32_t sh;    // position of that bit in it
  bool valid;     // id in range
};

// The id of row `row`, or -1 past the batch.  The load itself is
// unconditional (clamped row): see g_zero16.
__device__ __forceinline__ int64_t load_id(const GatherArgs& a, uint64_t row) {
  const int64_t id = a.ids[row < a.n_ids ? row : a.n_ids - 1];
  return row < a.n_ids ? id : -1;
}

// Participation word and offset entry of tensor `id` (lane c: chunk c).
// Unconditional loads: an invalid id reads tensor 0's entries, ignored later.
__device__ __forceinline__ RowMeta load_meta(const GatherArgs& a, int64_t id, uint32_t lane) {
  RowMeta m;
  m.valid = id >= 0 && (uint64_t)id < a.n_tensors;
  m.t = m.valid ? (uint64_t)id : 0ull;
  const uint32_t c = min(lane % kWave, a.sh.n_c - 1u);
  const uint64_t bit = m.t * a.sh.n_c + c;
  m.word = a.part_bits[bit >> 5];
  m.sh = (uint32_t)(bit & 31);
  m.o = load_offset(a, m.t);
  return m;
}

// Participation, chunk offsets and payload length of one tensor (first wave).
__device__ __forceinline__ void scan_row(const GatherArgs& a, const RowMeta& m, uint32_t lane,
                                         const uint32_t* s_kc, GroupHdr* hdr, uint32_t* obuf) {
  const Source src = source_of(a, m.t, m.o);
  const bool valid = m.valid && src.ok;
  const bool p = valid && lane < a.sh.n_c && ((m.word >> m.sh) & 1u);
  const uint32_t size = !valid || lane >= a.sh.n_c ? 0u : (p ? s_kc[lane] : chunk_bits(a.sh, lane));
  const uint32_t incl = wave_inclusive_sum(size);
  if (lane < a.sh.n_c) obuf[lane] = incl - size;
  const uint64_t pm = __ballot(p);
  const uint32_t total = __shfl(incl, kWave - 1, kWave);
  if (lane == 0) {
    hdr->pmask = pm;
    hdr->valid = valid;
    hdr->len = (total + 7u) >> 3;
    hdr->addr = src.addr;
    hdr->avail = src.avail;
  }
}

// Number of 16 B payload units to read: the payload rounded up to 16 B,
// never past the end of its store or cache.
__device__ __forceinline__ uint32_t payload_units(const GatherArgs& a, const GroupHdr& h) {
  if (!h.valid) return 0;
  const uint32_t want = (h.len + 15u) & ~15u;
  return (uint32_t)(min((uint64_t)want, h.avail) >> 4);
}

// Decodes one tensor staged in LDS (pb32) and stores its words: thread gl
// owns words gl + G j.  With chunks of at least 64 words, the 64 words a wave
// handles for one j lie in one chunk, so the chunk, its participation and its
// offset (obuf, from the chunk scan) are wave-uniform.
template <int J>
__device__ __forceinline__ void decode_group_tensor(const GatherArgs& a, const WordRegs<J>& R,
                                                    const GroupHdr& h, const uint32_t* obuf,
                                                    const uint32_t* pb32, uint32_t gl, uint32_t G,
                                                    uint32_t* orow) {
  const uint32_t W = a.sh.W;
  const uint32_t wave_w0 = uniform(gl) & ~(kWave - 1u);
  if (!uniform(h.valid)) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint32_t w = gl + G * j;
      if (w < W) store_out(orow + w, 0u);
    }
    return;
  }
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
    if (w < W) store_out(orow + w, v);
  }
}

// The body of the group kernel for workgroup `block` of `blocks` (the whole
// grid, or the workgroups of one segment of k_gather_decompress_seg).
template <int J>
__device__ __forceinline__ void gather_group_body(GatherArgs& a, uint32_t block, uint32_t blocks) {
  extern __shared__ __align__(16) uint8_t smem[];
  const GatherLds L(a.sh.W, a.pbuf_bytes);
  uint32_t* s_pref = (uint32_t*)(smem + L.pref);
  uint32_t* s_kc = (uint32_t*)(smem + L.kc);
  uint32_t* s_wsum = (uint32_t*)(smem + L.wsum);

  const uint32_t G = a.sh.group;
  const uint32_t g = uniform(threadIdx.x / G);  // G >= 64: one group per wave or more
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
  const uint64_t step = (uint64_t)blocks * a.groups;
  const uint64_t row0 = (uint64_t)block * a.groups + g;

  // Metadata runs ahead of the payloads so that no wait for it also waits
  // for a payload still in flight (vector loads retire in issue order):
  // ids three tensors ahead, participation words and offsets two ahead, the
  // scan one ahead.
  // (every wave loads the few metadata bytes, so no load sits behind a
  // branch; only the first wave uses them)
  // the first two tensors' metadata round trips overlap the chunk counts;
  // the first payload is requested before the per-word registers are built,
  // so its fetch overlaps that arithmetic
  const int64_t id_a = load_id(a, row0);
  const int64_t id_b = load_id(a, row0 + step);
  int64_t id_next2 = load_id(a, row0 + 2 * step);  // tensor row+2*step
  PlanRun run;
  load_plan_run(a.mask, a.sh, run);
  WordRegs<J> R;
  load_plan_fetch<J>(a.mask, a.bitval, a.sh, gl, R);
  const RowMeta m0 = load_meta(a, id_a, gl);
  RowMeta meta_next = load_meta(a, id_b, gl);      // tensor row+step

  load_plan_counts(run, a.sh, s_pref, s_kc, s_wsum);

  if (row0 >= a.n_ids) return;  // uniform per group; no workgroup barrier follows for it

  // The first tensor's payload is at least ceil(K / 8) bytes (K = kept bits
  // of the Mask: every chunk packed), so in slot mode its first ceil(K / 128)
  // units are requested as soon as its id is known, before its participation
  // word and chunk scan; the rest follows the scan.
  uint32_t spec = 0;
  uint4 s0, s1;
  {
    const uint64_t so = m0.t * a.slot_bytes;
    const uint64_t avail = so < a.store_bytes ? (a.store_bytes - so) >> 4 : 0ull;
    if (a.offsets == nullptr && a.store != nullptr && m0.valid)
      spec = (uint32_t)min((uint64_t)((s_pref[W] + 127u) >> 7), avail);
    const uint4* src = (const uint4*)((const uint8_t*)a.store + so);
    s0 = load_global(gl < spec ? src + gl : &g_zero16);
    s1 = load_global(gl + G < spec ? src + gl + G : &g_zero16);
  }
  if (first_wave) scan_row(a, m0, gl, s_kc, &hdrs[0], obufs);
  group_sync(single);

  // payload registers of the tensor in flight; lanes past the payload read
  // g_zero16 rather than skip the load (exact wait counts, see g_zero16)
  uint4 v0, v1;
  {
    const GroupHdr h = hdrs[0];
    const uint32_t n16 = payload_units(a, h);
    const uint4* src = (const uint4*)h.addr;
    v0 = load_global(gl < n16 && gl >= spec ? src + gl : &g_zero16);
    v1 = load_global(gl + G < n16 && gl + G >= spec ? src + gl + G : &g_zero16);
  }

  load_plan_words<J>(a.sh, s_pref, gl, R);
  if (gl < spec) v0 = s0;
  if (gl + G < spec) v1 = s1;

  uint32_t cur = 0;
  for (uint64_t row = row0; row < a.n_ids; row += step, cur ^= 1u) {
    const bool has_next = row + step < a.n_ids;
    keep_stage_flags<J>(R);
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
    meta_next = load_meta(a, id_next2, gl);
    id_next2 = load_id(a, row + 3 * step);
    {
      const GroupHdr hn = hdrs[cur ^ 1u];
      const uint32_t n16 = has_next ? payload_units(a, hn) : 0u;
      const uint4* src = (const uint4*)hn.addr;
      v0 = load_global(gl < n16 ? src + gl : &g_zero16);
      v1 = load_global(gl + G < n16 ? src + gl + G : &g_zero16);
    }
    // 4. decode this tensor's words and store them
    decode_group_tensor<J>(a, R, h, obufs + 64u * cur, pb32, gl, G, a.out + row * W);
    group_sync(single);
  }
}

template <int J>
__global__ __launch_bounds__(1024) void k_gather_decompress(GatherArgs a) {
  gather_group_body<J>(a, blockIdx.x, gridDim.x);
}

// Several gathers of one tensor shape in one launch, each segment with its
// own Mask/Bitval (the K/V decode step: one segment per (layer, K|V) pair).
// Segment s is ids [off[s], off[s+1]) -> out rows [off[s], off[s+1]), with
// the Mask and Bitval words at s * W.  The grid is n_seg * per_seg
// workgroups; workgroup b serves segment b / per_seg as workgroup
// b % per_seg of per_seg, so it builds that segment's plan once, and the
// launch pays its fixed cost once for all segments.
struct SegTable {
  uint64_t off[kMaxSegments + 1];
  uint32_t n_seg;
  uint32_t per_seg;
};

// The arguments of the segment that this workgroup serves (segment
// blockIdx.x / per_seg; the grid is n_seg * per_seg); false when it is empty.
__device__ __forceinline__ bool segment_args(const GatherArgs& a, const SegTable& t,
                                             GatherArgs& b) {
  const uint32_t seg = blockIdx.x / t.per_seg;
  const uint64_t o = t.off[seg], n = t.off[seg + 1] - o;
  b = a;
  b.ids = a.ids + o;
  b.n_ids = n;
  b.out = a.out + o * a.sh.W;
  b.mask = a.mask + (uint64_t)seg * a.sh.W;
  b.bitval = a.bitval + (uint64_t)seg * a.sh.W;
  return n != 0;
}

template <int J>
__global__ __launch_bounds__(1024) void k_gather_decompress_seg(GatherArgs a, SegTable t) {
  GatherArgs b;
  if (!segment_args(a, t, b)) return;  // the whole workgroup, before any barrier
  gather_group_body<J>(b, blockIdx.x % t.per_seg, t.per_seg);
}

// Group kernel with XCD-aware routing (see k_gather_tile_routed), for
// payloads read from their slots, one group per workgroup.  The group's first
// wave scans its segment of the batch a window of 64 ids at a time and lists
// the rows whose tensor hashes to this XCD; the group decodes the listed rows
// in order with a one-deep pipeline: the next tensor's chunk scan and payload
// loads are issued before the current tensor is decoded, and the metadata of
// the one after that before those.
__host__ __device__ constexpr uint32_t routed_group_list_bytes() {
  return (uint32_t)kWave * 12u + 16u;  // ids, rows, count
}

// Workgroup `block` of `blocks` (a multiple of 8) must run on XCD block % 8:
// the whole grid, or one segment of k_gather_decompress_routed_seg whose
// per_seg is a multiple of 8.
template <int J>
__device__ __forceinline__ void gather_group_routed_body(GatherArgs& a, uint32_t block,
                                                         uint32_t blocks) {
  extern __shared__ __align__(16) uint8_t smem[];
  const GatherLds L(a.sh.W, a.pbuf_bytes);
  uint32_t* s_pref = (uint32_t*)(smem + L.pref);
  uint32_t* s_kc = (uint32_t*)(smem + L.kc);
  uint32_t* s_wsum = (uint32_t*)(smem + L.wsum);
  const uint32_t G = blockDim.x;  // one group per workgroup
  const uint32_t gl = threadIdx.x;
  uint8_t* gbase = smem + L.group0;
  GroupHdr* hdrs = (GroupHdr*)gbase;                            // [2]
  uint32_t* obufs = (uint32_t*)(gbase + 2 * sizeof(GroupHdr));  // [2][64]
  uint8_t* pbuf = gbase + 2 * sizeof(GroupHdr) + 512;
  const uint32_t* pb32 = (const uint32_t*)pbuf;
  uint4* pb128 = (uint4*)pbuf;
  int64_t* list_id = (int64_t*)(smem + L.total(1));  // [64]
  uint32_t* list_row = (uint32_t*)(list_id + kWave);  // [64]
  uint32_t* s_n = list_row + kWave;                   // [1]
  const bool first_wave = gl < kWave;
  const uint32_t W = a.sh.W;

  const uint32_t xcd = block % kXcds;
  const uint64_t wc = blocks / kXcds;
  const uint64_t wk = block / kXcds;
  const uint64_t seg = (a.n_ids + wc - 1) / wc;
  const uint64_t s0 = min(wk * seg, a.n_ids), s1 = min(s0 + seg, a.n_ids);

  PlanRun run;
  load_plan_run(a.mask, a.sh, run);
  WordRegs<J> R;
  load_plan_fetch<J>(a.mask, a.bitval, a.sh, gl, R);
  const int64_t win_id = a.ids[min(s0 + gl % kWave, a.n_ids - 1)];
  load_plan_counts(run, a.sh, s_pref, s_kc, s_wsum);  // workgroup barriers
  if (s0 >= s1) return;                               // the whole workgroup

  bool planned = false;
  for (uint64_t base = s0; base < s1; base += kWave) {
    if (first_wave) {
      const uint64_t r = base + gl;
      const bool in = r < s1;
      const int64_t id = base == s0 ? win_id : a.ids[in ? r : s1 - 1];
      const bool mine = in && xcd_of_tensor(id) == xcd;
      const uint64_t bal = __ballot(mine);
      const uint32_t before = (uint32_t)__popcll(bal & ((1ull << gl) - 1ull));
      if (mine) {
        list_id[before] = id;
        list_row[before] = (uint32_t)r;
      }
      if (gl == 0) s_n[0] = (uint32_t)__popcll(bal);
    }
    __syncthreads();
    const uint32_t n = s_n[0];
    if (n != 0u) {
      // prologue: the first listed tensor's scan and payload, the second's metadata
      {
        const RowMeta m = load_meta(a, list_id[0], gl);
        if (first_wave) scan_row(a, m, gl, s_kc, &hdrs[0], obufs);
      }
      __syncthreads();
      uint4 v0, v1;
      {
        const GroupHdr h = hdrs[0];
        const uint32_t n16 = payload_units(a, h);
        const uint4* src = (const uint4*)h.addr;
        v0 = load_global(gl < n16 ? src + gl : &g_zero16);
        v1 = load_global(gl + G < n16 ? src + gl + G : &g_zero16);
      }
      RowMeta meta_next = load_meta(a, list_id[min(1u, n - 1u)], gl);
      if (!planned) {
        load_plan_words<J>(a.sh, s_pref, gl, R);
        planned = true;
      }
      for (uint32_t k = 0; k < n; ++k) {
        const uint32_t cur = k & 1u;
        const bool has_next = k + 1u < n;
        // 1. this payload -> LDS; the next tensor's scan
        const GroupHdr h = hdrs[cur];
        {
          const uint32_t n16 = payload_units(a, h);
          if (gl < n16) pb128[gl] = v0;
          if (gl + G < n16) pb128[gl + G] = v1;
        }
        if (first_wave && has_next)
          scan_row(a, meta_next, gl, s_kc, &hdrs[cur ^ 1u], obufs + 64u * (cur ^ 1u));
        __syncthreads();
        // 2. the next payload and the metadata after it, before this decode
        {
          const GroupHdr hn = hdrs[cur ^ 1u];
          const uint32_t n16 = has_next ? payload_units(a, hn) : 0u;
          const uint4* src = (const uint4*)hn.addr;
          v0 = load_global(gl < n16 ? src + gl : &g_zero16);
          v1 = load_global(gl + G < n16 ? src + gl + G : &g_zero16);
        }
        meta_next = load_meta(a, list_id[min(k + 2u, n - 1u)], gl);
        // 3. decode and store this tensor
        decode_group_tensor<J>(a, R, h, obufs + 64u * cur, pb32, gl, G,
                               a.out + (uint64_t)list_row[k] * W);
        __syncthreads();
      }
    }
    __syncthreads();  // the list and its count are rewritten by the next window
  }
}

template <int J>
__global__ __launch_bounds__(1024) void k_gather_decompress_routed(GatherArgs a) {
  gather_group_routed_body<J>(a, blockIdx.x, gridDim.x);
}

// Routed, over segments: per_seg is a multiple of 8, so a segment's workgroup
// k runs on XCD k % 8.
template <int J>
__global__ __launch_bounds__(1024) void k_gather_decompress_routed_seg(GatherArgs a, SegTable t) {
  GatherArgs b;
  if (!segment_args(a, t, b)) return;  // the whole workgroup, before any barrier
  gather_group_routed_body<J>(b, blockIdx.x % t.per_seg, t.per_seg);
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
  uint64_t addr;    // payload address
  uint32_t n16;     // 16 B units to read
  uint32_t pmask;
  uint32_t valid;
  uint32_t off[3];  // bit offsets of chunks 1..3 (chunk 0 starts at 0)
};

// Per-lane metadata of tensor (lane % T) of a tile, loaded ahead of use.
// Every lane loads (lanes >= T duplicate lane % T) and ids are clamped into
// range, so the loads are unconditional.
struct TileMeta {
  uint64_t t;       // tensor index (0 for an invalid id)
  uint64_t o;       // offset-table entry as loaded
  uint32_t w0, w1;  // bitmap words holding the tensor's chunk bits
  uint32_t sh;      // bit position of chunk 0 in w0
  bool valid;       // id in range
};

__device__ __forceinline__ int64_t tile_row_id(const GatherArgs& a, uint64_t row) {
  return a.ids[row < a.n_ids ? row : a.n_ids - 1];
}

__device__ __forceinline__ TileMeta load_tile_meta(const GatherArgs& a, int64_t id) {
  TileMeta m;
  m.valid = id >= 0 && (uint64_t)id < a.n_tensors;
  m.t = m.valid ? (uint64_t)id : 0ull;
  const uint64_t bit = m.t * a.sh.n_c;
  const uint64_t q = bit >> 5;
  const uint64_t last_word = (a.n_tensors * a.sh.n_c - 1) >> 5;
  m.sh = bit & 31;
  m.w0 = a.part_bits[q];
  m.w1 = a.part_bits[q < last_word ? q + 1 : q];
  m.o = load_offset(a, m.t);
  return m;
}

__device__ __forceinline__ TileHdr make_tile_hdr(const GatherArgs& a, const TileMeta& m,
                                                 const uint32_t* s_kc) {
  TileHdr h;
  const Source src = source_of(a, m.t, m.o);
  const bool valid = m.valid && src.ok;
  h.valid = valid;
  h.addr = src.addr;
  const uint32_t n_c = a.sh.n_c;
  const uint64_t word = (uint64_t)m.w0 | ((uint64_t)m.w1 << 32);
  const uint32_t pm = valid ? (uint32_t)(word >> m.sh) & ((1u << n_c) - 1u) : 0u;
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
  // 16 B units: the payload rounded up to 16 B, never past the end of its
  // store or cache
  const uint32_t len = valid ? (o + 7u) >> 3 : 0u;
  h.n16 = (uint32_t)(min((uint64_t)((len + 15u) & ~15u), src.avail) >> 4);
  return h;
}

// Decodes word j of one tensor of a tile (chunk, participation and offset
// wave-uniform, see below).
template <int J>
__device__ __forceinline__ uint32_t tile_word(const GatherArgs& a, const WordRegs<J>& R, int j,
                                              const uint32_t* pb32, uint32_t pm, uint32_t o1,
                                              uint32_t o2, uint32_t o3) {
  const uint32_t c = ((uint32_t)kWave * j) >> a.sh.wpc_log2;  // uniform
  const uint32_t o = c == 0 ? 0u : c == 1 ? o1 : c == 2 ? o2 : o3;
  uint32_t v;
  if ((pm >> c) & 1u) {
    v = window32(pb32, o + (R.info[j] & 0xFFFFu));
    v = bfi_op(R.mask[j], R.bitval[j], unpack_stages(v, R.mv[j], R.stages[j]));
  } else {
    v = window32(pb32, o + (R.info[j] >> 16));
  }
  return v;
}

// Unpack stages applied to N words of one word position at once: the stage
// tests are made once for all of them.
template <int N>
__device__ __forceinline__ void unpack_stages_n(uint32_t (&x)[N], const uint32_t mv[5],
                                                uint32_t stages) {
  if (stages & 16u) {
#pragma unroll
    for (int q = 0; q < N; ++q) x[q] = bfi_op(mv[4], x[q] << 16, x[q]);
  }
  if (stages & 8u) {
#pragma unroll
    for (int q = 0; q < N; ++q) x[q] = bfi_op(mv[3], x[q] << 8, x[q]);
  }
  if (stages & 4u) {
#pragma unroll
    for (int q = 0; q < N; ++q) x[q] = bfi_op(mv[2], x[q] << 4, x[q]);
  }
  if (stages & 2u) {
#pragma unroll
    for (int q = 0; q < N; ++q) x[q] = bfi_op(mv[1], x[q] << 2, x[q]);
  }
  if (stages & 1u) {
#pragma unroll
    for (int q = 0; q < N; ++q) x[q] = bfi_op(mv[0], x[q] << 1, x[q]);
  }
}

#ifndef IBP_TILE_GROUP
#define IBP_TILE_GROUP 8  // tensors of a full tile decoded side by side (4 when J >= 4)
#endif
#ifndef IBP_DIRECT_TG
#define IBP_DIRECT_TG 8   // tensors per tile of k_gather_direct (half when J >= 3)
#endif
#ifndef IBP_BIG_NL
#define IBP_BIG_NL 8      // load instructions per tile on large batches
#endif

// Decodes and stores one full tile (W == 64 J) held in LDS.  Word position
// j = the words lane + 64 j of every tensor: its chunk c_j is the same for
// all lanes and tensors, so per tensor only the chunk's bit offset (read
// across lanes from the header lane) and its participation bit (one ballot
// per tile and j) vary.  Up to 16 tensors are decoded side by side, so their
// LDS reads overlap and the stage tests are made once for all of them.
// Invalid tensors have no participating chunk and an all-zero slot, so they
// decode to zero words without a select.
// ROUTED: tensor i's output row is held by lane i (trow); else it is row0 + i.
template <int J, int T, bool ROUTED = false>
__device__ __forceinline__ void decode_full_tile(const GatherArgs& a, const WordRegs<J>& R,
                                                 const uint8_t* pbufs, const TileHdr* hcur,
                                                 uint32_t lane, uint64_t row0, uint32_t trow = 0) {
  constexpr uint32_t kW = (uint32_t)kWave * J;  // words per tensor
  constexpr uint32_t kSlot = 4u * kW + 16u;     // LDS bytes per tensor
  constexpr int TGmax = J >= 4 && IBP_TILE_GROUP > 4 ? 4 : IBP_TILE_GROUP;  // registers of J words
  constexpr int TG = T < TGmax ? T : TGmax;  // tensors decoded side by side
  const TileHdr& hl = hcur[lane & (uint32_t)(T - 1)];
  const uint32_t hpm = hl.pmask, ho1 = hl.off[0], ho2 = hl.off[1], ho3 = hl.off[2];
  uint32_t* obase = a.out + row0 * kW + lane;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const uint32_t c = uniform(((uint32_t)kWave * j) >> a.sh.wpc_log2);
    const uint32_t oj = c == 0 ? 0u : c == 1 ? ho1 : c == 2 ? ho2 : ho3;
    const uint32_t pbits = (uint32_t)__builtin_amdgcn_ballot_w64(((hpm >> c) & 1u) != 0u);
    const uint32_t lo = R.info[j] & 0xFFFFu, hi = R.info[j] >> 16;
#pragma unroll
    for (int i0 = 0; i0 < T; i0 += TG) {
      uint32_t x[TG];
#pragma unroll
      for (int q = 0; q < TG; ++q) {
        const int i = i0 + q;
        const uint32_t o = __builtin_amdgcn_readlane(oj, i);
        const uint32_t* pb32 = (const uint32_t*)(pbufs + i * kSlot);
        x[q] = window32(pb32, o + (((pbits >> i) & 1u) ? lo : hi));
      }
      constexpr uint32_t gmask = TG == 32 ? ~0u : (1u << TG) - 1u;
      const uint32_t gp = (pbits >> i0) & gmask;
      if (gp == gmask) {  // every tensor of the group keeps chunk c packed
        unpack_stages_n<TG>(x, R.mv[j], R.stages[j]);
#pragma unroll
        for (int q = 0; q < TG; ++q) x[q] = bfi_op(R.mask[j], R.bitval[j], x[q]);
      } else if (gp != 0u) {  // some tensors store chunk c whole: one at a time
#pragma unroll
        for (int q = 0; q < TG; ++q)
          if ((gp >> q) & 1u)
            x[q] = bfi_op(R.mask[j], R.bitval[j], unpack_stages(x[q], R.mv[j], R.stages[j]));
      }
#pragma unroll
      for (int q = 0; q < TG; ++q) {
        uint32_t* dst = ROUTED ? a.out + (uint64_t)lane_u32(trow, i0 + q) * kW + lane
                               : obase + (uint64_t)(i0 + q) * kW;
        store_out(dst + (uint32_t)kWave * j, x[q]);
      }
    }
  }
}

// RPI tensors per load instruction (LPR = 64/RPI lanes each, one 16 B unit
// per lane: LPR >= the payload's units).  FULL: W == 64*J, so every lane has
// a word in every j.
template <int J, int T, int RPI, bool FULL>
__device__ __forceinline__ void tile_body(GatherArgs& a, uint32_t block, uint32_t blocks) {
  constexpr uint32_t LPR = kWave / RPI;
  constexpr int NL = T / RPI;  // load instructions per tile
  extern __shared__ __align__(16) uint8_t smem[];
  const GatherLds L(a.sh.W, a.pbuf_bytes);  // pref/kc/wsum as the group kernel
  uint32_t* s_pref = (uint32_t*)(smem + L.pref);
  uint32_t* s_kc = (uint32_t*)(smem + L.kc);
  uint32_t* s_wsum = (uint32_t*)(smem + L.wsum);
  const uint32_t wave = uniform(threadIdx.x / kWave);
  const uint32_t lane = threadIdx.x % kWave;
  uint8_t* wbase = smem + L.group0 + wave * (2 * T * (uint32_t)sizeof(TileHdr) + T * a.pbuf_bytes);
  TileHdr* hdrs = (TileHdr*)wbase;  // [2][T]
  uint8_t* pbufs = wbase + 2 * T * sizeof(TileHdr);

  const uint32_t W = a.sh.W;
  const uint64_t n_tiles = (a.n_ids + T - 1) / T;
  const uint64_t n_full = a.n_ids / T;  // tiles whose T rows all exist
  const uint64_t waves = (uint64_t)blocks * (blockDim.x / kWave);
  const uint64_t tile0 = (uint64_t)block * (blockDim.x / kWave) + wave;
  const uint32_t mrow = lane % T;  // the tile row this lane's metadata is for

  // Tile metadata runs ahead of the payloads: ids three tiles ahead, bitmap
  // words and offsets two ahead, the headers one ahead.
  // (the first tile's metadata round trips overlap the chunk counts; its
  // payloads are requested before the per-word registers are built)
  const int64_t id_a = tile_row_id(a, tile0 * T + mrow);
  const int64_t id_b = tile_row_id(a, (tile0 + waves) * T + mrow);
  PlanRun run;
  load_plan_run(a.mask, a.sh, run);
  WordRegs<J> R;
  load_plan_fetch<J>(a.mask, a.bitval, a.sh, lane, R);
  const TileMeta m0 = load_tile_meta(a, id_a);

  load_plan_counts(run, a.sh, s_pref, s_kc, s_wsum);
  // short batches (NL == 2: a tile or two per wave) build the per-word plan
  // once per workgroup (load_plan_words_shared, a barrier below), so idle
  // waves stay until then
  constexpr bool kSharedPlan = NL == 2;
  if (!kSharedPlan && tile0 >= n_tiles) return;  // per wave; no workgroup barrier follows

  TileMeta meta_next = load_tile_meta(a, id_b);
  if (lane < (uint32_t)T) hdrs[lane] = make_tile_hdr(a, m0, s_kc);
  int64_t id_next2 = tile_row_id(a, (tile0 + 2 * waves) * T + mrow);
  wave_sync();

  // payload registers of the tile in flight: NL <= 8 named registers (an
  // array would be indexed through scratch memory)
  static_assert(NL <= 8, "at most 8 load instructions per tile");
  uint4 v0, v1, v2, v3, v4, v5, v6, v7;
  uint32_t n0 = 0, n1 = 0, n2 = 0, n3 = 0, n4 = 0, n5 = 0, n6 = 0, n7 = 0;
  const uint32_t lrow = lane / LPR, lunit = lane % LPR;
  // every unit of a slot that a lane covers is written (zeros past the
  // payload: lanes past it loaded g_zero16), so a slot never holds a stale
  // payload and an invalid tensor's slot is all zero
  const uint32_t slot16 = a.pbuf_bytes >> 4;
  const uint64_t zero_addr = (uint64_t)&g_zero16;
#define IBP_TILE_LOAD(k, hdr)                                                                  \
  if constexpr (k < NL) {                                                                      \
    const TileHdr& h_ = (hdr)[k * RPI + lrow];                                                 \
    n##k = h_.n16;                                                                             \
    v##k = load_global((const uint4*)(lunit < n##k ? h_.addr + 16u * lunit : zero_addr));     \
  }
#define IBP_TILE_ISSUE_LOADS(hdr)                                                              \
  IBP_TILE_LOAD(0, hdr) IBP_TILE_LOAD(1, hdr) IBP_TILE_LOAD(2, hdr) IBP_TILE_LOAD(3, hdr)      \
  IBP_TILE_LOAD(4, hdr) IBP_TILE_LOAD(5, hdr) IBP_TILE_LOAD(6, hdr) IBP_TILE_LOAD(7, hdr)
#define IBP_TILE_STAGE(k)                                                                      \
  if constexpr (k < NL) {                                                                      \
    if (lunit < slot16) ((uint4*)(pbufs + (k * RPI + lrow) * a.pbuf_bytes))[lunit] = v##k;     \
  }
  IBP_TILE_ISSUE_LOADS(hdrs)

  if constexpr (kSharedPlan) {
    uint32_t* s_mv = (uint32_t*)(smem + L.group0 +
                                 (blockDim.x / kWave) *
                                     (2 * T * (uint32_t)sizeof(TileHdr) + T * a.pbuf_bytes));
    load_plan_words_shared<J>(a.sh, s_pref, lane, wave, R, s_mv);
    if (tile0 >= n_tiles) return;  // per wave; no workgroup barrier follows
  } else {
    load_plan_words<J>(a.sh, s_pref, lane, R);
  }

  uint32_t cur = 0;
  for (uint64_t tile = tile0; tile < n_tiles; tile += waves, cur ^= 1u) {
    const bool has_next = tile + waves < n_tiles;
    TileHdr* hcur = hdrs + cur * T;
    TileHdr* hnext = hdrs + (cur ^ 1u) * T;
    // a. this tile's payloads -> LDS
    IBP_TILE_STAGE(0) IBP_TILE_STAGE(1) IBP_TILE_STAGE(2) IBP_TILE_STAGE(3)
    IBP_TILE_STAGE(4) IBP_TILE_STAGE(5) IBP_TILE_STAGE(6) IBP_TILE_STAGE(7)
    // b. next tile's headers (metadata loaded an iteration ago); past the
    //    last tile they are invalid, so its loads below read only g_zero16
    if (lane < (uint32_t)T) {
      TileHdr h = make_tile_hdr(a, meta_next, s_kc);
      if (!has_next) h.valid = 0, h.n16 = 0;
      hnext[lane] = h;
    }
    wave_sync();
    // c. metadata two and three tiles ahead, d. next tile's payload loads
    meta_next = load_tile_meta(a, id_next2);
    id_next2 = tile_row_id(a, (tile + 3 * waves) * T + mrow);
    IBP_TILE_ISSUE_LOADS(hnext)
    // e. decode this tile and store it.  Chunks hold at least 64 words, so
    //    the 64 words lane l handles for one j lie in one chunk: chunk,
    //    participation and offset are wave-uniform.
    const uint64_t row0 = tile * T;
    if (FULL && tile < n_full) {
      decode_full_tile<J, T>(a, R, pbufs, hcur, lane, row0);
    } else if (tile < n_full) {
#pragma unroll 1
      for (int i = 0; i < T; ++i) {
        const TileHdr* hp = hcur + i;
        const bool valid = uniform(hp->valid) != 0u;
        const uint32_t pm = uniform(hp->pmask);
        const uint32_t o1 = uniform(hp->off[0]), o2 = uniform(hp->off[1]), o3 = uniform(hp->off[2]);
        const uint32_t* pb32 = (const uint32_t*)(pbufs + i * a.pbuf_bytes);
        uint32_t* orow = a.out + (row0 + i) * W;
#pragma unroll
        for (int j = 0; j < J; ++j) {
          const uint32_t w = lane + kWave * j;
          const uint32_t val = tile_word<J>(a, R, j, pb32, pm, o1, o2, o3);
          if (FULL || w < W) store_out(orow + w, valid ? val : 0u);
        }
      }
    } else {
      // the last, partial tile
      for (int i = 0; i < T; ++i) {
        const uint64_t row = row0 + i;
        if (row >= a.n_ids) break;
        const TileHdr* hp = hcur + i;
        const bool valid = uniform(hp->valid) != 0u;
        const uint32_t pm = uniform(hp->pmask);
        const uint32_t o1 = uniform(hp->off[0]), o2 = uniform(hp->off[1]), o3 = uniform(hp->off[2]);
        const uint32_t* pb32 = (const uint32_t*)(pbufs + i * a.pbuf_bytes);
        uint32_t* orow = a.out + row * W;
#pragma unroll
        for (int j = 0; j < J; ++j) {
          const uint32_t w = lane + kWave * j;
          const uint32_t val = tile_word<J>(a, R, j, pb32, pm, o1, o2, o3);
          if (w < W) store_out(orow + w, valid ? val : 0u);
        }
      }
      break;  // it is the last tile
    }
    wave_sync();
  }
#undef IBP_TILE_ISSUE_LOADS
#undef IBP_TILE_LOAD
#undef IBP_TILE_STAGE
}

template <int J, int T, int RPI, bool FULL>
__global__ __launch_bounds__(256) void k_gather_tile(GatherArgs a) {
  tile_body<J, T, RPI, FULL>(a, blockIdx.x, gridDim.x);
}

// The tile kernel over segments, as k_gather_decompress_seg (many embedding
// tables, each with its own Mask, in one launch).
template <int J, int T, int RPI, bool FULL>
__global__ __launch_bounds__(256) void k_gather_tile_seg(GatherArgs a, SegTable t) {
  GatherArgs b;
  if (!segment_args(a, t, b)) return;  // the whole workgroup, before any barrier
  tile_body<J, T, RPI, FULL>(b, blockIdx.x % t.per_seg, t.per_seg);
}

template <int J, int T, int RPI, bool FULL>
static hipError_t launch_tile(const Geometry& g, GatherArgs a, hipStream_t s) {
  a.sh.group = kWave;  // lane l owns words l + 64j
  const uint32_t waves = 4;
  const GatherLds L(g.W, a.pbuf_bytes);
  const uint32_t shared_plan = T / RPI == 2 ? 20u * g.W : 0u;  // move masks, see k_gather_tile
  const uint32_t lds = L.group0 + waves * (2 * T * (uint32_t)sizeof(TileHdr) + T * a.pbuf_bytes) +
                       shared_plan;
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_gather_tile<J, T, RPI, FULL>,
                                                   waves * 64, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  const uint64_t tiles = (a.n_ids + T - 1) / T;
  const uint64_t want = (tiles + waves - 1) / waves;
  const uint64_t cap = (uint64_t)per_cu * (uint64_t)di.cus;
  const uint32_t blocks = (uint32_t)(want < cap ? want : cap);
  hipLaunchKernelGGL((k_gather_tile<J, T, RPI, FULL>), dim3(blocks), dim3(waves * 64), lds, s, a);
  return hipGetLastError();
}

template <int J, int T, int RPI, bool FULL>
static hipError_t launch_tile_seg(const Geometry& g, GatherArgs a, SegTable& t, uint64_t max_rows,
                                  hipStream_t s) {
  a.sh.group = kWave;
  const uint32_t waves = 4;
  const GatherLds L(g.W, a.pbuf_bytes);
  const uint32_t shared_plan = T / RPI == 2 ? 20u * g.W : 0u;
  const uint32_t lds = L.group0 + waves * (2 * T * (uint32_t)sizeof(TileHdr) + T * a.pbuf_bytes) +
                       shared_plan;
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_gather_tile_seg<J, T, RPI, FULL>,
                                                   waves * 64, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  // the resident capacity shared evenly by the segments, but no more
  // workgroups per segment than its largest one has tiles for
  const uint64_t cap = (uint64_t)per_cu * (uint64_t)di.cus;
  uint64_t per = cap / t.n_seg;
  const uint64_t need = ((max_rows + T - 1) / T + waves - 1) / waves;
  if (per > need) per = need;
  if (per < 1) per = 1;
  t.per_seg = (uint32_t)per;
  hipLaunchKernelGGL((k_gather_tile_seg<J, T, RPI, FULL>), dim3((uint32_t)(per * t.n_seg)),
                     dim3(waves * 64), lds, s, a, t);
  return hipGetLastError();
}

// Segmented launches of small tensors: tiles of 8 loads when the whole
// launch fills every CU with such tiles, else 2 (as launch_small).
template <int J, int RPI>
static hipError_t launch_small_seg(const Geometry& g, const GatherArgs& a, SegTable& t,
                                   uint64_t max_rows, hipStream_t s) {
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  const bool full = g.W == (uint32_t)kWave * J;
  const bool big = a.n_ids >= (uint64_t)8 * RPI * 8 * (uint64_t)di.cus;
  if (big)
    return full ? launch_tile_seg<J, IBP_BIG_NL * RPI, RPI, true>(g, a, t, max_rows, s)
                : launch_tile_seg<J, IBP_BIG_NL * RPI, RPI, false>(g, a, t, max_rows, s);
  return full ? launch_tile_seg<J, 2 * RPI, RPI, true>(g, a, t, max_rows, s)
              : launch_tile_seg<J, 2 * RPI, RPI, false>(g, a, t, max_rows, s);
}

// ---------------------------------------------------------------------------
// Cache-mode kernel for short batches of small tensors (W == 64 J) whose
// payloads are all in HBM.
//
// The tile kernel stages every payload in LDS by way of registers.  A payload
// in HBM can be read where it lies instead: each lane reads the 8 bytes that
// hold its word's bits straight from the cache (neighbouring lanes' windows
// share cache lines, so L1 serves most of them).  Nothing is staged and no
// workgroup barrier follows the plan, so a launch's chain of dependent steps
// (ids, metadata, payload, store) is shorter: on batches of a few thousand
// ids, which latency bounds, that wins.  On long batches the tile kernel's
// 16 B loads move more bytes per instruction and it is faster, so it keeps
// those.  A wave decodes TG tensors at a time, J word positions each.
// Pipeline per wave: the windows of tile k+1 are requested after tile k is
// decoded and before its rows are stored, so waiting for them never waits for
// those stores; the metadata of tile k+2 (and the ids of tile k+3) are
// requested just before.  Not for payloads in host memory, which this would
// read more than once.

// Per-lane header of tensor (lane % TG) of a tile.
struct DirectHdr {
  uint64_t addr;    // payload address (g_zero16 when nothing is readable)
  uint32_t pmask;   // participation bits
  uint32_t off[3];  // bit offsets of chunks 1..3
  uint32_t lim;     // readable bytes at addr, when an 8 B window may pass them
  uint32_t tail;    // 1: windows are bounded by lim (the cache's last entries)
};

__device__ __forceinline__ DirectHdr make_direct_hdr(const GatherArgs& a, const TileMeta& m,
                                                     const uint32_t* s_kc) {
  DirectHdr h;
  const Source src = source_of(a, m.t, m.o);
  const bool valid = m.valid && src.ok;
  const uint32_t n_c = a.sh.n_c;
  const uint64_t word = (uint64_t)m.w0 | ((uint64_t)m.w1 << 32);
  const uint32_t pm = valid ? (uint32_t)(word >> m.sh) & ((1u << n_c) - 1u) : 0u;
  uint32_t o = 0, offs[4];
#pragma unroll
  for (uint32_t c = 0; c < 4; ++c) {  // n_c <= 4
    offs[c] = o;
    if (c < n_c) o += ((pm >> c) & 1u) ? s_kc[c] : chunk_bits(a.sh, c);
  }
  h.off[0] = offs[1];
  h.off[1] = offs[2];
  h.off[2] = offs[3];
  h.pmask = pm;
  // a window starts at most 4 bytes before the payload's 16 B-rounded end
  const uint64_t len16 = valid ? (uint64_t)((((o + 7u) >> 3) + 15u) & ~15u) : 0ull;
  const bool readable = valid && len16 > 0 && src.avail >= len16;
  h.addr = readable ? src.addr : (uint64_t)&g_zero16;
  const uint64_t lim = src.avail < len16 + 16u ? src.avail : len16 + 16u;
  h.lim = readable ? (uint32_t)lim : 16u;
  h.tail = (!readable || src.avail < len16 + 4) ? 1u : 0u;
  return h;
}

// The 8 bytes at byte `byte` of a payload; past `lim` (tail headers only)
// they read as zero.  Invalid or empty payloads read g_zero16, whose words
// are all zero, so their windows are zero whatever the offset.
__device__ __forceinline__ uint2 direct_window(uint64_t base, uint32_t byte, bool tail,
                                               uint32_t lim) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2), aligned(4)));
  typedef __attribute__((address_space(1))) const u32x2 global_u32x2;
  typedef __attribute__((address_space(1))) const uint32_t global_u32;
  if (!tail) {
    const u32x2 v = *(global_u32x2*)(uintptr_t)(base + byte);
    return make_uint2(v.x, v.y);
  }
  const uint32_t b0 = byte + 4u <= lim ? byte : 0u;
  const uint32_t b1 = byte + 8u <= lim ? byte + 4u : 0u;
  const uint32_t d0 = *(global_u32*)(uintptr_t)(base + b0);
  const uint32_t d1 = *(global_u32*)(uintptr_t)(base + b1);
  return make_uint2(byte + 4u <= lim ? d0 : 0u, byte + 8u <= lim ? d1 : 0u);
}

template <int J, int TG>
__global__ __launch_bounds__(256) void k_gather_direct(GatherArgs a) {
  constexpr uint32_t kW = (uint32_t)kWave * J;
  extern __shared__ __align__(16) uint8_t smem[];
  const GatherLds L(a.sh.W, a.pbuf_bytes);
  uint32_t* s_pref = (uint32_t*)(smem + L.pref);
  uint32_t* s_kc = (uint32_t*)(smem + L.kc);
  uint32_t* s_wsum = (uint32_t*)(smem + L.wsum);
  const uint32_t wave = uniform(threadIdx.x / kWave);
  const uint32_t lane = threadIdx.x % kWave;
  const uint64_t n_tiles = (a.n_ids + TG - 1) / TG;
  const uint64_t waves = (uint64_t)gridDim.x * (blockDim.x / kWave);
  const uint64_t tile0 = (uint64_t)blockIdx.x * (blockDim.x / kWave) + wave;
  const uint32_t mrow = lane % TG;

  const int64_t id_a = tile_row_id(a, tile0 * TG + mrow);
  const int64_t id_b = tile_row_id(a, (tile0 + waves) * TG + mrow);
  PlanRun run;
  load_plan_run(a.mask, a.sh, run);
  WordRegs<J> R;
  load_plan_fetch<J>(a.mask, a.bitval, a.sh, lane, R);
  const TileMeta m0 = load_tile_meta(a, id_a);
  TileMeta meta_next = load_tile_meta(a, id_b);
  int64_t id_next2 = tile_row_id(a, (tile0 + 2 * waves) * TG + mrow);
  load_plan_counts(run, a.sh, s_pref, s_kc, s_wsum);  // workgroup barriers: every thread
  if (tile0 >= n_tiles) return;                       // per wave; no workgroup barrier follows
  load_plan_words<J>(a.sh, s_pref, lane, R);

  // windows of the tile in flight: [j][q]
  uint2 win[J][TG];
  DirectHdr h = make_direct_hdr(a, m0, s_kc);
#define IBP_DIRECT_ISSUE(hdr)                                                                 \
  {                                                                                           \
    const uint32_t hpm_ = (hdr).pmask;                                                        \
    _Pragma("unroll") for (int j = 0; j < J; ++j) {                                           \
      const uint32_t c_ = uniform(((uint32_t)kWave * j) >> a.sh.wpc_log2);                    \
      const uint32_t oj_ = c_ == 0 ? 0u : c_ == 1 ? (hdr).off[0] : c_ == 2 ? (hdr).off[1]     \
                                                                          : (hdr).off[2];     \
      const uint32_t pb_ = (uint32_t)__builtin_amdgcn_ballot_w64(((hpm_ >> c_) & 1u) != 0u);  \
      const uint32_t lo_ = R.info[j] & 0xFFFFu, hi_ = R.info[j] >> 16;                        \
      _Pragma("unroll") for (int q = 0; q < TG; ++q) {                                        \
        const uint64_t base_ = lane_u64((hdr).addr, q);                                       \
        const uint32_t bit_ = lane_u32(oj_, q) + (((pb_ >> q) & 1u) ? lo_ : hi_);             \
        const bool tail_ = lane_u32((hdr).tail, q) != 0u;                                     \
        win[j][q] = direct_window(base_, (bit_ >> 5) << 2, tail_, lane_u32((hdr).lim, q));    \
        const int k_ = j * TG + q;                                                            \
        shp[k_ / 6] = (k_ % 6 == 0 ? 0u : shp[k_ / 6]) | ((bit_ & 31u) << (5 * (k_ % 6)));     \
      }                                                                                       \
    }                                                                                         \
  }
  // the windows' bit shifts, 5 bits each (applied once the windows arrive;
  // alignbit reads only the low 5 bits of its shift operand)
  uint32_t shp[(J * TG + 5) / 6];
  IBP_DIRECT_ISSUE(h)
  uint32_t pm_cur = h.pmask;

  for (uint64_t tile = tile0; tile < n_tiles; tile += waves) {
    const bool has_next = tile + waves < n_tiles;
    // 1. decode this tile's windows
    uint32_t x[J][TG];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint32_t c = uniform(((uint32_t)kWave * j) >> a.sh.wpc_log2);
      const uint32_t pbits = (uint32_t)__builtin_amdgcn_ballot_w64(((pm_cur >> c) & 1u) != 0u);
#pragma unroll
      for (int q = 0; q < TG; ++q) {
        const int k = j * TG + q;
        x[j][q] = __builtin_amdgcn_alignbit(win[j][q].y, win[j][q].x, shp[k / 6] >> (5 * (k % 6)));
      }
      constexpr uint32_t gmask = TG == 32 ? ~0u : (1u << TG) - 1u;
      const uint32_t gp = pbits & gmask;
      if (gp == gmask) {
        unpack_stages_n<TG>(x[j], R.mv[j], R.stages[j]);
#pragma unroll
        for (int q = 0; q < TG; ++q) x[j][q] = bfi_op(R.mask[j], R.bitval[j], x[j][q]);
      } else if (gp != 0u) {
#pragma unroll
        for (int q = 0; q < TG; ++q)
          if ((gp >> q) & 1u)
            x[j][q] = bfi_op(R.mask[j], R.bitval[j], unpack_stages(x[j][q], R.mv[j], R.stages[j]));
      }
    }
    // 2. next tile: header, metadata two ahead, windows
    if (has_next) {
      h = make_direct_hdr(a, meta_next, s_kc);
      meta_next = load_tile_meta(a, id_next2);
      id_next2 = tile_row_id(a, (tile + 3 * waves) * TG + mrow);
      IBP_DIRECT_ISSUE(h)
      pm_cur = h.pmask;
    }
    // 3. store this tile (rows past the batch are not written)
    const uint64_t row0 = tile * TG;
#pragma unroll
    for (int q = 0; q < TG; ++q) {
      if (row0 + q < a.n_ids) {
        uint32_t* dst = a.out + (row0 + q) * kW + lane;
#pragma unroll
        for (int j = 0; j < J; ++j) store_out(dst + (uint32_t)kWave * j, x[j][q]);
      }
    }
  }
#undef IBP_DIRECT_ISSUE
}

template <int J, int TG>
static hipError_t launch_direct(const Geometry& g, GatherArgs a, hipStream_t s) {
  a.sh.group = kWave;  // lane l owns words l + 64j
  const uint32_t waves = 4;
  const GatherLds L(g.W, a.pbuf_bytes);
  const uint32_t lds = L.group0;
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_gather_direct<J, TG>, waves * 64,
                                                   lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  const uint64_t tiles = (a.n_ids + TG - 1) / TG;
  const uint64_t want = (tiles + waves - 1) / waves;
  const uint64_t cap = (uint64_t)per_cu * (uint64_t)di.cus;
  const uint32_t blocks = (uint32_t)(want < cap ? want : cap);
  hipLaunchKernelGGL((k_gather_direct<J, TG>), dim3(blocks), dim3(waves * 64), lds, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Tile kernel with XCD-aware routing, for payloads read from their slots.
//
// The eight XCDs have an L2 each, and workgroups are dispatched to them round
// robin (block b on XCD b % 8).  When a batch repeats ids (Zipf), a tensor
// read by waves on several XCDs crosses the host link (or HBM) once per XCD.
// Here every id is routed to one XCD, chosen by a hash of the tensor index:
// the waves of XCD x split the batch into equal segments, and each wave keeps
// the rows of its segment whose tensor hashes to x, in a small LDS list, and
// decodes them T at a time.  Every row is processed exactly once: by the wave
// whose segment holds it, on the XCD its tensor hashes to.  A last, partial
// tile is padded with copies of its last row (written twice, with the same
// bytes).  Tiles are processed one after another (no prefetch across tiles):
// the launches this serves are short and have about one tile per wave.

// LDS bytes of one wave: T headers, T payload slots, the row list.
__host__ __device__ constexpr uint32_t routed_list_cap(uint32_t T) { return T + (uint32_t)kWave; }
__host__ __device__ inline uint32_t routed_wave_bytes(uint32_t T, uint32_t pbuf_bytes) {
  return T * (uint32_t)sizeof(TileHdr) + T * pbuf_bytes + ((routed_list_cap(T) * 12u + 15u) & ~15u);
}

// Workgroup `block` of `blocks` (a multiple of 8) must run on XCD block % 8,
// as for gather_group_routed_body.
template <int J, int T, int RPI, bool FULL>
__device__ __forceinline__ void tile_routed_body(GatherArgs& a, uint32_t block, uint32_t blocks) {
  constexpr uint32_t LPR = kWave / RPI;
  constexpr int NL = T / RPI;
  static_assert(NL <= 8, "at most 8 load instructions per tile");
  constexpr uint32_t kCap = routed_list_cap(T);
  extern __shared__ __align__(16) uint8_t smem[];
  const GatherLds L(a.sh.W, a.pbuf_bytes);
  uint32_t* s_pref = (uint32_t*)(smem + L.pref);
  uint32_t* s_kc = (uint32_t*)(smem + L.kc);
  uint32_t* s_wsum = (uint32_t*)(smem + L.wsum);
  const uint32_t wave = uniform(threadIdx.x / kWave);
  const uint32_t lane = threadIdx.x % kWave;
  const uint32_t wpb = blockDim.x / kWave;
  uint8_t* wbase = smem + L.group0 + wave * routed_wave_bytes(T, a.pbuf_bytes);
  TileHdr* hdrs = (TileHdr*)wbase;                                    // [T]
  uint8_t* pbufs = wbase + T * sizeof(TileHdr);                       // [T][pbuf_bytes]
  int64_t* list_id = (int64_t*)(pbufs + T * a.pbuf_bytes);           // [kCap]
  uint32_t* list_row = (uint32_t*)(list_id + kCap);                   // [kCap]

  // this wave's XCD and segment of the batch (the grid is a multiple of 8)
  const uint32_t xcd = block % kXcds;
  const uint64_t wc = (uint64_t)(blocks / kXcds) * wpb;
  const uint64_t wk = (uint64_t)(block / kXcds) * wpb + wave;
  const uint64_t seg = (a.n_ids + wc - 1) / wc;
  const uint64_t s0 = min(wk * seg, a.n_ids), s1 = min(s0 + seg, a.n_ids);

  // The Mask words and the first window of ids are requested first; the
  // per-word registers are built once the first tile's payloads are in
  // flight.
  PlanRun run;
  load_plan_run(a.mask, a.sh, run);
  WordRegs<J> R;
  load_plan_fetch<J>(a.mask, a.bitval, a.sh, lane, R);
  int64_t win_id = a.ids[min(s0 + lane, a.n_ids - 1)];
  load_plan_counts(run, a.sh, s_pref, s_kc, s_wsum);  // workgroup barriers: every thread
  if (s0 >= s1) return;  // per wave; no workgroup barrier follows

  const uint32_t lrow = lane / LPR, lunit = lane % LPR;
  const uint32_t slot16 = a.pbuf_bytes >> 4;
  const uint64_t zero_addr = (uint64_t)&g_zero16;
  const uint32_t W = a.sh.W;
  bool planned = false;  // per-word registers built (wave-uniform)
  uint32_t count = 0;    // rows in the list (wave-uniform)
  for (uint64_t base = s0; base < s1; base += kWave) {
    // 1. this window's rows that belong to this XCD -> the list
    {
      const uint64_t r = base + lane;
      const bool in = r < s1;
      const int64_t id = base == s0 ? win_id : a.ids[in ? r : s1 - 1];
      const bool mine = in && xcd_of_tensor(id) == xcd;
      const uint64_t bal = __ballot(mine);
      const uint32_t before = (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
      if (mine) {
        list_id[count + before] = id;
        list_row[count + before] = (uint32_t)r;
      }
      count += (uint32_t)__popcll(bal);
      wave_sync();
    }
    const bool last = base + kWave >= s1;
    // 2. full tiles (and, after the last window, the rest)
    while (count >= (uint32_t)T || (last && count > 0u)) {
      const uint32_t n = count < (uint32_t)T ? count : (uint32_t)T;
      const uint32_t e = min(lane % (uint32_t)T, n - 1u);
      const uint32_t trow = list_row[e];
      const TileMeta m = load_tile_meta(a, list_id[e]);
      if (lane < (uint32_t)T) hdrs[lane] = make_tile_hdr(a, m, s_kc);
      wave_sync();
      uint4 v0, v1, v2, v3, v4, v5, v6, v7;
#define IBP_RT_LOAD(k)                                                                          \
      if constexpr (k < NL) {                                                                   \
        const TileHdr& h_ = hdrs[k * RPI + lrow];                                               \
        v##k = load_global((const uint4*)(lunit < h_.n16 ? h_.addr + 16u * lunit : zero_addr)); \
      }
#define IBP_RT_STAGE(k)                                                                         \
      if constexpr (k < NL) {                                                                   \
        if (lunit < slot16) ((uint4*)(pbufs + (k * RPI + lrow) * a.pbuf_bytes))[lunit] = v##k;  \
      }
      IBP_RT_LOAD(0) IBP_RT_LOAD(1) IBP_RT_LOAD(2) IBP_RT_LOAD(3)
      IBP_RT_LOAD(4) IBP_RT_LOAD(5) IBP_RT_LOAD(6) IBP_RT_LOAD(7)
      if (!planned) {
        load_plan_words<J>(a.sh, s_pref, lane, R);
        planned = true;
      }
      IBP_RT_STAGE(0) IBP_RT_STAGE(1) IBP_RT_STAGE(2) IBP_RT_STAGE(3)
      IBP_RT_STAGE(4) IBP_RT_STAGE(5) IBP_RT_STAGE(6) IBP_RT_STAGE(7)
#undef IBP_RT_LOAD
#undef IBP_RT_STAGE
      wave_sync();
      if constexpr (FULL) {
        decode_full_tile<J, T, true>(a, R, pbufs, hdrs, lane, 0, trow);
      } else {
        for (uint32_t i = 0; i < n; ++i) {
          const TileHdr* hp = hdrs + i;
          const bool valid = uniform(hp->valid) != 0u;
          const uint32_t pm = uniform(hp->pmask);
          const uint32_t o1 = uniform(hp->off[0]), o2 = uniform(hp->off[1]), o3 = uniform(hp->off[2]);
          const uint32_t* pb32 = (const uint32_t*)(pbufs + i * a.pbuf_bytes);
          uint32_t* orow = a.out + (uint64_t)lane_u32(trow, i) * W;
#pragma unroll
          for (int j = 0; j < J; ++j) {
            const uint32_t w = lane + kWave * j;
            const uint32_t val = tile_word<J>(a, R, j, pb32, pm, o1, o2, o3);
            if (w < W) store_out(orow + w, valid ? val : 0u);
          }
        }
      }
      // 3. drop the tile's rows from the list
      const uint32_t rest = count - n;
      int64_t keep_id = 0;
      uint32_t keep_row = 0;
      if (lane < rest) {
        keep_id = list_id[n + lane];
        keep_row = list_row[n + lane];
      }
      wave_sync();
      if (lane < rest) {
        list_id[lane] = keep_id;
        list_row[lane] = keep_row;
      }
      count = rest;
      wave_sync();
    }
  }
}

template <int J, int T, int RPI, bool FULL>
__global__ __launch_bounds__(256) void k_gather_tile_routed(GatherArgs a) {
  tile_routed_body<J, T, RPI, FULL>(a, blockIdx.x, gridDim.x);
}

// Routed, over segments (per_seg a multiple of 8, as k_gather_decompress_routed_seg).
template <int J, int T, int RPI, bool FULL>
__global__ __launch_bounds__(256) void k_gather_tile_routed_seg(GatherArgs a, SegTable t) {
  GatherArgs b;
  if (!segment_args(a, t, b)) return;  // the whole workgroup, before any barrier
  tile_routed_body<J, T, RPI, FULL>(b, blockIdx.x % t.per_seg, t.per_seg);
}

template <int J, int T, int RPI, bool FULL>
static hipError_t launch_tile_routed(const Geometry& g, GatherArgs a, hipStream_t s) {
  a.sh.group = kWave;
  const uint32_t waves = 4;
  const GatherLds L(g.W, a.pbuf_bytes);
  const uint32_t lds = L.group0 + waves * routed_wave_bytes(T, a.pbuf_bytes);
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_gather_tile_routed<J, T, RPI, FULL>,
                                                   waves * 64, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  const uint64_t tiles = (a.n_ids + T - 1) / T;
  const uint64_t want = (tiles + waves - 1) / waves;
  const uint64_t cap = (uint64_t)per_cu * (uint64_t)di.cus;
  uint64_t blocks = want < cap ? want : cap;
  blocks = blocks < kXcds ? kXcds : blocks / kXcds * kXcds;  // every XCD class has the same blocks
  hipLaunchKernelGGL((k_gather_tile_routed<J, T, RPI, FULL>), dim3((uint32_t)blocks),
                     dim3(waves * 64), lds, s, a);
  return hipGetLastError();
}

// Workgroups per segment of a routed segmented launch: the resident capacity
// shared evenly by the segments, no more than `need`, rounded down to a
// multiple of 8 (every XCD class of a segment has the same workgroups), at
// least 8.
static uint32_t routed_per_seg(uint64_t cap, uint32_t n_seg, uint64_t need) {
  uint64_t per = cap / n_seg;
  if (per > need) per = need;
  per = per / kXcds * kXcds;
  return (uint32_t)(per < kXcds ? kXcds : per);
}

template <int J, int T, int RPI, bool FULL>
static hipError_t launch_tile_routed_seg(const Geometry& g, GatherArgs a, SegTable& t,
                                         uint64_t max_rows, hipStream_t s) {
  a.sh.group = kWave;
  const uint32_t waves = 4;
  const GatherLds L(g.W, a.pbuf_bytes);
  const uint32_t lds = L.group0 + waves * routed_wave_bytes(T, a.pbuf_bytes);
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &per_cu, k_gather_tile_routed_seg<J, T, RPI, FULL>, waves * 64, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  const uint64_t need = ((max_rows + T - 1) / T + waves - 1) / waves;
  t.per_seg = routed_per_seg((uint64_t)per_cu * (uint64_t)di.cus, t.n_seg, need);
  hipLaunchKernelGGL((k_gather_tile_routed_seg<J, T, RPI, FULL>), dim3(t.per_seg * t.n_seg),
                     dim3(waves * 64), lds, s, a, t);
  return hipGetLastError();
}

template <int J, int RPI>
static hipError_t launch_small_routed_seg(const Geometry& g, const GatherArgs& a, SegTable& t,
                                          uint64_t max_rows, hipStream_t s) {
  const bool full = g.W == (uint32_t)kWave * J;
  return full ? launch_tile_routed_seg<J, 2 * RPI, RPI, true>(g, a, t, max_rows, s)
              : launch_tile_routed_seg<J, 2 * RPI, RPI, false>(g, a, t, max_rows, s);
}

// Small tensors (W <= 256): rows per load instruction RPI from the payload's
// 16 B units (J fixes them: J = 1 -> <= 16 units, 2 -> <= 32, 3 and 4 ->
// <= 64), and NL load instructions per tile: 8 when the batch gives every CU
// at least 8 waves of such tiles, else 2 (short batches need many waves in
// flight more than they need the per-tile overhead amortised).
template <int J, int RPI>
static hipError_t launch_small(const Geometry& g, const GatherArgs& a, hipStream_t s) {
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  const bool full = g.W == (uint32_t)kWave * J;
  const bool big = a.n_ids >= (uint64_t)8 * RPI * 8 * (uint64_t)di.cus;
  // one-chunk tensors of 64, 128 or 256 words, every payload in HBM
  if (cache_kernel_fits(g) && a.offsets != nullptr && a.store == nullptr && !a.route)
    return launch_gather_cache_table(g, a.cache, a.cache_bytes, a.offsets, a.part_bits,
                                     a.n_tensors, a.ids, a.n_ids, a.mask, a.bitval, a.out, s);
  // other short launches with every payload in HBM (no host slots): read in place
  if (full && !big && a.offsets != nullptr && a.store == nullptr && !a.route)
    return launch_direct<J, (J >= 3 ? IBP_DIRECT_TG / 2 : IBP_DIRECT_TG)>(g, a, s);
  if (a.route)
    return full ? launch_tile_routed<J, 2 * RPI, RPI, true>(g, a, s)
                : launch_tile_routed<J, 2 * RPI, RPI, false>(g, a, s);
  if (big)
    return full ? launch_tile<J, IBP_BIG_NL * RPI, RPI, true>(g, a, s)
                : launch_tile<J, IBP_BIG_NL * RPI, RPI, false>(g, a, s);
  return full ? launch_tile<J, 2 * RPI, RPI, true>(g, a, s) : launch_tile<J, 2 * RPI, RPI, false>(g, a, s);
}

template <int J>
static hipError_t launch_j_routed(const Geometry& g, const GatherArgs& a, hipStream_t s) {
  const GatherLds L(g.W, a.pbuf_bytes);
  const uint32_t lds = L.total(1) + routed_group_list_bytes();
  const uint32_t threads = g.group;
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_gather_decompress_routed<J>, threads,
                                                   lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  const uint64_t cap = (uint64_t)per_cu * (uint64_t)di.cus;
  uint64_t blocks = a.n_ids < cap ? a.n_ids : cap;
  blocks = blocks < kXcds ? kXcds : blocks / kXcds * kXcds;
  hipLaunchKernelGGL(k_gather_decompress_routed<J>, dim3((uint32_t)blocks), dim3(threads), lds, s,
                     a);
  return hipGetLastError();
}

template <int J>
static hipError_t launch_j(const Geometry& g, const GatherArgs& a, hipStream_t s) {
  if (a.route && g.groups == 1) return launch_j_routed<J>(g, a, s);
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
                         uint64_t slot_bytes, const uint64_t* offsets, const uint8_t* cache,
                         uint64_t cache_bytes, const uint32_t* part_bits, uint64_t n_tensors,
                         const int64_t* ids, uint64_t n_ids, const uint32_t* mask,
                         const uint32_t* bitval, uint32_t* out, bool route, hipStream_t s) {
  if (n_ids == 0) return hipSuccess;
  // no tensors: every id is out of range and every row is zero
  if (n_tensors == 0) return launch_fill_u32(out, n_ids * (uint64_t)g.W, 0u, s);
  GatherArgs a;
  a.store = store;
  a.store_bytes = store ? store_bytes : 0;
  a.slot_bytes = slot_bytes;
  a.offsets = offsets;
  a.cache = cache;
  a.cache_bytes = cache ? cache_bytes : 0;
  a.part_bits = part_bits;
  a.n_tensors = n_tensors;
  a.ids = ids;
  a.n_ids = n_ids;
  a.mask = mask;
  a.bitval = bitval;
  a.out = out;
  a.sh = Shape{g.W, g.n_c, g.wpc_log2, g.last_bits, g.group};
  a.groups = g.groups;
  a.route = route && offsets == nullptr && n_ids < (1ull << 32);
  // payload rounded to 16 B, plus one word read past the end by the window
  a.pbuf_bytes = ((g.tensor_bytes + 15u) & ~15u) + 16u;
  if (g.W <= 4 * (uint32_t)kWave) {
    // small tensors: tile kernel, lane l owns words l + 64j
    switch ((g.W + kWave - 1) / kWave) {
      case 1: return launch_small<1, 4>(g, a, s);  // <= 256 B: <= 16 units
      case 2: return launch_small<2, 2>(g, a, s);  // <= 512 B: <= 32 units
      case 3: return launch_small<3, 1>(g, a, s);  // <= 1 KB: <= 64 units
      case 4: return launch_small<4, 1>(g, a, s);
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

template <int J>
static hipError_t launch_j_routed_seg(const Geometry& g, const GatherArgs& a, const SegTable& t0,
                                      uint64_t max_rows, hipStream_t s) {
  const GatherLds L(g.W, a.pbuf_bytes);
  const uint32_t lds = L.total(1) + routed_group_list_bytes();
  const uint32_t threads = g.group;
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_gather_decompress_routed_seg<J>,
                                                   threads, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  SegTable t = t0;
  t.per_seg = routed_per_seg((uint64_t)per_cu * (uint64_t)di.cus, t.n_seg, max_rows);
  hipLaunchKernelGGL(k_gather_decompress_routed_seg<J>, dim3(t.per_seg * t.n_seg), dim3(threads),
                     lds, s, a, t);
  return hipGetLastError();
}

template <int J>
static hipError_t launch_j_seg(const Geometry& g, const GatherArgs& a, const SegTable& t0,
                               uint64_t max_rows, hipStream_t s) {
  if (a.route && g.groups == 1) return launch_j_routed_seg<J>(g, a, t0, max_rows, s);
  const GatherLds L(g.W, a.pbuf_bytes);
  const uint32_t lds = L.total(g.groups);
  const uint32_t threads = g.group * g.groups;
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_gather_decompress_seg<J>, threads,
                                                   lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  // the resident capacity shared evenly by the segments, but no more
  // workgroups per segment than its largest one has rows for
  SegTable t = t0;
  const uint64_t cap = (uint64_t)per_cu * (uint64_t)di.cus;
  uint64_t per = cap / t.n_seg;
  const uint64_t need = (max_rows + g.groups - 1) / g.groups;
  if (per > need) per = need;
  if (per < 1) per = 1;
  t.per_seg = (uint32_t)per;
  hipLaunchKernelGGL(k_gather_decompress_seg<J>, dim3((uint32_t)(per * t.n_seg)), dim3(threads),
                     lds, s, a, t);
  return hipGetLastError();
}

hipError_t launch_gather_segments(const Geometry& g, const uint8_t* store, uint64_t store_bytes,
                                  uint64_t slot_bytes, const uint64_t* offsets,
                                  const uint8_t* cache, uint64_t cache_bytes,
                                  const uint32_t* part_bits, uint64_t n_tensors,
                                  const int64_t* ids, const uint64_t* seg_off, uint32_t n_seg,
                                  const uint32_t* masks, const uint32_t* bitvals, uint32_t* out,
                                  bool route, hipStream_t s) {
  const uint64_t n_ids = seg_off[n_seg];
  if (n_ids == 0) return hipSuccess;
  if (n_tensors == 0) {
    // no tensors: every row is zero (one fill per non-empty segment)
    for (uint32_t k = 0; k < n_seg; ++k) {
      const uint64_t o = seg_off[k], n = seg_off[k + 1] - o;
      if (n == 0) continue;
      const hipError_t e = launch_gather(g, store, store_bytes, slot_bytes, offsets, cache,
                                         cache_bytes, part_bits, n_tensors, ids + o, n,
                                         masks + (uint64_t)k * g.W, bitvals + (uint64_t)k * g.W,
                                         out + o * g.W, false, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  GatherArgs a;
  a.store = store;
  a.store_bytes = store ? store_bytes : 0;
  a.slot_bytes = slot_bytes;
  a.offsets = offsets;
  a.cache = cache;
  a.cache_bytes = cache ? cache_bytes : 0;
  a.part_bits = part_bits;
  a.n_tensors = n_tensors;
  a.ids = ids;
  a.n_ids = n_ids;
  a.mask = masks;
  a.bitval = bitvals;
  a.out = out;
  a.sh = Shape{g.W, g.n_c, g.wpc_log2, g.last_bits, g.group};
  a.groups = g.groups;
  a.route = route && offsets == nullptr && n_ids < (1ull << 32);
  a.pbuf_bytes = ((g.tensor_bytes + 15u) & ~15u) + 16u;
  SegTable t;
  uint64_t max_rows = 0;
  for (uint32_t k = 0; k <= n_seg; ++k) t.off[k] = seg_off[k];
  for (uint32_t k = 0; k < n_seg; ++k)
    max_rows = seg_off[k + 1] - seg_off[k] > max_rows ? seg_off[k + 1] - seg_off[k] : max_rows;
  t.n_seg = n_seg;
  t.per_seg = 1;
  if (g.W <= 4 * (uint32_t)kWave) {
    // small tensors: the tile kernel, lane l owns words l + 64j
    if (a.route) {
      switch ((g.W + kWave - 1) / kWave) {
        case 1: return launch_small_routed_seg<1, 4>(g, a, t, max_rows, s);
        case 2: return launch_small_routed_seg<2, 2>(g, a, t, max_rows, s);
        case 3: return launch_small_routed_seg<3, 1>(g, a, t, max_rows, s);
        case 4: return launch_small_routed_seg<4, 1>(g, a, t, max_rows, s);
        default: return hipErrorInvalidValue;
      }
    }
    switch ((g.W + kWave - 1) / kWave) {
      case 1: return launch_small_seg<1, 4>(g, a, t, max_rows, s);
      case 2: return launch_small_seg<2, 2>(g, a, t, max_rows, s);
      case 3: return launch_small_seg<3, 1>(g, a, t, max_rows, s);
      case 4: return launch_small_seg<4, 1>(g, a, t, max_rows, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (g.J) {
    case 1: return launch_j_seg<1>(g, a, t, max_rows, s);
    case 2: return launch_j_seg<2>(g, a, t, max_rows, s);
    case 3: return launch_j_seg<3>(g, a, t, max_rows, s);
    case 4: return launch_j_seg<4>(g, a, t, max_rows, s);
    case 5: return launch_j_seg<5>(g, a, t, max_rows, s);
    case 6: return launch_j_seg<6>(g, a, t, max_rows, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ibp
