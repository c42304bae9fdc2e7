// gather_cache.hip -- gather + decompress of one-chunk tensors held in a
// compacted HBM cache ([G-EN] System Integration, cache compression; Core
// Algorithm, Decompression).  A one-chunk tensor (chunk size >= tensor size)
// is either packed -- exactly K payload bits, K the kept (non-Mask) bits of
// the Mask -- or stored whole, so its payload length follows from its
// participation bit alone and it needs no chunk scan.
//
// Two ways to find an entry:
//   table  offsets[t] (one u64 per tensor, kNotCached = zero row) and the
//          participation bitmap, as ibp_gather_decompress takes them;
//   index  one u64 per 32 tensors: the participation word (low half) and the
//          number of participating tensors before it (high half).  With
//          entries of size s_p (packed) and s_r (whole), each rounded up to
//          the entry alignment A, entry t starts at
//              t * s_r - r1(t) * (s_r - s_p),
//          r1(t) the participating tensors before t.  The index is 1/32 of
//          the bitmap's tensors in u64 words (2 MB for 2^23 tensors), so it
//          stays in L2, where a per-tensor table costs a line per distinct
//          tensor; with A = 128 every entry starts on a 128 B line and
//          occupies the fewest lines its length allows.
//
// Launch shape: a wave takes S steps' rows, S * TPS consecutive rows.  A step
// moves TPS = 64 / L tensors, each with L = 16 J lanes loading one 16 B unit
// each (a plain row copy's shape).  Lane r of the wave resolves row r's entry
// (address, 16 B units to read, packed or not), then the wave requests all S
// payloads at once and decodes them step by step.  Lane u of a tensor owns
// words 4u..4u+3, the 16 B it loads for a whole tensor and stores in every
// case: a packed tensor's payload goes through an LDS slot, from which the
// lane reads its words' windows and decodes them in registers; a whole
// tensor's unit is already its words.  A batch whose waves fit one
// round of resident waves takes the fewest steps per wave that fit (S = 1, 2
// or 4; eight waves per SIMD for S <= 2); a longer batch takes S = 4 with a
// grid-stride loop over blocks, the next block's ids requested while the
// current payloads are in flight.
//
// Decode of one word w of a packed tensor: a 64-bit window of the payload at
// the word's kept-bit offset pre_w (two LDS words, v_alignbit), then the kept
// bits are spread to their positions and Bitval inserted under the Mask.
// When the kept bits of every word form at most two runs (the common case for
// float data: a run of invariant exponent bits splits the word), spreading is
// two shifts and one bit-field insert; otherwise the five-stage expand of
// ibp_device.h.  A whole (non-participating) tensor's word is its payload
// word.  Every select is a per-lane select, with no divergent branch.
#include "ibp_internal.h"
#include "ibp_device.h"

namespace ibp {

namespace {

// 1 KB of zeros: rows with no source (invalid id, no entry, an entry past the
// end of the cache) read 16 B per lane from here.
__device__ __align__(16) uint4 g_cache_zero[64];

constexpr uint64_t kNoEntry = ~0ull;

struct CacheArgs {
  const uint8_t* cache;
  uint64_t cache_bytes;
  const uint64_t* offsets;   // table mode
  const uint32_t* part_bits; // table mode
  const uint64_t* index;     // index mode
  uint64_t n_tensors;
  const int64_t* ids;
  uint64_t n_ids;
  const uint32_t* mask;
  const uint32_t* bitval;
  uint32_t* out;
  uint32_t align;            // index mode: entry alignment (power of two)
};

__device__ __forceinline__ uint64_t ld_u64(const uint64_t* p) { return load_global(p); }

__device__ __forceinline__ uint32_t ld_u32(const uint32_t* p) {
  typedef __attribute__((address_space(1))) const uint32_t global_u32;
  return *(global_u32*)(uintptr_t)p;
}

__device__ __forceinline__ int64_t row_id(const CacheArgs& a, uint64_t row) {
  const int64_t id = (int64_t)ld_u64((const uint64_t*)a.ids + (row < a.n_ids ? row : a.n_ids - 1));
  return row < a.n_ids ? id : -1;
}

// What lane r loads for row r of a block: the tensor's entry in the table
// (offset + participation word) or in the index.  Unconditional loads (an
// invalid id reads tensor 0's), resolved one step later.
struct RowRaw {
  uint64_t e;   // table: offset entry; index: index word
  uint32_t pw;  // table: participation word
  uint32_t t;   // tensor index mod 2^32 (bit position, rank)
  bool valid;
};

template <bool INDEXED>
__device__ __forceinline__ RowRaw row_raw(const CacheArgs& a, int64_t id) {
  RowRaw r;
  r.valid = id >= 0 && (uint64_t)id < a.n_tensors;
  const uint64_t t = r.valid ? (uint64_t)id : 0ull;
  r.t = (uint32_t)t;
  if (INDEXED) {
    r.e = ld_u64(a.index + (t >> 5));
    r.pw = 0;
  } else {
    r.e = ld_u64(a.offsets + t);
    r.pw = ld_u32(a.part_bits + (t >> 5));
  }
  return r;
}

// Row r's payload source, packed into two words for the lanes that read it:
//   lo = address bits 0..31, hi = address bits 32..47 | (units - 1) << 16 |
//   packed << 24.  A row with no source reads the zero block as a whole row.
struct RowMeta {
  uint32_t lo, hi;
};

template <bool INDEXED>
__device__ __forceinline__ RowMeta row_resolve(const CacheArgs& a, const RowRaw& r, uint32_t n16p,
                                               uint32_t n16r, uint64_t s_p, uint64_t s_r) {
  uint64_t off;
  bool p;
  if (INDEXED) {
    const uint32_t word = (uint32_t)r.e, rank = (uint32_t)(r.e >> 32);
    const uint32_t bit = r.t & 31u;
    p = (word >> bit) & 1u;
    const uint64_t r1 = (uint64_t)rank + (uint64_t)__popc(word & ((1u << bit) - 1u));
    off = (uint64_t)r.t * s_r - r1 * (s_r - s_p);
  } else {
    off = r.e;
    p = (r.pw >> (r.t & 31u)) & 1u;
  }
  const uint32_t want = p ? n16p : n16r;
  // the entry's units must lie inside the cache, else a zero row; a packed
  // entry of no units (every bit invariant) reads nothing and decodes to Bitval
  const bool empty = want == 0u;
  const bool inside = off < a.cache_bytes && (a.cache_bytes - off) >> 4 >= want;
  const bool src = r.valid && off != kNoEntry && (empty || inside);
  const bool rd = src && !empty;
  const uint64_t addr = rd ? (uint64_t)a.cache + off : (uint64_t)&g_cache_zero[0];
  const uint32_t units = rd ? want : 64u;
  RowMeta m;
  m.lo = (uint32_t)addr;
  m.hi = (uint32_t)(addr >> 32) | ((units - 1u) << 16) | ((uint32_t)(src && p) << 24);
  return m;
}

// Per-lane decode constants of one output word.
struct WordDec {
  uint32_t mk, bv;  // Mask, Bitval & Mask
  uint32_t ap, sp;  // LDS byte address and bit shift of the packed window
  uint32_t c[5];    // two-run: c[0] = first-run shift, c[1] = second-run shift, c[2] = first run;
                    // else the five move masks
};

// Kept bits of a word in at most two runs: first run (lowest kept bits) from
// packed bit 0 to position s1; second run from packed bit n1 to position s2.
__device__ __forceinline__ bool two_runs(uint32_t keep, uint32_t c[5]) {
  const uint32_t low = keep & (0u - keep);
  const uint32_t run1 = keep & ~(keep + low);
  const uint32_t rest = keep & ~run1;
  const uint32_t low2 = rest & (0u - rest);
  const bool ok = (rest & (rest + low2)) == 0u;  // rest is one run (or empty)
  const uint32_t s1 = keep ? (uint32_t)__builtin_ctz(keep) : 0u;
  const uint32_t n1 = (uint32_t)__popc(run1);
  const uint32_t s2 = rest ? (uint32_t)__builtin_ctz(rest) : n1;
  c[0] = s1;
  c[1] = s2 - n1;
  c[2] = run1;
  c[3] = 0;
  c[4] = 0;
  return ok;
}

template <bool RUNS>
__device__ __forceinline__ uint32_t spread(uint32_t p, const WordDec& d) {
  if (RUNS) return bfi_op(d.c[2], p << d.c[0], p << d.c[1]);
  uint32_t y = p;
  y = bfi_op(d.c[4], y << 16, y);
  y = bfi_op(d.c[3], y << 8, y);
  y = bfi_op(d.c[2], y << 4, y);
  y = bfi_op(d.c[1], y << 2, y);
  y = bfi_op(d.c[0], y << 1, y);
  return y;
}

constexpr uint32_t kCacheWaves = 4;

template <int J>
struct CacheGeo {
  static constexpr uint32_t L = 16u * J;                 // lanes (16 B units) per tensor
  static constexpr uint32_t TPS = (uint32_t)kWave / L;   // tensors per step
  static constexpr uint32_t kW = 4u * L;                 // words per tensor
  static constexpr uint32_t kSlot = 16u * L + 16u;       // LDS bytes per tensor + the word a window reads past
  // LDS: one payload slot per tensor of a step, per wave
  static constexpr uint32_t slots = 0;
  static constexpr uint32_t bytes = slots + kCacheWaves * TPS * kSlot;
};

// The kernel's LDS (static, so LDS addresses fold into instruction offsets).
template <int J>
struct CacheLds {
  uint8_t b[CacheGeo<J>::bytes];
};

// Decodes this lane's words 4u..4u+3 of a packed tensor, from the windows at
// their kept-bit offsets in the LDS slot, into registers.
template <bool RUNS>
__device__ __forceinline__ void decode_regs(const uint8_t* lds, const WordDec (&dw)[4],
                                            uint32_t (&z)[4]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const WordDec& d = dw[q];
    const uint32_t d0 = *(const uint32_t*)(lds + d.ap);
    const uint32_t d1 = *(const uint32_t*)(lds + d.ap + 4u);
    const uint32_t p = __builtin_amdgcn_alignbit(d1, d0, d.sp);
    z[q] = bfi_op(d.mk, d.bv, spread<RUNS>(p, d));
  }
}

// Kept-bit prefix of this lane's words 4u..4u+3 (the kept bits of all words
// before each) and K, the kept bits of the whole Mask, from the wave's own
// Mask words: the L lanes of a tensor hold every word once, so one scan of
// the lanes' kept-bit totals over each group of L lanes gives the prefixes,
// with no workgroup barrier.
template <int J>
__device__ __forceinline__ uint32_t kept_prefix(const WordDec (&dw)[4], uint32_t u,
                                                uint32_t (&pre)[4]) {
  constexpr uint32_t L = CacheGeo<J>::L;
  uint32_t x[4], t = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    x[q] = (uint32_t)__popc(~dw[q].mk);
    t += x[q];
  }
  uint32_t incl = t;
#pragma unroll
  for (uint32_t d = 1; d < L; d <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)incl, d, (int)L);
    if (u >= d) incl += y;
  }
  uint32_t run = incl - t;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    pre[q] = run;
    run += x[q];
  }
  return (uint32_t)__shfl((int)incl, (int)(L - 1u), (int)L);
}

// This lane's per-word decode constants (words 4u..4u+3) from their kept-bit
// prefixes.  Returns whether the kept bits of every word form at most two
// runs (the same answer in every lane of the wave).
__device__ __forceinline__ bool word_constants(WordDec (&dw)[4], const uint32_t (&pre)[4],
                                               uint32_t slot) {
  bool runs_ok = true;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    WordDec& d = dw[q];
    d.bv &= d.mk;
    d.ap = slot + 4u * (pre[q] >> 5);
    d.sp = pre[q] & 31u;
    runs_ok = two_runs(~d.mk, d.c) && runs_ok;
  }
  const bool runs = __ballot(!runs_ok) == 0ull;
  if (!runs) {
#pragma unroll
    for (int q = 0; q < 4; ++q) move_masks(~dw[q].mk, dw[q].c);
  }
  return runs;
}

// Wave w takes S steps' rows, w * S * TPS onwards, resolves their entries,
// requests all S payloads at once, then decodes them step by step.  Without
// LOOP the grid covers the batch once, so a launch's critical path is one
// chain: id -> entry -> payload -> decode -> store.  With LOOP the waves walk
// the batch with a grid stride, each block's ids requested while the previous
// block's payloads are in flight.
template <int J, bool INDEXED, uint32_t S, bool LOOP>
__global__ __launch_bounds__(256) void k_gather_cache(CacheArgs a) {
  using G = CacheGeo<J>;
  constexpr uint32_t L = G::L, TPS = G::TPS, kW = G::kW;
  constexpr uint32_t R = S * TPS;  // rows per wave
  static_assert(R <= (uint32_t)kWave, "one row per lane at most");
  __shared__ __align__(16) CacheLds<J> s_lds;
  uint8_t* lds = s_lds.b;
  const uint32_t wave = uniform(threadIdx.x / kWave);
  const uint32_t lane = threadIdx.x % kWave;
  const uint32_t g = lane / L, u = lane % L;
  const uint32_t slot = G::slots + (wave * TPS + g) * G::kSlot;
  uint64_t row0 = ((uint64_t)blockIdx.x * kCacheWaves + wave) * R;
  const uint64_t stride = (uint64_t)gridDim.x * kCacheWaves * R;

  // one round: per wave (that form has no workgroup barrier)
  if (!LOOP && row0 >= a.n_ids) return;

  // this wave's ids and their entries, the Mask/Bitval words, then the
  // kept-bit prefix of this lane's words (a scan within the wave)
  int64_t id = row_id(a, row0 + (lane < R ? lane : R - 1u));
  WordDec dw[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    dw[q].mk = ld_u32(a.mask + 4u * u + q);
    dw[q].bv = ld_u32(a.bitval + 4u * u + q);
  }
  RowRaw rr = row_raw<INDEXED>(a, id);
  uint32_t pre[4];
  const uint32_t K = kept_prefix<J>(dw, u, pre);
  if (LOOP) {
    // the grid-stride form starts its waves together: without this barrier
    // the 1M-id Zipf launches ran 6 % slower (dense_gnn, 170 against 160 us)
    __syncthreads();
    if (row0 >= a.n_ids) return;  // per wave; no workgroup barrier follows
  }
  const uint32_t n16p = (K + 127u) >> 7;
  const uint64_t amask = (uint64_t)a.align - 1u;
  const uint64_t s_p = (((uint64_t)K + 7u) / 8u + amask) & ~amask;
  const uint64_t s_r = ((uint64_t)(4u * kW) + amask) & ~amask;
  bool runs = true, planned = false;
  for (;;) {
    const RowMeta m = row_resolve<INDEXED>(a, rr, n16p, L, s_p, s_r);
    uint4 v[S];
    uint32_t pk[S];
#pragma unroll
    for (uint32_t d = 0; d < S; ++d) {
      const uint32_t i = d * TPS + g;
      const uint32_t lo = (uint32_t)__shfl((int)m.lo, (int)i, kWave);
      const uint32_t hi = (uint32_t)__shfl((int)m.hi, (int)i, kWave);
      const uint32_t un = min(u, (hi >> 16) & 63u);
      v[d] = load_global((const uint4*)((((uint64_t)(hi & 0xFFFFu) << 32) | lo) + 16ull * un));
      pk[d] = hi >> 24;
    }
    // the next block's ids (clamped, unconditional) while these payloads fly
    const uint64_t next = row0 + stride;
    if (LOOP) id = row_id(a, next + (lane < R ? lane : R - 1u));
    if (!planned) {
      runs = word_constants(dw, pre, slot);
      planned = true;
    }
    uint32_t* orow = a.out + (row0 + g) * kW + 4u * u;
#pragma unroll
    for (uint32_t d = 0; d < S; ++d) {
      *(uint4*)(lds + slot + 16u * u) = v[d];  // the windows of a packed payload
      wave_sync();
      const bool in = row0 + d * TPS + g < a.n_ids;
      // a whole tensor's unit is its words 4u..4u+3; a packed one's words
      // are decoded from the windows in the slot
      uint32_t z[4] = {v[d].x, v[d].y, v[d].z, v[d].w};
      if (in && pk[d] != 0u) {
        if (runs)
          decode_regs<true>(lds, dw, z);
        else
          decode_regs<false>(lds, dw, z);
      }
      if (in) {
        // one store site per step, so the streaming hint stays on every store
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 row = {z[0], z[1], z[2], z[3]};
        __builtin_nontemporal_store(row, (u32x4*)orow);
      }
      orow += TPS * kW;
      wave_sync();  // every window read before the next step's payload lands
    }
    if (!LOOP || next >= a.n_ids) break;
    row0 = next;
    rr = row_raw<INDEXED>(a, id);
  }
}

// Resident waves of one k_gather_cache instance on the current device.
template <int J, bool INDEXED, uint32_t S, bool LOOP>
hipError_t resident_waves(int cus, uint64_t* waves) {
  int per_cu = 0;
  const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &per_cu, k_gather_cache<J, INDEXED, S, LOOP>, kCacheWaves * kWave, 0);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  *waves = (uint64_t)per_cu * (uint64_t)cus * kCacheWaves;
  return hipSuccess;
}

// One round with S steps per wave if the batch's waves fit (*done set).
template <int J, bool INDEXED, uint32_t S>
hipError_t try_one_round(const CacheArgs& a, int cus, bool* done, hipStream_t s) {
  constexpr uint64_t R = S * CacheGeo<J>::TPS;
  uint64_t resident = 0;
  hipError_t e = resident_waves<J, INDEXED, S, false>(cus, &resident);
  if (e != hipSuccess) return e;
  const uint64_t waves = (a.n_ids + R - 1) / R;
  *done = waves <= resident;
  if (!*done) return hipSuccess;
  hipLaunchKernelGGL((k_gather_cache<J, INDEXED, S, false>),
                     dim3((uint32_t)((waves + kCacheWaves - 1) / kCacheWaves)),
                     dim3(kCacheWaves * kWave), 0, s, a);
  return hipGetLastError();
}

template <int J, bool INDEXED>
hipError_t launch_cache_j(const CacheArgs& a, hipStream_t s) {
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  // the fewest steps per wave whose waves fit one round
  bool done = false;
  if ((e = try_one_round<J, INDEXED, 1>(a, di.cus, &done, s)) != hipSuccess || done) return e;
  if ((e = try_one_round<J, INDEXED, 2>(a, di.cus, &done, s)) != hipSuccess || done) return e;
  if ((e = try_one_round<J, INDEXED, 4>(a, di.cus, &done, s)) != hipSuccess || done) return e;
  // longer batches: four steps per wave, every resident wave, grid stride (one
  // or two steps per wave, and six or eight at fewer waves per SIMD, measured
  // slower)
  constexpr uint32_t SL = 4;
  uint64_t resident = 0;
  if ((e = resident_waves<J, INDEXED, SL, true>(di.cus, &resident)) != hipSuccess) return e;
  hipLaunchKernelGGL((k_gather_cache<J, INDEXED, SL, true>),
                     dim3((uint32_t)(resident / kCacheWaves)), dim3(kCacheWaves * kWave), 0, s, a);
  return hipGetLastError();
}

template <bool INDEXED>
hipError_t launch_cache(const Geometry& g, const CacheArgs& a, hipStream_t s) {
  switch (g.W) {
    case 64: return launch_cache_j<1, INDEXED>(a, s);
    case 128: return launch_cache_j<2, INDEXED>(a, s);
    case 256: return launch_cache_j<4, INDEXED>(a, s);
    default: return hipErrorInvalidValue;
  }
}

CacheArgs cache_args(const Geometry& g, const uint8_t* cache, uint64_t cache_bytes,
                     const int64_t* ids, uint64_t n_ids, uint64_t n_tensors,
                     const uint32_t* mask, const uint32_t* bitval, uint32_t* out) {
  CacheArgs a;
  a.cache = cache;
  a.cache_bytes = cache_bytes;
  a.offsets = nullptr;
  a.part_bits = nullptr;
  a.index = nullptr;
  a.n_tensors = n_tensors;
  a.ids = ids;
  a.n_ids = n_ids;
  a.mask = mask;
  a.bitval = bitval;
  a.out = out;
  a.align = 16;
  return a;
}

}  // namespace

bool cache_kernel_fits(const Geometry& g) {
  return g.n_c == 1 && (g.W == 64 || g.W == 128 || g.W == 256);
}

hipError_t launch_gather_cache_table(const Geometry& g, const uint8_t* cache, uint64_t cache_bytes,
                                     const uint64_t* offsets, const uint32_t* part_bits,
                                     uint64_t n_tensors, const int64_t* ids, uint64_t n_ids,
                                     const uint32_t* mask, const uint32_t* bitval, uint32_t* out,
                                     hipStream_t s) {
  if (n_ids == 0) return hipSuccess;
  CacheArgs a = cache_args(g, cache, cache_bytes, ids, n_ids, n_tensors, mask, bitval, out);
  a.offsets = offsets;
  a.part_bits = part_bits;
  return launch_cache<false>(g, a, s);
}

hipError_t launch_gather_cache_index(const Geometry& g, const uint8_t* cache, uint64_t cache_bytes,
                                     uint32_t entry_align, const uint64_t* index,
                                     uint64_t n_tensors, const int64_t* ids, uint64_t n_ids,
                                     const uint32_t* mask, const uint32_t* bitval, uint32_t* out,
                                     hipStream_t s) {
  if (n_ids == 0) return hipSuccess;
  // no tensors (and an empty index): every id is out of range, every row zero
  if (n_tensors == 0) return launch_fill_u32(out, n_ids * (uint64_t)g.W, 0u, s);
  CacheArgs a = cache_args(g, cache, cache_bytes, ids, n_ids, n_tensors, mask, bitval, out);
  a.index = index;
  a.align = entry_align;
  return launch_cache<true>(g, a, s);
}

}  // namespace ibp
