// ibp_plan.h -- per-kernel preparation of the Mask/Bitval metadata (gfx950).
//
// A "group" of G threads (G = 64, 128, ..., 1024) handles one tensor at a
// time.  Thread gl of a group owns the output words w = gl + G*j, j < J, for
// every tensor it touches, so everything that depends only on the metadata is
// computed once per workgroup and kept in that thread's registers:
//   - the five move masks of its words (ibp_device.h),
//   - Mask and Bitval of its words,
//   - `info`: the bit offset of the word's kept bits inside its chunk when the
//     chunk participates (low 16 bits) and inside its chunk when the chunk is
//     raw (high 16 bits, = 32 * word index in the chunk).
// The per-chunk payload sizes K_c (kept bits of a participating chunk) go to
// LDS, read by the lanes that own chunks ([G-EN] Core Algorithm: metadata is
// global, reused for every tensor; [JH]: one thread per chunk).
#pragma once

#include "ibp_device.h"

namespace ibp {

struct Shape {
  uint32_t W;          // 32-bit words per tensor
  uint32_t n_c;        // chunks per tensor (<= 64)
  uint32_t wpc_log2;   // log2(words per chunk)
  uint32_t last_bits;  // bits in the last chunk (the others have 32 << wpc_log2)
  uint32_t group;      // threads per tensor (multiple of 64)
};

__device__ __forceinline__ uint32_t chunk_bits(const Shape& sh, uint32_t c) {
  return c + 1 < sh.n_c ? (32u << sh.wpc_log2) : sh.last_bits;
}

template <int J>
struct WordRegs {
  uint32_t mv[J][5];
  uint32_t mask[J];
  uint32_t bitval[J];
  uint32_t info[J];
  uint32_t stages[J];  // wave-uniform: unpack stages with a non-zero move mask
};

// Workgroup-wide inclusive sum (blockDim.x a multiple of 64, <= 1024).
// s_wsum: 16 words of LDS.  Contains barriers: every thread must call it.
__device__ __forceinline__ uint32_t block_inclusive_sum(uint32_t v, uint32_t* s_wsum,
                                                        uint32_t* total) {
  const uint32_t incl = wave_inclusive_sum(v);
  const uint32_t wid = threadIdx.x / kWave, nw = blockDim.x / kWave;
  if (lane_id() == kWave - 1) s_wsum[wid] = incl;
  __syncthreads();
  uint32_t off = 0, tot = 0;
  for (uint32_t i = 0; i < nw; ++i) {
    const uint32_t s = s_wsum[i];
    off += i < wid ? s : 0u;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return incl + off;
}

// The plan is built in two parts, so that a kernel can issue its first
// payload loads between them:
//   load_plan_run +   the kept-bit prefix of every word (s_pref) and the kept
//   load_plan_counts  bits K_c of every chunk (s_kc), which the chunk scan
//                     needs; a workgroup scan, so every thread must call it;
//   load_plan_fetch   the Mask/Bitval words thread gl decodes, into registers;
//   load_plan_words   the per-word registers of thread gl from them (move
//                     masks, bit offsets in the chunk stream, wave-uniform
//                     stage flags): arithmetic and LDS reads only, no
//                     workgroup barrier.
// s_pref: W+1 words of LDS, s_kc: 64 words.  The exclusive prefix of kept
// bits over all words takes one workgroup scan: each thread sums a
// contiguous run of words, the runs are scanned, then each thread writes the
// prefixes of its run.
// Words per thread in the kept-bit scan: every launch has W <= 6 * threads
// (groups of G threads with G * 6 >= W; tile kernels: W <= 256 words, 256
// threads).
constexpr int kMaxRun = 6;

// The Mask words of this thread's contiguous run, loaded ahead of the
// counts (clamped, unconditional loads) so they can be requested before
// anything else is waited for.
struct PlanRun {
  uint32_t m[kMaxRun];
};

__device__ __forceinline__ void load_plan_run(const uint32_t* __restrict__ mask, const Shape& sh,
                                              PlanRun& r) {
  const uint32_t nt = blockDim.x, tid = threadIdx.x;
  const uint32_t per = (sh.W + nt - 1) / nt;
  const uint32_t w0 = min(tid * per, sh.W - 1u);
#pragma unroll
  for (int k = 0; k < kMaxRun; ++k) r.m[k] = mask[min(w0 + (uint32_t)k, sh.W - 1u)];
}

__device__ void load_plan_counts(const PlanRun& r, const Shape& sh, uint32_t* s_pref,
                                 uint32_t* s_kc, uint32_t* s_wsum) {
  const uint32_t nt = blockDim.x, tid = threadIdx.x;
  const uint32_t per = (sh.W + nt - 1) / nt;
  const uint32_t w0 = min(tid * per, sh.W), w1 = min(w0 + per, sh.W);
  uint32_t local = 0;
#pragma unroll
  for (int k = 0; k < kMaxRun; ++k)
    if (w0 + (uint32_t)k < w1) local += (uint32_t)__popc(~r.m[k]);
  uint32_t total;
  uint32_t run = block_inclusive_sum(local, s_wsum, &total) - local;
#pragma unroll
  for (int k = 0; k < kMaxRun; ++k) {
    if (w0 + (uint32_t)k < w1) {
      s_pref[w0 + k] = run;
      run += (uint32_t)__popc(~r.m[k]);
    }
  }
  if (tid == 0) s_pref[sh.W] = total;
  __syncthreads();
  for (uint32_t c = tid; c < sh.n_c; c += nt) {
    const uint32_t lo = c << sh.wpc_log2;
    const uint32_t hi = min((c + 1) << sh.wpc_log2, sh.W);
    s_kc[c] = s_pref[hi] - s_pref[lo];
  }
  __syncthreads();
}

// Mask and Bitval words of thread gl into R.mask / R.bitval (clamped,
// unconditional loads; words past W become 0 in load_plan_words).  Issued
// before the first payload loads, so that waiting for them never waits for a
// payload.
template <int J>
__device__ __forceinline__ void load_plan_fetch(const uint32_t* __restrict__ mask,
                                                const uint32_t* __restrict__ bitval,
                                                const Shape& sh, uint32_t gl, WordRegs<J>& R) {
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const uint32_t w = min(gl + sh.group * j, sh.W - 1u);
    R.mask[j] = mask[w];
    R.bitval[j] = bitval[w];
  }
}

template <int J>
__device__ void load_plan_words(const Shape& sh, const uint32_t* s_pref, uint32_t gl,
                                WordRegs<J>& R) {
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const uint32_t w = gl + sh.group * j;
    if (w < sh.W) {
      const uint32_t m = R.mask[j];
      move_masks(~m, R.mv[j]);
      R.bitval[j] &= m;
      const uint32_t first = (w >> sh.wpc_log2) << sh.wpc_log2;
      R.info[j] = (s_pref[w] - s_pref[first]) | ((32u * (w - first)) << 16);
    } else {
#pragma unroll
      for (int s = 0; s < 5; ++s) R.mv[j][s] = 0;
      R.mask[j] = 0;
      R.bitval[j] = 0;
      R.info[j] = 0;
    }
    uint32_t st = 0;
#pragma unroll
    for (int s = 0; s < 5; ++s) st |= (__ballot(R.mv[j][s] != 0u) != 0ull ? 1u : 0u) << s;
    R.stages[j] = uniform(st);
  }
}

// load_plan_words for a workgroup of four waves that all own the same words
// (lane l: words l + 64 j, j < J <= 4, as in the tile kernel): wave k
// computes the move masks of word position j = k from the Mask words it holds
// and shares them through LDS (s_mv: 5 * W words), so each wave does a
// quarter of that arithmetic.  Contains a workgroup barrier: every thread of
// the workgroup must call it.
template <int J>
__device__ void load_plan_words_shared(const Shape& sh, const uint32_t* s_pref, uint32_t lane,
                                       uint32_t wave, WordRegs<J>& R, uint32_t* s_mv) {
  static_assert(J <= 4, "one word position per wave of four");
  const uint32_t W = sh.W;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const uint32_t w = lane + (uint32_t)kWave * j;
    if (wave == (uint32_t)j && w < W) {
      uint32_t mv[5];
      move_masks(~R.mask[j], mv);
#pragma unroll
      for (int q = 0; q < 5; ++q) s_mv[q * W + w] = mv[q];
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const uint32_t w = lane + (uint32_t)kWave * j;
    if (w < W) {
      const uint32_t m = R.mask[j];
#pragma unroll
      for (int q = 0; q < 5; ++q) R.mv[j][q] = s_mv[q * W + w];
      R.bitval[j] &= m;
      const uint32_t first = (w >> sh.wpc_log2) << sh.wpc_log2;
      R.info[j] = (s_pref[w] - s_pref[first]) | ((32u * (w - first)) << 16);
    } else {
#pragma unroll
      for (int q = 0; q < 5; ++q) R.mv[j][q] = 0;
      R.mask[j] = 0;
      R.bitval[j] = 0;
      R.info[j] = 0;
    }
    uint32_t st = 0;
#pragma unroll
    for (int q = 0; q < 5; ++q) st |= (__ballot(R.mv[j][q] != 0u) != 0ull ? 1u : 0u) << q;
    R.stages[j] = uniform(st);
  }
}

// Synchronises the threads of one group: a wave, or the whole workgroup.
__device__ __forceinline__ void group_sync(bool single_wave) {
  if (single_wave)
    wave_sync();
  else
    __syncthreads();
}

// Per-group state shared between the chunk-owning wave and the others.
struct GroupHdr {
  uint64_t pmask;  // participation bits of the current tensor's chunks
  uint64_t addr;   // payload address
  uint32_t len;    // payload bytes
  uint32_t valid;  // id in range and a source for it
  uint64_t avail;  // whole 16 B units readable at addr, in bytes
};

}  // namespace ibp
