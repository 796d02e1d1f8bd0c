// Causal top-k per query row on gfx950.
//
// Selection rule (DSV2-Lite IndexCache card, intro: causal key selection with a budget of
// k tokens; DSA ablation card, "Benchmarks": a row shorter than k keeps every key):
// a row with n = p+1 <= k candidates keeps keys 0..p; otherwise the k largest scores,
// equal scores resolved toward the lower key index, -0.0 == +0.0.  Output ascending,
// -1 padded.
//
// Rows of up to 6144 keys: one wave per row (topk_short_kernel, below).  Longer rows:
// one 1024-thread workgroup per row.  Scores become order-preserving uint32 keys.  A radix
// select over LDS histograms finds the k-th largest key K*: the first pass bins the
// row's actual [min, max] key range into 2048 bins (so the populated bins spread out and
// LDS atomics rarely collide), later passes refine inside the threshold bin only, at
// most three passes in all.  Rows of up to 65536 keys stay in registers for every pass.
// The kept set (keys > K*, plus the lowest-index ties == K*) is marked in LDS bitmaps and
// emitted in index order from a block-wide prefix count of each thread's bit span.
#include "common.hpp"
#include "internal.hpp"
#include "selection.hpp"
#include "seglist.hpp"

namespace dsa {

namespace {

constexpr int NT = 1024;
constexpr int NWAVES = NT / 64;
constexpr int ITEMS = 64;               // keys per thread per segment
constexpr int SEG = NT * ITEMS;         // 65536 positions per segment
constexpr int NBINS = kSelBins;
constexpr int BIN_BITS = kSelBinBits;
constexpr int SEG_WORDS = SEG / 32;     // bitmap words per segment

// -0.0 and +0.0 share a key; larger floats get larger keys; 0 marks "no candidate".
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0) u = 0;  // canonical +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the workgroup in thread order; also returns the total.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* red, uint32_t& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t wsum;
  const uint32_t incl = wave_incl_scan_u32(v, &wsum);
  if (lane == 0) red[wid] = wsum;
  __syncthreads();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NWAVES; ++i) {
    const uint32_t r = red[i];
    pre += (i < wid) ? r : 0u;
    tot += r;
  }
  __syncthreads();
  total = tot;
  return pre + incl - v;
}

__device__ __forceinline__ uint32_t block_min(uint32_t v, uint32_t* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, (uint32_t)__shfl_xor(v, o, 64));
  if (lane == 0) red[wid] = v;
  __syncthreads();
  uint32_t r = red[0];
#pragma unroll
  for (int i = 1; i < NWAVES; ++i) r = min(r, red[i]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor(v, o, 64));
  if (lane == 0) red[wid] = v;
  __syncthreads();
  uint32_t r = red[0];
#pragma unroll
  for (int i = 1; i < NWAVES; ++i) r = max(r, red[i]);
  __syncthreads();
  return r;
}

template <bool CACHED>
__global__ __launch_bounds__(NT, 1) void topk_kernel(const float* __restrict__ scores, int64_t ld,
                                                      int64_t score_bstride, const int32_t* __restrict__ kv_len,
                                                      int Tq, int Tk, int k, int row0, int32_t* __restrict__ idx) {
  __shared__ uint32_t hist[NBINS];
  __shared__ uint32_t sel_bits[SEG_WORDS];
  __shared__ uint32_t tie_bits[SEG_WORDS];
  __shared__ uint32_t red[NWAVES];
  __shared__ uint32_t state[4];

  const int tid = threadIdx.x;
  const int r = blockIdx.x, b = blockIdx.y;
  const int64_t L = seq_len(kv_len, b, Tk);
  const int64_t p = L - Tq + row0 + r;
  const int64_t n = p + 1;  // candidates 0..p
  int32_t* out = idx + ((int64_t)b * Tq + row0 + r) * k;

  if (n <= k) {  // every causal key (or none), then padding
    for (int j = tid; j < k; j += NT) out[j] = (j < n) ? j : -1;
    return;
  }
  if (CACHED && n > SEG) return;  // launched only for rows that fit

  const float* row = scores + (int64_t)b * score_bstride + (int64_t)r * ld;
  const int nseg = CACHED ? 1 : (int)((n + SEG - 1) / SEG);
  constexpr int UNR = CACHED ? ITEMS : 8;  // cached keys need compile-time indices
  // key of item j of segment sg (0 = no candidate); range-checked buffer loads.
  // Positions are < 2^24 + 1, so 32-bit arithmetic suffices.
  const int n32 = (int)n;
  auto fetch = [&](int sg, int j) -> uint32_t {
    const int seg0 = sg * SEG;
    const int nrem = min(SEG, n32 - seg0);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(row + seg0, (uint32_t)nrem * 4u);
    const uint32_t key = order_key(buf_load_f32(rs, tid * 4u, (uint32_t)(NT * 4 * j)));
    return tid + NT * j < nrem ? key : 0u;
  };
  uint32_t keys[CACHED ? ITEMS : 1];
  if constexpr (CACHED) {
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) keys[j] = fetch(0, j);
  }
  auto key_at = [&](int sg, int j) -> uint32_t {
    if constexpr (CACHED) return keys[j];
    else return fetch(sg, j);
  };

  // range of the candidates' keys
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  for (int sg = 0; sg < nseg; ++sg) {
    _Pragma("nounroll") for (int j0 = 0; j0 < ITEMS; j0 += UNR) {
#pragma unroll
      for (int jj = 0; jj < UNR; ++jj) {
        const uint32_t key = key_at(sg, j0 + jj);
        kmin = min(kmin, key ? key : 0xFFFFFFFFu);
        kmax = max(kmax, key);
      }
    }
  }
  kmin = block_min(kmin, red);
  kmax = block_max(kmax, red);

  // radix select of the k-th largest key
  uint32_t lo = kmin, hi = kmax;
  const uint32_t span = kmax - kmin;
  int shift = span == 0 ? 0 : max(0, 32 - __clz(span) - BIN_BITS);
  uint32_t need = (uint32_t)k;  // how many to take from keys in [lo, hi]
  uint32_t kstar;
  for (;;) {
    for (int i = tid; i < NBINS; i += NT) hist[i] = 0;
    __syncthreads();
    for (int sg = 0; sg < nseg; ++sg) {
      _Pragma("nounroll") for (int j0 = 0; j0 < ITEMS; j0 += UNR) {
#pragma unroll
        for (int jj = 0; jj < UNR; ++jj) {
          const uint32_t key = key_at(sg, j0 + jj);
          if (key >= lo && key <= hi) atomicAdd(&hist[(key - lo) >> shift], 1u);
        }
      }
    }
    __syncthreads();
    // bins from the top: thread t covers bins 2047-2t and 2046-2t
    const int bh = NBINS - 1 - 2 * tid, bl = bh - 1;
    const uint32_t ch = hist[bh], cl = hist[bl];
    uint32_t tot;
    const uint32_t above = block_excl_scan(ch + cl, red, tot);
    if (above < need && need <= above + ch) {
      state[0] = (uint32_t)bh;
      state[1] = above;
    } else if (above + ch < need && need <= above + ch + cl) {
      state[0] = (uint32_t)bl;
      state[1] = above + ch;
    }
    __syncthreads();
    const uint32_t bstar = state[0];
    need -= state[1];
    lo = lo + (bstar << shift);
    if (shift == 0) {
      kstar = lo;
      break;
    }
    hi = (uint32_t)min((uint64_t)lo + ((1u << shift) - 1u), (uint64_t)hi);
    shift = max(0, shift - BIN_BITS);
    __syncthreads();
  }
  // need = number of ties (key == kstar) to keep, lowest indices first; k - need keys > kstar.
  // (kstar is a candidate's key, so kstar >= 1 and the 0 of non-candidates never matches.)

  uint32_t sel_before = 0, tie_before = 0;  // running counts over previous segments
  constexpr int WPT = SEG_WORDS / NT;        // bitmap words per thread (2)
  for (int sg = 0; sg < nseg; ++sg) {
    for (int i = tid; i < SEG_WORDS; i += NT) {
      sel_bits[i] = 0;
      tie_bits[i] = 0;
    }
    __syncthreads();
    _Pragma("nounroll") for (int j0 = 0; j0 < ITEMS; j0 += UNR) {
#pragma unroll
      for (int jj = 0; jj < UNR; ++jj) {
        const uint32_t key = key_at(sg, j0 + jj);
        const int e = tid + NT * (j0 + jj);  // position within the segment
        if (key > kstar) atomicOr(&sel_bits[e >> 5], 1u << (e & 31));
        else if (key == kstar) atomicOr(&tie_bits[e >> 5], 1u << (e & 31));
      }
    }
    __syncthreads();
    uint32_t sw[WPT], tw[WPT];
    uint32_t cs = 0, ct = 0;
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      sw[i] = sel_bits[tid * WPT + i];
      tw[i] = tie_bits[tid * WPT + i];
      cs += __popc(sw[i]);
      ct += __popc(tw[i]);
    }
    uint32_t ts, tt;
    uint32_t sp = block_excl_scan(cs, red, ts) + sel_before;
    uint32_t tp = block_excl_scan(ct, red, tt) + tie_before;
    const int pos0 = sg * SEG + tid * WPT * 32;
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      uint32_t m = sw[i] | tw[i];
      while (m) {
        const int bit = __ffs(m) - 1;
        m &= m - 1;
        const int32_t pos = pos0 + i * 32 + bit;
        // slots stay below k by construction (k - need keys above kstar); the guard only
        // keeps a violated invariant from writing outside this row
        if ((sw[i] >> bit) & 1u) {
          const uint32_t slot = sp + min(tp, need);
          if (slot < (uint32_t)k) out[slot] = pos;
          ++sp;
        } else {
          if (tp < need && sp + tp < (uint32_t)k) out[sp + tp] = pos;
          ++tp;
        }
      }
    }
    sel_before += ts;
    tie_before += tt;
    __syncthreads();
  }
}

// Rows of up to one segment (65536 keys), keys in registers (64 per thread).
//
// 1. A sample of 8 keys per thread (slots spread over the whole row) is histogrammed to
//    pick a threshold T0 expected to keep about 2k keys.
// 2. Each thread marks its keys >= T0 in a 64-bit mask; one block scan of the mask counts
//    gives every thread its place in an LDS candidate list (no atomics).
// 3. If k <= #candidates <= kCandCap, one wave runs an exact radix select on the list and
//    marks the kept keys (> K*) and the ties (== K*) in LDS bitmaps.  Otherwise (a poor
//    sample, or massive ties) the whole workgroup runs the exact radix select over the
//    registers.
// 4. The bitmaps are emitted in position order from a block-wide prefix count.
constexpr int kCandCap = 8192;
constexpr int kSamples = 8;  // per thread

// Row r of the chunk in sequence b, by one 1024-thread workgroup (also the split route's
// exact fallback).
__device__ __forceinline__ void topk_fast_row(const float* __restrict__ scores, int64_t ld, int64_t score_bstride,
                                              const int32_t* __restrict__ kv_len, int Tq, int Tk, int k, int row0,
                                              int32_t* __restrict__ idx, int r, int b) {
  __shared__ uint32_t hist[NBINS];
  __shared__ __attribute__((aligned(8))) uint32_t sel_bits[SEG_WORDS];
  __shared__ __attribute__((aligned(8))) uint32_t tie_bits[SEG_WORDS];
  __shared__ uint32_t cand_key[kCandCap + 1];  // last slot absorbs non-candidate writes
  __shared__ int32_t cand_pos[kCandCap + 1];
  __shared__ uint32_t red[3 * NWAVES];
  __shared__ uint32_t state[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int64_t L = seq_len(kv_len, b, Tk);
  const int64_t p = L - Tq + row0 + r;
  int32_t* out = idx + ((int64_t)b * Tq + row0 + r) * k;
  if (p + 1 <= k) {  // every causal key (or none), then padding
    for (int j = tid; j < k; j += NT) out[j] = (j <= p) ? j : -1;
    return;
  }
  if (p + 1 > SEG) return;  // launched only for rows that fit
  const int n = (int)(p + 1);
  const int nj = (n + NT - 1) / NT;  // item slots in use (uniform)

  // ---- keys: batched range-checked loads (slots past the row read 0 and are zeroed)
  const float* row = scores + (int64_t)b * score_bstride + (int64_t)r * ld;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(row, (uint32_t)n * 4u);
  uint32_t keys[ITEMS];
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) keys[j] = __float_as_uint(buf_load_f32(rs, tid * 4u, (uint32_t)(NT * 4 * j)));
  // slots are handled in blocks of 8 (8192 positions); a block past the row is skipped
  // with one uniform branch (per-slot branches would pin 64 conditions in scalar registers)
  constexpr int JB = 8;
#pragma unroll
  for (int jb = 0; jb < ITEMS / JB; ++jb) {
    if (jb * JB < nj) {
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        const int j = jb * JB + jj;
        // order-preserving map; adding +0 first turns -0 into +0, so the two tie
        const uint32_t u = __float_as_uint(__uint_as_float(keys[j]) + 0.0f);
        const uint32_t key = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
        keys[j] = (tid + NT * j < n) ? key : 0u;  // 0 marks "no candidate"
      }
    } else {
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) keys[jb * JB + jj] = 0u;
    }
  }
  for (int i = tid; i < SEG_WORDS; i += NT) {
    sel_bits[i] = 0;
    tie_bits[i] = 0;
  }
  for (int i = tid; i < NBINS; i += NT) hist[i] = 0;

  // ---- 1. sample: thread t takes slots (t % 8) + 8m, m = 0..7
  uint32_t smp[kSamples];
#pragma unroll
  for (int m = 0; m < kSamples; ++m) {
    uint32_t v = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) v = ((tid & 7) == q) ? keys[8 * m + q] : v;
    smp[m] = v;
  }
  uint32_t smin = 0xFFFFFFFFu, smax = 0u, scount = 0;
#pragma unroll
  for (int m = 0; m < kSamples; ++m) {
    smin = min(smin, smp[m] - 1u);  // 0 (no candidate) wraps to the top and drops out
    smax = max(smax, smp[m]);
    scount += smp[m] != 0u;
  }
  smin = wave_min_u32(smin);
  smax = wave_max_u32(smax);
  scount = wave_sum_u32(scount);
  if (lane == 0) {
    red[wave] = smin;
    red[NWAVES + wave] = smax;
    red[2 * NWAVES + wave] = scount;
  }
  __syncthreads();
  smin = red[0];
  smax = red[NWAVES];
  scount = red[2 * NWAVES];
#pragma unroll
  for (int i = 1; i < NWAVES; ++i) {
    smin = min(smin, red[i]);
    smax = max(smax, red[NWAVES + i]);
    scount += red[2 * NWAVES + i];
  }
  smin += 1u;
  const uint32_t sspan = smax - smin;
  const int sshift = sspan == 0 ? 0 : max(0, 32 - __clz(sspan) - BIN_BITS);
#pragma unroll
  for (int m = 0; m < kSamples; ++m)
    if (smp[m]) atomicAdd(&hist[(smp[m] - smin) >> sshift], 1u);
  __syncthreads();
  if (wave == 0) {
    // aim at about twice k keys: the bin where the sampled count from the top reaches
    // 2k * (samples / n)
    uint32_t target = (uint32_t)min((uint64_t)scount, ((uint64_t)2 * k * scount + n - 1) / n);
    target = max(target, 1u);
    uint32_t bin, above;
    wave_find_bin_from_top(hist, target, bin, above);
    if (lane == 0) state[0] = smin + (bin << sshift);
  }
  __syncthreads();
  const uint32_t t0 = state[0];  // >= smin >= 1

  // ---- 2. candidates: keys >= t0, placed by one block scan of per-thread counts
  uint32_t ccount = 0;
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) ccount += keys[j] >= t0;
  uint32_t c0;
  const uint32_t cbase = block_excl_scan(ccount, red, c0);

  uint32_t need = (uint32_t)k;
  uint32_t kstar;
  if (c0 >= (uint32_t)k && c0 <= (uint32_t)kCandCap) {
    // (t0 re-read after the scan's barriers: the compares are redone here rather than
    // 64 results kept live across the scan)
    const uint32_t t0c = state[0];
    uint32_t off = cbase, cmax = 0;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const bool c = keys[j] >= t0c;
      const uint32_t slot = c ? off : (uint32_t)kCandCap;
      cand_key[slot] = keys[j];
      cand_pos[slot] = tid + NT * j;
      off += c;
      cmax = max(cmax, keys[j]);
    }
    cmax = wave_max_u32(cmax);
    for (int i = tid; i < NBINS; i += NT) hist[i] = 0;
    if (lane == 0) red[2 * NWAVES + wave] = cmax;
    if (tid == 0) state[2] = 0;  // members of the threshold bin
    __syncthreads();
    cmax = red[2 * NWAVES];
#pragma unroll
    for (int i = 1; i < NWAVES; ++i) cmax = max(cmax, red[2 * NWAVES + i]);
    // block-wide radix passes over the list until the threshold bin is small
    uint32_t lo = t0c, hi = cmax;
    int sh = (hi == lo) ? 0 : max(0, 32 - __clz(hi - lo) - BIN_BITS);
    uint32_t m;
    for (;;) {
      for (uint32_t c = tid; c < c0; c += NT) {
        const uint32_t key = cand_key[c];
        if (key >= lo && key <= hi) atomicAdd(&hist[(key - lo) >> sh], 1u);
      }
      __syncthreads();
      if (wave == 0) {
        uint32_t bin, above;
        wave_find_bin_from_top(hist, need, bin, above);
        if (lane == 0) {
          state[0] = bin;
          state[1] = above;
          state[3] = hist[bin];
        }
      }
      __syncthreads();
      const uint32_t bin = state[0];
      m = state[3];
      const uint32_t blo = lo + (bin << sh);
      const uint32_t bhi = (uint32_t)min((uint64_t)blo + ((1u << sh) - 1u), (uint64_t)hi);
      // keys above the threshold bin are kept
      for (uint32_t c = tid; c < c0; c += NT) {
        const uint32_t key = cand_key[c];
        if (key > bhi && key <= hi) {
          const int e = cand_pos[c];
          atomicOr(&sel_bits[e >> 5], 1u << (e & 31));
        }
      }
      need -= state[1];
      lo = blo;
      hi = bhi;
      if (sh == 0 || m <= 64) break;
      sh = max(0, sh - BIN_BITS);
      for (int i = tid; i < NBINS; i += NT) hist[i] = 0;
      __syncthreads();
    }
    if (sh > 0 || m <= 64) {
      // the threshold bin's m <= 64 members: rank them exactly (score, then position)
      // in one wave and keep the first `need`
      __shared__ uint32_t mem_key[64];
      __shared__ int32_t mem_pos[64];
      for (uint32_t c = tid; c < c0; c += NT) {
        const uint32_t key = cand_key[c];
        if (key >= lo && key <= hi) {
          const uint32_t slot = atomicAdd(&state[2], 1u);
          mem_key[slot] = key;
          mem_pos[slot] = cand_pos[c];
        }
      }
      __syncthreads();
      if (wave == 0) {
        const uint32_t mk = lane < (int)m ? mem_key[lane] : 0u;
        const int32_t mp = lane < (int)m ? mem_pos[lane] : 0x7FFFFFFF;
        uint32_t rank = 0;
        for (uint32_t j = 0; j < m; ++j) {
          const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)mk, (int)j);
          const int32_t pj = __builtin_amdgcn_readlane(mp, (int)j);
          rank += (kj > mk) || (kj == mk && pj < mp);
        }
        if (lane < (int)m && rank < need) atomicOr(&sel_bits[mp >> 5], 1u << (mp & 31));
      }
      need = 0;  // every kept key is in sel_bits
    } else {
      // a threshold bin of one key value held by more than 64 candidates: its members
      // are ties; keep the first `need` by position
      kstar = lo;
      for (uint32_t c = tid; c < c0; c += NT) {
        const uint32_t key = cand_key[c];
        if (key == kstar) {
          const int e = cand_pos[c];
          atomicOr(&tie_bits[e >> 5], 1u << (e & 31));
        }
      }
    }
    __syncthreads();
  } else {
    // exact radix select over the registers, by the whole workgroup
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      kmin = min(kmin, keys[j] - 1u);
      kmax = max(kmax, keys[j]);
    }
    kmin = wave_min_u32(kmin);
    kmax = wave_max_u32(kmax);
    if (lane == 0) {
      red[wave] = kmin;
      red[NWAVES + wave] = kmax;
    }
    __syncthreads();
    kmin = red[0];
    kmax = red[NWAVES];
#pragma unroll
    for (int i = 1; i < NWAVES; ++i) {
      kmin = min(kmin, red[i]);
      kmax = max(kmax, red[NWAVES + i]);
    }
    kmin += 1u;
    uint32_t lo = kmin, hi = kmax;
    int sh = (kmax == kmin) ? 0 : max(0, 32 - __clz(kmax - kmin) - BIN_BITS);
    for (;;) {
      for (int i = tid; i < NBINS; i += NT) hist[i] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < ITEMS; ++j) {
        const uint32_t key = keys[j];
        if (key && key >= lo && key <= hi) atomicAdd(&hist[(key - lo) >> sh], 1u);
      }
      __syncthreads();
      if (wave == 0) {
        uint32_t bin, above;
        wave_find_bin_from_top(hist, need, bin, above);
        if (lane == 0) {
          state[0] = bin;
          state[1] = above;
        }
      }
      __syncthreads();
      need -= state[1];
      lo += state[0] << sh;
      if (sh == 0) break;
      hi = (uint32_t)min((uint64_t)lo + ((1u << sh) - 1u), (uint64_t)hi);
      sh = max(0, sh - BIN_BITS);
      __syncthreads();
    }
    kstar = lo;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const uint32_t key = keys[j];
      const int e = tid + NT * j;
      if (key > kstar) atomicOr(&sel_bits[e >> 5], 1u << (e & 31));
      else if (key == kstar && key) atomicOr(&tie_bits[e >> 5], 1u << (e & 31));
    }
    __syncthreads();
  }
  // need = ties (key == kstar) to keep, lowest positions first; k - need keys > kstar

  // ---- 4. emission in position order: thread t owns positions 64t .. 64t+63
  constexpr int WPT = SEG_WORDS / NT;  // 2 bitmap words per thread
  uint32_t sw[WPT], tw[WPT];
  uint32_t cs = 0, ct = 0;
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    sw[i] = sel_bits[tid * WPT + i];
    tw[i] = tie_bits[tid * WPT + i];
    cs += __popc(sw[i]);
    ct += __popc(tw[i]);
  }
  // one scan for both counts: kept-above count (< 4096) in the high bits, ties below
  uint32_t tot;
  const uint32_t packed = block_excl_scan((cs << 17) | ct, red, tot);
  uint32_t sp = packed >> 17, tp = packed & 0x1FFFFu;
  const int pos0 = tid * WPT * 32;
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    uint32_t m = sw[i] | tw[i];
    while (m) {
      const int bit = __ffs(m) - 1;
      m &= m - 1;
      const int32_t pos = pos0 + i * 32 + bit;
      // slots stay below k by construction; the guard keeps a violated invariant in-row
      if ((sw[i] >> bit) & 1u) {
        const uint32_t slot = sp + min(tp, need);
        if (slot < (uint32_t)k) out[slot] = pos;
        ++sp;
      } else {
        if (tp < need && sp + tp < (uint32_t)k) out[sp + tp] = pos;
        ++tp;
      }
    }
  }
}

__global__ __launch_bounds__(NT, 1) void topk_fast_kernel(const float* __restrict__ scores, int64_t ld,
                                                          int64_t score_bstride, const int32_t* __restrict__ kv_len,
                                                          int Tq, int Tk, int k, int row0, int32_t* __restrict__ idx) {
  topk_fast_row(scores, ld, score_bstride, kv_len, Tq, Tk, k, row0, idx, blockIdx.x, blockIdx.y);
}

// ---------------------------------------------------------------------------------------
// Streaming top-k for rows of up to 65536 keys: 256 threads per row and few registers, so
// several rows share a CU and one row's loads overlap another's selection.
//
// 1. Threshold: 4096 scores from 256 blocks of 16 positions spread over the row are binned
//    twice (2048 bins over their range, then inside the chosen bin); the m-th largest
//    sample, m = alpha*k*4096/n, is a threshold expected to keep about alpha*k keys
//    (alpha = 1.31 for k = 2048).
// 2. Filter: one coalesced 16-byte-per-lane pass over the row appends every key >= the
//    threshold to an LDS candidate list.  Each wave fills its own quarter of the list from
//    a wave-uniform counter (ballots place the lanes), so no atomic sits on the path.
// 3. If k <= candidates <= capacity, the k largest keys of the whole row are exactly the k
//    largest candidates (every key at or above the k-th largest passed the filter), and a
//    radix select over the list marks them in position bitmaps.  A sample that misjudged
//    the row (too few candidates, or an overflowing list: scores with positional structure
//    can do that) has its rank m rescaled by the count the filter saw, and the filter runs
//    again, up to three passes in all; after that an exact radix select streams the row
//    from global memory.
// 4. The bitmaps are emitted in position order from a block-wide prefix count.
constexpr int ST_NT = 256;
constexpr int ST_NW = ST_NT / 64;
constexpr int ST_CAP = 3584;                    // candidate list entries
constexpr int ST_WCAP = ST_CAP / ST_NW;         // entries per wave (896)
constexpr int ST_DUMMY = ST_CAP;                // + 256 slots where lanes without a candidate write
// Rows up to this length keep every key: wave w takes positions 256w .. 256w+255 of each
// 1024, so its part of the list then holds at most 3*256 + 128 = ST_WCAP of them.
constexpr int ST_KEEP = (ST_WCAP / 256) * 4 * 256 + ST_WCAP % 256;
constexpr int ST_SBLK = 256, ST_SLEN = 16;      // sampled blocks (one per thread) and their length
constexpr int ST_SAMPLES = ST_SBLK * ST_SLEN;   // 4096, 16 per thread
constexpr int ST_WPT = SEG_WORDS / ST_NT;       // 8 bitmap words per thread
constexpr int ST_U = 8;                         // 16-byte loads in flight per thread

__device__ __forceinline__ uint32_t st_excl_scan(uint32_t v, uint32_t* red, uint32_t& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t wsum;
  const uint32_t incl = wave_incl_scan_u32(v, &wsum);
  if (lane == 0) red[wid] = wsum;
  __syncthreads();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < ST_NW; ++i) {
    const uint32_t r = red[i];
    pre += (i < wid) ? r : 0u;
    tot += r;
  }
  __syncthreads();
  total = tot;
  return pre + incl - v;
}

// min and max over the workgroup (one barrier pair)
__device__ __forceinline__ void st_minmax(uint32_t& mn, uint32_t& mx, uint32_t* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  if (lane == 0) {
    red[wid] = mn;
    red[ST_NW + wid] = mx;
  }
  __syncthreads();
  mn = red[0];
  mx = red[ST_NW];
#pragma unroll
  for (int i = 1; i < ST_NW; ++i) {
    mn = min(mn, red[i]);
    mx = max(mx, red[ST_NW + i]);
  }
  __syncthreads();
}

__device__ __forceinline__ uint32_t st_key(float f) { return sel_key(f); }

__global__ __launch_bounds__(ST_NT, 4) void topk_stream_kernel(const float* __restrict__ scores, int64_t ld,
                                                              int64_t score_bstride, const int32_t* __restrict__ kv_len,
                                                              int Tq, int Tk, int k, int row0, int32_t* __restrict__ idx) {
  // 40 KB of LDS: four rows per CU.  The tie bitmap reuses the histogram, which is
  // cleared once the last histogram pass is done.
  __shared__ uint32_t hist[NBINS];
  __shared__ uint32_t sel_bits[SEG_WORDS];
  uint32_t* const tie_bits = hist;
  static_assert(NBINS == SEG_WORDS, "tie bitmap aliases the histogram");
  __shared__ uint32_t cand_key[ST_CAP + 256];
  __shared__ uint16_t cand_pos[ST_CAP + 256];  // positions < 65536
  __shared__ uint32_t mem_key[64];
  __shared__ int32_t mem_pos[64];
  __shared__ uint32_t red[2 * ST_NW];
  __shared__ uint32_t state[4];
  __shared__ uint32_t wcount[ST_NW];  // candidates each wave appended

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int r = blockIdx.x, b = blockIdx.y;
  const int64_t L = seq_len(kv_len, b, Tk);
  const int64_t p = L - Tq + row0 + r;
  int32_t* out = idx + ((int64_t)b * Tq + row0 + r) * k;
  if (p + 1 <= k) {  // every causal key (or none), then padding
    for (int j = tid; j < k; j += ST_NT) out[j] = (j <= p) ? j : -1;
    return;
  }
  if (p + 1 > SEG) return;  // launched only for rows that fit
  const int n = (int)(p + 1);
  // slot c of the list is in use iff it lies below its wave's count
  auto in_list = [&](int c) { return (uint32_t)(c % ST_WCAP) < wcount[c / ST_WCAP]; };
  const float* row = scores + (int64_t)b * score_bstride + (int64_t)r * ld;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(row, (uint32_t)n * 4u);
  // four scores at pos0 .. pos0+3 (pos0 a multiple of 4): one 16-byte load where the row
  // is 16-byte aligned (ld is free in the API), and dword loads for a group that crosses
  // the end of the row, so no load depends on how a partly out-of-range access is handled
  const bool al16 = ((uintptr_t)row & 15u) == 0;
  auto load4 = [&](int pos0) -> u32x4 {
    u32x4 v;
    if (al16 && pos0 + 4 <= n) {
      v = buf_load_16(rs, (uint32_t)pos0 * 4u, 0);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = __float_as_uint(buf_load_f32(rs, (uint32_t)(pos0 + e) * 4u, 0));
    }
    return v;
  };

  for (int i = tid; i < SEG_WORDS; i += ST_NT) sel_bits[i] = 0;
  for (int i = tid; i < NBINS; i += ST_NT) hist[i] = 0;
  if (tid < 4) state[tid] = 0;

  // ---- 1. the sample: thread t reads the 16 scores of block t (rows up to ST_KEEP keys
  // keep every key and need no sample)
  uint32_t sk[16];
  uint32_t smin = 0xFFFFFFFFu, smax = 0u;
  int ssh = 0;  // bin shift of the sample's range
  if (n > ST_KEEP) {
    const int base = (int)(((int64_t)tid * (n - ST_SLEN)) / (ST_SBLK - 1)) & ~3;  // base + 16 <= n
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const u32x4 v = load4(base + 4 * qd);
#pragma unroll
      for (int e = 0; e < 4; ++e) sk[4 * qd + e] = st_key(__uint_as_float(v[e]));
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      smin = min(smin, sk[i]);
      smax = max(smax, sk[i]);
    }
    st_minmax(smin, smax, red);  // (its barriers also order the clears above)
    ssh = smax == smin ? 0 : max(0, 32 - __clz(smax - smin) - BIN_BITS);
  }
  // The m-th largest sample, within 2^(ssh-11) keys (two histogram passes; a bin edge alone
  // could keep half again as many candidates).  The histogram is zero before and after.
  auto threshold = [&](uint32_t m) -> uint32_t {
    const int sh = ssh;
#pragma unroll
    for (int i = 0; i < 16; ++i) atomicAdd(&hist[(sk[i] - smin) >> sh], 1u);
    __syncthreads();
    if (wave == 0) {
      uint32_t bin, above;
      wave_find_bin_from_top(hist, m, bin, above);
      if (lane == 0) {
        state[0] = bin;
        state[1] = above;
      }
    }
    __syncthreads();
    const uint32_t blo = smin + (state[0] << sh);
    const uint32_t bhi = (uint32_t)min((uint64_t)blo + ((1u << sh) - 1u), (uint64_t)smax);
    const uint32_t m2 = m - state[1];
    uint32_t th = blo;
    if (sh > 0) {
      for (int i = tid; i < NBINS; i += ST_NT) hist[i] = 0;
      __syncthreads();
      const int sh2 = max(0, sh - BIN_BITS);
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (sk[i] >= blo && sk[i] <= bhi) atomicAdd(&hist[(sk[i] - blo) >> sh2], 1u);
      __syncthreads();
      if (wave == 0) {
        uint32_t bin, above;
        wave_find_bin_from_top(hist, m2, bin, above);
        if (lane == 0) state[0] = blo + (bin << sh2);
      }
      __syncthreads();
      th = state[0];
    }
    for (int i = tid; i < NBINS; i += ST_NT) hist[i] = 0;
    __syncthreads();
    return th;
  };

  // ---- 2. filter: keys >= theta go to this wave's part of the candidate list.  Every lane
  // stores every step (no branches): a lane without a candidate writes a dummy slot of its
  // own past the list.  A slot past the wave's part is clamped to its last entry: that only
  // happens on overflow, and an overflowing list is not used.  Returns the count of keys
  // >= theta (all of them, also past the capacity); `overflow`: some wave's part overflowed.
  bool overflow = false;
  auto filter = [&](uint32_t theta) -> uint32_t {
    const int nit = (n + 4 * ST_NT - 1) / (4 * ST_NT);
    const int nfull = n / (4 * ST_NT);  // steps whose 1024 positions all lie in the row
    uint32_t wcnt = 0;                  // wave-uniform
    const int dslot = ST_DUMMY + wave * 64 + lane;
    auto step = [&](const u32x4& v, int pos0, bool tail) {
      uint32_t tot = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t key = st_key(__uint_as_float(v[e]));
        if (tail) key = (pos0 + e < n) ? key : 0u;
        const bool c = key >= theta;
        const uint64_t bal = __ballot(c);
        const uint32_t slot =
            wcnt + tot + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
        int at = c ? wave * ST_WCAP + (int)min(slot, (uint32_t)ST_WCAP - 1u) : dslot;
        asm volatile("" : "+v"(at));  // keep the select: one store per array, not two masked ones
        cand_key[at] = key;
        cand_pos[at] = (uint16_t)(pos0 + e);
        tot += (uint32_t)__popcll(bal);
      }
      wcnt += tot;
    };
    for (int it0 = 0; it0 < nit; it0 += ST_U) {
      u32x4 v[ST_U];
      if (al16 && it0 + ST_U <= nfull) {  // uniform: whole 16-byte groups inside the row
#pragma unroll
        for (int u = 0; u < ST_U; ++u) v[u] = buf_load_16(rs, (uint32_t)((it0 + u) * 4 * ST_NT + 4 * tid) * 4u, 0);
#pragma unroll
        for (int u = 0; u < ST_U; ++u) step(v[u], (it0 + u) * 4 * ST_NT + 4 * tid, false);
      } else {
#pragma unroll
        for (int u = 0; u < ST_U; ++u) v[u] = load4((it0 + u) * 4 * ST_NT + 4 * tid);  // past n: zeros
#pragma unroll
        for (int u = 0; u < ST_U; ++u)
          if (it0 + u < nit) step(v[u], (it0 + u) * 4 * ST_NT + 4 * tid, true);
      }
    }
    if (lane == 0) {
      wcount[wave] = min(wcnt, (uint32_t)ST_WCAP);
      red[wave] = wcnt;
    }
    __syncthreads();
    uint32_t cnt = 0;
    overflow = false;
#pragma unroll
    for (int i = 0; i < ST_NW; ++i) {
      cnt += red[i];
      overflow |= red[i] > (uint32_t)ST_WCAP;
    }
    __syncthreads();
    return cnt;
  };

  uint32_t c0;
  if (n <= ST_KEEP) {
    c0 = filter(1u);  // every key is >= 1
  } else {
    const float alpha = fminf(1.5f, 0.75f * ST_CAP / (float)k);
    float m = fminf((float)ST_SAMPLES, ceilf(alpha * (float)k * (float)ST_SAMPLES / (float)n));
    for (int attempt = 0;; ++attempt) {  // uniform: every quantity below is the workgroup's
      c0 = filter(threshold((uint32_t)fmaxf(1.f, m)));
      if ((c0 >= (uint32_t)k && !overflow) || attempt == 2) break;
      // rescale the sample rank by what the filter saw
      const float target = alpha * (float)k;
      m = fminf((float)ST_SAMPLES, fmaxf(1.f, ceilf(m * target / fmaxf(1.f, (float)c0))));
    }
  }
  if (tid == 0) state[2] = 0;  // members of the final bin (exact ranking)

  // ---- 3. exact selection
  uint32_t need = (uint32_t)k;
  if (c0 >= (uint32_t)k && !overflow) {
    uint32_t cmin = 0xFFFFFFFFu, cmax = 0u;
    for (int c = tid; c < ST_CAP; c += ST_NT)
      if (in_list(c)) {
        cmin = min(cmin, cand_key[c]);
        cmax = max(cmax, cand_key[c]);
      }
    st_minmax(cmin, cmax, red);
    uint32_t lo = cmin, hi = cmax;
    int sh = (hi == lo) ? 0 : max(0, 32 - __clz(hi - lo) - BIN_BITS);
    uint32_t m;
    for (;;) {
      for (int c = tid; c < ST_CAP; c += ST_NT) {
        const uint32_t key = cand_key[c];
        if (in_list(c) && key >= lo && key <= hi) atomicAdd(&hist[(key - lo) >> sh], 1u);
      }
      __syncthreads();
      if (wave == 0) {
        uint32_t bin, above;
        wave_find_bin_from_top(hist, need, bin, above);
        if (lane == 0) {
          state[0] = bin;
          state[1] = above;
          state[3] = hist[bin];
        }
      }
      __syncthreads();
      const uint32_t bin = state[0];
      m = state[3];
      const uint32_t blo = lo + (bin << sh);
      const uint32_t bhi = (uint32_t)min((uint64_t)blo + ((1u << sh) - 1u), (uint64_t)hi);
      // keys above the threshold bin are kept
      for (int c = tid; c < ST_CAP; c += ST_NT) {
        const uint32_t key = cand_key[c];
        if (in_list(c) && key > bhi && key <= hi) {
          const int e = cand_pos[c];
          atomicOr(&sel_bits[e >> 5], 1u << (e & 31));
        }
      }
      need -= state[1];
      lo = blo;
      hi = bhi;
      if (sh == 0 || m <= 64) break;
      sh = max(0, sh - BIN_BITS);
      for (int i = tid; i < NBINS; i += ST_NT) hist[i] = 0;
      __syncthreads();
    }
    __syncthreads();  // last histogram reads done: it becomes the (empty) tie bitmap
    for (int i = tid; i < NBINS; i += ST_NT) hist[i] = 0;
    __syncthreads();
    if (sh > 0 || m <= 64) {
      // the final bin's m <= 64 members: rank them exactly (score, then position) in one
      // wave and keep the first `need`
      for (int c = tid; c < ST_CAP; c += ST_NT) {
        const uint32_t key = cand_key[c];
        if (in_list(c) && key >= lo && key <= hi) {
          const uint32_t slot = atomicAdd(&state[2], 1u);
          mem_key[slot] = key;
          mem_pos[slot] = cand_pos[c];
        }
      }
      __syncthreads();
      if (wave == 0) {
        const uint32_t mk = lane < (int)m ? mem_key[lane] : 0u;
        const int32_t mp = lane < (int)m ? mem_pos[lane] : 0x7FFFFFFF;
        uint32_t rank = 0;
        for (uint32_t j = 0; j < m; ++j) {
          const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)mk, (int)j);
          const int32_t pj = __builtin_amdgcn_readlane(mp, (int)j);
          rank += (kj > mk) || (kj == mk && pj < mp);
        }
        if (lane < (int)m && rank < need) atomicOr(&sel_bits[mp >> 5], 1u << (mp & 31));
      }
      need = 0;  // every kept key is in sel_bits
    } else {
      // a final bin of one key value held by more than 64 candidates: its members are
      // ties; keep the first `need` by position
      const uint32_t kstar = lo;
      for (int c = tid; c < ST_CAP; c += ST_NT) {
        if (in_list(c) && cand_key[c] == kstar) {
          const int e = cand_pos[c];
          atomicOr(&tie_bits[e >> 5], 1u << (e & 31));
        }
      }
    }
    __syncthreads();
  } else {
    // exact radix select over the whole row, re-read from global memory for each pass:
    // three passes of 11, 11 and 10 bits from the top of the key
    uint32_t lo = 1u, hi = 0xFFFFFFFFu;
    int sh = 32 - BIN_BITS;
    for (;;) {
      for (int i = tid; i < NBINS; i += ST_NT) hist[i] = 0;
      __syncthreads();
      for (int pos0 = 4 * tid; pos0 < n; pos0 += 4 * ST_NT) {
        const u32x4 v = load4(pos0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t key = (pos0 + e < n) ? st_key(__uint_as_float(v[e])) : 0u;
          if (key >= lo && key <= hi) atomicAdd(&hist[(key - lo) >> sh], 1u);
        }
      }
      __syncthreads();
      if (wave == 0) {
        uint32_t bin, above;
        wave_find_bin_from_top(hist, need, bin, above);
        if (lane == 0) {
          state[0] = bin;
          state[1] = above;
        }
      }
      __syncthreads();
      need -= state[1];
      lo += state[0] << sh;
      if (sh == 0) break;
      hi = (uint32_t)min((uint64_t)lo + ((1u << sh) - 1u), (uint64_t)hi);
      sh = max(0, sh - BIN_BITS);
      __syncthreads();
    }
    __syncthreads();  // last histogram reads done: it becomes the (empty) tie bitmap
    for (int i = tid; i < NBINS; i += ST_NT) hist[i] = 0;
    __syncthreads();
    const uint32_t kstar = lo;
    for (int pos0 = 4 * tid; pos0 < n; pos0 += 4 * ST_NT) {
      const u32x4 v = load4(pos0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pos = pos0 + e;
        const uint32_t key = (pos < n) ? st_key(__uint_as_float(v[e])) : 0u;
        if (key > kstar) atomicOr(&sel_bits[pos >> 5], 1u << (pos & 31));
        else if (key == kstar && key) atomicOr(&tie_bits[pos >> 5], 1u << (pos & 31));
      }
    }
    __syncthreads();
  }
  // need = ties (key == kstar) to keep, lowest positions first; k - need keys above

  // ---- 4. emission in position order: thread t owns positions 256t .. 256t+255
  uint32_t sw[ST_WPT], tw[ST_WPT];
  uint32_t cs = 0, ct = 0;
#pragma unroll
  for (int i = 0; i < ST_WPT; ++i) {
    sw[i] = sel_bits[tid * ST_WPT + i];
    tw[i] = tie_bits[tid * ST_WPT + i];
    cs += __popc(sw[i]);
    ct += __popc(tw[i]);
  }
  // one scan for both counts: kept-above count (< 4096) in the high bits, ties below
  uint32_t tot;
  const uint32_t packed = st_excl_scan((cs << 17) | ct, red, tot);
  uint32_t sp = packed >> 17, tp = packed & 0x1FFFFu;
  const int pbase = tid * ST_WPT * 32;
#pragma unroll
  for (int i = 0; i < ST_WPT; ++i) {
    uint32_t mm = sw[i] | tw[i];
    while (mm) {
      const int bit = __ffs(mm) - 1;
      mm &= mm - 1;
      const int32_t pos = pbase + i * 32 + bit;
      // slots stay below k by construction; the guard keeps a violated invariant in-row
      if ((sw[i] >> bit) & 1u) {
        const uint32_t slot = sp + min(tp, need);
        if (slot < (uint32_t)k) out[slot] = pos;
        ++sp;
      } else {
        if (tp < need && sp + tp < (uint32_t)k) out[sp + tp] = pos;
        ++tp;
      }
    }
  }
}

// Rows of at most 64*EPL keys (up to 6144): one wave per row, the row's scores in
// registers (the lane's item i is position 64 i + lane), and the same wave-local radix
// select as the fused route's list select: histogram passes over [lo, hi] narrow to the bin
// holding the k-th largest key, a final bin of at most 64 keys is ranked exactly (score,
// then position), a bin of one key value keeps its lowest positions; kept positions are
// written in increasing order.  Four rows per workgroup, 32 KB of LDS.
constexpr int SH_NW = 4;

__device__ __forceinline__ uint32_t sh_mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

template <int EPL>
__global__ __launch_bounds__(64 * SH_NW) void topk_short_kernel(const float* __restrict__ scores, int64_t ld,
                                                                int64_t score_bstride,
                                                                const int32_t* __restrict__ kv_len, int Tq, int Tk,
                                                                int k, int row0, int nrows,
                                                                int32_t* __restrict__ idx) {
  __shared__ uint32_t hists[SH_NW][kSelBins];
  __shared__ uint32_t mems[SH_NW][64];
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int r = blockIdx.x * SH_NW + wave, b = blockIdx.y;
  if (r >= nrows) return;
  const int64_t p = seq_len(kv_len, b, Tk) - Tq + row0 + r;
  int32_t* out = idx + ((int64_t)b * Tq + row0 + r) * k;
  if (p + 1 <= k) {  // every causal key (or none), then padding
    for (int j = lane; j < k; j += 64) out[j] = (j <= p) ? j : -1;
    return;
  }
  const int n = (int)min<int64_t>(p + 1, Tk);
  const int nr = (n + 63) / 64;
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(scores + (int64_t)b * score_bstride + (int64_t)r * ld, (uint32_t)n * 4u);
  uint32_t key[EPL];
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int i0 = 0; i0 < EPL; i0 += 8) {
#pragma unroll
    for (int i = i0; i < i0 + 8; ++i) key[i] = 0u;  // 0: no entry (every real key is >= 1)
    if (i0 >= nr) continue;
#pragma unroll
    for (int i = i0; i < i0 + 8; ++i) {
      const int e = 64 * i + lane;
      const float sc = buf_load_f32(rs, (uint32_t)lane * 4u, (uint32_t)(256 * i));
      key[i] = e < n ? sel_key(sc) : 0u;
      mn = min(mn, e < n ? key[i] : 0xFFFFFFFFu);
      mx = max(mx, key[i]);
    }
  }
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  uint32_t* const hist = hists[wave];
  uint32_t need = (uint32_t)k, lo = mn, hi = mx, m;
  int sh = sel_shift(lo, hi);
  for (;;) {
    for (int j = lane; j < kSelBins; j += 64) hist[j] = 0;
#pragma unroll
    for (int i0 = 0; i0 < EPL; i0 += 8) {
      if (i0 >= nr) continue;
#pragma unroll
      for (int i = i0; i < i0 + 8; ++i)
        if (key[i] >= lo && key[i] <= hi) atomicAdd(&hist[(key[i] - lo) >> sh], 1u);
    }
    uint32_t bin, above;
    wave_find_bin_from_top(hist, need, bin, above);
    m = __builtin_amdgcn_readfirstlane(hist[bin]);
    need -= above;
    lo += bin << sh;
    hi = (uint32_t)min((uint64_t)lo + ((1u << sh) - 1u), (uint64_t)hi);
    if (sh == 0 || m <= 64) break;
    sh = sel_shift(lo, hi);
  }
  // a final bin of m <= 64 keys over several values: rank them exactly (score, then
  // position); bit j of keptm = the j-th of them in position order is kept
  uint64_t keptm = 0;
  if (sh > 0) {
    uint32_t* const mem = mems[wave];
    uint32_t cm = 0;
#pragma unroll
    for (int i0 = 0; i0 < EPL; i0 += 8) {
      if (i0 >= nr) continue;
#pragma unroll
      for (int i = i0; i < i0 + 8; ++i) {
        const bool inb = key[i] >= lo && key[i] <= hi;
        const uint64_t bl = __ballot(inb);
        if (inb) mem[cm + sh_mbcnt(bl)] = key[i];
        cm += (uint32_t)__popcll(bl);
      }
    }
    const uint32_t mk = lane < (int)m ? mem[lane] : 0u;
    uint32_t rank = 0;
    for (uint32_t j = 0; j < m; ++j) {
      const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)mk, (int)j);
      rank += (kj > mk) || (kj == mk && (int)j < lane);
    }
    keptm = __ballot(lane < (int)m && rank < need);
  }
  // emission in position order (item i of every lane before item i+1)
  uint32_t acc = 0, before = 0;
#pragma unroll
  for (int i0 = 0; i0 < EPL; i0 += 8) {
    if (i0 >= nr) continue;
#pragma unroll
    for (int i = i0; i < i0 + 8; ++i) {
      const uint32_t kv = key[i];  // 0 past the row: never kept
      bool kp;
      if (sh > 0) {
        const bool inb = kv >= lo && kv <= hi;
        const uint64_t bl = __ballot(inb);
        kp = kv > hi || (inb && ((keptm >> (before + sh_mbcnt(bl))) & 1u));
        before += (uint32_t)__popcll(bl);
      } else {  // one key value K* = lo: ties kept lowest position first
        const bool tie = kv == lo;
        const uint64_t bl = __ballot(tie);
        kp = kv > lo || (tie && before + sh_mbcnt(bl) < need);
        before += (uint32_t)__popcll(bl);
      }
      const uint64_t bk = __ballot(kp);
      const uint32_t slot = acc + sh_mbcnt(bk);
      acc += (uint32_t)__popcll(bk);
      if (kp && slot < (uint32_t)k) out[slot] = 64 * i + lane;
    }
  }
}

// ---------------------------------------------------------------------------------------
// Split top-k for few long rows (decode: a few dozen rows of up to 65536 keys), so that a
// row's load and selection spread over the chip instead of one CU.
//
// topk_seg_kernel: one 256-thread workgroup per 4096-position segment of a row builds the
// segment's list and meta word (seglist.hpp).
// topk_merge_kernel: one workgroup per row, wave j holding segment j's list.  With
// theta = max_j theta_j, the k best entries (score, then lower position) among the listed
// keys >= theta are the row's k best whenever at least k listed keys are >= theta: the
// k-th best of them, E, then has key(E) >= theta >= theta_j for every segment, so every
// key a list lacks (below its segment's theta_j) ranks below E, while every row key
// equal to or above E is listed (ties included, so the lowest positions among them are
// too).  Rows where this fails, a list overflowed (a bin of one value held by more than
// SP_CAP keys) or the row is too short for lists (S < 4k / SP_CAP) take the one-workgroup
// kernel's path instead, so the output is the one-workgroup result in every case.
static_assert(SP_ROW_MAX == SEG, "a row the lists serve fits the one-workgroup kernel");
constexpr int SP_ROUNDS = SP_MAXSEG * SP_CAP / NT;  // union entries per merge thread
constexpr int SP_SPEC = 6;                  // list rounds the merge loads before it knows the length
constexpr int SP_PASSES = 3;                // radix passes over 32-bit keys (11 + 11 + 10 bits)

__global__ __launch_bounds__(SP_NT) void topk_seg_kernel(const float* __restrict__ scores, int64_t ld,
                                                         int64_t score_bstride, const int32_t* __restrict__ kv_len,
                                                         int Tq, int Tk, int k, int row0, int nrows,
                                                         uint2* __restrict__ lists, uint4* __restrict__ meta) {
  __shared__ SpScratch sc[1];
  const int tid = threadIdx.x;
  const int j = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const int64_t p = seq_len(kv_len, b, Tk) - Tq + row0 + r;
  if (p + 1 > SEG || !sp_uses_lists((int)(p + 1), k)) return;  // the merge kernel's own path
  const int n = (int)(p + 1);
  const int s0 = j * SP_SEG;
  if (s0 >= n) return;  // the merge reads the row's segments only
  const int nv = min(SP_SEG, n - s0);
  const int S = (n + SP_SEG - 1) / SP_SEG;
  const int64_t slot = ((int64_t)b * nrows + r) * SP_MAXSEG + j;

  // keys: thread t holds positions 1024 i + 4t + e (coalesced 16-byte loads); positions
  // past the row read 0 through the range check and get key 0 ("none")
  const float* row = scores + (int64_t)b * score_bstride + (int64_t)r * ld + s0;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(row, (uint32_t)nv * 4u);
  uint32_t key[1][16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 v = buf_load_16(rs, (uint32_t)(16 * tid), (uint32_t)(4096 * i));
#pragma unroll
    for (int e = 0; e < 4; ++e) key[0][4 * i + e] = (1024 * i + 4 * tid + e < nv) ? sel_key(__uint_as_float(v[e])) : 0u;
  }
  const int nvs[1] = {nv}, s0s[1] = {s0};
  uint2* lst[1] = {lists + slot * SP_CAP};
  uint4* mt[1] = {meta + slot};
  sp_make_lists<1>(key, nvs, s0s, S, k, lst, mt, sc);
}

__global__ __launch_bounds__(NT, 1) void topk_merge_kernel(const float* __restrict__ scores, int64_t ld,
                                                           int64_t score_bstride, const int32_t* __restrict__ kv_len,
                                                           int Tq, int Tk, int k, int row0, int nrows,
                                                           const uint2* __restrict__ lists,
                                                           const uint4* __restrict__ meta, int32_t* __restrict__ idx) {
  __shared__ uint32_t mhist[SP_PASSES][kSelPadBins];  // one histogram per radix pass, zeroed up front
  __shared__ uint32_t mstate[SP_PASSES][4];
  __shared__ uint32_t wtot[NWAVES];
  static_assert(NWAVES == SP_MAXSEG && SP_CAP == 64 * SP_ROUNDS, "wave j reads segment j's list");
  static_assert(SP_PASSES * BIN_BITS >= 32, "the last pass reaches single key values");
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int r = blockIdx.x, b = blockIdx.y;
  const int64_t p = seq_len(kv_len, b, Tk) - Tq + row0 + r;
  bool exact = true;  // take the one-workgroup path (every branch to it is uniform)
  do {
    if (p + 1 > SEG || !sp_uses_lists((int)(p + 1), k)) break;
    const int n = (int)(p + 1);
    const int S = (n + SP_SEG - 1) / SP_SEG;
    const int64_t slot0 = ((int64_t)b * nrows + r) * SP_MAXSEG;
    int32_t* out = idx + ((int64_t)b * Tq + row0 + r) * k;
    // wave j holds segment j's list, entry lane + 64 i in round i, so the union in (wave,
    // round, lane) order is in position order.  The first SP_SPEC rounds are loaded before
    // the list's length arrives (the slot holds SP_CAP entries, so the loads stay inside
    // it); entries past the length are masked to key 0 ("none") below.
    const __amdgpu_buffer_rsrc_t lrs = make_rsrc(lists + (slot0 + wave) * SP_CAP, SP_CAP * (uint32_t)sizeof(uint2));
    uint32_t key[SP_ROUNDS], pos[SP_ROUNDS];
#pragma unroll
    for (int i = 0; i < SP_SPEC; ++i) {
      const auto e = __builtin_amdgcn_raw_buffer_load_b64(lrs, (lane + 64 * i) * (int)sizeof(uint2), 0, 0);
      key[i] = e[0];
      pos[i] = e[1];
    }
    // every wave reads the row's meta words: list lengths, thetas, segment maxima
    uint32_t U = 0, theta = 0, hi = 0, cnt_w = 0;
    bool ok = true;
#pragma unroll
    for (int j = 0; j < SP_MAXSEG; ++j) {
      if (j < S) {
        const uint4 m = meta[slot0 + j];
        ok = ok && m.x != SP_OVERFLOW;
        U += m.x == SP_OVERFLOW ? 0u : m.x;
        theta = max(theta, m.y);
        hi = max(hi, m.z);
        cnt_w = j == wave ? m.x : cnt_w;
      }
    }
    for (int i = tid; i < SP_PASSES * kSelPadBins; i += NT) (&mhist[0][0])[i] = 0;
    if (!ok || U < (uint32_t)k) break;
    const int nr = (int)((cnt_w + 63) / 64);  // (wave-uniform; cnt_w <= SP_CAP)
#pragma unroll
    for (int i = SP_SPEC; i < SP_ROUNDS; ++i) {
      key[i] = pos[i] = 0u;
      if (i < nr) {
        const auto e = __builtin_amdgcn_raw_buffer_load_b64(lrs, (lane + 64 * i) * (int)sizeof(uint2), 0, 0);
        key[i] = e[0];
        pos[i] = e[1];
      }
    }
#pragma unroll
    for (int i = 0; i < SP_ROUNDS; ++i) key[i] = (uint32_t)(lane + 64 * i) < cnt_w ? key[i] : 0u;
    // exact radix select of the k-th best key among the listed keys >= theta; pass 0 also
    // counts them (fewer than k: the lists cannot decide the row)
    uint32_t lo = max(theta, 1u), need = (uint32_t)k, blo = lo, bhi = hi;
    int sh = sel_shift(lo, hi);
    bool whole_bin = false, decided = false;
    __syncthreads();  // histograms zeroed
#pragma unroll
    for (int ps = 0; ps < SP_PASSES; ++ps) {
      uint32_t* h = mhist[ps];
#pragma unroll
      for (int i = 0; i < SP_ROUNDS; ++i)
        if (i < nr && key[i] >= lo && key[i] <= hi) atomicAdd(&h[sel_pad((key[i] - lo) >> sh)], 1u);
      __syncthreads();
      if (wave == 0) {
        uint32_t bin, above, total;
        wave_find_bin_padded(h, need, bin, above, &total);
        if (lane == 0) {
          mstate[ps][0] = bin;
          mstate[ps][1] = above;
          mstate[ps][2] = h[sel_pad(bin)];
          mstate[ps][3] = total;
        }
      }
      __syncthreads();
      if (ps == 0 && mstate[0][3] < (uint32_t)k) break;  // decided stays false
      const uint32_t bin = mstate[ps][0], m = mstate[ps][2];
      need -= mstate[ps][1];
      blo = lo + (bin << sh);
      bhi = (uint32_t)min((uint64_t)blo + ((1u << sh) - 1u), (uint64_t)hi);
      whole_bin = m == need;  // every member of the bin is kept
      if (whole_bin || sh == 0) {
        decided = true;
        break;
      }
      lo = blo;
      hi = bhi;
      sh = max(0, sh - BIN_BITS);
    }
    if (!decided) break;
    // kept: keys > bhi, and the bin (all of it, or its first `need` ties by position).
    // Emission in position order: each wave's counts of kept keys above the bin (high
    // half) and of bin members (low half), then a running count through its rounds.
    uint32_t wsum = 0;
#pragma unroll
    for (int i = 0; i < SP_ROUNDS; ++i) {
      if (i < nr) {
        const bool a = whole_bin ? key[i] >= blo : key[i] > bhi;
        const bool t = !whole_bin && key[i] == blo;
        wsum += ((uint32_t)__popcll(__ballot(a)) << 16) | (uint32_t)__popcll(__ballot(t));
      }
    }
    if (lane == 0) wtot[wave] = wsum;
    __syncthreads();
    uint32_t base = 0;
    for (int w = 0; w < wave; ++w) base += wtot[w];
    uint32_t ap = base >> 16, tp = base & 0xFFFFu;
#pragma unroll
    for (int i = 0; i < SP_ROUNDS; ++i) {
      if (i < nr) {
        const bool a = whole_bin ? key[i] >= blo : key[i] > bhi;
        const bool t = !whole_bin && key[i] == blo;
        const uint64_t ba = __ballot(a), bt = __ballot(t);
        const uint32_t ai = ap + sh_mbcnt(ba), ti = tp + sh_mbcnt(bt);
        if (a) {
          const uint32_t o = ai + min(ti, need);
          if (o < (uint32_t)k) out[o] = (int32_t)pos[i];
        } else if (t && ti < need) {
          if (ai + ti < (uint32_t)k) out[ai + ti] = (int32_t)pos[i];
        }
        ap += (uint32_t)__popcll(ba);
        tp += (uint32_t)__popcll(bt);
      }
    }
    exact = false;
  } while (false);
  if (exact) {
    __syncthreads();  // this kernel's LDS reads are done
    topk_fast_row(scores, ld, score_bstride, kv_len, Tq, Tk, k, row0, idx, r, b);
  }
}

}  // namespace

size_t topk_split_workspace_bytes(int B, int nrows, int Tk, int k) {
  // rows the one-workgroup kernel would take, with room for segment lists
  if (B <= 0 || nrows <= 0 || Tk <= 64 * 96 || Tk > SEG || (int64_t)nrows * B >= 1024 ||
      (int64_t)((Tk + SP_SEG - 1) / SP_SEG) * (SP_CAP / 2) < 2 * (int64_t)k)
    return 0;
  return (size_t)B * nrows * SP_MAXSEG * (SP_CAP * sizeof(uint2) + sizeof(uint4));  // lists, then meta words
}

bool topk_split_route(const TopkArgs& A) {
  return A.nrows > 0 && A.B > 0 && A.Tk > 64 * 96 && topk_split_workspace_bytes(A.B, A.nrows, A.Tk, A.k) && A.ws &&
         A.ld % 4 == 0 && A.score_bstride % 4 == 0 && (reinterpret_cast<uintptr_t>(A.scores) & 15) == 0;
}

hipError_t launch_topk(const TopkArgs& A, hipStream_t st) {
  if (A.nrows <= 0 || A.B <= 0) return hipSuccess;
  if (A.lists_ready && !topk_split_route(A)) return hipErrorInvalidValue;
  dim3 grid(A.nrows, A.B);
  // rows see at most Tk keys.  Up to 6144: a wave per row.  Up to one segment (65536) they
  // stay in registers: many rows take the streaming kernel (256 threads, four rows per CU),
  // few rows (decode) 1024 threads per row, which keeps the chip busy.
  if (A.Tk <= 64 * 96) {
    dim3 g2((unsigned)((A.nrows + SH_NW - 1) / SH_NW), A.B);
    if (A.Tk <= 64 * 48)
      hipLaunchKernelGGL(topk_short_kernel<48>, g2, dim3(64 * SH_NW), 0, st, A.scores, A.ld, A.score_bstride,
                         A.kv_len, A.Tq, A.Tk, A.k, A.row0, A.nrows, A.idx);
    else
      hipLaunchKernelGGL(topk_short_kernel<96>, g2, dim3(64 * SH_NW), 0, st, A.scores, A.ld, A.score_bstride,
                         A.kv_len, A.Tq, A.Tk, A.k, A.row0, A.nrows, A.idx);
  } else if (topk_split_route(A)) {
    uint2* lists = reinterpret_cast<uint2*>(A.ws);
    uint4* meta = reinterpret_cast<uint4*>(lists + (size_t)A.B * A.nrows * SP_MAXSEG * SP_CAP);
    const int segs = (A.Tk + SP_SEG - 1) / SP_SEG;
    if (!A.lists_ready)  // (else the scores' producer built them)
      hipLaunchKernelGGL(topk_seg_kernel, dim3(segs, A.nrows, A.B), dim3(SP_NT), 0, st, A.scores, A.ld,
                         A.score_bstride, A.kv_len, A.Tq, A.Tk, A.k, A.row0, A.nrows, lists, meta);
    hipLaunchKernelGGL(topk_merge_kernel, grid, dim3(NT), 0, st, A.scores, A.ld, A.score_bstride, A.kv_len, A.Tq,
                       A.Tk, A.k, A.row0, A.nrows, lists, meta, A.idx);
  } else if (A.Tk <= SEG && (int64_t)A.nrows * A.B >= 1024)
    hipLaunchKernelGGL(topk_stream_kernel, grid, dim3(ST_NT), 0, st, A.scores, A.ld, A.score_bstride, A.kv_len,
                       A.Tq, A.Tk, A.k, A.row0, A.idx);
  else if (A.Tk <= SEG)
    hipLaunchKernelGGL(topk_fast_kernel, grid, dim3(NT), 0, st, A.scores, A.ld, A.score_bstride, A.kv_len, A.Tq,
                       A.Tk, A.k, A.row0, A.idx);
  else
    hipLaunchKernelGGL(topk_kernel<false>, grid, dim3(NT), 0, st, A.scores, A.ld, A.score_bstride, A.kv_len, A.Tq,
                       A.Tk, A.k, A.row0, A.idx);
  return hipGetLastError();
}

}  // namespace dsa
