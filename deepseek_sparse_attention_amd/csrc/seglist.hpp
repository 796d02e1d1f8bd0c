// Segment lists of the split top-k (few long rows, e.g. decode): a row of up to 65536
// positions is cut into segments of SP_SEG positions, and one 256-thread workgroup lists,
// for each of its NSEG segments, every key >= theta_j of the segment in position order,
// theta_j chosen so that the list holds at least c = ceil(2k / S) keys (S = the row's
// segments) and at most SP_CAP: the lower edge of the histogram bin of its c-th largest key
// (a second pass inside that bin, and a third, if the first overshoots).  A segment of at
// most SP_CAP keys lists all of them (theta 0 in its meta word).  The meta word of a
// segment holds the list's length, theta_j and the segment's largest key; a bin of one key
// value held by more than SP_CAP positions gives SP_OVERFLOW instead.  The merge (one
// workgroup per row, topk.hip) selects the row's k best among the listed keys.
//
// The builder is shared by the segment kernel (keys read from the score rows) and the
// decode indexer (keys read from the scores it holds in LDS), so both produce the same
// lists.
#pragma once

#include "selection.hpp"

namespace dsa {

constexpr int SP_SEG = 4096;                // positions per segment
constexpr int SP_NT = 256;                  // threads of a list-building workgroup: 16 keys each
constexpr int SP_CAP = 1024;                // list entries per segment
constexpr int SP_ROW_MAX = 65536;           // longest row the lists serve
constexpr int SP_MAXSEG = SP_ROW_MAX / SP_SEG;  // segments per row, at most 16
constexpr uint32_t SP_OVERFLOW = 0xFFFFFFFFu;

// Rows that use segment lists: every segment can hold its share of twice k.
__device__ __host__ __forceinline__ bool sp_uses_lists(int n, int k) {
  const int S = (n + SP_SEG - 1) / SP_SEG;
  return n <= SP_ROW_MAX && S * (SP_CAP / 2) >= 2 * k && n > k;
}

// LDS of one segment's selection.
struct SpScratch {
  uint32_t hist[kSelPadBins];
  uint32_t red[2 * (SP_NT / 64)];
  uint32_t cnt[3 * (SP_NT / 64)];
  uint32_t state[4];
};

// Lists of NSEG segments at once.  Thread t holds key[g][4i + e] = the order key of
// position s0[g] + 1024 i + 4t + e (0, "none", past the segment's nv[g] valid keys); a
// segment with nv[g] <= 0 writes nothing.  Every thread of the workgroup calls this (it
// has barriers, taken by all of them the same number of times); sc[g] is segment g's LDS.
// lst[g] / mt[g]: the segment's list slot (SP_CAP entries) and meta word.
template <int NSEG>
__device__ __forceinline__ void sp_make_lists(uint32_t (&key)[NSEG][16], const int (&nv)[NSEG], const int (&s0)[NSEG],
                                              int S, int k, uint2* (&lst)[NSEG], uint4* (&mt)[NSEG],
                                              SpScratch* sc) {
  constexpr int SW = SP_NT / 64;
  static_assert(NSEG <= SW, "one wave searches each segment's histogram");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t theta[NSEG], count[NSEG];
  bool ovf[NSEG];
  bool any_big = false;
#pragma unroll
  for (int g = 0; g < NSEG; ++g) {
    theta[g] = 1u;  // every valid key (keys are >= 1)
    count[g] = 0;
    ovf[g] = false;
    any_big = any_big || nv[g] > SP_CAP;
  }
  if (any_big) {  // (uniform: nv is)
    uint32_t lo[NSEG], hi[NSEG], need[NSEG], taken[NSEG];
    int sh[NSEG];
    bool done[NSEG];
#pragma unroll
    for (int g = 0; g < NSEG; ++g) {
      uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        kmin = min(kmin, key[g][e] - 1u);  // 0 wraps to the top and drops out
        kmax = max(kmax, key[g][e]);
      }
      kmin = wave_min_u32(kmin);
      kmax = wave_max_u32(kmax);
      if (lane == 0) {
        sc[g].red[wave] = kmin;
        sc[g].red[SW + wave] = kmax;
      }
      for (int i = tid; i < kSelPadBins; i += SP_NT) sc[g].hist[i] = 0;
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < NSEG; ++g) {
      uint32_t l = sc[g].red[0], h = sc[g].red[SW];
#pragma unroll
      for (int w = 1; w < SW; ++w) {
        l = min(l, sc[g].red[w]);
        h = max(h, sc[g].red[SW + w]);
      }
      lo[g] = l + 1u;
      hi[g] = h;
      sh[g] = sel_shift(lo[g], hi[g]);
      need[g] = (uint32_t)((2 * k + S - 1) / S);
      taken[g] = 0;
      done[g] = nv[g] <= SP_CAP;  // (lists every valid key, theta 1)
    }
    for (;;) {
#pragma unroll
      for (int g = 0; g < NSEG; ++g) {
        if (done[g]) continue;
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (key[g][e] >= lo[g] && key[g][e] <= hi[g]) atomicAdd(&sc[g].hist[sel_pad((key[g][e] - lo[g]) >> sh[g])], 1u);
      }
      __syncthreads();
#pragma unroll
      for (int g = 0; g < NSEG; ++g) {
        if (!done[g] && wave == g) {
          uint32_t bin, above;
          wave_find_bin_padded(sc[g].hist, need[g], bin, above);
          if (lane == 0) {
            sc[g].state[0] = bin;
            sc[g].state[1] = above;
            sc[g].state[2] = sc[g].hist[sel_pad(bin)];
          }
        }
      }
      __syncthreads();
      bool all_done = true;
#pragma unroll
      for (int g = 0; g < NSEG; ++g) {
        if (done[g]) continue;
        const uint32_t bin = sc[g].state[0], above = sc[g].state[1], m = sc[g].state[2];
        const uint32_t blo = lo[g] + (bin << sh[g]);
        count[g] = taken[g] + above + m;
        if (count[g] <= (uint32_t)SP_CAP || sh[g] == 0) {
          theta[g] = blo;
          done[g] = true;
          ovf[g] = count[g] > (uint32_t)SP_CAP;  // one key value held by too many positions
          continue;
        }
        // the bin overshoots the list: split it
        all_done = false;
        taken[g] += above;
        need[g] -= above;
        hi[g] = (uint32_t)min((uint64_t)blo + ((1u << sh[g]) - 1u), (uint64_t)hi[g]);
        lo[g] = blo;
        sh[g] = max(0, sh[g] - kSelBinBits);
        for (int i = tid; i < kSelPadBins; i += SP_NT) sc[g].hist[i] = 0;
      }
      if (all_done) break;
      __syncthreads();  // histograms zeroed before the next pass
    }
  }

  // each list in position order (i, then t, then e): per-thread counts of rounds 0/1 and
  // 2/3 packed in 16-bit fields (block totals <= 1024 when the list fits), one block scan each
  uint32_t c[NSEG][4], pk01[NSEG], pk23[NSEG], in01[NSEG], in23[NSEG];
#pragma unroll
  for (int g = 0; g < NSEG; ++g) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[g][i] = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) c[g][i] += key[g][4 * i + e] >= theta[g];
    }
    pk01[g] = c[g][0] | (c[g][1] << 16);
    pk23[g] = c[g][2] | (c[g][3] << 16);
    uint32_t w01, w23, kx = 0;
    in01[g] = wave_incl_scan_u32(pk01[g], &w01);
    in23[g] = wave_incl_scan_u32(pk23[g], &w23);
#pragma unroll
    for (int e = 0; e < 16; ++e) kx = max(kx, key[g][e]);
    kx = wave_max_u32(kx);
    if (lane == 0) {
      sc[g].cnt[wave] = w01;
      sc[g].cnt[SW + wave] = w23;
      sc[g].cnt[2 * SW + wave] = kx;
    }
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < NSEG; ++g) {
    if (nv[g] <= 0) continue;
    if (ovf[g]) {
      if (tid == 0) *mt[g] = make_uint4(SP_OVERFLOW, 0u, 0u, 0u);
      continue;
    }
    uint32_t pre01 = 0, pre23 = 0, tot01 = 0, tot23 = 0, segmax = 0;
#pragma unroll
    for (int w = 0; w < SW; ++w) {
      pre01 += w < wave ? sc[g].cnt[w] : 0u;
      pre23 += w < wave ? sc[g].cnt[SW + w] : 0u;
      tot01 += sc[g].cnt[w];
      tot23 += sc[g].cnt[SW + w];
      segmax = max(segmax, sc[g].cnt[2 * SW + w]);
    }
    const uint32_t ex01 = pre01 + in01[g] - pk01[g], ex23 = pre23 + in23[g] - pk23[g];
    const uint32_t T0 = tot01 & 0xFFFFu, T1 = tot01 >> 16, T2 = tot23 & 0xFFFFu, T3 = tot23 >> 16;
    uint32_t base[4] = {ex01 & 0xFFFFu, T0 + (ex01 >> 16), T0 + T1 + (ex23 & 0xFFFFu), T0 + T1 + T2 + (ex23 >> 16)};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (key[g][4 * i + e] >= theta[g]) {
          lst[g][base[i]] = make_uint2(key[g][4 * i + e], (uint32_t)(s0[g] + 1024 * i + 4 * tid + e));
          ++base[i];
        }
      }
    }
    if (tid == 0) *mt[g] = make_uint4(T0 + T1 + T2 + T3, nv[g] > SP_CAP ? theta[g] : 0u, segmax, 0u);
  }
}

}  // namespace dsa
