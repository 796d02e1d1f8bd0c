// Causal top-k per query row on gfx950.
//
// Selection rule (DSV2-Lite IndexCache card, intro: causal key selection with a budget of
// k tokens; DSA ablation card, "Benchmarks": a row shorter than k keeps every key):
// a row with n = p+1 <= k candidates keeps keys 0..p; otherwise the k largest scores,
// equal scores resolved toward the lower key index, -0.0 == +0.0.  Output ascending,
// -1 padded.
//
// One 1024-thread workgroup per row.  Scores become order-preserving uint32 keys.  A radix
// select over LDS histograms finds the k-th largest key K*: the first pass bins the
// row's actual [min, max] key range into 2048 bins (so the populated bins spread out and
// LDS atomics rarely collide), later passes refine inside the threshold bin only, at
// most three passes in all.  Rows of up to 65536 keys stay in registers for every pass.
// The kept set (keys > K*, plus the lowest-index ties == K*) is marked in LDS bitmaps and
// emitted in index order from a block-wide prefix count of each thread's bit span.
#include "common.hpp"
#include "internal.hpp"

namespace dsa {

namespace {

constexpr int NT = 1024;
constexpr int NWAVES = NT / 64;
constexpr int ITEMS = 64;               // keys per thread per segment
constexpr int SEG = NT * ITEMS;         // 65536 positions per segment
constexpr int NBINS = 2048;
constexpr int BIN_BITS = 11;
constexpr int SEG_WORDS = SEG / 32;     // bitmap words per segment

// -0.0 and +0.0 share a key; larger floats get larger keys; 0 marks "no candidate".
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0) u = 0;  // canonical +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive prefix sum over the workgroup in thread order; also returns the total.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* red, uint32_t& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t incl = wave_incl_scan(v, lane);
  if (lane == 63) red[wid] = incl;
  __syncthreads();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NWAVES; ++i) {
    uint32_t r = red[i];
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

}  // namespace

hipError_t launch_topk(const TopkArgs& A, hipStream_t st) {
  if (A.nrows <= 0 || A.B <= 0) return hipSuccess;
  dim3 grid(A.nrows, A.B);
  // rows see at most Tk keys: up to one segment they are kept in registers
  if (A.Tk <= SEG)
    hipLaunchKernelGGL(topk_kernel<true>, grid, dim3(NT), 0, st, A.scores, A.ld, A.score_bstride, A.kv_len, A.Tq,
                       A.Tk, A.k, A.row0, A.idx);
  else
    hipLaunchKernelGGL(topk_kernel<false>, grid, dim3(NT), 0, st, A.scores, A.ld, A.score_bstride, A.kv_len, A.Tq,
                       A.Tk, A.k, A.row0, A.idx);
  return hipGetLastError();
}

}  // namespace dsa
