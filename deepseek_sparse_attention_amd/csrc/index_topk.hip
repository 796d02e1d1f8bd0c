// Fused lightning indexer -> causal top-k on gfx950: the selection runs on the scores while
// the indexer produces them, so no fp32 score row is written to or read back from memory.
//
// What is computed is exactly what the indexer followed by top-k computes (DSA ablation card,
// model list: ReLU indexer; DSV2-Lite IndexCache card, intro: causal selection of k keys;
// DSA ablation card, "Benchmarks": short rows keep every key; lower index wins a tie,
// -0 == +0).  Every score comes from the shared per-wave core (indexer_core.hpp), so it is
// the same fp32 value the score kernel would store, and the selection is exact:
//
// 1. sample:    each wave scores its rows against ~1/16 of their keys (whole 32-key tiles
//               spread evenly over the keys every row of the wave can see);
// 2. threshold: per row, a score expected to be exceeded by about alpha*k keys (alpha
//               ~1.65 at k = 2048): the m-th largest sample, m = alpha*k*samples/n;
// 3. filter:    each wave scores its rows against all their keys and appends every score at
//               or above its row's threshold, with its key index, to the row's candidate
//               list: one range-checked 8-byte store per score epilogue, dropped for lanes
//               without a candidate.  A wave owns whole rows, so a list needs no atomics
//               and comes out in key order;
// 4. select:    per row, if the list holds at least k and at most kFusedCap entries it holds
//               the whole top-k (every key at or above the k-th largest score passed the
//               threshold test, which is monotone in the score); a radix select over the
//               list finds the k-th largest key and the ties to keep, and the kept entries
//               are written in list order, i.e. ascending key index;
// 5. exact:     rows whose list was too short or overflowed are redone from scratch: one
//               workgroup recomputes the row's scores in each of five passes (three radix
//               histogram passes, a count pass and an emission pass).  With the default
//               alpha this path is astronomically rare; it keeps the result exact anyway.
#include "indexer_core.hpp"
#include "internal.hpp"
#include "selection.hpp"

namespace dsa {

namespace {

constexpr int FZ_CAP = kFusedCap;      // candidate entries per row
constexpr int FZ_NT = 256;
constexpr int FZ_NW = FZ_NT / 64;
constexpr int FZ_KEEP = FZ_CAP;         // rows of up to this many keys keep every key
static_assert(FZ_CAP % 64 == 0, "list rounds");

// Threshold score of a key from the order-preserving map (keys from finite scores map back
// to finite floats).
__device__ __forceinline__ float key_to_float(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key ^ 0x80000000u) : ~key);
}

__device__ __forceinline__ uint32_t mbcnt64(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Block-wide min / max of the valid keys (every thread passes its partial values).
__device__ __forceinline__ void fz_minmax(uint32_t& mn, uint32_t& mx, uint32_t* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  if (lane == 0) {
    red[wid] = mn;
    red[FZ_NW + wid] = mx;
  }
  __syncthreads();
  mn = red[0];
  mx = red[FZ_NW];
#pragma unroll
  for (int i = 1; i < FZ_NW; ++i) {
    mn = min(mn, red[i]);
    mx = max(mx, red[FZ_NW + i]);
  }
  __syncthreads();
}

// Exclusive prefix sum over the workgroup in thread order; also returns the total.
__device__ __forceinline__ uint32_t fz_excl_scan(uint32_t v, uint32_t* red, uint32_t& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t wsum;
  const uint32_t incl = wave_incl_scan_u32(v, &wsum);
  if (lane == 0) red[wid] = wsum;
  __syncthreads();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < FZ_NW; ++i) {
    const uint32_t r = red[i];
    pre += (i < wid) ? r : 0u;
    tot += r;
  }
  __syncthreads();
  total = tot;
  return pre + incl - v;
}

template <int H_I, int D_I>
using FzWave = IdxWave<H_I, D_I, idx_query_tiles<H_I, D_I>()>;

// Rows of a wave / workgroup and the wave geometry shared by the sample and filter kernels.
struct FzRows {
  int64_t pos_base;  // position of chunk row r is pos_base + r
  int wrow0, wrows;  // the wave's first chunk row and row count
  int64_t p_first, p_last;
};

template <int ROWS>
__device__ __forceinline__ bool fz_rows(const int32_t* kv_len, int Tq, int Tk, int row0, int nrows, int nblocks,
                                        FzRows& R) {
  const int wave = wave_id();
  const int64_t L = seq_len(kv_len, blockIdx.z, Tk);
  R.pos_base = L - Tq + row0;
  const int blk = nblocks - 1 - (int)blockIdx.x;  // blocks with the longest rows first
  R.wrow0 = blk * 4 * ROWS + wave * ROWS;
  if (R.wrow0 >= nrows) return false;
  R.wrows = min(ROWS, nrows - R.wrow0);
  R.p_first = R.pos_base + R.wrow0;
  R.p_last = R.p_first + R.wrows - 1;
  return true;
}

// ---- 1. sample scores (as order keys) of ~1/16 of the keys of each row
template <int H_I, int D_I>
__global__ __launch_bounds__(256, 2) void fz_sample_kernel(const uint16_t* __restrict__ q,
                                                           const uint16_t* __restrict__ k,
                                                           const uint16_t* __restrict__ w,
                                                           const int32_t* __restrict__ kv_len, int Tq, int Tk,
                                                           int row0, int nrows, int nblocks, uint32_t* __restrict__ smp,
                                                           int smax, int32_t* __restrict__ ns) {
  using W = FzWave<H_I, D_I>;
  __shared__ __attribute__((aligned(16))) uint8_t wks[4][W::kLdsBytes];
  FzRows R;
  if (!fz_rows<W::ROWS>(kv_len, Tq, Tk, row0, nrows, nblocks, R)) return;
  if (R.p_last + 1 <= FZ_KEEP) return;  // every row of the wave keeps all its keys
  const int b = blockIdx.z, lane = threadIdx.x & 63;
  // the keys every row of the wave sees: 0 .. p_first (p_first + 1 > FZ_KEEP - 16 >= 512)
  const int span = (int)(R.p_first + 1);
  const int nst = fz_sample_tiles(span);
  const int step = span / nst, half = step / 2 - 16;  // tile j is centred in [j*step, (j+1)*step)
  const int64_t rbase = (int64_t)b * nrows + R.wrow0;
  if (lane < R.wrows) ns[rbase + lane] = nst * 32;
  W wv;
  wv.load(q + ((int64_t)b * Tq + row0 + R.wrow0) * H_I * D_I, w + ((int64_t)b * Tq + row0 + R.wrow0) * H_I, R.wrows);
  const __amdgpu_buffer_rsrc_t k_rs = make_rsrc(k + (int64_t)b * Tk * D_I, (uint32_t)Tk * D_I * 2);
  // rows past the wave's count fall outside the store range and are dropped
  const u32x4 s_rs = rsrc_words(smp + rbase * smax, (uint32_t)(R.wrows * smax * 4));
  const int col = wv.col;
  wv.template run<W::EPIS>(k_rs, wks[wave_id()], nst,
                           [&](int j) { return min(max(j * step + half, 0), span - 32); },
         [&](int j, int, int t, int qq, float tot) {
           const uint32_t off = (uint32_t)(wv.row_of(t, qq) * smax + j * 32 + col) * 4u;
           buf_store1_b32(sel_key(tot), s_rs, off);  // one store per call (EPIS per tile)
         });
}

// ---- 2. per-row threshold: the m-th largest sample (to within a fine histogram bin below
// it), m = alpha*k*samples/n; rows that keep every key get -inf.  One wave per row (four
// rows per workgroup, no barriers): the samples sit in registers (sample 64*i + lane in
// round i), two passes over a per-wave LDS histogram.
constexpr int FZ_SPL = 32 * kFusedMaxSampleTiles / 64;  // samples per lane, at most

__global__ __launch_bounds__(FZ_NT) void fz_threshold_kernel(const uint32_t* __restrict__ smp, int smax,
                                                             const int32_t* __restrict__ ns,
                                                             const int32_t* __restrict__ kv_len, int Tq, int Tk,
                                                             int row0, int nrows, int topk, float alpha,
                                                             float* __restrict__ thr) {
  __shared__ uint32_t hists[FZ_NW][kSelBins];
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int r = blockIdx.x * FZ_NW + wave, b = blockIdx.y;
  if (r >= nrows) return;
  const int64_t n = seq_len(kv_len, b, Tk) - Tq + row0 + r + 1;
  const int64_t rowi = (int64_t)b * nrows + r;
  if (n <= FZ_KEEP) {
    if (lane == 0) thr[rowi] = -__builtin_inff();
    return;
  }
  const int nsr = ns[rowi];  // a multiple of 32, at most 64 * FZ_SPL
  const uint32_t m = (uint32_t)fminf((float)nsr, fmaxf(1.f, ceilf(alpha * (float)topk * (float)nsr / (float)n)));
  const __amdgpu_buffer_rsrc_t s_rs = make_rsrc(smp + rowi * smax, (uint32_t)nsr * 4u);
  uint32_t key[FZ_SPL];
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  const int nrd = (nsr + 63) / 64;
#pragma unroll
  for (int i0 = 0; i0 < FZ_SPL; i0 += 8) {
#pragma unroll
    for (int i = i0; i < i0 + 8; ++i) key[i] = 0u;  // 0: no sample (every real key is >= 1)
    if (i0 >= nrd) continue;
#pragma unroll
    for (int i = i0; i < i0 + 8; ++i) {
      key[i] = __builtin_amdgcn_raw_buffer_load_b32(s_rs, lane * 4, 256 * i, 0);  // past nsr: 0
      mn = min(mn, key[i] ? key[i] : 0xFFFFFFFFu);
      mx = max(mx, key[i]);
    }
  }
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  uint32_t* const hist = hists[wave];
  auto pass = [&](uint32_t lo, uint32_t hi, int sh, uint32_t need, uint32_t& bin, uint32_t& above) {
    for (int j = lane; j < kSelBins; j += 64) hist[j] = 0;
#pragma unroll
    for (int i0 = 0; i0 < FZ_SPL; i0 += 8) {
      if (i0 >= nrd) continue;
#pragma unroll
      for (int i = i0; i < i0 + 8; ++i)
        if (key[i] >= lo && key[i] <= hi) atomicAdd(&hist[(key[i] - lo) >> sh], 1u);
    }
    wave_find_bin_from_top(hist, need, bin, above);
  };
  const int sh = sel_shift(mn, mx);
  uint32_t bin, above;
  pass(mn, mx, sh, m, bin, above);
  uint32_t th = mn + (bin << sh);
  if (sh > 0) {  // refine inside the bin: a bin edge alone could pass many more keys
    const uint32_t bhi = (uint32_t)min((uint64_t)th + ((1u << sh) - 1u), (uint64_t)mx);
    const int sh2 = sel_shift(th, bhi);
    uint32_t bin2, above2;
    pass(th, bhi, sh2, m - above, bin2, above2);
    th += bin2 << sh2;
  }
  // at least m samples have keys >= th, so the filter's count is near alpha*k
  if (lane == 0) thr[rowi] = key_to_float(th);
}

// ---- 3. scores of every causal key, filtered into per-row candidate lists
template <int H_I, int D_I>
__global__ __launch_bounds__(256, 2) void fz_filter_kernel(const uint16_t* __restrict__ q,
                                                           const uint16_t* __restrict__ k,
                                                           const uint16_t* __restrict__ w,
                                                           const int32_t* __restrict__ kv_len, int Tq, int Tk,
                                                           int row0, int nrows, int nblocks, int topk,
                                                           const float* __restrict__ thr, uint32_t* __restrict__ cnt,
                                                           uint2* __restrict__ list) {
  using W = FzWave<H_I, D_I>;
  constexpr int ROWS = W::ROWS;
  __shared__ __attribute__((aligned(16))) uint8_t wks[4][W::kLdsBytes];
  FzRows R;
  if (!fz_rows<ROWS>(kv_len, Tq, Tk, row0, nrows, nblocks, R)) return;
  if (R.p_last + 1 <= topk) return;  // every row keeps all its keys: nothing to select
  const int b = blockIdx.z, lane = threadIdx.x & 63;
  const int64_t rbase = (int64_t)b * nrows + R.wrow0;
  W wv;
  wv.load(q + ((int64_t)b * Tq + row0 + R.wrow0) * H_I * D_I, w + ((int64_t)b * Tq + row0 + R.wrow0) * H_I, R.wrows);
  const __amdgpu_buffer_rsrc_t k_rs = make_rsrc(k + (int64_t)b * Tk * D_I, (uint32_t)Tk * D_I * 2);
  // the wave's lists (rows past the chunk would fall outside; they never pass anyway)
  const u32x4 l_rs = rsrc_words(list + rbase * FZ_CAP, (uint32_t)(R.wrows * FZ_CAP * 8));
  // the lane's rows: last causal key (-1 for rows past the chunk) and threshold
  int lim[ROWS / W::QPT][W::QPL];
  float th[ROWS / W::QPT][W::QPL];
#pragma unroll
  for (int t = 0; t < ROWS / W::QPT; ++t) {
#pragma unroll
    for (int qq = 0; qq < W::QPL; ++qq) {
      const int r = wv.row_of(t, qq);
      lim[t][qq] = r < R.wrows ? (int)(R.p_first + r) : -1;
      th[t][qq] = r < R.wrows ? thr[rbase + r] : 0.f;
    }
  }
  uint32_t fill[ROWS];  // candidates of each row so far (wave-uniform)
#pragma unroll
  for (int r = 0; r < ROWS; ++r) fill[r] = 0;
  const int col = wv.col, g = wv.g;
  const uint32_t lane_list = (uint32_t)(g * W::QPL * FZ_CAP) * 8u;  // list of row rA + g*QPL
  wv.template run<W::EPIS>(k_rs, wks[wave_id()], (int)((R.p_last + 32) / 32), [](int j) { return 32 * j; },
         [&](int, int s0, int t, int qq, float tot) {
           const int skey = s0 + col;
           const bool c = skey <= lim[t][qq] && tot >= th[t][qq];
           const uint64_t bal = __ballot(skey <= lim[t][qq]) & __ballot(tot >= th[t][qq]);
           const uint32_t n0 = __popc((uint32_t)bal), n1 = __popc((uint32_t)(bal >> 32));
           const int rA = t * W::QPT + qq, rB = rA + W::QPL;  // the rows of lane groups 0 and 1
           // slot in the lane's row: its row's count so far plus the row's passing lanes
           // below it; entries past the capacity all land on the last slot (such a row
           // fails its count check and is recomputed)
           const uint32_t slot = min((g ? fill[rB] - n0 : fill[rA]) + mbcnt64(bal), (uint32_t)FZ_CAP - 1u);
           uint32_t addr = lane_list + (uint32_t)(rA * FZ_CAP) * 8u + slot * 8u;
           asm volatile("" : "+v"(addr));  // computed on every lane: the select stays a select
           const uint32_t at = c ? addr : kOffNone;
           buf_store1_b64(u32x2{__float_as_uint(tot), (uint32_t)skey}, l_rs, at);  // one store per call
           fill[rA] += n0;
           fill[rB] += n1;
         });
  // each row's count: all candidates, also past the capacity
  uint32_t mine = 0;
#pragma unroll
  for (int r = 0; r < ROWS; ++r) mine = lane == r ? fill[r] : mine;
  if (lane < R.wrows) cnt[rbase + lane] = mine;
}

__device__ __forceinline__ bool fz_row_failed(uint32_t c, int topk) { return c < (uint32_t)topk || c > (uint32_t)FZ_CAP; }

// ---- 4. exact top-k of each row's candidate list: one wave per row (four rows per
// workgroup, no barriers).  The wave keeps the list's keys in registers (entry e = 64*i +
// lane in round i: coalesced loads, list order = (round, lane) order), narrows the bin of
// the k-th largest key with LDS histogram passes until it holds at most 64 entries or one
// key value, ranks such a bin's entries exactly, and writes the kept entries' key indices
// in list order (= ascending key index).  Built for four workgroups per CU: the register
// budget then spills a few values to scratch, and the kernel is still 10% faster at
// T=65536 than at three workgroups per CU without spills (0.62 against 0.69 ms).
constexpr int FZ_EPL = FZ_CAP / 64;  // list entries per lane, at most

__global__ __launch_bounds__(FZ_NT, 4) void fz_select_kernel(const uint32_t* __restrict__ cnt,
                                                          const uint2* __restrict__ list,
                                                          const int32_t* __restrict__ kv_len, int Tq, int Tk, int row0,
                                                          int nrows, int topk, int32_t* __restrict__ idx) {
  __shared__ uint32_t hists[FZ_NW][kSelBins];
  __shared__ uint32_t mems[FZ_NW][64];
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int r = blockIdx.x * FZ_NW + wave, b = blockIdx.y;
  if (r >= nrows) return;
  const int64_t p = seq_len(kv_len, b, Tk) - Tq + row0 + r;
  int32_t* out = idx + ((int64_t)b * Tq + row0 + r) * topk;
  if (p + 1 <= topk) {  // every causal key (or none), then padding
    for (int j = lane; j < topk; j += 64) out[j] = (j <= p) ? j : -1;
    return;
  }
  const int64_t rowi = (int64_t)b * nrows + r;
  const uint32_t c = cnt[rowi];
  if (fz_row_failed(c, topk)) return;  // the exact pass redoes this row
  const int nr = (int)((c + 63) / 64);
  const __amdgpu_buffer_rsrc_t l_rs = make_rsrc(list + rowi * FZ_CAP, c * 8u);
  uint32_t key[FZ_EPL];
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  // (loads past the list fall outside the buffer range: they read zero and move no data;
  // the round's base goes in the scalar offset)
#pragma unroll
  for (int i0 = 0; i0 < FZ_EPL; i0 += 8) {
#pragma unroll
    for (int i = i0; i < i0 + 8; ++i) key[i] = 0u;  // 0: no entry (every real key is >= 1)
    if (i0 >= nr) continue;
#pragma unroll
    for (int i = i0; i < i0 + 8; ++i) {
      const uint32_t e = (uint32_t)(64 * i + lane);
      const float sc = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(l_rs, lane * 8, 512 * i, 0));
      key[i] = e < c ? sel_key(sc) : 0u;
      mn = min(mn, e < c ? key[i] : 0xFFFFFFFFu);
      mx = max(mx, key[i]);
    }
  }
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  uint32_t* const hist = hists[wave];
  // radix passes narrow [lo, hi] to the bin holding the k-th largest key; `need` = entries
  // of that bin to keep.  One wave's LDS operations complete in order.
  uint32_t need = (uint32_t)topk, lo = mn, hi = mx, m;
  int sh = sel_shift(lo, hi);
  for (;;) {
    for (int j = lane; j < kSelBins; j += 64) hist[j] = 0;
    // (rounds in groups of eight: entries past the list hold key 0 and never count; one
    // guard per group keeps the per-round conditions from piling up in scalar registers)
#pragma unroll
    for (int i0 = 0; i0 < FZ_EPL; i0 += 8) {
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
  // a bin of m <= 64 entries over several key values: rank them exactly (score, then list
  // position); keptm bit j = the j-th of them in list order is kept
  uint64_t keptm = 0;
  if (sh > 0) {
    uint32_t* const mem = mems[wave];
    uint32_t cm = 0;
#pragma unroll
    for (int i0 = 0; i0 < FZ_EPL; i0 += 8) {
      if (i0 >= nr) continue;
#pragma unroll
      for (int i = i0; i < i0 + 8; ++i) {
        const bool inb = key[i] >= lo && key[i] <= hi;
        const uint64_t bl = __ballot(inb);
        if (inb) mem[cm + mbcnt64(bl)] = key[i];
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
  // emission in list order, eight rounds at a time; the key indices of the next eight rounds
  // are loaded while this one is written (issued before its stores, and the compiler
  // barrier keeps later loads from moving further ahead).
  // Slots stay below k by construction (k - need keys above the bin); the guard keeps a
  // violated invariant inside the row.
  uint32_t acc = 0, before = 0;
  uint32_t kidx[2][8];
#pragma unroll
  for (int u = 0; u < 8; ++u) kidx[0][u] = __builtin_amdgcn_raw_buffer_load_b32(l_rs, lane * 8 + 4, 512 * u, 0);
#pragma unroll
  for (int i0 = 0; i0 < FZ_EPL; i0 += 8) {
    const int cur = (i0 / 8) & 1;
    if (i0 >= nr) continue;  // (uniform; a break would keep the loop from unrolling)
    if (i0 + 8 < nr) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        kidx[cur ^ 1][u] = __builtin_amdgcn_raw_buffer_load_b32(l_rs, lane * 8 + 4, 512 * (i0 + 8 + u), 0);
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t k = key[i0 + u];  // 0 past the list: never kept
      bool kp;
      if (sh > 0) {
        const bool inb = k >= lo && k <= hi;
        const uint64_t bl = __ballot(inb);
        kp = k > hi || (inb && ((keptm >> (before + mbcnt64(bl))) & 1u));
        before += (uint32_t)__popcll(bl);
      } else {  // one key value K* = lo: ties kept lowest position first
        const bool tie = k == lo;
        const uint64_t bl = __ballot(tie);
        kp = k > lo || (tie && before + mbcnt64(bl) < need);
        before += (uint32_t)__popcll(bl);
      }
      const uint64_t bk = __ballot(kp);
      const uint32_t slot = acc + mbcnt64(bk);
      acc += (uint32_t)__popcll(bk);
      if (kp && slot < (uint32_t)topk) out[slot] = (int32_t)kidx[cur][u];
    }
  }
}

// Exact top-k of row r (n > k keys) from recomputed scores, by the whole workgroup.
template <int H_I, int D_I>
__device__ __forceinline__ void fz_exact_row(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                             const uint16_t* __restrict__ w, int Tq, int Tk, int row0, int nrows,
                                             int topk, int b, int r, int64_t n, int32_t* __restrict__ idx,
                                             uint8_t (*wks)[IdxWave<H_I, D_I, 1>::kLdsBytes], uint32_t* hist,
                                             uint32_t (*wc)[FZ_NW], uint32_t* state) {
  using W = IdxWave<H_I, D_I, 1>;
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int t0 = r - r % W::QPT;  // first chunk row of the query tile holding row r
  const int gsel = (r - t0) / W::QPL, qsel = (r - t0) % W::QPL;
  W wv;
  wv.load(q + ((int64_t)b * Tq + row0 + t0) * H_I * D_I, w + ((int64_t)b * Tq + row0 + t0) * H_I, min(W::QPT, nrows - t0));
  const __amdgpu_buffer_rsrc_t k_rs = make_rsrc(k + (int64_t)b * Tk * D_I, (uint32_t)Tk * D_I * 2);
  const int ntiles = (int)((n + 31) / 32), per = (ntiles + FZ_NW - 1) / FZ_NW;
  const int j0 = wave * per, nt = max(0, min(per, ntiles - j0));
  const bool mine = wv.g == gsel;
  // on_key(valid, key index, order key) for every key of this wave's tiles (uniform calls)
  auto pass = [&](auto&& on_key) {
    if (nt > 0)
      wv.run(k_rs, wks[wave], nt, [&](int j) { return 32 * (j0 + j); },
             [&](int, int s0, int, int qq, float tot) {
               const int skey = s0 + wv.col;
               on_key(mine && qq == qsel && skey < n, skey, sel_key(tot));
             });
  };
  // three radix passes of 11, 11 and 10 bits from the top of the key
  uint32_t lo = 1u, hi = 0xFFFFFFFFu, need = (uint32_t)topk;
  int sh = 32 - kSelBinBits;
  for (;;) {
    for (int i = tid; i < kSelBins; i += FZ_NT) hist[i] = 0;
    __syncthreads();
    pass([&](bool v, int, uint32_t key) {
      if (v && key >= lo && key <= hi) atomicAdd(&hist[(key - lo) >> sh], 1u);
    });
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
    sh = max(0, sh - kSelBinBits);
    __syncthreads();
  }
  const uint32_t kstar = lo;
  // keys above K* and ties at K* in each wave's key range, then emission in key order
  uint32_t na = 0, nq = 0;
  pass([&](bool v, int, uint32_t key) {
    na += __popcll(__ballot(v && key > kstar));
    nq += __popcll(__ballot(v && key == kstar));
  });
  if (lane == 0) {
    wc[0][wave] = na;
    wc[1][wave] = nq;
  }
  __syncthreads();
  uint32_t A = 0, E = 0;
  for (int i = 0; i < wave; ++i) {
    A += wc[0][i];
    E += wc[1][i];
  }
  int32_t* out = idx + ((int64_t)b * Tq + row0 + r) * topk;
  pass([&](bool v, int skey, uint32_t key) {
    const bool above = v && key > kstar, tie = v && key == kstar;
    const uint64_t ba = __ballot(above), bt = __ballot(tie);
    const uint32_t ia = mbcnt64(ba), it = E + mbcnt64(bt);
    const uint32_t slot = A + ia + min(it, need);  // below k by construction
    if (above && slot < (uint32_t)topk) out[slot] = skey;
    if (tie && it < need && slot < (uint32_t)topk) out[slot] = skey;
    A += __popcll(ba);
    E += __popcll(bt);
  });
  __syncthreads();  // the workgroup may take another row with the same LDS
}

// ---- 5. rows whose list failed: exact top-k from recomputed scores
template <int H_I, int D_I>
__global__ __launch_bounds__(FZ_NT) void fz_exact_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ w,
                                                         const int32_t* __restrict__ kv_len, int Tq, int Tk, int row0,
                                                         int nrows, int topk, const uint32_t* __restrict__ cnt,
                                                         int32_t* __restrict__ idx) {
  using W = IdxWave<H_I, D_I, 1>;  // one query tile: the row and its tile neighbours
  __shared__ __attribute__((aligned(16))) uint8_t wks[FZ_NW][W::kLdsBytes];
  __shared__ uint32_t hist[kSelBins];
  __shared__ uint32_t wc[2][FZ_NW];
  __shared__ uint32_t state[2];
  // each workgroup checks four rows and recomputes those whose list failed (rare)
  const int b = blockIdx.y;
  for (int rr = 0; rr < FZ_NW; ++rr) {
    const int r = blockIdx.x * FZ_NW + rr;
    if (r >= nrows) return;
    const int64_t n = seq_len(kv_len, b, Tk) - Tq + row0 + r + 1;
    if (n > topk && fz_row_failed(cnt[(int64_t)b * nrows + r], topk))
      fz_exact_row<H_I, D_I>(q, k, w, Tq, Tk, row0, nrows, topk, b, r, n, idx, wks, hist, wc, state);
  }
}

template <int H_I, int D_I>
hipError_t launch_fz(const IndexTopkArgs& A, const FusedLayout& Lw, hipStream_t st) {
  using W = FzWave<H_I, D_I>;
  const int nblocks = (A.nrows + 4 * W::ROWS - 1) / (4 * W::ROWS);
  const float alpha = A.oversample > 0.f ? A.oversample : fused_default_alpha(A.k_top);
  char* ws = reinterpret_cast<char*>(A.ws);
  uint32_t* smp = reinterpret_cast<uint32_t*>(ws + Lw.smp);
  int32_t* ns = reinterpret_cast<int32_t*>(ws + Lw.ns);
  float* thr = reinterpret_cast<float*>(ws + Lw.thr);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(ws + Lw.cnt);
  uint2* list = reinterpret_cast<uint2*>(ws + Lw.list);
  const dim3 wgrid(nblocks, 1, A.B);
  hipLaunchKernelGGL((fz_sample_kernel<H_I, D_I>), wgrid, dim3(256), 0, st, A.q, A.k, A.w, A.kv_len, A.Tq, A.Tk,
                     A.row0, A.nrows, nblocks, smp, Lw.smax, ns);
  hipLaunchKernelGGL(fz_threshold_kernel, dim3((A.nrows + FZ_NW - 1) / FZ_NW, A.B), dim3(FZ_NT), 0, st, smp, Lw.smax,
                     ns, A.kv_len, A.Tq, A.Tk, A.row0,
                     A.nrows, A.k_top, alpha, thr);
  hipLaunchKernelGGL((fz_filter_kernel<H_I, D_I>), wgrid, dim3(256), 0, st, A.q, A.k, A.w, A.kv_len, A.Tq, A.Tk,
                     A.row0, A.nrows, nblocks, A.k_top, thr, cnt, list);
  hipLaunchKernelGGL(fz_select_kernel, dim3((A.nrows + FZ_NW - 1) / FZ_NW, A.B), dim3(FZ_NT), 0, st, cnt, list,
                     A.kv_len, A.Tq, A.Tk, A.row0, A.nrows, A.k_top, A.idx);
  hipLaunchKernelGGL((fz_exact_kernel<H_I, D_I>), dim3((A.nrows + FZ_NW - 1) / FZ_NW, A.B), dim3(FZ_NT), 0, st, A.q, A.k, A.w, A.kv_len, A.Tq, A.Tk,
                     A.row0, A.nrows, A.k_top, cnt, A.idx);
  return hipGetLastError();
}

}  // namespace

FusedLayout fused_layout(int B, int nrows, int Tk) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  FusedLayout L;
  const size_t R = (size_t)std::max(0, B) * (size_t)std::max(0, nrows);
  L.smax = 32 * fz_sample_tiles(std::max(Tk, 1));
  L.smp = 0;
  L.ns = up(R * L.smax * 4);
  L.thr = L.ns + up(R * 4);
  L.cnt = L.thr + up(R * 4);
  L.list = L.cnt + up(R * 4);
  L.bytes = L.list + up(R * (size_t)kFusedCap * 8);
  return L;
}

bool index_topk_fused_supported(int H_I, int d_I, int k) {
  return (H_I == 8 || H_I == 16) && (d_I == 16 || d_I == 32 || d_I == 64 || d_I == 128) && k >= 1 &&
         k <= kFusedMaxK;
}

hipError_t launch_index_topk(const IndexTopkArgs& A, hipStream_t st) {
  if (A.nrows <= 0 || A.B <= 0) return hipSuccess;
  const FusedLayout L = fused_layout(A.B, A.nrows, A.Tk);
#define DSA_FZ_CASE(h, d) \
  if (A.H_I == h && A.d_I == d) return launch_fz<h, d>(A, L, st);
  DSA_FZ_CASE(8, 16) DSA_FZ_CASE(8, 32) DSA_FZ_CASE(8, 64) DSA_FZ_CASE(8, 128)
  DSA_FZ_CASE(16, 16) DSA_FZ_CASE(16, 32) DSA_FZ_CASE(16, 64) DSA_FZ_CASE(16, 128)
#undef DSA_FZ_CASE
  return hipErrorInvalidValue;
}

}  // namespace dsa
