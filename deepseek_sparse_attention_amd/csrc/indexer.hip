// Lightning-indexer scores on gfx950, stored as fp32 score rows:
//   I[t,s] = sum_j w[t,j] * max(0, sum_d q[t,j,d] * k[s,d])   for keys s <= p(t)
// (DSA ablation model card, model list).  The per-wave MFMA core is in indexer_core.hpp; a
// workgroup (4 waves) covers a block of queries against one segment of keys.
#include "indexer_core.hpp"
#include "internal.hpp"

namespace dsa {

namespace {

// PAGED: key s of sequence b sits in row bt[b*max_blocks + s/P]*P + s%P of a shared pool of
// pool_tokens rows (P = 1 << page_shift, a multiple of 32, so no 32-key tile crosses a page).
// wave_keys > 0 (launches with no more rows than one wave holds, e.g. decode): the four
// waves share the same rows and split the workgroup's key segment, wave w taking keys
// [w * wave_keys, (w + 1) * wave_keys) of it, so every wave streams keys.
template <int H_I, int D_I, bool PAGED>
__global__ __launch_bounds__(256, 2) void index_scores_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ w,
    const int32_t* __restrict__ kv_len, int Tq, int Tk, int row0, int nrows, float* __restrict__ scores,
    int64_t ld, int64_t score_bstride, int key_seg, int wave_keys, const int32_t* __restrict__ bt, int max_blocks,
    int page_shift, int64_t pool_tokens) {
  using W = IdxWave<H_I, D_I, idx_query_tiles<H_I, D_I>()>;
  constexpr int QB = 4 * W::ROWS;  // queries per workgroup
  __shared__ __attribute__((aligned(16))) uint8_t wks[4][W::kLdsBytes];
  const int wave = wave_id();
  const int b = blockIdx.z;
  const int64_t L = seq_len(kv_len, b, Tk);
  const int64_t pos_base = L - Tq + row0;  // position of chunk row r is pos_base + r
  const bool wsplit = wave_keys > 0;
  const int wrow0 = wsplit ? blockIdx.x * W::ROWS : blockIdx.x * QB + wave * W::ROWS;
  if (wrow0 >= nrows) return;
  const int wrows = min(W::ROWS, nrows - wrow0);
  const int64_t pmax = pos_base + wrow0 + wrows - 1;  // last position of this wave
  const int64_t seg0 = (int64_t)blockIdx.y * key_seg + (wsplit ? (int64_t)wave * wave_keys : 0);
  if (pmax < 0 || seg0 > pmax) return;
  const int64_t seg_end = min((int64_t)min((int64_t)Tk, seg0 + (wsplit ? wave_keys : key_seg)), pmax + 1);

  W wv;
  wv.load(q + ((int64_t)b * Tq + row0 + wrow0) * H_I * D_I, w + ((int64_t)b * Tq + row0 + wrow0) * H_I, wrows);
  // Range-checked views: keys past Tk (or past the pool) read as zero, and score stores
  // outside this wave's rows are dropped.
  const __amdgpu_buffer_rsrc_t k_rs = PAGED ? make_rsrc(k, (uint32_t)(pool_tokens * D_I * 2))
                                            : make_rsrc(k + (int64_t)b * Tk * D_I, (uint32_t)Tk * D_I * 2);
  float* sw = scores + (int64_t)b * score_bstride + (int64_t)wrow0 * ld;
  const __amdgpu_buffer_rsrc_t s_rs = make_rsrc(sw, (uint32_t)(wrows * ld * 4));
  // Row r = t*QPT + g*QPL + qq of the wave sits at position pos0 + r and score offset
  // r*ld*4; only the lane part (g*QPL) lives in registers (positions and keys fit in 32
  // bits: Tk <= ld <= 2^22).  Rows past the chunk need no mask: their score offsets fall
  // outside the store range and are dropped.
  const int pos0 = (int)(pos_base + wrow0) + wv.g * W::QPL;
  const uint32_t off0 = (uint32_t)(wv.g * W::QPL * ld) * 4u;
  const uint32_t row_bytes = (uint32_t)ld * 4u;
  const int col = wv.col;
  const int s_first = (int)seg0;
  auto start = [&](int j) { return s_first + 32 * j; };
  auto epi = [&](int, int s0, int t, int qq, float tot) {
    // tiles never cross a segment edge, so the causal bound is the only mask
    const int skey = s0 + col;
    const int rr = t * W::QPT + qq;  // row offset from the lane's first row (a constant)
    buf_store_f32(tot, s_rs, skey - rr <= pos0 ? off0 + (uint32_t)rr * row_bytes + (uint32_t)skey * 4u : kOffNone, 0);
  };
  const int ntiles = (int)((seg_end - seg0 + 31) / 32);
  if constexpr (PAGED) {
    // tiles past the sequence (prefetch) clamp to its last table entry; a page id outside
    // the pool reads zeros through the range check
    const int32_t* btb = bt + (int64_t)b * max_blocks;
    const int pmask = (1 << page_shift) - 1;
    wv.template run<W::EPIS>(k_rs, wks[wave], ntiles, start, epi, [](int) {}, [&](int j) {
      const int s0 = start(j);
      return (btb[min(s0 >> page_shift, max_blocks - 1)] << page_shift) + (s0 & pmask);
    });
  } else {
    wv.template run<W::EPIS>(k_rs, wks[wave], ntiles, start, epi);
  }
}

template <int H_I, int D_I>
hipError_t launch_t(const IndexerArgs& A, hipStream_t st) {
  const bool paged = A.block_table != nullptr;
  constexpr int ROWS = idx_query_tiles<H_I, D_I>() * (32 / H_I);  // query rows per wave
  constexpr int QB = 4 * ROWS;
  const bool wsplit = A.nrows <= ROWS;  // one wave's rows: the waves split keys instead
  const int qblocks = wsplit ? 1 : (A.nrows + QB - 1) / QB;
  // keys any row of the chunk can see (kv_len <= Tk)
  const int64_t maxkeys = std::min<int64_t>(A.Tk, (int64_t)A.Tk - A.Tq + A.row0 + A.nrows);
  if (qblocks == 0 || maxkeys <= 0) return hipSuccess;
  const int64_t tiles = (maxkeys + 31) / 32;
  // Aim at ~2048 workgroups per launch when query blocks are full (prefill chunks): twice
  // what the chip holds at once, with segments short enough that the causal tail of a launch
  // stays small.  Few-row launches keep ~1024 workgroups; with the waves splitting keys
  // (one wave's rows) a segment is a multiple of four tiles.
  const int64_t target = A.nrows >= 8 * QB ? 2048 : 1024;
  int64_t segs = std::max<int64_t>(1, std::min<int64_t>(tiles, target / std::max<int64_t>(1, (int64_t)qblocks * A.B)));
  int64_t seg_tiles = (tiles + segs - 1) / segs;
  if (wsplit) seg_tiles = (seg_tiles + 3) / 4 * 4;
  segs = (tiles + seg_tiles - 1) / seg_tiles;
  const int wave_keys = wsplit ? (int)(seg_tiles / 4 * 32) : 0;
  dim3 grid(qblocks, (unsigned)segs, A.B);
  if (paged)
    hipLaunchKernelGGL((index_scores_kernel<H_I, D_I, true>), grid, dim3(256), 0, st, A.q, A.k, A.w, A.kv_len, A.Tq,
                       A.Tk, A.row0, A.nrows, A.scores, A.ld, A.score_bstride, (int)(seg_tiles * 32), wave_keys,
                       A.block_table, A.max_blocks, A.page_shift, A.pool_tokens);
  else
    hipLaunchKernelGGL((index_scores_kernel<H_I, D_I, false>), grid, dim3(256), 0, st, A.q, A.k, A.w, A.kv_len, A.Tq,
                       A.Tk, A.row0, A.nrows, A.scores, A.ld, A.score_bstride, (int)(seg_tiles * 32), wave_keys,
                       nullptr, 0, 0, (int64_t)0);
  return hipGetLastError();
}

}  // namespace

bool indexer_supported(int H_I, int d_I, int64_t ld) {
  // a wave's score rows (at most 4 * 32/H_I of them) are addressed with 32-bit byte offsets
  return (H_I == 1 || H_I == 2 || H_I == 4 || H_I == 8 || H_I == 16) &&
         (d_I == 16 || d_I == 32 || d_I == 64 || d_I == 128) && ld <= kIndexerMaxLd;
}

hipError_t launch_index_scores(const IndexerArgs& A, hipStream_t st) {
#define DSA_IDX_CASE(h, d) \
  if (A.H_I == h && A.d_I == d) return launch_t<h, d>(A, st);
#define DSA_IDX_D(h) DSA_IDX_CASE(h, 16) DSA_IDX_CASE(h, 32) DSA_IDX_CASE(h, 64) DSA_IDX_CASE(h, 128)
  DSA_IDX_D(1) DSA_IDX_D(2) DSA_IDX_D(4) DSA_IDX_D(8) DSA_IDX_D(16)
#undef DSA_IDX_D
#undef DSA_IDX_CASE
  return hipErrorInvalidValue;
}

}  // namespace dsa
