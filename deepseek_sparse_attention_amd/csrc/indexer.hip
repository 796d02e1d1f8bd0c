// Lightning-indexer scores on gfx950, stored as fp32 score rows:
//   I[t,s] = sum_j w[t,j] * max(0, sum_d q[t,j,d] * k[s,d])   for keys s <= p(t)
// (DSA ablation model card, model list).  The per-wave MFMA core is in indexer_core.hpp; a
// workgroup (4 waves) covers a block of queries against one segment of keys.
#include "indexer_core.hpp"
#include "internal.hpp"
#include "seglist.hpp"

namespace dsa {

namespace {

// PAGED: key s of sequence b sits in row bt[b*max_blocks + s/P]*P + s%P of a shared pool of
// pool_tokens rows (P = 1 << page_shift, a multiple of 32, so no 32-key tile crosses a page).
// wave_keys > 0 (launches with no more rows than one wave holds, e.g. decode): the four
// waves share the same rows and split the workgroup's key segment, wave w taking keys
// [w * wave_keys, (w + 1) * wave_keys) of it, so every wave streams keys.
// A launch of one query tile per wave (QP 1: decode) with at least 8 heads keeps its scores
// out of the key stream: stores and loads share one in-order completion count, so the next
// key wait after a store covers the store's write too (on the 64 x 65536 decode keys: 99.6
// us with a store per tile, 81.5 us with no stores at all).  HOLD > 0 (the wave's rows x key
// tiles fit HOLD): the wave keeps all its scores in LDS and writes them once its stream has
// ended (91.0 us, two workgroups per CU for the LDS); otherwise it stages them in LDS and
// writes 1 KB at a time, 16 bytes per lane, one row's scores every eight tiles (97.6-98.1
// us, three workgroups per CU).
// sp_lists (held launches of one row per sequence, key_seg one or two top-k segments): the
// workgroup also builds the split top-k's segment lists and meta words (seglist.hpp) for
// its key range from the scores it holds, so that the top-k that follows is the merge alone.
template <int H_I, int D_I, bool PAGED, int QP = idx_query_tiles<H_I, D_I>(), int HOLD = 0>
__global__ __launch_bounds__(256, 2) void index_scores_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ w,
    const int32_t* __restrict__ kv_len, int Tq, int Tk, int row0, int nrows, float* __restrict__ scores,
    int64_t ld, int64_t score_bstride, int key_seg, int wave_keys, const int32_t* __restrict__ bt, int max_blocks,
    int page_shift, int64_t pool_tokens, uint2* __restrict__ sp_lists, int sp_k) {
  using W = IdxWave<H_I, D_I, QP, QP == 1>;  // one query tile per wave: keys read once
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
  // segment lists: a row that takes them (one row: the launch passes lists only then), and a
  // workgroup whose key range starts inside it; every wave then stays for the lists' barriers
  const int64_t wg_key0 = (int64_t)blockIdx.y * key_seg;
  const bool lists = HOLD > 0 && sp_lists != nullptr && pmax >= wg_key0 && sp_uses_lists((int)min<int64_t>(pmax + 1, SP_ROW_MAX + 1), sp_k);
  const bool live = !(pmax < 0 || seg0 > pmax);
  if (!live && !lists) return;
  const int64_t seg_end = min((int64_t)min((int64_t)Tk, seg0 + (wsplit ? wave_keys : key_seg)), pmax + 1);

  W wv;
  wv.load(q + ((int64_t)b * Tq + row0 + wrow0) * H_I * D_I, w + ((int64_t)b * Tq + row0 + wrow0) * H_I, wrows);
  // Range-checked views: keys past Tk (or past the pool) read as zero, and score stores
  // outside this wave's rows are dropped.
  const __amdgpu_buffer_rsrc_t k_rs = PAGED ? make_rsrc(k, (uint32_t)(pool_tokens * D_I * 2))
                                            : make_rsrc(k + (int64_t)b * Tk * D_I, (uint32_t)Tk * D_I * 2);
  float* sw = scores + (int64_t)b * score_bstride + (int64_t)wrow0 * ld;
  const u32x4 s_rs = rsrc_words(sw, (uint32_t)(wrows * ld * 4));
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
    // one store instruction per call: the key pipeline's waits count EPIS per tile
    buf_store1_b32(__float_as_uint(tot), s_rs,
                   skey - rr <= pos0 ? off0 + (uint32_t)rr * row_bytes + (uint32_t)skey * 4u : kOffNone);
  };
  const int ntiles = (int)((seg_end - seg0 + 31) / 32);
  // tiles past the sequence (prefetch) clamp to its last table entry; a page id outside
  // the pool reads zeros through the range check
  const int32_t* btb = PAGED ? bt + (int64_t)b * max_blocks : nullptr;
  const int pmask = (1 << page_shift) - 1;
  auto phys = [&](int j) {
    const int s0 = start(j);
    return PAGED ? (btb[min(s0 >> page_shift, max_blocks - 1)] << page_shift) + (s0 & pmask) : s0;
  };
  if constexpr (HOLD > 0) {
    static_assert(QP == 1 && W::QPT <= 4, "held scores: one query tile per wave");
    // row r of tile j at held[wave][(r ntiles + j) 32 + col]: each row's keys contiguous
    // (the launch checks R * ntiles <= HOLD)
    __shared__ __attribute__((aligned(16))) float held[4][HOLD * 32];
    const int R = wrows <= 1 ? 1 : wrows <= 2 ? 2 : 4;
    float* hw = held[wave];
    auto epi1 = [&](int j, int, int, int qq, float tot) {
      const int r = wv.g * W::QPL + qq;
      if (r < R) hw[(r * ntiles + j) * 32 + col] = tot;
    };
    if (live) wv.template run<0>(k_rs, wks[wave], ntiles, start, epi1, [](int) {}, phys);
    // (run ends with every key load done; this wave alone wrote hw, in program order)
    const int lane = threadIdx.x & 63;
    const int nchunk = live ? 8 * ntiles : 0;  // 16-byte chunks per row
    const int kend = s_first + 32 * ntiles;
    for (int r = 0; r < R; ++r) {
      const int fpos = (int)(pos_base + wrow0) + r;  // rows past the wave's drop out of the range
      for (int c = lane; c < nchunk; c += 64) {
        const int key = s_first + 4 * c;
        const u32x4 v = *reinterpret_cast<const u32x4*>(&hw[r * ntiles * 32 + 4 * c]);
        const uint32_t off = (uint32_t)r * row_bytes + (uint32_t)key * 4u;
        if (key + 3 <= fpos && key + 3 < kend) {
          buf_store1_b128(v, s_rs, off);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            buf_store1_b32(v[e], s_rs, key + e <= fpos && key + e < kend ? off + 4u * e : kOffNone);
        }
      }
    }
    if constexpr (4 * W::kLdsBytes >= 2 * sizeof(SpScratch)) {
      if (lists) {
        // one row (wrows 1): the workgroup's scores, key wg_key0 + w * wave_keys + o at
        // held[w][o], become the keys of its one or two segments; the key tile buffers, free
        // once every wave's stream has ended, hold the selection's LDS
        __syncthreads();
        SpScratch* sc = reinterpret_cast<SpScratch*>(&wks[0][0]);
        const int n = (int)(pmax + 1);
        const int S = (n + SP_SEG - 1) / SP_SEG;
        uint4* meta = reinterpret_cast<uint4*>(sp_lists + (int64_t)gridDim.z * nrows * SP_MAXSEG * SP_CAP);
        auto build = [&](auto nseg_tag) {
          constexpr int NSEG = decltype(nseg_tag)::value;
          uint32_t key[NSEG][16];
          int nv[NSEG], s0[NSEG];
          uint2* lst[NSEG];
          uint4* mt[NSEG];
          const int tid = threadIdx.x;
#pragma unroll
          for (int g = 0; g < NSEG; ++g) {
            s0[g] = (int)wg_key0 + g * SP_SEG;
            nv[g] = max(0, min(SP_SEG, n - s0[g]));
            const int64_t slot = ((int64_t)b * nrows + wrow0) * SP_MAXSEG + s0[g] / SP_SEG;
            lst[g] = sp_lists + slot * SP_CAP;
            mt[g] = meta + slot;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int rel = g * SP_SEG + 1024 * i + 4 * tid;  // (a multiple of 4: one wave's range)
              const u32x4 v = *reinterpret_cast<const u32x4*>(&held[rel / wave_keys][rel % wave_keys]);
#pragma unroll
              for (int e = 0; e < 4; ++e)
                key[g][4 * i + e] = (1024 * i + 4 * tid + e < nv[g]) ? sel_key(__uint_as_float(v[e])) : 0u;
            }
          }
          sp_make_lists<NSEG>(key, nv, s0, S, sp_k, lst, mt, sc);
        };
        if (key_seg == 2 * SP_SEG)
          build(std::integral_constant<int, 2>{});
        else
          build(std::integral_constant<int, 1>{});
      }
    }
  } else if constexpr (QP == 1 && W::QPT <= 4) {
    // Scores of the wave's R real rows (its row count rounded up to a power of two) over G
    // consecutive tiles, G = 8 / R (32 G keys), in LDS: row r of tile j at
    // stg[wave][(r G + j % G) 32 + col] (lane group g holds rows g QPL .. g QPL + QPL - 1);
    // flushed after the group's last tile, lane l writing keys 4 (l % 8G) .. +3 of row
    // l / 8G: 1 KB per flush, 16 bytes per lane (rows past the wave's drop out of the range)
    const int R = wrows <= 1 ? 1 : wrows <= 2 ? 2 : 4;  // (wrows <= QPT <= 4)
    const int G = 8 / R;
    __shared__ __attribute__((aligned(16))) float stg[4][256];
    const int lane = threadIdx.x & 63, frow = lane / (8 * G), fk = 4 * (lane % (8 * G));
    const int fpos = (int)(pos_base + wrow0) + frow;  // position of the flushed row
    const int kend = s_first + 32 * ntiles;            // past the wave's last tile
    auto epi1 = [&](int j, int, int, int qq, float tot) {
      const int r = wv.g * W::QPL + qq;
      if (r < R) stg[wave][(r * G + j % G) * 32 + col] = tot;
    };
    auto post1 = [&](int j) {
      if (j % G != G - 1 && j != ntiles - 1) return;
      const int key = start(j - j % G) + fk;  // this lane's first key (tiles are contiguous)
      const u32x4 v = *reinterpret_cast<const u32x4*>(&stg[wave][frow * 32 * G + fk]);
      const uint32_t off = (uint32_t)frow * row_bytes + (uint32_t)key * 4u;
      if (key + 3 <= fpos && key + 3 < kend) {
        buf_store1_b128(v, s_rs, off);
      } else {  // the causal edge, or a last group of fewer than G tiles: only computed keys
#pragma unroll
        for (int e = 0; e < 4; ++e)
          buf_store1_b32(v[e], s_rs, key + e <= fpos && key + e < kend ? off + 4u * e : kOffNone);
      }
    };
    // EPI_VM 0: a flush comes every G tiles, so no tile has a store to count on
    wv.template run<0>(k_rs, wks[wave], ntiles, start, epi1, post1, phys);
  } else {
    wv.template run<W::EPIS>(k_rs, wks[wave], ntiles, start, epi, [](int) {}, phys);
  }
}

// Held-score launches: tiles of scores per wave (R rows x tiles), workgroups per CU.
constexpr int kIdxHoldTiles = 64;
constexpr int kIdxHoldPerCu = 2;

template <int H_I, int D_I>
hipError_t launch_t(const IndexerArgs& A, hipStream_t st) {
  const bool paged = A.block_table != nullptr;
  constexpr int ROWS = idx_query_tiles<H_I, D_I>() * (32 / H_I);  // query rows per wave
  constexpr int QB = 4 * ROWS;
  const bool wsplit = A.nrows <= ROWS;  // one wave's rows: the waves split keys instead
  // rows of one query tile (decode: one query per sequence) need no more MFMA and epilogue
  // work than that tile: the key-streaming launch then uses one query tile per wave
  constexpr int ROWS1 = 32 / H_I;
  const bool one_tile = wsplit && A.nrows <= ROWS1;
  const int qblocks = wsplit ? 1 : (A.nrows + QB - 1) / QB;
  // keys any row of the chunk can see (kv_len <= Tk)
  const int64_t maxkeys = std::min<int64_t>(A.Tk, (int64_t)A.Tk - A.Tq + A.row0 + A.nrows);
  if (qblocks == 0 || maxkeys <= 0) return hipSuccess;
  const int64_t tiles = (maxkeys + 31) / 32;
  // Aim at ~2048 workgroups per launch when query blocks are full (prefill chunks): twice
  // what the chip holds at once, with segments short enough that the causal tail of a launch
  // stays small.  Other few-row launches take ~1536.  A launch of one query tile (decode)
  // streams its keys once, in one round of resident workgroups: 512 held-score workgroups
  // (two per CU) when their scores fit, else 768 staging ones (three per CU; measured on the
  // 64 x 65536 decode key cache before the held variant: 99.0 us against 101.6 at 512, 104.3
  // at 640, 103.6 at 1024, 101.7 at 1536 and 104.9 at 2304).  With the waves splitting keys
  // (one wave's rows) a segment is a multiple of four tiles.
  auto plan = [&](int64_t target, int64_t& segs, int64_t& seg_tiles) {
    segs = std::max<int64_t>(1, std::min<int64_t>(tiles, target / std::max<int64_t>(1, (int64_t)qblocks * A.B)));
    seg_tiles = (tiles + segs - 1) / segs;
    if (wsplit) seg_tiles = (seg_tiles + 3) / 4 * 4;
    segs = (tiles + seg_tiles - 1) / seg_tiles;
  };
  int64_t segs, seg_tiles;
  plan(A.nrows >= 8 * QB ? 2048 : one_tile ? 3 * (int64_t)device_cus() : 1536, segs, seg_tiles);
  // A launch of one query tile whose waves' scores fit the held-score LDS runs the held
  // variant instead: its LDS allows two workgroups per CU, so one round of them is 512.
  bool hold = false;
  if (one_tile && H_I >= 8 && D_I <= 64) {  // (128-wide keys: their tile buffers leave no room)
    int64_t hsegs, htiles;
    plan(kIdxHoldPerCu * (int64_t)device_cus(), hsegs, htiles);
    const int64_t R = A.nrows <= 1 ? 1 : A.nrows <= 2 ? 2 : 4;
    if (R * (htiles / 4) <= kIdxHoldTiles) {
      hold = true;
      segs = hsegs;
      seg_tiles = htiles;
    }
  }
  const int wave_keys = wsplit ? (int)(seg_tiles / 4 * 32) : 0;
  // the split top-k's segment lists, built by held workgroups of one row per sequence whose
  // key range is one or two whole segments (their LDS must hold two segments' selection)
  const bool lists = hold && A.topk_ws != nullptr && A.topk_k > 0 && A.nrows == 1 && D_I >= 32 &&
                     A.Tk <= SP_ROW_MAX && (seg_tiles * 32 == SP_SEG || seg_tiles * 32 == 2 * SP_SEG);
  if (A.lists_made) *A.lists_made = lists;
  uint2* sp_lists = lists ? reinterpret_cast<uint2*>(A.topk_ws) : nullptr;
  dim3 grid(qblocks, (unsigned)segs, A.B);
#define DSA_IDX_LAUNCH(PG, QP, HOLD)                                                                                  \
  hipLaunchKernelGGL((index_scores_kernel<H_I, D_I, PG, QP, HOLD>), grid, dim3(256), 0, st, A.q, A.k, A.w, A.kv_len, \
                     A.Tq, A.Tk, A.row0, A.nrows, A.scores, A.ld, A.score_bstride, (int)(seg_tiles * 32), wave_keys, \
                     PG ? A.block_table : nullptr, PG ? A.max_blocks : 0, PG ? A.page_shift : 0,                    \
                     PG ? A.pool_tokens : (int64_t)0, sp_lists, A.topk_k)
  constexpr int QPF = idx_query_tiles<H_I, D_I>();
  constexpr int HT = H_I >= 8 && D_I <= 64 ? kIdxHoldTiles : 0;  // (a held instance only where it runs)
  if (paged && hold)
    DSA_IDX_LAUNCH(true, 1, HT);
  else if (paged && one_tile)
    DSA_IDX_LAUNCH(true, 1, 0);
  else if (paged)
    DSA_IDX_LAUNCH(true, QPF, 0);
  else if (hold)
    DSA_IDX_LAUNCH(false, 1, HT);
  else if (one_tile)
    DSA_IDX_LAUNCH(false, 1, 0);
  else
    DSA_IDX_LAUNCH(false, QPF, 0);
#undef DSA_IDX_LAUNCH
  return hipGetLastError();
}

// Entries s = p+1 .. ld-1 of every score row (keys a query cannot see, and the row's
// padding past Tk) become -inf, so a caller's row is defined everywhere.  One workgroup
// per row: scalar stores up to a 16-byte boundary, then 16-byte stores, then the tail.
__global__ __launch_bounds__(256) void fill_masked_kernel(float* __restrict__ scores, int64_t ld,
                                                          int64_t score_bstride, const int32_t* __restrict__ kv_len,
                                                          int Tq, int Tk) {
  const int b = blockIdx.y;
  const int r = blockIdx.x;
  const int64_t p = seq_len(kv_len, b, Tk) - Tq + r;  // last visible key (< 0: none)
  const int64_t s0 = p < 0 ? 0 : p + 1;
  if (s0 >= ld) return;
  float* row = scores + (int64_t)b * score_bstride + (int64_t)r * ld;
  const float ninf = -INFINITY;
  // first 16-byte-aligned entry at or after s0
  const int64_t mis = (int64_t)((reinterpret_cast<uintptr_t>(row + s0) >> 2) & 3);
  const int64_t a0 = min(ld, s0 + ((4 - mis) & 3));
  const int64_t nvec = (ld - a0) >> 2;
  for (int64_t s = s0 + threadIdx.x; s < a0; s += 256) row[s] = ninf;
  float4* v = reinterpret_cast<float4*>(row + a0);
  for (int64_t i = threadIdx.x; i < nvec; i += 256) v[i] = make_float4(ninf, ninf, ninf, ninf);
  for (int64_t s = a0 + 4 * nvec + threadIdx.x; s < ld; s += 256) row[s] = ninf;
}

}  // namespace

hipError_t launch_fill_masked(float* scores, int64_t ld, int64_t score_bstride, const int32_t* kv_len, int B, int Tq,
                              int Tk, hipStream_t st) {
  if ((int64_t)B * Tq == 0 || ld == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_masked_kernel, dim3((unsigned)Tq, (unsigned)B), dim3(256), 0, st, scores, ld, score_bstride,
                     kv_len, Tq, Tk);
  return hipGetLastError();
}

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
