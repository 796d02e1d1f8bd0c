// Lightning-indexer scores on gfx950:
//   I[t,s] = sum_j w[t,j] * max(0, sum_d q[t,j,d] * k[s,d])   for keys s <= p(t)
// (DSA ablation model card, model list: ReLU indexer with a few small heads; one key per
// token shared by the heads, as its parameter count fixes).
//
// One 32x32x16 bf16 MFMA tile covers 32 (query, head) rows against 32 keys.  The rows are
// ordered so that the 16 accumulator values of a lane are all H_I heads of 16/H_I queries
// for one key: the ReLU and the head-weighted sum then run inside the lane, with no
// cross-lane traffic, and each lane ends with finished scores.  A wave keeps QP query
// tiles of Q in registers and streams key tiles; a workgroup (4 waves) covers a block of
// queries against one segment of keys.
#include "common.hpp"
#include "internal.hpp"

namespace dsa {

namespace {

constexpr int kQP = 4;  // query tiles per wave

template <int H_I, int D_I>
__global__ __launch_bounds__(256, 2) void index_scores_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ w,
    const int32_t* __restrict__ kv_len, int Tq, int Tk, int row0, int nrows, float* __restrict__ scores,
    int64_t ld, int64_t score_bstride, int key_seg) {
  constexpr int QPT = 32 / H_I;          // queries per MFMA tile
  constexpr int QPL = 16 / H_I;          // queries per lane (per tile)
  constexpr int KS = D_I / 16;           // MFMA k-steps over the indexer width
  constexpr int QB = 4 * kQP * QPT;      // queries per workgroup
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.z;
  const int64_t L = seq_len(kv_len, b, Tk);
  const int64_t pos_base = L - Tq + row0;  // position of chunk row r is pos_base + r
  const int wrow0 = blockIdx.x * QB + wave * kQP * QPT;
  if (wrow0 >= nrows) return;
  const int wrows = min(kQP * QPT, nrows - wrow0);
  const int64_t pmax = pos_base + wrow0 + wrows - 1;  // last position of this wave
  const int64_t seg0 = (int64_t)blockIdx.y * key_seg;
  if (pmax < 0 || seg0 > pmax) return;
  const int64_t seg_end = min((int64_t)min((int64_t)Tk, seg0 + key_seg), pmax + 1);

  // A operand: lane row m = lane%32 <-> (query, head) such that D lane group g = lane/32
  // holds all heads of queries g*QPL .. g*QPL+QPL-1 of the tile.
  const int m = lane & 31;
  const int mi = (m >> 3) * 4 + (m & 3);         // accumulator slot of row m
  const int mq = ((m >> 2) & 1) * QPL + mi / H_I; // query within tile
  const int mh = mi % H_I;                        // head
  const int kh = (lane >> 5) * 8;                 // k offset of this lane within a k-step
  bf16x8 a[kQP][KS];
#pragma unroll
  for (int t = 0; t < kQP; ++t) {
    const int r = wrow0 + t * QPT + mq;
    const bool ok = r < nrows;
    const uint16_t* src = q + (((int64_t)b * Tq + row0 + (ok ? r : 0)) * H_I + mh) * D_I + kh;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 v = ok ? ld16(src + s * 16) : u32x4{0, 0, 0, 0};
      a[t][s] = as_bf16x8(v);
    }
  }
  // head weights of the lane's queries (fp32), and their positions
  const int g = lane >> 5;
  float wt[kQP][16];
  int64_t qpos[kQP][QPL];
  int qrow[kQP][QPL];
#pragma unroll
  for (int t = 0; t < kQP; ++t) {
#pragma unroll
    for (int qq = 0; qq < QPL; ++qq) {
      const int r = wrow0 + t * QPT + g * QPL + qq;
      const bool ok = r < nrows;
      qrow[t][qq] = ok ? r : -1;
      qpos[t][qq] = ok ? pos_base + r : -1;
#pragma unroll
      for (int h = 0; h < H_I; ++h)
        wt[t][qq * H_I + h] = ok ? bf16_bits_to_f32(w[((int64_t)b * Tq + row0 + r) * H_I + h]) : 0.f;
    }
  }

  const int col = lane & 31;
  const uint16_t* kbase = k + (int64_t)b * Tk * D_I + kh;
  float* sbase = scores + (int64_t)b * score_bstride;
  for (int64_t s0 = seg0; s0 < seg_end; s0 += 32) {
    const int64_t key = min(s0 + col, (int64_t)Tk - 1);
    bf16x8 bk[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) bk[s] = as_bf16x8(ld16(kbase + key * D_I + s * 16));
    const int64_t skey = s0 + col;
#pragma unroll
    for (int t = 0; t < kQP; ++t) {
      if (t * QPT >= wrows) break;
      f32x16 acc = {};
#pragma unroll
      for (int s = 0; s < KS; ++s) acc = mfma32(a[t][s], bk[s], acc);
#pragma unroll
      for (int qq = 0; qq < QPL; ++qq) {
        float tot = wt[t][qq * H_I] * fmaxf(acc[qq * H_I], 0.f);
#pragma unroll
        for (int h = 1; h < H_I; ++h) tot = fmaf(wt[t][qq * H_I + h], fmaxf(acc[qq * H_I + h], 0.f), tot);
        if (skey <= qpos[t][qq] && skey < seg_end) sbase[(int64_t)qrow[t][qq] * ld + skey] = tot;
      }
    }
  }
}

template <int H_I, int D_I>
hipError_t launch_t(const IndexerArgs& A, hipStream_t st) {
  constexpr int QB = 4 * kQP * (32 / H_I);
  const int qblocks = (A.nrows + QB - 1) / QB;
  // keys any row of the chunk can see (kv_len <= Tk)
  const int64_t maxkeys = std::min<int64_t>(A.Tk, (int64_t)A.Tk - A.Tq + A.row0 + A.nrows);
  if (qblocks == 0 || maxkeys <= 0) return hipSuccess;
  const int64_t tiles = (maxkeys + 31) / 32;
  // enough workgroups to fill the chip: aim at ~1024 workgroups per launch
  int64_t segs = std::max<int64_t>(1, std::min<int64_t>(tiles, 1024 / std::max<int64_t>(1, (int64_t)qblocks * A.B)));
  int64_t seg_tiles = (tiles + segs - 1) / segs;
  segs = (tiles + seg_tiles - 1) / seg_tiles;
  dim3 grid(qblocks, (unsigned)segs, A.B);
  hipLaunchKernelGGL((index_scores_kernel<H_I, D_I>), grid, dim3(256), 0, st, A.q, A.k, A.w, A.kv_len, A.Tq,
                     A.Tk, A.row0, A.nrows, A.scores, A.ld, A.score_bstride, (int)(seg_tiles * 32));
  return hipGetLastError();
}

}  // namespace

bool indexer_supported(int H_I, int d_I) {
  return (H_I == 1 || H_I == 2 || H_I == 4 || H_I == 8 || H_I == 16) &&
         (d_I == 16 || d_I == 32 || d_I == 64 || d_I == 128);
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
