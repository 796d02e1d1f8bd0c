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

// Query tiles per wave: as many (up to four) as fit the register file without spilling,
// next to the weights and the key pipeline (two tiles of rows, two of operands).
template <int H_I, int D_I>
constexpr int query_tiles() {
  if (D_I <= 32 || (D_I == 64 && H_I >= 8)) return 4;
  return (D_I == 64 && H_I >= 2) || H_I >= 8 ? 2 : 1;
}

template <int H_I, int D_I>
__global__ __launch_bounds__(256, 2) void index_scores_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ w,
    const int32_t* __restrict__ kv_len, int Tq, int Tk, int row0, int nrows, float* __restrict__ scores,
    int64_t ld, int64_t score_bstride, int key_seg) {
  constexpr int QPT = 32 / H_I;          // queries per MFMA tile
  constexpr int QPL = 16 / H_I;          // queries per lane (per tile)
  constexpr int KS = D_I / 16;           // MFMA k-steps over the indexer width
  constexpr int kQP = query_tiles<H_I, D_I>();
  constexpr int QB = 4 * kQP * QPT;      // queries per workgroup
  const int lane = threadIdx.x & 63, wave = wave_id();
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

  // Range-checked views: rows past the chunk read as zero, keys past Tk read as zero,
  // and score stores outside this wave's rows are dropped.
  const uint16_t* qw = q + ((int64_t)b * Tq + row0 + wrow0) * H_I * D_I;
  const __amdgpu_buffer_rsrc_t q_rs = make_rsrc(qw, (uint32_t)wrows * H_I * D_I * 2);
  const __amdgpu_buffer_rsrc_t k_rs = make_rsrc(k + (int64_t)b * Tk * D_I, (uint32_t)Tk * D_I * 2);
  float* sw = scores + (int64_t)b * score_bstride + (int64_t)wrow0 * ld;
  const __amdgpu_buffer_rsrc_t s_rs = make_rsrc(sw, (uint32_t)(wrows * ld * 4));

  // A operand: lane row m = lane%32 <-> (query, head) such that D lane group g = lane/32
  // holds all heads of queries g*QPL .. g*QPL+QPL-1 of the tile.
  const int m = lane & 31;
  const int mi = (m >> 3) * 4 + (m & 3);          // accumulator slot of row m
  const int mq = ((m >> 2) & 1) * QPL + mi / H_I;  // query within tile
  const int mh = mi % H_I;                         // head
  const int kh = (lane >> 5) * 8;                  // k offset of this lane within a k-step
  bf16x8 a[kQP][KS];
#pragma unroll
  for (int t = 0; t < kQP; ++t) {
    const uint32_t off = (uint32_t)(((t * QPT + mq) * H_I + mh) * D_I + kh) * 2;
#pragma unroll
    for (int s = 0; s < KS; ++s) a[t][s] = as_bf16x8(buf_load_16(q_rs, off + s * 32, 0));
  }
  // head weights of the lane's queries (fp32)
  const int g = lane >> 5;
  const __amdgpu_buffer_rsrc_t w_rs =
      make_rsrc(w + ((int64_t)b * Tq + row0 + wrow0) * H_I, (uint32_t)wrows * H_I * 2);
  float wt[kQP][16];
#pragma unroll
  for (int t = 0; t < kQP; ++t) {
#pragma unroll
    for (int qq = 0; qq < QPL; ++qq) {
      const int r = t * QPT + g * QPL + qq;  // row within the wave
      if constexpr (H_I == 1) {  // a lone bf16 weight: 2-byte aligned only
        const uint32_t bits = __builtin_amdgcn_raw_buffer_load_b16(w_rs, r * 2, 0, 0);
        wt[t][qq] = __uint_as_float(bits << 16);
      } else {  // head pairs: 4-byte aligned
#pragma unroll
        for (int h = 0; h < H_I; h += 2) {
          const uint32_t bits = __builtin_amdgcn_raw_buffer_load_b32(w_rs, (r * H_I + h) * 2, 0, 0);
          wt[t][qq * H_I + h] = __uint_as_float(bits << 16);
          wt[t][qq * H_I + h + 1] = __uint_as_float(bits & 0xFFFF0000u);
        }
      }
    }
  }

  // Row r = t*QPT + g*QPL + qq of the wave sits at position pos0 + r and score offset
  // r*ld*4; only the lane part (g*QPL) lives in registers (positions and keys fit in 32
  // bits: Tk <= ld <= 2^22).  Rows past the chunk need no mask: their score offsets fall
  // outside the store range and are dropped.
  const int pos0 = (int)(pos_base + wrow0) + g * QPL;
  const uint32_t off0 = (uint32_t)(g * QPL * ld) * 4u;
  const uint32_t row_bytes = (uint32_t)ld * 4u;
  const int col = lane & 31;
  const int kend = (int)seg_end;
  // Key tiles pass through a private LDS buffer of the wave: global loads then read whole
  // key rows (KPI keys of D_I*2 bytes per instruction) rather than 32 keys x 16 bytes in the
  // MFMA operand layout, and the operand comes back with one ds_read_b128 per k-step.  Only
  // this wave touches its buffer and LDS operations of one wave complete in order, so no
  // barrier is needed.
  constexpr uint32_t kTileBytes = 32 * D_I * 2;
  constexpr int CPK = D_I / 8;   // 16-byte chunks per key row
  constexpr int KPI = 64 / CPK;  // keys per load instruction
  constexpr int NLD = 32 / KPI;  // load instructions per tile
  __shared__ __attribute__((aligned(16))) uint8_t wks[4][2][kTileBytes];
  uint8_t* const wk0 = wks[wave][0];
  uint8_t* const wk1 = wks[wave][1];
  // chunk c of key j sits at chunk position c ^ ((j/2) mod 8): the row-wise writes and the
  // operand reads (32 keys, one chunk each) both spread over all banks
  auto kl_off = [](int key, int chunk) {
    return key * (D_I * 2) + ((chunk ^ ((key >> 1) & (CPK < 8 ? CPK - 1 : 7))) << 4);
  };
  const int lk = lane / CPK, lc = lane % CPK;
  uint32_t gkoff = (uint32_t)(((int)seg0 + lk) * D_I + lc * 8) * 2;
  auto gload = [&](u32x4 (&gr)[NLD]) {  // keys past Tk read as zero
#pragma unroll
    for (int i = 0; i < NLD; ++i) gr[i] = buf_load_16(k_rs, gkoff + i * KPI * D_I * 2, 0);
    gkoff += kTileBytes;
  };
  auto lstore = [&](uint8_t* wk, const u32x4 (&gr)[NLD]) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) *reinterpret_cast<u32x4*>(wk + kl_off(i * KPI + lk, lc)) = gr[i];
  };
  auto lread = [&](const uint8_t* wk, bf16x8 (&bk)[KS]) {  // B operand: key col, dims 16s + 8g
#pragma unroll
    for (int s = 0; s < KS; ++s) bk[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(wk + kl_off(col, 2 * s + g)));
  };
  auto tile = [&](int s0, const bf16x8 (&bk)[KS]) {
    const int skey = s0 + col;
#pragma unroll
    for (int t = 0; t < kQP; ++t) {
      f32x16 acc = {};
#pragma unroll
      for (int s = 0; s < KS; ++s) acc = mfma32(a[t][s], bk[s], acc);
#pragma unroll
      for (int qq = 0; qq < QPL; ++qq) {
        float tot = wt[t][qq * H_I] * relu(acc[qq * H_I]);
#pragma unroll
        for (int h = 1; h < H_I; ++h) tot = fmaf(wt[t][qq * H_I + h], relu(acc[qq * H_I + h]), tot);
        // tiles never cross a segment edge, so the causal bound is the only mask
        const int rr = t * QPT + qq;  // row offset from the lane's first row (a constant)
        buf_store_f32(tot, s_rs, skey - rr <= pos0 ? off0 + (uint32_t)rr * row_bytes + (uint32_t)skey * 4u : kOffNone, 0);
      }
    }
  };
  // Pipeline: global rows of the next two tiles in flight in registers, the next tile's
  // operand read from LDS while the current tile computes.  Loads past the segment read
  // keys nobody stores, or zeros past Tk.
  u32x4 G0[NLD], G1[NLD];
  bf16x8 B0[KS], B1[KS];
  gload(G0);  // tile 0
  gload(G1);  // tile 1
  lstore(wk0, G0);
  gload(G0);  // tile 2
  lread(wk0, B0);
  for (int s0 = (int)seg0; s0 < kend; s0 += 64) {
    lstore(wk1, G1);  // tile j+1
    gload(G1);        // tile j+3
    tile(s0, B0);
    lread(wk1, B1);
    if (s0 + 32 >= kend) break;
    lstore(wk0, G0);  // tile j+2
    gload(G0);        // tile j+4
    tile(s0 + 32, B1);
    lread(wk0, B0);
  }
}

template <int H_I, int D_I>
hipError_t launch_t(const IndexerArgs& A, hipStream_t st) {
  constexpr int QB = 4 * query_tiles<H_I, D_I>() * (32 / H_I);
  const int qblocks = (A.nrows + QB - 1) / QB;
  // keys any row of the chunk can see (kv_len <= Tk)
  const int64_t maxkeys = std::min<int64_t>(A.Tk, (int64_t)A.Tk - A.Tq + A.row0 + A.nrows);
  if (qblocks == 0 || maxkeys <= 0) return hipSuccess;
  const int64_t tiles = (maxkeys + 31) / 32;
  // Aim at ~2048 workgroups per launch: twice what the chip holds at once, with segments
  // short enough that the causal tail of a launch stays small.
  int64_t segs = std::max<int64_t>(1, std::min<int64_t>(tiles, 2048 / std::max<int64_t>(1, (int64_t)qblocks * A.B)));
  int64_t seg_tiles = (tiles + segs - 1) / segs;
  segs = (tiles + seg_tiles - 1) / seg_tiles;
  dim3 grid(qblocks, (unsigned)segs, A.B);
  hipLaunchKernelGGL((index_scores_kernel<H_I, D_I>), grid, dim3(256), 0, st, A.q, A.k, A.w, A.kv_len, A.Tq,
                     A.Tk, A.row0, A.nrows, A.scores, A.ld, A.score_bstride, (int)(seg_tiles * 32));
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
