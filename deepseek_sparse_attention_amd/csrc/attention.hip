// Attention restricted to each query's selected keys, on gfx950.
//
//   out[h] = sum_s softmax_s(sm_scale * q[h] . K[s]) V[s],  s over the row's index list
//
// MLA form (DeepSeek-V2-Lite-Chat SIQ card, "Measured": one 576-wide latent row per token,
// 512 compressed-KV values then 64 rotary values; V = the first 512 values of the same
// row).  A workgroup serves one query row and 16 heads.  Per tile of 64 selected keys the
// gathered rows are staged once in LDS and used twice: as K (all 576 columns) for
// S = Q K^T with the 16 heads as the MFMA M dimension, and as V (columns 0..511) for
// O += P V, read transposed straight from LDS with ds_read_b64_tr_b16.  The 4 waves split
// the keys of a tile for Q K^T and the 512 value columns for P V; softmax statistics are
// exchanged through LDS (online softmax in base 2).  The next tile's gather is issued into
// registers before the current tile is computed.  fp8 (OCP e4m3) rows are widened to bf16
// exactly while staged; their per-token scale multiplies the logit and the probability.
// Decode rows (few queries) split the key list over workgroups and merge the partial
// results by log-sum-exp in a second kernel, in a fixed order.
//
// Multi-head form (DSA ablation card: 4 heads of width 32, RoPE'd inputs): one wave per
// head, logits in LDS, three fixed-order passes.
#include "common.hpp"
#include "internal.hpp"

namespace dsa {

namespace {

constexpr int kDqk = 576, kDv = 512;
constexpr int kTile = 32;                // selected keys per tile
constexpr int kPitch = kDqk * 2 + 16;    // LDS row pitch in bytes (1168: 16-B skew per row)
constexpr int kQSteps = kDqk / 32 / 2;   // MFMA k-steps of Q K^T per wave (half of 18)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Gather of one tile: wave w fetches tile keys 8w..8w+7; lane l owns key 8w + l/8 and the
// 16-byte parts l%8, l%8+8, ... of its row, so every load instruction reads eight full
// 128-byte lines.  Rows go through registers into LDS (bf16; fp8 widened exactly).
template <bool FP8>
struct TileStage;

template <>
struct TileStage<false> {  // bf16 row: 72 parts of 16 B, 9 per lane
  static constexpr int kChunks = 9;
  static constexpr uint32_t kRowBytes = kDqk * 2;
  u32x4 r[kChunks];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int s, int part0) {
#pragma unroll
    for (int c = 0; c < kChunks; ++c) r[c] = buf_load_16(rs, (uint32_t)s * kRowBytes + (part0 + 8 * c) * 16, 0);
  }
  __device__ __forceinline__ void store(uint8_t* lds_row, int part0) const {
#pragma unroll
    for (int c = 0; c < kChunks; ++c) *reinterpret_cast<u32x4*>(lds_row + (part0 + 8 * c) * 16) = r[c];
  }
};

template <>
struct TileStage<true> {  // e4m3 row: 36 parts of 16 B, up to 5 per lane
  static constexpr int kChunks = 5;
  static constexpr uint32_t kRowBytes = kDqk;
  u32x4 r[kChunks];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int s, int part0) {
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int part = part0 + 8 * c;
      if (part < 36) r[c] = buf_load_16(rs, (uint32_t)s * kRowBytes + part * 16, 0);
    }
  }
  template <bool HI>
  __device__ __forceinline__ static uint32_t widen2(uint32_t word) {
    f32x2 f = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, HI);
    // e4m3 values are exact in bf16: the low 16 bits of the fp32 pattern are zero
    return (__float_as_uint(f[0]) >> 16) | (__float_as_uint(f[1]) & 0xFFFF0000u);
  }
  __device__ __forceinline__ void store(uint8_t* lds_row, int part0) const {
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int part = part0 + 8 * c;
      if (part >= 36) continue;
      u32x4 lo, hi;
      lo[0] = widen2<false>(r[c][0]);
      lo[1] = widen2<true>(r[c][0]);
      lo[2] = widen2<false>(r[c][1]);
      lo[3] = widen2<true>(r[c][1]);
      hi[0] = widen2<false>(r[c][2]);
      hi[1] = widen2<true>(r[c][2]);
      hi[2] = widen2<false>(r[c][3]);
      hi[3] = widen2<true>(r[c][3]);
      uint8_t* dst = lds_row + part * 32;
      *reinterpret_cast<u32x4*>(dst) = lo;
      *reinterpret_cast<u32x4*>(dst + 16) = hi;
    }
  }
};

template <bool FP8>
__global__ __launch_bounds__(256, 2) void mla_attn_kernel(const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv,
                                                          const float* __restrict__ kv_scale,
                                                          const int32_t* __restrict__ idx, int Tq, int Tk, int H, int k,
                                                          float scale_log2, int tiles_per_split,
                                                          uint16_t* __restrict__ out, float* __restrict__ lse,
                                                          float* __restrict__ part_o, float* __restrict__ part_ml) {
  __shared__ __attribute__((aligned(16))) uint8_t kvs[2][kTile * kPitch];
  __shared__ __attribute__((aligned(16))) float sbuf[4][4][64];  // partial S^T per wave, accumulator layout
  __shared__ float tile_scale[2][kTile];
  __shared__ int tile_valid[2][kTile];
  __shared__ int jmax_red[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int HG = H >> 4;
  const int64_t rowh = blockIdx.x;  // (b*Tq + t)*HG + hg
  const int64_t row = rowh / HG;
  const int hg = (int)(rowh % HG);
  const int b = (int)(row / Tq);
  const int split = blockIdx.y, nsplit = gridDim.y;
  const int32_t* ix = idx + row * k;
  constexpr uint32_t kRowBytes = TileStage<FP8>::kRowBytes;
  const __amdgpu_buffer_rsrc_t kv_rs = make_rsrc(kv + (int64_t)b * Tk * kRowBytes, (uint32_t)Tk * kRowBytes);

  // extent of the index list that holds valid entries
  int jm = -1;
  for (int j = tid; j < k; j += 256) {
    const int sj = ix[j];
    if (sj >= 0 && sj < Tk) jm = j;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) jm = max(jm, __shfl_xor(jm, o, 64));
  if (lane == 0) jmax_red[wave] = jm;
  __syncthreads();
  jm = max(max(jmax_red[0], jmax_red[1]), max(jmax_red[2], jmax_red[3]));
  const int ntiles = (jm + kTile) / kTile;  // tiles covering entries 0..jm
  const int t_begin = split * tiles_per_split;
  const int t_end = min(ntiles, t_begin + tiles_per_split);

  // Lane roles.  hl = lane % 16 is this lane's head in S^T and O^T; gq = lane / 16 picks
  // which 4 keys of each 16-key half it holds (keys 4gq..4gq+3 and 16+4gq..16+4gq+3).
  // Wave roles in S^T = K Q^T: key half kh (tile keys 16kh..16kh+15), k-step half ksh.
  const int hl = lane & 15, gq = lane >> 4;
  const int kh = wave >> 1, ksh = wave & 1;
  bf16x8 qb[kQSteps];  // Q^T as the B operand: column = head hl, 8 dims per k-step
  {
    const uint16_t* qp = q + (row * H + hg * 16 + hl) * kDqk + (ksh * kQSteps) * 32 + gq * 8;
#pragma unroll
    for (int s = 0; s < kQSteps; ++s) qb[s] = as_bf16x8(ld16(qp + s * 32));
  }
  // gather: this lane's key of the tile and its first 16-byte part
  const int gk = 8 * wave + (lane >> 3), part0 = lane & 7;
  const bool key_owner = (lane & 7) == 0;
  auto entry = [&](int t) -> int {  // validated key index of this lane's entry in tile t, or -1
    const int j = t * kTile + gk;
    const int sj = j < k ? ix[j] : -1;
    return (sj >= 0 && sj < Tk) ? sj : -1;
  };

  f32x4 o_acc[8];  // O^T: rows = dims wave*128 + n*16 + 4gq + i, column = head hl
#pragma unroll
  for (int n = 0; n < 8; ++n) o_acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  TileStage<FP8> stage;
  int s_cur = -1, s_next = -1;
  float sc_cur = 1.f;
  if (t_begin < t_end) {
    s_cur = entry(t_begin);
    stage.load(kv_rs, max(s_cur, 0), part0);
    if (FP8 && key_owner && s_cur >= 0) sc_cur = kv_scale[(int64_t)b * Tk + s_cur];
    if (t_begin + 1 < t_end) s_next = entry(t_begin + 1);
  }
  for (int t = t_begin; t < t_end; ++t) {
    const int buf = (t - t_begin) & 1;
    uint8_t* kvb = kvs[buf];
    stage.store(kvb + gk * kPitch, part0);
    if (key_owner) {
      tile_valid[buf][gk] = s_cur >= 0;
      tile_scale[buf][gk] = sc_cur;
    }
    __syncthreads();  // tile t staged (the other buffer may still be read by PV of t-1)
    if (t + 1 < t_end) {
      s_cur = s_next;
      stage.load(kv_rs, max(s_cur, 0), part0);
      sc_cur = 1.f;
      if (FP8 && key_owner && s_cur >= 0) sc_cur = kv_scale[(int64_t)b * Tk + s_cur];
      s_next = (t + 2 < t_end) ? entry(t + 2) : -1;
    }

    // ---- partial S^T = K Q^T over this wave's k-steps, keys 16kh .. 16kh+15
    {
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
      const uint8_t* krow = kvb + (16 * kh + hl) * kPitch + (ksh * kQSteps) * 64 + gq * 16;
#pragma unroll
      for (int s = 0; s < kQSteps; ++s) {
        const bf16x8 ka = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(krow + s * 64));
        sacc = mfma16(ka, qb[s], sacc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sbuf[wave][i][lane] = sacc[i];
    }
    __syncthreads();  // partial sums visible

    // ---- logits of the lane's 8 keys for head hl, online softmax in base 2
    float sv[8], ksc[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 16 * h + 4 * gq + i;
        ksc[4 * h + i] = tile_scale[buf][key];
        const float sfull = sbuf[2 * h][i][lane] + sbuf[2 * h + 1][i][lane];
        sv[4 * h + i] = tile_valid[buf][key] ? sfull * (ksc[4 * h + i] * scale_log2) : -INFINITY;
      }
    }
    float tm = sv[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) tm = fmaxf(tm, sv[e]);
    tm = fmaxf(tm, __shfl_xor(tm, 16, 64));
    tm = fmaxf(tm, __shfl_xor(tm, 32, 64));
    const float mn = fmaxf(m_run, tm);
    const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2(m_run - mn);
    float pv[8], ts = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pv[e] = (sv[e] == -INFINITY) ? 0.f : fast_exp2(sv[e] - mn);
      ts += pv[e];
    }
    ts += __shfl_xor(ts, 16, 64);
    ts += __shfl_xor(ts, 32, 64);
    l_run = l_run * alpha + ts;
    m_run = mn;
    // P^T as the B operand: k-slot e of group gq <-> key 4gq+e (e<4), 16+4gq+(e-4) (e>=4);
    // probabilities carry the fp8 row scale for V
    u32x4 pw;
#pragma unroll
    for (int e = 0; e < 4; ++e) pw[e] = pack_bf16x2(pv[2 * e] * ksc[2 * e], pv[2 * e + 1] * ksc[2 * e + 1]);
    const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) o_acc[n][i] *= alpha;

    // ---- O^T[dims wave*128 .. +128] += V^T P^T  (V read transposed from the staged rows)
    {
      const int kb0 = 4 * gq + (hl >> 2);
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const int col = wave * 128 + n * 16 + 4 * (hl & 3);
        const i16x4 v0 = lds_read_tr16(kvb + kb0 * kPitch + col * 2);
        const i16x4 v1 = lds_read_tr16(kvb + (kb0 + 16) * kPitch + col * 2);
        typedef short i16x8 __attribute__((ext_vector_type(8)));
        const i16x8 vv = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        o_acc[n] = mfma16(__builtin_bit_cast(bf16x8, vv), pb, o_acc[n]);
      }
    }
  }

  // ---- results: lane holds O[head hl][wave*128 + n*16 + 4gq + i]
  const int h = hg * 16 + hl;
  if (nsplit == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    uint16_t* op = out + (row * H + h) * kDv + wave * 128 + 4 * gq;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const uint32_t lo = pack_bf16x2(o_acc[n][0] * inv, o_acc[n][1] * inv);
      const uint32_t hi = pack_bf16x2(o_acc[n][2] * inv, o_acc[n][3] * inv);
      *reinterpret_cast<uint2*>(op + n * 16) = make_uint2(lo, hi);
    }
    if (lse && wave == 0 && gq == 0) lse[row * H + h] = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
  } else {
    const int64_t nrowh = (int64_t)gridDim.x * 16;  // (row, head) pairs over all rows
    const int64_t rh = rowh * 16 + hl;
    float* po = part_o + ((int64_t)split * nrowh + rh) * kDv + wave * 128 + 4 * gq;
#pragma unroll
    for (int n = 0; n < 8; ++n)
      *reinterpret_cast<float4*>(po + n * 16) = make_float4(o_acc[n][0], o_acc[n][1], o_acc[n][2], o_acc[n][3]);
    if (wave == 0 && gq == 0) {
      part_ml[((int64_t)split * nrowh + rh) * 2 + 0] = m_run;
      part_ml[((int64_t)split * nrowh + rh) * 2 + 1] = l_run;
    }
  }
}

// Merge split-key partial results (fixed split order).  One workgroup per (row, head).
__global__ __launch_bounds__(256) void mla_combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                                                          int nsplit, int64_t nrowh, int H, uint16_t* __restrict__ out,
                                                          float* __restrict__ lse) {
  const int64_t rh = blockIdx.x;
  float m = -INFINITY;
  for (int s = 0; s < nsplit; ++s) m = fmaxf(m, part_ml[((int64_t)s * nrowh + rh) * 2]);
  float l = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float ms = part_ml[((int64_t)s * nrowh + rh) * 2];
    if (ms != -INFINITY) l += part_ml[((int64_t)s * nrowh + rh) * 2 + 1] * fast_exp2(ms - m);
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  for (int d = threadIdx.x; d < kDv; d += blockDim.x) {
    float o = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const float ms = part_ml[((int64_t)s * nrowh + rh) * 2];
      if (ms != -INFINITY) o += part_o[((int64_t)s * nrowh + rh) * kDv + d] * fast_exp2(ms - m);
    }
    out[rh * kDv + d] = f32_to_bf16_bits(o * inv);
  }
  if (lse && threadIdx.x == 0) lse[rh] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
}

// Multi-head form: Dqk = Dv = 32, Hkv = H, one wave per head (heads strided over 4 waves),
// logits of up to kMhaMaxK selected keys kept in LDS.
constexpr int kMhaD = 32;
constexpr int kMhaMaxK = 4096;

__global__ __launch_bounds__(256) void mha_attn_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kk,
                                                       const uint16_t* __restrict__ vv, const int32_t* __restrict__ idx,
                                                       int Tq, int Tk, int H, int k, float scale_log2,
                                                       uint16_t* __restrict__ out, float* __restrict__ lse) {
  __shared__ float zb[4][kMhaMaxK];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int64_t row = blockIdx.x;
  const int b = (int)(row / Tq);
  const int32_t* ix = idx + row * k;
  float* z = zb[wave];
  // every wave runs the same number of rounds, so the barriers below are uniform
  for (int h0 = 0; h0 < H; h0 += 4) {
    const int h = h0 + wave;
    const bool active = h < H;
    float m = -INFINITY, l = 0.f;
    if (active) {
      float qf[kMhaD];
      const uint16_t* qp = q + (row * H + h) * kMhaD;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 w4 = ld16(qp + c * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qf[c * 8 + 2 * e] = __uint_as_float(w4[e] << 16);
          qf[c * 8 + 2 * e + 1] = __uint_as_float(w4[e] & 0xFFFF0000u);
        }
      }
      for (int j = lane; j < k; j += 64) {
        const int s = ix[j];
        float zz = -INFINITY;
        if (s >= 0 && s < Tk) {
          const uint16_t* kp = kk + (((int64_t)b * Tk + s) * H + h) * kMhaD;
          float dot = 0.f;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const u32x4 w4 = ld16(kp + c * 8);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              dot = fmaf(qf[c * 8 + 2 * e], __uint_as_float(w4[e] << 16), dot);
              dot = fmaf(qf[c * 8 + 2 * e + 1], __uint_as_float(w4[e] & 0xFFFF0000u), dot);
            }
          }
          zz = dot * scale_log2;
        }
        z[j] = zz;
        m = fmaxf(m, zz);
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      for (int j = lane; j < k; j += 64) {
        const float p = (z[j] == -INFINITY) ? 0.f : fast_exp2(z[j] - m);
        z[j] = p;
        l += p;
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o, 64);
    }
    __syncthreads();  // probabilities written by other lanes are read below
    if (active) {
      // P V: lane -> (column d = lane % 32, half = lane / 32), keys of that parity
      const int d = lane & 31, half = lane >> 5;
      float o = 0.f;
      for (int j = half; j < k; j += 2) {
        const float p = z[j];
        if (p != 0.f) {
          const int s = ix[j];
          o = fmaf(p, bf16_bits_to_f32(vv[(((int64_t)b * Tk + s) * H + h) * kMhaD + d]), o);
        }
      }
      o += __shfl_xor(o, 32, 64);
      if (half == 0) out[(row * H + h) * kMhaD + d] = f32_to_bf16_bits(l > 0.f ? o / l : 0.f);
      if (lse && lane == 0) lse[row * H + h] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
    }
    __syncthreads();  // z is reused by the next round
  }
}

}  // namespace

bool attn_mla_supported(const AttnArgs& a) {
  // the gather addresses a sequence's rows with 32-bit byte offsets
  const int64_t seq_bytes = (int64_t)a.Tk * (a.fp8 ? kDqk : kDqk * 2);
  return a.Hkv == 1 && a.Dqk == kDqk && a.Dv == kDv && a.v == nullptr && a.H % 16 == 0 && a.H > 0 && a.k >= 1 &&
         a.k <= 65536 && seq_bytes < (int64_t(1) << 32);
}

bool attn_mha_supported(const AttnArgs& a) {
  return !a.fp8 && a.Hkv == a.H && a.H >= 1 && a.H <= 16 && a.Dqk == kMhaD && a.Dv == kMhaD && a.v != nullptr &&
         a.k >= 1 && a.k <= kMhaMaxK;
}

int attn_mla_splits(int B, int Tq, int H, int k) {
  // few rows (decode): split each row's key list so ~512 workgroups (2 per CU) run
  const int64_t wgs = (int64_t)B * Tq * (H / 16);
  const int tiles = (k + kTile - 1) / kTile;
  if (wgs >= 256) return 1;
  int s = (int)std::min<int64_t>(tiles, (512 + wgs - 1) / std::max<int64_t>(1, wgs));
  if (s <= 1) return 1;
  const int per = (tiles + s - 1) / s;
  return (tiles + per - 1) / per;
}

size_t attn_workspace_bytes(int B, int Tq, int H, int Dv, int k, bool mla) {
  if (!mla) return 0;
  const int s = attn_mla_splits(B, Tq, H, k);
  if (s <= 1) return 0;
  const size_t nrowh = (size_t)B * Tq * H;
  return (size_t)s * nrowh * ((size_t)Dv + 2) * sizeof(float);
}

hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t st) {
  const int64_t rows = (int64_t)a.B * a.Tq;
  if (rows == 0) return hipSuccess;
  if (attn_mla_supported(a)) {
    const float sl2 = a.sm_scale * kLog2e;
    const int tiles = (a.k + kTile - 1) / kTile;
    const int nsplit = attn_mla_splits(a.B, a.Tq, a.H, a.k);
    const int per = (tiles + nsplit - 1) / nsplit;
    const int64_t nrowh = rows * a.H;
    float* part_o = nullptr;
    float* part_ml = nullptr;
    if (nsplit > 1) {
      part_o = reinterpret_cast<float*>(a.ws);
      part_ml = part_o + (size_t)nsplit * nrowh * kDv;
    }
    dim3 grid((unsigned)(rows * (a.H / 16)), nsplit);
    if (a.fp8)
      hipLaunchKernelGGL(mla_attn_kernel<true>, grid, dim3(256), 0, st, a.q, (const uint8_t*)a.kv, a.kv_scale, a.idx,
                         a.Tq, a.Tk, a.H, a.k, sl2, per, a.out, a.lse, part_o, part_ml);
    else
      hipLaunchKernelGGL(mla_attn_kernel<false>, grid, dim3(256), 0, st, a.q, (const uint8_t*)a.kv, nullptr, a.idx,
                         a.Tq, a.Tk, a.H, a.k, sl2, per, a.out, a.lse, part_o, part_ml);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || nsplit == 1) return e;
    hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)nrowh), dim3(256), 0, st, part_o, part_ml, nsplit, nrowh,
                       a.H, a.out, a.lse);
    return hipGetLastError();
  }
  if (attn_mha_supported(a)) {
    hipLaunchKernelGGL(mha_attn_kernel, dim3((unsigned)rows), dim3(256), 0, st, a.q, (const uint16_t*)a.kv, a.v,
                       a.idx, a.Tq, a.Tk, a.H, a.k, a.sm_scale * kLog2e, a.out, a.lse);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace dsa
