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
// MXFP4 rows (OCP microscaling: 32-value blocks of e2m1 elements sharing an E8M0 scale;
// the same card's "Measured" section names an nvfp4 latent cache for sparse MLA) are
// decoded with their block scales while staged, also exactly: e2m1 times a power of two
// has two significant bits.
// Decode rows (few queries) split the key list over workgroups and merge the partial
// results by log-sum-exp in a second kernel, in a fixed order.
//
// Multi-head form (DSA ablation card: 4 heads of width 32, RoPE'd inputs): a workgroup per
// query row, key rows read as 16-byte chunks spread over the lanes, logits in LDS, three
// fixed-order passes.
#include "common.hpp"
#include "internal.hpp"

namespace dsa {

namespace {

constexpr int kDqk = 576, kDv = 512;
constexpr int kTile = 32;                // selected keys per tile
constexpr int kRowB = kDqk * 2;          // staged bf16 row: 1152 B = 72 chunks of 16 B
constexpr int kQSteps = kDqk / 32 / 2;   // MFMA k-steps of Q K^T per wave (half of 18)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// LDS rows are XOR-swizzled in 16-byte chunks: chunk c of row r sits at c ^ (r mod 8), so
// chunks stay inside their aligned group of 8 (72 = 9 x 8).  Measured on gfx950 with the
// LDS bank-conflict counter, this leaves all three access patterns of a tile (the row
// stores, the K reads of Q K^T and the transposed V reads) free of conflicts; a
// swizzle that spreads rows over only half of the chunk slots per 8-lane group cost 4
// extra cycles per K read and 2 per V read.
__device__ __forceinline__ int swz(int r) { return r & 7; }
__device__ __forceinline__ int lds_off(int r, int chunk) { return r * kRowB + ((chunk ^ swz(r)) << 4); }

// Gather of one tile: wave w fetches tile keys 8w..8w+7; lane l owns key 8w + l/8 and the
// 16-byte parts l%8, l%8+8, ... of its row, so every load instruction reads eight full
// 128-byte lines.  Rows go through registers into LDS (bf16; fp8 and fp4 widened exactly).
// Row offsets use a 24-bit multiply (rows < 2^24 here): a 64-bit multiply-add would read an
// undefined high addend register and could force a wait on an unrelated load.  A missing
// row (s < 0) is read at offsets from kRowNone, past every buffer range these kernels
// accept: zeros, no memory access.  Every part is loaded unconditionally, so all paths
// issue the same loads and the compiler's load-count waits stay exact.
enum : int { kKvBf16 = 0, kKvFp8 = 1, kKvMxfp4 = 2 };
constexpr uint32_t kRowNone = 0xFFFFF000u;  // + any part offset of a row stays below 2^32

template <int FMT>
struct TileStage;

template <>
struct TileStage<kKvBf16> {  // bf16 row: 72 parts of 16 B, 9 per lane
  static constexpr int kChunks = 9;
  static constexpr uint32_t kRowBytes = kDqk * 2;
  u32x4 r[kChunks];
  int s = -1;      // key index of this lane's entry (-1: none)
  float sc = 1.f;  // its scale (fp8 only)
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int part0) {
    const uint32_t base = (s >= 0 ? __umul24((uint32_t)s, kRowBytes) : kRowNone) + part0 * 16;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) r[c] = buf_load_16(rs, base + 128 * c, 0);
  }
  __device__ __forceinline__ void store(uint8_t* lds, int key, int part0) const {
#pragma unroll
    for (int c = 0; c < kChunks; ++c) *reinterpret_cast<u32x4*>(lds + lds_off(key, part0 + 8 * c)) = r[c];
  }
};

template <>
struct TileStage<kKvFp8> {  // e4m3 row: 36 parts of 16 B, up to 5 per lane
  static constexpr int kChunks = 5;
  static constexpr uint32_t kRowBytes = kDqk;
  u32x4 r[kChunks];
  int s = -1;
  float sc = 1.f;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int part0) {
    const uint32_t base = (s >= 0 ? __umul24((uint32_t)s, kRowBytes) : kRowNone) + part0 * 16;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      // part part0 + 8c; the fifth exists for part0 < 4 only (36 parts)
      const uint32_t off = (c < 4 || part0 < 4) ? base + 128 * c : kRowNone;
      r[c] = buf_load_16(rs, off, 0);
    }
  }
  template <bool HI>
  __device__ __forceinline__ static uint32_t widen2(uint32_t word) {
    f32x2 f = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, HI);
    // e4m3 values are exact in bf16: the low 16 bits of the fp32 pattern are zero
    return (__float_as_uint(f[0]) >> 16) | (__float_as_uint(f[1]) & 0xFFFF0000u);
  }
  __device__ __forceinline__ void store(uint8_t* lds, int key, int part0) const {
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
      *reinterpret_cast<u32x4*>(lds + lds_off(key, 2 * part)) = lo;  // bf16 chunks 2p, 2p+1
      *reinterpret_cast<u32x4*>(lds + lds_off(key, 2 * part + 1)) = hi;
    }
  }
};

// MXFP4 row, 320 B: block j's 32 e2m1 elements in bytes 16j..16j+15 (element 2i in the low
// nibble of byte i), j < 18; then 8 scale words, word p holding the E8M0 scales of blocks
// p, p+8 and p+16 in its bytes 0, 1 and 2.  Lane part0 = p loads blocks p, p+8 (p+16 for
// p < 2) and word p: every 16-byte part is one block, and its scale arrives with it.
template <>
struct TileStage<kKvMxfp4> {
  static constexpr int kChunks = 3;
  static constexpr int kBlocks = kDqk / 32;
  static constexpr uint32_t kRowBytes = kDqk / 2 + 32;
  u32x4 r[kChunks];
  uint32_t e = 0;  // scales of this lane's blocks
  int s = -1;
  float sc = 1.f;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int part0) {
    const uint32_t row = s >= 0 ? __umul24((uint32_t)s, kRowBytes) : kRowNone;
    const uint32_t base = row + part0 * 16;
    r[0] = buf_load_16(rs, base, 0);
    r[1] = buf_load_16(rs, base + 128, 0);
    r[2] = buf_load_16(rs, part0 < kBlocks - 16 ? base + 256 : kRowNone, 0);
    e = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(row + kDqk / 2 + 4 * part0), 0, 0);
  }
  // elements 2B and 2B+1 of an 8-element word, times the scale, as a bf16 pair (low first)
  template <int B>
  __device__ __forceinline__ static uint32_t pair(uint32_t word, float scale) {
    const f32x2 f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, scale, B);
    return (__float_as_uint(f[0]) >> 16) | (__float_as_uint(f[1]) & 0xFFFF0000u);
  }
  __device__ __forceinline__ void store(uint8_t* lds, int key, int part0) const {
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int blk = part0 + 8 * c;
      if (blk >= kBlocks) continue;
      // the E8M0 byte as the exponent field of an fp32: the conversion reads only that
      // field, as an E8M0 scale (measured on gfx950: byte 0 scales by 2^-127, byte 255
      // gives NaN, as the format defines)
      const float scale = __uint_as_float(((e >> (8 * c)) & 0xFFu) << 23);
#pragma unroll
      for (int w = 0; w < 4; ++w) {  // values 32 blk + 8w .. +7 -> staged chunk 4 blk + w
        u32x4 o;
        o[0] = pair<0>(r[c][w], scale);
        o[1] = pair<1>(r[c][w], scale);
        o[2] = pair<2>(r[c][w], scale);
        o[3] = pair<3>(r[c][w], scale);
        *reinterpret_cast<u32x4*>(lds + lds_off(key, 4 * blk + w)) = o;
      }
    }
  }
};

// Two schedules.  WIDE = 0: two row stages in registers, two LDS tile buffers, two
// workgroups per CU.  WIDE = 1 (bf16 rows, no key split, at most kWideMaxTk keys): one
// register stage and one LDS buffer, three workgroups per CU.  The tile body is a latency
// chain and a third workgroup hides more of it; measured 4.7% faster at T=16384 and 1.5%
// slower at T=32768 (the extra workgroups' rows then cost more in cache than they gain).
constexpr int kWideMaxTk = 24576;

// Per-layer operands of one launch: blockIdx.z picks the layer.  Layers that share one
// index list (an 'F' layer and the 'S' layers after it) run in one launch, so a decode
// step's short, latency-bound attention layers overlap instead of running back to back.
struct MlaLayers {
  const uint16_t* q[kMaxAttnLayers];
  const uint8_t* kv[kMaxAttnLayers];
  const float* kv_scale[kMaxAttnLayers];
  uint16_t* out[kMaxAttnLayers];
  float* lse[kMaxAttnLayers];
};

template <int FMT, int WIDE>
__global__ __launch_bounds__(256, WIDE ? 3 : 2) void mla_attn_kernel(const MlaLayers Ls,
                                                          const int32_t* __restrict__ idx, int Tq, int Tk,
                                                          int64_t kv_bstride, int H, int k, float scale_log2,
                                                          int tiles_per_split, float* __restrict__ part_o,
                                                          float* __restrict__ part_ml, int64_t part_layer) {
  // layer z's operands; its split partials sit part_layer floats after layer z-1's
  const int z = blockIdx.z;
  const uint16_t* __restrict__ q = Ls.q[z];
  const uint8_t* __restrict__ kv = Ls.kv[z];
  const float* __restrict__ kv_scale = Ls.kv_scale[z];
  uint16_t* __restrict__ out = Ls.out[z];
  float* __restrict__ lse = Ls.lse[z];
  part_o += z * part_layer;
  part_ml += z * part_layer;
  constexpr int NBUF = WIDE ? 1 : 2;  // LDS tile buffers
  constexpr int NST = WIDE ? 1 : 2;   // row stages in registers (tiles in flight)
  __shared__ __attribute__((aligned(16))) uint8_t kvs[NBUF][kTile * kRowB];
  __shared__ __attribute__((aligned(16))) f32x4 sbuf[4][64];           // partial S^T per wave and lane
  __shared__ __attribute__((aligned(16))) float tile_bias[NBUF][kTile];   // 0 for a valid key, -inf otherwise
  __shared__ __attribute__((aligned(16))) float tile_scale[NBUF][kTile];  // fp8 row scales
  __shared__ int jmax_red[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int HG = H >> 4;
  const int64_t rowh = blockIdx.x;  // (b*Tq + t)*HG + hg
  const int64_t row = rowh / HG;
  const int hg = (int)(rowh % HG);
  const int b = (int)(row / Tq);
  const int split = blockIdx.y, nsplit = gridDim.y;
  const int32_t* ix = idx + row * k;
  constexpr bool FP8 = FMT == kKvFp8;  // per-token scale on logits and probabilities
  constexpr uint32_t kRowBytes = TileStage<FMT>::kRowBytes;
  // sequence b's rows start kv_bstride rows after sequence b-1's (0: one shared pool)
  const __amdgpu_buffer_rsrc_t kv_rs = make_rsrc(kv + b * kv_bstride * kRowBytes, (uint32_t)Tk * kRowBytes);

  // This split's tiles.  Index entries are validated against its nominal range; the scan
  // below only trims trailing tiles that hold no valid entry, so it can run while the first
  // loads are in flight (it used to sit in front of them as one more memory round trip).
  const int t_begin = split * tiles_per_split;
  const int t_lim = min((k + kTile - 1) / kTile, t_begin + tiles_per_split);

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
  // Index entries are fetched two tiles ahead of the rows they name, as unconditional
  // buffer loads (past the list or past this split: the range check returns 0), and
  // validated only when the row gather is issued: waiting on a load retires every older
  // load too, so an index consumed right after its load would drain the row prefetch.
  const __amdgpu_buffer_rsrc_t ix_rs = make_rsrc(ix, (uint32_t)k * 4);
  const __amdgpu_buffer_rsrc_t sc_rs = make_rsrc(FP8 ? kv_scale + b * kv_bstride : nullptr, FP8 ? (uint32_t)Tk * 4 : 0u);
  auto raw_entry = [&](int t) -> int {
    const int j = t * kTile + gk;
    return (int)__builtin_amdgcn_raw_buffer_load_b32(ix_rs, t < t_lim ? j * 4 : (int)kOffNone, 0, 0);
  };
  auto valid_entry = [&](int t, int raw) -> int {  // key index of this lane's entry in tile t, or -1
    const int lim = (t < t_lim && t * kTile + gk < k) ? Tk : 0;  // the raw value is always read
    return (uint32_t)raw < (uint32_t)lim ? raw : -1;
  };
  auto fetch = [&](TileStage<FMT>& st, int s_idx) {  // issue the gather of one tile
    st.s = s_idx;
    st.load(kv_rs, part0);
    if (FP8) st.sc = buf_load_f32(sc_rs, s_idx >= 0 ? (uint32_t)s_idx * 4 : kOffNone, 0);
  };

  // prologue: index entries of tiles t_begin .. t_begin + 2*NST - 1, rows of the first NST
  // in flight
  TileStage<FMT> st0, st1;
  int nx0, nx1 = 0;
  {
    const int e0 = raw_entry(t_begin);
    if constexpr (NST == 2) {
      const int e1 = raw_entry(t_begin + 1);
      nx0 = raw_entry(t_begin + 2);
      nx1 = raw_entry(t_begin + 3);
      fetch(st0, valid_entry(t_begin, e0));
      fetch(st1, valid_entry(t_begin + 1, e1));
    } else {
      nx0 = raw_entry(t_begin + 1);
      fetch(st0, valid_entry(t_begin, e0));
    }
  }

  // extent of this split's entries that are valid: the loop ends after its last tile
  int jm = -1;
  for (int j = t_begin * kTile + tid; j < min(k, t_lim * kTile); j += 256) {
    const int sj = ix[j];
    if (sj >= 0 && sj < Tk) jm = j;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) jm = max(jm, __shfl_xor(jm, o, 64));
  if (lane == 0) jmax_red[wave] = jm;
  __syncthreads();
  jm = max(max(jmax_red[0], jmax_red[1]), max(jmax_red[2], jmax_red[3]));
  const int t_end = min((jm + kTile) / kTile, t_lim);  // tiles covering entries 0..jm

  f32x4 o_acc[8];  // O^T: rows = dims wave*128 + n*16 + 4gq + i, column = head hl
#pragma unroll
  for (int n = 0; n < 8; ++n) o_acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  auto tile = [&](int t, TileStage<FMT>& st, int& nx) {  // nx: raw index entry of tile t+NST
    const int buf = NBUF == 2 ? (t - t_begin) & 1 : 0;
    uint8_t* kvb = kvs[buf];
    if constexpr (NBUF == 1) __syncthreads();  // every wave is done with the previous tile
    st.store(kvb, gk, part0);
    if (key_owner) {
      tile_bias[buf][gk] = st.s >= 0 ? 0.f : -INFINITY;
      if (FP8) tile_scale[buf][gk] = st.sc;
    }
    __syncthreads();  // tile t staged (the other buffer may still be read by PV of t-1)
    // refill this stage with tile t+NST; its index entry arrived with tile t's rows
    {
      const int s2 = valid_entry(t + NST, nx);
      nx = raw_entry(t + 2 * NST);
      fetch(st, s2);
    }

    // ---- partial S^T = K Q^T over this wave's k-steps, keys 16kh .. 16kh+15
    {
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
      const int krow = 16 * kh + hl;
#pragma unroll
      for (int s = 0; s < kQSteps; ++s) {
        const int chunk = (ksh * kQSteps + s) * 4 + gq;
        const bf16x8 ka = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kvb + lds_off(krow, chunk)));
        sacc = mfma16(ka, qb[s], sacc);
      }
      sbuf[wave][lane] = sacc;
    }
    __syncthreads();  // partial sums visible

    // ---- logits of the lane's 8 keys for head hl, online softmax in base 2
    // (the lane's keys 16h+4gq .. +3 are contiguous: one 16-byte LDS read per half)
    float sv[8], ksc[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 pa = sbuf[2 * h][lane], pb2 = sbuf[2 * h + 1][lane];
      const f32x4 bias = *reinterpret_cast<const f32x4*>(&tile_bias[buf][16 * h + 4 * gq]);
      f32x4 kscv = {1.f, 1.f, 1.f, 1.f};
      if (FP8) kscv = *reinterpret_cast<const f32x4*>(&tile_scale[buf][16 * h + 4 * gq]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ksc[4 * h + i] = kscv[i];
        const float sfull = pa[i] + pb2[i];
        sv[4 * h + i] = __builtin_fmaf(sfull, FP8 ? kscv[i] * scale_log2 : scale_log2, bias[i]);  // -inf if masked
      }
    }
    float tm = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    tm = rows_max(tm);
    const float mn = fmaxf(m_run, tm);
    // exp2(-inf) = 0 covers masked keys and a first valid tile; only a head with no valid
    // key yet (mn = -inf) needs a finite reference to avoid -inf - -inf
    const float mref = (mn == -INFINITY) ? 0.f : mn;
    const float alpha = fast_exp2(m_run - mref);
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(sv[e] - mref);
    const float ts = rows_sum(((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7])));
    l_run = l_run * alpha + ts;
    m_run = mn;
    // P^T as the B operand: k-slot e of group gq <-> key 4gq+e (e<4), 16+4gq+(e-4) (e>=4);
    // probabilities carry the fp8 row scale for V
    u32x4 pw;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      pw[e] = FP8 ? cvt_bf16x2(pv[2 * e] * ksc[2 * e], pv[2 * e + 1] * ksc[2 * e + 1]) : cvt_bf16x2(pv[2 * e], pv[2 * e + 1]);
    const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
    if (__ballot(alpha != 1.f)) {  // rescale only when some head's running max moved
#pragma unroll
      for (int n = 0; n < 8; ++n) o_acc[n] *= alpha;
    }

    // ---- O^T[dims wave*128 .. +128] += V^T P^T  (V read transposed from the staged rows)
    {
      const int r0 = 4 * gq + (hl >> 2);
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const int dim = wave * 128 + n * 16 + 4 * (hl & 3);  // 4 dims = 8 bytes
        const int chunk = dim >> 3, half = (dim & 7) * 2;
        const i16x4 v0 = lds_read_tr16(kvb + lds_off(r0, chunk) + half);
        const i16x4 v1 = lds_read_tr16(kvb + lds_off(r0 + 16, chunk) + half);
        typedef short i16x8 __attribute__((ext_vector_type(8)));
        const i16x8 vv = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        o_acc[n] = mfma16(__builtin_bit_cast(bf16x8, vv), pb, o_acc[n]);
      }
    }
  };

  if constexpr (NST == 1) {
    for (int t = t_begin; t < t_end; ++t) tile(t, st0, nx0);
  } else {
    int t = t_begin;
    for (; t + 1 < t_end; t += 2) {
      tile(t, st0, nx0);
      tile(t + 1, st1, nx1);
    }
    if (t < t_end) tile(t, st0, nx0);
  }

  // ---- results: lane holds O[head hl][wave*128 + n*16 + 4gq + i]
  const int h = hg * 16 + hl;
  if (nsplit == 1) {
    const float inv = l_run == 0.f ? 0.f : 1.f / l_run;  // (a NaN sum stays NaN)
    uint16_t* op = out + (row * H + h) * kDv + wave * 128 + 4 * gq;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const uint32_t lo = cvt_bf16x2(o_acc[n][0] * inv, o_acc[n][1] * inv);
      const uint32_t hi = cvt_bf16x2(o_acc[n][2] * inv, o_acc[n][3] * inv);
      *reinterpret_cast<uint2*>(op + n * 16) = make_uint2(lo, hi);
    }
    if (lse && wave == 0 && gq == 0) lse[row * H + h] = l_run == 0.f ? -INFINITY : (m_run + __log2f(l_run)) * kLn2;
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

// Merge split-key partial results (fixed split order).  One workgroup per (row, 4 heads),
// one wave per head: lane s holds split s's (m, l) (up to 64 splits), the wave reduces
// them, and each lane then sums 8 output dims over the splits with 16-byte loads.
__global__ __launch_bounds__(256) void mla_combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                                                          int64_t part_layer, int nsplit, int64_t nrowh, int H,
                                                          const MlaLayers Ls) {
  const int z = blockIdx.y;  // layer
  part_o += z * part_layer;
  part_ml += z * part_layer;
  uint16_t* __restrict__ out = Ls.out[z];
  float* __restrict__ lse = Ls.lse[z];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int64_t rh = (int64_t)blockIdx.x * 4 + wave;  // (row, head)
  if (rh >= nrowh) return;
  float ms = -INFINITY, ls = 0.f;
  if (lane < nsplit) {
    ms = part_ml[((int64_t)lane * nrowh + rh) * 2];
    ls = part_ml[((int64_t)lane * nrowh + rh) * 2 + 1];
  }
  float m = ms;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  const float wgt = (ms == -INFINITY) ? 0.f : fast_exp2(ms - m);  // this lane's split weight
  float l = ls * wgt;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o, 64);  // butterfly: same order in every lane
  const float inv = l == 0.f ? 0.f : 1.f / l;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const float* po = part_o + rh * kDv + lane * 8;
  for (int sp = 0; sp < nsplit; ++sp) {
    const float w = __shfl(wgt, sp, 64);
    const float4 a0 = *reinterpret_cast<const float4*>(po + (int64_t)sp * nrowh * kDv);
    const float4 a1 = *reinterpret_cast<const float4*>(po + (int64_t)sp * nrowh * kDv + 4);
    acc[0] += a0.x * w; acc[1] += a0.y * w; acc[2] += a0.z * w; acc[3] += a0.w * w;
    acc[4] += a1.x * w; acc[5] += a1.y * w; acc[6] += a1.z * w; acc[7] += a1.w * w;
  }
  uint32_t pk[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) pk[e] = cvt_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
  *reinterpret_cast<uint4*>(out + rh * kDv + lane * 8) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  if (lse && lane == 0) lse[rh] = l == 0.f ? -INFINITY : (m + __log2f(l)) * kLn2;
}

// Multi-head form (Dqk = Dv = 32, Hkv = H <= 16): one workgroup per query row, heads taken
// in groups of G (a power of two: all H, padded, when G x k logits fit the LDS area).  A
// key's rows of a group, K[s][h0 .. h0+G-1][32] and likewise V, are G*64 contiguous bytes:
// C = 4G lanes read them as 16-byte chunks (chunk c: head c/4, dims 8(c%4) .. +7), so a
// wave reads 64/C keys per step with every load 16 contiguous bytes.  Pass 1 forms the
// logits (partial dot per lane, two shuffles over a head's four chunk lanes) into LDS;
// pass 2 turns each head's logits into probabilities (a wave per head: max, exp2, sum);
// pass 3 accumulates P V per lane for its (head, 8 dims) over its keys, then lanes with the
// same chunk and the four waves are summed in a fixed order.
constexpr int kMhaD = 32;
constexpr int kMhaMaxK = 4096;

template <int G, int ZCAP>  // heads per round, logits per round held in LDS
__global__ __launch_bounds__(256) void mha_attn_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kk,
                                                       const uint16_t* __restrict__ vv, const int32_t* __restrict__ idx,
                                                       int Tq, int Tk, int H, int k, float scale_log2,
                                                       uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int C = 4 * G;      // lanes per key (one 16-byte chunk each)
  constexpr int KW = 64 / C;    // keys per wave step
  constexpr int KB = 4 * KW;    // keys per workgroup step
  __shared__ float zs[ZCAP];                    // [G][k] logits, then probabilities
  __shared__ float qs[G][kMhaD];                // the group's queries, times sm_scale * log2(e)
  __shared__ float stat[G][2];                  // per head: max, sum
  __shared__ __attribute__((aligned(16))) float ored[4][G * kMhaD];  // P V per wave
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int64_t row = blockIdx.x;
  const int b = (int)(row / Tq);
  const int32_t* ix = idx + row * k;
  const int kl = lane / C, c = lane % C;
  const int hh = c >> 2, dc = c & 3;  // this lane's head within the group, dim chunk
  for (int h0 = 0; h0 < H; h0 += G) {  // uniform rounds
    for (int x = tid; x < G * kMhaD; x += 256) {
      const int h = h0 + x / kMhaD;
      qs[x / kMhaD][x % kMhaD] = h < H ? bf16_bits_to_f32(q[(row * H + h) * kMhaD + x % kMhaD]) * scale_log2 : 0.f;
    }
    __syncthreads();
    const bool hv = h0 + hh < H;
    // ---- pass 1: base-2 logits
#pragma unroll 4
    for (int j = wave * KW + kl; j < k; j += KB) {
      const int s = ix[j];
      const bool ok = hv && s >= 0 && s < Tk;
      float part = 0.f;
      if (ok) {
        const u32x4 w4 = ld16(kk + (((int64_t)b * Tk + s) * H + h0 + hh) * kMhaD + dc * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          part = fmaf(qs[hh][dc * 8 + 2 * e], __uint_as_float(w4[e] << 16), part);
          part = fmaf(qs[hh][dc * 8 + 2 * e + 1], __uint_as_float(w4[e] & 0xFFFF0000u), part);
        }
      }
      part += __shfl_xor(part, 1, 64);
      part += __shfl_xor(part, 2, 64);
      if (dc == 0) zs[hh * k + j] = ok ? part : -INFINITY;
    }
    __syncthreads();
    // ---- pass 2: probabilities, a wave per head
    for (int g = wave; g < G; g += 4) {
      float m = -INFINITY;
      for (int j = lane; j < k; j += 64) m = fmaxf(m, zs[g * k + j]);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      float l = 0.f;
      for (int j = lane; j < k; j += 64) {
        const float z = zs[g * k + j];
        const float pj = z == -INFINITY ? 0.f : fast_exp2(z - m);
        zs[g * k + j] = pj;
        l += pj;
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o, 64);
      if (lane == 0) stat[g][0] = m, stat[g][1] = l;
    }
    __syncthreads();
    // ---- pass 3: P V for this lane's head and 8 dims over its keys
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int j = wave * KW + kl; j < k; j += KB) {
      const float pj = hv ? zs[hh * k + j] : 0.f;
      if (pj != 0.f) {  // (a masked or missing key has probability 0)
        const int s = ix[j];
        const u32x4 w4 = ld16(vv + (((int64_t)b * Tk + s) * H + h0 + hh) * kMhaD + dc * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] = fmaf(pj, __uint_as_float(w4[e] << 16), acc[2 * e]);
          acc[2 * e + 1] = fmaf(pj, __uint_as_float(w4[e] & 0xFFFF0000u), acc[2 * e + 1]);
        }
      }
    }
#pragma unroll
    for (int o = C; o < 64; o <<= 1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o, 64);
    }
    if (kl == 0) {
      *reinterpret_cast<float4*>(&ored[wave][hh * kMhaD + dc * 8]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      *reinterpret_cast<float4*>(&ored[wave][hh * kMhaD + dc * 8 + 4]) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
    __syncthreads();
    for (int x = tid; x < G * kMhaD; x += 256) {
      const int g = x / kMhaD, h = h0 + g;
      if (h < H) {
        const float l = stat[g][1];
        const float o = (ored[0][x] + ored[1][x]) + (ored[2][x] + ored[3][x]);
        out[(row * H + h) * kMhaD + x % kMhaD] = f32_to_bf16_bits(l == 0.f ? 0.f : o / l);
        if (lse && x % kMhaD == 0) lse[row * H + h] = l == 0.f ? -INFINITY : (stat[g][0] + __log2f(l)) * kLn2;
      }
    }
    __syncthreads();  // the LDS areas are reused by the next round
  }
}

// heads per round and LDS capacity of the multi-head kernel: all heads (padded to a power
// of two) when they fit, else as many as 16384 logits allow (k <= 4096: at least four)
int mha_group(int H, int k) {
  int hp = 1;
  while (hp < H) hp <<= 1;
  int g = hp;
  while (g > 1 && (int64_t)g * k > 16384) g >>= 1;
  return g;
}

// Paged latent cache: selected key s of sequence b (an index row of Tq*k entries per
// sequence) becomes pool row block_table[b][s >> shift] << shift | (s & (page - 1)); entries
// outside [0, L_b), and rows a table entry places outside the pool, become -1 (skipped).
__global__ __launch_bounds__(256) void page_translate_kernel(const int32_t* __restrict__ idx, int32_t* __restrict__ phys,
                                                             int64_t n, int64_t per_seq, const int32_t* __restrict__ kv_len,
                                                             int Tk, const int32_t* __restrict__ bt, int max_blocks,
                                                             int page_shift, int64_t pool_tokens) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  const int b = (int)(e / per_seq);
  const int64_t L = seq_len(kv_len, b, Tk);
  const int s = idx[e];
  int r = -1;
  if (s >= 0 && s < L) {
    const int64_t pr = ((int64_t)bt[(int64_t)b * max_blocks + (s >> page_shift)] << page_shift) +
                       (s & ((1 << page_shift) - 1));
    r = pr >= 0 && pr < pool_tokens ? (int)pr : -1;
  }
  phys[e] = r;
}

}  // namespace

bool attn_mla_supported(const AttnArgs& a) {
  // the gather addresses a sequence's rows with 32-bit byte offsets
  // (and a missing row's offsets, from kRowNone, must stay past the range)
  const int64_t row_bytes = a.kv_fmt == kKvMxfp4 ? TileStage<kKvMxfp4>::kRowBytes
                            : a.kv_fmt == kKvFp8 ? TileStage<kKvFp8>::kRowBytes
                                                 : TileStage<kKvBf16>::kRowBytes;
  const int64_t seq_bytes = (int64_t)a.Tk * row_bytes;
  return a.kv_fmt >= kKvBf16 && a.kv_fmt <= kKvMxfp4 && a.Hkv == 1 && a.Dqk == kDqk && a.Dv == kDv &&
         a.v == nullptr && a.H % 16 == 0 && a.H > 0 && a.k >= 1 && a.k <= 65536 && seq_bytes <= kRowNone;
}

bool attn_mha_supported(const AttnArgs& a) {
  return a.kv_fmt == kKvBf16 && a.Hkv == a.H && a.H >= 1 && a.H <= 16 && a.Dqk == kMhaD && a.Dv == kMhaD && a.v != nullptr &&
         a.k >= 1 && a.k <= kMhaMaxK;
}

int attn_mla_splits(int B, int Tq, int H, int k, int nlayers) {
  // few rows (decode): split each row's key list so ~512 workgroups (2 per CU) run; a
  // launch of several layers aims at ~768 in all (measured on the 64-row decode step with
  // three layers: 4 splits per layer 0.213 ms, 8 splits 0.226 ms, 16 splits 0.238 ms)
  const int64_t wgs = (int64_t)B * Tq * (H / 16);
  const int tiles = (k + kTile - 1) / kTile;
  if (wgs >= 256) return 1;
  const int64_t target = nlayers > 1 ? 768 / nlayers : 512;
  // (at most 64: the merge holds one split per lane)
  int s = (int)std::min<int64_t>(std::min(tiles, 64), (target + wgs - 1) / std::max<int64_t>(1, wgs));
  if (nlayers > 1) {  // a power of two (even splits of a power-of-two tile count); rounding down
    int p = 1;
    while (2 * p <= s) p *= 2;
    s = p;
  }
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

hipError_t launch_page_translate(const int32_t* idx, int32_t* phys, int B, int Tq, int k, const int32_t* kv_len,
                                 int Tk, const int32_t* block_table, int max_blocks, int page_shift,
                                 int64_t pool_tokens, hipStream_t st) {
  const int64_t n = (int64_t)B * Tq * k;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(page_translate_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, idx, phys, n,
                     (int64_t)Tq * k, kv_len, Tk, block_table, max_blocks, page_shift, pool_tokens);
  return hipGetLastError();
}

hipError_t launch_sparse_attn_layers(const AttnArgs& a, const AttnLayer* layers, int nlayers, hipStream_t st) {
  const int64_t rows = (int64_t)a.B * a.Tq;
  if (rows == 0 || nlayers < 1) return hipSuccess;
  if (nlayers > kMaxAttnLayers || (nlayers > 1 && !attn_mla_supported(a))) return hipErrorInvalidValue;
  if (attn_mla_supported(a)) {
    const float sl2 = a.sm_scale * kLog2e;
    const int tiles = (a.k + kTile - 1) / kTile;
    const int nsplit = attn_mla_splits(a.B, a.Tq, a.H, a.k, nlayers);
    const int per = (tiles + nsplit - 1) / nsplit;
    const int64_t nrowh = rows * a.H;
    MlaLayers Ls = {};
    for (int z = 0; z < nlayers; ++z) {
      Ls.q[z] = layers[z].q;
      Ls.kv[z] = (const uint8_t*)layers[z].kv;
      Ls.kv_scale[z] = layers[z].kv_scale;
      Ls.out[z] = layers[z].out;
      Ls.lse[z] = layers[z].lse;
    }
    // split partials of layer z: one single-layer workspace slice (sized for the most splits
    // any launch of this shape takes; O then (m, l)) after layer z-1's
    float* part_o = nullptr;
    float* part_ml = nullptr;
    const int64_t part_layer = (int64_t)(attn_workspace_bytes(a.B, a.Tq, a.H, a.Dv, a.k, true) / sizeof(float));
    if (nsplit > 1) {
      part_o = reinterpret_cast<float*>(a.ws);
      part_ml = part_o + (size_t)nsplit * nrowh * kDv;
    }
    dim3 grid((unsigned)(rows * (a.H / 16)), nsplit, nlayers);
    const int64_t bstride = a.kv_bstride < 0 ? (int64_t)a.Tk : a.kv_bstride;
    const bool wide = a.kv_fmt == kKvBf16 && nsplit == 1 && a.Tk <= kWideMaxTk;
#define DSA_MLA_LAUNCH(F, W)                                                                                       \
  hipLaunchKernelGGL((mla_attn_kernel<F, W>), grid, dim3(256), 0, st, Ls, a.idx, a.Tq, a.Tk, bstride, a.H, a.k, sl2, \
                     per, part_o, part_ml, part_layer)
    if (a.kv_fmt == kKvFp8)
      DSA_MLA_LAUNCH(kKvFp8, 0);
    else if (a.kv_fmt == kKvMxfp4)
      DSA_MLA_LAUNCH(kKvMxfp4, 0);
    else if (wide)
      DSA_MLA_LAUNCH(kKvBf16, 1);
    else
      DSA_MLA_LAUNCH(kKvBf16, 0);
#undef DSA_MLA_LAUNCH
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || nsplit == 1) return e;
    hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)((nrowh + 3) / 4), nlayers), dim3(256), 0, st, part_o,
                       part_ml, part_layer, nsplit, nrowh, a.H, Ls);
    return hipGetLastError();
  }
  if (attn_mha_supported(a)) {
    const int g = mha_group(a.H, a.k);
    const bool small = (int64_t)g * a.k <= 2048;
    const float sl2 = a.sm_scale * kLog2e;
#define DSA_MHA_LAUNCH(G, Z)                                                                                      \
  hipLaunchKernelGGL((mha_attn_kernel<G, Z>), dim3((unsigned)rows), dim3(256), 0, st, a.q, (const uint16_t*)a.kv, \
                     a.v, a.idx, a.Tq, a.Tk, a.H, a.k, sl2, a.out, a.lse)
#define DSA_MHA_CAP(G) \
  if (small) DSA_MHA_LAUNCH(G, 2048); else DSA_MHA_LAUNCH(G, 16384);
    switch (g) {
      case 1: DSA_MHA_CAP(1); break;
      case 2: DSA_MHA_CAP(2); break;
      case 4: DSA_MHA_CAP(4); break;
      case 8: DSA_MHA_CAP(8); break;
      default: DSA_MHA_CAP(16); break;
    }
#undef DSA_MHA_CAP
#undef DSA_MHA_LAUNCH
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t st) {
  const AttnLayer l0{a.q, a.kv, a.kv_scale, a.out, a.lse};
  return launch_sparse_attn_layers(a, &l0, 1, st);
}

}  // namespace dsa
