// Attention restricted to each query's selected keys, on gfx950.
//
//   out[h] = sum_s softmax_s(sm_scale * q[h] . K[s]) V[s],  s over the row's index list
//
// MLA form (DeepSeek-V2-Lite-Chat SIQ card, "Measured": one 576-wide latent row per token,
// 512 compressed-KV values then 64 rotary values; V = the first 512 values of the same
// row).  A workgroup of four waves serves one query row and 16 heads; each wave owns the
// 16-key steps w, w + 4, ... of the row's index list with its own online softmax (base 2)
// and O, and the waves' results are merged once per row.  A step's gathered rows are staged
// in the wave's LDS and used twice: as K (all 576 columns) for S^T = K Q^T with the keys as
// the MFMA M dimension, and as V (columns 0..511) for O^T += V^T P^T, read transposed
// straight from LDS with ds_read_b64_tr_b16.  The next step's gather is issued into
// registers before the current step is computed.  fp8 (OCP e4m3) rows are widened to bf16
// exactly while staged; their per-token scale multiplies the logit and the probability.
// MXFP4 rows (OCP microscaling: 32-value blocks of e2m1 elements sharing an E8M0 scale;
// the same card's "Measured" section names an nvfp4 latent cache for sparse MLA) are
// decoded with their block scales while staged, also exactly: e2m1 times a power of two
// has two significant bits.  Decode rows (few queries) split the key list over
// workgroups and merge the partial results by log-sum-exp in a second kernel, in a fixed
// order.
//
// Multi-head form (DSA ablation card: 4 heads of width 32, RoPE'd inputs): a workgroup per
// query row, key rows read as 16-byte chunks spread over the lanes, logits in LDS, three
// fixed-order passes.
#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace dsa {

namespace {

constexpr int kDqk = 576, kDv = 512;
constexpr int kTile = 32;                // selected keys per tile
constexpr int kRowB = kDqk * 2;          // staged bf16 row: 1152 B = 72 chunks of 16 B
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
// The swizzle moves a chunk only inside its group of 8, so lds_off(r, c + 8 g) = lds_off(r, c)
// + 128 g: a lane's reads and writes of a row take one base per chunk residue and carry the
// rest as the LDS instruction's immediate offset (no per-access address arithmetic).

// Gather of a key row: eight lanes per row, lane l owning the 16-byte parts l%8, l%8+8, ...,
// so every load instruction reads eight full 128-byte lines.  Rows go through registers into LDS (bf16; fp8 and fp4 widened exactly).
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
    uint8_t* b = lds + lds_off(key, part0);  // chunk part0 + 8c
#pragma unroll
    for (int c = 0; c < kChunks; ++c) *reinterpret_cast<u32x4*>(b + 128 * c) = r[c];
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
  // bytes 2*HI and 2*HI+1 of a word as a bf16 pair (e4m3 values are exact in bf16): one
  // scaled conversion (scale 1), which gives the same bits as widening through fp32 for all
  // 65536 byte pairs, NaN payloads included (checked on the device)
  template <bool HI>
  __device__ __forceinline__ static uint32_t widen2(uint32_t word) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, HI));
  }
  __device__ __forceinline__ void store(uint8_t* lds, int key, int part0) const {
    // bf16 chunks 2 part and 2 part + 1, part = part0 + 8c: two bases, 256 B per c
    uint8_t* b0 = lds + lds_off(key, 2 * part0);
    uint8_t* b1 = lds + lds_off(key, 2 * part0 + 1);
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
      *reinterpret_cast<u32x4*>(b0 + 256 * c) = lo;
      *reinterpret_cast<u32x4*>(b1 + 256 * c) = hi;
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
  // elements 2B and 2B+1 of an 8-element word, times the scale, as a bf16 pair (low first):
  // one scaled conversion, which gives the same bits as converting to fp32 and keeping the
  // upper halves for every byte value, byte position and E8M0 scale, NaNs included (e2m1
  // times a power of two has two significant bits; checked on the device, 524288 cases)
  template <int B>
  __device__ __forceinline__ static uint32_t pair(uint32_t word, float scale) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, B));
  }
  __device__ __forceinline__ void store(uint8_t* lds, int key, int part0) const {
    uint8_t* b[4];  // staged chunk 4 blk + w, blk = part0 + 8c: base w, 512 B per c
#pragma unroll
    for (int w = 0; w < 4; ++w) b[w] = lds + lds_off(key, 4 * part0 + w);
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
        *reinterpret_cast<u32x4*>(b[w] + 512 * c) = o;
      }
    }
  }
};

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


// ---- the MLA kernel: one wave per key step ------------------------------------------------
// A workgroup of kWkWaves waves serves one query row and 16 heads.  Wave w takes the 16-key
// steps w, w + NW, w + 2 NW, ... of the row's index list (entries 16 (NW i + w) .. +15) and
// keeps its own online-softmax state and O for all 16 heads and 512 dims, so the key loop has
// no barrier: each wave stages its rows in two LDS slots of its own (the swizzle above).
// Four waves (one workgroup per CU, 145 KB of LDS) keep 256 rows in flight; at T=65536 that
// gathers with fewer L2 misses than two waves at two workgroups per CU (13.3 against 14.9 ms)
// or one wave at four (16.4 ms): concurrent rows at the same list position read the same
// key range, and fewer, faster rows keep that range narrower.
// Per step:
//   S^T (16 keys x 16 heads) = K Q^T in 18 MFMA k-steps, the keys as M (K rows from LDS,
//   Q^T in registers); the softmax leaves each lane the probabilities of its 4 keys for its
//   head, which is exactly the B operand of O^T += V^T P^T over those 16 keys (16x16x16
//   MFMAs, V read transposed from LDS).
// The waves' (m, l, O) are merged once per row, in a fixed order.  Rows are gathered
// into registers and written to the free slot one step before they are used.
// O is never rescaled inside the loop: each head's reference is the max of its first tile
// with a valid key, and later probabilities exp2(s - ref) may reach 2^kWkSlack, which fp32
// sums and bf16 probabilities hold.  A tile that exceeds its head's reference by more than
// that flags the row, which is then computed again from the head's exact max (a pass of
// Q K^T alone first); ordinary rows never take that path, and the loop keeps O in the
// accumulator registers (a rescale inside it made the compiler move O to vector registers
// and spill).
constexpr int kWkKeys = 16;               // keys per wave step
constexpr int kWkWaves = 4;               // waves per workgroup (query row)
constexpr int kWkSlot = kWkKeys * kRowB;  // 18 KB
constexpr float kWkSlack = 64.f;

__device__ __forceinline__ f32x4 mfma16k16(i16x4 a, i16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

template <int FMT, int NW>  // row format; waves per workgroup (query row)
__global__ __launch_bounds__(64 * NW, NW >= 4 ? 1 : 4 / NW) void mla_attn_wk_kernel(
    const MlaLayers Ls, const int32_t* __restrict__ idx, int Tq, int Tk, int64_t kv_bstride, int H, int k,
    float scale_log2, int tiles_per_split, float* __restrict__ part_o, float* __restrict__ part_ml, int64_t part_layer,
    const int32_t* __restrict__ tail_kv_len, int tail_Tk, int64_t nrg) {
  constexpr bool FP8 = FMT == kKvFp8;  // per-token scale on logits and probabilities
  constexpr uint32_t kRowBytes = TileStage<FMT>::kRowBytes;
  __shared__ __attribute__((aligned(16))) uint8_t kvs[NW][2][kWkSlot];  // [wave][slot]: bf16 rows once staged
  __shared__ __attribute__((aligned(16))) float kscale[NW][2][kWkKeys];  // fp8 row scales of each slot
  __shared__ float ml_red[NW][16][3];

  // layer z's operands; its split partials sit part_layer floats after layer z-1's
  const int z = blockIdx.z;
  const uint16_t* __restrict__ q = Ls.q[z];
  const uint8_t* __restrict__ kv = Ls.kv[z];
  const float* __restrict__ kv_scale = Ls.kv_scale[z];
  uint16_t* __restrict__ out = Ls.out[z];
  float* __restrict__ lse = Ls.lse[z];
  part_o += z * part_layer;
  part_ml += z * part_layer;

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int HG = H >> 4;
  // (row, head group) pairs: a launch of more pairs than CUs keeps one resident workgroup
  // per CU, which takes every gridDim.x-th pair and moves on to its next one instead of a
  // new workgroup being dispatched (rows in flight stay consecutive).  Rows whose extent
  // comes from their position (top-k rows: the first k rows are shorter) go last to first,
  // so the long rows keep the workgroups in step and the short ones fill the end; a
  // front-to-back walk let the workgroups that drew short rows run ahead, which widened
  // the window of rows in flight (T=65536: 12.8-13.1 ms against 11.9-12.4 reversed).
  // Lists read in full (every row the same length) go front to back.  Inside a full window
  // of gridDim.x consecutive pairs, workgroup w takes slot (w % 8) * (gridDim.x / 8) + w / 8:
  // workgroups are dispatched over the 8 XCDs round-robin, so each XCD's L2 then serves
  // adjacent rows, whose top-k lists overlap most (T=65536 plain call, front to back:
  // 12.13-12.17 against 12.65-12.75 ms with slot w; the layer stack's last-to-first walk
  // 12.2 ms either way).  Partial windows keep slot w.
  for (int64_t rwi0 = blockIdx.x; rwi0 < nrg; rwi0 += gridDim.x) {
  const int64_t win0 = rwi0 - blockIdx.x;
  const bool full = gridDim.x % 8 == 0 && win0 + gridDim.x <= nrg;
  const int64_t rwi = full ? win0 + (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8 : rwi0;
  const int64_t rowh = tail_Tk > 0 ? nrg - 1 - rwi : rwi;
  const int64_t row = rowh / HG;
  const int hg = (int)(rowh % HG);
  const int b = (int)(row / Tq);
  const int split = blockIdx.y, nsplit = gridDim.y;
  const int32_t* ix = idx + row * k;
  const __amdgpu_buffer_rsrc_t kv_rs = make_rsrc(kv + b * kv_bstride * kRowBytes, (uint32_t)Tk * kRowBytes);
  const __amdgpu_buffer_rsrc_t sc_rs = make_rsrc(FP8 ? kv_scale + b * kv_bstride : nullptr, FP8 ? (uint32_t)Tk * 4 : 0u);
  const __amdgpu_buffer_rsrc_t ix_rs = make_rsrc(ix, (uint32_t)k * 4);

  // lane roles: hl = head (S^T and O^T column), gq = which 4 keys of a step (rows 4gq..)
  const int hl = lane & 15, gq = lane >> 4;
  bf16x8 qb[18];  // Q^T as the B operand: column = head hl, dims 32s + 8gq .. +7
  {
    const uint16_t* qp = q + (row * H + hg * 16 + hl) * kDqk + gq * 8;
#pragma unroll
    for (int s = 0; s < 18; ++s) qb[s] = as_bf16x8(ld16(qp + s * 32));
    // Q^T lives in accumulator registers (an MFMA reads its B operand from there too),
    // leaving the vector registers to the row stage and the LDS operands read ahead
#pragma unroll
    for (int s = 0; s < 18; ++s) asm volatile("" : "+a"(qb[s]));
  }

  // This split's entries [e_lo, e_hi).  Entries past a row's valid ones add nothing (they
  // read no row and their logits are -inf), so the loop covers the split's whole range
  // unless the list is a top-k row, whose valid entries are its first min(k, p+1): then the
  // range ends there.  (A scan of the list for its last valid entry, with a barrier, cost 9%
  // at T=65536: 13.5 against 12.3 ms.)
  const int e_lo = split * tiles_per_split * kTile;
  int e_hi = min(k, e_lo + tiles_per_split * kTile);
  if (tail_Tk > 0) {
    const int64_t p = seq_len(tail_kv_len, b, tail_Tk) - Tq + (int)(row % Tq);
    e_hi = (int)min<int64_t>(e_hi, max<int64_t>(0, min<int64_t>(k, p + 1)));
  }
  const int nblk = e_hi > e_lo ? (e_hi - e_lo + kWkKeys - 1) / kWkKeys : 0;
  const int nsteps = (nblk - wave + NW - 1) / NW;  // this wave's blocks: wave, wave + NW, ... < nblk

  // gather roles: lane l loads the rows of keys l/8 and 8 + l/8 of a step, 16-byte parts
  // l%8 + 8c (eight lanes per row: every load instruction reads eight full 128-byte lines)
  const int gkey = lane >> 3, part0 = lane & 7;
  auto entry_off = [&](int i, int g) -> int { return e_lo + (NW * i + wave) * kWkKeys + gkey + 8 * g; };
  auto raw_entry = [&](int i, int g) -> int {
    return (int)__builtin_amdgcn_raw_buffer_load_b32(ix_rs, i < nsteps ? entry_off(i, g) * 4 : (int)kOffNone, 0, 0);
  };
  auto valid_entry = [&](int i, int g, int raw) -> int {
    const int lim = (i < nsteps && entry_off(i, g) < e_hi) ? Tk : 0;
    return (uint32_t)raw < (uint32_t)lim ? raw : -1;
  };
  TileStage<FMT> st[2];  // the register stage: rows gkey and gkey + 8 of one step
  uint32_t rmask = 0;    // its valid keys (bit r: key r of the step)
  auto gather = [&](int i, int e0, int e1) __attribute__((always_inline)) {
    st[0].s = valid_entry(i, 0, e0);
    st[1].s = valid_entry(i, 1, e1);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      st[g].load(kv_rs, part0);
      if (FP8) st[g].sc = buf_load_f32(sc_rs, st[g].s >= 0 ? (uint32_t)st[g].s * 4 : kOffNone, 0);
    }
    // lanes 8r .. 8r+7 hold keys r and 8 + r, so each byte of a ballot is 0 or 0xFF: one
    // bit per byte, gathered by a multiply (bits 0, 8, 16, 24 land on 24 .. 27 alone)
    const uint64_t v0 = __ballot(st[0].s >= 0), v1 = __ballot(st[1].s >= 0);
    auto gather4 = [](uint32_t x) { return ((x & 0x01010101u) * 0x01020408u) >> 24; };
    rmask = gather4((uint32_t)v0) | gather4((uint32_t)(v0 >> 32)) << 4 | gather4((uint32_t)v1) << 8 |
            gather4((uint32_t)(v1 >> 32)) << 12;
  };
  auto stage = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < 2; ++g) st[g].store(kvs[wave][slot], gkey + 8 * g, part0);
    if (FP8 && part0 == 0) {
      kscale[wave][slot][gkey] = st[0].sc;
      kscale[wave][slot][gkey + 8] = st[1].sc;
    }
  };

  f32x4 o_acc[32];  // O^T: rows = dims 16n + 4gq + i, column = head hl
#pragma unroll
  for (int n = 0; n < 32; ++n) o_acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  // m_run: the head's reference (uniform over its lanes); l_run and l_rnd: this lane's share
  // of the sum of exponentials, exact and as rounded into the P V operand (bf16 and MXFP4
  // rows normalize by the rounded sum, so the weights of O sum to one exactly; the exact
  // sum gives lse).  Both are reduced over the head's lanes once, after the loop.
  float m_run = -INFINITY, l_run = 0.f, l_rnd = 0.f;

  // base-2 logits of the lane's 4 keys for head hl (-inf for a missing key); ksc: the keys'
  // fp8 scales (1 otherwise)
  auto qk = [&](int slot, uint32_t msk, float (&sv)[4], float (&ksc)[4]) __attribute__((always_inline)) {
    const uint8_t* sl = kvs[wave][slot];
    // two accumulation chains (even and odd k-steps), added at the end
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
    // K operand s is chunk 4s + gq of row hl: base s & 1, then 128 B per pair of steps
    const uint8_t* kb[2] = {sl + lds_off(hl, gq), sl + lds_off(hl, 4 + gq)};
    u32x4 kr[18];  // every K operand read first, so the reads overlap
#pragma unroll
    for (int s = 0; s < 18; ++s) kr[s] = *reinterpret_cast<const u32x4*>(kb[s & 1] + 128 * (s >> 1));
#pragma unroll
    for (int s = 0; s < 18; s += 2) {
      a0 = mfma16(as_bf16x8(kr[s]), qb[s], a0);
      a1 = mfma16(as_bf16x8(kr[s + 1]), qb[s + 1], a1);
    }
    // six reads ahead, then one MFMA per read (the scheduler otherwise waits on each read
    // right before its MFMA)
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int g = 0; g < 12; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
    f32x4 kscv = {1.f, 1.f, 1.f, 1.f};
    if (FP8) kscv = *reinterpret_cast<const f32x4*>(&kscale[wave][slot][4 * gq]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ksc[e] = kscv[e];
      sv[e] = ((msk >> (4 * gq + e)) & 1u) ? (a0[e] + a1[e]) * (FP8 ? kscv[e] * scale_log2 : scale_log2) : -INFINITY;
    }
  };
  bool redo = false;
  // online softmax of one step's logits: P^T as the B operand of P V (probabilities carry
  // the fp8 row scale for V; the sum does not)
  auto softmax = [&](const float (&sv)[4], const float (&ksc)[4]) __attribute__((always_inline)) -> i16x4 {
    const float tm = rows_max(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
    if (m_run == -INFINITY)
      m_run = tm;  // the head's first valid keys (O and l are still 0); stays -inf otherwise
    else if (tm > m_run + kWkSlack)
      redo = true;
    const float mref = m_run == -INFINITY ? 0.f : m_run;  // (then every sv is -inf)
    float p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = fast_exp2(sv[e] - mref);
    l_run += (p[0] + p[1]) + (p[2] + p[3]);
    if (FP8) {
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] *= ksc[e];
    }
    const uint32_t w0 = cvt_bf16x2(p[0], p[1]), w1 = cvt_bf16x2(p[2], p[3]);
    if (!FP8)
      l_rnd += (__uint_as_float(w0 << 16) + __uint_as_float(w0 & 0xffff0000u)) +
               (__uint_as_float(w1 << 16) + __uint_as_float(w1 & 0xffff0000u));
    return __builtin_bit_cast(i16x4, make_uint2(w0, w1));
  };
  // O^T += V^T P^T: lane (gq, hl) reads keys 4gq .. 4gq+3 at dim 16n + hl (transposed)
  auto pv = [&](int slot, i16x4 pb) __attribute__((always_inline)) {
    const uint8_t* sl = kvs[wave][slot];
    const int r0 = 4 * gq + (hl >> 2);
    // dims 16m + 4(hl & 3) .. +3 of row r0: chunk 2m + ((hl >> 1) & 1), byte 8 (hl & 1) in it,
    // so base m & 3, then 128 B per four m
    const uint8_t* vb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) vb[j] = sl + lds_off(r0, 2 * j + ((hl >> 1) & 1)) + 8 * (hl & 1);
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {  // sixteen operand reads, then their MFMAs
      i16x4 v[16];
#pragma unroll
      for (int n = 0; n < 16; ++n) {
        const int m = 16 * h2 + n;
        v[n] = lds_read_tr16(vb[m & 3] + 128 * (m >> 2));
      }
#pragma unroll
      for (int n = 0; n < 16; ++n) o_acc[16 * h2 + n] = mfma16k16(v[n], pb, o_acc[16 * h2 + n]);
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
      for (int g = 0; g < 10; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
    }
  };
  auto compute = [&](int slot, uint32_t msk) __attribute__((always_inline)) {
    float sv[4], ksc[4];
    qk(slot, msk, sv, ksc);
    pv(slot, softmax(sv, ksc));
  };

  for (int attempt = 0;; ++attempt) {
    if (attempt == 1) {
      // a tile outgrew its head's reference: the exact max of every head first (Q K^T
      // alone, one step at a time), then the row again from it
      float mt = -INFINITY;
      for (int i = 0; i < nsteps; ++i) {
        gather(i, raw_entry(i, 0), raw_entry(i, 1));
        stage(0);
        float sv[4], ksc[4];
        qk(0, rmask, sv, ksc);
        mt = fmaxf(mt, rows_max(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]))));
      }
      m_run = mt;
      l_run = 0.f;
      l_rnd = 0.f;
#pragma unroll
      for (int n = 0; n < 32; ++n) o_acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    redo = false;
    // one register stage.  Iteration i (parity P) finds step i in slot P and step i+1 in the
    // register stage; it stages step i+1 into slot 1-P, gathers step i+2 and computes step i.
    uint32_t mask_slot[2];
    int en0, en1;
    {
      const int e00 = raw_entry(0, 0), e01 = raw_entry(0, 1);
      const int e10 = raw_entry(1, 0), e11 = raw_entry(1, 1);
      en0 = raw_entry(2, 0);
      en1 = raw_entry(2, 1);
      gather(0, e00, e01);
      stage(0);
      mask_slot[0] = rmask;
      gather(1, e10, e11);
    }
    auto iter = [&](auto par_c, int i) __attribute__((always_inline)) {
      constexpr int P = decltype(par_c)::value;
      stage(1 - P);
      mask_slot[1 - P] = rmask;
      __builtin_amdgcn_sched_barrier(0);  // the stage's registers are free before the next gather
      gather(i + 2, en0, en1);
      en0 = raw_entry(i + 3, 0);
      en1 = raw_entry(i + 3, 1);
      compute(P, mask_slot[P]);
    };
    {
      int i = 0;
      for (; i + 1 < nsteps; i += 2) {
        iter(std::integral_constant<int, 0>{}, i);
        iter(std::integral_constant<int, 1>{}, i + 1);
      }
      if (i < nsteps) iter(std::integral_constant<int, 0>{}, i);
    }
    if (!__syncthreads_or(redo) || attempt == 1) break;  // (the second pass never flags)
  }

  // ---- results: merge the waves ((m, l) per head, then O over the waves in wave order),
  // then the normalized output, or this split's partial (O relative to m, and (m, l))
  const int h = hg * 16 + hl;
  l_run = rows_sum(l_run);
  l_rnd = FP8 ? l_run : rows_sum(l_rnd);
  float mx = m_run, lt = l_run, lr = l_rnd;
  if constexpr (NW > 1) {
    __syncthreads();  // every wave is done with its slots
    if (gq == 0) {
      ml_red[wave][hl][0] = m_run;
      ml_red[wave][hl][1] = l_run;
      ml_red[wave][hl][2] = l_rnd;
    }
    __syncthreads();
    mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, ml_red[w][hl][0]);
    const float mxr0 = mx == -INFINITY ? 0.f : mx;
    float mine = 0.f;
    lt = 0.f;
    lr = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = fast_exp2(ml_red[w][hl][0] - mxr0);
      lt += ml_red[w][hl][1] * f;
      lr += ml_red[w][hl][2] * f;
      mine = w == wave ? f : mine;
    }
    f32x4* ob = reinterpret_cast<f32x4*>(&kvs[wave][0][0]);  // 32 KB of this wave's region
#pragma unroll
    for (int n = 0; n < 32; ++n) ob[n * 64 + lane] = o_acc[n] * mine;
    __syncthreads();
  }
  const float mxr = mx == -INFINITY ? 0.f : mx;
  constexpr int NT = 32 / NW;  // dim tiles each wave writes
  auto o_tile = [&](int n) -> f32x4 {
    if constexpr (NW == 1) {
      return o_acc[n];
    } else {
      f32x4 x = reinterpret_cast<const f32x4*>(&kvs[0][0][0])[n * 64 + lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) x += reinterpret_cast<const f32x4*>(&kvs[w][0][0])[n * 64 + lane];
      return x;
    }
  };
  if (nsplit == 1) {
    const float inv = lr == 0.f ? 0.f : 1.f / lr;  // (a NaN sum stays NaN)
    uint16_t* op = out + (row * H + h) * kDv + 4 * gq;
#pragma unroll
    for (int nn = 0; nn < NT; ++nn) {
      const int n = wave * NT + nn;
      const f32x4 x = o_tile(n);
      const uint32_t lo = cvt_bf16x2(x[0] * inv, x[1] * inv);
      const uint32_t hi = cvt_bf16x2(x[2] * inv, x[3] * inv);
      *reinterpret_cast<uint2*>(op + n * 16) = make_uint2(lo, hi);
    }
    if (lse && wave == 0 && gq == 0) lse[row * H + h] = lt == 0.f ? -INFINITY : (mxr + __log2f(lt)) * kLn2;
  } else {
    const int64_t nrowh = nrg * 16;  // (row, head) pairs over all rows
    const int64_t rh = rowh * 16 + hl;
    float* po = part_o + ((int64_t)split * nrowh + rh) * kDv + 4 * gq;
    // the partial carries the exact sum: O rescaled to it from the rounded one
    const float corr = lr == 0.f ? 1.f : lt / lr;
#pragma unroll
    for (int nn = 0; nn < NT; ++nn) {
      const int n = wave * NT + nn;
      *reinterpret_cast<f32x4*>(po + n * 16) = o_tile(n) * corr;
    }
    if (wave == 0 && gq == 0) {
      part_ml[((int64_t)split * nrowh + rh) * 2 + 0] = mx;
      part_ml[((int64_t)split * nrowh + rh) * 2 + 1] = lt;
    }
  }
  __syncthreads();  // the next row reuses the slots and the merge buffers
  }  // rows
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

// Compute units of the current device (cached per device; 256 on MI355X).  Calls may come
// from several host threads: the cache entries are atomic (a race only repeats the query).
int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

int attn_mla_splits(int B, int Tq, int H, int k, int nlayers) {
  // few rows (decode): split each row's key list so that one round of whole-key workgroups
  // (one per CU) covers the launch, every layer of a grouped launch alike: a lone 64-row
  // layer takes four splits (256 workgroups), three grouped 64-row layers none (192, and no
  // merge).  A power of two: even splits of a power-of-two tile count.
  const int64_t wgs = (int64_t)B * Tq * (H / 16) * std::max(1, nlayers);
  const int tiles = (k + kTile - 1) / kTile;
  if (wgs >= 256) return 1;
  // (at most 64: the merge holds one split per lane)
  int s = (int)std::min<int64_t>(std::min(tiles, 64), 256 / std::max<int64_t>(1, wgs));
  int p = 1;
  while (2 * p <= s) p *= 2;
  s = p;
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
    // one workgroup per (row, head group) and split, or, for unsplit launches of more rows
    // than the chip holds at once (one workgroup per CU), one per CU looping over rows
    const int64_t nrg = rows * (a.H / 16);
    const int64_t resident = std::max<int64_t>(1, device_cus() / nlayers);
    dim3 grid((unsigned)(nsplit == 1 ? std::min(nrg, resident) : nrg), nsplit, nlayers);
    const int64_t bstride = a.kv_bstride < 0 ? (int64_t)a.Tk : a.kv_bstride;
    {
#define DSA_WK_LAUNCH(F)                                                                                           \
  hipLaunchKernelGGL((mla_attn_wk_kernel<F, kWkWaves>), grid, dim3(64 * kWkWaves), 0, st, Ls, a.idx, a.Tq, a.Tk,   \
                     bstride, a.H, a.k, sl2, per, part_o, part_ml, part_layer, a.tail_kv_len, a.tail_Tk, nrg)
      if (a.kv_fmt == kKvFp8)
        DSA_WK_LAUNCH(kKvFp8);
      else if (a.kv_fmt == kKvMxfp4)
        DSA_WK_LAUNCH(kKvMxfp4);
      else
        DSA_WK_LAUNCH(kKvBf16);
#undef DSA_WK_LAUNCH
    }
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
