// Per-wave core of the lightning-indexer kernels:
//   I[t,s] = sum_j w[t,j] * max(0, sum_d q[t,j,d] * k[s,d])
// (DSA ablation model card, model list: ReLU indexer with a few small heads; one key per
// token shared by the heads, as its parameter count fixes).
//
// One 32x32x16 bf16 MFMA tile covers 32 (query, head) rows against 32 keys.  The rows are
// ordered so that the 16 accumulator values of a lane are all H_I heads of 16/H_I queries
// for one key: the ReLU and the head-weighted sum then run inside the lane, with no
// cross-lane traffic, and each lane ends with finished scores.  A wave keeps kQP query
// tiles of Q in registers and streams 32-key tiles through LDS; what happens to each
// finished score is the caller's epilogue (store it, sample it, filter it, histogram it).  Every kernel that
// scores a (query, key) pair goes through this code, so all of them produce the same fp32
// value for it: the MFMA k-steps, the head order of the sum and the rounding are fixed here.
#pragma once

#include "common.hpp"

namespace dsa {

// Query tiles per wave: as many (up to four) as fit the register file without spilling,
// next to the weights and the key pipeline (two tiles of rows, two of operands).
template <int H_I, int D_I>
constexpr int idx_query_tiles() {
  if (D_I <= 32 || (D_I == 64 && H_I >= 8)) return 4;
  return (D_I == 64 && H_I >= 2) || H_I >= 8 ? 2 : 1;
}

// Waits until at most N vector memory operations of this wave are outstanding (they
// complete in issue order); also a compiler barrier for memory accesses.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// STREAM: every key is read by this wave's rows only (a launch of one query tile, e.g.
// decode), so the key loads carry the non-temporal hint; measured on the 64 x 65536 decode
// keys: 104.3 against 106.5 us per launch, while prefill chunks, whose key tiles other
// query blocks read again from L2, ran 5% slower with it.
template <int H_I, int D_I, int kQP, bool STREAM = false>
struct IdxWave {
  static constexpr int QPT = 32 / H_I;   // queries per MFMA tile
  static constexpr int QPL = 16 / H_I;   // queries per lane (per tile)
  static constexpr int KS = D_I / 16;    // MFMA k-steps over the indexer width
  static constexpr int ROWS = kQP * QPT; // query rows of the wave
  static constexpr int EPIS = kQP * QPL; // epilogue calls per key tile
  static constexpr int CPK = D_I / 8;    // 16-byte chunks per key row
  static constexpr int KPI = 64 / CPK;   // keys per load instruction
  static constexpr int NLD = 32 / KPI;   // load instructions per tile
  static constexpr uint32_t kTileBytes = 32 * D_I * 2;
  // key tiles in flight, and LDS tile buffers: one more than in flight, so that a buffer is
  // refilled only once the operand reads of its last tile have completed.  128-wide keys
  // keep one tile in flight so that two workgroups still fit a CU.  A streaming wave (one
  // query tile) keeps two: 48 KB of LDS per workgroup lets three workgroups share a CU
  // (169 registers per lane allow three), which beat two workgroups with three tiles in
  // flight each on the 64 x 65536 decode keys (101.6 against 104.3 us; four tiles: 107.7).
  static constexpr int DEPTH = D_I >= 128 ? 1 : (STREAM ? 2 : 3);
  static constexpr int NB = DEPTH + 1;
  static constexpr uint32_t kLdsBytes = NB * kTileBytes;  // the wave's private key buffers

  bf16x8 a[kQP][KS];
  float wt[kQP][16];
  int g, col;  // lane group (query half of a tile) and key column

  // Wave-local row of (tile t, lane query qq): t*QPT + g*QPL + qq.
  __device__ __forceinline__ int row_of(int t, int qq) const { return t * QPT + g * QPL + qq; }

  // Q and head weights of rows [0, wrows) at q (bf16 [rows][H_I][D_I]) and w (bf16
  // [rows][H_I]); rows past wrows read as zero.
  __device__ __forceinline__ void load(const uint16_t* q, const uint16_t* w, int wrows) {
    const int lane = threadIdx.x & 63;
    g = lane >> 5;
    col = lane & 31;
    const __amdgpu_buffer_rsrc_t q_rs = make_rsrc(q, (uint32_t)max(wrows, 0) * H_I * D_I * 2);
    // A operand: lane row m = lane%32 <-> (query, head) such that D lane group g holds all
    // heads of queries g*QPL .. g*QPL+QPL-1 of the tile.
    const int m = lane & 31;
    const int mi = (m >> 3) * 4 + (m & 3);          // accumulator slot of row m
    const int mq = ((m >> 2) & 1) * QPL + mi / H_I;  // query within tile
    const int mh = mi % H_I;                         // head
    const int kh = (lane >> 5) * 8;                  // k offset of this lane within a k-step
#pragma unroll
    for (int t = 0; t < kQP; ++t) {
      const uint32_t off = (uint32_t)(((t * QPT + mq) * H_I + mh) * D_I + kh) * 2;
#pragma unroll
      for (int s = 0; s < KS; ++s) a[t][s] = as_bf16x8(buf_load_16(q_rs, off + s * 32, 0));
    }
    const __amdgpu_buffer_rsrc_t w_rs = make_rsrc(w, (uint32_t)max(wrows, 0) * H_I * 2);
#pragma unroll
    for (int t = 0; t < kQP; ++t) {
#pragma unroll
      for (int qq = 0; qq < QPL; ++qq) {
        const int r = row_of(t, qq);
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
  }

  template <int EPI_VM = 0, class Start, class Epi>
  __device__ __forceinline__ void run(__amdgpu_buffer_rsrc_t k_rs, uint8_t* lds, int ntiles, Start start, Epi epi) {
    run<EPI_VM>(k_rs, lds, ntiles, start, epi, [](int) {}, start);
  }
  template <int EPI_VM = 0, class Start, class Epi, class Post>
  __device__ __forceinline__ void run(__amdgpu_buffer_rsrc_t k_rs, uint8_t* lds, int ntiles, Start start, Epi epi,
                                      Post post) {
    run<EPI_VM>(k_rs, lds, ntiles, start, epi, post, start);
  }

  // Scores the wave's rows against key tiles j = 0 .. ntiles-1 (ntiles >= 1); tile j holds
  // keys start(j) .. start(j)+31 (wave-uniform; keys past the range of k_rs read as zero).
  // epi(j, s0, t, qq, score) runs on every lane for each tile j (s0 = start(j)), query tile
  // t and lane query qq, in a fixed order; the lane's key is s0 + col, its row row_of(t, qq).
  // post(j) runs after the last epilogue of tile j: work that branches belongs there, so
  // the MFMAs of one query tile can overlap the epilogue of the previous one.  phys(j) is
  // where tile j's 32 key rows sit in k_rs (start(j) for a dense key array; a page of a
  // paged cache otherwise): keys are loaded from there, masks and outputs use start(j).
  // EPI_VM is a lower bound on the vector memory operations that epi and post issue per
  // tile; the load waits count them (0 is always safe, only slower).  The kernels that pass
  // EPIS issue exactly one store per epi call as a single assembly instruction
  // (buf_store1_*), so the count holds whatever the compiler does around it.
  //
  // Key tiles go from memory straight into the wave's private LDS buffers (`lds`,
  // kLdsBytes) with buffer loads that write LDS: each load instruction reads whole key rows
  // (KPI keys of D_I*2 bytes), so no registers hold rows in flight, and DEPTH tiles are in
  // flight while one computes (a lane whose row is past the range of k_rs writes zeros to
  // its LDS slot, as a register load would return them: checked on the device).  The next
  // tile's MFMA operand comes back with one
  // ds_read_b128 per k-step before the current tile computes.  Only this wave touches its
  // buffers, so there is no barrier: the explicit waits order each tile's LDS writes before
  // its reads, and a buffer is refilled only after the reads of its previous tile.
  template <int EPI_VM = 0, class Start, class Epi, class Post, class Phys>
  __device__ __forceinline__ void run(__amdgpu_buffer_rsrc_t k_rs, uint8_t* lds, int ntiles, Start start, Epi epi,
                                      Post post, Phys phys) {
    const int lane = threadIdx.x & 63;
    constexpr int MASK = CPK < 8 ? CPK - 1 : 7;
    // chunk c of key j sits at chunk position c ^ ((j/2) & MASK): the operand reads (32 keys,
    // one chunk each) spread over all banks
    auto kl_off = [](int key, int chunk) { return key * (D_I * 2) + ((chunk ^ ((key >> 1) & MASK)) << 4); };
    // load instruction i: lane l fills LDS bytes 16*l of the instruction's KPI keys, i.e.
    // key i*KPI + l/CPK at chunk position l%CPK, so it reads chunk (l%CPK) ^ swizzle(key)
    uint32_t loff[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int key = i * KPI + lane / CPK;
      loff[i] = (uint32_t)(key * D_I * 2 + (((lane % CPK) ^ ((key >> 1) & MASK)) << 4));
    }
    // Tiles are loaded strictly in order (0, 1, 2, ...): one running offset, advanced by the
    // distance to the next tile's start.
    uint32_t gkoff = (uint32_t)phys(0) * (D_I * 2);
    int jn = 0;
    auto gload = [&](int buf) {
      typedef __attribute__((address_space(3))) uint8_t lds_u8;
      lds_u8* dst = (lds_u8*)(lds + buf * kTileBytes);
#pragma unroll
      for (int i = 0; i < NLD; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(k_rs, (__attribute__((address_space(3))) void*)(dst + i * KPI * D_I * 2),
                                                 16, gkoff + loff[i], 0, 0, STREAM ? 2 : 0);
      gkoff += (uint32_t)(phys(jn + 1) - phys(jn)) * (D_I * 2);
      ++jn;
    };
    auto lread = [&](int buf, bf16x8 (&bk)[KS]) {  // B operand: key col, dims 16s + 8g
      const uint8_t* wk = lds + buf * kTileBytes;
#pragma unroll
      for (int s = 0; s < KS; ++s)
        bk[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(wk + kl_off(col, 2 * s + g)));
    };
    auto tile = [&](int j, const bf16x8 (&bk)[KS]) {
      const int s0 = start(j);
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
          epi(j, s0, t, qq, tot);
        }
      }
      post(j);
    };
    bf16x8 B0[KS], B1[KS];
    constexpr int kWE = EPI_VM < 63 ? EPI_VM : 63;
    if constexpr (DEPTH == 1) {
      // tile j+1 loads (into the buffer of tile j-1, read before tile j-1 computed) while
      // tile j computes; its load is older than tile j's epilogue operations
      gload(0);
      vm_wait<0>();
      lread(0, B0);
      for (int j = 0; j < ntiles; j += 2) {
        gload(1);
        tile(j, B0);
        vm_wait<kWE>();
        lread(1, B1);
        if (j + 1 >= ntiles) break;
        gload(0);
        tile(j + 1, B1);
        vm_wait<kWE>();
        lread(0, B0);
      }
    } else {
      // Tiles 0 .. DEPTH-1 in flight, tile 0's operand in registers.  Tile j+DEPTH loads into
      // the buffer of tile j-1 (read before tile j-1 computed); then tile j+1's operand is
      // read.  At that point the loads of tiles j+2 .. j+DEPTH and the epilogue operations of
      // tiles max(0, j+1-DEPTH) .. j-1 may still be in flight, and vector memory operations
      // complete in issue order: the first DEPTH-1 tiles wait as if no epilogue operation
      // had been issued, the rest count DEPTH-1 tiles' worth.
      constexpr int kWHead = (DEPTH - 1) * NLD;
      constexpr int kWFull = (DEPTH - 1) * (NLD + EPI_VM) < 63 ? (DEPTH - 1) * (NLD + EPI_VM) : 63;
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) gload(d);
      vm_wait<kWHead>();
      lread(0, B0);
      int j = 0;
#pragma unroll
      for (; j < DEPTH - 1; ++j) {  // unrolled: B0 / B1 alternate with j
        if (j >= ntiles) break;
        gload((j + DEPTH) % NB);
        vm_wait<kWHead>();
        if (j % 2 == 0) {
          lread((j + 1) % NB, B1);
          tile(j, B0);
        } else {
          lread((j + 1) % NB, B0);
          tile(j, B1);
        }
      }
      if constexpr ((DEPTH - 1) % 2 == 0) {
        for (; j < ntiles; j += 2) {
          gload((j + DEPTH) % NB);
          vm_wait<kWFull>();
          lread((j + 1) % NB, B1);
          tile(j, B0);
          if (j + 1 >= ntiles) break;
          gload((j + 1 + DEPTH) % NB);
          vm_wait<kWFull>();
          lread((j + 2) % NB, B0);
          tile(j + 1, B1);
        }
      } else {
        for (; j < ntiles; j += 2) {
          gload((j + DEPTH) % NB);
          vm_wait<kWFull>();
          lread((j + 1) % NB, B0);
          tile(j, B1);
          if (j + 1 >= ntiles) break;
          gload((j + 1 + DEPTH) % NB);
          vm_wait<kWFull>();
          lread((j + 2) % NB, B1);
          tile(j + 1, B0);
        }
      }
    }
    vm_wait<0>();  // no load may land in the buffers after the wave moves on
  }
};

}  // namespace dsa
