// Indexer training objective on gfx950: KL divergence of the indexer's distribution from
// the detached main attention distribution, and its gradients with respect to the indexer
// inputs ("DSA ablation model card", model list: the indexer is trained with a KL loss
// against the main attention, held fixed, after a dense warm-up).  For query row t with
// key set S (its valid index entries; every causal key in the warm-up):
//
//   P_s = (1/H) sum_h softmax_s(sm_scale * q_h . K_{s,h})    target (multi-head attention)
//   Q_s = softmax_s(I_s),  I_s = sum_j w_j ReLU(q_j . k_s)     indexer distribution
//   loss_t = sum_s P_s (ln P_s - ln Q_s)
//   G_s = Q_s - P_s;  dw_j = sum_s G_s ReLU(d_js);  dq_j = sum_s G_s w_j [d_js > 0] k_s;
//   dk_s += sum_j G_s w_j [d_js > 0] q_j  (over all rows that list s),  d_js = q_j . k_s.
//
// One workgroup (256 threads) per query row.  Pass 1: for each main head in turn, and then
// for the indexer, each thread folds entries e, e+256, ... into an online (max, sum) in
// base 2 and the workgroup merges them.  Pass 2: recompute the logits, form P, Q, the loss
// and G, with G kept in LDS.  Pass 3, per chunk of 256 entries: a thread per entry stages
// its indexer key row in LDS, forms c_js = G_s w_j [d_js > 0] and keeps its share of dw;
// then threads own (head, dim) pairs of dq (or slices of them) and sum c_js k_s over the
// chunk from LDS.  Main-attention keys are re-read in pass 2 rather than kept: at 32 values
// per head they come back from L2.
//
// dk is a sum over the rows that list a key, so it is formed key-major, in a fixed order,
// and every output is bit-identical from run to run.  The row kernel stores each entry's
// c_j (and, for index lists, the entry's key); a stable LSD radix sort groups the sparse
// entries by key, keeping row order inside a key; one workgroup per key then adds its
// entries' c_j q_j in that order.  In the dense warm-up key s is entry s of every row at
// position >= s, so that pass walks the rows directly and needs no sort.
#include "common.hpp"
#include "internal.hpp"

namespace dsa {

namespace {

constexpr int kKlThreads = 256;
constexpr int kKlHeads = 16;   // main heads and indexer heads, at most
constexpr int kKlD = 32;       // main attention head width (multi-head form)
constexpr float kLog2eKl = 1.4426950408889634f;
constexpr float kLn2Kl = 0.6931471805599453f;

// (m, l) of two partial base-2 softmax sums, merged
__device__ __forceinline__ void ml_merge(float& m, float& l, float m2, float l2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  l = l * fast_exp2(m - mn) + l2 * fast_exp2(m2 - mn);
  m = mn;
}

__device__ __forceinline__ void wave_ml(float& m, float& l) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), l2 = __shfl_xor(l, o, 64);
    ml_merge(m, l, m2, l2);
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// NH: heads (main and indexer) the instance holds, MAXK: key entries per row; LDS is sized
// by both, so small shapes (the ablation: 4 + 2 heads, 512 keys) fit several workgroups
// per CU.
template <int D_I, int NH, int MAXK>
__global__ __launch_bounds__(kKlThreads) void indexer_kl_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx, const uint16_t* __restrict__ w_idx,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ kv_len, int Tq, int Tk, int H_I, int H, int kk, float scale_log2,
    float* __restrict__ loss, float* __restrict__ dq, float* __restrict__ dw, float* __restrict__ cw,
    int32_t* __restrict__ kw, int nkeys) {
  __shared__ float qf[NH][kKlD];           // main query, per head
  __shared__ float qif[NH][D_I];           // indexer query, per head
  __shared__ float wf[NH];
  __shared__ float gbuf[MAXK];             // I, then G, per entry
  __shared__ __attribute__((aligned(16))) uint16_t kchunk[kKlThreads][D_I];  // indexer key rows of a chunk
  __shared__ float cbuf[NH][kKlThreads];   // G w_j [d_j > 0] of a chunk's entries
  __shared__ float red[4][NH + 1][2];      // cross-wave (m, l) / sums
  __shared__ float lse2[NH + 1];           // base-2 log-sum-exp per head; [H]: indexer
  // small instances keep pass 1's logits for pass 2 instead of re-reading the keys
  constexpr bool kKeepZ = NH * MAXK <= 4096;
  __shared__ float zbuf[kKeepZ ? NH : 1][kKeepZ ? MAXK : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int64_t row = blockIdx.x;
  const int b = (int)(row / Tq), i = (int)(row % Tq);
  const int64_t L = seq_len(kv_len, b, Tk);
  const int64_t p = L - Tq + i;  // the query's position: it may attend keys 0..p
  const bool dense = idx == nullptr;
  const int n = dense ? (int)max<int64_t>(0, min<int64_t>(p + 1, Tk)) : kk;

  for (int x = tid; x < NH * kKlD; x += kKlThreads) {
    const int h = x / kKlD, d = x % kKlD;
    qf[h][d] = h < H ? bf16_bits_to_f32(q[(row * H + h) * kKlD + d]) : 0.f;
  }
  for (int x = tid; x < NH * D_I; x += kKlThreads) {
    const int j = x / D_I, d = x % D_I;
    qif[j][d] = j < H_I ? bf16_bits_to_f32(q_idx[(row * H_I + j) * D_I + d]) : 0.f;
  }
  if (tid < NH) wf[tid] = tid < H_I ? bf16_bits_to_f32(w_idx[row * H_I + tid]) : 0.f;
  __syncthreads();

  auto key_of = [&](int e) -> int {  // key of entry e, or -1
    if (dense) return e;
    const int s = idx[row * kk + e];
    return (s >= 0 && s < Tk) ? s : -1;
  };
  // base-2 logit of main head h (< H) for key s
  auto logit = [&](int s, int h) -> float {
    const uint16_t* kr = k + (((int64_t)b * Tk + s) * H + h) * kKlD;
    float dot = 0.f;
#pragma unroll
    for (int c = 0; c < kKlD / 8; ++c) {
      const u32x4 w4 = ld16(kr + c * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dot = fmaf(qf[h][c * 8 + 2 * e], __uint_as_float(w4[e] << 16), dot);
        dot = fmaf(qf[h][c * 8 + 2 * e + 1], __uint_as_float(w4[e] & 0xFFFF0000u), dot);
      }
    }
    return dot * scale_log2;
  };
  // this thread's indexer key row: loaded into its LDS slot, then read back per head
  auto stage_key = [&](int s) {
    const uint16_t* kp = k_idx + ((int64_t)b * Tk + s) * D_I;
#pragma unroll
    for (int c = 0; c < D_I / 8; ++c) *reinterpret_cast<u32x4*>(&kchunk[tid][c * 8]) = ld16(kp + c * 8);
  };
  auto index_dot = [&](int j) -> float {  // q_j . k_s for the staged row
    float dot = 0.f;
#pragma unroll
    for (int c = 0; c < D_I / 8; ++c) {
      const u32x4 w4 = *reinterpret_cast<const u32x4*>(&kchunk[tid][c * 8]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dot = fmaf(qif[j][c * 8 + 2 * e], __uint_as_float(w4[e] << 16), dot);
        dot = fmaf(qif[j][c * 8 + 2 * e + 1], __uint_as_float(w4[e] & 0xFFFF0000u), dot);
      }
    }
    return dot;
  };

  // ---- pass 1: softmax statistics of each main head's logits (one head at a time), then
  // of the indexer scores (kept in gbuf)
  for (int h = 0; h < H; ++h) {
    float mh = -INFINITY, lh = 0.f;
    for (int e = tid; e < n; e += kKlThreads) {
      const int s = key_of(e);
      if (s >= 0) {
        const float z = logit(s, h);
        if constexpr (kKeepZ) zbuf[h][e] = z;
        ml_merge(mh, lh, z, 1.f);
      }
    }
    wave_ml(mh, lh);
    if (lane == 0) red[wave][h][0] = mh, red[wave][h][1] = lh;
  }
  {
    float mi = -INFINITY, li = 0.f;
    for (int e = tid; e < n; e += kKlThreads) {
      const int s = key_of(e);
      float iv = -INFINITY;
      if (s >= 0) {
        stage_key(s);
        float tot = 0.f;
        for (int j = 0; j < H_I; ++j) tot = fmaf(wf[j], relu(index_dot(j)), tot);
        iv = tot;
        ml_merge(mi, li, tot * kLog2eKl, 1.f);
      }
      gbuf[e] = iv;
    }
    wave_ml(mi, li);
    if (lane == 0) red[wave][NH][0] = mi, red[wave][NH][1] = li;
  }
  __syncthreads();
  if (tid < H || tid == NH) {
    float mm = red[0][tid][0], ll = red[0][tid][1];
    for (int w = 1; w < 4; ++w) ml_merge(mm, ll, red[w][tid][0], red[w][tid][1]);
    lse2[tid] = ll > 0.f ? mm + __log2f(ll) : -INFINITY;
  }
  __syncthreads();

  // ---- pass 2: P, Q, the loss and G = Q - P
  float part = 0.f;
  const float inv_h = 1.f / (float)H;
  for (int e = tid; e < n; e += kKlThreads) {
    const int s = key_of(e);
    float g = 0.f;
    if (s >= 0) {
      float pe = 0.f;
      for (int h = 0; h < H; ++h) {
        float z;
        if constexpr (kKeepZ)
          z = zbuf[h][e];  // written by this thread in pass 1
        else
          z = logit(s, h);
        pe += fast_exp2(z - lse2[h]);
      }
      pe *= inv_h;
      const float lq2 = gbuf[e] * kLog2eKl - lse2[NH];  // log2 Q_s
      if (pe > 0.f) part += pe * (__log2f(pe) - lq2);
      g = fast_exp2(lq2) - pe;
    }
    gbuf[e] = g;
  }
  part = wave_sum(part);
  __syncthreads();  // (red is reused)
  if (lane == 0) red[wave][0][0] = part;
  __syncthreads();
  if (tid == 0) loss[row] = ((red[0][0][0] + red[1][0][0]) + (red[2][0][0] + red[3][0][0])) * kLn2Kl;
  if (!dq && !dw && !cw) return;

  // ---- pass 3: gradients of the indexer inputs, 256 entries per chunk.  Entry thread:
  // cbuf[j] = G w_j [d_j > 0], its own share of dw (G ReLU(d_j)) and, for dk, its c_j (and
  // key) stored for the key-major pass; then the dq pairs (head, dim) sum c_j k over the
  // chunk from LDS, split into S entry slices per pair when the pairs are fewer than the
  // threads (slices combined at the end in slice order).
  constexpr int kPairs = (NH * D_I + kKlThreads - 1) / kKlThreads;
  const int P = H_I * D_I;
  const int S = P <= kKlThreads ? kKlThreads / P : 0;  // entry slices per dq pair
  float dq_acc[kPairs];
#pragma unroll
  for (int r = 0; r < kPairs; ++r) dq_acc[r] = 0.f;
  float dw_part[NH];
#pragma unroll
  for (int j = 0; j < NH; ++j) dw_part[j] = 0.f;
  for (int c0 = 0; c0 < n; c0 += kKlThreads) {
    const int e = c0 + tid;
    const int s = e < n ? key_of(e) : -1;
    if (s >= 0) {
      stage_key(s);
      const float g = gbuf[e];
      bool any = false;
#pragma unroll
      for (int j = 0; j < NH; ++j) {
        float c = 0.f;
        if (j < H_I) {
          const float d = index_dot(j);
          c = d > 0.f ? g * wf[j] : 0.f;
          dw_part[j] = fmaf(g, relu(d), dw_part[j]);
        }
        cbuf[j][tid] = c;
        any |= c != 0.f;
      }
      if (cw) {
        // dense rows keep every causal entry (the key pass reads them by position); index
        // lists keep the entries that add to dk, the rest take the key past every real one
        const int64_t f = dense ? row * Tk + e : row * kk + e;
        if (dense || any) {
          for (int j = 0; j < H_I; ++j) cw[f * H_I + j] = cbuf[j][tid];
        }
        if (!dense) kw[f] = any ? b * Tk + s : nkeys;
      }
    } else {
      if (cw && !dense && e < n) kw[row * kk + e] = nkeys;
#pragma unroll
      for (int j = 0; j < NH; ++j) cbuf[j][tid] = 0.f;
#pragma unroll
      for (int c = 0; c < D_I / 8; ++c) *reinterpret_cast<u32x4*>(&kchunk[tid][c * 8]) = u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
    const int cn = min(kKlThreads, n - c0);
    if (dq) {
      if (S > 0) {
        if (tid < P * S) {
          const int pr = tid % P, sl = tid / P;
          const int j = pr / D_I, d = pr % D_I;
          float acc = dq_acc[0];
          for (int t = sl; t < cn; t += S) acc = fmaf(cbuf[j][t], bf16_bits_to_f32(kchunk[t][d]), acc);
          dq_acc[0] = acc;
        }
      } else {
#pragma unroll
        for (int r = 0; r < kPairs; ++r) {
          const int x = tid + r * kKlThreads;
          const int j = x / D_I, d = x % D_I;
          if (j < H_I) {
            float acc = dq_acc[r];
            for (int t = 0; t < cn; ++t) acc = fmaf(cbuf[j][t], bf16_bits_to_f32(kchunk[t][d]), acc);
            dq_acc[r] = acc;
          }
        }
      }
    }
    __syncthreads();  // the chunk buffers are refilled
  }
  if (dq) {
    if (S > 0) {
      float* part = &cbuf[0][0];  // free now: the slices' partial sums, slice-major
      part[tid] = tid < P * S ? dq_acc[0] : 0.f;
      __syncthreads();
      if (tid < P) {
        float v = part[tid];
        for (int sl = 1; sl < S; ++sl) v += part[sl * P + tid];
        dq[row * P + tid] = v;
      }
    } else {
#pragma unroll
      for (int r = 0; r < kPairs; ++r) {
        const int x = tid + r * kKlThreads;
        if (x / D_I < H_I) dq[row * P + x] = dq_acc[r];
      }
    }
  }
  if (dw) {
    __syncthreads();  // red held the loss partials (and no chunk ran for an empty row)
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      const float v = wave_sum(dw_part[j]);
      if (lane == 0) red[wave][j][0] = v;
    }
    __syncthreads();
    if (tid < H_I) dw[row * H_I + tid] = (red[0][tid][0] + red[1][tid][0]) + (red[2][tid][0] + red[3][tid][0]);
  }
}

// ---- stable LSD radix sort of (key, entry) pairs, a few bits of the key per pass ----
// A tile is 2048 pairs: 8 rounds of 256, round-major, so round r thread t holds pair
// tile * 2048 + r * 256 + t and the input order inside a tile is (round, wave, lane).

constexpr int kSortItems = 8;
constexpr int kSortTile = 256 * kSortItems;
constexpr int kScanItems = 16;
constexpr int kScanBlock = 256 * kScanItems;

// exclusive scan over the workgroup (NT threads, NT / 64 waves); *total gets the sum
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* total) {
  __shared__ int wsum[NT / 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const int sw = wsum[i];
    off += i < w ? sw : 0;
    tot += sw;
  }
  __syncthreads();  // wsum is reused by the next call
  *total = tot;
  return off + x - v;
}

// per tile, how many of its pairs fall in each digit; stored digit-major, so one flat
// exclusive scan of hist gives every (digit, tile) its first output slot
__global__ __launch_bounds__(256) void sort_hist_kernel(const int32_t* __restrict__ keys, int64_t n, int shift,
                                                        int mask, int ntiles, int32_t* __restrict__ hist) {
  __shared__ int cnt[256];
  const int tid = threadIdx.x, tile = blockIdx.x;
  cnt[tid] = 0;
  __syncthreads();
  const int64_t base = (int64_t)tile * kSortTile;
#pragma unroll
  for (int r = 0; r < kSortItems; ++r) {
    const int64_t i = base + r * 256 + tid;
    if (i < n) atomicAdd(&cnt[(keys[i] >> shift) & mask], 1);  // integer counts: order-free
  }
  __syncthreads();
  if (tid <= mask) hist[(int64_t)tid * ntiles + tile] = cnt[tid];
}

// exclusive scan of x[0, n) in three launches: block sums, a scan of the sums, then each
// block's own scan from its offset
__global__ __launch_bounds__(256) void scan_sums_kernel(const int32_t* __restrict__ x, int64_t n,
                                                        int32_t* __restrict__ bsum) {
  const int64_t base = (int64_t)blockIdx.x * kScanBlock;
  int v = 0;
#pragma unroll
  for (int r = 0; r < kScanItems; ++r) {
    const int64_t i = base + r * 256 + threadIdx.x;
    if (i < n) v += x[i];
  }
  int tot;
  block_exclusive_scan<256>(v, &tot);
  if (threadIdx.x == 0) bsum[blockIdx.x] = tot;
}

__global__ __launch_bounds__(1024) void scan_block_sums_kernel(int32_t* __restrict__ bsum, int nb) {
  int carry = 0;
  for (int b0 = 0; b0 < nb; b0 += 1024) {
    const int i = b0 + (int)threadIdx.x;
    const int v = i < nb ? bsum[i] : 0;
    int tot;
    const int ex = block_exclusive_scan<1024>(v, &tot);
    if (i < nb) bsum[i] = carry + ex;
    carry += tot;
  }
}

// OWN_OFFSET: bsum holds the raw block sums and each block adds up those before its own
// (few blocks); otherwise bsum is already scanned
template <bool OWN_OFFSET>
__global__ __launch_bounds__(256) void scan_apply_kernel(int32_t* __restrict__ x, int64_t n,
                                                         const int32_t* __restrict__ bsum) {
  int boff;
  if constexpr (OWN_OFFSET) {
    int part = 0;
    for (int i = (int)threadIdx.x; i < (int)blockIdx.x; i += 256) part += bsum[i];
    int tot;
    block_exclusive_scan<256>(part, &tot);
    boff = tot;
  } else {
    boff = bsum[blockIdx.x];
  }
  // thread t scans items base + 16 t .. base + 16 t + 15 in order
  const int64_t base = (int64_t)blockIdx.x * kScanBlock + (int64_t)threadIdx.x * kScanItems;
  int v[kScanItems];
  int sum = 0;
#pragma unroll
  for (int r = 0; r < kScanItems; ++r) {
    v[r] = base + r < n ? x[base + r] : 0;
    sum += v[r];
  }
  int tot;
  int run = boff + block_exclusive_scan<256>(sum, &tot);
#pragma unroll
  for (int r = 0; r < kScanItems; ++r) {
    if (base + r < n) x[base + r] = run;
    run += v[r];
  }
}

// each pair to its slot: the tile's first slot for its digit, plus the pairs of that digit
// before it in the tile (earlier rounds, earlier waves of this round, lower lanes of its
// wave): equal digits keep their input order, so every pass is stable
__global__ __launch_bounds__(256) void sort_scatter_kernel(const int32_t* __restrict__ kin,
                                                           const int32_t* __restrict__ vin, int64_t n, int shift,
                                                           int bits, int ntiles, const int32_t* __restrict__ off,
                                                           int32_t* __restrict__ kout, int32_t* __restrict__ vout) {
  __shared__ int next[256];     // next free slot of each digit
  __shared__ int wcnt[4][256];  // pairs of each digit in each wave of the round
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, tile = blockIdx.x;
  const int mask = (1 << bits) - 1;
  if (tid <= mask) next[tid] = off[(int64_t)tid * ntiles + tile];
  const uint64_t below = (uint64_t(1) << lane) - 1;
  for (int r = 0; r < kSortItems; ++r) {
    const int64_t i = (int64_t)tile * kSortTile + r * 256 + tid;
    const bool valid = i < n;
    const int key = valid ? kin[i] : 0;
    const int val = valid ? (vin ? vin[i] : (int)i) : 0;
    const int d = (key >> shift) & mask;
    for (int x = tid; x < 4 * 256; x += 256) wcnt[x >> 8][x & 255] = 0;
    __syncthreads();
    // lanes of this wave with the same digit
    uint64_t peers = __ballot(valid);
    for (int bt = 0; bt < bits; ++bt) {
      const bool set = (d >> bt) & 1;
      const uint64_t bb = __ballot(set);
      peers &= set ? bb : ~bb;
    }
    const int rank = __popcll(peers & below);
    if (valid && rank == 0) wcnt[wave][d] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int pos = next[d] + rank;
      for (int w2 = 0; w2 < wave; ++w2) pos += wcnt[w2][d];
      kout[pos] = key;
      vout[pos] = val;
    }
    __syncthreads();
    if (tid <= mask) next[tid] += (wcnt[0][tid] + wcnt[1][tid]) + (wcnt[2][tid] + wcnt[3][tid]);
    __syncthreads();
  }
}

// start[K] = first slot of the sorted keys holding a key >= K, for K = 0 .. nkeys (the
// sentinel nkeys marks the entries that add nothing): each boundary slot fills the keys
// between its neighbours
__global__ __launch_bounds__(256) void key_starts_kernel(const int32_t* __restrict__ keys, int64_t n, int nkeys,
                                                         int32_t* __restrict__ start) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i > n) return;
  const int prev = i == 0 ? -1 : keys[i - 1];
  const int cur = i == n ? nkeys + 1 : keys[i];
  for (int K = prev + 1; K <= min(cur, nkeys); ++K) start[K] = (int32_t)i;
}

// dk[K] = sum over the entries of key K, in order, of sum_j c_j q_j: one wave per key.  A
// lane owns 16 dims of one entry slot (D_I / 16 lanes per entry, NSLOT = 64 / (D_I / 16)
// slots); slot u takes entries u, u + NSLOT, ... (heads in order inside an entry), and the
// slots are then added by an xor butterfly, so every addition happens in a fixed order.
// DENSE: the entries of key s are the rows at position >= s.
template <int D_I, bool DENSE>
__global__ __launch_bounds__(256) void kl_dk_kernel(const float* __restrict__ cw, const int32_t* __restrict__ start,
                                                    const int32_t* __restrict__ sval, const uint16_t* __restrict__ q_idx,
                                                    const int32_t* __restrict__ kv_len, int Tq, int Tk, int H_I,
                                                    int kk, int nkeys, float* __restrict__ dk) {
  constexpr int DG = D_I / 16, NSLOT = 64 / DG;
  const int lane = threadIdx.x & 63;
  const int64_t K = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (K >= nkeys) return;  // a whole wave; no workgroup barrier follows
  const int slot = lane / DG, g = lane % DG;
  const int b = (int)(K / Tk), s = (int)(K % Tk);
  int64_t lo, hi;
  if constexpr (DENSE) {
    const int64_t L = seq_len(kv_len, b, Tk);
    lo = max<int64_t>(0, s - (L - Tq));  // first row whose position L - Tq + t reaches s
    hi = s < L ? Tq : lo;
  } else {
    lo = start[K];
    hi = start[K + 1];
  }
  float acc[16];
#pragma unroll
  for (int x = 0; x < 16; ++x) acc[x] = 0.f;
#pragma unroll 2
  for (int64_t i = lo + slot; i < hi; i += NSLOT) {
    int64_t f, row;
    if constexpr (DENSE) {
      row = (int64_t)b * Tq + i;
      f = row * Tk + s;
    } else {
      const int fi = sval[i];  // entries < 2^31
      f = fi;
      row = fi / kk;
    }
    const float* c = cw + f * H_I;
    const uint16_t* qr = q_idx + row * H_I * D_I + g * 16;
    for (int j = 0; j < H_I; ++j) {
      const float cj = c[j];
      const u32x4 lo4 = ld16(qr + j * D_I), hi4 = ld16(qr + j * D_I + 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] = fmaf(cj, __uint_as_float(lo4[e] << 16), acc[2 * e]);
        acc[2 * e + 1] = fmaf(cj, __uint_as_float(lo4[e] & 0xFFFF0000u), acc[2 * e + 1]);
        acc[8 + 2 * e] = fmaf(cj, __uint_as_float(hi4[e] << 16), acc[8 + 2 * e]);
        acc[8 + 2 * e + 1] = fmaf(cj, __uint_as_float(hi4[e] & 0xFFFF0000u), acc[8 + 2 * e + 1]);
      }
    }
  }
#pragma unroll
  for (int o = DG; o < 64; o <<= 1) {
#pragma unroll
    for (int x = 0; x < 16; ++x) acc[x] += __shfl_xor(acc[x], o, 64);
  }
  if (slot == 0) {  // dk is only 4-byte aligned
#pragma unroll
    for (int x = 0; x < 16; ++x) dk[K * D_I + g * 16 + x] = acc[x];
  }
}

// workspace of the dk pass, carved in this order (each piece 256-byte aligned)
struct KlDkPlan {
  int64_t entries;  // stored entries: rows * kk, or rows * Tk for the dense warm-up
  int nkeys;        // B * Tk; also the sentinel key
  int64_t ntiles, nhist, nscan_blocks;
  int passes, bits_per_pass, key_bits;
  size_t c_off, ka_off, va_off, kb_off, vb_off, hist_off, bsum_off, start_off, bytes;
};

size_t kl_align(size_t x) { return (x + 255) / 256 * 256; }

KlDkPlan plan_kl_dk(int B, int Tq, int Tk, int H_I, int kk, bool dense) {
  KlDkPlan P{};
  const int64_t rows = (int64_t)std::max(0, B) * std::max(0, Tq);
  P.nkeys = (int)std::min<int64_t>((int64_t)std::max(0, B) * std::max(0, Tk), INT32_MAX);
  P.entries = rows * (dense ? std::max(0, Tk) : std::max(0, kk));
  size_t o = 0;
  P.c_off = o;
  o += kl_align((size_t)P.entries * H_I * 4);
  if (!dense) {
    P.key_bits = 1;
    while ((int64_t(1) << P.key_bits) <= P.nkeys) ++P.key_bits;  // keys 0 .. nkeys (the sentinel)
    P.passes = (P.key_bits + 7) / 8;
    P.bits_per_pass = (P.key_bits + P.passes - 1) / P.passes;
    P.ntiles = (P.entries + kSortTile - 1) / kSortTile;
    P.nhist = (int64_t(1) << P.bits_per_pass) * P.ntiles;
    P.nscan_blocks = (P.nhist + kScanBlock - 1) / kScanBlock;
    const size_t pairs = kl_align((size_t)P.entries * 4);
    P.ka_off = o;
    P.va_off = o + pairs;
    P.kb_off = o + 2 * pairs;
    P.vb_off = o + 3 * pairs;
    o += 4 * pairs;
    P.hist_off = o;
    o += kl_align((size_t)P.nhist * 4);
    P.bsum_off = o;
    o += kl_align((size_t)P.nscan_blocks * 4);
    P.start_off = o;
    o += kl_align(((size_t)P.nkeys + 1) * 4);
  }
  P.bytes = o;
  return P;
}

hipError_t scan_exclusive(int32_t* x, int64_t n, int32_t* bsum, int64_t nb, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(scan_sums_kernel, dim3((unsigned)nb), dim3(256), 0, st, x, n, bsum);
  if (nb <= 1024) {  // each block adds up the sums before it
    hipLaunchKernelGGL(scan_apply_kernel<true>, dim3((unsigned)nb), dim3(256), 0, st, x, n, bsum);
  } else {
    hipLaunchKernelGGL(scan_block_sums_kernel, dim3(1), dim3(1024), 0, st, bsum, (int)nb);
    hipLaunchKernelGGL(scan_apply_kernel<false>, dim3((unsigned)nb), dim3(256), 0, st, x, n, bsum);
  }
  return hipGetLastError();
}

}  // namespace

bool indexer_kl_supported(int H_I, int d_I, int H, int Hkv, int Dqk) {
  return H_I >= 1 && H_I <= kKlHeads && (d_I == 16 || d_I == 32 || d_I == 64 || d_I == 128) && H >= 1 &&
         H <= kKlHeads && Hkv == H && Dqk == kKlD;
}

size_t indexer_kl_workspace_bytes(int B, int Tq, int Tk, int H_I, int kk, bool dense) {
  return plan_kl_dk(B, Tq, Tk, H_I, kk, dense).bytes;
}

hipError_t launch_indexer_kl(const IndexerKlArgs& a, void* ws, hipStream_t st) {
  const int64_t rows = (int64_t)a.B * a.Tq;
  const bool dense = a.idx == nullptr;
  const KlDkPlan P = plan_kl_dk(a.B, a.Tq, a.Tk, a.H_I, a.kk, dense);
  char* wsb = static_cast<char*>(ws);
  float* cw = a.dk ? reinterpret_cast<float*>(wsb + P.c_off) : nullptr;
  int32_t* keys = a.dk && !dense ? reinterpret_cast<int32_t*>(wsb + P.ka_off) : nullptr;
  if (rows > 0) {
    const float sl2 = a.sm_scale * kLog2eKl;
    const bool few_heads = a.H <= 4 && a.H_I <= 4;
    const bool few_keys = (a.idx ? a.kk : a.Tk) <= 1024;
#define DSA_KL_LAUNCH(DI, NH, MK)                                                                                \
  hipLaunchKernelGGL((indexer_kl_kernel<DI, NH, MK>), dim3((unsigned)rows), dim3(kKlThreads), 0, st, a.q_idx,     \
                     a.k_idx, a.w_idx, a.q, a.k, a.idx, a.kv_len, a.Tq, a.Tk, a.H_I, a.H, a.kk, sl2, a.loss, a.dq, \
                     a.dw, cw, keys, P.nkeys)
#define DSA_KL_SIZES(DI)                                  \
  if (few_heads && few_keys) DSA_KL_LAUNCH(DI, 4, 1024);  \
  else if (few_heads) DSA_KL_LAUNCH(DI, 4, kKlMaxKeys);   \
  else if (few_keys) DSA_KL_LAUNCH(DI, kKlHeads, 1024);   \
  else DSA_KL_LAUNCH(DI, kKlHeads, kKlMaxKeys);
    switch (a.d_I) {
      case 16: DSA_KL_SIZES(16); break;
      case 32: DSA_KL_SIZES(32); break;
      case 64: DSA_KL_SIZES(64); break;
      case 128: DSA_KL_SIZES(128); break;
      default: return hipErrorInvalidValue;
    }
#undef DSA_KL_SIZES
#undef DSA_KL_LAUNCH
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!a.dk || P.nkeys == 0) return hipSuccess;

  // ---- dk, key-major
  const int32_t* start = nullptr;
  const int32_t* sval = nullptr;
  if (!dense) {
    int32_t* kin = keys;
    int32_t* vin = nullptr;  // first pass: the entry number is the pair's input position
    int32_t* kout = reinterpret_cast<int32_t*>(wsb + P.kb_off);
    int32_t* vout = reinterpret_cast<int32_t*>(wsb + P.vb_off);
    int32_t* spare_v = reinterpret_cast<int32_t*>(wsb + P.va_off);
    int32_t* hist = reinterpret_cast<int32_t*>(wsb + P.hist_off);
    int32_t* bsum = reinterpret_cast<int32_t*>(wsb + P.bsum_off);
    for (int p = 0; p < P.passes && P.entries > 0; ++p) {
      const int shift = p * P.bits_per_pass;
      const int bits = std::min(P.bits_per_pass, P.key_bits - shift);
      const int mask = (1 << bits) - 1;
      const int64_t nhist = (int64_t(mask) + 1) * P.ntiles;
      hipLaunchKernelGGL(sort_hist_kernel, dim3((unsigned)P.ntiles), dim3(256), 0, st, kin, P.entries, shift, mask,
                         (int)P.ntiles, hist);
      hipError_t e = scan_exclusive(hist, nhist, bsum, (nhist + kScanBlock - 1) / kScanBlock, st);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(sort_scatter_kernel, dim3((unsigned)P.ntiles), dim3(256), 0, st, kin, vin, P.entries,
                         shift, bits, (int)P.ntiles, hist, kout, vout);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      int32_t* nk = kin;  // ping-pong: the next pass reads what this one wrote
      int32_t* nv = vin ? vin : spare_v;
      kin = kout;
      vin = vout;
      kout = nk;
      vout = nv;
    }
    int32_t* st_arr = reinterpret_cast<int32_t*>(wsb + P.start_off);
    hipLaunchKernelGGL(key_starts_kernel, dim3((unsigned)((P.entries + 1 + 255) / 256)), dim3(256), 0, st, kin,
                       P.entries, P.nkeys, st_arr);
    start = st_arr;
    sval = vin;
  }
#define DSA_KL_DK(DI)                                                                                             \
  if (dense)                                                                                                      \
    hipLaunchKernelGGL((kl_dk_kernel<DI, true>), dim3((unsigned)((P.nkeys + 3) / 4)), dim3(256), 0, st, cw,     \
                       start, sval, a.q_idx, a.kv_len, a.Tq, a.Tk, a.H_I, a.kk, P.nkeys, a.dk);                   \
  else                                                                                                            \
    hipLaunchKernelGGL((kl_dk_kernel<DI, false>), dim3((unsigned)((P.nkeys + 3) / 4)), dim3(256), 0, st, cw,    \
                       start, sval, a.q_idx, a.kv_len, a.Tq, a.Tk, a.H_I, a.kk, P.nkeys, a.dk);
  switch (a.d_I) {
    case 16: DSA_KL_DK(16); break;
    case 32: DSA_KL_DK(32); break;
    case 64: DSA_KL_DK(64); break;
    case 128: DSA_KL_DK(128); break;
    default: return hipErrorInvalidValue;
  }
#undef DSA_KL_DK
  return hipGetLastError();
}

}  // namespace dsa
