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
// base 2 and the workgroup merges them.  Pass 2: recompute the logits, form P, Q, the loss and G, with G kept in
// LDS.  Pass 3, per chunk of 256 entries: a thread per entry stages its indexer key row in
// LDS, forms c_js = G_s w_j [d_js > 0] and keeps its share of dw; then threads own (head,
// dim) pairs of dq (or slices of them) and sum c_js k_s over the chunk from LDS, and
// (entry, dim) pairs add the dk rows with fp32 atomics (rows that share a key add in no
// fixed order; every other sum runs in a fixed order: loss, dq and dw are deterministic).  Main-attention keys are re-read in pass 2
// rather than kept: at 32 values per head they come back from L2.
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
    float* __restrict__ loss, float* __restrict__ dq, float* __restrict__ dw, float* __restrict__ dk) {
  __shared__ float qf[NH][kKlD];           // main query, per head
  __shared__ float qif[NH][D_I];           // indexer query, per head
  __shared__ float wf[NH];
  __shared__ float gbuf[MAXK];             // I, then G, per entry
  __shared__ __attribute__((aligned(16))) uint16_t kchunk[kKlThreads][D_I];  // indexer key rows of a chunk
  __shared__ float cbuf[NH][kKlThreads];   // G w_j [d_j > 0] of a chunk's entries
  __shared__ int ckey[kKlThreads];               // a chunk entry's key, -1 if it adds nothing to dk
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
  if (!dq && !dw && !dk) return;

  // ---- pass 3: gradients of the indexer inputs, 256 entries per chunk.  Entry thread:
  // cbuf[j] = G w_j [d_j > 0] and its own share of dw (G ReLU(d_j)); then the dq pairs
  // (head, dim) sum c_j k over the chunk from LDS, split into S entry slices per pair when
  // the pairs are fewer than the threads (slices combined at the end in slice order), and
  // (entry, dim) pairs add the dk rows with fp32 atomics.
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
      ckey[tid] = any ? s : -1;
    } else {
      ckey[tid] = -1;
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
    if (dk) {
      // (entry, dim) pairs: consecutive lanes add consecutive dims of one key row, so an
      // atomic instruction covers 64 / D_I rows instead of 64
      for (int x = tid; x < cn * D_I; x += kKlThreads) {
        const int t = x / D_I, d = x % D_I;
        const int key = ckey[t];
        if (key < 0) continue;
        float acc = 0.f;
        for (int j = 0; j < H_I; ++j) acc = fmaf(cbuf[j][t], qif[j][d], acc);
        unsafeAtomicAdd(dk + ((int64_t)b * Tk + key) * D_I + d, acc);
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

__global__ __launch_bounds__(256) void zero_f32_kernel(float* __restrict__ x, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) x[i] = 0.f;
}

}  // namespace

bool indexer_kl_supported(int H_I, int d_I, int H, int Hkv, int Dqk) {
  return H_I >= 1 && H_I <= kKlHeads && (d_I == 16 || d_I == 32 || d_I == 64 || d_I == 128) && H >= 1 &&
         H <= kKlHeads && Hkv == H && Dqk == kKlD;
}

hipError_t launch_indexer_kl(const IndexerKlArgs& a, hipStream_t st) {
  const int64_t rows = (int64_t)a.B * a.Tq;
  if (a.dk && (int64_t)a.B * a.Tk * a.d_I > 0) {
    const int64_t nk = (int64_t)a.B * a.Tk * a.d_I;
    hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)((nk + 255) / 256)), dim3(256), 0, st, a.dk, nk);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (rows == 0) return hipSuccess;
  const float sl2 = a.sm_scale * kLog2eKl;
  const bool few_heads = a.H <= 4 && a.H_I <= 4;
  const bool few_keys = (a.idx ? a.kk : a.Tk) <= 1024;
#define DSA_KL_LAUNCH(DI, NH, MK)                                                                                \
  hipLaunchKernelGGL((indexer_kl_kernel<DI, NH, MK>), dim3((unsigned)rows), dim3(kKlThreads), 0, st, a.q_idx,     \
                     a.k_idx, a.w_idx, a.q, a.k, a.idx, a.kv_len, a.Tq, a.Tk, a.H_I, a.H, a.kk, sl2, a.loss, a.dq, \
                     a.dw, a.dk)
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
  return hipGetLastError();
}

}  // namespace dsa
