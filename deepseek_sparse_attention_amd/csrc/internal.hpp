// Host-side launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace dsa {

// Indexer scores for rows [row0, row0 + nrows) of the Tq query rows of every sequence.
// Score row r (0 <= r < nrows) of sequence b is at scores + b*score_bstride + r*ld.
struct IndexerArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* w;
  const int32_t* kv_len;
  int B, Tq, Tk, H_I, d_I;
  int row0, nrows;
  float* scores;
  int64_t ld, score_bstride;
};
constexpr int64_t kIndexerMaxLd = int64_t(1) << 22;
bool indexer_supported(int H_I, int d_I, int64_t ld);
hipError_t launch_index_scores(const IndexerArgs& a, hipStream_t st);

// Top-k for rows [row0, row0 + nrows): score row r of sequence b at
// scores + b*score_bstride + r*ld; index row (row0 + r) of sequence b at
// idx + (b*Tq + row0 + r)*k.
struct TopkArgs {
  const float* scores;
  int64_t ld, score_bstride;
  const int32_t* kv_len;
  int B, Tq, Tk, k;
  int row0, nrows;
  int32_t* idx;
};
constexpr int kTopkMaxK = 4096;
constexpr int64_t kTopkMaxTk = int64_t(1) << 24;
hipError_t launch_topk(const TopkArgs& a, hipStream_t st);

struct AttnArgs {
  const uint16_t* q;
  const void* kv;
  const float* kv_scale;
  const uint16_t* v;
  bool fp8;
  const int32_t* idx;
  int B, Tq, Tk, H, Hkv, Dqk, Dv, k;
  float sm_scale;
  uint16_t* out;
  float* lse;
  void* ws;
};
// MLA form: Hkv = 1, Dqk = 576, Dv = 512, V shared with K, H % 16 == 0.
bool attn_mla_supported(const AttnArgs& a);
// Multi-head form: Hkv = H <= 16, Dqk = Dv = 32, separate V, bf16.
bool attn_mha_supported(const AttnArgs& a);
// Split-key factor the MLA kernel uses for this shape (1 = no partial results).
int attn_mla_splits(int B, int Tq, int H, int k);
size_t attn_workspace_bytes(int B, int Tq, int H, int Dv, int k, bool mla);
hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t st);

}  // namespace dsa
