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
  // paged keys (block_table != nullptr): key s of sequence b is row
  // block_table[b*max_blocks + s >> page_shift] << page_shift | (s & (page - 1)) of the pool k
  const int32_t* block_table = nullptr;
  int max_blocks = 0, page_shift = 0;
  int64_t pool_tokens = 0;
  // optional: the split top-k's workspace (topk_split_workspace_bytes of B, nrows, Tk,
  // topk_k) for a launch whose rows take that route; a launch of one query row per
  // sequence that holds its scores in LDS then also builds the segment lists there and sets
  // *lists_made (else leaves it false)
  void* topk_ws = nullptr;
  int topk_k = 0;
  bool* lists_made = nullptr;
};
constexpr int64_t kIndexerMaxLd = int64_t(1) << 22;
bool indexer_supported(int H_I, int d_I, int64_t ld);
hipError_t launch_index_scores(const IndexerArgs& a, hipStream_t st);
// -inf into entries p+1 .. ld-1 of each score row (row r of sequence b at
// scores + b*score_bstride + r*ld, query position p = kv_len[b] - Tq + r).
hipError_t launch_fill_masked(float* scores, int64_t ld, int64_t score_bstride, const int32_t* kv_len, int B, int Tq,
                              int Tk, hipStream_t st);

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
  // optional workspace of topk_split_workspace_bytes(): few long rows then split each row
  // over the chip (segment lists, then a merge per row); null keeps one workgroup per row
  void* ws = nullptr;
  // the segment lists in ws were built by the launch that wrote the scores (the decode
  // indexer): only the merge runs; only with the split route
  bool lists_ready = false;
};
size_t topk_split_workspace_bytes(int B, int nrows, int Tk, int k);
// Whether launch_topk splits A's rows over the chip (segment lists in A.ws, then a merge).
bool topk_split_route(const TopkArgs& A);
constexpr int kTopkMaxK = 4096;
constexpr int64_t kTopkMaxTk = int64_t(1) << 24;
hipError_t launch_topk(const TopkArgs& a, hipStream_t st);

// Fused indexer -> top-k for rows [row0, row0 + nrows): the indices of index_scores + topk
// without the score rows.  Workspace: fused_layout(B, nrows, Tk).bytes.
constexpr int kFusedCap = 6144;             // candidate entries per row
constexpr int kFusedMaxSampleTiles = 128;   // sampled 32-key tiles per row, at most
constexpr int kFusedMaxK = 4096;
// Sampled tiles for a row that sees `span` keys: about one key in 16.
__host__ __device__ inline int fz_sample_tiles(int64_t span) {
  const int64_t t = span / 512;
  return (int)(t < 1 ? 1 : (t > kFusedMaxSampleTiles ? kFusedMaxSampleTiles : t));
}
// Expected candidates per row as a multiple of k: ~3400 of the 6144 slots at k = 2048.
__host__ __device__ inline float fused_default_alpha(int k) {
  const float a = 0.55f * (float)kFusedCap / (float)(k < 1 ? 1 : k);
  return a < 1.25f ? 1.25f : (a > 4.f ? 4.f : a);
}
struct IndexTopkArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* w;
  const int32_t* kv_len;
  int B, Tq, Tk, H_I, d_I, k_top;
  int row0, nrows;
  float oversample;  // expected candidates per row / k; <= 0: fused_default_alpha
  int32_t* idx;      // [B][Tq][k_top]
  void* ws;
};
struct FusedLayout {
  size_t smp, ns, thr, cnt, list, bytes;  // byte offsets in the workspace, total
  int smax;                               // sample slots per row
};
FusedLayout fused_layout(int B, int nrows, int Tk);
bool index_topk_fused_supported(int H_I, int d_I, int k);
hipError_t launch_index_topk(const IndexTopkArgs& a, hipStream_t st);

// Indexer KL objective (multi-head main attention): one row of the loss and the gradients
// of the indexer inputs.  idx == nullptr: every causal key (dense warm-up).  dq, dw, dk
// may each be null (not computed); dk is cleared and then accumulated.
struct IndexerKlArgs {
  const uint16_t *q_idx, *k_idx, *w_idx, *q, *k;
  const int32_t *idx, *kv_len;
  int B, Tq, Tk, H_I, d_I, H, kk;
  float sm_scale;
  float *loss, *dq, *dw, *dk;
};
constexpr int kKlMaxKeys = 4096;  // key entries per row
bool indexer_kl_supported(int H_I, int d_I, int H, int Hkv, int Dqk);
// workspace of the key-major dk pass (rows * entries coefficients, plus the key sort for
// index lists); none is needed without dk
size_t indexer_kl_workspace_bytes(int B, int Tq, int Tk, int H_I, int kk, bool dense);
hipError_t launch_indexer_kl(const IndexerKlArgs& a, void* ws, hipStream_t st);

struct AttnArgs {
  const uint16_t* q;
  const void* kv;
  const float* kv_scale;
  const uint16_t* v;
  int kv_fmt;  // latent rows: 0 bf16, 1 fp8 e4m3 + per-token scale, 2 MXFP4 (320-byte rows)
  const int32_t* idx;
  int B, Tq, Tk, H, Hkv, Dqk, Dv, k;
  float sm_scale;
  uint16_t* out;
  float* lse;
  void* ws;
  // rows between two sequences' first rows: -1 for Tk (dense [B][Tk] caches), 0 for one
  // pool shared by all sequences (paged caches: idx then holds pool rows, Tk the pool size)
  int64_t kv_bstride = -1;
  // tail_Tk > 0: idx rows are the library's own top-k output (valid entries first, then -1
  // padding) for sequences of tail_kv_len[b] (NULL: tail_Tk) keys
  const int32_t* tail_kv_len = nullptr;
  int tail_Tk = 0;
};
// MLA form: Hkv = 1, Dqk = 576, Dv = 512, V shared with K, H % 16 == 0.
bool attn_mla_supported(const AttnArgs& a);
// Multi-head form: Hkv = H <= 16, Dqk = Dv = 32, separate V, bf16.
bool attn_mha_supported(const AttnArgs& a);
// Split-key factor the MLA kernel uses for this shape in a launch of nlayers layers (1 = no
// partial results); never more than for one layer, whose count sizes the workspace.
int attn_mla_splits(int B, int Tq, int H, int k, int nlayers = 1);
// Compute units of the current device (cached per device; 256 on MI355X).
int device_cus();
size_t attn_workspace_bytes(int B, int Tq, int H, int Dv, int k, bool mla);
hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t st);
// Layers that share a's index list and shape in one launch (MLA form; at most
// kMaxAttnLayers): layer z reads layers[z]'s q / kv / kv_scale and writes its out / lse
// (a's own pointers are not used), and takes the z-th attn_workspace_bytes slice of a.ws.
constexpr int kMaxAttnLayers = 4;
struct AttnLayer {
  const uint16_t* q;
  const void* kv;
  const float* kv_scale;
  uint16_t* out;
  float* lse;
};
hipError_t launch_sparse_attn_layers(const AttnArgs& a, const AttnLayer* layers, int nlayers, hipStream_t st);
// Selected keys of sequence b (rows of k entries, Tq rows per sequence) to rows of a paged
// pool; -1 for entries outside [0, kv_len[b]) or table entries outside the pool.
hipError_t launch_page_translate(const int32_t* idx, int32_t* phys, int B, int Tq, int k, const int32_t* kv_len,
                                 int Tk, const int32_t* block_table, int max_blocks, int page_shift,
                                 int64_t pool_tokens, hipStream_t st);

}  // namespace dsa
