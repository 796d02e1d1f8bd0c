// C ABI of the DSA library: argument checks, workspace planning and the IndexCache layer
// stack.  Every check runs on the host before anything is enqueued.
#include <math.h>
#include <string.h>

#include <mutex>
#include <string>

#include "dsa.h"
#include "internal.hpp"

namespace {

thread_local std::string g_last_error;

dsa_status fail(dsa_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

dsa_status launch_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return DSA_OK;
  return fail(DSA_ERR_LAUNCH, std::string(what) + ": " + hipGetErrorString(e));
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Score chunk of the layer stack: at most this many bytes of fp32 score rows at a time.
// Measured at T=65536: 1 GiB chunks (4096 rows) run the indexer and top-k launches 14%
// faster than 128 MiB chunks that would stay in the last-level cache, since each launch
// then has enough work to amortize its ramp and tail; the workspace is small next to HBM.
constexpr int64_t kChunkBytes = int64_t(1) << 30;

int64_t stack_ld(int Tk) { return ((int64_t)Tk + 63) / 64 * 64; }

int chunk_rows(const dsa_shape& s) {
  const int64_t per_row = (int64_t)std::max(1, s.B) * stack_ld(s.Tk) * 4;
  int64_t rows = std::max<int64_t>(1, kChunkBytes / std::max<int64_t>(1, per_row));
  if (rows >= 64) rows = rows / 64 * 64;
  return (int)std::min<int64_t>(rows, std::max(1, s.Tq));
}

// Route of dsa_index_topk: the fused kernels over chunks of `rows` query rows (candidate
// lists instead of score rows), or the score kernel + top-k over score chunks.  The fused
// kernels give every wave whole rows, so a launch needs many rows to balance (rows of all
// lengths at once): the whole Tq in one chunk up to kFusedBytes of workspace.  The fused
// route runs where it pays: many rows, and keys beyond the keep-everything length.
constexpr size_t kFusedBytes = size_t(8) << 30;
constexpr int64_t kFusedMinRows = 1024;

struct IndexTopkPlan {
  bool fused;
  int rows;     // query rows per chunk
  size_t ws;    // workspace bytes
  size_t split_off = 0;  // score route: segment lists of the split top-k (few long rows), if any
};

IndexTopkPlan plan_index_topk(const dsa_shape& s, bool force_unfused) {
  IndexTopkPlan P;
  // (up to kFusedCap keys every row keeps all its keys, and score rows are the cheaper
  // hand-over: measured even at 6144 keys, 20-30% in favour of fusion from 12288 on)
  P.fused = !force_unfused && dsa::index_topk_fused_supported(s.H_I, s.d_I, s.k) &&
            (int64_t)std::max(0, s.B) * std::max(0, s.Tq) >= kFusedMinRows && s.Tk > dsa::kFusedCap;
  if (P.fused) {
    const size_t per_row = std::max<size_t>(1, dsa::fused_layout(s.B, 1, s.Tk).bytes);
    int64_t rows = std::max<int64_t>(1, (int64_t)(kFusedBytes / per_row));
    if (rows >= 64) rows = rows / 64 * 64;
    P.rows = (int)std::min<int64_t>(rows, std::max(1, s.Tq));
    P.ws = dsa::fused_layout(s.B, P.rows, s.Tk).bytes;
  } else {
    P.rows = chunk_rows(s);
    P.ws = (size_t)std::max(0, s.B) * P.rows * stack_ld(s.Tk) * sizeof(float);
    const size_t lists = dsa::topk_split_workspace_bytes(s.B, P.rows, s.Tk, s.k);
    if (lists) {
      P.split_off = align_up(P.ws);
      P.ws = P.split_off + lists;
    }
  }
  return P;
}

// Indices of rows [0, Tq) of every sequence by the planned route.
dsa_status run_index_topk(const IndexTopkPlan& P, const void* q_idx, const void* k_idx, const void* w_idx,
                          const dsa_shape& s, float oversample, int32_t* idx, void* ws, hipStream_t strm,
                          const char* who, const dsa_paged_kv* pages = nullptr) {
  for (int r0 = 0; r0 < s.Tq; r0 += P.rows) {
    const int n = std::min(P.rows, s.Tq - r0);
    if (P.fused) {
      dsa::IndexTopkArgs a{(const uint16_t*)q_idx, (const uint16_t*)k_idx, (const uint16_t*)w_idx, s.kv_len,
                           s.B, s.Tq, s.Tk, s.H_I, s.d_I, s.k, r0, n, oversample, idx, ws};
      dsa_status st = launch_status(dsa::launch_index_topk(a, strm), who);
      if (st != DSA_OK) return st;
    } else {
      const int64_t ld = stack_ld(s.Tk);
      float* scores = reinterpret_cast<float*>(ws);
      dsa::TopkArgs ta{scores, ld, (int64_t)P.rows * ld, s.kv_len, s.B, s.Tq, s.Tk, s.k, r0, n, idx,
                       P.split_off ? reinterpret_cast<char*>(ws) + P.split_off : nullptr};
      if (s.Tk > 0) {
        dsa::IndexerArgs ia{(const uint16_t*)q_idx, (const uint16_t*)k_idx, (const uint16_t*)w_idx, s.kv_len,
                            s.B, s.Tq, s.Tk, s.H_I, s.d_I, r0, n, scores, ld, (int64_t)P.rows * ld};
        if (dsa::topk_split_route(ta)) {  // the indexer may build the top-k's segment lists
          ia.topk_ws = ta.ws;
          ia.topk_k = s.k;
          ia.lists_made = &ta.lists_ready;
        }
        if (pages) {  // k_idx is a key pool (the fused route is never planned for pools)
          ia.block_table = pages->block_table;
          ia.max_blocks = pages->max_blocks;
          ia.page_shift = __builtin_ctz((unsigned)pages->page_size);
          ia.pool_tokens = (int64_t)pages->num_pages * pages->page_size;
        }
        dsa_status st = launch_status(dsa::launch_index_scores(ia, strm), who);
        if (st != DSA_OK) return st;
      }
      // (no keys at all: every row selects nothing, and top-k reads no score)
      dsa_status st = launch_status(dsa::launch_topk(ta, strm), who);
      if (st != DSA_OK) return st;
    }
  }
  return DSA_OK;
}

// The kernels move bf16 / fp8 rows in 16-byte pieces and fp32 / int32 values in 4-byte ones.
bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

dsa_status check_indexer(const void* q, const void* k, const void* w, int B, int Tq, int Tk, int H_I, int d_I,
                         const float* scores, int64_t ld) {
  if (B < 0 || Tq < 0 || Tk < 0) return fail(DSA_ERR_SHAPE, "B, Tq and Tk must be >= 0");
  if (H_I < 1 || d_I < 1) return fail(DSA_ERR_SHAPE, "H_I and d_I must be >= 1");
  if (ld < Tk) return fail(DSA_ERR_SHAPE, "ld must be >= Tk");
  if (!dsa::indexer_supported(H_I, d_I, ld))
    return fail(DSA_ERR_UNSUPPORTED, "indexer supports H_I in {1,2,4,8,16}, d_I in {16,32,64,128}, ld <= 2^22");
  if ((int64_t)B * Tq == 0) return DSA_OK;
  if (!q || !k || !w || !scores) return fail(DSA_ERR_NULL, "q_idx, k_idx, w_idx and scores are required");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(w, H_I == 1 ? 2 : 4) || !aligned(scores, 4))
    return fail(DSA_ERR_UNSUPPORTED, "q_idx and k_idx must be 16-byte aligned, w_idx 4-byte (2 for H_I=1), scores 4-byte");
  return DSA_OK;
}

dsa_status check_topk(const float* scores, int64_t ld, int B, int Tq, int Tk, int k, const int32_t* idx) {
  if (B < 0 || Tq < 0 || Tk < 0) return fail(DSA_ERR_SHAPE, "B, Tq and Tk must be >= 0");
  if (k < 1) return fail(DSA_ERR_SHAPE, "k must be >= 1");
  if (ld < Tk) return fail(DSA_ERR_SHAPE, "ld must be >= Tk");
  if (k > dsa::kTopkMaxK) return fail(DSA_ERR_UNSUPPORTED, "k must be <= 4096");
  if (Tk > dsa::kTopkMaxTk) return fail(DSA_ERR_UNSUPPORTED, "Tk must be <= 2^24");
  if ((int64_t)B * Tq == 0) return DSA_OK;
  if (!scores || !idx) return fail(DSA_ERR_NULL, "scores and idx are required");
  if (!aligned(scores, 4) || !aligned(idx, 4)) return fail(DSA_ERR_UNSUPPORTED, "scores and idx must be 4-byte aligned");
  return DSA_OK;
}

dsa_status check_attn(const dsa::AttnArgs& a, size_t ws_bytes) {
  if (a.B < 0 || a.Tq < 0 || a.Tk < 0) return fail(DSA_ERR_SHAPE, "B, Tq and Tk must be >= 0");
  if (a.H < 1 || a.Hkv < 1 || a.Dqk < 1 || a.Dv < 1 || a.k < 1)
    return fail(DSA_ERR_SHAPE, "H, Hkv, Dqk, Dv and k must be >= 1");
  if (a.H % a.Hkv) return fail(DSA_ERR_SHAPE, "H must be a multiple of Hkv");
  if (!a.v && a.Dv > a.Dqk) return fail(DSA_ERR_SHAPE, "Dv > Dqk needs a separate v");
  if (!isfinite(a.sm_scale)) return fail(DSA_ERR_SHAPE, "sm_scale must be finite");
  if (a.kv_fmt != DSA_KV_BF16 && a.v) return fail(DSA_ERR_UNSUPPORTED, "fp8 and MXFP4 rows need V taken from kv (v = NULL)");
  if (a.kv_fmt == DSA_KV_MXFP4 && a.kv_scale)
    return fail(DSA_ERR_UNSUPPORTED, "MXFP4 rows carry their own block scales: kv_scale must be NULL");
  if (!dsa::attn_mla_supported(a) && !dsa::attn_mha_supported(a))
    return fail(DSA_ERR_UNSUPPORTED,
                "supported: MLA (Hkv=1, Dqk=576, Dv=512, v=NULL, H%16==0, k<=65536, bf16/fp8/MXFP4) or "
                "multi-head (Hkv=H<=16, Dqk=Dv=32, bf16, v given, k<=4096)");
  if ((int64_t)a.B * a.Tq == 0) return DSA_OK;
  if (!a.q || !a.kv || !a.idx || !a.out) return fail(DSA_ERR_NULL, "q, kv, idx and out are required");
  if (a.kv_fmt == DSA_KV_FP8_E4M3 && !a.kv_scale) return fail(DSA_ERR_NULL, "kv_scale is required for fp8 rows");
  if (!aligned(a.q, 16) || !aligned(a.kv, 16) || !aligned(a.v, 16) || !aligned(a.out, 16) || !aligned(a.ws, 16) ||
      !aligned(a.idx, 4) || !aligned(a.kv_scale, 4) || !aligned(a.lse, 4))
    return fail(DSA_ERR_UNSUPPORTED, "q, kv, v, out and ws must be 16-byte aligned; idx, kv_scale and lse 4-byte");
  const size_t need = dsa::attn_workspace_bytes(a.B, a.Tq, a.H, a.Dv, a.k, dsa::attn_mla_supported(a));
  if (need && (!a.ws || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "attention workspace too small: need " + std::to_string(need) + " bytes");
  return DSA_OK;
}

dsa::AttnArgs attn_args(const void* q, const void* kv, const float* kv_scale, const void* v, dsa_kv_dtype kv_dtype,
                        const int32_t* idx, int B, int Tq, int Tk, int H, int Hkv, int Dqk, int Dv, int k,
                        float sm_scale, void* out, float* lse, void* ws) {
  dsa::AttnArgs a;
  a.q = (const uint16_t*)q;
  a.kv = kv;
  a.kv_scale = kv_scale;
  a.v = (const uint16_t*)v;
  a.kv_fmt = (int)kv_dtype;
  a.idx = idx;
  a.B = B;
  a.Tq = Tq;
  a.Tk = Tk;
  a.H = H;
  a.Hkv = Hkv;
  a.Dqk = Dqk;
  a.Dv = Dv;
  a.k = k;
  a.sm_scale = sm_scale;
  a.out = (uint16_t*)out;
  a.lse = lse;
  a.ws = ws;
  return a;
}

bool valid_kv_dtype(dsa_kv_dtype d) { return d == DSA_KV_BF16 || d == DSA_KV_FP8_E4M3 || d == DSA_KV_MXFP4; }

// A paged layout for sequences of up to Tk keys over pools of row_bytes-wide rows.
dsa_status check_pages(const dsa_paged_kv* pg, int Tk, int64_t row_bytes, int64_t max_rows, const char* pool) {
  if (!pg || !pg->block_table) return fail(DSA_ERR_NULL, "pages and its block_table are required");
  if (pg->page_size < 32 || pg->page_size > 65536 || (pg->page_size & (pg->page_size - 1)))
    return fail(DSA_ERR_UNSUPPORTED, "page_size must be a power of two in [32, 65536]");
  if (pg->max_blocks < 1 || pg->num_pages < 1) return fail(DSA_ERR_SHAPE, "max_blocks and num_pages must be >= 1");
  if ((int64_t)pg->max_blocks * pg->page_size < Tk)
    return fail(DSA_ERR_SHAPE, "max_blocks * page_size must cover Tk");
  const int64_t rows = (int64_t)pg->num_pages * pg->page_size;
  if (rows > max_rows || rows * row_bytes >= (int64_t(1) << 32))
    return fail(DSA_ERR_UNSUPPORTED, std::string(pool) + " pool too large for the kernels' 32-bit row offsets");
  if (!aligned(pg->block_table, 4)) return fail(DSA_ERR_UNSUPPORTED, "block_table must be 4-byte aligned");
  return DSA_OK;
}

int page_shift(int page_size) { return __builtin_ctz((unsigned)page_size); }
int64_t pool_rows(const dsa_paged_kv& pg) { return (int64_t)pg.num_pages * pg.page_size; }

// Pool rows of the attention gather: the kernel scales row indices with a 24-bit multiply.
constexpr int64_t kMaxAttnPoolRows = int64_t(1) << 24;
int64_t latent_row_bytes(dsa_kv_dtype d) { return d == DSA_KV_MXFP4 ? 320 : d == DSA_KV_FP8_E4M3 ? 576 : 1152; }

size_t paged_idx_bytes(const dsa_shape& s) { return align_up((size_t)std::max(0, s.B) * std::max(0, s.Tq) * s.k * 4); }

}  // namespace

extern "C" {

int dsa_abi_version(void) { return DSA_ABI_VERSION; }

const char* dsa_last_error(void) { return g_last_error.c_str(); }

const char* dsa_status_string(dsa_status s) {
  switch (s) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_NULL: return "DSA_ERR_NULL";
    case DSA_ERR_SHAPE: return "DSA_ERR_SHAPE";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED";
    case DSA_ERR_PATTERN: return "DSA_ERR_PATTERN";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE";
    case DSA_ERR_LAUNCH: return "DSA_ERR_LAUNCH";
    case DSA_ERR_DEVICE: return "DSA_ERR_DEVICE";
  }
  return "DSA_ERR_UNKNOWN";
}

dsa_status dsa_index_scores(const void* q_idx, const void* k_idx, const void* w_idx, const int32_t* kv_len, int B,
                            int Tq, int Tk, int H_I, int d_I, float* scores, int64_t ld, void* stream) {
  dsa_status st = check_indexer(q_idx, k_idx, w_idx, B, Tq, Tk, H_I, d_I, scores, ld);
  if (st != DSA_OK || (int64_t)B * Tq == 0) return st;
  st = launch_status(dsa::launch_fill_masked(scores, ld, (int64_t)Tq * ld, kv_len, B, Tq, Tk, as_stream(stream)),
                     "dsa_index_scores: -inf fill");
  if (st != DSA_OK || Tk == 0) return st;
  dsa::IndexerArgs a{(const uint16_t*)q_idx, (const uint16_t*)k_idx, (const uint16_t*)w_idx, kv_len, B, Tq, Tk,
                     H_I, d_I, 0, Tq, scores, ld, (int64_t)Tq * ld};
  return launch_status(dsa::launch_index_scores(a, as_stream(stream)), "dsa_index_scores");
}

dsa_status dsa_topk(const float* scores, int64_t ld, const int32_t* kv_len, int B, int Tq, int Tk, int k,
                    int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  dsa_status st = check_topk(scores, ld, B, Tq, Tk, k, idx);
  if (st != DSA_OK || (int64_t)B * Tq == 0) return st;
  // the optional workspace: few long rows then split over the chip
  const size_t need = dsa::topk_split_workspace_bytes(B, Tq, Tk, k);
  if (ws && ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "topk workspace too small: need " + std::to_string(need) + " bytes");
  if (!aligned(ws, 16)) return fail(DSA_ERR_UNSUPPORTED, "ws must be 16-byte aligned");
  dsa::TopkArgs a{scores, ld, (int64_t)Tq * ld, kv_len, B, Tq, Tk, k, 0, Tq, idx, need ? ws : nullptr};
  return launch_status(dsa::launch_topk(a, as_stream(stream)), "dsa_topk");
}

dsa_status dsa_index_topk(const void* q_idx, const void* k_idx, const void* w_idx, const int32_t* kv_len, int B,
                          int Tq, int Tk, int H_I, int d_I, int k, float oversample, int32_t* idx, void* ws,
                          size_t ws_bytes, void* stream) {
  dsa_shape s{};
  s.B = B;
  s.Tq = Tq;
  s.Tk = Tk;
  s.H_I = H_I;
  s.d_I = d_I;
  s.k = k;
  s.kv_len = kv_len;
  // the score rows, when used, live in the workspace (checked below)
  const float* ws_scores = reinterpret_cast<const float*>(&s);
  dsa_status st = check_indexer(q_idx, k_idx, w_idx, B, Tq, Tk, H_I, d_I, ws_scores, stack_ld(Tk));
  if (st != DSA_OK) return st;
  st = check_topk(ws_scores, stack_ld(Tk), B, Tq, Tk, k, idx);
  if (st != DSA_OK) return st;
  if (!isfinite(oversample)) return fail(DSA_ERR_SHAPE, "oversample must be finite");
  if ((int64_t)B * Tq == 0) return DSA_OK;
  const IndexTopkPlan P = plan_index_topk(s, false);
  if (P.ws && (!ws || ws_bytes < P.ws))
    return fail(DSA_ERR_WORKSPACE, "index_topk workspace too small: need " + std::to_string(P.ws) + " bytes");
  if (!aligned(ws, 16)) return fail(DSA_ERR_UNSUPPORTED, "ws must be 16-byte aligned");
  return run_index_topk(P, q_idx, k_idx, w_idx, s, oversample, idx, ws, as_stream(stream), "dsa_index_topk");
}

dsa_status dsa_indexer_kl(const void* q_idx, const void* k_idx, const void* w_idx, const void* q, const void* k,
                          const int32_t* idx, const int32_t* kv_len, int B, int Tq, int Tk, int H_I, int d_I, int H,
                          int Dqk, int kk, float sm_scale, float* loss, float* dq_idx, float* dw_idx, float* dk_idx,
                          void* ws, size_t ws_bytes, void* stream) {
  if (B < 0 || Tq < 0 || Tk < 0) return fail(DSA_ERR_SHAPE, "B, Tq and Tk must be >= 0");
  if (H_I < 1 || d_I < 1 || H < 1 || Dqk < 1) return fail(DSA_ERR_SHAPE, "H_I, d_I, H and Dqk must be >= 1");
  if (idx && kk < 1) return fail(DSA_ERR_SHAPE, "kk must be >= 1 when idx is given");
  if (!isfinite(sm_scale)) return fail(DSA_ERR_SHAPE, "sm_scale must be finite");
  if (!dsa::indexer_kl_supported(H_I, d_I, H, H, Dqk))
    return fail(DSA_ERR_UNSUPPORTED, "indexer KL supports H_I <= 16, d_I in {16,32,64,128}, H <= 16, Dqk = 32");
  if (idx ? kk > dsa::kKlMaxKeys : Tk > dsa::kKlMaxKeys)
    return fail(DSA_ERR_UNSUPPORTED, "indexer KL takes at most 4096 keys per row (kk, or Tk without idx)");
  if (dk_idx && ((int64_t)B * Tk >= INT32_MAX || (idx && (int64_t)B * Tq * kk >= INT32_MAX)))
    return fail(DSA_ERR_UNSUPPORTED, "indexer KL key gradients need B * Tk and B * Tq * kk below 2^31 - 1");
  if ((int64_t)B * Tq == 0 && !(dk_idx && (int64_t)B * Tk > 0)) return DSA_OK;
  if (!q_idx || !k_idx || !w_idx || !q || !k || !loss)
    return fail(DSA_ERR_NULL, "q_idx, k_idx, w_idx, q, k and loss are required");
  if (!aligned(q_idx, 16) || !aligned(k_idx, 16) || !aligned(q, 16) || !aligned(k, 16) || !aligned(w_idx, 2) ||
      !aligned(idx, 4) || !aligned(loss, 4) || !aligned(dq_idx, 4) || !aligned(dw_idx, 4) || !aligned(dk_idx, 4))
    return fail(DSA_ERR_UNSUPPORTED, "q_idx, k_idx, q and k must be 16-byte aligned; w_idx 2-byte; idx and outputs 4");
  if (dk_idx) {
    const size_t need = dsa::indexer_kl_workspace_bytes(B, Tq, Tk, H_I, kk, idx == nullptr);
    if (need && (!ws || ws_bytes < need))
      return fail(DSA_ERR_WORKSPACE, "indexer KL workspace too small: need " + std::to_string(need) + " bytes");
    if (!aligned(ws, 256)) return fail(DSA_ERR_UNSUPPORTED, "ws must be 256-byte aligned");
  }
  dsa::IndexerKlArgs a{(const uint16_t*)q_idx, (const uint16_t*)k_idx, (const uint16_t*)w_idx, (const uint16_t*)q,
                       (const uint16_t*)k, idx, kv_len, B, Tq, Tk, H_I, d_I, H, idx ? kk : 0, sm_scale, loss,
                       dq_idx, dw_idx, dk_idx};
  return launch_status(dsa::launch_indexer_kl(a, ws, as_stream(stream)), "dsa_indexer_kl");
}

dsa_status dsa_index_scores_paged(const void* q_idx, const void* k_pool, const void* w_idx, const dsa_paged_kv* pages,
                                  const int32_t* kv_len, int B, int Tq, int Tk, int H_I, int d_I, float* scores,
                                  int64_t ld, void* stream) {
  dsa_status st = check_indexer(q_idx, k_pool, w_idx, B, Tq, Tk, H_I, d_I, scores, ld);
  if (st != DSA_OK) return st;
  st = check_pages(pages, Tk, (int64_t)d_I * 2, INT64_MAX, "key");
  if (st != DSA_OK || (int64_t)B * Tq == 0) return st;
  st = launch_status(dsa::launch_fill_masked(scores, ld, (int64_t)Tq * ld, kv_len, B, Tq, Tk, as_stream(stream)),
                     "dsa_index_scores_paged: -inf fill");
  if (st != DSA_OK || Tk == 0) return st;
  dsa::IndexerArgs a{(const uint16_t*)q_idx, (const uint16_t*)k_pool, (const uint16_t*)w_idx, kv_len, B, Tq, Tk,
                     H_I, d_I, 0, Tq, scores, ld, (int64_t)Tq * ld};
  a.block_table = pages->block_table;
  a.max_blocks = pages->max_blocks;
  a.page_shift = page_shift(pages->page_size);
  a.pool_tokens = pool_rows(*pages);
  return launch_status(dsa::launch_index_scores(a, as_stream(stream)), "dsa_index_scores_paged");
}

dsa_status dsa_sparse_attn_paged(const void* q, const void* kv_pool, const float* kv_scale_pool, dsa_kv_dtype kv_dtype,
                                 const dsa_paged_kv* pages, const int32_t* idx, const int32_t* kv_len, int B, int Tq,
                                 int Tk, int H, int Dqk, int Dv, int k, float sm_scale, void* out, float* lse, void* ws,
                                 size_t ws_bytes, void* stream) {
  if (!valid_kv_dtype(kv_dtype)) return fail(DSA_ERR_SHAPE, "unknown kv dtype");
  dsa::AttnArgs a = attn_args(q, kv_pool, kv_scale_pool, nullptr, kv_dtype, idx, B, Tq, Tk, H, 1, Dqk, Dv, k, sm_scale,
                              out, lse, ws);
  dsa_status st = check_attn(a, (size_t)-1);
  if (st != DSA_OK) return st;
  if (!dsa::attn_mla_supported(a)) return fail(DSA_ERR_UNSUPPORTED, "paged attention supports the MLA form only");
  st = check_pages(pages, Tk, latent_row_bytes(kv_dtype), kMaxAttnPoolRows, "latent");
  if (st != DSA_OK || (int64_t)B * Tq == 0) return st;
  dsa_shape s{};
  s.B = B;
  s.Tq = Tq;
  s.Tk = Tk;
  s.H = H;
  s.Hkv = 1;
  s.Dqk = Dqk;
  s.Dv = Dv;
  s.k = k;
  const size_t need = dsa_workspace_size(&s, DSA_OP_ATTN_PAGED);
  if (!ws || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "paged attention workspace too small: need " + std::to_string(need) + " bytes");
  hipStream_t strm = as_stream(stream);
  int32_t* phys = reinterpret_cast<int32_t*>(ws);
  st = launch_status(dsa::launch_page_translate(idx, phys, B, Tq, k, kv_len, Tk, pages->block_table, pages->max_blocks,
                                                page_shift(pages->page_size), pool_rows(*pages), strm),
                     "dsa_sparse_attn_paged: translate");
  if (st != DSA_OK) return st;
  a.idx = phys;
  a.Tk = (int)pool_rows(*pages);
  a.kv_bstride = 0;
  a.ws = reinterpret_cast<char*>(ws) + paged_idx_bytes(s);
  return launch_status(dsa::launch_sparse_attn(a, strm), "dsa_sparse_attn_paged");
}

dsa_status dsa_sparse_attn(const void* q, const void* kv, const float* kv_scale, const void* v,
                           dsa_kv_dtype kv_dtype, const int32_t* idx, int B, int Tq, int Tk, int H, int Hkv, int Dqk,
                           int Dv, int k, float sm_scale, void* out, float* lse, void* ws, size_t ws_bytes,
                           void* stream) {
  if (!valid_kv_dtype(kv_dtype)) return fail(DSA_ERR_SHAPE, "unknown kv dtype");
  dsa::AttnArgs a = attn_args(q, kv, kv_scale, v, kv_dtype, idx, B, Tq, Tk, H, Hkv, Dqk, Dv, k, sm_scale, out, lse, ws);
  dsa_status st = check_attn(a, ws_bytes);
  if (st != DSA_OK || (int64_t)B * Tq == 0) return st;
  return launch_status(dsa::launch_sparse_attn(a, as_stream(stream)), "dsa_sparse_attn");
}

}  // extern "C"

namespace {

// Device-resident scratch of dsa_sparse_attn_noalloc: the split-key partial results of a
// call live here instead of in a caller's workspace.  Each device holds its own copy from
// the library's load until the process ends; host code addresses it only through the
// pointer hipGetSymbolAddress returns for the current device (the array's name is a host
// stand-in, not a device address).
// The split planner keeps splits x workgroups within one round of 256, so the partials of
// any shape fit: 256 x 16 (row, head) pairs x (512 + 2) floats = 8,421,376 bytes.
constexpr size_t kNoAllocScratchBytes = size_t(256) * 16 * (512 + 2) * sizeof(float);
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address, looked up once per device (with it current).
dsa_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(DSA_ERR_DEVICE, std::string("dsa_sparse_attn_noalloc: no usable device: ") + hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(DSA_ERR_DEVICE, std::string("dsa_sparse_attn_noalloc: scratch lookup failed: ") +
                                      hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

}  // namespace

extern "C" {

size_t dsa_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

dsa_status dsa_sparse_attn_noalloc(const void* q, const void* kv, const float* kv_scale, const void* v,
                                   dsa_kv_dtype kv_dtype, const int32_t* idx, int B, int Tq, int Tk, int H, int Hkv,
                                   int Dqk, int Dv, int k, float sm_scale, void* out, float* lse, void* stream) {
  if (!valid_kv_dtype(kv_dtype)) return fail(DSA_ERR_SHAPE, "unknown kv dtype");
  dsa::AttnArgs a = attn_args(q, kv, kv_scale, v, kv_dtype, idx, B, Tq, Tk, H, Hkv, Dqk, Dv, k, sm_scale, out, lse,
                              nullptr);
  // the workspace check below is the scratch limit; check_attn sees an unlimited one
  const size_t need = dsa::attn_workspace_bytes(B, Tq, H, Dv, k, dsa::attn_mla_supported(a));
  a.ws = reinterpret_cast<void*>(uintptr_t(256));  // alignment placeholder for the checks only
  dsa_status st = check_attn(a, (size_t)-1);
  if (st != DSA_OK || (int64_t)B * Tq == 0) return st;
  if (need > kNoAllocScratchBytes)
    return fail(DSA_ERR_UNSUPPORTED, "dsa_sparse_attn_noalloc: this shape needs " + std::to_string(need) +
                                         " bytes of split-key scratch; the built-in scratch holds " +
                                         std::to_string(kNoAllocScratchBytes) + " (use dsa_sparse_attn with a workspace)");
  a.ws = nullptr;
  if (need) {
    st = scratch_for_current_device(&a.ws);
    if (st != DSA_OK) return st;
  }
  return launch_status(dsa::launch_sparse_attn(a, as_stream(stream)), "dsa_sparse_attn_noalloc");
}

dsa_status dsa_check_pattern(const char* pattern, int n_layers, unsigned flags) {
  if (!pattern) return fail(DSA_ERR_NULL, "pattern is required");
  if (n_layers < 0) return fail(DSA_ERR_PATTERN, "n_layers must be >= 0");
  const size_t len = strnlen(pattern, (size_t)n_layers + 1);
  if (len != (size_t)n_layers) return fail(DSA_ERR_PATTERN, "pattern length must equal n_layers");
  for (int i = 0; i < n_layers; ++i)
    if (pattern[i] != 'F' && pattern[i] != 'S')
      return fail(DSA_ERR_PATTERN, "pattern character " + std::to_string(i) + " is not 'F' or 'S'");
  if (n_layers > 0 && pattern[0] == 'S' && !(flags & DSA_CACHE_PREFILLED))
    return fail(DSA_ERR_PATTERN, "a leading 'S' layer has no cached indices (set DSA_CACHE_PREFILLED)");
  return DSA_OK;
}

dsa_status dsa_pattern_from_freq(int freq, int n_layers, char* out) {
  if (!out) return fail(DSA_ERR_NULL, "out is required");
  if (freq < 1 || n_layers < 0) return fail(DSA_ERR_PATTERN, "freq must be >= 1 and n_layers >= 0");
  for (int i = 0; i < n_layers; ++i) out[i] = (i % freq == 0) ? 'F' : 'S';
  out[n_layers] = '\0';
  return DSA_OK;
}

int dsa_stack_chunk_rows(const dsa_shape* shape) { return shape ? chunk_rows(*shape) : 1; }

size_t dsa_workspace_size(const dsa_shape* s, dsa_op op) {
  if (!s || s->B < 0 || s->Tq < 0 || s->Tk < 0) return 0;
  if (op == DSA_OP_INDEXER_KL_DENSE)
    return s->H_I < 1 ? 0 : dsa::indexer_kl_workspace_bytes(s->B, s->Tq, s->Tk, s->H_I, 0, true);
  if (op == DSA_OP_INDEXER_KL)
    return s->H_I < 1 || s->k < 1 ? 0 : dsa::indexer_kl_workspace_bytes(s->B, s->Tq, s->Tk, s->H_I, s->k, false);
  if (s->H < 1 || s->Dv < 1 || s->k < 1) return 0;
  const bool mla = s->Hkv == 1 && s->Dqk == 576 && s->Dv == 512;
  switch (op) {
    case DSA_OP_SCORES: return 0;
    case DSA_OP_TOPK: return dsa::topk_split_workspace_bytes(s->B, s->Tq, s->Tk, s->k);
    case DSA_OP_ATTN: return dsa::attn_workspace_bytes(s->B, s->Tq, s->H, s->Dv, s->k, mla);
    case DSA_OP_INDEX_TOPK: return plan_index_topk(*s, false).ws;
    case DSA_OP_ATTN_PAGED: return paged_idx_bytes(*s) + dsa::attn_workspace_bytes(s->B, s->Tq, s->H, s->Dv, s->k, true);
    // stacks: the attention of up to kMaxAttnLayers layers that share an index list runs in
    // one launch, each layer with its own split partials
    case DSA_OP_STACK_PAGED:  // score chunks (paged keys take the score route) + pool rows + attention
      return align_up(plan_index_topk(*s, true).ws) + paged_idx_bytes(*s) +
             dsa::kMaxAttnLayers * dsa::attn_workspace_bytes(s->B, s->Tq, s->H, s->Dv, s->k, true);
    case DSA_OP_INDEXER_KL:
    case DSA_OP_INDEXER_KL_DENSE: return 0;  // handled above
    case DSA_OP_STACK: {
      // either route of the 'F' layers fits (DSA_STACK_UNFUSED picks the score chunks)
      const size_t sel = std::max(plan_index_topk(*s, false).ws, plan_index_topk(*s, true).ws);
      return align_up(sel) + dsa::kMaxAttnLayers * dsa::attn_workspace_bytes(s->B, s->Tq, s->H, s->Dv, s->k, mla);
    }
  }
  return 0;
}

}  // extern "C"

namespace {

// dsa_layer_stack, over dense caches (pages == nullptr) or paged pools.
dsa_status stack_impl(const char* pattern, int n_layers, const dsa_layer_io* layers, const dsa_shape* shape,
                      const dsa_paged_kv* pages, int32_t* index_cache, unsigned flags, void* ws, size_t ws_bytes,
                      void* stream) {
  if (!shape) return fail(DSA_ERR_NULL, "shape is required");
  dsa_status st = dsa_check_pattern(pattern, n_layers, flags);
  if (st != DSA_OK) return st;
  if (n_layers > 0 && !layers) return fail(DSA_ERR_NULL, "layers is required");
  const dsa_shape& s = *shape;
  if (!valid_kv_dtype(s.kv_dtype)) return fail(DSA_ERR_SHAPE, "unknown kv dtype");
  if (pages) {
    st = check_pages(pages, s.Tk, (int64_t)s.d_I * 2, INT64_MAX, "key");
    if (st == DSA_OK) st = check_pages(pages, s.Tk, latent_row_bytes(s.kv_dtype), kMaxAttnPoolRows, "latent");
    if (st != DSA_OK) return st;
  }
  // validate every layer before enqueueing anything
  for (int l = 0; l < n_layers; ++l) {
    const dsa_layer_io& L = layers[l];
    const std::string at = " (layer " + std::to_string(l) + ")";
    if (pattern[l] == 'F') {
      // the score rows live in the workspace, which is checked below
      const float* ws_scores = reinterpret_cast<const float*>(&s);
      st = check_indexer(L.q_idx, L.k_idx, L.w_idx, s.B, s.Tq, s.Tk, s.H_I, s.d_I, ws_scores, stack_ld(s.Tk));
      if (st != DSA_OK) return fail(st, g_last_error + at);
      st = check_topk(ws_scores, stack_ld(s.Tk), s.B, s.Tq, s.Tk, s.k, index_cache);
      if (st != DSA_OK) return fail(st, g_last_error + at);
    }
    dsa::AttnArgs a = attn_args(L.q, L.kv, L.kv_scale, L.v, s.kv_dtype, index_cache, s.B, s.Tq, s.Tk, s.H, s.Hkv,
                                s.Dqk, s.Dv, s.k, s.sm_scale, L.out, L.lse, ws);
    st = check_attn(a, (size_t)-1);
    if (st != DSA_OK) return fail(st, g_last_error + at);
    if (pages && !dsa::attn_mla_supported(a)) return fail(DSA_ERR_UNSUPPORTED, "paged caches: MLA form only" + at);
  }
  if ((int64_t)s.B * s.Tq == 0 || n_layers == 0) return DSA_OK;
  if (!index_cache) return fail(DSA_ERR_NULL, "index_cache is required");
  const size_t need = dsa_workspace_size(shape, pages ? DSA_OP_STACK_PAGED : DSA_OP_STACK);
  if (need && (!ws || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "stack workspace too small: need " + std::to_string(need) + " bytes");

  // workspace: selection (score chunks or fused lists) | [pool rows of the cache] | attention
  const IndexTopkPlan P = plan_index_topk(s, pages != nullptr || (flags & DSA_STACK_UNFUSED) != 0);
  const size_t sel = pages ? P.ws : std::max(plan_index_topk(s, false).ws, plan_index_topk(s, true).ws);
  char* const wsb = reinterpret_cast<char*>(ws);
  int32_t* const phys = pages ? reinterpret_cast<int32_t*>(wsb + align_up(sel)) : nullptr;
  void* attn_ws = wsb + align_up(sel) + (pages ? paged_idx_bytes(s) : 0);
  hipStream_t strm = as_stream(stream);
  auto translate = [&]() {
    return launch_status(dsa::launch_page_translate(index_cache, phys, s.B, s.Tq, s.k, s.kv_len, s.Tk,
                                                    pages->block_table, pages->max_blocks,
                                                    page_shift(pages->page_size), pool_rows(*pages), strm),
                         "dsa_layer_stack_paged: translate");
  };
  if (pages && pattern[0] == 'S') {  // a prefilled cache
    st = translate();
    if (st != DSA_OK) return st;
  }
  bool any_full = false;
  for (int l = 0; l < n_layers;) {
    const dsa_layer_io& L = layers[l];
    if (pattern[l] == 'F') {
      any_full = true;
      st = run_index_topk(P, L.q_idx, L.k_idx, L.w_idx, s, 0.f, index_cache, ws, strm, "dsa_layer_stack: index/top-k",
                          pages);
      if (st == DSA_OK && pages) st = translate();
      if (st != DSA_OK) return st;
    }
    dsa::AttnArgs a = attn_args(L.q, L.kv, L.kv_scale, L.v, s.kv_dtype, index_cache, s.B, s.Tq, s.Tk, s.H, s.Hkv,
                                s.Dqk, s.Dv, s.k, s.sm_scale, L.out, L.lse, attn_ws);
    // the cache holds this library's top-k rows (valid entries first), unless the caller
    // prefilled it with other rows and no 'F' layer has run yet
    if (!(flags & DSA_CACHE_PREFILLED) || any_full || (flags & DSA_CACHE_TOPK_ROWS)) {
      a.tail_kv_len = s.kv_len;
      a.tail_Tk = s.Tk;
    }
    if (pages) {
      a.idx = phys;
      a.Tk = (int)pool_rows(*pages);
      a.kv_bstride = 0;
    }
    // layer l and the 'S' layers right after it read the same indices: when the MLA kernel
    // splits keys (few query rows, each launch latency-bound) they share one launch
    int n = 1;
    if (dsa::attn_mla_supported(a) && dsa::attn_mla_splits(s.B, s.Tq, s.H, s.k) > 1)
      while (n < dsa::kMaxAttnLayers && l + n < n_layers && pattern[l + n] == 'S') ++n;
    dsa::AttnLayer group[dsa::kMaxAttnLayers];
    for (int i = 0; i < n; ++i) {
      const dsa_layer_io& Li = layers[l + i];
      group[i] = {static_cast<const uint16_t*>(Li.q), Li.kv, Li.kv_scale, static_cast<uint16_t*>(Li.out), Li.lse};
    }
    st = launch_status(dsa::launch_sparse_attn_layers(a, group, n, strm), "dsa_layer_stack: attention");
    if (st != DSA_OK) return st;
    l += n;
  }
  return DSA_OK;
}

}  // namespace

extern "C" {

dsa_status dsa_layer_stack(const char* pattern, int n_layers, const dsa_layer_io* layers, const dsa_shape* shape,
                           int32_t* index_cache, unsigned flags, void* ws, size_t ws_bytes, void* stream) {
  return stack_impl(pattern, n_layers, layers, shape, nullptr, index_cache, flags, ws, ws_bytes, stream);
}

dsa_status dsa_layer_stack_paged(const char* pattern, int n_layers, const dsa_layer_io* layers, const dsa_shape* shape,
                                 const dsa_paged_kv* pages, int32_t* index_cache, unsigned flags, void* ws,
                                 size_t ws_bytes, void* stream) {
  if (!pages) return fail(DSA_ERR_NULL, "pages is required");
  return stack_impl(pattern, n_layers, layers, shape, pages, index_cache, flags, ws, ws_bytes, stream);
}

}  // extern "C"
