/*
 * dsa.h - C ABI of the DeepSeek Sparse Attention (DSA) hot path on AMD Instinct MI355X
 * (gfx950).  Plain C99: no HIP or torch types.  Streams are passed as `void*` holding a
 * hipStream_t (NULL = the default stream).
 *
 * The path (as the source pages describe DSA):
 *   1. lightning-indexer scores  I[t,s] = sum_j w[t,j] * ReLU(q_I[t,j] . k_I[s]) over causal
 *      keys s <= t ("DSA ablation model card", model list: a ReLU indexer with a few small
 *      heads selects each query's top keys; its parameter count fixes one indexer key per
 *      token, shared by the heads);
 *   2. a per-query causal top-k (k = 512 on that card; 2048 on the "DSV2-Lite-IndexCache-
 *      Sparse-1250" card, intro), where a query with fewer than k causal keys keeps all of
 *      them (ablation card, "Benchmarks" note);
 *   3. softmax attention over the selected keys only, in multi-head form or in the MLA
 *      latent form (one shared 576-wide row per token: 512 compressed-KV values then 64
 *      rotary values, "DeepSeek-V2-Lite-Chat SIQ K4/K3" card, "Measured"; V = the first
 *      512 values of the same row);
 *   4. IndexCache reuse across layers: 'F' layers compute and store the top-k indices, 'S'
 *      layers attend with the indices handed down the stack ("IndexCache" vLLM feature
 *      doc, "How It Works"; pattern semantics from its "Configuration Reference").
 *
 * Conventions shared by every entry point
 *   - Tensors are dense, row-major, in device memory the caller allocated; the library
 *     never allocates, frees or synchronizes.  All work is enqueued in order on `stream`.
 *     Inputs must stay valid until that work completes.  Outputs must not alias inputs.
 *   - bf16 tensors hold IEEE bfloat16 values; fp8 tensors hold OCP e4m3 ("e4m3fn") bytes;
 *     fp4 latent rows are OCP MXFP4 (see dsa_kv_dtype).
 *   - Alignment: bf16, fp8 and fp4 tensors and workspaces start on 16-byte boundaries, fp32 and
 *     int32 tensors on 4-byte ones (w_idx: 4, or 2 when H_I = 1); otherwise the call
 *     returns DSA_ERR_UNSUPPORTED.  Row pitches follow from the dense layouts.
 *   - Positions: sequence b holds L_b = kv_len[b] keys (kv_len: device int32[B], or NULL
 *     meaning L_b = Tk for every b).  Query row i of the Tq rows of sequence b sits at
 *     position p = L_b - Tq + i and may attend keys 0..p (its own key included).  Prefill:
 *     Tq = Tk = T.  Decode: Tq = 1, kv_len = cache lengths.  Values of kv_len are clamped
 *     to [0, Tk] on the device; rows with p < 0 have no candidates.
 *   - Errors: arguments are checked on the host before anything is enqueued; a status
 *     other than DSA_OK means nothing ran.  DSA_ERR_LAUNCH reports a failed kernel launch
 *     (work enqueued before it in the same call may have run).  Device faults surface at
 *     the caller's next synchronization.  dsa_last_error() gives a message for the calling
 *     thread's last failure.
 *   - Determinism: identical inputs and shapes give bit-identical outputs (fixed reduction
 *     orders), whatever chunk size the library picks.  Inside dsa_layer_stack, the attention
 *     of an 'F' layer and the 'S' layers after it may run as one launch with fewer key splits
 *     per layer than a lone dsa_sparse_attn call takes (few query rows), so such a layer's
 *     outputs can differ from the lone call's in the last bits (not between runs).
 *   - Thread safety: re-entrant; concurrent calls on different streams need separate
 *     workspaces.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 1

typedef enum {
  DSA_OK = 0,
  DSA_ERR_NULL = 1,        /* a required pointer is NULL */
  DSA_ERR_SHAPE = 2,       /* a size is negative, zero where it must not be, or inconsistent */
  DSA_ERR_UNSUPPORTED = 3, /* a valid shape this build has no kernel for */
  DSA_ERR_PATTERN = 4,     /* bad F/S pattern */
  DSA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than dsa_workspace_size() */
  DSA_ERR_LAUNCH = 6,      /* a HIP launch failed */
  DSA_ERR_DEVICE = 7       /* no usable gfx950 device / HIP runtime error */
} dsa_status;

/*
 * Latent row formats (MLA form; the multi-head form reads bf16 only).
 *   DSA_KV_BF16      Dqk bf16 values.
 *   DSA_KV_FP8_E4M3  Dqk e4m3 bytes; value = code * kv_scale[row] (one fp32 per row).
 *   DSA_KV_MXFP4     OCP Microscaling FP4, Dqk/2 + 32 = 320 bytes per row: 18 blocks of 32
 *                    values, each an e2m1 element times its block's E8M0 scale 2^(E-127).
 *                    Bytes 16j..16j+15 hold block j's elements, element 2i in the low nibble
 *                    of byte 16j+i; bytes 288 + 4p .. 288 + 4p + 2 hold the scales of blocks
 *                    p, p + 8 and p + 16 (p < 8; the byte of a block >= 18 and every fourth
 *                    byte are ignored).  kv_scale must be NULL.  A block with scale byte 255
 *                    (NaN) makes the outputs of every query that selects its row NaN.
 *                    (The "DeepSeek-V2-Lite-Chat SIQ K4/K3" card,
 *                    "Measured", names an nvfp4 latent cache for sparse MLA on sparse-indexer
 *                    models; MXFP4 is the block-scaled fp4 that gfx950 converts natively, and
 *                    this byte layout is the library's.)
 */
typedef enum { DSA_KV_BF16 = 0, DSA_KV_FP8_E4M3 = 1, DSA_KV_MXFP4 = 2 } dsa_kv_dtype;

typedef enum {
  DSA_OP_SCORES = 0,
  DSA_OP_TOPK = 1,
  DSA_OP_ATTN = 2,
  DSA_OP_STACK = 3,
  DSA_OP_INDEX_TOPK = 4,
  DSA_OP_ATTN_PAGED = 5,
  DSA_OP_STACK_PAGED = 6,
  DSA_OP_INDEXER_KL = 7,      /* dsa_indexer_kl with index lists of shape k entries */
  DSA_OP_INDEXER_KL_DENSE = 8 /* dsa_indexer_kl over every causal key (idx NULL; k ignored) */
} dsa_op;

/* flags of dsa_layer_stack */
#define DSA_CACHE_PREFILLED 1u /* index_cache already holds indices: a leading 'S' may reuse them */
#define DSA_STACK_UNFUSED 2u   /* 'F' layers run dsa_index_scores + dsa_topk over score chunks
                                  even where the fused path of dsa_index_topk applies (same
                                  indices; for comparison) */
#define DSA_CACHE_TOPK_ROWS 4u /* with DSA_CACHE_PREFILLED: the prefilled rows are as dsa_topk
                                  writes them (each row's min(k, p+1) valid entries first,
                                  then -1), e.g. a previous stack's cache; attention then takes
                                  each row's extent from its position instead of scanning the
                                  row (any row otherwise is read entry by entry) */

int dsa_abi_version(void);
const char* dsa_last_error(void);
const char* dsa_status_string(dsa_status s);

/*
 * Lightning-indexer scores (step 1).
 *   q_idx  bf16 [B][Tq][H_I][d_I]  per-query indexer heads
 *   k_idx  bf16 [B][Tk][d_I]       one indexer key per token, shared by all heads
 *   w_idx  bf16 [B][Tq][H_I]       per-query head weights
 *   scores fp32 [B][Tq][ld], ld >= Tk: for every row, entries s = 0..p are written with
 *          I[t,s] (fp32 accumulation of the bf16 products, ReLU per head, then the weighted
 *          head sum in head order) and entries s = p+1 .. ld-1 (keys the query cannot see,
 *          then the padding past Tk) with -inf; every entry of every row is written.
 * Supported: H_I in {1,2,4,8,16}, d_I in {16,32,64,128}, ld <= 2^22.
 */
dsa_status dsa_index_scores(const void* q_idx, const void* k_idx, const void* w_idx,
                            const int32_t* kv_len, int B, int Tq, int Tk, int H_I, int d_I,
                            float* scores, int64_t ld, void* stream);

/*
 * Causal top-k (step 2).
 *   scores fp32 [B][Tq][ld]: only entries 0..p of each row are read.
 *   idx    int32 [B][Tq][k]: if p+1 <= k, the keys 0..p; otherwise the k keys of largest
 *          score, equal scores resolved toward the lower key index, -0.0 equal to +0.0;
 *          either way sorted ascending and padded with -1 up to k entries.
 * Scores must not be NaN.  Supported: 1 <= k <= 4096, Tk <= 65536 (rows kept in
 * registers) or Tk <= 2^24 (rows re-read per pass).
 *   ws     optional, 16-byte aligned, at least dsa_workspace_size(shape, DSA_OP_TOPK) bytes
 *          (shape fields used: B, Tq, Tk, k; nonzero only for fewer than 1024 rows of
 *          6145..65536 keys, about 128 KB per row).  With it such rows are split over the
 *          chip: per-segment candidate lists, then an exact merge per row that falls back to
 *          the whole row where the lists cannot decide; NULL runs one workgroup per row.
 *          idx is the same either way.  A non-NULL ws smaller than the size is
 *          DSA_ERR_WORKSPACE.
 */
dsa_status dsa_topk(const float* scores, int64_t ld, const int32_t* kv_len, int B, int Tq, int Tk,
                    int k, int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/*
 * Indexer scores and top-k in one call (steps 1 and 2 together).  idx is, bit for bit, what
 * dsa_index_scores followed by dsa_topk on its scores gives (same layouts and rules as
 * there), but where the fused path applies no score row is written: each wave scores a
 * sample of ~1/16 of its rows' keys, derives a per-row threshold expected to pass about
 * oversample*k keys, rescores every key and keeps only those at or above the threshold in a
 * per-row candidate list, from which an exact selection takes the top k.  A row whose list
 * ends up shorter than k or longer than its capacity (6144) is recomputed exactly, so the
 * result does not depend on the sample.
 *   oversample  expected candidates per row as a multiple of k (<= 0: the library default,
 *               min(4, max(1.25, 3379/k))); any value gives the same idx, only the speed
 *               differs.
 *   idx         int32 [B][Tq][k]
 *   ws          at least dsa_workspace_size(shape, DSA_OP_INDEX_TOPK) bytes (shape fields
 *               used: B, Tq, Tk, H_I, d_I, k): sample keys, thresholds and candidate lists
 *               (about 64 KB per query row at Tk = 65536), or, where the fused path does not
 *               apply, one chunk of score rows.
 * Supported: the shapes of dsa_index_scores with 1 <= k <= 4096.  The fused path runs for
 * H_I in {8, 16} with at least 1024 query rows in all (B*Tq) and Tk > 6144 (shorter rows keep
 * every key, and score rows are then the cheaper hand-over); other shapes run the two steps
 * over chunks of score rows in the workspace.
 */
dsa_status dsa_index_topk(const void* q_idx, const void* k_idx, const void* w_idx,
                          const int32_t* kv_len, int B, int Tq, int Tk, int H_I, int d_I, int k,
                          float oversample, int32_t* idx, void* ws, size_t ws_bytes,
                          void* stream);

/*
 * Attention restricted to the selected keys (step 3).
 *   q     bf16 [B][Tq][H][Dqk]
 *   kv    [B][Tk][Hkv][row], row = Dqk bf16 (DSA_KV_BF16), Dqk e4m3 bytes (DSA_KV_FP8_E4M3)
 *         or Dqk/2 + 32 MXFP4 bytes (DSA_KV_MXFP4), see dsa_kv_dtype
 *   kv_scale fp32 [B][Tk] for fp8 (key row value = e4m3 value * kv_scale[b][s]); else NULL
 *   v     bf16 [B][Tk][Hkv][Dv], or NULL: V is kv[..., 0:Dv] (MLA shared latent row)
 *   idx   int32 [B][Tq][k]: key indices per query row, shared by all heads; entries
 *         outside [0, Tk) (e.g. the -1 padding) are skipped, and a key listed twice is two
 *         terms of the softmax sum
 *   out   bf16 [B][Tq][H][Dv] = sum_s softmax_s(sm_scale * q[h].K[s]) V[s] over valid s
 *         (0 for a row with no valid entry); head h reads kv head h*Hkv/H
 *   lse   fp32 [B][Tq][H] natural-log sum-exp of the scaled logits (-inf if none), or NULL
 *   ws    device workspace of at least dsa_workspace_size(shape, DSA_OP_ATTN) bytes (may be
 *         NULL when that size is 0); used for split-key partial results
 * Supported: MLA (Hkv = 1, Dqk = 576, Dv = 512, v = NULL, H a multiple of 16, any row format,
 * Tk * row bytes <= 2^32 - 4096) and multi-head (Hkv = H <= 16, Dqk = Dv = 32, bf16, v given);
 * 1 <= k <= 65536.
 */
dsa_status dsa_sparse_attn(const void* q, const void* kv, const float* kv_scale, const void* v,
                           dsa_kv_dtype kv_dtype, const int32_t* idx, int B, int Tq, int Tk, int H,
                           int Hkv, int Dqk, int Dv, int k, float sm_scale, void* out, float* lse,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * Indexer training objective: the indexer is trained with a KL loss against the detached
 * main attention distribution, dense attention first ("DSA ablation model card", model list).
 * The card gives no formula; per query row t (position p) with key set S (the valid entries
 * of idx[b][t]; every key 0..p when idx is NULL, the dense warm-up):
 *   P_s = (1/H) sum_h softmax_{s in S}(sm_scale * q[h] . k[s][h])     target, held fixed
 *   Q_s = softmax_{s in S}(I_s), I_s the indexer score of dsa_index_scores
 *   loss[b][t] = sum_s P_s (ln P_s - ln Q_s)
 * and the gradients of sum(loss) with respect to the indexer inputs (ReLU'(0) = 0).
 *   q_idx, k_idx, w_idx  bf16, as in dsa_index_scores
 *   q     bf16 [B][Tq][H][Dqk], k bf16 [B][Tk][H][Dqk]: the main attention's queries and
 *         keys (multi-head form, Dqk = 32)
 *   idx   int32 [B][Tq][kk] (entries outside [0, Tk) skipped; a duplicate counts twice), or
 *         NULL (kk ignored)
 *   loss  fp32 [B][Tq] (0 for a row with no key)
 *   dq_idx fp32 [B][Tq][H_I][d_I], dw_idx fp32 [B][Tq][H_I], dk_idx fp32 [B][Tk][d_I]: each
 *         may be NULL (not computed).  dk_idx is overwritten.  Every output is deterministic,
 *         bit for bit: dk_idx adds, for each key, the terms of the rows that list it in row
 *         order (then list order), through the workspace.
 *   ws    with dk_idx, at least dsa_workspace_size(shape, DSA_OP_INDEXER_KL) bytes (index
 *         lists; shape.k = kk) or DSA_OP_INDEXER_KL_DENSE (idx NULL), 256-byte aligned; the
 *         shape fields read are B, Tq, Tk, H_I (and k).  It holds every entry's head terms
 *         (B Tq kk H_I floats, or B Tq Tk H_I dense) and, for index lists, the key sort
 *         (16 bytes per entry plus per-key offsets).  Unused without dk_idx (may be NULL).
 * Supported: 1 <= H_I <= 16, d_I in {16, 32, 64, 128}, 1 <= H <= 16, Dqk = 32; at most 4096
 * keys per row (kk <= 4096, or Tk <= 4096 without idx); with dk_idx, B Tk and B Tq kk below
 * 2^31 - 1.
 */
dsa_status dsa_indexer_kl(const void* q_idx, const void* k_idx, const void* w_idx, const void* q,
                          const void* k, const int32_t* idx, const int32_t* kv_len, int B, int Tq,
                          int Tk, int H_I, int d_I, int H, int Dqk, int kk, float sm_scale,
                          float* loss, float* dq_idx, float* dw_idx, float* dk_idx, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * Paged caches, for serving batches (the pages serve many sequences at once through vLLM
 * with an fp8 KV cache, "DeepSeek-V2-Lite-Chat SIQ K4/K3" card, "How to run"; they do not
 * describe a page layout, so this one is the library's): token s of sequence b is row
 *     block_table[b][s / page_size] * page_size + s % page_size
 * of a pool shared by all sequences, each row laid out as in the dense calls.  Table entries
 * past a sequence's length are never used for its keys (they may hold anything); a row the
 * table places outside the pool is treated as absent.
 */
typedef struct {
  const int32_t* block_table; /* device int32 [B][max_blocks] */
  int max_blocks;             /* table entries per sequence; max_blocks * page_size >= Tk */
  int page_size;              /* tokens per page: a power of two, 32 .. 65536 */
  int num_pages;              /* pages in each pool */
} dsa_paged_kv;

/*
 * dsa_index_scores with the indexer keys in a paged pool:
 *   k_pool bf16 [num_pages * page_size][d_I]; other arguments and results as there (Tk = the
 *   longest sequence; kv_len gives each sequence's length; -inf past each row's last key).
 *   Same scores, bit for bit.
 * Supported: as dsa_index_scores, and num_pages * page_size * d_I * 2 < 2^32 bytes.
 */
dsa_status dsa_index_scores_paged(const void* q_idx, const void* k_pool, const void* w_idx,
                                  const dsa_paged_kv* pages, const int32_t* kv_len, int B, int Tq,
                                  int Tk, int H_I, int d_I, float* scores, int64_t ld, void* stream);

/*
 * dsa_sparse_attn (MLA form) with the latent rows in a paged pool:
 *   kv_pool        [num_pages * page_size][row], rows as in dsa_sparse_attn (bf16, e4m3 or
 *                  MXFP4)
 *   kv_scale_pool  fp32 [num_pages * page_size] for fp8 (NULL otherwise)
 *   idx            int32 [B][Tq][k] key positions (as from dsa_topk); entries outside
 *                  [0, kv_len[b]) are skipped
 *   ws             at least dsa_workspace_size(shape, DSA_OP_ATTN_PAGED) bytes: the pool rows
 *                  of the selected keys plus the attention workspace
 * Same outputs, bit for bit, as dsa_sparse_attn on the dense cache holding the same rows.
 * Supported: MLA (H a multiple of 16, Dqk = 576, Dv = 512); pools of fewer than 2^24 rows and
 * at most 2^32 - 4096 bytes.
 */
dsa_status dsa_sparse_attn_paged(const void* q, const void* kv_pool, const float* kv_scale_pool,
                                 dsa_kv_dtype kv_dtype, const dsa_paged_kv* pages,
                                 const int32_t* idx, const int32_t* kv_len, int B, int Tq, int Tk,
                                 int H, int Dqk, int Dv, int k, float sm_scale, void* out,
                                 float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * dsa_sparse_attn for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same arguments and
 * results without ws / ws_bytes.  The split-key partial results that few-row (decode)
 * shapes need go to a scratch area built into the library, one per device, held from the
 * library's load until the process ends; the call itself never allocates.  The shapes that
 * need no workspace (dsa_workspace_size(shape, DSA_OP_ATTN) == 0) use none.
 *   Limit: dsa_noalloc_scratch_bytes() bytes (8.4 MB) of partial results, i.e. the
 *   workspace dsa_sparse_attn would take for the shape; the library splits keys so that
 *   splits x (row, 16-head group) pairs stay within 256, which keeps every shape's partials
 *   within that size (8.4 MB for 64 decode rows of 16 heads at k = 2048).  A larger need
 *   would return DSA_ERR_UNSUPPORTED with nothing enqueued.
 *   Every call on one device shares that device's scratch and overwrites it: calls whose
 *   work overlaps on one device (different streams, or host threads without ordering)
 *   race and give undefined outputs.  Calls ordered on one stream are safe.
 * Outputs equal dsa_sparse_attn's for the same inputs, bit for bit.
 */
dsa_status dsa_sparse_attn_noalloc(const void* q, const void* kv, const float* kv_scale, const void* v,
                                   dsa_kv_dtype kv_dtype, const int32_t* idx, int B, int Tq, int Tk,
                                   int H, int Hkv, int Dqk, int Dv, int k, float sm_scale, void* out,
                                   float* lse, void* stream);
size_t dsa_noalloc_scratch_bytes(void);

/* Shape of one layer of a stack (all layers share it). */
typedef struct {
  int B, Tq, Tk;        /* sequences, query rows per sequence, keys per sequence */
  int H_I, d_I;         /* indexer heads and width */
  int H, Hkv, Dqk, Dv;  /* attention heads, kv heads, q/k width, v width */
  int k;                /* top-k budget */
  float sm_scale;       /* softmax scale (e.g. 1/sqrt(Dqk)); not fixed by the pages */
  dsa_kv_dtype kv_dtype;
  const int32_t* kv_len; /* device int32[B] or NULL */
} dsa_shape;

/* Per-layer tensors (layouts as in the calls above).  q_idx/k_idx/w_idx are read on 'F'
 * layers only and may be NULL on 'S' layers. */
typedef struct {
  const void* q_idx;
  const void* k_idx;
  const void* w_idx;
  const void* q;
  const void* kv;
  const float* kv_scale;
  const void* v;
  void* out;
  float* lse;
} dsa_layer_io;

/*
 * IndexCache layer stack (step 4 around steps 1-3).
 *   pattern  host string of n_layers characters, 'F' (full) or 'S' (shared)
 *   layers   host array [n_layers]
 *   index_cache int32 [B][Tq][k] device buffer handed down the stack: an 'F' layer overwrites
 *            it with its own top-k indices, every layer then attends with it as it stands.
 *            A leading 'S' is rejected unless flags has DSA_CACHE_PREFILLED.
 *   ws       at least dsa_workspace_size(shape, DSA_OP_STACK) bytes: what the 'F' layers'
 *            dsa_index_topk needs (or one chunk of score rows, whichever is larger: the full
 *            Tq x Tk score matrix is never held) plus four layers' attention workspace (with
 *            few query rows, up to four consecutive layers that share the index cache run
 *            their attention in one launch).
 */
dsa_status dsa_layer_stack(const char* pattern, int n_layers, const dsa_layer_io* layers,
                           const dsa_shape* shape, int32_t* index_cache, unsigned flags, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * dsa_layer_stack over paged caches: each layer's k_idx is a key pool and kv / kv_scale a
 * latent pool (MLA form), all laid out by `pages` (one block table for every layer, as a
 * serving cache shares it across layers).  'F' layers score over the key pool and select as
 * dsa_topk does (score chunks); every layer attends through the pool rows of the cached
 * indices.  index_cache holds key positions, as in dsa_layer_stack, and the outputs equal
 * that call's on dense caches holding the same rows, bit for bit.
 *   ws  at least dsa_workspace_size(shape, DSA_OP_STACK_PAGED) bytes.
 */
dsa_status dsa_layer_stack_paged(const char* pattern, int n_layers, const dsa_layer_io* layers,
                                 const dsa_shape* shape, const dsa_paged_kv* pages,
                                 int32_t* index_cache, unsigned flags, void* ws, size_t ws_bytes,
                                 void* stream);

/* Workspace bytes an operation needs for `shape` (0 if none); 0 also for an invalid shape. */
size_t dsa_workspace_size(const dsa_shape* shape, dsa_op op);

/* Query rows per score chunk that dsa_layer_stack uses for `shape` (>= 1). */
int dsa_stack_chunk_rows(const dsa_shape* shape);

/* Check an F/S pattern: DSA_OK, or DSA_ERR_PATTERN (wrong length, a character other than
 * 'F'/'S', or a leading 'S' without DSA_CACHE_PREFILLED). */
dsa_status dsa_check_pattern(const char* pattern, int n_layers, unsigned flags);

/* The pattern of index_topk_freq = freq ("compute on 1/freq of layers", IndexCache doc,
 * "Configuration Reference"): layer i is 'F' iff i % freq == 0.  out: n_layers + 1 chars
 * (NUL-terminated).  freq = 1 gives all 'F' (IndexCache off). */
dsa_status dsa_pattern_from_freq(int freq, int n_layers, char* out);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
