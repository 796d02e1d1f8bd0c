/* Plain CPU oracle of the DSA hot path (test infrastructure only; see dsa_oracle.c).
 * All tensors are dense row-major; bf16 values are passed as their uint16 bit patterns,
 * fp8 values as OCP e4m3 bytes.  Every function returns 0 on success, nonzero on a bad
 * argument.  `kv_len` may be NULL (every sequence holds Tk keys). */
#ifndef DSA_ORACLE_H
#define DSA_ORACLE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif
double oracle_bf16_to_double(uint16_t h);
double oracle_e4m3_to_double(uint8_t b);
double oracle_e2m1_to_double(uint8_t c);
double oracle_e8m0_to_double(uint8_t e);
int64_t oracle_mxfp4_row_bytes(int D);
double oracle_mxfp4_value(const uint8_t* row, int D, int d);
/* q [B][Tq][H][D], k [B][Tk][D], w [B][Tq][H] -> scores float [B][Tq][ld] */
int oracle_index_scores(const uint16_t* q, const uint16_t* k, const uint16_t* w,
                        const int32_t* kv_len, int B, int Tq, int Tk, int H, int D,
                        float* scores, int64_t ld, int nthreads);
/* scores [B][Tq][ld] -> idx int32 [B][Tq][k] (ascending, -1 padded) */
int oracle_topk(const float* scores, int64_t ld, const int32_t* kv_len, int B, int Tq, int Tk,
                int k, int32_t* idx, int nthreads);
/* q bf16 [B][Tq][H][Dqk]; kv (kv_fmt 0) bf16 [B][Tk][Hkv][Dqk], (1) e4m3 [B][Tk][Hkv][Dqk]
 * with kv_scale [B][Tk], (2) MXFP4 rows [B][Tk][Hkv][Dqk/2 + 32] bytes (kv_scale NULL);
 * v bf16 [B][Tk][Hkv][Dv] or NULL (V = kv[..., :Dv]); idx [B][Tq][k]
 * -> out double [B][Tq][H][Dv], lse double [B][Tq][H] (may be NULL) */
int oracle_sparse_attn(const void* q, const void* kv, const float* kv_scale, const void* v,
                       int kv_fmt, const int32_t* idx, int B, int Tq, int Tk, int H, int Hkv,
                       int Dqk, int Dv, int k, double sm_scale, double* out, double* lse,
                       int nthreads);
/* Rows `rows[0..nrows)` of one prefill sequence (query t sees keys 0..t), streamed row by
 * row through scores, top-k and MLA attention (Hkv = 1, V = kv[..., :Dv]). */
int oracle_dsa_rows(const uint16_t* q_idx, const uint16_t* k_idx, const uint16_t* w_idx,
                    const uint16_t* q, const void* kv, const float* kv_scale, int kv_fmt,
                    const int32_t* rows, int nrows, int Tk, int H_I, int d_I, int H, int Dqk,
                    int Dv, int k, double sm_scale, int32_t* idx_out, double* out, int nthreads);
/* Indexer KL objective (see dsa_oracle.c): q_idx [B][Tq][H_I][d_I], k_idx [B][Tk][d_I],
 * w_idx [B][Tq][H_I], q [B][Tq][H][Dqk], k [B][Tk][Hkv][Dqk] (main attention keys), idx
 * [B][Tq][kk] or NULL (every causal key) -> loss [B][Tq], dq_idx, dw_idx (shapes of the
 * inputs) and dk_idx [B][Tk][d_I], all double.  The _f64 form takes doubles. */
int oracle_indexer_kl_f64(const double* q_idx, const double* k_idx, const double* w_idx,
                          const double* q, const double* k, const int32_t* kv_len,
                          const int32_t* idx, int B, int Tq, int Tk, int H_I, int d_I, int H,
                          int Hkv, int Dqk, int kk, double sm_scale, double* loss,
                          double* dq_idx, double* dw_idx, double* dk_idx, int nthreads);
int oracle_indexer_kl(const uint16_t* q_idx, const uint16_t* k_idx, const uint16_t* w_idx,
                      const uint16_t* q, const uint16_t* k, const int32_t* kv_len,
                      const int32_t* idx, int B, int Tq, int Tk, int H_I, int d_I, int H, int Hkv,
                      int Dqk, int kk, double sm_scale, double* loss, double* dq_idx,
                      double* dw_idx, double* dk_idx, int nthreads);
#ifdef __cplusplus
}
#endif
#endif
