/*
 * CPU oracle for absorbed-MLA tree-verify attention over a page_size=1 latent pool.
 *
 * TEST INFRASTRUCTURE ONLY. This is the plain, slow, obviously-correct definition
 * that the GPU path is checked against. Only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg may load it. It shares no code, header, table
 * or helper with the HIP library.
 *
 * What it computes, for every sequence b, tree node i and head h:
 *   visible set  V(b,i) = { p : 0 <= p < S_b - N }                      (prefix)
 *                       u { S_b - N + j : bit j of tree_mask[b][i] set } (tree)
 *   score        s_p    = scale * sum_{d<576} q[b,i,h,d] * pool[page_table[b,p], d]
 *   lse                 = ln sum_{p in V} exp(s_p)
 *   out[c]              = sum_{p in V} exp(s_p - lse) * pool[page_table[b,p], c],  c < 512
 * The pages fix the ingredients: a per-token gather through a page table
 * ("The 130x Slowdown", The Reasoning, step 4), one compressed latent per token
 * serving as key and value (same page, The Technical Depth), a prefix that needs
 * no mask and a small tree block that does ("The Moment of Certainty", The Path
 * Forward), and a tree visibility bitmask ("The GPU That Wasn't There", The Native
 * Engine Thesis). The 512 + 64 split, the scale and the LSE output are the
 * problem statement's.
 *
 * Arithmetic: bf16 inputs are widened exactly; scores, softmax and the weighted
 * sum are taken in IEEE double in plain ascending order (built without FMA
 * contraction or reassociation). out is rounded once, double -> bf16, to nearest
 * even; lse is rounded double -> float. An empty visible set gives out = 0 and
 * lse = -inf.
 */
#ifndef MTV_ORACLE_H
#define MTV_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes */
#define MTV_ORACLE_OK 0
#define MTV_ORACLE_ERR_ARG -1     /* null pointer or bad shape */
#define MTV_ORACLE_ERR_SEQLEN -2  /* seq_lens[b] outside [N, max_kv] */
#define MTV_ORACLE_ERR_INDEX -3   /* a referenced page index outside [0, num_slots) */
#define MTV_ORACLE_ERR_NOMEM -4

/*
 * q          bf16 bits [B][N][H][576]
 * kv_pool    bf16 bits [num_slots][576]
 * page_table int32     [B][max_kv]
 * seq_lens   int32     [B]
 * tree_mask  uint32    [B][N][W], W = ceil(N/32)
 * rows       optional list of nrows flat row ids r = (b*N + i)*H + h to compute;
 *            NULL computes every row (nrows ignored)
 * out_bf16   bf16 bits [B][N][H][512]   (rows not computed are left untouched)
 * lse_f32    float     [B][N][H]
 * out_f64, lse_f64: optional (may be NULL) unrounded results, same shapes
 * threads    worker threads over rows (<= 0: one)
 */
int mtv_oracle_run(int B, int N, int H, int max_kv, int64_t num_slots,
                   const uint16_t* q, const uint16_t* kv_pool,
                   const int32_t* page_table, const int32_t* seq_lens,
                   const uint32_t* tree_mask, double scale,
                   const int64_t* rows, int64_t nrows,
                   uint16_t* out_bf16, float* lse_f32,
                   double* out_f64, double* lse_f64, int threads);

/* Round-to-nearest-even of a double to bf16 bits (exposed for its own tests). */
uint16_t mtv_oracle_f64_to_bf16(double x);

/* Exact widening of bf16 bits to double. */
double mtv_oracle_bf16_to_f64(uint16_t x);

#ifdef __cplusplus
}
#endif
#endif
