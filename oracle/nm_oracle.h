/*
 * nm_oracle.h -- CPU oracle for N:M magnitude masking, compression and the
 * compressed-sparse x dense product.
 *
 * TEST INFRASTRUCTURE ONLY.  This is a plain, slow, single-threaded C99
 * implementation written from the definitions on the source pages.  It shares
 * no code, header, table or constant with the GPU library; only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load it.
 *
 * Sources (cited by page title and section):
 *   [SRSTE]  "量化友好的SR-STE稀疏化训练" (blog.bakeneko-kuro.com)
 *            - section "概念": N:M means N non-zero among every M consecutive weights.
 *            - section "NVIDA Apex内的静态掩码稀疏": ASP's m4n2_1d / mn_1d_best
 *              scores every valid N-of-M pattern by the L1 norm of the weights it
 *              keeps and takes the best pattern per group of M along the last,
 *              contiguous dimension.
 *            - section "基于直通估计的动态掩码精炼化稀疏(SR-STE)": the mask is
 *              recomputed from |w| at every forward step, the layer uses weight
 *              times mask, and the backward returns grad + decay*(1-mask)*weight
 *              (decay 0.0002 by default).
 *   [ASDNN]  "[리뷰] Accelerating Sparse Deep Neural Networks" (moon-walker.medium.com)
 *            - section "2:4 Sparsity의 benefits": compressed matrix of R*C/2 values,
 *              2-bit position metadata per kept value, always N values stored per
 *              group; 4 fp16 values take 36 bits instead of 64.
 *            - section "Tensor Scores 상에서 구조적인 sparse GEMM": sparse (first,
 *              compressed) operand times dense operand gives a dense result.
 *            - section "Step-2: Weight Pruning": drop the two smallest of each four;
 *              permute the weight's columns first (Fig. 6) so that large values spread
 *              over the groups and the mask keeps a larger total (83.7 -> 102.9 in the
 *              figure's example, whose matrix is not given).
 *   [TRANS]  "[论文解读] Accelerated Sparse Neural Training: A Provable and Efficient
 *            Method to Find N:M Transposable Masks" (nubint.ai)
 *            - ABSTRACT and section "提出的方法": a transposable mask makes W and its
 *              transpose follow the same N:M pattern, chosen per M x M block to
 *              maximise the kept L1 norm with N per row and column; the optimum is a
 *              minimum-cost flow, the fast method a greedy 2-approximation.
 *
 * Readings where the pages are silent:
 *   - N counts KEPT elements; exactly N values are stored per group.
 *   - Ties between equally good patterns go to the lexicographically first
 *     ascending index tuple (lower index wins).
 *   - Pattern scores are summed EXACTLY (integer arithmetic), not in fp32.
 *   - |w| is ordered by the format's bits with the sign cleared; the exact
 *     magnitude of an Inf/NaN bit pattern continues that integer order
 *     (so NaN ranks above Inf, Inf above every finite value).
 *   - Metadata: b = log2(M) bits per kept value; field f = g*N + j of a row
 *     (j-th kept index of group g, ascending) sits at bit f*b of the row's
 *     uint32 bitstream, least significant bit first; every row starts on a
 *     word boundary; pad bits are zero.
 *   - Decompression writes +0 (all-zero bits) at pruned positions.
 *   - SR-STE's masked weight (weight times mask) is a selection: kept elements
 *     bit for bit, +0 at pruned ones (the decompression rule).  Its mask is the
 *     same best-pattern mask (the printed argsort leaves ties open).
 *   - SR-STE's gradient is G bit for bit where the weight is kept (the decay
 *     term is zero there); where it is pruned it is fl32(fl32(decay*w) + g),
 *     rounded once more to the element type, in the printed backward's order.
 *   - Channel permutation: the objective is the kept L1 of the N:M mask of W with
 *     its columns permuted (only group membership matters).  The search, which the
 *     pages leave open, runs rounds: every pair of groups gets its best single
 *     column swap (largest kept-L1 gain summed over all rows, first (a, b) on ties);
 *     positive gains are applied in descending order (ties: smaller group indices),
 *     each group at most once per round; it stops when a round applies nothing.
 *   - Transposable masks: M x M blocks aligned at multiples of M (R and K must be
 *     multiples of M).  The greedy takes a block's entries by descending exact
 *     magnitude, equal magnitudes in ascending row-major position, and keeps an
 *     entry while its row and its column hold fewer than N; rows and columns can
 *     end with fewer than N kept (at least M-N zeros, the review's own count).
 *
 * Conventions: every matrix is dense row-major; W is R x K with groups along
 * K; values R x (K*N/M); meta R x words_per_row uint32; X K x T; Y R x T.
 * Element types: dt = 0 (fp32), 1 (fp16), 2 (bf16), 3 (int8); 16-bit types are
 * passed as raw uint16 bit patterns, int8 as raw bytes.  int8 (the ASDNN review's
 * INT8 sparse Tensor Core type, "Tensor Scores 상에서 구조적인 sparse GEMM") takes |w|
 * as the integer magnitude (|-128| = 128) and is accepted by mask, compress,
 * decompress and the products, whose double sums are then exact integers.  FP8 (dt 4,
 * OCP E4M3 bytes) is ranked by its sign-cleared bits like the other floating types
 * and is accepted by the same four functions.  Return value 0 = success, negative = bad args.
 */
#ifndef NM_ORACLE_H
#define NM_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NMO_F32 0
#define NMO_F16 1
#define NMO_BF16 2
#define NMO_I8 3 /* int8 two's complement; products are exact integers */
#define NMO_FP8 4 /* OCP FP8 E4M3: bias 7, no infinities, S.1111.111 is NaN */

/* metadata bits per kept value, log2(m); -1 if m is not a power of two in [2,16] */
int nmo_meta_bits(int m);
/* uint32 words of metadata per row: ceil(K/m * n * b / 32) */
int64_t nmo_meta_words_per_row(int64_t K, int n, int m);

/* mask[r*K+k] = 1 if W[r,k] is kept, else 0 (exhaustive search over all patterns) */
int nmo_mask(const void* W, int dt, int64_t R, int64_t K, int n, int m, uint8_t* mask);

/* values (R x K*n/m, dtype dt) and meta (R x words_per_row) of W */
int nmo_compress(const void* W, int dt, int64_t R, int64_t K, int n, int m, void* values,
                 uint32_t* meta);

/* dense R x K matrix with the stored values at their positions and +0 elsewhere */
int nmo_decompress(const void* values, const uint32_t* meta, int dt, int64_t R, int64_t K, int n,
                   int m, void* W_out);

/* Y (R x T, double) = decompress(values, meta) * X, summed in double over ascending k */
int nmo_spmm(const void* values, const uint32_t* meta, int64_t R, int64_t K, int n, int m,
             const void* X, int64_t T, int dt, double* Y);

/* rows [r0, r1) of the product above, written to Y (R x T layout, only those rows touched) */
int nmo_spmm_rows(const void* values, const uint32_t* meta, int64_t R, int64_t K, int n, int m,
                  const void* X, int64_t T, int dt, int64_t r0, int64_t r1, double* Y);

/* out[i] = Y[rs[i], ts[i]] of the product above, one dot product per sample */
int nmo_spmm_sample(const void* values, const uint32_t* meta, int64_t R, int64_t K, int n, int m,
                    const void* X, int64_t T, int dt, const int64_t* rs, const int64_t* ts,
                    int64_t count, double* out);

/* W_out = W where kept, +0 where pruned (SR-STE forward weight) */
int nmo_prune(const void* W, int dt, int64_t R, int64_t K, int n, int m, void* W_out);

/* G_out = G where W is kept; fl32(g + fl32(decay * w)) rounded to dt where pruned
 * (SR-STE backward) */
int nmo_srste_grad(const void* W, const void* G, int dt, int64_t R, int64_t K, int n, int m,
                   float decay, void* G_out);

/* transposable mask by the greedy 2-approximation (R % m == 0, K % m == 0) */
int nmo_tmask_greedy(const void* W, int dt, int64_t R, int64_t K, int n, int m, uint8_t* mask);

/* transposable mask of maximal kept L1 per block (minimum-cost flow, double costs);
 * *kept_l1 (if not NULL) receives the kept L1 norm summed over all blocks */
int nmo_tmask_optimal(const void* W, int dt, int64_t R, int64_t K, int n, int m, uint8_t* mask,
                      double* kept_l1);

/* W where the greedy transposable mask keeps it, +0 elsewhere */
int nmo_tprune(const void* W, int dt, int64_t R, int64_t K, int n, int m, void* W_out);

/* kept L1 of the N:M mask of W with its columns permuted (perm[i] = column at
 * position i); -1 for bad arguments */
double nmo_kept_l1(const void* W, int dt, int64_t R, int64_t K, int n, int m,
                   const int32_t* perm);

/* best swap gain and choice (a*m + b) for every pair of groups g1 < g2 ((K/m)^2 tables) */
int nmo_perm_gains(const void* W, int dt, int64_t R, int64_t K, int n, int m,
                   const int32_t* perm, double* gain, int32_t* pick);

/* rounds of disjoint best swaps, at most max_rounds; perm updated in place */
int nmo_perm_search(const void* W, int dt, int64_t R, int64_t K, int n, int m, int max_rounds,
                    int32_t* perm, int* rounds_done);

/* out[i] = in[i] rounded to dt (round to nearest, ties to even; fp32 copies) */
int nmo_round_from_f32(const float* in, int dt, int64_t count, void* out);

/* exact value of one element as a double (helper used by the Python side of the oracle) */
double nmo_to_double(const void* p, int dt, int64_t i);

#ifdef __cplusplus
}
#endif
#endif
