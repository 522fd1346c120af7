/*
 * nm.h -- C ABI of libnm: N:M magnitude masking, compression and the
 * compressed-sparse x dense product on AMD Instinct MI355X (gfx950).
 *
 * Plain C; no HIP or PyTorch types appear in the signatures.  Pointer arguments
 * are DEVICE pointers to memory the caller owns, except where a declaration says
 * host memory (nm_perm_search's permutation, nm_check_meta's metadata).  The
 * library's state is a once-initialised record of which devices it has checked and,
 * per device, the fixed scratch buffer of nm_perm_gains_static.  It allocates no
 * device memory, with one exception: nm_spmm takes a workspace from the
 * stream-ordered pool (hipMallocAsync, freed in stream order) when the environment
 * variable NM_SPMM_TILE=3 forces its split schedule onto a shape whose 256 x 256 tiles
 * do not divide evenly over the compute units.  Calls are asynchronous on `stream` (a
 * hipStream_t passed as void*, NULL = the default stream): NM_OK means the
 * work was enqueued, and a fault inside a kernel surfaces at the caller's next
 * synchronisation.  Arguments are validated before anything is launched; on
 * any error nothing is written.  Outputs must not alias inputs.
 *
 * Element types: nm_mask, nm_compress, nm_mask_compress, nm_decompress and nm_spmm take
 * NM_F32, NM_F16, NM_BF16, NM_I8 and NM_FP8; the SR-STE and transposable-mask calls take the three
 * 16/32-bit floating-point types only.
 *
 * Dense arrays (row-major, no padding between rows):
 *   W      R x K            elements of `dt`; groups are M consecutive elements along K
 *   mask   R x K            uint8, 1 = kept, 0 = pruned
 *   X      K x T            elements of `dt`
 *   Y      R x T            elements of `y_dt`
 *
 * The compressed pair (values, meta) is stored in one of two layouts:
 *
 *   NM_LAYOUT_ROWS -- the plain format.
 *     values R x (K*N/M)    elements of `dt`; the N kept values of each group, in
 *                           ascending position order, groups in order along the row
 *     meta   R x words      uint32; see nm_meta_words_per_row
 *
 *   NM_LAYOUT_BLOCKED -- the same bytes regrouped in the order the sparse product
 *     streams them (K must be a multiple of 64).  Rows are taken in groups of 16
 *     (G = ceil(R / 16); rows R .. 16G-1 are stored as zeros) and K in steps of
 *     64 (S = K / 64).  Per row and step there are V = 64*N/M values and
 *     B = V*b/8 metadata bytes (b bits per field as below; B is always whole).
 *     Block (g, s) holds rows 16g .. 16g+15 of step s, row after row:
 *       value j (0 <= j < V) of row 16g+r, step s, is element
 *         ((g*S + s)*16 + r)*V + j        of values
 *         = element (16g+r)*(K*N/M) + s*V + j of the ROWS values;
 *       metadata byte i (0 <= i < B) of row 16g+r, step s, is byte
 *         ((g*S + s)*16 + r)*B + i        of meta
 *         = byte s*B + i of row 16g+r's ROWS bitstream (bits 8(s*B+i) .. +7).
 *     values has G*16*(K*N/M) elements, meta G*16*S*B bytes (a multiple of 4).
 *     With 16-bit values and N/M = 1/2 one block of values is 1 KB and one block
 *     of metadata 128 (2:4) or 64 (1:2) bytes, each a single contiguous read.
 *
 * Sources, cited by page title and section:
 *   "量化友好的SR-STE稀疏化训练" (blog.bakeneko-kuro.com), section "概念" (N:M keeps
 *   N non-zero weights in every M consecutive ones) and section "NVIDA Apex内的静态
 *   掩码稀疏" (ASP's exhaustive search: score every N-of-M pattern by the L1 norm of
 *   the weights it keeps, take the best per group of M along the contiguous dim).
 *   "[리뷰] Accelerating Sparse Deep Neural Networks" (moon-walker.medium.com),
 *   section "2:4 Sparsity의 benefits" (R*C/2 value array plus 2 bits of position
 *   per value; N values stored per group even when it holds more zeros) and
 *   section "Tensor Scores 상에서 구조적인 sparse GEMM" (sparse first operand,
 *   compressed by the application, times a dense operand gives a dense result;
 *   16-bit inputs and outputs, fp32 only in a reduced mode).
 *   "量化友好的SR-STE稀疏化训练", section "基于直通估计的动态掩码精炼化稀疏(SR-STE)"
 *   (the mask is searched again from the weights at every training step; the
 *   backward adds decay * w to the gradient where the mask prunes w).
 *   "[리뷰] Accelerating Sparse Deep Neural Networks", section "Step-2: Weight Pruning",
 *   Fig. 6 (permuting W's columns before the mask keeps a larger total magnitude).
 *   "[论文解读] Accelerated Sparse Neural Training: A Provable and Efficient Method
 *   to Find N:M Transposable Masks", ABSTRACT and section "提出的方法" (one mask per
 *   M x M block with N kept per row and column serves W and its transpose; a
 *   greedy 2-approximation finds it in near-linear time).
 */
#ifndef NM_H
#define NM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NM_ABI_VERSION 10

/* The enumerations are int-sized in C and C++ alike.  In C++ they are declared with int
 * as their underlying type, so that an out-of-range value a caller passes (an unknown
 * dtype, layout or status code) is a valid value the checks reject, not undefined
 * behaviour. */
#ifdef __cplusplus
#define NM_INT_ENUM : int
#else
#define NM_INT_ENUM
#endif

typedef enum NM_INT_ENUM {
  NM_OK = 0,
  NM_ERR_NULL = 1,        /* a required pointer is NULL                              */
  NM_ERR_SHAPE = 2,       /* negative size, K not a multiple of M, or R*K >= 2^36    */
  NM_ERR_PATTERN = 3,     /* N:M outside 1 <= N <= M, M in {2, 4, 8}                 */
  NM_ERR_DTYPE = 4,       /* unknown dtype, y_dt not allowed for dt, or int8 where a
                             floating-point weight is required                       */
  NM_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned                        */
  NM_ERR_UNSUPPORTED = 6, /* valid arguments the library has no kernel for (int8 and fp8 
                             in the blocked layout need 16 n / m divisible by 4)     */
  NM_ERR_DEVICE = 7,      /* no usable gfx950 device, or the launch failed           */
  NM_ERR_LAYOUT = 8,      /* unknown layout, or NM_LAYOUT_BLOCKED with K % 64 != 0   */
  NM_ERR_ALIAS = 9,       /* an output overlaps an input it may not replace          */
  NM_ERR_SCRATCH = 10     /* the call needs more than the library's fixed device scratch
                             buffer (NM_STATIC_SCRATCH_BYTES)                         */
} nm_status;

/* NM_I8: int8 two's complement ("Tensor Scores 상에서 구조적인 sparse GEMM" lists INT8 among
 * the sparse product's input types), ranked by |w| as an integer (|-128| = 128).
 * NM_I32 is an output type only: the exact int32 result of an int8 product.
 * NM_FP8: OCP FP8 E4M3 bytes (bias 7, no infinities, S.1111.111 is NaN), ranked by the
 * sign-cleared bits like the other floating types; not one of the pages' types, the
 * same method one format narrower. */
typedef enum NM_INT_ENUM {
  NM_F32 = 0, NM_F16 = 1, NM_BF16 = 2, NM_I8 = 3, NM_I32 = 4, NM_FP8 = 5
} nm_dtype;

typedef enum NM_INT_ENUM { NM_LAYOUT_ROWS = 0, NM_LAYOUT_BLOCKED = 1 } nm_layout;

typedef void* nm_stream_t; /* a hipStream_t; NULL selects the default stream */

/* NM_ABI_VERSION of the loaded library. */
int nm_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* nm_status_str(nm_status s);

/* Bytes of the value array ("2:4 Sparsity의 benefits": the compressed weight keeps
 * n of every m values, an R x C*n/m array of the weight's type):
 * R * (K / m * n) * sizeof(dt) for NM_LAYOUT_ROWS, 16 * ceil(R / 16) * (K / m * n) *
 * sizeof(dt) for NM_LAYOUT_BLOCKED; 0 for invalid arguments. */
size_t nm_values_bytes(int64_t R, int64_t K, int n, int m, nm_dtype dt, nm_layout layout);

/* Bytes of the metadata array ("2:4 Sparsity의 benefits": position bits beside the
 * values): R * 4 * nm_meta_words_per_row(K, n, m) for
 * NM_LAYOUT_ROWS, 16 * ceil(R / 16) * (K / 64) * B for NM_LAYOUT_BLOCKED; 0 for
 * invalid arguments. */
size_t nm_meta_bytes(int64_t R, int64_t K, int n, int m, nm_layout layout);

/* Metadata words per row ("2:4 Sparsity의 benefits": 2 bits record the position of
 * each kept value among its group of 4; the same rule with log2(m) bits is this
 * library's reading for other m): ceil((K / m) * n * b / 32) with b = log2(m) bits per
 * kept value (1 for 1:2, 2 for 2:4, 3 for 4:8).  Field f = g*n + j of a row holds the
 * position (0..m-1) of the j-th kept value of group g at bit offset f*b of the
 * row's bitstream, least significant bit first (word f*b/32, bit f*b%32; a 3-bit
 * field may straddle two words).  Every row starts on a word boundary and unused
 * high bits are zero.  For 2:4 this makes each group one nibble i0 | i1 << 2.
 * Returns -1 for invalid arguments. */
int64_t nm_meta_words_per_row(int64_t K, int n, int m);

/* Debug check of compressed metadata, on the HOST (meta_host is host memory; nothing
 * runs on the GPU).  The product trusts its metadata ("Tensor Scores 상에서 구조적인
 * sparse GEMM": the application supplies the compressed operand), so a caller that builds
 * metadata itself can check it here first.  Well formed means: the n positions of every
 * group are strictly ascending, and the unused high bits of every NM_LAYOUT_ROWS row are
 * zero.  Returns -1 if all R rows are well formed; else the row-major index r * (K / m) + g
 * of the first malformed group (a row with non-zero padding bits counts as malformed at
 * its last group); -2 for invalid arguments (pattern, shape, layout, or a NULL pointer
 * with R * K > 0). */
int64_t nm_check_meta(const uint32_t* meta_host, int64_t R, int64_t K, int n, int m,
                      nm_layout layout);

/* Magnitude-best N:M mask of W ("NVIDA Apex内的静态掩码稀疏"): in every group of m
 * consecutive elements along K the n positions with the largest sum of |w| are
 * kept; equal sums go to the lexicographically first position tuple (lower
 * index wins).  |w| is compared exactly (as the sign-cleared bit pattern, which
 * also ranks NaN above Inf above every finite value).  Writes mask (R x K). */
nm_status nm_mask(const void* W, nm_dtype dt, int64_t R, int64_t K, int n, int m, uint8_t* mask,
                  nm_stream_t stream);

/* Mask and compress in one pass ("2:4 Sparsity의 benefits"): the kept values of
 * each group in ascending position order go to `values` (bitwise copies, so -0
 * stays -0) and their positions to `meta`, in `layout` (see above; the padding
 * rows of NM_LAYOUT_BLOCKED are written as zeros). */
nm_status nm_compress(const void* W, nm_dtype dt, int64_t R, int64_t K, int n, int m,
                      nm_layout layout, void* values, uint32_t* meta, nm_stream_t stream);

/* nm_mask and nm_compress in one pass over W: the mask (R x K, uint8, as nm_mask writes
 * it) and the compressed pair in `layout` (as nm_compress writes it).  The pages' mask
 * and compression are one search ("NVIDA Apex内的静态掩码稀疏" keeps the best pattern of
 * every group; "2:4 Sparsity의 benefits" stores its values and positions), so W is read
 * once.  No output may overlap W or another output (NM_ERR_ALIAS). */
nm_status nm_mask_compress(const void* W, nm_dtype dt, int64_t R, int64_t K, int n, int m,
                           nm_layout layout, uint8_t* mask, void* values, uint32_t* meta,
                           nm_stream_t stream);

/* Inverse of nm_compress ("2:4 Sparsity의 benefits": the position metadata is what
 * restores each stored value to its place in the dense row): W_out (R x K) gets each
 * stored value at its recorded position and +0 (all-zero bits) everywhere else, i.e.
 * select(mask, W, +0), this library's reading of the pages' masked weight W * mask.  The metadata is trusted: a
 * field that repeats a position within a group leaves the later value there. */
nm_status nm_decompress(const void* values, const uint32_t* meta, nm_dtype dt, int64_t R,
                        int64_t K, int n, int m, nm_layout layout, void* W_out,
                        nm_stream_t stream);

/* Y = W_sparse * X ("Tensor Scores 상에서 구조적인 sparse GEMM"): W_sparse is the
 * R x K matrix that (values, meta) encode, X is K x T, Y is R x T.  Products of 16- and
 * 32-bit inputs are accumulated in fp32 and rounded once to y_dt (round to nearest even); y_dt
 * must be dt or NM_F32.  For dt = NM_I8 (W and X int8) y_dt must be NM_I32 and Y is
 * the exact integer product (K < 2^17, else NM_ERR_SHAPE, so no sum can overflow).
 * For dt = NM_FP8, y_dt is NM_F32 or NM_BF16.  2:4 and 1:2 fp8 products on the 8-bit
 * structured-sparse matrix cores do NOT sum every product in fp32: the instruction adds
 * the products of each run of 16 consecutive K (of the dense row) in fixed point aligned
 * to the run's largest product, dropping bits below 2^(e - 13) where 2^e bounds that
 * product, and adds the run sums into fp32 accumulators; the element error is at most
 * sum over runs of 7 * 2^(e_run - 13) plus the fp32 summation bound of the run sums.
 * Every other fp8 pattern or shape sums in fp32 (one rounding to y_dt).  The
 * metadata is trusted (well-formedness is the caller's responsibility, as for any
 * compressed operand; nm_check_meta checks it on the host).  Every shape and pattern
 * is accepted.  Fastest: 2:4 or 1:2 (16-bit on the structured-sparse matrix cores,
 * int8 and fp8 on their 8-bit form), NM_LAYOUT_BLOCKED (NM_LAYOUT_ROWS runs at a lower
 * rate), K % 64 == 0 (K % 128 for 8-bit) and T % 8 == 0 (T % 16 for 8-bit); even T
 * runs on the same 16-bit kernels with narrower X loads; every other case runs on the
 * dense matrix cores over tiles expanded in LDS (8-bit elements widened exactly to bf16;
 * int8 sums exact). */
nm_status nm_spmm(const void* values, const uint32_t* meta, int64_t R, int64_t K, int n, int m,
                  nm_layout layout, const void* X, int64_t T, nm_dtype dt, void* Y,
                  nm_dtype y_dt, nm_stream_t stream);

/* SR-STE forward weight ("基于直通估计的动态掩码精炼化稀疏(SR-STE)"): the mask is
 * searched from W on every call (the nm_mask rule) and W_out (R x K, dt) gets W
 * where it is kept, bit for bit, and +0 where it is pruned -- the dense masked
 * weight of the forward step (nm_compress gives the same step in compressed form).
 * W_out may be W itself (in place); any other overlap returns NM_ERR_ALIAS.
 * W and W_out must be 16-byte aligned. */
nm_status nm_prune(const void* W, nm_dtype dt, int64_t R, int64_t K, int n, int m, void* W_out,
                   nm_stream_t stream);

/* SR-STE backward for the dense weights ("基于直通估计的动态掩码精炼化稀疏(SR-STE)"):
 * G (R x K, dt) is the gradient with respect to the masked weight; G_out gets
 *   G                      where W is kept (bit for bit),
 *   G + decay * W          where W is pruned,
 * the latter evaluated as one fp32 product decay * w, one fp32 sum with g (never
 * fused into one rounding), then one rounding to dt (nearest, ties to even).  The
 * mask is recomputed from W (the nm_mask rule), so W must be the weight of the
 * same step's forward.  The page's default decay is 0.0002.  G_out may be G
 * itself (in place); an output overlapping W, or G partially, returns
 * NM_ERR_ALIAS.  W, G and G_out must be 16-byte aligned. */
nm_status nm_srste_grad(const void* W, const void* G, nm_dtype dt, int64_t R, int64_t K, int n,
                        int m, float decay, void* G_out, nm_stream_t stream);

/* Transposable N:M mask ("Accelerated Sparse Neural Training ... N:M Transposable
 * Masks", "提出的方法"), greedy 2-approximation: W is cut into m x m blocks (R and K
 * must be multiples of m, else NM_ERR_SHAPE); in each block the entries are taken by
 * descending |w| (the nm_mask order: NaN > Inf > finite, equal magnitudes in
 * ascending row-major position within the block) and an entry is kept while its row
 * and its column of the block hold fewer than n kept entries.  Every row and column
 * of a block then keeps at most n (a row and a column can end with fewer), so W and
 * W^T both have at most n nonzeros in every group of m along their rows.  Writes
 * mask (R x K, uint8, 1 = kept); mask must not overlap W (NM_ERR_ALIAS). */
nm_status nm_tmask(const void* W, nm_dtype dt, int64_t R, int64_t K, int n, int m, uint8_t* mask,
                   nm_stream_t stream);

/* W_out (R x K, dt) = W where nm_tmask keeps it (bit for bit), +0 elsewhere: the weight
 * both products of a training step use.  nm_compress of W_out gives the forward
 * operand and nm_compress_t of W_out the backward one; both keep every nonzero of
 * W_out.  W_out may be W itself; any other overlap returns NM_ERR_ALIAS. */
nm_status nm_tprune(const void* W, nm_dtype dt, int64_t R, int64_t K, int n, int m, void* W_out,
                    nm_stream_t stream);

/* nm_compress of W's transpose, without forming it: W is R x K row-major; the output
 * describes the K x R matrix W^T, groups of m running along R (R % m == 0, else
 * NM_ERR_SHAPE; NM_LAYOUT_BLOCKED needs R % 64 == 0, else NM_ERR_LAYOUT).  values
 * and meta have the sizes nm_values_bytes(K, R, n, m, dt, layout) and
 * nm_meta_bytes(K, R, n, m, layout), and the layout of nm_compress for a K x R
 * matrix, so nm_spmm(values, meta, K, R, ..., dY, T, ...) computes W^T dY, the
 * backward product ("Tensor Scores 상에서 구조적인 sparse GEMM" with the transposed
 * operand).  NM_LAYOUT_BLOCKED is the fast path (row-contiguous reads of W, whole
 * 1 KB blocks written); NM_LAYOUT_ROWS is correct but slower.  values and meta must
 * not overlap W (NM_ERR_ALIAS). */
nm_status nm_compress_t(const void* W, nm_dtype dt, int64_t R, int64_t K, int n, int m,
                        nm_layout layout, void* values, uint32_t* meta, nm_stream_t stream);

/* Channel permutation ("Step-2: Weight Pruning", Fig. 6).  For a column permutation perm
 * (perm[i] = the column of W placed at position i; groups are positions g*m .. g*m+m-1)
 * the objective is the kept L1 of the N:M mask of W[:, perm]: the sum over rows and
 * groups of the n largest |w| (NaN counted as the largest).  These calls search for a
 * better perm by swapping columns between groups.  They take any nm_dtype of W except
 * NM_I32, need R*K < 2^31, and use a caller-provided device workspace of at least
 * nm_perm_workspace_bytes(R, K, n, m) bytes (16-byte aligned; contents are scratch). */
size_t nm_perm_workspace_bytes(int64_t R, int64_t K, int n, int m);

/* One round's evaluation.  perm: DEVICE int32[K], trusted to be a permutation.  For every
 * pair of groups g1 < g2 (G = K/m), gain[g1*G + g2] receives the largest change of the
 * kept L1 over the swaps of position a of g1 with position b of g2 (summed over the rows
 * in fp32), and pick[g1*G + g2] = a*m + b of the first such swap in row-major (a, b)
 * order; gain and pick are DEVICE arrays of G*G entries whose other entries are left as
 * they are. */
nm_status nm_perm_gains(const void* W, nm_dtype dt, int64_t R, int64_t K, int n, int m,
                        const int32_t* perm, float* gain, int32_t* pick, void* workspace,
                        size_t workspace_bytes, nm_stream_t stream);

/* Bytes of the fixed device scratch buffer behind nm_perm_gains_static: 64 MiB, held on
 * every device the library runs on (reserved when the library's device code is loaded
 * there) until the process ends. */
#define NM_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

/* nm_perm_gains without a workspace argument and without any device allocation, for
 * callers that cannot allocate device memory in the call (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same arguments, checks and
 * results as nm_perm_gains; the permuted fp32 copy of W is built in the library's
 * per-device static scratch buffer instead of a workspace, so R*K*4 rounded up to 256
 * bytes must not exceed NM_STATIC_SCRATCH_BYTES (R*K <= 16,777,216), else NM_ERR_SCRATCH.
 * The kernels run on the current device, and `stream` must belong to it (else
 * NM_ERR_DEVICE).  All calls on one device share its buffer, and each call overwrites
 * it before reading it: calls that overlap in time on one device (on different streams,
 * or from different host threads) race and must be ordered by the caller. */
nm_status nm_perm_gains_static(const void* W, nm_dtype dt, int64_t R, int64_t K, int n, int m,
                               const int32_t* perm, float* gain, int32_t* pick,
                               nm_stream_t stream);

/* The search: rounds of nm_perm_gains; each round applies the positive gains in
 * descending order (ties: smaller g1, then smaller g2), skipping a pair when either
 * group was already changed in that round, and the search stops when a round applies
 * nothing or after max_rounds rounds.  perm: HOST int32[K], the starting permutation on
 * entry (it must be one, else NM_ERR_SHAPE) and the result on return; *rounds (if not
 * NULL) receives the number of rounds that applied a swap.  The call returns when the
 * search is done (it synchronises `stream`); host scratch of O((K/m)^2) is allocated
 * for the call's duration. */
nm_status nm_perm_search(const void* W, nm_dtype dt, int64_t R, int64_t K, int n, int m,
                         int max_rounds, int32_t* perm, int* rounds, void* workspace,
                         size_t workspace_bytes, nm_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* NM_H */
