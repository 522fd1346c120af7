// nm_spmm_sk.hip -- the 2:4 16-bit product on large shapes: 256 x 256 tiles, one wave per
// SIMD, split over the compute units by K steps ("stream-K").
//
// The product is the one of "[리뷰] Accelerating Sparse Deep Neural Networks", section
// "Tensor Scores 상에서 구조적인 sparse GEMM": the compressed weight (2:4 values and 2-bit
// positions) times a dense K x T operand, accumulated in fp32.  On gfx950 the
// structured-sparse instruction v_smfmac_f32_32x32x32_{bf16,f16} takes each lane's stored
// values with a 16-bit index word whose 2-bit fields are exactly this library's 2:4
// metadata, so compressed rows reach the matrix cores unchanged.
//
// Why this kernel: a compute unit can hold at most 256 x 256 fp32 accumulators (four
// waves of 256 accumulator registers), and the direct global -> LDS path that feeds it
// moves about 64 bytes per clock.  A 256 x 128 tile needs ~68 bytes per clock at the
// matrix cores' rate; 256 x 256 needs ~50 (per 64-wide K step: 16 KB of values, 2 KB of
// metadata and 32 KB of X for 4 x 32 smfmac).  So each workgroup is four waves, one per
// SIMD, each owning 256 rows x 64 columns of the tile (eight 32-row A fragments, two
// 32-column B fragments per 32-wide K substep), and every wave issues its share of the
// direct loads.  A 3-stage LDS ring holds steps s .. s+2; one barrier per step, placed
// after the first substep, certifies step s+1 landed and frees the stage of step s.
//
// 256 x 256 tiles are few on the shapes where this matters (the 11008 x 4096 and
// 4096 x 11008 projections at 2048 columns give 344 and 128 tiles for 256 compute units),
// so the work is split by K steps: the (tile, step) pairs are one list, and workgroup w
// takes an equal contiguous run of it.  A tile cut between workgroups is finished by the
// workgroup that holds its first steps (at the end of its run); the others (each at the
// start of its run) write their fp32 partial sums to a workspace slot and raise a flag.
// The finisher adds the slots in workgroup order, so results do not depend on timing.  A
// finisher waits for a flag a bounded time only: if a contributor has not run (the grid
// did not fit the device at once), it computes the missing steps itself.
#include <atomic>

#include "nm_launch.h"
#include "nm_mfma.h"

namespace nm {
namespace {

constexpr int kSkBM = 256, kSkBN = 256, kSkStages = 3;
constexpr int kSkXRowBytes = kSkBN * 2;                      // 512
constexpr int kSkXChunks = kSkBN / 8;                        // 16-byte chunks per K row
constexpr int kSkXBytes = kKStep * kSkXRowBytes;             // 32 KB
constexpr int kSkABytes = kSkBM * 64;                        // 16 KB
constexpr int kSkMBytes = kSkBM * 8;                         // 2 KB
constexpr int kSkStageBytes = kSkXBytes + kSkABytes + kSkMBytes;
constexpr int kSkXLoads = kSkXBytes / 1024 / 4;              // per wave and step
constexpr int kSkALoads = kSkABytes / 1024 / 4;
constexpr int kSkLoads = kSkXLoads + kSkALoads + 1;          // + one metadata load
constexpr int kSkSlotFloats = kSkBM * kSkBN;                 // one partial tile
constexpr uint64_t kSkFlagMagic = 0x4E4D534Bull << 32;       // flag = magic | call tag
static_assert(kSkStages * kSkStageBytes <= 160 * 1024, "LDS budget");
static_assert(4 * kEpilogueBytes <= kSkStageBytes, "epilogue slabs fit one stage");

struct SkArgs {
  int R, K, T;
  int tiles_m, tiles_n, nsteps;
  int per_group;   // tiles per workgroup when they divide evenly (no tile is cut), else 0
  int gm, gn;      // tile order: blocks of gm row tiles x gn column tiles
  int groups, per_xcd, xcds;
  int64_t total;   // tiles * nsteps
  float* slots;    // groups x kSkSlotFloats
  uint64_t* flags; // groups
  uint64_t tag;    // this call's flag value
  int spin_limit;  // polls of a flag before the finisher computes the steps itself
};

// Output tile (tm, tn) of list position v.  When every workgroup gets whole tiles, the
// list is dealt round by round (workgroup w's j-th tile is tile j * groups + w), so the
// workgroups run their tiles' K steps in lockstep; tiles are then taken in blocks of gm x gn
// (column-major inside), so the 32 workgroups an XCD runs at once share rows of A and
// columns of X in its L2.
__device__ __forceinline__ void sk_tile(const SkArgs& a, int v, int& tm, int& tn) {
  int t = v;
  if (a.per_group > 0) t = (v % a.per_group) * a.groups + v / a.per_group;
  const int g_m = t / (a.gm * a.tiles_n);
  const int rows = min(a.gm, a.tiles_m - g_m * a.gm);
  const int u = t - g_m * a.gm * a.tiles_n;
  const int g_n = u / (rows * a.gn);
  const int r = u - g_n * rows * a.gn;
  tm = g_m * a.gm + r % rows;
  tn = g_n * a.gn + r / rows;
}

// First (tile, step) pair of workgroup w's run.
__device__ __forceinline__ int64_t sk_begin(const SkArgs& a, int w) {
  return a.total * w / a.groups;
}

struct SkFrags {
  u32x4_t a[8];
  uint32_t ix[8];
  short16_t b[2];
};

__device__ __forceinline__ short16_t sk_join(short4_t n0, short4_t n1, short4_t n2, short4_t n3) {
  return __builtin_shufflevector(__builtin_shufflevector(n0, n1, 0, 1, 2, 3, 4, 5, 6, 7),
                                 __builtin_shufflevector(n2, n3, 0, 1, 2, 3, 4, 5, 6, 7),
                                 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
}

// One block of a substep: four smfmac (acc[fm][f] for four fm, one B fragment), with LDS
// reads of fragments needed later issued first and waited for at the end, so they land
// while the matrix core works.  A block's reads write registers that no smfmac of the
// previous block reads; d*/e*/dk are those the previous block read last, passed in so the
// compiler cannot hand them to this block's reads while that block's smfmac still run.
#define NM_SK_SM4(OP)                                                                  \
  OP " %[c0], %[a0], %[b], %[i0]\n\t" OP " %[c1], %[a1], %[b], %[i1]\n\t" OP          \
     " %[c2], %[a2], %[b], %[i2]\n\t" OP " %[c3], %[a3], %[b], %[i3]\n\t"
#define NM_SK_OUT [c0] "+a"(c0), [c1] "+a"(c1), [c2] "+a"(c2), [c3] "+a"(c3)
#define NM_SK_IN                                                                          \
  [a0] "v"(a0), [a1] "v"(a1), [a2] "v"(a2), [a3] "v"(a3), [i0] "v"(i0), [i1] "v"(i1),     \
      [i2] "v"(i2), [i3] "v"(i3), [b] "v"(b), [aa] "v"(aa), [d0] "v"(d0), [d1] "v"(d1),   \
      [d2] "v"(d2), [d3] "v"(d3), [e0] "v"(e0), [e1] "v"(e1), [e2] "v"(e2), [e3] "v"(e3), \
      [dk] "v"(dk)
#define NM_SK_ARGS                                                                          \
  float16v_t &c0, float16v_t &c1, float16v_t &c2, float16v_t &c3, const u32x4_t &a0,         \
      const u32x4_t &a1, const u32x4_t &a2, const u32x4_t &a3, uint32_t i0, uint32_t i1,      \
      uint32_t i2, uint32_t i3, const short16_t &b, uint32_t aa, const u32x4_t &d0,           \
      const u32x4_t &d1, const u32x4_t &d2, const u32x4_t &d3, uint32_t e0, uint32_t e1,      \
      uint32_t e2, uint32_t e3, const short16_t &dk
#define NM_SK_READ_A2 "ds_read_b128 %[na0], %[aa]\n\tds_read_b128 %[na1], %[aa] offset:2048\n\t"
#define NM_SK_READ_M2 "ds_read_b64 %[nm0], %[ma]\n\tds_read_b64 %[nm1], %[ma] offset:256\n\t"
#define NM_SK_READ_B                                                                       \
  "ds_read_b64_tr_b16 %[n0], %[b0]\n\tds_read_b64_tr_b16 %[n1], %[b1]\n\t"                  \
  "ds_read_b64_tr_b16 %[n2], %[b0] offset:8192\n\tds_read_b64_tr_b16 %[n3], %[b1] offset:8192\n\t"
#define NM_SK_BOUT [n0] "=&v"(n0), [n1] "=&v"(n1), [n2] "=&v"(n2), [n3] "=&v"(n3)

// reads: two A fragments
template <bool BF16>
__device__ __forceinline__ void sk_blk_a(NM_SK_ARGS, u32x4_t& na0, u32x4_t& na1) {
#define NM_SK_BLK(OP)                                                                   \
  asm volatile("s_nop 2\n\t" NM_SK_READ_A2 NM_SK_SM4(OP) "s_waitcnt lgkmcnt(0)"         \
               : [na0] "=&v"(na0), [na1] "=&v"(na1), NM_SK_OUT                          \
               : NM_SK_IN                                                               \
               : "memory")
  if constexpr (BF16) NM_SK_BLK("v_smfmac_f32_32x32x32_bf16");
  else NM_SK_BLK("v_smfmac_f32_32x32x32_f16");
#undef NM_SK_BLK
}
// reads: two A fragments and the 8 metadata bytes of two fragments' rows
template <bool BF16>
__device__ __forceinline__ void sk_blk_am(NM_SK_ARGS, u32x4_t& na0, u32x4_t& na1, u32x2_t& nm0,
                                          u32x2_t& nm1, uint32_t ma) {
#define NM_SK_BLK(OP)                                                                   \
  asm volatile("s_nop 2\n\t" NM_SK_READ_A2 NM_SK_READ_M2 NM_SK_SM4(OP)                  \
               "s_waitcnt lgkmcnt(0)"                                                   \
               : [na0] "=&v"(na0), [na1] "=&v"(na1), [nm0] "=&v"(nm0), [nm1] "=&v"(nm1), \
                 NM_SK_OUT                                                              \
               : NM_SK_IN, [ma] "v"(ma)                                                 \
               : "memory")
  if constexpr (BF16) NM_SK_BLK("v_smfmac_f32_32x32x32_bf16");
  else NM_SK_BLK("v_smfmac_f32_32x32x32_f16");
#undef NM_SK_BLK
}
// reads: two A fragments and one B fragment (four transposing reads)
template <bool BF16>
__device__ __forceinline__ void sk_blk_ab(NM_SK_ARGS, u32x4_t& na0, u32x4_t& na1, short16_t& nb,
                                          uint32_t b0, uint32_t b1) {
  short4_t n0 = {}, n1 = {}, n2 = {}, n3 = {};
#define NM_SK_BLK(OP)                                                                   \
  asm volatile("s_nop 2\n\t" NM_SK_READ_B NM_SK_READ_A2 NM_SK_SM4(OP)                   \
               "s_waitcnt lgkmcnt(0)"                                                   \
               : NM_SK_BOUT, [na0] "=&v"(na0), [na1] "=&v"(na1), NM_SK_OUT              \
               : NM_SK_IN, [b0] "v"(b0), [b1] "v"(b1)                                   \
               : "memory")
  if constexpr (BF16) NM_SK_BLK("v_smfmac_f32_32x32x32_bf16");
  else NM_SK_BLK("v_smfmac_f32_32x32x32_f16");
#undef NM_SK_BLK
  nb = sk_join(n0, n1, n2, n3);
}
// reads: two A fragments, one B fragment and the metadata of two fragments
template <bool BF16>
__device__ __forceinline__ void sk_blk_abm(NM_SK_ARGS, u32x4_t& na0, u32x4_t& na1, short16_t& nb,
                                           uint32_t b0, uint32_t b1, u32x2_t& nm0, u32x2_t& nm1,
                                           uint32_t ma) {
  short4_t n0 = {}, n1 = {}, n2 = {}, n3 = {};
#define NM_SK_BLK(OP)                                                                   \
  asm volatile("s_nop 2\n\t" NM_SK_READ_B NM_SK_READ_A2 NM_SK_READ_M2 NM_SK_SM4(OP)     \
               "s_waitcnt lgkmcnt(0)"                                                   \
               : NM_SK_BOUT, [na0] "=&v"(na0), [na1] "=&v"(na1), [nm0] "=&v"(nm0),       \
                 [nm1] "=&v"(nm1), NM_SK_OUT                                            \
               : NM_SK_IN, [b0] "v"(b0), [b1] "v"(b1), [ma] "v"(ma)                     \
               : "memory")
  if constexpr (BF16) NM_SK_BLK("v_smfmac_f32_32x32x32_bf16");
  else NM_SK_BLK("v_smfmac_f32_32x32x32_f16");
#undef NM_SK_BLK
  nb = sk_join(n0, n1, n2, n3);
}

// A wave's 128 x 64 block of accumulators plus the partial sums of the same outputs that
// other workgroups left in row-major 256 x 256 fp32 slots (slot j of `parts` for each set
// bit j of part_mask below nparts, added in that order), written to Y as YT.  Each 32-row slab passes through this wave's LDS region
// as fp32 (kEpilogueBytes), then leaves in pieces of four outputs of one row.  (row0,
// col0) is the block's first output in Y, (trow, tcol) the same in the tile.
template <int YT>
__device__ __forceinline__ void sk_store_sum(const float16v_t (&acc)[4][2], uint8_t* lds, void* Y,
                                             int row0, int col0, int trow, int tcol, int R,
                                             int T, int lane, const float* parts, int nparts,
                                             uint64_t part_mask) {
  constexpr int kPitch = 64 * 4 + 16;  // fp32 slab row pitch
  const int l32 = lane & 31, q = lane >> 5;
  uint8_t* y = static_cast<uint8_t*>(Y);
#pragma unroll
  for (int fm = 0; fm < 4; ++fm) {
#pragma unroll
    for (int f = 0; f < 2; ++f) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        *reinterpret_cast<float*>(lds + (8 * (i / 4) + 4 * q + (i % 4)) * kPitch +
                                  (32 * f + l32) * 4) = acc[fm][f][i];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {  // 32 rows x 16 pieces of four outputs
      const int pc = k * 64 + lane, r = pc >> 4, cp = pc & 15;
      float4_t v = *reinterpret_cast<const float4_t*>(lds + r * kPitch + cp * 16);
      const int64_t at = (int64_t)(trow + 32 * fm + r) * kSkBN + tcol + 4 * cp;
      for (int j = 0; j < nparts; ++j)
        if ((part_mask >> j) & 1u)
          v += *reinterpret_cast<const float4_t*>(parts + (int64_t)j * kSkSlotFloats + at);
      const int row = row0 + 32 * fm + r, col = col0 + 4 * cp;
      if (row < R && col < T) {  // T % 8 == 0: a piece is wholly inside or outside
        uint8_t* d = y + ((int64_t)row * T + col) * (YT == kF32 ? 4 : 2);
        if constexpr (YT == kF32) {
          *reinterpret_cast<float4_t*>(d) = v;
        } else {
          u32x2_t h;
          h[0] = YT == kBF16 ? (f32_to_bf16(v[0]) | f32_to_bf16(v[1]) << 16)
                             : (f32_to_f16(v[0]) | f32_to_f16(v[1]) << 16);
          h[1] = YT == kBF16 ? (f32_to_bf16(v[2]) | f32_to_bf16(v[3]) << 16)
                             : (f32_to_f16(v[2]) | f32_to_f16(v[3]) << 16);
          *reinterpret_cast<u32x2_t*>(d) = h;
        }
      }
    }
  }
}

constexpr int kSkMaxParts = 64;  // later parts of one tile added from slots

template <bool BF16, int YT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
    smfmac_sk_spmm_kernel(const uint16_t* __restrict__ values, const uint32_t* __restrict__ meta,
                          const uint16_t* __restrict__ X, void* __restrict__ Y, SkArgs args) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  __shared__ int s_ready[kSkMaxParts];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // workgroup b runs on XCD b % xcds; consecutive runs of the (tile, step) list go to one XCD
  const int w = (int)(blockIdx.x % args.xcds) * args.per_xcd + (int)(blockIdx.x / args.xcds);
  if (w >= args.groups) return;  // whole workgroup, before any load
  const int R = args.R, T = args.T, nsteps = args.nsteps;
  const int last_g = ((R + 15) >> 4) - 1;
  const uint32_t smem_base = lds_addr(smem);

  // ---- fragment read addresses within a stage (independent of the tile) ----
  const int l32 = lane & 31, q = lane >> 5, l16 = lane & 15, blk = lane >> 4;
  const int aswz = (l32 >> 2) & 3;
  // A fragment fm of substep t: tile row 32 fm + l32, 16-byte chunk (2t + q) ^ ((row >> 2) & 3)
  const uint32_t a_rd0 = (uint32_t)(kSkXBytes + l32 * 64 + (((0 + q) ^ aswz) << 4));
  const uint32_t a_rd1 = (uint32_t)(kSkXBytes + l32 * 64 + (((2 + q) ^ aswz) << 4));
  // the row's 8 metadata bytes: four 16-bit index units, unit 2t + q for substep t
  const uint32_t m_rd = (uint32_t)(kSkXBytes + kSkABytes + l32 * 8);
  const uint32_t sel0 = q ? 0x0302u : 0x0100u;  // v_perm selectors: unit q of the low word
  const uint32_t sel1 = q ? 0x0706u : 0x0504u;  // unit 2 + q (the high word)
  // B fragment (t, f): K rows 32t + {8q .. 8q+7, 16+8q .. 16+8q+7} of columns
  // 64 wave + 32 f + (lane % 32); lane i of a 16-lane block reads K row kb + (i >> 2),
  // columns 4 (i & 3) .. +3 of the block's 16 columns
  const int rb = 8 * q + (l16 >> 2);
  uint32_t b_rd[2][2][2];  // [substep][f][rows kb / kb + 4]
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int lp = (wave * 64 + 32 * f + 16 * (blk & 1)) / 16;  // logical 32-byte pair
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int r0 = rb + 32 * t, r1 = rb + 4 + 32 * t;
      b_rd[t][f][0] =
          (uint32_t)(r0 * kSkXRowBytes + ((lp ^ xpair_swizzle(r0)) << 5) + 8 * (l16 & 3));
      b_rd[t][f][1] =
          (uint32_t)(r1 * kSkXRowBytes + ((lp ^ xpair_swizzle(r1)) << 5) + 8 * (l16 & 3));
    }
  }

  float16v_t acc[8][2];

  // Accumulates steps ka .. kb-1 of tile (tm, tn) into acc.  Ends with every direct load
  // landed and all waves past a barrier, so LDS may be reused.
  auto segment = [&](int tm, int tn, int ka, int kb) __attribute__((always_inline)) {
    const int m0 = tm * kSkBM, t0 = tn * kSkBN, g0 = m0 >> 4;
    const int last = kb - 1;
    const uint8_t* xg = reinterpret_cast<const uint8_t*>(X);
    const uint8_t* vg = reinterpret_cast<const uint8_t*>(values) + (int64_t)g0 * nsteps * 1024;
    const uint8_t* mg = reinterpret_cast<const uint8_t*>(meta) + (int64_t)g0 * nsteps * 128;
    // this wave's direct loads of a step: X 1 KB windows (two K rows), 16-row value blocks,
    // and four 16-row metadata blocks on half of the lanes; per-lane offsets from the
    // step's base; rows past R and columns past T read valid data (outputs dropped)
    uint32_t x_off[kSkXLoads], a_off[kSkALoads], m_off;
    uint32_t x_dst[kSkXLoads], a_dst[kSkALoads], m_dst;
#pragma unroll
    for (int j = 0; j < kSkXLoads; ++j) {
      const int w1k = j * 4 + wave;
      const int slot = w1k * 64 + lane;
      const int r = slot / kSkXChunks, pc = slot % kSkXChunks;
      const int lc = 2 * ((pc >> 1) ^ xpair_swizzle(r)) + (pc & 1);
      const int col = t0 + 8 * lc < T ? t0 + 8 * lc : 0;
      x_off[j] = (uint32_t)(((int64_t)r * T + col) * 2);
      x_dst[j] = (uint32_t)(w1k * 1024);
    }
#pragma unroll
    for (int j = 0; j < kSkALoads; ++j) {
      const int b16 = j * 4 + wave;
      const int i = 16 * b16 + (lane >> 2);
      const int lc = (lane & 3) ^ ((i >> 2) & 3);
      const int g = min(g0 + b16, last_g) - g0;
      a_off[j] = (uint32_t)(g * nsteps * 1024 + (lane >> 2) * 64 + 16 * lc);
      a_dst[j] = (uint32_t)(kSkXBytes + b16 * 1024);
    }
    {
      const int g = min(g0 + 4 * wave + ((lane & 31) >> 3), last_g) - g0;
      m_off = (uint32_t)(g * nsteps * 128 + 16 * (lane & 7));
      m_dst = (uint32_t)(kSkXBytes + kSkABytes + wave * 512);
    }
    // load j (0 .. kSkLoads-1) of step `step` into its stage; steps past the segment
    // re-read its last step into that step's stage (the same bytes)
    auto issue = [&](int j, int step) __attribute__((always_inline)) {
      step = step < last ? step : last;
      uint8_t* st = smem + ((step - ka) % kSkStages) * kSkStageBytes;
      if (j < kSkXLoads) {
        global_to_lds<16>(xg + (int64_t)step * kKStep * T * 2 + x_off[j], st + x_dst[j]);
      } else if (j < kSkXLoads + kSkALoads) {
        global_to_lds<16>(vg + (int64_t)step * 1024 + a_off[j - kSkXLoads],
                          st + a_dst[j - kSkXLoads]);
      } else if (lane < 32) {
        global_to_lds<16>(mg + (int64_t)step * 128 + m_off, st + m_dst);
      }
    };
#pragma unroll
    for (int k = 0; k < kSkStages; ++k)
#pragma unroll
      for (int j = 0; j < kSkLoads; ++j) issue(j, ka + k);
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * kSkLoads) : "memory");

    // substep-0 fragments of the first step, and its metadata
    SkFrags F0, F1;
    u32x2_t raw[8];
#pragma unroll
    for (int fm = 0; fm < 8; ++fm) {
      u32x4_t v;
      u32x2_t mw;
      asm volatile("ds_read_b128 %0, %2\n\tds_read_b64 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                   : "=&v"(v), "=&v"(mw)
                   : "v"(smem_base + a_rd0 + fm * 2048), "v"(smem_base + m_rd + fm * 256)
                   : "memory");
      F0.a[fm] = v;
      raw[fm] = mw;
    }
#pragma unroll
    for (int fm = 0; fm < 8; ++fm) {
      F0.ix[fm] = __builtin_amdgcn_perm(raw[fm][1], raw[fm][0], sel0);
      F1.ix[fm] = F0.ix[fm];
    }
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      short4_t n0, n1, n2, n3;
      asm volatile(
          "ds_read_b64_tr_b16 %0, %4\n\tds_read_b64_tr_b16 %1, %5\n\t"
          "ds_read_b64_tr_b16 %2, %4 offset:8192\n\tds_read_b64_tr_b16 %3, %5 offset:8192\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(n0), "=&v"(n1), "=&v"(n2), "=&v"(n3)
          : "v"(smem_base + b_rd[0][f][0]), "v"(smem_base + b_rd[0][f][1])
          : "memory");
      F0.b[f] = sk_join(n0, n1, n2, n3);
    }
#pragma unroll
    for (int fm = 0; fm < 8; ++fm) F1.a[fm] = F0.a[fm];
    F1.b[0] = F0.b[0];
    F1.b[1] = F0.b[1];

    int cur = 0;
    for (int s = ka; s < kb; ++s) {
      // invariant: steps s and s+1 landed (s+1 certified at the previous barrier, or by
      // the prologue); F0 holds substep 0 of step s, raw its metadata words
      const int nxt = cur == kSkStages - 1 ? 0 : cur + 1;
      const uint32_t st = smem_base + cur * kSkStageBytes, sn = smem_base + nxt * kSkStageBytes;
      // ---- substep 0 (C = F0); reads step s, substep 1 (F1) from this stage ----
      sk_blk_a<BF16>(acc[0][0], acc[1][0], acc[2][0], acc[3][0], F0.a[0], F0.a[1], F0.a[2],
                     F0.a[3], F0.ix[0], F0.ix[1], F0.ix[2], F0.ix[3], F0.b[0], st + a_rd1, F1.a[4],
                     F1.a[5], F1.a[6], F1.a[7], F1.ix[4], F1.ix[5], F1.ix[6], F1.ix[7], F1.b[1],
                     F1.a[0], F1.a[1]);
      // substep-1 index words of step s (F1.ix was last read one block back)
#pragma unroll
      for (int fm = 0; fm < 8; ++fm) F1.ix[fm] = __builtin_amdgcn_perm(raw[fm][1], raw[fm][0], sel1);
      sk_blk_a<BF16>(acc[4][0], acc[5][0], acc[6][0], acc[7][0], F0.a[4], F0.a[5], F0.a[6],
                     F0.a[7], F0.ix[4], F0.ix[5], F0.ix[6], F0.ix[7], F0.b[0],
                     st + a_rd1 + 2 * 2048, F0.a[0], F0.a[1], F0.a[2], F0.a[3], F0.ix[0],
                     F0.ix[1], F0.ix[2], F0.ix[3], F0.b[0], F1.a[2], F1.a[3]);
      sk_blk_ab<BF16>(acc[0][1], acc[1][1], acc[2][1], acc[3][1], F0.a[0], F0.a[1], F0.a[2],
                      F0.a[3], F0.ix[0], F0.ix[1], F0.ix[2], F0.ix[3], F0.b[1],
                      st + a_rd1 + 4 * 2048, F0.a[4], F0.a[5], F0.a[6], F0.a[7], F0.ix[4],
                      F0.ix[5], F0.ix[6], F0.ix[7], F0.b[0], F1.a[4], F1.a[5], F1.b[0],
                      st + b_rd[1][0][0], st + b_rd[1][0][1]);
      sk_blk_ab<BF16>(acc[4][1], acc[5][1], acc[6][1], acc[7][1], F0.a[4], F0.a[5], F0.a[6],
                      F0.a[7], F0.ix[4], F0.ix[5], F0.ix[6], F0.ix[7], F0.b[1],
                      st + a_rd1 + 6 * 2048, F0.a[0], F0.a[1], F0.a[2], F0.a[3], F0.ix[0],
                      F0.ix[1], F0.ix[2], F0.ix[3], F0.b[0], F1.a[6], F1.a[7], F1.b[1],
                      st + b_rd[1][1][0], st + b_rd[1][1][1]);
      // step s+1 landed (its loads were issued during the previous step or the prologue),
      // and after the barrier no wave reads the stage of step s
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kSkLoads) : "memory");
      // ---- substep 1 (C = F1); reads step s+1, substep 0 (F0) and its metadata from
      // the next stage, and issues the loads of step s+3 into the stage of step s ----
      issue(0, s + 3);
      issue(1, s + 3);
      issue(2, s + 3);
      issue(3, s + 3);
      sk_blk_am<BF16>(acc[0][0], acc[1][0], acc[2][0], acc[3][0], F1.a[0], F1.a[1], F1.a[2],
                      F1.a[3], F1.ix[0], F1.ix[1], F1.ix[2], F1.ix[3], F1.b[0], sn + a_rd0,
                      F0.a[4], F0.a[5], F0.a[6], F0.a[7], F0.ix[4], F0.ix[5], F0.ix[6], F0.ix[7],
                      F0.b[1], F0.a[0], F0.a[1], raw[0], raw[1], sn + m_rd);
      issue(4, s + 3);
      issue(5, s + 3);
      issue(6, s + 3);
      sk_blk_am<BF16>(acc[4][0], acc[5][0], acc[6][0], acc[7][0], F1.a[4], F1.a[5], F1.a[6],
                      F1.a[7], F1.ix[4], F1.ix[5], F1.ix[6], F1.ix[7], F1.b[0],
                      sn + a_rd0 + 2 * 2048, F1.a[0], F1.a[1], F1.a[2], F1.a[3], F1.ix[0],
                      F1.ix[1], F1.ix[2], F1.ix[3], F1.b[0], F0.a[2], F0.a[3], raw[2], raw[3],
                      sn + m_rd + 2 * 256);
      issue(7, s + 3);
      issue(8, s + 3);
      issue(9, s + 3);
      sk_blk_abm<BF16>(acc[0][1], acc[1][1], acc[2][1], acc[3][1], F1.a[0], F1.a[1], F1.a[2],
                       F1.a[3], F1.ix[0], F1.ix[1], F1.ix[2], F1.ix[3], F1.b[1],
                       sn + a_rd0 + 4 * 2048, F1.a[4], F1.a[5], F1.a[6], F1.a[7], F1.ix[4],
                       F1.ix[5], F1.ix[6], F1.ix[7], F1.b[0], F0.a[4], F0.a[5], F0.b[0],
                       sn + b_rd[0][0][0], sn + b_rd[0][0][1], raw[4], raw[5],
                       sn + m_rd + 4 * 256);
      issue(10, s + 3);
      issue(11, s + 3);
      issue(12, s + 3);
      sk_blk_abm<BF16>(acc[4][1], acc[5][1], acc[6][1], acc[7][1], F1.a[4], F1.a[5], F1.a[6],
                       F1.a[7], F1.ix[4], F1.ix[5], F1.ix[6], F1.ix[7], F1.b[1],
                       sn + a_rd0 + 6 * 2048, F1.a[0], F1.a[1], F1.a[2], F1.a[3], F1.ix[0],
                       F1.ix[1], F1.ix[2], F1.ix[3], F1.b[0], F0.a[6], F0.a[7], F0.b[1],
                       sn + b_rd[0][1][0], sn + b_rd[0][1][1], raw[6], raw[7],
                       sn + m_rd + 6 * 256);
      // substep-0 index words of step s+1 (F0.ix was last read four blocks back)
#pragma unroll
      for (int fm = 0; fm < 8; ++fm) F0.ix[fm] = __builtin_amdgcn_perm(raw[fm][1], raw[fm][0], sel0);
      cur = nxt;
    }
    // loads past the segment have landed before LDS is reused, and the last smfmac
    // results land before plain instructions read the accumulators
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  };

  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int fm = 0; fm < 8; ++fm)
#pragma unroll
      for (int f = 0; f < 2; ++f) acc[fm][f] = float16v_t{};
  };
  // the tile's outputs (plus later parts from slots) to Y; the slabs are read before the
  // next segment's loads refill LDS
  auto store_tile = [&](int tm, int tn, const float* parts, int nparts, uint64_t mask)
                        __attribute__((always_inline)) {
    // an opaque copy of the lane index keeps the epilogue's addresses from being computed
    // ahead of the main loop (they would hold registers through it)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int m0 = tm * kSkBM, c0 = tn * kSkBN + 64 * wave;
    uint8_t* slab = smem + wave * kEpilogueBytes;
    sk_store_sum<YT>(*reinterpret_cast<const float16v_t(*)[4][2]>(&acc[0][0]), slab, Y, m0, c0,
                     0, 64 * wave, R, T, ln, parts, nparts, mask);
    sk_store_sum<YT>(*reinterpret_cast<const float16v_t(*)[4][2]>(&acc[4][0]), slab, Y,
                     m0 + 128, c0, 128, 64 * wave, R, T, ln, parts, nparts, mask);
    __syncthreads();
  };
  auto slot_of = [&](int v) __attribute__((always_inline)) {
    return args.slots + (int64_t)v * kSkSlotFloats;
  };

  int64_t it = sk_begin(args, w);
  const int64_t end = sk_begin(args, w + 1);
  while (it < end) {
    const int tile = (int)(it / nsteps);
    const int ka = (int)(it - (int64_t)tile * nsteps);
    const int kb = (int)min<int64_t>(nsteps, ka + (end - it));
    int tm, tn;
    sk_tile(args, tile, tm, tn);
    const int64_t tile_base = (int64_t)tile * nsteps, tile_end = tile_base + nsteps;
    // the later parts of the tile when this run holds its first steps (always the run's
    // last segment): the next workgroups, in order
    int nv = 0;
    if (ka == 0 && kb < nsteps)
      while (w + 1 + nv < args.groups && sk_begin(args, w + 1 + nv) < tile_end) ++nv;
    uint64_t part_mask = 0;  // bit i: part i is added from its slot
    zero_acc();
    // steps ka .. kb-1, then the steps of any later part whose flag does not rise in time
    // (its workgroup has not run), computed here instead; one call site keeps one copy of
    // the pipeline in the kernel
    int cka = ka, ckb = kb, next_part = 0;
    while (true) {
      segment(tm, tn, cka, ckb);
      if (cka == ka && nv > 0) {  // after the first segment: which parts are published
        if (tid == 0) {
          // relaxed polls (an acquire per poll would invalidate this XCD's L2 each time),
          // then one acquire fence for the slots' contents
          for (int i = 0; i < nv && i < kSkMaxParts; ++i) {
            int ready = 0;
            for (int n = 0; n < args.spin_limit; ++n) {
              if (__hip_atomic_load(args.flags + w + 1 + i, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT) == args.tag) {
                ready = 1;
                break;
              }
              __builtin_amdgcn_s_sleep(8);
            }
            s_ready[i] = ready;
          }
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
        __syncthreads();
      }
      while (next_part < nv && next_part < kSkMaxParts && s_ready[next_part])
        part_mask |= 1ull << next_part++;
      if (next_part >= nv) break;
      const int v = w + 1 + next_part++;
      cka = (int)(sk_begin(args, v) - tile_base);
      ckb = (int)(min(sk_begin(args, v + 1), tile_end) - tile_base);
    }
    if (ka > 0) {
      // a later part of the tile (always this run's first segment): its fp32 sums go to
      // this workgroup's slot as a row-major 256 x 256 tile, then the flag is raised
      int ln = lane;
      asm volatile("" : "+v"(ln));
      uint8_t* slab = smem + wave * kEpilogueBytes;
      float* mine = slot_of(w);
      store_block_128x64<kF32>(*reinterpret_cast<const float16v_t(*)[4][2]>(&acc[0][0]), slab,
                               mine, 0, 64 * wave, kSkBM, kSkBN, ln);
      store_block_128x64<kF32>(*reinterpret_cast<const float16v_t(*)[4][2]>(&acc[4][0]), slab,
                               mine, 128, 64 * wave, kSkBM, kSkBN, ln);
      // every wave's slot stores complete, then one release (it writes the L2 back once)
      // before the flag
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (tid == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __hip_atomic_store(args.flags + w, args.tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else {
      store_tile(tm, tn, nv > 0 ? slot_of(w + 1) : args.slots, min(nv, kSkMaxParts), part_mask);
    }
    it += kb - ka;
  }
}

#undef NM_SK_SM4
#undef NM_SK_OUT
#undef NM_SK_IN
#undef NM_SK_ARGS
#undef NM_SK_READ_A2
#undef NM_SK_READ_M2
#undef NM_SK_READ_B
#undef NM_SK_BOUT

std::atomic<uint32_t> g_sk_calls{0};

int64_t sk_flag_bytes(int groups) { return ((int64_t)groups * 8 + 255) / 256 * 256; }

template <bool BF16, int YT>
hipError_t run_sk(const void* values, const uint32_t* meta, int64_t R, int64_t K, const void* X,
                  int64_t T, void* Y, int groups, void* workspace, hipStream_t s) {
  const int xcds = xcd_count();
  SkArgs a;
  a.R = (int)R;
  a.K = (int)K;
  a.T = (int)T;
  a.tiles_m = (int)((R + kSkBM - 1) / kSkBM);
  a.tiles_n = (int)((T + kSkBN - 1) / kSkBN);
  a.per_group = (a.tiles_m * a.tiles_n) % groups == 0 ? a.tiles_m * a.tiles_n / groups : 0;
  a.gn = a.tiles_n < 4 ? a.tiles_n : 4;
  a.gm = 32 / a.gn;
  a.nsteps = (int)(K / kKStep);
  a.total = (int64_t)((R + kSkBM - 1) / kSkBM) * a.tiles_n * a.nsteps;
  a.groups = groups;
  a.xcds = xcds;
  a.per_xcd = (groups + xcds - 1) / xcds;
  a.flags = static_cast<uint64_t*>(workspace);
  a.slots = workspace ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                                 sk_flag_bytes(groups))
                      : nullptr;
  a.tag = kSkFlagMagic | (uint64_t)(g_sk_calls.fetch_add(1, std::memory_order_relaxed) + 1u);
  a.spin_limit = 1 << 16;
  auto kernel = smfmac_sk_spmm_kernel<BF16, YT>;
  const size_t lds = (size_t)kSkStages * kSkStageBytes;
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  kernel<<<a.per_xcd * xcds, 256, lds, s>>>(static_cast<const uint16_t*>(values), meta,
                                             static_cast<const uint16_t*>(X), Y, a);
  return hipGetLastError();
}

}  // namespace

int64_t sk_workspace_bytes(int64_t R, int64_t T, int groups) {
  // none when every workgroup gets whole tiles: no partial sums are exchanged
  const int64_t tiles = ((R + kSkBM - 1) / kSkBM) * ((T + kSkBN - 1) / kSkBN);
  if (tiles % groups == 0) return 0;
  return sk_workspace_bytes(groups);
}

int64_t sk_workspace_bytes(int groups) {
  return sk_flag_bytes(groups) + (int64_t)groups * kSkSlotFloats * 4;
}

int sk_groups(int64_t R, int64_t K, int64_t T) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (cus <= 0) cus = 256;
  const int64_t total = ((R + kSkBM - 1) / kSkBM) * ((T + kSkBN - 1) / kSkBN) * (K / kKStep);
  const int64_t g = total < cus ? total : cus;
  return (int)(g > 0 ? g : 1);
}

bool sk_shape_ok(int64_t R, int64_t K, int64_t T) {
  // whole 64-wide K steps and 16-byte X rows; per-lane byte offsets (64 rows of X, 16
  // value blocks of a tile) within 32 bits
  if (K <= 0 || K % kKStep != 0 || T % 8 != 0 || R <= 0 || T <= 0) return false;
  return R < (1 << 30) && T < (1 << 24) && K < (1 << 22);
}

bool sk_preferred(int64_t R, int64_t K, int64_t T) {
  // Never taken on its own: the 256 x 128 wave-specialised kernel, whose consumers keep
  // their LDS reads in flight across blocks, now runs every measured shape faster (the
  // fp16 4096 x 4096 x 8192 2:4 product, 512 tiles of this kernel on 256 compute units:
  // 146 against 160 us; the LLaMA-7B MLP shapes, where tiles would have to be cut between
  // workgroups: 107 / 92 against 167 / 143 us).  NM_SPMM_TILE=3 still selects it.
  (void)R;
  (void)K;
  (void)T;
  return false;
}

hipError_t launch_spmm_sk(const void* values, const uint32_t* meta, int64_t R, int64_t K,
                          const void* X, int64_t T, int dt, void* Y, int y_dt, void* workspace,
                          int groups, hipStream_t s) {
  const bool bf16 = dt == 2;
  if (y_dt == 0)
    return bf16 ? run_sk<true, kF32>(values, meta, R, K, X, T, Y, groups, workspace, s)
                : run_sk<false, kF32>(values, meta, R, K, X, T, Y, groups, workspace, s);
  return bf16 ? run_sk<true, kBF16>(values, meta, R, K, X, T, Y, groups, workspace, s)
              : run_sk<false, kF16>(values, meta, R, K, X, T, Y, groups, workspace, s);
}

}  // namespace nm
