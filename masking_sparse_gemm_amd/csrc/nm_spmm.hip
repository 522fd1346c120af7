// nm_spmm.hip -- Y = W_sparse * X for the compressed N:M format (gfx950).
//
// The product ("[리뷰] Accelerating Sparse Deep Neural Networks", section "Tensor
// Scores 상에서 구조적인 sparse GEMM") takes the compressed weight as the first
// operand and a dense K x T activation matrix as the second; the result is dense.
//
// 2:4 and 1:2 with 16-bit inputs run on gfx950's structured-sparse matrix cores
// (v_smfmac_f32_16x16x64_{bf16,f16}).  That instruction takes, per lane, eight
// stored values covering sixteen consecutive K positions of one row (four groups
// of four) plus a 16-bit index whose 2-bit fields give each value's position in
// its group, least significant field first -- exactly one half-word of this
// library's 2:4 metadata -- so compressed rows feed the matrix cores with no
// conversion, and the hardware gathers the matching rows of X.  1:2 metadata (one
// bit per value) is widened to that nibble form in registers: pairs of 1:2 groups
// are 2:4 groups with one value in each half.
//
// Tiling.  A workgroup owns a BM x BN tile of Y and walks K in steps of 128.  X
// tiles are staged through LDS (double-buffered, one barrier per step) and read
// back with ds_read_b64_tr_b16, which hands each lane four consecutive K rows of
// one column -- the K-major order the matrix-core B operand needs -- from the
// row-major tile.  Compressed values and metadata go straight from global memory
// to registers, one step ahead.  Inside a 128-wide K step the contraction order
// is permuted so that lane group q of the instruction covers K [32q, 32q+32): its
// stored values are then 32 contiguous bytes and its metadata one 32-bit word
// whose low and high halves serve the two instructions of the step through the
// instruction's index-half selector.  The accumulators are fp32; the result is
// rounded once to the output type (round to nearest even).
//
// Every other pattern, fp32, and shapes the tiled kernel does not take (K not a
// multiple of 128, T not a multiple of 8) use a plain LDS-tiled kernel that
// expands the compressed rows to fp32 and accumulates with fp32 FMAs.
#include "nm_device.h"
#include "nm_launch.h"

namespace nm {

namespace {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef short short16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16_t __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x16_t __attribute__((ext_vector_type(16)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

enum { kF32 = 0, kF16 = 1, kBF16 = 2 };

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ float f16_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {  // round to nearest even
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) & 0x8000u) | 0x7FC0u;  // NaN
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t f32_to_f16(float x) {  // hardware conversion, RNE
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}
template <int DT>
__device__ __forceinline__ float load_as_f32(const void* p, int64_t i) {
  if constexpr (DT == kF32) return static_cast<const float*>(p)[i];
  else if constexpr (DT == kBF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  else return f16_to_f32(static_cast<const uint16_t*>(p)[i]);
}
template <int YT>
__device__ __forceinline__ void store_from_f32(void* p, int64_t i, float v) {
  if constexpr (YT == kF32) static_cast<float*>(p)[i] = v;
  else if constexpr (YT == kBF16) static_cast<uint16_t*>(p)[i] = (uint16_t)f32_to_bf16(v);
  else static_cast<uint16_t*>(p)[i] = (uint16_t)f32_to_f16(v);
}

// ===========================================================================
// Structured-sparse matrix-core kernel (2:4, or 1:2 widened to 2:4).
// ===========================================================================
constexpr int kKStep = 128;  // K per main-loop step (two smfmac instructions)

template <int BM, int BN, int WAVES_M, int WAVES_N>
struct SmfmacTile {
  static constexpr int kThreads = 64 * WAVES_M * WAVES_N;
  static constexpr int kWM = BM / WAVES_M;
  static constexpr int kWN = BN / WAVES_N;
  static constexpr int kFM = kWM / 16;
  static constexpr int kFN = kWN / 16;
  static constexpr int kLdsStride = BN + 8;  // halves per LDS row (16-byte pad)
  static constexpr int kLdsStage = kKStep * kLdsStride;
  static constexpr int kXChunks = kKStep * BN / 8 / kThreads;  // 16-byte X loads per thread
  static_assert(kWM % 16 == 0 && kWN % 16 == 0, "wave tile must be whole 16x16 fragments");
  static_assert((kKStep * BN / 8) % kThreads == 0, "X tile must split evenly over threads");
};

// 1:2 metadata bits (one per value) of 32 K positions -> eight 2:4 nibbles.
__device__ __forceinline__ uint32_t widen_1_2(uint32_t x16) {
  uint32_t x = x16 & 0xFFFFu;  // bit i -> bit 2i
  x = (x | (x << 8)) & 0x00FF00FFu;
  x = (x | (x << 4)) & 0x0F0F0F0Fu;
  x = (x | (x << 2)) & 0x33333333u;
  x = (x | (x << 1)) & 0x55555555u;
  return x | 0x88888888u;  // second value of each pair sits in the upper half (2 + bit)
}

template <bool BF16>
__device__ __forceinline__ float4_t smfmac(const uint4& a, const short16_t& b, const float4_t& c,
                                           uint32_t idx, int half) {
  if constexpr (BF16) {
    const bf16x8_t av = __builtin_bit_cast(bf16x8_t, a);
    const bf16x16_t bv = __builtin_bit_cast(bf16x16_t, b);
    return half == 0 ? __builtin_amdgcn_smfmac_f32_16x16x64_bf16(av, bv, c, (int)idx, 0, 0)
                     : __builtin_amdgcn_smfmac_f32_16x16x64_bf16(av, bv, c, (int)idx, 0, 1);
  } else {
    const f16x8_t av = __builtin_bit_cast(f16x8_t, a);
    const f16x16_t bv = __builtin_bit_cast(f16x16_t, b);
    return half == 0 ? __builtin_amdgcn_smfmac_f32_16x16x64_f16(av, bv, c, (int)idx, 0, 0)
                     : __builtin_amdgcn_smfmac_f32_16x16x64_f16(av, bv, c, (int)idx, 0, 1);
  }
}

__device__ __forceinline__ short4_t lds_tr_read(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(p));
}

template <bool BF16, bool kPat12, int YT, int BM, int BN, int WAVES_M, int WAVES_N>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N)
    smfmac_spmm_kernel(const uint16_t* __restrict__ values, const uint32_t* __restrict__ meta,
                       const uint16_t* __restrict__ X, void* __restrict__ Y, int R, int K, int T,
                       int tiles_n) {
  using TL = SmfmacTile<BM, BN, WAVES_M, WAVES_N>;
  constexpr int FM = TL::kFM, FN = TL::kFN, NT = TL::kThreads;
  __shared__ __attribute__((aligned(16))) uint16_t xs[2 * TL::kLdsStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int tile_m = blockIdx.x / tiles_n, tile_n = blockIdx.x % tiles_n;
  const int m0 = tile_m * BM, t0 = tile_n * BN;
  const int l16 = lane & 15, q = lane >> 4;

  const int64_t vals_per_row = K / 2;
  // metadata words per row: 2:4 -> K/32, 1:2 -> K/64
  const int64_t meta_per_row = kPat12 ? K / 64 : K / 32;

  // ---- per-lane A pointers (one row per fragment; rows past R are clamped) ----
  const uint16_t* a_ptr[FM];
  const uint32_t* m_ptr[FM];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    int row = m0 + wm * TL::kWM + fm * 16 + l16;
    row = row < R ? row : R - 1;
    a_ptr[fm] = values + (int64_t)row * vals_per_row + 16 * q;
    m_ptr[fm] = meta + (int64_t)row * meta_per_row + (kPat12 ? (q >> 1) : q);
  }

  // ---- X tile loader: chunk c -> (row c / (BN/8), 8 columns at 8*(c % (BN/8))) ----
  uint4 xr[TL::kXChunks];
  auto load_x = [&](int k0) {
#pragma unroll
    for (int i = 0; i < TL::kXChunks; ++i) {
      const int c = tid + i * NT;
      const int r = c / (BN / 8), col = t0 + 8 * (c % (BN / 8));
      if (col < T)
        xr[i] = *reinterpret_cast<const uint4*>(X + (int64_t)(k0 + r) * T + col);
      else
        xr[i] = make_uint4(0, 0, 0, 0);
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int i = 0; i < TL::kXChunks; ++i) {
      const int c = tid + i * NT;
      const int r = c / (BN / 8), col = 8 * (c % (BN / 8));
      *reinterpret_cast<uint4*>(&xs[buf * TL::kLdsStage + r * TL::kLdsStride + col]) = xr[i];
    }
  };

  uint4 a_cur[FM][2], a_nxt[FM][2];
  uint32_t i_cur[FM], i_nxt[FM];
  auto load_a = [&](int k0, uint4 (&a)[FM][2], uint32_t (&ix)[FM]) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const uint4* p = reinterpret_cast<const uint4*>(a_ptr[fm] + k0 / 2);
      a[fm][0] = p[0];
      a[fm][1] = p[1];
      if constexpr (kPat12) {
        const uint32_t w = m_ptr[fm][k0 / 64];
        ix[fm] = widen_1_2(w >> (16 * (q & 1)));
      } else {
        ix[fm] = m_ptr[fm][k0 / 32];
      }
    }
  };

  float4_t acc[FM][FN];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = float4_t{0.f, 0.f, 0.f, 0.f};

  const int nsteps = K / kKStep;
  load_x(0);
  load_a(0, a_cur, i_cur);
  store_x(0);
  __syncthreads();

  // LDS read offsets of this lane for the transposing loads (see the layout note above):
  // lane i' of a 16-lane block reads row kb + (i' >> 2), columns 4 * (i' & 3) .. +3.
  const int tr_row = l16 >> 2, tr_col = 4 * (l16 & 3);

  for (int s = 0; s < nsteps; ++s) {
    const int cur = s & 1;
    const bool more = s + 1 < nsteps;
    if (more) {
      load_x((s + 1) * kKStep);
      load_a((s + 1) * kKStep, a_nxt, i_nxt);
    }
    const uint16_t* xb = xs + cur * TL::kLdsStage;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      // K rows (within the step) holding B elements 0..7 and 8..15 of lane group q
      const int kb0 = 32 * (q >> 1) + 16 * half + 8 * (q & 1);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const uint16_t* base = xb + tr_row * TL::kLdsStride + wn * TL::kWN + fn * 16 + tr_col;
        const short4_t b0 = lds_tr_read(base + (kb0 + 0) * TL::kLdsStride);
        const short4_t b1 = lds_tr_read(base + (kb0 + 4) * TL::kLdsStride);
        const short4_t b2 = lds_tr_read(base + (kb0 + 64) * TL::kLdsStride);
        const short4_t b3 = lds_tr_read(base + (kb0 + 68) * TL::kLdsStride);
        const short8_t lo = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
        const short8_t hi = __builtin_shufflevector(b2, b3, 0, 1, 2, 3, 4, 5, 6, 7);
        const short16_t bfrag =
            __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
          acc[fm][fn] = smfmac<BF16>(a_cur[fm][half], bfrag, acc[fm][fn], i_cur[fm], half);
      }
    }
    if (more) {
      store_x(cur ^ 1);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        a_cur[fm][0] = a_nxt[fm][0];
        a_cur[fm][1] = a_nxt[fm][1];
        i_cur[fm] = i_nxt[fm];
      }
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds rows 4q..4q+3, column l16 of each 16x16 fragment ----
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int col = t0 + wn * TL::kWN + fn * 16 + l16;
      if (col >= T) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m0 + wm * TL::kWM + fm * 16 + 4 * q + i;
        if (row < R) store_from_f32<YT>(Y, (int64_t)row * T + col, acc[fm][fn][i]);
      }
    }
  }
}

// ===========================================================================
// Shape-agnostic kernel: any N:M, any dtype, any shape with K % M == 0.
// ===========================================================================
constexpr int kGT = 64;   // tile rows and columns
constexpr int kGK = 32;   // K per step (a multiple of every supported M)

template <int DT, int YT, int N, int M>
__global__ void __launch_bounds__(256) generic_spmm_kernel(const void* __restrict__ values,
                                                           const uint32_t* __restrict__ meta,
                                                           const void* __restrict__ X,
                                                           void* __restrict__ Y, int64_t R,
                                                           int64_t K, int64_t T) {
  constexpr int b = meta_bits(M);
  __shared__ float ws[kGT][kGK + 1];
  __shared__ float xs[kGK][kGT + 4];
  const int tid = threadIdx.x;
  const int64_t m0 = (int64_t)blockIdx.y * kGT, t0 = (int64_t)blockIdx.x * kGT;
  const int64_t gpr = K / M, wpr = (gpr * N * b + 31) / 32;
  const int ty = tid / 16, tx = tid % 16;
  float acc[4][4] = {};

  for (int64_t k0 = 0; k0 < K; k0 += kGK) {
    // expand the compressed rows of this K step into fp32 (zeros where pruned)
    constexpr int kGroupsPerRow = kGK / M;
    for (int i = tid; i < kGT * kGroupsPerRow; i += 256) {
      const int r = i / kGroupsPerRow, gl = i % kGroupsPerRow;
      const int64_t row = m0 + r, g = k0 / M + gl;
      float o[M];
#pragma unroll
      for (int e = 0; e < M; ++e) o[e] = 0.f;
      if (row < R && g < gpr) {
        const uint32_t* mrow = meta + row * wpr;
#pragma unroll
        for (int j = 0; j < N; ++j) {
          const int64_t bit = (g * N + j) * b;
          uint64_t window = mrow[bit / 32];
          if ((bit % 32) + b > 32) window |= (uint64_t)mrow[bit / 32 + 1] << 32;
          const int p = (int)((window >> (bit % 32)) & ((1u << b) - 1u));
          const float v = load_as_f32<DT>(values, row * (gpr * N) + g * N + j);
#pragma unroll
          for (int e = 0; e < M; ++e) o[e] = (p == e) ? v : o[e];
        }
      }
#pragma unroll
      for (int e = 0; e < M; ++e) ws[r][gl * M + e] = o[e];
    }
    for (int i = tid; i < kGK * kGT; i += 256) {
      const int kk = i / kGT, c = i % kGT;
      const int64_t k = k0 + kk, col = t0 + c;
      xs[kk][c] = (k < K && col < T) ? load_as_f32<DT>(X, k * T + col) : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < kGK; ++kk) {
      float wv[4], xv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[i] = ws[ty * 4 + i][kk];
#pragma unroll
      for (int j = 0; j < 4; ++j) xv[j] = xs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(wv[i], xv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = m0 + ty * 4 + i;
    if (row >= R) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = t0 + tx * 4 + j;
      if (col < T) store_from_f32<YT>(Y, row * T + col, acc[i][j]);
    }
  }
}

__global__ void zero_fill_kernel(uint32_t* __restrict__ p, int64_t words, int64_t tail_halves) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < words) p[i] = 0u;
  if (i == words && tail_halves) reinterpret_cast<uint16_t*>(p + words)[0] = 0;
}

template <int DT, int YT>
hipError_t run_generic(const void* values, const uint32_t* meta, int64_t R, int64_t K, int n,
                       int m, const void* X, int64_t T, void* Y, hipStream_t s) {
  const dim3 grid((unsigned)((T + kGT - 1) / kGT), (unsigned)((R + kGT - 1) / kGT));
#define NM_G(NN, MM)                                                                         \
  if (n == NN && m == MM) {                                                                  \
    generic_spmm_kernel<DT, YT, NN, MM><<<grid, 256, 0, s>>>(values, meta, X, Y, R, K, T); \
    return hipGetLastError();                                                                \
  }
  NM_G(1, 2) NM_G(2, 2)
  NM_G(1, 4) NM_G(2, 4) NM_G(3, 4) NM_G(4, 4)
  NM_G(1, 8) NM_G(2, 8) NM_G(3, 8) NM_G(4, 8)
  NM_G(5, 8) NM_G(6, 8) NM_G(7, 8) NM_G(8, 8)
#undef NM_G
  return hipErrorInvalidValue;
}

// Tile configuration of the matrix-core kernel.
constexpr int kBM = 128, kBN = 128, kWavesM = 2, kWavesN = 2;

template <bool BF16, bool kPat12, int YT>
hipError_t run_smfmac(const void* values, const uint32_t* meta, int64_t R, int64_t K,
                      const void* X, int64_t T, void* Y, hipStream_t s) {
  using TL = SmfmacTile<kBM, kBN, kWavesM, kWavesN>;
  const int tiles_m = (int)((R + kBM - 1) / kBM), tiles_n = (int)((T + kBN - 1) / kBN);
  smfmac_spmm_kernel<BF16, kPat12, YT, kBM, kBN, kWavesM, kWavesN>
      <<<tiles_m * tiles_n, TL::kThreads, 0, s>>>(
          static_cast<const uint16_t*>(values), meta, static_cast<const uint16_t*>(X), Y, (int)R,
          (int)K, (int)T, tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_spmm(const void* values, const uint32_t* meta, int64_t R, int64_t K, int n,
                       int m, const void* X, int64_t T, int dt, void* Y, int y_dt, hipStream_t s) {
  if (R == 0 || T == 0) return hipSuccess;
  const bool pat24 = (n == 2 && m == 4), pat12 = (n == 1 && m == 2);
  const bool tiled_shape = K > 0 && K % kKStep == 0 && T % 8 == 0 && R < (1 << 30) &&
                           T < (1 << 30) && K < (1 << 30);
  if (dt != kF32 && (pat24 || pat12) && tiled_shape) {
    const bool yf32 = y_dt == kF32;
#define NM_S(BF, P12)                                                                        \
  return yf32 ? run_smfmac<BF, P12, kF32>(values, meta, R, K, X, T, Y, s)                    \
              : run_smfmac<BF, P12, (BF ? kBF16 : kF16)>(values, meta, R, K, X, T, Y, s);
    if (dt == kBF16) {
      if (pat24) { NM_S(true, false) } else { NM_S(true, true) }
    } else {
      if (pat24) { NM_S(false, false) } else { NM_S(false, true) }
    }
#undef NM_S
  }
  if (K == 0) {
    // empty contraction: Y = 0, written by a fill kernel (safe under stream capture)
    const int64_t words = R * T * (y_dt == kF32 ? 4 : 2) / 4;
    const int64_t tail_halves = (R * T * (y_dt == kF32 ? 4 : 2) % 4) / 2;
    zero_fill_kernel<<<(unsigned)((words + 255) / 256 + 1), 256, 0, s>>>(
        static_cast<uint32_t*>(Y), words, tail_halves);
    return hipGetLastError();
  }
  if (dt == kF32) return run_generic<kF32, kF32>(values, meta, R, K, n, m, X, T, Y, s);
  if (dt == kBF16)
    return y_dt == kF32 ? run_generic<kBF16, kF32>(values, meta, R, K, n, m, X, T, Y, s)
                        : run_generic<kBF16, kBF16>(values, meta, R, K, n, m, X, T, Y, s);
  return y_dt == kF32 ? run_generic<kF16, kF32>(values, meta, R, K, n, m, X, T, Y, s)
                      : run_generic<kF16, kF16>(values, meta, R, K, n, m, X, T, Y, s);
}

}  // namespace nm
