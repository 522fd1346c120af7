// nm_tmask.hip -- transposable N:M masks (gfx950).
//
// "[论文解读] Accelerated Sparse Neural Training: A Provable and Efficient Method to
// Find N:M Transposable Masks" (ABSTRACT, section "提出的方法"): W is cut into M x M
// blocks and each block keeps at most N entries per row and per column, so W and its
// transpose are both N:M along their contiguous dimension and one mask serves the
// forward product (W X) and the backward one (W^T dY).  The fast method is a greedy
// 2-approximation of the best (maximal kept L1) such mask: take the block's entries
// by descending magnitude and keep an entry while its row and column have room.
//
// One thread per block.  Consecutive threads take consecutive blocks along K, so row
// i of every block of a wave is one contiguous run (M elements per lane, 8 to 32
// bytes), loaded with one or two vector loads.  Each entry gets a composite key, its
// magnitude (sign-cleared bits: NaN > Inf > finite, as for the row mask) above its
// reversed position inside the block, so that a descending order of keys is the
// greedy's order with equal magnitudes in ascending row-major position.  A bitonic
// network sorts the M^2 keys in registers (all indices compile-time), then one pass
// over the sorted keys applies the row and column caps, with the M row counts and M
// column counts held as 4-bit fields of two registers.
#include "nm_device.h"
#include "nm_launch.h"

namespace nm {

namespace {

constexpr int kThreads = 256;

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

template <typename E>
struct TKey {
  using T = uint32_t;  // 15-bit magnitude + up to 6 position bits
};
template <>
struct TKey<uint32_t> {
  using T = uint64_t;  // 31-bit magnitude + up to 6 position bits
};

// Row of M elements as raw element bits, loaded with the widest aligned vectors.
template <typename E, int M>
__device__ __forceinline__ void load_row(const E* p, uint32_t (&v)[M]) {
  constexpr int kBytes = M * (int)sizeof(E);
  uint32_t w[kBytes / 4 > 0 ? kBytes / 4 : 1];
  if constexpr (kBytes == 4) {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (kBytes == 8) {
    const u32x2_t x = *reinterpret_cast<const u32x2_t*>(p);
    w[0] = x[0];
    w[1] = x[1];
  } else {
#pragma unroll
    for (int i = 0; i < kBytes / 16; ++i) {
      const u32x4_t x = reinterpret_cast<const u32x4_t*>(p)[i];
      w[4 * i] = x[0];
      w[4 * i + 1] = x[1];
      w[4 * i + 2] = x[2];
      w[4 * i + 3] = x[3];
    }
  }
#pragma unroll
  for (int j = 0; j < M; ++j) v[j] = word_elem<E>(w, j);
}

template <typename E, int M>
__device__ __forceinline__ void store_row(E* p, const uint32_t (&v)[M]) {
  constexpr int kBytes = M * (int)sizeof(E);
  constexpr int kWords = kBytes / 4 > 0 ? kBytes / 4 : 1;
  uint32_t w[kWords];
#pragma unroll
  for (int i = 0; i < kWords; ++i) w[i] = 0;
#pragma unroll
  for (int j = 0; j < M; ++j) {
    if constexpr (sizeof(E) == 2)
      w[j / 2] |= v[j] << (16 * (j % 2));
    else
      w[j] = v[j];
  }
  if constexpr (kBytes == 4) {
    *reinterpret_cast<uint32_t*>(p) = w[0];
  } else if constexpr (kBytes == 8) {
    *reinterpret_cast<u32x2_t*>(p) = u32x2_t{w[0], w[1]};
  } else {
#pragma unroll
    for (int i = 0; i < kBytes / 16; ++i)
      reinterpret_cast<u32x4_t*>(p)[i] = u32x4_t{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
  }
}

// Sort a[0..L) into descending order (bitonic network, L a power of two).
template <typename T, int L>
__host__ __device__ __forceinline__ void sort_descending(T (&a)[L]) {
#pragma unroll
  for (int k = 2; k <= L; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
#pragma unroll
      for (int i = 0; i < L; ++i) {
        const int l = i ^ j;
        if (l > i) {
          const T x = a[i], y = a[l];
          const T hi = x > y ? x : y, lo = x > y ? y : x;
          // runs with (i & k) == 0 end descending, the others ascending; the last
          // merge (k == L) makes the whole array descending
          if ((i & k) == 0) {
            a[i] = hi;
            a[l] = lo;
          } else {
            a[i] = lo;
            a[l] = hi;
          }
        }
      }
    }
  }
}

// Greedy keep mask of one block (bit r*M + c = entry (r, c) kept).
template <typename E, int N, int M>
__host__ __device__ __forceinline__ uint64_t greedy_keep(const uint32_t (&v)[M][M]) {
  using T = typename TKey<E>::T;
  constexpr int L = M * M, kPosBits = ilog2(L);
  T key[L];
#pragma unroll
  for (int r = 0; r < M; ++r)
#pragma unroll
    for (int c = 0; c < M; ++c) {
      const int e = r * M + c;
      key[e] = ((T)(v[r][c] & Elem<E>::kKeyMask) << kPosBits) | (T)(L - 1 - e);
    }
  if constexpr (L > 1) sort_descending<T, L>(key);
  uint32_t rows = 0, cols = 0;  // 4-bit counters
  uint64_t keep = 0;
#pragma unroll
  for (int t = 0; t < L; ++t) {
    const int e = L - 1 - (int)(key[t] & (T)(L - 1));
    const int r = e / M, c = e % M;
    const uint32_t rc = (rows >> (4 * r)) & 15u, cc = (cols >> (4 * c)) & 15u;
    const bool take = rc < (uint32_t)N && cc < (uint32_t)N;
    rows += take ? (1u << (4 * r)) : 0u;
    cols += take ? (1u << (4 * c)) : 0u;
    keep |= take ? (1ull << e) : 0ull;
  }
  return keep;
}

// kPrune: W_out = W where kept, +0 elsewhere; otherwise mask bytes (1 = kept).
template <typename E, int N, int M, bool kPrune>
__global__ void __launch_bounds__(kThreads) tmask_kernel(const E* __restrict__ W, int64_t K,
                                                         int64_t block_cols, int64_t blocks,
                                                         void* __restrict__ out) {
  const int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (b >= blocks) return;
  const int64_t r0 = (b / block_cols) * M, c0 = (b % block_cols) * M;
  uint32_t v[M][M];
#pragma unroll
  for (int r = 0; r < M; ++r) load_row<E, M>(W + (r0 + r) * K + c0, v[r]);
  const uint64_t keep = greedy_keep<E, N, M>(v);
#pragma unroll
  for (int r = 0; r < M; ++r) {
    if constexpr (kPrune) {
      uint32_t o[M];
#pragma unroll
      for (int c = 0; c < M; ++c) o[c] = ((keep >> (r * M + c)) & 1u) ? v[r][c] : 0u;
      store_row<E, M>(static_cast<E*>(out) + (r0 + r) * K + c0, o);
    } else {
      uint8_t* dst = static_cast<uint8_t*>(out) + (r0 + r) * K + c0;
      const uint32_t bits = (uint32_t)(keep >> (r * M)) & ((1u << M) - 1u);
      // byte c = bit c of the row
      uint64_t bytes = 0;
#pragma unroll
      for (int c = 0; c < M; ++c) bytes |= (uint64_t)((bits >> c) & 1u) << (8 * c);
      if constexpr (M == 8)
        *reinterpret_cast<uint64_t*>(dst) = bytes;
      else if constexpr (M == 4)
        *reinterpret_cast<uint32_t*>(dst) = (uint32_t)bytes;
      else
        *reinterpret_cast<uint16_t*>(dst) = (uint16_t)bytes;
    }
  }
}

template <typename E, bool kPrune>
hipError_t run_tmask(int n, int m, const void* W, int64_t R, int64_t K, void* out, hipStream_t s) {
  const int64_t block_cols = K / m, blocks = (R / m) * block_cols;
  if (blocks == 0) return hipSuccess;
  const unsigned grid = (unsigned)((blocks + kThreads - 1) / kThreads);
  const E* w = static_cast<const E*>(W);
#define NM_TMASK_CASE(NN, MM)                                                                  \
  if (n == NN && m == MM) {                                                                    \
    tmask_kernel<E, NN, MM, kPrune><<<grid, kThreads, 0, s>>>(w, K, block_cols, blocks, out);  \
    return hipGetLastError();                                                                  \
  }
  NM_TMASK_CASE(1, 2) NM_TMASK_CASE(2, 2)
  NM_TMASK_CASE(1, 4) NM_TMASK_CASE(2, 4) NM_TMASK_CASE(3, 4) NM_TMASK_CASE(4, 4)
  NM_TMASK_CASE(1, 8) NM_TMASK_CASE(2, 8) NM_TMASK_CASE(3, 8) NM_TMASK_CASE(4, 8)
  NM_TMASK_CASE(5, 8) NM_TMASK_CASE(6, 8) NM_TMASK_CASE(7, 8) NM_TMASK_CASE(8, 8)
#undef NM_TMASK_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_tmask(const void* W, int elem_bytes, int64_t R, int64_t K, int n, int m,
                        bool prune, void* out, hipStream_t s) {
  if (elem_bytes == 2)
    return prune ? run_tmask<uint16_t, true>(n, m, W, R, K, out, s)
                 : run_tmask<uint16_t, false>(n, m, W, R, K, out, s);
  return prune ? run_tmask<uint32_t, true>(n, m, W, R, K, out, s)
               : run_tmask<uint32_t, false>(n, m, W, R, K, out, s);
}

}  // namespace nm
