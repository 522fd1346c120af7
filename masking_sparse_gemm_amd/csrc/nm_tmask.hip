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
// One thread per block, or per 16-byte-wide run of adjacent blocks (two 4 x 4 blocks of
// 16-bit values, four 2 x 2): consecutive threads take consecutive blocks along K, so
// row i of every block of a wave is one contiguous run, loaded and stored with
// non-temporal vector accesses.  Each entry gets a composite key, its
// magnitude (sign-cleared bits: NaN > Inf > finite, as for the row mask) above its
// reversed position inside the block, so that a descending order of keys is the
// greedy's order with equal magnitudes in ascending row-major position.  An odd-even
// merge network sorts the M^2 keys in registers (all indices compile-time), then one pass
// over the sorted keys applies the row and column caps, with the M row counts and M
// column counts held as 4-bit fields of two registers.
#include <utility>

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
    w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
  } else if constexpr (kBytes == 8) {
    const u32x2_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    w[0] = x[0];
    w[1] = x[1];
  } else {
#pragma unroll
    for (int i = 0; i < kBytes / 16; ++i) {
      const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p) + i);
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
    __builtin_nontemporal_store(w[0], reinterpret_cast<uint32_t*>(p));
  } else if constexpr (kBytes == 8) {
    __builtin_nontemporal_store(u32x2_t{w[0], w[1]}, reinterpret_cast<u32x2_t*>(p));
  } else {
#pragma unroll
    for (int i = 0; i < kBytes / 16; ++i)
      __builtin_nontemporal_store(u32x4_t{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]},
                                  reinterpret_cast<u32x4_t*>(p) + i);
  }
}

// Batcher's odd-even merge sorting network on L = 2^k inputs, as a list of comparator
// pairs (lo, hi) built at compile time: 5 / 63 / 543 comparators for L = 4 / 16 / 64,
// against 6 / 80 / 672 for the bitonic network.
template <int L>
struct SortNet {
  int n = 0;
  int lo[L * L / 2 + 8] = {};
  int hi[L * L / 2 + 8] = {};
  constexpr void merge(int base, int m, int r) {
    const int step = 2 * r;
    if (step < m) {
      merge(base, m, step);
      merge(base + r, m, step);
      for (int i = base + r; i < base + m - r; i += step) add(i, i + r);
    } else {
      add(base, base + r);
    }
  }
  constexpr void sort(int base, int m) {
    if (m > 1) {
      sort(base, m / 2);
      sort(base + m / 2, m / 2);
      merge(base, m, 1);
    }
  }
  constexpr void add(int i, int j) {
    lo[n] = i;
    hi[n] = j;
    ++n;
  }
  constexpr SortNet() { sort(0, L); }
};

template <typename T>
__host__ __device__ __forceinline__ void compare_exchange(T& x, T& y) {
  const T a = x, b = y;
  x = a > b ? a : b;
  y = a > b ? b : a;
}

template <typename T, int L, int... I>
__host__ __device__ __forceinline__ void apply_net(T (&a)[L], std::integer_sequence<int, I...>) {
  constexpr SortNet<L> net{};
  (compare_exchange(a[net.lo[I]], a[net.hi[I]]), ...);
}

// Sort a[0..L) into descending order (L a power of two).
template <typename T, int L>
__host__ __device__ __forceinline__ void sort_descending(T (&a)[L]) {
  constexpr int kPairs = SortNet<L>{}.n;
  apply_net(a, std::make_integer_sequence<int, kPairs>{});
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
  // The low bits of a sorted key give p = L-1-e: row M-1-p/M, column M-1-p%M.  Counters
  // are kept per reversed row and column (field p/M of `rows`, p%M of `cols`, 4 bits
  // each), which is the same partition, and the kept set is collected by p and reversed
  // at the end.  Each field starts at 8 - N, so it reaches 8 (bit 3 set) exactly when
  // its row or column holds N kept entries: an entry is taken iff neither bit 3 is set.
  constexpr int kLogM = ilog2(M);
  constexpr uint32_t kBias = (uint32_t)(8 - N) * (M == 8 ? 0x11111111u : M == 4 ? 0x1111u : 0x11u);
  uint32_t rows = kBias, cols = kBias;
  uint64_t keep_rev = 0;
#pragma unroll
  for (int t = 0; t < L; ++t) {
    const uint32_t p = (uint32_t)(key[t] & (T)(L - 1));
    const uint32_t sh_r = (p >> kLogM) << 2, sh_c = (p & (M - 1)) << 2;
    const uint32_t full = (rows >> sh_r) | (cols >> sh_c);
    const uint32_t take = ((full >> 3) & 1u) ^ 1u;
    rows += take << sh_r;
    cols += take << sh_c;
    keep_rev |= (uint64_t)take << p;
  }
  if constexpr (L == 64)
    return __builtin_bitreverse64(keep_rev);
  else
    return __builtin_bitreverse32((uint32_t)keep_rev) >> (32 - L);
}

// kPrune: W_out = W where kept, +0 elsewhere; otherwise mask bytes (1 = kept).
// A thread takes BPT horizontally adjacent blocks (BPT * M elements of each row, at
// most 16 bytes), so its loads and stores are as wide as possible and the BPT
// independent sorts interleave.
template <typename E, int N, int M, int BPT, bool kPrune>
__global__ void __launch_bounds__(kThreads) tmask_kernel(const E* __restrict__ W, int64_t K,
                                                         int64_t units_per_row, int64_t units,
                                                         void* __restrict__ out) {
  constexpr int C = BPT * M;  // columns per thread
  const int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (u >= units) return;
  int64_t ur, uc;  // unit row and column
  if (units <= 0xFFFFFFFFll) {  // 32-bit division where it fits (every practical size)
    ur = (uint32_t)u / (uint32_t)units_per_row;
    uc = (uint32_t)u - (uint32_t)ur * (uint32_t)units_per_row;
  } else {
    ur = u / units_per_row;
    uc = u % units_per_row;
  }
  const int64_t r0 = ur * M, c0 = uc * C;
  uint32_t row[M][C];
#pragma unroll
  for (int r = 0; r < M; ++r) load_row<E, C>(W + (r0 + r) * K + c0, row[r]);
  uint64_t keep[BPT];
#pragma unroll
  for (int b = 0; b < BPT; ++b) {
    uint32_t v[M][M];
#pragma unroll
    for (int r = 0; r < M; ++r)
#pragma unroll
      for (int c = 0; c < M; ++c) v[r][c] = row[r][b * M + c];
    keep[b] = greedy_keep<E, N, M>(v);
  }
#pragma unroll
  for (int r = 0; r < M; ++r) {
    if constexpr (kPrune) {
      uint32_t o[C];
#pragma unroll
      for (int b = 0; b < BPT; ++b)
#pragma unroll
        for (int c = 0; c < M; ++c)
          o[b * M + c] = ((keep[b] >> (r * M + c)) & 1u) ? row[r][b * M + c] : 0u;
      store_row<E, C>(static_cast<E*>(out) + (r0 + r) * K + c0, o);
    } else {
      uint8_t* dst = static_cast<uint8_t*>(out) + (r0 + r) * K + c0;
      uint64_t bytes = 0;  // byte j = column j of the thread's row
#pragma unroll
      for (int b = 0; b < BPT; ++b)
#pragma unroll
        for (int c = 0; c < M; ++c)
          bytes |= (uint64_t)((keep[b] >> (r * M + c)) & 1u) << (8 * (b * M + c));
      static_assert(C <= 8, "at most 16 bytes of 16-bit values or 8 fp32 per thread row");
      if constexpr (C == 8) {
        __builtin_nontemporal_store(bytes, reinterpret_cast<uint64_t*>(dst));
      } else if constexpr (C == 4) {
        __builtin_nontemporal_store((uint32_t)bytes, reinterpret_cast<uint32_t*>(dst));
      } else {
        __builtin_nontemporal_store((uint16_t)bytes, reinterpret_cast<uint16_t*>(dst));
      }
    }
  }
}

template <typename E, int N, int M, int BPT, bool kPrune>
hipError_t launch_tmask_bpt(const E* w, int64_t R, int64_t K, void* out, hipStream_t s) {
  const int64_t per_row = K / (BPT * M), units = (R / M) * per_row;
  if (units == 0) return hipSuccess;
  tmask_kernel<E, N, M, BPT, kPrune>
      <<<(unsigned)((units + kThreads - 1) / kThreads), kThreads, 0, s>>>(w, K, per_row, units, out);
  return hipGetLastError();
}

template <typename E, int N, int M, bool kPrune>
hipError_t launch_tmask_nm(const E* w, int64_t R, int64_t K, void* out, hipStream_t s) {
  // widest thread: BPT blocks side by side, up to 16 bytes of a row
  constexpr int kWide = 16 / (M * (int)sizeof(E)) > 1 ? 16 / (M * (int)sizeof(E)) : 1;
  if constexpr (kWide > 1) {
    if (K % (kWide * M) == 0) return launch_tmask_bpt<E, N, M, kWide, kPrune>(w, R, K, out, s);
  }
  return launch_tmask_bpt<E, N, M, 1, kPrune>(w, R, K, out, s);
}

template <typename E, bool kPrune>
hipError_t run_tmask(int n, int m, const void* W, int64_t R, int64_t K, void* out, hipStream_t s) {
  if (R == 0 || K == 0) return hipSuccess;
  const E* w = static_cast<const E*>(W);
#define NM_TMASK_CASE(NN, MM) \
  if (n == NN && m == MM) return launch_tmask_nm<E, NN, MM, kPrune>(w, R, K, out, s);
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
