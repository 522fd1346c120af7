// nm_perm.hip -- channel permutation before N:M masking (gfx950).
//
// "[리뷰] Accelerating Sparse Deep Neural Networks", section "Step-2: Weight Pruning"
// (Fig. 6): permuting the weight's columns before the mask is taken spreads the large
// values over the groups, so the mask keeps a larger total magnitude.  The objective is
// the kept L1 of the N:M mask of W[:, perm]; only which columns share a group matters.
//
// The search is rounds of pairwise swaps.  A round evaluates, for every pair of groups
// (g1 < g2), the gain in kept L1 of swapping position a of g1 with position b of g2,
// summed over all rows, and keeps the best (a, b) of each pair; the host then applies
// positive gains to disjoint pairs in descending order.  The evaluation is the costly,
// data-parallel part (pairs x rows x M^2 swaps) and runs here:
//
//  * permute_kernel gathers W[:, perm] into a contiguous copy (one pass over W), so that
//    every later read of a group is a contiguous run of M elements;
//  * gains_kernel gives each thread one pair of groups; a workgroup covers 16 x 16 pairs
//    and walks the rows in chunks of 32, staging the magnitudes of its 32 groups in LDS
//    together with, per group, row and position a, the kept sums of the other M-1
//    magnitudes: A[a] (top N of them) and B[a] (top N-1).  Putting x in place of
//    position a then keeps max(A[a], B[a] + x), so one swap costs two max and four adds:
//      delta(a, b) = max(A1[a], B1[a] + u2[b]) + max(A2[b], B2[b] + u1[a]) - T1 - T2.
//
// Gains are accumulated in fp32 (exact whenever the magnitudes are multiples of a common
// power of two whose sums stay below 2^24 of it; otherwise the rounding of an fp32 sum
// over the rows).
#include <algorithm>
#include <vector>

#include "nm_device.h"
#include "nm_launch.h"

namespace nm {

namespace {

constexpr int kThreads = 256;
constexpr int kPB = 16;        // groups per block side: a workgroup takes 16 x 16 pairs
constexpr int kRowChunk = 32;  // rows staged in LDS at a time

enum { kF32 = 0, kF16 = 1, kBF16 = 2, kI8 = 3, kFP8 = 5 };

template <int DT>
__device__ __forceinline__ float magnitude(const void* W, int64_t i) {
  float x;
  if constexpr (DT == kF32) {
    x = fabsf(static_cast<const float*>(W)[i]);
  } else if constexpr (DT == kBF16) {
    x = fabsf(__uint_as_float((uint32_t) static_cast<const uint16_t*>(W)[i] << 16));
  } else if constexpr (DT == kF16) {
    x = fabsf((float)__builtin_bit_cast(_Float16, static_cast<const uint16_t*>(W)[i]));
  } else if constexpr (DT == kFP8) {
    x = fabsf(e4m3_to_f32(static_cast<const uint8_t*>(W)[i]));
  } else {
    x = fabsf((float) static_cast<const int8_t*>(W)[i]);
  }
  return x != x ? __builtin_inff() : x;  // NaN ranks above every magnitude
}

// Wp[r, i] = |W[r, perm[i]]| as fp32 (one thread per element; a row's gathers stay in
// the caches the row's first touches fill).
template <int DT>
__global__ void __launch_bounds__(kThreads) permute_kernel(const void* __restrict__ W, int64_t R,
                                                           int64_t K,
                                                           const int32_t* __restrict__ perm,
                                                           float* __restrict__ Wp) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= R * K) return;
  const int64_t r = idx / K, i = idx % K;
  Wp[idx] = magnitude<DT>(W, r * K + perm[i]);
}

// Sum of the n largest of the m values v (insertion-sorted copy, m <= 8).
template <int M>
__device__ __forceinline__ float top_sum(const float (&v)[M], int take) {
  float c[M];
#pragma unroll
  for (int i = 0; i < M; ++i) c[i] = v[i];
  // sorting network by repeated passes (M is tiny and compile-time)
#pragma unroll
  for (int i = 0; i < M; ++i)
#pragma unroll
    for (int j = 0; j < M - 1; ++j) {
      const float hi = fmaxf(c[j], c[j + 1]), lo = fminf(c[j], c[j + 1]);
      c[j] = hi;
      c[j + 1] = lo;
    }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < M; ++i) s += (i < take) ? c[i] : 0.f;
  return s;
}

// Per row and group of the LDS stage: magnitudes u[M], A[M], B[M] and T (kept sum).
template <int M>
struct StageRow {
  float u[M], A[M], B[M], T;
};

template <int N, int M>
__global__ void __launch_bounds__(kThreads) gains_kernel(const float* __restrict__ Wp, int64_t R,
                                                         int64_t K, int nblocks,
                                                         float* __restrict__ gain,
                                                         int32_t* __restrict__ pick) {
  // block pair (b1, b2) with b1 <= b2, from the linear workgroup index
  int b1 = 0, rem = (int)blockIdx.x;
  while (rem >= nblocks - b1) {
    rem -= nblocks - b1;
    ++b1;
  }
  const int b2 = b1 + rem;
  const int64_t G = K / M;
  __shared__ StageRow<M> st[kRowChunk][2 * kPB];
  const int tid = threadIdx.x;
  const int64_t g1 = (int64_t)b1 * kPB + tid / kPB, g2 = (int64_t)b2 * kPB + tid % kPB;
  const bool active = g1 < G && g2 < G && g1 < g2;
  const int s1 = tid / kPB, s2 = kPB + tid % kPB;  // stage slots of the two groups
  float acc[M * M];
#pragma unroll
  for (int i = 0; i < M * M; ++i) acc[i] = 0.f;

  for (int64_t r0 = 0; r0 < R; r0 += kRowChunk) {
    // stage: 32 rows x 32 groups, one (row, group) per thread and pass
    for (int e = tid; e < kRowChunk * 2 * kPB; e += kThreads) {
      const int rr = e / (2 * kPB), slot = e % (2 * kPB);
      const int64_t row = r0 + rr;
      const int64_t g = (slot < kPB) ? (int64_t)b1 * kPB + slot : (int64_t)b2 * kPB + slot - kPB;
      StageRow<M>& sr = st[rr][slot];
      float u[M];
      if (row < R && g < G) {
#pragma unroll
        for (int i = 0; i < M; ++i) u[i] = Wp[row * K + g * M + i];
      } else {
#pragma unroll
        for (int i = 0; i < M; ++i) u[i] = 0.f;
      }
#pragma unroll
      for (int a = 0; a < M; ++a) {
        float o[M];
#pragma unroll
        for (int i = 0; i < M; ++i) o[i] = (i == a) ? 0.f : u[i];  // magnitudes are >= 0
        sr.u[a] = u[a];
        sr.A[a] = top_sum<M>(o, N);
        sr.B[a] = top_sum<M>(o, N - 1);
      }
      sr.T = top_sum<M>(u, N);
    }
    __syncthreads();
    if (active) {
      const int rows = (int)((R - r0) < kRowChunk ? (R - r0) : kRowChunk);
      for (int rr = 0; rr < rows; ++rr) {
        const StageRow<M>& p = st[rr][s1];
        const StageRow<M>& q = st[rr][s2];
        const float base = p.T + q.T;
#pragma unroll
        for (int a = 0; a < M; ++a)
#pragma unroll
          for (int b = 0; b < M; ++b)
            acc[a * M + b] +=
                (fmaxf(p.A[a], p.B[a] + q.u[b]) + fmaxf(q.A[b], q.B[b] + p.u[a])) - base;
      }
    }
    __syncthreads();
  }
  if (active) {
    // first strict maximum; the value is carried along so that no register array is
    // indexed at run time (which moved the 64 accumulators of 8-wide groups to scratch
    // memory)
    int best = 0;
    float bv = acc[0];
#pragma unroll
    for (int i = 1; i < M * M; ++i) {
      const bool up = acc[i] > bv;
      best = up ? i : best;
      bv = up ? acc[i] : bv;
    }
    gain[g1 * G + g2] = bv;
    pick[g1 * G + g2] = best;
  }
}

template <int DT>
hipError_t run_permute(const void* W, int64_t R, int64_t K, const int32_t* perm, float* Wp,
                       hipStream_t s) {
  const int64_t n = R * K;
  permute_kernel<DT><<<(unsigned)((n + kThreads - 1) / kThreads), kThreads, 0, s>>>(W, R, K, perm,
                                                                                    Wp);
  return hipGetLastError();
}

hipError_t launch_permute(const void* W, int dt, int64_t R, int64_t K, const int32_t* perm,
                          float* Wp, hipStream_t s) {
  switch (dt) {
    case kF32: return run_permute<kF32>(W, R, K, perm, Wp, s);
    case kF16: return run_permute<kF16>(W, R, K, perm, Wp, s);
    case kBF16: return run_permute<kBF16>(W, R, K, perm, Wp, s);
    case kFP8: return run_permute<kFP8>(W, R, K, perm, Wp, s);
    default: return run_permute<kI8>(W, R, K, perm, Wp, s);
  }
}

hipError_t launch_gains_kernel(const float* Wp, int64_t R, int64_t K, int n, int m, float* gain,
                               int32_t* pick, hipStream_t s) {
  const int64_t G = K / m;
  const int nb = (int)((G + kPB - 1) / kPB);
  const unsigned grid = (unsigned)((int64_t)nb * (nb + 1) / 2);
#define NM_PG(NN, MM)                                                                       \
  if (n == NN && m == MM) {                                                                 \
    gains_kernel<NN, MM><<<grid, kThreads, 0, s>>>(Wp, R, K, nb, gain, pick);               \
    return hipGetLastError();                                                               \
  }
  NM_PG(1, 2) NM_PG(2, 2)
  NM_PG(1, 4) NM_PG(2, 4) NM_PG(3, 4) NM_PG(4, 4)
  NM_PG(1, 8) NM_PG(2, 8) NM_PG(3, 8) NM_PG(4, 8)
  NM_PG(5, 8) NM_PG(6, 8) NM_PG(7, 8) NM_PG(8, 8)
#undef NM_PG
  return hipErrorInvalidValue;
}

}  // namespace

size_t perm_workspace_bytes(int64_t R, int64_t K, int m) {
  const int64_t G = K / m;
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  return up((size_t)R * K * 4) + up((size_t)K * 4) + up((size_t)G * G * 4) +
         up((size_t)G * G * 4);
}

namespace {
struct Workspace {
  float* Wp;
  int32_t* perm;
  float* gain;
  int32_t* pick;
};
Workspace carve(void* ws, int64_t R, int64_t K, int m) {
  const int64_t G = K / m;
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  uint8_t* p = static_cast<uint8_t*>(ws);
  Workspace w;
  w.Wp = reinterpret_cast<float*>(p);
  p += up((size_t)R * K * 4);
  w.perm = reinterpret_cast<int32_t*>(p);
  p += up((size_t)K * 4);
  w.gain = reinterpret_cast<float*>(p);
  p += up((size_t)G * G * 4);
  w.pick = reinterpret_cast<int32_t*>(p);
  return w;
}
}  // namespace

hipError_t launch_perm_gains(const void* W, int dt, int64_t R, int64_t K, int n, int m,
                             const int32_t* perm, float* gain, int32_t* pick, void* workspace,
                             hipStream_t s) {
  Workspace w = carve(workspace, R, K, m);
  hipError_t e = launch_permute(W, dt, R, K, perm, w.Wp, s);
  if (e != hipSuccess) return e;
  return launch_gains_kernel(w.Wp, R, K, n, m, gain, pick, s);
}

hipError_t run_perm_search(const void* W, int dt, int64_t R, int64_t K, int n, int m,
                           int max_rounds, int32_t* perm_host, int* rounds, void* workspace,
                           hipStream_t s) {
  const int64_t G = K / m;
  Workspace w = carve(workspace, R, K, m);
  std::vector<float> gain((size_t)(G * G));
  std::vector<int32_t> pick((size_t)(G * G));
  std::vector<int64_t> cand;
  std::vector<uint8_t> used((size_t)G);
  int done = 0;
  for (int round = 0; round < max_rounds; ++round) {
    hipError_t e = hipMemcpyAsync(w.perm, perm_host, (size_t)K * 4, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = launch_permute(W, dt, R, K, w.perm, w.Wp, s);
    if (e == hipSuccess) e = launch_gains_kernel(w.Wp, R, K, n, m, w.gain, w.pick, s);
    if (e == hipSuccess)
      e = hipMemcpyAsync(gain.data(), w.gain, gain.size() * 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess)
      e = hipMemcpyAsync(pick.data(), w.pick, pick.size() * 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return e;
    // positive gains in descending order, ties to the smaller (g1, g2); apply each pair
    // whose two groups are still untouched in this round
    cand.clear();
    for (int64_t g1 = 0; g1 < G; ++g1)
      for (int64_t g2 = g1 + 1; g2 < G; ++g2)
        if (gain[g1 * G + g2] > 0.f) cand.push_back(g1 * G + g2);
    std::stable_sort(cand.begin(), cand.end(),
                     [&](int64_t x, int64_t y) { return gain[x] > gain[y]; });
    std::fill(used.begin(), used.end(), 0);
    int applied = 0;
    for (int64_t c : cand) {
      const int64_t g1 = c / G, g2 = c % G;
      if (used[g1] || used[g2]) continue;
      const int a = pick[c] / m, b = pick[c] % m;
      std::swap(perm_host[g1 * m + a], perm_host[g2 * m + b]);
      used[g1] = used[g2] = 1;
      ++applied;
    }
    if (!applied) break;
    ++done;
  }
  if (rounds) *rounds = done;
  return hipSuccess;
}

}  // namespace nm
