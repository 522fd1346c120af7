// nm_device.h -- device-side building blocks shared by the libnm kernels (gfx950).
//
// Group selection.  ASP's exhaustive search ("量化友好的SR-STE稀疏化训练", section
// "NVIDA Apex内的静态掩码稀疏") keeps, in each group of M, the N positions whose
// magnitudes have the largest sum, the first such tuple on ties.  The kernels reach
// the same set without enumerating patterns: element i is kept iff fewer than N
// elements beat it, where j beats i when |w_j| > |w_i|, or |w_j| == |w_i| and j < i.
// Every optimal pattern holds all elements above the N-th largest magnitude plus
// enough elements equal to it; taking the lowest-index equal ones gives the
// lexicographically first optimal tuple, and the count rule takes exactly those
// (it is also the "drop the smallest of each group" reading of "[리뷰] Accelerating
// Sparse Deep Neural Networks", section "Step-2: Weight Pruning").
//
// Magnitudes are compared as integers: the bit pattern with the sign cleared orders
// exactly as |w| for every finite value and infinity (and puts NaN above Inf).  int8
// weights (stored as raw bytes) use the integer magnitude of the two's-complement value,
// |-128| = 128.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nm {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// OCP FP8 E4M3 bytes: a type of its own, so that its magnitude key (sign-cleared bits,
// NaN above 448) is not int8's.
enum class fp8_t : uint8_t {};

// Raw storage of one element: uint8_t for int8, fp8_t for fp8, uint16_t for bf16 / fp16,
// uint32_t for fp32.  key(raw) is the element's magnitude as an unsigned integer.
template <typename E>
struct Elem;
template <>
struct Elem<fp8_t> {
  static constexpr int kBytes = 1;
  __host__ __device__ static constexpr uint32_t key(uint32_t raw) { return raw & 0x7Fu; }
};
template <>
struct Elem<uint8_t> {
  static constexpr int kBytes = 1;
  __host__ __device__ static constexpr uint32_t key(uint32_t raw) {
    const int x = (int)((raw & 0xFFu) ^ 0x80u) - 128;  // the signed value
    return (uint32_t)(x < 0 ? -x : x);
  }
};
template <>
struct Elem<uint16_t> {
  static constexpr uint32_t kKeyMask = 0x7FFFu;
  static constexpr int kBytes = 2;
  __host__ __device__ static constexpr uint32_t key(uint32_t raw) { return raw & kKeyMask; }
};
template <>
struct Elem<uint32_t> {
  static constexpr uint32_t kKeyMask = 0x7FFFFFFFu;
  static constexpr int kBytes = 4;
  __host__ __device__ static constexpr uint32_t key(uint32_t raw) { return raw & kKeyMask; }
};

// OCP FP8 E4M3 byte -> fp32 (exact): bias 7, subnormals f * 2^-9, S.1111.111 is NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, f = b & 7u;
  float v = e == 0 ? (float)f * 0x1p-9f : __builtin_ldexpf((float)(8u + f), (int)e - 10);
  v = (e == 15u && f == 7u) ? __builtin_nanf("") : v;
  return (b & 0x80u) ? -v : v;
}

constexpr int meta_bits(int m) { return m == 2 ? 1 : m == 4 ? 2 : m == 8 ? 3 : m == 16 ? 4 : 0; }

// Bit i of the result is set iff element i of the group is kept (count rule above).
template <int N, int M>
__device__ __forceinline__ uint32_t keep_bits(const uint32_t (&key)[M]) {
  int beaten[M];
#pragma unroll
  for (int i = 0; i < M; ++i) beaten[i] = 0;
#pragma unroll
  for (int i = 0; i < M; ++i) {
#pragma unroll
    for (int j = i + 1; j < M; ++j) {
      const int i_wins = key[i] >= key[j];  // equal magnitudes: the lower index wins
      beaten[j] += i_wins;
      beaten[i] += 1 - i_wins;
    }
  }
  uint32_t keep = 0;
#pragma unroll
  for (int i = 0; i < M; ++i) keep |= (beaten[i] < N ? 1u : 0u) << i;
  return keep;
}

// 2:4 for elements of at most 16 bits.  The composite key 4 |w| + (3 - i) is distinct
// within a group and orders as the rule above (larger magnitude first, then the lower
// index), so the kept pair is the top two of four distinct integers: eight min / max
// operations instead of six pairwise counts.  Returns the kept positions p0 < p1.
__device__ __forceinline__ void top2_of_4(uint32_t k0, uint32_t k1, uint32_t k2, uint32_t k3,
                                          int& p0, int& p1) {
  const uint32_t c0 = (k0 << 2) | 3u, c1 = (k1 << 2) | 2u, c2 = (k2 << 2) | 1u, c3 = k3 << 2;
  const uint32_t a = max(c0, c1), b = min(c0, c1), c = max(c2, c3), d = min(c2, c3);
  const uint32_t t1 = max(a, c), t2 = max(min(a, c), max(b, d));
  const uint32_t l1 = t1 & 3u, l2 = t2 & 3u;
  p0 = (int)(3u - max(l1, l2));
  p1 = (int)(3u - min(l1, l2));
}

// 4:8 for elements of at most 16 bits.  The composite key 8 |w| + (7 - i) is again
// distinct within a group and orders as the rule above, so the kept set is the top four
// of eight distinct integers.  Each half of four is sorted (five compare-exchanges), the
// first half descending and the second ascending; the eight then form a bitonic sequence,
// whose element-wise maxima of the two halves are its four largest values.  That is 24
// min / max operations instead of 28 pairwise counts.  Returns the keep mask (bit i set iff
// element i is kept).
__host__ __device__ __forceinline__ uint32_t top4_of_8(const uint32_t (&key)[8]) {
  uint32_t a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = (key[i] << 3) | (7u - i);
    b[i] = (key[4 + i] << 3) | (3u - i);
  }
  constexpr int kNet[5][2] = {{0, 1}, {2, 3}, {0, 2}, {1, 3}, {1, 2}};  // sorts four
#pragma unroll
  for (int c = 0; c < 5; ++c) {
    const int i = kNet[c][0], j = kNet[c][1];
    const uint32_t ahi = a[i] > a[j] ? a[i] : a[j], alo = a[i] > a[j] ? a[j] : a[i];
    const uint32_t bhi = b[i] > b[j] ? b[i] : b[j], blo = b[i] > b[j] ? b[j] : b[i];
    a[i] = ahi;  // descending
    a[j] = alo;
    b[i] = blo;  // ascending
    b[j] = bhi;
  }
  uint32_t keep = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t t = a[i] > b[i] ? a[i] : b[i];
    keep |= 0x80u >> (t & 7u);
  }
  return keep;
}

template <typename E, int N, int M>
constexpr bool fast24() { return N == 2 && M == 4 && sizeof(E) <= 2; }

template <typename E, int N, int M>
constexpr bool fast48() { return N == 4 && M == 8 && sizeof(E) <= 2; }

// Keep mask of one group: the network above for 4:8 on elements of at most 16 bits, the
// count rule otherwise.
template <typename E, int N, int M>
__device__ __forceinline__ uint32_t group_keep(const uint32_t (&key)[M]) {
  if constexpr (fast48<E, N, M>())
    return top4_of_8(key);
  else
    return keep_bits<N, M>(key);
}

// Kept values of consecutive 2:4 groups gathered with byte permutes (fast24 types):
// 16-bit elements, group g in words 2g, 2g+1 -> word g; 8-bit elements, group g in word
// g -> half g % 2 of word g / 2.
template <typename E, int G>
__device__ __forceinline__ void pack_kept24(const uint32_t* w, const int (&p)[G][2], uint32_t* vw) {
  if constexpr (sizeof(E) == 2) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint32_t sel = (uint32_t)p[g][0] * 0x0202u + (uint32_t)p[g][1] * 0x02020000u + 0x01000100u;
      vw[g] = __builtin_amdgcn_perm(w[2 * g + 1], w[2 * g], sel);
    }
  } else {
    static_assert(G % 2 == 0, "8-bit groups pair up into words");
#pragma unroll
    for (int g = 0; g < G; g += 2) {
      const uint32_t sel = (uint32_t)p[g][0] | ((uint32_t)p[g][1] << 8) |
                           ((uint32_t)p[g + 1][0] + 4u) << 16 | ((uint32_t)p[g + 1][1] + 4u) << 24;
      vw[g / 2] = __builtin_amdgcn_perm(w[g + 1], w[g], sel);
    }
  }
}

// Positions of the N set bits of `keep`, ascending.
template <int N>
__device__ __forceinline__ void kept_positions(uint32_t keep, int (&pos)[N]) {
#pragma unroll
  for (int j = 0; j < N; ++j) {
    pos[j] = __builtin_ctz(keep);
    keep &= keep - 1u;
  }
}

// w[idx] for a compile-time-sized register array and a run-time idx, as a select tree
// (no dynamic register indexing, so nothing spills to scratch).
template <int NW>
__device__ __forceinline__ uint32_t pick_word(const uint32_t* w, int idx) {
  if constexpr (NW == 1) {
    return w[0];
  } else {
    const uint32_t lo = pick_word<NW / 2>(w, idx & (NW / 2 - 1));
    const uint32_t hi = pick_word<NW / 2>(w + NW / 2, idx & (NW / 2 - 1));
    return (idx & (NW / 2)) ? hi : lo;
  }
}

// Element `pos` of a group of M elements stored little-endian in 32-bit words.
template <typename E, int M>
__device__ __forceinline__ uint32_t group_elem(const uint32_t* gw, int pos) {
  if constexpr (sizeof(E) == 2) {
    const uint32_t w = pick_word<(M / 2 > 0 ? M / 2 : 1)>(gw, pos >> 1);
    return (w >> ((pos & 1) * 16)) & 0xFFFFu;
  } else {
    return pick_word<M>(gw, pos);
  }
}

// Element e of a register array of words.
template <typename E>
__device__ __forceinline__ uint32_t word_elem(const uint32_t* w, int e) {
  if constexpr (sizeof(E) == 1)
    return (w[e >> 2] >> ((e & 3) * 8)) & 0xFFu;
  else if constexpr (sizeof(E) == 2)
    return (w[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
  else
    return w[e];
}

// Element `pos` (run-time) of group g (compile-time) of M elements in a register array
// of words that starts at group 0.
template <typename E, int M>
__device__ __forceinline__ uint32_t group_elem_at(const uint32_t* w, int g, int pos) {
  if constexpr (sizeof(E) == 1) {
    if constexpr (M >= 4) {
      const uint32_t word = pick_word<M / 4>(w + g * M / 4, pos >> 2);
      return (word >> (8 * (pos & 3))) & 0xFFu;
    } else {  // two groups of two bytes per word
      return (w[(g * M) / 4] >> (8 * ((g * M) % 4 + pos))) & 0xFFu;
    }
  } else {
    return group_elem<E, M>(w + g * M * (int)sizeof(E) / 4, pos);
  }
}

// Set element e of a register array of words to v (v holds only the element's bits).
template <typename E>
__device__ __forceinline__ void put_elem(uint32_t* w, int e, uint32_t v) {
  if constexpr (sizeof(E) == 1)
    w[e >> 2] |= v << (8 * (e & 3));
  else if constexpr (sizeof(E) == 2)
    w[e >> 1] |= v << (16 * (e & 1));
  else
    w[e] = v;
}

}  // namespace nm
