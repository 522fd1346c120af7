// nm_compress.hip -- mask, compress and decompress kernels (gfx950).
//
// These passes move bytes and compare integers; no matrix core is involved.  Their
// roofline is HBM bandwidth, but the selection is enough vector work to bound them when it
// is written naively, so it is kept lean (a top-two network for 2:4, byte permutes for the
// kept values, wave-uniform index math).  The fast ("flat") kernels treat W as one stream
// of 16-byte units: a lane loads one unit (8 x 16-bit or 4 x fp32 elements, or 8 fp32 for
// M = 8) with a single coalesced 16-byte load, selects its groups in registers, writes its
// kept values with one 4/8/16-byte store and packs its metadata bits into 32-bit words
// together with its neighbours: wave shuffles when a whole number of lanes fills a word, a
// per-wave LDS bit buffer otherwise.  The flat kernels need every row to hold a whole
// number of units and of metadata words, so that rows concatenate into one stream; any
// other shape uses the simple per-group / per-word kernels at the bottom, which make no
// such assumption and loop over their work with a capped grid (nm_grid.h), so that no
// accepted shape needs more work-items than one launch may have.
//
// Formats ("[리뷰] Accelerating Sparse Deep Neural Networks", section
// "2:4 Sparsity의 benefits"): values hold the N kept elements of each group in
// ascending position order; metadata field f = g*N + j of a row holds position
// j of group g in b = log2(M) bits at bit f*b of the row, least significant first.
// The blocked layout stores the same values and bits in blocks of 16 rows x 64
// columns (include/nm.h).  Its kernels give each wave one block, or two consecutive
// blocks where a dense row segment would otherwise be half a cache line, and stage dense
// outputs (mask, decompressed weight) through LDS so that every store instruction writes
// whole row segments: lines assembled from several store instructions measured extra HBM
// write traffic.
#include <utility>

#include "nm_device.h"
#include "nm_grid.h"
#include "nm_launch.h"

namespace nm {

namespace {

constexpr int kThreads = 256;
constexpr int kUnitsPerThread = 4;

template <typename E, int M>
struct UnitShape {
  static constexpr int kElems = (16 / (int)sizeof(E)) > M ? (16 / (int)sizeof(E)) : M;
  static constexpr int kWords = kElems * (int)sizeof(E) / 4;  // 32-bit words loaded
  static constexpr int kGroups = kElems / M;
};

template <int NW>
__device__ __forceinline__ void load_words(const uint32_t* p, uint32_t (&w)[NW]) {
  static_assert(NW % 4 == 0, "units are whole 16-byte vectors");
#pragma unroll
  for (int i = 0; i < NW / 4; ++i) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p) + i);
    w[4 * i + 0] = v[0];
    w[4 * i + 1] = v[1];
    w[4 * i + 2] = v[2];
    w[4 * i + 3] = v[3];
  }
}

template <int NW>
__device__ __forceinline__ void store_words(uint32_t* p, const uint32_t (&w)[NW]) {
  if constexpr (NW == 4) {
    __builtin_nontemporal_store(u32x4_t{w[0], w[1], w[2], w[3]}, reinterpret_cast<u32x4_t*>(p));
  } else if constexpr (NW == 2) {
    __builtin_nontemporal_store(u32x2_t{w[0], w[1]}, reinterpret_cast<u32x2_t*>(p));
  } else if constexpr (NW == 1) {
    __builtin_nontemporal_store(w[0], p);
  } else {
#pragma unroll
    for (int i = 0; i < NW; ++i) p[i] = w[i];
  }
}

// Selection for every group of one unit: kept positions and the unit's metadata bits.
template <typename E, int N, int M>
struct UnitSelection {
  using S = UnitShape<E, M>;
  int pos[S::kGroups][N];
  uint32_t keep[S::kGroups];

  __device__ __forceinline__ void run(const uint32_t (&w)[S::kWords]) {
#pragma unroll
    for (int g = 0; g < S::kGroups; ++g) {
      uint32_t key[M];
#pragma unroll
      for (int i = 0; i < M; ++i) key[i] = Elem<E>::key(word_elem<E>(w, g * M + i));
      if constexpr (fast24<E, N, M>()) {
        int p0, p1;
        top2_of_4(key[0], key[1], key[2], key[3], p0, p1);
        pos[g][0] = p0;
        pos[g][1] = p1;
        keep[g] = (1u << p0) | (1u << p1);
      } else {
        keep[g] = group_keep<E, N, M>(key);
        kept_positions<N>(keep[g], pos[g]);
      }
    }
  }
  // this unit's metadata: S::kGroups * N fields of b bits, first field in the low bits
  // (up to 48 bits: sixteen int8 elements at 8:8)
  __device__ __forceinline__ uint64_t meta_bits_of_unit() const {
    constexpr int b = meta_bits(M);
    uint64_t bits = 0;
#pragma unroll
    for (int g = 0; g < S::kGroups; ++g)
#pragma unroll
      for (int j = 0; j < N; ++j) bits |= (uint64_t)pos[g][j] << ((g * N + j) * b);
    return bits;
  }
};

// OR-reduce `v` over aligned runs of L lanes (L a power of two <= 32).
template <int L>
__device__ __forceinline__ uint32_t or_reduce_lanes(uint32_t v) {
#pragma unroll
  for (int s = 1; s < L; s <<= 1) v |= __shfl_xor(v, s);
  return v;
}

// ---------------------------------------------------------------------------
// Flat mask / compress kernel.
// ---------------------------------------------------------------------------
template <typename E, int N, int M, bool kMask, bool kCompress>
__global__ void __launch_bounds__(kThreads) flat_select_kernel(const uint32_t* __restrict__ W,
                                                               int64_t units,
                                                               uint32_t* __restrict__ values,
                                                               uint32_t* __restrict__ meta,
                                                               uint8_t* __restrict__ mask) {
  using S = UnitShape<E, M>;
  constexpr int b = meta_bits(M);
  constexpr int kUnitBits = S::kGroups * N * b;       // metadata bits per unit
  constexpr int kValWords = S::kGroups * N * (int)sizeof(E) / 4;
  constexpr bool kShuffle = (32 % kUnitBits) == 0;   // a whole number of units per word
  constexpr int kWaveWords = 64 * kUnitBits / 32;    // words one wave-step writes
  __shared__ uint32_t lds_bits[kThreads / 64][kShuffle ? 1 : kWaveWords];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t block_first = (int64_t)blockIdx.x * kThreads * kUnitsPerThread;

#pragma unroll
  for (int it = 0; it < kUnitsPerThread; ++it) {
    const int64_t wave_first = block_first + (int64_t)it * kThreads + wave * 64;
    const int64_t u = wave_first + lane;
    const bool live = u < units;
    uint32_t w[S::kWords];
    if (live) {
      load_words<S::kWords>(W + u * S::kWords, w);
    } else {
#pragma unroll
      for (int i = 0; i < S::kWords; ++i) w[i] = 0;
    }
    UnitSelection<E, N, M> sel;
    sel.run(w);

    if constexpr (kMask) {
      if (live) {
        // one byte per element, 1 = kept
        uint32_t mb[S::kElems / 4];
#pragma unroll
        for (int i = 0; i < S::kElems / 4; ++i) mb[i] = 0;
#pragma unroll
        for (int g = 0; g < S::kGroups; ++g)
#pragma unroll
          for (int i = 0; i < M; ++i) {
            const int e = g * M + i;
            mb[e / 4] |= ((sel.keep[g] >> i) & 1u) << (8 * (e % 4));
          }
        store_words<S::kElems / 4>(reinterpret_cast<uint32_t*>(mask + u * S::kElems), mb);
      }
    }
    if constexpr (kCompress) {
      if (live) {
        uint32_t vw[kValWords];
#pragma unroll
        for (int i = 0; i < kValWords; ++i) vw[i] = 0;
        if constexpr (fast24<E, N, M>()) {
          pack_kept24<E, S::kGroups>(w, sel.pos, vw);
        } else {
#pragma unroll
          for (int g = 0; g < S::kGroups; ++g)
#pragma unroll
            for (int j = 0; j < N; ++j) {
              const uint32_t v = group_elem_at<E, M>(w, g, sel.pos[g][j]);
              put_elem<E>(vw, g * N + j, v);  // value index inside the unit
            }
        }
        store_words<kValWords>(values + u * kValWords, vw);
      }
      const uint64_t bits = live ? sel.meta_bits_of_unit() : 0u;
      if constexpr (kShuffle) {
        constexpr int L = 32 / kUnitBits;  // lanes per metadata word
        const uint32_t word = or_reduce_lanes<L>((uint32_t)bits << ((lane % L) * kUnitBits));
        const int64_t widx = u / L;
        if ((lane % L) == 0 && live) meta[widx] = word;
      } else {
        // bits of lane l start at bit l*kUnitBits of this wave-step's kWaveWords words
        uint32_t* buf = lds_bits[wave];
        for (int i = lane; i < kWaveWords; i += 64) buf[i] = 0;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        const int bit = lane * kUnitBits;
        const int sh = bit % 32;
        atomicOr(&buf[bit / 32], (uint32_t)(bits << sh));
        if (sh + kUnitBits > 32) atomicOr(&buf[bit / 32 + 1], (uint32_t)(bits >> (32 - sh)));
        if (sh + kUnitBits > 64) atomicOr(&buf[bit / 32 + 2], (uint32_t)(bits >> (64 - sh)));
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();
        const int64_t total_words = units * kUnitBits / 32;
        const int64_t first_word = wave_first * kUnitBits / 32;
        for (int i = lane; i < kWaveWords; i += 64)
          if (first_word + i < total_words) meta[first_word + i] = buf[i];
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Flat decompress kernel: one unit of output per lane.
// ---------------------------------------------------------------------------
// 2:4 groups of 8- or 16-bit elements (field 2g, 2g+1 of `bits` = the positions of group
// g): each output word is one byte permute of the group's stored values, with selector
// 0x0c (a zero byte) except where the two positions point; the second position is
// written last, so a repeated position keeps the later value.
template <typename E, int G>
__device__ __forceinline__ void expand24(uint64_t bits, const uint32_t* vw, uint32_t* ow) {
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const uint32_t p0 = (uint32_t)(bits >> (4 * gi)) & 3u;
    const uint32_t p1 = (uint32_t)(bits >> (4 * gi + 2)) & 3u;
    if constexpr (sizeof(E) == 1) {  // the group's two values: bytes 2(gi&1), +1 of a word
      const uint32_t b0 = 2u * (gi & 1);
      uint32_t sel = 0x0C0C0C0Cu;
      sel = (sel & ~(0xFFu << (8 * p0))) | (b0 << (8 * p0));
      sel = (sel & ~(0xFFu << (8 * p1))) | ((b0 + 1u) << (8 * p1));
      ow[gi] = __builtin_amdgcn_perm(0u, vw[gi >> 1], sel);
    } else {  // the group's two values are word gi; slot s is bytes 2s, 2s+1 of 8
      uint64_t sel = 0x0C0C0C0C0C0C0C0Cull;
      sel = (sel & ~(0xFFFFull << (16 * p0))) | (0x0100ull << (16 * p0));
      sel = (sel & ~(0xFFFFull << (16 * p1))) | (0x0302ull << (16 * p1));
      ow[2 * gi] = __builtin_amdgcn_perm(0u, vw[gi], (uint32_t)sel);
      ow[2 * gi + 1] = __builtin_amdgcn_perm(0u, vw[gi], (uint32_t)(sel >> 32));
    }
  }
}

// 4:8 groups of 16-bit elements (fields 4g .. 4g+3 of `bits`, 3 bits each, the positions of
// group g's four values, which sit in words 2g and 2g+1): byte i of `slot` records 1 + the
// value written to position i (0: none), the fields taken in order so that a repeated
// position keeps the later value; each output word (positions 2w, 2w+1) is then one byte
// permute of the two value words, value j being bytes 2j, 2j+1 and selector 0x0c a zero byte.
template <int G>
__device__ __forceinline__ void expand48_16(uint64_t bits, const uint32_t* vw, uint32_t* ow) {
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    uint64_t slot = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t sh = 8u * ((uint32_t)(bits >> (3 * (4 * gi + j))) & 7u);
      slot = (slot & ~(0xFFull << sh)) | ((uint64_t)(j + 1) << sh);
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t lo = (uint32_t)(slot >> (16 * w)) & 0xFFu;
      const uint32_t hi = (uint32_t)(slot >> (16 * w + 8)) & 0xFFu;
      const uint32_t s_lo = lo ? 0x0202u * lo - 0x0102u : 0x0C0Cu;
      const uint32_t s_hi = hi ? 0x0202u * hi - 0x0102u : 0x0C0Cu;
      ow[4 * gi + w] = __builtin_amdgcn_perm(vw[2 * gi + 1], vw[2 * gi], s_lo | (s_hi << 16));
    }
  }
}

template <typename E, int N, int M>
__global__ void __launch_bounds__(kThreads) flat_decompress_kernel(
    const uint32_t* __restrict__ values, const uint32_t* __restrict__ meta, int64_t units,
    uint32_t* __restrict__ out) {
  using S = UnitShape<E, M>;
  constexpr int b = meta_bits(M);
  constexpr int kUnitBits = S::kGroups * N * b;
  constexpr int kValWords = S::kGroups * N * (int)sizeof(E) / 4;
  const int64_t block_first = (int64_t)blockIdx.x * kThreads * kUnitsPerThread;
#pragma unroll
  for (int it = 0; it < kUnitsPerThread; ++it) {
    const int64_t u = block_first + (int64_t)it * kThreads + threadIdx.x;
    if (u >= units) continue;
    uint32_t vw[kValWords];
    if constexpr (kValWords == 4) {
      const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(values) + u);
      vw[0] = v[0]; vw[1] = v[1]; vw[2] = v[2]; vw[3] = v[3];
    } else if constexpr (kValWords == 2) {
      const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(values) + u);
      vw[0] = v[0]; vw[1] = v[1];
    } else {
#pragma unroll
      for (int i = 0; i < kValWords; ++i) vw[i] = values[u * kValWords + i];
    }
    const int64_t bit = u * kUnitBits;
    const int sh = (int)(bit % 32);
    uint64_t bits = (uint64_t)meta[bit / 32] >> sh;
    if (sh + kUnitBits > 32) bits |= (uint64_t)meta[bit / 32 + 1] << (32 - sh);
    if (sh + kUnitBits > 64) bits |= (uint64_t)meta[bit / 32 + 2] << (64 - sh);
    uint32_t ow[S::kWords];
#pragma unroll
    for (int i = 0; i < S::kWords; ++i) ow[i] = 0;
    if constexpr (N == 2 && M == 4 && sizeof(E) <= 2) {
      expand24<E, S::kGroups>(bits, vw, ow);
    } else {
#pragma unroll
      for (int g = 0; g < S::kGroups; ++g) {
#pragma unroll
        for (int j = 0; j < N; ++j) {
          const int k = g * N + j;
          const int p = (bits >> (k * b)) & ((1u << b) - 1u);
          const uint32_t v = word_elem<E>(vw, k);
          // out[g*M + p] = v, as selects over the M compile-time positions
#pragma unroll
          for (int i = 0; i < M; ++i) {
            const int e = g * M + i;
            if constexpr (sizeof(E) < 4) {
              constexpr int kPer = 4 / (int)sizeof(E);
              constexpr uint32_t kMask = sizeof(E) == 1 ? 0xFFu : 0xFFFFu;
              const uint32_t sh = 8 * (int)sizeof(E) * (e % kPer);
              const uint32_t cur = ow[e / kPer];
              ow[e / kPer] = (p == i) ? ((cur & ~(kMask << sh)) | (v << sh)) : cur;
            } else {
              ow[e] = (p == i) ? v : ow[e];
            }
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < S::kWords / 4; ++i)
      __builtin_nontemporal_store(u32x4_t{ow[4 * i], ow[4 * i + 1], ow[4 * i + 2], ow[4 * i + 3]},
                                  reinterpret_cast<u32x4_t*>(out + u * S::kWords) + i);
  }
}

// ---------------------------------------------------------------------------
// Blocked layout (see include/nm.h): one wave per block of 16 rows x one 64-wide K
// step.  Lane l takes row l / 4 of the block and elements 16 (l % 4) .. +15 of the
// step; its kept values and its metadata bits then sit at lane-linear offsets of the
// block (value l * 16N/M, bit l * 16Nb/M), so a wave writes the block's values and its
// metadata as two contiguous runs.  Rows past R are stored as zeros.
// ---------------------------------------------------------------------------
template <typename E, int N, int M>
struct LaneShape {
  static constexpr int kWords = 16 * (int)sizeof(E) / 4;      // 16 elements of W
  static constexpr int kGroups = 16 / M;
  static constexpr int kVals = kGroups * N;                   // kept values per lane
  static constexpr int kValWords = kVals * (int)sizeof(E) / 4;
  static constexpr int kBits = kVals * meta_bits(M);          // metadata bits per lane
  static constexpr int kBlockMetaWords = 64 * kBits / 32;
  static constexpr bool kShuffle = 32 % kBits == 0;           // whole lanes per word
  static constexpr bool kLdsBits = !kShuffle && kBits != 24;  // packed in an LDS buffer
};

// Selection, value packing and metadata packing of one lane's 16 elements of a block
// (row l / 4 of the block, elements 16 (l % 4) .. +15 of its step); `live` false writes
// the zeros of a padding row.  `bits_buf` is the wave's LDS word buffer (used when a
// lane's metadata bits do not divide 32).  Returns the lane's keep mask (bit e set iff
// element e of its 16 is kept).
template <typename E, int N, int M>
__device__ __forceinline__ uint32_t blocked_emit(const uint32_t (&w)[LaneShape<E, N, M>::kWords],
                                             bool live, int64_t blk, int lane, uint32_t* bits_buf,
                                             uint32_t* __restrict__ values,
                                             uint32_t* __restrict__ meta) {
  using L = LaneShape<E, N, M>;
  constexpr int b = meta_bits(M);
  uint32_t vw[L::kValWords];
#pragma unroll
  for (int i = 0; i < L::kValWords; ++i) vw[i] = 0;
  uint64_t bits = 0;
  uint32_t keep16 = 0;
  if constexpr (fast24<E, N, M>()) {
    int pos[L::kGroups][2];
#pragma unroll
    for (int gi = 0; gi < L::kGroups; ++gi) {
      uint32_t key[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) key[i] = Elem<E>::key(word_elem<E>(w, gi * 4 + i));
      top2_of_4(key[0], key[1], key[2], key[3], pos[gi][0], pos[gi][1]);
      bits |= (uint64_t)(pos[gi][0] | (pos[gi][1] << 2)) << (4 * gi);
      keep16 |= ((1u << pos[gi][0]) | (1u << pos[gi][1])) << (4 * gi);
    }
    pack_kept24<E, L::kGroups>(w, pos, vw);
  } else {
#pragma unroll
    for (int gi = 0; gi < L::kGroups; ++gi) {
      uint32_t key[M];
#pragma unroll
      for (int i = 0; i < M; ++i) key[i] = Elem<E>::key(word_elem<E>(w, gi * M + i));
      int pos[N];
      const uint32_t kb = group_keep<E, N, M>(key);
      keep16 |= kb << (M * gi);
      kept_positions<N>(kb, pos);
#pragma unroll
      for (int j = 0; j < N; ++j) {
        const int k = gi * N + j;
        put_elem<E>(vw, k, group_elem_at<E, M>(w, gi, pos[j]));
        bits |= (uint64_t)pos[j] << (k * b);
      }
    }
  }
  if (!live) bits = 0;  // padding rows: zero values (w = 0) and zero metadata
  store_words<L::kValWords>(values + blk * (64 * L::kValWords) + lane * L::kValWords, vw);

  uint32_t* mblk = meta + blk * L::kBlockMetaWords;
  if constexpr (L::kShuffle) {
    constexpr int LPW = 32 / L::kBits;  // lanes per metadata word
    const uint32_t word = or_reduce_lanes<LPW>((uint32_t)bits << ((lane % LPW) * L::kBits));
    if (lane % LPW == 0) mblk[lane / LPW] = word;
  } else if constexpr (L::kBits == 24) {
    // 4:8 (eight 3-bit fields a lane): four lanes' 24-bit runs make three whole words.
    // Lane 4j + i (i < 3) writes word 3j + i: its own bits from bit 8i on, and the next
    // lane's bits above them.
    const uint32_t own = (uint32_t)bits;
    const uint32_t next = __shfl_down(own, 1);
    const int i = lane & 3;
    if (i < 3) mblk[3 * (lane >> 2) + i] = (own >> (8 * i)) | (next << (24 - 8 * i));
  } else {
    uint32_t* buf = bits_buf;
    for (int i = lane; i < L::kBlockMetaWords; i += 64) buf[i] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const int o = lane * L::kBits, wi = o / 32, sh = o % 32;
    atomicOr(&buf[wi], (uint32_t)(bits << sh));
    if (sh + L::kBits > 32) atomicOr(&buf[wi + 1], (uint32_t)(bits >> (32 - sh)));
    if (sh + L::kBits > 64) atomicOr(&buf[wi + 2], (uint32_t)(bits >> (64 - sh)));
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    for (int i = lane; i < L::kBlockMetaWords; i += 64) mblk[i] = buf[i];
  }
  return keep16;
}

template <typename E, int N, int M>
__global__ void __launch_bounds__(kThreads) blocked_select_kernel(const uint32_t* __restrict__ W,
                                                                  int64_t R, int64_t K,
                                                                  int64_t blocks,
                                                                  uint32_t* __restrict__ values,
                                                                  uint32_t* __restrict__ meta) {
  using L = LaneShape<E, N, M>;
  __shared__ uint32_t lds_bits[kThreads / 64][L::kLdsBits ? L::kBlockMetaWords : 1];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar math
  const int64_t blk = (int64_t)blockIdx.x * (kThreads / 64) + wave;
  if (blk >= blocks) return;  // the whole wave
  const int64_t steps = K / 64;
  int64_t rb, st;  // row block and step of this block
  if (blocks <= 0xFFFFFFFFll) {  // 32-bit division where it fits (every practical size)
    rb = (uint32_t)blk / (uint32_t)steps;
    st = (uint32_t)blk - (uint32_t)rb * (uint32_t)steps;
  } else {
    rb = blk / steps;
    st = blk % steps;
  }
  const int64_t row = 16 * rb + (lane >> 2);
  const bool live = row < R;
  uint32_t w[L::kWords];
  if (live) {
    load_words<L::kWords>(W + (row * K + 64 * st + 16 * (lane & 3)) * sizeof(E) / 4, w);
  } else {
#pragma unroll
    for (int i = 0; i < L::kWords; ++i) w[i] = 0;
  }
  blocked_emit<E, N, M>(w, live, blk, lane, lds_bits[wave], values, meta);
}

// Mask, values and metadata in one pass: the compressed pair in the blocked layout and the
// dense uint8 mask (R x K, row-major).  A wave takes kPer consecutive blocks of one row
// block (2 when the step count is even), so that it holds 64 kPer mask bytes of each of
// its 16 rows; they are staged in the wave's LDS slice and stored back as whole row
// segments (for kPer = 2 each store instruction writes eight full 128-byte lines), since
// lines assembled from several store instructions cost extra write traffic.
template <typename E, int N, int M, int kPer>
__global__ void __launch_bounds__(kThreads) blocked_select_mask_kernel(
    const uint32_t* __restrict__ W, int64_t R, int64_t K, int64_t blocks,
    uint32_t* __restrict__ values, uint32_t* __restrict__ meta, uint8_t* __restrict__ mask) {
  using L = LaneShape<E, N, M>;
  constexpr int kRowWords = 16 * kPer;  // mask words per row segment
  __shared__ uint32_t lds_bits[kThreads / 64][L::kLdsBits ? L::kBlockMetaWords : 1];
  __shared__ __align__(16) uint32_t stage[kThreads / 64][16 * kRowWords];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar math
  const int64_t blk = ((int64_t)blockIdx.x * (kThreads / 64) + wave) * kPer;
  if (blk >= blocks) return;  // the whole wave
  const int64_t steps = K / 64;
  int64_t rb, st;  // row block and first step of this wave's blocks
  if (blocks <= 0xFFFFFFFFll) {
    rb = (uint32_t)blk / (uint32_t)steps;
    st = (uint32_t)blk - (uint32_t)rb * (uint32_t)steps;
  } else {
    rb = blk / steps;
    st = blk % steps;
  }
  const int rr = lane >> 2, q = lane & 3;
  const int64_t row = 16 * rb + rr;
  const bool live = row < R;
  uint32_t w[kPer][L::kWords];
#pragma unroll
  for (int p = 0; p < kPer; ++p) {
    if (live) {
      load_words<L::kWords>(W + (row * K + 64 * (st + p) + 16 * q) * sizeof(E) / 4, w[p]);
    } else {
#pragma unroll
      for (int i = 0; i < L::kWords; ++i) w[p][i] = 0;
    }
  }
  uint32_t* sw = stage[wave];
#pragma unroll
  for (int p = 0; p < kPer; ++p) {
    const uint32_t keep = blocked_emit<E, N, M>(w[p], live, blk + p, lane, lds_bits[wave],
                                                values, meta);
    uint32_t mw[4];  // one byte per element, 1 = kept
#pragma unroll
    for (int j = 0; j < 4; ++j) mw[j] = (((keep >> (4 * j)) & 0xFu) * 0x00204081u) & 0x01010101u;
    *reinterpret_cast<u32x4_t*>(sw + rr * kRowWords + 16 * p + 4 * q) =
        u32x4_t{mw[0], mw[1], mw[2], mw[3]};
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  constexpr int C = 4 * kPer;  // 16-byte chunks per row segment
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int r2 = i * (64 / C) + lane / C, ch = lane % C;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(sw + (r2 * C + ch) * 4);
    const int64_t r = 16 * rb + r2;
    if (r < R)  // padding rows have no mask
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(mask + r * K + 64 * st) + ch);
  }
}

// The blocked layout of W's TRANSPOSE (K x R, groups of M along R; R % 64 == 0): block
// (g, s) holds transposed rows 16g .. 16g+15, i.e. columns 16g .. of W, and step s,
// i.e. rows 64s .. 64s+63 of W.  A wave takes a column quad (column groups 4c .. 4c+3,
// 64 columns of W) and one step: it stages the 64 x 64 tile of W in its LDS slice with
// whole 128-byte row segments per load instruction, then for each of the four column
// groups every lane gathers its 16 elements down one column and proceeds as for W
// itself.  (Quarter-line reads by four waves had fetched 15% more than W's bytes.)  The
// four waves of a workgroup take four consecutive steps of one quad and consecutive
// workgroups continue down its steps, so each column group's blocks are written front
// to back.  Columns past K are padding (zeros).
template <typename E>
struct TileT {
  static constexpr int kChunkElems = 16 / (int)sizeof(E);  // elements per 16-byte chunk
  static constexpr int kRowChunks = 64 / kChunkElems;      // chunks per 64-column row
  static constexpr int kRowWords = 16 * kRowChunks / 4;    // LDS words per row
  // Rows 16q .. 16q+15 start kShift * q words further, so that the column gathers of
  // the four quarters (lanes with q = 0..3) fall in different banks.
  static constexpr int kShift = sizeof(E) == 4 ? 16 : 8;
  static constexpr int kWords = 64 * kRowWords + 3 * kShift;
  __device__ static constexpr int row_word(int r) { return r * kRowWords + (r >> 4) * kShift; }
};

template <typename E, int N, int M>
__global__ void __launch_bounds__(kThreads) blocked_select_t_kernel(
    const E* __restrict__ W, int64_t R, int64_t K, uint32_t* __restrict__ values,
    uint32_t* __restrict__ meta) {
  using L = LaneShape<E, N, M>;
  using TT = TileT<E>;
  __shared__ uint32_t lds_bits[kThreads / 64][L::kLdsBits ? L::kBlockMetaWords : 1];
  __shared__ __align__(16) uint32_t tile[kThreads / 64][TT::kWords];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t steps = R / 64, groups = (K + 15) / 16;
  // (blockIdx.x < 2^32, and step_quads <= the grid size fits 32 bits)
  const uint32_t step_quads = (uint32_t)((steps + 3) / 4);
  const int64_t quad = blockIdx.x / step_quads;
  const int64_t st = (int64_t)(blockIdx.x % step_quads) * 4 + wave;
  if (st >= steps) return;  // the whole wave
  const int64_t c0 = 64 * quad;
  const bool vec_ok = (K * (int64_t)sizeof(E)) % 16 == 0;
  uint32_t* tw = tile[wave];
#pragma unroll
  for (int it = 0; it < TT::kRowChunks; ++it) {
    const int chunk = it * 64 + lane;  // 64 rows x kRowChunks chunks
    const int r = chunk / TT::kRowChunks, ch = chunk % TT::kRowChunks;
    const int64_t col = c0 + ch * TT::kChunkElems;
    const E* src = W + (64 * st + r) * K + col;
    uint32_t* dst = tw + TT::row_word(r) + 4 * ch;
    if (vec_ok && col + TT::kChunkElems <= K) {
      *reinterpret_cast<u32x4_t*>(dst) =
          __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src));
    } else {
      uint32_t v[4] = {0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < TT::kChunkElems; ++e)
        put_elem<E>(v, e, (col + e < K) ? (uint32_t)src[e] : 0u);
      *reinterpret_cast<u32x4_t*>(dst) = u32x4_t{v[0], v[1], v[2], v[3]};
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int cl = lane >> 2, q = lane & 3;
  const E* te = reinterpret_cast<const E*>(tw);
#pragma unroll
  for (int cg = 0; cg < 4; ++cg) {
    const int64_t g = 4 * quad + cg;
    if (g >= groups) break;  // the same for the whole wave
    const int col = 16 * cg + cl;
    uint32_t w[L::kWords];
#pragma unroll
    for (int i = 0; i < L::kWords; ++i) w[i] = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      put_elem<E>(w, i, (uint32_t)te[TT::row_word(16 * q + i) * (4 / (int)sizeof(E)) + col]);
    blocked_emit<E, N, M>(w, c0 + col < K, g * steps + st, lane, lds_bits[wave], values, meta);
  }
}

// Row layout of W's transpose, slow path: one thread per transposed group (W column k,
// rows gM .. gM+M-1), consecutive threads along k so that each of the M reads is
// coalesced; the N values go to row k of the transposed value array.
template <typename E, int N, int M>
__global__ void __launch_bounds__(kThreads) group_t_kernel(const E* __restrict__ W, int64_t R,
                                                           int64_t K, E* __restrict__ values) {
  const int64_t work = R / M * K;
  for (int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x; idx < work;
       idx += (int64_t)gridDim.x * kThreads) {
  const int64_t g = idx / K, k = idx % K;
  uint32_t key[M], v[M];
#pragma unroll
  for (int i = 0; i < M; ++i) {
    v[i] = W[(g * M + i) * K + k];
    key[i] = Elem<E>::key(v[i]);
  }
  int pos[N];
  kept_positions<N>(group_keep<E, N, M>(key), pos);
  E* dst = values + k * (R / M * N) + g * N;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    uint32_t x = v[0];
#pragma unroll
    for (int i = 1; i < M; ++i) x = (pos[j] == i) ? v[i] : x;
    dst[j] = (E)x;
  }
  }
}

// Metadata words of the transposed row layout: one thread per (W column k, word w).
template <typename E, int N, int M>
__global__ void __launch_bounds__(kThreads) meta_word_t_kernel(const E* __restrict__ W, int64_t R,
                                                               int64_t K, int64_t wpr,
                                                               uint32_t* __restrict__ meta) {
  constexpr int b = meta_bits(M);
  for (int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x; idx < K * wpr;
       idx += (int64_t)gridDim.x * kThreads) {
  const int64_t w = idx / K, k = idx % K;
  const int64_t fields = R / M * N;
  const int64_t f0 = (32 * w) / b;
  int64_t f1 = (32 * w + 31) / b;
  if (f1 > fields - 1) f1 = fields - 1;
  uint32_t word = 0;
  for (int64_t g = f0 / N; g <= f1 / N; ++g) {
    uint32_t key[M];
#pragma unroll
    for (int i = 0; i < M; ++i) key[i] = Elem<E>::key((uint32_t)W[(g * M + i) * K + k]);
    int pos[N];
    kept_positions<N>(group_keep<E, N, M>(key), pos);
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int64_t f = g * N + j;
      if (f < f0 || f > f1) continue;
      const int64_t off = f * b - 32 * w;
      word |= off >= 0 ? (uint32_t)pos[j] << off : (uint32_t)pos[j] >> (-off);
    }
  }
  meta[k * wpr + w] = word;
  }
}

template <typename E, int N, int M>
__device__ __forceinline__ void decompress_lane(const uint32_t* __restrict__ values,
                                                const uint32_t* __restrict__ meta, int64_t blk,
                                                int lane, uint32_t (&ow)[LaneShape<E, N, M>::kWords]) {
  using L = LaneShape<E, N, M>;
  constexpr int b = meta_bits(M);
  const uint32_t* vsrc = values + blk * (64 * L::kValWords) + lane * L::kValWords;
  uint32_t vw[L::kValWords];
#pragma unroll
  for (int i = 0; i < L::kValWords; ++i) vw[i] = vsrc[i];
  const uint32_t* mblk = meta + blk * L::kBlockMetaWords;
  const int o = lane * L::kBits, wi = o / 32, sh = o % 32;
  uint64_t window = mblk[wi];
  if (sh + L::kBits > 32) window |= (uint64_t)mblk[wi + 1] << 32;
  uint64_t bits = window >> sh;
  if (sh + L::kBits > 64) bits |= (uint64_t)mblk[wi + 2] << (64 - sh);
  if constexpr (N == 2 && M == 4 && sizeof(E) <= 2) {
    expand24<E, L::kGroups>(bits, vw, ow);
    return;
  }
  if constexpr (N == 4 && M == 8 && sizeof(E) == 2) {
    expand48_16<L::kGroups>(bits, vw, ow);
    return;
  }
#pragma unroll
  for (int i = 0; i < L::kWords; ++i) ow[i] = 0;
#pragma unroll
  for (int gi = 0; gi < L::kGroups; ++gi) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int k = gi * N + j;
      const int p = (int)((bits >> (k * b)) & ((1u << b) - 1u));
      const uint32_t v = word_elem<E>(vw, k);
#pragma unroll
      for (int i = 0; i < M; ++i) {
        const int e = gi * M + i;
        if constexpr (sizeof(E) < 4) {
          constexpr int kPer = 4 / (int)sizeof(E);
          constexpr uint32_t kMask = sizeof(E) == 1 ? 0xFFu : 0xFFFFu;
          const uint32_t sh = 8 * (int)sizeof(E) * (e % kPer);
          const uint32_t cur = ow[e / kPer];
          ow[e / kPer] = (p == i) ? ((cur & ~(kMask << sh)) | (v << sh)) : cur;
        } else {
          ow[e] = (p == i) ? v : ow[e];
        }
      }
    }
  }
}

// kPer consecutive blocks per wave (2 for 1-byte elements when the step count is even, so
// that a row segment of the two blocks is one 128-byte line).  The 4 lanes of a row hold
// its 16-byte chunks in lane order; written as they are, a row's 128-byte line would come
// from several store instructions, which the write counter showed to cost extra HBM write
// traffic (109 MB for 90 MB of bf16 output).  Each wave therefore stages its blocks in
// its LDS slice and stores them back row by row: lane l writes chunk l % C of row l / C
// (C chunks per row segment), one instruction covering 64 / C whole row segments.
template <typename E, int N, int M, int kPer>
__global__ void __launch_bounds__(kThreads) blocked_decompress_kernel(
    const uint32_t* __restrict__ values, const uint32_t* __restrict__ meta, int64_t R, int64_t K,
    int64_t blocks, uint32_t* __restrict__ out) {
  using L = LaneShape<E, N, M>;
  constexpr int S = L::kWords / 4;  // 16-byte chunks per lane and block
  constexpr int C = 4 * S * kPer;   // 16-byte chunks per row segment
  __shared__ __align__(16) uint32_t stage[kThreads / 64][64 * L::kWords * kPer];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar math
  const int64_t blk = ((int64_t)blockIdx.x * (kThreads / 64) + wave) * kPer;
  if (blk >= blocks) return;
  const int64_t steps = K / 64;
  int64_t rb, st;  // row block and (first) step of this wave's blocks
  if (blocks <= 0xFFFFFFFFll) {
    rb = (uint32_t)blk / (uint32_t)steps;
    st = (uint32_t)blk - (uint32_t)rb * (uint32_t)steps;
  } else {
    rb = blk / steps;
    st = blk % steps;
  }
  uint32_t* sw = stage[wave];
  const int rr0 = lane >> 2, q = lane & 3;
#pragma unroll
  for (int p = 0; p < kPer; ++p) {
    uint32_t ow[L::kWords];
    decompress_lane<E, N, M>(values, meta, blk + p, lane, ow);
#pragma unroll
    for (int c = 0; c < S; ++c)
      *reinterpret_cast<u32x4_t*>(sw + (rr0 * C + p * 4 * S + q * S + c) * 4) =
          u32x4_t{ow[4 * c], ow[4 * c + 1], ow[4 * c + 2], ow[4 * c + 3]};
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int i = 0; i < S * kPer; ++i) {
    const int rr = i * (64 / C) + lane / C, ch = lane % C;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(sw + (rr * C + ch) * 4);
    const int64_t r = 16 * rb + rr;
    if (r < R)  // padding rows have no output
      __builtin_nontemporal_store(
          v, reinterpret_cast<u32x4_t*>(out + (r * K + 64 * st) * sizeof(E) / 4) + ch);
  }
}

// ---------------------------------------------------------------------------
// Shape-agnostic kernels (any R, K with K % M == 0).
// ---------------------------------------------------------------------------
template <typename E, int N, int M>
__device__ __forceinline__ void select_group(const E* W, int64_t base, int (&pos)[N],
                                             uint32_t& keep) {
  uint32_t key[M];
#pragma unroll
  for (int i = 0; i < M; ++i) key[i] = Elem<E>::key((uint32_t)W[base + i]);
  keep = group_keep<E, N, M>(key);
  kept_positions<N>(keep, pos);
}

// one thread per group: mask bytes and/or values
template <typename E, int N, int M, bool kMask, bool kValues>
__global__ void __launch_bounds__(kThreads) group_kernel(const E* __restrict__ W, int64_t groups,
                                                         E* __restrict__ values,
                                                         uint8_t* __restrict__ mask) {
  for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < groups;
       g += (int64_t)gridDim.x * kThreads) {
    int pos[N];
    uint32_t keep;
    select_group<E, N, M>(W, g * M, pos, keep);
    if constexpr (kMask)
#pragma unroll
      for (int i = 0; i < M; ++i) mask[g * M + i] = (keep >> i) & 1u;
    if constexpr (kValues)
#pragma unroll
      for (int j = 0; j < N; ++j) values[g * N + j] = W[g * M + pos[j]];
  }
}

// one thread per metadata word
template <typename E, int N, int M>
__global__ void __launch_bounds__(kThreads) meta_word_kernel(const E* __restrict__ W, int64_t R,
                                                             int64_t K, int64_t wpr,
                                                             uint32_t* __restrict__ meta) {
  constexpr int b = meta_bits(M);
  for (int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x; idx < R * wpr;
       idx += (int64_t)gridDim.x * kThreads) {
  const int64_t r = idx / wpr, w = idx % wpr;
  const int64_t fields = K / M * N;
  const int64_t f0 = (32 * w) / b;
  int64_t f1 = (32 * w + 31) / b;
  if (f1 > fields - 1) f1 = fields - 1;
  uint32_t word = 0;
  for (int64_t g = f0 / N; g <= f1 / N; ++g) {
    int pos[N];
    uint32_t keep;
    select_group<E, N, M>(W, r * K + g * M, pos, keep);
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int64_t f = g * N + j;
      if (f < f0 || f > f1) continue;
      const int64_t off = f * b - 32 * w;  // may be negative for a field straddling in
      word |= off >= 0 ? (uint32_t)pos[j] << off : (uint32_t)pos[j] >> (-off);
    }
  }
  meta[idx] = word;
  }
}

// one thread per group of the output
template <typename E, int N, int M>
__global__ void __launch_bounds__(kThreads) group_decompress_kernel(
    const E* __restrict__ values, const uint32_t* __restrict__ meta, int64_t R, int64_t K,
    int64_t wpr, E* __restrict__ out) {
  constexpr int b = meta_bits(M);
  const int64_t gpr = K / M;
  for (int64_t gi = (int64_t)blockIdx.x * kThreads + threadIdx.x; gi < R * gpr;
       gi += (int64_t)gridDim.x * kThreads) {
  const int64_t r = gi / gpr, g = gi % gpr;
  const uint32_t* mrow = meta + r * wpr;
  E o[M];
#pragma unroll
  for (int i = 0; i < M; ++i) o[i] = E{};
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const int64_t bit = (g * N + j) * b;
    uint64_t window = mrow[bit / 32];
    if ((bit % 32) + b > 32) window |= (uint64_t)mrow[bit / 32 + 1] << 32;
    const int p = (int)((window >> (bit % 32)) & ((1u << b) - 1u));
    const E v = values[r * (gpr * N) + g * N + j];
#pragma unroll
    for (int i = 0; i < M; ++i) o[i] = (p == i) ? v : o[i];
  }
#pragma unroll
  for (int i = 0; i < M; ++i) out[r * K + g * M + i] = o[i];
  }
}

inline unsigned blocks_for(int64_t work, int64_t per_block) {
  return (unsigned)((work + per_block - 1) / per_block);
}

// Does one unit's value output fill a 4-, 8- or 16-byte store?
template <typename E, int N, int M>
constexpr bool flat_kernel_exists() {
  constexpr int kValBytes = UnitShape<E, M>::kGroups * N * (int)sizeof(E);
  return kValBytes == 4 || kValBytes == 8 || kValBytes == 16;
}

// Can rows be concatenated into one stream of whole units and whole metadata words?
template <typename E, int N, int M>
bool flat_ok(int64_t K) {
  using S = UnitShape<E, M>;
  constexpr int kUnitBits = S::kGroups * N * meta_bits(M);
  if (!flat_kernel_exists<E, N, M>()) return false;
  if (K % S::kElems != 0) return false;
  const int64_t row_bits = (K / S::kElems) * kUnitBits;
  if (row_bits % 32 != 0) return false;
  // the LDS packing path writes whole 64-lane wave-steps; rows must hold whole words
  return true;
}

// Does a lane's share of a block (16 elements) keep a whole number of 32-bit words of
// values?  Always for 16- and 32-bit elements; for bytes, 16 N / M must divide by 4.
template <typename E, int N, int M>
constexpr bool blocked_kernel_exists() {
  return (16 * N / M * (int)sizeof(E)) % 4 == 0;
}

template <typename E, int N, int M>
hipError_t run_select(const void* W, int64_t R, int64_t K, bool blocked, void* values,
                      uint32_t* meta, uint8_t* mask, hipStream_t s) {
  using S = UnitShape<E, M>;
  const int64_t elems = R * K;
  if (elems == 0) return hipSuccess;
  const bool want_mask = mask != nullptr, want_compress = values != nullptr;
  if (blocked) {  // compress, with the (dense, row-major) mask in the same pass if asked
    if constexpr (blocked_kernel_exists<E, N, M>()) {
      const int64_t blocks = (R + 15) / 16 * (K / 64);
      const uint32_t* w = static_cast<const uint32_t*>(W);
      uint32_t* v = static_cast<uint32_t*>(values);
      if (!want_mask) {
        blocked_select_kernel<E, N, M><<<blocks_for(blocks, kThreads / 64), kThreads, 0, s>>>(
            w, R, K, blocks, v, meta);
      } else if ((K / 64) % 2 == 0) {
        blocked_select_mask_kernel<E, N, M, 2>
            <<<blocks_for(blocks / 2, kThreads / 64), kThreads, 0, s>>>(w, R, K, blocks, v, meta,
                                                                        mask);
      } else {
        blocked_select_mask_kernel<E, N, M, 1>
            <<<blocks_for(blocks, kThreads / 64), kThreads, 0, s>>>(w, R, K, blocks, v, meta,
                                                                    mask);
      }
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  if constexpr (flat_kernel_exists<E, N, M>()) {
   if (flat_ok<E, N, M>(K)) {
    const int64_t units = elems / S::kElems;
    const unsigned grid = blocks_for(units, (int64_t)kThreads * kUnitsPerThread);
    const uint32_t* w = static_cast<const uint32_t*>(W);
    uint32_t* v = static_cast<uint32_t*>(values);
    if (want_mask && want_compress)
      flat_select_kernel<E, N, M, true, true><<<grid, kThreads, 0, s>>>(w, units, v, meta, mask);
    else if (want_mask)
      flat_select_kernel<E, N, M, true, false><<<grid, kThreads, 0, s>>>(w, units, v, meta, mask);
    else
      flat_select_kernel<E, N, M, false, true><<<grid, kThreads, 0, s>>>(w, units, v, meta, mask);
    return hipGetLastError();
   }
  }
  const int64_t groups = elems / M;
  const unsigned grid = stride_grid(groups, kThreads);
  const E* w = static_cast<const E*>(W);
  E* v = static_cast<E*>(values);
  if (want_mask && want_compress)
    group_kernel<E, N, M, true, true><<<grid, kThreads, 0, s>>>(w, groups, v, mask);
  else if (want_mask)
    group_kernel<E, N, M, true, false><<<grid, kThreads, 0, s>>>(w, groups, v, mask);
  else
    group_kernel<E, N, M, false, true><<<grid, kThreads, 0, s>>>(w, groups, v, mask);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !want_compress) return e;
  const int64_t wpr = ((K / M) * N * meta_bits(M) + 31) / 32;
  if (R * wpr > 0)
    meta_word_kernel<E, N, M><<<stride_grid(R * wpr, kThreads), kThreads, 0, s>>>(w, R, K, wpr, meta);
  return hipGetLastError();
}

template <typename E, int N, int M>
hipError_t run_select_t(const void* W, int64_t R, int64_t K, bool blocked, void* values,
                        uint32_t* meta, hipStream_t s) {
  if (R * K == 0) return hipSuccess;
  const E* w = static_cast<const E*>(W);
  if (blocked) {
    const int64_t steps = R / 64, groups = (K + 15) / 16;
    const int64_t wg = (groups + 3) / 4 * ((steps + 3) / 4);  // column quads x step quads
    blocked_select_t_kernel<E, N, M><<<(unsigned)wg, kThreads, 0, s>>>(
        w, R, K, static_cast<uint32_t*>(values), meta);
    return hipGetLastError();
  }
  group_t_kernel<E, N, M><<<stride_grid(R / M * K, kThreads), kThreads, 0, s>>>(
      w, R, K, static_cast<E*>(values));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t wpr = ((R / M) * N * meta_bits(M) + 31) / 32;
  meta_word_t_kernel<E, N, M><<<stride_grid(K * wpr, kThreads), kThreads, 0, s>>>(w, R, K, wpr,
                                                                                 meta);
  return hipGetLastError();
}

template <typename E, int N, int M>
hipError_t run_decompress(const void* values, const uint32_t* meta, int64_t R, int64_t K,
                          bool blocked, void* out, hipStream_t s) {
  using S = UnitShape<E, M>;
  const int64_t elems = R * K;
  if (elems == 0) return hipSuccess;
  if (blocked) {
    if constexpr (blocked_kernel_exists<E, N, M>()) {
      const int64_t blocks = (R + 15) / 16 * (K / 64);
      if (sizeof(E) == 1 && (K / 64) % 2 == 0)
        blocked_decompress_kernel<E, N, M, 2>
            <<<blocks_for(blocks / 2, kThreads / 64), kThreads, 0, s>>>(
                static_cast<const uint32_t*>(values), meta, R, K, blocks,
                static_cast<uint32_t*>(out));
      else
        blocked_decompress_kernel<E, N, M, 1>
            <<<blocks_for(blocks, kThreads / 64), kThreads, 0, s>>>(
                static_cast<const uint32_t*>(values), meta, R, K, blocks,
                static_cast<uint32_t*>(out));
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  if constexpr (flat_kernel_exists<E, N, M>()) {
    if (flat_ok<E, N, M>(K)) {
      const int64_t units = elems / S::kElems;
      flat_decompress_kernel<E, N, M>
          <<<blocks_for(units, (int64_t)kThreads * kUnitsPerThread), kThreads, 0, s>>>(
              static_cast<const uint32_t*>(values), meta, units, static_cast<uint32_t*>(out));
      return hipGetLastError();
    }
  }
  const int64_t wpr = ((K / M) * N * meta_bits(M) + 31) / 32;
  group_decompress_kernel<E, N, M><<<stride_grid(elems / M, kThreads), kThreads, 0, s>>>(
      static_cast<const E*>(values), meta, R, K, wpr, static_cast<E*>(out));
  return hipGetLastError();
}

// Compile-time dispatch over the supported N:M patterns.
template <typename E, template <typename, int, int> class F, typename... A>
hipError_t dispatch_nm(int n, int m, A... args) {
#define NM_CASE(NN, MM) \
  if (n == NN && m == MM) return F<E, NN, MM>::run(args...);
  NM_CASE(1, 2) NM_CASE(2, 2)
  NM_CASE(1, 4) NM_CASE(2, 4) NM_CASE(3, 4) NM_CASE(4, 4)
  NM_CASE(1, 8) NM_CASE(2, 8) NM_CASE(3, 8) NM_CASE(4, 8)
  NM_CASE(5, 8) NM_CASE(6, 8) NM_CASE(7, 8) NM_CASE(8, 8)
#undef NM_CASE
  return hipErrorInvalidValue;
}

template <typename E, int N, int M>
struct SelectOp {
  static hipError_t run(const void* W, int64_t R, int64_t K, bool blocked, void* values,
                        uint32_t* meta, uint8_t* mask, hipStream_t s) {
    return run_select<E, N, M>(W, R, K, blocked, values, meta, mask, s);
  }
};
template <typename E, int N, int M>
struct SelectTOp {
  static hipError_t run(const void* W, int64_t R, int64_t K, bool blocked, void* values,
                        uint32_t* meta, hipStream_t s) {
    return run_select_t<E, N, M>(W, R, K, blocked, values, meta, s);
  }
};
template <typename E, int N, int M>
struct DecompressOp {
  static hipError_t run(const void* values, const uint32_t* meta, int64_t R, int64_t K,
                        bool blocked, void* out, hipStream_t s) {
    return run_decompress<E, N, M>(values, meta, R, K, blocked, out, s);
  }
};

}  // namespace

hipError_t launch_select(const void* W, int dt, int64_t R, int64_t K, int n, int m,
                         bool blocked, void* values, uint32_t* meta, uint8_t* mask,
                         hipStream_t s) {
  // dt: nm_dtype code (0 fp32, 1 fp16, 2 bf16, 3 int8, 5 fp8)
  if (dt == 3)
    return dispatch_nm<uint8_t, SelectOp>(n, m, W, R, K, blocked, values, meta, mask, s);
  if (dt == 5)
    return dispatch_nm<fp8_t, SelectOp>(n, m, W, R, K, blocked, values, meta, mask, s);
  if (dt == 1 || dt == 2)
    return dispatch_nm<uint16_t, SelectOp>(n, m, W, R, K, blocked, values, meta, mask, s);
  return dispatch_nm<uint32_t, SelectOp>(n, m, W, R, K, blocked, values, meta, mask, s);
}

hipError_t launch_select_t(const void* W, int elem_bytes, int64_t R, int64_t K, int n, int m,
                           bool blocked, void* values, uint32_t* meta, hipStream_t s) {
  if (elem_bytes == 2)
    return dispatch_nm<uint16_t, SelectTOp>(n, m, W, R, K, blocked, values, meta, s);
  return dispatch_nm<uint32_t, SelectTOp>(n, m, W, R, K, blocked, values, meta, s);
}

hipError_t launch_decompress(const void* values, const uint32_t* meta, int elem_bytes, int64_t R,
                             int64_t K, int n, int m, bool blocked, void* out, hipStream_t s) {
  if (elem_bytes == 1)
    return dispatch_nm<uint8_t, DecompressOp>(n, m, values, meta, R, K, blocked, out, s);
  if (elem_bytes == 2)
    return dispatch_nm<uint16_t, DecompressOp>(n, m, values, meta, R, K, blocked, out, s);
  return dispatch_nm<uint32_t, DecompressOp>(n, m, values, meta, R, K, blocked, out, s);
}

}  // namespace nm
