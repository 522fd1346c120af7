// nm_srste.hip -- SR-STE's per-step weight passes (gfx950).
//
// SR-STE ("量化友好的SR-STE稀疏化训练", section
// "基于直通估计的动态掩码精炼化稀疏(SR-STE)") searches the N:M mask again from the
// current weights at every forward step, runs the layer on the masked weights, and
// in the backward hands the dense weights the incoming gradient plus decay * w at
// the positions the mask prunes.  Both passes are elementwise over W with the group
// selection of nm_device.h in between, so each is one HBM stream:
//
//   prune:  W_out = W where kept, +0 where pruned          (read W, write W_out)
//   grad:   G_out = G where kept,                           (read W and G, write G_out)
//           fl(fl32(g + fl32(decay * w))) where pruned
//
// The backward recomputes the mask from W instead of reading a stored one: it must
// read W for the decay term anyway, so the mask costs no extra traffic, and W has not
// changed since the forward of the same step.  Arithmetic follows the printed
// backward for a float32 decay: one fp32 multiply, one fp32 add (never fused), then
// one rounding to the element type, round to nearest even.
//
// Layout of the work: W, G and the output are one stream of 16-byte units (8 x 16-bit
// or 4 x fp32 elements, 8 fp32 for M = 8); every unit holds whole groups because M
// divides the unit and K.  A lane takes kUnitsPerThread units a block-width apart
// (each load instruction of a wave covers 1 KB of consecutive memory), issues all its
// loads before any arithmetic, and writes each unit with one store.  Elements past the
// last whole unit (fewer than one unit, whole groups) go to a one-thread-per-group
// kernel.  A lane reads a unit entirely before writing it, so the output may be the
// same array as W (prune) or G (grad).
#include "nm_device.h"
#include "nm_launch.h"

namespace nm {

namespace {

constexpr int kThreads = 256;
constexpr int kUnitsPerThread = 2;

enum { kF32 = 0, kF16 = 1, kBF16 = 2 };

template <int DT>
struct Fmt {
  using E = uint16_t;
};
template <>
struct Fmt<kF32> {
  using E = uint32_t;
};

template <int DT, int M>
struct SrsteUnit {
  using E = typename Fmt<DT>::E;
  static constexpr int kElems = (16 / (int)sizeof(E)) > M ? (16 / (int)sizeof(E)) : M;
  static constexpr int kWords = kElems * (int)sizeof(E) / 4;
  static constexpr int kGroups = kElems / M;
};

template <int NW>
__device__ __forceinline__ void load_unit(const uint32_t* p, uint32_t (&w)[NW]) {
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
__device__ __forceinline__ void store_unit(uint32_t* p, const uint32_t (&w)[NW]) {
#pragma unroll
  for (int i = 0; i < NW / 4; ++i)
    __builtin_nontemporal_store(u32x4_t{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]},
                                reinterpret_cast<u32x4_t*>(p) + i);
}

// Bit e set iff element e of the unit is kept.
template <int DT, int N, int M, int NW>
__device__ __forceinline__ uint32_t unit_keep(const uint32_t (&w)[NW]) {
  using U = SrsteUnit<DT, M>;
  using E = typename U::E;
  uint32_t keep = 0;
#pragma unroll
  for (int g = 0; g < U::kGroups; ++g) {
    uint32_t key[M];
#pragma unroll
    for (int i = 0; i < M; ++i) key[i] = word_elem<E>(w, g * M + i) & Elem<E>::kKeyMask;
    keep |= group_keep<E, N, M>(key) << (g * M);
  }
  return keep;
}

template <int DT>
__device__ __forceinline__ float elem_to_f32(uint32_t bits) {
  if constexpr (DT == kF32) return __uint_as_float(bits);
  else if constexpr (DT == kBF16) return __uint_as_float(bits << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

template <int DT>
__device__ __forceinline__ uint32_t f32_to_elem(float x) {
  if constexpr (DT == kF32) {
    return __float_as_uint(x);
  } else if constexpr (DT == kBF16) {  // round to nearest even on the fp32 bits
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) & 0x8000u) | 0x7FC0u;  // NaN
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  } else {  // hardware conversion in the default round-to-nearest-even mode
    return __builtin_bit_cast(uint16_t, (_Float16)x);
  }
}

// g + decay * w with each operation rounded to fp32 on its own, then rounded to DT.
template <int DT>
__device__ __forceinline__ uint32_t refined(uint32_t w_bits, uint32_t g_bits, float decay) {
#pragma clang fp contract(off)
  const float p = decay * elem_to_f32<DT>(w_bits);
  const float s = elem_to_f32<DT>(g_bits) + p;
  return f32_to_elem<DT>(s);
}

// Output unit from the keep bits: kGrad ? (kept ? g : refined) : (kept ? w : +0).
template <int DT, int M, bool kGrad, int NW>
__device__ __forceinline__ void unit_output(uint32_t keep, const uint32_t (&w)[NW],
                                            const uint32_t (&g)[NW], float decay,
                                            uint32_t (&o)[NW]) {
  using U = SrsteUnit<DT, M>;
  static_assert(NW == U::kWords, "unit size");
  if constexpr (DT == kF32) {
#pragma unroll
    for (int e = 0; e < U::kElems; ++e) {
      const bool kept = (keep >> e) & 1u;
      if constexpr (kGrad)
        o[e] = kept ? g[e] : refined<DT>(w[e], g[e], decay);
      else
        o[e] = kept ? w[e] : 0u;
    }
  } else {
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const uint32_t sel = (((keep >> (2 * i)) & 1u) ? 0x0000FFFFu : 0u) |
                           (((keep >> (2 * i + 1)) & 1u) ? 0xFFFF0000u : 0u);
      if constexpr (kGrad) {
        const uint32_t lo = refined<DT>(w[i] & 0xFFFFu, g[i] & 0xFFFFu, decay);
        const uint32_t hi = refined<DT>(w[i] >> 16, g[i] >> 16, decay);
        o[i] = (g[i] & sel) | ((lo | (hi << 16)) & ~sel);
      } else {
        o[i] = w[i] & sel;
      }
    }
  }
}

template <int DT, int N, int M, bool kGrad>
__global__ void __launch_bounds__(kThreads) srste_unit_kernel(const uint32_t* W, const uint32_t* G,
                                                              int64_t units, float decay,
                                                              uint32_t* out) {
  using U = SrsteUnit<DT, M>;
  constexpr int NW = U::kWords;
  const int64_t first = (int64_t)blockIdx.x * kThreads * kUnitsPerThread + threadIdx.x;
  uint32_t w[kUnitsPerThread][NW], g[kUnitsPerThread][NW];
#pragma unroll
  for (int it = 0; it < kUnitsPerThread; ++it) {
    const int64_t u = first + (int64_t)it * kThreads;
    if (u < units) {
      load_unit<NW>(W + u * NW, w[it]);
      if constexpr (kGrad) load_unit<NW>(G + u * NW, g[it]);
    }
  }
#pragma unroll
  for (int it = 0; it < kUnitsPerThread; ++it) {
    const int64_t u = first + (int64_t)it * kThreads;
    if (u >= units) break;
    const uint32_t keep = unit_keep<DT, N, M, NW>(w[it]);
    uint32_t o[NW];
    unit_output<DT, M, kGrad, NW>(keep, w[it], g[it], decay, o);
    store_unit<NW>(out + u * NW, o);
  }
}

// Groups first_group .. first_group + groups - 1, one thread each.
template <int DT, int N, int M, bool kGrad>
__global__ void __launch_bounds__(kThreads) srste_group_kernel(const void* W, const void* G,
                                                               int64_t first_group,
                                                               int64_t groups, float decay,
                                                               void* out) {
  using E = typename Fmt<DT>::E;
  const int64_t gi = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (gi >= groups) return;
  const int64_t base = (first_group + gi) * M;
  const E* w = static_cast<const E*>(W) + base;
  uint32_t key[M], wv[M], gv[M];
#pragma unroll
  for (int i = 0; i < M; ++i) {
    wv[i] = w[i];
    key[i] = wv[i] & Elem<E>::kKeyMask;
    if constexpr (kGrad) gv[i] = static_cast<const E*>(G)[base + i];
  }
  const uint32_t keep = group_keep<E, N, M>(key);
  E* o = static_cast<E*>(out) + base;
#pragma unroll
  for (int i = 0; i < M; ++i) {
    const bool kept = (keep >> i) & 1u;
    if constexpr (kGrad)
      o[i] = (E)(kept ? gv[i] : refined<DT>(wv[i], gv[i], decay));
    else
      o[i] = (E)(kept ? wv[i] : 0u);
  }
}

inline unsigned grid_for(int64_t work, int64_t per_block) {
  return (unsigned)((work + per_block - 1) / per_block);
}

template <int DT, int N, int M, bool kGrad>
hipError_t run_srste(const void* W, const void* G, int64_t elems, float decay, void* out,
                     hipStream_t s) {
  using U = SrsteUnit<DT, M>;
  const int64_t units = elems / U::kElems;
  if (units > 0) {
    srste_unit_kernel<DT, N, M, kGrad>
        <<<grid_for(units, (int64_t)kThreads * kUnitsPerThread), kThreads, 0, s>>>(
            static_cast<const uint32_t*>(W), static_cast<const uint32_t*>(G), units, decay,
            static_cast<uint32_t*>(out));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t tail_groups = (elems - units * U::kElems) / M;
  if (tail_groups > 0) {
    srste_group_kernel<DT, N, M, kGrad><<<grid_for(tail_groups, kThreads), kThreads, 0, s>>>(
        W, G, units * U::kElems / M, tail_groups, decay, out);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <int DT, bool kGrad>
hipError_t dispatch_srste(int n, int m, const void* W, const void* G, int64_t elems, float decay,
                          void* out, hipStream_t s) {
#define NM_SRSTE_CASE(NN, MM) \
  if (n == NN && m == MM) return run_srste<DT, NN, MM, kGrad>(W, G, elems, decay, out, s);
  NM_SRSTE_CASE(1, 2) NM_SRSTE_CASE(2, 2)
  NM_SRSTE_CASE(1, 4) NM_SRSTE_CASE(2, 4) NM_SRSTE_CASE(3, 4) NM_SRSTE_CASE(4, 4)
  NM_SRSTE_CASE(1, 8) NM_SRSTE_CASE(2, 8) NM_SRSTE_CASE(3, 8) NM_SRSTE_CASE(4, 8)
  NM_SRSTE_CASE(5, 8) NM_SRSTE_CASE(6, 8) NM_SRSTE_CASE(7, 8) NM_SRSTE_CASE(8, 8)
#undef NM_SRSTE_CASE
  return hipErrorInvalidValue;
}

template <bool kGrad>
hipError_t launch_srste(const void* W, const void* G, int dt, int64_t R, int64_t K, int n, int m,
                        float decay, void* out, hipStream_t s) {
  const int64_t elems = R * K;
  if (elems == 0) return hipSuccess;
  if (dt == kF32) return dispatch_srste<kF32, kGrad>(n, m, W, G, elems, decay, out, s);
  if (dt == kF16) return dispatch_srste<kF16, kGrad>(n, m, W, G, elems, decay, out, s);
  return dispatch_srste<kBF16, kGrad>(n, m, W, G, elems, decay, out, s);
}

}  // namespace

hipError_t launch_prune(const void* W, int dt, int64_t R, int64_t K, int n, int m, void* out,
                        hipStream_t s) {
  return launch_srste<false>(W, nullptr, dt, R, K, n, m, 0.0f, out, s);
}

hipError_t launch_srste_grad(const void* W, const void* G, int dt, int64_t R, int64_t K, int n,
                             int m, float decay, void* out, hipStream_t s) {
  return launch_srste<true>(W, G, dt, R, K, n, m, decay, out, s);
}

}  // namespace nm
