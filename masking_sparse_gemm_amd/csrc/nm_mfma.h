// nm_mfma.h -- device pieces shared by the matrix-core product kernels (gfx950): vector
// types, element conversions, direct global -> LDS loads, the X-tile swizzle of the 32x32
// kernels and the LDS-staged epilogue that writes a wave's accumulators to Y.
#pragma once

#include "nm_device.h"

namespace nm {
namespace {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef short short16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16_t __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x16_t __attribute__((ext_vector_type(16)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

enum { kF32 = 0, kF16 = 1, kBF16 = 2, kI8 = 3, kI32 = 4, kFP8 = 5 };

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ float f16_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
// fp32 -> bf16 with the hardware conversion (v_cvt_pk_bf16_f32): round to nearest even,
// NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ uint32_t f32_to_f16(float x) {  // hardware conversion, RNE
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}
template <int YT>
__device__ __forceinline__ void store_from_f32(void* p, int64_t i, float v) {
  if constexpr (YT == kF32) static_cast<float*>(p)[i] = v;
  else if constexpr (YT == kBF16) static_cast<uint16_t*>(p)[i] = (uint16_t)f32_to_bf16(v);
  else static_cast<uint16_t*>(p)[i] = (uint16_t)f32_to_f16(v);
}

constexpr int kKStep = 64;  // K per pipeline step: one smfmac per fragment pair

typedef __attribute__((address_space(3))) void lds_void_t;

// Direct global -> LDS loads (global_load_lds_dword / _dwordx4): lane l of the wave
// writes its bytes at lds_wave_base + size * l.  The builtin is device-only; keeping it
// out of the host pass keeps the host-side launch stubs of the kernels that use it.
template <int kSize>
__device__ __forceinline__ void global_to_lds(const void* src, uint8_t* lds_wave_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  static_assert(kSize == 4 || kSize == 16, "dword or dwordx4");
  if constexpr (kSize == 16)
    __builtin_amdgcn_global_load_lds(src, (lds_void_t*)lds_wave_base, 16, 0, 0);
  else
    __builtin_amdgcn_global_load_lds(src, (lds_void_t*)lds_wave_base, 4, 0, 0);
#endif
}

// The same load with the address split into a wave-uniform 64-bit base (scalar
// registers) and a 32-bit per-lane offset: the saddr form of the instruction, which needs
// no per-lane 64-bit address arithmetic.  lds is the wave's LDS destination (written to M0;
// one wait state must separate that write from the load).  Operands are read when the
// instruction issues, and the load writes only LDS.
template <int kSize>
__device__ __forceinline__ void global_to_lds_sv(const void* sbase, uint32_t voff, uint32_t lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  static_assert(kSize == 4 || kSize == 16, "dword or dwordx4");
  if constexpr (kSize == 16)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(lds)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(lds)
                 : "memory", "m0");
#endif
}

// The same with a per-lane 64-bit address (the instruction's "off" form), for sources whose
// per-lane offsets do not fit 32 bits.
template <int kSize>
__device__ __forceinline__ void global_to_lds_v(const void* src, uint32_t lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  static_assert(kSize == 4 || kSize == 16, "dword or dwordx4");
  if constexpr (kSize == 16)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(src), "s"(lds)
                 : "memory", "m0");
#endif
}

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)(p);
}

typedef float float16v_t __attribute__((ext_vector_type(16)));

// LDS layout of an X stage for the 32x32 kernels: K row r holds BN columns as 32-byte
// pairs (16 columns each), logical pair p at physical pair p ^ xpair_swizzle(r).  A
// transposing B read has its two 16-lane column halves (adjacent logical pairs) on four
// rows r..r+3; the swizzle 2 (r & 3) puts one half on even and the other on odd pairs,
// so the 32 lanes of a pass touch all 64 banks exactly once.
__device__ __forceinline__ int xpair_swizzle(int r) { return (r & 3) << 1; }

// Stores one wave's 128 x 64 block of fp32 accumulators (32x32 fragments: fm = 0..3 down,
// f = 0..1 across; lane l holds column 32f + l % 32 and rows 8(i/4) + 4(l/32) + i%4 of
// fragment fm) to Y as YT.  Each 32-row slab passes through `lds` (this wave's own
// kEpilogueBytes, row-major) so that Y is written in 16-byte pieces of one row -- eight
// 16-bit or four fp32 outputs -- instead of one output per store.  When rows of Y are whole
// 16-byte pieces a piece is either wholly inside the matrix or wholly outside; for any other
// T each output of a piece is stored on its own.  A wave's LDS accesses complete in order,
// so the reads see this slab's writes and the next slab's writes follow the reads.
constexpr int kEpilogueBytes = 32 * (64 * 4 + 16);
template <int YT, typename AccV = float16v_t>
__device__ __forceinline__ void store_block_128x64(const AccV (&acc)[4][2], uint8_t* lds,
                                                   void* Y, int row0, int col0, int R, int T,
                                                   int lane) {
  constexpr int kEB = (YT == kF32 || YT == kI32) ? 4 : 2;   // bytes per output
  constexpr int kPitch = 64 * kEB + 16;     // LDS row pitch, padded against bank conflicts
  constexpr int kPer16 = 16 / kEB;          // outputs per 16-byte piece
  constexpr int kRowPieces = 64 / kPer16;
  static_assert(32 * kPitch <= kEpilogueBytes, "slab fits the wave's LDS region");
  const int l32 = lane & 31, q = lane >> 5;
  uint8_t* y = static_cast<uint8_t*>(Y);
#pragma unroll
  for (int fm = 0; fm < 4; ++fm) {
#pragma unroll
    for (int f = 0; f < 2; ++f) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        uint8_t* d = lds + (8 * (i / 4) + 4 * q + (i % 4)) * kPitch + (32 * f + l32) * kEB;
        const auto v = acc[fm][f][i];
        if constexpr (YT == kI32)
          *reinterpret_cast<int32_t*>(d) = v;
        else if constexpr (YT == kF32)
          *reinterpret_cast<float*>(d) = v;
        else if constexpr (YT == kBF16)
          *reinterpret_cast<uint16_t*>(d) = (uint16_t)f32_to_bf16(v);
        else
          *reinterpret_cast<uint16_t*>(d) = (uint16_t)f32_to_f16(v);
      }
    }
#pragma unroll
    for (int k = 0; k < 32 * kRowPieces / 64; ++k) {
      const int pc = k * 64 + lane, r = pc / kRowPieces, cp = pc % kRowPieces;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(lds + r * kPitch + cp * 16);
      const int row = row0 + 32 * fm + r, col = col0 + cp * kPer16;
      if (T % kPer16 == 0) {  // rows of Y are whole 16-byte pieces
        if (row < R && col < T)
          *reinterpret_cast<u32x4_t*>(y + ((int64_t)row * T + col) * kEB) = v;
      } else if (row < R) {  // any other T: one store per output, none past the last column
        const uint32_t w[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
        for (int e = 0; e < kPer16; ++e) {
          if (col + e < T) {
            uint8_t* d = y + ((int64_t)row * T + col + e) * kEB;
            if constexpr (kEB == 4)
              *reinterpret_cast<uint32_t*>(d) = w[e];
            else
              *reinterpret_cast<uint16_t*>(d) = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
          }
        }
      }
    }
  }
}


}  // namespace
}  // namespace nm
