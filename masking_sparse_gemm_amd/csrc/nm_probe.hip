// nm_probe.hip -- rate loops that bound the sparse product on this device
// (include/nm_probe.h).  Nothing here computes part of the method.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/nm_probe.h"
#include "nm_mfma.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16_t __attribute__((ext_vector_type(16)));
typedef float float16v_t __attribute__((ext_vector_type(16)));
typedef unsigned short u16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned short u16x16_t __attribute__((ext_vector_type(16)));

constexpr int kSets = 4;
constexpr int kPerLane = 24;  // 8 A values + 16 B values

// The six legal 2:4 nibbles (i0 | i1 << 2 with i0 < i1), four to a 16-bit index word.
__device__ __forceinline__ int index_word(int k) {
  const int nib[6] = {0x4, 0x8, 0xC, 0x9, 0xD, 0xE};
  return nib[k % 6] | nib[(k + 1) % 6] << 4 | nib[(k + 2) % 6] << 8 | nib[(k + 3) % 6] << 12;
}

template <int KIND>
__global__ void __launch_bounds__(256) probe_kernel(const uint16_t* __restrict__ ops, int iters,
                                                    int64_t* __restrict__ clocks,
                                                    float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a[kSets];
  bf16x16_t b[kSets];
#pragma unroll
  for (int s = 0; s < kSets; ++s) {
    const uint16_t* p = ops + ((size_t)s * 64 + lane) * kPerLane;
    u16x8_t av;
    u16x16_t bv;
#pragma unroll
    for (int i = 0; i < 8; ++i) av[i] = p[i];
#pragma unroll
    for (int i = 0; i < 16; ++i) bv[i] = p[8 + i];
    a[s] = __builtin_bit_cast(bf16x8_t, av);
    b[s] = __builtin_bit_cast(bf16x16_t, bv);
  }
  const int ix0 = index_word(lane), ix1 = index_word(lane + 1), ix2 = index_word(lane + 2),
            ix3 = index_word(lane + 3);
  float16v_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const bool timer = threadIdx.x == 0;
  int64_t t0 = 0, r0 = 0;
  if (timer) {
    t0 = (int64_t)__builtin_amdgcn_s_memtime();
    r0 = (int64_t)__builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; ++it) {
    // 16 instructions: four independent accumulators, each operand set in turn
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int s0 = r, s1 = (r + 1) & 3, s2 = (r + 2) & 3, s3 = (r + 3) & 3;
      if constexpr (KIND == 0) {
        c0 = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a[s0], b[s1], c0, ix0, 0, 0);
        c1 = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a[s1], b[s2], c1, ix1, 0, 0);
        c2 = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a[s2], b[s3], c2, ix2, 0, 0);
        c3 = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a[s3], b[s0], c3, ix3, 0, 0);
      } else {
        const bf16x8_t b0 = __builtin_shufflevector(b[s1], b[s1], 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8_t b1 = __builtin_shufflevector(b[s2], b[s2], 8, 9, 10, 11, 12, 13, 14, 15);
        const bf16x8_t b2 = __builtin_shufflevector(b[s3], b[s3], 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8_t b3 = __builtin_shufflevector(b[s0], b[s0], 8, 9, 10, 11, 12, 13, 14, 15);
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s0], b0, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s1], b1, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s2], b2, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s3], b3, c3, 0, 0, 0);
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  if (timer) {
    const int64_t t1 = (int64_t)__builtin_amdgcn_s_memtime();
    const int64_t r1 = (int64_t)__builtin_amdgcn_s_memrealtime();
    int64_t* c = clocks + 4 * blockIdx.x;
    c[0] = t0;
    c[1] = t1;
    c[2] = r0;
    c[3] = r1;
  }
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// VALU issue-rate loop: 16 independent fp32 chains per lane, 64 wave instructions of one
// kind per iteration, nothing but registers.  OP 0: v_add_f32, 1: v_max_f32, 2: v_fma_f32.
template <int OP>
__global__ void __launch_bounds__(256) valu_probe_kernel(int iters, int64_t* __restrict__ clocks,
                                                         float* __restrict__ sink) {
  float a[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) a[i] = (float)(threadIdx.x + i) * 0.25f;
  const float b = 1.0f / (float)(threadIdx.x + 3);
  const float c = 0.5f;
  const bool timer = threadIdx.x == 0;
  int64_t t0 = 0, r0 = 0;
  if (timer) {
    t0 = (int64_t)__builtin_amdgcn_s_memtime();
    r0 = (int64_t)__builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if constexpr (OP == 0) {
          asm volatile("v_add_f32 %0, %0, %1" : "+v"(a[i]) : "v"(b));
        } else if constexpr (OP == 1) {
          asm volatile("v_max_f32 %0, %0, %1" : "+v"(a[i]) : "v"(b));
        } else {
          asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(a[i]) : "v"(b), "v"(c));
        }
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += a[i];
  if (timer) {
    const int64_t t1 = (int64_t)__builtin_amdgcn_s_memtime();
    const int64_t r1 = (int64_t)__builtin_amdgcn_s_memrealtime();
    int64_t* cl = clocks + 4 * blockIdx.x;
    cl[0] = t0;
    cl[1] = t1;
    cl[2] = r0;
    cl[3] = r1;
  }
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Plain streaming copy, 16 bytes per lane per iteration, non-temporal on both sides: the
// HBM rate a pass that reads and writes once can reach.  Grid-stride over n16 pieces.
typedef unsigned int u32x4v_t __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) copy_probe_kernel(const u32x4v_t* __restrict__ src,
                                                         u32x4v_t* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// ---------------------------------------------------------------------------------------
// The direct-load stream of the 2:4 16-bit product on 256 x 128 tiles (blocked layout,
// T % 8 == 0) with nothing else: per 64-wide K step and tile, 16 KB of X rows, 16 KB of
// compressed values and 2 KB of metadata land in a 4-stage LDS ring, issued by four
// producer waves with the same addresses, wait counts and one barrier per step as the
// product's producers, while four idle waves pass the same barriers in place of the
// consumers (so one workgroup holds a compute unit's LDS, as the product's does).  Its time
// is what the product's loads take alone.
// ---------------------------------------------------------------------------------------
constexpr int kLpBM = 256, kLpBN = 128, kLpStages = 4, kLpProducers = 4;
constexpr int kLpXBytes = nm::kKStep * kLpBN * 2;  // 64 K rows of 128 columns
constexpr int kLpABytes = kLpBM * 64;               // 32 kept values a row
constexpr int kLpMBytes = kLpBM * 8;                // 64 metadata bits a row
constexpr int kLpStageBytes = kLpXBytes + kLpABytes + kLpMBytes;
constexpr int kLpXLoads = kLpXBytes / 1024 / kLpProducers;
constexpr int kLpALoads = kLpABytes / 1024 / kLpProducers;
constexpr int kLpLoads = kLpXLoads + kLpALoads + 1;

// Workgroup -> tile: workgroup b runs on XCD b % xcds; each XCD takes a contiguous range
// of the tile order, which walks gm x gn groups of tiles (the product's mapping).
struct LpMap {
  int tiles_m, tiles_n, xcds, per_xcd, gm, gn;
  __device__ bool tile_of(int b, int& tm, int& tn) const {
    const int t = (b % xcds) * per_xcd + b / xcds;
    if (t >= tiles_m * tiles_n) return false;
    const int g_m = t / (gm * tiles_n);
    const int rows = min(gm, tiles_m - g_m * gm);
    const int u = t - g_m * gm * tiles_n;
    const int g_n = u / (rows * gn);
    const int v = u - g_n * rows * gn;
    tm = g_m * gm + v % rows;
    tn = g_n * gn + v / rows;
    return true;
  }
};

__global__ void __launch_bounds__(512) load_path_probe_kernel(const uint8_t* __restrict__ values,
                                                              const uint8_t* __restrict__ meta,
                                                              const uint8_t* __restrict__ X,
                                                              int R, int K, int T, LpMap map) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  int tile_m, tile_n;
  if (!map.tile_of(blockIdx.x, tile_m, tile_n)) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m0 = tile_m * kLpBM, t0 = tile_n * kLpBN;
  const int nsteps = K / nm::kKStep;
  if (wave < 4) {  // in place of the consumers: the same barriers, nothing else
    for (int s = 0; s < nsteps + 2; ++s) asm volatile("s_barrier" ::: "memory");
    return;
  }
  const int pw = wave - 4;
  const int last_step = nsteps - 1;
  // X: load j fills 1 KB window w = 4 j + pw of the stage (K rows 4w .. 4w+3); lane l takes
  // row 4w + l / 16 and the 16-byte piece that lands at physical piece l % 16
  const int r = lane >> 4, pc = lane & 15;
  const int lc = 2 * ((pc >> 1) ^ nm::xpair_swizzle(r)) + (pc & 1);
  int col = t0 + 8 * lc;
  col = col < T ? col : 0;
  const uint32_t x_off = (uint32_t)(((int64_t)r * T + col) * 2);
  // values: load j fills the 1 KB block of tile rows 16 (4 j + pw) .. +15 for the step
  const int last = ((R + 15) >> 4) - 1;
  const uint32_t a_off = (uint32_t)((lane >> 2) * 64 + 16 * ((lane & 3) ^ ((lane >> 4) & 3)));
  // metadata: four 128-byte blocks per producer, one 16-byte piece on each of 32 lanes
  int g0 = (m0 >> 4) + 4 * pw;
  g0 = g0 < last ? g0 : last;
  int g = (m0 >> 4) + 4 * pw + ((lane & 31) >> 3);
  g = g < last ? g : last;
  const uint8_t* m16_base = meta + (int64_t)g0 * nsteps * 128;
  const uint32_t m16_off = (uint32_t)((g - g0) * nsteps * 128 + 16 * (lane & 7));
  auto issue_step = [&](int step) {
    const uint32_t sta = nm::lds_addr(smem + (step % kLpStages) * kLpStageBytes);
    step = step < last_step ? step : last_step;
    const int64_t kx = (int64_t)step * nm::kKStep * T * 2;
#pragma unroll
    for (int j = 0; j < kLpXLoads; ++j) {
      const int w = j * kLpProducers + pw;
      nm::global_to_lds_sv<16>(X + (int64_t)(4 * w) * T * 2 + kx, x_off, sta + (uint32_t)(w * 1024));
    }
#pragma unroll
    for (int j = 0; j < kLpALoads; ++j) {
      const int b16 = j * kLpProducers + pw;
      int gb = (m0 >> 4) + b16;
      gb = gb < last ? gb : last;
      nm::global_to_lds_sv<16>(values + (int64_t)gb * nsteps * 1024 + (int64_t)step * 1024, a_off,
                               sta + (uint32_t)(kLpXBytes + b16 * 1024));
    }
    if (lane < 32)
      nm::global_to_lds_sv<16>(m16_base + (int64_t)step * 128, m16_off,
                               sta + (uint32_t)(kLpXBytes + kLpABytes + pw * 512));
  };
#pragma unroll
  for (int k = 0; k < kLpStages - 1; ++k) issue_step(k);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kLpStages - 3) * kLpLoads) : "memory");
  asm volatile("s_barrier" ::: "memory");
  for (int s = 0; s < nsteps; ++s) {
    issue_step(s + kLpStages - 1);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kLpStages - 3) * kLpLoads) : "memory");
    asm volatile("s_barrier" ::: "memory");
  }
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace

extern "C" {

int64_t nm_probe_operand_bytes(void) { return (int64_t)kSets * 64 * kPerLane * 2; }

int nm_probe_matrix_core(int kind, const void* operands, int cus, int waves_per_simd, int iters,
                         int64_t* clocks, float* sink, void* stream) {
  if ((kind != 0 && kind != 1) || operands == nullptr || clocks == nullptr || sink == nullptr ||
      cus < 1 || cus > 4096 || waves_per_simd < 1 || waves_per_simd > 8 || iters < 1)
    return 1;
  // one workgroup of four waves (one per SIMD) per compute unit and wave per SIMD
  auto k = kind == 0 ? probe_kernel<0> : probe_kernel<1>;
  hipLaunchKernelGGL(k, dim3(cus * waves_per_simd), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(operands),
                     iters, clocks, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int nm_probe_valu(int op, int cus, int waves_per_simd, int iters, int64_t* clocks, float* sink,
                  void* stream) {
  if (op < 0 || op > 2 || clocks == nullptr || sink == nullptr || cus < 1 || cus > 4096 ||
      waves_per_simd < 1 || waves_per_simd > 8 || iters < 1)
    return 1;
  auto k = op == 0 ? valu_probe_kernel<0> : op == 1 ? valu_probe_kernel<1> : valu_probe_kernel<2>;
  hipLaunchKernelGGL(k, dim3(cus * waves_per_simd), dim3(256), 0,
                     static_cast<hipStream_t>(stream), iters, clocks, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int nm_probe_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (src == nullptr || dst == nullptr || bytes <= 0 || bytes % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(src) & 15) != 0 || (reinterpret_cast<uintptr_t>(dst) & 15) != 0)
    return 1;
  const int64_t n16 = bytes / 16;
  // about four pieces per lane, at most 65536 workgroups
  int64_t blocks = (n16 + 256 * 4 - 1) / (256 * 4);
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(copy_probe_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4v_t*>(src),
                     static_cast<u32x4v_t*>(dst), n16);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int nm_probe_load_path(const void* values, const void* meta, const void* X, int64_t R,
                       int64_t K, int64_t T, void* stream) {
  const auto misaligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; };
  if (values == nullptr || meta == nullptr || X == nullptr || misaligned(values) ||
      misaligned(meta) || misaligned(X) || R <= 0 || K <= 0 || T <= 0 || K % 64 != 0 ||
      T % 8 != 0 || R >= (1 << 28) || K >= (1 << 22) || T >= (1 << 24))
    return 1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 2;
  LpMap map;
  map.tiles_m = (int)((R + kLpBM - 1) / kLpBM);
  map.tiles_n = (int)((T + kLpBN - 1) / kLpBN);
  map.xcds = cus % 8 == 0 ? 8 : 1;
  map.per_xcd = (map.tiles_m * map.tiles_n + map.xcds - 1) / map.xcds;
  map.gn = map.tiles_n < 4 ? map.tiles_n : 4;
  map.gm = 32 / map.gn;
  const int lds = kLpStages * kLpStageBytes;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(load_path_probe_kernel),
      hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return 2;
  hipLaunchKernelGGL(load_path_probe_kernel, dim3(map.xcds * map.per_xcd), dim3(512), lds,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(values),
                     static_cast<const uint8_t*>(meta), static_cast<const uint8_t*>(X), (int)R,
                     (int)K, (int)T, map);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
