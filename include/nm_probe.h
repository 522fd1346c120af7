/*
 * nm_probe.h -- C ABI of libnm_probe: measurement kernels that bound the sparse product
 * from above on this device.  They compute nothing of the method; bench.py uses them to
 * state what the matrix cores themselves sustain on the product's kind of data, beside
 * what the product reaches.
 *
 * "[리뷰] Accelerating Sparse Deep Neural Networks", section "Tensor Scores 상에서
 * 구조적인 sparse GEMM", gives the structured-sparse product up to twice the dense math
 * rate; on gfx950 the rate of the sparse instruction also depends on the operand values
 * (the device lowers its clock under heavy matrix-core load, more so for values with many
 * toggling bits), so the probe runs the instruction alone on caller-chosen operands.
 *
 * The VALU loop does the same for the vector ALU, the unit the permutation search's gains
 * kernel is bound by, and the load-path probe replays the product's direct loads alone.
 *
 * Pointers are DEVICE pointers owned by the caller; calls are asynchronous on `stream`
 * (a hipStream_t as void*, NULL = the default stream).  Returns 0 when the launch was
 * enqueued, 1 for invalid arguments, 2 for a launch error.
 */
#ifndef NM_PROBE_H
#define NM_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of the operand buffer nm_probe_matrix_core reads: 4 operand sets x 64 lanes x
 * 24 16-bit values (8 for the A operand, 16 for the B operand of each lane). */
int64_t nm_probe_operand_bytes(void);

/* Matrix-core rate loop.  kind 0: v_smfmac_f32_32x32x32_bf16 (2:4 structured-sparse,
 * 65,536 dense-equivalent flops per instruction, 32,768 algorithmic); kind 1: dense
 * v_mfma_f32_32x32x16_bf16 (32,768 flops).  Every wave loads the 4 operand sets of its
 * lane from `operands` (bf16 bit patterns, layout [set][lane][24]) and then issues
 * `iters` x 16 instructions over 4 independent accumulators, rotating the operand sets so
 * that consecutive instructions see different values; the index operand of the sparse
 * instruction cycles through the six legal 2:4 nibbles.  The grid is cus * waves_per_simd
 * workgroups of four waves (1 <= waves_per_simd <= 8); workgroups that do not fit on the
 * device at once run after the others.  clocks (int64[4 * cus * waves_per_simd])
 * receives, per workgroup, the shader-clock counter (s_memtime) and the 100 MHz real-time
 * counter (s_memrealtime) read by its first wave at the start and at the end of its loop:
 * [memtime0, memtime1, realtime0, realtime1]; sink (float[cus * waves_per_simd * 256])
 * receives one accumulator sum per lane so the work is not optimised away. */
int nm_probe_matrix_core(int kind, const void* operands, int cus, int waves_per_simd, int iters,
                         int64_t* clocks, float* sink, void* stream);

/* VALU issue-rate loop, the bound of the permutation gains kernel (fp32 max, min, add and
 * select on registers).  op 0: v_add_f32, 1: v_max_f32, 2: v_fma_f32 (plain, not packed).
 * Every lane keeps 16 independent fp32 chains; every wave issues iters x 64 instructions of
 * that one kind.  Grid, clocks and sink as in nm_probe_matrix_core. */
int nm_probe_valu(int op, int cus, int waves_per_simd, int iters, int64_t* clocks, float* sink,
                  void* stream);

/* HBM streaming copy: dst[0, bytes) = src[0, bytes) with 16-byte non-temporal loads and
 * stores per lane (bytes a multiple of 16, both pointers 16-byte aligned, the ranges not
 * overlapping; else 1).  The rate a pass that reads and writes each byte once can reach. */
int nm_probe_copy(const void* src, void* dst, int64_t bytes, void* stream);

/* The direct-load stream of the 2:4 16-bit product on its 256 x 128 tiles, alone: the
 * same global -> LDS loads (X rows, compressed values and metadata in the blocked layout,
 * 34,816 bytes per 64-wide K step and tile), the same 4-stage LDS ring, wait counts,
 * barrier per step and workgroup -> tile mapping as the product's producer waves, with
 * idle waves in place of the consumers; nothing is computed or written.  values and meta
 * are a 2:4 16-bit compressed pair of an R x K weight in NM_LAYOUT_BLOCKED (as nm_compress
 * writes it), X is K x T 16-bit: the product's inputs.  Requires K % 64 == 0, T % 8 == 0,
 * 16-byte aligned pointers, R < 2^28, K < 2^22, T < 2^24 (else 1).  Its time is what the
 * product's loads take without its matrix work: a bound on the product from above. */
int nm_probe_load_path(const void* values, const void* meta, const void* X, int64_t R,
                       int64_t K, int64_t T, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* NM_PROBE_H */
