// nm_launch.h -- internal launchers behind the C ABI (validated arguments only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nm {

// `blocked` selects NM_LAYOUT_BLOCKED for the compressed pair (K % 64 == 0 checked).

// Mask and/or compress: mask may be null (compress only); values/meta may be null (mask only).
// dt is the nm_dtype code of W (its magnitude key depends on it, not only on its size).
hipError_t launch_select(const void* W, int dt, int64_t R, int64_t K, int n, int m,
                         bool blocked, void* values, uint32_t* meta, uint8_t* mask,
                         hipStream_t s);

hipError_t launch_decompress(const void* values, const uint32_t* meta, int elem_bytes, int64_t R,
                             int64_t K, int n, int m, bool blocked, void* out, hipStream_t s);

// XCDs of the current device (8 on MI355X; 1 if unknown), looked up once per device.
int xcd_count();

// dt / y_dt use the nm_dtype codes: 0 fp32, 1 fp16, 2 bf16.
hipError_t launch_spmm(const void* values, const uint32_t* meta, int64_t R, int64_t K, int n,
                       int m, bool blocked, const void* X, int64_t T, int dt, void* Y, int y_dt,
                       hipStream_t s);

// The 2:4 16-bit product on 256 x 256 tiles split over the compute units by K steps
// (nm_spmm_sk.hip), blocked layout, dt / y_dt as for launch_spmm.  sk_shape_ok: the
// shapes it takes (K % 64 == 0, T % 8 == 0, sizes within its 32-bit offsets);
// sk_preferred: shapes where it is taken without NM_SPMM_TILE=3 (none at present: the
// wave-specialised kernel is faster on every measured shape).  The workspace (device memory
// of sk_workspace_bytes(R, T, groups) bytes, 256-byte aligned; none, and NULL may be
// passed, when every workgroup gets whole tiles) holds one flag and one partial 256 x 256
// fp32 tile per workgroup; its initial contents do not matter.
bool sk_shape_ok(int64_t R, int64_t K, int64_t T);
bool sk_preferred(int64_t R, int64_t K, int64_t T);
int sk_groups(int64_t R, int64_t K, int64_t T);
int64_t sk_workspace_bytes(int groups);                    // the largest it may need
int64_t sk_workspace_bytes(int64_t R, int64_t T, int groups);  // 0: no tile is cut
hipError_t launch_spmm_sk(const void* values, const uint32_t* meta, int64_t R, int64_t K,
                          const void* X, int64_t T, int dt, void* Y, int y_dt, void* workspace,
                          int groups, hipStream_t s);

// Compress of W's transpose (the K x R matrix, groups of m along R; R % m == 0, and
// R % 64 == 0 for the blocked layout).
hipError_t launch_select_t(const void* W, int elem_bytes, int64_t R, int64_t K, int n, int m,
                           bool blocked, void* values, uint32_t* meta, hipStream_t s);

// Transposable mask of W (R % m == K % m == 0): mask bytes, or the pruned weight if `prune`.
hipError_t launch_tmask(const void* W, int elem_bytes, int64_t R, int64_t K, int n, int m,
                        bool prune, void* out, hipStream_t s);

// Channel permutation (nm_perm.hip): workspace bytes, one round's gains (device perm and
// outputs), and the whole search (host perm, synchronous on s).
size_t perm_workspace_bytes(int64_t R, int64_t K, int m);
hipError_t launch_perm_gains(const void* W, int dt, int64_t R, int64_t K, int n, int m,
                             const int32_t* perm, float* gain, int32_t* pick, void* workspace,
                             hipStream_t s);
hipError_t run_perm_search(const void* W, int dt, int64_t R, int64_t K, int n, int m,
                           int max_rounds, int32_t* perm_host, int* rounds, void* workspace,
                           hipStream_t s);

// SR-STE passes (dt in nm_dtype codes); `out` may be W (prune) or G (grad).
hipError_t launch_prune(const void* W, int dt, int64_t R, int64_t K, int n, int m, void* out,
                        hipStream_t s);
hipError_t launch_srste_grad(const void* W, const void* G, int dt, int64_t R, int64_t K, int n,
                             int m, float decay, void* out, hipStream_t s);

}  // namespace nm
