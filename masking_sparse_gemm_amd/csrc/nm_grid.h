// nm_grid.h -- launch sizes of the grid-stride kernels.  Plain C++ with no HIP types, so
// that a host-only test can compile it and check the sizes for shapes no GPU run reaches.
#ifndef NM_GRID_H
#define NM_GRID_H

#include <cstdint>

namespace nm {

// The most workgroups a grid-stride launch takes: 65,536 workgroups of 256 work-items is
// 2^24 work-items, 256 per compute unit, far below the 2^32 work-items one launch may
// have, and enough to keep every compute unit busy.
constexpr int64_t kMaxStrideBlocks = 65536;

// Workgroups for `work` items at one item per work-item and `per_block` work-items per
// workgroup: one pass when that needs at most kMaxStrideBlocks workgroups, else
// kMaxStrideBlocks, and the kernel visits items i, i + gridDim.x * per_block, ... .  At
// least one workgroup (work == 0 launches one that does nothing).
inline unsigned stride_grid(int64_t work, int64_t per_block) {
  const int64_t blocks = (work + per_block - 1) / per_block;
  return (unsigned)(blocks < 1 ? 1 : blocks > kMaxStrideBlocks ? kMaxStrideBlocks : blocks);
}

}  // namespace nm

#endif  // NM_GRID_H
