// Launch interface of the pyramid kernels (one streaming pass per cache refresh).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wf {

constexpr int kPyrMaxLevels = 7;

struct PyramidLaunch {
  const void* k;
  int64_t head_stride;  // elements
  int heads_total;      // batch * heads
  int n_prompt, head_dim, levels;
  bool bf16;            // element type of k: bfloat16, else float32
  bool all_levels;      // also store A_1..A_{L-1} and D_1..D_L
  bool db2;             // Daubechies four-tap filters with periodic extension (implies all_levels)
  float* base;          // pyramid buffer
  uint64_t band_off_a[kPyrMaxLevels + 1];  // byte offsets, A_j (j = L at 0)
  uint64_t band_off_d[kPyrMaxLevels + 1];  // byte offsets, D_j
};

hipError_t launch_pyramid(const PyramidLaunch& a, hipStream_t s);

// Incremental refresh of A_L: items (one per layer) list level-L blocks whose
// prompt keys changed; one wave per (item, head, listed block).
constexpr int kMaxRefreshItems = 32;
struct RefreshItem {
  const void* k;            // prompt keys of the layer
  int64_t head_stride;      // elements
  float* a_top;             // A_L of the layer's pyramid [heads_total][n_top][d]
  const int32_t* blocks;    // device [n_blocks]; entries outside [0, n_top) are skipped
  int64_t unit_begin;       // first wave index of this item
  int n_blocks, n_top, levels;
  float scale;              // 2^{-L/2}, computed as the full build does
};
struct RefreshLaunch {
  RefreshItem items[kMaxRefreshItems];
  int n_items, head_dim;
  bool bf16;
  int64_t units_total;      // sum over items of n_blocks * heads_total
};

hipError_t launch_refresh(const RefreshLaunch& r, hipStream_t s);

}  // namespace wf
