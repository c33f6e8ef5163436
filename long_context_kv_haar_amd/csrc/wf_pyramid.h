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
  float* base;          // pyramid buffer
  uint64_t band_off_a[kPyrMaxLevels + 1];  // byte offsets, A_j (j = L at 0)
  uint64_t band_off_d[kPyrMaxLevels + 1];  // byte offsets, D_j
};

hipError_t launch_pyramid(const PyramidLaunch& a, hipStream_t s);

}  // namespace wf
