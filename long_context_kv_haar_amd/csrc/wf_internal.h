// Host-side launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/wavefilter.h"

namespace wf {

constexpr int kMaxLevels = WF_MAX_LEVELS;
constexpr int kCoverTokensPerWave = 64;  // positions per wave in the coverage kernel
constexpr int kAttendChunkBf16 = 64;     // tokens per attention chunk (bf16)
constexpr int kAttendChunkF32 = 32;      // tokens per attention chunk (f32)
constexpr int kMaxSplit = 16;            // attention splits per head
constexpr int kRefineThreads = 512;
constexpr int kRefineLdsBytes = 64 * 1024;

struct PyramidLaunch {
  const void* k;
  int64_t head_stride;  // elements
  int heads_total;      // batch * heads
  int n_prompt, head_dim, dtype, levels;
  uint32_t flags;
  float* base;          // pyramid buffer
  uint64_t band_off_a[kMaxLevels + 1];  // byte offsets, A_j (j = L at 0)
  uint64_t band_off_d[kMaxLevels + 1];  // byte offsets, D_j
};

// Byte layout of the per-call workspace, and the resolved launch shape.
struct SelectPlan {
  int heads_total, n_q, n_top, n_prompt, head_dim, dtype, levels, n_tot, n_gen;
  int budgets[kMaxLevels + 1];  // k_L .. k_0
  int k_top, k0, sum_k;
  int64_t covered;              // k_L 2^L
  int64_t cov_len;              // floats per head over levels 0..L-1
  int64_t cov_off[kMaxLevels];  // float offset of level j inside a head's slice
  int n_att, n_chunks, n_split, chunks_per_split;
  int refine_lds;               // dynamic LDS bytes of the refine kernel
  // workspace sections (byte offsets)
  uint64_t off_counters, off_keys, off_sel_top, off_cov, off_sel0, off_part_ml, off_part_o, total;
};

struct SelectLaunch {
  SelectPlan plan;
  const void* q;
  const float* a_top;
  const void* k;
  const void* v;
  const int32_t* gen_idx;
  float* out;
  int32_t* sel_out;
  int32_t* sel_levels;
  float* score_levels;
  uint8_t* ws;
};

hipError_t launch_pyramid(const PyramidLaunch& a, hipStream_t s);
hipError_t launch_select_attend(const SelectLaunch& a, hipStream_t s);

}  // namespace wf
