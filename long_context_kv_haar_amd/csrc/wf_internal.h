// Host-side launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/wavefilter.h"
#include "wf_pyramid.h"

namespace wf {

constexpr int kMaxLevels = WF_MAX_LEVELS;
static_assert(kMaxLevels == kPyrMaxLevels, "one level limit");
constexpr int kAttendGroups = 2;          // waves per query tile in the attention workgroup
constexpr int kMaxSplit = 16;             // attention splits per head
constexpr int kMaxCoarseLds = 16384;      // coarse keys staged in LDS up to this count
constexpr int kMaxKeepTop = 16384;        // k_L limit (kept coarse regions live in LDS)
constexpr int kLdsLimit = 160 * 1024;     // LDS per workgroup on gfx950
constexpr int kTopKSharedReserve = 20 * 1024;  // static LDS of the Top-K scratch and friends
constexpr int kRefineThreads = 512;       // one refinement workgroup per head
constexpr int kMaskGroup = 2048;          // least positions a refinement mask spans
constexpr int kCoverThreads = 256;

// Byte layout of the per-call workspace, and the resolved launch shape.
struct SelectPlan {
  int heads_total, n_q, n_top, n_prompt, head_dim, dtype, levels, n_tot, n_gen;
  int budgets[kMaxLevels + 1];  // k_L .. k_0
  int k_top, k0, sum_k;
  int64_t covered;              // k_L 2^L
  int64_t cov_len;              // floats per head over levels 0..L-1 (each level 16-byte aligned)
  int64_t cov_off[kMaxLevels];  // float offset of level j inside a head's slice
  // attention
  int n_att, chunk, n_chunks, n_split, chunks_per_split;
  // LDS plans (bytes)
  int cover_lds;                // kept coarse regions (+ coarse keys when staged)
  int coarse_keys_in_lds;
  int refine_nmax, refine_kmax; // candidate / kept capacity (words, multiples of 4)
  int refine_mask_words;        // words of one bitmask over the covered positions
  int refine_cov_in_lds;        // coverage scores staged in LDS
  int refine_lds;               // refinement workgroup: its state (kept sets, candidate lists)
  int att_t_words;              // words of the attended-set list (T) region
  int attend_lds;               // T list + K/V chunk buffers
  // workspace sections (byte offsets)
  uint64_t off_keys, off_sel_top, off_cov, off_lvl, off_sel, off_part_ml, off_part_o, total;
};

struct SelectLaunch {
  SelectPlan plan;
  const void* q;
  const float* a_top;
  const void* k;
  const void* v;
  const int32_t* gen_idx;
  const int32_t* sel_in;  // attention only: the kept prompt tokens [heads_total][k0] (NULL if k0 == 0)
  int attend_only;        // 1: skip selection, attend over sel_in and gen_idx
  float* out;
  int32_t* sel_out;
  int32_t* sel_levels;
  float* score_levels;
  uint8_t* ws;
};

hipError_t launch_select_attend(const SelectLaunch& a, hipStream_t s);

// Tokens per attention chunk; each of the kAttendGroups waves of a query
// tile takes an equal slice.
constexpr int attend_chunk(int dtype) { return dtype == WF_BF16 ? 128 : 64; }

// LDS bytes after the attended-set list: the chunk buffers (K rows,
// transposed V), aliased at the end by the merge slots of the wave states
// (kAttendGroups / 2 slots per query tile).
inline int attend_buffer_bytes(int dtype, int head_dim, int nqt) {
  const bool bf = dtype == WF_BF16;
  const int es = bf ? 2 : 4;
  const int ch = attend_chunk(dtype);
  const int kpad = bf ? 8 : 4, vpad = bf ? 16 : 4;
  const int kv = ch * (head_dim + kpad) * es + head_dim * (ch + vpad) * es;
  const int merge = (kAttendGroups / 2) * nqt * 64 * (head_dim / 4 + 2) * 4;
  return kv > merge ? kv : merge;
}

}  // namespace wf
