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
constexpr int kMaxItems = WF_MAX_LAYER_ITEMS;  // layers of one batched select-attend call
constexpr int kMaxCoarseLds = 16384;      // general coarse Top-K: keys staged in LDS up to this count
constexpr int kMaxKeepTop = 16384;        // k_L limit (kept coarse regions live in LDS)
constexpr int kLdsLimit = 160 * 1024;     // LDS per workgroup on gfx950
constexpr int kTopKSharedReserve = 20 * 1024;  // static LDS of the selection scratch and friends
constexpr int kCoverThreads = 256;
constexpr int kRegSelMax = 256 * 32;      // coarse regions the in-register coarse Top-K holds
constexpr int kRefineThreadsHost = 1024;  // threads of the refinement workgroup

// Byte layout of the per-call workspace, and the resolved launch shape.
struct SelectPlan {
  int heads_total, n_q, n_top, n_prompt, head_dim, dtype, levels, n_tot, n_gen;
  int budgets[kMaxLevels + 1];  // k_L .. k_0
  int k_top, k0, sum_k;
  int64_t covered;              // k_L 2^L
  int64_t cov_len;              // floats per head over levels 0..L-1 (each level 16-byte aligned)
  int64_t cov_off[kMaxLevels];  // float offset of level j inside a head's slice
  // attention: T = kept prompt tokens [0, k0) then generated positions
  // [k0, k0 + n_gen), each part cut into chunks of `chunk` tokens on its own;
  // splits 0 .. n_split_p - 1 take cps_p prompt chunks each, the remaining
  // n_split - n_split_p take cps_g generated chunks each
  int n_att, chunk, n_split, n_split_p, cps_p, cps_g;
  // launch shapes and LDS plans (bytes)
  int coarse_wg, cover_wg;      // workgroups per head of the coarse and cover launches
  int topk_s;                   // coarse keys per thread of the in-register coarse Top-K (0: general path)
  int coarse_keys_in_lds;       // general coarse Top-K: keys staged in LDS
  int coarse_lds;               // coarse launch: the staged keys
  int cover_lds;                // cover launch: the kept coarse regions
  int refine_s0;                // level-0 positions per thread of the in-register refinement (0: list-based)
  int refine_nmax, refine_kmax; // list-based refinement: candidate / kept capacity (words, multiples of 4)
  int refine_cov_in_lds;        // list-based refinement: coverage scores staged in LDS
  int refine_lds;               // list-based refinement workgroup: its state
  int stored_bands;             // levels 1 .. L-1 scored from stored A_j (longer bases)
  int soft;                     // softmax-probability scores: 0 off, 1 maximum, 2 mean over the query rows
  int n_top4;                   // n_top rounded up to a multiple of four (the row stride of level-L logits)
  int refine_soft_lds;          // softmax refinement workgroup: kept coarse regions + candidate list
  uint64_t band_off[kMaxLevels];  // byte offset of A_j inside the pyramid buffer, when stored
  int att_t_words;              // words of the attended-set list (T) region
  int attend_lds;               // T list + K/V chunk buffers
  // level-0 positions per thread of the refinement when it shares its launch
  // with the generated positions' attention splits (0: its own launch)
  int fuse_s0;
  // workspace sections (byte offsets)
  uint64_t off_keys, off_sel_top, off_cov, off_lvl, off_sel, off_part_ml, off_part_o, off_logits, total;
};

struct SelectLaunch {
  SelectPlan plan;
  // per layer of a batched call (n_items = 1 otherwise); plan.heads_total =
  // n_items * heads_per_item
  int n_items, heads_per_item;
  const void* q[kMaxItems];
  const float* a_top[kMaxItems];
  const void* k[kMaxItems];
  const void* v[kMaxItems];
  float* out[kMaxItems];
  int32_t* sel_out[kMaxItems];
  const int32_t* gen_idx;
  const int32_t* sel_in;  // attention only: the kept prompt tokens [heads_total][k0] (NULL if k0 == 0)
  int attend_only;        // 1: skip selection, attend over sel_in and gen_idx
  int agg_mean;           // 1: region scores average the query rows (else their maximum)
  int32_t* sel_levels;
  float* score_levels;
  uint8_t* ws;
};

hipError_t launch_select_attend(const SelectLaunch& a, hipStream_t s);

// The input checks of WF_OPT_CHECK (wf_check.hip): the status word sits in
// the first kStatusBytes of every workspace.
constexpr uint64_t kStatusBytes = 256;
struct CheckArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* a_top;     // NULL: no pyramid to check
  int64_t q_bytes, kv_bytes, a_bytes;
  const int32_t* gen_idx;
  int64_t n_gen;
  const int32_t* sel;     // NULL: no selection handed in
  int64_t n_sel;
  int n_tot;              // index entries must lie in [0, n_tot)
  bool bf16;
  uint32_t* status;
};
hipError_t launch_check_clear(uint32_t* status, hipStream_t s);
hipError_t launch_check(const CheckArgs& c, hipStream_t s);

// Waves per SIMD the attention kernel is compiled for: with two query tiles
// its 256-thread workgroup fits 256 registers without spilling, so two
// workgroups share a compute unit; larger workgroups take one each.
constexpr int attend_waves_per_simd(int nqt) { return nqt == 2 ? 2 : 1; }

// Whether a selecting call's refinement may share its launch with the
// generated positions' attention splits (refine_gen_kernel, workgroups of the
// attention's size): at most 256 heads (one round of refinement workgroups)
// and at least two attention workgroups per head fitting the chip at once.
inline bool gen_beside_fits(const SelectPlan* P) {
  const int per_cu = attend_waves_per_simd((P->n_q + 15) / 16);  // attention workgroups per compute unit
  return P->heads_total <= 256 && 256 * per_cu >= 2 * P->heads_total;
}

// Split plan of the attention over T (fills n_att .. cps_g from k0, n_gen,
// chunk, n_q and heads_total).  beside: the generated positions' splits run
// in the refinement's launch, so the prompt part takes about as many splits
// per head as fit the chip (they start together once the selection is out,
// alone in the attention launch) and the generated part splits of as many
// chunks within kMaxSplit.  Otherwise (the attention-only call, and
// selecting calls whose refinement runs apart) both parts share one count
// of chunks per split, about as many splits over all heads as fit the chip
// in one round.
inline void plan_attention_splits(SelectPlan* P, bool beside) {
  const int ch = P->chunk;
  P->n_att = P->k0 + P->n_gen;
  const int nc_p = (P->k0 + ch - 1) / ch, nc_g = (P->n_gen + ch - 1) / ch;
  const int per_cu = attend_waves_per_simd((P->n_q + 15) / 16);  // attention workgroups per compute unit
  const int slots = 256 * per_cu;
  auto cut = [](int chunks, int splits, int& cps, int& n) {  // chunks over at most `splits` splits
    if (chunks == 0) {
      cps = 1;
      n = 0;
      return;
    }
    cps = (chunks + splits - 1) / splits;
    n = (chunks + cps - 1) / cps;
  };
  if (beside) {
    int tp = slots / P->heads_total;
    if (tp > kMaxSplit - (nc_g > 0 ? 1 : 0)) tp = kMaxSplit - (nc_g > 0 ? 1 : 0);
    int n_p, n_g;
    cut(nc_p, tp, P->cps_p, n_p);
    const int tg = (nc_g + P->cps_p - 1) / P->cps_p;
    cut(nc_g, tg < kMaxSplit - n_p ? tg : kMaxSplit - n_p, P->cps_g, n_g);
    P->n_split_p = n_p;
    P->n_split = n_p + n_g;
  } else {
    int target = (slots + P->heads_total - 1) / P->heads_total;
    if (target > kMaxSplit) target = kMaxSplit;
    if (target < 2) target = 2;  // room for a prompt and a generated split
    int cps = (nc_p + nc_g + target - 1) / target;
    if (cps < 1) cps = 1;
    while ((nc_p + cps - 1) / cps + (nc_g + cps - 1) / cps > target) ++cps;
    P->cps_p = P->cps_g = cps;
    P->n_split_p = (nc_p + cps - 1) / cps;
    P->n_split = P->n_split_p + (nc_g + cps - 1) / cps;
  }
  const int cps_max = P->cps_p > P->cps_g ? P->cps_p : P->cps_g;
  P->att_t_words = (cps_max * ch + 3) & ~3;  // one split's part of T
}
// Both branches keep n_split <= kMaxSplit: the merge folds at most that many.
inline bool attention_plan_ok(const SelectPlan* P) { return P->n_split >= 1 && P->n_split <= kMaxSplit; }

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
