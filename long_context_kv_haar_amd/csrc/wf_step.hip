// WaveFilter per-denoising-step kernels for gfx950 (MI355X).  One call is a
// chain of launches on the caller's stream:
//
//   coarse_*_kernel   s_L[n] = max_i (or mean_i) q_i . A_L[n] / sqrt(d) on
//                     MFMA (Figure 2 (c))
//   coarse_topk_kernel
//                     the coarse Top-K, one workgroup per head, for large
//                     coarse levels (n_L > 1 024) or L = 0; otherwise every
//                     cover workgroup computes it for itself
//   cover_*_kernel    the coarse Top-K (Figure 2 (c)), then q_i . k_t for
//                     every token the kept regions cover, on MFMA, summed in
//                     registers into the scores of all their sub-regions at
//                     levels 0 .. L-1 (A_j by linearity from the token dot
//                     products; from the stored bands for a longer basis)
//   refine_sel_kernel the recursive refinement (Figure 2 (d)), one workgroup
//                     of 1 024 threads per head, the coverage scores in
//                     registers (refine_lists_kernel beyond 8 192 covered
//                     positions); writes the kept prompt tokens
//   attend_kernel     split-K online-softmax attention over the kept prompt
//                     tokens plus the generated positions (eq. 3 restricted
//                     to that set); also serves a selection handed in
//   combine_kernel    log-sum-exp merge of the split partials into O
//
// Citations are to WaveFilter (arXiv 2606.00724).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "wf_device.h"
#include "wf_internal.h"
#include "wf_select.h"

static_assert(wf::kRefineThreads == wf::kRefineThreadsHost, "one refinement workgroup size");

namespace wf {

struct StepArgs {
  // Per layer (item) of a batched call: the heads of the n_items layers are
  // stacked, head = item * heads_per_item + its index inside the layer.
  const void* q[kMaxItems];
  const float* a_top[kMaxItems];
  const void* k[kMaxItems];
  const void* v[kMaxItems];
  float* out[kMaxItems];
  int32_t* sel_out[kMaxItems];
  int n_items, heads_per_item;
  const int32_t* gen_idx;
  const int32_t* sel_in;  // the kept prompt tokens [heads_total][k0] the attention reads (NULL if k0 == 0)
  int32_t* sel_ws;        // where the selection writes them [heads_total][k0]
  int32_t* sel_levels;
  float* score_levels;
  uint32_t* keys_top;    // [heads_total][n_top]
  int32_t* sel_top;      // [heads_total][k_top]
  float* cov;            // [heads_total][cov_len]
  uint32_t* lvl_mm;      // [heads_total][cover waves][kMaxLevels][2]: order keys of each level's least and
                         // greatest score over the positions of one coverage wave
  float* part_ml;        // [heads_total][n_split][n_q][2]: (m, l) of each split's partial state
  float* part_o;         // [heads_total][n_split][n_q][d]
  int heads_total, n_q, n_top, n_prompt, n_tot, n_gen, levels;
  int k_top, k0, sum_k;
  int64_t covered, cov_len;
  int64_t cov_off[kMaxLevels];
  int budgets[kMaxLevels + 1];
  int n_att, n_split, n_split_p, cps_p, cps_g, att_t_words;
  int topk_s;             // coarse keys per thread of the in-register coarse Top-K (0: the general path)
  int coarse_keys_in_lds; // general path: keys staged in LDS
  int refine_s0;          // level-0 positions per thread of the in-register refinement (0: refine_lists_kernel)
  int refine_cov_in_lds, refine_nmax, refine_kmax;  // refine_lists_kernel
  float inv_sqrt_d;
  float inv_nq;  // 1 / n_q, for the mean over query rows
  int stored_bands;                    // score levels 1 .. L-1 from stored A_j (longer bases)
  // softmax-probability scores (0: off, 1: maximum, 2: mean over the rows):
  // every row's scaled logits per head, level L [n_q][n_top4], then level j
  // [n_q][padded level length] at n_q * n_top4 + n_q * cov_off[j]
  int soft, n_top4;
  float* logits;
  const float* band_a[kMaxLevels];     // A_j [heads_total][n_prompt >> j][d], when stored
};

// The layer of a head and the head's index inside that layer.
struct HeadRef {
  int item;
  int64_t local;
};
__device__ __forceinline__ HeadRef head_ref(int n_items, int heads_per_item, int head) {
  const int item = n_items == 1 ? 0 : head / heads_per_item;
  return {item, (int64_t)(head - item * heads_per_item)};
}
__device__ __forceinline__ HeadRef head_ref(const StepArgs& a, int head) {
  return head_ref(a.n_items, a.heads_per_item, head);
}

// Leading kernel arguments.  The first 14 dwords of a kernel's arguments are
// placed in scalar registers before its waves start (kernarg preloading), so
// what a stage needs for its first loads goes there: the loads then wait for
// no round trip to the argument segment, and on a single-layer call not for
// the layer's pointers either.  Each stage states what p[] and i[] hold; the
// same values are in StepArgs for everything else.
struct Lead {
  const void* p[3];
  int i[8];
};
#define WF_LEAD_PARAMS                                                                                      \
  const void *lead_p0, const void *lead_p1, const void *lead_p2, int lead_i0, int lead_i1, int lead_i2,     \
      int lead_i3, int lead_i4, int lead_i5, int lead_i6, int lead_i7
#define WF_LEAD \
  (Lead{{lead_p0, lead_p1, lead_p2}, {lead_i0, lead_i1, lead_i2, lead_i3, lead_i4, lead_i5, lead_i6, lead_i7}})

// What the cover stage's first loads (the coarse keys) need.
struct CoverLead {
  const uint32_t* keys;  // [heads_total][n_top]
  int n_top, k_top, topk_s, levels, soft, n_items, heads_per_item;
  __host__ __device__ static CoverLead of(const Lead& l) {
    return {static_cast<const uint32_t*>(l.p[0]), l.i[0], l.i[1], l.i[2], l.i[3], l.i[4], l.i[5], l.i[6]};
  }
  __host__ __device__ Lead lead() const {
    return {{keys, nullptr, nullptr}, {n_top, k_top, topk_s, levels, soft, n_items, heads_per_item, 0}};
  }
};
// What the refinement's first loads (coverage scores, level ranges, kept
// coarse regions) need; the level offsets inside a head's scores follow
// from `covered`.
struct RefineLead {
  const float* cov;       // [heads_total][cov_len]
  const int32_t* sel_top; // [heads_total][k_top]
  const uint32_t* lvl;    // [heads_total][cover waves][kMaxLevels][2]
  int covered, levels, k_top, cov_len, n_top, heads_total;
  __host__ __device__ static RefineLead of(const Lead& l) {
    return {static_cast<const float*>(l.p[0]), static_cast<const int32_t*>(l.p[1]),
            static_cast<const uint32_t*>(l.p[2]), l.i[0], l.i[1], l.i[2], l.i[3], l.i[4], l.i[5]};
  }
  __host__ __device__ Lead lead() const {
    return {{cov, sel_top, lvl}, {covered, levels, k_top, cov_len, n_top, heads_total, 0, 0}};
  }
};
// What the attention's first loads (its part of the attended-set list) need.
struct AttendLead {
  const int32_t* sel_in;   // kept prompt tokens [heads_total][k0]
  const int32_t* gen_idx;  // [n_gen]
  int n_split_p, cps_p, cps_g, k0, n_att, n_tot, n_items, heads_per_item;
  __host__ __device__ static AttendLead of(const Lead& l) {
    return {static_cast<const int32_t*>(l.p[0]), static_cast<const int32_t*>(l.p[1]), l.i[0], l.i[1], l.i[2], l.i[3],
            l.i[4], l.i[5], l.i[6], l.i[7]};
  }
  __host__ __device__ Lead lead() const {
    return {{sel_in, gen_idx, nullptr}, {n_split_p, cps_p, cps_g, k0, n_att, n_tot, n_items, heads_per_item}};
  }
};
// What the split merge's loads need.
struct CombineLead {
  const float* part_ml;
  const float* part_o;
  int n_q, heads_total, n_split;
  __host__ __device__ static CombineLead of(const Lead& l) {
    return {static_cast<const float*>(l.p[0]), static_cast<const float*>(l.p[1]), l.i[0], l.i[1], l.i[2]};
  }
  __host__ __device__ Lead lead() const {
    return {{part_ml, part_o, nullptr}, {n_q, heads_total, n_split, 0, 0, 0, 0, 0}};
  }
};

// Max across the 16 lanes of a row; every lane of the row ends with it.
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_f<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_f<0x141>(x));  // row_half_mirror
  x = fmaxf(x, dpp_f<0x140>(x));  // row_mirror
  return x;
}

// Max over the 16 lanes of a row of each of M values per lane (M = 1, 2, 4,
// 8 or 16), left scattered over the row: value k ends in the lanes whose row
// index, shifted right by log2(16 / M), is k.  Step s pairs every lane with
// the lane its row index maps to under row mirror, half-row mirror, and the
// two quad swaps (s = 0..3): each pairing flips bit 3 - s of the index and only
// lower bits, so a pair always holds the same values, and while more than one
// value is left, that bit picks the half a lane keeps (the partner keeps the
// other).  M / 2 + M / 4 + ... + 4 - log2(M) DPP steps instead of 4 per value.
template <int S> struct ScatterDpp;
template <> struct ScatterDpp<0> { static constexpr int CTRL = 0x140; };  // row_mirror
template <> struct ScatterDpp<1> { static constexpr int CTRL = 0x141; };  // row_half_mirror
template <> struct ScatterDpp<2> { static constexpr int CTRL = 0x4E; };   // quad_perm [2,3,0,1]
template <> struct ScatterDpp<3> { static constexpr int CTRL = 0xB1; };   // quad_perm [1,0,3,2]
// SUM: the sum over the row instead of the maximum (in another order than a
// per-value reduction, so it may differ from one in the last bit).
template <bool SUM, int M, int S = 0>
__device__ __forceinline__ float row_scatter(const float (&v)[M], int l16) {
  if constexpr (S == 4) {
    static_assert(M == 1, "16 lanes hold at most 16 values");
    return v[0];
  } else if constexpr (M == 1) {
    const float o = dpp_f<ScatterDpp<S>::CTRL>(v[0]);
    const float w[1] = {SUM ? v[0] + o : fmaxf(v[0], o)};
    return row_scatter<SUM, 1, S + 1>(w, l16);
  } else {
    const bool up = (l16 >> (3 - S)) & 1;
    float h[M / 2];
#pragma unroll
    for (int k = 0; k < M / 2; ++k) {
      const float keep = up ? v[M / 2 + k] : v[k];
      const float give = up ? v[k] : v[M / 2 + k];
      const float o = dpp_f<ScatterDpp<S>::CTRL>(give);
      h[k] = SUM ? keep + o : fmaxf(keep, o);
    }
    return row_scatter<SUM, M / 2, S + 1>(h, l16);
  }
}
template <int M>
__device__ __forceinline__ float row_max_scatter(const float (&v)[M], int l16) {
  return row_scatter<false, M>(v, l16);
}

// The same for unsigned keys.
template <int M, int S = 0>
__device__ __forceinline__ uint32_t row_max_scatter_u(const uint32_t (&v)[M], int l16) {
  if constexpr (S == 4) {
    static_assert(M == 1, "16 lanes hold at most 16 values");
    return v[0];
  } else if constexpr (M == 1) {
    const uint32_t w[1] = {max(v[0], dpp_u<ScatterDpp<S>::CTRL>(v[0]))};
    return row_max_scatter_u<1, S + 1>(w, l16);
  } else {
    const bool up = (l16 >> (3 - S)) & 1;
    uint32_t h[M / 2];
#pragma unroll
    for (int k = 0; k < M / 2; ++k) {
      const uint32_t keep = up ? v[M / 2 + k] : v[k];
      const uint32_t give = up ? v[k] : v[M / 2 + k];
      h[k] = max(keep, dpp_u<ScatterDpp<S>::CTRL>(give));
    }
    return row_max_scatter_u<M / 2, S + 1>(h, l16);
  }
}

// How the query rows of a block combine into a region score: the maximum
// (rows past n_q are set to -inf) or the mean (rows past n_q hold 0, the sum
// is scaled by 1/n_q).  comb() folds two rows a lane holds, row() the 16 rows
// spread over the lanes of a 16-lane row.
template <bool MEAN> struct QueryAgg;
template <> struct QueryAgg<false> {
  __device__ __forceinline__ static float comb(float x, float y) { return fmaxf(x, y); }
  __device__ __forceinline__ static float row(float x) { return row_max16(x); }
};
template <> struct QueryAgg<true> {
  __device__ __forceinline__ static float comb(float x, float y) { return x + y; }
  __device__ __forceinline__ static float row(float x) {
#pragma unroll
    for (int lvl = 1; lvl <= 4; ++lvl) x = group_sum_step(x, lvl);
    return x;
  }
};

// The query block of one head staged once per workgroup in LDS (rows padded
// like the attention's K rows, so fragment reads are free of bank conflicts),
// instead of every wave reading all of Q from memory.
template <typename T> struct QueryLds;
template <> struct QueryLds<bf16_t> { static constexpr int PAD = 8; };
template <> struct QueryLds<float> { static constexpr int PAD = 4; };

// Query rows staged in LDS with every load of a thread issued (clamped in
// bounds) before the first LDS store: one round trip for the block instead
// of one per vector.  issue() loads a thread's vectors into registers and
// store() writes them to LDS, so that other work can run in between while
// the loads are in flight.
template <typename T, int D, int NT, int RT>
struct QueryStage {
  static constexpr int VE = 16 / sizeof(T), NV = D / VE, QS = D + QueryLds<T>::PAD;
  static constexpr int IT = (16 * RT * NV + NT - 1) / NT;  // n_q <= 16 RT
  u32x4 v[IT];
  __device__ __forceinline__ void issue(const T* qh, int n_q) {
    const int total = n_q * NV;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int e = min((int)threadIdx.x + i * NT, total - 1);
      const int row = e / NV, cv = e - row * NV;
      v[i] = *reinterpret_cast<const u32x4*>(qh + (int64_t)row * D + cv * VE);
    }
  }
  __device__ __forceinline__ void store(int n_q, T* qs) const {
    const int total = n_q * NV;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int e = (int)threadIdx.x + i * NT;
      const int row = e / NV, cv = e - row * NV;
      if (e < total) *reinterpret_cast<u32x4*>(qs + row * QS + cv * VE) = v[i];
    }
  }
};

// Query fragments as the B operand from the staged rows: lane (l16, g)
// supplies query row 16 qt + l16; zero beyond n_q.
template <typename T, int D, int RT>
__device__ __forceinline__ void load_query_frags(const T* qs, int n_q, int l16, int g, Frag<T, D> (&qf)[RT]) {
  constexpr int QS = D + QueryLds<T>::PAD;
#pragma unroll
  for (int qt = 0; qt < RT; ++qt) {
    const int row = 16 * qt + l16;
    if (row < n_q) qf[qt].load(qs + row * QS, g);
    else qf[qt].zero();
  }
}

// LDS scratch shared by the general Top-K variants a workgroup of NT threads
// uses (large coarse sets and the list-based refinement): the strided
// register Top-K on min(NT, 256) threads (up to 32 slots) and the
// LDS-resident one.
constexpr size_t cmax(size_t x, size_t y) { return x > y ? x : y; }
template <int NT> struct TopKRaw {
  static constexpr int ACT0 = NT < 256 ? NT : 256;
  static constexpr size_t BYTES = cmax(sizeof(TopKFastShared<NT>), sizeof(TopKSel<ACT0, 32>));
};

// ---------------------------------------------------------------------------
// Coarse Top-K (Figure 2 (c)) of one head: the k_L best regions from the
// order keys of s_L, handed to emit(o, i, s) in ascending order.  In
// registers with S keys per thread (n_L <= 256 S), else by the general
// Top-K with the keys in LDS (up to kMaxCoarseLds) or read from memory.
// ---------------------------------------------------------------------------
template <int S, class Emit, class Pre>
__device__ __forceinline__ void coarse_topk_sel(const uint32_t* keys, int n, int k, SelShared<kSelThreads>& sh,
                                                Emit emit, Pre pre) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int pos0 = t * S;
  uint32_t kv[S];
#pragma unroll
  for (int i = 0; i < S; ++i) kv[i] = keys[min(pos0 + i, n - 1)];
  // the caller's own loads go after the keys, which the selection waits for
  // first, and the selection state is cleared while they are in flight
  __builtin_amdgcn_sched_barrier(0);
  pre();
  sel_init(sh);
  float sc[S];
  uint32_t valid = 0u, mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const bool in = pos0 + i < n;
    const uint32_t key = kv[i];
    sc[i] = key_to_f32(key);
    valid |= in ? (1u << i) : 0u;
    mn = in ? min(mn, key) : mn;
    mx = in ? max(mx, key) : mx;
  }
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  if (lane == 0) {
    sh.wmn[w] = mn;
    sh.wmx[w] = mx;
  }
  __syncthreads();
  mn = 0xFFFFFFFFu;
  mx = 0u;
#pragma unroll
  for (int i = 0; i < kSelThreads / 64; ++i) {
    mn = min(mn, sh.wmn[i]);
    mx = max(mx, sh.wmx[i]);
  }
  SelCursor cur;
  const uint32_t kept = select_level<kSelThreads, S>(sc, valid, valid, pos0, k, key_to_f32(mn), key_to_f32(mx), sh, cur);
  int o = block_excl_scan(__popc(kept), sh, 1);
#pragma unroll
  for (int i = 0; i < S; ++i)
    if ((kept >> i) & 1u) {
      if (o < k) emit(o, pos0 + i, sc[i]);  // exactly k are kept; the bound guards the buffers
      ++o;
    }
}

// The in-register coarse Top-K for topk_s in {1, 2, 4} (what a cover
// workgroup runs), or with LARGE also {8, 16, 32} and the general path (the
// Top-K's own launch).  pre() issues the caller's loads that are not needed
// before the Top-K ends: after the keys' loads where they are in registers,
// else first.
template <bool LARGE, class Emit, class Pre>
__device__ __forceinline__ void coarse_topk_run(const StepArgs& a, const CoverLead& cl, int head, unsigned char* raw,
                                                uint32_t* keys_l, Emit emit, Pre pre) {
  const uint32_t* keys = cl.keys + (int64_t)head * cl.n_top;
  const int n = cl.n_top, k = cl.k_top;
  SelShared<kSelThreads>& sh = *reinterpret_cast<SelShared<kSelThreads>*>(raw);
  switch (cl.topk_s) {
    case 1: coarse_topk_sel<1>(keys, n, k, sh, emit, pre); return;
    case 2: coarse_topk_sel<2>(keys, n, k, sh, emit, pre); return;
    case 4: coarse_topk_sel<4>(keys, n, k, sh, emit, pre); return;
    default: break;
  }
  if constexpr (LARGE) {
    switch (cl.topk_s) {
      case 8: coarse_topk_sel<8>(keys, n, k, sh, emit, pre); return;
      case 16: coarse_topk_sel<16>(keys, n, k, sh, emit, pre); return;
      case 32: coarse_topk_sel<32>(keys, n, k, sh, emit, pre); return;
      default: break;
    }
    pre();
    auto& fs = *reinterpret_cast<TopKFastShared<kSelThreads>*>(raw);
    auto out = [&](int o, int i) {
      if (o < k) emit(o, i, key_to_f32(keys[i]));
    };
    if (a.coarse_keys_in_lds) {
      for (int i = threadIdx.x; i < n; i += kSelThreads) keys_l[i] = keys[i];
      __syncthreads();
      topk_fast<kSelThreads>([&](int i) { return keys_l[i]; }, n, k, fs, out);
    } else {
      topk_fast<kSelThreads>([&](int i) { return keys[i]; }, n, k, fs, out);
    }
  }
}

// Where the coarse Top-K runs: in every cover workgroup of the head (each
// computes the same set; n_L <= 1 024 and L > 0), else in a launch of its
// own, one workgroup per head.
__host__ __device__ __forceinline__ bool topk_in_cover(const CoverLead& cl) {
  return cl.topk_s >= 1 && cl.topk_s <= 4 && cl.levels > 0 && cl.soft == 0;
}
__host__ __device__ __forceinline__ CoverLead cover_lead(const StepArgs& a) {
  return {a.keys_top, a.n_top, a.k_top, a.topk_s, a.levels, a.soft, a.n_items, a.heads_per_item};
}
__host__ __device__ __forceinline__ AttendLead attend_lead(const StepArgs& a) {
  return {a.sel_in, a.gen_idx, a.n_split_p, a.cps_p, a.cps_g, a.k0, a.n_att, a.n_tot, a.n_items, a.heads_per_item};
}
__host__ __device__ __forceinline__ RefineLead refine_lead(const StepArgs& a) {
  return {a.cov, a.sel_top, a.lvl_mm, (int)a.covered, a.levels, a.k_top, (int)a.cov_len, a.n_top, a.heads_total};
}
__host__ __device__ __forceinline__ CombineLead combine_lead(const StepArgs& a) {
  return {a.part_ml, a.part_o, a.n_q, a.heads_total, a.n_split};
}

// The softmax scores' logits of one head (level L first).
__device__ __forceinline__ float* head_logits(const StepArgs& a, int head) {
  return a.logits + (int64_t)head * a.n_q * (a.n_top4 + a.cov_len);
}

// The coarse Top-K's outputs beside emit_sel(o, i): the kept regions
// (workgroup `writer` of the head only), the level-L sinks, and for L = 0
// the kept tokens.
template <class F>
__device__ __forceinline__ auto coarse_emitter(const StepArgs& a, int head, const HeadRef& hr, bool writer,
                                               F emit_sel) {
  const bool report = writer && (a.sel_levels || a.score_levels);
  int32_t* sel_g = writer ? a.sel_top + (int64_t)head * a.k_top : nullptr;
  int32_t* dbg_sel = report && a.sel_levels ? a.sel_levels + (int64_t)head * a.sum_k : nullptr;
  float* dbg_score = report && a.score_levels ? a.score_levels + (int64_t)head * a.sum_k : nullptr;
  // with L = 0 the coarse level is the tokens themselves: these are the kept tokens
  int32_t* tsel = (writer && a.levels == 0) ? a.sel_ws + (int64_t)head * a.k0 : nullptr;
  int32_t* tout = (writer && a.levels == 0 && a.sel_out[hr.item]) ? a.sel_out[hr.item] + hr.local * a.k0 : nullptr;
  return [=](int o, int i, float sc) {
    emit_sel(o, i);
    if (sel_g) sel_g[o] = i;
    if (dbg_sel) dbg_sel[o] = i;
    if (dbg_score) dbg_score[o] = a.soft ? expf(sc) : sc;  // softmax scores are ranked as log-probabilities
    if (tsel) {
      tsel[o] = i;
      if (tout) tout[o] = i;
    }
  };
}

// Selection scratch of a workgroup that runs the general coarse Top-K.
constexpr size_t kSelRawBytes = cmax(sizeof(SelShared<kSelThreads>), TopKRaw<kSelThreads>::BYTES);

// ---------------------------------------------------------------------------
// Coarse scores.  Wave w of block x scores level-L regions
// n = 64 x + 16 w + [0, 16): tile = A_L rows (A operand) x Q^T (B operand),
// so lane (query 16 qt + l16, g) holds regions 16 w + 4 g + r.  For bfloat16
// inputs the float32 coefficients are split into bf16 hi + lo parts, both
// multiplied exactly, accumulated in float32.  Max over queries: in registers
// over qt, then across the 16 lanes of a row.
// ---------------------------------------------------------------------------
template <typename T, int D, int RT, bool MEAN, bool ONE>
__device__ __forceinline__ void coarse_stage(const StepArgs& a, const Lead& ld) {
  using AG = QueryAgg<MEAN>;
  __shared__ __align__(16) T qs[16 * RT * (D + QueryLds<T>::PAD)];
  const int head = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  // leading arguments: the layer's A_L and Q (single-layer calls), n_top, n_q
  const int n_top = ld.i[0], n_q = ld.i[1];

  const int n = blockIdx.x * 64 + w * 16 + l16;  // region supplied by this lane (A operand)
  const bool valid = n < n_top;
  const HeadRef hr = ONE ? HeadRef{0, head} : head_ref(a, head);
  const float* atop = ONE ? static_cast<const float*>(ld.p[0]) : a.a_top[hr.item];
  const T* qh = (ONE ? static_cast<const T*>(ld.p[1]) : reinterpret_cast<const T*>(a.q[hr.item])) + hr.local * n_q * D;
  const float* arow = atop + (hr.local * n_top + (valid ? n : 0)) * D;
  f32x4 acc[RT];
#pragma unroll
  for (int qt = 0; qt < RT; ++qt) acc[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the query block is requested first: it goes to LDS while the coefficient
  // rows are still in flight
  QueryStage<T, D, 256, RT> qstage;
  qstage.issue(qh, n_q);
  if constexpr (sizeof(T) == 2) {
    constexpr int STEPS = D / 32;
    // step s of lane group g: coefficients [32 s + 8 g, 32 s + 8 g + 8), as Frag<bf16_t>
    const float4* p = reinterpret_cast<const float4*>(arow);
    float4 x[2 * STEPS];
    // unconditional loads (arow is row 0 for an absent region): a load under
    // a condition becomes a branch, and the wait for the query block at its
    // join would then take the rows too
#pragma unroll
    for (int i = 0; i < 2 * STEPS; ++i) x[i] = p[8 * (i >> 1) + 2 * g + (i & 1)];
    qstage.store(n_q, qs);
    __syncthreads();
    Frag<T, D> qf[RT];
    load_query_frags<T, D, RT>(qs, n_q, l16, g, qf);
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      u32x4 hi, lo;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float4 v = valid ? x[2 * s + h] : make_float4(0.f, 0.f, 0.f, 0.f);
        { const Bf16Split t = split_pk_bf16(v.x, v.y); hi[2 * h] = t.hi; lo[2 * h] = t.lo; }
        { const Bf16Split t = split_pk_bf16(v.z, v.w); hi[2 * h + 1] = t.hi; lo[2 * h + 1] = t.lo; }
      }
#pragma unroll
      for (int qt = 0; qt < RT; ++qt) {
        acc[qt] = mma_bf16(hi, qf[qt].v[s], acc[qt]);
        acc[qt] = mma_bf16(lo, qf[qt].v[s], acc[qt]);
      }
    }
  } else {
    Frag<float, D> b;
    b.load(arow, g);  // unconditional, as above
    if (!valid) b.zero();
    qstage.store(n_q, qs);
    __syncthreads();
    Frag<T, D> qf[RT];
    load_query_frags<T, D, RT>(qs, n_q, l16, g, qf);
#pragma unroll
    for (int qt = 0; qt < RT; ++qt) acc[qt] = mma_tile<D>(b, qf[qt], acc[qt]);
  }
  if (a.soft) {  // uniform: every query row's scaled logits, for the softmax scores
    float* lg = head_logits(a, head);
    const int n0 = blockIdx.x * 64 + w * 16 + 4 * g;
#pragma unroll
    for (int qt = 0; qt < RT; ++qt) {
      const int query = 16 * qt + l16;
      if (query < n_q)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n0 + r < n_top) lg[(int64_t)query * a.n_top4 + n0 + r] = acc[qt][r] * a.inv_sqrt_d;
    }
    return;
  }
  float m[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float x = acc[0][r];  // query tile 0 always holds a valid row
#pragma unroll
    for (int qt = 1; qt < RT; ++qt)
      if (MEAN || 16 * qt + l16 < n_q) x = AG::comb(x, acc[qt][r]);  // absent rows: 0 from zero query rows
    if (!MEAN && l16 >= n_q) x = -INFINITY;
    m[r] = x;
  }
  const float sc = MEAN ? a.inv_sqrt_d * a.inv_nq : a.inv_sqrt_d;
  uint32_t* keys = a.keys_top + (int64_t)head * n_top;
  const int n0 = blockIdx.x * 64 + w * 16 + 4 * g;  // first region of this row
  // the four regions' row maxima (or sums) scattered over the row: region
  // n0 + r ends in lanes l16 = 4 r .. 4 r + 3
  const int r = l16 >> 2;
  const float x = row_scatter<MEAN, 4>(m, l16);
  if ((l16 & 3) == 0 && n0 + r < n_top) keys[n0 + r] = order_key(x * sc);
}

template <typename T, int D, int RT, bool ONE>
__global__ __launch_bounds__(256) void coarse_max_kernel(WF_LEAD_PARAMS, StepArgs a) {
  coarse_stage<T, D, RT, false, ONE>(a, WF_LEAD);
}
template <typename T, int D, int RT, bool ONE>
__global__ __launch_bounds__(256) void coarse_mean_kernel(WF_LEAD_PARAMS, StepArgs a) {
  coarse_stage<T, D, RT, true, ONE>(a, WF_LEAD);
}

// One 16-row tile of float32 coefficient rows (A operand; lane row l16,
// k-slice g) against the staged query tiles (B operands): bfloat16 queries
// take the rows as exact hi + lo bf16 parts, float32 queries the fp32 MFMA.
// f32_row_load fetches a lane's part of its row (D/16 float4 either way);
// f32_rows_mma multiplies it, so a caller can put several tiles' loads in
// flight before the first multiply.
template <typename T, int D>
__device__ __forceinline__ void f32_row_load(const float* arow, int g, float4 (&x)[D / 16]) {
  const float4* p = reinterpret_cast<const float4*>(arow);
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    if constexpr (sizeof(T) == 2) x[i] = p[8 * (i >> 1) + 2 * g + (i & 1)];  // step i/2, half i%2: [32 s + 8 g, +8)
    else x[i] = p[g * (D / 16) + i];                                         // the quarter [g D/4, (g+1) D/4)
  }
}

template <typename T, int D, int RT>
__device__ __forceinline__ void f32_rows_mma(const float4 (&x)[D / 16], const Frag<T, D> (&qf)[RT],
                                             f32x4 (&acc)[RT]) {
#pragma unroll
  for (int qt = 0; qt < RT; ++qt) acc[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (sizeof(T) == 2) {
    constexpr int STEPS = D / 32;
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      u32x4 hi, lo;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float4 v = x[2 * s + h];
        { const Bf16Split t = split_pk_bf16(v.x, v.y); hi[2 * h] = t.hi; lo[2 * h] = t.lo; }
        { const Bf16Split t = split_pk_bf16(v.z, v.w); hi[2 * h + 1] = t.hi; lo[2 * h + 1] = t.lo; }
      }
#pragma unroll
      for (int qt = 0; qt < RT; ++qt) {
        acc[qt] = mma_bf16(hi, qf[qt].v[s], acc[qt]);
        acc[qt] = mma_bf16(lo, qf[qt].v[s], acc[qt]);
      }
    }
  } else {
    Frag<float, D> b;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      b.v[4 * i] = x[i].x;
      b.v[4 * i + 1] = x[i].y;
      b.v[4 * i + 2] = x[i].z;
      b.v[4 * i + 3] = x[i].w;
    }
#pragma unroll
    for (int qt = 0; qt < RT; ++qt) acc[qt] = mma_tile<D>(b, qf[qt], acc[qt]);
  }
}

// Coverage scores from stored approximation bands, for a longer basis whose
// level-j coefficient is not the scaled sum of its own 2^j tokens: wave
// `wave_base / 64` scores positions [wave_base, wave_base + 64) of every
// level j < L (level 0 from the key rows, the others from A_j) against the
// query block, writes them, and publishes each level's score range of its
// positions (a neutral range where it has none).  The level's four 16-row
// tiles go in pairs, both tiles' rows requested before either is multiplied;
// rows past the level's end repeat its last row (in bounds) and are never
// written.
template <typename T, int D, int RT, bool MEAN>
__device__ __forceinline__ void cover_from_bands(const StepArgs& a, int head, const int* sel_l, const Frag<T, D> (&qf)[RT],
                                                 int64_t wave_base, int lane, int g, int l16) {
  using AG = QueryAgg<MEAN>;
  const int L = a.levels;
  const float sc = MEAN ? a.inv_sqrt_d * a.inv_nq : a.inv_sqrt_d;
  float* cov = a.cov + (int64_t)head * a.cov_len;
  const int nwav = (int)((a.covered + 63) >> 6);
  uint32_t* lvl = a.lvl_mm + ((int64_t)head * nwav + (wave_base >> 6)) * 2 * kMaxLevels;
  const HeadRef hr = head_ref(a, head);
  const T* kh = reinterpret_cast<const T*>(a.k[hr.item]) + hr.local * a.n_tot * D;
  for (int j = 0; j < L; ++j) {
    const int64_t nj = a.covered >> j;
    const int sh = L - j;
    uint32_t rmn = 0xFFFFFFFFu, rmx = 0u;
    if (wave_base < nj) {  // wave-uniform: this wave has positions at level j
#pragma unroll
      for (int tp = 0; tp < 2; ++tp) {  // tile pairs: both tiles' rows in flight together
        int64_t idx[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          int64_t p = wave_base + 16 * (2 * tp + u) + l16;  // the A-operand row of this lane
          p = p < nj ? p : nj - 1;
          idx[u] = ((int64_t)clampi(sel_l[p >> sh], 0, a.n_top - 1) << sh) + (p & ((1 << sh) - 1));
        }
        f32x4 acc[2][RT];
        if (j == 0) {
          Frag<T, D> kf[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) kf[u].load(kh + idx[u] * D, g);
          __builtin_amdgcn_sched_barrier(0);  // both row loads ahead of the math
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int qt = 0; qt < RT; ++qt) acc[u][qt] = mma_tile<D>(kf[u], qf[qt], f32x4{0.f, 0.f, 0.f, 0.f});
        } else {
          const float* band = a.band_a[j] + (int64_t)head * (a.n_prompt >> j) * D;
          float4 xr[2][D / 16];
#pragma unroll
          for (int u = 0; u < 2; ++u) f32_row_load<T, D>(band + idx[u] * D, g, xr[u]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int u = 0; u < 2; ++u) f32_rows_mma<T, D, RT>(xr[u], qf, acc[u]);
        }
        // the pair's eight positions (4 u + r) in one scattered row reduction:
        // position 16 (2 tp + u) + 4 g + r ends in lanes l16 = 2 (4 u + r), + 1
        float v[8];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float x = acc[u][0][r];
#pragma unroll
            for (int qt = 1; qt < RT; ++qt)
              if (MEAN || 16 * qt + l16 < a.n_q) x = AG::comb(x, acc[u][qt][r]);
            if (!MEAN && l16 >= a.n_q) x = -INFINITY;
            v[4 * u + r] = x;
          }
        const float m = row_scatter<MEAN, 8>(v, l16) * sc;
        const int e = l16 >> 1, u = e >> 2, r = e & 3;
        const int64_t pr = wave_base + 16 * (2 * tp + u) + 4 * g + r;
        const bool in = pr < nj;
        if (in && (l16 & 1) == 0) cov[a.cov_off[j] + pr] = m;
        const uint32_t k = order_key(m);
        rmn = in ? min(rmn, k) : rmn;
        rmx = in ? max(rmx, k) : rmx;
      }
    }
    rmn = wave_min_u32(rmn);
    rmx = wave_max_u32(rmx);
    if (lane == 0) {
      lvl[2 * j] = rmn;
      lvl[2 * j + 1] = rmx;
    }
  }
}

// The Haar coverage scores of one wave with the maximum (or the mean) over
// the query rows (cover_haar below sets up s, the per-query token logits of
// the wave's four tiles): each level sums its blocks in registers or across
// lane groups, then combines the 16 query rows of every block with one
// scattered row reduction, so that every lane ends with one block's score (or a copy of
// it) and the stores and the score range take one value per lane.  Level j's
// value for block k of the wave sits in the lanes of row g with l16 >> (j < 3
// ? j : 2) == the block's index inside the row's tiles, as worked out below.
template <bool MEAN, int RT>
__device__ __forceinline__ void cover_levels(const StepArgs& a, f32x4 (&s)[4][RT], float* cov, float isd,
                                             uint32_t* lvl, int64_t wave_base, int lane, int g, int l16, int jmax) {
  const int64_t covered = a.covered;
  // each level's score range over the wave, as order keys: the greatest in
  // kmx, the least complemented in kmn (so that both reduce by maximum)
  uint32_t kmn[kMaxLevels], kmx[kMaxLevels];
#pragma unroll
  for (int j = 0; j < kMaxLevels; ++j) kmn[j] = kmx[j] = 0u;
  auto track = [&](int j, bool in, float v) {
    const uint32_t k = order_key(v);
    kmx[j] = in ? k : 0u;
    kmn[j] = in ? ~k : 0u;
  };
  do {  // the levels; a break skips those past the pyramid's top
    // level 0: value 4 t + r (token 16 t + 4 g + r) ends in lane l16 = 4 t + r
    {
      float v[16];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x = s[t][0][r];
#pragma unroll
          for (int qt = 1; qt < RT; ++qt) x = MEAN ? x + s[t][qt][r] : fmaxf(x, s[t][qt][r]);
          v[4 * t + r] = x;
        }
      const float m = row_scatter<MEAN, 16>(v, l16) * isd;
      const int64_t p = wave_base + 16 * (l16 >> 2) + 4 * g + (l16 & 3);
      const bool in = p < covered;
      if (in) cov[a.cov_off[0] + p] = m;
      track(0, in, m);
    }
    if (jmax <= 1) break;
    // level 1: token pairs (r = 0,1 and 2,3) summed in place into s[t][qt][0]
    // and [2]; value 2 t + h ends in lanes l16 = 4 t + 2 h and 4 t + 2 h + 1
    {
      float v[8];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int qt = 0; qt < RT; ++qt) {
          s[t][qt][0] += s[t][qt][1];
          s[t][qt][2] += s[t][qt][3];
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float x = s[t][0][2 * h];
#pragma unroll
          for (int qt = 1; qt < RT; ++qt) x = MEAN ? x + s[t][qt][2 * h] : fmaxf(x, s[t][qt][2 * h]);
          v[2 * t + h] = x;
        }
      }
      const float m = row_scatter<MEAN, 8>(v, l16) * (isd * 0.70710678118654752440f);
      const int64_t p = wave_base + 16 * (l16 >> 2) + 4 * g + 2 * ((l16 >> 1) & 1);  // first token of the pair
      const bool in = p < covered;
      if (in && (l16 & 1) == 0) cov[a.cov_off[1] + (p >> 1)] = m;
      track(1, in, m);
    }
    if (jmax <= 2) break;
    // level 2: 4-token blocks (one per lane group) into s[t][qt][0]; value t
    // ends in lanes l16 = 4 t .. 4 t + 3
    {
      float v[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int qt = 0; qt < RT; ++qt) s[t][qt][0] += s[t][qt][2];
        float x = s[t][0][0];
#pragma unroll
        for (int qt = 1; qt < RT; ++qt) x = MEAN ? x + s[t][qt][0] : fmaxf(x, s[t][qt][0]);
        v[t] = x;
      }
      const float m = row_scatter<MEAN, 4>(v, l16) * (isd * 0.5f);
      const int64_t p = wave_base + 16 * (l16 >> 2) + 4 * g;
      const bool in = p < covered;
      if (in && (l16 & 3) == 0) cov[a.cov_off[2] + (p >> 2)] = m;
      track(2, in, m);
    }
    if (jmax <= 3) break;
    // level 3: 8-token blocks = lane groups {0,1} and {2,3}; as level 2, with
    // groups g and g ^ 1 holding the same values
    {
      float v[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int qt = 0; qt < RT; ++qt) s[t][qt][0] = sum_xor16(s[t][qt][0]);
        float x = s[t][0][0];
#pragma unroll
        for (int qt = 1; qt < RT; ++qt) x = MEAN ? x + s[t][qt][0] : fmaxf(x, s[t][qt][0]);
        v[t] = x;
      }
      const float m = row_scatter<MEAN, 4>(v, l16) * (isd * 0.35355339059327376220f);
      const int64_t p = wave_base + 16 * (l16 >> 2) + 8 * (g >> 1);
      const bool in = p < covered;
      if (in && (l16 & 3) == 0 && (g & 1) == 0) cov[a.cov_off[3] + (p >> 3)] = m;
      track(3, in, m);
    }
    if (jmax <= 4) break;
    // level 4: 16-token blocks = whole tiles, every lane group the same
    {
      float v[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int qt = 0; qt < RT; ++qt) s[t][qt][0] = sum_xor32(s[t][qt][0]);
        float x = s[t][0][0];
#pragma unroll
        for (int qt = 1; qt < RT; ++qt) x = MEAN ? x + s[t][qt][0] : fmaxf(x, s[t][qt][0]);
        v[t] = x;
      }
      const float m = row_scatter<MEAN, 4>(v, l16) * (isd * 0.25f);
      const int64_t p = wave_base + 16 * (l16 >> 2);
      const bool in = p < covered;
      if (in && (l16 & 3) == 0 && g == 0) cov[a.cov_off[4] + (p >> 4)] = m;
      track(4, in, m);
    }
    if (jmax <= 5) break;
    // level 5: tile pairs, value h ends in lanes l16 = 8 h .. 8 h + 7; level 6:
    // the whole wave
    {
      float v[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float x = s[2 * h][0][0] + s[2 * h + 1][0][0];
#pragma unroll
        for (int qt = 1; qt < RT; ++qt) {
          const float pair = s[2 * h][qt][0] + s[2 * h + 1][qt][0];
          x = MEAN ? x + pair : fmaxf(x, pair);
        }
        v[h] = x;
      }
      float xall = (s[0][0][0] + s[1][0][0]) + (s[2][0][0] + s[3][0][0]);
#pragma unroll
      for (int qt = 1; qt < RT; ++qt) {
        const float all = (s[0][qt][0] + s[1][qt][0]) + (s[2][qt][0] + s[3][qt][0]);
        xall = MEAN ? xall + all : fmaxf(xall, all);
      }
      const float m = row_scatter<MEAN, 2>(v, l16) * (isd * 0.17677669529663688110f);  // 2^{-5/2}
      const int64_t p = wave_base + 32 * (l16 >> 3);
      const bool in = p < covered;
      if (in && (l16 & 7) == 0 && g == 0) cov[a.cov_off[5] + (p >> 5)] = m;
      track(5, in, m);
      if (jmax > 6) {
        const float xw[1] = {xall};
        xall = row_scatter<MEAN, 1>(xw, l16) * (isd * 0.125f);  // 2^{-3}
        if (lane == 0) cov[a.cov_off[6] + (wave_base >> 6)] = xall;
        track(6, lane == 0, xall);
      }
    }
  } while (false);
  // the ranges of all levels in one scattered reduction: value l of the row
  // (l < 8: level l's least key, complemented; l >= 8: level l - 8's greatest)
  // ends in lane l16 = l, then the four rows combine
  uint32_t w[16];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    w[j] = j < kMaxLevels ? kmn[j] : 0u;
    w[8 + j] = j < kMaxLevels ? kmx[j] : 0u;
  }
  uint32_t r = row_max_scatter_u<16>(w, l16);
  r = max(r, lane_xor16(r));
  r = max(r, lane_xor32(r));
  const int j = lane & 7;
  if (lane < 16 && j < jmax) lvl[2 * j + (lane >> 3)] = lane < 8 ? ~r : r;
}

// ---------------------------------------------------------------------------
// Haar coverage scores of one wave.  The kept coarse regions, ascending,
// cover positions p = 0 .. k_L 2^L - 1; position p is token
// sel_L[p >> L] 2^L + (p mod 2^L).  The wave owns positions
// wave_base + [0, 64) as four 16-token tiles t; tile = K rows (A operand) x
// Q^T (B operand), so lane (query 16 qt + l16, g) holds
// S[query][tokens 16 t + 4 g + r].  Sums along the token axis: levels 1 and
// 2 in-lane (r), levels 3 and 4 across lane groups g (xor 16, xor 32),
// levels 5 and 6 across tiles in registers.  The score of a block is the max
// over queries: over qt in registers, then across the 16 lanes of a row.
// Scores are written per level at the block's position p >> j, and so is
// each level's score range over the wave.
// ---------------------------------------------------------------------------
template <typename T, int D, int RT, bool MEAN>
__device__ __forceinline__ void cover_haar(const StepArgs& a, int head, const int* sel_l, const Frag<T, D> (&qf)[RT],
                                           int64_t wave_base, int lane, int g, int l16) {
  using AG = QueryAgg<MEAN>;
  const int L = a.levels;
  const HeadRef hr = head_ref(a, head);
  const T* kh = reinterpret_cast<const T*>(a.k[hr.item]) + hr.local * a.n_tot * D;
  Frag<T, D> kf[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    int64_t p = wave_base + 16 * t + l16;
    p = p < a.covered ? p : a.covered - 1;  // past the end: any covered row, never written out
    const int r = clampi(sel_l[p >> L], 0, a.n_top - 1);
    const int64_t tok = ((int64_t)r << L) + (p & ((1 << L) - 1));
    kf[t].load(kh + tok * D, g);
  }
  // all 16 row loads stay ahead of the math: left to itself the scheduler
  // interleaves them with the MFMAs, three or four in flight at a time, and
  // the gather runs as several serial round trips
  __builtin_amdgcn_sched_barrier(0);
  f32x4 s[4][RT];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int qt = 0; qt < RT; ++qt) s[t][qt] = mma_tile<D>(kf[t], qf[qt], f32x4{0.f, 0.f, 0.f, 0.f});
  // rows of absent queries never win a max (for the mean they hold 0, from
  // zero query rows)
  if (!MEAN)
#pragma unroll
    for (int qt = 0; qt < RT; ++qt)
      if (16 * qt + l16 >= a.n_q)
#pragma unroll
        for (int t = 0; t < 4; ++t) s[t][qt] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};

  float* cov = a.cov + (int64_t)head * a.cov_len;
  const int jmax = L < 7 ? L : 7;  // levels 0 .. jmax-1 are scored here
  const float isd = MEAN ? a.inv_sqrt_d * a.inv_nq : a.inv_sqrt_d;
  const bool writer = (l16 == 0);
  const int64_t tb = wave_base + 4 * g;  // first position of this row in tile 0
  // each level's least and greatest score over the wave, one slot per wave
  const int nwav = (int)((a.covered + 63) >> 6);
  uint32_t* lvl = a.lvl_mm + ((int64_t)head * nwav + (wave_base >> 6)) * 2 * kMaxLevels;
  uint32_t rmn, rmx;
  auto track = [&](bool in, float v) {
    const uint32_t k = order_key(v);
    rmn = in ? min(rmn, k) : rmn;
    rmx = in ? max(rmx, k) : rmx;
  };
  auto publish = [&](int j) {
    rmn = wave_min_u32(rmn);
    rmx = wave_max_u32(rmx);
    if (lane == 0) {
      lvl[2 * j] = rmn;
      lvl[2 * j + 1] = rmx;
    }
  };
  // softmax scores: every query row's level-j logits (the block sums scaled
  // by 2^{-j/2} / sqrt(d)), row `query` of level j at lg(j) + query * plen(j)
  const bool soft = a.soft != 0;
  float* lgh = soft ? head_logits(a, head) + (int64_t)a.n_q * a.n_top4 : nullptr;
  auto lgrow = [&](int j, int query) {
    return lgh + (int64_t)a.n_q * a.cov_off[j] + (int64_t)query * ((((a.covered >> j) + 3) >> 2) << 2);
  };
  const float isd_raw = a.inv_sqrt_d;
  if (!soft) {  // uniform
    cover_levels<MEAN, RT>(a, s, cov, isd, lvl, wave_base, lane, g, l16, jmax);
    return;
  }
  // level 0
  rmn = 0xFFFFFFFFu;
  rmx = 0u;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    float m[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x = s[t][0][r];
#pragma unroll
      for (int qt = 1; qt < RT; ++qt) x = AG::comb(x, s[t][qt][r]);
      m[r] = AG::row(x) * isd;
    }
    const int64_t p = tb + 16 * t;
    if (writer && p < a.covered)  // (level arrays are padded to multiples of four)
      *reinterpret_cast<float4*>(cov + a.cov_off[0] + p) = make_float4(m[0], m[1], m[2], m[3]);
    if (soft && p < a.covered)
#pragma unroll
      for (int qt = 0; qt < RT; ++qt)
        if (16 * qt + l16 < a.n_q)
          *reinterpret_cast<float4*>(lgrow(0, 16 * qt + l16) + p) =
              make_float4(s[t][qt][0] * isd_raw, s[t][qt][1] * isd_raw, s[t][qt][2] * isd_raw, s[t][qt][3] * isd_raw);
#pragma unroll
    for (int r = 0; r < 4; ++r) track(writer && p + r < a.covered, m[r]);
  }
  publish(0);
  if (jmax <= 1) return;
  // level 1: token pairs (r = 0,1 and 2,3), in place into s[t][qt][0] and [2]
  rmn = 0xFFFFFFFFu;
  rmx = 0u;
  {
    const float sc = isd * 0.70710678118654752440f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int qt = 0; qt < RT; ++qt) {
        s[t][qt][0] += s[t][qt][1];
        s[t][qt][2] += s[t][qt][3];
      }
      float m[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float x = s[t][0][2 * h];
#pragma unroll
        for (int qt = 1; qt < RT; ++qt) x = AG::comb(x, s[t][qt][2 * h]);
        m[h] = AG::row(x) * sc;
      }
      const int64_t p = tb + 16 * t;
      if (writer && p < a.covered) *reinterpret_cast<float2*>(cov + a.cov_off[1] + (p >> 1)) = make_float2(m[0], m[1]);
      if (soft && p < a.covered) {
        const float f = isd_raw * 0.70710678118654752440f;
#pragma unroll
        for (int qt = 0; qt < RT; ++qt)
          if (16 * qt + l16 < a.n_q)
            *reinterpret_cast<float2*>(lgrow(1, 16 * qt + l16) + (p >> 1)) = make_float2(s[t][qt][0] * f, s[t][qt][2] * f);
      }
      track(writer && p < a.covered, m[0]);
      track(writer && p + 2 < a.covered, m[1]);
    }
  }
  publish(1);
  if (jmax <= 2) return;
  // level 2: 4-token blocks (one per lane group), into s[t][qt][0]
  rmn = 0xFFFFFFFFu;
  rmx = 0u;
  {
    const float sc = isd * 0.5f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int qt = 0; qt < RT; ++qt) s[t][qt][0] += s[t][qt][2];
      float x = s[t][0][0];
#pragma unroll
      for (int qt = 1; qt < RT; ++qt) x = AG::comb(x, s[t][qt][0]);
      x = AG::row(x) * sc;
      const int64_t p = tb + 16 * t;
      if (writer && p < a.covered) cov[a.cov_off[2] + (p >> 2)] = x;
      if (soft && p < a.covered)
#pragma unroll
        for (int qt = 0; qt < RT; ++qt)
          if (16 * qt + l16 < a.n_q) lgrow(2, 16 * qt + l16)[p >> 2] = s[t][qt][0] * (isd_raw * 0.5f);
      track(writer && p < a.covered, x);
    }
  }
  publish(2);
  if (jmax <= 3) return;
  // level 3: 8-token blocks = lane groups {0,1} and {2,3}
  rmn = 0xFFFFFFFFu;
  rmx = 0u;
  {
    const float sc = isd * 0.35355339059327376220f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int qt = 0; qt < RT; ++qt) s[t][qt][0] = sum_xor16(s[t][qt][0]);
      float x = s[t][0][0];
#pragma unroll
      for (int qt = 1; qt < RT; ++qt) x = AG::comb(x, s[t][qt][0]);
      x = AG::row(x) * sc;
      const int64_t p = tb + 16 * t;
      if (writer && (g & 1) == 0 && p < a.covered) cov[a.cov_off[3] + (p >> 3)] = x;
      if (soft && (g & 1) == 0 && p < a.covered)
#pragma unroll
        for (int qt = 0; qt < RT; ++qt)
          if (16 * qt + l16 < a.n_q)
            lgrow(3, 16 * qt + l16)[p >> 3] = s[t][qt][0] * (isd_raw * 0.35355339059327376220f);
      track(writer && (g & 1) == 0 && p < a.covered, x);
    }
  }
  publish(3);
  if (jmax <= 4) return;
  // level 4: 16-token blocks = whole tiles
  rmn = 0xFFFFFFFFu;
  rmx = 0u;
  {
    const float sc = isd * 0.25f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int qt = 0; qt < RT; ++qt) s[t][qt][0] = sum_xor32(s[t][qt][0]);
      float x = s[t][0][0];
#pragma unroll
      for (int qt = 1; qt < RT; ++qt) x = AG::comb(x, s[t][qt][0]);
      x = AG::row(x) * sc;
      const int64_t p = wave_base + 16 * t;
      if (writer && g == 0 && p < a.covered) cov[a.cov_off[4] + (p >> 4)] = x;
      if (soft && g == 0 && p < a.covered)
#pragma unroll
        for (int qt = 0; qt < RT; ++qt)
          if (16 * qt + l16 < a.n_q) lgrow(4, 16 * qt + l16)[p >> 4] = s[t][qt][0] * (isd_raw * 0.25f);
      track(writer && g == 0 && p < a.covered, x);
    }
  }
  publish(4);
  if (jmax <= 5) return;
  // level 5: tile pairs; level 6: the whole wave
  {
    float x01 = s[0][0][0] + s[1][0][0], x23 = s[2][0][0] + s[3][0][0];
    float xall = x01 + x23;
#pragma unroll
    for (int qt = 1; qt < RT; ++qt) {
      const float a01 = s[0][qt][0] + s[1][qt][0];
      const float a23 = s[2][qt][0] + s[3][qt][0];
      x01 = AG::comb(x01, a01);
      x23 = AG::comb(x23, a23);
      xall = AG::comb(xall, a01 + a23);
    }
    x01 = AG::row(x01) * (isd * 0.17677669529663688110f);  // 2^{-5/2}
    x23 = AG::row(x23) * (isd * 0.17677669529663688110f);
    xall = AG::row(xall) * (isd * 0.125f);                 // 2^{-3}
    if (lane == 0) {
      if (wave_base < a.covered) cov[a.cov_off[5] + (wave_base >> 5)] = x01;
      if (wave_base + 32 < a.covered) cov[a.cov_off[5] + (wave_base >> 5) + 1] = x23;
      if (jmax > 6) cov[a.cov_off[6] + (wave_base >> 6)] = xall;
    }
    if (soft && g == 0)
#pragma unroll
      for (int qt = 0; qt < RT; ++qt) {
        const int query = 16 * qt + l16;
        if (query >= a.n_q) continue;
        const float a01 = s[0][qt][0] + s[1][qt][0], a23 = s[2][qt][0] + s[3][qt][0];
        if (wave_base < a.covered) lgrow(5, query)[wave_base >> 5] = a01 * (isd_raw * 0.17677669529663688110f);
        if (wave_base + 32 < a.covered) lgrow(5, query)[(wave_base >> 5) + 1] = a23 * (isd_raw * 0.17677669529663688110f);
        if (jmax > 6) lgrow(6, query)[wave_base >> 6] = (a01 + a23) * (isd_raw * 0.125f);
      }
    rmn = 0xFFFFFFFFu;
    rmx = 0u;
    track(lane == 0 && wave_base < a.covered, x01);
    track(lane == 0 && wave_base + 32 < a.covered, x23);
    publish(5);
    if (jmax > 6) {
      rmn = 0xFFFFFFFFu;
      rmx = 0u;
      track(lane == 0, xall);
      publish(6);
    }
  }
}

// ---------------------------------------------------------------------------
// Recursive refinement (Figure 2 (d)) of one head in registers, by one
// workgroup of NT threads: thread t holds the level-0 positions
// [t S0, t S0 + S0) and their ancestors (see wf_select.h).  Every level's
// coverage scores and score range are loaded at the start, then a loop over
// the levels keeps the k_j best children of the kept parents.  The loop body is one copy of the level code, so the
// instructions a single workgroup runs stay few and, after the first level,
// cached.  Writes the kept tokens ascending, and with the per-level sinks
// every level's kept regions.
// ---------------------------------------------------------------------------
template <int S0, int J> struct Held { static constexpr int N = (S0 >> J) > 0 ? (S0 >> J) : 1; };
template <int S0> struct HeldScores {
  float s0[Held<S0, 0>::N], s1[Held<S0, 1>::N], s2[Held<S0, 2>::N], s3[Held<S0, 3>::N];
  float s4[Held<S0, 4>::N], s5[Held<S0, 5>::N], s6[Held<S0, 6>::N];
  template <int J> __device__ __forceinline__ auto& get() {
    if constexpr (J == 0) return s0;
    else if constexpr (J == 1) return s1;
    else if constexpr (J == 2) return s2;
    else if constexpr (J == 3) return s3;
    else if constexpr (J == 4) return s4;
    else if constexpr (J == 5) return s5;
    else return s6;
  }
  // a level past the pyramid's top: never read, held at zero
  template <int J> __device__ __forceinline__ void clear() {
#pragma unroll
    for (int i = 0; i < Held<S0, J>::N; ++i) get<J>()[i] = 0.f;
  }
  // level j's first P slots (P is the level's count of held slots)
  template <int P> __device__ __forceinline__ void first(int j, float (&sc)[P]) {
#pragma unroll
    for (int i = 0; i < P; ++i) sc[i] = 0.f;
    switch (j) {
      case 0: take<0>(sc); break;
      case 1: take<1>(sc); break;
      case 2: take<2>(sc); break;
      case 3: take<3>(sc); break;
      case 4: take<4>(sc); break;
      case 5: take<5>(sc); break;
      default: take<6>(sc); break;
    }
  }
  template <int J, int P> __device__ __forceinline__ void take(float (&sc)[P]) {
    constexpr int n = Held<S0, J>::N < P ? Held<S0, J>::N : P;
#pragma unroll
    for (int i = 0; i < n; ++i) sc[i] = get<J>()[i];
  }
  template <int J> __device__ __forceinline__ void load(const float* src, int nj, int p0) {
    auto& s = get<J>();
    if constexpr (Held<S0, J>::N >= 2) {
#pragma unroll
      for (int i = 0; i < Held<S0, J>::N; i += 2) {
        const float2 v = *reinterpret_cast<const float2*>(src + min(p0 + i, nj - 2));
        s[i] = v.x;
        s[i + 1] = v.y;
      }
    } else {
      s[0] = src[min(p0, nj - 1)];
    }
  }
};
static_assert(kMaxLevels == 7, "the refinement holds seven levels");

// A level's bins and budget k_j, read from LDS one level ahead.
struct LevelPar {
  float scale, off;
  int k;
};

// One refinement level over the P = max(1, S0 >> j) slots a thread holds at
// level j (the per-slot work of the level scales with P, not with S0):
// candidates are the held positions whose parent was kept (keptp, the
// parent level's slots); returns the kept mask over the P slots and, with
// the per-level sinks, writes the level's kept regions at off.
template <int NT, int S0, int P>
__device__ __forceinline__ uint32_t refine_level(const StepArgs& a, const RefineLead& rl, int head, HeldScores<S0>& hs,
                                                 int j, const LevelPar& lp, uint32_t keptp, const int* sel_l,
                                                 SelShared<NT>& sh, SelCursor& cur, int off) {
  const int t = threadIdx.x;
  const int L = rl.levels;
  float sc[P];
  hs.template first<P>(j, sc);
  const int p0 = (t * S0) >> j, nj = rl.covered >> j;
  const bool own = P > 1 || ((t * S0) & ((1 << j) - 1)) == 0;
  uint32_t valid = 0u;
#pragma unroll
  for (int i = 0; i < P; ++i) valid |= ((p0 + i < nj) & ((keptp >> (i >> 1)) & 1u)) ? (1u << i) : 0u;
  const uint32_t owned = own ? valid : 0u;
  const int kj = lp.k;
  const uint32_t kept = select_level<NT, P>(sc, valid, owned, p0, kj, LinBins(lp.scale, lp.off, true), sh, cur);
  int32_t* dbg_sel = sh.dsel;
  float* dbg_score = sh.dscore;
  if (dbg_sel || dbg_score) {  // uniform: level j's kept regions, ascending, with their scores
    const uint32_t km = own ? kept : 0u;
    int o = block_excl_scan(__popc(km), sh, 2 + (j & 1));
    const int shl = L - j;
#pragma unroll
    for (int i = 0; i < P; ++i)
      if ((km >> i) & 1u) {
        const int p = p0 + i;
        if (o < kj) {
          if (dbg_sel) dbg_sel[off + o] = (sel_l[min(p >> shl, rl.k_top - 1)] << shl) + (p & ((1 << shl) - 1));
          if (dbg_score) dbg_score[off + o] = sc[i];
        }
        ++o;
      }
  }
  return kept;
}

template <int NT, int S0>
__device__ __forceinline__ void refine_sel(const StepArgs& a, const RefineLead& rl, int head, int* sel_l,
                                           SelShared<NT>& sh) {
  const int t = threadIdx.x, lane = t & 63;
  const int L = rl.levels;
  const int covered = rl.covered;
  const float* cov = rl.cov + (int64_t)head * rl.cov_len;
  // level j's scores start at sum_{i<j} roundup4(covered >> i) inside the head's slice
  int coff[kMaxLevels + 1];
  coff[0] = 0;
#pragma unroll
  for (int j = 0; j < kMaxLevels; ++j) coff[j + 1] = coff[j] + (((covered >> j) + 3) & ~3);
  // Every load of the stage is requested before any is waited for, so the
  // coverage scores, the level ranges and the kept coarse regions arrive in
  // one round trip.  Each level's score range: the cover waves' slots (at most 128 per head
  // here, lanes l and l + 64 of wave 0), reduced by wave 0, which publishes
  // the level's bins to LDS.  Loads are unconditional, from clamped slots;
  // slots past the last wave take the neutral range by an all-ones mask.
  // They are requested first, then the kept coarse regions, then the scores
  // (coarsest level first), so that wave 0's reduction and the first barrier
  // wait only for the first two while the finer levels' scores still arrive.
  const int nwav = (covered + 63) >> 6;
  const uint32_t* lm = rl.lvl + (int64_t)head * nwav * 2 * kMaxLevels;
  // (every wave requests them, so that no branch separates them from the
  // loads below; only wave 0 reads them)
  uint32_t x[2][kMaxLevels][2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int v = min(lane + 64 * r, nwav - 1);
#pragma unroll
    for (int j = 0; j < kMaxLevels; ++j) {
      const uint2 p = *reinterpret_cast<const uint2*>(lm + (int64_t)v * 2 * kMaxLevels + 2 * j);
      x[r][j][0] = p.x;
      x[r][j][1] = p.y;
    }
  }
  // the kept coarse regions [k_L] (from the cover launch), this thread's first one
  const int32_t* sel_g = rl.sel_top + (int64_t)head * rl.k_top;
  const int sel0 = sel_g[min(t, rl.k_top - 1)];
  __builtin_amdgcn_sched_barrier(0);  // the loads above stay ahead of the score loads
  // every level's scores into registers (clamped positions; slots past a
  // level's end are never valid; a level past the pyramid's top loads level
  // 0's slots and is never read)
  HeldScores<S0> hs;
#define WF_LOAD_LEVEL(J) \
  hs.template load<J>(J < L ? cov + coff[J] : cov, J < L ? covered >> J : covered, (t * S0) >> J);
  WF_LOAD_LEVEL(6)
  WF_LOAD_LEVEL(5)
  WF_LOAD_LEVEL(4)
  WF_LOAD_LEVEL(3)
  WF_LOAD_LEVEL(2)
  WF_LOAD_LEVEL(1)
  WF_LOAD_LEVEL(0)
#undef WF_LOAD_LEVEL
  if (t < 64) {
    // all levels' least keys (complemented) and greatest keys in one
    // scattered reduction: value l (l < 8: level l's least, l >= 8: level
    // l - 8's greatest) ends in lane l16 = l of every row, then the rows combine
    uint32_t w[16];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t mn = 0u, mx = 0u;
      if (j < kMaxLevels) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const uint32_t off = (uint32_t)((nwav - 1 - (lane + 64 * r)) >> 31);  // ~0u past the last wave
          mn = max(mn, ~(x[r][j][0] | off));
          mx = max(mx, x[r][j][1] & ~off);
        }
      }
      w[j] = mn;
      w[8 + j] = mx;
    }
    uint32_t q = row_max_scatter_u<16>(w, lane & 15);
    q = max(q, lane_xor16(q));
    q = max(q, lane_xor32(q));
    // lane j < 7 takes level j's greatest key from lane j + 8 (row_ror:8) and
    // publishes the level's bins, built once here rather than in every wave
    const uint32_t qx = dpp_u<0x128>(q);
    const LinBins bin(key_to_f32(~q), key_to_f32(qx));
    if (lane < kMaxLevels) {
      sh.rsc[lane] = bin.scale;
      sh.rof[lane] = bin.off;
    }
  }
  // the kept coarse regions into LDS (more than one per thread only when k_L > NT)
  if (t < rl.k_top) sel_l[t] = clampi(sel0, 0, rl.n_top - 1);
  for (int i = t + NT; i < rl.k_top; i += NT) sel_l[i] = clampi(sel_g[i], 0, rl.n_top - 1);
  // the level budgets and the output pointers, read while the loads above are
  // in flight: read after the barrier, each would wait for a trip to memory
  if (t == 0) {
#pragma unroll
    for (int j = 0; j <= kMaxLevels; ++j) sh.bud[j] = a.budgets[j];
    sh.dsel = a.sel_levels ? a.sel_levels + (int64_t)head * a.sum_k : nullptr;
    sh.dscore = a.score_levels ? a.score_levels + (int64_t)head * a.sum_k : nullptr;
    sh.k0 = a.k0;
    const HeadRef hr = head_ref(a, head);
    sh.tsel = a.sel_ws + (int64_t)head * a.k0;
    sh.sout = a.sel_out[hr.item] ? a.sel_out[hr.item] + hr.local * a.k0 : nullptr;
  }
  sel_init(sh);
  __syncthreads();

  // level L: every kept coarse region (positions [0, k_L))
  uint32_t keptp = 0u;
  {
    const int pl0 = (t * S0) >> L;
    const int pl = (S0 >> L) > 0 ? (S0 >> L) : 1;
    for (int m = 0; m < pl; ++m) keptp |= (pl0 + m < rl.k_top) ? (1u << m) : 0u;
  }
  int off = rl.k_top;
  SelCursor cur;
  LevelPar nxt{sh.rsc[L - 1], sh.rof[L - 1], sh.bud[1]};
  for (int j = L - 1; j >= 0; --j) {  // each level on its own count of held slots
    const LevelPar lp = nxt;
    const int jn = j > 0 ? j - 1 : 0;
    nxt = LevelPar{sh.rsc[jn], sh.rof[jn], sh.bud[L - jn]};  // the next level's, requested before this level waits
    const int pj = (S0 >> j) > 0 ? (S0 >> j) : 1;
    uint32_t kept;
    if (pj == 1) {
      kept = refine_level<NT, S0, 1>(a, rl, head, hs, j, lp, keptp, sel_l, sh, cur, off);
    } else if constexpr (S0 >= 2) {
      if (pj == 2) {
        kept = refine_level<NT, S0, 2>(a, rl, head, hs, j, lp, keptp, sel_l, sh, cur, off);
      } else if constexpr (S0 >= 4) {
        if (pj == 4) kept = refine_level<NT, S0, 4>(a, rl, head, hs, j, lp, keptp, sel_l, sh, cur, off);
        else kept = refine_level<NT, S0, S0>(a, rl, head, hs, j, lp, keptp, sel_l, sh, cur, off);
      } else {
        kept = 0u;  // not reached: pj <= S0
      }
    } else {
      kept = 0u;  // not reached: pj <= S0
    }
    off += lp.k;
    keptp = kept;
  }

  // the kept tokens, ascending
  int o = block_excl_scan(__popc(keptp), sh, 1);
  int32_t* tsel = sh.tsel;
  int32_t* so = sh.sout;
  const int k0 = sh.k0;
  const int mask = (1 << L) - 1;
#pragma unroll
  for (int i = 0; i < S0; ++i)
    if ((keptp >> i) & 1u) {
      const int p = t * S0 + i;
      const int tok = (sel_l[min(p >> L, rl.k_top - 1)] << L) + (p & mask);
      if (o < k0) {  // exactly k_0 are kept; the bound guards the buffers
        tsel[o] = tok;
        if (so) so[o] = tok;
      }
      ++o;
    }
}

// ---------------------------------------------------------------------------
// Cover stage: the kept coarse regions (the coarse Top-K, computed by every
// workgroup of the head, or read from the Top-K's own launch), then the
// coverage scores of this workgroup's 256 covered positions.
// ---------------------------------------------------------------------------
template <typename T, int D, int RT, bool MEAN, bool BANDS>
__device__ __forceinline__ void cover_stage(const StepArgs& a, const CoverLead& cl) {
  constexpr int NT = kCoverThreads;
  static_assert(NT == kSelThreads, "the coarse Top-K runs on the cover workgroup");
  extern __shared__ __align__(16) uint32_t lds[];  // the kept coarse regions [k_L], ascending
  __shared__ __align__(16) unsigned char raw[sizeof(SelShared<NT>)];
  __shared__ __align__(16) T qs[16 * RT * (D + QueryLds<T>::PAD)];
  const int head = blockIdx.y;
  int* sel_l = reinterpret_cast<int*>(lds);
  QueryStage<T, D, NT, RT> qstage;  // the query block is in flight during the Top-K
  const HeadRef hr = head_ref(cl.n_items, cl.heads_per_item, head);
  auto issue_q = [&] { qstage.issue(reinterpret_cast<const T*>(a.q[hr.item]) + hr.local * a.n_q * D, a.n_q); };
  if (topk_in_cover(cl)) {  // uniform: every workgroup of the head computes the same kept regions
    auto emit = coarse_emitter(a, head, hr, blockIdx.x == 0, [&](int o, int i) { sel_l[o] = i; });
    coarse_topk_run<false>(a, cl, head, raw, nullptr, emit, issue_q);
  } else {  // the Top-K's own launch wrote them
    issue_q();
    const int32_t* sel_g = a.sel_top + (int64_t)head * a.k_top;
    for (int i = threadIdx.x; i < a.k_top; i += NT) sel_l[i] = clampi(sel_g[i], 0, a.n_top - 1);
  }
  qstage.store(a.n_q, qs);
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int64_t wave_base = (int64_t)blockIdx.x * 256 + w * 64;
  if (wave_base >= a.covered) return;  // no workgroup barrier below
  Frag<T, D> qf[RT];
  load_query_frags<T, D, RT>(qs, a.n_q, l16, g, qf);
  if constexpr (BANDS) cover_from_bands<T, D, RT, MEAN>(a, head, sel_l, qf, wave_base, lane, g, l16);
  else cover_haar<T, D, RT, MEAN>(a, head, sel_l, qf, wave_base, lane, g, l16);
}

// With one or two query tiles (and bfloat16 rows, or head dim 64) the Haar
// cover kernel fits 128 registers without spilling: four workgroups per
// compute unit, so large launches take fewer rounds; otherwise it keeps the
// registers its loads in flight need.
template <typename T, int D>
constexpr int cover_waves_per_simd(int rt) { return (sizeof(T) == 2 || D == 64) && rt <= 2 ? 4 : 1; }
template <typename T, int D, int RT>
__global__ __launch_bounds__(kCoverThreads, (cover_waves_per_simd<T, D>(RT))) void cover_max_kernel(WF_LEAD_PARAMS,
                                                                                                StepArgs a) {
  cover_stage<T, D, RT, false, false>(a, CoverLead::of(WF_LEAD));
}
template <typename T, int D, int RT>
__global__ __launch_bounds__(kCoverThreads, (cover_waves_per_simd<T, D>(RT))) void cover_mean_kernel(WF_LEAD_PARAMS,
                                                                                                 StepArgs a) {
  cover_stage<T, D, RT, true, false>(a, CoverLead::of(WF_LEAD));
}
template <typename T, int D, int RT>
__global__ __launch_bounds__(kCoverThreads) void cover_bands_max_kernel(WF_LEAD_PARAMS, StepArgs a) {
  cover_stage<T, D, RT, false, true>(a, CoverLead::of(WF_LEAD));
}
template <typename T, int D, int RT>
__global__ __launch_bounds__(kCoverThreads) void cover_bands_mean_kernel(WF_LEAD_PARAMS, StepArgs a) {
  cover_stage<T, D, RT, true, true>(a, CoverLead::of(WF_LEAD));
}

// One refinement level with the candidates in registers (n <= ACT * MAXS):
// candidate i is child (i & 1) of kept parent cur[i >> 1]; the kept ones go
// to nxt in ascending order, the others to its spare slot nxt[kj].
template <int NT, int ACT, int MAXS>
__device__ __forceinline__ void refine_level(const float* cj, int nj, const int* cur, int* nxt, int n, int kj,
                                             unsigned char* raw) {
  auto& sh = *reinterpret_cast<TopKSel<ACT, MAXS>*>(raw);
  int pos[MAXS];
  topk_strided<NT, ACT, MAXS>(
      n, kj, sh,
      [&](int i, int j) {
        const int p = clampi(2 * cur[i >> 1] + (i & 1), 0, nj - 1);
        pos[j] = p;
        return order_key(cj[p]);
      },
      [&](int o, bool kept, int, int j) { nxt[kept ? o : kj] = pos[j]; });
}

// ---------------------------------------------------------------------------
// Recursive refinement (Figure 2 (d)) for one head with sorted index lists,
// for covered sets beyond the in-register refinement: one workgroup per
// head, in a launch of its own after the cover launch.  Positions at level j
// index the level-j blocks inside the covered set, ascending; the block at
// position p has children 2p and 2p+1 and global index
// sel_L[p >> (L-j)] 2^{L-j} + (p mod 2^{L-j}).  State lives in LDS:
// keys[nmax] | cur[kmax] | nxt[kmax] | (coverage scores, when they fit).
// Writes the kept tokens (ascending) to tsel[0 .. k0), sel_out and the
// per-level outputs of levels L-1 .. 0.
// ---------------------------------------------------------------------------
template <int NT>
__device__ __forceinline__ void refine_head_lists(const StepArgs& a, int head, uint32_t* lds, unsigned char* tk_raw,
                                                  int* tsel) {
  const int L = a.levels;
  uint32_t* keys = lds;
  int* cur = reinterpret_cast<int*>(lds + a.refine_nmax);
  int* nxt = cur + a.refine_kmax;
  float* cov_l = reinterpret_cast<float*>(nxt + a.refine_kmax);
  const int32_t* sel_top = a.sel_top + (int64_t)head * a.k_top;
  const float* cov_g = a.cov + (int64_t)head * a.cov_len;
  const float* cov = a.refine_cov_in_lds ? cov_l : cov_g;
  if (a.refine_cov_in_lds) {
    const float4* src = reinterpret_cast<const float4*>(cov_g);
    float4* dst = reinterpret_cast<float4*>(cov_l);
    const int n4 = (int)(a.cov_len / 4);
    for (int i = threadIdx.x; i < n4; i += NT) dst[i] = src[i];
  }
  int32_t* dbg_sel = a.sel_levels ? a.sel_levels + (int64_t)head * a.sum_k : nullptr;
  float* dbg_score = a.score_levels ? a.score_levels + (int64_t)head * a.sum_k : nullptr;
  for (int i = threadIdx.x; i < a.k_top; i += NT) cur[i] = i;
  __syncthreads();
  int kprev = a.k_top, dbg_off = a.k_top;
  for (int j = L - 1; j >= 0; --j) {
    const int kj = a.budgets[L - j];
    const int n = 2 * kprev;
    const int nj = (int)(a.covered >> j);  // level-j positions in the covered set
    const float* cj = cov + a.cov_off[j];
    constexpr int A0 = TopKRaw<NT>::ACT0;
    if (n <= A0 * 4) {
      refine_level<NT, A0, 4>(cj, nj, cur, nxt, n, kj, tk_raw);
    } else if (n <= A0 * 8) {
      refine_level<NT, A0, 8>(cj, nj, cur, nxt, n, kj, tk_raw);
    } else if (n <= A0 * 16) {
      refine_level<NT, A0, 16>(cj, nj, cur, nxt, n, kj, tk_raw);
    } else if (n <= A0 * 32) {
      refine_level<NT, A0, 32>(cj, nj, cur, nxt, n, kj, tk_raw);
    } else {
      auto& sh = *reinterpret_cast<TopKFastShared<NT>*>(tk_raw);
      for (int c = threadIdx.x; c < n; c += NT) keys[c] = order_key(cj[clampi(2 * cur[c >> 1] + (c & 1), 0, nj - 1)]);
      __syncthreads();
      topk_fast<NT>([&](int i) { return keys[i]; }, n, kj, sh, [&](int o, int i) {
        if (o < kj) nxt[o] = clampi(2 * cur[i >> 1] + (i & 1), 0, nj - 1);
      });
    }
    __syncthreads();
    if (dbg_sel || dbg_score) {
      const int sh_l = L - j;
      for (int o = threadIdx.x; o < kj; o += NT) {
        const int p = nxt[o];
        if (dbg_sel)
          dbg_sel[dbg_off + o] =
              (clampi(sel_top[clampi(p >> sh_l, 0, a.k_top - 1)], 0, a.n_top - 1) << sh_l) + (p & ((1 << sh_l) - 1));
        if (dbg_score) dbg_score[dbg_off + o] = cj[p];
      }
    }
    int* tmp = cur;
    cur = nxt;
    nxt = tmp;
    kprev = kj;
    dbg_off += kj;
  }
  const HeadRef hr = head_ref(a, head);
  int32_t* so = a.sel_out[hr.item] ? a.sel_out[hr.item] + hr.local * a.k0 : nullptr;
  for (int o = threadIdx.x; o < a.k0; o += NT) {
    const int p = cur[o];
    const int tok = (clampi(sel_top[clampi(p >> L, 0, a.k_top - 1)], 0, a.n_top - 1) << L) + (p & ((1 << L) - 1));
    tsel[o] = tok;
    if (so) so[o] = tok;
  }
}

#if !defined(WF_STEP_T)  // one compile unit holds these
// The coarse Top-K in a launch of its own, one workgroup per head (n_L >
// 1 024, or L = 0).
__global__ __launch_bounds__(kSelThreads) void coarse_topk_kernel(StepArgs a) {
  extern __shared__ __align__(16) uint32_t keys_l[];  // general path: the keys, when staged
  __shared__ __align__(16) unsigned char raw[kSelRawBytes];
  const int head = blockIdx.x;
  coarse_topk_run<true>(a, cover_lead(a), head, raw, keys_l,
                        coarse_emitter(a, head, head_ref(a, head), true, [](int, int) {}), [] {});
}

// ---------------------------------------------------------------------------
// Softmax-probability scores.  A query row's probability of candidate c at a
// level is p_i[c] = exp(l_i[c] - lse_i), lse_i = log sum over the level's
// candidates c' of exp(l_i[c']), from the per-row logits l_i the coarse and
// cover launches wrote; the score is max_i p_i[c] or (1/n_q) sum_i p_i[c].
// Candidates are ranked by the logarithm of that score (a monotone map, so
// the same ones are kept): probabilities far below the largest (exp(-100)
// and less) underflow float32 and would tie at zero, their logarithms do
// not.  The per-level score outputs report the probabilities themselves.
// ---------------------------------------------------------------------------
// Online log-sum-exp: (m, s) with s = sum exp(x - m) over the values seen.
__device__ __forceinline__ void lse_add(float& m, float& s, float x) {
  if (x > m) {
    s = s * expf(m - x) + 1.f;
    m = x;
  } else {
    s += expf(x - m);
  }
}
// Merge the state of lane ^ off into this lane's.
__device__ __forceinline__ void lse_merge(float& m, float& s, int off) {
  const float m2 = __shfl_xor(m, off, 64), s2 = __shfl_xor(s, off, 64);
  const float mm = fmaxf(m, m2);
  s = (m == -INFINITY ? 0.f : s * expf(m - mm)) + (m2 == -INFINITY ? 0.f : s2 * expf(m2 - mm));
  m = mm;
}
// The logarithm of one candidate's score from its column of logits (row
// stride `stride`): max_i (l_i - lse_i), or the log of the mean over the rows
// of exp(l_i - lse_i) by an online log-sum-exp.
__device__ __forceinline__ float soft_score(const StepArgs& a, const float* col, int64_t stride, const float* lse) {
  if (a.soft == 1) {
    float m = -INFINITY;
    for (int r = 0; r < a.n_q; ++r) m = fmaxf(m, col[(int64_t)r * stride] - lse[r]);
    return m;
  }
  float m = -INFINITY, sum = 0.f;
  for (int r = 0; r < a.n_q; ++r) lse_add(m, sum, col[(int64_t)r * stride] - lse[r]);
  return m + logf(sum * a.inv_nq);
}

// Level L (every region a candidate): each row's log-sum-exp (four threads
// per row), then every region's score as an order key for the coarse Top-K
// launch that follows.
__global__ __launch_bounds__(kSelThreads) void soft_top_kernel(StepArgs a) {
  __shared__ float lse[64];
  const int head = blockIdx.x, t = threadIdx.x;
  const float* lg = head_logits(a, head);
  {
    const int row = t >> 2, part = t & 3;
    float m = -INFINITY, sum = 0.f;
    if (row < a.n_q)
      for (int c = part; c < a.n_top; c += 4) lse_add(m, sum, lg[(int64_t)row * a.n_top4 + c]);
    lse_merge(m, sum, 1);
    lse_merge(m, sum, 2);
    if (part == 0 && row < a.n_q) lse[row] = m + logf(sum);
  }
  __syncthreads();
  uint32_t* keys = a.keys_top + (int64_t)head * a.n_top;
  for (int c = t; c < a.n_top; c += kSelThreads) keys[c] = order_key(soft_score(a, lg + c, a.n_top4, lse));
}

// The refinement with softmax scores: refine_sel's slot layout and level
// loop, with each level's scores formed in the loop: the candidates (valid
// positions) are listed in LDS, each row's log-sum-exp over them is taken by
// 16 threads per row, then every slot's score from its column of logits and
// the level's score range for the binning.
template <int S0>
__global__ __launch_bounds__(kRefineThreads) void refine_soft_kernel(StepArgs a) {
  constexpr int NT = kRefineThreads;
  extern __shared__ __align__(16) uint32_t lds[];  // kept coarse regions [k_L], then the candidate list
  __shared__ __align__(16) SelShared<NT> sh;
  __shared__ float lse[64];
  __shared__ uint32_t smn, smx;
  const int head = blockIdx.x, t = threadIdx.x, lane = t & 63;
  const int L = a.levels;
  const int covered = (int)a.covered;
  int* sel_l = reinterpret_cast<int*>(lds);
  int* clist = sel_l + ((a.k_top + 3) & ~3);
  for (int i = t; i < a.k_top; i += NT) sel_l[i] = clampi(a.sel_top[(int64_t)head * a.k_top + i], 0, a.n_top - 1);
  sel_init(sh);
  __syncthreads();
  const float* lgh = head_logits(a, head) + (int64_t)a.n_q * a.n_top4;

  uint32_t keptp = 0u;  // level L: every kept coarse region
  {
    const int pl0 = (t * S0) >> L;
    const int pl = (S0 >> L) > 0 ? (S0 >> L) : 1;
    for (int m = 0; m < pl; ++m) keptp |= (pl0 + m < a.k_top) ? (1u << m) : 0u;
  }
  const bool report = a.sel_levels || a.score_levels;
  int32_t* dbg_sel = a.sel_levels ? a.sel_levels + (int64_t)head * a.sum_k : nullptr;
  float* dbg_score = a.score_levels ? a.score_levels + (int64_t)head * a.sum_k : nullptr;
  int off = a.k_top;
  SelCursor cur;
  for (int j = L - 1; j >= 0; --j) {
    const int pj = (S0 >> j) > 0 ? (S0 >> j) : 1;
    const int p0 = (t * S0) >> j, nj = covered >> j;
    const bool own = pj > 1 || ((t * S0) & ((1 << j) - 1)) == 0;
    uint32_t valid = 0u;
#pragma unroll
    for (int i = 0; i < S0; ++i)
      valid |= ((i < pj) & (p0 + i < nj) & ((keptp >> (i >> 1)) & 1u)) ? (1u << i) : 0u;
    const uint32_t owned = own ? valid : 0u;
    const int64_t plen = ((nj + 3) >> 2) << 2;
    const float* lgj = lgh + (int64_t)a.n_q * a.cov_off[j];
    // 1. the candidates, ascending
    int nv;
    {
      int o = block_excl_scan(__popc(owned), sh, 4 + (j & 1), &nv);
#pragma unroll
      for (int i = 0; i < S0; ++i)
        if ((owned >> i) & 1u) clist[o++] = p0 + i;
    }
    if (t == 0) {
      smn = 0xFFFFFFFFu;
      smx = 0u;
    }
    __syncthreads();
    // 2. each row's log-sum-exp over the candidates
    {
      const int row = t >> 4, part = t & 15;
      float m = -INFINITY, sum = 0.f;
      if (row < a.n_q) {
        const float* lr = lgj + (int64_t)row * plen;
        for (int e = part; e < nv; e += 16) lse_add(m, sum, lr[clist[e]]);
      }
      lse_merge(m, sum, 1);
      lse_merge(m, sum, 2);
      lse_merge(m, sum, 4);
      lse_merge(m, sum, 8);
      if (part == 0 && row < a.n_q) lse[row] = m + logf(sum);
    }
    __syncthreads();
    // 3. the slots' scores and the level's score range
    float sc[S0];
    uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
    for (int i = 0; i < S0; ++i) {
      sc[i] = 0.f;
      if ((valid >> i) & 1u) {
        sc[i] = soft_score(a, lgj + p0 + i, plen, lse);
        const uint32_t k = order_key(sc[i]);
        kmn = ((owned >> i) & 1u) ? min(kmn, k) : kmn;
        kmx = ((owned >> i) & 1u) ? max(kmx, k) : kmx;
      }
    }
    kmn = wave_min_u32(kmn);
    kmx = wave_max_u32(kmx);
    if (lane == 0) {
      atomicMin(&smn, kmn);
      atomicMax(&smx, kmx);
    }
    __syncthreads();
    const int kj = a.budgets[L - j];
    const uint32_t kept = select_level<NT, S0>(sc, valid, owned, p0, kj, key_to_f32(smn), key_to_f32(smx), sh, cur);
    if (report) {  // uniform: level j's kept regions, ascending, with their scores
      const uint32_t km = own ? kept : 0u;
      int o = block_excl_scan(__popc(km), sh, 2 + (j & 1));
      const int shl = L - j;
#pragma unroll
      for (int i = 0; i < S0; ++i)
        if ((km >> i) & 1u) {
          const int p = p0 + i;
          if (o < kj) {
            if (dbg_sel) dbg_sel[off + o] = (sel_l[min(p >> shl, a.k_top - 1)] << shl) + (p & ((1 << shl) - 1));
            if (dbg_score) dbg_score[off + o] = expf(sc[i]);
          }
          ++o;
        }
    }
    off += kj;
    keptp = kept;
  }

  // the kept tokens, ascending
  int o = block_excl_scan(__popc(keptp), sh, 1);
  int32_t* tsel = a.sel_ws + (int64_t)head * a.k0;
  const HeadRef hr = head_ref(a, head);
  int32_t* so = a.sel_out[hr.item] ? a.sel_out[hr.item] + hr.local * a.k0 : nullptr;
  const int mask = (1 << L) - 1;
#pragma unroll
  for (int i = 0; i < S0; ++i)
    if ((keptp >> i) & 1u) {
      const int p = t * S0 + i;
      const int tok = (sel_l[min(p >> L, a.k_top - 1)] << L) + (p & mask);
      if (o < a.k0) {
        tsel[o] = tok;
        if (so) so[o] = tok;
      }
      ++o;
    }
}

// The in-register refinement, one workgroup of 1 024 threads per head, with
// S0 = 1 .. 8 level-0 positions per thread (covered sets up to 8 192).
template <int S0>
__global__ __launch_bounds__(kRefineThreads) void refine_sel_kernel(WF_LEAD_PARAMS, StepArgs a) {
  extern __shared__ __align__(16) uint32_t lds[];  // the kept coarse regions [k_L]
  __shared__ __align__(16) SelShared<kRefineThreads> sh;
  const int head = blockIdx.x;
  refine_sel<kRefineThreads, S0>(a, RefineLead::of(WF_LEAD), head, reinterpret_cast<int*>(lds), sh);
}

__global__ __launch_bounds__(kSelThreads) void refine_lists_kernel(StepArgs a) {
  extern __shared__ __align__(16) uint32_t lds[];
  __shared__ __align__(16) unsigned char tk_raw[TopKRaw<kSelThreads>::BYTES];
  const int head = blockIdx.x;
  refine_head_lists<kSelThreads>(a, head, lds, tk_raw, a.sel_ws + (int64_t)head * a.k0);
}
#endif

// ---------------------------------------------------------------------------
// Sparse attention (eq. 3 over T = kept prompt tokens, then gen_idx).
// Workgroup (split, head) loads its split's part of T (kept prompt tokens
// from the refinement or the caller, then generated positions) into LDS,
// then walks chunks of CH tokens.  Wave w owns query tile
// qt = w / TG and token group tg = w % TG: the CW = CH / TG tokens
// [tg CW, tg CW + CW) of every chunk, with an online-softmax state of its
// own; the TG states of a query tile are merged through LDS at the end, so
// there are TG waves per query tile to hide one another's latencies.  Per
// chunk: K rows -> LDS (row-major, padded), V -> LDS transposed (V^T);
// S^T = K Q^T on MFMA (lane (query l16, g) holds tokens 16 t + 4 g + r);
// online softmax per query row in float32; O^T += V^T P^T on MFMA with P
// split into bf16 hi + lo (float32 MFMA for float32 inputs).  The next
// chunk's rows are fetched into registers while the current one computes.
// Writes the split's partial (m, l, O) to the workspace.
// ---------------------------------------------------------------------------
// x of lane l ^ NV: a DPP row rotation by 8 for NV = 8, a lane permute for 16.
template <int NV>
__device__ __forceinline__ uint32_t lane_xor_nv(uint32_t x) {
  static_assert(NV == 8 || NV == 16, "pair partners NV lanes apart");
  if constexpr (NV == 8) return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xF, 0xF, false);  // row_ror:8
  else return lane_xor16(x);
}

template <typename T> struct AttendTraits;
template <> struct AttendTraits<bf16_t> { static constexpr int KPAD = 8, VPAD = 16, DT = WF_BF16; };
template <> struct AttendTraits<float> { static constexpr int KPAD = 4, VPAD = 4, DT = WF_F32; };

// Online-softmax state of one wave: lane (query l16, g) holds m and l of its
// query row and O^T[16 dt + 4 g + r][query].
template <int D> struct SoftmaxState {
  float m, l;
  f32x4 o[D / 16];
};

// Merge `b` into `a` (m in log2 units; an empty state has m = -inf, l = 0, O = 0).
template <int D>
__device__ __forceinline__ void merge_state(SoftmaxState<D>& a, float mb, float lb, const f32x4* ob) {
  const float mm = fmaxf(a.m, mb);
  const float sa = (a.m == -INFINITY) ? 0.f : exp2f(a.m - mm);
  const float sb = (mb == -INFINITY) ? 0.f : exp2f(mb - mm);
  a.m = mm;
  a.l = a.l * sa + lb * sb;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) a.o[dt] = a.o[dt] * sa + ob[dt] * sb;
}

template <typename T, int D, int NQT>
__device__ __forceinline__ void attend_split(const StepArgs& a, const AttendLead& al, uint32_t* lds, int head,
                                             int split) {
  constexpr int TG = kAttendGroups;
  constexpr int NT = 64 * NQT * TG;
  constexpr int CH = attend_chunk(AttendTraits<T>::DT);
  constexpr int CW = CH / TG;                     // tokens of one wave per chunk
  constexpr int KS = D + AttendTraits<T>::KPAD;   // Ks row stride (elements)
  constexpr int VS = CH + AttendTraits<T>::VPAD;  // Vt row stride (elements)
  constexpr int VE = 16 / sizeof(T);              // elements per 16-byte vector
  constexpr int NV = D / VE;                      // vectors per row
  constexpr int PER = (CH * NV + NT - 1) / NT;    // vectors per thread per tensor
  static_assert(CW % 16 == 0 && (sizeof(T) != 2 || CW % 32 == 0), "whole MFMA tiles per wave");
  int* tlist = reinterpret_cast<int*>(lds);        // this split's part of T (kept prompt tokens, then gen_idx)
  uint32_t* scratch = lds + a.att_t_words;         // K/V buffers, merge slots
  T* Ks = reinterpret_cast<T*>(scratch);
  T* Vt = Ks + CH * KS;

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int qt = w / TG, tg = w - qt * TG;
  const int g = lane >> 4, l16 = lane & 15;
  const int query = 16 * qt + l16;
  const bool qvalid = query < a.n_q;
  const HeadRef hr = head_ref(al.n_items, al.heads_per_item, head);
  const T* kh = reinterpret_cast<const T*>(a.k[hr.item]) + hr.local * al.n_tot * D;
  const T* vh = reinterpret_cast<const T*>(a.v[hr.item]) + hr.local * al.n_tot * D;

  // the attended tokens of this split: T positions [t0, t_end), in nck chunks
  // (prompt splits first, then the generated positions' splits)
  const bool gen_part = split >= al.n_split_p;
  const int cps = gen_part ? al.cps_g : al.cps_p;
  const int t0 = gen_part ? al.k0 + (split - al.n_split_p) * cps * CH : split * cps * CH;
  const int t_end = min(gen_part ? al.n_att : al.k0, t0 + cps * CH);
  const int tcount = max(0, t_end - t0);
  const int nck = (tcount + CH - 1) / CH;
  for (int i = threadIdx.x; i < tcount; i += NT) {
    const int gi = t0 + i;
    tlist[i] = clampi(gi < al.k0 ? al.sel_in[(int64_t)head * al.k0 + gi] : al.gen_idx[gi - al.k0], 0, al.n_tot - 1);
  }
  // this wave's query fragment, requested after the token list (which the
  // gathers wait for) and in flight during the first chunk's gathers
  Frag<T, D> qf;
  const T* qh = reinterpret_cast<const T*>(a.q[hr.item]) + hr.local * a.n_q * D;
  if (qvalid) qf.load(qh + (int64_t)query * D, g); else qf.zero();
  __syncthreads();

  const float sl2 = a.inv_sqrt_d * 1.44269504088896340736f;  // log2(e)/sqrt(d)
  SoftmaxState<D> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // K and V: vector e = (row, cv) of the chunk, row-major, so each wave-wide
  // load reads whole rows.  K rows go to LDS as they are.  bfloat16 V goes to
  // LDS transposed (V^T, d-major) as 32-bit words holding one element of two
  // consecutive tokens: the lanes holding rows 2p and 2p + 1 at the same
  // column block (lanes l and l ^ NV) swap half their vector, then each writes
  // four words.  V^T word column p of d-row d is stored at p ^ vswz(d), an XOR
  // swizzle that keeps these stores and the 8-byte fragment reads below free
  // of bank conflicts.  Vectors e >= CH * NV (when NT does not divide the
  // chunk) are idle; pair partners e and e ^ NV are both idle or both not, and
  // every lane takes part in the swap.
  static_assert(NV <= 32 && NT % (2 * NV) == 0, "pair partners within one wave");
  constexpr int VW = VS / 2;               // V^T words per d-row (bfloat16)
  constexpr int VSWM = (CH / 2 - 1) & ~1;  // swizzle keeps columns inside [0, CH/2)
  auto vswz = [](int d) { return ((d >> 2) * 2) & VSWM; };
  u32x4 kreg[PER], vreg[PER];
  auto fetch = [&](int chunk) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = threadIdx.x + i * NT;
      const int row = e / NV, cv = e - row * NV;
      const int pos = t0 + chunk * CH + row;
      kreg[i] = u32x4{0u, 0u, 0u, 0u};
      vreg[i] = u32x4{0u, 0u, 0u, 0u};
      if (e < CH * NV && pos < t_end) {  // plain loads: the non-temporal hint slows scattered row gathers
        const int64_t tok = tlist[pos - t0];
        kreg[i] = *reinterpret_cast<const u32x4*>(kh + tok * D + cv * VE);
        vreg[i] = *reinterpret_cast<const u32x4*>(vh + tok * D + cv * VE);
      }
    }
  };
  if (nck > 0) fetch(0);
  for (int chunk = 0; chunk < nck; ++chunk) {  // chunk: index within this split
    const int pos0 = t0 + chunk * CH + tg * CW;  // first token of this wave's slice
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = threadIdx.x + i * NT;
      const int row = e / NV, cv = e - row * NV;
      const bool act = e < CH * NV;
      if (act) *reinterpret_cast<u32x4*>(Ks + row * KS + cv * VE) = kreg[i];
      if constexpr (sizeof(T) != 2) {
        if (act)
#pragma unroll
          for (int c = 0; c < 4; ++c) Vt[(cv * VE + c) * VS + row] = __uint_as_float(vreg[i][c]);
      } else {
        const u32x4 x = vreg[i];
        const bool odd = row & 1;  // odd rows write elements 4..7 of the pair, even rows 0..3
        const uint32_t r0 = lane_xor_nv<NV>(odd ? x[0] : x[2]);
        const uint32_t r1 = lane_xor_nv<NV>(odd ? x[1] : x[3]);
        const uint32_t lo0 = odd ? r0 : x[0], hi0 = odd ? x[2] : r0;  // element pairs (row 2p, row 2p + 1)
        const uint32_t lo1 = odd ? r1 : x[1], hi1 = odd ? x[3] : r1;
        const uint32_t w4[4] = {(lo0 & 0xFFFFu) | (hi0 << 16), (lo0 >> 16) | (hi0 & 0xFFFF0000u),
                                (lo1 & 0xFFFFu) | (hi1 << 16), (lo1 >> 16) | (hi1 & 0xFFFF0000u)};
        uint32_t* vw = reinterpret_cast<uint32_t*>(Vt);
        const int pcol = row >> 1, d0 = cv * VE + (odd ? 4 : 0);
        if (act)
#pragma unroll
          for (int c = 0; c < 4; ++c) vw[(d0 + c) * VW + (pcol ^ vswz(d0 + c))] = w4[c];
      }
    }
    __syncthreads();
    if (chunk + 1 < nck) fetch(chunk + 1);  // overlaps with the math below

    if (pos0 < t_end) {  // wave-uniform: a slice wholly past the end has no work
      f32x4 sv[CW / 16];
#pragma unroll
      for (int t = 0; t < CW / 16; ++t) {
        Frag<T, D> kf;
        kf.load(Ks + (tg * CW + 16 * t + l16) * KS, g);
        sv[t] = mma_tile<D>(kf, qf, f32x4{0.f, 0.f, 0.f, 0.f});
      }
      if (pos0 + CW > t_end) {  // wave-uniform: only a split's last chunk has positions past its end
#pragma unroll
        for (int t = 0; t < CW / 16; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (pos0 + 16 * t + 4 * g + r >= t_end) sv[t][r] = -INFINITY;
      }
      float cmax = -INFINITY;
#pragma unroll
      for (int t = 0; t < CW / 16; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) cmax = fmaxf(cmax, sv[t][r]);
      // the scaled maximum (rounding is monotone: it is the maximum of the scaled scores)
      cmax = wave_max_xor_16_32(cmax) * sl2;
      const float m_new = fmaxf(st.m, cmax);  // finite: the slice holds a valid token
      // p = 2^(s sl2 - m), a single v_exp_f32 each: weights below 2^-126 of the
      // running maximum flush to zero
      const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
      float psum = 0.f;
#pragma unroll
      for (int t = 0; t < CW / 16; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sv[t][r], sl2, -m_new));
          sv[t][r] = p;
          psum += p;
        }
      st.l = st.l * alpha + psum;
      st.m = m_new;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) st.o[dt] *= alpha;

      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int s2 = 0; s2 < CW / 32; ++s2) {
          u32x4 ph, pl;
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const f32x4 p = sv[2 * s2 + hh];
            { const Bf16Split t = split_pk_bf16(p[0], p[1]); ph[2 * hh] = t.hi; pl[2 * hh] = t.lo; }
            { const Bf16Split t = split_pk_bf16(p[2], p[3]); ph[2 * hh + 1] = t.hi; pl[2 * hh + 1] = t.lo; }
          }
          // V^T rows d, tokens tg CW + 32 s2 + 4 g + [0,4) and + 16 (word columns c0, c0 + 8)
          const int c0 = (tg * CW) / 2 + 16 * s2 + 2 * g;
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt) {
            const int d = 16 * dt + l16;
            const uint32_t* vr = reinterpret_cast<const uint32_t*>(Vt) + d * VW;
            const u32x2 v0 = *reinterpret_cast<const u32x2*>(vr + (c0 ^ vswz(d)));
            const u32x2 v1 = *reinterpret_cast<const u32x2*>(vr + ((c0 + 8) ^ vswz(d)));
            const u32x4 vf = {v0[0], v0[1], v1[0], v1[1]};
            st.o[dt] = mma_bf16(vf, ph, st.o[dt]);
            st.o[dt] = mma_bf16(vf, pl, st.o[dt]);
          }
        }
      } else {
#pragma unroll
        for (int t = 0; t < CW / 16; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
              const float vf = Vt[(16 * dt + l16) * VS + tg * CW + 16 * t + 4 * g + r];
              st.o[dt] = mma_f32(vf, sv[t][r], st.o[dt]);
            }
      }
    }
    __syncthreads();
  }

  // Row sums over the four lane groups, then a tree merge of the TG states of
  // each query tile through LDS (slots alias the K/V buffers).
  st.l = wave_sum_xor_16_32(st.l);
  constexpr int SLOT = 64 * (D / 4 + 2);  // floats per merge slot
  float* slots = reinterpret_cast<float*>(scratch);
#pragma unroll
  for (int half = TG / 2; half >= 1; half /= 2) {
    if (tg >= half && tg < 2 * half) {
      float* sl = slots + (qt * (TG / 2) + (tg - half)) * SLOT;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) reinterpret_cast<f32x4*>(sl)[dt * 64 + lane] = st.o[dt];
      reinterpret_cast<float2*>(sl + 64 * (D / 4))[lane] = make_float2(st.m, st.l);
    }
    __syncthreads();
    if (tg < half) {
      const float* sl = slots + (qt * (TG / 2) + tg) * SLOT;
      f32x4 ob[D / 16];
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) ob[dt] = reinterpret_cast<const f32x4*>(sl)[dt * 64 + lane];
      const float2 ml = reinterpret_cast<const float2*>(sl + 64 * (D / 4))[lane];
      merge_state<D>(st, ml.x, ml.y, ob);
    }
    __syncthreads();
  }
  if (tg == 0 && qvalid) {
    float* pml = a.part_ml + (((int64_t)head * a.n_split + split) * a.n_q + query) * 2;
    float* po = a.part_o + ((int64_t)head * a.n_split + split) * a.n_q * D + (int64_t)query * D;
    // non-temporal stores: the merge launch reads the partials (about 10 MB at
    // 64K) from memory, and they need not sit dirty in this XCD's L2 when the
    // launch ends (the small hand-offs between the other launches measured
    // slower this way: their readers then miss the caches)
    if (g == 0) __builtin_nontemporal_store(f32x2_t{st.m, st.l}, reinterpret_cast<f32x2_t*>(pml));
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      __builtin_nontemporal_store(st.o[dt], reinterpret_cast<f32x4*>(po + 16 * dt + 4 * g));
  }
}

template <typename T, int D, int NQT>
__global__ __launch_bounds__(64 * NQT * kAttendGroups, attend_waves_per_simd(NQT)) void attend_kernel(WF_LEAD_PARAMS,
                                                                                                    StepArgs a) {
  extern __shared__ __align__(16) uint32_t lds[];
  attend_split<T, D, NQT>(a, AttendLead::of(WF_LEAD), lds, blockIdx.y, blockIdx.x);
}

// The refinement of every head and the generated positions' attention
// splits in one launch, with the attention's workgroup size: workgroups
// [0, H) refine head blockIdx.x, the rest take the splits of the generated
// positions, which need no selection and so run beside the refinement.  The
// attention launch after it takes only the prompt splits.  No workgroup
// waits for another.
template <typename T, int D, int NQT, int S0>
__global__ __launch_bounds__(64 * NQT * kAttendGroups, attend_waves_per_simd(NQT)) void refine_gen_kernel(
    WF_LEAD_PARAMS, StepArgs a) {
  constexpr int NT = 64 * NQT * kAttendGroups;
  extern __shared__ __align__(16) uint32_t lds[];
  const RefineLead rl = RefineLead::of(WF_LEAD);
  const int H = rl.heads_total;
  if ((int)blockIdx.x < H) {
    const int head = blockIdx.x;
    // the kept coarse regions [k_L], then the selection state
    SelShared<NT>& sh = *reinterpret_cast<SelShared<NT>*>(lds + ((rl.k_top + 3) & ~3));
    refine_sel<NT, S0>(a, rl, head, reinterpret_cast<int*>(lds), sh);
    return;
  }
  const int ns_g = a.n_split - a.n_split_p;
  const int r = blockIdx.x - H;
  const int head = r / ns_g;
  attend_split<T, D, NQT>(a, attend_lead(a), lds, head, a.n_split_p + (r - head * ns_g));
}

// ---------------------------------------------------------------------------
// Merge of the split partials in a launch of its own:
// O = sum_s e^{m_s - M} O_s / sum_s e^{m_s - M} l_s, M = max_s m_s (m in
// log2 units; an empty split has m = -inf, l = 0).  Thread = one float4 of
// the output (head, query, 4 columns), so the merge is one round of
// independent loads spread over the whole chip; the splits are folded in
// index order.
// ---------------------------------------------------------------------------
#if !defined(WF_STEP_T)  // one compile unit holds it
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(WF_LEAD_PARAMS, StepArgs a) {
  constexpr int C4 = D / 4;
  const CombineLead cl = CombineLead::of(WF_LEAD);
  const int head = blockIdx.y;  // the grid's rows are the heads: no division by a run-time size
  const int rem = (int)blockIdx.x * 256 + (int)threadIdx.x;
  if (rem >= cl.n_q * C4) return;
  const int query = rem / C4, c4 = rem - query * C4;
  const int ns = cl.n_split;
  float mv[kMaxSplit], lv[kMaxSplit];
  float4 ov[kMaxSplit];
#pragma unroll
  for (int sp = 0; sp < kMaxSplit; ++sp) {  // every load issued before any is used
    mv[sp] = -INFINITY;
    lv[sp] = 0.f;
    ov[sp] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (sp < ns) {  // uniform: only the splits that exist are read
      const int64_t row = ((int64_t)head * ns + sp) * cl.n_q + query;
      const float2 ml = *reinterpret_cast<const float2*>(cl.part_ml + row * 2);
      mv[sp] = ml.x;
      lv[sp] = ml.y;
      ov[sp] = *reinterpret_cast<const float4*>(cl.part_o + row * D + 4 * c4);
    }
  }
  // the head's output rows, read from the arguments while the loads above are
  // in flight (read after them, the argument read would wait a trip of its own)
  const HeadRef hr = head_ref(a, head);
  float* const ob = a.out[hr.item] + (int64_t)hr.local * a.n_q * D;
  asm volatile("" ::"s"(ob));
  float mm = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < kMaxSplit; ++sp) mm = fmaxf(mm, mv[sp]);
  float den = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int sp = 0; sp < kMaxSplit; ++sp) {
    const float wv = (mv[sp] == -INFINITY) ? 0.f : exp2f(mv[sp] - mm);
    den += wv * lv[sp];
    acc.x += wv * ov[sp].x;
    acc.y += wv * ov[sp].y;
    acc.z += wv * ov[sp].z;
    acc.w += wv * ov[sp].w;
  }
  const float inv = 1.0f / den;
  *reinterpret_cast<float4*>(ob + query * D + 4 * c4) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}
#endif

// ---------------------------------------------------------------------------
// Launches.  This file is compiled once per (input type, head dimension,
// query tiles) with WF_STEP_T, WF_STEP_D and WF_STEP_RT set, each unit
// instantiating that combination's kernels (so the units build in
// parallel), and once without them for the dispatcher and the list-based
// refinement.
// ---------------------------------------------------------------------------
template <class K>
static hipError_t allow_lds(K kernel, int bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             bytes);
}

template <class K>
static hipError_t launch_one(K kernel, dim3 grid, dim3 block, int lds, hipStream_t s, const StepArgs& a) {
  hipError_t e = allow_lds(kernel, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kernel, grid, block, lds, s, a);
  return hipGetLastError();
}
template <class K>
static hipError_t launch_lead(K kernel, dim3 grid, dim3 block, int lds, hipStream_t s, const Lead& l,
                              const StepArgs& a) {
  hipError_t e = allow_lds(kernel, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kernel, grid, block, lds, s, l.p[0], l.p[1], l.p[2], l.i[0], l.i[1], l.i[2], l.i[3], l.i[4],
                     l.i[5], l.i[6], l.i[7], a);
  return hipGetLastError();
}

// The coarse and cover stages, for one (T, D, RT).
template <typename T, int D, int RT>
hipError_t launch_select(const StepArgs& a, const SelectLaunch& L, int stage, hipStream_t s) {
  const SelectPlan& P = L.plan;
  const int H = P.heads_total;
  if (stage == 0) {
    const dim3 coarse_grid(P.coarse_wg, H);
    const Lead ld{{a.a_top[0], a.q[0], nullptr}, {P.n_top, P.n_q, 0, 0, 0, 0, 0, 0}};
    if (L.n_items == 1)
      return L.agg_mean ? launch_lead(coarse_mean_kernel<T, D, RT, true>, coarse_grid, dim3(256), 0, s, ld, a)
                        : launch_lead(coarse_max_kernel<T, D, RT, true>, coarse_grid, dim3(256), 0, s, ld, a);
    return L.agg_mean ? launch_lead(coarse_mean_kernel<T, D, RT, false>, coarse_grid, dim3(256), 0, s, ld, a)
                      : launch_lead(coarse_max_kernel<T, D, RT, false>, coarse_grid, dim3(256), 0, s, ld, a);
  }
  hipError_t e;
  const dim3 cover_grid(P.cover_wg, H);
  const dim3 blk(kCoverThreads);
  const int lds = P.cover_lds;
  const Lead ld = cover_lead(a).lead();
  if (P.stored_bands)
    e = L.agg_mean ? launch_lead(cover_bands_mean_kernel<T, D, RT>, cover_grid, blk, lds, s, ld, a)
                   : launch_lead(cover_bands_max_kernel<T, D, RT>, cover_grid, blk, lds, s, ld, a);
  else
    e = L.agg_mean ? launch_lead(cover_mean_kernel<T, D, RT>, cover_grid, blk, lds, s, ld, a)
                   : launch_lead(cover_max_kernel<T, D, RT>, cover_grid, blk, lds, s, ld, a);
  return e;
}

// The attention stage, for one (T, D, RT): every split, or only the prompt
// splits when the refinement's launch took the generated ones.
template <typename T, int D, int RT>
hipError_t launch_attend(const StepArgs& a, const SelectLaunch& L, hipStream_t s) {
  const SelectPlan& P = L.plan;
  const bool gen_done = !L.attend_only && P.fuse_s0 > 0;
  return launch_lead(attend_kernel<T, D, RT>, dim3(gen_done ? P.n_split_p : P.n_split, P.heads_total),
                     dim3(64 * RT * kAttendGroups), P.attend_lds, s, attend_lead(a).lead(), a);
}

// The refinement with the generated positions' splits (refine_gen_kernel), for one (T, D, RT).
template <typename T, int D, int RT>
hipError_t launch_refine_gen(const StepArgs& a, const SelectLaunch& L, hipStream_t s) {
  const SelectPlan& P = L.plan;
  constexpr int NT = 64 * RT * kAttendGroups;
  const int refine_lds = 4 * ((P.k_top + 3) & ~3) + (int)sizeof(SelShared<NT>);
  const int lds = P.attend_lds > refine_lds ? P.attend_lds : refine_lds;
  const dim3 grid(P.heads_total * (1 + P.n_split - P.n_split_p));
  const Lead ld = refine_lead(a).lead();
  switch (P.fuse_s0) {
    case 1: return launch_lead(refine_gen_kernel<T, D, RT, 1>, grid, dim3(NT), lds, s, ld, a);
    case 2: return launch_lead(refine_gen_kernel<T, D, RT, 2>, grid, dim3(NT), lds, s, ld, a);
    case 4: return launch_lead(refine_gen_kernel<T, D, RT, 4>, grid, dim3(NT), lds, s, ld, a);
    default: return launch_lead(refine_gen_kernel<T, D, RT, 8>, grid, dim3(NT), lds, s, ld, a);
  }
}

#if defined(WF_STEP_T)
template hipError_t launch_select<WF_STEP_T, WF_STEP_D, WF_STEP_RT>(const StepArgs&, const SelectLaunch&, int,
                                                                    hipStream_t);
template hipError_t launch_attend<WF_STEP_T, WF_STEP_D, WF_STEP_RT>(const StepArgs&, const SelectLaunch&, hipStream_t);
template hipError_t launch_refine_gen<WF_STEP_T, WF_STEP_D, WF_STEP_RT>(const StepArgs&, const SelectLaunch&, hipStream_t);
#else
#define WF_EXTERN_SEL(T, D, RT) \
  extern template hipError_t launch_select<T, D, RT>(const StepArgs&, const SelectLaunch&, int, hipStream_t);
#define WF_EXTERN_ATT(T, D, RT) \
  extern template hipError_t launch_attend<T, D, RT>(const StepArgs&, const SelectLaunch&, hipStream_t);
#define WF_EXTERN_RG(T, D, RT) \
  extern template hipError_t launch_refine_gen<T, D, RT>(const StepArgs&, const SelectLaunch&, hipStream_t);
#define WF_EXTERN_STAGES(T, D)                                                              \
  WF_EXTERN_SEL(T, D, 1) WF_EXTERN_SEL(T, D, 2) WF_EXTERN_SEL(T, D, 3) WF_EXTERN_SEL(T, D, 4) \
  WF_EXTERN_ATT(T, D, 1) WF_EXTERN_ATT(T, D, 2) WF_EXTERN_ATT(T, D, 3) WF_EXTERN_ATT(T, D, 4) \
  WF_EXTERN_RG(T, D, 1) WF_EXTERN_RG(T, D, 2) WF_EXTERN_RG(T, D, 3) WF_EXTERN_RG(T, D, 4)
WF_EXTERN_STAGES(bf16_t, 128)
WF_EXTERN_STAGES(bf16_t, 64)
WF_EXTERN_STAGES(float, 128)
WF_EXTERN_STAGES(float, 64)
#undef WF_EXTERN_STAGES
#undef WF_EXTERN_SEL
#undef WF_EXTERN_ATT
#undef WF_EXTERN_RG

template <typename T, int D>
static hipError_t launch_rt_select(int rt, int stage, const StepArgs& a, const SelectLaunch& L, hipStream_t s) {
  hipError_t e = hipSuccess;
  {
    switch (rt) {
      case 1: e = launch_select<T, D, 1>(a, L, stage, s); break;
      case 2: e = launch_select<T, D, 2>(a, L, stage, s); break;
      case 3: e = launch_select<T, D, 3>(a, L, stage, s); break;
      default: e = launch_select<T, D, 4>(a, L, stage, s); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// The selection launches after the coarse one that some shapes need.
static hipError_t launch_apart(const StepArgs& a, const SelectLaunch& L, int stage, hipStream_t s) {
  const SelectPlan& P = L.plan;
  const dim3 grid(P.heads_total), block(kSelThreads);
  if (stage == 0) {  // between the coarse and the cover launches
    if (P.topk_s >= 1 && P.topk_s <= 4 && P.levels > 0 && !P.soft) return hipSuccess;  // the cover workgroups take it
    if (P.soft) {  // the level-L softmax scores first
      const hipError_t e = launch_one(soft_top_kernel, grid, block, 0, s, a);
      if (e != hipSuccess) return e;
    }
    return launch_one(coarse_topk_kernel, grid, block, P.coarse_lds, s, a);
  }
  if (P.levels == 0) return hipSuccess;  // between the cover and the attention launches
  const dim3 rblock(kRefineThreads);
  if (P.soft) {
    switch (P.refine_s0) {
      case 1: return launch_one(refine_soft_kernel<1>, grid, rblock, P.refine_soft_lds, s, a);
      case 2: return launch_one(refine_soft_kernel<2>, grid, rblock, P.refine_soft_lds, s, a);
      case 4: return launch_one(refine_soft_kernel<4>, grid, rblock, P.refine_soft_lds, s, a);
      default: return launch_one(refine_soft_kernel<8>, grid, rblock, P.refine_soft_lds, s, a);
    }
  }
  switch (P.refine_s0) {
    case 1: return launch_lead(refine_sel_kernel<1>, grid, rblock, P.cover_lds, s, refine_lead(a).lead(), a);
    case 2: return launch_lead(refine_sel_kernel<2>, grid, rblock, P.cover_lds, s, refine_lead(a).lead(), a);
    case 4: return launch_lead(refine_sel_kernel<4>, grid, rblock, P.cover_lds, s, refine_lead(a).lead(), a);
    case 8: return launch_lead(refine_sel_kernel<8>, grid, rblock, P.cover_lds, s, refine_lead(a).lead(), a);
    default: return launch_one(refine_lists_kernel, grid, block, P.refine_lds, s, a);
  }
}

template <typename T, int D>
static hipError_t launch_rt_attend(int rt, const StepArgs& a, const SelectLaunch& L, hipStream_t s) {
  switch (rt) {
    case 1: return launch_attend<T, D, 1>(a, L, s);
    case 2: return launch_attend<T, D, 2>(a, L, s);
    case 3: return launch_attend<T, D, 3>(a, L, s);
    default: return launch_attend<T, D, 4>(a, L, s);
  }
}

template <typename T, int D>
static hipError_t launch_rt_refine_gen(int rt, const StepArgs& a, const SelectLaunch& L, hipStream_t s) {
  switch (rt) {
    case 1: return launch_refine_gen<T, D, 1>(a, L, s);
    case 2: return launch_refine_gen<T, D, 2>(a, L, s);
    case 3: return launch_refine_gen<T, D, 3>(a, L, s);
    default: return launch_refine_gen<T, D, 4>(a, L, s);
  }
}

hipError_t launch_select_attend(const SelectLaunch& L, hipStream_t s) {
  const SelectPlan& P = L.plan;
  StepArgs a;
  a.n_items = L.n_items;
  a.heads_per_item = L.heads_per_item;
  for (int i = 0; i < kMaxItems; ++i) {
    const bool in = i < L.n_items;
    a.q[i] = in ? L.q[i] : nullptr;
    a.a_top[i] = in ? L.a_top[i] : nullptr;
    a.k[i] = in ? L.k[i] : nullptr;
    a.v[i] = in ? L.v[i] : nullptr;
    a.out[i] = in ? L.out[i] : nullptr;
    a.sel_out[i] = in ? L.sel_out[i] : nullptr;
  }
  a.gen_idx = L.gen_idx;
  a.sel_ws = reinterpret_cast<int32_t*>(L.ws + P.off_sel);
  a.sel_in = L.attend_only ? L.sel_in : a.sel_ws;
  a.sel_levels = L.sel_levels;
  a.score_levels = L.score_levels;
  a.keys_top = reinterpret_cast<uint32_t*>(L.ws + P.off_keys);
  a.sel_top = reinterpret_cast<int32_t*>(L.ws + P.off_sel_top);
  a.cov = reinterpret_cast<float*>(L.ws + P.off_cov);
  a.lvl_mm = reinterpret_cast<uint32_t*>(L.ws + P.off_lvl);
  a.part_ml = reinterpret_cast<float*>(L.ws + P.off_part_ml);
  a.part_o = reinterpret_cast<float*>(L.ws + P.off_part_o);
  a.heads_total = P.heads_total;
  a.n_q = P.n_q;
  a.n_top = P.n_top;
  a.n_prompt = P.n_prompt;
  a.n_tot = P.n_tot;
  a.n_gen = P.n_gen;
  a.levels = P.levels;
  a.k_top = P.k_top;
  a.k0 = P.k0;
  a.sum_k = P.sum_k;
  a.covered = P.covered;
  a.cov_len = P.cov_len;
  for (int j = 0; j < kMaxLevels; ++j) a.cov_off[j] = P.cov_off[j];
  for (int j = 0; j <= kMaxLevels; ++j) a.budgets[j] = P.budgets[j];
  a.n_att = P.n_att;
  a.n_split = P.n_split;
  a.n_split_p = P.n_split_p;
  a.cps_p = P.cps_p;
  a.cps_g = P.cps_g;
  a.att_t_words = P.att_t_words;
  a.topk_s = P.topk_s;
  a.coarse_keys_in_lds = P.coarse_keys_in_lds;
  a.refine_s0 = P.refine_s0;
  a.refine_cov_in_lds = P.refine_cov_in_lds;
  a.refine_nmax = P.refine_nmax;
  a.refine_kmax = P.refine_kmax;
  a.inv_sqrt_d = 1.0f / sqrtf((float)P.head_dim);
  a.inv_nq = 1.0f / (float)P.n_q;
  a.stored_bands = P.stored_bands;
  a.soft = P.soft;
  a.n_top4 = P.n_top4;
  a.logits = reinterpret_cast<float*>(L.ws + P.off_logits);
  for (int j = 0; j < kMaxLevels; ++j)
    a.band_a[j] = P.stored_bands && j > 0 && j < P.levels
                      ? reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(L.a_top[0]) + P.band_off[j])
                      : nullptr;

  const int rt = (P.n_q + 15) / 16;
  const bool bf = P.dtype == WF_BF16;
  const bool d128 = P.head_dim == 128;
  hipError_t e;
  if (!L.attend_only) {
    for (int stage = 0; stage < 2; ++stage) {
      if (stage == 1 && P.levels == 0) break;
      e = bf ? (d128 ? launch_rt_select<bf16_t, 128>(rt, stage, a, L, s) : launch_rt_select<bf16_t, 64>(rt, stage, a, L, s))
             : (d128 ? launch_rt_select<float, 128>(rt, stage, a, L, s) : launch_rt_select<float, 64>(rt, stage, a, L, s));
      if (e != hipSuccess) return e;
      if (stage == 1 && P.fuse_s0 > 0)  // the refinement with the generated positions' splits
        e = bf ? (d128 ? launch_rt_refine_gen<bf16_t, 128>(rt, a, L, s) : launch_rt_refine_gen<bf16_t, 64>(rt, a, L, s))
               : (d128 ? launch_rt_refine_gen<float, 128>(rt, a, L, s) : launch_rt_refine_gen<float, 64>(rt, a, L, s));
      else
        e = launch_apart(a, L, stage, s);
      if (e != hipSuccess) return e;
    }
  }
  e = bf ? (d128 ? launch_rt_attend<bf16_t, 128>(rt, a, L, s) : launch_rt_attend<bf16_t, 64>(rt, a, L, s))
         : (d128 ? launch_rt_attend<float, 128>(rt, a, L, s) : launch_rt_attend<float, 64>(rt, a, L, s));
  if (e != hipSuccess) return e;
  const dim3 comb_grid((unsigned)((P.n_q * (P.head_dim / 4) + 255) / 256), (unsigned)P.heads_total);
  const Lead ld = combine_lead(a).lead();
  return d128 ? launch_lead(combine_kernel<128>, comb_grid, dim3(256), 0, s, ld, a)
              : launch_lead(combine_kernel<64>, comb_grid, dim3(256), 0, s, ld, a);
}
#endif

}  // namespace wf
