// C ABI of the WaveFilter library: argument checks, buffer layout, launch.
// Every check runs on the host before anything is enqueued.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/wavefilter.h"
#include "wf_internal.h"

namespace {

constexpr uint32_t kPyramidMagic = 0x57465059u;  // "WFPY"
constexpr uint64_t kAlign = 256;

uint64_t align_up(uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
int pow2_at_least(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}
int elem_bytes(int dtype) { return dtype == WF_BF16 ? 2 : 4; }

bool valid_pyramid_shape(int32_t batch, int32_t heads, int32_t n_prompt, int32_t head_dim, int32_t levels) {
  if (batch < 1 || heads < 1 || n_prompt < 1) return false;
  if ((int64_t)batch * heads > WF_MAX_HEADS) return false;
  if (head_dim != 64 && head_dim != 128) return false;
  if (levels < 0 || levels > WF_MAX_LEVELS) return false;
  if (n_prompt % (1 << levels) != 0) return false;
  return true;
}

uint64_t band_bytes(int64_t heads_total, int32_t n_prompt, int32_t head_dim, int j) {
  return align_up((uint64_t)heads_total * (uint64_t)(n_prompt >> j) * (uint64_t)head_dim * 4u);
}

// Offsets of every stored band; returns the total size.
uint64_t pyramid_layout(int64_t heads_total, int32_t n_prompt, int32_t head_dim, int32_t levels, uint32_t flags,
                        uint64_t* off_a, uint64_t* off_d) {
  for (int j = 0; j <= WF_MAX_LEVELS; ++j) {
    off_a[j] = UINT64_MAX;
    off_d[j] = UINT64_MAX;
  }
  off_a[levels] = 0;
  uint64_t off = band_bytes(heads_total, n_prompt, head_dim, levels);
  if (flags & (WF_PYR_ALL_LEVELS | WF_PYR_DB2)) {
    for (int j = 1; j <= levels; ++j) {
      off_d[j] = off;
      off += band_bytes(heads_total, n_prompt, head_dim, j);
    }
    for (int j = 1; j < levels; ++j) {
      off_a[j] = off;
      off += band_bytes(heads_total, n_prompt, head_dim, j);
    }
  }
  return off;
}

bool pyramid_ok(const wf_pyramid* p) {
  return p && p->magic == kPyramidMagic && p->base &&
         valid_pyramid_shape(p->batch, p->heads, p->n_prompt, p->head_dim, p->levels) &&
         (p->dtype == WF_F32 || p->dtype == WF_BF16);
}

// Resolve budgets and the workspace layout for n_items layers of the
// pyramid's shape; returns a status.
int make_plan(const wf_pyramid* pyr, int32_t n_q, int32_t n_gen, const int32_t* budgets, wf::SelectPlan* P,
              int32_t n_items = 1, int32_t aggregation = WF_AGG_MAX) {
  if (!pyramid_ok(pyr)) return pyr ? WF_ERR_PYRAMID : WF_ERR_NULL;
  if (!budgets) return WF_ERR_NULL;
  if (n_q < 1 || n_q > WF_MAX_QUERIES || n_gen < 0) return WF_ERR_SHAPE;
  if (n_items < 1 || n_items > WF_MAX_LAYER_ITEMS) return WF_ERR_SHAPE;
  if ((int64_t)n_items * pyr->batch * pyr->heads > WF_MAX_HEADS) return WF_ERR_SHAPE;
  if (aggregation < WF_AGG_MAX || aggregation > WF_AGG_SOFTMAX_MEAN) return WF_ERR_OPTION;
  memset(P, 0, sizeof(*P));
  const int L = pyr->levels;
  P->heads_total = n_items * pyr->batch * pyr->heads;
  P->soft = aggregation == WF_AGG_SOFTMAX_MAX ? 1 : (aggregation == WF_AGG_SOFTMAX_MEAN ? 2 : 0);
  // softmax scores: one layer per call, Haar pyramids without stored bands
  if (P->soft && (n_items != 1 || (pyr->flags & WF_PYR_DB2))) return WF_ERR_OPTION;
  P->n_q = n_q;
  P->n_prompt = pyr->n_prompt;
  P->n_top = pyr->n_prompt >> L;
  P->head_dim = pyr->head_dim;
  P->dtype = pyr->dtype;
  P->levels = L;
  P->n_gen = n_gen;
  // budgets: 1 <= k_L <= n_L ; 1 <= k_j <= min(2 k_{j+1}, n_j)
  int kmax = 0, nmax = 0;
  int64_t sum_k = 0;
  for (int i = 0; i <= L; ++i) {
    const int j = L - i;
    const int64_t k = budgets[i];
    const int64_t n_j = pyr->n_prompt >> j;
    const int64_t cap = (i == 0) ? n_j : (2 * (int64_t)budgets[i - 1] < n_j ? 2 * (int64_t)budgets[i - 1] : n_j);
    if (k < 1 || k > cap) return WF_ERR_BUDGET;
    P->budgets[i] = (int)k;
    sum_k += k;
    if (k > kmax) kmax = (int)k;
    if (i < L && 2 * k > nmax) nmax = (int)(2 * k);
  }
  P->k_top = P->budgets[0];
  P->k0 = P->budgets[L];
  P->sum_k = (int)sum_k;
  if (P->k_top > wf::kMaxKeepTop) return WF_ERR_BUDGET;
  // the attended set T (kept tokens + generated positions) is indexed in int
  // and chunked per split: same bound as the attention-only plan
  if ((int64_t)P->k0 + n_gen > (1 << 24)) return WF_ERR_SHAPE;
  P->covered = (int64_t)P->k_top << L;
  int64_t off = 0;
  for (int j = 0; j < L; ++j) {  // level arrays start on 16-byte boundaries
    P->cov_off[j] = off;
    off += ((P->covered >> j) + 3) / 4 * 4;
  }
  P->cov_len = off;
  // coarse launch: 64 regions per workgroup; the head's last workgroup takes
  // the Top-K in registers (up to 8 192 regions), else with the keys in LDS
  // or read from memory
  P->coarse_wg = (P->n_top + 63) / 64;
  P->topk_s = P->n_top <= wf::kRegSelMax ? pow2_at_least((P->n_top + wf::kCoverThreads - 1) / wf::kCoverThreads) : 0;
  P->coarse_keys_in_lds = P->topk_s == 0 && P->n_top <= wf::kMaxCoarseLds;
  P->coarse_lds = P->coarse_keys_in_lds ? 4 * P->n_top : 0;
  // cover launch: 256 covered positions per workgroup, the kept coarse
  // regions in LDS.  The refinement runs in a launch of its own, one
  // workgroup of 1 024 threads per head holding 1 .. 8 level-0 positions
  // each (covered sets up to 8 192), else list-based
  P->cover_wg = L > 0 ? (int)((P->covered + wf::kCoverThreads - 1) / wf::kCoverThreads) : 0;
  P->cover_lds = 4 * ((P->k_top + 3) & ~3);
  P->refine_s0 = (L > 0 && P->covered <= 8 * wf::kRefineThreadsHost)
                     ? pow2_at_least((int)((P->covered + wf::kRefineThreadsHost - 1) / wf::kRefineThreadsHost))
                     : 0;
  // a longer basis: its finer approximation bands are read from the pyramid
  P->stored_bands = (pyr->flags & WF_PYR_DB2) != 0;
  if (P->stored_bands) {
    uint64_t off_a[WF_MAX_LEVELS + 1], off_d[WF_MAX_LEVELS + 1];
    pyramid_layout((int64_t)pyr->batch * pyr->heads, pyr->n_prompt, pyr->head_dim, pyr->levels, pyr->flags, off_a,
                   off_d);
    for (int j = 1; j < pyr->levels; ++j) P->band_off[j] = off_a[j];
  }
  // the refinement shares its launch with the generated positions'
  // attention splits where it fits (see gen_beside_fits), for the
  // in-register refinement with at most 8 covered positions per attention
  // thread and the maximum or mean over the query rows
  const int nt_att = 64 * ((n_q + 15) / 16) * wf::kAttendGroups;
  if (wf::gen_beside_fits(P) && L > 0 && !P->soft && P->refine_s0 > 0 && P->covered <= 8 * (int64_t)nt_att)
    P->fuse_s0 = pow2_at_least((int)((P->covered + nt_att - 1) / nt_att));
  // attention splits
  P->chunk = wf::attend_chunk(pyr->dtype);
  wf::plan_attention_splits(P, P->fuse_s0 > 0);
  if (!wf::attention_plan_ok(P)) return WF_ERR_SHAPE;
  // list-based refinement (one workgroup per head): the kept sets and
  // candidate lists, plus the coverage scores when they fit
  const int64_t budget = wf::kLdsLimit - wf::kTopKSharedReserve;
  if (L > 0 && P->refine_s0 == 0) {
    P->refine_nmax = (nmax + 3) / 4 * 4;
    P->refine_kmax = (kmax + 1 + 3) / 4 * 4;  // + a spare slot for rejected candidates
    const int64_t list_base = 4 * ((int64_t)P->refine_nmax + 2 * (int64_t)P->refine_kmax);
    if (list_base > budget) return WF_ERR_BUDGET;
    P->refine_cov_in_lds = (list_base + 4 * P->cov_len) <= budget;
    P->refine_lds = (int)(list_base + (P->refine_cov_in_lds ? 4 * P->cov_len : 0));
  }
  // attention workgroup LDS: the split's part of T, then the K/V chunk buffers
  const int64_t buf_bytes = wf::attend_buffer_bytes(pyr->dtype, pyr->head_dim, (n_q + 15) / 16);
  if (buf_bytes > wf::kLdsLimit - wf::kTopKSharedReserve - 4 * (int64_t)P->att_t_words) return WF_ERR_BUDGET;
  P->attend_lds = (int)(4 * (int64_t)P->att_t_words + buf_bytes);
  // workspace sections
  const uint64_t H = (uint64_t)P->heads_total;
  uint64_t w = wf::kStatusBytes;  // the debug status word comes first
  P->off_keys = w;     w += align_up(H * (uint64_t)P->n_top * 4);
  P->off_sel_top = w;  w += align_up(H * (uint64_t)P->k_top * 4);
  P->off_cov = w;      w += align_up(H * (uint64_t)(P->cov_len > 0 ? P->cov_len : 1) * 4);
  P->off_lvl = w;      w += align_up(H * (uint64_t)((P->covered + 63) / 64) * wf::kMaxLevels * 2 * 4);
  P->off_sel = w;      w += align_up(H * (uint64_t)(P->k0 > 0 ? P->k0 : 1) * 4);
  P->off_part_ml = w;  w += align_up(H * (uint64_t)P->n_split * 2 * n_q * 4);
  P->off_part_o = w;   w += align_up(H * (uint64_t)P->n_split * n_q * P->head_dim * 4);
  // softmax scores: every query row's logits, level L [n_q][n_top4] then
  // levels 0 .. L-1 [n_q][padded level length], per head; and the
  // refinement's LDS (kept coarse regions, the candidate list, row lse)
  P->n_top4 = (P->n_top + 3) & ~3;
  P->off_logits = w;
  if (P->soft) {
    if (L > 0 && P->refine_s0 == 0) return WF_ERR_BUDGET;  // covered sets beyond 8 192 positions
    w += align_up(H * (uint64_t)n_q * ((uint64_t)P->n_top4 + (uint64_t)P->cov_len) * 4);
    P->refine_soft_lds = (int)(4 * (((int64_t)P->k_top + 3) / 4 * 4 + P->covered + 64));
  }
  P->total = w;
  return WF_OK;
}

// Attention-only plan (a selection handed in): the chunking, split and LDS
// layout of the attention stage and the workspace sections it uses.
int make_attend_plan(int32_t batch, int32_t heads, int32_t head_dim, int32_t dtype, int32_t n_q, int32_t k0,
                     int32_t n_gen, wf::SelectPlan* P) {
  if (batch < 1 || heads < 1 || (int64_t)batch * heads > WF_MAX_HEADS) return WF_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return WF_ERR_SHAPE;
  if (dtype != WF_F32 && dtype != WF_BF16) return WF_ERR_DTYPE;
  if (n_q < 1 || n_q > WF_MAX_QUERIES || k0 < 0 || n_gen < 0 || (int64_t)k0 + n_gen < 1) return WF_ERR_SHAPE;
  if ((int64_t)k0 + n_gen > (1 << 24)) return WF_ERR_SHAPE;
  memset(P, 0, sizeof(*P));
  P->heads_total = batch * heads;
  P->n_q = n_q;
  P->head_dim = head_dim;
  P->dtype = dtype;
  P->k0 = k0;
  P->n_gen = n_gen;
  P->chunk = wf::attend_chunk(dtype);
  wf::plan_attention_splits(P, false);
  if (!wf::attention_plan_ok(P)) return WF_ERR_SHAPE;
  const int64_t budget = wf::kLdsLimit - wf::kTopKSharedReserve - 4 * (int64_t)P->att_t_words;
  const int64_t buf_bytes = wf::attend_buffer_bytes(dtype, head_dim, (n_q + 15) / 16);
  if (buf_bytes > budget) return WF_ERR_BUDGET;
  P->attend_lds = (int)(4 * (int64_t)P->att_t_words + buf_bytes);
  const uint64_t H = (uint64_t)P->heads_total;
  uint64_t w = wf::kStatusBytes;  // the debug status word comes first
  P->off_part_ml = w;  w += align_up(H * (uint64_t)P->n_split * 2 * n_q * 4);
  P->off_part_o = w;   w += align_up(H * (uint64_t)P->n_split * n_q * head_dim * 4);
  P->total = w;
  return WF_OK;
}

// The scan of WF_OPT_CHECK over one set of inputs (the status word is
// cleared by the caller once per call).
hipError_t check_inputs(const void* q, const void* k, const void* v, const wf_pyramid* pyr, int64_t heads_total,
                        int n_q, int n_tot, int head_dim, int dtype, const int32_t* gen_idx, int n_gen,
                        const int32_t* sel, int64_t n_sel, void* workspace, hipStream_t s) {
  wf::CheckArgs c;
  const int64_t es = elem_bytes(dtype);
  c.q = q;
  c.k = k;
  c.v = v;
  c.a_top = pyr ? reinterpret_cast<const float*>(pyr->base) : nullptr;
  c.q_bytes = heads_total * n_q * head_dim * es;
  c.kv_bytes = heads_total * (int64_t)n_tot * head_dim * es;
  c.a_bytes = pyr ? heads_total * (int64_t)(pyr->n_prompt >> pyr->levels) * head_dim * 4 : 0;
  c.gen_idx = n_gen > 0 ? gen_idx : nullptr;
  c.n_gen = n_gen;
  c.sel = n_sel > 0 ? sel : nullptr;
  c.n_sel = n_sel;
  c.n_tot = n_tot;
  c.bf16 = dtype == WF_BF16;
  c.status = reinterpret_cast<uint32_t*>(workspace);
  return wf::launch_check(c, s);
}

}  // namespace

// Scratch of wf_select_attend_noalloc: one array per device (each GPU holds
// its own copy at its own address), kept until the process ends.  Host code
// never uses this name as an address: it uses the pointer that
// hipGetSymbolAddress returns for the device.
static __device__ __align__(256) uint8_t scratch[WF_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices];  // device address of `scratch`, looked up once per device

// The device address of `scratch` on the device that owns `stream` (the
// current device for the null stream), looked up on first use with that
// device current.
int device_scratch(hipStream_t stream, void** ptr) {
  int dev = -1;
  if (stream) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return WF_ERR_HIP;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return WF_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxScratchDevices) return WF_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return WF_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return WF_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return WF_ERR_HIP;
    if (e != hipSuccess || !p) return WF_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return WF_OK;
}

}  // namespace

extern "C" {

const char* wf_version(void) { return "wavefilter-gfx950 0.1.0"; }

const char* wf_status_string(int status) {
  switch (status) {
    case WF_OK: return "ok";
    case WF_ERR_NULL: return "a required pointer is NULL";
    case WF_ERR_SHAPE: return "a size is out of range or inconsistent";
    case WF_ERR_DTYPE: return "unsupported or mismatched element type";
    case WF_ERR_LEVELS: return "level count out of range or prompt length not a multiple of 2^L";
    case WF_ERR_BUDGET: return "per-level keep counts infeasible or beyond the supported size";
    case WF_ERR_WORKSPACE: return "workspace or pyramid buffer too small";
    case WF_ERR_ALIGN: return "pointer or stride not 16-byte aligned";
    case WF_ERR_HIP: return "HIP launch or runtime call failed";
    case WF_ERR_PYRAMID: return "pyramid descriptor not built by wf_build_pyramid";
    case WF_ERR_OPTION: return "an option argument has no defined meaning";
    default: return "unknown status";
  }
}

uint64_t wf_pyramid_bytes(int32_t batch, int32_t heads, int32_t n_prompt, int32_t head_dim, int32_t levels,
                          uint32_t flags) {
  if (!valid_pyramid_shape(batch, heads, n_prompt, head_dim, levels)) return 0;
  if (flags & ~(WF_PYR_ALL_LEVELS | WF_PYR_DB2)) return 0;
  uint64_t off_a[WF_MAX_LEVELS + 1], off_d[WF_MAX_LEVELS + 1];
  return pyramid_layout((int64_t)batch * heads, n_prompt, head_dim, levels, flags, off_a, off_d);
}

uint64_t wf_pyramid_offset(const wf_pyramid* pyr, int32_t band, int32_t level) {
  if (!pyramid_ok(pyr) || level < 0 || level > pyr->levels || (band != 0 && band != 1)) return UINT64_MAX;
  uint64_t off_a[WF_MAX_LEVELS + 1], off_d[WF_MAX_LEVELS + 1];
  pyramid_layout((int64_t)pyr->batch * pyr->heads, pyr->n_prompt, pyr->head_dim, pyr->levels, pyr->flags, off_a,
                 off_d);
  return band == 0 ? off_a[level] : off_d[level];
}

int wf_build_pyramid(const void* k_prompt, int64_t head_stride, int32_t batch, int32_t heads, int32_t n_prompt,
                     int32_t head_dim, int32_t dtype, int32_t levels, uint32_t flags, void* pyr_mem,
                     uint64_t pyr_bytes, wf_pyramid* out, void* stream) {
  if (!k_prompt || !pyr_mem || !out) return WF_ERR_NULL;
  if (dtype != WF_F32 && dtype != WF_BF16) return WF_ERR_DTYPE;
  if (levels < 0 || levels > WF_MAX_LEVELS) return WF_ERR_LEVELS;
  if (n_prompt >= 1 && n_prompt % (1 << levels) != 0) return WF_ERR_LEVELS;
  if (!valid_pyramid_shape(batch, heads, n_prompt, head_dim, levels)) return WF_ERR_SHAPE;
  if (flags & ~(WF_PYR_ALL_LEVELS | WF_PYR_DB2)) return WF_ERR_OPTION;
  if (head_stride < (int64_t)n_prompt * head_dim) return WF_ERR_SHAPE;
  {
    // one workgroup per run of max(2^L, rows one wave-wide load covers) rows of a head
    const int64_t rpp = 64 / (head_dim / (dtype == WF_BF16 ? 8 : 4));
    const int64_t run = (1 << levels) > rpp ? (1 << levels) : rpp;
    if ((int64_t)batch * heads * ((n_prompt + run - 1) / run) > 0x7FFFFFFF) return WF_ERR_SHAPE;
  }
  if (!aligned16(k_prompt) || !aligned16(pyr_mem) || (head_stride * elem_bytes(dtype)) % 16 != 0)
    return WF_ERR_ALIGN;
  wf::PyramidLaunch a;
  const int64_t heads_total = (int64_t)batch * heads;
  const uint64_t need = pyramid_layout(heads_total, n_prompt, head_dim, levels, flags, a.band_off_a, a.band_off_d);
  if (pyr_bytes < need) return WF_ERR_WORKSPACE;
  a.k = k_prompt;
  a.head_stride = head_stride;
  a.heads_total = (int)heads_total;
  a.n_prompt = n_prompt;
  a.head_dim = head_dim;
  a.bf16 = dtype == WF_BF16;
  a.levels = levels;
  a.all_levels = (flags & (WF_PYR_ALL_LEVELS | WF_PYR_DB2)) != 0;
  a.db2 = (flags & WF_PYR_DB2) != 0;
  a.base = reinterpret_cast<float*>(pyr_mem);
  if (wf::launch_pyramid(a, reinterpret_cast<hipStream_t>(stream)) != hipSuccess) return WF_ERR_HIP;
  out->batch = batch;
  out->heads = heads;
  out->n_prompt = n_prompt;
  out->head_dim = head_dim;
  out->levels = levels;
  out->dtype = dtype;
  out->flags = flags;
  out->magic = kPyramidMagic;
  out->base = pyr_mem;
  out->bytes = pyr_bytes;
  return WF_OK;
}

int wf_refresh_pyramids(const wf_refresh_item* items, int32_t n_items, void* stream) {
  if (!items) return WF_ERR_NULL;
  if (n_items < 1 || n_items > WF_MAX_REFRESH_ITEMS) return WF_ERR_SHAPE;
  static_assert(WF_MAX_REFRESH_ITEMS == wf::kMaxRefreshItems, "refresh item capacity");
  wf::RefreshLaunch r;
  memset(&r, 0, sizeof(r));
  int64_t units = 0;
  for (int i = 0; i < n_items; ++i) {
    const wf_refresh_item& it = items[i];
    if (!it.k_prompt || !it.pyr) return WF_ERR_NULL;
    if (!pyramid_ok(it.pyr)) return WF_ERR_PYRAMID;
    if (it.pyr->flags & (WF_PYR_ALL_LEVELS | WF_PYR_DB2)) return WF_ERR_OPTION;  // stored finer bands are not refreshed
    if (i > 0 && (it.pyr->dtype != items[0].pyr->dtype || it.pyr->head_dim != items[0].pyr->head_dim))
      return WF_ERR_DTYPE;
    if (it.n_blocks < 0) return WF_ERR_SHAPE;
    if (it.n_blocks > 0 && !it.blocks) return WF_ERR_NULL;
    if (it.head_stride < (int64_t)it.pyr->n_prompt * it.pyr->head_dim) return WF_ERR_SHAPE;
    if (!aligned16(it.k_prompt) || (it.head_stride * elem_bytes(it.pyr->dtype)) % 16 != 0 ||
        (it.blocks && !aligned4(it.blocks)))
      return WF_ERR_ALIGN;
    wf::RefreshItem& d = r.items[i];
    d.k = it.k_prompt;
    d.head_stride = it.head_stride;
    d.a_top = reinterpret_cast<float*>(it.pyr->base);  // A_L sits at offset 0 of the pyramid buffer
    d.blocks = it.blocks;
    d.unit_begin = units;
    d.n_blocks = it.n_blocks;
    d.n_top = it.pyr->n_prompt >> it.pyr->levels;
    d.levels = it.pyr->levels;
    const int L = it.pyr->levels;
    d.scale = (float)ldexp(1.0, -L / 2) * ((L & 1) ? 0.70710678118654752440f : 1.0f);
    units += (int64_t)it.n_blocks * it.pyr->batch * it.pyr->heads;
  }
  r.n_items = n_items;
  r.head_dim = items[0].pyr->head_dim;
  r.bf16 = items[0].pyr->dtype == WF_BF16;
  r.units_total = units;
  if (units > 0x7FFFFFFF) return WF_ERR_SHAPE;  // one workgroup per (item, head, listed block)
  if (wf::launch_refresh(r, reinterpret_cast<hipStream_t>(stream)) != hipSuccess) return WF_ERR_HIP;
  return WF_OK;
}

uint64_t wf_select_attend_workspace_bytes(const wf_pyramid* pyr, int32_t n_q, int32_t n_gen,
                                          const int32_t* budgets, int32_t aggregation) {
  wf::SelectPlan P;
  if (make_plan(pyr, n_q, n_gen, budgets, &P, 1, aggregation & ~WF_OPT_CHECK) != WF_OK) return 0;
  return P.total;
}

int wf_select_attend(const void* q, const wf_pyramid* pyr, const void* k, const void* v, int32_t n_tot,
                     const int32_t* gen_idx, int32_t n_gen, const int32_t* budgets, int32_t n_q,
                     int32_t aggregation, float* out, int32_t* sel_out, int32_t* sel_levels, float* score_levels,
                     void* workspace, uint64_t ws_bytes, void* stream) {
  if (!q || !pyr || !k || !v || !out || !workspace || !budgets) return WF_ERR_NULL;
  if (n_gen > 0 && !gen_idx) return WF_ERR_NULL;
  const bool check = (aggregation & WF_OPT_CHECK) != 0;
  aggregation &= ~WF_OPT_CHECK;
  if (aggregation < WF_AGG_MAX || aggregation > WF_AGG_SOFTMAX_MEAN) return WF_ERR_OPTION;
  wf::SelectPlan P;
  const int st = make_plan(pyr, n_q, n_gen, budgets, &P, 1, aggregation);
  if (st != WF_OK) return st;
  if (n_tot < pyr->n_prompt || n_tot < 1) return WF_ERR_SHAPE;
  P.n_tot = n_tot;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(workspace) ||
      !aligned16(pyr->base))
    return WF_ERR_ALIGN;
  if ((gen_idx && !aligned4(gen_idx)) || (sel_out && !aligned4(sel_out)) || (sel_levels && !aligned4(sel_levels)) ||
      (score_levels && !aligned4(score_levels)))
    return WF_ERR_ALIGN;
  if (ws_bytes < P.total) return WF_ERR_WORKSPACE;
  wf::SelectLaunch a;
  a.plan = P;
  a.n_items = 1;
  a.heads_per_item = P.heads_total;
  a.q[0] = q;
  a.a_top[0] = reinterpret_cast<const float*>(pyr->base);
  a.k[0] = k;
  a.v[0] = v;
  a.out[0] = out;
  a.sel_out[0] = sel_out;
  a.gen_idx = gen_idx;
  a.sel_in = nullptr;
  a.attend_only = 0;
  a.agg_mean = aggregation == WF_AGG_MEAN;
  a.sel_levels = sel_levels;
  a.score_levels = score_levels;
  a.ws = reinterpret_cast<uint8_t*>(workspace);
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (check && (wf::launch_check_clear(reinterpret_cast<uint32_t*>(workspace), s) != hipSuccess ||
                check_inputs(q, k, v, pyr, P.heads_total, n_q, n_tot, pyr->head_dim, pyr->dtype, gen_idx, n_gen,
                             nullptr, 0, workspace, s) != hipSuccess))
    return WF_ERR_HIP;
  if (wf::launch_select_attend(a, s) != hipSuccess) return WF_ERR_HIP;
  return WF_OK;
}

int wf_select_attend_noalloc(const void* q, const wf_pyramid* pyr, const void* k, const void* v, int32_t n_tot,
                             const int32_t* gen_idx, int32_t n_gen, const int32_t* budgets, int32_t n_q,
                             int32_t aggregation, float* out, int32_t* sel_out, int32_t* sel_levels,
                             float* score_levels, void* stream) {
  if (!q || !pyr || !k || !v || !out || !budgets) return WF_ERR_NULL;
  wf::SelectPlan P;
  const int st = make_plan(pyr, n_q, n_gen, budgets, &P, 1, aggregation & ~WF_OPT_CHECK);
  if (st != WF_OK) return st;
  if (P.total > WF_NOALLOC_SCRATCH_BYTES) return WF_ERR_WORKSPACE;
  void* ws = nullptr;
  const int sst = device_scratch(reinterpret_cast<hipStream_t>(stream), &ws);
  if (sst != WF_OK) return sst;
  return wf_select_attend(q, pyr, k, v, n_tot, gen_idx, n_gen, budgets, n_q, aggregation, out, sel_out, sel_levels,
                          score_levels, ws, WF_NOALLOC_SCRATCH_BYTES, stream);
}

uint64_t wf_select_attend_layers_workspace_bytes(const wf_pyramid* pyr, int32_t n_items, int32_t n_q, int32_t n_gen,
                                                 const int32_t* budgets) {
  wf::SelectPlan P;
  if (pyr && (pyr->flags & (WF_PYR_ALL_LEVELS | WF_PYR_DB2))) return 0;
  if (make_plan(pyr, n_q, n_gen, budgets, &P, n_items) != WF_OK) return 0;
  return P.total;
}

int wf_select_attend_layers(const wf_layer_item* items, int32_t n_items, int32_t n_tot, const int32_t* gen_idx,
                            int32_t n_gen, const int32_t* budgets, int32_t n_q, int32_t aggregation, void* workspace,
                            uint64_t ws_bytes, void* stream) {
  if (!items || !workspace || !budgets) return WF_ERR_NULL;
  if (n_items < 1 || n_items > WF_MAX_LAYER_ITEMS) return WF_ERR_SHAPE;
  if (n_gen > 0 && !gen_idx) return WF_ERR_NULL;
  const bool check = (aggregation & WF_OPT_CHECK) != 0;
  aggregation &= ~WF_OPT_CHECK;
  if (aggregation != WF_AGG_MAX && aggregation != WF_AGG_MEAN) return WF_ERR_OPTION;
  const wf_pyramid* p0 = items[0].pyr;
  for (int i = 0; i < n_items; ++i) {
    const wf_layer_item& it = items[i];
    if (!it.q || !it.pyr || !it.k || !it.v || !it.out) return WF_ERR_NULL;
    if (!pyramid_ok(it.pyr)) return WF_ERR_PYRAMID;
    if (it.pyr->flags & (WF_PYR_ALL_LEVELS | WF_PYR_DB2)) return WF_ERR_OPTION;  // A_L-only Haar pyramids
    if (it.pyr->dtype != p0->dtype) return WF_ERR_DTYPE;
    if (it.pyr->batch != p0->batch || it.pyr->heads != p0->heads || it.pyr->n_prompt != p0->n_prompt ||
        it.pyr->head_dim != p0->head_dim || it.pyr->levels != p0->levels)
      return WF_ERR_SHAPE;
    if (!aligned16(it.q) || !aligned16(it.k) || !aligned16(it.v) || !aligned16(it.out) || !aligned16(it.pyr->base))
      return WF_ERR_ALIGN;
    if (it.sel_out && !aligned4(it.sel_out)) return WF_ERR_ALIGN;
  }
  wf::SelectPlan P;
  const int st = make_plan(p0, n_q, n_gen, budgets, &P, n_items);
  if (st != WF_OK) return st;
  if (n_tot < p0->n_prompt || n_tot < 1) return WF_ERR_SHAPE;
  P.n_tot = n_tot;
  if (!aligned16(workspace) || (gen_idx && !aligned4(gen_idx))) return WF_ERR_ALIGN;
  if (ws_bytes < P.total) return WF_ERR_WORKSPACE;
  wf::SelectLaunch a;
  a.plan = P;
  a.n_items = n_items;
  a.heads_per_item = p0->batch * p0->heads;
  for (int i = 0; i < n_items; ++i) {
    a.q[i] = items[i].q;
    a.a_top[i] = reinterpret_cast<const float*>(items[i].pyr->base);
    a.k[i] = items[i].k;
    a.v[i] = items[i].v;
    a.out[i] = items[i].out;
    a.sel_out[i] = items[i].sel_out;
  }
  a.gen_idx = gen_idx;
  a.sel_in = nullptr;
  a.attend_only = 0;
  a.agg_mean = aggregation == WF_AGG_MEAN;
  a.sel_levels = nullptr;
  a.score_levels = nullptr;
  a.ws = reinterpret_cast<uint8_t*>(workspace);
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (check) {
    if (wf::launch_check_clear(reinterpret_cast<uint32_t*>(workspace), s) != hipSuccess) return WF_ERR_HIP;
    for (int i = 0; i < n_items; ++i)
      if (check_inputs(items[i].q, items[i].k, items[i].v, items[i].pyr, a.heads_per_item, n_q, n_tot,
                       p0->head_dim, p0->dtype, i == 0 ? gen_idx : nullptr, i == 0 ? n_gen : 0, nullptr, 0,
                       workspace, s) != hipSuccess)
        return WF_ERR_HIP;
  }
  if (wf::launch_select_attend(a, s) != hipSuccess) return WF_ERR_HIP;
  return WF_OK;
}

uint64_t wf_attend_selected_workspace_bytes(int32_t batch, int32_t heads, int32_t head_dim, int32_t dtype,
                                            int32_t n_q, int32_t k0, int32_t n_gen) {
  wf::SelectPlan P;
  if (make_attend_plan(batch, heads, head_dim, dtype, n_q, k0, n_gen, &P) != WF_OK) return 0;
  return P.total;
}

int wf_attend_selected(const void* q, const void* k, const void* v, int32_t batch, int32_t heads, int32_t n_tot,
                       int32_t head_dim, int32_t dtype, const int32_t* sel, int32_t k0, const int32_t* gen_idx,
                       int32_t n_gen, int32_t n_q, int32_t options, float* out, void* workspace, uint64_t ws_bytes,
                       void* stream) {
  if (!q || !k || !v || !out || !workspace) return WF_ERR_NULL;
  if ((k0 > 0 && !sel) || (n_gen > 0 && !gen_idx)) return WF_ERR_NULL;
  if (options & ~WF_OPT_CHECK) return WF_ERR_OPTION;
  wf::SelectPlan P;
  const int st = make_attend_plan(batch, heads, head_dim, dtype, n_q, k0, n_gen, &P);
  if (st != WF_OK) return st;
  if (n_tot < 1) return WF_ERR_SHAPE;
  P.n_tot = n_tot;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(workspace)) return WF_ERR_ALIGN;
  if ((sel && !aligned4(sel)) || (gen_idx && !aligned4(gen_idx))) return WF_ERR_ALIGN;
  if (ws_bytes < P.total) return WF_ERR_WORKSPACE;
  wf::SelectLaunch a;
  a.plan = P;
  a.n_items = 1;
  a.heads_per_item = P.heads_total;
  a.q[0] = q;
  a.a_top[0] = nullptr;
  a.k[0] = k;
  a.v[0] = v;
  a.out[0] = out;
  a.sel_out[0] = nullptr;
  a.gen_idx = gen_idx;
  a.sel_in = sel;  // NULL when k0 == 0
  a.attend_only = 1;
  a.agg_mean = 0;
  a.sel_levels = nullptr;
  a.score_levels = nullptr;
  a.ws = reinterpret_cast<uint8_t*>(workspace);
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if ((options & WF_OPT_CHECK) &&
      (wf::launch_check_clear(reinterpret_cast<uint32_t*>(workspace), s) != hipSuccess ||
       check_inputs(q, k, v, nullptr, P.heads_total, n_q, n_tot, head_dim, dtype, gen_idx, n_gen, sel,
                    (int64_t)P.heads_total * k0, workspace, s) != hipSuccess))
    return WF_ERR_HIP;
  if (wf::launch_select_attend(a, s) != hipSuccess) return WF_ERR_HIP;
  return WF_OK;
}

int wf_check_status(const void* workspace, void* stream, uint32_t* status) {
  if (!status) return WF_ERR_NULL;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const void* src = workspace;
  if (!src) {
    void* p = nullptr;
    const int st = device_scratch(s, &p);
    if (st != WF_OK) return st;
    src = p;
  }
  if (hipMemcpyAsync(status, src, sizeof(uint32_t), hipMemcpyDeviceToHost, s) != hipSuccess) return WF_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return WF_ERR_HIP;
  return WF_OK;
}

}  // extern "C"
