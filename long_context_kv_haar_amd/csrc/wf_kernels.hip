// WaveFilter kernels for gfx950 (MI355X).
//
// Pyramid (per cache refresh):
//   pyramid_top_kernel    A_L of the prompt keys in one streaming pass
//   pyramid_level_kernel  one analysis level, for the all-levels inspection mode
// Per denoising step:
//   coarse_kernel   s_L = max_i q_i . A_L[n] / sqrt(d) on MFMA, then (last
//                   workgroup of each head) the coarse Top-K
//   cover_kernel    token scores q_i . k_t of every token covered by the kept
//                   coarse regions on MFMA, summed in registers into the
//                   scores of all their sub-regions at levels 0..L-1
//   refine_kernel   per head: child expansion + Top-K for j = L-1 .. 0
//   attend_kernel   split-K online-softmax attention over the kept prompt
//                   tokens plus the generated positions (QK^T and PV on
//                   MFMA, float32 accumulation), and (last workgroup of each
//                   head) the log-sum-exp merge of the partial results
//
// Citations are to WaveFilter (arXiv 2606.00724).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "wf_device.h"
#include "wf_internal.h"

namespace wf {

// ===========================================================================
// Pyramid: A_L[n] = 2^{-L/2} sum_{t in [n 2^L, (n+1) 2^L)} k_t
// (section 2.2, eq. 5 iterated L times with orthonormal Haar filters: the
// pairwise sums telescope into one block sum).  One wave owns a run of
// rows_per_item consecutive prompt rows; lane (r, col) streams 16-byte
// vectors of rows r, r + RPP, ... at column block col, so each wave-wide
// load reads 1 KiB of contiguous memory.  Row groups of one block are
// reduced with cross-lane shuffles.
// ===========================================================================
template <typename T> struct Vec16;
template <> struct Vec16<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void add(const float* p, float* acc) {
    float4 x = *reinterpret_cast<const float4*>(p);
    acc[0] += x.x; acc[1] += x.y; acc[2] += x.z; acc[3] += x.w;
  }
};
template <> struct Vec16<bf16_t> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void add(const bf16_t* p, float* acc) {
    u32x4 x = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += bf16_to_f32(x[i] & 0xFFFFu);
      acc[2 * i + 1] += bf16_to_f32(x[i] >> 16);
    }
  }
};

template <typename T, int D>
__global__ __launch_bounds__(256) void pyramid_top_kernel(const T* __restrict__ k, int64_t head_stride,
                                                          int heads_total, int n_prompt, int levels,
                                                          int rows_per_item, int64_t items_per_head,
                                                          float scale, float* __restrict__ a_top) {
  constexpr int VE = Vec16<T>::N;
  constexpr int V = D / VE;     // vectors per row
  constexpr int RPP = 64 / V;   // rows per wave pass
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= items_per_head * heads_total) return;
  const int64_t head = item / items_per_head;
  const int64_t it = item - head * items_per_head;
  const int col = lane % V, r = lane / V;
  const int64_t row0 = it * rows_per_item + r;
  const T* src = k + head * head_stride + row0 * D + col * VE;
  float acc[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) acc[e] = 0.f;
  const int passes = rows_per_item / RPP;
  if (row0 + (int64_t)(passes - 1) * RPP < n_prompt) {
#pragma unroll 8
    for (int p = 0; p < passes; ++p) Vec16<T>::add(src + (int64_t)p * RPP * D, acc);
  } else {
    for (int p = 0; p < passes; ++p)
      if (row0 + (int64_t)p * RPP < n_prompt) Vec16<T>::add(src + (int64_t)p * RPP * D, acc);
  }
  const int block_rows = 1 << levels;
  const int G = block_rows < RPP ? block_rows : RPP;  // row groups per block inside one pass
  for (int o = V; o < V * G; o <<= 1) {
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[e] += __shfl_xor(acc[e], o, 64);
  }
  if ((r & (G - 1)) == 0 && row0 < n_prompt) {
    const int n_top = n_prompt >> levels;
    const int64_t out_row = head * n_top + (row0 >> levels);
    float* dst = a_top + out_row * D + col * VE;
#pragma unroll
    for (int e = 0; e < VE; e += 4)
      *reinterpret_cast<float4*>(dst + e) =
          make_float4(acc[e] * scale, acc[e + 1] * scale, acc[e + 2] * scale, acc[e + 3] * scale);
  }
}

// One analysis level (section 2.2, eq. 5): A_j[n] = (x[2n] + x[2n+1])/sqrt2,
// D_j[n] = (x[2n] - x[2n+1])/sqrt2, with x = A_{j-1} (x = keys for j = 1).
template <typename T>
__device__ __forceinline__ float load_elem(const T* p);
template <> __device__ __forceinline__ float load_elem<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load_elem<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }

template <typename T>
__global__ __launch_bounds__(256) void pyramid_level_kernel(const T* __restrict__ src, int64_t src_head_stride,
                                                            int heads_total, int n_out, int d,
                                                            float* __restrict__ a_out, float* __restrict__ d_out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_head = (int64_t)n_out * d;
  if (idx >= per_head * heads_total) return;
  const int64_t head = idx / per_head;
  const int64_t rem = idx - head * per_head;
  const int64_t n = rem / d, c = rem - n * d;
  const T* base = src + head * src_head_stride;
  const float x0 = load_elem<T>(base + (2 * n) * d + c);
  const float x1 = load_elem<T>(base + (2 * n + 1) * d + c);
  const float inv_sqrt2 = 0.70710678118654752440f;
  a_out[idx] = (x0 + x1) * inv_sqrt2;
  d_out[idx] = (x0 - x1) * inv_sqrt2;
}

hipError_t launch_pyramid(const PyramidLaunch& a, hipStream_t s) {
  const int L = a.levels;
  uint8_t* base = reinterpret_cast<uint8_t*>(a.base);
  if (a.flags & WF_PYR_ALL_LEVELS) {
    // level by level, each level reading the previous one
    for (int j = 1; j <= L; ++j) {
      const int n_out = a.n_prompt >> j;
      const int64_t total = (int64_t)n_out * a.head_dim * a.heads_total;
      const unsigned grid = (unsigned)((total + 255) / 256);
      float* a_out = reinterpret_cast<float*>(base + a.band_off_a[j]);
      float* d_out = reinterpret_cast<float*>(base + a.band_off_d[j]);
      if (j == 1) {
        if (a.dtype == WF_BF16)
          hipLaunchKernelGGL(pyramid_level_kernel<bf16_t>, dim3(grid), dim3(256), 0, s,
                             reinterpret_cast<const bf16_t*>(a.k), a.head_stride, a.heads_total, n_out,
                             a.head_dim, a_out, d_out);
        else
          hipLaunchKernelGGL(pyramid_level_kernel<float>, dim3(grid), dim3(256), 0, s,
                             reinterpret_cast<const float*>(a.k), a.head_stride, a.heads_total, n_out,
                             a.head_dim, a_out, d_out);
      } else {
        const float* prev = reinterpret_cast<const float*>(base + a.band_off_a[j - 1]);
        hipLaunchKernelGGL(pyramid_level_kernel<float>, dim3(grid), dim3(256), 0, s, prev,
                           (int64_t)(a.n_prompt >> (j - 1)) * a.head_dim, a.heads_total, n_out,
                           a.head_dim, a_out, d_out);
      }
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (L > 0) return hipSuccess;
    // L == 0: A_0 is the keys themselves, converted below by the streaming kernel
  }
  const int vec_elems = (a.dtype == WF_BF16) ? 8 : 4;
  const int rpp = 64 / (a.head_dim / vec_elems);
  const int rows_per_item = (1 << L) > rpp ? (1 << L) : rpp;
  const int64_t items_per_head = (a.n_prompt + rows_per_item - 1) / rows_per_item;
  const int64_t items = items_per_head * a.heads_total;
  const unsigned grid = (unsigned)((items + 3) / 4);
  const float scale = (float)ldexp(1.0, -L / 2) * ((L & 1) ? 0.70710678118654752440f : 1.0f);
#define WF_PYR(T, D)                                                                                   \
  hipLaunchKernelGGL((pyramid_top_kernel<T, D>), dim3(grid), dim3(256), 0, s,                         \
                     reinterpret_cast<const T*>(a.k), a.head_stride, a.heads_total, a.n_prompt, L,    \
                     rows_per_item, items_per_head, scale, a.base)
  if (a.dtype == WF_BF16) {
    if (a.head_dim == 128) WF_PYR(bf16_t, 128); else WF_PYR(bf16_t, 64);
  } else {
    if (a.head_dim == 128) WF_PYR(float, 128); else WF_PYR(float, 64);
  }
#undef WF_PYR
  return hipGetLastError();
}

// ===========================================================================
// Per-step selection + attention.
// ===========================================================================
struct StepArgs {
  const void* q;
  const float* a_top;
  const void* k;
  const void* v;
  const int32_t* gen_idx;
  float* out;
  int32_t* sel_out;
  int32_t* sel_levels;
  float* score_levels;
  int32_t* counters;     // [WF_MAX_HEADS + 1][2]: coarse, attend
  uint32_t* keys_top;    // [heads_total][n_top]
  int32_t* sel_top;      // [heads_total][k_top]
  float* cov;            // [heads_total][cov_len]
  int32_t* sel0;         // [heads_total][k0]
  float* part_ml;        // [heads_total][n_split][2][n_q]
  float* part_o;         // [heads_total][n_split][n_q][d]
  int n_q, n_top, n_prompt, n_tot, n_gen, levels;
  int k_top, k0, sum_k;
  int64_t covered, cov_len;
  int64_t cov_off[kMaxLevels];
  int budgets[kMaxLevels + 1];
  int n_att, n_chunks, n_split, chunks_per_split;
  float inv_sqrt_d;
};

// Query fragments (A operand of the score tiles): rows 16 qt + l16 of the
// head's query block, zero for rows >= n_q.
template <typename T, int D, int RT>
__device__ __forceinline__ void load_query_frags(const T* qh, int n_q, int l16, int g, Frag<T, D> (&qf)[RT]) {
#pragma unroll
  for (int qt = 0; qt < RT; ++qt) {
    const int row = 16 * qt + l16;
    if (row < n_q) qf[qt].load(qh + (int64_t)row * D, g);
    else qf[qt].zero();
  }
}

// Last-arriving workgroup of a head: every workgroup publishes its writes
// (device-scope release), bumps the head's counter; the one that brings it
// to `expected` acquires and returns true, and resets the counter to zero
// for the next call.
__device__ __forceinline__ bool last_arrival(int32_t* counter, int expected) {
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = atomicAdd(counter, 1);
    s_last = (prev == expected - 1);
    if (s_last) atomicExch(counter, 0);
  }
  __syncthreads();
  if (s_last) __threadfence();
  return s_last != 0;
}

// ---------------------------------------------------------------------------
// Coarse scores and coarse Top-K (Figure 2 (c)).  Wave w of block x scores
// level-L regions n = 64 x + 16 w + l16 against all queries:
// acc[qt] = Q_tile(qt) . A_L_tile^T with Q as the A operand.  For bfloat16
// inputs the float32 coefficients are split into bf16 hi + lo parts, both
// multiplied exactly and accumulated in float32.
// ---------------------------------------------------------------------------
template <typename T, int D, int RT>
__global__ __launch_bounds__(256) void coarse_kernel(StepArgs a) {
  const int head = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const T* qh = reinterpret_cast<const T*>(a.q) + (int64_t)head * a.n_q * D;
  Frag<T, D> qf[RT];
  load_query_frags<T, D, RT>(qh, a.n_q, l16, g, qf);

  const int n = blockIdx.x * 64 + w * 16 + l16;
  const bool valid = n < a.n_top;
  const float* arow = a.a_top + ((int64_t)head * a.n_top + (valid ? n : 0)) * D;
  f32x4 acc[RT];
#pragma unroll
  for (int qt = 0; qt < RT; ++qt) acc[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (sizeof(T) == 2) {
    constexpr int STEPS = D / 32;
    const float4* p = reinterpret_cast<const float4*>(arow + g * (D / 4));
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      u32x4 hi, lo;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float4 x = valid ? p[2 * s + h] : make_float4(0.f, 0.f, 0.f, 0.f);
        float xs[4] = {x.x, x.y, x.z, x.w};
        uint32_t hb[4], lb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hb[e] = f32_to_bf16(xs[e]);
          lb[e] = f32_to_bf16(xs[e] - bf16_to_f32(hb[e]));
        }
        hi[2 * h] = pack_bf16(hb[0], hb[1]);
        hi[2 * h + 1] = pack_bf16(hb[2], hb[3]);
        lo[2 * h] = pack_bf16(lb[0], lb[1]);
        lo[2 * h + 1] = pack_bf16(lb[2], lb[3]);
      }
#pragma unroll
      for (int qt = 0; qt < RT; ++qt) {
        acc[qt] = mma_bf16(qf[qt].v[s], hi, acc[qt]);
        acc[qt] = mma_bf16(qf[qt].v[s], lo, acc[qt]);
      }
    }
  } else {
    Frag<float, D> b;
    if (valid) b.load(arow, g); else b.zero();
#pragma unroll
    for (int qt = 0; qt < RT; ++qt) acc[qt] = mma_tile<D>(qf[qt], b, acc[qt]);
  }
  float m = -INFINITY;
#pragma unroll
  for (int qt = 0; qt < RT; ++qt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (16 * qt + 4 * g + r < a.n_q) m = fmaxf(m, acc[qt][r]);
  m = wave_max_xor_16_32(m);
  uint32_t* keys = a.keys_top + (int64_t)head * a.n_top;
  if (g == 0 && valid) keys[n] = order_key(m * a.inv_sqrt_d);

  if (!last_arrival(a.counters + head * 2 + 0, gridDim.x)) return;
  __shared__ TopKShared<256> sh;
  auto key = [&](int i) { return keys[i]; };
  const Threshold t = radix_select<256>(key, a.n_top, a.k_top, sh);
  int32_t* sel = a.sel_top + (int64_t)head * a.k_top;
  topk_compact<256>(key, a.n_top, t, sh, [&](int o, int i) {
    if (o < a.k_top) sel[o] = i;
  });
}

// ---------------------------------------------------------------------------
// Coverage scores (Figure 2 (d), with the level-j coefficients taken from
// token dot products by linearity: q . A_j[c] = 2^{-j/2} sum_{t in c} q . k_t).
// The kept coarse regions, in ascending order, cover positions
// p = 0 .. k_L 2^L - 1, position p being token sel_L[p >> L] 2^L + (p mod 2^L).
// Wave w of block x owns positions 256 x + 64 w + [0, 64): four 16-token
// tiles t, token p on lane l16 = p mod 16.  acc[qt][t] holds
// S[query 16 qt + 4 g + r][token] with Q as the A operand.  Level-j sums run
// along the token axis: inside a tile by DPP row operations (j <= 4), across
// the wave's tiles in registers (j = 5, 6).  The level-j score of a block is
// the max over the valid query rows (in-lane over qt, r, then across the four
// lane groups g).
// ---------------------------------------------------------------------------
template <typename T, int D, int RT>
__global__ __launch_bounds__(256) void cover_kernel(StepArgs a) {
  const int head = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int64_t wave_base = (int64_t)blockIdx.x * 256 + w * 64;
  if (wave_base >= a.covered) return;  // no workgroup barrier in this kernel
  const T* qh = reinterpret_cast<const T*>(a.q) + (int64_t)head * a.n_q * D;
  Frag<T, D> qf[RT];
  load_query_frags<T, D, RT>(qh, a.n_q, l16, g, qf);

  const int L = a.levels;
  const int32_t* sel = a.sel_top + (int64_t)head * a.k_top;
  const T* kh = reinterpret_cast<const T*>(a.k) + (int64_t)head * a.n_tot * D;
  f32x4 acc[RT][4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t p = wave_base + 16 * t + l16;
    Frag<T, D> b;
    if (p < a.covered) {
      const int r = clampi(sel[p >> L], 0, a.n_top - 1);  // kept region (clamped: memory safety)
      const int64_t tok = ((int64_t)r << L) + (p & ((1 << L) - 1));
      b.load(kh + tok * D, g);
    } else {
      b.zero();
    }
#pragma unroll
    for (int qt = 0; qt < RT; ++qt) acc[qt][t] = mma_tile<D>(qf[qt], b, f32x4{0.f, 0.f, 0.f, 0.f});
  }
  // validity of query rows held by this lane
  bool qv[RT][4];
#pragma unroll
  for (int qt = 0; qt < RT; ++qt)
#pragma unroll
    for (int r = 0; r < 4; ++r) qv[qt][r] = (16 * qt + 4 * g + r) < a.n_q;

  float* cov = a.cov + (int64_t)head * a.cov_len;
  const int jmax = L < 7 ? L : 7;  // levels 0 .. jmax-1 are scored here
  float scale = a.inv_sqrt_d;      // 2^{-j/2} / sqrt(d)
#pragma unroll
  for (int j = 0; j <= 4; ++j) {
    if (j >= jmax) break;
    if (j > 0) {
#pragma unroll
      for (int qt = 0; qt < RT; ++qt)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[qt][t][r] = group_sum_step(acc[qt][t][r], j);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float m = -INFINITY;
#pragma unroll
      for (int qt = 0; qt < RT; ++qt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (qv[qt][r]) m = fmaxf(m, acc[qt][t][r]);
      m = wave_max_xor_16_32(m);
      const int64_t p = wave_base + 16 * t + l16;
      if (g == 0 && (l16 & ((1 << j) - 1)) == 0 && p < a.covered) cov[a.cov_off[j] + (p >> j)] = m * scale;
    }
    scale *= 0.70710678118654752440f;
  }
  if (jmax > 5) {
    // level 5: 32-token blocks = tile pairs (0,1) and (2,3); level 6: all four tiles
    float m01 = -INFINITY, m23 = -INFINITY, mall = -INFINITY;
#pragma unroll
    for (int qt = 0; qt < RT; ++qt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (!qv[qt][r]) continue;
        const float s01 = acc[qt][0][r] + acc[qt][1][r];
        const float s23 = acc[qt][2][r] + acc[qt][3][r];
        m01 = fmaxf(m01, s01);
        m23 = fmaxf(m23, s23);
        mall = fmaxf(mall, s01 + s23);
      }
    m01 = wave_max_xor_16_32(m01);
    m23 = wave_max_xor_16_32(m23);
    mall = wave_max_xor_16_32(mall);
    const float sc5 = a.inv_sqrt_d * 0.17677669529663688110f;  // 2^{-5/2}
    if (lane == 0) {
      if (wave_base < a.covered) cov[a.cov_off[5] + (wave_base >> 5)] = m01 * sc5;
      if (wave_base + 32 < a.covered) cov[a.cov_off[5] + (wave_base >> 5) + 1] = m23 * sc5;
      if (jmax > 6) cov[a.cov_off[6] + (wave_base >> 6)] = mall * (a.inv_sqrt_d * 0.125f);  // 2^{-3}
    }
  }
}

// ---------------------------------------------------------------------------
// Recursive refinement (Figure 2 (d)), one workgroup per head.  Positions at
// level j index the level-j blocks inside the covered set, ascending; block
// at position p has children 2p and 2p+1 and global index
// sel_L[p >> (L-j)] 2^{L-j} + (p mod 2^{L-j}).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kRefineThreads) void refine_kernel(StepArgs a) {
  constexpr int NT = kRefineThreads;
  const int head = blockIdx.x;
  const int L = a.levels;
  extern __shared__ uint32_t lds[];
  __shared__ TopKShared<NT> sh;
  int kmax = 0, nmax = 0;
  for (int i = 0; i <= L; ++i) kmax = max(kmax, a.budgets[i]);
  for (int i = 0; i < L; ++i) nmax = max(nmax, 2 * a.budgets[i]);
  uint32_t* keys = lds;
  int* cur = reinterpret_cast<int*>(lds + nmax);
  int* nxt = cur + kmax;

  const int32_t* sel_top = a.sel_top + (int64_t)head * a.k_top;
  const uint32_t* keys_top = a.keys_top + (int64_t)head * a.n_top;
  int32_t* dbg_sel = a.sel_levels ? a.sel_levels + (int64_t)head * a.sum_k : nullptr;
  float* dbg_score = a.score_levels ? a.score_levels + (int64_t)head * a.sum_k : nullptr;
  for (int i = threadIdx.x; i < a.k_top; i += NT) {
    cur[i] = i;
    const int r = clampi(sel_top[i], 0, a.n_top - 1);
    if (dbg_sel) dbg_sel[i] = r;
    if (dbg_score) dbg_score[i] = key_to_f32(keys_top[r]);
  }
  __syncthreads();
  int kprev = a.k_top, dbg_off = a.k_top;
  for (int j = L - 1; j >= 0; --j) {
    const int kj = a.budgets[L - j];
    const int n = 2 * kprev;
    const float* cj = a.cov + (int64_t)head * a.cov_len + a.cov_off[j];
    const int nj = (int)(a.covered >> j);  // level-j positions in the covered set
    for (int c = threadIdx.x; c < n; c += NT) keys[c] = order_key(cj[clampi(2 * cur[c >> 1] + (c & 1), 0, nj - 1)]);
    __syncthreads();
    auto key = [&](int i) { return keys[i]; };
    const Threshold t = radix_select<NT>(key, n, kj, sh);
    topk_compact<NT>(key, n, t, sh, [&](int o, int i) {
      if (o < kj) nxt[o] = clampi(2 * cur[i >> 1] + (i & 1), 0, nj - 1);
    });
    __syncthreads();
    if (dbg_sel || dbg_score) {
      const int sh_l = L - j;
      for (int o = threadIdx.x; o < kj; o += NT) {
        const int p = nxt[o];
        if (dbg_sel) dbg_sel[dbg_off + o] = (clampi(sel_top[p >> sh_l], 0, a.n_top - 1) << sh_l) + (p & ((1 << sh_l) - 1));
        if (dbg_score) dbg_score[dbg_off + o] = cj[p];
      }
    }
    int* tmp = cur;
    cur = nxt;
    nxt = tmp;
    kprev = kj;
    dbg_off += kj;
    __syncthreads();
  }
  int32_t* s0 = a.sel0 + (int64_t)head * a.k0;
  int32_t* so = a.sel_out ? a.sel_out + (int64_t)head * a.k0 : nullptr;
  for (int o = threadIdx.x; o < a.k0; o += NT) {
    const int p = cur[o];
    const int tok = (clampi(sel_top[clampi(p >> L, 0, a.k_top - 1)], 0, a.n_top - 1) << L) + (p & ((1 << L) - 1));
    s0[o] = tok;
    if (so) so[o] = tok;
  }
}

// ---------------------------------------------------------------------------
// Sparse attention (eq. 3 over T = kept prompt tokens, then gen_idx).
// Workgroup (split, head) walks chunks of 64 tokens; wave w owns query tile
// w.  Per chunk: K rows -> LDS (row-major, padded), V rows -> LDS transposed;
// S^T = K Q^T on MFMA (lane (query l16, g) holds tokens 16 t + 4 g + r);
// online softmax per query row in float32; O^T += V^T P^T on MFMA with P
// split into bf16 hi + lo (float32 MFMA for float32 inputs).  Partials
// (m, l, O) go to the workspace; the head's last workgroup merges them.
// ---------------------------------------------------------------------------
template <typename T> struct AttendTraits;
template <> struct AttendTraits<bf16_t> { static constexpr int CH = kAttendChunkBf16, KPAD = 8, VPAD = 4; };
template <> struct AttendTraits<float> { static constexpr int CH = kAttendChunkF32, KPAD = 4, VPAD = 4; };

template <typename T, int D, int NQT>
__global__ __launch_bounds__(64 * NQT) void attend_kernel(StepArgs a) {
  constexpr int NT = 64 * NQT;
  constexpr int CH = AttendTraits<T>::CH;
  constexpr int KS = D + AttendTraits<T>::KPAD;   // Ks row stride (elements)
  constexpr int VS = CH + AttendTraits<T>::VPAD;  // Vt row stride (elements)
  constexpr int VE = 16 / sizeof(T);
  constexpr int NV = D / VE;  // 16-byte vectors per row
  __shared__ __attribute__((aligned(16))) T Ks[CH * KS];
  __shared__ __attribute__((aligned(16))) T Vt[D * VS];
  __shared__ int tok_idx[CH];

  const int head = blockIdx.y, split = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int query = 16 * w + l16;
  const bool qvalid = query < a.n_q;
  const T* kh = reinterpret_cast<const T*>(a.k) + (int64_t)head * a.n_tot * D;
  const T* vh = reinterpret_cast<const T*>(a.v) + (int64_t)head * a.n_tot * D;
  const int32_t* s0 = a.sel0 + (int64_t)head * a.k0;

  Frag<T, D> qf;
  const T* qh = reinterpret_cast<const T*>(a.q) + (int64_t)head * a.n_q * D;
  if (qvalid) qf.load(qh + (int64_t)query * D, g); else qf.zero();

  const float sl2 = a.inv_sqrt_d * 1.44269504088896340736f;  // log2(e)/sqrt(d)
  float m = -INFINITY, lsum = 0.f;
  f32x4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int c_begin = split * a.chunks_per_split;
  const int c_end = min(a.n_chunks, c_begin + a.chunks_per_split);
  for (int chunk = c_begin; chunk < c_end; ++chunk) {
    const int pos0 = chunk * CH;
    for (int i = threadIdx.x; i < CH; i += NT) {
      const int pos = pos0 + i;
      int tok = -1;
      if (pos < a.k0) tok = s0[pos];
      else if (pos < a.n_att) tok = a.gen_idx[pos - a.k0];
      if (tok >= a.n_tot) tok = a.n_tot - 1;
      if (pos < a.n_att && tok < 0) tok = 0;
      tok_idx[i] = tok;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < CH * NV; e += NT) {
      const int row = e / NV, cv = e - row * NV;
      const int tok = tok_idx[row];
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (tok >= 0) {
        kv = *reinterpret_cast<const u32x4*>(kh + (int64_t)tok * D + cv * VE);
        vv = *reinterpret_cast<const u32x4*>(vh + (int64_t)tok * D + cv * VE);
      }
      *reinterpret_cast<u32x4*>(Ks + row * KS + cv * VE) = kv;
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          Vt[(cv * VE + 2 * i) * VS + row] = (bf16_t)(vv[i] & 0xFFFFu);
          Vt[(cv * VE + 2 * i + 1) * VS + row] = (bf16_t)(vv[i] >> 16);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) Vt[(cv * VE + i) * VS + row] = __uint_as_float(vv[i]);
      }
    }
    __syncthreads();

    // S^T tiles
    f32x4 s[CH / 16];
#pragma unroll
    for (int t = 0; t < CH / 16; ++t) {
      Frag<T, D> kf;
      kf.load(Ks + (16 * t + l16) * KS, g);
      s[t] = mma_tile<D>(kf, qf, f32x4{0.f, 0.f, 0.f, 0.f});
    }
    float cmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < CH / 16; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pos = pos0 + 16 * t + 4 * g + r;
        const float x = (pos < a.n_att) ? s[t][r] * sl2 : -INFINITY;
        s[t][r] = x;
        cmax = fmaxf(cmax, x);
      }
    cmax = wave_max_xor_16_32(cmax);
    const float m_new = fmaxf(m, cmax);
    const float alpha = exp2f(m - m_new);
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < CH / 16; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = exp2f(s[t][r] - m_new);
        s[t][r] = p;
        psum += p;
      }
    lsum = lsum * alpha + psum;
    m = m_new;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt] *= alpha;

    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int st = 0; st < CH / 32; ++st) {
        u32x4 ph, pl;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          uint32_t hb[4], lb[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = s[2 * st + hh][r];
            hb[r] = f32_to_bf16(p);
            lb[r] = f32_to_bf16(p - bf16_to_f32(hb[r]));
          }
          ph[2 * hh] = pack_bf16(hb[0], hb[1]);
          ph[2 * hh + 1] = pack_bf16(hb[2], hb[3]);
          pl[2 * hh] = pack_bf16(lb[0], lb[1]);
          pl[2 * hh + 1] = pack_bf16(lb[2], lb[3]);
        }
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const T* vr = Vt + (16 * dt + l16) * VS + 32 * st + 4 * g;
          const u32x2 v0 = *reinterpret_cast<const u32x2*>(vr);
          const u32x2 v1 = *reinterpret_cast<const u32x2*>(vr + 16);
          const u32x4 vf = {v0[0], v0[1], v1[0], v1[1]};
          o[dt] = mma_bf16(vf, ph, o[dt]);
          o[dt] = mma_bf16(vf, pl, o[dt]);
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < CH / 16; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt) {
            const float vf = Vt[(16 * dt + l16) * VS + 16 * t + 4 * g + r];
            o[dt] = mma_f32(vf, s[t][r], o[dt]);
          }
    }
    __syncthreads();
  }

  lsum = wave_sum_xor_16_32(lsum);
  float* pml = a.part_ml + ((int64_t)head * a.n_split + split) * 2 * a.n_q;
  float* po = a.part_o + ((int64_t)head * a.n_split + split) * a.n_q * D;
  if (qvalid) {
    if (g == 0) {
      pml[query] = m;
      pml[a.n_q + query] = lsum;
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      *reinterpret_cast<float4*>(po + (int64_t)query * D + 16 * dt + 4 * g) =
          make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
  }

  if (!last_arrival(a.counters + head * 2 + 1, gridDim.x)) return;
  // merge: O = sum_s e^{m_s - M} O_s / sum_s e^{m_s - M} l_s
  __shared__ float wgt[kMaxSplit * 64];
  const float* ml = a.part_ml + (int64_t)head * a.n_split * 2 * a.n_q;
  const int ns = a.n_split;
  for (int qi = threadIdx.x; qi < a.n_q; qi += NT) {
    float mm = -INFINITY;
    for (int sp = 0; sp < ns; ++sp) mm = fmaxf(mm, ml[sp * 2 * a.n_q + qi]);
    float den = 0.f;
    for (int sp = 0; sp < ns; ++sp) den += exp2f(ml[sp * 2 * a.n_q + qi] - mm) * ml[sp * 2 * a.n_q + a.n_q + qi];
    const float inv = 1.0f / den;
    for (int sp = 0; sp < ns; ++sp) wgt[sp * 64 + qi] = exp2f(ml[sp * 2 * a.n_q + qi] - mm) * inv;
  }
  __syncthreads();
  const float* pob = a.part_o + (int64_t)head * a.n_split * a.n_q * D;
  float* outh = a.out + (int64_t)head * a.n_q * D;
  for (int e = threadIdx.x; e < a.n_q * (D / 4); e += NT) {
    const int qi = e / (D / 4), c4 = e - qi * (D / 4);
    float4 acc4 = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int sp = 0; sp < ns; ++sp) {
      const float wv = wgt[sp * 64 + qi];
      const float4 x = *reinterpret_cast<const float4*>(pob + ((int64_t)sp * a.n_q + qi) * D + 4 * c4);
      acc4.x += wv * x.x; acc4.y += wv * x.y; acc4.z += wv * x.z; acc4.w += wv * x.w;
    }
    *reinterpret_cast<float4*>(outh + (int64_t)qi * D + 4 * c4) = acc4;
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_select_attend(const SelectLaunch& L, hipStream_t s) {
  const SelectPlan& P = L.plan;
  StepArgs a;
  a.q = L.q;
  a.a_top = L.a_top;
  a.k = L.k;
  a.v = L.v;
  a.gen_idx = L.gen_idx;
  a.out = L.out;
  a.sel_out = L.sel_out;
  a.sel_levels = L.sel_levels;
  a.score_levels = L.score_levels;
  a.counters = reinterpret_cast<int32_t*>(L.ws + P.off_counters);
  a.keys_top = reinterpret_cast<uint32_t*>(L.ws + P.off_keys);
  a.sel_top = reinterpret_cast<int32_t*>(L.ws + P.off_sel_top);
  a.cov = reinterpret_cast<float*>(L.ws + P.off_cov);
  a.sel0 = reinterpret_cast<int32_t*>(L.ws + P.off_sel0);
  a.part_ml = reinterpret_cast<float*>(L.ws + P.off_part_ml);
  a.part_o = reinterpret_cast<float*>(L.ws + P.off_part_o);
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
  a.n_chunks = P.n_chunks;
  a.n_split = P.n_split;
  a.chunks_per_split = P.chunks_per_split;
  a.inv_sqrt_d = 1.0f / sqrtf((float)P.head_dim);

  const int H = P.heads_total;
  const int rt = (P.n_q + 15) / 16;
  const bool bf = P.dtype == WF_BF16;
  const bool d128 = P.head_dim == 128;

#define WF_DISPATCH(KERNEL, GRID, BLOCK)                                                       \
  do {                                                                                         \
    switch (rt) {                                                                              \
      case 1: WF_DISPATCH_RT(KERNEL, 1, GRID, BLOCK); break;                                   \
      case 2: WF_DISPATCH_RT(KERNEL, 2, GRID, BLOCK); break;                                   \
      case 3: WF_DISPATCH_RT(KERNEL, 3, GRID, BLOCK); break;                                   \
      default: WF_DISPATCH_RT(KERNEL, 4, GRID, BLOCK); break;                                  \
    }                                                                                          \
  } while (0)
#define WF_DISPATCH_RT(KERNEL, RTV, GRID, BLOCK)                                               \
  do {                                                                                         \
    if (bf && d128) hipLaunchKernelGGL((KERNEL<bf16_t, 128, RTV>), GRID, BLOCK, 0, s, a);      \
    else if (bf) hipLaunchKernelGGL((KERNEL<bf16_t, 64, RTV>), GRID, BLOCK, 0, s, a);          \
    else if (d128) hipLaunchKernelGGL((KERNEL<float, 128, RTV>), GRID, BLOCK, 0, s, a);        \
    else hipLaunchKernelGGL((KERNEL<float, 64, RTV>), GRID, BLOCK, 0, s, a);                   \
  } while (0)

  hipError_t e;
  WF_DISPATCH(coarse_kernel, dim3((P.n_top + 63) / 64, H), dim3(256));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (P.levels > 0) {
    WF_DISPATCH(cover_kernel, dim3((unsigned)((P.covered + 255) / 256), H), dim3(256));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(refine_kernel, dim3(H), dim3(kRefineThreads), P.refine_lds, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  WF_DISPATCH(attend_kernel, dim3(P.n_split, H), dim3(64 * rt));
  return hipGetLastError();
#undef WF_DISPATCH
#undef WF_DISPATCH_RT
}

}  // namespace wf
