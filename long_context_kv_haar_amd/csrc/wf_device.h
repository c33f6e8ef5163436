// Device-side building blocks shared by the WaveFilter kernels (gfx950).
//
// - element access for float32 and bfloat16 rows (16-byte vector loads);
// - the 16x16 MFMA tiles used for every dense contraction;
// - order-preserving integer keys for float scores;
// - a workgroup-wide radix select + stable compaction implementing the
//   Top-K rule (higher score first, lower index on ties, output ascending).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wf_types.h"

namespace wf {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two float32 values -> a packed bfloat16 pair (a in the low half), rounded
// to nearest even by the hardware conversion (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// a and b as bfloat16 hi + lo pairs: hi = bf16(x), lo = bf16(x - hi), packed
// two per word like cvt_pk_bf16 (hi + lo carries 16 significant bits).
struct Bf16Split {
  uint32_t hi, lo;
};
__device__ __forceinline__ Bf16Split split_pk_bf16(float a, float b) {
  const uint32_t hi = cvt_pk_bf16(a, b);
  return {hi, cvt_pk_bf16(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xFFFF0000u))};
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// ---------------------------------------------------------------------------
// MFMA 16x16 tiles.  D[i][j] += sum_k A[i][k] B[k][j]; lane l supplies row
// i = l % 16 of A and column j = l % 16 of B, with k-slots chosen by
// g = l / 16; the accumulator holds D[4g + r][l % 16], r = 0..3.  Only the
// pairing of A's and B's k-slots matters for a dot product, so the kernels
// choose the permutation of the contraction axis that suits the loads:
//   bfloat16: step s of lane group g takes elements [32 s + 8 g, 32 s + 8 g + 8),
//     so the four lane groups of a row read 64 contiguous bytes per step;
//   float32:  lane group g takes the contiguous quarter [g d/4, (g+1) d/4).
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Operand fragments for one 16-row tile over the full contraction axis D.
//   bf16: D/32 steps of 8 elements (one u32x4) per lane;
//   f32:  D/4 steps of 1 element per lane.
template <typename T, int D> struct Frag;

template <int D> struct Frag<bf16_t, D> {
  static constexpr int STEPS = D / 32;
  u32x4 v[STEPS];
  // Row `row` of a row-major [*, D] bfloat16 matrix, lane group g.
  __device__ __forceinline__ void load(const bf16_t* row, int g) {
    const u32x4* p = reinterpret_cast<const u32x4*>(row + 8 * g);
#pragma unroll
    for (int s = 0; s < STEPS; ++s) v[s] = p[4 * s];
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int s = 0; s < STEPS; ++s) v[s] = u32x4{0u, 0u, 0u, 0u};
  }
};

template <int D> struct Frag<float, D> {
  static constexpr int STEPS = D / 4;
  float v[STEPS];
  __device__ __forceinline__ void load(const float* row, int g) {
    const float4* p = reinterpret_cast<const float4*>(row + g * (D / 4));
#pragma unroll
    for (int s = 0; s < STEPS / 4; ++s) {
      float4 x = p[s];
      v[4 * s + 0] = x.x;
      v[4 * s + 1] = x.y;
      v[4 * s + 2] = x.z;
      v[4 * s + 3] = x.w;
    }
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int s = 0; s < STEPS; ++s) v[s] = 0.f;
  }
};

template <int D>
__device__ __forceinline__ f32x4 mma_tile(const Frag<bf16_t, D>& a, const Frag<bf16_t, D>& b, f32x4 c) {
#pragma unroll
  for (int s = 0; s < Frag<bf16_t, D>::STEPS; ++s) c = mma_bf16(a.v[s], b.v[s], c);
  return c;
}

template <int D>
__device__ __forceinline__ f32x4 mma_tile(const Frag<float, D>& a, const Frag<float, D>& b, f32x4 c) {
#pragma unroll
  for (int s = 0; s < Frag<float, D>::STEPS; ++s) c = mma_f32(a.v[s], b.v[s], c);
  return c;
}

// ---------------------------------------------------------------------------
// Cross-lane helpers.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Sum of x over aligned groups of 2^lvl consecutive lanes within a 16-lane
// row, given x already summed over groups of 2^(lvl-1) lanes; every lane of
// the group ends with the group total.
__device__ __forceinline__ float group_sum_step(float x, int lvl) {
  switch (lvl) {
    case 1: return x + dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]
    case 2: return x + dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]
    case 3: return x + dpp_f<0x141>(x);  // row_half_mirror
    default: return x + dpp_f<0x140>(x); // row_mirror
  }
}

// Exchanges across 16-lane rows with the gfx950 lane permutes, which stay in
// the VALU (a shuffle through ds_bpermute is an LDS round trip).
// permlane16_swap(x, x) returns (x of rows 0,0,2,2 ; x of rows 1,1,3,3) and
// permlane32_swap(x, x) returns (x of halves lo,lo ; x of halves hi,hi), so
// the two results hold each lane's value and its partner's.
__device__ __forceinline__ uint32_t lane_xor16(uint32_t x) {  // x of lane l ^ 16
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return ((threadIdx.x >> 4) & 1) ? r[0] : r[1];
}
__device__ __forceinline__ uint32_t lane_xor32(uint32_t x) {  // x of lane l ^ 32
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return ((threadIdx.x >> 5) & 1) ? r[0] : r[1];
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_max_xor_16_32(float x) { return max_xor32(max_xor16(x)); }
__device__ __forceinline__ float wave_sum_xor_16_32(float x) { return sum_xor32(sum_xor16(x)); }

// ---------------------------------------------------------------------------
// Order-preserving keys: key(a) > key(b)  <=>  a > b for finite floats;
// -0 and +0 map to the same key.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = (f == 0.0f) ? 0u : __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_f32(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// ---------------------------------------------------------------------------
// Workgroup-wide Top-K on 32-bit keys.
//
// select_threshold narrows the k-th largest key by range bisection: the keys
// still in play lie in [lo, lo + range]; each pass counts them into at most
// 4 NT bins of width 2^s (bin = (key - lo) >> s) with LDS atomics, finds
// the bin holding the k-th largest, and recurses into it.  Starting from the
// actual [min, max] of the keys spreads them over the bins (scores of one
// level share their leading bits, so fixed-digit radix passes would pile
// every key into one bin and serialise the atomics); a pass ends the search
// once every key of the chosen bin is kept, or the bin holds a single value.
// The bin search is spread over the whole workgroup: thread t owns the four
// contiguous bins [4 t, 4 t + 4), read with one 16-byte LDS load, and one
// workgroup scan of the per-thread totals locates the bin.
//
// The kept set is: every key > hi, and of the keys in [lo, hi] the `need`
// ones with the lowest indices (when the search narrowed to one value,
// lo == hi and these are ties, resolved toward lower indices).  topk_compact
// emits the kept indices in ascending order with a single workgroup scan.
// NT = threads of the workgroup (a multiple of 64, at most 1024); all threads
// must call these functions together.
// ---------------------------------------------------------------------------
constexpr int kTopKBinsPerThread = 4;  // histogram bins owned by each thread in the bin search
constexpr int floor_log2(int x) { return x <= 1 ? 0 : 1 + floor_log2(x / 2); }

template <int NT> struct TopKShared {
  int hist[kTopKBinsPerThread * NT];
  uint32_t wmin[NT / 64], wmax[NT / 64];
  int wsum_a[NT / 64], wsum_b[NT / 64];
  int bcast[4];
};

struct Threshold {
  uint32_t lo, hi;
  int need;
};

// Wave-wide reductions and scans on DPP row operations plus readlane (a
// few cycles each, no LDS round trip).  All 64 lanes must be active.
template <int CTRL>
__device__ __forceinline__ int dpp_or0(int x) {  // x of the source lane, 0 where none
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  x = min(x, dpp_u<0xB1>(x));   // quad_perm [1,0,3,2]
  x = min(x, dpp_u<0x4E>(x));   // quad_perm [2,3,0,1]
  x = min(x, dpp_u<0x141>(x));  // row_half_mirror
  x = min(x, dpp_u<0x140>(x));  // row_mirror: every lane holds its row's min
  const uint32_t a = __builtin_amdgcn_readlane(x, 0), b = __builtin_amdgcn_readlane(x, 16);
  const uint32_t c = __builtin_amdgcn_readlane(x, 32), d = __builtin_amdgcn_readlane(x, 48);
  return min(min(a, b), min(c, d));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, dpp_u<0xB1>(x));
  x = max(x, dpp_u<0x4E>(x));
  x = max(x, dpp_u<0x141>(x));
  x = max(x, dpp_u<0x140>(x));
  const uint32_t a = __builtin_amdgcn_readlane(x, 0), b = __builtin_amdgcn_readlane(x, 16);
  const uint32_t c = __builtin_amdgcn_readlane(x, 32), d = __builtin_amdgcn_readlane(x, 48);
  return max(max(a, b), max(c, d));
}
// Inclusive prefix sum over the lanes of a wave; *total receives the sum.
__device__ __forceinline__ int wave_incl_scan(int x, int* total) {
  x += dpp_or0<0x111>(x);  // row_shr:1
  x += dpp_or0<0x112>(x);  // row_shr:2
  x += dpp_or0<0x114>(x);  // row_shr:4
  x += dpp_or0<0x118>(x);  // row_shr:8 -> inclusive within each row of 16
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31);
  const int r2 = __builtin_amdgcn_readlane(x, 47), r3 = __builtin_amdgcn_readlane(x, 63);
  const int row = (threadIdx.x & 63) >> 4;
  x += (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
  *total = r0 + r1 + r2 + r3;
  return x;
}

// Inclusive scan of one int per thread across the workgroup (one barrier;
// the caller must not touch `wsum` again before another barrier).
template <int NT>
__device__ __forceinline__ int block_incl_scan(int a, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int t;
  const int x = wave_incl_scan(a, &t);
  if (lane == 0) wsum[w] = t;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const int v = wsum[i];
    base += (i < w) ? v : 0;
    tot += v;
  }
  *total = tot;
  return base + x;
}

// Exclusive scan of two ints per thread across the workgroup.
template <int NT>
__device__ __forceinline__ void block_exclusive_scan2(int a, int b, int* wa, int* wb, int& ea, int& eb) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int ta, tb;
  const int x = wave_incl_scan(a, &ta);
  const int y = wave_incl_scan(b, &tb);
  if (lane == 0) {
    wa[w] = ta;
    wb[w] = tb;
  }
  __syncthreads();
  int ba = 0, bb = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    if (i < w) {
      ba += wa[i];
      bb += wb[i];
    }
  }
  __syncthreads();
  ea = ba + x - a;
  eb = bb + y - b;
}

template <int NT, class KeyFn>
__device__ __forceinline__ Threshold select_threshold(KeyFn key, int n, int k, TopKShared<NT>& sh) {
  constexpr int BPT = kTopKBinsPerThread;     // bins per thread in the bin search
  constexpr int LOGB = floor_log2(NT * BPT);   // bins used per pass: 2^LOGB
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for (int i = threadIdx.x; i < n; i += NT) {
    const uint32_t x = key(i);
    mn = min(mn, x);
    mx = max(mx, x);
  }
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  if (lane == 0) {
    sh.wmin[w] = mn;
    sh.wmax[w] = mx;
  }
  int4* own = reinterpret_cast<int4*>(sh.hist + threadIdx.x * BPT);
#pragma unroll
  for (int i = 0; i < BPT / 4; ++i) own[i] = make_int4(0, 0, 0, 0);
  __syncthreads();
  mn = 0xFFFFFFFFu;
  mx = 0u;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    mn = min(mn, sh.wmin[i]);
    mx = max(mx, sh.wmax[i]);
  }
  uint32_t lo = mn, range = mx - mn;
  int need = k;
  while (range != 0) {
    const int bits = 32 - __clz(range);
    const int s = bits > LOGB ? bits - LOGB : 0;  // (key - lo) >> s < 2^LOGB
    for (int i = threadIdx.x; i < n; i += NT) {
      const uint32_t d = key(i) - lo;  // wraps above range for keys below lo
      if (d <= range) atomicAdd(&sh.hist[d >> s], 1);
    }
    __syncthreads();
    // bin search: per-thread totals of its own bins, then a workgroup scan
    int h[BPT];
    int tot = 0;
#pragma unroll
    for (int i = 0; i < BPT / 4; ++i) {
      const int4 v = own[i];
      h[4 * i] = v.x;
      h[4 * i + 1] = v.y;
      h[4 * i + 2] = v.z;
      h[4 * i + 3] = v.w;
      tot += v.x + v.y + v.z + v.w;
    }
    int all;
    const int incl = block_incl_scan<NT>(tot, sh.wsum_a, &all);
    int above = all - incl;  // keys in bins owned by higher threads
    if (above < need && need <= above + tot) {
#pragma unroll
      for (int i = BPT - 1; i >= 0; --i) {
        if (above < need && need <= above + h[i]) {
          sh.bcast[0] = threadIdx.x * BPT + i;
          sh.bcast[1] = need - above;
          sh.bcast[2] = h[i];
        }
        above += h[i];
      }
    }
#pragma unroll
    for (int i = 0; i < BPT / 4; ++i) own[i] = make_int4(0, 0, 0, 0);
    __syncthreads();
    const int b = sh.bcast[0];
    need = sh.bcast[1];
    const int cnt = sh.bcast[2];
    lo += (uint32_t)b << s;
    const uint32_t rest = range - ((uint32_t)b << s);
    range = s == 0 ? 0u : min(rest, (1u << s) - 1u);
    if (cnt == need) break;
    __syncthreads();  // bcast and wsum are rewritten by the next pass
  }
  return Threshold{lo, lo + range, need};
}

// Calls out(o, i) for the kept indices i in ascending order, o = 0..k-1.
template <int NT, class KeyFn, class OutFn>
__device__ __forceinline__ void topk_compact(KeyFn key, int n, Threshold t, TopKShared<NT>& sh, OutFn out) {
  const int seg = (n + NT - 1) / NT;
  const int i0 = min(n, (int)threadIdx.x * seg), i1 = min(n, i0 + seg);
  int g = 0, e = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t x = key(i);
    g += x > t.hi;
    e += (x >= t.lo) & (x <= t.hi);
  }
  int G, E;
  block_exclusive_scan2<NT>(g, e, sh.wsum_a, sh.wsum_b, G, E);
  for (int i = i0; i < i1; ++i) {
    const uint32_t x = key(i);
    const bool gt = x > t.hi;
    const bool eq = (x >= t.lo) & (x <= t.hi);
    if (gt || (eq && E < t.need)) out(G + min(E, t.need), i);
    G += gt;
    E += eq;
  }
}

// ---------------------------------------------------------------------------
// Top-K in (usually) one histogram pass.  The kept set of "the k best by
// (key descending, index ascending)" is exactly the set of indices i with
// bin(key_i) > b, or bin(key_i) == b and (key_i > tk or (key_i == tk and
// i <= ti)), for any bin function that is monotone in the key, where b is the
// bin of the k-th best (key, index) pair and (tk, ti) that pair.  The bins
// split the scores' value range [min, max] linearly (bin = (x - min) * scale,
// a composition of monotone float operations, so it never inverts an order);
// linear bins spread clustered scores far better than bins of the key bits,
// which give each binade only a handful of bins.  One pass counts the keys
// into 4 NT bins and a workgroup scan finds b.  If every key of bin b is
// kept, (tk, ti) are not needed; otherwise the bin's keys (a handful) are
// gathered with their indices and ranked exactly inside one wave.  A bin with
// more than kGatherMax keys (heavy ties) falls back to select_threshold +
// topk_compact.  Emits the kept indices in ascending order with one scan.
// ---------------------------------------------------------------------------
constexpr int kGatherMax = 64;

template <int NT> struct TopKFastShared {
  TopKShared<NT> base;
  uint32_t gkey[kGatherMax];
  int gidx[kGatherMax];
  int gcount;
  uint32_t tk;
  int ti;
};

// Bin of a key: linear in the float value when the range allows it, else by
// the key bits (range shift s).  Monotone non-decreasing in the key.
struct BinFn {
  float fmin, scale;
  uint32_t kmin;
  int shift, nb;
  bool linear;
  __device__ __forceinline__ int operator()(uint32_t x) const {
    if (linear) return min(nb - 1, (int)((key_to_f32(x) - fmin) * scale));
    return (int)((x - kmin) >> shift);
  }
};

template <int NT, class KeyFn, class OutFn>
__device__ __forceinline__ void topk_fast(KeyFn key, int n, int k, TopKFastShared<NT>& fs, OutFn out) {
  constexpr int BPT = kTopKBinsPerThread;
  constexpr int LOGB = floor_log2(NT * BPT);
  TopKShared<NT>& sh = fs.base;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for (int i = threadIdx.x; i < n; i += NT) {
    const uint32_t x = key(i);
    mn = min(mn, x);
    mx = max(mx, x);
  }
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  if (lane == 0) {
    sh.wmin[w] = mn;
    sh.wmax[w] = mx;
  }
  int4* own = reinterpret_cast<int4*>(sh.hist + threadIdx.x * BPT);
#pragma unroll
  for (int i = 0; i < BPT / 4; ++i) own[i] = make_int4(0, 0, 0, 0);
  if (threadIdx.x == 0) fs.gcount = 0;
  __syncthreads();
  mn = 0xFFFFFFFFu;
  mx = 0u;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    mn = min(mn, sh.wmin[i]);
    mx = max(mx, sh.wmax[i]);
  }
  const uint32_t range = mx - mn;
  uint32_t tk = 0u;
  int ti = 0x7FFFFFFF;
  int b = -1;  // bins above b are kept whole; -1: no bins (all keys equal)
  BinFn bin;
  bool general = false;
  if (range == 0) {  // all keys equal: the k lowest indices
    tk = mn;
    ti = k - 1;
  } else {
    const float fmin = key_to_f32(mn), span = key_to_f32(mx) - fmin;
    const float scale = (float)(1 << LOGB) / span;
    const int bits = 32 - __clz(range);
    bin.fmin = fmin;
    bin.scale = scale;
    bin.kmin = mn;
    bin.shift = bits > LOGB ? bits - LOGB : 0;
    bin.nb = 1 << LOGB;
    bin.linear = span > 0.f && span < 3.0e38f && scale < 3.0e38f;  // finite, non-degenerate range
    for (int i = threadIdx.x; i < n; i += NT) atomicAdd(&sh.hist[bin(key(i))], 1);
    __syncthreads();
    int h[BPT];
    int tot = 0;
#pragma unroll
    for (int i = 0; i < BPT / 4; ++i) {
      const int4 v = own[i];
      h[4 * i] = v.x;
      h[4 * i + 1] = v.y;
      h[4 * i + 2] = v.z;
      h[4 * i + 3] = v.w;
      tot += v.x + v.y + v.z + v.w;
    }
    int all;
    const int incl = block_incl_scan<NT>(tot, sh.wsum_a, &all);
    int above = all - incl;
    if (above < k && k <= above + tot) {  // exactly one thread
      int bn = 0, rem = 0, c = 0;
#pragma unroll
      for (int i = BPT - 1; i >= 0; --i) {
        const bool hit = (above < k) & (k <= above + h[i]);
        bn = hit ? i : bn;
        rem = hit ? k - above : rem;
        c = hit ? h[i] : c;
        above += h[i];
      }
      sh.bcast[0] = threadIdx.x * BPT + bn;
      sh.bcast[1] = rem;
      sh.bcast[2] = c;
    }
    __syncthreads();
    b = sh.bcast[0];
    const int need = sh.bcast[1], cnt = sh.bcast[2];
    if (cnt == need) {  // the whole bin is kept: any key passes (tk, ti) = (0, max)
    } else if (cnt <= kGatherMax) {
      for (int i = threadIdx.x; i < n; i += NT) {
        const uint32_t x = key(i);
        if (bin(x) == b) {
          const int slot = atomicAdd(&fs.gcount, 1);
          fs.gkey[slot] = x;
          fs.gidx[slot] = i;
        }
      }
      __syncthreads();
      if (threadIdx.x < 64) {  // rank the gathered keys; rank need-1 is the threshold
        const bool act = lane < cnt;
        const uint32_t x = act ? fs.gkey[lane] : 0u;
        const int xi = act ? fs.gidx[lane] : 0;
        int rank = 0;
        for (int m = 0; m < cnt; ++m) {
          const uint32_t y = fs.gkey[m];
          const int yi = fs.gidx[m];
          rank += (y > x) | ((y == x) & (yi < xi));
        }
        if (act && rank == need - 1) {
          fs.tk = x;
          fs.ti = xi;
        }
      }
      __syncthreads();
      tk = fs.tk;
      ti = fs.ti;
    } else {
      general = true;
    }
  }
  if (general) {  // heavily tied bin: multi-pass search
    __syncthreads();
    const Threshold t = select_threshold<NT>(key, n, k, sh);
    topk_compact<NT>(key, n, t, sh, out);
    return;
  }
  // compaction in index order
  auto kept = [&](uint32_t x, int i) {
    if (b < 0) return (x > tk) | ((x == tk) & (i <= ti));
    const int bx = bin(x);
    return (bx > b) | ((bx == b) & ((x > tk) | ((x == tk) & (i <= ti))));
  };
  const int seg = (n + NT - 1) / NT;
  const int i0 = min(n, (int)threadIdx.x * seg), i1 = min(n, i0 + seg);
  int c = 0;
  for (int i = i0; i < i1; ++i) c += kept(key(i), i);
  int all;
  int o = block_incl_scan<NT>(c, sh.wsum_a, &all) - c;
  for (int i = i0; i < i1; ++i)
    if (kept(key(i), i)) out(o++, i);
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Strided Top-K for n <= ACT * MAXS keys, same rule and output as topk_fast.
// Key i lives in register slot i / ACT of thread i mod ACT, so every active
// thread holds ceil(n / ACT) slots (balanced), and only the first ACT threads
// (ACT / 64 waves, ideally one per SIMD) do any work: the others just meet
// the barriers.  No per-key branches: keys that must not be counted go to a trash bin of
// their lane (distinct LDS words, so those atomics never queue on one word).
//  1. min and max of the keys;
//  2. one histogram pass with bins linear in the score value over [min, max]
//     (monotone, so a key in a higher bin is strictly greater than every key
//     in a lower one); a scan finds bin b holding the k-th best;
//  3. the exact key range [lo, hi] of bin b is taken: every key above hi is
//     kept; unless bin b is kept whole, histogram passes over [lo, hi] in key
//     space narrow the boundary until the boundary range is kept whole or
//     holds a single key value (ties: the lowest indices win);
//  4. compaction in index order (slot-major, thread-minor): per-slot wave
//     ballots plus one prefix over (slot, wave) totals computed by wave 0.
// Slots are processed in straight-line groups of four (one uniform branch
// per group), so their LDS reads are in flight together.  load(i, j) returns
// key i for register slot j (i < n; slots past the end get i = n - 1 and are
// ignored) and may keep data of its own in slot j; out(o, kept, i, j) is
// called for every slot of the used groups with its output slot o, which is
// meaningful only when kept (the caller writes the others to a spare slot,
// with no branch).  All NT threads must call it.
// ---------------------------------------------------------------------------
template <int ACT, int MAXS> struct TopKSel {
  static constexpr int W = ACT / 64;
  static constexpr int NB = 4 * ACT;
  int hist[NB + 64];         // NB bins, then one trash bin per lane (never read)
  uint32_t wmn[W], wmx[W];
  int wtot[W];
  int cnt[MAXS * W];         // compaction: per (slot, wave) packed counts (16 + 16 bits), then prefixes
  int bc[4];
};

template <int NT, int ACT, int MAXS, class Load, class Out>
__device__ __forceinline__ void topk_strided(int n, int k, TopKSel<ACT, MAXS>& sh, Load load, Out out) {
  constexpr int W = ACT / 64;
  constexpr int NB = 4 * ACT;
  constexpr int LOGNB = floor_log2(NB);
  static_assert((NB & (NB - 1)) == 0 && ACT <= NT && MAXS * W <= 128, "Top-K layout");
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const bool act = t < ACT;  // wave-uniform
  const int ns = (n + ACT - 1) / ACT;
  int4* hist4 = reinterpret_cast<int4*>(sh.hist);

  // bin search: thread t < ACT owns bins [4t, 4t+4) (read and cleared here);
  // the thread holding the want-th best key writes (bin, need in bin, count)
  auto search = [&](int want) {
    int4 h = make_int4(0, 0, 0, 0);
    int incl = 0, tot = 0;
    if (act) {
      h = hist4[t];
      hist4[t] = make_int4(0, 0, 0, 0);
      tot = h.x + h.y + h.z + h.w;
      int wt;
      incl = wave_incl_scan(tot, &wt);
      if (lane == 63) sh.wtot[w] = wt;
    }
    __syncthreads();
    if (act) {
      int base = 0, all = 0;
#pragma unroll
      for (int i = 0; i < W; ++i) {
        const int v = sh.wtot[i];
        base += (i < w) ? v : 0;
        all += v;
      }
      int above = all - (base + incl);  // keys in bins of higher threads
      if (above < want && want <= above + tot) {
        const int hv[4] = {h.x, h.y, h.z, h.w};
        int bb = 0, rem = 0, c = 0;
#pragma unroll
        for (int i = 3; i >= 0; --i) {
          const bool hit = (above < want) & (want <= above + hv[i]);
          bb = hit ? i : bb;
          rem = hit ? want - above : rem;
          c = hit ? hv[i] : c;
          above += hv[i];
        }
        sh.bc[0] = 4 * t + bb;
        sh.bc[1] = rem;
        sh.bc[2] = c;
      }
    }
  };

  // 1. load, min and max; clear the histogram
  static_assert(MAXS % 4 == 0, "slot groups of four");
  uint32_t key[MAXS];
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  if (act) {
#pragma unroll
    for (int j0 = 0; j0 < MAXS; j0 += 4) {
#pragma unroll
      for (int j = j0; j < j0 + 4; ++j) key[j] = 0u;
      if (j0 < ns) {
#pragma unroll
        for (int j = j0; j < j0 + 4; ++j) {
          const int i = j * ACT + t;
          const bool valid = i < n;
          const uint32_t x = load(valid ? i : n - 1, j);
          key[j] = valid ? x : 0u;
          mn = min(mn, valid ? x : 0xFFFFFFFFu);
          mx = max(mx, key[j]);
        }
      }
    }
    mn = wave_min_u32(mn);
    mx = wave_max_u32(mx);
    if (lane == 0) {
      sh.wmn[w] = mn;
      sh.wmx[w] = mx;
    }
    hist4[t] = make_int4(0, 0, 0, 0);
  }
  __syncthreads();
  mn = 0xFFFFFFFFu;
  mx = 0u;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    mn = min(mn, sh.wmn[i]);
    mx = max(mx, sh.wmx[i]);
  }

  // 2./3. the boundary: keep every key > hi and `need` keys of [lo, hi]
  int bn[MAXS];
  uint32_t lo = mn, hi = mn;
  int need = k;
  if (mx != mn) {
    const float fmin = key_to_f32(mn), span = key_to_f32(mx) - fmin;
    const float scale = (float)NB / span;
    const bool linear = span > 0.f && span < 3.0e38f && scale < 3.0e38f;
    const int bits = 32 - __clz(mx - mn);
    const int shift = bits > LOGNB ? bits - LOGNB : 0;
    // the bin function is chosen once, outside the slot loops
    auto pass1 = [&](auto bin_of) {
#pragma unroll
      for (int j0 = 0; j0 < MAXS; j0 += 4) {
#pragma unroll
        for (int j = j0; j < j0 + 4; ++j) bn[j] = -1;
        if (j0 < ns) {
#pragma unroll
          for (int j = j0; j < j0 + 4; ++j) {
            const bool valid = j * ACT + t < n;
            const int bj = bin_of(key[j]);
            bn[j] = valid ? bj : -1;
            atomicAdd(&sh.hist[valid ? bj : NB + lane], 1);
          }
        }
      }
    };
    if (act) {
      if (linear)
        pass1([&](uint32_t x) { return min(NB - 1, (int)((key_to_f32(x) - fmin) * scale)); });
      else
        pass1([&](uint32_t x) { return (int)((x - mn) >> shift); });
    }
    __syncthreads();
    search(k);
    __syncthreads();
    const int b = sh.bc[0];
    const int nb_need = sh.bc[1], nb_cnt = sh.bc[2];
    {
      // exact key range of bin b
      uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
      if (act) {
#pragma unroll
        for (int j = 0; j < MAXS; ++j) {  // slots past the end have bn = -1
          const bool in = bn[j] == b;
          kmn = min(kmn, in ? key[j] : 0xFFFFFFFFu);
          kmx = max(kmx, in ? key[j] : 0u);
        }
        kmn = wave_min_u32(kmn);
        kmx = wave_max_u32(kmx);
        if (lane == 0) {
          sh.wmn[w] = kmn;
          sh.wmx[w] = kmx;
        }
      }
      __syncthreads();
      lo = 0xFFFFFFFFu;
      hi = 0u;
#pragma unroll
      for (int i = 0; i < W; ++i) {
        lo = min(lo, sh.wmn[i]);
        hi = max(hi, sh.wmx[i]);
      }
      need = nb_need;
      // narrow [lo, hi] in key space unless bin b is kept whole; the
      // histogram was cleared by search()
      while (nb_cnt != nb_need && lo != hi) {
        const uint32_t range = hi - lo;
        const int rb = 32 - __clz(range);
        const int s = rb > LOGNB ? rb - LOGNB : 0;
        if (act) {
#pragma unroll
          for (int j0 = 0; j0 < MAXS; j0 += 4)
            if (j0 < ns) {
#pragma unroll
              for (int j = j0; j < j0 + 4; ++j) {
                const uint32_t d = key[j] - lo;  // wraps above range below lo
                const bool in = (j * ACT + t < n) & (d <= range);
                atomicAdd(&sh.hist[in ? (int)(d >> s) : NB + lane], 1);
              }
            }
        }
        __syncthreads();
        search(need);
        __syncthreads();
        const int bb = sh.bc[0], need2 = sh.bc[1], cnt2 = sh.bc[2];
        __syncthreads();  // every thread has read bc before the next pass rewrites it
        lo += (uint32_t)bb << s;
        hi = lo + (s == 0 ? 0u : min(range - ((uint32_t)bb << s), (1u << s) - 1u));
        need = need2;
        if (cnt2 == need2) break;  // the boundary range is kept whole
      }
    }
  }

  // 4. compaction in index order: g = strictly above the boundary, e = in the
  // boundary range [lo, hi] (kept while fewer than `need` precede it)
  auto classify = [&](int j, bool& g, bool& e) {
    const bool valid = j * ACT + t < n;
    g = valid & (key[j] > hi);
    e = valid & (key[j] >= lo) & (key[j] <= hi);
  };
  if (act) {
#pragma unroll
    for (int j0 = 0; j0 < MAXS; j0 += 4)
      if (j0 < ns) {
#pragma unroll
        for (int j = j0; j < j0 + 4; ++j) {
          bool g, e;
          classify(j, g, e);
          const int cg = __popcll(__ballot(g)), ce = __popcll(__ballot(e));
          if (lane == 0) sh.cnt[j * W + w] = cg | (ce << 16);
        }
      }
  }
  __syncthreads();
  if (w == 0) {  // exclusive prefix over (slot, wave) in index order
    int run = 0;
    const int used = ((ns + 3) & ~3) * W;  // every slot of the used groups
#pragma unroll
    for (int base = 0; base < MAXS * W; base += 64) {
      const int idx = base + lane;
      const bool in = idx < used;
      const int v = in ? sh.cnt[idx] : 0;
      int tot;
      const int incl = wave_incl_scan(v, &tot);
      if (in) sh.cnt[idx] = run + incl - v;
      run += tot;
    }
  }
  __syncthreads();
  if (act) {
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int j0 = 0; j0 < MAXS; j0 += 4)
      if (j0 < ns) {
#pragma unroll
        for (int j = j0; j < j0 + 4; ++j) {
          bool g, e;
          classify(j, g, e);  // false past the end
          const uint64_t gm = __ballot(g), em = __ballot(e);
          const int pre = sh.cnt[j * W + w];
          const int G = (pre & 0xFFFF) + __popcll(gm & below);
          const int E = (pre >> 16) + __popcll(em & below);
          const int i = j * ACT + t;
          out(G + min(E, need), g | (e & (E < need)), i < n ? i : n - 1, j);
        }
      }
  }
}

}  // namespace wf
