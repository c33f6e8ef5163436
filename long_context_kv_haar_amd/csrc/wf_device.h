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

namespace wf {

typedef uint16_t bf16_t;  // bfloat16 storage
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Round-to-nearest-even float32 -> bfloat16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

__device__ __forceinline__ uint32_t pack_bf16(uint32_t lo, uint32_t hi) { return lo | (hi << 16); }

// ---------------------------------------------------------------------------
// MFMA 16x16 tiles.  D[i][j] += sum_k A[i][k] B[k][j]; lane l supplies row
// i = l % 16 of A and column j = l % 16 of B, with k-slots chosen by
// g = l / 16; the accumulator holds D[4g + r][l % 16], r = 0..3.  Only the
// pairing of A's and B's k-slots matters for a dot product, so every kernel
// assigns lane group g the contiguous quarter [g d/4, (g+1) d/4) of the
// contraction axis, read as one run of contiguous bytes.
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
  // Row `row` of a row-major [*, D] bfloat16 matrix, quarter g.
  __device__ __forceinline__ void load(const bf16_t* row, int g) {
    const u32x4* p = reinterpret_cast<const u32x4*>(row + g * (D / 4));
#pragma unroll
    for (int s = 0; s < STEPS; ++s) v[s] = p[s];
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

__device__ __forceinline__ float wave_max_xor_16_32(float x) {
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  x = fmaxf(x, __shfl_xor(x, 32, 64));
  return x;
}

__device__ __forceinline__ float wave_sum_xor_16_32(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

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
// Workgroup-wide Top-K by radix select on 32-bit keys (8-bit digits, most
// significant first), followed by a stable compaction in index order.  The
// kept set is: every key above the threshold, and of the keys equal to it,
// the ones with the lowest indices.  NT = threads in the workgroup (a
// multiple of 64).  All threads must call these functions together.
// ---------------------------------------------------------------------------
template <int NT> struct TopKShared {
  int hist[256];
  int wsum[NT / 64];
  int bcast[4];
};

template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    int s = wsum[i];
    base += (i < w) ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

struct Threshold {
  uint32_t prefix;  // kept: (key & mask) > prefix, or == prefix and among the first `need`
  uint32_t mask;
  int need;
};

template <int NT, class KeyFn>
__device__ Threshold radix_select(KeyFn key, int n, int k, TopKShared<NT>& sh) {
  Threshold t{0u, 0u, k};
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += NT) sh.hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += NT) {
      uint32_t x = key(i);
      if ((x & t.mask) == t.prefix) atomicAdd(&sh.hist[(x >> shift) & 255u], 1);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      const int h0 = sh.hist[4 * lane], h1 = sh.hist[4 * lane + 1];
      const int h2 = sh.hist[4 * lane + 2], h3 = sh.hist[4 * lane + 3];
      const int s = h0 + h1 + h2 + h3;
      int x = s;  // inclusive suffix sum over lanes
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        int y = __shfl_down(x, o, 64);
        if (lane + o < 64) x += y;
      }
      const int kk = t.need;
      int a = x - s;  // keys in higher lanes' bins
      int digit = -1, rem = 0, cnt = 0;
      if (a < kk && kk <= a + h3) { digit = 4 * lane + 3; rem = kk - a; cnt = h3; }
      a += h3;
      if (digit < 0 && a < kk && kk <= a + h2) { digit = 4 * lane + 2; rem = kk - a; cnt = h2; }
      a += h2;
      if (digit < 0 && a < kk && kk <= a + h1) { digit = 4 * lane + 1; rem = kk - a; cnt = h1; }
      a += h1;
      if (digit < 0 && a < kk && kk <= a + h0) { digit = 4 * lane; rem = kk - a; cnt = h0; }
      if (digit >= 0) {
        sh.bcast[0] = digit;
        sh.bcast[1] = rem;
        sh.bcast[2] = cnt;
      }
    }
    __syncthreads();
    const int digit = sh.bcast[0];
    t.need = sh.bcast[1];
    const int cnt = sh.bcast[2];
    t.prefix |= (uint32_t)digit << shift;
    t.mask |= 255u << shift;
    __syncthreads();
    if (cnt == t.need) break;  // the whole bin is kept: no tie to resolve below
  }
  return t;
}

// Calls out(o, i) for the kept indices i in ascending order, o = 0..k-1.
template <int NT, class KeyFn, class OutFn>
__device__ void topk_compact(KeyFn key, int n, Threshold t, TopKShared<NT>& sh, OutFn out) {
  const int seg = (n + NT - 1) / NT;
  const int i0 = min(n, (int)threadIdx.x * seg), i1 = min(n, i0 + seg);
  int eq = 0;
  for (int i = i0; i < i1; ++i) eq += ((key(i) & t.mask) == t.prefix);
  int tot;
  const int eq_before = block_exclusive_scan<NT>(eq, sh.wsum, &tot);
  int r = eq_before, cnt = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t x = key(i) & t.mask;
    const bool e = (x == t.prefix);
    cnt += (x > t.prefix) || (e && r < t.need);
    r += e;
  }
  int o = block_exclusive_scan<NT>(cnt, sh.wsum, &tot);
  r = eq_before;
  for (int i = i0; i < i1; ++i) {
    const uint32_t x = key(i) & t.mask;
    const bool e = (x == t.prefix);
    if ((x > t.prefix) || (e && r < t.need)) out(o++, i);
    r += e;
  }
}

}  // namespace wf
