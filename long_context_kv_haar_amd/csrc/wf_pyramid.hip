// WaveFilter pyramid kernels for gfx950 (MI355X), run once per cache refresh:
//   pyramid_top_kernel    A_L of the prompt keys in one streaming pass
//   pyramid_level_kernel  one analysis level, for the all-levels inspection mode
//
// Citations are to WaveFilter (arXiv 2606.00724).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "wf_pyramid.h"
#include "wf_types.h"

namespace wf {

// ===========================================================================
// Pyramid: A_L[n] = 2^{-L/2} sum_{t in [n 2^L, (n+1) 2^L)} k_t
// (section 2.2, eq. 5 iterated L times with orthonormal Haar filters: the
// pairwise sums telescope into one block sum).  One wave owns a run of
// rows_per_item consecutive prompt rows; lane (r, col) streams 16-byte
// vectors of rows r, r + RPP, ... at column block col, so each wave-wide
// load reads 1 KiB of contiguous memory.  The keys are read once, so the
// loads are non-temporal (they do not displace reusable cache lines; this
// streams measurably faster).  Row groups of one block are reduced with
// cross-lane shuffles.  A workgroup is one wave, with its 16 loads in
// flight together (measured at 64K tokens: 6.38 TB/s, against 6.28 with one
// load in flight per wave and 6.06 with 4-wave workgroups).
// ===========================================================================
template <typename T> struct Vec16;
template <> struct Vec16<float> {
  static constexpr int N = 4;
  typedef f32x4 Raw;
  __device__ __forceinline__ static Raw load(const float* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  }
  __device__ __forceinline__ static void add(const Raw& x, float* acc) {
    acc[0] += x[0]; acc[1] += x[1]; acc[2] += x[2]; acc[3] += x[3];
  }
};
template <> struct Vec16<bf16_t> {
  static constexpr int N = 8;
  typedef u32x4 Raw;
  __device__ __forceinline__ static Raw load(const bf16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  }
  __device__ __forceinline__ static void add(const Raw& x, float* acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += bf16_to_f32(x[i] & 0xFFFFu);
      acc[2 * i + 1] += bf16_to_f32(x[i] >> 16);
    }
  }
};

// acc += the vectors at src + p * stride for p = 0 .. npass - 1, added in
// that order.  Each group of 16 passes is requested before any of it is
// added (passes past the end load the last one again, in bounds, and are
// not added), so a wave keeps up to 16 loads in flight; left to itself the
// compiler adds each vector as it arrives, one load at a time.  The build
// and the refresh both sum through here, so their rows agree bit for bit.
template <typename T>
__device__ __forceinline__ void sum_passes(const T* src, int64_t stride, int npass, float* acc) {
  constexpr int G = 16;
  for (int g0 = 0; g0 < npass; g0 += G) {
    typename Vec16<T>::Raw x[G];
#pragma unroll
    for (int i = 0; i < G; ++i) x[i] = Vec16<T>::load(src + (int64_t)min(g0 + i, npass - 1) * stride);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < G; ++i)
      if (g0 + i < npass) Vec16<T>::add(x[i], acc);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(64) void pyramid_top_kernel(const T* __restrict__ k, int64_t head_stride,
                                                          int heads_total, int n_prompt, int levels,
                                                          int rows_per_item, int64_t items_per_head,
                                                          float scale, float* __restrict__ a_top) {
  constexpr int VE = Vec16<T>::N;
  constexpr int V = D / VE;     // vectors per row
  constexpr int RPP = 64 / V;   // rows per wave pass
  const int lane = threadIdx.x & 63;
  const int64_t item = blockIdx.x;
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
    sum_passes<T>(src, (int64_t)RPP * D, passes, acc);
  } else {  // the last rows of a prompt that is not a whole number of items
    for (int p = 0; p < passes; ++p)
      if (row0 + (int64_t)p * RPP < n_prompt) Vec16<T>::add(Vec16<T>::load(src + (int64_t)p * RPP * D), acc);
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

// ===========================================================================
// Incremental refresh (the cached prompt keys change on the cache's schedule,
// section 2.1 eq. 4; the low-frequency keys of section 3.1 follow them): one
// wave per (item, head, listed block) recomputes A_L[block] from the block's
// 2^L rows.  Lane layout, pass order and the cross-lane reduction tree are
// those of pyramid_top_kernel, so a refreshed row is bit for bit the row a
// full rebuild on the same keys writes.
// ===========================================================================
template <typename T, int D>
__global__ __launch_bounds__(64) void pyramid_refresh_kernel(RefreshLaunch r) {
  constexpr int VE = Vec16<T>::N;
  constexpr int V = D / VE;     // vectors per row
  constexpr int RPP = 64 / V;   // rows per wave pass
  const int lane = threadIdx.x & 63;
  // one wave per workgroup, so the unit and everything derived from it are
  // scalar: the item descriptor comes through scalar loads
  const int64_t unit = blockIdx.x;
  if (unit >= r.units_total) return;
  int it = 0;  // the item holding this unit
  for (int i = 1; i < r.n_items; ++i)
    if (unit >= r.items[i].unit_begin) it = i;
  const RefreshItem& I = r.items[it];
  const int64_t u = unit - I.unit_begin;
  const int64_t head = (u <= 0x7FFFFFFF) ? (int64_t)((uint32_t)u / (uint32_t)I.n_blocks) : u / I.n_blocks;
  const int block = I.blocks[u - head * I.n_blocks];
  if (block < 0 || block >= I.n_top) return;  // wave-uniform
  const int rows = 1 << I.levels;
  const int col = lane % V, rr = lane / V;
  const T* src = reinterpret_cast<const T*>(I.k) + head * I.head_stride + ((int64_t)block * rows + rr) * D + col * VE;
  float acc[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) acc[e] = 0.f;
  if (rows >= RPP) {  // whole passes (rows is a power of two), summed as the build sums them
    sum_passes<T>(src, (int64_t)RPP * D, rows / RPP, acc);
  } else if (rr < rows) {  // a block smaller than one pass
    Vec16<T>::add(Vec16<T>::load(src), acc);
  }
  const int G = rows < RPP ? rows : RPP;  // row groups holding this block's rows
  for (int o = V; o < V * G; o <<= 1) {
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[e] += __shfl_xor(acc[e], o, 64);
  }
  if (rr == 0) {
    const float scale = I.scale;
    float* dst = I.a_top + (head * I.n_top + block) * D + col * VE;
#pragma unroll
    for (int e = 0; e < VE; e += 4)
      *reinterpret_cast<float4*>(dst + e) =
          make_float4(acc[e] * scale, acc[e + 1] * scale, acc[e + 2] * scale, acc[e + 3] * scale);
  }
}

// One analysis level with Daubechies' four-tap filters and periodic
// extension (the longer-basis variant of section 3.1's wavelet psi):
// A[n] = sum_m g[m] x[(2n + m) mod n_in], D[n] likewise with h, in the same
// alignment as the Haar level above (output n starts at input 2n).
struct Db2Filters {
  float g[4], h[4];
};

// Four consecutive columns of one input row as float32.
template <typename T>
__device__ __forceinline__ void load4(const T* p, float (&x)[4]);
template <> __device__ __forceinline__ void load4<float>(const float* p, float (&x)[4]) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}
template <> __device__ __forceinline__ void load4<bf16_t>(const bf16_t* p, float (&x)[4]) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  x[0] = bf16_to_f32(v.x & 0xFFFFu); x[1] = bf16_to_f32(v.x >> 16);
  x[2] = bf16_to_f32(v.y & 0xFFFFu); x[3] = bf16_to_f32(v.y >> 16);
}

// Thread = four consecutive columns of one output row (one float4 of A and
// of D); the four input rows are all requested before the arithmetic.
template <typename T>
__global__ __launch_bounds__(256) void pyramid_level_db2_kernel(const T* __restrict__ src, int64_t src_head_stride,
                                                                int heads_total, int n_in, int d, Db2Filters f,
                                                                float* __restrict__ a_out, float* __restrict__ d_out) {
  const int n_out = n_in >> 1;
  const int d4 = d >> 2;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_head = (int64_t)n_out * d4;
  if (idx >= per_head * heads_total) return;
  const int64_t head = idx / per_head;
  const int64_t rem = idx - head * per_head;
  const int64_t n = rem / d4, c = (rem - n * d4) * 4;
  const T* base = src + head * src_head_stride;
  float x[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m) load4<T>(base + ((2 * n + m) % n_in) * d + c, x[m]);
  float a[4] = {0.f, 0.f, 0.f, 0.f}, dd[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[e] += f.g[m] * x[m][e];
      dd[e] += f.h[m] * x[m][e];
    }
  *reinterpret_cast<float4*>(a_out + 4 * idx) = make_float4(a[0], a[1], a[2], a[3]);
  *reinterpret_cast<float4*>(d_out + 4 * idx) = make_float4(dd[0], dd[1], dd[2], dd[3]);
}

hipError_t launch_refresh(const RefreshLaunch& r, hipStream_t s) {
  if (r.units_total <= 0) return hipSuccess;
  if (r.units_total > 0x7FFFFFFF) return hipErrorInvalidValue;  // one workgroup per unit
  const unsigned grid = (unsigned)r.units_total;
  if (r.bf16) {
    if (r.head_dim == 128)
      hipLaunchKernelGGL((pyramid_refresh_kernel<bf16_t, 128>), dim3(grid), dim3(64), 0, s, r);
    else
      hipLaunchKernelGGL((pyramid_refresh_kernel<bf16_t, 64>), dim3(grid), dim3(64), 0, s, r);
  } else {
    if (r.head_dim == 128)
      hipLaunchKernelGGL((pyramid_refresh_kernel<float, 128>), dim3(grid), dim3(64), 0, s, r);
    else
      hipLaunchKernelGGL((pyramid_refresh_kernel<float, 64>), dim3(grid), dim3(64), 0, s, r);
  }
  return hipGetLastError();
}

hipError_t launch_pyramid(const PyramidLaunch& a, hipStream_t s) {
  const int L = a.levels;
  uint8_t* base = reinterpret_cast<uint8_t*>(a.base);
  if (a.db2) {
    Db2Filters f;
    const double s3 = sqrt(3.0), den = 4.0 * sqrt(2.0);
    const double g[4] = {(1.0 + s3) / den, (3.0 + s3) / den, (3.0 - s3) / den, (1.0 - s3) / den};
    for (int m = 0; m < 4; ++m) {
      f.g[m] = (float)g[m];
      f.h[m] = (float)((m & 1) ? -g[3 - m] : g[3 - m]);
    }
    for (int j = 1; j <= L; ++j) {
      const int n_in = a.n_prompt >> (j - 1);
      const int64_t total = (int64_t)(n_in >> 1) * (a.head_dim / 4) * a.heads_total;  // one thread per float4
      const unsigned grid = (unsigned)((total + 255) / 256);
      float* a_out = reinterpret_cast<float*>(base + a.band_off_a[j]);
      float* d_out = reinterpret_cast<float*>(base + a.band_off_d[j]);
      if (j == 1 && a.bf16)
        hipLaunchKernelGGL(pyramid_level_db2_kernel<bf16_t>, dim3(grid), dim3(256), 0, s,
                           reinterpret_cast<const bf16_t*>(a.k), a.head_stride, a.heads_total, n_in, a.head_dim, f,
                           a_out, d_out);
      else if (j == 1)
        hipLaunchKernelGGL(pyramid_level_db2_kernel<float>, dim3(grid), dim3(256), 0, s,
                           reinterpret_cast<const float*>(a.k), a.head_stride, a.heads_total, n_in, a.head_dim, f,
                           a_out, d_out);
      else
        hipLaunchKernelGGL(pyramid_level_db2_kernel<float>, dim3(grid), dim3(256), 0, s,
                           reinterpret_cast<const float*>(base + a.band_off_a[j - 1]), (int64_t)n_in * a.head_dim,
                           a.heads_total, n_in, a.head_dim, f, a_out, d_out);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (L > 0) return hipSuccess;
    // L == 0: A_0 is the keys themselves, converted below by the streaming kernel
  } else if (a.all_levels) {
    // level by level, each level reading the previous one
    for (int j = 1; j <= L; ++j) {
      const int n_out = a.n_prompt >> j;
      const int64_t total = (int64_t)n_out * a.head_dim * a.heads_total;
      const unsigned grid = (unsigned)((total + 255) / 256);
      float* a_out = reinterpret_cast<float*>(base + a.band_off_a[j]);
      float* d_out = reinterpret_cast<float*>(base + a.band_off_d[j]);
      if (j == 1) {
        if (a.bf16)
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
  const int vec_elems = a.bf16 ? 8 : 4;
  const int rpp = 64 / (a.head_dim / vec_elems);
  const int rows_per_item = (1 << L) > rpp ? (1 << L) : rpp;
  const int64_t items_per_head = (a.n_prompt + rows_per_item - 1) / rows_per_item;
  const int64_t items = items_per_head * a.heads_total;
  const unsigned grid = (unsigned)items;  // one wave per item
  const float scale = (float)ldexp(1.0, -L / 2) * ((L & 1) ? 0.70710678118654752440f : 1.0f);
#define PYR_LAUNCH(T, D)                                                                                   \
  hipLaunchKernelGGL((pyramid_top_kernel<T, D>), dim3(grid), dim3(64), 0, s,                          \
                     reinterpret_cast<const T*>(a.k), a.head_stride, a.heads_total, a.n_prompt, L,    \
                     rows_per_item, items_per_head, scale, a.base)
  if (a.bf16) {
    if (a.head_dim == 128) PYR_LAUNCH(bf16_t, 128); else PYR_LAUNCH(bf16_t, 64);
  } else {
    if (a.head_dim == 128) PYR_LAUNCH(float, 128); else PYR_LAUNCH(float, 64);
  }
#undef PYR_LAUNCH
  return hipGetLastError();
}

}  // namespace wf
