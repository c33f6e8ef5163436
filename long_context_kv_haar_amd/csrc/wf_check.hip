// Input checks of the debug option (WF_OPT_CHECK): one scan over a call's
// inputs that records, in a status word at the start of the call's
// workspace, which preconditions the inputs break.  The selection and
// attention kernels themselves are unchanged: they still clamp every index
// they read into its buffer, so a bad entry never leads to an access outside
// the buffers; the scan reports that a clamp happened.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wf_internal.h"

namespace wf {

namespace {

constexpr int kCheckThreads = 256;
constexpr int kCheckBlocks = 2048;

// A 16-byte vector of float32 (or of bfloat16) holds a NaN or an infinity:
// its exponent field is all ones.
__device__ __forceinline__ uint32_t ones_f32(uint32_t w) { return (w & 0x7F800000u) == 0x7F800000u ? 1u : 0u; }
__device__ __forceinline__ uint32_t ones_bf16x2(uint32_t w) {
  return ((w & 0x7F80u) == 0x7F80u ? 1u : 0u) | ones_f32(w);  // the high half has the float32 field's position
}
__device__ __forceinline__ bool nonfinite_f32(uint4 v) {
  return (ones_f32(v.x) | ones_f32(v.y) | ones_f32(v.z) | ones_f32(v.w)) != 0u;
}
__device__ __forceinline__ bool nonfinite_bf16(uint4 v) {
  return (ones_bf16x2(v.x) | ones_bf16x2(v.y) | ones_bf16x2(v.z) | ones_bf16x2(v.w)) != 0u;
}

// Any non-finite value among n16 16-byte vectors, grid-stride.
__device__ __forceinline__ bool scan_nonfinite(const void* p, int64_t n16, bool bf16) {
  const uint4* v = reinterpret_cast<const uint4*>(p);
  bool bad = false;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const uint4 x = v[i];
    bad = bad || (bf16 ? nonfinite_bf16(x) : nonfinite_f32(x));
  }
  return bad;
}

// Any entry outside [0, hi) among n int32 values, grid-stride.
__device__ __forceinline__ bool scan_range(const int32_t* p, int64_t n, int hi) {
  bool bad = false;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int32_t x = p[i];
    bad = bad || x < 0 || x >= hi;
  }
  return bad;
}

__global__ __launch_bounds__(1) void check_clear_kernel(uint32_t* status) { *status = 0u; }

__global__ __launch_bounds__(kCheckThreads) void check_inputs_kernel(CheckArgs c) {
  uint32_t bits = 0u;
  bits |= scan_nonfinite(c.q, c.q_bytes / 16, c.bf16) ? WF_CHECK_NONFINITE_Q : 0u;
  bits |= scan_nonfinite(c.k, c.kv_bytes / 16, c.bf16) ? WF_CHECK_NONFINITE_K : 0u;
  bits |= scan_nonfinite(c.v, c.kv_bytes / 16, c.bf16) ? WF_CHECK_NONFINITE_V : 0u;
  if (c.a_top) bits |= scan_nonfinite(c.a_top, c.a_bytes / 16, false) ? WF_CHECK_NONFINITE_PYRAMID : 0u;
  if (c.gen_idx) bits |= scan_range(c.gen_idx, c.n_gen, c.n_tot) ? WF_CHECK_GEN_INDEX : 0u;
  if (c.sel) bits |= scan_range(c.sel, c.n_sel, c.n_tot) ? WF_CHECK_SEL_INDEX : 0u;
  // one atomic per wave that found something
  const uint32_t lo = (uint32_t)__ballot(bits != 0u);
  const uint32_t hi = (uint32_t)(__ballot(bits != 0u) >> 32);
  if (lo | hi) {
    uint32_t all = bits;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) all |= (uint32_t)__shfl_xor((int)all, off, 64);
    if ((threadIdx.x & 63) == 0) atomicOr(c.status, all);
  }
}

}  // namespace

hipError_t launch_check_clear(uint32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(check_clear_kernel, dim3(1), dim3(1), 0, s, status);
  return hipGetLastError();
}

hipError_t launch_check(const CheckArgs& c, hipStream_t s) {
  hipLaunchKernelGGL(check_inputs_kernel, dim3(kCheckBlocks), dim3(kCheckThreads), 0, s, c);
  return hipGetLastError();
}

}  // namespace wf
