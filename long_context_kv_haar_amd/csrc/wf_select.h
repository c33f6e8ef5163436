// Workgroup-level selection machinery of the coarse Top-K and the recursive
// refinement (WaveFilter, Figure 2 (c)-(d)), and the hand-over of data
// between the workgroups of one launch.
//
// Selection rule everywhere: keep the k best candidates, higher score first
// and on equal scores the lower position; kept sets are reported ascending.
//
// Layout.  A workgroup of kSelThreads threads holds one level's positions
// in contiguous runs: thread t holds the S positions [t S, t S + S) (S a
// power of two).  The refinement descends a binary tree, so with S0
// level-0 positions per thread, thread t holds level-j positions
// [(t S0) >> j, ...): max(1, S0 >> j) of them.  A position's two children
// are held by the same thread as the position, so whether a candidate's
// parent was kept is known in registers, without any exchange.  At levels
// with 2^j > S0 one position spans several threads; each of them holds a
// copy, the first one (its owner) counts it, and every copy takes the same
// decision (the rule below is a function of the score, the position and
// shared state only).
//
// One level (select_level), all threads:
//   A. every valid owned candidate adds one to a histogram of kSelBins bins
//      linear in the score over [smin, smax] (monotone in the score, so a
//      higher bin holds only greater scores);                   barrier B
//   S. every wave finds by itself the bin b of the k-th best, the count
//      still needed from it and its size (a wave scan over the bins);
//   W. if bin b is kept whole, the decision is bin >= b: no more barriers;
//   L. else the owned candidates of bin b are listed as (order key, ~pos)
//      pairs;                                                    barrier C
//      every holder ranks its bin-b candidates against the list (greater
//      key, or equal key and lower position, ranks higher) and keeps those
//      ranked below the count needed;
//   D. a bin with more candidates than the list holds (heavy ties) is
//      narrowed by histogram passes over the key bits, and ties on one key
//      value go to the lowest positions (a workgroup scan in position order).
// Histograms are triple-buffered and lists double-buffered, each cleared
// one level after its last read, so a level costs barrier B, plus C when
// its boundary bin is not kept whole.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wf_device.h"

namespace wf {

constexpr int kSelThreads = 256;                // threads of a selecting workgroup
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelBins = 512;                   // linear histogram bins: 8 per lane of a wave
constexpr int kSelList = 256;                   // boundary-bin list capacity
constexpr int kSelMaxSlots = 32;                // positions per thread held in registers

// ---------------------------------------------------------------------------
// Hand-over between the workgroups of one launch.  The L2 of an XCD is not
// coherent with the other XCDs' L2, so data that another workgroup of the
// same launch reads is written with agent-scope stores (written through to
// memory) and read with agent-scope loads (never served from a stale line of
// the reader's L2).  A workgroup counts its arrival only after its own
// stores have completed; the last one to arrive sees every other's data.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent2(float* p, float x, float y) {  // p 8-byte aligned
  const uint64_t v = (uint64_t)__float_as_uint(x) | ((uint64_t)__float_as_uint(y) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
  return __uint_as_float(__hip_atomic_load(const_cast<uint32_t*>(reinterpret_cast<const uint32_t*>(p)),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ uint32_t load_agent(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_agent2(const float* p) {  // p 8-byte aligned
  const uint64_t v = __hip_atomic_load(const_cast<uint64_t*>(reinterpret_cast<const uint64_t*>(p)), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}

// Arrival of this workgroup at a counter shared by the n workgroups of one
// item; true, uniformly, in the last one to arrive.  The counter wraps back
// to zero on the last arrival (the atomic increment with bound n - 1), so it
// is ready for the next launch.  Every thread must call it; each wave's
// agent-scope stores complete before the barrier.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t n, int* flag_lds) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's stores are visible at agent scope
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0)
    *flag_lds = __builtin_amdgcn_atomic_inc32(counter, n - 1u, __ATOMIC_RELAXED, "agent") == n - 1u;
  __syncthreads();
  return *flag_lds != 0;
}

// ---------------------------------------------------------------------------
// Selection state in LDS.
// ---------------------------------------------------------------------------
struct SelShared {
  int hist[3][kSelBins];          // triple-buffered histograms (zero between uses)
  uint64_t list[2][kSelList];     // boundary lists by level parity
  int list_n[2];
  int last;                       // arrive_last flag
  int pad;
  uint32_t wmn[kSelWaves], wmx[kSelWaves];
  int wsum[8][kSelWaves];         // per-wave totals of the workgroup scans
};

struct SelCursor {
  int hb = 0, lb = 0;  // histogram buffer and list buffer of the next level
};

// Zero the selection state; the caller synchronises before the first level.
__device__ __forceinline__ void sel_init(SelShared& sh) {
  for (int i = threadIdx.x; i < 3 * kSelBins; i += kSelThreads) (&sh.hist[0][0])[i] = 0;
  if (threadIdx.x < 2) sh.list_n[threadIdx.x] = 0;
}

// Bins linear in the score over [smin, smax]: a composition of monotone
// float operations, so it never inverts an order.  A degenerate range puts
// everything in bin 0.
struct LinBins {
  float scale, off;
  bool ok;
  __device__ __forceinline__ LinBins(float smin, float smax) {
    const float span = smax - smin;
    scale = __fdividef((float)kSelBins, span);
    ok = span > 0.f && span < 3.0e38f && scale > 0.f && scale < 3.0e38f;
    off = -smin * scale;
  }
  __device__ __forceinline__ int operator()(float s) const {
    return ok ? min(kSelBins - 1, max(0, (int)fmaf(s, scale, off))) : 0;
  }
};

// Ranking key of a candidate: greater is better (higher score, then lower position).
__device__ __forceinline__ uint64_t rank_key(uint32_t okey, int pos) {
  return ((uint64_t)okey << 32) | (uint64_t)(~(uint32_t)pos);
}

// The bin holding the want-th best entry (1-based, counted from the top) of
// a kSelBins-bin histogram: its index, the count still needed from it and
// its size.  Each wave computes it on its own; want <= total is required.
__device__ __forceinline__ void find_bin(const int* hist, int want, int& b, int& need, int& cnt) {
  const int lane = threadIdx.x & 63;
  const int4* h4 = reinterpret_cast<const int4*>(hist + 8 * lane);
  const int r = lane & 1;  // read order alternates between lanes (spreads the LDS banks)
  const int4 x = h4[r], y = h4[r ^ 1];
  const int4 lo = r ? y : x, hi = r ? x : y;
  const int c[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  int tot = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) tot += c[i];
  int all;
  const int incl = wave_incl_scan(tot, &all);
  const int above = all - incl;  // entries in the bins of higher lanes
  const uint64_t om = __ballot((above < want) & (want <= above + tot));
  const int owner = om ? (int)__ffsll((unsigned long long)om) - 1 : 0;
  int ab = above, bb = 0, nd = 0, ct = 0;
#pragma unroll
  for (int i = 7; i >= 0; --i) {
    const bool hit = (ab < want) & (want <= ab + c[i]);
    bb = hit ? i : bb;
    nd = hit ? want - ab : nd;
    ct = hit ? c[i] : ct;
    ab += c[i];
  }
  b = 8 * owner + __builtin_amdgcn_readlane(bb, owner);
  need = __builtin_amdgcn_readlane(nd, owner);
  cnt = __builtin_amdgcn_readlane(ct, owner);
}

// Exclusive prefix over the workgroup of one int per thread, in thread
// order; row r of sh.wsum holds the wave totals (one barrier; the caller
// must not reuse row r before another barrier).
__device__ __forceinline__ int block_excl_scan(int x, SelShared& sh, int r, int* total = nullptr) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int wt;
  const int incl = wave_incl_scan(x, &wt);
  if (lane == 63) sh.wsum[r][w] = wt;
  __syncthreads();
  int base = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kSelWaves; ++i) {
    const int v = sh.wsum[r][i];
    base += (i < w) ? v : 0;
    all += v;
  }
  if (total) *total = all;
  return base + incl - x;
}

// One level: returns the kept mask over this thread's S slots.
//   sc     the slots' scores (slot i is position pos0 + i)
//   valid  candidates (a slot past the level's end is never valid)
//   owned  valid slots this thread counts (all of them, except copies of a
//          position whose first holder is another thread)
//   k      how many to keep (at most the number of valid candidates)
//   smin, smax  a range holding every candidate's score (any finite range
//          keeps the result exact; a tight one keeps the lists short)
// All threads of the workgroup call it with the same k, smin, smax.
template <int S>
__device__ __forceinline__ uint32_t select_level(const float (&sc)[S], uint32_t valid, uint32_t owned, int pos0, int k,
                                                 float smin, float smax, SelShared& sh, SelCursor& cur) {
  const int t = threadIdx.x;
  const LinBins bin(smin, smax);
  int* hist = sh.hist[cur.hb];
  // A. histogram of the owned candidates
#pragma unroll
  for (int i = 0; i < S; ++i)
    if ((owned >> i) & 1u) atomicAdd(&hist[bin(sc[i])], 1);
  __syncthreads();  // B
  // the previous level's histogram and list are read no more: clear them
  // for the levels after this one
  {
    int* old = sh.hist[(cur.hb + 2) % 3];
    for (int i = t; i < kSelBins; i += kSelThreads) old[i] = 0;
    if (t == 0) sh.list_n[cur.lb ^ 1] = 0;
  }
  int b, need, cnt;
  find_bin(hist, k, b, need, cnt);
  uint32_t kept = 0u;
  if (cnt == need) {  // W. bin b is kept whole (uniform)
#pragma unroll
    for (int i = 0; i < S; ++i) kept |= (((valid >> i) & 1u) && bin(sc[i]) >= b) ? (1u << i) : 0u;
  } else if (cnt <= kSelList) {  // L. exact ranks inside bin b (uniform)
    uint64_t* list = sh.list[cur.lb];
    uint32_t inb = 0u;
#pragma unroll
    for (int i = 0; i < S; ++i) inb |= (((valid >> i) & 1u) && bin(sc[i]) == b) ? (1u << i) : 0u;
    const uint32_t mine = inb & owned;
    {
      const int n = __popc(mine);
      int wt;
      const int incl = wave_incl_scan(n, &wt);
      int base = 0;
      if ((threadIdx.x & 63) == 63 && wt > 0) base = atomicAdd(&sh.list_n[cur.lb], wt);
      base = __builtin_amdgcn_readlane(base, 63) + incl - n;
#pragma unroll
      for (int i = 0; i < S; ++i)
        if ((mine >> i) & 1u) list[base++] = rank_key(order_key(sc[i]), pos0 + i);
    }
    __syncthreads();  // C
    const int nl = sh.list_n[cur.lb];
#pragma unroll
    for (int i = 0; i < S; ++i) {
      if ((inb >> i) & 1u) {
        const uint64_t me = rank_key(order_key(sc[i]), pos0 + i);
        int rank = 0;
        for (int e = 0; e < nl; ++e) rank += list[e] > me ? 1 : 0;
        kept |= rank < need ? (1u << i) : 0u;
      }
      kept |= (((valid >> i) & 1u) && bin(sc[i]) > b) ? (1u << i) : 0u;
    }
  } else {  // D. heavy ties: narrow bin b by the key bits
    const int lane = t & 63, w = t >> 6;
    uint32_t inb = 0u;
    uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const bool in = ((valid >> i) & 1u) && bin(sc[i]) == b;
      inb |= in ? (1u << i) : 0u;
      const uint32_t key = order_key(sc[i]);
      kmn = in ? min(kmn, key) : kmn;
      kmx = in ? max(kmx, key) : kmx;
    }
    kmn = wave_min_u32(kmn);
    kmx = wave_max_u32(kmx);
    if (lane == 0) {
      sh.wmn[w] = kmn;
      sh.wmx[w] = kmx;
    }
    __syncthreads();
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int i = 0; i < kSelWaves; ++i) {
      lo = min(lo, sh.wmn[i]);
      hi = max(hi, sh.wmx[i]);
    }
    int nd = need;
    bool whole = false;
    int* h2 = sh.hist[(cur.hb + 1) % 3];  // the next level's histogram: zero now, zero again on exit
    while (!whole && lo != hi) {          // uniform
      const uint32_t range = hi - lo;
      const int rb = 32 - __clz(range);
      const int s = rb > 9 ? rb - 9 : 0;  // (range >> s) < kSelBins
#pragma unroll
      for (int i = 0; i < S; ++i) {
        const uint32_t key = order_key(sc[i]);
        if (((inb & owned) >> i) & 1u && key >= lo && key <= hi) atomicAdd(&h2[(key - lo) >> s], 1);
      }
      __syncthreads();
      int b2, nd2, cnt2;
      find_bin(h2, nd, b2, nd2, cnt2);
      __syncthreads();  // every wave has read h2
      for (int i = t; i < kSelBins; i += kSelThreads) h2[i] = 0;
      __syncthreads();
      const uint32_t nlo = lo + ((uint32_t)b2 << s);
      hi = (s == 0) ? nlo : min(hi, nlo + ((1u << s) - 1u));
      lo = nlo;
      nd = nd2;
      whole = cnt2 == nd2;
    }
    // above the narrowed range: kept; inside: all (whole) or the nd lowest positions (ties)
    uint32_t tie = 0u;
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const uint32_t key = order_key(sc[i]);
      const bool ib = (inb >> i) & 1u;
      kept |= ((((valid >> i) & 1u) && bin(sc[i]) > b) || (ib && key > hi)) ? (1u << i) : 0u;
      tie |= (ib && key >= lo && key <= hi) ? (1u << i) : 0u;
    }
    if (whole) {
      kept |= tie;
    } else {
      const int before = block_excl_scan(__popc(tie & owned), sh, 0);
      // a copy held by a non-owner was counted by its owner, an earlier thread
      int r = before - ((tie & ~owned) ? 1 : 0);
#pragma unroll
      for (int i = 0; i < S; ++i)
        if ((tie >> i) & 1u) {
          kept |= (r < nd) ? (1u << i) : 0u;
          r += ((owned >> i) & 1u) ? 1 : 0;
        }
      __syncthreads();  // the scan row is free again
    }
  }
  cur.hb = (cur.hb + 1) % 3;
  cur.lb ^= 1;
  return kept;
}

}  // namespace wf
