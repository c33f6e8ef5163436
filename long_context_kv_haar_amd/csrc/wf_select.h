// Workgroup-level selection machinery of the coarse Top-K and the recursive
// refinement (WaveFilter, Figure 2 (c)-(d)).
//
// Selection rule everywhere: keep the k best candidates, higher score first
// and on equal scores the lower position; kept sets are reported ascending.
//
// Layout.  A workgroup of NT threads holds one level's positions
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
//   1. every valid owned candidate adds one to a histogram of kSelBins bins
//      linear in the score over [smin, smax] (monotone in the score, so a
//      higher bin holds only greater scores);                   barrier
//      every wave finds by itself the bin b of the k-th best, the count
//      still needed from it and its size (one wave scan over the bins);
//      if bin b is kept whole, the decision is bin >= b;
//   2. else the owned candidates of bin b add one to a histogram of kSelBins
//      sub-bins linear in the score over bin b's range;        barrier
//      every wave finds the sub-bin b2 of the still-needed best; with a few
//      dozen candidates in bin b it is almost always kept whole;
//   3. else the owned candidates of that cell are listed as (order key,
//      ~pos) pairs (greater pair = higher score, or equal score and lower
//      position);                                                barrier
//      the pair ranked at the count still needed is the threshold: a holder
//      keeps its cell candidates whose pair is at or above it;
//   4. a cell with more candidates than the list holds (heavy ties) is
//      narrowed by histogram passes over the key bits, and ties on one key
//      value go to the lowest positions (a workgroup scan in position order).
// Pass-1 histograms are triple-buffered, pass-2 histograms and lists
// double-buffered, each cleared one level after its last read, so a level
// costs one barrier, two when bin b is not kept whole.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wf_device.h"

namespace wf {

constexpr int kSelThreads = 256;                // threads of a cover workgroup (coarse Top-K)
constexpr int kRefineThreads = 1024;            // threads of a refinement workgroup
constexpr int kSelBins = 256;                   // linear histogram bins: 4 per lane of a wave
constexpr int kSelList = 256;                   // boundary-bin list capacity

// ---------------------------------------------------------------------------
// Selection state in LDS, for a workgroup of NT threads.
// ---------------------------------------------------------------------------
template <int NT> struct SelShared {
  static constexpr int NW = NT / 64;
  int hist[3][kSelBins + 64];     // triple-buffered pass-1 histograms (zero between uses), then a trash bin per lane
  int hist2[2][kSelBins + 64];    // double-buffered pass-2 histograms
  uint64_t list[2][kSelList];     // boundary lists by level parity
  int list_n[2];
  uint32_t wmn[NW], wmx[NW];
  int wsum[8][NW];                // per-wave totals of the workgroup scans
  float rsc[8], rof[8];           // the refinement: each level's bins over its score range (LinBins)
  int bc[4];                      // a level's boundary bin, broadcast by wave 0
  uint64_t tau;                   // a level's threshold pair, broadcast by wave 0
  // the refinement's per-call values, staged before its first barrier
  int bud[8];                     // k_L .. k_0
  int k0;                         // k_0
  int32_t* tsel;                  // the head's kept tokens (workspace)
  int32_t* sout;                  // and the caller's copy (or null)
  int32_t* dsel;                  // the head's per-level kept regions (or null)
  float* dscore;                  // and their scores (or null)
};

struct SelCursor {
  int hb = 0, lb = 0;  // histogram buffer and list buffer of the next level
};

// Zero the selection state; the caller synchronises before the first level.
template <int NT>
__device__ __forceinline__ void sel_init(SelShared<NT>& sh) {
  for (int i = threadIdx.x; i < 3 * (kSelBins + 64); i += NT) (&sh.hist[0][0])[i] = 0;
  for (int i = threadIdx.x; i < 2 * (kSelBins + 64); i += NT) (&sh.hist2[0][0])[i] = 0;
  if (threadIdx.x < 2) sh.list_n[threadIdx.x] = 0;
}

// Bins linear in the score over [smin, smax]: a composition of monotone
// float operations, so it never inverts an order.  A degenerate range puts
// everything in bin 0.
struct LinBins {
  float scale, off;  // both zero when the range is empty or not finite: every score then takes bin 0
  __device__ __forceinline__ LinBins(float scale_, float off_, bool) : scale(scale_), off(off_) {}
  __device__ __forceinline__ LinBins(float smin, float smax) {
    const float span = smax - smin;
    const float sc = (float)kSelBins * __builtin_amdgcn_rcpf(span);  // any monotone map will do: no exact division
    const bool ok = span > 0.f && span < 3.0e38f && sc > 0.f && sc < 3.0e38f;
    scale = ok ? sc : 0.f;
    off = ok ? -smin * sc : 0.f;
  }
  __device__ __forceinline__ int operator()(float s) const {
    return min(kSelBins - 1, max(0, (int)fmaf(s, scale, off)));
  }
  // kSelBins sub-bins over bin b's range: another monotone map of the score
  // (it orders only the candidates of bin b, so it need not match the bin
  // edges exactly)
  __device__ __forceinline__ LinBins sub(int b) const {
    LinBins r = *this;
    const bool ok = scale * (float)kSelBins < 3.0e38f;
    r.scale = ok ? scale * (float)kSelBins : 0.f;
    r.off = ok ? (off - (float)b) * (float)kSelBins : 0.f;
    return r;
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
  static_assert(kSelBins == 256, "four bins per lane");
  const int lane = threadIdx.x & 63;
  const int4 x = reinterpret_cast<const int4*>(hist)[lane];
  const int tot = x.x + x.y + x.z + x.w;
  // inclusive prefix of the lane totals: within each row of 16 lanes, then
  // the rows' totals carried to the rows above them by row broadcasts
  int s = tot;
  s += dpp_or0<0x111>(s);  // row_shr:1
  s += dpp_or0<0x112>(s);  // row_shr:2
  s += dpp_or0<0x114>(s);  // row_shr:4
  s += dpp_or0<0x118>(s);  // row_shr:8
  s += __builtin_amdgcn_update_dpp(0, s, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1 and 3
  s += __builtin_amdgcn_update_dpp(0, s, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2 and 3
  const int above = __builtin_amdgcn_readlane(s, 63) - s;  // entries in the bins of higher lanes
  const uint64_t om = __ballot((above < want) & (want <= above + tot));
  const int owner = om ? (int)__ffsll((unsigned long long)om) - 1 : 0;
  // the owner's bins, highest first: suffix counts within the lane
  const int a2 = above + x.w, a1 = a2 + x.z, a0 = a1 + x.y;
  const bool h3 = want <= a2, h2 = want <= a1, h1 = want <= a0;
  const int ab = h3 ? above : h2 ? a2 : h1 ? a1 : a0;
  const int ct = h3 ? x.w : h2 ? x.z : h1 ? x.y : x.x;
  const int bb = h3 ? 3 : h2 ? 2 : h1 ? 1 : 0;
  const uint32_t pk = __builtin_amdgcn_readlane((uint32_t)ct << 2 | (uint32_t)bb, owner);
  b = 4 * owner + (int)(pk & 3u);
  need = want - __builtin_amdgcn_readlane(ab, owner);
  cnt = (int)(pk >> 2);
}

// Exclusive prefix over the workgroup of one int per thread, in thread
// order; row r of sh.wsum holds the wave totals (one barrier; the caller
// must not reuse row r before another barrier).
template <int NT>
__device__ __forceinline__ int block_excl_scan(int x, SelShared<NT>& sh, int r, int* total = nullptr) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int wt;
  const int incl = wave_incl_scan(x, &wt);
  if (lane == 63) sh.wsum[r][w] = wt;
  __syncthreads();
  int base = 0, all = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
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
//          keeps the result exact; a tight one keeps the boundary bins small)
// All threads of the workgroup call it with the same k, smin, smax.
template <int NT, int S>
__device__ __forceinline__ uint32_t select_level(const float (&sc)[S], uint32_t valid, uint32_t owned, int pos0, int k,
                                                 const LinBins bin, SelShared<NT>& sh, SelCursor& cur) {
  const int t = threadIdx.x, lane = t & 63;
  const int trash = kSelBins + lane;  // this lane's bin for slots that do not count
  int* hist = sh.hist[cur.hb];
  // 1. histogram of the owned candidates (no branch per slot)
#pragma unroll
  for (int i = 0; i < S; ++i) atomicAdd(&hist[((owned >> i) & 1u) ? bin(sc[i]) : trash], 1);
  __syncthreads();
  // the previous level's histograms and list are read no more: clear them
  // for the levels after this one
  {
    int* old = sh.hist[(cur.hb + 2) % 3];
    int* old2 = sh.hist2[cur.lb ^ 1];
    for (int i = t; i < kSelBins; i += NT) {
      old[i] = 0;
      old2[i] = 0;
    }
    if (t == 0) sh.list_n[cur.lb ^ 1] = 0;
  }
  int b, need, cnt;
  find_bin(hist, k, b, need, cnt);
  uint32_t above = 0u, cell = 0u;  // candidates above the boundary cell, and in it
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const int bi = bin(sc[i]);
    const bool v = (valid >> i) & 1u;
    above |= (v && bi > b) ? (1u << i) : 0u;
    cell |= (v && bi == b) ? (1u << i) : 0u;
  }
  uint32_t kept;
  if (cnt == need) {  // bin b is kept whole (uniform)
    kept = above | cell;
  } else {
    // 2. sub-bins of bin b
    const LinBins sub = bin.sub(b);
    int* h2 = sh.hist2[cur.lb];
#pragma unroll
    for (int i = 0; i < S; ++i) atomicAdd(&h2[(((owned & cell) >> i) & 1u) ? sub(sc[i]) : trash], 1);
    __syncthreads();
    int b2, need2, cnt2;
    find_bin(h2, need, b2, need2, cnt2);
    uint32_t cell2 = 0u;
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const int si = sub(sc[i]);
      const bool c = (cell >> i) & 1u;
      above |= (c && si > b2) ? (1u << i) : 0u;
      cell2 |= (c && si == b2) ? (1u << i) : 0u;
    }
    cell = cell2;
    need = need2;
    if (cnt2 == need2) {  // the sub-bin is kept whole (uniform)
      kept = above | cell;
    } else if (cnt2 <= kSelList) {  // 3. exact ranks inside the cell (uniform)
      uint64_t* list = sh.list[cur.lb];
      const uint32_t mine = cell & owned;
      {
        const int n = __popc(mine);
        int wt;
        const int incl = wave_incl_scan(n, &wt);
        int base = 0;
        if (lane == 63 && wt > 0) base = atomicAdd(&sh.list_n[cur.lb], wt);
        base = __builtin_amdgcn_readlane(base, 63) + incl - n;
#pragma unroll
        for (int i = 0; i < S; ++i)
          if ((mine >> i) & 1u) list[base++] = rank_key(order_key(sc[i]), pos0 + i);
      }
      __syncthreads();
      // the need-th best entry of the list, tau: lane l ranks entries l,
      // l + 64, ... against the whole list (its ranks are 0 .. nl-1, the keys
      // being distinct), and the entry of rank need - 1 is broadcast
      const int nl = sh.list_n[cur.lb];
      uint32_t tau_hi = 0u, tau_lo = 0u;
      for (int e0 = 0; e0 < nl; e0 += 64) {  // uniform
        const int e = e0 + lane;
        const uint64_t me = e < nl ? list[e] : 0ull;
        int rank = 0;
        int f = 0;
        for (; f + 4 <= nl; f += 4) {  // four reads in flight per step
          const uint64_t x0 = list[f], x1 = list[f + 1], x2 = list[f + 2], x3 = list[f + 3];
          rank += (x0 > me ? 1 : 0) + (x1 > me ? 1 : 0) + (x2 > me ? 1 : 0) + (x3 > me ? 1 : 0);
        }
        for (; f < nl; ++f) rank += list[f] > me ? 1 : 0;
        const uint64_t hit = __ballot((e < nl) & (rank == need - 1));
        if (hit) {  // uniform
          const int src = (int)__ffsll((unsigned long long)hit) - 1;
          tau_hi = __builtin_amdgcn_readlane((uint32_t)(me >> 32), src);
          tau_lo = __builtin_amdgcn_readlane((uint32_t)me, src);
        }
      }
      const uint64_t tau = ((uint64_t)tau_hi << 32) | tau_lo;
      // kept: above the cell, and in it the entries ranked at or above tau
      // (exactly `need` of them; a copy held by a non-owner decides the same)
      kept = above;
#pragma unroll
      for (int i = 0; i < S; ++i)
        kept |= (((cell >> i) & 1u) && rank_key(order_key(sc[i]), pos0 + i) >= tau) ? (1u << i) : 0u;
    } else {  // 4. heavy ties: narrow the cell by the key bits (uniform)
      const int w = t >> 6;
      uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
      for (int i = 0; i < S; ++i) {
        const bool in = (cell >> i) & 1u;
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
      for (int i = 0; i < NT / 64; ++i) {
        lo = min(lo, sh.wmn[i]);
        hi = max(hi, sh.wmx[i]);
      }
      int nd = need;
      bool whole = false;
      int* h3 = sh.hist[(cur.hb + 1) % 3];  // the next level's pass-1 histogram: zero now, zero again on exit
      while (!whole && lo != hi) {          // uniform
        const uint32_t range = hi - lo;
        const int rb = 32 - __clz(range);
        const int s8 = rb > 8 ? rb - 8 : 0;  // (range >> s8) < kSelBins
#pragma unroll
        for (int i = 0; i < S; ++i) {
          const uint32_t key = order_key(sc[i]);
          if (((cell & owned) >> i) & 1u && key >= lo && key <= hi) atomicAdd(&h3[(key - lo) >> s8], 1);
        }
        __syncthreads();
        int b3, nd3, cnt3;
        find_bin(h3, nd, b3, nd3, cnt3);
        __syncthreads();  // every wave has read h3
        for (int i = t; i < kSelBins; i += NT) h3[i] = 0;
        __syncthreads();
        const uint32_t nlo = lo + ((uint32_t)b3 << s8);
        hi = (s8 == 0) ? nlo : min(hi, nlo + ((1u << s8) - 1u));
        lo = nlo;
        nd = nd3;
        whole = cnt3 == nd3;
      }
      // above the narrowed range: kept; inside: all (whole) or the nd lowest positions (ties)
      uint32_t tie = 0u;
      kept = above;
#pragma unroll
      for (int i = 0; i < S; ++i) {
        const uint32_t key = order_key(sc[i]);
        const bool in = (cell >> i) & 1u;
        kept |= (in && key > hi) ? (1u << i) : 0u;
        tie |= (in && key >= lo && key <= hi) ? (1u << i) : 0u;
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
  }
  cur.hb = (cur.hb + 1) % 3;
  cur.lb ^= 1;
  return kept;
}

// The same with the bins built here from the score range.
template <int NT, int S>
__device__ __forceinline__ uint32_t select_level(const float (&sc)[S], uint32_t valid, uint32_t owned, int pos0, int k,
                                                 float smin, float smax, SelShared<NT>& sh, SelCursor& cur) {
  return select_level<NT, S>(sc, valid, owned, pos0, k, LinBins(smin, smax), sh, cur);
}

}  // namespace wf
