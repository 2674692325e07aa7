// Fine-grained top-k selection on gfx950.
//
// Per query row at position t: keep the n = min(k, t+1) positions with the largest
// indexer scores among 0..t (DeepSeek-V3.2-Exp paper, section 1 text after Eq. 1
// and section 2.1: S_t = positions of the top-k scores, k = 2048).  Equal scores
// are taken from the lowest position first, so the set is unique; it is written in
// ascending position order and padded with -1.
//
// One 1024-thread block per row, reading four consecutive scores per thread and
// step.  Rows of up to 32768 positions are staged once in LDS (128 KB) and every
// pass reads them there; longer rows (up to 131072) are streamed from global memory
// once per pass.
//   1. min / max of the row (while staging it).
//   2. histogram of 2048 equal-width value bins over [min, max] in LDS.  The bin
//      map is monotone in the score, so every bin above the one holding the n-th
//      largest score (found by a block-wide scan) is selected outright.  Equal-width
//      bins spread real score rows evenly, which keeps LDS atomic collisions rare.
//   3. positions in higher bins are marked in an LDS position bitmap; the members
//      of the threshold bin (typically a few dozen) are ranked exactly by (score
//      descending, position ascending) and the winners marked too.  Bins with more
//      than 256 members (mass ties) fall back to four 8-bit radix rounds over
//      order-preserving keys, which yield the exact threshold key T; positions with
//      key > T are marked selected and those with key == T as ties, of which the
//      lowest positions are taken.
//   4. output: one block scan over the bitmap words' popcounts gives every thread
//      the output slot of its first marked position; marked positions are written
//      in ascending order.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int TK_T = 1024;
constexpr int TK_W = TK_T / 64;
constexpr int NBIN = 2048;
constexpr int CMAX = 256;              // threshold-bin members ranked directly
constexpr int BITMAP_POS = kTopkMaxPositions;  // positions covered by the streaming bitmap

struct TopkShared {
  uint32_t hist[NBIN];
  uint32_t cg[TK_T];
  uint32_t ce[TK_T];
  uint32_t wtot[2][TK_W];
  float fred[2][TK_W];
  uint32_t ckey[CMAX];
  int cpos[CMAX];
  int misc[8];
};

// Run by one whole wave: find the bin holding the need-th largest element of
// hist[0..NB) (1 <= need <= total).  res[0] = bin, res[1] = count in higher bins.
template <int NB>
__device__ __forceinline__ void find_bin_desc(const uint32_t* hist, uint32_t need, int* res) {
  constexpr int PER = NB / 64;
  const int l = lane_id();
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) local += hist[l * PER + i];
  const uint32_t incl = wave_incl_scan(local);
  const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  const uint32_t suf = total - incl + local;  // sum over lanes >= l
  const uint32_t above = suf - local;
  if (above < need && need <= suf) {
    uint32_t acc = above;
    for (int i = PER - 1; i >= 0; --i) {
      const uint32_t c = hist[l * PER + i];
      if (acc + c >= need) {
        res[0] = l * PER + i;
        res[1] = (int)acc;
        break;
      }
      acc += c;
    }
  }
}

// Inclusive block-wide scan of one value per thread; returns the inclusive prefix.
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* wtot) {
  const int l = lane_id(), wv = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (l == 63) wtot[wv] = inc;
  __syncthreads();
  uint32_t base = 0;
#pragma unroll
  for (int i = 0; i < TK_W; ++i)
    if (i < wv) base += wtot[i];
  return base + inc;
}

// Exclusive scan, in place, of a[0..M) and b[0..M) (M <= TK_T); returns totals.
__device__ __forceinline__ uint2 block_scan2(uint32_t* a, uint32_t* b, int M,
                                             uint32_t (*wtot)[TK_W]) {
  const int tid = threadIdx.x, l = lane_id(), wv = tid >> 6;
  const uint32_t va = tid < M ? a[tid] : 0u, vb = tid < M ? b[tid] : 0u;
  const uint32_t ia = wave_incl_scan(va), ib = wave_incl_scan(vb);
  if (l == 63) {
    wtot[0][wv] = ia;
    wtot[1][wv] = ib;
  }
  __syncthreads();
  uint32_t basea = 0, baseb = 0, ta = 0, tb = 0;
#pragma unroll
  for (int i = 0; i < TK_W; ++i) {
    const uint32_t xa = wtot[0][i], xb = wtot[1][i];
    if (i < wv) {
      basea += xa;
      baseb += xb;
    }
    ta += xa;
    tb += xb;
  }
  if (tid < M) {
    a[tid] = basea + ia - va;
    b[tid] = baseb + ib - vb;
  }
  __syncthreads();
  return make_uint2(ta, tb);
}

// Positions are visited in chunks of CH = 4 * 1024 * JV: within a chunk, thread tid
// owns the float4 groups j * 1024 + tid (j < JV), i.e. positions
// c * CH + 4 (j * 1024 + tid) + e, e < 4.  Selected positions are marked in LDS
// bitmaps and the ordered output is produced from the bitmaps, so no pass depends
// on which thread owns a position.
constexpr int kResidentMax = 32768;  // longest row staged in LDS (128 KB)

// One row at position t (0 <= t < CAP): row = its scores, orow = its k outputs.
// sel / tie are LDS bitmaps covering CAP positions.
template <bool RESIDENT, int JV>
__device__ __forceinline__ void topk_row(const float* __restrict__ row, int t, int topk,
                                         int vec_ok, int32_t* __restrict__ orow,
                                         TopkShared& sh, uint32_t* sel, uint32_t* tie) {
  constexpr int CH = 4 * TK_T * JV;
  constexpr int CAP = RESIDENT ? CH : BITMAP_POS;  // positions the bitmaps cover
  constexpr int BM_WORDS = CAP / 32;
  const int tid = threadIdx.x, l = lane_id(), wv = tid >> 6;
  const int L = t + 1;
  const int n = min(topk, L);
  if (n == L) {  // every candidate is selected
    for (int i = tid; i < topk; i += TK_T) orow[i] = i < L ? i : -1;
    return;
  }
  if (tid < 8) sh.misc[tid] = 0;
  const int nchunks = (L + CH - 1) / CH;
  const int words = (L + 31) >> 5;

  // four consecutive scores starting at position s (s % 4 == 0); lanes past the
  // row end read as -inf and are masked by position everywhere
  auto fetch = [&](int s) -> f32x4 {
    f32x4 v;
    if (vec_ok && s + 3 < L) {
      v = *reinterpret_cast<const f32x4*>(row + s);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = s + e < L ? row[s + e] : -INFINITY;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (v[e] != v[e]) ? -INFINITY : v[e];
    return v;
  };

  // ---- 1. (keep the row in registers and) min / max.  A resident row (one chunk)
  //      stays in rv for every later pass: thread tid holds groups j * 1024 + tid.
  f32x4 rv[RESIDENT ? JV : 1];
  float mn = INFINITY, mx = -INFINITY;
  for (int c = 0; c < nchunks; ++c) {
    f32x4 v[JV];
#pragma unroll
    for (int j = 0; j < JV; ++j) {
      const int s = c * CH + 4 * (j * TK_T + tid);
      if (s < L) {
        if (vec_ok && s + 3 < L) {
          v[j] = *reinterpret_cast<const f32x4*>(row + s);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[j][e] = s + e < L ? row[s + e] : -INFINITY;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < JV; ++j) {
      const int s = c * CH + 4 * (j * TK_T + tid);
      if (s < L) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x = v[j][e];
          x = (x != x) ? -INFINITY : x;
          v[j][e] = x;
          if (s + e < L) {
            mn = fminf(mn, x);
            mx = fmaxf(mx, x);
          }
        }
      }
      if (RESIDENT) rv[j] = s < L ? v[j] : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
  }
  mn = wave_min(mn);
  mx = wave_max(mx);
  if (l == 0) {
    sh.fred[0][wv] = mn;
    sh.fred[1][wv] = mx;
  }
  for (int i = tid; i < NBIN; i += TK_T) sh.hist[i] = 0u;
  __syncthreads();
  mn = sh.fred[0][0];
  mx = sh.fred[1][0];
#pragma unroll
  for (int i = 1; i < TK_W; ++i) {
    mn = fminf(mn, sh.fred[0][i]);
    mx = fmaxf(mx, sh.fred[1][i]);
  }
  if (!(mx > mn)) {  // all candidates equal: the n lowest positions
    for (int i = tid; i < topk; i += TK_T) orow[i] = i < n ? i : -1;
    return;
  }

  float inv = (float)NBIN / (mx - mn);
  if (!(inv < INFINITY)) inv = 0.f;
  // bin of v: floor((v - lo) * sc) clamped to [0, NBIN); NaN (from inv = 0) and -inf
  // land in bin 0.  Min / max / convert only, so no compare masks are made.
  auto bin_with = [&](float v, float lo, float sc) -> int {
    return (int)fminf(fmaxf((v - lo) * sc, 0.f), (float)(NBIN - 1));
  };
  // 1 if a < b (ints of either sign whose difference fits), as plain arithmetic
  auto lt1 = [](int a, int b) -> uint32_t { return (uint32_t)(a - b) >> 31; };
  auto bin_of = [&](float v) -> int { return bin_with(v, mn, inv); };
  // visit every float4 group with all lanes (uniform control flow, for shuffles):
  // fn(s, v) with s the group's first position; lanes past the row end see -inf
  auto for_each_group = [&](auto&& fn) {
    if constexpr (RESIDENT) {
      // a fresh (opaque) position base per pass: otherwise the compiler keeps every
      // position and its validity from one pass to the next, past the register file
      int p0 = 4 * tid;
      asm volatile("" : "+v"(p0));
#pragma unroll
      for (int j = 0; j < JV; ++j) fn(p0 + 4 * j * TK_T, rv[j]);
    } else {
      for (int c = 0; c < nchunks; ++c) {
#pragma unroll 2
        for (int j = 0; j < JV; ++j) {
          const int s = c * CH + 4 * (j * TK_T + tid);
          const f32x4 v = s < L ? fetch(s) : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
          fn(s, v);
        }
      }
    }
  };
  // visit every valid position: fn(s, value)
  auto for_each = [&](auto&& fn) {
    for_each_group([&](int s, const f32x4 v) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (s + e < L) fn(s + e, v[e]);
    });
  };

  // ---- 2. equal-width value histogram and the bin of the n-th largest score
  // branch-free: a position past the row end (value -inf, bin 0) adds 0
  for_each_group([&](int s, const f32x4 v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) atomicAdd(&sh.hist[bin_of(v[e])], lt1(s + e, L));
  });
  __syncthreads();
  {
    const int hi = NBIN - 1 - 2 * tid;  // this thread's bins, from the top down
    const uint32_t c1 = sh.hist[hi], c0 = sh.hist[hi - 1];
    const uint32_t incl = block_incl_scan(c0 + c1, sh.wtot[0]);
    const uint32_t excl = incl - c0 - c1;
    if (excl < (uint32_t)n && (uint32_t)n <= incl) {
      const bool upper = excl + c1 >= (uint32_t)n;
      sh.misc[0] = upper ? hi : hi - 1;
      sh.misc[1] = (int)(upper ? excl : excl + c1);
    }
  }
  __syncthreads();
  const int bstar = sh.misc[0];
  const uint32_t above = (uint32_t)sh.misc[1];
  const uint32_t need = (uint32_t)n - above;  // members of bin bstar to take
  const uint32_t cnt_b = sh.hist[bstar];
  const bool fast = cnt_b <= (uint32_t)CMAX;

  uint32_t m_ties = 0u;
  if (fast) {
    // ---- 3a. mark the bins above bstar; collect bstar's members.  The 8 lanes
    //      whose 4-position groups make up one 32-bit bitmap word OR their nibbles
    //      together and one of them stores the word (every word below the row end
    //      is written once, so the bitmap needs no clearing and no atomics).  Bin
    //      members take wave-aggregated slots: one LDS atomic per wave and group.
    const uint64_t lt = lanemask_lt();
    // the same bin scale through an opaque copy: recomputing the bins is cheaper
    // than keeping the histogram pass's 32 bin indices alive in registers
    float inv_m = inv, mn_m = mn;
    asm volatile("" : "+v"(inv_m), "+v"(mn_m));
    for_each_group([&](int s, const f32x4 v) {
      uint32_t m = 0u, mem = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int bn = bin_with(v[e], mn_m, inv_m);
        const uint32_t ok = lt1(s + e, L);
        m |= (lt1(bstar, bn) & ok) << e;                          // bn > bstar
        mem |= ((((uint32_t)(bn ^ bstar)) - 1u) >> 31 & ok) << e;  // bn == bstar
      }
      const uint32_t wd = or8(m << (4 * (l & 7)));
      if ((l & 7) == 0 && s < L) sel[s >> 5] = wd;
      if (__ballot(mem != 0u) != 0ull) {  // wave-uniform; rare
        uint32_t below = 0u, tot = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint64_t bal = __ballot((mem >> e) & 1u);
          below += (uint32_t)__popcll(bal & lt);
          tot += (uint32_t)__popcll(bal);
        }
        int base = 0;
        if (l == 0) base = atomicAdd(&sh.misc[4], (int)tot);
        base = __builtin_amdgcn_readfirstlane(base) + (int)below;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if ((mem >> e) & 1u) {
            sh.ckey[base] = float_key(v[e]);
            sh.cpos[base] = s + e;
            ++base;
          }
      }
    });
    __syncthreads();
    // exact rank of each member by (key desc, position asc); four threads per
    // member, each over a quarter of the others
    for (int c0 = 0; c0 < (int)cnt_b; c0 += TK_T / 4) {
      const int c = c0 + (tid >> 2), part = tid & 3;
      uint32_t rank = 0;
      uint32_t k = 0;
      int p = 0;
      if (c < (int)cnt_b) {
        k = sh.ckey[c];
        p = sh.cpos[c];
        for (int u = part; u < (int)cnt_b; u += 4) {
          const uint32_t ku = sh.ckey[u];
          rank += (ku > k) || (ku == k && sh.cpos[u] < p);
        }
      }
      rank += dpp<kDppXor1>(rank);
      rank += dpp<kDppXor2>(rank);
      if (c < (int)cnt_b && part == 0 && rank < need) atomicOr(&sel[p >> 5], 1u << (p & 31));
    }
  } else {
    // the fallback marks with atomics: clear both bitmaps first (the radix rounds
    // below start with a barrier)
    for (int i = tid; i < words; i += TK_T) {
      sel[i] = 0u;
      tie[i] = 0u;
    }
    // ---- 3b. exact threshold key T inside bin bstar by 8-bit radix rounds, then
    //          mark key > T as selected and key == T as ties
    uint32_t prefix = 0u, pmask = 0u, rem = need, gt = above;
#pragma unroll 1
    for (int shift = 24; shift >= 0; shift -= 8) {
      __syncthreads();
      if (tid < 256) sh.hist[tid] = 0u;
      __syncthreads();
      for_each([&](int, float v) {
        if (bin_of(v) == bstar) {
          const uint32_t k = float_key(v);
          if ((k & pmask) == prefix) atomicAdd(&sh.hist[(k >> shift) & 255u], 1u);
        }
      });
      __syncthreads();
      if (wv == 0) find_bin_desc<256>(sh.hist, rem, sh.misc + 2);
      __syncthreads();
      const uint32_t d = (uint32_t)sh.misc[2], ab = (uint32_t)sh.misc[3];
      prefix |= d << shift;
      pmask |= 255u << shift;
      rem -= ab;
      gt += ab;
    }
    const uint32_t T = prefix;
    m_ties = (uint32_t)n - gt;  // positions with key == T to take, lowest first
    for_each([&](int s, float v) {
      const uint32_t k = float_key(v);
      if (k > T) atomicOr(&sel[s >> 5], 1u << (s & 31));
      else if (k == T) atomicOr(&tie[s >> 5], 1u << (s & 31));
    });
  }
  __syncthreads();

  // ---- 4. ordered output from the bitmaps: thread tid owns words [tid*WPT, +WPT).
  // Output slot of a position = #selected before + min(#ties before, m_ties).
  constexpr int WPT = BM_WORDS > TK_T ? BM_WORDS / TK_T : 1;  // words per thread
  uint32_t sw[WPT], tw[WPT], ns = 0u, nt = 0u;
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int w = tid * WPT + i;
    sw[i] = w < words ? sel[w] : 0u;
    tw[i] = (w < words && !fast) ? tie[w] : 0u;  // no ties on the fast path
    ns += (uint32_t)__popc(sw[i]);
    nt += (uint32_t)__popc(tw[i]);
  }
  sh.cg[tid] = ns;
  sh.ce[tid] = nt;
  __syncthreads();
  block_scan2(sh.cg, sh.ce, TK_T, sh.wtot);
  uint32_t S = sh.cg[tid], E = sh.ce[tid];
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    uint32_t a = sw[i], b = tw[i];
    const int base = (tid * WPT + i) * 32;
    while (a | b) {
      const uint32_t la = a ? (uint32_t)__ffs(a) - 1u : 32u;
      const uint32_t lb = b ? (uint32_t)__ffs(b) - 1u : 32u;
      if (la < lb) {  // next set position is a selected one
        const uint32_t at = S + min(E, m_ties);
        if (at < (uint32_t)n) orow[at] = base + (int)la;
        ++S;
        a &= a - 1u;
      } else {        // next set position is a tie
        if (E < m_ties && S + E < (uint32_t)n) orow[S + E] = base + (int)lb;
        ++E;
        b &= b - 1u;
      }
    }
  }
  for (int i = n + tid; i < topk; i += TK_T) orow[i] = -1;
}

// One 1024-thread block per row, for rows shorter than 4 * 1024 * JV positions
// (RESIDENT) or up to BITMAP_POS (streamed).
template <bool RESIDENT, int JV>
__global__ __launch_bounds__(TK_T) void topk_kernel(const float* __restrict__ scores, int64_t ld,
                                                    const int32_t* __restrict__ row_pos,
                                                    int max_pos, int topk, int vec_ok,
                                                    int32_t* __restrict__ out) {
  constexpr int CAP = RESIDENT ? 4 * TK_T * JV : BITMAP_POS;
  __shared__ TopkShared sh;
  __shared__ uint32_t sel[CAP / 32];   // positions selected outright
  __shared__ uint32_t tie[CAP / 32];   // fallback: positions whose key equals T
  const int r = blockIdx.x;
  const int t = row_pos[r];
  int32_t* orow = out + (size_t)r * topk;
  if (t < 0 || t > max_pos || (int64_t)t >= ld || t >= CAP) {
    for (int i = threadIdx.x; i < topk; i += TK_T) orow[i] = -1;
    return;
  }
  topk_row<RESIDENT, JV>(scores + (size_t)r * ld, t, topk, vec_ok, orow, sh, sel, tie);
}

// Rows of any length up to BITMAP_POS, chosen per row: a row of at most
// kResidentMax positions is held in registers, a longer one is streamed.  Used when
// the host bound on the positions is above kResidentMax, since a looser bound (a
// chunk of a long prefill, say) says nothing about each row's own length.
__global__ __launch_bounds__(TK_T) void topk_kernel_any(const float* __restrict__ scores,
                                                        int64_t ld,
                                                        const int32_t* __restrict__ row_pos,
                                                        int max_pos, int topk, int vec_ok,
                                                        int32_t* __restrict__ out) {
  __shared__ TopkShared sh;
  __shared__ uint32_t sel[BITMAP_POS / 32];
  __shared__ uint32_t tie[BITMAP_POS / 32];
  const int r = blockIdx.x;
  const int t = row_pos[r];
  int32_t* orow = out + (size_t)r * topk;
  if (t < 0 || t > max_pos || (int64_t)t >= ld || t >= BITMAP_POS) {
    for (int i = threadIdx.x; i < topk; i += TK_T) orow[i] = -1;
    return;
  }
  const float* row = scores + (size_t)r * ld;
  if (t < kResidentMax)  // block-uniform
    topk_row<true, kResidentMax / (4 * TK_T)>(row, t, topk, vec_ok, orow, sh, sel, tie);
  else
    topk_row<false, 4>(row, t, topk, vec_ok, orow, sh, sel, tie);
}

}  // namespace

hipError_t launch_topk(const dsa_rows& rows, int topk, const float* scores, int64_t ld,
                       int32_t* indices, hipStream_t stream) {
  const int R = rows.num_rows;
  const int L = rows.max_pos + 1;
  const int vec_ok = (ld % 4 == 0) && (reinterpret_cast<uintptr_t>(scores) % 16 == 0);
  if (L <= 4 * TK_T * 2) {
    hipLaunchKernelGGL((topk_kernel<true, 2>), dim3(R), dim3(TK_T), 0, stream, scores, ld,
                       rows.row_pos, rows.max_pos, topk, vec_ok, indices);
  } else if (L <= kResidentMax) {
    hipLaunchKernelGGL((topk_kernel<true, 8>), dim3(R), dim3(TK_T), 0, stream, scores, ld,
                       rows.row_pos, rows.max_pos, topk, vec_ok, indices);
  } else if (L <= BITMAP_POS) {
    hipLaunchKernelGGL(topk_kernel_any, dim3(R), dim3(TK_T), 0, stream, scores, ld, rows.row_pos,
                       rows.max_pos, topk, vec_ok, indices);
  } else {
    return hipErrorInvalidValue;  // rows longer than the bitmap capacity
  }
  return hipGetLastError();
}

}  // namespace dsa
