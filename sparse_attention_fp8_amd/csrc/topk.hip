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
// sel / tie are LDS bitmaps covering CAP positions.  A streamed row whose score
// extremes are known (have_mm: lo / hi over its non-NaN scores) skips the min / max
// pass.  Any lo < hi gives the same selection (the bins only need to be the same in
// every pass: a score below lo, or a NaN read as -inf, lands in bin 0); lo >= hi
// (all scores equal, or none known) takes the pass, which reads NaN as -inf.
template <bool RESIDENT, int JV>
__device__ __forceinline__ void topk_row(const float* __restrict__ row, int t, int topk,
                                         int vec_ok, int32_t* __restrict__ orow,
                                         TopkShared& sh, uint32_t* sel, uint32_t* tie,
                                         bool have_mm = false, float mm_lo = 0.f,
                                         float mm_hi = 0.f) {
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
  const bool pass1 = RESIDENT || !have_mm || !(mm_hi > mm_lo);  // block-uniform
  for (int c = 0; pass1 && c < nchunks; ++c) {
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
  if (pass1) {
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (l == 0) {
      sh.fred[0][wv] = mn;
      sh.fred[1][wv] = mx;
    }
  }
  for (int i = tid; i < NBIN; i += TK_T) sh.hist[i] = 0u;
  __syncthreads();
  if (pass1) {
    mn = sh.fred[0][0];
    mx = sh.fred[1][0];
#pragma unroll
    for (int i = 1; i < TK_W; ++i) {
      mn = fminf(mn, sh.fred[0][i]);
      mx = fmaxf(mx, sh.fred[1][i]);
    }
  } else {
    mn = mm_lo;
    mx = mm_hi;
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

// float of an order-preserving key (inverse of float_key; +0.0 for either zero)
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Rows of any length up to BITMAP_POS, chosen per row: a row of at most
// kResidentMax positions is held in registers, a longer one is streamed.  Used when
// the host bound on the positions is above kResidentMax, since a looser bound (a
// chunk of a long prefill, say) says nothing about each row's own length.
// rowmm (optional): the score extremes of every row, two words per row as the
// tiled indexer leaves them (2 r: max key, 2 r + 1: ~min key, over the non-NaN
// scores); a streamed row uses them instead of its min / max pass, and every row's
// block sets its two words back to zero for the next indexer launch.
__global__ __launch_bounds__(TK_T) void topk_kernel_any(const float* __restrict__ scores,
                                                        int64_t ld,
                                                        const int32_t* __restrict__ row_pos,
                                                        int max_pos, int topk, int vec_ok,
                                                        int32_t* __restrict__ out,
                                                        uint32_t* __restrict__ rowmm) {
  __shared__ TopkShared sh;
  __shared__ uint32_t sel[BITMAP_POS / 32];
  __shared__ uint32_t tie[BITMAP_POS / 32];
  __shared__ uint32_t mmw[2];
  const int r = blockIdx.x;
  if (rowmm != nullptr) {  // block-uniform
    if (threadIdx.x == 0) {
      mmw[0] = rowmm[2 * r];
      mmw[1] = rowmm[2 * r + 1];
      rowmm[2 * r] = 0u;
      rowmm[2 * r + 1] = 0u;
    }
    __syncthreads();
  }
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
    topk_row<false, 4>(row, t, topk, vec_ok, orow, sh, sel, tie, rowmm != nullptr,
                       key_float(~mmw[1]), key_float(mmw[0]));
}

// ---------------------------------------------------------------------------
// Few rows (decode): many blocks per row, one kernel.  Block (r, p) owns positions
// [4096 p, 4096 p + 4096) of row r.
//   1. Every block of the row derives the same lower bound tau of the threshold
//      key from a fixed sample of the row (64 runs of 64 scores, evenly spaced): the
//      sample's k'-th largest key, k' chosen so that about 1.5 n scores of the row
//      lie above it, rounded down to a multiple of 2^8.  Rows of at most 8192
//      positions use tau = 0: every position is a candidate.
//   2. The block writes its positions whose key is >= tau, in position order, to
//      its slot of the workspace (key and position), with device-scope stores, and
//      their count.  Then it counts itself done (an atomic per row; no block waits
//      for another).
//   3. The last block of the row to finish selects exactly among the candidates,
//      which are in position order: three radix levels (key bits 31..20, 19..8,
//      7..0) find the threshold key; candidates above it are taken, and of those
//      equal to it the first in position order.  If fewer than n positions reached
//      tau (the sample misled), the same selection runs over the whole row.
// The per-row counts must be zero when the kernel starts (topk_mb_zero_kernel).
// ---------------------------------------------------------------------------
constexpr int MB_CHUNK = 4 * TK_T;   // positions per block
constexpr int MB_NBIN = 4096;        // radix bins per level (12 bits)
constexpr int MB_SAMPLE = 4 * TK_T;  // sample size: 64 runs of 64 scores
constexpr int MB_ALL = 8192;         // rows up to this long take every position
constexpr int MB_CAP = 8192 + CMAX;  // candidates held in LDS, plus CMAX for a bin's members

struct MbShared {
  uint32_t hist[MB_NBIN];
  uint32_t ckey[MB_CAP];
  int cpos[MB_CAP];
  uint32_t pref[kTopkMaxPositions / MB_CHUNK + 1];
  uint32_t wtot[2][TK_W];
  int misc[8];
};

// Whole block: the bin of hist[0..NB) holding the need-th largest element
// (1 <= need <= total), counting from the top.  res[0] = bin, res[1] = count in
// the bins above it.  The caller synchronises before reading res.
template <int NB>
__device__ __forceinline__ void find_desc_block(const uint32_t* hist, uint32_t need,
                                                uint32_t* wtot, int* res) {
  constexpr int PER = NB >= TK_T ? NB / TK_T : 1;
  const int tid = threadIdx.x;
  uint32_t c[PER];
  uint32_t local = 0u;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = tid * PER + j;  // i-th bin from the top
    c[j] = i < NB ? hist[NB - 1 - i] : 0u;
    local += c[j];
  }
  const uint32_t incl = block_incl_scan(local, wtot);
  const uint32_t excl = incl - local;
  if (excl < need && need <= incl) {
    uint32_t acc = excl;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (acc + c[j] >= need) {
        res[0] = NB - 1 - (tid * PER + j);
        res[1] = (int)acc;
        break;
      }
      acc += c[j];
    }
  }
}

// four scores from position s (s % 4 == 0); past the row end and NaN read as -inf
__device__ __forceinline__ f32x4 fetch4(const float* __restrict__ row, int s, int L, int vec_ok) {
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
}

__device__ __forceinline__ void store_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_agent(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent2(uint2* p, uint32_t key, uint32_t pos) {
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p),
                     ((unsigned long long)pos << 32) | key, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint2 load_agent2(const uint2* p) {
  const unsigned long long x = __hip_atomic_load(
      reinterpret_cast<unsigned long long*>(const_cast<uint2*>(p)), __ATOMIC_RELAXED,
      __HIP_MEMORY_SCOPE_AGENT);
  return make_uint2((uint32_t)x, (uint32_t)(x >> 32));
}

__global__ __launch_bounds__(256) void topk_mb_zero_kernel(uint32_t* __restrict__ counts, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) counts[i] = 0u;
}

// Block-wide min and max of one key per thread.
__device__ __forceinline__ uint2 block_minmax(uint32_t lo, uint32_t hi, MbShared& sh) {
  lo = wave_reduce_bits(lo, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
  hi = wave_reduce_bits(hi, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
  const int wv = threadIdx.x >> 6;
  __syncthreads();
  if (lane_id() == 0) {
    sh.wtot[0][wv] = lo;
    sh.wtot[1][wv] = hi;
  }
  __syncthreads();
  uint32_t rlo = sh.wtot[0][0], rhi = sh.wtot[1][0];
#pragma unroll
  for (int w = 1; w < TK_W; ++w) {
    rlo = min(rlo, sh.wtot[0][w]);
    rhi = max(rhi, sh.wtot[1][w]);
  }
  __syncthreads();
  return make_uint2(rlo, rhi);
}

// shift that maps key - lo for keys in [lo, hi] onto at most 4096 bins
__device__ __forceinline__ int span_shift(uint32_t lo, uint32_t hi) {
  const uint32_t span = hi - lo;
  const int bits = span == 0u ? 0 : 32 - __clz(span);
  return bits > 12 ? bits - 12 : 0;
}

// Exact selection of the n largest keys (ties to the lower position) among C
// candidates given in position order by get(i) -> (key, pos), written ascending to
// orow.  Whole block.  The keys are binned over their own range [lo, hi] (4096
// bins), which finds the bin of the n-th largest; its members, typically a handful,
// are ranked directly by (key desc, position asc).  A bin with more than CMAX
// members (keys packed into a narrow range) is binned again over its own range, down
// to a single key, whose members are ties taken in position order.
template <typename Get>
__device__ __forceinline__ void select_ordered(MbShared& sh, Get&& get, int C, int n,
                                               int32_t* __restrict__ orow) {
  const int tid = threadIdx.x;
  uint32_t klo = 0xFFFFFFFFu, khi = 0u;
  for (int i = tid; i < C; i += TK_T) {
    const uint32_t k = get(i).x;
    klo = min(klo, k);
    khi = max(khi, k);
  }
  const uint2 mm = block_minmax(klo, khi, sh);
  uint32_t lo = mm.x, hi = mm.y, need = (uint32_t)n;
  uint32_t kstar = 0u, m_ties = 0u;
  uint32_t* mk = sh.ckey + (MB_CAP - CMAX);  // the members of a bin
  int* mp = sh.cpos + (MB_CAP - CMAX);
#pragma unroll 1
  for (;;) {
    // the keys in [lo, hi] hold the remaining `need` winners; bin them
    const int shift = span_shift(lo, hi);
    for (int i = tid; i < MB_NBIN; i += TK_T) sh.hist[i] = 0u;
    if (tid == 0) {
      sh.misc[4] = 0;
      sh.misc[6] = 0;
    }
    __syncthreads();
    for (int i = tid; i < C; i += TK_T) {
      const uint32_t k = get(i).x;
      if (k >= lo && k <= hi) atomicAdd(&sh.hist[(k - lo) >> shift], 1u);
    }
    __syncthreads();
    find_desc_block<MB_NBIN>(sh.hist, need, sh.wtot[0], sh.misc + 2);
    __syncthreads();
    const uint32_t tb = (uint32_t)sh.misc[2];
    need -= (uint32_t)sh.misc[3];
    const uint32_t m = sh.hist[tb];
    const uint32_t blo = lo + (tb << shift);
    const uint32_t bhi = shift == 0 ? blo : min(hi, blo + ((1u << shift) - 1u));
    if (blo == bhi) {  // a single key: ties, taken in position order
      kstar = blo;
      m_ties = need;
      break;
    }
    if (m > (uint32_t)CMAX) {  // refine over the bin's own range
      lo = blo;
      hi = bhi;
      __syncthreads();
      continue;
    }
    // collect the bin's members and rank them directly
    for (int i = tid; i < C; i += TK_T) {
      const uint2 kp = get(i);
      if (kp.x >= blo && kp.x <= bhi) {
        const int at = atomicAdd(&sh.misc[4], 1);
        mk[at] = kp.x;
        mp[at] = (int)kp.y;
      }
    }
    __syncthreads();
    // four threads per member, each over a quarter of the others: the member of
    // rank need - 1 is the last winner; its key is kstar
    for (int c0 = 0; c0 < (int)m; c0 += TK_T / 4) {
      const int c = c0 + (tid >> 2), part = tid & 3;
      uint32_t rank = 0u, k = 0u;
      int pp = 0;
      if (c < (int)m) {
        k = mk[c];
        pp = mp[c];
        for (int u = part; u < (int)m; u += 4) {
          const uint32_t ku = mk[u];
          rank += (ku > k) || (ku == k && mp[u] < pp);
        }
      }
      rank += dpp<kDppXor1>(rank);
      rank += dpp<kDppXor2>(rank);
      if (c < (int)m && part == 0 && rank == need - 1u) sh.misc[5] = (int)k;
    }
    __syncthreads();
    kstar = (uint32_t)sh.misc[5];
    // the winners equal to kstar (the first of them in position order)
    for (int c = tid; c < (int)m; c += TK_T) {
      if (mk[c] != kstar) continue;
      uint32_t rank = 0u;
      for (int u = 0; u < (int)m; ++u) rank += (mk[u] > kstar) || (mk[u] == kstar && mp[u] < mp[c]);
      if (rank < need) atomicAdd(&sh.misc[6], 1);
    }
    __syncthreads();
    m_ties = (uint32_t)sh.misc[6];
    break;
  }
  __syncthreads();
  // ordered output: the keys above kstar, and the first m_ties equal to it in
  // position order; tiles of 4 candidates per thread
  uint32_t sel_base = 0u, tie_base = 0u;
  for (int c0 = 0; c0 < C; c0 += 4 * TK_T) {
    uint32_t ksel = 0u, ktie = 0u;
    int pos[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = c0 + 4 * tid + e;
      uint2 kp = make_uint2(0u, 0u);
      if (i < C) kp = get(i);
      pos[e] = (int)kp.y;
      ksel |= (i < C && kp.x > kstar ? 1u : 0u) << e;
      ktie |= (i < C && kp.x == kstar ? 1u : 0u) << e;
    }
    __syncthreads();
    const uint32_t ns = (uint32_t)__popc(ksel), nt = (uint32_t)__popc(ktie);
    const uint32_t is = block_incl_scan(ns, sh.wtot[0]);
    __syncthreads();
    const uint32_t it = block_incl_scan(nt, sh.wtot[1]);
    uint32_t S = sel_base + is - ns, E = tie_base + it - nt;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if ((ksel >> e) & 1u) {
        const uint32_t at = S + min(E, m_ties);
        if (at < (uint32_t)n) orow[at] = pos[e];
        ++S;
      } else if ((ktie >> e) & 1u) {
        if (E < m_ties && S + E < (uint32_t)n) orow[S + E] = pos[e];
        ++E;
      }
    }
    uint32_t tot_s = 0u, tot_t = 0u;
#pragma unroll
    for (int w = 0; w < TK_W; ++w) {
      tot_s += sh.wtot[0][w];
      tot_t += sh.wtot[1][w];
    }
    sel_base += tot_s;
    tie_base += tot_t;
  }
}

__global__ __launch_bounds__(TK_T) void topk_mb_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ row_pos,
    int max_pos, int topk, int vec_ok, int32_t* __restrict__ out, uint2* __restrict__ cand,
    uint32_t* __restrict__ ccount, uint32_t* __restrict__ done, int nchunk) {
  __shared__ MbShared sh;
  const int r = blockIdx.x / nchunk, p = blockIdx.x - r * nchunk;
  const int tid = threadIdx.x;
  const int t = row_pos[r];
  int32_t* orow = out + (size_t)r * topk;
  if (t < 0 || t > max_pos || (int64_t)t >= ld || t >= kTopkMaxPositions) {
    if (p == 0)
      for (int i = tid; i < topk; i += TK_T) orow[i] = -1;
    return;
  }
  const int L = t + 1;
  const int n = min(topk, L);
  if (n == L) {  // every candidate is selected
    if (p == 0)
      for (int i = tid; i < topk; i += TK_T) orow[i] = i < L ? i : -1;
    return;
  }
  const int P = (L + MB_CHUNK - 1) / MB_CHUNK;  // blocks of this row
  if (p >= P) return;
  const float* row = scores + (size_t)r * ld;
  uint2* crow = cand + (size_t)r * nchunk * MB_CHUNK;
  uint32_t* cnt = ccount + (size_t)r * nchunk;

  // this block's scores, requested first
  const int s0 = p * MB_CHUNK + 4 * tid;
  const f32x4 v = fetch4(row, s0, L, vec_ok);

  // ---- 1. tau from the sample
  uint32_t tau = 0u;
  if (L > MB_ALL) {
    const int seg = (L / 64) & ~3;  // >= 128
    const f32x4 sv = fetch4(row, (tid >> 4) * seg + 4 * (tid & 15), L, vec_ok);
    // about 1.5 n of the row above the k'-th largest sample
    const int ks = (int)(((int64_t)n * MB_SAMPLE + L - 1) / L);
    const int kp = min(MB_SAMPLE, ks + ks / 4 + 4 * (int)ceilf(sqrtf((float)ks)) + 8);
    uint32_t sk[4], slo = 0xFFFFFFFFu, shi = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sk[e] = float_key(sv[e]);
      slo = min(slo, sk[e]);
      shi = max(shi, sk[e]);
    }
    const uint2 mm = block_minmax(slo, shi, sh);
    const int shift = span_shift(mm.x, mm.y);
    for (int i = tid; i < MB_NBIN; i += TK_T) sh.hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 4; ++e) atomicAdd(&sh.hist[(sk[e] - mm.x) >> shift], 1u);
    __syncthreads();
    find_desc_block<MB_NBIN>(sh.hist, (uint32_t)kp, sh.wtot[0], sh.misc + 2);
    __syncthreads();
    // the lower edge of the bin holding the k'-th largest sample key
    tau = mm.x + ((uint32_t)sh.misc[2] << shift);
    __syncthreads();
  }

  // ---- 2. this block's candidates, in position order
  uint32_t key[4], flag = 0u;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    key[e] = float_key(v[e]);
    flag |= (s0 + e < L && key[e] >= tau ? 1u : 0u) << e;
  }
  const uint32_t nc = (uint32_t)__popc(flag);
  const uint32_t incl = block_incl_scan(nc, sh.wtot[0]);
  uint32_t at = incl - nc;
  uint2* cblk = crow + (size_t)p * MB_CHUNK;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if ((flag >> e) & 1u) store_agent2(cblk + at++, key[e], (uint32_t)(s0 + e));
  if (tid == TK_T - 1) store_agent(cnt + p, incl);
  // every store of this block has been performed before it counts itself done
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0)
    sh.misc[0] = __hip_atomic_fetch_add(&done[r], 1u, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(P - 1) ? 1 : 0;
  __syncthreads();
  if (sh.misc[0] == 0) return;

  // ---- 3. the last block: exact selection among the row's candidates
  if (tid <= P) sh.pref[tid] = tid < P ? load_agent(cnt + tid) : 0u;
  __syncthreads();
  if (tid == 0) {
    uint32_t acc = 0u;
    for (int i = 0; i <= P; ++i) {
      const uint32_t c = sh.pref[i];
      sh.pref[i] = acc;
      acc += c;
    }
  }
  __syncthreads();
  const int C = (int)sh.pref[P];
  // position-ordered candidate i: chunk q with pref[q] <= i < pref[q + 1]
  auto cand_at = [&](int i) -> uint2 {
    int q = 0;
    while (q + 1 < P && sh.pref[q + 1] <= (uint32_t)i) ++q;
    return load_agent2(crow + (size_t)q * MB_CHUNK + (i - (int)sh.pref[q]));
  };
  if (C < n) {
    // the sample put tau too high: select over the whole row
    select_ordered(sh, [&](int i) -> uint2 {
      return make_uint2(float_key(fetch4(row, i & ~3, L, vec_ok)[i & 3]), (uint32_t)i);
    }, L, n, orow);
  } else if (C <= MB_CAP - CMAX) {
    // gather chunk by chunk: each wave takes chunks in turn, every lane four
    // candidates at a time with their loads in flight together
    const int wv = tid >> 6, ln = lane_id();
    for (int q = wv; q < P; q += TK_W) {
      const int cq = (int)(sh.pref[q + 1] - sh.pref[q]);
      const uint2* src = crow + (size_t)q * MB_CHUNK;
      const int dst = (int)sh.pref[q];
      for (int j0 = 0; j0 < cq; j0 += 256) {
        uint2 kp[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = j0 + 64 * e + ln;
          kp[e] = j < cq ? load_agent2(src + j) : make_uint2(0u, 0u);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = j0 + 64 * e + ln;
          if (j < cq) {
            sh.ckey[dst + j] = kp[e].x;
            sh.cpos[dst + j] = (int)kp[e].y;
          }
        }
      }
    }
    __syncthreads();
    select_ordered(sh, [&](int i) -> uint2 {
      return make_uint2(sh.ckey[i], (uint32_t)sh.cpos[i]);
    }, C, n, orow);
  } else {
    select_ordered(sh, cand_at, C, n, orow);
  }
  for (int i = n + tid; i < topk; i += TK_T) orow[i] = -1;
}

}  // namespace

// The many-blocks-per-row path serves calls with too few rows to fill the GPU
// with one block per row, when the rows are longer than a block holds in its
// registers: a row of up to kResidentMax positions is faster on one block (decode
// at 32K: 15 us, against 17-20 us split over 8 blocks plus their hand-off).
static bool topk_use_multi(const dsa_rows& rows) {
  return rows.num_rows < 128 && rows.max_pos + 1 > kResidentMax;
}

static int topk_chunks(const dsa_rows& rows) { return (rows.max_pos + MB_CHUNK) / MB_CHUNK; }

ClearWords topk_counts(const dsa_rows& rows, void* workspace) {
  ClearWords c;
  if (!topk_use_multi(rows) || workspace == nullptr) return c;
  const size_t R = (size_t)rows.num_rows, P = (size_t)topk_chunks(rows);
  c.ptr = reinterpret_cast<uint32_t*>(static_cast<uint2*>(workspace) + R * P * MB_CHUNK) + R * P;
  c.n = (int)R;
  return c;
}

size_t topk_workspace_bytes(const dsa_rows& rows) {
  if (!topk_use_multi(rows)) return 0;
  const size_t R = (size_t)rows.num_rows, P = (size_t)topk_chunks(rows);
  // candidates [R, P, 4096] (key, position), their counts [R, P], done counts [R]
  return R * P * MB_CHUNK * sizeof(uint2) + ((R * P + R) * sizeof(uint32_t) + 15) / 16 * 16;
}

hipError_t launch_zero_words(uint32_t* p, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_mb_zero_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

bool topk_streams_rows(const dsa_rows& rows) {
  return !topk_use_multi(rows) && rows.max_pos + 1 > kResidentMax;
}

hipError_t launch_topk(const dsa_rows& rows, int topk, const float* scores, int64_t ld,
                       int32_t* indices, void* workspace, hipStream_t stream,
                       bool counts_cleared, uint32_t* rowmm) {
  const int R = rows.num_rows;
  const int L = rows.max_pos + 1;
  const int vec_ok = (ld % 4 == 0) && (reinterpret_cast<uintptr_t>(scores) % 16 == 0);
  if (L > BITMAP_POS) return hipErrorInvalidValue;  // refused on the host before this
  if (rowmm != nullptr && !topk_streams_rows(rows)) return hipErrorInvalidValue;
  if (topk_use_multi(rows)) {
    const int nchunk = topk_chunks(rows);
    uint2* cand = static_cast<uint2*>(workspace);
    uint32_t* ccount = reinterpret_cast<uint32_t*>(cand + (size_t)R * nchunk * MB_CHUNK);
    uint32_t* done = ccount + (size_t)R * nchunk;
    if (!counts_cleared) {
      hipLaunchKernelGGL(topk_mb_zero_kernel, dim3((R + 255) / 256), dim3(256), 0, stream, done, R);
      const hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(topk_mb_kernel, dim3(R * nchunk), dim3(TK_T), 0, stream, scores, ld,
                       rows.row_pos, rows.max_pos, topk, vec_ok, indices, cand, ccount, done,
                       nchunk);
  } else if (L <= 4 * TK_T * 2) {
    hipLaunchKernelGGL((topk_kernel<true, 2>), dim3(R), dim3(TK_T), 0, stream, scores, ld,
                       rows.row_pos, rows.max_pos, topk, vec_ok, indices);
  } else if (L <= kResidentMax) {
    hipLaunchKernelGGL((topk_kernel<true, 8>), dim3(R), dim3(TK_T), 0, stream, scores, ld,
                       rows.row_pos, rows.max_pos, topk, vec_ok, indices);
  } else {
    hipLaunchKernelGGL(topk_kernel_any, dim3(R), dim3(TK_T), 0, stream, scores, ld, rows.row_pos,
                       rows.max_pos, topk, vec_ok, indices, rowmm);
  }
  return hipGetLastError();
}

}  // namespace dsa
