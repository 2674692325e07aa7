// Fine-grained top-k selection on gfx950.
//
// Per query row at position t: keep the n = min(k, t+1) positions with the largest
// indexer scores among 0..t (DeepSeek-V3.2-Exp paper, section 1 text after Eq. 1
// and section 2.1: S_t = positions of the top-k scores, k = 2048).  Equal scores
// are taken from the lowest position first, so the set is unique; it is written in
// ascending position order and padded with -1.
//
// One 1024-thread block per row.  The row is held in registers when it fits
// (L <= 1024 * JC) and streamed from global memory once per pass otherwise.
//   pass 0  min / max of the row
//   pass 1  histogram of 2048 equal-width value bins over [min, max] in LDS.  The
//           bin map is monotone in the score, so every bin above the one holding the
//           n-th largest score is selected outright.  Equal-width bins spread real
//           score rows evenly, which keeps LDS atomic collisions rare.
//   pass 2  exact 32-bit threshold T inside that bin: four 8-bit radix rounds over
//           the order-preserving keys of its members.
//   pass 3  ordered compaction: ballots and a block scan give every selected
//           position its rank; positions with key > T are taken, and of those with
//           key == T the lowest (n - #{key > T}) positions.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int TK_T = 1024;
constexpr int TK_W = TK_T / 64;
constexpr int NBIN = 2048;
constexpr int JC_MAX = 32;

struct TopkShared {
  uint32_t hist[NBIN];
  uint32_t cg[JC_MAX * TK_W];
  uint32_t ce[JC_MAX * TK_W];
  uint32_t wtot[2][TK_W];
  float fred[2][TK_W];
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
  uint32_t suf = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t v = __shfl_down(suf, o);
    if (l + o < 64) suf += v;
  }
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

// Exclusive scan, in place, of a[0..M) and b[0..M) (M <= TK_T); returns totals.
__device__ __forceinline__ uint2 block_scan2(uint32_t* a, uint32_t* b, int M,
                                             uint32_t (*wtot)[TK_W]) {
  const int tid = threadIdx.x, l = lane_id(), wv = tid >> 6;
  const uint32_t va = tid < M ? a[tid] : 0u, vb = tid < M ? b[tid] : 0u;
  uint32_t ia = va, ib = vb;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t ua = __shfl_up(ia, o), ub = __shfl_up(ib, o);
    if (l >= o) {
      ia += ua;
      ib += ub;
    }
  }
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

template <int JC, bool CACHED>
__global__ __launch_bounds__(TK_T) void topk_kernel(const float* __restrict__ scores, int64_t ld,
                                                    const int32_t* __restrict__ row_pos,
                                                    int max_pos, int topk,
                                                    int32_t* __restrict__ out) {
  __shared__ TopkShared sh;
  const int r = blockIdx.x, tid = threadIdx.x, l = lane_id(), wv = tid >> 6;
  const int t = row_pos[r];
  int32_t* orow = out + (size_t)r * topk;
  if (t < 0 || t > max_pos || (int64_t)t >= ld) {
    for (int i = tid; i < topk; i += TK_T) orow[i] = -1;
    return;
  }
  const int L = t + 1;
  const int n = min(topk, L);
  if (n == L) {  // every candidate is selected
    for (int i = tid; i < topk; i += TK_T) orow[i] = i < L ? i : -1;
    return;
  }
  const float* row = scores + (size_t)r * ld;
  if (tid < 8) sh.misc[tid] = 0;
  constexpr int CH = JC * TK_T;
  const int nchunks = CACHED ? 1 : (L + CH - 1) / CH;

  float x[JC];
  auto load = [&](int c0) {
#pragma unroll
    for (int j = 0; j < JC; ++j) {
      const int s = c0 + j * TK_T + tid;
      const float v = s < L ? row[s] : 0.f;
      x[j] = (v != v) ? -INFINITY : v;
    }
  };
  if (CACHED) load(0);

  // ---- pass 0: min / max
  float mn = INFINITY, mx = -INFINITY;
  for (int c = 0; c < nchunks; ++c) {
    if (!CACHED) load(c * CH);
#pragma unroll
    for (int j = 0; j < JC; ++j)
      if (c * CH + j * TK_T + tid < L) {
        mn = fminf(mn, x[j]);
        mx = fmaxf(mx, x[j]);
      }
  }
  mn = wave_min(mn);
  mx = wave_max(mx);
  if (l == 0) {
    sh.fred[0][wv] = mn;
    sh.fred[1][wv] = mx;
  }
  __syncthreads();
  mn = sh.fred[0][0];
  mx = sh.fred[1][0];
#pragma unroll
  for (int i = 1; i < TK_W; ++i) {
    mn = fminf(mn, sh.fred[0][i]);
    mx = fmaxf(mx, sh.fred[1][i]);
  }

  uint32_t T, cnt_gt;
  if (!(mx > mn)) {  // all candidates equal: the n lowest positions
    T = float_key(mx);
    cnt_gt = 0;
  } else {
    float inv = (float)NBIN / (mx - mn);
    if (!(inv < INFINITY)) inv = 0.f;
    auto bin_of = [&](float v) -> int {
      const float f = (v - mn) * inv;
      if (f < (float)(NBIN - 1)) return (int)f;
      return (f != f) ? 0 : NBIN - 1;
    };
    // ---- pass 1: equal-width value histogram
    for (int i = tid; i < NBIN; i += TK_T) sh.hist[i] = 0u;
    __syncthreads();
    for (int c = 0; c < nchunks; ++c) {
      if (!CACHED) load(c * CH);
#pragma unroll
      for (int j = 0; j < JC; ++j)
        if (c * CH + j * TK_T + tid < L) atomicAdd(&sh.hist[bin_of(x[j])], 1u);
    }
    __syncthreads();
    if (wv == 0) find_bin_desc<NBIN>(sh.hist, (uint32_t)n, sh.misc);
    __syncthreads();
    const int bstar = sh.misc[0];
    cnt_gt = (uint32_t)sh.misc[1];
    uint32_t need = (uint32_t)n - cnt_gt;

    uint32_t cand = 0u;  // bit j: element j of the cached row lies in bin bstar
    if (CACHED) {
#pragma unroll
      for (int j = 0; j < JC; ++j)
        if (j * TK_T + tid < L && bin_of(x[j]) == bstar) cand |= 1u << j;
    }
    // ---- pass 2: exact threshold key inside bin bstar
    uint32_t prefix = 0u, pmask = 0u;
#pragma unroll 1
    for (int shift = 24; shift >= 0; shift -= 8) {
      __syncthreads();
      if (tid < 256) sh.hist[tid] = 0u;
      __syncthreads();
      for (int c = 0; c < nchunks; ++c) {
        if (!CACHED) load(c * CH);
#pragma unroll
        for (int j = 0; j < JC; ++j) {
          const bool in = CACHED ? ((cand >> j) & 1u)
                                 : (c * CH + j * TK_T + tid < L && bin_of(x[j]) == bstar);
          if (in) {
            const uint32_t k = float_key(x[j]);
            if ((k & pmask) == prefix) atomicAdd(&sh.hist[(k >> shift) & 255u], 1u);
          }
        }
      }
      __syncthreads();
      if (wv == 0) find_bin_desc<256>(sh.hist, need, sh.misc + 2);
      __syncthreads();
      const uint32_t d = (uint32_t)sh.misc[2], ab = (uint32_t)sh.misc[3];
      prefix |= d << shift;
      pmask |= 255u << shift;
      need -= ab;
      cnt_gt += ab;
    }
    T = prefix;
  }
  const uint32_t m = (uint32_t)n - cnt_gt;  // positions with key == T to take

  // ---- pass 3: ordered compaction (position order = chunk, slot j, wave, lane)
  const uint64_t lt = lanemask_lt();
  uint32_t carry_g = 0u, carry_e = 0u;
  for (int c = 0; c < nchunks; ++c) {
    if (!CACHED) load(c * CH);
#pragma unroll
    for (int j = 0; j < JC; ++j) {
      const bool valid = c * CH + j * TK_T + tid < L;
      const uint32_t k = float_key(x[j]);
      const uint64_t bg = __ballot(valid && k > T);
      const uint64_t be = __ballot(valid && k == T);
      if (l == 0) {
        sh.cg[j * TK_W + wv] = (uint32_t)__popcll(bg);
        sh.ce[j * TK_W + wv] = (uint32_t)__popcll(be);
      }
    }
    __syncthreads();
    const uint2 tot = block_scan2(sh.cg, sh.ce, JC * TK_W, sh.wtot);
#pragma unroll
    for (int j = 0; j < JC; ++j) {
      const int s = c * CH + j * TK_T + tid;
      const bool valid = s < L;
      const uint32_t k = float_key(x[j]);
      const bool gt = valid && k > T, eq = valid && k == T;
      const uint64_t bg = __ballot(gt);
      const uint64_t be = __ballot(eq);
      const uint32_t G = carry_g + sh.cg[j * TK_W + wv] + (uint32_t)__popcll(bg & lt);
      const uint32_t E = carry_e + sh.ce[j * TK_W + wv] + (uint32_t)__popcll(be & lt);
      const uint32_t at = G + min(E, m);
      if ((gt || (eq && E < m)) && at < (uint32_t)n) orow[at] = s;
    }
    carry_g += tot.x;
    carry_e += tot.y;
    __syncthreads();
  }
  for (int i = n + tid; i < topk; i += TK_T) orow[i] = -1;
}

}  // namespace

hipError_t launch_topk(const dsa_rows& rows, int topk, const float* scores, int64_t ld,
                       int32_t* indices, hipStream_t stream) {
  const int R = rows.num_rows;
  const int L = rows.max_pos + 1;
  if (L <= 8 * TK_T) {
    hipLaunchKernelGGL((topk_kernel<8, true>), dim3(R), dim3(TK_T), 0, stream, scores, ld,
                       rows.row_pos, rows.max_pos, topk, indices);
  } else if (L <= 32 * TK_T) {
    hipLaunchKernelGGL((topk_kernel<32, true>), dim3(R), dim3(TK_T), 0, stream, scores, ld,
                       rows.row_pos, rows.max_pos, topk, indices);
  } else {
    hipLaunchKernelGGL((topk_kernel<16, false>), dim3(R), dim3(TK_T), 0, stream, scores, ld,
                       rows.row_pos, rows.max_pos, topk, indices);
  }
  return hipGetLastError();
}

}  // namespace dsa
