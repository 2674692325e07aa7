// Indexer training loss of the sparse stage and its gradients.
//
// DeepSeek-V3.2-Exp paper, section 2.1 (dense warm-up and sparse training stages):
// for query token t the main attention scores are summed over all heads and
// L1-normalised along the sequence into a target p[t,:], and the indexer is trained
// with KL(p[t,:] || Softmax(I[t,:])), in the sparse stage over the selected set S_t;
// the indexer's inputs are detached, so this loss trains the indexer alone.
//
//   target:   a[h,i] = exp(scale q[h] . c[s_i] - lse[h])   (each head's softmax
//             weights over S_t; lse is the attention call's output)
//             u[i] = sum_h a[h,i]                       (attn_target_kernel)
//   loss:     p = u / sum_i u;  L = sum_i p_i (log p_i - log softmax(I[S_t])_i)
//             dI_i = softmax(I[S_t])_i - p_i            (indexer_kl_kernel)
//   backward: with d = q_j . k_s (dequantised) and m = [d > 0]
//             dw_j += dI_s relu(d),  dq_j += dI_s w_j m k_s,  dk_s += dI_s w_j m q_j
//                                                       (indexer_bwd_kernel)
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int H = kHeads;      // 128
constexpr int DK = kQkDim;     // 576
constexpr int IH = kIdxHeads;  // 64
constexpr int ID = kIdxDim;    // 128

// ---------------------------------------------------------------------------
// Target u[r, i] for the entries of one slice of row r's selection.  Eight waves,
// wave w owns heads [16 w, 16 w + 16) with their queries in registers; entries are
// staged 32 at a time in LDS (16-byte pieces XOR-swizzled by entry) and multiplied
// on the bf16 MFMA as S^T tiles (16 entries x 16 heads), so each lane ends with 4
// entries of one head.  The head sum is a DPP row reduction plus an LDS sum over
// the waves.
// ---------------------------------------------------------------------------
constexpr int TT = 512;            // threads per target block
constexpr int TBE = 32;            // entries per stage
constexpr int TCH = DK * 2 / 16;   // 72 pieces of 16 bytes per entry
constexpr int TKS = DK / 32;       // 18 contraction steps

__global__ __launch_bounds__(TT) void attn_target_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ latent,
    const int32_t* __restrict__ indices, const float* __restrict__ lse,
    const int32_t* __restrict__ row_seq, const int32_t* __restrict__ row_pos, int R, int B,
    int N, int topk, int splits, float scale_log2, float* __restrict__ u, PageMap pm) {
  __shared__ __attribute__((aligned(16))) i32x4 tile[TBE * TCH];
  __shared__ float part[TT / 64][TBE];
  const int r = blockIdx.x / splits, sp = blockIdx.x - r * splits;
  if (r >= R) return;
  const int b = row_seq[r], t = row_pos[r];
  const int ES = topk / splits;
  const int32_t* irow = indices + (size_t)r * topk + (size_t)sp * ES;
  float* urow = u + (size_t)r * topk + (size_t)sp * ES;
  if (b < 0 || b >= B || t < 0 || t >= N) {
    for (int i = threadIdx.x; i < ES; i += TT) urow[i] = 0.f;
    return;
  }
  const int tid = threadIdx.x, l = lane_id(), g = l >> 4, n = l & 15;
  const int wv = tid >> 6;
  const bool paged = pm.table != nullptr;
  const uint8_t* base = reinterpret_cast<const uint8_t*>(paged ? latent : latent + (size_t)b * N * DK);
  auto row_of = [&](int p) -> uint32_t { return paged ? paged_row(pm, b, p) : (uint32_t)p; };
  const uint32_t row0 = row_of(0);

  // queries of heads 16 wv + n, contraction step s: dims [32 s + 8 g, +8)
  i32x4 qr[TKS];
  const uint16_t* qrow = q + ((size_t)r * H + 16 * wv + n) * DK + 8 * g;
#pragma unroll
  for (int s = 0; s < TKS; ++s) qr[s] = *reinterpret_cast<const i32x4*>(qrow + 32 * s);
  // log2-domain lse of this lane's head
  const float lse2 = lse[(size_t)r * H + 16 * wv + n] * 1.44269504088896340736f;

  // The next stage's pieces are fetched into registers while this stage computes:
  // piece tid + TT j (j < 5; the last only for tid < 256) of the 32 x 72 tile.
  constexpr int SPT = (TBE * TCH + TT - 1) / TT;  // 5
  i32x4 spf[SPT];
  auto sfetch = [&](int e0) {
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int c = tid + TT * j;
      if (j < SPT - 1 || tid < TT / 2) {
        const int e = c / TCH, pc = c - e * TCH;
        const int p = irow[e0 + e];
        const uint32_t row = (p >= 0 && p <= t) ? row_of(p) : row0;
        spf[j] = *reinterpret_cast<const i32x4*>(base + (size_t)row * (DK * 2) + 16 * pc);
      }
    }
  };
  auto sstash = [&]() {
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int c = tid + TT * j;
      if (j < SPT - 1 || tid < TT / 2) {
        const int e = c / TCH, pc = c - e * TCH;
        tile[e * TCH + (pc ^ (e & 7))] = spf[j];
      }
    }
  };
  if (ES > 0) sfetch(0);
  for (int e0 = 0; e0 < ES; e0 += TBE) {
    __syncthreads();  // previous stage's tile reads are done
    sstash();
    __syncthreads();
    if (e0 + TBE < ES) sfetch(e0 + TBE);
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int s = 0; s < TKS; ++s)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int e = 16 * mt + n;
        const bf16x8 a = as_bf16x8(tile[e * TCH + ((4 * s + g) ^ (e & 7))]);
        acc[mt] = mfma_bf16_16x16x32(a, as_bf16x8(qr[s]), acc[mt]);
      }
    // lane: entries 16 mt + 4 g + v of head 16 wv + n
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float x = exp2f(acc[mt][v] * scale_log2 - lse2);
        uint32_t xb = __float_as_uint(x);
        xb = __float_as_uint(__uint_as_float(xb) + __uint_as_float(dpp<kDppXor1>(xb)));
        xb = __float_as_uint(__uint_as_float(xb) + __uint_as_float(dpp<kDppXor2>(xb)));
        xb = __float_as_uint(__uint_as_float(xb) + __uint_as_float(dpp<kDppHalfMirror>(xb)));
        xb = __float_as_uint(__uint_as_float(xb) + __uint_as_float(dpp<kDppMirror>(xb)));
        if (n == 0) part[wv][16 * mt + 4 * g + v] = __uint_as_float(xb);
      }
    __syncthreads();
    if (tid < TBE) {
      float sum = 0.f;
#pragma unroll
      for (int w8 = 0; w8 < TT / 64; ++w8) sum += part[w8][tid];
      const int p = irow[e0 + tid];
      urow[e0 + tid] = (p >= 0 && p <= t) ? sum : 0.f;  // entries outside [0, t]: padding
    }
  }
}

// ---------------------------------------------------------------------------
// Dense warm-up target over every causal position s <= t, in chunks of DCP
// contiguous positions per block (same wave layout and MFMA tiles as above).
// LSE_PASS: each block leaves the per-head (max, sum) of exp2(scale_log2 q.c) over
// its chunk in part[r, chunk, h] (log2 domain).  Target pass: each block merges its
// row's chunk partials into the head's lse and writes u[r, s] for its chunk.
// ---------------------------------------------------------------------------
constexpr int DCP = 1024;  // positions per dense chunk

template <bool LSE_PASS>
__global__ __launch_bounds__(TT) void dense_target_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ latent,
    const int32_t* __restrict__ row_seq, const int32_t* __restrict__ row_pos, int R, int B, int N,
    int max_pos, int C, float scale_log2, float2* __restrict__ part, float* __restrict__ u,
    int64_t ldu) {
  __shared__ __attribute__((aligned(16))) i32x4 tile[TBE * TCH];
  __shared__ float hsum[TT / 64][TBE];
  const int r = blockIdx.x / C, c = blockIdx.x - (blockIdx.x / C) * C;
  if (r >= R) return;
  const int b = row_seq[r], t = row_pos[r];
  // a row past max_pos has no chunk partials or target space: it is not processed
  const bool ok = b >= 0 && b < B && t >= 0 && t < N && t <= max_pos;
  const int p0 = c * DCP;
  const int pend = ok ? min(t + 1, p0 + DCP) : p0;  // this chunk's positions: [p0, pend)
  const int tid = threadIdx.x, l = lane_id(), g = l >> 4, n = l & 15;
  const int wv = tid >> 6;
  const int head = 16 * wv + n;
  float2* prow = part + (size_t)r * C * H;
  if (pend <= p0) {  // no position of this row in the chunk
    if (LSE_PASS && g == 0) prow[(size_t)c * H + head] = make_float2(-INFINITY, 0.f);
    return;
  }
  const uint8_t* base = reinterpret_cast<const uint8_t*>(latent + (size_t)b * N * DK);

  // queries of heads 16 wv + n, contraction step s: dims [32 s + 8 g, +8)
  i32x4 qr[TKS];
  const uint16_t* qrow = q + ((size_t)r * H + head) * DK + 8 * g;
#pragma unroll
  for (int s = 0; s < TKS; ++s) qr[s] = *reinterpret_cast<const i32x4*>(qrow + 32 * s);
  float lse2 = 0.f;
  if (!LSE_PASS) {  // merge the row's chunk partials of this lane's head
    const int nc = (t + DCP) / DCP;
    float M = -INFINITY;
    for (int k = 0; k < nc; ++k) M = fmaxf(M, prow[(size_t)k * H + head].x);
    float S = 0.f;
    for (int k = 0; k < nc; ++k) {
      const float2 pm = prow[(size_t)k * H + head];
      if (pm.x != -INFINITY) S += pm.y * exp2f(pm.x - M);
    }
    lse2 = M + log2f(S);
  }
  float m_run = -INFINITY, l_run = 0.f;

  // The next stage's pieces are fetched into registers while this stage computes:
  // piece tid + TT j (j < 5; the last only for tid < 256) of the 32 x 72 tile.
  constexpr int PPT = (TBE * TCH + TT - 1) / TT;  // 5
  static_assert(TBE * TCH - (PPT - 1) * TT == TT / 2, "the last piece: half the threads");
  i32x4 pf[PPT];
  auto fetch = [&](int e0) {
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int cc = tid + TT * j;
      if (j < PPT - 1 || tid < TT / 2) {
        const int e = cc / TCH, pc = cc - e * TCH;
        const int pos = min(e0 + e, pend - 1);  // past the end: a valid entry, masked below
        pf[j] = *reinterpret_cast<const i32x4*>(base + (size_t)pos * (DK * 2) + 16 * pc);
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int cc = tid + TT * j;
      if (j < PPT - 1 || tid < TT / 2) {
        const int e = cc / TCH, pc = cc - e * TCH;
        tile[e * TCH + (pc ^ (e & 7))] = pf[j];
      }
    }
  };
  fetch(p0);
  for (int e0 = p0; e0 < pend; e0 += TBE) {
    __syncthreads();  // previous stage's tile reads are done
    stash();
    __syncthreads();
    if (e0 + TBE < pend) fetch(e0 + TBE);
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int s = 0; s < TKS; ++s)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int e = 16 * mt + n;
        const bf16x8 a = as_bf16x8(tile[e * TCH + ((4 * s + g) ^ (e & 7))]);
        acc[mt] = mfma_bf16_16x16x32(a, as_bf16x8(qr[s]), acc[mt]);
      }
    // lane: entries 16 mt + 4 g + v of head 16 wv + n
    if (LSE_PASS) {
      float z[8];
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const bool in = e0 + 16 * mt + 4 * g + v < pend;
          z[4 * mt + v] = in ? acc[mt][v] * scale_log2 : -INFINITY;
          mx = fmaxf(mx, z[4 * mt + v]);
        }
      const float m_new = fmaxf(m_run, mx);
      if (m_new != -INFINITY) {
        float add = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) add += z[i] == -INFINITY ? 0.f : exp2f(z[i] - m_new);
        l_run = (m_run == -INFINITY ? 0.f : l_run * exp2f(m_run - m_new)) + add;
        m_run = m_new;
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float x = exp2f(acc[mt][v] * scale_log2 - lse2);
          uint32_t xb = __float_as_uint(x);
          xb = __float_as_uint(__uint_as_float(xb) + __uint_as_float(dpp<kDppXor1>(xb)));
          xb = __float_as_uint(__uint_as_float(xb) + __uint_as_float(dpp<kDppXor2>(xb)));
          xb = __float_as_uint(__uint_as_float(xb) + __uint_as_float(dpp<kDppHalfMirror>(xb)));
          xb = __float_as_uint(__uint_as_float(xb) + __uint_as_float(dpp<kDppMirror>(xb)));
          if (n == 0) hsum[wv][16 * mt + 4 * g + v] = __uint_as_float(xb);
        }
      __syncthreads();
      if (tid < TBE && e0 + tid < pend) {
        float sum = 0.f;
#pragma unroll
        for (int w8 = 0; w8 < TT / 64; ++w8) sum += hsum[w8][tid];
        u[(size_t)r * ldu + e0 + tid] = sum;
      }
    }
  }
  if (LSE_PASS) {
    // merge the four lanes (g) that hold this head's entries
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const float mo = __shfl_xor(m_run, o), lo = __shfl_xor(l_run, o);
      const float mn = fmaxf(m_run, mo);
      if (mn != -INFINITY) {
        l_run = (m_run == -INFINITY ? 0.f : l_run * exp2f(m_run - mn)) +
                (mo == -INFINITY ? 0.f : lo * exp2f(mo - mn));
        m_run = mn;
      }
    }
    if (g == 0) prow[(size_t)c * H + head] = make_float2(m_run, l_run);
  }
}

// ---------------------------------------------------------------------------
// KL(p || softmax(I over the selection)) and its gradient for one row per block.
// ---------------------------------------------------------------------------
constexpr int KT = 256;

__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum_f(v);
  __syncthreads();
  if (lane_id() == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < KT / 64; ++i) s += red[i];
  return s;
}
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  __syncthreads();
  if (lane_id() == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = -INFINITY;
#pragma unroll
  for (int i = 0; i < KT / 64; ++i) s = fmaxf(s, red[i]);
  return s;
}

__global__ __launch_bounds__(KT) void indexer_kl_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ indices,
    const float* __restrict__ u, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_pos, int B, int N, int topk, float* __restrict__ loss,
    float* __restrict__ dscores) {
  __shared__ float red[KT / 64];
  const int r = blockIdx.x;
  const int b = row_seq[r], t = row_pos[r];
  const int32_t* irow = indices + (size_t)r * topk;
  const float* urow = u + (size_t)r * topk;
  float* grow = dscores + (size_t)r * topk;
  const bool ok = b >= 0 && b < B && t >= 0 && t < N && (int64_t)t < ld;
  const float* srow = scores + (size_t)r * ld;
  auto valid = [&](int p) { return ok && p >= 0 && p <= t; };
  float m = -INFINITY, us = 0.f;
  for (int i = threadIdx.x; i < topk; i += KT) {
    const int p = irow[i];
    if (valid(p)) {
      m = fmaxf(m, srow[p]);
      us += urow[i];
    }
  }
  m = block_max(m, red);
  us = block_sum(us, red);
  float z = 0.f;
  for (int i = threadIdx.x; i < topk; i += KT) {
    const int p = irow[i];
    if (valid(p)) z += expf(srow[p] - m);
  }
  z = block_sum(z, red);
  const float lz = m + logf(z);
  const float inv_u = us > 0.f ? 1.f / us : 0.f;
  float kl = 0.f;
  for (int i = threadIdx.x; i < topk; i += KT) {
    const int p = irow[i];
    float gi = 0.f;
    if (valid(p)) {
      const float pi = urow[i] * inv_u;
      const float lq = srow[p] - lz;
      if (pi > 0.f) kl += pi * (logf(pi) - lq);
      gi = expf(lq) - pi;
    }
    grow[i] = gi;
  }
  kl = block_sum(kl, red);
  if (threadIdx.x == 0) loss[r] = (ok && z > 0.f) ? kl : 0.f;
}

// KL(p || softmax(I over all s <= t)) and its gradient, one row per block: the
// dense warm-up loss, from the dense target u[r, s].
__global__ __launch_bounds__(KT) void indexer_kl_dense_kernel(
    const float* __restrict__ scores, int64_t ld, const float* __restrict__ u, int64_t ldu,
    const int32_t* __restrict__ row_seq, const int32_t* __restrict__ row_pos, int B, int N,
    int max_pos, float* __restrict__ loss, float* __restrict__ dscores) {
  __shared__ float red[KT / 64];
  const int r = blockIdx.x;
  const int b = row_seq[r], t = row_pos[r];
  // t <= max_pos keeps every read of the target row u inside its ldu entries
  const bool ok = b >= 0 && b < B && t >= 0 && t < N && t <= max_pos && (int64_t)t < ld;
  const int np = ok ? t + 1 : 0;
  const float* srow = scores + (size_t)r * ld;
  const float* urow = u + (size_t)r * ldu;
  float* grow = dscores + (size_t)r * ld;
  float m = -INFINITY, us = 0.f;
  for (int p = threadIdx.x; p < np; p += KT) {
    m = fmaxf(m, srow[p]);
    us += urow[p];
  }
  m = block_max(m, red);
  us = block_sum(us, red);
  float z = 0.f;
  for (int p = threadIdx.x; p < np; p += KT) z += expf(srow[p] - m);
  z = block_sum(z, red);
  const float lz = m + logf(z);
  const float inv_u = us > 0.f ? 1.f / us : 0.f;
  float kl = 0.f;
  for (int64_t p = threadIdx.x; p < ld; p += KT) {
    float gi = 0.f;
    if (p < np) {
      const float pi = urow[p] * inv_u;
      const float lq = srow[p] - lz;
      if (pi > 0.f) kl += pi * (logf(pi) - lq);
      gi = expf(lq) - pi;
    }
    grow[p] = gi;
  }
  kl = block_sum(kl, red);
  if (threadIdx.x == 0) loss[r] = (ok && z > 0.f) ? kl : 0.f;
}

// ---------------------------------------------------------------------------
// Backward into the indexer for 4 groups of 64 selected entries of one row per
// block.  The
// 64-head x 64-key dots come from the fp8 MFMA exactly as in the forward (exact
// fp8 MFMA dots); each wave owns one 16-key tile, each lane 16 heads of
// one key.  The coefficient matrices for dq and dk go through LDS; the two
// 64 x 64 x 128 products run in fp32 on the VALU (each thread 4 heads or 4 keys
// x 8 dims), and the results are added with atomics (dq over the row's blocks,
// dk over the rows that select a key, dw over the row's blocks).
// ---------------------------------------------------------------------------
constexpr int BT = 256;
constexpr int BG = 64;   // entries per group
constexpr int BGPB = 4;  // groups per block (dq and dw stay in registers across them)

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t s = (c & 0x80u) << 24, e = (c >> 3) & 15u, m = c & 7u;
  const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  return __uint_as_float(__float_as_uint(mag) | s);
}

// DENSE: the entries are every causal position 0..t (no index list), with dscores
// [R, ld] indexed by position (the dense warm-up loss's gradient); nblk_dense
// blocks per row cover positions up to max_pos.
template <bool DENSE>
__global__ __launch_bounds__(BT) void indexer_bwd_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ k_idx,
    const float* __restrict__ k_scale, const int32_t* __restrict__ indices,
    const float* __restrict__ dscores, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_pos, int B, int N, int max_pos, int topk,
    float* __restrict__ dq, float* __restrict__ dw, float* __restrict__ dk, PageMap pm, int64_t ld,
    int nblk_dense) {
  __shared__ __attribute__((aligned(16))) float kf[BG][ID + 4];   // dequantised keys
  __shared__ __attribute__((aligned(16))) float qf[IH][ID + 4];   // dequantised queries
  __shared__ __attribute__((aligned(16))) float cq[IH][BG + 4];   // dI w m, head-major
  __shared__ __attribute__((aligned(16))) float ck[BG][IH + 4];   // the same, key-major
  __shared__ float dwp[BT / 64][IH];
  __shared__ int rows_s[BG];
  __shared__ float g_s[BG], ks_s[BG];
  const int nblk = DENSE ? nblk_dense : topk / (BG * BGPB);
  const int r = blockIdx.x / nblk, ebase = (blockIdx.x - r * nblk) * BG * BGPB;
  const int b = row_seq[r], t = row_pos[r];
  // a row past max_pos is not processed (the dense blocks and dscores columns only
  // reach max_pos)
  if (b < 0 || b >= B || t < 0 || t >= N || t > max_pos) return;
  if (DENSE && ebase > t) return;  // every position of this block is past the row
  const int tid = threadIdx.x, l = lane_id(), g = l >> 4, n = l & 15, wv = tid >> 6;
  const bool paged = pm.table != nullptr;
  const uint8_t* kbase = paged ? k_idx : k_idx + (size_t)b * N * ID;
  const float* sbase = paged ? k_scale : k_scale + (size_t)b * N;
  const uint8_t* qr = q_idx + (size_t)r * IH * ID;

  // dequantised queries, once per block
  for (int c = tid; c < IH * ID / 4; c += BT) {
    const int j = c / (ID / 4), d4 = c - j * (ID / 4);
    const uint32_t word = *reinterpret_cast<const uint32_t*>(qr + (size_t)j * ID + 4 * d4);
    const float sc = q_scale[(size_t)r * IH + j];
#pragma unroll
    for (int i = 0; i < 4; ++i) qf[j][4 * d4 + i] = e4m3_value((word >> (8 * i)) & 0xffu) * sc;
  }
  // this lane's fp8 queries for the dots (A operand of head tile mt)
  i32x8 qa[4];
  float qsj[16], wjj[16];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const i32x4* qp = reinterpret_cast<const i32x4*>(qr + (size_t)(16 * mt + n) * ID + 32 * g);
    const i32x4 b0 = qp[0], b1 = qp[1];
    qa[mt] = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int j = 16 * mt + 4 * g + v;
      qsj[4 * mt + v] = q_scale[(size_t)r * IH + j];
      wjj[4 * mt + v] = w[(size_t)r * IH + j];
    }
  }
  float dwacc = 0.f;                       // head tid (tid < 64), over the block's groups
  const int j0 = 4 * (tid >> 4), d0 = 8 * (tid & 15);
  float accq[4][8] = {};                   // dq of heads j0.., dims d0.., over the groups

  for (int gi = 0; gi < BGPB; ++gi) {
    const int e0 = ebase + gi * BG;
    __syncthreads();  // the previous group's LDS reads are done
    if (tid < BG) {
      const int p = DENSE ? e0 + tid : indices[(size_t)r * topk + e0 + tid];
      const bool v = p >= 0 && p <= t;
      const int row = v ? (paged ? (int)paged_row(pm, b, p) : p) : -1;
      rows_s[tid] = row;
      g_s[tid] = v ? (DENSE ? dscores[(size_t)r * ld + p] : dscores[(size_t)r * topk + e0 + tid]) : 0.f;
      ks_s[tid] = v ? sbase[row] : 0.f;
    }
    __syncthreads();
    for (int c = tid; c < BG * ID / 4; c += BT) {
      const int e = c / (ID / 4), d4 = c - e * (ID / 4);
      const int row = rows_s[e];
      const uint32_t word =
          row >= 0 ? *reinterpret_cast<const uint32_t*>(kbase + (size_t)row * ID + 4 * d4) : 0u;
      const float sc = ks_s[e];
#pragma unroll
      for (int i = 0; i < 4; ++i) kf[e][4 * d4 + i] = e4m3_value((word >> (8 * i)) & 0xffu) * sc;
    }
    // fp8 dots of the 64 heads with this wave's 16 keys (the forward's arithmetic)
    {
      const int e = 16 * wv + n;  // this lane's key
      const int row = rows_s[e];
      i32x8 kb = {0, 0, 0, 0, 0, 0, 0, 0};
      if (row >= 0) {
        const i32x4* kp = reinterpret_cast<const i32x4*>(kbase + (size_t)row * ID + 32 * g);
        const i32x4 a0 = kp[0], a1 = kp[1];
        kb = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
      }
      const float ge = g_s[e], kse = ks_s[e];
      float dwl[16];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4 d8 = mfma_fp8_16x16x128(qa[mt], kb, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int j = 16 * mt + 4 * g + v;
          const bool pos = d8[v] > 0.f;
          // kf and qf hold dequantised values, so the coefficient carries no scale
          const float c = pos ? ge * wjj[4 * mt + v] : 0.f;
          dwl[4 * mt + v] = pos ? ge * d8[v] * qsj[4 * mt + v] * kse : 0.f;
          cq[j][e] = c;
          ck[e][j] = c;
        }
      }
      // dw: sum over the wave's 16 keys (the 16 lanes of a row), then over waves
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        uint32_t x = __float_as_uint(dwl[i]);
        x = __float_as_uint(__uint_as_float(x) + __uint_as_float(dpp<kDppXor1>(x)));
        x = __float_as_uint(__uint_as_float(x) + __uint_as_float(dpp<kDppXor2>(x)));
        x = __float_as_uint(__uint_as_float(x) + __uint_as_float(dpp<kDppHalfMirror>(x)));
        x = __float_as_uint(__uint_as_float(x) + __uint_as_float(dpp<kDppMirror>(x)));
        if (n == 0) dwp[wv][16 * (i >> 2) + 4 * g + (i & 3)] = __uint_as_float(x);
      }
    }
    __syncthreads();
    if (tid < IH) dwacc += dwp[0][tid] + dwp[1][tid] + dwp[2][tid] + dwp[3][tid];
    // dq[j][d] += sum_e cq[j][e] kf[e][d]: thread = 4 heads x 8 dims, kept in registers
    for (int e = 0; e < BG; ++e) {
      const float4 k0 = *reinterpret_cast<const float4*>(&kf[e][d0]);
      const float4 k1 = *reinterpret_cast<const float4*>(&kf[e][d0 + 4]);
      const float kv[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const float c = cq[j0 + a][e];
#pragma unroll
        for (int d = 0; d < 8; ++d) accq[a][d] = fmaf(c, kv[d], accq[a][d]);
      }
    }
    // dk[e][d] += sum_j ck[e][j] qf[j][d]: thread = 4 keys x 8 dims, added per group
    {
      float acc[4][8] = {};
      for (int j = 0; j < IH; ++j) {
        const float4 q0 = *reinterpret_cast<const float4*>(&qf[j][d0]);
        const float4 q1 = *reinterpret_cast<const float4*>(&qf[j][d0 + 4]);
        const float qv[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const float c = ck[j0 + a][j];
#pragma unroll
          for (int d = 0; d < 8; ++d) acc[a][d] = fmaf(c, qv[d], acc[a][d]);
        }
      }
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int row = rows_s[j0 + a];
        if (row < 0) continue;
        float* dkr = dk + (paged ? (size_t)row : (size_t)b * N + row) * ID;
#pragma unroll
        for (int d = 0; d < 8; ++d)
          if (acc[a][d] != 0.f) atomicAdd(&dkr[d0 + d], acc[a][d]);
      }
    }
  }
  if (tid < IH && dwacc != 0.f) atomicAdd(&dw[(size_t)r * IH + tid], dwacc);
  float* dqr = dq + (size_t)r * IH * ID;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int d = 0; d < 8; ++d)
      if (accq[a][d] != 0.f) atomicAdd(&dqr[(size_t)(j0 + a) * ID + d0 + d], accq[a][d]);
}

}  // namespace

size_t indexer_loss_workspace_bytes(int num_rows, int topk) {
  return (size_t)num_rows * topk * sizeof(float);
}

hipError_t launch_indexer_loss(const dsa_rows& rows, const void* q, const void* latent,
                               const int32_t* indices, const float* lse, float softmax_scale,
                               const float* scores, int64_t ld, float* loss, float* dscores,
                               void* workspace, hipStream_t stream, const PageMap& pm) {
  const int R = rows.num_rows;
  if (R == 0) return hipSuccess;
  int splits = 1;
  while (splits < kTopk / TBE && (int64_t)R * splits < 256) splits <<= 1;
  float* u = static_cast<float*>(workspace);
  hipLaunchKernelGGL(attn_target_kernel, dim3(R * splits), dim3(TT), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(latent), indices,
                     lse, rows.row_seq, rows.row_pos, R, rows.num_seqs, rows.max_ctx, kTopk, splits,
                     softmax_scale * 1.44269504088896340736f, u, pm);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(indexer_kl_kernel, dim3(R), dim3(KT), 0, stream, scores, ld, indices, u,
                     rows.row_seq, rows.row_pos, rows.num_seqs, rows.max_ctx, kTopk, loss, dscores);
  return hipGetLastError();
}

size_t indexer_loss_dense_workspace_bytes(int num_rows, int max_pos) {
  const size_t C = (size_t)(max_pos + DCP) / DCP;
  return (size_t)num_rows * C * (DCP * sizeof(float) + H * sizeof(float2));
}

hipError_t launch_indexer_loss_dense(const dsa_rows& rows, const void* q, const void* latent,
                                     float softmax_scale, const float* scores, int64_t ld,
                                     float* loss, float* dscores, void* workspace,
                                     hipStream_t stream) {
  const int R = rows.num_rows;
  if (R == 0) return hipSuccess;
  const int C = (rows.max_pos + DCP) / DCP;
  const int64_t ldu = (int64_t)C * DCP;
  float* u = static_cast<float*>(workspace);
  float2* part = reinterpret_cast<float2*>(u + (size_t)R * ldu);
  const float sl2 = softmax_scale * 1.44269504088896340736f;
  const dim3 grid((unsigned)((int64_t)R * C));
  hipLaunchKernelGGL(dense_target_kernel<true>, grid, dim3(TT), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(latent),
                     rows.row_seq, rows.row_pos, R, rows.num_seqs, rows.max_ctx, rows.max_pos, C, sl2,
                     part, u, ldu);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(dense_target_kernel<false>, grid, dim3(TT), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(latent),
                     rows.row_seq, rows.row_pos, R, rows.num_seqs, rows.max_ctx, rows.max_pos, C, sl2,
                     part, u, ldu);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(indexer_kl_dense_kernel, dim3(R), dim3(KT), 0, stream, scores, ld, u, ldu,
                     rows.row_seq, rows.row_pos, rows.num_seqs, rows.max_ctx, rows.max_pos, loss,
                     dscores);
  return hipGetLastError();
}

hipError_t launch_indexer_backward(const dsa_rows& rows, const uint8_t* q_idx,
                                   const float* q_scale, const float* w, const uint8_t* k_idx,
                                   const float* k_scale, const int32_t* indices,
                                   const float* dscores, float* dq, float* dw, float* dk,
                                   hipStream_t stream, const PageMap& pm) {
  const int R = rows.num_rows;
  if (R == 0) return hipSuccess;
  hipLaunchKernelGGL(indexer_bwd_kernel<false>, dim3(R * (kTopk / (BG * BGPB))), dim3(BT), 0, stream,
                     q_idx, q_scale, w, k_idx, k_scale, indices, dscores, rows.row_seq, rows.row_pos,
                     rows.num_seqs, rows.max_ctx, rows.max_pos, kTopk, dq, dw, dk, pm, (int64_t)0, 0);
  return hipGetLastError();
}

hipError_t launch_indexer_backward_dense(const dsa_rows& rows, const uint8_t* q_idx,
                                         const float* q_scale, const float* w, const uint8_t* k_idx,
                                         const float* k_scale, const float* dscores, int64_t ld,
                                         float* dq, float* dw, float* dk, hipStream_t stream) {
  const int R = rows.num_rows;
  if (R == 0) return hipSuccess;
  const int nblk = (rows.max_pos + BG * BGPB) / (BG * BGPB);
  hipLaunchKernelGGL(indexer_bwd_kernel<true>, dim3((unsigned)((int64_t)R * nblk)), dim3(BT), 0,
                     stream, q_idx, q_scale, w, k_idx, k_scale, nullptr, dscores, rows.row_seq,
                     rows.row_pos, rows.num_seqs, rows.max_ctx, rows.max_pos, kTopk, dq, dw, dk,
                     PageMap{}, ld, nblk);
  return hipGetLastError();
}

}  // namespace dsa
