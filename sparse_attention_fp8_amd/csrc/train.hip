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
//                     (bwd_count_kernel, indexer_bwd_kernel, bwd_reduce_kernel,
//                      bwd_finalize_kernel)
#include <algorithm>

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
// Backward into the indexer.  A row's entries are cut into E chunks of G groups of
// 64 entries, and block (row, chunk) takes one chunk.  The 64-head x 64-key dots
// of a group come from the fp8 MFMA exactly as in the forward (each wave owns one
// 16-key tile, each lane 16 heads of one key).  The two 64 x 64 x 128 products,
//   dq[j][d] += sum_e (dI_e w_j m_je k_scale_e) code_k[e][d]  and
//   dk[e][d] += sum_j (dI_e w_j m_je q_scale_j) code_q[j][d],
// run on the bf16 MFMA with fp32 accumulation: the fp8 codes are bf16 values
// exactly, and each fp32 coefficient is split into three bf16 parts that sum to it
// (to within 2^-25 of it), so every product is the fp32 one.  A group's fp8 keys
// are staged once in LDS (for the dots, and as bf16 in dim-major order for dq); the
// next group's entries and key bytes are loaded into registers while the current
// group's products run; the dk terms go through LDS, so that each wave then writes
// whole key rows (every instruction whole cache lines).
//
// Every sum is formed in an order that the call's shape fixes, so the outputs are
// the same bits from run to run:
//  * dq and dw: with one chunk per row the block adds its sums into the row's dq and
//    dw, the only writer of them.  With several chunks each block stores its sums in
//    a partial slot of its own, and bwd_reduce_kernel adds the slots into dq and dw
//    in chunk order.
//  * dk: bwd_count_kernel first counts how often each key is selected in the call.
//    A key selected once has one writer, which adds into dk directly.  A key selected
//    more than once gets an accumulator of 128 64-bit integers.  Every contribution
//    is added there as a fixed-point integer, v 2^s rounded to nearest; integer
//    addition gives the same sum in any order.  bwd_finalize_kernel then adds
//    sum 2^-s into dk.  One exponent s serves the whole call: the largest for which
//    (largest count) x (bound on any contribution) stays below 2^62, so no sum can
//    overflow.  The bound is max |dI| over the call times the largest over rows of
//    max_d sum_j |w_rj| |q_rj[d]|, with q dequantised.  Each
//    contribution is then exact to within 2^-(s+1).  If the call has more such
//    keys than accumulators, or the bound is not finite (inf or NaN inputs), those
//    keys are added into dk with fp32 atomics instead, whose order, and last bits,
//    vary.
// ---------------------------------------------------------------------------
constexpr int BT = 256;
constexpr int BG = 64;                    // entries per group
constexpr int kPartLen = IH * ID + IH;    // floats of one partial slot: dq, then dw
constexpr int kBwdTargetBlocks = 256;     // one block per CU (the LDS allows one)

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t s = (c & 0x80u) << 24, e = (c >> 3) & 15u, m = c & 7u;
  const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  return __uint_as_float(__float_as_uint(mag) | s);
}

// Workspace of the backward (the host lays it out; every piece 256-byte aligned)
struct BwdWs {
  int* hdr;            // [0] accumulators in use, [1] max |dI| (float bits), [2] largest
                       // count, [3] max over rows of max_d sum_j |w_j q_j[d]| (float bits)
  int* rowflag;        // [R] 1: the row's keys are each selected once in the call
  int* cnt;            // [B * (max_pos + 1)] selections of each key
  int* slot;           // [B * (max_pos + 1)] accumulator of a key selected twice or more
  int* slotkey;        // [cap] key (b * (max_pos + 1) + p) of each accumulator
  long long* acc;      // [cap * ID] fixed-point sums
  float* part;         // [R * E * kPartLen] chunk sums of dq and dw (E > 1 only)
  int cap;             // accumulators
};

// A row is processed when its sequence and position are in range and t <= max_pos
// (the dense blocks and the dscores columns only reach max_pos).
__device__ __forceinline__ bool bwd_row_ok(int b, int t, int B, int N, int max_pos) {
  return b >= 0 && b < B && t >= 0 && t < N && t <= max_pos;
}

// Exponent s of the fixed-point sums: up = 2^s, down = 2^-s, the largest s with
// (largest count) x max|dI| x max_r max_d sum_j |w_j q_j[d]| < 2^62.  False when a
// bound is not finite.
__device__ __forceinline__ bool bwd_scale(const int* hdr, double& up, double& down) {
  const uint32_t gb = (uint32_t)hdr[1], sb = (uint32_t)hdr[3];
  if (gb >= 0x7f800000u || sb >= 0x7f800000u) return false;  // inf or NaN (never negative)
  const double lim = (double)__uint_as_float(gb) * (double)__uint_as_float(sb) *
                     (double)max(hdr[2], 1);
  int e = 0;
  if (lim > 0.0) frexp(lim, &e);  // lim < 2^e
  up = ldexp(1.0, 62 - e);
  down = ldexp(1.0, e - 62);
  return true;
}

// Clears the header and the selection counts (a fill kernel, so that a captured
// graph holds no memset node).  n4 = int4 words of the count table.
__global__ __launch_bounds__(BT) void bwd_clear_kernel(int* __restrict__ hdr,
                                                       int4* __restrict__ cnt, int64_t n4) {
  if (blockIdx.x == 0 && threadIdx.x < 4) hdr[threadIdx.x] = 0;
  for (int64_t i = (int64_t)blockIdx.x * BT + threadIdx.x; i < n4; i += (int64_t)gridDim.x * BT)
    cnt[i] = make_int4(0, 0, 0, 0);
}

// One block per row.  A row is "simple" when no other row of the call has its
// sequence (checked by scanning the call's sequences when it has at most
// kSimpleScan rows) and its valid entries are distinct positions (an LDS bitmap of
// positions 0..t): then each of its keys is selected once in the call, and the row
// adds into dk in place without touching the count table.  Any other row counts
// the selections of each of its keys, gives a key its accumulator at its second
// selection (and zeroes it), and raises the header's largest count, max |dI| and
// the query bound max_d sum_j |w_j q_j[d]|.
constexpr int kSimpleScan = 16384;

template <bool DENSE>
__global__ __launch_bounds__(BT) void bwd_count_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ q_scale,
    const float* __restrict__ w, const int32_t* __restrict__ indices,
    const float* __restrict__ dscores, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_pos, int R, int B, int N, int max_pos, int topk, int64_t ld,
    BwdWs ws) {
  __shared__ uint32_t seen[kTopkMaxPositions / 32];  // (t < max_pos + 1 <= 131072)
  __shared__ float part_s[BT / 32][ID];
  __shared__ uint32_t red[BT / 64];
  __shared__ int shared_s;
  const int r = blockIdx.x, tid = threadIdx.x;
  const int b = row_seq[r], t = row_pos[r];
  if (!bwd_row_ok(b, t, B, N, max_pos)) return;
  const int nent = DENSE ? t + 1 : topk;
  // another row on this sequence, or (sparse) a position listed twice
  if (tid == 0) shared_s = R > kSimpleScan ? 1 : 0;
  for (int i = tid; i < (t + 32) / 32; i += BT) seen[i] = 0u;
  __syncthreads();
  if (R <= kSimpleScan) {
    bool other = false;
    for (int i = tid; i < R; i += BT) other |= i != r && row_seq[i] == b;
    if (other) shared_s = 1;  // (every writer stores 1)
  }
  if (!DENSE) {
    bool dup = false;
    for (int i = tid; i < nent; i += BT) {
      const int p = indices[(size_t)r * topk + i];
      if (p >= 0 && p <= t) {
        const uint32_t bit = 1u << (p & 31);
        dup |= (atomicOr(&seen[p >> 5], bit) & bit) != 0u;
      }
    }
    if (dup) shared_s = 1;
  }
  __syncthreads();
  const bool simple = shared_s == 0;
  if (tid == 0) ws.rowflag[r] = simple ? 1 : 0;
  if (simple) return;
  uint32_t gbits = 0, cmax = 0;  // (non-negative floats order as their bits)
  for (int i = tid; i < nent; i += BT) {
    const int p = DENSE ? i : indices[(size_t)r * topk + i];
    if (p < 0 || p > t) continue;
    const float g = DENSE ? dscores[(size_t)r * ld + p] : dscores[(size_t)r * topk + i];
    gbits = max(gbits, __float_as_uint(fabsf(g)));
    const int key = b * (max_pos + 1) + p;
    const int c = atomicAdd(&ws.cnt[key], 1);
    if (c == 1) {  // the key's second selection
      const int sl = atomicAdd(&ws.hdr[0], 1);
      if (sl < ws.cap) {
        ws.slotkey[sl] = key;
        longlong2* a = reinterpret_cast<longlong2*>(ws.acc + (size_t)sl * ID);
#pragma unroll 8
        for (int d = 0; d < ID / 2; ++d) a[d] = make_longlong2(0, 0);
        ws.slot[key] = sl;
      } else {
        ws.slot[key] = -1;
      }
    }
    cmax = max(cmax, (uint32_t)c + 1);
  }
  const auto umax = [](uint32_t x, uint32_t y) { return max(x, y); };
  gbits = wave_reduce_bits(gbits, umax);
  cmax = wave_reduce_bits(cmax, umax);
  if (lane_id() == 0) {
    if (gbits) atomicMax(reinterpret_cast<unsigned int*>(&ws.hdr[1]), gbits);
    if (cmax) atomicMax(&ws.hdr[2], (int)cmax);
  }
  // max_d sum_j |w_j q_scale_j| |e4m3(q_j[d])|: thread = 4 dims x 8 heads, then over
  // the 8 head groups through LDS
  {
    const int d4 = tid & 31, hg = tid >> 5;
    float acc4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int j = 8 * hg + jj;
      const uint32_t word =
          *reinterpret_cast<const uint32_t*>(q_idx + ((size_t)r * IH + j) * ID + 4 * d4);
      const float f = fabsf(w[(size_t)r * IH + j] * q_scale[(size_t)r * IH + j]);
#pragma unroll
      for (int k = 0; k < 4; ++k) acc4[k] += f * fabsf(e4m3_value((word >> (8 * k)) & 0xffu));
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) part_s[hg][4 * d4 + k] = acc4[k];
  }
  __syncthreads();
  uint32_t sbits = 0;
  if (tid < ID) {
    float sd = 0.f;
#pragma unroll
    for (int hg = 0; hg < BT / 32; ++hg) sd += part_s[hg][tid];
    sbits = __float_as_uint(fabsf(sd));
  }
  sbits = wave_reduce_bits(sbits, umax);
  if (lane_id() == 0) red[tid >> 6] = sbits;
  __syncthreads();
  if (tid == 0) {
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < BT / 64; ++k) m = max(m, red[k]);
    atomicMax(reinterpret_cast<unsigned int*>(&ws.hdr[3]), m);
  }
}

constexpr int KRS = ID + 16;  // bytes per raw key row in LDS (padded against bank conflicts)
constexpr int KTS = BG + 8;   // bf16 per row of the transposed codes and coefficient tiles

// One group's entry (tid < 64): position (-1: padding or past t) and gradient.
// DENSE: the entries are every causal position 0..t (no index list), with dscores
// [R, ld] indexed by position (the dense warm-up loss's gradient).
template <bool DENSE>
__device__ __forceinline__ void bwd_entry(int e, int r, int t, int topk, int64_t ld,
                                          const int32_t* __restrict__ indices,
                                          const float* __restrict__ dscores, int& p, float& g) {
  const int pp = DENSE ? e : indices[(size_t)r * topk + e];
  const bool v = pp >= 0 && pp <= t;
  const float gr = DENSE ? (v ? dscores[(size_t)r * ld + pp] : 0.f) : dscores[(size_t)r * topk + e];
  p = v ? pp : -1;
  g = v ? gr : 0.f;
}

// fp8 (OCP e4m3) bytes 2h, 2h + 1 of w as a bf16 pair (exact: every e4m3 value is
// a bf16 value)
__device__ __forceinline__ uint32_t e4m3_pair_bf16(uint32_t w, bool h) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = h ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                       : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  return __builtin_bit_cast(uint32_t, v);
}

// x = hi + mid + lo with three bf16 values (hi and mid round to nearest; the
// remainder has at most 9 significant bits, so lo holds it to within 2^-25 |x|)
__device__ __forceinline__ void split3(float x, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
  hi = bf16_bits(x);
  const float r1 = x - __uint_as_float((uint32_t)hi << 16);
  mid = bf16_bits(r1);
  lo = bf16_bits(r1 - __uint_as_float((uint32_t)mid << 16));
}

template <bool DENSE>
__global__ __launch_bounds__(BT) void indexer_bwd_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ k_idx,
    const float* __restrict__ k_scale, const int32_t* __restrict__ indices,
    const float* __restrict__ dscores, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_pos, int B, int N, int max_pos, int topk, int64_t ld,
    int E, int G, float* __restrict__ dq, float* __restrict__ dw, float* __restrict__ dk,
    BwdWs ws) {
  // the group's key codes as bf16, dim-major (B operand of the dq product)
  __shared__ __attribute__((aligned(16))) uint16_t kT[ID][KTS];
  // coefficients in three bf16 parts: dI w m k_scale, head-major (A of dq), and
  // dI w m q_scale, key-major (A of dk)
  __shared__ __attribute__((aligned(16))) uint16_t cq3[3][IH][KTS];
  __shared__ __attribute__((aligned(16))) uint16_t ck3[3][BG][KTS];
  __shared__ __attribute__((aligned(16))) float dkt[BG][ID + 4];   // the group's dk terms
  __shared__ __attribute__((aligned(16))) uint8_t kraw[BG][KRS];   // the group's fp8 keys
  __shared__ float dwp[BT / 64][IH];
  __shared__ int pos_s[BG], pn_s[BG];
  __shared__ float g_s[BG], ks_s[BG];
  const int r = blockIdx.x / E, chunk = blockIdx.x - r * E, ebase = chunk * G * BG;
  const int b = row_seq[r], t = row_pos[r];
  if (!bwd_row_ok(b, t, B, N, max_pos)) return;
  if (DENSE && ebase > t) return;  // every position of this chunk is past the row
  const int tid = threadIdx.x, l = lane_id(), g = l >> 4, n = l & 15;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint8_t* kbase = k_idx + (size_t)b * N * ID;
  const float* sbase = k_scale + (size_t)b * N;
  const uint8_t* qr = q_idx + (size_t)r * IH * ID;
  double up = 0.0, down = 0.0;
  const bool fixed = bwd_scale(ws.hdr, up, down);
  const bool simple = ws.rowflag[r] != 0;  // each of the row's keys is selected once
  const int ke = tid >> 2, kc = tid & 3;  // the key and 32-byte piece this thread stages

  // the first group's entries
  int pe = -1, pe_n = -1;
  float ge = 0.f, ge_n = 0.f, kse = 0.f;
  if (tid < BG) {
    bwd_entry<DENSE>(ebase + tid, r, t, topk, ld, indices, dscores, pe, ge);
    pn_s[tid] = pe;
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
  // B operand of the dk product, kept for the block: query codes as bf16 for the
  // wave's dims 32 wv + 16 nt + n and heads 32 ks + 8 g .. + 7
  bf16x8 qb[2][2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint8_t* src = qr + (size_t)(32 * ks + 8 * g) * ID + 32 * wv + 16 * nt + n;
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w0 |= (uint32_t)src[(size_t)i * ID] << (8 * i);
        w1 |= (uint32_t)src[(size_t)(4 + i) * ID] << (8 * i);
      }
      const i32x4 v = {(int)e4m3_pair_bf16(w0, false), (int)e4m3_pair_bf16(w0, true),
                       (int)e4m3_pair_bf16(w1, false), (int)e4m3_pair_bf16(w1, true)};
      qb[nt][ks] = as_bf16x8(v);
    }
  __syncthreads();
  i32x4 kr0 = {0, 0, 0, 0}, kr1 = {0, 0, 0, 0};
  {
    const int p = pn_s[ke];
    if (p >= 0) {
      const i32x4* kp = reinterpret_cast<const i32x4*>(kbase + (size_t)p * ID + 32 * kc);
      kr0 = kp[0];
      kr1 = kp[1];
    }
    if (tid < BG && pe >= 0) kse = sbase[pe];
  }
  float dwacc = 0.f;  // head tid (tid < 64), over the block's groups
  // dq over the block's groups: lane holds dq[16 mt + 4 g + v][32 wv + 16 nt + n]
  f32x4 dqa[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) dqa[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int gi = 0; gi < G; ++gi) {
    const int e0 = ebase + gi * BG;
    if (DENSE && e0 > t) break;  // (uniform over the block)
    const bool more = gi + 1 < G && !(DENSE && e0 + BG > t);
    __syncthreads();  // the previous group's LDS reads are done
    if (tid < BG) {
      pos_s[tid] = pe;
      g_s[tid] = ge;
      ks_s[tid] = kse;
      if (more) bwd_entry<DENSE>(e0 + BG + tid, r, t, topk, ld, indices, dscores, pe_n, ge_n);
    }
    *reinterpret_cast<i32x4*>(&kraw[ke][32 * kc]) = kr0;
    *reinterpret_cast<i32x4*>(&kraw[ke][32 * kc + 16]) = kr1;
    {  // this thread's 32 codes of key ke, as bf16, into the dim-major tile
      const uint32_t wd[8] = {(uint32_t)kr0[0], (uint32_t)kr0[1], (uint32_t)kr0[2], (uint32_t)kr0[3],
                              (uint32_t)kr1[0], (uint32_t)kr1[1], (uint32_t)kr1[2], (uint32_t)kr1[3]};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint32_t lo = e4m3_pair_bf16(wd[q], false), hi = e4m3_pair_bf16(wd[q], true);
        kT[32 * kc + 4 * q + 0][ke] = (uint16_t)lo;
        kT[32 * kc + 4 * q + 1][ke] = (uint16_t)(lo >> 16);
        kT[32 * kc + 4 * q + 2][ke] = (uint16_t)hi;
        kT[32 * kc + 4 * q + 3][ke] = (uint16_t)(hi >> 16);
      }
    }
    __syncthreads();
    // the dk rows of the wave's 16 keys, for the keys selected once in the call, and
    // the selection counts and accumulators of the others; in flight during the
    // dots and products
    int cnt_l = 1, slot_l = -1;
    float x0[16], x1[16];
    {
      const int pl = pos_s[16 * wv + (l & 15)];
      if (!simple && l < 16 && pl >= 0) {
        const int key = b * (max_pos + 1) + pl;
        cnt_l = ws.cnt[key];
        slot_l = ws.slot[key];
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) {  // (read for every valid key; used when selected once)
        const int p = pos_s[16 * wv + k];
        x0[k] = x1[k] = 0.f;
        if (p >= 0) {
          const float* src = dk + ((size_t)b * N + p) * ID;
          x0[k] = src[l];
          x1[k] = src[64 + l];
        }
      }
    }
    // fp8 dots of the 64 heads with this wave's 16 keys (the forward's arithmetic),
    // the coefficients in three bf16 parts, and dw
    {
      const int e = 16 * wv + n;  // this lane's key
      const i32x4 a0 = *reinterpret_cast<const i32x4*>(&kraw[e][32 * g]);
      const i32x4 a1 = *reinterpret_cast<const i32x4*>(&kraw[e][32 * g + 16]);
      const i32x8 kb = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
      const float gev = g_s[e], kse_e = ks_s[e];
      float dwl[16];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4 d8 = mfma_fp8_16x16x128(qa[mt], kb, f32x4{0.f, 0.f, 0.f, 0.f});
        uint16_t kh[4], km[4], kl[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int j = 16 * mt + 4 * g + v;
          const bool pos = d8[v] > 0.f;
          const float c = pos ? gev * wjj[4 * mt + v] : 0.f;
          uint16_t h, m, lo;
          split3(c * kse_e, h, m, lo);
          cq3[0][j][e] = h;
          cq3[1][j][e] = m;
          cq3[2][j][e] = lo;
          split3(c * qsj[4 * mt + v], kh[v], km[v], kl[v]);
          dwl[4 * mt + v] = pos ? gev * d8[v] * qsj[4 * mt + v] * kse_e : 0.f;
        }
        const int j0 = 16 * mt + 4 * g;
        *reinterpret_cast<uint2*>(&ck3[0][e][j0]) =
            make_uint2(kh[0] | ((uint32_t)kh[1] << 16), kh[2] | ((uint32_t)kh[3] << 16));
        *reinterpret_cast<uint2*>(&ck3[1][e][j0]) =
            make_uint2(km[0] | ((uint32_t)km[1] << 16), km[2] | ((uint32_t)km[3] << 16));
        *reinterpret_cast<uint2*>(&ck3[2][e][j0]) =
            make_uint2(kl[0] | ((uint32_t)kl[1] << 16), kl[2] | ((uint32_t)kl[3] << 16));
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
    if (tid < BG) pn_s[tid] = pe_n;
    __syncthreads();
    if (tid < IH) dwacc += dwp[0][tid] + dwp[1][tid] + dwp[2][tid] + dwp[3][tid];
    // the next group's key bytes and scales, in flight during the products
    if (more) {
      const int p = pn_s[ke];
      kr0 = i32x4{0, 0, 0, 0};
      kr1 = i32x4{0, 0, 0, 0};
      if (p >= 0) {
        const i32x4* kp = reinterpret_cast<const i32x4*>(kbase + (size_t)p * ID + 32 * kc);
        kr0 = kp[0];
        kr1 = kp[1];
      }
      if (tid < BG) kse = pe_n >= 0 ? sbase[pe_n] : 0.f;
    }
    // dq[j][d] += sum_e (dI w m k_scale)[j][e] code_k[e][d] and
    // dk terms [e][d] = sum_j (dI w m q_scale)[e][j] code_q[j][d], on the bf16 MFMA
    // with each coefficient as three exact parts: the wave's dims 32 wv .. + 31
    f32x4 dka[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) dka[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 kb2[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        kb2[nt] = as_bf16x8(*reinterpret_cast<const i32x4*>(&kT[32 * wv + 16 * nt + n][32 * ks + 8 * g]));
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int sp = 0; sp < 3; ++sp) {
          const bf16x8 aq =
              as_bf16x8(*reinterpret_cast<const i32x4*>(&cq3[sp][16 * mt + n][32 * ks + 8 * g]));
          const bf16x8 ak =
              as_bf16x8(*reinterpret_cast<const i32x4*>(&ck3[sp][16 * mt + n][32 * ks + 8 * g]));
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            dqa[mt][nt] = mfma_bf16_16x16x32(aq, kb2[nt], dqa[mt][nt]);
            dka[mt][nt] = mfma_bf16_16x16x32(ak, qb[nt][ks], dka[mt][nt]);
          }
        }
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int v = 0; v < 4; ++v) dkt[16 * mt + 4 * g + v][32 * wv + 16 * nt + n] = dka[mt][nt][v];
    __syncthreads();
    // into dk: wave wv takes keys 16 wv .. 16 wv + 15, lane = dims l and 64 + l, so
    // that every load, store or atomic instruction covers whole cache lines (the
    // rows of keys selected once were read after the group's positions came in)
    {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int e = 16 * wv + k, p = pos_s[e];
        if (p < 0) continue;
        const int c = __builtin_amdgcn_readlane(cnt_l, k);
        const int sl = __builtin_amdgcn_readlane(slot_l, k);
        const float v0 = dkt[e][l], v1 = dkt[e][64 + l];
        float* dst = dk + ((size_t)b * N + p) * ID;
        if (c == 1) {  // the key's only selection in the call: add in place
          dst[l] = x0[k] + v0;
          dst[64 + l] = x1[k] + v1;
        } else if (fixed && sl >= 0) {
          unsigned long long* ac = reinterpret_cast<unsigned long long*>(ws.acc + (size_t)sl * ID);
          if (v0 != 0.f) atomicAdd(&ac[l], (unsigned long long)__double2ll_rn((double)v0 * up));
          if (v1 != 0.f) atomicAdd(&ac[64 + l], (unsigned long long)__double2ll_rn((double)v1 * up));
        } else {
          if (v0 != 0.f) atomicAdd(&dst[l], v0);
          if (v1 != 0.f) atomicAdd(&dst[64 + l], v1);
        }
      }
    }
    pe = pe_n;
    ge = ge_n;
  }
  (void)down;
  // dq and dw: into the row's outputs when the block is the row's only one, else
  // into the chunk's own partial slot (same layout)
  float* dqo = E == 1 ? dq + (size_t)r * IH * ID : ws.part + ((size_t)r * E + chunk) * kPartLen;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float* o = dqo + (size_t)(16 * mt + 4 * g + v) * ID + 32 * wv + 16 * nt + n;
        *o = E == 1 ? *o + dqa[mt][nt][v] : dqa[mt][nt][v];
      }
  if (tid < IH) {
    if (E == 1)
      dw[(size_t)r * IH + tid] += dwacc;
    else
      dqo[IH * ID + tid] = dwacc;
  }
}

// dq and dw of each row += its chunks' partial sums, added in chunk order.  Block
// (row, piece): 256 float4 words of the kPartLen / 4 of a slot.
template <bool DENSE>
__global__ __launch_bounds__(BT) void bwd_reduce_kernel(
    const int32_t* __restrict__ row_seq, const int32_t* __restrict__ row_pos, int B, int N,
    int max_pos, int E, int G, const float* __restrict__ part, float* __restrict__ dq,
    float* __restrict__ dw) {
  constexpr int NP = (kPartLen / 4 + BT - 1) / BT;
  const int r = blockIdx.x / NP, i4 = (blockIdx.x - r * NP) * BT + threadIdx.x;
  const int b = row_seq[r], t = row_pos[r];
  if (!bwd_row_ok(b, t, B, N, max_pos) || i4 >= kPartLen / 4) return;
  // the chunks that ran (a dense row's chunks past t did not)
  const int nc = DENSE ? min(E, t / (G * BG) + 1) : E;
  const float4* pp = reinterpret_cast<const float4*>(part + (size_t)r * E * kPartLen) + i4;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c = 0; c < nc; ++c) {
    const float4 v = pp[(size_t)c * (kPartLen / 4)];
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  float4* dst = 4 * i4 < IH * ID
                    ? reinterpret_cast<float4*>(dq + (size_t)r * IH * ID) + i4
                    : reinterpret_cast<float4*>(dw + (size_t)r * IH) + (i4 - IH * ID / 4);
  float4 x = *dst;
  x.x += s.x; x.y += s.y; x.z += s.z; x.w += s.w;
  *dst = x;
}

// dk of each key selected more than once += its fixed-point sum x 2^-s.  64 threads
// per accumulator (2 dims each), 4 accumulators per block.
__global__ __launch_bounds__(BT) void bwd_finalize_kernel(int N, int max_pos, BwdWs ws,
                                                          float* __restrict__ dk) {
  const int s = blockIdx.x * (BT / 64) + (threadIdx.x >> 6), d = 2 * lane_id();
  if (s >= min(ws.hdr[0], ws.cap)) return;
  double up = 0.0, down = 0.0;
  if (!bwd_scale(ws.hdr, up, down)) return;  // these keys went to fp32 atomics
  const int key = ws.slotkey[s];
  const int b = key / (max_pos + 1), p = key - b * (max_pos + 1);
  const longlong2 v = *reinterpret_cast<const longlong2*>(ws.acc + (size_t)s * ID + d);
  float2* dst = reinterpret_cast<float2*>(dk + ((size_t)b * N + p) * ID + d);
  float2 x = *dst;
  x.x += (float)((double)v.x * down);
  x.y += (float)((double)v.y * down);
  *dst = x;
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

namespace {

// Workspace layout of the backward; the accumulators take what the caller's bytes
// leave after the fixed pieces, up to the most the call's shape can use.
struct BwdLayout {
  size_t rowflag, cnt, slot, part, slotkey, acc, base;
  int E, G;
  int64_t cap_max;  // keys that the call's shape lets be selected twice or more
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

BwdLayout bwd_layout(const dsa_rows& rows, int topk, bool dense) {
  BwdLayout L{};
  const int64_t R = rows.num_rows;
  const int64_t nkeys = (int64_t)rows.num_seqs * (rows.max_pos + 1);
  const int64_t epr = dense ? (int64_t)rows.max_pos + 1 : topk;  // entries per row
  const int ngroups = (int)((epr + BG - 1) / BG);
  int E = 1;
  while (E < ngroups && R * E < kBwdTargetBlocks) E <<= 1;
  L.E = E < ngroups ? E : ngroups;
  L.G = (ngroups + L.E - 1) / L.E;
  L.cap_max = std::min(nkeys, R * epr / 2);
  size_t off = 256;  // header
  L.rowflag = off;
  off += align256((size_t)R * sizeof(int));
  L.cnt = off;
  off += align256((size_t)((nkeys + 3) / 4) * 16);
  L.slot = off;
  off += align256((size_t)nkeys * sizeof(int));
  L.part = off;
  if (L.E > 1) off += align256((size_t)R * L.E * kPartLen * sizeof(float));
  L.base = off;
  return L;
}

// accumulators that ws_bytes holds beside the fixed pieces
int64_t bwd_cap(const BwdLayout& L, size_t ws_bytes) {
  if (ws_bytes < L.base + 256) return 0;
  const int64_t c = (int64_t)((ws_bytes - L.base - 256) / (ID * sizeof(long long) + sizeof(int)));
  return std::min(c, L.cap_max);
}

template <bool DENSE>
hipError_t launch_bwd(const dsa_rows& rows, const uint8_t* q_idx, const float* q_scale,
                      const float* w, const uint8_t* k_idx, const float* k_scale,
                      const int32_t* indices, const float* dscores, int64_t ld, float* dq,
                      float* dw, float* dk, void* workspace, size_t ws_bytes,
                      hipStream_t stream) {
  const int R = rows.num_rows;
  if (R == 0) return hipSuccess;
  const BwdLayout L = bwd_layout(rows, kTopk, DENSE);
  const int64_t cap = bwd_cap(L, ws_bytes);
  char* base = static_cast<char*>(workspace);
  BwdWs ws;
  ws.hdr = reinterpret_cast<int*>(base);
  ws.rowflag = reinterpret_cast<int*>(base + L.rowflag);
  ws.cnt = reinterpret_cast<int*>(base + L.cnt);
  ws.slot = reinterpret_cast<int*>(base + L.slot);
  ws.part = reinterpret_cast<float*>(base + L.part);
  ws.slotkey = reinterpret_cast<int*>(base + L.base);
  ws.acc = reinterpret_cast<long long*>(base + L.base + align256((size_t)cap * sizeof(int)));
  ws.cap = (int)cap;
  const int64_t n4 = ((int64_t)rows.num_seqs * (rows.max_pos + 1) + 3) / 4;
  const int cblocks = (int)std::max<int64_t>(1, std::min<int64_t>((n4 + BT - 1) / BT, 2048));
  hipLaunchKernelGGL(bwd_clear_kernel, dim3(cblocks), dim3(BT), 0, stream, ws.hdr,
                     reinterpret_cast<int4*>(ws.cnt), n4);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(bwd_count_kernel<DENSE>, dim3(R), dim3(BT), 0, stream, q_idx, q_scale, w,
                     indices, dscores, rows.row_seq, rows.row_pos, R, rows.num_seqs, rows.max_ctx,
                     rows.max_pos, kTopk, ld, ws);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(indexer_bwd_kernel<DENSE>, dim3((unsigned)((int64_t)R * L.E)), dim3(BT), 0,
                     stream, q_idx, q_scale, w, k_idx, k_scale, indices, dscores, rows.row_seq,
                     rows.row_pos, rows.num_seqs, rows.max_ctx, rows.max_pos, kTopk, ld, L.E, L.G,
                     dq, dw, dk, ws);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (L.E > 1) {
    constexpr int NP = (kPartLen / 4 + BT - 1) / BT;
    hipLaunchKernelGGL(bwd_reduce_kernel<DENSE>, dim3((unsigned)((int64_t)R * NP)), dim3(BT), 0,
                       stream, rows.row_seq, rows.row_pos, rows.num_seqs, rows.max_ctx,
                       rows.max_pos, L.E, L.G, ws.part, dq, dw);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (cap > 0) {
    const int fblocks = (int)std::min<int64_t>((cap + 3) / 4, 1024);
    hipLaunchKernelGGL(bwd_finalize_kernel, dim3(fblocks), dim3(BT), 0, stream, rows.max_ctx,
                       rows.max_pos, ws, dk);
    err = hipGetLastError();
  }
  return err;
}

}  // namespace

size_t indexer_backward_workspace_bytes(const dsa_rows& rows, int topk, bool dense,
                                        int64_t shared_keys) {
  const BwdLayout L = bwd_layout(rows, topk, dense);
  const int64_t cap = shared_keys < 0 ? L.cap_max : std::min(shared_keys, L.cap_max);
  return L.base + align256((size_t)cap * sizeof(int)) + (size_t)cap * ID * sizeof(long long);
}

hipError_t launch_indexer_backward(const dsa_rows& rows, const uint8_t* q_idx,
                                   const float* q_scale, const float* w, const uint8_t* k_idx,
                                   const float* k_scale, const int32_t* indices,
                                   const float* dscores, float* dq, float* dw, float* dk,
                                   void* workspace, size_t ws_bytes, hipStream_t stream) {
  return launch_bwd<false>(rows, q_idx, q_scale, w, k_idx, k_scale, indices, dscores, 0, dq, dw,
                           dk, workspace, ws_bytes, stream);
}

hipError_t launch_indexer_backward_dense(const dsa_rows& rows, const uint8_t* q_idx,
                                         const float* q_scale, const float* w, const uint8_t* k_idx,
                                         const float* k_scale, const float* dscores, int64_t ld,
                                         float* dq, float* dw, float* dk, void* workspace,
                                         size_t ws_bytes, hipStream_t stream) {
  return launch_bwd<true>(rows, q_idx, q_scale, w, k_idx, k_scale, nullptr, dscores, ld, dq, dw,
                          dk, workspace, ws_bytes, stream);
}

}  // namespace dsa
