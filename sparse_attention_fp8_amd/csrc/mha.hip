// Masked MHA mode of the sparse attention, for short prefill.
//
// DeepSeek-V3.2-Exp paper, section 3 ("inference cost"): for short-sequence
// prefill a masked MHA mode simulates DSA; Appendix A, Fig. 4: MLA's MHA mode
// (training and prefill) and MQA mode (decoding).  In MHA mode every head has its
// own key and value, decompressed from the shared latent entry c_s:
//   k[h,s] = [W_UK[h] c_s[:512] ; c_s[512:576]]     (128 + 64 dims)
//   v[h,s] = W_UV[h] c_s[:512]                       (128 dims)
// and query row r attends, per head, over the positions the indexer selected:
//   o[r,h] = sum_{s in S_r} softmax_s(scale q[r,h] . k[h,s]) v[h,s]
// which equals W_UV[h] times the MQA-mode output with the absorbed query.
//
// Three kernels: mha_decompress_kernel (bf16 MFMA GEMM of the latent rows with the
// stacked W_UK / W_UV; keys stored [s][h][128], values transposed [h][128][s]),
// mha_mask_kernel (the selection as one bit per causal position), and
// mha_attn_kernel (flash attention per head over 32-key stages with the mask).
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int H = kHeads;    // 128
constexpr int DL = kVDim;    // 512 latent dims
constexpr int DR = kQkDim - kVDim;  // 64 rope dims
constexpr int DH = kMhaHeadDim;     // 128 nope / value dims per head
constexpr int DQ = DH + DR;         // 192 query dims per head
constexpr int KCOLS = H * DH;       // 16384 key columns, then as many value columns

// ---------------------------------------------------------------------------
// Decompression: y[s, :] = W c_s with W = [W_UK; W_UV] (32768 x 512).  Block =
// 4 waves, 64 positions x 256 columns; wave w owns columns [64 w, 64 w + 64) for
// all 64 positions (4 x 4 MFMA tiles).  Per contraction step of 32 the block
// stages the A tile (64 positions x 32) and the B tile (256 weight rows x 32) in
// LDS (rows padded to 80 bytes, so a tile column's 16 rows hit distinct banks),
// double-buffered: the next step's tiles are loaded into registers while this
// step's MFMAs run, then stored to the other buffer, one barrier per step.
// ---------------------------------------------------------------------------
constexpr int DKS = 32;          // contraction step
constexpr int DPAD = DKS + 8;    // padded tile row (bf16)
constexpr int DPOS = 64;         // positions per block
constexpr int DCOL = 256;        // columns per block
constexpr int DCH = (DPOS + DCOL) * (DKS / 8);  // 16-byte chunks per step (1280)
static_assert(DCH % 256 == 0, "whole chunks per thread");

__global__ __launch_bounds__(256) void mha_decompress_kernel(
    const uint16_t* __restrict__ latent, const uint16_t* __restrict__ w_uk,
    const uint16_t* __restrict__ w_uv, int N, int Lc, int L, uint16_t* __restrict__ kout,
    uint16_t* __restrict__ vtout) {
  // positions [0, Lc) hold entries; the rest of the padded length L repeats the last
  // one, so every position of the outputs is finite
  __shared__ __attribute__((aligned(16))) uint16_t at[2][DPOS][DPAD];
  __shared__ __attribute__((aligned(16))) uint16_t bt[2][DCOL][DPAD];
  const int b = blockIdx.z;
  const int s0 = blockIdx.y * DPOS;
  const int c0 = blockIdx.x * DCOL;
  const int tid = threadIdx.x, l = lane_id(), wv = tid >> 6, g = l >> 4, n = l & 15;
  const uint16_t* lat = latent + (size_t)b * N * kQkDim;
  // this thread's chunks of a step: chunk c = tid + 256 j is row c / 4 (A rows
  // first, then B rows), dims 8 (c % 4) .. +8 of the step
  constexpr int CPT = DCH / 256;  // 5
  const uint16_t* src[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int c = tid + 256 * j, row = c >> 2, d8 = c & 3;
    if (row < DPOS) {
      src[j] = lat + (size_t)min(s0 + row, Lc - 1) * kQkDim + 8 * d8;
    } else {
      const int col = c0 + row - DPOS;
      src[j] = (col < KCOLS ? w_uk + (size_t)col * DL : w_uv + (size_t)(col - KCOLS) * DL) + 8 * d8;
    }
  }
  i32x4 pf[CPT];
  auto fetch = [&](int ks) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) pf[j] = *reinterpret_cast<const i32x4*>(src[j] + DKS * ks);
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = tid + 256 * j, row = c >> 2, d8 = c & 3;
      uint16_t* dst = row < DPOS ? &at[buf][row][8 * d8] : &bt[buf][row - DPOS][8 * d8];
      *reinterpret_cast<i32x4*>(dst) = pf[j];
    }
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  fetch(0);
  stash(0);
  constexpr int NKS = DL / DKS;  // 16
  for (int ks = 0; ks < NKS; ++ks) {
    const int cur = ks & 1;
    __syncthreads();  // buffer cur is complete; every wave is done with buffer cur ^ 1
    if (ks + 1 < NKS) fetch(ks + 1);
    bf16x8 a[4], bb[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      a[mt] = as_bf16x8(*reinterpret_cast<const i32x4*>(&at[cur][16 * mt + n][8 * g]));
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      bb[nt] = as_bf16x8(*reinterpret_cast<const i32x4*>(&bt[cur][64 * wv + 16 * nt + n][8 * g]));
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma_bf16_16x16x32(a[mt], bb[nt], acc[mt][nt]);
    if (ks + 1 < NKS) stash(cur ^ 1);
  }
  // lane holds positions s0 + 16 mt + 4 g + v of column c0 + 64 wv + 16 nt + n
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int col = c0 + 64 * wv + 16 * nt + n;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int sp = s0 + 16 * mt + 4 * g;  // L is a multiple of 64: all four exist
      if (col < KCOLS) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          kout[((size_t)b * L + sp + v) * KCOLS + col] = bf16_bits(acc[mt][nt][v]);
      } else {  // four consecutive positions of one value row
        uint16_t* dst = vtout + ((size_t)b * KCOLS + (col - KCOLS)) * L + sp;
        *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(acc[mt][nt][0], acc[mt][nt][1]),
                                                    pack_bf16x2(acc[mt][nt][2], acc[mt][nt][3]));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Selection mask: bit s of row r (words [R, L / 32]) is set when s is one of the
// row's selected positions (0 <= s <= t).  One block per row, built in LDS.
// ---------------------------------------------------------------------------
constexpr int kMaxMhaLen = 16384;

__global__ __launch_bounds__(256) void mha_mask_kernel(const int32_t* __restrict__ indices,
                                                       const int32_t* __restrict__ row_pos,
                                                       int topk, int L, uint32_t* __restrict__ mask) {
  __shared__ uint32_t words[kMaxMhaLen / 32];
  const int r = blockIdx.x, W = L / 32;
  const int t = row_pos[r];
  for (int i = threadIdx.x; i < W; i += 256) words[i] = 0u;
  __syncthreads();
  for (int i = threadIdx.x; i < topk; i += 256) {
    const int p = indices[(size_t)r * topk + i];
    if (p >= 0 && p <= t && p < L) atomicOr(&words[p >> 5], 1u << (p & 31));
  }
  __syncthreads();
  for (int i = threadIdx.x; i < W; i += 256) mask[(size_t)r * W + i] = words[i];
}

// ---------------------------------------------------------------------------
// Attention: block = (head h, 128 query rows), 8 waves of 16 rows.  Per stage of
// 32 keys the block stages the keys (32 x 192: decompressed nope part + the
// entries' rope part) and the transposed values (128 x 32) in LDS.  Each wave
// forms S^T tiles (keys x rows), so a lane holds 8 keys of one row: exactly the
// B operand (P^T) of the O^T = V^T P^T product, whose A operand (V^T) is read from
// the transposed value tile in the same key order.  Online softmax in the exp2
// domain; masked keys get -inf.
// ---------------------------------------------------------------------------
// Reductions over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one row's four key
// groups): v_permlane16_swap and v_permlane32_swap pair each lane with its partner
// in VALU, without the LDS round trip of a shuffle.
__device__ __forceinline__ float max4g(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum4g(float v) {
  // both lanes of a pair add the same two values in the same order
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

constexpr int AW = 8;            // waves
constexpr int RT = 2;            // 16-row tiles per wave
constexpr int AR = 16 * RT * AW; // rows per block (256)
constexpr int AKS = 64;          // keys per stage
constexpr int KST = DQ + 8;      // key tile row stride (bf16), padded
constexpr int VST = AKS + 8;     // value tile row stride (bf16), padded

// Position of key k (0..31 within a 32-key half) in a value row of the tile: the
// keys 16 a + 4 g + v that lane group g holds for the value product (a, v = 0..3)
// sit together at 8 g + 4 a + v, so a lane's A operand is one 16-byte read.
__device__ __forceinline__ int vperm(int k) { return 8 * ((k >> 2) & 3) + 4 * (k >> 4) + (k & 3); }

__global__ __launch_bounds__(AW * 64) void mha_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ latent,
    const uint16_t* __restrict__ kdec, const uint16_t* __restrict__ vtdec,
    const uint32_t* __restrict__ mask, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_pos, int R, int B, int N, int Lc, int L, float scale_log2,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) uint16_t kt[AKS][KST];
  __shared__ __attribute__((aligned(16))) uint16_t vt[DH][VST];
  __shared__ int tmax_s[AW];
  __shared__ int seq_s[AW];
  // Block order: XCD x (block id mod 8) runs heads x, x + 8, ... one after the
  // other, each head's row blocks longest first, so the row blocks that stream one
  // head's keys and values run together on one L2.
  const int nrb = (R + AR - 1) / AR;
  const int xcd = blockIdx.x & 7, within = blockIdx.x >> 3;
  const int h = 8 * (within / nrb) + xcd;
  const int r0 = (nrb - 1 - within % nrb) * AR;
  const int tid = threadIdx.x, l = lane_id(), g = l >> 4, n = l & 15;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int W = L / 32;

  // this lane's rows (B operand column n of the S^T tiles of tile i) and sequences
  int rr[RT], bb[RT], tt[RT];
  bool valid[RT];
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    rr[i] = r0 + 16 * (RT * wv + i) + n;
    const bool rv = rr[i] < R;
    bb[i] = rv ? row_seq[rr[i]] : -1;
    tt[i] = rv ? row_pos[rr[i]] : -1;
    valid[i] = rv && bb[i] >= 0 && bb[i] < B && tt[i] >= 0 && tt[i] < Lc;
  }

  // One pass over the keys per distinct sequence among the block's rows, in
  // ascending sequence order: a single pass when the rows are grouped by sequence.
  int bdone = -1;
  for (;;) {
    // the next sequence: the smallest above bdone among the block's valid rows
    int bn = INT_MAX;
#pragma unroll
    for (int i = 0; i < RT; ++i)
      if (valid[i] && bb[i] > bdone) bn = min(bn, bb[i]);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) bn = min(bn, __shfl_xor(bn, o));
    if (l == 0) seq_s[wv] = bn;
    __syncthreads();
    int bseq = INT_MAX;
#pragma unroll
    for (int i = 0; i < AW; ++i) bseq = min(bseq, seq_s[i]);
    if (bseq == INT_MAX) break;  // the same for every thread of the block
    bdone = bseq;
    bool ok[RT];
    int tw = -1;
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      ok[i] = valid[i] && bb[i] == bseq;
      if (ok[i]) tw = max(tw, tt[i]);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) tw = max(tw, __shfl_xor(tw, o));
    if (l == 0) tmax_s[wv] = tw;
    __syncthreads();
    int tmax = -1;
#pragma unroll
    for (int i = 0; i < AW; ++i) tmax = max(tmax, tmax_s[i]);
    const uint16_t* kseq = kdec + (size_t)bseq * L * KCOLS + (size_t)h * DH;
    const uint16_t* vseq = vtdec + ((size_t)bseq * KCOLS + (size_t)h * DH) * L;
    const uint16_t* lseq = latent + (size_t)bseq * N * kQkDim;
    // queries of this lane's rows, contraction step s: dims [32 s + 8 g, +8)
    i32x4 qr[RT][DQ / 32];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const uint16_t* qp = q + ((size_t)(rr[i] < R ? rr[i] : 0) * H + h) * DQ + 8 * g;
#pragma unroll
      for (int s2 = 0; s2 < DQ / 32; ++s2) qr[i][s2] = *reinterpret_cast<const i32x4*>(qp + 32 * s2);
    }

    f32x4 acc[RT][DH / 16];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int d = 0; d < DH / 16; ++d) acc[i][d] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[RT], l_run[RT];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      m_run[i] = -INFINITY;
      l_run[i] = 0.f;
    }

    // Stage k0's tiles are fetched into registers one stage ahead (the loads are in
    // flight while the previous stage computes): key chunks tid + 64 AW j (64 keys x
    // 24 chunks), value chunks tid + 64 AW j (128 dims x 8 chunks of 8 keys), and the
    // two mask words of each of this lane's rows.
    constexpr int KCH = AKS * (DQ / 8) / (AW * 64), VCH = DH * (AKS / 8) / (AW * 64);
    static_assert(KCH * AW * 64 == AKS * (DQ / 8) && VCH * AW * 64 == DH * (AKS / 8), "chunk counts");
    i32x4 pf_k[KCH], pf_v[VCH];
    uint2 pf_m[RT];
    // a stage's two mask words of row r0 + 32 wv + 16 i + n, in 8-byte units (W is
    // even, and the stage's words start at an even word): a wave-uniform base plus
    // one lane offset shared by the tiles
    const uint2* mask2 = reinterpret_cast<const uint2*>(mask) + (size_t)(r0 + 32 * wv) * (W / 2);
    const int mlane = n * (W / 2);
    auto fetch = [&](int k0) {
#pragma unroll
      for (int j = 0; j < KCH; ++j) {
        const int c = tid + AW * 64 * j, e = c / (DQ / 8), d8 = c - e * (DQ / 8);
        const int s2 = min(k0 + e, L - 1);
        const uint16_t* src = d8 < DH / 8
                                  ? kseq + (size_t)s2 * KCOLS + 8 * d8
                                  : lseq + (size_t)min(s2, Lc - 1) * kQkDim + DL + 8 * (d8 - DH / 8);
        pf_k[j] = *reinterpret_cast<const i32x4*>(src);
      }
#pragma unroll
      for (int j = 0; j < VCH; ++j) {
        const int c = tid + AW * 64 * j, d = c / (AKS / 8), k8 = c - d * (AKS / 8);
        pf_v[j] = *reinterpret_cast<const i32x4*>(vseq + (size_t)d * L + k0 + 8 * k8);
      }
#pragma unroll
      for (int i = 0; i < RT; ++i)
        pf_m[i] = ok[i] ? mask2[16 * i * (W / 2) + (k0 >> 6) + mlane] : make_uint2(0u, 0u);
    };
    auto stash = [&]() {
#pragma unroll
      for (int j = 0; j < KCH; ++j) {
        const int c = tid + AW * 64 * j, e = c / (DQ / 8), d8 = c - e * (DQ / 8);
        *reinterpret_cast<i32x4*>(&kt[e][8 * d8]) = pf_k[j];
      }
#pragma unroll
      for (int j = 0; j < VCH; ++j) {
        const int c = tid + AW * 64 * j, d = c / (AKS / 8), k8 = c - d * (AKS / 8);
        const int base = 32 * (k8 >> 2) + vperm(8 * (k8 & 3));  // keys 8 k8 .. + 3
        *reinterpret_cast<uint2*>(&vt[d][base]) = make_uint2((uint32_t)pf_v[j][0], (uint32_t)pf_v[j][1]);
        *reinterpret_cast<uint2*>(&vt[d][base + 8]) = make_uint2((uint32_t)pf_v[j][2], (uint32_t)pf_v[j][3]);
      }
    };
    if (tmax >= 0) fetch(0);
    for (int k0 = 0; k0 <= tmax; k0 += AKS) {
      __syncthreads();  // previous stage's tile reads are done
      stash();
      uint32_t mw[RT][2];
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        mw[i][0] = pf_m[i].x;
        mw[i][1] = pf_m[i].y;
      }
      __syncthreads();
      if (k0 + AKS <= tmax) fetch(k0 + AKS);
      // the stage's two 32-key halves in turn: S^T = K Q^T (lane holds keys
      // 32 hf + 16 a + 4 g + v of row n of each tile), the online softmax, O^T += V^T P^T
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        f32x4 st[RT][2];
#pragma unroll
        for (int i = 0; i < RT; ++i) st[i][0] = st[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < DQ / 32; ++s2)
#pragma unroll
          for (int a2 = 0; a2 < 2; ++a2) {
            const bf16x8 ka = as_bf16x8(
                *reinterpret_cast<const i32x4*>(&kt[32 * hf + 16 * a2 + n][32 * s2 + 8 * g]));
#pragma unroll
            for (int i = 0; i < RT; ++i) st[i][a2] = mfma_bf16_16x16x32(ka, as_bf16x8(qr[i][s2]), st[i][a2]);
          }
        i32x4 pb[RT];
        float alpha[RT];
        bool rescale[RT];
#pragma unroll
        for (int i = 0; i < RT; ++i) {
          // masked raw scores; a wave whose rows see every key of the half skips
          // the mask tests
          float sm[8];
          const uint32_t m0 = mw[i][hf];
          if (__all(m0 == 0xffffffffu)) {
#pragma unroll
            for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
              for (int v = 0; v < 4; ++v) sm[4 * a2 + v] = st[i][a2][v];
          } else {
#pragma unroll
            for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
              for (int v = 0; v < 4; ++v)
                sm[4 * a2 + v] = ((m0 >> (16 * a2 + 4 * g + v)) & 1u) ? st[i][a2][v] : -INFINITY;
          }
          float mx = sm[0];
#pragma unroll
          for (int k = 1; k < 8; ++k) mx = fmaxf(mx, sm[k]);
          mx = max4g(mx);
          // running max in log2 units (the scale is positive, so it commutes with max);
          // exp2 of -inf is 0, which covers masked keys and the first stage
          const float m_new = fmaxf(m_run[i], mx * scale_log2);
          const float m_use = m_new == -INFINITY ? 0.f : m_new;
          alpha[i] = exp2f(m_run[i] - m_use);
          rescale[i] = !__all(alpha[i] == 1.f);
          float psum = 0.f;
          float pv[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            pv[k] = exp2f(fmaf(sm[k], scale_log2, -m_use));
            psum += pv[k];
          }
          psum = sum4g(psum);
          l_run[i] = l_run[i] * alpha[i] + psum;
          m_run[i] = m_new;
          pb[i] = i32x4{(int)pack_bf16x2(pv[0], pv[1]), (int)pack_bf16x2(pv[2], pv[3]),
                        (int)pack_bf16x2(pv[4], pv[5]), (int)pack_bf16x2(pv[6], pv[7])};
        }
#pragma unroll
        for (int i = 0; i < RT; ++i)
          if (rescale[i])  // (uniform over the wave)
#pragma unroll
            for (int dt = 0; dt < DH / 16; ++dt)
#pragma unroll
              for (int v = 0; v < 4; ++v) acc[i][dt][v] *= alpha[i];
#pragma unroll
        for (int dt = 0; dt < DH / 16; ++dt) {
          const bf16x8 va = as_bf16x8(*reinterpret_cast<const i32x4*>(&vt[16 * dt + n][32 * hf + 8 * g]));
#pragma unroll
          for (int i = 0; i < RT; ++i) acc[i][dt] = mfma_bf16_16x16x32(va, as_bf16x8(pb[i]), acc[i][dt]);
        }
      }
    }
    // lane holds dims 16 dt + 4 g + v of row n of each tile
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      if (!ok[i]) continue;
      const float inv = l_run[i] > 0.f ? 1.f / l_run[i] : 0.f;
      uint16_t* orow = out + ((size_t)rr[i] * H + h) * DH;
#pragma unroll
      for (int dt = 0; dt < DH / 16; ++dt)
        *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * g) =
            make_uint2(pack_bf16x2(acc[i][dt][0] * inv, acc[i][dt][1] * inv),
                       pack_bf16x2(acc[i][dt][2] * inv, acc[i][dt][3] * inv));
      if (lse != nullptr && g == 0)
        lse[(size_t)rr[i] * H + h] =
            l_run[i] > 0.f ? (m_run[i] + log2f(l_run[i])) * 0.69314718055994530942f : -INFINITY;
    }
    __syncthreads();  // the pass's LDS reads are done before the next pass writes
  }
}

}  // namespace

size_t mha_workspace_bytes(int num_rows, int num_seqs, int max_pos) {
  const size_t L = (size_t)(max_pos + 1 + 63) / 64 * 64;
  return (size_t)num_seqs * L * KCOLS * 2 * sizeof(uint16_t) + (size_t)num_rows * (L / 32) * 4;
}

hipError_t launch_mha(const dsa_rows& rows, const void* q, const void* latent, const void* w_uk,
                      const void* w_uv, const int32_t* indices, float softmax_scale, void* out,
                      float* lse, void* workspace, hipStream_t stream) {
  const int R = rows.num_rows, B = rows.num_seqs;
  if (R == 0) return hipSuccess;
  const int L = (rows.max_pos + 1 + 63) / 64 * 64;
  uint16_t* kdec = static_cast<uint16_t*>(workspace);
  uint16_t* vtdec = kdec + (size_t)B * L * KCOLS;
  uint32_t* mask = reinterpret_cast<uint32_t*>(vtdec + (size_t)B * L * KCOLS);
  const int Lc = rows.max_pos + 1 <= rows.max_ctx ? rows.max_pos + 1 : rows.max_ctx;
  hipLaunchKernelGGL(mha_decompress_kernel, dim3(2 * KCOLS / 256, L / 64, B), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(latent), static_cast<const uint16_t*>(w_uk),
                     static_cast<const uint16_t*>(w_uv), rows.max_ctx, Lc, L, kdec, vtdec);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(mha_mask_kernel, dim3(R), dim3(256), 0, stream, indices, rows.row_pos, kTopk,
                     L, mask);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  static_assert(H % 8 == 0, "heads spread evenly over the XCDs");
  hipLaunchKernelGGL(mha_attn_kernel, dim3(H * ((R + AR - 1) / AR)), dim3(AW * 64), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(latent), kdec,
                     vtdec, mask, rows.row_seq, rows.row_pos, R, B, rows.max_ctx, Lc, L,
                     softmax_scale * 1.44269504088896340736f, static_cast<uint16_t*>(out), lse);
  return hipGetLastError();
}

}  // namespace dsa
