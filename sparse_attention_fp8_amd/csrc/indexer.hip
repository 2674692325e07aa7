// Lightning-indexer scores on gfx950.
//
// I[t,s] = sum_j w[t,j] * ReLU(q[t,j] . k[s]) over positions s <= t
// (DeepSeek-V3.2-Exp paper, section 1 "Architecture", Eq. 1 and its prose; the
// paper notes the indexer has few heads and can run in FP8).
//
// FP8 path: q and k are e4m3fn codes with one positive fp32 scale per 128-wide
// vector.  Because a positive scale commutes with ReLU,
//   I[t,s] = k_scale[s] * sum_j (w[t,j] * q_scale[t,j]) * ReLU(q8[t,j] . k8[s]),
// so the fp8 dot products run unscaled on the 16x16x128 fp8 MFMA (d_I = 128 is
// exactly one contraction; the products are exact, and the instruction sums them
// in groups of 8 consecutive bytes, cutting each toward zero at 2^-13 of its
// group's largest product before the fp32 sum of the groups) and the scales,
// ReLU and the weighted head sum form the fp32 epilogue.
//
// MFMA tile: M = 16 indexer heads, N = 16 keys.  Four tiles cover the 64 heads, so
// each lane ends with 16 heads of one key and the head sum is 16 in-lane FMAs
// plus a 3-shuffle reduce-scatter across the four lane groups.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int IH = kIdxHeads;  // 64
constexpr int ID = kIdxDim;    // 128

__device__ __forceinline__ i32x8 load_frag32(const uint8_t* p) {
  const i32x4* v = reinterpret_cast<const i32x4*>(p);
  i32x4 a = v[0];
  i32x4 b = v[1];
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Lane partial of sum_j wq[j] * ReLU(dot[j, key]) over the lane's 16 heads for the
// 16-key tile `kb` (key = lane & 15).
__device__ __forceinline__ float head_partial(const i32x8 (&qa)[4], const float (&wq)[16],
                                              i32x8 kb) {
  // one accumulation chain per head tile, summed at the end (independent FMAs)
  float p[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const f32x4 acc = mfma_fp8_16x16x128(qa[mt], kb, f32x4{0.f, 0.f, 0.f, 0.f});
    p[mt] = wq[mt * 4] * relu_bits(acc[0]);
#pragma unroll
    for (int v = 1; v < 4; ++v) p[mt] = fmaf(wq[mt * 4 + v], relu_bits(acc[v]), p[mt]);
  }
  return (p[0] + p[1]) + (p[2] + p[3]);
}

// p_i is the lane's partial for key tile i (keys 16i..16i+15 of a 64-key group,
// key = lane & 15).  Returns the full head sum for key `lane` of the group:
// exchange halves across lanes l^32, then across l^16 (reduce-scatter).
__device__ __forceinline__ float reduce_groups(float p0, float p1, float p2, float p3) {
  const int l = lane_id();
  const bool hi = l >= 32;
  float keep0 = hi ? p2 : p0, keep1 = hi ? p3 : p1;
  const float send0 = hi ? p0 : p2, send1 = hi ? p1 : p3;
  keep0 += xor32(send0);
  keep1 += xor32(send1);
  const bool odd = (l >> 4) & 1;
  const float send = odd ? keep0 : keep1;
  const float keep = odd ? keep1 : keep0;
  return keep + xor16(send);
}

// The query row r as MFMA operands (lane: head 16 mt + (lane & 15), bytes
// [32 g, 32 g + 32)) and the lane's 16 products head weight x query scale.
__device__ __forceinline__ void load_query(const uint8_t* __restrict__ q_idx,
                                           const float* __restrict__ q_scale,
                                           const float* __restrict__ w, int r, i32x8 (&qa)[4],
                                           float (&wq)[16]) {
  const int l = lane_id(), g = l >> 4, n = l & 15;
  const uint8_t* qr = q_idx + (size_t)r * IH * ID;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) qa[mt] = load_frag32(qr + (16 * mt + n) * ID + 32 * g);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int h = 16 * mt + 4 * g + v;
      wq[mt * 4 + v] = w[(size_t)r * IH + h] * q_scale[(size_t)r * IH + h];
    }
}

// ---------------------------------------------------------------------------
// Prefill tiling: each wave owns RW consecutive query rows (their fp8 queries stay
// in registers) and walks the block's key range; every 16-key fragment feeds the
// MFMAs of all RW rows.  The four waves of a block read the same keys, which the
// L1/L2 serve.  Rows of a wave that belong to different sequences fall back to one
// row at a time.  Grid: row_tiles * key_blocks blocks.
// ---------------------------------------------------------------------------
template <int NR, bool PAGED>
__device__ __forceinline__ void prefill_rows(const uint8_t* __restrict__ q_idx,
                                             const float* __restrict__ q_scale,
                                             const float* __restrict__ w,
                                             const uint8_t* __restrict__ kc,
                                             const float* __restrict__ ksc, const int* rr,
                                             const int* tt, int kb0, int kend,
                                             float* __restrict__ scores, int64_t ld,
                                             const PageMap& pm, int b, float* mx, float* mn) {
  const int l = lane_id(), g = l >> 4, n = l & 15;
  i32x8 qa[NR][4];
  float wq[NR][16];
#pragma unroll
  for (int i = 0; i < NR; ++i) load_query(q_idx, q_scale, w, rr[i], qa[i], wq[i]);
  const int klast = kend - 1;
  // k is a multiple of 64 and a page holds at least 64 entries: one page per group
  auto load_group = [&](int k, i32x8(&kb)[4], float& ks) {
    if constexpr (PAGED) {
      const uint32_t row0 = paged_row(pm, b, k);
      const uint8_t* gb = kc + (size_t)row0 * ID;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        kb[kt] = load_frag32(gb + (size_t)(min(k + 16 * kt + n, klast) - k) * ID + 32 * g);
      ks = ksc[row0 + (min(k + l, klast) - k)];
    } else {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        kb[kt] = load_frag32(kc + (size_t)min(k + 16 * kt + n, klast) * ID + 32 * g);
      ks = ksc[min(k + l, klast)];
    }
  };
  auto compute = [&](int k, const i32x8(&kb)[4], float ks) {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      if (k > tt[i]) continue;  // wave-uniform
      const float p0 = head_partial(qa[i], wq[i], kb[0]);
      const float p1 = head_partial(qa[i], wq[i], kb[1]);
      const float p2 = head_partial(qa[i], wq[i], kb[2]);
      const float p3 = head_partial(qa[i], wq[i], kb[3]);
      const float s = reduce_groups(p0, p1, p2, p3) * ks;
      if (k + l <= tt[i]) {
        scores[(size_t)rr[i] * ld + k + l] = s;
        mx[i] = fmaxf(mx[i], s);  // a NaN score leaves both unchanged
        mn[i] = fminf(mn[i], s);
      }
    }
  };
  i32x8 ka[4], kb[4];
  float sa, sb;
  int k0 = kb0;
  load_group(k0, ka, sa);
  for (;;) {
    const int k1 = k0 + 64;
    if (k1 < kend) load_group(k1, kb, sb);
    compute(k0, ka, sa);
    if (k1 >= kend) break;
    const int k2 = k1 + 64;
    if (k2 < kend) load_group(k2, ka, sa);
    compute(k1, kb, sb);
    if (k2 >= kend) break;
    k0 = k2;
  }
}

// Direct global -> LDS loads for the block's key groups (inline asm: the kernel
// orders them itself with s_waitcnt vmcnt and barriers, so the compiler must not
// make later LDS reads wait for them).  They write no register; M0 is restored.
__device__ __forceinline__ void lds_dma16(const uint8_t* base, uint32_t off, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(base), "s"(lds)
      : "memory");
}
// The same with the non-temporal hint, for bytes read once per call (a decode row's
// keys): they stream through the caches without displacing what is reused.
__device__ __forceinline__ void lds_dma16_nt(const uint8_t* base, uint32_t off, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dwordx4 %1, %2 nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(base), "s"(lds)
      : "memory");
}
__device__ __forceinline__ void lds_dma4(const uint8_t* base, uint32_t off, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dword %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(base), "s"(lds)
      : "memory");
}
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)(p));
}

// ---------------------------------------------------------------------------
// Decode streaming tiling: one query row per block row, SKPB keys per block.  Each
// wave owns a ring of SDEPTH groups of 64 keys in LDS and copies its groups (the
// block's groups wv, wv + SW, ...) HBM -> LDS with contiguous 1 KB direct loads, plus
// the group's 64 key scales; it reads its MFMA fragments from its own ring, so the
// loop has no block barrier (a wave waits on its own loads only).  The query row
// comes in by direct loads too, ahead of the first groups, so that its arrival is
// awaited with the same counter instead of a wait for every load in flight.  Inside
// a group the 16-byte chunk c of key e sits in slot e * 8 + (c ^ (e & 7)), which
// spreads a fragment read over the LDS banks.  Scores are staged in LDS and written
// once the block's keys are done, so the loop's memory counter counts only the
// copies.  Grid: num_rows * key_blocks blocks (row-major), SW waves each.
// ---------------------------------------------------------------------------
constexpr int SW = 4;           // waves per block
constexpr int SKPB = 4096;      // keys per block
constexpr int SDEPTH = 3;       // groups in a wave's ring
constexpr int SGK = 64;         // keys per group
constexpr int SGB = SGK * ID;   // 8 KB per group
constexpr int SLOADS = SGB / 1024 + 1;  // direct loads per group: 8 x 1 KB of keys + the scales

template <bool PAGED>
__global__ __launch_bounds__(SW * 64) void indexer_fp8_stream_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ k_idx,
    const float* __restrict__ k_scale, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_pos, int B, int N, int nkb, float* __restrict__ scores,
    int64_t ld, PageMap pm, ClearWords clear) {
  __shared__ __attribute__((aligned(16))) uint8_t kring[SW][SDEPTH][SGB];
  __shared__ __attribute__((aligned(16))) float sring[SW][SDEPTH][SGK];
  __shared__ __attribute__((aligned(16))) float sout[SKPB];
  __shared__ __attribute__((aligned(16))) uint8_t qlds[IH * ID];
  __shared__ __attribute__((aligned(16))) float wlds[2][IH];  // head weights, query scales
  static_assert(SW * 2048 == IH * ID, "each wave copies 2 KB of the query row");
  if (blockIdx.x == 0)  // words a following launch needs zeroed
    for (int i = threadIdx.x; i < clear.n; i += SW * 64) clear.ptr[i] = 0u;
  const int r = blockIdx.x / nkb;
  const int kb0 = (blockIdx.x - r * nkb) * SKPB;
  const int b = row_seq[r], t = row_pos[r];
  if (b < 0 || b >= B || t < 0 || t >= N || (int64_t)t >= ld || kb0 > t) return;
  const int kend = min(kb0 + SKPB, t + 1);
  const int ngroups = (kend - kb0 + SGK - 1) / SGK;
  const int l = lane_id(), g = l >> 4, n = l & 15;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int mine = ngroups > wv ? (ngroups - wv + SW - 1) / SW : 0;  // groups wv, wv + SW, ...

  // this wave's 2 KB of the query row; waves 0 and 1 also the head weights and scales
  const uint8_t* qsrc = q_idx + (size_t)r * IH * ID;
  lds_dma16(qsrc, (uint32_t)(2048 * wv + 16 * l), lds_u32(qlds + 2048 * wv));
  lds_dma16(qsrc, (uint32_t)(2048 * wv + 1024 + 16 * l), lds_u32(qlds + 2048 * wv + 1024));
  if (wv < 2)
    lds_dma4(reinterpret_cast<const uint8_t*>((wv == 0 ? w : q_scale) + (size_t)r * IH),
             (uint32_t)(4 * l), lds_u32(wlds[wv]));

  // paged: offsets from the pool bases; contiguous: from this sequence's caches
  const uint8_t* kc = PAGED ? k_idx : k_idx + (size_t)b * N * ID;
  const uint8_t* ksc = reinterpret_cast<const uint8_t*>(PAGED ? k_scale : k_scale + (size_t)b * N);
  // group j of this wave into ring slot j % SDEPTH: lane l of copy i fetches the
  // chunk whose swizzled slot is 64 i + l.  Keys past kend read key kend - 1 (their
  // scores are never written).  A group of 64 keys lies in one page.
  auto issue = [&](int j) {
    const int k0 = kb0 + SGK * (wv + SW * j);
    uint32_t base = (uint32_t)k0;
    if constexpr (PAGED) base = paged_row(pm, b, k0);
    const int last = kend - 1 - k0;
    uint8_t* dst = kring[wv][j % SDEPTH];
#pragma unroll
    for (int i = 0; i < SGB / 1024; ++i) {
      const int P = 64 * i + l;
      const int e = P >> 3;
      const int c = (P & 7) ^ (e & 7);
      lds_dma16_nt(kc, (base + (uint32_t)min(e, last)) * (uint32_t)ID + (uint32_t)(16 * c),
                lds_u32(dst + 1024 * i));
    }
    lds_dma4(ksc, (base + (uint32_t)min(l, last)) * 4u, lds_u32(sring[wv][j % SDEPTH]));
  };
  const int x = n & 7;  // key & 7 for every tile's key 16 kt + n
  const int c0 = (2 * g) ^ x, c1 = (2 * g + 1) ^ x;
  for (int j = 0; j < SDEPTH - 1 && j < mine; ++j) issue(j);
  // the query copies are older than the group copies just issued: wait for them,
  // then for the other waves' (one block barrier, outside the loop)
  const int ahead = min(mine, SDEPTH - 1);
  if (ahead == 2)
    asm volatile("s_waitcnt vmcnt(18)\n\ts_barrier" ::: "memory");
  else if (ahead == 1)
    asm volatile("s_waitcnt vmcnt(9)\n\ts_barrier" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  i32x8 qa[4];
  float wq[16];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const uint8_t* qrow = qlds + (16 * mt + n) * ID + 32 * g;
    const i32x4 h0 = *reinterpret_cast<const i32x4*>(qrow);
    const i32x4 h1 = *reinterpret_cast<const i32x4*>(qrow + 16);
    qa[mt] = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int h = 16 * mt + 4 * g + v;
      wq[mt * 4 + v] = wlds[0][h] * wlds[1][h];
    }
  }
  for (int j = 0; j < mine; ++j) {
    if (j + SDEPTH - 1 < mine) issue(j + SDEPTH - 1);
    // group j is in: the copies of the (up to SDEPTH - 1) later groups may still fly
    const int later = min(mine - 1 - j, SDEPTH - 1);
    if (later == 2)
      asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
    else if (later == 1)
      asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    static_assert(SLOADS == 9 && SDEPTH == 3, "wait counts above");
    const uint8_t* kg = kring[wv][j % SDEPTH];
    i32x8 kf[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const uint8_t* row = kg + (16 * kt + n) * ID;
      const i32x4 a0 = *reinterpret_cast<const i32x4*>(row + 16 * c0);
      const i32x4 a1 = *reinterpret_cast<const i32x4*>(row + 16 * c1);
      kf[kt] = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    // 16 MFMAs (key tile kt = m >> 2, head tile mt = m & 3); step m issues MFMA m and
    // the epilogue of MFMA m - 2, a scheduling fence closing each step
    float p[4], hp[4];
    f32x4 acc[3];
#pragma unroll
    for (int m = 0; m < 18; ++m) {
      if (m < 16) acc[m % 3] = mfma_fp8_16x16x128(qa[m & 3], kf[m >> 2], f32x4{0.f, 0.f, 0.f, 0.f});
      if (m >= 2) {
        const int e = m - 2, mt = e & 3;
        const f32x4 x = acc[e % 3];
        float c = wq[mt * 4] * relu_bits(x[0]);
#pragma unroll
        for (int v = 1; v < 4; ++v) c = fmaf(wq[mt * 4 + v], relu_bits(x[v]), c);
        hp[mt] = c;
        if (mt == 3) p[e >> 2] = (hp[0] + hp[1]) + (hp[2] + hp[3]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    sout[SGK * (wv + SW * j) + l] = reduce_groups(p[0], p[1], p[2], p[3]) * sring[wv][j % SDEPTH][l];
  }
  __syncthreads();
  // the block's scores, keys [kb0, kend)
  float* out = scores + (size_t)r * ld + kb0;
  const int cnt = kend - kb0;
  const bool vec = (reinterpret_cast<uintptr_t>(out) & 15u) == 0u;
  for (int i = 4 * (int)threadIdx.x; i < cnt; i += 4 * SW * 64) {
    if (vec && i + 3 < cnt) {
      *reinterpret_cast<f32x4*>(out + i) = *reinterpret_cast<const f32x4*>(sout + i);
    } else {
      for (int e = 0; e < 4 && i + e < cnt; ++e) out[i + e] = sout[i + e];
    }
  }
}

// Prefill block: PW waves x PRW query rows (fp8 queries in registers) over PKPB keys.
// The keys are staged once per block, 128 at a time, HBM -> LDS by direct loads
// into two buffers, one group ahead; every wave reads its MFMA fragments from LDS,
// so the block fetches each key once instead of once per wave.  Two blocks share a
// CU (LDS and registers allow exactly two), so one block's barrier and copy waits
// overlap the other's MFMAs (against one 8-wave block with four buffers three groups
// ahead: 1-2 % faster on the 128K chunks, 2.4 % on 32K rows).  Inside a group, the
// 16-byte chunk c of key e sits in slot e * 8 + (c ^ (e & 7)), which spreads the 16
// rows of a fragment read over the LDS banks.
constexpr int PW = 4, PRW = 2, PROWS = PW * PRW, PKPB = 1024, PG = 128, PNBUF = 2;
constexpr int PGB = PG * ID;          // 16 KB per group
constexpr int PLW = PGB / (PW * 1024);  // 1 KB direct loads per wave and group
constexpr int PSW = PG / PW;          // key scales per wave and group
static_assert(PLW * PW * 1024 == PGB && PSW <= 64, "a group's copies split evenly over the waves");

template <bool PAGED>
__global__ __launch_bounds__(PW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void indexer_fp8_prefill_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ k_idx,
    const float* __restrict__ k_scale, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_pos, int R, int B, int N, int ksplit,
    float* __restrict__ scores, int64_t ld, PageMap pm, ClearWords clear,
    uint32_t* __restrict__ rowmm) {
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[PNBUF][PGB];
  if (blockIdx.x == 0)  // words a following launch needs zeroed
    for (int i = threadIdx.x; i < clear.n; i += PW * 64) clear.ptr[i] = 0u;
  __shared__ float ksbuf[PNBUF][PG];
  __shared__ __attribute__((aligned(16))) float sbuf[PROWS][PKPB];  // one key block's scores
  __shared__ int info[PW][3];
  // block (tile, ks) walks key blocks ks, ks + ksplit, ... up to its rows' last
  // position, so the grid does not depend on a bound of the positions
  const int tile = blockIdx.x / ksplit;
  const int ks = blockIdx.x - tile * ksplit;
  const int l = lane_id(), g = l >> 4, n = l & 15;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  int rr[PRW], tt[PRW], bs[PRW];
  int bmin = 1 << 30, bmax = -1, tmax = -1;
#pragma unroll
  for (int i = 0; i < PRW; ++i) {
    const int r = tile * PROWS + wv * PRW + i;
    int b = -1, t = -1;
    if (r < R) {
      b = row_seq[r];
      t = row_pos[r];
      if (b < 0 || b >= B || t < 0 || t >= N || (int64_t)t >= ld) t = -1;
    }
    rr[i] = r < R ? r : 0;
    tt[i] = t;
    bs[i] = b;
    if (t >= 0) {
      bmin = min(bmin, b);
      bmax = max(bmax, b);
      tmax = max(tmax, t);
    }
  }
  if (l == 0) {
    info[wv][0] = bmin;
    info[wv][1] = bmax;
    info[wv][2] = tmax;
  }
  __syncthreads();
  int Bmin = 1 << 30, Bmax = -1, Tmax = -1;
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    Bmin = min(Bmin, info[i][0]);
    Bmax = max(Bmax, info[i][1]);
    Tmax = max(Tmax, info[i][2]);
  }
  if (Tmax < ks * PKPB) return;  // block-uniform

  if (Bmin != Bmax) {
    // rows of several sequences: each wave walks its own rows' keys from global memory
    float mx[PRW], mn[PRW];
#pragma unroll
    for (int i = 0; i < PRW; ++i) {
      mx[i] = -INFINITY;
      mn[i] = INFINITY;
    }
    for (int kb0 = ks * PKPB; kb0 <= Tmax; kb0 += ksplit * PKPB) {
#pragma unroll
      for (int i = 0; i < PRW; ++i) {
        if (tt[i] < kb0) continue;
        const int kend = min(kb0 + PKPB, tt[i] + 1);
        prefill_rows<1, PAGED>(q_idx, q_scale, w, PAGED ? k_idx : k_idx + (size_t)bs[i] * N * ID,
                               PAGED ? k_scale : k_scale + (size_t)bs[i] * N, &rr[i], &tt[i],
                               kb0, kend, scores, ld, pm, bs[i], &mx[i], &mn[i]);
      }
    }
    if (rowmm != nullptr) {
#pragma unroll
      for (int i = 0; i < PRW; ++i) {
        const float a = wave_max(mx[i]), c = wave_min(mn[i]);
        if (l == 0 && tt[i] >= 0) {
          atomicMax(&rowmm[2 * rr[i]], float_key(a));
          atomicMax(&rowmm[2 * rr[i] + 1], ~float_key(c));
        }
      }
    }
    return;
  }

  const uint8_t* kc = PAGED ? k_idx : k_idx + (size_t)Bmin * N * ID;
  const uint8_t* ksc = reinterpret_cast<const uint8_t*>(PAGED ? k_scale : k_scale + (size_t)Bmin * N);

  i32x8 qa[PRW][4];
  float wq[PRW][16];
#pragma unroll
  for (int i = 0; i < PRW; ++i) load_query(q_idx, q_scale, w, rr[i], qa[i], wq[i]);
  // the queries are in before the key loop (s_waitcnt vmcnt(0), as a builtin the
  // compiler's wait bookkeeping sees): the loop's vmcnt counts only the key copies
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // B fragment of key tile kt: row e = 16 kt + n, bytes [32 g, 32 g + 32) = chunks
  // 2 g and 2 g + 1, each at its swizzled slot
  const int x = n & 7;  // e & 7 for every tile
  const int c0 = (2 * g) ^ x, c1 = (2 * g + 1) ^ x;

  // extremes of the scores this thread writes out, per write-out step (one row each)
  constexpr int V4 = PKPB / 4;
  constexpr int WJ = PROWS * V4 / (PW * 64);  // write-out steps per thread
  static_assert(V4 % 64 == 0 && PROWS * V4 == WJ * PW * 64, "one row per wave and step");
  float wmx[WJ], wmn[WJ];
#pragma unroll
  for (int j = 0; j < WJ; ++j) {
    wmx[j] = -INFINITY;
    wmn[j] = INFINITY;
  }
  for (int kb0 = ks * PKPB; kb0 <= Tmax; kb0 += ksplit * PKPB) {
    const int kend = min(kb0 + PKPB, Tmax + 1);
    const int ngroups = (kend - kb0 + PG - 1) / PG;
    const int klast = kend - 1;
    // group gi of this key block (128 keys): wave wv fetches LDS slots
    // [64 PLW wv, 64 PLW (wv + 1)) of the keys and the scales of keys [PSW wv, PSW (wv + 1))
    auto issue_group = [&](int gi) {
      const int k0 = kb0 + gi * PG;
      // paged: a group's keys lie in page k0 >> shift and (pages of 64) the next one
      int p0 = 0;
      uint32_t pg0 = 0, pg1 = 0;
      if constexpr (PAGED) {
        p0 = k0 >> pm.shift;
        pg0 = paged_row(pm, Bmin, p0 << pm.shift) >> pm.shift;
        pg1 = paged_row(pm, Bmin, min(p0 + 1, pm.pps - 1) << pm.shift) >> pm.shift;
      }
      auto row = [&](int key) -> uint32_t {
        if constexpr (!PAGED) return (uint32_t)key;
        const uint32_t pg = (key >> pm.shift) == p0 ? pg0 : pg1;
        return (pg << pm.shift) | (uint32_t)(key & ((1 << pm.shift) - 1));
      };
#pragma unroll
      for (int h = 0; h < PLW; ++h) {
        const int P = 64 * (PLW * wv + h) + l;
        const int e = P >> 3;
        const int c = (P & 7) ^ (e & 7);
        const uint32_t off = row(min(k0 + e, klast)) * (uint32_t)ID + (uint32_t)(16 * c);
        lds_dma16(kc, off, lds_u32(&kbuf[gi % PNBUF][1024 * (PLW * wv + h)]));
      }
      if (l < PSW)
        lds_dma4(ksc, row(min(k0 + PSW * wv + l, klast)) * 4u,
                 lds_u32(&ksbuf[gi % PNBUF][PSW * wv]));
    };
    // every wave is past the previous key block's reads of kbuf and sbuf
    __syncthreads();
    if (ngroups > 0) issue_group(0);

    for (int gi = 0; gi < ngroups; ++gi) {
      // group gi is in (this wave's copies are its only loads in flight) and every
      // wave is done with group gi - 1, whose buffer group gi + 1 takes
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (gi + 1 < ngroups) issue_group(gi + 1);
      const uint8_t* kg = kbuf[gi % PNBUF];
      const float* ksg = ksbuf[gi % PNBUF];
      // The group as one pipeline of 64 MFMAs: m = 4 v + mt, unit v = (half u,
      // key tile kt, row i) with v = 8 u + 2 kt + i, head tile mt.  Step m issues
      // MFMA m and the epilogue of MFMA m - LAG (ReLU and 4 weighted head terms,
      // 8 VALU ops, into head chain mt of its unit); a scheduling fence closes
      // every step, so the matrix pipe and the VALU always have independent work
      // (left to itself the compiler consumes each MFMA's result right after it
      // and waits out its latency).  Fragment f = 4 u + kt (B operand of key tile
      // kt of half u) is read from LDS when the group starts (f < 4) or once
      // fragment f - 4 has issued its last MFMA.  Rows past their last position
      // are computed too; such scores are never written out.
      static_assert(PRW == 2 && PG == 128, "unit order v = 8 u + 2 kt + i");
      constexpr int LAG = 2, NM = 64;
      i32x8 kf[8];
      auto read_frag = [&](int f) {
        const uint8_t* row = kg + (64 * (f >> 2) + 16 * (f & 3) + n) * ID;
        const i32x4 a = *reinterpret_cast<const i32x4*>(row + 16 * c0);
        const i32x4 b = *reinterpret_cast<const i32x4*>(row + 16 * c1);
        kf[f] = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
      };
#pragma unroll
      for (int f = 0; f < 4; ++f) read_frag(f);
      const float ks0 = ksg[l], ks1 = ksg[64 + l];
      f32x4 acc[LAG + 1];
      float a[4], p[PRW][4];
#pragma unroll
      for (int m = 0; m < NM + LAG; ++m) {
        if (m < NM) {
          const int v = m >> 2, mt = m & 3, f = v >> 1, i = v & 1;
          acc[m % (LAG + 1)] = mfma_fp8_16x16x128(qa[i][mt], kf[f], f32x4{0.f, 0.f, 0.f, 0.f});
          if (mt == 3 && i == 1 && f + 4 < 8) read_frag(f + 4);
        }
        if (m >= LAG) {
          const int e = m - LAG, v = e >> 2, mt = e & 3, i = v & 1, kt = (v >> 1) & 3;
          const f32x4 x = acc[e % (LAG + 1)];
          float c = wq[i][mt * 4] * relu_bits(x[0]);
#pragma unroll
          for (int j = 1; j < 4; ++j) c = fmaf(wq[i][mt * 4 + j], relu_bits(x[j]), c);
          a[mt] = c;
          if (mt == 3) p[i][kt] = (a[0] + a[1]) + (a[2] + a[3]);
          if ((e & 31) == 31) {  // both rows of half e >> 5 are complete
            const int u = e >> 5;
#pragma unroll
            for (int r = 0; r < PRW; ++r)
              sbuf[wv * PRW + r][gi * PG + 64 * u + l] =
                  reduce_groups(p[r][0], p[r][1], p[r][2], p[r][3]) * (u ? ks1 : ks0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // The key block's scores leave LDS after its loop, so that no vector-memory
    // store sits between the direct loads whose completion the loop counts with
    // vmcnt.  Each valid row writes keys [kb0, kend) (entries past its own
    // position are left unspecified, as the interface allows).
    // Write-out step j of a thread covers row (threadIdx.x + 512 j) / V4, the same
    // row in every key block; the scores at positions <= the row's own also update
    // the step's extremes (fmaxf / fminf pass over a NaN).
    __syncthreads();
    const int nv4 = (kend - kb0 + 3) / 4;
#pragma unroll
    for (int j = 0; j < WJ; ++j) {
      const int idx = threadIdx.x + j * PW * 64;
      const int row = idx / V4, c4 = idx - row * V4;  // row is wave-uniform
      const int r = tile * PROWS + row;
      if (c4 < nv4 && r < R) {
        const int t = row_pos[r];
        const int s0 = kb0 + 4 * c4;
        if (t >= s0) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(&sbuf[row][4 * c4]);
          float* dst = scores + (size_t)r * ld + s0;
          if (s0 + 4 <= kend && ((reinterpret_cast<uintptr_t>(dst) & 15) == 0)) {
            *reinterpret_cast<f32x4*>(dst) = v;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (s0 + e < kend) dst[e] = v[e];
          }
          if (s0 + 3 <= t) {
            wmx[j] = fmaxf(wmx[j], fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
            wmn[j] = fminf(wmn[j], fminf(fminf(v[0], v[1]), fminf(v[2], v[3])));
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (s0 + e <= t) {
                wmx[j] = fmaxf(wmx[j], v[e]);
                wmn[j] = fminf(wmn[j], v[e]);
              }
          }
        }
      }
    }
  }
  if (rowmm != nullptr) {  // block-uniform
#pragma unroll
    for (int j = 0; j < WJ; ++j) {
      const int r = tile * PROWS + ((int)threadIdx.x + j * PW * 64) / V4;
      const float a = wave_max(wmx[j]), c = wave_min(wmn[j]);
      if (l == 0 && r < R) {
        atomicMax(&rowmm[2 * r], float_key(a));
        atomicMax(&rowmm[2 * r + 1], ~float_key(c));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 correctness path (any H_I <= 64, d_I <= 128): one thread per key.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void indexer_f32_kernel(
    const float* __restrict__ q_idx, const float* __restrict__ w,
    const float* __restrict__ k_idx, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_pos, int B, int N, int HI, int DI, int nkb,
    float* __restrict__ scores, int64_t ld) {
  __shared__ float qs[64 * 128];
  __shared__ float ws[64];
  const int r = blockIdx.x / nkb;
  const int s0 = (blockIdx.x - r * nkb) * 256;
  const int b = row_seq[r], t = row_pos[r];
  if (b < 0 || b >= B || t < 0 || t >= N || (int64_t)t >= ld || s0 > t) return;
  for (int i = threadIdx.x; i < HI * DI; i += 256) qs[i] = q_idx[(size_t)r * HI * DI + i];
  for (int i = threadIdx.x; i < HI; i += 256) ws[i] = w[(size_t)r * HI + i];
  __syncthreads();
  const int s = s0 + threadIdx.x;
  if (s > t) return;
  const float* kv = k_idx + ((size_t)b * N + s) * DI;
  float acc = 0.f;
  for (int j = 0; j < HI; ++j) {
    float dot = 0.f;
    for (int d = 0; d < DI; ++d) dot = fmaf(qs[j * DI + d], kv[d], dot);
    acc = fmaf(ws[j], fmaxf(dot, 0.f), acc);
  }
  scores[(size_t)r * ld + s] = acc;
}

}  // namespace

bool indexer_uses_tiles(const dsa_rows& rows) {
  return rows.num_rows >= 8 && rows.num_rows >= 4 * rows.num_seqs;
}

hipError_t launch_indexer_fp8(const dsa_rows& rows, const uint8_t* q_idx, const float* q_scale,
                              const float* w, const uint8_t* k_idx, const float* k_scale,
                              float* scores, int64_t ld, hipStream_t stream, const PageMap& pm,
                              ClearWords clear, uint32_t* rowmm) {
  const bool paged = pm.table != nullptr;
  const int R = rows.num_rows;
  const int L = rows.max_pos + 1;
  if (indexer_uses_tiles(rows)) {
    // key blocks are split over ksplit blocks per row tile (enough blocks to fill
    // the GPU several times over); each block loops over its share
    const int nkb = (L + PKPB - 1) / PKPB;
    const int tiles = (R + PROWS - 1) / PROWS;
    int ksplit = 1;
    while (ksplit < nkb && (int64_t)tiles * ksplit < 2048) ksplit <<= 1;
    auto kern = paged ? indexer_fp8_prefill_kernel<true> : indexer_fp8_prefill_kernel<false>;
    hipLaunchKernelGGL(kern, dim3(tiles * ksplit), dim3(PW * 64), 0, stream, q_idx, q_scale, w,
                       k_idx, k_scale, rows.row_seq, rows.row_pos, R, rows.num_seqs,
                       rows.max_ctx, ksplit, scores, ld, pm, clear, rowmm);
  } else {
    if (rowmm != nullptr) return hipErrorInvalidValue;  // only the tiled kernel keeps extremes
    const int nkb = (L + SKPB - 1) / SKPB;
    auto kern = paged ? indexer_fp8_stream_kernel<true> : indexer_fp8_stream_kernel<false>;
    hipLaunchKernelGGL(kern, dim3(R * nkb), dim3(SW * 64), 0, stream, q_idx, q_scale, w, k_idx,
                       k_scale, rows.row_seq, rows.row_pos, rows.num_seqs, rows.max_ctx, nkb,
                       scores, ld, pm, clear);
  }
  return hipGetLastError();
}

hipError_t launch_indexer_f32(const dsa_rows& rows, const dsa_dims& dims, const float* q_idx,
                              const float* w, const float* k_idx, float* scores, int64_t ld,
                              hipStream_t stream) {
  const int L = rows.max_pos + 1;
  const int nkb = (L + 255) / 256;
  hipLaunchKernelGGL(indexer_f32_kernel, dim3(rows.num_rows * nkb), dim3(256), 0, stream, q_idx,
                     w, k_idx, rows.row_seq, rows.row_pos, rows.num_seqs, rows.max_ctx,
                     dims.n_idx_heads, dims.idx_dim, nkb, scores, ld);
  return hipGetLastError();
}

}  // namespace dsa
