// Sparse MLA attention in MQA mode on gfx950.
//
// For query row r (sequence b) and head h over the selected positions S_r:
//   z[s] = scale * q[r,h,:] . c[b,s,:]          (576 = 512 latent + 64 rope)
//   o[r,h,:] = sum_s softmax(z)[s] * c[b,s,0:512],  lse[r,h] = log sum_s e^z[s]
// (DeepSeek-V3.2-Exp paper, section 1 Eq. 2 prose and "Instantiate DSA under MLA":
// every latent entry is shared by all query heads of the token; Appendix A, Fig. 4:
// MQA mode of MLA.)
//
// Kernel design (bf16 path, H = 128, D_k = 576, D_v = 512):
// * one 512-thread block (8 waves) per (row, split); a split is a contiguous slice
//   of the row's selected positions.  Splits of a row are mapped to one XCD so
//   the row's queries come from HBM once per XCD L2.
// * wave w owns head group hg = w/2 (32 heads) and half hf = w%2.  Its share of
//   the 576-long contraction is latent dims [256 hf, 256 hf + 256), whose queries
//   stay in registers (64 VGPRs), plus rope dims [512 + 32 hf, +32), read from a
//   16 KB LDS copy of the row's rope queries.  It accumulates output columns
//   [256 hf, 256 hf + 256) (128 registers).  The two halves of S = q c^T are
//   summed through LDS, so both waves of a pair see the same fp32 logits.  The
//   kernel fits 255 VGPRs with no scratch: a spill reload inside the loop would
//   wait on the in-flight gather (vmcnt is in order) and serialise the pipeline.
// * positions are processed 32 at a time.  The 32 gathered latent rows (36 KB)
//   are copied HBM -> LDS by direct global_load_lds, double-buffered, so the next
//   gather overlaps this block's MFMAs.  A 16-byte chunk swizzle inside each row
//   keeps the operand reads spread over the LDS banks.
// * S^T tiles (M = 16 positions, N = 16 heads) leave each lane with 4 consecutive
//   positions of one head: exactly the P operand of the P.V MFMA (M = 16 heads,
//   K = 32 positions) after a bf16 cast, with no shuffles.  The V operand needs
//   the row-major tile read column-wise; ds_read_b64_tr_b16 does that: within
//   each 16-lane group, lane L receives element L%4 of the 8-byte chunks addressed
//   by lanes 4i + L/4 (i = 0..3), so lanes pointing at V[e_i][d0 + 4j .. +3]
//   deliver V[e_0..e_3][d0 + L] to lane L.
// * online softmax in the exp2 domain with a stale-max rule: the running max is
//   raised (and the accumulators rescaled) only when a block's max exceeds it by
//   more than 2^8, which bounds every weight by 2^8 and skips nearly all rescales.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

// Index-domain flag of this device: an attention kernel that meets an index entry
// past its row's position t (a future position, which no causal selection holds)
// stores 1 here with a plain vector store; the entry is treated as padding either
// way.  The host reads and clears it through dsa_check_index_domain.
__device__ uint32_t g_index_domain_flag = 0u;

__device__ __forceinline__ void flag_index_domain() {
  *static_cast<volatile uint32_t*>(&g_index_domain_flag) = 1u;
}

constexpr int H = kHeads;           // 128
constexpr int DK = kQkDim;          // 576
constexpr int DV = kVDim;           // 512
constexpr int BE = 32;              // positions per block
constexpr int KROW = DK * 2;        // 1152 bytes per latent row
constexpr int KCH = KROW / 16;      // 72 chunks of 16 bytes
constexpr int STAGE = BE * KROW;    // 36864 bytes per gathered block
constexpr int NT = 512;             // 8 waves
constexpr int NWAVE = NT / 64;
constexpr int LOADS = STAGE / 1024; // 36 direct loads of 1 KB per block
constexpr int KS_LAT = DV / 32 / 2;   // 8 latent contraction steps of 32 per half
constexpr int RD = DK - DV;           // 64 rope dims
constexpr int QR_STRIDE = RD * 2 + 16;  // bytes per head row of the rope queries in LDS
constexpr int DT_HALF = DV / 16 / 2;  // 16 output column tiles per half
constexpr float kStaleMax = 8.0f;   // log2 headroom of the stale running max
constexpr float kLn2 = 0.69314718055994530942f;
static_assert(((LOADS * 64 - 1) * 3641 >> 18) == (LOADS * 64 - 1) / KCH, "slot / 72 by multiply");

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_t;

// physical 16-byte slot of logical chunk c of entry e inside its 1152-byte row
__device__ __forceinline__ int kswz(int e, int c) { return (c & ~7) | ((c ^ e) & 7); }

// Direct 16-byte global -> LDS load: lane l's 16 bytes from base + off go to LDS
// bytes [lds + 16 l, lds + 16 l + 16) (lds is wave-uniform, passed in M0).  It is
// written as inline asm so that the compiler does not order later LDS reads (of
// other stage buffers) behind it: the kernel orders the gathers itself, with
// s_waitcnt vmcnt and barriers.  It writes no register; M0 is restored.
__device__ __forceinline__ void gather16(const uint8_t* base, uint32_t off, uint32_t lds) {
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

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)(p));
}

// max of v over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the same nn, every g):
// v_permlane16_swap(x, x) leaves {x[l & ~16], x[l | 16]} and v_permlane32_swap
// {x[l & ~32], x[l | 32]} in its two results, so each swap pairs l with its partner
// without a trip through LDS.
__device__ __forceinline__ float max_over_g(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ i32x2 ds_read_tr16(const uint8_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)(p));
  return __builtin_bit_cast(i32x2, v);
}

template <bool PAGED>
__global__ __launch_bounds__(NT, 1) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ latent,
    const int32_t* __restrict__ indices, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_pos, int R, int B, int N, int topk, int splits,
    float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse,
    uint16_t* __restrict__ o_part, float* __restrict__ lse_part, PageMap pm) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];
  __shared__ __attribute__((aligned(16))) float xbuf[NWAVE][16][64];  // S partials
  __shared__ int sidx[kTopk];
  // rope part of the 128 queries (q[r, h, 512:576]), rows padded to spread banks
  __shared__ __attribute__((aligned(16))) uint8_t qrope[H * QR_STRIDE];

  const int tid = threadIdx.x, l = lane_id(), g = l >> 4, nn = l & 15;
  // wave-uniform indices live in scalar registers
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = wv >> 1, hf = wv & 1;
  // XCD-aware decode of the block id: all splits of row r run on XCD r % 8.
  const int xcd = blockIdx.x & 7;
  const int rest = blockIdx.x >> 3;
  const int sp = rest % splits;
  const int r = (rest / splits) * 8 + xcd;
  if (r >= R) return;

  const int ES = topk / splits;  // positions of this split
  const int nblk = ES / BE;
  const int32_t* irow = indices + (size_t)r * topk + (size_t)sp * ES;

  // Prologue, ordered so that the memory latencies do not add up.  What needs only
  // the row goes out first, before the row's sequence and position are known: the
  // first block's gather positions (straight from the index row), the rest of the
  // row and the rope queries.  The first gather is issued as soon as its positions
  // and the sequence arrive, and the latent queries (needed only by the first
  // block's products) last.
  constexpr int MAXL = (LOADS + NWAVE - 1) / NWAVE;  // 5 direct loads per wave and block
  int p_first[MAXL];
#pragma unroll
  for (int j = 0; j < MAXL; ++j) {
    const int i = wv + j * NWAVE;
    const int P = (i < LOADS ? i : 0) * 64 + l;
    const int e = (P * 3641) >> 18;  // P / 72 for P < 2304
    p_first[j] = nblk > 0 ? irow[e] : 0;
  }
  constexpr int IPT = kTopk / NT;  // selected positions per thread (at most)
  int pv[IPT];
#pragma unroll
  for (int k = 0; k < IPT; ++k) {
    const int i = tid + NT * k;
    pv[k] = i < ES ? irow[i] : -1;
  }
  // rope queries of all 128 heads (8 chunks of 16 bytes per head), bound for LDS
  constexpr int QRC = H * (RD / 8) / NT;  // 2 chunks per thread
  i32x4 qrv[QRC];
#pragma unroll
  for (int k = 0; k < QRC; ++k) {
    const int c = tid + NT * k, h = c >> 3, j = c & 7;
    qrv[k] = *reinterpret_cast<const i32x4*>(q + ((size_t)r * H + h) * DK + DV + 8 * j);
  }

  const int b = row_seq[r], t = row_pos[r];
  if (b < 0 || b >= B || t < 0 || t >= N) return;
  // paged: offsets from the pool base (pool rows from the block table); contiguous:
  // from this sequence's cache
  const uint16_t* lat = PAGED ? latent : latent + (size_t)b * N * DK;
  const uint8_t* lat_bytes = reinterpret_cast<const uint8_t*>(lat);
  auto cache_row = [&](int p) -> int { return PAGED ? (int)paged_row(pm, b, p) : p; };
  // Padding slots gather the sequence's own entry 0 (present, since t >= 0) and are
  // then masked: a masked row still meets a zero softmax weight in the value
  // product, so it must hold finite data, which an unused page need not.
  const int row0 = cache_row(0);

  uint32_t off_first[MAXL];
#pragma unroll
  for (int j = 0; j < MAXL; ++j) {
    const int i = wv + j * NWAVE;
    const int P = (i < LOADS ? i : 0) * 64 + l;
    const int e = (P * 3641) >> 18;  // P / 72 for P < 2304
    const int c = kswz(e, P - e * KCH);
    const int p = p_first[j];
    off_first[j] = __umul24((uint32_t)((p >= 0 && p <= t) ? cache_row(p) : row0), (uint32_t)KROW) +
                   (uint32_t)(16 * c);
  }
  if (nblk > 0) {
#pragma unroll
    for (int j = 0; j < MAXL; ++j) {
      const int i = wv + j * NWAVE;
      if (i < LOADS) gather16(lat_bytes, off_first[j], lds_addr(smem + i * 1024));
    }
  }
  // The latent queries are requested after the first gather and the rope queries:
  // the barrier below waits for the rope queries (they go to LDS), and a memory
  // counter that waited for them must not also wait for 128 KB of latent queries.
  // Contraction split: half hf owns latent dims [256 hf, 256 hf + 256) (k-steps
  // 8 hf .. 8 hf + 7, queries in registers) and rope dims [512 + 32 hf, +32)
  // (k-step 16 + hf, queries read from LDS).
  // registers: queries of heads 32hg + 16nt + nn, dims 256hf + 32ks + 8g .. +7
  i32x4 qr[2][KS_LAT];
  {
    const uint16_t* qrow = q + ((size_t)r * H + 32 * hg) * DK + 256 * hf;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int ks = 0; ks < KS_LAT; ++ks)
        qr[nt][ks] = *reinterpret_cast<const i32x4*>(qrow + (16 * nt + nn) * DK + 32 * ks + 8 * g);
  }
  // Causal rule: entries outside [0, t] are padding.  An entry past t (a future
  // position the selection cannot contain) also raises the index-domain flag.
  bool future = false;
#pragma unroll
  for (int k = 0; k < IPT; ++k) {
    const int i = tid + NT * k;
    if (i < ES) {
      sidx[i] = (pv[k] >= 0 && pv[k] <= t) ? cache_row(pv[k]) : -1;
      future |= pv[k] > t;
    }
  }
  if (future) flag_index_domain();
#pragma unroll
  for (int k = 0; k < QRC; ++k) {
    const int c = tid + NT * k, h = c >> 3, j = c & 7;
    *reinterpret_cast<i32x4*>(qrope + h * QR_STRIDE + 16 * j) = qrv[k];
  }
  // sidx and the rope queries visible; an unfenced barrier, so the gather and the
  // query loads stay in flight
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  // Gather of block blk into stage buffer kb: direct load i (wave wv issues
  // i = wv + 8 j) fills LDS bytes [1024 i, 1024 i + 1024); lane l fetches the
  // 16-byte chunk whose swizzled slot is its lane-linear destination P = 64 i + l:
  // entry P / 72, slot P % 72 (kswz is an involution, so the slot's chunk is kswz
  // of the slot).  The source offsets are computed before the barrier that frees
  // the buffer, so the loads issue right after it.
  // source offset of load j of this wave for block blk, from a lane id read afresh
  // (volatile asm, so that the compiler does not keep the loop-invariant slot
  // arithmetic in registers across the loop: it is cheap to redo)
  auto fresh_lane = [&]() {
    int lane;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
    return lane;
  };
  auto gather_offset = [&](int blk, int j, int lane) -> uint32_t {
    const int i = wv + j * NWAVE;
    const int P = (i < LOADS ? i : 0) * 64 + lane;
    const int e = (P * 3641) >> 18;  // P / 72 for P < 2304
    const int c = kswz(e, P - e * KCH);
    const int pos = sidx[blk * BE + e];
    // 32-bit offset from the sequence base or the pool base (a sequence's cache and
    // a pool are < 4 GiB, so rows are < 2^24)
    return __umul24((uint32_t)(pos >= 0 ? pos : row0), (uint32_t)KROW) + (uint32_t)(16 * c);
  };
  // The first MAXL - 1 offsets are computed before the barrier that frees the
  // buffer; the last load (waves 0..3 only) computes its own when it issues.
  auto gather_offsets = [&](int blk, uint32_t (&off)[MAXL - 1]) {
    const int lane = fresh_lane();
#pragma unroll
    for (int j = 0; j < MAXL - 1; ++j) off[j] = gather_offset(blk, j, lane);
  };
  auto issue_gather_one = [&](int blk, int j, const uint32_t (&off)[MAXL - 1], uint8_t* kb) {
    const int i = wv + j * NWAVE;
    if (i < LOADS)
      gather16(lat_bytes, j < MAXL - 1 ? off[j] : gather_offset(blk, j, fresh_lane()),
               lds_addr(kb + i * 1024));
  };

  // Per-lane LDS base offsets.  With x = e & 7 the swizzled slot of chunk c = 4k + u
  // (u < 4) is c ^ x = 4 (k ^ (x >> 2)) + (u ^ (x & 3)), and k ^ (x >> 2) is
  // k + (x >> 2) for even k and k - (x >> 2) for odd k; so every operand address
  // below is one of a few per-lane bases plus a compile-time offset.
  // QK^T A operand: entry 16 mt + nn, latent chunk 4 (8 hf + ks) + g (k = 8 hf + ks
  // has the parity of ks); rope chunk 4 (16 + hf) + g.
  const int xq = nn & 7;
  const int qa_base = nn * KROW + 16 * (g ^ (xq & 3)) + 512 * hf;
  const int qa_even = qa_base + 64 * (xq >> 2);  // ks even
  const int qa_odd = qa_base - 64 * (xq >> 2);   // ks odd
  const int qa_rope = hf ? qa_odd + 576 : qa_even + 1024;
  const int qb_rope = (32 * hg + nn) * QR_STRIDE + 64 * hf + 16 * g;  // B operand, nt = 0
  // P.V B operand (transposed reads): entry ei (+16), dims 256 hf + 16 dt + 4 (nn & 3),
  // chunk 32 hf + 8 (dt >> 2) + (2 (dt & 3) + hh), hh = (nn >> 1) & 1.
  const int ei = 4 * g + (nn >> 2);
  const int xv = ei & 7;
  const int hh = (nn >> 1) & 1;
  // slot (2j + hh) ^ xv = 2 (j ^ (xv >> 1)) + (hh ^ (xv & 1)) for column tile group j
  const int tr_base = ei * KROW + 512 * hf + 16 * (hh ^ (xv & 1)) + 8 * (nn & 1);
  const int tr_x = xv >> 1;

  f32x4 O[2][DT_HALF];
#pragma unroll
  for (int hm = 0; hm < 2; ++hm)
#pragma unroll
    for (int dt = 0; dt < DT_HALF; ++dt) O[hm][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_part[2] = {0.f, 0.f};

  for (int blk = 0; blk < nblk; ++blk) {
    const int st = blk & 1;
    const bool more = blk + 1 < nblk;
    uint32_t offn[MAXL - 1];
    if (more) gather_offsets(blk + 1, offn);
    // Block blk is in LDS and every wave is done with block blk-1.  A plain
    // s_barrier (in the asm, so no memory access moves across it): a fenced one
    // would also wait for the gather issued in the previous iteration, since
    // that is an outstanding LDS write.
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    uint8_t* const nxt = smem + (st ^ 1) * STAGE;
    const uint8_t* kb = smem + st * STAGE;
    // bit 16 mt + v of vbits: position 16 mt + 4 g + v of the block is not padding
    const uint32_t vbits = (uint32_t)__ballot(sidx[blk * BE + (l & (BE - 1))] >= 0) >> (4 * g);

    // ---- partial S^T over this wave's contraction half:
    //      acc[mt][nt] lane holds S^T[16mt + 4g + v][16nt + nn]
    f32x4 acc[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks <= KS_LAT; ++ks) {
      const bool rope = ks == KS_LAT;
      const uint8_t* ap = kb + (rope ? qa_rope : (((ks & 1) ? qa_odd : qa_even) + 64 * ks));
      bf16x8 a[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        a[mt] = as_bf16x8(*reinterpret_cast<const i32x4*>(ap + 16 * KROW * mt));
      bf16x8 bq[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        bq[nt] = rope ? as_bf16x8(*reinterpret_cast<const i32x4*>(qrope + qb_rope + 16 * QR_STRIDE * nt))
                      : as_bf16x8(qr[nt][rope ? 0 : ks]);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          acc[mt][nt] = mfma_bf16_16x16x32(a[mt], bq[nt], acc[mt][nt]);
      // the next block's direct loads go out one per contraction step, so the
      // address unit works through them while the MFMAs run
      if (more && ks < MAXL) issue_gather_one(blk + 1, ks, offn, nxt);
    }
    // ---- sum the two halves through LDS (same addition order in both waves)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int v = 0; v < 4; ++v) xbuf[wv][(mt * 2 + nt) * 4 + v][l] = acc[mt][nt][v];
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    float sfull[2][2][4];  // [mt][nt][v]
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float other = xbuf[wv ^ 1][(mt * 2 + nt) * 4 + v][l];
          const float mine = acc[mt][nt][v];
          sfull[mt][nt][v] = hf == 0 ? mine + other : other + mine;
        }

    // V operand of output column tile dt (transposed reads of the stage rows)
    auto read_v = [&](int dt) {
      const uint8_t* vp = kb + tr_base + 32 * ((dt & 3) ^ tr_x) + 128 * (dt >> 2);
      const i32x2 v0 = ds_read_tr16(vp);
      const i32x2 v1 = ds_read_tr16(vp + 16 * KROW);
      const i32x4 vv = {v0[0], v0[1], v1[0], v1[1]};
      return as_bf16x8(vv);
    };
    // the first tile's operands do not depend on P: read them before the softmax
    bf16x8 vnext = read_v(0);

    // ---- online softmax (exp2 domain) for the lane's heads 16nt + nn
    float bm[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float s = ((vbits >> (16 * mt + v)) & 1u) ? sfull[mt][nt][v] * scale_log2 : -INFINITY;
          sfull[mt][nt][v] = s;
          mx = fmaxf(mx, s);
        }
      bm[nt] = max_over_g(mx);
    }
    const bool raise = (bm[0] > m_run[0] + kStaleMax) || (bm[1] > m_run[1] + kStaleMax);
    if (__any(raise)) {
      float alpha[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const float mnew = fmaxf(m_run[nt], bm[nt]);
        alpha[nt] = (mnew == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[nt] - mnew);
        l_part[nt] *= alpha[nt];
        m_run[nt] = mnew;
      }
#pragma unroll
      for (int hm = 0; hm < 2; ++hm)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float a = __shfl(alpha[hm], 4 * g + v);
#pragma unroll
          for (int dt = 0; dt < DT_HALF; ++dt) O[hm][dt][v] *= a;
        }
    }
    bf16x8 pa[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const float mref = (m_run[nt] == -INFINITY) ? 0.f : m_run[nt];
      float p[2][4];
      float sum = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          p[mt][v] = __builtin_amdgcn_exp2f(sfull[mt][nt][v] - mref);
          sum += p[mt][v];
        }
      l_part[nt] += sum;
      i32x4 pk;
      pk[0] = (int)pack_bf16x2(p[0][0], p[0][1]);
      pk[1] = (int)pack_bf16x2(p[0][2], p[0][3]);
      pk[2] = (int)pack_bf16x2(p[1][0], p[1][1]);
      pk[3] = (int)pack_bf16x2(p[1][2], p[1][3]);
      pa[nt] = as_bf16x8(pk);
    }

    // ---- O += P V for output columns 256hf + 16dt + nn.  B operand slots 0..3 are
    //      positions 4g..4g+3, slots 4..7 positions 16+4g..16+4g+3 (the P layout).
    //      The operands of tile dt + 1 are read while the MFMAs of tile dt run.
    bf16x8 bv = vnext;
#pragma unroll
    for (int dt = 0; dt < DT_HALF; ++dt) {
      if (dt + 1 < DT_HALF) vnext = read_v(dt + 1);
      O[0][dt] = mfma_bf16_16x16x32(pa[0], bv, O[0][dt]);
      O[1][dt] = mfma_bf16_16x16x32(pa[1], bv, O[1][dt]);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // 2 LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // then 2 MFMAs
      bv = vnext;
    }
  }

  // ---- finalize: normalise by the softmax denominator of each output head
  float l_tot[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    float s = l_part[nt];
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    l_tot[nt] = s;
  }
#pragma unroll
  for (int hm = 0; hm < 2; ++hm)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float L = __shfl(l_tot[hm], 4 * g + v);
      const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
      for (int dt = 0; dt < DT_HALF; ++dt) O[hm][dt][v] *= inv;
    }
  // Output through LDS: each wave writes its 16-head half of the 32 x 256 output
  // tile as bf16 into its own region of the (now free) stage buffers, then reads it
  // back as 16-byte pieces, so that each store instruction writes whole 512-byte
  // head rows.  (Straight from the MFMA layout every lane would store 2-byte values
  // 32 bytes apart.)
  constexpr int EP_PITCH = 256 * 2 + 16;  // bytes per head row in LDS (bank spread)
  static_assert(NWAVE * 16 * EP_PITCH <= 2 * STAGE, "the epilogue tiles fit the stage buffers");
  uint8_t* ep = smem + wv * 16 * EP_PITCH;
  const int head0 = 32 * hg;
  uint16_t* obase = splits == 1 ? out + (size_t)r * H * DV
                                : o_part + ((size_t)r * splits + sp) * H * DV;
  // every wave is done with the last stage buffer before any overwrites it
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
  for (int hm = 0; hm < 2; ++hm) {
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int dt = 0; dt < DT_HALF; ++dt)
        *reinterpret_cast<uint16_t*>(ep + (4 * g + v) * EP_PITCH + 2 * (16 * dt + nn)) =
            bf16_bits(O[hm][dt][v]);
    // the wave reads back what it wrote (LDS operations of one wave are ordered)
    uint16_t* orow = obase + (size_t)(head0 + 16 * hm) * DV + 256 * hf;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int c = l + 64 * k, hr = c >> 5, j = c & 31;  // head row hr, piece j
      const i32x4 val = *reinterpret_cast<const i32x4*>(ep + hr * EP_PITCH + 16 * j);
      // streamed out: a split's partials are read once, by the combine, and the
      // output by the caller's next step; neither is worth keeping in the caches
      __builtin_nontemporal_store(val, reinterpret_cast<i32x4*>(orow + (size_t)hr * DV + 8 * j));
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next writes
  }
  float* lrow = splits == 1 ? lse : lse_part + ((size_t)r * splits + sp) * H - (size_t)r * H;
  if (lrow != nullptr && g == 0 && hf == 0) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
      lrow[(size_t)r * H + head0 + 16 * nt + nn] =
          l_tot[nt] > 0.f ? (m_run[nt] + __log2f(l_tot[nt])) * kLn2 : -INFINITY;
  }
}

// LSE-weighted merge of the splits: out = sum_i e^{lse_i - LSE} o_i.  64 threads per
// (row, head), four (row, head) pairs per block; each thread merges 8 output
// columns with 16-byte loads.  The split outputs o_i are bf16 (normalised, so
// |o_i| <= max |value|), their lse_i fp32; the merge runs in fp32.  The partials
// are loaded 8 at a time before any is used, so their latencies overlap.
constexpr int CMB_T = 64;                 // threads per (row, head)
constexpr int CMB_RH = 4;                 // (row, head) pairs per block
static_assert(DV == CMB_T * 8, "8 columns per thread");
__global__ __launch_bounds__(CMB_T * CMB_RH) void attn_combine_kernel(
    const uint16_t* __restrict__ o_part, const float* __restrict__ lse_part, int R, int splits,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int B8 = 8;
  const int rh = blockIdx.x * CMB_RH + (threadIdx.x / CMB_T);
  const int c8 = threadIdx.x % CMB_T;
  const int r = rh / H, h = rh - (rh / H) * H;
  if (r >= R) return;
  const float* lp = lse_part + (size_t)r * splits * H + h;
  const uint16_t* op = o_part + ((size_t)r * splits * H + h) * DV + 8 * c8;
  const size_t ostride = (size_t)H * DV;
  // one pass over batches of B8 splits, every load of a batch in flight at once;
  // the running max M rises per batch (a batch that raises it rescales what is
  // summed so far), so up to B8 splits take a single round trip
  float M = -INFINITY;
  float den = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < splits; s0 += B8) {
    uint4 v[B8];
    float x[B8];
#pragma unroll
    for (int i = 0; i < B8; ++i) {
      const int s = min(s0 + i, splits - 1);
      x[i] = s0 + i < splits ? lp[(size_t)s * H] : -INFINITY;
      const i32x4 raw = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(op + (size_t)s * ostride));
      v[i] = make_uint4((uint32_t)raw[0], (uint32_t)raw[1], (uint32_t)raw[2], (uint32_t)raw[3]);
    }
    float bm = M;
#pragma unroll
    for (int i = 0; i < B8; ++i) bm = fmaxf(bm, x[i]);
    if (bm > M) {
      // everything summed so far is zero while M is still -inf
      const float c = (M == -INFINITY) ? 0.f : __expf(M - bm);
      den *= c;
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] *= c;
      M = bm;
    }
#pragma unroll
    for (int i = 0; i < B8; ++i) {
      const float wgt = (x[i] == -INFINITY) ? 0.f : __expf(x[i] - M);
      den += wgt;
      const uint32_t u[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[2 * k] += wgt * __uint_as_float(u[k] << 16);
        acc[2 * k + 1] += wgt * __uint_as_float(u[k] & 0xffff0000u);
      }
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  uint4 pk;
  pk.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  pk.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  pk.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
  pk.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
  *reinterpret_cast<uint4*>(out + ((size_t)r * H + h) * DV + 8 * c8) = pk;
  if (lse != nullptr && c8 == 0)
    lse[(size_t)r * H + h] = den > 0.f ? M + __logf(den) : -INFINITY;
}

// ---------------------------------------------------------------------------
// fp32 correctness path (any H <= 128, D_v <= D_k <= 576, topk <= 2048):
// one block per (row, head), two-pass softmax.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ latent,
    const int32_t* __restrict__ indices, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_pos, int B, int N, int nh, int dk, int dv, int topk,
    float scale, float* __restrict__ out, float* __restrict__ lse) {
  __shared__ float z[kTopk];
  __shared__ int pos[kTopk];
  __shared__ float qs[kQkDim];
  __shared__ float red[8];
  const int r = blockIdx.x / nh, h = blockIdx.x - (blockIdx.x / nh) * nh;
  const int b = row_seq[r], t = row_pos[r];
  if (b < 0 || b >= B || t < 0 || t >= N) return;
  const int tid = threadIdx.x, l = lane_id(), wv = tid >> 6;
  for (int d = tid; d < dk; d += 256) qs[d] = q[((size_t)r * nh + h) * dk + d];
  __syncthreads();
  const float* lat = latent + (size_t)b * N * dk;
  float mx = -INFINITY;
  for (int i = tid; i < topk; i += 256) {
    const int p = indices[(size_t)r * topk + i];
    const bool ok = p >= 0 && p <= t;  // entries outside [0, t] are padding
    if (p > t) flag_index_domain();
    float s = -INFINITY;
    if (ok) {
      float dot = 0.f;
      for (int d = 0; d < dk; ++d) dot = fmaf(qs[d], lat[(size_t)p * dk + d], dot);
      s = dot * scale;
    }
    z[i] = s;
    pos[i] = ok ? p : -1;
    mx = fmaxf(mx, s);
  }
  mx = wave_max(mx);
  if (l == 0) red[wv] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float sum = 0.f;
  for (int i = tid; i < topk; i += 256) {
    const float e = pos[i] >= 0 ? expf(z[i] - mx) : 0.f;
    z[i] = e;
    sum += e;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
  if (l == 0) red[4 + wv] = sum;
  __syncthreads();
  sum = red[4] + red[5] + red[6] + red[7];
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  for (int d = tid; d < dv; d += 256) {
    float acc = 0.f;
    for (int i = 0; i < topk; ++i)
      if (pos[i] >= 0) acc = fmaf(z[i], lat[(size_t)pos[i] * dk + d], acc);
    out[((size_t)r * nh + h) * dv + d] = acc * inv;
  }
  if (lse != nullptr && tid == 0)
    lse[(size_t)r * nh + h] = sum > 0.f ? mx + logf(sum) : -INFINITY;
}

int splits_override() {
  static const int v = [] {
    const char* e = getenv("DSA_ATTN_SPLITS");
    return e ? atoi(e) : 0;
  }();
  return v;
}

}  // namespace

int attn_num_splits(int num_rows, int topk) {
  const int nblk = topk / BE;
  int s = splits_override();
  if (s <= 0) {
    // one block per CU in flight: aim for >= 256 blocks, but give a block at least 4
    // stages while >= 128 blocks remain.  A block's fixed cost (the query load and
    // the first gather) dominates shorter ones, and twice the splits double the
    // partials the combine reads (decode 128K, 8 rows: 16 splits 71.9 us per step,
    // 32 splits 74.7 us; decode 32K, 32 rows, keeps 8 splits of 8 stages).
    s = 1;
    while (s < nblk && (int64_t)num_rows * s < 256) s <<= 1;
    while (s > 1 && nblk / s < 4 && (int64_t)num_rows * (s / 2) >= 128) s >>= 1;
  }
  while (s > 1 && (nblk % s) != 0) s >>= 1;
  return s < 1 ? 1 : s;
}

size_t attn_workspace_bytes(int num_rows, const dsa_dims& dims) {
  if (dims.attn_dtype != DSA_BF16) return 0;
  const int s = attn_num_splits(num_rows, dims.topk);
  if (s <= 1) return 0;
  // bf16 split outputs [R, S, H, D_v] followed by fp32 split lse [R, S, H]
  return (size_t)num_rows * s * H * (DV * sizeof(uint16_t) + sizeof(float));
}

hipError_t launch_attn_bf16(const dsa_rows& rows, const void* q, const void* latent,
                            const int32_t* indices, float softmax_scale, void* out, float* lse,
                            void* workspace, hipStream_t stream, const PageMap& pm) {
  const int R = rows.num_rows;
  const int S = attn_num_splits(R, kTopk);
  uint16_t* o_part = nullptr;
  float* lse_part = nullptr;
  if (S > 1) {
    o_part = static_cast<uint16_t*>(workspace);
    lse_part = reinterpret_cast<float*>(o_part + (size_t)R * S * H * DV);
  }
  const int row_groups = (R + 7) / 8;
  const float scale_log2 = softmax_scale * 1.44269504088896340736f;
  auto kern = pm.table != nullptr ? attn_bf16_kernel<true> : attn_bf16_kernel<false>;
  hipLaunchKernelGGL(kern, dim3(row_groups * 8 * S), dim3(NT), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(latent), indices,
                     rows.row_seq, rows.row_pos, R, rows.num_seqs, rows.max_ctx, kTopk, S,
                     scale_log2, static_cast<uint16_t*>(out), lse, o_part, lse_part, pm);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || S == 1) return err;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((R * H + CMB_RH - 1) / CMB_RH), dim3(CMB_T * CMB_RH),
                     0, stream, o_part, lse_part, R, S, static_cast<uint16_t*>(out), lse);
  return hipGetLastError();
}

hipError_t read_index_domain_flag(uint32_t* seen) {
  hipError_t err = hipDeviceSynchronize();
  if (err != hipSuccess) return err;
  uint32_t v = 0u;
  err = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_index_domain_flag), sizeof(v), 0, hipMemcpyDeviceToHost);
  if (err != hipSuccess) return err;
  const uint32_t zero = 0u;
  err = hipMemcpyToSymbol(HIP_SYMBOL(g_index_domain_flag), &zero, sizeof(zero), 0, hipMemcpyHostToDevice);
  if (err != hipSuccess) return err;
  *seen = v;
  return hipDeviceSynchronize();
}

hipError_t launch_attn_f32(const dsa_rows& rows, const dsa_dims& dims, const float* q,
                           const float* latent, const int32_t* indices, float softmax_scale,
                           float* out, float* lse, hipStream_t stream) {
  hipLaunchKernelGGL(attn_f32_kernel, dim3(rows.num_rows * dims.n_heads), dim3(256), 0, stream, q,
                     latent, indices, rows.row_seq, rows.row_pos, rows.num_seqs, rows.max_ctx,
                     dims.n_heads, dims.qk_dim, dims.v_dim, dims.topk, softmax_scale, out, lse);
  return hipGetLastError();
}

}  // namespace dsa
