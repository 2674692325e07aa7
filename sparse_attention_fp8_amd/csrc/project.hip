// Projections of new tokens with fused fp8 quantisation and cache append.
//
// The first step of the four-step DSA workflow (query and key projection, then
// indexer scoring, top-k selection and sparse MLA; "DeepSeek-V3.2开源技术报告",
// "DSA principle").  The indexer query heads q[t,j] and head weights w[t,j] are
// derived from the token h_t and the indexer key k[s] from h_s (DeepSeek-V3.2-Exp
// paper, section 1, text around Eq. 1); the latent entry c_s is derived from h_s
// as well.  All four are linear maps of h, computed here as one GEMM
//   y[r, :] = W h[r]   with W = [w_q; w_k; w_c; w_w]  (8192 + 128 + 576 + 64 rows)
// on bf16 MFMA with fp32 accumulation.  The epilogue stores every output in the
// format the later steps read:
//   q heads  -> e4m3fn codes + one power-of-two fp32 scale per (token, head)
//   k        -> e4m3fn codes + scale per token, written into the key cache row
//   latent   -> bf16 (round to nearest even), written into the latent cache row
//   w        -> fp32
// The quantiser takes scale = 2^e with the smallest e such that amax <= 448 * 2^e
// (amax over the 128-wide vector; 1 when amax = 0) and code = RNE(y / scale), so
// the division is exact and the fp8 cast is the only rounding.
//
// Layout: h [R, d] and every weight matrix [rows, d] are K-contiguous, the natural
// layout of both MFMA operands.  A block computes a tile of ROWS tokens x COLS
// outputs: the h tile is shared by the block's four waves through LDS, while the
// weight rows (each read by one wave only) go straight from global memory into
// registers, several 64-element chunks ahead.  With few tokens (decode) the
// weights dominate the traffic (~128 MB at d = 7168) and the contraction is split
// over blocks, whose fp32 partial sums a second kernel adds in a fixed order
// before the same epilogue.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kColK = kIdxHeads * kIdxDim;  // 8192: first indexer-key column
constexpr int kColC = kColK + kIdxDim;      // 8320: first latent column
constexpr int kColW = kColC + kQkDim;       // 8896: first head-weight column
constexpr int kCols = kColW + kIdxHeads;    // 8960 outputs per token
constexpr int KC = 64;                      // contraction elements per chunk (128 bytes)
constexpr int NTH = 256;                    // 4 waves per block

struct ProjParams {
  const uint16_t* h;
  const uint16_t* wq;
  const uint16_t* wk;
  const uint16_t* wc;
  const uint16_t* ww;
  const int32_t* row_seq;
  const int32_t* row_pos;
  int R, d, B, N;
  uint8_t* q_idx;
  float* q_scale;
  float* w_out;
  uint8_t* k_idx;
  float* k_scale;
  uint16_t* latent;
  float* part;  // [ksplit][R][kCols] partial sums (split contraction only)
  int ksplit;
  int mtiles, ntiles;  // tile grid of the GEMM launch
  PageMap pm;   // cache rows: contiguous (table == nullptr) or a page pool
};

// cache row of token r, or -1 when its (sequence, position) is out of range
__device__ __forceinline__ int64_t cache_row(const ProjParams& p, int r) {
  const int b = p.row_seq[r], t = p.row_pos[r];
  if (b < 0 || b >= p.B || t < 0 || t >= p.N) return -1;
  return p.pm.table != nullptr ? (int64_t)paged_row(p.pm, b, t) : (int64_t)b * p.N + t;
}

__device__ __forceinline__ const uint16_t* weight_row(const ProjParams& p, int col) {
  const uint16_t* base;
  int r;
  if (col < kColK) {
    base = p.wq;
    r = col;
  } else if (col < kColC) {
    base = p.wk;
    r = col - kColK;
  } else if (col < kColW) {
    base = p.wc;
    r = col - kColC;
  } else {
    base = p.ww;
    r = col - kColW;
  }
  return base + (size_t)r * p.d;
}

// e4m3fn code of x, |x| <= 448, round to nearest even.  Normal range: round the
// float32 mantissa to 3 bits and rebias the exponent (127 -> 7); below 2^-6 the
// codes are the multiples of 2^-9, so rint(|x| * 512) is the code itself.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  uint32_t u = __float_as_uint(a);
  u += 0x7FFFFu + ((u >> 20) & 1u);
  const uint32_t normal = (u >> 20) - (120u << 3);
  const uint32_t sub = (uint32_t)__builtin_rintf(a * 512.0f);
  return sign | (a < 0x1p-6f ? sub : normal);
}

// Smallest e with amax <= 448 * 2^e (0 for amax = 0), clamped to the range where
// 2^e and 2^-e are normal floats.  amax = (1 + M / 2^23) 2^(E - 127) and
// 448 = 1.75 * 2^8, so e = E - 135, plus one when the mantissa exceeds 0.75.
__device__ __forceinline__ int pow2_exponent(float amax) {
  const uint32_t u = __float_as_uint(amax);
  if (u == 0u) return 0;
  const int e = (int)(u >> 23) - 135 + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return min(max(e, -126), 126);
}

// Epilogue for V consecutive outputs col .. col+V-1 of token r held by this
// thread.  The 128 / V threads that share a 128-wide vector are consecutive lanes
// of one DPP row, so the vector's amax is a 3- or 4-step lane reduction.  Every
// lane takes part in the reduction; only valid ones store.
template <int V>
__device__ __forceinline__ void finish(const ProjParams& p, const float (&v)[V], int r, int col,
                                       bool valid) {
  static_assert(V == 8 || V == 16, "8 or 16 outputs per thread");
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < V; ++i) m = fmaxf(m, fabsf(v[i]));
  // non-negative floats order like their bit patterns; absent lanes give 0
  uint32_t mb = __float_as_uint(m);
  mb = max(mb, dpp<kDppXor1>(mb));
  mb = max(mb, dpp<kDppXor2>(mb));
  mb = max(mb, dpp<kDppHalfMirror>(mb));
  if constexpr (V == 8) mb = max(mb, dpp<kDppMirror>(mb));
  if (!valid) return;

  if (col < kColC) {  // indexer query head or indexer key: quantise
    const int e = pow2_exponent(__uint_as_float(mb));
    const float inv = __uint_as_float((uint32_t)(127 - e) << 23);
    const float scale = __uint_as_float((uint32_t)(127 + e) << 23);
    uint32_t words[V / 4];
#pragma unroll
    for (int i = 0; i < V / 4; ++i) {
      uint32_t w = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float x = fminf(fmaxf(v[4 * i + b] * inv, -448.0f), 448.0f);
        w |= e4m3_code(x) << (8 * b);
      }
      words[i] = w;
    }
    uint8_t* dst;
    float* sdst;
    if (col < kColK) {
      dst = p.q_idx + (size_t)r * kColK + col;
      sdst = p.q_scale + (size_t)r * kIdxHeads + col / kIdxDim;
    } else {
      const int64_t row = cache_row(p, r);
      if (row < 0) return;
      dst = p.k_idx + (size_t)row * kIdxDim + (col - kColK);
      sdst = p.k_scale + row;
    }
    if constexpr (V == 16) {
      *reinterpret_cast<uint4*>(dst) = make_uint4(words[0], words[1], words[2], words[3]);
    } else {
      *reinterpret_cast<uint2*>(dst) = make_uint2(words[0], words[1]);
    }
    if ((col & (kIdxDim - 1)) == 0) *sdst = scale;
  } else if (col < kColW) {  // latent entry: bf16 into the cache row
    const int64_t row = cache_row(p, r);
    if (row < 0) return;
    uint16_t* dst = p.latent + (size_t)row * kQkDim + (col - kColC);
#pragma unroll
    for (int i = 0; i < V / 8; ++i)
      reinterpret_cast<uint4*>(dst)[i] =
          make_uint4(pack_bf16x2(v[8 * i + 0], v[8 * i + 1]), pack_bf16x2(v[8 * i + 2], v[8 * i + 3]),
                     pack_bf16x2(v[8 * i + 4], v[8 * i + 5]), pack_bf16x2(v[8 * i + 6], v[8 * i + 7]));
  } else {  // head weights: fp32
    float* dst = p.w_out + (size_t)r * kIdxHeads + (col - kColW);
#pragma unroll
    for (int i = 0; i < V / 4; ++i)
      reinterpret_cast<float4*>(dst)[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  }
}

// Tile of a block in a 1-D grid of mtiles * ntiles blocks.  Blocks are dealt to the
// 8 XCDs round-robin, so the block ids are first regrouped to give each XCD a
// contiguous run of tiles; the run is walked in groups of 8 token tiles, output
// tile by output tile, so the ~32 blocks an XCD runs at once share 4 weight tiles
// and 8 h tiles through its L2 instead of each fetching its own.
__device__ __forceinline__ void tile_of_block(const ProjParams& p, int L, int G, int& m, int& n) {
  constexpr int GM = 8;
  const int id = (G % 8 == 0) ? (L % 8) * (G / 8) + L / 8 : L;
  const int per_group = GM * p.ntiles;
  const int first_m = (id / per_group) * GM;
  const int gm = min(p.mtiles - first_m, GM);
  const int in = id % per_group;
  m = first_m + in % gm;
  n = in / gm;
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Tile of 16*MT tokens x 64*NS outputs over the chunks of split blockIdx.z.
// Wave w owns outputs [16*NS*w, 16*NS*(w+1)) of the tile, all tokens.  Weight
// chunks are prefetched PD chunks ahead into registers; h chunks ride along in
// the same register ring and are copied into a double-buffered LDS tile one chunk
// ahead (16-byte pieces XOR-swizzled by row so that the fragment reads of 16 rows
// spread over the banks).
template <int MT, int NS, int PD>
__global__ __launch_bounds__(NTH) void proj_gemm_kernel(ProjParams p) {
  constexpr int ROWS = 16 * MT;
  constexpr int COLS = 64 * NS;
  constexpr int APT = ROWS * 8 / NTH;  // 16-byte h pieces per thread and chunk
  constexpr int V = 4 * NS;            // epilogue outputs per thread
  static_assert(APT >= 1 && (ROWS * 8) % NTH == 0, "tile rows");
  __shared__ __attribute__((aligned(16))) uint4 abuf[2][ROWS * 8];
  __shared__ __attribute__((aligned(16))) float etile[16][COLS + 4];

  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63;
  const int g = l >> 4, ln = l & 15;
  int mt_i, nt_i;
  tile_of_block(p, blockIdx.x, gridDim.x, mt_i, nt_i);
  const int n0 = nt_i * COLS, m0 = mt_i * ROWS, ks = blockIdx.z;
  const int nch = p.d / KC;
  const int c0 = (int)((int64_t)nch * ks / p.ksplit);
  const int c1 = (int)((int64_t)nch * (ks + 1) / p.ksplit);

  const uint16_t* wrow[NS];
#pragma unroll
  for (int ns = 0; ns < NS; ++ns) wrow[ns] = weight_row(p, n0 + wv * 16 * NS + 16 * ns + ln) + 8 * g;
  const uint16_t* hrow[APT];
  int aslot[APT];
#pragma unroll
  for (int i = 0; i < APT; ++i) {
    const int pc = tid + NTH * i, row = pc >> 3, c = pc & 7;
    const int tok = min(m0 + row, p.R - 1);  // rows past the end repeat the last token
    hrow[i] = p.h + (size_t)tok * p.d + 8 * c;
    aslot[i] = row * 8 + (c ^ (row & 7));
  }

  i32x4 wr[PD][NS][2];
  i32x4 ar[PD][APT];
  f32x4 acc[MT][NS];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) acc[mt][ns] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto issue = [&](int slot, int ch) {
#pragma unroll
    for (int ns = 0; ns < NS; ++ns)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        wr[slot][ns][hf] = *reinterpret_cast<const i32x4*>(wrow[ns] + (size_t)ch * KC + 32 * hf);
#pragma unroll
    for (int i = 0; i < APT; ++i)
      ar[slot][i] = *reinterpret_cast<const i32x4*>(hrow[i] + (size_t)ch * KC);
  };

  // The main loop body has no data-dependent branch, so the compiler's wait
  // counts stay exact across iterations: a split of n chunks runs n / PD full
  // groups, then up to PD - 1 chunks with guards.  Loads past the last chunk repeat
  // it (cache hits; never consumed).
  const int n = c1 - c0;  // >= 1 chunks in this split
  const int groups = n / PD;
  auto step = [&](int q, int j) {
    const i32x4* ab = reinterpret_cast<const i32x4*>(abuf[j & 1]);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int row = 16 * mt + ln;
        const bf16x8 a = as_bf16x8(ab[row * 8 + ((4 * s + g) ^ (row & 7))]);
#pragma unroll
        for (int ns = 0; ns < NS; ++ns)
          acc[mt][ns] = mfma_bf16_16x16x32(a, as_bf16x8(wr[q][ns][s]), acc[mt][ns]);
      }
    issue(q, c0 + min(j + PD, n - 1));
    // keep the new loads ahead of the LDS stores below, so that waiting for the
    // next h tile leaves them in flight
    asm volatile("" ::: "memory");
    i32x4* nb = reinterpret_cast<i32x4*>(abuf[(j + 1) & 1]);
#pragma unroll
    for (int i = 0; i < APT; ++i) nb[aslot[i]] = ar[(q + 1) % PD][i];
    lds_barrier();
  };
#pragma unroll
  for (int q = 0; q < PD; ++q) issue(q, c0 + min(q, n - 1));
#pragma unroll
  for (int i = 0; i < APT; ++i) reinterpret_cast<i32x4*>(abuf[0])[aslot[i]] = ar[0][i];
  lds_barrier();
  for (int gi = 0; gi < groups; ++gi) {
#pragma unroll
    for (int q = 0; q < PD; ++q) step(q, gi * PD + q);
  }
#pragma unroll
  for (int q = 0; q + 1 < PD; ++q)
    if (groups * PD + q < n) step(q, groups * PD + q);

  // epilogue, one 16-token slab at a time through LDS
  const int erow = tid >> 4, eseg = tid & 15;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int ns = 0; ns < NS; ++ns)
#pragma unroll
      for (int v = 0; v < 4; ++v) etile[4 * g + v][wv * 16 * NS + 16 * ns + ln] = acc[mt][ns][v];
    lds_barrier();
    float vals[V];
#pragma unroll
    for (int i = 0; i < V / 4; ++i) {
      const float4 x = reinterpret_cast<const float4*>(&etile[erow][eseg * V])[i];
      vals[4 * i] = x.x;
      vals[4 * i + 1] = x.y;
      vals[4 * i + 2] = x.z;
      vals[4 * i + 3] = x.w;
    }
    const int r = m0 + 16 * mt + erow, col = n0 + eseg * V;
    if (p.ksplit > 1) {
      if (r < p.R) {
        float* dst = p.part + ((size_t)ks * p.R + r) * kCols + col;
#pragma unroll
        for (int i = 0; i < V / 4; ++i)
          reinterpret_cast<float4*>(dst)[i] =
              make_float4(vals[4 * i], vals[4 * i + 1], vals[4 * i + 2], vals[4 * i + 3]);
      }
    } else {
      finish<V>(p, vals, r, col, r < p.R);
    }
    lds_barrier();
  }
}

// Sum of the split partials in split order, then the epilogue: block = 16 tokens x
// 64*NS outputs, thread = V consecutive outputs of one token.
template <int NS>
__global__ __launch_bounds__(NTH) void proj_finish_kernel(ProjParams p) {
  constexpr int V = 4 * NS, COLS = 64 * NS;
  const int tid = threadIdx.x;
  const int r = blockIdx.y * 16 + (tid >> 4), col = blockIdx.x * COLS + (tid & 15) * V;
  float vals[V];
#pragma unroll
  for (int i = 0; i < V; ++i) vals[i] = 0.0f;
  if (r < p.R) {
    for (int ks = 0; ks < p.ksplit; ++ks) {
      const float4* src = reinterpret_cast<const float4*>(p.part + ((size_t)ks * p.R + r) * kCols + col);
#pragma unroll
      for (int i = 0; i < V / 4; ++i) {
        const float4 x = src[i];
        vals[4 * i] += x.x;
        vals[4 * i + 1] += x.y;
        vals[4 * i + 2] += x.z;
        vals[4 * i + 3] += x.w;
      }
    }
  }
  finish<V>(p, vals, r, col, r < p.R);
}

// Launch shape for R tokens and width d: large token counts take 128 x 256 tiles
// with the whole contraction per block; small ones 32 x 128 tiles, with the
// contraction split until about 512 blocks are in flight.
constexpr int kBigRows = 1024;

struct ProjShape {
  bool big;
  int ksplit;
};

ProjShape proj_shape(int R, int d) {
  if (R >= kBigRows) return {true, 1};
  const int tiles = (kCols / 128) * ((R + 31) / 32);
  const int nch = d / KC;
  int ks = 512 / tiles;
  ks = ks < 1 ? 1 : ks;
  ks = ks > nch / 4 ? nch / 4 : ks;  // at least 4 chunks per split
  return {false, ks < 1 ? 1 : ks};
}

}  // namespace

size_t project_workspace_bytes(int num_rows, int d_model) {
  if (num_rows <= 0 || d_model < KC) return 0;
  const ProjShape s = proj_shape(num_rows, d_model);
  return s.ksplit > 1 ? (size_t)s.ksplit * num_rows * kCols * sizeof(float) : 0;
}

hipError_t launch_project(const dsa_rows& rows, int d_model, const uint16_t* h, const uint16_t* wq,
                          const uint16_t* wk, const uint16_t* wc, const uint16_t* ww, uint8_t* q_idx,
                          float* q_scale, float* w, uint8_t* k_idx, float* k_scale,
                          uint16_t* latent, void* workspace, hipStream_t stream,
                          const PageMap& pm) {
  const int R = rows.num_rows;
  if (R == 0) return hipSuccess;
  const ProjShape s = proj_shape(R, d_model);
  ProjParams p{h, wq, wk, wc, ww, rows.row_seq, rows.row_pos, R, d_model, rows.num_seqs,
               rows.max_ctx, q_idx, q_scale, w, k_idx, k_scale, latent,
               static_cast<float*>(workspace), s.ksplit, 0, 0, pm};
  if (s.big) {
    p.mtiles = (R + 127) / 128;
    p.ntiles = kCols / 256;
    proj_gemm_kernel<8, 4, 2><<<dim3(p.mtiles * p.ntiles, 1, 1), NTH, 0, stream>>>(p);
  } else {
    p.mtiles = (R + 31) / 32;
    p.ntiles = kCols / 128;
    proj_gemm_kernel<2, 2, 4><<<dim3(p.mtiles * p.ntiles, 1, s.ksplit), NTH, 0, stream>>>(p);
    if (s.ksplit > 1) {
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      proj_finish_kernel<2><<<dim3(kCols / 128, (R + 15) / 16), NTH, 0, stream>>>(p);
    }
  }
  return hipGetLastError();
}

}  // namespace dsa
