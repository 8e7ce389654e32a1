// libroutedfp4, batched path: the routed experts of many tokens at once as
// grouped GEMMs on the CDNA4 matrix cores.
//
// Used for C >= 2 tokens per call (decode batches and prefill chunks).  The
// layer is the same as the decode path's (page "Kimi-K3 on 2x A40 -- measured
// findings", section "Why the placement experiments all looked the same":
// MUL_MAT_ID over the selected experts; page "SparkInfer-K3", section "How the
// TP module works": router -> top-k -> experts -> sum), arranged so that every
// selected expert's weights are read once per tile of the tokens that chose it
// (page "Kimi-K3 on the same pod, two engines", section "Where our build is
// still ahead": a batched prompt pass reads each expert once per chunk).
//
// Exactness.  Every weight e2m1 * scale is exact in bf16 (NVFP4: at most 6
// significant bits; MXFP4: a power-of-two scale), so the weights go to the
// matrix cores as bf16 without rounding.  Activations are fp32: each is split
// into three bf16 pieces whose sum is the fp32 value exactly (8 + 8 + 8
// significant bits), and each piece is multiplied separately; a piece that is
// zero for every token of a tile (bf16-exact input) is skipped.  Products are
// therefore exact and only the fp32 accumulation rounds.  The NVFP4 per-tensor
// scale multiplies the accumulated sums.
//
// Kernels, in stream order:
//   k_bsplit    x -> three bf16 planes + per-token flags (zeroes the counters)
//   k_bcount    (token, slot) pairs per expert
//   k_bscan     offsets and the tile list (each expert's pairs in tiles of
//               16 or 64)
//   k_bscatter  pairs grouped by expert
//   k_bgu       per (tile, 64 rows of I): gate and up on MFMA, SwiGLU, h as
//               three bf16 planes
//   k_bdn       per (tile, 64 rows of H): down on MFMA, times the routing
//               weight, one fp32 row per pair
//   k_bcombine  out[t] = sum of its pairs' rows in slot order (deterministic)
// and for the router of many tokens:
//   k_brouter   logits = x * W_r^T with fp32 MFMA
//   k_btopk     one wave per token: the same exact top-k as the decode path
#include "common.h"

namespace rf4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBK = 128;             // K elements per block: 64 code bytes of a row
constexpr int kBRows = 64;           // weight rows per workgroup (16 per wave)
constexpr int kXStride = kBK + 8;    // bf16 per staged activation row (272 B)
constexpr int kRK = 32;              // router: K elements per staged chunk

struct BArgs {
  const uint8_t* base;
  int64_t stride;
  int64_t off[MOE_NUM_TENSORS];
  int E, H, I, k, C;
  const int32_t* idx;     // [C][k]
  const float* w;         // [C][k]
  const float* x;         // [C][H]
  uint16_t* xp;           // [3][C][H] bf16 planes of x
  uint32_t* xflag;        // [C]: bit 0 plane 1 non-zero, bit 1 plane 2 non-zero
  uint16_t* hp;           // [3][C*k][I] bf16 planes of h
  float* part;            // [C*k][H]
  float* out;             // [C][H]
  uint32_t* count;        // [E]
  uint32_t* cursor;       // [E]
  uint32_t* boff;         // [E+1]
  uint32_t* meta;         // [0]: number of tiles
  int32_t* tiles;         // [tiles][2]: expert, first pair within the expert
  int32_t* perm;          // [C*k]: pairs grouped by expert
  int ntok;               // tokens per tile
};

// bf16 (round to nearest even) of an fp32 value, as its 16 bits.
__device__ __forceinline__ uint16_t bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ float bf16_float(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// f = p0 + p1 + p2 exactly (finite f, |f| >= 2^-100): each remainder is exact
// in fp32 (Sterbenz) and the last has at most 8 significant bits.
__device__ __forceinline__ void split3(float f, uint16_t& p0, uint16_t& p1, uint16_t& p2) {
  p0 = bf16_bits(f);
  const float r1 = f - bf16_float(p0);
  p1 = bf16_bits(r1);
  const float r2 = r1 - bf16_float(p1);
  p2 = bf16_bits(r2);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t view(const uint8_t* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), (short)0, (int)bytes, 0x00020000);
}

// Eight weights (dword `wd` of a lane's 16 code bytes) as the bf16 A operand.
// MXFP4: one e8m0 byte `sc` for the lane's 32 elements; the convert applies a
// power-of-two scale exactly.  NVFP4: e4m3 byte `sc` for these 16 elements;
// e2m1 * e4m3 is exact in fp32 and in bf16.
template <int FMT>
__device__ __forceinline__ bf16x8_t dequant8(uint32_t wd, uint32_t sc) {
  bf16x8_t r;
  if (FMT == MOE_FMT_MXFP4) {
    const float s = __uint_as_float((sc & 0xFFu) << 23);   // 2^(sc-127), exponent field only
    const bf16x2_t a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, s, 0);
    const bf16x2_t a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, s, 1);
    const bf16x2_t a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, s, 2);
    const bf16x2_t a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, s, 3);
    r[0] = a0[0]; r[1] = a0[1]; r[2] = a1[0]; r[3] = a1[1];
    r[4] = a2[0]; r[5] = a2[1]; r[6] = a3[0]; r[7] = a3[1];
  } else {
    const float s = e4m3_to_f32(sc);
    const float2 v0 = fp4x2<0>(wd), v1 = fp4x2<1>(wd), v2 = fp4x2<2>(wd), v3 = fp4x2<3>(wd);
    r[0] = (__bf16)(v0.x * s); r[1] = (__bf16)(v0.y * s);
    r[2] = (__bf16)(v1.x * s); r[3] = (__bf16)(v1.y * s);
    r[4] = (__bf16)(v2.x * s); r[5] = (__bf16)(v2.y * s);
    r[6] = (__bf16)(v3.x * s); r[7] = (__bf16)(v3.y * s);
  }
  return r;
}

__device__ __forceinline__ bf16x8_t lds_bf16x8(const uint16_t* p) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ uint32_t scale_word(const uint4& q, int s) {
  return s == 0 ? q.x : s == 1 ? q.y : s == 2 ? q.z : q.w;
}

// Workgroup-wide exclusive scan (blockDim.x = 1024, 16 waves).
__device__ int block_excl_scan_1024(int v, int* s_w, int* total) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int incl = wave_incl_scan(v);
  if (lane == 63) s_w[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int t = lane < 16 ? s_w[lane] : 0;
    const int ti = wave_incl_scan(t);
    if (lane < 16) s_w[16 + lane] = ti - t;
    if (lane == 15) s_w[32] = ti;
  }
  __syncthreads();
  const int r = s_w[16 + wave] + incl - v;
  *total = s_w[32];
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------------------
// Dispatch
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bsplit(BArgs a) {
  const int t = blockIdx.x, H = a.H;
  if (t == 0)
    for (int e = threadIdx.x; e < a.E; e += 256) { a.count[e] = 0u; a.cursor[e] = 0u; }
  const size_t plane = (size_t)a.C * H;
  int nz = 0;
  for (int i = threadIdx.x * 4; i < H; i += 256 * 4) {
    const float4 v = *reinterpret_cast<const float4*>(a.x + (size_t)t * H + i);
    const float f[4] = {v.x, v.y, v.z, v.w};
    uint16_t p[3][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) split3(f[j], p[0][j], p[1][j], p[2][j]);
#pragma unroll
    for (int pl = 0; pl < 3; ++pl) {
      const uint2 u = make_uint2((uint32_t)p[pl][0] | ((uint32_t)p[pl][1] << 16),
                                 (uint32_t)p[pl][2] | ((uint32_t)p[pl][3] << 16));
      *reinterpret_cast<uint2*>(a.xp + pl * plane + (size_t)t * H + i) = u;
      if (pl > 0 && (u.x | u.y) != 0u) nz |= pl;
    }
  }
  const uint32_t f1 = __syncthreads_or(nz & 1) ? 1u : 0u;
  const uint32_t f2 = __syncthreads_or(nz & 2) ? 2u : 0u;
  if (threadIdx.x == 0) a.xflag[t] = f1 | f2;
}

__global__ __launch_bounds__(256) void k_bcount(BArgs a) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= a.C * a.k) return;
  const int e = a.idx[p];
  if (e >= 0 && e < a.E) atomicAdd(&a.count[e], 1u);
}

__global__ __launch_bounds__(1024) void k_bscan(BArgs a) {
  __shared__ int s_w[48];
  const int e = threadIdx.x;
  const int c = e < a.E ? (int)a.count[e] : 0;
  const int nt = (c + a.ntok - 1) / a.ntok;
  int npairs = 0, ntiles = 0;
  const int off = block_excl_scan_1024(c, s_w, &npairs);
  const int toff = block_excl_scan_1024(nt, s_w, &ntiles);
  if (e < a.E) {
    a.boff[e] = (uint32_t)off;
    for (int i = 0; i < nt; ++i) {
      a.tiles[2 * (toff + i)] = e;
      a.tiles[2 * (toff + i) + 1] = i * a.ntok;
    }
  }
  if (e == 0) {
    a.boff[a.E] = (uint32_t)npairs;
    a.meta[0] = (uint32_t)ntiles;
  }
}

__global__ __launch_bounds__(256) void k_bscatter(BArgs a) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= a.C * a.k) return;
  const int e = a.idx[p];
  if (e >= 0 && e < a.E) a.perm[a.boff[e] + atomicAdd(&a.cursor[e], 1u)] = p;
}

// ---------------------------------------------------------------------------
// Grouped GEMMs
// ---------------------------------------------------------------------------
// Shared structure of k_bgu and k_bdn.  A workgroup owns one tile (up to NTOK
// pairs of one expert) and 64 rows of one weight matrix (two for gate/up);
// wave w owns rows 16w..16w+15.  The K dimension runs in blocks of 128: lane l
// reads 16 code bytes of row (l % 16) at K offset 32 * (l / 16) of the block,
// and MFMA step s (0..3) uses its elements 8s..8s+7.  The activations are
// staged in LDS with the same K order, so A and B agree on which K each slot
// of the 16x16x32 product holds.  Weight loads run one block ahead.
template <int NR>
struct WeightRows {
  __amdgpu_buffer_rsrc_t codes[NR], scales[NR];
  uint32_t coff, soff;       // this lane's offsets in block 0
  int cstep, sstep;          // bytes per K block (codes, scales)
};

template <int FMT, int NR>
__device__ __forceinline__ void load_block(const WeightRows<NR>& W, int kb, uint4 (&q)[NR],
                                           uint32_t (&sc)[NR]) {
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(W.codes[r], (int)(W.coff + kb * W.cstep), 0,
                                                         kCachePolicyNt);
    q[r] = make_uint4(v[0], v[1], v[2], v[3]);
    if (FMT == MOE_FMT_MXFP4)
      sc[r] = __builtin_amdgcn_raw_buffer_load_b8(W.scales[r], (int)(W.soff + kb * W.sstep), 0,
                                                  kCachePolicyNt);
    else
      sc[r] = __builtin_amdgcn_raw_buffer_load_b16(W.scales[r], (int)(W.soff + kb * W.sstep), 0,
                                                   kCachePolicyNt);
  }
}

// acc[r][nb] += rows r (this wave's 16) x staged columns nb*16..nb*16+15 over
// one K block, for planes 0..np-1 of the staged activations.
template <int FMT, int NR, int NB, int NTOK>
__device__ __forceinline__ void mfma_block(const uint4 (&q)[NR], const uint32_t (&sc)[NR],
                                           const uint16_t (*xs)[NTOK][kXStride], int np,
                                           f32x4_t (&acc)[NR][NB]) {
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    bf16x8_t A[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const uint32_t sb = (FMT == MOE_FMT_MXFP4) ? sc[r] : ((sc[r] >> (8 * (s >> 1))) & 0xFFu);
      A[r] = dequant8<FMT>(scale_word(q[r], s), sb);
    }
    for (int pl = 0; pl < np; ++pl) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const bf16x8_t B = lds_bf16x8(&xs[pl][nb * 16 + r16][32 * g + 8 * s]);
#pragma unroll
        for (int r = 0; r < NR; ++r)
          acc[r][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[r], B, acc[r][nb], 0, 0, 0);
      }
    }
  }
}

struct TileInfo {
  int e, cnt, np;
};

// The tile of this workgroup: its expert, its pairs (s_pair) and the rows
// of the staged source each column reads (s_row); zero-fills the stage.
template <int NTOK>
__device__ __forceinline__ bool tile_setup(const BArgs& a, bool rows_are_tokens, uint16_t* xs_flat,
                                           int xs_words, int* s_pair, int* s_row, int* s_flags,
                                           TileInfo& T) {
  const int tile = blockIdx.y;
  if (tile >= (int)a.meta[0]) return false;
  T.e = a.tiles[2 * tile];
  const int t0 = a.tiles[2 * tile + 1];
  T.cnt = min(NTOK, (int)a.count[T.e] - t0);
  const int tid = threadIdx.x;
  if (tid == 0) *s_flags = 0;
  __syncthreads();
  if (tid < NTOK) {
    const int p = tid < T.cnt ? a.perm[a.boff[T.e] + t0 + tid] : -1;
    s_pair[tid] = p;
    const int row = p < 0 ? -1 : (rows_are_tokens ? p / a.k : p);
    s_row[tid] = row;
    if (rows_are_tokens && row >= 0) atomicOr(s_flags, (int)a.xflag[row]);
  }
  for (int i = tid; i < xs_words; i += blockDim.x) reinterpret_cast<uint32_t*>(xs_flat)[i] = 0u;
  __syncthreads();
  const int fl = rows_are_tokens ? *s_flags : 3;
  T.np = (fl & 2) ? 3 : ((fl & 1) ? 2 : 1);
  return true;
}

// Stage K block kb of the tile's source rows (planes 0..np-1) into LDS.
template <int NTOK>
__device__ __forceinline__ void stage_block(uint16_t (*xs)[NTOK][kXStride], const uint16_t* src,
                                            size_t plane_elems, int row_elems, const int* s_row,
                                            int cnt, int np, int kb) {
  for (int q = threadIdx.x; q < np * NTOK * 16; q += blockDim.x) {
    const int pl = q / (NTOK * 16), rem = q - pl * (NTOK * 16), c = rem >> 4, ch = rem & 15;
    if (c < cnt) {
      const uint4 v = *reinterpret_cast<const uint4*>(src + pl * plane_elems +
                                                      (size_t)s_row[c] * row_elems + kb * kBK + ch * 8);
      *reinterpret_cast<uint4*>(&xs[pl][c][ch * 8]) = v;
    }
  }
}

template <int FMT, int NB>
__global__ __launch_bounds__(256) void k_bgu(BArgs a) {
  constexpr int NTOK = 16 * NB;
  __shared__ __attribute__((aligned(16))) uint16_t xs[3][NTOK][kXStride];
  __shared__ int s_pair[NTOK], s_row[NTOK], s_flags;
  TileInfo T;
  if (!tile_setup<NTOK>(a, true, &xs[0][0][0], 3 * NTOK * kXStride / 2, s_pair, s_row, &s_flags, T))
    return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  const int H = a.H, I = a.I, B = (FMT == MOE_FMT_MXFP4) ? 32 : 16;
  const int row = blockIdx.x * kBRows + wave * 16 + r16;
  const uint8_t* rec = a.base + (size_t)T.e * a.stride;
  WeightRows<2> W;
  const uint32_t cbytes = (uint32_t)I * (H / 2), sbytes = (uint32_t)I * (H / B);
  W.codes[0] = view(rec + a.off[MOE_T_GATE_CODES], cbytes);
  W.codes[1] = view(rec + a.off[MOE_T_UP_CODES], cbytes);
  W.scales[0] = view(rec + a.off[MOE_T_GATE_SCALES], sbytes);
  W.scales[1] = view(rec + a.off[MOE_T_UP_SCALES], sbytes);
  W.coff = (uint32_t)row * (H / 2) + g * 16;
  W.soff = (uint32_t)row * (H / B) + g * (32 / B);
  W.cstep = kBK / 2;
  W.sstep = kBK / B;
  f32x4_t acc[2][NB];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[r][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int nkb = H / kBK;
  uint4 q[2], qn[2];
  uint32_t sc[2], scn[2];
  load_block<FMT, 2>(W, 0, qn, scn);
  for (int kb = 0; kb < nkb; ++kb) {
    __syncthreads();
    stage_block<NTOK>(xs, a.xp, (size_t)a.C * H, H, s_row, T.cnt, T.np, kb);
#pragma unroll
    for (int r = 0; r < 2; ++r) { q[r] = qn[r]; sc[r] = scn[r]; }
    if (kb + 1 < nkb) load_block<FMT, 2>(W, kb + 1, qn, scn);
    __syncthreads();
    mfma_block<FMT, 2, NB, NTOK>(q, sc, xs, T.np, acc);
  }
  float gg = 1.0f, gu = 1.0f;
  if (FMT == MOE_FMT_NVFP4) {
    const float* gl = reinterpret_cast<const float*>(rec + a.off[MOE_T_GLOBALS]);
    gg = gl[0];
    gu = gl[1];
  }
  const size_t CK = (size_t)a.C * a.k;
  const int irow = blockIdx.x * kBRows + wave * 16 + 4 * g;     // this lane's 4 output rows
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int p = s_pair[nb * 16 + r16];
    if (p < 0) continue;
    uint16_t hb[3][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float h = silu(gg * acc[0][nb][j]) * (gu * acc[1][nb][j]);
      split3(h, hb[0][j], hb[1][j], hb[2][j]);
    }
#pragma unroll
    for (int pl = 0; pl < 3; ++pl)
      *reinterpret_cast<uint2*>(a.hp + (pl * CK + p) * I + irow) =
          make_uint2((uint32_t)hb[pl][0] | ((uint32_t)hb[pl][1] << 16),
                     (uint32_t)hb[pl][2] | ((uint32_t)hb[pl][3] << 16));
  }
}

template <int FMT, int NB>
__global__ __launch_bounds__(256) void k_bdn(BArgs a) {
  constexpr int NTOK = 16 * NB;
  __shared__ __attribute__((aligned(16))) uint16_t xs[3][NTOK][kXStride];
  __shared__ int s_pair[NTOK], s_row[NTOK], s_flags;
  TileInfo T;
  if (!tile_setup<NTOK>(a, false, &xs[0][0][0], 3 * NTOK * kXStride / 2, s_pair, s_row, &s_flags, T))
    return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  const int H = a.H, I = a.I, B = (FMT == MOE_FMT_MXFP4) ? 32 : 16;
  const int row = blockIdx.x * kBRows + wave * 16 + r16;
  const uint8_t* rec = a.base + (size_t)T.e * a.stride;
  WeightRows<1> W;
  W.codes[0] = view(rec + a.off[MOE_T_DOWN_CODES], (uint32_t)H * (I / 2));
  W.scales[0] = view(rec + a.off[MOE_T_DOWN_SCALES], (uint32_t)H * (I / B));
  W.coff = (uint32_t)row * (I / 2) + g * 16;
  W.soff = (uint32_t)row * (I / B) + g * (32 / B);
  W.cstep = kBK / 2;
  W.sstep = kBK / B;
  f32x4_t acc[1][NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[0][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int nkb = I / kBK;
  const size_t CK = (size_t)a.C * a.k;
  uint4 q[1], qn[1];
  uint32_t sc[1], scn[1];
  load_block<FMT, 1>(W, 0, qn, scn);
  for (int kb = 0; kb < nkb; ++kb) {
    __syncthreads();
    stage_block<NTOK>(xs, a.hp, CK * I, I, s_row, T.cnt, T.np, kb);
    q[0] = qn[0];
    sc[0] = scn[0];
    if (kb + 1 < nkb) load_block<FMT, 1>(W, kb + 1, qn, scn);
    __syncthreads();
    mfma_block<FMT, 1, NB, NTOK>(q, sc, xs, T.np, acc);
  }
  float gd = 1.0f;
  if (FMT == MOE_FMT_NVFP4) gd = reinterpret_cast<const float*>(rec + a.off[MOE_T_GLOBALS])[2];
  const int hrow = blockIdx.x * kBRows + wave * 16 + 4 * g;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int p = s_pair[nb * 16 + r16];
    if (p < 0) continue;
    const float wp = a.w[p] * gd;
    *reinterpret_cast<float4*>(a.part + (size_t)p * H + hrow) =
        make_float4(wp * acc[0][nb][0], wp * acc[0][nb][1], wp * acc[0][nb][2], wp * acc[0][nb][3]);
  }
}

// out[t][j] = sum over the valid slots s of part[t*k + s][j], in slot order.
__global__ __launch_bounds__(256) void k_bcombine(BArgs a) {
  const int t = blockIdx.y;
  const int j = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (j >= a.H) return;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int sl = 0; sl < a.k; ++sl) {
    const int p = t * a.k + sl;
    const int e = a.idx[p];
    if (e < 0 || e >= a.E) continue;
    const float4 v = *reinterpret_cast<const float4*>(a.part + (size_t)p * a.H + j);
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  *reinterpret_cast<float4*>(a.out + (size_t)t * a.H + j) = s;
}

// ---------------------------------------------------------------------------
// Router for many tokens
// ---------------------------------------------------------------------------
// logits[t][e] = sum_h x[t][h] * W_r[e][h]: a 64-token x 64-expert tile per
// workgroup, wave w owns tokens 16w..16w+15 against all 64 experts (four
// 16x16 fp32 MFMA tiles), K in staged chunks of 32.
__global__ __launch_bounds__(256) void k_brouter(const float* x, const float* Wr, float* logits,
                                                 int C, int H, int E) {
  __shared__ float xsm[64][kRK + 1];
  __shared__ float wsm[64][kRK + 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const int tb = blockIdx.y * 64, eb = blockIdx.x * 64;
  f32x4_t acc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < H; k0 += kRK) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = tid + 256 * u;                 // 512 float4 per matrix chunk
      const int r = q >> 3, c4 = (q & 7) * 4;
      const int t = tb + r, e = eb + r;
      float4 xv = make_float4(0.f, 0.f, 0.f, 0.f), wv = xv;
      if (t < C) xv = *reinterpret_cast<const float4*>(x + (size_t)t * H + k0 + c4);
      if (e < E) wv = *reinterpret_cast<const float4*>(Wr + (size_t)e * H + k0 + c4);
      xsm[r][c4] = xv.x; xsm[r][c4 + 1] = xv.y; xsm[r][c4 + 2] = xv.z; xsm[r][c4 + 3] = xv.w;
      wsm[r][c4] = wv.x; wsm[r][c4 + 1] = wv.y; wsm[r][c4 + 2] = wv.z; wsm[r][c4 + 3] = wv.w;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kRK; kk += 4) {
      const float av = xsm[16 * wave + r16][kk + g];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, wsm[nb * 16 + r16][kk + g], acc[nb], 0, 0, 0);
    }
  }
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int e = eb + nb * 16 + r16;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = tb + 16 * wave + 4 * g + j;
      if (t < C && e < E) logits[(size_t)t * E + e] = acc[nb][j];
    }
  }
}

// One wave per token: the decode path's exact top-k and renormalised sigmoid
// weights.
__global__ __launch_bounds__(512) void k_btopk(const float* logits, int C, int E, int k,
                                               int32_t* idx, float* w) {
  __shared__ SelectLds S[8];
  constexpr int NPL = MOE_MAX_EXPERTS / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 8 + wave;
  if (t >= C) return;                       // whole waves leave; no barrier follows
  uint64_t ck[NPL];
  float lv[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    lv[i] = e < E ? logits[(size_t)t * E + e] : 0.0f;
    ck[i] = e < E ? sel_key(lv[i], e) : 0;
  }
  wave_select<NPL>(ck, lv, k, S[wave]);
  const float l = lane < k ? S[wave].sel_l[lane] : 0.0f;
  const float wt = route_weight(l, lane, k);
  if (lane < k) {
    idx[(size_t)t * k + lane] = S[wave].sel_e[lane];
    w[(size_t)t * k + lane] = wt;
  }
}

moe_status status_of_launch() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE; }

}  // namespace

moe_status launch_batched_route(const float* x, const float* Wr, const float* logits_in,
                                float* logits_out, int C, int H, int E, int k, int32_t* idx,
                                float* w, uint8_t* ws, const WsLayout& L, hipStream_t st) {
  const float* lg = logits_in;
  if (x) {
    float* dst = logits_out ? logits_out : reinterpret_cast<float*>(ws + L.logits);
    if (H % kRK) return MOE_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(k_brouter, dim3((E + 63) / 64, (C + 63) / 64), dim3(256), 0, st, x, Wr, dst,
                       C, H, E);
    lg = dst;
  }
  hipLaunchKernelGGL(k_btopk, dim3((C + 7) / 8), dim3(512), 0, st, lg, C, E, k, idx, w);
  return status_of_launch();
}

moe_status launch_batched_experts(const moe_bank* b, const float* x, int C, int k,
                                  const int32_t* idx, const float* w, float* out, uint8_t* ws,
                                  const WsLayout& L, hipStream_t st) {
  const int H = b->hidden, I = b->inter;
  if (H % kBK || I % kBK) return MOE_ERR_UNSUPPORTED;
  BArgs a;
  a.base = static_cast<const uint8_t*>(b->base);
  a.stride = b->expert_stride;
  for (int t = 0; t < MOE_NUM_TENSORS; ++t) a.off[t] = b->offset[t];
  a.E = b->num_experts; a.H = H; a.I = I; a.k = k; a.C = C;
  a.idx = idx; a.w = w; a.x = x;
  a.xp = reinterpret_cast<uint16_t*>(ws + L.xp);
  a.xflag = reinterpret_cast<uint32_t*>(ws + L.xflag);
  a.hp = reinterpret_cast<uint16_t*>(ws + L.hp);
  a.part = reinterpret_cast<float*>(ws + L.part);
  a.out = out;
  a.count = reinterpret_cast<uint32_t*>(ws + L.bcount);
  a.cursor = reinterpret_cast<uint32_t*>(ws + L.bcursor);
  a.boff = reinterpret_cast<uint32_t*>(ws + L.boff);
  a.meta = reinterpret_cast<uint32_t*>(ws + L.bmeta);
  a.tiles = reinterpret_cast<int32_t*>(ws + L.btile);
  a.perm = reinterpret_cast<int32_t*>(ws + L.perm);
  a.ntok = batch_ntok(C);
  const int CK = C * k;
  const unsigned maxt = (unsigned)batch_max_tiles(a.E, k, C);
  hipLaunchKernelGGL(k_bsplit, dim3(C), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_bcount, dim3((CK + 255) / 256), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_bscan, dim3(1), dim3(1024), 0, st, a);
  hipLaunchKernelGGL(k_bscatter, dim3((CK + 255) / 256), dim3(256), 0, st, a);
  const dim3 ggu(I / kBRows, maxt), gdn(H / kBRows, maxt);
  if (b->format == MOE_FMT_MXFP4) {
    if (a.ntok == 16) {
      hipLaunchKernelGGL((k_bgu<MOE_FMT_MXFP4, 1>), ggu, dim3(256), 0, st, a);
      hipLaunchKernelGGL((k_bdn<MOE_FMT_MXFP4, 1>), gdn, dim3(256), 0, st, a);
    } else {
      hipLaunchKernelGGL((k_bgu<MOE_FMT_MXFP4, 4>), ggu, dim3(256), 0, st, a);
      hipLaunchKernelGGL((k_bdn<MOE_FMT_MXFP4, 4>), gdn, dim3(256), 0, st, a);
    }
  } else {
    if (a.ntok == 16) {
      hipLaunchKernelGGL((k_bgu<MOE_FMT_NVFP4, 1>), ggu, dim3(256), 0, st, a);
      hipLaunchKernelGGL((k_bdn<MOE_FMT_NVFP4, 1>), gdn, dim3(256), 0, st, a);
    } else {
      hipLaunchKernelGGL((k_bgu<MOE_FMT_NVFP4, 4>), ggu, dim3(256), 0, st, a);
      hipLaunchKernelGGL((k_bdn<MOE_FMT_NVFP4, 4>), gdn, dim3(256), 0, st, a);
    }
  }
  hipLaunchKernelGGL(k_bcombine, dim3((H / 4 + 255) / 256, C), dim3(256), 0, st, a);
  return status_of_launch();
}

}  // namespace rf4
