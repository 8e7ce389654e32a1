// libroutedfp4, batched path: the routed experts of many tokens at once,
// as row dot products for decode batches (C = 2..16) and as grouped GEMMs on
// the CDNA4 matrix cores for wider calls (prefill chunks).
//
// Used for C >= 2 tokens per call.  The
// layer is the same as the decode path's (page "Kimi-K3 on 2x A40 -- measured
// findings", section "Why the placement experiments all looked the same":
// MUL_MAT_ID over the selected experts; page "SparkInfer-K3", section "How the
// TP module works": router -> top-k -> experts -> sum), arranged so that every
// selected expert's weights are read once per tile of the tokens that chose it
// (page "Kimi-K3 on the same pod, two engines", section "Where our build is
// still ahead": a batched prompt pass reads each expert once per chunk).
//
// Precision.  Every weight e2m1 * scale is exact in bf16 (NVFP4: at most 6
// significant bits; MXFP4: a power-of-two scale), so the weights go to the
// matrix cores as bf16 without rounding.  x is fp32: each value is split into
// three bf16 pieces whose sum is the value exactly (8 + 8 + 8 significant
// bits) and each piece is multiplied separately; a piece that is zero for every
// token of a tile (bf16-exact input) is skipped, so the gate/up products are
// exact and only the fp32 accumulation rounds.  The SwiGLU output h goes to the
// down product as two pieces (hi + lo), which carry h to within 2^-17
// relative.  The NVFP4 per-tensor scale multiplies the accumulated sums.
//
// Decode batches (C <= 16), in stream order (precision as the batch-1
// kernel: fp32 products and sums):
//   k_btopk<16> the top-k of every token, then the dispatch table
//   k_dstream   gate/up with SwiGLU, then down: each distinct expert streamed
//               once over cost-balanced row ranges (see "Decode batches")
//   k_bcombine  out[t] = sum of its pairs' rows in slot order
// Wider calls, in stream order:
//   k_bsplit    x -> three bf16 planes + per-token flags (zeroes the counters)
//   k_bcount    (token, slot) pairs per expert
//   k_bscan     offsets and the tile list (each expert's pairs in tiles of
//               16 or 64)
//   k_bscatter  pairs grouped by expert
//   k_bmm<GU>   per (tile, 256 rows of I): gate and up on MFMA, SwiGLU, h as
//               two bf16 planes
//   k_bmm<DN>   per (tile, 512 rows of H): down on MFMA, times the routing
//               weight, one fp32 row per pair (k_bmm_dnp: the same as
//               persistent workgroups where I spans four K stages or more)
//   k_bcombine  out[t] = sum of its pairs' rows in slot order (deterministic)
// and for the router of many tokens:
//   k_brouter   logits = x * W_r^T with fp32 MFMA
//   k_btopk     one wave per token: the same exact top-k as the decode path
#include "common.h"

#include <atomic>
#include <type_traits>

namespace rf4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRmGU = 1;             // gate/up: 16-row MFMA tiles per wave
constexpr int kRmDN = 2;             // down: 16-row MFMA tiles per wave
constexpr int kNwGU = 16;            // gate/up: waves per workgroup (256 rows of each matrix)
constexpr int kNwDN = 16;            // down: waves per workgroup (512 rows)
constexpr int kRmGUn = 2;            // narrow tiles: gate/up 128 rows per workgroup
constexpr int kRmDNn = 4;            // narrow tiles: down 256 rows per workgroup
constexpr int kRK = 32;              // router: K elements per staged chunk
constexpr int kQueueDN = 16;         // meta[16]: the persistent down GEMM's item counter

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
  uint16_t* hp;           // [2][C*k][I] bf16 planes of h (hi, lo)
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
    a.meta[kQueueDN] = 0u;
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
// k_bmm: one grouped GEMM (gate/up with SwiGLU, or down) for one tile of up
// to NTOK = 16 * NB pairs of one expert and 16 * RM * NW rows of each of NMAT
// weight matrices (wave w of NW owns rows 16 RM w .. 16 RM w + 16 RM - 1, as
// RM MFMA row tiles).  Sixteen waves share one staged activation tile, so
// the tile's reads from L2 per weight byte are a quarter of what four waves
// need (at four they matched the weight bytes), and the 128-register limit
// of a 1024-thread workgroup still gives one workgroup of 16 waves per CU.
//
// K runs in stages of 256 elements: lane l of a wave reads 32 contiguous code
// bytes of row (l % 16) of each row tile, at K offset 64 (l / 16) of the
// stage, so a row tile's loads are 16 whole 128-byte rows segments.  MFMA
// step t (0..7) of a stage takes elements 8t..8t+7 of the lane's 64, i.e. K
// offset 64 (l / 16) + 8 t + j for k-slot 8 (l / 16) + j of the 16x16x32
// product; the activations are staged in LDS in plain K order and read with
// the same mapping, so A and B agree.  Weights are loaded two stages ahead
// (registers), the next activation stage one ahead (registers, then LDS).
// Activation planes: x has up to 3 (skipped when zero for the whole tile),
// h has 2 (hi + lo: h to within 2^-17 relative).
constexpr int kSK = 256;                 // K elements per stage
constexpr int kSStride = kSK + 8;        // bf16 per staged row (528 B)

template <int FMT, int NMAT, int RM>
struct StageW {
  uint4 q[NMAT][RM][2];                  // 32 code bytes per row tile and matrix
  uint32_t sc[NMAT][RM];                 // MX: 2 e8m0 bytes; NV: 4 e4m3 bytes
};

// Loads are unconditional: a stage past the end (valid false) reads from an
// offset beyond the buffer, which returns zeros without touching memory, so
// the compiler can count outstanding loads exactly (no vmcnt(0) at joins).
constexpr uint32_t kNoLoad = 0x80000000u;
// The grouped GEMMs load weights with the default cache policy: every tile
// of an expert reads that expert's weights again, and when the row blocks
// per tile are a multiple of the XCD count (the K3 shape: 24 and 56) the
// tiles of one row block all run on one XCD, whose L2 can then serve the
// repeats.  (Non-temporal loads, right for a stream read once, made every
// tile fetch them from memory again: 9.95 -> 8.59 ms for the 2048-token K3
// chunk, 4.60 -> 3.72 ms for the W50 one.)
constexpr int kCachePolicyGemmW = 0;

template <int FMT, int NMAT, int RM>
__device__ __forceinline__ void load_stage(const __amdgpu_buffer_rsrc_t (&codes)[NMAT],
                                           const __amdgpu_buffer_rsrc_t (&scales)[NMAT],
                                           const uint32_t (&coff)[RM], const uint32_t (&soff)[RM],
                                           int kb, bool valid, StageW<FMT, NMAT, RM>& W) {
#pragma unroll
  for (int m = 0; m < NMAT; ++m) {
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      const int co = valid ? (int)(coff[r] + kb * (kSK / 2)) : (int)kNoLoad;
      const int so = valid ? (int)(soff[r] + kb * (kSK / (FMT == MOE_FMT_MXFP4 ? 32 : 16))) : (int)kNoLoad;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(codes[m], co + 16 * c, 0, kCachePolicyGemmW);
        W.q[m][r][c] = make_uint4(v[0], v[1], v[2], v[3]);
      }
      if (FMT == MOE_FMT_MXFP4)
        W.sc[m][r] = __builtin_amdgcn_raw_buffer_load_b16(scales[m], so, 0, kCachePolicyGemmW);
      else
        W.sc[m][r] = __builtin_amdgcn_raw_buffer_load_b32(scales[m], so, 0, kCachePolicyGemmW);
    }
  }
}

template <int NTOK, int PL, int NTHR>
struct StageB {
  uint4 v[PL][NTOK * 32 / NTHR];         // PL planes of NTOK rows x 256 bf16 / NTHR threads
};

// Activation stage kb, planes pl0 .. pl0+PL-1 (those below np), of the tile's
// first `rows` rows (rows past cnt read as zero) into registers.
template <int NTOK, int PL, int NTHR>
__device__ __forceinline__ void load_b(__amdgpu_buffer_rsrc_t src, uint32_t plane_bytes, int row_elems,
                                       const int* s_row, int cnt, int pl0, int np, int kb,
                                       StageB<NTOK, PL, NTHR>& B) {
#pragma unroll
  for (int pl = 0; pl < PL; ++pl)
#pragma unroll
    for (int u = 0; u < NTOK * 32 / NTHR; ++u) {
      const int q = threadIdx.x + NTHR * u, c = q >> 5, ch = q & 31;
      const bool ok = c < cnt && pl0 + pl < np;
      const uint32_t off = ok ? (uint32_t)(pl0 + pl) * plane_bytes +
                                    ((uint32_t)s_row[c] * row_elems + kb * kSK + ch * 8) * 2u
                              : kNoLoad;
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(src, (int)off, 0, 0);
      B.v[pl][u] = make_uint4(v[0], v[1], v[2], v[3]);
    }
}

// Every row is stored (rows past the tile's pairs hold zeros): a store under a
// branch would cost the compiler its exact count of outstanding loads.
template <int NTOK, int PL, int NTHR>
__device__ __forceinline__ void store_b(uint16_t (*xs)[NTOK][kSStride], const StageB<NTOK, PL, NTHR>& B) {
#pragma unroll
  for (int pl = 0; pl < PL; ++pl)
#pragma unroll
    for (int u = 0; u < NTOK * 32 / NTHR; ++u) {
      const int q = threadIdx.x + NTHR * u, c = q >> 5, ch = q & 31;
      *reinterpret_cast<uint4*>(&xs[pl][c][ch * 8]) = B.v[pl][u];
    }
}

// One K stage: for each MFMA step the weights are dequantised once and used
// for the column tiles that hold pairs and the PL staged planes.  Without
// DYN their count NBR (<= NB) is a compile-time constant, so the steps hold
// no branches and the compiler can move a step's LDS reads and
// dequantisation ahead of the previous step's products; with DYN the count
// is the runtime nbr (a branch per column tile, fewer registers live).
template <int FMT, int NMAT, int RM, int NB, int NTOK, int PL, int NBR, bool DYN>
__device__ __forceinline__ void mfma_stage(const StageW<FMT, NMAT, RM>& W,
                                           const uint16_t (*xs)[NTOK][kSStride], int nbr,
                                           f32x4_t (&acc)[NMAT][RM][NB]) {
  static_assert(NBR >= 1 && NBR <= NB, "column tiles");
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int c = t >> 2, s = t & 3;
    bf16x8_t A[NMAT][RM];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int r = 0; r < RM; ++r) {
        const uint32_t sb = (FMT == MOE_FMT_MXFP4) ? ((W.sc[m][r] >> (8 * c)) & 0xFFu)
                                                   : ((W.sc[m][r] >> (8 * (2 * c + (s >> 1)))) & 0xFFu);
        A[m][r] = dequant8<FMT>(scale_word(W.q[m][r][c], s), sb);
      }
#pragma unroll
    for (int pl = 0; pl < PL; ++pl) {
#pragma unroll
      for (int nb = 0; nb < NBR; ++nb) {
        if (DYN && nb >= nbr) break;
        const bf16x8_t Bv = lds_bf16x8(&xs[pl][nb * 16 + r16][64 * g + 8 * t]);
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int r = 0; r < RM; ++r)
            acc[m][r][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[m][r], Bv, acc[m][r][nb], 0, 0, 0);
      }
    }
  }
}

// GU: gate and up against x (K = H), SwiGLU, h out as two bf16 planes.
// DN: down against h (K = I), times the routing weight, one fp32 row per pair.
// NB column tiles of 16 pairs at most (the tile's own count decides how many
// run); PL activation planes staged per K stage (both h planes at once; x
// planes one group at a time for wide tiles, whose x is usually bf16-exact).
template <int FMT, bool GU, int RM, int NB, int NW>
__global__ __launch_bounds__(64 * NW) void k_bmm(BArgs a) {
  constexpr int NMAT = GU ? 2 : 1;
  constexpr int NTOK = 16 * NB;
  constexpr int NTHR = 64 * NW;
  static_assert(NTOK * 32 % NTHR == 0, "activation stage split");
  constexpr int PL = GU ? (NB == 1 ? 3 : 1) : 2;   // h: both planes at once
  extern __shared__ __attribute__((aligned(16))) uint8_t bmm_lds[];   // two activation stages
  uint16_t (*const xs0)[NTOK][kSStride] = reinterpret_cast<uint16_t (*)[NTOK][kSStride]>(bmm_lds);
  uint16_t (*const xs1)[NTOK][kSStride] = xs0 + PL;
  __shared__ int s_pair[NTOK], s_row[NTOK], s_flags;
  const int tile = blockIdx.y;
  if (tile >= (int)a.meta[0]) return;
  const int e = a.tiles[2 * tile], t0 = a.tiles[2 * tile + 1];
  const int cnt = min(NTOK, (int)a.count[e] - t0);
  const int nbr = (cnt + 15) >> 4;              // column tiles that hold pairs
  const int tid = threadIdx.x;
  if (tid == 0) s_flags = 0;
  __syncthreads();
  if (tid < NTOK) {
    const int p = tid < cnt ? a.perm[a.boff[e] + t0 + tid] : -1;
    s_pair[tid] = p;
    const int row = p < 0 ? -1 : (GU ? p / a.k : p);
    s_row[tid] = row;
    if (GU && row >= 0) atomicOr(&s_flags, (int)a.xflag[row]);
  }
  __syncthreads();
  const int fl = s_flags;
  const int np = GU ? ((fl & 2) ? 3 : ((fl & 1) ? 2 : 1)) : 2;
  static_assert(!GU || PL == 1 || NB == 1, "x planes staged one at a time in wide tiles");
  static_assert(GU || PL == 2, "both h planes staged together");
  const int ngr = (np + PL - 1) / PL;           // plane groups per K stage (every group holds PL planes)

  const int wave = tid >> 6, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const int H = a.H, I = a.I, B = (FMT == MOE_FMT_MXFP4) ? 32 : 16;
  const int K = GU ? H : I, N = GU ? I : H;
  const int row0 = blockIdx.x * (16 * RM * NW) + wave * (16 * RM);
  const uint8_t* rec = a.base + (size_t)e * a.stride;
  __amdgpu_buffer_rsrc_t codes[NMAT], scales[NMAT];
  const uint32_t cbytes = (uint32_t)N * (K / 2), sbytes = (uint32_t)N * (K / B);
  if (GU) {
    codes[0] = view(rec + a.off[MOE_T_GATE_CODES], cbytes);
    scales[0] = view(rec + a.off[MOE_T_GATE_SCALES], sbytes);
    codes[NMAT - 1] = view(rec + a.off[MOE_T_UP_CODES], cbytes);
    scales[NMAT - 1] = view(rec + a.off[MOE_T_UP_SCALES], sbytes);
  } else {
    codes[0] = view(rec + a.off[MOE_T_DOWN_CODES], cbytes);
    scales[0] = view(rec + a.off[MOE_T_DOWN_SCALES], sbytes);
  }
  uint32_t coff[RM], soff[RM];
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    const int row = row0 + 16 * r + r16;
    coff[r] = (uint32_t)row * (K / 2) + g * 32;
    soff[r] = (uint32_t)row * (K / B) + g * (64 / B);
  }
  const size_t CK = (size_t)a.C * a.k;
  const uint32_t plane_bytes = (uint32_t)((GU ? (size_t)a.C * H : CK * I) * 2);
  const __amdgpu_buffer_rsrc_t src = view(reinterpret_cast<const uint8_t*>(GU ? a.xp : a.hp),
                                          plane_bytes * (uint32_t)(GU ? 3 : 2));

  f32x4_t acc[NMAT][RM][NB];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int r = 0; r < RM; ++r)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[m][r][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // K stages in pairs (nkb is even): weight buffer W0 and LDS stage xs0 serve
  // even stages, W1 and xs1 odd ones, so a weight buffer is reloaded in place
  // after use and no register copy of an in-flight load is ever needed (a
  // copy would wait for the load).  The activations of stage kb + 1 go from
  // registers into the other LDS stage before stage kb's products, whose
  // reads of that stage (kb - 1) ended at the previous barrier: one barrier
  // per stage.  Plane groups beyond the first (wide tiles of non-bf16-exact
  // x only) stream the weights again.
  const int nkb = K / kSK;
  // the K loop for a compile-time count of column tiles
  auto kloop = [&](auto nbr_c) {
    constexpr int NBR = decltype(nbr_c)::value;
    for (int gr = 0; gr < ngr; ++gr) {
      const int pl0 = gr * PL;
      StageW<FMT, NMAT, RM> W0, W1;
      StageB<NTOK, PL, NTHR> Bs;
      // Issue order as at the loop's back edge (activations of the next
      // stage, then the weights of the stage after it), so the compiler's
      // count of outstanding loads agrees on both paths into the loop and
      // its waits stay partial (a mismatch makes it wait for every load,
      // the prefetches included).
      load_stage<FMT, NMAT, RM>(codes, scales, coff, soff, 0, true, W0);
      load_b<NTOK, PL, NTHR>(src, plane_bytes, K, s_row, cnt, pl0, np, 0, Bs);
      store_b<NTOK, PL, NTHR>(xs0, Bs);
      load_b<NTOK, PL, NTHR>(src, plane_bytes, K, s_row, cnt, pl0, np, 1, Bs);
      load_stage<FMT, NMAT, RM>(codes, scales, coff, soff, 1, true, W1);
      __syncthreads();
      for (int kb = 0; kb < nkb; kb += 2) {
        store_b<NTOK, PL, NTHR>(xs1, Bs);
        load_b<NTOK, PL, NTHR>(src, plane_bytes, K, s_row, kb + 2 < nkb ? cnt : 0, pl0, np, kb + 2, Bs);
        mfma_stage<FMT, NMAT, RM, NB, NTOK, PL, NBR, !GU>(W0, xs0, nbr, acc);
        load_stage<FMT, NMAT, RM>(codes, scales, coff, soff, kb + 2, kb + 2 < nkb, W0);
        __syncthreads();
        store_b<NTOK, PL, NTHR>(xs0, Bs);        // stage kb + 2 (zeros past the last)
        load_b<NTOK, PL, NTHR>(src, plane_bytes, K, s_row, kb + 3 < nkb ? cnt : 0, pl0, np, kb + 3, Bs);
        mfma_stage<FMT, NMAT, RM, NB, NTOK, PL, NBR, !GU>(W1, xs1, nbr, acc);
        load_stage<FMT, NMAT, RM>(codes, scales, coff, soff, kb + 3, kb + 3 < nkb, W1);
        __syncthreads();
      }
    }
  };
  // gate/up: one instance per column-tile count; down (two planes, twice the
  // fragments per step) keeps the runtime count, which spills no registers
  static_assert(NB == 4, "column-tile dispatch below");
  if (!GU) {
    kloop(std::integral_constant<int, 4>{});
  } else {
    switch (nbr) {
      case 1: kloop(std::integral_constant<int, 1>{}); break;
      case 2: kloop(std::integral_constant<int, 2>{}); break;
      case 3: kloop(std::integral_constant<int, 3>{}); break;
      default: kloop(std::integral_constant<int, 4>{}); break;
    }
  }

  const int orow0 = row0 + 4 * g;              // + 16 r + j: this lane's output rows
  if (GU) {
    float gg = 1.0f, gu = 1.0f;
    if (FMT == MOE_FMT_NVFP4) {
      const float* gl = reinterpret_cast<const float*>(rec + a.off[MOE_T_GLOBALS]);
      gg = gl[0];
      gu = gl[1];
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int p = s_pair[nb * 16 + r16];
      if (p < 0) continue;
#pragma unroll
      for (int r = 0; r < RM; ++r) {
        uint16_t hi[4], lo[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float h = silu(gg * acc[0][r][nb][j]) * (gu * acc[NMAT - 1][r][nb][j]);
          hi[j] = bf16_bits(h);
          lo[j] = bf16_bits(h - bf16_float(hi[j]));
        }
        const size_t o = (size_t)p * I + orow0 + 16 * r;
        *reinterpret_cast<uint2*>(a.hp + o) =
            make_uint2((uint32_t)hi[0] | ((uint32_t)hi[1] << 16), (uint32_t)hi[2] | ((uint32_t)hi[3] << 16));
        *reinterpret_cast<uint2*>(a.hp + CK * I + o) =
            make_uint2((uint32_t)lo[0] | ((uint32_t)lo[1] << 16), (uint32_t)lo[2] | ((uint32_t)lo[3] << 16));
      }
    }
  } else {
    float gd = 1.0f;
    if (FMT == MOE_FMT_NVFP4) gd = reinterpret_cast<const float*>(rec + a.off[MOE_T_GLOBALS])[2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int p = s_pair[nb * 16 + r16];
      if (p < 0) continue;
      const float wp = a.w[p] * gd;
#pragma unroll
      for (int r = 0; r < RM; ++r)
        *reinterpret_cast<float4*>(a.part + (size_t)p * H + orow0 + 16 * r) =
            make_float4(wp * acc[0][r][nb][0], wp * acc[0][r][nb][1], wp * acc[0][r][nb][2],
                        wp * acc[0][r][nb][3]);
    }
  }
}

// k_bmm_dnp: the down GEMM as persistent workgroups, one per CU, for K of
// at least four stages.  A workgroup takes (tile, row block) items from a
// counter in the workspace (item = tile * R + row block) and runs them as
// one stream of K stages: the last stages of an item load the next item's
// first weight and activation stages, so loads stay in flight across the
// epilogue and the change of item, where a workgroup that ends and one that
// starts leave the CU with none (per-workgroup clocks of k_bmm<DN> put ~13%
// of its time there).  Item bookkeeping lives in three LDS slots (the item
// being multiplied, the next one, whose loads start in this one's last
// stages, and the one after it, taken from the counter and set up during
// this one's first stages); the routing weights of an item's pairs are
// staged with them.  Arithmetic, order of sums and outputs as k_bmm<DN>.
template <int FMT, int RM, int NB, int NW>
__global__ __launch_bounds__(64 * NW) void k_bmm_dnp(BArgs a) {
  constexpr int NTOK = 16 * NB;
  constexpr int NTHR = 64 * NW;
  constexpr int PL = 2;                               // h: hi and lo planes
  static_assert(NTOK * 32 % NTHR == 0, "activation stage split");
  extern __shared__ __attribute__((aligned(16))) uint8_t bmm_lds[];   // two activation stages
  uint16_t (*const xs0)[NTOK][kSStride] = reinterpret_cast<uint16_t (*)[NTOK][kSStride]>(bmm_lds);
  uint16_t (*const xs1)[NTOK][kSStride] = xs0 + PL;
  __shared__ int s_pair[3][NTOK], s_row[3][NTOK];
  __shared__ float s_wgt[3][NTOK];
  __shared__ int s_item[3], s_e[3], s_cnt[3];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: the views below are scalar
  const int H = a.H, I = a.I, B = (FMT == MOE_FMT_MXFP4) ? 32 : 16;
  const int K = I, N = H;
  const int R = N / (16 * RM * NW);
  const int nitems = (int)a.meta[0] * R;
  const int nkb = K / kSK;                            // even, >= 4
  uint32_t* const q = a.meta + kQueueDN;
  const size_t CK = (size_t)a.C * a.k;
  const uint32_t plane_bytes = (uint32_t)(CK * I * 2);
  const __amdgpu_buffer_rsrc_t src = view(reinterpret_cast<const uint8_t*>(a.hp), plane_bytes * 2u);
  const uint32_t cbytes = (uint32_t)N * (K / 2), sbytes = (uint32_t)N * (K / B);

  // slot sl <- item it (it >= 0): expert, pair count, pairs, their rows and
  // routing weights (times the NVFP4 global)
  auto setup = [&](int sl, int it) {
    const int tile = it / R;
    const int e = a.tiles[2 * tile], t0 = a.tiles[2 * tile + 1];
    const int cnt = min(NTOK, (int)a.count[e] - t0);
    if (tid < NTOK) {
      const int pr = tid < cnt ? a.perm[a.boff[e] + t0 + tid] : -1;
      s_pair[sl][tid] = pr;
      s_row[sl][tid] = pr;
      float gd = 1.0f;
      if (FMT == MOE_FMT_NVFP4 && pr >= 0)
        gd = reinterpret_cast<const float*>(a.base + (size_t)e * a.stride + a.off[MOE_T_GLOBALS])[2];
      s_wgt[sl][tid] = pr >= 0 ? a.w[pr] * gd : 0.0f;
    }
    if (tid == 0) {
      s_e[sl] = e;
      s_cnt[sl] = cnt;
    }
  };
  // this lane's offsets from its wave's first row (the same for every item)
  uint32_t coff[RM], soff[RM];
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    coff[r] = (uint32_t)(16 * r + r16) * (K / 2) + g * 32;
    soff[r] = (uint32_t)(16 * r + r16) * (K / B) + g * (64 / B);
  }
  // the weight views of item it from this wave's first row on (uniform
  // values only; it < 0: empty views, no loads)
  struct View {
    __amdgpu_buffer_rsrc_t codes[1], scales[1];
    int cnt, sl;
  };
  auto view_of = [&](int sl, int it, View& v) {
    v.sl = sl;
    v.cnt = __builtin_amdgcn_readfirstlane(it >= 0 ? s_cnt[sl] : 0);
    const int e = __builtin_amdgcn_readfirstlane(it >= 0 ? s_e[sl] : 0);
    const int row0 = (it >= 0 ? it % R : 0) * (16 * RM * NW) + wave * (16 * RM);
    const uint8_t* rec = a.base + (size_t)e * a.stride;
    v.codes[0] = view(rec + a.off[MOE_T_DOWN_CODES] + (size_t)row0 * (K / 2),
                      it >= 0 ? cbytes - (uint32_t)row0 * (K / 2) : 0u);
    v.scales[0] = view(rec + a.off[MOE_T_DOWN_SCALES] + (size_t)row0 * (K / B),
                       it >= 0 ? sbytes - (uint32_t)row0 * (K / B) : 0u);
  };

  // items 0 and 1 of this workgroup
  if (tid == 0) {
    const uint32_t i0 = atomicAdd(q, 1u), i1 = atomicAdd(q, 1u);
    s_item[0] = i0 < (uint32_t)nitems ? (int)i0 : -1;
    s_item[1] = i1 < (uint32_t)nitems ? (int)i1 : -1;
  }
  __syncthreads();
  int cur = __builtin_amdgcn_readfirstlane(s_item[0]), nxt = __builtin_amdgcn_readfirstlane(s_item[1]);
  if (cur < 0) return;
  setup(0, cur);
  if (nxt >= 0) setup(1, nxt);
  __syncthreads();
  View vc, vn;
  view_of(0, cur, vc);
  view_of(1, nxt, vn);

  StageW<FMT, 1, RM> W0, W1;
  StageB<NTOK, PL, NTHR> Bs;
  load_stage<FMT, 1, RM>(vc.codes, vc.scales, coff, soff, 0, true, W0);
  load_b<NTOK, PL, NTHR>(src, plane_bytes, K, s_row[vc.sl], vc.cnt, 0, PL, 0, Bs);
  store_b<NTOK, PL, NTHR>(xs0, Bs);
  load_b<NTOK, PL, NTHR>(src, plane_bytes, K, s_row[vc.sl], vc.cnt, 0, PL, 1, Bs);
  load_stage<FMT, 1, RM>(vc.codes, vc.scales, coff, soff, 1, true, W1);
  __syncthreads();

  int seq = 0;                                        // this workgroup's item count
  for (;;) {
    f32x4_t acc[1][RM][NB];
#pragma unroll
    for (int r = 0; r < RM; ++r)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[0][r][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int nbr = (vc.cnt + 15) >> 4;
    const int sl2 = (seq + 2) % 3;                    // slot of the item after the next
    for (int kb = 0; kb < nkb; kb += 2) {
      const bool last = kb + 2 >= nkb;
      store_b<NTOK, PL, NTHR>(xs1, Bs);
      if (!last) load_b<NTOK, PL, NTHR>(src, plane_bytes, K, s_row[vc.sl], vc.cnt, 0, PL, kb + 2, Bs);
      else load_b<NTOK, PL, NTHR>(src, plane_bytes, K, s_row[vn.sl], vn.cnt, 0, PL, 0, Bs);
      mfma_stage<FMT, 1, RM, NB, NTOK, PL, NB, true>(W0, xs0, nbr, acc);
      if (!last) load_stage<FMT, 1, RM>(vc.codes, vc.scales, coff, soff, kb + 2, true, W0);
      else load_stage<FMT, 1, RM>(vn.codes, vn.scales, coff, soff, 0, nxt >= 0, W0);
      __syncthreads();
      // after the first barrier of an item the slot of the item before it is
      // free: take the item after the next from the counter
      if (kb == 0 && tid == 0) {
        const uint32_t i2 = nxt >= 0 ? atomicAdd(q, 1u) : 0xFFFFFFFFu;
        s_item[sl2] = i2 < (uint32_t)nitems ? (int)i2 : -1;
      }
      // ... and set it up in the second stage pair (visible from the next
      // barrier on, before the next item's last stages load from it)
      if (kb == 2) {
        const int it2 = __builtin_amdgcn_readfirstlane(s_item[sl2]);
        if (it2 >= 0) setup(sl2, it2);
      }
      store_b<NTOK, PL, NTHR>(xs0, Bs);
      if (!last) load_b<NTOK, PL, NTHR>(src, plane_bytes, K, s_row[vc.sl], vc.cnt, 0, PL, kb + 3, Bs);
      else load_b<NTOK, PL, NTHR>(src, plane_bytes, K, s_row[vn.sl], vn.cnt, 0, PL, 1, Bs);
      mfma_stage<FMT, 1, RM, NB, NTOK, PL, NB, true>(W1, xs1, nbr, acc);
      // (the next item's second weight stage is loaded after the epilogue,
      // which then holds fewer registers)
      if (!last) load_stage<FMT, 1, RM>(vc.codes, vc.scales, coff, soff, kb + 3, true, W1);
      __syncthreads();
    }
    // epilogue of the current item: weighted rows out, one per pair
    {
      const int orow0 = (cur % R) * (16 * RM * NW) + wave * (16 * RM) + 4 * g;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int pr = s_pair[vc.sl][nb * 16 + r16];
        if (pr < 0) continue;
        const float wp = s_wgt[vc.sl][nb * 16 + r16];
#pragma unroll
        for (int r = 0; r < RM; ++r)
          *reinterpret_cast<float4*>(a.part + (size_t)pr * H + orow0 + 16 * r) =
              make_float4(wp * acc[0][r][nb][0], wp * acc[0][r][nb][1], wp * acc[0][r][nb][2],
                          wp * acc[0][r][nb][3]);
      }
    }
    if (nxt < 0) break;
    load_stage<FMT, 1, RM>(vn.codes, vn.scales, coff, soff, 1, true, W1);
    ++seq;
    cur = nxt;
    vc = vn;
    nxt = __builtin_amdgcn_readfirstlane(s_item[sl2]);
    view_of(sl2, nxt, vn);
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
// 16x16 fp32 MFMA tiles), K in staged chunks of 32.  Two LDS chunk buffers:
// the next chunk is loaded into registers while the current one is
// multiplied and stored into the other buffer before it, whose readers (the
// previous chunk) finished at the last barrier, so one barrier per chunk.
__global__ __launch_bounds__(256) void k_brouter(const float* x, const float* Wr, float* logits,
                                                 int C, int H, int E) {
  __shared__ float xsm[2][64][kRK + 1];
  __shared__ float wsm[2][64][kRK + 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const int tb = blockIdx.y * 64, eb = blockIdx.x * 64;
  float4 xv[2], wv[2];
  auto fetch = [&](int k0) {                       // 512 float4 per matrix chunk
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = tid + 256 * u;
      const int r = q >> 3, c4 = (q & 7) * 4;
      const int t = tb + r, e = eb + r;
      xv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      wv[u] = xv[u];
      if (t < C) xv[u] = *reinterpret_cast<const float4*>(x + (size_t)t * H + k0 + c4);
      if (e < E) wv[u] = *reinterpret_cast<const float4*>(Wr + (size_t)e * H + k0 + c4);
    }
  };
  auto put = [&](int b) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = tid + 256 * u;
      const int r = q >> 3, c4 = (q & 7) * 4;
      xsm[b][r][c4] = xv[u].x; xsm[b][r][c4 + 1] = xv[u].y; xsm[b][r][c4 + 2] = xv[u].z; xsm[b][r][c4 + 3] = xv[u].w;
      wsm[b][r][c4] = wv[u].x; wsm[b][r][c4 + 1] = wv[u].y; wsm[b][r][c4 + 2] = wv[u].z; wsm[b][r][c4 + 3] = wv[u].w;
    }
  };
  f32x4_t acc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  fetch(0);
  put(0);
  if (kRK < H) fetch(kRK);
  __syncthreads();
  int b = 0;
  for (int k0 = 0; k0 < H; k0 += kRK, b ^= 1) {
    if (k0 + kRK < H) put(b ^ 1);
    if (k0 + 2 * kRK < H) fetch(k0 + 2 * kRK);
    // The instruction adds its 4 products to the accumulator as 4 chained
    // FMAs (measured), so a chunk's products go into an accumulator of their
    // own (32 roundings) that is then added to the running sum: the longest
    // rounding chain of a logit is 32 + H/32 instead of H.
    f32x4_t part[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) part[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < kRK; kk += 4) {
      const float av = xsm[b][16 * wave + r16][kk + g];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        part[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, wsm[b][nb * 16 + r16][kk + g], part[nb], 0, 0, 0);
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[nb] += part[nb];
    __syncthreads();
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

// The same exact top-k as wave_select (same keys, same result), with fewer
// steps for the usual case, as the single-launch decode kernel selects: T is
// the largest 16-bit key prefix that at least k lane maxima reach (a 16-step
// ballot search), so every key of the top k is at or above it; the keys at or
// above T are gathered into LDS by a per-lane bit mask and a prefix count and
// each is ranked by the candidates ahead of it (broadcast LDS reads).  More
// than 64 candidates fall back to wave_select.
template <int NPL>
__device__ void wave_select_fast(uint64_t (&ck)[NPL], const float (&lv)[NPL], int k, SelectLds& S) {
  const int lane = threadIdx.x & 63;
  uint32_t m = 0;                                  // this lane's largest 32-bit key
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const uint32_t kk = (uint32_t)(ck[i] >> 32);
    m = kk > m ? kk : m;
  }
  uint32_t T = 0;
  for (int bit = 31; bit >= 16; --bit) {
    const uint32_t c = T | (1u << bit);
    if (__popcll(__ballot(m >= c)) >= k) T = c;
  }
  uint32_t cm = 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i)
    cm |= (ck[i] != 0 && (uint32_t)(ck[i] >> 32) >= T) ? (1u << i) : 0u;
  const int cnt = __popc(cm);
  const int incl = wave_incl_scan(cnt);
  const int n = __builtin_amdgcn_readlane(incl, 63);
  if (n > 64) {
    wave_select<NPL>(ck, lv, k, S);
    return;
  }
  int pos = incl - cnt;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    if ((cm >> i) & 1u) {
      S.cand_key[pos] = ck[i];
      S.cand_l[pos] = lv[i];
      ++pos;
    }
  }
  // zero keys after the last candidate up to a multiple of 4 (never ahead of a real key)
  if (lane >= n && lane < ((n + 3) & ~3)) S.cand_key[lane] = 0;
  wave_lds_fence();
  const uint64_t mine = lane < n ? S.cand_key[lane] : 0;
  const float ml = lane < n ? S.cand_l[lane] : 0.0f;
  int rk = 0;                                      // candidates ahead of this one
  for (int j = 0; j < n; j += 4) {
    const uint64_t c0 = S.cand_key[j], c1 = S.cand_key[j + 1];
    const uint64_t c2 = S.cand_key[j + 2], c3 = S.cand_key[j + 3];
    rk += (c0 > mine) + (c1 > mine) + (c2 > mine) + (c3 > mine);
  }
  if (lane < n && rk < k) {
    S.sel_e[rk] = (int32_t)~(uint32_t)mine;
    S.sel_l[rk] = ml;
  }
  wave_lds_fence();
}

// One wave per token: the decode path's exact top-k and renormalised sigmoid
// weights.  The logits are given, or are the sums of ksplit partial sums
// lpart[s][t][e], added in split order (and then stored to logits_out if
// that is not null).  With `disp`, all C <= 16 tokens are in this one
// workgroup (1024 threads) and it also writes the dispatch table: distinct
// experts in order of first use (pair order), each with its pairs in token
// order.  A router selection names distinct experts per token, so the pairs
// of expert e are marked by a token bitmask and a pair's place in the list is
// the number of earlier tokens in the mask.
template <int NW>
__global__ __launch_bounds__(64 * NW) void k_btopk(const float* logits, const float* lpart, int ksplit,
                                                   float* logits_out, int C, int E, int k,
                                                   int32_t* idx, float* w, int32_t* disp) {
  __shared__ SelectLds S[NW];
  constexpr int NPL = MOE_MAX_EXPERTS / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * NW + wave;
  if (t < C) {
    uint64_t ck[NPL];
    float lv[NPL];
    if (lpart) {
      // every partial load in flight before the first add; added in split order
      float pv[kKsplitMax][NPL];
#pragma unroll
      for (int sp = 0; sp < kKsplitMax; ++sp)
#pragma unroll
        for (int i = 0; i < NPL; ++i) {
          const int e = lane + 64 * i;
          pv[sp][i] = (e < E && sp < ksplit) ? lpart[((size_t)sp * C + t) * E + e] : 0.0f;
        }
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        float l = pv[0][i];
#pragma unroll
        for (int sp = 1; sp < kKsplitMax; ++sp)
          if (sp < ksplit) l += pv[sp][i];
        lv[i] = l;
      }
    } else {
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        const int e = lane + 64 * i;
        lv[i] = e < E ? logits[(size_t)t * E + e] : 0.0f;
      }
    }
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = lane + 64 * i;
      if (lpart && logits_out && e < E) logits_out[(size_t)t * E + e] = lv[i];
      ck[i] = e < E ? sel_key(lv[i], e) : 0;
    }
    wave_select_fast<NPL>(ck, lv, k, S[wave]);
    const float l = lane < k ? S[wave].sel_l[lane] : 0.0f;
    const float wt = route_weight(l, lane, k);
    if (lane < k) {
      idx[(size_t)t * k + lane] = S[wave].sel_e[lane];
      w[(size_t)t * k + lane] = wt;
    }
  }
  if (NW < MOE_MAX_DECODE_TOKENS || !disp) return;   // uniform: no barrier follows
  __shared__ uint32_t s_mask[MOE_MAX_EXPERTS];
  __shared__ int s_uof[MOE_MAX_EXPERTS];
  __shared__ int s_w[48];
  const int tid = threadIdx.x, CK = C * k;
  for (int e = tid; e < E; e += 64 * NW) s_mask[e] = 0u;
  __syncthreads();
  const int pt = tid / k, ps = tid - pt * k;          // pair tid = (token, slot)
  const int pe = tid < CK ? S[pt].sel_e[ps] : -1;
  if (tid < CK) atomicOr(&s_mask[pe], 1u << pt);
  __syncthreads();
  const uint32_t m = tid < CK ? s_mask[pe] : 0u;
  const int first = (tid < CK && (int)__builtin_ctz(m) == pt) ? 1 : 0;
  int nu = 0;
  const int u = block_excl_scan_1024(first, s_w, &nu);
  if (first) {
    s_uof[pe] = u;
    disp[disp_uexp(CK) + u] = pe;
    disp[disp_untok(CK) + u] = __builtin_popcount(m);
  }
  __syncthreads();
  if (tid < CK) disp[disp_upair(CK) + s_uof[pe] * C + __builtin_popcount(m & ((1u << pt) - 1u))] = tid;
  if (tid == 0) disp[0] = nu;
}

// ---------------------------------------------------------------------------
// Narrow tiles (up to 16 pairs, decode batches).  Each wave streams its rows'
// weights into registers, one K stage ahead, like the wide kernel; the
// activations, shared by the four waves, go straight from L2 into LDS with
// buffer_load ... lds (double-buffered, one stage ahead).  Those loads are
// issued from inline assembly: the compiler then does not know they write
// LDS and does not make every LDS read wait for all loads in flight; the
// kernel waits for them explicitly, by count.
// ---------------------------------------------------------------------------

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer descriptor words (the layout __builtin_amdgcn_make_buffer_rsrc
// builds): base, stride 0, num_records, flags.
__device__ __forceinline__ i32x4_t desc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return i32x4_t{(int)(uint32_t)b, (int)((uint32_t)(b >> 32) & 0xFFFFu), (int)bytes, 0x00020000};
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}
// lane l's 16 bytes at LDS m0 + 16 l (m0 must be the same in the whole wave)
__device__ __forceinline__ void dma16(i32x4_t r, uint32_t m0, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :
               : "s"(m0), "v"(voff), "s"(r)
               : "memory", "m0");
}
// lane l's 4 bytes at LDS m0 + 4 l
__device__ __forceinline__ void dma4(i32x4_t r, uint32_t m0, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen nt lds"
               :
               : "s"(m0), "v"(voff), "s"(r)
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

template <int FMT, bool GU, int RM>
__global__ __launch_bounds__(256) void k_bdma(BArgs a) {
  constexpr int NMAT = GU ? 2 : 1;
  constexpr int NT = NMAT * RM;                       // row tiles per wave
  constexpr int PL = GU ? 3 : 2;                      // activation planes
  constexpr int BPLANE = 16 * 512;                    // 16 rows x 256 bf16
  constexpr int NB_LD = PL * 2;                       // activation loads per thread per stage
  constexpr int NW_LD = NT * 3;                       // weight loads per thread per stage
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* bl = smem;                                 // [2][PL][BPLANE]
  __shared__ int s_pair[16], s_row[16], s_flags;

  const int tile = blockIdx.y;
  if (tile >= (int)a.meta[0]) return;
  const int e = a.tiles[2 * tile], t0 = a.tiles[2 * tile + 1];
  const int cnt = min(16, (int)a.count[e] - t0);
  const int tid = threadIdx.x;
  if (tid == 0) s_flags = 0;
  __syncthreads();
  if (tid < 16) {
    const int p = tid < cnt ? a.perm[a.boff[e] + t0 + tid] : -1;
    s_pair[tid] = p;
    const int row = p < 0 ? -1 : (GU ? p / a.k : p);
    s_row[tid] = row;
    if (GU && row >= 0) atomicOr(&s_flags, (int)a.xflag[row]);
  }
  __syncthreads();
  const int fl = s_flags;
  const int np = GU ? ((fl & 2) ? 3 : ((fl & 1) ? 2 : 1)) : 2;

  const int wave = tid >> 6, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const int H = a.H, I = a.I, B = (FMT == MOE_FMT_MXFP4) ? 32 : 16;
  const int K = GU ? H : I, N = GU ? I : H;
  const int row0 = blockIdx.x * (64 * RM) + wave * (16 * RM);
  const uint8_t* rec = a.base + (size_t)e * a.stride;
  __amdgpu_buffer_rsrc_t codes[NMAT], scales[NMAT];
  const uint32_t cbytes = (uint32_t)N * (K / 2), sbytes = (uint32_t)N * (K / B);
  codes[0] = view(rec + a.off[GU ? MOE_T_GATE_CODES : MOE_T_DOWN_CODES], cbytes);
  scales[0] = view(rec + a.off[GU ? MOE_T_GATE_SCALES : MOE_T_DOWN_SCALES], sbytes);
  if (GU) {
    codes[NMAT - 1] = view(rec + a.off[MOE_T_UP_CODES], cbytes);
    scales[NMAT - 1] = view(rec + a.off[MOE_T_UP_SCALES], sbytes);
  }
  uint32_t coff[RM], soff[RM];
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    const int row = row0 + 16 * r + r16;
    coff[r] = (uint32_t)row * (K / 2) + g * 32;
    soff[r] = (uint32_t)row * (K / B) + g * (64 / B);
  }
  const size_t CK = (size_t)a.C * a.k;
  const uint32_t plane_bytes = (uint32_t)((GU ? (size_t)a.C * H : CK * I) * 2);
  const i32x4_t src = desc(GU ? (const void*)a.xp : (const void*)a.hp, plane_bytes * (uint32_t)PL);
  const uint32_t bbase = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(bl));

  // this thread's part of an activation stage: for plane pl, DMA slot u of
  // wave w covers LDS bytes [(2w + u) * 1 KB, +1 KB) of the 8 KB plane, so
  // lane l writes row P / 512, 16-byte slot (P / 16) % 32 (P = its byte); it
  // loads the chunk that lands there under the swizzle chunk ^ (row & 15).
  uint32_t boff[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int P = (2 * wave + u) * 1024 + lane * 16;
    const int row = P >> 9, ch = ((P >> 4) & 31) ^ (row & 15);
    boff[u] = (row < cnt) ? ((uint32_t)s_row[row] * (uint32_t)K + (uint32_t)ch * 8u) * 2u : kNoLoad;
  }
  const int nkb = K / kSK;
  auto issue_b = [&](int kb) {
    const uint32_t buf = bbase + (uint32_t)((kb & 1) * PL * BPLANE);
    const bool ok = kb < nkb;
#pragma unroll
    for (int pl = 0; pl < PL; ++pl)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint32_t o = (ok && pl < np && boff[u] != kNoLoad)
                               ? boff[u] + (uint32_t)pl * plane_bytes + (uint32_t)kb * (kSK * 2)
                               : kNoLoad;
        dma16(src, (uint32_t)__builtin_amdgcn_readfirstlane(
                       (int)(buf + pl * BPLANE + (2 * wave + u) * 1024)), o);
      }
  };

  f32x4_t acc[NMAT][RM][1];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int r = 0; r < RM; ++r) acc[m][r][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // one K stage: activations of stage kb resident in LDS buffer kb & 1
  auto stage = [&](int kb, const StageW<FMT, NMAT, RM>& W) {
    const uint8_t* bb = bl + (kb & 1) * PL * BPLANE;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int c = t >> 2, s4 = t & 3;
      bf16x8_t A[NMAT][RM];
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int r = 0; r < RM; ++r) {
          const uint32_t sb = (FMT == MOE_FMT_MXFP4) ? ((W.sc[m][r] >> (8 * c)) & 0xFFu)
                                                     : ((W.sc[m][r] >> (8 * (2 * c + (s4 >> 1)))) & 0xFFu);
          A[m][r] = dequant8<FMT>(scale_word(W.q[m][r][c], s4), sb);
        }
      const int k16 = 8 * g + t;
      const uint8_t* bp = bb + r16 * 512 + ((k16 ^ r16) * 16);
#pragma unroll
      for (int pl = 0; pl < PL; ++pl) {
        if (pl >= np) break;
        const bf16x8_t Bv = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(bp + pl * BPLANE));
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int r = 0; r < RM; ++r)
            acc[m][r][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[m][r], Bv, acc[m][r][0], 0, 0, 0);
      }
    }
  };

  // Issue order W(0) B(0) W(1), then per stage kb: B(kb+1), [compute kb],
  // W(kb+2).  At stage kb the loads issued after B(kb) are W(kb+1) and
  // B(kb+1): waiting for at most NW_LD + NB_LD outstanding lands B(kb).  The
  // weights are registers the compiler waits for itself; W0/W1 alternate so a
  // buffer is reloaded in place after its stage (nkb is even).
  StageW<FMT, NMAT, RM> W0, W1;
  load_stage<FMT, NMAT, RM>(codes, scales, coff, soff, 0, true, W0);
  issue_b(0);
  load_stage<FMT, NMAT, RM>(codes, scales, coff, soff, 1, true, W1);
  for (int kb = 0; kb < nkb; kb += 2) {
    __syncthreads();                     // stage kb-1 is done: its buffer may be refilled
    issue_b(kb + 1);
    wait_vm<NW_LD + NB_LD>();            // this wave's activations of stage kb have landed
    __syncthreads();                     // ... and every wave's
    stage(kb, W0);
    load_stage<FMT, NMAT, RM>(codes, scales, coff, soff, kb + 2, kb + 2 < nkb, W0);
    __syncthreads();
    issue_b(kb + 2);
    wait_vm<NW_LD + NB_LD>();
    __syncthreads();
    stage(kb + 1, W1);
    load_stage<FMT, NMAT, RM>(codes, scales, coff, soff, kb + 3, kb + 3 < nkb, W1);
  }
  wait_vm<0>();                          // no load may still be writing LDS at exit

  const int orow0 = row0 + 4 * g;
  const int p = s_pair[r16];
  if (p < 0) return;
  if (GU) {
    float gg = 1.0f, gu = 1.0f;
    if (FMT == MOE_FMT_NVFP4) {
      const float* gl = reinterpret_cast<const float*>(rec + a.off[MOE_T_GLOBALS]);
      gg = gl[0];
      gu = gl[1];
    }
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      uint16_t hi[4], lo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float h = silu(gg * acc[0][r][0][j]) * (gu * acc[NMAT - 1][r][0][j]);
        hi[j] = bf16_bits(h);
        lo[j] = bf16_bits(h - bf16_float(hi[j]));
      }
      const size_t o = (size_t)p * I + orow0 + 16 * r;
      *reinterpret_cast<uint2*>(a.hp + o) =
          make_uint2((uint32_t)hi[0] | ((uint32_t)hi[1] << 16), (uint32_t)hi[2] | ((uint32_t)hi[3] << 16));
      *reinterpret_cast<uint2*>(a.hp + CK * I + o) =
          make_uint2((uint32_t)lo[0] | ((uint32_t)lo[1] << 16), (uint32_t)lo[2] | ((uint32_t)lo[3] << 16));
    }
  } else {
    float gd = 1.0f;
    if (FMT == MOE_FMT_NVFP4) gd = reinterpret_cast<const float*>(rec + a.off[MOE_T_GLOBALS])[2];
    const float wp = a.w[p] * gd;
#pragma unroll
    for (int r = 0; r < RM; ++r)
      *reinterpret_cast<float4*>(a.part + (size_t)p * H + orow0 + 16 * r) =
          make_float4(wp * acc[0][r][0][0], wp * acc[0][r][0][1], wp * acc[0][r][0][2],
                      wp * acc[0][r][0][3]);
  }
}

template <int FMT, bool GU, int RM, int NB, int NW>
moe_status launch_bmm(const BArgs& a, dim3 grid, hipStream_t st) {
  constexpr int PL = GU ? (NB == 1 ? 3 : 1) : 2;
  constexpr int bytes = 2 * PL * 16 * NB * kSStride * 2;
  static std::atomic<bool> attr_set[64];   // per device, set once (concurrent setters agree)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (!attr_set[dev].load(std::memory_order_relaxed)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(k_bmm<FMT, GU, RM, NB, NW>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess)
      return MOE_ERR_DEVICE;
    attr_set[dev].store(true, std::memory_order_relaxed);
  }
  hipLaunchKernelGGL((k_bmm<FMT, GU, RM, NB, NW>), grid, dim3(64 * NW), bytes, st, a);
  return MOE_OK;
}

template <int FMT, int RM, int NB, int NW>
moe_status launch_bmm_dnp(const BArgs& a, dim3 grid, hipStream_t st) {
  constexpr int bytes = 2 * 2 * 16 * NB * kSStride * 2;
  static std::atomic<bool> attr_set[64];   // per device, set once (concurrent setters agree)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (!attr_set[dev].load(std::memory_order_relaxed)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(k_bmm_dnp<FMT, RM, NB, NW>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess)
      return MOE_ERR_DEVICE;
    attr_set[dev].store(true, std::memory_order_relaxed);
  }
  hipLaunchKernelGGL((k_bmm_dnp<FMT, RM, NB, NW>), grid, dim3(64 * NW), bytes, st, a);
  return MOE_OK;
}

template <int FMT, bool GU, int RM>
constexpr int bdma_lds_bytes() {
  return 2 * (GU ? 3 : 2) * 16 * 512;
}

template <int FMT, bool GU, int RM>
moe_status launch_bdma(const BArgs& a, dim3 grid, hipStream_t st) {
  constexpr int bytes = bdma_lds_bytes<FMT, GU, RM>();
  static std::atomic<bool> attr_set[64];   // per device, set once (concurrent setters agree)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (!attr_set[dev].load(std::memory_order_relaxed)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(k_bdma<FMT, GU, RM>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess)
      return MOE_ERR_DEVICE;
    attr_set[dev].store(true, std::memory_order_relaxed);
  }
  hipLaunchKernelGGL((k_bdma<FMT, GU, RM>), grid, dim3(256), bytes, st, a);
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// Decode batches: each distinct expert streamed once, as dot products
// ---------------------------------------------------------------------------
// For C <= MOE_MAX_DECODE_TOKENS tokens the selected experts are read once
// each (the dispatch table lists the distinct experts and their pairs), as in
// the batch-1 kernel: 16-lane groups walk weight rows 256 contiguous bytes per
// instruction, dequantise in registers and take dot products with the staged
// activations of every pair of the expert.  k_dstream<GU> computes gate and up
// (K = H) with SwiGLU into h; k_dstream<DN> computes down (K = I) times the
// routing weight into one row per pair; k_bcombine adds each token's rows.
//
// Work split.  The row steps of all distinct experts (GU: 32 rows of I, one
// gate and up row per lane group; DN: 64 rows of H, two per lane group) are
// laid end to end and cut into one contiguous range per workgroup of equal
// cost, a row step of expert u costing passes_u * dm_costw(GU, K) + 4 tokens_u
// (weight bytes plus per-token work, in quarters of one token's work).  A workgroup walks its range expert by
// expert; for each it stages the activations of up to ntp pairs in LDS
// (fp32, 36 floats per 32 so the 16 lanes of a group hit distinct banks) and
// streams its rows through a register pipeline of kDPipe stages of kDSC
// chunks per lane.
constexpr int kDWG = 512;                  // threads per workgroup
constexpr int kDGrp = kDWG / 16;           // 16-lane groups per workgroup
constexpr int kDSC = 2;                    // 16-byte chunks per lane per pipeline stage
constexpr int kDPipe = 3;                  // register buffers of the weight stream
// One weight pass of a row step in quarters of a token's work on it (the
// matrix-core products, their LDS operands and the epilogue): per-workgroup
// clocks put a pass of a row step (64 rows of K) at about K / 270 tokens on
// gate/up and K / 380 on down.
__device__ __forceinline__ int dm_costw(bool GU, int K) { return GU ? (4 * K + 135) / 270 : (4 * K + 190) / 380; }
constexpr int kDLds = 131072;              // LDS bytes for staged activations
constexpr int kDMaxU = MOE_MAX_DECODE_TOKENS * MOE_MAX_TOPK;   // distinct experts at most

struct DArgs {
  const uint8_t* base;
  int64_t stride;
  int64_t off[MOE_NUM_TENSORS];
  int E, H, I, k, C;
  const int32_t* disp;    // dispatch table
  const float* x;         // [C][H]
  const float* w;         // [C*k]
  float* h;               // [C*k][I]
  float* part;            // [C*k][H]
  int ntp;                // pairs staged per pass (1, 2, 4 or 8)
};

// Staged activations of the matrix-core streams: two bf16 planes (hi, lo) of
// every staged pair, pair t of plane p at byte p * dm_ps + t * dm_ts.  The
// strides are 32 and 16 bytes past a multiple of 128, so the 8 lanes of each
// phase of a 16-byte LDS read (4 columns x 2 chunks) hit distinct banks.
__host__ __device__ __forceinline__ int dm_ts(int K) { return 2 * K + 32; }
__host__ __device__ __forceinline__ int dm_slots(int ntp) { return ntp < 2 ? 2 : ntp; }
__host__ __device__ __forceinline__ int dm_ps(int K, int ntp) {
  return (dm_slots(ntp) * dm_ts(K) + 127) / 128 * 128 + 16;
}

typedef short bf16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x4_t as_bf16x4(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(bf16x4_t, u32x2_t{lo, hi});
}

// acc[r][g] += one 32-element chunk of NR rows against the pairs of column
// group g (< ng), on the 4 x 4 x 4 matrix-core product of 16 blocks: lane
// 4b + i holds row i's chunk b (A: 4 K values per product, 8 products per
// chunk), lane 4b + j holds column j of the same K values (B: plane j & 1 of
// pair 2g + (j >> 1)), and lane 4b + j's accumulator i is row i, column j,
// summed over chunk b's K values only (the epilogue adds the 16 blocks).
// MXFP4: the conversion applies the block's power-of-two scale exactly.
// NVFP4: each 16-element half is summed on its own and multiplied by its
// row's e4m3 scale, which the lane takes from the quad lane that loaded it.
template <int FMT, int NR, int G>
__device__ __forceinline__ void chunk_mfma(const uint4 (&q)[NR], const uint32_t (&sc)[NR],
                                           const uint8_t* xb, uint32_t gstride, int nt,
                                           f32x4_t (&acc)[NR][G]) {
  const int ng = (nt + 1) / 2;
  constexpr bool MX = FMT == MOE_FMT_MXFP4;
  bf16x4_t av[NR][8];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const float s = MX ? __uint_as_float((sc[r] & 0xFFu) << 23) : 1.0f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t wd = (d == 0) ? q[r].x : (d == 1) ? q[r].y : (d == 2) ? q[r].z : q[r].w;
      const uint32_t p0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, s, 0));
      const uint32_t p1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, s, 1));
      const uint32_t p2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, s, 2));
      const uint32_t p3 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, s, 3));
      av[r][2 * d] = as_bf16x4(p0, p1);
      av[r][2 * d + 1] = as_bf16x4(p2, p3);
    }
  }
  float ns[NR][2][4];                    // NVFP4: [row stream][half][row i of the quad]
  if (!MX) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int w0 = __builtin_amdgcn_mov_dpp((int)sc[r], 0x00, 0xF, 0xF, false);
      const int w1 = __builtin_amdgcn_mov_dpp((int)sc[r], 0x55, 0xF, 0xF, false);
      const int w2 = __builtin_amdgcn_mov_dpp((int)sc[r], 0xAA, 0xF, 0xF, false);
      const int w3 = __builtin_amdgcn_mov_dpp((int)sc[r], 0xFF, 0xF, 0xF, false);
      ns[r][0][0] = __builtin_amdgcn_cvt_f32_fp8(w0, 0); ns[r][1][0] = __builtin_amdgcn_cvt_f32_fp8(w0, 1);
      ns[r][0][1] = __builtin_amdgcn_cvt_f32_fp8(w1, 0); ns[r][1][1] = __builtin_amdgcn_cvt_f32_fp8(w1, 1);
      ns[r][0][2] = __builtin_amdgcn_cvt_f32_fp8(w2, 0); ns[r][1][2] = __builtin_amdgcn_cvt_f32_fp8(w2, 1);
      ns[r][0][3] = __builtin_amdgcn_cvt_f32_fp8(w3, 0); ns[r][1][3] = __builtin_amdgcn_cvt_f32_fp8(w3, 1);
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (g >= ng) break;
    // a column of a pair past the pass's count stays zero without an LDS read
    uint4 b0 = make_uint4(0u, 0u, 0u, 0u), b1 = b0, b2 = b0, b3 = b0;
    if (2 * g + ((threadIdx.x >> 1) & 1) < nt) {
      const uint4* bp = reinterpret_cast<const uint4*>(xb + g * gstride);
      b0 = bp[0]; b1 = bp[1]; b2 = bp[2]; b3 = bp[3];
    }
    const bf16x4_t bv[8] = {as_bf16x4(b0.x, b0.y), as_bf16x4(b0.z, b0.w), as_bf16x4(b1.x, b1.y),
                            as_bf16x4(b1.z, b1.w), as_bf16x4(b2.x, b2.y), as_bf16x4(b2.z, b2.w),
                            as_bf16x4(b3.x, b3.y), as_bf16x4(b3.z, b3.w)};
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      if (MX) {
#pragma unroll
        for (int m = 0; m < 8; ++m)
          acc[r][g] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(av[r][m], bv[m], acc[r][g], 0, 0, 0);
      } else {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          f32x4_t t = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int m = 4 * hf; m < 4 * hf + 4; ++m)
            t = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(av[r][m], bv[m], t, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[r][g][i] += ns[r][hf][i] * t[i];
        }
      }
    }
  }
}

// One wave's stream over `rows` row groups of one expert (4 rows each; lane
// 4b + i loads row i's 16-byte slot b of each 256-byte chunk; row group ri at
// byte offset coff[r] + ri * rstride of stream r, scales likewise), kch
// chunks per row, pipelined across row groups.  xb: this lane's B column in
// LDS (plane, pair and slot applied), chunks 1024 bytes apart.  done(ri, acc)
// gets the accumulators after each row group's last chunk.
template <int FMT, int NR, int G, class Done>
__device__ __forceinline__ void dmma_rows(const __amdgpu_buffer_rsrc_t (&crs)[NR],
                                          const __amdgpu_buffer_rsrc_t (&srs)[NR],
                                          const uint32_t (&coff)[NR], const uint32_t (&soff)[NR],
                                          uint32_t rstride, uint32_t sstride, int rows, int kch,
                                          const uint8_t* xb, uint32_t gstride, int nt, Done done) {
  constexpr int SB = (FMT == MOE_FMT_MXFP4) ? 16 : 32;   // scale bytes per chunk of a row
  uint4 q[kDPipe][kDSC][NR];
  uint32_t sc[kDPipe][kDSC][NR];
  int lrow = 0, lc = 0;                  // next chunk to load
  int crow = 0, cc = 0;                  // next chunk to multiply
  // Loads are unconditional: past the last row the offset is out of range,
  // which reads zeros without touching memory and keeps the count exact.
  auto load = [&](uint4 (&qq)[kDSC][NR], uint32_t (&ss)[kDSC][NR]) {
#pragma unroll
    for (int b = 0; b < kDSC; ++b) {
      const bool ok = lrow < rows;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const uint32_t co = ok ? coff[r] + (uint32_t)lrow * rstride + 256u * (uint32_t)lc : kNoLoad;
        const uint32_t so = ok ? soff[r] + (uint32_t)lrow * sstride + (uint32_t)(SB * lc) : kNoLoad;
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(crs[r], (int)co, 0, kCachePolicyNt);
        qq[b][r] = make_uint4(v[0], v[1], v[2], v[3]);
        if (FMT == MOE_FMT_MXFP4)
          ss[b][r] = __builtin_amdgcn_raw_buffer_load_b8(srs[r], (int)so, 0, kCachePolicyNt);
        else
          ss[b][r] = __builtin_amdgcn_raw_buffer_load_b16(srs[r], (int)so, 0, kCachePolicyNt);
      }
      if (++lc == kch) { lc = 0; ++lrow; }
    }
  };
  f32x4_t acc[NR][G];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int g = 0; g < G; ++g) acc[r][g] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  auto step = [&](const uint4 (&qq)[kDSC][NR], const uint32_t (&ss)[kDSC][NR]) {
#pragma unroll
    for (int b = 0; b < kDSC; ++b) {
      if (crow < rows) {
        chunk_mfma<FMT, NR, G>(qq[b], ss[b], xb + 1024 * cc, gstride, nt, acc);
        if (cc == kch - 1) {
          done(crow, acc);
#pragma unroll
          for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int g = 0; g < G; ++g) acc[r][g] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
        if (++cc == kch) { cc = 0; ++crow; }
      }
    }
  };
  // Whole groups of kDPipe stages, with no exit between them: stages past
  // the last load zeros without memory traffic and multiply nothing (the
  // crow < rows test), and a straight loop body lets the compiler keep its
  // waits partial (an exit inside the group made it wait for nearly every
  // load in flight at the end of each pass through the loop).
  const int nst = (rows * kch + kDSC - 1) / kDSC;
#pragma unroll
  for (int j = 0; j < kDPipe - 1; ++j) load(q[j], sc[j]);
  for (int st0 = 0; st0 < nst; st0 += kDPipe) {
#pragma unroll
    for (int j = 0; j < kDPipe; ++j) {
      __builtin_amdgcn_sched_barrier(0);
      load(q[(j + kDPipe - 1) % kDPipe], sc[(j + kDPipe - 1) % kDPipe]);
      __builtin_amdgcn_sched_barrier(0);
      step(q[j], sc[j]);
    }
  }
}

// Sum of a row-group accumulator over the 16 blocks (lanes 4b + j, same j)
// and over the hi and lo planes (columns j and j ^ 1).  Returns, in each lane
// of 16-lane row q, row q's dot product with pair 2g + ((lane >> 1) & 1): the
// four rows' sums are first split across the lane rows (two exchanges that
// each halve what a lane carries), then the row's four blocks of the same
// column and the two planes are added with DPP.  The same lane always holds
// the result a store takes, so the sums are the same bits on every call.
__device__ __forceinline__ float dm_reduce(const f32x4_t& v) {
  const int q = (threadIdx.x >> 4) & 3;
  const bool up = q >= 2, odd = q & 1;
  float k0 = up ? v[2] : v[0], k1 = up ? v[3] : v[1];
  const float s0 = up ? v[0] : v[2], s1 = up ? v[1] : v[3];
  k0 += __shfl_xor(s0, 32, 64);
  k1 += __shfl_xor(s1, 32, 64);
  float k = odd ? k1 : k0;
  k += __shfl_xor(odd ? k0 : k1, 16, 64);
  k += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(k), 0x124, 0xF, 0xF, false));  // row_ror:4
  k += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(k), 0x128, 0xF, 0xF, false));  // row_ror:8
  k += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(k), 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
  return k;
}

// Workgroup-wide exclusive scan (blockDim.x = kDWG).
__device__ int block_excl_scan_dwg(int v, int* s_w, int* total) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int incl = wave_incl_scan(v);
  if (lane == 63) s_w[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kDWG / 64; ++w) {
    const int s = s_w[w];
    if (w < wave) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

// One pass of one distinct expert's rows [rsb, rse) of row steps against NTC
// staged pairs (nt of them used): the gate/up rows with SwiGLU into h, or the
// down rows times the routing weight into part.  NTC is a compile-time bound
// (2, 4 or 8 pairs: 1, 2 or 4 column groups of the matrix-core product), so
// that no column group past the pass's pairs is multiplied.  Wave w's rows of
// a row step are 4w .. 4w + 3 (gate/up: of the step's 32; down: of each half
// of its 64).
template <int FMT, bool GU, int NTC>
__device__ __forceinline__ void dstream_pass(const DArgs& a, const uint8_t* rec, int rsb, int rse,
                                             const uint8_t* xs, int ps, int ts, int nt,
                                             const int* s_pairs, const float* s_wgt) {
  const int H = a.H, I = a.I, K = GU ? H : I;
  const int B = (FMT == MOE_FMT_MXFP4) ? 32 : 16;
  constexpr int RS = GU ? kDGrp : 2 * kDGrp;          // rows per row step
  constexpr int G = NTC / 2;                          // column groups of 2 pairs
  const int kch = K / 512;                            // 256-byte chunks per row
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int il = lane & 3, bq = lane >> 2;            // load: row il of the wave's 4, slot bq
  const int iw = lane >> 4, tw = (lane >> 1) & 1;       // store: row iw, pair 2g + tw
  const bool writer = (lane & 13) == 0;                   // lanes 16 iw + 2 tw
  const uint32_t rowb = (uint32_t)(K / 2), srowb = (uint32_t)(K / B);
  const int rows = rse - rsb;
  const int ng = (nt + 1) / 2;
  const uint8_t* xb = xs + (lane & 1) * ps + ((lane >> 1) & 1) * ts + 64 * bq;
  const uint32_t gstride = 2u * (uint32_t)ts;
  const int grp = 4 * wave + il;                      // this lane's load row within a row step
  const int gw = 4 * wave + iw;                       // this lane's store row
  if (GU) {
    __amdgpu_buffer_rsrc_t crs[2], srs[2];
    crs[0] = view(rec + a.off[MOE_T_GATE_CODES], (uint32_t)I * rowb);
    crs[1] = view(rec + a.off[MOE_T_UP_CODES], (uint32_t)I * rowb);
    srs[0] = view(rec + a.off[MOE_T_GATE_SCALES], (uint32_t)I * srowb);
    srs[1] = view(rec + a.off[MOE_T_UP_SCALES], (uint32_t)I * srowb);
    const int row0 = rsb * RS + grp;
    const uint32_t coff[2] = {(uint32_t)row0 * rowb + bq * 16, (uint32_t)row0 * rowb + bq * 16};
    const uint32_t soff[2] = {(uint32_t)row0 * srowb + bq * (32 / B), (uint32_t)row0 * srowb + bq * (32 / B)};
    float gg = 1.0f, gu = 1.0f;
    if (FMT == MOE_FMT_NVFP4) {
      const float* gl = reinterpret_cast<const float*>(rec + a.off[MOE_T_GLOBALS]);
      gg = gl[0];
      gu = gl[1];
    }
    dmma_rows<FMT, 2, G>(crs, srs, coff, soff, RS * rowb, RS * srowb, rows, kch, xb, gstride, nt,
                         [&](int ri, f32x4_t (&acc)[2][G]) {
      const int j = (rsb + ri) * RS + gw;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (g >= ng) break;
        const float gs = dm_reduce(acc[0][g]);
        const float us = dm_reduce(acc[1][g]);
        const int t = 2 * g + tw;
        if (writer && t < nt) a.h[(size_t)s_pairs[t] * I + j] = silu(gg * gs) * (gu * us);
      }
    });
  } else {
    __amdgpu_buffer_rsrc_t crs[2], srs[2];
    crs[0] = crs[1] = view(rec + a.off[MOE_T_DOWN_CODES], (uint32_t)H * rowb);
    srs[0] = srs[1] = view(rec + a.off[MOE_T_DOWN_SCALES], (uint32_t)H * srowb);
    const int row0 = rsb * RS + grp;                // and row0 + kDGrp
    const uint32_t coff[2] = {(uint32_t)row0 * rowb + bq * 16, (uint32_t)(row0 + kDGrp) * rowb + bq * 16};
    const uint32_t soff[2] = {(uint32_t)row0 * srowb + bq * (32 / B),
                              (uint32_t)(row0 + kDGrp) * srowb + bq * (32 / B)};
    float gd = 1.0f;
    if (FMT == MOE_FMT_NVFP4) gd = reinterpret_cast<const float*>(rec + a.off[MOE_T_GLOBALS])[2];
    dmma_rows<FMT, 2, G>(crs, srs, coff, soff, RS * rowb, RS * srowb, rows, kch, xb, gstride, nt,
                         [&](int ri, f32x4_t (&acc)[2][G]) {
      const int j = (rsb + ri) * RS + gw;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (g >= ng) break;
        const float y0 = dm_reduce(acc[0][g]);
        const float y1 = dm_reduce(acc[1][g]);
        const int t = 2 * g + tw;
        if (writer && t < nt) {
          const int p = s_pairs[t];
          const float wp = s_wgt[t] * gd;               // routing weight, staged with the pairs
          a.part[(size_t)p * H + j] = wp * y0;
          a.part[(size_t)p * H + j + kDGrp] = wp * y1;
        }
      }
    });
  }
}

template <int FMT, bool GU, int NT>
__global__ __launch_bounds__(kDWG) void k_dstream(DArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];   // [2][dm_slots(ntp)] bf16 rows
  __shared__ int s_pref[kDMaxU + 1];
  __shared__ int s_w[kDWG / 64];
  __shared__ int s_bound[2];
  __shared__ int s_pairs[MOE_MAX_DECODE_TOKENS];
  __shared__ float s_wgt[MOE_MAX_DECODE_TOKENS];      // down: the pairs' routing weights
  const int tid = threadIdx.x;
  const int CK = a.C * a.k;
  const int nu = a.disp[0];
  const int H = a.H, I = a.I, K = GU ? H : I, N = GU ? I : H;
  constexpr int RS = GU ? kDGrp : 2 * kDGrp;          // rows per row step
  const int nrs = N / RS;
  const int ntp = a.ntp;
  const int ts = dm_ts(K), ps = dm_ps(K, ntp);        // LDS bytes: pair and plane strides

  // cost prefix over the distinct experts, then this workgroup's range
  const int ntok = tid < CK ? a.disp[disp_untok(CK) + tid] : 0;   // loaded beside nu
  const int wu = tid < nu ? ((ntok + ntp - 1) / ntp) * dm_costw(GU, K) + 4 * ntok : 0;
  int total = 0;
  const int pre = block_excl_scan_dwg(tid < nu ? wu * nrs : 0, s_w, &total);
  if (tid < nu) s_pref[tid] = pre;
  if (tid == 0) {
    s_pref[nu] = total;
    s_bound[0] = s_bound[1] = nu * nrs;
  }
  __syncthreads();
  const int G = (int)gridDim.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t v = (int64_t)(blockIdx.x + i) * total / G;
    if (tid < nu && v >= s_pref[tid] && v < s_pref[tid + 1]) {
      const int rs = (int)((v - s_pref[tid] + wu - 1) / wu);   // first row step starting at or after v
      s_bound[i] = tid * nrs + rs;
    }
  }
  __syncthreads();
  const int g0 = s_bound[0], g1 = s_bound[1];

  for (int u = g0 / nrs; u * nrs < g1; ++u) {
    const int rsb = max(g0 - u * nrs, 0), rse = min(g1 - u * nrs, nrs);
    if (rsb >= rse) continue;
    const int e = a.disp[disp_uexp(CK) + u];
    const int nt_u = a.disp[disp_untok(CK) + u];
    const uint8_t* rec = a.base + (size_t)e * a.stride;
    for (int p0 = 0; p0 < nt_u; p0 += ntp) {
      const int nt = min(ntp, nt_u - p0);
      __syncthreads();                                  // the previous pass is done with LDS
      if (tid < nt) {
        const int p = a.disp[disp_upair(CK) + u * a.C + p0 + tid];
        s_pairs[tid] = p;
        if (!GU) s_wgt[tid] = a.w[p];
      }
      __syncthreads();
      // each activation as hi = bf16(v) and lo = bf16(v - hi) (v - hi is exact
      // in fp32; hi + lo is v to within 2^-17 relative); the pair slot after
      // an odd count is zero, so the last column group's second pair adds 0
      const int ntc = (nt + 1) & ~1;
      for (int q = tid * 4; q < ntc * K; q += kDWG * 4) {
        const int t = q / K, kk = q - t * K;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (t < nt) {
          const int p = s_pairs[t];
          v = GU ? *reinterpret_cast<const float4*>(a.x + (size_t)(p / a.k) * H + kk)
                 : *reinterpret_cast<const float4*>(a.h + (size_t)p * I + kk);
        }
        const uint16_t h0 = bf16_bits(v.x), h1 = bf16_bits(v.y), h2 = bf16_bits(v.z), h3 = bf16_bits(v.w);
        const uint16_t l0 = bf16_bits(v.x - bf16_float(h0)), l1 = bf16_bits(v.y - bf16_float(h1));
        const uint16_t l2 = bf16_bits(v.z - bf16_float(h2)), l3 = bf16_bits(v.w - bf16_float(h3));
        uint8_t* d = xs + t * ts + 2 * kk;
        *reinterpret_cast<uint2*>(d) = make_uint2(h0 | ((uint32_t)h1 << 16), h2 | ((uint32_t)h3 << 16));
        *reinterpret_cast<uint2*>(d + ps) = make_uint2(l0 | ((uint32_t)l1 << 16), l2 | ((uint32_t)l3 << 16));
      }
      __syncthreads();
      // the smallest instance that holds the pass, so that no column group
      // past its pairs is multiplied
      if (NT <= 2 || nt <= 2) dstream_pass<FMT, GU, 2>(a, rec, rsb, rse, xs, ps, ts, nt, s_pairs, s_wgt);
      else if (NT == 4 || nt <= 4) dstream_pass<FMT, GU, 4>(a, rec, rsb, rse, xs, ps, ts, nt, s_pairs, s_wgt);
      else dstream_pass<FMT, GU, 8>(a, rec, rsb, rse, xs, ps, ts, nt, s_pairs, s_wgt);
    }
  }
}

template <int FMT, bool GU, int NT>
moe_status launch_dstream_nt(const DArgs& a, int grid, int lds, hipStream_t st) {
  static std::atomic<bool> attr_set[64];   // per device, set once (concurrent setters agree)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (!attr_set[dev].load(std::memory_order_relaxed)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(k_dstream<FMT, GU, NT>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kDLds) != hipSuccess)
      return MOE_ERR_DEVICE;
    attr_set[dev].store(true, std::memory_order_relaxed);
  }
  hipLaunchKernelGGL((k_dstream<FMT, GU, NT>), dim3(grid), dim3(kDWG), lds, st, a);
  return MOE_OK;
}

// The kernel instance with NT = a.ntp register slots per row for the pairs.
template <int FMT, bool GU>
moe_status launch_dstream(const DArgs& a, int grid, int lds, hipStream_t st) {
  switch (a.ntp) {
    case 1: return launch_dstream_nt<FMT, GU, 1>(a, grid, lds, st);
    case 2: return launch_dstream_nt<FMT, GU, 2>(a, grid, lds, st);
    case 4: return launch_dstream_nt<FMT, GU, 4>(a, grid, lds, st);
    case 8: return launch_dstream_nt<FMT, GU, 8>(a, grid, lds, st);
    default: return MOE_ERR_UNSUPPORTED;
  }
}

// Pairs per activation pass: the largest of 8, 4, 2, 1 whose two bf16 planes
// fit the LDS budget; 0 if not even one does.
int dstream_ntp(int K) {
  for (int n = 8; n >= 1; n >>= 1)
    if (2 * dm_ps(K, n) <= kDLds) return n;
  return 0;
}

// Workgroups of the decode-batch streams: one per compute unit.
int dstream_grid() {
  static std::atomic<int> cache[64];   // per device, 0 until first asked
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
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
  hipLaunchKernelGGL(k_btopk<8>, dim3((C + 7) / 8), dim3(512), 0, st, lg, nullptr, 0, nullptr, C, E,
                     k, idx, w, nullptr);
  return status_of_launch();
}

moe_status launch_topk_parts(const float* lpart, int ksplit, float* logits_out, int C, int E, int k,
                             int32_t* idx, float* w, int32_t* disp, hipStream_t st) {
  if (disp) {
    if (C > MOE_MAX_DECODE_TOKENS || C * k > 1024) return MOE_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(k_btopk<MOE_MAX_DECODE_TOKENS>, dim3(1), dim3(64 * MOE_MAX_DECODE_TOKENS), 0,
                       st, nullptr, lpart, ksplit, logits_out, C, E, k, idx, w, disp);
  } else {
    hipLaunchKernelGGL(k_btopk<8>, dim3((C + 7) / 8), dim3(512), 0, st, nullptr, lpart, ksplit,
                       logits_out, C, E, k, idx, w, nullptr);
  }
  return status_of_launch();
}

moe_status launch_batched_experts(const moe_bank* b, const float* x, int C, int k,
                                  const int32_t* idx, const float* w, float* out, uint8_t* ws,
                                  const WsLayout& L, hipStream_t st) {
  const int H = b->hidden, I = b->inter;
  if (!batched_shape_ok(b)) return MOE_ERR_UNSUPPORTED;
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
  const dim3 ggu(I / (16 * kRmGU * kNwGU), maxt), gdn(H / (16 * kRmDN * kNwDN), maxt);
  const dim3 gpers(dstream_grid());                // persistent down GEMM: one workgroup per CU
  const dim3 ggun(I / (64 * kRmGUn), maxt), gdnn(H / (64 * kRmDNn), maxt);
#define RF4_BMM(F)                                                                        \
  do {                                                                                    \
    if (a.ntok == 16) {                                                                   \
      moe_status m = launch_bdma<F, true, kRmGUn>(a, ggun, st);                           \
      if (m == MOE_OK) m = launch_bdma<F, false, kRmDNn>(a, gdnn, st);                    \
      if (m != MOE_OK) return m;                                                          \
    } else {                                                                              \
      moe_status m = launch_bmm<F, true, kRmGU, 4, kNwGU>(a, ggu, st);                    \
      if (m == MOE_OK)                                                                    \
        m = I >= 4 * kSK ? launch_bmm_dnp<F, kRmDN, 4, kNwDN>(a, gpers, st)               \
                         : launch_bmm<F, false, kRmDN, 4, kNwDN>(a, gdn, st);             \
      if (m != MOE_OK) return m;                                                          \
    }                                                                                     \
  } while (0)
  if (b->format == MOE_FMT_MXFP4) RF4_BMM(MOE_FMT_MXFP4);
  else RF4_BMM(MOE_FMT_NVFP4);
#undef RF4_BMM
  hipLaunchKernelGGL(k_bcombine, dim3((H / 4 + 255) / 256, C), dim3(256), 0, st, a);
  return status_of_launch();
}

bool batched_decode_shape(const moe_bank* b, int C) {
  const int H = b->hidden, I = b->inter;
  return batched_shape_ok(b) && C >= 1 && C <= MOE_MAX_DECODE_TOKENS && dstream_ntp(H) > 0 &&
         dstream_ntp(I) > 0 && (size_t)H * (size_t)I < ((size_t)1 << 32);
}

moe_status launch_batched_decode(const moe_bank* b, const float* x, int C, int k,
                                 const int32_t* idx, const float* w, float* out, uint8_t* ws,
                                 const WsLayout& L, hipStream_t st) {
  if (!batched_decode_shape(b, C)) return MOE_ERR_UNSUPPORTED;
  const int H = b->hidden, I = b->inter;
  int cp = 1;                                   // C rounded up to a power of two
  while (cp < C) cp <<= 1;
  const int ntg = dstream_ntp(H) < cp ? dstream_ntp(H) : cp;
  const int ntd = dstream_ntp(I) < cp ? dstream_ntp(I) : cp;
  DArgs a;
  a.base = static_cast<const uint8_t*>(b->base);
  a.stride = b->expert_stride;
  for (int t = 0; t < MOE_NUM_TENSORS; ++t) a.off[t] = b->offset[t];
  a.E = b->num_experts; a.H = H; a.I = I; a.k = k; a.C = C;
  a.disp = reinterpret_cast<const int32_t*>(ws + L.disp);
  a.x = x;
  a.w = w;
  a.h = reinterpret_cast<float*>(ws + L.h);
  a.part = reinterpret_cast<float*>(ws + L.part);
  const int grid = dstream_grid();
  moe_status m;
  a.ntp = ntg;
  const int lds_g = 2 * dm_ps(H, ntg);
  if (b->format == MOE_FMT_MXFP4) m = launch_dstream<MOE_FMT_MXFP4, true>(a, grid, lds_g, st);
  else m = launch_dstream<MOE_FMT_NVFP4, true>(a, grid, lds_g, st);
  if (m != MOE_OK) return m;
  a.ntp = ntd;
  const int lds_d = 2 * dm_ps(I, ntd);
  if (b->format == MOE_FMT_MXFP4) m = launch_dstream<MOE_FMT_MXFP4, false>(a, grid, lds_d, st);
  else m = launch_dstream<MOE_FMT_NVFP4, false>(a, grid, lds_d, st);
  if (m != MOE_OK) return m;
  BArgs c;
  c.E = a.E; c.H = H; c.I = I; c.k = k; c.C = C;
  c.idx = idx;
  c.part = a.part;
  c.out = out;
  hipLaunchKernelGGL(k_bcombine, dim3((H / 4 + 255) / 256, C), dim3(256), 0, st, c);
  return status_of_launch();
}

}  // namespace rf4
