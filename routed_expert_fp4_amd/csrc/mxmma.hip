// libroutedfp4, MXFP4 experts on the block-scaled FP4 matrix cores.
//
// Page "SparkInfer-K3", Roadmap, "Later · B200 / B300 -- the Blackwell delta",
// notes that Hopper has no FP4 tensor core, so every low-bit expert product
// first dequantises the weights to bf16; a matrix core that takes FP4 operands
// with block scales removes that step.  CDNA4 has one:
// v_mfma_scale_f32_16x16x128_f8f6f4 takes A and B in FP4/FP6/FP8 with one
// E8M0 scale per 32 K values of each row and column.  An MXFP4 weight row is
// exactly such an operand (e2m1 codes, one e8m0 scale per 32), so the weights
// go from HBM to the matrix core as they are stored.  NVFP4 (e4m3 per 16) has
// no such form and stays on the bf16 path.
//
// The activations (x, then h) are fp32.  They go in as T terms of OCP e4m3
// with an E8M0 scale per 32 values each: term 1 is x rounded to e4m3 under a
// scale that puts the block's largest magnitude in [128, 256); term 2 the same
// for what is left, and so on.  Each term takes about 4 more bits of every
// value.  T = 1 is the lossy single-term mode.
//
// The instruction's own sums are not exact.  Measured on the device with
// in-bounds probes: it adds the products of each aligned group of 8 K values
// in fixed point, with the quantum 2^(emax - 13), emax being the group's
// largest exponent sum (the two operands' exponents plus their scales'), and
// truncates each product toward zero to that quantum; the 16 group sums then
// go into the fp32 accumulator with round-to-nearest-even.  (One K = 128 sum
// of 256 + 127 * 2^-6 comes out as 257.875: the 7 small products in the
// group of the 256 are lost.)  The term split therefore keeps every group's
// exponents within a window where no product is truncated (k_mq_split), so
// from T = 4 on the only errors are the unrepresented remainder and the fp32
// accumulation: a near-exact mode.
//
// Operand layouts of the 16x16x128 instruction (established on the device
// with in-bounds probes): lane l holds row or column l % 16.  FP4 A: the 16
// bytes of lane group g = l / 16 are K values 32g .. 32g+31, low nibble
// first, and the lane's scale byte covers exactly those.  FP8 B: the lane's
// bytes 0..15 are K values 16g .. 16g+15 and bytes 16..31 are K values
// 64+16g .. 64+16g+15; the scale byte of lane group g covers K values
// 32g .. 32g+31.  Output: lane l holds rows 4 (l / 16) .. +3 of column l % 16.
//
// Kernels (one call, all on the caller's stream):
//   k_mq_split   fp32 rows -> T e4m3 terms + E8M0 scales (x, later h); the x
//                launch also clears the per-expert counters
//   k_mcount, k_mscan, k_mscatter   pairs grouped by expert, 64-pair tiles
//   k_mgemm<GU>  gate and up for a tile (128 rows of I, up to 64 pairs),
//                SwiGLU into h
//   k_mgemm<DN>  down (256 rows of H) times the routing weight, into part
//   k_mcombine   out[t] = sum over slots of part, in slot order
#include "common.h"

namespace rf4 {
namespace {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));

constexpr int kMTile = 64;      // pairs per tile (4 column tiles of 16)
constexpr int kMRows = 256;     // the row blocks divide H and I
// row tiles of 16 per wave: gate/up holds two matrices' accumulators
template <bool GU> constexpr int mrt() { return GU ? 1 : 2; }

struct MArgs {
  const uint8_t* base;
  int64_t stride;
  int64_t off[MOE_NUM_TENSORS];
  int E, H, I, k, C, T;
  const int32_t* idx;     // [C][k]
  const float* w;         // [C][k]
  uint8_t* xq;            // [T][C][H] e4m3 terms of x
  uint8_t* xs;            // [T][C][H/32] their E8M0 scales
  float* h;               // [C*k][I]
  uint8_t* hq;            // [T][C*k][I]
  uint8_t* hs;            // [T][C*k][I/32]
  float* part;            // [C*k][H]
  float* out;             // [C][H]
  uint32_t* count;        // [E]
  uint32_t* cursor;       // [E]
  uint32_t* boff;         // [E+1]
  uint32_t* meta;         // [0]: tiles
  int32_t* tiles;         // [tiles][2]: expert, first pair within the expert
  int32_t* perm;          // [C*k]: pairs grouped by expert
};

size_t mx_max_tiles(int E, int k, int C) {
  const size_t CK = (size_t)C * k;
  return CK / kMTile + (CK < (size_t)E ? CK : (size_t)E);
}

struct MxWs {
  size_t count, cursor, boff, meta, tiles, perm, xq, xs, h, hq, hs, part, total;
};

MxWs mx_ws(int E, int H, int I, int k, int C, int T) {
  MxWs W;
  size_t o = 0;
  const size_t CK = (size_t)C * k;
  W.count = o;  o = align256(o + (size_t)E * 4);
  W.cursor = o; o = align256(o + (size_t)E * 4);
  W.boff = o;   o = align256(o + (size_t)(E + 1) * 4);
  W.meta = o;   o = align256(o + 64);
  W.tiles = o;  o = align256(o + mx_max_tiles(E, k, C) * 8);
  W.perm = o;   o = align256(o + CK * 4);
  W.xq = o;     o = align256(o + (size_t)T * C * H);
  W.xs = o;     o = align256(o + (size_t)T * C * (H / 32));
  W.h = o;      o = align256(o + CK * I * 4);
  W.hq = o;     o = align256(o + (size_t)T * CK * I);
  W.hs = o;     o = align256(o + (size_t)T * CK * (I / 32));
  W.part = o;   o = align256(o + CK * H * 4);
  W.total = o;
  return W;
}

// One thread per 32-value block of one row: T terms, each the block's
// remainder rounded to e4m3 under the power of two that puts its largest
// magnitude in [128, 256) (E8M0 byte clamped to 0..254), then subtracted
// exactly (the rounded value times a power of two is within the remainder's
// own precision).  Two kinds of value are left in the remainder for a later
// term: those that would round to e4m3 subnormals (the matrix core does not
// take them), and, within each aligned group of 8 (one fixed-point group of
// the instruction), those whose exponent is more than kGroupSpan below the
// group's largest.  With the weights' e2m1 exponents spanning 3 values and 2
// significant bits, and e4m3's 4, every product of such a group then has its
// lowest bit at or above the group's quantum (13 bits below the largest
// exponent sum), so the instruction truncates nothing.
constexpr uint32_t kGroupSpan = 7;

__global__ __launch_bounds__(256) void k_mq_split(const float* src, int R, int K, int T, uint8_t* q,
                                                  uint8_t* s, uint32_t* zero, int nzero) {
  const int row = blockIdx.y, nb = K / 32;
  const int blk = blockIdx.x * 256 + threadIdx.x;
  if (zero && row == 0 && blockIdx.x == 0)
    for (int i = threadIdx.x; i < nzero; i += 256) zero[i] = 0u;
  if (blk >= nb) return;
  float r[32];
  const float4* sp = reinterpret_cast<const float4*>(src + (size_t)row * K + 32 * blk);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 v = sp[i];
    r[4 * i] = v.x; r[4 * i + 1] = v.y; r[4 * i + 2] = v.z; r[4 * i + 3] = v.w;
  }
  for (int t = 0; t < T; ++t) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(r[i]));
    int sb = 0;
    if (m > 0.0f && m <= 3.0e38f) sb = ilogbf(m) - 7 + 127;
    sb = sb < 0 ? 0 : (sb > 254 ? 254 : sb);
    const float inv = ldexpf(1.0f, 127 - sb), sc = ldexpf(1.0f, sb - 127);
    uint32_t d[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int v = __builtin_amdgcn_cvt_pk_fp8_f32(r[4 * j] * inv, r[4 * j + 1] * inv, 0, false);
      v = __builtin_amdgcn_cvt_pk_fp8_f32(r[4 * j + 2] * inv, r[4 * j + 3] * inv, v, true);
      // subnormal codes (exponent field 0) become zeros
      const uint32_t ex = (uint32_t)v & 0x78787878u;
      const uint32_t nz = ((ex + 0x7F7F7F7Fu) & 0x80808080u) >> 7;
      d[j] = (uint32_t)v & (nz * 0xFFu);
    }
    // the exponent window of each group of 8 (words 2g, 2g + 1)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint32_t emax = 0;
#pragma unroll
      for (int w = 0; w < 2; ++w)
#pragma unroll
        for (int b = 0; b < 4; ++b) emax = max(emax, (d[2 * g + w] >> (8 * b + 3)) & 15u);
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        uint32_t keep = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b)
          if (((d[2 * g + w] >> (8 * b + 3)) & 15u) + kGroupSpan >= emax) keep |= 0xFFu << (8 * b);
        d[2 * g + w] &= keep;
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int v = (int)d[j];
      r[4 * j] -= __builtin_amdgcn_cvt_f32_fp8(v, 0) * sc;
      r[4 * j + 1] -= __builtin_amdgcn_cvt_f32_fp8(v, 1) * sc;
      r[4 * j + 2] -= __builtin_amdgcn_cvt_f32_fp8(v, 2) * sc;
      r[4 * j + 3] -= __builtin_amdgcn_cvt_f32_fp8(v, 3) * sc;
    }
    uint4* qp = reinterpret_cast<uint4*>(q + ((size_t)t * R + row) * K + 32 * blk);
    qp[0] = make_uint4(d[0], d[1], d[2], d[3]);
    qp[1] = make_uint4(d[4], d[5], d[6], d[7]);
    s[((size_t)t * R + row) * nb + blk] = (uint8_t)sb;
  }
}

__global__ __launch_bounds__(256) void k_mcount(MArgs a) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= a.C * a.k) return;
  const int e = a.idx[p];
  if (e >= 0 && e < a.E) atomicAdd(&a.count[e], 1u);
}

// Exclusive scan over the workgroup (1024 threads).
__device__ int scan1024(int v, int* s_w, int* total) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(incl, d, 64);
    if (lane >= d) incl += u;
  }
  if (lane == 63) s_w[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < 16; ++w) {
    if (w < wave) base += s_w[w];
    tot += s_w[w];
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

__global__ __launch_bounds__(1024) void k_mscan(MArgs a) {
  __shared__ int s_w[16];
  const int e = threadIdx.x;
  const int c = e < a.E ? (int)a.count[e] : 0;
  const int nt = (c + kMTile - 1) / kMTile;
  int npairs = 0, ntiles = 0;
  const int off = scan1024(c, s_w, &npairs);
  const int toff = scan1024(nt, s_w, &ntiles);
  if (e < a.E) {
    a.boff[e] = (uint32_t)off;
    for (int i = 0; i < nt; ++i) {
      a.tiles[2 * (toff + i)] = e;
      a.tiles[2 * (toff + i) + 1] = i * kMTile;
    }
  }
  if (e == 0) {
    a.boff[a.E] = (uint32_t)npairs;
    a.meta[0] = (uint32_t)ntiles;
  }
}

__global__ __launch_bounds__(256) void k_mscatter(MArgs a) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= a.C * a.k) return;
  const int e = a.idx[p];
  if (e >= 0 && e < a.E) a.perm[a.boff[e] + atomicAdd(&a.cursor[e], 1u)] = p;
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }

// One tile (expert e, up to 64 pairs) against 64 RT weight rows (RT = 2 for
// gate/up, whose two matrices double the accumulators, 4 for down): wave w
// takes rows 16 RT w .. 16 RT w + 16 RT - 1 as RT row tiles of 16, for every
// 16-pair column tile of the tile and every term.  Per K step of 128: one
// 16-byte code load and one scale byte per row tile and matrix (straight from
// HBM, no conversion); per stage (K step, term) the tile's activation
// fragments once for the workgroup, through LDS.
template <bool GU>
__global__ __launch_bounds__(256, 2) void k_mgemm(MArgs a) {
  constexpr int NM = GU ? 2 : 1, RT = mrt<GU>();
  __shared__ int s_pair[kMTile], s_row[kMTile];
  __shared__ __attribute__((aligned(16))) uint8_t s_b[2][kMTile][144];   // 128 bytes + pad per pair
  __shared__ uint32_t s_bs[2][kMTile];
  const int tile = blockIdx.y;
  if (tile >= (int)a.meta[0]) return;
  const int e = a.tiles[2 * tile], first = a.tiles[2 * tile + 1];
  const int cnt = min(kMTile, (int)a.count[e] - first);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  if (tid < kMTile) {
    const int p = tid < cnt ? a.perm[a.boff[e] + first + tid] : -1;
    s_pair[tid] = p;
    s_row[tid] = p < 0 ? 0 : (GU ? p / a.k : p);
  }
  __syncthreads();
  const int K = GU ? a.H : a.I;
  const int R = GU ? a.C : a.C * a.k;
  const int KB = K / 32;
  const uint8_t* q = GU ? a.xq : a.hq;
  const uint8_t* qs = GU ? a.xs : a.hs;
  const uint8_t* rec = a.base + (size_t)e * a.stride;
  const uint8_t* cb[NM];
  const uint8_t* sbp[NM];
  if (GU) {
    cb[0] = rec + a.off[MOE_T_GATE_CODES];
    sbp[0] = rec + a.off[MOE_T_GATE_SCALES];
    cb[NM - 1] = rec + a.off[MOE_T_UP_CODES];
    sbp[NM - 1] = rec + a.off[MOE_T_UP_SCALES];
  } else {
    cb[0] = rec + a.off[MOE_T_DOWN_CODES];
    sbp[0] = rec + a.off[MOE_T_DOWN_SCALES];
  }
  const int nrow0 = (blockIdx.x * 4 + wave) * 16 * RT;
  const int nsub = (cnt + 15) / 16;

  v4f_t acc[RT][NM][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) acc[rt][m][sb] = v4f_t{0.f, 0.f, 0.f, 0.f};

  // Stages (K step, term), in order.  A stage's activation fragments for
  // the whole tile (64 pairs x 128 bytes + 4 scale bytes each) are loaded
  // once per workgroup, one stage ahead, into registers and then into a
  // double-buffered LDS tile that the four waves read.  The weights of even
  // and odd K steps sit in two register sets (A0, A1), each reloaded for the
  // step after next as soon as its own step's MFMAs are issued, so no copies
  // between them make a load wait.
  v8i_t A0[RT][NM], A1[RT][NM];
  int S0[RT][NM], S1[RT][NM];
  auto load_a = [&](int k0, v8i_t (&A)[RT][NM], int (&S)[RT][NM]) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const size_t row = (size_t)(nrow0 + 16 * rt + c16);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const uint4 c = *reinterpret_cast<const uint4*>(cb[m] + row * (K / 2) + k0 / 2 + 16 * g);
        A[rt][m] = v8i_t{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
        S[rt][m] = sbp[m][row * KB + k0 / 32 + g];
      }
    }
  };
  const int lp = tid >> 2, lc = tid & 3;            // loader: pair, 32-byte chunk
  const int lrow = s_row[lp];
  uint4 g0, g1;
  uint32_t gsc = 0u;
  auto gload = [&](int k0, int t) {
    const size_t qrow = (size_t)t * R + lrow;
    const uint8_t* qp = q + qrow * K + k0 + 32 * lc;
    g0 = *reinterpret_cast<const uint4*>(qp);
    g1 = *reinterpret_cast<const uint4*>(qp + 16);
    gsc = *reinterpret_cast<const uint32_t*>(qs + qrow * KB + k0 / 32);   // all lanes: no branch
  };
  auto sstore = [&](int buf) {
    *reinterpret_cast<uint4*>(&s_b[buf][lp][32 * lc]) = g0;
    *reinterpret_cast<uint4*>(&s_b[buf][lp][32 * lc + 16]) = g1;
    if (lc == 0) s_bs[buf][lp] = gsc;
  };
  const int T = a.T;
  int buf = 0;
  // the T stages of K step k0 with weights A / S
  auto run_step = [&](int k0, const v8i_t (&A)[RT][NM], const int (&S)[RT][NM]) {
    for (int t = 0; t < T; ++t) {
      const bool more = t + 1 < T || k0 + 128 < K;
      if (more) gload(t + 1 < T ? k0 : k0 + 128, t + 1 < T ? t + 1 : 0);
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) {
        if (sb < nsub) {
          const int pr = 16 * sb + c16;
          const uint4 b0 = *reinterpret_cast<const uint4*>(&s_b[buf][pr][16 * g]);
          const uint4 b1 = *reinterpret_cast<const uint4*>(&s_b[buf][pr][64 + 16 * g]);
          const v8i_t bv = v8i_t{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                                 (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
          const int bsc = (int)((s_bs[buf][pr] >> (8 * g)) & 0xFFu);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int m = 0; m < NM; ++m)
              acc[rt][m][sb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  A[rt][m], bv, acc[rt][m][sb], 4, 0, 0, S[rt][m], 0, bsc);
        }
      }
      if (more) sstore(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  };
  load_a(0, A0, S0);
  load_a(128, A1, S1);                               // K is a multiple of 256
  gload(0, 0);
  sstore(0);
  __syncthreads();
  for (int k0 = 0; k0 < K; k0 += 256) {
    run_step(k0, A0, S0);
    if (k0 + 256 < K) load_a(k0 + 256, A0, S0);
    run_step(k0 + 128, A1, S1);
    if (k0 + 384 < K) load_a(k0 + 384, A1, S1);
  }

#pragma unroll
  for (int sb = 0; sb < 4; ++sb) {
    const int p = sb < nsub ? s_pair[16 * sb + c16] : -1;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if (p < 0) break;
      const int n = nrow0 + 16 * rt + 4 * g;
      if (GU) {
        const v4f_t gv = acc[rt][0][sb], uv = acc[rt][NM - 1][sb];
        *reinterpret_cast<float4*>(a.h + (size_t)p * a.I + n) =
            make_float4(silu_f(gv[0]) * uv[0], silu_f(gv[1]) * uv[1], silu_f(gv[2]) * uv[2],
                        silu_f(gv[3]) * uv[3]);
      } else {
        const float wp = a.w[p];
        const v4f_t dv = acc[rt][0][sb];
        *reinterpret_cast<float4*>(a.part + (size_t)p * a.H + n) =
            make_float4(wp * dv[0], wp * dv[1], wp * dv[2], wp * dv[3]);
      }
    }
  }
}

__global__ __launch_bounds__(256) void k_mcombine(MArgs a) {
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

constexpr int kMaxTerms = 6;

bool mx_ok(const moe_bank* b, int C, int k, int T) {
  if (!b || !b->base || b->format != MOE_FMT_MXFP4) return false;
  const int E = b->num_experts, H = b->hidden, I = b->inter;
  if (E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > MOE_MAX_TOPK || k > E) return false;
  if (C < 1 || C > MOE_MAX_TOKENS || T < 1 || T > kMaxTerms) return false;
  if (H < kMRows || I < kMRows || H % kMRows || I % kMRows) return false;
  if ((uintptr_t)b->base % 16 || b->expert_stride % 16) return false;
  for (int t = MOE_T_GATE_CODES; t <= MOE_T_DOWN_CODES; ++t)
    if (b->offset[t] % 16) return false;
  return true;
}

}  // namespace
}  // namespace rf4

using namespace rf4;

extern "C" {

size_t moe_mx_mma_workspace_size(const moe_bank* bank, int32_t top_k, int32_t C, int32_t terms) {
  if (!mx_ok(bank, C, top_k, terms)) return 0;
  return mx_ws(bank->num_experts, bank->hidden, bank->inter, top_k, C, terms).total;
}

moe_status moe_expert_fwd_mx_mma(const moe_bank* bank, const float* x, int32_t C, int32_t k,
                                 const int32_t* topk_idx, const float* topk_w, float* out,
                                 int32_t terms, void* ws, size_t ws_bytes, void* stream) {
  if (!bank || !x || !topk_idx || !topk_w || !out || x == out) return MOE_ERR_INVALID_ARG;
  if ((uintptr_t)x % 16 || (uintptr_t)out % 16) return MOE_ERR_INVALID_ARG;
  if (!mx_ok(bank, C, k, terms)) return MOE_ERR_UNSUPPORTED;
  const int E = bank->num_experts, H = bank->hidden, I = bank->inter;
  const MxWs W = mx_ws(E, H, I, k, C, terms);
  if (!ws || ws_bytes < W.total || (uintptr_t)ws % 256) return MOE_ERR_WORKSPACE;
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  MArgs a;
  a.base = static_cast<const uint8_t*>(bank->base);
  a.stride = bank->expert_stride;
  for (int t = 0; t < MOE_NUM_TENSORS; ++t) a.off[t] = bank->offset[t];
  a.E = E; a.H = H; a.I = I; a.k = k; a.C = C; a.T = terms;
  a.idx = topk_idx; a.w = topk_w;
  a.xq = w8 + W.xq; a.xs = w8 + W.xs;
  a.h = reinterpret_cast<float*>(w8 + W.h);
  a.hq = w8 + W.hq; a.hs = w8 + W.hs;
  a.part = reinterpret_cast<float*>(w8 + W.part);
  a.out = out;
  a.count = reinterpret_cast<uint32_t*>(w8 + W.count);
  a.cursor = reinterpret_cast<uint32_t*>(w8 + W.cursor);
  a.boff = reinterpret_cast<uint32_t*>(w8 + W.boff);
  a.meta = reinterpret_cast<uint32_t*>(w8 + W.meta);
  a.tiles = reinterpret_cast<int32_t*>(w8 + W.tiles);
  a.perm = reinterpret_cast<int32_t*>(w8 + W.perm);
  const int CK = C * k;
  const unsigned maxt = (unsigned)mx_max_tiles(E, k, C);
  // count and cursor are adjacent: one clear of 2 * 256-aligned E words
  const int nzero = (int)((W.boff - W.count) / 4);
  hipLaunchKernelGGL(k_mq_split, dim3((H / 32 + 255) / 256, C), dim3(256), 0, st, x, C, H, terms,
                     a.xq, a.xs, a.count, nzero);
  hipLaunchKernelGGL(k_mcount, dim3((CK + 255) / 256), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_mscan, dim3(1), dim3(1024), 0, st, a);
  hipLaunchKernelGGL(k_mscatter, dim3((CK + 255) / 256), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_mgemm<true>, dim3(I / (64 * mrt<true>()), maxt), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_mq_split, dim3((I / 32 + 255) / 256, CK), dim3(256), 0, st, a.h, CK, I,
                     terms, a.hq, a.hs, nullptr, 0);
  hipLaunchKernelGGL(k_mgemm<false>, dim3(H / (64 * mrt<false>()), maxt), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_mcombine, dim3((H / 4 + 255) / 256, C), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

}  // extern "C"
