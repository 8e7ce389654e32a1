// libroutedfp4 -- the routed-expert FFN at decode time on MI355X (gfx950).
//
// One MoE layer (the MUL_MAT_ID of page "Kimi-K3 on 2x A40 -- measured
// findings", section "Why the placement experiments all looked the same"; the
// router -> top-k -> selected experts -> sum structure of page "SparkInfer-K3",
// section "How the TP module works") runs as three kernels on one stream:
//
//   k_route    router mat-vec streamed across all CUs (split-K partial sums);
//              the last workgroup to finish (atomic ticket) adds the partials
//              in a fixed order, runs a wave64 radix-select top-k per token,
//              the renormalised sigmoid weights, and builds the expert dispatch
//              table (each distinct expert once, with the tokens that chose it).
//   k_gate_up  per (distinct expert, 16-row block of I): gate and up rows
//              streamed with 16-byte lane loads, e2m1 codes converted in
//              registers (v_cvt_scalef32_pk_f32_fp4), block scales applied per
//              block, x staged in LDS, SwiGLU in the epilogue.
//   k_down     per (distinct expert, 64-row block of H): down rows against the
//              intermediate activations; the routing weight is applied and
//              the per-slot result written; the last expert to finish a row
//              block (atomic ticket) sums the slots in slot order, which keeps
//              the combine deterministic (fixed-order add, page "Kimi-K3 on the
//              same pod, two engines", section "Reason 1").
//
// The whole path stays on the device: no host read-back of the routing.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include "routed_fp4.h"

namespace {

constexpr int kWG = 256;           // threads per workgroup (4 waves of 64)
constexpr int kKsplitMax = 4;      // router split-K factor limit
constexpr int kGuRows = 16;        // gate/up: I rows per item (one per lane group)
constexpr int kDnRowsPerGroup = 4; // down: rows per 16-lane group
constexpr int kDnRows = 16 * kDnRowsPerGroup;  // down: H rows per item
constexpr int kXsFloats = 10240;   // LDS floats for staged activations (40 KiB)
constexpr int kRouteXs = 8192;     // LDS floats for the router's x tile (32 KiB)

// ---------------------------------------------------------------------------
// Workspace layout
// ---------------------------------------------------------------------------
struct WsLayout {
  size_t ctrl, dtick, lpart, logits, idx, w, disp, h, part, total;
};

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

WsLayout ws_layout(int E, int H, int I, int k, int C) {
  WsLayout L;
  size_t o = 0;
  const size_t CK = (size_t)C * k;
  L.ctrl = o;   o = align256(o + 64 * sizeof(uint32_t));
  L.dtick = o;  o = align256(o + (size_t)((H + kDnRows - 1) / kDnRows) * sizeof(uint32_t));
  L.lpart = o;  o = align256(o + (size_t)kKsplitMax * C * E * sizeof(float));
  L.logits = o; o = align256(o + (size_t)C * E * sizeof(float));
  L.idx = o;    o = align256(o + CK * sizeof(int32_t));
  L.w = o;      o = align256(o + CK * sizeof(float));
  L.disp = o;   o = align256(o + (16 + 2 * CK + CK * C) * sizeof(int32_t));
  L.h = o;      o = align256(o + CK * I * sizeof(float));
  L.part = o;   o = align256(o + CK * H * sizeof(float));
  L.total = o;
  return L;
}

// Dispatch table (int32): [0] number of distinct experts U; then
// uexp[CK] (expert id of distinct expert u), untok[CK] (tokens that chose it),
// upair[CK][C] (their (token, slot) pairs p = t*k + s, in token order).
__host__ __device__ inline int disp_uexp(int) { return 16; }
__host__ __device__ inline int disp_untok(int CK) { return 16 + CK; }
__host__ __device__ inline int disp_upair(int CK) { return 16 + 2 * CK; }

// ---------------------------------------------------------------------------
// Small device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  // 2^(b-127); b = 0 is the fp32 subnormal 2^-127; 0xFF is NaN.
  const uint32_t u = (b == 0u) ? 0x00400000u : ((b == 255u) ? 0x7FC00000u : (b << 23));
  return __uint_as_float(u);
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  // OCP fp8 e4m3 ("FN"): bias 7, no infinities, S.1111.111 is NaN.
  const uint32_t s = (b & 0x80u) << 24, E = (b >> 3) & 15u, m = b & 7u;
  if (E == 15u && m == 7u) return __uint_as_float(0x7FC00000u);
  if (E == 0u) {
    const float v = (float)m * 0x1p-9f;          // (m/8) * 2^-6, exact
    return __uint_as_float(__float_as_uint(v) | s);
  }
  return __uint_as_float(s | ((E + 120u) << 23) | (m << 20));
}

// Two e2m1 elements of byte `sel` of `w`: element 2j (bits 3..0) in .x and
// element 2j+1 (bits 7..4) in .y, unscaled (the scale operand is 1.0).
template <int SEL>
__device__ __forceinline__ float2 fp4x2(uint32_t w) {
  auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
  return make_float2(v[0], v[1]);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ float group16_sum(float v) {
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) v += __shfl_xor(v, m, 16);
  return v;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// Orderable key of an fp32 logit: larger logit -> larger key; -0 == +0;
// NaN -> 0 (below every number).
__device__ __forceinline__ uint32_t logit_key(float l) {
  if (l != l) return 0u;
  uint32_t u = __float_as_uint(l);
  if ((u & 0x7FFFFFFFu) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the 64 lanes of a wave (lane order).
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

// ---------------------------------------------------------------------------
// Router
// ---------------------------------------------------------------------------
struct RouteArgs {
  const float* x;          // [C][H], or null (logits-in mode)
  const float* Wr;         // [E][H]
  const float* logits_in;  // [C][E] (logits-in mode)
  float* logits_out;       // [C][E] or null
  float* lpart;            // [ksplit][C][E]
  int32_t* idx_out;        // [C][k]
  float* w_out;            // [C][k]
  uint32_t* ctrl;          // ctrl[0]: router ticket
  int32_t* disp;           // dispatch table or null
  int C, H, E, k, ksplit, kper;
};

struct TopkShared {
  uint32_t hist[4][256];
  uint32_t sel_key[4][32];
  int32_t sel_e[4][32];
  float sel_l[4][32];
  float sorted_l[4][32];
  int32_t sidx[MOE_MAX_DECODE_TOKENS * MOE_MAX_TOPK];
  int32_t first[MOE_MAX_EXPERTS];
  int32_t uexp[MOE_MAX_DECODE_TOKENS * MOE_MAX_TOPK];
  int32_t wtot[4];
};

// Top-k of one token by one wave (all four waves call this together, with
// `active` false for waves without a token; barriers are workgroup-wide).
// Selection is exact on the fp32 logits: a 4-pass, 8-bit radix select finds
// the k-th largest key; keys above it are taken, equal keys by lowest index;
// the k winners are ranked by (key desc, index asc).
__device__ void topk_token(const RouteArgs& a, TopkShared& S, int t, bool active) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int E = a.E, k = a.k;
  uint32_t key[16];
  float lv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = lane + 64 * i;
    float l = 0.0f;
    if (active && e < E) {
      if (a.x) {
        l = a.lpart[(size_t)t * E + e];
        for (int s = 1; s < a.ksplit; ++s) l += a.lpart[((size_t)s * a.C + t) * E + e];
        if (a.logits_out) a.logits_out[(size_t)t * E + e] = l;
      } else {
        l = a.logits_in[(size_t)t * E + e];
      }
    }
    lv[i] = l;
    key[i] = logit_key(l);
  }
  uint32_t prefix = 0, pmask = 0;
  int r = k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
#pragma unroll
    for (int j = 0; j < 4; ++j) S.hist[wave][lane * 4 + j] = 0;
    __syncthreads();
    if (active) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int e = lane + 64 * i;
        if (e < E && (key[i] & pmask) == prefix)
          atomicAdd(&S.hist[wave][(key[i] >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    const int h0 = S.hist[wave][lane * 4 + 0], h1 = S.hist[wave][lane * 4 + 1];
    const int h2 = S.hist[wave][lane * 4 + 2], h3 = S.hist[wave][lane * 4 + 3];
    const int s = h0 + h1 + h2 + h3;
    // count in lanes above this one: total - inclusive scan
    const int incl = wave_incl_scan(s);
    const int total = __shfl(incl, 63, 64);
    const int above3 = total - incl;
    const int above2 = above3 + h3, above1 = above2 + h2, above0 = above1 + h1;
    int bin = -1, nr = 0;
    if (above3 < r && r <= above3 + h3) { bin = lane * 4 + 3; nr = r - above3; }
    else if (above2 < r && r <= above2 + h2) { bin = lane * 4 + 2; nr = r - above2; }
    else if (above1 < r && r <= above1 + h1) { bin = lane * 4 + 1; nr = r - above1; }
    else if (above0 < r && r <= above0 + h0) { bin = lane * 4 + 0; nr = r - above0; }
    const unsigned long long m = __ballot(bin >= 0);
    const int src = m ? (__ffsll((long long)m) - 1) : 0;
    bin = __shfl(bin, src, 64);
    nr = __shfl(nr, src, 64);
    prefix |= (uint32_t)(bin < 0 ? 0 : bin) << shift;
    pmask |= 0xFFu << shift;
    r = nr;
  }
  const uint32_t T = prefix;   // the k-th largest key
  // keys strictly above T
  int cg = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) cg += (active && lane + 64 * i < E && key[i] > T) ? 1 : 0;
  const int ginc = wave_incl_scan(cg);
  const int m_gt = __shfl(ginc, 63, 64);
  int pos = ginc - cg;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = lane + 64 * i;
    if (active && e < E && key[i] > T) {
      S.sel_key[wave][pos] = key[i]; S.sel_e[wave][pos] = e; S.sel_l[wave][pos] = lv[i];
      ++pos;
    }
  }
  // keys equal to T, lowest index first (index order is i-major, then lane)
  int taken = 0;
  const int need = k - m_gt;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = lane + 64 * i;
    const bool eq = active && e < E && key[i] == T;
    const unsigned long long mm = __ballot(eq);
    const int below = __popcll(mm & ((1ull << lane) - 1ull));
    if (eq && taken + below < need) {
      const int p = m_gt + taken + below;
      S.sel_key[wave][p] = key[i]; S.sel_e[wave][p] = e; S.sel_l[wave][p] = lv[i];
    }
    taken += __popcll(mm);
  }
  __syncthreads();
  // rank the k winners: (key desc, index asc)
  if (active && lane < k) {
    const uint32_t mk = S.sel_key[wave][lane];
    const int me = S.sel_e[wave][lane];
    int rank = 0;
    for (int j = 0; j < k; ++j) {
      const uint32_t kj = S.sel_key[wave][j];
      const int ej = S.sel_e[wave][j];
      rank += (kj > mk || (kj == mk && ej < me)) ? 1 : 0;
    }
    a.idx_out[(size_t)t * k + rank] = me;
    S.sidx[t * k + rank] = me;
    S.sorted_l[wave][rank] = S.sel_l[wave][lane];
  }
  __syncthreads();
  if (active) {
    const float sg = (lane < k) ? 1.0f / (1.0f + expf(-S.sorted_l[wave][lane])) : 0.0f;
    const float tot = wave_sum(sg);
    if (lane < k) a.w_out[(size_t)t * k + lane] = sg / tot;
  }
}

// Exclusive scan of one int per thread over the workgroup.
__device__ int block_excl_scan(int v, int32_t* wtot, int* total) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int incl = wave_incl_scan(v);
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < 4; ++w) {
    if (w < wave) base += wtot[w];
    tot += wtot[w];
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

// Expert dispatch table from the selection held in S.sidx ([C][k]).
__device__ void build_dispatch(TopkShared& S, int32_t* disp, int C, int k, int E) {
  const int tid = threadIdx.x;
  const int P = C * k, CK = C * k;
  for (int e = tid; e < E; e += kWG) S.first[e] = 0x7FFFFFFF;
  __syncthreads();
  for (int p = tid; p < P; p += kWG) {
    const int e = S.sidx[p];
    if (e >= 0 && e < E) atomicMin(&S.first[e], p);
  }
  __syncthreads();
  // P <= 512: two pairs per thread
  const int p0 = 2 * tid, p1 = 2 * tid + 1;
  const int e0 = p0 < P ? S.sidx[p0] : -1, e1 = p1 < P ? S.sidx[p1] : -1;
  const int f0 = (e0 >= 0 && e0 < E && S.first[e0] == p0) ? 1 : 0;
  const int f1 = (e1 >= 0 && e1 < E && S.first[e1] == p1) ? 1 : 0;
  int nu = 0;
  const int base = block_excl_scan(f0 + f1, S.wtot, &nu);
  if (f0) { disp[disp_uexp(CK) + base] = e0; S.uexp[base] = e0; }
  if (f1) { disp[disp_uexp(CK) + base + f0] = e1; S.uexp[base + f0] = e1; }
  if (tid == 0) disp[0] = nu;
  __syncthreads();
  // thread u lists the pairs of distinct expert u in pair (= token) order
  for (int u = tid; u < nu; u += kWG) {
    const int e = S.uexp[u];
    int n = 0;
    for (int p = 0; p < P; ++p)
      if (S.sidx[p] == e) disp[disp_upair(CK) + u * C + (n++)] = p;
    disp[disp_untok(CK) + u] = n;
  }
}

template <int CM>
__global__ __launch_bounds__(kWG) void k_route(RouteArgs a) {
  __shared__ float xs[kRouteXs];
  __shared__ TopkShared S;
  __shared__ int s_last;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  if (a.x) {
    constexpr int KT = kRouteXs / CM;          // x tile per token (floats)
    const int b = blockIdx.x;
    const int rbk = b / a.ksplit, ks = b - rbk * a.ksplit;
    const int e = rbk * 4 + wave;
    const int k0 = ks * a.kper;
    const int k1 = min(a.H, k0 + a.kper);
    float acc[CM];
#pragma unroll
    for (int t = 0; t < CM; ++t) acc[t] = 0.0f;
    for (int kt = k0; kt < k1; kt += KT) {
      const int kn = min(KT, k1 - kt);
      __syncthreads();
      for (int i = tid * 4; i < a.C * kn; i += kWG * 4) {
        const int t = i / kn, col = i - t * kn;
        *reinterpret_cast<float4*>(&xs[t * KT + col]) =
            *reinterpret_cast<const float4*>(&a.x[(size_t)t * a.H + kt + col]);
      }
      __syncthreads();
      if (e < a.E) {
        const float4* wrow = reinterpret_cast<const float4*>(a.Wr + (size_t)e * a.H + kt);
        const float4* x4 = reinterpret_cast<const float4*>(xs);
        const int n4 = kn >> 2;
        for (int c = lane; c < n4; c += 64 * 4) {
          float4 wv[4];
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (c + 64 * u < n4) wv[u] = wrow[c + 64 * u];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if (c + 64 * u < n4) {
#pragma unroll
              for (int t = 0; t < CM; ++t) {
                if (t < a.C) {
                  const float4 xv = x4[(t * KT >> 2) + c + 64 * u];
                  acc[t] += wv[u].x * xv.x + wv[u].y * xv.y + wv[u].z * xv.z + wv[u].w * xv.w;
                }
              }
            }
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < CM; ++t) {
      if (t < a.C) {
        const float v = wave_sum(acc[t]);
        if (lane == 0 && e < a.E) a.lpart[((size_t)ks * a.C + t) * a.E + e] = v;
      }
    }
    // the last workgroup to finish runs the selection
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = (atomicAdd(&a.ctrl[0], 1u) == gridDim.x - 1) ? 1 : 0;
    __syncthreads();
    if (!s_last) return;
    __threadfence();
  }
  for (int t0 = 0; t0 < a.C; t0 += 4) topk_token(a, S, t0 + wave, t0 + wave < a.C);
  __syncthreads();
  if (a.disp) build_dispatch(S, a.disp, a.C, a.k, a.E);
  if (a.x && tid == 0) atomicExch(&a.ctrl[0], 0u);
}

// Dispatch table from a caller-given selection (moe_expert_fwd).
__global__ __launch_bounds__(kWG) void k_dispatch(const int32_t* idx, int32_t* disp, int C,
                                                  int k, int E) {
  __shared__ TopkShared S;
  for (int p = threadIdx.x; p < C * k; p += kWG) S.sidx[p] = idx[p];
  __syncthreads();
  build_dispatch(S, disp, C, k, E);
}

// ---------------------------------------------------------------------------
// Expert GEMVs
// ---------------------------------------------------------------------------
struct ExpArgs {
  const uint8_t* base;
  int64_t stride;
  int64_t off[MOE_NUM_TENSORS];
  int E, H, I, k, C;
  const float* x;        // [C][H]
  const int32_t* disp;   // dispatch table
  const int32_t* idx;    // [C][k]
  const float* w;        // [C][k]
  float* h;              // [C*k][I]
  float* part;           // [C*k][H]
  float* out;            // [C][H]
  uint32_t* dtick;       // per down row block
};

// Scale bytes of one 32-element chunk: MX one e8m0 byte, NV two e4m3 bytes.
template <int FMT>
__device__ __forceinline__ uint32_t load_scales(const uint8_t* srow, int c) {
  if (FMT == MOE_FMT_MXFP4) return srow[c];
  return *reinterpret_cast<const uint16_t*>(srow + 2 * c);
}

// Staged activations: token i, element col at  i*stride + col + (col/32)*4
// (4 floats of padding per 32 keeps the 16 lanes of a group on distinct banks).
template <int NT>
struct Stage {
  static constexpr int KT = (NT == 1) ? 8192 : (NT == 2) ? 4096 : (NT == 4) ? 2048 : 1024;
  static constexpr int STRIDE = KT + KT / 8;
  static_assert(NT * STRIDE <= kXsFloats, "LDS stage too large");
};

// rows of x (or h) for tokens pairs[0..nt) -> LDS, columns [kt, kt+kn)
template <int NT>
__device__ void stage_rows(float* xs, const float* src, size_t src_stride, const int* rows,
                           int nt, int kt, int kn) {
  for (int i = threadIdx.x * 4; i < nt * kn; i += kWG * 4) {
    const int t = i / kn, col = i - t * kn;
    const float4 v = *reinterpret_cast<const float4*>(src + (size_t)rows[t] * src_stride + kt + col);
    *reinterpret_cast<float4*>(&xs[t * Stage<NT>::STRIDE + col + (col >> 5) * 4]) = v;
  }
}

// acc[r][i] += sum over one 32-element chunk of w_r * x_i for NR rows and NT
// tokens.  q: the chunk's 16 code bytes per row; sc: its scale bytes.
template <int FMT, int NR, int NT>
__device__ __forceinline__ void chunk_fma(const uint4 (&q)[NR], const uint32_t (&sc)[NR],
                                          const float* xs, int xoff, int nt,
                                          float (&acc)[NR][NT]) {
  const float4* x4 = reinterpret_cast<const float4*>(xs + xoff);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    float blk[NR][NT];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int i = 0; i < NT; ++i) blk[r][i] = 0.0f;
#pragma unroll
    for (int dd = 0; dd < 2; ++dd) {
      const int d = half * 2 + dd;             // dword of the chunk: elements 8d..8d+7
      float2 v[NR][4];
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const uint32_t wd = (d == 0) ? q[r].x : (d == 1) ? q[r].y : (d == 2) ? q[r].z : q[r].w;
        v[r][0] = fp4x2<0>(wd);
        v[r][1] = fp4x2<1>(wd);
        v[r][2] = fp4x2<2>(wd);
        v[r][3] = fp4x2<3>(wd);
      }
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        if (i < nt) {
          const float4 xa = x4[(i * Stage<NT>::STRIDE >> 2) + 2 * d];
          const float4 xb = x4[(i * Stage<NT>::STRIDE >> 2) + 2 * d + 1];
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            float b = blk[r][i];
            b += v[r][0].x * xa.x; b += v[r][0].y * xa.y;
            b += v[r][1].x * xa.z; b += v[r][1].y * xa.w;
            b += v[r][2].x * xb.x; b += v[r][2].y * xb.y;
            b += v[r][3].x * xb.z; b += v[r][3].y * xb.w;
            blk[r][i] = b;
          }
        }
      }
    }
    // one scale per 16 elements: NV has its own byte per half, MX shares one
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const float s = (FMT == MOE_FMT_NVFP4) ? e4m3_to_f32((sc[r] >> (8 * half)) & 0xFFu)
                                             : e8m0_to_f32(sc[r]);
#pragma unroll
      for (int i = 0; i < NT; ++i) acc[r][i] += s * blk[r][i];
    }
  }
}

// Rows of one expert matrix against NT staged tokens.  Each 16-lane group owns
// NR rows; lane l16 reads chunk c = l16 + 16*j (16 code bytes + its scales) of
// each row, so one wave-wide load covers 4 rows x 256 contiguous bytes.
template <int FMT, int NR, int NT>
__device__ __forceinline__ void rows_dot(const uint8_t* const (&crow)[NR],
                                         const uint8_t* const (&srow)[NR], int c0, int nc,
                                         const float* xs, int nt, float (&acc)[NR][NT]) {
  const int l16 = threadIdx.x & 15;
  constexpr int BATCH = (NR >= 4) ? 2 : 4;
  for (int cb = 0; cb < nc; cb += 16 * BATCH) {
    uint4 q[BATCH][NR];
    uint32_t sc[BATCH][NR];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int c = cb + l16 + 16 * b;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        if (c < nc) {
          q[b][r] = *reinterpret_cast<const uint4*>(crow[r] + (size_t)(c0 + c) * 16);
          sc[b][r] = load_scales<FMT>(srow[r], c0 + c);
        } else {
          q[b][r] = make_uint4(0, 0, 0, 0);
          sc[b][r] = 0;
        }
      }
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int c = cb + l16 + 16 * b;
      if (c < nc) chunk_fma<FMT, NR, NT>(q[b], sc[b], xs, c * 36, nt, acc);
    }
  }
}

template <int FMT, int NT>
__device__ void gate_up_item(const ExpArgs& a, float* xs, int e, int rb, const int* pairs,
                             int nt, int* staged_sig) {
  using St = Stage<NT>;
  const int lg = threadIdx.x >> 4, l16 = threadIdx.x & 15;
  const int H = a.H, I = a.I, CK = a.C * a.k;
  const int B = (FMT == MOE_FMT_MXFP4) ? 32 : 16;
  const int j = rb * kGuRows + lg;
  const uint8_t* rec = a.base + (size_t)e * a.stride;
  const uint8_t* crow[2] = {rec + a.off[MOE_T_GATE_CODES] + (size_t)j * (H / 2),
                            rec + a.off[MOE_T_UP_CODES] + (size_t)j * (H / 2)};
  const uint8_t* srow[2] = {rec + a.off[MOE_T_GATE_SCALES] + (size_t)j * (H / B),
                            rec + a.off[MOE_T_UP_SCALES] + (size_t)j * (H / B)};
  __shared__ int s_rows[8];
  // token rows of x for this group
  int sig = NT;
  for (int i = 0; i < nt; ++i) sig = sig * 31 + (pairs[i] / a.k) + 1;
  float acc[2][NT];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int i = 0; i < NT; ++i) acc[r][i] = 0.0f;
  for (int kt = 0; kt < H; kt += St::KT) {
    const int kn = min(St::KT, H - kt);
    const int tsig = sig * 7 + kt;
    if (!(tsig == *staged_sig && kn == H)) {
      __syncthreads();
      if (threadIdx.x < nt) s_rows[threadIdx.x] = pairs[threadIdx.x] / a.k;
      __syncthreads();
      stage_rows<NT>(xs, a.x, (size_t)H, s_rows, nt, kt, kn);
      __syncthreads();
      *staged_sig = (kn == H) ? tsig : -1;
    }
    rows_dot<FMT, 2, NT>(crow, srow, kt / 32, kn / 32, xs, nt, acc);
  }
  float gg = 1.0f, gu = 1.0f;
  if (FMT == MOE_FMT_NVFP4) {
    const float* g = reinterpret_cast<const float*>(rec + a.off[MOE_T_GLOBALS]);
    gg = g[0];
    gu = g[1];
  }
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const float sg = group16_sum(acc[0][i]);
    const float su = group16_sum(acc[1][i]);
    if (l16 == 0 && i < nt && j < I) a.h[(size_t)pairs[i] * I + j] = silu(gg * sg) * (gu * su);
  }
  (void)CK;
}

// NTMAX: the most tokens any distinct expert can have (min(C, 8) rounded up to
// a power of two); it bounds the register footprint of the compiled paths.
template <int FMT, int NTMAX>
__global__ __launch_bounds__(kWG) void k_gate_up(ExpArgs a) {
  __shared__ float xs[kXsFloats];
  const int CK = a.C * a.k;
  const int nu = a.disp[0];
  const int nrb = a.I / kGuRows;
  const int items = nu * nrb;
  int sig = -1;   // identifies what xs holds (same value in every thread)
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int u = item / nrb, rb = item - u * nrb;
    const int e = a.disp[disp_uexp(CK) + u];
    const int ntok = a.disp[disp_untok(CK) + u];
    const int* pairs = a.disp + disp_upair(CK) + u * a.C;
    for (int g0 = 0; g0 < ntok; g0 += NTMAX) {
      const int nt = min(NTMAX, ntok - g0);
      if (NTMAX == 1 || nt == 1) gate_up_item<FMT, 1>(a, xs, e, rb, pairs + g0, nt, &sig);
      else if (NTMAX == 2 || nt == 2) gate_up_item<FMT, (NTMAX >= 2 ? 2 : 1)>(a, xs, e, rb, pairs + g0, nt, &sig);
      else if (NTMAX == 4 || nt <= 4) gate_up_item<FMT, (NTMAX >= 4 ? 4 : 1)>(a, xs, e, rb, pairs + g0, nt, &sig);
      else gate_up_item<FMT, (NTMAX >= 8 ? 8 : 1)>(a, xs, e, rb, pairs + g0, nt, &sig);
    }
  }
}

template <int FMT, int NT>
__device__ void down_item(const ExpArgs& a, float* xs, int e, int rb, const int* pairs, int nt) {
  using St = Stage<NT>;
  constexpr int NR = kDnRowsPerGroup;
  const int lg = threadIdx.x >> 4, l16 = threadIdx.x & 15;
  const int H = a.H, I = a.I;
  const int B = (FMT == MOE_FMT_MXFP4) ? 32 : 16;
  const uint8_t* rec = a.base + (size_t)e * a.stride;
  int jr[NR];
  const uint8_t* crow[NR];
  const uint8_t* srow[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    jr[r] = rb * kDnRows + lg * NR + r;
    const int jj = min(jr[r], H - 1);    // rows past H read row H-1, never stored
    crow[r] = rec + a.off[MOE_T_DOWN_CODES] + (size_t)jj * (I / 2);
    srow[r] = rec + a.off[MOE_T_DOWN_SCALES] + (size_t)jj * (I / B);
  }
  __shared__ int s_rows[8];
  float acc[NR][NT];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int i = 0; i < NT; ++i) acc[r][i] = 0.0f;
  for (int kt = 0; kt < I; kt += St::KT) {
    const int kn = min(St::KT, I - kt);
    __syncthreads();
    if (threadIdx.x < nt) s_rows[threadIdx.x] = pairs[threadIdx.x];
    __syncthreads();
    stage_rows<NT>(xs, a.h, (size_t)I, s_rows, nt, kt, kn);
    __syncthreads();
    rows_dot<FMT, NR, NT>(crow, srow, kt / 32, kn / 32, xs, nt, acc);
  }
  float gd = 1.0f;
  if (FMT == MOE_FMT_NVFP4) gd = reinterpret_cast<const float*>(rec + a.off[MOE_T_GLOBALS])[2];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const float y = group16_sum(acc[r][i]);
      if (l16 == 0 && i < nt && jr[r] < H) {
        const int p = pairs[i];
        a.part[(size_t)p * H + jr[r]] = a.w[p] * (gd * y);
      }
    }
  }
}

template <int FMT, int NTMAX>
__global__ __launch_bounds__(kWG) void k_down(ExpArgs a) {
  __shared__ float xs[kXsFloats];
  __shared__ int s_last;
  const int CK = a.C * a.k;
  const int nu = a.disp[0];
  const int nrb = (a.H + kDnRows - 1) / kDnRows;
  const int items = nu * nrb;
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int u = item / nrb, rb = item - u * nrb;
    const int e = a.disp[disp_uexp(CK) + u];
    const int ntok = a.disp[disp_untok(CK) + u];
    const int* pairs = a.disp + disp_upair(CK) + u * a.C;
    for (int g0 = 0; g0 < ntok; g0 += NTMAX) {
      const int nt = min(NTMAX, ntok - g0);
      if (NTMAX == 1 || nt == 1) down_item<FMT, 1>(a, xs, e, rb, pairs + g0, nt);
      else if (NTMAX == 2 || nt == 2) down_item<FMT, (NTMAX >= 2 ? 2 : 1)>(a, xs, e, rb, pairs + g0, nt);
      else down_item<FMT, (NTMAX >= 4 ? 4 : 1)>(a, xs, e, rb, pairs + g0, nt);
    }
    // the last distinct expert to finish this row block sums the slots
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) s_last = (atomicAdd(&a.dtick[rb], 1u) == (uint32_t)(nu - 1)) ? 1 : 0;
    __syncthreads();
    if (s_last) {
      __threadfence();
      const int j0 = rb * kDnRows;
      for (int q = threadIdx.x; q < a.C * kDnRows; q += kWG) {
        const int t = q / kDnRows, j = j0 + (q - t * kDnRows);
        if (j < a.H) {
          float s = 0.0f;
          for (int sl = 0; sl < a.k; ++sl) {
            const int p = t * a.k + sl;
            const int ee = a.idx[p];
            if (ee >= 0 && ee < a.E) s += a.part[(size_t)p * a.H + j];
          }
          a.out[(size_t)t * a.H + j] = s;
        }
      }
      if (threadIdx.x == 0) atomicExch(&a.dtick[rb], 0u);
    }
  }
}

// Tokens whose every slot names an out-of-range expert get no combine from
// k_down (no distinct expert covers them); this zero-fills such rows.
__global__ void k_zero_uncovered(ExpArgs a) {
  const int t = blockIdx.x;
  bool any = false;
  for (int s = 0; s < a.k; ++s) {
    const int e = a.idx[t * a.k + s];
    any |= (e >= 0 && e < a.E);
  }
  if (any) return;
  for (int j = threadIdx.x; j < a.H; j += blockDim.x) a.out[(size_t)t * a.H + j] = 0.0f;
}

// ---------------------------------------------------------------------------
// Dequant export and workspace fill
// ---------------------------------------------------------------------------
template <int FMT>
__global__ void k_dequant(const uint8_t* codes, const uint8_t* scales, const float* gptr,
                          int N, int K, float* out) {
  const int64_t chunk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nch = (int64_t)N * (K / 32);
  if (chunk >= nch) return;
  const int64_t n = chunk / (K / 32), c = chunk - n * (K / 32);
  const uint4 q = *reinterpret_cast<const uint4*>(codes + (size_t)n * (K / 2) + c * 16);
  const uint32_t sc = load_scales<FMT>(scales + (size_t)n * (K / (FMT == MOE_FMT_MXFP4 ? 32 : 16)), (int)c);
  const float g = (FMT == MOE_FMT_NVFP4) ? *gptr : 1.0f;
  float* o = out + (size_t)n * K + c * 32;
  const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const float s = (FMT == MOE_FMT_MXFP4) ? e8m0_to_f32(sc)
                                          : e4m3_to_f32((sc >> (8 * (d >> 1))) & 0xFFu);
    float2 v[4] = {fp4x2<0>(wd[d]), fp4x2<1>(wd[d]), fp4x2<2>(wd[d]), fp4x2<3>(wd[d])};
    float r[8];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (FMT == MOE_FMT_MXFP4) {
        r[2 * b] = v[b].x * s;
        r[2 * b + 1] = v[b].y * s;
      } else {
        const float p0 = v[b].x * s, p1 = v[b].y * s;   // exact (<= 6 significant bits)
        r[2 * b] = p0 * g;                              // the one rounding
        r[2 * b + 1] = p1 * g;
      }
    }
    *reinterpret_cast<float4*>(o + 8 * d) = make_float4(r[0], r[1], r[2], r[3]);
    *reinterpret_cast<float4*>(o + 8 * d + 4) = make_float4(r[4], r[5], r[6], r[7]);
  }
}

__global__ void k_fill_zero(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
int device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t tensor_bytes(int fmt, int H, int I, int t) {
  const int B = fmt == MOE_FMT_MXFP4 ? 32 : 16;
  switch (t) {
    case MOE_T_GATE_CODES: case MOE_T_UP_CODES: return (size_t)I * H / 2;
    case MOE_T_DOWN_CODES: return (size_t)H * I / 2;
    case MOE_T_GATE_SCALES: case MOE_T_UP_SCALES: return (size_t)I * (H / B);
    case MOE_T_DOWN_SCALES: return (size_t)H * (I / B);
    default: return fmt == MOE_FMT_NVFP4 ? 12 : 0;
  }
}

moe_status check_bank(const moe_bank* b) {
  if (!b || !b->base) return MOE_ERR_INVALID_ARG;
  if (b->format != MOE_FMT_MXFP4 && b->format != MOE_FMT_NVFP4) return MOE_ERR_UNSUPPORTED;
  if (b->num_experts < 1 || b->num_experts > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
  if (b->hidden < 32 || b->inter < 32 || b->hidden % 32 || b->inter % 32) return MOE_ERR_INVALID_ARG;
  if (b->hidden > 65536 || b->inter > 65536) return MOE_ERR_UNSUPPORTED;
  if (!aligned(b->base, 16) || b->expert_stride % 16) return MOE_ERR_INVALID_ARG;
  for (int t = 0; t < MOE_NUM_TENSORS; ++t) {
    if (b->offset[t] < 0) return MOE_ERR_INVALID_ARG;
    const size_t nb = tensor_bytes(b->format, b->hidden, b->inter, t);
    if (nb && (size_t)b->offset[t] + nb > (size_t)b->expert_stride) return MOE_ERR_INVALID_ARG;
  }
  for (int t = MOE_T_GATE_CODES; t <= MOE_T_DOWN_CODES; ++t)
    if (b->offset[t] % 16) return MOE_ERR_INVALID_ARG;
  if (b->format == MOE_FMT_NVFP4) {
    if (b->offset[MOE_T_GLOBALS] % 4) return MOE_ERR_INVALID_ARG;
    for (int t = MOE_T_GATE_SCALES; t <= MOE_T_DOWN_SCALES; ++t)
      if (b->offset[t] % 2) return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

moe_status launch_status() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

// Router launch (x may be null for logits-in mode).
moe_status launch_route(const float* x, const float* Wr, const float* logits_in,
                        float* logits_out, int C, int H, int E, int k, int32_t* idx,
                        float* w, int32_t* disp, uint8_t* ws, const WsLayout& L,
                        hipStream_t st) {
  RouteArgs a;
  a.x = x;
  a.Wr = Wr;
  a.logits_in = logits_in;
  a.logits_out = logits_out;
  a.lpart = reinterpret_cast<float*>(ws + L.lpart);
  a.idx_out = idx;
  a.w_out = w;
  a.ctrl = reinterpret_cast<uint32_t*>(ws + L.ctrl);
  a.disp = disp;
  a.C = C; a.H = H; a.E = E; a.k = k;
  int grid = 1;
  if (x) {
    const int nrb = (E + 3) / 4;
    const int want = 2 * device_cu_count();
    int ks = (want + nrb - 1) / nrb;
    ks = ks < 1 ? 1 : (ks > kKsplitMax ? kKsplitMax : ks);
    int kper = (H + ks - 1) / ks;
    kper = (kper + 31) / 32 * 32;
    ks = (H + kper - 1) / kper;
    a.ksplit = ks;
    a.kper = kper;
    grid = nrb * ks;
  } else {
    a.ksplit = 1;
    a.kper = H;
  }
  if (C == 1) hipLaunchKernelGGL(k_route<1>, dim3(grid), dim3(kWG), 0, st, a);
  else if (C <= 4) hipLaunchKernelGGL(k_route<4>, dim3(grid), dim3(kWG), 0, st, a);
  else hipLaunchKernelGGL(k_route<16>, dim3(grid), dim3(kWG), 0, st, a);
  return launch_status();
}

moe_status launch_experts(const moe_bank* b, const float* x, int C, int k, const int32_t* idx,
                          const float* w, float* out, uint8_t* ws, const WsLayout& L,
                          hipStream_t st) {
  ExpArgs a;
  a.base = static_cast<const uint8_t*>(b->base);
  a.stride = b->expert_stride;
  for (int t = 0; t < MOE_NUM_TENSORS; ++t) a.off[t] = b->offset[t];
  a.E = b->num_experts; a.H = b->hidden; a.I = b->inter; a.k = k; a.C = C;
  a.x = x;
  a.disp = reinterpret_cast<const int32_t*>(ws + L.disp);
  a.idx = idx;
  a.w = w;
  a.h = reinterpret_cast<float*>(ws + L.h);
  a.part = reinterpret_cast<float*>(ws + L.part);
  a.out = out;
  a.dtick = reinterpret_cast<uint32_t*>(ws + L.dtick);
  const int ncu = device_cu_count();
  const int umax = (C * k < a.E) ? C * k : a.E;
  const int gu_items = umax * (a.I / kGuRows);
  const int dn_items = umax * ((a.H + kDnRows - 1) / kDnRows);
  const int gu_grid = gu_items < 2 * ncu ? gu_items : 2 * ncu;
  const int dn_grid = dn_items < 2 * ncu ? dn_items : 2 * ncu;
  // token-group width: gate/up up to 8 tokens per weight pass, down up to 4
#define RF4_LAUNCH(F, GU, DN)                                                          \
  do {                                                                                 \
    hipLaunchKernelGGL((k_gate_up<F, GU>), dim3(gu_grid), dim3(kWG), 0, st, a);        \
    hipLaunchKernelGGL((k_down<F, DN>), dim3(dn_grid), dim3(kWG), 0, st, a);           \
  } while (0)
  if (b->format == MOE_FMT_MXFP4) {
    if (C == 1) RF4_LAUNCH(MOE_FMT_MXFP4, 1, 1);
    else if (C == 2) RF4_LAUNCH(MOE_FMT_MXFP4, 2, 2);
    else if (C <= 4) RF4_LAUNCH(MOE_FMT_MXFP4, 4, 4);
    else RF4_LAUNCH(MOE_FMT_MXFP4, 8, 4);
  } else {
    if (C == 1) RF4_LAUNCH(MOE_FMT_NVFP4, 1, 1);
    else if (C == 2) RF4_LAUNCH(MOE_FMT_NVFP4, 2, 2);
    else if (C <= 4) RF4_LAUNCH(MOE_FMT_NVFP4, 4, 4);
    else RF4_LAUNCH(MOE_FMT_NVFP4, 8, 4);
  }
#undef RF4_LAUNCH
  hipLaunchKernelGGL(k_zero_uncovered, dim3(C), dim3(256), 0, st, a);
  return launch_status();
}

bool tokens_ok(int C) { return C >= 1 && C <= MOE_MAX_DECODE_TOKENS; }
bool topk_ok(int k, int E) { return k >= 1 && k <= MOE_MAX_TOPK && k <= E; }

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

int32_t moe_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or size";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_DEVICE: return "device launch failed";
    default: return "unknown status";
  }
}

moe_status moe_bank_layout(int32_t format, int32_t hidden, int32_t inter,
                           int64_t offset[MOE_NUM_TENSORS], int64_t* expert_stride) {
  if (!offset || !expert_stride) return MOE_ERR_INVALID_ARG;
  if (format != MOE_FMT_MXFP4 && format != MOE_FMT_NVFP4) return MOE_ERR_UNSUPPORTED;
  if (hidden < 32 || inter < 32 || hidden % 32 || inter % 32) return MOE_ERR_INVALID_ARG;
  size_t o = 0;
  for (int t = 0; t < MOE_NUM_TENSORS; ++t) {
    offset[t] = (int64_t)o;
    o = align256(o + tensor_bytes(format, hidden, inter, t));
  }
  *expert_stride = (int64_t)((o + 4095) & ~size_t(4095));
  return MOE_OK;
}

size_t moe_workspace_size(int32_t num_experts, int32_t hidden, int32_t inter, int32_t top_k,
                          int32_t C) {
  if (num_experts < 1 || num_experts > MOE_MAX_EXPERTS || hidden < 32 || inter < 32 ||
      !tokens_ok(C) || !topk_ok(top_k, num_experts))
    return 0;
  return ws_layout(num_experts, hidden, inter, top_k, C).total;
}

moe_status moe_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws || ws_bytes == 0 || !aligned(ws, 4)) return MOE_ERR_INVALID_ARG;
  const size_t n = ws_bytes / 4;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<uint32_t*>(ws), n);
  return launch_status();
}

moe_status moe_route(const float* x, const float* w_router, float* logits, int32_t C, int32_t H,
                     int32_t E, int32_t k, int32_t* topk_idx, float* topk_w, void* ws,
                     size_t ws_bytes, void* stream) {
  if (!topk_idx || !topk_w) return MOE_ERR_INVALID_ARG;
  if (E < 1 || E > MOE_MAX_EXPERTS || !tokens_ok(C) || !topk_ok(k, E)) return MOE_ERR_UNSUPPORTED;
  if (H < 32 || H % 32) return MOE_ERR_INVALID_ARG;
  if (x) {
    if (!w_router || !aligned(x, 16) || !aligned(w_router, 16)) return MOE_ERR_INVALID_ARG;
  } else if (!logits) {
    return MOE_ERR_INVALID_ARG;
  }
  if (!ws) return MOE_ERR_WORKSPACE;
  // the router needs only the counters and partial sums: size for I = 32
  const WsLayout L = ws_layout(E, H, 32, k, C);
  if (ws_bytes < L.total || !aligned(ws, 256)) return MOE_ERR_WORKSPACE;
  return launch_route(x, w_router, x ? nullptr : logits, x ? logits : nullptr, C, H, E, k,
                      topk_idx, topk_w, nullptr, static_cast<uint8_t*>(ws), L,
                      reinterpret_cast<hipStream_t>(stream));
}

moe_status moe_expert_fwd(const moe_bank* bank, const float* x, int32_t C, int32_t k,
                          const int32_t* topk_idx, const float* topk_w, float* out, void* ws,
                          size_t ws_bytes, void* stream) {
  moe_status s = check_bank(bank);
  if (s != MOE_OK) return s;
  if (!x || !topk_idx || !topk_w || !out || !aligned(x, 16)) return MOE_ERR_INVALID_ARG;
  if (x == out) return MOE_ERR_INVALID_ARG;
  if (!tokens_ok(C) || !topk_ok(k, bank->num_experts)) return MOE_ERR_UNSUPPORTED;
  if (!ws) return MOE_ERR_WORKSPACE;
  const WsLayout L = ws_layout(bank->num_experts, bank->hidden, bank->inter, k, C);
  if (ws_bytes < L.total || !aligned(ws, 256)) return MOE_ERR_WORKSPACE;
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(k_dispatch, dim3(1), dim3(kWG), 0, st, topk_idx,
                     reinterpret_cast<int32_t*>(w8 + L.disp), C, k, bank->num_experts);
  if ((s = launch_status()) != MOE_OK) return s;
  return launch_experts(bank, x, C, k, topk_idx, topk_w, out, w8, L, st);
}

moe_status moe_layer_fwd(const moe_bank* bank, const float* w_router, const float* x, int32_t C,
                         int32_t k, float* out, int32_t* topk_idx_out, float* topk_w_out,
                         void* ws, size_t ws_bytes, void* stream) {
  moe_status s = check_bank(bank);
  if (s != MOE_OK) return s;
  if (!w_router || !x || !out || !aligned(x, 16) || !aligned(w_router, 16) || x == out)
    return MOE_ERR_INVALID_ARG;
  if (!tokens_ok(C) || !topk_ok(k, bank->num_experts)) return MOE_ERR_UNSUPPORTED;
  if (!ws) return MOE_ERR_WORKSPACE;
  const WsLayout L = ws_layout(bank->num_experts, bank->hidden, bank->inter, k, C);
  if (ws_bytes < L.total || !aligned(ws, 256)) return MOE_ERR_WORKSPACE;
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  int32_t* idx = topk_idx_out ? topk_idx_out : reinterpret_cast<int32_t*>(w8 + L.idx);
  float* w = topk_w_out ? topk_w_out : reinterpret_cast<float*>(w8 + L.w);
  s = launch_route(x, w_router, nullptr, nullptr, C, bank->hidden, bank->num_experts, k, idx, w,
                   reinterpret_cast<int32_t*>(w8 + L.disp), w8, L, st);
  if (s != MOE_OK) return s;
  return launch_experts(bank, x, C, k, idx, w, out, w8, L, st);
}

moe_status moe_dequant(const moe_bank* bank, int32_t expert, int32_t matrix, float* out,
                       void* stream) {
  moe_status s = check_bank(bank);
  if (s != MOE_OK) return s;
  if (!out || expert < 0 || expert >= bank->num_experts || matrix < 0 || matrix > 2)
    return MOE_ERR_INVALID_ARG;
  const int H = bank->hidden, I = bank->inter;
  const int N = matrix == 2 ? H : I, K = matrix == 2 ? I : H;
  const uint8_t* rec = static_cast<const uint8_t*>(bank->base) + (size_t)expert * bank->expert_stride;
  const uint8_t* codes = rec + bank->offset[MOE_T_GATE_CODES + matrix];
  const uint8_t* scales = rec + bank->offset[MOE_T_GATE_SCALES + matrix];
  const float* g = reinterpret_cast<const float*>(rec + bank->offset[MOE_T_GLOBALS]) + matrix;
  const int64_t nch = (int64_t)N * (K / 32);
  const unsigned blocks = (unsigned)((nch + 255) / 256);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (bank->format == MOE_FMT_MXFP4)
    hipLaunchKernelGGL(k_dequant<MOE_FMT_MXFP4>, dim3(blocks), dim3(256), 0, st, codes, scales, g, N, K, out);
  else
    hipLaunchKernelGGL(k_dequant<MOE_FMT_NVFP4>, dim3(blocks), dim3(256), 0, st, codes, scales, g, N, K, out);
  return launch_status();
}

}  // extern "C"
