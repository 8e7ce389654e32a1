// libroutedfp4 -- the routed-expert FFN at decode time on MI355X (gfx950).
//
// One MoE layer (the MUL_MAT_ID of page "Kimi-K3 on 2x A40 -- measured
// findings", section "Why the placement experiments all looked the same"; the
// router -> top-k -> selected experts -> sum structure of page "SparkInfer-K3",
// section "How the TP module works") runs one of two ways.
//
// One token (C = 1) on a built shape: k_moe1, the whole layer in one launch
// of co-resident workgroups that hand results to one another through
// epoch-tagged words (see "Batch-1 decode" below).
//
// Otherwise (C = 2..16, or other shapes) three kernels on one stream:
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

#include <atomic>

#include "routed_fp4.h"
#include "common.h"

#ifndef RF4_PIPE_DEPTH
#define RF4_PIPE_DEPTH 2
#endif

namespace {

using namespace rf4;

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
  int select;              // 0: the split-K sums are left for k_btopk (several tokens)
};

struct TopkShared {
  uint32_t hist[4][256];
  uint32_t sel_key[4][32];
  int32_t sel_e[4][32];
  float sel_l[4][32];
  float sorted_l[4][32];
  int32_t sorted_e[32];
  int32_t sidx[MOE_MAX_DECODE_TOKENS * MOE_MAX_TOPK];
  int32_t first[MOE_MAX_EXPERTS];
  int32_t uexp[MOE_MAX_DECODE_TOKENS * MOE_MAX_TOPK];
  int32_t wtot[4];
};

// Top-k over the E values one wave holds (value e in lane e%64, slot e/64, as
// orderable keys `key` and raw logits `lv`).  All four waves call this together,
// with `active` false for waves that have no token; barriers are workgroup-wide.
// Selection is exact on the fp32 logits: a 4-pass, 8-bit radix select finds the
// k-th largest key; keys above it are taken, equal keys by lowest index; the k
// winners are ranked by (key desc, index asc).  Output, in rank order:
// S.sel_e[wave][0..k) and S.sorted_l[wave][0..k).
__device__ void wave_topk(TopkShared& S, const uint32_t (&key)[16], const float (&lv)[16],
                          int E, int k, bool active) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
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
  int my_e = 0, rank = 0;
  float my_l = 0.0f;
  if (active && lane < k) {
    const uint32_t mk = S.sel_key[wave][lane];
    my_e = S.sel_e[wave][lane];
    my_l = S.sel_l[wave][lane];
    for (int j = 0; j < k; ++j) {
      const uint32_t kj = S.sel_key[wave][j];
      const int ej = S.sel_e[wave][j];
      rank += (kj > mk || (kj == mk && ej < my_e)) ? 1 : 0;
    }
  }
  __syncthreads();
  if (active && lane < k) {
    S.sel_e[wave][rank] = my_e;
    S.sorted_l[wave][rank] = my_l;
  }
  __syncthreads();
}

// Top-k of token t by one wave of the router's last workgroup.
__device__ void topk_token(const RouteArgs& a, TopkShared& S, int t, bool active) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int E = a.E, k = a.k;
  uint32_t key[16];
  float lv[16];
  if (a.x) {
    // every split-K partial of the lane's 16 experts in flight at once (loads
    // outside the view read zeros), then added in split order
    const __amdgpu_buffer_rsrc_t lp =
        coherent_view(a.lpart, (uint32_t)((size_t)a.ksplit * a.C * E * sizeof(float)));
    float pv[kKsplitMax][16];
#pragma unroll
    for (int s = 0; s < kKsplitMax; ++s)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int e = lane + 64 * i;
        const bool in = active && e < E && s < a.ksplit;
        pv[s][i] = coherent_ld(lp, in ? (uint32_t)((((size_t)s * a.C + t) * E + e) * 4) : 0x80000000u);
      }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float l = pv[0][i];
#pragma unroll
      for (int s = 1; s < kKsplitMax; ++s)
        if (s < a.ksplit) l += pv[s][i];
      const int e = lane + 64 * i;
      if (!(active && e < E)) l = 0.0f;
      else if (a.logits_out) a.logits_out[(size_t)t * E + e] = l;
      lv[i] = l;
      key[i] = logit_key(l);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = lane + 64 * i;
      const float l = (active && e < E) ? a.logits_in[(size_t)t * E + e] : 0.0f;
      lv[i] = l;
      key[i] = logit_key(l);
    }
  }
  wave_topk(S, key, lv, E, k, active);
  if (active) {
    const float l = (lane < k) ? S.sorted_l[wave][lane] : 0.0f;
    const float w = route_weight(l, lane, k);
    if (lane < k) {
      const int e = S.sel_e[wave][lane];
      a.idx_out[(size_t)t * k + lane] = e;
      a.w_out[(size_t)t * k + lane] = w;
      S.sidx[t * k + lane] = e;
    }
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

constexpr int kRouteWt = 2048;           // router: most columns per x tile (8 float4 per lane)

template <int CM>
__global__ __launch_bounds__(kWG) void k_route(RouteArgs a) {
  __shared__ float xs[kRouteXs];
  __shared__ TopkShared S;
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: the row view below is scalar

  if (a.x) {
    // x tiles of KT columns per token (KT: a multiple of 256 that fits the
    // call's C tokens in LDS, at most kRouteWt).  A tile's x loads (all of
    // them at once: at most kRouteXs / 4 float4, kRouteXs / (4 kWG) per
    // thread) are issued first and the wave's row loads after them, so
    // storing x into LDS waits for x alone (loads complete in issue order)
    // while the rows stay in flight.
    const int KT = min(kRouteWt, (kRouteXs / a.C) & ~255);
    const int b = blockIdx.x;
    const int rbk = b / a.ksplit, ks = b - rbk * a.ksplit;
    const int e = rbk * 4 + wave;
    const int k0 = ks * a.kper;
    const int k1 = min(a.H, k0 + a.kper);
    // x of all tokens, and this wave's router row (empty past the last expert)
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.x), (short)0, a.C * a.H * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.Wr + (size_t)(e < a.E ? e : 0) * a.H), (short)0, e < a.E ? a.H * 4 : 0,
        0x00020000);
    float acc[CM];
#pragma unroll
    for (int t = 0; t < CM; ++t) acc[t] = 0.0f;
    for (int kt = k0; kt < k1; kt += KT) {
      const int kn = min(KT, k1 - kt);
      const int n4 = kn >> 2;
      constexpr int kXv = kRouteXs / 4 / kWG;  // float4 of the x tile per thread
      const int n4t = (a.C * kn) >> 2;
      // buffer loads, every one issued (those out of range read zeros
      // without memory traffic), so the compiler counts them exactly
      float4 xv[kXv];
#pragma unroll
      for (int u = 0; u < kXv; ++u) {
        const int i = 4 * (tid + kWG * u), t = i / kn, col = i - t * kn;
        const uint32_t o = tid + kWG * u < n4t ? (uint32_t)((t * a.H + kt + col) * 4) : 0x80000000u;
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(xrs, (int)o, 0, 0);
        xv[u] = make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                            __uint_as_float(v[3]));
      }
      float4 wv[kRouteWt / 256];
#pragma unroll
      for (int u = 0; u < kRouteWt / 256; ++u) {
        const int c = lane + 64 * u;
        const uint32_t o = c < n4 ? (uint32_t)((kt + 4 * c) * 4) : 0x80000000u;
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(wrs, (int)o, 0, 0);
        wv[u] = make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                            __uint_as_float(v[3]));
      }
      __syncthreads();                         // the previous tile's products are done
#pragma unroll
      for (int u = 0; u < kXv; ++u) {
        const int i = 4 * (tid + kWG * u), t = i / kn, col = i - t * kn;
        if (tid + kWG * u < n4t) *reinterpret_cast<float4*>(&xs[t * KT + col]) = xv[u];
      }
      __syncthreads();
      if (e < a.E) {
        const float4* x4 = reinterpret_cast<const float4*>(xs);
#pragma unroll
        for (int u = 0; u < kRouteWt / 256; ++u) {
          const int c = lane + 64 * u;
          if (c < n4) {
#pragma unroll
            for (int t = 0; t < CM; ++t) {
              if (t < a.C) {
                const float4 xv = x4[(t * KT >> 2) + c];
                acc[t] += wv[u].x * xv.x + wv[u].y * xv.y + wv[u].z * xv.z + wv[u].w * xv.w;
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
        if (lane == 0 && e < a.E) store_coherent(&a.lpart[((size_t)ks * a.C + t) * a.E + e], v);
      }
    }
    // the last workgroup to finish runs the selection (or a separate launch
    // selects, one wave per token)
    if (!a.select || !last_to_arrive(&a.ctrl[0], gridDim.x, &s_last)) return;
  }
  for (int t0 = 0; t0 < a.C; t0 += 4) topk_token(a, S, t0 + wave, t0 + wave < a.C);
  __syncthreads();
  if (a.disp) build_dispatch(S, a.disp, a.C, a.k, a.E);
  if (a.x && tid == 0) reset_ticket(&a.ctrl[0]);
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
        store_coherent(&a.part[(size_t)p * H + jr[r]], a.w[p] * (gd * y));
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
    if (last_to_arrive(&a.dtick[rb], (uint32_t)nu, &s_last)) {
      const int j0 = rb * kDnRows;
      for (int q = threadIdx.x; q < a.C * kDnRows; q += kWG) {
        const int t = q / kDnRows, j = j0 + (q - t * kDnRows);
        if (j < a.H) {
          const __amdgpu_buffer_rsrc_t pv =
              coherent_view(a.part, (uint32_t)((size_t)a.C * a.k * a.H * sizeof(float)));
          float s = 0.0f;
          for (int sl = 0; sl < a.k; ++sl) {
            const int p = t * a.k + sl;
            const int ee = a.idx[p];
            const float v = coherent_ld(pv, (uint32_t)(((size_t)p * a.H + j) * 4));
            if (ee >= 0 && ee < a.E) s += v;
          }
          a.out[(size_t)t * a.H + j] = s;
        }
      }
      if (threadIdx.x == 0) reset_ticket(&a.dtick[rb]);
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
// Batch-1 decode: the whole layer as one kernel of co-resident workgroups
// ---------------------------------------------------------------------------
// Hand-offs between workgroups carry the call's epoch: a producer writes
// (epoch, value) as one 64-bit agent-coherent store and moves on; a consumer
// polls until every value it needs carries the current epoch.  No producer
// ever waits for its stores and no work item takes a ticket.  Every
// workgroup writes an arrival word once it has read the epoch; one workgroup
// of the combine publishes the next epoch after seeing all of them.
enum { kCtrlRouteTicket = 0, kCtrlErr = 4, kCtrlEpoch = 5, kCtrlArrive = 64 };
constexpr int kG1 = 256;                  // workgroups of the batch-1 kernel (one per CU)
constexpr int kWG1 = 512;                 // threads per batch-1 workgroup (8 waves)
constexpr int kMaxH1 = 8192;              // batch-1 kernel limits
constexpr int kMaxI1 = 4096;
constexpr int kXcds = 8;                   // XCDs; workgroup w is dispatched to XCD w % 8
constexpr uint32_t kXcdPolls = 256;       // XCD-copy polls before the coherent copy
constexpr uint32_t kSpinLimit = 1u << 22; // ~seconds: a wait that never ends gives up

// (epoch, fp32) hand-off words
__device__ __forceinline__ void store_tagged(uint64_t* p, uint32_t epoch, float v) {
  __hip_atomic_store(p, ((uint64_t)epoch << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
// The same word for readers on this XCD only: it stays in the XCD's L2, where
// their coherent loads find it at L2 latency instead of a memory round trip
// behind the weight stream.
__device__ __forceinline__ void store_tagged_xcd(uint64_t* p, uint32_t epoch, float v) {
  __hip_atomic_store(p, ((uint64_t)epoch << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_WORKGROUP);
}
// two tagged words with one 16-byte coherent load: {lo0, epoch0, lo1, epoch1}
__device__ __forceinline__ uint4 coherent_ld_u4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, kCachePolicySc1);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 coherent_ld_u2(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)byte_off, 0, kCachePolicySc1);
  return make_uint2(v[0], v[1]);
}

struct Moe1Args {
  const uint8_t* base;
  int64_t stride;
  int64_t off[MOE_NUM_TENSORS];
  int E, H, I, k;
  const float* x;          // [H] expert input (and the router's, unless XR)
  const float* Wr;         // [E][H] (XR: [E][Hr]), or null: selection given in idx_in / w_in
  const int32_t* idx_in;   // [k]
  const float* w_in;       // [k]
  int32_t* idx_out;        // [k] or null
  float* w_out;            // [k] or null
  uint64_t* tlogits;       // ws [E]      tagged router logits
  uint64_t* th;            // ws [2][k][I] tagged intermediate activations: XCD copy, coherent copy
  uint64_t* tpart;         // ws [k][H]   tagged per-slot down outputs
  float* out;              // [H]
  uint32_t* ctrl;
  int n_router;
  const float* xr;         // XR instances: the router's own input [Hr]
  int Hr;
};

struct Moe1Shared {
  union {
    float xs[kMaxH1 + kMaxH1 / 8];   // x, padded 4 floats per 32 (router, gate/up)
    float hs[kMaxI1 + kMaxI1 / 8];   // h of the slot (down)
  } u;
  SelectLds sel;                   // wave 0's selection scratch
  float ys[kWG1];                  // the combine's slot results [k][H / kG1]
  int32_t sidx[MOE_MAX_TOPK];
  float sw[MOE_MAX_TOPK];
  int flag;
};

__device__ __forceinline__ bool wg_any(bool v, int* s_flag) {
  if (threadIdx.x == 0) *s_flag = 0;
  __syncthreads();
  if (v) *s_flag = 1;
  __syncthreads();
  return *s_flag != 0;
}

// Router: the 2E half rows of W_r are spread evenly, hpw = ceil(2E / kG1) <= 8
// per workgroup, one per wave: wave w of workgroup g takes half row
// hr = g * hpw + w (row hr / 2, columns (hr & 1) * H/2 .. +H/2).  Each half's
// dot product goes out, tagged, to every replica; the selection adds the two
// halves of a row in a fixed order.  The loads are issued first
// (moe1_router_load) so they can be in flight while x is staged.
constexpr int kRouterRU = kMaxH1 / 2 / 4 / 64;     // float4 loads per lane (max)

__device__ __forceinline__ int router_half_row(const Moe1Args& a) {
  const int hpw = (2 * a.n_router + kG1 - 1) / kG1;
  // uniform per wave (readfirstlane), so the half row's view is scalar and
  // its loads need no per-lane loop
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hr = blockIdx.x * hpw + wave;
  return (wave < hpw && hr < 2 * a.n_router) ? hr : -1;
}

// Every load is issued (those past the half row, or of a wave without one,
// fall outside the view and read zeros), so the loads form one straight run
// and later waits can count them exactly.
template <bool XR>
__device__ __forceinline__ void moe1_router_load(const Moe1Args& a, int hr, float4 (&wv)[kRouterRU]) {
  const int lane = threadIdx.x & 63;
  const int Hr = XR ? a.Hr : a.H;
  const int q = Hr / 2;                           // columns per half row
  const int e = hr >= 0 ? hr >> 1 : 0, half = hr & 1;
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(hr >= 0 ? a.Wr + (size_t)e * Hr : a.x), (short)0, hr >= 0 ? Hr * 4 : 0,
      0x00020000);
  const uint32_t woff = (uint32_t)(half * q + lane * 4) * 4;
#pragma unroll
  for (int u = 0; u < kRouterRU; ++u) {
    const int c = (lane + 64 * u) * 4;
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(
        wr, (int)(c < q ? woff + 1024 * u : 0x80000000u), 0, kCachePolicyNt);
    wv[u] = make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                        __uint_as_float(v[3]));
  }
}

template <bool XR>
__device__ __forceinline__ void moe1_router_finish(const Moe1Args& a, Moe1Shared& S, int hr,
                                                   const float4 (&wv)[kRouterRU], uint32_t epoch) {
  const int lane = threadIdx.x & 63;
  const int q = (XR ? a.Hr : a.H) / 2;
  if (hr < 0) return;                             // whole waves
  const int e = hr >> 1, half = hr & 1;
  float acc = 0.0f;
#pragma unroll
  for (int u = 0; u < kRouterRU; ++u) {
    const int c = (lane + 64 * u) * 4;
    if (c < q) {
      const int col = half * q + c;
      const float4 xv = *reinterpret_cast<const float4*>(&S.u.xs[col + (col >> 5) * 4]);
      acc += wv[u].x * xv.x + wv[u].y * xv.y + wv[u].z * xv.z + wv[u].w * xv.w;
    }
  }
  acc = wave_sum(acc);
  if (lane < kLogitCopies) store_tagged(&a.tlogits[(size_t)lane * 2 * a.E + 2 * e + half], epoch, acc);
}

// The selection, computed by every workgroup for itself from the tagged
// logits (or taken from the caller when the selection is given), by wave 0
// alone while the other waves wait at the closing barrier: it polls all E
// logits of one replica (lane l holds experts l + 64 i), reading again only
// the entries that do not yet carry this call's epoch; then a threshold on
// the lane maxima, the candidates above it gathered to LDS, each ranked by
// the number of candidates ahead of it (the same exact top-k as
// wave_select, which remains the fallback for clustered winners).
__device__ __forceinline__ void moe1_routing(const Moe1Args& a, Moe1Shared& S, uint32_t epoch, bool writer) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int k = a.k;
  constexpr int NPL = MOE_MAX_EXPERTS / 64;
  if (a.Wr) {
    if (wave == 0) {
      const __amdgpu_buffer_rsrc_t lr = coherent_view(
          a.tlogits + (size_t)(blockIdx.x % kLogitCopies) * 2 * a.E, (uint32_t)a.E * 16);
      uint4 t[NPL];                                  // {half 0, tag, half 1, tag}
      bool need[NPL];
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        need[i] = lane + 64 * i < a.E;
        t[i] = make_uint4(0u, 0u, 0u, 0u);
      }
      for (uint32_t it = 0;; ++it) {
#pragma unroll
        for (int i = 0; i < NPL; ++i)
          if (need[i]) t[i] = coherent_ld_u4(lr, (uint32_t)(lane + 64 * i) * 16);
        bool missing = false;
#pragma unroll
        for (int i = 0; i < NPL; ++i) {
          need[i] = need[i] && (t[i].y != epoch || t[i].w != epoch);
          missing |= need[i];
        }
        if (!__any(missing)) break;
        if (it == kSpinLimit) {
          if (lane == 0)
            __hip_atomic_store(&a.ctrl[kCtrlErr], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
      uint64_t ck[NPL];
      float lv[NPL];
      uint32_t m = 0;                                // this lane's largest 32-bit key
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        const int e = lane + 64 * i;
        const bool in = e < a.E;
        lv[i] = in ? __uint_as_float(t[i].x) + __uint_as_float(t[i].z) : 0.0f;
        const uint32_t kk = in ? logit_key(lv[i]) : 0u;
        ck[i] = in ? (((uint64_t)kk << 32) | (uint64_t)(~(uint32_t)e)) : 0;
        m = kk > m ? kk : m;
      }
      // T: the largest t whose low 16 bits are zero such that k lane maxima
      // are >= t (a bit-by-bit search over the upper half of the orderable
      // keys).  Those k lanes hold k experts with keys >= T, so every expert
      // of the top k has a key >= T; the candidates are the (usually few
      // more than k) experts at or above it.
      uint32_t T = 0;
      for (int bit = 31; bit >= 16; --bit) {
        const uint32_t c = T | (1u << bit);
        if (__popcll(__ballot(m >= c)) >= k) T = c;
      }
      // candidates: a bit per entry, placed by a prefix count over the lanes
      uint32_t cm = 0;
#pragma unroll
      for (int i = 0; i < NPL; ++i)
        cm |= (ck[i] != 0 && (uint32_t)(ck[i] >> 32) >= T) ? (1u << i) : 0u;
      const int cnt = __popc(cm);
      const int incl = wave_incl_scan(cnt);
      const int n = __builtin_amdgcn_readlane(incl, 63);
      int pos = incl - cnt;
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        if ((cm >> i) & 1u) {
          if (pos < 64) {
            S.sel.cand_key[pos] = ck[i];
            S.sel.cand_l[pos] = lv[i];
          }
          ++pos;
        }
      }
      if (n <= 64) {
        // zero keys after the last candidate up to a multiple of 4 (never ahead of a real key)
        if (lane >= n && lane < ((n + 3) & ~3)) S.sel.cand_key[lane] = 0;
        wave_lds_fence();
        const uint64_t mine = lane < n ? S.sel.cand_key[lane] : 0;
        const float ml = lane < n ? S.sel.cand_l[lane] : 0.0f;
        const float sg = 1.0f / (1.0f + expf(-ml));  // independent of the rank
        int rk = 0;                                  // candidates ahead (broadcast LDS reads)
        for (int j = 0; j < n; j += 4) {
          const uint64_t c0 = S.sel.cand_key[j], c1 = S.sel.cand_key[j + 1];
          const uint64_t c2 = S.sel.cand_key[j + 2], c3 = S.sel.cand_key[j + 3];
          rk += (c0 > mine) + (c1 > mine) + (c2 > mine) + (c3 > mine);
        }
        if (lane < n && rk < k) {
          S.sel.sel_e[rk] = (int32_t)~(uint32_t)mine;
          S.sel.sel_l[rk] = sg;                      // here the sigmoid, not the logit
        }
        wave_lds_fence();
        // the weights in slot order: sigmoid / the sum over the k slots
        const float sgk = lane < k ? S.sel.sel_l[lane] : 0.0f;
        const float w = sgk / wave_sum(sgk);
        if (lane < k) {
          const int e = S.sel.sel_e[lane];
          S.sidx[lane] = e;
          S.sw[lane] = w;
          if (writer && a.idx_out) a.idx_out[lane] = e;
          if (writer && a.w_out) a.w_out[lane] = w;
        }
      } else {
        wave_select<NPL>(ck, lv, k, S.sel);          // clustered winners
        const float l = lane < k ? S.sel.sel_l[lane] : 0.0f;
        const float w = route_weight(l, lane, k);
        if (lane < k) {
          const int e = S.sel.sel_e[lane];
          S.sidx[lane] = e;
          S.sw[lane] = w;
          if (writer && a.idx_out) a.idx_out[lane] = e;
          if (writer && a.w_out) a.w_out[lane] = w;
        }
      }
    }
  } else if (threadIdx.x < k) {
    S.sidx[threadIdx.x] = a.idx_in[threadIdx.x];
    S.sw[threadIdx.x] = a.w_in[threadIdx.x];
  }
  __syncthreads();
}

// acc[r] += sum over one 32-element chunk of w_r * x for NR rows and one token,
// one 8-element dword at a time (the barrier keeps the conversions of later
// dwords from being hoisted, which would hold a register per value).
template <int FMT, int NR>
__device__ __forceinline__ void chunk_fma1(const uint4 (&q)[NR], const uint32_t (&sc)[NR],
                                           const float* xs, int xoff, float (&acc)[NR][1]) {
  const float4* x4 = reinterpret_cast<const float4*>(xs + xoff);
  float blk[NR];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    if ((d & 1) == 0) {
#pragma unroll
      for (int r = 0; r < NR; ++r) blk[r] = 0.0f;
    }
    const float4 xa = x4[2 * d];
    const float4 xb = x4[2 * d + 1];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const uint32_t wd = (d == 0) ? q[r].x : (d == 1) ? q[r].y : (d == 2) ? q[r].z : q[r].w;
      const float2 v0 = fp4x2<0>(wd), v1 = fp4x2<1>(wd), v2 = fp4x2<2>(wd), v3 = fp4x2<3>(wd);
      float b = blk[r];
      b += v0.x * xa.x; b += v0.y * xa.y; b += v1.x * xa.z; b += v1.y * xa.w;
      b += v2.x * xb.x; b += v2.y * xb.y; b += v3.x * xb.z; b += v3.y * xb.w;
      blk[r] = b;
    }
    if (d & 1) {
      // one scale per 16 elements: NV has its own byte per half, MX shares one
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const float s = (FMT == MOE_FMT_NVFP4) ? e4m3_to_f32((sc[r] >> (8 * (d >> 1))) & 0xFFu)
                                               : e8m0_to_f32(sc[r]);
        acc[r][0] += s * blk[r];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One tensor of one expert as a buffer descriptor.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tensor_view(const uint8_t* rec, int64_t off,
                                                              uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(rec + off), (short)0, (int)bytes,
                                           0x00020000);
}

constexpr int kGuStage = 4;   // chunks per lane per pipeline stage (gate/up)
constexpr int kDnStage = 8;   // (down, one row per lane group at a time)
constexpr int kPipe = RF4_PIPE_DEPTH;   // register buffers of the weight stream

// Streamed dot products of one 16-lane group over NSEG consecutive segments
// (segment s = NR rows, one per row stream r, at offset coff[r] + s*seg_stride);
// lane l16 reads chunks l16 + 16*i (i < KCH) of each row.  The NSEG*KCH chunks
// run as one pipeline in stages of PB: the loads of stage t+1 are in flight
// while stage t is multiplied, across segment boundaries too.  After the last
// chunk of a segment, done(s, acc) receives the lane's partial sums.
template <int FMT, int NR, int NSEG, int KCH, int PB>
struct SegStream {
  static constexpr int NF = NSEG * KCH;
  static constexpr int NST = (NF + PB - 1) / PB;
  __amdgpu_buffer_rsrc_t crs[NR];
  __amdgpu_buffer_rsrc_t srs[NR];
  uint32_t coff[NR], soff[NR];       // segment 0, this lane's first chunk
  uint32_t seg_stride, seg_sstride;  // bytes between segments (codes, scales)
  __device__ __forceinline__ void load(int st, uint4 (&q)[PB][NR], uint32_t (&sc)[PB][NR]) const {
#pragma unroll
    for (int b = 0; b < PB; ++b) {
      const int f = st * PB + b;
      if (f < NF) {
        const int sg = f / KCH, i = f - sg * KCH;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const auto v = __builtin_amdgcn_raw_buffer_load_b128(
              crs[r], (int)(coff[r] + sg * seg_stride + 256 * i), 0, kCachePolicyNt);
          q[b][r] = make_uint4(v[0], v[1], v[2], v[3]);
          if (FMT == MOE_FMT_MXFP4)
            sc[b][r] = __builtin_amdgcn_raw_buffer_load_b8(
                srs[r], (int)(soff[r] + sg * seg_sstride + 16 * i), 0, kCachePolicyNt);
          else
            sc[b][r] = __builtin_amdgcn_raw_buffer_load_b16(
                srs[r], (int)(soff[r] + sg * seg_sstride + 32 * i), 0, kCachePolicyNt);
        }
      }
    }
  }
  template <class Done>
  __device__ __forceinline__ void fma(int st, const uint4 (&q)[PB][NR], const uint32_t (&sc)[PB][NR],
                                      const float* xs, float (&acc)[NR][1], Done& done) const {
    const int l16 = threadIdx.x & 15;
#pragma unroll
    for (int b = 0; b < PB; ++b) {
      const int f = st * PB + b;
      if (f < NF) {
        const int sg = f / KCH, i = f - sg * KCH;
        chunk_fma1<FMT, NR>(q[b], sc[b], xs, (l16 + 16 * i) * 36, acc);
        if (i == KCH - 1) {
          done(sg, acc);
#pragma unroll
          for (int r = 0; r < NR; ++r) acc[r][0] = 0.0f;
        }
      }
    }
  }
  // All stages, with D register buffers: the loads of stage t+D-1 are issued
  // just before stage t is multiplied (the barriers keep the compiler from
  // issuing them earlier, which would need more registers).  The caller may
  // have issued stages 0..npre-1 already (into q[0..npre-1]).
  template <int D, class Done>
  __device__ __forceinline__ void run(const float* xs, uint4 (&q)[D][PB][NR], uint32_t (&sc)[D][PB][NR],
                                      int npre, Done done) const {
    float acc[NR][1];
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[r][0] = 0.0f;
#pragma unroll
    for (int st = 0; st < D - 1; ++st)
      if (st >= npre && st < NST) load(st, q[st], sc[st]);
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      __builtin_amdgcn_sched_barrier(0);
      if (st + D - 1 < NST) load(st + D - 1, q[(st + D - 1) % D], sc[(st + D - 1) % D]);
      __builtin_amdgcn_sched_barrier(0);
      fma(st, q[st % D], sc[st % D], xs, acc, done);
    }
  }
};

// Gate/up slice: rows b*16*SGU + lg + 16*s (s < SGU) of slot u's expert;
// h = silu(g) * u goes out as tagged words.
template <int FMT, int KG, int SGU>
__device__ __forceinline__ void moe1_gate_up_slice(const Moe1Args& a, Moe1Shared& S, int u, int b, uint32_t epoch) {
  const int e = S.sidx[u];
  if (e < 0 || e >= a.E) return;                 // an invalid slot contributes nothing
  const int lg = threadIdx.x >> 4, l16 = threadIdx.x & 15;
  const int H = a.H, I = a.I;
  const int B = (FMT == MOE_FMT_MXFP4) ? 32 : 16;
  const int row0 = b * (kWG1 / 16) * SGU + lg;
  const uint8_t* rec = a.base + (size_t)e * a.stride;
  SegStream<FMT, 2, SGU, KG, kGuStage> ss;
  const uint32_t cbytes = (uint32_t)I * (H / 2), sbytes = (uint32_t)I * (H / B);
  ss.crs[0] = tensor_view(rec, a.off[MOE_T_GATE_CODES], cbytes);
  ss.crs[1] = tensor_view(rec, a.off[MOE_T_UP_CODES], cbytes);
  ss.srs[0] = tensor_view(rec, a.off[MOE_T_GATE_SCALES], sbytes);
  ss.srs[1] = tensor_view(rec, a.off[MOE_T_UP_SCALES], sbytes);
  ss.coff[0] = ss.coff[1] = (uint32_t)row0 * (H / 2) + l16 * 16;
  ss.soff[0] = ss.soff[1] = (uint32_t)row0 * (H / B) + l16 * (32 / B);
  ss.seg_stride = (kWG1 / 16) * (uint32_t)(H / 2);
  ss.seg_sstride = (kWG1 / 16) * (uint32_t)(H / B);
  float gg = 1.0f, gu = 1.0f;
  if (FMT == MOE_FMT_NVFP4) {
    const float* g = reinterpret_cast<const float*>(rec + a.off[MOE_T_GLOBALS]);
    gg = g[0];
    gu = g[1];
  }
  uint64_t* hout = a.th + (size_t)u * I;
  uint64_t* hcoh = hout + (size_t)a.k * I;
  auto done = [&](int sg, float (&acc)[2][1]) {
    const float gsum = group16_sum(acc[0][0]);
    const float usum = group16_sum(acc[1][0]);
    if (l16 == 0) {
      const int j = row0 + (kWG1 / 16) * sg;
      const float h = silu(gg * gsum) * (gu * usum);
      store_tagged_xcd(&hout[j], epoch, h);
      store_tagged(&hcoh[j], epoch, h);
    }
  };
  uint4 q[kPipe][kGuStage][2];
  uint32_t sc[kPipe][kGuStage][2];
  ss.template run<kPipe>(S.u.xs, q, sc, 0, done);
}

// Down slice: rows b*R + lg + 16*s (within the block of R = H / workgroups per
// slot) of slot u's expert, against h_u; the results go out as tagged words,
// or, for the last slot, to LDS for the combine.
template <int FMT, int KD, int SDN, int KT>
__device__ __forceinline__ void moe1_down_slice(const Moe1Args& a, Moe1Shared& S, int u, int b, int R,
                                uint32_t epoch, bool xcd_local) {
  const int e = S.sidx[u];
  const bool valid = e >= 0 && e < a.E;
  const int lg = threadIdx.x >> 4, l16 = threadIdx.x & 15;
  const int H = a.H, I = a.I;
  const int B = (FMT == MOE_FMT_MXFP4) ? 32 : 16;
  const int row0 = b * R + lg;
  if (valid) {
    const uint8_t* rec = a.base + (size_t)e * a.stride;
    SegStream<FMT, 1, SDN, KD, kDnStage> ss;
    // rows past the tensor read zeros (descriptor bounds) and are never stored
    ss.crs[0] = tensor_view(rec, a.off[MOE_T_DOWN_CODES], (uint32_t)H * (I / 2));
    ss.srs[0] = tensor_view(rec, a.off[MOE_T_DOWN_SCALES], (uint32_t)H * (I / B));
    ss.coff[0] = (uint32_t)row0 * (I / 2) + l16 * 16;
    ss.soff[0] = (uint32_t)row0 * (I / B) + l16 * (32 / B);
    ss.seg_stride = (kWG1 / 16) * (uint32_t)(I / 2);
    ss.seg_sstride = (kWG1 / 16) * (uint32_t)(I / B);
    uint4 q[kPipe][kDnStage][1];
    uint32_t sc[kPipe][kDnStage][1];
#pragma unroll
    for (int st = 0; st < kPipe - 1; ++st) ss.load(st, q[st], sc[st]);
    // the first weights are in flight; now fetch this slot's h (polling until
    // every value carries this call's epoch) into LDS, over the dead x stage
    __syncthreads();
    {
      // The slot's workgroups share this XCD (see k_moe1), so h is read from
      // the XCD copy, which stays in its L2.  Should they not (another
      // dispatch order), the XCD copy never arrives here and the polls move to
      // the coherent copy after kXcdPolls tries.
      const __amdgpu_buffer_rsrc_t hx = coherent_view(a.th + (size_t)u * I, (uint32_t)I * 8);
      const __amdgpu_buffer_rsrc_t hc = coherent_view(a.th + (size_t)(a.k + u) * I, (uint32_t)I * 8);
      constexpr int NP = (KD * 512 / 2 + kWG1 - 1) / kWG1;   // 16-byte pairs per thread
      for (uint32_t it = 0;; ++it) {
        const __amdgpu_buffer_rsrc_t hv = (xcd_local && it < kXcdPolls) ? hx : hc;
        bool missing = false;
        uint4 t[NP];
#pragma unroll
        for (int v = 0; v < NP; ++v) {                     // all loads in flight at once
          const int i = (threadIdx.x + v * kWG1) * 2;
          t[v] = coherent_ld_u4(hv, (uint32_t)i * 8);      // past the end reads zeros
        }
#pragma unroll
        for (int v = 0; v < NP; ++v) {
          const int i = (threadIdx.x + v * kWG1) * 2;
          if (i < I) {
            missing |= (t[v].y != epoch) | (t[v].w != epoch);
            *reinterpret_cast<float2*>(&S.u.hs[i + (i >> 5) * 4]) =
                make_float2(__uint_as_float(t[v].x), __uint_as_float(t[v].z));
          }
        }
        if (!wg_any(missing, &S.flag)) break;
        if (it == kSpinLimit) {
          if (threadIdx.x == 0)
            __hip_atomic_store(&a.ctrl[kCtrlErr], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    float gd = 1.0f;
    if (FMT == MOE_FMT_NVFP4) gd = reinterpret_cast<const float*>(rec + a.off[MOE_T_GLOBALS])[2];
    const float wgt = S.sw[u] * gd;
    auto done = [&](int sg, float (&acc)[1][1]) {
      const float y = wgt * group16_sum(acc[0][0]);
      const int rl = lg + (kWG1 / 16) * sg, j = b * R + rl;
      if (l16 == 0 && rl < R && j < H) store_tagged(&a.tpart[(size_t)u * H + j], epoch, y);
    };
    ss.template run<kPipe>(S.u.hs, q, sc, kPipe - 1, done);
  }
}

// The combine: workgroup g adds the k slot results of rows g * RC .. g * RC +
// RC - 1 (RC = H / kG1) in slot order, one tagged word per thread in flight
// at once, so the last hop of the layer is one small poll on every CU.
// Then workgroup 0 publishes the next epoch once every workgroup has read
// this call's: `arrived` holds the arrival words as read after the selection
// (they are written at each workgroup's start, so normally all are there);
// any that were not are polled again here.
template <int KT>
__device__ __forceinline__ void moe1_combine(const Moe1Args& a, Moe1Shared& S, uint32_t epoch, uint32_t arrived) {
  const int H = a.H, RC = H / kG1;
  const int j0 = blockIdx.x * RC, tid = threadIdx.x;
  const int sl = tid / RC, r = tid - sl * RC;
  const bool in = tid < KT * RC;
  const int e = in ? S.sidx[sl] : -1;
  const bool mine = in && e >= 0 && e < a.E;
  const __amdgpu_buffer_rsrc_t pv = coherent_view(a.tpart, (uint32_t)((size_t)KT * H * 8));
  uint2 t = make_uint2(0u, 0u);
  for (uint32_t it = 0;; ++it) {
    t = coherent_ld_u2(pv, mine ? (uint32_t)(((size_t)sl * H + j0 + r) * 8) : 0x80000000u);
    if (!wg_any(mine && t.y != epoch, &S.flag)) break;
    if (it == kSpinLimit) {
      if (tid == 0) __hip_atomic_store(&a.ctrl[kCtrlErr], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  if (in) S.ys[tid] = __uint_as_float(t.x);
  __syncthreads();
  if (tid < RC) {
    float acc = 0.0f;
    for (int s2 = 0; s2 < KT; ++s2) {
      const int e2 = S.sidx[s2];
      if (e2 >= 0 && e2 < a.E) acc += S.ys[s2 * RC + tid];
    }
    a.out[j0 + tid] = acc;
  }
  if (blockIdx.x == 0) {
    const __amdgpu_buffer_rsrc_t av = coherent_view(&a.ctrl[kCtrlArrive], kG1 * 4);
    for (uint32_t it = 0;; ++it) {
      if (it > 0 && tid < kG1) arrived = __float_as_uint(coherent_ld(av, tid * 4));
      if (!wg_any(tid < kG1 && arrived != epoch, &S.flag)) break;
      if (it == kSpinLimit) {
        if (tid == 0) __hip_atomic_store(&a.ctrl[kCtrlErr], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (tid == 0) __hip_atomic_store(&a.ctrl[kCtrlEpoch], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The whole layer for one token, kG1 workgroups (all resident at once).
// Every workgroup has a fixed share of each phase, and every expert has the
// same size, so the work is balanced whatever the routing (the one-GPU form
// of slicing every expert across workers, page "Kimi-K3 on the same pod, two
// engines", section "Reason 1"):
//   1. router: ceil(2E / G) half rows per workgroup, one per wave
//   2. the selection: every workgroup reads all E tagged logits and runs the
//      same top-k on them
//   3. gate/up: slot u's G/k workgroups (on one XCD), I / (G/k) rows each
//   4. down: the same workgroups, H / (G/k) rows of H each
//   5. combine: H / G rows per workgroup, the k slot results in slot order.
// Hand-offs carry the call's epoch (see above); the polls form a chain
// router -> selection -> gate/up -> down -> combine, so with every workgroup
// resident each poll ends, and each is bounded anyway.
// KG = H/512, KD = I/512 (16-byte chunks per lane per row); SGU, SDN: row
// segments per 16-lane group in the gate/up and down slices.  XR: the router
// reads an input of its own, xr [Hr] (a latent layer routes on the hidden
// state while its experts take the latent vector).
template <int FMT, int KG, int KD, int SGU, int SDN, int KT, bool XR>
__global__ __launch_bounds__(kWG1, 1) void k_moe1(Moe1Args a) {
  __shared__ Moe1Shared S;
  const int tid = threadIdx.x;
  // the epoch first, ahead of the router stream in this CU's memory queue
  const uint32_t epoch =
      __hip_atomic_load(&a.ctrl[kCtrlEpoch], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  // x next, then the router rows; x goes to LDS (where it stays through the
  // gate/up slice) as soon as its own loads are in, while the rows stream
  constexpr int kXv = kMaxH1 / (kWG1 * 4);              // float4 of x per thread
  float4 xv[kXv];
#pragma unroll
  for (int j = 0; j < kXv; ++j) {
    const int i = (tid + j * kWG1) * 4;
    const int Hr = XR ? a.Hr : a.H;
    xv[j] = i < Hr ? *reinterpret_cast<const float4*>((XR ? a.xr : a.x) + i)
                   : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __builtin_amdgcn_sched_barrier(0);
  float4 wv[kRouterRU];
  const int hr = router_half_row(a);
  moe1_router_load<XR>(a, hr, wv);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < kXv; ++j) {
    const int i = (tid + j * kWG1) * 4;
    if (i < (XR ? a.Hr : a.H)) *reinterpret_cast<float4*>(&S.u.xs[i + (i >> 5) * 4]) = xv[j];
  }
  // this workgroup has read the epoch (the combine waits for all of these
  // before it publishes the next one)
  if (tid == 0)
    __hip_atomic_store(&a.ctrl[kCtrlArrive + blockIdx.x], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  moe1_router_finish<XR>(a, S, hr, wv, epoch);
  if (XR) {
    // the expert input replaces the router's in LDS for the gate/up slice
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kXv; ++j) {
      const int i = (tid + j * kWG1) * 4;
      if (i < a.H)
        *reinterpret_cast<float4*>(&S.u.xs[i + (i >> 5) * 4]) = *reinterpret_cast<const float4*>(a.x + i);
    }
    __syncthreads();
  }
  moe1_routing(a, S, epoch, blockIdx.x == 0);
  // the arrival words, read early (used by the combine of workgroup 0)
  uint32_t arrived = 0u;
  if (blockIdx.x == 0 && tid < kG1)
    arrived = __float_as_uint(coherent_ld(coherent_view(&a.ctrl[kCtrlArrive], kG1 * 4), tid * 4));
  // Slot u's wpe workgroups: with k a multiple of kXcds they all run on one
  // XCD (workgroup w is dispatched to XCD w % kXcds), which keeps the h
  // hand-off between them in that XCD's L2.
  const int wpe = gridDim.x / a.k;               // workgroups per slot
  const bool xcd_local = a.k % kXcds == 0;
  int u, b;
  if (xcd_local) {
    const int x = blockIdx.x % kXcds, r = blockIdx.x / kXcds;
    u = x * (a.k / kXcds) + r / wpe;
    b = r % wpe;
  } else {
    u = blockIdx.x / wpe;
    b = blockIdx.x - u * wpe;
  }
  moe1_gate_up_slice<FMT, KG, SGU>(a, S, u, b, epoch);
  moe1_down_slice<FMT, KD, SDN, KT>(a, S, u, b, a.H / wpe, epoch, xcd_local);
  moe1_combine<KT>(a, S, epoch, arrived);
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
  // With x, the top-k (and the dispatch table) runs as its own launch, one
  // wave per token, instead of in the router's last workgroup (one token:
  // the one-wave selection of the separate launch is also the faster).
  a.select = x ? 0 : 1;
  if (C == 1) hipLaunchKernelGGL(k_route<1>, dim3(grid), dim3(kWG), 0, st, a);
  else if (C <= 4) hipLaunchKernelGGL(k_route<4>, dim3(grid), dim3(kWG), 0, st, a);
  else hipLaunchKernelGGL(k_route<16>, dim3(grid), dim3(kWG), 0, st, a);
  moe_status s = launch_status();
  if (s == MOE_OK && !a.select)
    s = launch_topk_parts(a.lpart, a.ksplit, logits_out, C, E, k, idx, w, disp, st);
  return s;
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

// The batch-1 kernel instances that are built: (format, H, I, k) -> template.
// Each needs k | kG1, 16 | I*k/kG1 rows per gate/up slice, and kG1/k | H.
struct Moe1Shape {
  int H, I, k;
};

template <int FMT, int KG, int KD, int SGU, int SDN, int KT, bool XR = false>
moe_status launch_moe1_kernel(Moe1Args a, hipStream_t st) {
  // per device: 1 = kG1 workgroups fit at once, -1 = they do not (0: not yet known)
  static std::atomic<int> ok_dev[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int ok = ok_dev[dev].load(std::memory_order_relaxed);
  if (ok == 0) {
    // two threads may both query; they store the same answer
    int per_cu = 0;
    const bool fits = hipOccupancyMaxActiveBlocksPerMultiprocessor(
                          &per_cu, k_moe1<FMT, KG, KD, SGU, SDN, KT, XR>, kWG1, 0) == hipSuccess &&
                      per_cu * device_cu_count() >= kG1;
    ok = fits ? 1 : -1;
    ok_dev[dev].store(ok, std::memory_order_relaxed);
  }
  if (ok < 0) return MOE_ERR_UNSUPPORTED;
  // A plain launch: with at most one workgroup per CU and kG1 <= the CUs
  // that can hold one, every workgroup is resident once the stream's earlier
  // work has drained, so every wait ends.  (The cooperative launch API gives
  // the same guarantee but costs about 17 us more per call on this stack.)
  // Should other work hold CUs indefinitely, the bounded waits give up and set
  // the workspace's error word instead of hanging.
  hipLaunchKernelGGL((k_moe1<FMT, KG, KD, SGU, SDN, KT, XR>), dim3(kG1), dim3(kWG1), 0, st, a);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return MOE_ERR_DEVICE;
  return MOE_OK;
}

template <int FMT>
moe_status launch_moe1_fmt(const Moe1Args& a, hipStream_t st) {
  // SGU = I*k / (kG1 * 32), SDN = ceil(H*k / (kG1 * 32))
  if (a.xr) {
    // latent layers (router on the hidden state): the latent K3 and W50 shapes
    if (a.H == 3584 && a.I == 3072 && a.k == 16) return launch_moe1_kernel<FMT, 7, 6, 6, 7, 16, true>(a, st);
    if (a.H == 3584 && a.I == 3072 && a.k == 8) return launch_moe1_kernel<FMT, 7, 6, 3, 4, 8, true>(a, st);
    return MOE_ERR_UNSUPPORTED;
  }
  if (a.H == 7168 && a.I == 1536 && a.k == 16) return launch_moe1_kernel<FMT, 14, 3, 3, 14, 16>(a, st);
  if (a.H == 3584 && a.I == 3072 && a.k == 16) return launch_moe1_kernel<FMT, 7, 6, 6, 7, 16>(a, st);
  if (a.H == 3584 && a.I == 3072 && a.k == 8) return launch_moe1_kernel<FMT, 7, 6, 3, 4, 8>(a, st);
  return MOE_ERR_UNSUPPORTED;
}

bool moe1_fits(const moe_bank* b, int C, int k) {
  if (C != 1) return false;
  const int H = b->hidden, I = b->inter;
  const bool built = (H == 7168 && I == 1536 && k == 16) || (H == 3584 && I == 3072 && (k == 16 || k == 8));
  // the combine holds k slot results of H / kG1 rows in LDS, one per thread
  return built && H % kG1 == 0 && k * (H / kG1) <= kWG1;
}

// MOE_ERR_UNSUPPORTED when the device cannot hold all kG1 workgroups at once
// (the caller then takes the multi-kernel path); nothing has been enqueued in
// that case.
moe_status launch_moe1(const moe_bank* b, const float* Wr, const float* x, int k,
                       const int32_t* idx_in, const float* w_in, int32_t* idx_out, float* w_out,
                       float* out, uint8_t* ws, const WsLayout& L, hipStream_t st,
                       const float* xr = nullptr, int Hr = 0) {
  Moe1Args a;
  a.base = static_cast<const uint8_t*>(b->base);
  a.stride = b->expert_stride;
  for (int t = 0; t < MOE_NUM_TENSORS; ++t) a.off[t] = b->offset[t];
  a.E = b->num_experts; a.H = b->hidden; a.I = b->inter; a.k = k;
  a.x = x; a.Wr = Wr;
  a.xr = xr;             // null: the router reads x
  a.Hr = xr ? Hr : 0; a.idx_in = idx_in; a.w_in = w_in; a.idx_out = idx_out; a.w_out = w_out;
  a.tlogits = reinterpret_cast<uint64_t*>(ws + L.tlogits);
  a.th = reinterpret_cast<uint64_t*>(ws + L.th);
  a.tpart = reinterpret_cast<uint64_t*>(ws + L.tpart);
  a.out = out;
  a.ctrl = reinterpret_cast<uint32_t*>(ws + L.ctrl);
  a.n_router = Wr ? a.E : 0;
  return b->format == MOE_FMT_MXFP4 ? launch_moe1_fmt<MOE_FMT_MXFP4>(a, st)
                                    : launch_moe1_fmt<MOE_FMT_NVFP4>(a, st);
}

bool tokens_ok(int C) { return C >= 1 && C <= MOE_MAX_TOKENS; }
bool batched_shape(const moe_bank* b) { return batched_shape_ok(b); }
bool topk_ok(int k, int E) { return k >= 1 && k <= MOE_MAX_TOPK && k <= E; }

}  // namespace

namespace rf4 {
moe_status layer1_router_input(const moe_bank* b, const float* w_router, const float* xr, int Hr,
                               const float* x, int k, float* out, int32_t* idx, float* w,
                               void* ws, size_t ws_bytes, hipStream_t st) {
  if (check_bank(b) != MOE_OK || !moe1_fits(b, 1, k) || !topk_ok(k, b->num_experts))
    return MOE_ERR_UNSUPPORTED;
  if (Hr < 32 || Hr % 32 || Hr > kMaxH1) return MOE_ERR_UNSUPPORTED;
  if (!w_router || !xr || !x || !out || !idx || !w || !aligned(xr, 16) || !aligned(x, 16) ||
      !aligned(w_router, 16))
    return MOE_ERR_INVALID_ARG;
  const WsLayout L = ws_layout(b->num_experts, b->hidden, b->inter, k, 1);
  if (!ws || ws_bytes < L.total || !aligned(ws, 256)) return MOE_ERR_WORKSPACE;
  return launch_moe1(b, w_router, x, k, nullptr, nullptr, idx, w, out, static_cast<uint8_t*>(ws), L,
                     st, xr, Hr);
}
moe_status bank_status(const moe_bank* b) { return check_bank(b); }
}  // namespace rf4

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
  // the router needs only the counters, partial sums and logits: size for I = 32
  const WsLayout L = ws_layout(E, H, 32, k, C);
  if (ws_bytes < L.total || !aligned(ws, 256)) return MOE_ERR_WORKSPACE;
  if (C > MOE_MAX_DECODE_TOKENS)
    return launch_batched_route(x, w_router, x ? nullptr : logits, x ? logits : nullptr, C, H, E,
                                k, topk_idx, topk_w, static_cast<uint8_t*>(ws), L,
                                reinterpret_cast<hipStream_t>(stream));
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
  if (moe1_fits(bank, C, k)) {
    const moe_status m = launch_moe1(bank, nullptr, x, k, topk_idx, topk_w, nullptr, nullptr, out,
                                     w8, L, st);
    if (m != MOE_ERR_UNSUPPORTED) return m;
  }
  if (batched_shape(bank) && !batched_decode_shape(bank, C))
    return launch_batched_experts(bank, x, C, k, topk_idx, topk_w, out, w8, L, st);
  if (C > MOE_MAX_DECODE_TOKENS) return MOE_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(k_dispatch, dim3(1), dim3(kWG), 0, st, topk_idx,
                     reinterpret_cast<int32_t*>(w8 + L.disp), C, k, bank->num_experts);
  if ((s = launch_status()) != MOE_OK) return s;
  if (batched_shape(bank))
    return launch_batched_decode(bank, x, C, k, topk_idx, topk_w, out, w8, L, st);
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
  if (moe1_fits(bank, C, k)) {
    const moe_status m = launch_moe1(bank, w_router, x, k, nullptr, nullptr, idx, w, out, w8, L, st);
    if (m != MOE_ERR_UNSUPPORTED) return m;
  }
  const bool batched = batched_shape(bank);
  if (!batched && C > MOE_MAX_DECODE_TOKENS) return MOE_ERR_UNSUPPORTED;
  if (C > MOE_MAX_DECODE_TOKENS)
    s = launch_batched_route(x, w_router, nullptr, nullptr, C, bank->hidden, bank->num_experts, k,
                             idx, w, w8, L, st);
  else
    s = launch_route(x, w_router, nullptr, nullptr, C, bank->hidden, bank->num_experts, k, idx, w,
                     (batched && !batched_decode_shape(bank, C))
                         ? nullptr
                         : reinterpret_cast<int32_t*>(w8 + L.disp),
                     w8, L, st);
  if (s != MOE_OK) return s;
  if (batched && batched_decode_shape(bank, C))
    return launch_batched_decode(bank, x, C, k, idx, w, out, w8, L, st);
  if (batched) return launch_batched_experts(bank, x, C, k, idx, w, out, w8, L, st);
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
