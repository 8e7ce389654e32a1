// libroutedfp4, latent MoE layer: the steps either side of the routed experts.
//
// Page "SparkInfer-K3", section "How the TP module works", splits a K3 MoE layer
// into a partial phase (router, routed_down, the routed experts) and a finish
// phase (routed_norm, routed_up, shared experts); section "Why the reduce is at
// 3584 and not 7168" puts the RMS norm after the sum of the routed experts,
// because the norm is not linear; section "The model" gives 896 routed experts,
// top-16, 2 shared experts, a latent width of 3584 and an expert FFN of 3072.
// On one GPU the layer is
//
//   idx, w = top-k(x W_r^T)                       (router on the hidden x)
//   x_lat  = W_down x                             (hidden -> latent, dense)
//   y_lat  = sum_s w_s FFN_e(s)(x_lat)            (routed experts, latent)
//   out    = W_up (gamma * y_lat / rms(y_lat)) + sum_j FFN_shared_j(x)
//
// with rms(y) = sqrt(mean(y^2) + eps).  The dense matrices are bf16 with fp32
// products and sums; the experts run in the library's expert paths.
//
// Kernels:
//   k_gemv      y[t] (+)= s_t * W (g * x[t]) for C <= 16 tokens: bf16 W [N][K],
//               fp32 x [C][K]; with g (the norm's gamma) the row scale s_t is
//               1 / rms(x[t]), else s_t = 1 and g = 1.  The routed_down launch
//               also writes the shared experts' selection (every token, every
//               shared expert, weight 1).
//   k_lat_in    one token: routed_down (as k_gemv) and, in the same launch,
//               the shared experts' gate/up with SwiGLU as row-blocked
//               mat-vecs (both read only x)
//   k_lat_out   one token: per block of 8 output rows, the shared experts'
//               down sum plus routed_up with the norm folded in
//   (more tokens: k_gemv for the dense steps and the library's decode-batch
//   streams for the shared experts)
#include "common.h"

namespace rf4 {
namespace {

struct GemvArgs {
  const uint16_t* W;      // [N][K] bf16
  const float* x;         // [C][K]
  const float* gamma;     // [K], or null: no norm
  float eps;
  float* y;               // [C][N]
  int C, N, K;
  int accumulate;         // 1: y += result
  int32_t* sel_idx;       // or null: [C][ns] shared-expert selection to write
  float* sel_w;
  int32_t* sel_disp;      // or null: the shared experts' dispatch table to write
  int ns;
};

constexpr int kGemvWG = 256;

// Weight bytes are read once per call: non-temporal loads keep them from
// displacing the activations in the caches (1 to 1.5 us per launch on the
// K3 latent shape against plain loads).
// Weight loads as buffer loads that are always issued: an offset past the
// view (kOutside) reads zeros without memory traffic, so no load sits in a
// branch and the compiler's count of loads in flight stays exact (with
// loads in branches it waits for all of them where they join, before the
// next stream's loads are even issued).
constexpr uint32_t kOutside = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t lview(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t v, uint32_t off) {
  const auto t = __builtin_amdgcn_raw_buffer_load_b128(v, (int)off, 0, kCachePolicyNt);
  return make_uint4(t[0], t[1], t[2], t[3]);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Sum over the wave with DPP row shifts and row broadcasts; every lane gets
// lane 63's total.
template <int CTRL, int RMASK>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, RMASK, 0xF, false));
}

__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f<0x111, 0xF>(v);   // row_shr:1
  v += dpp_f<0x112, 0xF>(v);   // row_shr:2
  v += dpp_f<0x114, 0xF>(v);   // row_shr:4
  v += dpp_f<0x118, 0xF>(v);   // row_shr:8
  v += dpp_f<0x142, 0xA>(v);   // row_bcast:15
  v += dpp_f<0x143, 0xC>(v);   // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// The shared experts' selection (every token, every shared expert, weight 1)
// and, where asked for, their dispatch table: distinct experts in order of
// first use (0 .. ns-1), each with every token's pair t * ns + u in token
// order.  Block 0 of the routed_down launch writes them.
__device__ void write_shared_selection(const GemvArgs& a) {
  const int tid = threadIdx.x, ns = a.ns, C = a.C, CK = C * ns;
  for (int i = tid; i < CK; i += kGemvWG) {
    a.sel_idx[i] = i % ns;
    a.sel_w[i] = 1.0f;
  }
  if (a.sel_disp) {
    if (tid == 0) a.sel_disp[0] = ns;
    for (int u = tid; u < ns; u += kGemvWG) {
      a.sel_disp[disp_uexp(CK) + u] = u;
      a.sel_disp[disp_untok(CK) + u] = C;
    }
    for (int i = tid; i < CK; i += kGemvWG) {
      const int u = i / C, t = i - u * C;
      a.sel_disp[disp_upair(CK) + u * C + t] = t * ns + u;
    }
  }
}

// Rows n0 .. n0+RB-1, the whole K, per-thread partial sums: the 256 threads
// split each row into 16-byte chunks (8 bf16), NCH chunks per thread per slab
// of 2048 * NCH elements; every weight load of a slab is issued before any
// arithmetic, and x (with gamma applied) comes straight from L2 into
// registers for each chunk, in groups of up to 4 tokens.  With the norm, the
// same x values give each token's sum of squares over K (ss).
template <int RB, int CM, int NCH, bool ONE = false>
__device__ __forceinline__ void gemv_dot(const GemvArgs& a, int n0, float (&acc)[RB][CM],
                                         float (&ss)[CM]) {
  constexpr int TG = CM < 4 ? CM : 4;                 // tokens per x group
  const int tid = threadIdx.x;
  const int C = a.C, K = a.K, N = a.N, K8 = K >> 3;
  const bool norm = a.gamma != nullptr;
#pragma unroll
  for (int t = 0; t < CM; ++t) {
    ss[t] = 0.0f;
#pragma unroll
    for (int r = 0; r < RB; ++r) acc[r][t] = 0.0f;
  }

  __amdgpu_buffer_rsrc_t wv[RB];                     // row n0 + r (empty past N)
#pragma unroll
  for (int r = 0; r < RB; ++r)
    wv[r] = lview(a.W + (size_t)(n0 + r < N ? n0 + r : 0) * K, n0 + r < N ? (uint32_t)K * 2u : 0u);
  // ONE: K fits one slab (K / 8 <= kGemvWG * NCH); then there is no loop,
  // and a caller's weight loads issued before this call stay in flight with
  // these (a loop's entry makes the compiler wait for them)
  const int c0end = ONE ? 1 : K8;
  for (int c0 = 0; c0 < c0end; c0 += kGemvWG * NCH) {
    uint4 wq[RB][NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = c0 + tid + kGemvWG * j;
#pragma unroll
      for (int r = 0; r < RB; ++r) wq[r][j] = bload16(wv[r], c < K8 ? 16u * (uint32_t)c : kOutside);
    }
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = c0 + tid + kGemvWG * j;
      if (c >= K8) break;
      float4 ga = make_float4(1.f, 1.f, 1.f, 1.f), gb = ga;
      if (norm) {
        ga = *reinterpret_cast<const float4*>(a.gamma + 8 * c);
        gb = *reinterpret_cast<const float4*>(a.gamma + 8 * c + 4);
      }
#pragma unroll
      for (int t0 = 0; t0 < CM; t0 += TG) {
        if (t0 >= C) break;
        float4 xa[TG], xb[TG];
#pragma unroll
        for (int u = 0; u < TG; ++u) {
          const int t = t0 + u < C ? t0 + u : t0;
          xa[u] = *reinterpret_cast<const float4*>(a.x + (size_t)t * K + 8 * c);
          xb[u] = *reinterpret_cast<const float4*>(a.x + (size_t)t * K + 8 * c + 4);
        }
#pragma unroll
        for (int u = 0; u < TG; ++u) {
          if (t0 + u >= C) break;
          float4 p = xa[u], q = xb[u];
          if (norm) {
            float s = ss[t0 + u];
            s += p.x * p.x; s += p.y * p.y; s += p.z * p.z; s += p.w * p.w;
            s += q.x * q.x; s += q.y * q.y; s += q.z * q.z; s += q.w * q.w;
            ss[t0 + u] = s;
            p.x *= ga.x; p.y *= ga.y; p.z *= ga.z; p.w *= ga.w;
            q.x *= gb.x; q.y *= gb.y; q.z *= gb.z; q.w *= gb.w;
          }
#pragma unroll
          for (int r = 0; r < RB; ++r) {
            const uint4 w = wq[r][j];
            float s = acc[r][t0 + u];
            s += bf16_lo(w.x) * p.x; s += bf16_hi(w.x) * p.y;
            s += bf16_lo(w.y) * p.z; s += bf16_hi(w.y) * p.w;
            s += bf16_lo(w.z) * q.x; s += bf16_hi(w.z) * q.y;
            s += bf16_lo(w.w) * q.z; s += bf16_hi(w.w) * q.w;
            acc[r][t0 + u] = s;
          }
        }
      }
    }
  }
}

// Block blk of the mat-vec: rows blk*RB .. blk*RB+RB-1.  The per-thread
// partial sums are reduced over the wave (DPP) and then over the four waves
// in order.
template <int RB, int CM, int NCH, bool ONE = false>
__device__ __forceinline__ void gemv_block(const GemvArgs& a, int blk) {
  __shared__ float s_part[kGemvWG / 64][RB * CM + CM];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int C = a.C, K = a.K, N = a.N;
  const int n0 = blk * RB;
  const bool norm = a.gamma != nullptr;
  if (a.sel_idx && blk == 0) write_shared_selection(a);

  float acc[RB][CM], ss[CM];
  gemv_dot<RB, CM, NCH, ONE>(a, n0, acc, ss);

#pragma unroll
  for (int t = 0; t < CM; ++t) {
    if (t < C) {
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const float v = wave_sum_dpp(acc[r][t]);
        if (lane == 0) s_part[wave][r * CM + t] = v;
      }
      if (norm) {
        const float v = wave_sum_dpp(ss[t]);
        if (lane == 0) s_part[wave][RB * CM + t] = v;
      }
    }
  }
  __syncthreads();
  if (tid < RB * C) {
    const int r = tid / C, t = tid - r * C, n = n0 + r;
    if (n < N) {
      const int i = r * CM + t;
      float v = ((s_part[0][i] + s_part[1][i]) + s_part[2][i]) + s_part[3][i];
      if (norm) {
        const int j = RB * CM + t;
        const float sq = ((s_part[0][j] + s_part[1][j]) + s_part[2][j]) + s_part[3][j];
        v *= 1.0f / sqrtf(sq / (float)K + a.eps);
      }
      float* yp = a.y + (size_t)t * N + n;
      *yp = a.accumulate ? *yp + v : v;
    }
  }
}

template <int RB, int CM, int NCH>
__global__ __launch_bounds__(kGemvWG) void k_gemv(GemvArgs a) {
  gemv_block<RB, CM, NCH>(a, blockIdx.x);
}

template <int RB, int CM, int NCH>
void launch_gemv_t(const GemvArgs& a, hipStream_t st) {
  const int grid = (a.N + RB - 1) / RB;
  hipLaunchKernelGGL((k_gemv<RB, CM, NCH>), dim3(grid), dim3(kGemvWG), 0, st, a);
}

moe_status launch_gemv(const GemvArgs& a, hipStream_t st) {
  if (a.C <= 1) launch_gemv_t<8, 1, 4>(a, st);
  else if (a.C <= 4) launch_gemv_t<4, 4, 4>(a, st);
  else launch_gemv_t<4, 16, 2>(a, st);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

// ---------------------------------------------------------------------------
// Shared experts for one token: every shared expert, weight 1, as row-blocked
// mat-vecs folded into the two dense launches (the decode-batch streams,
// built for many experts, leave most CUs idle on two).
// ---------------------------------------------------------------------------
struct SArgs {
  const uint8_t* base;
  int64_t stride;
  int64_t off[MOE_NUM_TENSORS];
  int ns, H, I;
  const float* x;   // [H]
  float* h;         // [ns][I]
};

constexpr int kSRowsGU = 4;      // intermediate rows (gate and up) per workgroup
constexpr int kSRowsDN = 8;      // output rows per workgroup
constexpr int kSMaxCh = 2;       // 32-element chunks per thread at most (K <= 16384)

// sum over one 32-element chunk of w * x: MXFP4 with the power-of-two scale
// applied in the conversion, NVFP4 as two 16-element block sums times their
// e4m3 scales (the tensor's global scale is applied by the caller)
template <int FMT>
__device__ __forceinline__ float sdot32(const uint4& q, uint32_t sc, const float* xv) {
  constexpr bool MX = FMT == MOE_FMT_MXFP4;
  const float s = MX ? __uint_as_float((sc & 0xFFu) << 23) : 1.0f;
  float b[2] = {0.0f, 0.0f};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t wd = d == 0 ? q.x : d == 1 ? q.y : d == 2 ? q.z : q.w;
    const auto v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd, s, 0);
    const auto v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd, s, 1);
    const auto v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd, s, 2);
    const auto v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd, s, 3);
    float t = b[d >> 1];
    t += v0[0] * xv[8 * d + 0]; t += v0[1] * xv[8 * d + 1];
    t += v1[0] * xv[8 * d + 2]; t += v1[1] * xv[8 * d + 3];
    t += v2[0] * xv[8 * d + 4]; t += v2[1] * xv[8 * d + 5];
    t += v3[0] * xv[8 * d + 6]; t += v3[1] * xv[8 * d + 7];
    b[d >> 1] = t;
  }
  if (MX) return b[0] + b[1];
  return b[0] * __builtin_amdgcn_cvt_f32_fp8((int)sc, 0) + b[1] * __builtin_amdgcn_cvt_f32_fp8((int)sc, 1);
}

// the scale(s) of 32-element chunk c at byte offset o of view v (o past the
// view: zeros): one e8m0 byte (MXFP4) or two e4m3 bytes (NVFP4)
template <int FMT>
__device__ __forceinline__ uint32_t sscale(__amdgpu_buffer_rsrc_t v, uint32_t o) {
  if (FMT == MOE_FMT_MXFP4) return __builtin_amdgcn_raw_buffer_load_b8(v, (int)o, 0, kCachePolicyNt);
  return __builtin_amdgcn_raw_buffer_load_b16(v, (int)o, 0, kCachePolicyNt);
}

// gate and up rows i0 .. i0+3 of shared expert blockIdx.y: the 256 threads
// split K into 32-element chunks (x in registers), every weight load is
// issued first, sums are reduced over the wave (DPP) and the four waves in
// order; h = silu(g) * u.
template <int FMT, int MAXCH>
__device__ __forceinline__ void sgu_block(const SArgs& a, int j, int i0) {
  constexpr int B = FMT == MOE_FMT_MXFP4 ? 32 : 16;
  __shared__ float s_part[4][2 * kSRowsGU];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int H = a.H, nch = H / 32;
  const uint8_t* rec = a.base + (size_t)j * a.stride;
  // rows i0 .. i0 + kSRowsGU - 1 of the gate and up codes and scales
  const uint32_t cbytes = (uint32_t)kSRowsGU * (H / 2), sbytes = (uint32_t)kSRowsGU * (H / B);
  const __amdgpu_buffer_rsrc_t cv[2] = {
      lview(rec + a.off[MOE_T_GATE_CODES] + (size_t)i0 * (H / 2), cbytes),
      lview(rec + a.off[MOE_T_UP_CODES] + (size_t)i0 * (H / 2), cbytes)};
  const __amdgpu_buffer_rsrc_t sv[2] = {
      lview(rec + a.off[MOE_T_GATE_SCALES] + (size_t)i0 * (H / B), sbytes),
      lview(rec + a.off[MOE_T_UP_SCALES] + (size_t)i0 * (H / B), sbytes)};
  uint4 q[MAXCH][kSRowsGU][2];
  uint32_t sc[MAXCH][kSRowsGU][2];
#pragma unroll
  for (int u = 0; u < MAXCH; ++u) {
    const int c = tid + 256 * u;
#pragma unroll
    for (int r = 0; r < kSRowsGU; ++r)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        q[u][r][m] = bload16(cv[m], c < nch ? (uint32_t)(r * (H / 2) + 16 * c) : kOutside);
        sc[u][r][m] = sscale<FMT>(sv[m], c < nch ? (uint32_t)(r * (H / B) + (32 / B) * c) : kOutside);
      }
  }
  float acc[kSRowsGU][2];
#pragma unroll
  for (int r = 0; r < kSRowsGU; ++r) { acc[r][0] = 0.0f; acc[r][1] = 0.0f; }
#pragma unroll
  for (int u = 0; u < MAXCH; ++u) {
    const int c = tid + 256 * u;
    if (c < nch) {
      float xv[32];
      const float4* xp = reinterpret_cast<const float4*>(a.x + 32 * c);
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const float4 f = xp[v];
        xv[4 * v] = f.x; xv[4 * v + 1] = f.y; xv[4 * v + 2] = f.z; xv[4 * v + 3] = f.w;
      }
#pragma unroll
      for (int r = 0; r < kSRowsGU; ++r)
#pragma unroll
        for (int m = 0; m < 2; ++m) acc[r][m] += sdot32<FMT>(q[u][r][m], sc[u][r][m], xv);
    }
  }
#pragma unroll
  for (int r = 0; r < kSRowsGU; ++r)
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const float v = wave_sum_dpp(acc[r][m]);
      if (lane == 0) s_part[wave][2 * r + m] = v;
    }
  __syncthreads();
  if (tid < kSRowsGU) {
    float gv = ((s_part[0][2 * tid] + s_part[1][2 * tid]) + s_part[2][2 * tid]) + s_part[3][2 * tid];
    float uv = ((s_part[0][2 * tid + 1] + s_part[1][2 * tid + 1]) + s_part[2][2 * tid + 1]) +
               s_part[3][2 * tid + 1];
    if (FMT == MOE_FMT_NVFP4) {
      const float* gl = reinterpret_cast<const float*>(rec + a.off[MOE_T_GLOBALS]);
      gv *= gl[0];
      uv *= gl[1];
    }
    a.h[(size_t)j * a.I + i0 + tid] = gv / (1.0f + expf(-gv)) * uv;
  }
}

// Shared-expert down rows n0 .. n0+RD-1: the threads split the concatenated
// K (every shared expert's I) into 32-element chunks; sdn_load issues the
// weight loads, sdn_dot the per-thread partial sums.
template <int RD, int MAXCH>
struct SdnW {
  uint4 q[MAXCH][RD];
  uint32_t sc[MAXCH][RD];
};

template <int FMT, int RD, int MAXCH>
__device__ __forceinline__ void sdn_load(const SArgs& a, int n0, SdnW<RD, MAXCH>& w) {
  constexpr int B = FMT == MOE_FMT_MXFP4 ? 32 : 16;
  const int tid = threadIdx.x, I = a.I, nchI = I / 32, ntot = a.ns * nchI;
  // the whole shared bank (ns * stride < 2^31 bytes, checked on the host)
  const __amdgpu_buffer_rsrc_t bv = lview(a.base, (uint32_t)(a.ns * a.stride));
#pragma unroll
  for (int u = 0; u < MAXCH; ++u) {
    const int cc = tid + 256 * u;
    const int j = cc < ntot ? cc / nchI : 0, c = cc < ntot ? cc - j * nchI : 0;
    const uint32_t rec = (uint32_t)(j * a.stride);
#pragma unroll
    for (int r = 0; r < RD; ++r) {
      const uint32_t row = (uint32_t)(n0 + r);
      w.q[u][r] = bload16(bv, cc < ntot ? rec + (uint32_t)a.off[MOE_T_DOWN_CODES] + row * (I / 2) + 16u * c
                                        : kOutside);
      w.sc[u][r] = sscale<FMT>(bv, cc < ntot ? rec + (uint32_t)a.off[MOE_T_DOWN_SCALES] + row * (I / B) +
                                                   (uint32_t)((32 / B) * c)
                                             : kOutside);
    }
  }
}

template <int FMT, int RD, int MAXCH>
__device__ __forceinline__ void sdn_dot(const SArgs& a, const SdnW<RD, MAXCH>& w, float (&acc)[RD]) {
  const int tid = threadIdx.x, I = a.I, nchI = I / 32, ntot = a.ns * nchI;
#pragma unroll
  for (int r = 0; r < RD; ++r) acc[r] = 0.0f;
#pragma unroll
  for (int u = 0; u < MAXCH; ++u) {
    const int cc = tid + 256 * u;
    if (cc < ntot) {
      const int j = cc / nchI, c = cc - j * nchI;
      float g = 1.0f;
      if (FMT == MOE_FMT_NVFP4)
        g = reinterpret_cast<const float*>(a.base + (size_t)j * a.stride + a.off[MOE_T_GLOBALS])[2];
      float hv[32];
      const float4* hp = reinterpret_cast<const float4*>(a.h + (size_t)j * I + 32 * c);
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const float4 f = hp[v];
        hv[4 * v] = f.x; hv[4 * v + 1] = f.y; hv[4 * v + 2] = f.z; hv[4 * v + 3] = f.w;
      }
#pragma unroll
      for (int r = 0; r < RD; ++r) acc[r] += g * sdot32<FMT>(w.q[u][r], w.sc[u][r], hv);
    }
  }
}

// ---------------------------------------------------------------------------
// One token: the dense mat-vecs and the shared experts in two launches.
// ---------------------------------------------------------------------------
// First: x_lat = W_down x (blocks 0 .. nA-1, kLatRowsA rows each) and the
// shared experts' gate/up with SwiGLU (the other blocks, kSRowsGU rows of one
// expert each).  Both read only x, so one launch streams both weight sets.
constexpr int kLatRowsA = 8;

template <int FMT, int MAXCH>
__global__ __launch_bounds__(256) void k_lat_in(GemvArgs g, SArgs s, int nA) {
  const int b = blockIdx.x;
  if (b < nA) {
    gemv_block<kLatRowsA, 1, 4, true>(g, b);
  } else {
    const int per = s.I / kSRowsGU, q = b - nA;
    sgu_block<FMT, MAXCH>(s, q / per, (q - (q / per) * per) * kSRowsGU);
  }
}

// Last: out rows n0 .. n0+7 = (sum over the shared experts of W_down h) +
// W_up (gamma * y_lat) / rms(y_lat), both in one workgroup: the shared
// experts' down weights are loaded first, then the W_up rows stream while
// those loads are in flight.  The sum is formed in the same order as the
// shared-down launch followed by the accumulating W_up launch.
template <int FMT, int MAXCH>
__global__ __launch_bounds__(256) void k_lat_out(GemvArgs g, SArgs s) {
  constexpr int RB = kSRowsDN;
  __shared__ float s_part[4][2 * RB + 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n0 = blockIdx.x * RB;
  SdnW<RB, MAXCH> w;
  sdn_load<FMT, RB, MAXCH>(s, n0, w);
  float acc[RB][1], ss[1];
  gemv_dot<RB, 1, 2, true>(g, n0, acc, ss);
  float sacc[RB];
  sdn_dot<FMT, RB, MAXCH>(s, w, sacc);
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const float v = wave_sum_dpp(acc[r][0]);
    const float u = wave_sum_dpp(sacc[r]);
    if (lane == 0) {
      s_part[wave][r] = v;
      s_part[wave][RB + r] = u;
    }
  }
  const float q = wave_sum_dpp(ss[0]);
  if (lane == 0) s_part[wave][2 * RB] = q;
  __syncthreads();
  if (tid < RB) {
    float v = ((s_part[0][tid] + s_part[1][tid]) + s_part[2][tid]) + s_part[3][tid];
    const float sq = ((s_part[0][2 * RB] + s_part[1][2 * RB]) + s_part[2][2 * RB]) + s_part[3][2 * RB];
    v *= 1.0f / sqrtf(sq / (float)g.K + g.eps);
    const float sh = ((s_part[0][RB + tid] + s_part[1][RB + tid]) + s_part[2][RB + tid]) +
                     s_part[3][RB + tid];
    g.y[n0 + tid] = sh + v;
  }
}

bool shared1_ok(const moe_bank* S, int H) {
  return S->hidden == H && H % 32 == 0 && S->inter % 32 == 0 && H / 32 <= 256 * kSMaxCh &&
         (int64_t)S->num_experts * S->expert_stride < ((int64_t)1 << 31) &&
         S->num_experts * (S->inter / 32) <= 256 * kSMaxCh && H % kSRowsDN == 0 &&
         S->inter % kSRowsGU == 0 && (S->format == MOE_FMT_MXFP4 || S->format == MOE_FMT_NVFP4);
}

SArgs shared_args(const moe_bank* S, const float* x, float* h) {
  SArgs a;
  a.base = static_cast<const uint8_t*>(S->base);
  a.stride = S->expert_stride;
  for (int t = 0; t < MOE_NUM_TENSORS; ++t) a.off[t] = S->offset[t];
  a.ns = S->num_experts; a.H = S->hidden; a.I = S->inter;
  a.x = x; a.h = h;
  return a;
}

// One token: routed_down (g) and the shared experts' gate/up into h.
// The instances hold the chunks per thread that K needs (one up to K = 8192).
moe_status launch_lat_in(const GemvArgs& g, const SArgs& s, int fmt, hipStream_t st) {
  const int nA = (g.N + kLatRowsA - 1) / kLatRowsA;
  const dim3 grid(nA + s.ns * (s.I / kSRowsGU));
  const bool one = s.H / 32 <= 256;
  if (fmt == MOE_FMT_MXFP4) {
    if (one) hipLaunchKernelGGL((k_lat_in<MOE_FMT_MXFP4, 1>), grid, dim3(256), 0, st, g, s, nA);
    else hipLaunchKernelGGL((k_lat_in<MOE_FMT_MXFP4, 2>), grid, dim3(256), 0, st, g, s, nA);
  } else {
    if (one) hipLaunchKernelGGL((k_lat_in<MOE_FMT_NVFP4, 1>), grid, dim3(256), 0, st, g, s, nA);
    else hipLaunchKernelGGL((k_lat_in<MOE_FMT_NVFP4, 2>), grid, dim3(256), 0, st, g, s, nA);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

// One token: out = shared experts' down sum + routed_up (g, with the norm).
moe_status launch_lat_out(const GemvArgs& g, const SArgs& s, int fmt, hipStream_t st) {
  const dim3 grid(g.N / kSRowsDN);
  const bool one = s.ns * (s.I / 32) <= 256;
  if (fmt == MOE_FMT_MXFP4) {
    if (one) hipLaunchKernelGGL((k_lat_out<MOE_FMT_MXFP4, 1>), grid, dim3(256), 0, st, g, s);
    else hipLaunchKernelGGL((k_lat_out<MOE_FMT_MXFP4, 2>), grid, dim3(256), 0, st, g, s);
  } else {
    if (one) hipLaunchKernelGGL((k_lat_out<MOE_FMT_NVFP4, 1>), grid, dim3(256), 0, st, g, s);
    else hipLaunchKernelGGL((k_lat_out<MOE_FMT_NVFP4, 2>), grid, dim3(256), 0, st, g, s);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

// Workspace of the latent layer: the routed experts', the router's and the
// shared experts' workspaces, x_lat, y_lat, the routed selection and the
// shared one.  The routed experts' region comes first, so that its error word
// (set should a bounded wait of the single-launch expert kernel expire) is the
// latent workspace's own, at byte offset 16.
struct LatentWs {
  size_t routed, route, shared, xlat, ylat, idx, w, sidx, sw, total;
};

bool latent_ok(const moe_latent_layer* p, int32_t k, int32_t C) {
  if (!p || !p->w_router || !p->w_down || !p->w_up || !p->norm_gamma) return false;
  const moe_bank& r = p->routed;
  const moe_bank& s = p->shared;
  const int H = p->hidden, L = r.hidden;
  if (C < 1 || C > MOE_MAX_DECODE_TOKENS || k < 1 || k > MOE_MAX_TOPK || k > r.num_experts) return false;
  if (H < 32 || H % 32 || L < 32 || L % 32 || s.hidden != H) return false;
  if (s.num_experts < 1 || s.num_experts > MOE_MAX_TOPK) return false;
  if (!(p->norm_eps >= 0.0f)) return false;
  return true;
}

LatentWs latent_ws(const moe_latent_layer* p, int32_t k, int32_t C) {
  LatentWs W;
  size_t o = 0;
  const moe_bank& r = p->routed;
  const moe_bank& s = p->shared;
  const int ns = s.num_experts;
  W.routed = o; o = align256(o + ws_layout(r.num_experts, r.hidden, r.inter, k, C).total);
  W.route = o;  o = align256(o + ws_layout(r.num_experts, p->hidden, 32, k, C).total);
  W.shared = o; o = align256(o + ws_layout(ns, s.hidden, s.inter, ns, C).total);
  W.xlat = o;   o = align256(o + (size_t)C * r.hidden * sizeof(float));
  W.ylat = o;   o = align256(o + (size_t)C * r.hidden * sizeof(float));
  W.idx = o;    o = align256(o + (size_t)C * k * sizeof(int32_t));
  W.w = o;      o = align256(o + (size_t)C * k * sizeof(float));
  W.sidx = o;   o = align256(o + (size_t)C * ns * sizeof(int32_t));
  W.sw = o;     o = align256(o + (size_t)C * ns * sizeof(float));
  W.total = o;
  return W;
}

}  // namespace
}  // namespace rf4

using namespace rf4;

extern "C" {

size_t moe_latent_workspace_size(const moe_latent_layer* layer, int32_t top_k, int32_t C) {
  if (!latent_ok(layer, top_k, C)) return 0;
  return latent_ws(layer, top_k, C).total;
}

moe_status moe_latent_layer_fwd(const moe_latent_layer* layer, const float* x, int32_t C, int32_t k,
                                float* out, int32_t* topk_idx_out, float* topk_w_out, void* ws,
                                size_t ws_bytes, void* stream) {
  if (!layer || !x || !out || x == out) return MOE_ERR_INVALID_ARG;
  if (!latent_ok(layer, k, C)) return MOE_ERR_UNSUPPORTED;
  if (!ws) return MOE_ERR_WORKSPACE;
  const LatentWs W = latent_ws(layer, k, C);
  if (ws_bytes < W.total || ((uintptr_t)ws % 256)) return MOE_ERR_WORKSPACE;
  if (((uintptr_t)x % 16) || ((uintptr_t)layer->w_down % 16) || ((uintptr_t)layer->w_up % 16) ||
      ((uintptr_t)layer->norm_gamma % 16))
    return MOE_ERR_INVALID_ARG;
  const moe_bank& R = layer->routed;
  const moe_bank& S = layer->shared;
  const int H = layer->hidden, L = R.hidden, ns = S.num_experts;
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  uint8_t* wr = w8 + W.routed;
  int32_t* idx = topk_idx_out ? topk_idx_out : reinterpret_cast<int32_t*>(w8 + W.idx);
  float* w = topk_w_out ? topk_w_out : reinterpret_cast<float*>(w8 + W.w);
  float* xlat = reinterpret_cast<float*>(w8 + W.xlat);
  float* ylat = reinterpret_cast<float*>(w8 + W.ylat);
  int32_t* sidx = reinterpret_cast<int32_t*>(w8 + W.sidx);
  float* sw = reinterpret_cast<float*>(w8 + W.sw);
  const size_t wr_bytes = W.route - W.routed, wq_bytes = W.shared - W.route,
               ws_bytes_s = W.xlat - W.shared;

  // partial phase: routed_down, then the router on x and the routed experts
  // on x_lat (one launch for one token where the bank's shape is built for
  // the single-launch kernel, else the router and the expert path apart)
  GemvArgs g;
  g.W = layer->w_down; g.x = x; g.gamma = nullptr; g.eps = 0.0f; g.y = xlat;
  g.C = C; g.N = L; g.K = H; g.accumulate = 0;
  g.sel_idx = sidx; g.sel_w = sw; g.ns = ns;     // the shared experts' selection
  // and, where the decode-batch streams take the shared bank, its dispatch
  // table (every token, every shared expert), so no dispatch launch is needed
  // (the one-token launches take W_down and W_up in one slab each: H <= 8192
  // and L <= 4096)
  const bool shared_one = C == 1 && bank_status(&S) == MOE_OK && shared1_ok(&S, H) &&
                          H / 8 <= kGemvWG * 4 && L / 8 <= kGemvWG * 2;
  const bool shared_streams =
      !shared_one && bank_status(&S) == MOE_OK && batched_decode_shape(&S, C);
  const WsLayout Ls = ws_layout(ns, S.hidden, S.inter, ns, C);
  g.sel_disp = shared_streams ? reinterpret_cast<int32_t*>(w8 + W.shared + Ls.disp) : nullptr;
  float* sh = reinterpret_cast<float*>(w8 + W.shared + Ls.h);
  const SArgs sa = shared_args(&S, x, sh);
  moe_status s = shared_one ? launch_lat_in(g, sa, S.format, st) : launch_gemv(g, st);
  if (s != MOE_OK) return s;
  s = C == 1 ? layer1_router_input(&R, layer->w_router, x, H, xlat, k, ylat, idx, w, wr, wr_bytes, st)
             : MOE_ERR_UNSUPPORTED;
  if (s == MOE_ERR_UNSUPPORTED) {
    s = moe_route(x, layer->w_router, nullptr, C, H, R.num_experts, k, idx, w, w8 + W.route,
                  wq_bytes, stream);
    if (s != MOE_OK) return s;
    s = moe_expert_fwd(&R, xlat, C, k, idx, w, ylat, wr, wr_bytes, stream);
  }
  if (s != MOE_OK) return s;
  // finish phase: shared experts into out, then routed_norm and routed_up
  // added (one launch for one token)
  g.W = layer->w_up; g.x = ylat; g.gamma = layer->norm_gamma; g.eps = layer->norm_eps; g.y = out;
  g.C = C; g.N = H; g.K = L; g.accumulate = 1;
  g.sel_idx = nullptr; g.sel_w = nullptr; g.sel_disp = nullptr; g.ns = 0;
  if (shared_one) return launch_lat_out(g, sa, S.format, st);
  s = shared_streams ? launch_batched_decode(&S, x, C, ns, sidx, sw, out, w8 + W.shared, Ls, st)
                     : moe_expert_fwd(&S, x, C, ns, sidx, sw, out, w8 + W.shared, ws_bytes_s, stream);
  if (s != MOE_OK) return s;
  return launch_gemv(g, st);
}

}  // extern "C"
