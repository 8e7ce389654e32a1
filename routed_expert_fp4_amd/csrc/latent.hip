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

// RB rows per workgroup, the whole K: the 256 threads split each row into
// 16-byte chunks (8 bf16), NCH chunks per thread per slab of 2048 * NCH
// elements; every weight load of a slab is issued before any arithmetic, and x
// (with gamma applied) comes straight from L2 into registers for each chunk, in
// groups of up to 4 tokens.  With the norm, the same x values give each
// token's sum of squares over K.  The per-thread partial sums are reduced over
// the wave (DPP) and then over the four waves in order.
template <int RB, int CM, int NCH>
__global__ __launch_bounds__(kGemvWG) void k_gemv(GemvArgs a) {
  constexpr int TG = CM < 4 ? CM : 4;                 // tokens per x group
  __shared__ float s_part[kGemvWG / 64][RB * CM + CM];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int C = a.C, K = a.K, N = a.N, K8 = K >> 3;
  const int n0 = blockIdx.x * RB;
  const bool norm = a.gamma != nullptr;

  if (a.sel_idx && blockIdx.x == 0) {
    const int ns = a.ns, CK = C * ns;
    for (int i = tid; i < CK; i += kGemvWG) {
      a.sel_idx[i] = i % ns;
      a.sel_w[i] = 1.0f;
    }
    if (a.sel_disp) {
      // distinct experts in order of first use (0 .. ns-1), each with every
      // token's pair t * ns + u in token order
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

  float acc[RB][CM], ss[CM];
#pragma unroll
  for (int t = 0; t < CM; ++t) {
    ss[t] = 0.0f;
#pragma unroll
    for (int r = 0; r < RB; ++r) acc[r][t] = 0.0f;
  }

  for (int c0 = 0; c0 < K8; c0 += kGemvWG * NCH) {
    uint4 wq[RB][NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = c0 + tid + kGemvWG * j;
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const int n = n0 + r;
        wq[r][j] = (c < K8 && n < N)
                       ? reinterpret_cast<const uint4*>(a.W + (size_t)n * K)[c]
                       : make_uint4(0u, 0u, 0u, 0u);
      }
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
  const bool shared_streams = bank_status(&S) == MOE_OK && batched_decode_shape(&S, C);
  const WsLayout Ls = ws_layout(ns, S.hidden, S.inter, ns, C);
  g.sel_disp = shared_streams ? reinterpret_cast<int32_t*>(w8 + W.shared + Ls.disp) : nullptr;
  moe_status s = launch_gemv(g, st);
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
  // finish phase: shared experts into out, then routed_norm and routed_up added
  s = shared_streams
          ? launch_batched_decode(&S, x, C, ns, sidx, sw, out, w8 + W.shared, Ls, st)
          : moe_expert_fwd(&S, x, C, ns, sidx, sw, out, w8 + W.shared, ws_bytes_s, stream);
  if (s != MOE_OK) return s;
  g.W = layer->w_up; g.x = ylat; g.gamma = layer->norm_gamma; g.eps = layer->norm_eps; g.y = out;
  g.C = C; g.N = H; g.K = L; g.accumulate = 1;
  g.sel_idx = nullptr; g.sel_w = nullptr; g.sel_disp = nullptr; g.ns = 0;
  return launch_gemv(g, st);
}

}  // extern "C"
