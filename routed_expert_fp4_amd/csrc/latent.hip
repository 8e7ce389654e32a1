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
//               1 / rms(x[t]), else s_t = 1 and g = 1
//   k_shared_sel the shared experts' selection: every token, every shared
//               expert, weight 1
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
};

constexpr int kGemvRows = 2;             // output rows per wave
constexpr int kGemvWG = 256;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Each wave takes kGemvRows rows for every token; a lane reads 16 bytes (8
// weights) of a row at a time, rows along K, and the x tile of the current K
// chunk (all tokens) sits in LDS.  With the norm, every workgroup first sums
// each token's squares over all of K (wave t % 4 takes token t), and gamma is
// applied to x as it is staged; 1 / rms multiplies the finished dot product.
template <int CM>
__global__ __launch_bounds__(kGemvWG) void k_gemv(GemvArgs a) {
  constexpr int KT = kRouteXs / CM;                   // staged floats per token per chunk
  __shared__ float xs[kRouteXs];
  __shared__ float s_rs[CM];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int C = a.C, K = a.K, N = a.N;
  const int n0 = (blockIdx.x * (kGemvWG / 64) + wave) * kGemvRows;

  if (a.gamma) {
    for (int t = wave; t < C; t += kGemvWG / 64) {
      float ss = 0.0f;
      for (int i = lane * 4; i < K; i += 64 * 4) {
        const float4 v = *reinterpret_cast<const float4*>(a.x + (size_t)t * K + i);
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
      }
      ss = wave_sum(ss);
      if (lane == 0) s_rs[t] = 1.0f / sqrtf(ss / (float)K + a.eps);
    }
  }

  float acc[kGemvRows][CM];
#pragma unroll
  for (int r = 0; r < kGemvRows; ++r)
#pragma unroll
    for (int t = 0; t < CM; ++t) acc[r][t] = 0.0f;

  for (int kt = 0; kt < K; kt += KT) {
    const int kn = min(KT, K - kt);
    __syncthreads();
    for (int i = tid * 4; i < C * kn; i += kGemvWG * 4) {
      const int t = i / kn, col = i - t * kn;
      float4 v = *reinterpret_cast<const float4*>(a.x + (size_t)t * K + kt + col);
      if (a.gamma) {
        const float4 g = *reinterpret_cast<const float4*>(a.gamma + kt + col);
        v.x *= g.x; v.y *= g.y; v.z *= g.z; v.w *= g.w;
      }
      *reinterpret_cast<float4*>(&xs[t * KT + col]) = v;
    }
    __syncthreads();
    const int n8 = kn >> 3;                           // 16-byte chunks of a row in this K chunk
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) {
      const int n = n0 + r;
      if (n >= N) break;
      const uint4* wrow = reinterpret_cast<const uint4*>(a.W + (size_t)n * K + kt);
      for (int c = lane; c < n8; c += 64) {
        const uint4 wq = wrow[c];
        const float w0 = bf16_lo(wq.x), w1 = bf16_hi(wq.x), w2 = bf16_lo(wq.y), w3 = bf16_hi(wq.y);
        const float w4 = bf16_lo(wq.z), w5 = bf16_hi(wq.z), w6 = bf16_lo(wq.w), w7 = bf16_hi(wq.w);
#pragma unroll
        for (int t = 0; t < CM; ++t) {
          if (t >= C) break;
          const float4 xa = *reinterpret_cast<const float4*>(&xs[t * KT + 8 * c]);
          const float4 xb = *reinterpret_cast<const float4*>(&xs[t * KT + 8 * c + 4]);
          float s = acc[r][t];
          s += w0 * xa.x; s += w1 * xa.y; s += w2 * xa.z; s += w3 * xa.w;
          s += w4 * xb.x; s += w5 * xb.y; s += w6 * xb.z; s += w7 * xb.w;
          acc[r][t] = s;
        }
      }
    }
  }

#pragma unroll
  for (int r = 0; r < kGemvRows; ++r) {
    const int n = n0 + r;
#pragma unroll
    for (int t = 0; t < CM; ++t) {
      if (t >= C) break;
      const float v = wave_sum(acc[r][t]);
      if (lane == 0 && n < N) {
        const float s = a.gamma ? s_rs[t] * v : v;
        float* yp = a.y + (size_t)t * N + n;
        *yp = a.accumulate ? *yp + s : s;
      }
    }
  }
}

__global__ void k_shared_sel(int32_t* idx, float* w, int C, int ns) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < C * ns) {
    idx[i] = i % ns;
    w[i] = 1.0f;
  }
}

moe_status launch_gemv(const GemvArgs& a, hipStream_t st) {
  const int waves = (a.N + kGemvRows - 1) / kGemvRows;
  const int grid = (waves + kGemvWG / 64 - 1) / (kGemvWG / 64);
  if (a.C <= 1) hipLaunchKernelGGL(k_gemv<1>, dim3(grid), dim3(kGemvWG), 0, st, a);
  else if (a.C <= 4) hipLaunchKernelGGL(k_gemv<4>, dim3(grid), dim3(kGemvWG), 0, st, a);
  else hipLaunchKernelGGL(k_gemv<16>, dim3(grid), dim3(kGemvWG), 0, st, a);
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

  // partial phase: router on x, routed_down, routed experts
  moe_status s = moe_route(x, layer->w_router, nullptr, C, H, R.num_experts, k, idx, w, w8 + W.route,
                           wq_bytes, stream);
  if (s != MOE_OK) return s;
  GemvArgs g;
  g.W = layer->w_down; g.x = x; g.gamma = nullptr; g.eps = 0.0f; g.y = xlat;
  g.C = C; g.N = L; g.K = H; g.accumulate = 0;
  if ((s = launch_gemv(g, st)) != MOE_OK) return s;
  s = moe_expert_fwd(&R, xlat, C, k, idx, w, ylat, wr, wr_bytes, stream);
  if (s != MOE_OK) return s;
  // finish phase: shared experts into out, then routed_norm and routed_up added
  hipLaunchKernelGGL(k_shared_sel, dim3((C * ns + 255) / 256), dim3(256), 0, st, sidx, sw, C, ns);
  s = moe_expert_fwd(&S, x, C, ns, sidx, sw, out, w8 + W.shared, ws_bytes_s, stream);
  if (s != MOE_OK) return s;
  g.W = layer->w_up; g.x = ylat; g.gamma = layer->norm_gamma; g.eps = layer->norm_eps; g.y = out;
  g.C = C; g.N = H; g.K = L; g.accumulate = 1;
  return launch_gemv(g, st);
}

}  // extern "C"
