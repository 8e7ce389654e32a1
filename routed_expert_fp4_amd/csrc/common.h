// Internal header of libroutedfp4: workspace layout, device helpers and the
// selection routine shared by the decode kernels (routed_fp4.hip) and the
// batched grouped-GEMM path (batched.hip).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "routed_fp4.h"

namespace rf4 {

constexpr int kWG = 256;           // threads per workgroup (4 waves of 64)
constexpr int kKsplitMax = 4;      // router split-K factor limit
constexpr int kGuRows = 16;        // gate/up: I rows per item (one per lane group)
constexpr int kDnRowsPerGroup = 4; // down: rows per 16-lane group
constexpr int kDnRows = 16 * kDnRowsPerGroup;  // down: H rows per item
constexpr int kXsFloats = 10240;   // LDS floats for staged activations (40 KiB)
constexpr int kRouteXs = 8192;     // LDS floats for the router's x tile (32 KiB)
constexpr int kLogitCopies = 16;   // batch-1 kernel: replicas of the tagged logits

// ---------------------------------------------------------------------------
// Workspace layout
// ---------------------------------------------------------------------------
struct WsLayout {
  size_t ctrl, dtick, lpart, logits, idx, w, disp, h, part, tlogits, th, tpart;
  // batched path: per-expert counts, cursors and offsets, the tile list, the
  // (token, slot) pairs grouped by expert, x as three bf16 planes, h as two
  size_t bcount, bcursor, boff, bmeta, btile, perm, xp, xflag, hp;
  size_t total;
};

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Tokens per tile of the batched path: 16 up to kBatchWideC tokens, else 64.
constexpr int kBatchWideC = 64;
inline int batch_ntok(int C) { return C <= kBatchWideC ? 16 : 64; }
// Upper bound on the batched path's tiles: every expert's last tile may be
// partial, all others are full.
inline size_t batch_max_tiles(int E, int k, int C) {
  const size_t CK = (size_t)C * k;
  return CK / (size_t)batch_ntok(C) + (CK < (size_t)E ? CK : (size_t)E);
}

inline WsLayout ws_layout(int E, int H, int I, int k, int C) {
  WsLayout L;
  size_t o = 0;
  const size_t CK = (size_t)C * k;
  const bool decode = C <= MOE_MAX_DECODE_TOKENS;   // the split-K router path
  L.ctrl = o;   o = align256(o + (64 + 256) * sizeof(uint32_t));   // control words, arrival words
  L.dtick = o;  o = align256(o + (size_t)((H + kDnRows - 1) / kDnRows) * sizeof(uint32_t));
  L.lpart = o;  o = align256(o + (decode ? (size_t)kKsplitMax * C * E * sizeof(float) : 0));
  L.logits = o; o = align256(o + (size_t)C * E * sizeof(float));
  L.idx = o;    o = align256(o + CK * sizeof(int32_t));
  L.w = o;      o = align256(o + CK * sizeof(float));
  L.disp = o;   o = align256(o + (decode ? (16 + 2 * CK + CK * C) * sizeof(int32_t) : 0));
  L.h = o;      o = align256(o + (decode ? CK * I * sizeof(float) : 0));
  L.part = o;   o = align256(o + CK * H * sizeof(float));
  // batch-1 kernel: (epoch, value) words
  L.tlogits = o; o = align256(o + (size_t)kLogitCopies * 2 * E * sizeof(uint64_t));
  L.th = o;      o = align256(o + 2 * (size_t)k * I * sizeof(uint64_t));   // XCD copy, coherent copy
  L.tpart = o;   o = align256(o + (size_t)k * H * sizeof(uint64_t));
  // batched path
  L.bcount = o;  o = align256(o + (size_t)E * sizeof(uint32_t));
  L.bcursor = o; o = align256(o + (size_t)E * sizeof(uint32_t));
  L.boff = o;    o = align256(o + (size_t)(E + 1) * sizeof(uint32_t));
  L.bmeta = o;   o = align256(o + 32 * sizeof(uint32_t));   // tile count, item counter
  L.btile = o;   o = align256(o + batch_max_tiles(E, k, C) * 2 * sizeof(int32_t));
  L.perm = o;    o = align256(o + CK * sizeof(int32_t));
  L.xp = o;      o = align256(o + 3 * (size_t)C * H * sizeof(uint16_t));
  L.xflag = o;   o = align256(o + (size_t)C * sizeof(uint32_t));
  L.hp = o;      o = align256(o + 2 * CK * I * sizeof(uint16_t));
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
  // OCP fp8 e4m3 ("FN": bias 7, no infinities, S.1111.111 is NaN), decoded by
  // the hardware conversion of the low byte.
  return __builtin_amdgcn_cvt_f32_fp8((int)(b & 0xFFu), 0);
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

// Cross-workgroup hand-off without cache-maintenance fences.  An agent-scope
// fence on gfx950 writes back and invalidates the XCD's L2 (about a
// microsecond, serialised per XCD), so the kernels never use one.  Instead the
// data one workgroup hands to another is written with agent-coherent stores
// (sc1), each producer waits for its stores to complete before it takes a
// ticket with a relaxed device-scope atomic, and the consumer that draws the
// last ticket reads the data with agent-coherent loads.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Bulk coherent reads go through buffer loads with the sc1 cache-policy bit:
// unlike atomic loads they are not serialised one round trip at a time.
// (Buffer resource word 3 for gfx9-family raw buffers; out-of-range offsets
// read zero.)
constexpr int kCachePolicySc1 = 16;
constexpr int kCachePolicyNt = 2;   // non-temporal: weights are read once per call
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_view(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ float coherent_ld(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)byte_off, 0, kCachePolicySc1));
}
// All of this workgroup's stores are complete, then one ticket; returns true
// (in every thread) for the workgroup that drew ticket n-1.
__device__ __forceinline__ bool last_to_arrive(uint32_t* ticket, uint32_t n, int* s_flag) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    *s_flag = (__hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               n - 1u) ? 1 : 0;
  __syncthreads();
  return *s_flag != 0;
}
__device__ __forceinline__ void reset_ticket(uint32_t* ticket) {
  __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

struct SelectLds {                 // one wave's selection scratch in LDS
  uint64_t cand_key[64];
  float cand_l[64];
  int32_t sel_e[MOE_MAX_TOPK];     // the selection in rank order
  float sel_l[MOE_MAX_TOPK];
};

// Selection key of expert e with logit l: larger is better; equal logits go
// to the lower index; 0 marks an empty entry (every real key is above it).
__device__ __forceinline__ uint64_t sel_key(float l, int e) {
  return ((uint64_t)logit_key(l) << 32) | (uint64_t)(~(uint32_t)e);
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m, 64);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}

// Orders LDS accesses of one wave (a compiler fence only: a wave's LDS
// operations complete in issue order).
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Exact top-k of the entries one wave holds, NPL per lane (key ck[i], logit
// lv[i]; empty entries have key 0), k <= 32 and at least k entries non-empty.
// Writes the winners' experts and logits, best first, to S.sel_e / S.sel_l
// (S is this wave's own LDS block).
//
// A threshold first: T = the k-th largest of the 64 lane maxima.  The k lanes
// whose maxima are >= T hold k entries >= T, so the top k are all >= T.  The
// entries >= T (usually a few more than k) are gathered one per lane, and each
// one's rank is the number of gathered keys above it.  When more than 64
// entries pass the threshold (heavily clustered winners), k rounds of "take
// the wave's best remaining entry" do the job instead.
template <int NPL>
__device__ void wave_select(uint64_t (&ck)[NPL], const float (&lv)[NPL], int k, SelectLds& S) {
  const int lane = threadIdx.x & 63;
  uint64_t m = 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i) m = ck[i] > m ? ck[i] : m;
  int r = 0;                                   // rank of this lane's maximum
  for (int j = 0; j < 64; ++j) r += readlane_u64(m, j) > m ? 1 : 0;
  // non-empty maxima are distinct, so exactly one lane has rank k - 1
  const unsigned long long at = __ballot(r == k - 1);
  const uint64_t T = at ? readlane_u64(m, __ffsll((long long)at) - 1) : 0;
  int n = 0;
  unsigned long long pass[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    pass[i] = __ballot(ck[i] >= T && ck[i] != 0);
    n += __popcll(pass[i]);
  }
  if (n <= 64) {
    int base = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      if ((pass[i] >> lane) & 1ull) {
        const int pos = base + __popcll(pass[i] & ((1ull << lane) - 1ull));
        S.cand_key[pos] = ck[i];
        S.cand_l[pos] = lv[i];
      }
      base += __popcll(pass[i]);
    }
    wave_lds_fence();
    const uint64_t mine = lane < n ? S.cand_key[lane] : 0;
    const float ml = lane < n ? S.cand_l[lane] : 0.0f;
    int rk = 0;
    for (int j = 0; j < n; ++j) rk += readlane_u64(mine, j) > mine ? 1 : 0;
    if (lane < n && rk < k) {
      S.sel_e[rk] = (int32_t)~(uint32_t)mine;
      S.sel_l[rk] = ml;
    }
  } else {
    for (int s = 0; s < k; ++s) {
      uint64_t b = 0;
#pragma unroll
      for (int i = 0; i < NPL; ++i) b = ck[i] > b ? ck[i] : b;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint64_t o = shfl_xor_u64(b, d);
        b = o > b ? o : b;
      }
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        if (b != 0 && ck[i] == b) {          // one entry of one lane
          S.sel_e[s] = (int32_t)~(uint32_t)b;
          S.sel_l[s] = lv[i];
          ck[i] = 0;
        }
      }
    }
  }
  wave_lds_fence();
}

// sigmoid(l_s) / sum over the k of sigmoid(l), for lane s < k of a wave
// (the same value in every lane's sum: the butterfly adds pairs commutatively).
__device__ __forceinline__ float route_weight(float l, int lane, int k) {
  const float sg = (lane < k) ? 1.0f / (1.0f + expf(-l)) : 0.0f;
  return sg / wave_sum(sg);
}

// Shapes the batched path is built for: K stages of 256 elements taken in
// pairs, row tiles of 128 (gate/up) and 256 (down) rows, scale tensors at
// 4-byte aligned offsets (their words are loaded whole).
inline bool batched_shape_ok(const moe_bank* b) {
  if (b->hidden % 512 || b->inter % 512) return false;
  for (int t = MOE_T_GATE_SCALES; t <= MOE_T_DOWN_SCALES; ++t)
    if (b->offset[t] % 4) return false;
  return true;
}

// Host side of the batched path (batched.hip).  Both enqueue on `st` only.
// launch_batched_route: logits (x * W_r^T on the matrix cores, or the
// caller's logits when x is null) and the per-token top-k, for any C.
moe_status launch_batched_route(const float* x, const float* Wr, const float* logits_in,
                                float* logits_out, int C, int H, int E, int k, int32_t* idx,
                                float* w, uint8_t* ws, const WsLayout& L, hipStream_t st);
// launch_topk_parts: the top-k of C tokens (one wave each) from ksplit
// partial router sums lpart[s][t][e], added in split order; the logits go to
// logits_out too when it is not null, and the dispatch table to disp when it
// is not null (C <= MOE_MAX_DECODE_TOKENS).
moe_status launch_topk_parts(const float* lpart, int ksplit, float* logits_out, int C, int E, int k,
                             int32_t* idx, float* w, int32_t* disp, hipStream_t st);
// launch_batched_experts: the selected experts of C tokens as grouped GEMMs
// on the matrix cores, then the fixed-order combine into out.
moe_status launch_batched_experts(const moe_bank* b, const float* x, int C, int k,
                                  const int32_t* idx, const float* w, float* out, uint8_t* ws,
                                  const WsLayout& L, hipStream_t st);
// launch_batched_decode: C <= MOE_MAX_DECODE_TOKENS tokens whose distinct
// experts are listed in the workspace's dispatch table: each distinct expert
// streamed once (gate/up with SwiGLU, then down), then the fixed-order
// combine into out.  batched_decode_shape says which shapes it takes.
bool batched_decode_shape(const moe_bank* b, int C);
moe_status launch_batched_decode(const moe_bank* b, const float* x, int C, int k,
                                 const int32_t* idx, const float* w, float* out, uint8_t* ws,
                                 const WsLayout& L, hipStream_t st);
// layer1_router_input: one token through a layer whose router reads an input
// of its own, xr [Hr] against w_router [E][Hr], while the experts take x [H]
// (a latent layer: routed on the hidden state, experts in the latent width).
// The single-launch kernel when the bank's shape is built for it; otherwise
// MOE_ERR_UNSUPPORTED with nothing enqueued.  ws is the bank's workspace
// (ws_layout(E, H, I, k, 1)).
moe_status layer1_router_input(const moe_bank* b, const float* w_router, const float* xr, int Hr,
                               const float* x, int k, float* out, int32_t* idx, float* w,
                               void* ws, size_t ws_bytes, hipStream_t st);
// bank_status: the checks every expert entry point makes of a bank (format,
// sizes, alignment, tensor offsets within the stride).
moe_status bank_status(const moe_bank* b);

}  // namespace rf4
