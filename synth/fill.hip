// Device-side fill of a synthetic expert bank.
//
// Input generation only (none of the method's arithmetic).  Every byte is the
// same pure function of (seed, layer, expert, tensor, index) that
// synth/__init__.py evaluates on the host: the SplitMix64 output function
// (Steele, Lea, Flood, OOPSLA 2014) applied to key + (i+1)*GAMMA, where the key
// chains the same mixing over seed, layer, expert and tensor id.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t GAMMA = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t stream_key(uint64_t seed, uint64_t layer,
                                               uint64_t expert, uint64_t tensor) {
  uint64_t k = mix64(seed + GAMMA);
  k = mix64(k ^ (layer + GAMMA));
  k = mix64(k ^ (expert + 2 * GAMMA));
  k = mix64(k ^ (tensor + 3 * GAMMA));
  return k;
}

// kind 0: code bytes (one word -> 8 bytes); 1: MX scale bytes; 2: NV scale
// bytes (one word -> 1 byte, 8 bytes per thread); 3: NV fp32 globals.
__global__ void fill_kernel(uint8_t* base, int64_t stride, int64_t offset,
                            int64_t nbytes, int kind, int tensor, uint64_t seed,
                            int layer, int expert0) {
  const int64_t e = (int64_t)blockIdx.y + expert0;
  const uint64_t key = stream_key(seed, (uint64_t)layer, (uint64_t)e, (uint64_t)tensor);
  uint8_t* dst = base + e * stride + offset;
  const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
  if (kind == 3) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < 3) {
      const uint64_t w = mix64(key + (uint64_t)(i + 1) * GAMMA);
      const float g = 1.0f + (float)(w >> 41) * 0x1p-23f;   // exact: 23-bit mantissa
      reinterpret_cast<float*>(dst)[i] = g;
    }
    return;
  }
  const int64_t nwords = nbytes / 8;   // callers guarantee nbytes % 8 == 0
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords; i += nthreads) {
    uint64_t out;
    if (kind == 0) {
      out = mix64(key + (uint64_t)(i + 1) * GAMMA);
    } else {
      out = 0;
      for (int b = 0; b < 8; ++b) {
        const uint64_t j = (uint64_t)(i * 8 + b);
        const uint64_t w = mix64(key + (j + 1) * GAMMA);
        const uint64_t v = (kind == 1) ? (127u - (w % 5u)) : (0x18u + (w % 32u));
        out |= v << (8 * b);
      }
    }
    reinterpret_cast<uint64_t*>(dst)[i] = out;
  }
}

// The bench's read-bandwidth calibration (not part of the method): every
// thread reads 16-byte words of [p, p + n16 * 16) with non-temporal loads, in
// a grid-stride walk (consecutive lanes, consecutive words; four words in
// flight per thread), and folds them into one word per workgroup so that no
// load can be dropped.
__global__ __launch_bounds__(256) void read_kernel(const uint4* p, int64_t n16, uint32_t* sink) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  uint32_t acc = 0;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * step < n16; i += 4 * step) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + i + u * step));
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += step) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + i));
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
    for (int t = 0; t < 256; ++t) a ^= red[t];
    sink[blockIdx.x] = a;
  }
}

}  // namespace

extern "C" {

// Streaming read of nbytes (a multiple of 16, 16-byte aligned) at device
// address p with `blocks` workgroups of 256 threads; sink holds `blocks`
// words.  Returns 0 or the HIP error code of the launch.
int synth_stream_read(const void* p, int64_t nbytes, int32_t blocks, uint32_t* sink, void* stream) {
  if (!p || !sink || nbytes <= 0 || nbytes % 16 || (uintptr_t)p % 16 || blocks < 1) return -1;
  hipLaunchKernelGGL(read_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const uint4*>(p),
                     nbytes / 16, sink);
  hipError_t err = hipGetLastError();
  return err == hipSuccess ? 0 : (int)err;
}

// Fill tensor `tensor` (0..6, the ids of synth/__init__.py) of experts
// [0, num_experts) of a bank at `base` (device memory): expert e's tensor starts
// at base + e*expert_stride + tensor_offset and holds `nbytes` bytes.
// fmt: 1 = MX (e8m0 scales), 2 = NV (e4m3 scales + fp32 globals).
// Returns 0, or -1 for bad arguments, or the HIP error code of the launch.
int synth_fill_tensor(void* base, int64_t expert_stride, int32_t num_experts,
                      int64_t tensor_offset, int64_t nbytes, int32_t tensor,
                      int32_t fmt, uint64_t seed, int32_t layer, void* stream) {
  if (!base || num_experts < 1 || tensor < 0 || tensor > 6 || tensor_offset < 0 ||
      expert_stride < tensor_offset + nbytes)
    return -1;
  int kind;
  if (tensor <= 2) kind = 0;
  else if (tensor <= 5) kind = (fmt == 1) ? 1 : 2;
  else {
    if (fmt != 2) return 0;   // MX banks have no globals
    kind = 3;
  }
  if (kind != 3 && (nbytes % 8 != 0 || tensor_offset % 8 != 0 || expert_stride % 8 != 0))
    return -1;
  if (kind == 3 && (tensor_offset % 4 != 0 || nbytes < 12)) return -1;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t nwords = kind == 3 ? 1 : nbytes / 8;
  int64_t gx = (nwords + 255) / 256;
  if (gx > 1024) gx = 1024;
  // blockIdx.y is limited to 65535: fill experts in slices
  for (int32_t e0 = 0; e0 < num_experts; e0 += 65535) {
    const int32_t ne = (num_experts - e0 < 65535) ? (num_experts - e0) : 65535;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)gx, (unsigned)ne), dim3(256), 0, s,
                       static_cast<uint8_t*>(base), expert_stride, tensor_offset, nbytes,
                       kind, tensor, seed, layer, e0);
  }
  hipError_t err = hipGetLastError();
  return err == hipSuccess ? 0 : (int)err;
}

}  // extern "C"
