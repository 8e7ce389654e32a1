// Test probes of two matrix-core instructions, one wave per call (in-bounds:
// call c reads and writes only its own 64-lane slice).  TEST INFRASTRUCTURE:
// used by tests/test_gpu_fp4_mfma_model.py to measure how the instructions
// round; the library does not use this file.
//   probe_mfma_f32: v_mfma_f32_16x16x4f32, per call a[64], b[64] fp32 and the
//     accumulator c[64][4] -> d[64][4] (lane l: A row l%16 col l/16, B row
//     l/16 col l%16, D rows 4(l/16)..+3 of col l%16).
//   probe_mfma_fp4: v_mfma_scale_f32_16x16x128_f8f6f4 with an e2m1 A and an
//     e4m3 B, per call a[64][16] and b[64][32] bytes, one scale byte per lane
//     for each, c[64][4] -> d[64][4].
//   probe_cvt_fp4_bf16: v_cvt_scalef32_pk_bf16_fp4, per element a dword of 8
//     e2m1 codes and an fp32 scale -> 8 bf16 (element i reads words[i] and
//     scales[i], writes out[8i..8i+7]; threads past n do nothing).
//   probe_mfma_4x4_bf16: v_mfma_f32_4x4x4_16b_bf16, per call and lane 4 bf16
//     of A, 4 bf16 of B and 4 fp32 of the accumulator -> 4 fp32 (lane l of
//     call c reads and writes element c * 64 + l of each array).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float v4f_t __attribute__((ext_vector_type(4)));
typedef int v8i_t __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(64) void k_probe_f32(const float* a, const float* b, const float* c, float* d) {
  const size_t i = (size_t)blockIdx.x * 64 + threadIdx.x;
  v4f_t acc = {c[4 * i], c[4 * i + 1], c[4 * i + 2], c[4 * i + 3]};
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], acc, 0, 0, 0);
  for (int j = 0; j < 4; ++j) d[4 * i + j] = acc[j];
}

__global__ __launch_bounds__(64) void k_probe_fp4(const uint32_t* a, const uint32_t* b, const uint8_t* sa,
                                                  const uint8_t* sb, const float* c, float* d) {
  const size_t i = (size_t)blockIdx.x * 64 + threadIdx.x;
  const v8i_t A = {(int)a[4 * i], (int)a[4 * i + 1], (int)a[4 * i + 2], (int)a[4 * i + 3], 0, 0, 0, 0};
  const v8i_t B = {(int)b[8 * i], (int)b[8 * i + 1], (int)b[8 * i + 2], (int)b[8 * i + 3],
                   (int)b[8 * i + 4], (int)b[8 * i + 5], (int)b[8 * i + 6], (int)b[8 * i + 7]};
  v4f_t acc = {c[4 * i], c[4 * i + 1], c[4 * i + 2], c[4 * i + 3]};
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc, 4, 0, 0, (int)sa[i], 0, (int)sb[i]);
  for (int j = 0; j < 4; ++j) d[4 * i + j] = acc[j];
}

typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));

__global__ __launch_bounds__(256) void k_probe_cvt(const uint32_t* words, const float* scales, uint16_t* out,
                                                   int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const uint32_t w = words[i];
  const float s = scales[i];
  v2bf_t v[4];
  v[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0);
  v[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1);
  v[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2);
  v[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3);
  // each result register holds two bf16 (element 2j in bits 15..0): stored whole
  uint32_t* o = reinterpret_cast<uint32_t*>(out + 8 * (size_t)i);
  for (int j = 0; j < 4; ++j) o[j] = __builtin_bit_cast(uint32_t, v[j]);
}

typedef short v4s_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(64) void k_probe_m4(const v4s_t* a, const v4s_t* b, const v4f_t* c, v4f_t* d) {
  const size_t i = (size_t)blockIdx.x * 64 + threadIdx.x;
  d[i] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a[i], b[i], c[i], 0, 0, 0);
}

extern "C" {
int probe_mfma_4x4_bf16(const void* a, const void* b, const float* c, float* d, int ncalls, void* stream) {
  if (ncalls < 1 || !a || !b || !c || !d) return -1;
  hipLaunchKernelGGL(k_probe_m4, dim3(ncalls), dim3(64), 0, (hipStream_t)stream,
                     reinterpret_cast<const v4s_t*>(a), reinterpret_cast<const v4s_t*>(b),
                     reinterpret_cast<const v4f_t*>(c), reinterpret_cast<v4f_t*>(d));
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int probe_cvt_fp4_bf16(const uint32_t* words, const float* scales, uint16_t* out, int n, void* stream) {
  if (n < 1 || !words || !scales || !out) return -1;
  hipLaunchKernelGGL(k_probe_cvt, dim3((n + 255) / 256), dim3(256), 0, (hipStream_t)stream, words, scales, out, n);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int probe_mfma_f32(const float* a, const float* b, const float* c, float* d, int ncalls, void* stream) {
  if (ncalls < 1 || !a || !b || !c || !d) return -1;
  hipLaunchKernelGGL(k_probe_f32, dim3(ncalls), dim3(64), 0, (hipStream_t)stream, a, b, c, d);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
int probe_mfma_fp4(const uint32_t* a, const uint32_t* b, const uint8_t* sa, const uint8_t* sb,
                   const float* c, float* d, int ncalls, void* stream) {
  if (ncalls < 1 || !a || !b || !sa || !sb || !c || !d) return -1;
  hipLaunchKernelGGL(k_probe_fp4, dim3(ncalls), dim3(64), 0, (hipStream_t)stream, a, b, sa, sb, c, d);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
}
