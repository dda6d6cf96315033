// Static per-tensor activation quantization, bf16 -> E4M3.
//
// [CF-157] "Verification": the reference quantizer divides by the exported
// input_scale, clamps to the FP8 range and rounds (three eager passes over
// HBM there); here it is one streaming pass: 2 bytes read and 1 byte written
// per element.
//
// Layout: the tensor is processed as a flat array of 8-element vectors
// (16 bytes of bf16 in, 8 bytes of codes out). Consecutive lanes take
// consecutive vectors, so every load and store instruction of a wave covers
// one contiguous 1 KiB / 512 B span.
#include <cmath>

#include "device.h"
#include "internal.h"

namespace fp8lin {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // vectors in flight per thread

template <bool kPow2>
__device__ __forceinline__ u32x2 quantize8(const u32x4 v, float s, float r, bool exact_ok) {
  uint32_t doubt = 0;
  uint32_t p0, p1, p2, p3;
  if constexpr (kPow2) {
    p0 = quant_pair_pow2(v.x, r, doubt);
    p1 = quant_pair_pow2(v.y, r, doubt);
    p2 = quant_pair_pow2(v.z, r, doubt);
    p3 = quant_pair_pow2(v.w, r, doubt);
  } else {
    p0 = quant_pair_fast(v.x, r, doubt);
    p1 = quant_pair_fast(v.y, r, doubt);
    p2 = quant_pair_fast(v.z, r, doubt);
    p3 = quant_pair_fast(v.w, r, doubt);
  }
  u32x2 out;
  out.x = pick_codes(p0, p1);
  out.y = pick_codes(p2, p3);
  if (doubt) {
    out.x = quant_word_exact(v.x, s, r, exact_ok) | (quant_word_exact(v.y, s, r, exact_ok) << 16);
    out.y = quant_word_exact(v.z, s, r, exact_ok) | (quant_word_exact(v.w, s, r, exact_ok) << 16);
  }
  return out;
}

// Full chunks of kThreads * kUnroll vectors are processed with all loads
// issued back to back (no per-load guard, so nothing serializes them); the
// remaining vectors, fewer than one chunk, one per thread with a guard.
template <bool kPow2>
__global__ __launch_bounds__(kThreads) void quantize_static_kernel(const u32x4* __restrict__ x,
                                                                   u32x2* __restrict__ q, int64_t nvec,
                                                                   float s, float r, bool exact_ok) {
  constexpr int64_t kChunk = kThreads * kUnroll;
  const int64_t full = nvec / kChunk * kChunk;
  const int64_t step = (int64_t)gridDim.x * kChunk;
  for (int64_t base = (int64_t)blockIdx.x * kChunk + threadIdx.x; base < full; base += step) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(x + base + u * kThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      __builtin_nontemporal_store(quantize8<kPow2>(v[u], s, r, exact_ok), q + base + u * kThreads);
  }
  for (int64_t i = full + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * kThreads)
    q[i] = quantize8<kPow2>(x[i], s, r, exact_ok);
}

}  // namespace

hipError_t launch_quantize(const void* x, void* q, int64_t n, float scale, hipStream_t s) {
  const int64_t nvec = n / 8;
  const int64_t per_block = kThreads * kUnroll;
  int64_t blocks = (nvec + per_block - 1) / per_block;
  if (blocks > 65536) blocks = 65536;  // one chunk per workgroup up to 2^26 vectors
  const float r = 1.0f / scale;  // correctly rounded on the host
  int e = 0;
  const bool pow2 = std::frexp(scale, &e) == 0.5f;  // scale = 2^(e-1), and 1/scale is normal
  const bool exact_ok = scale >= 0x1p-92f;
  if (pow2)
    hipLaunchKernelGGL(quantize_static_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                       static_cast<const u32x4*>(x), static_cast<u32x2*>(q), nvec, scale, r, exact_ok);
  else
    hipLaunchKernelGGL(quantize_static_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                       static_cast<const u32x4*>(x), static_cast<u32x2*>(q), nvec, scale, r, exact_ok);
  return hipGetLastError();
}

}  // namespace fp8lin
