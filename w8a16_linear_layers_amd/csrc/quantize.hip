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
#include "device.h"
#include "internal.h"

namespace fp8lin {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // vectors in flight per thread

__global__ __launch_bounds__(kThreads) void quantize_static_kernel(const u32x4* __restrict__ x,
                                                                   u32x2* __restrict__ q, int64_t nvec,
                                                                   float s, float r) {
  const int64_t step = (int64_t)gridDim.x * (kThreads * kUnroll);
  for (int64_t base = (int64_t)blockIdx.x * (kThreads * kUnroll); base < nvec; base += step) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + u * kThreads + threadIdx.x;
      if (i < nvec) v[u] = __builtin_nontemporal_load(x + i);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + u * kThreads + threadIdx.x;
      if (i < nvec) {
        uint32_t doubt = 0;
        const uint32_t p0 = quant_pair_fast(v[u].x, r, doubt);
        const uint32_t p1 = quant_pair_fast(v[u].y, r, doubt);
        const uint32_t p2 = quant_pair_fast(v[u].z, r, doubt);
        const uint32_t p3 = quant_pair_fast(v[u].w, r, doubt);
        u32x2 out;
        out.x = pick_codes(p0, p1);
        out.y = pick_codes(p2, p3);
        if (doubt) {
          out.x = quant_word_exact(v[u].x, s) | (quant_word_exact(v[u].y, s) << 16);
          out.y = quant_word_exact(v[u].z, s) | (quant_word_exact(v[u].w, s) << 16);
        }
        __builtin_nontemporal_store(out, q + i);
      }
    }
  }
}

}  // namespace

hipError_t launch_quantize(const void* x, void* q, int64_t n, float scale, hipStream_t s) {
  const int64_t nvec = n / 8;
  const int64_t per_block = kThreads * kUnroll;
  int64_t blocks = (nvec + per_block - 1) / per_block;
  if (blocks > 4096) blocks = 4096;
  const float r = 1.0f / scale;  // correctly rounded on the host
  hipLaunchKernelGGL(quantize_static_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                     static_cast<const u32x4*>(x), static_cast<u32x2*>(q), nvec, scale, r);
  return hipGetLastError();
}

}  // namespace fp8lin
