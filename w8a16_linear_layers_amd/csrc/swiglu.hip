// Two-input SwiGLU: h = silu(gate) * up from two separate 16-bit tensors
// (bf16 or fp16), emitted as E4M3 codes (scaled by the down projection's
// static input scale) or in the input's format on 16-bit steps.
//
// [TRT-17476] "What changed": the split gated MLP feeds SiLU(G) * U from
// two tensors straight into an FP8 output, avoiding the concatenated
// [M, 2I] intermediate; the pages attribute its speed to DRAM utilization,
// so this is one streaming pass: 4 bytes read and 1 (or 2) written per
// element, 8 elements per lane-vector, consecutive lanes on consecutive
// vectors.
#include "device.h"
#include "internal.h"

namespace fp8lin {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 2;

template <bool kF16, bool kFp8Out>
__device__ __forceinline__ void swiglu8(const u32x4 gv, const u32x4 uv, void* out, int64_t i, float rs) {
  float h[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[2 * e] = silu_mul(h16_lo<kF16>(gv[e]), h16_lo<kF16>(uv[e]));
    h[2 * e + 1] = silu_mul(h16_hi<kF16>(gv[e]), h16_hi<kF16>(uv[e]));
  }
  if constexpr (kFp8Out) {
    u32x2 o;
    o.x = swiglu_codes4(h[0], h[1], h[2], h[3], rs);
    o.y = swiglu_codes4(h[4], h[5], h[6], h[7], rs);
    __builtin_nontemporal_store(o, static_cast<u32x2*>(out) + i);
  } else {
    u32x4 o;
    o.x = h16x2<kF16>(h[0], h[1]);
    o.y = h16x2<kF16>(h[2], h[3]);
    o.z = h16x2<kF16>(h[4], h[5]);
    o.w = h16x2<kF16>(h[6], h[7]);
    __builtin_nontemporal_store(o, static_cast<u32x4*>(out) + i);
  }
}

// Full chunks with unguarded back-to-back loads, then a guarded tail.
template <bool kF16, bool kFp8Out>
__global__ __launch_bounds__(kThreads) void swiglu_2in_kernel(const u32x4* __restrict__ g,
                                                              const u32x4* __restrict__ u, void* __restrict__ out,
                                                              int64_t nvec, float rs) {
  constexpr int64_t kChunk = kThreads * kUnroll;
  const int64_t full = nvec / kChunk * kChunk;
  const int64_t step = (int64_t)gridDim.x * kChunk;
  for (int64_t base = (int64_t)blockIdx.x * kChunk + threadIdx.x; base < full; base += step) {
    u32x4 gv[kUnroll], uv[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      gv[k] = __builtin_nontemporal_load(g + base + k * kThreads);
      uv[k] = __builtin_nontemporal_load(u + base + k * kThreads);
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) swiglu8<kF16, kFp8Out>(gv[k], uv[k], out, base + k * kThreads, rs);
  }
  for (int64_t i = full + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * kThreads)
    swiglu8<kF16, kFp8Out>(g[i], u[i], out, i, rs);
}

}  // namespace

hipError_t launch_swiglu(const void* g, const void* u, void* out, bool f16, bool fp8_out, int64_t n, float scale,
                         hipStream_t s) {
  const int64_t nvec = n / 8;
  const int64_t per_block = kThreads * kUnroll;
  int64_t blocks = (nvec + per_block - 1) / per_block;
  if (blocks > 65536) blocks = 65536;  // one chunk per workgroup up to 2^25 vectors
  const float rs = fp8_out ? 1.0f / scale : 1.0f;
  auto kernel = f16 ? (fp8_out ? swiglu_2in_kernel<true, true> : swiglu_2in_kernel<true, false>)
                    : (fp8_out ? swiglu_2in_kernel<false, true> : swiglu_2in_kernel<false, false>);
  hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, static_cast<const u32x4*>(g),
                     static_cast<const u32x4*>(u), out, nvec, rs);
  return hipGetLastError();
}

}  // namespace fp8lin
