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
  u32x2 out;
  if constexpr (kPow2) {
    out.x = quant_quad_pow2(v.x, v.y, r, doubt);
    out.y = quant_quad_pow2(v.z, v.w, r, doubt);
  } else {
    const uint32_t p0 = quant_pair_fast(v.x, r, doubt);
    const uint32_t p1 = quant_pair_fast(v.y, r, doubt);
    const uint32_t p2 = quant_pair_fast(v.z, r, doubt);
    const uint32_t p3 = quant_pair_fast(v.w, r, doubt);
    out.x = pick_codes(p0, p1);
    out.y = pick_codes(p2, p3);
  }
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
__device__ __forceinline__ void quantize_range(const u32x4* __restrict__ x, u32x2* __restrict__ q, int64_t nvec,
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

template <bool kPow2>
__global__ __launch_bounds__(kThreads) void quantize_static_kernel(const u32x4* __restrict__ x,
                                                                   u32x2* __restrict__ q, int64_t nvec,
                                                                   float s, float r, bool exact_ok) {
  quantize_range<kPow2>(x, q, nvec, s, r, exact_ok);
}

// ---------------------------------------------------------------- dynamic
//
// Dynamic per-tensor scale: s = fl32(amax) / 448 over the finite elements,
// at least 2^-126, then the static rule with s. Pass 1 reduces amax into a
// 32-bit word as bf16 magnitude bits (non-finite elements count as 0; for
// finite values the order of the bits is the order of the magnitudes), pass
// 2 derives s, 1 / s and the exactness flags on the device and quantizes.

__global__ void amax_clear_kernel(uint32_t* ws) { *ws = 0u; }

// Largest finite bf16 magnitude (bits) of the two values packed in w.
__device__ __forceinline__ uint32_t finite_mag2(uint32_t w) {
  const uint32_t lo = w & 0x7fffu, hi = (w >> 16) & 0x7fffu;
  return max(lo < 0x7f80u ? lo : 0u, hi < 0x7f80u ? hi : 0u);
}

// 16 waves per workgroup and 256 workgroups: four times the loads in flight
// of 256-thread workgroups at half the atomics on the amax word (A/B on one
// box: 69.9 -> 67.3 us for amax + quantize of 16384 x 4096, cold inputs).
constexpr int kAmaxThreads = 1024;

__global__ __launch_bounds__(kAmaxThreads) void amax_kernel(const u32x4* __restrict__ x, int64_t nvec,
                                                            uint32_t* __restrict__ ws) {
  // full chunks with kUnroll loads in flight per thread, then the tail
  constexpr int64_t kChunk = kAmaxThreads * kUnroll;
  const int64_t full = nvec / kChunk * kChunk;
  uint32_t m = 0;
  for (int64_t base = (int64_t)blockIdx.x * kChunk + threadIdx.x; base < full; base += (int64_t)gridDim.x * kChunk) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(x + base + u * kAmaxThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      m = max(m, max(max(finite_mag2(v[u].x), finite_mag2(v[u].y)), max(finite_mag2(v[u].z), finite_mag2(v[u].w))));
  }
  for (int64_t i = full + (int64_t)blockIdx.x * kAmaxThreads + threadIdx.x; i < nvec;
       i += (int64_t)gridDim.x * kAmaxThreads) {
    const u32x4 v = x[i];
    m = max(m, max(max(finite_mag2(v.x), finite_mag2(v.y)), max(finite_mag2(v.z), finite_mag2(v.w))));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  __shared__ uint32_t wave_max[kAmaxThreads / 64];
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t b = wave_max[0];
#pragma unroll
    for (int w = 1; w < kAmaxThreads / 64; ++w) b = max(b, wave_max[w]);
    atomicMax(ws, b);
  }
}

__device__ __forceinline__ float dynamic_scale_of(uint32_t amax_bits) {
  const float amax = __uint_as_float(amax_bits << 16);
  return fmaxf(amax / 448.0f, 0x1p-126f);  // correctly rounded division
}

__global__ __launch_bounds__(kThreads) void quantize_dynamic_kernel(const u32x4* __restrict__ x,
                                                                    u32x2* __restrict__ q, int64_t nvec,
                                                                    const uint32_t* __restrict__ ws,
                                                                    float* __restrict__ scale_out) {
  const float s = dynamic_scale_of(*ws);
  const float r = 1.0f / s;
  const bool exact_ok = s >= 0x1p-92f;
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = s;
  if ((__float_as_uint(s) & 0x7fffffu) == 0)
    quantize_range<true>(x, q, nvec, s, r, exact_ok);
  else
    quantize_range<false>(x, q, nvec, s, r, exact_ok);
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

hipError_t launch_quantize_dynamic(const void* x, void* q, int64_t n, uint32_t* amax_ws, float* scale_out,
                                  hipStream_t s) {
  const int64_t nvec = n / 8;
  hipLaunchKernelGGL(amax_clear_kernel, dim3(1), dim3(1), 0, s, amax_ws);
  // 256 workgroups: enough loads in flight to stream x, few enough that their
  // atomics on the one amax word (serialized in memory) stay cheap
  int64_t ablocks = (nvec + kAmaxThreads * kUnroll - 1) / (kAmaxThreads * kUnroll);
  if (ablocks < 1) ablocks = 1;
  if (ablocks > 256) ablocks = 256;
  hipLaunchKernelGGL(amax_kernel, dim3((unsigned)ablocks), dim3(kAmaxThreads), 0, s, static_cast<const u32x4*>(x),
                     nvec, amax_ws);
  int64_t blocks = (nvec + kThreads * kUnroll - 1) / (kThreads * kUnroll);
  if (blocks < 1) blocks = 1;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(quantize_dynamic_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                     static_cast<const u32x4*>(x), static_cast<u32x2*>(q), nvec, amax_ws, scale_out);
  return hipGetLastError();
}

}  // namespace fp8lin
