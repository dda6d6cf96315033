// Float32 activations for the W8A16 GEMM: each value is split exactly into
// three bf16 pieces, x = hi + mid + lo, so the bf16 MFMA path computes the
// product with exact terms and float32 accumulation.
//
// [DF-14664] "Tests" lists a float32-activation W8A16 case: the weight is
// dequantized to the activation's dtype and the linear runs in float32.
// Every E4M3 value is exact in bf16, and a bf16 piece times it is exact in
// float32, so sum_p piece_p * w over the three pieces is the float32
// product's exact value; only the accumulation rounds (3 K terms).
//
// Split (truncation): hi = x with the low 16 bits cleared, r = x - hi
// (exact), mid = r with its low 16 bits cleared, lo = r - mid (exact, at
// most 8 significant bits). Non-finite values go whole into hi (a NaN
// stays a NaN). For |x| below about 2^-110 the low piece falls under the
// bf16 subnormal quantum and loses bits.
//
// Layout: x [rows, k] float32 -> x3 [rows, 3 kp] bf16 with kp = 64 *
// ceil(k / 64); block b (64 values) of a row becomes blocks 3 b (hi),
// 3 b + 1 (mid) and 3 b + 2 (lo), the GEMM's stage order. Values past k are
// zero. One lane handles 8 consecutive values: two 16-byte loads, three
// 16-byte stores.
#include "device.h"
#include "internal.h"

namespace fp8lin {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void split_one(uint32_t x, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  if ((x & 0x7f800000u) == 0x7f800000u) {  // Inf / NaN
    hi = (x >> 16) | ((x & 0x7fffffu) ? 0x40u : 0u);
    mid = lo = 0;
    return;
  }
  const uint32_t h = x & 0xffff0000u;
  const float r = __uint_as_float(x) - __uint_as_float(h);
  const uint32_t rb = __float_as_uint(r);
  const uint32_t m = rb & 0xffff0000u;
  const float l = r - __uint_as_float(m);
  hi = h >> 16;
  mid = m >> 16;
  lo = __float_as_uint(l) >> 16;
}

__global__ __launch_bounds__(kThreads) void split3_kernel(const float* __restrict__ x, uint16_t* __restrict__ x3,
                                                          int64_t groups, int64_t k, int64_t kp) {
  const int64_t per_row = kp / 8;  // 8-value groups per row, padding included
  for (int64_t gi = (int64_t)blockIdx.x * kThreads + threadIdx.x; gi < groups;
       gi += (int64_t)gridDim.x * kThreads) {
    const int64_t row = gi / per_row;
    const int64_t c = (gi - row * per_row) * 8;  // first value of the group
    u32x4 v0 = {0, 0, 0, 0}, v1 = {0, 0, 0, 0};
    if (c < k) {  // k % 16 == 0: a group is wholly inside or wholly past k
      const u32x4* src = reinterpret_cast<const u32x4*>(x + row * k + c);
      v0 = __builtin_nontemporal_load(src);
      v1 = __builtin_nontemporal_load(src + 1);
    }
    uint32_t hi[8], mid[8], lo[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      split_one(v0[e], hi[e], mid[e], lo[e]);
      split_one(v1[e], hi[4 + e], mid[4 + e], lo[4 + e]);
    }
    u32x4 ph, pm, pl;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ph[e] = hi[2 * e] | (hi[2 * e + 1] << 16);
      pm[e] = mid[2 * e] | (mid[2 * e + 1] << 16);
      pl[e] = lo[2 * e] | (lo[2 * e + 1] << 16);
    }
    const int64_t b = c / 64, cc = c - b * 64;
    uint16_t* dst = x3 + row * 3 * kp + b * 192 + cc;
    __builtin_nontemporal_store(ph, reinterpret_cast<u32x4*>(dst));
    __builtin_nontemporal_store(pm, reinterpret_cast<u32x4*>(dst + 64));
    __builtin_nontemporal_store(pl, reinterpret_cast<u32x4*>(dst + 128));
  }
}

}  // namespace

hipError_t launch_split3(const float* x, void* x3, int64_t rows, int64_t k, hipStream_t s) {
  const int64_t kp = (k + 63) / 64 * 64;
  const int64_t groups = rows * (kp / 8);
  int64_t blocks = (groups + kThreads - 1) / kThreads;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(split3_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, x, static_cast<uint16_t*>(x3),
                     groups, k, kp);
  return hipGetLastError();
}

}  // namespace fp8lin
