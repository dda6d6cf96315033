// Per-head QK RMSNorm followed by rotate-half RoPE, on the contiguous Q and
// K outputs of separate projections.
//
// [TRT-17476] "It is also faster": separate projections hand the per-head
// QK RMSNorm and the rotary embedding contiguous rows (a fused QKV output
// would give them strided views). Per head of D values x, in float32:
//   r = rsqrt(sum(x^2) / D + eps),  y = x * r * w
//   out[i]         = y[i] * cos[t, i] - y[i + D/2] * sin[t, i]
//   out[i + D/2]   = y[i + D/2] * cos[t, i] + y[i] * sin[t, i]    (i < D/2)
// rounded once to bf16.
//
// Layout: q [tokens, q_heads * D] and k [tokens, k_heads * D] bf16, rows
// contiguous, so head unit u (token u / heads, head u % heads) is the D
// values at u * D. One unit takes L = D / 16 lanes; lane l holds values
// [8 l, 8 l + 8) and [D/2 + 8 l, D/2 + 8 l + 8): both halves of its eight
// RoPE pairs, so the rotation needs no exchange and the sum of squares one
// butterfly over L lanes. Every access is 16 bytes per lane, L lanes
// covering a contiguous span.
// HBM-bound: 2 bytes read and 2 written per value, plus the tables (D
// float32 per token, shared by the token's heads through the caches).
#include "device.h"
#include "internal.h"

namespace fp8lin {
namespace {

constexpr int kThreads = 256;

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct QkPart {
  const uint16_t* x;
  uint16_t* out;
  const uint16_t* w;  // bf16 [D], or null for a unit weight
  int64_t units;      // tokens * heads
  int heads;
};

// Load the unit's values for lane l: a = [8 l, 8 l + 8), b = the same
// positions of the second half.
struct UnitVals {
  u32x4 a, b;
};

template <int D>
__device__ __forceinline__ UnitVals load_unit(const QkPart& p, int64_t u, int l) {
  const u32x4* src = reinterpret_cast<const u32x4*>(p.x + u * D);
  return UnitVals{__builtin_nontemporal_load(src + l), __builtin_nontemporal_load(src + D / 16 + l)};
}

__device__ __forceinline__ void unpack8(const u32x4 v, float (&f)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = bf16_lo(v[e]);
    f[2 * e + 1] = bf16_hi(v[e]);
  }
}

template <int D>
__device__ __forceinline__ void norm_rope_store(const QkPart& p, int64_t u, int l, const UnitVals& v,
                                                const float* __restrict__ cos, const float* __restrict__ sin,
                                                float eps) {
  constexpr int L = D / 16;
  const int64_t t = u / p.heads;
  float a[8], b[8];
  unpack8(v.a, a);
  unpack8(v.b, b);
  float ss = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += a[e] * a[e] + b[e] * b[e];
#pragma unroll
  for (int off = L / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  const float r = rsqrtf(ss * (1.0f / D) + eps);
  float wa[8], wb[8];
  if (p.w != nullptr) {
    unpack8(reinterpret_cast<const u32x4*>(p.w)[l], wa);
    unpack8(reinterpret_cast<const u32x4*>(p.w)[D / 16 + l], wb);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) wa[e] = wb[e] = 1.0f;
  }
  const f32x4* cr = reinterpret_cast<const f32x4*>(cos + t * (D / 2)) + 2 * l;
  const f32x4* sr = reinterpret_cast<const f32x4*>(sin + t * (D / 2)) + 2 * l;
  const f32x4 c0 = cr[0], c1 = cr[1], s0 = sr[0], s1 = sr[1];
  const float c[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
  const float s[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
  float oa[8], ob[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float ya = a[e] * r * wa[e];
    const float yb = b[e] * r * wb[e];
    oa[e] = ya * c[e] - yb * s[e];
    ob[e] = yb * c[e] + ya * s[e];
  }
  u32x4 pa, pb;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    pa[e] = h16x2<false>(oa[2 * e], oa[2 * e + 1]);
    pb[e] = h16x2<false>(ob[2 * e], ob[2 * e + 1]);
  }
  u32x4* dst = reinterpret_cast<u32x4*>(p.out + u * D);
  __builtin_nontemporal_store(pa, dst + l);
  __builtin_nontemporal_store(pb, dst + D / 16 + l);
}

// Units [0, q.units) are Q heads, then k.units K heads. Each group of
// L = D / 16 lanes takes two units per iteration, both loaded before
// either is computed.
template <int D>
__global__ __launch_bounds__(kThreads) void qk_norm_rope_kernel(const QkPart q, const QkPart k,
                                                                const float* __restrict__ cos,
                                                                const float* __restrict__ sin, float eps) {
  constexpr int L = D / 16;
  constexpr int kGroups = kThreads / L;  // lane groups per workgroup
  const int l = threadIdx.x % L;
  const int64_t total = q.units + k.units;
  const int64_t stride = (int64_t)gridDim.x * kGroups * 2;
  for (int64_t u0 = ((int64_t)blockIdx.x * kGroups + threadIdx.x / L) * 2; u0 < total; u0 += stride) {
    const int64_t u1 = u0 + 1;
    const bool has1 = u1 < total;
    const UnitVals v0 = u0 < q.units ? load_unit<D>(q, u0, l) : load_unit<D>(k, u0 - q.units, l);
    UnitVals v1 = v0;
    if (has1) v1 = u1 < q.units ? load_unit<D>(q, u1, l) : load_unit<D>(k, u1 - q.units, l);
    if (u0 < q.units)
      norm_rope_store<D>(q, u0, l, v0, cos, sin, eps);
    else
      norm_rope_store<D>(k, u0 - q.units, l, v0, cos, sin, eps);
    if (has1) {
      if (u1 < q.units)
        norm_rope_store<D>(q, u1, l, v1, cos, sin, eps);
      else
        norm_rope_store<D>(k, u1 - q.units, l, v1, cos, sin, eps);
    }
  }
}

}  // namespace

hipError_t launch_qk_norm_rope(const void* q, void* q_out, int q_heads, const void* q_w, const void* k, void* k_out,
                               int k_heads, const void* k_w, int64_t tokens, int head_dim, const float* cos,
                               const float* sin, float eps, hipStream_t s) {
  QkPart pq{static_cast<const uint16_t*>(q), static_cast<uint16_t*>(q_out), static_cast<const uint16_t*>(q_w),
            tokens * q_heads, q_heads};
  QkPart pk{static_cast<const uint16_t*>(k), static_cast<uint16_t*>(k_out), static_cast<const uint16_t*>(k_w),
            tokens * k_heads, k_heads > 0 ? k_heads : 1};
  const int per_block = 2 * kThreads / (head_dim / 16);  // units per workgroup iteration
  int64_t blocks = (pq.units + pk.units + per_block - 1) / per_block;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  if (head_dim == 64)
    hipLaunchKernelGGL(qk_norm_rope_kernel<64>, dim3((unsigned)blocks), dim3(kThreads), 0, s, pq, pk, cos, sin, eps);
  else
    hipLaunchKernelGGL(qk_norm_rope_kernel<128>, dim3((unsigned)blocks), dim3(kThreads), 0, s, pq, pk, cos, sin,
                       eps);
  return hipGetLastError();
}

}  // namespace fp8lin
