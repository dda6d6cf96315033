// Internal interface between the C-ABI layer (api.hip) and the kernel
// translation units. Launchers assume validated arguments: they do no checks
// of their own and return the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8lin {

// Tile shape shared by both GEMMs: a workgroup computes a 256 (M) x 256 (N)
// output tile with four waves of 128 x 128.
constexpr int kTileM = 256;
constexpr int kTileN = 256;
constexpr int kMaxGroups = 4;

// One projection of a grouped GEMM: all groups share the activation.
struct GemmGroup {
  const uint8_t* w;  // E4M3 [n, k]
  void* y;           // bf16 [m, ldy]
  int32_t n;
  int32_t ldy;
  float alpha;       // output scale: s_in * s_w (W8A8) or s_w (W8A16)
  int32_t tile_begin;  // first global tile index of this group
  int32_t tiles_n;     // ceil(n / kTileN)
  int32_t koff;        // split-K: first K element of this group's slice (0 otherwise)
};

struct GemmArgs {
  const void* x;  // E4M3 [m, k] (W8A8) or 16-bit [m, xk] (W8A16)
  int32_t m;
  int32_t k;
  int32_t xk;     // W8A16 activation row length: k, or 3 * 64 * ceil(k / 64) for
                  // the three-piece float32 form (0: set to k by the plans)
  int32_t ks;     // split-K: the K length (elements) of each group's slice (k is the row pitch)
  int32_t tiles_m;
  int32_t ngroups;
  int32_t total_tiles;
  float out_rs;   // fused gate/up + SwiGLU: 1 / s_h (the down projection's input scale)
  GemmGroup g[kMaxGroups];
  const float* in_scale_dev;  // W8A8 with a device input scale: alpha = g.alpha * *in_scale_dev
  // W8A8 with the per-head QK RMSNorm + RoPE epilogue on groups 0 and 1
  // (heads of 128 columns): bf16 norm weights (null: 1), float32 cos/sin
  // tables [m, 64], epsilon
  const uint16_t* nr_w[2];
  const float* nr_cos;
  const float* nr_sin;
  float nr_eps;
};

// Fills tile_begin / tiles_n / tiles_m / total_tiles from m, n of each group.
void gemm_plan(GemmArgs& a);

// Tile plan of the fused gate/up + SwiGLU GEMM (ngroups = 1; g[0] = gate with
// the h output, n = I; g[1] = up): tiles of 256 rows by 128 columns of h.
void gate_up_plan(GemmArgs& a);

hipError_t launch_quantize(const void* x, void* q, int64_t n, float scale, hipStream_t s);
// Dynamic: clears amax_ws, reduces the finite amax of x into it, then
// quantizes with s = max(fl32(amax) / 448, 2^-126) and stores s to scale_out.
hipError_t launch_quantize_dynamic(const void* x, void* q, int64_t n, uint32_t* amax_ws, float* scale_out,
                                   hipStream_t s);
hipError_t launch_gemm_w8a8(const GemmArgs& a, hipStream_t s);
// Split-K W8A8: group s multiplies K bytes [koff, koff + ks) of x and w and
// writes float32 partial sums (no scale) to its y [m, ldy]; then
// y = bf16(alpha * sum_s partial_s) over `splits` partials of [m, n] each.
hipError_t launch_gemm_w8a8_splitk(const GemmArgs& a, hipStream_t s);
// Compute units of the current device.
int device_cu_count();
// True when a W8A8 or 16-bit W8A16 GEMM launch whose 256 x 256 tiles number
// big_tiles runs on the 128 x 128 tile kernels instead (those tiles would
// keep at most 60% of the compute units busy).
bool small_tiles_for(int64_t big_tiles);
// The current device's copy of the library's static scratch array
// (FP8LIN_SCRATCH_BYTES bytes), looked up once per device and kept.
hipError_t device_scratch(void** ptr);
hipError_t launch_splitk_reduce(const float* partials, int splits, void* y, int64_t m, int64_t n, int64_t ldy,
                                float alpha, hipStream_t s);
// The same grouped launch with the QK RMSNorm + RoPE epilogue on groups 0, 1.
hipError_t launch_gemm_w8a8_norm_rope(const GemmArgs& a, hipStream_t s);
// W8A16 activation forms: bf16, binary16, float32 as three bf16 pieces
constexpr int kW16Bf16 = 0, kW16F16 = 1, kW16F32 = 2;
hipError_t launch_gemm_w8a16(const GemmArgs& a, int form, hipStream_t s);
// Split-K W8A16 (bf16 activations): group s multiplies K elements [koff,
// koff + ks) of x and w and writes its float32 partial sums (no scale) to its
// y [m, ldy]; launch_splitk_reduce then writes y = bf16(alpha * sum).
hipError_t launch_gemm_w8a16_splitk(const GemmArgs& a, hipStream_t s);
// Per-head RMSNorm + rotate-half RoPE of q [tokens, q_heads * head_dim] and
// k [tokens, k_heads * head_dim] (bf16; k_heads may be 0), head_dim 64 or 128.
hipError_t launch_qk_norm_rope(const void* q, void* q_out, int q_heads, const void* q_w, const void* k, void* k_out,
                               int k_heads, const void* k_w, int64_t tokens, int head_dim, const float* cos,
                               const float* sin, float eps, hipStream_t s);
// x [rows, k] float32 -> x3 [rows, 3 * 64 * ceil(k / 64)] bf16 pieces
hipError_t launch_split3(const float* x, void* x3, int64_t rows, int64_t k, hipStream_t s);
// Fused gate/up + SwiGLU: W8A8 (E4M3 h, a.out_rs) or W8A16 (bf16 h, or
// binary16 h from a binary16 activation with f16).
hipError_t launch_gate_up_swiglu(const GemmArgs& a, bool w8a16, bool f16, hipStream_t s);
hipError_t launch_swiglu(const void* g, const void* u, void* out, bool f16, bool fp8_out, int64_t n, float scale,
                         hipStream_t s);

}  // namespace fp8lin
