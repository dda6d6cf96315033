// C ABI of libfp8lin: argument validation, dispatch to the kernel launchers,
// the diffusion step policy and the error strings. Everything is validated
// before the first launch, so a failing call enqueues nothing.
#include <atomic>
#include <cmath>
#include <cstring>

#include "fp8lin.h"
#include "internal.h"

namespace {

using fp8lin::GemmArgs;

std::atomic<int64_t> g_launches[FP8LIN_KERNEL_KINDS];

void count_launch(int kind) { g_launches[kind].fetch_add(1, std::memory_order_relaxed); }

constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxK = int64_t(1) << 24;
constexpr int64_t kMaxElems = int64_t(1) << 40;
// GEMM tiles are addressed through buffer resources with 32-bit offsets: 256
// rows of a bf16 activation (2 K bytes each) and 128 output rows (2 ldy bytes
// each) must stay below the 2^31 out-of-range offset.
constexpr int64_t kMaxGemmDim = int64_t(1) << 22;
// The three-piece float32 activation has 3 * 64 * ceil(K / 64) bf16 values
// per row; 256 such rows must stay below the same 2^31 offset.
constexpr int64_t kMaxF32K = int64_t(1) << 20;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A static scale must be finite and in [2^-126, 2^126], so 1/s is normal.
bool scale_ok(float s) { return std::isfinite(s) && s >= 0x1p-126f && s <= 0x1p126f; }

int32_t check_matrix(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0) return FP8LIN_EINVAL;
  if (rows > kMaxRows || cols >= kMaxK || rows * cols >= kMaxElems) return FP8LIN_EUNSUPPORTED;
  if (cols % 16 != 0) return FP8LIN_ELAYOUT;
  return FP8LIN_OK;
}

// The tile plans count M in 256-row tiles with 32-bit arithmetic: M + 255
// must not overflow.
constexpr int64_t kMaxGemmRows = (int64_t(1) << 31) - 256;

int32_t check_gemm_matrix(int64_t M, int64_t K) {
  const int32_t st = check_matrix(M, K);
  if (st != FP8LIN_OK) return st;
  return K >= kMaxGemmDim || M > kMaxGemmRows ? FP8LIN_EUNSUPPORTED : FP8LIN_OK;
}

// Shared checks of one projection of a GEMM (weight [n, k], output [m, ldy]).
int32_t check_output(const void* qw, const void* y, int64_t N, int64_t ldy, int64_t M) {
  if (qw == nullptr || (M > 0 && y == nullptr)) return FP8LIN_EINVAL;
  if (N <= 0 || ldy <= 0) return FP8LIN_EINVAL;
  if (N >= kMaxGemmDim || ldy >= kMaxGemmDim) return FP8LIN_EUNSUPPORTED;
  if (N % 8 != 0 || ldy % 8 != 0 || ldy < N) return FP8LIN_ELAYOUT;
  if (!aligned16(qw) || !aligned16(y)) return FP8LIN_ELAYOUT;  // NULL is aligned
  return FP8LIN_OK;
}

int32_t finish_plan(GemmArgs& a) {
  int64_t tiles = 0;
  const int64_t tm = (a.m + fp8lin::kTileM - 1) / fp8lin::kTileM;
  for (int i = 0; i < a.ngroups; ++i) tiles += tm * ((a.g[i].n + fp8lin::kTileN - 1) / fp8lin::kTileN);
  if (tiles >= (int64_t(1) << 31)) return FP8LIN_EUNSUPPORTED;
  fp8lin::gemm_plan(a);
  return FP8LIN_OK;
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? FP8LIN_OK : FP8LIN_EHIP; }

}  // namespace

extern "C" {

int32_t fp8lin_quantize_static(const void* x_bf16, void* q_e4m3, int64_t rows, int64_t cols, float input_scale,
                               hipStream_t stream) {
  int32_t st = check_matrix(rows, cols);
  if (st != FP8LIN_OK) return st;
  if (!scale_ok(input_scale)) return FP8LIN_ESCALE;
  if (rows == 0 || cols == 0) return FP8LIN_OK;  // empty: pointers may be NULL
  if (x_bf16 == nullptr || q_e4m3 == nullptr) return FP8LIN_EINVAL;
  if (!aligned16(x_bf16) || !aligned16(q_e4m3)) return FP8LIN_ELAYOUT;
  count_launch(FP8LIN_KERNEL_QUANTIZE);
  return hip_status(fp8lin::launch_quantize(x_bf16, q_e4m3, rows * cols, input_scale, stream));
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int32_t fp8lin_quantize_dynamic(const void* x_bf16, void* q_e4m3, int64_t rows, int64_t cols, float* scale_out,
                                uint32_t* amax_ws, hipStream_t stream) {
  int32_t st = check_matrix(rows, cols);
  if (st != FP8LIN_OK) return st;
  if (rows == 0 || cols == 0) return FP8LIN_OK;  // empty: nothing launched, scale_out untouched
  if (x_bf16 == nullptr || q_e4m3 == nullptr || scale_out == nullptr || amax_ws == nullptr) return FP8LIN_EINVAL;
  if (!aligned16(x_bf16) || !aligned16(q_e4m3) || !aligned4(scale_out) || !aligned4(amax_ws)) return FP8LIN_ELAYOUT;
  count_launch(FP8LIN_KERNEL_AMAX);
  count_launch(FP8LIN_KERNEL_QUANTIZE);
  return hip_status(fp8lin::launch_quantize_dynamic(x_bf16, q_e4m3, rows * cols, amax_ws, scale_out, stream));
}

int32_t fp8lin_gemm_w8a8_dev_scale(const void* qx, const void* qw, void* y_bf16, int64_t M, int64_t N, int64_t K,
                                   int64_t ldy, const float* input_scale_dev, float weight_scale,
                                   hipStream_t stream) {
  int32_t st = check_gemm_matrix(M, K);
  if (st != FP8LIN_OK) return st;
  if (K == 0 || (M > 0 && qx == nullptr) || input_scale_dev == nullptr) return FP8LIN_EINVAL;
  if ((st = check_output(qw, y_bf16, N, ldy, M)) != FP8LIN_OK) return st;
  if (!aligned16(qx) || !aligned4(input_scale_dev)) return FP8LIN_ELAYOUT;
  if (!scale_ok(weight_scale)) return FP8LIN_ESCALE;
  if (M == 0) return FP8LIN_OK;
  GemmArgs a{};
  a.x = qx;
  a.m = (int32_t)M;
  a.k = (int32_t)K;
  a.ngroups = 1;
  a.in_scale_dev = input_scale_dev;
  a.g[0].w = static_cast<const uint8_t*>(qw);
  a.g[0].y = y_bf16;
  a.g[0].n = (int32_t)N;
  a.g[0].ldy = (int32_t)ldy;
  a.g[0].alpha = weight_scale;
  if ((st = finish_plan(a)) != FP8LIN_OK) return st;
  count_launch(FP8LIN_KERNEL_GEMM_W8A8);
  return hip_status(fp8lin::launch_gemm_w8a8(a, stream));
}

int32_t fp8lin_gemm_w8a8(const void* qx, const void* qw, void* y_bf16, int64_t M, int64_t N, int64_t K, int64_t ldy,
                         float input_scale, float weight_scale, hipStream_t stream) {
  int32_t st = check_gemm_matrix(M, K);
  if (st != FP8LIN_OK) return st;
  if (K == 0 || (M > 0 && qx == nullptr)) return FP8LIN_EINVAL;
  if ((st = check_output(qw, y_bf16, N, ldy, M)) != FP8LIN_OK) return st;
  if (!aligned16(qx)) return FP8LIN_ELAYOUT;
  if (!scale_ok(input_scale) || !scale_ok(weight_scale)) return FP8LIN_ESCALE;
  const float alpha = input_scale * weight_scale;
  if (!std::isfinite(alpha) || alpha == 0.0f) return FP8LIN_ESCALE;
  if (M == 0) return FP8LIN_OK;
  GemmArgs a{};
  a.x = qx;
  a.m = (int32_t)M;
  a.k = (int32_t)K;
  a.ngroups = 1;
  a.g[0].w = static_cast<const uint8_t*>(qw);
  a.g[0].y = y_bf16;
  a.g[0].n = (int32_t)N;
  a.g[0].ldy = (int32_t)ldy;
  a.g[0].alpha = alpha;
  if ((st = finish_plan(a)) != FP8LIN_OK) return st;
  count_launch(FP8LIN_KERNEL_GEMM_W8A8);
  return hip_status(fp8lin::launch_gemm_w8a8(a, stream));
}

int32_t fp8lin_gemm_w8a16(const void* x, int32_t x_dtype, const void* qw, void* y_bf16, int64_t M, int64_t N,
                          int64_t K, int64_t ldy, float weight_scale, hipStream_t stream) {
  // FP8 activations are refused; float32 ones take fp8lin_gemm_w8a16_f32
  if (x_dtype == FP8LIN_DT_E4M3 || x_dtype == FP8LIN_DT_F32) return FP8LIN_EDTYPE;
  if (x_dtype != FP8LIN_DT_BF16 && x_dtype != FP8LIN_DT_F16) return FP8LIN_EINVAL;
  int32_t st = check_gemm_matrix(M, K);
  if (st != FP8LIN_OK) return st;
  if (K == 0 || (M > 0 && x == nullptr)) return FP8LIN_EINVAL;
  if ((st = check_output(qw, y_bf16, N, ldy, M)) != FP8LIN_OK) return st;
  if (!aligned16(x)) return FP8LIN_ELAYOUT;
  if (!scale_ok(weight_scale)) return FP8LIN_ESCALE;
  if (M == 0) return FP8LIN_OK;
  GemmArgs a{};
  a.x = x;
  a.m = (int32_t)M;
  a.k = (int32_t)K;
  a.ngroups = 1;
  a.g[0].w = static_cast<const uint8_t*>(qw);
  a.g[0].y = y_bf16;
  a.g[0].n = (int32_t)N;
  a.g[0].ldy = (int32_t)ldy;
  a.g[0].alpha = weight_scale;
  if ((st = finish_plan(a)) != FP8LIN_OK) return st;
  count_launch(FP8LIN_KERNEL_GEMM_W8A16);
  return hip_status(
      fp8lin::launch_gemm_w8a16(a, x_dtype == FP8LIN_DT_F16 ? fp8lin::kW16F16 : fp8lin::kW16Bf16, stream));
}

int64_t fp8lin_w8a16_f32_workspace_bytes(int64_t M, int64_t K) {
  if (M < 0 || K < 0 || K >= kMaxF32K || M > kMaxRows) return -1;
  return M * 3 * ((K + 63) / 64 * 64) * 2;
}

int32_t fp8lin_gemm_w8a16_f32(const void* x_f32, const void* qw, void* y_f32, int64_t M, int64_t N, int64_t K,
                              int64_t ldy, float weight_scale, void* workspace, int64_t workspace_bytes,
                              hipStream_t stream) {
  int32_t st = check_gemm_matrix(M, K);
  if (st != FP8LIN_OK) return st;
  if (K >= kMaxF32K) return FP8LIN_EUNSUPPORTED;
  if (K == 0 || (M > 0 && (x_f32 == nullptr || workspace == nullptr))) return FP8LIN_EINVAL;
  if ((st = check_output(qw, y_f32, N, ldy, M)) != FP8LIN_OK) return st;
  if (!aligned16(x_f32) || !aligned16(workspace)) return FP8LIN_ELAYOUT;
  if (!scale_ok(weight_scale)) return FP8LIN_ESCALE;
  if (M == 0) return FP8LIN_OK;
  if (workspace_bytes < fp8lin_w8a16_f32_workspace_bytes(M, K)) return FP8LIN_EINVAL;
  GemmArgs a{};
  a.x = workspace;
  a.m = (int32_t)M;
  a.k = (int32_t)K;
  a.xk = (int32_t)(3 * ((K + 63) / 64 * 64));
  a.ngroups = 1;
  a.g[0].w = static_cast<const uint8_t*>(qw);
  a.g[0].y = y_f32;
  a.g[0].n = (int32_t)N;
  a.g[0].ldy = (int32_t)ldy;
  a.g[0].alpha = weight_scale;
  if ((st = finish_plan(a)) != FP8LIN_OK) return st;
  count_launch(FP8LIN_KERNEL_SPLIT);
  count_launch(FP8LIN_KERNEL_GEMM_W8A16);
  hipError_t e = fp8lin::launch_split3(static_cast<const float*>(x_f32), workspace, M, K, stream);
  if (e != hipSuccess) return FP8LIN_EHIP;
  return hip_status(fp8lin::launch_gemm_w8a16(a, fp8lin::kW16F32, stream));
}

int32_t fp8lin_qkv_shared(const void* x_bf16, int64_t M, int64_t K, int32_t nproj, const void* const qw[],
                          const int64_t n_out[], const float weight_scale[], const float input_scale[],
                          void* const y_bf16[], void* qx_workspace, int32_t mode, hipStream_t stream) {
  if (qw == nullptr || n_out == nullptr || weight_scale == nullptr || input_scale == nullptr || y_bf16 == nullptr)
    return FP8LIN_EINVAL;
  if (nproj < 1 || nproj > fp8lin::kMaxGroups) return FP8LIN_EINVAL;
  if (mode != FP8LIN_MODE_W8A8 && mode != FP8LIN_MODE_W8A16) return FP8LIN_EINVAL;
  int32_t st = check_gemm_matrix(M, K);
  if (st != FP8LIN_OK) return st;
  if (K == 0 || (M > 0 && x_bf16 == nullptr)) return FP8LIN_EINVAL;
  if (!aligned16(x_bf16)) return FP8LIN_ELAYOUT;
  if (mode == FP8LIN_MODE_W8A8) {
    if (M > 0 && qx_workspace == nullptr) return FP8LIN_EINVAL;
    if (!aligned16(qx_workspace)) return FP8LIN_ELAYOUT;
  }
  uint32_t s0;
  std::memcpy(&s0, &input_scale[0], sizeof s0);
  for (int i = 0; i < nproj; ++i) {
    if ((st = check_output(qw[i], y_bf16[i], n_out[i], n_out[i], M)) != FP8LIN_OK) return st;
    uint32_t si;
    std::memcpy(&si, &input_scale[i], sizeof si);
    if (si != s0) return FP8LIN_ESCALE;  // the group must share one calibrated input scale
    if (!scale_ok(weight_scale[i])) return FP8LIN_ESCALE;
  }
  if (!scale_ok(input_scale[0])) return FP8LIN_ESCALE;
  GemmArgs a{};
  a.x = mode == FP8LIN_MODE_W8A8 ? qx_workspace : x_bf16;
  a.m = (int32_t)M;
  a.k = (int32_t)K;
  a.ngroups = nproj;
  for (int i = 0; i < nproj; ++i) {
    a.g[i].w = static_cast<const uint8_t*>(qw[i]);
    a.g[i].y = y_bf16[i];
    a.g[i].n = (int32_t)n_out[i];
    a.g[i].ldy = (int32_t)n_out[i];
    a.g[i].alpha = mode == FP8LIN_MODE_W8A8 ? input_scale[0] * weight_scale[i] : weight_scale[i];
    if (!std::isfinite(a.g[i].alpha) || a.g[i].alpha == 0.0f) return FP8LIN_ESCALE;
  }
  if ((st = finish_plan(a)) != FP8LIN_OK) return st;
  if (M == 0) return FP8LIN_OK;
  if (mode == FP8LIN_MODE_W8A8) {
    count_launch(FP8LIN_KERNEL_QUANTIZE);
    if ((st = hip_status(fp8lin::launch_quantize(x_bf16, qx_workspace, M * K, input_scale[0], stream))) != FP8LIN_OK)
      return st;
    count_launch(FP8LIN_KERNEL_GEMM_W8A8);
    return hip_status(fp8lin::launch_gemm_w8a8(a, stream));
  }
  count_launch(FP8LIN_KERNEL_GEMM_W8A16);
  return hip_status(fp8lin::launch_gemm_w8a16(a, fp8lin::kW16Bf16, stream));
}

int32_t fp8lin_gemm_w8a8_group(const void* qx, int64_t M, int64_t K, int32_t nproj, const void* const qw[],
                               const int64_t n_out[], const float weight_scale[], float input_scale,
                               void* const y_bf16[], hipStream_t stream) {
  if (qw == nullptr || n_out == nullptr || weight_scale == nullptr || y_bf16 == nullptr) return FP8LIN_EINVAL;
  if (nproj < 1 || nproj > fp8lin::kMaxGroups) return FP8LIN_EINVAL;
  int32_t st = check_gemm_matrix(M, K);
  if (st != FP8LIN_OK) return st;
  if (K == 0 || (M > 0 && qx == nullptr)) return FP8LIN_EINVAL;
  if (!aligned16(qx)) return FP8LIN_ELAYOUT;
  if (!scale_ok(input_scale)) return FP8LIN_ESCALE;
  GemmArgs a{};
  a.x = qx;
  a.m = (int32_t)M;
  a.k = (int32_t)K;
  a.ngroups = nproj;
  for (int i = 0; i < nproj; ++i) {
    if ((st = check_output(qw[i], y_bf16[i], n_out[i], n_out[i], M)) != FP8LIN_OK) return st;
    if (!scale_ok(weight_scale[i])) return FP8LIN_ESCALE;
    a.g[i].w = static_cast<const uint8_t*>(qw[i]);
    a.g[i].y = y_bf16[i];
    a.g[i].n = (int32_t)n_out[i];
    a.g[i].ldy = (int32_t)n_out[i];
    a.g[i].alpha = input_scale * weight_scale[i];
    if (!std::isfinite(a.g[i].alpha) || a.g[i].alpha == 0.0f) return FP8LIN_ESCALE;
  }
  if ((st = finish_plan(a)) != FP8LIN_OK) return st;
  if (M == 0) return FP8LIN_OK;
  count_launch(FP8LIN_KERNEL_GEMM_W8A8);
  return hip_status(fp8lin::launch_gemm_w8a8(a, stream));
}

int32_t fp8lin_gemm_w8a8_splitk_choice(int64_t M, int64_t N, int64_t K) {
  // A split helped only where the 256 x 256 tiles fill at most half the device (1024 x 4096 x 4096 with
  // 2 slices: 0.96-1.02 PFLOP/s against 0.86-0.94 unsplit). There the unsplit call now runs 128 x 128
  // tiles instead (1.75-1.79 PFLOP/s), which beat every split; elsewhere no split helps.
  (void)M;
  (void)N;
  (void)K;
  return 1;
}

}  // extern "C"

namespace {

// Checks of a split-K W8A8 call (splits 2 or 4) apart from its workspace.
int32_t check_splitk_w8a8(const void* qx, const void* qw, void* y_bf16, int64_t M, int64_t N, int64_t K, int64_t ldy,
                          float input_scale, float weight_scale, int32_t splits) {
  int32_t st = check_gemm_matrix(M, K);
  if (st != FP8LIN_OK) return st;
  if (K == 0 || (M > 0 && qx == nullptr)) return FP8LIN_EINVAL;
  if ((st = check_output(qw, y_bf16, N, ldy, M)) != FP8LIN_OK) return st;
  if (!aligned16(qx)) return FP8LIN_ELAYOUT;
  if (K % (16 * splits) != 0) return FP8LIN_ELAYOUT;
  if (!scale_ok(input_scale) || !scale_ok(weight_scale)) return FP8LIN_ESCALE;
  const float alpha = input_scale * weight_scale;
  if (!std::isfinite(alpha) || alpha == 0.0f) return FP8LIN_ESCALE;
  if (M * N >= kMaxElems) return FP8LIN_EUNSUPPORTED;
  return FP8LIN_OK;
}

// The split-K W8A8 launches on a checked call with M > 0 and a workspace of
// at least splits * M * N * 4 bytes.
int32_t launch_splitk_w8a8(const void* qx, const void* qw, void* y_bf16, int64_t M, int64_t N, int64_t K, int64_t ldy,
                           float input_scale, float weight_scale, int32_t splits, void* workspace,
                           hipStream_t stream) {
  const float alpha = input_scale * weight_scale;
  int32_t st;
  GemmArgs a{};
  a.x = qx;
  a.m = (int32_t)M;
  a.k = (int32_t)K;
  a.ks = (int32_t)(K / splits);
  a.ngroups = splits;
  for (int sp = 0; sp < splits; ++sp) {
    a.g[sp].w = static_cast<const uint8_t*>(qw);
    a.g[sp].y = static_cast<uint8_t*>(workspace) + (int64_t)sp * M * N * 4;
    a.g[sp].n = (int32_t)N;
    a.g[sp].ldy = (int32_t)N;
    a.g[sp].alpha = 1.0f;
    a.g[sp].koff = sp * a.ks;
  }
  if ((st = finish_plan(a)) != FP8LIN_OK) return st;
  count_launch(FP8LIN_KERNEL_GEMM_W8A8);
  count_launch(FP8LIN_KERNEL_SPLITK_REDUCE);
  hipError_t e = fp8lin::launch_gemm_w8a8_splitk(a, stream);
  if (e != hipSuccess) return FP8LIN_EHIP;
  return hip_status(
      fp8lin::launch_splitk_reduce(static_cast<const float*>(workspace), splits, y_bf16, M, N, ldy, alpha, stream));
}

}  // namespace

extern "C" {

int32_t fp8lin_gemm_w8a8_splitk(const void* qx, const void* qw, void* y_bf16, int64_t M, int64_t N, int64_t K,
                                int64_t ldy, float input_scale, float weight_scale, int32_t splits, void* workspace,
                                int64_t workspace_bytes, hipStream_t stream) {
  if (splits != 1 && splits != 2 && splits != 4) return FP8LIN_EINVAL;
  if (splits == 1)
    return fp8lin_gemm_w8a8(qx, qw, y_bf16, M, N, K, ldy, input_scale, weight_scale, stream);
  int32_t st = check_splitk_w8a8(qx, qw, y_bf16, M, N, K, ldy, input_scale, weight_scale, splits);
  if (st != FP8LIN_OK) return st;
  if (!aligned16(workspace)) return FP8LIN_ELAYOUT;
  if (M == 0) return FP8LIN_OK;
  if (workspace == nullptr || workspace_bytes < (int64_t)splits * M * N * 4) return FP8LIN_EINVAL;
  return launch_splitk_w8a8(qx, qw, y_bf16, M, N, K, ldy, input_scale, weight_scale, splits, workspace, stream);
}

int32_t fp8lin_gemm_w8a8_splitk_noalloc(const void* qx, const void* qw, void* y_bf16, int64_t M, int64_t N, int64_t K,
                                        int64_t ldy, float input_scale, float weight_scale, int32_t splits,
                                        hipStream_t stream) {
  if (splits != 1 && splits != 2 && splits != 4) return FP8LIN_EINVAL;
  if (splits == 1)
    return fp8lin_gemm_w8a8(qx, qw, y_bf16, M, N, K, ldy, input_scale, weight_scale, stream);
  int32_t st = check_splitk_w8a8(qx, qw, y_bf16, M, N, K, ldy, input_scale, weight_scale, splits);
  if (st != FP8LIN_OK) return st;
  if (M == 0) return FP8LIN_OK;
  if ((int64_t)splits * M * N * 4 > FP8LIN_SCRATCH_BYTES) return FP8LIN_EUNSUPPORTED;
  void* scratch = nullptr;
  if (fp8lin::device_scratch(&scratch) != hipSuccess) return FP8LIN_EHIP;
  return launch_splitk_w8a8(qx, qw, y_bf16, M, N, K, ldy, input_scale, weight_scale, splits, scratch, stream);
}

int32_t fp8lin_gemm_w8a16_splitk_choice(int64_t M, int64_t N, int64_t K) {
  // As for W8A8: where slices helped (1024 x 4096 x 4096: 0.68-0.72 PFLOP/s with 4 slices against 0.40
  // unsplit) the unsplit call now runs 128 x 128 tiles (1.0 PFLOP/s).
  (void)M;
  (void)N;
  (void)K;
  return 1;
}

int32_t fp8lin_gemm_w8a16_splitk(const void* x, int32_t x_dtype, const void* qw, void* y_bf16, int64_t M, int64_t N,
                                 int64_t K, int64_t ldy, float weight_scale, int32_t splits, void* workspace,
                                 int64_t workspace_bytes, hipStream_t stream) {
  if (splits != 1 && splits != 2 && splits != 4) return FP8LIN_EINVAL;
  if (x_dtype == FP8LIN_DT_E4M3 || x_dtype == FP8LIN_DT_F32) return FP8LIN_EDTYPE;
  if (x_dtype != FP8LIN_DT_BF16 && x_dtype != FP8LIN_DT_F16) return FP8LIN_EINVAL;
  if (splits == 1) return fp8lin_gemm_w8a16(x, x_dtype, qw, y_bf16, M, N, K, ldy, weight_scale, stream);
  if (x_dtype != FP8LIN_DT_BF16) return FP8LIN_EUNSUPPORTED;  // the reduction writes bf16
  int32_t st = check_gemm_matrix(M, K);
  if (st != FP8LIN_OK) return st;
  if (K == 0 || (M > 0 && x == nullptr)) return FP8LIN_EINVAL;
  if ((st = check_output(qw, y_bf16, N, ldy, M)) != FP8LIN_OK) return st;
  if (!aligned16(x) || !aligned16(workspace)) return FP8LIN_ELAYOUT;
  if (K % (16 * splits) != 0) return FP8LIN_ELAYOUT;
  if (!scale_ok(weight_scale)) return FP8LIN_ESCALE;
  if (M == 0) return FP8LIN_OK;
  if (M * N >= kMaxElems) return FP8LIN_EUNSUPPORTED;
  if (workspace == nullptr || workspace_bytes < (int64_t)splits * M * N * 4) return FP8LIN_EINVAL;
  GemmArgs a{};
  a.x = x;
  a.m = (int32_t)M;
  a.k = (int32_t)K;
  a.ks = (int32_t)(K / splits);
  a.ngroups = splits;
  for (int sp = 0; sp < splits; ++sp) {
    a.g[sp].w = static_cast<const uint8_t*>(qw);
    a.g[sp].y = static_cast<uint8_t*>(workspace) + (int64_t)sp * M * N * 4;
    a.g[sp].n = (int32_t)N;
    a.g[sp].ldy = (int32_t)N;
    a.g[sp].alpha = 1.0f;
    a.g[sp].koff = sp * a.ks;
  }
  if ((st = finish_plan(a)) != FP8LIN_OK) return st;
  count_launch(FP8LIN_KERNEL_GEMM_W8A16);
  count_launch(FP8LIN_KERNEL_SPLITK_REDUCE);
  hipError_t e = fp8lin::launch_gemm_w8a16_splitk(a, stream);
  if (e != hipSuccess) return FP8LIN_EHIP;
  return hip_status(fp8lin::launch_splitk_reduce(static_cast<const float*>(workspace), splits, y_bf16, M, N, ldy,
                                                 weight_scale, stream));
}

int32_t fp8lin_qkv_w8a8_norm_rope(const void* qx, int64_t M, int64_t K, int32_t nproj, const void* const qw[],
                                  const int64_t n_out[], const float weight_scale[], float input_scale,
                                  void* const y_bf16[], const void* q_norm_weight, const void* k_norm_weight,
                                  const float* cos, const float* sin, float eps, hipStream_t stream) {
  if (qw == nullptr || n_out == nullptr || weight_scale == nullptr || y_bf16 == nullptr) return FP8LIN_EINVAL;
  if (nproj < 2 || nproj > 3) return FP8LIN_EINVAL;
  if (!std::isfinite(eps) || !(eps > 0.0f)) return FP8LIN_EINVAL;
  int32_t st = check_gemm_matrix(M, K);
  if (st != FP8LIN_OK) return st;
  if (K == 0 || (M > 0 && (qx == nullptr || cos == nullptr || sin == nullptr))) return FP8LIN_EINVAL;
  if (!aligned16(qx) || !aligned16(cos) || !aligned16(sin) || !aligned16(q_norm_weight) ||
      !aligned16(k_norm_weight))
    return FP8LIN_ELAYOUT;
  if (!scale_ok(input_scale)) return FP8LIN_ESCALE;
  GemmArgs a{};
  a.x = qx;
  a.m = (int32_t)M;
  a.k = (int32_t)K;
  a.ngroups = nproj;
  for (int i = 0; i < nproj; ++i) {
    if ((st = check_output(qw[i], y_bf16[i], n_out[i], n_out[i], M)) != FP8LIN_OK) return st;
    if (i < 2 && n_out[i] % 128 != 0) return FP8LIN_ELAYOUT;  // whole heads of 128
    if (!scale_ok(weight_scale[i])) return FP8LIN_ESCALE;
    a.g[i].w = static_cast<const uint8_t*>(qw[i]);
    a.g[i].y = y_bf16[i];
    a.g[i].n = (int32_t)n_out[i];
    a.g[i].ldy = (int32_t)n_out[i];
    a.g[i].alpha = input_scale * weight_scale[i];
    if (!std::isfinite(a.g[i].alpha) || a.g[i].alpha == 0.0f) return FP8LIN_ESCALE;
  }
  a.nr_w[0] = static_cast<const uint16_t*>(q_norm_weight);
  a.nr_w[1] = static_cast<const uint16_t*>(k_norm_weight);
  a.nr_cos = cos;
  a.nr_sin = sin;
  a.nr_eps = eps;
  if ((st = finish_plan(a)) != FP8LIN_OK) return st;
  if (M == 0) return FP8LIN_OK;
  count_launch(FP8LIN_KERNEL_GEMM_W8A8);
  return hip_status(fp8lin::launch_gemm_w8a8_norm_rope(a, stream));
}

int32_t fp8lin_gate_up_swiglu_w8a8(const void* qx, int64_t M, int64_t K, const void* qw_gate, const void* qw_up,
                                   int64_t I, float input_scale, float gate_scale, float up_scale, float out_scale,
                                   void* h_e4m3, hipStream_t stream) {
  int32_t st = check_gemm_matrix(M, K);
  if (st != FP8LIN_OK) return st;
  if (K == 0 || (M > 0 && (qx == nullptr || h_e4m3 == nullptr))) return FP8LIN_EINVAL;
  if (qw_gate == nullptr || qw_up == nullptr || I <= 0) return FP8LIN_EINVAL;
  if (I >= kMaxGemmDim) return FP8LIN_EUNSUPPORTED;
  if (I % 16 != 0) return FP8LIN_ELAYOUT;
  if (!aligned16(qx) || !aligned16(qw_gate) || !aligned16(qw_up) || !aligned16(h_e4m3)) return FP8LIN_ELAYOUT;
  if (!scale_ok(input_scale) || !scale_ok(gate_scale) || !scale_ok(up_scale) || !scale_ok(out_scale))
    return FP8LIN_ESCALE;
  const float ag = input_scale * gate_scale, au = input_scale * up_scale;
  if (!std::isfinite(ag) || ag == 0.0f || !std::isfinite(au) || au == 0.0f) return FP8LIN_ESCALE;
  if (M == 0) return FP8LIN_OK;
  GemmArgs a{};
  a.x = qx;
  a.m = (int32_t)M;
  a.k = (int32_t)K;
  a.ngroups = 1;
  a.out_rs = 1.0f / out_scale;
  a.g[0].w = static_cast<const uint8_t*>(qw_gate);
  a.g[0].y = h_e4m3;
  a.g[0].n = (int32_t)I;
  a.g[0].ldy = (int32_t)I;
  a.g[0].alpha = ag;
  a.g[1].w = static_cast<const uint8_t*>(qw_up);
  a.g[1].n = (int32_t)I;
  a.g[1].alpha = au;
  const int64_t tiles = ((M + fp8lin::kTileM - 1) / fp8lin::kTileM) * ((I + fp8lin::kTileN / 2 - 1) / (fp8lin::kTileN / 2));
  if (tiles >= (int64_t(1) << 31)) return FP8LIN_EUNSUPPORTED;
  fp8lin::gate_up_plan(a);
  count_launch(FP8LIN_KERNEL_GATE_UP_SWIGLU);
  return hip_status(fp8lin::launch_gate_up_swiglu(a, false, false, stream));
}

int32_t fp8lin_gate_up_swiglu_w8a16(const void* x_bf16, int32_t x_dtype, int64_t M, int64_t K, const void* qw_gate,
                                    const void* qw_up, int64_t I, float gate_scale, float up_scale, void* h_bf16,
                                    hipStream_t stream) {
  if (x_dtype == FP8LIN_DT_E4M3 || x_dtype == FP8LIN_DT_F32) return FP8LIN_EDTYPE;
  if (x_dtype != FP8LIN_DT_BF16 && x_dtype != FP8LIN_DT_F16) return FP8LIN_EINVAL;
  int32_t st = check_gemm_matrix(M, K);
  if (st != FP8LIN_OK) return st;
  if (K == 0 || (M > 0 && (x_bf16 == nullptr || h_bf16 == nullptr))) return FP8LIN_EINVAL;
  if (qw_gate == nullptr || qw_up == nullptr || I <= 0) return FP8LIN_EINVAL;
  if (I >= kMaxGemmDim) return FP8LIN_EUNSUPPORTED;
  if (I % 16 != 0) return FP8LIN_ELAYOUT;
  if (!aligned16(x_bf16) || !aligned16(qw_gate) || !aligned16(qw_up) || !aligned16(h_bf16)) return FP8LIN_ELAYOUT;
  if (!scale_ok(gate_scale) || !scale_ok(up_scale)) return FP8LIN_ESCALE;
  if (M == 0) return FP8LIN_OK;
  GemmArgs a{};
  a.x = x_bf16;
  a.m = (int32_t)M;
  a.k = (int32_t)K;
  a.ngroups = 1;
  a.out_rs = 1.0f;
  a.g[0].w = static_cast<const uint8_t*>(qw_gate);
  a.g[0].y = h_bf16;
  a.g[0].n = (int32_t)I;
  a.g[0].ldy = (int32_t)I;
  a.g[0].alpha = gate_scale;
  a.g[1].w = static_cast<const uint8_t*>(qw_up);
  a.g[1].n = (int32_t)I;
  a.g[1].alpha = up_scale;
  const int64_t tiles = ((M + fp8lin::kTileM - 1) / fp8lin::kTileM) * ((I + fp8lin::kTileN / 2 - 1) / (fp8lin::kTileN / 2));
  if (tiles >= (int64_t(1) << 31)) return FP8LIN_EUNSUPPORTED;
  fp8lin::gate_up_plan(a);
  count_launch(FP8LIN_KERNEL_GATE_UP_SWIGLU);
  return hip_status(fp8lin::launch_gate_up_swiglu(a, true, x_dtype == FP8LIN_DT_F16, stream));
}

int32_t fp8lin_swiglu_2in_quant(const void* gate_bf16, const void* up_bf16, void* out, int32_t out_dtype, int64_t rows,
                                int64_t cols, float out_scale, hipStream_t stream) {
  if (out_dtype != FP8LIN_DT_E4M3 && out_dtype != FP8LIN_DT_BF16) return FP8LIN_EINVAL;
  int32_t st = check_matrix(rows, cols);
  if (st != FP8LIN_OK) return st;
  const bool fp8_out = out_dtype == FP8LIN_DT_E4M3;
  if (fp8_out && !scale_ok(out_scale)) return FP8LIN_ESCALE;
  if (rows == 0 || cols == 0) return FP8LIN_OK;  // empty: pointers may be NULL
  if (gate_bf16 == nullptr || up_bf16 == nullptr || out == nullptr) return FP8LIN_EINVAL;
  if (!aligned16(gate_bf16) || !aligned16(up_bf16) || !aligned16(out)) return FP8LIN_ELAYOUT;
  count_launch(FP8LIN_KERNEL_SWIGLU);
  return hip_status(fp8lin::launch_swiglu(gate_bf16, up_bf16, out, false, fp8_out, rows * cols, out_scale, stream));
}

int32_t fp8lin_swiglu_2in(const void* gate, const void* up, int32_t in_dtype, void* out, int32_t out_dtype,
                          int64_t rows, int64_t cols, float out_scale, hipStream_t stream) {
  const auto known = [](int32_t d) {
    return d == FP8LIN_DT_BF16 || d == FP8LIN_DT_E4M3 || d == FP8LIN_DT_F16 || d == FP8LIN_DT_F32;
  };
  if (!known(in_dtype) || !known(out_dtype)) return FP8LIN_EINVAL;
  if (in_dtype != FP8LIN_DT_BF16 && in_dtype != FP8LIN_DT_F16) return FP8LIN_EDTYPE;
  if (out_dtype != FP8LIN_DT_E4M3 && out_dtype != in_dtype) return FP8LIN_EDTYPE;
  int32_t st = check_matrix(rows, cols);
  if (st != FP8LIN_OK) return st;
  const bool fp8_out = out_dtype == FP8LIN_DT_E4M3;
  if (fp8_out && !scale_ok(out_scale)) return FP8LIN_ESCALE;
  if (rows == 0 || cols == 0) return FP8LIN_OK;  // empty: pointers may be NULL
  if (gate == nullptr || up == nullptr || out == nullptr) return FP8LIN_EINVAL;
  if (!aligned16(gate) || !aligned16(up) || !aligned16(out)) return FP8LIN_ELAYOUT;
  count_launch(FP8LIN_KERNEL_SWIGLU);
  return hip_status(
      fp8lin::launch_swiglu(gate, up, out, in_dtype == FP8LIN_DT_F16, fp8_out, rows * cols, out_scale, stream));
}

int32_t fp8lin_qk_norm_rope(const void* q, const void* k, void* q_out, void* k_out, int64_t tokens, int32_t q_heads,
                            int32_t k_heads, int32_t head_dim, const void* q_weight, const void* k_weight,
                            const float* cos, const float* sin, float eps, hipStream_t stream) {
  if (tokens < 0 || q_heads <= 0 || k_heads < 0) return FP8LIN_EINVAL;
  if (!std::isfinite(eps) || !(eps > 0.0f)) return FP8LIN_EINVAL;
  if (head_dim != 64 && head_dim != 128) return FP8LIN_EUNSUPPORTED;
  const int64_t heads = (int64_t)q_heads + k_heads;
  if (tokens > kMaxRows || heads * head_dim >= kMaxK || tokens * heads * head_dim >= kMaxElems)
    return FP8LIN_EUNSUPPORTED;
  if (tokens == 0) return FP8LIN_OK;
  if (q == nullptr || q_out == nullptr || cos == nullptr || sin == nullptr) return FP8LIN_EINVAL;
  if (k_heads > 0 && (k == nullptr || k_out == nullptr)) return FP8LIN_EINVAL;
  if (!aligned16(q) || !aligned16(q_out) || !aligned16(k) || !aligned16(k_out) || !aligned16(cos) ||
      !aligned16(sin) || !aligned16(q_weight) || !aligned16(k_weight))
    return FP8LIN_ELAYOUT;
  count_launch(FP8LIN_KERNEL_QK_NORM_ROPE);
  return hip_status(fp8lin::launch_qk_norm_rope(q, q_out, q_heads, q_weight, k, k_out, k_heads, k_weight, tokens,
                                                head_dim, cos, sin, eps, stream));
}

int32_t fp8lin_policy_validate(const fp8lin_policy* p) {
  if (p == nullptr) return FP8LIN_EINVAL;
  if ((p->present_mask & FP8LIN_PF_UNKNOWN_FIELD) != 0) return FP8LIN_EPOLICY;
  if ((p->present_mask & FP8LIN_PF_ALL) != FP8LIN_PF_ALL) return FP8LIN_EPOLICY;
  if (p->schema_version != 1) return FP8LIN_EPOLICY;
  if (p->type != FP8LIN_POLICY_TYPE_FIRST_LAST_STEPS) return FP8LIN_EPOLICY;
  if (p->index_space != FP8LIN_POLICY_INDEX_SCHEDULER_STEP) return FP8LIN_EPOLICY;
  if (p->default_mode != FP8LIN_MODE_W8A8) return FP8LIN_EPOLICY;
  if (p->overlap != FP8LIN_POLICY_OVERLAP_A16) return FP8LIN_EPOLICY;
  if (p->first_steps < 0 || p->last_steps < 0) return FP8LIN_EPOLICY;
  if (p->reasoner_mode != FP8LIN_MODE_W8A8 && p->reasoner_mode != FP8LIN_MODE_W8A16) return FP8LIN_EPOLICY;
  return FP8LIN_OK;
}

int32_t fp8lin_step_policy(const fp8lin_policy* p, int32_t tower, int32_t step, int32_t num_steps,
                           int32_t* mode_out) {
  if (mode_out == nullptr) return FP8LIN_EINVAL;
  if (tower != FP8LIN_TOWER_GENERATION && tower != FP8LIN_TOWER_REASONER) return FP8LIN_EINVAL;
  if (num_steps < 1 || step < 0 || step >= num_steps) return FP8LIN_EINVAL;
  if (p == nullptr) {
    *mode_out = FP8LIN_MODE_W8A8;
    return FP8LIN_OK;
  }
  const int32_t st = fp8lin_policy_validate(p);
  if (st != FP8LIN_OK) return st;
  if (tower == FP8LIN_TOWER_REASONER) {
    *mode_out = p->reasoner_mode;
    return FP8LIN_OK;
  }
  if (num_steps == 1) {
    *mode_out = FP8LIN_MODE_W8A8;
    return FP8LIN_OK;
  }
  const bool first = step < p->first_steps;
  const bool last = (int64_t)step >= (int64_t)num_steps - (int64_t)p->last_steps;
  *mode_out = (first || last) ? FP8LIN_MODE_W8A16 : FP8LIN_MODE_W8A8;
  return FP8LIN_OK;
}

const char* fp8lin_strerror(int32_t status) {
  switch (status) {
    case FP8LIN_OK: return "success";
    case FP8LIN_EINVAL: return "invalid argument (null pointer, negative size or unknown enum value)";
    case FP8LIN_ELAYOUT: return "unsupported layout (alignment, divisibility or leading dimension)";
    case FP8LIN_EDTYPE: return "activation dtype not accepted by this call";
    case FP8LIN_ESCALE: return "invalid scale, or input scales of a shared group differ";
    case FP8LIN_EPOLICY: return "invalid diffusion step policy";
    case FP8LIN_EUNSUPPORTED: return "size beyond the supported limits";
    case FP8LIN_EHIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

int64_t fp8lin_launch_count(int32_t kind) {
  if (kind < 0 || kind >= FP8LIN_KERNEL_KINDS) return -1;
  return g_launches[kind].load(std::memory_order_relaxed);
}

}  // extern "C"
