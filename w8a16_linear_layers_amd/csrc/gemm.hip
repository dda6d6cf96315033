// Grouped static-FP8 GEMMs on the gfx950 matrix cores.
//
//   W8A8  ([CF-157] "Verification", a real FP8 x FP8 GEMM):
//     y[m, n] = bf16( sum_k qx[m, k] qw[n, k] * (s_in * s_w) )
//     v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3, float32 accumulate).
//   W8A16 ([TRT-17476] "Denoising-step activation precision", same resident
//   FP8 weight, 16-bit activation, no dequantized weight copy):
//     y[m, n] = bf16( sum_k x[m, k] dec(qw[n, k]) * s_w )
//     The E4M3 weight tile is staged in LDS at one byte per element and
//     converted exactly to bf16 (v_cvt_scalef32_pk_bf16_fp8, scale 1) on its
//     way to v_mfma_f32_32x32x16_bf16.
//
// Both kernels share one structure:
//   * A workgroup of 4 waves owns a 256 (M) x 256 (N) output tile; wave
//     (wm, wn) owns the 128 x 128 quarter (wm, wn) as 4 x 4 blocks of 32 x 32.
//   * The weight is the MFMA "A" operand and the activation the "B" operand,
//     so the accumulator D[n][m] gives every lane four consecutive n of one
//     output row: the epilogue writes 8-byte bf16 quads.
//   * K advances in stages of 64 elements. Global memory is copied straight
//     into LDS by global_load_lds_dwordx4 (no VGPR round trip), several
//     stages ahead (4 buffers for W8A8, 3 for W8A16), with one
//     s_waitcnt vmcnt(n) + s_barrier per stage.
//   * LDS rows are 64 B (E4M3) or 128 B (bf16) with the 16-byte chunks of a
//     row permuted by an XOR of the row index, chosen so that the lanes of a
//     ds_read_b128 phase hit distinct banks for 32- or 64-bank LDS.
//   * The copies are buffer loads against a per-tile resource: rows beyond
//     M or N fall outside it and K chunks beyond K get an out-of-range offset,
//     and both read as zero, so edge tiles need no other masking until the
//     store.
//   * Tiles of all groups form one index space, remapped so that the
//     workgroups dispatched to one XCD (ids congruent mod 8) take a
//     contiguous run of tiles, rasterized in bands of 8 M-tiles for L2 reuse.
#include "internal.h"

namespace fp8lin {

void gemm_plan(GemmArgs& a) {
  a.tiles_m = (a.m + kTileM - 1) / kTileM;
  int32_t t = 0;
  for (int i = 0; i < a.ngroups; ++i) {
    a.g[i].tiles_n = (a.g[i].n + kTileN - 1) / kTileN;
    a.g[i].tile_begin = t;
    t += a.tiles_m * a.g[i].tiles_n;
  }
  a.total_tiles = t;
}

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kBK = 64;          // K elements per stage
constexpr int kStages8 = 4;      // W8A8 LDS buffers: 4 x 32 KiB
constexpr int kStages16 = 3;     // W8A16 LDS buffers: 3 x 48 KiB
constexpr int kXcds = 8;
constexpr int kBandM = 8;        // M-tiles per raster band


__shared__ __attribute__((aligned(16))) uint8_t lds_w8[kStages8][kTileN * kBK];   // E4M3 weight tiles
__shared__ __attribute__((aligned(16))) uint8_t lds_x8[kStages8][kTileM * kBK];   // E4M3 activation tiles
__shared__ __attribute__((aligned(16))) uint8_t lds_w16[kStages16][kTileN * kBK];      // E4M3 weight tiles
__shared__ __attribute__((aligned(16))) uint8_t lds_x16[kStages16][kTileM * kBK * 2];  // bf16 activation tiles

// Permutation of the four 16-byte chunks of a 64-byte row, and of the eight
// chunks of a 128-byte row (XOR with a per-row constant: a bijection).
__device__ __forceinline__ int swz4(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }
__device__ __forceinline__ int swz8(int r) { return (r & 7) ^ ((r >> 3) & 1); }

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over `bytes` bytes at `base` (stride 0: raw byte offsets).
// Loads at offsets >= bytes return zero, which pads edge tiles.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = (int32_t)(uint32_t)b;
  r[1] = (int32_t)((uint32_t)(b >> 32) & 0xffffu);
  r[2] = (int32_t)bytes;
  r[3] = 0x00020000;
  return r;
}

constexpr uint32_t kOutOfRange = 0x80000000u;  // an offset beyond every resource

// One 16-byte global -> LDS copy per lane (buffer_load_dwordx4 ... lds):
// lane l reads resource bytes [voff + soff, +16) and writes LDS bytes
// [lds + 16 l, +16), lds being wave-uniform. Issued as inline asm so that
// the compiler does not add a vmcnt(0) before every LDS read (it cannot
// tell the stage buffers apart); the waits are explicit instead.
__device__ __forceinline__ void dma16(const i32x4& rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff),
               "s"(lds)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>(p);
}

template <int N>
__device__ __forceinline__ void wait_vmem_and_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

struct TileCoord {
  int group;
  int m0;
  int n0;
};

__device__ __forceinline__ TileCoord tile_of(const GemmArgs& a) {
  // XCD-aware remap: block b runs on XCD b % 8; give each XCD a contiguous run.
  const int T = a.total_tiles;
  const int b = blockIdx.x;
  const int xcd = b % kXcds, idx = b / kXcds;
  const int q = T / kXcds, r = T % kXcds;
  const int t = xcd * q + min(xcd, r) + idx;
  int gi = 0;
#pragma unroll
  for (int i = 1; i < kMaxGroups; ++i)
    if (i < a.ngroups && t >= a.g[i].tile_begin) gi = i;
  const int local = t - a.g[gi].tile_begin;
  const int tiles_n = a.g[gi].tiles_n;
  const int per_band = kBandM * tiles_n;
  const int band = local / per_band;
  const int first_m = band * kBandM;
  const int band_m = min(a.tiles_m - first_m, kBandM);
  const int in_band = local - band * per_band;
  TileCoord c;
  c.group = gi;
  c.m0 = (first_m + in_band % band_m) * kTileM;
  c.n0 = (in_band / band_m) * kTileN;
  return c;
}

// Per-thread copy plan of one operand tile. The tile holds 256 rows of 64
// K-elements; chunk position p (16 bytes) = j * 256 + tid holds logical
// chunk (p % cpr) ^ swizzle(row) of row p / cpr (cpr = chunks per row).
// voff[j] is the byte offset of that chunk inside the tile's resource at
// K = 0; the stage's K offset travels in the scalar offset.
template <int kChunks>  // 4: E4M3 rows of 64 B; 8: bf16 rows of 128 B
struct CopyPlan {
  static constexpr int kPerThread = kChunks;  // 256 rows * kChunks / 256 threads
  i32x4 rsrc;
  uint32_t voff[kPerThread];
  int kchunk[kPerThread];  // first K element of the chunk, relative to the stage

  __device__ __forceinline__ void init(const uint8_t* src, int row0, int rows, int64_t ld_bytes, int tid) {
    const int valid = rows < 256 ? rows : 256;
    rsrc = make_rsrc(src + (int64_t)row0 * ld_bytes, (uint32_t)(valid * ld_bytes));
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int p = j * kThreads + tid;
      const int r = p / kChunks;
      const int c = (p % kChunks) ^ (kChunks == 4 ? swz4(r) : swz8(r));
      voff[j] = (uint32_t)(r * ld_bytes) + (uint32_t)c * 16u;
      kchunk[j] = c * (kChunks == 4 ? 16 : 8);
    }
  }

  // Copy stage `kt` into the LDS tile; chunks at K >= k read as zero.
  __device__ __forceinline__ void copy(const uint8_t* lds_tile, int kt, int k, int tid) const {
    const int wave = tid >> 6;
    const uint32_t base = lds_addr(lds_tile);
    const int k0 = kt * kBK;
    const uint32_t soff = (uint32_t)k0 * (kChunks == 4 ? 1u : 2u);
    const bool tail = k0 + kBK > k;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const uint32_t v = (tail && k0 + kchunk[j] >= k) ? kOutOfRange : voff[j];
      dma16(rsrc, v, soff, __builtin_amdgcn_readfirstlane(base + (j * kThreads + wave * 64) * 16));
    }
  }
};

__device__ __forceinline__ u32x4 lds_chunk(const uint8_t* tile, int byte_offset) {
  return *reinterpret_cast<const u32x4*>(tile + byte_offset);
}

// 32 x 64 E4M3 fragment of rows [row, row+32): lane (r, g) holds logical
// chunks 2g and 2g+1 (32 bytes of K) of row + r.
__device__ __forceinline__ v8i frag_e4m3(const uint8_t* tile, int row, int g) {
  const int s = swz4(row);
  const u32x4 a = lds_chunk(tile, row * 64 + ((2 * g) ^ s) * 16);
  const u32x4 b = lds_chunk(tile, row * 64 + ((2 * g + 1) ^ s) * 16);
  v8i v;
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
  return v;
}

// Store four consecutive bf16 outputs (n .. n+3 of row m).
__device__ __forceinline__ void store_quad(void* y, int64_t ldy, int m, int n, float a, float b, float c, float d) {
  const __bf16 h0 = (__bf16)a, h1 = (__bf16)b, h2 = (__bf16)c, h3 = (__bf16)d;
  u32x2 v;
  v[0] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
  v[1] = (uint32_t)__builtin_bit_cast(uint16_t, h2) | ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16);
  *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(y) + (int64_t)m * ldy + n) = v;
}

// acc[i][j] holds D[n][m] of the 32 x 32 block (n-block i, m-block j):
// lane l, register v -> m = l % 32, n = 8 (v / 4) + 4 (l / 32) + v % 4.
__device__ __forceinline__ void epilogue(const v16f (&acc)[4][4], const GemmGroup& grp, int M, int m_base, int n_base,
                                         int lane) {
  const float alpha = grp.alpha;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m_base + j * 32 + (lane & 31);
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int n = n_base + i * 32 + 8 * t + 4 * (lane >> 5);
        if (n < grp.n)
          store_quad(grp.y, grp.ldy, m, n, acc[i][j][4 * t] * alpha, acc[i][j][4 * t + 1] * alpha,
                     acc[i][j][4 * t + 2] * alpha, acc[i][j][4 * t + 3] * alpha);
      }
    }
  }
}

// Wait until stage `kt + 1` has landed in LDS, given that the loads of at
// most one later stage may still be in flight (8 DMA loads per thread per
// stage), then synchronize the workgroup.
__device__ __forceinline__ void w8a8_wait_next(int kt, int KT) {
  if (kt + 2 < KT)
    wait_vmem_and_barrier<8>();
  else
    wait_vmem_and_barrier<0>();
}

__device__ __forceinline__ void w8a8_frags(int buf, int row_w, int row_x, int g, v8i (&wf)[4], v8i (&xf)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) wf[i] = frag_e4m3(lds_w8[buf], row_w + i * 32, g);
#pragma unroll
  for (int j = 0; j < 4; ++j) xf[j] = frag_e4m3(lds_x8[buf], row_x + j * 32, g);
}

__device__ __forceinline__ void w8a8_mma(v16f (&acc)[4][4], const v8i (&wf)[4], const v8i (&xf)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[i], xf[j], acc[i][j], 0, 0, 0, 0, 0, 0);
}

// Pipeline: stage s is copied into LDS buffer s % 4 three stages ahead; the
// MFMA fragments of stage kt + 1 are read from LDS while the matrix cores
// work on stage kt. The buffer refilled in iteration kt held stage kt - 1,
// whose fragments were read in iteration kt - 2, before the barrier.
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1))) void
gemm_w8a8_kernel(const GemmArgs a) {
  const TileCoord tc = tile_of(a);
  const GemmGroup& grp = a.g[tc.group];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int K = a.k;
  const int KT = (K + kBK - 1) / kBK;
  CopyPlan<4> pw, px;
  pw.init(grp.w, tc.n0, grp.n - tc.n0, K, tid);
  px.init(static_cast<const uint8_t*>(a.x), tc.m0, a.m - tc.m0, K, tid);

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

#pragma unroll
  for (int s = 0; s < kStages8 - 1; ++s) {
    if (s < KT) {
      pw.copy(lds_w8[s], s, K, tid);
      px.copy(lds_x8[s], s, K, tid);
    }
  }

  const int row_w = wn * 128 + (lane & 31);
  const int row_x = wm * 128 + (lane & 31);
  const int g = lane >> 5;

  // stage 0: at most two later stages in flight
  if (KT >= 3)
    wait_vmem_and_barrier<16>();
  else if (KT == 2)
    wait_vmem_and_barrier<8>();
  else
    wait_vmem_and_barrier<0>();
  v8i wa[4], xa[4], wb[4], xb[4];
  w8a8_frags(0, row_w, row_x, g, wa, xa);

  // Stages in pairs: the even one's fragments sit in (wa, xa), the odd
  // one's in (wb, xb). The steady-state loop has no branches besides its
  // back edge (every prefetch it issues exists), so the compiler tracks the
  // LDS-read counters exactly; the last stages drain in a guarded loop. Both
  // loops have a single exit, so the accumulators stay in place; an odd last
  // stage is already in (wa, xa) when they end.
  int kt = 0;
  for (; kt + 5 < KT; kt += 2) {
    wait_vmem_and_barrier<8>();
    pw.copy(lds_w8[(kt + 3) % kStages8], kt + 3, K, tid);
    px.copy(lds_x8[(kt + 3) % kStages8], kt + 3, K, tid);
    w8a8_frags((kt + 1) % kStages8, row_w, row_x, g, wb, xb);
    w8a8_mma(acc, wa, xa);
    wait_vmem_and_barrier<8>();
    pw.copy(lds_w8[kt % kStages8], kt + 4, K, tid);
    px.copy(lds_x8[kt % kStages8], kt + 4, K, tid);
    w8a8_frags((kt + 2) % kStages8, row_w, row_x, g, wa, xa);
    w8a8_mma(acc, wb, xb);
  }
  for (; kt + 1 < KT; kt += 2) {
    w8a8_wait_next(kt, KT);
    if (kt + 3 < KT) {
      const int sb = (kt + 3) % kStages8;
      pw.copy(lds_w8[sb], kt + 3, K, tid);
      px.copy(lds_x8[sb], kt + 3, K, tid);
    }
    w8a8_frags((kt + 1) % kStages8, row_w, row_x, g, wb, xb);
    w8a8_mma(acc, wa, xa);
    if (kt + 2 < KT) {
      w8a8_wait_next(kt + 1, KT);
      if (kt + 4 < KT) {
        const int sb = (kt + 4) % kStages8;
        pw.copy(lds_w8[sb], kt + 4, K, tid);
        px.copy(lds_x8[sb], kt + 4, K, tid);
      }
      w8a8_frags((kt + 2) % kStages8, row_w, row_x, g, wa, xa);
    }
    w8a8_mma(acc, wb, xb);
  }
  if (kt < KT) w8a8_mma(acc, wa, xa);

  epilogue(acc, grp, a.m, tc.m0 + wm * 128, tc.n0 + wn * 128, lane);
}

// Eight exact E4M3 -> bf16 conversions of one dword pair.
__device__ __forceinline__ v8bf dequant8(uint32_t d0, uint32_t d1) {
  const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false);
  const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true);
  const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false);
  const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true);
  v8bf v;
  v[0] = p0[0]; v[1] = p0[1]; v[2] = p1[0]; v[3] = p1[1];
  v[4] = p2[0]; v[5] = p2[1]; v[6] = p3[0]; v[7] = p3[1];
  return v;
}

__device__ __forceinline__ v8bf as_v8bf(u32x4 c) { return __builtin_bit_cast(v8bf, c); }

__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1))) void
gemm_w8a16_kernel(const GemmArgs a) {
  const TileCoord tc = tile_of(a);
  const GemmGroup& grp = a.g[tc.group];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int K = a.k;
  const int KT = (K + kBK - 1) / kBK;
  CopyPlan<4> pw;
  CopyPlan<8> px;
  pw.init(grp.w, tc.n0, grp.n - tc.n0, K, tid);
  px.init(static_cast<const uint8_t*>(a.x), tc.m0, a.m - tc.m0, (int64_t)K * 2, tid);

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

#pragma unroll
  for (int s = 0; s < kStages16 - 1; ++s) {
    if (s < KT) {
      pw.copy(lds_w16[s], s, K, tid);
      px.copy(lds_x16[s], s, K, tid);
    }
  }

  const int row_w = wn * 128 + (lane & 31);
  const int row_x = wm * 128 + (lane & 31);
  const int g = lane >> 5;

  for (int kt = 0; kt < KT; ++kt) {
    // 12 loads per stage per thread
    if (kt + 1 < KT)
      wait_vmem_and_barrier<12>();
    else
      wait_vmem_and_barrier<0>();

    const int next = kt + kStages16 - 1;
    if (next < KT) {
      const int sb = next % kStages16;
      pw.copy(lds_w16[sb], next, K, tid);
      px.copy(lds_x16[sb], next, K, tid);
    }

    const int cb = kt % kStages16;
    // Two halves of the stage: K [0, 32) and [32, 64). In half h, lane group
    // g holds K [32h + 16g, 32h + 16g + 16): weight chunk 2h + g (16 E4M3)
    // and activation chunks 4h + 2g, 4h + 2g + 1 (8 bf16 each); MFMA step
    // 2h + e uses the e-th 8-element half of each.
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v8bf wf[4][2], xf[4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = row_w + i * 32;
        const u32x4 c = lds_chunk(lds_w16[cb], r * 64 + ((2 * h + g) ^ swz4(r)) * 16);
        wf[i][0] = dequant8(c[0], c[1]);
        wf[i][1] = dequant8(c[2], c[3]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = row_x + j * 32;
        xf[j][0] = as_v8bf(lds_chunk(lds_x16[cb], r * 128 + ((4 * h + 2 * g) ^ swz8(r)) * 16));
        xf[j][1] = as_v8bf(lds_chunk(lds_x16[cb], r * 128 + ((4 * h + 2 * g + 1) ^ swz8(r)) * 16));
      }
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[i][e], xf[j][e], acc[i][j], 0, 0, 0);
    }
  }

  epilogue(acc, grp, a.m, tc.m0 + wm * 128, tc.n0 + wn * 128, lane);
}

}  // namespace

hipError_t launch_gemm_w8a8(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(gemm_w8a8_kernel, dim3((unsigned)a.total_tiles), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_w8a16(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(gemm_w8a16_kernel, dim3((unsigned)a.total_tiles), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace fp8lin
