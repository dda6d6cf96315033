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


// One LDS arena per workgroup. W8A8: E4M3 weight stages, then E4M3
// activation stages (16 KiB each). W8A16: E4M3 weight stages (16 KiB), then
// bf16 activation stages (32 KiB). After the K loop the epilogue reuses the
// first 128 KiB as four 32 KiB per-wave output tiles.
constexpr int kStageE4M3 = kTileN * kBK;     // 16 KiB
constexpr int kStageBf16 = kTileM * kBK * 2;  // 32 KiB
constexpr int kLdsW8A8 = 2 * kStages8 * kStageE4M3;
constexpr int kLdsW8A16 = kStages16 * (kStageE4M3 + kStageBf16);
constexpr int kLdsBytes = kLdsW8A8 > kLdsW8A16 ? kLdsW8A8 : kLdsW8A16;
static_assert(kLdsBytes >= 4 * 128 * 256, "epilogue staging needs 128 KiB");
static_assert(kLdsBytes <= 160 * 1024, "gfx950 LDS per workgroup");
__shared__ __attribute__((aligned(16))) uint8_t lds_mem[kLdsBytes];

__device__ __forceinline__ uint8_t* lds_w8(int s) { return lds_mem + s * kStageE4M3; }
__device__ __forceinline__ uint8_t* lds_x8(int s) { return lds_mem + (kStages8 + s) * kStageE4M3; }
__device__ __forceinline__ uint8_t* lds_w16(int s) { return lds_mem + s * kStageE4M3; }
__device__ __forceinline__ uint8_t* lds_x16(int s) { return lds_mem + kStages16 * kStageE4M3 + s * kStageBf16; }

// LDS tile layouts. A ds_read_b128 wave is served 16 lanes per cycle; the
// layouts below keep every MFMA fragment read free of bank conflicts for
// the lane groupings a 64-bank LDS may use (16 consecutive lanes, lanes
// {8k..8k+7} with {8k+32..8k+39}, or lanes sharing lane-index bits 1 and
// 4 -- the grouping the LDS bank-conflict counters of the first layout
// pointed to), for every read pattern of both kernels.
//   E4M3 tiles, 64-byte rows: logical row r sits in physical row
//     row64(r) = r ^ (bit3(r) << 1)   (a swap inside groups of 4 rows)
//   and its 16-byte chunk c in physical chunk c ^ swz4(r).
//   bf16 tiles, 128-byte rows: chunk c of row r in physical chunk c ^ swz8(r).
// All three are involutions / XORs, hence bijections on the tile.
__device__ __forceinline__ int row64(int r) { return r ^ (((r >> 3) & 1) << 1); }
__device__ __forceinline__ int swz4(int r) { return ((r >> 2) & 1) | ((((r >> 1) ^ (r >> 2)) & 1) << 1); }
__device__ __forceinline__ int swz8(int r) {
  return ((r >> 2) & 1) | (((r >> 1) & 1) << 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 2);
}

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
// K-elements; chunk position p (16 bytes) = j * 256 + tid of physical row
// P = p / cpr (cpr = chunks per row) holds logical chunk (p % cpr) ^ swz(r)
// of logical row r = row64(P) (E4M3) or P (bf16).
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
      const int r = kChunks == 4 ? row64(p / kChunks) : p / kChunks;  // logical row stored there
      const int c = (p % kChunks) ^ (kChunks == 4 ? swz4(r) : swz8(r));
      voff[j] = (uint32_t)(r * ld_bytes) + (uint32_t)c * 16u;
      kchunk[j] = c * (kChunks == 4 ? 16 : 8);
    }
  }

  // Copy chunk j of stage `kt` (no K tail: the stage lies inside [0, k)).
  __device__ __forceinline__ void copy_one(const uint8_t* lds_tile, int kt, int j, int tid) const {
    const uint32_t soff = (uint32_t)(kt * kBK) * (kChunks == 4 ? 1u : 2u);
    dma16(rsrc, voff[j], soff,
          __builtin_amdgcn_readfirstlane(lds_addr(lds_tile) + (j * kThreads + (tid >> 6) * 64) * 16));
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
  const int s = swz4(row), base = row64(row) * 64;
  const u32x4 a = lds_chunk(tile, base + ((2 * g) ^ s) * 16);
  const u32x4 b = lds_chunk(tile, base + ((2 * g + 1) ^ s) * 16);
  v8i v;
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
  return v;
}

__device__ __forceinline__ uint32_t bf16x2(float a, float b) {
  const __bf16 lo = (__bf16)a, hi = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

// Epilogue: scale by alpha, round to bf16 and write the wave's 128 x 128
// output. acc[i][j] holds D[n][m] of the 32 x 32 block (n-block i, m-block
// j): lane l, register v -> m = l % 32, n = 8 (v / 4) + 4 (l / 32) + v % 4,
// i.e. four consecutive n of one row per register quad. Written straight to
// memory that would scatter every store over 32 rows, so the tile goes
// through LDS first: the wave's 32 KiB staging area holds row m (0..127) as
// 16 chunks of 16 bytes, chunk c at physical chunk c ^ (m % 16). Read back
// row by row, 16 lanes cover a row's 256 contiguous bytes and every global
// store is a full 16-byte-per-lane, row-contiguous write.
__device__ __forceinline__ void epilogue(const v16f (&acc)[4][4], const GemmGroup& grp, int M, int m_base, int n_base,
                                         int lane, int wave) {
  __syncthreads();  // every wave is done with the pipeline buffers
  uint8_t* stage = lds_mem + wave * (128 * 256);
  const float alpha = grp.alpha;
  const int h = lane >> 5;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = j * 32 + (lane & 31);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int c = i * 4 + t;  // 16-byte chunk of n = 32 i + 8 t + 4 h
        u32x2 v;
        v[0] = bf16x2(acc[i][j][4 * t] * alpha, acc[i][j][4 * t + 1] * alpha);
        v[1] = bf16x2(acc[i][j][4 * t + 2] * alpha, acc[i][j][4 * t + 3] * alpha);
        *reinterpret_cast<u32x2*>(stage + m * 256 + ((c ^ (m & 15)) * 16) + h * 8) = v;
      }
    }
  }
  const int c = lane & 15;
  const int n = n_base + c * 8;
  const bool n_ok = n < grp.n;
#pragma unroll 8
  for (int q = 0; q < 32; ++q) {
    const int ml = q * 4 + (lane >> 4);
    const u32x4 v = *reinterpret_cast<const u32x4*>(stage + ml * 256 + ((c ^ (ml & 15)) * 16));
    const int m = m_base + ml;
    if (n_ok && m < M) *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(grp.y) + (int64_t)m * grp.ldy + n) = v;
  }
}

// Wait until every DMA load except those of the last `later` stages issued
// has landed (`per_stage` loads per thread per stage), then synchronize the
// workgroup. vmcnt needs an immediate, hence the switch.
template <int kPerStage>
__device__ __forceinline__ void wait_stages(int later) {
  switch (later) {
    case 0: wait_vmem_and_barrier<0>(); break;
    case 1: wait_vmem_and_barrier<kPerStage>(); break;
    case 2: wait_vmem_and_barrier<2 * kPerStage>(); break;
    default: wait_vmem_and_barrier<3 * kPerStage>(); break;
  }
}

__device__ __forceinline__ void w8a8_frags(int buf, int row_w, int row_x, int g, v8i (&wf)[4], v8i (&xf)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) wf[i] = frag_e4m3(lds_w8(buf), row_w + i * 32, g);
#pragma unroll
  for (int j = 0; j < 4; ++j) xf[j] = frag_e4m3(lds_x8(buf), row_x + j * 32, g);
}

__device__ __forceinline__ void w8a8_mma(v16f (&acc)[4][4], const v8i (&wf)[4], const v8i (&xf)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[i], xf[j], acc[i][j], 0, 0, 0, 0, 0, 0);
}

// One steady-state half step: the 16 MFMAs of the stage whose fragments are
// in (wc, xc), interleaved one by one with the 8 LDS copies of stage
// `copy_kt` (into buffer `copy_buf`) and the 16 fragment reads of the next
// stage (from buffer `read_buf` into (wn, xn)), read in the order the next
// half consumes them (W0, X0..X3, W1..W3), so each read has at least seven
// MFMAs of cover before its first use. sched_barrier keeps the compiler from
// regrouping the slots, so copies and reads issue in the shadow of the
// matrix-core work instead of in a burst before it.
__device__ __forceinline__ void w8a8_half(v16f (&acc)[4][4], const v8i (&wc)[4], const v8i (&xc)[4], v8i (&wn)[4],
                                          v8i (&xn)[4], const CopyPlan<4>& pw, const CopyPlan<4>& px, int copy_kt,
                                          int copy_buf, int read_buf, int row_w, int row_x, int g, int tid) {
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const int i = t >> 2, j = t & 3;
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wc[i], xc[j], acc[i][j], 0, 0, 0, 0, 0, 0);
    if (t < 4)
      pw.copy_one(lds_w8(copy_buf), copy_kt, t, tid);
    else if (t < 8)
      px.copy_one(lds_x8(copy_buf), copy_kt, t - 4, tid);
    else if (t == 8)
      wn[0] = frag_e4m3(lds_w8(read_buf), row_w, g);
    else if (t < 13)
      xn[t - 9] = frag_e4m3(lds_x8(read_buf), row_x + (t - 9) * 32, g);
    else
      wn[t - 12] = frag_e4m3(lds_w8(read_buf), row_w + (t - 12) * 32, g);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Guarded step for the first and last stages: stage kt + 1 must have
// landed before its fragments are read; stage kt + S - 1 is copied if it
// exists (with the K-tail masking).
__device__ __forceinline__ void w8a8_edge_step(v16f (&acc)[4][4], const v8i (&wc)[4], const v8i (&xc)[4],
                                               v8i (&wn)[4], v8i (&xn)[4], const CopyPlan<4>& pw,
                                               const CopyPlan<4>& px, int kt, int KT, int K, int row_w, int row_x,
                                               int g, int tid) {
  if (kt + 1 < KT) {
    // stages issued after kt + 1: up to kt + S - 2
    wait_stages<8>(min(kt + kStages8 - 2, KT - 1) - (kt + 1));
    const int c = kt + kStages8 - 1;
    if (c < KT) {
      pw.copy(lds_w8(c % kStages8), c, K, tid);
      px.copy(lds_x8(c % kStages8), c, K, tid);
    }
    w8a8_frags((kt + 1) % kStages8, row_w, row_x, g, wn, xn);
  }
  w8a8_mma(acc, wc, xc);
}

// Pipeline over kStages8 LDS buffers: stage s is copied into buffer
// s % kStages8 kStages8 - 1 stages ahead; the MFMA fragments of stage
// s + 1 are read from LDS while the matrix cores work on stage s. The buffer
// refilled while stage s computes held stage s - 1, whose fragments were
// read during stage s - 2, before the barrier that opens stage s.
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
      pw.copy(lds_w8(s), s, K, tid);
      px.copy(lds_x8(s), s, K, tid);
    }
  }

  const int row_w = wn * 128 + (lane & 31);
  const int row_x = wm * 128 + (lane & 31);
  const int g = lane >> 5;

  wait_stages<8>(min(kStages8 - 2, KT - 1));  // stage 0 landed
  v8i wa[4], xa[4], wb[4], xb[4];
  w8a8_frags(0, row_w, row_x, g, wa, xa);

  // Stages in pairs: the even one's fragments sit in (wa, xa), the odd
  // one's in (wb, xb). The steady-state loop runs while every copy it
  // issues is a full stage (stage kt + S <= KT - 2), so it has no branches
  // besides its back edge and the compiler tracks the LDS-read counters
  // exactly; the remaining stages take guarded steps. Both loops have a
  // single exit, so the accumulators stay in place; an odd last stage is
  // already in (wa, xa) when they end.
  int kt = 0;
  for (; kt + kStages8 + 2 <= KT; kt += 2) {
    wait_vmem_and_barrier<8 * (kStages8 - 3)>();
    w8a8_half(acc, wa, xa, wb, xb, pw, px, kt + kStages8 - 1, (kt + kStages8 - 1) % kStages8, (kt + 1) % kStages8,
              row_w, row_x, g, tid);
    wait_vmem_and_barrier<8 * (kStages8 - 3)>();
    w8a8_half(acc, wb, xb, wa, xa, pw, px, kt + kStages8, kt % kStages8, (kt + 2) % kStages8, row_w, row_x, g, tid);
  }
  for (; kt + 1 < KT; kt += 2) {
    w8a8_edge_step(acc, wa, xa, wb, xb, pw, px, kt, KT, K, row_w, row_x, g, tid);
    w8a8_edge_step(acc, wb, xb, wa, xa, pw, px, kt + 1, KT, K, row_w, row_x, g, tid);
  }
  if (kt < KT) w8a8_mma(acc, wa, xa);

  epilogue(acc, grp, a.m, tc.m0 + wm * 128, tc.n0 + wn * 128, lane, wave);
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
      pw.copy(lds_w16(s), s, K, tid);
      px.copy(lds_x16(s), s, K, tid);
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
      pw.copy(lds_w16(sb), next, K, tid);
      px.copy(lds_x16(sb), next, K, tid);
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
        const u32x4 c = lds_chunk(lds_w16(cb), row64(r) * 64 + ((2 * h + g) ^ swz4(r)) * 16);
        wf[i][0] = dequant8(c[0], c[1]);
        wf[i][1] = dequant8(c[2], c[3]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = row_x + j * 32;
        xf[j][0] = as_v8bf(lds_chunk(lds_x16(cb), r * 128 + ((4 * h + 2 * g) ^ swz8(r)) * 16));
        xf[j][1] = as_v8bf(lds_chunk(lds_x16(cb), r * 128 + ((4 * h + 2 * g + 1) ^ swz8(r)) * 16));
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

  epilogue(acc, grp, a.m, tc.m0 + wm * 128, tc.n0 + wn * 128, lane, wave);
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
