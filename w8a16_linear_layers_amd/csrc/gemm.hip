// Grouped static-FP8 GEMMs on the gfx950 matrix cores.
//
//   W8A8  ([CF-157] "Verification", a real FP8 x FP8 GEMM):
//     y[m, n] = bf16( sum_k qx[m, k] qw[n, k] * (s_in * s_w) )
//     v_mfma_f32_16x16x128_f8f6f4 (E4M3 x E4M3, float32 accumulate).
//   W8A16 ([TRT-17476] "Denoising-step activation precision", same resident
//   FP8 weight, 16-bit activation, no dequantized weight copy):
//     y[m, n] = bf16( sum_k x[m, k] dec(qw[n, k]) * s_w )
//     The E4M3 weight tile is staged in LDS at one byte per element and
//     converted exactly to bf16 (v_cvt_scalef32_pk_bf16_fp8, scale 1) on its
//     way to v_mfma_f32_16x16x32_bf16.
//
// Shared structure:
//   * A workgroup of 4 waves owns a 256 (M) x 256 (N) output tile; wave
//     (wm, wn) owns the 128 x 128 quarter (wm, wn) as 8 x 8 blocks of 16 x 16.
//   * The weight is the MFMA "A" operand and the activation the "B" operand,
//     so the accumulator D[n][m] gives every lane four consecutive n of one
//     output row.
//   * Global memory is copied straight into LDS by buffer_load_dwordx4 ... lds
//     against a per-tile buffer resource: rows beyond M or N fall outside it
//     and K chunks beyond K get an out-of-range offset, and both read as zero,
//     so edge tiles need no other masking until the store.
//   * Tiles of all groups form one index space, remapped so that the
//     workgroups dispatched to one XCD (ids congruent mod 8) take a
//     contiguous run of tiles, rasterized in bands of 4 M-tiles for L2 reuse.
#include <mutex>
#include <type_traits>
#include <utility>

#include "fp8lin.h"

#include "device.h"
#include "internal.h"

namespace fp8lin {

void gemm_plan(GemmArgs& a) {
  if (a.xk == 0) a.xk = a.k;
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
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kXcds = 8;
// M-tiles per raster band: an XCD's 32 concurrent tiles then span 4 activation and
// 8 weight row blocks, the fewest bytes for W8A16's 2-byte activations (W8A16
// +1.3% against bands of 8 on one box; W8A8 the same; bands of 2 slower)
constexpr int kBandM = 4;

// ------------------------------------------------------------------ LDS arena
// W8A8: two stages of 256 x 128-byte E4M3 tiles for each operand (128 KiB),
//       then a 32 KiB epilogue area (8 KiB per wave).
// W8A16: three stages of a 256 x 64-byte E4M3 weight tile (16 KiB) and a
//       256 x 64-element bf16 activation tile (32 KiB); its epilogue stages
//       rows in the activation tile of the buffer the tile's last stage used.
constexpr int kW8A8Stage = kTileN * 128;  // 32 KiB per operand per stage
constexpr int kW8A8EpiOffset = 4 * kW8A8Stage;
constexpr int kW8A8EpiWave = 32 * 256;  // 32 output rows of 256 bytes per wave
constexpr int kStages16 = 3;
constexpr int kStageE4M3 = kTileN * 64;      // 16 KiB
constexpr int kStageBf16 = kTileM * 64 * 2;  // 32 KiB
constexpr int kLdsW8A8 = kW8A8EpiOffset + 4 * kW8A8EpiWave;
constexpr int kLdsW8A16 = kStages16 * (kStageE4M3 + kStageBf16);
constexpr int kLdsBytes = kLdsW8A8 > kLdsW8A16 ? kLdsW8A8 : kLdsW8A16;
static_assert(kStageBf16 >= 4 * kW8A8EpiWave, "the W8A16 epilogue stages 8 KiB per wave");
static_assert(kLdsBytes <= 160 * 1024, "gfx950 LDS per workgroup");
__shared__ __attribute__((aligned(16))) uint8_t lds_mem[kLdsBytes];

__device__ __forceinline__ uint8_t* lds8_w(int buf) { return lds_mem + buf * kW8A8Stage; }
__device__ __forceinline__ uint8_t* lds8_x(int buf) { return lds_mem + (2 + buf) * kW8A8Stage; }
__device__ __forceinline__ uint8_t* lds16_w(int s) { return lds_mem + s * kStageE4M3; }
__device__ __forceinline__ uint8_t* lds16_x(int s) { return lds_mem + kStages16 * kStageE4M3 + s * kStageBf16; }

// LDS tile layouts (fragment reads take 16-row blocks, lane (r, q) =
// (l % 16, l / 16) reading row r). The swizzles come from measurement: every
// linear XOR swizzle of a 16-row block (a 3-bit chunk XOR from the 4 low row
// bits, 4096 candidates) was read on one MI355X in the kernels' own lane
// pattern, and SQ_LDS_BANK_CONFLICT per ds_read_b128 is either 0 (1344
// swizzles; a conflict-free 16-byte read takes 4 LDS cycles), 3.56, 10.67 or
// 24.89 cycles. Bijective swizzles can still conflict (for instance chunk
// bits from row bits 1 + 3, 2, 1 for the W8A8 tiles read at 3.56, nearly
// doubling the LDS time of every fragment read); the ones below read at 0.
//   128-byte rows of the W8A8 E4M3 tiles (lane quarters 32 bytes apart,
//     halves e = 0, 1): chunk c of row r in physical chunk c ^ swz16(r),
//     swz16(r) = 2 (r & 3) + bit 2 of r.
//   128-byte rows of the W8A16 bf16 activation tiles (lane quarters 16
//     bytes apart): chunk c of row r in physical chunk c ^ swz8(r),
//     swz8(r) = r & 7.
//   64-byte rows of the W8A16 E4M3 weight tile (ds_read_b64, lane quarters 8
//     bytes apart): logical row r in physical row row64(r) = r ^ (bit3(r) << 1)
//     (a swap inside groups of 4 rows), chunk c in physical chunk c ^ swz4(r);
//     measured at 0 as well (1.78 without the row swap).
// All are XORs / involutions, hence bijections on the tile, and depend only on
// row bits below 5 (the copy plans rely on it).
__device__ __forceinline__ int row64(int r) { return r ^ (((r >> 3) & 1) << 1); }
__device__ __forceinline__ int swz4(int r) { return ((r >> 2) & 1) | ((((r >> 1) ^ (r >> 2)) & 1) << 1); }
__device__ __forceinline__ int swz8(int r) { return r & 7; }
__device__ __forceinline__ int swz16(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

// ------------------------------------------------------------------ copies

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

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) { return (uint32_t)reinterpret_cast<uintptr_t>(p); }

template <int N>
__device__ __forceinline__ void wait_vmem_and_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Per-thread copy plan of one 256-row operand tile with `kChunks` 16-byte
// chunks per row (8: 128-byte rows, 4: 64-byte rows). Chunk position
// p = j * 256 + tid of physical row P = p / kChunks holds logical chunk
// (p % kChunks) ^ swizzle(r) of logical row r (= P for 128-byte rows,
// row64(P) for 64-byte rows). Rows 0-127 and 128-255 come from two buffer
// resources (the two halves of one matrix, or two matrices such as the gate
// and up weights), and chunk j lies in the upper half iff j >= kChunks / 2.
// off(j) is the chunk's byte offset inside its resource at K = 0; a stage's
// K offset travels in the scalar offset. The swizzles depend only on row
// bits below 5, which j does not change, so a thread copies the same
// logical chunk of every row it serves (kbyte), and the rows of chunks j and
// j' of one half differ by a wave-uniform multiple of 256 / kChunks rows.
// kSwz16: 128-byte rows in the W8A8 layout (swz16 instead of swz8). The
// offsets are kept one register per chunk: forming them at issue time from
// one register and a scalar step saves registers but costs vector
// instructions in the stage loops, each of which costs matrix-core time.
template <int kChunks, bool kSwz16 = false>
struct CopyPlan {
  i32x4 lo, hi;
  uint32_t voff[kChunks];
  int kbyte;  // first K byte of the thread's chunk within a stage row

  // Rows [0, 128) from src_lo (rows_lo of them valid), rows [128, 256) from
  // src_hi (rows_hi valid); rows beyond the valid ones read as zero.
  __device__ __forceinline__ void init2(const uint8_t* src_lo, int rows_lo, const uint8_t* src_hi, int rows_hi,
                                        int64_t ld_bytes, int tid) {
    // readfirstlane: the (uniform) clamps may be computed in vector registers,
    // and the resources must stay scalar for the copies
    const int n_lo = __builtin_amdgcn_readfirstlane(max(0, min(rows_lo, 128)));
    const int n_hi = __builtin_amdgcn_readfirstlane(max(0, min(rows_hi, 128)));
    lo = make_rsrc(src_lo, (uint32_t)(n_lo * ld_bytes));
    hi = make_rsrc(src_hi, (uint32_t)(n_hi * ld_bytes));
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
      const int p = j * kThreads + tid;
      const int r = kChunks == 4 ? row64(p / kChunks) : p / kChunks;
      const int c = (p % kChunks) ^ (kChunks == 4 ? swz4(r) : kSwz16 ? swz16(r) : swz8(r));
      voff[j] = (uint32_t)((r & 127) * ld_bytes) + (uint32_t)c * 16u;
      if (j == 0) kbyte = c * 16;
    }
  }

  // Offset of chunk j (a compile-time constant in the unrolled callers).
  __device__ __forceinline__ uint32_t off(int j) const { return voff[j]; }

  // Rows [row0, row0 + 256) of one matrix with `rows` valid rows from row0.
  __device__ __forceinline__ void init(const uint8_t* src, int row0, int rows, int64_t ld_bytes, int tid) {
    const uint8_t* base = src + (int64_t)row0 * ld_bytes;
    init2(base, rows, base + 128 * ld_bytes, rows - 128, ld_bytes, tid);
  }

  // One copy of chunk j with offset v (j is a compile-time constant once the
  // callers' loops are unrolled, so the resource choice folds away).
  __device__ __forceinline__ void dma(int j, uint32_t v, uint32_t k0b, uint32_t lds) const {
    if (j < kChunks / 2)
      dma16(lo, v, k0b, lds);
    else
      dma16(hi, v, k0b, lds);
  }

  // Chunk j of the full stage starting at byte `k0b` of each row.
  __device__ __forceinline__ void copy_one(const uint8_t* lds_tile, uint32_t k0b, int j, uint32_t wave_off) const {
    dma(j, off(j), k0b, lds_addr(lds_tile) + j * kThreads * 16 + wave_off);
  }

  // Chunk j of the stage starting at byte `k0b`, zero at or beyond byte `kb`
  // of a row (the K tail).
  __device__ __forceinline__ void copy_masked(const uint8_t* lds_tile, int k0b, int kb, int j,
                                              uint32_t wave_off) const {
    dma(j, k0b + kbyte >= kb ? kOutOfRange : off(j), (uint32_t)k0b, lds_addr(lds_tile) + j * kThreads * 16 + wave_off);
  }

  // All chunks of the stage starting at byte `k0b`; chunks at or beyond
  // byte `kb` of a row (the K tail) read as zero.
  __device__ __forceinline__ void copy(const uint8_t* lds_tile, int k0b, int kb, uint32_t wave_off) const {
    const bool beyond = k0b + kbyte >= kb;
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
      const uint32_t o = off(j);
      dma(j, beyond ? kOutOfRange : o, (uint32_t)k0b, lds_addr(lds_tile) + j * kThreads * 16 + wave_off);
    }
  }

  // Every later copy reads zeros.
  __device__ __forceinline__ void exhaust() {
    lo[2] = 0;
    hi[2] = 0;
  }
};

__device__ __forceinline__ u32x4 lds_chunk(const uint8_t* tile, int byte_offset) {
  return *reinterpret_cast<const u32x4*>(tile + byte_offset);
}

// ------------------------------------------------------------------ tiles

struct TileCoord {
  int group;
  int m0;
  int n0;
};

// Logical tile of dispatch slot `slot`: slot b runs on XCD b % 8, and each
// XCD gets a contiguous run of tiles, rasterized in bands of kBandM M-tiles.
// Tiles are kTM rows of M by kTN columns of N.
template <int kTN = kTileN, int kTM = kTileM>
__device__ __forceinline__ TileCoord tile_at(const GemmArgs& a, int slot) {
  const int T = a.total_tiles;
  const int xcd = slot % kXcds, idx = slot / kXcds;
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
  // the arithmetic above is uniform; say so, so that the values stay scalar
  TileCoord c;
  c.group = __builtin_amdgcn_readfirstlane(gi);
  c.m0 = __builtin_amdgcn_readfirstlane((first_m + in_band % band_m) * kTM);
  c.n0 = __builtin_amdgcn_readfirstlane((in_band / band_m) * kTN);
  return c;
}

// ------------------------------------------------------------------ epilogues

__device__ __forceinline__ uint32_t bf16x2(float a, float b) { return h16x2<false>(a, b); }

// Cache policy of the GEMM output stores: slc (streaming). Output rows are
// written once and never re-read by the kernel; streaming them keeps the
// caches for the operand rows (measured on one box: a single 16384x4096x4096
// launch +7.5%, the grouped QKV launch +2%, the split gated MLP 1.07 ->
// 1.02 ms, no row slower).
constexpr int kStreamStore = 2;
// Split-K partials are re-read at once by the reduction: default policy.
constexpr int kSplitPartialStore = 0;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Output rows leave through LDS: rows [32 j, 32 j + 32) of a wave's 128 x 128
// tile are staged in its 8 KiB area, staged row m holding the tile's 128
// columns as 16 chunks of 16 bytes (8 16-bit values, or 4 float32 values of
// a 64-column half) with chunk c at physical chunk c ^ (m % 16). Read back
// row by row, 16 lanes cover a row's 256 contiguous bytes and every global
// store writes 16 bytes per lane; straight from the accumulators every
// store instruction would scatter over 16 or 32 rows.
//
// Accumulators: 16 x 16 blocks, acc[i][b] = D[n][m] of n-block i, m-block b;
// lane l, register v -> m = 16 b + l % 16, n = 16 i + 4 (l / 16) + v (four
// consecutive n of one row per lane); rows [32 j, 32 j + 32) are m-blocks
// 2 j and 2 j + 1.

// Stage bf16(acc * alpha) (binary16 with kF16) of rows [32 j, 32 j + 32).
template <bool kF16>
__device__ __forceinline__ void stage_rows(const f32x4 (&acc)[8][8], int j, uint8_t* stage, float alpha, int lane) {
  const int q = lane >> 4;
  const int r = lane & 15;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int m = 16 * b + r;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = 2 * i + (q >> 1);  // 16-byte chunk of n = 16 i + 4 q
      const f32x4 x = acc[i][2 * j + b];
      u32x2 v;
      v[0] = h16x2<kF16>(x[0] * alpha, x[1] * alpha);
      v[1] = h16x2<kF16>(x[2] * alpha, x[3] * alpha);
      *reinterpret_cast<u32x2*>(stage + m * 256 + ((c ^ r) * 16) + (q & 1) * 8) = v;
    }
  }
}

// Stage acc * alpha in float32, columns [64 hf, 64 hf + 64) of rows
// [32 j, 32 j + 32).
__device__ __forceinline__ void stage_rows_f32(const f32x4 (&acc)[8][8], int j, int hf, uint8_t* stage, float alpha,
                                               int lane) {
  const int q = lane >> 4;
  const int r = lane & 15;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int m = 16 * b + r;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int c = 4 * ii + q;  // 16-byte chunk of n = 64 hf + 16 ii + 4 q
      const f32x4 x = acc[4 * hf + ii][2 * j + b];
      u32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = __float_as_uint(x[e] * alpha);
      *reinterpret_cast<u32x4*>(stage + m * 256 + ((c ^ r) * 16)) = v;
    }
  }
}

// Buffer stores a thread issues per output tile, derived from the epilogue
// loops below (the waits that skip a tile's stores count them):
//   store_rows: 16 lanes per 256-byte staged row, so a 32-row pass is
//     32 / (64 / 16) = 8 stores per lane; 4 passes per 128-row wave tile,
//     twice for float32 output (two 64-column halves);
//   epilogue_swiglu: 8 lanes per h row, 16 rows per wave and pass, so 2 rows
//     per lane, each one 16-byte store of E4M3 codes or two of 16-bit values.
constexpr int kEpiPassRows = 32;
constexpr int kEpiPasses = 128 / kEpiPassRows;
constexpr int kStoreRowsStores = kEpiPassRows / (64 / 16);
constexpr int kSwiGLURowsPerLane = (kEpiPassRows / 2) / (64 / 8);
template <bool kFp8Out>
constexpr int kSwiGLUPassStores = kSwiGLURowsPerLane * (kFp8Out ? 1 : 2);
// per tile: kind 0 = 16-bit rows, 1 = float32 rows, 2 = SwiGLU E4M3 h, 3 = SwiGLU 16-bit h
constexpr int tile_stores(int kind) {
  return kind == 0   ? kEpiPasses * kStoreRowsStores
         : kind == 1 ? kEpiPasses * 2 * kStoreRowsStores
         : kind == 2 ? kEpiPasses * kSwiGLUPassStores<true>
                     : kEpiPasses * kSwiGLUPassStores<false>;
}
static_assert(tile_stores(0) == 32 && tile_stores(1) == 64 && tile_stores(2) == 8 && tile_stores(3) == 16,
              "stores per tile");
// The largest count an s_waitcnt vmcnt can encode. A wait that should skip
// more younger operations than this waits for some of them too: correct,
// only more conservative.
constexpr int kMaxVmcnt = 63;
constexpr int clamp_vmcnt(int n) { return n < kMaxVmcnt ? n : kMaxVmcnt; }

// Store the staged rows [32 j, 32 j + 32) of kElem-byte elements, 16 bytes
// per lane, the row's first column being n0. Columns at or beyond N get an
// out-of-range offset, so every lane issues the same kStoreRowsStores
// stores. The staging writes come from the same wave, whose LDS operations
// complete in order.
template <int kElem, int kPolicy>
__device__ __forceinline__ void store_rows(const uint8_t* stage, int j, const GemmGroup& grp,
                                           __amdgpu_buffer_rsrc_t out, int n0, int lane) {
  const int c = lane & 15;
  const int n = n0 + c * (16 / kElem);
  // the group's sizes, loaded once (scalar) rather than beside every store
  const int gn = __builtin_amdgcn_readfirstlane(grp.n), gld = __builtin_amdgcn_readfirstlane(grp.ldy);
  u32x4 v[kStoreRowsStores];
#pragma unroll
  for (int q = 0; q < kStoreRowsStores; ++q) {
    const int ml = q * 4 + (lane >> 4);
    v[q] = *reinterpret_cast<const u32x4*>(stage + ml * 256 + ((c ^ (ml & 15)) * 16));
  }
#pragma unroll
  for (int q = 0; q < kStoreRowsStores; ++q) {
    const int ml = kEpiPassRows * j + q * 4 + (lane >> 4);
    const uint32_t off = n < gn ? (uint32_t)(ml * gld + n) * (uint32_t)kElem : kOutOfRange;
    __builtin_amdgcn_raw_buffer_store_b128(v[q], out, (int)off, 0, kPolicy);
  }
}

// Output resource of a wave's 128 x 128 tile: rows [m_base, min(M, m_base +
// 128)) of y, so stores to rows beyond M fall outside it and are dropped.
// Rows m_base..+128 of a group's output of kBytes-byte elements.
template <int kBytes = 2>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rsrc(const GemmGroup& grp, int M, int m_base) {
  // readfirstlane keeps the (uniform) count scalar: a clamp may be computed
  // in a vector register, and a resource in vector registers costs a loop
  const int rows = __builtin_amdgcn_readfirstlane(max(0, min(M - m_base, 128)));
  uint8_t* base = static_cast<uint8_t*>(grp.y) + (int64_t)min(m_base, M) * grp.ldy * kBytes;
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, rows * grp.ldy * kBytes, 0x00020000);
}

// Rows [32 j, 32 j + 32) of the wave's tile, scaled by alpha and rounded to
// bf16 (binary16 with kF16), through the wave's 8 KiB staging area.
template <bool kF16 = false, class Acc>
__device__ __forceinline__ void epilogue_rows(const Acc& acc, int j, uint8_t* stage, const GemmGroup& grp, float alpha,
                                              __amdgpu_buffer_rsrc_t out, int n_base, int lane) {
  // The lane-dependent offsets below are cheap; an opaque copy of the lane
  // index keeps the compiler from holding them in registers across the K loop.
  asm volatile("" : "+v"(lane));
  stage_rows<kF16>(acc, j, stage, alpha, lane);
  store_rows<2, kStreamStore>(stage, j, grp, out, n_base, lane);
}

// Float32 form: columns [64 hf, 64 hf + 64) of rows [32 j, 32 j + 32),
// scaled by alpha, through the same 8 KiB area (two calls per row block).
template <int kPolicy = kStreamStore, class Acc>
__device__ __forceinline__ void epilogue_rows_f32(const Acc& acc, int j, int hf, uint8_t* stage, const GemmGroup& grp,
                                                  float alpha, __amdgpu_buffer_rsrc_t out, int n_base, int lane) {
  asm volatile("" : "+v"(lane));
  stage_rows_f32(acc, j, hf, stage, alpha, lane);
  store_rows<4, kPolicy>(stage, j, grp, out, n_base + 64 * hf, lane);
}

// bf16 rounding of a float32 value, back as float32 (exact).
__device__ __forceinline__ float bf16_round(float v) { return bf16_lo(bf16x2(v, 0.0f)); }

// epilogue_rows for a 128-column block that is one head of a Q or K
// projection (W8A8 accumulators): y = bf16(acc * alpha), the value the plain
// epilogue writes, then per row the head's RMSNorm and rotate-half RoPE in
// float32 (r = rsqrt(sum(y^2) / 128 + eps); out[d] = y[d] r w[d] cos[t, d] -
// y[d + 64] r w[d + 64] sin[t, d], out[d + 64] = y[d + 64] r w[d + 64]
// cos[t, d] + y[d] r w[d] sin[t, d] for d < 64), rounded to bf16 and stored
// like epilogue_rows. Lane (r, q) = (l % 16, l / 16) holds columns
// 16 i + 4 q + v of rows 16 b + r (b = 0, 1 in the pass), lanes r + 16 q'
// the rest of the row (two butterfly steps complete the sum of squares),
// and the RoPE partner of a column of block i < 4 is the same position of
// block i + 4 in the same lane. row0: the first output row of the wave's
// tile (rows at or past M are never stored; their table row is clamped to
// M - 1). With active = false (a V tile) r = 1, w = 1 and no rotation,
// which reproduces epilogue_rows bit for bit: one code path for every tile
// of the launch.
__device__ __forceinline__ void epilogue_rows_norm_rope(const f32x4 (&acc)[8][8], int j, uint8_t* stage,
                                                        const GemmGroup& grp, float alpha,
                                                        __amdgpu_buffer_rsrc_t out, int n_base, int lane, int row0,
                                                        int M, bool active, const uint16_t* w, const float* cos,
                                                        const float* sin, float eps) {
  asm volatile("" : "+v"(lane));
  const int q = lane >> 4;
  const int r = lane & 15;
  // the lane's norm weights, the same for both rows of the pass: loaded once per pass
  u32x2 wv[8];
  if (active && w != nullptr) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wv[i] = *reinterpret_cast<const u32x2*>(w + 16 * i + 4 * q);
      wv[i + 4] = *reinterpret_cast<const u32x2*>(w + 64 + 16 * i + 4 * q);
    }
  }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int mb = 2 * j + b;  // m-block
    const int m = 16 * b + r;  // row within the pass
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float y = bf16_round(acc[i][mb][e] * alpha);
        ss += y * y;
      }
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    const float rr = active ? rsqrtf(ss * (1.0f / 128) + eps) : 1.0f;
    const int token = min(row0 + 32 * j + m, M - 1);
    const float* cr = cos + (int64_t)token * 64;
    const float* sr = sin + (int64_t)token * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 16 * i + 4 * q;
      f32x4 c = {1.0f, 1.0f, 1.0f, 1.0f}, s = {0.0f, 0.0f, 0.0f, 0.0f};
      if (active) {
        c = *reinterpret_cast<const f32x4*>(cr + d);
        s = *reinterpret_cast<const f32x4*>(sr + d);
      }
      float wa[4] = {1.0f, 1.0f, 1.0f, 1.0f}, wb[4] = {1.0f, 1.0f, 1.0f, 1.0f};
      if (active && w != nullptr) {
        const u32x2 ga = wv[i], gb = wv[i + 4];
        wa[0] = bf16_lo(ga.x); wa[1] = bf16_hi(ga.x); wa[2] = bf16_lo(ga.y); wa[3] = bf16_hi(ga.y);
        wb[0] = bf16_lo(gb.x); wb[1] = bf16_hi(gb.x); wb[2] = bf16_lo(gb.y); wb[3] = bf16_hi(gb.y);
      }
      float oa[4], ob[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ya = bf16_round(acc[i][mb][e] * alpha) * rr * wa[e];
        const float yb = bf16_round(acc[i + 4][mb][e] * alpha) * rr * wb[e];
        oa[e] = active ? ya * c[e] - yb * s[e] : ya;  // inactive: no cross term (an inf stays inf)
        ob[e] = active ? yb * c[e] + ya * s[e] : yb;
      }
      const int ca = 2 * i + (q >> 1), cb = 2 * (i + 4) + (q >> 1);  // chunks of the staged row, as in stage_rows
      *reinterpret_cast<u32x2*>(stage + m * 256 + ((ca ^ r) * 16) + (q & 1) * 8) =
          u32x2{bf16x2(oa[0], oa[1]), bf16x2(oa[2], oa[3])};
      *reinterpret_cast<u32x2*>(stage + m * 256 + ((cb ^ r) * 16) + (q & 1) * 8) =
          u32x2{bf16x2(ob[0], ob[1]), bf16x2(ob[2], ob[3])};
    }
  }
  store_rows<2, kStreamStore>(stage, j, grp, out, n_base, lane);
}

// ------------------------------------------------------------------ W8A8

// Half e (16 bytes) of a 16 x 128 E4M3 fragment of a 128-byte-row stage
// tile for v_mfma_f32_16x16x128_f8f6f4: lane (r, q) = (l % 16, l / 16)
// holds bytes [32 q, 32 q + 32) of row r of the block, i.e. logical chunks
// 2 q and 2 q + 1 (both operands use the same K bytes per lane, so the
// products pair up). Blocks are 16 rows apart, which leaves row bits 1-3
// and with them the swizzle unchanged, so the lane's two byte offsets in
// block 0 (frag16_offset) serve every block f at + 2048 f.
__device__ __forceinline__ int frag16_offset(int row, int q, int e) {
  return row * 128 + (((2 * q + e) ^ swz16(row)) * 16);
}

__device__ __forceinline__ u32x4 frag16_half(const uint8_t* tile, int off, int f) {
  return lds_chunk(tile, off + 2048 * f);
}

__device__ __forceinline__ void set_half(v8i& f, int e, const u32x4 v) {
  f[4 * e + 0] = (int)v[0];
  f[4 * e + 1] = (int)v[1];
  f[4 * e + 2] = (int)v[2];
  f[4 * e + 3] = (int)v[3];
}

__device__ __forceinline__ void read_frag16(v8i& v, const uint8_t* tile, const int (&off)[2], int f) {
  set_half(v, 0, frag16_half(tile, off[0], f));
  set_half(v, 1, frag16_half(tile, off[1], f));
}

// One stage (128 K bytes) of a wave's 128 x 128 tile: 64 MFMAs
// v_mfma_f32_16x16x128_f8f6f4 over weight blocks wf[i] (16 rows of N each)
// and activation blocks xf[b] (16 rows of M each), in two halves: MFMA t of
// the first half multiplies (i, b) = (t % 4, t / 4), of the second half
// (4 + t % 4, t / 4). So wf[0..3] are done after the first half, xf[b] after
// MFMA 32 + 4 b + 3 of the second, and wf[4..7] are first needed in the
// second half -- each register block is refilled in place as soon as it is
// done, and the 16 blocks (128 VGPRs) are all the fragments there are.
// Each MFMA is followed by at most one memory operation (slot plan below);
// a tile's last stage (kLast) has no stage s + 1 and reads nothing for one;
// after the barrier that frees its buffer it copies the next tile's stage 1
// there (stage KT - 2 copied that tile's stage 0; plans pw, px of that tile,
// none when has_next is false). sched_barrier keeps the compiler from
// regrouping slots.
//
// Why 16 x 16 x 128 and not 32 x 32 x 64 (same 128 x 128 wave tile, same
// LDS traffic): on one MI355X, back-to-back FP8 MFMAs sustain 4.36-4.47
// PFLOP/s in the 16 x 16 form against 3.96-4.10 in the 32 x 32 form, and the
// GEMM held 1.79-1.96 GHz against 1.67 GHz with the 32 x 32 form -- the board is
// power-limited and the smaller instruction costs less energy per FLOP. The
// twice as many, half as long MFMAs leave half the time per slot, so the
// copies are spread three slots apart (two: -1%, one: -6%).
constexpr int kSlotFree = 12;   // barrier that frees this stage's buffer
constexpr int kCopyStride = 3;  // slots between the copies of stage s + 2
constexpr int kSlotMid = 32;    // barrier after which stage s + 1 is readable

// Across a tile change the copies keep the steady rhythm: stage KT - 2
// issues the next tile's stage 0 and the last stage its stage 1 (KT = 1:
// stage 0), each into the buffer it frees, at the steady stage's copy slots.
// A tile's stage s uses buffer (s + p) % 2, p the tile's buffer parity.

// ------------------------------------------------------------------ overlapped epilogue
// Most of the plain bf16 epilogue runs beside the matrix cores' work of a
// tile's last stage instead of after it. A wave's 128 x 128 output block
// leaves in two parts of 64 columns:
//   part A, acc[0..3][*] (weight blocks 0-3), is final once the first half
//     of the stage has run (acc[i][b] takes its last MFMA at slot 4 b + i);
//   part B, acc[4..7][*], becomes final through the second half (last MFMA
//     at slot 32 + 4 b + i).
// Each part is 4 passes of 32 rows (pass j: m-blocks 2 j, 2 j + 1). A pass is
// 8 units -- unit u scales acc[4 P + (u & 3)][2 j + (u >> 2)] by alpha,
// rounds to bf16 and writes it to the wave's staging area (one ds_write_b64
// per lane) -- then 4 reads of 8 staged rows (ds_read_b128) and 4 stores of
// those rows (buffer_store_dwordx4, 8 lanes per 128-byte row segment).
// Passes alternate between the two 4 KiB halves of the wave's 8 KiB area.
// The plan below places the 8 passes one unit per slot from slot kEpi0:
// all of part A and 3 of part B's passes' units fall inside the stage, the
// rest runs right after it, before the next tile starts. Within a slot the
// order is: MFMA, own fragment read, free barrier, copy, epilogue unit,
// epilogue read, epilogue store.
//
// Measured on one box (16384 x 4096 x 4096, one launch): 2941 -> 2993 and
// 2956 -> 3022 TFLOP/s with part A in the stage against the whole epilogue
// after it, and 3026 -> 3040 with part B's first passes moved in as well;
// with no epilogue at all (a diagnostic build) 3234-3283. Timing builds
// that drop one part at a time place the remaining cost in the global
// stores (+7% without them), not in the units' arithmetic (+0.4% without
// it): the stores share the CU's vector-memory requests with the copies,
// whose rate bounds this kernel. Part B in the first half of
// the next tile's stage 0 (whose MFMAs start from zero and write only
// acc[0..3] there) ran out of registers beside stage 0's fragments and
// spilled; stores straight from the accumulators (no staging) were 15-30%
// slower overall; a software-pipelined part B measured the same.
constexpr int kEpiHalf = 4096;  // bytes of one pass: 32 rows x 128 bytes
static_assert(2 * kEpiHalf == kW8A8EpiWave, "two pass areas per wave");

struct EpiSlot {
  int unit, rd, st;  // -1, or pass * 8 + unit / pass * 4 + read / pass * 4 + store
};
// Passes 0-3 are part A, 4-7 part B (pass p: part p / 4, rows 32 (p % 4) ..,
// staging half p % 2). Slots 0-63 go with the last stage's MFMAs; later
// slots only order what runs after the stage.
constexpr int kEpiSlots = 128;
struct EpiPlan {
  EpiSlot op[kEpiSlots];
  int end;  // one past the last slot in use
  bool ok;
};
constexpr int kMfmaLatencySlots = 4;  // slots between an accumulator's last MFMA and its first read
// First slot at which unit u of pass p reads a final accumulator:
// acc[4 P + (u & 3)][2 j + (u >> 2)] takes its last MFMA at slot 32 P + 4 b + i.
constexpr int epi_ready(int p, int u) {
  return 32 * (p >> 2) + 4 * (2 * (p & 3) + (u >> 2)) + (u & 3) + kMfmaLatencySlots;
}

// Greedy plan, one unit, one read and one store per slot at most: the units
// of pass p in order, from slot a0, each once its accumulator is final and,
// for pass p >= 2, after the last read of pass p - 2 (same staging half);
// read k of pass p after the pass's units, two slots after read k - 1 and
// after store k of pass p - 1 (same registers); each store kStoreLag slots
// after its read.
constexpr int kStoreLag = 3;
constexpr EpiPlan make_epi_plan(int a0) {
  EpiPlan p{};
  p.ok = true;
  p.end = 0;
  for (int t = 0; t < kEpiSlots; ++t) p.op[t] = EpiSlot{-1, -1, -1};
  int last_unit = a0 - 1, last_rd[8] = {}, st_of[8][4] = {};
  for (int q = 0; q < 8; ++q) {
    for (int u = 0; u < 8; ++u) {
      int t = last_unit + 1;
      if (t < epi_ready(q, u)) t = epi_ready(q, u);
      if (q >= 2 && t <= last_rd[q - 2]) t = last_rd[q - 2] + 1;
      while (t < kEpiSlots && p.op[t].unit >= 0) ++t;
      if (t >= kEpiSlots) {
        p.ok = false;
        return p;
      }
      p.op[t].unit = 8 * q + u;
      last_unit = t;
    }
    int t = last_unit + 1;
    for (int k = 0; k < 4; ++k) {
      if (q >= 1 && t <= st_of[q - 1][k]) t = st_of[q - 1][k] + 1;
      while (t < kEpiSlots && p.op[t].rd >= 0) ++t;
      int ts = t + kStoreLag;
      while (ts < kEpiSlots && p.op[ts].st >= 0) ++ts;
      if (ts >= kEpiSlots) {
        p.ok = false;
        return p;
      }
      p.op[t].rd = 4 * q + k;
      p.op[ts].st = 4 * q + k;
      st_of[q][k] = ts;
      last_rd[q] = t;
      if (ts + 1 > p.end) p.end = ts + 1;
      t += 2;
    }
  }
  return p;
}
constexpr int epi_slot_of(const EpiPlan& p, int kind, int id) {  // kind 0 unit, 1 read, 2 store
  for (int t = 0; t < kEpiSlots; ++t)
    if ((kind == 0 ? p.op[t].unit : kind == 1 ? p.op[t].rd : p.op[t].st) == id) return t;
  return -1;
}
constexpr int epi_stores_from(const EpiPlan& p, int t0) {  // stores at slots >= t0
  int n = 0;
  for (int t = t0; t < kEpiSlots; ++t) n += p.op[t].st >= 0;
  return n;
}
constexpr int kEpi0 = 8;
constexpr EpiPlan kEpiPlan = make_epi_plan(kEpi0);
constexpr bool epi_plan_ok(const EpiPlan& q) {
  if (!q.ok || q.end > kEpiSlots) return false;
  for (int p = 0; p < 8; ++p) {
    for (int u = 0; u < 8; ++u) {
      const int tu = epi_slot_of(q, 0, 8 * p + u);
      if (tu < 0 || (tu < 64 && tu < epi_ready(p, u))) return false;
      if (u > 0 && tu <= epi_slot_of(q, 0, 8 * p + u - 1)) return false;
    }
    for (int k = 0; k < 4; ++k) {
      const int tr = epi_slot_of(q, 1, 4 * p + k), ts = epi_slot_of(q, 2, 4 * p + k);
      if (tr < 0 || ts <= tr) return false;
      for (int u = 0; u < 8; ++u)  // a pass's reads follow all of its units
        if (tr <= epi_slot_of(q, 0, 8 * p + u)) return false;
      // the next pass's read k reuses the same registers: after this store
      if (p < 7 && epi_slot_of(q, 1, 4 * (p + 1) + k) <= ts) return false;
      // pass p + 2 writes the same area: after all of pass p's reads
      if (p < 6 && epi_slot_of(q, 0, 8 * (p + 2)) <= tr) return false;
    }
  }
  return true;
}
static_assert(epi_plan_ok(kEpiPlan), "the overlapped epilogue's windows, order and staging reuse");

// Where a wave's output rows go, and how they are scaled.
struct EpiCtx {
  uint8_t* area;               // the wave's 8 KiB staging area
  __amdgpu_buffer_rsrc_t out;  // rows m_base .. m_base + 128 of the group's output
  float alpha;
  int col0;                    // first output column of the wave's 128-column block
  int gn, gld;                 // the group's N and ldy
};

// Unit u of pass j of part P: bf16(acc[4 P + (u & 3)][2 j + (u >> 2)] * alpha)
// into staged row m = 16 (u >> 2) + r of the pass, 16-byte chunk
// c = 2 (u & 3) + q / 2 at physical chunk c ^ (m % 8).
template <int P>
__device__ __forceinline__ void epi_unit(const f32x4 (&acc)[8][8], int j, int u, const EpiCtx& e, int lane) {
  const int q = lane >> 4, r = lane & 15;
  const int m = 16 * (u >> 2) + r;
  const int c = 2 * (u & 3) + (q >> 1);
  const f32x4 x = acc[4 * P + (u & 3)][2 * j + (u >> 2)];
  u32x2 v;
  v[0] = bf16x2(x[0] * e.alpha, x[1] * e.alpha);
  v[1] = bf16x2(x[2] * e.alpha, x[3] * e.alpha);
  *reinterpret_cast<u32x2*>(e.area + (j & 1) * kEpiHalf + m * 128 + ((c ^ (m & 7)) * 16) + (q & 1) * 8) = v;
}

// Read k of pass j: staged rows 8 k .. 8 k + 7, lane l holding chunk l % 8 of
// row 8 k + l / 8.
__device__ __forceinline__ u32x4 epi_read(int j, int k, const EpiCtx& e, int lane) {
  const int row = 8 * k + (lane >> 3), c = lane & 7;
  return *reinterpret_cast<const u32x4*>(e.area + (j & 1) * kEpiHalf + row * 128 + ((c ^ (row & 7)) * 16));
}

// Store k of pass j of part P: those 16 bytes to row 32 j + 8 k + l / 8 of the
// wave's block, columns col0 + 64 P + 8 (l % 8) ..; columns at or past N get
// an out-of-range offset, rows past M fall outside the resource.
template <int P>
__device__ __forceinline__ void epi_store(const u32x4& v, int j, int k, const EpiCtx& e, int lane) {
  const int row = 32 * j + 8 * k + (lane >> 3);
  const int col = e.col0 + 64 * P + 8 * (lane & 7);
  const uint32_t off = col < e.gn ? (uint32_t)(row * e.gld + col) * 2u : kOutOfRange;
  __builtin_amdgcn_raw_buffer_store_b128(v, e.out, (int)off, 0, kStreamStore);
}

// What one stage needs besides the fragments and accumulators.
struct StageCtx {
  const CopyPlan<8, true>& pw;
  const CopyPlan<8, true>& px;
  int cur, nxt;   // LDS buffer of this stage and of the next
  uint32_t k2;    // K byte of stage s + 2
  int K, KT;
  bool has_next;  // kLast: a next tile exists
  const int (&ow)[2];
  const int (&ox)[2];
  uint32_t wave_off;
  const EpiCtx& epi;  // kEpi: whose rows the epilogue part writes
  int lane;
};

// The memory operation after MFMA t of a steady stage (at most one each).
enum SlotKind : int { kSlotNone, kSlotOwn, kSlotCopy, kSlotW, kSlotX };
struct SlotOp {
  int kind, a, e;  // own: read a (0..9); copy: chunk a (0..15); W / X: block a, half e
};
struct SlotPlan {
  SlotOp op[64];
  int copies_before_mid;  // copies of stage s + 2 issued before the mid-stage barrier
  int last_copy;          // slot of the last copy of stage s + 2
  bool ok;
};

// Slot plan of a steady stage: this stage's xf[7] and wf[4..7] at slots
// 0-9; the barrier that frees this stage's buffer at kFree; the 16 copies of
// stage s + 2 at kFree + kStride u (or the next free slot); the mid-stage
// barrier (stage s + 1 landed) at kMid; then stage s + 1's wf[0..3] and
// xf[0..6] in the earliest free slots at or after kMid and after the last
// use of the register block they replace (wf[f]: MFMA 28 + f; xf[b]: MFMA
// 35 + 4 b). Copies issued in consecutive slots cost matrix-core time.
constexpr SlotPlan make_slot_plan(int kFree, int kStride, int kMid) {
  SlotPlan p{};
  p.ok = kFree >= 10 && kMid >= 28;
  for (int t = 0; t < 64; ++t) p.op[t] = SlotOp{kSlotNone, 0, 0};
  for (int r = 0; r < 10; ++r) p.op[r] = SlotOp{kSlotOwn, r, 0};
  int t = kFree;
  for (int u = 0; u < 16; ++u) {
    int want = kFree + kStride * u;
    if (want < t) want = t;
    while (want < 64 && p.op[want].kind != kSlotNone) ++want;
    if (want >= 64) {
      p.ok = false;
      return p;
    }
    p.op[want] = SlotOp{kSlotCopy, u, 0};
    if (want < kMid) ++p.copies_before_mid;
    p.last_copy = want;
    t = want + 1;
  }
  auto place = [&](int kind, int blk, int e, int earliest) {
    int s = earliest < kMid ? kMid : earliest;
    while (s < 64 && p.op[s].kind != kSlotNone) ++s;
    if (s >= 64) {
      p.ok = false;
      return;
    }
    p.op[s] = SlotOp{kind, blk, e};
  };
  for (int f = 0; f < 4; ++f)
    for (int e = 0; e < 2; ++e) place(kSlotW, f, e, 28 + f);
  for (int b = 0; b < 7; ++b)
    for (int e = 0; e < 2; ++e) place(kSlotX, b, e, 35 + 4 * b);
  return p;
}

constexpr SlotPlan kSlotPlan = make_slot_plan(kSlotFree, kCopyStride, kSlotMid);
static_assert(kSlotPlan.ok, "the W8A8 stage's memory operations must fit its 64 slots");

// VMEM operations (copies and stores) younger than the previous tile's
// last stage's last copy (its slot kSlotPlan.last_copy; a store follows the
// copy of its slot, and the epilogue's stores at slots 64 and later follow
// the stage): the overlapped epilogue's stores from that slot on. They are
// what a tile's stage 0 skips in its wait for stage 1 (KT > 1), and in its
// start's wait for stage 0 when KT = 1; with KT > 1 stage 0 came from stage
// KT - 2, so the start skips stage 1's copies and all of the stores.
constexpr int kEpiStores = 32;  // 8 passes x 4 stores
constexpr int kEpiStoresAfterLastCopy = epi_stores_from(kEpiPlan, kSlotPlan.last_copy);
static_assert(epi_stores_from(kEpiPlan, 0) == kEpiStores, "8 passes x 4 stores");
static_assert(16 + kEpiStores <= kMaxVmcnt && kEpiStoresAfterLastCopy + kSlotPlan.copies_before_mid <= kMaxVmcnt,
              "vmcnt range");

// kEpi: the stage carries the overlapped epilogue (a tile's last stage).
constexpr bool kEpiNone = false, kEpiOverlap = true;

// The epilogue operations of slot t of the plan.
template <int t>
__device__ __forceinline__ void epi_slot_ops(const f32x4 (&acc)[8][8], u32x4 (&eb)[4], const EpiCtx& e, int lane) {
  constexpr EpiSlot eo = kEpiPlan.op[t];
  if constexpr (eo.unit >= 0) epi_unit<(eo.unit >> 5)>(acc, (eo.unit >> 3) & 3, eo.unit & 7, e, lane);
  if constexpr (eo.rd >= 0) eb[eo.rd & 3] = epi_read((eo.rd >> 2) & 3, eo.rd & 3, e, lane);
  if constexpr (eo.st >= 0) epi_store<(eo.st >> 4)>(eb[eo.st & 3], (eo.st >> 2) & 3, eo.st & 3, e, lane);
}

// MFMA t of the stage and the memory operations that follow it. kExtraVm:
// VMEM operations issued after stage s + 1's copies besides this stage's
// own copies and epilogue stores (the previous tile's output stores, in a
// tile's stage 0). kFirst: the tile's stage 0, whose MFMAs start from zero.
template <int t, int kCopy, int kExtraVm, bool kLast, bool kFirst, bool kEpi>
__device__ __forceinline__ void w8a8_slot(f32x4 (&acc)[8][8], v8i (&wf)[8], v8i (&xf)[8], u32x4 (&eb)[4],
                                          const StageCtx& c) {
  constexpr int kFree = kSlotFree, kMid = kSlotMid;
  constexpr SlotOp op = kSlotPlan.op[t];
  constexpr int i = (t < 32 ? 0 : 4) + (t & 3), b = (t & 31) >> 2;
  const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
  acc[i][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[i], xf[b], kFirst ? zero : acc[i][b], 0, 0, 0, 0,
                                                               0, 0);
  if constexpr (op.kind == kSlotOwn) {
    constexpr int r = op.a;
    if constexpr (r < 2)
      set_half(xf[7], r, frag16_half(lds8_x(c.cur), c.ox[r], 7));
    else
      set_half(wf[4 + (r - 2) / 2], r & 1, frag16_half(lds8_w(c.cur), c.ow[r & 1], 4 + (r - 2) / 2));
  }
  if constexpr (t == kFree) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // this stage's buffer is free
  if constexpr (kLast) {
    // no stage s + 1: the next tile's stage 1 into this buffer (KT = 1: its
    // stage 0 into the other one)
    if constexpr (op.kind == kSlotCopy) {
      constexpr int u = op.a, j = u & 7;
      if (c.has_next) {
        const int buf = c.KT > 1 ? c.cur : c.nxt, k0b = c.KT > 1 ? 128 : 0;
        if constexpr (u < 8)
          c.pw.copy_masked(lds8_w(buf), k0b, c.K, j, c.wave_off);
        else
          c.px.copy_masked(lds8_x(buf), k0b, c.K, j, c.wave_off);
      }
    }
  } else {
    if constexpr (op.kind == kSlotCopy) {
      constexpr int u = op.a, j = u & 7;
      if constexpr (kCopy == 1) {
        if constexpr (u < 8)
          c.pw.copy_one(lds8_w(c.cur), c.k2, j, c.wave_off);
        else
          c.px.copy_one(lds8_x(c.cur), c.k2, j, c.wave_off);
      } else if constexpr (kCopy == 2) {
        if constexpr (u < 8)
          c.pw.copy_masked(lds8_w(c.cur), (int)c.k2, c.K, j, c.wave_off);
        else
          c.px.copy_masked(lds8_x(c.cur), (int)c.k2, c.K, j, c.wave_off);
      } else if constexpr (kCopy == 3) {
        // the next tile's stage 0 (pw, px already planned for it); without a
        // next tile every lane's offset is out of range (zeros into a buffer
        // no one reads, no memory read), so the waits count the same copies
        const int kb = c.has_next ? c.K : 0;
        if constexpr (u < 8)
          c.pw.copy_masked(lds8_w(c.cur), 0, kb, j, c.wave_off);
        else
          c.px.copy_masked(lds8_x(c.cur), 0, kb, j, c.wave_off);
      }
    }
    if constexpr (t == kMid) {
      constexpr int kVm = (kCopy != 0 ? kSlotPlan.copies_before_mid : 0) + kExtraVm;
      static_assert(kVm <= kMaxVmcnt, "vmcnt range");
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kVm) : "memory");
    }
    if constexpr (op.kind == kSlotW) set_half(wf[op.a], op.e, frag16_half(lds8_w(c.nxt), c.ow[op.e], op.a));
    if constexpr (op.kind == kSlotX) set_half(xf[op.a], op.e, frag16_half(lds8_x(c.nxt), c.ox[op.e], op.a));
  }
  if constexpr (kEpi) epi_slot_ops<t>(acc, eb, c.epi, c.lane);
  __builtin_amdgcn_sched_barrier(0);
}

// The epilogue's slots past the stage's 64, in order.
template <int... ts>
__device__ __forceinline__ void epi_after_stage(const f32x4 (&acc)[8][8], u32x4 (&eb)[4], const StageCtx& c,
                                                std::integer_sequence<int, ts...>) {
  (epi_slot_ops<64 + ts>(acc, eb, c.epi, c.lane), ...);
}

template <int kCopy, int kExtraVm, bool kLast, bool kFirst, bool kEpi, int... ts>
__device__ __forceinline__ void w8a8_slots(f32x4 (&acc)[8][8], v8i (&wf)[8], v8i (&xf)[8], const StageCtx& c,
                                           std::integer_sequence<int, ts...>) {
  u32x4 eb[4];  // epilogue reads in flight to their stores
  (w8a8_slot<ts, kCopy, kExtraVm, kLast, kFirst, kEpi>(acc, wf, xf, eb, c), ...);
  if constexpr (kEpi) epi_after_stage(acc, eb, c, std::make_integer_sequence<int, kEpiPlan.end - 64>{});
}

template <int kCopy, int kExtraVm, bool kLast, bool kFirst = false, bool kEpi = kEpiNone>
__device__ __forceinline__ void w8a8_stage(f32x4 (&acc)[8][8], v8i (&wf)[8], v8i (&xf)[8],
                                           const CopyPlan<8, true>& pw, const CopyPlan<8, true>& px, int s, int p,
                                           int K, int KT, bool has_next, const int (&ow)[2], const int (&ox)[2],
                                           uint32_t wave_off, const EpiCtx& epi, int lane) {
  uint32_t k2 = (uint32_t)(s + 2) * 128u;
  // the masked copies' offsets are loop-invariant where s is known: keep
  // them from being hoisted out of the tile loop into registers
  if constexpr (kCopy == 2) asm volatile("" : "+s"(k2));
  const int b = (s + p) & 1;  // this stage's buffer
  const StageCtx c{pw, px, b, b ^ 1, k2, K, KT, has_next, ow, ox, wave_off, epi, lane};
  w8a8_slots<kCopy, kExtraVm, kLast, kFirst, kEpi>(acc, wf, xf, c, std::make_integer_sequence<int, 64>{});
}

// Issue the copies of stages 0 and 1 of a tile into buffers 0 and 1.
__device__ __forceinline__ void w8a8_first_stages(const CopyPlan<8, true>& pw, const CopyPlan<8, true>& px, int K,
                                                  int KT, uint32_t wave_off) {
  pw.copy(lds8_w(0), 0, K, wave_off);
  px.copy(lds8_x(0), 0, K, wave_off);
  if (KT > 1) {
    pw.copy(lds8_w(1), 128, K, wave_off);
    px.copy(lds8_x(1), 128, K, wave_off);
  }
}

// Fused gate/up + SwiGLU epilogue for rows [32 j, 32 j + 32) of the tile.
// Waves (wm, 0) hold the gate and (wm, 1) the up projection of the same
// 128 x 128 block of h. Each wave stages bf16(acc * alpha) of its rows in
// its 8 KiB area `epi + wave * 8 KiB` (the layout of epilogue_rows) -- the
// same bf16 values the separate GEMMs would write -- then, after a barrier,
// wave (wm, wn) combines rows [16 wn, 16 wn + 16) of the pass: silu(g) * u
// in float32 (the two-input SwiGLU rule) and either its E4M3 code with
// rs = 1 / s_h (kFp8Out) or its bf16 rounding, 16 columns per lane and row,
// stored through the h resource of rows m_base..+128 (rows past M and
// columns past I dropped). A second barrier frees the areas. With kF16 the
// staged values and a 16-bit h are binary16 instead of bf16 (the fp16
// activation form of the separate GEMMs and SwiGLU).
template <bool kFp8Out, bool kF16 = false, class Acc>
__device__ __forceinline__ void epilogue_swiglu(const Acc& acc, int j, uint8_t* epi, int wm, int wn, float alpha,
                                                float rs, __amdgpu_buffer_rsrc_t out, int n_base, int I, int lane) {
  asm volatile("" : "+v"(lane));
  stage_rows<kF16>(acc, j, epi + (wm * 2 + wn) * kW8A8EpiWave, alpha, lane);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  const uint8_t* ga = epi + (wm * 2) * kW8A8EpiWave;
  const uint8_t* ua = ga + kW8A8EpiWave;
  const int cp = lane & 7;  // columns [16 cp, 16 cp + 16) of the block
  const int col = n_base + 16 * cp;
  constexpr int kBytes = kFp8Out ? 1 : 2;  // per h element
#pragma unroll
  for (int q = 0; q < kSwiGLURowsPerLane; ++q) {
    const int r = 16 * wn + 8 * q + (lane >> 3);  // row within the pass
    u32x4 gv[2], uv[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int off = r * 256 + (((2 * cp + e) ^ (r & 15)) * 16);
      gv[e] = *reinterpret_cast<const u32x4*>(ga + off);
      uv[e] = *reinterpret_cast<const u32x4*>(ua + off);
    }
    float hv[16];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const uint32_t gw = gv[w >> 2][w & 3], uw = uv[w >> 2][w & 3];
      hv[2 * w] = silu_mul(h16_lo<kF16>(gw), h16_lo<kF16>(uw));
      hv[2 * w + 1] = silu_mul(h16_hi<kF16>(gw), h16_hi<kF16>(uw));
    }
    const uint32_t o = col < I ? (uint32_t)(((32 * j + r) * I + col) * kBytes) : kOutOfRange;
    if constexpr (kFp8Out) {
      u32x4 codes;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        codes[w] = swiglu_codes4(hv[4 * w], hv[4 * w + 1], hv[4 * w + 2], hv[4 * w + 3], rs);
      __builtin_amdgcn_raw_buffer_store_b128(codes, out, (int)o, 0, 0);
    } else {
      u32x4 lo, hi;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        lo[w] = h16x2<kF16>(hv[2 * w], hv[2 * w + 1]);
        hi[w] = h16x2<kF16>(hv[8 + 2 * w], hv[8 + 2 * w + 1]);
      }
      __builtin_amdgcn_raw_buffer_store_b128(lo, out, (int)o, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(hi, out, (int)(o + 16u), 0, 0);
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Output resource of the fused h: rows [m_base, min(M, m_base + 128)) of an
// [M, I] tensor of `bytes`-byte elements.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t h_rsrc(void* h, int M, int m_base, int I, int bytes) {
  const int rows = __builtin_amdgcn_readfirstlane(max(0, min(M - m_base, 128)));
  return __builtin_amdgcn_make_buffer_rsrc(static_cast<uint8_t*>(h) + (int64_t)min(m_base, M) * I * bytes, (short)0,
                                           rows * I * bytes, 0x00020000);
}

// Persistent W8A8 kernel: one workgroup per CU walks the tiles of dispatch
// slots blockIdx.x, blockIdx.x + gridDim.x, ... The copies run across tile
// changes at the steady rate of one stage per stage: a tile's stage KT - 2
// copies the next tile's stage 0 and its last stage the next tile's stage 1,
// each into the buffer it frees (so a tile starts on the buffer parity the
// previous one left), and their latency overlaps the last MFMAs and the
// tile's output stores (which go through an LDS area of each wave's own).
// The next tile waits for its stage 0 with a count that skips those stores
// (they were issued later), and for stage 1 inside its stage 0, so it never
// waits for the stores.
// kSwiGLU: the fused gate/up + SwiGLU form. A tile is 256 rows of M by 128
// columns of h; weight rows 0-127 of the tile are the gate rows and 128-255
// the up rows of those columns (a.g[0]: gate, h output, alpha s_in s_gate;
// a.g[1]: up, alpha s_in s_up; a.out_rs = 1 / s_h), so the accumulators of
// waves (wm, 0) and (wm, 1) are g and u of the same block.
// kNormRope: groups 0 and 1 (Q and K, heads of 128 columns) take the
// per-head RMSNorm + RoPE epilogue (a.nr_*), the other groups the plain one.
// kSplit: split-K; every group is one K slice (a.ks bytes from g.koff, row
// pitch a.k) of the same product and stores its unscaled float32 partial.
template <bool kSwiGLU, bool kNormRope = false, bool kSplit = false>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1))) void
gemm_w8a8_kernel(const GemmArgs a) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave >> 1, wn = wave & 1;
  const int LD = a.k;                 // row pitch of x and w
  const int K = kSplit ? a.ks : a.k;  // K bytes this launch's groups multiply
  const int KT = (K + 127) / 128;
  const uint32_t wave_off = (uint32_t)wave * 64 * 16;
  // the lane's fragment offsets in weight / activation block 0 (halves 0, 1)
  const int ow[2] = {frag16_offset(wn * 128 + (lane & 15), lane >> 4, 0),
                     frag16_offset(wn * 128 + (lane & 15), lane >> 4, 1)};
  const int ox[2] = {frag16_offset(wm * 128 + (lane & 15), lane >> 4, 0),
                     frag16_offset(wm * 128 + (lane & 15), lane >> 4, 1)};
  uint8_t* epi = lds_mem + kW8A8EpiOffset + wave * kW8A8EpiWave;
  // dynamic quantization: the input scale is read from device memory and
  // multiplies the host's weight_scale (the same float product as s_in * s_w)
  const float alpha_mul = a.in_scale_dev != nullptr ? *a.in_scale_dev : 1.0f;

  CopyPlan<8, true> pw, px;
  auto plan_tile = [&](const TileCoord& t) {
    if constexpr (kSwiGLU) {
      const int64_t off = (int64_t)t.n0 * K;
      const int rows = a.g[0].n - t.n0;
      pw.init2(a.g[0].w + off, rows, a.g[1].w + off, rows, K, tid);
    } else {
      pw.init(a.g[t.group].w + (kSplit ? a.g[t.group].koff : 0), t.n0, a.g[t.group].n - t.n0, LD, tid);
    }
    px.init(static_cast<const uint8_t*>(a.x) + (kSplit ? a.g[t.group].koff : 0), t.m0, a.m - t.m0, LD, tid);
  };
  constexpr int kTN = kSwiGLU ? kTileN / 2 : kTileN;
  // The previous tile's epilogue stores are younger than this tile's stage 0
  // and 1 copies; the waits below skip them, as many as a wait can encode
  // beside the kStageCopies copies of stage 1.
  constexpr int kStageCopies = 2 * 8;  // pw and px, 8 chunks each
  constexpr int kStores = clamp_vmcnt(tile_stores(kSwiGLU ? 2 : kSplit ? 1 : 0) + kStageCopies) - kStageCopies;
  static_assert(kStores > 0 && kStageCopies + kStores <= kMaxVmcnt, "vmcnt range");

  // The plain bf16 output leaves through the overlapped epilogue; the fused
  // forms (SwiGLU, QK norm, split-K partials) keep a separate epilogue after
  // the tile's last stage.
  constexpr bool kOverlap = !kSwiGLU && !kNormRope && !kSplit;

  int slot = blockIdx.x;
  TileCoord tc = tile_at<kTN>(a, slot);
  plan_tile(tc);
  w8a8_first_stages(pw, px, K, KT, wave_off);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  f32x4 acc[8][8];
  int p = 0;  // buffer parity: a tile's stage s uses buffer (s + p) % 2
  for (;;) {
    const TileCoord cur = tc;
    const GemmGroup& grp = a.g[cur.group];
    const int next = slot + (int)gridDim.x;
    const bool has_next = next < a.total_tiles;
    // stage 0 has landed for every wave. Younger, after the first tile: with
    // KT > 1 stage 1's copies and all of the previous tile's stores (stage 0
    // came from that tile's stage KT - 2); with KT = 1 the stores issued
    // after the last stage's last copy.
    constexpr int kStartVm = kStageCopies + (kOverlap ? kEpiStores : kStores);
    constexpr int kStartVm1 = kOverlap ? kEpiStoresAfterLastCopy : kStores;
    static_assert(kStartVm <= kMaxVmcnt, "vmcnt range");
    if (KT > 1)
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kStartVm) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kStartVm1) : "memory");
    // stage 0's fragments but xf[7] and wf[4..7], which the stage reads itself
    v8i wf[8], xf[8];
#pragma unroll
    for (int f = 0; f < 4; ++f) read_frag16(wf[f], lds8_w(p), ow, f);
#pragma unroll
    for (int f = 0; f < 7; ++f) read_frag16(xf[f], lds8_x(p), ox, f);
    if constexpr (!kOverlap) {
      // the fused epilogues' register allocation comes out better with
      // accumulators cleared at the tile start than with stage 0 from zero
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[i][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    EpiCtx ctx{};
    if constexpr (kOverlap) {
      ctx.area = epi;
      ctx.out = out_rsrc(grp, a.m, cur.m0 + wm * 128);
      ctx.alpha = grp.alpha * alpha_mul;
      ctx.col0 = cur.n0 + wn * 128;
      ctx.gn = __builtin_amdgcn_readfirstlane(grp.n);
      ctx.gld = __builtin_amdgcn_readfirstlane(grp.ldy);
    }
    // the next tile's copies start in stage KT - 2 (KT = 1: the last stage)
    auto plan_next = [&] {
      if (has_next) {
        tc = tile_at<kTN>(a, next);
        plan_tile(tc);
      }
    };

    // Stage kinds: s <= KT - 4 copies stage s + 2 (never the last, so no K
    // tail); s = KT - 3 copies the last stage with its tail masked; s = KT - 2
    // copies the next tile's stage 0; s = KT - 1 is the last. Stage 0's
    // mid-stage wait also skips the previous tile's stores issued after its
    // last copy; with the overlapped epilogue stage 0 starts from zero
    // accumulators instead of cleared ones.
    constexpr int kExtra0 = kOverlap ? kEpiStoresAfterLastCopy : kStores;
    int s = 0;
    if (KT >= 2) {
      if (KT >= 4) {
        w8a8_stage<1, kExtra0, false, kOverlap>(acc, wf, xf, pw, px, 0, p, K, KT, has_next, ow, ox, wave_off, ctx,
                                                lane);
      } else if (KT == 3) {
        w8a8_stage<2, kExtra0, false, kOverlap>(acc, wf, xf, pw, px, 0, p, K, KT, has_next, ow, ox, wave_off, ctx,
                                                lane);
      } else {
        plan_next();
        w8a8_stage<3, kExtra0, false, kOverlap>(acc, wf, xf, pw, px, 0, p, K, KT, has_next, ow, ox, wave_off, ctx,
                                                lane);
      }
      for (s = 1; s + 3 < KT; ++s)
        w8a8_stage<1, 0, false>(acc, wf, xf, pw, px, s, p, K, KT, has_next, ow, ox, wave_off, ctx, lane);
      if (s == KT - 3) {
        w8a8_stage<2, 0, false>(acc, wf, xf, pw, px, s, p, K, KT, has_next, ow, ox, wave_off, ctx, lane);
        ++s;
      }
      if (s == KT - 2) {
        plan_next();
        w8a8_stage<3, 0, false>(acc, wf, xf, pw, px, s, p, K, KT, has_next, ow, ox, wave_off, ctx, lane);
        ++s;
      }
    } else {
      plan_next();
    }
    constexpr bool kEpiLast = kOverlap;  // the overlapped epilogue
    if (kOverlap && KT == 1)
      w8a8_stage<0, 0, true, kOverlap, kEpiLast>(acc, wf, xf, pw, px, s, p, K, KT, has_next, ow, ox, wave_off, ctx,
                                                 lane);
    else
      w8a8_stage<0, 0, true, false, kEpiLast>(acc, wf, xf, pw, px, s, p, K, KT, has_next, ow, ox, wave_off, ctx,
                                              lane);
    if constexpr (kSwiGLU) {
      const int I = grp.n;
      const __amdgpu_buffer_rsrc_t out = h_rsrc(grp.y, a.m, cur.m0 + wm * 128, I, 1);
      const float alpha = wn ? a.g[1].alpha : a.g[0].alpha;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        epilogue_swiglu<true>(acc, j, lds_mem + kW8A8EpiOffset, wm, wn, alpha, a.out_rs, out, cur.n0, I, lane);
    } else if constexpr (kSplit) {
      const __amdgpu_buffer_rsrc_t out4 = out_rsrc<4>(grp, a.m, cur.m0 + wm * 128);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
          epilogue_rows_f32<kSplitPartialStore>(acc, j, hf, epi, grp, 1.0f, out4, cur.n0 + wn * 128, lane);
    } else if constexpr (kNormRope) {
      const __amdgpu_buffer_rsrc_t out = out_rsrc(grp, a.m, cur.m0 + wm * 128);
      const bool active = cur.group < 2;
      const uint16_t* nw = cur.group == 0 ? a.nr_w[0] : a.nr_w[1];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        epilogue_rows_norm_rope(acc, j, epi, grp, grp.alpha, out, cur.n0 + wn * 128, lane, cur.m0 + wm * 128, a.m,
                                active, nw, a.nr_cos, a.nr_sin, a.nr_eps);
    }  // else the output went out with the last stage
    if (!has_next) break;
    slot = next;
    p = (p + KT) & 1;
  }
}

// ------------------------------------------------------------------ W8A16

// Activation and output forms of the W8A16 kernel.
enum W16Form : int {
  kFormBf16 = kW16Bf16,  // bf16 activation and output, bf16 MFMA
  kFormF16 = kW16F16,    // binary16 activation and output, fp16 MFMA
  kFormF32 = kW16F32,    // float32 activation as three bf16 pieces per
                         // 64-element block (hi, mid, lo: 3 K exact
                         // products), float32 output
};

// The MFMA operand format: binary16 for kFormF16, else bf16.
template <int kForm>
using W16Op = typename std::conditional<kForm == kFormF16, v8h, v8bf>::type;

// Eight exact E4M3 -> bf16 (or binary16) conversions of one dword pair;
// every E4M3 value is representable in both formats.
template <int kForm>
__device__ __forceinline__ W16Op<kForm> dequant8(uint32_t d0, uint32_t d1) {
  if constexpr (kForm == kFormF16) {
    const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, false);
    const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, true);
    const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, false);
    const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, true);
    v8h v;
    v[0] = p0[0]; v[1] = p0[1]; v[2] = p1[0]; v[3] = p1[1];
    v[4] = p2[0]; v[5] = p2[1]; v[6] = p3[0]; v[7] = p3[1];
    return v;
  } else {
    const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false);
    const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true);
    const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false);
    const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true);
    v8bf v;
    v[0] = p0[0]; v[1] = p0[1]; v[2] = p1[0]; v[3] = p1[1];
    v[4] = p2[0]; v[5] = p2[1]; v[6] = p3[0]; v[7] = p3[1];
    return v;
  }
}

template <int kForm>
__device__ __forceinline__ f32x4 w16_mfma(W16Op<kForm> w, u32x4 x, f32x4 acc) {
  if constexpr (kForm == kFormF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(w, __builtin_bit_cast(v8h, x), acc, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(w, __builtin_bit_cast(v8bf, x), acc, 0, 0, 0);
}

constexpr int kW16Copies = 4 + 8;  // copies per thread per stage: 4 weight and 8 activation chunks
// Buffer stores per thread per tile of the epilogue forms.
template <bool kSwiGLU, int kForm, bool kSplit = false>
constexpr int kW16EpilogueStores = tile_stores(kSwiGLU ? 3 : (kForm == kFormF32 || kSplit) ? 1 : 0);

// Persistent W8A16 pipeline: K stages of 64 elements; one workgroup per CU
// walks the tiles of dispatch slots blockIdx.x, blockIdx.x + gridDim.x, ...
// Stage g (counted over all tiles of the workgroup) sits in LDS buffer g % 3.
// The copy cursor runs two stages ahead of the matrix cores, across tile
// boundaries, so the first stages of the next tile are in flight while a
// tile finishes; past the workgroup's last tile it copies zeros into
// buffers no one reads. Fragments are double-buffered in registers by half
// stage (32 K each): set A holds (g, h0), set B (g, h1).
// kSwiGLU: tiles of 128 columns whose weight rows 0-127 are gate and
// 128-255 up rows (a.g[0], a.g[1]), as in the fused W8A8 kernel.
// kForm == kFormF32: the activation is the three-piece bf16 form, 3 stages
// per 64-element weight block (stage k reads weight block k / 3).
// kSplit: group g multiplies K elements [g.koff, g.koff + a.ks) (row pitch
// a.k), so its copies start koff elements into the weight and activation rows.
// kKTail: K (or the slice) is not a whole number of 64-element stages, so the
// last stage's chunks beyond it must read zero. Otherwise every copy lies
// inside K (the cursor moves to the next tile after a tile's last stage) and
// needs no per-lane test: each vector instruction in the stage loop costs
// matrix-core time.
template <bool kSwiGLU, int kForm, bool kSplit = false, bool kKTail = true>
struct W16Copier {
  CopyPlan<4> pw;  // E4M3 weight, 64-byte stage rows
  CopyPlan<8> px;                   // bf16 activation, 128-byte stage rows
  int tile_slot;   // dispatch slot of the tile being copied
  int k;           // next stage of that tile

  __device__ __forceinline__ void start_tile(const GemmArgs& a, int slot, int tid) {
    const TileCoord tc = tile_at<kSwiGLU ? kTileN / 2 : kTileN>(a, slot);
    tile_slot = slot;
    k = 0;
    if constexpr (kSwiGLU) {
      const int64_t off = (int64_t)tc.n0 * a.k;
      const int rows = a.g[0].n - tc.n0;
      pw.init2(a.g[0].w + off, rows, a.g[1].w + off, rows, a.k, tid);
    } else {
      pw.init(a.g[tc.group].w + (kSplit ? a.g[tc.group].koff : 0), tc.n0, a.g[tc.group].n - tc.n0, a.k, tid);
    }
    px.init(static_cast<const uint8_t*>(a.x) + (kSplit ? 2 * (int64_t)a.g[tc.group].koff : 0), tc.m0, a.m - tc.m0,
            (int64_t)(kForm == kFormF32 ? a.xk : a.k) * 2, tid);
  }

  // Copy c of the current stage into buffer `buf`: c < 4 weight chunk c,
  // else activation chunk c - 4; weight chunks beyond K and activation
  // chunks beyond XK (the activation row length) read as zero.
  __device__ __forceinline__ void issue(int c, int buf, int K, int XK, uint32_t wave_off) const {
    if (c < 4) {
      const int k0b = (kForm == kFormF32 ? k / 3 : k) * 64;
      const uint32_t o = pw.off(c);
      pw.dma(c, kKTail && k0b + pw.kbyte >= K ? kOutOfRange : o, (uint32_t)k0b,
            lds_addr(lds16_w(buf)) + c * kThreads * 16 + wave_off);
    } else {
      const int k0b = k * 128;
      const uint32_t o = px.off(c - 4);
      px.dma(c - 4, kKTail && k0b + px.kbyte >= 2 * XK ? kOutOfRange : o, (uint32_t)k0b,
            lds_addr(lds16_x(buf)) + (c - 4) * kThreads * 16 + wave_off);
    }
  }

  __device__ __forceinline__ void advance(const GemmArgs& a, int KT, int tid) {
    if (++k == KT) {
      const int next = tile_slot + (int)gridDim.x;
      if (next < a.total_tiles) {
        start_tile(a, next, tid);
      } else {
        k = 0;
        pw.exhaust();
        px.exhaust();
      }
    }
  }
};

// One half stage (32 K values) of fragments for v_mfma_f32_16x16x32_bf16
// (or _f16): lane (r, q) = (l % 16, l / 16) holds K values [8 q, 8 q + 8) of
// the half for row r of each 16-row block -- weight block i as 8 E4M3 bytes
// (w[i]), activation block b as 8 bf16 (x[b]). Both operands take the same
// K values per lane, so the products pair up.
struct W16Half {
  u32x2 w[8];
  u32x4 x[8];
};

// Per-lane byte offsets of a lane's fragments for half h inside the weight
// and activation tiles of a buffer; block i or b adds 1024 (16 rows of 64
// bytes) or 2048 (16 rows of 128 bytes). Blocks 16 rows apart keep row bits
// 0-3 and with them row64, swz4 and swz8 of the lane's row.
struct W16Addr {
  uint32_t w[2], x[2];
  __device__ __forceinline__ void init(int row_w, int row_x, int q) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // E4M3 bytes [32 h + 8 q, +8) of the 64-byte weight row: half (q & 1) of chunk 2 h + q / 2
      w[h] = row64(row_w) * 64 + ((2 * h + (q >> 1)) ^ swz4(row_w)) * 16 + (q & 1) * 8;
      // bf16 values [32 h + 8 q, +8) of the 128-byte activation row: chunk 4 h + q
      x[h] = row_x * 128 + ((4 * h + q) ^ swz8(row_x)) * 16;
    }
  }
};

// Read r (0..15) of half h of the stage in buffer b into f: r < 8 weight
// block r, else activation block r - 8. The buffer's base is passed in
// (lds_w, lds_x) so that the compiler forms one address per half and uses
// the instruction offset for the block.
__device__ __forceinline__ void w16_read(W16Half& f, int r, const uint8_t* lds_w, const uint8_t* lds_x, int h,
                                         const W16Addr& ad) {
  if (r < 8)
    f.w[r] = *reinterpret_cast<const u32x2*>(lds_w + ad.w[h] + r * 1024);
  else
    f.x[r - 8] = lds_chunk(lds_x, ad.x[h] + (r - 8) * 2048);
}

// Half stage on set f: 64 MFMAs, weight-block-major (MFMA t: weight block
// t / 8, activation block t % 8); weight block i + 1 is dequantized four
// MFMAs before its first use. Each MFMA is followed by at most one memory
// operation, placed by the slot plan below:
//   first half : the 16 reads of the second half's fragments (set nf) at
//                odd slots 1-31, and copies 0-5 of stage g + 2 five slots
//                apart from slot 34. Their buffer held stage g - 1, which
//                every wave finished reading before the previous stage's
//                barrier (lgkmcnt(0) precedes it).
//   second half: after MFMA 3, vmcnt + lgkmcnt(0) + barrier: stage g + 1 has
//                landed for every wave (only the first half's copies, and
//                after a tile change the previous tile's output stores, are
//                younger than its copies); then the 16 reads of the next
//                stage's first-half fragments at even slots 4-34, and copies
//                6-11 five slots apart from slot 37.
enum W16SlotKind : int { kW16None, kW16Read, kW16Copy };
struct W16Slot {
  int kind, a;  // read: fragment block a (0-15); copy: chunk a (0-11)
};
struct W16Plan {
  W16Slot op[2][64];       // [half][MFMA]
  int wait_slot;           // second half: stage g + 1 is waited for after this MFMA
  int copies_before_wait;  // copies of stage g + 2 issued before that wait
  bool ok;
};

constexpr W16Plan make_w16_plan() {
  W16Plan p{};
  p.ok = true;
  p.wait_slot = 3;
  auto put = [&](int h, int t, int kind, int a) {
    if (t < 0 || t >= 64 || p.op[h][t].kind != kW16None) p.ok = false;
    else p.op[h][t] = W16Slot{kind, a};
  };
  for (int r = 0; r < 16; ++r) put(0, 1 + 2 * r, kW16Read, r);
  for (int c = 0; c < kW16Copies / 2; ++c) put(0, 34 + 5 * c, kW16Copy, c);
  for (int r = 0; r < 16; ++r) put(1, 4 + 2 * r, kW16Read, r);
  for (int c = 0; c < kW16Copies / 2; ++c) put(1, 37 + 5 * c, kW16Copy, kW16Copies / 2 + c);
  // every chunk copied exactly once per stage, every fragment block read once per half
  int copies = 0, reads[2] = {0, 0};
  for (int h = 0; h < 2; ++h)
    for (int t = 0; t < 64; ++t) {
      if (p.op[h][t].kind == kW16Copy) {
        if (p.op[h][t].a != copies) p.ok = false;  // chunks in order
        ++copies;
        if (h == 0 || t <= p.wait_slot) ++p.copies_before_wait;
      }
      if (p.op[h][t].kind == kW16Read) {
        if (p.op[h][t].a != reads[h]) p.ok = false;
        ++reads[h];
        // the second half reads stage g + 1: only after its wait and barrier
        if (h == 1 && t <= p.wait_slot) p.ok = false;
      }
    }
  if (copies != kW16Copies || reads[0] != 16 || reads[1] != 16) p.ok = false;
  return p;
}

constexpr W16Plan kW16Plan = make_w16_plan();
static_assert(kW16Plan.ok, "the W8A16 half stages' memory operations must fit their slots");
// vmcnt of the wait for stage g + 1: the copies issued after its last copy
constexpr int kW16StageWait = kW16Plan.copies_before_wait;
static_assert(kW16StageWait == kW16Copies / 2 && kW16StageWait <= kMaxVmcnt, "vmcnt of the stage wait");
// ... and in a tile's first stage, where the previous tile's epilogue stores
// are younger too (clamped: a larger count would wait for some stores too)
template <bool kSwiGLU, int kForm, bool kSplit = false>
constexpr int kW16AfterStoresWait = clamp_vmcnt(kW16StageWait + kW16EpilogueStores<kSwiGLU, kForm, kSplit>);
static_assert(kW16AfterStoresWait<false, kFormBf16> == 38 && kW16AfterStoresWait<true, kFormBf16> == 22 &&
                  kW16AfterStoresWait<false, kFormF32> == kMaxVmcnt,
              "after-stores waits");

// MFMA t of a half stage and the memory operation that follows it.
template <int t, bool kSecond, bool kReadNext, bool kSwiGLU, int kForm, bool kSplit, class Copier>
__device__ __forceinline__ void w16_slot(f32x4 (&acc)[8][8], const W16Half& f, W16Half& nf, W16Op<kForm>& wcur,
                                         W16Op<kForm>& wnext, const uint8_t* nw, const uint8_t* nx, int nh,
                                         const W16Addr& ad, Copier& cp, int cbuf, int K, int XK, uint32_t wave_off,
                                         bool after_stores) {
  constexpr int i = t >> 3, b = t & 7;
  constexpr W16Slot op = kW16Plan.op[kSecond ? 1 : 0][t];
  if constexpr (b == 4 && i < 7) wnext = dequant8<kForm>(f.w[i + 1][0], f.w[i + 1][1]);
  acc[i][b] = w16_mfma<kForm>(wcur, f.x[b], acc[i][b]);
  if constexpr (b == 7) wcur = wnext;
  if constexpr (kSecond && t == kW16Plan.wait_slot) {
    if (after_stores)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kW16AfterStoresWait<kSwiGLU, kForm, kSplit>) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kW16StageWait) : "memory");
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  if constexpr (op.kind == kW16Read && (!kSecond || kReadNext)) w16_read(nf, op.a, nw, nx, nh, ad);
  if constexpr (op.kind == kW16Copy) cp.issue(op.a, cbuf, K, XK, wave_off);
  __builtin_amdgcn_sched_barrier(0);
}

template <bool kSecond, bool kReadNext, bool kSwiGLU, int kForm, bool kSplit, class Copier, int... ts>
__device__ __forceinline__ void w16_slots(f32x4 (&acc)[8][8], const W16Half& f, W16Half& nf, W16Op<kForm>& wcur,
                                          W16Op<kForm>& wnext, const uint8_t* nw, const uint8_t* nx, int nh,
                                          const W16Addr& ad, Copier& cp, int cbuf, int K, int XK, uint32_t wave_off,
                                          bool after_stores, std::integer_sequence<int, ts...>) {
  (w16_slot<ts, kSecond, kReadNext, kSwiGLU, kForm, kSplit>(acc, f, nf, wcur, wnext, nw, nx, nh, ad, cp, cbuf, K, XK,
                                                            wave_off, after_stores),
   ...);
}

// A half stage on set f, reading into nf from buffer nb (half nh of it).
// kSecond: the stage's second half (waits for stage g + 1, reads its first
// half unless kReadNext is false); after_stores: the tile's first stage
// after an epilogue (the wait skips that tile's stores).
template <bool kSecond, bool kReadNext, bool kSwiGLU, int kForm, bool kSplit, class Copier>
__device__ __forceinline__ void w16_half(f32x4 (&acc)[8][8], const W16Half& f, W16Half& nf, int nb, int nh,
                                         const W16Addr& ad, Copier& cp, int cbuf, int K, int XK, uint32_t wave_off,
                                         bool after_stores) {
  // the next set's buffer base, kept opaque so that per-block addresses are
  // not precomputed for every buffer
  uint32_t bw = lds_addr(lds16_w(nb)), bx = lds_addr(lds16_x(nb));
  asm volatile("" : "+s"(bw), "+s"(bx));
  const uint8_t* nw = lds_mem + (bw - lds_addr(lds_mem));
  const uint8_t* nx = lds_mem + (bx - lds_addr(lds_mem));
  W16Op<kForm> wcur = dequant8<kForm>(f.w[0][0], f.w[0][1]), wnext;
  w16_slots<kSecond, kReadNext, kSwiGLU, kForm, kSplit>(acc, f, nf, wcur, wnext, nw, nx, nh, ad, cp, cbuf, K, XK,
                                                        wave_off, after_stores, std::make_integer_sequence<int, 64>{});
}

// One stage: its first half on set fa (reading the second half's fragments
// into fb), its second half on fb (reading the next stage's first half into
// fa unless kReadNext is false). after_stores: the tile's first stage after
// another tile's epilogue.
template <bool kReadNext, bool kSwiGLU, int kForm, bool kSplit, class Copier>
__device__ __forceinline__ void w16_stage(f32x4 (&acc)[8][8], W16Half& fa, W16Half& fb, int b, const W16Addr& ad,
                                          Copier& cp, int K, int XK, uint32_t wave_off, bool after_stores) {
  const int nb = b == 2 ? 0 : b + 1;   // next stage's buffer
  const int cb = nb == 2 ? 0 : nb + 1;  // buffer of stage + 2 (so written, it stays scalar)
  w16_half<false, true, kSwiGLU, kForm, kSplit>(acc, fa, fb, b, 1, ad, cp, cb, K, XK, wave_off, false);
  w16_half<true, kReadNext, kSwiGLU, kForm, kSplit>(acc, fb, fa, nb, 0, ad, cp, cb, K, XK, wave_off, after_stores);
}

// kSwiGLU: the fused gate/up + SwiGLU form with a 16-bit h (the 16-bit
// step's split MLP), tiles and weight rows as in the fused W8A8 kernel;
// a.g[0]: gate, h output, alpha s_gate; a.g[1]: up, alpha s_up.
// kForm: bf16, binary16 or (not with kSwiGLU) the float32 three-piece form,
// whose activation rows hold a.xk = 3 * 64 * ceil(K / 64) bf16 values.
// kSplit (bf16 only): split-K; every group is one K slice (a.ks elements
// from g.koff, row pitch a.k) of the same product and stores its unscaled
// float32 partial to its y.
// kKTail: as for W16Copier (false only when K, or the slice, is a multiple
// of 64).
template <bool kSwiGLU, int kForm, bool kSplit = false, bool kKTail = true>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1))) void
gemm_w8a16_kernel(const GemmArgs a) {
  static_assert(!(kSwiGLU && kForm == kFormF32), "the fused SwiGLU form has a 16-bit h");
  static_assert(!kSplit || (!kSwiGLU && kForm == kFormBf16), "split-K: the plain bf16 form");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave >> 1, wn = wave & 1;
  const int K = kSplit ? a.ks : a.k;              // K elements this launch's groups multiply
  const int XK = kForm == kFormF32 ? a.xk : K;  // the 16-bit forms keep XK == K visible
  const int KT = (XK + 63) / 64;  // stages: 64 activation values each
  const uint32_t wave_off = (uint32_t)wave * 64 * 16;
  W16Addr ad;
  ad.init(wn * 128 + (lane & 15), wm * 128 + (lane & 15), lane >> 4);

  W16Copier<kSwiGLU, kForm, kSplit, kKTail> cp;
  cp.start_tile(a, blockIdx.x, tid);
#pragma unroll
  for (int v = 0; v < 2; ++v) {
#pragma unroll
    for (int c = 0; c < kW16Copies; ++c) cp.issue(c, v, K, XK, wave_off);
    cp.advance(a, KT, tid);
  }
  wait_vmem_and_barrier<kW16Copies>();  // stage 0 has landed

  W16Half fa, fb;
  int b = 0;  // buffer of the current stage
  if constexpr (kSwiGLU) {
#pragma unroll
    for (int r = 0; r < 16; ++r) w16_read(fa, r, lds16_w(0), lds16_x(0), 0, ad);
  }

  for (int tile_slot = blockIdx.x; tile_slot < a.total_tiles; tile_slot += (int)gridDim.x) {
    const bool first = tile_slot == (int)blockIdx.x;
    // The plain forms read the tile's first half-stage fragments here, not
    // during the previous tile's last stage, so that they are not live across
    // the epilogue (which spilled them). Stage 0 has landed for every wave:
    // before the first tile by the wait above, for later tiles by the wait in
    // the previous tile's last stage, and every wave has passed the barrier
    // that ends the epilogue. The fused SwiGLU form, whose register
    // allocation comes out better the other way, reads them in the last
    // stage of the previous tile.
    if constexpr (!kSwiGLU) {
#pragma unroll
      for (int r = 0; r < 16; ++r) w16_read(fa, r, lds16_w(b), lds16_x(b), 0, ad);
    }
    f32x4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // Stage s: its first half on set fa (reading the second half's
    // fragments into fb), its second half on fb (reading the next stage's
    // first half into fa, except in a plain form's last stage).
    const int full_stages = kSwiGLU ? KT : KT - 1;
    for (int s = 0; s < full_stages; ++s) {
      w16_stage<true, kSwiGLU, kForm, kSplit>(acc, fa, fb, b, ad, cp, K, XK, wave_off, s == 0 && !first);
      cp.advance(a, KT, tid);
      b = b == 2 ? 0 : b + 1;
    }
    if constexpr (!kSwiGLU) {
      w16_stage<false, kSwiGLU, kForm, kSplit>(acc, fa, fb, b, ad, cp, K, XK, wave_off, KT == 1 && !first);
      cp.advance(a, KT, tid);
      b = b == 2 ? 0 : b + 1;
    }

    // Epilogue: rows staged in the activation tile of the last stage's
    // buffer, which no wave reads once lgkmcnt(0) + barrier have passed.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    uint8_t* area = lds16_x(b == 0 ? 2 : b - 1);
    if constexpr (kSwiGLU) {
      const TileCoord tc = tile_at<kTileN / 2>(a, tile_slot);
      const int I = a.g[0].n;
      const __amdgpu_buffer_rsrc_t out = h_rsrc(a.g[0].y, a.m, tc.m0 + wm * 128, I, 2);
      const float alpha = wn ? a.g[1].alpha : a.g[0].alpha;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        epilogue_swiglu<false, kForm == kFormF16>(acc, j, area, wm, wn, alpha, 1.0f, out, tc.n0, I, lane);
    } else {
      const TileCoord tc = tile_at(a, tile_slot);
      const GemmGroup& grp = a.g[tc.group];
      uint8_t* stage = area + wave * (32 * 256);
      if constexpr (kSplit) {
        const __amdgpu_buffer_rsrc_t out = out_rsrc<4>(grp, a.m, tc.m0 + wm * 128);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
            epilogue_rows_f32<kSplitPartialStore>(acc, j, hf, stage, grp, 1.0f, out, tc.n0 + wn * 128, lane);
      } else if constexpr (kForm == kFormF32) {
        const __amdgpu_buffer_rsrc_t out = out_rsrc<4>(grp, a.m, tc.m0 + wm * 128);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
            epilogue_rows_f32(acc, j, hf, stage, grp, grp.alpha, out, tc.n0 + wn * 128, lane);
      } else {
        const __amdgpu_buffer_rsrc_t out = out_rsrc(grp, a.m, tc.m0 + wm * 128);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          epilogue_rows<kForm == kFormF16>(acc, j, stage, grp, grp.alpha, out, tc.n0 + wn * 128, lane);
      }
      // the next stage's first copies refill this buffer: every wave must be
      // done reading its staged rows first
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ------------------------------------------------------------------ small tiles
// Shapes whose 256 x 256 tiles cannot fill the device (M = 1024 rows of a
// 4096 -> 4096 projection: 64 tiles for 256 compute units) run on 128 x 128
// tiles instead, 4 waves each (W8A8: 64 x 64 per wave, 4 x 4 blocks of
// 16 x 16; W8A16: 32 output columns of all 128 rows, see its stage below),
// with the same MFMA forms, fragment layouts and LDS swizzles as the
// 256 x 256 kernels. K runs in stages held in kSmallBufs LDS buffers; the
// copies of stage s + 4 are issued during stage s, into the buffer stage s
// used, and every stage's fragments are read into registers during the
// previous stage (two register sets, so the stage loop is unrolled by two).
// One barrier per stage: after it, every wave's copies of stage s + 1 have
// landed and every wave has read stage s's buffer (lgkmcnt(0) precedes it).
// Every stage issues the same copies, so the waits count them uniformly;
// the copies of stages that reach past K (the K tail, and the stages after
// the tile's last one, into buffers no one reads) test each lane's chunk
// against K and read zeros there, which also keeps them inside the tensor
// (the K offset travels in the scalar offset, outside the buffer range
// check).
constexpr int kSmallTile = 128;
constexpr int kSmallBufs = 4;
constexpr int kSmall8Half = kSmallTile * 128;             // one operand of a W8A8 stage: 128 rows x 128 bytes
constexpr int kSmall8Stage = 2 * kSmall8Half;             // weight, then activation
constexpr int kSmall16W = kSmallTile * 64;                // W8A16: E4M3 weight, 128 rows x 64 bytes
constexpr int kSmall16Stage = kSmall16W + kSmallTile * 128;  // then the 16-bit activation, 128 x 64 values
constexpr int kSmallEpiOffset = kSmallBufs * kSmall8Stage;   // 8 KiB of staging per wave after the buffers
constexpr int kSmallEpiWave = 64 * 128;                      // 64 output rows of 128 bytes
static_assert(kSmallEpiOffset + 4 * kSmallEpiWave <= kLdsBytes, "small-tile LDS");
static_assert(kSmallBufs * kSmall16Stage <= kSmallEpiOffset, "small-tile W8A16 buffers");
constexpr int kSmall8Copies = 2 * (kSmallTile * 8 / kThreads);   // per thread per stage: 4 + 4
constexpr int kSmall16Copies = kSmallTile * 4 / kThreads + kSmallTile * 8 / kThreads;  // 2 + 4
// The wait before stage s's MFMAs is for stage s + 1; younger are the copies
// of stages s + 2 .. s + kSmallBufs - 1.
constexpr int kSmall8Wait = (kSmallBufs - 2) * kSmall8Copies;
constexpr int kSmall16Wait = (kSmallBufs - 2) * kSmall16Copies;
static_assert(kSmall8Wait <= kMaxVmcnt && kSmall16Wait <= kMaxVmcnt && (kSmallBufs - 1) * kSmall8Copies <= kMaxVmcnt,
              "vmcnt range");

__device__ __forceinline__ uint8_t* small8_w(int s) { return lds_mem + (s % kSmallBufs) * kSmall8Stage; }
__device__ __forceinline__ uint8_t* small8_x(int s) { return small8_w(s) + kSmall8Half; }
__device__ __forceinline__ uint8_t* small16_w(int s) { return lds_mem + (s % kSmallBufs) * kSmall16Stage; }
__device__ __forceinline__ uint8_t* small16_x(int s) { return small16_w(s) + kSmall16W; }

// Epilogue of a W8A8 small tile: the wave's 64 x 64 block, bf16(acc * alpha)
// (binary16 with kF16), staged in the wave's 8 KiB area (row m at m * 128,
// 16-byte chunk c at c ^ (m % 8)), then 8 stores of 8 rows x 128 bytes.
template <bool kF16>
__device__ __forceinline__ void small_epilogue(const f32x4 (&acc)[4][4], uint8_t* area, float alpha,
                                               __amdgpu_buffer_rsrc_t out, int col0, int gn, int gld, int lane) {
  asm volatile("" : "+v"(lane));
  const int q = lane >> 4, r = lane & 15;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 16 * b + r, c = 2 * i + (q >> 1);
      const f32x4 x = acc[i][b];
      u32x2 v;
      v[0] = h16x2<kF16>(x[0] * alpha, x[1] * alpha);
      v[1] = h16x2<kF16>(x[2] * alpha, x[3] * alpha);
      *reinterpret_cast<u32x2*>(area + m * 128 + ((c ^ (m & 7)) * 16) + (q & 1) * 8) = v;
    }
  const int c = lane & 7, col = col0 + 8 * c;
  u32x4 v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int row = 8 * k + (lane >> 3);
    v[k] = *reinterpret_cast<const u32x4*>(area + row * 128 + ((c ^ (row & 7)) * 16));
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int row = 8 * k + (lane >> 3);
    const uint32_t off = col < gn ? (uint32_t)(row * gld + col) * 2u : kOutOfRange;
    __builtin_amdgcn_raw_buffer_store_b128(v[k], out, (int)off, 0, kStreamStore);
  }
}

// W8A8 small-tile stage s: 16 MFMAs on set f (acc[i][b] += w[i] x[b], MFMA t
// = (t % 4, t / 4)); after the wait and barrier (MFMA kSmallBarrier) the 16
// reads of stage s + 1 into nf (r < 8: weight block r / 2 half r % 2, else
// activation block (r - 8) / 2) and the 8 copies of stage s + kSmallBufs
// (u < 4 weight chunk, else activation chunk) into the buffer of stage s,
// spread over the remaining slots.
struct Small8Frags {
  v8i w[4], x[4];
};
// The wait and barrier come after MFMA kSmallBarrier: the stage's own
// fragments are already in registers, so the first MFMAs hide the barrier.
constexpr int kSmallBarrier = 3;
// kMasked: the stage being copied may reach past K (the K tail, or the
// stages past the tile's last one, which read zeros into buffers no one
// reads); each lane then tests its chunk. Stages wholly inside K copy
// without the test.
template <bool kFirst, bool kMasked>
__device__ __forceinline__ void small8_stage(f32x4 (&acc)[4][4], const Small8Frags& f, Small8Frags& nf, int s,
                                             const CopyPlan<8, true>& pw, const CopyPlan<8, true>& px, int K,
                                             const int (&ow)[2], const int (&ox)[2], uint32_t wave_off) {
  const uint8_t* nw = small8_w(s + 1);
  const uint8_t* nx = small8_x(s + 1);
  const int kc = (s + kSmallBufs) * 128;  // K byte of the stage being copied
  const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const int i = t & 3, b = t >> 2;
    acc[i][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(f.w[i], f.x[b], kFirst ? zero : acc[i][b], 0, 0, 0,
                                                                 0, 0, 0);
    if (t == kSmallBarrier)
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(kSmall8Wait) : "memory");
    // reads r = 0..15 of stage s + 1 in slots kSmallBarrier + 1 .. 15 (two in the last ones)
    if (t > kSmallBarrier) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (r * (15 - kSmallBarrier) / 16 + kSmallBarrier + 1 == t) {
          if (r < 8)
            set_half(nf.w[r >> 1], r & 1, frag16_half(nw, ow[r & 1], r >> 1));
          else
            set_half(nf.x[(r - 8) >> 1], r & 1, frag16_half(nx, ox[r & 1], (r - 8) >> 1));
        }
    }
    // copies u = 0..7 of stage s + kSmallBufs at slots kSmallBarrier + 1 + 1.5 u
    if (t > kSmallBarrier) {
#pragma unroll
      for (int u = 0; u < kSmall8Copies; ++u)
        if ((3 * u) / 2 + kSmallBarrier + 1 == t) {
          if constexpr (kMasked) {
            if (u < 4)
              pw.copy_masked(small8_w(s), kc, K, u, wave_off);
            else
              px.copy_masked(small8_x(s), kc, K, u - 4, wave_off);
          } else {
            if (u < 4)
              pw.copy_one(small8_w(s), (uint32_t)kc, u, wave_off);
            else
              px.copy_one(small8_x(s), (uint32_t)kc, u - 4, wave_off);
          }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Persistent W8A8 small-tile kernel over 128 x 128 tiles of all groups.
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1))) void
gemm_w8a8_small_kernel(const GemmArgs a) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int K = a.k;
  const int KT = (K + 127) / 128;
  const uint32_t wave_off = (uint32_t)wave * 64 * 16;
  const int ow[2] = {frag16_offset(wn * 64 + (lane & 15), lane >> 4, 0),
                     frag16_offset(wn * 64 + (lane & 15), lane >> 4, 1)};
  const int ox[2] = {frag16_offset(wm * 64 + (lane & 15), lane >> 4, 0),
                     frag16_offset(wm * 64 + (lane & 15), lane >> 4, 1)};
  uint8_t* area = lds_mem + kSmallEpiOffset + wave * kSmallEpiWave;
  const float alpha_mul = a.in_scale_dev != nullptr ? *a.in_scale_dev : 1.0f;

  for (int slot = blockIdx.x; slot < a.total_tiles; slot += (int)gridDim.x) {
    const TileCoord tc = tile_at<kSmallTile, kSmallTile>(a, slot);
    const GemmGroup& grp = a.g[tc.group];
    CopyPlan<8, true> pw, px;
    {
      const uint8_t* w = grp.w + (int64_t)tc.n0 * K;
      const uint8_t* x = static_cast<const uint8_t*>(a.x) + (int64_t)tc.m0 * K;
      pw.init2(w, grp.n - tc.n0, w, 0, K, tid);
      px.init2(x, a.m - tc.m0, x, 0, K, tid);
    }
    // stages 0 .. kSmallBufs - 1
#pragma unroll
    for (int st = 0; st < kSmallBufs; ++st) {
#pragma unroll
      for (int u = 0; u < kSmall8Copies / 2; ++u) pw.copy_masked(small8_w(st), st * 128, K, u, wave_off);
#pragma unroll
      for (int u = 0; u < kSmall8Copies / 2; ++u) px.copy_masked(small8_x(st), st * 128, K, u, wave_off);
    }
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((kSmallBufs - 1) * kSmall8Copies) : "memory");
    Small8Frags fa, fb;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      read_frag16(fa.w[f], small8_w(0), ow, f);
      read_frag16(fa.x[f], small8_x(0), ox, f);
    }
    f32x4 acc[4][4];
    small8_stage<true, true>(acc, fa, fb, 0, pw, px, K, ow, ox, wave_off);
    // stage s copies stage s + kSmallBufs, wholly inside K while that is
    // below K / 128
    const int full_end = K / 128 - kSmallBufs;
    int s = 1;
    for (; s + 1 < KT && s + 1 < full_end; s += 2) {
      small8_stage<false, false>(acc, fb, fa, s, pw, px, K, ow, ox, wave_off);
      small8_stage<false, false>(acc, fa, fb, s + 1, pw, px, K, ow, ox, wave_off);
    }
    for (; s + 1 < KT; s += 2) {
      small8_stage<false, true>(acc, fb, fa, s, pw, px, K, ow, ox, wave_off);
      small8_stage<false, true>(acc, fa, fb, s + 1, pw, px, K, ow, ox, wave_off);
    }
    if (s < KT) small8_stage<false, true>(acc, fb, fa, s, pw, px, K, ow, ox, wave_off);

    const int gn = __builtin_amdgcn_readfirstlane(grp.n), gld = __builtin_amdgcn_readfirstlane(grp.ldy);
    const int rows = __builtin_amdgcn_readfirstlane(max(0, min(a.m - (tc.m0 + wm * 64), 64)));
    uint8_t* base = static_cast<uint8_t*>(grp.y) + (int64_t)min(tc.m0 + wm * 64, a.m) * gld * 2;
    const __amdgpu_buffer_rsrc_t out = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, rows * gld * 2, 0x00020000);
    small_epilogue<false>(acc, area, grp.alpha * alpha_mul, out, tc.n0 + wn * 64, gn, gld, lane);
    // the copies of stages past K are still landing in the buffers the next
    // tile's first copies refill, and every wave must be done with them
    asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
}

// W8A16 small tiles use a different wave split from W8A8: wave w takes the
// 32 output columns [32 w, 32 w + 32) of all 128 rows (2 weight blocks x 8
// activation blocks of 16), so each weight block it converts to bf16 (four
// v_cvt_scalef32_pk_bf16_fp8 per lane) feeds 8 MFMAs instead of 4; vector
// instructions in the stage loop are not hidden behind the 16-cycle MFMAs,
// and with 64 x 64 wave tiles the conversions (one per MFMA) were the
// kernel's largest cost. Reads per stage: 20 instead of 16.
//
// Stage s (64 K values, two halves of 32): 32 MFMAs on set f, weight-block
// major within a half (MFMA t of half h: weight block (t % 16) / 8,
// activation block t % 8), the next weight block converted two MFMAs before
// its first use; after the wait and barrier (MFMA kSmallBarrier) the 20
// reads of stage s + 1 into nf, one per slot (r = 10 h + j: j < 2 weight
// block j of half h, else activation block j - 2), and at t = 21, 23, .. 31
// copy (t - 21) / 2 of stage s + kSmallBufs (< 2 weight chunk, else
// activation chunk).
struct Small16Frags {
  u32x2 w[2][2];
  u32x4 x[2][8];
};
constexpr int kSmall16Reads = 2 * (2 + 8);
static_assert(kSmallBarrier + kSmall16Reads < 32, "the reads of the next stage fit the stage's slots");
// kMasked: as for small8_stage.
template <int kForm, bool kFirst, bool kMasked>
__device__ __forceinline__ void small16_stage(f32x4 (&acc)[2][8], const Small16Frags& f, Small16Frags& nf, int s,
                                              const CopyPlan<4>& pw, const CopyPlan<8>& px, int K,
                                              const W16Addr& ad, uint32_t wave_off) {
  const uint8_t* nw = small16_w(s + 1);
  const uint8_t* nx = small16_x(s + 1);
  const int kw = (s + kSmallBufs) * 64;   // weight K byte of the stage being copied
  const int kx = (s + kSmallBufs) * 128;  // activation K byte
  const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
  W16Op<kForm> wcur = dequant8<kForm>(f.w[0][0][0], f.w[0][0][1]), wnext;
#pragma unroll
  for (int t = 0; t < 32; ++t) {
    const int h = t >> 4, i = (t >> 3) & 1, b = t & 7;
    if (b == 6) {
      const int hn = i == 1 ? h + 1 : h, in = i ^ 1;
      if (hn < 2) wnext = dequant8<kForm>(f.w[hn][in][0], f.w[hn][in][1]);
    }
    acc[i][b] = w16_mfma<kForm>(wcur, f.x[h][b], (kFirst && h == 0) ? zero : acc[i][b]);
    if (b == 7) wcur = wnext;
    if (t == kSmallBarrier)
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(kSmall16Wait) : "memory");
    if (t > kSmallBarrier && t <= kSmallBarrier + kSmall16Reads) {
      const int r = t - kSmallBarrier - 1, hh = r / 10, j = r % 10;
      if (j < 2)
        nf.w[hh][j] = *reinterpret_cast<const u32x2*>(nw + ad.w[hh] + j * 1024);
      else
        nf.x[hh][j - 2] = lds_chunk(nx, ad.x[hh] + (j - 2) * 2048);
    }
    if (t >= 21 && (t & 1)) {
      const int u = (t - 21) >> 1;
      if constexpr (kMasked) {
        if (u < 2)
          pw.copy_masked(small16_w(s), kw, K, u, wave_off);
        else
          px.copy_masked(small16_x(s), kx, 2 * K, u - 2, wave_off);
      } else {
        if (u < 2)
          pw.copy_one(small16_w(s), (uint32_t)kw, u, wave_off);
        else
          px.copy_one(small16_x(s), (uint32_t)kx, u - 2, wave_off);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Epilogue of a W8A16 small tile: the wave's 128 x 32 block, bf16(acc *
// alpha) (binary16 with kF16), staged in the wave's 8 KiB area (row m at
// m * 64, 16-byte chunk c at c ^ (m % 4)), then 8 stores of 16 rows x 64
// bytes.
template <bool kF16>
__device__ __forceinline__ void small16_epilogue(const f32x4 (&acc)[2][8], uint8_t* area, float alpha,
                                                 __amdgpu_buffer_rsrc_t out, int col0, int gn, int gld, int lane) {
  asm volatile("" : "+v"(lane));
  const int q = lane >> 4, r = lane & 15;
#pragma unroll
  for (int b = 0; b < 8; ++b)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int m = 16 * b + r, c = 2 * i + (q >> 1);
      const f32x4 x = acc[i][b];
      u32x2 v;
      v[0] = h16x2<kF16>(x[0] * alpha, x[1] * alpha);
      v[1] = h16x2<kF16>(x[2] * alpha, x[3] * alpha);
      *reinterpret_cast<u32x2*>(area + m * 64 + ((c ^ (m & 3)) * 16) + (q & 1) * 8) = v;
    }
  const int c = lane & 3, col = col0 + 8 * c;
  u32x4 v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int row = 16 * k + (lane >> 2);
    v[k] = *reinterpret_cast<const u32x4*>(area + row * 64 + ((c ^ (row & 3)) * 16));
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int row = 16 * k + (lane >> 2);
    const uint32_t off = col < gn ? (uint32_t)(row * gld + col) * 2u : kOutOfRange;
    __builtin_amdgcn_raw_buffer_store_b128(v[k], out, (int)off, 0, kStreamStore);
  }
}

// Persistent W8A16 small-tile kernel (bf16 or binary16 activations and
// output) over 128 x 128 tiles of all groups.
template <int kForm>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1))) void
gemm_w8a16_small_kernel(const GemmArgs a) {
  static_assert(kForm != kFormF32, "16-bit activations");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = a.k;
  const int KT = (K + 63) / 64;
  const uint32_t wave_off = (uint32_t)wave * 64 * 16;
  W16Addr ad;
  ad.init(wave * 32 + (lane & 15), lane & 15, lane >> 4);
  uint8_t* area = lds_mem + kSmallEpiOffset + wave * kSmallEpiWave;

  for (int slot = blockIdx.x; slot < a.total_tiles; slot += (int)gridDim.x) {
    const TileCoord tc = tile_at<kSmallTile, kSmallTile>(a, slot);
    const GemmGroup& grp = a.g[tc.group];
    CopyPlan<4> pw;
    CopyPlan<8> px;
    {
      const uint8_t* w = grp.w + (int64_t)tc.n0 * K;
      const uint8_t* x = static_cast<const uint8_t*>(a.x) + (int64_t)tc.m0 * K * 2;
      pw.init2(w, grp.n - tc.n0, w, 0, K, tid);
      px.init2(x, a.m - tc.m0, x, 0, (int64_t)K * 2, tid);
    }
#pragma unroll
    for (int st = 0; st < kSmallBufs; ++st) {
#pragma unroll
      for (int u = 0; u < 2; ++u) pw.copy_masked(small16_w(st), st * 64, K, u, wave_off);
#pragma unroll
      for (int u = 0; u < 4; ++u) px.copy_masked(small16_x(st), st * 128, 2 * K, u, wave_off);
    }
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((kSmallBufs - 1) * kSmall16Copies) : "memory");
    Small16Frags fa, fb;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int j = 0; j < 2; ++j) fa.w[hh][j] = *reinterpret_cast<const u32x2*>(small16_w(0) + ad.w[hh] + j * 1024);
#pragma unroll
      for (int j = 0; j < 8; ++j) fa.x[hh][j] = lds_chunk(small16_x(0), ad.x[hh] + j * 2048);
    }
    f32x4 acc[2][8];
    small16_stage<kForm, true, true>(acc, fa, fb, 0, pw, px, K, ad, wave_off);
    // stage s copies stage s + kSmallBufs, wholly inside K while that is
    // below K / 64
    const int full_end = K / 64 - kSmallBufs;
    int s = 1;
    for (; s + 1 < KT && s + 1 < full_end; s += 2) {
      small16_stage<kForm, false, false>(acc, fb, fa, s, pw, px, K, ad, wave_off);
      small16_stage<kForm, false, false>(acc, fa, fb, s + 1, pw, px, K, ad, wave_off);
    }
    for (; s + 1 < KT; s += 2) {
      small16_stage<kForm, false, true>(acc, fb, fa, s, pw, px, K, ad, wave_off);
      small16_stage<kForm, false, true>(acc, fa, fb, s + 1, pw, px, K, ad, wave_off);
    }
    if (s < KT) small16_stage<kForm, false, true>(acc, fb, fa, s, pw, px, K, ad, wave_off);

    const int gn = __builtin_amdgcn_readfirstlane(grp.n), gld = __builtin_amdgcn_readfirstlane(grp.ldy);
    const int rows = __builtin_amdgcn_readfirstlane(max(0, min(a.m - tc.m0, 128)));
    uint8_t* base = static_cast<uint8_t*>(grp.y) + (int64_t)min(tc.m0, a.m) * gld * 2;
    const __amdgpu_buffer_rsrc_t out = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, rows * gld * 2, 0x00020000);
    small16_epilogue<kForm == kFormF16>(acc, area, grp.alpha, out, tc.n0 + wave * 32, gn, gld, lane);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
}

// Compute units of the current device (256 on MI355X).
int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    n = 256;
  return n;
}

}  // namespace

// One workgroup per CU (160 KiB of LDS each), a multiple of the 8 XCDs, at
// most one per tile.
int persistent_grid(int tiles) {
  static const int cus = cu_count();
  int grid = cus - cus % kXcds;
  if (grid <= 0) grid = kXcds;
  return grid > tiles ? tiles : grid;
}

// The 128 x 128 plan of a (already planned for 256 x 256 tiles) when its
// 256 x 256 tiles would keep at most 60% of the compute units busy; false (a
// unchanged) otherwise. Measured on one MI355X at N = K = 4096: M = 2048
// (256 x 256 tiles for half the CUs) runs faster on small tiles (W8A8 1953
// against 1775 TFLOP/s, W8A16 1055 against 810), M = 3072 (three quarters)
// on the big ones (2480 against 2022, 1209 against 1080).
bool small_tiles_for(int64_t big_tiles) {
  static const int cus = cu_count();
  return 5 * big_tiles <= 3 * (int64_t)cus;
}

bool small_tiles(GemmArgs& a) {
  if (!small_tiles_for(a.total_tiles)) return false;
  a.tiles_m = (a.m + kSmallTile - 1) / kSmallTile;
  int32_t t = 0;
  for (int i = 0; i < a.ngroups; ++i) {
    a.g[i].tiles_n = (a.g[i].n + kSmallTile - 1) / kSmallTile;
    a.g[i].tile_begin = t;
    t += a.tiles_m * a.g[i].tiles_n;
  }
  a.total_tiles = t;
  return true;
}

hipError_t launch_gemm_w8a8(const GemmArgs& a, hipStream_t s) {
  GemmArgs b = a;
  if (small_tiles(b))
    hipLaunchKernelGGL(gemm_w8a8_small_kernel, dim3((unsigned)persistent_grid(b.total_tiles)), dim3(kThreads), 0, s,
                       b);
  else
    hipLaunchKernelGGL(gemm_w8a8_kernel<false>, dim3((unsigned)persistent_grid(a.total_tiles)), dim3(kThreads), 0,
                       s, a);
  return hipGetLastError();
}

int device_cu_count() { return cu_count(); }

// Scratch of the calls that allocate nothing (fp8lin_gemm_w8a8_splitk_noalloc:
// the float32 split-K partials). Every GPU the library runs on holds its own
// copy until the process ends. In host code `scratch` names a host-side
// stand-in, not a device address: kernels get the device address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device and kept.
static __device__ __attribute__((used)) __align__(256) uint8_t scratch[FP8LIN_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t device_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_gemm_w8a8_splitk(const GemmArgs& a, hipStream_t s) {
  static const int cus = cu_count();
  int grid = cus - cus % kXcds;
  if (grid <= 0) grid = kXcds;
  if (grid > a.total_tiles) grid = a.total_tiles;
  hipLaunchKernelGGL((gemm_w8a8_kernel<false, false, true>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

// y[m, n] = bf16(alpha * sum_s p[s][m][n]) over `splits` float32 partials of
// [m, n] each (s in order, so the result is deterministic); 8 columns per
// thread: two 16-byte loads per partial, one 16-byte store.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const f32x4* __restrict__ p, int splits,
                                                            uint16_t* __restrict__ y, int64_t m, int64_t n,
                                                            int64_t ldy, float alpha) {
  const int64_t groups_per_row = n / 8;
  const int64_t total = m * groups_per_row;
  const int64_t plane = m * n / 4;  // float4 per partial
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t row = i / groups_per_row;
    const int64_t c = (i - row * groups_per_row) * 8;
    const int64_t v = (row * n + c) / 4;
    f32x4 lo = p[v], hi = p[v + 1];
    for (int sp = 1; sp < splits; ++sp) {
      lo += p[sp * plane + v];
      hi += p[sp * plane + v + 1];
    }
    u32x4 o;
    o.x = bf16x2(lo[0] * alpha, lo[1] * alpha);
    o.y = bf16x2(lo[2] * alpha, lo[3] * alpha);
    o.z = bf16x2(hi[0] * alpha, hi[1] * alpha);
    o.w = bf16x2(hi[2] * alpha, hi[3] * alpha);
    *reinterpret_cast<u32x4*>(y + row * ldy + c) = o;
  }
}

hipError_t launch_splitk_reduce(const float* partials, int splits, void* y, int64_t m, int64_t n, int64_t ldy,
                                float alpha, hipStream_t s) {
  const int64_t total = m * (n / 8);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<const f32x4*>(partials), splits, static_cast<uint16_t*>(y), m, n, ldy, alpha);
  return hipGetLastError();
}

hipError_t launch_gemm_w8a8_norm_rope(const GemmArgs& a, hipStream_t s) {
  static const int cus = cu_count();
  int grid = cus - cus % kXcds;
  if (grid <= 0) grid = kXcds;
  if (grid > a.total_tiles) grid = a.total_tiles;
  hipLaunchKernelGGL((gemm_w8a8_kernel<false, true>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

void gate_up_plan(GemmArgs& a) {
  if (a.xk == 0) a.xk = a.k;
  a.tiles_m = (a.m + kTileM - 1) / kTileM;
  a.g[0].tiles_n = (a.g[0].n + kTileN / 2 - 1) / (kTileN / 2);
  a.g[0].tile_begin = 0;
  a.total_tiles = a.tiles_m * a.g[0].tiles_n;
}

hipError_t launch_gate_up_swiglu(const GemmArgs& a, bool w8a16, bool f16, hipStream_t s) {
  static const int cus = cu_count();
  int grid = cus - cus % kXcds;
  if (grid <= 0) grid = kXcds;
  if (grid > a.total_tiles) grid = a.total_tiles;
  const bool tail = a.k % 64 != 0;
  auto kernel = !w8a16 ? gemm_w8a8_kernel<true>
                : f16  ? (tail ? gemm_w8a16_kernel<true, kFormF16> : gemm_w8a16_kernel<true, kFormF16, false, false>)
                       : (tail ? gemm_w8a16_kernel<true, kFormBf16> : gemm_w8a16_kernel<true, kFormBf16, false, false>);
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_w8a16_splitk(const GemmArgs& a, hipStream_t s) {
  static const int cus = cu_count();
  int grid = cus - cus % kXcds;
  if (grid <= 0) grid = kXcds;
  if (grid > a.total_tiles) grid = a.total_tiles;
  auto kernel = a.ks % 64 != 0 ? gemm_w8a16_kernel<false, kFormBf16, true> : gemm_w8a16_kernel<false, kFormBf16, true, false>;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_w8a16(const GemmArgs& a, int form, hipStream_t s) {
  GemmArgs b = a;
  if (form != kW16F32 && small_tiles(b)) {
    auto kernel = form == kW16F16 ? gemm_w8a16_small_kernel<kFormF16> : gemm_w8a16_small_kernel<kFormBf16>;
    hipLaunchKernelGGL(kernel, dim3((unsigned)persistent_grid(b.total_tiles)), dim3(kThreads), 0, s, b);
    return hipGetLastError();
  }
  const bool tail = a.k % 64 != 0;
  auto kernel = form == kW16F16
                    ? (tail ? gemm_w8a16_kernel<false, kFormF16> : gemm_w8a16_kernel<false, kFormF16, false, false>)
                : form == kW16F32
                    ? (tail ? gemm_w8a16_kernel<false, kFormF32> : gemm_w8a16_kernel<false, kFormF32, false, false>)
                    : (tail ? gemm_w8a16_kernel<false, kFormBf16> : gemm_w8a16_kernel<false, kFormBf16, false, false>);
  hipLaunchKernelGGL(kernel, dim3((unsigned)persistent_grid(a.total_tiles)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace fp8lin
