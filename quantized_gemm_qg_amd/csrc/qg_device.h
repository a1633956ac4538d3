// Device-side helpers shared by the gfx950 kernels: vector types, the bf16
// MFMA wrapper, register-level unpacking of the packed integer layout (see
// qg_internal.h), direct global -> LDS copies, explicit memory-counter waits
// and the XCD-aware tile order.
#pragma once

#include <hip/hip_runtime.h>

#include "qg_internal.h"

namespace qg {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(8))) int32_t i32x8;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

typedef __attribute__((ext_vector_type(4))) int32_t i32x4;

// The scaled f8f6f4 MFMA with its operand vectors sized by format: the LLVM
// intrinsic is overloaded on them, and an e2m1 operand (32 codes per lane)
// needs 4 registers where the clang builtin always passes 8.
extern "C" __device__ f32x4 qg_mfma_scale_16x16x128_f8_f4(i32x8 a, i32x4 b, f32x4 c, int fmt_a, int fmt_b,
                                                          int opsel_a, int scale_a, int opsel_b, int scale_b)
    __asm("llvm.amdgcn.mfma.scale.f32.16x16x128.f8f6f4.v8i32.v4i32");

// acc += (e4m3 A, e8m0 scale sa) x (e2m1 B, e8m0 scale: byte SB of sb_word),
// one 16x16x128 step; the instruction's scale byte select picks SB
template <int SB>
__device__ __forceinline__ f32x4 mfma_e4m3_e2m1(i32x8 a, i32x4 b, f32x4 c, int sa, int sb_word) {
  return qg_mfma_scale_16x16x128_f8_f4(a, b, c, 0, 4, 0, sa, SB, sb_word);
}

typedef __attribute__((ext_vector_type(16))) float f32x16;

// acc (32 x 32) += A (32 x 16 bf16) x B (16 x 32 bf16)
__device__ __forceinline__ f32x16 mfma32_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 4-bit: slots (i, i+4) -> bf16 pair 1 + u/16, code at mantissa bits 3..6.
__device__ __forceinline__ u32x4 unpack4(uint32_t w) {
  u32x4 r;
  r.x = ((w << 3) & 0x00780078u) | 0x3F803F80u;
  r.y = ((w >> 1) & 0x00780078u) | 0x3F803F80u;
  r.z = ((w >> 5) & 0x00780078u) | 0x3F803F80u;
  r.w = ((w >> 9) & 0x00780078u) | 0x3F803F80u;
  return r;
}

// 3-bit codes in bits 0..2 of each nibble slot -> bf16 pair 1 + u/8.
__device__ __forceinline__ u32x4 unpack3(uint32_t w) {
  u32x4 r;
  r.x = ((w << 4) & 0x00700070u) | 0x3F803F80u;
  r.y = (w & 0x00700070u) | 0x3F803F80u;
  r.z = ((w >> 4) & 0x00700070u) | 0x3F803F80u;
  r.w = ((w >> 8) & 0x00700070u) | 0x3F803F80u;
  return r;
}

// The fourth MFMA of a 3-bit lane slice: bit b of each code sits in bit 3 of
// the nibble slot of dword b; gather them into bits 0..2.
__device__ __forceinline__ uint32_t gather3(uint32_t d0, uint32_t d1, uint32_t d2) {
  return ((d0 >> 3) & 0x11111111u) | ((d1 >> 2) & 0x22222222u) | ((d2 >> 1) & 0x44444444u);
}

// B operand of K32 step j (0..3) of a lane's packed slice of one 128-K block.
template <int BITS>
__device__ __forceinline__ u32x4 unpack_b(const u32x4 &w, int j) {
  if constexpr (BITS == 4) {
    return unpack4(w[j]);
  } else {
    return j < 3 ? unpack3(w[j]) : unpack3(gather3(w.x, w.y, w.z));
  }
}

// Same conversions with the mask and the bf16 magic held in registers (the
// mask uniform, the magic in a VGPR), so each pair is one shift plus one
// v_and_or_b32: VOP3 cannot encode two literal constants.
__device__ __forceinline__ u32x4 unpack4r(uint32_t w, uint32_t mask, uint32_t magic) {
  u32x4 r;
  r.x = ((w << 3) & mask) | magic;
  r.y = ((w >> 1) & mask) | magic;
  r.z = ((w >> 5) & mask) | magic;
  r.w = ((w >> 9) & mask) | magic;
  return r;
}
__device__ __forceinline__ u32x4 unpack3r(uint32_t w, uint32_t mask, uint32_t magic) {
  u32x4 r;
  r.x = ((w << 4) & mask) | magic;
  r.y = (w & mask) | magic;
  r.z = ((w >> 4) & mask) | magic;
  r.w = ((w >> 8) & mask) | magic;
  return r;
}
template <int BITS>
__device__ __forceinline__ u32x4 unpack_br(const u32x4 &w, int j, uint32_t mask, uint32_t magic) {
  if constexpr (BITS == 4) {
    return unpack4r(w[j], mask, magic);
  } else {
    return unpack3r(j < 3 ? w[j] : gather3(w.x, w.y, w.z), mask, magic);
  }
}

// Opaque register copies of constants (the compiler cannot fold them back
// into literals).
__device__ __forceinline__ uint32_t vgpr_const(uint32_t c) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
  return r;
}
__device__ __forceinline__ uint32_t sgpr_const(uint32_t c) {
  uint32_t r;
  asm volatile("s_mov_b32 %0, %1" : "=s"(r) : "i"(c));
  return r;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Direct global -> LDS copies: each lane's 16 or 4 bytes land at lds + lane *
// size.  Non-template device functions, so the host pass never analyzes the
// device-only builtin.
__device__ __forceinline__ void lds_dma16(const void *g, void *l) {
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
}
__device__ __forceinline__ void lds_dma4(const void *g, void *l) {
  __builtin_amdgcn_global_load_lds(g, l, 4, 0, 0);
}

// s_waitcnt with vmcnt <= n (n <= 63), expcnt and lgkmcnt unconstrained
#define QG_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
// Wait for this wave's LDS writes (and scalar loads) only: a bare s_barrier
// does not wait for them, so LDS stores that other waves read after one are
// waited for first.
#define QG_WAIT_LGKMCNT0() __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4))

constexpr int kXcds = 8;  // L2 domains; workgroup ids are dealt round-robin over them

// Workgroup id -> (m-tile, n-tile).  Each XCD gets a contiguous range of a
// raster that walks group_m m-tiles across all n-tiles, so the tiles running
// together on one XCD share activation rows and weight columns in its L2.
// Returns false for ids past the last tile (the grid is rounded up to a
// multiple of kXcds, and MoE grids cover the tile list's capacity).
__device__ __forceinline__ bool tile_of(int pid, int m_tiles, int n_tiles, int group_m, int *tm,
                                        int *tn) {
  const int total = m_tiles * n_tiles;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  // one-to-one only for pid / kXcds < per_xcd; larger grids (MoE launches
  // sized for the tile list's capacity) must not revisit tiles
  if (pid / kXcds >= per_xcd) return false;
  const int t = (pid % kXcds) * per_xcd + pid / kXcds;
  if (t >= total) return false;
  const int group = group_m * n_tiles;
  const int first_m = (t / group) * group_m;
  const int gm = min(group_m, m_tiles - first_m);
  const int r = t % group;
  *tm = first_m + r % gm;
  *tn = r / gm;
  return true;
}

// Exclusive prefix sum of v over the workgroup (blockDim.x a multiple of 64,
// at most 16 waves); *total gets the sum.  wave_tot: 16 ints of LDS.
__device__ __forceinline__ int block_scan_excl(int v, int *wave_tot, int *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wave_tot[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    const int t = wave_tot[w];
    base += w < wave ? t : 0;
    tot += t;
  }
  __syncthreads();  // wave_tot may be reused
  *total = tot;
  return base + x - v;
}

// Rows of one tiled-kernel tile.  Dense: rows m0 .. m0 + BM - 1 of X and Y.
// MoE: sorted positions pos0 .. pos0 + rows - 1 of one expert's segment; the
// X row of a position follows the x row mode (the token p / topk of pair
// p = sorted_ids[pos], the pair itself, or the position), the Y row the y row
// mode.  Rows past the tile's valid rows map to its last valid row, so their
// loads stay in bounds; their outputs are never stored.
struct TileRows {
  int base;  // m0 (dense) or pos0 (MoE)
  int rows;  // valid rows in the tile
  bool moe;

  __device__ __forceinline__ int64_t x(const GemmArgs &a, int r) const {
    const int pos = base + min(r, rows - 1);
    if (!moe || a.x_rows == QG_ROWS_SORTED) return pos;
    const int p = a.sorted_ids[pos];
    return a.x_rows == QG_ROWS_BY_TOKEN ? (int64_t)(p / a.topk) : (int64_t)p;
  }
  __device__ __forceinline__ int64_t y(const GemmArgs &a, int r) const {
    const int pos = base + r;
    if (!moe || a.y_rows == QG_ROWS_SORTED) return pos;
    return a.sorted_ids[pos];
  }
};

// Workgroup id -> (tile rows, n-tile, weight base) of a tiled kernel; false if
// the workgroup has no tile.  MoE tiles come from the tile list (see
// launch_moe_tiles); the raster runs over the list entries.
template <int BM>
__device__ __forceinline__ bool tiled_work(const GemmArgs &a, bool moe, int n_tiles_wg, TileRows *tr,
                                           int *tn, const uint8_t **wexp) {
  int tm;
  if (!moe) {
    if (!tile_of(blockIdx.x, (a.m + BM - 1) / BM, n_tiles_wg, a.group_m, &tm, tn)) return false;
    *tr = TileRows{tm * BM, min(BM, a.m - tm * BM), false};
    *wexp = a.wbase;
    return true;
  }
  const int count = a.tiles[0];
  if (!tile_of(blockIdx.x, count, n_tiles_wg, a.group_m, &tm, tn)) return false;
  const int e = a.tiles[2 + 2 * tm], pos0 = a.tiles[3 + 2 * tm];
  const int rows = min(BM, a.offsets[e + 1] - pos0);
  if (rows <= 0) return false;
  *tr = TileRows{pos0, rows, true};
  *wexp = a.wbase + (uint64_t)e * a.expert_stride;
  return true;
}

// Epilogue of the tiled kernels: a wave's (16 MI) x (16 NJ) accumulator tile
// (C layout: block (i, j), lane (q, r) holds rows 4q..4q+3 of column r) goes
// out through a wave-private LDS buffer, 16 rows at a time, so that every
// lane stores 16 contiguous bytes of one output row (the C layout alone
// would give 2- or 4-byte stores, 32 bytes per row per instruction).  The
// wave's output row indices are gathered into LDS first, all loads before
// the first store (MoE rows come from the sorted pair list, and a load after
// a store to y could not be hoisted above it).  Rows at or past tr.rows and
// columns at or past N are not stored.  `lds` must hold store_tile_lds_bytes
// and may overlap nothing another wave still reads.
template <int MI, int NJ>
constexpr int store_tile_lds_bytes() {
  return 16 * (16 * NJ * 4 + 16) + 16 * MI * 4;
}

// The store path of store_tile for any accumulator layout: write_slab(i, lds,
// pitch, f32) writes the wave's 16-row slab i ([16][16 NJ] of fp32 or bf16 at
// `pitch` bytes per row); the rows are then stored from LDS.  The element
// type is a template constant here (store_slabs below picks the instance
// once), so the per-element writes of the slabs carry no branch on it.
template <int MI, int NJ, bool F32, typename W>
__device__ __forceinline__ void store_slabs_el(const GemmArgs &a, const TileRows &tr, W &write_slab, int row0,
                                               int col0, uint8_t *lds) {
  constexpr int WN = 16 * NJ;  // columns of the wave tile
  const int lane = threadIdx.x & 63;
  constexpr bool f32 = F32;
  constexpr int el = f32 ? 4 : 2;
  constexpr int pitch = WN * el + 16;       // padded row pitch (bytes)
  constexpr int cpr = WN * el / 16;         // 16-byte chunks per row
  constexpr int rows_per_pass = 64 / cpr;
  const bool vec16 = ((a.ldy * el) & 15) == 0;  // y itself is 16-byte aligned
  int *yrow = (int *)(lds + 16 * (WN * 4 + 16));  // [16 MI] output rows of the wave
#pragma unroll
  for (int t = 0; t < (16 * MI + 63) / 64; ++t) {
    const int r = 64 * t + lane;
    if (r < 16 * MI) yrow[r] = row0 + r < tr.rows ? (int)tr.y(a, row0 + r) : -1;
  }
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    write_slab(i, lds, pitch, f32);
    // the wave's own LDS accesses complete in order; this keeps the compiler
    // from moving the reads above the writes
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    for (int pass = 0; pass < (16 + rows_per_pass - 1) / rows_per_pass; ++pass) {
      const int rr = pass * rows_per_pass + lane / cpr, c = lane % cpr;
      // lanes past the pass's rows idle (cpr need not divide 64; 16-column
      // bf16 tiles cover the block with 32 lanes)
      if (lane >= rows_per_pass * cpr || rr >= 16) continue;
      const u32x4 v = *(const u32x4 *)(lds + rr * pitch + 16 * c);
      const int yr = yrow[16 * i + rr];
      const int col = col0 + c * (16 / el);
      if (yr >= 0 && col < a.n) {
        uint8_t *dst = (uint8_t *)a.y + ((int64_t)yr * a.ldy + col) * el;
        if (col + 16 / el <= a.n) {
          if (vec16) {
            *(u32x4 *)dst = v;
          } else {  // rows only 4-byte aligned (ldy * elem size not a multiple of 16)
            uint32_t *d4 = (uint32_t *)dst;
            d4[0] = v.x; d4[1] = v.y; d4[2] = v.z; d4[3] = v.w;
          }
        } else {  // right edge of the matrix: the chunk's first (N - col) elements, byte by byte
          const int nb = (a.n - col) * el;
#pragma unroll
          for (int b = 0; b < 16; ++b) {
            const uint32_t dw = b < 4 ? v.x : b < 8 ? v.y : b < 12 ? v.z : v.w;
            if (b < nb) dst[b] = (uint8_t)(dw >> (8 * (b & 3)));
          }
        }
      }
    }
    asm volatile("" ::: "memory");  // next slab's writes stay below these reads
  }
}

template <int MI, int NJ, typename W>
__device__ __forceinline__ void store_slabs(const GemmArgs &a, const TileRows &tr, W &&write_slab,
                                            int row0, int col0, uint8_t *lds) {
  if (a.otype == QG_O_F32)
    store_slabs_el<MI, NJ, true>(a, tr, write_slab, row0, col0, lds);
  else
    store_slabs_el<MI, NJ, false>(a, tr, write_slab, row0, col0, lds);
}

// one fp32 / bf16 element of a slab in LDS
__device__ __forceinline__ void slab_put(uint8_t *lds, int pitch, bool f32, int row, int col, float v) {
  uint8_t *p = lds + row * pitch + col * (f32 ? 4 : 2);
  if (f32)
    *(float *)p = v;
  else
    *(__bf16 *)p = (__bf16)v;
}

// acc_at(i, j): the f32x4 of 16 x 16 block (i, j) in the 16x16 MFMA layout
// (lane: column lane % 16, rows 4 (lane / 16) + e)
template <int MI, int NJ, typename F>
__device__ __forceinline__ void store_tile(const GemmArgs &a, const TileRows &tr, F &&acc_at,
                                           int row0, int col0, uint8_t *lds) {
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4, r16 = lane & 15;
  store_slabs<MI, NJ>(
      a, tr,
      [&](int i, uint8_t *l, int pitch, bool f32) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const f32x4 v = acc_at(i, j);
#pragma unroll
          for (int e = 0; e < 4; ++e) slab_put(l, pitch, f32, 4 * q + e, 16 * j + r16, v[e]);
        }
      },
      row0, col0, lds);
}

}  // namespace qg
