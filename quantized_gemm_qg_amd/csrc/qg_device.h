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

constexpr int kXcds = 8;    // L2 domains; workgroup ids are dealt round-robin over them
constexpr int kGroupM = 4;  // m-tiles per raster group

// Workgroup id -> (m-tile, n-tile).  Each XCD gets a contiguous range of a
// raster that walks kGroupM m-tiles across all n-tiles, so the tiles running
// together on one XCD share activation rows and weight columns in its L2.
// Returns false for ids past the last tile (the grid is rounded up to a
// multiple of kXcds).
__device__ __forceinline__ bool tile_of(int pid, int m_tiles, int n_tiles, int *tm, int *tn) {
  const int total = m_tiles * n_tiles;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int t = (pid % kXcds) * per_xcd + pid / kXcds;
  if (t >= total) return false;
  const int group = kGroupM * n_tiles;
  const int first_m = (t / group) * kGroupM;
  const int gm = min(kGroupM, m_tiles - first_m);
  const int r = t % group;
  *tm = first_m + r % gm;
  *tn = r / gm;
  return true;
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
    if (!tile_of(blockIdx.x, (a.m + BM - 1) / BM, n_tiles_wg, &tm, tn)) return false;
    *tr = TileRows{tm * BM, min(BM, a.m - tm * BM), false};
    *wexp = a.wbase;
    return true;
  }
  const int count = a.tiles[0];
  if (!tile_of(blockIdx.x, count, n_tiles_wg, &tm, tn)) return false;
  const int e = a.tiles[2 + 2 * tm], pos0 = a.tiles[3 + 2 * tm];
  const int rows = min(BM, a.offsets[e + 1] - pos0);
  if (rows <= 0) return false;
  *tr = TileRows{pos0, rows, true};
  *wexp = a.wbase + (uint64_t)e * a.expert_stride;
  return true;
}

}  // namespace qg
