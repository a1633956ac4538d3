// Large-M tiled kernel for MXFP4 weights x MXFP8 activations on gfx950.
//
// The announcement's "W8A8 / W4A8 / W4A4" section describes the W4A8-MXFP4
// path as MXFP4 weights dequantized at load time and multiplied on FP8 tensor
// cores.  On CDNA4 the matrix core takes e2m1 and e4m3 operands with their
// e8m0 block scales directly (v_mfma_scale_f32_16x16x128_f8f6f4), so nothing is
// dequantized: the kernel only moves bytes.
//
// Tiling: a workgroup computes a BM x 256 tile of Y with WM x WN waves, each
// (BM / WM) x (256 / WN) as blocks of 16 x 16.  The default is 8 waves (4 x 2,
// two per SIMD, wave tile 64 x 128, 128 fp32 accumulators per lane): while one
// wave of a SIMD waits on its LDS reads or the stage barrier, the other keeps
// the matrix core busy; LDS traffic stays at 256 B per MFMA (16 KB per wave
// and K step).  The 4-wave form (2 x 2, one wave per SIMD, wave tile
// (BM / 2) x 128) is kept for comparison.  Large workgroup tiles halve the
// L2 -> LDS bytes per flop.  K advances 128 per step through a 3-stage LDS ring filled directly
// from global memory by global_load_lds_dwordx4 (no register staging), so two
// K steps are in flight while a third is multiplied.  One stage holds
//   A   BM rows x 128 e4m3 bytes; each row's eight 16-byte chunks are stored
//       in XOR-swizzled order (chunk c at slot c ^ (row & 7)) so the 16 rows
//       of an MFMA fragment read hit all LDS banks without padding;
//   B   16 packed weight blocks of 1 KB copied verbatim (the packed layout
//       already stores each lane's 16-byte B operand contiguously);
//   SA  the four e8m0 scales of each activation row for this K step;
//   SW  for each of the 256 weight columns and quarters q, the dword holding
//       its e8m0 scales of K steps kb & ~3 .. +3.
// Every wave issues the same number of loads per stage, so "stage kb has
// landed" is a wait until at most one stage of the wave's loads is
// outstanding, followed by a workgroup barrier.  Inside a K step the next row
// block's LDS reads are scheduled ahead of the current block's 8 MFMAs.
//
// Work order: workgroups are dealt round-robin to the 8 XCDs; the tile index
// is remapped so each XCD owns a contiguous range of a grouped (GM m-tiles at
// a time) raster, so the tiles running together on one XCD share activation
// rows and weight columns in that XCD's L2.
#include <hip/hip_runtime.h>

#include "qg_device.h"
#include "qg_internal.h"

namespace qg {

constexpr int kTBN = 256;   // tile columns
constexpr int kStages = 3;

// BM x 256 tile, WM x WN waves, each wave (BM / WM) x (256 / WN)
template <int BM, int WM, int WN>
struct MxCfg {
  static constexpr int WAVES = WM * WN;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int A = BM * 128;
  static constexpr int B = (kTBN / 16) * 1024;   // 16 KB
  static constexpr int SA = BM * 4;
  static constexpr int SW = kTBN * 4 * 4;        // 4 KB
  static constexpr int STAGE = A + B + SA + SW;
  static constexpr int A_LOADS = BM * 128 / 1024 / WAVES;  // 1-KB copies of A per wave
  static constexpr int B_LOADS = 16 / WAVES;                // 1-KB blocks of B per wave
  static constexpr int SW_LOADS = 16 / WAVES;               // 256-B pieces of SW per wave
  static constexpr int LOADS = A_LOADS + B_LOADS + 1 + SW_LOADS;  // + one SA piece
  static constexpr int MB = BM / WM / 16;                   // 16-row blocks per wave
  static constexpr int NB = kTBN / WN / 16;                 // 16-column blocks per wave
  static_assert(A_LOADS >= 1 && B_LOADS >= 1 && SW_LOADS >= 1, "too many waves");
  static_assert(WAVES >= BM / 64 || BM / 64 % WAVES == 0, "SA pieces");
};

template <int BM, int WM, int WN, bool MOE>
__global__ __launch_bounds__(64 * WM * WN) void mx_tiled_kernel(GemmArgs a) {
  using C = MxCfg<BM, WM, WN>;
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int q = lane >> 4, r16 = lane & 15;

  TileRows tr;
  int tn;
  const uint8_t *wexp;
  if (!tiled_work<BM>(a, MOE, (a.n_tiles * 16 + kTBN - 1) / kTBN, &tr, &tn, &wexp)) return;
  const int nt0 = tn * (kTBN / 16);  // first 16-column n-tile
  const int kbs = a.k_blocks;
  const int kq = a.k >> 5;           // activation scale bytes per row
  const uint8_t *x = (const uint8_t *)a.x;
  const uint8_t *wsc = wexp + a.scales_offset;

  // per-lane source offsets (32-bit, added to wave-uniform bases at issue)
  uint32_t a_off[C::A_LOADS];
#pragma unroll
  for (int i = 0; i < C::A_LOADS; ++i) {
    const int row = 8 * (wave * C::A_LOADS + i) + (lane >> 3);
    const int c = (lane & 7) ^ (row & 7);
    a_off[i] = (uint32_t)(tr.x(a, row) * a.ldx + 16 * c);
  }
  const uint8_t *b_base = wexp + 16 * lane;
  uint32_t b_blk[C::B_LOADS];  // first packed block of each of the wave's n-tiles
#pragma unroll
  for (int i = 0; i < C::B_LOADS; ++i)
    b_blk[i] = (uint32_t)min(nt0 + wave * C::B_LOADS + i, a.n_tiles - 1) * kbs;
  // SA: BM rows of 4 bytes = BM / 64 pieces of 256 B; waves past them repeat
  // earlier pieces (same bytes to the same place)
  const int sa_piece = wave % (BM / 64);
  const uint8_t *sa_src = a.x_scales + tr.x(a, sa_piece * 64 + lane) * kq;
  uint32_t sw_off[C::SW_LOADS];
#pragma unroll
  for (int i = 0; i < C::SW_LOADS; ++i) {
    const int e = (wave * C::SW_LOADS + i) * 64 + lane;  // (column, quarter) pair
    const int n = min(nt0 * 16 + (e >> 2), a.n_tiles * 16 - 1);
    sw_off[i] = (uint32_t)(((uint64_t)n * 4 + (e & 3)) * a.kb_pad);
  }

  auto issue = [&](int kb, int buf) {
    uint8_t *st = smem + buf * C::STAGE;
    const uint8_t *xk = x + kb * 128;
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i)
      lds_dma16(xk + a_off[i], st + (wave * C::A_LOADS + i) * 1024);
#pragma unroll
    for (int i = 0; i < C::B_LOADS; ++i)
      lds_dma16(b_base + ((uint64_t)(b_blk[i] + kb) << 10), st + C::A + (wave * C::B_LOADS + i) * 1024);
    lds_dma4(sa_src + 4 * kb, st + C::A + C::B + sa_piece * 256);
    const uint8_t *wk = wsc + (kb & ~3);
#pragma unroll
    for (int i = 0; i < C::SW_LOADS; ++i)
      lds_dma4(wk + sw_off[i], st + C::A + C::B + C::SA + (wave * C::SW_LOADS + i) * 256);
  };

  f32x4 acc[C::MB][C::NB];
#pragma unroll
  for (int i = 0; i < C::MB; ++i)
#pragma unroll
    for (int j = 0; j < C::NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  issue(0, 0);
  if (kbs > 1) issue(1, 1);
  for (int kb = 0; kb < kbs; ++kb) {
    if (kb + 1 < kbs) {
      QG_WAIT_VMCNT(C::LOADS);
    } else {
      QG_WAIT_VMCNT(0);
    }
    __builtin_amdgcn_s_barrier();  // stage kb is in LDS; stage kb - 1 is free
    if (kb + 2 < kbs) issue(kb + 2, (kb + 2) % kStages);
    const uint8_t *st = smem + (kb % kStages) * C::STAGE;
    i32x8 bf[C::NB];
    int bsc[C::NB];
#pragma unroll
    for (int j = 0; j < C::NB; ++j) {
      const int blk = wn * C::NB + j;
      const u32x4 v = *(const u32x4 *)(st + C::A + blk * 1024 + 16 * lane);
      bf[j] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      const uint32_t sw = *(const uint32_t *)(st + C::A + C::B + C::SA + ((blk * 16 + r16) * 4 + q) * 4);
      bsc[j] = (int)((sw >> (8 * (kb & 3))) & 0xFFu);
    }
    auto read_a = [&](int i, i32x8 &af, int &asc) {
      const int row = wm * (BM / WM) + i * 16 + r16;
      const uint8_t *ap = st + row * 128;
      const u32x4 lo = *(const u32x4 *)(ap + 16 * (q ^ (row & 7)));
      const u32x4 hi = *(const u32x4 *)(ap + 16 * ((4 + q) ^ (row & 7)));
      af = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                 (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      asc = st[C::A + C::B + 4 * row + q];
    };
    i32x8 af[2];
    int asc[2];
    read_a(0, af[0], asc[0]);
    // B (2 NB reads) and A block 0 (3 reads) first
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * C::NB + 3, 0);
#pragma unroll
    for (int i = 0; i < C::MB; ++i) {
      if (i + 1 < C::MB) read_a(i + 1, af[(i + 1) & 1], asc[(i + 1) & 1]);
#pragma unroll
      for (int j = 0; j < C::NB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i & 1], bf[j], acc[i][j], 0, 4,
                                                                      0, asc[i & 1], 0, bsc[j]);
      if (i + 1 < C::MB) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // next block's reads
      __builtin_amdgcn_sched_group_barrier(0x008, C::NB, 0);                // this block's MFMAs
    }
  }

  // output through LDS (the ring is free once every wave is past its last stage)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  store_tile<C::MB, C::NB>(a, tr, [&](int i, int j) { return acc[i][j]; }, wm * (BM / WM),
                           (nt0 + wn * C::NB) * 16, smem + wave * store_tile_lds_bytes<C::MB, C::NB>());
}

template <int BM, int WM, int WN, bool MOE>
static hipError_t launch_mx_tiled_bm(const GemmArgs &a, int64_t tiles_cap, hipStream_t s) {
  using C = MxCfg<BM, WM, WN>;
  static_assert(kStages * C::STAGE >= C::WAVES * store_tile_lds_bytes<C::MB, C::NB>(), "epilogue LDS");
  const int64_t m_tiles = MOE ? tiles_cap : (a.m + BM - 1) / BM;
  const int64_t n_tiles_wg = (a.n_tiles * 16 + kTBN - 1) / kTBN;
  const int64_t total = m_tiles * n_tiles_wg;
  const int64_t per_xcd = (total + kXcds - 1) / kXcds;
  const size_t lds = (size_t)kStages * C::STAGE;
  hipError_t e = hipFuncSetAttribute((const void *)mx_tiled_kernel<BM, WM, WN, MOE>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((mx_tiled_kernel<BM, WM, WN, MOE>), dim3((unsigned)(per_xcd * kXcds)),
                     dim3(C::THREADS), lds, s, a);
  return hipGetLastError();
}

// Dense: bm-row tiles (128 or 256), tiles bm x 256.  MoE: the tile list a.tiles
// (capacity tiles_cap) of kMoeTileRows-row tiles.  waves: 4 (2 x 2, one per
// SIMD) or 8 (4 x 2, two per SIMD).
hipError_t launch_mx_tiled(const GemmArgs &a, int bm, bool moe, int64_t tiles_cap, int waves,
                           hipStream_t s) {
  if (a.k % 128 != 0) return hipErrorInvalidValue;
  if (waves == 8) {
    if (moe) return launch_mx_tiled_bm<kMoeTileRows, 4, 2, true>(a, tiles_cap, s);
    return bm == 256 ? launch_mx_tiled_bm<256, 4, 2, false>(a, 0, s)
                     : launch_mx_tiled_bm<128, 4, 2, false>(a, 0, s);
  }
  if (moe) return launch_mx_tiled_bm<kMoeTileRows, 2, 2, true>(a, tiles_cap, s);
  return bm == 256 ? launch_mx_tiled_bm<256, 2, 2, false>(a, 0, s)
                   : launch_mx_tiled_bm<128, 2, 2, false>(a, 0, s);
}

}  // namespace qg
