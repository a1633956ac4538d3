// Large-M tiled kernel for the integer weight formats (INT4 / UINT4 / INT3 /
// UINT3 codes, bf16 group scales along K, optional 4-bit zero points) with
// bf16 activations, on gfx950's v_mfma_f32_16x16x32_bf16.
//
// The announcement's "Shared CUDA components" section puts dequantization and
// scaling inside the GEMM's data path, between the operand loads and the
// matrix-core step.  Here the packed codes travel HBM -> LDS untouched (a
// quarter of the bytes of a bf16 weight); each wave turns its columns' codes
// into bf16 MFMA operands in registers, once per 128-K step, and reuses them
// for all BM / WM rows of its tile.
//
// Arithmetic.  An offset-binary code u becomes the bf16 value 1 + u / MAG
// (MAG = 16 for 4-bit, 8 for 3-bit codes: the code lands in the top mantissa
// bits).  Per K-group the wave computes on the matrix core
//     G = sum_k x_k * (1 + u_k / MAG) - (1 + z / MAG) * xs,   xs = sum_k x_k
// by starting the MFMA accumulation from the second term, so G = sum x (u - z)
// / MAG exactly up to fp32 rounding, and then adds G * (MAG * s) to the output
// accumulator: one fp32 FMA per accumulator per group.  For symmetric formats
// z = 2^(b-1) is a constant and the starting value depends on the row only.
// xs (the group row sums of X, for symmetric formats already multiplied by
// -(1 + z / MAG)) comes from a small pre-pass kernel that reads X once; the
// dequantized weight is the exact real (u - z) * s.
//
// Tiling: a workgroup of WM x 2 waves computes a BM x 128 tile of Y, each wave
// (BM / WM) x 64 as (BM / WM / 16) x 4 blocks of 16 x 16; the default is 8
// waves (WM = 4, two per SIMD, so one wave's waits hide behind the other's
// work), the 4-wave form (WM = 2) is kept for comparison.  K advances 128 per
// stage; one step uses
//   A   BM rows x 128 bf16 (256 B per row, 16-byte chunks XOR-swizzled by
//       the row's low 4 bits so the 16 rows of a fragment read hit distinct
//       banks),
//   SX  the group row sums of the tile's rows for this step's groups,
//   B   the 8 packed 16 x 128 blocks of the tile's columns, copied verbatim,
//   SS  per column the 16-byte run of bf16 scales holding this step's groups,
//   SZ  per column the dword of zero-point nibbles (formats with zero points).
// A and SX fill one ring, B, SS and SZ another, both straight from global
// memory with global_load_lds (no register staging).  The activation ring is
// 2 (BM = 256) or 3 (BM = 128) stages deep; the weight ring, whose bytes come
// from HBM with little reuse when every expert has its own weights, runs as
// deep as LDS allows (up to 5 stages ahead).  Every wave issues the same number
// of loads per stage, so "stage kb has landed" is an explicit vmcnt wait plus
// a workgroup barrier.  The workgroup order is the
// XCD-aware raster of the MX tiled kernel.
#include <hip/hip_runtime.h>

#include "qg_device.h"
#include "qg_internal.h"

namespace qg {

constexpr int kLdsBytes = 160 * 1024;

template <int BM, int BN, int WM, int WN, int BITS, bool ZP, int GROUP>
struct A16Cfg {
  static constexpr int WAVES = WM * WN;           // WM (M) x WN (N)
  static constexpr int NBLK = BN / 16;            // packed n-tiles per tile
  static constexpr int NJ = NBLK / WN;            // 16-column blocks per wave
  static constexpr int LB = BITS == 4 ? 16 : 12;  // packed bytes per lane per block
  static constexpr int BB = 64 * LB;              // packed bytes per 16 x 128 block
  static constexpr int GPB = 128 / GROUP;         // groups per 128-K step
  static constexpr int JPG = GROUP / 32;          // K32 MFMA steps per group
  // activation ring stage: A tile, then the group row sums (rows padded to 64:
  // one 64-lane copy per group)
  static constexpr int SXR = BM < 64 ? 64 : BM;
  static constexpr int A = BM * 256;
  static constexpr int SX = GPB * SXR * 4;
  static constexpr int A_STAGE = A + SX;
  // weight ring stage: packed blocks, scales, zero points
  static constexpr int B = NBLK * BB;
  static constexpr int SS = BN * 16;
  static constexpr int SZ = ZP ? BN * 4 : 0;
  static constexpr int SS_PIECES = BN / 64;       // 64-column copies of SS / SZ
  static constexpr int OFF_SS = B;
  static constexpr int OFF_SZ = OFF_SS + SS;
  static constexpr int B_STAGE = OFF_SZ + SZ;
  // ring depths: the weights come from HBM with little reuse across
  // workgroups (MoE experts), so their ring runs as deep as LDS allows.  Small
  // tiles (WM = 1) keep to half of LDS so that two workgroups share a CU: one
  // fills its rings while the other computes (short-K layers spend much of a
  // tile in the prologue).
  static constexpr int LDS_CAP = WM == 1 ? kLdsBytes / 2 : kLdsBytes;
  // (256-column tiles: three weight stages at least when both rings fit)
  static constexpr int NA = WM == 1 ? 2 : (3 * A_STAGE + (BN > 128 ? 3 : 2) * B_STAGE <= LDS_CAP ? 3 : 2);
  static constexpr int NB_FIT = (LDS_CAP - NA * A_STAGE) / B_STAGE;
  static constexpr int NB = NB_FIT > 6 ? 6 : NB_FIT;
  static constexpr int OFF_BRING = NA * A_STAGE;
  static constexpr int LDS = NA * A_STAGE + NB * B_STAGE;
  // loads per wave and stage
  static constexpr int A_LOADS = BM * 256 / 1024 / WAVES;            // 1-KB copies of A
  static constexpr int B_LOADS = (BITS == 4 ? NBLK : 3 * NBLK) / WAVES;  // 1-KB (4-bit) or 256-B (3-bit) copies
  // the group row sums (SX) are copied by the first SXR / 64 waves, the
  // scales and zero points (SS, SZ) by the first SS_PIECES: per-wave counts
  static constexpr int SX_WAVES = SXR / 64;
  static constexpr int A_ISSUE = A_LOADS + GPB;             // an SX wave
  static constexpr int B_ISSUE = B_LOADS + 1 + (ZP ? 1 : 0);  // an SS wave
  // Each step issues its activation loads, then its weight loads.  In steady
  // state, the loads issued after the later of stage kb's two groups: stage
  // kb's weights went out in an earlier step than its activations when the
  // weight ring is deeper (followed by that step's weight loads), in the same
  // step otherwise.
  static constexpr int after(int ai, int bi) { return (NB > NA ? bi : 0) + (NA - 2) * (ai + bi); }
  static constexpr int AFTER_A = after(A_ISSUE, B_ISSUE);   // the largest
  static constexpr int MI = BM / WM / 16;             // 16-row blocks per wave
  // wave tiles that are multiples of 32 x 32 run v_mfma_f32_32x32x16_bf16
  // (measured on gfx950: 2.18 PFLOP/s sustained from registers, against
  // 1.43 for 16x16x32); the small tiles (16-column waves) keep 16x16x32
  static constexpr bool M32 = WM > 1 && (BM / WM) % 32 == 0 && (BN / WN) % 32 == 0;
  static constexpr int MB2 = BM / WM / 32;            // 32-row blocks per wave (M32)
  static constexpr int NB2 = BN / WN / 32;            // 32-column blocks per wave (M32)
  static constexpr int MPG = GROUP / 16;              // K16 MFMA steps per group (M32)
  // small tiles (one wave per 16 columns, every wave all BM rows) are for
  // MoE experts with few rows: row blocks past the tile's rows are skipped
  static constexpr bool SKIP_ROWS = WM == 1;
  static constexpr float MAG = BITS == 4 ? 16.f : 8.f;
  static constexpr int ZSYM = BITS == 4 ? 8 : 4;
  static_assert(NB >= 2 && NB >= NA, "weight ring too shallow");
  static_assert(LDS <= LDS_CAP, "rings exceed LDS");
  static_assert(AFTER_A <= 63, "vmcnt range");
  static_assert(SX_WAVES <= WAVES && SS_PIECES <= WAVES, "copy pieces");
};

// Wait of step kb for a wave that issues AI activation and BI weight copies
// per stage: once at most after(AI, BI) loads are outstanding, both groups of
// stage kb have landed (memory counters retire in issue order).  Near the end
// fewer loads follow, so the wait is tightened, never loosened; in the
// prologue more loads follow, so it is conservative.
template <typename C, int AI, int BI>
__device__ __forceinline__ void a16_stage_wait(int kb, int kbs) {
  constexpr int AFTER = C::after(AI, BI);
  if (kb + C::NB - 2 < kbs) {
    QG_WAIT_VMCNT(AFTER);
  } else if (C::NA == 3 && kb + 1 < kbs) {
    QG_WAIT_VMCNT(AI);
  } else {
    QG_WAIT_VMCNT(0);
  }
}

// Workgroup barrier that the compiler may not move LDS accesses across; the
// memory-counter waits are explicit (QG_WAIT_VMCNT) so that loads of later
// stages stay in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// FP4: MXFP4 weights x bf16 activations (e2m1 codes in standard nibble order,
// group 32, bf16 power-of-two scales): each B operand is the exact bf16
// e2m1 x scale from the fp4 conversion, so the MFMAs accumulate straight into
// the output accumulators (no group row sums, no per-group FMA).
template <int BM, int BN, int WM, int WN, int BITS, bool ZP, int GROUP, bool MOE, bool FP4 = false>
__global__ __launch_bounds__(64 * WM * WN) void a16_tiled_kernel(GemmArgs a, const float *xs,
                                                                 int xs_rows) {
  using C = A16Cfg<BM, BN, WM, WN, BITS, ZP, GROUP>;
  static_assert(!FP4 || (BITS == 4 && !ZP && GROUP == 32), "fp4 codes: 4-bit, group 32");
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int q = lane >> 4, r16 = lane & 15;

  TileRows tr;
  int tn;
  const uint8_t *wexp;
  if (!tiled_work<BM>(a, MOE, (a.n_tiles + C::NBLK - 1) / C::NBLK, &tr, &tn, &wexp)) return;
  const int nt0 = tn * C::NBLK;
  const int kbs = a.k_blocks, gp = a.groups_padded;
  const uint32_t umask = sgpr_const(BITS == 4 ? 0x00780078u : 0x00700070u);
  const uint32_t umagic = vgpr_const(0x3F803F80u);

  // ---- per-lane source offsets (32-bit, added to uniform bases at issue) ----
  // A: copy i of this wave fills tile rows 4 (wave * A_LOADS + i) + lane / 16,
  // LDS slot lane % 16, with the row's chunk (slot ^ (row & 15))
  const uint8_t *x = (const uint8_t *)a.x;
  uint32_t a_off[C::A_LOADS];
#pragma unroll
  for (int i = 0; i < C::A_LOADS; ++i) {
    const int row = 4 * (wave * C::A_LOADS + i) + (lane >> 4);
    const int c = (lane & 15) ^ (row & 15);
    a_off[i] = (uint32_t)(tr.x(a, row) * a.ldx * 2 + 16 * c);
  }
  // B: 4-bit, copy i = block B_LOADS wave + i; 3-bit, copy i = 256-byte
  // piece B_LOADS wave + i of the NBLK blocks (three pieces per 768-byte block)
  uint32_t b_off[C::B_LOADS];
#pragma unroll
  for (int i = 0; i < C::B_LOADS; ++i) {
    if constexpr (BITS == 4) {
      const int blk = C::B_LOADS * wave + i;
      b_off[i] = (uint32_t)(min(nt0 + blk, a.n_tiles - 1) * kbs) * 1024u + 16u * lane;
    } else {
      const int piece = C::B_LOADS * wave + i, blk = piece / 3;
      b_off[i] = (uint32_t)(min(nt0 + blk, a.n_tiles - 1) * kbs) * 768u + 256u * (piece % 3) + 4u * lane;
    }
  }
  // SS / SZ: wave w < SS_PIECES copies columns 64 w .. 64 w + 63 of the tile
  const int ncol = min(nt0 * 16 + 64 * (wave % C::SS_PIECES) + lane, a.n_tiles * 16 - 1);
  const uint8_t *ss_src = wexp + a.scales_offset + (uint64_t)ncol * gp * 2;
  const uint32_t *sz_src = (const uint32_t *)(wexp + a.zeros_offset) + (uint64_t)ncol * (gp >> 3);
  const bool sx_wave = !FP4 && wave < C::SX_WAVES, ss_wave = wave < C::SS_PIECES;  // FP4: no row sums
  const int sx_row = 64 * (sx_wave ? wave : 0) + lane;
  const float *sx_src = FP4 ? xs : xs + tr.x(a, sx_row);

  auto issue_a = [&](int kb) {
    uint8_t *st = smem + (kb % C::NA) * C::A_STAGE;
    const uint8_t *xk = x + kb * 256;
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i)
      lds_dma16(xk + a_off[i], st + (wave * C::A_LOADS + i) * 1024);
    if (sx_wave) {
#pragma unroll
      for (int gi = 0; gi < C::GPB; ++gi)
        lds_dma4(sx_src + (int64_t)(kb * C::GPB + gi) * xs_rows, st + C::A + (gi * C::SXR + 64 * wave) * 4);
    }
  };
  auto issue_b = [&](int kb) {
    uint8_t *st = smem + C::OFF_BRING + (kb % C::NB) * C::B_STAGE;
#pragma unroll
    for (int i = 0; i < C::B_LOADS; ++i) {
      if constexpr (BITS == 4)
        lds_dma16(wexp + b_off[i] + kb * 1024u, st + (C::B_LOADS * wave + i) * 1024);
      else
        lds_dma4(wexp + b_off[i] + kb * 768u, st + (C::B_LOADS * wave + i) * 256);
    }
    if (ss_wave) {
      const int g0 = kb * C::GPB;
      lds_dma16(ss_src + (g0 & ~7) * 2, st + C::OFF_SS + wave * 1024);
      if constexpr (ZP) lds_dma4(sz_src + (g0 >> 3), st + C::OFF_SZ + wave * 256);
    }
  };

  f32x4 acc[C::M32 ? 1 : C::MI][C::M32 ? 1 : C::NJ];
  f32x16 acc32[C::M32 ? C::MB2 : 1][C::M32 ? C::NB2 : 1];
  if constexpr (C::M32) {
#pragma unroll
    for (int i = 0; i < C::MB2; ++i)
#pragma unroll
      for (int j = 0; j < C::NB2; ++j) acc32[i][j] = f32x16{};
  } else {
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // prologue: activations NA - 1 stages ahead, weights NB - 1 stages ahead
  for (int s = 0; s < C::NB - 1; ++s) {
    if (s < C::NA - 1 && s < kbs) issue_a(s);
    if (s < kbs) issue_b(s);
  }
  for (int kb = 0; kb < kbs; ++kb) {
    if (sx_wave) {
      if (ss_wave) a16_stage_wait<C, C::A_ISSUE, C::B_ISSUE>(kb, kbs);
      else a16_stage_wait<C, C::A_ISSUE, C::B_LOADS>(kb, kbs);
    } else {
      if (ss_wave) a16_stage_wait<C, C::A_LOADS, C::B_ISSUE>(kb, kbs);
      else a16_stage_wait<C, C::A_LOADS, C::B_LOADS>(kb, kbs);
    }
    lds_barrier();  // stage kb is in LDS; the buffers of stage kb - 1 are free
    if (kb + C::NA - 1 < kbs) issue_a(kb + C::NA - 1);
    if (kb + C::NB - 1 < kbs) issue_b(kb + C::NB - 1);
    const uint8_t *st = smem + (kb % C::NA) * C::A_STAGE;
    const uint8_t *sb = smem + C::OFF_BRING + (kb % C::NB) * C::B_STAGE;

    if constexpr (C::M32) {
      // 32 x 32 blocks.  Lane l works on column / row l % 32 of a block and
      // K16 half h = l / 32.  The B operand of K16 step m (k = 16 m + 8 h +
      // 0..7 of the stage) is dword m / 2 of the packed lane slot with quarter
      // 2 (m % 2) + h, i.e. slots (l % 16) + 16 h and that + 32 of the
      // block's n-tile; A is 16-byte chunk 2 m + h of the row.  Accumulator
      // element 4 ii + e holds row 8 ii + 4 h + e.
      const int h = lane >> 5, c32 = lane & 31;
      u32x4 bw[C::NB2][8];
#pragma unroll
      for (int j = 0; j < C::NB2; ++j) {
        const int blk = 2 * (wn * C::NB2 + j) + (c32 >> 4);
        const int slot = (c32 & 15) + 16 * h;
        u32x4 v[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          if constexpr (BITS == 4) {
            v[hh] = *(const u32x4 *)(sb + blk * 1024 + 16 * (slot + 32 * hh));
          } else {
            const uint32_t *p = (const uint32_t *)(sb + blk * 768 + 12 * (slot + 32 * hh));
            v[hh] = u32x4{p[0], p[1], p[2], 0u};
          }
        }
        if constexpr (FP4) {
          // dword jj of both slots holds K-group kb * GPB + jj of column col
          const int col = wn * 32 * C::NB2 + 32 * j + c32;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int gg = kb * C::GPB + jj;
            const float sc = bf16_bits_to_f32(*(const uint16_t *)(sb + C::OFF_SS + col * 16 + 2 * (gg & 7)));
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const uint32_t wd = v[hh][jj];
              bw[j][2 * jj + hh] =
                  u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc, 0)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc, 1)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc, 2)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc, 3))};
            }
          }
        } else {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            bw[j][2 * jj] = unpack_br<BITS>(v[0], jj, umask, umagic);
            bw[j][2 * jj + 1] = unpack_br<BITS>(v[1], jj, umask, umagic);
          }
        }
      }
      if constexpr (FP4) {
#pragma unroll
        for (int i = 0; i < C::MB2; ++i) {
          const int r0 = wm * (BM / WM) + 32 * i;
          const uint8_t *arow = st + (r0 + c32) * 256;
#pragma unroll
          for (int mm = 0; mm < 8; ++mm) {
            const u32x4 af = *(const u32x4 *)(arow + 16 * ((2 * mm + h) ^ (c32 & 15)));
#pragma unroll
            for (int j = 0; j < C::NB2; ++j) acc32[i][j] = mfma32_bf16(af, bw[j][mm], acc32[i][j]);
          }
        }
        continue;
      }
#pragma unroll
      for (int gi = 0; gi < C::GPB; ++gi) {
        const int gg = kb * C::GPB + gi;
        float c1[C::NB2], zf[C::NB2];
#pragma unroll
        for (int j = 0; j < C::NB2; ++j) {
          const int col = wn * 32 * C::NB2 + 32 * j + c32;
          const uint32_t sbits = *(const uint16_t *)(sb + C::OFF_SS + col * 16 + 2 * (gg & 7));
          c1[j] = C::MAG * bf16_bits_to_f32(sbits);
          int z = C::ZSYM;
          if constexpr (ZP) z = (int)((*(const uint32_t *)(sb + C::OFF_SZ + col * 4) >> (4 * (gg & 7))) & 15u);
          zf[j] = ZP ? -(1.f + (float)z / C::MAG) : 1.f;
        }
#pragma unroll
        for (int i = 0; i < C::MB2; ++i) {
          const int r0 = wm * (BM / WM) + 32 * i;
          const uint8_t *arow = st + (r0 + c32) * 256;
          u32x4 af[C::MPG];
#pragma unroll
          for (int ss = 0; ss < C::MPG; ++ss)
            af[ss] = *(const u32x4 *)(arow + 16 * ((2 * (gi * C::MPG + ss) + h) ^ (c32 & 15)));
          f32x4 sxq[4];
#pragma unroll
          for (int ii = 0; ii < 4; ++ii)
            sxq[ii] = *(const f32x4 *)(st + C::A + (gi * C::SXR + r0 + 8 * ii + 4 * h) * 4);
          f32x16 g[C::NB2];
#pragma unroll
          for (int j = 0; j < C::NB2; ++j)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
#pragma unroll
              for (int e = 0; e < 4; ++e) g[j][4 * ii + e] = ZP ? sxq[ii][e] * zf[j] : sxq[ii][e];
#pragma unroll
          for (int ss = 0; ss < C::MPG; ++ss)
#pragma unroll
            for (int j = 0; j < C::NB2; ++j) g[j] = mfma32_bf16(af[ss], bw[j][gi * C::MPG + ss], g[j]);
#pragma unroll
          for (int j = 0; j < C::NB2; ++j)
#pragma unroll
            for (int t = 0; t < 16; ++t) acc32[i][j][t] = __builtin_fmaf(g[j][t], c1[j], acc32[i][j][t]);
        }
      }
      continue;
    }

    // weight operands of the wave's NJ column blocks for the 4 K32 steps
    u32x4 bw[C::NJ][4];
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) {
      const int blk = wn * C::NJ + j;
      u32x4 v;
      if constexpr (BITS == 4) {
        v = *(const u32x4 *)(sb + blk * 1024 + 16 * lane);
      } else {
        const uint32_t *p = (const uint32_t *)(sb + blk * 768 + 12 * lane);
        v = u32x4{p[0], p[1], p[2], 0u};
      }
      if constexpr (FP4) {
        // K32 step s is K-group kb * GPB + s of column col
        const int col = wn * 16 * C::NJ + 16 * j + r16;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int gg = kb * C::GPB + s;
          const float sc = bf16_bits_to_f32(*(const uint16_t *)(sb + C::OFF_SS + col * 16 + 2 * (gg & 7)));
          bw[j][s] = u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v[s], sc, 0)),
                           __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v[s], sc, 1)),
                           __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v[s], sc, 2)),
                           __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v[s], sc, 3))};
        }
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) bw[j][s] = unpack_br<BITS>(v, s, umask, umagic);
      }
    }
    if constexpr (FP4) {
#pragma unroll
      for (int i = 0; i < C::MI; ++i) {
        const int r0 = wm * (BM / WM) + 16 * i;
        if (C::SKIP_ROWS && r0 >= tr.rows) continue;  // workgroup-uniform
        const uint8_t *arow = st + (r0 + r16) * 256;
#pragma unroll
        for (int ss = 0; ss < 4; ++ss) {
          const u32x4 af = *(const u32x4 *)(arow + 16 * ((4 * ss + q) ^ r16));
#pragma unroll
          for (int j = 0; j < C::NJ; ++j) acc[i][j] = mfma_bf16(af, bw[j][ss], acc[i][j]);
        }
      }
      continue;
    }
#pragma unroll
    for (int gi = 0; gi < C::GPB; ++gi) {
      const int gg = kb * C::GPB + gi;
      float c1[C::NJ], zf[C::NJ];
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) {
        const int col = wn * 16 * C::NJ + 16 * j + r16;
        const uint32_t sbits = *(const uint16_t *)(sb + C::OFF_SS + col * 16 + 2 * (gg & 7));
        c1[j] = C::MAG * bf16_bits_to_f32(sbits);
        int z = C::ZSYM;
        if constexpr (ZP) z = (int)((*(const uint32_t *)(sb + C::OFF_SZ + col * 4) >> (4 * (gg & 7))) & 15u);
        // symmetric formats: the row sums arrive pre-multiplied by -(1 + z / MAG)
        zf[j] = ZP ? -(1.f + (float)z / C::MAG) : 1.f;
      }
#pragma unroll
      for (int i = 0; i < C::MI; ++i) {
        const int r0 = wm * (BM / WM) + 16 * i;
        if (C::SKIP_ROWS && r0 >= tr.rows) continue;  // workgroup-uniform
        const uint8_t *arow = st + (r0 + r16) * 256;
        u32x4 af[C::JPG];
#pragma unroll
        for (int ss = 0; ss < C::JPG; ++ss)
          af[ss] = *(const u32x4 *)(arow + 16 * ((4 * (gi * C::JPG + ss) + q) ^ r16));
        const f32x4 sx = *(const f32x4 *)(st + C::A + (gi * C::SXR + r0 + 4 * q) * 4);
        f32x4 g[C::NJ];
#pragma unroll
        for (int j = 0; j < C::NJ; ++j) g[j] = ZP ? sx * zf[j] : sx;
#pragma unroll
        for (int ss = 0; ss < C::JPG; ++ss)
#pragma unroll
          for (int j = 0; j < C::NJ; ++j) g[j] = mfma_bf16(af[ss], bw[j][gi * C::JPG + ss], g[j]);
#pragma unroll
        for (int j = 0; j < C::NJ; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(g[j][e], c1[j], acc[i][j][e]);
      }
    }
  }

  // output through LDS (the ring is free once every wave is past its last stage)
  lds_barrier();
  if constexpr (C::M32) {
    // 16-row slab s = rows 16 s .. 16 s + 15 of the wave tile: 32-row block
    // s / 2, accumulator rows 8 ii + 4 h + e with ii in {2 (s % 2), 2 (s % 2) + 1}
    const int h = lane >> 5, c32 = lane & 31;
    store_slabs<C::MI, C::NJ>(
        a, tr,
        [&](int sl, uint8_t *l, int pitch, bool f32) {
#pragma unroll
          for (int i = 0; i < C::MB2; ++i) {
            if (i != sl / 2) continue;
#pragma unroll
            for (int j = 0; j < C::NB2; ++j)
#pragma unroll
              for (int iq = 0; iq < 2; ++iq)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const int ii = 2 * (sl & 1) + iq;
                  slab_put(l, pitch, f32, 8 * iq + 4 * h + e, 32 * j + c32, acc32[i][j][4 * ii + e]);
                }
          }
        },
        wm * (BM / WM), (nt0 + wn * C::NJ) * 16, smem + wave * store_tile_lds_bytes<C::MI, C::NJ>());
  } else {
    store_tile<C::MI, C::NJ>(a, tr, [&](int i, int j) { return acc[i][j]; }, wm * (BM / WM),
                             (nt0 + wn * C::NJ) * 16, smem + wave * store_tile_lds_bytes<C::MI, C::NJ>());
  }
}

// Group row sums of bf16 X: xs[g * rows + r] = factor * (sum of x[r, g*GROUP ..
// + GROUP-1]) in fp32.  One wave per row; lane l sums 16-byte chunks l, l + 64,
// ..., and the GROUP / 8 lanes holding one group's chunks combine by butterfly.
template <int GROUP>
__global__ __launch_bounds__(256) void group_sums_kernel(const uint16_t *x, int64_t ldx, int rows,
                                                         int k, float factor, float *xs) {
  constexpr int CPG = GROUP / 8;  // chunks per group
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint16_t *xr = x + (int64_t)row * ldx;
  const int chunks = k / 8;  // a multiple of 16 (K % 128 == 0)
  for (int c = lane; c < chunks; c += 64) {
    const u32x4 v = *(const u32x4 *)(xr + 8 * c);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s += __uint_as_float(v[e] << 16);
      s += __uint_as_float(v[e] & 0xFFFF0000u);
    }
#pragma unroll
    for (int off = 1; off < CPG; off <<= 1) s += __shfl_xor(s, off);
    if ((lane & (CPG - 1)) == 0) xs[(int64_t)(c / CPG) * rows + row] = s * factor;
  }
}

template <int BM, int BN, int WM, int WN, int BITS, bool ZP, int GROUP, bool MOE, bool FP4 = false>
static hipError_t launch_a16_tiled_t(const GemmArgs &a, int64_t xs_rows, int64_t tiles_cap, float *xs,
                                     bool sums, hipStream_t s) {
  using C = A16Cfg<BM, BN, WM, WN, BITS, ZP, GROUP>;
  static_assert(C::LDS >= C::WAVES * store_tile_lds_bytes<C::MI, C::NJ>(), "epilogue LDS");
  hipError_t e;
  if (sums && !FP4) {
    const float factor = ZP ? 1.f : -(1.f + (float)C::ZSYM / C::MAG);
    const int64_t rows_blocks = (xs_rows + 3) / 4;
    hipLaunchKernelGGL(group_sums_kernel<GROUP>, dim3((unsigned)rows_blocks), dim3(256), 0, s,
                       (const uint16_t *)a.x, a.ldx, (int)xs_rows, a.k, factor, xs);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t m_tiles = MOE ? tiles_cap : (a.m + BM - 1) / BM;
  const int64_t n_tiles_wg = (a.n_tiles + C::NBLK - 1) / C::NBLK;
  const int64_t total = m_tiles * n_tiles_wg;
  const int64_t per_xcd = (total + kXcds - 1) / kXcds;
  const size_t lds = (size_t)C::LDS;
  auto kern = a16_tiled_kernel<BM, BN, WM, WN, BITS, ZP, GROUP, MOE, FP4>;
  e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)(per_xcd * kXcds)), dim3(64 * C::WAVES), lds, s, a,
                     (const float *)xs, (int)xs_rows);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int BITS, bool ZP, bool MOE>
static hipError_t launch_group(const GemmArgs &a, int group, int64_t xs_rows, int64_t cap, float *xs,
                               bool sums, hipStream_t s) {
  switch (group) {
    case 32: return launch_a16_tiled_t<BM, BN, WM, WN, BITS, ZP, 32, MOE>(a, xs_rows, cap, xs, sums, s);
    case 64: return launch_a16_tiled_t<BM, BN, WM, WN, BITS, ZP, 64, MOE>(a, xs_rows, cap, xs, sums, s);
    case 128: return launch_a16_tiled_t<BM, BN, WM, WN, BITS, ZP, 128, MOE>(a, xs_rows, cap, xs, sums, s);
  }
  return hipErrorInvalidValue;
}

template <int BM, int BN, int WM, int WN, bool MOE>
static hipError_t launch_fmt(const GemmArgs &a, const qg_layer_desc &d, int64_t xs_rows, int64_t cap,
                             float *xs, bool sums, hipStream_t s) {
  const int g = d.group_size;
  switch (d.wtype) {
    case QG_W_INT4:
    case QG_W_E0M3:  // stored as offset-binary INT4
      return launch_group<BM, BN, WM, WN, 4, false, MOE>(a, g, xs_rows, cap, xs, sums, s);
    case QG_W_UINT4: return launch_group<BM, BN, WM, WN, 4, true, MOE>(a, g, xs_rows, cap, xs, sums, s);
    case QG_W_INT3: return launch_group<BM, BN, WM, WN, 3, false, MOE>(a, g, xs_rows, cap, xs, sums, s);
    case QG_W_UINT3: return launch_group<BM, BN, WM, WN, 3, true, MOE>(a, g, xs_rows, cap, xs, sums, s);
    case QG_W_MXFP4:  // MXFP4 x bf16
      if (fp4_a16(d) && g == 32) return launch_a16_tiled_t<BM, BN, WM, WN, 4, false, 32, MOE, true>(a, xs_rows, cap, xs, false, s);
      return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

uint64_t a16_tiled_ws_bytes(const qg_layer_desc &d, int64_t m) {
  return align_up((uint64_t)(d.k / d.group_size) * (uint64_t)m * 4, 256);
}

// Dense: a.m rows in bm x bn tiles (256 x 128, 128 x 128 or 128 x 256).
// MoE: the tile list a.tiles (capacity tiles_cap) of bm-row tiles, bm = 128
// (large experts; 128 or 256 columns) or 64 / 32 (small experts: 8 waves of
// 16 columns each).
// waves: 4 (2 x 2, one per SIMD) or 8 (4 x 2, or 2 x 4 for 256 columns).
// sums = false reuses the group row sums already in ws.
hipError_t launch_a16_tiled(const GemmArgs &a, const qg_layer_desc &d, int bm, int bn, bool moe,
                            int64_t xs_rows, int64_t tiles_cap, int waves, void *ws, bool sums,
                            hipStream_t s) {
  if (a.k % 128 != 0) return hipErrorInvalidValue;
  float *xs = (float *)ws;
  if (moe) {
    if (bm == 64) return launch_fmt<64, 128, 1, 8, true>(a, d, xs_rows, tiles_cap, xs, sums, s);
    if (bm == 32) return launch_fmt<32, 128, 1, 8, true>(a, d, xs_rows, tiles_cap, xs, sums, s);
    if (bm != kMoeTileRows) return hipErrorInvalidValue;
    if (bn == 256 && waves == 8) return launch_fmt<kMoeTileRows, 256, 2, 4, true>(a, d, xs_rows, tiles_cap, xs, sums, s);
    return waves == 8 ? launch_fmt<kMoeTileRows, 128, 4, 2, true>(a, d, xs_rows, tiles_cap, xs, sums, s)
                      : launch_fmt<kMoeTileRows, 128, 2, 2, true>(a, d, xs_rows, tiles_cap, xs, sums, s);
  }
  if (bn == 256) {
    if (bm != 128 || waves != 8) return hipErrorInvalidValue;
    return launch_fmt<128, 256, 2, 4, false>(a, d, xs_rows, 0, xs, sums, s);
  }
  if (waves == 8)
    return bm == 256 ? launch_fmt<256, 128, 4, 2, false>(a, d, xs_rows, 0, xs, sums, s)
                     : launch_fmt<128, 128, 4, 2, false>(a, d, xs_rows, 0, xs, sums, s);
  return bm == 256 ? launch_fmt<256, 128, 2, 2, false>(a, d, xs_rows, 0, xs, sums, s)
                   : launch_fmt<128, 128, 2, 2, false>(a, d, xs_rows, 0, xs, sums, s);
}

}  // namespace qg
