// Large-M tiled kernel for MXFP4 weights x MXFP8 activations on gfx950.
//
// The announcement's "W8A8 / W4A8 / W4A4" section describes the W4A8-MXFP4
// path as MXFP4 weights dequantized at load time and multiplied on FP8 tensor
// cores.  On CDNA4 the matrix core takes e2m1 and e4m3 operands with their
// e8m0 block scales directly (v_mfma_scale_f32_16x16x128_f8f6f4), so nothing is
// dequantized: the kernel only moves bytes.
//
// Tiling: a workgroup computes a BM x BN tile of Y (BN = 256, or 224 / 192 so
// that the tile count fills whole rounds of the 256 CUs) with WM x WN waves,
// each (BM / WM) x (BN / WN) as blocks of 16 x 16.  The default is 8 waves (4 x 2,
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
//   B   BN / 16 packed weight blocks of 1 KB copied verbatim (the packed
//       layout already stores each lane's 16-byte B operand contiguously);
//   SA  the four e8m0 scales of each activation row for this K step (dense
//       launches read them from a copy regrouped by K step, so for 256-row
//       tiles one 16-byte-per-lane copy moves all of them).
// The weight scales change every fourth K step only: a separate two-slot ring
// SW holds, for each of the BN weight columns and quarters q, the dword with
// its e8m0 scales of K steps 4j .. 4j + 3, loaded with stage 4j as whole
// 256-byte units (one per n-tile, four per 16-byte-per-lane copy).  Scale
// copies of a dword per lane cost the load path about as much as a 1-KB copy,
// so every scale copy here is a 16-byte one wherever the layout allows.  Each
// wave counts its own loads: "stage kb has landed" is a wait until only the
// wave's loads of stage kb + 1 are outstanding (where the blocks do not
// divide evenly, the last waves copy the final block again, the same bytes to
// the same place; SA and SW copies go to the first few waves), followed by a
// workgroup barrier.  Inside a K step the next row
// block's LDS reads are scheduled ahead of the current block's 8 MFMAs.
//
// W8A8 block FP8 (F8; the announcement's "W8A8 / W4A8 / W4A4" section): e4m3
// weights in 2-KB blocks of the scaled MFMA's 8-bit operand layout with one
// fp32 scale per 128 x 128 block, e4m3 activations with one fp32 scale per
// row and 128 K.  Per K step each 16 x 16 block is one scaled MFMA with unit
// scales and C = 0 (the weights as its A operand, so lane (q, r) receives
// columns 4q .. 4q + 3 of activation row r), then one fp32 fma per element
// with fl32(sa[row] * sw[n-tile]); the epilogue stores the transposed blocks.
// The activation scales are copied per step, 4 bytes per row (a 64-lane
// gather per 64 rows); the weight scales go to the SW ring as 16 bytes (four
// steps) per n-tile.
//
// Per-token FP8 activations (RS; the announcement's "End to end" section
// serves W4A8 with them): e4m3 A operands under a unit block scale (code
// 127), no SA copies, and each output row multiplied by its row's fp32 scale
// in the epilogue.
//
// W4A4 (A4: MXFP4 activations, the announcement's "W8A8 / W4A8 / W4A4"
// section): the same kernel with e2m1 A operands.  A row holds 64 bytes per K
// step, a lane's operand is the 16 bytes of K 32q .. 32q + 31 (the layout the
// packed weights use for B), and each row's four 16-byte chunks sit at slot
// c ^ ((row >> 1) & 3), so the eight lanes of one LDS read phase (rows r .. r
// + 7, one chunk) cover all 128 bytes of a bank row.
//
// Work order: workgroups are dealt round-robin to the 8 XCDs; the tile index
// is remapped so each XCD owns a contiguous range of a grouped (GM m-tiles at
// a time) raster, so the tiles running together on one XCD share activation
// rows and weight columns in that XCD's L2.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "qg_device.h"
#include "qg_internal.h"

namespace qg {

constexpr int kStages = 3;

// acc += (e2m1 A, e8m0 scale sa) x (e2m1 B, e8m0 scale: byte SB of sb_word)
extern "C" __device__ f32x4 qg_mfma_scale_16x16x128_f4_f4(i32x4 a, i32x4 b, f32x4 c, int fmt_a, int fmt_b,
                                                          int opsel_a, int scale_a, int opsel_b, int scale_b)
    __asm("llvm.amdgcn.mfma.scale.f32.16x16x128.f8f6f4.v4i32.v4i32");

template <int SB>
__device__ __forceinline__ f32x4 mfma_e2m1_e2m1(i32x4 a, i32x4 b, f32x4 c, int sa, int sb_word) {
  return qg_mfma_scale_16x16x128_f4_f4(a, b, c, 4, 4, 0, sa, SB, sb_word);
}

// BM x BN tile, WM x WN waves, each wave (BM / WM) x (BN / WN).  SAR: the
// activation scales go to a two-slot ring of 4-step runs (16 bytes per row)
// instead of 4 bytes per row in every stage.  A4: e2m1 activations.  F8:
// W8A8 (2-KB weight blocks, fp32 scales).
template <int BM, int BN, int WM, int WN, bool SAR, bool A4 = false, bool F8 = false>
struct MxCfg {
  static constexpr int WAVES = WM * WN;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int NBLK = BN / 16;                      // packed n-tiles per tile
  static constexpr int AROW = A4 ? 64 : 128;                // A bytes per row and K step
  static constexpr int A = BM * AROW;
  static constexpr int BBLK = F8 ? 2048 : 1024;             // bytes of one packed block
  static constexpr int B = NBLK * BBLK;
  static constexpr int B_COPIES = B / 1024;                 // 1-KB copies of B per stage
  static constexpr int SA = SAR ? 0 : BM * 4;
  // 1-KB copies: 4 n-tiles' 256-B units each (F8: one copy, 16 bytes per n-tile)
  static constexpr int SW_PIECES = F8 ? 1 : (NBLK + 3) / 4;
  static constexpr int SW = SW_PIECES * 1024;               // one slot (units past NBLK unused)
  static constexpr int STAGE = A + B + SA;
  static constexpr int OFF_SW = 3 * STAGE;                  // the two SW slots
  static constexpr int SAR_SLOT = SAR ? BM * 16 : 0;        // [row][4 steps x 4 bytes]
  static constexpr int OFF_SAR = OFF_SW + 2 * SW;           // the two SA ring slots
  static constexpr int LDS = OFF_SAR + 2 * SAR_SLOT;
  static constexpr int A_COPIES = BM * AROW / 1024;          // 1-KB copies of A per stage
  // per wave; where they do not divide evenly (e2m1 64-row tiles: 4 copies,
  // 8 waves) the last waves repeat the final copy, the same bytes to the
  // same place
  static constexpr int A_LOADS = (A_COPIES + WAVES - 1) / WAVES;
  static constexpr int B_LOADS = (B_COPIES + WAVES - 1) / WAVES;  // 1-KB copies of B per wave
  static constexpr int SA_WAVES = BM / 64;                  // waves that copy a 256-B SA piece
  static constexpr int AB_LOADS = A_LOADS + B_LOADS;
  static constexpr int MB = BM / WM / 16;                   // 16-row blocks per wave
  static constexpr int NB = BN / WN / 16;                   // 16-column blocks per wave
  static_assert(BN % (16 * WN) == 0, "column blocks per wave");
  static_assert(A_COPIES >= 1 && BM * AROW % 1024 == 0, "A copies");
  static_assert(WAVES >= SA_WAVES && WAVES >= SW_PIECES, "SA / SW pieces");
  static_assert(!F8 || (!SAR && !A4 && NBLK <= 64), "W8A8: per-step activation scales, e4m3 rows");
  static_assert(LDS <= 160 * 1024, "LDS");
};

template <int BM, int BN, int WM, int WN, bool MOE, bool SAR, bool A4, bool RS, bool F8>
__global__ __launch_bounds__(64 * WM * WN) void mx_tiled_kernel(GemmArgs a) {
  static_assert(!RS || (!SAR && !A4), "per-token scales: e4m3 rows, no activation scale ring");
  static_assert(!(RS && F8), "one activation scale form");
  using C = MxCfg<BM, BN, WM, WN, SAR, A4, F8>;
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
  const int nt0 = tn * C::NBLK;      // first 16-column n-tile
  const int kbs = a.k_blocks;
  const int kq = F8 ? kbs * 4 : a.k >> 5;  // activation scale bytes per row
  const uint8_t *x = (const uint8_t *)a.x;
  const uint8_t *wsc = wexp + a.scales_offset;

  // per-lane source offsets (32-bit, added to wave-uniform bases at issue)
  uint32_t a_off[C::A_LOADS];
  auto a_copy = [&](int i) { return min(wave * C::A_LOADS + i, C::A_COPIES - 1); };
#pragma unroll
  for (int i = 0; i < C::A_LOADS; ++i) {
    if constexpr (A4) {
      // 16 rows of 4 chunks per copy: lane -> row lane / 4, slot lane % 4
      const int row = 16 * a_copy(i) + (lane >> 2);
      const int c = (lane & 3) ^ ((row >> 1) & 3);
      a_off[i] = (uint32_t)(tr.x(a, row) * a.ldx + 16 * c);
    } else {
      const int row = 8 * a_copy(i) + (lane >> 3);
      const int c = (lane & 7) ^ (row & 7);
      a_off[i] = (uint32_t)(tr.x(a, row) * a.ldx + 16 * c);
    }
  }
  const uint8_t *b_base = wexp + 16 * lane;
  // copy i of this wave: 1-KB piece (and LDS slot) min(B_LOADS wave + i,
  // B_COPIES - 1) of the tile's blocks (F8: two pieces per 2-KB block)
  constexpr int PB = F8 ? 1 : 0;  // log2 of the pieces per block
  auto blk_of = [&](int i) { return min(wave * C::B_LOADS + i, C::B_COPIES - 1); };
  uint32_t b_blk[C::B_LOADS];  // first packed block of the n-tile of each of the wave's pieces
#pragma unroll
  for (int i = 0; i < C::B_LOADS; ++i)
    b_blk[i] = (uint32_t)min(nt0 + (blk_of(i) >> PB), a.n_tiles - 1) * kbs;
  // SA: BM rows of 4 bytes.  Dense 256-row tiles: one 1-KB copy by wave 0
  // from the scales regrouped by K step (rows padded to 256, so the copy
  // stays in the buffer; rows past M are never stored).  Otherwise BM / 64
  // pieces of 256 B, one per wave of the first BM / 64, with rows clamped.
  // With SAR (K % 512 == 0 and 16-byte aligned scales) the first BM / 64
  // waves copy, every fourth step, the 16 bytes of 4 steps of one row per
  // lane straight from the row-major scales into the SA ring.
  constexpr bool SA_X4 = !F8 && !SAR && !MOE && BM == 256;
  const bool sa_wave = !RS && (SA_X4 ? wave == 0 : wave < C::SA_WAVES);
  const int64_t m_pad = ((int64_t)a.m + 255) & ~(int64_t)255;  // regrouped row stride
  const int64_t sa_row = SA_X4 ? (int64_t)tr.base + 4 * lane : tr.x(a, (sa_wave ? wave : 0) * 64 + lane);
  // per K step: + 4 bytes (rows of kq bytes) or + 4 m_pad bytes (dense, regrouped by step)
  const bool sa_rows = MOE || SAR || F8;
  const uint8_t *sa_src = RS ? nullptr : sa_rows ? a.x_scales + sa_row * kq : (const uint8_t *)(a.x_scales_t + sa_row);
  const int64_t sa_step = sa_rows ? 4 : 4 * m_pad;
  // SW: copy p (by wave p < SW_PIECES) moves the 256-B units of n-tiles
  // 4p .. 4p + 3 of the tile for K steps 4j .. 4j + 3 (unit of n-tile nt at
  // nt * kb_pad / 4 * 256 + 256 j); lanes 16u .. 16u + 15 copy unit u
  // F8: lane l copies the 16 bytes (four steps' fp32 scales) of n-tile
  // nt0 + l (clamped; lanes past the tile's n-tiles fill unused slot bytes)
  const bool sw_wave = wave < C::SW_PIECES;
  const uint32_t sw_off =
      F8 ? (uint32_t)((uint64_t)min(nt0 + lane, a.n_tiles - 1) * a.kb_pad * 4)
         : (uint32_t)((uint64_t)min(nt0 + 4 * wave + (lane >> 4), a.n_tiles - 1) * (a.kb_pad >> 2) * 256 +
                      16 * (lane & 15));
  constexpr int SW_STEP = F8 ? 4 : 64;  // scale bytes per n-tile and K step

  auto issue = [&](int kb, int buf) {
    uint8_t *st = smem + buf * C::STAGE;
    const uint8_t *xk = x + kb * C::AROW;
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i)
      lds_dma16(xk + a_off[i], st + a_copy(i) * 1024);
#pragma unroll
    for (int i = 0; i < C::B_LOADS; ++i)
      lds_dma16(b_base + ((uint64_t)(b_blk[i] + kb) << (10 + PB)) + (F8 ? (blk_of(i) & 1) * 1024 : 0),
                st + C::A + blk_of(i) * 1024);
    if constexpr (SAR) {
      if ((kb & 3) == 0 && sa_wave)
        lds_dma16(sa_src + sa_step * kb, smem + C::OFF_SAR + ((kb >> 2) & 1) * C::SAR_SLOT + wave * 1024);
    } else if (sa_wave) {
      if constexpr (SA_X4)
        lds_dma16(sa_src + sa_step * kb, st + C::A + C::B);
      else
        lds_dma4(sa_src + sa_step * kb, st + C::A + C::B + wave * 256);
    }
    if ((kb & 3) == 0 && sw_wave)
      lds_dma16(wsc + SW_STEP * kb + sw_off, smem + C::OFF_SW + ((kb >> 2) & 1) * C::SW + wave * 1024);
  };

  f32x4 acc[C::MB][C::NB];
#pragma unroll
  for (int i = 0; i < C::MB; ++i)
#pragma unroll
    for (int j = 0; j < C::NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  issue(0, 0);
  if (kbs > 1) issue(1, 1);
  // the wave's B scale dwords of the current 4-step group (one byte per step,
  // picked by the MFMA's scale byte select)
  uint32_t swv[C::NB];
  // one K step; S = kb % 4 is a compile-time constant (the loop below is
  // unrolled by four) because the byte select is an instruction field
  auto step = [&](int kb, auto s_tag) {
    constexpr int S = decltype(s_tag)::value;
    // outstanding after stage kb: this wave's loads of stage kb + 1
    if (kb + 1 < kbs) {
      const bool ring_next = ((kb + 1) & 3) == 0;  // stage kb + 1 also fills the scale rings
      const int extra = ((SAR ? ring_next : true) && sa_wave ? 1 : 0) + (ring_next && sw_wave ? 1 : 0);
      if (extra == 0) {
        QG_WAIT_VMCNT(C::AB_LOADS);
      } else if (extra == 1) {
        QG_WAIT_VMCNT(C::AB_LOADS + 1);
      } else {
        QG_WAIT_VMCNT(C::AB_LOADS + 2);
      }
    } else {
      QG_WAIT_VMCNT(0);
    }
    __builtin_amdgcn_s_barrier();  // stage kb is in LDS; stage kb - 1 is free
    if (kb + 2 < kbs) issue(kb + 2, (kb + 2) % kStages);
    const uint8_t *st = smem + (kb % kStages) * C::STAGE;
    if constexpr (F8) {
      // weights (A operand, 32 bytes per lane) and their step scales
      i32x8 wf[C::NB];
      float swf[C::NB];
#pragma unroll
      for (int j = 0; j < C::NB; ++j) {
        const int blk = wn * C::NB + j;
        const u32x4 lo = *(const u32x4 *)(st + C::A + blk * 2048 + 32 * lane);
        const u32x4 hi = *(const u32x4 *)(st + C::A + blk * 2048 + 32 * lane + 16);
        wf[j] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        swf[j] = *(const float *)(smem + C::OFF_SW + ((kb >> 2) & 1) * C::SW + blk * 16 + 4 * (kb & 3));
      }
      const int mbv = WM == 1 ? min(C::MB, (tr.rows + 15) >> 4) : C::MB;  // (small tiles: live row blocks)
#pragma unroll
      for (int i = 0; i < C::MB; ++i) {
        if (i >= mbv) continue;  // workgroup-uniform
        const int row = wm * (BM / WM) + i * 16 + r16;
        const uint8_t *ap = st + row * C::AROW;
        const u32x4 lo = *(const u32x4 *)(ap + 16 * (q ^ (row & 7)));
        const u32x4 hi = *(const u32x4 *)(ap + 16 * ((4 + q) ^ (row & 7)));
        const i32x8 af = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        const float sa = *(const float *)(st + C::A + C::B + 4 * row);
#pragma unroll
        for (int j = 0; j < C::NB; ++j) {
          // cbsz = blgp = 0: both operands e4m3; scale codes 127 = 2^0
          const f32x4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[j], af, f32x4{0.f, 0.f, 0.f, 0.f},
                                                                            0, 0, 0, 127, 0, 127);
          const float f = sa * swf[j];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(p[e], f, acc[i][j][e]);
        }
      }
      return;
    }
    i32x4 bf[C::NB];
#pragma unroll
    for (int j = 0; j < C::NB; ++j) {
      const int blk = wn * C::NB + j;
      const u32x4 v = *(const u32x4 *)(st + C::A + blk * 1024 + 16 * lane);
      bf[j] = i32x4{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
      if constexpr (S == 0)  // the SW slot of steps kb .. kb + 3 landed with stage kb
        swv[j] = *(const uint32_t *)(smem + C::OFF_SW + ((kb >> 2) & 1) * C::SW + ((blk * 16 + r16) * 4 + q) * 4);
    }
    using AFrag = std::conditional_t<A4, i32x4, i32x8>;
    auto read_a = [&](int i, AFrag &af, int &asc) {
      const int row = wm * (BM / WM) + i * 16 + r16;
      const uint8_t *ap = st + row * C::AROW;
      if constexpr (A4) {
        const u32x4 v = *(const u32x4 *)(ap + 16 * (q ^ ((row >> 1) & 3)));
        af = i32x4{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
      } else {
        const u32x4 lo = *(const u32x4 *)(ap + 16 * (q ^ (row & 7)));
        const u32x4 hi = *(const u32x4 *)(ap + 16 * ((4 + q) ^ (row & 7)));
        af = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                   (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
      if constexpr (RS)
        asc = 127;  // unit scale: the row's fp32 scale is applied to the output
      else if constexpr (SAR)
        asc = smem[C::OFF_SAR + ((kb >> 2) & 1) * C::SAR_SLOT + 16 * row + 4 * (kb & 3) + q];
      else
        asc = st[C::A + C::B + 4 * row + q];
    };
    auto mma = [&](const AFrag &af, const i32x4 &bf, f32x4 c, int sa, int sb) {
      if constexpr (A4)
        return mfma_e2m1_e2m1<S>(af, bf, c, sa, sb);
      else
        return mfma_e4m3_e2m1<S>(af, bf, c, sa, sb);
    };
    AFrag af[2];
    int asc[2];
    if constexpr (WM == 1) {
      // small tiles (MoE experts with few rows): row blocks past the tile's
      // rows are skipped (workgroup-uniform)
      const int mbv = min(C::MB, (tr.rows + 15) >> 4);
#pragma unroll
      for (int i = 0; i < C::MB; ++i) {
        if (i < mbv) {
          read_a(i, af[0], asc[0]);
#pragma unroll
          for (int j = 0; j < C::NB; ++j)
            acc[i][j] = mma(af[0], bf[j], acc[i][j], asc[0], (int)swv[j]);
        }
      }
      return;
    }
    read_a(0, af[0], asc[0]);
    // B (NB reads, plus NB scale dwords every fourth step) and A block 0 (3
    // reads; 2 for e2m1) first
    constexpr int AR = A4 ? 2 : 3;
    __builtin_amdgcn_sched_group_barrier(0x100, (S == 0 ? 2 : 1) * C::NB + AR, 0);
#pragma unroll
    for (int i = 0; i < C::MB; ++i) {
      if (i + 1 < C::MB) read_a(i + 1, af[(i + 1) & 1], asc[(i + 1) & 1]);
#pragma unroll
      for (int j = 0; j < C::NB; ++j)
        acc[i][j] = mma(af[i & 1], bf[j], acc[i][j], asc[i & 1], (int)swv[j]);
      if (i + 1 < C::MB) __builtin_amdgcn_sched_group_barrier(0x100, AR, 0);  // next block's reads
      __builtin_amdgcn_sched_group_barrier(0x008, C::NB, 0);                // this block's MFMAs
    }
  };
  for (int kb = 0; kb < kbs; kb += 4) {
    step(kb, std::integral_constant<int, 0>{});
    if (kb + 1 < kbs) step(kb + 1, std::integral_constant<int, 1>{});
    if (kb + 2 < kbs) step(kb + 2, std::integral_constant<int, 2>{});
    if (kb + 3 < kbs) step(kb + 3, std::integral_constant<int, 3>{});
  }

  // per-token FP8: the fp32 scales of the lane's output rows (4 (lane / 16)
  // + e of each 16-row block; rows past the tile read the last row's)
  float rsc[RS ? C::MB : 1][4];
  if constexpr (RS) {
#pragma unroll
    for (int i = 0; i < C::MB; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        rsc[i][e] = ((const float *)a.x_scales)[tr.x(a, wm * (BM / WM) + i * 16 + 4 * q + e)];
  }
  // output through LDS (the ring is free once every wave is past its last stage)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  if constexpr (F8) {
    // transposed blocks: lane (q, r) holds row r, columns 4q .. 4q + 3
    store_slabs<C::MB, C::NB>(
        a, tr,
        [&](int i, uint8_t *l, int pitch, bool f32) {
#pragma unroll
          for (int j = 0; j < C::NB; ++j) {
            const f32x4 v = acc[i][j];
#pragma unroll
            for (int e = 0; e < 4; ++e) slab_put(l, pitch, f32, r16, 16 * j + 4 * q + e, v[e]);
          }
        },
        wm * (BM / WM), (nt0 + wn * C::NB) * 16, smem + wave * store_tile_lds_bytes<C::MB, C::NB>());
    return;
  }
  store_tile<C::MB, C::NB>(a, tr,
                           [&](int i, int j) {
                             f32x4 v = acc[i][j];
                             if constexpr (RS) {
#pragma unroll
                               for (int e = 0; e < 4; ++e) v[e] *= rsc[i][e];
                             }
                             return v;
                           },
                           wm * (BM / WM), (nt0 + wn * C::NB) * 16,
                           smem + wave * store_tile_lds_bytes<C::MB, C::NB>());
}

// Activation scales regrouped by K step: out[kb * m_pad + r] holds the 4 bytes
// of row r's scales for K step kb (bytes 4 kb .. 4 kb + 3 of the row); m_pad =
// m rounded up to 256 (rows m .. m_pad - 1 are not written).  A workgroup
// transposes 16 rows x 64 K steps through LDS (16 rows so that M = 4096 gives
// 256 workgroups): reads run along the rows, writes along the steps.
__global__ __launch_bounds__(256) void mx_scales_by_step_kernel(const uint8_t *xs, int m, int64_t m_pad,
                                                                int kq, int kbs, uint32_t *out) {
  __shared__ uint32_t tile[64][17];
  const int r0 = blockIdx.x * 16, kb0 = blockIdx.y * 64;
  const bool dword = ((uintptr_t)xs & 3) == 0;  // kq % 4 == 0, so every row is aligned too
  for (int i = threadIdx.x; i < 16 * 64; i += 256) {
    const int r = i >> 6, kb = i & 63;
    if (r0 + r < m && kb0 + kb < kbs) {
      const uint8_t *p = xs + (int64_t)(r0 + r) * kq + 4 * (kb0 + kb);
      tile[kb][r] = dword ? *(const uint32_t *)p
                          : ((uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) |
                             ((uint32_t)p[3] << 24));
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 16 * 64; i += 256) {
    const int kb = i >> 4, r = i & 15;
    if (r0 + r < m && kb0 + kb < kbs) out[(int64_t)(kb0 + kb) * m_pad + r0 + r] = tile[kb][r];
  }
}

uint64_t mx_tiled_ws_bytes(int64_t m, int64_t k_blocks) {
  return (uint64_t)((m + 255) & ~(int64_t)255) * (uint64_t)k_blocks * 4;
}

template <int BM, int BN, int WM, int WN, bool MOE, bool SAR, bool A4 = false, bool RS = false,
          bool F8 = false>
static hipError_t launch_mx_tiled_bm(const GemmArgs &a, int64_t tiles_cap, hipStream_t s) {
  using C = MxCfg<BM, BN, WM, WN, SAR, A4, F8>;
  static_assert(C::LDS >= C::WAVES * store_tile_lds_bytes<C::MB, C::NB>(), "epilogue LDS");
  const int64_t m_tiles = MOE ? tiles_cap : (a.m + BM - 1) / BM;
  const int64_t n_tiles_wg = (a.n_tiles + C::NBLK - 1) / C::NBLK;
  const int64_t total = m_tiles * n_tiles_wg;
  const int64_t per_xcd = (total + kXcds - 1) / kXcds;
  const size_t lds = (size_t)C::LDS;
  auto kern = mx_tiled_kernel<BM, BN, WM, WN, MOE, SAR, A4, RS, F8>;
  hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)(per_xcd * kXcds)), dim3(C::THREADS), lds, s, a);
  return hipGetLastError();
}

template <bool SAR>
static hipError_t launch_mx_shape(const GemmArgs &a, int bm, int bn, bool moe, int64_t tiles_cap, int waves,
                                  hipStream_t s) {
  if (waves == 8) {
    if (moe && bm == 64) return launch_mx_tiled_bm<64, 128, 1, 8, true, SAR>(a, tiles_cap, s);
    if (moe && bn == 128) return launch_mx_tiled_bm<kMoeTileRows, 128, 4, 2, true, SAR>(a, tiles_cap, s);
    if (moe) return launch_mx_tiled_bm<kMoeTileRows, 256, 4, 2, true, SAR>(a, tiles_cap, s);
    if (bm == 256) {
      if (bn == 192) return launch_mx_tiled_bm<256, 192, 4, 2, false, SAR>(a, 0, s);
      if (bn == 224) return launch_mx_tiled_bm<256, 224, 4, 2, false, SAR>(a, 0, s);
      return launch_mx_tiled_bm<256, 256, 4, 2, false, SAR>(a, 0, s);
    }
    if (bn == 192) return launch_mx_tiled_bm<128, 192, 4, 2, false, SAR>(a, 0, s);
    if (bn == 224) return launch_mx_tiled_bm<128, 224, 4, 2, false, SAR>(a, 0, s);
    return launch_mx_tiled_bm<128, 256, 4, 2, false, SAR>(a, 0, s);
  }
  if (moe) return launch_mx_tiled_bm<kMoeTileRows, 256, 2, 2, true, SAR>(a, tiles_cap, s);
  return bm == 256 ? launch_mx_tiled_bm<256, 256, 2, 2, false, SAR>(a, 0, s)
                   : launch_mx_tiled_bm<128, 256, 2, 2, false, SAR>(a, 0, s);
}

// e2m1 activations: the same tile shapes as MXFP8.
template <bool SAR>
static hipError_t launch_mx_shape_a4(const GemmArgs &a, int bm, int bn, bool moe, int64_t tiles_cap, int waves,
                                     hipStream_t s) {
  if (moe) {
    if (waves == 8 && bm == 64) return launch_mx_tiled_bm<64, 128, 1, 8, true, SAR, true>(a, tiles_cap, s);
    if (waves == 8 && bn == 128) return launch_mx_tiled_bm<kMoeTileRows, 128, 4, 2, true, SAR, true>(a, tiles_cap, s);
    if (waves == 8) return launch_mx_tiled_bm<kMoeTileRows, 256, 4, 2, true, SAR, true>(a, tiles_cap, s);
    return launch_mx_tiled_bm<kMoeTileRows, 256, 2, 2, true, SAR, true>(a, tiles_cap, s);
  }
  if (waves == 8) {
    if (bm == 256) {
      if (bn == 192) return launch_mx_tiled_bm<256, 192, 4, 2, false, SAR, true>(a, 0, s);
      if (bn == 224) return launch_mx_tiled_bm<256, 224, 4, 2, false, SAR, true>(a, 0, s);
      return launch_mx_tiled_bm<256, 256, 4, 2, false, SAR, true>(a, 0, s);
    }
    if (bn == 192) return launch_mx_tiled_bm<128, 192, 4, 2, false, SAR, true>(a, 0, s);
    if (bn == 224) return launch_mx_tiled_bm<128, 224, 4, 2, false, SAR, true>(a, 0, s);
    return launch_mx_tiled_bm<128, 256, 4, 2, false, SAR, true>(a, 0, s);
  }
  return bm == 256 ? launch_mx_tiled_bm<256, 256, 2, 2, false, SAR, true>(a, 0, s)
                   : launch_mx_tiled_bm<128, 256, 2, 2, false, SAR, true>(a, 0, s);
}

// Per-token FP8 activations: the 8-wave shapes of MXFP8, no scale ring.
static hipError_t launch_mx_shape_rs(const GemmArgs &a, int bm, int bn, bool moe, int64_t tiles_cap, hipStream_t s) {
  if (moe) {
    if (bm == 64) return launch_mx_tiled_bm<64, 128, 1, 8, true, false, false, true>(a, tiles_cap, s);
    if (bn == 128) return launch_mx_tiled_bm<kMoeTileRows, 128, 4, 2, true, false, false, true>(a, tiles_cap, s);
    return launch_mx_tiled_bm<kMoeTileRows, 256, 4, 2, true, false, false, true>(a, tiles_cap, s);
  }
  if (bm == 256) {
    if (bn == 192) return launch_mx_tiled_bm<256, 192, 4, 2, false, false, false, true>(a, 0, s);
    if (bn == 224) return launch_mx_tiled_bm<256, 224, 4, 2, false, false, false, true>(a, 0, s);
    return launch_mx_tiled_bm<256, 256, 4, 2, false, false, false, true>(a, 0, s);
  }
  if (bn == 192) return launch_mx_tiled_bm<128, 192, 4, 2, false, false, false, true>(a, 0, s);
  if (bn == 224) return launch_mx_tiled_bm<128, 224, 4, 2, false, false, false, true>(a, 0, s);
  return launch_mx_tiled_bm<128, 256, 4, 2, false, false, false, true>(a, 0, s);
}

// W8A8: 128-column tiles (the 2-KB weight blocks fill LDS twice as fast);
// dense 256 or 128 rows, MoE 128-row tiles and 64 x 128 small tiles.
static hipError_t launch_mx_shape_f8(const GemmArgs &a, int bm, bool moe, int64_t tiles_cap, hipStream_t s) {
  if (moe) {
    if (bm == 64) return launch_mx_tiled_bm<64, 128, 1, 8, true, false, false, false, true>(a, tiles_cap, s);
    return launch_mx_tiled_bm<kMoeTileRows, 128, 4, 2, true, false, false, false, true>(a, tiles_cap, s);
  }
  if (bm == 256) return launch_mx_tiled_bm<256, 128, 4, 2, false, false, false, false, true>(a, 0, s);
  return launch_mx_tiled_bm<128, 128, 4, 2, false, false, false, false, true>(a, 0, s);
}

// Dense: bm-row tiles (128 or 256) of bn columns (192, 224 or 256 with 8
// waves; 256 with 4).  MoE: the tile list a.tiles (capacity tiles_cap) of
// kMoeTileRows x 256 tiles, or (bm = 64, 8 waves) 64 x 128 small tiles, one
// wave per 16 columns and all rows, for experts with few rows.  The
// activation scales go through the SA ring when K % 512 == 0 and they are
// 16-byte aligned; otherwise dense launches first regroup them by K step into
// ws and MoE launches copy 4 bytes per row and step.  a4: e2m1 activations
// (a.ldx in bytes).  rs: per-token FP8 activations (8 waves whatever `waves`
// says).
hipError_t launch_mx_tiled(const GemmArgs &a_in, int bm, int bn, bool moe, int64_t tiles_cap, int waves,
                           void *ws, hipStream_t s, bool a4, bool rs, bool f8) {
  if (a_in.k % 128 != 0) return hipErrorInvalidValue;
  if (f8) return (a4 || rs || bn != 128) ? hipErrorInvalidValue : launch_mx_shape_f8(a_in, bm, moe, tiles_cap, s);
  if (rs) return a4 ? hipErrorInvalidValue : launch_mx_shape_rs(a_in, bm, bn, moe, tiles_cap, s);
  GemmArgs a = a_in;
  const bool sar = a.k % 512 == 0 && ((uintptr_t)a.x_scales & 15) == 0;
  if (sar) return a4 ? launch_mx_shape_a4<true>(a, bm, bn, moe, tiles_cap, waves, s)
                     : launch_mx_shape<true>(a, bm, bn, moe, tiles_cap, waves, s);
  if (!moe) {
    if (!ws) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mx_scales_by_step_kernel, dim3((unsigned)((a.m + 15) / 16), (unsigned)((a.k_blocks + 63) / 64)),
                       dim3(256), 0, s, a.x_scales, a.m, ((int64_t)a.m + 255) & ~(int64_t)255, a.k >> 5,
                       a.k_blocks, (uint32_t *)ws);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.x_scales_t = (const uint32_t *)ws;
  }
  return a4 ? launch_mx_shape_a4<false>(a, bm, bn, moe, tiles_cap, waves, s)
            : launch_mx_shape<false>(a, bm, bn, moe, tiles_cap, waves, s);
}

}  // namespace qg
