// Wave bodies and kernel templates of the skinny (16-row tile) and decode
// (activations in LDS) GEMM kernels, shared by the translation units that
// instantiate them for the different weight formats (qg_kernels.hip: the
// 4- and 3-bit integer formats and MXFP4; qg_formats.hip: the 1-, 2- and
// 8-bit integer formats, e4m3 weights, per-token and block-scaled FP8).
// Device code only; see qg_kernels.hip for the design of the data path.
#pragma once

#include <hip/hip_runtime.h>

#include "qg_device.h"
#include "qg_internal.h"

// Weight slices are read once per launch: stream them with non-temporal loads.
#ifndef QG_WEIGHT_NT
#define QG_WEIGHT_NT 1
#endif

template <typename V>
__device__ __forceinline__ V load_stream(const V *p) {
#if QG_WEIGHT_NT
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

namespace qg {

constexpr int kMaxWaves = 16;

__device__ __forceinline__ void store_out(void *y, int64_t ldy, int otype, int64_t row, int col,
                                          float v) {
  if (otype == QG_O_F32) {
    ((float *)y)[row * ldy + col] = v;
  } else {
    __bf16 b = (__bf16)v;  // round to nearest even
    ((__bf16 *)y)[row * ldy + col] = b;
  }
}

// Sum in split order of the n >= 1 fp32 partials p[0], p[stride], ...,
// read with agent-scope loads (written by other workgroups): the loads go out
// eight at a time, unconditionally (indices past n re-read the last partial,
// which is not added), so the combine costs one memory round trip per eight
// splits instead of one per split.
__device__ __forceinline__ float sum_partials(const float *p, int64_t stride, int n) {
  float sum = 0.f;
  for (int s0 = 0; s0 < n; s0 += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      v[j] = __hip_atomic_load(p + min(s0 + j, n - 1) * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int j = 0; j < 8; ++j) sum = s0 + j < n ? sum + v[j] : sum;
  }
  return sum;
}

// sum_partials of four values at once (p + e * 64, e = 0..3): all 32 loads of
// a group of eight splits go out before the first add.
__device__ __forceinline__ f32x4 sum_partials4(const float *p, int64_t stride, int n) {
  f32x4 sum = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < n; s0 += 8) {
    float v[8][4];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[j][e] = __hip_atomic_load(p + min(s0 + j, n - 1) * stride + e * 64, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) sum[e] = s0 + j < n ? sum[e] + v[j][e] : sum[e];
  }
  return sum;
}

// ---------------------------------------------------------------------------
// work-item decoding shared by the dense and MoE launches
// ---------------------------------------------------------------------------

struct Item {
  int expert;
  int row0;    // first row of the 16-row tile (dense: row; MoE: sorted position)
  int rows;    // valid rows in the tile (1..16)
  int nb;      // n-block
  int split;   // K split
};

// 16-row tiles of an expert with c rows for the skinny kernel; experts with
// at least min_rows rows (min_rows > 0) belong to the tiled kernels.
__device__ __forceinline__ int skinny_tiles(int c, int min_rows) {
  return (min_rows > 0 && c >= min_rows) ? 0 : (c + 15) >> 4;
}

// Exclusive prefix of per-expert 16-row tile counts, in LDS.  Returns total tiles.
__device__ inline int moe_tile_prefix(const int32_t *offsets, int experts, int min_rows, int *prefix) {
  const int tid = threadIdx.x, nth = blockDim.x;
  __shared__ int wave_tot[kMaxWaves];
  const int per = (experts + nth - 1) / nth;
  const int e0 = tid * per;
  int local = 0;
  for (int e = e0; e < e0 + per && e < experts; ++e)
    local += skinny_tiles(offsets[e + 1] - offsets[e], min_rows);
  int total;
  int run = block_scan_excl(local, wave_tot, &total);
  for (int e = e0; e < e0 + per && e < experts; ++e) {
    prefix[e] = run;
    run += skinny_tiles(offsets[e + 1] - offsets[e], min_rows);
  }
  if (tid == 0) prefix[experts] = total;
  __syncthreads();
  return total;
}

__device__ __forceinline__ Item decode_item(const GemmArgs &a, bool moe, int64_t item,
                                            int n_blocks, int total_tiles, const int *prefix) {
  Item it;
  if (!moe) {
    // dense: x = n-block fastest so neighbouring workgroups share the X tile
    it.expert = 0;
    it.nb = (int)(item % n_blocks);
    const int64_t rest = item / n_blocks;
    const int64_t m_tiles = (a.m + 15) / 16;
    const int mt = (int)(rest % m_tiles);
    it.split = (int)(rest / m_tiles);
    it.row0 = mt * 16;
    it.rows = min(16, a.m - it.row0);
    return it;
  }
  // MoE: m-tile fastest so the tiles of one expert run together and share
  // that expert's weight slice in L2.
  const int mt = (int)(item % total_tiles);
  it.nb = (int)(item / total_tiles);
  it.split = 0;
  int lo = 0, hi = a.num_experts;  // largest e with prefix[e] <= mt
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= mt) lo = mid; else hi = mid;
  }
  it.expert = lo;
  const int seg0 = a.offsets[lo], seg1 = a.offsets[lo + 1];
  it.row0 = seg0 + (mt - prefix[lo]) * 16;
  it.rows = min(16, seg1 - it.row0);
  return it;
}

// Row of the activation operand for tile row r (or -1).
__device__ __forceinline__ int64_t x_row_of(const GemmArgs &a, bool moe, const Item &it, int r) {
  if (r >= it.rows) return -1;
  const int pos = it.row0 + r;
  if (!moe) return pos;
  if (a.x_rows == QG_ROWS_SORTED) return pos;
  const int p = a.sorted_ids[pos];
  return a.x_rows == QG_ROWS_BY_TOKEN ? (int64_t)(p / a.topk) : (int64_t)p;
}

__device__ __forceinline__ int64_t y_row_of(const GemmArgs &a, bool moe, const Item &it, int r) {
  const int pos = it.row0 + r;
  if (!moe || a.y_rows == QG_ROWS_SORTED) return pos;
  return a.sorted_ids[pos];
}

// ---------------------------------------------------------------------------
// wave bodies: one wave computes acc[t] (16 rows x 16 columns of n-tile nt0+t)
// over k-blocks [kb0, kb0 + KR) of its expert.
// ---------------------------------------------------------------------------

struct NoHook {
  __device__ __forceinline__ void operator()() const {}
};

// Kernel format (FMT) of an instance:
//   0 INT4, 1 UINT4 + zero point, 2 INT3, 3 UINT3 + zp     bf16 activations
//   4 MXFP4 x MXFP8, 5 MXFP4 x bf16, 6 MXFP4 x MXFP4 (activations widened to e4m3)
//   7 INT8 (also e0m7), 8 UINT8 + zp, 9 INT2, 10 UINT2 + zp, 11 INT1,
//   12 UINT1 + zp, 13 e4m3 weights                          bf16 activations
//   14 MXFP4 x per-token FP8 (e4m3, one fp32 scale per row)
//   15 W8A8: e4m3 x e4m3, fp32 scales per 128 x 128 weight block and per row and 128 K
template <int FMT>
struct FmtTraits {
  static constexpr bool MXW = FMT == 4 || FMT == 6 || FMT == 14;  // mx_wave
  static constexpr bool F8 = FMT == 15;                            // f8_wave
  static constexpr bool EXT = FMT >= 7 && FMT <= 13;               // a16x_wave
  static constexpr int BITS = (FMT <= 1 || FMT == 5) ? 4
                              : FMT <= 3                           ? 3
                              : (FMT == 7 || FMT == 8 || FMT == 13) ? 8
                              : (FMT == 9 || FMT == 10)             ? 2
                              : (FMT == 11 || FMT == 12)            ? 1
                                                                    : 4;
  static constexpr bool ZP = FMT == 1 || FMT == 3 || FMT == 8 || FMT == 10 || FMT == 12;
  static constexpr bool ROW_SCALE = FMT == 14;  // output rows times the activation row's fp32 scale
  static constexpr bool SWAP = FMT == 15;       // accumulator lane (q, r16) = (columns 4q + e, row r16)
};

// Weight blocks a decode-kernel wave keeps in flight (see a16_wave): 4 of its
// KR = 8 blocks; every block at once elsewhere.
template <bool XL, int KR>
constexpr int a16_pipe_depth() {
  return XL && KR > 4 ? 4 : KR;
}

// XL: the activation row comes from LDS (xrow is an LDS address holding the
// row's K values from K = xk0 on); its fragments are read at their MFMA
// instead of being held in registers.  after_issue() runs once every global load of the wave has
// been issued, before the first use of any.
// ER: accumulator elements e < ER get their group corrections (row 4q + e of
// lane group q).  ER = 1 serves a single-row tile (only row 0 is stored);
// rows past the tile read a valid row, so the extra work of ER = 4 on them is
// finite and never stored.
// FP4: the codes are e2m1 in standard order (group 32, no zero point) and the
// scales bf16 powers of two; each MFMA operand is the exact bf16 e2m1 x scale
// from the fp4 -> bf16 conversion, so the MFMA accumulates into acc directly.
template <int BITS, bool ZP, int GROUP, int T, int KR, bool XL = false, int ER = 4,
          typename Hook = NoHook, bool FP4 = false>
__device__ __forceinline__ void a16_wave(const GemmArgs &a, const uint8_t *wexp,
                                         const uint16_t *xrow, int nt0, int kb0, f32x4 (&acc)[T],
                                         Hook after_issue = Hook(), int xk0 = 0) {
  static_assert(!FP4 || (BITS == 4 && !ZP && GROUP == 32), "fp4 codes: 4-bit, group 32, no zero point");
  constexpr int LB = BITS == 4 ? 16 : 12;    // packed bytes per lane per block
  constexpr int BB = 64 * LB;                // packed bytes per block
  constexpr int JPG = GROUP / 32;            // MFMAs per K-group
  constexpr int GPB = 128 / GROUP;           // K-groups per block
  constexpr float MAG = BITS == 4 ? 16.f : 8.f;
  constexpr int ZSYM = BITS == 4 ? 8 : 4;
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4, r16 = lane & 15;
  const int kbs = a.k_blocks, gp = a.groups_padded;

  // Every load of the wave is issued before the first wait, so one memory
  // round trip covers the whole item: scales and zero points first (every
  // block's correction needs them), then the activation fragments, then the
  // weight blocks in consumption order, so the compiler's progressive waits
  // let block kb's work start while later blocks are still arriving.  Loads
  // are unconditional: rows past the tile read a valid row (their outputs are
  // never stored), K past the end reads k = 0 (those K-groups carry scale 0),
  // and out-of-range n-tiles or k-blocks read a clamped block (n-tiles past N
  // are never stored; k-blocks past K have scale 0).
  // 1. per-group scales (bf16 pairs) and zero points (nibbles) of this lane's
  //    column for groups g0 .. g0 + NG - 1; g0 is a multiple of NG and the
  //    padded group count a multiple of 32, so no vector load crosses a row
  constexpr int NG = KR * GPB;
  constexpr int SW = (NG + 1) / 2;           // dwords of scales
  constexpr int ZW = ZP ? (NG + 7) / 8 : 1;  // dwords of zero points
  const int g0 = kb0 * GPB;
  const int gl = min(g0, gp - NG);           // clamped (a wave past K reads padding)
  uint32_t sw[T][SW], zw[T][ZW];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int n = min(nt0 + t, a.n_tiles - 1) * 16 + r16;
    const uint8_t *sp = wexp + a.scales_offset + ((uint64_t)n * gp + gl) * 2;
    if constexpr (NG == 1) {
      sw[t][0] = (uint32_t)*(const uint16_t *)sp;
    } else if constexpr (NG == 2) {
      sw[t][0] = *(const uint32_t *)sp;
    } else if constexpr (NG == 4) {
      const uint2 v = *(const uint2 *)sp;
      sw[t][0] = v.x; sw[t][1] = v.y;
    } else {
#pragma unroll
      for (int c = 0; c < SW / 4; ++c) {
        const u32x4 v = *(const u32x4 *)(sp + 16 * c);
        sw[t][4 * c] = v.x; sw[t][4 * c + 1] = v.y; sw[t][4 * c + 2] = v.z; sw[t][4 * c + 3] = v.w;
      }
    }
    if constexpr (ZP) {
      const uint32_t *zp = (const uint32_t *)(wexp + a.zeros_offset) + (uint64_t)n * (gp >> 3) + (gl >> 3);
#pragma unroll
      for (int c = 0; c < ZW; ++c) zw[t][c] = zp[c];
    } else {
      zw[t][0] = 0u;
    }
  }
  // 2. activation fragments, A operand: row r16, k = 128 kb + 32 j + 8 q .. +7
  u32x4 xf[XL ? 1 : KR][4];
  auto xfrag = [&](int kb, int j) -> u32x4 {
    const int k = (kb0 + kb) * 128 + 32 * j + 8 * q;
    if constexpr (XL) return *(const u32x4 *)(xrow + (k - xk0));  // LDS row zero-padded past K
    return *(const u32x4 *)(xrow + (k < a.k ? k : 0));
  };
  if constexpr (!XL) {
#pragma unroll
    for (int kb = 0; kb < KR; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j) xf[kb][j] = xfrag(kb, j);
  }
  // 3. weight slices, in the order the MFMAs consume them.  XL (the decode
  //    kernel): DP blocks go out first and block kb + DP right after block
  //    kb's work, so the wave computes while the CU's memory queue drains
  //    (a wave that issued all its loads up front sat blocked on the full
  //    queue until its last load went out); otherwise every block at once.
  constexpr int DP = a16_pipe_depth<XL, KR>();
  u32x4 wq[T][KR];
  auto issue = [&](int kb) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int nt = min(nt0 + t, a.n_tiles - 1), b = min(kb0 + kb, kbs - 1);
      const uint8_t *p = wexp + ((uint64_t)nt * kbs + b) * BB + lane * LB;
      if constexpr (BITS == 4) {
        wq[t][kb] = load_stream((const u32x4 *)p);
      } else {
        const uint32_t *p32 = (const uint32_t *)p;
        wq[t][kb] = u32x4{load_stream(p32), load_stream(p32 + 1), load_stream(p32 + 2), 0u};
      }
    }
  };
#pragma unroll
  for (int kb = 0; kb < DP; ++kb) issue(kb);
  // keep these loads above this point (the hook's waits count them)
  __builtin_amdgcn_sched_barrier(0);
  after_issue();
  if (kb0 >= kbs) return;  // wave-uniform: a wave entirely past K adds nothing
  // One row in LDS (ER = 1): the group row sums of the wave's NG groups come
  // from the LDS copy once, lane l summing values 16 l .. 16 l + 15 of the
  // wave's K range with dot products against ones, GROUP / 16 lanes per group
  // combined by butterfly; group i's sum is then read from lane i * GROUP / 16
  // into a scalar.  (With more rows the MFMA against all-ones gives the sums
  // of 16 rows at once.)
  constexpr bool XS_LDS = XL && ER == 1 && !FP4;
  static_assert(!XS_LDS || KR <= 8, "one row: a wave's K range spans at most its 64 lanes x 16 values");
  float xsum_lane = 0.f;
  if constexpr (XS_LDS) {
    // the wave's KR blocks are KR * 8 lanes' worth (KR * 128 values)
    if (KR == 8 || lane < KR * 8) {
      const u32x4 *xp = (const u32x4 *)(xrow + (kb0 * 128 - xk0) + 16 * lane);
      const u32x4 v0 = xp[0], v1 = xp[1];
      const bf16x2 one2 = __builtin_bit_cast(bf16x2, 0x3F803F80u);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // (element copied out first: a bit cast of a vector element lvalue
        // reads element 0)
        const uint32_t d0 = v0[e], d1 = v1[e];
        xsum_lane = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, d0), one2, xsum_lane, false);
        xsum_lane = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, d1), one2, xsum_lane, false);
      }
    }
#pragma unroll
    for (int off = 1; off < GROUP / 16; off <<= 1) xsum_lane += __shfl_xor(xsum_lane, off);
  }
  // scale s and zero point z of group g0 + i -> (MAG * s, -(MAG + z) * s)
  auto group_consts = [&](int t, int i, float &c1, float &c2) {
    const float s = bf16_bits_to_f32((sw[t][i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
    int z = ZSYM;
    if constexpr (ZP) z = (int)((zw[t][i >> 3] >> (4 * ((g0 + i) & 7))) & 15u);
    c1 = MAG * s;
    c2 = -(MAG + (float)z) * s;
  };

  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const uint32_t umask = sgpr_const(BITS == 4 ? 0x00780078u : 0x00700070u);
  const uint32_t umagic = vgpr_const(0x3F803F80u);
  f32x4 c[T];
#pragma unroll
  for (int t = 0; t < T; ++t) c[t] = acc[t];
#pragma unroll
  for (int kb = 0; kb < KR; ++kb) {
    u32x4 xk[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) xk[j] = XL ? xfrag(kb, j) : xf[XL ? 0 : kb][j];
    // the next block's loads go out once this block's operands are read
    auto issue_next = [&]() {
      if constexpr (DP < KR) {
        if (kb + DP < KR) {
          __builtin_amdgcn_sched_barrier(0);
          issue(kb + DP);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    if constexpr (FP4) {
      // one K-group per MFMA: operand = e2m1 x 2^(e - 127), exact in bf16.
      // The conversion takes its scale as a power of two (a 0.0 scale acts as
      // 2^-127), so a padding group's zero scale does not zero the operand:
      // k-blocks past K (clamped re-reads of the last block, against
      // activations clamped to k = 0) are skipped instead (wave-uniform);
      // padding inside the last block holds code 0, which converts to 0.
      if (kb0 + kb >= kbs) {
        issue_next();
        continue;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = kb * GPB + j;
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const float s = bf16_bits_to_f32((sw[t][i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
          const uint32_t wd = wq[t][kb][j];
          const u32x4 b = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, s, 0)),
                           __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, s, 1)),
                           __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, s, 2)),
                           __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, s, 3))};
          c[t] = mfma_bf16(xk[j], b, c[t]);
        }
      }
      issue_next();
      continue;
    }
#pragma unroll
    for (int gi = 0; gi < GPB; ++gi) {
      const int i = kb * GPB + gi;
      // 4. group row sums of X: from the lanes' dot products (one row), or
      //    on the matrix core (B = all ones)
      f32x4 xs = {0.f, 0.f, 0.f, 0.f};
      if constexpr (XS_LDS) {
        xs[0] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, xsum_lane),
                                                                    i * (GROUP / 16)));
      } else {
#pragma unroll
        for (int j = gi * JPG; j < (gi + 1) * JPG; ++j) xs = mfma_bf16(xk[j], ones, xs);
      }
      // 5. dequantize + MFMA + per-group scaling
#pragma unroll
      for (int t = 0; t < T; ++t) {
        f32x4 g = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = gi * JPG; j < (gi + 1) * JPG; ++j)
          g = mfma_bf16(xk[j], unpack_br<BITS>(wq[t][kb], j, umask, umagic), g);
        float c1, c2;
        group_consts(t, i, c1, c2);
#pragma unroll
        for (int e = 0; e < ER; ++e) {
          c[t][e] = __builtin_fmaf(xs[e], c2, c[t][e]);
          c[t][e] = __builtin_fmaf(g[e], c1, c[t][e]);
        }
      }
    }
    issue_next();
  }
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = c[t];
}

// Four e2m1 codes (the low 16 bits of h, code i in bits 4i .. 4i + 3) -> the
// four e4m3 bytes of the same values: every e2m1 magnitude (0, 0.5, 1, 1.5, 2,
// 3, 4, 6) is an e4m3 value, looked up in an 8-byte table with v_perm_b32
// (selector bytes 0-3 pick bytes of the second operand, 4-7 of the first);
// the sign moves from bit 3 to bit 7.
__device__ __forceinline__ uint32_t e2m1x4_to_e4m3(uint32_t h) {
  const uint32_t n = (h & 0xFu) | ((h & 0xF0u) << 4) | ((h & 0xF00u) << 8) | ((h & 0xF000u) << 12);
  const uint32_t mag = __builtin_amdgcn_perm(0x4C484440u, 0x3C383000u, n & 0x07070707u);
  return mag | ((n & 0x08080808u) << 4);
}

// MXFP4 weights x MXFP8 activations: one scaled MFMA per 16x128 block.  A4:
// the activation rows hold e2m1 codes (two per byte, xrow in bytes of those
// rows); each fragment is widened to e4m3 in registers (same values, same
// block scales).
// RS: per-token FP8 activations (e4m3 with one fp32 scale per row, applied
// to the output row): the A scales are 2^0.
template <int T, int KR, typename Hook = NoHook, bool A4 = false, bool RS = false>
__device__ __forceinline__ void mx_wave(const GemmArgs &a, const uint8_t *wexp,
                                        const uint8_t *xrow, const uint8_t *xsrow, int nt0, int kb0,
                                        f32x4 (&acc)[T], Hook after_issue = Hook()) {
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4, r16 = lane & 15;
  const int kbs = a.k_blocks;
  // A operand (8-bit) of v_mfma_scale_f32_16x16x128_f8f6f4: lane group q holds
  // K 16q..16q+15 in VGPRs 0-3 and K 64+16q..64+16q+15 in VGPRs 4-7 of the
  // 128-K step, while its scale byte names K-block q (32q..32q+31).  The 4-bit
  // B operand holds K 32q..32q+31 contiguously, as packed.  Loads are
  // unconditional with clamped addresses (see a16_wave); a chunk past K reads
  // k = 0 and is zeroed, since e8m0 has no zero scale.
  i32x8 xf[KR];
  int xsc[KR];
#pragma unroll
  for (int kb = 0; kb < KR; ++kb) {
    const int k0 = (kb0 + kb) * 128;
    const int klo = k0 + 16 * q, khi = k0 + 64 + 16 * q;
    u32x4 lo, hi;
    if constexpr (A4) {
      const uint2 l4 = *(const uint2 *)(xrow + ((klo < a.k ? klo : 0) >> 1));
      const uint2 h4 = *(const uint2 *)(xrow + ((khi < a.k ? khi : 0) >> 1));
      lo = u32x4{e2m1x4_to_e4m3(l4.x), e2m1x4_to_e4m3(l4.x >> 16), e2m1x4_to_e4m3(l4.y),
                 e2m1x4_to_e4m3(l4.y >> 16)};
      hi = u32x4{e2m1x4_to_e4m3(h4.x), e2m1x4_to_e4m3(h4.x >> 16), e2m1x4_to_e4m3(h4.y),
                 e2m1x4_to_e4m3(h4.y >> 16)};
    } else {
      lo = *(const u32x4 *)(xrow + (klo < a.k ? klo : 0));
      hi = *(const u32x4 *)(xrow + (khi < a.k ? khi : 0));
    }
    const int kb32 = (k0 >> 5) + q;
    const int sc = RS ? 127 : xsrow[kb32 < (a.k >> 5) ? kb32 : 0];
    const bool lo_ok = klo < a.k, hi_ok = khi < a.k;
    xf[kb] = i32x8{(int)(lo_ok ? lo.x : 0u), (int)(lo_ok ? lo.y : 0u), (int)(lo_ok ? lo.z : 0u),
                   (int)(lo_ok ? lo.w : 0u), (int)(hi_ok ? hi.x : 0u), (int)(hi_ok ? hi.y : 0u),
                   (int)(hi_ok ? hi.z : 0u), (int)(hi_ok ? hi.w : 0u)};
    xsc[kb] = sc;
  }
  u32x4 wq[T][KR];
#pragma unroll
  for (int kb = 0; kb < KR; ++kb)
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int nt = min(nt0 + t, a.n_tiles - 1), b = min(kb0 + kb, kbs - 1);
      wq[t][kb] = load_stream((const u32x4 *)(wexp + ((uint64_t)nt * kbs + b) * 1024 + lane * 16));
    }
  const uint8_t *sbase = wexp + a.scales_offset;
  int wsc[T][KR];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int n = min(nt0 + t, a.n_tiles - 1) * 16 + r16;
#pragma unroll
    for (int kb = 0; kb < KR; ++kb) {
      const int b = min(kb0 + kb, kbs - 1);
      wsc[t][kb] = sbase[((uint64_t)(n >> 4) * (a.kb_pad >> 2) + (b >> 2)) * 256 + ((n & 15) * 4 + q) * 4 + (b & 3)];
    }
  }
  // keep every load above this point: the wave waits once for all of them
  __builtin_amdgcn_sched_barrier(0);
  after_issue();
#pragma unroll
  for (int t = 0; t < T; ++t) {
    f32x4 c = acc[t];
#pragma unroll
    for (int kb = 0; kb < KR; ++kb) {
      const bool ok = kb0 + kb < kbs;  // wave-uniform
      const u32x4 w = wq[t][kb];
      const i32x8 bw = {(int)(ok ? w.x : 0u), (int)(ok ? w.y : 0u), (int)(ok ? w.z : 0u),
                        (int)(ok ? w.w : 0u), 0, 0, 0, 0};
      // cbsz = 0: A is fp8 e4m3; blgp = 4: B is fp4 e2m1
      c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(xf[kb], bw, c, 0, 4, 0, xsc[kb], 0,
                                                            wsc[t][kb]);
    }
    acc[t] = c;
  }
}

// bf16 MFMA operand j (k = 32 j + 8 q + e, e = 0..7) of a lane's packed
// slice w (BITS dwords) for the formats of a16x_wave.  Integer codes u:
//   2-bit: dword j / 2, code e in slot 4 (j % 2) + e / 2 + 8 (e % 2) (2-bit
//          slots), so a pair (e = 2i, 2i + 1) sits 16 bits apart and one shift
//          + and/or puts it at mantissa bits 5..6: bf16 1 + u / 4;
//   1-bit: one dword, code e in bit 4 j + e / 2 + 16 (e % 2), moved to
//          mantissa bit 6: bf16 1 + u / 2;
//   8-bit: bytes 8 j .. 8 j + 7 in order; each byte becomes an exact fp32
//          (v_cvt_f32_ubyte) whose top half is the exact bf16 of u, paired
//          with v_perm.
// e4m3 (FMT 13): the bytes as for 8-bit, converted by the fp8 -> bf16 pair
// conversion with unit scale (every e4m3 value is a bf16 value).
template <int FMT>
__device__ __forceinline__ u32x4 unpack_x(const uint32_t *w, int j) {
  constexpr int BITS = FmtTraits<FMT>::BITS;
  u32x4 r;
  if constexpr (FMT == 13) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t d = w[2 * j + h];
      r[2 * h] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d, 1.f, false));
      r[2 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d, 1.f, true));
    }
  } else if constexpr (BITS == 8) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t d = w[2 * j + h];
      const float f0 = (float)(d & 255u), f1 = (float)((d >> 8) & 255u);
      const float f2 = (float)((d >> 16) & 255u), f3 = (float)(d >> 24);
      r[2 * h] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
      r[2 * h + 1] = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
    }
  } else if constexpr (BITS == 2) {
    const uint32_t d = w[j >> 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sh = 2 * (4 * (j & 1) + i) - 5;
      const uint32_t t = sh >= 0 ? d >> sh : d << -sh;
      r[i] = (t & 0x00600060u) | 0x3F803F80u;
    }
  } else {
    const uint32_t d = w[0];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sh = 4 * j + i - 6;
      const uint32_t t = sh >= 0 ? d >> sh : d << -sh;
      r[i] = (t & 0x00400040u) | 0x3F803F80u;
    }
  }
  return r;
}

// The 1-, 2- and 8-bit integer formats and e4m3 weights with bf16
// activations (FMT 7 .. 13; the announcement's "WnA16" section: integer and
// floating-point weights of every width on one dequantize-and-compute path).
// The structure of a16_wave: every load of the wave issued before the first
// wait (scales, zero points, activation fragments, weight slices), then per
// K-group bf16 MFMA partials scaled in fp32.  An integer operand is v = OFF +
// u / MAG (OFF = 1 with MAG = 4 / 2 for 2- / 1-bit codes, OFF = 0 with MAG =
// 1 for 8-bit codes), so per group
//   sum x (u - z) s = MAG s * sum x v - (MAG OFF + z) s * sum x,
// z = 2^(b-1) for the signed formats; sum x comes from an MFMA against all
// ones.  e4m3 operands are the weights' exact values: sum x w s, no correction.
template <int FMT, int GROUP, int T, int KR, bool XL = false, int ER = 4, typename Hook = NoHook>
__device__ __forceinline__ void a16x_wave(const GemmArgs &a, const uint8_t *wexp, const uint16_t *xrow,
                                          int nt0, int kb0, f32x4 (&acc)[T], Hook after_issue = Hook(),
                                          int xk0 = 0) {
  using Fm = FmtTraits<FMT>;
  constexpr int BITS = Fm::BITS;
  constexpr bool ZP = Fm::ZP;
  constexpr bool E4 = FMT == 13;
  constexpr int NV = BITS;                  // packed dwords per lane per block
  constexpr int BB = 256 * BITS;            // packed bytes per block
  constexpr int JPG = GROUP / 32, GPB = 128 / GROUP;
  constexpr float MAG = BITS == 8 ? 1.f : (float)(1 << BITS);
  constexpr float OFF = BITS == 8 ? 0.f : 1.f;
  constexpr int ZSYM = 1 << (BITS - 1);
  constexpr int ZPW = BITS == 8 ? 4 : 8;    // zero points per dword (bytes or nibbles)
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4, r16 = lane & 15;
  const int kbs = a.k_blocks, gp = a.groups_padded;

  // 1. scales (bf16 pairs) and zero points of groups g0 .. g0 + NG - 1
  //    (NG and ZPW are powers of two and g0 a multiple of NG, so the run never
  //    straddles a zero-point word it does not start)
  constexpr int NG = KR * GPB;
  constexpr int SW = (NG + 1) / 2;
  constexpr int ZW = ZP ? (NG + ZPW - 1) / ZPW : 1;
  const int g0 = kb0 * GPB;
  const int gl = min(g0, gp - NG);
  uint32_t sw[T][SW], zw[T][ZW];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int n = min(nt0 + t, a.n_tiles - 1) * 16 + r16;
    const uint8_t *sp = wexp + a.scales_offset + ((uint64_t)n * gp + gl) * 2;
    if constexpr (NG == 1) {
      sw[t][0] = (uint32_t)*(const uint16_t *)sp;
    } else if constexpr (NG == 2) {
      sw[t][0] = *(const uint32_t *)sp;
    } else if constexpr (NG == 4) {
      const uint2 v = *(const uint2 *)sp;
      sw[t][0] = v.x; sw[t][1] = v.y;
    } else {
#pragma unroll
      for (int c = 0; c < SW / 4; ++c) {
        const u32x4 v = *(const u32x4 *)(sp + 16 * c);
        sw[t][4 * c] = v.x; sw[t][4 * c + 1] = v.y; sw[t][4 * c + 2] = v.z; sw[t][4 * c + 3] = v.w;
      }
    }
    if constexpr (ZP) {
      const uint32_t *zp = (const uint32_t *)(wexp + a.zeros_offset) + (uint64_t)n * (gp / ZPW) + gl / ZPW;
#pragma unroll
      for (int c = 0; c < ZW; ++c) zw[t][c] = zp[c];
    } else {
      zw[t][0] = 0u;
    }
  }
  // 2. activation fragments (A operand: row r16, k = 128 kb + 32 j + 8 q .. +7)
  u32x4 xf[XL ? 1 : KR][4];
  auto xfrag = [&](int kb, int j) -> u32x4 {
    const int k = (kb0 + kb) * 128 + 32 * j + 8 * q;
    if constexpr (XL) return *(const u32x4 *)(xrow + (k - xk0));
    return *(const u32x4 *)(xrow + (k < a.k ? k : 0));
  };
  if constexpr (!XL) {
#pragma unroll
    for (int kb = 0; kb < KR; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j) xf[kb][j] = xfrag(kb, j);
  }
  // 3. weight slices (BITS dwords per lane and block), in consumption order
  uint32_t wq[T][KR][NV];
#pragma unroll
  for (int kb = 0; kb < KR; ++kb)
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int nt = min(nt0 + t, a.n_tiles - 1), b = min(kb0 + kb, kbs - 1);
      const uint8_t *p = wexp + ((uint64_t)nt * kbs + b) * BB + lane * (4 * NV);
      if constexpr (NV == 8) {
        const u32x4 v0 = load_stream((const u32x4 *)p), v1 = load_stream((const u32x4 *)p + 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          wq[t][kb][i] = v0[i];
          wq[t][kb][4 + i] = v1[i];
        }
      } else if constexpr (NV == 2) {
        typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
        const u32x2 v = load_stream((const u32x2 *)p);
        wq[t][kb][0] = v.x;
        wq[t][kb][1] = v.y;
      } else {
        wq[t][kb][0] = load_stream((const uint32_t *)p);
      }
    }
  __builtin_amdgcn_sched_barrier(0);
  after_issue();
  if (kb0 >= kbs) return;  // wave-uniform

  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  f32x4 c[T];
#pragma unroll
  for (int t = 0; t < T; ++t) c[t] = acc[t];
#pragma unroll
  for (int kb = 0; kb < KR; ++kb) {
    u32x4 xk[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) xk[j] = XL ? xfrag(kb, j) : xf[XL ? 0 : kb][j];
#pragma unroll
    for (int gi = 0; gi < GPB; ++gi) {
      const int i = kb * GPB + gi;
      f32x4 xs = {0.f, 0.f, 0.f, 0.f};
      if constexpr (!E4) {
#pragma unroll
        for (int j = gi * JPG; j < (gi + 1) * JPG; ++j) xs = mfma_bf16(xk[j], ones, xs);
      }
#pragma unroll
      for (int t = 0; t < T; ++t) {
        f32x4 g = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = gi * JPG; j < (gi + 1) * JPG; ++j) g = mfma_bf16(xk[j], unpack_x<FMT>(wq[t][kb], j), g);
        const float s = bf16_bits_to_f32((sw[t][i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
        if constexpr (E4) {
#pragma unroll
          for (int e = 0; e < ER; ++e) c[t][e] = __builtin_fmaf(g[e], s, c[t][e]);
        } else {
          int z = ZSYM;
          if constexpr (ZP) {
            constexpr int ZB = 32 / ZPW;  // bits per zero point
            z = (int)((zw[t][i / ZPW] >> (ZB * ((g0 + i) % ZPW))) & ((1u << ZB) - 1u));
          }
          const float c1 = MAG * s, c2 = -(MAG * OFF + (float)z) * s;
#pragma unroll
          for (int e = 0; e < ER; ++e) {
            c[t][e] = __builtin_fmaf(xs[e], c2, c[t][e]);
            c[t][e] = __builtin_fmaf(g[e], c1, c[t][e]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = c[t];
}

// W8A8 FP8 with block scales (FMT 15; the announcement's "W8A8 / W4A8 /
// W4A4" section).  Per 128-K step one scaled MFMA with unit scales takes the
// n-tile's 16 weight rows as its A operand and the 16 activation rows as B
// (both e4m3, 32 bytes per lane: K 16 q .. 16 q + 15 and 64 + 16 q .. + 15 of
// the step, the f8f6f4 8-bit operand layout), so lane (q, r16) receives the
// partial sums of columns 4 q + e and activation row r16; the step's partial
// is scaled by sa[row][kb] * sw[n-tile][kb] (the weight scale is shared by
// the 128 rows of W of its block, so one per n-tile) and added to acc in fp32.
template <int T, int KR, typename Hook = NoHook>
__device__ __forceinline__ void f8_wave(const GemmArgs &a, const uint8_t *wexp, const uint8_t *xrow,
                                        const float *xsrow, int nt0, int kb0, f32x4 (&acc)[T],
                                        Hook after_issue = Hook()) {
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4;
  const int kbs = a.k_blocks;
  // activations (B operand) and their step scales; K % 128 == 0, steps past
  // K read step 0 and are dropped below (wave-uniform)
  i32x8 xf[KR];
  float xs[KR];
#pragma unroll
  for (int kb = 0; kb < KR; ++kb) {
    const int b = kb0 + kb < kbs ? kb0 + kb : 0;
    const u32x4 lo = *(const u32x4 *)(xrow + b * 128 + 16 * q);
    const u32x4 hi = *(const u32x4 *)(xrow + b * 128 + 64 + 16 * q);
    xf[kb] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    xs[kb] = xsrow[b];
  }
  // weights (A operand): 2 KB per 16 x 128 block, 32 bytes per lane
  u32x4 wq[T][KR][2];
  float ws[T][KR];
  const float *wsc = (const float *)(wexp + a.scales_offset);
#pragma unroll
  for (int kb = 0; kb < KR; ++kb)
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int nt = min(nt0 + t, a.n_tiles - 1), b = min(kb0 + kb, kbs - 1);
      const u32x4 *p = (const u32x4 *)(wexp + ((uint64_t)nt * kbs + b) * 2048 + lane * 32);
      wq[t][kb][0] = load_stream(p);
      wq[t][kb][1] = load_stream(p + 1);
      ws[t][kb] = wsc[(uint64_t)nt * a.kb_pad + b];
    }
  __builtin_amdgcn_sched_barrier(0);
  after_issue();
#pragma unroll
  for (int t = 0; t < T; ++t) {
    f32x4 c = acc[t];
#pragma unroll
    for (int kb = 0; kb < KR; ++kb) {
      if (kb0 + kb >= kbs) continue;  // wave-uniform
      const u32x4 w0 = wq[t][kb][0], w1 = wq[t][kb][1];
      const i32x8 wf = {(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w, (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
      // cbsz = blgp = 0: both operands e4m3; scale codes 127 = 2^0
      const f32x4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf, xf[kb], f32x4{0.f, 0.f, 0.f, 0.f}, 0,
                                                                        0, 0, 127, 0, 127);
      const float sc = xs[kb] * ws[t][kb];
#pragma unroll
      for (int e = 0; e < 4; ++e) c[e] = __builtin_fmaf(p[e], sc, c[e]);
    }
    acc[t] = c;
  }
}

// Waits 16 wait states with the accumulators as operands, so the wait sits
// between the MFMAs that write them and every later read.
__device__ __forceinline__ void mfma_drain(f32x4 (&acc)[1]) { asm volatile("s_nop 7\n\ts_nop 7" : "+v"(acc[0])); }
__device__ __forceinline__ void mfma_drain(f32x4 (&acc)[2]) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(acc[0]), "+v"(acc[1]));
}
__device__ __forceinline__ void mfma_drain(f32x4 (&acc)[4]) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]));
}

// ---------------------------------------------------------------------------
// the kernel: a loop over work items (one item per workgroup for dense
// launches; a persistent grid for MoE)
// ---------------------------------------------------------------------------

template <int FMT, int GROUP, int T, int KR>
__global__ __launch_bounds__(kMaxWaves * 64) void skinny_kernel(GemmArgs a, int moe,
                                                                int64_t total_items_dense) {
  // FMT: see FmtTraits
  using Fm = FmtTraits<FMT>;
  extern __shared__ float red[];  // [waves][T][256]: sized by the launcher
  __shared__ int prefix[kMaxExperts + 1];
  __shared__ int last_flag;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  const int r16 = lane & 15;
  const int n_blocks = (a.n_tiles + T - 1) / T;

  int total_tiles = 0;
  int64_t total_items = total_items_dense;
  if (moe) {
    total_tiles = moe_tile_prefix(a.offsets, a.num_experts, a.moe_min_rows, prefix);
    total_items = (int64_t)total_tiles * n_blocks;
  }

  // The item's activation rows (for MoE, pair ids loaded from the sorted list)
  // are resolved one item ahead, while the previous item's loads are in
  // flight, so an item's loads never wait on that dependent round trip.
  // rows past the tile read the tile's first row: their outputs are never stored
  int nxt_xr = 0;  // rows < 2^30
  if ((int64_t)blockIdx.x < total_items) {
    const Item first = decode_item(a, moe != 0, blockIdx.x, n_blocks, total_tiles, prefix);
    nxt_xr = (int)x_row_of(a, moe != 0, first, r16 < first.rows ? r16 : 0);
  }
  // K blocks one pass of the launch covers; beyond that every workgroup
  // loops over K (pass p, split s, wave w takes blocks from ((p * splits + s)
  // * waves + w) * KR), accumulating in registers
  const int span = nwaves * KR * a.splits;
  const int passes = (a.k_blocks + span - 1) / span;
  for (int64_t item = blockIdx.x; item < total_items; item += gridDim.x) {
    const Item it = decode_item(a, moe != 0, item, n_blocks, total_tiles, prefix);
    const int64_t xr = nxt_xr;
    const uint8_t *wexp = a.wbase + (uint64_t)it.expert * a.expert_stride;
    const int nt0 = it.nb * T;
    auto prefetch_next = [&]() {
      const int64_t next = item + gridDim.x;
      if (next < total_items) {  // workgroup-uniform
        const Item n_it = decode_item(a, moe != 0, next, n_blocks, total_tiles, prefix);
        nxt_xr = (int)x_row_of(a, moe != 0, n_it, r16 < n_it.rows ? r16 : 0);
      }
    };

    f32x4 acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = {0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < passes; ++p) {
      const int kb0 = ((p * a.splits + it.split) * nwaves + wave) * KR;
      // the next item's rows are resolved once, behind the first pass's loads
      auto hook = [&]() {
        if (p == 0) prefetch_next();
      };
      if (kb0 < a.k_blocks) {
        if constexpr (Fm::MXW) {
          const uint8_t *xrow = (const uint8_t *)a.x + xr * a.ldx;
          const uint8_t *xsrow = a.x_scales + xr * (int64_t)(a.k >> 5);
          mx_wave<T, KR, decltype(hook), FMT == 6, FMT == 14>(a, wexp, xrow, xsrow, nt0, kb0, acc, hook);
        } else if constexpr (Fm::F8) {
          const uint8_t *xrow = (const uint8_t *)a.x + xr * a.ldx;
          const float *xsrow = (const float *)a.x_scales + xr * (int64_t)a.k_blocks;
          f8_wave<T, KR, decltype(hook)>(a, wexp, xrow, xsrow, nt0, kb0, acc, hook);
        } else if constexpr (Fm::EXT) {
          const uint16_t *xrow = (const uint16_t *)a.x + xr * a.ldx;
          a16x_wave<FMT, GROUP, T, KR, false, 4, decltype(hook)>(a, wexp, xrow, nt0, kb0, acc, hook);
        } else {
          const uint16_t *xrow = (const uint16_t *)a.x + xr * a.ldx;
          constexpr int BITS = Fm::BITS;
          constexpr bool ZP = Fm::ZP;
          a16_wave<BITS, ZP, GROUP, T, KR, false, 4, decltype(hook), FMT == 5>(a, wexp, xrow, nt0, kb0, acc, hook);
        }
      } else {
        hook();
      }
    }

    // The last MFMA of the K loop may still be writing acc: the compiler
    // does not count its write-back latency across the loop's exit, so the
    // wait is explicit (16 wait states; the MFMAs here need at most 12)
    mfma_drain(acc);

    // reduce the K-split waves of the workgroup in a fixed order
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[(wave * T + t) * 256 + e * 64 + lane] = acc[t][e];
    __syncthreads();

    // tile element idx = (t, e, lane): row 4 (lane / 16) + e and column lane
    // % 16 of n-tile t, or (SWAP) row lane % 16 and column 4 (lane / 16) + e
    auto out_row = [](int idx) { return Fm::SWAP ? (idx & 15) : 4 * ((idx & 63) >> 4) + ((idx >> 6) & 3); };
    auto out_col = [](int idx) { return Fm::SWAP ? 4 * ((idx & 63) >> 4) + ((idx >> 6) & 3) : (idx & 15); };
    const bool split_k = a.splits > 1;
    for (int idx = threadIdx.x; idx < T * 256; idx += blockDim.x) {
      float s = 0.f;
      for (int w = 0; w < nwaves; ++w) s += red[w * T * 256 + idx];
      red[idx] = s;  // wave 0's slot now holds the workgroup sum (same thread reads it)
    }
    if (split_k) {
      // Write this split's partial tile (valid rows only), then the last
      // workgroup of the tile sums the splits in split order and resets the
      // tile's counter to zero for the next call.  Partials move with
      // agent-scope atomic stores/loads (write-through, coherent across the
      // XCD L2s), so no L2 write-back or invalidate fence is needed: the stores
      // are complete (vmcnt = 0) before the counter add that publishes them,
      // and the last workgroup's loads are issued after that add returns.
      const int64_t m_tiles = (a.m + 15) / 16;
      const int64_t tile = (int64_t)(it.row0 / 16) * n_blocks + it.nb;
      float *part = a.partials + ((int64_t)it.split * m_tiles * n_blocks + tile) * (T * 256);
      for (int idx = threadIdx.x; idx < T * 256; idx += blockDim.x)
        if (out_row(idx) < it.rows)
          __hip_atomic_store(part + idx, red[idx], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(a.counters + tile, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        last_flag = (prev == (uint32_t)(a.splits - 1));
      }
      __syncthreads();
      if (!last_flag) continue;  // uniform across the workgroup
      for (int idx = threadIdx.x; idx < T * 256; idx += blockDim.x) {
        float s = 0.f;
        if (out_row(idx) < it.rows)
          s = sum_partials(a.partials + tile * (T * 256) + idx, m_tiles * n_blocks * (T * 256), a.splits);
        red[idx] = s;
      }
      if (threadIdx.x == 0)
        __hip_atomic_store(a.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // output stage (per-token FP8: times the activation row's scale)
    for (int idx = threadIdx.x; idx < T * 256; idx += blockDim.x) {
      const int t = idx >> 8;
      const int r = out_row(idx);
      const int col = (nt0 + t) * 16 + out_col(idx);
      if (r < it.rows && col < a.n && nt0 + t < a.n_tiles) {
        float v = red[idx];
        if constexpr (Fm::ROW_SCALE) v *= ((const float *)a.x_scales)[x_row_of(a, moe != 0, it, r)];
        store_out(a.y, a.ldy, a.otype, y_row_of(a, moe != 0, it, r), col, v);
      }
    }
    __syncthreads();  // red[] and last_flag are reused by the next item
  }
}

// ---------------------------------------------------------------------------
// dense decode (M <= 16 rows, integer formats): the workgroup covers all of K
// (or 1 / splits of it)
// ---------------------------------------------------------------------------
//
// The skinny kernel keeps every wave's activation fragments in registers (16
// VGPRs per 128-K block), which caps a 1024-thread workgroup at 16 waves x 2
// blocks and forces a cross-workgroup K split for long K.  Here the rows are
// copied once into LDS with global_load_lds, issued before the weight loads
// so that a partial wait covers them while the weights are still in flight;
// waves read fragments from LDS at their MFMA.  KR = 8 blocks per wave then
// fits, 16 waves cover K = 16384 in one workgroup, and the output needs only
// the in-workgroup reduction (of the valid rows).  One workgroup per T
// n-tiles.  Requires K % 512 == 0 (each 64-lane copy stays within a row) and
// rows * (2K + 16) bytes of LDS.
//
// Long K with few n-tiles (one 14-wave workgroup per CU) leaves the
// dequantization of the last-arriving blocks exposed; there a launch with
// gridDim.y = splits > 1 gives each workgroup 1 / splits of K (its rows' K
// range in LDS) and combines the splits as the skinny kernel does: fp32
// partial tiles and a per-tile arrival counter, the last arriver sums the
// splits in order and resets the counter.  Then W * KR * 128 must be a
// multiple of 512 and the splits must all start inside K.
template <int FMT, int GROUP, int T, int KR, int ER>
__global__ __launch_bounds__(kMaxWaves * 64) void decode_kernel(GemmArgs a) {
  constexpr int BITS = FmtTraits<FMT>::BITS;  // FMT 5: MXFP4 codes x bf16
  constexpr bool ZP = FmtTraits<FMT>::ZP;
  extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  const int rows = ER == 1 ? 1 : a.m;         // 1..16 (ER = 1: a single row)
  const int kspan = nwaves * KR * 128;        // K covered by the waves of one split
  const int xpitch = kspan * 2 + 16;          // bytes per row in LDS (padded: bank spread)
  // [waves][T][rows][16]: behind the rows for one row, else over them (written
  // after the barrier that ends every wave's reads of the rows)
  float *red = (float *)(ER == 1 ? dsm + ((rows * xpitch + 255) & ~255) : dsm);
  __shared__ int last_flag;
  const int nt0 = blockIdx.x * T;
  const int split = blockIdx.y;
  const int ks0 = split * kspan;              // first K of this split (< K)
  const int kk = min(kspan, a.k - ks0);       // K values of this split (a multiple of 512)

  // 1. activations -> LDS, 512 values (64 lanes x 16 B) per copy; columns
  //    kk .. kspan (a partial last wave) are zeros.  With KR >= 4 each wave
  //    copies the K range it reads itself (KR / 4 copies per row), so it only
  //    waits for its own copies; with fewer blocks per wave the waves copy
  //    the rows together and meet at a barrier.
  constexpr bool OWN_X = KR >= 4;
  if constexpr (OWN_X) {
    const int kw = wave * KR * 128;  // the wave's first K (within the split)
#pragma unroll
    for (int c = 0; c < KR / 4; ++c) {
      const int c0 = kw + c * 512;
      for (int r = 0; r < rows; ++r) {
        if (c0 < kk)  // wave-uniform
          lds_dma16((const uint16_t *)a.x + (int64_t)r * a.ldx + ks0 + c0 + lane * 8, dsm + r * xpitch + c0 * 2);
        else
          *(u32x4 *)(dsm + r * xpitch + c0 * 2 + lane * 16) = u32x4{0u, 0u, 0u, 0u};
      }
    }
  } else {
    const int per_row = kk >> 9;
    for (int i = wave; i < rows * per_row; i += nwaves) {
      const int r = i / per_row, c0 = (i - r * per_row) << 9;
      lds_dma16((const uint16_t *)a.x + (int64_t)r * a.ldx + ks0 + c0 + lane * 8, dsm + r * xpitch + c0 * 2);
    }
    const int tail = (kspan - kk) >> 3;  // 16-byte chunks per row
    for (int i = threadIdx.x; i < rows * tail; i += blockDim.x) {
      const int r = i / tail;
      *(u32x4 *)(dsm + r * xpitch + kk * 2 + (i - r * tail) * 16) = u32x4{0u, 0u, 0u, 0u};
    }
    QG_WAIT_LGKMCNT0();  // the zeros, before the barrier that publishes them
  }
  __builtin_amdgcn_sched_barrier(0);

  // 2. weights (the first loads in flight), then the wait that covers the
  //    copies above: at least T * (blocks issued) weight loads went out after
  //    them
  f32x4 acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = {0.f, 0.f, 0.f, 0.f};
  const uint16_t *xrow = (const uint16_t *)(dsm + min(r16, rows - 1) * xpitch);
  constexpr int ISSUED = FmtTraits<FMT>::EXT ? KR : a16_pipe_depth<true, KR>();
  auto x_ready = [&]() {
    QG_WAIT_VMCNT(T * ISSUED);
    asm volatile("" ::: "memory");
    if constexpr (!OWN_X) __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  if constexpr (FmtTraits<FMT>::EXT)
    a16x_wave<FMT, GROUP, T, KR, true, ER, decltype(x_ready)>(a, a.wbase, xrow, nt0, (split * nwaves + wave) * KR,
                                                              acc, x_ready, ks0);
  else
    a16_wave<BITS, ZP, GROUP, T, KR, true, ER, decltype(x_ready), FMT == 5>(
        a, a.wbase, xrow, nt0, (split * nwaves + wave) * KR, acc, x_ready, ks0);

  // 3. reduce the waves (valid rows only) and store
  if constexpr (ER != 1) __syncthreads();  // (the partials overwrite the rows)
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * q + e;
      if (r < rows) red[((wave * T + t) * rows + r) * 16 + r16] = acc[t][e];
    }
  __syncthreads();
  const int n_out = T * rows * 16;
  if (gridDim.y == 1) {
    for (int idx = threadIdx.x; idx < n_out; idx += blockDim.x) {
      float sum = 0.f;
      for (int w = 0; w < nwaves; ++w) sum += red[w * T * rows * 16 + idx];
      const int t = idx / (rows * 16), r = (idx / 16) % rows, col = (nt0 + t) * 16 + (idx & 15);
      if (col < a.n && nt0 + t < a.n_tiles) store_out(a.y, a.ldy, a.otype, r, col, sum);
    }
    return;
  }
  // split K: partial tile of this split (T * 256 floats per tile, element
  // (t, r, c) at t * 256 + r * 16 + c), published by the counter add after
  // the agent-scope stores have completed
  float *part = a.partials + ((int64_t)split * gridDim.x + blockIdx.x) * (T * 256);
  for (int idx = threadIdx.x; idx < n_out; idx += blockDim.x) {
    float sum = 0.f;
    for (int w = 0; w < nwaves; ++w) sum += red[w * T * rows * 16 + idx];
    const int t = idx / (rows * 16), rc = idx - t * rows * 16;
    __hip_atomic_store(part + t * 256 + rc, sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(a.counters + blockIdx.x, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    last_flag = (prev == gridDim.y - 1);
  }
  __syncthreads();
  if (!last_flag) return;  // uniform across the workgroup
  for (int idx = threadIdx.x; idx < n_out; idx += blockDim.x) {
    const int t = idx / (rows * 16), rc = idx - t * rows * 16, r = rc / 16;
    const float sum = sum_partials(a.partials + (int64_t)blockIdx.x * (T * 256) + t * 256 + rc,
                                   (int64_t)gridDim.x * (T * 256), (int)gridDim.y);
    const int col = (nt0 + t) * 16 + (idx & 15);
    if (col < a.n && nt0 + t < a.n_tiles) store_out(a.y, a.ldy, a.otype, r, col, sum);
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(a.counters + blockIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}



// ---------------------------------------------------------------------------
// dense decode, wide form (2 .. 16 rows): the workgroup's waves run along N
// ---------------------------------------------------------------------------
//
// The form above copies its rows over the whole K range of the workgroup, for
// every column tile: at 16 rows and K = 14336 that is 459 KB per workgroup,
// 117 MB over the launch against 30.5 MB of weights.  Here the W waves of a
// workgroup take W consecutive n-tiles (one each) over one K slice of KR
// blocks, and the rows' slice is copied into LDS once for all of them:
// gridDim.y = ceil(K / (KR * 128)) slices, each workgroup's activation copy
// rows * KR * 256 bytes (4096 x 14336 at 16 rows: 7.3 MB in all).  The
// waves copy the slice together and issue their first weight loads, then wait
// for their copies and meet at a barrier; each wave then runs the decode wave
// body on its n-tile (pipelined weight loads) and writes its 16 x 16 tile:
// directly with one slice, else as an fp32 partial, combined in slice order
// by the last workgroup of the column group to arrive (per-group arrival
// counter, reset by that workgroup).  Requires K % 512 == 0.
template <int FMT, int GROUP, int KR, int ER>
__global__ __launch_bounds__(kMaxWaves * 64) void decode_wide_kernel(GemmArgs a) {
  constexpr int BITS = FmtTraits<FMT>::BITS;
  constexpr bool ZP = FmtTraits<FMT>::ZP;
  constexpr int KS = KR * 128;       // K values of one slice
  constexpr int XP = KS * 2 + 16;    // LDS bytes per row (padded: bank spread)
  constexpr int PER_ROW = KS / 512;  // 64-lane copies per row
  extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
  __shared__ int last_flag;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  const int rows = ER == 1 ? 1 : a.m;
  const int nt0 = blockIdx.x * nwaves + wave;  // this wave's n-tile (past N: clamped loads, no stores)
  const int split = blockIdx.y;
  const int ks0 = split * KS;
  const int kk = min(KS, a.k - ks0);           // a multiple of 512

  // 1. the rows' K slice -> LDS (zeros past K), the copies shared out over
  //    the waves
  for (int i = wave; i < rows * PER_ROW; i += nwaves) {
    const int r = i / PER_ROW, c0 = (i % PER_ROW) * 512;
    if (c0 < kk)  // wave-uniform
      lds_dma16((const uint16_t *)a.x + (int64_t)r * a.ldx + ks0 + c0 + lane * 8, dsm + r * XP + c0 * 2);
    else
      *(u32x4 *)(dsm + r * XP + c0 * 2 + lane * 16) = u32x4{0u, 0u, 0u, 0u};
  }
  QG_WAIT_LGKMCNT0();  // the zeros, before the barrier that publishes them
  __builtin_amdgcn_sched_barrier(0);

  // 2. the wave's n-tile over the slice: its first weight loads go out, then
  //    it waits for its own copies (issued before them) and meets the other
  //    waves at a barrier, after which every copy of the slice has landed
  f32x4 acc[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
  const uint16_t *xrow = (const uint16_t *)(dsm + min(r16, rows - 1) * XP);
  constexpr int ISSUED = FmtTraits<FMT>::EXT ? KR : a16_pipe_depth<true, KR>();
  auto x_ready = [&]() {
    QG_WAIT_VMCNT(ISSUED);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  if constexpr (FmtTraits<FMT>::EXT)
    a16x_wave<FMT, GROUP, 1, KR, true, ER, decltype(x_ready)>(a, a.wbase, xrow, nt0, split * KR, acc, x_ready,
                                                              ks0);
  else
    a16_wave<BITS, ZP, GROUP, 1, KR, true, ER, decltype(x_ready), FMT == 5>(a, a.wbase, xrow, nt0, split * KR,
                                                                            acc, x_ready, ks0);

  // 3. store: element (e, lane) is row 4 (lane / 16) + e, column lane % 16 of the tile
  const int col = nt0 * 16 + r16;
  const bool col_ok = nt0 < a.n_tiles && col < a.n;
  if (gridDim.y == 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * q + e;
      if (r < rows && col_ok) store_out(a.y, a.ldy, a.otype, r, col, acc[0][e]);
    }
    return;
  }
  float *part = a.partials + (((int64_t)split * gridDim.x + blockIdx.x) * nwaves + wave) * 256;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    __hip_atomic_store(part + e * 64 + lane, acc[0][e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(a.counters + blockIdx.x, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    last_flag = (prev == gridDim.y - 1);
  }
  __syncthreads();
  if (!last_flag) return;  // uniform across the workgroup
  const f32x4 sum = sum_partials4(a.partials + ((int64_t)blockIdx.x * nwaves + wave) * 256 + lane,
                                  (int64_t)gridDim.x * nwaves * 256, (int)gridDim.y);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = 4 * q + e;
    const float v = sum[e];  // (element copied out: see the bit-cast note in a16_wave)
    if (r < rows && col_ok) store_out(a.y, a.ldy, a.otype, r, col, v);
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(a.counters + blockIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace qg
