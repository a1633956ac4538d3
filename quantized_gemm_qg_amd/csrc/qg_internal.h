// Internal declarations shared by the host side of libqg (validation, repack,
// dispatch) and the HIP kernel launchers.  Not part of the public ABI.
//
// Packed layout, version 2 (QG_LAYOUT_VERSION; one section per expert, each part 256-B aligned):
//
//   codes   k-blocks of 128 along K, n-tiles of 16 along N, block (t, kb) at
//           byte ((t * k_blocks) + kb) * block_bytes.  Inside a block, lane
//           l = 0..63 of a wave owns a contiguous slice: output column
//           n = 16 t + (l % 16) and the K range the bf16 / f8f6f4 MFMA B
//           operand of that lane covers (q = l / 16):
//     * 4-bit integer (block 1024 B, 16 B per lane = 4 dwords): dword j
//       (one 16x16x32 MFMA) holds k = 128 kb + 32 j + 8 q + e, e = 0..7, with
//       code e in nibble slot (e / 2) + 4 (e % 2), so one shift + and/or turns
//       slots (i, i + 4) into the bf16 pair (e = 2i, 2i + 1).
//     * 3-bit integer (block 768 B, 12 B per lane = 3 dwords): dword j < 3
//       holds MFMA j's eight codes in bits 0..2 of the same nibble slots; the
//       eight codes of MFMA 3 are spread over the slots' bit 3, bit b of a code
//       living in dword b.
//     * 8-bit integer and e4m3 weights x bf16 (block 2048 B, 32 B per lane =
//       8 dwords): bytes 8 j .. 8 j + 7 hold MFMA j's codes e = 0..7 in order.
//     * 2-bit integer (block 512 B, 8 B per lane): dword j / 2 holds MFMAs j
//       and j + 1 (j even); code e of MFMA j in 2-bit slot 4 (j % 2) + e / 2 +
//       8 (e % 2).
//     * 1-bit integer (block 256 B, 4 B per lane): code e of MFMA j in bit
//       4 j + e / 2 + 16 (e % 2).
//     * Integer codes are stored offset-binary (u = c + 2^(b-1) for signed
//       formats), so every integer format computes (u - z) with z = 2^(b-1)
//       implied for signed formats; e0m3 / e0m7 codes (sign and magnitude)
//       become the offset-binary code of their value, u = v + 8 / v + 128.
//     * W8A8 e4m3 (block 2048 B, 32 B per lane): the lane's bytes are K 16 q
//       .. 16 q + 15 and 64 + 16 q .. 64 + 16 q + 15 of the block for column
//       n = 16 t + l % 16 (the scaled MFMA's 8-bit operand).
//     * e2m1 (block 1024 B, 16 B per lane): the lane's 32 codes k = 128 kb +
//       32 q + e in standard order (two per byte, low nibble first), i.e. the
//       16-B chunk of the standard row that one 16x16x128 scaled MFMA lane reads.
//     * e2m1 for bf16 activations: the 4-bit integer lane order above (dword
//       j = the codes of bf16 MFMA j) with the eight codes in standard order
//       (byte i = codes 2i, 2i + 1, low nibble first), the order the
//       fp4 -> bf16 pair conversion emits.
//   scales  A16: bf16 [n_pad][groups_padded] (groups rounded up to 32); for
//           e2m1 with bf16 activations each e8m0 code c is stored as the bf16
//           2^(c - 127) (c = 0: 0x0040).
//           MXFP4: e8m0 in 256-byte units [n_tile][kb_pad / 4], each
//           [16 columns c][4 quarters q][4 k-blocks]: byte (n, q, kb) scales
//           k = 128 kb + 32 q .. +31 of column n = 16 n_tile + c; kb_pad =
//           k_blocks rounded up to 4.  A lane reads four k-blocks' scales of
//           its (column, quarter) as one dword, and 64 lanes read one unit
//           (a whole n-tile) as 256 contiguous bytes.
//           W8A8: fp32 [n_tile][kb_pad], the scale of the 128 x 128 block
//           holding n-tile n_tile and k-block kb.
//   zeros   UINT formats: [n_pad][groups_padded / 8] uint32, group g in nibble
//           g % 8 of word g / 8; UINT8: [n_pad][groups_padded / 4] uint32,
//           group g in byte g % 4 of word g / 4.
//
// Padding (n >= N, k >= K) holds code 0 with scale 0 (A16) or scale code 0
// (MX), so padded weights are exactly zero; kernels also zero activations
// beyond K.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/qg.h"

namespace qg {

// MXFP4 weights with MXFP8 activations run the MX kernels (codes straight
// into the scaled MFMA); with bf16 activations they run the integer-format
// skinny kernel, the codes dequantized to exact bf16 by the fp4 conversion.
inline bool mx_a8(const qg_layer_desc &d) { return d.wtype == QG_W_MXFP4 && d.atype == QG_A_MXFP8; }
inline bool fp4_a16(const qg_layer_desc &d) { return d.wtype == QG_W_MXFP4 && d.atype == QG_A_BF16; }
// MXFP4 weights with MXFP4 activations (W4A4): the MX layout, the large-M MX
// kernel with e2m1 A operands, dense layers only.
inline bool mx_a4(const qg_layer_desc &d) { return d.wtype == QG_W_MXFP4 && d.atype == QG_A_MXFP4; }
// MXFP4 weights with per-token FP8 activations: the MX layout, the MX skinny
// kernel with unit activation block scales and the row scale in the output.
inline bool mx_tok(const qg_layer_desc &d) { return d.wtype == QG_W_MXFP4 && d.atype == QG_A_FP8_TOKEN; }
// W8A8 FP8 with block scales (e4m3 x e4m3, fp32 scales)
inline bool w8a8(const qg_layer_desc &d) { return d.wtype == QG_W_FP8 && d.atype == QG_A_FP8_BLOCK; }
// Layers of the MX tiled kernel (MXFP4 weights with MXFP8, MXFP4 or per-token
// FP8 activations; W8A8)
inline bool mx_tiled_fmt(const qg_layer_desc &d) { return mx_a8(d) || mx_a4(d) || mx_tok(d) || w8a8(d); }

// Kernel format of a layer (the FMT of the skinny and decode kernels, see
// FmtTraits in qg_wave.h).  e0m3 weights are stored as offset-binary INT4 and
// e0m7 as offset-binary INT8 (the same values), so they run those formats.
inline int kernel_fmt(const qg_layer_desc &d) {
  switch (d.wtype) {
    case QG_W_INT4: case QG_W_E0M3: return 0;
    case QG_W_UINT4: return 1;
    case QG_W_INT3: return 2;
    case QG_W_UINT3: return 3;
    case QG_W_INT8: case QG_W_E0M7: return 7;
    case QG_W_UINT8: return 8;
    case QG_W_INT2: return 9;
    case QG_W_UINT2: return 10;
    case QG_W_INT1: return 11;
    case QG_W_UINT1: return 12;
    case QG_W_FP8: return d.atype == QG_A_FP8_BLOCK ? 15 : 13;
    default: return fp4_a16(d) ? 5 : mx_a4(d) ? 6 : mx_tok(d) ? 14 : 4;
  }
}
// Formats of a16x_wave (1-, 2-, 8-bit integers, e4m3 weights; bf16 activations)
inline bool ext_a16(const qg_layer_desc &d) {
  const int f = kernel_fmt(d);
  return f >= 7 && f <= 13;
}
// Largest T * KR of a spill-free skinny wave for the formats of a16x_wave
// and W8A8 (T <= 2): 2 for 8-bit slices and for group 32, else 4.
inline int ext_wave_cap(const qg_layer_desc &d) {
  const int f = kernel_fmt(d);
  return (f == 7 || f == 8 || f == 13 || (f >= 7 && f <= 13 && d.group_size == 32)) ? 2 : 4;
}
// Formats served by the LDS-tiled kernels (large M, MoE tiles): the 4- and
// 3-bit integer formats (e0m3 included), MXFP4 with bf16, MXFP8, MXFP4 or
// per-token FP8 activations, and W8A8.  The others run the decode and skinny
// kernels.
inline bool has_tiled(const qg_layer_desc &d) {
  const int f = kernel_fmt(d);
  return f <= 6 || f >= 14;
}

constexpr int kTileN = 16;    // N per tile
constexpr int kBlockK = 128;  // K per block

struct Layout {
  int n_tiles = 0;
  int k_blocks = 0;
  int groups = 0;         // K / group
  int groups_padded = 0;  // rounded up to 32
  int kb_pad = 0;         // k_blocks rounded up to 4
  int bits = 0;
  bool has_zp = false;
  bool is_mx = false;     // MX kernels (MXFP4 x MXFP8, or x MXFP4 with a4)
  bool mx_pack = false;   // MX code and scale layout (is_mx, or per-token FP8 activations)
  bool a4 = false;        // MXFP4 activations (two e2m1 codes per byte)
  bool fp4 = false;       // MXFP4 weights x bf16 activations (integer-format layout, bf16 scales)
  bool f8 = false;        // W8A8: e4m3 codes in the 8-bit MFMA operand layout, fp32 block scales
  bool x8 = false;        // one byte per activation element (e4m3)
  int xs_kind = 0;        // activation scales: 0 none, 1 e8m0 per 32, 2 fp32 per row, 3 fp32 per row and 128 K
  uint64_t block_bytes = 0;
  uint64_t codes_bytes = 0;
  uint64_t scales_offset = 0;
  uint64_t scales_bytes = 0;
  uint64_t zeros_offset = 0;
  uint64_t zeros_bytes = 0;
  uint64_t expert_stride = 0;
  uint64_t total_bytes = 0;
};

inline uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

// LDS of the decode kernel: the rows (m x W KR 128 bf16, each row padded by 16
// bytes) and the waves' partial tiles (W x T x m x 16 floats).  With more than
// one row the partials reuse the rows' space once every wave is done with
// them (one workgroup barrier), so up to 8 rows of 4096 fit two workgroups
// per CU and 16 rows fit one.
inline uint64_t decode_lds_bytes(int64_t m, int W, int T, int KR) {
  const uint64_t x = align_up((uint64_t)m * ((uint64_t)W * KR * 256 + 16), 256);
  const uint64_t red = (uint64_t)W * T * m * 64;
  return m == 1 ? x + red : (x > red ? x : red);
}

// Validates a descriptor; fills the layout on success.
qg_status make_layout(const qg_layer_desc *d, Layout *out);

// Bytes of one expert's standard-format codes, scales and zero points.
void std_sizes(const qg_layer_desc &d, const Layout &L, uint64_t *codes, uint64_t *scales, uint64_t *zeros);

// Host repack of one expert's standard-format tensors into its packed section.
void repack_expert(const qg_layer_desc &d, const Layout &L, const uint8_t *codes,
                   const uint8_t *scales, const uint8_t *zeros, uint8_t *dst);

// Thread-local record of the last HIP error.
void set_last_hip_error(int32_t e);

// ---------------------------------------------------------------------------
// kernel launch parameters
// ---------------------------------------------------------------------------

struct GemmArgs {
  // packed weight
  const uint8_t *wbase;
  uint64_t expert_stride;
  uint64_t scales_offset;
  uint64_t zeros_offset;
  int32_t n_tiles, k_blocks, groups_padded, kb_pad;
  int32_t n, k;
  // activations / output
  const void *x;
  const uint8_t *x_scales;
  // dense MX tiled kernel: the activation scales regrouped by K step,
  // dword [kb * m + row] = the 4 e8m0 scales of row `row` in K step kb
  const uint32_t *x_scales_t;
  int64_t ldx;
  void *y;
  int64_t ldy;
  int32_t otype;
  int32_t m;  // dense rows
  // split-K workspace (dense)
  float *partials;
  uint32_t *counters;
  int32_t splits;
  // MoE
  const int32_t *sorted_ids;
  const int32_t *offsets;
  int32_t num_experts;
  int32_t topk;
  int32_t x_rows;
  int32_t y_rows;
  // MoE split between the two kernels: the tiled kernels walk the tile list
  // [count, 0, (expert, first sorted row) ...] of experts with at least
  // moe_min_rows rows; the skinny kernel skips those experts (0 = skips none)
  const int32_t *tiles;
  int32_t moe_min_rows;
  // tiled kernels: m-tiles per raster group (see tile_of)
  int32_t group_m;
};

constexpr int kMaxExperts = 1024;  // LDS-resident per-expert tables

// Dense workspaces begin with the arrival counters of split-K launches (one
// uint32 per output tile, left at zero by every launch); partial tiles and
// the tiled kernels' scratch follow this prefix.
constexpr uint64_t kSplitCounterBytes = 64 * 1024;
constexpr int64_t kMaxSplitCounters = (int64_t)(kSplitCounterBytes / 4);

// One entry of the tuning table: a kernel variant and its tile parameters.
struct Variant {
  int kind;    // 0 = skinny (16-row tiles, weights streamed to VGPRs), 1 = MX tiled (LDS),
               // 2 = integer-format tiled (LDS, bf16 MFMA), 3 = decode (activations in LDS),
               // 4 = wide decode (waves along N over one K slice, activations in LDS)
  int T;       // n-tiles per wave
  int KR;      // k-blocks per wave
  int W;       // waves per workgroup (split of K inside the workgroup)
  int splits;  // split of K across workgroups
  int bm;      // tiled: workgroup tile rows (128 or 256)
  int tbn;     // tiled: workgroup tile columns (MX: 192, 224 or 256; integer formats: 128)
};

Variant select_dense(const qg_weight &w, int64_t m);
Variant select_moe(const qg_weight &w, int64_t pairs);

hipError_t launch_dense_a16(const GemmArgs &a, const qg_layer_desc &d, const Variant &v,
                            hipStream_t s);
// Skinny and decode instances of the formats 7 .. 15 (qg_formats.hip): the
// same contracts as the launches above for those formats.
hipError_t launch_skinny_ext(const GemmArgs &a, int fmt, int group, const Variant &v, bool moe, int64_t grid,
                             int64_t items, hipStream_t s);
hipError_t launch_decode_ext(const GemmArgs &a, int fmt, int group, const Variant &v, hipStream_t s);
hipError_t launch_dense_mx(const GemmArgs &a, const qg_layer_desc &d, const Variant &v,
                           hipStream_t s);
// Dense decode for the integer formats (m <= 16, K % 512 == 0): activations
// staged in LDS, one workgroup per v.T n-tiles over all of K (v.W * v.KR * 128 >= K).
hipError_t launch_decode_a16(const GemmArgs &a, const qg_layer_desc &d, const Variant &v,
                             hipStream_t s);
// Wide decode form (kind 4; 2 <= m <= 16, K % 512 == 0): v.W waves along N
// per workgroup, one K slice of v.KR blocks each, v.splits slices.
hipError_t launch_decode_wide(const GemmArgs &a, const qg_layer_desc &d, const Variant &v, hipStream_t s);
hipError_t launch_decode_wide_ext(const GemmArgs &a, int fmt, int group, const Variant &v, hipStream_t s);
hipError_t launch_moe_a16(const GemmArgs &a, const qg_layer_desc &d, const Variant &v,
                          int64_t max_tiles, hipStream_t s);
hipError_t launch_moe_mx(const GemmArgs &a, const qg_layer_desc &d, const Variant &v,
                         int64_t max_tiles, hipStream_t s);
// MoE launches of the tiled kernels walk the tile list a.tiles of capacity
// tiles_cap, cut at kMoeTileRows rows; experts with fewer rows than the
// tiled threshold go to the integer formats' small-tile form in one
// kMoeSmallTileRows-row tile each.
constexpr int kMoeTileRows = 128;
constexpr int kMoeSmallTileRows = 64;
// Dense launches first regroup the activation scales by K step into ws
// (mx_tiled_ws_bytes); MoE launches read them in place.
// a4: the activations are e2m1 (a.ldx then counts bytes, K / 2 per row
// minimum).  rs: e4m3 activations with one fp32 scale per row (a.x_scales):
// unit block scales in the MFMA, each output row times its row's scale; no
// scale copies, no workspace; 8-wave forms.  f8: W8A8 (e4m3 x e4m3, fp32
// block scales; bn must be 128; no workspace).
hipError_t launch_mx_tiled(const GemmArgs &a, int bm, int bn, bool moe, int64_t tiles_cap, int waves,
                           void *ws, hipStream_t s, bool a4 = false, bool rs = false, bool f8 = false);
uint64_t mx_tiled_ws_bytes(int64_t m, int64_t k_blocks);
int mx_tiled_waves();  // QG_MX_WAVES (4 or 8), else the default
// Integer formats at large M: group row sums of X into ws, then the tiled
// kernel.  ws holds (K / group) * m floats (a16_tiled_ws_bytes).
// xs_rows: rows of X (dense: m; MoE: tokens or pairs, by the x row mode).
// sums = false skips the row sums (already in ws from an earlier launch on the
// same X).
hipError_t launch_a16_tiled(const GemmArgs &a, const qg_layer_desc &d, int bm, int bn, bool moe,
                            int64_t xs_rows, int64_t tiles_cap, int waves, void *ws, bool sums,
                            hipStream_t s);
int a16_tiled_waves();  // QG_A16_WAVES (4 or 8), else the default
int a16_tiled_bn();     // tile columns of the integer-format tiled kernel (QG_A16_BN)
uint64_t a16_tiled_ws_bytes(const qg_layer_desc &d, int64_t m);
// MoE tile list for the tiled kernels (experts with min_rows <= rows <
// max_rows, max_rows = 0 for no bound; bm-row tiles): tiles[0] = count, then
// (expert, first sorted row) pairs.
hipError_t launch_moe_tiles(const int32_t *offsets, int32_t experts, int32_t min_rows,
                            int32_t max_rows, int32_t bm, int32_t pairs, int32_t capacity,
                            int32_t *tiles, hipStream_t s);
// Both lists of a split in one launch: experts with >= min_rows rows in
// kMoeTileRows-row tiles (tiles, capacity) and the others with rows in
// small_bm-row tiles (tiles_small, capacity_small).
hipError_t launch_moe_tiles2(const int32_t *offsets, int32_t experts, int32_t pairs, int32_t min_rows,
                             int32_t capacity, int32_t *tiles, int32_t small_bm, int32_t capacity_small,
                             int32_t *tiles_small, hipStream_t s);
hipError_t launch_stream_read(const void *src, uint64_t bytes, void *sink, hipStream_t s);
hipError_t launch_stream_copy(void *dst, const void *src, uint64_t bytes, hipStream_t s);
// Activation-side kernels (qg_act.hip): bf16 -> MXFP8, SiLU-gated product,
// weighted top-k combine.  Shapes and alignment are validated by the callers.
hipError_t launch_quantize_mxfp4(const void *x, int64_t rows, int64_t k, int64_t ldx, void *q, int64_t ldq,
                                 void *qs, hipStream_t s);
hipError_t launch_quantize_mxfp8(const void *x, int64_t rows, int64_t k, int64_t ldx, void *q, int64_t ldq,
                                 void *qs, hipStream_t s);
// bf16 -> e4m3 with fp32 scales per row (block 0) or per 128 values (block 128)
hipError_t launch_quantize_fp8(const void *x, int64_t rows, int64_t k, int64_t ldx, int block, void *q,
                               int64_t ldq, float *qs, hipStream_t s);
hipError_t launch_silu_mul(const void *gu, bool gu_f32, int64_t rows, int64_t inter, int64_t ldgu, bool mx,
                           void *h, int64_t ldh, void *hs, hipStream_t s);
hipError_t launch_moe_combine(const void *y, bool y_f32, int64_t ldy, const float *wts, int64_t tokens, int topk,
                              int64_t n, const void *bias, void *out, bool out_f32, int64_t ldo, hipStream_t s);
hipError_t launch_moe_sort(const int32_t *ids, int64_t pairs, int32_t experts,
                           int32_t *sorted, int32_t *offsets, int32_t *ws_counts,
                           hipStream_t s);

}  // namespace qg
