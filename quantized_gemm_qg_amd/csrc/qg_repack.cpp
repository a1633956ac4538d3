// Validation of layer descriptors and the host repack from the standard format
// into the packed kernel layout (the announcement's "Per-workload tuning and JIT
// compilation" section: preprocessing validates parameters, pads dimensions and
// repacks tensors for the target kernel).  Pure CPU code.
#include <string.h>

#include <algorithm>
#include <thread>
#include <vector>

#include "qg_internal.h"

namespace qg {

// Formats with bf16 group scales and bf16 activations, and their code widths.
static int a16_bits(int w) {
  switch (w) {
    case QG_W_INT4: case QG_W_UINT4: case QG_W_E0M3: return 4;
    case QG_W_INT3: case QG_W_UINT3: return 3;
    case QG_W_INT8: case QG_W_UINT8: case QG_W_E0M7: case QG_W_FP8: return 8;
    case QG_W_INT2: case QG_W_UINT2: return 2;
    case QG_W_INT1: case QG_W_UINT1: return 1;
  }
  return 0;
}
static bool has_zp_type(int w) {
  return w == QG_W_UINT4 || w == QG_W_UINT3 || w == QG_W_UINT8 || w == QG_W_UINT2 || w == QG_W_UINT1;
}

qg_status make_layout(const qg_layer_desc *d, Layout *out) {
  if (!d || !out) return QG_ERR_INVALID_ARGUMENT;
  if (d->abi_version != QG_ABI_VERSION) return QG_ERR_INVALID_ARGUMENT;
  if (d->wtype < QG_W_INT4 || d->wtype > QG_W_FP8) return QG_ERR_INVALID_ARGUMENT;
  if (d->stype < QG_S_BF16 || d->stype > QG_S_F32) return QG_ERR_INVALID_ARGUMENT;
  if (d->atype < QG_A_BF16 || d->atype > QG_A_FP8_BLOCK) return QG_ERR_INVALID_ARGUMENT;
  if (d->n <= 0 || d->k <= 0 || d->num_experts <= 0 || d->group_size <= 0) return QG_ERR_SHAPE;
  if (d->n > (1 << 24) || d->k > (1 << 24) || d->num_experts > 4096) return QG_ERR_UNSUPPORTED;
  if (d->k % 32 != 0 || d->k % d->group_size != 0) return QG_ERR_SHAPE;
  Layout L;
  if (d->wtype == QG_W_FP8 && d->atype == QG_A_FP8_BLOCK) {
    // W8A8: fp32 scales per 128 x 128 block, the 8-bit MFMA operand layout
    if (d->stype != QG_S_F32 || d->group_size != 128) return QG_ERR_UNSUPPORTED;
    L.bits = 8;
    L.f8 = true;
    L.x8 = true;
    L.xs_kind = 3;
  } else if (a16_bits(d->wtype) != 0) {
    if (d->stype != QG_S_BF16 || d->atype != QG_A_BF16) return QG_ERR_UNSUPPORTED;
    if (d->group_size != 32 && d->group_size != 64 && d->group_size != 128) return QG_ERR_UNSUPPORTED;
    L.bits = a16_bits(d->wtype);
    L.has_zp = has_zp_type(d->wtype);
  } else {
    if (d->stype != QG_S_E8M0 || d->group_size != 32) return QG_ERR_UNSUPPORTED;
    L.bits = 4;
    // MXFP8 or MXFP4 activations: the MX layout (W4A4 needs K % 128 == 0,
    // the MX tiled kernel's K step); bf16 activations: the 4-bit integer
    // layout with each e8m0 scale stored as its (exact) bf16 power of two
    if (d->atype == QG_A_MXFP4 && d->k % kBlockK != 0) return QG_ERR_UNSUPPORTED;
    if (d->atype == QG_A_FP8_BLOCK) return QG_ERR_UNSUPPORTED;
    L.is_mx = d->atype == QG_A_MXFP8 || d->atype == QG_A_MXFP4;
    L.mx_pack = L.is_mx || d->atype == QG_A_FP8_TOKEN;
    L.a4 = d->atype == QG_A_MXFP4;
    L.fp4 = d->atype == QG_A_BF16;
    L.x8 = d->atype == QG_A_MXFP8 || d->atype == QG_A_FP8_TOKEN;
    L.xs_kind = L.is_mx ? 1 : d->atype == QG_A_FP8_TOKEN ? 2 : 0;
  }
  L.n_tiles = (int)((d->n + kTileN - 1) / kTileN);
  L.k_blocks = (int)((d->k + kBlockK - 1) / kBlockK);
  L.groups = (int)(d->k / d->group_size);
  const int groups_in_padded_k = L.k_blocks * kBlockK / d->group_size;
  L.groups_padded = (int)align_up((uint64_t)groups_in_padded_k, 32);
  L.kb_pad = (int)align_up((uint64_t)L.k_blocks, 4);
  L.block_bytes = 256 * (uint64_t)L.bits;  // 64 lanes x 4 * bits bytes (MX: 16 B per lane)
  const uint64_t n_pad = (uint64_t)L.n_tiles * kTileN;
  L.codes_bytes = (uint64_t)L.n_tiles * L.k_blocks * L.block_bytes;
  L.scales_offset = align_up(L.codes_bytes, 256);
  L.scales_bytes = L.mx_pack ? n_pad * 4 * (uint64_t)L.kb_pad
                   : L.f8    ? (uint64_t)L.n_tiles * L.kb_pad * 4
                             : n_pad * (uint64_t)L.groups_padded * 2;
  uint64_t end = L.scales_offset + L.scales_bytes;
  if (L.has_zp) {
    L.zeros_offset = align_up(end, 256);
    L.zeros_bytes = n_pad * (uint64_t)L.groups_padded * (L.bits == 8 ? 1 : 0) +
                    (L.bits == 8 ? 0 : n_pad * (uint64_t)(L.groups_padded / 8) * 4);
    end = L.zeros_offset + L.zeros_bytes;
  }
  L.expert_stride = align_up(end, 256);
  L.total_bytes = L.expert_stride * (uint64_t)d->num_experts;
  *out = L;
  return QG_OK;
}

// nibble slot of code e (0..7) inside a 4-bit dword: pairs (e = 2i, 2i + 1)
// sit in slots (i, i + 4)
static inline int slot_of(int e) { return (e >> 1) + 4 * (e & 1); }

static inline uint32_t read_bits(const uint8_t *row, uint64_t bitpos, int bits) {
  uint32_t v = 0;
  for (int b = 0; b < bits; ++b) {
    const uint64_t p = bitpos + b;
    v |= (uint32_t)((row[p >> 3] >> (p & 7)) & 1u) << b;
  }
  return v;
}

// Offset-binary code u of a standard-format integer or e0m code c (b bits):
// signed formats add 2^(b-1) (flip the sign bit), e0m codes (sign bit b-1,
// magnitude below it) become their value + 2^(b-1).
static inline uint32_t offset_code(int wtype, uint32_t c, int bits) {
  const uint32_t half = 1u << (bits - 1);
  switch (wtype) {
    case QG_W_INT8: case QG_W_INT4: case QG_W_INT3: case QG_W_INT2: case QG_W_INT1:
      return c ^ half;
    case QG_W_E0M3: case QG_W_E0M7: {
      const uint32_t mag = c & (half - 1);
      return (c & half) ? half - mag : half + mag;
    }
  }
  return c;  // unsigned formats, e4m3
}

// fp4: e2m1 codes keep their standard order inside the dword (byte i = codes
// 2i, 2i + 1, low nibble first: the order the fp4 -> bf16 pair conversion
// produces its two values in); integer codes go to the nibble slots above.
static void repack_codes_int4(const qg_layer_desc &d, const Layout &L, const uint8_t *codes,
                              uint8_t *dst) {
  const uint64_t row_bytes = (uint64_t)d.k / 2;
  const uint32_t flip = (d.wtype == QG_W_INT4) ? 0x88888888u : 0u;
  const bool natural = L.fp4;
  for (int64_t n = 0; n < d.n; ++n) {
    const uint8_t *row = codes + n * row_bytes;
    const int t = (int)(n / kTileN), ln = (int)(n % kTileN);
    for (int64_t k0 = 0; k0 < d.k; k0 += 8) {
      // eight codes k0..k0+7 = four bytes of the standard row, code e in bits 4e
      uint32_t w;
      memcpy(&w, row + k0 / 2, 4);
      uint32_t out = 0;
      if (natural) {
        out = w;
      } else {
        for (int e = 0; e < 8; ++e) out |= ((w >> (4 * e)) & 15u) << (4 * slot_of(e));
        out ^= flip;
      }
      const int kb = (int)(k0 / kBlockK), kk = (int)(k0 % kBlockK);
      const int j = kk / 32, q = (kk % 32) / 8;
      const int lane = ln + 16 * q;
      uint8_t *blk = dst + ((uint64_t)t * L.k_blocks + kb) * L.block_bytes;
      memcpy(blk + lane * 16 + j * 4, &out, 4);
    }
  }
}

// e0m3: the 4-bit integer layout of the offset-binary code of each value.
static void repack_codes_e0m3(const qg_layer_desc &d, const Layout &L, const uint8_t *codes, uint8_t *dst) {
  const uint64_t row_bytes = (uint64_t)d.k / 2;
  for (int64_t n = 0; n < d.n; ++n) {
    const uint8_t *row = codes + n * row_bytes;
    const int t = (int)(n / kTileN), ln = (int)(n % kTileN);
    for (int64_t k0 = 0; k0 < d.k; k0 += 8) {
      uint32_t w;
      memcpy(&w, row + k0 / 2, 4);
      uint32_t out = 0;
      for (int e = 0; e < 8; ++e) out |= offset_code(d.wtype, (w >> (4 * e)) & 15u, 4) << (4 * slot_of(e));
      const int kb = (int)(k0 / kBlockK), kk = (int)(k0 % kBlockK);
      const int j = kk / 32, q = (kk % 32) / 8;
      uint8_t *blk = dst + ((uint64_t)t * L.k_blocks + kb) * L.block_bytes;
      memcpy(blk + (ln + 16 * q) * 16 + j * 4, &out, 4);
    }
  }
}

static void repack_codes_int3(const qg_layer_desc &d, const Layout &L, const uint8_t *codes,
                              uint8_t *dst) {
  const uint64_t row_bytes = (uint64_t)d.k * 3 / 8;
  const uint32_t off = (d.wtype == QG_W_INT3) ? 4u : 0u;
  for (int64_t n = 0; n < d.n; ++n) {
    const uint8_t *row = codes + n * row_bytes;
    const int t = (int)(n / kTileN), ln = (int)(n % kTileN);
    for (int64_t k = 0; k < d.k; ++k) {
      const uint32_t u = (read_bits(row, (uint64_t)k * 3, 3) ^ off) & 7u;
      const int kb = (int)(k / kBlockK), kk = (int)(k % kBlockK);
      const int j = kk / 32, q = (kk % 32) / 8, e = kk % 8;
      const int lane = ln + 16 * q;
      uint8_t *blk = dst + ((uint64_t)t * L.k_blocks + kb) * L.block_bytes + lane * 12;
      const int s = slot_of(e);
      if (j < 3) {
        uint32_t w;
        memcpy(&w, blk + 4 * j, 4);
        w |= u << (4 * s);
        memcpy(blk + 4 * j, &w, 4);
      } else {
        for (int b = 0; b < 3; ++b) {
          uint32_t w;
          memcpy(&w, blk + 4 * b, 4);
          w |= ((u >> b) & 1u) << (4 * s + 3);
          memcpy(blk + 4 * b, &w, 4);
        }
      }
    }
  }
}

static void repack_codes_mx(const qg_layer_desc &d, const Layout &L, const uint8_t *codes,
                            uint8_t *dst) {
  const uint64_t row_bytes = (uint64_t)d.k / 2;
  for (int64_t n = 0; n < d.n; ++n) {
    const uint8_t *row = codes + n * row_bytes;
    const int t = (int)(n / kTileN), ln = (int)(n % kTileN);
    for (int64_t k0 = 0; k0 < d.k; k0 += 32) {
      const int kb = (int)(k0 / kBlockK), q = (int)((k0 % kBlockK) / 32);
      const int lane = ln + 16 * q;
      uint8_t *blk = dst + ((uint64_t)t * L.k_blocks + kb) * L.block_bytes;
      memcpy(blk + lane * 16, row + k0 / 2, 16);
    }
  }
}

// 1-, 2- and 8-bit integers and e4m3 with bf16 activations: code (j, e) of
// lane l = column % 16 + 16 q, for k = 128 kb + 32 j + 8 q + e, goes to the
// slot of qg_internal.h's layout.
static void repack_codes_ext(const qg_layer_desc &d, const Layout &L, const uint8_t *codes, uint8_t *dst) {
  const int bits = L.bits;
  const uint64_t row_bytes = (uint64_t)d.k * bits / 8;
  for (int64_t n = 0; n < d.n; ++n) {
    const uint8_t *row = codes + n * row_bytes;
    const int t = (int)(n / kTileN), ln = (int)(n % kTileN);
    for (int64_t k = 0; k < d.k; ++k) {
      const uint32_t c = bits == 8 ? row[k] : read_bits(row, (uint64_t)k * bits, bits);
      const uint32_t u = offset_code(d.wtype, c, bits);
      const int kb = (int)(k / kBlockK), kk = (int)(k % kBlockK);
      const int j = kk / 32, q = (kk % 32) / 8, e = kk % 8;
      uint8_t *lane = dst + ((uint64_t)t * L.k_blocks + kb) * L.block_bytes + (uint64_t)(ln + 16 * q) * 4 * bits;
      if (bits == 8) {
        lane[8 * j + e] = (uint8_t)u;
      } else {
        const int word = bits == 2 ? j / 2 : 0;
        const int slot = bits == 2 ? 4 * (j % 2) + e / 2 + 8 * (e % 2) : 4 * j + e / 2 + 16 * (e % 2);
        uint32_t w;
        memcpy(&w, lane + 4 * word, 4);
        w |= u << (bits * slot);
        memcpy(lane + 4 * word, &w, 4);
      }
    }
  }
}

// W8A8 e4m3 codes: lane l = column % 16 + 16 q of block (t, kb) holds K 16 q
// .. 16 q + 15 then 64 + 16 q .. 64 + 16 q + 15 of the block.
static void repack_codes_f8(const qg_layer_desc &d, const Layout &L, const uint8_t *codes, uint8_t *dst) {
  for (int64_t n = 0; n < d.n; ++n) {
    const uint8_t *row = codes + n * d.k;
    const int t = (int)(n / kTileN), ln = (int)(n % kTileN);
    for (int64_t k0 = 0; k0 < d.k; k0 += 16) {
      const int kb = (int)(k0 / kBlockK), kk = (int)(k0 % kBlockK);
      const int q = (kk % 64) / 16, half = kk / 64;
      uint8_t *lane = dst + ((uint64_t)t * L.k_blocks + kb) * L.block_bytes + (uint64_t)(ln + 16 * q) * 32;
      memcpy(lane + 16 * half, row + k0, 16);
    }
  }
}

void repack_expert(const qg_layer_desc &d, const Layout &L, const uint8_t *codes,
                   const uint8_t *scales, const uint8_t *zeros, uint8_t *dst) {
  memset(dst, 0, L.expert_stride);
  if (L.f8) {
    repack_codes_f8(d, L, codes, dst);
    // block (n / 128, kb) scale -> every n-tile of the block
    const int nb128 = (int)((d.n + 127) / 128);
    float *ds = (float *)(dst + L.scales_offset);
    for (int t = 0; t < L.n_tiles; ++t)
      for (int kb = 0; kb < L.k_blocks; ++kb) {
        const int b = t * kTileN / 128;
        memcpy(&ds[(uint64_t)t * L.kb_pad + kb], scales + ((uint64_t)b * L.k_blocks + kb) * 4, 4);
      }
    (void)nb128;
    return;
  }
  if (L.mx_pack) {
    repack_codes_mx(d, L, codes, dst);
    const int nb32 = (int)(d.k / 32);
    for (int64_t n = 0; n < d.n; ++n)
      for (int i = 0; i < nb32; ++i) {
        const int kb = i / 4, q = i % 4;
        // 256-byte unit (n-tile, kb / 4): [16 columns][4 quarters][4 k-blocks]
        const uint64_t unit = (uint64_t)(n / 16) * (L.kb_pad / 4) + kb / 4;
        dst[L.scales_offset + unit * 256 + ((n % 16) * 4 + q) * 4 + kb % 4] = scales[n * nb32 + i];
      }
    return;
  }
  if (L.bits == 4 && d.wtype != QG_W_E0M3)
    repack_codes_int4(d, L, codes, dst);
  else if (L.bits == 3)
    repack_codes_int3(d, L, codes, dst);
  else if (L.bits == 4)
    repack_codes_e0m3(d, L, codes, dst);
  else
    repack_codes_ext(d, L, codes, dst);
  uint16_t *ds = (uint16_t *)(dst + L.scales_offset);
  if (L.fp4) {
    // e8m0 code c -> bf16 2^(c - 127): exponent field c (c = 0: the subnormal
    // 2^-127 = mantissa bit 6; c = 255: NaN)
    for (int64_t n = 0; n < d.n; ++n)
      for (int g = 0; g < L.groups; ++g) {
        const uint8_t c = scales[n * L.groups + g];
        ds[n * L.groups_padded + g] = c == 0 ? 0x0040 : c == 255 ? 0x7FC0 : (uint16_t)(c << 7);
      }
    return;
  }
  const uint16_t *s16 = (const uint16_t *)scales;
  for (int64_t n = 0; n < d.n; ++n)
    for (int g = 0; g < L.groups; ++g) ds[n * L.groups_padded + g] = s16[n * L.groups + g];
  if (L.has_zp && L.bits == 8) {
    // one byte per group
    for (int64_t n = 0; n < d.n; ++n)
      memcpy(dst + L.zeros_offset + (uint64_t)n * L.groups_padded, zeros + n * L.groups, L.groups);
  } else if (L.has_zp) {
    uint32_t *dz = (uint32_t *)(dst + L.zeros_offset);
    const int words = L.groups_padded / 8;
    for (int64_t n = 0; n < d.n; ++n)
      for (int g = 0; g < L.groups; ++g)
        dz[n * words + g / 8] |= (uint32_t)(zeros[n * L.groups + g] & 15u) << (4 * (g % 8));
  }
}

// Bytes of one expert's standard-format tensors.
void std_sizes(const qg_layer_desc &d, const Layout &L, uint64_t *codes, uint64_t *scales, uint64_t *zeros) {
  *codes = (uint64_t)d.n * d.k * L.bits / 8;
  if (L.f8)
    *scales = (uint64_t)((d.n + 127) / 128) * (d.k / 128) * 4;
  else
    *scales = (uint64_t)d.n * (d.k / d.group_size) * ((L.mx_pack || L.fp4) ? 1 : 2);
  *zeros = L.has_zp ? (uint64_t)d.n * (d.k / d.group_size) : 0;
}

}  // namespace qg

using namespace qg;

extern "C" qg_status qg_packed_size(const qg_layer_desc *desc, uint64_t *bytes) {
  if (!bytes) return QG_ERR_INVALID_ARGUMENT;
  Layout L;
  qg_status st = make_layout(desc, &L);
  if (st != QG_OK) return st;
  *bytes = L.total_bytes;
  return QG_OK;
}

extern "C" qg_status qg_repack_host(const qg_layer_desc *desc, const void *codes,
                                    const void *scales, const void *zeros, int32_t expert_begin,
                                    int32_t expert_count, void *dst, uint64_t dst_bytes) {
  Layout L;
  qg_status st = make_layout(desc, &L);
  if (st != QG_OK) return st;
  if (!codes || !scales || !dst) return QG_ERR_INVALID_ARGUMENT;
  if (L.has_zp && !zeros) return QG_ERR_INVALID_ARGUMENT;
  if (expert_begin < 0 || expert_count < 0 ||
      (int64_t)expert_begin + expert_count > desc->num_experts)
    return QG_ERR_INVALID_ARGUMENT;
  if (dst_bytes < L.total_bytes) return QG_ERR_BUFFER_TOO_SMALL;
  uint64_t cb, sb, zb;
  std_sizes(*desc, L, &cb, &sb, &zb);
  const int nthreads =
      std::max(1, std::min<int>(expert_count, (int)std::min(16u, std::thread::hardware_concurrency())));
  auto work = [&](int tid) {
    for (int e = tid; e < expert_count; e += nthreads) {
      const uint8_t *c = (const uint8_t *)codes + (uint64_t)e * cb;
      const uint8_t *s = (const uint8_t *)scales + (uint64_t)e * sb;
      const uint8_t *z = L.has_zp ? (const uint8_t *)zeros + (uint64_t)e * zb : nullptr;
      repack_expert(*desc, L, c, s, z, (uint8_t *)dst + (uint64_t)(expert_begin + e) * L.expert_stride);
    }
  };
  if (nthreads == 1) {
    work(0);
  } else {
    std::vector<std::thread> pool;
    for (int t = 0; t < nthreads; ++t) pool.emplace_back(work, t);
    for (auto &th : pool) th.join();
  }
  return QG_OK;
}
