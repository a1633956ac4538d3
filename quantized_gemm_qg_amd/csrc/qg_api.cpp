// The C ABI of libqg: argument validation, the tuning table keyed on the M
// range, and dispatch to the HIP kernels on the caller's stream.
//
// Configuration selection follows the announcement's tuning section: a
// configuration is prepared per input-size (M) range and picked at run time by
// a device heuristic; here the heuristic is compiled in for one device
// (MI355X / gfx950) and indexed by (format, M bucket, N, K).
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "qg_internal.h"

namespace qg {

static thread_local int32_t g_last_hip_error = 0;

constexpr int kNumCUs = 256;  // MI355X compute units (8 XCDs x 32)
void set_last_hip_error(int32_t e) { g_last_hip_error = e; }

static qg_status hip_status(hipError_t e) {
  if (e == hipSuccess) return QG_OK;
  set_last_hip_error((int32_t)e);
  return QG_ERR_HIP;
}

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// ---------------------------------------------------------------------------
// Experiment overrides of the tuning table.  The QG_* environment variables
// are read once, at the first dispatch; qg_set_override changes them later.
// Dispatch reads one immutable snapshot through an atomic pointer, so the
// per-call path neither parses strings nor touches the environment, and a
// concurrent qg_set_override never tears a read (replaced snapshots are kept
// until the process ends: they are few and small).
// ---------------------------------------------------------------------------
namespace {
struct Overrides {
  bool tune = false;  // QG_TUNE "T,KR,W,splits": the skinny kernel with these parameters
  int tune_v[4] = {0, 0, 0, 0};
  bool decode_off = false;  // QG_DECODE "0"
  int decode_n = 0;         // QG_DECODE "T,KR[,splits]": number of fields parsed (2 or 3)
  int decode_v[3] = {0, 0, 1};
  int wide = -1;            // QG_DECODE_WIDE: "0" off, "W,KR" the wide decode form, unset: heuristics
  int wide_v[2] = {16, 8};
  bool tiled_off = false;   // QG_TILED "0"
  bool tiled_set = false;   // QG_TILED present (any value): the autotune table is bypassed
  int tiled_bm = 0;         // QG_TILED_BM: 128 or 256
  int mx_bn = 0;            // QG_MX_BN: 192, 224 or 256
  int mx_waves = 0;         // QG_MX_WAVES: 4 or 8
  int a16_waves = 0;        // QG_A16_WAVES: 4 or 8
  int a16_bn = 0;           // QG_A16_BN: 128 or 256 (fixes the integer-format tile width)
  int moe_tiled_min = -1;   // QG_MOE_TILED_MIN: >= 0 (0 disables the tiled MoE kernels)
  int moe_group_m = 0;      // QG_MOE_GROUP_M: 1..64
  int moe_small_bm = 0;     // QG_MOE_SMALL_BM: 32
  int moe_small = -1;       // QG_MOE_SMALL: 0 or 1
  int moe_mx_bn = 0;        // QG_MOE_MX_BN: 128 or 256 (columns of the MX MoE tiles)
  int group_m = 0;          // QG_GROUP_M: 1..64
};

const char *const kOverrideNames[] = {"QG_TUNE", "QG_DECODE", "QG_DECODE_WIDE", "QG_TILED", "QG_TILED_BM", "QG_MX_BN",
                                      "QG_MX_WAVES", "QG_A16_WAVES", "QG_A16_BN", "QG_MOE_TILED_MIN",
                                      "QG_MOE_GROUP_M", "QG_MOE_SMALL_BM", "QG_MOE_SMALL", "QG_MOE_MX_BN",
                                      "QG_GROUP_M"};

// Applies one named override to o (value NULL or "" clears it).  Returns
// false for an unknown name.
bool apply_override(Overrides *o, const char *name, const char *val) {
  const bool set = val && *val;
  const int iv = set ? atoi(val) : 0;
  if (!strcmp(name, "QG_TUNE")) {
    int T, KR, W, S;
    o->tune = set && sscanf(val, "%d,%d,%d,%d", &T, &KR, &W, &S) == 4 && T >= 1 && KR >= 1 && W >= 1 &&
              W <= 16 && S >= 1;
    if (o->tune) {
      o->tune_v[0] = T; o->tune_v[1] = KR; o->tune_v[2] = W; o->tune_v[3] = S;
    }
  } else if (!strcmp(name, "QG_DECODE")) {
    o->decode_off = set && *val == '0';
    o->decode_n = 0;
    int T, KR, S = 1;
    if (set && !o->decode_off) {
      const int n = sscanf(val, "%d,%d,%d", &T, &KR, &S);
      if (n >= 2) {
        o->decode_n = n;
        o->decode_v[0] = T; o->decode_v[1] = KR; o->decode_v[2] = n == 3 ? S : 1;
      }
    }
  } else if (!strcmp(name, "QG_DECODE_WIDE")) {
    int W, KR;
    o->wide = -1;
    if (set && *val == '0') {
      o->wide = 0;
    } else if (set && sscanf(val, "%d,%d", &W, &KR) == 2 && W >= 1 && W <= 16 && (KR == 8 || KR == 16)) {
      o->wide = 1;
      o->wide_v[0] = W; o->wide_v[1] = KR;
    }
  } else if (!strcmp(name, "QG_TILED")) {
    o->tiled_set = set;
    o->tiled_off = set && *val == '0';
  } else if (!strcmp(name, "QG_TILED_BM")) {
    o->tiled_bm = (iv == 128 || iv == 256) ? iv : 0;
  } else if (!strcmp(name, "QG_MX_BN")) {
    o->mx_bn = (iv == 192 || iv == 224 || iv == 256) ? iv : 0;
  } else if (!strcmp(name, "QG_MX_WAVES")) {
    o->mx_waves = (iv == 4 || iv == 8) ? iv : 0;
  } else if (!strcmp(name, "QG_A16_WAVES")) {
    o->a16_waves = (iv == 4 || iv == 8) ? iv : 0;
  } else if (!strcmp(name, "QG_A16_BN")) {
    o->a16_bn = (iv == 128 || iv == 256) ? iv : 0;
  } else if (!strcmp(name, "QG_MOE_TILED_MIN")) {
    o->moe_tiled_min = set ? std::max(0, iv) : -1;
  } else if (!strcmp(name, "QG_MOE_GROUP_M")) {
    o->moe_group_m = (iv >= 1 && iv <= 64) ? iv : 0;
  } else if (!strcmp(name, "QG_MOE_MX_BN")) {
    o->moe_mx_bn = (iv == 128 || iv == 256) ? iv : 0;
  } else if (!strcmp(name, "QG_MOE_SMALL_BM")) {
    o->moe_small_bm = iv == 32 ? 32 : 0;
  } else if (!strcmp(name, "QG_MOE_SMALL")) {
    o->moe_small = set ? (iv != 0) : -1;
  } else if (!strcmp(name, "QG_GROUP_M")) {
    o->group_m = (iv >= 1 && iv <= 64) ? iv : 0;
  } else {
    return false;
  }
  return true;
}

std::atomic<const Overrides *> g_overrides{nullptr};
std::mutex g_overrides_mu;

const Overrides *overrides_from_env() {
  Overrides *o = new Overrides();
  for (const char *name : kOverrideNames) apply_override(o, name, getenv(name));
  return o;
}
}  // namespace

// The current override snapshot (the environment's on first use).
static const Overrides &ov() {
  const Overrides *o = g_overrides.load(std::memory_order_acquire);
  if (o) return *o;
  std::lock_guard<std::mutex> lock(g_overrides_mu);
  o = g_overrides.load(std::memory_order_relaxed);
  if (!o) {
    o = overrides_from_env();
    g_overrides.store(o, std::memory_order_release);
  }
  return *o;
}

// QG_TUNE: the skinny kernel with explicit (T, KR, W, splits).
static bool env_variant(Variant *v) {
  const Overrides &o = ov();
  if (!o.tune) return false;
  *v = Variant{0, o.tune_v[0], o.tune_v[1], o.tune_v[2], o.tune_v[3], 0, 0};
  return true;
}

// Kernel instances compiled ahead of time (see the launchers): T (n-tiles per
// wave) in {1, 2, 4}, KR (k-blocks per wave) in {1, 2, 4}, W in 1..16.  Each
// wave keeps all its activation fragments (16 VGPRs per k-block) and weight
// slices (4 per block) in registers, and 1024-thread workgroups cap a lane at
// 128 VGPRs, so only the spill-free (T, KR) pairs are used: T * KR <= 4 or
// (T, KR) = (4, 2) for the integer formats, T * KR <= 8 but not (4, 4) for MX.
static bool variant_ok(const qg_layer_desc &d, int T, int KR) {
  if ((T != 1 && T != 2 && T != 4) || (KR != 1 && KR != 2 && KR != 4)) return false;
  if (mx_a8(d) || mx_a4(d) || mx_tok(d)) return T * KR <= 8 && !(T == 4 && KR == 4);
  // 1-, 2-, 8-bit integers, e4m3 weights, W8A8: T <= 2 (fewer instances);
  // spill-free: T * KR <= 2 for 8-bit slices (8 registers per block) and for
  // group 32 (16 scales per block), 4 otherwise
  if (ext_a16(d) || w8a8(d)) return T <= 2 && T * KR <= ext_wave_cap(d);
  return T * KR <= 4 || (T == 4 && KR == 2);
}

// Formats with a decode-kernel instance (bf16 activations, A16 formats)
static bool decode_capable(const qg_layer_desc &d) {
  const int f = kernel_fmt(d);
  return f <= 3 || f == 5 || ext_a16(d);
}

static int clamp_kr(const qg_layer_desc &d, int T, int kr) {
  for (int c = 4; c >= 1; c /= 2)
    if (c <= kr && variant_ok(d, T, c)) return c;
  return 1;
}

// Skinny path: each wave streams T n-tiles x KR k-blocks (8 KB of INT4 codes
// at T * KR = 8), a workgroup of W waves covers W * KR k-blocks and `splits`
// workgroups cover K.  Every load of a wave is issued before its first wait, so
// the launch is one memory round trip per wave; the table aims for ~8 blocks
// per wave and enough workgroups to cover all 256 CUs, and avoids a K split
// (which costs a partials round trip and a counter-clearing launch) unless N
// alone gives too few workgroups.
// m: the dense call's rows (0 for MoE and batch-invariant dispatch, whose
// choice must not depend on them).
static Variant skinny_for(const qg_layer_desc &d, int n_tiles, int k_blocks, int64_t m_tiles, int64_t m = 0) {
  const bool mx = mx_a8(d) || mx_a4(d) || mx_tok(d);
  // T x KR per wave: 4 x 2 (integer formats), 2 x 4 (MX), 2 x 2 (1-, 2-,
  // 8-bit integers, e4m3 weights, W8A8); fewer for short K.
  // Measured on the decode shapes: fewer, fuller workgroups beat more, emptier
  // ones (224 workgroups of 8 KB waves beat 448 of 4 KB), so T shrinks only
  // when N alone would leave more than half of the CUs idle.
  const bool narrow = ext_a16(d) || w8a8(d);
  int T = mx || narrow ? 2 : 4, KR = mx ? 4 : 2;
  const bool mx8 = mx_a8(d) || mx_tok(d), int_a16 = !mx && !narrow && !fp4_a16(d);
  int pass_cap = 0;  // the few-row two-pass rules' waves per workgroup
  if (w8a8(d) && m >= 1 && m <= 8) {
    // W8A8 up to 8 rows: one n-tile of 4 blocks per wave (one row: 14336 x
    // 4096 15.1 against 17.9 us, 28672 x 4096 24.5 against 33.6, 4096 x
    // 14336 18.0 against 19.5; at 16 rows no gain); K of 4096 to 8191: 2
    // blocks in two passes of 8 waves (14336 x 4096 at one row 14.6
    // against 15.0, 28672 x 4096 at 8 rows 28.9 against 30.1)
    T = 1;
    KR = 4;
    if (k_blocks >= 32 && k_blocks < 64) {
      KR = 2;
      pass_cap = 8;
    }
  } else if (mx8 && k_blocks <= 32 && n_tiles >= 800 && (m >= 4 || (m >= 1 && n_tiles > 1024 && k_blocks >= 32))) {
    // MX activations from 4 rows, K <= 4096 over many columns: four n-tiles
    // of 2 blocks per wave, 16 waves (14336 x 4096 at 16 rows: 10.3 against
    // 12.1 us per-token, 10.8 against 13.3 MXFP8; at 4 rows 3-8 % less);
    // beyond 16384 columns, from one row, two passes of 8 waves (28672 x
    // 4096 per-token at 4 rows 15.3 against 17.8, at one row 15.0 against
    // 16.4; MXFP8 at 16 rows 18.3 against 20.5)
    T = 4;
    KR = 2;
    if (n_tiles > 1024 && k_blocks >= 32) pass_cap = 8;
  } else if (mx8 && m == 1 && (k_blocks == 32 || k_blocks > 64)) {
    // MX activations at one row over K = 4096 or K > 8192: 2 n-tiles of 2
    // blocks in two passes of up to 8 waves (14336 x 4096 per-token 8.9
    // against 9.5 us, 4096 x 14336 10.7 against 11.4; at K = 8192 one pass
    // of 16 waves needs no K split and stays faster, 10.2 against 10.6)
    T = 2;
    KR = 2;
    pass_cap = 8;
  }
  // dense launches over K >= 4096 of several 16-row tiles (W8A8 from 9
  // rows): each wave walks its K range in two passes (see below)
  bool two_pass = pass_cap > 0 || (k_blocks >= 32 && (w8a8(d) ? m > 8 : (mx8 || int_a16) && m > 16));
  if (two_pass && mx8 && !pass_cap) {
    T = 4;
    KR = 2;
  }
  // UINT4 (zero points) in two passes up to 32 rows: 2 n-tiles per wave
  // (24 rows of 14336 x 4096: 23.1 against 26.0 us, 8192 x 8192 28.6
  // against 30.9; from 64 rows four tiles are as fast or faster)
  if (two_pass && d.wtype == QG_W_UINT4 && m <= 32) T = 2;
  while (KR > 1 && KR > k_blocks) KR /= 2;
  const bool long_k = (k_blocks + KR - 1) / KR > 16;  // K gets split anyway
  while (!long_k && T > 1 && (int64_t)((n_tiles + T - 1) / T) * m_tiles < 128) T /= 2;
  KR = clamp_kr(d, T, KR);
  Variant v{0, T, KR, 1, 1, 0, 0};
  const int64_t n_blocks = (n_tiles + T - 1) / T;
  const int waves_k = (k_blocks + KR - 1) / KR;
  int splits = 1;
  // split K when the workgroup would exceed 16 waves, or when N alone gives
  // fewer than 128 workgroups and each split keeps >= 4 waves
  while (splits < waves_k &&
         ((waves_k + splits - 1) / splits > 16 ||
          (n_blocks * m_tiles * splits < 128 && waves_k / (splits + 1) >= 4)))
    ++splits;
  // W8A8 up to 8 rows over K of 16 waves or more: two K passes where N
  // gives 128 column blocks (4096 x 14336 at one row: 15.7 against 18.9 us
  // for one pass of 14 waves x 2 splits; 8192 x 8192 15.5 against 17.9 for
  // one pass of 16 waves), else beyond 16 waves 4 waves per split, at most
  // 8 splits (1024 x 28672: 10.5 us)
  if (w8a8(d) && m >= 1 && m <= 8 && waves_k >= 16) {
    if (n_blocks >= 128) two_pass = true;
    else if (waves_k > 16) splits = std::max(splits, std::min(8, (waves_k + 3) / 4));
  }
  v.W = (waves_k + splits - 1) / splits;
  v.splits = (waves_k + v.W - 1) / v.W;
  if (two_pass) {
    // Each wave accumulates its two passes in registers, leaving fewer
    // partials to reduce and fewer, fuller workgroups; the waves per
    // workgroup shrink as the rows grow (the rest of K splits across
    // workgroups).  Autotune sweeps over 4096 x 14336, 8192 x 8192 and
    // 14336 x 4096: MXFP8 8192 x 8192 at 32 rows 16.7 against 25.1 us for
    // one pass over 4 waves x 4 splits, 4096 x 14336 at 128 rows 45.6
    // against 70.6 on the tiled kernel; W4A16 8192 x 8192 at 64 rows 40.4
    // against 51.2, 4096 x 14336 at 128 rows 66.3 against 94.0; W8A8 14336 x
    // 4096 at 16 rows 18.6 against 20.9
    const int w_cap = pass_cap ? pass_cap
                      : mx8 ? (m <= 32 ? 16 : m <= 64 ? 8 : 4)
                      : w8a8(d) ? (m <= 16 ? 8 : m <= 32 ? 16 : 4)
                                : (m <= 64 ? 8 : 4);
    const int per = (waves_k + 1) / 2;
    const int sp = (per + w_cap - 1) / w_cap;
    v.W = (per + sp - 1) / sp;
    v.splits = (per + v.W - 1) / v.W;
  }
  // a cross-workgroup split needs one arrival counter per output tile in the
  // workspace's counter prefix; past that the workgroup loops over K instead
  if (v.splits > 1 && n_blocks * m_tiles > kMaxSplitCounters) {
    v.KR = clamp_kr(d, v.T, 4);
    v.W = std::min(16, (k_blocks + v.KR - 1) / v.KR);
    v.splits = 1;
  }
  return v;
}

// Split-K arrival counters of a dense launch (one per output tile), or 0.
static int64_t split_counters(const qg_weight &w, const Variant &v, int64_t m) {
  if (v.splits <= 1) return 0;
  if (v.kind == 4) return (w.n_tiles + v.W - 1) / v.W;  // wide decode: one per column group
  const int64_t n_blocks = (w.n_tiles + v.T - 1) / v.T;
  return v.kind == 3 ? n_blocks : ((m + 15) / 16) * n_blocks;
}

static void sanitize(const qg_layer_desc &d, Variant *v) {
  if (!variant_ok(d, v->T, v->KR)) v->KR = clamp_kr(d, v->T, v->KR);
  if (!variant_ok(d, v->T, v->KR)) v->T = 1;
}

// Large M: the LDS-tiled kernels, scaled MFMA for MX (BM x 256 tiles, from
// M = 128) and bf16 MFMA for the integer formats (BM x 128 tiles, from M = 256,
// where the 16-row skinny kernel stops being weight-bound).
// Columns of the MX tiled kernel's workgroup tile.  One workgroup runs per CU
// (the LDS ring fills it), so the tile count should fill whole rounds of the
// 256 CUs: among 256, 224 and 192 columns take the one with the best
// (round fill x column fill), discounted 3% per 32 columns below 256 for the
// lower reuse of the activation tile.  QG_MX_BN overrides.
static int mx_tile_cols(int64_t n, int64_t m, int bm) {
  if (mx_tiled_waves() != 8) return 256;  // the 4-wave form is built for 256 only
  if (ov().mx_bn) return ov().mx_bn;
  constexpr int kCus = kNumCUs;
  const int64_t m_tiles = (m + bm - 1) / bm;
  int best = 256;
  double best_eff = 0.0;
  for (int bn : {256, 224, 192}) {
    const int64_t n_groups = (n + bn - 1) / bn;
    const int64_t tiles = m_tiles * n_groups;
    const int64_t rounds = (tiles + kCus - 1) / kCus;
    const double eff = (double)tiles / (double)(rounds * kCus) * (double)n / (double)(n_groups * bn) *
                       (1.0 - 0.03 * (256 - bn) / 32);
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = bn;
    }
  }
  return best;
}

// Tile shape of a dense tiled launch (mx: the MX / W8A8 kernel, else the
// integer-format kernel) for M >= 128, or any M for W4A4.
static Variant tiled_shape(const qg_weight &w, int64_t m, bool mx) {
  const bool w8 = w8a8(w.desc);
  if (ov().tiled_bm || ov().mx_bn || ov().a16_bn || ov().mx_waves || ov().a16_waves) {
    // explicit tile or wave overrides: 256-row tiles from 256 rows (integer
    // formats: 128 x 256, or QG_TILED_BM rows x 128 with QG_A16_BN=128)
    int bm = m >= 256 ? 256 : 128;
    if (ov().tiled_bm) bm = ov().tiled_bm;
    int bn = 128;
    if (!mx && a16_tiled_bn() == 256 && m >= 256) {
      bm = 128;
      bn = 256;
    }
    return Variant{mx ? 1 : 2, 1, 1, 1, 1, bm, w8 ? 128 : mx ? mx_tile_cols(w.desc.n, m, bm) : bn};
  }
  // The larger tile (256 rows for MX and W8A8, 128 x 256 for the integer
  // formats, from 256 rows) halves the re-reads of one operand and wins
  // once the tiles fill the CUs (M = 4096); over fewer tiles than CUs the
  // 128-row (128 x 128) tile doubles the workgroups.  Cost: rounds of 256
  // CUs (one workgroup each) times the tile's area, the smaller tile's
  // taken dearer for its lower reuse: 15 % (MX, W8A8), 40 % (integer
  // formats, whose 128 x 256 tile also unpacks each code for fewer waves;
  // 3072 x 4096 at M = 4096: 128.2 us in two rounds of 128 x 256 against
  // 140.2 in three of 128 x 128).  Autotune sweeps at 256 to 4096 rows:
  // W4A8 per-token 4096 x 14336 at 256 rows 70.9 against 118.2 us, 14336 x
  // 4096 24.1 against 39.1; W8A8 8192 x 8192 56.6 against 90.5, 3072 x 4096
  // at M = 4096 BM = 128; W4A16 8192 x 8192 95.2 against 126.4, 14336 x
  // 4096 at 384 rows and above keeping 128 x 256.
  auto cost = [&](int tbm, int tbn, bool small) {
    const int64_t tiles = ((m + tbm - 1) / tbm) * ((w.desc.n + tbn - 1) / tbn);
    return (double)((tiles + kNumCUs - 1) / kNumCUs) * tbm * tbn * (small ? (mx ? 1.15 : 1.4) : 1.0);
  };
  // (W8A8: 128-column tiles, the only width its 2-KB weight blocks fit)
  int bm = 128, bn = w8 ? 128 : mx ? mx_tile_cols(w.desc.n, m, 128) : 128;
  if (m >= 256) {
    const int bm2 = mx ? 256 : 128, bn2 = w8 ? 128 : mx ? mx_tile_cols(w.desc.n, m, 256) : 256;
    if (cost(bm2, bn2, false) <= cost(bm, bn, true)) {
      bm = bm2;
      bn = bn2;
    }
  }
  return Variant{mx ? 1 : 2, 1, 1, 1, 1, bm, bn};
}

static bool tiled_for(const qg_weight &w, int64_t m, Variant *v) {
  if (w.desc.k % 128 != 0 || !has_tiled(w.desc)) return false;
  if (ov().tiled_off) return false;
  const bool mx = mx_tiled_fmt(w.desc);
  // the integer-format kernel addresses X and the codes with 32-bit offsets
  if (!mx && ((uint64_t)m * w.desc.k * 2 >= (1ull << 31) ||
              (uint64_t)w.n_tiles * w.k_blocks * 1024 >= (1ull << 31)))
    return false;
  // (W4A4 has only the MX tiled kernel, which serves every M)
  if (m < (mx_a4(w.desc) ? 1 : mx ? 128 : 384)) {
    // MX and W8A8 below 128 rows: the skinny kernel streams the weights
    // once per 16 rows, the tiled kernel once, so where N gives enough
    // 128-row tiles the tiled kernel wins from a few dozen rows (W8A8 14336
    // x 4096 at 32 rows: 29.5 against 39.5 us, 28672 x 4096 at 16 rows: 30.4
    // against 39.6; W4A8 14336 x 4096 at 64 rows: 23.6 against 35.3, 28672
    // x 4096 at 32 rows: 23.9 against 35.9; 8192 x 8192 and 4096 x 14336,
    // with fewer tiles, stay on the skinny kernel's K splits)
    // Integer formats below 384 rows: from 128 rows where N gives 96 or
    // more 128-column tiles, from 192 rows where it gives 64 (W4A16 14336 x
    // 4096 at 128 rows: 49.4 against 78.3 us; 8192 x 8192 at 200 rows 95.1
    // against 117.8, at 128 rows the skinny kernel's two-pass splits win;
    // 4096 x 14336 at 256 rows 121.5 against 161.5 and 3072 x 4096 28.4
    // against 49.0 on them; from 256 rows over K < 4096, where the skinny
    // kernel takes one pass, and from 384 rows the tiled kernel)
    if (!mx) {
      const int64_t tiles = (w.desc.n + 127) / 128;
      if (m < 256 || w.k_blocks >= 32)  // (from 256 rows over K < 4096: tiled)
        if (m < 128 || tiles < 64 || (tiles < 96 && m < 192)) return false;
    } else {
      if (m <= 8) return false;
      const int64_t tbn = w8a8(w.desc) ? 128 : mx_tile_cols(w.desc.n, m, 128);
      const int64_t wgs = (w.desc.n + tbn - 1) / tbn;
      const bool go = w8a8(w.desc) ? (m > 32 && wgs >= 64) || (m > 16 && wgs >= 100) || wgs >= 200
                                   : (m > 32 && wgs >= 64) || (m > 16 && wgs >= 128);
      if (!go) return false;
    }
  } else if (mx && !mx_a4(w.desc) && !w8a8(w.desc) && m < 256 && w.k_blocks >= 32 &&
             (w.desc.n + mx_tile_cols(w.desc.n, m, 128) - 1) / mx_tile_cols(w.desc.n, m, 128) < 32) {
    // MX from 128 rows over fewer than 32 column tiles and K >= 4096: the
    // tiled kernel leaves most CUs idle, the skinny kernel's two-pass K
    // splits fill them
    // (4096 x 14336 at 128 rows: 45.6 against 70.6 us per-token, 52.2
    // against 73.4 MXFP8; 8192 x 8192, 43 tiles, stays tiled)
    return false;
  }
  *v = tiled_shape(w, m, mx);
  return true;
}

// Dense decode kernel (integer formats, M <= 16, K % 512 == 0): the rows sit
// in LDS and one workgroup covers all of K (or half of it for long K over few
// column tiles, combined through the workspace).  (T, KR) pairs
// compiled: (4, 2), (2, 4), (1, 4), (1, 8), (2, 8) for group 128, the first
// two for group 64 (group 32 stays on the skinny kernel);
// W = ceil(k_blocks / (KR * splits)) <= 16.  QG_DECODE="T,KR[,splits]" picks
// one, "0" disables the kernel.
static bool decode_fits(const qg_weight &w, int64_t m, int T, int KR, int S, Variant *v) {
  const int g = w.desc.group_size;
  if (!decode_capable(w.desc)) return false;
  // (1-, 2-, 8-bit integers and e4m3 weights: T = 1, KR = 4 or 8)
  const bool compiled = ext_a16(w.desc) ? (T == 1 && (KR == 4 || KR == 8))
                        : (g == 32 && T == 1 && (KR == 4 || KR == 8)) ||
                              (!fp4_a16(w.desc) &&
                               ((g == 128 && ((T == 4 && KR == 2) || (T == 4 && KR == 4) || (T == 2 && KR == 4) || (T == 1 && KR == 4) ||
                                              (T == 1 && KR == 8) || (T == 2 && KR == 8))) ||
                                (g == 64 && ((T == 4 && KR == 2) || (T == 2 && KR == 4)))));
  if (!compiled || S < 1 || S > 8) return false;
  const int kbs = w.k_blocks;
  const int W = (kbs + KR * S - 1) / (KR * S);
  if (W > 16 || W < 1) return false;
  // splits: each starts inside K and copies whole 512-value chunks
  if (S > 1 && ((W * KR) % 4 != 0 || (S - 1) * W * KR >= kbs)) return false;
  const int gpb = 128 / w.desc.group_size;
  if ((int64_t)W * KR * S * gpb > w.groups_padded) return false;  // scale reads stay in the row
  if (S > 1 && (w.n_tiles + T - 1) / T > kMaxSplitCounters) return false;  // one counter per column block
  if (decode_lds_bytes(m, W, T, KR) > 160 * 1024 - 256) return false;  // (+ the kernel's static LDS)
  *v = Variant{3, T, KR, W, S, 0, 0};
  return true;
}

// Rounds of resident workgroups a decode launch takes: a CU holds as many
// workgroups as its LDS (160 KB) and its waves allow; the waves per CU follow
// the instances' registers (T * KR = 16: ~124 VGPRs, 4 waves per SIMD; the
// others up to 90, 5 to 8 waves per SIMD, taken as 7).
static int64_t decode_rounds(const qg_weight &w, int64_t m, const Variant &v) {
  const uint64_t lds = decode_lds_bytes(m, v.W, v.T, v.KR) + 256;
  int64_t per_cu = (int64_t)((160 * 1024) / lds);
  per_cu = std::min<int64_t>(per_cu, (v.T * v.KR >= 16 ? 16 : 28) / v.W);
  if (per_cu < 1) per_cu = 1;
  const int64_t wgs = (int64_t)((w.n_tiles + v.T - 1) / v.T) * v.splits;
  return (wgs + kNumCUs * per_cu - 1) / (kNumCUs * per_cu);
}

// Wide decode form (2 .. 16 rows, K % 512 == 0): W waves along N, one K slice
// of KR blocks per workgroup, ceil(K / (KR * 128)) slices.  Instances: KR 8 or
// 16 for the decode-capable formats and groups, KR 8 only for the 8-bit
// slices (e4m3 and 8-bit integers: 16 blocks of them in flight spill).
static bool decode_wide_fits(const qg_weight &w, int64_t m, int W, int KR, Variant *v) {
  const qg_layer_desc &d = w.desc;
  if (!decode_capable(d) || m < 2 || m > 16 || d.k % 512 != 0 || W < 1 || W > 16 || (KR != 8 && KR != 16))
    return false;
  const int f = kernel_fmt(d);
  if (KR == 16 && (f == 7 || f == 8 || f == 13)) return false;
  // a slice's NG = KR * 128 / group scales are read as one run starting at a
  // multiple of NG, which stays inside the row's padded groups only if NG
  // divides them (always for NG <= 32: the padding is to a multiple of 32)
  const int ng = KR * (128 / d.group_size);
  if (w.groups_padded % ng != 0) return false;
  if (fp4_a16(d) && d.group_size != 32) return false;
  const int S = (w.k_blocks + KR - 1) / KR;
  if (S > 1 && (w.n_tiles + W - 1) / W > kMaxSplitCounters) return false;
  *v = Variant{4, 1, KR, W, S, 0, 0};
  return true;
}

// The wide form's K slice: 16 blocks, or 8 where K has at most 64 blocks, so
// that 4 slices do not leave one workgroup of 8 waves per CU (8192 x 8192,
// INT4 at M = 16: 11.4 against 12.7 us; 4096 x 14336, 7 slices of 16: 10.7
// against 14 slices of 8, slower).
static bool decode_wide_pick(const qg_weight &w, int64_t m, Variant *v) {
  if (w.k_blocks <= 64 && decode_wide_fits(w, m, 8, 8, v)) return true;
  return decode_wide_fits(w, m, 8, 16, v) || decode_wide_fits(w, m, 8, 8, v);
}

static bool decode_for(const qg_weight &w, int64_t m, Variant *v) {
  const qg_layer_desc &d = w.desc;
  if (!decode_capable(d) || m < 1 || m > 16 || d.k % 512 != 0) return false;
  const Overrides &o = ov();
  if (o.decode_off) return false;
  if (o.decode_n >= 2) return decode_fits(w, m, o.decode_v[0], o.decode_v[1], o.decode_v[2], v);
  if (o.wide == 1) return decode_wide_fits(w, m, o.wide_v[0], o.wide_v[1], v);
  // Measured on the decode shapes (N x K = 14336 x 4096 and 4096 x 14336,
  // UINT4 and INT3, M = 1 .. 16): at one row one n-tile and 8 k-blocks per
  // wave wins; from two rows two n-tiles of 4 k-blocks (the activation
  // fragments read from LDS serve both tiles: 14336 x 4096 at M = 8 9.6 us
  // against 12.1 us, at M = 16 12.6 against 17.9 us for the skinny kernel)
  // wherever N gives enough workgroups; rows that do not fit LDS over all of
  // K take a K split in two (4096 x 14336 at M = 8: 14.7 against 20.8 us on
  // the skinny kernel), else the skinny kernel.
  // 1-, 2- and 8-bit integer and e4m3 weights run one n-tile per decode
  // workgroup, which copies its rows for every tile: from 8 rows (9 for the
  // 8-bit slices) the wide form wins (14336 x 4096 at M = 16: UINT2 10.8
  // against 19.9 us, INT8 18.5 against 24.8 us; at M = 8 UINT2 10.3 against
  // 11.2 us, INT8 17.9 against 17.0 us)
  if (ext_a16(d)) {
    const int f = kernel_fmt(d);
    const bool bits8 = f == 7 || f == 8 || f == 13;
    if (m >= (bits8 ? 9 : 8) && decode_wide_fits(w, m, bits8 ? 4 : 8, 8, v)) return true;
  }
  // Rows that fill more than half of a CU's LDS leave one two-tile workgroup
  // per CU, and more such workgroups than CUs run in two rounds; four tiles
  // per workgroup take fewer rounds, each row copy serving twice the columns
  // (14336 x 4096 at M = 16: 11.1 against 12.9 us; at M = 8, where two
  // two-tile workgroups share a CU and one round covers N, 10.3 against 9.8)
  if (!ext_a16(d) && m > 1) {
    Variant v2, v4;
    if (decode_fits(w, m, 2, 4, 1, &v2) && decode_fits(w, m, 4, 4, 1, &v4) &&
        decode_rounds(w, m, v4) < decode_rounds(w, m, v2)) {
      *v = v4;
      return true;
    }
  }
  // INT3 (3-bit, no zero points) at one row: two n-tiles of 8 blocks per wave
  // while that leaves 200 to 512 workgroups (14336 x 4096: 6.75 against 7.00
  // us; 8192 x 8192: 6.83 against 7.10; 28672 x 4096, 896 workgroups: 10.7
  // against 10.0 us for one n-tile; UINT3 and the 4-bit formats: no gain)
  if (m == 1 && d.wtype == QG_W_INT3) {
    const int64_t wgs = (w.n_tiles + 1) / 2;
    if (wgs >= 200 && wgs <= 512 && decode_fits(w, m, 2, 8, 1, v)) return true;
  }
  static const int pairs_one[][2] = {{1, 8}, {2, 4}, {2, 8}, {4, 2}};
  static const int pairs_rows[][2] = {{2, 4}, {1, 8}, {2, 8}, {4, 2}};
  static const int pairs_ext[][2] = {{1, 8}, {1, 4}, {1, 4}, {1, 4}};
  const int kbs = w.k_blocks;
  for (const auto &p : ext_a16(d) ? pairs_ext : m == 1 ? pairs_one : pairs_rows) {
    if ((kbs + p[1] - 1) / p[1] > 16) continue;
    if ((w.n_tiles + p[0] - 1) / p[0] < 200 && p[0] > 1) continue;
    if (decode_fits(w, m, p[0], p[1], 1, v)) {
      // a K split only when the column tiles leave CUs idle: the split's
      // partial round trip (store, counter, reload) costs about 1.5 us
      // (4096 x 14336 at M = 1: 7.9 us in one workgroup per tile, 9.4 us
      // with two K halves)
      Variant s;
      if ((w.n_tiles + v->T - 1) / v->T < 192 && v->W > 8 && decode_fits(w, m, v->T, v->KR, 2, &s)) *v = s;
      return true;
    }
    // rows too long for LDS over all of K: the wide form, which copies each
    // K slice once per 8 column tiles (4096 x 14336, UINT4: 10.6 us at M = 8
    // against 14.1 us for two K halves in this form, 11.3 us at M = 16
    // against 20.6 us on the skinny kernel), else K halves
    if (m > 1 && decode_wide_pick(w, m, v)) return true;
    if (m > 1 && decode_fits(w, m, p[0], p[1], 2, v)) return true;
  }
  return m > 1 && decode_wide_pick(w, m, v);
}

// Batch-invariant dispatch: the variant depends on (N, K) only, so each
// output row is reduced over K in one fixed order whatever M is.  The tiled
// kernels (K % 128 == 0) sum every element in K-step order with a per-element
// MFMA chain independent of the tile's position; the skinny kernel with a
// variant fixed by (N, K) sums its waves' and splits' partials in index order.
// Tile widths do not change any element's order; they are fixed anyway.
static Variant select_dense_invariant(const qg_weight &w) {
  const bool mx = mx_tiled_fmt(w.desc);  // (W4A4 layers have K % 128 == 0)
  if (has_tiled(w.desc) && w.desc.k % 128 == 0 &&
      (mx || (uint64_t)w.n_tiles * w.k_blocks * 1024 < (1ull << 31))) {
    const int bn = w8a8(w.desc) ? 128 : mx ? 256 : a16_tiled_bn();
    return Variant{mx ? 1 : 2, 1, 1, 1, 1, (mx || bn == 256) ? 128 : 256, bn};
  }
  // the skinny kernel with the workgroup looping over K: the reduction order
  // (passes in K order per wave, then the waves in index order) depends on
  // (N, K) only
  Variant v = skinny_for(w.desc, w.n_tiles, w.k_blocks, 1);
  if (v.splits > 1) {
    v.W = std::min(16, (w.k_blocks + v.KR - 1) / v.KR);
    v.splits = 1;
  }
  return v;
}

// ---------------------------------------------------------------------------
// Autotune table (announcement, "Future plans": benchmark candidate
// configurations on the target device to find better execution parameters
// per workload, complementing the heuristics).  qg_gemm_autotune times the
// candidates of one (layer, M) and keeps the fastest here, per layer shape and
// M bucket; select_dense consults it before its heuristics.
// ---------------------------------------------------------------------------
namespace {
struct TuneEntry {
  int32_t wtype, atype, group, bucket;
  int64_t n, k;
  Variant v;
};
std::mutex g_tune_mu;
std::vector<TuneEntry> g_tune;
}  // namespace

// M buckets of the table: 1, 2-4, 5-8, 9-16, 17-64, 65-256, 257-1024, > 1024
static int m_bucket(int64_t m) {
  static const int64_t edges[] = {1, 4, 8, 16, 64, 256, 1024};
  int b = 0;
  while (b < 7 && m > edges[b]) ++b;
  return b;
}

static bool same_variant(const Variant &a, const Variant &b) {
  return a.kind == b.kind && a.T == b.T && a.KR == b.KR && a.W == b.W && a.splits == b.splits && a.bm == b.bm &&
         a.tbn == b.tbn;
}

// Whether v can serve m rows of w (a table entry serves every M of its bucket)
static bool variant_valid(const qg_weight &w, int64_t m, const Variant &v) {
  const qg_layer_desc &d = w.desc;
  const bool mx = mx_tiled_fmt(d);
  if (mx_a4(d) && v.kind != 1 && v.kind != 0) return false;  // W4A4: the MX tiled or MX skinny kernel
  switch (v.kind) {
    case 0:
      return variant_ok(d, v.T, v.KR) && v.W >= 1 && v.W <= 16 && v.splits >= 1 &&
             split_counters(w, v, m) <= kMaxSplitCounters;
    case 1:
      if (w8a8(d)) return d.k % 128 == 0 && (v.bm == 128 || v.bm == 256) && v.tbn == 128;
      return mx && d.k % 128 == 0 && (v.bm == 128 || v.bm == 256) &&
             (v.tbn == 256 || (mx_tiled_waves() == 8 && (v.tbn == 192 || v.tbn == 224)));
    case 2:
      return !mx && has_tiled(d) && d.k % 128 == 0 && (uint64_t)m * d.k * 2 < (1ull << 31) &&
             (uint64_t)w.n_tiles * w.k_blocks * 1024 < (1ull << 31) &&
             ((v.bm == 128 && v.tbn == 256 && a16_tiled_waves() == 8) || ((v.bm == 128 || v.bm == 256) && v.tbn == 128));
    case 3: {
      Variant t;
      return !mx && m >= 1 && m <= 16 && d.k % 512 == 0 && decode_fits(w, m, v.T, v.KR, v.splits, &t) && t.W == v.W;
    }
    case 4: {
      Variant t;
      return decode_wide_fits(w, m, v.W, v.KR, &t) && t.splits == v.splits;
    }
  }
  return false;
}

static bool tuned_lookup(const qg_weight &w, int64_t m, Variant *v) {
  std::lock_guard<std::mutex> lock(g_tune_mu);
  const int b = m_bucket(m);
  for (const TuneEntry &e : g_tune)
    if (e.wtype == w.desc.wtype && e.atype == w.desc.atype && e.group == w.desc.group_size && e.n == w.desc.n &&
        e.k == w.desc.k && e.bucket == b) {
      if (!variant_valid(w, m, e.v)) return false;
      *v = e.v;
      return true;
    }
  return false;
}

static void tuned_store(const qg_weight &w, int64_t m, const Variant &v) {
  std::lock_guard<std::mutex> lock(g_tune_mu);
  const int b = m_bucket(m);
  for (TuneEntry &e : g_tune)
    if (e.wtype == w.desc.wtype && e.atype == w.desc.atype && e.group == w.desc.group_size && e.n == w.desc.n &&
        e.k == w.desc.k && e.bucket == b) {
      e.v = v;
      return;
    }
  g_tune.push_back(TuneEntry{w.desc.wtype, w.desc.atype, w.desc.group_size, b, w.desc.n, w.desc.k, v});
}

static Variant select_dense_heuristic(const qg_weight &w, int64_t m);

Variant select_dense(const qg_weight &w, int64_t m) {
  Variant v;
  // experiment overrides win over the table
  const Overrides &o = ov();
  if (!o.tune && !o.decode_off && o.decode_n == 0 && !o.tiled_set && tuned_lookup(w, m, &v)) return v;
  return select_dense_heuristic(w, m);
}

static Variant select_dense_heuristic(const qg_weight &w, int64_t m) {
  Variant v;
  if (mx_a4(w.desc)) {
    // from 128 rows the tiled kernel with e2m1 operands; below, the MX skinny
    // kernel, which widens each e2m1 fragment exactly to e4m3 in registers
    if (m >= 128 && !ov().tiled_off) return tiled_shape(w, m, true);
    if (env_variant(&v)) {
      sanitize(w.desc, &v);
      if (split_counters(w, v, m) > kMaxSplitCounters) v.splits = 1;
      return v;
    }
    return skinny_for(w.desc, w.n_tiles, w.k_blocks, (m + 15) / 16, m);
  }
  if (tiled_for(w, m, &v)) return v;
  if (!ov().tune && decode_for(w, m, &v)) return v;
  if (env_variant(&v)) {
    sanitize(w.desc, &v);
    // (K beyond W * KR * splits blocks: the workgroups loop over K)
    if (split_counters(w, v, m) > kMaxSplitCounters) v.splits = 1;
    return v;
  }
  const int64_t m_tiles = (m + 15) / 16;
  return skinny_for(w.desc, w.n_tiles, w.k_blocks, m_tiles, m);
}

Variant select_moe(const qg_weight &w, int64_t pairs) {
  Variant v;
  if (env_variant(&v)) {
    sanitize(w.desc, &v);
    v.splits = 1;
    return v;
  }
  // the grouped kernel keeps K inside one workgroup (no cross-workgroup
  // split); past W waves of KR blocks the workgroup loops over K
  const qg_layer_desc &d = w.desc;
  if (!mx_a8(d) && !mx_a4(d) && !mx_tok(d) && !ext_a16(d) && !w8a8(d)) {
    // 4- and 3-bit integers, MXFP4 x bf16: four n-tiles of 2 blocks, 4
    // waves, looping over K; the persistent grid then holds 4x the
    // workgroups of 16-wave ones (E = 256 top-8, 4096 x 7168 gate_up at T =
    // 1: 31.8 against 58.9 us for (1, 4) over 14 waves, at T = 16 144
    // against 329, MXFP4 x bf16 138 against 321; 7168 x 2048 down at T = 16
    // 80.0 against 90.2 for (4, 2) over 8 waves)
    const int kr = clamp_kr(d, 4, 2);
    return Variant{0, 4, kr, std::max(1, std::min(4, (w.k_blocks + kr - 1) / kr)), 1, 0, 0};
  }
  if (w8a8(d) && w.k_blocks > 8) {
    // W8A8 over K > 1024: 4 waves looping over K, one n-tile of 4 blocks
    // below 64 pairs, two of 2 from 64 (E = 128 top-8, 1280 x 4096 gate_up
    // at T = 1: 15.0 against 16.9 us for one pass over 16 waves; at T = 16
    // 47.4 against 62.2)
    const int t = pairs >= 64 ? 2 : 1, kr = clamp_kr(d, t, pairs >= 64 ? 2 : 4);
    return Variant{0, t, kr, std::max(1, std::min(4, (w.k_blocks + kr - 1) / kr)), 1, 0, 0};
  }
  if (mx_a8(d) || mx_tok(d)) {
    // MXFP8 and per-token activations: two n-tiles of 2 blocks, 4 waves,
    // looping over K (E = 128 top-8 W4A8, 1280 x 4096 gate_up at T = 1:
    // 11.1 against 11.9 us; 4096 x 640 down at T = 64: 24.7 against 25.5)
    // From 64 pairs over K <= 1024 (8 blocks): four n-tiles on 2 waves
    // (4096 x 640 down at T = 8: 15.3 against 18.6 us, T = 31 26.1 against
    // 33.3, per-token at T = 16 21.9 against 24.6)
    const bool short_k = pairs >= 64 && w.k_blocks <= 8;
    const int t = short_k ? 4 : 2, kr = clamp_kr(d, t, 2);
    return Variant{0, t, kr, std::max(1, std::min(short_k ? 2 : 4, (w.k_blocks + kr - 1) / kr)), 1, 0, 0};
  }
  const int64_t m_tiles = std::max<int64_t>(1, (pairs + 15) / 16);
  Variant s = skinny_for(w.desc, w.n_tiles, w.k_blocks, m_tiles);
  if (s.splits > 1 || (int64_t)s.W * s.KR < w.k_blocks) {
    // long K: the deepest spill-free wave (KR = 4), T reduced to fit
    s.T = (mx_a8(w.desc) || mx_tok(w.desc)) ? 2 : 1;
    s.KR = clamp_kr(w.desc, s.T, 4);
    s.W = std::min(16, (w.k_blocks + s.KR - 1) / s.KR);
    s.splits = 1;
  }
  return s;
}

// MoE: experts with at least this many rows go to the tiled kernels (128-row
// tiles); the rest to the small-tile form of the integer formats' tiled kernel
// or (MXFP4) to the skinny kernel; 0 = skinny only.  QG_MOE_TILED_MIN
// overrides (0 disables the tiled kernels).
static bool moe_small_tiles(const qg_weight &w, int64_t pairs, int min_rows);

// Whether the tiled kernels can serve this MoE call at all.
static bool moe_tiled_ok(const qg_weight &w, int64_t x_rows_count) {
  const qg_layer_desc &d = w.desc;
  if (d.k % 128 != 0 || d.num_experts > kMaxExperts || !has_tiled(d)) return false;
  const bool mx = mx_a8(d) || mx_tok(d) || w8a8(d);  // one byte per activation element
  // 32-bit offsets inside the kernels
  return (uint64_t)x_rows_count * d.k * (mx ? 1 : 2) < (1ull << 31) &&
         (uint64_t)w.n_tiles * w.k_blocks * 1024 < (1ull << 31);
}

static int moe_tiled_min_rows(const qg_weight &w, int64_t pairs, int64_t x_rows_count) {
  if (!moe_tiled_ok(w, x_rows_count)) return 0;
  int min_rows = 64;
  const qg_layer_desc &d = w.desc;
  if (ov().moe_tiled_min >= 0) {
    min_rows = ov().moe_tiled_min;
  } else if (pairs < 256 && !mx_a4(d) && !ext_a16(d) && !fp4_a16(d) && !w8a8(d)) {
    // 4- and 3-bit integers, MXFP8 and per-token activations below 256
    // pairs: every expert on the skinny kernel's 4-wave launch, a hot
    // expert's 64+ rows included (E = 256 top-8 W4A16, 4096 x 7168 gate_up
    // at T = 16: 122 against 140 us with that expert on 128-row tiles; E =
    // 128 top-8 W4A8 gate_up + down at T = 31 69.9 against 78.2, per-token
    // at T = 16 49.4 against 58.0)
    return 0;
  }
  if (min_rows <= 0) return 0;
  // no expert can reach the threshold: all go to the small-tile form
  // (integer formats) or the skinny kernel
  if (pairs < min_rows && !moe_small_tiles(w, pairs, min_rows)) return 0;
  return min_rows;
}

// Waves of the MX tiled kernel: 8 (two per SIMD, wave tile 64 x 128) keeps
// the matrix core fed while the other wave of the SIMD waits on LDS reads or
// the stage barrier; measured 1.3x faster than 4 at M = 4096.
int mx_tiled_waves() {
  return ov().mx_waves ? ov().mx_waves : 8;
}

// Waves of the integer-format tiled kernel: 8 (4 x 2, two per SIMD, wave
// tile (BM / 4) x 64) hides one wave's waits behind the other's MFMAs and
// dequantization; measured 1.15-1.25x faster than 4 at M = 4096.
int a16_tiled_waves() {
  return ov().a16_waves ? ov().a16_waves : 8;
}

// Columns of the integer-format tiled kernel's tile: 256 (with 128 rows, 2 x 4
// waves) moves fewer activation bytes per flop than 256 x 128 and unpacks
// each code for 2 waves instead of 4; measured 1.03-1.08x at M = 4096.
// QG_A16_BN=128 keeps 128 columns (then QG_TILED_BM picks the rows).
int a16_tiled_bn() {
  if (a16_tiled_waves() != 8) return 128;
  return ov().a16_bn == 128 ? 128 : 256;
}

// Raster group of the tiled MoE launches (QG_MOE_GROUP_M overrides).
// Columns of the MX tiled kernel's 128-row MoE tiles: 128.  A 128 x 128 tile
// needs half the LDS of a 128 x 256 one and under 100 VGPRs per lane, so two
// workgroups share a CU and one tile's ring fill and output store overlap the
// other's MFMAs (E = 128 top-8 W4A8 at T = 4096: gate_up 231 against 252 us,
// down 268 against 272 us; T = 512 down 69.6 against 76.7 us).  W8A8 has only
// the 128-column form.  QG_MOE_MX_BN = 256 selects the wide tiles.
static int moe_mx_bn(const qg_weight &w) {
  if (w8a8(w.desc)) return 128;
  if (ov().moe_mx_bn) return ov().moe_mx_bn;
  return 128;
}

static int moe_group_m() {
  return ov().moe_group_m ? ov().moe_group_m : 1;
}

// Tile-list capacity: one tile per 128 rows plus one partial tile per expert
// that has tiles (at most pairs / min_rows of them).
static int64_t moe_tiles_cap(const qg_weight &w, int64_t pairs, int min_rows) {
  return pairs / kMoeTileRows + std::min<int64_t>(w.desc.num_experts, pairs / min_rows) + 1;
}

// Rows of the small tiles: 64, or 32 (QG_MOE_SMALL_BM).
static int moe_small_bm() {
  return ov().moe_small_bm == 32 ? 32 : kMoeSmallTileRows;
}

// Small-tile list capacity (experts with 1 .. min_rows - 1 rows): one tile per
// small-tile rows plus one partial tile per such expert.
static int64_t moe_small_tiles_cap(const qg_weight &w, int64_t pairs) {
  return pairs / moe_small_bm() + std::min<int64_t>(w.desc.num_experts, pairs) + 1;
}

// Experts below the tiled threshold run the tiled kernels' small-tile form
// (one pass over the expert's weights for all of its rows, through the same
// deep LDS ring) instead of the skinny kernel, which re-reads the weights per
// 16 rows and cannot keep enough bytes in flight with one item per workgroup.
// Below 256 pairs (a few tokens) the skinny kernel's K split across waves
// keeps more loads in flight than the few small-tile workgroups, so it stays.
// QG_MOE_SMALL=0 keeps small experts on the skinny kernel, =1 forces the
// small tiles.
static bool moe_small_tiles(const qg_weight &w, int64_t pairs, int min_rows) {
  if (min_rows <= 0) return false;
  if (ov().moe_small >= 0) return ov().moe_small != 0;
  return pairs >= 256;
}

static uint64_t moe_list_bytes(int64_t cap) { return align_up((uint64_t)(2 + 2 * cap) * 4, 256); }

// Autotune limits: timed launches per candidate, and the sink of the cache
// flush reads at the end of an autotune workspace.
constexpr int kTuneMaxReps = 64;
constexpr uint64_t kTuneSinkBytes = 16384;

// The MoE dispatch of one call: experts with >= min_rows rows run the tiled
// kernels' 128-row tiles (min_rows 0: none do), the others the small-tile
// form (small) or the skinny kernel; mx_bn: columns of the MX tiled kernel's
// 128-row tiles.
struct MoePlan {
  int min_rows;
  bool small;
  int mx_bn;
};

// Row threshold of a plan that puts every expert on the small tiles (no
// 128-row tile list or launch).
constexpr int kMoeAllSmall = 1 << 30;

// MoE autotune table (announcement, "Future plans": autotune on the target
// device; here for the grouped GEMM's dispatch): the fastest plan per layer
// shape and pair-count bucket, consulted unless an experiment override of the
// MoE dispatch is set.
namespace {
struct MoeTuneEntry {
  int32_t wtype, atype, group, experts, bucket;
  int64_t n, k;
  MoePlan plan;
};
std::mutex g_moe_tune_mu;
std::vector<MoeTuneEntry> g_moe_tune;
}  // namespace

// pair-count buckets: 1-8, 9-64, 65-512, 513-4096, 4097-32768, more
static int pairs_bucket(int64_t pairs) {
  static const int64_t edges[] = {8, 64, 512, 4096, 32768};
  int b = 0;
  while (b < 5 && pairs > edges[b]) ++b;
  return b;
}

static bool moe_tune_key(const MoeTuneEntry &e, const qg_weight &w, int b) {
  const qg_layer_desc &d = w.desc;
  return e.wtype == d.wtype && e.atype == d.atype && e.group == d.group_size && e.experts == d.num_experts &&
         e.bucket == b && e.n == d.n && e.k == d.k;
}

static bool moe_overridden() {
  return ov().moe_tiled_min >= 0 || ov().moe_small >= 0 || ov().moe_mx_bn != 0;
}

static MoePlan moe_plan(const qg_weight &w, int64_t pairs, int64_t x_rows_count) {
  if (!moe_overridden()) {
    std::lock_guard<std::mutex> lock(g_moe_tune_mu);
    const int b = pairs_bucket(pairs);
    for (const MoeTuneEntry &e : g_moe_tune)
      if (moe_tune_key(e, w, b)) {
        MoePlan p = e.plan;
        if (p.min_rows > 0 && !moe_tiled_ok(w, x_rows_count)) p = MoePlan{0, false, p.mx_bn};
        return p;
      }
  }
  MoePlan p;
  p.min_rows = moe_tiled_min_rows(w, pairs, x_rows_count);
  p.small = moe_small_tiles(w, pairs, p.min_rows);
  p.mx_bn = moe_mx_bn(w);
  return p;
}

// MoE workspace: [tile list][small-tile list][group row sums of X (integer
// formats)]
static uint64_t moe_ws_bytes(const qg_weight &w, int64_t pairs, int64_t x_rows_count, const MoePlan &plan) {
  const int min_rows = plan.min_rows;
  if (min_rows <= 0) return 0;
  uint64_t b = moe_list_bytes(moe_tiles_cap(w, pairs, min_rows));
  if (plan.small) b += moe_list_bytes(moe_small_tiles_cap(w, pairs));
  if (!mx_a8(w.desc) && !mx_tok(w.desc) && !w8a8(w.desc)) b += a16_tiled_ws_bytes(w.desc, x_rows_count);
  return b;
}

static qg_status check_weight(const qg_weight *w, Layout *L) {
  if (!w || !w->data) return QG_ERR_INVALID_ARGUMENT;
  qg_status st = make_layout(&w->desc, L);
  if (st != QG_OK) return st;
  if (w->layout_version != QG_LAYOUT_VERSION) return QG_ERR_INVALID_ARGUMENT;
  if (w->bytes < L->total_bytes) return QG_ERR_BUFFER_TOO_SMALL;
  if (w->n_tiles != L->n_tiles || w->k_blocks != L->k_blocks ||
      w->groups_padded != L->groups_padded || w->expert_stride != L->expert_stride)
    return QG_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)w->data & 255u) != 0) return QG_ERR_ALIGNMENT;
  return QG_OK;
}

static void fill_weight(const qg_layer_desc *d, const Layout &L, void *dev, uint64_t bytes,
                        qg_weight *out) {
  memset(out, 0, sizeof(*out));
  out->desc = *d;
  out->data = dev;
  out->bytes = bytes;
  out->layout_version = QG_LAYOUT_VERSION;
  out->n_tiles = L.n_tiles;
  out->k_blocks = L.k_blocks;
  out->groups_padded = L.groups_padded;
  out->expert_stride = L.expert_stride;
  out->scales_offset = L.scales_offset;
  out->zeros_offset = L.has_zp ? L.zeros_offset : 0;
}

// Dense workspace layout: [split-K arrival counters, kSplitCounterBytes]
// [fp32 partial tiles of a split launch, or the tiled kernels' scratch].
// The counter prefix sits at the same place for every layer and M and is
// never written by anything but the counters, which every split launch
// leaves at zero; so one workspace, zero-filled once, serves any sequence of
// calls on one stream.  Launches that use neither need no workspace.
static uint64_t dense_ws_bytes(const qg_weight &w, const Variant &v, int64_t m) {
  if (m <= 0) return 0;
  if (v.kind == 2) return kSplitCounterBytes + a16_tiled_ws_bytes(w.desc, m);
  if (v.kind == 1) return kSplitCounterBytes + mx_tiled_ws_bytes(m, w.k_blocks);
  if (v.splits <= 1) return 0;
  if (v.kind == 4)  // wide decode: a 16 x 16 partial per wave, slice and column group
    return kSplitCounterBytes + (uint64_t)v.splits * ((w.n_tiles + v.W - 1) / v.W) * v.W * 256 * 4;
  const int64_t m_tiles = v.kind == 3 ? 1 : (m + 15) / 16;
  const int64_t n_blocks = (w.n_tiles + v.T - 1) / v.T;
  return kSplitCounterBytes + (uint64_t)v.splits * m_tiles * n_blocks * (uint64_t)v.T * 256 * 4;
}

static void base_args(const qg_weight &w, GemmArgs *a) {
  memset(a, 0, sizeof(*a));
  a->wbase = (const uint8_t *)w.data;
  a->expert_stride = w.expert_stride;
  a->scales_offset = w.scales_offset;
  a->zeros_offset = w.zeros_offset;
  a->n_tiles = w.n_tiles;
  a->k_blocks = w.k_blocks;
  a->groups_padded = w.groups_padded;
  a->kb_pad = (int32_t)align_up((uint64_t)w.k_blocks, 4);
  a->n = (int32_t)w.desc.n;
  a->k = (int32_t)w.desc.k;
  a->splits = 1;
  // raster group of the dense tiled launches (QG_GROUP_M overrides)
  a->group_m = ov().group_m ? ov().group_m : 4;
}

}  // namespace qg

using namespace qg;

extern "C" const char *qg_status_string(qg_status s) {
  switch (s) {
    case QG_OK: return "ok";
    case QG_ERR_INVALID_ARGUMENT: return "invalid argument";
    case QG_ERR_SHAPE: return "invalid shape";
    case QG_ERR_ALIGNMENT: return "misaligned pointer or leading dimension";
    case QG_ERR_UNSUPPORTED: return "unsupported combination";
    case QG_ERR_BUFFER_TOO_SMALL: return "buffer too small";
    case QG_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

extern "C" int32_t qg_last_hip_error(void) { return g_last_hip_error; }

extern "C" qg_status qg_weight_bind(const qg_layer_desc *desc, void *dst_dev, uint64_t dst_bytes,
                                    qg_weight *out) {
  Layout L;
  qg_status st = make_layout(desc, &L);
  if (st != QG_OK) return st;
  if (!dst_dev || !out) return QG_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)dst_dev & 255u) != 0) return QG_ERR_ALIGNMENT;
  if (dst_bytes < L.total_bytes) return QG_ERR_BUFFER_TOO_SMALL;
  fill_weight(desc, L, dst_dev, dst_bytes, out);
  return QG_OK;
}

extern "C" qg_status qg_preprocess(const qg_layer_desc *desc, const void *codes,
                                   const void *scales, const void *zeros, int32_t expert_begin,
                                   int32_t expert_count, void *dst_dev, uint64_t dst_bytes,
                                   hipStream_t stream, qg_weight *out) {
  Layout L;
  qg_status st = make_layout(desc, &L);
  if (st != QG_OK) return st;
  if (!codes || !scales || !dst_dev || !out) return QG_ERR_INVALID_ARGUMENT;
  if (L.has_zp && !zeros) return QG_ERR_INVALID_ARGUMENT;
  if (expert_begin < 0 || expert_count <= 0 ||
      (int64_t)expert_begin + expert_count > desc->num_experts)
    return QG_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)dst_dev & 255u) != 0) return QG_ERR_ALIGNMENT;
  if (dst_bytes < L.total_bytes) return QG_ERR_BUFFER_TOO_SMALL;
  // Stage through a pinned host buffer in chunks of experts (bounded host memory).
  const uint64_t chunk_experts =
      std::max<uint64_t>(1, std::min<uint64_t>(expert_count, (1ull << 30) / L.expert_stride));
  const uint64_t stage_bytes = chunk_experts * L.expert_stride;
  void *stage = nullptr;
  hipError_t he = hipHostMalloc(&stage, stage_bytes, hipHostMallocDefault);
  if (he != hipSuccess) return hip_status(he);
  uint64_t cb, sb, zb;
  std_sizes(*desc, L, &cb, &sb, &zb);
  qg_status result = QG_OK;
  for (int64_t e0 = 0; e0 < expert_count; e0 += (int64_t)chunk_experts) {
    const int cnt = (int)std::min<int64_t>((int64_t)chunk_experts, expert_count - e0);
    // repack into the stage as if it held experts [0, cnt)
    qg_layer_desc d1 = *desc;
    d1.num_experts = cnt;
    st = qg_repack_host(&d1, (const uint8_t *)codes + e0 * cb, (const uint8_t *)scales + e0 * sb,
                        L.has_zp ? (const uint8_t *)zeros + e0 * zb : nullptr, 0, cnt, stage,
                        stage_bytes);
    if (st != QG_OK) {
      result = st;
      break;
    }
    uint8_t *dst = (uint8_t *)dst_dev + (uint64_t)(expert_begin + e0) * L.expert_stride;
    he = hipMemcpyAsync(dst, stage, (uint64_t)cnt * L.expert_stride, hipMemcpyHostToDevice, stream);
    if (he == hipSuccess) he = hipStreamSynchronize(stream);
    if (he != hipSuccess) {
      result = hip_status(he);
      break;
    }
  }
  hipHostFree(stage);
  if (result == QG_OK) fill_weight(desc, L, dst_dev, dst_bytes, out);
  return result;
}

// One dense GEMM with variant v (arguments already validated; ws holds
// dense_ws_bytes(w, v, m) bytes, its split-K counters zero).
// Row pitch of the activations in bytes: ldx elements of bf16, e4m3 or (two
// per byte) e2m1.
static uint64_t x_pitch(const Layout &L, int64_t ldx) {
  return L.a4 ? (uint64_t)ldx / 2 : (uint64_t)ldx * (L.x8 ? 1 : 2);
}

static hipError_t launch_dense_variant(const qg_weight &w, const Layout &L, const Variant &v, const void *x,
                                       const void *x_scales, int64_t m, int64_t ldx, void *y, int32_t otype,
                                       int64_t ldy, void *ws, hipStream_t stream) {
  const qg_layer_desc &d = w.desc;
  GemmArgs a;
  base_args(w, &a);
  a.x = x;
  a.x_scales = (const uint8_t *)x_scales;
  a.ldx = ldx;
  a.y = y;
  a.ldy = ldy;
  a.otype = otype;
  a.m = (int32_t)m;
  a.splits = v.splits;
  // counters start at zero (the caller zero-fills the workspace once) and
  // every call leaves them at zero again; the scratch behind them is free
  void *scratch = ws ? (void *)((uint8_t *)ws + kSplitCounterBytes) : nullptr;
  if (v.splits > 1) {
    a.counters = (uint32_t *)ws;
    a.partials = (float *)scratch;
  }
  if (v.kind == 1) {
    if (L.a4) a.ldx = ldx / 2;  // the kernel addresses e2m1 rows in bytes
    return launch_mx_tiled(a, v.bm, v.tbn, false, 0, mx_tiled_waves(), scratch, stream, L.a4, mx_tok(d), L.f8);
  }
  if (L.a4) {
    // the MX skinny kernel widens the e2m1 fragments to e4m3 in registers
    a.ldx = ldx / 2;
    return launch_dense_mx(a, d, v, stream);
  }
  if (v.kind == 3) return launch_decode_a16(a, d, v, stream);
  if (v.kind == 4) return launch_decode_wide(a, d, v, stream);
  if (v.kind == 2) return launch_a16_tiled(a, d, v.bm, v.tbn, false, m, 0, a16_tiled_waves(), scratch, true, stream);
  return L.is_mx ? launch_dense_mx(a, d, v, stream) : launch_dense_a16(a, d, v, stream);
}

static Variant dense_variant(const qg_weight &w, int64_t m, uint32_t flags) {
  return (flags & QG_GEMM_BATCH_INVARIANT) ? select_dense_invariant(w) : select_dense(w, m);
}

extern "C" qg_status qg_gemm_workspace_size_ex(const qg_weight *w, int64_t m, uint32_t flags, uint64_t *bytes) {
  Layout L;
  qg_status st = check_weight(w, &L);
  if (st != QG_OK) return st;
  if (!bytes || m < 0 || (flags & ~(uint32_t)QG_GEMM_BATCH_INVARIANT) != 0) return QG_ERR_INVALID_ARGUMENT;
  *bytes = dense_ws_bytes(*w, dense_variant(*w, m, flags), m);
  return QG_OK;
}

extern "C" qg_status qg_gemm_workspace_size(const qg_weight *w, int64_t m, uint64_t *bytes) {
  return qg_gemm_workspace_size_ex(w, m, 0, bytes);
}

extern "C" qg_status qg_gemm(const qg_weight *w, const void *x, const void *x_scales, int64_t m,
                             int64_t ldx, void *y, int32_t otype, int64_t ldy, void *ws,
                             uint64_t ws_bytes, hipStream_t stream) {
  return qg_gemm_ex(w, x, x_scales, m, ldx, y, otype, ldy, ws, ws_bytes, 0, stream);
}

extern "C" qg_status qg_gemm_ex(const qg_weight *w, const void *x, const void *x_scales, int64_t m,
                                int64_t ldx, void *y, int32_t otype, int64_t ldy, void *ws,
                                uint64_t ws_bytes, uint32_t flags, hipStream_t stream) {
  Layout L;
  qg_status st = check_weight(w, &L);
  if (st != QG_OK) return st;
  const qg_layer_desc &d = w->desc;
  if (d.num_experts != 1) return QG_ERR_INVALID_ARGUMENT;
  if (m < 0 || (otype != QG_O_BF16 && otype != QG_O_F32)) return QG_ERR_INVALID_ARGUMENT;
  if ((flags & ~(uint32_t)QG_GEMM_BATCH_INVARIANT) != 0) return QG_ERR_INVALID_ARGUMENT;
  if (m > (1ll << 30)) return QG_ERR_UNSUPPORTED;
  if (m == 0) return QG_OK;
  if (!x || !y) return QG_ERR_INVALID_ARGUMENT;
  if (L.xs_kind && !x_scales) return QG_ERR_INVALID_ARGUMENT;
  if (ldx < d.k || ldy < d.n) return QG_ERR_SHAPE;
  if (L.xs_kind >= 2 && ((uintptr_t)x_scales & 3u) != 0) return QG_ERR_ALIGNMENT;
  const int yel = otype == QG_O_F32 ? 4 : 2;
  if (!aligned16(x) || !aligned16(y) || x_pitch(L, ldx) % 16 != 0 || (L.a4 && (ldx & 1)) || (ldy * yel) % 4 != 0)
    return QG_ERR_ALIGNMENT;
  const Variant v = dense_variant(*w, m, flags);
  // the tiled kernels address X with 32-bit offsets; a batch-invariant call
  // may not move to another kernel past that size
  if (v.kind == 2 && (uint64_t)m * d.k * 2 >= (1ull << 31)) return QG_ERR_UNSUPPORTED;
  if (v.kind == 1 && (uint64_t)m * x_pitch(L, ldx) >= (1ull << 32)) return QG_ERR_UNSUPPORTED;
  const uint64_t need = dense_ws_bytes(*w, v, m);
  if (need > 0) {
    if (!ws) return QG_ERR_INVALID_ARGUMENT;
    if (ws_bytes < need) return QG_ERR_BUFFER_TOO_SMALL;
    if (((uintptr_t)ws & 255u) != 0) return QG_ERR_ALIGNMENT;
  }
  return hip_status(launch_dense_variant(*w, L, v, x, x_scales, m, ldx, y, otype, ldy, ws, stream));
}

// ---------------------------------------------------------------------------
// qg_gemm without a caller workspace: the scratch (split-K counters, partial
// tiles, the large-M kernels' pre-pass results) is a static device array.
// Its host-side name is only a stand-in: the device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[QG_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

__global__ void zero_fill_kernel(uint32_t *p, uint64_t words) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (uint64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// The scratch array of the current device: its address on first use there,
// with the split-K counter prefix cleared on `stream` by a fill kernel (not a
// memset node, so a first call inside graph capture stays correct).
static qg_status noalloc_scratch(hipStream_t stream, void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return QG_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (!ptr) return QG_ERR_HIP;
    hipLaunchKernelGGL(zero_fill_kernel, dim3(64), dim3(256), 0, stream, (uint32_t *)ptr, kSplitCounterBytes / 4);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_status(e);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return QG_OK;
}

extern "C" qg_status qg_gemm_noalloc(const qg_weight *w, const void *x, const void *x_scales, int64_t m,
                                     int64_t ldx, void *y, int32_t otype, int64_t ldy, hipStream_t stream) {
  Layout L;
  qg_status st = check_weight(w, &L);
  if (st != QG_OK) return st;
  if (m < 0) return QG_ERR_INVALID_ARGUMENT;
  // the scratch this call needs must fit the static array
  if (m > 0 && dense_ws_bytes(*w, dense_variant(*w, m, 0), m) > QG_NOALLOC_SCRATCH_BYTES)
    return QG_ERR_BUFFER_TOO_SMALL;
  if (m == 0) return qg_gemm_ex(w, x, x_scales, m, ldx, y, otype, ldy, nullptr, 0, 0, stream);
  void *ws = nullptr;
  st = noalloc_scratch(stream, &ws);
  if (st != QG_OK) return st;
  return qg_gemm_ex(w, x, x_scales, m, ldx, y, otype, ldy, ws, QG_NOALLOC_SCRATCH_BYTES, 0, stream);
}

// The weight as the MoE dispatch sees it: a W4A4 layer takes W4A8's kernel
// choices and workspace (the packed layout is the same); its launches then
// read e2m1 rows (the tiled kernel's A4 form, the skinny kernel's FMT 6).
static qg_weight mx_kernel_weight(const qg_weight &w, const Layout &L) {
  qg_weight k = w;
  if (L.a4) k.desc.atype = QG_A_MXFP8;
  return k;
}

extern "C" qg_status qg_moe_workspace_size(const qg_weight *w, int64_t num_tokens, int32_t topk,
                                           uint64_t *bytes) {
  Layout L;
  qg_status st = check_weight(w, &L);
  if (st != QG_OK) return st;
  if (!bytes || num_tokens < 0 || topk <= 0) return QG_ERR_INVALID_ARGUMENT;
  const int64_t pairs = num_tokens * topk;
  // the sort's need, or the grouped GEMM's with X indexed by pair (the larger
  // of the two x row counts); W4A4 needs what W4A8 does
  const qg_weight wk = mx_kernel_weight(*w, L);
  const uint64_t gemm = moe_ws_bytes(wk, pairs, pairs, moe_plan(wk, pairs, pairs));
  *bytes = std::max<uint64_t>(align_up((uint64_t)(w->desc.num_experts + 1) * 4, 256), gemm);
  return QG_OK;
}

extern "C" qg_status qg_moe_sort(const int32_t *topk_ids, int64_t num_tokens, int32_t topk,
                                 int32_t num_experts, int32_t *sorted_pair_ids,
                                 int32_t *expert_offsets, void *ws, uint64_t ws_bytes,
                                 hipStream_t stream) {
  if (num_tokens < 0 || topk <= 0 || num_experts <= 0) return QG_ERR_INVALID_ARGUMENT;
  if (num_experts > kMaxExperts) return QG_ERR_UNSUPPORTED;
  if (num_tokens * (int64_t)topk > (1ll << 30)) return QG_ERR_UNSUPPORTED;
  if (!expert_offsets || !ws) return QG_ERR_INVALID_ARGUMENT;
  if (num_tokens > 0 && (!topk_ids || !sorted_pair_ids)) return QG_ERR_INVALID_ARGUMENT;
  if (ws_bytes < align_up((uint64_t)(num_experts + 1) * 4, 256)) return QG_ERR_BUFFER_TOO_SMALL;
  if (((uintptr_t)ws & 3u) != 0 || ((uintptr_t)expert_offsets & 3u) != 0) return QG_ERR_ALIGNMENT;
  return hip_status(launch_moe_sort(topk_ids, num_tokens * topk, num_experts, sorted_pair_ids,
                                    expert_offsets, (int32_t *)ws, stream));
}

// The launches of one validated MoE call under `plan` (ws holds at least
// moe_ws_bytes of it).
static hipError_t moe_run(const qg_weight *w, const Layout &L, const MoePlan &plan, const void *x,
                          const void *x_scales, int32_t x_rows, const int32_t *sorted_pair_ids,
                          const int32_t *expert_offsets, int64_t num_tokens, int32_t topk, void *y, int32_t otype,
                          int32_t y_rows, void *ws, hipStream_t stream) {
  // W4A4: W4A8's dispatch, launched on e2m1 rows
  const qg_weight wk = mx_kernel_weight(*w, L);
  const qg_layer_desc &d = wk.desc;
  const int64_t pairs = num_tokens * topk;
  const Variant v = select_moe(wk, pairs);
  const int64_t x_rows_count = x_rows == QG_ROWS_BY_TOKEN ? num_tokens : pairs;
  const int min_rows = plan.min_rows;
  GemmArgs a;
  base_args(wk, &a);
  a.x = x;
  a.x_scales = (const uint8_t *)x_scales;
  a.ldx = L.a4 ? d.k / 2 : d.k;  // bytes of an e2m1 row
  a.y = y;
  a.ldy = d.n;
  a.otype = otype;
  a.sorted_ids = sorted_pair_ids;
  a.offsets = expert_offsets;
  a.num_experts = d.num_experts;
  a.topk = topk;
  a.x_rows = x_rows;
  a.y_rows = y_rows;
  hipError_t he = hipSuccess;
  const bool mxt = L.mx_pack || L.f8;  // the MX tiled kernel's layouts
  if (min_rows > 0) {
    // experts with >= min_rows rows: tile list, then the tiled kernel
    const int64_t cap = moe_tiles_cap(wk, pairs, min_rows);
    const bool small = plan.small;
    const int64_t cap_s = small ? moe_small_tiles_cap(wk, pairs) : 0;
    int32_t *tiles = (int32_t *)ws;
    int32_t *tiles_s = (int32_t *)((uint8_t *)ws + moe_list_bytes(cap));
    void *xs = (uint8_t *)tiles_s + (small ? moe_list_bytes(cap_s) : 0);  // integer formats only
    // the small tiles' rows (QG_MOE_SMALL_BM applies to the integer formats)
    const int sbm = mxt ? kMoeSmallTileRows : moe_small_bm();
    const bool both = small && min_rows < kMoeAllSmall;
    if (both)  // the two tile lists in one launch
      he = launch_moe_tiles2(expert_offsets, d.num_experts, (int32_t)pairs, min_rows, (int32_t)cap, tiles, sbm,
                             (int32_t)cap_s, tiles_s, stream);
    else if (!small)
      he = launch_moe_tiles(expert_offsets, d.num_experts, min_rows, 0, kMoeTileRows, (int32_t)pairs,
                            (int32_t)cap, tiles, stream);
    if (he != hipSuccess) return he;
    if (!small || min_rows < kMoeAllSmall) {
      a.tiles = tiles;
      a.group_m = moe_group_m();
      if (mxt)
        he = launch_mx_tiled(a, kMoeTileRows, plan.mx_bn, true, cap, mx_tiled_waves(), nullptr, stream, L.a4,
                             mx_tok(d), L.f8);
      else
        he = launch_a16_tiled(a, d, kMoeTileRows, a16_tiled_bn(), true, x_rows_count, cap, a16_tiled_waves(),
                              xs, true, stream);
      if (he != hipSuccess) return he;
    }
    if (small) {
      // (the list capacity covers either small-tile height)
      if (!both) {
        he = launch_moe_tiles(expert_offsets, d.num_experts, 1, min_rows, sbm, (int32_t)pairs,
                              (int32_t)cap_s, tiles_s, stream);
        if (he != hipSuccess) return he;
      }
      a.tiles = tiles_s;
      a.group_m = 1;
      // (the integer formats' row sums come from the 128-row launch unless it
      // was skipped)
      return mxt ? launch_mx_tiled(a, sbm, 128, true, cap_s, 8, nullptr, stream, L.a4, mx_tok(d), L.f8)
                 : launch_a16_tiled(a, d, sbm, 128, true, x_rows_count, cap_s, 8, xs, min_rows >= kMoeAllSmall,
                                    stream);
      // (every expert with rows is covered)
    }
    a.moe_min_rows = min_rows;
  }
  // the remaining (small) experts
  const int64_t max_tiles = (pairs + 15) / 16 + d.num_experts;
  // (the skinny kernel's format comes from the layer's own description:
  // FMT 6 widens e2m1 fragments in registers)
  return L.is_mx ? launch_moe_mx(a, w->desc, v, max_tiles, stream) : launch_moe_a16(a, d, v, max_tiles, stream);
}

// Argument checks shared by qg_moe_gemm and qg_moe_autotune (pairs > 0 only;
// the workspace is checked by the caller).
static qg_status moe_check(const qg_weight *w, const Layout &L, const void *x, const void *x_scales, int32_t x_rows,
                           const int32_t *sorted_pair_ids, const int32_t *expert_offsets, int32_t otype,
                           int32_t y_rows, const void *y) {
  const qg_layer_desc &d = w->desc;
  if (!x || !y || !sorted_pair_ids || !expert_offsets) return QG_ERR_INVALID_ARGUMENT;
  if (x_rows < QG_ROWS_BY_TOKEN || x_rows > QG_ROWS_SORTED) return QG_ERR_INVALID_ARGUMENT;
  if (y_rows != QG_ROWS_BY_PAIR && y_rows != QG_ROWS_SORTED) return QG_ERR_INVALID_ARGUMENT;
  if (L.xs_kind && !x_scales) return QG_ERR_INVALID_ARGUMENT;
  if (L.xs_kind >= 2 && ((uintptr_t)x_scales & 3u) != 0) return QG_ERR_ALIGNMENT;
  const int yel = otype == QG_O_F32 ? 4 : 2;
  if (!aligned16(x) || !aligned16(y) || x_pitch(L, d.k) % 16 != 0 || (d.n * yel) % 4 != 0)
    return QG_ERR_ALIGNMENT;
  return QG_OK;
}

extern "C" qg_status qg_moe_gemm(const qg_weight *w, const void *x, const void *x_scales,
                                 int32_t x_rows, const int32_t *sorted_pair_ids,
                                 const int32_t *expert_offsets, int64_t num_tokens, int32_t topk,
                                 void *y, int32_t otype, int32_t y_rows, void *ws,
                                 uint64_t ws_bytes, hipStream_t stream) {
  Layout L;
  qg_status st = check_weight(w, &L);
  if (st != QG_OK) return st;
  const qg_weight wk = mx_kernel_weight(*w, L);
  if (num_tokens < 0 || topk <= 0 || (otype != QG_O_BF16 && otype != QG_O_F32))
    return QG_ERR_INVALID_ARGUMENT;
  if (x_rows < QG_ROWS_BY_TOKEN || x_rows > QG_ROWS_SORTED) return QG_ERR_INVALID_ARGUMENT;
  if (y_rows != QG_ROWS_BY_PAIR && y_rows != QG_ROWS_SORTED) return QG_ERR_INVALID_ARGUMENT;
  if (w->desc.num_experts > kMaxExperts) return QG_ERR_UNSUPPORTED;
  const int64_t pairs = num_tokens * topk;
  if (pairs > (1ll << 30)) return QG_ERR_UNSUPPORTED;
  if (pairs == 0) return QG_OK;
  st = moe_check(w, L, x, x_scales, x_rows, sorted_pair_ids, expert_offsets, otype, y_rows, y);
  if (st != QG_OK) return st;
  const int64_t x_rows_count = x_rows == QG_ROWS_BY_TOKEN ? num_tokens : pairs;
  const MoePlan plan = moe_plan(wk, pairs, x_rows_count);
  const uint64_t need = moe_ws_bytes(wk, pairs, x_rows_count, plan);
  if (need > 0) {
    if (!ws) return QG_ERR_INVALID_ARGUMENT;
    if (ws_bytes < need) return QG_ERR_BUFFER_TOO_SMALL;
    if (((uintptr_t)ws & 255u) != 0) return QG_ERR_ALIGNMENT;
  }
  return hip_status(moe_run(w, L, plan, x, x_scales, x_rows, sorted_pair_ids, expert_offsets, num_tokens, topk, y,
                            otype, y_rows, ws, stream));
}

// MoE autotune candidates: every expert on the skinny kernel, every expert on
// the small tiles, or the 128-row tiles from 16, 32, 64 or 128 rows with the
// rest on the small tiles or the skinny kernel, for the MX tiled kernel in
// 128- and 256-column tiles (E = 128 top-8 W4A8 gate_up at T = 512: 77.6 us
// on small tiles only against 89.4 us with the default threshold).
static void moe_tune_candidates(const qg_weight &wk, int64_t pairs, int64_t x_rows_count, std::vector<MoePlan> *out) {
  const MoePlan heur = moe_plan(wk, pairs, x_rows_count);
  out->push_back(heur);
  auto add = [&](const MoePlan &p) {
    for (const MoePlan &q : *out)
      if (q.min_rows == p.min_rows && q.small == p.small && q.mx_bn == p.mx_bn) return;
    out->push_back(p);
  };
  add(MoePlan{0, false, heur.mx_bn});
  if (!moe_tiled_ok(wk, x_rows_count)) return;
  const bool mxt = mx_tiled_fmt(wk.desc);
  add(MoePlan{kMoeAllSmall, true, heur.mx_bn});
  for (int r : {16, 32, 64, 128})
    for (int small = 0; small < 2; ++small)
      for (int bn : {128, 256}) {
        if (bn == 256 && (!mxt || w8a8(wk.desc))) continue;
        add(MoePlan{r, small != 0, bn});
      }
}

static void describe_moe_plan(const qg_weight &wk, const Layout &L, const MoePlan &plan, int64_t pairs, char *buf,
                              uint64_t buf_bytes);

extern "C" qg_status qg_moe_autotune_workspace_size(const qg_weight *w, int64_t num_tokens, int32_t topk,
                                                    uint64_t *bytes) {
  Layout L;
  qg_status st = check_weight(w, &L);
  if (st != QG_OK) return st;
  if (!bytes || num_tokens < 0 || topk <= 0) return QG_ERR_INVALID_ARGUMENT;
  const qg_weight wk = mx_kernel_weight(*w, L);
  const int64_t pairs = num_tokens * topk;
  std::vector<MoePlan> cand;
  moe_tune_candidates(wk, std::max<int64_t>(pairs, 1), pairs, &cand);
  uint64_t b = 0;
  for (const MoePlan &p : cand) b = std::max(b, moe_ws_bytes(wk, pairs, pairs, p));
  *bytes = align_up(b, 256) + kTuneSinkBytes;
  return QG_OK;
}

extern "C" qg_status qg_moe_autotune(const qg_weight *w, const void *x, const void *x_scales, int32_t x_rows,
                                     const int32_t *sorted_pair_ids, const int32_t *expert_offsets,
                                     int64_t num_tokens, int32_t topk, void *y, int32_t otype, int32_t y_rows,
                                     void *ws, uint64_t ws_bytes, const void *flush, uint64_t flush_bytes,
                                     int32_t reps, hipStream_t stream, char *chosen, uint64_t chosen_bytes,
                                     float *chosen_us) {
  Layout L;
  qg_status st = check_weight(w, &L);
  if (st != QG_OK) return st;
  const qg_weight wk = mx_kernel_weight(*w, L);
  if (num_tokens < 1 || topk <= 0 || reps < 1 || reps > kTuneMaxReps) return QG_ERR_INVALID_ARGUMENT;
  if (otype != QG_O_BF16 && otype != QG_O_F32) return QG_ERR_INVALID_ARGUMENT;
  if (w->desc.num_experts > kMaxExperts) return QG_ERR_UNSUPPORTED;
  const int64_t pairs = num_tokens * topk;
  if (pairs > (1ll << 30)) return QG_ERR_UNSUPPORTED;
  st = moe_check(w, L, x, x_scales, x_rows, sorted_pair_ids, expert_offsets, otype, y_rows, y);
  if (st != QG_OK) return st;
  if (!ws || ((uintptr_t)ws & 255u) != 0) return !ws ? QG_ERR_INVALID_ARGUMENT : QG_ERR_ALIGNMENT;
  if (flush && (flush_bytes % 16 != 0 || !aligned16(flush))) return QG_ERR_ALIGNMENT;
  const int64_t x_rows_count = x_rows == QG_ROWS_BY_TOKEN ? num_tokens : pairs;
  std::vector<MoePlan> cand;
  moe_tune_candidates(wk, pairs, x_rows_count, &cand);
  uint64_t db = 0;
  for (const MoePlan &p : cand) db = std::max(db, moe_ws_bytes(wk, pairs, x_rows_count, p));
  db = align_up(db, 256);
  if (ws_bytes < db + kTuneSinkBytes) return QG_ERR_BUFFER_TOO_SMALL;
  uint8_t *sink = (uint8_t *)ws + db;

  hipEvent_t ev[2 * kTuneMaxReps];
  int made = 0;
  hipError_t he = hipSuccess;
  for (; made < 2 * reps; ++made)
    if ((he = hipEventCreate(&ev[made])) != hipSuccess) break;
  int best = -1;
  float best_us = 0.f;
  for (size_t i = 0; he == hipSuccess && i < cand.size(); ++i) {
    const MoePlan &p = cand[i];
    auto run = [&]() {
      return moe_run(w, L, p, x, x_scales, x_rows, sorted_pair_ids, expert_offsets, num_tokens, topk, y, otype,
                     y_rows, ws, stream);
    };
    if (run() != hipSuccess) continue;  // a form this shape does not compile to: skip it
    for (int r = 0; r < reps && he == hipSuccess; ++r) {
      if (flush && flush_bytes) he = launch_stream_read(flush, flush_bytes, sink, stream);
      if (he == hipSuccess) he = hipEventRecord(ev[2 * r], stream);
      if (he == hipSuccess) he = run();
      if (he == hipSuccess) he = hipEventRecord(ev[2 * r + 1], stream);
    }
    if (he == hipSuccess) he = hipEventSynchronize(ev[2 * reps - 1]);
    float total = 0.f;
    for (int r = 0; r < reps && he == hipSuccess; ++r) {
      float ms = 0.f;
      he = hipEventElapsedTime(&ms, ev[2 * r], ev[2 * r + 1]);
      total += ms;
    }
    if (he != hipSuccess) break;
    const float us = total * 1000.f / (float)reps;
    if (best < 0 || us < best_us) {
      best = (int)i;
      best_us = us;
    }
  }
  for (int e = 0; e < made; ++e) hipEventDestroy(ev[e]);
  if (he != hipSuccess) return hip_status(he);
  if (best < 0) return QG_ERR_UNSUPPORTED;
  {
    std::lock_guard<std::mutex> lock(g_moe_tune_mu);
    const int b = pairs_bucket(pairs);
    bool found = false;
    for (MoeTuneEntry &e : g_moe_tune)
      if (moe_tune_key(e, wk, b)) {
        e.plan = cand[best];
        found = true;
      }
    if (!found)
      g_moe_tune.push_back(MoeTuneEntry{wk.desc.wtype, wk.desc.atype, wk.desc.group_size, wk.desc.num_experts, b,
                                        wk.desc.n, wk.desc.k, cand[best]});
  }
  if (chosen && chosen_bytes) describe_moe_plan(wk, L, cand[best], pairs, chosen, chosen_bytes);
  if (chosen_us) *chosen_us = best_us;
  return QG_OK;
}

static void describe_variant(const Variant &v, const Layout &L, int k_blocks, char *buf, uint64_t buf_bytes);

static void describe_moe_plan(const qg_weight &wk, const Layout &L, const MoePlan &plan, int64_t pairs, char *buf,
                              uint64_t buf_bytes) {
  const Variant v = select_moe(wk, std::max<int64_t>(pairs, 1));
  char skinny[96];
  describe_variant(v, L, wk.k_blocks, skinny, sizeof skinny);
  const int min_rows = plan.min_rows;
  const bool mxt = L.mx_pack || L.f8;
  const char *fam = L.f8 ? "f8" : L.mx_pack ? "mx" : "a16";
  const int bn = mxt ? plan.mx_bn : a16_tiled_bn();
  if (min_rows <= 0)
    snprintf(buf, buf_bytes, "%s for every expert", skinny);
  else if (plan.small && min_rows >= kMoeAllSmall)
    snprintf(buf, buf_bytes, "%s_tiled small BM=%d for every expert", fam, mxt ? kMoeSmallTileRows : moe_small_bm());
  else if (plan.small)
    snprintf(buf, buf_bytes, "%s_tiled BM=%d BN=%d for experts with >= %d rows; %s_tiled small BM=%d below", fam,
             kMoeTileRows, bn, min_rows, fam, mxt ? kMoeSmallTileRows : moe_small_bm());
  else
    snprintf(buf, buf_bytes, "%s_tiled BM=%d BN=%d for experts with >= %d rows; %s below", fam, kMoeTileRows, bn,
             min_rows, skinny);
}

extern "C" qg_status qg_describe_moe_dispatch(const qg_weight *w, int64_t num_tokens, int32_t topk, char *buf,
                                              uint64_t buf_bytes) {
  Layout L;
  qg_status st = check_weight(w, &L);
  if (st != QG_OK) return st;
  if (!buf || buf_bytes == 0 || num_tokens < 0 || topk <= 0) return QG_ERR_INVALID_ARGUMENT;
  const qg_weight wk = mx_kernel_weight(*w, L);
  const int64_t pairs = num_tokens * topk;
  const MoePlan plan = pairs > 0 ? moe_plan(wk, pairs, pairs) : MoePlan{0, false, moe_mx_bn(wk)};
  describe_moe_plan(wk, L, plan, pairs, buf, buf_bytes);
  return QG_OK;
}

extern "C" qg_status qg_stream_read(const void *src, uint64_t bytes, void *sink,
                                    hipStream_t stream) {
  if (bytes == 0) return QG_OK;
  if (!src || !sink) return QG_ERR_INVALID_ARGUMENT;
  if (bytes % 16 != 0 || !aligned16(src) || ((uintptr_t)sink & 3u) != 0) return QG_ERR_ALIGNMENT;
  return hip_status(launch_stream_read(src, bytes, sink, stream));
}

extern "C" qg_status qg_stream_copy(void *dst, const void *src, uint64_t bytes,
                                    hipStream_t stream) {
  if (bytes == 0) return QG_OK;
  if (!src || !dst) return QG_ERR_INVALID_ARGUMENT;
  if (bytes % 16 != 0 || !aligned16(src) || !aligned16(dst)) return QG_ERR_ALIGNMENT;
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
  if (a < b + bytes && b < a + bytes) return QG_ERR_INVALID_ARGUMENT;  // overlap
  return hip_status(launch_stream_copy(dst, src, bytes, stream));
}

static bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

extern "C" qg_status qg_quantize_mxfp8(const void *x, int64_t rows, int64_t k, int64_t ldx, void *q,
                                       int64_t ldq, void *q_scales, hipStream_t stream) {
  if (rows < 0 || k < 0) return QG_ERR_INVALID_ARGUMENT;
  if (k % 32 != 0 || ldx < k || ldq < k) return QG_ERR_SHAPE;
  if (rows == 0 || k == 0) return QG_OK;
  if (!x || !q || !q_scales) return QG_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || ldx % 8 != 0 || !aligned(q, 8) || ldq % 8 != 0) return QG_ERR_ALIGNMENT;
  return hip_status(launch_quantize_mxfp8(x, rows, k, ldx, q, ldq, q_scales, stream));
}

extern "C" qg_status qg_quantize_mxfp4(const void *x, int64_t rows, int64_t k, int64_t ldx, void *q,
                                       int64_t ldq, void *q_scales, hipStream_t stream) {
  if (rows < 0 || k < 0) return QG_ERR_INVALID_ARGUMENT;
  if (k % 32 != 0 || ldx < k || ldq < k) return QG_ERR_SHAPE;
  if (rows == 0 || k == 0) return QG_OK;
  if (!x || !q || !q_scales) return QG_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || ldx % 8 != 0 || !aligned(q, 4) || ldq % 8 != 0) return QG_ERR_ALIGNMENT;
  return hip_status(launch_quantize_mxfp4(x, rows, k, ldx, q, ldq, q_scales, stream));
}

extern "C" qg_status qg_quantize_fp8(const void *x, int64_t rows, int64_t k, int64_t ldx, int32_t block, void *q,
                                     int64_t ldq, float *q_scales, hipStream_t stream) {
  if (rows < 0 || k < 0 || (block != 0 && block != 128)) return QG_ERR_INVALID_ARGUMENT;
  if (k % 8 != 0 || ldx < k || ldq < k) return QG_ERR_SHAPE;
  if (rows == 0 || k == 0) return QG_OK;
  if (!x || !q || !q_scales) return QG_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || ldx % 8 != 0 || !aligned16(q) || ldq % 16 != 0 || !aligned(q_scales, 4))
    return QG_ERR_ALIGNMENT;
  return hip_status(launch_quantize_fp8(x, rows, k, ldx, block, q, ldq, q_scales, stream));
}

extern "C" qg_status qg_silu_mul(const void *gu, int32_t gu_type, int64_t rows, int64_t inter, int64_t ldgu,
                                 void *h, int32_t h_type, int64_t ldh, void *h_scales, hipStream_t stream) {
  if (rows < 0 || inter < 0) return QG_ERR_INVALID_ARGUMENT;
  if ((gu_type != QG_O_BF16 && gu_type != QG_O_F32) || (h_type != QG_A_BF16 && h_type != QG_A_MXFP8))
    return QG_ERR_INVALID_ARGUMENT;
  const bool mx = h_type == QG_A_MXFP8;
  if (inter % (mx ? 32 : 8) != 0 || ldgu < 2 * inter || ldh < inter) return QG_ERR_SHAPE;
  if (rows == 0 || inter == 0) return QG_OK;
  if (!gu || !h || (mx && !h_scales)) return QG_ERR_INVALID_ARGUMENT;
  const bool f32 = gu_type == QG_O_F32;
  if (!aligned16(gu) || ldgu % (f32 ? 4 : 8) != 0) return QG_ERR_ALIGNMENT;
  if (mx ? (!aligned(h, 8) || ldh % 8 != 0) : (!aligned16(h) || ldh % 8 != 0)) return QG_ERR_ALIGNMENT;
  return hip_status(launch_silu_mul(gu, f32, rows, inter, ldgu, mx, h, ldh, h_scales, stream));
}

extern "C" qg_status qg_moe_combine(const void *y, int32_t y_type, int64_t ldy, const float *topk_weights,
                                    int64_t num_tokens, int32_t topk, int64_t n, const void *bias, void *out,
                                    int32_t out_type, int64_t ldout, hipStream_t stream) {
  if (num_tokens < 0 || n < 0 || topk < 1) return QG_ERR_INVALID_ARGUMENT;
  if ((y_type != QG_O_BF16 && y_type != QG_O_F32) || (out_type != QG_O_BF16 && out_type != QG_O_F32))
    return QG_ERR_INVALID_ARGUMENT;
  if (n % 8 != 0 || ldy < n || ldout < n) return QG_ERR_SHAPE;
  if (num_tokens == 0 || n == 0) return QG_OK;
  if (!y || !topk_weights || !out) return QG_ERR_INVALID_ARGUMENT;
  const bool yf = y_type == QG_O_F32, of = out_type == QG_O_F32;
  if (!aligned16(y) || ldy % (yf ? 4 : 8) != 0 || !aligned16(out) || ldout % (of ? 4 : 8) != 0 ||
      !aligned(topk_weights, 4) || (bias && !aligned16(bias)))
    return QG_ERR_ALIGNMENT;
  return hip_status(launch_moe_combine(y, yf, ldy, topk_weights, num_tokens, topk, n, bias, out, of, ldout, stream));
}

static void describe_variant(const Variant &v, const Layout &L, int k_blocks, char *buf, uint64_t buf_bytes) {
  const bool mx = L.mx_pack || L.f8;  // (the MX tiled kernel also serves per-token FP8 and W8A8)
  // skinny-kernel family: MX (also per-token FP8 activations), W8A8, A16
  const char *fam = L.mx_pack ? "mx" : L.f8 ? "f8" : "a16";
  if (v.kind == 3)
    snprintf(buf, buf_bytes, v.splits > 1 ? "a16_decode T=%d KR=%d W=%d splits=%d" : "a16_decode T=%d KR=%d W=%d",
             v.T, v.KR, v.W, v.splits);
  else if (v.kind == 4)
    snprintf(buf, buf_bytes, "a16_decode_wide KR=%d W=%d splits=%d", v.KR, v.W, v.splits);
  else if (v.kind == 1 || v.kind == 2)
    snprintf(buf, buf_bytes, "%s_tiled BM=%d BN=%d", L.f8 ? "f8" : mx ? "mx" : "a16", v.bm, v.tbn);
  else {
    // (K beyond W * KR * splits blocks: the workgroups loop over K)
    const int span = v.W * v.KR * v.splits, passes = (k_blocks + span - 1) / span;
    snprintf(buf, buf_bytes, passes > 1 ? "%s_skinny T=%d KR=%d W=%d splits=%d passes=%d" : "%s_skinny T=%d KR=%d W=%d splits=%d",
             fam, v.T, v.KR, v.W, v.splits, passes);
  }
}

// Candidates of one dense (layer, M): the heuristic's choice first, then the
// decode kernel's compiled (T, KR) pairs with 1, 2 or 4 K splits (integer
// formats, M <= 16, K % 512 == 0), the skinny kernel's spill-free (T, KR)
// with 1, 2, 4 or 8 K splits (M <= 256), and the tiled kernels' tile shapes
// (K % 128 == 0).
static void tune_candidates(const qg_weight &w, int64_t m, std::vector<Variant> *out) {
  const qg_layer_desc &d = w.desc;
  const bool mx = mx_tiled_fmt(d);
  auto add = [&](const Variant &v) {
    for (const Variant &u : *out)
      if (same_variant(u, v)) return;
    if (variant_valid(w, m, v)) out->push_back(v);
  };
  add(select_dense_heuristic(w, m));
  if (!mx && m <= 16 && d.k % 512 == 0) {
    static const int pairs[][2] = {{1, 8}, {2, 4}, {2, 8}, {4, 2}, {1, 4}};
    for (const auto &p : pairs)
      for (int S : {1, 2, 4}) {
        Variant v;
        if (decode_fits(w, m, p[0], p[1], S, &v)) add(v);
      }
    for (int W : {8, 16})
      for (int KR : {8, 16}) {
        Variant v;
        if (decode_wide_fits(w, m, W, KR, &v)) add(v);
      }
  }
  if (m <= 256) {
    const int kbs = w.k_blocks;
    for (int T : {1, 2, 4})
      for (int KR : {1, 2, 4}) {
        if (!variant_ok(d, T, KR)) continue;
        const int waves_k = (kbs + KR - 1) / KR;
        for (int S : {1, 2, 4, 8}) {
          const int W = (waves_k + S - 1) / S;
          if (W < 1 || W > 16) continue;
          add(Variant{0, T, KR, W, (waves_k + W - 1) / W, 0, 0});
          // each wave walking its K range in two passes
          const int per = (waves_k + 1) / 2, W2 = (per + S - 1) / S;
          if (waves_k >= 8 && W2 >= 1 && W2 <= 16) add(Variant{0, T, KR, W2, (per + W2 - 1) / W2, 0, 0});
        }
      }
  }
  if (d.k % 128 == 0) {
    if (mx) {
      for (int bm : {128, 256})
        for (int bn : {128, 192, 224, 256}) add(Variant{1, 1, 1, 1, 1, bm, bn});  // (variant_valid filters)
    } else {
      add(Variant{2, 1, 1, 1, 1, 128, 256});
      add(Variant{2, 1, 1, 1, 1, 256, 128});
      add(Variant{2, 1, 1, 1, 1, 128, 128});
    }
  }
}


// Autotune workspace: a dense workspace for every candidate (the counter
// prefix, cleared by the call, then the largest candidate's partials or
// scratch), then the flush sink.
static uint64_t tune_ws_dense_bytes(const qg_weight &w, int64_t m, const std::vector<Variant> &c) {
  uint64_t b = kSplitCounterBytes;
  for (const Variant &v : c) b = std::max(b, align_up(dense_ws_bytes(w, v, m), 256));
  return b;
}

extern "C" qg_status qg_gemm_autotune_workspace_size(const qg_weight *w, int64_t m, uint64_t *bytes) {
  Layout L;
  qg_status st = check_weight(w, &L);
  if (st != QG_OK) return st;
  if (!bytes || m < 0 || w->desc.num_experts != 1) return QG_ERR_INVALID_ARGUMENT;
  if (m == 0) {
    *bytes = 0;
    return QG_OK;
  }
  std::vector<Variant> c;
  tune_candidates(*w, m, &c);
  *bytes = tune_ws_dense_bytes(*w, m, c) + kTuneSinkBytes;
  return QG_OK;
}

extern "C" qg_status qg_gemm_autotune(const qg_weight *w, const void *x, const void *x_scales, int64_t m,
                                      int64_t ldx, void *y, int32_t otype, int64_t ldy, void *ws, uint64_t ws_bytes,
                                      const void *flush, uint64_t flush_bytes, int32_t reps, hipStream_t stream,
                                      char *chosen, uint64_t chosen_bytes, float *chosen_us) {
  Layout L;
  qg_status st = check_weight(w, &L);
  if (st != QG_OK) return st;
  const qg_layer_desc &d = w->desc;
  if (d.num_experts != 1 || m < 1 || reps < 1 || reps > kTuneMaxReps) return QG_ERR_INVALID_ARGUMENT;
  if (otype != QG_O_BF16 && otype != QG_O_F32) return QG_ERR_INVALID_ARGUMENT;
  if (m > (1ll << 30)) return QG_ERR_UNSUPPORTED;
  if (!x || !y || !ws || (L.xs_kind && !x_scales)) return QG_ERR_INVALID_ARGUMENT;
  if (ldx < d.k || ldy < d.n) return QG_ERR_SHAPE;
  if (L.xs_kind >= 2 && ((uintptr_t)x_scales & 3u) != 0) return QG_ERR_ALIGNMENT;
  const int yel = otype == QG_O_F32 ? 4 : 2;
  if (!aligned16(x) || !aligned16(y) || x_pitch(L, ldx) % 16 != 0 || (L.a4 && (ldx & 1)) || (ldy * yel) % 4 != 0 ||
      ((uintptr_t)ws & 255u) != 0)
    return QG_ERR_ALIGNMENT;
  if ((L.mx_pack || L.f8) && (uint64_t)m * x_pitch(L, ldx) >= (1ull << 32)) return QG_ERR_UNSUPPORTED;
  if (flush && (flush_bytes % 16 != 0 || !aligned16(flush))) return QG_ERR_ALIGNMENT;
  std::vector<Variant> cand;
  tune_candidates(*w, m, &cand);
  const uint64_t db = tune_ws_dense_bytes(*w, m, cand);
  if (ws_bytes < db + kTuneSinkBytes) return QG_ERR_BUFFER_TOO_SMALL;
  uint8_t *sink = (uint8_t *)ws + db;
  // the split-K counters must start at zero; the rest is scratch (this call
  // synchronizes its stream, so it is never part of a captured graph)
  const hipError_t me = hipMemsetAsync(ws, 0, kSplitCounterBytes, stream);
  if (me != hipSuccess) return hip_status(me);

  hipEvent_t ev[2 * kTuneMaxReps];
  int made = 0;
  hipError_t he = hipSuccess;
  for (; made < 2 * reps; ++made)
    if ((he = hipEventCreate(&ev[made])) != hipSuccess) break;
  int best = -1;
  float best_us = 0.f;
  for (size_t i = 0; he == hipSuccess && i < cand.size(); ++i) {
    const Variant &v = cand[i];
    auto run = [&]() { return launch_dense_variant(*w, L, v, x, x_scales, m, ldx, y, otype, ldy, ws, stream); };
    if (run() != hipSuccess) continue;  // an instance this shape does not compile to: skip it
    for (int r = 0; r < reps && he == hipSuccess; ++r) {
      if (flush && flush_bytes) he = launch_stream_read(flush, flush_bytes, sink, stream);
      if (he == hipSuccess) he = hipEventRecord(ev[2 * r], stream);
      if (he == hipSuccess) he = run();
      if (he == hipSuccess) he = hipEventRecord(ev[2 * r + 1], stream);
    }
    if (he == hipSuccess) he = hipEventSynchronize(ev[2 * reps - 1]);
    float total = 0.f;
    for (int r = 0; r < reps && he == hipSuccess; ++r) {
      float ms = 0.f;
      he = hipEventElapsedTime(&ms, ev[2 * r], ev[2 * r + 1]);
      total += ms;
    }
    if (he != hipSuccess) break;
    const float us = total * 1000.f / (float)reps;
    if (best < 0 || us < best_us) {
      best = (int)i;
      best_us = us;
    }
  }
  for (int e = 0; e < made; ++e) hipEventDestroy(ev[e]);
  if (he != hipSuccess) return hip_status(he);
  if (best < 0) return QG_ERR_UNSUPPORTED;
  tuned_store(*w, m, cand[best]);
  if (chosen && chosen_bytes) describe_variant(cand[best], L, w->k_blocks, chosen, chosen_bytes);
  if (chosen_us) *chosen_us = best_us;
  return QG_OK;
}

extern "C" qg_status qg_set_override(const char *name, const char *value) {
  if (!name) return QG_ERR_INVALID_ARGUMENT;
  ov();  // the environment's snapshot exists from here on
  std::lock_guard<std::mutex> lock(g_overrides_mu);
  Overrides *o = new Overrides(*g_overrides.load(std::memory_order_relaxed));
  if (!apply_override(o, name, value)) {
    delete o;
    return QG_ERR_INVALID_ARGUMENT;
  }
  g_overrides.store(o, std::memory_order_release);
  return QG_OK;
}

extern "C" void qg_clear_overrides(void) {
  ov();
  std::lock_guard<std::mutex> lock(g_overrides_mu);
  g_overrides.store(new Overrides(), std::memory_order_release);
}

extern "C" void qg_autotune_reset(void) {
  {
    std::lock_guard<std::mutex> lock(g_tune_mu);
    g_tune.clear();
  }
  std::lock_guard<std::mutex> lock(g_moe_tune_mu);
  g_moe_tune.clear();
}

extern "C" qg_status qg_describe_dispatch_ex(const qg_weight *w, int64_t m, uint32_t flags, char *buf,
                                             uint64_t buf_bytes) {
  Layout L;
  qg_status st = check_weight(w, &L);
  if (st != QG_OK) return st;
  if (!buf || buf_bytes == 0 || m < 0 || (flags & ~(uint32_t)QG_GEMM_BATCH_INVARIANT) != 0)
    return QG_ERR_INVALID_ARGUMENT;
  if (flags && w->desc.num_experts > 1) return QG_ERR_INVALID_ARGUMENT;
  const Variant v = w->desc.num_experts > 1 ? select_moe(*w, m) : dense_variant(*w, m, flags);
  describe_variant(v, L, w->k_blocks, buf, buf_bytes);
  return QG_OK;
}

extern "C" qg_status qg_describe_dispatch(const qg_weight *w, int64_t m, char *buf, uint64_t buf_bytes) {
  return qg_describe_dispatch_ex(w, m, 0, buf, buf_bytes);
}
