/*
 * qg.h -- C ABI of the MI355X (gfx950) quantized GEMM library (libqg.so).
 *
 * The library computes Y = X * dequant(W)^T for low-bit weights with the
 * dequantization done inside the GEMM kernels, for dense layers and for
 * token-sorted MoE grouped layers.  The operations follow the problem
 * statement of the Humming announcement (vLLM / Ant Group, "Announcing
 * Humming", spke.com Japanese translation):
 *   - section "Unified quantization representation": a weight format is
 *     described by its bit width / number format, scale granularity, scale
 *     type and an optional zero point; activations have their own format.
 *   - section "Per-workload tuning and JIT compilation": preprocessing
 *     validates parameters, pads dimensions and repacks the tensors into the
 *     layout of the target kernel; at inference the chosen kernel runs on the
 *     preprocessed weights and the runtime activations; configurations are
 *     prepared per input-size (M) range and dispatched at run time.
 *   - section "Shared CUDA components": dequantization and scaling happen
 *     inside the kernel; dense and MoE GEMMs have their own task mapping.
 * and the AIREITER benchmark page ("vLLM Humming performance benchmark"),
 * sections "H100 group-32 W4A8" (MXFP4 weights x MXFP8 activations, one scale
 * per 32) and "SM80 single-request decode" (INT3 weights, M = 1).
 *
 * Conventions for every entry point:
 *   - Plain C, no exceptions cross the boundary, no abort/assert on caller
 *     input.  Every call validates all arguments before it launches anything;
 *     a failed validation has no side effects and returns a status.
 *   - "device" pointers are HIP device memory on the current device, "host"
 *     pointers are ordinary process memory.  The caller owns every buffer,
 *     including packed weights and workspaces; the library allocates nothing
 *     that outlives a call and has no destroy call.
 *   - Device work is enqueued on the caller's stream and is asynchronous;
 *     only qg_preprocess synchronizes (its stream) before returning.
 *   - Calls are thread-safe; two calls that share a workspace must be ordered
 *     on one stream.
 *
 * Standard (input) format handed to qg_preprocess, per expert:
 *   codes  : [N][K] row-major, each row an LSB-first bitstream of b-bit codes
 *            (code k sits in bits [b*k, b*k+b) of the row; rows are K*b/8
 *            bytes).  INT-b codes are two's complement, UINT-b codes are plain,
 *            e2m1 uses bit 3 as its sign, e0m codes bit b-1, e4m3 bit 7.
 *   scales : [N][K/g]: bf16 bit patterns (A16 formats) or e8m0 bytes (MXFP4);
 *            W8A8: fp32 [ceil(N/128)][K/128].
 *   zeros  : [N][K/g] uint8 in 0..2^b-1 for UINT-b formats, NULL otherwise.
 * Activations: x is [rows][ldx] row-major: bf16, e4m3 bytes (MXFP8), or e2m1
 * codes two per byte (MXFP4: element k in the low nibble of byte k/2 when k is
 * even, the high nibble when odd; ldx counts elements), the MX types with
 * x_scales [rows][K/32] e8m0 bytes (row stride K/32), per desc.atype; e4m3
 * bytes with fp32 x_scales [rows] (FP8_TOKEN) or [rows][K/128] (FP8_BLOCK).
 * y is [rows][ldy] row-major, bf16 or fp32.
 *
 * Numerics (the contract the CPU oracle checks):
 *   - A16 formats: the dequantized weight is the exact real (q - z) * s, with
 *     q the decoded code, z the group's zero point (0 for signed formats) and
 *     s the group's bf16 scale.  Kernels form sum_k x*(q - z) per K-group with
 *     bf16 MFMA (codes are exact in bf16) and apply s per group in fp32.
 *   - Per-token FP8: y[r] = s_r * sum_k e4m3(a[r,k]) * Wdq[n,k] (MXFP4 Wdq).
 *   - W8A8: sum over 128-K blocks kb of sa[r][kb] * sw[n/128][kb] * the
 *     block's sum of e4m3 products, each block's partial scaled in fp32.
 *   - MXFP4 x MXFP8: e2m1 * 2^(e-127) times e4m3 * 2^(ea-127), exact operands
 *     into gfx950 scaled MFMA; MXFP4 x MXFP4 likewise with e2m1 activations.
 *   - fp32 accumulation; QG_O_BF16 output is the fp32 result rounded to
 *     nearest-even; QG_O_F32 exposes the fp32 accumulators.
 */
#ifndef QG_H_
#define QG_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QG_ABI_VERSION 1
#define QG_LAYOUT_VERSION 2

typedef enum {
  QG_OK = 0,
  QG_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad enum, negative size */
  QG_ERR_SHAPE = 2,            /* K % group != 0, K % 32 != 0, ld too small, ... */
  QG_ERR_ALIGNMENT = 3,        /* a device pointer or leading dimension misaligned */
  QG_ERR_UNSUPPORTED = 4,      /* valid request with no kernel: caller may fall back */
  QG_ERR_BUFFER_TOO_SMALL = 5, /* packed buffer or workspace below the required size */
  QG_ERR_HIP = 6               /* a HIP call failed; see qg_last_hip_error() */
} qg_status;

typedef enum {
  QG_W_INT4 = 0,   /* signed two's complement [-8, 7], no zero point */
  QG_W_UINT4 = 1,  /* unsigned [0, 15] with a uint4 zero point per group */
  QG_W_INT3 = 2,   /* signed two's complement [-4, 3], no zero point */
  QG_W_UINT3 = 3,  /* unsigned [0, 7] with a zero point per group */
  QG_W_MXFP4 = 4,  /* OCP e2m1 with one e8m0 scale per 32 along K */
  QG_W_INT8 = 5,   /* signed two's complement [-128, 127], no zero point */
  QG_W_UINT8 = 6,  /* unsigned [0, 255] with a uint8 zero point per group */
  QG_W_INT2 = 7,   /* signed two's complement [-2, 1], no zero point */
  QG_W_UINT2 = 8,  /* unsigned [0, 3] with a zero point per group */
  QG_W_INT1 = 9,   /* signed two's complement 1-bit: code 0 = 0, code 1 = -1 */
  QG_W_UINT1 = 10, /* unsigned [0, 1] with a zero point per group */
  QG_W_E0M3 = 11,  /* zero-exponent float: sign bit 3, magnitude bits 0..2 (-7..7) */
  QG_W_E0M7 = 12,  /* zero-exponent float: sign bit 7, magnitude bits 0..6 (-127..127) */
  QG_W_FP8 = 13    /* OCP e4m3 (one byte per weight) */
} qg_wtype;

typedef enum { QG_S_BF16 = 0, QG_S_E8M0 = 1, QG_S_F32 = 2 } qg_stype;
/* FP8_TOKEN: e4m3 bytes with one fp32 scale per row (x_scales [rows]).
 * FP8_BLOCK: e4m3 bytes with one fp32 scale per row and 128 K (x_scales
 * [rows][K/128], row stride K/128). */
typedef enum { QG_A_BF16 = 0, QG_A_MXFP8 = 1, QG_A_MXFP4 = 2, QG_A_FP8_TOKEN = 3, QG_A_FP8_BLOCK = 4 } qg_atype;
typedef enum { QG_O_BF16 = 0, QG_O_F32 = 1 } qg_otype;

/* How MoE rows are addressed.  A pair p = t*topk + j is token t's j-th expert
 * choice.  BY_TOKEN: row t of the operand (gate/up input).  BY_PAIR: row p
 * (down input, and the usual output).  SORTED: row i of the expert-sorted
 * order, i.e. the row of pair sorted_pair_ids[i]. */
typedef enum { QG_ROWS_BY_TOKEN = 0, QG_ROWS_BY_PAIR = 1, QG_ROWS_SORTED = 2 } qg_rowmode;

/* Layer + compute description ("Layer Config" / "Compute Config" of the
 * announcement's tuning section).  Supported (wtype, stype, atype, group):
 *   INT4/UINT4/INT3/UINT3, BF16 scales, BF16 activations, group 32, 64 or 128;
 *   INT8/UINT8/INT2/UINT2/INT1/UINT1, E0M3/E0M7 and FP8 (e4m3), BF16 scales,
 *   BF16 activations, group 32, 64 or 128 (the announcement's "WnA16"
 *   section: integer and floating-point weights of 1 to 8 bits on the shared
 *   dequantize-and-compute path; e0m codes, section "Quantization support",
 *   hold the values of INT4 without -8 / INT8 without -128 and are stored as
 *   those integers; the LDS-tiled large-M kernels serve the 4- and 3-bit
 *   formats and E0M3; the others run the decode kernels up to 16 rows when
 *   K % 512 == 0 and the 16-row skinny kernel otherwise);
 *   MXFP4, E8M0 scales, FP8_TOKEN activations, group 32 (W4A8 with per-token
 *   FP8 activations, section "End to end": the scaled MFMA with unit
 *   activation block scales, each output row times its row's fp32 scale;
 *   skinny kernel below 128 rows (dense) or for experts with few rows (MoE),
 *   the LDS-tiled scaled-MFMA kernel otherwise);
 *   FP8 (e4m3), F32 scales, FP8_BLOCK activations, group 128 (W8A8 with
 *   block-wise scaling, section "W8A8 / W4A8 / W4A4": one fp32 scale per
 *   128 x 128 block of W, scales [N/128 rounded up][K/128]; K % 128 == 0;
 *   skinny kernel below 128 rows (dense) or for experts with few rows (MoE),
 *   the LDS-tiled e4m3 x e4m3 scaled-MFMA kernel otherwise);
 *   MXFP4, E8M0 scales, MXFP8 activations, group 32 (W4A8 on the scaled MFMA);
 *   MXFP4, E8M0 scales, BF16 activations, group 32 (each code dequantized in
 *   the kernel to the exact bf16 e2m1 * 2^(e-127); the announcement's
 *   "Choosing the activation type": MXFP4 checkpoints on a bf16 compute path);
 *   MXFP4, E8M0 scales, MXFP4 activations, group 32, K % 128 == 0 (W4A4, the
 *   announcement's "W8A8 / W4A8 / W4A4" section: dense calls from 128 rows
 *   put both e2m1 operands into the scaled MFMA, and so do qg_moe_gemm's
 *   tiled kernels; the skinny kernel (dense below 128 rows, MoE experts with
 *   few rows) widens each activation fragment to e4m3 in registers -- every
 *   e2m1 value is an e4m3 value under the same scale).
 * Other valid combinations return QG_ERR_UNSUPPORTED. */
typedef struct {
  int32_t abi_version; /* must be QG_ABI_VERSION */
  int32_t wtype;       /* qg_wtype */
  int32_t stype;       /* qg_stype */
  int32_t group_size;  /* K elements per scale */
  int32_t atype;       /* qg_atype the weights will be multiplied with */
  int32_t num_experts; /* 1 for a dense layer */
  int64_t n;           /* output features (rows of W) */
  int64_t k;           /* input features; must be a multiple of 32 and of group_size */
} qg_layer_desc;

/* A preprocessed weight: plain data, owned by the caller, safe to copy.
 * Filled by qg_preprocess (or qg_weight_bind for a blob packed earlier). */
typedef struct {
  qg_layer_desc desc;
  void *data;              /* device buffer holding the packed layout */
  uint64_t bytes;          /* size of data in bytes */
  int32_t layout_version;  /* QG_LAYOUT_VERSION */
  int32_t n_tiles;         /* ceil(N / 16) */
  int32_t k_blocks;        /* K / 128 rounded up */
  int32_t groups_padded;   /* K / group rounded up to a multiple of 32 */
  uint64_t expert_stride;  /* bytes from one expert's section to the next */
  uint64_t scales_offset;  /* byte offset of the scales inside an expert section */
  uint64_t zeros_offset;   /* byte offset of the zero points (0 if none) */
} qg_weight;

/* Bytes of device memory the packed layout of `desc` needs (all experts). */
qg_status qg_packed_size(const qg_layer_desc *desc, uint64_t *bytes);

/* Host-only repack of experts [expert_begin, expert_begin + expert_count) from
 * the standard format into the packed layout.  codes/scales/zeros point at the
 * first of those experts (host memory, standard format).  dst is a host buffer
 * of qg_packed_size bytes laid out for all experts; only the given experts'
 * sections are written.  Runs on the CPU; needs no GPU. */
qg_status qg_repack_host(const qg_layer_desc *desc, const void *codes, const void *scales,
                         const void *zeros, int32_t expert_begin, int32_t expert_count,
                         void *dst, uint64_t dst_bytes);

/* Validate, pad and repack host standard-format tensors for experts
 * [expert_begin, expert_begin + expert_count) and copy them into the device
 * buffer dst_dev (qg_packed_size bytes, 256-byte aligned).  Fills *out (which
 * is valid once every expert has been preprocessed).  Synchronizes `stream`
 * before returning. */
qg_status qg_preprocess(const qg_layer_desc *desc, const void *codes, const void *scales,
                        const void *zeros, int32_t expert_begin, int32_t expert_count,
                        void *dst_dev, uint64_t dst_bytes, hipStream_t stream, qg_weight *out);

/* Describe an already packed device blob (e.g. one restored from storage that
 * qg_repack_host produced) without touching it. */
qg_status qg_weight_bind(const qg_layer_desc *desc, void *dst_dev, uint64_t dst_bytes,
                         qg_weight *out);

/* Workspace bytes qg_gemm needs for `m` rows (0 when none is needed).
 * Layout of a dense workspace: the first 64 KiB hold the arrival counters of
 * split-K launches (one per output tile; a launch that splits K counts its
 * workgroups in and leaves the counters at zero again), and the bytes after
 * them are scratch (fp32 partial tiles, the large-M kernels' pre-pass
 * results) whose contents never matter.  So a workspace must be zero-filled
 * once before its first use (its first 64 KiB suffice) and then serves any
 * sequence of qg_gemm / qg_gemm_ex calls -- any layer, any m -- ordered on one
 * stream, provided it holds the size each call asks for. */
qg_status qg_gemm_workspace_size(const qg_weight *w, int64_t m, uint64_t *bytes);

/* Dense GEMM: y[m][n] = x[m][:K] * dequant(W)^T.
 *   x        device, [m][ldx] bf16, e4m3 bytes or e2m1 nibble pairs (per
 *            desc.atype), 16-B aligned, ldx >= K and the row pitch (ldx
 *            elements) a multiple of 16 bytes (ldx % 32 == 0 for MXFP4).
 *   x_scales device, [m][K/32] e8m0 (MX activations), fp32 [m] (FP8_TOKEN)
 *            or fp32 [m][K/128] (FP8_BLOCK), 4-B aligned for fp32; ignored /
 *            may be NULL for bf16 activations.
 * The MX large-M kernel addresses X with 32-bit offsets: an MX call whose
 * activation rows span 4 GiB or more (m * row pitch) returns
 * QG_ERR_UNSUPPORTED.
 *   y        device, [m][ldy] of otype, 16-B aligned, ldy >= N.
 *   ws       device workspace of at least qg_gemm_workspace_size bytes
 *            (may be NULL when that size is 0).
 * m == 0 is a no-op returning QG_OK.  Asynchronous on `stream`. */
qg_status qg_gemm(const qg_weight *w, const void *x, const void *x_scales, int64_t m,
                  int64_t ldx, void *y, int32_t otype, int64_t ldy, void *ws, uint64_t ws_bytes,
                  hipStream_t stream);
/* (ws, when needed, must hold zeros on entry; see qg_gemm_workspace_size.) */

/* qg_gemm for callers that cannot allocate memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * kernels, with the workspace replaced by a static device array of
 * QG_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds until the
 * process ends.  The call allocates nothing (no hipMalloc / hipFree, no
 * allocating library call); on its first use on a device it looks the
 * array's address up and clears its split-K counter prefix with a kernel on
 * `stream`.  Every call on one GPU shares that GPU's array and the array
 * keeps the last call's contents: calls that may overlap on one GPU (other
 * streams, other threads) race and must be ordered by the caller.  A call
 * whose kernels would need more scratch than the array holds returns
 * QG_ERR_BUFFER_TOO_SMALL before launching anything (qg_gemm with a caller
 * workspace serves it).  Arguments and all other errors as in qg_gemm. */
#define QG_NOALLOC_SCRATCH_BYTES (8u << 20)
qg_status qg_gemm_noalloc(const qg_weight *w, const void *x, const void *x_scales, int64_t m, int64_t ldx,
                          void *y, int32_t otype, int64_t ldy, hipStream_t stream);

/* Compute options of qg_gemm_ex (the announcement's "Compute Config" names
 * batch invariance among the compute options of a GEMM, section "Per-workload
 * tuning and JIT compilation").
 *   QG_GEMM_BATCH_INVARIANT: every output row is bit-identical whatever m is
 *   (and whatever the other rows hold): the kernel and its reduction order
 *   are chosen from (N, K) only, never from m.  Slower than the default at
 *   small m (the large-M kernel serves every m when K % 128 == 0).  An
 *   integer-format layer with m * K * 2 >= 2^31 returns QG_ERR_UNSUPPORTED
 *   rather than switching kernels. */
#define QG_GEMM_BATCH_INVARIANT 1u

/* qg_gemm_workspace_size for the compute options `flags` (0 = qg_gemm's). */
qg_status qg_gemm_workspace_size_ex(const qg_weight *w, int64_t m, uint32_t flags, uint64_t *bytes);

/* qg_gemm with compute options `flags` (a combination of QG_GEMM_* bits;
 * unknown bits: QG_ERR_INVALID_ARGUMENT).  flags == 0 is exactly qg_gemm.
 * ws must hold qg_gemm_workspace_size_ex(w, m, flags) bytes, zero-filled once
 * as for qg_gemm. */
qg_status qg_gemm_ex(const qg_weight *w, const void *x, const void *x_scales, int64_t m,
                     int64_t ldx, void *y, int32_t otype, int64_t ldy, void *ws, uint64_t ws_bytes,
                     uint32_t flags, hipStream_t stream);

/* Autotune of the dense tuning table (announcement, "Future plans": candidate
 * configurations are benchmarked on the target device to find better
 * execution parameters per workload, complementing the heuristics).
 * qg_gemm_autotune runs the dense GEMM of this call once per candidate kernel
 * variant (the heuristic's choice, the decode / skinny / tiled kernels' other
 * compiled shapes that can serve m rows), times each with HIP events over
 * `reps` launches (1..64) after one warm-up launch, and records the fastest in
 * a process-wide table keyed by (wtype, group, N, K) and the M bucket of m
 * (1, 2-4, 5-8, 9-16, 17-64, 65-256, 257-1024, > 1024).  From then on qg_gemm,
 * qg_gemm_workspace_size and qg_describe_dispatch use that variant for every
 * m of the bucket it can serve (otherwise the heuristics); batch-invariant
 * calls ignore the table.  Query qg_gemm_workspace_size again after tuning:
 * the tuned variant may need a different workspace.
 *   x, x_scales, ldx, y, otype, ldy  as in qg_gemm; y is overwritten (the
 *            result of the last candidate run).
 *   ws       device, 256-B aligned, qg_gemm_autotune_workspace_size bytes;
 *            contents on entry do not matter (the call clears what must
 *            start at zero).  Not a qg_gemm workspace: it leaves scratch.
 *   flush    optional device buffer (16-B aligned, flush_bytes a multiple of
 *            16) read in full before every timed launch so that each launch
 *            starts from cold caches (pass more than the 256 MB MALL), or NULL.
 *   chosen   optional host buffer receiving the chosen variant's description;
 *   chosen_us optional host float receiving its mean time per launch (us).
 * Synchronizes `stream`.  Thread-safe (the table is guarded by a mutex). */
qg_status qg_gemm_autotune_workspace_size(const qg_weight *w, int64_t m, uint64_t *bytes);
qg_status qg_gemm_autotune(const qg_weight *w, const void *x, const void *x_scales, int64_t m,
                           int64_t ldx, void *y, int32_t otype, int64_t ldy, void *ws, uint64_t ws_bytes,
                           const void *flush, uint64_t flush_bytes, int32_t reps, hipStream_t stream,
                           char *chosen, uint64_t chosen_bytes, float *chosen_us);
/* MoE autotune (announcement, section "Future plans": benchmark candidate
 * configurations on the target device, complementing the heuristics).
 * qg_moe_autotune runs this grouped GEMM (the arguments of qg_moe_gemm, with
 * num_tokens >= 1 and the pairs already sorted by qg_moe_sort) once per
 * candidate dispatch plan -- every expert on the skinny kernel, or experts
 * with >= 16, 32, 64 or 128 rows on the tiled kernels' 128-row tiles and the
 * rest on the 64-row small tiles or the skinny kernel, MX tiles 128 or 256
 * columns wide -- times each with HIP events over `reps` calls (1..64) after
 * one warm-up call, and records the fastest plan in a process-wide table keyed
 * by (wtype, atype, group, N, K, experts) and the bucket of num_tokens * topk
 * (1-8, 9-64, 65-512, 513-4096, 4097-32768, more).  From then on qg_moe_gemm,
 * qg_moe_workspace_size and qg_describe_moe_dispatch use that plan for the
 * bucket (unless an experiment override of the MoE dispatch is set); query
 * qg_moe_workspace_size again after tuning.  y is overwritten (the last
 * candidate's result).
 *   ws     device, 256-B aligned, qg_moe_autotune_workspace_size bytes;
 *          contents on entry do not matter.  Not a qg_moe_gemm workspace.
 *   flush, flush_bytes, reps, chosen, chosen_bytes, chosen_us  as in
 *          qg_gemm_autotune (chosen: the plan's description).
 * Synchronizes `stream`.  Thread-safe (the table is guarded by a mutex). */
qg_status qg_moe_autotune_workspace_size(const qg_weight *w, int64_t num_tokens, int32_t topk, uint64_t *bytes);
qg_status qg_moe_autotune(const qg_weight *w, const void *x, const void *x_scales, int32_t x_rows,
                          const int32_t *sorted_pair_ids, const int32_t *expert_offsets, int64_t num_tokens,
                          int32_t topk, void *y, int32_t otype, int32_t y_rows, void *ws, uint64_t ws_bytes,
                          const void *flush, uint64_t flush_bytes, int32_t reps, hipStream_t stream, char *chosen,
                          uint64_t chosen_bytes, float *chosen_us);
/* Forget every autotuned entry, dense and MoE (back to the heuristics). */
void qg_autotune_reset(void);

/* Experiment overrides of the tuning table, for tests and parameter sweeps
 * (production code sets none).  At the first dispatch of the process the
 * library reads the environment variables of these names once; after that
 * only these calls change them.  name is one of QG_TUNE ("T,KR,W,splits": the
 * skinny kernel with these parameters), QG_DECODE ("0" disables the decode
 * kernel, "T,KR[,splits]" picks an instance), QG_TILED ("0" disables the
 * large-M kernels), QG_TILED_BM, QG_MX_BN, QG_MX_WAVES, QG_A16_WAVES,
 * QG_A16_BN, QG_MOE_TILED_MIN, QG_MOE_GROUP_M, QG_MOE_SMALL_BM, QG_MOE_SMALL,
 * QG_MOE_MX_BN, QG_DECODE_WIDE, QG_GROUP_M; value NULL or "" clears the override.  An unknown name returns
 * QG_ERR_INVALID_ARGUMENT.  A value outside an override's range is ignored
 * (the heuristic applies).  Thread-safe; a dispatch sees the overrides before
 * or after a concurrent change, never a mix.  qg_clear_overrides clears all
 * (the environment is not read again). */
qg_status qg_set_override(const char *name, const char *value);
void qg_clear_overrides(void);

/* Workspace bytes for qg_moe_sort and qg_moe_gemm with this many tokens (one
 * buffer of this size serves both; its contents on entry do not matter). */
qg_status qg_moe_workspace_size(const qg_weight *w, int64_t num_tokens, int32_t topk,
                                uint64_t *bytes);

/* Route-sort the pairs of a top-k router by expert (counting sort on the GPU).
 *   topk_ids        device int32 [num_tokens][topk], values in 0..num_experts-1
 *                   (out-of-range ids are skipped and counted nowhere).
 *   sorted_pair_ids device int32 [num_tokens*topk]: pair ids grouped by expert;
 *                   the order inside an expert's segment is unspecified.
 *   expert_offsets  device int32 [num_experts+1]: segment e is
 *                   [offsets[e], offsets[e+1]).
 *   ws              device workspace of qg_moe_workspace_size bytes.
 * Asynchronous on `stream`.  num_tokens == 0 writes zero offsets. */
qg_status qg_moe_sort(const int32_t *topk_ids, int64_t num_tokens, int32_t topk,
                      int32_t num_experts, int32_t *sorted_pair_ids, int32_t *expert_offsets,
                      void *ws, uint64_t ws_bytes, hipStream_t stream);

/* Grouped GEMM over the sorted pairs: for every pair p routed to expert e,
 * (any K that is a multiple of 32 and of the group; long K loops inside the
 * kernels' workgroups)
 *   y[row_y(p)] = x[row_x(p)] * dequant(W[e])^T
 * with row_x given by x_rows (BY_TOKEN: p / topk; BY_PAIR: p; SORTED: the
 * pair's position in sorted_pair_ids) and row_y by y_rows (BY_PAIR or SORTED).
 * x, x_scales, y as in qg_gemm with ldx = K and ldy = N (dense rows).
 * ws: device, 256-B aligned, at least qg_moe_workspace_size bytes (holds the
 * tile list of the large-expert kernel and, for integer formats, the group
 * row sums of x; overwritten by every call, so calls sharing one ws must be
 * ordered on one stream).
 * More than 1024 experts: QG_ERR_UNSUPPORTED (here and in qg_moe_sort).
 * Asynchronous on `stream`. */
qg_status qg_moe_gemm(const qg_weight *w, const void *x, const void *x_scales, int32_t x_rows,
                      const int32_t *sorted_pair_ids, const int32_t *expert_offsets,
                      int64_t num_tokens, int32_t topk, void *y, int32_t otype, int32_t y_rows,
                      void *ws, uint64_t ws_bytes, hipStream_t stream);

/* Activation quantization bf16 -> MXFP8 (announcement, section "Choosing the
 * activation type": a deployment may run a layer with MXFP8 activations on a
 * bf16 model, e.g. the MoE layers, so activations are quantized at run time
 * before the W4A8 GEMM).  Per row, per block of 32 values along K, following
 * the OCP Microscaling Formats v1.0 conversion: scale X = 2^(floor(log2
 * max|v|) - 8) clamped to 2^-127 .. 2^127 (X = 1 for an all-zero block), stored
 * as the e8m0 code log2(X) + 127; element = v / X rounded to the nearest e4m3
 * value, ties to the even code, magnitudes beyond 448 saturated to 448, sign
 * kept (a negative value that rounds to zero gives 0x80).  The result is
 * exact (no fp32 rounding is involved for bf16 inputs).
 *   x        device, bf16 [rows][ldx], 16-B aligned, ldx >= k, ldx % 8 == 0.
 *   q        device, e4m3 bytes [rows][ldq], 8-B aligned, ldq >= k, ldq % 8 == 0.
 *   q_scales device, e8m0 bytes [rows][k/32] (row stride k/32, the x_scales
 *            layout of qg_gemm / qg_moe_gemm), any alignment.
 * k % 32 != 0 or ld too small: QG_ERR_SHAPE.  rows == 0 or k == 0: no-op.
 * NaN / Inf inputs give unspecified codes.  Asynchronous on `stream`. */
qg_status qg_quantize_mxfp8(const void *x, int64_t rows, int64_t k, int64_t ldx, void *q,
                            int64_t ldq, void *q_scales, hipStream_t stream);

/* bf16 activations -> MXFP4 (e2m1 codes + e8m0 scales), the input of a W4A4
 * GEMM (announcement, section "W8A8 / W4A8 / W4A4": MXFP4 on both operands).
 * Per row, per block of 32 values along K, the OCP Microscaling Formats v1.0
 * conversion with e2m1's largest power of two, 2^2: scale X = 2^(floor(log2
 * max|v|) - 2) clamped to 2^-127 .. 2^127 (X = 1 for an all-zero block),
 * stored as the e8m0 code log2(X) + 127; element = v / X rounded to the
 * nearest e2m1 value (0, 0.5, 1, 1.5, 2, 3, 4, 6), ties to the even code,
 * magnitudes beyond 6 saturated to 6, sign kept (a negative value that rounds
 * to zero gives code 0x8).  Exact for bf16 inputs (no fp32 rounding).
 *   x        device, bf16 [rows][ldx], 16-B aligned, ldx >= k, ldx % 8 == 0.
 *   q        device, e2m1 nibble pairs [rows][ldq elements] (element j in the
 *            low nibble of byte j/2 when j is even), 4-B aligned, ldq >= k,
 *            ldq % 8 == 0.
 *   q_scales device, e8m0 bytes [rows][k/32] (row stride k/32), any alignment.
 * k % 32 != 0 or ld too small: QG_ERR_SHAPE.  rows == 0 or k == 0: no-op.
 * NaN / Inf inputs give unspecified codes.  Asynchronous on `stream`. */
qg_status qg_quantize_mxfp4(const void *x, int64_t rows, int64_t k, int64_t ldx, void *q,
                            int64_t ldq, void *q_scales, hipStream_t stream);

/* bf16 activations -> e4m3 with fp32 scales: per token (block == 0, one scale
 * per row; the announcement's section "End to end" serves W4A8 with per-token
 * FP8 activations) or per 128 values of a row (block == 128, the W8A8 input;
 * section "W8A8 / W4A8 / W4A4").  Per block with largest magnitude a (a
 * bf16 value, exact in fp32): scale s = a / 448 in IEEE fp32 (nearest-even;
 * s = 1 for an all-zero block); code = e4m3 of the fp32 quotient v / s
 * (IEEE division), nearest with ties to the even code, saturated at 448, sign
 * kept (a negative value that rounds to zero gives 0x80).
 *   x        device, bf16 [rows][ldx], 16-B aligned, ldx >= k, ldx % 8 == 0.
 *   q        device, e4m3 bytes [rows][ldq], 16-B aligned, ldq >= k, ldq % 16 == 0.
 *   q_scales device, fp32 [rows] (block 0) or [rows][ceil(k/128)] (block 128,
 *            row stride ceil(k/128)), 4-B aligned.
 * k % 8 != 0 or ld too small: QG_ERR_SHAPE; block not 0 or 128:
 * QG_ERR_INVALID_ARGUMENT.  rows == 0 or k == 0: no-op.  NaN / Inf inputs give
 * unspecified codes.  Asynchronous on `stream`. */
qg_status qg_quantize_fp8(const void *x, int64_t rows, int64_t k, int64_t ldx, int32_t block, void *q,
                          int64_t ldq, float *q_scales, hipStream_t stream);

/* SiLU-gated product of a fused gate/up projection (MoE output stage between
 * gate_up and down; announcement, section "Shared CUDA components": scaling
 * and bias work belongs to the output stage):
 *   h[r][j] = silu(gu[r][j]) * gu[r][inter + j],  silu(v) = v / (1 + e^-v),
 * for j < inter, computed in fp32 and rounded to bf16 (nearest-even).  With
 * h_type QG_A_MXFP8 those bf16 values are then quantized exactly as
 * qg_quantize_mxfp8 does, ready for an MXFP8 down projection.
 *   gu       device, [rows][ldgu] of gu_type (QG_O_BF16 or QG_O_F32, i.e. the
 *            gate_up GEMM's output type), 16-B aligned, ldgu >= 2*inter,
 *            rows 16-B aligned (ldgu % 8 for bf16, % 4 for fp32).
 *   h        device, [rows][ldh]: bf16 (16-B aligned, ldh % 8 == 0) or e4m3
 *            bytes (8-B aligned, ldh % 8 == 0), ldh >= inter.
 *   h_scales device, e8m0 [rows][inter/32] (QG_A_MXFP8 only, else ignored).
 * inter % 8 (bf16 output) or % 32 (MXFP8 output) != 0: QG_ERR_SHAPE.
 * rows == 0 is a no-op.  Asynchronous on `stream`. */
qg_status qg_silu_mul(const void *gu, int32_t gu_type, int64_t rows, int64_t inter, int64_t ldgu,
                      void *h, int32_t h_type, int64_t ldh, void *h_scales, hipStream_t stream);

/* Weighted combine of each token's top-k expert rows (MoE output stage):
 *   out[t][c] = sum_j topk_weights[t][j] * y[t*topk + j][c]  (+ bias[c])
 * summed in fp32 over j = 0 .. topk-1 in order, then stored as out_type
 * (bf16 nearest-even, or fp32).  y holds one row per pair p = t*topk + j, i.e.
 * the QG_ROWS_BY_PAIR output of qg_moe_gemm.
 *   y            device, [num_tokens*topk][ldy] of y_type (QG_O_BF16 / QG_O_F32),
 *                16-B aligned rows.
 *   topk_weights device, fp32 [num_tokens][topk], 4-B aligned.
 *   bias         device, bf16 [n] (16-B aligned) or NULL.
 *   out          device, [num_tokens][ldout] of out_type, 16-B aligned rows.
 * n % 8 != 0 or ld too small: QG_ERR_SHAPE; topk < 1: QG_ERR_INVALID_ARGUMENT.
 * num_tokens == 0 is a no-op.  out must not overlap y.  Asynchronous. */
qg_status qg_moe_combine(const void *y, int32_t y_type, int64_t ldy, const float *topk_weights,
                         int64_t num_tokens, int32_t topk, int64_t n, const void *bias, void *out,
                         int32_t out_type, int64_t ldout, hipStream_t stream);

/* Measurement utilities, used for roofline calibration and cold-cache timing.
 * qg_stream_read reads `bytes` (a multiple of 16; src 16-B aligned, device)
 * with 128-bit loads and folds them into `sink` (device, at least 16 KiB, any
 * contents); nothing else is written.  Reading a buffer larger than the 256 MB
 * MALL evicts earlier data from the caches.  qg_stream_copy copies `bytes`
 * (a multiple of 16, both pointers 16-B aligned, device, non-overlapping).
 * Both are asynchronous on `stream`. */
qg_status qg_stream_read(const void *src, uint64_t bytes, void *sink, hipStream_t stream);
qg_status qg_stream_copy(void *dst, const void *src, uint64_t bytes, hipStream_t stream);

/* Name of the kernel variant the tuning table selects for `m` rows (dense) or
 * `m` pairs (MoE: the skinny kernel's variant for experts with few rows) and
 * the tile parameters, written as a NUL-terminated string into buf.
 * qg_describe_dispatch_ex does the same for the compute options `flags` of
 * qg_gemm_ex (dense layers only). */
qg_status qg_describe_dispatch(const qg_weight *w, int64_t m, char *buf, uint64_t buf_bytes);
qg_status qg_describe_dispatch_ex(const qg_weight *w, int64_t m, uint32_t flags, char *buf, uint64_t buf_bytes);

/* The MoE dispatch of qg_moe_gemm for num_tokens * topk pairs, as text:
 * which kernel serves experts by row count (the tiled kernels' row threshold,
 * the small-tile form or the skinny kernel's variant below it).  Which
 * experts fall on which side depends on the routing (device data). */
qg_status qg_describe_moe_dispatch(const qg_weight *w, int64_t num_tokens, int32_t topk, char *buf,
                                   uint64_t buf_bytes);

/* Static description of a status code (never NULL). */
const char *qg_status_string(qg_status status);

/* The hipError_t behind the calling thread's last QG_ERR_HIP (0 if none). */
int32_t qg_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QG_H_ */
