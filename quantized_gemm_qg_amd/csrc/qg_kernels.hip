// HIP kernels for gfx950 (MI355X): quantized GEMM with in-kernel
// dequantization, dense and MoE-grouped, plus the MoE routing sort.
//
// The announcement's "Shared CUDA components" section splits a quantized GEMM
// kernel into task scheduling, data movement, dequantization + scaling,
// matrix-core compute and an output stage; the same split is used here, built
// for CDNA4:
//
//   scheduling   one work item = (16-row tile, 16*T output columns, K split);
//                dense launches one workgroup per item, the MoE launch loops a
//                persistent grid over items derived from the expert offsets.
//   data path    weights stream HBM -> VGPR with one 128-bit load per lane per
//                16x128 block (the packed layout puts each lane's MFMA B
//                operand in one contiguous 16-byte slice); activations go
//                straight from global memory (L2) into MFMA A-operand registers
//                and are reused for every output tile of the wave.
//   dequant      integer codes u become bf16 (1 + u/16) (INT4) or (1 + u/8)
//                (INT3) with one shift + and/or per pair of codes (the code
//                lands in the top mantissa bits); the offset and zero point
//                are removed per K-group on the MFMA partial sums:
//                  sum x*(u - z) = MAG * sum x*(1 + u/MAG) - (MAG + z) * sum x
//                so the group scale s applies as two fp32 FMAs per accumulator,
//                and (u - z) * s is exact.  MXFP4 x MXFP8 needs no conversion:
//                e2m1 codes and e8m0 scales feed the scaled MFMA directly.
//   compute      v_mfma_f32_16x16x32_bf16, v_mfma_scale_f32_16x16x128_f8f6f4.
//   output       workgroup waves (split along K) reduce through LDS in a fixed
//                order; a cross-workgroup K split writes fp32 partials and the
//                last workgroup of a tile (device-scope counter) sums them in
//                split order, so results do not depend on arrival order.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "qg_device.h"
#include "qg_internal.h"
#include "qg_wave.h"

namespace qg {

// Plain streaming kernels (measurement utilities): grid-stride 128-bit loads,
// four in flight per lane.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *src, uint64_t n16,
                                                          uint32_t *sink) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) sink[(blockIdx.x * blockDim.x + threadIdx.x) & 4095] = acc;  // keeps the loads live
}

__global__ __launch_bounds__(256) void stream_copy_kernel(u32x4 *dst, const u32x4 *src,
                                                          uint64_t n16) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    dst[i] = __builtin_nontemporal_load(src + i);
}

hipError_t launch_stream_read(const void *src, uint64_t bytes, void *sink, hipStream_t s) {
  const uint64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const uint64_t want = (n16 + 1023) / 1024;
  const unsigned blocks = (unsigned)std::min<uint64_t>(std::max<uint64_t>(want, 1), 256 * 16);
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, s, (const u32x4 *)src, n16,
                     (uint32_t *)sink);
  return hipGetLastError();
}

hipError_t launch_stream_copy(void *dst, const void *src, uint64_t bytes, hipStream_t s) {
  const uint64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<uint64_t>((n16 + 255) / 256, 256 * 16);
  hipLaunchKernelGGL(stream_copy_kernel, dim3(blocks), dim3(256), 0, s, (u32x4 *)dst,
                     (const u32x4 *)src, n16);
  return hipGetLastError();
}

// Counting sort of router pairs by expert in one workgroup (LDS histogram).
__global__ __launch_bounds__(1024) void moe_sort_kernel(const int32_t *ids, int64_t pairs,
                                                        int32_t experts, int32_t *sorted,
                                                        int32_t *offsets) {
  __shared__ int cnt[kMaxExperts + 1];
  __shared__ int cur[kMaxExperts];
  const int tid = threadIdx.x, nth = blockDim.x;
  for (int e = tid; e < experts; e += nth) cnt[e] = 0;
  __syncthreads();
  for (int64_t p = tid; p < pairs; p += nth) {
    const int e = ids[p];
    if (e >= 0 && e < experts) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < experts; ++e) {
      const int c = cnt[e];
      cnt[e] = run;
      cur[e] = run;
      run += c;
    }
    cnt[experts] = run;
  }
  __syncthreads();
  for (int e = tid; e <= experts; e += nth) offsets[e] = cnt[e];
  for (int64_t p = tid; p < pairs; p += nth) {
    const int e = ids[p];
    if (e >= 0 && e < experts) sorted[atomicAdd(&cur[e], 1)] = (int32_t)p;
  }
}

// Tile list of the tiled MoE kernels: experts with min_rows <= rows <
// max_rows (max_rows <= 0: no bound), cut into bm-row tiles.  tiles[0] =
// count, tiles[1] = 0, then (expert, first sorted row) per tile in expert
// order; at most `capacity` tiles are written (counts are clamped to [0,
// pairs], so malformed offsets cannot overrun it).  Workgroup b builds list
// b (a launch builds one list, or both lists of a split between 128-row and
// small tiles).
struct TileListArgs {
  int32_t min_rows, max_rows, bm, capacity;
  int32_t *tiles;
};

__global__ __launch_bounds__(1024) void moe_tiles_kernel(const int32_t *offsets, int32_t experts, int32_t pairs,
                                                         TileListArgs l0, TileListArgs l1) {
  __shared__ int wave_tot[16];
  const TileListArgs &l = blockIdx.x == 0 ? l0 : l1;
  const int min_rows = l.min_rows, max_rows = l.max_rows, bm = l.bm, capacity = l.capacity;
  int32_t *tiles = l.tiles;
  const int tid = threadIdx.x, nth = blockDim.x;
  const int per = (experts + nth - 1) / nth;
  const int e0 = tid * per;
  auto ntiles = [&](int e) {
    const int c = min(max(offsets[e + 1] - offsets[e], 0), pairs);
    return c >= min_rows && (max_rows <= 0 || c < max_rows) ? (c + bm - 1) / bm : 0;
  };
  int local = 0;
  for (int e = e0; e < e0 + per && e < experts; ++e) local += ntiles(e);
  int total;
  int run = block_scan_excl(local, wave_tot, &total);
  if (tid == 0) {
    tiles[0] = min(total, capacity);
    tiles[1] = 0;
  }
  for (int e = e0; e < e0 + per && e < experts; ++e) {
    const int n = ntiles(e), first = offsets[e];
    for (int t = 0; t < n; ++t, ++run) {
      if (run >= capacity) return;
      tiles[2 + 2 * run] = e;
      tiles[3 + 2 * run] = first + t * bm;
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

template <int FMT, int GROUP>
static hipError_t launch_skinny(const GemmArgs &a, const Variant &v, bool moe, int64_t grid,
                                int64_t items, hipStream_t s) {
  dim3 block(64 * v.W);
  dim3 g((unsigned)grid);
  const size_t lds = (size_t)v.W * v.T * 256 * sizeof(float);
#define QG_KR_CASE(KRV)                                                                   \
  case KRV:                                                                               \
    if (v.T == 4)                                                                         \
      hipLaunchKernelGGL((skinny_kernel<FMT, GROUP, 4, KRV>), g, block, lds, s, a, (int)moe, items); \
    else if (v.T == 2)                                                                    \
      hipLaunchKernelGGL((skinny_kernel<FMT, GROUP, 2, KRV>), g, block, lds, s, a, (int)moe, items); \
    else                                                                                  \
      hipLaunchKernelGGL((skinny_kernel<FMT, GROUP, 1, KRV>), g, block, lds, s, a, (int)moe, items); \
    break;
  switch (v.KR) {
    QG_KR_CASE(1)
    QG_KR_CASE(2)
    QG_KR_CASE(4)
    default: return hipErrorInvalidValue;
  }
#undef QG_KR_CASE
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_fmt(const GemmArgs &a, int group, const Variant &v, bool moe,
                             int64_t grid, int64_t items, hipStream_t s) {
  if constexpr (FMT >= 4) {
    return group == 32 ? launch_skinny<FMT, 32>(a, v, moe, grid, items, s) : hipErrorInvalidValue;
  } else {
    switch (group) {
      case 32: return launch_skinny<FMT, 32>(a, v, moe, grid, items, s);
      case 64: return launch_skinny<FMT, 64>(a, v, moe, grid, items, s);
      case 128: return launch_skinny<FMT, 128>(a, v, moe, grid, items, s);
    }
    return hipErrorInvalidValue;
  }
}

static hipError_t launch_any(const GemmArgs &a, const qg_layer_desc &d, const Variant &v, bool moe,
                             int64_t grid, int64_t items, hipStream_t s) {
  if (v.W < 1 || v.W > kMaxWaves || (v.T != 1 && v.T != 2 && v.T != 4)) return hipErrorInvalidValue;
  if (grid <= 0) return hipSuccess;
  const int fmt = kernel_fmt(d);
  if (fmt >= 7) return launch_skinny_ext(a, fmt, d.group_size, v, moe, grid, items, s);
  switch (fmt) {
    case 0: return launch_fmt<0>(a, d.group_size, v, moe, grid, items, s);
    case 1: return launch_fmt<1>(a, d.group_size, v, moe, grid, items, s);
    case 2: return launch_fmt<2>(a, d.group_size, v, moe, grid, items, s);
    case 3: return launch_fmt<3>(a, d.group_size, v, moe, grid, items, s);
    case 5: return launch_fmt<5>(a, d.group_size, v, moe, grid, items, s);
    case 6: return launch_fmt<6>(a, d.group_size, v, moe, grid, items, s);
    default: return launch_fmt<4>(a, d.group_size, v, moe, grid, items, s);
  }
}

static hipError_t launch_dense(const GemmArgs &a, const qg_layer_desc &d, const Variant &v,
                               hipStream_t s) {
  const int64_t n_blocks = (a.n_tiles + v.T - 1) / v.T;
  const int64_t m_tiles = (a.m + 15) / 16;
  const int64_t items = n_blocks * m_tiles * v.splits;
  if (items > 0x7fffffffLL) return hipErrorInvalidValue;
  return launch_any(a, d, v, false, items, items, s);
}

template <int FMT, int GROUP>
static hipError_t launch_decode_g(const GemmArgs &a, const Variant &v, hipStream_t s) {
  const int n_blocks = (a.n_tiles + v.T - 1) / v.T;
  const size_t lds = (size_t)decode_lds_bytes(a.m, v.W, v.T, v.KR);
  if (lds > 160 * 1024 - 256) return hipErrorInvalidValue;  // (+ the kernel's static LDS)
#define QG_DECODE_LAUNCH(TV, KRV)                                                            \
  {                                                                                          \
    auto kern = a.m == 1 ? decode_kernel<FMT, GROUP, TV, KRV, 1> : decode_kernel<FMT, GROUP, TV, KRV, 4>; \
    hipError_t e = hipFuncSetAttribute((const void *)kern,                                   \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
    if (e != hipSuccess) return e;                                                           \
    hipLaunchKernelGGL(kern, dim3(n_blocks, v.splits), dim3(64 * v.W), lds, s, a);           \
    return hipGetLastError();                                                                \
  }
  // instances without register spills (a wave holds KR * 128 / GROUP group
  // scales per n-tile): every pair for group 128, T * KR <= 8 for group 64
  if constexpr (GROUP >= 64) {
    if (v.T == 4 && v.KR == 2) QG_DECODE_LAUNCH(4, 2)
    if (v.T == 2 && v.KR == 4) QG_DECODE_LAUNCH(2, 4)
  }
  if constexpr (GROUP == 128) {
    if (v.T == 4 && v.KR == 4) QG_DECODE_LAUNCH(4, 4)
    if (v.T == 1 && v.KR == 4) QG_DECODE_LAUNCH(1, 4)
    if (v.T == 1 && v.KR == 8) QG_DECODE_LAUNCH(1, 8)
    if (v.T == 2 && v.KR == 8) QG_DECODE_LAUNCH(2, 8)
  }
  // group 32 (4 scales per k-block: 16 dwords at KR = 8), one n-tile per wave
  if constexpr (GROUP == 32) {
    if (v.T == 1 && v.KR == 4) QG_DECODE_LAUNCH(1, 4)
    if (v.T == 1 && v.KR == 8) QG_DECODE_LAUNCH(1, 8)
  }
#undef QG_DECODE_LAUNCH
  return hipErrorInvalidValue;
}

template <int FMT>
static hipError_t launch_decode_f(const GemmArgs &a, int group, const Variant &v, hipStream_t s) {
  switch (group) {
    case 32: return launch_decode_g<FMT, 32>(a, v, s);
    case 64: return launch_decode_g<FMT, 64>(a, v, s);
    case 128: return launch_decode_g<FMT, 128>(a, v, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_a16(const GemmArgs &a, const qg_layer_desc &d, const Variant &v,
                             hipStream_t s) {
  if (a.m < 1 || a.m > 16 || a.k % 512 != 0 || v.splits < 1 || v.W * v.KR * 128 * v.splits < a.k)
    return hipErrorInvalidValue;
  if (v.splits > 1 && ((v.W * v.KR) % 4 != 0 || (v.splits - 1) * v.W * v.KR >= a.k_blocks ||
                       !a.partials || !a.counters))
    return hipErrorInvalidValue;
  const int fmt = kernel_fmt(d);
  if (fmt >= 7) return launch_decode_ext(a, fmt, d.group_size, v, s);
  switch (fmt) {
    case 0: return launch_decode_f<0>(a, d.group_size, v, s);
    case 1: return launch_decode_f<1>(a, d.group_size, v, s);
    case 2: return launch_decode_f<2>(a, d.group_size, v, s);
    case 3: return launch_decode_f<3>(a, d.group_size, v, s);
    case 5: return d.group_size == 32 ? launch_decode_g<5, 32>(a, v, s) : hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

template <int FMT, int GROUP>
static hipError_t launch_decode_wide_g(const GemmArgs &a, const Variant &v, hipStream_t s) {
  if (a.m < 2 || a.m > 16 || a.k % 512 != 0 || v.W < 1 || v.W > kMaxWaves || v.splits < 1 ||
      v.splits * v.KR < a.k_blocks || (v.splits > 1 && (!a.partials || !a.counters)))
    return hipErrorInvalidValue;
  const unsigned groups = (unsigned)((a.n_tiles + v.W - 1) / v.W);
  const size_t lds = (size_t)a.m * ((size_t)v.KR * 256 + 16);
  auto launch = [&](auto kern) -> hipError_t {
    hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(groups, v.splits), dim3(64 * v.W), lds, s, a);
    return hipGetLastError();
  };
  if (v.KR == 8) return launch(decode_wide_kernel<FMT, GROUP, 8, 4>);
  if (v.KR == 16) return launch(decode_wide_kernel<FMT, GROUP, 16, 4>);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_wide(const GemmArgs &a, const qg_layer_desc &d, const Variant &v, hipStream_t s) {
  const int fmt = kernel_fmt(d);
  if (fmt >= 7) return launch_decode_wide_ext(a, fmt, d.group_size, v, s);
  const int g = d.group_size;
  switch (fmt) {
#define QG_WIDE_FMT(F)                                                 \
  case F:                                                              \
    if (g == 32) return launch_decode_wide_g<F, 32>(a, v, s);          \
    if (g == 64) return launch_decode_wide_g<F, 64>(a, v, s);          \
    if (g == 128) return launch_decode_wide_g<F, 128>(a, v, s);        \
    return hipErrorInvalidValue;
    QG_WIDE_FMT(0)
    QG_WIDE_FMT(1)
    QG_WIDE_FMT(2)
    QG_WIDE_FMT(3)
#undef QG_WIDE_FMT
    case 5: return g == 32 ? launch_decode_wide_g<5, 32>(a, v, s) : hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_dense_a16(const GemmArgs &a, const qg_layer_desc &d, const Variant &v,
                            hipStream_t s) {
  return launch_dense(a, d, v, s);
}

hipError_t launch_dense_mx(const GemmArgs &a, const qg_layer_desc &d, const Variant &v,
                           hipStream_t s) {
  return launch_dense(a, d, v, s);
}

static hipError_t launch_moe(const GemmArgs &a, const qg_layer_desc &d, const Variant &v,
                             int64_t max_tiles, hipStream_t s) {
  if (a.num_experts > kMaxExperts) return hipErrorInvalidValue;
  const int64_t n_blocks = (a.n_tiles + v.T - 1) / v.T;
  // persistent grid: enough workgroups to fill the chip, never more than the
  // largest possible item count
  const int64_t cap = 256 * std::max(1, 16 / v.W) * 2;
  const int64_t grid = std::min<int64_t>(max_tiles * n_blocks, cap);
  return launch_any(a, d, v, true, grid, 0, s);
}

hipError_t launch_moe_a16(const GemmArgs &a, const qg_layer_desc &d, const Variant &v,
                          int64_t max_tiles, hipStream_t s) {
  return launch_moe(a, d, v, max_tiles, s);
}

hipError_t launch_moe_mx(const GemmArgs &a, const qg_layer_desc &d, const Variant &v,
                         int64_t max_tiles, hipStream_t s) {
  return launch_moe(a, d, v, max_tiles, s);
}

hipError_t launch_moe_tiles(const int32_t *offsets, int32_t experts, int32_t min_rows,
                            int32_t max_rows, int32_t bm, int32_t pairs, int32_t capacity,
                            int32_t *tiles, hipStream_t s) {
  const TileListArgs l{min_rows, max_rows, bm, capacity, tiles};
  hipLaunchKernelGGL(moe_tiles_kernel, dim3(1), dim3(1024), 0, s, offsets, experts, pairs, l, l);
  return hipGetLastError();
}

hipError_t launch_moe_tiles2(const int32_t *offsets, int32_t experts, int32_t pairs, int32_t min_rows,
                             int32_t capacity, int32_t *tiles, int32_t small_bm, int32_t capacity_small,
                             int32_t *tiles_small, hipStream_t s) {
  const TileListArgs big{min_rows, 0, kMoeTileRows, capacity, tiles};
  const TileListArgs small{1, min_rows, small_bm, capacity_small, tiles_small};
  hipLaunchKernelGGL(moe_tiles_kernel, dim3(2), dim3(1024), 0, s, offsets, experts, pairs, big, small);
  return hipGetLastError();
}

hipError_t launch_moe_sort(const int32_t *ids, int64_t pairs, int32_t experts, int32_t *sorted,
                           int32_t *offsets, int32_t *ws_counts, hipStream_t s) {
  (void)ws_counts;
  if (experts > kMaxExperts) return hipErrorInvalidValue;
  hipLaunchKernelGGL(moe_sort_kernel, dim3(1), dim3(1024), 0, s, ids, pairs, experts, sorted,
                     offsets);
  return hipGetLastError();
}

}  // namespace qg
