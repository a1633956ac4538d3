// Skinny- and decode-kernel instances for the weight formats beyond the 4- and
// 3-bit integers and MXFP4 (FMT 7 .. 15 of FmtTraits in qg_wave.h):
//   * 1-, 2- and 8-bit integer weights (signed, or with zero points), e0m7
//     (stored as offset-binary INT8) and e4m3 weights, all with bf16 group
//     scales and bf16 activations -- the announcement's "WnA16" section puts
//     integer and floating-point weights of 1 to 8 bits on one shared
//     dequantize-and-compute path, here a16x_wave;
//   * MXFP4 weights with per-token FP8 activations (section "End to end"),
//     the MX wave with unit activation block scales and the row scale in the
//     output stage;
//   * W8A8 FP8 with block scales (section "W8A8 / W4A8 / W4A4"), f8_wave.
// Kept in a translation unit of their own so the library's sources compile in
// parallel.  Skinny instances: the spill-free (T, KR) of the host's
// variant_ok; group 32, 64 or 128 for the bf16-activation formats, 32 for
// the per-token MX format, 128 for W8A8.  Decode: (T, KR) = (1, 4), (1, 8);
// wide decode: KR = 8, and 16 below 8-bit slices.
#include <hip/hip_runtime.h>

#include "qg_device.h"
#include "qg_internal.h"
#include "qg_wave.h"

namespace qg {

template <int FMT, int GROUP>
static hipError_t launch_skinny_x(const GemmArgs &a, const Variant &v, bool moe, int64_t grid, int64_t items,
                                  hipStream_t s) {
  dim3 block(64 * v.W);
  dim3 g((unsigned)grid);
  const size_t lds = (size_t)v.W * v.T * 256 * sizeof(float);
  // the host's variant_ok: the MX rule (T * KR <= 8, not 4 x 4) for
  // per-token FP8; else T <= 2 and T * KR <= 2 for 8-bit slices and group 32,
  // 4 otherwise
  constexpr int CAP = (FMT == 7 || FMT == 8 || FMT == 13 || (FMT <= 13 && GROUP == 32)) ? 2 : 4;
  auto inst = [](int t, int kr) { return FMT == 14 ? t * kr <= 8 && !(t == 4 && kr == 4) : t <= 2 && t * kr <= CAP; };
#define QG_X_CASE(TV, KRV)                                                                             \
  if constexpr (inst(TV, KRV)) {                                                                       \
    if (v.T == TV && v.KR == KRV) {                                                                    \
      hipLaunchKernelGGL((skinny_kernel<FMT, GROUP, TV, KRV>), g, block, lds, s, a, (int)moe, items); \
      return hipGetLastError();                                                                        \
    }                                                                                                  \
  }
  QG_X_CASE(1, 1)
  QG_X_CASE(1, 2)
  QG_X_CASE(1, 4)
  QG_X_CASE(2, 1)
  QG_X_CASE(2, 2)
  QG_X_CASE(2, 4)
  QG_X_CASE(4, 1)
  QG_X_CASE(4, 2)
#undef QG_X_CASE
  return hipErrorInvalidValue;
}

template <int FMT>
static hipError_t launch_skinny_groups(const GemmArgs &a, int group, const Variant &v, bool moe, int64_t grid,
                                       int64_t items, hipStream_t s) {
  switch (group) {
    case 32: return launch_skinny_x<FMT, 32>(a, v, moe, grid, items, s);
    case 64: return launch_skinny_x<FMT, 64>(a, v, moe, grid, items, s);
    case 128: return launch_skinny_x<FMT, 128>(a, v, moe, grid, items, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_skinny_ext(const GemmArgs &a, int fmt, int group, const Variant &v, bool moe, int64_t grid,
                             int64_t items, hipStream_t s) {
  switch (fmt) {
    case 7: return launch_skinny_groups<7>(a, group, v, moe, grid, items, s);
    case 8: return launch_skinny_groups<8>(a, group, v, moe, grid, items, s);
    case 9: return launch_skinny_groups<9>(a, group, v, moe, grid, items, s);
    case 10: return launch_skinny_groups<10>(a, group, v, moe, grid, items, s);
    case 11: return launch_skinny_groups<11>(a, group, v, moe, grid, items, s);
    case 12: return launch_skinny_groups<12>(a, group, v, moe, grid, items, s);
    case 13: return launch_skinny_groups<13>(a, group, v, moe, grid, items, s);
    case 14: return group == 32 ? launch_skinny_x<14, 32>(a, v, moe, grid, items, s) : hipErrorInvalidValue;
    case 15: return group == 128 ? launch_skinny_x<15, 128>(a, v, moe, grid, items, s) : hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

template <int FMT, int GROUP>
static hipError_t launch_decode_x(const GemmArgs &a, const Variant &v, hipStream_t s) {
  const int n_blocks = (a.n_tiles + v.T - 1) / v.T;
  const size_t lds = (size_t)decode_lds_bytes(a.m, v.W, v.T, v.KR);
  if (lds > 160 * 1024 - 256) return hipErrorInvalidValue;  // (+ the kernel's static LDS)
  if (v.T != 1 || (v.KR != 4 && v.KR != 8)) return hipErrorInvalidValue;
  auto pick = [&](auto kr_tag) {
    constexpr int KRV = decltype(kr_tag)::value;
    return a.m == 1 ? decode_kernel<FMT, GROUP, 1, KRV, 1> : decode_kernel<FMT, GROUP, 1, KRV, 4>;
  };
  auto kern = v.KR == 8 ? pick(std::integral_constant<int, 8>{}) : pick(std::integral_constant<int, 4>{});
  hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(n_blocks, v.splits), dim3(64 * v.W), lds, s, a);
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_decode_groups(const GemmArgs &a, int group, const Variant &v, hipStream_t s) {
  switch (group) {
    case 32: return launch_decode_x<FMT, 32>(a, v, s);
    case 64: return launch_decode_x<FMT, 64>(a, v, s);
    case 128: return launch_decode_x<FMT, 128>(a, v, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_ext(const GemmArgs &a, int fmt, int group, const Variant &v, hipStream_t s) {
  switch (fmt) {
    case 7: return launch_decode_groups<7>(a, group, v, s);
    case 8: return launch_decode_groups<8>(a, group, v, s);
    case 9: return launch_decode_groups<9>(a, group, v, s);
    case 10: return launch_decode_groups<10>(a, group, v, s);
    case 11: return launch_decode_groups<11>(a, group, v, s);
    case 12: return launch_decode_groups<12>(a, group, v, s);
    case 13: return launch_decode_groups<13>(a, group, v, s);
  }
  return hipErrorInvalidValue;
}

template <int FMT, int GROUP>
static hipError_t launch_decode_wide_x(const GemmArgs &a, const Variant &v, hipStream_t s) {
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
  if constexpr (FmtTraits<FMT>::BITS < 8)  // (16 blocks of 8-bit slices in flight spill)
    if (v.KR == 16) return launch(decode_wide_kernel<FMT, GROUP, 16, 4>);
  return hipErrorInvalidValue;
}

template <int FMT>
static hipError_t launch_decode_wide_groups(const GemmArgs &a, int group, const Variant &v, hipStream_t s) {
  switch (group) {
    case 32: return launch_decode_wide_x<FMT, 32>(a, v, s);
    case 64: return launch_decode_wide_x<FMT, 64>(a, v, s);
    case 128: return launch_decode_wide_x<FMT, 128>(a, v, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_wide_ext(const GemmArgs &a, int fmt, int group, const Variant &v, hipStream_t s) {
  switch (fmt) {
    case 7: return launch_decode_wide_groups<7>(a, group, v, s);
    case 8: return launch_decode_wide_groups<8>(a, group, v, s);
    case 9: return launch_decode_wide_groups<9>(a, group, v, s);
    case 10: return launch_decode_wide_groups<10>(a, group, v, s);
    case 11: return launch_decode_wide_groups<11>(a, group, v, s);
    case 12: return launch_decode_wide_groups<12>(a, group, v, s);
    case 13: return launch_decode_wide_groups<13>(a, group, v, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace qg
