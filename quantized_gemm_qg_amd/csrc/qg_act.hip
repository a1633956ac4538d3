// Activation-side kernels around the GEMMs: bf16 -> MXFP8 quantization of the
// activations and the MoE output stage (SiLU-gated product of the fused
// gate/up projection, weighted combine of a token's top-k expert rows).
//
// The announcement's section "Choosing the activation type" lets a deployment
// run MoE layers with MXFP8 activations on a checkpoint whose activations are
// bf16, so the activations are quantized at run time before the W4A8 GEMM;
// its section "Shared CUDA components" puts scaling and bias additions in the
// output stage.  Every kernel here is a single streaming pass bound by HBM:
// one lane owns 8 consecutive values along the row (a 16-byte bf16 load), four
// lanes own one 32-value MX block, and the block's largest magnitude is
// combined across the four lanes with two DPP quad permutations.
//
// MXFP8 conversion (OCP Microscaling Formats v1.0, section 6.3): the block's
// scale is X = 2^(floor(log2 max|v|) - 8), clamped to 2^-127 .. 2^127, X = 1 for
// an all-zero block; each element is v / X rounded to the nearest e4m3 value,
// ties to the even code, saturating at 448, keeping v's sign.  The inputs are
// bf16, so floor(log2 max|v|) is the exponent field of the largest magnitude
// and v / X only moves the binary point (exact in fp32); the one rounding is
// the hardware's fp32 -> e4m3 conversion, nearest-even.
//
// MXFP4 conversion (for W4A4, the announcement's section "W8A8 / W4A8 /
// W4A4"): the same rule with e2m1 elements, X = 2^(floor(log2 max|v|) - 2), the
// element rounded by the hardware's fp32 -> e2m1 conversion (nearest, ties to
// even, sign kept; the clamp to +-6 gives the saturation).
#include <hip/hip_runtime.h>

#include "qg_device.h"
#include "qg_internal.h"

namespace qg {

namespace {

// Scale exponent of a block whose largest magnitude has the fp32 pattern amax
// (a bf16 value widened, sign cleared): floor(log2) - 8, clamped at -127; 0
// for an all-zero block.
__device__ __forceinline__ int mx_block_exp(uint32_t amax) {
  if (amax == 0) return 0;
  return max((int)(amax >> 23) - 135, -127);  // subnormal maxima give -127 too
}

// e4m3 codes of two values already divided by the block scale.  The division
// by a power of two is exact for bf16 inputs (fp32 denormals are kept), the
// clamp to +-448 gives the saturation (values in (448, 464) round to 448
// anyway), and v_cvt_pk_fp8_f32 rounds to nearest-even into OCP e4m3; the
// sign survives, so a negative value that rounds to zero becomes 0x80.
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b) {
  a = __builtin_amdgcn_fmed3f(a, -448.f, 448.f);
  b = __builtin_amdgcn_fmed3f(b, -448.f, 448.f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// largest value over the lane's quad (lanes 4i .. 4i + 3)
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));  // [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
  return v;
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Quantizes the 8 bf16 values of this lane (4 words, two values each, low
// half first) as part of its quad's 32-value block: writes the 8 e4m3 codes
// to q8 and, from the quad's first lane, the scale code to *scale.
__device__ __forceinline__ void mx_store8(const uint32_t (&w)[4], uint8_t *q8, uint8_t *scale, bool first) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  const int e = mx_block_exp(quad_max(__float_as_uint(m)));
  const float inv = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, e in [-127, 119]
  uint32_t c[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
    c[h] = e4m3_pair(v[4 * h] * inv, v[4 * h + 1] * inv) | (e4m3_pair(v[4 * h + 2] * inv, v[4 * h + 3] * inv) << 16);
  *(uint2 *)q8 = uint2{c[0], c[1]};
  if (first) *scale = (uint8_t)(e + 127);
}

// MXFP4 form of mx_store8: the block scale is 2^(floor(log2 max|v|) - 2)
// (e2m1's largest value 6 lies in [4, 8)); the 8 codes go out as one dword,
// value i in bits 4i .. 4i + 3.
__device__ __forceinline__ void mx4_store8(const uint32_t (&w)[4], uint8_t *q4, uint8_t *scale, bool first) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  const uint32_t amax = quad_max(__float_as_uint(m));
  const int e = amax == 0 ? 0 : max((int)(amax >> 23) - 129, -127);  // bf16 maxima: e <= 125
  const float inv = __uint_as_float((uint32_t)(127 - e) << 23);      // 2^-e
  // v_cvt_scalef32_pk_fp4_f32 rounds each pair (scale 1: the values are
  // already divided by X, exactly) to the nearest e2m1, ties to even, sign
  // kept, the first value in the low nibble of byte i; the clamp to +-6
  // gives the saturation
  float s8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) s8[i] = __builtin_amdgcn_fmed3f(v[i] * inv, -6.f, 6.f);
  uint32_t c = 0;
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, s8[0], s8[1], 1.f, 0);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, s8[2], s8[3], 1.f, 1);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, s8[4], s8[5], 1.f, 2);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, s8[6], s8[7], 1.f, 3);
  *(uint32_t *)q4 = c;
  if (first) *scale = (uint8_t)(e + 127);
}

// (row, chunk) of unit u with `per` chunks per row; 32-bit division whenever
// the unit count allows (a 64-bit divide is a long instruction sequence)
__device__ __forceinline__ void split_unit(int64_t u, int64_t per, bool wide, int64_t &row, int64_t &c) {
  if (wide) {
    row = u / per;
  } else {
    row = (int64_t)((uint32_t)u / (uint32_t)per);
  }
  c = u - row * per;
}

// 8 consecutive values of a bf16 or fp32 row as fp32
__device__ __forceinline__ void load8_f32(const void *row, int64_t c8, bool f32, float (&v)[8]) {
  if (f32) {
    const u32x4 a = *((const u32x4 *)row + 2 * c8), b = *((const u32x4 *)row + 2 * c8 + 1);
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(w[i]);
  } else {
    const u32x4 a = *((const u32x4 *)row + c8);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
      v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
  }
}

}  // namespace

// bf16 rows [rows][ldx] -> e2m1 rows [rows][ldq elements, two per byte] +
// e8m0 [rows][k / 32]; units as in quantize_mxfp8_kernel.
__global__ __launch_bounds__(256) void quantize_mxfp4_kernel(const uint16_t *x, int64_t ldx, uint8_t *q,
                                                             int64_t ldq, uint8_t *qs, int64_t k8,
                                                             int64_t units) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const bool first = (threadIdx.x & 3) == 0;
  const bool wide = units > 0xFFFFFFFFll;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < units; u += stride) {
    int64_t row, c8;
    split_unit(u, k8, wide, row, c8);
    const u32x4 v = *(const u32x4 *)(x + row * ldx + 8 * c8);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    mx4_store8(w, q + row * (ldq >> 1) + 4 * c8, qs + row * (k8 >> 2) + (c8 >> 2), first);
  }
}

// bf16 rows [rows][ldx] -> e4m3 rows [rows][ldq] + e8m0 [rows][k / 32].
// Unit u = (row, 8-value chunk c8); u runs over rows * k / 8 (a multiple of 4,
// so a quad's units are all in range or all out of it).
__global__ __launch_bounds__(256) void quantize_mxfp8_kernel(const uint16_t *x, int64_t ldx, uint8_t *q,
                                                             int64_t ldq, uint8_t *qs, int64_t k8,
                                                             int64_t units) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const bool first = (threadIdx.x & 3) == 0;
  const bool wide = units > 0xFFFFFFFFll;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < units; u += stride) {
    int64_t row, c8;
    split_unit(u, k8, wide, row, c8);
    const u32x4 v = *(const u32x4 *)(x + row * ldx + 8 * c8);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    mx_store8(w, q + row * ldq + 8 * c8, qs + row * (k8 >> 2) + (c8 >> 2), first);
  }
}

// FP8 with fp32 scales.  The scale of a block with largest magnitude a is
// s = a / 448 (IEEE fp32 division; 1 for an all-zero block) and each element
// becomes e4m3 of the fp32 quotient v / s (IEEE division, then the
// nearest-even e4m3 of e4m3_pair, saturated at 448).
__device__ __forceinline__ float fp8_block_scale(float amax) { return amax > 0.f ? amax / 448.f : 1.f; }

__device__ __forceinline__ uint2 fp8_store8(const float (&v)[8], float s) {
  uint32_t c[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
    c[h] = e4m3_pair(v[4 * h] / s, v[4 * h + 1] / s) | (e4m3_pair(v[4 * h + 2] / s, v[4 * h + 3] / s) << 16);
  return uint2{c[0], c[1]};
}

__device__ __forceinline__ void load8_bf16(const uint16_t *p, bool ok, float (&v)[8]) {
  u32x4 a = {0u, 0u, 0u, 0u};
  if (ok) a = *(const u32x4 *)p;
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
}

// Blocks of 128 values: 16 lanes per block (8 values, one 16-byte load each),
// the block maximum combined over the 16 lanes by butterfly.  Unit u = (row,
// block b); a block past K's end holds fewer values (k % 8 == 0), the lanes
// beyond it load nothing and count as zeros.
__global__ __launch_bounds__(256) void quantize_fp8_block_kernel(const uint16_t *x, int64_t ldx, int64_t k,
                                                                 uint8_t *q, int64_t ldq, float *qs, int64_t kb,
                                                                 int64_t units) {
  const int64_t stride = (int64_t)gridDim.x * (blockDim.x / 16);
  const int sub = threadIdx.x & 15;
  const bool wide = units > 0xFFFFFFFFll;
  // every lane of a 16-lane group runs the same iterations (u is uniform in the group)
  for (int64_t u = (int64_t)blockIdx.x * (blockDim.x / 16) + threadIdx.x / 16; u < units; u += stride) {
    int64_t row, b;
    split_unit(u, kb, wide, row, b);
    const int64_t c = b * 128 + 8 * sub;
    const bool ok = c < k;
    float v[8];
    load8_bf16(x + row * ldx + c, ok, v);
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
    const float s = fp8_block_scale(m);
    if (ok) *(uint2 *)(q + row * ldq + c) = fp8_store8(v, s);
    if (sub == 0) qs[row * kb + b] = s;
  }
}

// One scale per row: a workgroup per row (grid-stride over rows), the row
// maximum reduced over the workgroup, then the row quantized in a second pass
// over its values (from L2).
__global__ __launch_bounds__(256) void quantize_fp8_row_kernel(const uint16_t *x, int64_t ldx, int64_t k,
                                                               uint8_t *q, int64_t ldq, float *qs, int64_t rows) {
  __shared__ float wave_max[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const uint16_t *xr = x + row * ldx;
    float m = 0.f;
    for (int64_t c = 8 * (int64_t)threadIdx.x; c < k; c += 8 * (int64_t)blockDim.x) {
      float v[8];
      load8_bf16(xr + c, true, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
    if (lane == 0) wave_max[wave] = m;
    __syncthreads();
    m = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
    __syncthreads();  // wave_max is rewritten for the next row
    const float s = fp8_block_scale(m);
    for (int64_t c = 8 * (int64_t)threadIdx.x; c < k; c += 8 * (int64_t)blockDim.x) {
      float v[8];
      load8_bf16(xr + c, true, v);
      *(uint2 *)(q + row * ldq + c) = fp8_store8(v, s);
    }
    if (threadIdx.x == 0) qs[row] = s;
  }
}

// h[r][j] = silu(gu[r][j]) * gu[r][inter + j] for j < inter, in fp32, rounded
// to bf16; MX: the bf16 values are then quantized to MXFP8 as above.
template <bool MX>
__global__ __launch_bounds__(256) void silu_mul_kernel(const void *gu, bool gu_f32, int64_t ldgu, int64_t inter,
                                                       void *h, int64_t ldh, uint8_t *hs, int64_t i8,
                                                       int64_t units) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const bool first = (threadIdx.x & 3) == 0;
  const int esz = gu_f32 ? 4 : 2;
  const bool wide = units > 0xFFFFFFFFll;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < units; u += stride) {
    int64_t row, c8;
    split_unit(u, i8, wide, row, c8);
    const uint8_t *rp = (const uint8_t *)gu + row * ldgu * esz;
    float g[8], up[8];
    load8_f32(rp, c8, gu_f32, g);
    load8_f32(rp + inter * esz, c8, gu_f32, up);
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float h0 = g[2 * i] / (1.f + __expf(-g[2 * i])) * up[2 * i];
      const float h1 = g[2 * i + 1] / (1.f + __expf(-g[2 * i + 1])) * up[2 * i + 1];
      w[i] = f32_to_bf16_rne(h0) | (f32_to_bf16_rne(h1) << 16);
    }
    if constexpr (MX) {
      mx_store8(w, (uint8_t *)h + row * ldh + 8 * c8, hs + row * (i8 >> 2) + (c8 >> 2), first);
    } else {
      *((u32x4 *)((uint16_t *)h + row * ldh) + c8) = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
}

// out[t][c] = sum_j wts[t][j] * y[t * topk + j][c] (+ bias[c]) in fp32, j in
// order, stored as bf16 (RNE) or fp32.
__global__ __launch_bounds__(256) void moe_combine_kernel(const void *y, bool y_f32, int64_t ldy, const float *wts,
                                                          int topk, const uint16_t *bias, void *out, bool out_f32,
                                                          int64_t ldo, int64_t n8, int64_t units) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int esz = y_f32 ? 4 : 2;
  const bool wide = units > 0xFFFFFFFFll;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < units; u += stride) {
    int64_t t, c8;
    split_unit(u, n8, wide, t, c8);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < topk; ++j) {
      const float wj = wts[t * topk + j];
      float v[8];
      load8_f32((const uint8_t *)y + (t * topk + j) * ldy * esz, c8, y_f32, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(wj, v[i], acc[i]);
    }
    if (bias) {
      float b[8];
      load8_f32(bias, c8, false, b);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += b[i];
    }
    if (out_f32) {
      u32x4 *o = (u32x4 *)((float *)out + t * ldo) + 2 * c8;
      o[0] = u32x4{__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]), __float_as_uint(acc[3])};
      o[1] = u32x4{__float_as_uint(acc[4]), __float_as_uint(acc[5]), __float_as_uint(acc[6]), __float_as_uint(acc[7])};
    } else {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = f32_to_bf16_rne(acc[2 * i]) | (f32_to_bf16_rne(acc[2 * i + 1]) << 16);
      *((u32x4 *)((uint16_t *)out + t * ldo) + c8) = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
}

static unsigned stream_grid(int64_t units) {
  // one unit per lane per pass; at most 8 waves' worth of workgroups per CU
  const int64_t want = (units + 255) / 256;
  return (unsigned)std::min<int64_t>(std::max<int64_t>(want, 1), 256 * 32);
}

hipError_t launch_quantize_mxfp8(const void *x, int64_t rows, int64_t k, int64_t ldx, void *q, int64_t ldq,
                                 void *qs, hipStream_t s) {
  const int64_t units = rows * (k / 8);
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_mxfp8_kernel, dim3(stream_grid(units)), dim3(256), 0, s, (const uint16_t *)x, ldx,
                     (uint8_t *)q, ldq, (uint8_t *)qs, k / 8, units);
  return hipGetLastError();
}

hipError_t launch_quantize_mxfp4(const void *x, int64_t rows, int64_t k, int64_t ldx, void *q, int64_t ldq,
                                 void *qs, hipStream_t s) {
  const int64_t units = rows * (k / 8);
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_mxfp4_kernel, dim3(stream_grid(units)), dim3(256), 0, s, (const uint16_t *)x, ldx,
                     (uint8_t *)q, ldq, (uint8_t *)qs, k / 8, units);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8(const void *x, int64_t rows, int64_t k, int64_t ldx, int block, void *q,
                               int64_t ldq, float *qs, hipStream_t s) {
  if (rows == 0 || k == 0) return hipSuccess;
  if (block == 0) {
    const unsigned grid = (unsigned)std::min<int64_t>(rows, 256 * 8);
    hipLaunchKernelGGL(quantize_fp8_row_kernel, dim3(grid), dim3(256), 0, s, (const uint16_t *)x, ldx, k,
                       (uint8_t *)q, ldq, qs, rows);
  } else {
    const int64_t kb = (k + 127) / 128, units = rows * kb;
    const unsigned grid = (unsigned)std::min<int64_t>((units + 15) / 16, 256 * 32);
    hipLaunchKernelGGL(quantize_fp8_block_kernel, dim3(grid), dim3(256), 0, s, (const uint16_t *)x, ldx, k,
                       (uint8_t *)q, ldq, qs, kb, units);
  }
  return hipGetLastError();
}

hipError_t launch_silu_mul(const void *gu, bool gu_f32, int64_t rows, int64_t inter, int64_t ldgu, bool mx,
                           void *h, int64_t ldh, void *hs, hipStream_t s) {
  const int64_t units = rows * (inter / 8);
  if (units == 0) return hipSuccess;
  if (mx)
    hipLaunchKernelGGL(silu_mul_kernel<true>, dim3(stream_grid(units)), dim3(256), 0, s, gu, gu_f32, ldgu, inter,
                       h, ldh, (uint8_t *)hs, inter / 8, units);
  else
    hipLaunchKernelGGL(silu_mul_kernel<false>, dim3(stream_grid(units)), dim3(256), 0, s, gu, gu_f32, ldgu, inter,
                       h, ldh, (uint8_t *)hs, inter / 8, units);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const void *y, bool y_f32, int64_t ldy, const float *wts, int64_t tokens, int topk,
                              int64_t n, const void *bias, void *out, bool out_f32, int64_t ldo, hipStream_t s) {
  const int64_t units = tokens * (n / 8);
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(moe_combine_kernel, dim3(stream_grid(units)), dim3(256), 0, s, y, y_f32, ldy, wts, topk,
                     (const uint16_t *)bias, out, out_f32, ldo, n / 8, units);
  return hipGetLastError();
}

}  // namespace qg
