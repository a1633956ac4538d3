// Large-M tiled kernel for MXFP4 weights x MXFP8 activations on gfx950.
//
// The announcement's "W8A8 / W4A8 / W4A4" section describes the W4A8-MXFP4
// path as MXFP4 weights dequantized at load time and multiplied on FP8 tensor
// cores.  On CDNA4 the matrix core takes e2m1 and e4m3 operands with their
// e8m0 block scales directly (v_mfma_scale_f32_16x16x128_f8f6f4), so nothing is
// dequantized: the kernel only moves bytes.
//
// Tiling: a workgroup computes a 256 x BN tile of Y with 2 x (BN / 64) waves,
// each wave 128 x 64 (8 x 4 MFMA blocks of 16 x 16, 128 fp32 accumulators per
// lane).  K advances 128 per step through double-buffered LDS:
//   A  256 rows x 128 e4m3 bytes, row pitch 144 B (the 16 B pad spreads the
//      rows of one MFMA fragment read over all LDS banks);
//   B  BN / 16 packed weight blocks of 1 KB copied verbatim (the packed layout
//      already stores each lane's 16-byte B operand contiguously, so lane l
//      reads bytes [16 l, 16 l + 16) of a block: conflict-free);
//   SA the activations' four e8m0 scales of each row for this K step.
// Weight scales (one byte per lane per 16-column block and K step) are read
// from global memory a dword (four K steps) at a time.
//
// Work order: workgroups are dealt round-robin to the 8 XCDs; the tile index
// is remapped so each XCD owns a contiguous range of a grouped (GM m-tiles at
// a time) raster, so the tiles running together on one XCD share activation
// rows and weight columns in that XCD's L2.
#include <hip/hip_runtime.h>

#include "qg_internal.h"

namespace qg {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(8))) int32_t i32x8;

constexpr int kTBM = 256;        // tile rows
constexpr int kAPitch = 144;     // LDS bytes per A row
constexpr int kXcds = 8;
constexpr int kGroupM = 4;

template <int BN>
struct MxTile {
  static constexpr int WAVES_N = BN / 64;
  static constexpr int WAVES = 2 * WAVES_N;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int NBLK = BN / 16;                  // packed weight blocks per K step
  static constexpr int A_BYTES = kTBM * kAPitch;         // 36864
  static constexpr int B_BYTES = NBLK * 1024;
  static constexpr int SA_BYTES = kTBM * 4;
  static constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES;
  static constexpr int A_CHUNKS = kTBM * 8;              // 16-byte chunks of the A tile
  static constexpr int A_PER_T = A_CHUNKS / THREADS;
  static constexpr int B_PER_T = NBLK * 64 / THREADS;
};

__device__ __forceinline__ void tile_of(int pid, int m_tiles, int n_tiles, int *tm, int *tn) {
  const int total = m_tiles * n_tiles;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int t = (pid % kXcds) * per_xcd + pid / kXcds;  // contiguous range per XCD
  const int group = kGroupM * n_tiles;
  const int first_m = (t / group) * kGroupM;
  const int gm = min(kGroupM, m_tiles - first_m);
  const int r = t % group;
  *tm = first_m + r % gm;
  *tn = r / gm;
}

template <int BN>
__global__ __launch_bounds__(MxTile<BN>::THREADS) void mx_tiled_kernel(GemmArgs a) {
  using C = MxTile<BN>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int q = lane >> 4, r16 = lane & 15;

  const int m_tiles = (a.m + kTBM - 1) / kTBM;
  const int bn_tiles = (a.n_tiles * 16 + BN - 1) / BN;
  const int total = m_tiles * bn_tiles;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  if ((int)(blockIdx.x % kXcds) * per_xcd + (int)(blockIdx.x / kXcds) >= total) return;
  int tm, tn;
  tile_of(blockIdx.x, m_tiles, bn_tiles, &tm, &tn);
  const int m0 = tm * kTBM;
  const int nt0 = tn * C::NBLK;  // first 16-column n-tile
  const int kbs = a.k_blocks;
  const int kq = a.k >> 5;       // activation scale bytes per row

  const uint8_t *x = (const uint8_t *)a.x;
  // --- global -> register staging of one K step ---
  u32x4 sa_[C::A_PER_T];
  u32x4 sb_[C::B_PER_T];
  uint32_t ss_ = 0;
  auto load_stage = [&](int kb) {
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
      const int c = tid + i * C::THREADS;
      const int row = min(m0 + (c >> 3), a.m - 1);
      sa_[i] = *(const u32x4 *)(x + (int64_t)row * a.ldx + kb * 128 + 16 * (c & 7));
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) {
      const int c = tid + i * C::THREADS;
      const int nt = min(nt0 + (c >> 6), a.n_tiles - 1);
      sb_[i] = *(const u32x4 *)(a.wbase + ((uint64_t)nt * kbs + kb) * 1024 + 16 * (c & 63));
    }
    if (tid < kTBM) {
      const int row = min(m0 + tid, a.m - 1);
      ss_ = *(const uint32_t *)(a.x_scales + (int64_t)row * kq + 4 * kb);
    }
  };
  auto store_stage = [&](int buf) {
    uint8_t *s = smem + buf * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
      const int c = tid + i * C::THREADS;
      *(u32x4 *)(s + (c >> 3) * kAPitch + 16 * (c & 7)) = sa_[i];
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) {
      const int c = tid + i * C::THREADS;
      *(u32x4 *)(s + C::A_BYTES + 16 * c) = sb_[i];
    }
    if (tid < kTBM) *(uint32_t *)(s + C::A_BYTES + C::B_BYTES + 4 * tid) = ss_;
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // weight scales: lane (column n, quarter q) reads the dword holding K steps
  // kb & ~3 .. +3 of its column
  const uint8_t *wsc = a.wbase + a.scales_offset;
  int ncol[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    ncol[j] = min(nt0 + wn * 4 + j, a.n_tiles - 1) * 16 + r16;

  load_stage(0);
  store_stage(0);
  __syncthreads();
  uint32_t wsw[4] = {0u, 0u, 0u, 0u};
  for (int kb = 0; kb < kbs; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < kbs) load_stage(kb + 1);
    if ((kb & 3) == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        wsw[j] = *(const uint32_t *)(wsc + ((uint64_t)ncol[j] * 4 + q) * a.kb_pad + kb);
    }
    const uint8_t *s = smem + buf * C::STAGE;
    // B fragments and scales of the wave's four 16-column blocks
    i32x8 bf[4];
    int bsc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 v = *(const u32x4 *)(s + C::A_BYTES + (wn * 4 + j) * 1024 + 16 * lane);
      bf[j] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      bsc[j] = (int)((wsw[j] >> (8 * (kb & 3))) & 0xFFu);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = wm * 128 + i * 16 + r16;
      const uint8_t *ap = s + row * kAPitch;
      const u32x4 lo = *(const u32x4 *)(ap + 16 * q);
      const u32x4 hi = *(const u32x4 *)(ap + 64 + 16 * q);
      const i32x8 af = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                        (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      const int asc = s[C::A_BYTES + C::B_BYTES + 4 * row + q];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], acc[i][j], 0, 4, 0,
                                                                      asc, 0, bsc[j]);
    }
    if (kb + 1 < kbs) store_stage(buf ^ 1);
    __syncthreads();
  }

  // output: block (i, j) lane holds rows 4q..4q+3 of column r16
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = (nt0 + wn * 4 + j) * 16 + r16;
      if (col >= a.n) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + wm * 128 + i * 16 + 4 * q + e;
        if (row >= a.m) continue;
        if (a.otype == QG_O_F32)
          ((float *)a.y)[(int64_t)row * a.ldy + col] = acc[i][j][e];
        else
          ((__bf16 *)a.y)[(int64_t)row * a.ldy + col] = (__bf16)acc[i][j][e];
      }
    }
}

template <int BN>
static hipError_t launch_mx_tiled_bn(const GemmArgs &a, hipStream_t s) {
  using C = MxTile<BN>;
  const int m_tiles = (a.m + kTBM - 1) / kTBM;
  const int bn_tiles = (a.n_tiles * 16 + BN - 1) / BN;
  const int total = m_tiles * bn_tiles;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int grid = per_xcd * kXcds;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void *)mx_tiled_kernel<BN>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 2 * C::STAGE);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(mx_tiled_kernel<BN>, dim3(grid), dim3(C::THREADS), 2 * C::STAGE, s, a);
  return hipGetLastError();
}

hipError_t launch_mx_tiled(const GemmArgs &a, int bn, hipStream_t s) {
  if (a.k % 128 != 0) return hipErrorInvalidValue;
  return bn == 256 ? launch_mx_tiled_bn<256>(a, s) : launch_mx_tiled_bn<128>(a, s);
}

}  // namespace qg
