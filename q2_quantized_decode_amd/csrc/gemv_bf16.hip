// Q2_K weights x bf16 activations, f32 out: the single-token engram
// projection read straight off the raw Q2_K blocks (engram_v41/apply.rs, the
// engram_v41_wkv_q2k_gemv launch; engram_v41.rs, EngramLayerWeights::wkv_q2k,
// whose doc states that it agrees bit for bit with a bf16 GEMV over the bf16
// expansion of the same blocks).
//
// Every weight is expanded exactly as the row dequantisation expands it:
// v = d*sc*q - dmin*m in f32 (both products are exact, one rounding in the
// subtraction), then bf16 to nearest-even. The product of two bf16 values is
// exact in f32; the products are summed in fp64 and the sum is rounded once
// to f32. The output is the correctly rounded f32 of the exact dot product
// of the expansion with x (up to the fp64 rounding of partial sums, about
// 2^-53 of the sum), whatever order the sums take.
//
// Layout: lane l works on half block hb = l % group (+ group, + 2 group, ...
// for rows of more than 64 half blocks) of row l / group; P = 64 / group rows
// per wave step; wave w takes steps w, w + W, ... With one token and at most
// 64 half blocks per row, a lane's 128 activations stay in VGPRs for all its
// steps; otherwise they are read per half block and plane.
#include <stdlib.h>

#include "q2k_device.h"
#include "q2k_launch.h"

namespace q2k {

namespace {

struct GemvParams {
  const uint8_t* w;
  const uint16_t* x;     // bf16 [m, k], row stride x_stride elements
  int64_t x_stride;
  float* y;              // f32 [m, n]
  int32_t n, k;
  int32_t gs_log2;       // lanes per row = 1 << gs_log2
  int32_t total_waves;
};

// bf16 round-to-nearest-even of a finite f32, returned as the f32 it represents.
__device__ __forceinline__ float bf16_rne_f32(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7fffu + ((u >> 16) & 1u);
  return __uint_as_float(u & 0xffff0000u);
}

// One plane j (elements 32j .. 32j+31) of a half block: the 32 quants come
// from qs bytes 0..31 of the half (q0 = bytes 0..15, q1 = 16..31), bits 2j;
// elements l < 16 use sub-block scale byte s0, the rest s1. xw holds the
// plane's 32 bf16 activations as 16 dwords (element 2i in the low half).
__device__ __forceinline__ void plane_dot(const u32x4& q0, const u32x4& q1, uint32_t s0, uint32_t s1,
                                          float d, float dmin, int j, const uint32_t xw[16],
                                          double acc[4]) {
  const float dsc0 = d * (float)(s0 & 15u), dmm0 = dmin * (float)(s0 >> 4);
  const float dsc1 = d * (float)(s1 & 15u), dmm1 = dmin * (float)(s1 >> 4);
#pragma unroll
  for (int l = 0; l < 32; ++l) {
    const uint32_t word = l < 16 ? q0[l >> 2] : q1[(l - 16) >> 2];
    const uint32_t q = (word >> (8 * (l & 3) + 2 * j)) & 3u;
    const float wv = bf16_rne_f32(fmaf(l < 16 ? dsc0 : dsc1, (float)q, l < 16 ? -dmm0 : -dmm1));
    const uint32_t xb = xw[l >> 1];
    const float xv = __uint_as_float((l & 1) ? (xb & 0xffff0000u) : (xb << 16));
    acc[l & 3] += (double)(wv * xv);
  }
}

__device__ __forceinline__ void load_plane_x(const uint16_t* xrow, int e0, uint32_t xw[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 v = gload<u32x4>(xrow + e0 + 8 * i);
    xw[4 * i] = v[0];
    xw[4 * i + 1] = v[1];
    xw[4 * i + 2] = v[2];
    xw[4 * i + 3] = v[3];
  }
}

// M tokens; CACHE_X: one token and one half block per lane, activations kept
// in VGPRs across steps.
template <int M, bool CACHE_X>
__global__ __launch_bounds__(256) void gemv_bf16_kernel(const GemvParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  if (wave >= p.total_waves) return;
  const int nb = p.k >> 8;
  const int gs = 1 << p.gs_log2;
  const int P = 64 >> p.gs_log2;
  const int prow = lane >> p.gs_log2;
  const int hb0 = lane & (gs - 1);
  const size_t rowbytes = (size_t)nb * kBlockBytes;
  const int steps = (p.n + P - 1) / P;

  uint32_t xc[CACHE_X ? 4 : 1][CACHE_X ? 16 : 1];
  if constexpr (CACHE_X) {
    const int hb = hb0 < 2 * nb ? hb0 : 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) load_plane_x(p.x, 128 * hb + 32 * j, xc[j]);
  }

  for (int st = wave; st < steps; st += p.total_waves) {
    const int row = st * P + prow;
    double acc[M][4];
#pragma unroll
    for (int t = 0; t < M; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t][i] = 0.0;
    if (row < p.n) {
      for (int hb = hb0; hb < 2 * nb; hb += gs) {
        const int b = hb >> 1, h = hb & 1;
        const uint8_t* blk = p.w + (size_t)row * rowbytes + (size_t)b * kBlockBytes;
        const u32x4 q0 = gload<u32x4_a4>(blk + 16 + 32 * h);
        const u32x4 q1 = gload<u32x4_a4>(blk + 32 + 32 * h);
        const u32x2 sc = gload<u32x2_a4>(blk + 8 * h);
        const uint32_t dd = gload<uint32_t>(blk + 80);
        const float d = fp16_bits_to_f32(dd & 0xffffu);
        const float dmin = fp16_bits_to_f32(dd >> 16);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // sub-blocks 8h + 2j and 8h + 2j + 1: scale bytes 2j, 2j + 1 of this half
          const uint32_t sw = sc[j >> 1] >> (16 * (j & 1));
          const uint32_t s0 = sw & 0xffu, s1 = (sw >> 8) & 0xffu;
          if constexpr (CACHE_X) {
            plane_dot(q0, q1, s0, s1, d, dmin, j, xc[j], acc[0]);
          } else {
#pragma unroll
            for (int t = 0; t < M; ++t) {
              uint32_t xw[16];
              load_plane_x(p.x + (int64_t)t * p.x_stride, 256 * b + 128 * h + 32 * j, xw);
              plane_dot(q0, q1, s0, s1, d, dmin, j, xw, acc[t]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < M; ++t) {
      double v = (acc[t][0] + acc[t][1]) + (acc[t][2] + acc[t][3]);
      for (int off = gs >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off);
      if (hb0 == 0 && row < p.n) p.y[(int64_t)t * p.n + row] = (float)v;
    }
  }
}

int cu_count_gemv() {
  static int counts[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (counts[dev] == 0) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
      c = 256;
    counts[dev] = c;
  }
  return counts[dev];
}

template <int M>
void launch_m(const GemvParams& p, dim3 grid, bool cache_x, hipStream_t s) {
  if (M == 1 && cache_x)
    hipLaunchKernelGGL((gemv_bf16_kernel<1, true>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((gemv_bf16_kernel<M, false>), grid, dim3(256), 0, s, p);
}

}  // namespace

hipError_t launch_gemv_bf16(const void* w, const void* x, int64_t x_stride, float* y, int n, int k,
                            int m, hipStream_t stream) {
  GemvParams p{};
  p.w = static_cast<const uint8_t*>(w);
  p.x = static_cast<const uint16_t*>(x);
  p.x_stride = x_stride;
  p.y = y;
  p.n = n;
  p.k = k;
  const int half_blocks = 2 * (k / kBlockWeights);
  int gsl = 0;
  while ((1 << gsl) < half_blocks && gsl < 6) ++gsl;
  p.gs_log2 = gsl;
  const int P = 64 >> gsl;
  const int64_t steps = ((int64_t)n + P - 1) / P;
  // About 16 waves per CU, each taking every W-th step.
  const int64_t waves = steps < (int64_t)cu_count_gemv() * 16 ? steps : (int64_t)cu_count_gemv() * 16;
  p.total_waves = (int)waves;
  const dim3 grid((unsigned)((waves + 3) / 4));
  const bool cache_x = half_blocks <= 64;
  switch (m) {
    case 1: launch_m<1>(p, grid, cache_x, stream); break;
    case 2: launch_m<2>(p, grid, cache_x, stream); break;
    case 3: launch_m<3>(p, grid, cache_x, stream); break;
    case 4: launch_m<4>(p, grid, cache_x, stream); break;
    case 5: launch_m<5>(p, grid, cache_x, stream); break;
    case 6: launch_m<6>(p, grid, cache_x, stream); break;
    case 7: launch_m<7>(p, grid, cache_x, stream); break;
    default: launch_m<8>(p, grid, cache_x, stream); break;
  }
  return hipGetLastError();
}

}  // namespace q2k
