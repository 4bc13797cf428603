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
// steps; otherwise they are read per half block and plane. One token and at
// most 32 half blocks per row (k <= 4096, the engram projection's 2048
// among them): a quarter of a half block per lane, its 64 activations kept
// as f64, so each weight costs one f64 fma instead of an f32 product, a
// widening and an f64 add.
//
// Per weight the arithmetic is the table lookup (a selector and a v_perm
// per two weights, then the split of the pair), the widening of the weight
// to f64 and one f64 fma: about 6 VALU instructions, at one wave64
// instruction per 4 clocks per SIMD about 6.4 us for the 41.9 M weights of
// a [20480, 2048] matrix on 256 CUs at 2.4 GHz. The kernel is bound by that
// arithmetic, not by its 13.8 MB of weights (1.7 us at 8 TB/s).
//
// Each wave keeps the weights of its next row steps in flight while it
// computes the current one: one step ahead in the general kernel, two in
// the one-token quarter kernel (a ring of three steps; one step ahead left
// its waves waiting on the weights: 10.9 against 9.6 us on the engram
// projection [20480, 2048]).
#include <stdlib.h>

#include "q2k_device.h"
#include "q2k_launch.h"

namespace q2k {

namespace {

// Kernel arguments (scalars, preloaded into SGPRs at wave launch):
//   w        Q2_K rows [n, k/256] x 84 bytes
//   x        bf16 [m, k], row stride x_stride elements
//   y        f32 [m, n]
//   gs_log2  lanes per row = 1 << gs_log2

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// The four bf16 values one sub-block's 2-bit quants can take, T[q] =
// bf16_rne(d*sc*q - dmin*m) for q = 0..3 (the same f32 fma and rounding as
// the per-weight expansion), packed two per dword: lo = T0 | T1 << 16,
// hi = T2 | T3 << 16.
struct Table {
  uint32_t lo, hi;
};

__device__ __forceinline__ Table sub_block_table(float dsc, float dmm) {
  // v_cvt_pk_bf16_f32 rounds two f32 values to bf16, nearest-even (the
  // values here are never f32 subnormals: both products are multiples of
  // 2^-24); element 0 lands in the low half
  const f32x2_t t01 = {fmaf(dsc, 0.0f, -dmm), fmaf(dsc, 1.0f, -dmm)};
  const f32x2_t t23 = {fmaf(dsc, 2.0f, -dmm), fmaf(dsc, 3.0f, -dmm)};
  return Table{__builtin_bit_cast(uint32_t, __builtin_convertvector(t01, bf16x2_t)),
               __builtin_bit_cast(uint32_t, __builtin_convertvector(t23, bf16x2_t))};
}

// Lookup selectors of the four weights whose quants are bytes 0..3 of
// word >> 2j (bits 0..1 of each byte): selector bytes (2q, 2q + 1) pick
// T[q] out of the packed table. s01 serves weights 0 and 1, s23 weights 2
// and 3.
__device__ __forceinline__ void lookup_selectors(uint32_t word, int j, uint32_t& s01, uint32_t& s23) {
  const uint32_t q2 = (j == 0 ? word << 1 : word >> (2 * j - 1)) & 0x06060606u;   // 2q per byte
  const uint32_t q2p = q2 | 0x01010101u;                                            // 2q + 1
  s01 = __builtin_amdgcn_perm(q2p, q2, 0x05010400u);
  s23 = __builtin_amdgcn_perm(q2p, q2, 0x07030602u);
}

// f32 values (bf16 in the high half) of the two weights a selector serves.
__device__ __forceinline__ void lookup_pair(const Table& T, uint32_t sel, float& wa, float& wb) {
  const uint32_t pair = __builtin_amdgcn_perm(T.hi, T.lo, sel);   // T[qa] | T[qb] << 16
  wa = __uint_as_float(pair << 16);
  wb = __uint_as_float(pair & 0xffff0000u);
}

// One plane j (elements 32j .. 32j+31) of a half block: the 32 quants come
// from qs bytes 0..31 of the half (q0 = bytes 0..15, q1 = 16..31), bits 2j;
// elements l < 16 use sub-block table T0, the rest T1. xw holds the plane's
// 32 bf16 activations as 16 dwords (element 2i in the low half). Every
// product of two bf16 values is exact in f32 and is summed in fp64.
__device__ __forceinline__ void plane_dot(const u32x4& q0, const u32x4& q1, const Table& T0,
                                          const Table& T1, int j, const uint32_t xw[16], double acc[4]) {
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t sel[2];
    lookup_selectors(w < 4 ? q0[w] : q1[w - 4], j, sel[0], sel[1]);
    const Table& T = w < 4 ? T0 : T1;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float wa, wb;
      lookup_pair(T, sel[i], wa, wb);
      const uint32_t xb = xw[2 * w + i];
      const float xa = __uint_as_float(xb << 16);
      const float xbv = __uint_as_float(xb & 0xffff0000u);
      acc[2 * i] += (double)(wa * xa);
      acc[2 * i + 1] += (double)(wb * xbv);
    }
  }
}

// The same with the plane's activations already widened to f32 (xf[l] is
// element l of the plane).
__device__ __forceinline__ void plane_dot_f(const u32x4& q0, const u32x4& q1, const Table& T0,
                                            const Table& T1, int j, const float xf[32], double acc[4]) {
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t sel[2];
    lookup_selectors(w < 4 ? q0[w] : q1[w - 4], j, sel[0], sel[1]);
    const Table& T = w < 4 ? T0 : T1;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float wa, wb;
      lookup_pair(T, sel[i], wa, wb);
      acc[2 * i] += (double)(wa * xf[4 * w + 2 * i]);
      acc[2 * i + 1] += (double)(wb * xf[4 * w + 2 * i + 1]);
    }
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
__global__ __launch_bounds__(256) void gemv_bf16_kernel(const uint8_t* w, const uint16_t* x, float* y,
                                                        int64_t x_stride, int32_t n, int32_t k,
                                                        int32_t gs_log2, int32_t total_waves) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  if (wave >= total_waves) return;
  const int nb = k >> 8;
  const int gs = 1 << gs_log2;
  const int P = 64 >> gs_log2;
  const int prow = lane >> gs_log2;
  const int hb0 = lane & (gs - 1);
  const size_t rowbytes = (size_t)nb * kBlockBytes;
  const int steps = (n + P - 1) / P;

  // CACHE_X: the lane's 128 activations as f32, widened once
  float xc[CACHE_X ? 4 : 1][CACHE_X ? 32 : 1];
  if constexpr (CACHE_X) {
    const int hb = hb0 < 2 * nb ? hb0 : 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t xw[16];
      load_plane_x(x, 128 * hb + 32 * j, xw);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        xc[j][2 * i] = __uint_as_float(xw[i] << 16);
        xc[j][2 * i + 1] = __uint_as_float(xw[i] & 0xffff0000u);
      }
    }
  }

  // The weights of the wave's next row step are requested before the
  // current one is computed (a ring of two).
  struct HalfW {
    u32x4 q0, q1;
    u32x2 sc;
    uint32_t dd;
  };
  auto load_half = [&](int st, int hb) {
    HalfW r;
    const int row = min(st * P + prow, n - 1);
    const int b = hb >> 1, h = hb & 1;
    const uint8_t* blk = w + (size_t)row * rowbytes + (size_t)b * kBlockBytes;
    r.q0 = gload<u32x4_a4>(blk + 16 + 32 * h);
    r.q1 = gload<u32x4_a4>(blk + 32 + 32 * h);
    r.sc = gload<u32x2_a4>(blk + 8 * h);
    r.dd = gload<uint32_t>(blk + 80);
    return r;
  };
  const int hbl = hb0 < 2 * nb ? hb0 : 0;   // CACHE_X: the lane's one half block
  HalfW nxt{};
  if constexpr (CACHE_X) {
    if (wave < steps) nxt = load_half(wave, hbl);
  }
  for (int st = wave; st < steps; st += total_waves) {
    const int row = st * P + prow;
    double acc[M][4];
#pragma unroll
    for (int t = 0; t < M; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t][i] = 0.0;
    HalfW cur{};
    if constexpr (CACHE_X) {
      cur = nxt;
      if (st + total_waves < steps) nxt = load_half(st + total_waves, hbl);
    }
    if (row < n) {
      for (int hb = hb0; hb < 2 * nb; hb += gs) {
        const int b = hb >> 1, h = hb & 1;
        if constexpr (!CACHE_X) cur = load_half(st, hb);
        const u32x4 q0 = cur.q0, q1 = cur.q1;
        const u32x2 sc = cur.sc;
        const uint32_t dd = cur.dd;
        const float d = fp16_bits_to_f32(dd & 0xffffu);
        const float dmin = fp16_bits_to_f32(dd >> 16);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // sub-blocks 8h + 2j and 8h + 2j + 1: scale bytes 2j, 2j + 1 of this half
          const uint32_t sw = sc[j >> 1] >> (16 * (j & 1));
          const uint32_t s0 = sw & 0xffu, s1 = (sw >> 8) & 0xffu;
          const Table T0 = sub_block_table(d * (float)(s0 & 15u), dmin * (float)(s0 >> 4));
          const Table T1 = sub_block_table(d * (float)(s1 & 15u), dmin * (float)(s1 >> 4));
          if constexpr (CACHE_X) {
            plane_dot_f(q0, q1, T0, T1, j, xc[j], acc[0]);
          } else {
#pragma unroll
            for (int t = 0; t < M; ++t) {
              uint32_t xw[16];
              load_plane_x(x + (int64_t)t * x_stride, 256 * b + 128 * h + 32 * j, xw);
              plane_dot(q0, q1, T0, T1, j, xw, acc[t]);
            }
          }
        }
        if constexpr (CACHE_X) break;       // one half block per lane
      }
    }
#pragma unroll
    for (int t = 0; t < M; ++t) {
      double v = (acc[t][0] + acc[t][1]) + (acc[t][2] + acc[t][3]);
      switch (gs_log2) {
        case 0: break;
        case 1: v = group_sum_f64<1>(v, lane); break;
        case 2: v = group_sum_f64<2>(v, lane); break;
        case 3: v = group_sum_f64<3>(v, lane); break;
        case 4: v = group_sum_f64<4>(v, lane); break;
        case 5: v = group_sum_f64<5>(v, lane); break;
        default: v = group_sum_f64<6>(v, lane); break;
      }
      if (hb0 == 0 && row < n) y[(int64_t)t * n + row] = (float)v;
    }
  }
}

// One token, rows of at most 32 half blocks (k <= 4096): lane l of a row's
// group (4 k/256 lanes, rounded up to a power of two) takes quarter l of the
// row: quant bytes 16 (l & 1) .. 16 (l & 1) + 15 of half block l >> 1, i.e.
// the first or the second 16 elements of each of the half's four planes
// (sub-blocks 8h + 2j + (l & 1), j = 0..3), 64 weights per step. Its 64
// activations stay in VGPRs as f64 for all its steps, so a weight costs one
// f64 fma, acc + w * x: the product is exact, so this rounds exactly as
// adding the exact f32 product does.
constexpr int kRing = 3;   // row steps per wave in the quarter kernel's ring

template <int GSL>
__global__ __launch_bounds__(256) void gemv_bf16_quarter_kernel(const uint8_t* w, const uint16_t* x,
                                                                float* y, int32_t n, int32_t k,
                                                                int32_t total_waves) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  if (wave >= total_waves) return;
  const int nb = k >> 8;
  constexpr int gs = 1 << GSL;
  constexpr int P = 64 >> GSL;
  const int prow = lane >> GSL;
  const int ql = lane & (gs - 1);
  const bool q_ok = ql < 4 * nb;          // lanes past the row's quarters add +0
  const int qq = q_ok ? ql : 0;
  const int hb = qq >> 1, part = qq & 1;
  const int b = hb >> 1, h = hb & 1;
  const size_t rowbytes = (size_t)nb * kBlockBytes;
  const int steps = (n + P - 1) / P;

  double xd[4][16];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint16_t* xp = x + 256 * b + 128 * h + 32 * j + 16 * part;
    const u32x4 a0 = gload<u32x4>(xp);
    const u32x4 a1 = gload<u32x4>(xp + 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t v = i < 4 ? a0[i] : a1[i - 4];
      xd[j][2 * i] = q_ok ? (double)__uint_as_float(v << 16) : 0.0;
      xd[j][2 * i + 1] = q_ok ? (double)__uint_as_float(v & 0xffff0000u) : 0.0;
    }
  }

  struct QuarterW {
    u32x4 q;
    u32x2 sc;
    uint32_t dd;
  };
  // Ring of kRing steps per wave: slot r holds the weights of step
  // st0 + r W; once that step is computed the slot is refilled with step
  // st0 + (r + kRing) W, so kRing - 1 steps stay in flight while one is
  // computed, and the refill reuses the registers it replaces. Steps past
  // the end load the last row (in bounds) and are not computed.
  auto load_quarter = [&](int st) {
    QuarterW r;
    const int row = min(min(st, steps - 1) * P + prow, n - 1);
    const uint8_t* blk = w + (size_t)row * rowbytes + (size_t)b * kBlockBytes;
    r.q = gload<u32x4_a4>(blk + 16 + 32 * h + 16 * part);
    r.sc = gload<u32x2_a4>(blk + 8 * h);
    r.dd = gload<uint32_t>(blk + 80);
    return r;
  };
  QuarterW ring[kRing];
#pragma unroll
  for (int r = 0; r < kRing; ++r) ring[r] = load_quarter(wave + r * total_waves);
  for (int st0 = wave; st0 < steps; st0 += kRing * total_waves) {
#pragma unroll
    for (int r = 0; r < kRing; ++r) {
      const int st = st0 + r * total_waves;
      if (st < steps) {   // wave-uniform
        const int row = st * P + prow;
        const QuarterW& cur = ring[r];
        double acc[4] = {0.0, 0.0, 0.0, 0.0};
        const float d = fp16_bits_to_f32(cur.dd & 0xffffu);
        const float dmin = fp16_bits_to_f32(cur.dd >> 16);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // sub-block 8h + 2j + part: scale byte 2j + part of this half
          const uint32_t sv = (cur.sc[j >> 1] >> (16 * (j & 1) + 8 * part)) & 0xffu;
          const Table T = sub_block_table(d * (float)(sv & 15u), dmin * (float)(sv >> 4));
#pragma unroll
          for (int wi = 0; wi < 4; ++wi) {
            uint32_t sel[2];
            lookup_selectors(cur.q[wi], j, sel[0], sel[1]);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              float wa, wb;
              lookup_pair(T, sel[i], wa, wb);
              acc[2 * i] = fma((double)wa, xd[j][4 * wi + 2 * i], acc[2 * i]);
              acc[2 * i + 1] = fma((double)wb, xd[j][4 * wi + 2 * i + 1], acc[2 * i + 1]);
            }
          }
        }
        const double v = group_sum_f64<GSL>((acc[0] + acc[1]) + (acc[2] + acc[3]), lane);
        if (ql == 0 && row < n) y[row] = (float)v;
      }
      ring[r] = load_quarter(st + kRing * total_waves);
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

struct GemvArgs {
  const uint8_t* w;
  const uint16_t* x;
  float* y;
  int64_t x_stride;
  int32_t n, k, gs_log2, total_waves;
};

template <int M>
void launch_m(const GemvArgs& a, dim3 grid, bool cache_x, hipStream_t s) {
  if (M == 1 && cache_x)
    hipLaunchKernelGGL((gemv_bf16_kernel<1, true>), grid, dim3(256), 0, s, a.w, a.x, a.y, a.x_stride,
                       a.n, a.k, a.gs_log2, a.total_waves);
  else
    hipLaunchKernelGGL((gemv_bf16_kernel<M, false>), grid, dim3(256), 0, s, a.w, a.x, a.y, a.x_stride,
                       a.n, a.k, a.gs_log2, a.total_waves);
}

}  // namespace

hipError_t launch_gemv_bf16(const void* w, const void* x, int64_t x_stride, float* y, int n, int k,
                            int m, hipStream_t stream) {
  GemvArgs p{};
  p.w = static_cast<const uint8_t*>(w);
  p.x = static_cast<const uint16_t*>(x);
  p.x_stride = x_stride;
  p.y = y;
  p.n = n;
  p.k = k;
  const int half_blocks = 2 * (k / kBlockWeights);
  if (m == 1 && half_blocks <= 32) {
    // one token, k <= 4096: a quarter of a half block per lane
    int gsl = 0;
    while ((1 << gsl) < 2 * half_blocks) ++gsl;
    const int P = 64 >> gsl;
    const int64_t steps = ((int64_t)n + P - 1) / P;
    const int64_t waves = steps < (int64_t)cu_count_gemv() * 8 ? steps : (int64_t)cu_count_gemv() * 8;
    const dim3 grid((unsigned)((waves + 3) / 4));
#define Q2K_GEMV_Q(G) \
  hipLaunchKernelGGL(gemv_bf16_quarter_kernel<G>, grid, dim3(256), 0, stream, p.w, p.x, y, n, k, (int32_t)waves)
    switch (gsl) {
      case 2: Q2K_GEMV_Q(2); break;
      case 3: Q2K_GEMV_Q(3); break;
      case 4: Q2K_GEMV_Q(4); break;
      case 5: Q2K_GEMV_Q(5); break;
      default: Q2K_GEMV_Q(6); break;
    }
#undef Q2K_GEMV_Q
    return hipGetLastError();
  }
  int gsl = 0;
  while ((1 << gsl) < half_blocks && gsl < 6) ++gsl;
  p.gs_log2 = gsl;
  const int P = 64 >> gsl;
  const int64_t steps = ((int64_t)n + P - 1) / P;
  // About 8 waves per CU, each taking every W-th step (with the next
  // step's weights in flight).
  const int64_t waves = steps < (int64_t)cu_count_gemv() * 8 ? steps : (int64_t)cu_count_gemv() * 8;
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
