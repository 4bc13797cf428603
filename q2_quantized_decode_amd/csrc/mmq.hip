// Q2_K x q8_1 product for more than 8 tokens (prefill, batched verify) on the
// CDNA4 matrix cores: the route the pages take past 8 tokens (moe_v41/init.rs,
// MoeV41::new: the metrale_q2_k_mmq128_{nc,wc} kernels, whose source the pages
// do not show).
//
// * Tile: a workgroup of four waves takes 64 weight rows (16 per wave) and
//   16*G tokens, and walks the rows' super-blocks in order. Per super-block a
//   wave unpacks its 16 rows' weights once into matrix-core operands and uses
//   them for all G groups of 16 tokens.
// * Integer sums: q8 block c = 8b + 4h + p of the row (super-block b, half h,
//   plane p) is one v_mfma_i32_16x16x32_i8 per sum: the weights are the A
//   operand (row i; lane (g, i) holds K = 8g..8g+7 of the block, i.e. qs
//   bytes 32h + 8g .. +7 at bits 2p..2p+1, all in sub-block 8h + 2p + (g>>1)),
//   the activations the B operand (K x 16 tokens). A = sc*q (one 32-bit
//   multiply per four quants) gives I, A = m gives M: every output is
//   exactly one I (or M) of one (row, token, block).
// * Epilogue: lane (g, j) holds rows 4g..4g+3 of token j. The leaf of (row,
//   token, b, h) is formed as in every product kernel of the library (fI, fM
//   chained over the four planes, then RN(d*fI) - RN(dmin*fM), half_value);
//   the leaves are added in row order, (b, h) = (0, 0), (0, 1), (1, 0), ...,
//   to one running fp64 sum, and y = f32(T): the order this product fixes
//   (one register pair per output, where the pairwise tree of the
//   one-to-eight-token kernels would need a stack of partial sums per output).
// * Activations: each super-block's quants and fp64 d8 of the tile's tokens
//   are staged in LDS, double-buffered; the loads of block b + 1 (weights and
//   activations) are issued before block b is computed and consumed after
//   it, so no load is in flight across the loop's back edge.
#include <stdint.h>

#include "q2k_device.h"
#include "q2k_launch.h"

namespace q2k {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));

constexpr int kMmqWaves = 4;
constexpr int kMmqThreads = kMmqWaves * kWave;
constexpr int kMmqRows = 16 * kMmqWaves;   // weight rows per workgroup

// LDS of one staged super-block for T tokens:
//   quants [8 blocks][4 K-slices] slices of [T tokens][8 bytes], each slice
//          padded by 8 bytes: the B operand of one (block, token group) is
//          four runs of 128 consecutive bytes in lane order, and the 16
//          lanes that store one token's 16-byte chunks write 16 different
//          slices, which the padding puts on different banks (unpadded they
//          all hit the same two banks)
//   d8     [pair: blocks 4h + {0, 1} or {2, 3}][half h][T tokens] of 16
//          bytes (two fp64): the 16 lanes of a read take 16 consecutive
//          16-byte entries
template <int T>
struct MmqLds {
  static constexpr uint32_t kSlice = (uint32_t)T * 8u + 8u;
  static constexpr uint32_t kQuant = 8u * 4u * kSlice;
  static constexpr uint32_t kBuf = kQuant + (uint32_t)T * 64u;
  static constexpr uint32_t kBytes = 2u * kBuf;
};

// One lane's weight fields of one super-block: qs[32h + 8g .. +7] for both
// halves, the 16 scale bytes, d and dmin.
struct MmqW {
  u32x2 q[2];
  u32x4 sc;
  uint32_t dd;
};

__device__ __forceinline__ MmqW mmq_load_w(const uint8_t* blk, uint32_t qoff) {
  MmqW r;
  r.q[0] = gload<u32x2_a4>(blk + qoff);
  r.q[1] = gload<u32x2_a4>(blk + qoff + 32u);
  r.sc = gload<u32x4_a4>(blk);
  r.dd = gload<uint32_t>(blk + 80);
  return r;
}

// A operands of the lane's row for the 8 q8 blocks of a super-block:
// ai = sc*q (8 int8); mb = m in all 4 bytes (the M operand is mb twice).
// Four 2-bit quants q in the bytes of a word times sc <= 15 is sc*q in every
// byte (each product <= 45 stays inside its byte), one 32-bit multiply.
struct MmqA {
  int64_t ai[2][4];
  uint32_t mb[2][4];
};

__device__ __forceinline__ MmqA mmq_unpack(const MmqW& w, uint32_t soff) {
  MmqA a;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      // sub-block 8h + 2p + (g>>1): scale byte 8h + (g>>1) + 2p
      const uint32_t scw = w.sc[2 * h + (p >> 1)];
      const uint32_t off = soff + 16u * (p & 1);
      const uint32_t sc = __builtin_amdgcn_ubfe(scw, off, 4);
      const uint32_t mv = __builtin_amdgcn_ubfe(scw, off + 4u, 4);
      const uint32_t s0 = (w.q[h][0] >> (2 * p)) & 0x03030303u;
      const uint32_t s1 = (w.q[h][1] >> (2 * p)) & 0x03030303u;
      const uint32_t lo = s0 * sc;
      const uint32_t hi = s1 * sc;
      a.ai[h][p] = (int64_t)(((uint64_t)hi << 32) | lo);
      a.mb[h][p] = mv * 0x01010101u;
    }
  }
  return a;
}

// Staging of one super-block's activations: thread loads (issued before the
// block ahead of it is computed) and LDS stores (after it).
template <int T>
struct MmqStage {
  static constexpr int QC = T * 16 / kMmqThreads;   // 16-byte quant chunks per thread
  u32x4 q[QC];
  f32x4 d8;
};

template <int T>
__device__ __forceinline__ MmqStage<T> mmq_stage_load(const uint8_t* xq, int64_t rowb, int k, int t0,
                                                      int m, int b) {
  MmqStage<T> s;
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < MmqStage<T>::QC; ++it) {
    const int c = tid + it * kMmqThreads;   // chunk: token c / 16, bytes 16 * (c % 16)
    const int t = min(t0 + c / 16, m - 1);  // past the last token: the last token's row
    s.q[it] = gload<u32x4>(xq + (int64_t)t * rowb + 256 * b + 16 * (c % 16));
  }
  // d8: thread (token tid / 2, blocks 4 (tid & 1) .. +3)
  const int t = min(t0 + (tid >> 1), m - 1);
  s.d8 = gload<f32x4>(xq + (int64_t)t * rowb + k + 4 * (8 * b + 4 * (tid & 1)));
  return s;
}

// Token slots past m hold the last token's activations (the loads clamp
// the token): every output depends on its own token's column only, and the
// outputs of those slots are never stored, so nothing needs zeroing.
template <int T>
__device__ __forceinline__ void mmq_stage_store(uint8_t* buf, const MmqStage<T>& s) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < MmqStage<T>::QC; ++it) {
    const int c = tid + it * kMmqThreads;
    const int tl = c / 16, e = c % 16;       // 16 bytes = K-slices 2(e&1), +1 of block e/2
    const u32x4 v = s.q[it];
    const uint32_t blk = (uint32_t)(e >> 1), g0 = 2u * (uint32_t)(e & 1);
    *reinterpret_cast<u32x2*>(buf + (blk * 4u + g0) * MmqLds<T>::kSlice + tl * 8u) = u32x2{v[0], v[1]};
    *reinterpret_cast<u32x2*>(buf + (blk * 4u + g0 + 1u) * MmqLds<T>::kSlice + tl * 8u) = u32x2{v[2], v[3]};
  }
  if (tid < 2 * T) {
    const int tl = tid >> 1;
    const uint32_t h = (uint32_t)(tid & 1);   // the thread's blocks 4h .. 4h + 3
    uint8_t* dq = buf + MmqLds<T>::kQuant + (h * T + (uint32_t)tl) * 16u;
    *reinterpret_cast<f64x2*>(dq) = f64x2{(double)s.d8[0], (double)s.d8[1]};
    *reinterpret_cast<f64x2*>(dq + 2u * T * 16u) = f64x2{(double)s.d8[2], (double)s.d8[3]};
  }
}

__device__ __forceinline__ void mmq_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// d and dmin of rows 4g .. 4g + 3 (the lane's output rows) from the lanes
// that loaded them (lane i holds row i's).
__device__ __forceinline__ void mmq_row_scales(uint32_t dd, int g, double d[4], double dmin[4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t v = (uint32_t)__builtin_amdgcn_ds_bpermute((4 * g + r) * 4, (int)dd);
    d[r] = (double)fp16_bits_to_f32(v & 0xffffu);
    dmin[r] = (double)fp16_bits_to_f32(v >> 16);
  }
}

}  // namespace

// G groups of 16 tokens per workgroup; see the file comment. With DOTS the
// kernel writes every (I, M) of its outputs to dots instead of y.
// Registers allow four, three and two workgroups per CU at G = 1, 2, 4.
template <int G>
constexpr int mmq_wgs_per_cu() { return G == 1 ? 4 : G == 2 ? 3 : 2; }

template <int G, bool DOTS>
__global__ __launch_bounds__(kMmqThreads, mmq_wgs_per_cu<G>()) void mmq_kernel(const uint8_t* w, const uint8_t* xq,
                                                             float* y, int32_t* dots, int32_t n,
                                                             int32_t k, int32_t m, int32_t tok_tiles,
                                                             int32_t total_wgs, int32_t g8) {
  constexpr int T = 16 * G;
  using L = MmqLds<T>;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int wgi = (blockIdx.x & 7) * g8 + (blockIdx.x >> 3);   // XCD-major workgroup index
  if (wgi >= total_wgs) return;                                 // whole workgroup
  // the token tiles of one row tile are consecutive workgroups (one XCD,
  // the rows' weights through its L2)
  const int row_tile = wgi / tok_tiles;
  const int t0 = (wgi - row_tile * tok_tiles) * T;
  const int nb = k >> 8;
  const int64_t rowb = (int64_t)q8_row_bytes(k);
  const size_t wrow = (size_t)nb * kBlockBytes;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int g = lane >> 4, li = lane & 15;
  const int r0 = row_tile * kMmqRows + 16 * wv;
  // this lane's weight row (clamped: rows past n load row n - 1, never stored)
  const uint8_t* wl = w + (size_t)min(r0 + li, n - 1) * wrow;
  const uint32_t qoff = 16u + 8u * (uint32_t)g;
  const uint32_t soff = 8u * (uint32_t)(g >> 1);

  double acc[G][4];
#pragma unroll
  for (int tg = 0; tg < G; ++tg)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[tg][r] = 0.0;

  // block 0: weights and activations, staged before the loop
  MmqW wcur = mmq_load_w(wl, qoff);
  {
    const MmqStage<T> s0 = mmq_stage_load<T>(xq, rowb, k, t0, m, 0);
    mmq_stage_store<T>(lds, s0);
  }
  mmq_barrier();

  for (int b = 0; b < nb; ++b) {
    // block b's operands, then block b + 1's loads (into the same weight
    // registers; consumed after block b's work). The loads are
    // unconditional (the last block reloads itself, unused), since a load
    // under a branch would be waited for at the join.
    const MmqA a = mmq_unpack(wcur, soff);
    double d[4], dmin[4];
    mmq_row_scales(wcur.dd, g, d, dmin);
    const int bn = min(b + 1, nb - 1);
    wcur = mmq_load_w(wl + (size_t)bn * kBlockBytes, qoff);
    const MmqStage<T> snext = mmq_stage_load<T>(xq, rowb, k, t0, m, bn);
    const uint8_t* buf = lds + (uint32_t)(b & 1) * L::kBuf;
    // Each (token group, half) reads its activations at an offset that
    // passes through an empty asm together with the previous one's last
    // sum: the scheduler cannot hoist a later group's reads and matrix ops
    // above an earlier group's epilogue, so only one group's operands and
    // results are live at a time (all of them at once exceed the registers).
#pragma unroll
    for (int tg = 0; tg < G; ++tg) {
      const int tl = 16 * tg + li;                 // this lane's token within the tile
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t ofs = (uint32_t)tl * 8u;
        if constexpr (DOTS) {
          asm volatile("" : "+v"(ofs));
        } else {
          const int pt = h ? tg : tg - 1;
          if (tg + h > 0)
            asm volatile("" : "+v"(ofs) : "v"(acc[pt][0]), "v"(acc[pt][1]), "v"(acc[pt][2]), "v"(acc[pt][3]));
          else
            asm volatile("" : "+v"(ofs));
        }
        const uint8_t* d8p = buf + L::kQuant + (uint32_t)h * T * 16u + ofs * 2u;
        const f64x2 d8a = *reinterpret_cast<const f64x2*>(d8p);
        const f64x2 d8b = *reinterpret_cast<const f64x2*>(d8p + 2u * T * 16u);
        const double d8[4] = {d8a[0], d8a[1], d8b[0], d8b[1]};
        double fI[4] = {0.0, 0.0, 0.0, 0.0}, fM[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t blk = 4u * h + p;
          const int64_t bx = *reinterpret_cast<const int64_t*>(buf + (blk * 4u + (uint32_t)g) * L::kSlice + ofs);
          const v4i ci = __builtin_amdgcn_mfma_i32_16x16x32_i8(a.ai[h][p], bx, v4i{0, 0, 0, 0}, 0, 0, 0);
          const int64_t am = (int64_t)(((uint64_t)a.mb[h][p] << 32) | a.mb[h][p]);
          const v4i cm = __builtin_amdgcn_mfma_i32_16x16x32_i8(am, bx, v4i{0, 0, 0, 0}, 0, 0, 0);
          if constexpr (DOTS) {
            const int t = t0 + tl;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int row = r0 + 4 * g + r;
              if (t < m && row < n)
                *reinterpret_cast<u32x2*>(dots + (((int64_t)t * n + row) * (k / 32) + 8 * b + blk) * 2) =
                    u32x2{(uint32_t)ci[r], (uint32_t)cm[r]};
            }
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              fI[r] = fma(d8[p], (double)ci[r], fI[r]);
              fM[r] = fma(d8[p], (double)cm[r], fM[r]);
            }
          }
        }
        if constexpr (!DOTS) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[tg][r] = acc[tg][r] + half_value(d[r], dmin[r], fI[r], fM[r]);
        }
      }
    }
    mmq_stage_store<T>(lds + (uint32_t)((b + 1) & 1) * L::kBuf, snext);
    mmq_barrier();
  }

  if constexpr (!DOTS) {
#pragma unroll
    for (int tg = 0; tg < G; ++tg) {
      const int t = t0 + 16 * tg + li;
      if (t < m) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = r0 + 4 * g + r;
          if (row < n) y[(int64_t)t * n + row] = (float)acc[tg][r];
        }
      }
    }
  }
}

namespace {

template <int G, bool DOTS>
hipError_t launch_mmq_g(const uint8_t* w, const uint8_t* xq, float* y, int32_t* dots, int n, int k,
                        int m, hipStream_t stream) {
  constexpr int T = 16 * G;
  const int row_tiles = (n + kMmqRows - 1) / kMmqRows;
  const int tok_tiles = (m + T - 1) / T;
  const int64_t total = (int64_t)row_tiles * tok_tiles;
  const int g8 = (int)((total + 7) / 8);
  hipLaunchKernelGGL((mmq_kernel<G, DOTS>), dim3((unsigned)(8 * g8)), dim3(kMmqThreads),
                     MmqLds<T>::kBytes, stream, w, xq, y, dots, n, k, m, tok_tiles, (int32_t)total, g8);
  return hipGetLastError();
}

}  // namespace

// Products of 17 or more tokens, or their integer stage when dots != null
// (then y is unused). Arguments are validated by the ABI layer.
hipError_t launch_mmq(const void* w, const void* xq, float* y, int32_t* dots, int n, int k, int m,
                      hipStream_t stream) {
  const uint8_t* wb = static_cast<const uint8_t*>(w);
  const uint8_t* xb = static_cast<const uint8_t*>(xq);
  // 32 tokens per workgroup (64 take more registers than three workgroups
  // per CU leave, and measured slower at two)
  if (dots != nullptr) return launch_mmq_g<2, true>(wb, xb, y, dots, n, k, m, stream);
  return launch_mmq_g<2, false>(wb, xb, y, dots, n, k, m, stream);
}

}  // namespace q2k
