// Q2_K x q8_1 matrix-vector product for m = 1..8 tokens (single matrix,
// shared-input pair, expert-id batch) and its exported integer stage.
//
// The pages' kernels (moe_v41/init.rs: kquant_mmvq_q2_k_w,
// kquant_mmvq_q2_k_experts_w{2,,8}; attn_v41/decode.rs: mmvq_q2k_pair_w) are
// CUDA warp-count variants. This one is written for CDNA4 wave64:
//
// * Work unit: a "half block", the 128 weights of one super-block half
//   h (qs[32h..32h+31]). Lane -> half block is fixed; the 2*nb half blocks of
//   a row sit in a power-of-two group of lanes, so a wave covers P = 64/group
//   rows per step (P = 1 for k = 7168: 56 of 64 lanes busy).
// * Weights: each lane loads its 32 quant bytes (two 16-byte loads), its 8
//   scale bytes and the block's fp16 d/dmin straight from HBM. Lanes of a
//   step cover P consecutive whole rows, so each step streams one contiguous
//   run of bytes. A ring of DEPTH steps keeps loads in flight.
// * Activations: with one token the lane's 128 int8 quants, 4 block scales
//   and 8 half sums do not change from row to row, so they are loaded once
//   into VGPRs per wave and reused for every row it processes.
// * Arithmetic: v_dot4 on the 2-bit planes. Planes 0 and 2 are masked to
//   0..3; planes 1 and 3 are masked in place (4*q, still < 128) and the dot
//   is shifted back by 2, so each plane costs one AND. Per q8 block:
//   I = sc_lo*D_lo + sc_hi*D_hi, M = m_lo*S_lo + m_hi*S_hi (exact int32),
//   then y += d8 * (d*I - dmin*M) with exact fp64 terms, reduced across the
//   row's lanes by a fixed xor butterfly in fp64 and rounded once to f32
//   (bitwise independent of grid and DEPTH).
// * Grid: waves take contiguous runs of row steps; workgroup w runs on XCD
//   w % 8, so runs are numbered XCD-major and each XCD streams one
//   contiguous eighth of the rows through its own L2.
#include <stdlib.h>

#include <mutex>

#include "q2k_device.h"
#include "q2k_launch.h"

namespace q2k {

struct MmvqParams {
  const uint8_t* w[kMaxPlainJobs];   // plain: job matrices; expert mode: the bases
  float* y[kMaxPlainJobs];
  int32_t n[kMaxPlainJobs];
  int32_t wave_end[kMaxPlainJobs];   // plain mode: exclusive prefix of waves per job
  const uint8_t* xq;
  const int32_t* ids;                // expert mode when non-null
  int32_t n_ids;
  int32_t n_experts;
  int32_t x_per_id;
  int64_t expert_stride;
  int32_t* err_flag;
  int32_t* dots;
  int32_t waves_per_job;             // expert mode
  int32_t total_waves;
  int32_t chunk;                     // row steps per wave
  int32_t k;
  int32_t gs_log2;                   // lanes per row group = 1 << gs_log2
};

// The matrix one wave works on, and its run of row steps.
struct WaveJob {
  const uint8_t* w;    // row 0 of the matrix
  float* y;            // [m, n] output of the matrix
  const uint8_t* xq;   // q8_1 rows read by the matrix
  int n;
  int it;              // first row step
  int it_end;          // end of the run
  bool bad;            // expert id out of range
};

template <int M>
__device__ __forceinline__ WaveJob resolve_wave(const MmvqParams& p, int wave, int P) {
  WaveJob J;
  int lw;
  if (p.ids == nullptr) {
    const int j = (wave >= p.wave_end[0]) + (wave >= p.wave_end[1]) + (wave >= p.wave_end[2]);
    lw = wave - (j > 0 ? p.wave_end[j - 1] : 0);
    J.w = p.w[j];
    J.y = p.y[j];
    J.n = p.n[j];
    J.xq = p.xq;
    J.bad = false;
  } else {
    const int j = wave / p.waves_per_job;
    lw = wave - j * p.waves_per_job;
    const int base = j / p.n_ids;
    const int i = j - base * p.n_ids;
    const int id = p.ids[i];
    J.bad = id < 0 || id >= p.n_experts;
    J.w = p.w[base] + (int64_t)(J.bad ? 0 : id) * p.expert_stride;
    J.n = p.n[0];
    J.y = p.y[0] + (int64_t)j * M * p.n[0];
    J.xq = p.x_per_id ? p.xq + (int64_t)i * M * (int64_t)q8_row_bytes(p.k) : p.xq;
  }
  const int iters = (J.n + P - 1) / P;
  J.it = lw * p.chunk;
  J.it_end = min(J.it + p.chunk, iters);
  return J;
}

// One lane's weights: quant bytes qs[32h..32h+31], scale bytes
// scales[8h..8h+7] and the block's (d, dmin) pair.
struct WHalf {
  u32x4 q0, q1;
  u32x2 sc;
  uint32_t dd;
};

__device__ __forceinline__ WHalf load_whalf(const uint8_t* blk, int h) {
  WHalf r;
  r.q0 = gload<u32x4_a4>(blk + 16 + 32 * h);
  r.q1 = gload<u32x4_a4>(blk + 32 + 32 * h);
  r.sc = gload<u32x2_a4>(blk + 8 * h);
  r.dd = gload<uint32_t>(blk + 80);
  return r;
}

__device__ __forceinline__ WHalf zero_whalf() {
  WHalf r;
  r.q0 = u32x4{0, 0, 0, 0};
  r.q1 = u32x4{0, 0, 0, 0};
  r.sc = u32x2{0, 0};
  r.dd = 0;
  return r;
}

// One lane's activations for one token: x[2j+s] = quants of elements
// 128h + 32j + 16s .. +15 of the super-block; d8[j] = scale of q8 block
// 8b+4h+j; s holds the 8 int16 half sums of those four q8 blocks.
struct AHalf {
  u32x4 x[8];
  f32x4 d8;
  u32x4 s;
};

__device__ __forceinline__ AHalf load_ahalf(const uint8_t* row, int k, int b, int h) {
  AHalf a;
  const uint8_t* xb = row + 256 * b + 128 * h;
#pragma unroll
  for (int i = 0; i < 8; ++i) a.x[i] = gload<u32x4>(xb + 16 * i);
  a.d8 = gload<f32x4>(row + q8_scale_offset(k) + (size_t)(8 * b + 4 * h) * 4);
  a.s = gload<u32x4>(row + q8_sum_offset(k) + (size_t)(16 * b + 8 * h) * 2);
  return a;
}

__device__ __forceinline__ AHalf zero_ahalf() {
  AHalf a;
#pragma unroll
  for (int i = 0; i < 8; ++i) a.x[i] = u32x4{0, 0, 0, 0};
  a.d8 = f32x4{0.f, 0.f, 0.f, 0.f};
  a.s = u32x4{0, 0, 0, 0};
  return a;
}

// Exact integer sums of the lane's four q8 blocks c = 8b + 4h + j:
// I[j] = sum sc*q*xq, Mv[j] = sum m*xq.
__device__ __forceinline__ void half_block_dots(const WHalf& w, const AHalf& a, int I[4],
                                                int Mv[4]) {
  const uint32_t q[8] = {w.q0[0], w.q0[1], w.q0[2], w.q0[3], w.q1[0], w.q1[1], w.q1[2], w.q1[3]};
  int D[4][2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    int d0 = 0, d1 = 0, d2 = 0, d3 = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t v = q[4 * s + i];
      const uint32_t v4 = v >> 4;
      d0 = sdot4(v & 0x03030303u, a.x[0 + s][i], d0);
      d1 = sdot4(v & 0x0C0C0C0Cu, a.x[2 + s][i], d1);
      d2 = sdot4(v4 & 0x03030303u, a.x[4 + s][i], d2);
      d3 = sdot4(v4 & 0x0C0C0C0Cu, a.x[6 + s][i], d3);
    }
    D[0][s] = d0;
    D[1][s] = d1 >> 2;   // exact: every term is a multiple of 4
    D[2][s] = d2;
    D[3][s] = d3 >> 2;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t scw = (j < 2) ? w.sc[0] : w.sc[1];
    const int sh = (j & 1) * 16;
    const uint32_t b0 = (scw >> sh) & 0xffu;
    const uint32_t b1 = (scw >> (sh + 8)) & 0xffu;
    // Every factor fits in 24 signed bits (|D| <= 16*3*127, |S| <= 16*127),
    // so the full-rate 24-bit multiplies are exact.
    I[j] = __mul24((int)(b0 & 15u), D[j][0]) + __mul24((int)(b1 & 15u), D[j][1]);
    const int s0 = (int)(int16_t)(a.s[j] & 0xffffu);
    const int s1 = (int)(int16_t)(a.s[j] >> 16);
    Mv[j] = __mul24((int)(b0 >> 4), s0) + __mul24((int)(b1 >> 4), s1);
  }
}

// The lane's contribution d * sum_j d8_j I_j - dmin * sum_j d8_j M_j, in
// fp64: d8 (f32) times I (< 2^18) and then times d (fp16) stay within 53
// bits, so every term is exact and only the sums round (fp64 rounding of
// terms whose f32 sum would cancel badly: post-SwiGLU activations reach
// 10^3 while outputs cross zero).
__device__ __forceinline__ double half_block_value(const WHalf& w, const AHalf& a) {
  int I[4], Mv[4];
  half_block_dots(w, a, I, Mv);
  double fI = 0.0, fM = 0.0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const double d8 = (double)a.d8[j];
    fI = fma(d8, (double)I[j], fI);
    fM = fma(d8, (double)Mv[j], fM);
  }
  const double d = (double)fp16_bits_to_f32(w.dd & 0xffffu);
  const double dmin = (double)fp16_bits_to_f32(w.dd >> 16);
  return d * fI - dmin * fM;
}

__device__ __forceinline__ double group_sum(double v, int gs) {
  for (int off = gs >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ void store_dots(int32_t* dots, const WHalf& w, const AHalf& a, int t,
                                           int n, int row, int k, int b, int h) {
  int I[4], Mv[4];
  half_block_dots(w, a, I, Mv);
  int32_t* o = dots + (((int64_t)t * n + row) * (k / 32) + 8 * b + 4 * h) * 2;
  *reinterpret_cast<u32x4*>(o) = u32x4{(uint32_t)I[0], (uint32_t)Mv[0], (uint32_t)I[1], (uint32_t)Mv[1]};
  *reinterpret_cast<u32x4*>(o + 4) = u32x4{(uint32_t)I[2], (uint32_t)Mv[2], (uint32_t)I[3], (uint32_t)Mv[3]};
}

// Narrow rows (2 * k/256 <= 64 half blocks): one half block per lane.
template <int M, bool CACHE, int DEPTH, bool DOTS>
__global__ __launch_bounds__(256) void mmvq_narrow_kernel(const MmvqParams p) {
  const int lane = threadIdx.x & 63;
  const int g8 = gridDim.x >> 3;
  const int wg = blockIdx.x;
  const int wave = (((wg & 7) * g8) + (wg >> 3)) * 4 + (threadIdx.x >> 6);
  if (wave >= p.total_waves) return;

  const int k = p.k;
  const int nb = k >> 8;
  const int gs = 1 << p.gs_log2;
  const int P = 64 >> p.gs_log2;
  const int prow = lane >> p.gs_log2;
  const int hb = lane & (gs - 1);
  const bool hb_ok = hb < 2 * nb;
  const int b = hb >> 1;
  const int h = hb & 1;
  const size_t rowbytes = (size_t)nb * kBlockBytes;
  const size_t rb = q8_row_bytes(k);

  const WaveJob J = resolve_wave<M>(p, wave, P);
  if (J.it >= J.it_end) return;
  const uint8_t* wlane = J.w + b * kBlockBytes;

  WHalf ws[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    const int row = (J.it + d) * P + prow;
    ws[d] = (J.it + d < J.it_end && hb_ok && row < J.n) ? load_whalf(wlane + row * rowbytes, h)
                                                        : zero_whalf();
  }
  AHalf act;
  if constexpr (CACHE) act = hb_ok ? load_ahalf(J.xq, k, b, h) : zero_ahalf();

  for (int base = J.it; base < J.it_end; base += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int cur = base + d;
      if (cur < J.it_end) {
        const WHalf w = ws[d];
        const int nxt = cur + DEPTH;
        const int nrow = nxt * P + prow;
        ws[d] = (nxt < J.it_end && hb_ok && nrow < J.n) ? load_whalf(wlane + nrow * rowbytes, h)
                                                        : zero_whalf();
        const int row = cur * P + prow;
        const bool live = hb_ok && row < J.n;
#pragma unroll
        for (int t = 0; t < M; ++t) {
          AHalf a;
          if constexpr (CACHE) {
            a = act;
          } else {
            a = hb_ok ? load_ahalf(J.xq + t * rb, k, b, h) : zero_ahalf();
          }
          if constexpr (DOTS) {
            if (live) store_dots(p.dots, w, a, t, J.n, row, k, b, h);
          } else {
            double part = live ? half_block_value(w, a) : 0.0;
            part = group_sum(part, gs);
            if (hb == 0 && row < J.n)
              J.y[(int64_t)t * J.n + row] = J.bad ? quiet_nan() : (float)part;
          }
        }
      }
    }
  }
  if (J.bad && lane == 0 && p.err_flag != nullptr) *p.err_flag = 1;
}

// Wide rows (more than 64 half blocks, k > 8192): one row per step, each
// lane walks half blocks lane, lane + 64, ...; activations come from memory.
template <int M, bool DOTS>
__global__ __launch_bounds__(256) void mmvq_wide_kernel(const MmvqParams p) {
  const int lane = threadIdx.x & 63;
  const int g8 = gridDim.x >> 3;
  const int wg = blockIdx.x;
  const int wave = (((wg & 7) * g8) + (wg >> 3)) * 4 + (threadIdx.x >> 6);
  if (wave >= p.total_waves) return;
  const int k = p.k;
  const int nb = k >> 8;
  const size_t rowbytes = (size_t)nb * kBlockBytes;
  const size_t rb = q8_row_bytes(k);
  const WaveJob J = resolve_wave<M>(p, wave, 1);
  for (int row = J.it; row < J.it_end; ++row) {
    double part[M];
#pragma unroll
    for (int t = 0; t < M; ++t) part[t] = 0.0;
    for (int hb = lane; hb < 2 * nb; hb += 64) {
      const int b = hb >> 1, h = hb & 1;
      const WHalf w = load_whalf(J.w + row * rowbytes + b * kBlockBytes, h);
#pragma unroll
      for (int t = 0; t < M; ++t) {
        const AHalf a = load_ahalf(J.xq + t * rb, k, b, h);
        if constexpr (DOTS) {
          store_dots(p.dots, w, a, t, J.n, row, k, b, h);
        } else {
          part[t] += half_block_value(w, a);
        }
      }
    }
    if constexpr (!DOTS) {
#pragma unroll
      for (int t = 0; t < M; ++t) {
        const double v = group_sum(part[t], 64);
        if (lane == 0) J.y[(int64_t)t * J.n + row] = J.bad ? quiet_nan() : (float)v;
      }
    }
  }
  if (J.bad && lane == 0 && p.err_flag != nullptr) *p.err_flag = 1;
}

namespace {

struct Tuning {
  int waves_per_cu = 16;
  int depth = 2;
};

const Tuning& tuning() {
  static Tuning t;
  static std::once_flag once;
  std::call_once(once, [] {
    if (const char* s = getenv("Q2K_MMVQ_WAVES_PER_CU")) {
      const int v = atoi(s);
      if (v >= 1 && v <= 64) t.waves_per_cu = v;
    }
    if (const char* s = getenv("Q2K_MMVQ_DEPTH")) {
      const int v = atoi(s);
      if (v == 1 || v == 2 || v == 4) t.depth = v;
    }
  });
  return t;
}

int cu_count() {
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
void dispatch_narrow(const MmvqParams& p, dim3 grid, bool dots, int depth, hipStream_t s) {
  if (dots) {
    hipLaunchKernelGGL((mmvq_narrow_kernel<M, false, 1, true>), grid, dim3(256), 0, s, p);
  } else if (M == 1) {
    if (depth == 1)
      hipLaunchKernelGGL((mmvq_narrow_kernel<M, true, 1, false>), grid, dim3(256), 0, s, p);
    else if (depth == 4)
      hipLaunchKernelGGL((mmvq_narrow_kernel<M, true, 4, false>), grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((mmvq_narrow_kernel<M, true, 2, false>), grid, dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL((mmvq_narrow_kernel<M, false, 2, false>), grid, dim3(256), 0, s, p);
  }
}

template <int M>
void dispatch_wide(const MmvqParams& p, dim3 grid, bool dots, hipStream_t s) {
  if (dots)
    hipLaunchKernelGGL((mmvq_wide_kernel<M, true>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((mmvq_wide_kernel<M, false>), grid, dim3(256), 0, s, p);
}

}  // namespace

hipError_t launch_mmvq(const MmvqLaunch& a, hipStream_t stream) {
  MmvqParams p{};
  const int nb = a.k / kBlockWeights;
  const int lanes = 2 * nb;
  const bool wide = lanes > 64;
  int gs_log2 = 0;
  if (wide) {
    gs_log2 = 6;
  } else {
    while ((1 << gs_log2) < lanes) ++gs_log2;
  }
  const int P = wide ? 1 : 64 >> gs_log2;

  for (int j = 0; j < kMaxPlainJobs; ++j) {
    p.w[j] = static_cast<const uint8_t*>(a.w[j]);
    p.y[j] = a.y[j];
    p.n[j] = a.n[j];
  }
  p.xq = static_cast<const uint8_t*>(a.xq);
  p.ids = a.ids;
  p.n_ids = a.n_ids;
  p.n_experts = a.n_experts;
  p.x_per_id = a.x_per_id;
  p.expert_stride = a.expert_stride;
  p.err_flag = a.err_flag;
  p.dots = a.dots;
  p.k = a.k;
  p.gs_log2 = gs_log2;

  // Row steps per job, then a run length that spreads them over about
  // waves_per_cu waves per CU, then whole runs per job (no run straddles
  // two matrices, so each wave resolves its matrix once).
  const int n_jobs = a.ids == nullptr ? a.njobs : a.njobs * a.n_ids;
  int64_t total_iters = 0;
  int64_t iters_of[kMaxPlainJobs] = {0, 0, 0, 0};
  if (a.ids == nullptr) {
    for (int j = 0; j < a.njobs; ++j) {
      iters_of[j] = (a.n[j] + P - 1) / P;
      total_iters += iters_of[j];
    }
  } else {
    iters_of[0] = (a.n[0] + P - 1) / P;
    total_iters = iters_of[0] * n_jobs;
  }
  if (total_iters == 0) return hipSuccess;
  const Tuning& tu = tuning();
  const int64_t target_waves = (int64_t)cu_count() * tu.waves_per_cu;
  const int64_t chunk = (total_iters + target_waves - 1) / target_waves;
  p.chunk = (int)chunk;
  int64_t total_waves = 0;
  if (a.ids == nullptr) {
    for (int j = 0; j < kMaxPlainJobs; ++j) {
      total_waves += j < a.njobs ? (iters_of[j] + chunk - 1) / chunk : 0;
      p.wave_end[j] = (int)total_waves;
    }
  } else {
    p.waves_per_job = (int)((iters_of[0] + chunk - 1) / chunk);
    total_waves = (int64_t)p.waves_per_job * n_jobs;
  }
  p.total_waves = (int)total_waves;
  int64_t groups = (total_waves + 3) / 4;
  groups = (groups + 7) / 8 * 8;
  const dim3 grid((unsigned)groups);
  const bool dots = a.dots != nullptr;

  if (wide) {
    switch (a.m) {
      case 1: dispatch_wide<1>(p, grid, dots, stream); break;
      case 2: dispatch_wide<2>(p, grid, dots, stream); break;
      case 3: dispatch_wide<3>(p, grid, dots, stream); break;
      case 4: dispatch_wide<4>(p, grid, dots, stream); break;
      case 5: dispatch_wide<5>(p, grid, dots, stream); break;
      case 6: dispatch_wide<6>(p, grid, dots, stream); break;
      case 7: dispatch_wide<7>(p, grid, dots, stream); break;
      default: dispatch_wide<8>(p, grid, dots, stream); break;
    }
  } else {
    switch (a.m) {
      case 1: dispatch_narrow<1>(p, grid, dots, tu.depth, stream); break;
      case 2: dispatch_narrow<2>(p, grid, dots, tu.depth, stream); break;
      case 3: dispatch_narrow<3>(p, grid, dots, tu.depth, stream); break;
      case 4: dispatch_narrow<4>(p, grid, dots, tu.depth, stream); break;
      case 5: dispatch_narrow<5>(p, grid, dots, tu.depth, stream); break;
      case 6: dispatch_narrow<6>(p, grid, dots, tu.depth, stream); break;
      case 7: dispatch_narrow<7>(p, grid, dots, tu.depth, stream); break;
      default: dispatch_narrow<8>(p, grid, dots, tu.depth, stream); break;
    }
  }
  return hipGetLastError();
}

}  // namespace q2k
