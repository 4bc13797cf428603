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
#include <atomic>

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
  int32_t n_ids;                     // expert mode: ids; grouped mode: groups
  int32_t n_experts;
  int32_t x_per_id;
  int64_t expert_stride;
  int32_t* err_flag;
  int32_t* dots;
  int32_t groups;                    // grouped mode when > 0
  int32_t waves_per_job;             // expert and grouped modes
  int32_t total_waves;
  int32_t chunk;                     // row steps per wave
  int32_t interleave;                // 1: a job's waves take its steps round-robin
  int32_t k;
  int32_t gs_log2;                   // lanes per row group = 1 << gs_log2
  int32_t g8;                        // workgroups per XCD (grid / 8)
  int32_t tsplit;                    // tokens taken by separate waves (1: none)
  const float* sg;                   // SwiGLU prologue: gate rows [n_ids, k]
  const float* su;                   // and up rows
  const uint8_t* xb16;               // narrow kernel with FQ: the token's bf16 row
  uint8_t* xq_out;                   // narrow kernel with FQ: receives its q8_1 row
  EngramRows eg;                     // run kernel with FQ = 3: the engram rows of the input
  uint8_t* sw_hq;                    // run kernel with FQ = 4: q8_1 rows of the SwiGLU
  uint16_t* sw_h;                    // and (nullable) its bf16 rows, [n_ids, n]
  int32_t pair_blocks;               // FQ = 4: 64-row blocks per matrix
  int64_t x_row_bytes;               // FQ = 5: row stride of the bf16 input, bytes
};

// Touches every field of the argument block at once, so that its scalar
// loads are issued together and waited for once at the top of the kernel;
// left to the compiler, the loads of each field go out where it is first
// needed, and every dependent round costs a memory latency before the first
// weight load. Later reads of the same fields hit the scalar cache.
__device__ __forceinline__ void prefetch_args(const MmvqParams& p) {
  asm volatile("" ::"s"(p.w[0]), "s"(p.y[0]), "s"(p.n[0]), "s"(p.wave_end[0]), "s"(p.wave_end[1]),
               "s"(p.wave_end[2]), "s"(p.xq), "s"(p.ids), "s"(p.groups), "s"(p.total_waves),
               "s"(p.k), "s"(p.interleave), "s"(p.chunk), "s"(p.g8),
               "s"(p.tsplit));
}

// The matrix one wave works on, and its run of row steps.
struct WaveJob {
  const uint8_t* w;    // row 0 of the matrix
  float* y;            // output row 0 of the matrix; token t at y + t * ldy
  XView x;             // q8_1 activations read by the matrix
  int n;
  int ldy;
  int it;              // first row step
  int it_end;          // end of the run
  int stride;          // distance between the wave's consecutive steps
  bool bad;            // expert id out of range
  int xrow;            // expert mode: position of the id in the list (its input row)
};

// M is the kernel's token count; a token-split launch (tsplit > 1) runs the
// one-token kernel, and the launch's own token count sets the layouts.
template <int M>
__device__ __forceinline__ WaveJob resolve_wave(const MmvqParams& p, int wave, int P) {
  const int mt = M == 1 ? p.tsplit : M;
  WaveJob J;
  J.xrow = 0;
  int lw;
  if (p.ids == nullptr && p.groups == 0) {
    const int j = (wave >= p.wave_end[0]) + (wave >= p.wave_end[1]) + (wave >= p.wave_end[2]);
    lw = wave - (j > 0 ? p.wave_end[j - 1] : 0);
    J.w = p.w[j];
    J.y = p.y[j];
    J.n = p.n[j];
    J.ldy = J.n;
    J.x = xview(p.xq, p.k, 0);
    J.bad = false;
  } else if (p.groups > 0) {
    const int g = wave / p.waves_per_job;
    lw = wave - g * p.waves_per_job;
    J.bad = false;
    J.w = p.w[0] + (int64_t)g * p.expert_stride;
    J.n = p.n[0];
    J.ldy = p.groups * p.n[0];
    J.y = p.y[0] + (int64_t)g * p.n[0];
    J.x = xview(p.xq, p.groups * p.k, g * p.k);
  } else {
    const int j = wave / p.waves_per_job;
    lw = wave - j * p.waves_per_job;
    const int base = j / p.n_ids;
    const int i = j - base * p.n_ids;
    const int id = p.ids[i];
    J.xrow = i;
    J.bad = id < 0 || id >= p.n_experts;
    J.w = p.w[base] + (int64_t)(J.bad ? 0 : id) * p.expert_stride;
    J.n = p.n[0];
    J.ldy = J.n;
    J.y = p.y[0] + (int64_t)j * mt * p.n[0];
    J.x = xview(p.x_per_id ? p.xq + (int64_t)i * mt * (int64_t)q8_row_bytes(p.k) : p.xq, p.k, 0);
  }
  const int iters = (J.n + P - 1) / P;
  if (p.interleave) {
    int waves_of_job;
    if (p.ids == nullptr && p.groups == 0) {
      const int j = (wave >= p.wave_end[0]) + (wave >= p.wave_end[1]) + (wave >= p.wave_end[2]);
      waves_of_job = p.wave_end[j] - (j > 0 ? p.wave_end[j - 1] : 0);
    } else {
      waves_of_job = p.waves_per_job;
    }
    J.it = lw;
    J.it_end = iters;
    J.stride = waves_of_job;
  } else {
    J.it = lw * p.chunk;
    J.it_end = min(J.it + p.chunk, iters);
    J.stride = 1;
  }
  return J;
}

// FQ = 4 (gate and up with their SwiGLU): workgroup q takes id i = q /
// pair_blocks and rows 64 * (q % pair_blocks) .. +63 of both matrices; its
// wave w runs 32 consecutive rows, 32 * (w >> 1) .. +31 of the block, of
// matrix w & 1 (0 gate, 1 up).
__device__ __forceinline__ WaveJob resolve_pair(const MmvqParams& p, int wave, int P) {
  const int q = wave >> 2, w = wave & 3;
  const int i = q / p.pair_blocks;
  const int rb = q - i * p.pair_blocks;
  const int base = w & 1;
  const int id = p.ids[i];
  WaveJob J;
  J.xrow = i;
  J.bad = id < 0 || id >= p.n_experts;
  J.w = p.w[base] + (int64_t)(J.bad ? 0 : id) * p.expert_stride;
  J.n = p.n[0];
  J.ldy = J.n;
  J.y = p.y[0] + (int64_t)(base * p.n_ids + i) * p.n[0];
  J.x = xview(p.xq, p.k, 0);
  J.it = (64 * rb + 32 * (w >> 1)) / P;
  J.it_end = min(J.it + 32 / P, (J.n + P - 1) / P);
  J.stride = 1;
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

__device__ __forceinline__ AHalf load_ahalf(const XView& x, int t, int b, int h) {
  AHalf a;
  const int64_t to = (int64_t)t * x.stride;
  const uint8_t* xb = x.q + to + 256 * b + 128 * h;
#pragma unroll
  for (int i = 0; i < 8; ++i) a.x[i] = gload<u32x4>(xb + 16 * i);
  a.d8 = gload<f32x4>(x.s + to + (size_t)(8 * b + 4 * h) * 4);
  a.s = gload<u32x4>(x.m + to + (size_t)(16 * b + 8 * h) * 2);
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

// sdot4 that starts a chain: v_dot4_i32_i8 with an inline zero accumulator
// (the accumulating v_dot4c form would need a v_mov to clear it first).
__device__ __forceinline__ int sdot4_first(uint32_t a, uint32_t b) {
  int r;
  asm volatile("v_dot4_i32_i8 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Integer sums of the lane's four q8 blocks c = 8b + 4h + j:
// I4[j] = sum sc*q*xq and Mv[j] = sum m*xq, except that I4[1] and I4[3]
// come out multiplied by 4 (planes 1 and 3 are masked in place, q*4 < 128,
// instead of being shifted down; every term is then a multiple of 4).
__device__ __forceinline__ void half_block_dots_x4(const WHalf& w, const AHalf& a, int I4[4],
                                                   int Mv[4]) {
  const uint32_t q[8] = {w.q0[0], w.q0[1], w.q0[2], w.q0[3], w.q1[0], w.q1[1], w.q1[2], w.q1[3]};
  int D[4][2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const uint32_t v0 = q[4 * s], v04 = v0 >> 4;
    int d0 = sdot4_first(v0 & 0x03030303u, a.x[0 + s][0]);
    int d1 = sdot4_first(v0 & 0x0C0C0C0Cu, a.x[2 + s][0]);
    int d2 = sdot4_first(v04 & 0x03030303u, a.x[4 + s][0]);
    int d3 = sdot4_first(v04 & 0x0C0C0C0Cu, a.x[6 + s][0]);
#pragma unroll
    for (int i = 1; i < 4; ++i) {
      const uint32_t v = q[4 * s + i];
      const uint32_t v4 = v >> 4;
      d0 = sdot4(v & 0x03030303u, a.x[0 + s][i], d0);
      d1 = sdot4(v & 0x0C0C0C0Cu, a.x[2 + s][i], d1);
      d2 = sdot4(v4 & 0x03030303u, a.x[4 + s][i], d2);
      d3 = sdot4(v4 & 0x0C0C0C0Cu, a.x[6 + s][i], d3);
    }
    D[0][s] = d0;
    D[1][s] = d1;
    D[2][s] = d2;
    D[3][s] = d3;
  }
  // Scale bytes scales[8h + 2j + s]: low nibble sc, high nibble m.
  const uint32_t scn[2] = {w.sc[0] & 0x0F0F0F0Fu, w.sc[1] & 0x0F0F0F0Fu};
  const uint32_t mn[2] = {(w.sc[0] >> 4) & 0x0F0F0F0Fu, (w.sc[1] >> 4) & 0x0F0F0F0Fu};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int sh = (j & 1) * 16;
    const int sc0 = (int)((scn[j >> 1] >> sh) & 0xffu), sc1 = (int)((scn[j >> 1] >> (sh + 8)) & 0xffu);
    const int m0 = (int)((mn[j >> 1] >> sh) & 0xffu), m1 = (int)((mn[j >> 1] >> (sh + 8)) & 0xffu);
    // Every factor fits in 24 signed bits (|D| <= 16*12*127, |S| <= 16*127),
    // so the full-rate 24-bit multiplies are exact.
    I4[j] = __mul24(sc0, D[j][0]) + __mul24(sc1, D[j][1]);
    const int s0 = (int)(int16_t)(a.s[j] & 0xffffu);
    const int s1 = (int)(int16_t)(a.s[j] >> 16);
    Mv[j] = __mul24(m0, s0) + __mul24(m1, s1);
  }
}

// Exact integer sums I[j] = sum sc*q*xq, Mv[j] = sum m*xq of the lane's four
// q8 blocks (the x4 of planes 1 and 3 shifted out: exact).
__device__ __forceinline__ void half_block_dots(const WHalf& w, const AHalf& a, int I[4],
                                                int Mv[4]) {
  half_block_dots_x4(w, a, I, Mv);
  I[1] >>= 2;
  I[3] >>= 2;
}

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
  return half_value(d, dmin, fI, fM);
}

// Sum over a group of gs lanes holding the half blocks of one row in the
// order 2b + h: lane offsets 2, 4, .., gs/2 first (the pairwise tree over
// the row's super-blocks for each half), then 1 (the two halves), the same
// tree as every other product kernel.
template <int GSL>
__device__ __forceinline__ double group_sum_t(double v, int lane) {
  if constexpr (GSL >= 2) v += dpp_f64<DppPartner<2>::ctrl>(v);
  if constexpr (GSL >= 3) v += xor4_f64(v);
  if constexpr (GSL >= 4) v += dpp_f64<DppPartner<8>::ctrl>(v);
  if constexpr (GSL >= 5) v = halve<16>(v, v, lane);
  if constexpr (GSL >= 6) v = halve<32>(v, v, lane);
  return v + dpp_f64<DppPartner<1>::ctrl>(v);
}

__device__ __forceinline__ double group_sum(double v, int gs, int lane) {
  switch (gs) {
    case 2: return group_sum_t<1>(v, lane);
    case 4: return group_sum_t<2>(v, lane);
    case 8: return group_sum_t<3>(v, lane);
    case 16: return group_sum_t<4>(v, lane);
    case 32: return group_sum_t<5>(v, lane);
    default: return group_sum_t<6>(v, lane);
  }
}

__device__ __forceinline__ void store_dots(int32_t* dots, const WHalf& w, const AHalf& a, int t,
                                           int n, int row, int k, int b, int h) {
  int I[4], Mv[4];
  half_block_dots(w, a, I, Mv);
  int32_t* o = dots + (((int64_t)t * n + row) * (k / 32) + 8 * b + 4 * h) * 2;
  *reinterpret_cast<u32x4*>(o) = u32x4{(uint32_t)I[0], (uint32_t)Mv[0], (uint32_t)I[1], (uint32_t)Mv[1]};
  *reinterpret_cast<u32x4*>(o + 4) = u32x4{(uint32_t)I[2], (uint32_t)Mv[2], (uint32_t)I[3], (uint32_t)Mv[3]};
}

// Sum eight per-lane values a[0..7] (eight row steps) over groups of
// GS = 1 << GSL lanes (GS >= 8) at once. Lanes hold half blocks in the order
// 2b + h, so the pairwise tree over the super-blocks takes the lane offsets
// 2, 4, .., GS/2 and the two halves offset 1, last. Three halving levels
// (offsets 2, 4, 8; for GS = 8: 2, 4, 1) leave lane l holding step
// reduce8_slot(l) summed over its 8 lanes; the remaining offsets finish the
// group.
template <int GSL>
__device__ __forceinline__ double reduce8(const double a[8], int lane) {
  constexpr int GS = 1 << GSL;
  constexpr int O3 = GS >= 16 ? 8 : 1;
  double b4[4], b2[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) b4[i] = halve<2>(a[2 * i], a[2 * i + 1], lane);
#pragma unroll
  for (int i = 0; i < 2; ++i) b2[i] = halve<4>(b4[2 * i], b4[2 * i + 1], lane);
  double v = halve<O3>(b2[0], b2[1], lane);
  if constexpr (GS >= 32) v = halve<16>(v, v, lane);
  if constexpr (GS >= 64) v = halve<32>(v, v, lane);
  if constexpr (GS >= 16) v += dpp_f64<DppPartner<1>::ctrl>(v);
  return v;
}

// The step (0..7) that reduce8 leaves on lane l, and whether l is the one
// lane of its row group that writes it.
template <int GSL>
__device__ __forceinline__ int reduce8_slot(int lane) {
  if constexpr (GSL >= 4) return (lane >> 1) & 7;
  return ((lane >> 1) & 3) | ((lane & 1) << 2);
}

template <int GSL>
__device__ __forceinline__ bool reduce8_writer(int lane) {
  if constexpr (GSL >= 4) return (lane & ((1 << GSL) - 1) & ~0xE) == 0;
  return true;
}

// half_block_value for the run kernel: dq holds d8_j with the x4 of planes
// 1 and 3 folded in (d8/4 is exact, so dq * I4 == d8 * I exactly).
__device__ __forceinline__ double half_block_value_m1(const WHalf& w, const AHalf& a,
                                                      const double dq[4], const double dm[4]) {
  int I4[4], Mv[4];
  half_block_dots_x4(w, a, I4, Mv);
  double fI = 0.0, fM = 0.0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    fI = fma(dq[j], (double)I4[j], fI);
    fM = fma(dm[j], (double)Mv[j], fM);
  }
  const double d = (double)fp16_bits_to_f32(w.dd & 0xffffu);
  const double dmin = (double)fp16_bits_to_f32(w.dd >> 16);
  return half_value(d, dmin, fI, fM);
}

// Weight fields of one lane at fixed 32-bit byte offsets from a uniform
// (SGPR) base, so the loads use the scalar-base + vector-offset form.
struct LaneOffsets {
  uint32_t q;    // qs[32h]
  uint32_t sc;   // scales[8h]
  uint32_t dd;   // d, dmin
};

// The empty asm makes each offset an opaque 32-bit VGPR value, so the
// compiler keeps "uniform base + 32-bit offset" instead of reassociating the
// sum into per-step 64-bit vector address arithmetic.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ LaneOffsets lane_offsets(uint32_t blk_off, int h) {
  return LaneOffsets{opaque(blk_off + 16u + 32u * (uint32_t)h), opaque(blk_off + 8u * (uint32_t)h),
                     opaque(blk_off + 80u)};
}

__device__ __forceinline__ WHalf load_whalf_at(const uint8_t* base, const LaneOffsets& o) {
  WHalf r;
  r.q0 = gload<u32x4_a4>(base + o.q);
  r.q1 = gload<u32x4_a4>(base + o.q + 16u);
  r.sc = gload<u32x2_a4>(base + o.sc);
  r.dd = gload<uint32_t>(base + o.dd);
  return r;
}

// The lane's activations from a q8_1 row held in LDS (same layout as in
// device memory: k quants, k/32 scales, k/16 half sums).
__device__ __forceinline__ AHalf load_ahalf_lds(const uint8_t* xs, int k, int b, int h) {
  AHalf a;
  const uint8_t* q = xs + 256 * b + 128 * h;
#pragma unroll
  for (int i = 0; i < 8; ++i) a.x[i] = *reinterpret_cast<const u32x4*>(q + 16 * i);
  a.d8 = *reinterpret_cast<const f32x4*>(xs + q8_scale_offset(k) + (size_t)(8 * b + 4 * h) * 4);
  a.s = *reinterpret_cast<const u32x4*>(xs + q8_sum_offset(k) + (size_t)(16 * b + 8 * h) * 2);
  return a;
}

// q8_1 of one 32-value block of bf16 (raw: its 64 bytes) into a q8_1 row
// in LDS and, when gout is non-null, into the same row in device memory.
// Same arithmetic as q8_1_rows (q8_1_scale, q8_1_quant), so the same bytes.
__device__ __forceinline__ void q8_1_block_store(uint8_t* xs, uint8_t* gout, const u32x4 raw[4],
                                                 int blk, int k, bool active) {
  float v[32];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t w = raw[i >> 2][i & 3];
    v[2 * i] = bf16_bits_to_f32(w & 0xffffu);
    v[2 * i + 1] = bf16_bits_to_f32(w >> 16);
  }
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) a = fmaxf(a, fabsf(v[i]));
  const float d = q8_1_scale(a);
  int qv[32];
  q8_1_quant_lane<32>(v, d, qv);
  uint32_t qw[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int s0 = 0, s1 = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int q = qv[i];
    if (i < 16) s0 += q; else s1 += q;
    qw[i >> 2] |= (uint32_t)(q & 0xff) << (8 * (i & 3));
  }
  if (!active) return;
  const u32x4 lo{qw[0], qw[1], qw[2], qw[3]}, hi{qw[4], qw[5], qw[6], qw[7]};
  const uint32_t sums = ((uint32_t)s0 & 0xffffu) | ((uint32_t)s1 << 16);
  const size_t so = q8_scale_offset(k) + (size_t)blk * 4, mo = q8_sum_offset(k) + (size_t)blk * 4;
  *reinterpret_cast<u32x4*>(xs + 32 * blk) = lo;
  *reinterpret_cast<u32x4*>(xs + 32 * blk + 16) = hi;
  *reinterpret_cast<float*>(xs + so) = d;
  *reinterpret_cast<uint32_t*>(xs + mo) = sums;
  if (gout != nullptr) {
    *reinterpret_cast<u32x4*>(gout + 32 * blk) = lo;
    *reinterpret_cast<u32x4*>(gout + 32 * blk + 16) = hi;
    *reinterpret_cast<float*>(gout + so) = d;
    *reinterpret_cast<uint32_t*>(gout + mo) = sums;
  }
}

// The same for one half (16 values, raw: their 32 bytes) of a 32-value
// block, the lane pair 2j, 2j + 1 holding block j (halves 0 and 1): the
// block maximum is one exchange between the pair, each lane quantises and
// sums its own 16 values. Rows of k <= 4096 (at most 256 halves) take one
// half per thread, so the prologue's quantisation is half as long.
__device__ __forceinline__ void q8_1_half_store(uint8_t* xs, uint8_t* gout, const u32x4 raw[2], int hb,
                                                int k, bool active) {
  float v[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t w = raw[i >> 2][i & 3];
    v[2 * i] = bf16_bits_to_f32(w & 0xffffu);
    v[2 * i + 1] = bf16_bits_to_f32(w >> 16);
  }
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(v[i]));
  a = fmaxf(a, __uint_as_float(dpp_u32<0xB1>(__float_as_uint(a))));
  const float d = q8_1_scale(a);
  int qv[16];
  q8_1_quant_lane<16>(v, d, qv);
  uint32_t qw[4] = {0, 0, 0, 0};
  int sum = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    sum += qv[i];
    qw[i >> 2] |= (uint32_t)(qv[i] & 0xff) << (8 * (i & 3));
  }
  if (!active) return;
  const int blk = hb >> 1, h = hb & 1;
  const u32x4 q4{qw[0], qw[1], qw[2], qw[3]};
  const size_t so = q8_scale_offset(k) + (size_t)blk * 4, mo = q8_sum_offset(k) + (size_t)blk * 4 + 2 * h;
  *reinterpret_cast<u32x4*>(xs + 32 * blk + 16 * h) = q4;
  if (h == 0) *reinterpret_cast<float*>(xs + so) = d;
  *reinterpret_cast<int16_t*>(xs + mo) = (int16_t)sum;
  if (gout != nullptr) {
    *reinterpret_cast<u32x4*>(gout + 32 * blk + 16 * h) = q4;
    if (h == 0) *reinterpret_cast<float*>(gout + so) = d;
    *reinterpret_cast<int16_t*>(gout + mo) = (int16_t)sum;
  }
}

// Workgroup barrier that orders LDS only: weight loads stay in flight.
// A wave-uniform 8-byte load through the scalar data cache, waited for
// inside the same asm statement. It counts on the scalar memory counter, so
// waiting for it does not wait for the vector loads the wave has in flight.
__device__ __forceinline__ int64_t scalar_load_i64(const int64_t* p) {
  int64_t v;
  asm volatile("s_load_dwordx2 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p));
  return v;
}

__device__ __forceinline__ void lds_barrier_m1() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One token, rows of at most 64 half blocks and at least 8 lanes per row
// (k from 1024 to 8192). Each wave owns a run of CH row steps (CH a multiple
// of 8, known at compile time), either consecutive or interleaved with the
// other runs of the matrix (stride S) so that the waves sweep the matrix
// together. A step is P whole rows (contiguous bytes); lane l works on half
// block l % GS of row l / GS. Per step:
//  * each lane loads its half block's fields (32 quant bytes, 8 scale bytes,
//    d/dmin) into a ring of R register sets, R steps ahead of the arithmetic
//    (a variant that brought each step in by coalesced 16-byte loads through
//    LDS measured slower: bank conflicts on the field reads);
//  * the activations stay in VGPRs for the whole run; the sums of eight
//    consecutive steps are reduced together (one transposed butterfly).
// A full run is straight-line code, so the hardware wait counters are exact
// and no wait drains the ring. Runs cut short by the end of the matrix take
// a guarded path with one direct load per step.
//
// The leading scalar arguments describe the whole launch when it is one
// matrix with interleaved runs (plain != 0): they are preloaded into SGPRs at
// wave launch (kernel-argument preloading, enabled for this file), so that
// case issues its first loads without reading the argument block at all.
// Otherwise the block is fetched and resolved as for the other kernels.
//
// FQ = 1 (fused quantisation, one token, one input row shared by every
// matrix of the launch: a single matrix or an expert batch with a shared
// input): xq0 is the bf16 row instead. FQ = 3 (one matrix, one token): the
// input row is a decode token's engram rows (p.eg): threads 0..cols-1 of
// each workgroup compute the token's row ids of one hashed layer with the
// hash kernels' device functions (workgroup 0 also stores the position's
// compressed id into the cache and raises the error flag), then every
// thread gathers, dequantises and quantises 8 values per pass into the LDS
// row (workgroup 0 also writes it to xq_out), as engram_rows_q8_1 does. FQ = 2 (expert batch, one input row
// per id, every workgroup inside one id's waves): the workgroup forms the
// bf16 SwiGLU of its id's gate and up rows (p.sg, p.su) and quantises it;
// the workgroup holding the id's first wave writes that q8_1 row to
// xq_out + id position * row bytes. FQ = 4 (expert batch of two bases, gate
// and up, one shared bf16 row): the FQ = 1 prologue, the rows of each
// workgroup paired as resolve_pair states, and an epilogue in which the
// workgroup forms the bf16 SwiGLU of its 64 gate and up outputs and their two
// q8_1 blocks (p.sw_hq, p.sw_h), as swiglu_q8_1_rows does. FQ = 5 (one
// matrix or several with plain jobs, m = p.tsplit tokens, bf16 rows x0 with
// stride p.x_row_bytes): workgroup q takes token q % m and that token's
// waves 4 (q / m) .. +3 (total_waves is the count per token), quantises
// that token's row into LDS as FQ = 1 does, and the token's first
// workgroup writes it to row q of xq_out.
// Each workgroup issues its bf16 loads and then its weight ring,
// quantises the row into LDS (one thread per 32-value block; workgroup 0
// also writes it to xq_out), and waits for LDS only, so the quantisation
// overlaps the weights' memory latency and no separate q8_1 launch is
// needed.
template <int GSL, int R, int CH, int FQ>
__global__ __launch_bounds__(256) void mmvq_m1_kernel(const uint8_t* w0, const uint8_t* xq0, float* y0,
                                                      int32_t n0, int32_t k0, int32_t total_waves,
                                                      int32_t g8, int32_t plain, uint8_t* xq_out,
                                                      const MmvqParams p) {
  constexpr int GS = 1 << GSL;
  constexpr int P = 64 >> GSL;
  constexpr int V = 8;
  static_assert(CH % V == 0 && R >= 2, "run and ring shapes");
  static_assert(FQ != 4 || P * CH == 32, "FQ = 4: 32 rows per wave");
  // FQ = 4: the workgroup's gate (0) and up (1) outputs, rows of its block
  __shared__ float ysw[2][64];
  const int lane = threadIdx.x & 63;
  const int wiw = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wg = blockIdx.x;
  int wave = (((wg & 7) * g8) + (wg >> 3)) * 4 + wiw;
  int tok5 = 0;
  bool xq_writer5 = false;
  if constexpr (FQ == 5) {
    const int q = wave >> 2;
    tok5 = q % p.tsplit;
    xq_writer5 = q < p.tsplit;
    wave = (q / p.tsplit) * 4 + wiw;
  }
  // with FQ every wave of the workgroup takes part in the quantisation; a
  // wave past the end resolves the last wave's job (valid addresses only)
  if (!FQ && wave >= total_waves) return;
  const bool in_grid = wave < total_waves;
  // FQ = 2: this workgroup writes its id's q8_1 row (its first wave starts the id)
  const bool row_writer = FQ == 2 && in_grid && ((wave - wiw) % p.waves_per_job) == 0;
  if (FQ && !in_grid) wave = total_waves - 1;
  // FQ = 2: the gate and up rows of this id position go out before the id
  // itself is read (the row is the id's position in the list, not the id)
  f32x4 gv[2], uv[2];
  const int k_in = k0;
  const bool sthread = FQ == 2 && (int)threadIdx.x < (k_in >> 3);   // 8 values per thread
  const int se0 = sthread ? 8 * (int)threadIdx.x : 0;
  if constexpr (FQ == 2) {
    const int srow = (wave / p.waves_per_job) % p.n_ids;
    const size_t ro = (size_t)srow * (size_t)k_in + (size_t)se0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      gv[i] = gload<f32x4>(p.sg + ro + 4 * i);
      uv[i] = gload<f32x4>(p.su + ro + 4 * i);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  WaveJob J;
  int tok = 0;
  if (plain) {
    // one matrix, runs interleaved: wave w takes steps w, w + W, ...
    J.w = w0;
    J.y = y0;
    J.x = xview(xq0, k0, 0);
    J.n = n0;
    J.ldy = n0;
    J.it = wave;
    J.it_end = (n0 + P - 1) / P;
    J.stride = total_waves;
    J.bad = false;
  } else {
    prefetch_args(p);
    if constexpr (FQ == 4) {
      J = resolve_pair(p, wave, P);
    } else if constexpr (FQ == 5) {
      J = resolve_wave<1>(p, wave, P);
      J.y += (int64_t)tok5 * J.ldy;
    } else {
      // token split: the tsplit waves of one run are consecutive (same or
      // neighbouring workgroup, same XCD), so they share the run's weights
      // through that XCD's L2
      const int ts = p.tsplit;
      if (ts > 1) {
        tok = wave % ts;
        wave /= ts;
      }
      J = resolve_wave<1>(p, wave, P);
      J.y += (int64_t)tok * J.ldy;
    }
  }
  const bool live = in_grid && J.it < J.it_end;
  if (!FQ && !live) return;

  const int k = k0;
  const int nb = k >> 8;
  // lane l of a row group takes half h = l & 1 of super-block b = (l & (GS-1))
  // >> 1 (GS/2 is the row's block count rounded up to a power of two);
  // lanes past the row's blocks read block 0 and add +0
  const int hb = lane & (GS - 1);
  const int prow = lane >> GSL;
  const int braw = hb >> 1;
  const bool hb_ok = braw < nb;
  const int b = hb_ok ? braw : 0;
  const int h = hb & 1;
  const uint32_t rowbytes = (uint32_t)nb * kBlockBytes;
  const uint32_t step_bytes = (uint32_t)P * rowbytes;
  const int slot = reduce8_slot<GSL>(lane);      // the step reduce8 leaves on this lane
  const bool writer = reduce8_writer<GSL>(lane);

  // The run's steps are J.it + st * S, st = 0..CH-1.
  const int S = J.stride;
  const size_t run_stride = (size_t)S * step_bytes;
  const uint8_t* wrun = J.w + (size_t)J.it * step_bytes;
  const int last_step = J.it + (CH - 1) * S;
  const bool full = last_step < J.it_end && (last_step + 1) * P <= J.n;

  // Each lane loads its own half block's fields.
  const LaneOffsets off = lane_offsets((uint32_t)prow * rowbytes + (uint32_t)b * kBlockBytes, h);
  WHalf ws[R];
  AHalf act;
  if constexpr (FQ != 0) {
    extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
    const int tid = threadIdx.x;
    // The input loads go out first, then the ring, so waiting for the input
    // does not wait for the weights (loads complete in issue order).
    // Unconditional loads: a wave without a full run reads row 0 and never
    // uses it.
    u32x4 raw[4];
    bool qthread = sthread;
    // k <= 4096 (GSL <= 5): one 16-value half block per thread
    constexpr bool HALVES = (FQ == 4 || FQ == 5 || FQ == 1) && GSL <= 5;
    if constexpr (FQ == 1 || FQ == 4 || FQ == 5) {
      const uint8_t* xrow = xq0;
      if constexpr (FQ == 5) xrow += (size_t)tok5 * (size_t)p.x_row_bytes;
      if constexpr (HALVES) {
        qthread = tid < (k >> 4);
        const uint8_t* xb = xrow + 32 * (qthread ? tid : 0);
#pragma unroll
        for (int i = 0; i < 2; ++i) raw[i] = gload<u32x4>(xb + 16 * i);
      } else {
        qthread = tid < (k >> 5);               // one 32-value block per thread (k <= 8192)
        const uint8_t* xb = xrow + 64 * (qthread ? tid : 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) raw[i] = gload<u32x4>(xb + 16 * i);
      }
    }
    // FQ = 3: the hash's independent loads (the token, the window's cached
    // ids, the layer's multipliers, the column's prime and offset) also go
    // out before the ring
    constexpr int NG3 = FQ == 3 ? kMaxNgram : 1;
    int32_t h_t0 = 0;
    int64_t h_cw[NG3], h_mu[NG3], h_pr = 0, h_of = 0;
    if constexpr (FQ == 3) {
      const EngramRows& E = p.eg;
      // every argument field the prologue reads, fetched in one round now
      asm volatile("" ::"s"(E.token_map), "s"(E.vocab), "s"(E.mult), "s"(E.primes), "s"(E.offsets),
                   "s"(E.layer), "s"(E.ng), "s"(E.n_heads), "s"(E.pad_id), "s"(E.cache), "s"(E.token),
                   "s"(E.pos), "s"(E.table), "s"(E.n_table_rows), "s"(E.err_flag));
      const int cols = k >> 8;
      const int c = tid < cols ? tid : 0;
      h_t0 = E.token[0];
#pragma unroll
      for (int i = 0; i < kMaxNgram; ++i) {
        const int ii = i < E.ng ? i : E.ng - 1;
        h_cw[i] = E.cache[E.pos >= ii ? E.pos - ii : 0];
        h_mu[i] = E.mult[(int64_t)E.layer * E.ng + ii];
      }
      h_pr = E.primes[(int64_t)E.layer * cols + c];
      h_of = E.offsets[(int64_t)E.layer * cols + c];
    }
    __builtin_amdgcn_sched_barrier(0);
    const bool ring_ok = live && full;
    const LaneOffsets o0 = ring_ok ? off : lane_offsets((uint32_t)b * kBlockBytes, h);
    const uint8_t* wr = ring_ok ? wrun : J.w;
    const size_t rs = ring_ok ? run_stride : 0;
#pragma unroll
    for (int r = 0; r < R; ++r) ws[r] = load_whalf_at(wr + (size_t)r * rs, o0);
    __builtin_amdgcn_sched_barrier(0);   // keep the ring ahead of the quantisation
    if constexpr (FQ == 1 || FQ == 4 || FQ == 5) {
      uint8_t* gout = nullptr;
      if constexpr (FQ == 5) {
        if (xq_writer5) gout = xq_out + (size_t)tok5 * q8_row_bytes(k);
      } else {
        if (blockIdx.x == 0) gout = xq_out;
      }
      if constexpr (HALVES) q8_1_half_store(xs, gout, raw, tid, k, qthread);
      else q8_1_block_store(xs, gout, raw, tid, k, qthread);
    } else if constexpr (FQ == 3) {
      __shared__ int64_t rid[32];
      const EngramRows& E = p.eg;
      const int cols = k >> 8;
      // Thread c < cols computes row id c with the hash kernels' rules
      // (hash_window, hash_cols) from the loads issued before the ring; the
      // token -> compressed id lookup is a scalar load (it waits on the
      // scalar counter only, not behind the ring); the ids' table rows are
      // the third and last dependent round.
      const bool hthread = tid < cols;
      const int c = hthread ? tid : 0;
      const int nh = E.n_heads;
      const int64_t pos = E.pos;
      // The loaded values enter through empty asm statements, as opaque VGPR
      // values: otherwise the compiler, seeing uniform values, moves them to
      // scalar registers right after their loads, which means waiting for
      // the loads before the ring can go out.
#pragma unroll
      for (int i = 0; i < kMaxNgram; ++i) asm volatile("" : "+v"(h_cw[i]), "+v"(h_mu[i]));
      asm volatile("" : "+v"(h_t0), "+v"(h_pr), "+v"(h_of));
      const int32_t t0 = __builtin_amdgcn_readfirstlane(h_t0);
      const int64_t* cw = h_cw;
      const int64_t* mu = h_mu;
      const int64_t pr = h_pr, of = h_of;
      const bool tok_ok = t0 >= 0 && (int64_t)t0 < E.vocab;
      const int64_t own = tok_ok ? scalar_load_i64(E.token_map + t0) : -1;
      int64_t tk[kMaxNgram];
      bool blocked = own == -1;
      tk[0] = blocked ? E.pad_id : own;
#pragma unroll
      for (int i = 1; i < kMaxNgram; ++i) {
        blocked = blocked | (pos < i) | (cw[i] == -1);   // no short-circuit branches
        tk[i] = blocked ? E.pad_id : cw[i];
      }
      const int ic = c / nh + 1;                   // the window length of column c
      // rolling xor of the window's products: the running xor over i, then
      // column c's value at i = ic picked without branches
      uint64_t acc = (uint64_t)tk[0] * (uint64_t)mu[0];
      uint64_t rolling = acc;
#pragma unroll
      for (int i = 1; i < kMaxNgram; ++i) {
        acc ^= (uint64_t)tk[i] * (uint64_t)mu[i];
        rolling = i == ic ? acc : rolling;
      }
      // a prime <= 0 makes its column and every later one -1 (column order)
      const uint64_t badp = __ballot(hthread && pr <= 0);
      const bool ok = tok_ok && (badp & ((2ull << c) - 1ull)) == 0;
      const int64_t r = mod_euclid_i64((int64_t)rolling, ok ? pr : 1);
      const int64_t v = ok ? (int64_t)((uint64_t)r + (uint64_t)of) : -1;
      if (hthread) {
        rid[tid] = v;
        if (blockIdx.x == 0) {
          if (tid == 0) E.cache[pos] = own;
          if (!ok && E.err_flag != nullptr) *E.err_flag = 1;
        }
      }
      lds_barrier_m1();
      for (int c0 = 0; c0 < (k >> 3); c0 += 256) {
        const int chunk = c0 + tid;
        const bool active = chunk < (k >> 3);
        const int e0 = active ? chunk * 8 : 0;
        const int64_t id = rid[e0 >> 8];
        const int e = e0 & 255;
        uint32_t bits[8];
        if (id < 0 || id >= E.n_table_rows) {
#pragma unroll
          for (int i = 0; i < 8; ++i) bits[i] = 0x7fc0u;
          if (blockIdx.x == 0 && active && e == 0 && E.err_flag != nullptr) *E.err_flag = 1;
        } else {
          const uint8_t* blk = E.table + id * kBlockBytes;
          q2k_dequant4(blk, e, bits);
          q2k_dequant4(blk, e + 4, bits + 4);
        }
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = bf16_bits_to_f32(bits[i]);
        const Q8Lane r8 = q8_1_quant8(v);
        if (active) {
          q8_1_put8(r8, xs, e0, k);
          if (blockIdx.x == 0 && xq_out != nullptr) q8_1_put8(r8, xq_out, e0, k);
        }
      }
    } else {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        v[i] = qthread ? bf16_bits_to_f32(swiglu_bf16_bits(gv[i >> 2][i & 3], uv[i >> 2][i & 3])) : 0.0f;
      const Q8Lane r8 = q8_1_quant8(v);
      if (qthread) {
        q8_1_put8(r8, xs, se0, k);
        if (row_writer) q8_1_put8(r8, xq_out + (size_t)J.xrow * q8_row_bytes(k), se0, k);
      }
    }
    lds_barrier_m1();
    if (!live) return;
    act = load_ahalf_lds(xs, k, b, h);
  } else {
    // Activations first: the first step waits for them and ring slot 0 only.
    act = load_ahalf(J.x, tok, b, h);
  }
  double dq[4], dm[4];

  if (full) {
    if constexpr (FQ == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) ws[r] = load_whalf_at(wrun + (size_t)r * run_stride, off);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dm[j] = (double)act.d8[j];
      dq[j] = (j & 1) ? 0.25 * dm[j] : dm[j];
    }
#pragma unroll
    for (int g = 0; g < CH / V; ++g) {
      double acc[V];
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int st = g * V + v;                      // step within the run
        const double t = half_block_value_m1(ws[v % R], act, dq, dm);
        if (st + R < CH) ws[v % R] = load_whalf_at(wrun + (size_t)(st + R) * run_stride, off);
        acc[v] = hb_ok ? t : 0.0;
        __builtin_amdgcn_sched_barrier(0);
      }
      const double tot = reduce8<GSL>(acc, lane);
      if constexpr (FQ == 4) {
        const int row = (J.it + (g * V + slot) * S) * P + prow;
        const float yv = J.bad ? quiet_nan() : (float)tot;
        if (writer) {
          J.y[row] = yv;
          ysw[wiw & 1][row & 63] = yv;
        }
      } else {
        if (writer) J.y[(J.it + (g * V + slot) * S) * P + prow] = J.bad ? quiet_nan() : (float)tot;
      }
    }
  } else {
    // Guarded path: one direct load per step, rows past n read the step's
    // first row instead.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dm[j] = (double)act.d8[j];
      dq[j] = (j & 1) ? 0.25 * dm[j] : dm[j];
    }
    const LaneOffsets first = lane_offsets((uint32_t)b * kBlockBytes, h);
    for (int g0 = J.it; g0 < J.it_end; g0 += V * S) {
      double acc[V];
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int step = g0 + v * S;
        double val = 0.0;
        if (step < J.it_end) {
          const bool in = step * P + prow < J.n;
          const WHalf w = load_whalf_at(J.w + (size_t)step * step_bytes, in ? off : first);
          const double t = half_block_value_m1(w, act, dq, dm);
          val = (hb_ok && in) ? t : 0.0;
        }
        acc[v] = val;
      }
      const double tot = reduce8<GSL>(acc, lane);
      const int step = g0 + slot * S;
      const int row = step * P + prow;
      if constexpr (FQ == 4) {
        if (writer && step < J.it_end && row < J.n) {
          const float yv = J.bad ? quiet_nan() : (float)tot;
          J.y[row] = yv;
          ysw[wiw & 1][row & 63] = yv;
        }
      } else {
        if (writer && step < J.it_end && row < J.n) J.y[row] = J.bad ? quiet_nan() : (float)tot;
      }
    }
  }
  if constexpr (FQ == 4) {
    // The workgroup's 64 (gate, up) pairs -> bf16 SwiGLU -> two q8_1
    // blocks, one element per lane of wave 0: lane r forms h of row r; the
    // block maximum, the 16-wide sums and the packing of four quants per
    // word are cross-lane steps within the lane's 32-lane block.
    const int q = wave >> 2;
    const int i = q / p.pair_blocks;
    const int e = 64 * (q - i * p.pair_blocks) + lane;   // element of h's row
    lds_barrier_m1();
    if (wiw == 0) {
      const uint32_t hb = swiglu_bf16_bits(ysw[0][lane], ysw[1][lane]);
      if (p.sw_h != nullptr) p.sw_h[(size_t)i * J.n + e] = (uint16_t)hb;
      const float v = bf16_bits_to_f32(hb);
      float a = fmaxf(0.0f, fabsf(v));   // a NaN counts as 0, as in q8_1_quant8
      a = fmaxf(a, __uint_as_float(dpp_u32<0xB1>(__float_as_uint(a))));
      a = fmaxf(a, __uint_as_float(dpp_u32<0x4E>(__float_as_uint(a))));
      a = fmaxf(a, __uint_as_float(xor4_u32(__float_as_uint(a))));
      a = fmaxf(a, __uint_as_float(dpp_u32<0x128>(__float_as_uint(a))));
      {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
        a = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
      }
      const float d = q8_1_scale(a);
      int qv;
      q8_1_quant_lane<1>(&v, d, &qv);   // halves away from zero
      int sum = qv;
      sum += (int)dpp_u32<0xB1>((uint32_t)sum);
      sum += (int)dpp_u32<0x4E>((uint32_t)sum);
      sum += (int)xor4_u32((uint32_t)sum);
      sum += (int)dpp_u32<0x128>((uint32_t)sum);
      uint32_t word = ((uint32_t)qv & 0xffu) << (8 * (lane & 3));
      word |= dpp_u32<0xB1>(word);
      word |= dpp_u32<0x4E>(word);
      uint8_t* row = p.sw_hq + (size_t)i * q8_row_bytes(J.n);
      if ((lane & 3) == 0) *reinterpret_cast<uint32_t*>(row + e) = word;
      if ((lane & 31) == 0) *reinterpret_cast<float*>(row + q8_scale_offset(J.n) + (size_t)(e / 32) * 4) = d;
      if ((lane & 15) == 0)
        *reinterpret_cast<int16_t*>(row + q8_sum_offset(J.n) + (size_t)(e / 16) * 2) = (int16_t)sum;
    }
  }
  if (J.bad && lane == 0 && p.err_flag != nullptr) *p.err_flag = 1;
}

// Narrow rows (2 * k/256 <= 64 half blocks): one half block per lane.
//
// FQ (one token, one bf16 row p.xb16 shared by every matrix): the workgroup
// quantises the row into LDS as mmvq_m1_kernel's FQ = 1 prologue does
// (workgroup 0 also writes p.xq_out), after issuing its first weight loads.
template <int M, bool CACHE, int DEPTH, bool DOTS, bool FQ = false>
__global__ __launch_bounds__(256) void mmvq_narrow_kernel(const MmvqParams p) {
  static_assert(!FQ || (M == 1 && CACHE && !DOTS), "fused quantisation: one token, products only");
  prefetch_args(p);
  const int lane = threadIdx.x & 63;
  const int g8 = p.g8;
  const int wg = blockIdx.x;
  int wave = (((wg & 7) * g8) + (wg >> 3)) * 4 +
             __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const bool in_grid = wave < p.total_waves;
  if (!FQ && !in_grid) return;
  if (FQ && !in_grid) wave = p.total_waves - 1;   // a valid job; the wave exits after the barrier

  const int k = p.k;
  const int nb = k >> 8;
  const int gs = 1 << p.gs_log2;
  const int P = 64 >> p.gs_log2;
  const int prow = lane >> p.gs_log2;
  // half h = hb & 1 of super-block hb >> 1, as in mmvq_m1_kernel (lanes
  // past the row's blocks take block 0 and add +0)
  const int hb = lane & (gs - 1);
  const int braw = hb >> 1;
  const bool hb_ok = braw < nb;
  const int b = hb_ok ? braw : 0;
  const int h = hb & 1;
  const size_t rowbytes = (size_t)nb * kBlockBytes;

  // token split (one-token kernel only): as in mmvq_m1_kernel
  int tok = 0, jw = wave;
  if (M == 1 && p.tsplit > 1) {
    tok = wave % p.tsplit;
    jw = wave / p.tsplit;
  }
  WaveJob J = resolve_wave<M>(p, jw, P);
  J.y += (int64_t)tok * J.ldy;
  const bool live = in_grid && J.it < J.it_end;
  if (!FQ && !live) return;
  const uint8_t* wlane = J.w + b * kBlockBytes;

  WHalf ws[DEPTH];
  AHalf act;
  if constexpr (FQ) {
    extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
    const int tid = threadIdx.x;
    // one 32-value block per thread, or one 16-value half for k <= 4096
    // (the last two loads of a half then re-read its first, unused)
    const bool halves = k <= 4096;
    const bool qthread = tid < (halves ? (k >> 4) : (k >> 5));
    const uint8_t* xb = p.xb16 + (halves ? 32 : 64) * (qthread ? tid : 0);
    u32x4 raw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = gload<u32x4>(xb + ((halves && i >= 2) ? 0 : 16 * i));
    // first weight loads, unconditional and in bounds (block 0 of row 0
    // where the lane or the step has nothing to read), zeroed afterwards
    const uint8_t* wsafe = J.w + (hb_ok ? b : 0) * kBlockBytes;
    const int hs = hb_ok ? h : 0;
    bool wok[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int st = J.it + d * J.stride;
      const int row = st * P + prow;
      wok[d] = live && st < J.it_end && hb_ok && row < J.n;
      ws[d] = load_whalf(wsafe + (size_t)(wok[d] ? row : 0) * rowbytes, hs);
    }
    __builtin_amdgcn_sched_barrier(0);   // keep the weight loads ahead of the quantisation
    if (halves) q8_1_half_store(xs, blockIdx.x == 0 ? p.xq_out : nullptr, raw, tid, k, qthread);
    else q8_1_block_store(xs, blockIdx.x == 0 ? p.xq_out : nullptr, raw, tid, k, qthread);
    lds_barrier_m1();
    if (!live) return;
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
      if (!wok[d]) ws[d] = zero_whalf();
    act = hb_ok ? load_ahalf_lds(xs, k, b, h) : zero_ahalf();
  } else {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int st = J.it + d * J.stride;
      const int row = st * P + prow;
      ws[d] = (st < J.it_end && hb_ok && row < J.n) ? load_whalf(wlane + row * rowbytes, h)
                                                   : zero_whalf();
    }
    if constexpr (CACHE) act = hb_ok ? load_ahalf(J.x, tok, b, h) : zero_ahalf();
  }

  for (int base = J.it; base < J.it_end; base += DEPTH * J.stride) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int cur = base + d * J.stride;
      if (cur < J.it_end) {
        const WHalf w = ws[d];
        const int nxt = cur + DEPTH * J.stride;
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
            a = hb_ok ? load_ahalf(J.x, t, b, h) : zero_ahalf();
          }
          if constexpr (DOTS) {
            if (live) store_dots(p.dots, w, a, t, J.n, row, k, b, h);
          } else {
            double part = live ? half_block_value(w, a) : 0.0;
            part = group_sum(part, gs, lane);
            if (hb == 0 && row < J.n)
              J.y[(int64_t)t * J.ldy + row] = J.bad ? quiet_nan() : (float)part;
          }
        }
      }
    }
  }
  if (J.bad && lane == 0 && p.err_flag != nullptr) *p.err_flag = 1;
}

// Wide rows (more than 64 half blocks, k > 8192): one row per step. Lane
// l takes half h = l >> 5 of super-blocks 32c + (l & 31) for chunks
// c = 0, 1, ...; each chunk is summed over its 32 lanes neighbours first and
// the chunk sums are combined pairwise (a binary counter over the chunks, the
// row's block count rounded up to a power of two), then the two halves: the
// same tree as every other product kernel. Activations come from memory; the
// tokens are taken one after the other (each reloads the row, from cache).
constexpr int kWideLevels = 20;   // chunk tree depth: rows of up to 2^24 blocks

template <int M, bool DOTS>
__global__ __launch_bounds__(256) void mmvq_wide_kernel(const MmvqParams p) {
  prefetch_args(p);
  const int lane = threadIdx.x & 63;
  const int g8 = p.g8;
  const int wg = blockIdx.x;
  const int wave = (((wg & 7) * g8) + (wg >> 3)) * 4 +
                   __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  if (wave >= p.total_waves) return;
  const int k = p.k;
  const int nb = k >> 8;
  int chunks = 1;
  while (32 * chunks < nb) chunks <<= 1;
  int top = 0;
  while ((1 << top) < chunks) ++top;
  const size_t rowbytes = (size_t)nb * kBlockBytes;
  const int h = lane >> 5;
  const int jl = lane & 31;
  const WaveJob J = resolve_wave<M>(p, wave, 1);
  for (int row = J.it; row < J.it_end; row += J.stride) {
#pragma unroll 1
    for (int t = 0; t < M; ++t) {
      double stk[kWideLevels];
#pragma unroll
      for (int l = 0; l < kWideLevels; ++l) stk[l] = 0.0;
      for (int c = 0; c < chunks; ++c) {
        const int b = 32 * c + jl;
        double v = 0.0;
        if (b < nb) {
          const WHalf w = load_whalf(J.w + row * rowbytes + b * kBlockBytes, h);
          const AHalf a = load_ahalf(J.x, t, b, h);
          if constexpr (DOTS) {
            store_dots(p.dots, w, a, t, J.n, row, k, b, h);
          } else {
            v = half_block_value(w, a);
          }
        }
        if constexpr (!DOTS) {
          // the chunk's 32 leaves, neighbours first (partners l ^ 1 .. l ^ 16)
          v += dpp_f64<DppPartner<1>::ctrl>(v);
          v += dpp_f64<DppPartner<2>::ctrl>(v);
          v += xor4_f64(v);
          v += dpp_f64<DppPartner<8>::ctrl>(v);
          v = halve<16>(v, v, lane);
          // binary counter: chunk c closes the subtrees of its trailing ones
          bool carry = true;
#pragma unroll
          for (int l = 0; l < kWideLevels; ++l) {
            if (carry) {
              if ((c >> l) & 1) {
                v = stk[l] + v;
              } else {
                stk[l] = v;
                carry = false;
              }
            }
          }
        }
      }
      if constexpr (!DOTS) {
        double tot = 0.0;
#pragma unroll
        for (int l = 0; l < kWideLevels; ++l)
          if (l == top) tot = stk[l];
        tot = halve<32>(tot, tot, lane);   // the two halves
        if (lane == 0) J.y[(int64_t)t * J.ldy + row] = J.bad ? quiet_nan() : (float)tot;
      }
    }
  }
  if (J.bad && lane == 0 && p.err_flag != nullptr) *p.err_flag = 1;
}

namespace {

// Launch shapes, fixed at compile time (measured on MI355X). None of them
// changes a result bit: every kernel's result is independent of its grid,
// run length and ring depth, and all kernels follow one summation order.
struct Tuning {
  int waves_per_cu = 16;        // one-step kernel: waves per CU
  int depth = 2;                // one-step kernel: row steps in flight per wave
  int interleave = 1;           // a matrix's waves take its row steps round-robin
  int ring = 4;                 // run kernel: weight steps in flight per wave
  int m1_waves_per_cu = 4;      // run kernel: waves per CU (one per SIMD)
  int64_t m1_min_steps = 2048;  // run kernel from this many (row step, token) pairs
};

constexpr Tuning kTuning{};

const Tuning& tuning() { return kTuning; }

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

// One matrix, one token, interleaved runs: the run kernel needs only its
// leading scalar arguments (and can take the bf16 row itself).
bool plain_launch(const MmvqParams& p) {
  return p.ids == nullptr && p.groups == 0 && p.wave_end[0] == p.total_waves && p.interleave &&
         p.tsplit == 1;
}

// The run kernel with fused quantisation: x_bf16 is the token's bf16 row
// (shared by every matrix of the launch), xq receives its q8_1 row. One
// token, default ring.
template <int FQ>
void dispatch_m1_fused(const MmvqParams& p, dim3 grid, const void* x_bf16, uint8_t* xq,
                       hipStream_t s) {
  const int ch = p.chunk;
  const size_t lds = q8_row_bytes(p.k);
  const uint8_t* x = static_cast<const uint8_t*>(x_bf16);
  const int32_t plain = plain_launch(p) ? 1 : 0;
#define Q2K_M1F(G, R, C)                                                                       \
  hipLaunchKernelGGL((mmvq_m1_kernel<G, R, C, FQ>), grid, dim3(256), lds, s, p.w[0], x,        \
                     p.y[0], p.n[0], p.k, p.total_waves, p.g8, plain, xq, p)
#define Q2K_M1F_CH(G)                            \
  do {                                           \
    if (ch == 8) Q2K_M1F(G, 4, 8);               \
    else if (ch == 16) Q2K_M1F(G, 4, 16);        \
    else Q2K_M1F(G, 4, 32);                      \
  } while (0)
  switch (p.gs_log2) {
    case 3: Q2K_M1F_CH(3); return;
    case 4: Q2K_M1F_CH(4); return;
    case 5: Q2K_M1F_CH(5); return;
    default: Q2K_M1F_CH(6); return;
  }
#undef Q2K_M1F_CH
#undef Q2K_M1F
}

// FQ = 4: 32 rows per wave, so the run length follows the row group size.
void dispatch_m1_swiglu(const MmvqParams& p, dim3 grid, const void* x_bf16, uint8_t* xq,
                        hipStream_t s) {
  const size_t lds = q8_row_bytes(p.k);
  const uint8_t* x = static_cast<const uint8_t*>(x_bf16);
#define Q2K_M1S(G, C)                                                                          \
  hipLaunchKernelGGL((mmvq_m1_kernel<G, 4, C, 4>), grid, dim3(256), lds, s, p.w[0], x, p.y[0], \
                     p.n[0], p.k, p.total_waves, p.g8, 0, xq, p)
  if (p.gs_log2 == 4) Q2K_M1S(4, 8);
  else if (p.gs_log2 == 5) Q2K_M1S(5, 16);
  else Q2K_M1S(6, 32);
#undef Q2K_M1S
}

template <int M>
void dispatch_narrow(const MmvqParams& p, dim3 grid, bool dots, int depth, bool run_kernel,
                     hipStream_t s) {
  if (M == 1 && run_kernel) {
    const int ring = tuning().ring;
    const int ch = p.chunk;
    const int32_t plain = plain_launch(p) ? 1 : 0;
#define Q2K_M1_ARGS p.w[0], p.xq, p.y[0], p.n[0], p.k, p.total_waves, p.g8, plain, nullptr, p
#define Q2K_M1(G, R, C) \
  hipLaunchKernelGGL((mmvq_m1_kernel<G, R, C, 0>), grid, dim3(256), 0, s, Q2K_M1_ARGS)
#define Q2K_M1_CH(G, R)                          \
  do {                                           \
    if (ch == 8) Q2K_M1(G, R, 8);                \
    else if (ch == 16) Q2K_M1(G, R, 16);         \
    else Q2K_M1(G, R, 32);                       \
  } while (0)
#define Q2K_M1_RING(G)                           \
  do {                                           \
    if (ring == 2) Q2K_M1_CH(G, 2);              \
    else if (ring == 8) Q2K_M1_CH(G, 8);         \
    else Q2K_M1_CH(G, 4);                        \
  } while (0)
    switch (p.gs_log2) {
      case 3: Q2K_M1_RING(3); return;
      case 4: Q2K_M1_RING(4); return;
      case 5: Q2K_M1_RING(5); return;
      default: Q2K_M1_RING(6); return;
    }
#undef Q2K_M1_RING
#undef Q2K_M1_CH
#undef Q2K_M1
#undef Q2K_M1_ARGS
  }
  if (dots) {
    hipLaunchKernelGGL((mmvq_narrow_kernel<M, false, 1, true>), grid, dim3(256), 0, s, p);
  } else if constexpr (M == 1) {
    // products take one token per wave (m > 1: token split)
    if (depth == 1)
      hipLaunchKernelGGL((mmvq_narrow_kernel<M, true, 1, false>), grid, dim3(256), 0, s, p);
    else if (depth == 4)
      hipLaunchKernelGGL((mmvq_narrow_kernel<M, true, 4, false>), grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((mmvq_narrow_kernel<M, true, 2, false>), grid, dim3(256), 0, s, p);
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

// Product kernel choice (q2k_set_product_kernel): 0 automatic (the cost
// model), 1 matrix cores where supported, 2 packed dots only. Every choice
// returns the same bits (one summation order in every kernel); it only
// changes which kernel runs.
static std::atomic<int> g_product_kernel{0};

static int product_kernel() { return g_product_kernel.load(std::memory_order_relaxed); }

int set_product_kernel(int choice) {
  return g_product_kernel.exchange(choice, std::memory_order_relaxed);
}

bool takes_mfma(const MmvqLaunch& a) {
  const int choice = product_kernel();
  return choice == 1 ? (a.m >= 2 && mfma_supports(a.k)) : choice == 2 ? false : mfma_preferred(a);
}

// The SwiGLU epilogue (FQ = 4) takes gate and up of one token, one shared
// bf16 row, rows of 2048 to 8192 values on the run kernel's ring of 4, and
// whole 64-row blocks.
static bool swiglu_epilogue_fits(const MmvqLaunch& a, bool mfma) {
  return a.ids != nullptr && a.njobs == 2 && a.m == 1 && a.x_per_id == 0 && a.x_bf16 != nullptr &&
         a.dots == nullptr && a.sg == nullptr && !mfma && a.k >= 2048 && a.k <= 8192 &&
         a.n[0] % 64 == 0 && tuning().ring == 4;
}

hipError_t launch_mmvq(const MmvqLaunch& a, hipStream_t stream) {
  // the integer stage (dots) goes to the kernel the product would take
  const bool mfma = takes_mfma(a);
  if (a.sw_hq != nullptr && !swiglu_epilogue_fits(a, mfma)) {
    // the product, then the SwiGLU launch on its two result sets
    MmvqLaunch b = a;
    b.sw_hq = b.sw_h = nullptr;
    const hipError_t e = launch_mmvq(b, stream);
    if (e != hipSuccess) return e;
    const float* yg = a.y[0];
    const float* yu = a.y[0] + (size_t)a.n_ids * a.n[0];
    return launch_swiglu_q8_1_rows(yg, yu, a.sw_h, a.sw_hq, a.n_ids, a.n[0], stream);
  }
  if (a.sg != nullptr && (mfma || a.m > kMaxM)) {
    const hipError_t e = launch_swiglu_q8_1_rows(a.sg, a.su, nullptr, const_cast<void*>(a.xq),
                                                 a.n_ids * a.m, a.k, stream);
    if (e != hipSuccess) return e;
    MmvqLaunch b = a;
    b.sg = b.su = nullptr;
    return launch_mmvq(b, stream);
  }
  if (a.x_bf16 != nullptr && (mfma || a.m > kMaxM)) {
    // quantisation first, then the product on the q8_1 rows
    const hipError_t e = launch_q8_1_rows(a.x_bf16, a.x_stride, const_cast<void*>(a.xq), a.m, a.k,
                                          stream);
    if (e != hipSuccess) return e;
    MmvqLaunch b = a;
    b.x_bf16 = nullptr;
    return launch_mmvq(b, stream);
  }
  if (mfma) return launch_mmvq_mfma(a, stream);
  if (a.m > kMaxM) {
    // More tokens than the packed-dot kernels take: one launch per group of
    // kMaxM tokens (plain single-matrix launches only).
    if (a.ids != nullptr || a.groups > 0 || a.njobs != 1) return hipErrorInvalidValue;
    const size_t rb = q8_row_bytes(a.k);
    for (int t0 = 0; t0 < a.m; t0 += kMaxM) {
      MmvqLaunch g = a;
      g.m = a.m - t0 < kMaxM ? a.m - t0 : kMaxM;
      g.xq = static_cast<const uint8_t*>(a.xq) + (size_t)t0 * rb;
      if (a.dots != nullptr) g.dots = a.dots + (size_t)t0 * a.n[0] * (a.k / 32) * 2;
      else g.y[0] = a.y[0] + (size_t)t0 * a.n[0];
      const hipError_t e = launch_mmvq(g, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
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
  p.groups = a.groups;
  p.k = a.k;
  p.gs_log2 = gs_log2;

  // Row steps per job, then a run length that spreads them over about
  // waves_per_cu waves per CU, then whole runs per job (no run straddles
  // two matrices, so each wave resolves its matrix once).
  const int n_jobs = uniform_jobs(a) ? a.njobs * a.n_ids : a.njobs;
  int64_t total_iters = 0;
  int64_t iters_of[kMaxPlainJobs] = {0, 0, 0, 0};
  if (!uniform_jobs(a)) {
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
  // m > 1 on the packed-dot path (rows of at most 8192 values): the
  // one-token kernels with the tokens taken by separate waves, so the
  // activations stay in registers (a wave that took all m tokens reloaded
  // them for every token and step: 13 us against 5.9 us on the attention
  // pair at m = 8)
  const int tsplit = (a.dots == nullptr && !wide) ? a.m : 1;
  p.tsplit = tsplit;
  // The run kernel (runs of 8 to 32 steps per wave) needs enough steps to
  // fill the chip; smaller launches take one step per wave.
  const bool m1_path = a.dots == nullptr && !wide && gs_log2 >= 3 &&
                       total_iters * tsplit >= tu.m1_min_steps;
  // A one-token launch that quantises its own input (one bf16 row shared by
  // every matrix) does it in the run kernel's prologue when the product
  // takes the run kernel anyway (so the bits are those of the separate
  // calls).
  const bool fuse_x = a.x_bf16 != nullptr && m1_path && tu.ring == 4 && a.groups == 0 &&
                      a.m == 1 && (a.ids == nullptr || a.x_per_id == 0);
  // Several tokens that quantise their own rows (plain jobs): one token per
  // workgroup in the run kernel (FQ = 5), each workgroup quantising only its
  // token's row in its prologue (with the tokens split over the waves of a
  // workgroup it would quantise four rows: 12.5 against 8.5 us for the q8_1
  // launch and the product on the attention pair at m = 4; one row per
  // workgroup: 8.42 against 8.50 us, m = 8: 8.35 against 8.57 us).
  const bool fuse_xs = a.x_bf16 != nullptr && m1_path && tu.ring == 4 && a.groups == 0 &&
                       a.ids == nullptr && a.m > 1 && tsplit == a.m && a.k <= 8192;
  const int64_t target_waves =
      (int64_t)cu_count() * (m1_path ? tu.m1_waves_per_cu : tu.waves_per_cu);
  int64_t chunk = (total_iters * tsplit + target_waves - 1) / target_waves;
  if (tsplit > 1 && !m1_path) chunk = 1;
  if (m1_path) {
    // runs of 8, 16 or 32 steps (compile-time run lengths of the m = 1 kernel)
    chunk = chunk <= 8 ? 8 : chunk <= 16 ? 16 : 32;
  }
  p.chunk = (int)chunk;
  int64_t total_waves = 0;
  if (!uniform_jobs(a)) {
    for (int j = 0; j < kMaxPlainJobs; ++j) {
      total_waves += j < a.njobs ? (iters_of[j] + chunk - 1) / chunk : 0;
      p.wave_end[j] = (int)total_waves;
    }
  } else {
    p.waves_per_job = (int)((iters_of[0] + chunk - 1) / chunk);
    total_waves = (int64_t)p.waves_per_job * n_jobs;
  }
  const int64_t waves_per_token = total_waves;
  total_waves *= tsplit;
  p.total_waves = (int)total_waves;
  p.interleave = tu.interleave;
  int64_t groups = (total_waves + 3) / 4;
  groups = (groups + 7) / 8 * 8;
  p.g8 = (int)(groups / 8);
  const dim3 grid((unsigned)groups);
  const bool dots = a.dots != nullptr;
  if (a.sg != nullptr) {
    // SwiGLU + q8_1 of each id's row inside the down product when every
    // workgroup lies inside one id's waves; else the SwiGLU launch first
    p.sg = a.sg;
    p.su = a.su;
    if (m1_path && a.m == 1 && !dots && a.ids != nullptr && a.x_per_id == 1 && a.k <= 2048 &&
        p.waves_per_job % 4 == 0 && tu.ring == 4) {
      dispatch_m1_fused<2>(p, grid, nullptr, static_cast<uint8_t*>(const_cast<void*>(a.xq)), stream);
      return hipGetLastError();
    }
    const hipError_t e = launch_swiglu_q8_1_rows(a.sg, a.su, nullptr, const_cast<void*>(a.xq),
                                                 a.n_ids * a.m, a.k, stream);
    if (e != hipSuccess) return e;
  }
  if (a.eg != nullptr) {
    // the input row is a decode token's engram rows: formed in the run
    // kernel's prologue when the product takes it, else by the rows launch
    p.eg = *a.eg;
    if (m1_path && a.m == 1 && a.njobs == 1 && a.ids == nullptr && a.groups == 0 && !dots &&
        a.k <= 8192 && tu.ring == 4) {
      dispatch_m1_fused<3>(p, grid, nullptr, static_cast<uint8_t*>(const_cast<void*>(a.xq)), stream);
      return hipGetLastError();
    }
    const EngramRows& E = *a.eg;
    const hipError_t e = launch_engram_rows_q8_1(E.token_map, E.vocab, E.mult, E.primes, E.offsets,
                                                 E.layer, E.ng, E.n_heads, E.pad_id, E.cache, E.token,
                                                 E.pos, E.table, E.n_table_rows, nullptr, nullptr,
                                                 const_cast<void*>(a.xq), E.err_flag, stream);
    if (e != hipSuccess) return e;
  }
  if (a.sw_hq != nullptr) {
    // gate and up with their SwiGLU in the epilogue: workgroups of 64 rows
    // of one id, both matrices (resolve_pair)
    p.pair_blocks = a.n[0] / 64;
    p.chunk = 32 / P;
    p.interleave = 0;
    p.total_waves = a.n_ids * p.pair_blocks * 4;
    const int64_t wgs = ((int64_t)a.n_ids * p.pair_blocks + 7) / 8 * 8;
    p.g8 = (int)(wgs / 8);
    p.sw_hq = static_cast<uint8_t*>(a.sw_hq);
    p.sw_h = static_cast<uint16_t*>(a.sw_h);
    dispatch_m1_swiglu(p, dim3((unsigned)wgs), a.x_bf16,
                       static_cast<uint8_t*>(const_cast<void*>(a.xq)), stream);
    return hipGetLastError();
  }
  if (a.x_bf16 != nullptr) {
    if (fuse_x) {
      dispatch_m1_fused<1>(p, grid, a.x_bf16, static_cast<uint8_t*>(const_cast<void*>(a.xq)), stream);
      return hipGetLastError();
    }
    if (fuse_xs) {
      const int64_t wgs = ((waves_per_token + 3) / 4 * tsplit + 7) / 8 * 8;
      p.total_waves = (int)waves_per_token;
      p.g8 = (int)(wgs / 8);
      p.x_row_bytes = a.x_stride * 2;
      dispatch_m1_fused<5>(p, dim3((unsigned)wgs), a.x_bf16,
                           static_cast<uint8_t*>(const_cast<void*>(a.xq)), stream);
      return hipGetLastError();
    }
    // the same prologue in the one-step kernel, for the smaller one-token
    // launches (same kernel as without it, so the same bits)
    if (!m1_path && !wide && !dots && a.m == 1 && a.groups == 0 &&
        (a.ids == nullptr || a.x_per_id == 0)) {
      p.xb16 = static_cast<const uint8_t*>(a.x_bf16);
      p.xq_out = static_cast<uint8_t*>(const_cast<void*>(a.xq));
      const size_t lds = q8_row_bytes(a.k);
      if (tu.depth == 1)
        hipLaunchKernelGGL((mmvq_narrow_kernel<1, true, 1, false, true>), grid, dim3(256), lds, stream, p);
      else if (tu.depth == 4)
        hipLaunchKernelGGL((mmvq_narrow_kernel<1, true, 4, false, true>), grid, dim3(256), lds, stream, p);
      else
        hipLaunchKernelGGL((mmvq_narrow_kernel<1, true, 2, false, true>), grid, dim3(256), lds, stream, p);
      return hipGetLastError();
    }
    const hipError_t e = launch_q8_1_rows(a.x_bf16, a.x_stride, const_cast<void*>(a.xq), a.m, a.k,
                                          stream);
    if (e != hipSuccess) return e;
  }

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
  } else if (tsplit > 1) {
    dispatch_narrow<1>(p, grid, dots, tu.depth, m1_path, stream);
  } else {
    switch (a.m) {
      case 1: dispatch_narrow<1>(p, grid, dots, tu.depth, m1_path, stream); break;
      case 2: dispatch_narrow<2>(p, grid, dots, tu.depth, false, stream); break;
      case 3: dispatch_narrow<3>(p, grid, dots, tu.depth, false, stream); break;
      case 4: dispatch_narrow<4>(p, grid, dots, tu.depth, false, stream); break;
      case 5: dispatch_narrow<5>(p, grid, dots, tu.depth, false, stream); break;
      case 6: dispatch_narrow<6>(p, grid, dots, tu.depth, false, stream); break;
      case 7: dispatch_narrow<7>(p, grid, dots, tu.depth, false, stream); break;
      default: dispatch_narrow<8>(p, grid, dots, tu.depth, false, stream); break;
    }
  }
  return hipGetLastError();
}

}  // namespace q2k
