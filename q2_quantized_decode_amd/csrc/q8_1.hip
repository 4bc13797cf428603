// q8_1 activation rows and the fused bf16 SwiGLU + q8_1 re-quantisation.
//
// q8_1 (moe_v41/init.rs: kquant_q8_1_rows_bf16; attn_v41/decode.rs,
// q_kv_projections): each 32-wide block of a row gets d = amax / 127 and
// int8 quants round(x / d). This library stores d as f32 and, for the Q2_K
// min term, the integer sum of every 16 quants.
//
// Launch shape: one lane per 8 consecutive values (one 16-byte bf16 load),
// four lanes per 32-block; the block's amax and the 16-wide sums are
// combined across those lanes with shuffles. The quantiser is latency bound
// (at most a few tens of thousands of values per call), so the only goal is
// one pass with coalesced 16-byte loads.
#include "q2k_device.h"
#include "q2k_launch.h"

namespace q2k {

__global__ __launch_bounds__(256) void q8_1_rows_kernel(const uint16_t* __restrict__ x,
                                                        int64_t stride, uint8_t* __restrict__ xq,
                                                        int m, int k) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_row = k / 8;
  const int64_t total = (int64_t)m * per_row;
  const bool active = gid < total;
  const int64_t row = active ? gid / per_row : 0;
  const int e0 = active ? (int)(gid - row * per_row) * 8 : 0;
  float v[8];
  if (active) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(x + row * stride + e0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_bits_to_f32(raw[i] & 0xffffu);
      v[2 * i + 1] = bf16_bits_to_f32(raw[i] >> 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }
  q8_1_store8(v, xq + row * q8_row_bytes(k), e0, k, active);
}

// h = bf16(silu(g) * u), then q8_1 of h. silu(g) = g / (1 + exp(-g)), in f32.
__global__ __launch_bounds__(256) void swiglu_q8_1_rows_kernel(const float* __restrict__ g,
                                                               const float* __restrict__ u,
                                                               uint16_t* __restrict__ h_out,
                                                               uint8_t* __restrict__ hq,
                                                               int rows, int k) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_row = k / 8;
  const int64_t total = (int64_t)rows * per_row;
  const bool active = gid < total;
  const int64_t row = active ? gid / per_row : 0;
  const int e0 = active ? (int)(gid - row * per_row) * 8 : 0;
  float v[8];
  uint32_t hb[8];
  if (active) {
    const size_t off = (size_t)row * k + e0;
    const f32x4 g0 = *reinterpret_cast<const f32x4*>(g + off);
    const f32x4 g1 = *reinterpret_cast<const f32x4*>(g + off + 4);
    const f32x4 u0 = *reinterpret_cast<const f32x4*>(u + off);
    const f32x4 u1 = *reinterpret_cast<const f32x4*>(u + off + 4);
    const float gg[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
    const float uu[8] = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      hb[i] = swiglu_bf16_bits(gg[i], uu[i]);
      v[i] = bf16_bits_to_f32(hb[i]);
    }
    if (h_out != nullptr) {
      u32x4 packed;
#pragma unroll
      for (int i = 0; i < 4; ++i) packed[i] = hb[2 * i] | (hb[2 * i + 1] << 16);
      *reinterpret_cast<u32x4*>(h_out + off) = packed;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }
  q8_1_store8(v, hq + row * q8_row_bytes(k), e0, k, active);
}

// Gathered Q2_K table rows -> bf16 (optional output) -> one q8_1 row of
// width 256 * n_rows: lane i takes elements 8i..8i+7, i.e. elements
// e = 8i mod 256 .. +7 of row 8i / 256, dequantised exactly as
// dequant_rows_kernel does and quantised exactly as q8_1_rows_kernel does
// (an id outside the table gives that row NaN bf16 values, as there).
__global__ __launch_bounds__(256) void dequant_rows_q8_1_kernel(const uint8_t* __restrict__ table,
                                                                int64_t n_table_rows,
                                                                const int64_t* __restrict__ ids,
                                                                int n_rows, uint16_t* __restrict__ out,
                                                                uint8_t* __restrict__ xq,
                                                                int32_t* err_flag) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int k = n_rows * kBlockWeights;
  const bool active = gid < k / 8;
  const int e0 = active ? (int)gid * 8 : 0;
  const int row = e0 / kBlockWeights, e = e0 % kBlockWeights;
  const int64_t id = ids ? ids[row] : row;
  const bool bad = id < 0 || id >= n_table_rows;
  uint32_t bits[8];
  if (bad) {
#pragma unroll
    for (int i = 0; i < 8; ++i) bits[i] = 0x7fc0u;
    if (active && e == 0 && err_flag != nullptr) *err_flag = 1;
  } else {
    const uint8_t* blk = table + id * kBlockBytes;
    q2k_dequant4(blk, e, bits);
    q2k_dequant4(blk, e + 4, bits + 4);
  }
  if (active && out != nullptr) {
    u32x4 packed;
#pragma unroll
    for (int i = 0; i < 4; ++i) packed[i] = bits[2 * i] | (bits[2 * i + 1] << 16);
    *reinterpret_cast<u32x4*>(out + e0) = packed;
  }
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = bf16_bits_to_f32(bits[i]);
  q8_1_store8(v, xq, e0, k, active);
}

hipError_t launch_dequant_rows_q8_1(const void* table, int64_t n_table_rows, const int64_t* ids,
                                    int n_rows, void* out, void* xq, int32_t* err_flag,
                                    hipStream_t stream) {
  const int64_t lanes = (int64_t)n_rows * (kBlockWeights / 8);
  const int64_t blocks = (lanes + 255) / 256;
  hipLaunchKernelGGL(dequant_rows_q8_1_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(table), n_table_rows, ids, n_rows,
                     static_cast<uint16_t*>(out), static_cast<uint8_t*>(xq), err_flag);
  return hipGetLastError();
}

hipError_t launch_q8_1_rows(const void* x, int64_t stride, void* xq, int m, int k,
                            hipStream_t stream) {
  const int64_t lanes = (int64_t)m * (k / 8);
  const int64_t blocks = (lanes + 255) / 256;
  hipLaunchKernelGGL(q8_1_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(x), stride, static_cast<uint8_t*>(xq), m, k);
  return hipGetLastError();
}

hipError_t launch_swiglu_q8_1_rows(const float* g, const float* u, void* h, void* hq, int rows,
                                   int k, hipStream_t stream) {
  const int64_t lanes = (int64_t)rows * (k / 8);
  const int64_t blocks = (lanes + 255) / 256;
  hipLaunchKernelGGL(swiglu_q8_1_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, g, u,
                     static_cast<uint16_t*>(h), static_cast<uint8_t*>(hq), rows, k);
  return hipGetLastError();
}

}  // namespace q2k
