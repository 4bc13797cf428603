// Engram row gather + Q2_K dequantisation to bf16, and the engram gate.
//
// Rows (engram_v41.rs, EngramV41::rows_from_q2k and its dequant_q2_k_to_bf16
// launch): each table row is one 256-wide Q2_K block. The pages gather the
// blocks on the host and upload them; here the row ids are read on the
// device, so the table stays resident in HBM and only ids cross PCIe.
// One wave per row, four elements per lane, one 8-byte bf16 store per lane.
//
// Gate (engram_v41/apply.rs, engram_v41_gate with grid [T, hc]; engram_v41.rs
// module doc step 4): one 256-thread workgroup per (token, stream) forms
// three sums over dim in a fixed order, then updates the stream in place
// (16-byte loads, all issued at once, when dim % 4 == 0, dim <= 16384 and
// the pointers are 16-byte aligned; strided scalar loads otherwise).
//
// N-gram hash (engram_v41.rs, EngramHasher::hash, which the pages run on the
// host): one thread per (position, hashed layer), so the row ids are made on
// the device next to the table they index.
#include "q2k_device.h"
#include "q2k_launch.h"

namespace q2k {

__global__ __launch_bounds__(256) void dequant_rows_kernel(const uint8_t* __restrict__ table,
                                                           int64_t n_table_rows,
                                                           const int64_t* __restrict__ ids,
                                                           int n_rows, uint16_t* __restrict__ out,
                                                           int32_t* err_flag) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n_rows) return;
  const int lane = threadIdx.x & 63;
  const int64_t id = ids ? ids[row] : row;
  uint16_t* o = out + (int64_t)row * kBlockWeights + 4 * lane;
  if (id < 0 || id >= n_table_rows) {
    *reinterpret_cast<u32x2*>(o) = u32x2{0x7fc07fc0u, 0x7fc07fc0u};
    if (lane == 0 && err_flag != nullptr) *err_flag = 1;
    return;
  }
  uint32_t bits[4];
  q2k_dequant4(table + id * kBlockBytes, 4 * lane, bits);
  *reinterpret_cast<u32x2*>(o) = u32x2{bits[0] | (bits[1] << 16), bits[2] | (bits[3] << 16)};
}

// The three gate sums over a 256-thread workgroup at once: each wave folds
// its 64 lanes (wave_sum_f32: partners l ^ 1 .. l ^ 32), then the four wave
// sums are added as (w0 + w1) + (w2 + w3). One barrier for all three.
__device__ __forceinline__ void block_sum3_256(float& a, float& b, float& c, float* lds) {
  a = wave_sum_f32(a);
  b = wave_sum_f32(b);
  c = wave_sum_f32(c);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    lds[wave] = a;
    lds[4 + wave] = b;
    lds[8 + wave] = c;
  }
  __syncthreads();
  a = (lds[0] + lds[1]) + (lds[2] + lds[3]);
  b = (lds[4] + lds[5]) + (lds[6] + lds[7]);
  c = (lds[8] + lds[9]) + (lds[10] + lds[11]);
}

__global__ __launch_bounds__(256) void engram_gate_kernel(float* __restrict__ h,
                                                          const float* __restrict__ kv,
                                                          const float* __restrict__ qk, int hc,
                                                          int dim, float eps) {
  __shared__ float lds[12];
  const int t = blockIdx.x;
  const int j = blockIdx.y;
  float* hs = h + ((int64_t)t * hc + j) * dim;
  const float* key = kv + (int64_t)t * (hc + 1) * dim + (int64_t)j * dim;
  const float* val = kv + (int64_t)t * (hc + 1) * dim + (int64_t)hc * dim;
  const float* w = qk + (int64_t)j * dim;
  float shh = 0.0f, skk = 0.0f, sqk = 0.0f;
  for (int i = threadIdx.x; i < dim; i += 256) {
    const float x = hs[i];
    const float kk = key[i];
    shh = fmaf(x, x, shh);
    skk = fmaf(kk, kk, skk);
    sqk = fmaf(w[i] * x, kk, sqk);
  }
  block_sum3_256(shh, skk, sqk, lds);
  const float rh = sqrtf(shh / (float)dim + eps);
  const float rk = sqrtf(skk / (float)dim + eps);
  const float s = sqk / (rh * rk * sqrtf((float)dim));
  const float sg = copysignf(sqrtf(fabsf(s)), s);
  const float g = 1.0f / (1.0f + expf(-sg));
  for (int i = threadIdx.x; i < dim; i += 256) hs[i] = fmaf(g, val[i], hs[i]);
}

// The same gate with 16-byte loads: thread i takes float4 elements i, i + 256,
// ... (NV4 of them per array, dim = 4 * n4 <= 1024 * NV4), and every load of
// the stream, key, weights and value goes out before the first sum, so the
// kernel waits for memory once instead of once per strided scalar load.
// Each thread sums its values in a fixed order, then the same fixed tree.
template <int NV4>
__global__ __launch_bounds__(256) void engram_gate_vec_kernel(float* __restrict__ h,
                                                              const float* __restrict__ kv,
                                                              const float* __restrict__ qk,
                                                              int hc, int dim, float eps) {
  __shared__ float lds[12];
  const int t = blockIdx.x;
  const int j = blockIdx.y;
  const int n4 = dim >> 2;
  f32x4* hs = reinterpret_cast<f32x4*>(h + ((int64_t)t * hc + j) * dim);
  const f32x4* key = reinterpret_cast<const f32x4*>(kv + (int64_t)t * (hc + 1) * dim + (int64_t)j * dim);
  const f32x4* val = reinterpret_cast<const f32x4*>(kv + (int64_t)t * (hc + 1) * dim + (int64_t)hc * dim);
  const f32x4* w = reinterpret_cast<const f32x4*>(qk + (int64_t)j * dim);
  f32x4 x[NV4], kk[NV4], ww[NV4], vv[NV4];
#pragma unroll
  for (int c = 0; c < NV4; ++c) {
    const int i = (int)threadIdx.x + 256 * c;
    const int ic = i < n4 ? i : 0;   // unconditional loads, zeroed below
    x[c] = hs[ic];
    kk[c] = key[ic];
    ww[c] = w[ic];
    vv[c] = val[ic];
  }
  float shh = 0.0f, skk = 0.0f, sqk = 0.0f;
#pragma unroll
  for (int c = 0; c < NV4; ++c) {
    if ((int)threadIdx.x + 256 * c < n4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        shh = fmaf(x[c][e], x[c][e], shh);
        skk = fmaf(kk[c][e], kk[c][e], skk);
        sqk = fmaf(ww[c][e] * x[c][e], kk[c][e], sqk);
      }
    }
  }
  block_sum3_256(shh, skk, sqk, lds);
  const float rh = sqrtf(shh / (float)dim + eps);
  const float rk = sqrtf(skk / (float)dim + eps);
  const float s = sqk / (rh * rk * sqrtf((float)dim));
  const float sg = copysignf(sqrtf(fabsf(s)), s);
  const float g = 1.0f / (1.0f + expf(-sg));
#pragma unroll
  for (int c = 0; c < NV4; ++c) {
    const int i = (int)threadIdx.x + 256 * c;
    if (i < n4) {
      f32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = fmaf(g, vv[c][e], x[c][e]);
      hs[i] = o;
    }
  }
}

// Row ids of the engram n-gram hash. Thread (s, l): position pos = start_pos + s,
// hashed layer l. Window token i (i < ng) is the compressed id of position
// pos - i (position 0 when pos < i): from this call's token ids when that
// position is >= start_pos, else from the cache; from the first i with
// pos < i or an unmapped (-1) id on, the token is pad_id. Then
// rolling = tok[0]*mult[l][0], rolling ^= tok[i]*mult[l][i] (64-bit
// wrapping), and row id (i, h) = (rolling mod prime, in [0, prime)) + offset.
// Output layout [n_layers][seqlen][cols]. The thread of layer 0 stores the
// compressed id of its position into the cache (only positions >= start_pos
// are written; only positions < start_pos are read from the cache).
// A token id outside [0, vocab), or a prime <= 0, gives -1 for every row id
// whose window reads it, -1 in the cache, and *err_flag = 1.
__global__ __launch_bounds__(256) void engram_hash_kernel(
    const int64_t* __restrict__ token_map, int64_t vocab, const int64_t* __restrict__ mult,
    const int64_t* __restrict__ primes, const int64_t* __restrict__ offsets, int n_layers, int ng,
    int n_heads, int64_t pad_id, int64_t* cache, const int32_t* __restrict__ ids, int seqlen,
    int64_t start_pos, int64_t* __restrict__ out, int32_t* err_flag) {
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= seqlen * n_layers) return;
  const int s = tid / n_layers;
  const int l = tid - s * n_layers;
  const int64_t pos = start_pos + s;
  const int cols = (ng - 1) * n_heads;
  bool ok = true;
  int64_t tok[kMaxNgram];
  const int64_t own = hash_window(token_map, vocab, ng, pad_id, cache, ids, start_pos, pos, tok, ok);
  if (l == 0) cache[pos] = own;
  int64_t* o = out + ((int64_t)l * seqlen + s) * cols;
  ok = hash_cols(tok, mult, primes, offsets, l, ng, n_heads, ok, 0, cols, o);
  if (!ok && err_flag != nullptr) *err_flag = 1;
}

// One decode token, one hashed layer, in one workgroup: the layer's row ids
// (thread c computes column c with hash_window and hash_cols, as the hash
// kernel would for that position and layer; thread 0 also stores the
// position's compressed id into the cache), then the gather, dequantisation
// and q8_1 of those rows viewed as one row, as dequant_rows_q8_1_kernel does
// (8 values per thread and pass). cols <= 32 (rows of up to 8192 values).
__global__ __launch_bounds__(256) void engram_rows_q8_1_kernel(
    const int64_t* __restrict__ token_map, int64_t vocab, const int64_t* __restrict__ mult,
    const int64_t* __restrict__ primes, const int64_t* __restrict__ offsets, int layer, int ng,
    int n_heads, int64_t pad_id, int64_t* cache, const int32_t* __restrict__ token, int64_t pos,
    const uint8_t* __restrict__ table, int64_t n_table_rows, int64_t* __restrict__ ids_out,
    uint16_t* __restrict__ rows_out, uint8_t* __restrict__ xq, int32_t* err_flag) {
  __shared__ int64_t rid[32];
  const int cols = (ng - 1) * n_heads;
  const int tid = threadIdx.x;
  if (tid < cols) {
    bool ok = true;
    int64_t tok[kMaxNgram];
    const int64_t own = hash_window(token_map, vocab, ng, pad_id, cache, token, pos, pos, tok, ok);
    if (tid == 0) cache[pos] = own;
    int64_t v;
    ok = hash_cols(tok, mult, primes, offsets, layer, ng, n_heads, ok, tid, tid + 1, &v);
    rid[tid] = v;
    if (ids_out != nullptr) ids_out[tid] = v;
    if (!ok && err_flag != nullptr) *err_flag = 1;
  }
  __syncthreads();
  const int k = cols * kBlockWeights;
  for (int c0 = 0; c0 < k / 8; c0 += 256) {
    const int chunk = c0 + tid;
    const bool active = chunk < k / 8;
    const int e0 = active ? chunk * 8 : 0;
    const int row = e0 / kBlockWeights, e = e0 % kBlockWeights;
    const int64_t id = rid[row];
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
    if (active && rows_out != nullptr) {
      u32x4 packed;
#pragma unroll
      for (int i = 0; i < 4; ++i) packed[i] = bits[2 * i] | (bits[2 * i + 1] << 16);
      *reinterpret_cast<u32x4*>(rows_out + e0) = packed;
    }
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = bf16_bits_to_f32(bits[i]);
    q8_1_store8(v, xq, e0, k, active);
  }
}

hipError_t launch_engram_rows_q8_1(const int64_t* token_map, int64_t vocab, const int64_t* mult,
                                   const int64_t* primes, const int64_t* offsets, int layer, int ng,
                                   int n_heads, int64_t pad_id, int64_t* cache, const int32_t* token,
                                   int64_t pos, const void* table, int64_t n_table_rows,
                                   int64_t* ids_out, void* rows_out, void* xq, int32_t* err_flag,
                                   hipStream_t stream) {
  hipLaunchKernelGGL(engram_rows_q8_1_kernel, dim3(1), dim3(256), 0, stream, token_map, vocab, mult,
                     primes, offsets, layer, ng, n_heads, pad_id, cache, token, pos,
                     static_cast<const uint8_t*>(table), n_table_rows, ids_out,
                     static_cast<uint16_t*>(rows_out), static_cast<uint8_t*>(xq), err_flag);
  return hipGetLastError();
}

hipError_t launch_engram_hash(const int64_t* token_map, int64_t vocab, const int64_t* mult,
                              const int64_t* primes, const int64_t* offsets, int n_layers, int ng,
                              int n_heads, int64_t pad_id, int64_t* cache, const int32_t* ids,
                              int seqlen, int64_t start_pos, int64_t* out, int32_t* err_flag,
                              hipStream_t stream) {
  const int64_t threads = (int64_t)seqlen * n_layers;
  hipLaunchKernelGGL(engram_hash_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                     token_map, vocab, mult, primes, offsets, n_layers, ng, n_heads, pad_id, cache,
                     ids, seqlen, start_pos, out, err_flag);
  return hipGetLastError();
}

hipError_t launch_dequant_rows(const void* table, int64_t n_table_rows, const int64_t* ids,
                               int n_rows, void* out, int32_t* err_flag, hipStream_t stream) {
  const unsigned blocks = (unsigned)((n_rows + 3) / 4);
  hipLaunchKernelGGL(dequant_rows_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(table), n_table_rows, ids, n_rows,
                     static_cast<uint16_t*>(out), err_flag);
  return hipGetLastError();
}

hipError_t launch_engram_gate(float* h, const float* kv, const float* qk, int t, int hc, int dim,
                              float eps, hipStream_t stream) {
  const dim3 grid((unsigned)t, (unsigned)hc);
  const bool a16 = ((reinterpret_cast<uintptr_t>(h) | reinterpret_cast<uintptr_t>(kv) |
                     reinterpret_cast<uintptr_t>(qk)) & 15u) == 0;
  if (a16 && dim % 4 == 0 && dim <= 16384) {
    const int nv4 = (dim / 4 + 255) / 256;
#define Q2K_GATE_VEC(N) \
  hipLaunchKernelGGL(engram_gate_vec_kernel<N>, grid, dim3(256), 0, stream, h, kv, qk, hc, dim, eps)
    if (nv4 <= 1) Q2K_GATE_VEC(1);
    else if (nv4 <= 2) Q2K_GATE_VEC(2);
    else if (nv4 <= 4) Q2K_GATE_VEC(4);
    else if (nv4 <= 8) Q2K_GATE_VEC(8);
    else Q2K_GATE_VEC(16);
#undef Q2K_GATE_VEC
  } else {
    hipLaunchKernelGGL(engram_gate_kernel, grid, dim3(256), 0, stream, h, kv, qk, hc, dim, eps);
  }
  return hipGetLastError();
}

}  // namespace q2k
