// Internal launchers behind the C ABI. Arguments are validated by the ABI
// layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q2k {

// Up to this many matrices in one plain (non-expert) product launch.
constexpr int kMaxPlainJobs = 4;
// Tokens one packed-dot launch takes (the q2k_mmvq limit); q2k_mmq goes past it.
constexpr int kMaxM = 8;
// q2k_mmq from this many tokens runs the tile kernel (launch_mmq, its own
// summation order); up to 16 tokens it runs the q2k_mmvq kernels on groups
// of 8 (their order), which keep more waves busy on so few tokens.
constexpr int kMmqTileMinM = 17;
constexpr int kMaxExpertBases = 4;

// One decode token's engram rows as the input of a product: the token's
// hashed row ids of one hashed layer, the gathered table rows, dequantised
// and quantised to one q8_1 row (engram_rows_q8_1 in the product's
// prologue).
struct EngramRows {
  const int64_t* token_map = nullptr;
  int64_t vocab = 0;
  const int64_t* mult = nullptr;
  const int64_t* primes = nullptr;
  const int64_t* offsets = nullptr;
  int32_t layer = 0;
  int32_t ng = 0;
  int32_t n_heads = 0;
  int64_t pad_id = 0;
  int64_t* cache = nullptr;
  const int32_t* token = nullptr;
  int64_t pos = 0;
  const uint8_t* table = nullptr;
  int64_t n_table_rows = 0;
  int32_t* err_flag = nullptr;
};

struct MmvqLaunch {
  // Plain mode (ids == nullptr, groups == 0): job j multiplies w[j] [n[j], k]
  // by xq.
  // Expert mode (ids != nullptr): job base*n_ids + i multiplies the matrix
  // w[base] + ids[i] * expert_stride by xq (shared) or by the i-th group of
  // m rows of xq (x_per_id), writing y[0] + (base*n_ids + i) * m * n[0].
  // Grouped mode (groups > 0): job g multiplies rows g*n[0] .. g*n[0]+n[0]-1
  // of w[0] (expert_stride = n[0] row bytes apart) by elements g*k .. g*k+k-1
  // of each q8_1 row of width groups*k, writing y[0][t, g*n[0] + r] (output
  // rows groups*n[0] apart); n_ids == groups, njobs == 1.
  const void* w[kMaxPlainJobs];
  float* y[kMaxPlainJobs];
  int32_t n[kMaxPlainJobs];
  int32_t njobs;
  const void* xq;
  const int32_t* ids;
  int32_t n_ids;
  int32_t n_experts;
  int32_t x_per_id;
  int64_t expert_stride;
  int32_t* err_flag;
  int32_t* dots;   // non-null: write the int32 (I, M) block sums instead of y (plain, one job)
  int32_t groups;  // grouped mode when > 0
  int32_t k;
  int32_t m;
  // Non-null: bf16 rows [m, k] (row stride x_stride elements) that the
  // launch quantises into xq itself before the product (plain mode): in the
  // product kernel when it can (one matrix, one token, run kernel), else by
  // a q8_1 launch ahead of it.
  const void* x_bf16 = nullptr;
  int64_t x_stride = 0;
  // Non-null (expert mode, x_per_id): f32 gate and up rows [n_ids * m, k];
  // the launch forms xq = q8_1(bf16 SwiGLU) of them before the product, in
  // the product kernel when it can, else by a SwiGLU launch ahead of it.
  const float* sg = nullptr;
  const float* su = nullptr;
  // Non-null (plain mode, one matrix, m = 1): the input row is this decode
  // token's engram rows; xq receives their q8_1 row. In the product kernel
  // when it can (run kernel), else by an engram_rows_q8_1 launch ahead of it.
  const EngramRows* eg = nullptr;
  // Non-null (expert mode with two bases, gate and up, x_bf16 shared, one
  // token): after the product, sw_hq receives the q8_1 rows [n_ids, n] of
  // h = bf16 SwiGLU(gate rows, up rows) and sw_h (nullable) h itself; in the
  // product kernel's epilogue when it can, else by a SwiGLU launch after it.
  void* sw_hq = nullptr;
  void* sw_h = nullptr;
};

// Expert and grouped launches are n_jobs equal-sized jobs.
inline bool uniform_jobs(const MmvqLaunch& a) { return a.ids != nullptr || a.groups > 0; }

hipError_t launch_q8_1_rows(const void* x, int64_t stride, void* xq, int m, int k,
                            hipStream_t stream);
hipError_t launch_swiglu_q8_1_rows(const float* g, const float* u, void* h, void* hq, int rows,
                                   int k, hipStream_t stream);
hipError_t launch_mmvq(const MmvqLaunch& a, hipStream_t stream);
// Product kernel choice (0 automatic, 1 matrix cores, 2 packed dots); returns
// the previous one.
int set_product_kernel(int choice);
// True when launch_mmvq runs this launch (product or integer stage) on the
// matrix-core kernel under the current choice.
bool takes_mfma(const MmvqLaunch& a);
// 2..8 tokens on the matrix cores, rows of 4, 8, 16 or 28 super-blocks.
hipError_t launch_mmvq_mfma(const MmvqLaunch& a, hipStream_t stream);
bool mfma_supports(int k);
// True when the matrix-core kernel is the faster choice for this launch.
bool mfma_preferred(const MmvqLaunch& a);
// More than 8 tokens on the matrix cores (q2k_mmq; its own summation order:
// the leaves of each half added in row order). With dots non-null the
// launch writes the int32 (I, M) block sums instead of y.
hipError_t launch_mmq(const void* w, const void* xq, float* y, int32_t* dots, int n, int k, int m,
                      hipStream_t stream);
// Q2_K x bf16 activations (exact expansion, fp64 sums), m = 1..8.
hipError_t launch_gemv_bf16(const void* w, const void* x, int64_t x_stride, float* y, int n, int k,
                            int m, hipStream_t stream);
hipError_t launch_dequant_rows(const void* table, int64_t n_table_rows, const int64_t* ids,
                               int n_rows, void* out, int32_t* err_flag, hipStream_t stream);
// Gathered rows -> optional bf16 copy -> one q8_1 row of width 256 * n_rows.
hipError_t launch_dequant_rows_q8_1(const void* table, int64_t n_table_rows, const int64_t* ids,
                                    int n_rows, void* out, void* xq, int32_t* err_flag,
                                    hipStream_t stream);
hipError_t launch_engram_gate(float* h, const float* kv, const float* qk, int t, int hc, int dim,
                              float eps, hipStream_t stream);
// One decode token: hashed layer `layer`'s row ids, then their gather,
// dequantisation and q8_1 as one row (one workgroup).
hipError_t launch_engram_rows_q8_1(const int64_t* token_map, int64_t vocab, const int64_t* mult,
                                   const int64_t* primes, const int64_t* offsets, int layer, int ng,
                                   int n_heads, int64_t pad_id, int64_t* cache, const int32_t* token,
                                   int64_t pos, const void* table, int64_t n_table_rows,
                                   int64_t* ids_out, void* rows_out, void* xq, int32_t* err_flag,
                                   hipStream_t stream);
hipError_t launch_engram_hash(const int64_t* token_map, int64_t vocab, const int64_t* mult,
                              const int64_t* primes, const int64_t* offsets, int n_layers, int ng,
                              int n_heads, int64_t pad_id, int64_t* cache, const int32_t* ids,
                              int seqlen, int64_t start_pos, int64_t* out, int32_t* err_flag,
                              hipStream_t stream);

}  // namespace q2k
