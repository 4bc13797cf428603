// extern "C" entry points of libq2kdecode.so (declared in q2k_decode.h).
//
// Every argument check runs here, on the host, before any HIP call (the
// pages refuse bad shapes "before any launch": engram_v41/apply.rs module
// invariants, moe_v41/init.rs MoeV41::new, attn_v41/decode.rs m <= 8), and
// in release builds too. Kernels are only enqueued on the caller's stream.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>
#include <stdint.h>

#include <mutex>

#include "../../include/q2k_decode.h"
#include "q2k_device.h"
#include "q2k_launch.h"

namespace {

thread_local char g_err[512] = "";

int32_t fail(int32_t code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int32_t launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(Q2K_ELAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return Q2K_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// [a, a + na) and [b, b + nb) overlap
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na > 0 && nb > 0 && x < y + nb && y < x + na;
}

// The engram step's kv rows in its workspace, rounded to 256 bytes; the
// q8_1 row of the gathered rows follows them.
size_t engram_kv_bytes(int32_t hc, int32_t dim) {
  return ((size_t)(hc + 1) * (size_t)dim * 4 + 255) / 256 * 256;
}

size_t q2k_matrix_bytes(int64_t n, int64_t k) { return (size_t)n * (size_t)(k / 256) * 84; }

int32_t check_k(const char* fn, int32_t k) {
  if (k <= 0 || k % 256 != 0)
    return fail(Q2K_ESHAPE, "%s: k = %d is not a positive multiple of 256 (Q2_K super-blocks)", fn, k);
  return Q2K_OK;
}

int32_t check_m(const char* fn, int32_t m) {
  if (m < 1 || m > Q2K_MAX_M)
    return fail(Q2K_ESHAPE, "%s: m = %d outside 1..%d", fn, m, Q2K_MAX_M);
  return Q2K_OK;
}

}  // namespace

extern "C" {

int32_t q2k_abi_version(void) { return Q2K_ABI_VERSION; }

const char* q2k_last_error(void) { return g_err; }

int32_t q2k_set_product_kernel(int32_t choice) {
  if (choice != Q2K_KERNEL_AUTO && choice != Q2K_KERNEL_MATRIX_CORES &&
      choice != Q2K_KERNEL_PACKED_DOTS)
    return fail(Q2K_EINVAL, "q2k_set_product_kernel: unknown choice %d", choice);
  return q2k::set_product_kernel(choice);
}

size_t q8_1_rows_bytes(int32_t m, int32_t k) {
  if (m < 1 || k <= 0 || k % 256 != 0) return 0;
  return (size_t)m * q2k::q8_row_bytes(k);
}

int32_t q8_1_rows(const void* x_bf16_dev, int64_t x_row_stride, void* xq_dev, size_t xq_bytes,
                  int32_t m, int32_t k, void* stream) {
  const char* fn = "q8_1_rows";
  if (!x_bf16_dev || !xq_dev) return fail(Q2K_EINVAL, "%s: null pointer", fn);
  if (m < 1) return fail(Q2K_ESHAPE, "%s: m = %d < 1", fn, m);
  if (int32_t r = check_k(fn, k)) return r;
  if (x_row_stride < k) return fail(Q2K_ESHAPE, "%s: row stride %lld < k = %d", fn, (long long)x_row_stride, k);
  if (!aligned(x_bf16_dev, 16) || x_row_stride % 8 != 0)
    return fail(Q2K_EALIGN, "%s: x must be 16-byte aligned with a row stride that is a multiple of 8", fn);
  if (!aligned(xq_dev, 16)) return fail(Q2K_EALIGN, "%s: xq must be 16-byte aligned", fn);
  const size_t need = q8_1_rows_bytes(m, k);
  if (xq_bytes < need) return fail(Q2K_ESPACE, "%s: xq holds %zu bytes, %zu needed", fn, xq_bytes, need);
  const size_t xbytes = ((size_t)(m - 1) * x_row_stride + k) * 2;
  if (overlap(x_bf16_dev, xbytes, xq_dev, need)) return fail(Q2K_EINVAL, "%s: x and xq overlap", fn);
  return launched(q2k::launch_q8_1_rows(x_bf16_dev, x_row_stride, xq_dev, m, k, (hipStream_t)stream), fn);
}

static int32_t check_matrix(const char* fn, const char* name, const void* w, int32_t n) {
  if (!w) return fail(Q2K_EINVAL, "%s: %s is null", fn, name);
  if (n < 1) return fail(Q2K_ESHAPE, "%s: %s has n = %d rows", fn, name, n);
  if (!aligned(w, 4)) return fail(Q2K_EALIGN, "%s: %s must be 4-byte aligned", fn, name);
  return Q2K_OK;
}

static int32_t check_out(const char* fn, const char* name, const void* y) {
  if (!y) return fail(Q2K_EINVAL, "%s: %s is null", fn, name);
  if (!aligned(y, 4)) return fail(Q2K_EALIGN, "%s: %s must be 4-byte aligned", fn, name);
  return Q2K_OK;
}

int32_t q2k_mmvq(const void* w_dev, const void* xq_dev, float* y_dev, int32_t n, int32_t k,
                 int32_t m, void* stream) {
  const char* fn = "q2k_mmvq";
  if (int32_t r = check_matrix(fn, "w", w_dev, n)) return r;
  if (int32_t r = check_out(fn, "y", y_dev)) return r;
  if (!xq_dev) return fail(Q2K_EINVAL, "%s: xq is null", fn);
  if (int32_t r = check_k(fn, k)) return r;
  if (int32_t r = check_m(fn, m)) return r;
  if (!aligned(xq_dev, 16)) return fail(Q2K_EALIGN, "%s: xq must be 16-byte aligned", fn);
  const size_t ybytes = (size_t)m * n * 4;
  if (overlap(y_dev, ybytes, w_dev, q2k_matrix_bytes(n, k)) ||
      overlap(y_dev, ybytes, xq_dev, q8_1_rows_bytes(m, k)))
    return fail(Q2K_EINVAL, "%s: y overlaps an input", fn);
  q2k::MmvqLaunch a{};
  a.w[0] = w_dev;
  a.y[0] = y_dev;
  a.n[0] = n;
  a.njobs = 1;
  a.xq = xq_dev;
  a.k = k;
  a.m = m;
  return launched(q2k::launch_mmvq(a, (hipStream_t)stream), fn);
}

int32_t q8_1_q2k_mmvq(const void* w_dev, const void* x_bf16_dev, int64_t x_row_stride, void* xq_dev,
                      size_t xq_bytes, float* y_dev, int32_t n, int32_t k, int32_t m, void* stream) {
  const char* fn = "q8_1_q2k_mmvq";
  if (int32_t r = check_matrix(fn, "w", w_dev, n)) return r;
  if (int32_t r = check_out(fn, "y", y_dev)) return r;
  if (!x_bf16_dev || !xq_dev) return fail(Q2K_EINVAL, "%s: null pointer", fn);
  if (int32_t r = check_k(fn, k)) return r;
  if (int32_t r = check_m(fn, m)) return r;
  if (x_row_stride < k) return fail(Q2K_ESHAPE, "%s: row stride %lld < k = %d", fn, (long long)x_row_stride, k);
  if (!aligned(x_bf16_dev, 16) || x_row_stride % 8 != 0)
    return fail(Q2K_EALIGN, "%s: x must be 16-byte aligned with a row stride that is a multiple of 8", fn);
  if (!aligned(xq_dev, 16)) return fail(Q2K_EALIGN, "%s: xq must be 16-byte aligned", fn);
  const size_t need = q8_1_rows_bytes(m, k);
  if (xq_bytes < need) return fail(Q2K_ESPACE, "%s: xq holds %zu bytes, %zu needed", fn, xq_bytes, need);
  const size_t xbytes = ((size_t)(m - 1) * x_row_stride + k) * 2;
  const size_t ybytes = (size_t)m * n * 4;
  const size_t wbytes = q2k_matrix_bytes(n, k);
  if (overlap(x_bf16_dev, xbytes, xq_dev, need) || overlap(xq_dev, need, w_dev, wbytes))
    return fail(Q2K_EINVAL, "%s: xq overlaps an input", fn);
  if (overlap(y_dev, ybytes, w_dev, wbytes) || overlap(y_dev, ybytes, x_bf16_dev, xbytes) ||
      overlap(y_dev, ybytes, xq_dev, need))
    return fail(Q2K_EINVAL, "%s: y overlaps an input or xq", fn);
  q2k::MmvqLaunch a{};
  a.w[0] = w_dev;
  a.y[0] = y_dev;
  a.n[0] = n;
  a.njobs = 1;
  a.xq = xq_dev;
  a.k = k;
  a.m = m;
  a.x_bf16 = x_bf16_dev;
  a.x_stride = x_row_stride;
  return launched(q2k::launch_mmvq(a, (hipStream_t)stream), fn);
}

int32_t q2k_mmq(const void* w_dev, const void* xq_dev, float* y_dev, int32_t n, int32_t k, int32_t m,
                void* stream) {
  const char* fn = "q2k_mmq";
  if (int32_t r = check_matrix(fn, "w", w_dev, n)) return r;
  if (int32_t r = check_out(fn, "y", y_dev)) return r;
  if (!xq_dev) return fail(Q2K_EINVAL, "%s: xq is null", fn);
  if (int32_t r = check_k(fn, k)) return r;
  if (m < 1 || m > Q2K_MMQ_MAX_M) return fail(Q2K_ESHAPE, "%s: m = %d outside 1..%d", fn, m, Q2K_MMQ_MAX_M);
  if (!aligned(xq_dev, 16)) return fail(Q2K_EALIGN, "%s: xq must be 16-byte aligned", fn);
  if ((int64_t)m * n > (int64_t)1 << 31) return fail(Q2K_ESHAPE, "%s: output larger than 2^31 values", fn);
  const size_t ybytes = (size_t)m * n * 4;
  if (overlap(y_dev, ybytes, w_dev, q2k_matrix_bytes(n, k)) ||
      overlap(y_dev, ybytes, xq_dev, (size_t)m * q2k::q8_row_bytes(k)))
    return fail(Q2K_EINVAL, "%s: y overlaps an input", fn);
  if (m >= q2k::kMmqTileMinM)
    return launched(q2k::launch_mmq(w_dev, xq_dev, y_dev, nullptr, n, k, m, (hipStream_t)stream), fn);
  q2k::MmvqLaunch a{};
  a.w[0] = w_dev;
  a.y[0] = y_dev;
  a.n[0] = n;
  a.njobs = 1;
  a.xq = xq_dev;
  a.k = k;
  a.m = m;
  return launched(q2k::launch_mmvq(a, (hipStream_t)stream), fn);
}

// Checks of the pair forms and their launch description.
static int32_t pair_launch(const char* fn, const void* wa_dev, float* ya_dev, int32_t na,
                           const void* wb_dev, float* yb_dev, int32_t nb, const void* xq_dev,
                           int32_t k, int32_t m, q2k::MmvqLaunch* out) {
  if (int32_t r = check_matrix(fn, "wa", wa_dev, na)) return r;
  if (int32_t r = check_matrix(fn, "wb", wb_dev, nb)) return r;
  if (int32_t r = check_out(fn, "ya", ya_dev)) return r;
  if (int32_t r = check_out(fn, "yb", yb_dev)) return r;
  if (!xq_dev) return fail(Q2K_EINVAL, "%s: xq is null", fn);
  if (int32_t r = check_k(fn, k)) return r;
  if (int32_t r = check_m(fn, m)) return r;
  if (!aligned(xq_dev, 16)) return fail(Q2K_EALIGN, "%s: xq must be 16-byte aligned", fn);
  const size_t ya_bytes = (size_t)m * na * 4, yb_bytes = (size_t)m * nb * 4;
  if (overlap(ya_dev, ya_bytes, yb_dev, yb_bytes)) return fail(Q2K_EINVAL, "%s: ya and yb overlap", fn);
  const size_t xqb = q8_1_rows_bytes(m, k);
  if (overlap(ya_dev, ya_bytes, wa_dev, q2k_matrix_bytes(na, k)) ||
      overlap(ya_dev, ya_bytes, wb_dev, q2k_matrix_bytes(nb, k)) ||
      overlap(yb_dev, yb_bytes, wa_dev, q2k_matrix_bytes(na, k)) ||
      overlap(yb_dev, yb_bytes, wb_dev, q2k_matrix_bytes(nb, k)) ||
      overlap(ya_dev, ya_bytes, xq_dev, xqb) || overlap(yb_dev, yb_bytes, xq_dev, xqb))
    return fail(Q2K_EINVAL, "%s: an output overlaps an input", fn);
  q2k::MmvqLaunch a{};
  a.w[0] = wa_dev;
  a.y[0] = ya_dev;
  a.n[0] = na;
  a.w[1] = wb_dev;
  a.y[1] = yb_dev;
  a.n[1] = nb;
  a.njobs = 2;
  a.xq = xq_dev;
  a.k = k;
  a.m = m;
  *out = a;
  return Q2K_OK;
}

int32_t q2k_mmvq_pair(const void* wa_dev, float* ya_dev, int32_t na, const void* wb_dev,
                      float* yb_dev, int32_t nb, const void* xq_dev, int32_t k, int32_t m,
                      void* stream) {
  const char* fn = "q2k_mmvq_pair";
  q2k::MmvqLaunch a;
  if (int32_t r = pair_launch(fn, wa_dev, ya_dev, na, wb_dev, yb_dev, nb, xq_dev, k, m, &a)) return r;
  return launched(q2k::launch_mmvq(a, (hipStream_t)stream), fn);
}

int32_t q8_1_q2k_mmvq_pair(const void* wa_dev, float* ya_dev, int32_t na, const void* wb_dev,
                           float* yb_dev, int32_t nb, const void* x_bf16_dev, int64_t x_row_stride,
                           void* xq_dev, size_t xq_bytes, int32_t k, int32_t m, void* stream) {
  const char* fn = "q8_1_q2k_mmvq_pair";
  q2k::MmvqLaunch a;
  if (int32_t r = pair_launch(fn, wa_dev, ya_dev, na, wb_dev, yb_dev, nb, xq_dev, k, m, &a)) return r;
  if (!x_bf16_dev) return fail(Q2K_EINVAL, "%s: x is null", fn);
  if (x_row_stride < k) return fail(Q2K_ESHAPE, "%s: row stride %lld < k = %d", fn, (long long)x_row_stride, k);
  if (!aligned(x_bf16_dev, 16) || x_row_stride % 8 != 0)
    return fail(Q2K_EALIGN, "%s: x must be 16-byte aligned with a row stride that is a multiple of 8", fn);
  const size_t need = q8_1_rows_bytes(m, k);
  if (xq_bytes < need) return fail(Q2K_ESPACE, "%s: xq holds %zu bytes, %zu needed", fn, xq_bytes, need);
  const size_t xbytes = ((size_t)(m - 1) * x_row_stride + k) * 2;
  if (overlap(x_bf16_dev, xbytes, xq_dev, need) ||
      overlap(xq_dev, need, wa_dev, q2k_matrix_bytes(na, k)) ||
      overlap(xq_dev, need, wb_dev, q2k_matrix_bytes(nb, k)))
    return fail(Q2K_EINVAL, "%s: xq overlaps an input", fn);
  if (overlap(ya_dev, (size_t)m * na * 4, x_bf16_dev, xbytes) ||
      overlap(yb_dev, (size_t)m * nb * 4, x_bf16_dev, xbytes))
    return fail(Q2K_EINVAL, "%s: an output overlaps x", fn);
  a.x_bf16 = x_bf16_dev;
  a.x_stride = x_row_stride;
  return launched(q2k::launch_mmvq(a, (hipStream_t)stream), fn);
}

// Checks of the expert-batch forms and their launch description (xq is the
// q8_1 input as the product reads it).
static int32_t experts_launch(const char* fn, const void* const* bases, int32_t n_bases,
                              int64_t expert_stride_bytes, int32_t n_experts, const int32_t* ids_dev,
                              int32_t n_ids, const void* xq_dev, int32_t x_per_id, float* y_dev,
                              int32_t n, int32_t k, int32_t m, int32_t* err_flag_dev,
                              q2k::MmvqLaunch* a) {
  if (!bases) return fail(Q2K_EINVAL, "%s: bases is null", fn);
  if (n_bases < 1 || n_bases > q2k::kMaxExpertBases)
    return fail(Q2K_ESHAPE, "%s: n_bases = %d outside 1..%d", fn, n_bases, q2k::kMaxExpertBases);
  for (int i = 0; i < n_bases; ++i)
    if (int32_t r = check_matrix(fn, "bases[i]", bases[i], n)) return r;
  if (!ids_dev || !xq_dev) return fail(Q2K_EINVAL, "%s: null pointer", fn);
  if (int32_t r = check_out(fn, "y", y_dev)) return r;
  if (int32_t r = check_k(fn, k)) return r;
  if (int32_t r = check_m(fn, m)) return r;
  if (n_experts < 1) return fail(Q2K_ESHAPE, "%s: n_experts = %d < 1", fn, n_experts);
  if (n_ids < 1 || n_ids > 64) return fail(Q2K_ESHAPE, "%s: n_ids = %d outside 1..64", fn, n_ids);
  if (x_per_id != 0 && x_per_id != 1) return fail(Q2K_ESHAPE, "%s: x_per_id = %d", fn, x_per_id);
  const size_t mat = q2k_matrix_bytes(n, k);
  if (expert_stride_bytes < (int64_t)mat)
    return fail(Q2K_ESHAPE, "%s: expert stride %lld < matrix size %zu", fn, (long long)expert_stride_bytes, mat);
  if (expert_stride_bytes % 4 != 0) return fail(Q2K_EALIGN, "%s: expert stride must be a multiple of 4", fn);
  if (!aligned(xq_dev, 16)) return fail(Q2K_EALIGN, "%s: xq must be 16-byte aligned", fn);
  if (!aligned(ids_dev, 4)) return fail(Q2K_EALIGN, "%s: ids must be 4-byte aligned", fn);
  if ((int64_t)n_bases * n_ids * m * (int64_t)n > (int64_t)1 << 31)
    return fail(Q2K_ESHAPE, "%s: output larger than 2^31 values", fn);
  const size_t ybytes = (size_t)n_bases * n_ids * m * n * 4;
  const size_t set_bytes = (size_t)expert_stride_bytes * (size_t)(n_experts - 1) + mat;
  for (int i = 0; i < n_bases; ++i)
    if (overlap(y_dev, ybytes, bases[i], set_bytes)) return fail(Q2K_EINVAL, "%s: y overlaps a base", fn);
  if (overlap(y_dev, ybytes, xq_dev, q8_1_rows_bytes(x_per_id ? n_ids * m : m, k)))
    return fail(Q2K_EINVAL, "%s: y overlaps xq", fn);
  *a = q2k::MmvqLaunch{};
  for (int i = 0; i < n_bases; ++i) a->w[i] = bases[i];
  a->y[0] = y_dev;
  a->n[0] = n;
  a->njobs = n_bases;
  a->xq = xq_dev;
  a->ids = ids_dev;
  a->n_ids = n_ids;
  a->n_experts = n_experts;
  a->x_per_id = x_per_id;
  a->expert_stride = expert_stride_bytes;
  a->err_flag = err_flag_dev;
  a->k = k;
  a->m = m;
  return Q2K_OK;
}

int32_t q2k_mmvq_experts(const void* const* bases, int32_t n_bases, int64_t expert_stride_bytes,
                         int32_t n_experts, const int32_t* ids_dev, int32_t n_ids,
                         const void* xq_dev, int32_t x_per_id, float* y_dev, int32_t n, int32_t k,
                         int32_t m, int32_t* err_flag_dev, void* stream) {
  const char* fn = "q2k_mmvq_experts";
  q2k::MmvqLaunch a;
  if (int32_t r = experts_launch(fn, bases, n_bases, expert_stride_bytes, n_experts, ids_dev, n_ids,
                                 xq_dev, x_per_id, y_dev, n, k, m, err_flag_dev, &a))
    return r;
  return launched(q2k::launch_mmvq(a, (hipStream_t)stream), fn);
}

int32_t q8_1_q2k_mmvq_experts(const void* const* bases, int32_t n_bases, int64_t expert_stride_bytes,
                              int32_t n_experts, const int32_t* ids_dev, int32_t n_ids,
                              const void* x_bf16_dev, int64_t x_row_stride, void* xq_dev,
                              size_t xq_bytes, float* y_dev, int32_t n, int32_t k, int32_t m,
                              int32_t* err_flag_dev, void* stream) {
  const char* fn = "q8_1_q2k_mmvq_experts";
  q2k::MmvqLaunch a;
  if (int32_t r = experts_launch(fn, bases, n_bases, expert_stride_bytes, n_experts, ids_dev, n_ids,
                                 xq_dev, 0, y_dev, n, k, m, err_flag_dev, &a))
    return r;
  if (!x_bf16_dev) return fail(Q2K_EINVAL, "%s: x is null", fn);
  if (x_row_stride < k) return fail(Q2K_ESHAPE, "%s: row stride %lld < k = %d", fn, (long long)x_row_stride, k);
  if (!aligned(x_bf16_dev, 16) || x_row_stride % 8 != 0)
    return fail(Q2K_EALIGN, "%s: x must be 16-byte aligned with a row stride that is a multiple of 8", fn);
  const size_t need = q8_1_rows_bytes(m, k);
  if (xq_bytes < need) return fail(Q2K_ESPACE, "%s: xq holds %zu bytes, %zu needed", fn, xq_bytes, need);
  const size_t xbytes = ((size_t)(m - 1) * x_row_stride + k) * 2;
  const size_t ybytes = (size_t)n_bases * n_ids * m * n * 4;
  const size_t set_bytes = (size_t)expert_stride_bytes * (size_t)(n_experts - 1) + q2k_matrix_bytes(n, k);
  if (overlap(x_bf16_dev, xbytes, xq_dev, need) || overlap(y_dev, ybytes, x_bf16_dev, xbytes))
    return fail(Q2K_EINVAL, "%s: x overlaps xq or y", fn);
  for (int i = 0; i < n_bases; ++i)
    if (overlap(xq_dev, need, bases[i], set_bytes)) return fail(Q2K_EINVAL, "%s: xq overlaps a base", fn);
  if (overlap(xq_dev, need, ids_dev, (size_t)n_ids * 4))
    return fail(Q2K_EINVAL, "%s: xq overlaps ids", fn);
  a.x_bf16 = x_bf16_dev;
  a.x_stride = x_row_stride;
  return launched(q2k::launch_mmvq(a, (hipStream_t)stream), fn);
}

int32_t q8_1_q2k_mmvq_experts_swiglu(const void* const* bases, int64_t expert_stride_bytes,
                                     int32_t n_experts, const int32_t* ids_dev, int32_t n_ids,
                                     const void* x_bf16_dev, void* xq_dev, size_t xq_bytes,
                                     float* y_dev, void* h_bf16_dev, void* hq_dev, size_t hq_bytes,
                                     int32_t n, int32_t k, int32_t* err_flag_dev, void* stream) {
  const char* fn = "q8_1_q2k_mmvq_experts_swiglu";
  q2k::MmvqLaunch a;
  if (int32_t r = experts_launch(fn, bases, 2, expert_stride_bytes, n_experts, ids_dev, n_ids,
                                 xq_dev, 0, y_dev, n, k, 1, err_flag_dev, &a))
    return r;
  if (n % 256 != 0)
    return fail(Q2K_ESHAPE, "%s: n = %d is not a multiple of 256 (h is the down product's input)", fn, n);
  if (!x_bf16_dev || !hq_dev) return fail(Q2K_EINVAL, "%s: x or hq is null", fn);
  if (!aligned(x_bf16_dev, 16) || !aligned(hq_dev, 16) || (h_bf16_dev && !aligned(h_bf16_dev, 16)))
    return fail(Q2K_EALIGN, "%s: x, h and hq must be 16-byte aligned", fn);
  const size_t need = q8_1_rows_bytes(1, k);
  if (xq_bytes < need) return fail(Q2K_ESPACE, "%s: xq holds %zu bytes, %zu needed", fn, xq_bytes, need);
  const size_t hneed = q8_1_rows_bytes(n_ids, n);
  if (hq_bytes < hneed) return fail(Q2K_ESPACE, "%s: hq holds %zu bytes, %zu needed", fn, hq_bytes, hneed);
  const size_t xbytes = (size_t)k * 2;
  const size_t ybytes = (size_t)2 * n_ids * n * 4;
  const size_t hbytes = (size_t)n_ids * n * 2;
  const size_t set_bytes = (size_t)expert_stride_bytes * (size_t)(n_experts - 1) + q2k_matrix_bytes(n, k);
  // every output against every other buffer of the call
  const struct { const void* p; size_t n; } out[3] = {{xq_dev, need}, {hq_dev, hneed}, {h_bf16_dev, hbytes}};
  const struct { const void* p; size_t n; } all[8] = {
      {x_bf16_dev, xbytes}, {ids_dev, (size_t)n_ids * 4}, {bases[0], set_bytes}, {bases[1], set_bytes},
      {y_dev, ybytes},      {xq_dev, need},               {hq_dev, hneed},       {h_bf16_dev, hbytes}};
  for (int i = 0; i < 3; ++i) {
    if (!out[i].p) continue;
    for (int j = 0; j < 8; ++j)   // all[5 + i] is out[i] itself
      if (j != 5 + i && all[j].p && overlap(out[i].p, out[i].n, all[j].p, all[j].n))
        return fail(Q2K_EINVAL, "%s: an output overlaps another buffer of the call", fn);
  }
  if (overlap(y_dev, ybytes, x_bf16_dev, xbytes)) return fail(Q2K_EINVAL, "%s: y overlaps x", fn);
  a.x_bf16 = x_bf16_dev;
  a.x_stride = k;
  a.sw_hq = hq_dev;
  a.sw_h = h_bf16_dev;
  return launched(q2k::launch_mmvq(a, (hipStream_t)stream), fn);
}

int32_t swiglu_q2k_mmvq_experts(const void* const* bases, int32_t n_bases, int64_t expert_stride_bytes,
                                int32_t n_experts, const int32_t* ids_dev, int32_t n_ids,
                                const float* g_dev, const float* u_dev, void* hq_dev,
                                size_t hq_bytes, float* y_dev, int32_t n, int32_t k,
                                int32_t* err_flag_dev, void* stream) {
  const char* fn = "swiglu_q2k_mmvq_experts";
  q2k::MmvqLaunch a;
  if (int32_t r = experts_launch(fn, bases, n_bases, expert_stride_bytes, n_experts, ids_dev, n_ids,
                                 hq_dev, 1, y_dev, n, k, 1, err_flag_dev, &a))
    return r;
  if (!g_dev || !u_dev) return fail(Q2K_EINVAL, "%s: g or u is null", fn);
  if (!aligned(g_dev, 16) || !aligned(u_dev, 16))
    return fail(Q2K_EALIGN, "%s: g and u must be 16-byte aligned", fn);
  const size_t need = q8_1_rows_bytes(n_ids, k);
  if (hq_bytes < need) return fail(Q2K_ESPACE, "%s: hq holds %zu bytes, %zu needed", fn, hq_bytes, need);
  const size_t gbytes = (size_t)n_ids * k * 4;
  const size_t ybytes = (size_t)n_bases * n_ids * n * 4;
  const size_t set_bytes = (size_t)expert_stride_bytes * (size_t)(n_experts - 1) + q2k_matrix_bytes(n, k);
  if (overlap(hq_dev, need, g_dev, gbytes) || overlap(hq_dev, need, u_dev, gbytes) ||
      overlap(hq_dev, need, ids_dev, (size_t)n_ids * 4))
    return fail(Q2K_EINVAL, "%s: hq overlaps g, u or ids", fn);
  for (int i = 0; i < n_bases; ++i)
    if (overlap(hq_dev, need, bases[i], set_bytes)) return fail(Q2K_EINVAL, "%s: hq overlaps a base", fn);
  if (overlap(y_dev, ybytes, g_dev, gbytes) || overlap(y_dev, ybytes, u_dev, gbytes))
    return fail(Q2K_EINVAL, "%s: y overlaps g or u", fn);
  a.sg = g_dev;
  a.su = u_dev;
  return launched(q2k::launch_mmvq(a, (hipStream_t)stream), fn);
}

int32_t q2k_mmvq_grouped(const void* w_dev, const void* xq_dev, float* y_dev, int32_t groups,
                         int32_t rows_per_group, int32_t k, int32_t m, void* stream) {
  const char* fn = "q2k_mmvq_grouped";
  if (groups < 1) return fail(Q2K_ESHAPE, "%s: groups = %d < 1", fn, groups);
  if (rows_per_group < 1) return fail(Q2K_ESHAPE, "%s: rows_per_group = %d < 1", fn, rows_per_group);
  if (int32_t r = check_k(fn, k)) return r;
  if (int32_t r = check_m(fn, m)) return r;
  const int64_t n_total = (int64_t)groups * rows_per_group;
  const int64_t k_total = (int64_t)groups * k;
  if (n_total > INT32_MAX || k_total > INT32_MAX)
    return fail(Q2K_ESHAPE, "%s: groups * rows_per_group or groups * k exceeds 2^31 - 1", fn);
  if ((int64_t)m * n_total > (int64_t)1 << 31) return fail(Q2K_ESHAPE, "%s: output larger than 2^31 values", fn);
  if (int32_t r = check_matrix(fn, "w", w_dev, (int32_t)n_total)) return r;
  if (int32_t r = check_out(fn, "y", y_dev)) return r;
  if (!xq_dev) return fail(Q2K_EINVAL, "%s: xq is null", fn);
  if (!aligned(xq_dev, 16)) return fail(Q2K_EALIGN, "%s: xq must be 16-byte aligned", fn);
  const size_t ybytes = (size_t)m * (size_t)n_total * 4;
  if (overlap(y_dev, ybytes, w_dev, q2k_matrix_bytes(n_total, k)) ||
      overlap(y_dev, ybytes, xq_dev, q8_1_rows_bytes(m, (int32_t)k_total)))
    return fail(Q2K_EINVAL, "%s: y overlaps an input", fn);
  q2k::MmvqLaunch a{};
  a.w[0] = w_dev;
  a.y[0] = y_dev;
  a.n[0] = rows_per_group;
  a.njobs = 1;
  a.xq = xq_dev;
  a.groups = groups;
  a.n_ids = groups;
  a.expert_stride = (int64_t)q2k_matrix_bytes(rows_per_group, k);
  a.k = k;
  a.m = m;
  return launched(q2k::launch_mmvq(a, (hipStream_t)stream), fn);
}

int32_t q2k_gemv_bf16(const void* w_dev, const void* x_bf16_dev, int64_t x_row_stride, float* y_dev,
                      int32_t n, int32_t k, int32_t m, void* stream) {
  const char* fn = "q2k_gemv_bf16";
  if (int32_t r = check_matrix(fn, "w", w_dev, n)) return r;
  if (int32_t r = check_out(fn, "y", y_dev)) return r;
  if (!x_bf16_dev) return fail(Q2K_EINVAL, "%s: x is null", fn);
  if (int32_t r = check_k(fn, k)) return r;
  if (int32_t r = check_m(fn, m)) return r;
  if (x_row_stride < k) return fail(Q2K_ESHAPE, "%s: row stride %lld < k = %d", fn, (long long)x_row_stride, k);
  if (!aligned(x_bf16_dev, 16) || x_row_stride % 8 != 0)
    return fail(Q2K_EALIGN, "%s: x must be 16-byte aligned with a row stride that is a multiple of 8", fn);
  if ((int64_t)m * n > (int64_t)1 << 31) return fail(Q2K_ESHAPE, "%s: output larger than 2^31 values", fn);
  const size_t ybytes = (size_t)m * n * 4;
  const size_t xbytes = ((size_t)(m - 1) * x_row_stride + k) * 2;
  if (overlap(y_dev, ybytes, w_dev, q2k_matrix_bytes(n, k)) || overlap(y_dev, ybytes, x_bf16_dev, xbytes))
    return fail(Q2K_EINVAL, "%s: y overlaps an input", fn);
  return launched(q2k::launch_gemv_bf16(w_dev, x_bf16_dev, x_row_stride, y_dev, n, k, m, (hipStream_t)stream),
                  fn);
}

int32_t swiglu_q8_1_rows(const float* g_dev, const float* u_dev, void* h_bf16_dev, void* hq_dev,
                         size_t hq_bytes, int32_t rows, int32_t k, void* stream) {
  const char* fn = "swiglu_q8_1_rows";
  if (!g_dev || !u_dev || !hq_dev) return fail(Q2K_EINVAL, "%s: null pointer", fn);
  if (rows < 1) return fail(Q2K_ESHAPE, "%s: rows = %d < 1", fn, rows);
  if (int32_t r = check_k(fn, k)) return r;
  if (!aligned(g_dev, 16) || !aligned(u_dev, 16) || !aligned(hq_dev, 16) ||
      (h_bf16_dev && !aligned(h_bf16_dev, 16)))
    return fail(Q2K_EALIGN, "%s: g, u, h and hq must be 16-byte aligned", fn);
  const size_t need = q8_1_rows_bytes(rows, k);
  if (hq_bytes < need) return fail(Q2K_ESPACE, "%s: hq holds %zu bytes, %zu needed", fn, hq_bytes, need);
  const size_t fb = (size_t)rows * k * 4, hb = (size_t)rows * k * 2;
  if (overlap(hq_dev, need, g_dev, fb) || overlap(hq_dev, need, u_dev, fb) ||
      (h_bf16_dev && (overlap(h_bf16_dev, hb, g_dev, fb) || overlap(h_bf16_dev, hb, u_dev, fb) ||
                      overlap(h_bf16_dev, hb, hq_dev, need))))
    return fail(Q2K_EINVAL, "%s: an output overlaps an input or the other output", fn);
  return launched(q2k::launch_swiglu_q8_1_rows(g_dev, u_dev, h_bf16_dev, hq_dev, rows, k,
                                               (hipStream_t)stream), fn);
}

int32_t q2k_dequant_rows(const void* table_dev, int64_t n_table_rows, const int64_t* ids_dev,
                         int32_t n_rows, void* out_bf16_dev, int32_t* err_flag_dev, void* stream) {
  const char* fn = "q2k_dequant_rows";
  if (!table_dev || !out_bf16_dev) return fail(Q2K_EINVAL, "%s: null pointer", fn);
  if (n_rows < 1) return fail(Q2K_ESHAPE, "%s: n_rows = %d < 1", fn, n_rows);
  if (n_table_rows < 1) return fail(Q2K_ESHAPE, "%s: empty table", fn);
  if (!ids_dev && n_rows > n_table_rows)
    return fail(Q2K_ESPACE, "%s: %d contiguous rows from a %lld-row table", fn, n_rows, (long long)n_table_rows);
  if (!aligned(table_dev, 4) || !aligned(out_bf16_dev, 8) || (ids_dev && !aligned(ids_dev, 8)))
    return fail(Q2K_EALIGN, "%s: table must be 4-byte, out and ids 8-byte aligned", fn);
  if (overlap(out_bf16_dev, (size_t)n_rows * 512, table_dev, (size_t)n_table_rows * 84))
    return fail(Q2K_EINVAL, "%s: out overlaps the table", fn);
  return launched(q2k::launch_dequant_rows(table_dev, n_table_rows, ids_dev, n_rows, out_bf16_dev,
                                           err_flag_dev, (hipStream_t)stream), fn);
}

int32_t engram_rows_q8_1(const int64_t* token_map_dev, int64_t vocab, const int64_t* multipliers_dev,
                         const int64_t* primes_dev, const int64_t* offsets_dev, int32_t n_layers,
                         int32_t max_ngram, int32_t n_heads, int64_t pad_id, int64_t* cache_dev,
                         int64_t cache_len, const int32_t* token_dev, int64_t pos, int32_t layer,
                         const void* table_dev, int64_t n_table_rows, int64_t* ids_out_dev,
                         void* rows_out_dev, void* xq_dev, size_t xq_bytes, int32_t* err_flag_dev,
                         void* stream) {
  const char* fn = "engram_rows_q8_1";
  if (!token_map_dev || !multipliers_dev || !primes_dev || !offsets_dev || !cache_dev || !token_dev ||
      !table_dev || !xq_dev)
    return fail(Q2K_EINVAL, "%s: null pointer", fn);
  if (vocab < 1) return fail(Q2K_ESHAPE, "%s: vocab = %lld < 1", fn, (long long)vocab);
  if (n_layers < 1 || n_layers > 64) return fail(Q2K_ESHAPE, "%s: n_layers = %d outside 1..64", fn, n_layers);
  if (max_ngram < 2 || max_ngram > 8) return fail(Q2K_ESHAPE, "%s: max_ngram = %d outside 2..8", fn, max_ngram);
  if (n_heads < 1 || n_heads > 64) return fail(Q2K_ESHAPE, "%s: n_heads = %d outside 1..64", fn, n_heads);
  if (layer < 0 || layer >= n_layers) return fail(Q2K_ESHAPE, "%s: layer = %d outside 0..%d", fn, layer, n_layers - 1);
  const int32_t cols = (max_ngram - 1) * n_heads;
  if (cols > 32) return fail(Q2K_ESHAPE, "%s: %d row ids per token, at most 32 (one workgroup)", fn, cols);
  if (pos < 0 || cache_len < pos + 1)
    return fail(Q2K_ESHAPE, "%s: position %lld outside the cache of %lld", fn, (long long)pos, (long long)cache_len);
  if (n_table_rows < 1) return fail(Q2K_ESHAPE, "%s: empty table", fn);
  if (!aligned(token_map_dev, 8) || !aligned(multipliers_dev, 8) || !aligned(primes_dev, 8) ||
      !aligned(offsets_dev, 8) || !aligned(cache_dev, 8) || !aligned(token_dev, 4) ||
      (ids_out_dev && !aligned(ids_out_dev, 8)) || !aligned(table_dev, 4) || !aligned(xq_dev, 16) ||
      (rows_out_dev && !aligned(rows_out_dev, 16)))
    return fail(Q2K_EALIGN, "%s: 64-bit arrays 8-byte, token and table 4-byte, rows and xq 16-byte aligned", fn);
  const int32_t k = cols * 256;
  const size_t need = q8_1_rows_bytes(1, k);
  if (xq_bytes < need) return fail(Q2K_ESPACE, "%s: xq holds %zu bytes, %zu needed", fn, xq_bytes, need);
  const size_t cache_bytes = (size_t)cache_len * 8, tb = (size_t)n_table_rows * 84, ob = (size_t)k * 2;
  const size_t ib = (size_t)cols * 8, vb = (size_t)vocab * 8;
  const void* outs[3] = {xq_dev, rows_out_dev, ids_out_dev};
  const size_t out_b[3] = {need, ob, ib};
  for (int a = 0; a < 3; ++a) {
    if (!outs[a]) continue;
    if (overlap(outs[a], out_b[a], cache_dev, cache_bytes) || overlap(outs[a], out_b[a], table_dev, tb) ||
        overlap(outs[a], out_b[a], token_map_dev, vb) || overlap(outs[a], out_b[a], token_dev, 4))
      return fail(Q2K_EINVAL, "%s: an output overlaps an input or the cache", fn);
    for (int b = a + 1; b < 3; ++b)
      if (outs[b] && overlap(outs[a], out_b[a], outs[b], out_b[b]))
        return fail(Q2K_EINVAL, "%s: two outputs overlap", fn);
  }
  if (overlap(cache_dev, cache_bytes, token_map_dev, vb) || overlap(cache_dev, cache_bytes, token_dev, 4) ||
      overlap(cache_dev, cache_bytes, table_dev, tb))
    return fail(Q2K_EINVAL, "%s: the cache overlaps an input", fn);
  return launched(q2k::launch_engram_rows_q8_1(token_map_dev, vocab, multipliers_dev, primes_dev,
                                               offsets_dev, layer, max_ngram, n_heads, pad_id, cache_dev,
                                               token_dev, pos, table_dev, n_table_rows, ids_out_dev,
                                               rows_out_dev, xq_dev, err_flag_dev, (hipStream_t)stream),
                  fn);
}

}  // extern "C"

namespace {

// engram_step on a workspace ws of ws_bytes bytes (the caller's, or the
// library's own scratch array for engram_step_noalloc: ws_is_scratch, when
// ws is null during the checks and the pointer is fetched afterwards).
// check_only: run every argument check, launch nothing (no HIP call).
int32_t engram_step_on(const char* fn, bool check_only, bool ws_is_scratch, const int64_t* token_map_dev, int64_t vocab,
                       const int64_t* multipliers_dev, const int64_t* primes_dev,
                       const int64_t* offsets_dev, int32_t n_layers, int32_t max_ngram, int32_t n_heads,
                       int64_t pad_id, int64_t* cache_dev, int64_t cache_len, const int32_t* token_dev,
                       int64_t pos, int32_t layer, const void* table_dev, int64_t n_table_rows,
                       const void* wkv_dev, const float* qk_dev, float* h_dev, int32_t hc, int32_t dim,
                       float eps, void* ws, size_t ws_bytes, int32_t* err_flag_dev, void* stream) {
  if (!token_map_dev || !multipliers_dev || !primes_dev || !offsets_dev || !cache_dev || !token_dev ||
      !table_dev || !wkv_dev || !qk_dev || !h_dev || (!ws && !ws_is_scratch))
    return fail(Q2K_EINVAL, "%s: null pointer", fn);
  if (vocab < 1) return fail(Q2K_ESHAPE, "%s: vocab = %lld < 1", fn, (long long)vocab);
  if (n_layers < 1 || n_layers > 64) return fail(Q2K_ESHAPE, "%s: n_layers = %d outside 1..64", fn, n_layers);
  if (max_ngram < 2 || max_ngram > 8) return fail(Q2K_ESHAPE, "%s: max_ngram = %d outside 2..8", fn, max_ngram);
  if (n_heads < 1 || n_heads > 64) return fail(Q2K_ESHAPE, "%s: n_heads = %d outside 1..64", fn, n_heads);
  if (layer < 0 || layer >= n_layers) return fail(Q2K_ESHAPE, "%s: layer = %d outside 0..%d", fn, layer, n_layers - 1);
  const int32_t cols = (max_ngram - 1) * n_heads;
  if (cols > 32) return fail(Q2K_ESHAPE, "%s: %d row ids per token, at most 32", fn, cols);
  if (pos < 0 || cache_len < pos + 1)
    return fail(Q2K_ESHAPE, "%s: position %lld outside the cache of %lld", fn, (long long)pos, (long long)cache_len);
  if (n_table_rows < 1) return fail(Q2K_ESHAPE, "%s: empty table", fn);
  if (hc < 1 || hc > 4) return fail(Q2K_ESHAPE, "%s: hc = %d outside 1..4", fn, hc);
  if (dim < 1 || (int64_t)(hc + 1) * dim > INT32_MAX / 4)
    return fail(Q2K_ESHAPE, "%s: dim = %d outside 1..(2^31/4)/(hc+1)", fn, dim);
  if (!(eps >= 0.0f)) return fail(Q2K_ESHAPE, "%s: eps must be >= 0", fn);
  if (!aligned(token_map_dev, 8) || !aligned(multipliers_dev, 8) || !aligned(primes_dev, 8) ||
      !aligned(offsets_dev, 8) || !aligned(cache_dev, 8) || !aligned(token_dev, 4) ||
      !aligned(table_dev, 4) || !aligned(wkv_dev, 4) || !aligned(qk_dev, 4) || !aligned(h_dev, 4) ||
      (!ws_is_scratch && !aligned(ws, 256)))
    return fail(Q2K_EALIGN, "%s: 64-bit arrays 8-byte, token, table, wkv, qk and h 4-byte, the "
                "workspace 256-byte aligned", fn);
  const int32_t n = (hc + 1) * dim, k = cols * 256;
  const size_t kvb = engram_kv_bytes(hc, dim);
  const size_t need = kvb + q8_1_rows_bytes(1, k);
  if (ws_bytes < need)
    return fail(Q2K_ESPACE, "%s: %s holds %zu bytes, %zu needed", fn,
                ws_is_scratch ? "the library's scratch array" : "the workspace", ws_bytes, need);
  // written: h, cache, workspace; read: everything else
  const void* wr[3] = {h_dev, cache_dev, ws};
  const size_t wr_b[3] = {(size_t)hc * dim * 4, (size_t)cache_len * 8, need};
  const void* rd[8] = {token_map_dev, multipliers_dev, primes_dev, offsets_dev, token_dev, table_dev,
                       wkv_dev, qk_dev};
  const size_t rd_b[8] = {(size_t)vocab * 8, (size_t)n_layers * max_ngram * 8,
                          (size_t)n_layers * (max_ngram - 1) * n_heads * 8, (size_t)n_layers * cols * 8, 4,
                          (size_t)n_table_rows * 84, q2k_matrix_bytes(n, k), (size_t)hc * dim * 4};
  for (int a = 0; a < 3; ++a) {
    if (a == 2 && ws_is_scratch) continue;   // the library's own array overlaps nothing of the caller's
    for (int b = a + 1; b < 3; ++b)
      if (!(b == 2 && ws_is_scratch) && overlap(wr[a], wr_b[a], wr[b], wr_b[b]))
        return fail(Q2K_EINVAL, "%s: h, the cache and the workspace must not overlap", fn);
    for (int b = 0; b < 8; ++b)
      if (overlap(wr[a], wr_b[a], rd[b], rd_b[b])) return fail(Q2K_EINVAL, "%s: h, the cache or the workspace overlaps an input", fn);
  }
  if (check_only) return Q2K_OK;
  q2k::EngramRows E;
  E.token_map = token_map_dev;
  E.vocab = vocab;
  E.mult = multipliers_dev;
  E.primes = primes_dev;
  E.offsets = offsets_dev;
  E.layer = layer;
  E.ng = max_ngram;
  E.n_heads = n_heads;
  E.pad_id = pad_id;
  E.cache = cache_dev;
  E.token = token_dev;
  E.pos = pos;
  E.table = static_cast<const uint8_t*>(table_dev);
  E.n_table_rows = n_table_rows;
  E.err_flag = err_flag_dev;
  float* kv = static_cast<float*>(ws);
  q2k::MmvqLaunch a{};
  a.w[0] = wkv_dev;
  a.y[0] = kv;
  a.n[0] = n;
  a.njobs = 1;
  a.xq = static_cast<uint8_t*>(ws) + kvb;
  a.k = k;
  a.m = 1;
  a.eg = &E;
  const hipStream_t st = (hipStream_t)stream;
  if (int32_t r = launched(q2k::launch_mmvq(a, st), fn)) return r;
  return launched(q2k::launch_engram_gate(h_dev, kv, qk_dev, 1, hc, dim, eps, st), fn);
}


// The engram step's workspace for engram_step_noalloc, for callers that
// cannot allocate: kv of up to 40960 values (hc + 1 = 5 streams of 8192)
// and the q8_1 row of up to 32 gathered rows (8192 values), 163840 + 10240
// bytes, rounded to 176 KiB. Each GPU the library runs on holds its own copy
// until the process ends. In host code `scratch` names a host-side stand-in:
// only the per-device address from hipGetSymbolAddress is handed to kernels.
__device__ __align__(256) uint8_t scratch[Q2K_ENGRAM_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_dev[64];   // per device: the device address of its `scratch`

// The current device's address of `scratch`, looked up once per device with
// that device current.
int32_t scratch_address(const char* fn, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(Q2K_EDEVICE, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(Q2K_EDEVICE, "%s: device %d, at most 64 are tracked", fn, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(Q2K_EDEVICE, "%s: hipGetSymbolAddress(scratch) failed: %s", fn, hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return Q2K_OK;
}

}  // namespace

extern "C" {

int32_t engram_step(const int64_t* token_map_dev, int64_t vocab, const int64_t* multipliers_dev,
                    const int64_t* primes_dev, const int64_t* offsets_dev, int32_t n_layers,
                    int32_t max_ngram, int32_t n_heads, int64_t pad_id, int64_t* cache_dev,
                    int64_t cache_len, const int32_t* token_dev, int64_t pos, int32_t layer,
                    const void* table_dev, int64_t n_table_rows, const void* wkv_dev,
                    const float* qk_dev, float* h_dev, int32_t hc, int32_t dim, float eps,
                    void* workspace_dev, size_t workspace_bytes, int32_t* err_flag_dev, void* stream) {
  return engram_step_on("engram_step", false, false, token_map_dev, vocab, multipliers_dev, primes_dev, offsets_dev,
                        n_layers, max_ngram, n_heads, pad_id, cache_dev, cache_len, token_dev, pos, layer,
                        table_dev, n_table_rows, wkv_dev, qk_dev, h_dev, hc, dim, eps, workspace_dev,
                        workspace_bytes, err_flag_dev, stream);
}

int32_t engram_step_noalloc(const int64_t* token_map_dev, int64_t vocab, const int64_t* multipliers_dev,
                            const int64_t* primes_dev, const int64_t* offsets_dev, int32_t n_layers,
                            int32_t max_ngram, int32_t n_heads, int64_t pad_id, int64_t* cache_dev,
                            int64_t cache_len, const int32_t* token_dev, int64_t pos, int32_t layer,
                            const void* table_dev, int64_t n_table_rows, const void* wkv_dev,
                            const float* qk_dev, float* h_dev, int32_t hc, int32_t dim, float eps,
                            int32_t* err_flag_dev, void* stream) {
  const char* fn = "engram_step_noalloc";
  // every check first (no HIP call), then the scratch address, then the launches
  if (int32_t r = engram_step_on(fn, true, true, token_map_dev, vocab, multipliers_dev, primes_dev,
                                 offsets_dev, n_layers, max_ngram, n_heads, pad_id, cache_dev, cache_len,
                                 token_dev, pos, layer, table_dev, n_table_rows, wkv_dev, qk_dev, h_dev, hc,
                                 dim, eps, nullptr, Q2K_ENGRAM_SCRATCH_BYTES, err_flag_dev, stream))
    return r;
  void* ws = nullptr;
  if (int32_t r = scratch_address(fn, &ws)) return r;
  return engram_step_on(fn, false, true, token_map_dev, vocab, multipliers_dev, primes_dev, offsets_dev,
                        n_layers, max_ngram, n_heads, pad_id, cache_dev, cache_len, token_dev, pos, layer,
                        table_dev, n_table_rows, wkv_dev, qk_dev, h_dev, hc, dim, eps, ws,
                        Q2K_ENGRAM_SCRATCH_BYTES, err_flag_dev, stream);
}

int32_t q2k_dequant_rows_q8_1(const void* table_dev, int64_t n_table_rows, const int64_t* ids_dev,
                              int32_t n_rows, void* out_bf16_dev, void* xq_dev, size_t xq_bytes,
                              int32_t* err_flag_dev, void* stream) {
  const char* fn = "q2k_dequant_rows_q8_1";
  if (!table_dev || !xq_dev) return fail(Q2K_EINVAL, "%s: null pointer", fn);
  if (n_rows < 1 || n_rows > (1 << 20)) return fail(Q2K_ESHAPE, "%s: n_rows = %d outside 1..2^20", fn, n_rows);
  if (n_table_rows < 1) return fail(Q2K_ESHAPE, "%s: empty table", fn);
  if (!ids_dev && n_rows > n_table_rows)
    return fail(Q2K_ESPACE, "%s: %d contiguous rows from a %lld-row table", fn, n_rows, (long long)n_table_rows);
  if (!aligned(table_dev, 4) || !aligned(xq_dev, 16) || (ids_dev && !aligned(ids_dev, 8)) ||
      (out_bf16_dev && !aligned(out_bf16_dev, 16)))
    return fail(Q2K_EALIGN, "%s: table must be 4-byte, ids 8-byte, out and xq 16-byte aligned", fn);
  const int32_t k = n_rows * 256;
  const size_t need = q8_1_rows_bytes(1, k);
  if (xq_bytes < need) return fail(Q2K_ESPACE, "%s: xq holds %zu bytes, %zu needed", fn, xq_bytes, need);
  const size_t tb = (size_t)n_table_rows * 84, ob = (size_t)k * 2;
  if (overlap(xq_dev, need, table_dev, tb) ||
      (out_bf16_dev && (overlap(out_bf16_dev, ob, table_dev, tb) || overlap(out_bf16_dev, ob, xq_dev, need))))
    return fail(Q2K_EINVAL, "%s: an output overlaps the table or the other output", fn);
  return launched(q2k::launch_dequant_rows_q8_1(table_dev, n_table_rows, ids_dev, n_rows, out_bf16_dev,
                                                xq_dev, err_flag_dev, (hipStream_t)stream), fn);
}

int32_t engram_gate(float* h_dev, const float* kv_dev, const float* qk_dev, int32_t t, int32_t hc,
                    int32_t dim, float eps, void* stream) {
  const char* fn = "engram_gate";
  if (!h_dev || !kv_dev || !qk_dev) return fail(Q2K_EINVAL, "%s: null pointer", fn);
  if (hc < 1 || hc > 4) return fail(Q2K_ESHAPE, "%s: hc = %d outside 1..4", fn, hc);
  if (dim < 1) return fail(Q2K_ESHAPE, "%s: dim = %d < 1", fn, dim);
  if (t < 1 || t > 65535) return fail(Q2K_ESHAPE, "%s: t = %d outside 1..65535", fn, t);
  if (!(eps >= 0.0f)) return fail(Q2K_ESHAPE, "%s: eps must be >= 0", fn);
  if (!aligned(h_dev, 4) || !aligned(kv_dev, 4) || !aligned(qk_dev, 4))
    return fail(Q2K_EALIGN, "%s: pointers must be 4-byte aligned", fn);
  const size_t hb = (size_t)t * hc * dim * 4;
  if (overlap(h_dev, hb, kv_dev, (size_t)t * (hc + 1) * dim * 4) ||
      overlap(h_dev, hb, qk_dev, (size_t)hc * dim * 4))
    return fail(Q2K_EINVAL, "%s: h overlaps kv or qk", fn);
  return launched(q2k::launch_engram_gate(h_dev, kv_dev, qk_dev, t, hc, dim, eps, (hipStream_t)stream), fn);
}

int32_t engram_hash(const int64_t* token_map_dev, int64_t vocab, const int64_t* multipliers_dev,
                    const int64_t* primes_dev, const int64_t* offsets_dev, int32_t n_layers,
                    int32_t max_ngram, int32_t n_heads, int64_t pad_id, int64_t* cache_dev,
                    int64_t cache_len, const int32_t* ids_dev, int32_t seqlen, int64_t start_pos,
                    int64_t* out_dev, int32_t* err_flag_dev, void* stream) {
  const char* fn = "engram_hash";
  if (!token_map_dev || !multipliers_dev || !primes_dev || !offsets_dev || !cache_dev || !ids_dev ||
      !out_dev)
    return fail(Q2K_EINVAL, "%s: null pointer", fn);
  if (vocab < 1) return fail(Q2K_ESHAPE, "%s: vocab = %lld < 1", fn, (long long)vocab);
  if (n_layers < 1 || n_layers > 64) return fail(Q2K_ESHAPE, "%s: n_layers = %d outside 1..64", fn, n_layers);
  if (max_ngram < 2 || max_ngram > 8) return fail(Q2K_ESHAPE, "%s: max_ngram = %d outside 2..8", fn, max_ngram);
  if (n_heads < 1 || n_heads > 64) return fail(Q2K_ESHAPE, "%s: n_heads = %d outside 1..64", fn, n_heads);
  if (seqlen < 1) return fail(Q2K_ESHAPE, "%s: seqlen = %d < 1", fn, seqlen);
  if (start_pos < 0 || cache_len < start_pos + seqlen)
    return fail(Q2K_ESHAPE, "%s: positions %lld..%lld outside the cache of %lld", fn, (long long)start_pos,
                (long long)(start_pos + seqlen), (long long)cache_len);
  if ((int64_t)seqlen * n_layers > INT32_MAX) return fail(Q2K_ESHAPE, "%s: seqlen * n_layers too large", fn);
  if (!aligned(token_map_dev, 8) || !aligned(multipliers_dev, 8) || !aligned(primes_dev, 8) ||
      !aligned(offsets_dev, 8) || !aligned(cache_dev, 8) || !aligned(out_dev, 8) || !aligned(ids_dev, 4))
    return fail(Q2K_EALIGN, "%s: 64-bit arrays must be 8-byte aligned, ids 4-byte aligned", fn);
  const int64_t cols = (int64_t)(max_ngram - 1) * n_heads;
  const size_t out_bytes = (size_t)n_layers * seqlen * cols * 8;
  const size_t cache_bytes = (size_t)cache_len * 8;
  if (overlap(out_dev, out_bytes, cache_dev, cache_bytes) ||
      overlap(out_dev, out_bytes, token_map_dev, (size_t)vocab * 8) ||
      overlap(out_dev, out_bytes, ids_dev, (size_t)seqlen * 4) ||
      overlap(cache_dev, cache_bytes, token_map_dev, (size_t)vocab * 8) ||
      overlap(cache_dev, cache_bytes, ids_dev, (size_t)seqlen * 4))
    return fail(Q2K_EINVAL, "%s: out or cache overlaps another argument", fn);
  return launched(q2k::launch_engram_hash(token_map_dev, vocab, multipliers_dev, primes_dev, offsets_dev,
                                          n_layers, max_ngram, n_heads, pad_id, cache_dev, ids_dev, seqlen,
                                          start_pos, out_dev, err_flag_dev, (hipStream_t)stream),
                  fn);
}

size_t engram_step_workspace_bytes(int32_t max_ngram, int32_t n_heads, int32_t hc, int32_t dim) {
  if (max_ngram < 2 || max_ngram > 8 || n_heads < 1 || n_heads > 64 || hc < 1 || hc > 4 || dim < 1)
    return 0;
  const int32_t cols = (max_ngram - 1) * n_heads;
  if (cols > 32) return 0;
  return engram_kv_bytes(hc, dim) + q8_1_rows_bytes(1, cols * 256);
}

int32_t q2k_product_kernel(int32_t n, int32_t k, int32_t m) {
  const char* fn = "q2k_product_kernel";
  if (n < 1) return fail(Q2K_ESHAPE, "%s: n must be >= 1", fn);
  if (int32_t r = check_k(fn, k)) return r;
  if (m < 1 || m > Q2K_MMQ_MAX_M) return fail(Q2K_ESHAPE, "%s: m must be in 1..%d", fn, Q2K_MMQ_MAX_M);
  if (m >= q2k::kMmqTileMinM) return Q2K_KERNEL_MATRIX_CORES;   // q2k_mmq's tile kernel, any choice
  q2k::MmvqLaunch a{};
  a.n[0] = n;
  a.njobs = 1;
  a.k = k;
  a.m = m;
  return q2k::takes_mfma(a) ? Q2K_KERNEL_MATRIX_CORES : Q2K_KERNEL_PACKED_DOTS;
}

int32_t q2k_block_dots(const void* w_dev, const void* xq_dev, int32_t* out_dev, int32_t n,
                       int32_t k, int32_t m, void* stream) {
  const char* fn = "q2k_block_dots";
  if (int32_t r = check_matrix(fn, "w", w_dev, n)) return r;
  if (!xq_dev || !out_dev) return fail(Q2K_EINVAL, "%s: null pointer", fn);
  if (int32_t r = check_k(fn, k)) return r;
  if (m < 1 || m > Q2K_MMQ_MAX_M) return fail(Q2K_ESHAPE, "%s: m = %d outside 1..%d", fn, m, Q2K_MMQ_MAX_M);
  if (!aligned(xq_dev, 16) || !aligned(out_dev, 16))
    return fail(Q2K_EALIGN, "%s: xq and out must be 16-byte aligned", fn);
  if ((int64_t)m * n * (k / 32) * 2 > (int64_t)1 << 31)
    return fail(Q2K_ESHAPE, "%s: output larger than 2^31 values", fn);
  if (overlap(out_dev, (size_t)m * n * (k / 32) * 8, w_dev, q2k_matrix_bytes(n, k)) ||
      overlap(out_dev, (size_t)m * n * (k / 32) * 8, xq_dev, (size_t)m * q2k::q8_row_bytes(k)))
    return fail(Q2K_EINVAL, "%s: out overlaps an input", fn);
  if (m >= q2k::kMmqTileMinM)
    return launched(q2k::launch_mmq(w_dev, xq_dev, nullptr, out_dev, n, k, m, (hipStream_t)stream), fn);
  q2k::MmvqLaunch a{};
  a.w[0] = w_dev;
  a.n[0] = n;
  a.njobs = 1;
  a.xq = xq_dev;
  a.dots = out_dev;
  a.k = k;
  a.m = m;
  return launched(q2k::launch_mmvq(a, (hipStream_t)stream), fn);
}

}  // extern "C"
