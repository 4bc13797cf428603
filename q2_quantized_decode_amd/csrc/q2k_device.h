// Device-side helpers shared by the gfx950 kernels of libq2kdecode.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace q2k {

constexpr int kBlockBytes = 84;     // GGUF Q2_K super-block (engram_v41.rs ENGRAM_ROW_BYTES)
constexpr int kBlockWeights = 256;
constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// Same vectors with only 4-byte alignment: Q2_K blocks are 84 bytes, so a
// field inside one is dword aligned but not 8/16-byte aligned.
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// q8_1 row layout of this library: k int8 quants, k/32 f32 scales, k/16
// int16 sums of 16 quants.
__host__ __device__ constexpr size_t q8_row_bytes(int k) { return (size_t)k * 5 / 4; }
__host__ __device__ constexpr size_t q8_scale_offset(int k) { return (size_t)k; }
__host__ __device__ constexpr size_t q8_sum_offset(int k) { return (size_t)k + (size_t)k / 8; }

// Where a product reads its q8_1 activations: the quants, block scales and
// half sums of token 0, and the byte distance between tokens. A whole row of
// K values starting at `row` has its fields at row, row + K and row + 9K/8;
// the sub-row of that row starting at element e0 (a multiple of 256) has the
// same layout shifted by e0 quant bytes and e0/8 scale and sum bytes.
struct XView {
  const uint8_t* q;
  const uint8_t* s;
  const uint8_t* m;
  int64_t stride;
};

__host__ __device__ inline XView xview(const uint8_t* row, int K, int e0) {
  return XView{row + e0, row + q8_scale_offset(K) + e0 / 8, row + q8_sum_offset(K) + e0 / 8,
               (int64_t)q8_row_bytes(K)};
}

// Load through an explicit global (address space 1) pointer, so the access
// is a global_load with an SGPR base rather than a flat load.
template <typename T>
__device__ __forceinline__ T gload(const void* p) {
  return *(const __attribute__((address_space(1))) T*)(p);
}

// ---------------------------------------------------------------------------
// Cross-lane helpers on fp64 values (moved as two dwords).

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xf, 0xf, false);
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// DPP controls whose partner is exactly lane l ^ OFF: quad_perm [1,0,3,2]
// and [2,3,0,1] for 1 and 2, row_ror:8 for 8 (a rotation by half of a
// 16-lane row).
template <int OFF> struct DppPartner;
template <> struct DppPartner<8> { static constexpr int ctrl = 0x128; };
template <> struct DppPartner<2> { static constexpr int ctrl = 0x4E; };
template <> struct DppPartner<1> { static constexpr int ctrl = 0xB1; };

__device__ __forceinline__ uint64_t bits64(double v) { return __builtin_bit_cast(uint64_t, v); }
__device__ __forceinline__ double from_bits(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Lane l ^ 4's value (ds_swizzle in xor mode, within 32 lanes).
__device__ __forceinline__ double xor4_f64(double v) {
  const uint64_t b = bits64(v);
  const int lo = __builtin_amdgcn_ds_swizzle((int)(uint32_t)b, 0x101F);
  const int hi = __builtin_amdgcn_ds_swizzle((int)(uint32_t)(b >> 32), 0x101F);
  return from_bits((uint32_t)lo, (uint32_t)hi);
}

// One halving level of a transposed reduction: lanes whose bit OFF is 0 end
// with X summed over the lane pair (l, l ^ OFF), the others with Y summed
// over the pair.
template <int OFF>
__device__ __forceinline__ double halve(double x, double y, int lane) {
  if constexpr (OFF == 32) {
    // swaps lanes 32..63 of the first operand with lanes 0..31 of the second
    const uint64_t bx = bits64(x), by = bits64(y);
    const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)bx, (uint32_t)by, false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(bx >> 32), (uint32_t)(by >> 32),
                                                     false, false);
    return from_bits(lo[0], hi[0]) + from_bits(lo[1], hi[1]);
  } else if constexpr (OFF == 16) {
    // swaps the odd 16-lane rows of the first operand with the even rows of the second
    const uint64_t bx = bits64(x), by = bits64(y);
    const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)bx, (uint32_t)by, false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(bx >> 32), (uint32_t)(by >> 32),
                                                     false, false);
    return from_bits(lo[0], hi[0]) + from_bits(lo[1], hi[1]);
  } else {
    const bool up = (lane & OFF) != 0;
    const double send = up ? x : y;
    const double keep = up ? y : x;
    if constexpr (OFF == 4) {
      return keep + xor4_f64(send);
    } else {
      return keep + dpp_f64<DppPartner<OFF>::ctrl>(send);
    }
  }
}


// 32-bit cross-lane partners: DPP for l ^ 1, l ^ 2 and l ^ 8, ds_swizzle in
// xor mode for l ^ 4, and the permlane swaps for the sums with l ^ 16 and
// l ^ 32 (each lane gets its own value plus its partner's).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ uint32_t xor4_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x101F);
}
__device__ __forceinline__ float sum_xor16_f32(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32_f32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// f32 sum over all 64 lanes, left on every lane: partners l ^ 1, l ^ 2, ..,
// l ^ 32 in that order.
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += __uint_as_float(dpp_u32<0xB1>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x4E>(__float_as_uint(v)));
  v += __uint_as_float(xor4_u32(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x128>(__float_as_uint(v)));
  v = sum_xor16_f32(v);
  return sum_xor32_f32(v);
}

// The sum of v over each aligned group of 1 << GSL lanes (GSL <= 6), left on
// every lane of the group: partners l ^ 1, l ^ 2, l ^ 4, l ^ 8, l ^ 16, l ^ 32
// in that order, each level one exchange and one add (DPP, ds_swizzle or
// permlane swaps: no LDS round trip).
template <int GSL>
__device__ __forceinline__ double group_sum_f64(double v, int lane) {
  static_assert(GSL >= 0 && GSL <= 6, "at most one wave");
  if constexpr (GSL >= 1) v += dpp_f64<DppPartner<1>::ctrl>(v);
  if constexpr (GSL >= 2) v += dpp_f64<DppPartner<2>::ctrl>(v);
  if constexpr (GSL >= 3) v += xor4_f64(v);
  if constexpr (GSL >= 4) v += dpp_f64<DppPartner<8>::ctrl>(v);
  if constexpr (GSL >= 5) v = halve<16>(v, v, lane);
  if constexpr (GSL >= 6) v = halve<32>(v, v, lane);
  return v;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// f32 -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float fp16_bits_to_f32(uint32_t h) {
  _Float16 v = __builtin_bit_cast(_Float16, (uint16_t)h);
  return (float)v;
}

// Signed 4 x int8 dot product accumulated into c (v_dot4c_i32_i8).
__device__ __forceinline__ int sdot4(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// The fixed summation order of every Q2_K x q8_1 product kernel (so that
// all of them return the same bits for the same inputs):
//  * leaf, one half block (super-block b, half h: q8 blocks c = 8b+4h+j,
//    j = 0..3) of one row and token: fI = ((d8_0 I_0 + d8_1 I_1) + d8_2 I_2)
//    + d8_3 I_3, one fma per term from +0 (every d8 * I is exact in fp64:
//    24 + 18 bits), fM likewise with M, and v = RN(d * fI) - RN(dmin * fM);
//  * per half h, the pairwise tree over b = 0 .. NBP-1 (NBP: the row's block
//    count rounded up to a power of two, leaves past the row are +0),
//    neighbours first;
//  * the two halves added, then rounded once to f32.
// fp64 because post-SwiGLU activations reach 10^3 while outputs cross zero.
__device__ __forceinline__ double half_value(double d, double dmin, double fI, double fM) {
#pragma clang fp contract(off)
  const double a = d * fI;
  const double c = dmin * fM;
  return a - c;
}

__device__ __forceinline__ float quiet_nan() { return __uint_as_float(0x7fc00000u); }

// q8_1 of one 32-value block (every quantiser of this library uses these
// two, so fused and separate quantisation give the same bytes): d = amax/127
// as a correctly rounded f32 division, and q = round-half-away-from-zero of
// the correctly rounded quotient v/d, clamped to [-127, 127]; 0 when d == 0.
__device__ __forceinline__ float q8_1_scale(float amax) { return amax / 127.0f; }

__device__ __forceinline__ int q8_1_quant(float v, float d) {
  const float r = fminf(fmaxf(roundf(v / d), -127.0f), 127.0f);   // no branch: d == 0 selects 0
  return d > 0.0f ? (int)r : 0;
}

// q8_1_quant(v[i], d) for the NV values of one lane (all of one block), with
// one correctly rounded division rd = 1.0f / d instead of one per value.
// For a normal d, |v| <= amax = 127.x * d, so a = v * rd is within 2^-16
// (two roundings of 2^-24 relative) of v / d and within 2^-15.6 of its
// correctly rounded f32 quotient, and |a| < 127.5. Where a is more than
// 2^-14 away from the nearest half-integer, both round to the same integer
// and no tie is involved, so round-to-nearest-even of a (one instruction)
// equals the half-away rounding of the quotient, already within +-127.
// A value closer than that (ties included), a NaN, or a d that is zero or
// subnormal is recomputed with the division, after the loop and only where
// some lane of the wave needs it: exact ties are common (any element equal
// to half its block's maximum gives v/d = 63.5), so redoing a whole lane's
// values whenever one of them is near a tie had most waves take every
// division.
template <int NV>
__device__ __forceinline__ void q8_1_quant_lane(const float* v, float d, int* q) {
  const float rd = 1.0f / d;
  const bool dslow = !(d >= 0x1p-126f);
  bool slow = dslow;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const float a = v[i] * rd;
    const float r = rintf(a);
    slow = slow || !(fabsf(a - r) < 0.5f - 0x1p-14f);
    q[i] = (int)r;
  }
  if (slow) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const float a = v[i] * rd;
      if (dslow || !(fabsf(a - rintf(a)) < 0.5f - 0x1p-14f)) q[i] = q8_1_quant(v[i], d);
    }
  }
}


// q8_1 of 8 values v (elements e0..e0+7 of one row), lanes 4i..4i+3 of the
// wave holding one 32-block (all lanes call it): the block scale d, the 8
// quants and the sum of the lane's 16-wide half (lanes 2i and 2i+1).
struct Q8Lane {
  float d;
  uint32_t lo, hi;   // the 8 quants, bytes
  int s;             // sum of the 16 quants of the lane pair
};

__device__ __forceinline__ Q8Lane q8_1_quant8(const float* v) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[i]));
  a = fmaxf(a, __uint_as_float(dpp_u32<0xB1>(__float_as_uint(a))));
  a = fmaxf(a, __uint_as_float(dpp_u32<0x4E>(__float_as_uint(a))));
  Q8Lane r;
  r.d = q8_1_scale(a);
  int q[8];
  q8_1_quant_lane<8>(v, r.d, q);   // halves away from zero
  int s = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += q[i];
  r.s = s + (int)dpp_u32<0xB1>((uint32_t)s);
  r.lo = (uint32_t)(q[0] & 0xff) | ((uint32_t)(q[1] & 0xff) << 8) |
         ((uint32_t)(q[2] & 0xff) << 16) | ((uint32_t)(q[3] & 0xff) << 24);
  r.hi = (uint32_t)(q[4] & 0xff) | ((uint32_t)(q[5] & 0xff) << 8) |
         ((uint32_t)(q[6] & 0xff) << 16) | ((uint32_t)(q[7] & 0xff) << 24);
  return r;
}

// Stores a lane's part of a q8_1 row (row base: device memory or LDS).
__device__ __forceinline__ void q8_1_put8(const Q8Lane& r, uint8_t* row, int e0, int k) {
  *reinterpret_cast<u32x2*>(row + e0) = u32x2{r.lo, r.hi};
  const int lane = threadIdx.x & 63;
  if ((lane & 3) == 0)
    *reinterpret_cast<float*>(row + q8_scale_offset(k) + (size_t)(e0 / 32) * 4) = r.d;
  if ((lane & 1) == 0)
    *reinterpret_cast<int16_t*>(row + q8_sum_offset(k) + (size_t)(e0 / 16) * 2) = (int16_t)r.s;
}

__device__ __forceinline__ void q8_1_store8(const float* v, uint8_t* row, int e0, int k,
                                            bool active) {
  const Q8Lane r = q8_1_quant8(v);
  if (active) q8_1_put8(r, row, e0, k);
}

// bf16 bits of silu(g) * u (the bf16 SwiGLU of the expert batch), in f32:
// silu(g) = g * sigmoid(g), with exp taken of -|g| so it cannot overflow
// (sigmoid = 1/(1+e) for g >= 0, e/(1+e) for g < 0), then round to nearest
// even. Every SwiGLU of this library uses it, so they give the same bits.
__device__ __forceinline__ uint32_t swiglu_bf16_bits(float g, float u) {
  const float e = expf(-fabsf(g));
  const float sig = g >= 0.0f ? 1.0f / (1.0f + e) : e / (1.0f + e);
  return f32_to_bf16_bits(g * sig * u);
}

// bf16 bits of elements e..e+3 (e a multiple of 4) of one 84-byte Q2_K block:
// v = d*sc*q - dmin*m formed in f32 (d*(sc*q) and dmin*m are exact, so the
// subtraction is the only rounding), then bf16 to nearest-even. The four
// elements share h = e>>7, plane j = (e>>5)&3 and sub-block e>>4.
__device__ __forceinline__ void q2k_dequant4(const uint8_t* blk, int e, uint32_t bits[4]) {
  const int h = e >> 7;
  const int j = (e >> 5) & 3;
  const int l = e & 31;
  const uint32_t qw = *reinterpret_cast<const uint32_t*>(blk + 16 + 32 * h + l) >> (2 * j);
  const uint32_t sb = blk[e >> 4];
  const uint32_t dd = *reinterpret_cast<const uint32_t*>(blk + 80);
  const float d = fp16_bits_to_f32(dd & 0xffffu);
  const float dmin = fp16_bits_to_f32(dd >> 16);
  const float mterm = dmin * (float)(sb >> 4);   // exact: <= 15 significant bits
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t q = (qw >> (8 * i)) & 3u;
    const float v = d * (float)((sb & 15u) * q) - mterm;
    bits[i] = f32_to_bf16_bits(v);
  }
}

// x mod p in [0, p) for p > 0 (the Euclidean remainder: C's % then + p when
// negative). For p < 2^32 the unsigned remainder is taken 16 bits at a time
// in fp64: every partial dividend is below p * 2^16 < 2^48, so it, the
// quotient estimate's product and the difference are exact, and the
// estimate floor(D * (1/p)) is off by at most one, which one compare each
// way corrects. Larger p take the integer division.
__device__ __forceinline__ int64_t mod_euclid_i64(int64_t x, int64_t p) {
  const bool neg = x < 0;
  const uint64_t u = neg ? 0ull - (uint64_t)x : (uint64_t)x;
  uint64_t r;
  if ((uint64_t)p >> 32 == 0) {
    const double pd = (double)p;
    const double inv = 1.0 / pd;
    double rr = 0.0;
#pragma unroll
    for (int k = 3; k >= 0; --k) {
      const double dv = fma(rr, 65536.0, (double)((u >> (16 * k)) & 0xffffull));
      const double q = floor(dv * inv);
      double t = fma(-q, pd, dv);
      t = t < 0.0 ? t + pd : t;
      rr = t >= pd ? t - pd : t;
    }
    r = (uint64_t)rr;
  } else {
    r = u % (uint64_t)p;
  }
  return (int64_t)(neg && r != 0 ? (uint64_t)p - r : r);
}

// Engram n-gram hash helpers (engram_v41.rs, EngramHasher::hash), shared by
// the hash kernels and the product's engram prologue.
constexpr int kMaxNgram = 8;

// Window of position pos = start_pos + s for the hash: tok[0..ng-1] and
// whether every token id it reads is valid. Position p >= start_pos reads
// this call's ids, earlier positions the cache; from the first i with
// pos < i or an unmapped (-1) id on, the token is pad_id. Returns the
// compressed id of pos itself (what the cache keeps for it).
__device__ __forceinline__ int64_t hash_window(const int64_t* __restrict__ token_map, int64_t vocab,
                                               int ng, int64_t pad_id, const int64_t* cache,
                                               const int32_t* __restrict__ ids, int64_t start_pos,
                                               int64_t pos, int64_t tok[kMaxNgram], bool& ok) {
  bool blocked = false;
  int64_t own = -1;
  for (int i = 0; i < ng; ++i) {
    const int64_t p = pos >= i ? pos - i : 0;
    int64_t src;
    if (p >= start_pos) {
      const int32_t id = ids[p - start_pos];
      if (id < 0 || id >= vocab) {
        ok = false;
        src = -1;
      } else {
        src = token_map[id];
      }
    } else {
      src = cache[p];
    }
    if (i == 0) own = src;
    blocked = blocked || pos < i || src == -1;
    tok[i] = blocked ? pad_id : src;
  }
  return own;
}

// Row ids of hashed layer l for a window: rolling = tok[0]*mult[l][0], then
// rolling ^= tok[i]*mult[l][i] (64-bit wrapping); id (i, h) = (rolling mod
// prime, in [0, prime)) + offset; -1 once the window is bad or a prime <= 0
// has been met (in (i, h) order). Writes o[c] for c in [c0, c1) and returns
// false when any id so far is -1.
__device__ __forceinline__ bool hash_cols(const int64_t tok[kMaxNgram], const int64_t* __restrict__ mult,
                                          const int64_t* __restrict__ primes,
                                          const int64_t* __restrict__ offsets, int l, int ng,
                                          int n_heads, bool ok, int c0, int c1, int64_t* o) {
  const int cols = (ng - 1) * n_heads;
  const int64_t* ml = mult + (int64_t)l * ng;
  uint64_t rolling = (uint64_t)tok[0] * (uint64_t)ml[0];
  for (int i = 1; i < ng; ++i) {
    rolling ^= (uint64_t)tok[i] * (uint64_t)ml[i];
    for (int h = 0; h < n_heads; ++h) {
      const int col = (i - 1) * n_heads + h;
      const int64_t pr = primes[((int64_t)l * (ng - 1) + (i - 1)) * n_heads + h];
      int64_t v = -1;
      if (ok && pr > 0) {
        const int64_t r = mod_euclid_i64((int64_t)rolling, pr);
        v = (int64_t)((uint64_t)r + (uint64_t)offsets[(int64_t)l * cols + col]);
      } else {
        ok = false;
      }
      if (col >= c0 && col < c1) o[col - c0] = v;
    }
    if (i * n_heads >= c1) break;   // later columns are not asked for
  }
  return ok;
}


}  // namespace q2k
