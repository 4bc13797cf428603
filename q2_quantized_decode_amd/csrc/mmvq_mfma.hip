// Q2_K x q8_1 product for 2..8 tokens (and, by groups of 8, any number of
// tokens) on the CDNA4 matrix cores.
//
// The weights are GGUF Q2_K super-blocks as the file ships them (engram_v41.rs:
// ENGRAM_ROW_BYTES = 84 bytes per 256 weights, EngramLayerWeights::wkv_q2k);
// the activations are this library's q8_1 rows. The pages' own kernels for
// this product (moe_v41/init.rs: kquant_mmvq_q2_k_w, the experts variants,
// metrale_q2_k_mmq128_*) are CUDA warp kernels whose source is not shown.
// With 8 tokens a packed-dot formulation spends two int8 dot instructions per
// 4 weights on the vector ALUs; here both exact integer block sums go through
// v_mfma_i32_16x16x64_i8 and the vector ALUs unpack the 2-bit weights and
// run the fp64 epilogue.
//
// * Tile: one wave computes 16 weight rows x 8 token slots over a range of
//   super-blocks, one 256-weight super-block b at a time. Weights are the B
//   operand: lane (g = lane/16, j = lane%16) loads only its own row r0 + j
//   (16 bytes of qs, 8 scale bytes, d/dmin), 28 bytes per super-block.
// * Integer sums: plane p = 0..3 of a super-block is two MFMAs with K = 64
//   weights; K-group g holds the 16 weights 128(g>>1) + 32p + 16(g&1) + 0..15,
//   i.e. qs bytes 16g..16g+15 at bits 2p..2p+1, all in sub-block
//   s = 8(g>>1) + 2p + (g&1). For I the B operand is sc_s * q (<= 45, so
//   four masked quants times sc in one 32-bit multiply); for M it is m_s in
//   every byte. The A operand (activations) is block diagonal: A-row a = token
//   (a&7), half (a>>3) carries that token's quants of q8 block 4(a>>3) + p in
//   the two K-groups of that half and zeros elsewhere, so each output is
//   exactly one I (or M) of one (token, q8 block, row).
// * Epilogue: the library's fixed summation order (q2k_device.h, half_value):
//   lane (g, j) holds half h = g>>1 of tokens 4(g&1) + 0..3, so the four
//   planes of a super-block are that half block's four q8 blocks; the leaf
//   value is formed exactly as in the packed-dot kernels, the leaves of the
//   wave's super-blocks are combined pairwise, the two waves of a tile meet
//   through LDS (left + right subtree) and the halves across lanes g, g ^ 2.
// * Activations of the workgroup's matrix (8 token slots of quants and fp64
//   d8, plus an all-zero slot) are staged once in LDS; the waves of a
//   workgroup take eight consecutive tiles of one matrix.
//
// A workgroup is sixteen waves: two per tile, wave 0 taking super-blocks
// [0, NBP/2) in order and wave 1 the rest [NBP/2, NB) from the end (NBP: NB
// rounded up to a power of two), so that each 128-byte line shared by two
// super-blocks (84-byte blocks straddle lines, also at the split and from one
// row to the next) is read by both waves at about the same time and comes
// from L2 the second time. Four waves per SIMD hide the dependency chains of
// one tile.
#include <stdint.h>

#include "q2k_device.h"
#include "q2k_launch.h"

namespace q2k {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef double v4d __attribute__((ext_vector_type(4)));

constexpr int kSlots = 8;              // token slots of a tile (m <= 8; unused slots are zero)
constexpr int kTabSlots = kSlots + 1;  // plus one all-zero slot
constexpr int kTilesPerWg = 8;
constexpr uint32_t kMfmaMaxLds = 160 * 1024;
constexpr int kThreads = 2 * kTilesPerWg * kWave;   // two waves per tile
// The second waves hand their 4 fp64 subtree sums per lane to the first.
constexpr uint32_t kXchgBytes = kTilesPerWg * kWave * 4 * 8;

struct MfmaParams {
  const uint8_t* w[kMaxPlainJobs];   // plain: job matrices; expert mode: the bases
  float* y[kMaxPlainJobs];
  int32_t n[kMaxPlainJobs];
  int32_t wg_end[kMaxPlainJobs];     // plain mode: exclusive prefix of workgroups per job
  const uint8_t* xq;
  const int32_t* ids;                // expert mode when non-null
  int32_t n_ids;                     // expert mode: ids; grouped mode: groups
  int32_t n_experts;
  int32_t x_per_id;
  int64_t expert_stride;
  int32_t* err_flag;
  int32_t* dots;                     // DOTS kernel: int32 (I, M) per (token, row, q8 block)
  int32_t groups;                    // grouped mode when > 0
  int32_t wgs_per_job;               // expert and grouped modes
  int32_t total_wgs;
  int32_t m;                         // tokens of the launch (any count)
  int32_t tgroups;                   // groups of kSlots tokens: ceil(m / kSlots)
  int32_t g8;                        // workgroups per XCD (grid / 8)
};

// Touches the fields the prologue needs at once, so that their scalar loads
// are issued together and waited for once instead of in dependent rounds
// (each a memory latency before the first weight load).
__device__ __forceinline__ void prefetch_args(const MfmaParams& p) {
  asm volatile("" ::"s"(p.w[0]), "s"(p.y[0]), "s"(p.n[0]), "s"(p.wg_end[0]), "s"(p.wg_end[1]),
               "s"(p.wg_end[2]), "s"(p.xq), "s"(p.ids), "s"(p.groups), "s"(p.total_wgs),
               "s"(p.m), "s"(p.tgroups), "s"(p.g8));
}

// Row blocks rounded up to a power of two (the summation tree's width).
__host__ __device__ constexpr int pow2_ceil(int v) {
  int r = 1;
  while (r < v) r <<= 1;
  return r;
}

// LDS layout (bytes) for row length k:
//   quants  [kTabSlots][k + 16]   slot stride padded by 16 bytes so the eight
//                                 token slots fall on different banks
//   d8      k/32 x kSlots fp64    in the order of d8_index
//   xchg    kXchgBytes            the second waves' subtree sums
__host__ __device__ constexpr uint32_t q_stride(int k) { return (uint32_t)k + 16u; }
__host__ __device__ constexpr uint32_t lds_d8_off(int k) { return kTabSlots * q_stride(k); }
__host__ __device__ constexpr uint32_t lds_xchg_off(int k) {
  return lds_d8_off(k) + (uint32_t)(k / 32) * kSlots * 8u;
}
__host__ __device__ constexpr uint32_t lds_bytes(int k) { return lds_xchg_off(k) + kXchgBytes; }
// Element index (fp64) of d8 of q8 block blk (within the row) of token t:
// [super-block][plane p][half h][token], so the four 32-byte reads of one
// plane (K-groups g = 2h + token/4) are 128 consecutive bytes.
__device__ __forceinline__ uint32_t d8_index(uint32_t blk, uint32_t t) {
  return (((blk >> 3) * 4u + (blk & 3u)) * 2u + ((blk >> 2) & 1u)) * 8u + t;
}

template <typename T>
__device__ __forceinline__ T lds_load(const uint8_t* base, uint32_t off) {
  return *reinterpret_cast<const T*>(base + off);
}

__device__ __forceinline__ uint32_t opaque_v(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Weight fields of one lane for one super-block.
struct Blk {
  u32x4 qs;     // qs[16g .. 16g + 15]
  u32x2 sc;     // scales[8(g>>1) .. 8(g>>1) + 7]
  uint32_t dd;  // d (low half), dmin (high half)
};

struct BlkOffsets {
  uint32_t q, s, d;
};

__device__ __forceinline__ Blk load_blk(const uint8_t* base, const BlkOffsets& o) {
  Blk x;
  x.qs = gload<u32x4_a4>(base + o.q);
  x.sc = gload<u32x2_a4>(base + o.s);
  x.dd = gload<uint32_t>(base + o.d);
  return x;
}

// The matrix, output and activations of one workgroup.
struct Job {
  const uint8_t* W;
  float* Y;    // output row 0; token t at Y + t * ldy
  XView X;
  int n;
  int ldy;
  int lwg;     // workgroup index within the job
  bool bad;    // expert id out of range: outputs NaN, error flag set
};

template <int k>
__device__ __forceinline__ Job resolve_job(const MfmaParams& p, int wgi) {
  Job J;
  J.bad = false;
  if (p.ids == nullptr && p.groups == 0) {
    const int j = (wgi >= p.wg_end[0]) + (wgi >= p.wg_end[1]) + (wgi >= p.wg_end[2]);
    J.lwg = wgi - (j > 0 ? p.wg_end[j - 1] : 0);
    J.W = p.w[j];
    J.Y = p.y[j];
    J.n = p.n[j];
    J.ldy = J.n;
    J.X = xview(p.xq, k, 0);
  } else if (p.groups > 0) {
    const int g = wgi / p.wgs_per_job;
    J.lwg = wgi - g * p.wgs_per_job;
    J.W = p.w[0] + (int64_t)g * p.expert_stride;
    J.n = p.n[0];
    J.ldy = p.groups * p.n[0];
    J.Y = p.y[0] + (int64_t)g * p.n[0];
    J.X = xview(p.xq, p.groups * k, g * k);
  } else {
    const int j = wgi / p.wgs_per_job;
    J.lwg = wgi - j * p.wgs_per_job;
    const int base = j / p.n_ids;
    const int i = j - base * p.n_ids;
    const int id = p.ids[i];
    J.bad = id < 0 || id >= p.n_experts;
    J.W = p.w[base] + (int64_t)(J.bad ? 0 : id) * p.expert_stride;
    J.n = p.n[0];
    J.ldy = J.n;
    J.Y = p.y[0] + (int64_t)j * p.m * J.n;
    J.X = xview(p.x_per_id ? p.xq + (int64_t)i * p.m * (int64_t)q8_row_bytes(k) : p.xq, k, 0);
  }
  return J;
}

// Staging of the activations of m tokens (k wide) in LDS, in two parts: the
// loads (stage_load), issued before the weight ring so that waiting for them
// does not wait for the weights (loads complete in issue order), and the LDS
// stores (stage_store). Every load is issued before the first store, so the
// staging costs one memory latency.
template <int k, int THREADS>
struct StageRegs {
  static constexpr int QC = k / 16;  // 16-byte quant chunks per token
  static constexpr int QIT = (kSlots * QC + THREADS - 1) / THREADS;
  static constexpr int C4 = k / 128;
  u32x4 qv[QIT];
  f32x4 d8v;
};

template <int k, int THREADS>
__device__ __forceinline__ StageRegs<k, THREADS> stage_load(const XView& X, int m) {
  using SR = StageRegs<k, THREADS>;
  static_assert(kSlots * SR::C4 <= THREADS, "one scale group per thread");
  SR r;
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < SR::QIT; ++it) {
    const int idx = tid + it * THREADS;
    const int t = idx / SR::QC, e = idx - (idx / SR::QC) * SR::QC;
    // Unconditional load (slots past m read token 0) and a select after it:
    // a load under a branch makes the compiler wait for it at the join,
    // which would serialise the staging loads.
    const bool ok = idx < kSlots * SR::QC && t < m;
    r.qv[it] = gload<u32x4>(ok ? X.q + t * X.stride + 16 * e : X.q);
  }
  // Scales: thread (token t2, group c4) takes q8 blocks 4c4..4c4+3.
  const int t2 = tid / SR::C4, c4 = tid - (tid / SR::C4) * SR::C4;
  const bool sv_ok = tid < kSlots * SR::C4 && t2 < m;
  r.d8v = gload<f32x4>(sv_ok ? X.s + t2 * X.stride + 16 * c4 : X.s);
  return r;
}

template <int k, int THREADS>
__device__ __forceinline__ void stage_store(uint8_t* lds, const StageRegs<k, THREADS>& r, int m) {
  using SR = StageRegs<k, THREADS>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < SR::QIT; ++it) {
    const int idx = tid + it * THREADS;
    const int t = idx / SR::QC, e = idx - (idx / SR::QC) * SR::QC;
    const u32x4 v = t < m ? r.qv[it] : u32x4{0, 0, 0, 0};
    if (idx < kSlots * SR::QC) *reinterpret_cast<u32x4*>(lds + t * q_stride(k) + 16 * e) = v;
  }
  for (int e = tid; e < SR::QC; e += THREADS)
    *reinterpret_cast<u32x4*>(lds + kSlots * q_stride(k) + 16 * e) = u32x4{0, 0, 0, 0};
  const int t2 = tid / SR::C4, c4 = tid - (tid / SR::C4) * SR::C4;
  if (tid < kSlots * SR::C4) {
    const bool live = t2 < m;
    double* d8t = reinterpret_cast<double*>(lds + lds_d8_off(k));
#pragma unroll
    for (int i = 0; i < 4; ++i) d8t[d8_index(4 * c4 + i, t2)] = live ? (double)r.d8v[i] : 0.0;
  }
}

// Workgroup barrier that orders LDS only: weight loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Per-lane constants of a tile.
struct Lane {
  int g, j16;
  uint32_t a_base;    // A operand (activation quants)
  uint32_t d8_base;   // d8 of the lane's four outputs
  uint32_t sc_shift;  // 8 * (g & 1)
};

template <int k>
__device__ __forceinline__ Lane lane_consts() {
  Lane L;
  const int lane = threadIdx.x & 63;
  L.g = lane >> 4;
  L.j16 = lane & 15;
  const int g = L.g, j16 = L.j16;
  // A: A-row j16 = token (j16 & 7), half (j16 >> 3); K-group g is non-zero
  // only in its own half (other lanes read the all-zero slot).
  const uint32_t a_slot = ((g >> 1) == (j16 >> 3)) ? (uint32_t)(j16 & 7) : (uint32_t)kSlots;
  L.a_base = opaque_v(a_slot * q_stride(k) + 128u * (g >> 1) + 16u * (g & 1));
  // d8 of the lane's four outputs: tokens 4(g&1) + 0..3 of q8 block 8b + 4(g>>1) + p.
  L.d8_base = opaque_v(lds_d8_off(k) + 32u * (uint32_t)g);
  L.sc_shift = 8u * (g & 1);
  return L;
}

// Logical right shift of a 64-bit register pair by a constant, as one
// v_lshrrev_b64: the compiler splits the shift into two 32-bit shifts when it
// sees that the bits crossing between the halves are masked off afterwards.
template <int S>
__device__ __forceinline__ uint64_t lshr64(uint64_t v) {
  uint64_t r;
  asm("v_lshrrev_b64 %0, %2, %1" : "=v"(r) : "v"(v), "n"(S));
  return r;
}

// B operand of plane pl: sc * q of the lane's 16 weights. scw holds the
// lane's scale bytes; sc is the 4-bit field at bit off. Two qs dwords are
// shifted at once: bits crossing from the high dword land in bits 26..31 of
// the low one (shift <= 6), which the 0x03 byte mask drops. Four masked
// quants times sc is sc * q in every byte (each at most 45, no carry), one
// v_mul_lo_u32 (a full-rate instruction on gfx950) per four weights.
template <int PL>
__device__ __forceinline__ v4i plane_weights(const u32x4& qs, uint32_t scw, uint32_t off) {
  const uint32_t sc = __builtin_amdgcn_ubfe(scw, off, 4);
  uint32_t sel[4];
  if constexpr (PL == 0) {
#pragma unroll
    for (int w = 0; w < 4; ++w) sel[w] = qs[w];
  } else {
    const uint64_t lo = lshr64<2 * PL>(((uint64_t)qs[1] << 32) | qs[0]);
    const uint64_t hi = lshr64<2 * PL>(((uint64_t)qs[3] << 32) | qs[2]);
    sel[0] = (uint32_t)lo;
    sel[1] = (uint32_t)(lo >> 32);
    sel[2] = (uint32_t)hi;
    sel[3] = (uint32_t)(hi >> 32);
  }
  v4i wq;
#pragma unroll
  for (int w = 0; w < 4; ++w) wq[w] = (int)((sel[w] & 0x03030303u) * sc);
  return wq;
}

// The subtree sums of one wave of a tile: super-blocks [KH * HB, KH * HB +
// HB) with HB = NBP/2 leaves, the leaves past the row (wave 1 only) +0.
// Wave 0 walks its blocks forward, wave 1 backward; a binary counter over
// the visiting order combines each pair of subtrees as soon as both exist
// (the same pairwise tree either way: addition is commutative). Writes the
// four tokens' sums to tot; with DOTS also every (I, M) of the lane.
template <int NB, int R, int KH, bool DOTS>
__device__ __forceinline__ void tile_half(const uint8_t* lds, const uint8_t* Wrow,
                                          const BlkOffsets& off, const Lane& L, Blk (&ring)[R],
                                          double tot[4], int32_t* dots, int m, int n, int row) {
  constexpr int NBP = pow2_ceil(NB);
  constexpr int HB = NBP / 2;
  constexpr int NR = KH == 0 ? HB : NB - HB;     // real blocks of this wave
  constexpr int PAD = HB - NR;                   // leading +0 leaves (wave 1)
  constexpr int LV = __builtin_ctz(HB) + 1;      // counter levels
  constexpr int k = NB * kBlockWeights;
  double stk[LV][4];
#pragma unroll
  for (int c = 0; c < HB; ++c) {
    double v[4];
    if (c < PAD) {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = 0.0;
    } else {
      const int q = c - PAD;                               // q-th real block visited
      const int b = KH == 0 ? q : NB - 1 - q;              // its index in the row
      const Blk cur = ring[q % R];
      if (q + R < NR) {
        const int bn = KH == 0 ? q + R : NB - 1 - (q + R);
        ring[q % R] = load_blk(Wrow + bn * kBlockBytes, off);
      }
      double fI[4] = {0.0, 0.0, 0.0, 0.0}, fM[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int pl = 0; pl < 4; ++pl) {
        const v4i aq = lds_load<v4i>(lds, L.a_base + 256u * b + 32u * pl);
        const uint32_t scw = cur.sc[pl >> 1], so = L.sc_shift + 16u * (pl & 1);
        const v4i wq = pl == 0 ? plane_weights<0>(cur.qs, scw, so)
                     : pl == 1 ? plane_weights<1>(cur.qs, scw, so)
                     : pl == 2 ? plane_weights<2>(cur.qs, scw, so)
                               : plane_weights<3>(cur.qs, scw, so);
        // the min nibble in all four bytes
        const int mb = (int)(__builtin_amdgcn_ubfe(scw, so + 4u, 4) * 0x01010101u);
        const v4i wm = v4i{mb, mb, mb, mb};
        const v4i cI = __builtin_amdgcn_mfma_i32_16x16x64_i8(aq, wq, v4i{0, 0, 0, 0}, 0, 0, 0);
        const v4i cM = __builtin_amdgcn_mfma_i32_16x16x64_i8(aq, wm, v4i{0, 0, 0, 0}, 0, 0, 0);
        const v4d d8 = lds_load<v4d>(lds, L.d8_base + 512u * b + 128u * pl);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          fI[i] = fma(d8[i], (double)cI[i], fI[i]);
          fM[i] = fma(d8[i], (double)cM[i], fM[i]);
        }
        if constexpr (DOTS) {
          const int c8 = 8 * b + 4 * (L.g >> 1) + pl;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = 4 * (L.g & 1) + i;
            if (t < m && row < n)
              *reinterpret_cast<u32x2*>(dots + (((int64_t)t * n + row) * (k / 32) + c8) * 2) =
                  u32x2{(uint32_t)cI[i], (uint32_t)cM[i]};
          }
        }
      }
      const double d = (double)fp16_bits_to_f32(cur.dd & 0xffffu);
      const double dmin = (double)fp16_bits_to_f32(cur.dd >> 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = half_value(d, dmin, fI[i], fM[i]);
    }
    // binary counter over the visiting order: visit c closes the subtrees
    // of its trailing one bits
    int lvl = 0;
#pragma unroll
    for (int l = 0; l < LV - 1; ++l) {
      if (((c >> l) & 1) == 0) break;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = stk[l][i] + v[i];
      lvl = l + 1;
    }
    // Pin the new subtree sum here: otherwise every super-block's epilogue
    // is sunk to its first use, keeping the MFMA results live.
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(v[i]));
#pragma unroll
    for (int l = 0; l < LV; ++l)
      if (l == lvl) {
#pragma unroll
        for (int i = 0; i < 4; ++i) stk[l][i] = v[i];
      }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) tot[i] = stk[LV - 1][i];
}

}  // namespace

// Sixteen waves per workgroup: wave w takes tile w & 7, super-block half
// w >> 3 (see tile_half). The first waves add the second waves' subtree sums
// (received through LDS) to their own, then the two halves are added across
// lanes g and g ^ 2, so the result does not depend on timing and is the same
// as the packed-dot kernels'.
//
// The leading scalar arguments describe the whole launch when it is one
// matrix (plain != 0); they are preloaded into SGPRs at wave launch
// (kernel-argument preloading), so that case starts its loads without
// reading the argument block.
template <int NB, int R, bool DOTS>
__global__ __launch_bounds__(kThreads) void mmvq_mfma_kernel(const uint8_t* w0, const uint8_t* xq0,
                                                             float* y0, int32_t n0, int32_t m_all,
                                                             int32_t tgroups, int32_t total_wgs,
                                                             int32_t g8, int32_t plain,
                                                             const MfmaParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int k = NB * kBlockWeights;
  constexpr int HB = pow2_ceil(NB) / 2;
  static_assert(NB > HB && NB <= 2 * HB, "two waves per tile");
  constexpr uint32_t rowbytes = (uint32_t)NB * kBlockBytes;
  const int wgi = (blockIdx.x & 7) * g8 + (blockIdx.x >> 3);   // XCD-major workgroup index
  if (wgi >= total_wgs) return;                                // whole workgroup
  // Token group tg of a row block: its kSlots tokens (fewer in the last
  // group). The groups of one block are consecutive workgroups, so they run
  // together on one XCD and read the block's weights through its L2.
  const int job_wg = wgi / tgroups;
  const int tg = wgi - job_wg * tgroups;
  Job J;
  if (plain) {
    J.W = w0;
    J.Y = y0;
    J.X = xview(xq0, k, 0);
    J.n = n0;
    J.ldy = n0;
    J.lwg = job_wg;
    J.bad = false;
  } else {
    prefetch_args(p);
    J = resolve_job<k>(p, job_wg);
  }
  const int m = min(kSlots, m_all - kSlots * tg);
  {
    const int64_t t0 = (int64_t)kSlots * tg;
    J.X.q += t0 * J.X.stride;
    J.X.s += t0 * J.X.stride;
    J.X.m += t0 * J.X.stride;
    J.Y += t0 * J.ldy;
  }

  const int wiw = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int tw = wiw & (kTilesPerWg - 1);
  const int kh = wiw >> 3;
  const int tiles = (J.n + 15) >> 4;
  const int tile_raw = J.lwg * kTilesPerWg + tw;
  const bool active = tile_raw < tiles;                        // wave-uniform
  const int r0 = (active ? tile_raw : tiles - 1) * 16;
  const Lane L = lane_consts<k>();
  const uint32_t lrow = (uint32_t)(min(r0 + L.j16, J.n - 1) - r0);
  const uint8_t* Wt = J.W + (size_t)r0 * rowbytes;
  const BlkOffsets off{opaque_v(lrow * rowbytes + 16u + 16u * L.g), opaque_v(lrow * rowbytes + 8u * (L.g >> 1)),
                       opaque_v(lrow * rowbytes + 80u)};
  const StageRegs<k, kThreads> staged = stage_load<k, kThreads>(J.X, m);
  // the first R blocks of this wave's visiting order
  Blk ring[R];
  if (kh == 0) {
#pragma unroll
    for (int q = 0; q < R; ++q) ring[q] = load_blk(Wt + q * kBlockBytes, off);
  } else {
#pragma unroll
    for (int q = 0; q < R; ++q)
      if (q < NB - HB) ring[q] = load_blk(Wt + (NB - 1 - q) * kBlockBytes, off);
  }

  stage_store<k, kThreads>(lds, staged, m);
  lds_barrier();

  double tot[4] = {0.0, 0.0, 0.0, 0.0};
  const int row = r0 + L.j16;
  // DOTS (one matrix): this token group's (I, M) start kSlots * tg tokens in
  int32_t* const dots = DOTS ? p.dots + (int64_t)kSlots * tg * J.n * (k / 32) * 2 : nullptr;
  if (active) {
    if (kh == 0)
      tile_half<NB, R, 0, DOTS>(lds, Wt, off, L, ring, tot, dots, m, J.n, row);
    else
      tile_half<NB, R, 1, DOTS>(lds, Wt, off, L, ring, tot, dots, m, J.n, row);
  }

  // Second waves -> LDS -> first waves: left + right subtree, then the halves.
  double* xchg = reinterpret_cast<double*>(lds + lds_xchg_off(k));
  const int slot = (tw * kWave + (int)(threadIdx.x & 63)) * 4;
  if (kh == 1 && active) {
#pragma unroll
    for (int i = 0; i < 4; ++i) xchg[slot + i] = tot[i];
  }
  lds_barrier();
  if (kh == 0 && active && !DOTS) {
    double yv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double t = tot[i] + xchg[slot + i];
      yv[i] = halve<32>(t, t, (int)(threadIdx.x & 63));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int token = 4 * L.g + i;
      if (L.g < 2 && token < m && row < J.n)
        J.Y[(int64_t)token * J.ldy + row] = J.bad ? quiet_nan() : (float)yv[i];
    }
  }
  if (J.bad && threadIdx.x == 0 && p.err_flag != nullptr) *p.err_flag = 1;
}

namespace {

constexpr int kRing = 2;

int nb_slot(int nb) {
  switch (nb) {
    case 4: return 0;
    case 8: return 1;
    case 16: return 2;
    case 28: return 3;
    default: return -1;
  }
}

template <int NB, bool DOTS>
hipError_t launch_nb(const MfmaParams& p, dim3 gd, size_t shm, hipStream_t stream) {
  // More than 64 KB of dynamic LDS must be allowed explicitly, once per
  // device and kernel.
  static bool set_for[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!set_for[dev]) {
    const hipError_t e = hipFuncSetAttribute((const void*)mmvq_mfma_kernel<NB, kRing, DOTS>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMfmaMaxLds);
    if (e != hipSuccess) return e;
    set_for[dev] = true;
  }
  const int32_t plain = (p.ids == nullptr && p.groups == 0 && p.wg_end[0] * p.tgroups == p.total_wgs) ? 1 : 0;
  hipLaunchKernelGGL((mmvq_mfma_kernel<NB, kRing, DOTS>), gd, dim3(kThreads), shm, stream, p.w[0], p.xq,
                     p.y[0], p.n[0], p.m, p.tgroups, p.total_wgs, p.g8, plain, p);
  return hipGetLastError();
}

int64_t workgroups(const MmvqLaunch& a) {
  const int tile_rows = 16 * kTilesPerWg;
  if (uniform_jobs(a)) return (int64_t)((a.n[0] + tile_rows - 1) / tile_rows) * a.njobs * a.n_ids;
  int64_t total = 0;
  for (int j = 0; j < a.njobs; ++j) total += (a.n[j] + tile_rows - 1) / tile_rows;
  return total;
}

}  // namespace

bool mfma_supports(int k) {
  return nb_slot(k / kBlockWeights) >= 0 && lds_bytes(k) <= kMfmaMaxLds;
}

bool mfma_preferred(const MmvqLaunch& a) {
  // More than kSlots tokens always go to the matrix cores when they can.
  // Otherwise the faster of two measured cost models (one MI355X, microseconds
  // over a fixed ~4 us of launch and latency):
  //  * matrix cores: ~0.75 us per super-block of a row for every round of
  //    up to 256 workgroups (one workgroup per CU: LDS), whatever m is;
  //  * packed dots with the tokens split over waves: ~1e-5 us per
  //    (row, super-block, token), all of it vector-ALU issue.
  // The choice changes no result bit (every kernel sums in the same order).
  if (!mfma_supports(a.k) || a.m < 2) return false;
  if (a.m > kSlots) return true;
  const int nb = a.k / kBlockWeights;
  int64_t rows = 0;
  if (uniform_jobs(a)) {
    rows = (int64_t)a.n[0] * a.njobs * a.n_ids;
  } else {
    for (int j = 0; j < a.njobs; ++j) rows += a.n[j];
  }
  const double rounds = (double)((workgroups(a) + 255) / 256);
  const double t_mfma = 0.75 * nb * rounds;
  const double t_dots = 1e-5 * (double)rows * nb * a.m;
  return t_mfma < t_dots;
}

hipError_t launch_mmvq_mfma(const MmvqLaunch& a, hipStream_t stream) {
  const int nb = a.k / kBlockWeights;
  const int which = nb_slot(nb);
  if (which < 0) return hipErrorInvalidValue;
  const bool dots = a.dots != nullptr;
  if (dots && (uniform_jobs(a) || a.njobs != 1)) return hipErrorInvalidValue;
  MfmaParams p{};
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
  p.m = a.m;
  p.tgroups = (a.m + kSlots - 1) / kSlots;

  // Eight consecutive 16-row tiles per workgroup.
  const int tile_rows = 16 * kTilesPerWg;
  int64_t total_wgs = 0;
  if (!uniform_jobs(a)) {
    for (int j = 0; j < kMaxPlainJobs; ++j) {
      if (j < a.njobs) total_wgs += (a.n[j] + tile_rows - 1) / tile_rows;
      p.wg_end[j] = (int)total_wgs;
    }
  } else {
    p.wgs_per_job = (a.n[0] + tile_rows - 1) / tile_rows;
    total_wgs = (int64_t)p.wgs_per_job * a.njobs * a.n_ids;
  }
  if (total_wgs == 0) return hipSuccess;
  total_wgs *= p.tgroups;
  if (total_wgs > INT32_MAX - 8) return hipErrorInvalidValue;
  p.total_wgs = (int)total_wgs;
  const dim3 gd((unsigned)((total_wgs + 7) / 8 * 8));
  p.g8 = (int)(gd.x / 8);
  const size_t shm = lds_bytes(a.k);
#define Q2K_NB(NBV) (dots ? launch_nb<NBV, true>(p, gd, shm, stream) : launch_nb<NBV, false>(p, gd, shm, stream))
  switch (which) {
    case 0: return Q2K_NB(4);
    case 1: return Q2K_NB(8);
    case 2: return Q2K_NB(16);
    default: return Q2K_NB(28);
  }
#undef Q2K_NB
}

}  // namespace q2k
