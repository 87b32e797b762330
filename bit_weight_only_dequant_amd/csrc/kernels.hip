// kernels.hip - HIP kernels for gfx950 (CDNA4) and the device entry points of
// libqgemm: y = x . dequant(W)^T for low-bit group-quantized weights.
//
// The operation is the dequantizing matmul of the skyzh/tiny-llm feature list
// ("Dequantizing Runtimes", "Quantized Matrix Multiplication"): weights are
// brought back to full precision inside the compute pass, never written out.
// Formats: INT4 / INT2 with per-group fp16 scale and zero point (TinyLoop
// README, "Status" and "Current Runtime Snapshot"), q4_0, q8_0 and the k-quant
// q4k (torchnative guide "Inference with real transformers", "Quantise while
// loading").
//
// Kernels
//   qpack / qunpack      one-time permutation of codes into the tile order of
//                        layout.h (HBM-bound, elementwise).
//   gemv<FMT, 1>         M == 1.  Bandwidth-bound.  One 16-byte code load per
//                        lane per 16x16-word tile, unpack by mask into fp16
//                        pairs holding exact (q - z), v_dot2_f32_f16 against x
//                        that each wave stages for itself in LDS, fp32 scale
//                        per 32 codes (q8_0: 16; q4k: d*sc and the offset
//                        dmin*m times the run's x sum), lane groups summed by
//                        DPP and ds_swizzle, waves through LDS.
//   gemv_half<FMT, R>    M <= 4 when 16-row workgroups would load the CUs
//                        unevenly (N = 6144: 384 blocks on 256 CUs): the same
//                        work on 8-row workgroups, twice as many.
//   gemv_mfma<FMT, R>    2 <= M <= 16.  Same loads and staging; every 8 codes,
//                        dequantized to fp16 weights, are one
//                        v_mfma_f32_16x16x32_f16 step (the packed layout is
//                        that MFMA's B operand), so the VALU work per code
//                        does not grow with M.
//   gemm<FMT>            M > 16.  64x64 workgroup tile; 8 waves split K and
//                        are summed through LDS.  x and codes stream into
//                        per-wave LDS rings with direct loads; codes are
//                        dequantized once per workgroup to fp16 weights in
//                        registers and fed to v_mfma_f32_32x32x16_f16.
//   dequant<FMT>         the same fp16 weights written out (debug, and the
//                        dequantize-at-load comparison).
//   Split-K (both)       fp32 partials in a workspace, summed in split order by a
//                        second small kernel (deterministic).  A kernel boundary
//                        orders the partials; an in-kernel device-scope fence
//                        per workgroup would write back the whole L2 each time.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <climits>
#include <mutex>
#include <vector>

#include "../../include/qgemm.h"
#include "internal.h"
#include "layout.h"

namespace qg {

typedef _Float16 f16;
typedef f16 h2 __attribute__((ext_vector_type(2)));
typedef f16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// unpack + dequant primitives
// ---------------------------------------------------------------------------
// A code c sits in a 16-bit half as c << (b*i).  OR-ing in 0x6400 (fp16 1024.0,
// whose unit in the last place is 1) gives the fp16 value 1024 + c*2^(b*i)
// exactly.  Scaling by 2^-(b*i) and adding -(1024*2^-(b*i) + z) leaves the
// exact small integer c - z (all intermediate values are integers below 2048,
// so no rounding happens).  With z an integer in [0, 2^b - 1] the pair
// (c_2i - z, c_2i+1 - z) is exact in fp16; one multiply by s then gives
// fp16_rne(s * (q - z)).

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ h2 splat(f16 v) { return h2{v, v}; }

// Zero-point constants for one group: zc[i] = -(1024 * 2^-(b*i) + z)
struct ZC4 { h2 c0, c1; };          // 4-bit: i = 0 (x1), 1 (x16)
struct ZC2 { h2 c0, c1, c2, c3; };  // 2-bit: x1, x4, x16, x64
struct ZC8 { h2 c0; };              // 8-bit: a byte fills the low 8 mantissa bits

__device__ __forceinline__ ZC8 make_zc8(f16 z) {
  ZC8 r;
  r.c0 = splat((f16)-1024.0f - z);
  return r;
}

__device__ __forceinline__ ZC4 make_zc4(f16 z) {
  ZC4 r;
  r.c0 = splat((f16)-1024.0f - z);
  r.c1 = splat((f16)-64.0f - z);
  return r;
}
__device__ __forceinline__ ZC2 make_zc2(f16 z) {
  ZC2 r;
  r.c0 = splat((f16)-1024.0f - z);
  r.c1 = splat((f16)-256.0f - z);
  r.c2 = splat((f16)-64.0f - z);
  r.c3 = splat((f16)-16.0f - z);
  return r;
}

// (w & m) | c as one VOP3 instruction.  With both constants literal the
// compiler emits v_and + v_or, since VOP3 on this target takes no literal;
// here the mask sits in an SGPR and the magic in a VGPR.
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t m, uint32_t c) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(w), "s"(m), "v"(c));
  return d;
}

// 4-bit packed word (8 codes) -> 4 pairs (c_2i - z, c_2i+1 - z), i = 0..3
__device__ __forceinline__ void qmz_int4(uint32_t w, const ZC4& zc, h2 out[4]) {
  const uint32_t magic = 0x64006400u, w8 = w >> 8;
  const h2 inv16 = splat((f16)0.0625f);
  out[0] = as_h2(and_or(w, 0x000F000Fu, magic)) + zc.c0;
  out[1] = as_h2(and_or(w, 0x00F000F0u, magic)) * inv16 + zc.c1;
  out[2] = as_h2(and_or(w8, 0x000F000Fu, magic)) + zc.c0;
  out[3] = as_h2(and_or(w8, 0x00F000F0u, magic)) * inv16 + zc.c1;
}

// 2-bit packed word, one half (8 codes): half 0 = codes 0..7, half 1 = 8..15
__device__ __forceinline__ void qmz_int2_half(uint32_t w, int half, const ZC2& zc, h2 out[4]) {
  const uint32_t magic = 0x64006400u, v = half ? (w >> 8) : w;
  out[0] = as_h2(and_or(v, 0x00030003u, magic)) + zc.c0;
  out[1] = as_h2(and_or(v, 0x000C000Cu, magic)) * splat((f16)0.25f) + zc.c1;
  out[2] = as_h2(and_or(v, 0x00300030u, magic)) * splat((f16)0.0625f) + zc.c2;
  out[3] = as_h2(and_or(v, 0x00C000C0u, magic)) * splat((f16)0.015625f) + zc.c3;
}

// 8-bit packed word (4 codes) -> 2 pairs (c_0 - z, c_1 - z), (c_2 - z, c_3 - z):
// the word holds codes 0, 2, 1, 3 in bytes 0..3, so masking bytes 0 and 2
// gives the first pair and, after a shift by 8, bytes 1 and 3 the second
// (1024 + u is exact in fp16 for u <= 255)
__device__ __forceinline__ void qmz_int8(uint32_t w, const ZC8& zc, h2 out[2]) {
  const uint32_t magic = 0x64006400u;
  out[0] = as_h2(and_or(w, 0x00FF00FFu, magic)) + zc.c0;
  out[1] = as_h2(and_or(w >> 8, 0x00FF00FFu, magic)) + zc.c0;
}

// Per format: bits, codes per word, codes per 16-byte lane chunk (LS), K per
// word tile (KT), codes per scale lookup (SW: a lane's chunk in runs of at
// most 32, the smallest group), runs per chunk (NSEG), the implicit zero
// point of the block formats as fp16 bits (8.0 and 128.0), and KQ for the
// k-quant q4k (codes unpacked with zero point 0; per 32-code sub-block a
// scale d*sc and an offset dmin*m instead of (s, z)).
template <int FMT> struct Fmt;
template <> struct Fmt<INT4_ASYM> { static constexpr int BITS = 4, CPW = 8,  LS = 32, KT = 128, SW = 32, NSEG = 1; static constexpr bool HAS_Z = true,  KQ = false; static constexpr uint32_t ZBITS = 0; };
template <> struct Fmt<INT2_ASYM> { static constexpr int BITS = 2, CPW = 16, LS = 64, KT = 256, SW = 32, NSEG = 2; static constexpr bool HAS_Z = true,  KQ = false; static constexpr uint32_t ZBITS = 0; };
template <> struct Fmt<Q4_0>      { static constexpr int BITS = 4, CPW = 8,  LS = 32, KT = 128, SW = 32, NSEG = 1; static constexpr bool HAS_Z = false, KQ = false; static constexpr uint32_t ZBITS = 0x4800; };
template <> struct Fmt<Q8_0>      { static constexpr int BITS = 8, CPW = 4,  LS = 16, KT = 64,  SW = 16, NSEG = 1; static constexpr bool HAS_Z = false, KQ = false; static constexpr uint32_t ZBITS = 0x5800; };
template <> struct Fmt<Q4K>       { static constexpr int BITS = 4, CPW = 8,  LS = 32, KT = 128, SW = 32, NSEG = 1; static constexpr bool HAS_Z = false, KQ = true;  static constexpr uint32_t ZBITS = 0; };

// q4k sub-block terms from the super-block pair ddm = d | dmin << 16 (fp16
// bits) and the sub-block bytes scm = sc | m << 8.  In fp32 they are exact
// (an fp16 value times a 6-bit integer): (d*sc, dmin*m).  For the fp16
// weight w = fma(q, fp16(d*sc), -fp16(dmin*m)) each is rounded once to
// fp16, returned as (bits of fp16(d*sc)) | (bits of -fp16(dmin*m)) << 16.
__device__ __forceinline__ float2 kq_terms(uint32_t ddm, uint32_t scm) {
  const float d = (float)__builtin_bit_cast(f16, (uint16_t)(ddm & 0xffffu));
  const float dmin = (float)__builtin_bit_cast(f16, (uint16_t)(ddm >> 16));
  return float2{d * (float)(scm & 0xffu), dmin * (float)((scm >> 8) & 0xffu)};
}
__device__ __forceinline__ uint32_t kq_half_pair(uint32_t ddm, uint32_t scm) {
  const float2 t = kq_terms(ddm, scm);
  const uint32_t ds = __builtin_bit_cast(uint16_t, (f16)t.x);
  const uint32_t nb = __builtin_bit_cast(uint16_t, (f16)(-t.y));
  return ds | (nb << 16);
}
// fp16 q4k weights of n pairs of exact codes: fma(q, ds, nb), one rounding
__device__ __forceinline__ void kq_weights(const h2* q, uint32_t dsnb, h2* w, int n) {
  const h2 ds = splat(__builtin_bit_cast(f16, (uint16_t)(dsnb & 0xffffu)));
  const h2 nb = splat(__builtin_bit_cast(f16, (uint16_t)(dsnb >> 16)));
#pragma unroll
  for (int i = 0; i < n; ++i) w[i] = __builtin_elementwise_fma(q[i], ds, nb);
}

// Exact (q - z) pairs, in k order, of run p (SW codes) of a lane's chunk c
template <int FMT>
__device__ __forceinline__ void run_qmz(const u4& c, int p, f16 z, h2* q) {
  if constexpr (FMT == INT2_ASYM) {
    const ZC2 zc = make_zc2(z);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int h = 0; h < 2; ++h) qmz_int2_half(c[2 * p + t], h, zc, q + 8 * t + 4 * h);
  } else if constexpr (FMT == Q8_0) {
    const ZC8 zc = make_zc8(z);
#pragma unroll
    for (int t = 0; t < 4; ++t) qmz_int8(c[t], zc, q + 2 * t);
  } else {
    const ZC4 zc = make_zc4(z);
#pragma unroll
    for (int t = 0; t < 4; ++t) qmz_int4(c[t], zc, q + 4 * t);
  }
}

// ---------------------------------------------------------------------------
// repack kernels
// ---------------------------------------------------------------------------
__global__ void qpack_kernel(const uint32_t* __restrict__ canon, uint32_t* __restrict__ packed,
                             int N, int Kw, int wordtiles, int bits, int64_t total) {
  for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < total;
       p += (int64_t)gridDim.x * blockDim.x) {
    const int t = (int)(p & 3);
    const int lane = (int)((p >> 2) & 63);
    const int64_t rest = p >> 8;
    const int64_t T = rest % wordtiles, rb = rest / wordtiles;
    const int64_t n = rb * 16 + (lane & 15);
    const int64_t kw = T * 16 + (lane >> 4) * 4 + t;
    uint32_t v = 0;
    if (n < N && kw < Kw) v = perm_word(canon[n * Kw + kw], bits);
    packed[p] = v;
  }
}

__global__ void qunpack_kernel(const uint32_t* __restrict__ packed, uint32_t* __restrict__ canon,
                               int N, int Kw, int wordtiles, int bits) {
  const int64_t total = (int64_t)N * Kw;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = i / Kw, kw = i % Kw;
    canon[i] = unperm_word(packed[packed_index(n, kw, wordtiles)], bits);
  }
}

__global__ void unpack_codes_kernel(const uint32_t* __restrict__ packed, uint8_t* __restrict__ codes,
                                    int N, int K, int wordtiles, int bits) {
  const int cpw = 32 / bits;
  const int64_t total = (int64_t)N * K;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = i / K, k = i % K;
    const uint32_t w = packed[packed_index(n, k / cpw, wordtiles)];
    const int slot = code_slot((int)(k % cpw), cpw);
    codes[i] = (uint8_t)((w >> (bits * slot)) & ((1u << bits) - 1u));
  }
}

// Dequantized weights written out (fp16 [N, K]), with the GEMM's register
// dequant: one wave per (row block, word tile), so each wave reads 1 KiB of
// codes contiguously; lane (g, r) turns its 16-byte chunk into 32 (4-bit), 64
// (INT2) or 16 (q8_0) weights of row 16*rb + r.  The wave's 16-row tile goes
// through LDS (rows padded by 16 bytes against bank conflicts) and is stored
// row by row, 16 bytes per lane, so each store instruction writes whole
// 64-to-256-byte row segments instead of 16 bytes per 64.
template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t* __restrict__ packed,
                                                      const f16* __restrict__ scales,
                                                      const f16* __restrict__ zeros, f16* __restrict__ w,
                                                      int N, int K, int group, int wordtiles, int64_t units) {
  using F = Fmt<FMT>;
  constexpr int KTP = F::KT + 8;                 // padded tile row, in halves
  constexpr int TB = 16 * KTP * 2;               // tile bytes per wave
  constexpr int LPR = F::KT / 8;                 // lanes per row when storing (16 bytes each)
  constexpr int ROUNDS = 16 * LPR / 64;          // store instructions per lane
  __shared__ __align__(16) uint8_t deq_smem[4 * TB];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t unit = (int64_t)blockIdx.x * 4 + wv;
  if (unit >= units) return;                     // the whole wave
  const int64_t rb = unit / wordtiles;
  const int T = (int)(unit - rb * wordtiles);
  const int g = lane >> 4, r = lane & 15;
  const int64_t n = rb * 16 + r;
  f16* tl = reinterpret_cast<f16*>(deq_smem + wv * TB);   // [16 rows][KTP]
  const u4 c = reinterpret_cast<const u4*>(packed)[unit * 64 + lane];
  const int ng = K / group;   // q4k: group = 32, the sub-block
#pragma unroll
  for (int p = 0; p < F::NSEG; ++p) {
    const int kl = g * F::LS + p * F::SW;          // this lane's first code inside the tile
    const int k = T * F::KT + kl;
    if (n >= N || k >= K) continue;
    const int grp = k / group;
    h2 q[F::SW / 2];
    h2 wq[F::SW / 2];
    if constexpr (F::KQ) {
      const uint32_t ddm = reinterpret_cast<const uint32_t*>(scales)[n * (ng >> 3) + (grp >> 3)];
      const uint32_t scm = reinterpret_cast<const uint16_t*>(zeros)[n * ng + grp];
      run_qmz<FMT>(c, p, (f16)0.0f, q);
      kq_weights(q, kq_half_pair(ddm, scm), wq, F::SW / 2);
    } else {
      const h2 s2 = splat(scales[n * ng + grp]);
      const f16 z = F::HAS_Z ? zeros[n * ng + grp] : __builtin_bit_cast(f16, (uint16_t)F::ZBITS);
      run_qmz<FMT>(c, p, z, q);
#pragma unroll
      for (int i = 0; i < F::SW / 2; ++i) wq[i] = q[i] * s2;
    }
    h8* dst = reinterpret_cast<h8*>(tl + r * KTP + kl);
#pragma unroll
    for (int v = 0; v < F::SW / 8; ++v)
      dst[v] = h8{wq[4 * v][0], wq[4 * v][1], wq[4 * v + 1][0], wq[4 * v + 1][1],
                  wq[4 * v + 2][0], wq[4 * v + 2][1], wq[4 * v + 3][0], wq[4 * v + 3][1]};
  }
  // only this wave reads its tile: a wave-level barrier orders the LDS traffic
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int v = 0; v < ROUNDS; ++v) {
    const int idx = v * 64 + lane;
    const int row = idx / LPR, ch = idx % LPR;
    const int64_t nn = rb * 16 + row;
    const int kk = T * F::KT + ch * 8;
    if (nn < N && kk < K)
      *reinterpret_cast<h8*>(w + nn * K + kk) = *reinterpret_cast<const h8*>(tl + row * KTP + ch * 8);
  }
}

__global__ void fill_zero_kernel(f16* __restrict__ y, int M, int N, int ldy,
                                 const f16* __restrict__ resid, int ldr) {
  const int64_t total = (int64_t)M * N;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = i / N, n = i % N;
    y[m * ldy + n] = resid ? resid[m * ldr + n] : (f16)0.0f;
  }
}

// ---------------------------------------------------------------------------
// decode GEMV (M <= 16)
// ---------------------------------------------------------------------------
struct GemvArgs {
  const f16* x; const uint32_t* packed; const f16* scales; const f16* zeros;
  const f16* resid; f16* y; float* ws;
  int ldx, ldr, ldy, M, N, K, group;
  int wordtiles, rowblocks, splits, tps;
};

// v plus its value in lane l ^ 8: a DPP rotate of each 16-lane row by 8 (no
// LDS round trip, no lane-index arithmetic)
__device__ __forceinline__ float add_lane_xor8(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false));
}

// v plus its value in lane l ^ 16: ds_swizzle in bit mode (and 0x1f, xor 0x10)
__device__ __forceinline__ float add_lane_xor16(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401f));
}

// LDS bytes of gemv_kernel: per wave its x slice, (scale, zero) pairs (q4k:
// fp32 (d*sc, dmin*m)) and, for q4k, the x sum of each 32-wide run; then the
// cross-wave sums
template <int FMT> constexpr size_t gemv_lds_bytes_for(int mmax, int tpw, int nw) {
  const int KW = tpw * Fmt<FMT>::KT;
  const int SZB = Fmt<FMT>::KQ ? 8 : 4;
  const int XSB = Fmt<FMT>::KQ ? mmax * (KW / 32) * 4 : 0;
  return (size_t)nw * (mmax * KW * 2 + 16 * (KW / 32) * SZB + XSB) + (size_t)nw * mmax * 32 * sizeof(float);
}
template <int FMT, int MMAX, int TPW, int NW> constexpr size_t gemv_lds_bytes() {
  return gemv_lds_bytes_for<FMT>(MMAX, TPW, NW);
}

// Decode GEMV (used for M == 1).  Workgroup = one 16-row block (x one K split); its NW
// waves (8 or 16) take consecutive runs of word tiles.  Each wave stages only its own x
// slice and (scale, zero) pairs in its own LDS region, so no wave waits for
// another until the final sum.  Per lane and tile: one 16-byte code load,
// masks into fp16 pairs holding exact (q - z) (one v_and_or_b32 plus one
// packed add or fma per pair), v_dot2_f32_f16 against fp16 x pairs, the fp32
// scale once per run of SW codes (32; 16 for q8_0).  q4k: exact q, then
// d*sc * (x . q) - dmin*m * sum(x) per 32-code sub-block, all in fp32.
template <int FMT, int MMAX, int TPW, int NW>
__global__ __launch_bounds__(NW * 64) void gemv_kernel(GemvArgs a) {
  using F = Fmt<FMT>;
  constexpr int KW = TPW * F::KT;              // k range of one wave
  constexpr int GWMAX = KW / 32;               // groups per wave, at most (group >= 32)
  constexpr int XCH = MMAX * KW / 8;           // 16-byte x chunks per wave
  constexpr int NXC = (XCH + 63) / 64;
  constexpr int NSZ = (16 * GWMAX + 63) / 64;  // (scale, zero) loads per lane, at most
  constexpr int SZB = F::KQ ? 8 : 4;
  constexpr int XB = MMAX * KW * 2, SB = 16 * GWMAX * SZB;
  constexpr int WB = XB + SB + (F::KQ ? MMAX * GWMAX * 4 : 0);
  __shared__ __align__(16) uint8_t gemv_smem[gemv_lds_bytes<FMT, MMAX, TPW, NW>()];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  f16* xs = reinterpret_cast<f16*>(gemv_smem + wave * WB);                 // [MMAX][KW]
  uint32_t* sz = reinterpret_cast<uint32_t*>(gemv_smem + wave * WB + XB);  // [16][GWMAX] s | z << 16
  float2* szk = reinterpret_cast<float2*>(gemv_smem + wave * WB + XB);     // q4k: [16][GWMAX] (d*sc, dmin*m)
  float* xsum = reinterpret_cast<float*>(gemv_smem + wave * WB + XB + SB); // q4k: [MMAX][GWMAX]
  float* red = reinterpret_cast<float*>(gemv_smem + NW * WB);              // [NW][MMAX][2][16]

  const int g = lane >> 4, r = lane & 15;
  const int rb = blockIdx.x, split = blockIdx.y;
  const int T0 = split * a.tps, T1 = min(a.wordtiles, T0 + a.tps);
  const int tpw = (T1 - T0 + NW - 1) / NW;           // <= TPW (the launch picks TPW)
  const int wt0 = T0 + wave * tpw;
  const int nt = max(0, min(T1, wt0 + tpw) - wt0);   // word tiles of this wave
  const int k0 = wt0 * F::KT;                         // a group boundary (KT % group == 0)
  const int lg = __builtin_ctz(a.group);
  const int ng = a.K >> lg;
  const int gstride = KW >> lg;                       // groups per full wave, a power of two
  const int lgs = __builtin_ctz(gstride);
  const int gs0 = k0 >> lg;

  // 1. Every global load first, with no branches (offsets of out-of-range
  //    entries clamped to 0, values masked later): scales and zeros, the
  //    residual, this wave's x slice, then its code tiles.
  const int64_t szbase = (int64_t)rb * 16 * ng * 2;
  // q4k: the (d, dmin) pair of each super-block (8 sub-blocks) as 32 bits,
  // so a row block's pairs start at rb * 16 * (ng / 8) * 4 bytes
  const char* sp = reinterpret_cast<const char*>(a.scales) + (F::KQ ? szbase / 4 : szbase);
  const char* zp = reinterpret_cast<const char*>(F::HAS_Z || F::KQ ? a.zeros : a.scales) + szbase;
  uint32_t sraw[NSZ], zraw[NSZ];
#pragma unroll
  for (int j = 0; j < NSZ; ++j) {
    const int e = lane + 64 * j;  // entry (row e >> lgs, group gs0 + e % gstride)
    const int er = e >> lgs, eg = gs0 + (e & (gstride - 1));
    const bool ok = e < 16 * gstride && rb * 16 + er < a.N && eg < ng;
    const uint32_t off = ok ? (uint32_t)(er * ng + eg) * 2u : 0u;
    if constexpr (F::KQ) {
      sraw[j] = *reinterpret_cast<const uint32_t*>(sp + (ok ? (uint32_t)(er * (ng >> 3) + (eg >> 3)) * 4u : 0u));
      zraw[j] = *reinterpret_cast<const uint16_t*>(zp + off);
    } else {
      sraw[j] = *reinterpret_cast<const uint16_t*>(sp + off);
      if constexpr (F::HAS_Z) zraw[j] = *reinterpret_cast<const uint16_t*>(zp + off);
      else zraw[j] = F::ZBITS;  // the implicit zero point
    }
  }
  const int om = tid >> 5, orow = tid & 15;   // output of thread tid < 32 MMAX (final sum)
  // residual, fp16 bits: loaded unconditionally (from x when there is none,
  // dropped at the store), since a load under a branch made the compiler
  // wait for it, and for every load before it, ahead of the x and code loads
  const bool has_res = a.resid && a.splits == 1;
  const uint32_t res = has_res ? reinterpret_cast<const uint16_t*>(a.resid)[(int64_t)min(om, a.M - 1) * a.ldr +
                                                                           min(rb * 16 + orow, a.N - 1)]
                               : reinterpret_cast<const uint16_t*>(a.x)[0];
  __builtin_amdgcn_sched_barrier(0);
  u4 xr[NXC];
#pragma unroll
  for (int j = 0; j < NXC; ++j) {
    const int c = lane + 64 * j;
    const int m = c / (KW / 8), k = k0 + (c % (KW / 8)) * 8;
    const bool ok = c < XCH && m < a.M && k < a.K;
    const uint32_t off = ok ? (uint32_t)(m * a.ldx + k) * 2u : 0u;
    xr[j] = *reinterpret_cast<const u4*>(reinterpret_cast<const char*>(a.x) + off);
  }
  __builtin_amdgcn_sched_barrier(0);
  u4 code[TPW];
  const char* pkrow = reinterpret_cast<const char*>(a.packed) + (int64_t)rb * a.wordtiles * 1024;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int T = min(wt0 + i, a.wordtiles - 1);
    code[i] = *reinterpret_cast<const u4*>(pkrow + (uint32_t)(T * 1024 + lane * 16));
  }
  __builtin_amdgcn_sched_barrier(0);

  // 2. Stage this wave's x (zeros beyond M and K) and its (scale, zero)
  //    pairs.  Only this wave reads them: LDS operations of one wave complete
  //    in order, so a wave-level barrier (no s_barrier) suffices.
#pragma unroll
  for (int j = 0; j < NXC; ++j) {
    const int c = lane + 64 * j;
    const int m = c / (KW / 8), kk = (c % (KW / 8)) * 8;
    const bool ok = m < a.M && k0 + kk < a.K;
    if (c < XCH) *reinterpret_cast<u4*>(xs + m * KW + kk) = ok ? xr[j] : u4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int j = 0; j < NSZ; ++j) {
    const int e = lane + 64 * j;
    if (e < 16 * gstride) {
      const int idx = (e >> lgs) * GWMAX + (e & (gstride - 1));
      if constexpr (F::KQ) szk[idx] = kq_terms(sraw[j], zraw[j]);
      else sz[idx] = (sraw[j] & 0xffffu) | (zraw[j] << 16);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if constexpr (F::KQ) {
    // x sum of every 32-wide run of the wave's range (zeros past K), one
    // lane per (row, run)
    for (int e = lane; e < MMAX * GWMAX; e += 64) {
      const h8* xp = reinterpret_cast<const h8*>(xs + (e / GWMAX) * KW + (e % GWMAX) * 32);
      float v = 0.0f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const h8 xv = xp[c];
#pragma unroll
        for (int t = 0; t < 4; ++t) v = __builtin_amdgcn_fdot2(h2{xv[2 * t], xv[2 * t + 1]}, splat((f16)1.0f), v, false);
      }
      xsum[e] = v;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // 3. Dot products, tile by tile and one run of SW codes at a time (a lane
  //    holds 32 INT4, 64 INT2 or 16 q8_0 codes, and a group may be 32 wide):
  //    exact (q - z) pairs against fp16 x pairs (v_dot2_f32_f16, fp32
  //    accumulation), fp32 scale once per run.
  float acc[MMAX];
#pragma unroll
  for (int m = 0; m < MMAX; ++m) acc[m] = 0.0f;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    if (i < nt) {
#pragma unroll
      for (int p = 0; p < F::NSEG; ++p) {
        const int run = (i * F::KT + g * F::LS + p * F::SW) >> lg;
        float sf, bk = 0.0f;
        f16 z;
        if constexpr (F::KQ) {
          const float2 t = szk[r * GWMAX + run];
          sf = t.x;
          bk = t.y;
          z = (f16)0.0f;
        } else {
          const uint32_t szv = sz[r * GWMAX + run];
          sf = (float)__builtin_bit_cast(f16, (uint16_t)(szv & 0xffffu));
          z = __builtin_bit_cast(f16, (uint16_t)(szv >> 16));
        }
        h2 q[F::SW / 2];
        run_qmz<FMT>(code[i], p, z, q);
#pragma unroll
        for (int m = 0; m < MMAX; ++m) {
          const h8* xp = reinterpret_cast<const h8*>(xs + m * KW + i * F::KT + g * F::LS + p * F::SW);
          float A0 = 0.0f, A1 = 0.0f;  // two chains for issue overlap
#pragma unroll
          for (int c = 0; c < F::SW / 8; ++c) {
            const h8 xv = xp[c];
            float t0 = (c & 1) ? A1 : A0;
            t0 = __builtin_amdgcn_fdot2(q[4 * c + 0], h2{xv[0], xv[1]}, t0, false);
            t0 = __builtin_amdgcn_fdot2(q[4 * c + 1], h2{xv[2], xv[3]}, t0, false);
            t0 = __builtin_amdgcn_fdot2(q[4 * c + 2], h2{xv[4], xv[5]}, t0, false);
            t0 = __builtin_amdgcn_fdot2(q[4 * c + 3], h2{xv[6], xv[7]}, t0, false);
            if (c & 1) A1 = t0; else A0 = t0;
          }
          acc[m] = fmaf(sf, A0 + A1, acc[m]);
          if constexpr (F::KQ) acc[m] = fmaf(-bk, xsum[m * GWMAX + run], acc[m]);
        }
      }
    }
  }

  // 4. Sum lane groups g and g ^ 1 across lanes; the pairs (0, 1) and (2, 3)
  //    of every wave go through LDS, summed over the waves in wave order
  //    (deterministic), then the two pairs across lanes.
#pragma unroll
  for (int m = 0; m < MMAX; ++m) {
    const float v = add_lane_xor16(acc[m]);
    if ((g & 1) == 0) red[((wave * MMAX + m) * 2 + (g >> 1)) * 16 + r] = v;
  }
  __syncthreads();
  if (tid >= MMAX * 32) return;
  float total = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) total += red[(w * MMAX + om) * 32 + (tid & 31)];
  total = add_lane_xor16(total);
  if (tid & 16) return;
  const int on = rb * 16 + orow;
  if (a.splits == 1) {
    if (om < a.M && on < a.N)
      a.y[(int64_t)om * a.ldy + on] = (f16)(has_res ? total + (float)__builtin_bit_cast(f16, (uint16_t)res) : total);
    return;
  }
  // split-K: this split's partial; gemv_reduce_kernel sums the splits in order
  a.ws[((int64_t)rb * a.splits + split) * MMAX * 16 + om * 16 + orow] = total;
}

// Decode GEMV on half row blocks (M = 1 or 2, used when the row blocks alone would
// leave the compute units unevenly loaded, e.g. 384 blocks on 256 CUs): a
// workgroup takes rows 8 hb .. 8 hb + 7 of row block blockIdx.x / 2
// (hb = blockIdx.x % 2), so twice as many workgroups of half the work.  Its NW
// waves take TPW word tiles each, two at a time: lane l = r8 + 8 g + 32 t reads
// the 16-byte chunk of row 8 hb + r8, lane group g, of tile 2 i + t of the
// wave's run -- one 16-byte load per lane and pair, as gemv_kernel.  Same
// dequant and dot products (MMAX rows of x share each exact (q - z) pair; q4k
// as in gemv_kernel); lanes sum over g and t, the waves through LDS in wave order.
// LDS bytes of gemv_half_body: per wave its x rows, (scale, zero) pairs and
// (q4k) group sums of x, then NW x MMAX x 16 fp32 for the sum over the waves
template <int FMT, int NW, int TPW, int MMAX> constexpr size_t gemv_half_lds_bytes() {
  using F = Fmt<FMT>;
  constexpr int KW = TPW * F::KT, GW = KW / 32;
  constexpr int WB = MMAX * KW * 2 + 8 * GW * (F::KQ ? 8 : 4) + (F::KQ ? MMAX * GW * 4 : 0);
  return (size_t)NW * WB + (size_t)NW * MMAX * 16 * sizeof(float);
}

// One half row block (bx: row block bx / 2, half bx % 2) and K split `by` of
// the decode GEMV, by a workgroup of NW waves, in half_smem
// (gemv_half_lds_bytes); the kernel below and the persistent looped block
// both run it.  COHERENT: the outputs are stored with agent scope (written
// through to the level every XCD reads), for readers in the same launch.
// COHERENT_IN: x and the residual are read with agent scope too (they were
// written in the same launch after this workgroup may have cached an older
// copy); the weights keep plain loads, so they can stay in the caches.
template <int FMT, int NW, int TPW, int MMAX, bool COHERENT = false, bool COHERENT_IN = false>
__device__ __forceinline__ void gemv_half_body(const GemvArgs& a, int bx, int by, uint8_t* half_smem) {
  using F = Fmt<FMT>;
  static_assert(TPW % 2 == 0, "tiles go in pairs");
  constexpr int NP = TPW / 2;                  // tile pairs per wave
  constexpr int KW = TPW * F::KT;              // k range of one wave
  constexpr int GWMAX = KW / 32;
  constexpr int XCH = MMAX * KW / 8;
  constexpr int NXC = (XCH + 63) / 64;
  constexpr int NSZ = (8 * GWMAX + 63) / 64;
  constexpr int SZB = F::KQ ? 8 : 4;           // q4k: fp32 (d*sc, dmin*m) per (row, sub-block)
  constexpr int XB = MMAX * KW * 2, SB = 8 * GWMAX * SZB;
  constexpr int WB = XB + SB + (F::KQ ? MMAX * GWMAX * 4 : 0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  f16* xs = reinterpret_cast<f16*>(half_smem + wave * WB);                 // [MMAX][KW]
  uint32_t* sz = reinterpret_cast<uint32_t*>(half_smem + wave * WB + XB);  // [8][GWMAX] s | z << 16
  float2* szk = reinterpret_cast<float2*>(half_smem + wave * WB + XB);     // q4k: [8][GWMAX] (d*sc, dmin*m)
  float* xsum = reinterpret_cast<float*>(half_smem + wave * WB + XB + SB); // q4k: [MMAX][GWMAX]
  float* red = reinterpret_cast<float*>(half_smem + NW * WB);              // [NW][MMAX][2][8]
  const int r8 = lane & 7, g = (lane >> 3) & 3, t = lane >> 5;
  const int rb = bx >> 1, hb = bx & 1, split = by;
  const int row0 = rb * 16 + hb * 8;
  const int T0 = split * a.tps, T1 = min(a.wordtiles, T0 + a.tps);
  const int wt0 = T0 + wave * TPW;
  const int nt = max(0, min(T1, wt0 + TPW) - wt0);   // tiles of this wave
  const int k0 = wt0 * F::KT;
  const int lg = __builtin_ctz(a.group);
  const int ng = a.K >> lg;
  const int gstride = KW >> lg;                   // groups per wave, a power of two
  const int lgs = __builtin_ctz(gstride);
  const int gs0 = k0 >> lg;
  // 1. loads: (scale, zero) entries of the 8 rows, the residual, x rows, one
  //    code chunk per tile pair; clamped, never out of range
  const int64_t szbase = (int64_t)row0 * ng * 2;
  // q4k: the (d, dmin) pair of each super-block (8 sub-blocks) as 32 bits,
  // so the 8 rows' pairs start at row0 * (ng / 8) * 4 bytes
  const char* sp = reinterpret_cast<const char*>(a.scales) + (F::KQ ? szbase / 4 : szbase);
  const char* zp = reinterpret_cast<const char*>(F::HAS_Z || F::KQ ? a.zeros : a.scales) + szbase;
  uint32_t sraw[NSZ], zraw[NSZ];
#pragma unroll
  for (int j = 0; j < NSZ; ++j) {
    const int e = lane + 64 * j;   // row e >> lgs, group gs0 + e % gstride
    const int er = e >> lgs, eg = gs0 + (e & (gstride - 1));
    const bool ok = e < 8 * gstride && row0 + er < a.N && eg < ng;
    const uint32_t off = ok ? (uint32_t)(er * ng + eg) * 2u : 0u;
    if constexpr (F::KQ) {
      sraw[j] = *reinterpret_cast<const uint32_t*>(sp + (ok ? (uint32_t)(er * (ng >> 3) + (eg >> 3)) * 4u : 0u));
      zraw[j] = *reinterpret_cast<const uint16_t*>(zp + off);
    } else {
      sraw[j] = *reinterpret_cast<const uint16_t*>(sp + off);
      if constexpr (F::HAS_Z) zraw[j] = *reinterpret_cast<const uint16_t*>(zp + off);
      else zraw[j] = F::ZBITS;
    }
  }
  const int om = (tid >> 4) % MMAX;   // output row of thread tid < 16 MMAX (final sum)
  // its residual, fp16 bits: loaded unconditionally (from x when there is
  // none, dropped at the store), since a load under a branch made the
  // compiler wait for it, and for every load before it, ahead of the x and
  // code loads
  const bool has_res = a.resid && a.splits == 1;
  const uint16_t* rp = has_res ? reinterpret_cast<const uint16_t*>(a.resid) + (int64_t)min(om, a.M - 1) * a.ldr +
                                     min(row0 + (tid & 7), a.N - 1)
                               : reinterpret_cast<const uint16_t*>(a.x);
  uint32_t res;
  if constexpr (COHERENT_IN)
    res = __hip_atomic_load(reinterpret_cast<const unsigned short*>(rp), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    res = *rp;
  __builtin_amdgcn_sched_barrier(0);
  u4 xr[NXC];
#pragma unroll
  for (int j = 0; j < NXC; ++j) {
    const int c = lane + 64 * j;   // one row: chunk c at k0 + 8c (lanes past the wave's slice read in range too)
    const int m = MMAX == 1 ? 0 : c / (KW / 8), k = k0 + (MMAX == 1 ? c : c % (KW / 8)) * 8;
    const bool ok = (MMAX == 1 || m < a.M) && k < a.K;
    const char* xp = reinterpret_cast<const char*>(a.x) + (ok ? ((uint32_t)m * a.ldx + k) * 2u : 0u);
    if constexpr (COHERENT_IN) {
      const unsigned* q = reinterpret_cast<const unsigned*>(xp);
#pragma unroll
      for (int d = 0; d < 4; ++d) xr[j][d] = __hip_atomic_load(q + d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      xr[j] = *reinterpret_cast<const u4*>(xp);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  u4 code[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int64_t tile = (int64_t)rb * a.wordtiles + min(wt0 + 2 * i + t, a.wordtiles - 1);
    code[i] = *reinterpret_cast<const u4*>(reinterpret_cast<const char*>(a.packed) + tile * 1024 +
                                           (g * 16 + hb * 8 + r8) * 16);
  }
  __builtin_amdgcn_sched_barrier(0);

  // 2. stage x (zero past M and K) and the (scale, zero) pairs in the wave's region
#pragma unroll
  for (int j = 0; j < NXC; ++j) {
    const int c = lane + 64 * j;
    const int m = c / (KW / 8), kk = (c % (KW / 8)) * 8;
    if (c < XCH) *reinterpret_cast<u4*>(xs + m * KW + kk) = (MMAX == 1 || m < a.M) && k0 + kk < a.K ? xr[j] : u4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int j = 0; j < NSZ; ++j) {
    const int e = lane + 64 * j;
    if (e < 8 * gstride) {
      const int idx = (e >> lgs) * GWMAX + (e & (gstride - 1));
      if constexpr (F::KQ) szk[idx] = kq_terms(sraw[j], zraw[j]);
      else sz[idx] = (sraw[j] & 0xffffu) | (zraw[j] << 16);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if constexpr (F::KQ) {
    // x sum of every 32-wide run of the wave's range (zeros past K), one lane
    // per (row of x, run)
    for (int e = lane; e < MMAX * GWMAX; e += 64) {
      const h8* xp = reinterpret_cast<const h8*>(xs + (e / GWMAX) * KW + (e % GWMAX) * 32);
      float v = 0.0f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const h8 xv = xp[c];
#pragma unroll
        for (int u = 0; u < 4; ++u) v = __builtin_amdgcn_fdot2(h2{xv[2 * u], xv[2 * u + 1]}, splat((f16)1.0f), v, false);
      }
      xsum[e] = v;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  // 3. dot products of the lane's chunk, one run of SW codes at a time; the
  //    exact (q - z) pairs serve every row of x
  float acc[MMAX];
#pragma unroll
  for (int m = 0; m < MMAX; ++m) acc[m] = 0.0f;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    if (2 * i + t >= nt) continue;
#pragma unroll
    for (int p = 0; p < F::NSEG; ++p) {
      const int kl = (2 * i + t) * F::KT + g * F::LS + p * F::SW;
      const int run = kl >> lg;
      float sf, bk = 0.0f;
      f16 z;
      if constexpr (F::KQ) {   // q4k: exact q; d*sc * (x . q) - dmin*m * sum(x), in fp32
        const float2 kt = szk[r8 * GWMAX + run];
        sf = kt.x;
        bk = kt.y;
        z = (f16)0.0f;
      } else {
        const uint32_t szv = sz[r8 * GWMAX + run];
        sf = (float)__builtin_bit_cast(f16, (uint16_t)(szv & 0xffffu));
        z = __builtin_bit_cast(f16, (uint16_t)(szv >> 16));
      }
      h2 q[F::SW / 2];
      run_qmz<FMT>(code[i], p, z, q);
#pragma unroll
      for (int m = 0; m < MMAX; ++m) {
        const h8* xp = reinterpret_cast<const h8*>(xs + m * KW + kl);
        float A0 = 0.0f, A1 = 0.0f;
#pragma unroll
        for (int c = 0; c < F::SW / 8; ++c) {
          const h8 xv = xp[c];
          float t0 = (c & 1) ? A1 : A0;
          t0 = __builtin_amdgcn_fdot2(q[4 * c + 0], h2{xv[0], xv[1]}, t0, false);
          t0 = __builtin_amdgcn_fdot2(q[4 * c + 1], h2{xv[2], xv[3]}, t0, false);
          t0 = __builtin_amdgcn_fdot2(q[4 * c + 2], h2{xv[4], xv[5]}, t0, false);
          t0 = __builtin_amdgcn_fdot2(q[4 * c + 3], h2{xv[6], xv[7]}, t0, false);
          if (c & 1) A1 = t0; else A0 = t0;
        }
        acc[m] = fmaf(sf, A0 + A1, acc[m]);
        if constexpr (F::KQ) acc[m] = fmaf(-bk, xsum[m * GWMAX + run], acc[m]);
      }
    }
  }
  // 4. sum over g across lanes (l ^ 8, l ^ 16); the two tiles t of every wave
  //    through LDS, summed over the waves in wave order, then over t across
  //    lanes (l ^ 8 within a 16-lane row)
#pragma unroll
  for (int m = 0; m < MMAX; ++m) {
    const float v = add_lane_xor16(add_lane_xor8(acc[m]));
    if (g == 0) red[(wave * MMAX + m) * 16 + t * 8 + r8] = v;
  }
  __syncthreads();
  if (tid >= MMAX * 16) return;
  float total = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) total += red[(w * MMAX + om) * 16 + (tid & 15)];
  total = add_lane_xor8(total);
  if (tid & 8) return;
  const int on = row0 + (tid & 7);
  if (a.splits == 1) {
    if (om < a.M && on < a.N) {
      const f16 v = (f16)(has_res ? total + (float)__builtin_bit_cast(f16, (uint16_t)res) : total);
      if constexpr (COHERENT)
        __hip_atomic_store(reinterpret_cast<unsigned short*>(a.y) + (int64_t)om * a.ldy + on,
                           __builtin_bit_cast(unsigned short, v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        a.y[(int64_t)om * a.ldy + on] = v;
    }
    return;
  }
  // split-K: the same partial layout as gemv_kernel with MMAX rows of x
  a.ws[((int64_t)rb * a.splits + split) * MMAX * 16 + om * 16 + hb * 8 + (tid & 7)] = total;
}

template <int FMT, int NW, int TPW, int MMAX>
__global__ __launch_bounds__(NW * 64) void gemv_half_kernel(GemvArgs a) {
  __shared__ __align__(16) uint8_t half_smem[gemv_half_lds_bytes<FMT, NW, TPW, MMAX>()];
  gemv_half_body<FMT, NW, TPW, MMAX>(a, blockIdx.x, blockIdx.y, half_smem);
}

// ---------------------------------------------------------------------------
// Persistent looped block at M = 1: one launch per loop runs the loop's four
// GEMVs (QKV, O + x, up, down + h) as phases over half row blocks, the
// workgroups of a co-resident grid taking blocks round robin, with a grid
// barrier between phases -- the shared-block loop of the TinyLoop README
// ("Why TinyLoop Exists"; "Status", on the weights staying cache-resident
// across the L iterations), without the three kernel boundaries per loop.

struct LoopArgs {
  GemvArgs lin[4];
  unsigned* counter;   // arrivals, zeroed before the call's first loop
  int* status;         // set to 1 when a barrier gives up waiting
  int barrier0;        // barriers passed before this launch
  int loops;           // loops this launch runs (1, or all L of the call)
  int cap;             // polls before a barrier gives up
};

// Barrier of all workgroups of the grid through arrival counters that only
// grow: the b-th barrier of the call waits until they sum to
// (b + 1) * gridDim.x.  Workgroup w arrives at counter w % 8 -- eight 128-byte
// lines, so arrivals do not all queue on one address.  The phases store their
// outputs with agent scope, visible to every XCD once complete: every wave
// waits for its own memory operations, then thread 0 arrives and polls
// (relaxed, agent scope) with sleeps.  A phase's inputs were produced earlier
// in the same launch and never read before them in it (the launch begins with
// clean caches), so no cache holds a stale copy and no cache maintenance is
// needed.  After `cap` polls, or once another workgroup has given up, thread
// 0 records the failure in *status and stops waiting, so the kernel always
// ends.
constexpr int LOOP_COUNTERS = 8, LOOP_COUNTER_STRIDE = 32;   // uint32 apart

__device__ __forceinline__ void grid_barrier(unsigned* counter, unsigned target, int* status, int cap) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(counter + LOOP_COUNTER_STRIDE * (blockIdx.x % LOOP_COUNTERS), 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    int polls = 0;
    while (true) {
      unsigned arrived = 0;
#pragma unroll
      for (int i = 0; i < LOOP_COUNTERS; ++i)
        arrived += __hip_atomic_load(counter + LOOP_COUNTER_STRIDE * i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (arrived >= target) break;
      if (polls++ >= cap || __hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
        __hip_atomic_store(status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
}

constexpr int LOOP_THREADS = 512;   // 8 waves, as the 8-row GEMV

// TA word tiles per wave for the K = D linears (QKV, O, up), TB for down (K = F).
// ALL: the launch runs all p.loops loops of the call, with a barrier between
// loops too, and reads its activations with agent scope (they are rewritten
// every loop); the workgroup that runs a block of rows runs it in every loop,
// so its XCD's L2 can keep those rows' weights from one loop to the next.
template <int FMT, int TA, int TB, bool ALL>
__global__ __launch_bounds__(LOOP_THREADS) void loop_block_kernel(LoopArgs p) {
  constexpr size_t LA = gemv_half_lds_bytes<FMT, 8, TA, 1>(), LB = gemv_half_lds_bytes<FMT, 8, TB, 1>();
  constexpr int BPL = ALL ? 4 : 3;   // barriers per loop
  __shared__ __align__(16) uint8_t smem[LA > LB ? LA : LB];
  const int loops = ALL ? p.loops : 1;
  for (int l = 0; l < loops; ++l) {
#pragma unroll
    for (int ph = 0; ph < 4; ++ph) {
      const int nb = 2 * p.lin[ph].rowblocks;
      for (int vb = blockIdx.x; vb < nb; vb += gridDim.x) {
        if (ph < 3) gemv_half_body<FMT, 8, TA, 1, true, ALL>(p.lin[ph], vb, 0, smem);
        else gemv_half_body<FMT, 8, TB, 1, true, ALL>(p.lin[ph], vb, 0, smem);
        __syncthreads();   // smem is reused by the next block
      }
      if (ph < 3 || l + 1 < loops)
        grid_barrier(p.counter, (unsigned)(p.barrier0 + BPL * l + ph + 1) * gridDim.x, p.status, p.cap);
    }
  }
}

__global__ void loop_reset_kernel(unsigned* counter, int* status) {
  for (int i = 0; i < LOOP_COUNTERS; ++i) counter[LOOP_COUNTER_STRIDE * i] = 0u;
  *status = 0;
}

// LDS bytes of gemv_mfma_kernel: per wave its x rows (padded by 16 bytes so
// that the A-fragment reads of 16 rows fall in distinct banks) and its
// (scale, zero) pairs, then one 16 x 16 fp32 block per wave for the final sum
template <int FMT, int MROWS, int TPW> constexpr size_t gemv_mfma_lds_bytes() {
  constexpr int KW = TPW * Fmt<FMT>::KT, NW = GEMV_THREADS / 64;
  return (size_t)NW * (MROWS * (KW + 8) * 2 + 16 * (KW / 32) * 4) + (size_t)NW * 64 * 16;
}

// Decode GEMV for 2 <= M <= 16 on the matrix cores.  Same workgroup and wave
// layout as gemv_kernel (one 16-row block x a K range; 8 waves, each staging
// its own x rows and (scale, zero) pairs), but the products run as
// v_mfma_f32_16x16x32_f16.  In that operand layout lane l = 16g + r supplies
// column r and k-slots 8g..8g+7 of B -- exactly the packed chunk of row r and
// lane group g -- so once 8 codes are dequantized to fp16 s*(q - z) (13 VALU
// for 4-bit codes, the GEMM's dequant, whatever M is) they are one MFMA step;
// A is row r of x (zero for r >= MROWS) at the same k.  The 16 x 16 accumulator holds
// y[4g + i][16 rb + r] in lane 16g + r, element i.
template <int FMT, int MROWS, int TPW, int CH>
__global__ __launch_bounds__(GEMV_THREADS) void gemv_mfma_kernel(GemvArgs a) {
  using F = Fmt<FMT>;
  constexpr int NW = GEMV_THREADS / 64;
  constexpr int KW = TPW * F::KT;              // k range of one chunk
  constexpr int KWP = KW + 8;                  // padded x row (halves)
  constexpr int GWMAX = KW / 32;
  constexpr int XCH = MROWS * KW / 8;          // 16-byte x chunks per wave and chunk
  constexpr int NXC = (XCH + 63) / 64;
  constexpr int NSZ = (16 * GWMAX + 63) / 64;
  constexpr int XB = MROWS * KWP * 2, WB = XB + 16 * GWMAX * 4;
  static_assert(MROWS == 4 || MROWS == 8 || MROWS == 16, "rows per MFMA block");
  __shared__ __align__(16) uint8_t smem[gemv_mfma_lds_bytes<FMT, MROWS, TPW>()];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  f16* xs = reinterpret_cast<f16*>(smem + wave * WB);                 // [MROWS][KWP]
  uint32_t* sz = reinterpret_cast<uint32_t*>(smem + wave * WB + XB);  // [16][GWMAX] s | z << 16
  f4* red = reinterpret_cast<f4*>(smem + NW * WB);                     // [NW][64 lanes]

  const int g = lane >> 4, r = lane & 15;
  const int rb = blockIdx.x, split = blockIdx.y;
  const int T0 = split * a.tps, T1 = min(a.wordtiles, T0 + a.tps);
  const int tpw = (T1 - T0 + NW - 1) / NW;           // <= CH * TPW (the launch picks CH)
  const int wt0 = T0 + wave * tpw;
  const int nt = max(0, min(T1, wt0 + tpw) - wt0);   // word tiles of this wave
  const int lg = __builtin_ctz(a.group);
  const int ng = a.K >> lg;
  const int gstride = KW >> lg;
  const int lgs = __builtin_ctz(gstride);

  // The wave streams its tiles in CH chunks of TPW tiles (KW of K): the loads
  // of chunk c + 1 are issued before chunk c is staged and multiplied, so one
  // chunk's loads are always in flight behind the current one's MFMAs.  Loads
  // are clamped, never out of range, and issued for every chunk (a chunk past
  // the wave's tiles only adds no products), so every wait is a fixed count.
  const int64_t szbase = (int64_t)rb * 16 * ng * 2;
  // q4k: the (d, dmin) pair of each super-block (8 sub-blocks) as 32 bits,
  // so a row block's pairs start at rb * 16 * (ng / 8) * 4 bytes
  const char* sp = reinterpret_cast<const char*>(a.scales) + (F::KQ ? szbase / 4 : szbase);
  const char* zp = reinterpret_cast<const char*>(F::HAS_Z || F::KQ ? a.zeros : a.scales) + szbase;
  const char* pkrow = reinterpret_cast<const char*>(a.packed) + (int64_t)rb * a.wordtiles * 1024;
  uint32_t sraw[2][NSZ], zraw[2][NSZ];
  u4 xr[2][NXC];
  u4 code[2][TPW];
  auto load_chunk = [&](int c, uint32_t (&sr)[NSZ], uint32_t (&zr)[NSZ], u4 (&xv)[NXC], u4 (&cv)[TPW]) {
    const int kc0 = (wt0 + c * TPW) * F::KT;            // a group boundary (KT % group == 0)
    const int gs0 = kc0 >> lg;
#pragma unroll
    for (int j = 0; j < NSZ; ++j) {
      const int e = lane + 64 * j;
      const int er = e >> lgs, eg = gs0 + (e & (gstride - 1));
      const bool ok = e < 16 * gstride && rb * 16 + er < a.N && eg < ng;
      const uint32_t off = ok ? (uint32_t)(er * ng + eg) * 2u : 0u;
      if constexpr (F::KQ) {
        sr[j] = *reinterpret_cast<const uint32_t*>(sp + (ok ? (uint32_t)(er * (ng >> 3) + (eg >> 3)) * 4u : 0u));
        zr[j] = *reinterpret_cast<const uint16_t*>(zp + off);
      } else {
        sr[j] = *reinterpret_cast<const uint16_t*>(sp + off);
        if constexpr (F::HAS_Z) zr[j] = *reinterpret_cast<const uint16_t*>(zp + off);
        else zr[j] = F::ZBITS;  // the implicit zero point
      }
    }
#pragma unroll
    for (int j = 0; j < NXC; ++j) {
      const int q = lane + 64 * j;
      const int m = q / (KW / 8), k = kc0 + (q % (KW / 8)) * 8;
      const bool ok = q < XCH && m < a.M && k < a.K;
      const uint32_t off = ok ? (uint32_t)(m * a.ldx + k) * 2u : 0u;
      xv[j] = *reinterpret_cast<const u4*>(reinterpret_cast<const char*>(a.x) + off);
    }
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int T = min(wt0 + c * TPW + i, a.wordtiles - 1);
      cv[i] = *reinterpret_cast<const u4*>(pkrow + (uint32_t)(T * 1024 + lane * 16));
    }
  };

  // 1. chunk 0's loads, the residual (raw fp16 bits, converted only at the
  //    store: a conversion here would make the wave wait for every load)
  load_chunk(0, sraw[0], zraw[0], xr[0], code[0]);
  uint32_t res[4] = {0u, 0u, 0u, 0u};
  if (a.resid && a.splits == 1 && wave == 0) {
    const int nc = min(rb * 16 + r, a.N - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      res[i] = reinterpret_cast<const uint16_t*>(a.resid)[(int64_t)min(4 * g + i, a.M - 1) * a.ldr + nc];
  }

  f4 acc = f4{0.f, 0.f, 0.f, 0.f};
  const bool arow = r < MROWS;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int b = c & 1;
    __builtin_amdgcn_sched_barrier(0);
    if (c + 1 < CH) load_chunk(c + 1, sraw[b ^ 1], zraw[b ^ 1], xr[b ^ 1], code[b ^ 1]);
    __builtin_amdgcn_sched_barrier(0);
    const int kc0 = (wt0 + c * TPW) * F::KT;

    // 2. stage the chunk's x rows (zeros beyond M and K) and (scale, zero)
    //    pairs; this wave's earlier LDS reads complete first (in order)
#pragma unroll
    for (int j = 0; j < NXC; ++j) {
      const int q = lane + 64 * j;
      const int m = q / (KW / 8), kk = (q % (KW / 8)) * 8;
      const bool ok = m < a.M && kc0 + kk < a.K;
      if (q < XCH) *reinterpret_cast<u4*>(xs + m * KWP + kk) = ok ? xr[b][j] : u4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < NSZ; ++j) {
      const int e = lane + 64 * j;
      if (e < 16 * gstride)
        sz[(e >> lgs) * GWMAX + (e & (gstride - 1))] =
            F::KQ ? kq_half_pair(sraw[b][j], zraw[b][j]) : (sraw[b][j] & 0xffffu) | (zraw[b][j] << 16);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // 3. per run of SW codes: dequantize to fp16 s*(q - z), one MFMA per 8 codes
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      if (c * TPW + i < nt) {
#pragma unroll
        for (int p = 0; p < F::NSEG; ++p) {
          const int kl = i * F::KT + g * F::LS + p * F::SW;  // this lane's run inside the chunk
          const uint32_t szv = sz[r * GWMAX + (kl >> lg)];
          const h2 s2 = splat(__builtin_bit_cast(f16, (uint16_t)(szv & 0xffffu)));
          // q4k: the high half is -fp16(dmin*m), codes are unpacked with zero point 0
          const f16 z = F::KQ ? (f16)0.0f : __builtin_bit_cast(f16, (uint16_t)(szv >> 16));
          h8 av[F::SW / 8];
#pragma unroll
          for (int t = 0; t < F::SW / 8; ++t)
            av[t] = arow ? *reinterpret_cast<const h8*>(xs + (arow ? r : 0) * KWP + kl + 8 * t) : h8{};
          h2 q[F::SW / 2];
          run_qmz<FMT>(code[b][i], p, z, q);
          if constexpr (F::KQ) kq_weights(q, szv, q, F::SW / 2);   // fma(q, d*sc, -dmin*m)
#pragma unroll
          for (int t = 0; t < F::SW / 8; ++t) {
            h2 w0 = q[4 * t], w1 = q[4 * t + 1], w2 = q[4 * t + 2], w3 = q[4 * t + 3];
            if constexpr (!F::KQ) {
              w0 *= s2; w1 *= s2; w2 *= s2; w3 *= s2;
            }
            const h8 bf = h8{w0[0], w0[1], w1[0], w1[1], w2[0], w2[1], w3[0], w3[1]};
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[t], bf, acc, 0, 0, 0);
          }
        }
      }
    }
  }

  // 4. sum the NW waves' blocks through LDS in wave order; wave 0 writes
  red[wave * 64 + lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  f4 tot = red[lane];
#pragma unroll
  for (int w = 1; w < NW; ++w) tot += red[w * 64 + lane];
  const int n = rb * 16 + r;
  if (a.splits == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * g + i;
      if (m < a.M && n < a.N)
        a.y[(int64_t)m * a.ldy + n] = (f16)(tot[i] + (float)__builtin_bit_cast(f16, (uint16_t)res[i]));
    }
    return;
  }
  // split-K: rows m < MROWS of this split's block, laid out as gemv_kernel's
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * g + i;
    if (m < MROWS) a.ws[((int64_t)rb * a.splits + split) * MROWS * 16 + m * 16 + r] = tot[i];
  }
}

// Sums the split-K partials of the GEMV in split order (deterministic), adds
// the residual and rounds once to fp16.  One thread per output.
__global__ void gemv_reduce_kernel(const float* __restrict__ ws, const f16* __restrict__ resid,
                                   f16* __restrict__ y, int M, int N, int ldr, int ldy, int splits,
                                   int mmax) {
  const int64_t total = (int64_t)M * N;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int m = (int)(i / N), n = (int)(i % N);
    const int rb = n >> 4, r = n & 15;
    const float* p = ws + ((int64_t)rb * splits) * mmax * 16 + m * 16 + r;
    const int64_t ps = (int64_t)mmax * 16;
    uint32_t rv = 0u;   // fp16 bits, in a register of its own (no wait before the partial loads)
    if (resid) rv = reinterpret_cast<const uint16_t*>(resid)[(int64_t)m * ldr + n];
    // partials eight splits at a time, all loads before the adds, split order kept
    float v = 0.0f;
    int s = 0;
    for (; s + 8 <= splits; s += 8) {
      float t[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) t[j] = p[(s + j) * ps];
#pragma unroll
      for (int j = 0; j < 8; ++j) v += t[j];
    }
    for (; s < splits; ++s) v += p[s * ps];
    if (resid) v += (float)__builtin_bit_cast(f16, (uint16_t)rv);
    y[(int64_t)m * ldy + n] = (f16)v;
  }
}

// ---------------------------------------------------------------------------
// prefill GEMM (M > 16): fp16 MFMA on register-dequantized weights
// ---------------------------------------------------------------------------
struct GemmArgs {
  const f16* x; const uint32_t* packed; const f16* scales; const f16* zeros;
  const f16* resid; f16* y; float* ws;
  int ldx, ldr, ldy, M, N, K, group;
  int wordtiles, rowblocks, tiles_n, splits, tps;
};

template <int N> __device__ __forceinline__ void wait_vm() {
  // s_waitcnt vmcnt(N) (GFX9 encoding), expcnt and lgkmcnt left at their maximum
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() {
  // s_waitcnt lgkmcnt(0), vmcnt and expcnt left at their maximum
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

// Accumulator row of element i (0..15) of a 32 x 32 block for lane l: the
// output layout of v_mfma_f32_32x32x16_f16 is D[8*(i/4) + 4*(l/32) + i%4][l%32].
__device__ __forceinline__ int acc_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

// Stage geometry.  A stage feeds four MFMA steps of 8 k per lane half g2
// (32 k per half).  4- and 2-bit codes (WIDE: a lane's chunk holds 32 or more
// codes): a stage is (word tile t, chunk h, 32-code run j) and lane half g2
// takes its 32 k from lane group g2 + 2h, run j, at seg_k(g2, h, j).  8-bit
// codes: a stage is a whole word tile and lane half g2 takes 16 k from each of
// lane groups g2 (steps 0, 1) and g2 + 2 (steps 2, 3), i.e. chunk h = step / 2.
// x part: 32*MB rows x 2 pieces (one per lane half) x 4 sub-chunks of 8 k
// (4 KiB per 32 rows); code part: CH chunks of the NB 32-column blocks
// (1 KiB per block and chunk).
template <int FMT, int MB, int NB> struct GemmStage {
  static constexpr int KT = Fmt<FMT>::KT;
  static constexpr bool WIDE = Fmt<FMT>::LS >= 32;
  static constexpr int SEG = WIDE ? Fmt<FMT>::LS / 32 : 1;  // 32-code runs per chunk
  static constexpr int CH = WIDE ? 1 : 2;                  // chunks per stage
  static constexpr int STAGES = WIDE ? 2 * SEG : 1;        // stages per word tile
  static constexpr int XB = 32 * MB * 64 * 2;              // x bytes per stage (LDS)
  static constexpr int SB = XB;                            // codes go to VGPRs
  static constexpr int DMA = XB / 1024 + NB * CH;          // vector loads per lane per stage (10, 12 at 2 x 2)
};

// Prefill GEMM (M > 16).  Workgroup tile 32*MB (M) x 32*NB (N) -- 64 x 64,
// 64 x 32 when M <= 64, 32 x 32 when M <= 32 -- over the workgroup's share of K; its NW waves
// split that share and are summed through LDS at the end, so every code is
// dequantized once per workgroup.  Each wave owns MB x NB blocks of
// v_mfma_f32_32x32x16_f16 (B operand lane l = column l % 32,
// k-slots 8*(l/32)..+7): lane l takes its codes from the 16-byte chunk of row
// block n0/16 + 2*nb + (l%32)/16, row l%16, lane group l/32 + 2h, one packed
// word (8 codes) per MFMA step, and the A fragment of the step reads the
// matching 8 k of x, so A and B agree on the k order.
//
// Each wave streams its stages through a private DEPTH-deep LDS ring with
// direct global->LDS loads (x and codes alike, so every wait is an explicit
// vmcnt).  Inside a stage x sits as [piece][row][4 x 16 B]; sub-chunk u of
// row m is stored at u ^ ((m >> 2) & 3), so the fragment reads of 16
// consecutive rows hit 16 distinct bank groups.  All LDS operands of a stage
// are read first; group barriers then interleave one MFMA with a few VALU of
// the dequantization so the two pipes overlap.
template <int FMT, int NW, int TPW, int DEPTH, int MB, int NB, bool ALL, int CP = 1>
__global__ __launch_bounds__(NW * 64) void gemm_kernel(GemmArgs a) {
  using F = Fmt<FMT>;
  using S = GemmStage<FMT, MB, NB>;
  constexpr int SEG = S::SEG;
  constexpr int TM = 32 * MB, TN = 32 * NB, NBLK = MB * NB;
  // per-wave LDS region: its stage ring, large enough to take the wave's
  // accumulators ([block][quad][lane] f4) at the end, so a wave writes them
  // as soon as its own K loop is done, without waiting for the others
  constexpr int UNITS = NBLK * 4;                        // 32 x 32 block quads
  constexpr int WS = DEPTH * S::SB > UNITS * 1024 ? DEPTH * S::SB : UNITS * 1024;
  constexpr int BIG = NW * WS;
  // (s | z << 16) per column and group; a column's row is padded by one
  // word so that the 32 columns one lookup reads fall in 32 distinct banks
  constexpr int SZS = GEMM_GCAP + 1;
  constexpr int SZB = TN * SZS * 4;
  static_assert(DEPTH >= 1 && DEPTH <= 3 && (DEPTH - 1) * S::DMA <= 63, "vmcnt range");
  __shared__ __align__(16) uint8_t smem[BIG + SZB];
  uint32_t* szl = reinterpret_cast<uint32_t*>(smem + BIG);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g2 = lane >> 5, r = lane & 15;
  const int tn = blockIdx.x, tm = blockIdx.y, split = blockIdx.z;
  const int m0 = tm * TM, n0 = tn * TN;
  const int kt0 = split * a.tps;
  const int kt1 = min(a.wordtiles, kt0 + a.tps);
  const int per = (kt1 - kt0 + NW - 1) / NW;
  const int wt0 = kt0 + wave * per;
  const int nt = max(0, min(kt1, wt0 + per) - wt0);     // <= TPW (plan guarantees)
  const int nst = nt * S::STAGES;
  const int lg = __builtin_ctz(a.group);
  const int ng = a.K >> lg;
  const int gw0 = (kt0 * F::KT) >> lg;                   // first group (KT % group == 0)
  const int gwn = min(ng, ((kt1 * F::KT) + a.group - 1) >> lg) - gw0;  // <= GEMM_GCAP (plan)
  uint8_t* wbuf = smem + wave * WS;

  auto seg_k = [](int gg, int h, int j) { return (gg + 2 * h) * F::LS + j * 32; };

  // 0. the residual of the quads this wave finishes (UPW quads of 32 x 32
  //    blocks: all NW waves share the final sums), fp16 bits, converted only
  //    in the epilogue; issued first, so no later wait depends on it
  constexpr int UPW = UNITS >= NW ? UNITS / NW : 1;
  static_assert(UNITS < NW || UNITS % NW == 0, "quads per wave");
  const bool fin = wave * UPW < UNITS;                  // this wave finishes quads
  uint32_t res[4 * UPW];
  if (a.resid && a.splits == 1 && fin) {
#pragma unroll
    for (int k = 0; k < UPW; ++k) {
      const int u = wave * UPW + k, blk = u >> 2, q = u & 3;
      const int colc = min(n0 + (blk % NB) * 32 + (lane & 31), a.N - 1);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = min(m0 + (blk / NB) * 32 + acc_row(4 * q + e, lane), a.M - 1);
        res[4 * k + e] = reinterpret_cast<const uint16_t*>(a.resid)[(int64_t)row * a.ldr + colc];
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4 * UPW; ++i) res[i] = 0u;
  }

  // 1. the workgroup's scales and zeros, loaded cooperatively (clamped) and
  //    staged in LDS as [column][group] (rows padded by one word)
  constexpr int NSZ = (TN * GEMM_GCAP + NW * 64 - 1) / (NW * 64);
  const int gsr = gwn <= 1 ? 1 : 1 << (32 - __builtin_clz(gwn - 1));   // groups, rounded to a power of two
  const int lgs = __builtin_ctz(gsr);
  const int nsz = (TN * gsr + NW * 64 - 1) / (NW * 64);
  uint32_t sraw[NSZ], zraw[NSZ];
#pragma unroll
  for (int j = 0; j < NSZ; ++j) {
    {   // unconditional (clamped): a branch here makes the compiler wait on the loads at once
      const int e = tid + NW * 64 * j;                   // column e >> lgs, group e % gsr
      const int ec = e >> lgs, eg = e & (gsr - 1);
      const bool ok = j < nsz && ec < TN && eg < gwn && n0 + ec < a.N;
      const int64_t off = ok ? ((int64_t)(n0 + ec) * ng + gw0 + eg) : 0;
      if constexpr (F::KQ) {   // (d, dmin) of the super-block, (sc, m) of the sub-block
        const int64_t soff = ok ? ((int64_t)(n0 + ec) * (ng >> 3) + ((gw0 + eg) >> 3)) : 0;
        sraw[j] = reinterpret_cast<const uint32_t*>(a.scales)[soff];
        zraw[j] = reinterpret_cast<const uint16_t*>(a.zeros)[off];
      } else {
        sraw[j] = reinterpret_cast<const uint16_t*>(a.scales)[off];
        if constexpr (F::HAS_Z) zraw[j] = reinterpret_cast<const uint16_t*>(a.zeros)[off];
        else zraw[j] = F::ZBITS;  // the implicit zero point
      }
    }
  }

  // 2. per-lane byte offsets (fixed for all stages): x row quarters, code rows
  uint32_t voff[2 * MB];
#pragma unroll
  for (int q = 0; q < 2 * MB; ++q) {
    const int m = q * 16 + (lane >> 2);
    const int u = (lane & 3) ^ ((m >> 2) & 3);
    const int ucol = S::WIDE ? u * 8 : 0;              // 8-bit codes: added per stage below
    voff[q] = (uint32_t)((min(m0 + m, a.M - 1) * a.ldx + ucol) * 2);   // rows past M: any finite data
  }
  // 8-bit codes: sub-chunk u of a piece sits 8 (u & 1) + 32 (u >> 1) past the
  // piece's first k (the second half from lane group g2 + 2); u is the same
  // for every q above, since q moves m by multiples of 16
  const int usub = (lane & 3) ^ ((lane >> 4) & 3);
  const int subk = 8 * (usub & 1) + 32 * (usub >> 1);
  const char* cb[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int rb = min((n0 >> 4) + 2 * nb + ((lane >> 4) & 1), a.rowblocks - 1);  // columns past N: never stored
    cb[nb] = reinterpret_cast<const char*>(a.packed) + (int64_t)rb * a.wordtiles * 1024 + (g2 * 16 + r) * 16;
  }
  // ALL: every wave issues all TPW * STAGES stages, those past its share with
  // the tile clamped in bounds (never computed), so the loads form one
  // straight-line sequence and every wait is a fixed count (the compiler's
  // own waits for the code registers then need no merge over branches).
  // Otherwise (splits that leave waves with few or no tiles) a wave issues
  // only its own stages.
  static_assert(CP == 1 || (CP == 2 && DEPTH == 1), "codes one stage ahead of x: one x stage in flight");
  constexpr int BQ = DEPTH > CP ? DEPTH : CP;
  constexpr int CL = S::CH * NB;                          // code loads per stage
  u4 bq[BQ][S::CH][NB];   // code chunks of the stages in flight
  auto issue_x = [&](int st) {
    const int t = st / S::STAGES, hj = st % S::STAGES, h = hj / SEG, j = hj % SEG;
    const int kt = min(wt0 + t, a.wordtiles - 1);
    uint8_t* dst = wbuf + (st % DEPTH) * S::SB;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const char* src;
      if constexpr (S::WIDE) {
        const int kp = kt * F::KT + seg_k(p, h, j);
        src = reinterpret_cast<const char*>(a.x) + (kp < a.K ? kp : 0) * 2;  // past K: scale 0
      } else {
        const int kk = kt * F::KT + 16 * p + subk;                          // this lane's sub-chunk
        src = reinterpret_cast<const char*>(a.x) + (kk < a.K ? kk : 0) * 2;
      }
#pragma unroll
      for (int q = 0; q < 2 * MB; ++q)
        __builtin_amdgcn_global_load_lds(
            (const void __attribute__((address_space(1)))*)(src + voff[q]),
            (void __attribute__((address_space(3)))*)(dst + (p * 2 * MB + q) * 1024), 16, 0, 0);
    }
  };
  auto issue_codes = [&](int st) {
    const int t = st / S::STAGES, hj = st % S::STAGES, h = hj / SEG;
    const int kt = min(wt0 + t, a.wordtiles - 1);
#pragma unroll
    for (int c = 0; c < S::CH; ++c)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        bq[st % BQ][c][nb] = *reinterpret_cast<const u4*>(cb[nb] + (int64_t)kt * 1024 + (h + c) * 512);
  };
  auto issue_stage = [&](int st) {
    issue_x(st);
    issue_codes(st);
    __builtin_amdgcn_sched_barrier(0);   // stages stay in issue order (the waits count them)
  };

  f16v acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int jn = 0; jn < NB; ++jn)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][jn][e] = 0.0f;

  // byte offset of the A fragment (m-block mb, step) inside a stage: piece
  // g2 holds TM rows of 64 bytes
  auto a_off = [&](int mb, int step) {
    const int m = mb * 32 + (lane & 31);
    return g2 * (TM * 64) + m * 64 + ((step ^ ((m >> 2) & 3)) << 4);
  };

  // 3. one stage: every LDS operand first, then B operands (13 VALU per
  //    4-bit word, 14 per two 8-bit words) interleaved with the 4*MB*NB MFMAs
  auto compute_stage = [&](int st) {
    const int t = st / S::STAGES, hj = st % S::STAGES, h = hj / SEG, j = hj % SEG;
    const int kt = wt0 + t;
    const uint8_t* sb = wbuf + (st % DEPTH) * S::SB;
    uint32_t szv[S::CH][NB];
    u4 bt[S::CH][NB];
    bool live[S::CH];
    h8 af[4][MB];
#pragma unroll
    for (int c = 0; c < S::CH; ++c) {
      // first k of this lane's codes in chunk c
      const int kseg = kt * F::KT + (S::WIDE ? seg_k(g2, h, j) : 16 * (g2 + 2 * c));
      live[c] = kseg < a.K;                             // codes past K: scale 0
      const int gi = min(max((kseg >> lg) - gw0, 0), gwn - 1);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        bt[c][nb] = bq[st % BQ][c][nb];
        szv[c][nb] = szl[(nb * 32 + (lane & 31)) * SZS + gi];
      }
    }
#pragma unroll
    for (int step = 0; step < 4; ++step)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) af[step][mb] = *reinterpret_cast<const h8*>(sb + a_off(mb, step));
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the math
    h2 s2[S::CH][NB];
    f16 z[S::CH][NB];
    uint32_t kqc[S::CH][NB];   // q4k: fp16 (d*sc) | -fp16(dmin*m) << 16, 0 past K
#pragma unroll
    for (int c = 0; c < S::CH; ++c)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        s2[c][nb] = splat(live[c] ? __builtin_bit_cast(f16, (uint16_t)(szv[c][nb] & 0xffffu)) : (f16)0.0f);
        z[c][nb] = F::KQ ? (f16)0.0f : __builtin_bit_cast(f16, (uint16_t)(szv[c][nb] >> 16));
        kqc[c][nb] = live[c] ? szv[c][nb] : 0u;
      }
    h8 bf[4][NB];
#pragma unroll
    for (int step = 0; step < 4; ++step)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int c = S::WIDE ? 0 : step >> 1;
        h2 q[4];
        if constexpr (FMT == INT2_ASYM) {
          qmz_int2_half(bt[0][nb][2 * j + (step >> 1)], step & 1, make_zc2(z[0][nb]), q);
        } else if constexpr (FMT == Q8_0) {
          const ZC8 zc = make_zc8(z[c][nb]);
          qmz_int8(bt[c][nb][2 * (step & 1)], zc, q);
          qmz_int8(bt[c][nb][2 * (step & 1) + 1], zc, q + 2);
        } else {
          qmz_int4(bt[0][nb][step], make_zc4(z[0][nb]), q);
        }
        h2 w0, w1, w2, w3;
        if constexpr (F::KQ) {
          h2 wq[4];
          kq_weights(q, kqc[0][nb], wq, 4);
          w0 = wq[0]; w1 = wq[1]; w2 = wq[2]; w3 = wq[3];
        } else {
          const h2 sc = s2[c][nb];
          w0 = q[0] * sc; w1 = q[1] * sc; w2 = q[2] * sc; w3 = q[3] * sc;
        }
        bf[step][nb] = h8{w0[0], w0[1], w1[0], w1[1], w2[0], w2[1], w3[0], w3[1]};
      }
#pragma unroll
    for (int step = 0; step < 4; ++step)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[step][mb], bf[step][nb], acc[mb][nb], 0, 0, 0);
    // schedule: the first step's operands, then per MFMA a share of the VALU
    // (2 x 2 blocks: 26, then 16 x (one MFMA, six VALU))
    constexpr int VFIRST = 13 * NB, VPER = NBLK == 4 ? 6 : 13 * NB / MB;
    __builtin_amdgcn_sched_group_barrier(0x002, VFIRST, 0);
#pragma unroll
    for (int i = 0; i < 4 * NBLK; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, VPER, 0);
    }
  };

  // 4. first stages in flight, then the scale/zero table (waiting for the
  //    scale/zero loads only)
  constexpr int NST = TPW * S::STAGES;
  const int lim = ALL ? NST : min(nst, NST);   // stages this wave issues
#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
    if (d < lim) issue_stage(d);
  if (CP == 2 && 1 < lim) {   // the next stage's codes behind the first stage
    issue_codes(1);
    __builtin_amdgcn_sched_barrier(0);
  }
  // the table is written with the stages still in flight: its stores are
  // plain ds_write_b32 in asm, since the compiler would otherwise wait for
  // every outstanding global->LDS load before an LDS store it cannot tell
  // apart from them (the table lies outside every wave's ring)
  if (CP == 2) {
    if (lim >= 2) wait_vm<(CP == 2 ? S::DMA + CL : 0)>();
    else if (lim == 1) wait_vm<S::DMA>();
    else wait_vm<0>();
  } else {
    const int ist = min(DEPTH, lim);
    if (ist >= 3) wait_vm<(DEPTH >= 3 ? 3 : 0) * S::DMA>();
    else if (ist == 2) wait_vm<(DEPTH >= 2 ? 2 : 0) * S::DMA>();
    else if (ist == 1) wait_vm<S::DMA>();
    else wait_vm<0>();
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < NSZ; ++j) {
    const int e = tid + NW * 64 * j;
    if (j < nsz && (e >> lgs) < TN) {
      const uint32_t v = F::KQ ? kq_half_pair(sraw[j], zraw[j]) : (sraw[j] & 0xffffu) | (zraw[j] << 16);
      const uint32_t addr = (uint32_t)(uintptr_t)(szl + (e >> lgs) * SZS + (e & (gsr - 1)));
      asm volatile("ds_write_b32 %0, %1" : : "v"(addr), "v"(v) : "memory");
    }
  }
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();

  // 5. the K loop: wait for stage st (newer stages may stay in flight),
  //    compute it, refill its buffer with stage st + DEPTH.  CP = 2: the
  //    codes of stage st + 1 are already in flight behind stage st's x, so
  //    their HBM latency hides under stage st's compute
  if constexpr (CP == 2) {
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      if (st < lim) {
        if (st + 1 < lim) wait_vm<CL>();   // all but the next stage's codes
        else wait_vm<0>();
        __builtin_amdgcn_sched_barrier(0);
        if (!ALL || st < nst) compute_stage(st);
        __builtin_amdgcn_sched_barrier(0);
        if (st + 1 < lim) {
          wait_lgkm0();  // this buffer's reads are back
          __builtin_amdgcn_sched_barrier(0);
          issue_x(st + 1);
        }
        // the waits above count the code loads as the newest: keep them behind
        // every x load of the stage
        __builtin_amdgcn_sched_barrier(0);
        if (st + 2 < lim) issue_codes(st + 2);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else
#pragma unroll
  for (int st = 0; st < NST; ++st) {
    if (st < lim) {
      const int newer = min(DEPTH - 1, lim - 1 - st);   // stages issued after st
      if (newer >= 2) wait_vm<(DEPTH >= 3 ? 2 : 0) * S::DMA>();
      else if (newer == 1) wait_vm<(DEPTH >= 2 ? 1 : 0) * S::DMA>();
      else wait_vm<0>();
      __builtin_amdgcn_sched_barrier(0);
      if (!ALL || st < nst) compute_stage(st);
      __builtin_amdgcn_sched_barrier(0);
      if (st + DEPTH < lim) {
        wait_lgkm0();  // this buffer's reads are back
        __builtin_amdgcn_sched_barrier(0);
        issue_stage(st + DEPTH);
      }
    }
  }

  // 6. sum the NW waves' accumulators through LDS in wave order
  //    (deterministic); each wave first writes its own into its ring region
  //    (its loads and LDS reads are done), then wave w finishes quads
  //    w * UPW .. + UPW - 1, so the reads, sums and stores spread over every wave
  f4* red = reinterpret_cast<f4*>(smem);
  constexpr int WSF = WS / 16;                           // region stride in f4
#pragma unroll
  for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f16v& A = acc[blk / NB][blk % NB];
      red[wave * WSF + (blk * 4 + q) * 64 + lane] = f4{A[4 * q], A[4 * q + 1], A[4 * q + 2], A[4 * q + 3]};
    }
  __syncthreads();
  if (!fin) return;
  f4 tot[UPW];
#pragma unroll
  for (int k = 0; k < UPW; ++k) {
    const int u = wave * UPW + k;                       // quad u & 3 of block u >> 2
    f4 v = red[u * 64 + lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) v += red[w * WSF + u * 64 + lane];
    tot[k] = v;
  }
  if (a.splits == 1) {
#pragma unroll
    for (int k = 0; k < UPW; ++k) {
      const int u = wave * UPW + k, blk = u >> 2, q = u & 3;
      const int col = n0 + (blk % NB) * 32 + (lane & 31);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + (blk / NB) * 32 + acc_row(4 * q + e, lane);
        if (row < a.M && col < a.N)
          a.y[(int64_t)row * a.ldy + col] = (f16)(tot[k][e] + (float)__builtin_bit_cast(f16, (uint16_t)res[4 * k + e]));
      }
    }
    return;
  }
  // split-K: this split's TM x TN partial; gemm_reduce_kernel sums the splits
  f4* wsp = reinterpret_cast<f4*>(a.ws);
  const int64_t tile = (int64_t)tm * a.tiles_n + tn;
  const int64_t base = (tile * a.splits + split) * UNITS;
#pragma unroll
  for (int k = 0; k < UPW; ++k) wsp[(base + wave * UPW + k) * 64 + lane] = tot[k];
}

// Sums a tile's split partials in split order (deterministic), adds the
// residual and rounds once to fp16.  One workgroup of 4 waves per 32 x 32
// block fb of the tile (grid: column tile, row tile, block), so the partials
// are read by MB * NB workgroups per tile; wave q owns quad q of the block in
// the GEMM's accumulator layout, 4 outputs per lane.
template <int MB, int NB>
__global__ __launch_bounds__(256) void gemm_reduce_kernel(GemmArgs a) {
  constexpr int NBLK = MB * NB;
  const int tn = blockIdx.x, tm = blockIdx.y, fb = blockIdx.z;
  const int q = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int m0 = tm * 32 * MB, n0 = tn * 32 * NB;
  const int64_t tile = (int64_t)tm * a.tiles_n + tn;
  const f4* wsp = reinterpret_cast<const f4*>(a.ws);
  const int col = n0 + (fb % NB) * 32 + (lane & 31);
  const int colc = min(col, a.N - 1);
  // every load is issued before the first use: residual, then the partials
  // four splits at a time, added in split order (deterministic)
  uint32_t rr[4] = {0u, 0u, 0u, 0u};   // fp16 bits, one per register (no packing wait)
  if (a.resid) {   // uniform branch: the four loads go out together
    const uint16_t* rb16 = reinterpret_cast<const uint16_t*>(a.resid);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = min(m0 + (fb / NB) * 32 + acc_row(4 * q + e, lane), a.M - 1);
      rr[e] = rb16[(int64_t)row * a.ldr + colc];
    }
  }
  const f4* pp = wsp + ((tile * a.splits * NBLK + fb) * 4 + q) * 64 + lane;
  const int64_t pstride = NBLK * 4 * 64;        // one split, in f4
  f4 sum = f4{0.f, 0.f, 0.f, 0.f};
  int s = 0;
  for (; s + 4 <= a.splits; s += 4) {
    const f4 p0 = pp[(s + 0) * pstride], p1 = pp[(s + 1) * pstride];
    const f4 p2 = pp[(s + 2) * pstride], p3 = pp[(s + 3) * pstride];
    sum += p0; sum += p1; sum += p2; sum += p3;
  }
  for (; s < a.splits; ++s) sum += pp[s * pstride];
  float res[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) res[e] = (float)__builtin_bit_cast(f16, (uint16_t)rr[e]);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = m0 + (fb / NB) * 32 + acc_row(4 * q + e, lane);
    if (row < a.M && col < a.N) a.y[(int64_t)row * a.ldy + col] = (f16)(sum[e] + res[e]);
  }
}

// ---------------------------------------------------------------------------
// host side: device state, workspace, launches
// ---------------------------------------------------------------------------
struct DeviceWs {
  void* ptr = nullptr;
  size_t bytes = 0;
  std::vector<void*> retired;   // outgrown buffers, kept until the process ends
};
static std::mutex g_ws_mutex;
static std::vector<DeviceWs> g_ws;

// Last HIP error seen by this thread inside the library (for qg_last_error).
static thread_local hipError_t g_last_hip = hipSuccess;

int hip_status(int err) {
  const hipError_t e = static_cast<hipError_t>(err);
  if (e == hipSuccess) return QG_OK;
  g_last_hip = e;
  return QG_E_DEVICE;
}

int current_device(int* dev) {
  int st = hip_status(hipGetDevice(dev));
  if (st != QG_OK) return st;
  int count = 0;
  st = hip_status(hipGetDeviceCount(&count));
  if (st != QG_OK) return st;
  return count > 0 ? QG_OK : QG_E_DEVICE;
}

// Clears any error an earlier, unrelated HIP call left pending, so that the
// status after a launch reports that launch only.
void clear_pending_error() { (void)hipGetLastError(); }

// Library-owned zero-initialised workspace of at least `bytes` on `dev`.
// Growing never frees the buffer it replaces: a HIP graph captured earlier
// holds that buffer's address in its kernel arguments and may be replayed
// later, so the outgrown buffer is retired (kept until the process ends).
// Sizes at least double, so the retired buffers total less than the live one.
static int library_ws(int dev, size_t bytes, void** out) {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  if ((int)g_ws.size() <= dev) g_ws.resize(dev + 1);
  DeviceWs& w = g_ws[dev];
  if (w.bytes < bytes) {
    const size_t want = std::max({bytes, 2 * w.bytes, (size_t)1 << 20});
    void* p = nullptr;
    if (hipMalloc(&p, want) != hipSuccess) {
      clear_pending_error();
      return QG_E_NOMEM;
    }
    if (hip_status(hipMemset(p, 0, want)) != QG_OK) {
      (void)hipFree(p);
      return QG_E_DEVICE;
    }
    if (w.ptr) w.retired.push_back(w.ptr);
    w.ptr = p;
    w.bytes = want;
  }
  *out = w.ptr;
  return QG_OK;
}

static int launch_status() { return hip_status(hipGetLastError()); }

static unsigned grid_for(int64_t total, int threads) {
  int64_t b = (total + threads - 1) / threads;
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(b, 65536));
}

// grid: x = row blocks, y = K splits
template <int FMT, int MMAX, int TPW, int NW>
static void launch_gemv_t(const GemvArgs& a, hipStream_t s) {
  static_assert(gemv_lds_bytes<FMT, MMAX, TPW, NW>() <= 80 * 1024, "GEMV LDS: at least two workgroups per CU");
  hipLaunchKernelGGL((gemv_kernel<FMT, MMAX, TPW, NW>), dim3((unsigned)a.rowblocks, (unsigned)a.splits),
                     dim3(NW * 64), 0, s, a);
}

// Largest power-of-two tiles per wave (<= GEMV_TPW_MAX) whose x slice fits
// the 32 KiB x stage and whose whole LDS leaves room for two workgroups per CU
template <int FMT, int NW> constexpr int gemv_dot_tmax() {
  int t = GEMV_TPW_MAX;
  while (t > 1 && (t * NW * Fmt<FMT>::KT * 2 > GEMV_LDS_X_BYTES || gemv_lds_bytes_for<FMT>(1, t, NW) > 80 * 1024))
    t >>= 1;
  return t;
}

// TPW: word tiles per wave, rounded up to a power of two, at most
// gemv_dot_tmax.  Returns false when the plan asks for more tiles per wave
// than that (never, for plans made by make_plan).
template <int FMT, int NW>
static bool launch_gemv_dot_w(const GemvArgs& a, int tps, hipStream_t s) {
  constexpr int TMAX = gemv_dot_tmax<FMT, NW>();
  static_assert(gemv_lds_bytes<FMT, 1, TMAX, NW>() <= 80 * 1024, "tile cap and LDS size disagree");
  static_assert(NW != 16 || NW * TMAX >= gemv_m1_tile_cap(FMT), "the plan's M = 1 tile cap exceeds the kernel's");
  constexpr int T2 = TMAX >= 2 ? 2 : 1, T4 = TMAX >= 4 ? 4 : T2, T8 = TMAX >= 8 ? 8 : T4;
  const int tpw = (tps + NW - 1) / NW;
  if (tpw > TMAX) return false;
  if (tpw <= 1) launch_gemv_t<FMT, 1, 1, NW>(a, s);
  else if (tpw <= 2) launch_gemv_t<FMT, 1, T2, NW>(a, s);
  else if (tpw <= 4) launch_gemv_t<FMT, 1, T4, NW>(a, s);
  else launch_gemv_t<FMT, 1, T8, NW>(a, s);
  return true;
}

// 16 waves when a workgroup has at least 16 word tiles (more waves in flight,
// one tile each at K = 2048), 8 otherwise
// half row blocks (8-row workgroups): 4 waves of 2 tiles, 8 of 2, 8 of 4 or 8 of 8
template <int FMT, int MMAX>
static bool launch_gemv_half(const GemvArgs& a, int tps, hipStream_t s) {
  {
    const dim3 grid((unsigned)(2 * a.rowblocks), (unsigned)a.splits);
    if (tps <= 8) hipLaunchKernelGGL((gemv_half_kernel<FMT, 4, 2, MMAX>), grid, dim3(256), 0, s, a);
    else if (tps <= 16) hipLaunchKernelGGL((gemv_half_kernel<FMT, 8, 2, MMAX>), grid, dim3(512), 0, s, a);
    else if (tps <= 32) hipLaunchKernelGGL((gemv_half_kernel<FMT, 8, 4, MMAX>), grid, dim3(512), 0, s, a);
    else if (tps <= 8 * GEMV_HALF_TPW) hipLaunchKernelGGL((gemv_half_kernel<FMT, 8, GEMV_HALF_TPW, MMAX>), grid, dim3(512), 0, s, a);
    else return false;
    return true;
  }
}

template <int FMT>
static bool launch_gemv_dot(const GemvArgs& a, int tps, int rows, hipStream_t s) {
  if (rows == 8) return launch_gemv_half<FMT, 1>(a, tps, s);
  if (rows != 16) return false;
  return tps >= 16 ? launch_gemv_dot_w<FMT, 16>(a, tps, s) : launch_gemv_dot_w<FMT, 8>(a, tps, s);
}

// grid: x = row blocks, y = K splits; a chunk covers at most GEMV_MFMA_KW of
// K, a wave up to GEMV_MFMA_CH chunks (1, 2, 4 or 8, the fewest that hold its tiles)
template <int FMT, int MROWS>
static bool launch_gemv_mfma(const GemvArgs& a, int tps, hipStream_t s) {
  constexpr int TMAX = GEMV_MFMA_KW / Fmt<FMT>::KT;
  const int tpw = (tps + GEMV_THREADS / 64 - 1) / (GEMV_THREADS / 64);
  static_assert(TMAX >= 1 && gemv_mfma_lds_bytes<FMT, MROWS, TMAX>() <= 80 * 1024,
                "MFMA GEMV LDS: at least two workgroups per CU");
  static_assert(GEMV_MFMA_CH == 8, "chunk counts instantiated below");
  const dim3 grid((unsigned)a.rowblocks, (unsigned)a.splits), block(GEMV_THREADS);
  if (tpw > TMAX * GEMV_MFMA_CH) return false;
  if (tpw <= 1) hipLaunchKernelGGL((gemv_mfma_kernel<FMT, MROWS, 1, 1>), grid, block, 0, s, a);
  else if (tpw <= TMAX) hipLaunchKernelGGL((gemv_mfma_kernel<FMT, MROWS, TMAX, 1>), grid, block, 0, s, a);
  else if (tpw <= 2 * TMAX) hipLaunchKernelGGL((gemv_mfma_kernel<FMT, MROWS, TMAX, 2>), grid, block, 0, s, a);
  else if (tpw <= 4 * TMAX) hipLaunchKernelGGL((gemv_mfma_kernel<FMT, MROWS, TMAX, 4>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((gemv_mfma_kernel<FMT, MROWS, TMAX, 8>), grid, block, 0, s, a);
  return true;
}

// mmax 1: v_dot2 GEMV (16- or 8-row workgroups); 2: v_dot2 on 8-row workgroups;
// 4: MFMA GEMV or v_dot2 on 8-row workgroups; 8, 16: MFMA GEMV
template <int FMT>
static bool launch_gemv_f(const GemvArgs& a, int mmax, int tps, int rows, hipStream_t s) {
  switch (mmax) {
    case 1: return launch_gemv_dot<FMT>(a, tps, rows, s);
    case 2: return rows == 8 && launch_gemv_half<FMT, 2>(a, tps, s);
    case 4: return rows == 8 ? launch_gemv_half<FMT, 4>(a, tps, s) : launch_gemv_mfma<FMT, 4>(a, tps, s);
    case 8: return launch_gemv_mfma<FMT, 8>(a, tps, s);
    default: return launch_gemv_mfma<FMT, 16>(a, tps, s);
  }
}

// grid: x = column tiles, y = row tiles, z = K splits; MB x NB blocks of 32 x 32.
// D x stages in flight per wave (launch_gemm_tiles picks it).  A second x
// stage adds L2 traffic at the start and no bandwidth on 64-row tiles: every
// CU of an XCD pulls its stage at once, at the L2's rate.  With one x stage in
// flight the codes of the next stage are already loading (their HBM latency
// hides under the current stage's compute).  TPW is the fewest word tiles per wave (1, 2, 4, or 8 on 32 x 32
// tiles) that cover the split, since every wave issues all TPW * STAGES stages.
template <int FMT, int D, int MB, int NB, int TPW>
static void launch_gemm_tpw(const GemmArgs& a, const Plan& p, hipStream_t s) {
  const dim3 grid((unsigned)p.tiles_n, (unsigned)p.tiles_m, (unsigned)p.splits), block(GEMM_THREADS);
  constexpr int NW = GEMM_THREADS / 64;
  constexpr int CP = D == 1 ? 2 : 1;   // one x stage in flight: the codes run a stage ahead
  // issue every stage in every wave when that wastes at most an eighth of them
  if ((int64_t)8 * (NW * TPW - p.tps) <= NW * TPW)
    hipLaunchKernelGGL((gemm_kernel<FMT, NW, TPW, D, MB, NB, true, CP>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((gemm_kernel<FMT, NW, TPW, D, MB, NB, false, CP>), grid, block, 0, s, a);
}

template <int FMT, int D, int MB, int NB>
static void launch_gemm_fmt(const GemmArgs& a, const Plan& p, hipStream_t s) {
  constexpr int NW = GEMM_THREADS / 64;
  constexpr int TMAX = MB * NB == 1 ? GEMM_TPW_SMALL : FMT == Q8_0 ? GEMM_TPW_Q8 : GEMM_TPW;
  static_assert(TMAX == 2 || TMAX == 4 || TMAX == 8, "tile counts instantiated below");
  const int per = (int)ceil_div(p.tps, NW);   // <= TMAX (the plan's cap)
  if (per <= 1) launch_gemm_tpw<FMT, D, MB, NB, 1>(a, p, s);
  else if (per <= 2 || TMAX == 2) launch_gemm_tpw<FMT, D, MB, NB, 2>(a, p, s);
  else if (per <= 4 || TMAX == 4) launch_gemm_tpw<FMT, D, MB, NB, (TMAX >= 4 ? 4 : 2)>(a, p, s);
  else launch_gemm_tpw<FMT, D, MB, NB, TMAX>(a, p, s);
}

template <int MB, int NB, int D>
static void launch_gemm_depth(const GemmArgs& a, const Plan& p, int fmt, hipStream_t s) {
  switch (fmt) {
    case QG_INT4_ASYM: launch_gemm_fmt<INT4_ASYM, D, MB, NB>(a, p, s); break;
    case QG_INT2_ASYM: launch_gemm_fmt<INT2_ASYM, D, MB, NB>(a, p, s); break;
    case QG_Q8_0: launch_gemm_fmt<Q8_0, D, MB, NB>(a, p, s); break;
    case QG_Q4K: launch_gemm_fmt<Q4K, D, MB, NB>(a, p, s); break;
    default: launch_gemm_fmt<Q4_0, D, MB, NB>(a, p, s); break;
  }
}

// One x stage in flight per wave, with the codes a stage ahead, on 64-row
// tiles and on 32 x 32 tiles up to M = 32; two x stages on 32 x 32 tiles for
// larger M, where that measured faster (the looped block's down projection,
// 128 x 2048 x 8192: 14.9 against 15.4 us).
template <int MB, int NB>
static void launch_gemm_tiles(const GemmArgs& a, const Plan& p, int fmt, hipStream_t s) {
  if constexpr (MB * NB == 1) {
    if (a.M > 32) {
      launch_gemm_depth<MB, NB, GEMM_DEPTH>(a, p, fmt, s);
      return;
    }
  }
  launch_gemm_depth<MB, NB, 1>(a, p, fmt, s);
}

// QGEMM_CHECK=1: every device pointer of a call must be device (or managed)
// memory of the current device; host memory is rejected before any launch.
// Costs one hipPointerGetAttributes per pointer, so it is off by default.
static bool pointer_check_on() {
  const char* v = getenv("QGEMM_CHECK");
  return v && v[0] == '1' && v[1] == 0;
}

static int check_device_pointers(const void* const* ptrs, int n) {
  if (!pointer_check_on()) return QG_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    clear_pending_error();
    return QG_E_DEVICE;
  }
  for (int i = 0; i < n; ++i) {
    if (!ptrs[i]) continue;
    hipPointerAttribute_t attr;
    memset(&attr, 0, sizeof(attr));
    const hipError_t e = hipPointerGetAttributes(&attr, ptrs[i]);
    if (e != hipSuccess) clear_pending_error();   // unregistered host memory reports an error
    const int st = classify_pointer((int)e, (int)attr.type, attr.device, dev);
    if (st != QG_OK) return st;
  }
  return QG_OK;
}

// Host-only validation of a call and its launch plan; no HIP call.
int validate_call(const Call& c, Plan* plan) {
  int st = check_shape(c.M, c.N, c.K, c.group, c.fmt);
  if (st != QG_OK) return st;
  if (c.M > 0 && c.N > 0) {
    if (!c.y) return QG_E_ARG;
    if (check_ld(c.ldy, c.N) != QG_OK) return QG_E_ARG;
    if (c.resid && check_ld(c.ldr, c.N) != QG_OK) return QG_E_ARG;
    if (c.resid && c.resid == c.y && c.ldr != c.ldy) return QG_E_ARG;
    if (check_align(c.y) != QG_OK || (c.resid && check_align(c.resid) != QG_OK)) return QG_E_ALIGN;
    if (c.K > 0) {
      if (!c.x || !c.packed || !c.scales) return QG_E_ARG;
      if (symmetric_format(c.fmt) != (c.zeros == nullptr)) return QG_E_ARG;
      if (check_ld(c.ldx, c.K) != QG_OK) return QG_E_ARG;
      if (c.ldx % 8 != 0) return QG_E_ALIGN;
      if (check_align(c.x) != QG_OK || check_align(c.packed) != QG_OK || check_align(c.scales) != QG_OK ||
          (c.zeros && check_align(c.zeros) != QG_OK))
        return QG_E_ALIGN;
    }
  }
  const Plan p = make_plan(c.M, c.N, c.K, c.group, c.fmt);
  if (c.M > 0 && c.N > 0 && c.K > 0) {
    if (p.path == 0) return QG_E_UNSUPPORTED;
    // the kernels form byte offsets of x rows and of one row block's codes in 32 bits
    if ((int64_t)c.M * c.ldx * 2 >= (int64_t)1 << 32 || p.splits > 65535) return QG_E_UNSUPPORTED;
    if (p.path == 1 && (int64_t)p.wordtiles * 1024 >= (int64_t)1 << 32) return QG_E_UNSUPPORTED;
    if (p.path == 2 && p.tiles_m > 65535) return QG_E_UNSUPPORTED;
  }
  *plan = p;
  return QG_OK;
}

// Launches a validated call on the current device.  ws: the split-K partials
// (at least p.ws_bytes() bytes) when the plan splits K.
int launch_call(const Call& c, const Plan& p, float* wsf, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  clear_pending_error();
  const int M = c.M, N = c.N, K = c.K, fmt = c.fmt;
  if (K == 0) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for((int64_t)M * N, 256)), dim3(256), 0, s,
                       reinterpret_cast<f16*>(c.y), M, N, c.ldy, reinterpret_cast<const f16*>(c.resid), c.ldr);
    return launch_status();
  }
  if (p.path == 1) {
    GemvArgs a;
    a.x = reinterpret_cast<const f16*>(c.x);
    a.packed = c.packed;
    a.scales = reinterpret_cast<const f16*>(c.scales);
    a.zeros = reinterpret_cast<const f16*>(c.zeros);
    a.resid = reinterpret_cast<const f16*>(c.resid);
    a.y = reinterpret_cast<f16*>(c.y);
    a.ws = wsf;
    a.ldx = c.ldx; a.ldr = c.ldr; a.ldy = c.ldy;
    a.M = M; a.N = N; a.K = K; a.group = meta_group(fmt, c.group);   // q4k: the 32-weight sub-block
    a.wordtiles = p.wordtiles; a.rowblocks = p.rowblocks; a.splits = p.splits; a.tps = p.tps;
    bool launched;
    switch (fmt) {
      case QG_INT4_ASYM: launched = launch_gemv_f<INT4_ASYM>(a, p.mmax, p.tps, p.rows, s); break;
      case QG_INT2_ASYM: launched = launch_gemv_f<INT2_ASYM>(a, p.mmax, p.tps, p.rows, s); break;
      case QG_Q8_0: launched = launch_gemv_f<Q8_0>(a, p.mmax, p.tps, p.rows, s); break;
      case QG_Q4K: launched = launch_gemv_f<Q4K>(a, p.mmax, p.tps, p.rows, s); break;
      default: launched = launch_gemv_f<Q4_0>(a, p.mmax, p.tps, p.rows, s); break;
    }
    if (!launched) return QG_E_UNSUPPORTED;
    if (p.splits > 1) {
      const int st = launch_status();
      if (st != QG_OK) return st;
      hipLaunchKernelGGL(gemv_reduce_kernel, dim3(grid_for((int64_t)M * N, 256)), dim3(256), 0, s, wsf,
                         a.resid, a.y, M, N, c.ldr, c.ldy, p.splits, p.mmax);
    }
    return launch_status();
  }
  GemmArgs a;
  a.x = reinterpret_cast<const f16*>(c.x);
  a.packed = c.packed;
  a.scales = reinterpret_cast<const f16*>(c.scales);
  a.zeros = reinterpret_cast<const f16*>(c.zeros);
  a.resid = reinterpret_cast<const f16*>(c.resid);
  a.y = reinterpret_cast<f16*>(c.y);
  a.ws = wsf;
  a.ldx = c.ldx; a.ldr = c.ldr; a.ldy = c.ldy;
  a.M = M; a.N = N; a.K = K; a.group = meta_group(fmt, c.group);   // q4k: the 32-weight sub-block
  a.wordtiles = p.wordtiles; a.rowblocks = p.rowblocks; a.tiles_n = p.tiles_n;
  a.splits = p.splits; a.tps = p.tps;
  if (p.tm == 32) launch_gemm_tiles<1, 1>(a, p, fmt, s);
  else if (p.tn == 32) launch_gemm_tiles<2, 1>(a, p, fmt, s);
  else launch_gemm_tiles<2, 2>(a, p, fmt, s);
  if (p.splits > 1) {
    const int st = launch_status();
    if (st != QG_OK) return st;
    if (p.tm == 32)
      hipLaunchKernelGGL((gemm_reduce_kernel<1, 1>), dim3((unsigned)p.tiles_n, (unsigned)p.tiles_m, 1), dim3(256), 0, s, a);
    else if (p.tn == 32)
      hipLaunchKernelGGL((gemm_reduce_kernel<2, 1>), dim3((unsigned)p.tiles_n, (unsigned)p.tiles_m, 2), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((gemm_reduce_kernel<2, 2>), dim3((unsigned)p.tiles_n, (unsigned)p.tiles_m, 4), dim3(256), 0, s, a);
  }
  return launch_status();
}

int call_pointers_ok(const Call& c) {
  const void* ptrs[6] = {c.x, c.packed, c.scales, c.zeros, c.resid, c.y};
  return check_device_pointers(ptrs, 6);
}

static int run_qgemm(const Call& c, void* workspace, size_t ws_bytes, void* stream) {
  Plan p;
  int st = validate_call(c, &p);
  if (st != QG_OK) return st;
  if (workspace && ws_bytes < p.ws_bytes()) return QG_E_WORKSPACE;
  if (workspace && check_align(workspace) != QG_OK) return QG_E_ALIGN;
  if (c.M == 0 || c.N == 0) return QG_OK;  // no-op, no HIP call
  int dev = 0;
  st = current_device(&dev);
  if (st != QG_OK) return st;
  st = call_pointers_ok(c);
  if (st != QG_OK) return st;
  if (workspace) {
    const void* w[1] = {workspace};
    st = check_device_pointers(w, 1);
    if (st != QG_OK) return st;
  }
  void* ws = workspace;
  if (p.ws_bytes() > 0 && !ws) {
    st = library_ws(dev, p.ws_bytes(), &ws);
    if (st != QG_OK) return st;
  }
  return launch_call(c, p, reinterpret_cast<float*>(ws), stream);
}

static int check_pack(const void* a, const void* b, int N, int K, int fmt) {
  if (!valid_format(fmt) || N < 0 || K < 0) return QG_E_ARG;
  if (K % cpw_of(fmt) != 0) return QG_E_ARG;
  if ((int64_t)N * K > 0) {
    if (!a || !b) return QG_E_ARG;
    if (check_align(a) != QG_OK || check_align(b) != QG_OK) return QG_E_ALIGN;
  }
  return QG_OK;
}

}  // namespace qg

using namespace qg;

extern "C" {

const char* qg_last_error(void) { return hipGetErrorString(g_last_hip); }

int qpack(const uint32_t* canon, uint32_t* packed, int N, int K, int fmt, void* stream) {
  int st = check_pack(canon, packed, N, K, fmt);
  if (st != QG_OK) return st;
  int dev = 0;
  st = current_device(&dev);
  if (st != QG_OK) return st;
  {
    const void* ptrs[2] = {canon, packed};
    st = check_device_pointers(ptrs, (int64_t)N * K > 0 ? 2 : 0);
    if (st != QG_OK) return st;
  }
  clear_pending_error();
  const int64_t total = (int64_t)(qg_packed_bytes(N, K, fmt) / sizeof(uint32_t));
  if (total == 0) return QG_OK;
  hipLaunchKernelGGL(qpack_kernel, dim3(grid_for(total, 256)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), canon, packed, N, K / cpw_of(fmt),
                     (int)n_wordtiles(K, fmt), bits_of(fmt), total);
  return launch_status();
}

int qunpack(const uint32_t* packed, uint32_t* canon, int N, int K, int fmt, void* stream) {
  int st = check_pack(packed, canon, N, K, fmt);
  if (st != QG_OK) return st;
  int dev = 0;
  st = current_device(&dev);
  if (st != QG_OK) return st;
  {
    const void* ptrs[2] = {packed, canon};
    st = check_device_pointers(ptrs, (int64_t)N * K > 0 ? 2 : 0);
    if (st != QG_OK) return st;
  }
  clear_pending_error();
  const int64_t total = (int64_t)N * (K / cpw_of(fmt));
  if (total == 0) return QG_OK;
  hipLaunchKernelGGL(qunpack_kernel, dim3(grid_for(total, 256)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), packed, canon, N, K / cpw_of(fmt),
                     (int)n_wordtiles(K, fmt), bits_of(fmt));
  return launch_status();
}

int qg_unpack_codes(const uint32_t* packed, uint8_t* codes, int N, int K, int fmt, void* stream) {
  int st = check_pack(packed, codes, N, K, fmt);
  if (st != QG_OK) return st;
  int dev = 0;
  st = current_device(&dev);
  if (st != QG_OK) return st;
  {
    const void* ptrs[2] = {packed, codes};
    st = check_device_pointers(ptrs, (int64_t)N * K > 0 ? 2 : 0);
    if (st != QG_OK) return st;
  }
  clear_pending_error();
  const int64_t total = (int64_t)N * K;
  if (total == 0) return QG_OK;
  hipLaunchKernelGGL(unpack_codes_kernel, dim3(grid_for(total, 256)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), packed, codes, N, K,
                     (int)n_wordtiles(K, fmt), bits_of(fmt));
  return launch_status();
}

int qg_dequant(const uint32_t* packed, const uint16_t* scales, const uint16_t* zeros, uint16_t* w,
               int N, int K, int group, int fmt, void* stream) {
  int st = check_shape(1, N, K, group, fmt);
  if (st != QG_OK) return st;
  const int64_t total = (int64_t)N * (K / cpw_of(fmt));
  if (total > 0) {
    if (!packed || !scales || !w) return QG_E_ARG;
    if (symmetric_format(fmt) != (zeros == nullptr)) return QG_E_ARG;
    if (check_align(packed) != QG_OK || check_align(w) != QG_OK || check_align(scales) != QG_OK ||
        (zeros && check_align(zeros) != QG_OK))
      return QG_E_ALIGN;
  }
  if (total == 0) return QG_OK;
  int dev = 0;
  st = current_device(&dev);
  if (st != QG_OK) return st;
  {
    const void* ptrs[4] = {packed, scales, zeros, w};
    st = check_device_pointers(ptrs, 4);
    if (st != QG_OK) return st;
  }
  clear_pending_error();
  const int wt = (int)n_wordtiles(K, fmt);
  const int64_t units = n_rowblocks(N) * wt;
  const int mg = meta_group(fmt, group);
  const dim3 grid((unsigned)ceil_div(units, 4)), block(256);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const f16* sc = reinterpret_cast<const f16*>(scales);
  const f16* zp = reinterpret_cast<const f16*>(zeros);
  f16* wo = reinterpret_cast<f16*>(w);
  switch (fmt) {
    case QG_INT4_ASYM: hipLaunchKernelGGL(dequant_kernel<INT4_ASYM>, grid, block, 0, s, packed, sc, zp, wo, N, K, mg, wt, units); break;
    case QG_INT2_ASYM: hipLaunchKernelGGL(dequant_kernel<INT2_ASYM>, grid, block, 0, s, packed, sc, zp, wo, N, K, mg, wt, units); break;
    case QG_Q8_0: hipLaunchKernelGGL(dequant_kernel<Q8_0>, grid, block, 0, s, packed, sc, zp, wo, N, K, mg, wt, units); break;
    case QG_Q4K: hipLaunchKernelGGL(dequant_kernel<Q4K>, grid, block, 0, s, packed, sc, zp, wo, N, K, mg, wt, units); break;
    default: hipLaunchKernelGGL(dequant_kernel<Q4_0>, grid, block, 0, s, packed, sc, zp, wo, N, K, mg, wt, units); break;
  }
  return launch_status();
}

int qgemm(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint16_t* zeros,
          int M, int N, int K, int group, int fmt, uint16_t* y, void* stream) {
  const Call c{x, K, packed, scales, zeros, nullptr, N, M, N, K, group, fmt, y, N};
  return run_qgemm(c, nullptr, 0, stream);
}

int qgemm_ex(const uint16_t* x, int ldx, const uint32_t* packed, const uint16_t* scales,
             const uint16_t* zeros, const uint16_t* residual, int ldr, int M, int N, int K, int group,
             int fmt, uint16_t* y, int ldy, void* workspace, size_t ws_bytes, void* stream) {
  const Call c{x, ldx, packed, scales, zeros, residual, ldr, M, N, K, group, fmt, y, ldy};
  return run_qgemm(c, workspace, ws_bytes, stream);
}

// The four calls of a loop of the shared block (QKV, O + x, up, down + h),
// validated with their plans and workspace size; nothing is launched.
struct LoopSetup {
  Call calls[4];
  Plan plans[4];
  size_t ws_need = 0;
};

static int loop_setup(uint16_t* x, const uint32_t* const* packed4, const uint16_t* const* scales4,
                      const uint16_t* const* zeros4, int M, int D, int F, int group, int fmt, int L,
                      uint16_t* scratch, LoopSetup* ls) {
  if (!packed4 || !scales4 || !zeros4 || L < 0 || D <= 0 || F <= 0 || M < 0) return QG_E_ARG;
  if (M > 0 && (!x || !scratch)) return QG_E_ARG;
  if (check_align(scratch) != QG_OK || check_align(x) != QG_OK) return QG_E_ALIGN;
  const int64_t D3 = 3 * (int64_t)D;
  if (D3 > INT_MAX) return QG_E_ARG;
  uint16_t* qkv = scratch;
  uint16_t* h = qkv + (int64_t)M * D3;
  uint16_t* u = h + (int64_t)M * D;
  const Call calls[4] = {
      {x, D, packed4[0], scales4[0], zeros4[0], nullptr, 0, M, (int)D3, D, group, fmt, qkv, (int)D3},
      {qkv + 2 * (int64_t)D, (int)D3, packed4[1], scales4[1], zeros4[1], x, D, M, D, D, group, fmt, h, D},
      {h, D, packed4[2], scales4[2], zeros4[2], nullptr, 0, M, F, D, group, fmt, u, F},
      {u, F, packed4[3], scales4[3], zeros4[3], h, D, M, D, F, group, fmt, x, D}};
  for (int i = 0; i < 4; ++i) {
    ls->calls[i] = calls[i];
    const int st = validate_call(calls[i], &ls->plans[i]);
    if (st != QG_OK) return st;
    ls->ws_need = std::max(ls->ws_need, ls->plans[i].ws_bytes());
  }
  return QG_OK;
}

static int record_event(void* const* events, int i, hipStream_t s) {
  if (events && events[i] && hip_status(hipEventRecord(reinterpret_cast<hipEvent_t>(events[i]), s)) != QG_OK)
    return QG_E_DEVICE;
  return QG_OK;
}

int qloop_block(uint16_t* x, const uint32_t* const* packed4, const uint16_t* const* scales4,
                const uint16_t* const* zeros4, int M, int D, int F, int group, int fmt, int L,
                uint16_t* scratch, void* const* events, void* stream) {
  // the four calls of a loop, validated (and their workspace obtained) before
  // anything is recorded or launched
  LoopSetup ls;
  int st = loop_setup(x, packed4, scales4, zeros4, M, D, F, group, fmt, L, scratch, &ls);
  if (st != QG_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (M == 0 || L == 0) {   // still time-stamp the (empty) loops
    for (int l = 0; l <= L; ++l)
      if (record_event(events, l, s) != QG_OK) return QG_E_DEVICE;
    return QG_OK;
  }
  int dev = 0;
  st = current_device(&dev);
  if (st != QG_OK) return st;
  for (int i = 0; i < 4; ++i) {
    st = call_pointers_ok(ls.calls[i]);
    if (st != QG_OK) return st;
  }
  void* ws = nullptr;
  if (ls.ws_need > 0) {
    st = library_ws(dev, ls.ws_need, &ws);
    if (st != QG_OK) return st;
  }
  if (record_event(events, 0, s) != QG_OK) return QG_E_DEVICE;
  for (int l = 0; l < L; ++l) {
    for (int i = 0; i < 4; ++i) {
      st = launch_call(ls.calls[i], ls.plans[i], reinterpret_cast<float*>(ws), s);
      if (st != QG_OK) return st;
    }
    if (record_event(events, l + 1, s) != QG_OK) return QG_E_DEVICE;
  }
  return QG_OK;
}

// --- the persistent looped block ------------------------------------------

static std::vector<unsigned*> g_loop_counter;   // per device, kept until the process ends

static int loop_counter(int dev, unsigned** out) {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  if ((int)g_loop_counter.size() <= dev) g_loop_counter.resize(dev + 1, nullptr);
  if (!g_loop_counter[dev]) {
    void* p = nullptr;
    if (hipMalloc(&p, LOOP_COUNTERS * LOOP_COUNTER_STRIDE * sizeof(unsigned)) != hipSuccess) {
      clear_pending_error();
      return QG_E_NOMEM;
    }
    g_loop_counter[dev] = reinterpret_cast<unsigned*>(p);
  }
  *out = g_loop_counter[dev];
  return QG_OK;
}

// word tiles per wave (2, 4 or 8) for 8 waves over `wordtiles`, 0 if more
static int loop_tpw(int64_t wordtiles) {
  for (int t = 2; t <= 8; t *= 2)
    if (8 * t >= wordtiles) return t;
  return 0;
}

extern "C++" {
template <int FMT, bool ALL>
static const void* loop_kernel_for(int ta, int tb) {
  if (ta == 2 && tb == 2) return reinterpret_cast<const void*>(&loop_block_kernel<FMT, 2, 2, ALL>);
  if (ta == 2 && tb == 4) return reinterpret_cast<const void*>(&loop_block_kernel<FMT, 2, 4, ALL>);
  if (ta == 2 && tb == 8) return reinterpret_cast<const void*>(&loop_block_kernel<FMT, 2, 8, ALL>);
  if (ta == 4 && tb == 4) return reinterpret_cast<const void*>(&loop_block_kernel<FMT, 4, 4, ALL>);
  if (ta == 4 && tb == 8) return reinterpret_cast<const void*>(&loop_block_kernel<FMT, 4, 8, ALL>);
  if (ta == 8 && tb == 8) return reinterpret_cast<const void*>(&loop_block_kernel<FMT, 8, 8, ALL>);
  return nullptr;
}
template <bool ALL>
static const void* loop_kernel_all(int fmt, int ta, int tb) {
  switch (fmt) {
    case QG_INT4_ASYM: return loop_kernel_for<INT4_ASYM, ALL>(ta, tb);
    case QG_INT2_ASYM: return loop_kernel_for<INT2_ASYM, ALL>(ta, tb);
    case QG_Q4_0: return loop_kernel_for<Q4_0, ALL>(ta, tb);
    case QG_Q4K: return loop_kernel_for<Q4K, ALL>(ta, tb);
    default: return nullptr;
  }
}
}  // extern "C++"

static const void* loop_kernel(int fmt, int ta, int tb, bool all) {
  return all ? loop_kernel_all<true>(fmt, ta, tb) : loop_kernel_all<false>(fmt, ta, tb);
}

int qloop_block_persistent(uint16_t* x, const uint32_t* const* packed4, const uint16_t* const* scales4,
                           const uint16_t* const* zeros4, int M, int D, int F, int group, int fmt, int L,
                           uint16_t* scratch, int mode, int* status, void* const* events, void* stream) {
  LoopSetup ls;
  int st = loop_setup(x, packed4, scales4, zeros4, M, D, F, group, fmt, L, scratch, &ls);
  if (st != QG_OK) return st;
  if (!status || (mode != 0 && mode != 1)) return QG_E_ARG;
  if (check_align(status) != QG_OK) return QG_E_ALIGN;
  if (M != 1) return QG_E_UNSUPPORTED;
  const int ta = loop_tpw(ls.plans[0].wordtiles), tb = loop_tpw(ls.plans[3].wordtiles);
  for (int i = 0; i < 3; ++i)
    if (ls.plans[i].wordtiles != ls.plans[0].wordtiles) return QG_E_UNSUPPORTED;
  const void* fn = ta && tb ? loop_kernel(fmt, ta, tb, mode == 1) : nullptr;
  if (!fn) return QG_E_UNSUPPORTED;
  int dev = 0;
  st = current_device(&dev);
  if (st != QG_OK) return st;
  for (int i = 0; i < 4; ++i) {
    st = call_pointers_ok(ls.calls[i]);
    if (st != QG_OK) return st;
  }
  const void* sp[1] = {status};
  st = check_device_pointers(sp, 1);
  if (st != QG_OK) return st;
  // the grid: one workgroup per compute unit (measured fastest: the barrier's
  // cost grows with the workgroup count faster than the phases shrink), never
  // more than are resident together, nor more than the widest phase's half
  // row blocks.  A plain launch: a cooperative one measured about 16 us more
  // per loop; if other work keeps some workgroups from starting, the bounded
  // waits end the kernel and *status reports it.
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, LOOP_THREADS, 0) != hipSuccess || per_cu < 1) {
    clear_pending_error();
    return QG_E_DEVICE;
  }
  int64_t widest = 0;
  for (int i = 0; i < 4; ++i) widest = std::max<int64_t>(widest, 2 * (int64_t)ls.plans[i].rowblocks);
  int64_t grid = std::min<int64_t>(std::min<int64_t>((int64_t)per_cu * cus, cus), widest);
  const int grid_env = env_int("QGEMM_LOOP_GRID", 0);
  if (grid_env > 0) grid = std::min<int64_t>(grid, grid_env);
  if ((int64_t)4 * L * grid >= (int64_t)UINT_MAX) return QG_E_UNSUPPORTED;   // the counters' range
  unsigned* counter = nullptr;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (L > 0) {
    st = loop_counter(dev, &counter);
    if (st != QG_OK) return st;
  }
  if (record_event(events, 0, s) != QG_OK) return QG_E_DEVICE;
  if (L == 0) return QG_OK;
  hipLaunchKernelGGL(loop_reset_kernel, dim3(1), dim3(1), 0, s, counter, status);
  st = launch_status();
  if (st != QG_OK) return st;
  LoopArgs la;
  for (int i = 0; i < 4; ++i) {
    const Call& c = ls.calls[i];
    const Plan& p = ls.plans[i];
    GemvArgs& a = la.lin[i];
    a.x = reinterpret_cast<const f16*>(c.x);
    a.packed = c.packed;
    a.scales = reinterpret_cast<const f16*>(c.scales);
    a.zeros = reinterpret_cast<const f16*>(c.zeros);
    a.resid = reinterpret_cast<const f16*>(c.resid);
    a.y = reinterpret_cast<f16*>(c.y);
    a.ws = nullptr;
    a.ldx = c.ldx; a.ldr = c.ldr; a.ldy = c.ldy;
    a.M = c.M; a.N = c.N; a.K = c.K; a.group = meta_group(fmt, c.group);
    a.wordtiles = p.wordtiles; a.rowblocks = p.rowblocks; a.splits = 1; a.tps = p.wordtiles;
  }
  la.counter = counter;
  la.status = status;
  la.cap = env_int("QGEMM_LOOP_SPIN_CAP", 1 << 18);
  // mode 0: one launch per loop (3 barriers each); mode 1: one launch for all
  // L loops (4 barriers per loop but the last), after which every per-loop
  // event is recorded
  const int launches = mode == 1 ? 1 : L;
  for (int l = 0; l < launches; ++l) {
    la.barrier0 = 3 * l;
    la.loops = mode == 1 ? L : 1;
    void* args[1] = {&la};
    st = hip_status(hipLaunchKernel(fn, dim3((unsigned)grid), dim3(LOOP_THREADS), args, 0, s));
    if (st != QG_OK) {
      clear_pending_error();
      return st;
    }
    for (int e = mode == 1 ? 1 : l + 1; e <= (mode == 1 ? L : l + 1); ++e)
      if (record_event(events, e, s) != QG_OK) return QG_E_DEVICE;
  }
  return QG_OK;
}

}  // extern "C"
