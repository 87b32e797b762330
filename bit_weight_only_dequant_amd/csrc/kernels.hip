// kernels.hip - HIP kernels for gfx950 (CDNA4) and the device entry points of
// libqgemm: y = x . dequant(W)^T for low-bit group-quantized weights.
//
// The operation is the dequantizing matmul of the skyzh/tiny-llm feature list
// ("Dequantizing Runtimes", "Quantized Matrix Multiplication"): weights are
// brought back to full precision inside the compute pass, never written out.
// Formats: INT4 / INT2 with per-group fp16 scale and zero point (TinyLoop
// README, "Status" and "Current Runtime Snapshot"), q4_0 (torchnative guide
// "Inference with real transformers", "Quantise while loading").
//
// Kernels
//   qpack / qunpack      one-time permutation of codes into the tile order of
//                        layout.h (HBM-bound, elementwise).
//   gemv<FMT, MMAX>      M <= 8.  Bandwidth-bound.  One 16-byte code load per
//                        lane per 16x16-word tile, unpack by mask into fp16
//                        pairs holding exact (q - z), v_dot2_f32_f16 against x
//                        staged in LDS, fp32 scale per group, reduction over
//                        lane groups and waves through LDS.
//   gemm<FMT>            M > 8.  128x128 workgroup tile, 2x2 waves of 64x64.
//                        x tiles staged in LDS (double-buffered); codes go
//                        straight from HBM to VGPRs in the MFMA B-operand
//                        layout, dequantized to fp16 s*(q-z) in registers and
//                        fed to v_mfma_f32_16x16x32_f16 (fp32 accumulation).
//   Split-K (both)       fp32 partials in a workspace; the last workgroup of a
//                        tile to arrive sums them in split order (deterministic)
//                        and resets the tile's counter.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
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

// 4-bit packed word (8 codes) -> 4 pairs (c_2i - z, c_2i+1 - z), i = 0..3
__device__ __forceinline__ void qmz_int4(uint32_t w, const ZC4& zc, h2 out[4]) {
  const h2 inv16 = splat((f16)0.0625f);
  const uint32_t w8 = w >> 8;
  out[0] = as_h2((w & 0x000F000Fu) | 0x64006400u) + zc.c0;
  out[1] = as_h2((w & 0x00F000F0u) | 0x64006400u) * inv16 + zc.c1;
  out[2] = as_h2((w8 & 0x000F000Fu) | 0x64006400u) + zc.c0;
  out[3] = as_h2((w8 & 0x00F000F0u) | 0x64006400u) * inv16 + zc.c1;
}

// 2-bit packed word, one half (8 codes): half 0 = codes 0..7, half 1 = 8..15
__device__ __forceinline__ void qmz_int2_half(uint32_t w, int half, const ZC2& zc, h2 out[4]) {
  const uint32_t v = half ? (w >> 8) : w;
  out[0] = as_h2((v & 0x00030003u) | 0x64006400u) + zc.c0;
  out[1] = as_h2((v & 0x000C000Cu) | 0x64006400u) * splat((f16)0.25f) + zc.c1;
  out[2] = as_h2((v & 0x00300030u) | 0x64006400u) * splat((f16)0.0625f) + zc.c2;
  out[3] = as_h2((v & 0x00C000C0u) | 0x64006400u) * splat((f16)0.015625f) + zc.c3;
}

template <int FMT> struct Fmt;
template <> struct Fmt<INT4_ASYM> { static constexpr int BITS = 4, CPW = 8,  LS = 32, KT = 128; static constexpr bool HAS_Z = true; };
template <> struct Fmt<INT2_ASYM> { static constexpr int BITS = 2, CPW = 16, LS = 64, KT = 256; static constexpr bool HAS_Z = true; };
template <> struct Fmt<Q4_0>      { static constexpr int BITS = 4, CPW = 8,  LS = 32, KT = 128; static constexpr bool HAS_Z = false; };

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

// One thread per canonical word: the GEMM's register dequant, written out.
template <int FMT>
__global__ void dequant_kernel(const uint32_t* __restrict__ packed, const f16* __restrict__ scales,
                               const f16* __restrict__ zeros, f16* __restrict__ w,
                               int N, int K, int group, int wordtiles) {
  using F = Fmt<FMT>;
  const int Kw = K / F::CPW, ng = K / group;
  const int64_t total = (int64_t)N * Kw;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = i / Kw, kw = i % Kw;
    const uint32_t word = packed[packed_index(n, kw, wordtiles)];
    const int grp = (int)(kw * F::CPW / group);
    const h2 s2 = splat(scales[n * ng + grp]);
    const f16 z = F::HAS_Z ? zeros[n * ng + grp] : (f16)8.0f;
    h2 out[8];
    if constexpr (FMT == INT2_ASYM) {
      const ZC2 zc = make_zc2(z);
      qmz_int2_half(word, 0, zc, out);
      qmz_int2_half(word, 1, zc, out + 4);
    } else {
      qmz_int4(word, make_zc4(z), out);
    }
    h2* dst = reinterpret_cast<h2*>(w + n * K + kw * F::CPW);
#pragma unroll
    for (int p = 0; p < F::CPW / 2; ++p) dst[p] = out[p] * s2;
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
// decode GEMV (M <= 8)
// ---------------------------------------------------------------------------
struct GemvArgs {
  const f16* x; const uint32_t* packed; const f16* scales; const f16* zeros;
  const f16* resid; f16* y; float* ws; uint32_t* cnt;
  int ldx, ldr, ldy, M, N, K, group;
  int wordtiles, rowblocks, splits, tps;
};

template <int FMT, int MMAX>
__global__ __launch_bounds__(GEMV_THREADS) void gemv_kernel(GemvArgs a) {
  using F = Fmt<FMT>;
  constexpr int TPW = GEMV_TPW_MAX;
  extern __shared__ __align__(16) uint8_t gemv_smem[];
  f16* xs = reinterpret_cast<f16*>(gemv_smem);                       // [MMAX][KS]
  float* red = reinterpret_cast<float*>(gemv_smem + GEMV_LDS_X_BYTES);  // [4 waves][4 g][MMAX][16]
  __shared__ int last_flag;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int rb = blockIdx.x % a.rowblocks;
  const int split = blockIdx.x / a.rowblocks;
  const int T0 = split * a.tps;
  const int T1 = min(a.wordtiles, T0 + a.tps);
  const int ntile = T1 - T0;
  const int tpw = (ntile + 3) >> 2;
  const int wt0 = T0 + wave * tpw;
  const int wt1 = min(T1, wt0 + tpw);
  const int KS = ntile * F::KT;             // k range staged for this workgroup
  const int ng = a.K / a.group;
  const int n = rb * 16 + r;
  const int nn = min(n, a.N - 1);

  // 1. issue every code load of this wave first
  const u4* pk = reinterpret_cast<const u4*>(a.packed);
  u4 code[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int T = wt0 + i;
    code[i] = u4{0u, 0u, 0u, 0u};
    if (T < wt1) code[i] = pk[((int64_t)rb * a.wordtiles + T) * 64 + lane];
  }
  // 2. scales / zero points: one group per 32 codes of a lane
  f16 sv[TPW][2], zv[TPW][2];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int T = wt0 + i;
#pragma unroll
    for (int p = 0; p < F::LS / 32; ++p) {
      sv[i][p] = (f16)0.0f;
      zv[i][p] = (f16)8.0f;
      if (T < wt1) {
        const int grp = min((T * F::KT + g * F::LS + p * 32) / a.group, ng - 1);
        sv[i][p] = a.scales[(int64_t)nn * ng + grp];
        if constexpr (F::HAS_Z) zv[i][p] = a.zeros[(int64_t)nn * ng + grp];
      }
    }
  }
  // 3. stage x[0..MMAX)[T0*KT .. T1*KT) in LDS (zeros beyond M and K)
  {
    const int chunks_per_row = KS >> 3;
    const int total = MMAX * chunks_per_row;
    for (int c = tid; c < total; c += GEMV_THREADS) {
      const int m = c / chunks_per_row, kk = (c - m * chunks_per_row) << 3;
      const int k = T0 * F::KT + kk;
      u4 v = u4{0u, 0u, 0u, 0u};
      if (m < a.M && k < a.K) v = *reinterpret_cast<const u4*>(a.x + (int64_t)m * a.ldx + k);
      *reinterpret_cast<u4*>(xs + m * KS + kk) = v;
    }
  }
  __syncthreads();

  // 4. dot products: exact (q - z) pairs against fp16 x pairs, fp32 per group
  float acc[MMAX];
#pragma unroll
  for (int m = 0; m < MMAX; ++m) acc[m] = 0.0f;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int T = wt0 + i;
    if (T < wt1) {
      const int kbase = (T - T0) * F::KT + g * F::LS;  // offset inside the staged slice
#pragma unroll
      for (int p = 0; p < F::LS / 32; ++p) {            // 32 codes = one group part
        float part[MMAX];
#pragma unroll
        for (int m = 0; m < MMAX; ++m) part[m] = 0.0f;
        h2 q[16];
        if constexpr (FMT == INT2_ASYM) {
          const ZC2 zc = make_zc2(zv[i][p]);
          qmz_int2_half(code[i][2 * p], 0, zc, q);
          qmz_int2_half(code[i][2 * p], 1, zc, q + 4);
          qmz_int2_half(code[i][2 * p + 1], 0, zc, q + 8);
          qmz_int2_half(code[i][2 * p + 1], 1, zc, q + 12);
        } else {
          const ZC4 zc = make_zc4(zv[i][p]);
          qmz_int4(code[i][0], zc, q);
          qmz_int4(code[i][1], zc, q + 4);
          qmz_int4(code[i][2], zc, q + 8);
          qmz_int4(code[i][3], zc, q + 12);
        }
#pragma unroll
        for (int m = 0; m < MMAX; ++m) {
          const h8* xp = reinterpret_cast<const h8*>(xs + m * KS + kbase + p * 32);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const h8 xv = xp[c];
            float s = part[m];
            s = __builtin_amdgcn_fdot2(q[4 * c + 0], h2{xv[0], xv[1]}, s, false);
            s = __builtin_amdgcn_fdot2(q[4 * c + 1], h2{xv[2], xv[3]}, s, false);
            s = __builtin_amdgcn_fdot2(q[4 * c + 2], h2{xv[4], xv[5]}, s, false);
            s = __builtin_amdgcn_fdot2(q[4 * c + 3], h2{xv[6], xv[7]}, s, false);
            part[m] = s;
          }
        }
        const float sf = (float)sv[i][p];
#pragma unroll
        for (int m = 0; m < MMAX; ++m) acc[m] = fmaf(sf, part[m], acc[m]);
      }
    }
  }

  // 5. reduce over the 4 lane groups and 4 waves (fixed order)
#pragma unroll
  for (int m = 0; m < MMAX; ++m) red[((wave * 4 + g) * MMAX + m) * 16 + r] = acc[m];
  __syncthreads();
  float total = 0.0f;
  const int om = tid >> 4, orow = tid & 15;
  if (tid < MMAX * 16) {
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) total += red[((w * 4 + gg) * MMAX + om) * 16 + orow];
  }
  const int on = rb * 16 + orow;
  if (a.splits == 1) {
    if (tid < MMAX * 16 && om < a.M && on < a.N) {
      float v = total;
      if (a.resid) v += (float)a.resid[(int64_t)om * a.ldr + on];
      a.y[(int64_t)om * a.ldy + on] = (f16)v;
    }
    return;
  }
  // split-K: publish the partial, the last arrival reduces in split order
  float* part = a.ws + ((int64_t)rb * a.splits) * MMAX * 16;
  if (tid < MMAX * 16) part[split * MMAX * 16 + tid] = total;
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = atomicAdd(&a.cnt[rb], 1u);
    last_flag = (old == (uint32_t)(a.splits - 1));
  }
  __syncthreads();
  if (!last_flag) return;
  __threadfence();
  if (tid < MMAX * 16) {
    float v = 0.0f;
    for (int s = 0; s < a.splits; ++s) {
      const float ps = (s == split) ? total : __builtin_nontemporal_load(&part[s * MMAX * 16 + tid]);
      v += ps;
    }
    if (om < a.M && on < a.N) {
      if (a.resid) v += (float)a.resid[(int64_t)om * a.ldr + on];
      a.y[(int64_t)om * a.ldy + on] = (f16)v;
    }
  }
  if (tid == 0) a.cnt[rb] = 0u;
}

// ---------------------------------------------------------------------------
// prefill GEMM (M > 8): fp16 MFMA on register-dequantized weights
// ---------------------------------------------------------------------------
constexpr int A_STRIDE = 272;             // bytes per staged x row (256 + 16 pad)
constexpr int A_BUF = GEMM_TM * A_STRIDE;  // one stage: 128 rows x 128 k

struct GemmArgs {
  const f16* x; const uint32_t* packed; const f16* scales; const f16* zeros;
  const f16* resid; f16* y; float* ws; uint32_t* cnt;
  int ldx, ldr, ldy, M, N, K, group;
  int wordtiles, rowblocks, tiles_n, splits, tps, xcd_remap;
};

template <int FMT>
__global__ __launch_bounds__(GEMM_THREADS) void gemm_kernel(GemmArgs a) {
  using F = Fmt<FMT>;
  constexpr int STAGES = F::LS / 32;        // 32-k stages per word tile (1 or 2)
  __shared__ __align__(16) uint8_t smem[2 * A_BUF];
  __shared__ int last_flag;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 4, r = lane & 15;

  // workgroup -> (tile, split); with remap, one tile's splits share an XCD
  int bid = blockIdx.x;
  if (a.xcd_remap) bid = (bid & 7) * (int)(gridDim.x >> 3) + (bid >> 3);
  const int tile = bid / a.splits, split = bid - tile * a.splits;
  const int tn = tile % a.tiles_n, tm = tile / a.tiles_n;
  const int m0 = tm * GEMM_TM, n0 = tn * GEMM_TN;
  const int kt0 = split * a.tps;
  const int kt1 = min(a.wordtiles, kt0 + a.tps);
  const int nst = (kt1 - kt0) * STAGES;
  const int rbw = (n0 >> 4) + wn * 4;       // first row block of this wave
  const int ng = a.K / a.group;
  const u4* pk = reinterpret_cast<const u4*>(a.packed);

  f4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

  u4 areg[8];
  u4 bcur[4], bnext[4];
  f16 scur[4], zcur[4], snext[4], znext[4];

  auto load_a = [&](int st) {
    const int kt = kt0 + st / STAGES, j = st % STAGES;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int chunk = tid + c * GEMM_THREADS;
      const int m = chunk >> 4, seg = (chunk >> 2) & 3, q = chunk & 3;
      const int k = kt * F::KT + seg * F::LS + j * 32 + q * 8;
      const int row = m0 + m;
      u4 v = u4{0u, 0u, 0u, 0u};
      if (row < a.M && k < a.K) v = *reinterpret_cast<const u4*>(a.x + (int64_t)row * a.ldx + k);
      areg[c] = v;
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int chunk = tid + c * GEMM_THREADS;
      const int m = chunk >> 4, seg = (chunk >> 2) & 3, q = chunk & 3;
      *reinterpret_cast<u4*>(smem + buf * A_BUF + m * A_STRIDE + seg * 64 + q * 16) = areg[c];
    }
  };
  auto load_b = [&](int kt, u4* dst) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rb = rbw + i;
      dst[i] = u4{0u, 0u, 0u, 0u};
      if (rb < a.rowblocks) dst[i] = pk[((int64_t)rb * a.wordtiles + kt) * 64 + lane];
    }
  };
  auto load_sz = [&](int st, f16* s, f16* z) {
    const int kt = kt0 + st / STAGES, j = st % STAGES;
    const int grp = min((kt * F::KT + g * F::LS + j * 32) / a.group, ng - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int nn = min((rbw + i) * 16 + r, a.N - 1);
      s[i] = a.scales[(int64_t)nn * ng + grp];
      z[i] = F::HAS_Z ? a.zeros[(int64_t)nn * ng + grp] : (f16)8.0f;
    }
  };

  load_a(0);
  load_sz(0, scur, zcur);
  load_b(kt0, bcur);
  store_a(0);
  __syncthreads();

  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    const int j = st % STAGES;
    const bool has_next = st + 1 < nst;
    const bool next_new_tile = ((st + 1) % STAGES) == 0;
    if (has_next) {
      load_a(st + 1);
      load_sz(st + 1, snext, znext);
      if (next_new_tile) load_b(kt0 + (st + 1) / STAGES, bnext);
    }
    // dequant constants of this stage
    h2 s2[4];
    ZC4 zc4[4];
    ZC2 zc2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s2[i] = splat(scur[i]);
      if constexpr (FMT == INT2_ASYM) zc2[i] = make_zc2(zcur[i]);
      else zc4[i] = make_zc4(zcur[i]);
    }
    const uint8_t* abase = smem + buf * A_BUF;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      h8 af[4], bf[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int m = wm * 64 + mb * 16 + r;
        af[mb] = *reinterpret_cast<const h8*>(abase + m * A_STRIDE + g * 64 + t * 16);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h2 q[4];
        if constexpr (FMT == INT2_ASYM) {
          qmz_int2_half(bcur[i][2 * j + (t >> 1)], t & 1, zc2[i], q);
        } else {
          qmz_int4(bcur[i][t], zc4[i], q);
        }
        const h2 w0 = q[0] * s2[i], w1 = q[1] * s2[i], w2 = q[2] * s2[i], w3 = q[3] * s2[i];
        bf[i] = h8{w0[0], w0[1], w1[0], w1[1], w2[0], w2[1], w3[0], w3[1]};
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[mb][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[mb], bf[i], acc[mb][i], 0, 0, 0);
    }
    if (has_next) {
      store_a(buf ^ 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        scur[i] = snext[i];
        zcur[i] = znext[i];
        if (next_new_tile) bcur[i] = bnext[i];
      }
    }
    __syncthreads();
  }

  // epilogue: lane holds D[4*g + e][r] of each 16x16 block
  auto write_out = [&](f4 (&v)[4][4]) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col = n0 + (wn * 4 + i) * 16 + r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = m0 + wm * 64 + mb * 16 + g * 4 + e;
          if (row < a.M && col < a.N) {
            float o = v[mb][i][e];
            if (a.resid) o += (float)a.resid[(int64_t)row * a.ldr + col];
            a.y[(int64_t)row * a.ldy + col] = (f16)o;
          }
        }
      }
  };

  if (a.splits == 1) {
    write_out(acc);
    return;
  }
  f4* wsp = reinterpret_cast<f4*>(a.ws);
  const int64_t base = (int64_t)tile * a.splits;
#pragma unroll
  for (int q = 0; q < 16; ++q) wsp[((base + split) * 16 + q) * GEMM_THREADS + tid] = acc[q >> 2][q & 3];
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = atomicAdd(&a.cnt[tile], 1u);
    last_flag = (old == (uint32_t)(a.splits - 1));
  }
  __syncthreads();
  if (!last_flag) return;
  __threadfence();
  f4 sum[4][4];
#pragma unroll
  for (int q = 0; q < 16; ++q) sum[q >> 2][q & 3] = f4{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < a.splits; ++s) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      f4 v;
      if (s == split) v = acc[q >> 2][q & 3];
      else v = __builtin_nontemporal_load(&wsp[((base + s) * 16 + q) * GEMM_THREADS + tid]);
      sum[q >> 2][q & 3] += v;
    }
  }
  write_out(sum);
  if (tid == 0) a.cnt[tile] = 0u;
}

// ---------------------------------------------------------------------------
// host side: device state, workspace, launches
// ---------------------------------------------------------------------------
struct DeviceWs {
  void* ptr = nullptr;
  size_t bytes = 0;
};
static std::mutex g_ws_mutex;
static std::vector<DeviceWs> g_ws;

// Last HIP error seen by this thread inside the library (for qg_last_error).
static thread_local hipError_t g_last_hip = hipSuccess;

static int hip_status(hipError_t e) {
  if (e == hipSuccess) return QG_OK;
  g_last_hip = e;
  return QG_E_DEVICE;
}

static int current_device(int* dev) {
  int st = hip_status(hipGetDevice(dev));
  if (st != QG_OK) return st;
  int count = 0;
  st = hip_status(hipGetDeviceCount(&count));
  if (st != QG_OK) return st;
  return count > 0 ? QG_OK : QG_E_DEVICE;
}

// Clears any error an earlier, unrelated HIP call left pending, so that the
// status after a launch reports that launch only.
static void clear_pending_error() { (void)hipGetLastError(); }

// Library-owned zero-initialised workspace of at least `bytes` on `dev`.
static int library_ws(int dev, size_t bytes, void** out) {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  if ((int)g_ws.size() <= dev) g_ws.resize(dev + 1);
  DeviceWs& w = g_ws[dev];
  if (w.bytes < bytes) {
    if (w.ptr) {
      if (hip_status(hipDeviceSynchronize()) != QG_OK) return QG_E_DEVICE;
      (void)hipFree(w.ptr);
      w.ptr = nullptr;
      w.bytes = 0;
    }
    size_t want = std::max(bytes, (size_t)1 << 20);
    void* p = nullptr;
    if (hipMalloc(&p, want) != hipSuccess) {
      clear_pending_error();
      return QG_E_NOMEM;
    }
    if (hip_status(hipMemset(p, 0, want)) != QG_OK) {
      (void)hipFree(p);
      return QG_E_DEVICE;
    }
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

template <int FMT, int MMAX>
static void launch_gemv_t(const GemvArgs& a, int64_t wgs, hipStream_t s) {
  const size_t shm = GEMV_LDS_X_BYTES + 4 * 4 * MMAX * 16 * sizeof(float);
  hipLaunchKernelGGL((gemv_kernel<FMT, MMAX>), dim3((unsigned)wgs), dim3(GEMV_THREADS), shm, s, a);
}

template <int FMT>
static void launch_gemv_f(const GemvArgs& a, int mmax, int64_t wgs, hipStream_t s) {
  switch (mmax) {
    case 1: launch_gemv_t<FMT, 1>(a, wgs, s); break;
    case 2: launch_gemv_t<FMT, 2>(a, wgs, s); break;
    case 4: launch_gemv_t<FMT, 4>(a, wgs, s); break;
    default: launch_gemv_t<FMT, 8>(a, wgs, s); break;
  }
}

static int run_qgemm(const uint16_t* x, int ldx, const uint32_t* packed, const uint16_t* scales,
                     const uint16_t* zeros, const uint16_t* resid, int ldr, int M, int N, int K,
                     int group, int fmt, uint16_t* y, int ldy, void* workspace, size_t ws_bytes,
                     void* stream) {
  // ---- validation (host only) ----
  int st = check_shape(M, N, K, group, fmt);
  if (st != QG_OK) return st;
  if (M > 0 && N > 0) {
    if (!y) return QG_E_ARG;
    if (check_ld(ldy, N) != QG_OK) return QG_E_ARG;
    if (resid && check_ld(ldr, N) != QG_OK) return QG_E_ARG;
    if (resid && resid == y && ldr != ldy) return QG_E_ARG;
    if (check_align(y) != QG_OK || (resid && check_align(resid) != QG_OK)) return QG_E_ALIGN;
    if (K > 0) {
      if (!x || !packed || !scales) return QG_E_ARG;
      if ((fmt == QG_Q4_0) != (zeros == nullptr)) return QG_E_ARG;
      if (check_ld(ldx, K) != QG_OK) return QG_E_ARG;
      if (ldx % 8 != 0) return QG_E_ALIGN;
      if (check_align(x) != QG_OK || check_align(packed) != QG_OK || check_align(scales) != QG_OK ||
          (zeros && check_align(zeros) != QG_OK))
        return QG_E_ALIGN;
    }
  }
  const Plan p = make_plan(M, N, K, group, fmt);
  if (M > 0 && N > 0 && K > 0 && p.path == 0) return QG_E_UNSUPPORTED;
  if (workspace && ws_bytes < p.ws_bytes()) return QG_E_WORKSPACE;
  if (workspace && check_align(workspace) != QG_OK) return QG_E_ALIGN;
  if (M == 0 || N == 0) return QG_OK;  // no-op, no HIP call
  // ---- device work ----
  int dev = 0;
  st = current_device(&dev);
  if (st != QG_OK) return st;
  clear_pending_error();
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (K == 0) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for((int64_t)M * N, 256)), dim3(256), 0, s,
                       reinterpret_cast<f16*>(y), M, N, ldy, reinterpret_cast<const f16*>(resid), ldr);
    return launch_status();
  }
  void* ws = workspace;
  if (p.ws_bytes() > 0 && !ws) {
    st = library_ws(dev, p.ws_bytes(), &ws);
    if (st != QG_OK) return st;
  }
  uint32_t* cnt = reinterpret_cast<uint32_t*>(ws);
  float* wsf = ws ? reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + WS_COUNTER_BYTES) : nullptr;
  if (p.path == 1) {
    GemvArgs a;
    a.x = reinterpret_cast<const f16*>(x);
    a.packed = packed;
    a.scales = reinterpret_cast<const f16*>(scales);
    a.zeros = reinterpret_cast<const f16*>(zeros);
    a.resid = reinterpret_cast<const f16*>(resid);
    a.y = reinterpret_cast<f16*>(y);
    a.ws = wsf;
    a.cnt = cnt;
    a.ldx = ldx; a.ldr = ldr; a.ldy = ldy;
    a.M = M; a.N = N; a.K = K; a.group = group;
    a.wordtiles = p.wordtiles; a.rowblocks = p.rowblocks; a.splits = p.splits; a.tps = p.tps;
    switch (fmt) {
      case QG_INT4_ASYM: launch_gemv_f<INT4_ASYM>(a, p.mmax, p.workgroups, s); break;
      case QG_INT2_ASYM: launch_gemv_f<INT2_ASYM>(a, p.mmax, p.workgroups, s); break;
      default: launch_gemv_f<Q4_0>(a, p.mmax, p.workgroups, s); break;
    }
    return launch_status();
  }
  GemmArgs a;
  a.x = reinterpret_cast<const f16*>(x);
  a.packed = packed;
  a.scales = reinterpret_cast<const f16*>(scales);
  a.zeros = reinterpret_cast<const f16*>(zeros);
  a.resid = reinterpret_cast<const f16*>(resid);
  a.y = reinterpret_cast<f16*>(y);
  a.ws = wsf;
  a.cnt = cnt;
  a.ldx = ldx; a.ldr = ldr; a.ldy = ldy;
  a.M = M; a.N = N; a.K = K; a.group = group;
  a.wordtiles = p.wordtiles; a.rowblocks = p.rowblocks; a.tiles_n = p.tiles_n;
  a.splits = p.splits; a.tps = p.tps;
  a.xcd_remap = (p.workgroups % 8 == 0) ? 1 : 0;
  const dim3 grid((unsigned)p.workgroups), block(GEMM_THREADS);
  switch (fmt) {
    case QG_INT4_ASYM: hipLaunchKernelGGL(gemm_kernel<INT4_ASYM>, grid, block, 0, s, a); break;
    case QG_INT2_ASYM: hipLaunchKernelGGL(gemm_kernel<INT2_ASYM>, grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL(gemm_kernel<Q4_0>, grid, block, 0, s, a); break;
  }
  return launch_status();
}

static int check_pack(const void* a, const void* b, int N, int K, int fmt) {
  if (fmt < 0 || fmt > 2 || N < 0 || K < 0) return QG_E_ARG;
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
    if ((fmt == QG_Q4_0) != (zeros == nullptr)) return QG_E_ARG;
    if (check_align(packed) != QG_OK || check_align(w) != QG_OK) return QG_E_ALIGN;
  }
  int dev = 0;
  st = current_device(&dev);
  if (st != QG_OK) return st;
  clear_pending_error();
  if (total == 0) return QG_OK;
  const dim3 grid(grid_for(total, 256)), block(256);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const f16* sc = reinterpret_cast<const f16*>(scales);
  const f16* zp = reinterpret_cast<const f16*>(zeros);
  f16* wo = reinterpret_cast<f16*>(w);
  const int wt = (int)n_wordtiles(K, fmt);
  switch (fmt) {
    case QG_INT4_ASYM: hipLaunchKernelGGL(dequant_kernel<INT4_ASYM>, grid, block, 0, s, packed, sc, zp, wo, N, K, group, wt); break;
    case QG_INT2_ASYM: hipLaunchKernelGGL(dequant_kernel<INT2_ASYM>, grid, block, 0, s, packed, sc, zp, wo, N, K, group, wt); break;
    default: hipLaunchKernelGGL(dequant_kernel<Q4_0>, grid, block, 0, s, packed, sc, zp, wo, N, K, group, wt); break;
  }
  return launch_status();
}

int qgemm(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint16_t* zeros,
          int M, int N, int K, int group, int fmt, uint16_t* y, void* stream) {
  return run_qgemm(x, K, packed, scales, zeros, nullptr, N, M, N, K, group, fmt, y, N, nullptr, 0,
                   stream);
}

int qgemm_ex(const uint16_t* x, int ldx, const uint32_t* packed, const uint16_t* scales,
             const uint16_t* zeros, const uint16_t* residual, int ldr, int M, int N, int K, int group,
             int fmt, uint16_t* y, int ldy, void* workspace, size_t ws_bytes, void* stream) {
  return run_qgemm(x, ldx, packed, scales, zeros, residual, ldr, M, N, K, group, fmt, y, ldy,
                   workspace, ws_bytes, stream);
}

int qloop_block(uint16_t* x, const uint32_t* const* packed4, const uint16_t* const* scales4,
                const uint16_t* const* zeros4, int M, int D, int F, int group, int fmt, int L,
                uint16_t* scratch, void* const* events, void* stream) {
  if (!packed4 || !scales4 || !zeros4 || L < 0 || D <= 0 || F <= 0 || M < 0) return QG_E_ARG;
  if (M > 0 && (!x || !scratch)) return QG_E_ARG;
  if (check_align(scratch) != QG_OK || check_align(x) != QG_OK) return QG_E_ALIGN;
  const int64_t D3 = 3 * (int64_t)D;
  uint16_t* qkv = scratch;
  uint16_t* h = qkv + (int64_t)M * D3;
  uint16_t* u = h + (int64_t)M * D;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (events && events[0] && hip_status(hipEventRecord(reinterpret_cast<hipEvent_t>(events[0]), s)) != QG_OK)
    return QG_E_DEVICE;
  for (int l = 0; l < L; ++l) {
    int st = run_qgemm(x, D, packed4[0], scales4[0], zeros4[0], nullptr, 0, M, (int)D3, D, group, fmt,
                       qkv, (int)D3, nullptr, 0, stream);
    if (st == QG_OK)
      st = run_qgemm(qkv + 2 * (int64_t)D, (int)D3, packed4[1], scales4[1], zeros4[1], x, D, M, D, D,
                     group, fmt, h, D, nullptr, 0, stream);
    if (st == QG_OK)
      st = run_qgemm(h, D, packed4[2], scales4[2], zeros4[2], nullptr, 0, M, F, D, group, fmt, u, F,
                     nullptr, 0, stream);
    if (st == QG_OK)
      st = run_qgemm(u, F, packed4[3], scales4[3], zeros4[3], h, D, M, D, F, group, fmt, x, D, nullptr,
                     0, stream);
    if (st != QG_OK) return st;
    if (events && events[l + 1] &&
        hip_status(hipEventRecord(reinterpret_cast<hipEvent_t>(events[l + 1]), s)) != QG_OK)
      return QG_E_DEVICE;
  }
  return QG_OK;
}

}  // extern "C"
