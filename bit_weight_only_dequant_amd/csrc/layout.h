// layout.h - index math of the packed (qpack) code layout, shared by the host
// repack, the device repack and the kernels of libqgemm.
//
// Packed order (uint32): [rb = N/16 row blocks][T = K/cpw/16 word tiles][64 lanes][4 words]
//   A word tile covers KT = 16 * cpw consecutive k of 16 rows (128 for 4-bit,
//   256 for 2-bit, 64 for 8-bit codes).  Lane l = 16*g + r holds codes of row
//   16*rb + r only; one 16-byte load per lane brings its 4 words, and one
//   wave-wide load reads 1 KiB that is contiguous in memory.
//   Inside a tile, code kt (0 <= kt < KT) belongs to lane group
//   g = (kt % 32) / 8 at position p = 8 * (kt / 32) + kt % 8 of that lane's
//   4 * cpw codes: word p / cpw, code j = p % cpw of that word.  So each
//   lane holds runs of 8 consecutive k, run s at kt = 32 s + 8 g: the four
//   lane groups of a 16-row block together cover 32 consecutive k per run --
//   exactly the B operand of one v_mfma_f32_16x16x32_f16 step (lane l
//   supplies column l % 16 and k-slots 8*(l/16) .. +7), whose A operand is
//   then 64 contiguous bytes of x per row.
// Inside a word, code j moves to slot (j & 1) * cpw/2 + (j >> 1): even codes
// fill the low 16 bits and odd codes the high 16 bits, so one mask yields
// codes (2i, 2i+1) in the two fp16 halves of a register.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define QG_HD __host__ __device__ inline
#else
#define QG_HD inline
#endif

namespace qg {

enum Format { INT4_ASYM = 0, INT2_ASYM = 1, Q4_0 = 2, Q8_0 = 3, Q4K = 4 };

QG_HD int bits_of(int fmt) { return fmt == INT2_ASYM ? 2 : fmt == Q8_0 ? 8 : 4; }
QG_HD bool valid_format(int fmt) { return fmt >= INT4_ASYM && fmt <= Q4K; }
// block formats with an implicit zero point (no zeros array)
QG_HD bool symmetric_format(int fmt) { return fmt == Q4_0 || fmt == Q8_0; }
QG_HD int cpw_of(int fmt) { return 32 / bits_of(fmt); }
QG_HD int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// 16 rows x 16 words per tile
QG_HD int64_t n_rowblocks(int64_t N) { return ceil_div(N, 16); }
QG_HD int64_t n_wordtiles(int64_t K, int fmt) { return ceil_div(K / cpw_of(fmt), 16); }
// K covered by one word tile: 16 words of cpw codes (128 for 4-bit, 256 for
// 2-bit, 64 for 8-bit)
// K covered by one scale/offset entry as the kernels see it: the group, or
// for q4k the 32-weight sub-block (its super-block of 256 holds 8)
QG_HD int meta_group(int fmt, int group) { return fmt == Q4K ? 32 : group; }
QG_HD int ktile_width(int fmt) { return 16 * cpw_of(fmt); }

// slot of code j inside a packed word, and its inverse
QG_HD int code_slot(int j, int cpw) { return (j & 1) * (cpw >> 1) + (j >> 1); }
QG_HD int slot_code(int slot, int cpw) { return 2 * (slot % (cpw >> 1)) + slot / (cpw >> 1); }

// packed word index and slot of code (n, k)
QG_HD int64_t packed_code_word(int64_t n, int64_t k, int cpw, int64_t wordtiles, int* slot) {
  const int ktw = 16 * cpw;
  const int64_t T = k / ktw;
  const int kt = (int)(k - T * ktw);
  const int g = (kt >> 3) & 3;
  const int p = 8 * (kt >> 5) + (kt & 7);
  *slot = code_slot(p % cpw, cpw);
  return ((((n >> 4) * wordtiles + T) * 64 + g * 16 + (n & 15)) * 4) + p / cpw;
}

// k inside its word tile of code j of word t of lane group g
QG_HD int packed_code_kt(int g, int t, int j, int cpw) {
  const int p = t * cpw + j;
  return 32 * (p >> 3) + 8 * g + (p & 7);
}

// packed word (row n, word tile T, lane group g, word t) gathered from the
// canonical words [N, Kw] (codes past N or K are zero)
QG_HD uint32_t gather_packed_word(const uint32_t* canon, int64_t n, int64_t N, int64_t K, int64_t T, int g,
                                  int t, int bits) {
  const int cpw = 32 / bits;
  const uint32_t mask = (1u << bits) - 1u;
  const int64_t kw_n = K / cpw;
  uint32_t out = 0;
  if (n >= N) return 0;
  for (int j = 0; j < cpw; ++j) {
    const int64_t k = T * 16 * cpw + packed_code_kt(g, t, j, cpw);
    if (k >= K) continue;
    const uint32_t c = (canon[n * kw_n + k / cpw] >> (bits * (int)(k % cpw))) & mask;
    out |= c << (bits * code_slot(j, cpw));
  }
  return out;
}

// canonical word (n, kw) gathered from the packed words
QG_HD uint32_t gather_canon_word(const uint32_t* packed, int64_t n, int64_t kw, int64_t wordtiles, int bits) {
  const int cpw = 32 / bits;
  const uint32_t mask = (1u << bits) - 1u;
  uint32_t out = 0;
  for (int j = 0; j < cpw; ++j) {
    int slot = 0;
    const int64_t w = packed_code_word(n, kw * cpw + j, cpw, wordtiles, &slot);
    out |= ((packed[w] >> (bits * slot)) & mask) << (bits * j);
  }
  return out;
}

}  // namespace qg
