// layout.h - index math of the packed (qpack) code layout, shared by the host
// repack, the device repack and the kernels of libqgemm.
//
// Packed order (uint32): [rb = N/16 row blocks][T = K/cpw/16 word tiles][64 lanes][4 words]
//   lane l = 16*g + r holds the canonical words 4g .. 4g+3 of word tile T of
//   row 16*rb + r.  One 16-byte load per lane therefore brings 4*cpw
//   consecutive codes of one row, and one wave-wide load reads 1 KiB that is
//   contiguous in memory.  In the MFMA 16x16x32 fp16 operand layout, lane
//   l supplies column (l % 16) and the eight k-slots 8*(l/16) .. +7, so the
//   same lane mapping feeds the matrix cores with no shuffles.
// Inside a word, code j of the canonical word moves to slot
//   (j & 1) * cpw/2 + (j >> 1):
//   even codes fill the low 16 bits and odd codes the high 16 bits, so one
//   mask yields codes (2i, 2i+1) in the two fp16 halves of a register.
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

// packed word index of canonical word (n, kw)
QG_HD int64_t packed_index(int64_t n, int64_t kw, int64_t wordtiles) {
  const int64_t rb = n >> 4, r = n & 15, T = kw >> 4, wi = kw & 15;
  const int64_t g = wi >> 2, t = wi & 3;
  return ((rb * wordtiles + T) * 64 + (g * 16 + r)) * 4 + t;
}

// slot of code j inside a packed word
QG_HD int code_slot(int j, int cpw) { return (j & 1) * (cpw >> 1) + (j >> 1); }

QG_HD uint32_t perm_word(uint32_t w, int bits) {
  const int cpw = 32 / bits;
  const uint32_t mask = (1u << bits) - 1u;
  uint32_t out = 0;
  for (int j = 0; j < cpw; ++j) {
    const uint32_t c = (w >> (bits * j)) & mask;
    out |= c << (bits * code_slot(j, cpw));
  }
  return out;
}

QG_HD uint32_t unperm_word(uint32_t p, int bits) {
  const int cpw = 32 / bits;
  const uint32_t mask = (1u << bits) - 1u;
  uint32_t out = 0;
  for (int j = 0; j < cpw; ++j) {
    const uint32_t c = (p >> (bits * code_slot(j, cpw))) & mask;
    out |= c << (bits * j);
  }
  return out;
}

}  // namespace qg
