// host.cpp - pure host part of libqgemm: argument validation, launch planning,
// the host repack, status strings.  Nothing here calls HIP, so every function
// in this file works (and is tested) on a machine without a GPU.
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <climits>

#include "../../include/qgemm.h"
#include "internal.h"

namespace qg {

int check_format_group(int fmt, int group) {
  if (fmt == QG_Q4_0 || fmt == QG_Q8_0) return group == 32 ? QG_OK : QG_E_ARG;
  if (fmt == QG_Q4K) return group == 256 ? QG_OK : QG_E_ARG;
  if (fmt == QG_INT4_ASYM || fmt == QG_INT2_ASYM)
    return (group == 32 || group == 64 || group == 128) ? QG_OK : QG_E_ARG;
  return QG_E_ARG;
}

int check_shape(int M, int N, int K, int group, int fmt) {
  int st = check_format_group(fmt, group);
  if (st != QG_OK) return st;
  if (M < 0 || N < 0 || K < 0) return QG_E_ARG;
  if (K % group != 0) return QG_E_ARG;
  return QG_OK;
}

int check_align(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0 ? QG_OK : QG_E_ALIGN;
}

int check_ld(int ld, int minimum) { return ld >= minimum ? QG_OK : QG_E_ARG; }

// hipMemoryType values (hip_runtime_api.h): 1 host, 2 device, 3 managed,
// 10 array, 11 unified.  Device memory must belong to the current device;
// managed and unified memory is reachable from any device.
int classify_pointer(int hip_rc, int memory_type, int ptr_device, int current_device) {
  if (hip_rc != 0) return QG_E_NOT_DEVICE;          // unregistered host memory, or not a pointer HIP knows
  switch (memory_type) {
    case 2: return ptr_device == current_device ? QG_OK : QG_E_NOT_DEVICE;
    case 3:
    case 11: return QG_OK;
    default: return QG_E_NOT_DEVICE;                // host (pinned or registered), arrays
  }
}

int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  if (!v || !*v) return dflt;
  return atoi(v);
}

static bool force_is(const char* what) {
  const char* v = getenv("QGEMM_FORCE");
  return v && strcmp(v, what) == 0;
}

Plan make_plan(int M, int N, int K, int group, int fmt) {
  Plan p;
  if (M == 0 || N == 0) return p;  // no-op
  p.rowblocks = (int)n_rowblocks(N);
  p.wordtiles = (int)n_wordtiles(K, fmt);
  if (K == 0) return p;             // zero fill
  const int kt_width = ktile_width(fmt);
  const bool gemv = !force_is("gemm") && M <= GEMV_MAX_M;
  const int split_env = env_int("QGEMM_SPLITK", 0);
  if (gemv) {
    p.path = 1;
    const int nw = GEMV_THREADS / 64;
    const int tps_lds = std::max(1, GEMV_LDS_X_BYTES / (kt_width * 2));
    // per-workgroup word-tile caps: v_dot2 kernel (M = 1), MFMA GEMV (M > 1),
    // 8-row v_dot2 kernel (M <= 4)
    const int cap16 = M <= 1 ? std::min(tps_lds, gemv_m1_tile_cap(fmt))
                             : nw * std::max(1, GEMV_MFMA_KW / kt_width) * GEMV_MFMA_CH;
    const int cap8 = nw * GEMV_HALF_TPW;
    const bool can8 = M <= 4;
    // K splits for a cap.  A split costs a second (reduce) launch and the fp32
    // partials, about 2 us, more than an unsplit launch loses to idle CUs:
    // split only when the cap forces it, or when fewer than GEMV_SPLIT_RB row
    // blocks each carry more than GEMV_SPLIT_TILES word tiles (long streams on
    // few CUs).  Once the reduce is paid, split far enough to fill the chip.
    const auto splits_for = [&](int cap) {
      const int s_min = (int)ceil_div(p.wordtiles, cap);
      const bool split = s_min > 1 || (p.rowblocks < GEMV_SPLIT_RB && p.wordtiles > GEMV_SPLIT_TILES);
      const int s_par = p.rowblocks >= GEMM_TARGET_WG ? 1 : (int)ceil_div(2 * GEMM_TARGET_WG, p.rowblocks);
      const int s_fill = (int)ceil_div(p.wordtiles, nw);  // keep every wave busy
      int s = split ? std::max(s_min, std::min(s_par, s_fill)) : 1;
      if (split_env > 0) s = std::max(s_min, split_env);
      s = std::min(std::max(s, 1), p.wordtiles);
      return (int)ceil_div(p.wordtiles, ceil_div(p.wordtiles, s));   // splits of equal tile counts
    };
    int s16 = splits_for(cap16);
    int s8 = can8 ? splits_for(cap8) : 0;
    const int rows_env = env_int("QGEMM_GEMV_ROWS", 0);
    bool half = false;
    {
      // Rows per workgroup (16 or 8; M > 2: the MFMA GEMV's 16) and K splits
      // from a cost model in units of one row of W times one word tile
      // streamed by a workgroup (about 5 ns measured): rounds of workgroups
      // over the 256 CUs x rows x tiles per workgroup, plus GEMV_SPLIT_COST
      // for a split's reduce launch and fp32 partials (about 2 us) and
      // GEMV_SPLIT_COST_PER per split (the reduce sums each output's partials
      // in order: about 20 ns each).  Ties go to fewer workgroups.  M = 2 on
      // 8-row workgroups takes the v_dot2 kernel with both rows sharing each
      // dequantized pair, on 16-row workgroups the MFMA GEMV.
      int64_t best_cost = INT64_MAX, best_wg = INT64_MAX;
      for (int rows = 16; rows >= 8; rows -= 8) {
        if (rows == 8 && M > 2) continue;
        if (M <= 2 && (rows_env == 8 || rows_env == 16)) {
          if (rows != rows_env) continue;
        }
        const int cap = rows == 16 ? cap16 : cap8;
        const int per = 16 / rows;   // workgroups per row block and split
        const int s_min = (int)ceil_div(p.wordtiles, cap);
        int s_top = std::min(p.wordtiles, std::max(s_min, (int)ceil_div(4 * GEMM_TARGET_WG, (int64_t)p.rowblocks * per)));
        // the MFMA GEMV streams K in chunks with the next chunk's loads in
        // flight, so a long unsplit stream costs less than the model's linear
        // tiles (M = 8, 2048 x 8192: unsplit 7.8 against 8.2 us in two splits):
        // with 64 row blocks or more it runs unsplit whenever its cap allows
        if (M > 2 && s_min == 1 && p.rowblocks >= 64 && split_env <= 0) s_top = 1;
        for (int s = s_min; s <= s_top; ++s) {
          const int tps = (int)ceil_div(p.wordtiles, s);
          if (ceil_div(p.wordtiles, tps) != s) continue;   // splits of equal tile counts only
          if (split_env > 0) {   // the forced split count, as equal tile counts make it
            const int se = std::max(s_min, std::min(split_env, p.wordtiles));
            if (s != (int)ceil_div(p.wordtiles, ceil_div(p.wordtiles, se))) continue;
          }
          const int64_t wg = (int64_t)p.rowblocks * per * s;
          const int64_t cost = ceil_div(wg, GEMM_TARGET_WG) * rows * tps +
                               (s > 1 ? GEMV_SPLIT_COST + GEMV_SPLIT_COST_PER * s : 0);
          if (cost < best_cost || (cost == best_cost && wg < best_wg)) {
            best_cost = cost;
            best_wg = wg;
            half = rows == 8;
            (half ? s8 : s16) = s;
          }
        }
      }
    }
    // M = 3, 4 run the 8-row v_dot2 kernel (four x rows per pair) only when a
    // test forces it: its dot products grow with M, and since the MFMA GEMV
    // streams K unsplit it is never ahead (M = 4, 2048 x 8192: 6.66 against 6.67 us)
    if (M > 2 && can8 && rows_env == 8) half = true;
    p.rows = half ? 8 : 16;
    p.mmax = half ? (M <= 2 ? M : 4) : M <= 1 ? 1 : M <= 4 ? 4 : M <= 8 ? 8 : 16;
    p.splits = half ? s8 : s16;
    p.tps = (int)ceil_div(p.wordtiles, p.splits);
    p.workgroups = (int64_t)p.rowblocks * p.splits * (half ? 2 : 1);
    if (p.splits > 1) p.ws_partial_bytes = (size_t)p.rowblocks * p.splits * p.mmax * 16 * sizeof(float);
    return p;
  }
  p.path = 2;
  // tile rows follow M (32 or 64); 64-row tiles are 32 columns wide up to
  // M = 64, so a single row of tiles still spreads over the CUs without a split
  p.tm = M <= GEMM_SMALL_M ? 32 : GEMM_TM;
  p.tn = M <= 2 * GEMM_SMALL_M ? 32 : GEMM_TN;
  const int nw = GEMM_THREADS / 64;
  const int mg = meta_group(fmt, group);   // scale entries the kernel stages per 'group'
  // fewest K splits a tile shape allows: word tiles per wave, groups per workgroup
  const auto s_min_for = [&](int tm, int tn) {
    const int s_tiles = (int)ceil_div(p.wordtiles, nw * gemm_tpw(fmt, tm == 32 && tn == 32));
    const int s_groups = (int)ceil_div((int64_t)p.wordtiles * kt_width / mg, GEMM_GCAP);
    return std::max(s_tiles, s_groups);
  };
  const int64_t split_below = (GEMM_TARGET_WG * 5) / 8;   // fewer tiles than this: split K
  // Where the M-sized tiles would leave the CUs idle and so split K, but
  // 32 x 32 tiles fill them with no split, one launch of 32 x 32 tiles beats
  // a split plus its reduce launch, though every code is then dequantized in
  // more workgroups (128 x 2048 x 2048: 4.8 against 9.3 us for 64 x 64 tiles
  // split 4 ways); measured up to M = 128
  if (s_min_for(32, 32) == 1 && M <= 2 * GEMM_TM &&
      (int64_t)ceil_div(N, p.tn) * ceil_div(M, p.tm) < split_below &&
      (int64_t)ceil_div(N, 32) * ceil_div(M, 32) >= split_below) {
    p.tm = 32;
    p.tn = 32;
  }
  const int tile_env = env_int("QGEMM_GEMM_TILE", 0);   // 3232, 6432 or 6464 (tuning, tests)
  if (tile_env == 3232 || tile_env == 6432 || tile_env == 6464) {
    p.tm = tile_env / 100;
    p.tn = tile_env % 100;
  }
  const bool small_tile = p.tm == 32 && p.tn == 32;
  const int tpw = gemm_tpw(fmt, small_tile);
  const int s_min = s_min_for(p.tm, p.tn);
  p.tiles_n = (int)ceil_div(N, p.tn);
  p.tiles_m = (int)ceil_div(M, p.tm);
  const int64_t tiles = (int64_t)p.tiles_n * p.tiles_m;
  // at most gemm_tpw word tiles per wave and GEMM_GCAP groups per workgroup;
  // split K across workgroups only when the tiles leave most compute units
  // idle, since a split writes fp32 partials and costs a second (reduce) launch
  int s = tiles >= split_below ? 1 : (int)ceil_div(GEMM_TARGET_WG, tiles);
  if (split_env > 0) s = split_env;
  s = std::min(std::max(s, s_min), p.wordtiles);
  p.tps = (int)ceil_div(p.wordtiles, s);
  p.splits = (int)ceil_div(p.wordtiles, p.tps);
  if (p.tps > nw * tpw || (int64_t)p.tps * kt_width / mg > GEMM_GCAP) {  // cannot happen: s >= s_min
    p.path = 0;
    return p;
  }
  p.workgroups = tiles * p.splits;
  if (p.splits > 1) p.ws_partial_bytes = (size_t)tiles * p.splits * p.tm * p.tn * sizeof(float);
  return p;
}

}  // namespace qg

using namespace qg;

extern "C" {

int qg_version(void) { return 100; }  // 0.1.0

const char* qg_status_str(int status) {
  switch (status) {
    case QG_OK: return "QG_OK";
    case QG_E_ARG: return "QG_E_ARG: invalid size, format, group or pointer";
    case QG_E_UNSUPPORTED: return "QG_E_UNSUPPORTED: request outside the implemented kernels";
    case QG_E_ALIGN: return "QG_E_ALIGN: pointer or leading dimension misaligned";
    case QG_E_DEVICE: return "QG_E_DEVICE: no usable HIP device or a HIP call failed";
    case QG_E_NOMEM: return "QG_E_NOMEM: workspace allocation failed";
    case QG_E_WORKSPACE: return "QG_E_WORKSPACE: caller workspace too small";
    case QG_E_NOT_DEVICE: return "QG_E_NOT_DEVICE: a pointer is not device memory of the current device";
    default: return "unknown qgemm status";
  }
}

size_t qg_packed_bytes(int64_t N, int64_t K, int fmt) {
  if (!valid_format(fmt) || N < 0 || K < 0) return 0;
  if (K % cpw_of(fmt) != 0) return 0;
  return (size_t)n_rowblocks(N) * (size_t)n_wordtiles(K, fmt) * 64 * 4 * sizeof(uint32_t);
}

static int check_pack_args(const void* a, const void* b, int N, int K, int fmt) {
  if (!valid_format(fmt) || N < 0 || K < 0) return QG_E_ARG;
  if (K % cpw_of(fmt) != 0) return QG_E_ARG;
  if ((int64_t)N * K > 0 && (!a || !b)) return QG_E_ARG;
  return QG_OK;
}

int qpack_host(const uint32_t* canon, uint32_t* packed, int N, int K, int fmt) {
  int st = check_pack_args(canon, packed, N, K, fmt);
  if (st != QG_OK) return st;
  const int bits = bits_of(fmt);
  const int64_t kw_n = K / cpw_of(fmt);
  const int64_t wt = n_wordtiles(K, fmt);
  const size_t total = qg_packed_bytes(N, K, fmt) / sizeof(uint32_t);
  if (total) memset(packed, 0, total * sizeof(uint32_t));
  for (int64_t n = 0; n < N; ++n)
    for (int64_t kw = 0; kw < kw_n; ++kw)
      packed[packed_index(n, kw, wt)] = perm_word(canon[n * kw_n + kw], bits);
  return QG_OK;
}

int qunpack_host(const uint32_t* packed, uint32_t* canon, int N, int K, int fmt) {
  int st = check_pack_args(packed, canon, N, K, fmt);
  if (st != QG_OK) return st;
  const int bits = bits_of(fmt);
  const int64_t kw_n = K / cpw_of(fmt);
  const int64_t wt = n_wordtiles(K, fmt);
  for (int64_t n = 0; n < N; ++n)
    for (int64_t kw = 0; kw < kw_n; ++kw)
      canon[n * kw_n + kw] = unperm_word(packed[packed_index(n, kw, wt)], bits);
  return QG_OK;
}

int qg_classify_pointer(int hip_rc, int memory_type, int ptr_device, int current_device) {
  return classify_pointer(hip_rc, memory_type, ptr_device, current_device);
}

size_t qgemm_workspace_bytes(int M, int N, int K, int group, int fmt) {
  if (check_shape(M, N, K, group, fmt) != QG_OK) return 0;
  return make_plan(M, N, K, group, fmt).ws_bytes();
}

int qg_plan(int M, int N, int K, int group, int fmt, int out[5]) {
  int st = check_shape(M, N, K, group, fmt);
  if (st != QG_OK) return st;
  if (!out) return QG_E_ARG;
  Plan p = make_plan(M, N, K, group, fmt);
  out[0] = p.path;
  out[1] = p.splits;
  out[2] = (int)p.workgroups;
  out[3] = p.path == 2 ? p.tm : p.mmax;
  out[4] = p.path == 2 ? p.tn : p.rows;
  return QG_OK;
}

}  // extern "C"
