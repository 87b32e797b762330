// internal.h - host-side declarations shared by the validation/planning code
// (host.cpp) and the launchers (kernels.hip).  Not part of the C ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "layout.h"

namespace qg {

// Path choice: decode GEMV for M <= GEMV_MAX_M (v_dot2 for M = 1, 16 x 16 MFMA
// blocks for 2..16 rows), MFMA GEMM above.
constexpr int GEMV_MAX_M = 16;
constexpr int GEMV_MFMA_KW = 256;        // K covered by one chunk of an MFMA GEMV wave, at most
constexpr int GEMV_MFMA_CH = 8;          // chunks one MFMA GEMV wave streams, at most
constexpr int GEMV_THREADS = 512;          // 8 waves per workgroup
constexpr int GEMV_TPW_MAX = 8;          // word tiles one wave streams per launch
constexpr int GEMV_LDS_X_BYTES = 32768;  // x slice staged per workgroup
constexpr int GEMV_HALF_TPW = 8;        // word tiles per wave of the half-row-block GEMV, at most
constexpr int GEMV_SPLIT_RB = 32;        // GEMV: split K unforced only below this many row blocks
constexpr int GEMV_SPLIT_TILES = 32;     // ... and above this many word tiles (32 KiB of codes) per row block
constexpr int64_t GEMV_SPLIT_COST = 370;  // M <= 2 plan: a split's reduce launch, in row x word-tile units
constexpr int64_t GEMV_SPLIT_COST_PER = 4;  // ... and per split (the in-order sum of the partials)
constexpr int GEMM_THREADS = 512;        // 8 waves; they split the workgroup's K range
constexpr int GEMM_TM = 64;              // workgroup tile rows (M)
constexpr int GEMM_TN = 64;              // workgroup tile columns (N)
constexpr int GEMM_SMALL_M = 32;         // M <= this: 32 x 32 tiles; M <= 2x this: 64 x 32
constexpr int GEMM_TPW = 2;              // word tiles per wave (K per workgroup <= 16 tiles)
constexpr int GEMM_TPW_Q8 = 4;           // q8_0: a tile is 64 wide, so 4 per wave (256 of K)
constexpr int GEMM_TPW_SMALL = 8;        // 32 x 32 tiles (two stages in flight): long K unsplit
constexpr int GEMM_DEPTH = 2;            // x stages in flight per wave on 32 x 32 tiles for M > 32
constexpr int GEMM_GCAP = 64;            // quantization groups per workgroup, at most
constexpr int GEMM_TARGET_WG = 256;      // one workgroup per compute unit

// word tiles one M = 1 GEMV workgroup of 16 waves streams, at most: 8 per wave
// within a 32 KiB x slice (INT2: 4 per wave), q4k 4 per wave (its fp32 terms
// and x sums keep the workgroup's LDS within 80 KiB); kernels.hip checks
// these against its own tile caps
inline constexpr int gemv_m1_tile_cap(int fmt) { return fmt == INT2_ASYM || fmt == Q4K ? 64 : 128; }

// word tiles one GEMM wave covers, at most
inline constexpr int gemm_tpw(int fmt, bool small_tile) {
  return small_tile ? GEMM_TPW_SMALL : fmt == Q8_0 ? GEMM_TPW_Q8 : GEMM_TPW;
}

struct Plan {
  int path = 0;        // 0 none (no-op / zero fill), 1 GEMV, 2 GEMM
  int mmax = 0;        // GEMV: rows of x per launch (1, 2, 4 on 8-row workgroups: v_dot2; 4, 8, 16: MFMA)
  int splits = 1;      // K splits
  int tps = 0;         // word tiles per split
  int wordtiles = 0;   // total word tiles along K
  int rowblocks = 0;   // N / 16 (rounded up)
  int rows = 16;       // GEMV: W rows per workgroup (16; 8 for the half-row-block kernel)
  int tm = 0, tn = 0;  // GEMM tile rows and columns (64 x 64; 64 x 32 or 32 x 32 for small M)
  int tiles_n = 0;     // GEMM tiles along N
  int tiles_m = 0;     // GEMM tiles along M
  int64_t workgroups = 0;
  size_t ws_partial_bytes = 0;  // fp32 split-K partials
  size_t ws_bytes() const { return splits > 1 ? ws_partial_bytes : 0; }
};

// Validation (pure host, no HIP call).  Return QG_OK or an error status.
int check_format_group(int fmt, int group);
int check_shape(int M, int N, int K, int group, int fmt);
int check_align(const void* p);
int check_ld(int ld, int minimum);
// QGEMM_CHECK=1 pointer test from the result of hipPointerGetAttributes:
// QG_OK for device memory of the current device (or managed / unified
// memory), QG_E_NOT_DEVICE otherwise.
int classify_pointer(int hip_rc, int memory_type, int ptr_device, int current_device);

// Launch plan for a validated problem.  Environment overrides (for tuning and
// tests): QGEMM_FORCE=gemm (the MFMA GEMM for any M), QGEMM_SPLITK=<n>, QGEMM_GEMV_ROWS=8|16 (M <= 4),
// QGEMM_GEMM_TILE=3232|6432|6464 (GEMM tile rows x columns).
Plan make_plan(int M, int N, int K, int group, int fmt);

// One qgemm call's arguments (device pointers, fp16 as uint16_t bits).
struct Call {
  const uint16_t* x; int ldx; const uint32_t* packed; const uint16_t* scales; const uint16_t* zeros;
  const uint16_t* resid; int ldr; int M, N, K, group, fmt; uint16_t* y; int ldy;
};

// Device-side helpers of kernels.hip, shared with the other entry points.
// validate_call: host-only checks of a call and its plan (no HIP call).
// launch_call: launches a validated call on `stream`; ws holds the split-K
// partials (plan.ws_bytes() bytes) when the plan splits K.
// call_pointers_ok: the QGEMM_CHECK=1 device-pointer test of a call.
int validate_call(const Call& c, Plan* plan);
int launch_call(const Call& c, const Plan& p, float* ws, void* stream);
int call_pointers_ok(const Call& c);
int current_device(int* dev);          // QG_OK when a HIP device is current
int hip_status(int hip_error);         // QG_OK, or QG_E_DEVICE (and records the error)
int env_int(const char* name, int dflt);   // integer environment setting (tuning, tests)
void clear_pending_error();

}  // namespace qg
