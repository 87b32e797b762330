// measure.hip - measurement helpers of libqgemm: the ceilings a qGEMM kernel
// is read against, taken on the device it runs on (the hot-op
// microbenchmarks of the TinyLoop README, "Validation", and the phase timings
// of its "Quick CLI Tour", "Benchmark").  None of these is on the qGEMM path.
//   qg_stream_read  - a plain streaming read of a byte range: the bandwidth
//                     one launch reaches over a given number of bytes;
//   qg_empty_launch - an empty kernel: the launch floor of a grid;
//   qg_mfma_probe   - back-to-back independent v_mfma_f32_16x16x32_f16 on
//                     every SIMD: the sustained dense fp16 matrix rate;
//   qg_device_info  - compute units and clocks as the runtime reports them;
//   qg_clock_stamp  - the device's constant-rate clock, stored by one wave in
//                     stream order: two stamps bracket the launches between
//                     them on the device (a graph's own launch latency, which
//                     events around the graph would include, stays outside);
//   qg_clock_rate   - that clock's rate.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qgemm.h"
#include "internal.h"

namespace qg {
namespace {

typedef uint32_t mu4 __attribute__((ext_vector_type(4)));
typedef _Float16 mh8 __attribute__((ext_vector_type(8)));
typedef float mf4 __attribute__((ext_vector_type(4)));

constexpr int STREAM_THREADS = 256;
constexpr int STREAM_UNROLL = 4;   // 16-byte loads in flight per lane per round

// Each lane reads 16-byte words at a grid stride, STREAM_UNROLL of them per
// round, and folds them into one word; the fold is written only if it equals
// a value no input produces in practice (the store keeps the loads alive and
// almost never happens; the sink holds one word per workgroup).
__global__ __launch_bounds__(STREAM_THREADS) void stream_read_kernel(const mu4* __restrict__ src, int64_t n16,
                                                                     const uint8_t* __restrict__ tail, int ntail,
                                                                     uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * STREAM_THREADS;
  int64_t i = (int64_t)blockIdx.x * STREAM_THREADS + threadIdx.x;
  mu4 acc = mu4{0u, 0u, 0u, 0u};
  for (; i + (STREAM_UNROLL - 1) * stride < n16; i += STREAM_UNROLL * stride) {
    mu4 v[STREAM_UNROLL];
#pragma unroll
    for (int u = 0; u < STREAM_UNROLL; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < STREAM_UNROLL; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= src[i];
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail) acc.x ^= tail[threadIdx.x];
  const uint32_t f = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (f == 0x9e3779b9u) sink[blockIdx.x] = f;
}

__global__ void empty_kernel() {}

// The stamp is read as the wave starts; stream order puts it after every
// earlier launch has completed and before any later one starts.
__global__ void clock_stamp_kernel(uint64_t* __restrict__ out) {
  const uint64_t t = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) out[0] = t;
}

// Every wave keeps 8 independent accumulators so that each MFMA waits for no
// earlier result; the sum of one element per accumulator is written per lane.
__global__ __launch_bounds__(256) void mfma_probe_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  mh8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)((float)lane * 0.001f + (float)i);
    b[i] = (_Float16)(0.5f - (float)i * 0.01f);
  }
  mf4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = mf4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j & 7] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[j & 7], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += acc[i][0];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace
}  // namespace qg

using namespace qg;

extern "C" int qg_stream_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, void* stream) {
  if ((bytes > 0 && !src) || !sink || workgroups <= 0) return QG_E_ARG;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0) return QG_E_ALIGN;
  if (bytes == 0) return QG_OK;
  const int64_t n16 = (int64_t)(bytes / 16);
  const int ntail = (int)(bytes % 16);
  const uint8_t* tail = reinterpret_cast<const uint8_t*>(src) + n16 * 16;
  hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(STREAM_THREADS), 0,
                     reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const mu4*>(src), n16, tail, ntail,
                     sink);
  return hip_status(hipGetLastError());
}

extern "C" int qg_empty_launch(int workgroups, int threads, void* stream) {
  if (workgroups <= 0 || threads <= 0 || threads > 1024) return QG_E_ARG;
  hipLaunchKernelGGL(empty_kernel, dim3(workgroups), dim3(threads), 0, reinterpret_cast<hipStream_t>(stream));
  return hip_status(hipGetLastError());
}

extern "C" int qg_clock_stamp(uint64_t* out, void* stream) {
  if (!out) return QG_E_ARG;
  if (reinterpret_cast<uintptr_t>(out) % 8 != 0) return QG_E_ALIGN;
  hipLaunchKernelGGL(clock_stamp_kernel, dim3(1), dim3(64), 0, reinterpret_cast<hipStream_t>(stream), out);
  return hip_status(hipGetLastError());
}

extern "C" int qg_clock_rate(int device, int* khz) {
  if (!khz) return QG_E_ARG;
  int v = 0;
  const int st = hip_status(hipDeviceGetAttribute(&v, hipDeviceAttributeWallClockRate, device));
  if (st != QG_OK) {
    clear_pending_error();
    return st;
  }
  *khz = v;
  return QG_OK;
}

extern "C" int qg_mfma_probe(float* out, int workgroups, int iters, void* stream) {
  if (!out || workgroups <= 0 || iters < 0) return QG_E_ARG;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(workgroups), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), out,
                     iters);
  return hip_status(hipGetLastError());
}

extern "C" int qg_device_info(int device, int* compute_units, int* clock_khz, int* memory_clock_khz,
                              int* memory_bus_bits) {
  if (!compute_units || !clock_khz || !memory_clock_khz || !memory_bus_bits) return QG_E_ARG;
  int v[4] = {0, 0, 0, 0};
  const hipDeviceAttribute_t at[4] = {hipDeviceAttributeMultiprocessorCount, hipDeviceAttributeClockRate,
                                      hipDeviceAttributeMemoryClockRate, hipDeviceAttributeMemoryBusWidth};
  for (int i = 0; i < 4; ++i) {
    const int st = hip_status(hipDeviceGetAttribute(&v[i], at[i], device));
    if (st != QG_OK) {
      clear_pending_error();
      return st;
    }
  }
  *compute_units = v[0];
  *clock_khz = v[1];
  *memory_clock_khz = v[2];
  *memory_bus_bits = v[3];
  return QG_OK;
}
