// stream_read.hip -- the read ceiling the decode kernels are measured against: a plain
// streaming read of a device buffer with the loads the decode kernels use (16 bytes per
// lane, non-temporal, each instruction one contiguous KiB), four waves per CU, each wave
// keeping 16 loads in flight over its own contiguous share ("Gemma 4 12B (unified
// multimodal)" record, "required kernel class": decode attention is bound by streaming the
// cache, so the rate of a bare stream is its practical ceiling).
#include "ga_device.h"
#include "ga_internal.h"

namespace ga {
namespace {

constexpr int kReadWaves = 4;
constexpr int kReadInFlight = 16;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Wave w reads KiB rows [w * per, min((w + 1) * per, rows)); a row past the end re-reads
// the wave's last row (never past the buffer), so every load is unconditional.  The XOR of
// everything read goes to sink[w * 64 + lane] so that no load is dead.
__global__ void __launch_bounds__(kReadWaves * 64)
    stream_read_kernel(const u32x4* __restrict__ src, long long rows, long long per,
                       u32x4* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const long long w = (long long)blockIdx.x * kReadWaves + (threadIdx.x >> 6);
  const long long r0 = w * per;
  const long long r1 = r0 + per < rows ? r0 + per : rows;
  u32x4 acc = {0u, 0u, 0u, 0u};
  if (r0 < r1) {
    auto row = [&](long long r) { return src + (r < r1 ? r : r1 - 1) * 64 + lane; };
    u32x4 buf[kReadInFlight];
#pragma unroll
    for (int j = 0; j < kReadInFlight; ++j) buf[j] = __builtin_nontemporal_load(row(r0 + j));
    for (long long r = r0 + kReadInFlight; r < r1 + kReadInFlight; r += kReadInFlight) {
#pragma unroll
      for (int j = 0; j < kReadInFlight; ++j) {
        acc ^= buf[j];
        buf[j] = __builtin_nontemporal_load(row(r + j));
        __builtin_amdgcn_sched_barrier(0);  // consume, then refill: 16 loads always in flight
      }
    }
#pragma unroll
    for (int j = 0; j < kReadInFlight; ++j) acc ^= buf[j];  // (re-reads of the last row)
  }
  sink[w * 64 + lane] = acc;
}

}  // namespace

hipError_t stream_read_launch(const void* src, size_t bytes, void* sink, int blocks,
                              hipStream_t stream) {
  const long long rows = (long long)(bytes / 1024);
  const long long waves = (long long)blocks * kReadWaves;
  const long long per = (rows + waves - 1) / waves;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kReadWaves * 64), 0, stream,
                     reinterpret_cast<const u32x4*>(src), rows, per,
                     reinterpret_cast<u32x4*>(sink));
  return hipGetLastError();
}

}  // namespace ga
