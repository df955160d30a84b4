// Measurement kernels of the benchmark (not part of the BitLinear path):
// declarations and contracts in include/blmeasure.h.
#include "../../include/blmeasure.h"
#include "device_util.h"

namespace {

constexpr int kThreads = 256;
constexpr int kLoads = 8;                                   // 16-byte loads per lane in flight
constexpr size_t kStepBytes = (size_t)kThreads * 16 * kLoads;  // 32 KiB per workgroup step
constexpr size_t kBlocks = 4096;                            // 16 per CU

// Workgroup b sweeps bytes [b * span, (b + 1) * span) in steps of 32 KiB: lane
// t of step s loads 16 bytes at s * 32 KiB + j * 4 KiB + 16 t, j = 0..7 (a
// wave covers 1 KiB contiguously per load).
__global__ __launch_bounds__(kThreads) void k_stream_read(const uint4* __restrict__ buf, uint64_t span,
                                                          uint64_t total, uint32_t* __restrict__ sink) {
  const uint64_t begin = (uint64_t)blockIdx.x * span;
  const uint64_t end = begin + span < total ? begin + span : total;
  uint32_t acc = 0;
  for (uint64_t base = begin; base < end; base += kStepBytes) {
    // the span and the buffer are multiples of 32 KiB: whole steps only
    const __amdgpu_buffer_rsrc_t r = bl::buffer_rsrc(reinterpret_cast<const uint8_t*>(buf) + base, (uint32_t)kStepBytes);
    uint4 v[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) v[j] = bl::buffer_load16_stream(r, (uint32_t)(j * kThreads * 16 + threadIdx.x * 16));
#pragma unroll
    for (int j = 0; j < kLoads; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  acc = (uint32_t)bl::wave_reduce<true>((int)(acc & 0x7FFFFFFFu));  // any fold that uses every word
  if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" {

size_t blmeasure_stream_read_sink_words(size_t bytes) { return bytes == 0 ? 0 : kBlocks; }

int blmeasure_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes == 0 || bytes % kStepBytes != 0 || ((uintptr_t)buf & 15) != 0) return 1;
  const uint64_t steps = bytes / kStepBytes;
  const uint64_t span = (steps + kBlocks - 1) / kBlocks * kStepBytes;
  const uint64_t blocks = (bytes + span - 1) / span;
  hipLaunchKernelGGL(k_stream_read, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream,
                     reinterpret_cast<const uint4*>(buf), span, (uint64_t)bytes, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
