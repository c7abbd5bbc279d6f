// A plain streaming device copy: the reference rate the benchmark sets beside
// every rotating kernel, measured on the same bytes read and written with no
// arithmetic.  What a copy reaches on MI355X depends on the size (how much of
// it the 256 MB memory-side cache holds) and on how it is timed, so the
// benchmark times this kernel under the same measure as the kernel it
// compares.
//
// Each wavefront owns one contiguous span of 64 lanes x kCopyUnroll x 16
// bytes: it issues every load of the span (each instruction covers 1 KB of
// consecutive bytes), then every store, both non-temporal (every byte is
// read once and written once).  Spans are addressed through a
// buffer descriptor sized to the bytes left, so the tail needs no branch:
// loads past the end return zeros and their stores are dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mrope_internal.h"

// 16-byte chunks per lane: spans of 4 KB per wavefront measured fastest on
// 302 MB with buffers the memory-side cache does not hold (94.1 us; 2 KB
// 93.9 us, 8 KB 95.7 us).  Cached loads: 99.3 us (2 KB 100.8 us, 8 KB 102.6
// us, 16 KB 106.6 us); cached loads and stores 107.6 us.
#ifndef MROPE_COPY_UNROLL
#define MROPE_COPY_UNROLL 4
#endif
#ifndef MROPE_COPY_NT_STORES
#define MROPE_COPY_NT_STORES 1
#endif
#ifndef MROPE_COPY_NT_LOADS
#define MROPE_COPY_NT_LOADS 1
#endif

namespace mrope {
namespace {

constexpr int kCopyUnroll = MROPE_COPY_UNROLL;
constexpr uint32_t kCopySpan = kWaveSize * kCopyUnroll * 16;
typedef uint32_t u32x4c_t __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kBlockThreads)
stream_copy_kernel(const char* src, char* dst, uint64_t bytes) {
  const int lane = threadIdx.x & (kWaveSize - 1);
  const uint64_t wave = (uint64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWaveSize;
  const uint64_t start = wave * kCopySpan;
  if (start >= bytes) return;
  const uint64_t left = bytes - start;
  const uint32_t n = left < kCopySpan ? (uint32_t)left : kCopySpan;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(src + start), 0, (int)n, 0x00020000);
  const __amdgpu_buffer_rsrc_t rd =
      __builtin_amdgcn_make_buffer_rsrc(dst + start, 0, (int)n, 0x00020000);
  u32x4c_t v[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u)
    v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)((u * kWaveSize + lane) * 16), 0,
                                                 MROPE_COPY_NT_LOADS ? 2 : 0);
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u)
    __builtin_amdgcn_raw_buffer_store_b128(v[u], rd, (uint32_t)((u * kWaveSize + lane) * 16), 0,
                                           MROPE_COPY_NT_STORES ? 2 : 0);
}

}  // namespace

int launch_stream_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  const uint64_t waves = ((uint64_t)bytes + kCopySpan - 1) / kCopySpan;
  const uint64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)blocks), dim3(kBlockThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const char*>(src),
                     static_cast<char*>(dst), (uint64_t)bytes);
  return (int)hipGetLastError();
}

}  // namespace mrope
