// gla_probe.hip -- plain streaming kernels that measure the GPU's memory
// bandwidth with the access path the mixer's kernels use (16-byte buffer
// loads and stores, non-temporal hints), so that achieved bandwidth can be
// reported next to a ceiling measured on the same GPU.  Not part of the
// mixer's computation.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gla.h"
#include "gla_device.h"

namespace gla {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeInFlight = 4;  // 16-byte loads per thread and stream in flight
constexpr uint32_t kProbeBlockBytes = kProbeThreads * 16 * kProbeInFlight;  // 16 KB

// Each block streams one contiguous 16 KB piece of each buffer: all of its
// loads at once, then (MODE 1) all of its stores, and exits.  Of the piece
// sizes, loads in flight and persistent grids measured on MI355X, this
// shape streamed fastest in both mixes.  MODE 0 reads src0 and src1; MODE 1
// also writes dst = src0 ^ src1.
template <int MODE>
__global__ __launch_bounds__(kProbeThreads) void stream_probe_kernel(const unsigned char* src0,
                                                                     const unsigned char* src1,
                                                                     unsigned char* dst,
                                                                     uint32_t bytes) {
  const __amdgpu_buffer_rsrc_t r0 = make_rsrc(src0, bytes);
  const __amdgpu_buffer_rsrc_t r1 = make_rsrc(src1, bytes);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(dst, bytes);
  const uint32_t begin = blockIdx.x * kProbeBlockBytes;
  const uint32_t end = begin + kProbeBlockBytes < bytes ? begin + kProbeBlockBytes : bytes;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (uint32_t o = begin + threadIdx.x * 16u; o < end; o += kProbeThreads * 16u * kProbeInFlight) {
    u32x4 a[kProbeInFlight], b[kProbeInFlight];
#pragma unroll
    for (int i = 0; i < kProbeInFlight; ++i) {
      const uint32_t off = o + (uint32_t)i * kProbeThreads * 16u;
      a[i] = load16_nt(r0, off < end ? off : kOob);
      b[i] = load16_nt(r1, off < end ? off : kOob);
    }
#pragma unroll
    for (int i = 0; i < kProbeInFlight; ++i) {
      if (MODE == 1) {
        const uint32_t off = o + (uint32_t)i * kProbeThreads * 16u;
        store16_nt(rd, off < end ? off : kOob, a[i] ^ b[i]);
      } else {
        acc ^= a[i] ^ b[i];
      }
    }
  }
  // keeps the reads alive; the pattern never occurs in practice, and dst
  // is the caller's buffer either way
  if (MODE == 0 && (acc[0] & acc[1] & acc[2] & acc[3]) == 0xFFFFFFFFu)
    store16_nt(rd, threadIdx.x * 16u, acc);
}

}  // namespace
}  // namespace gla

extern "C" int gla_stream_probe(const void* src0, const void* src1, void* dst, size_t bytes,
                                int mode, void* stream) {
  if (!src0 || !src1 || !dst) return GLA_ERR_NULL;
  if (((uintptr_t)src0 | (uintptr_t)src1 | (uintptr_t)dst) & 15u) return GLA_ERR_ALIGN;
  if (bytes == 0 || bytes % 16 != 0 || bytes >= (size_t)1 << 31 || (mode != 0 && mode != 1))
    return GLA_ERR_DIM;
  const unsigned blocks = (unsigned)((bytes + gla::kProbeBlockBytes - 1) / gla::kProbeBlockBytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const auto* a = static_cast<const unsigned char*>(src0);
  const auto* b = static_cast<const unsigned char*>(src1);
  auto* d = static_cast<unsigned char*>(dst);
  if (mode == 0)
    hipLaunchKernelGGL(gla::stream_probe_kernel<0>, dim3(blocks), dim3(gla::kProbeThreads), 0, s, a,
                       b, d, (uint32_t)bytes);
  else
    hipLaunchKernelGGL(gla::stream_probe_kernel<1>, dim3(blocks), dim3(gla::kProbeThreads), 0, s, a,
                       b, d, (uint32_t)bytes);
  return hipGetLastError() == hipSuccess ? GLA_OK : GLA_ERR_LAUNCH;
}
