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

// Any mix of one to three read streams and one or two write streams (each
// destination gets the XOR of the sources): the backward kernels' mixes.
// Same pieces and loads in flight per buffer as above.
struct ProbeBufs {
  const unsigned char* src[3];
  unsigned char* dst[2];
};

template <int NS, int ND>
__global__ __launch_bounds__(kProbeThreads) void stream_mix_kernel(ProbeBufs p, uint32_t bytes) {
  __amdgpu_buffer_rsrc_t rs[NS], rd[ND];
#pragma unroll
  for (int i = 0; i < NS; ++i) rs[i] = make_rsrc(p.src[i], bytes);
#pragma unroll
  for (int j = 0; j < ND; ++j) rd[j] = make_rsrc(p.dst[j], bytes);
  const uint32_t begin = blockIdx.x * kProbeBlockBytes;
  const uint32_t end = begin + kProbeBlockBytes < bytes ? begin + kProbeBlockBytes : bytes;
  for (uint32_t o = begin + threadIdx.x * 16u; o < end; o += kProbeThreads * 16u * kProbeInFlight) {
    u32x4 v[kProbeInFlight][NS];
#pragma unroll
    for (int k = 0; k < kProbeInFlight; ++k) {
      const uint32_t off = o + (uint32_t)k * kProbeThreads * 16u;
#pragma unroll
      for (int i = 0; i < NS; ++i) v[k][i] = load16_nt(rs[i], off < end ? off : kOob);
    }
#pragma unroll
    for (int k = 0; k < kProbeInFlight; ++k) {
      const uint32_t off = o + (uint32_t)k * kProbeThreads * 16u;
      u32x4 x = v[k][0];
#pragma unroll
      for (int i = 1; i < NS; ++i) x ^= v[k][i];
#pragma unroll
      for (int j = 0; j < ND; ++j) store16_nt(rd[j], off < end ? off : kOob, x);
    }
  }
}

template <int NS, int ND>
int launch_mix(const ProbeBufs& p, uint32_t bytes, hipStream_t s) {
  const unsigned blocks = (bytes + kProbeBlockBytes - 1) / kProbeBlockBytes;
  hipLaunchKernelGGL((stream_mix_kernel<NS, ND>), dim3(blocks), dim3(kProbeThreads), 0, s, p, bytes);
  return hipGetLastError() == hipSuccess ? GLA_OK : GLA_ERR_LAUNCH;
}

}  // namespace
}  // namespace gla

extern "C" int gla_stream_probe_mix(const void* const* srcs, int nsrc, void* const* dsts, int ndst,
                                    size_t bytes, void* stream) {
  if (!srcs || !dsts) return GLA_ERR_NULL;
  if (nsrc < 1 || nsrc > 3 || ndst < 1 || ndst > 2) return GLA_ERR_DIM;
  gla::ProbeBufs p{};
  for (int i = 0; i < nsrc; ++i) {
    if (!srcs[i]) return GLA_ERR_NULL;
    p.src[i] = static_cast<const unsigned char*>(srcs[i]);
  }
  for (int j = 0; j < ndst; ++j) {
    if (!dsts[j]) return GLA_ERR_NULL;
    p.dst[j] = static_cast<unsigned char*>(dsts[j]);
  }
  for (int i = 0; i < nsrc; ++i)
    if ((uintptr_t)p.src[i] & 15u) return GLA_ERR_ALIGN;
  for (int j = 0; j < ndst; ++j)
    if ((uintptr_t)p.dst[j] & 15u) return GLA_ERR_ALIGN;
  if (bytes == 0 || bytes % 16 != 0 || bytes >= (size_t)1 << 31) return GLA_ERR_DIM;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint32_t n = (uint32_t)bytes;
  switch (nsrc * 4 + ndst) {
    case 1 * 4 + 1: return gla::launch_mix<1, 1>(p, n, s);
    case 1 * 4 + 2: return gla::launch_mix<1, 2>(p, n, s);
    case 2 * 4 + 1: return gla::launch_mix<2, 1>(p, n, s);
    case 2 * 4 + 2: return gla::launch_mix<2, 2>(p, n, s);
    case 3 * 4 + 1: return gla::launch_mix<3, 1>(p, n, s);
    default: return gla::launch_mix<3, 2>(p, n, s);
  }
}

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
