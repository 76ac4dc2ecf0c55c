// Measurement aids: the two ceilings a kernel's roofline fraction is also
// quoted against, measured on the machine at hand.
//
//  mfma_probe_kernel  back-to-back independent bf16 MFMAs (16x16x32, eight
//                     accumulators per wave, eight waves per SIMD): the
//                     dense bf16 matrix rate the chip sustains.
//  copy_probe_kernel  a streaming device copy, 16 bytes per lane and step
//                     with non-temporal loads and stores, the whole copy in
//                     flight at once: the HBM rate a plain read-once /
//                     write-once stream sustains.
#include "../../include/gdn.h"

#include <hip/hip_runtime.h>

#include "gdn_device.h"

namespace gdn {
namespace {

constexpr int kProbeAcc = 8;

__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  // operands that depend on the lane, so nothing folds at compile time
  const float x = 1.0f + 1e-3f * (float)lane;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(x * (float)(i + 1));
    b[i] = (__bf16)(x - 0.01f * (float)i);
  }
  f32x4 acc[kProbeAcc];
#pragma unroll
  for (int j = 0; j < kProbeAcc; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kProbeAcc; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kProbeAcc; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// One 16-byte piece per lane and step, 8 steps per lane, all loads issued
// before the first store; a grid of n16 / 2048 workgroups puts the whole copy
// in flight at once (no grid-stride loop whose iterations wait on each other).
constexpr int kCopyPieces = 8;
__global__ __launch_bounds__(256) void copy_probe_kernel(const gdn_u4* src, gdn_u4* dst, size_t n16) {
  const size_t base = (size_t)blockIdx.x * 256 * kCopyPieces + threadIdx.x;
  gdn_u4 v[kCopyPieces];
#pragma unroll
  for (int j = 0; j < kCopyPieces; ++j)
    if (base + (size_t)j * 256 < n16) v[j] = __builtin_nontemporal_load(src + base + (size_t)j * 256);
#pragma unroll
  for (int j = 0; j < kCopyPieces; ++j)
    if (base + (size_t)j * 256 < n16) __builtin_nontemporal_store(v[j], dst + base + (size_t)j * 256);
}

}  // namespace
}  // namespace gdn

extern "C" {

int64_t gdn_probe_mfma_flops(int32_t iters, int32_t blocks) {
  return (int64_t)blocks * 4 * iters * gdn::kProbeAcc * 16 * 16 * 32 * 2;
}

gdn_status gdn_probe_mfma(int32_t iters, int32_t blocks, float* out, void* stream) {
  if (iters < 1 || blocks < 1 || !out) return GDN_ERR_INVALID_ARG;
  hipLaunchKernelGGL(gdn::mfma_probe_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), iters, out);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

gdn_status gdn_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst || bytes % 16 || (reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16)
    return GDN_ERR_INVALID_ARG;
  const char* s = static_cast<const char*>(src);
  char* d = static_cast<char*>(dst);
  if (s < d + bytes && d < s + bytes) return GDN_ERR_INVALID_ARG;
  if (bytes == 0) return GDN_OK;
  const size_t n16 = bytes / 16, per = (size_t)256 * gdn::kCopyPieces;
  const size_t grid = (n16 + per - 1) / per;
  if (grid > 0x7fffffff) return GDN_ERR_INVALID_ARG;
  hipLaunchKernelGGL(gdn::copy_probe_kernel, dim3((unsigned)grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const gdn::gdn_u4*>(src), static_cast<gdn::gdn_u4*>(dst), n16);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // extern "C"
