// Measurement helpers: what this GPU sustains on a plain HBM read and on back-to-back bf16
// MFMAs, read beside the published peaks when the kernels' roofline fractions are
// reported. They compute nothing of the method.
#include "common.h"

#include "../../include/ubs_bench.h"

namespace ubs {

// Plain read: block b streams bytes [b*span, (b+1)*span) of the buffer in 16-byte loads,
// four independent loads in flight per lane, folding them into an xor that is stored only
// if it equals a value it never takes (so the loads cannot be dropped and nothing is
// written).
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ buf, int64_t n16, int64_t span16,
                                                   uint32_t* __restrict__ sink) {
  const int64_t lo = (int64_t)blockIdx.x * span16;
  const int64_t hi = min(lo + span16, n16);
  uint32_t acc = 0;
  int64_t i = lo + threadIdx.x;
  for (; i + 3 * 256 < hi; i += 4 * 256) {
    const u32x4 a = buf[i], b = buf[i + 256], c = buf[i + 512], d = buf[i + 768];
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^ d[3];
  }
  for (; i < hi; i += 256) {
    const u32x4 a = buf[i];
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

// Back-to-back MFMAs: each wave runs `iters` rounds of four independent 32x32x16 bf16
// MFMA chains on register operands (32,768 flops each), then stores one accumulator
// element if it equals a value it never takes.
__global__ __launch_bounds__(256) void mfma_kernel(int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  u32x4 av, bv;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    av[e] = 0x3f803f80u ^ (uint32_t)(lane + e);   // bf16 pairs near 1
    bv[e] = 0x3f803f80u ^ (uint32_t)(lane * 3 + e);
  }
  const bf16x8 a = as_bf16x8(av), b = as_bf16x8(bv);
  typedef __attribute__((ext_vector_type(16))) float f32x16;
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  const float r = c0[0] + c1[1] + c2[2] + c3[3];
  if (r == -1.25f) out[0] = r;
}

}  // namespace ubs

namespace {
int device_cus(int* n) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return UBS_ERR_HIP;
  if (hipDeviceGetAttribute(n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || *n <= 0)
    return UBS_ERR_HIP;
  return UBS_OK;
}
}  // namespace

extern "C" int ubs_bench_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!buf || !sink || bytes < 16 || (uintptr_t)buf % 16 != 0) return UBS_ERR_INVALID_ARGUMENT;
  int cus = 0;
  if (int rc = device_cus(&cus)) return rc;
  const int64_t n16 = (int64_t)(bytes / 16);
  const int64_t blocks = (int64_t)cus * 8;
  const int64_t span16 = (n16 + blocks - 1) / blocks;
  hipLaunchKernelGGL(ubs::read_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const ubs::u32x4*>(buf), n16, span16, sink);
  return hipGetLastError() == hipSuccess ? UBS_OK : UBS_ERR_HIP;
}

extern "C" int64_t ubs_bench_mfma_waves(void) {
  int cus = 0;
  if (device_cus(&cus)) return 0;
  return (int64_t)cus * 8;   // two waves per SIMD
}

extern "C" int ubs_bench_mfma(int32_t iters, float* out, hipStream_t stream) {
  if (!out || iters <= 0) return UBS_ERR_INVALID_ARGUMENT;
  int cus = 0;
  if (int rc = device_cus(&cus)) return rc;
  hipLaunchKernelGGL(ubs::mfma_kernel, dim3((unsigned)(cus * 2)), dim3(256), 0, stream, (int)iters, out);
  return hipGetLastError() == hipSuccess ? UBS_OK : UBS_ERR_HIP;
}
