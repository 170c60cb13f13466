// HBM read ceiling: a kernel that only streams a buffer in.
//
// Decode is bound by how fast HBM delivers the K/V bytes.  The nominal
// 8 TB/s of MI355X is not reachable by any read pattern, so the benchmark
// measures, on the same device and in the same run, what a plain
// sequential read achieves, and reports the decode kernels against that
// as well as against the nominal peak.  Each thread reads 16-byte chunks in
// a grid-stride loop, four loads in flight, non-temporal (the data is used
// once), and folds them into one word that is stored only if it equals a
// constant no real buffer produces in practice, so the loads cannot be
// dropped and the kernel writes (almost) nothing.
#include "pa_common.h"
#include "pa_error.h"
#include "pagedattn.h"
#include "pagedattn_bench.h"

namespace pa {

typedef unsigned u32x4_sr __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4_sr *__restrict__ p, size_t n16,
                                                          uint32_t *__restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4_sr a = __builtin_nontemporal_load(p + i);
    const u32x4_sr b = __builtin_nontemporal_load(p + i + stride);
    const u32x4_sr c = __builtin_nontemporal_load(p + i + 2 * stride);
    const u32x4_sr d = __builtin_nontemporal_load(p + i + 3 * stride);
    acc ^= (a.x ^ a.y ^ a.z ^ a.w) + (b.x ^ b.y ^ b.z ^ b.w) + (c.x ^ c.y ^ c.z ^ c.w) + (d.x ^ d.y ^ d.z ^ d.w);
  }
  for (; i < n16; i += stride) {
    const u32x4_sr a = __builtin_nontemporal_load(p + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace pa

extern "C" int pa_stream_read(const void *buf, size_t bytes, void *sink, void *stream) {
  if (!buf || !sink) return pa::set_error(PA_ERR_NULL, "buf=%p sink=%p: both must be device pointers", buf, sink);
  if (bytes % 16) return pa::set_error(PA_ERR_SHAPE, "bytes %zu is not a multiple of 16", bytes);
  if (bytes == 0) return pa::clear_error();
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess && prop.multiProcessorCount > 0)
      cus = prop.multiProcessorCount;
  }
  const unsigned grid = (unsigned)(cus * 8);  // 8 work-groups of 4 waves per CU
  hipLaunchKernelGGL(pa::stream_read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const pa::u32x4_sr *>(buf), bytes / 16, static_cast<uint32_t *>(sink));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pa::set_error(PA_ERR_HIP, "stream_read launch: HIP error %d (%s)", (int)e, hipGetErrorString(e));
  return pa::clear_error();
}
