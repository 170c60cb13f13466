// Measurement helpers: the HBM read ceiling, the matrix-unit ceiling and
// the shader clock.
//
// HBM read ceiling: a kernel that only streams a buffer in.
//
// Decode is bound by how fast HBM delivers the K/V bytes.  The nominal
// 8 TB/s of MI355X is not reachable by any read pattern, so the benchmark
// measures, on the same device and in the same run, what a plain
// sequential read achieves, and reports the decode kernels against that
// as well as against the nominal peak.  Each thread reads one 16-byte
// chunk per iteration of a grid-stride loop over 4 work-groups of 256 per
// CU, so that at any moment the whole device reads one contiguous window
// of the buffer (of several read patterns tried, from 1 to 8 loads in
// flight per thread, plain or non-temporal, 4 to 64 work-groups per CU,
// this one was the fastest); the chunks are folded into one word that is
// stored only if it equals a constant no real buffer produces in
// practice, so the loads cannot be dropped and the kernel writes (almost)
// nothing.
#include "pa_common.h"
#include "pa_error.h"
#include "pagedattn.h"
#include "pagedattn_bench.h"

namespace pa {

typedef unsigned u32x4_sr __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4_sr *__restrict__ p, size_t n16,
                                                          uint32_t *__restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  uint32_t acc = 0;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
    const u32x4_sr a = p[i];
    acc += a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

// Shader clock: one wave reads the shader-cycle counter (s_memtime) and the
// constant 100 MHz reference counter (s_memrealtime) at its start, sleeps
// in short steps until `ticks` reference ticks have passed (or max_iter
// steps, whichever comes first, so the loop ends even if a counter stood
// still), reads both again and stores the two differences and the step
// count.  Cycles over ticks times 100 MHz is the clock the CU ran at over
// that interval; run beside other kernels, it is their clock.
__global__ void __launch_bounds__(64) clock_probe_kernel(unsigned long long *__restrict__ out, long long ticks,
                                                        int max_iter) {
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  unsigned long long r1 = r0;
  int i = 0;
  for (; i < max_iter; ++i) {
    r1 = __builtin_amdgcn_s_memrealtime();
    if ((long long)(r1 - r0) >= ticks) break;
    __builtin_amdgcn_s_sleep(2);
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) {
    out[0] = c1 - c0;
    out[1] = r1 - r0;
    out[2] = (unsigned long long)i;
  }
}

// Matrix-unit ceiling: every wave runs `iters` rounds of four independent
// chains of v_mfma_f32_32x32x16_bf16 (the prefill's product) on operands
// made from its lane ids, with no memory traffic; four chains keep the
// matrix pipeline full (each product waits only on the one four back).
// The accumulators are folded into one word that is stored only if it
// equals a constant no run produces in practice, so no product can be
// dropped.  FLOPs per launch = work-groups x 4 waves x iters x 4 x 32768.
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_mp;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_mp;
__global__ void __launch_bounds__(256) mfma_peak_kernel(float *__restrict__ sink, int iters) {
  bf16x8_mp a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)((float)((threadIdx.x * 7 + e * 13) & 63) * 0.015625f - 0.5f);
    b[e] = (__bf16)((float)((threadIdx.x * 5 + e * 11 + blockIdx.x) & 63) * 0.015625f - 0.5f);
  }
  f32x16_mp c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  float acc = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc += c0[r] + c1[r] + c2[r] + c3[r];
  if (acc == 1234567.75f) sink[0] = acc;
}

}  // namespace pa

extern "C" int pa_stream_read(const void *buf, size_t bytes, void *sink, void *stream) {
  if (!buf || !sink) return pa::set_error(PA_ERR_NULL, "buf=%p sink=%p: both must be device pointers", buf, sink);
  if (bytes % 16) return pa::set_error(PA_ERR_SHAPE, "bytes %zu is not a multiple of 16", bytes);
  if (bytes == 0) return pa::clear_error();
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  const unsigned grid = (unsigned)(cus * 4);  // 4 work-groups of 4 waves per CU
  hipLaunchKernelGGL(pa::stream_read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const pa::u32x4_sr *>(buf), bytes / 16, static_cast<uint32_t *>(sink));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pa::set_error(PA_ERR_HIP, "stream_read launch: HIP error %d (%s)", (int)e, hipGetErrorString(e));
  return pa::clear_error();
}

extern "C" int pa_clock_probe(void *out, int64_t ticks, void *stream) {
  if (!out) return pa::set_error(PA_ERR_NULL, "out=%p: must be a device pointer to 3 x 8 bytes", out);
  if (ticks < 1 || ticks > PA_CLOCK_PROBE_MAX_TICKS)
    return pa::set_error(PA_ERR_SHAPE, "ticks %lld outside [1, %lld]", (long long)ticks,
                         (long long)PA_CLOCK_PROBE_MAX_TICKS);
  // a sleep step takes at least 128 shader cycles, more than one reference
  // tick at any clock below 12.8 GHz, so while the counters advance the
  // step limit is never what ends the loop
  const int max_iter = (int)(ticks * 16 + 1024);
  hipLaunchKernelGGL(pa::clock_probe_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream,
                     static_cast<unsigned long long *>(out), (long long)ticks, max_iter);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pa::set_error(PA_ERR_HIP, "clock_probe launch: HIP error %d (%s)", (int)e, hipGetErrorString(e));
  return pa::clear_error();
}

extern "C" int pa_mfma_peak(void *sink, int32_t iters, void *stream) {
  if (!sink) return pa::set_error(PA_ERR_NULL, "sink=%p: must be a device pointer to 4 writable bytes", sink);
  if (iters < 1 || iters > PA_MFMA_PEAK_MAX_ITERS)
    return pa::set_error(PA_ERR_SHAPE, "iters %d outside [1, %d]", (int)iters, (int)PA_MFMA_PEAK_MAX_ITERS);
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  const unsigned grid = (unsigned)(cus * 4);  // 4 work-groups of 4 waves per CU: 4 waves per SIMD
  hipLaunchKernelGGL(pa::mfma_peak_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                     static_cast<float *>(sink), (int)iters);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pa::set_error(PA_ERR_HIP, "mfma_peak launch: HIP error %d (%s)", (int)e, hipGetErrorString(e));
  return pa::clear_error();
}
