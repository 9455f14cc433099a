// Benchmark probes (not part of the GEMM path): the shader clock under
// matrix-core load, and the time a plain read of a weight matrix's bytes takes.
//
// Shader-clock probe.
//
// The int8 GEMM's throughput is quoted against a peak taken at the chip's
// top clock, while sustained matrix-core load runs the shader clock lower.
// This kernel loads every SIMD the way the GEMM does -- independent int8
// 32x32x32 MFMA chains, four waves per SIMD -- and times a fixed stretch of
// them in two clocks at once: the shader-clock counter (s_memtime) and the
// constant 100 MHz counter (s_memrealtime).  Their ratio is the shader clock
// under that load.
#include "common.h"

namespace qg {

__global__ __launch_bounds__(256) void sclk_probe_kernel(uint64_t* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  v4i a = {lane, 3 * lane, lane ^ 5, 7};
  v4i b = {5 * lane, 11, lane, lane + 1};
  v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; it++) {
    asm volatile("" : "+v"(a), "+v"(b));  // keep the chains from being folded
    c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
  }
  int s = 0;
#pragma unroll
  for (int r = 0; r < 16; r++) s += c0[r] ^ c1[r] ^ c2[r] ^ c3[r];
  // drain the chains before the second reading
  asm volatile("" : "+v"(s));
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    out[0] = t1 - t0;
    out[1] = r1 - r0;
    out[2] = static_cast<uint64_t>(static_cast<uint32_t>(s));
  }
}

// Read probe: every byte of [src, src + 16*n16) read once in 16-byte loads,
// grid-stride (thread t reads chunks t, t + T, t + 2T, ...), nothing written.
// The floor a bandwidth-bound kernel reading the same bytes can reach from
// one launch (ramp-up and tail included).
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ src, int64_t n16) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  uint32_t acc = 0;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  asm volatile("" ::"v"(acc));  // the loads stay: their value is used
}

}  // namespace qg

// grid: eight workgroups of four waves (32 waves) per CU, the fastest of 4-32
// waves per CU and 1-4 loads in flight per lane for 8.6 MB to 511 MB (cold)
hipError_t qg_launch_read_probe(const void* src, int64_t bytes, hipStream_t stream) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (bytes == 0) return hipSuccess;
  qg::read_probe_kernel<<<dim3(static_cast<unsigned>(cus) * 8u), dim3(256), 0, stream>>>(
      static_cast<const uint4*>(src), bytes / 16);
  return hipGetLastError();
}

// grid: four waves per SIMD on every CU of the device
hipError_t qg_launch_sclk_probe(uint64_t* out, int iters, hipStream_t stream) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  qg::sclk_probe_kernel<<<dim3(static_cast<unsigned>(cus) * 4u), dim3(256), 0, stream>>>(out, iters);
  return hipGetLastError();
}
