// SwiGLU of a stacked gate+up projection output, as a kernel of its own:
// h[m][f] = bfloat16(silu(y[m][f]) * y[m][F + f]) from y [M][2F] fp32 -- the
// separate swiglu launch of a layer's per-token launch list in aprender issue
// #4220 ("CRUX parity spike: apr serve vs ollama", table of techniques
// llama.cpp uses, technique 2).  The library fuses this step into the gate+up
// GEMM's epilogue for Q4_K, Q5_K and Q8_0 problems on the LDS-tiled kernels;
// this kernel serves the problems that are not fused (decode-sized batches on
// the skinny kernel, Q4_K and Q5_K problems on the small-grid kernel, Q6_K
// weights) and the unfused comparison.  HBM-bound: 8 bytes in, 2 bytes out per
// element.
#include "common.h"

namespace qg {

// Four consecutive columns per lane (F % 4 == 0: 16-byte loads, 8-byte
// stores), else one.
template <bool VEC>
__global__ __launch_bounds__(256) void swiglu_kernel(const float* __restrict__ y, int64_t M, int64_t F,
                                                     uint16_t* __restrict__ h) {
  const int64_t per_row = VEC ? F / 4 : F;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= M * per_row) return;
  const int64_t m = idx / per_row, c = idx - m * per_row;
  const float* yr = y + m * 2 * F;
  if (VEC) {
    const float4 g = *reinterpret_cast<const float4*>(yr + 4 * c);
    const float4 u = *reinterpret_cast<const float4*>(yr + F + 4 * c);
    const uint32_t lo = swiglu_bf16(g.x, u.x) | (static_cast<uint32_t>(swiglu_bf16(g.y, u.y)) << 16);
    const uint32_t hi = swiglu_bf16(g.z, u.z) | (static_cast<uint32_t>(swiglu_bf16(g.w, u.w)) << 16);
    *reinterpret_cast<uint2*>(h + m * F + 4 * c) = make_uint2(lo, hi);
  } else {
    h[m * F + c] = swiglu_bf16(yr[c], yr[F + c]);
  }
}

}  // namespace qg

hipError_t qg_launch_swiglu(const float* y, int64_t M, int64_t F, uint16_t* h, hipStream_t stream) {
  const bool vec = F % 4 == 0;
  const int64_t n = M * (vec ? F / 4 : F);
  const dim3 grid(static_cast<unsigned>((n + 255) / 256));
  if (vec) qg::swiglu_kernel<true><<<grid, dim3(256), 0, stream>>>(y, M, F, h);
  else qg::swiglu_kernel<false><<<grid, dim3(256), 0, stream>>>(y, M, F, h);
  return hipGetLastError();
}
