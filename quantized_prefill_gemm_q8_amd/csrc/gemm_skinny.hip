// Skinny path for M <= 8 activation rows (decode-sized batches and the LM head
// on the last token only -- aprender issue #5305, sub-ticket #4313 "MMQ int8
// prefill matmul + LM head on the last token only").  Every weight byte is read
// once, so the kernel is bound by HBM bandwidth (the decode-GEMV yardstick of
// issue #5305's merged ticket #5221, "decode GEMV at 223-504 GB/s vs llama.cpp
// MMVQ 776-894").  Same arithmetic as the tiled kernel: int8 codes times int8
// activation codes summed per sub-block in int32 (v_dot4_i32_i8), scales and
// mins applied in fp32.
//
// One wavefront per weight row n; lane t handles the 32-value blocks t, t+64, ...
// of that row and the M activation rows; the per-lane fp32 partial sums are
// reduced across the wavefront at the end.
#include "common.h"

namespace qg {

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot4(static_cast<int>(a), static_cast<int>(b), c, false);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <int MR>
__global__ __launch_bounds__(256) void skinny_q4k_kernel(const uint8_t* __restrict__ W,
                                                         const int8_t* __restrict__ qx,
                                                         const float* __restrict__ dx,
                                                         const float* __restrict__ dS,
                                                         int64_t N, int64_t K,
                                                         float* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int64_t n = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (n >= N) return;  // whole wavefronts only
  const int64_t nsb = K / 256, nb = K / 32;
  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; m++) acc[m] = 0.0f;

  for (int64_t b = lane; b < nb; b += 64) {
    const int64_t sb = b >> 3;
    const int j = static_cast<int>(b & 7), c = j >> 1;
    const uint8_t* blk = W + (n * nsb + sb) * kQ4Bytes;
    const uint4 hdr = *reinterpret_cast<const uint4*>(blk);
    const Q4Scales s = unpack_q4_scales(hdr.y, hdr.z, hdr.w);
    const float d = half_to_float(hdr.x & 0xFFFFu), dmin = half_to_float(hdr.x >> 16);
    const float dsc = d * static_cast<float>(byte_of(j < 4 ? s.sc_lo : s.sc_hi, j & 3));
    const float dmn = dmin * static_cast<float>(byte_of(j < 4 ? s.m_lo : s.m_hi, j & 3));
    const uint4 r0 = *reinterpret_cast<const uint4*>(blk + 16 + 32 * c);
    const uint4 r1 = *reinterpret_cast<const uint4*>(blk + 32 + 32 * c);
    const int sh = 4 * (j & 1);
    const uint32_t w[8] = {(r0.x >> sh) & 0x0F0F0F0Fu, (r0.y >> sh) & 0x0F0F0F0Fu,
                           (r0.z >> sh) & 0x0F0F0F0Fu, (r0.w >> sh) & 0x0F0F0F0Fu,
                           (r1.x >> sh) & 0x0F0F0F0Fu, (r1.y >> sh) & 0x0F0F0F0Fu,
                           (r1.z >> sh) & 0x0F0F0F0Fu, (r1.w >> sh) & 0x0F0F0F0Fu};
#pragma unroll
    for (int m = 0; m < MR; m++) {
      const uint4* xa = reinterpret_cast<const uint4*>(qx + m * K + 32 * b);
      const uint4 a0 = xa[0], a1 = xa[1];
      int I = dot4(w[0], a0.x, 0);
      I = dot4(w[1], a0.y, I); I = dot4(w[2], a0.z, I); I = dot4(w[3], a0.w, I);
      I = dot4(w[4], a1.x, I); I = dot4(w[5], a1.y, I); I = dot4(w[6], a1.z, I);
      I = dot4(w[7], a1.w, I);
      const float dxm = dx[m * nb + b], ds = dS[m * nb + b];
      acc[m] = __builtin_fmaf(dsc * static_cast<float>(I), dxm, acc[m]);
      acc[m] = __builtin_fmaf(-dmn, ds, acc[m]);
    }
  }
#pragma unroll
  for (int m = 0; m < MR; m++) {
    const float v = wave_sum(acc[m]);
    if (lane == 0) y[m * N + n] = v;
  }
}

template <int MR>
__global__ __launch_bounds__(256) void skinny_q6k_kernel(const uint8_t* __restrict__ W,
                                                         const int8_t* __restrict__ qx,
                                                         const float* __restrict__ dx,
                                                         int64_t N, int64_t K,
                                                         float* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int64_t n = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const int64_t nsb = K / 256, nb = K / 32;
  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; m++) acc[m] = 0.0f;

  for (int64_t b = lane; b < nb; b += 64) {
    const int64_t sb = b >> 3;
    const int jj = static_cast<int>(b & 7);  // 32-value slot in the block: values 32jj..32jj+31
    const int half = jj >> 2, c = jj & 3;
    const uint8_t* blk = W + (n * nsb + sb) * kQ6Bytes;
    const uint8_t* pl = blk + 64 * half + 32 * (c & 1);
    const uint8_t* ph = blk + 128 + 32 * half;
    const int ls = 4 * (c >> 1), hs = 2 * c;
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const uint32_t lo = (load_u32_a2(pl + 4 * i) >> ls) & 0x0F0F0F0Fu;
      const uint32_t hi = ((load_u32_a2(ph + 4 * i) >> hs) & 0x03030303u) << 4;
      w[i] = q6_to_signed(lo | hi);
    }
    const float d = half_to_float(load_u16(blk + 208));
    const float sa = d * static_cast<float>(static_cast<int8_t>(blk[192 + 2 * jj]));
    const float sbv = d * static_cast<float>(static_cast<int8_t>(blk[193 + 2 * jj]));
#pragma unroll
    for (int m = 0; m < MR; m++) {
      const uint4* xa = reinterpret_cast<const uint4*>(qx + m * K + 32 * b);
      const uint4 a0 = xa[0], a1 = xa[1];
      int Ia = dot4(w[0], a0.x, 0);
      Ia = dot4(w[1], a0.y, Ia); Ia = dot4(w[2], a0.z, Ia); Ia = dot4(w[3], a0.w, Ia);
      int Ib = dot4(w[4], a1.x, 0);
      Ib = dot4(w[5], a1.y, Ib); Ib = dot4(w[6], a1.z, Ib); Ib = dot4(w[7], a1.w, Ib);
      const float t = __builtin_fmaf(sa, static_cast<float>(Ia), sbv * static_cast<float>(Ib));
      acc[m] = __builtin_fmaf(t, dx[m * nb + b], acc[m]);
    }
  }
#pragma unroll
  for (int m = 0; m < MR; m++) {
    const float v = wave_sum(acc[m]);
    if (lane == 0) y[m * N + n] = v;
  }
}

template <int MR>
static void launch_skinny(const uint8_t* W, int fmt, const QgWorkspace& ws, int64_t N,
                          int64_t K, float* y, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((N + 3) / 4));
  if (fmt == QG_Q4_K)
    skinny_q4k_kernel<MR><<<grid, dim3(256), 0, stream>>>(W, ws.q, ws.dx, ws.dS, N, K, y);
  else
    skinny_q6k_kernel<MR><<<grid, dim3(256), 0, stream>>>(W, ws.q, ws.dx, N, K, y);
}

}  // namespace qg

const char* qg_gemm_skinny_kernel_name(int fmt, int64_t M) {
  static const char* const q4[8] = {"skinny_q4k_kernel<1>", "skinny_q4k_kernel<2>", "skinny_q4k_kernel<3>",
                                    "skinny_q4k_kernel<4>", "skinny_q4k_kernel<5>", "skinny_q4k_kernel<6>",
                                    "skinny_q4k_kernel<7>", "skinny_q4k_kernel<8>"};
  static const char* const q6[8] = {"skinny_q6k_kernel<1>", "skinny_q6k_kernel<2>", "skinny_q6k_kernel<3>",
                                    "skinny_q6k_kernel<4>", "skinny_q6k_kernel<5>", "skinny_q6k_kernel<6>",
                                    "skinny_q6k_kernel<7>", "skinny_q6k_kernel<8>"};
  if (M < 1 || M > 8) return "?";
  return fmt == QG_Q4_K ? q4[M - 1] : q6[M - 1];
}

hipError_t qg_launch_gemm_skinny(const uint8_t* W, int fmt, const QgWorkspace& ws, int64_t M,
                                 int64_t N, int64_t K, float* y, hipStream_t stream) {
  switch (M) {
    case 1: qg::launch_skinny<1>(W, fmt, ws, N, K, y, stream); break;
    case 2: qg::launch_skinny<2>(W, fmt, ws, N, K, y, stream); break;
    case 3: qg::launch_skinny<3>(W, fmt, ws, N, K, y, stream); break;
    case 4: qg::launch_skinny<4>(W, fmt, ws, N, K, y, stream); break;
    case 5: qg::launch_skinny<5>(W, fmt, ws, N, K, y, stream); break;
    case 6: qg::launch_skinny<6>(W, fmt, ws, N, K, y, stream); break;
    case 7: qg::launch_skinny<7>(W, fmt, ws, N, K, y, stream); break;
    case 8: qg::launch_skinny<8>(W, fmt, ws, N, K, y, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
