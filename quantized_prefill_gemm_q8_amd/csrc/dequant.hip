// Debug decoder: GGUF Q4_K / Q5_K / Q6_K / Q8_0 blocks to fp32 weights, one thread per
// value.  Exposed as a test hook so the GPU's reading of the block layout can be
// compared value by value with an independent decoder.  Each output is the
// correctly rounded fp32 value of the exact decoded weight:
//   Q4_K, Q5_K: fma(d*sc, q, -(dmin*m)) -- d*sc and dmin*m are exact in fp32
//         (binary16 times a 6-bit integer), so the single rounding is the fma's;
//   Q6_K: (d*sc) * (q6 - 32)      -- d*sc exact, one rounding.
#include "common.h"

namespace qg {

// Q5: Q5_K blocks (the nibbles at byte 48, the fifth bit in qh at byte 16)
template <bool Q5>
__global__ __launch_bounds__(256) void dequant_q4k_kernel(const uint8_t* __restrict__ W,
                                                          int64_t total, float* __restrict__ w) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t blkno = i >> 8;
  const int v = static_cast<int>(i & 255);
  const uint8_t* blk = W + blkno * (Q5 ? kQ5Bytes : kQ4Bytes);
  const uint4 hdr = *reinterpret_cast<const uint4*>(blk);
  const Q4Scales s = unpack_q4_scales(hdr.y, hdr.z, hdr.w);
  const int j = v >> 5;
  const float d = half_to_float(hdr.x & 0xFFFFu), dmin = half_to_float(hdr.x >> 16);
  const float sc = static_cast<float>(byte_of(j < 4 ? s.sc_lo : s.sc_hi, j & 3));
  const float m = static_cast<float>(byte_of(j < 4 ? s.m_lo : s.m_hi, j & 3));
  const uint8_t byte = blk[(Q5 ? 48 : 16) + 32 * (v >> 6) + (v & 31)];
  int q = (v & 63) < 32 ? (byte & 15) : (byte >> 4);
  if (Q5) q |= ((blk[16 + (v & 31)] >> (v >> 5)) & 1) << 4;
  w[i] = __builtin_fmaf(d * sc, static_cast<float>(q), -(dmin * m));
}

// Q8_0: d * q, exact in fp32 (an 11-bit binary16 times an 8-bit integer).
__global__ __launch_bounds__(256) void dequant_q80_kernel(const uint8_t* __restrict__ W,
                                                          int64_t total, float* __restrict__ w) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const uint8_t* blk = W + (i >> 5) * kQ8Bytes;
  w[i] = half_to_float(load_u16(blk)) * static_cast<float>(static_cast<int8_t>(blk[2 + (i & 31)]));
}

__global__ __launch_bounds__(256) void dequant_q6k_kernel(const uint8_t* __restrict__ W,
                                                          int64_t total, float* __restrict__ w) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t blkno = i >> 8;
  const int v = static_cast<int>(i & 255);
  const uint8_t* blk = W + blkno * kQ6Bytes;
  const int half = v >> 7, r = v & 127, c = r >> 5, l = r & 31;
  const uint8_t lb = blk[64 * half + 32 * (c & 1) + l];
  const int lo = c < 2 ? (lb & 15) : (lb >> 4);
  const int hi = (blk[128 + 32 * half + l] >> (2 * c)) & 3;
  const float d = half_to_float(load_u16(blk + 208));
  const float dsc = d * static_cast<float>(static_cast<int8_t>(blk[192 + (v >> 4)]));
  w[i] = dsc * static_cast<float>((lo | (hi << 4)) - 32);
}

}  // namespace qg

hipError_t qg_launch_dequant(const uint8_t* W, int fmt, int64_t N, int64_t K, float* w,
                             hipStream_t stream) {
  const int64_t total = N * K;
  const dim3 grid(static_cast<unsigned>((total + 255) / 256));
  if (fmt == QG_Q4_K)
    qg::dequant_q4k_kernel<false><<<grid, dim3(256), 0, stream>>>(W, total, w);
  else if (fmt == QG_Q5_K)
    qg::dequant_q4k_kernel<true><<<grid, dim3(256), 0, stream>>>(W, total, w);
  else if (fmt == QG_Q8_0)
    qg::dequant_q80_kernel<<<grid, dim3(256), 0, stream>>>(W, total, w);
  else
    qg::dequant_q6k_kernel<<<grid, dim3(256), 0, stream>>>(W, total, w);
  return hipGetLastError();
}
