// Per-block int32 partials, for bit-exact comparison with an independent
// decoder: the same weight-fragment decoders and matrix instructions as the
// production kernels, with the int32 result of every block stored instead of
// being scaled.  One wave per 32x32 tile, four waves per workgroup.  Meant for
// small shapes (the output has M*N*K/32 or M*N*K/16 entries).
#include "common.h"
#include "mfma_epilogue.h"

namespace qg {

constexpr int kProbeWM = 2, kProbeWN = 2;

// Q5: Q5_K blocks (nibbles at byte 48, the fifth bit from qh)
template <bool Q5>
__global__ __launch_bounds__(256) void partials_q4k_kernel(const uint8_t* __restrict__ W,
                                                           const int8_t* __restrict__ qx, int64_t M,
                                                           int64_t N, int64_t K,
                                                           int32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * 32 * kProbeWM + 32 * (wave / kProbeWN);
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 32 * kProbeWN + 32 * (wave % kProbeWN);
  const int64_t n = n0 + l32, n_ld = n < N ? n : N - 1;
  const int64_t m_a = m0 + l32 < M ? m0 + l32 : M - 1;
  const int64_t nsb = K / 256, nb = K / 32;
  const int8_t* arow = qx + m_a * K + 16 * h;
  for (int64_t sb = 0; sb < nsb; sb++) {
    const uint8_t* blk = W + (n_ld * nsb + sb) * (Q5 ? kQ5Bytes : kQ4Bytes);
    const uint4 qh = Q5 ? *reinterpret_cast<const uint4*>(blk + 16 + 16 * h) : uint4{};
    for (int c = 0; c < 4; c++) {
      const uint4 raw = *reinterpret_cast<const uint4*>(blk + (Q5 ? 48 : 16) + 32 * c + 16 * h);
      for (int e = 0; e < 2; e++) {
        const int64_t b = 8 * sb + 2 * c + e;
        const v4i a = *reinterpret_cast<const v4i*>(arow + 32 * b);
        v4i bq = q4_codes(raw, e);
        if (Q5) bq |= q5_high(qh, 2 * c + e);
        const v16i I = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bq, v16i{}, 0, 0, 0);
        if (n < N) {
#pragma unroll
          for (int r = 0; r < 16; r++) {
            const int64_t m = m0 + acc_row(r, h);
            if (m < M) out[(m * N + n) * nb + b] = I[r];
          }
        }
      }
    }
  }
}

// Q8_0: the codes of each 32-value block as they are (the tiled kernel's reader)
__global__ __launch_bounds__(256) void partials_q80_kernel(const uint8_t* __restrict__ W,
                                                           const int8_t* __restrict__ qx, int64_t M,
                                                           int64_t N, int64_t K,
                                                           int32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * 32 * kProbeWM + 32 * (wave / kProbeWN);
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 32 * kProbeWN + 32 * (wave % kProbeWN);
  const int64_t n = n0 + l32, n_ld = n < N ? n : N - 1;
  const int64_t m_a = m0 + l32 < M ? m0 + l32 : M - 1;
  const int64_t nsb = K / 256, nb = K / 32;
  const int8_t* arow = qx + m_a * K + 16 * h;
  for (int64_t sb = 0; sb < nsb; sb++) {
    const uint8_t* slice = W + (n_ld * nsb + sb) * 8 * kQ8Bytes;
    for (int jb = 0; jb < 8; jb++) {
      const int64_t b = 8 * sb + jb;
      const v4i a = *reinterpret_cast<const v4i*>(arow + 32 * b);
      const v16i I = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, q8_codes(slice, jb, h), v16i{}, 0, 0, 0);
      if (n < N) {
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int64_t m = m0 + acc_row(r, h);
          if (m < M) out[(m * N + n) * nb + b] = I[r];
        }
      }
    }
  }
}

__global__ __launch_bounds__(256) void partials_q6k_kernel(const uint8_t* __restrict__ W,
                                                           const int8_t* __restrict__ qx, int64_t M,
                                                           int64_t N, int64_t K,
                                                           int32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * 32 * kProbeWM + 32 * (wave / kProbeWN);
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 32 * kProbeWN + 32 * (wave % kProbeWN);
  const int64_t n = n0 + l32, n_ld = n < N ? n : N - 1;
  const int64_t m_a = m0 + l32 < M ? m0 + l32 : M - 1;
  const int64_t nsb = K / 256, n16 = K / 16;
  const int8_t* arow = qx + m_a * K + 8 * h;
  for (int64_t sb = 0; sb < nsb; sb++) {
    const uint8_t* blk = W + (n_ld * nsb + sb) * kQ6Bytes;
    for (int s = 0; s < 16; s++) {
      const long a = *reinterpret_cast<const long*>(arow + 256 * sb + 16 * s);
      const v16i I = __builtin_amdgcn_mfma_i32_32x32x16_i8(a, q6_codes(blk, s, h), v16i{}, 0, 0, 0);
      const int64_t b16 = 16 * sb + s;
      if (n < N) {
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int64_t m = m0 + acc_row(r, h);
          if (m < M) out[(m * N + n) * n16 + b16] = I[r];
        }
      }
    }
  }
}

}  // namespace qg

hipError_t qg_launch_block_partials(const uint8_t* W, int fmt, const int8_t* qx, int64_t M,
                                    int64_t N, int64_t K, int32_t* out, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((N + 32 * qg::kProbeWN - 1) / (32 * qg::kProbeWN)),
                  static_cast<unsigned>((M + 32 * qg::kProbeWM - 1) / (32 * qg::kProbeWM)));
  if (fmt == QG_Q4_K)
    qg::partials_q4k_kernel<false><<<grid, dim3(256), 0, stream>>>(W, qx, M, N, K, out);
  else if (fmt == QG_Q5_K)
    qg::partials_q4k_kernel<true><<<grid, dim3(256), 0, stream>>>(W, qx, M, N, K, out);
  else if (fmt == QG_Q8_0)
    qg::partials_q80_kernel<<<grid, dim3(256), 0, stream>>>(W, qx, M, N, K, out);
  else
    qg::partials_q6k_kernel<<<grid, dim3(256), 0, stream>>>(W, qx, M, N, K, out);
  return hipGetLastError();
}
