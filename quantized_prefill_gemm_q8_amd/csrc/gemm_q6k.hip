// Tiled prefill GEMM for Q6_K weights on the int8 matrix cores (gfx950).
//
// Same scheme as the Q4_K kernel (fused decode in registers, int8 MFMA, fp32
// scale epilogue with the magic-constant accumulator and the DPP-broadcast
// activation scale), with Q6_K's 16-value sub-blocks: one
// v_mfma_i32_32x32x16_i8 per sub-block, its int32 partial scaled by the
// sub-block's d*sc, and the activation scale dx of the 32-value block holding
// it.  Codes are fed to the matrix core as the signed bytes q6 - 32, so there
// is no min term.
//
// Per y[m][n]: sum over 16-value sub-blocks s of dx[m][s/2] * d*sc[n][s] * I16.
// d*sc has at most 19 significant bits (binary16 d times an int8), so
// c = -12582912*d*sc is exact and fma(f, d*sc, c) = fl(I16 * d*sc).
#include "common.h"
#include "mfma_epilogue.h"

namespace qg {

constexpr int kQ6WM = 2, kQ6WN = 2;

__global__ __launch_bounds__(256) void gemm_q6k_kernel(const uint8_t* __restrict__ W,
                                                       const int8_t* __restrict__ qx,
                                                       const float* __restrict__ dx, int64_t M,
                                                       int64_t N, int64_t K, float* __restrict__ y) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * 32 * kQ6WM + 32 * (wave / kQ6WN);
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 32 * kQ6WN + 32 * (wave % kQ6WN);
  const int64_t n = n0 + l32, n_ld = n < N ? n : N - 1;
  const int64_t m_a = m0 + l32 < M ? m0 + l32 : M - 1;
  const int64_t nsb = K / 256, nb = K / 32;
  const int8_t* arow = qx + m_a * K + 8 * h;
  // rows beyond M read the workspace's padding rows (finite or not, they only
  // reach discarded outputs)
  const float* dxrow = dx + (m0 + dpp_scale_row(lane)) * nb;

  v16i magic;
#pragma unroll
  for (int r = 0; r < 16; r++) magic[r] = kMagicBits;
  float acc[16];
#pragma unroll
  for (int r = 0; r < 16; r++) acc[r] = 0.0f;

  for (int64_t sb = 0; sb < nsb; sb++) {
    const uint8_t* blk = W + (n_ld * nsb + sb) * kQ6Bytes;
    const float d = half_to_float(load_u16(blk + 208));
#pragma unroll 2
    for (int s = 0; s < 16; s++) {
      const long a = *reinterpret_cast<const long*>(arow + 256 * sb + 16 * s);
      const v16i D = __builtin_amdgcn_mfma_i32_32x32x16_i8(a, q6_codes(blk, s, h), magic, 0, 0, 0);
      const float dsc = d * static_cast<float>(static_cast<int8_t>(blk[192 + s]));
      epilogue_scale(acc, D, dsc, -kMagic * dsc, dxrow[8 * sb + (s >> 1)]);
    }
  }
  if (n < N) {
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int64_t m = m0 + acc_row(r, h);
      if (m < M) y[m * N + n] = acc[r];
    }
  }
}

}  // namespace qg

const char* qg_gemm_q6k_kernel_name(int64_t, int64_t, int64_t) { return "gemm_q6k_kernel"; }

hipError_t qg_launch_gemm_q6k(const uint8_t* W, const QgWorkspace& ws, int64_t M, int64_t N,
                              int64_t K, float* y, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((N + 32 * qg::kQ6WN - 1) / (32 * qg::kQ6WN)),
                  static_cast<unsigned>((M + 32 * qg::kQ6WM - 1) / (32 * qg::kQ6WM)));
  qg::gemm_q6k_kernel<<<grid, dim3(256), 0, stream>>>(W, ws.q, ws.dx, M, N, K, y);
  return hipGetLastError();
}
