// Tiled prefill GEMM on the int8 matrix cores, Q4_K and Q6_K weights.
//
// The fused design of sparkinfer PR #464 ("fused Q4K/Q6K->int8 dequant ...",
// section "Summary": super-blocks decoded in registers, an int8 tensor-core
// GEMM, no wider dequantised scratch), carried to CDNA4 without its second
// per-row weight quantisation: the weight codes go to the matrix core as they
// are and every sub-block's own scale and min are applied to its int32 partial.
//
// Per 32-value activation block b and weight sub-block:
//   I[m][n] = sum_t qw[n][t] * qx[m][t]                  (int8 MFMA, int32)
//   Q4_K: y += dx[m][b] * (d*sc[n][b] * I - dmin*m[n][b] * S[m][b])
//   Q6_K: y += dx[m][b] * d * (sc[n][2b] * I16a + sc[n][2b+1] * I16b)
//
// Lane mapping.  Weights sit on the lane axis (column n = lane % 32 of each
// 32x32 tile) so the per-sub-block weight scale dsc = d*sc is one scalar per
// lane.  dsc has at most 19 significant bits (binary16 d times a 6- or 8-bit
// integer), so c = -12582912*dsc is exact in fp32; the MFMA accumulator starts
// at the bit pattern of 12582912.0f, making its int32 result readable as the
// float 12582912 + I, and fma(f, dsc, c) is then exactly fl(I * dsc).  The
// epilogue is two fp32 FMAs per element for the scale plus one for the min.
//
// v_mfma_i32_32x32x32_i8 (Q4_K, one 32-value sub-block per instruction) and
// v_mfma_i32_32x32x16_i8 (Q6_K, one 16-value sub-block) both take their K
// split across the two lane halves; A (activations) and B (weights) use the
// same k-to-(lane half, byte) assignment, so any consistent assignment of the
// sub-block's values to bytes gives the same dot product.
#include "common.h"

namespace qg {

constexpr int kWavesM = 2, kWavesN = 2;  // waves per workgroup
constexpr int kTileM = 32 * kWavesM, kTileN = 32 * kWavesN;

// Output row of accumulator element r held by a lane in half h of the wave.
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// ---------------------------------------------------------------- Q4_K

// 16 weight codes of sub-block j (j = 2c or 2c+1) for lane half h: bytes
// qs[32c + 16h .. +15] hold sub-block 2c in their low nibbles and 2c+1 in the
// high nibbles.
__device__ __forceinline__ void q4_fragments(const uint8_t* blk, int c, int h, v4i& lo, v4i& hi) {
  const uint4 raw = *reinterpret_cast<const uint4*>(blk + 16 + 32 * c + 16 * h);
  lo = v4i{int(raw.x & 0x0F0F0F0Fu), int(raw.y & 0x0F0F0F0Fu), int(raw.z & 0x0F0F0F0Fu),
           int(raw.w & 0x0F0F0F0Fu)};
  hi = v4i{int((raw.x >> 4) & 0x0F0F0F0Fu), int((raw.y >> 4) & 0x0F0F0F0Fu),
           int((raw.z >> 4) & 0x0F0F0F0Fu), int((raw.w >> 4) & 0x0F0F0F0Fu)};
}

template <bool DUMP>
__global__ __launch_bounds__(256) void gemm_q4k_kernel(const uint8_t* __restrict__ W,
                                                       const int8_t* __restrict__ qx,
                                                       const float* __restrict__ dxT,
                                                       const float* __restrict__ dST, int64_t Mp,
                                                       int64_t M, int64_t N, int64_t K,
                                                       float* __restrict__ y,
                                                       int32_t* __restrict__ dump) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kTileM + 32 * (wave / kWavesN);
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kTileN + 32 * (wave % kWavesN);
  const int64_t n = n0 + l32;
  const int64_t n_ld = n < N ? n : N - 1;             // clamp loads; stores are masked
  const int64_t m_a = m0 + l32 < M ? m0 + l32 : M - 1;  // A-operand row for this lane
  const int64_t nsb = K / 256;
  const int8_t* arow = qx + m_a * K + 16 * h;

  v16i magic;
#pragma unroll
  for (int r = 0; r < 16; r++) magic[r] = kMagicBits;
  float acc[16];
#pragma unroll
  for (int r = 0; r < 16; r++) acc[r] = 0.0f;

  for (int64_t sb = 0; sb < nsb; sb++) {
    const uint8_t* blk = W + (n_ld * nsb + sb) * kQ4Bytes;
    const uint4 hdr = *reinterpret_cast<const uint4*>(blk);
    const float d = half_to_float(hdr.x & 0xFFFFu), dmin = half_to_float(hdr.x >> 16);
    const Q4Scales s = unpack_q4_scales(hdr.y, hdr.z, hdr.w);
#pragma unroll
    for (int c = 0; c < 4; c++) {
      v4i bfrag[2];
      q4_fragments(blk, c, h, bfrag[0], bfrag[1]);
#pragma unroll
      for (int e = 0; e < 2; e++) {
        const int j = 2 * c + e;
        const int64_t b = 8 * sb + j;
        const v4i afrag = *reinterpret_cast<const v4i*>(arow + 32 * b);
        if (DUMP) {
          v16i zero = {};
          const v16i I = __builtin_amdgcn_mfma_i32_32x32x32_i8(afrag, bfrag[e], zero, 0, 0, 0);
          if (n < N) {
#pragma unroll
            for (int r = 0; r < 16; r++) {
              const int64_t m = m0 + acc_row(r, h);
              if (m < M) dump[(m * N + n) * (K / 32) + b] = I[r];
            }
          }
          continue;
        }
        const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(afrag, bfrag[e], magic, 0, 0, 0);
        const uint32_t scj = byte_of(j < 4 ? s.sc_lo : s.sc_hi, j & 3);
        const uint32_t mj = byte_of(j < 4 ? s.m_lo : s.m_hi, j & 3);
        const float dsc = d * static_cast<float>(scj);
        const float cc = -kMagic * dsc;
        const float ndmn = -(dmin * static_cast<float>(mj));
        const float* dxb = dxT + b * Mp + m0 + 4 * h;
        const float* dsb = dST + b * Mp + m0 + 4 * h;
#pragma unroll
        for (int g = 0; g < 4; g++) {
          const float4 dx4 = *reinterpret_cast<const float4*>(dxb + 8 * g);
          const float4 ds4 = *reinterpret_cast<const float4*>(dsb + 8 * g);
          const float dxv[4] = {dx4.x, dx4.y, dx4.z, dx4.w};
          const float dsv[4] = {ds4.x, ds4.y, ds4.z, ds4.w};
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int r = 4 * g + i;
            const float u = __builtin_fmaf(bits_to_float(D[r]), dsc, cc);  // == fl(I * dsc)
            acc[r] = __builtin_fmaf(u, dxv[i], acc[r]);
            acc[r] = __builtin_fmaf(ndmn, dsv[i], acc[r]);
          }
        }
      }
    }
  }
  if (DUMP) return;
  if (n < N) {
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int64_t m = m0 + acc_row(r, h);
      if (m < M) y[m * N + n] = acc[r];
    }
  }
}

// ---------------------------------------------------------------- Q6_K

// 8 weight codes (as signed q6 - 32 bytes) of 16-value sub-block s for lane
// half h: values v = 16s + 8h + i, i < 8.  With half = s/8, quarter c = (s%8)/2
// and l0 = 16*(s%2) + 8h, the low nibbles are ql[64*half + 32*(c%2) + l0 + i]
// (low nibble for c < 2, high for c >= 2) and the top two bits are bits
// (2c, 2c+1) of qh[32*half + l0 + i].
__device__ __forceinline__ long q6_fragment(const uint8_t* blk, int s, int h) {
  const int half = s >> 3, c = (s & 7) >> 1, l0 = 16 * (s & 1) + 8 * h;
  const uint8_t* pl = blk + 64 * half + 32 * (c & 1) + l0;
  const uint8_t* ph = blk + 128 + 32 * half + l0;
  uint32_t lo0 = load_u32_a2(pl), lo1 = load_u32_a2(pl + 4);
  uint32_t hi0 = load_u32_a2(ph), hi1 = load_u32_a2(ph + 4);
  const int ls = (c >> 1) * 4, hs = 2 * c;
  lo0 = (lo0 >> ls) & 0x0F0F0F0Fu;
  lo1 = (lo1 >> ls) & 0x0F0F0F0Fu;
  hi0 = ((hi0 >> hs) & 0x03030303u) << 4;
  hi1 = ((hi1 >> hs) & 0x03030303u) << 4;
  const uint32_t w0 = q6_to_signed(lo0 | hi0), w1 = q6_to_signed(lo1 | hi1);
  return static_cast<long>((static_cast<uint64_t>(w1) << 32) | w0);
}

template <bool DUMP>
__global__ __launch_bounds__(256) void gemm_q6k_kernel(const uint8_t* __restrict__ W,
                                                       const int8_t* __restrict__ qx,
                                                       const float* __restrict__ dxT, int64_t Mp,
                                                       int64_t M, int64_t N, int64_t K,
                                                       float* __restrict__ y,
                                                       int32_t* __restrict__ dump) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kTileM + 32 * (wave / kWavesN);
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kTileN + 32 * (wave % kWavesN);
  const int64_t n = n0 + l32;
  const int64_t n_ld = n < N ? n : N - 1;
  const int64_t m_a = m0 + l32 < M ? m0 + l32 : M - 1;
  const int64_t nsb = K / 256;
  const int8_t* arow = qx + m_a * K + 8 * h;

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
      const long bfrag = q6_fragment(blk, s, h);
      const long afrag = *reinterpret_cast<const long*>(arow + 256 * sb + 16 * s);
      const int64_t b16 = 16 * sb + s;
      if (DUMP) {
        v16i zero = {};
        const v16i I = __builtin_amdgcn_mfma_i32_32x32x16_i8(afrag, bfrag, zero, 0, 0, 0);
        if (n < N) {
#pragma unroll
          for (int r = 0; r < 16; r++) {
            const int64_t m = m0 + acc_row(r, h);
            if (m < M) dump[(m * N + n) * (K / 16) + b16] = I[r];
          }
        }
        continue;
      }
      const v16i D = __builtin_amdgcn_mfma_i32_32x32x16_i8(afrag, bfrag, magic, 0, 0, 0);
      const float dsc = d * static_cast<float>(static_cast<int8_t>(blk[192 + s]));
      const float cc = -kMagic * dsc;
      const float* dxb = dxT + (b16 >> 1) * Mp + m0 + 4 * h;
#pragma unroll
      for (int g = 0; g < 4; g++) {
        const float4 dx4 = *reinterpret_cast<const float4*>(dxb + 8 * g);
        const float dxv[4] = {dx4.x, dx4.y, dx4.z, dx4.w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int r = 4 * g + i;
          const float u = __builtin_fmaf(bits_to_float(D[r]), dsc, cc);
          acc[r] = __builtin_fmaf(u, dxv[i], acc[r]);
        }
      }
    }
  }
  if (DUMP) return;
  if (n < N) {
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int64_t m = m0 + acc_row(r, h);
      if (m < M) y[m * N + n] = acc[r];
    }
  }
}

}  // namespace qg

hipError_t qg_launch_gemm_tiled(const uint8_t* W, int fmt, const QgWorkspace& ws, int64_t M,
                                int64_t N, int64_t K, float* y, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((N + qg::kTileN - 1) / qg::kTileN),
                  static_cast<unsigned>((M + qg::kTileM - 1) / qg::kTileM));
  if (fmt == QG_Q4_K)
    qg::gemm_q4k_kernel<false><<<grid, dim3(256), 0, stream>>>(W, ws.q, ws.dxT, ws.dST, ws.Mp, M,
                                                               N, K, y, nullptr);
  else
    qg::gemm_q6k_kernel<false><<<grid, dim3(256), 0, stream>>>(W, ws.q, ws.dxT, ws.Mp, M, N, K,
                                                               y, nullptr);
  return hipGetLastError();
}

hipError_t qg_launch_block_partials(const uint8_t* W, int fmt, const int8_t* qx, int64_t M,
                                    int64_t N, int64_t K, int32_t* out, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((N + qg::kTileN - 1) / qg::kTileN),
                  static_cast<unsigned>((M + qg::kTileM - 1) / qg::kTileM));
  if (fmt == QG_Q4_K)
    qg::gemm_q4k_kernel<true><<<grid, dim3(256), 0, stream>>>(W, qx, nullptr, nullptr, 0, M, N,
                                                              K, nullptr, out);
  else
    qg::gemm_q6k_kernel<true><<<grid, dim3(256), 0, stream>>>(W, qx, nullptr, 0, M, N, K,
                                                              nullptr, out);
  return hipGetLastError();
}
