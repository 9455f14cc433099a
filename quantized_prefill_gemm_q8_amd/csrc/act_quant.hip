// Activation quantiser: every row of x is cut into blocks of 32 consecutive
// values; each block becomes 32 int8 codes, one fp32 scale and the int32 sum of
// its codes -- the per-32 q8_1-style activation block of the quantised-activation
// kernels ranked as technique 5 on aprender issue #4220 ("CRUX parity spike:
// apr serve vs ollama ...", table "Techniques ollama/llama.cpp use that apr
// lacks").  The pages give no formula; this library takes the plainest
// symmetric one:
//   amax = max |x|;  d = amax / 127 (IEEE fp32 division);  id = 1 / d;
//   q = clamp(rint(x * id), -127, 127) with ties to even, and q = 0 where x = 0;
//   S = sum q;  an all-zero block has d = 0, S = 0.
// Each step is a single correctly rounded fp32 operation, so the result is
// bit-identical to any IEEE implementation of the same steps.
//
// Layout: four lanes per block, eight values per lane (one 16-byte bf16 load or
// two 16-byte fp32 loads); amax and S are combined across the four lanes with
// cross-lane shuffles.  HBM-bound: 2 (bf16) or 4 (fp32) bytes in per value,
// 1 byte + 8 bytes per 32 values out.
#include "common.h"

namespace qg {

template <int XDT>
__global__ __launch_bounds__(256) void act_quant_kernel(const void* __restrict__ x, int64_t M,
                                                        int64_t K, int8_t* __restrict__ q,
                                                        float* __restrict__ d, int64_t d_sb,
                                                        int64_t d_sm, int32_t* __restrict__ S_int,
                                                        float* __restrict__ dS) {
  const int64_t per_row = K / 8;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= M * per_row) return;  // whole groups of four lanes leave together
  const int64_t row = idx / per_row;
  const int64_t c8 = idx - row * per_row;
  const int64_t b = c8 >> 2;

  float v[8];
  if (XDT == QG_BF16) {
    const uint4 raw = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + row * K + 8 * c8);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[2 * i] = __builtin_bit_cast(float, w[i] << 16);
      v[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + row * K + 8 * c8);
    const float4 a = p[0], c = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
  }

  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));

  float dv = 0.0f, id = 0.0f;
  if (amax != 0.0f) {
    dv = amax / 127.0f;  // correctly rounded IEEE division
    id = 1.0f / dv;      // correctly rounded IEEE division (may be +inf for tiny blocks)
  }
  uint32_t packed[2] = {0u, 0u};
  int s = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    int qi = 0;
    if (v[i] != 0.0f) {
      float r = rintf(v[i] * id);
      r = r > 127.0f ? 127.0f : r;
      r = r < -127.0f ? -127.0f : r;
      qi = static_cast<int>(r);
    }
    s += qi;
    packed[i >> 2] |= (static_cast<uint32_t>(qi) & 0xFFu) << (8 * (i & 3));
  }
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);

  *reinterpret_cast<uint2*>(q + row * K + 8 * c8) = make_uint2(packed[0], packed[1]);
  if ((c8 & 3) == 0) {
    const int64_t o = b * d_sb + row * d_sm;
    d[o] = dv;
    if (S_int) S_int[o] = s;
    if (dS) dS[o] = dv * static_cast<float>(s);
  }
}

}  // namespace qg

hipError_t qg_launch_act_quant(const void* x, int x_dtype, int64_t M, int64_t K, int8_t* q,
                               float* d, int64_t d_sb, int64_t d_sm, int32_t* S_int, float* dS,
                               hipStream_t stream) {
  const int64_t threads = M * (K / 8);
  const int64_t blocks = (threads + 255) / 256;
  if (x_dtype == QG_BF16)
    qg::act_quant_kernel<QG_BF16><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(
        x, M, K, q, d, d_sb, d_sm, S_int, dS);
  else
    qg::act_quant_kernel<QG_F32><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(
        x, M, K, q, d, d_sb, d_sm, S_int, dS);
  return hipGetLastError();
}
