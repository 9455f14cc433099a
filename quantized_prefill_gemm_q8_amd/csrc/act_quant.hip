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
#include <atomic>

#include "common.h"

namespace qg {

// Split an fp32 value exactly into three bfloat16 pieces by truncation: each
// piece keeps the top 8 significant bits of what is left, so p0 + p1 + p2 == v
// for every v whose last piece is not below the fp32 normal range.
__device__ __forceinline__ void split3_bf16(float v, uint16_t& p0, uint16_t& p1, uint16_t& p2) {
  const uint32_t b0 = __builtin_bit_cast(uint32_t, v) & 0xFFFF0000u;
  const float r1 = v - __builtin_bit_cast(float, b0);  // exact
  const uint32_t b1 = __builtin_bit_cast(uint32_t, r1) & 0xFFFF0000u;
  const float r2 = r1 - __builtin_bit_cast(float, b1);  // exact
  p0 = static_cast<uint16_t>(b0 >> 16);
  p1 = static_cast<uint16_t>(b1 >> 16);
  p2 = static_cast<uint16_t>(__builtin_bit_cast(uint32_t, r2) >> 16);
}

// Values 8*c8 .. 8*c8+7 of row `row` of x (bf16 bits or fp32) as fp32: one
// 16-byte load (bf16) or two (fp32).
template <int XDT>
__device__ __forceinline__ void load8(const void* __restrict__ x, int64_t row, int64_t K, int64_t c8,
                                      float (&v)[8]) {
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
}

// The per-32 quantiser's steps for the eight values v of lane chunk c8 of a
// row (four consecutive lanes hold one 32-value block; all four must call
// this together) and the stores of its codes, scale and code sum.  WS: the
// GEMM workspace (q, dx, dxT, dS, dsp); otherwise the hook layout (q, d,
// S_int).
template <bool WS>
__device__ __forceinline__ void quantize8_store(const float (&v)[8], int64_t row, int64_t c8, int64_t K,
                                                int8_t* __restrict__ q, float* __restrict__ d,
                                                int32_t* __restrict__ S_int, float* __restrict__ dS,
                                                uint16_t* __restrict__ dsp, float* __restrict__ dxT,
                                                int64_t Mp) {
  const int64_t b = c8 >> 2;
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
    const int64_t nb = K / 32;
    if (WS) {
      const float ds = dv * static_cast<float>(s);
      d[row * nb + b] = dv;
      dxT[b * Mp + row] = dv;
      dS[row * nb + b] = ds;
      uint16_t p0, p1, p2;
      split3_bf16(ds, p0, p1, p2);
      uint16_t* o = dsp + ((row * (K / 256) + (b >> 3)) * 3) * 8 + (b & 7);
      o[0] = p0;
      o[8] = p1;
      o[16] = p2;
    } else {
      d[row * nb + b] = dv;
      S_int[row * nb + b] = s;
    }
  }
}

// WS: write the GEMM workspace (q, dx, dS, dsp); otherwise the test-hook
// layout (q [M][K], d [M][K/32], S [M][K/32] int32).
template <int XDT, bool WS>
__global__ __launch_bounds__(256) void act_quant_kernel(const void* __restrict__ x, int64_t M,
                                                        int64_t K, int8_t* __restrict__ q,
                                                        float* __restrict__ d,
                                                        int32_t* __restrict__ S_int,
                                                        float* __restrict__ dS,
                                                        uint16_t* __restrict__ dsp,
                                                        float* __restrict__ dxT, int64_t Mp,
                                                        int sleeps) {
  // planted delay (timing falsifier): the first wave of the first workgroup
  // sleeps before it starts; `sleeps` is bounded by the host
  if (sleeps > 0 && blockIdx.x == 0 && threadIdx.x < 64)
    for (int i = 0; i < sleeps; i++) __builtin_amdgcn_s_sleep(1);
  const int64_t per_row = K / 8;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= M * per_row) return;  // whole groups of four lanes leave together
  const int64_t row = idx / per_row;
  const int64_t c8 = idx - row * per_row;

  float v[8];
  load8<XDT>(x, row, K, c8, v);

  quantize8_store<WS>(v, row, c8, K, q, d, S_int, dS, dsp, dxT, Mp);
}

// RMSNorm fused into the per-32 quantiser: the norm of llama.cpp that aprender
// issue #4220 ("CRUX parity spike: apr serve vs ollama", table of techniques
// llama.cpp uses, technique 6) fuses with the multiply by its weight, here
// fused further into the activation quantiser so that the normalised row never
// leaves registers.  Per row:
//   ss = sum_k x_k^2            binary64 (every x_k^2 is exact in binary64)
//   r  = f32(1 / sqrt(ss/K + eps))   binary64 steps, rounded once to fp32
//   xn_k = f32(f32(x_k * r) * g_k)   then the per-32 quantiser on xn.
// Only the order of the binary64 sum is this kernel's own (lane partials over
// the lane's values in ascending order, a fixed butterfly across the wave,
// the four waves' sums in wave order); another order can move ss by a few
// units in its last place, which changes r only when r lies that close to a
// rounding boundary of fp32.
// One workgroup of 256 lanes per row; lane t holds the eight-value chunks
// t, t + 256, ... (NCH of them, so K <= 2048*NCH) in registers between the
// sum and the quantiser.
template <int XDT, bool WS, int NCH>
__global__ __launch_bounds__(256) void rmsnorm_quant_kernel(const void* __restrict__ x,
                                                            const float* __restrict__ g, float eps,
                                                            int64_t K, int8_t* __restrict__ q,
                                                            float* __restrict__ d,
                                                            int32_t* __restrict__ S_int,
                                                            float* __restrict__ dS,
                                                            uint16_t* __restrict__ dsp,
                                                            float* __restrict__ dxT, int64_t Mp) {
  __shared__ double s_part[4];
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t nch = K / 8;  // a multiple of 32: groups of four lanes are in or out together
  float v[NCH][8];
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < NCH; i++) {
    const int64_t c8 = t + 256 * i;
    if (c8 < nch) {
      load8<XDT>(x, row, K, c8, v[i]);
#pragma unroll
      for (int e = 0; e < 8; e++) ss = __builtin_fma(static_cast<double>(v[i][e]), static_cast<double>(v[i][e]), ss);
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
  if (lane == 0) s_part[wave] = ss;
  __syncthreads();
  const double tot = ((s_part[0] + s_part[1]) + s_part[2]) + s_part[3];
  const float r = static_cast<float>(1.0 / sqrt(tot / static_cast<double>(K) + static_cast<double>(eps)));
#pragma unroll
  for (int i = 0; i < NCH; i++) {
    const int64_t c8 = t + 256 * i;
    if (c8 < nch) {
      const float4 g0 = *reinterpret_cast<const float4*>(g + 8 * c8);
      const float4 g1 = *reinterpret_cast<const float4*>(g + 8 * c8 + 4);
      const float gw[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      float xn[8];
#pragma unroll
      for (int e = 0; e < 8; e++) xn[e] = (v[i][e] * r) * gw[e];
      quantize8_store<WS>(xn, row, c8, K, q, d, S_int, dS, dsp, dxT, Mp);
    }
  }
}

// Per-256 activation scales (the Q8_K-style block of aprender issue #5475,
// section "Ask"): the same steps over a whole 256-value super-block -- 32
// lanes of eight values, amax over the 32 lanes -- with the code sums kept per
// 32-value sub-block.  WS: the GEMM workspace of the per-32 quantiser with the
// super-block's scale in all eight of its blocks (dx, dxT) and dS = d * S per
// sub-block (so every GEMM kernel reads it unchanged); otherwise the hook
// layout (q [M][K], d [M][K/256], S [M][K/32] int32).
template <int XDT, bool WS>
__global__ __launch_bounds__(256) void act_quant256_kernel(const void* __restrict__ x, int64_t M,
                                                           int64_t K, int8_t* __restrict__ q,
                                                           float* __restrict__ d,
                                                           int32_t* __restrict__ S_int,
                                                           float* __restrict__ dS,
                                                           uint16_t* __restrict__ dsp,
                                                           float* __restrict__ dxT, int64_t Mp) {
  const int64_t per_row = K / 8;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= M * per_row) return;  // whole groups of 32 lanes leave together (K % 256 == 0)
  const int64_t row = idx / per_row;
  const int64_t c8 = idx - row * per_row;
  const int64_t b = c8 >> 2, sb = c8 >> 5;

  float v[8];
  load8<XDT>(x, row, K, c8, v);

  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int m = 1; m < 32; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));

  float dv = 0.0f, id = 0.0f;
  if (amax != 0.0f) {
    dv = amax / 127.0f;  // correctly rounded IEEE division
    id = 1.0f / dv;      // correctly rounded IEEE division
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
    const int64_t nb = K / 32;
    if (WS) {
      const float ds = dv * static_cast<float>(s);
      d[row * nb + b] = dv;
      dxT[b * Mp + row] = dv;
      dS[row * nb + b] = ds;
      uint16_t p0, p1, p2;
      split3_bf16(ds, p0, p1, p2);
      uint16_t* o = dsp + ((row * (K / 256) + (b >> 3)) * 3) * 8 + (b & 7);
      o[0] = p0;
      o[8] = p1;
      o[16] = p2;
    } else {
      S_int[row * nb + b] = s;
      if ((c8 & 31) == 0) d[row * (K / 256) + sb] = dv;
    }
  }
}

}  // namespace qg

hipError_t qg_launch_act_quant256_ws(const void* x, int x_dtype, int64_t M, int64_t K,
                                     const QgWorkspace& ws, hipStream_t stream) {
  const dim3 g(static_cast<unsigned>((M * (K / 8) + 255) / 256));
  if (x_dtype == QG_BF16)
    qg::act_quant256_kernel<QG_BF16, true><<<g, dim3(256), 0, stream>>>(x, M, K, ws.q, ws.dx, nullptr,
                                                                        ws.dS, ws.dsp, ws.dxT, ws.Mp);
  else
    qg::act_quant256_kernel<QG_F32, true><<<g, dim3(256), 0, stream>>>(x, M, K, ws.q, ws.dx, nullptr,
                                                                       ws.dS, ws.dsp, ws.dxT, ws.Mp);
  return hipGetLastError();
}

hipError_t qg_launch_act_quant256_hook(const void* x, int x_dtype, int64_t M, int64_t K, int8_t* q,
                                       float* d256, int32_t* S32, hipStream_t stream) {
  const dim3 g(static_cast<unsigned>((M * (K / 8) + 255) / 256));
  if (x_dtype == QG_BF16)
    qg::act_quant256_kernel<QG_BF16, false><<<g, dim3(256), 0, stream>>>(x, M, K, q, d256, S32, nullptr,
                                                                         nullptr, nullptr, 0);
  else
    qg::act_quant256_kernel<QG_F32, false><<<g, dim3(256), 0, stream>>>(x, M, K, q, d256, S32, nullptr,
                                                                        nullptr, nullptr, 0);
  return hipGetLastError();
}

namespace {
std::atomic<int> g_planted_quant_sleeps{0};
}  // namespace

void qg_set_planted_quant_sleeps(int sleeps) { g_planted_quant_sleeps.store(sleeps); }

hipError_t qg_launch_act_quant_ws(const void* x, int x_dtype, int64_t M, int64_t K,
                                  const QgWorkspace& ws, hipStream_t stream) {
  const int sleeps = g_planted_quant_sleeps.load(std::memory_order_relaxed);
  const int64_t blocks = (M * (K / 8) + 255) / 256;
  const dim3 g(static_cast<unsigned>(blocks));
  if (x_dtype == QG_BF16)
    qg::act_quant_kernel<QG_BF16, true><<<g, dim3(256), 0, stream>>>(x, M, K, ws.q, ws.dx, nullptr,
                                                                     ws.dS, ws.dsp, ws.dxT, ws.Mp, sleeps);
  else
    qg::act_quant_kernel<QG_F32, true><<<g, dim3(256), 0, stream>>>(x, M, K, ws.q, ws.dx, nullptr,
                                                                    ws.dS, ws.dsp, ws.dxT, ws.Mp, sleeps);
  return hipGetLastError();
}

hipError_t qg_launch_act_quant_hook(const void* x, int x_dtype, int64_t M, int64_t K, int8_t* q,
                                    float* d, int32_t* S, hipStream_t stream) {
  const int64_t blocks = (M * (K / 8) + 255) / 256;
  const dim3 g(static_cast<unsigned>(blocks));
  if (x_dtype == QG_BF16)
    qg::act_quant_kernel<QG_BF16, false><<<g, dim3(256), 0, stream>>>(x, M, K, q, d, S, nullptr,
                                                                      nullptr, nullptr, 0, 0);
  else
    qg::act_quant_kernel<QG_F32, false><<<g, dim3(256), 0, stream>>>(x, M, K, q, d, S, nullptr,
                                                                     nullptr, nullptr, 0, 0);
  return hipGetLastError();
}

namespace {

template <bool WS, int NCH>
void launch_rms_nch(const void* x, int x_dtype, const float* g, float eps, int64_t M, int64_t K, int8_t* q,
                    float* d, int32_t* S, float* dS, uint16_t* dsp, float* dxT, int64_t Mp,
                    hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(M));
  if (x_dtype == QG_BF16)
    qg::rmsnorm_quant_kernel<QG_BF16, WS, NCH><<<grid, dim3(256), 0, stream>>>(x, g, eps, K, q, d, S, dS, dsp,
                                                                               dxT, Mp);
  else
    qg::rmsnorm_quant_kernel<QG_F32, WS, NCH><<<grid, dim3(256), 0, stream>>>(x, g, eps, K, q, d, S, dS, dsp,
                                                                              dxT, Mp);
}

template <bool WS>
hipError_t launch_rms(const void* x, int x_dtype, const float* g, float eps, int64_t M, int64_t K, int8_t* q,
                      float* d, int32_t* S, float* dS, uint16_t* dsp, float* dxT, int64_t Mp,
                      hipStream_t stream) {
  if (K > kRmsMaxK) return hipErrorInvalidValue;
  const int64_t per_lane = (K / 8 + 255) / 256;  // chunks per lane
  if (per_lane <= 1) launch_rms_nch<WS, 1>(x, x_dtype, g, eps, M, K, q, d, S, dS, dsp, dxT, Mp, stream);
  else if (per_lane <= 2) launch_rms_nch<WS, 2>(x, x_dtype, g, eps, M, K, q, d, S, dS, dsp, dxT, Mp, stream);
  else if (per_lane <= 4) launch_rms_nch<WS, 4>(x, x_dtype, g, eps, M, K, q, d, S, dS, dsp, dxT, Mp, stream);
  else if (per_lane <= 8) launch_rms_nch<WS, 8>(x, x_dtype, g, eps, M, K, q, d, S, dS, dsp, dxT, Mp, stream);
  else launch_rms_nch<WS, 16>(x, x_dtype, g, eps, M, K, q, d, S, dS, dsp, dxT, Mp, stream);
  return hipGetLastError();
}

}  // namespace

hipError_t qg_launch_rmsnorm_quant_ws(const void* x, int x_dtype, const float* g, float eps, int64_t M,
                                      int64_t K, const QgWorkspace& ws, hipStream_t stream) {
  return launch_rms<true>(x, x_dtype, g, eps, M, K, ws.q, ws.dx, nullptr, ws.dS, ws.dsp, ws.dxT, ws.Mp, stream);
}

hipError_t qg_launch_rmsnorm_quant_hook(const void* x, int x_dtype, const float* g, float eps, int64_t M,
                                        int64_t K, int8_t* q, float* d, int32_t* S, hipStream_t stream) {
  return launch_rms<false>(x, x_dtype, g, eps, M, K, q, d, S, nullptr, nullptr, nullptr, 0, stream);
}
