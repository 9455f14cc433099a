// Device-side helpers shared by the gfx950 kernels of libqgemm.so.
//
// Everything here is written for CDNA4 (gfx950): 64-lane wavefronts, int8
// matrix-core instructions, binary16 conversions in hardware.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qgemm.h"

namespace qg {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kQ4Bytes = 144;  // bytes per Q4_K super-block (256 values)
constexpr int kQ6Bytes = 210;  // bytes per Q6_K super-block (256 values)
constexpr int kQ5Bytes = 176;  // bytes per Q5_K super-block (256 values)
constexpr int kQ8Bytes = 34;   // bytes per Q8_0 block (32 values)
constexpr int kRowPad = 256;   // activation rows are padded to this multiple in the workspace

// 1.5 * 2^23 as an fp32 bit pattern.  An int32 accumulator started at this
// value and increased by a small integer I (|I| < 2^22) reads back as the fp32
// number 12582912 + I, so the matrix core's int32 result needs no conversion
// instruction before the fp32 epilogue.
constexpr int kMagicBits = 0x4B400000;
constexpr float kMagic = 12582912.0f;

__device__ __forceinline__ float half_to_float(uint32_t bits16) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

__device__ __forceinline__ float bits_to_float(int b) { return __builtin_bit_cast(float, b); }

// Q4_K packed sub-block scales/mins: the 12 scale bytes as three little-endian
// dwords s0 (bytes 0-3), s1 (4-7), s2 (8-11).  Returns the eight 6-bit scales
// as two dwords of bytes (sc[0..3], sc[4..7]) and likewise the mins.
//   j < 4 : sc = low 6 bits of byte j, m = low 6 bits of byte j+4
//   j >= 4: low nibble from byte j+4 (sc: low half, m: high half), top 2 bits
//           from bits 6-7 of byte j-4 (sc) or byte j (m)
struct Q4Scales {
  uint32_t sc_lo, sc_hi, m_lo, m_hi;
};
__device__ __forceinline__ Q4Scales unpack_q4_scales(uint32_t s0, uint32_t s1, uint32_t s2) {
  Q4Scales r;
  r.sc_lo = s0 & 0x3F3F3F3Fu;
  r.m_lo = s1 & 0x3F3F3F3Fu;
  r.sc_hi = (s2 & 0x0F0F0F0Fu) | ((s0 >> 2) & 0x30303030u);
  r.m_hi = ((s2 >> 4) & 0x0F0F0F0Fu) | ((s1 >> 2) & 0x30303030u);
  return r;
}
__device__ __forceinline__ uint32_t byte_of(uint32_t w, int i) { return (w >> (8 * i)) & 0xFFu; }

// Byte j (0..7) of the eight-byte value hi:lo, for a run-time j.  Written as a
// bitwise select on values so the compiler never spills the pair to memory to
// index it.
__device__ __forceinline__ uint32_t sub_byte(uint32_t lo, uint32_t hi, int j) {
  const uint32_t mask = 0u - static_cast<uint32_t>(j >> 2);  // all ones when j >= 4
  const uint32_t w = lo ^ ((lo ^ hi) & mask);
  return __builtin_amdgcn_ubfe(w, 8 * (j & 3), 8);
}

// Q6_K codes arrive as bytes q6 in [0, 63]; the matrix core wants the signed
// value q6 - 32 in every byte.  Setting bit 7 first keeps the per-byte
// subtraction from borrowing into the next byte; flipping bit 7 back leaves
// (q6 - 32) mod 256 in each byte.
__device__ __forceinline__ uint32_t q6_to_signed(uint32_t q) {
  return ((q | 0x80808080u) - 0x20202020u) ^ 0x80808080u;
}

// Load 4 bytes from a 2-byte-aligned global address (Q6_K blocks are 210 bytes,
// so odd blocks start at 2 mod 4) with dword loads only.  Reads the aligned
// dword holding the first byte and, when the address is not dword aligned, the
// dword after it; the caller guarantees both lie inside the buffer.
__device__ __forceinline__ uint32_t load_u32_a2(const uint8_t* p) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  const uint32_t* base = reinterpret_cast<const uint32_t*>(a & ~uintptr_t(3));
  const uint32_t lo = base[0];
  if ((a & 3) == 0) return lo;
  const uint32_t hi = base[1];
  return __builtin_amdgcn_alignbyte(hi, lo, static_cast<uint32_t>(a & 3));
}

__device__ __forceinline__ uint16_t load_u16(const uint8_t* p) {
  return *reinterpret_cast<const uint16_t*>(p);
}

// Output element of a tiled GEMM: a non-temporal (streaming) store, so that
// the M x N fp32 output (8-15 MB for one 512-row ubatch, more than an XCD's
// 4 MB L2) does not evict the weight and activation tiles other workgroups
// still read (measured 1-5% faster on the workloads' shapes).
__device__ __forceinline__ void store_out(float* p, float v) { __builtin_nontemporal_store(v, p); }
// The same at device scope: written through to memory rather than kept in
// the XCD's L2, where it would push out activation tiles that later
// workgroups reuse (the one-tile Q4_K kernel at 512x4096->24576: 2 MB fewer
// L2 fills per launch, the same time).
__device__ __forceinline__ void store_out_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// fp32 -> bfloat16 bits, rounded to nearest with ties to even (a NaN stays a
// quiet NaN; values past the largest bfloat16 round to infinity).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((b >> 16) | 0x0040u);
  return static_cast<uint16_t>((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

// SwiGLU of one gate/up pair: silu(g) * u with silu(g) = g / (1 + e^-g),
// rounded once to bfloat16.  In fp32 on the hardware's exp2 and reciprocal
// (v_exp_f32, v_rcp_f32; 1 ulp each): e^-g = 2^(-g*log2 e), whose argument
// rounding moves e^-g by at most |g| * 2^-24 relative; with the add and the
// two products the fp32 value is within |g| * 2^-24 + 2^-20 of silu(g) * u
// relative, under 2^-17 for |g| < 88.7 and far below the 2^-8 of the bfloat16
// rounding.  For g < -87.3 the reciprocal falls below the normal range and
// returns 0 (below -88.7 e^-g overflows to infinity first), so silu evaluates
// to -0 where the exact value is below 1.1e-36 in magnitude; for large g it
// is g.
__device__ __forceinline__ uint16_t swiglu_bf16(float g, float u) {
  constexpr float kLog2e = 1.4426950408889634f;
  const float e = __builtin_amdgcn_exp2f(-g * kLog2e);
  return f32_to_bf16_rne(g * __builtin_amdgcn_rcpf(1.0f + e) * u);
}

}  // namespace qg

// ---- workspace: the quantised activations, as the GEMM kernels read them ----
//   q   [Mp][K]             int8 codes
//   dx  [Mp][K/32]          fp32 block scales, row-major
//   dxT [K/32][Mp]          the same scales, block-major
//   dS  [Mp][K/32]          fp32 dx * S (scaled block sums), row-major
//   dsp [Mp][K/256][3][8]   dS split exactly into three bfloat16 pieces
//                           (dS = p0 + p1 + p2), grouped per super-block
// Mp is M rounded up to kRowPad; rows M..Mp-1 are never written and only ever
// feed output rows that are discarded.
struct QgWorkspace {
  int8_t* q;
  float* dx;
  float* dxT;
  float* dS;
  uint16_t* dsp;
  int64_t Mp;
};

hipError_t qg_launch_act_quant_ws(const void* x, int x_dtype, int64_t M, int64_t K,
                                  const QgWorkspace& ws, hipStream_t stream);
// Planted delay of the workspace quantiser (timing falsifier), in units of 64
// shader clocks; 0 = none.
void qg_set_planted_quant_sleeps(int sleeps);
hipError_t qg_launch_act_quant_hook(const void* x, int x_dtype, int64_t M, int64_t K, int8_t* q,
                                    float* d, int32_t* S, hipStream_t stream);
// per-256 activation scales: the same workspace layout with each super-block's
// scale in all eight of its 32-value blocks; hook layout d [M][K/256], S [M][K/32]
hipError_t qg_launch_act_quant256_ws(const void* x, int x_dtype, int64_t M, int64_t K,
                                     const QgWorkspace& ws, hipStream_t stream);
hipError_t qg_launch_act_quant256_hook(const void* x, int x_dtype, int64_t M, int64_t K, int8_t* q,
                                       float* d256, int32_t* S32, hipStream_t stream);
hipError_t qg_launch_gemm_q4k(const uint8_t* W, const QgWorkspace& ws, int64_t M, int64_t N,
                              int64_t K, float* y, hipStream_t stream, bool a256 = false);
hipError_t qg_launch_gemm_q6k(const uint8_t* W, const QgWorkspace& ws, int64_t M, int64_t N,
                              int64_t K, float* y, hipStream_t stream);
hipError_t qg_launch_gemm_skinny(const uint8_t* W, int fmt, const QgWorkspace& ws, int64_t M,
                                 int64_t N, int64_t K, float* y, hipStream_t stream);
// Name of the kernel each launcher picks for a problem (diagnostics: matches
// the kernel names a profiler reports).
const char* qg_gemm_q4k_kernel_name(int64_t M, int64_t N, int64_t K, bool a256 = false);
// Q5_K: the Q4_K kernels with the fifth code bit or-ed into the nibble codes
hipError_t qg_launch_gemm_q5k(const uint8_t* W, const QgWorkspace& ws, int64_t M, int64_t N,
                              int64_t K, float* y, hipStream_t stream);
const char* qg_gemm_q5k_kernel_name(int64_t M, int64_t N, int64_t K);
// Q8_0: the tiled Q4_K kernel body with the int8 codes taken as they are
hipError_t qg_launch_gemm_q80(const uint8_t* W, const QgWorkspace& ws, int64_t M, int64_t N,
                              int64_t K, float* y, hipStream_t stream);
const char* qg_gemm_q80_kernel_name(int64_t M, int64_t N, int64_t K);
// Q4_K gate+up GEMM with the SwiGLU epilogue (W: 2F rows, gate then up; h:
// bfloat16 [M][F]).  Fusable when the problem takes one of the LDS-tiled
// kernels and the weight offsets fit the kernels' 32-bit load offsets.
bool qg_q4k_swiglu_fusable(int64_t M, int64_t F, int64_t K);
hipError_t qg_launch_gemm_q4k_swiglu(const uint8_t* W, const QgWorkspace& ws, int64_t M, int64_t F,
                                     int64_t K, uint16_t* h, hipStream_t stream);
const char* qg_gemm_q4k_swiglu_kernel_name(int64_t M, int64_t F, int64_t K);
// The same over Q4_K, Q5_K or Q8_0 weights (the format's own block shapes).
bool qg_swiglu_fusable(int fmt, int64_t M, int64_t F, int64_t K);
hipError_t qg_launch_gemm_swiglu(const uint8_t* W, int fmt, const QgWorkspace& ws, int64_t M, int64_t F,
                                 int64_t K, uint16_t* h, hipStream_t stream);
const char* qg_gemm_swiglu_kernel_name(int fmt, int64_t M, int64_t F, int64_t K);
// h [M][F] = bfloat16(silu(y[m][f]) * y[m][F + f]) from y [M][2F] fp32
hipError_t qg_launch_swiglu(const float* y, int64_t M, int64_t F, uint16_t* h, hipStream_t stream);
// RMSNorm fused into the per-32 quantiser (K <= kRmsMaxK)
constexpr int64_t kRmsMaxK = 32768;
hipError_t qg_launch_rmsnorm_quant_ws(const void* x, int x_dtype, const float* g, float eps, int64_t M,
                                      int64_t K, const QgWorkspace& ws, hipStream_t stream);
hipError_t qg_launch_rmsnorm_quant_hook(const void* x, int x_dtype, const float* g, float eps, int64_t M,
                                        int64_t K, int8_t* q, float* d, int32_t* S, hipStream_t stream);
const char* qg_gemm_q6k_kernel_name(int64_t M, int64_t N, int64_t K);
const char* qg_gemm_skinny_kernel_name(int fmt, int64_t M, int64_t N, int64_t K);
hipError_t qg_launch_dequant(const uint8_t* W, int fmt, int64_t N, int64_t K, float* w,
                             hipStream_t stream);
// the dequantise-to-fp16 branch
hipError_t qg_launch_to_f16(const void* x, int x_dtype, int64_t M, int64_t K, uint16_t* x16,
                            hipStream_t stream);
hipError_t qg_launch_dequant_f16(const uint8_t* W, int fmt, int64_t N, int64_t K, uint16_t* w16,
                                 hipStream_t stream);
hipError_t qg_launch_gemm_deq_f16(const uint8_t* W, int fmt, const uint16_t* x16, int64_t M,
                                  int64_t N, int64_t K, float* y, hipStream_t stream);
const char* qg_gemm_deq_f16_kernel_name(int fmt, int64_t M, int64_t N, int64_t K);
// shader-clock probe (benchmark receipts): ticks[0..2] as qgemm_sclk_probe documents
hipError_t qg_launch_sclk_probe(uint64_t* ticks, int iters, hipStream_t stream);
// read probe (benchmark floor): bytes read once from src, as qgemm_read_probe documents
hipError_t qg_launch_read_probe(const void* src, int64_t bytes, hipStream_t stream);
hipError_t qg_launch_block_partials(const uint8_t* W, int fmt, const int8_t* qx, int64_t M,
                                    int64_t N, int64_t K, int32_t* out, hipStream_t stream);
