// The other design branch: dequantise Q4_K weights to binary16 inside the GEMM
// and contract on the fp16 matrix cores (gfx950).
//
// aprender issue #5475 ("apr serve / apr run: Qwen3.5 on CPU prefills one token
// at a time ..."), section "Ask", item 1, weighs two kernels for the batched
// quantised matmul: dequantise a weight tile and call a float GEMM, or the
// row-batched fused Q4_K x int8 kernel that the rest of this library builds.
// This file is the first branch, measured beside the second on the same
// shapes.  On the matrix cores a float GEMM takes 16-bit operands; binary16 is
// used (11 significant bits against bfloat16's 8), and each step is rounded
// once, to nearest even:
//   x16 = f16(x)                                   to_f16_kernel
//   dsc = f16(d*sc[j]), dmn = f16(dmin*m[j])       per sub-block, in the GEMM
//   w16 = f16(dsc*q - dmn)                         one fp16 fma per weight
//   y   = sum_k x16*w16                            fp32 accumulation (MFMA)
// d*sc and dmin*m are exact in fp32 (binary16 times a 6-bit integer), so their
// conversions round once; q is exact in fp16.  Zero weights may come out as -0.
//
// Layout.  A workgroup of WM x WN waves computes a BM x BN output block, each
// wave TM x TN tiles of 32x32 (v_mfma_f32_32x32x16_f16).  K advances in stages
// of 64 values (one quarter q of a super-block: sub-blocks 2q and 2q+1), held
// in an NS-deep LDS ring filled by global_load_lds_dwordx4:
//   A  [BM][8 chunks of 16 B]  x16 rows; chunk c of row r sits at c ^ ((r/2)%8)
//                              so that the 16 lanes of one LDS pass, reading 16
//                              rows at the same chunk, hit 16 distinct bank groups
//   W  [3][BN][16 B]           per column: the block header (d, dmin, 12 scale
//                              bytes), then the quarter's 32 code bytes as two
//                              16-byte pieces; piece-major so that 32 lanes
//                              reading 32 columns read 512 contiguous bytes
// Lane (column n = lane%32, half h = lane/32) dequantises the 32 weights of its
// piece h: low nibbles (values 16h..16h+15 of sub-block 2q) and high nibbles
// (the same positions of sub-block 2q+1).  K-step t (of 4) of the quarter
// gives lane half h the eight values 16h + 8(t%2) + 32(t/2) + 0..7, and the
// activation fragment takes the same eight values of its row, so the two
// operands agree on every k.
//
// Dequantisation, two values per instruction (packed fp16):
//   v_perm_b32 puts two code bytes under the exponent byte 0x64 (binary16
//   1024 + q exactly), v_pk_add_f16 removes the 1024 (exact), v_pk_fma_f16
//   gives f16(dsc*q - dmn) for both.  About 1.9 vector instructions per
//   weight, shared by the TM row tiles of the wave.
#include "common.h"
#include "lds_stage.h"
#include "mfma_epilogue.h"

namespace qg {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- x -> fp16

// Eight values per thread: x (fp32 or bf16) to binary16, round to nearest even
// (v_cvt_f16_f32; bf16 widens to fp32 exactly first).
template <int XDT>
__global__ __launch_bounds__(256) void to_f16_kernel(const void* __restrict__ x, int64_t total8,
                                                     uint16_t* __restrict__ x16) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total8) return;
  float v[8];
  if (XDT == QG_BF16) {
    const uint4 raw = reinterpret_cast<const uint4*>(x)[i];
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int k = 0; k < 4; k++) {
      v[2 * k] = __builtin_bit_cast(float, w[k] << 16);
      v[2 * k + 1] = __builtin_bit_cast(float, w[k] & 0xFFFF0000u);
    }
  } else {
    const float4 a = reinterpret_cast<const float4*>(x)[2 * i];
    const float4 b = reinterpret_cast<const float4*>(x)[2 * i + 1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  uint32_t o[4];
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const h2 p = {static_cast<_Float16>(v[2 * k]), static_cast<_Float16>(v[2 * k + 1])};
    o[k] = __builtin_bit_cast(uint32_t, p);
  }
  reinterpret_cast<uint4*>(x16)[i] = make_uint4(o[0], o[1], o[2], o[3]);
}

// ---------------------------------------------------------------- dequantisation

// Two code bytes (bytes lo_sel, lo_sel+1 of L, each below 16) -> the pair
// f16(dsc*q - dmn) for both.  SEL is the v_perm_b32 selector that places byte
// 2p of L in bits 0-7 and byte 2p+1 in bits 16-23 under the byte 0x64 of the
// other operand: binary16 0x64qq = 1024 + qq.
template <uint32_t SEL>
__device__ __forceinline__ uint32_t deq_pair(uint32_t L, h2 dsc, h2 ndmn) {
  const h2 biased = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, L, SEL));
  const h2 q = biased + h2{static_cast<_Float16>(-1024.0f), static_cast<_Float16>(-1024.0f)};
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, dsc, ndmn));
}

// The 32 binary16 weights that one lane takes from 16 code bytes of quarter
// qt of a Q4_K super-block (raw: bytes 16h..16h+15 of the quarter's 32), as
// the B operands of the quarter's four K-steps (pairs of values per dword):
//   out[0], out[1]  low nibbles of bytes 0-7, 8-15   (sub-block 2qt)
//   out[2], out[3]  high nibbles of bytes 0-7, 8-15  (sub-block 2qt+1)
// hdr: the block's first 16 bytes (d, dmin, packed scales).
__device__ __forceinline__ void q4k_quarter_f16(const uint4& hdr, int qt, const uint4& raw,
                                                v4i (&out)[4]) {
  const Q4Scales s = unpack_q4_scales(hdr.y, hdr.z, hdr.w);
  const float d = half_to_float(hdr.x & 0xFFFFu), dmin = half_to_float(hdr.x >> 16);
  const int j0 = 2 * qt, j1 = 2 * qt + 1;
  // d*sc and dmin*m are exact in fp32; one rounding each to binary16
  const _Float16 dsc0 = static_cast<_Float16>(d * static_cast<float>(sub_byte(s.sc_lo, s.sc_hi, j0)));
  const _Float16 dsc1 = static_cast<_Float16>(d * static_cast<float>(sub_byte(s.sc_lo, s.sc_hi, j1)));
  const _Float16 dmn0 = static_cast<_Float16>(dmin * static_cast<float>(sub_byte(s.m_lo, s.m_hi, j0)));
  const _Float16 dmn1 = static_cast<_Float16>(dmin * static_cast<float>(sub_byte(s.m_lo, s.m_hi, j1)));
  const h2 a0 = {dsc0, dsc0}, a1 = {dsc1, dsc1};
  const h2 c0 = {-dmn0, -dmn0}, c1 = {-dmn1, -dmn1};
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const uint32_t lo = w[i] & 0x0F0F0F0Fu, hi = (w[i] >> 4) & 0x0F0F0F0Fu;
    const int t = i >> 1, e = 2 * (i & 1);
    out[t][e] = static_cast<int>(deq_pair<0x04010400u>(lo, a0, c0));
    out[t][e + 1] = static_cast<int>(deq_pair<0x04030402u>(lo, a0, c0));
    out[2 + t][e] = static_cast<int>(deq_pair<0x04010400u>(hi, a1, c1));
    out[2 + t][e + 1] = static_cast<int>(deq_pair<0x04030402u>(hi, a1, c1));
  }
}

// Test hook: every weight of W [N][K] as binary16 bits, through the same
// q4k_quarter_f16 as the GEMM.  One thread per (block, quarter, half).
__global__ __launch_bounds__(256) void dequant_f16_q4k_kernel(const uint8_t* __restrict__ W,
                                                              int64_t nthreads,
                                                              uint16_t* __restrict__ w16) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= nthreads) return;
  const int64_t blk = i >> 3;
  const int qt = static_cast<int>((i >> 1) & 3), h = static_cast<int>(i & 1);
  const uint8_t* b = W + blk * kQ4Bytes;
  const uint4 hdr = *reinterpret_cast<const uint4*>(b);
  const uint4 raw = *reinterpret_cast<const uint4*>(b + 16 + 32 * qt + 16 * h);
  v4i out[4];
  q4k_quarter_f16(hdr, qt, raw, out);
  // out[0..1]: values 64qt + 16h + 0..15; out[2..3]: values 64qt + 32 + 16h + 0..15
  v4i* o = reinterpret_cast<v4i*>(w16 + blk * 256 + 64 * qt + 16 * h);
  o[0] = out[0];
  o[1] = out[1];
  o[4] = out[2];
  o[5] = out[3];
}

// Q6_K: the 32 binary16 weights that lane half h takes from quarter qq of a
// super-block (values 64qq + 16t + 8h + 0..7 for K-steps t = 0..3: each
// K-step inside one 16-value sub-block, so one scale per step).  Value v of
// the quarter (l = v % 32) has its low 4 bits in ql[64(qq/2) + 32(v/32) + l]
// (the low nibble for even qq, the high one for odd) and its top 2 bits in
// qh[32(qq/2) + l], bits 4(qq%2) + 2(v/32) and up.  The lane passes its eight
// ql bytes of each K-step (ql[t]: bytes 16(t%2) + 8h + 0..7 of the 32 at
// offset 32(t/2)) and its qh bytes (qh[t%2]: bytes 16(t%2) + 8h + 0..7),
// the quarter's four int8 scales and d:  dsc = f16(d*sc), w16 = f16(dsc*(q6-32))
// (one rounding each: d*sc is exact in fp32, q6-32 in fp16).  0x64qq is the
// binary16 1024 + q6, so subtracting 1056 leaves q6 - 32 exactly.
__device__ __forceinline__ void q6k_quarter_f16(const uint2 (&ql)[4], const uint2 (&qh)[2],
                                                uint32_t sc4, uint32_t d_bits, int qq,
                                                v4i (&out)[4]) {
  const float d = half_to_float(d_bits);
  const uint32_t s_lo = 4u * static_cast<uint32_t>(qq & 1);
#pragma unroll
  for (int t = 0; t < 4; t++) {
    const float scf = static_cast<float>(static_cast<int8_t>((sc4 >> (8 * t)) & 0xFFu));
    const _Float16 dsc = static_cast<_Float16>(d * scf);
    const h2 a = {dsc, dsc};
    const uint32_t s_hi = s_lo + 2u * static_cast<uint32_t>(t >> 1);
    const uint32_t lw[2] = {ql[t].x, ql[t].y}, hw[2] = {qh[t & 1].x, qh[t & 1].y};
#pragma unroll
    for (int k = 0; k < 2; k++) {
      const uint32_t q6 = (((hw[k] >> s_hi) & 0x03030303u) << 4) | ((lw[k] >> s_lo) & 0x0F0F0F0Fu);
#pragma unroll
      for (int e = 0; e < 2; e++) {
        const uint32_t pb = __builtin_amdgcn_perm(0x64646464u, q6, e ? 0x04030402u : 0x04010400u);
        const h2 q = __builtin_bit_cast(h2, pb) +
                     h2{static_cast<_Float16>(-1056.0f), static_cast<_Float16>(-1056.0f)};
        out[t][2 * k + e] = static_cast<int>(__builtin_bit_cast(uint32_t, q * a));
      }
    }
  }
}

// Test hook for Q6_K: every weight as binary16 bits through q6k_quarter_f16.
// One thread per (block, quarter, half).
__global__ __launch_bounds__(256) void dequant_f16_q6k_kernel(const uint8_t* __restrict__ W,
                                                              int64_t nthreads,
                                                              uint16_t* __restrict__ w16) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= nthreads) return;
  const int64_t blk = i >> 3;
  const int qq = static_cast<int>((i >> 1) & 3), h = static_cast<int>(i & 1);
  const uint8_t* b = W + blk * kQ6Bytes;
  const uint8_t* qlp = b + 64 * (qq >> 1);
  const uint8_t* qhp = b + 128 + 32 * (qq >> 1);
  uint2 ql[4], qh[2];
#pragma unroll
  for (int t = 0; t < 4; t++)
    ql[t] = make_uint2(load_u32_a2(qlp + 32 * (t >> 1) + 16 * (t & 1) + 8 * h),
                       load_u32_a2(qlp + 32 * (t >> 1) + 16 * (t & 1) + 8 * h + 4));
#pragma unroll
  for (int k = 0; k < 2; k++)
    qh[k] = make_uint2(load_u32_a2(qhp + 16 * k + 8 * h), load_u32_a2(qhp + 16 * k + 8 * h + 4));
  v4i out[4];
  q6k_quarter_f16(ql, qh, load_u32_a2(b + 192 + 4 * qq), load_u16(b + 208), qq, out);
  v4i* o = reinterpret_cast<v4i*>(w16 + blk * 256 + 64 * qq + 8 * h);
#pragma unroll
  for (int t = 0; t < 4; t++) o[2 * t] = out[t];   // values 64qq + 16t + 8h + 0..7
}

// ---------------------------------------------------------------- the GEMM

// KS > 1: KS groups of WM x WN waves compute the same block over disjoint
// ranges of stages, each with its own ring; the partial blocks are summed
// through LDS in group order at the end (deterministic, no atomics).
// FMT: QG_Q4_K or QG_Q6_K.  Per column and stage the W region holds, piece-
// major (16 B per piece): Q4_K -- the block header and the quarter's 32 code
// bytes (3 pieces); Q6_K -- the 64 ql bytes and 32 qh bytes of the quarter's
// half super-block, the 16 scales and the block's last 16 bytes (holding d)
// (8 pieces).
template <int FMT, int TM, int TN, int WM, int WN, int NS, int OCC, int KS>
__global__ __launch_bounds__(64 * WM * WN * KS) __attribute__((amdgpu_waves_per_eu(OCC))) void gemm_deq_f16_kernel(
    const uint8_t* __restrict__ W, const uint16_t* __restrict__ x16, int64_t M, int64_t N, int64_t K,
    float* __restrict__ y) {
  constexpr int NW = WM * WN;
  constexpr int BM = 32 * TM * WM, BN = 32 * TN * WN;
  constexpr int A_WL = BM * 8 / 64;                    // wave-loads of A per stage (whole)
  constexpr bool Q6 = FMT == QG_Q6_K;
  constexpr int PIECES = Q6 ? 8 : 3, BLK = Q6 ? kQ6Bytes : kQ4Bytes;
  constexpr int W_CH = PIECES * BN, W_WLR = (W_CH + 63) / 64;  // W chunks, real wave-loads
  // W padded so that every wave issues the same number of loads per stage
  constexpr int TOT = ((A_WL + W_WLR + NW - 1) / NW) * NW, W_WL = TOT - A_WL;
  constexpr int LPT = TOT / NW;                        // loads per thread per stage
  constexpr int A_BYTES = A_WL * 1024, W_BYTES = W_WLR * 1024;
  constexpr int STAGE = A_BYTES + W_BYTES;
  static_assert(BM % 16 == 0 && BN % 32 == 0, "tile shape");
  static_assert(NS >= 2 && LPT * (NS - 1) < 64, "vmcnt range");
  static_assert(KS * NS * STAGE <= 160 * 1024, "LDS budget");
  static_assert(KS == 1 || (KS - 1) * NW * TM * TN * 4096 <= KS * NS * STAGE, "reduction space");
  __shared__ __attribute__((aligned(16))) uint8_t lds_all[KS * NS * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave_all / NW, wave = wave_all - grp * NW;  // K-group, wave within the group
  uint8_t* const lds = lds_all + grp * NS * STAGE;            // this group's ring
  const int h = lane >> 5, l32 = lane & 31;
  const int wm = wave / WN, wn = wave % WN;
  const int64_t m_cta = static_cast<int64_t>(blockIdx.y) * BM;
  const int64_t n_cta = static_cast<int64_t>(blockIdx.x) * BN;
  const int ml0 = 32 * TM * wm, nl0 = 32 * TN * wn;
  const int64_t nsb = K / 256, nst = K / 64;
  const int64_t wrow = nsb * BLK;
  // this group's stages: st0 .. st0 + cnt - 1 (the launcher keeps KS <= K/64);
  // every group runs the longest group's count so that the barriers match
  const int64_t st0 = grp * nst / KS, cnt = (grp + 1) * nst / KS - st0;
  const int64_t stages = (nst + KS - 1) / KS;

  // Per-lane byte offsets of this wave's loads (computed once; tail rows and
  // columns clamped to the last valid one).  Load it of this wave is wave-load
  // g = wave + it*NW of the combined list: A wave-loads first, then the W ones
  // (taken modulo the real count, so the padding repeats real wave-loads).
  uint32_t voff[LPT];
  // the W pieces that move within a block with the stage: Q4_K code pieces by
  // 32 bytes per quarter; Q6_K ql pieces by 64 and qh pieces by 32 bytes per
  // half super-block; 0 for the rest
  uint32_t qmul[LPT];
#pragma unroll
  for (int it = 0; it < LPT; it++) {
    const int g = wave + it * NW;
    if (g < A_WL) {
      const int p = g * 64 + lane, row = p >> 3, c = (p & 7) ^ ((row >> 1) & 7);
      const int64_t m = m_cta + row < M ? m_cta + row : M - 1;
      voff[it] = static_cast<uint32_t>((m - m_cta) * K * 2 + 16 * c);
      qmul[it] = 0;
    } else {
      const int p = ((g - A_WL) % W_WLR) * 64 + lane;
      const int piece = p / BN, col = p - piece * BN;
      const int64_t n = n_cta + col < N ? n_cta + col : N - 1;
      const bool real = p < W_CH;
      uint32_t off, mul;
      if (Q6) {
        // pieces: ql 0..3 (bytes 16p), qh 4..5 (128 + 16(p-4)), scales (192), tail (194)
        off = piece < 4 ? 16u * piece : piece < 6 ? 128u + 16u * (piece - 4) : piece == 6 ? 192u : 194u;
        mul = piece < 4 ? 64u : piece < 6 ? 32u : 0u;
      } else {
        off = piece == 0 ? 0u : 16u * piece;
        mul = piece > 0 ? 32u : 0u;
      }
      voff[it] = real ? static_cast<uint32_t>((n - n_cta) * wrow) + off : 0u;
      qmul[it] = real ? mul : 0u;
    }
  }
  const uint8_t* const a_base = reinterpret_cast<const uint8_t*>(x16) + m_cta * K * 2;
  const uint8_t* const w_base = W + n_cta * wrow;

  auto issue_stage = [&](int64_t sl, int buf) {
    const int64_t s = st0 + (sl < cnt ? sl : cnt - 1);  // past the group's range: reload its last
    const int64_t sb = s >> 2;
    // the stage's step inside its block: Q4_K the quarter, Q6_K the half
    const uint32_t qt = Q6 ? static_cast<uint32_t>((s & 3) >> 1) : static_cast<uint32_t>(s & 3);
    uint8_t* sbase = lds + buf * STAGE;
#pragma unroll
    for (int it = 0; it < LPT; it++) {
      const int g = wave + it * NW;
      auto load_a = [&] { lds_dma16_sv(a_base + s * 128, voff[it], sbase + 1024 * g); };
      auto load_w = [&] {
        const int wl = (g - A_WL) % W_WLR;
        lds_dma16_sv(w_base + sb * BLK, voff[it] + qmul[it] * qt, sbase + A_BYTES + 1024 * wl);
      };
      // once unrolled, whether load `it` is an A or a W load folds to a
      // constant unless the boundary falls inside this round of NW wave-loads
      if ((it + 1) * NW <= A_WL || (it * NW < A_WL && g < A_WL)) load_a();
      else load_w();
    }
  };

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++) acc[i][j] = v16f{};

#pragma unroll
  for (int s0 = 0; s0 < NS - 1; s0++)
    if (s0 < stages) issue_stage(s0, s0);
  for (int64_t s = 0; s < stages; s++) {
    const int buf = static_cast<int>(s % NS);
    // stage s has landed once at most the NS-2 later stages' loads are
    // outstanding (near the end: all); after the barrier no wave still reads
    // stage s-1, whose buffer the next issue refills
    if (s + NS - 1 <= stages) wait_vm_barrier<LPT * (NS - 2)>();
    else wait_vm_barrier<0>();
    if (s + NS - 1 < stages) issue_stage(s + NS - 1, static_cast<int>((s + NS - 1) % NS));
    if (KS > 1 && s >= cnt) continue;  // a shorter group idles through the last step

    const uint8_t* sA = lds + buf * STAGE;
    const uint8_t* sW = sA + A_BYTES;
    const int qt = static_cast<int>((st0 + s) & 3);
    v4i bq[TN][4];
#pragma unroll
    for (int j = 0; j < TN; j++) {
      const int col = nl0 + 32 * j + l32;
      if constexpr (Q6) {
        uint2 ql[4], qh[2];
#pragma unroll
        for (int t = 0; t < 4; t++)
          ql[t] = *reinterpret_cast<const uint2*>(sW + 16 * ((2 * (t >> 1) + (t & 1)) * BN + col) + 8 * h);
#pragma unroll
        for (int k = 0; k < 2; k++) qh[k] = *reinterpret_cast<const uint2*>(sW + 16 * ((4 + k) * BN + col) + 8 * h);
        const uint32_t sc4 = *reinterpret_cast<const uint32_t*>(sW + 16 * (6 * BN + col) + 4 * qt);
        const uint32_t dw = *reinterpret_cast<const uint32_t*>(sW + 16 * (7 * BN + col) + 12);
        q6k_quarter_f16(ql, qh, sc4, dw >> 16, qt, bq[j]);
      } else {
        const uint4 hdr = *reinterpret_cast<const uint4*>(sW + 16 * col);
        const uint4 raw = *reinterpret_cast<const uint4*>(sW + 16 * ((1 + h) * BN + col));
        q4k_quarter_f16(hdr, qt, raw, bq[j]);
      }
    }
#pragma unroll
    for (int t = 0; t < 4; t++) {
      // the activation chunk holding the K-step's eight values for this lane half
      const int c = Q6 ? 2 * t + h : 2 * h + (t & 1) + 4 * (t >> 1);
      h8 a[TM];
#pragma unroll
      for (int i = 0; i < TM; i++) {
        const int row = ml0 + 32 * i + l32;
        a[i] = *reinterpret_cast<const h8*>(sA + row * 128 + 16 * (c ^ ((row >> 1) & 7)));
      }
#pragma unroll
      for (int j = 0; j < TN; j++) {
        const h8 b = __builtin_bit_cast(h8, bq[j][t]);
#pragma unroll
        for (int i = 0; i < TM; i++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b, acc[i][j], 0, 0, 0);
      }
    }
  }

  if constexpr (KS > 1) {
    // groups 1..KS-1 leave their blocks in LDS (the rings are free once every
    // wave has passed the first barrier); group 0 adds them in group order
    float4* red = reinterpret_cast<float4*>(lds_all);  // [KS-1][NW][TM*TN*4][64]
    __syncthreads();
    if (grp > 0) {
#pragma unroll
      for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
          for (int q = 0; q < 4; q++)
            red[((((grp - 1) * NW + wave) * TM + i) * TN + j) * 4 * 64 + q * 64 + lane] =
                make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
    }
    __syncthreads();
    if (grp > 0) return;
#pragma unroll
    for (int g = 1; g < KS; g++)
#pragma unroll
      for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
          for (int q = 0; q < 4; q++) {
            const float4 v = red[((((g - 1) * NW + wave) * TM + i) * TN + j) * 4 * 64 + q * 64 + lane];
            acc[i][j][4 * q] += v.x;
            acc[i][j][4 * q + 1] += v.y;
            acc[i][j][4 * q + 2] += v.z;
            acc[i][j][4 * q + 3] += v.w;
          }
  }

#pragma unroll
  for (int j = 0; j < TN; j++) {
    const int64_t n = n_cta + nl0 + 32 * j + l32;
    if (n >= N) continue;
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int64_t m = m_cta + ml0 + 32 * i + acc_row(r, h);
        if (m < M) store_out(y + m * N + n, acc[i][j][r]);
      }
  }
}

template <int FMT, int TM, int TN, int WM, int WN, int NS, int OCC, int KS = 1>
static void launch_deq(const uint8_t* W, const uint16_t* x16, int64_t M, int64_t N, int64_t K,
                       float* y, hipStream_t stream) {
  constexpr int BM = 32 * TM * WM, BN = 32 * TN * WN;
  const dim3 grid(static_cast<unsigned>((N + BN - 1) / BN), static_cast<unsigned>((M + BM - 1) / BM));
  gemm_deq_f16_kernel<FMT, TM, TN, WM, WN, NS, OCC, KS><<<grid, dim3(64 * WM * WN * KS), 0, stream>>>(
      W, x16, M, N, K, y);
}

}  // namespace qg

namespace {
enum class DeqPick { k256x256, k256x128, k128x128, k64x128K2, k128x64K4, k128x64K3, k32x64K4 };

// Measured on the workloads' shapes.  Waves of 128x32 (four row tiles share
// one dequantised weight fragment) in 256x256 blocks of 16 waves (one per CU)
// when there are at least 160 of those (up to 399, or any number for
// K >= 4096), 256x128 blocks of 8 waves (two per CU) when they cover the CUs,
// else 128x128 blocks of 4 when there are at least 200.  Smaller grids split K
// inside the workgroup: Q4_K 64x128 blocks with two K-groups, 128x64 with four
// or 32x64 with four; Q6_K 128x64 with three or 32x64 with four.  Every split
// keeps at least one 64-value stage per group (K >= 256).
DeqPick pick_deq(int fmt, int64_t M, int64_t N, int64_t K) {
  const int64_t b256w = ((M + 255) / 256) * ((N + 255) / 256);
  const int64_t b256 = ((M + 255) / 256) * ((N + 127) / 128);
  const int64_t b128 = ((M + 127) / 128) * ((N + 127) / 128);
  const int64_t b64 = ((M + 63) / 64) * ((N + 127) / 128);
  if (b256w >= 160 && (b256w < 400 || K >= 4096)) return DeqPick::k256x256;
  if (b256 >= 256) return DeqPick::k256x128;
  if (b128 >= 200) return DeqPick::k128x128;
  // Q6_K (eight weight pieces per column): 128x64 blocks with three K-groups
  // from 128 such 64x128 blocks on (four two-stage rings would not fit LDS)
  if (fmt == QG_Q6_K) return b64 >= 128 ? DeqPick::k128x64K3 : DeqPick::k32x64K4;
  if (b64 >= 256) return DeqPick::k64x128K2;
  if (b64 >= 128) return DeqPick::k128x64K4;
  return DeqPick::k32x64K4;
}
}  // namespace

const char* qg_gemm_deq_f16_kernel_name(int fmt, int64_t M, int64_t N, int64_t K) {
  const bool q6 = fmt == QG_Q6_K;
  switch (pick_deq(fmt, M, N, K)) {
    case DeqPick::k256x256: return q6 ? "gemm_deq_f16_kernel<1, 4, 1, 2, 8, 2, 4, 1>" : "gemm_deq_f16_kernel<0, 4, 1, 2, 8, 2, 4, 1>";
    case DeqPick::k256x128: return q6 ? "gemm_deq_f16_kernel<1, 4, 1, 2, 4, 2, 4, 1>" : "gemm_deq_f16_kernel<0, 4, 1, 2, 4, 2, 4, 1>";
    case DeqPick::k128x128: return q6 ? "gemm_deq_f16_kernel<1, 4, 1, 1, 4, 2, 4, 1>" : "gemm_deq_f16_kernel<0, 4, 1, 1, 4, 2, 4, 1>";
    case DeqPick::k64x128K2: return q6 ? "gemm_deq_f16_kernel<1, 2, 1, 1, 4, 2, 4, 2>" : "gemm_deq_f16_kernel<0, 2, 1, 1, 4, 2, 4, 2>";
    case DeqPick::k128x64K4: return "gemm_deq_f16_kernel<0, 4, 1, 1, 2, 2, 2, 4>";
    case DeqPick::k128x64K3: return "gemm_deq_f16_kernel<1, 4, 1, 1, 2, 2, 2, 3>";
    case DeqPick::k32x64K4: return q6 ? "gemm_deq_f16_kernel<1, 1, 1, 1, 2, 2, 4, 4>" : "gemm_deq_f16_kernel<0, 1, 1, 1, 2, 2, 4, 4>";
  }
  return "?";
}

hipError_t qg_launch_to_f16(const void* x, int x_dtype, int64_t M, int64_t K, uint16_t* x16,
                            hipStream_t stream) {
  const int64_t total8 = M * K / 8;
  const dim3 g(static_cast<unsigned>((total8 + 255) / 256));
  if (x_dtype == QG_BF16)
    qg::to_f16_kernel<QG_BF16><<<g, dim3(256), 0, stream>>>(x, total8, x16);
  else
    qg::to_f16_kernel<QG_F32><<<g, dim3(256), 0, stream>>>(x, total8, x16);
  return hipGetLastError();
}

hipError_t qg_launch_dequant_f16(const uint8_t* W, int fmt, int64_t N, int64_t K, uint16_t* w16,
                                 hipStream_t stream) {
  if (fmt == QG_Q4_K) {
    const int64_t nthreads = N * (K / 256) * 8;
    qg::dequant_f16_q4k_kernel<<<dim3(static_cast<unsigned>((nthreads + 255) / 256)), dim3(256), 0,
                                 stream>>>(W, nthreads, w16);
  } else {
    const int64_t nthreads = N * (K / 256) * 8;
    qg::dequant_f16_q6k_kernel<<<dim3(static_cast<unsigned>((nthreads + 255) / 256)), dim3(256), 0,
                                 stream>>>(W, nthreads, w16);
  }
  return hipGetLastError();
}

template <int FMT>
static void launch_deq_fmt(DeqPick pick, const uint8_t* W, const uint16_t* x16, int64_t M, int64_t N,
                           int64_t K, float* y, hipStream_t stream) {
  switch (pick) {
    case DeqPick::k256x256: qg::launch_deq<FMT, 4, 1, 2, 8, 2, 4, 1>(W, x16, M, N, K, y, stream); break;
    case DeqPick::k256x128: qg::launch_deq<FMT, 4, 1, 2, 4, 2, 4, 1>(W, x16, M, N, K, y, stream); break;
    case DeqPick::k128x128: qg::launch_deq<FMT, 4, 1, 1, 4, 2, 4, 1>(W, x16, M, N, K, y, stream); break;
    case DeqPick::k64x128K2: qg::launch_deq<FMT, 2, 1, 1, 4, 2, 4, 2>(W, x16, M, N, K, y, stream); break;
    case DeqPick::k128x64K4:
      if constexpr (FMT == QG_Q4_K) qg::launch_deq<FMT, 4, 1, 1, 2, 2, 2, 4>(W, x16, M, N, K, y, stream);
      break;
    case DeqPick::k128x64K3:
      if constexpr (FMT == QG_Q6_K) qg::launch_deq<FMT, 4, 1, 1, 2, 2, 2, 3>(W, x16, M, N, K, y, stream);
      break;
    case DeqPick::k32x64K4: qg::launch_deq<FMT, 1, 1, 1, 2, 2, 4, 4>(W, x16, M, N, K, y, stream); break;
  }
}

hipError_t qg_launch_gemm_deq_f16(const uint8_t* W, int fmt, const uint16_t* x16, int64_t M, int64_t N,
                                  int64_t K, float* y, hipStream_t stream) {
  const DeqPick pick = pick_deq(fmt, M, N, K);
  if (fmt == QG_Q6_K) launch_deq_fmt<QG_Q6_K>(pick, W, x16, M, N, K, y, stream);
  else launch_deq_fmt<QG_Q4_K>(pick, W, x16, M, N, K, y, stream);
  return hipGetLastError();
}
