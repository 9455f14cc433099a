// Tiled prefill GEMM for Q6_K weights on the int8 matrix cores (gfx950).
//
// Same scheme as the Q4_K kernel (the fused "decode super-blocks in
// registers, int8 tensor-core GEMM" of sparkinfer PR #464, section "Summary"),
// with Q6_K's 16-value sub-blocks: one v_mfma_i32_32x32x16_i8 per sub-block,
// its int32 partial scaled by the sub-block's d*sc, and the activation scale
// dx of the 32-value block holding it.  Codes are fed to the matrix core as
// the signed bytes 4*(q6 - 32) (the six code bits in the top of the byte,
// which takes four instructions per four codes to build), and d*sc/4 scales
// the products, so there is no min term.
//
// Per y[m][n]: sum over 16-value sub-blocks s of dx[m][s/2] * d*sc[n][s] * I16.
// The accumulator starts at the bit pattern of M = 12582912.0f, so its int32
// result reads as the float f = M + I16.  The two sub-blocks a, b of one
// 32-value activation block share dx and are combined in two fmas:
// p = fma(f_a, dsc_a, -M*(dsc_a + dsc_b)) = I_a*dsc_a - M*dsc_b (the constant
// is exact: d*(sc_a + sc_b) has at most 20 significant bits), then
// t = fma(f_b, dsc_b, p) = I_a*dsc_a + I_b*dsc_b, and acc += t*dx.  p carries
// one rounding at the magnitude of M*dsc_b, i.e. an error below half a unit of
// I_b*dsc_b per block: far inside the output tolerance, and zero whenever the
// products are integers below 2^24 (unit scales).
//
// LDS pipeline (as the Q4_K kernel): WM x WN waves share super-block stages in
// an NS-deep ring (per K-group) filled by global_load_lds_dwordx4; one stage
// holds
//   A  [BM][256]  int8 activation codes, 16-byte chunks XOR-swizzled by row%16
//   W  [BN][224]  the 210-byte blocks: bytes 0..207 as 13 chunks, then bytes
//                 194..209 as a 14th chunk (so d sits at 222..223); the
//                 blocks start 2-byte aligned in global memory
//   DX [8][BM]    fp32 activation block scales, block-major (from dxT)
// Each wave owns TM x TN tiles of 32x32 outputs.  Per 32-value block a lane
// decodes the two sub-blocks' weight codes of its column from LDS (8 codes
// each: low nibbles from ql, two high bits from qh) and reads the 16 row
// scales its accumulator elements need.
//
// Two kernels share this arithmetic and differ in staging:
//   gemm_q6k_lds_kernel   one stage per super-block (above); large grids,
//                         2x1 tiles per wave (the decoded codes serve both)
//   gemm_q6k_half_kernel  one stage per half super-block (128 values), so
//                         that two stage buffers fit beside three more
//                         workgroups on a CU; one tile per wave, the
//                         activation chunks staged column-major (chunk c of
//                         every row, then chunk c+1), which turns every
//                         operand read into a per-lane base plus a constant
//                         offset, and the four blocks of a stage unrolled
#include "common.h"
#include "lds_stage.h"
#include "mfma_epilogue.h"

namespace qg {

constexpr int kQ6Row = 224;  // LDS bytes per staged Q6_K block

// KS groups of WM x WN waves compute the same BM x BN output block over
// disjoint super-block ranges of K and are summed through LDS in group order
// at the end (grids with few output blocks).  Stages sit in an NS-deep ring
// (NS >= 2).  Regions are padded to whole wave-loads; the extra loads of short
// waves repeat one of the region's wave-loads.
template <int TM, int TN, int WM, int WN, int NS, int OCC, int KS>
__global__ __launch_bounds__(64 * WM * WN * KS) __attribute__((amdgpu_waves_per_eu(OCC))) void gemm_q6k_lds_kernel(
    const uint8_t* __restrict__ W, const int8_t* __restrict__ qx, const float* __restrict__ dxT,
    int64_t Mp, int64_t M, int64_t N, int64_t K, float* __restrict__ y) {
  constexpr int NW = WM * WN;  // waves per group
  constexpr int BM = 32 * TM * WM, BN = 32 * TN * WN;
  static_assert(kRowPad % BM == 0, "BM must divide the workspace row padding");
  constexpr int A_CH = BM * 256 / 16, W_CH = BN * kQ6Row / 16, X_CH = BM * 32 / 16;
  constexpr int A_WL = (A_CH + 63) / 64, W_WL = (W_CH + 63) / 64, X_WL = (X_CH + 63) / 64;
  constexpr int A_BYTES = A_WL * 1024, W_BYTES = W_WL * 1024, X_BYTES = X_WL * 1024;
  constexpr int STAGE = A_BYTES + W_BYTES + X_BYTES;
  static_assert(NS >= 2, "a ring of at least two stages");
  static_assert(KS * NS * STAGE <= 160 * 1024, "LDS budget");
  static_assert(KS == 1 || (KS - 1) * NW * TM * TN * 4096 <= KS * NS * STAGE, "reduction space");
  __shared__ __attribute__((aligned(16))) uint8_t lds[KS * NS * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave_all / NW, wave = wave_all - grp * NW;  // K-group, wave within the group
  const int h = lane >> 5, l32 = lane & 31;
  const int wm = wave / WN, wn = wave % WN;
  const int64_t m_cta = static_cast<int64_t>(blockIdx.y) * BM;
  const int64_t n_cta = static_cast<int64_t>(blockIdx.x) * BN;
  const int ml0 = 32 * TM * wm, nl0 = 32 * TN * wn;
  const int64_t nsb = K / 256;
  const int64_t wrow_bytes = nsb * kQ6Bytes;
  uint8_t* const glds = lds + grp * NS * STAGE;  // this group's ring
  // this group's super-blocks: sb0 .. sb0 + cnt - 1 (the launcher keeps KS <= nsb)
  const int64_t sb0 = grp * nsb / KS, cnt = (grp + 1) * nsb / KS - sb0;
  const int64_t iters = (nsb + KS - 1) / KS;  // the longest group's count

  // Stage loads region by region (A, W, DX) with per-lane byte offsets
  // computed once and wave-uniform bases advanced per super-block; the group's
  // waves issue a region's wave-loads round robin, modulo the region's count,
  // so that every wave issues the same number per stage and a fixed vmcnt
  // waits for a whole stage.  Tail rows and columns are clamped to the last
  // valid one, lanes past a region's end read its first chunk into its padding.
  constexpr int LA = (A_WL + NW - 1) / NW, LW = (W_WL + NW - 1) / NW;
  constexpr int LX = (X_WL + NW - 1) / NW;
  constexpr int LPT = LA + LW + LX;  // loads per thread per stage
  static_assert(LPT * (NS - 1) < 64, "vmcnt range");
  uint32_t voff[LPT];
#pragma unroll
  for (int it = 0; it < LA; it++) {
    const int q = ((wave + it * NW) % A_WL) * 64 + lane;
    const int row = q >> 4, c16 = (q & 15) ^ (row & 15);
    const int64_t m = m_cta + row < M ? m_cta + row : M - 1;
    voff[it] = q < A_CH ? static_cast<uint32_t>((m - m_cta) * K + 16 * c16) : 0u;
  }
#pragma unroll
  for (int it = 0; it < LW; it++) {
    const int qq = ((wave + it * NW) % W_WL) * 64 + lane, row = qq / 14, part = qq - 14 * row;
    const int64_t n = n_cta + row < N ? n_cta + row : N - 1;
    voff[LA + it] = qq < W_CH ? static_cast<uint32_t>((n - n_cta) * wrow_bytes + (part < 13 ? 16 * part : 194))
                              : 0u;
  }
#pragma unroll
  for (int it = 0; it < LX; it++) {
    const int qq = ((wave + it * NW) % X_WL) * 64 + lane;
    const int jb = qq / (BM / 4), r4 = qq - jb * (BM / 4);
    voff[LA + LW + it] = qq < X_CH ? static_cast<uint32_t>((jb * Mp + 4 * r4) * 4) : 0u;
  }
  auto issue_region = [&](const void* rbase, int first, int count, int nwl, int off, uint8_t* sbase) {
#pragma unroll
    for (int it = 0; it < count; it++) {
      const int wl = (wave + it * NW) % nwl;
      lds_dma16_sv(rbase, voff[first + it], sbase + off + 1024 * wl);
    }
  };
  auto issue_stage = [&](int64_t s, int buf) {
    const int64_t sb = sb0 + (s < cnt ? s : cnt - 1);  // past the group's range: reload its last
    uint8_t* sbase = glds + buf * STAGE;
    issue_region(qx + m_cta * K + sb * 256, 0, LA, A_WL, 0, sbase);
    issue_region(W + n_cta * wrow_bytes + sb * kQ6Bytes, LA, LW, W_WL, A_BYTES, sbase);
    issue_region(dxT + 8 * sb * Mp + m_cta, LA + LW, LX, X_WL, A_BYTES + W_BYTES, sbase);
  };

  v16i magic;
#pragma unroll
  for (int r = 0; r < 16; r++) magic[r] = kMagicBits;
  float acc[TM][TN][16];
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

#pragma unroll
  for (int s0 = 0; s0 < NS - 1; s0++)
    if (s0 < iters) issue_stage(s0, s0);
  for (int64_t s = 0; s < iters; s++) {
    const int buf = static_cast<int>(s % NS);
    // stage s has landed once at most the NS-2 later stages' loads are
    // outstanding (near the end: all); after the barrier no wave still reads
    // stage s-1, whose buffer the next issue refills
    if (s + NS - 1 <= iters) wait_vm_barrier<LPT * (NS - 2)>();
    else wait_vm_barrier<0>();
    if (s + NS - 1 < iters) issue_stage(s + NS - 1, static_cast<int>((s + NS - 1) % NS));
    if (KS > 1 && s >= cnt) continue;  // a shorter group idles through the last step

    const uint8_t* sA = glds + buf * STAGE;
    const uint8_t* sW = sA + A_BYTES;
    const float* sX = reinterpret_cast<const float*>(sW + W_BYTES);
    const uint8_t* wr[TN];
    uint4 scv[TN];
    float d[TN];
#pragma unroll
    for (int j = 0; j < TN; j++) {
      wr[j] = sW + (nl0 + 32 * j + l32) * kQ6Row;
      scv[j] = *reinterpret_cast<const uint4*>(wr[j] + 192);
      d[j] = half_to_float(*reinterpret_cast<const uint16_t*>(wr[j] + 222));
    }

    // fully unrolled: the scale byte of each sub-block and every LDS offset
    // are compile-time constants (1.07-1.10x over a two-block unroll)
#pragma unroll
    for (int b = 0; b < 8; b++) {  // 32-value block of the super-block
      const int half = b >> 2, c = b & 3;
      // weight codes of the two sub-blocks s = 2b + e, this lane's 8 values
      // 16e + 8h + i of quarter c: low nibbles ql[64half + 32(c&1) + 16e + 8h + i]
      // (high nibble when c >= 2), top bits qh[32half + 16e + 8h + i] >> 2c
      long bq[TN][2];
      float dsc[TN][2], cc[TN][1];
#pragma unroll
      for (int j = 0; j < TN; j++) {
        const uint8_t* pl = wr[j] + 64 * half + 32 * (c & 1) + 8 * h;
        const uint8_t* ph = wr[j] + 128 + 32 * half + 8 * h;
#pragma unroll
        for (int e = 0; e < 2; e++) {
          const uint2 lo8 = *reinterpret_cast<const uint2*>(pl + 16 * e);
          const uint2 hi8 = *reinterpret_cast<const uint2*>(ph + 16 * e);
          const int ls = 4 * (c >> 1), hs = 2 * c;
          // each byte becomes 4*(q6 - 32) as a signed byte: the nibble in bits
          // 2..5 (a rotate brings either half there), the two high bits in
          // bits 6..7 with the top one flipped (XOR 0xAA.. flips the top bit of
          // every 2-bit field of qh); the factor 4 comes out of dsc below
          auto code4 = [&](uint32_t l, uint32_t hq) {
            const uint32_t lo = __builtin_amdgcn_alignbit(l, l, static_cast<uint32_t>(ls + 30) & 31u) & 0x3C3C3C3Cu;
            return (((hq ^ 0xAAAAAAAAu) << (6 - hs)) & 0xC0C0C0C0u) | lo;
          };
          const uint32_t w0 = code4(lo8.x, hi8.x);
          const uint32_t w1 = code4(lo8.y, hi8.y);
          bq[j][e] = static_cast<long>((static_cast<uint64_t>(w1) << 32) | w0);
          const int s = 2 * b + e;
          const uint32_t sw = s < 4 ? scv[j].x : s < 8 ? scv[j].y : s < 12 ? scv[j].z : scv[j].w;
          // d*sc/4 (exact): the products carry the codes' factor 4
          dsc[j][e] = 0.25f * d[j] * static_cast<float>(static_cast<int8_t>(byte_of(sw, s & 3)));
        }
        // exact: d*(sc0 + sc1) has at most 20 significant bits
        cc[j][0] = -kMagic * (dsc[j][0] + dsc[j][1]);
      }
#pragma unroll
      for (int i = 0; i < TM; i++) {
        const int row = ml0 + 32 * i + l32;
        float dxv[16];
#pragma unroll
        for (int g = 0; g < 4; g++) {
          const float4 v = *reinterpret_cast<const float4*>(sX + b * BM + ml0 + 32 * i + 8 * g + 4 * h);
          dxv[4 * g] = v.x; dxv[4 * g + 1] = v.y; dxv[4 * g + 2] = v.z; dxv[4 * g + 3] = v.w;
        }
        long a[2];
#pragma unroll
        for (int e = 0; e < 2; e++) {
          const int s = 2 * b + e;
          a[e] = *reinterpret_cast<const long*>(sA + row * 256 + 16 * (s ^ (row & 15)) + 8 * h);
        }
#pragma unroll
        for (int j = 0; j < TN; j++) {
          const v16i D0 = __builtin_amdgcn_mfma_i32_32x32x16_i8(a[0], bq[j][0], magic, 0, 0, 0);
          const v16i D1 = __builtin_amdgcn_mfma_i32_32x32x16_i8(a[1], bq[j][1], magic, 0, 0, 0);
          // t = I0*dsc0 + I1*dsc1 in two fmas: p = f0*dsc0 - M*(dsc0 + dsc1)
          // = I0*dsc0 - M*dsc1 (one rounding, at the scale of M*dsc1), then
          // t = f1*dsc1 + p; acc += t*dx
#pragma unroll
          for (int r = 0; r < 16; r++) {
            const float p = __builtin_fmaf(bits_to_float(D0[r]), dsc[j][0], cc[j][0]);
            const float t = __builtin_fmaf(bits_to_float(D1[r]), dsc[j][1], p);
            acc[i][j][r] = __builtin_fmaf(t, dxv[r], acc[i][j][r]);
          }
        }
      }
    }
  }

  if constexpr (KS > 1) {
    // groups 1..KS-1 leave their partial blocks in LDS, group 0 adds them in order
    float4* red = reinterpret_cast<float4*>(lds);  // [KS-1][NW][TM*TN*4][64]
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

// OCC: waves per SIMD the register allocation must allow; KS: K-groups per
// workgroup (at most the number of super-blocks)
template <int TM, int TN, int WM, int WN, int NS, int OCC, int KS>
static void launch_q6k_lds(const uint8_t* W, const QgWorkspace& ws, int64_t M, int64_t N, int64_t K,
                           float* y, hipStream_t stream) {
  constexpr int BM = 32 * TM * WM, BN = 32 * TN * WN;
  const dim3 grid(static_cast<unsigned>((N + BN - 1) / BN), static_cast<unsigned>((M + BM - 1) / BM));
  gemm_q6k_lds_kernel<TM, TN, WM, WN, NS, OCC, KS><<<grid, dim3(64 * WM * WN * KS), 0, stream>>>(
      W, ws.q, ws.dxT, ws.Mp, M, N, K, y);
}

// ---------------------------------------------------------------- half-stage kernel
//
// One stage = half a super-block (values 128hf .. 128hf+127 of every row):
//   A  [8][BM]    16-byte activation chunks, column-major: chunk c of all BM
//                 rows, then chunk c+1.  A wave-load takes one chunk of 64
//                 rows; a lane's operand for sub-block (c, e) sits at
//                 ((2c+e)*BM + row)*16 + 8h, a per-lane base plus a constant
//   W  [BN][9]    per weight row: the half's ql bytes (4 chunks), its qh
//                 bytes (2), the scale chunk (bytes 192..207), the chunk of
//                 bytes 194..209 that ends with d, and one padding chunk (a
//                 144-byte stride spreads 16 rows over distinct bank groups)
//   DX [4][BM]    fp32 activation scales of the half's four blocks (from dxT)
// Value 128hf + l of a row takes the low (l < 64) or high nibble of ql byte
// 64hf + l%64 and bits 2(l/32), 2(l/32)+1 of qh byte 32hf + l%32; for block
// c of the half and sub-block e those are ql chunk 2(c&1)+e with nibble c/2
// and qh chunk e with shift 2c.  The arithmetic per block is the scheme
// above (codes 4*(q6 - 32), two fmas per sub-block pair and one for dx).
template <int TM, int TN, int WM, int WN, int NS, int OCC, int KS>
__global__ __launch_bounds__(64 * WM * WN * KS) __attribute__((amdgpu_waves_per_eu(OCC))) void gemm_q6k_half_kernel(
    const uint8_t* __restrict__ W, const int8_t* __restrict__ qx, const float* __restrict__ dxT,
    int64_t Mp, int64_t M, int64_t N, int64_t K, float* __restrict__ y) {
  constexpr int NW = WM * WN;  // waves per group
  constexpr int BM = 32 * TM * WM, BN = 32 * TN * WN;
  constexpr int WROW = 9;      // staged chunks per weight row
  static_assert(kRowPad % BM == 0, "BM must divide the workspace row padding");
  static_assert(NS >= 2, "a ring of at least two stages");
  constexpr int A_CH = BM * 8, W_CH = BN * WROW, X_CH = BM;
  constexpr int A_WL = (A_CH + 63) / 64, W_WL = (W_CH + 63) / 64, X_WL = (X_CH + 63) / 64;
  constexpr int A_BYTES = A_WL * 1024, W_BYTES = W_WL * 1024, X_BYTES = X_WL * 1024;
  constexpr int STAGE = A_BYTES + W_BYTES + X_BYTES;
  static_assert(KS * NS * STAGE <= 160 * 1024, "LDS budget");
  static_assert(KS == 1 || (KS - 1) * NW * TM * TN * 4096 <= KS * NS * STAGE, "reduction space");
  __shared__ __attribute__((aligned(16))) uint8_t lds[KS * NS * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave_all / NW, wave = wave_all - grp * NW;  // K-group, wave within the group
  const int h = lane >> 5, l32 = lane & 31;
  const int wm = wave / WN, wn = wave % WN;
  const int64_t m_cta = static_cast<int64_t>(blockIdx.y) * BM;
  const int64_t n_cta = static_cast<int64_t>(blockIdx.x) * BN;
  const int ml0 = 32 * TM * wm, nl0 = 32 * TN * wn;
  const int64_t nsb = K / 256;
  const int64_t wrow_bytes = nsb * kQ6Bytes;
  uint8_t* const glds = lds + grp * NS * STAGE;  // this group's ring
  // this group's super-blocks sb0 .. sb0 + cnt - 1, i.e. half-stages 0 .. 2cnt - 1
  // (half-stage s is half s & 1 of super-block sb0 + s / 2)
  const int64_t sb0 = grp * nsb / KS, cnt = (grp + 1) * nsb / KS - sb0;
  const int64_t hcnt = 2 * cnt;
  const int64_t iters = 2 * ((nsb + KS - 1) / KS);  // the longest group's count

  // Per-lane byte offsets, computed once (tail rows and columns clamped to the
  // last valid one, lanes past a region's end to offset 0); the group's waves
  // issue a region's wave-loads round robin, modulo the region's count.
  constexpr int LA = (A_WL + NW - 1) / NW, LW = (W_WL + NW - 1) / NW, LX = (X_WL + NW - 1) / NW;
  constexpr int LPT = LA + LW + LX;  // loads per thread per stage
  static_assert(LPT * (NS - 1) < 64, "vmcnt range");
  uint32_t voffA[LA], voffW[LW], dW[LW], voffX[LX];
#pragma unroll
  for (int it = 0; it < LA; it++) {
    const int q = ((wave + it * NW) % A_WL) * 64 + lane;
    const int c8 = q / BM, row = q - c8 * BM;
    const int64_t m = m_cta + row < M ? m_cta + row : M - 1;
    voffA[it] = q < A_CH ? static_cast<uint32_t>((m - m_cta) * K + 16 * c8) : 0u;
  }
#pragma unroll
  for (int it = 0; it < LW; it++) {
    const int qq = ((wave + it * NW) % W_WL) * 64 + lane, row = qq / WROW, part = qq - WROW * row;
    const int64_t n = n_cta + row < N ? n_cta + row : N - 1;
    const int off = part < 4 ? 16 * part : part < 6 ? 128 + 16 * (part - 4) : part == 6 ? 192 : part == 7 ? 194 : 0;
    voffW[it] = qq < W_CH ? static_cast<uint32_t>((n - n_cta) * wrow_bytes + off) : 0u;
    dW[it] = qq < W_CH && part < 6 ? (part < 4 ? 64u : 32u) : 0u;  // ql / qh move with the half
  }
#pragma unroll
  for (int it = 0; it < LX; it++) {
    const int qq = ((wave + it * NW) % X_WL) * 64 + lane;
    const int c = qq / (BM / 4), r4 = qq - c * (BM / 4);
    voffX[it] = qq < X_CH ? static_cast<uint32_t>((c * Mp + 4 * r4) * 4) : 0u;
  }
  auto issue_stage = [&](int64_t s, int buf) {
    const int64_t sr = s < hcnt ? s : hcnt - 1;  // past the group's range: reload its last
    const int64_t sb = sb0 + (sr >> 1);
    const int hf = static_cast<int>(sr & 1);
    uint8_t* sbase = glds + buf * STAGE;
    const void* bA = qx + m_cta * K + sb * 256 + 128 * hf;
    const void* bW = W + n_cta * wrow_bytes + sb * kQ6Bytes;
    const void* bX = dxT + (8 * sb + 4 * hf) * Mp + m_cta;
#pragma unroll
    for (int it = 0; it < LA; it++) lds_dma16_sv(bA, voffA[it], sbase + 1024 * ((wave + it * NW) % A_WL));
#pragma unroll
    for (int it = 0; it < LW; it++)
      lds_dma16_sv(bW, voffW[it] + (hf ? dW[it] : 0u), sbase + A_BYTES + 1024 * ((wave + it * NW) % W_WL));
#pragma unroll
    for (int it = 0; it < LX; it++)
      lds_dma16_sv(bX, voffX[it], sbase + A_BYTES + W_BYTES + 1024 * ((wave + it * NW) % X_WL));
  };

  v16i magic;
#pragma unroll
  for (int r = 0; r < 16; r++) magic[r] = kMagicBits;
  float acc[TM][TN][16];
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

#pragma unroll
  for (int s0 = 0; s0 < NS - 1; s0++)
    if (s0 < iters) issue_stage(s0, s0);
  for (int64_t s = 0; s < iters; s++) {
    const int buf = static_cast<int>(s % NS);
    if (s + NS - 1 <= iters) wait_vm_barrier<LPT * (NS - 2)>();
    else wait_vm_barrier<0>();
    if (s + NS - 1 < iters) issue_stage(s + NS - 1, static_cast<int>((s + NS - 1) % NS));
    if (KS > 1 && s >= hcnt) continue;  // a shorter group idles through the last steps
    const int hf = static_cast<int>(s & 1);

    const uint8_t* sA = glds + buf * STAGE;
    const uint8_t* sW = sA + A_BYTES;
    const float* sX = reinterpret_cast<const float*>(sW + W_BYTES);
    // this lane's weight bytes of the half: ql[c&1][e], qh[e] (top bit of every
    // 2-bit field flipped once here), the half's eight scales and d/4
    uint2 ql[TN][2][2], qh[TN][2], scl[TN];
    float dq[TN];
#pragma unroll
    for (int j = 0; j < TN; j++) {
      const uint8_t* wr = sW + (nl0 + 32 * j + l32) * (16 * WROW);
#pragma unroll
      for (int c1 = 0; c1 < 2; c1++)
#pragma unroll
        for (int e = 0; e < 2; e++) ql[j][c1][e] = *reinterpret_cast<const uint2*>(wr + 16 * (2 * c1 + e) + 8 * h);
#pragma unroll
      for (int e = 0; e < 2; e++) {
        const uint2 v = *reinterpret_cast<const uint2*>(wr + 16 * (4 + e) + 8 * h);
        qh[j][e] = make_uint2(v.x ^ 0xAAAAAAAAu, v.y ^ 0xAAAAAAAAu);
      }
      scl[j] = *reinterpret_cast<const uint2*>(wr + 16 * 6 + 8 * hf);
      dq[j] = 0.25f * half_to_float(*reinterpret_cast<const uint16_t*>(wr + 16 * 7 + 14));
    }
#pragma unroll
    for (int c = 0; c < 4; c++) {  // 32-value block of the half
      long bq[TN][2];
      float dsc[TN][2], cc[TN];
#pragma unroll
      for (int j = 0; j < TN; j++) {
#pragma unroll
        for (int e = 0; e < 2; e++) {
          // 4*(q6 - 32) per byte: the nibble rotated into bits 2..5, the two
          // high bits shifted into bits 6..7 (their top bit already flipped)
          auto code4 = [&](uint32_t l, uint32_t hq) {
            const uint32_t lo = __builtin_amdgcn_alignbit(l, l, (c >> 1) ? 2u : 30u) & 0x3C3C3C3Cu;
            return ((hq << (6 - 2 * c)) & 0xC0C0C0C0u) | lo;
          };
          const uint32_t w0 = code4(ql[j][c & 1][e].x, qh[j][e].x);
          const uint32_t w1 = code4(ql[j][c & 1][e].y, qh[j][e].y);
          bq[j][e] = static_cast<long>((static_cast<uint64_t>(w1) << 32) | w0);
          const int si = 2 * c + e;  // sub-block within the half
          const uint32_t sw = si < 4 ? scl[j].x : scl[j].y;
          dsc[j][e] = dq[j] * static_cast<float>(static_cast<int8_t>(byte_of(sw, si & 3)));  // d*sc/4, exact
        }
        cc[j] = -kMagic * (dsc[j][0] + dsc[j][1]);  // exact: d*(sc0 + sc1) has at most 20 significant bits
      }
#pragma unroll
      for (int i = 0; i < TM; i++) {
        const int row = ml0 + 32 * i + l32;
        float dxv[16];
#pragma unroll
        for (int g = 0; g < 4; g++) {
          const float4 v = *reinterpret_cast<const float4*>(sX + c * BM + ml0 + 32 * i + 8 * g + 4 * h);
          dxv[4 * g] = v.x; dxv[4 * g + 1] = v.y; dxv[4 * g + 2] = v.z; dxv[4 * g + 3] = v.w;
        }
        long a[2];
#pragma unroll
        for (int e = 0; e < 2; e++) a[e] = *reinterpret_cast<const long*>(sA + ((2 * c + e) * BM + row) * 16 + 8 * h);
#pragma unroll
        for (int j = 0; j < TN; j++) {
          const v16i D0 = __builtin_amdgcn_mfma_i32_32x32x16_i8(a[0], bq[j][0], magic, 0, 0, 0);
          const v16i D1 = __builtin_amdgcn_mfma_i32_32x32x16_i8(a[1], bq[j][1], magic, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 16; r++) {
            const float p = __builtin_fmaf(bits_to_float(D0[r]), dsc[j][0], cc[j]);
            const float t = __builtin_fmaf(bits_to_float(D1[r]), dsc[j][1], p);
            acc[i][j][r] = __builtin_fmaf(t, dxv[r], acc[i][j][r]);
          }
        }
      }
    }
  }

  if constexpr (KS > 1) {
    // groups 1..KS-1 leave their partial blocks in LDS, group 0 adds them in order
    float4* red = reinterpret_cast<float4*>(lds);  // [KS-1][NW][TM*TN*4][64]
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

template <int TM, int TN, int WM, int WN, int NS, int OCC, int KS>
static void launch_q6k_half(const uint8_t* W, const QgWorkspace& ws, int64_t M, int64_t N, int64_t K,
                            float* y, hipStream_t stream) {
  constexpr int BM = 32 * TM * WM, BN = 32 * TN * WN;
  const dim3 grid(static_cast<unsigned>((N + BN - 1) / BN), static_cast<unsigned>((M + BM - 1) / BM));
  gemm_q6k_half_kernel<TM, TN, WM, WN, NS, OCC, KS><<<grid, dim3(64 * WM * WN * KS), 0, stream>>>(
      W, ws.q, ws.dxT, ws.Mp, M, N, K, y);
}

// Kernel choice (measured on the workloads' shapes and their neighbours):
// 128x128 one-stage blocks of 8 waves x 2x1 tiles (one per CU) when their
// grid fills whole rounds of the chip or at least eight rounds (long-K
// prompts from 1024 rows, the LM head at 512 rows); otherwise half-stage
// 64x64 blocks of 4 waves (up to four per CU; 64x128 blocks measured within
// 2% of them or 10% slower), with the K range split between two groups of 4
// waves when there are fewer 64x64 blocks than CUs.
enum class Q6Pick { k128x128, k64x64, k64x64K2 };

inline Q6Pick pick_q6k(int64_t M, int64_t N, int64_t K) {
  constexpr int64_t kCUs = 256;
  const int64_t b128 = ((M + 127) / 128) * ((N + 127) / 128);
  if (b128 >= kCUs && (b128 % kCUs == 0 || b128 >= 8 * kCUs)) return Q6Pick::k128x128;
  if (((M + 63) / 64) * ((N + 63) / 64) >= kCUs || K < 512) return Q6Pick::k64x64;
  return Q6Pick::k64x64K2;
}

}  // namespace qg

const char* qg_gemm_q6k_kernel_name(int64_t M, int64_t N, int64_t K) {
  switch (qg::pick_q6k(M, N, K)) {
    case qg::Q6Pick::k128x128: return "gemm_q6k_lds_kernel<2, 1, 2, 4, 2, 2, 1>";
    case qg::Q6Pick::k64x64: return "gemm_q6k_half_kernel<1, 1, 2, 2, 2, 4, 1>";
    case qg::Q6Pick::k64x64K2: return "gemm_q6k_half_kernel<1, 1, 2, 2, 2, 4, 2>";
  }
  return "?";
}

hipError_t qg_launch_gemm_q6k(const uint8_t* W, const QgWorkspace& ws, int64_t M, int64_t N,
                              int64_t K, float* y, hipStream_t stream) {
  switch (qg::pick_q6k(M, N, K)) {
    case qg::Q6Pick::k128x128: qg::launch_q6k_lds<2, 1, 2, 4, 2, 2, 1>(W, ws, M, N, K, y, stream); break;
    case qg::Q6Pick::k64x64: qg::launch_q6k_half<1, 1, 2, 2, 2, 4, 1>(W, ws, M, N, K, y, stream); break;
    case qg::Q6Pick::k64x64K2: qg::launch_q6k_half<1, 1, 2, 2, 2, 4, 2>(W, ws, M, N, K, y, stream); break;
  }
  return hipGetLastError();
}
