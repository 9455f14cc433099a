// Tiled prefill GEMM for Q4_K weights on the int8 matrix cores (gfx950).
//
// The fused design of sparkinfer PR #464 ("fused Q4K/Q6K->int8 dequant ...",
// section "Summary": super-blocks decoded in registers, an int8 tensor-core
// GEMM, no wider dequantised scratch), carried to CDNA4 without that page's
// second per-row weight quantisation: the 4-bit codes go to the matrix core as
// they are and every sub-block's own scale and min are applied afterwards.
//
// Per 32-value activation block b of row m and weight row n (sub-block j of
// super-block sb):
//   I = sum_t q[n][t] * qx[m][t]                        int8 MFMA, int32
//   y[m][n] += dx[m][b] * (d*sc[n][j]) * I              scale term, fp32
//   y[m][n] -= dmin[n][sb] * sum_j m[n][j] * dS[m][b]   min term, per super-block
//
// Scale term -- two vector-ALU instructions per output element and block:
//   * Weights sit on the lane axis (column n = lane % 32 of a 32x32 tile), so
//     dsc = d*sc is one scalar per lane.  dsc has at most 17 significant bits
//     (binary16 d times a 6-bit integer), hence c = -12582912*dsc is exact in
//     fp32.  The MFMA accumulator starts at the bit pattern of 12582912.0f, so
//     its int32 result reads as the float 12582912 + I, and fma(f, dsc, c) is
//     exactly fl(I * dsc).
//   * The activation scale dx differs per output row, i.e. per accumulator
//     element: the kernels read the 16 scales of a tile's rows for each block
//     from LDS as four 16-byte broadcasts (staged block-major, [8][BM]) and
//     accumulate acc = fma(u, dx, acc).  (The DPP=true variant instead keeps
//     one row's scale per lane and accumulates with v_fmac_f32 and a DPP
//     row_newbcast operand; it issues more slowly and is not dispatched.)
// Min term -- on the matrix core: the mins m are 6-bit integers (exact in
// bfloat16) and dS = dx*S is split exactly into three bfloat16 pieces by the
// activation quantiser, so two K=16 bf16 MFMAs per tile and super-block give
// sum_j m_j * dS_j to fp32 accuracy; one FMA per element then applies -dmin.
#include <type_traits>

#include "common.h"
#include "lds_stage.h"
#include "mfma_epilogue.h"

namespace qg {

// The eight 6-bit mins of a super-block as bfloat16 integers (exact): two
// dwords m[0..3], m[4..7] of bytes -> four dwords of bf16 pairs.
__device__ __forceinline__ v8bf mins_bf16(uint32_t m_lo, uint32_t m_hi) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const uint32_t src = i < 2 ? m_lo : m_hi;
    const float f0 = static_cast<float>(byte_of(src, 2 * (i & 1)));
    const float f1 = static_cast<float>(byte_of(src, 2 * (i & 1) + 1));
    // high halves of the two floats: integers below 256 are exact in bf16
    w[i] = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, f1), __builtin_bit_cast(uint32_t, f0),
                                 0x07060302u);
  }
  return __builtin_bit_cast(v8bf, v4i{int(w[0]), int(w[1]), int(w[2]), int(w[3])});
}

// ---------------------------------------------------------------- LDS-staged kernel
//
// KS groups of WM x WN waves; the waves of a group share super-block stages in
// LDS and each owns TM x TN tiles of 32x32 outputs.  The KS groups of a
// workgroup compute the same BM x BN output block over disjoint super-block
// ranges of K (a split of the reduction for grids with few output blocks) and
// are summed through LDS at the end in group order, so the result does not
// depend on timing.  One stage (256 values of K) holds, for the BM activation
// rows and BN weight rows of the block:
//   A   [BM][256]  int8 codes; each row's sixteen 16-byte chunks are XOR-
//                  swizzled by (row % 16) so that 16 lanes reading 16 rows at
//                  the same column hit 16 different bank groups
//   W   [BN][144]  raw Q4_K blocks (the 144-byte stride already spreads 16
//                  consecutive rows over distinct bank groups)
//   DX  [BM][8]    fp32 activation block scales
//   DSP [BM][3][8] bfloat16 pieces of dS
// Stages are filled by global_load_lds_dwordx4 (global memory straight into
// LDS) in an NS-deep ring per group: while super-block sb is computed, the
// loads of the next NS-1 super-blocks are in flight; one workgroup barrier per
// stage.  Each region is a whole number of wave-loads (64 chunks of 16 bytes);
// the lanes of a region's last wave-load that fall past its end re-read the
// region's first chunk into the region's padding.  Every wave issues the same
// number of loads per stage (the extra ones of the short waves repeat one of
// the region's wave-loads, writing the same bytes to the same place), so a
// fixed vmcnt waits for exactly one stage.
// DPP: activation scales staged row-major and applied with the DPP-broadcast
// epilogue; otherwise staged block-major ([8][BM], from dxT) and read as 16
// per-element values per tile (four 16-byte broadcast reads).
// A256: activations quantised with one scale per 256-value super-block (the
// workspace then holds that scale for each of its eight 32-value blocks).  The
// eight sub-block partials of a super-block are combined in integers,
// J = sum_j sc[j] * I[j] (v_mad_i32_i24 per element and block; |J| < 2^25), and
// the fp32 epilogue runs once per super-block: acc += fl(fl(J) * d) * dx.
// SW: SwiGLU epilogue over a gate+up weight stacked as [gate (F rows); up (F
// rows)] (N = 2F).  A block computes BN/2 output columns f: its tile columns
// 0..BN/2-1 are the gate rows f and BN/2..BN-1 the up rows F + f, so the
// waves wn < WN/2 hold gate values and the waves wn + WN/2 the up values of
// the same (row, column) in the same lane and register; the latter pass them
// through LDS and the former write h = silu(gate) * up as bfloat16 [M][F].
// Q5: Q5_K blocks (176 bytes: the Q4_K header, qh[32], the nibbles); each
// lane also stages its 16 qh bytes and ors bit jb of each into its codes.
// Q8: Q8_0 blocks (eight 34-byte blocks of an fp16 d and 32 int8 codes per
// 256 values): the codes go to the matrix core as they are, dsc = d per
// 32-value block, no min term (no dS pieces staged).
// EXT: the stage ring lives in the caller's LDS buffer ext_lds (a kernel that
// runs two block shapes), the block's place is (mt_in, nt_in) and output rows
// are ldy floats apart; otherwise the body declares its ring, takes its place
// from the grid and writes rows N floats apart.
template <int TM, int TN, int WM, int WN, bool DPP, int NS, int KS, bool A256, bool SW, bool Q5 = false,
          bool Q8 = false, bool EXT = false>
__device__ __forceinline__ void q4k_lds_body(
    const uint8_t* __restrict__ W, const int8_t* __restrict__ qx, const float* __restrict__ dx,
    const float* __restrict__ dxT, int64_t Mp, const uint16_t* __restrict__ dsp, int64_t M,
    int64_t N, int64_t K, float* __restrict__ y, uint16_t* __restrict__ hout, int64_t F,
    uint8_t* ext_lds = nullptr, uint32_t mt_in = 0, uint32_t nt_in = 0, int64_t ldy = 0) {
  static_assert(!SW || (WN % 2 == 0 && !A256 && !DPP), "SwiGLU pairs waves wn and wn + WN/2");
  static_assert(!(Q5 || Q8) || (!A256 && !DPP), "Q5_K and Q8_0 run the per-32 method");
  constexpr int NW = WM * WN;  // waves per group
  constexpr int BM = 32 * TM * WM, BN = 32 * TN * WN;
  // bytes per 256 values of a weight row, and where the Q4_K / Q5_K nibbles start
  constexpr int BB = Q8 ? 8 * kQ8Bytes : Q5 ? kQ5Bytes : kQ4Bytes, BB16 = BB / 16, QS = Q5 ? 48 : 16;
  static_assert(kRowPad % BM == 0, "BM must divide the workspace row padding");
  constexpr int A_CH = BM * 256 / 16, W_CH = BN * BB16, X_CH = BM * 32 / 16, P_CH = Q8 ? 0 : BM * 48 / 16;
  // wave-loads per region and region sizes in LDS (whole wave-loads)
  constexpr int A_WL = (A_CH + 63) / 64, W_WL = (W_CH + 63) / 64, X_WL = (X_CH + 63) / 64, P_WL = (P_CH + 63) / 64;
  constexpr int A_BYTES = A_WL * 1024, W_BYTES = W_WL * 1024, X_BYTES = X_WL * 1024, P_BYTES = P_WL * 1024;
  constexpr int STAGE = A_BYTES + W_BYTES + X_BYTES + P_BYTES;
  static_assert(KS * NS * STAGE <= 160 * 1024, "LDS budget");
  static_assert(KS == 1 || (KS - 1) * NW * TM * TN * 4096 <= KS * NS * STAGE, "reduction space");
  uint8_t* lds;
  if constexpr (EXT) {
    lds = ext_lds;
  } else {
    __shared__ __attribute__((aligned(16))) uint8_t lds_ring[KS * NS * STAGE];
    lds = lds_ring;
  }

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave_all / NW, wave = wave_all - grp * NW;  // K-group, wave within the group
  const int h = lane >> 5, l32 = lane & 31;
  const int wm = wave / WN, wn = wave % WN;
  // Tile order.  Workgroups go to the eight XCDs in turn (consecutive ids,
  // x fastest), each XCD with its own L2, which fills the activation row
  // tiles and weight column tiles of the blocks it runs.  For one-tile waves
  // in 64x128 blocks (one or two K-groups) the block grid is cut into eight
  // sub-grids of gy/a row tiles by gx/(8/a) column tiles, one per XCD, with
  // the a in 1, 2, 4, 8 whose sub-grid costs its L2 the fewest bytes (an
  // activation row brings 21 bytes per 16 values of K: codes, scale, dS
  // pieces; a weight row 9); a = 1 also where no cut is even: XCD k takes
  // the k-th eighth of the tiles, row tiles fastest.  Measured: 512x4096->
  // 24576 (a = 1) L2 fills 336 -> 104 MB per launch, the same time;
  // 512x9728->2560 (a = 2, two K-groups) 82.5 -> 55.9 MB, the same time;
  // 4096x9728->2560 (a = 4) 323 -> 316 us.  The 2x2-tile blocks (2-7%) and
  // the 32x64 blocks with four K-groups (4-6%) measured slower cut this way
  // and keep the grid order.  Only the block's place changes, not its sums.
  uint32_t mt = EXT ? mt_in : blockIdx.y, nt = EXT ? nt_in : blockIdx.x;
  if constexpr (TM == 1 && TN == 1 && KS <= 2 && !SW && !Q5 && !Q8 && !A256 && !EXT) {
    const uint32_t gx = gridDim.x, gy = gridDim.y, G = gx * gy;
    if (G % 8 == 0) {
      const uint32_t L = blockIdx.y * gx + blockIdx.x;
      const uint32_t x = L % 8, i = L / 8;  // the XCD, and the block's place in its sequence
      uint32_t a = 1;
      float best = static_cast<float>(gy) * (BM * 21.0f) + static_cast<float>((gx + 7) / 8) * (BN * 9.0f);
      for (uint32_t aa = 2; aa <= 8; aa *= 2) {
        if (gy % aa != 0 || gx % (8 / aa) != 0) continue;
        const float c = static_cast<float>(gy / aa) * (BM * 21.0f) + static_cast<float>(gx / (8 / aa)) * (BN * 9.0f);
        if (c < best) {
          best = c;
          a = aa;
        }
      }
      if (a == 1) {
        const uint32_t Lp = x * (G / 8) + i;
        mt = Lp % gy;
        nt = Lp / gy;
      } else {  // sub-grid (x / b, x % b) of sy x sx tiles, row tiles fastest
        const uint32_t b = 8 / a, sy = gy / a, sx = gx / b;
        mt = (x / b) * sy + i % sy;
        nt = (x % b) * sx + i / sy;
      }
    }
  }
  const int64_t m_cta = static_cast<int64_t>(mt) * BM;
  const int64_t n_cta = static_cast<int64_t>(nt) * (SW ? BN / 2 : BN);  // first weight row / column
  const int ml0 = 32 * TM * wm, nl0 = 32 * TN * wn;
  const int64_t nsb = K / 256, nb = K / 32;
  const int64_t wrow_bytes = nsb * BB;
  const int drow = dpp_scale_row(lane);
  uint8_t* const glds = lds + grp * NS * STAGE;  // this group's ring
  // this group's super-blocks: sb0 .. sb0 + cnt - 1 (the launcher keeps KS <= nsb)
  const int64_t sb0 = grp * nsb / KS, cnt = (grp + 1) * nsb / KS - sb0;
  const int64_t iters = (nsb + KS - 1) / KS;  // the longest group's count

  // Stage loads, region by region (A, W, DX, DSP).  A region of R_WL wave-
  // loads is issued by the group's waves round robin: wave w issues wave-loads
  // w, w+NW, ... (taken modulo R_WL, so that every wave issues the same count
  // per region).  Each load reads base(region, sb) + voff: the base is a
  // wave-uniform pointer advanced per super-block (SGPRs); voff is this lane's
  // byte offset, computed once (tail rows and columns clamped to the last valid
  // one, lanes past the region's end to offset 0).
  constexpr int LA = (A_WL + NW - 1) / NW, LW = (W_WL + NW - 1) / NW;
  constexpr int LX = (X_WL + NW - 1) / NW, LP = (P_WL + NW - 1) / NW;
  constexpr int P_WLM = P_WL > 0 ? P_WL : 1;  // modulus for the (empty, for Q8_0) dS-piece loops
  uint32_t voff[LA + LW + LX + LP];
#pragma unroll
  for (int it = 0; it < LA; it++) {
    const int q = ((wave + it * NW) % A_WL) * 64 + lane;
    const int row = q >> 4, c16 = (q & 15) ^ (row & 15);
    const int64_t m = m_cta + row < M ? m_cta + row : M - 1;
    voff[it] = q < A_CH ? static_cast<uint32_t>((m - m_cta) * K + 16 * c16) : 0u;
  }
#pragma unroll
  for (int it = 0; it < LW; it++) {
    const int qq = ((wave + it * NW) % W_WL) * 64 + lane, row = qq / BB16, part = qq - BB16 * row;
    int64_t n;
    if constexpr (SW) {  // tile column row -> gate row f or up row F + f
      const int o = row % (BN / 2);
      const int64_t f = n_cta + o < F ? n_cta + o : F - 1;
      n = (row >= BN / 2 ? F : 0) + f;
    } else {
      n = n_cta + row < N ? n_cta + row : N - 1;
    }
    voff[LA + it] = qq < W_CH ? static_cast<uint32_t>((n - n_cta) * wrow_bytes + 16 * part) : 0u;
  }
#pragma unroll
  for (int it = 0; it < LX; it++) {
    const int qq = ((wave + it * NW) % X_WL) * 64 + lane;
    uint32_t v;
    if (DPP) {
      const int row = qq >> 1, hf = qq & 1;
      v = static_cast<uint32_t>((row * nb + 4 * hf) * 4);
    } else {
      const int jb = qq / (BM / 4), r4 = qq - jb * (BM / 4);
      v = static_cast<uint32_t>((jb * Mp + 4 * r4) * 4);
    }
    voff[LA + LW + it] = qq < X_CH ? v : 0u;
  }
#pragma unroll
  for (int it = 0; it < LP; it++) {
    const int qq = ((wave + it * NW) % P_WLM) * 64 + lane, row = qq / 3, piece = qq - 3 * row;
    voff[LA + LW + LX + it] = qq < P_CH ? static_cast<uint32_t>(row * nsb * 48 + 16 * piece) : 0u;
  }
  constexpr int LPT = LA + LW + LX + LP;  // loads per thread per stage
  static_assert(LPT * (NS - 1) < 64, "vmcnt range");

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
    issue_region(W + n_cta * wrow_bytes + sb * BB, LA, LW, W_WL, A_BYTES, sbase);
    issue_region(DPP ? static_cast<const void*>(dx + m_cta * nb + 8 * sb)
                     : static_cast<const void*>(dxT + 8 * sb * Mp + m_cta),
                 LA + LW, LX, X_WL, A_BYTES + W_BYTES, sbase);
    issue_region(dsp + (m_cta * nsb + sb) * 24, LA + LW + LX, LP, P_WL, A_BYTES + W_BYTES + X_BYTES, sbase);
  };

  v16i magic;
#pragma unroll
  for (int r = 0; r < 16; r++) magic[r] = kMagicBits;
  static_assert(!(A256 && DPP), "the per-256 epilogue reads row scales from LDS");
  float acc[TM][TN][16];
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;
  v16i acc_i[TM][TN];  // A256: the super-block's integer sum J

#pragma unroll
  for (int s0 = 0; s0 < NS - 1; s0++)
    if (s0 < iters) issue_stage(s0, s0);
  for (int64_t s = 0; s < iters; s++) {
    const int buf = static_cast<int>(s % NS);
    // This wave's loads of stage s have landed once at most the loads of the
    // NS-2 later stages are outstanding (near the end fewer are: wait for
    // all); after the barrier every wave's have, and no wave still reads
    // stage s-1, whose buffer the next issue refills.
    if (s + NS - 1 <= iters) wait_vm_barrier<LPT * (NS - 2)>();
    else wait_vm_barrier<0>();
    if (s + NS - 1 < iters) issue_stage(s + NS - 1, static_cast<int>((s + NS - 1) % NS));
    if (KS > 1 && s >= cnt) continue;  // a shorter group idles through the last step

    const uint8_t* sA = glds + buf * STAGE;
    const uint8_t* sW = sA + A_BYTES;
    const float* sX = reinterpret_cast<const float*>(sW + W_BYTES);
    const uint8_t* sP = sW + W_BYTES + X_BYTES;

    float d[TN], dmin[TN];
    Q4Scales sc[TN];
    const uint8_t* wr[TN];
    uint4 qh5[TN];  // Q5: the lane's 16 qh bytes of each weight column
#pragma unroll
    for (int j = 0; j < TN; j++) {
      wr[j] = sW + (nl0 + 32 * j + l32) * BB;
      if constexpr (Q8) continue;  // no super-block header
      if constexpr (Q5) qh5[j] = *reinterpret_cast<const uint4*>(wr[j] + 16 + 16 * h);
      const uint4 hdr = *reinterpret_cast<const uint4*>(wr[j]);
      d[j] = half_to_float(hdr.x & 0xFFFFu);
      dmin[j] = half_to_float(hdr.x >> 16);
      sc[j] = unpack_q4_scales(hdr.y, hdr.z, hdr.w);
      // keep the masked scale bytes as values, so that each scale converts
      // with one v_cvt_f32_ubyteN instead of a field extract and a convert
      asm volatile("" : "+v"(sc[j].sc_lo), "+v"(sc[j].sc_hi));
    }
    float dxr[TM][8];
    if (DPP) {
#pragma unroll
      for (int i = 0; i < TM; i++) {
        const float4* p = reinterpret_cast<const float4*>(sX + (ml0 + 32 * i + drow) * 8);
        const float4 v0 = p[0], v1 = p[1];
        dxr[i][0] = v0.x; dxr[i][1] = v0.y; dxr[i][2] = v0.z; dxr[i][3] = v0.w;
        dxr[i][4] = v1.x; dxr[i][5] = v1.y; dxr[i][6] = v1.z; dxr[i][7] = v1.w;
      }
    }

#pragma unroll
    for (int c = 0; c < 4; c++) {
      uint4 wraw[TN];
#pragma unroll
      for (int j = 0; j < TN; j++)
        if constexpr (!Q8) wraw[j] = *reinterpret_cast<const uint4*>(wr[j] + QS + 32 * c + 16 * h);
      v4i a[TM][2];
#pragma unroll
      for (int i = 0; i < TM; i++) {
        const int row = ml0 + 32 * i + l32;
#pragma unroll
        for (int e = 0; e < 2; e++) {
          const int pos = (2 * (2 * c + e) + h) ^ (row & 15);
          a[i][e] = *reinterpret_cast<const v4i*>(sA + row * 256 + 16 * pos);
        }
      }
#pragma unroll
      for (int e = 0; e < 2; e++) {
        const int jb = 2 * c + e;
        v4i b[TN];
        float dsc[TN], cc[TN];
#pragma unroll
        for (int j = 0; j < TN; j++) {
          if constexpr (Q8) {
            b[j] = q8_codes(wr[j], jb, h);
            dsc[j] = q8_scale(wr[j], jb);
          } else {
            b[j] = q4_codes(wraw[j], e);
            if constexpr (Q5) b[j] |= q5_high(qh5[j], jb);
            dsc[j] = d[j] * static_cast<float>(sub_byte(sc[j].sc_lo, sc[j].sc_hi, jb));
          }
          cc[j] = -kMagic * dsc[j];
        }
        if constexpr (A256) {
          // I from a zero-started accumulator; J += sc * I in integers
#pragma unroll
          for (int i = 0; i < TM; i++)
#pragma unroll
            for (int j = 0; j < TN; j++) {
              const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i][e], b[j], v16i{}, 0, 0, 0);
              const int scj = static_cast<int>(sub_byte(sc[j].sc_lo, sc[j].sc_hi, jb));
              if (jb == 0) {
#pragma unroll
                for (int r = 0; r < 16; r++) acc_i[i][j][r] = __mul24(D[r], scj);
              } else {
#pragma unroll
                for (int r = 0; r < 16; r++) acc_i[i][j][r] = __mul24(D[r], scj) + acc_i[i][j][r];
              }
            }
          continue;
        }
        v16i D[TM][TN];
        // Waves of several tiles run two to a SIMD: a raised priority while
        // they issue their MFMAs keeps the matrix core from waiting behind
        // the other wave's epilogue (2x2 tiles at 2048x4096->24576: 1.02x on
        // the benchmark's weights, 1.07x on random bytes, which run the clock
        // lower; one-tile waves, four to a SIMD, measured 2-5% slower with it,
        // and the Q6_K kernel's 2x1-tile waves 12% slower)
        if constexpr (TM * TN > 1) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
          for (int j = 0; j < TN; j++)
            D[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i][e], b[j], magic, 0, 0, 0);
        if constexpr (TM * TN > 1) __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int i = 0; i < TM; i++) {
          if (DPP) {
            // dxr[i][jb] with a run-time jb when the loop is not unrolled
            float xs = dxr[i][0];
#pragma unroll
            for (int t = 1; t < 8; t++) xs = jb == t ? dxr[i][t] : xs;
#pragma unroll
            for (int j = 0; j < TN; j++) epilogue_scale(acc[i][j], D[i][j], dsc[j], cc[j], xs);
          } else {
            float dxv[16];
#pragma unroll
            for (int g = 0; g < 4; g++) {
              const float4 v = *reinterpret_cast<const float4*>(sX + jb * BM + ml0 + 32 * i + 8 * g + 4 * h);
              dxv[4 * g] = v.x; dxv[4 * g + 1] = v.y; dxv[4 * g + 2] = v.z; dxv[4 * g + 3] = v.w;
            }
#pragma unroll
            for (int j = 0; j < TN; j++)
#pragma unroll
              for (int r = 0; r < 16; r++) {
                const float u = __builtin_fmaf(bits_to_float(D[i][j][r]), dsc[j], cc[j]);  // fl(I*dsc)
                acc[i][j][r] = __builtin_fmaf(u, dxv[r], acc[i][j][r]);
              }
          }
        }
      }
    }
    if constexpr (A256) {
      // once per super-block: acc += fl(fl(J) * d) * dx, dx the rows' super-block
      // scale (the first of the stage's eight equal block scales)
#pragma unroll
      for (int i = 0; i < TM; i++) {
        float dxv[16];
#pragma unroll
        for (int g = 0; g < 4; g++) {
          const float4 v = *reinterpret_cast<const float4*>(sX + ml0 + 32 * i + 8 * g + 4 * h);
          dxv[4 * g] = v.x; dxv[4 * g + 1] = v.y; dxv[4 * g + 2] = v.z; dxv[4 * g + 3] = v.w;
        }
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
          for (int r = 0; r < 16; r++)
            acc[i][j][r] = __builtin_fmaf(static_cast<float>(acc_i[i][j][r]) * d[j], dxv[r], acc[i][j][r]);
      }
    }
    // min term of the super-block on the matrix core (Q8_0 has none)
    if constexpr (Q8) continue;
    v8bf mb[TN];
#pragma unroll
    for (int j = 0; j < TN; j++) mb[j] = mins_bf16(sc[j].m_lo, sc[j].m_hi);
#pragma unroll
    for (int i = 0; i < TM; i++) {
      const uint8_t* prow = sP + (ml0 + 32 * i + l32) * 48;
      const v8bf p01 = *reinterpret_cast<const v8bf*>(prow + 16 * h);  // piece 0 (h=0) / 1 (h=1)
      v8bf p2z = *reinterpret_cast<const v8bf*>(prow + 32);           // piece 2 (h=0) / zero (h=1)
      if (h) p2z = __builtin_bit_cast(v8bf, v4i{0, 0, 0, 0});
#pragma unroll
      for (int j = 0; j < TN; j++) {
        v16f T = {};
        T = __builtin_amdgcn_mfma_f32_32x32x16_bf16(p01, mb[j], T, 0, 0, 0);
        T = __builtin_amdgcn_mfma_f32_32x32x16_bf16(p2z, mb[j], T, 0, 0, 0);
        const float nd = -dmin[j];
#pragma unroll
        for (int r = 0; r < 16; r++) acc[i][j][r] = __builtin_fmaf(T[r], nd, acc[i][j][r]);
      }
    }
  }

  if constexpr (KS > 1) {
    // Sum the groups' partial blocks in group order: groups 1..KS-1 leave
    // theirs in LDS (the stage ring is free once every wave has passed this
    // barrier), group 0 adds them to its own and stores.
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
    if constexpr (!SW) {
      if (grp > 0) return;
    }
    if (grp == 0) {
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
  }

  if constexpr (SW) {
    // Wave pair (wm, wn) / (wm, wn + WN/2) holds the gate and the up values of
    // the same rows and output columns in the same lanes and registers.  Each
    // wave of the pair takes half of the SwiGLU work: the gate wave registers
    // 0..7, the up wave 8..15, after swapping the other halves through LDS.
    // The bf16 results go to an h tile [BM][BN/2] in LDS and leave it as
    // 16-byte row segments.
    constexpr int HW = WN / 2, BO = BN / 2;
    constexpr int XOFF = (KS - 1) * NW * TM * TN * 4096;  // past the K-group reduction space
    constexpr int HOFF = XOFF + HW * WM * TM * TN * 4096;
    static_assert(HOFF + BM * BO * 2 <= KS * NS * STAGE, "exchange space");
    float4* xch = reinterpret_cast<float4*>(lds + XOFF);  // [pair][TM][TN][side][2][64]
    uint16_t* ht = reinterpret_cast<uint16_t*>(lds + HOFF);
    const bool up_wave = wn >= HW;
    const int pair = wm * HW + (up_wave ? wn - HW : wn);
    // side 0: the gate wave's registers 8..15; side 1: the up wave's registers 0..7
    auto slot = [&](int i, int j, int side, int q) {
      return ((((pair * TM + i) * TN + j) * 2 + side) * 2 + q) * 64 + lane;
    };
    // The register halves are compile-time constants in each branch (a
    // run-time register index would put the accumulators in private memory).
    auto give = [&](auto up) {  // this wave's half that the partner finishes
      constexpr int r0 = decltype(up)::value ? 0 : 8;
#pragma unroll
      for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
          for (int q = 0; q < 2; q++)
            xch[slot(i, j, decltype(up)::value ? 1 : 0, q)] =
                make_float4(acc[i][j][r0 + 4 * q], acc[i][j][r0 + 4 * q + 1], acc[i][j][r0 + 4 * q + 2],
                            acc[i][j][r0 + 4 * q + 3]);
    };
    auto finish = [&](auto up) {  // the half this wave finishes, with the partner's values
      constexpr bool UP = decltype(up)::value;
      constexpr int r0 = UP ? 8 : 0;
      const int col0 = (UP ? nl0 - BO : nl0) + l32;
#pragma unroll
      for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
          for (int q = 0; q < 2; q++) {
            const float4 o4 = xch[slot(i, j, UP ? 0 : 1, q)];
            const float o[4] = {o4.x, o4.y, o4.z, o4.w};
#pragma unroll
            for (int e = 0; e < 4; e++) {
              const float a = acc[i][j][r0 + 4 * q + e];
              ht[(ml0 + 32 * i + acc_row(r0 + 4 * q + e, h)) * BO + col0 + 32 * j] =
                  UP ? swiglu_bf16(o[e], a) : swiglu_bf16(a, o[e]);
            }
          }
    };
    using kGate = std::integral_constant<bool, false>;
    using kUp = std::integral_constant<bool, true>;
    if constexpr (KS == 1) __syncthreads();  // no wave reads the stage ring any more
    if (grp == 0) {
      if (up_wave) give(kUp{});
      else give(kGate{});
    }
    __syncthreads();
    if (grp == 0) {
      if (up_wave) finish(kUp{});
      else finish(kGate{});
    }
    __syncthreads();
    constexpr int CPR = BO / 8;  // 16-byte chunks per h row of the block
    for (int c = tid; c < BM * CPR; c += 64 * NW * KS) {
      const int row = c / CPR, c8 = c - row * CPR;
      const int64_t m = m_cta + row, f = n_cta + 8 * c8;
      if (m >= M || f >= F) continue;
      const v4i v = *reinterpret_cast<const v4i*>(ht + row * BO + 8 * c8);
      uint16_t* dst = hout + m * F + f;
      if (F % 8 == 0) {  // then f + 8 <= F and dst is 16-byte aligned
        __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(dst));
      } else {
        const uint16_t* src = ht + row * BO + 8 * c8;
        for (int e = 0; e < 8 && f + e < F; e++) dst[e] = src[e];
      }
    }
    return;
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
        if (m < M) {
          float* const p = y + m * (EXT ? ldy : N) + n;
          if constexpr (TM == 1 && TN == 1 && KS == 1 && !Q5 && !Q8 && !A256) store_out_dev(p, acc[i][j][r]);
          else store_out(p, acc[i][j][r]);
        }
      }
  }
}

template <int TM, int TN, int WM, int WN, bool DPP, int NS, int OCC, int KS, bool A256 = false>
__global__ __launch_bounds__(64 * WM * WN * KS) __attribute__((amdgpu_waves_per_eu(OCC))) void gemm_q4k_lds_kernel(
    const uint8_t* __restrict__ W, const int8_t* __restrict__ qx, const float* __restrict__ dx,
    const float* __restrict__ dxT, int64_t Mp, const uint16_t* __restrict__ dsp, int64_t M,
    int64_t N, int64_t K, float* __restrict__ y) {
  q4k_lds_body<TM, TN, WM, WN, DPP, NS, KS, A256, false>(W, qx, dx, dxT, Mp, dsp, M, N, K, y, nullptr, 0);
}

// The same kernel over Q5_K weights.
template <int TM, int TN, int WM, int WN, int NS, int OCC, int KS>
__global__ __launch_bounds__(64 * WM * WN * KS) __attribute__((amdgpu_waves_per_eu(OCC))) void gemm_q5k_lds_kernel(
    const uint8_t* __restrict__ W, const int8_t* __restrict__ qx, const float* __restrict__ dxT,
    int64_t Mp, const uint16_t* __restrict__ dsp, int64_t M, int64_t N, int64_t K, float* __restrict__ y) {
  q4k_lds_body<TM, TN, WM, WN, false, NS, KS, false, false, true>(W, qx, nullptr, dxT, Mp, dsp, M, N, K, y,
                                                                  nullptr, 0);
}

// The same kernel over Q8_0 weights.
template <int TM, int TN, int WM, int WN, int NS, int OCC, int KS>
__global__ __launch_bounds__(64 * WM * WN * KS) __attribute__((amdgpu_waves_per_eu(OCC))) void gemm_q80_lds_kernel(
    const uint8_t* __restrict__ W, const int8_t* __restrict__ qx, const float* __restrict__ dxT,
    int64_t Mp, int64_t M, int64_t N, int64_t K, float* __restrict__ y) {
  q4k_lds_body<TM, TN, WM, WN, false, NS, KS, false, false, false, true>(W, qx, nullptr, dxT, Mp, nullptr, M, N,
                                                                         K, y, nullptr, 0);
}

// The same kernel with the SwiGLU epilogue: W holds 2F rows (gate, then up),
// the output is h [M][F] in bfloat16.
template <int TM, int TN, int WM, int WN, int NS, int OCC, int KS>
__global__ __launch_bounds__(64 * WM * WN * KS) __attribute__((amdgpu_waves_per_eu(OCC))) void gemm_q4k_swiglu_kernel(
    const uint8_t* __restrict__ W, const int8_t* __restrict__ qx, const float* __restrict__ dxT,
    int64_t Mp, const uint16_t* __restrict__ dsp, int64_t M, int64_t F, int64_t K,
    uint16_t* __restrict__ h) {
  q4k_lds_body<TM, TN, WM, WN, false, NS, KS, false, true>(W, qx, nullptr, dxT, Mp, dsp, M, 2 * F, K, nullptr,
                                                           h, F);
}

// ... over Q5_K weights
template <int TM, int TN, int WM, int WN, int NS, int OCC, int KS>
__global__ __launch_bounds__(64 * WM * WN * KS) __attribute__((amdgpu_waves_per_eu(OCC))) void gemm_q5k_swiglu_kernel(
    const uint8_t* __restrict__ W, const int8_t* __restrict__ qx, const float* __restrict__ dxT,
    int64_t Mp, const uint16_t* __restrict__ dsp, int64_t M, int64_t F, int64_t K,
    uint16_t* __restrict__ h) {
  q4k_lds_body<TM, TN, WM, WN, false, NS, KS, false, true, true>(W, qx, nullptr, dxT, Mp, dsp, M, 2 * F, K,
                                                                 nullptr, h, F);
}

// ... over Q8_0 weights
template <int TM, int TN, int WM, int WN, int NS, int OCC, int KS>
__global__ __launch_bounds__(64 * WM * WN * KS) __attribute__((amdgpu_waves_per_eu(OCC))) void gemm_q80_swiglu_kernel(
    const uint8_t* __restrict__ W, const int8_t* __restrict__ qx, const float* __restrict__ dxT,
    int64_t Mp, int64_t M, int64_t F, int64_t K, uint16_t* __restrict__ h) {
  q4k_lds_body<TM, TN, WM, WN, false, NS, KS, false, true, false, true>(W, qx, nullptr, dxT, Mp, nullptr, M, 2 * F,
                                                                        K, nullptr, h, F);
}

// ---------------------------------------------------------------- small-grid kernel
//
// For problems whose output has too few 128x256 tiles to fill the chip (one
// prompt ubatch through a small model's projections): one 32x32 output tile
// per wave, and the SK waves of a workgroup split the K range of the same
// tile between them.  Each wave loads its operands straight from global
// memory (L2-resident) a whole super-block ahead: 8 x 16 bytes of activation
// codes, 4 x 16 bytes of packed nibbles plus the 16-byte header, and 2 x 16
// bytes of dS pieces.  The activation scales of its 32 rows go through a
// wave-private LDS slice ([8][32] per super-block) and are read as 16-byte
// broadcasts.  The partial tiles are summed through LDS in ascending wave
// order, so the result does not depend on timing.
// RN: accumulator elements per lane that hold output rows.  With at most 8
// rows (decode-sized batches) only elements 0..3 of a lane do (rows 4h + r),
// so the epilogue, the min term and the activation loads skip the other
// rows (RN = 4; measured 1.1-1.4x on the decode shapes' grids).
struct SmallStage {
  v4i a[8];
  uint4 w[4], hdr, qh;  // qh: Q5_K only
  v4i p01, p2;
  float4 xs;
};

template <int SK, bool Q5, int RN>
__device__ __forceinline__ void q4k_small_body(
    const uint8_t* __restrict__ W, const int8_t* __restrict__ qx, const float* __restrict__ dxT,
    int64_t Mp, const uint16_t* __restrict__ dsp, int64_t M, int64_t N, int64_t K,
    float* __restrict__ y) {
  constexpr int BB = Q5 ? kQ5Bytes : kQ4Bytes, QS = Q5 ? 48 : 16;
  __shared__ __attribute__((aligned(16))) float s_x[SK][2][8 * 32];
  __shared__ __attribute__((aligned(16))) float4 s_red[SK > 1 ? SK : 1][4][64];

  const int lane = threadIdx.x & 63, kk = threadIdx.x >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * 32;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 32;
  const int64_t nsb = K / 256;
  const int64_t sb_begin = kk * nsb / SK, sb_end = (kk + 1) * nsb / SK;
  static_assert(RN == 4 || RN == 16, "rows per lane");
  int64_t m = m0 + l32, n = n0 + l32;
  m = m < M ? m : M - 1;
  n = n < N ? n : N - 1;
  const bool arow_used = RN == 16 || l32 < 8;  // activation rows that reach an output row
  const int8_t* arow = qx + m * K + 16 * h;
  const uint8_t* wrow = W + n * nsb * BB;
  const uint16_t* prow = dsp + (m0 + l32) * nsb * 24;  // rows up to the padding (m0 + 31 < Mp)

  auto load = [&](int64_t sb, SmallStage& st) {
#pragma unroll
    for (int b = 0; b < 8; b++)
      st.a[b] = arow_used ? *reinterpret_cast<const v4i*>(arow + 256 * sb + 32 * b) : v4i{0, 0, 0, 0};
    const uint8_t* blk = wrow + sb * BB;
    st.hdr = *reinterpret_cast<const uint4*>(blk);
#pragma unroll
    for (int c = 0; c < 4; c++) st.w[c] = *reinterpret_cast<const uint4*>(blk + QS + 32 * c + 16 * h);
    if constexpr (Q5) st.qh = *reinterpret_cast<const uint4*>(blk + 16 + 16 * h);
    st.p01 = *reinterpret_cast<const v4i*>(prow + sb * 24 + 8 * h);
    st.p2 = *reinterpret_cast<const v4i*>(prow + sb * 24 + 16);
    // activation scales of the 32 rows, 8 blocks: lane -> (block lane/8, rows 4*(lane%8)..+3)
    st.xs = *reinterpret_cast<const float4*>(dxT + (8 * sb + (lane >> 3)) * Mp + m0 + 4 * (lane & 7));
  };

  v16i magic;
#pragma unroll
  for (int r = 0; r < 16; r++) magic[r] = kMagicBits;
  float acc[16];
#pragma unroll
  for (int r = 0; r < 16; r++) acc[r] = 0.0f;

  SmallStage cur, nxt;
  if (sb_begin < sb_end) load(sb_begin, cur);
  for (int64_t sb = sb_begin; sb < sb_end; sb++) {
    if (sb + 1 < sb_end) load(sb + 1, nxt);
    float* sx = s_x[kk][sb & 1];
    *reinterpret_cast<float4*>(sx + 4 * lane) = cur.xs;  // [8][32]: block lane/8, rows 4*(lane%8)
    const float d = half_to_float(cur.hdr.x & 0xFFFFu), dmin = half_to_float(cur.hdr.x >> 16);
    const Q4Scales sc = unpack_q4_scales(cur.hdr.y, cur.hdr.z, cur.hdr.w);
#pragma unroll
    for (int jb = 0; jb < 8; jb++) {
      v4i bq = q4_codes(cur.w[jb >> 1], jb & 1);
      if constexpr (Q5) bq |= q5_high(cur.qh, jb);
      const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(cur.a[jb], bq, magic, 0, 0, 0);
      const float dsc = d * static_cast<float>(sub_byte(sc.sc_lo, sc.sc_hi, jb));
      const float cc = -kMagic * dsc;
      float dxv[16];
#pragma unroll
      for (int g = 0; g < 4; g++) {
        const float4 v = *reinterpret_cast<const float4*>(sx + jb * 32 + 8 * g + 4 * h);
        dxv[4 * g] = v.x; dxv[4 * g + 1] = v.y; dxv[4 * g + 2] = v.z; dxv[4 * g + 3] = v.w;
      }
#pragma unroll
      for (int r = 0; r < RN; r++) {
        const float u = __builtin_fmaf(bits_to_float(D[r]), dsc, cc);  // fl(I*dsc)
        acc[r] = __builtin_fmaf(u, dxv[r], acc[r]);
      }
    }
    {  // min term of the super-block
      const v8bf mb = mins_bf16(sc.m_lo, sc.m_hi);
      const v8bf p01 = __builtin_bit_cast(v8bf, cur.p01);
      const v8bf p2z = __builtin_bit_cast(v8bf, h ? v4i{0, 0, 0, 0} : cur.p2);
      v16f T = {};
      T = __builtin_amdgcn_mfma_f32_32x32x16_bf16(p01, mb, T, 0, 0, 0);
      T = __builtin_amdgcn_mfma_f32_32x32x16_bf16(p2z, mb, T, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < RN; r++) acc[r] = __builtin_fmaf(T[r], -dmin, acc[r]);
    }
    if (sb + 1 < sb_end) cur = nxt;
  }

  const int64_t nn = n0 + l32;
  if constexpr (SK > 1) {
#pragma unroll
    for (int g = 0; g < RN / 4; g++)
      s_red[kk][g][lane] = make_float4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
    __syncthreads();
    for (int g = kk; g < RN / 4; g += SK) {
      float4 s4 = s_red[0][g][lane];
      for (int w = 1; w < SK; w++) {
        const float4 v = s_red[w][g][lane];
        s4.x += v.x; s4.y += v.y; s4.z += v.z; s4.w += v.w;
      }
      const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
      if (nn < N) {
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const int64_t mm = m0 + acc_row(4 * g + q, h);
          if (mm < M) store_out(y + mm * N + nn, sv[q]);
        }
      }
    }
  } else {
    if (nn < N) {
#pragma unroll
      for (int r = 0; r < RN; r++) {
        const int64_t mm = m0 + acc_row(r, h);
        if (mm < M) store_out(y + mm * N + nn, acc[r]);
      }
    }
  }
}

template <int TM, int TN, int WM, int WN, int NS, int OCC, int KS, int FMT = QG_Q4_K>
static void launch_swiglu(const uint8_t* W, const QgWorkspace& ws, int64_t M, int64_t F, int64_t K,
                          uint16_t* h, hipStream_t stream) {
  constexpr int BM = 32 * TM * WM, BO = 16 * TN * WN;  // output columns per block: half the weight rows
  const dim3 grid(static_cast<unsigned>((F + BO - 1) / BO), static_cast<unsigned>((M + BM - 1) / BM));
  const dim3 block(64 * WM * WN * KS);
  if constexpr (FMT == QG_Q5_K)
    gemm_q5k_swiglu_kernel<TM, TN, WM, WN, NS, OCC, KS><<<grid, block, 0, stream>>>(W, ws.q, ws.dxT, ws.Mp, ws.dsp,
                                                                                 M, F, K, h);
  else if constexpr (FMT == QG_Q8_0)
    gemm_q80_swiglu_kernel<TM, TN, WM, WN, NS, OCC, KS><<<grid, block, 0, stream>>>(W, ws.q, ws.dxT, ws.Mp, M, F,
                                                                                 K, h);
  else
    gemm_q4k_swiglu_kernel<TM, TN, WM, WN, NS, OCC, KS><<<grid, block, 0, stream>>>(W, ws.q, ws.dxT, ws.Mp, ws.dsp,
                                                                                 M, F, K, h);
}

template <int SK, int RN>
__global__ __launch_bounds__(64 * SK) void gemm_q4k_small_kernel(
    const uint8_t* __restrict__ W, const int8_t* __restrict__ qx, const float* __restrict__ dxT,
    int64_t Mp, const uint16_t* __restrict__ dsp, int64_t M, int64_t N, int64_t K,
    float* __restrict__ y) {
  q4k_small_body<SK, false, RN>(W, qx, dxT, Mp, dsp, M, N, K, y);
}

template <int SK, int RN>
__global__ __launch_bounds__(64 * SK) void gemm_q5k_small_kernel(
    const uint8_t* __restrict__ W, const int8_t* __restrict__ qx, const float* __restrict__ dxT,
    int64_t Mp, const uint16_t* __restrict__ dsp, int64_t M, int64_t N, int64_t K,
    float* __restrict__ y) {
  q4k_small_body<SK, true, RN>(W, qx, dxT, Mp, dsp, M, N, K, y);
}

template <int SK, bool Q5 = false>
static void launch_small(const uint8_t* W, const QgWorkspace& ws, int64_t M, int64_t N, int64_t K,
                         float* y, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((N + 31) / 32), static_cast<unsigned>((M + 31) / 32));
  if constexpr (Q5) {
    if (M <= 8)
      gemm_q5k_small_kernel<SK, 4><<<grid, dim3(64 * SK), 0, stream>>>(W, ws.q, ws.dxT, ws.Mp, ws.dsp, M, N, K, y);
    else
      gemm_q5k_small_kernel<SK, 16><<<grid, dim3(64 * SK), 0, stream>>>(W, ws.q, ws.dxT, ws.Mp, ws.dsp, M, N, K, y);
  } else {
    if (M <= 8)
      gemm_q4k_small_kernel<SK, 4><<<grid, dim3(64 * SK), 0, stream>>>(W, ws.q, ws.dxT, ws.Mp, ws.dsp, M, N, K, y);
    else
      gemm_q4k_small_kernel<SK, 16><<<grid, dim3(64 * SK), 0, stream>>>(W, ws.q, ws.dxT, ws.Mp, ws.dsp, M, N, K, y);
  }
}

template <int TM, int TN, int WM, int WN, int NS, int OCC, int KS>
static void launch_q80_lds(const uint8_t* W, const QgWorkspace& ws, int64_t M, int64_t N, int64_t K,
                           float* y, hipStream_t stream) {
  constexpr int BM = 32 * TM * WM, BN = 32 * TN * WN;
  const dim3 grid(static_cast<unsigned>((N + BN - 1) / BN), static_cast<unsigned>((M + BM - 1) / BM));
  gemm_q80_lds_kernel<TM, TN, WM, WN, NS, OCC, KS><<<grid, dim3(64 * WM * WN * KS), 0, stream>>>(
      W, ws.q, ws.dxT, ws.Mp, M, N, K, y);
}

template <int TM, int TN, int WM, int WN, int NS, int OCC, int KS>
static void launch_q5k_lds(const uint8_t* W, const QgWorkspace& ws, int64_t M, int64_t N, int64_t K,
                           float* y, hipStream_t stream) {
  constexpr int BM = 32 * TM * WM, BN = 32 * TN * WN;
  const dim3 grid(static_cast<unsigned>((N + BN - 1) / BN), static_cast<unsigned>((M + BM - 1) / BM));
  gemm_q5k_lds_kernel<TM, TN, WM, WN, NS, OCC, KS><<<grid, dim3(64 * WM * WN * KS), 0, stream>>>(
      W, ws.q, ws.dxT, ws.Mp, ws.dsp, M, N, K, y);
}

// OCC: waves per SIMD the register allocation must allow (launch bound);
// KS: K-groups per workgroup (at most the number of super-blocks)
template <int TM, int TN, int WM, int WN, bool DPP, int NS, int OCC = (WM * WN + 3) / 4, int KS = 1,
          bool A256 = false>
static void launch_lds(const uint8_t* W, const QgWorkspace& ws, int64_t M, int64_t N, int64_t K,
                       float* y, hipStream_t stream) {
  constexpr int BM = 32 * TM * WM, BN = 32 * TN * WN;
  const dim3 grid(static_cast<unsigned>((N + BN - 1) / BN), static_cast<unsigned>((M + BM - 1) / BM));
  gemm_q4k_lds_kernel<TM, TN, WM, WN, DPP, NS, OCC, KS, A256><<<grid, dim3(64 * WM * WN * KS), 0, stream>>>(
      W, ws.q, ws.dx, ws.dxT, ws.Mp, ws.dsp, M, N, K, y);
}

// Mixed block shapes for grids whose 128x256 blocks would leave the last round
// partly empty (512x4096->24576: 384 of them on 256 CUs): columns [0, N1) in
// 128x256 blocks of 2x2-tile waves, exactly one round of them, and columns
// [N1, N) in 64x256 blocks of 1x2-tile waves (half the work each), one more
// round at most; one workgroup of 8 waves per CU in either shape, so the
// second round starts as the first ends.  Every output element still adds its
// 32-value blocks in K order, so the result equals any other one-K-group
// tile shape's bit for bit.  Measured at 512x4096->24576: 139-144 us against
// 151-166 for the one-tile kernel (three rounds of two 64x128 blocks per CU)
// and 162-167 for 128x256 blocks alone (one and a half rounds).
constexpr int q4k_ring_bytes(int BM, int BN) {  // two stages of the body's A, W, DX, DSP regions
  return 2 * 1024 * ((BM * 16 + 63) / 64 + (BN * (kQ4Bytes / 16) + 63) / 64 + (BM * 2 + 63) / 64 +
                     (BM * 3 + 63) / 64);
}

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void gemm_q4k_mix_kernel(
    const uint8_t* __restrict__ W, const int8_t* __restrict__ qx, const float* __restrict__ dx,
    const float* __restrict__ dxT, int64_t Mp, const uint16_t* __restrict__ dsp, int64_t M,
    int64_t N, int64_t K, float* __restrict__ y, int64_t N1) {
  static_assert(q4k_ring_bytes(128, 256) >= q4k_ring_bytes(64, 256), "one ring serves both shapes");
  __shared__ __attribute__((aligned(16))) uint8_t lds[q4k_ring_bytes(128, 256)];
  const uint32_t gxb = static_cast<uint32_t>(N1 / 256), gyb = static_cast<uint32_t>((M + 127) / 128);
  const uint32_t L = blockIdx.x;
  if (L < gxb * gyb) {
    q4k_lds_body<2, 2, 2, 4, false, 2, 1, false, false, false, false, true>(
        W, qx, dx, dxT, Mp, dsp, M, N1, K, y, nullptr, 0, lds, L / gxb, L % gxb, N);
  } else {
    const uint32_t L2 = L - gxb * gyb, gxs = static_cast<uint32_t>((N - N1 + 255) / 256);
    q4k_lds_body<1, 2, 2, 4, false, 2, 1, false, false, false, false, true>(
        W + N1 * (K / 256) * kQ4Bytes, qx, dx, dxT, Mp, dsp, M, N - N1, K, y + N1, nullptr, 0, lds, L2 / gxs,
        L2 % gxs, N);
  }
}

// The same two block shapes with the SwiGLU epilogue (W holds the 2F gate and
// up rows; h [M][F] bfloat16): a block covers 128 output columns in either
// shape, gate and up rows of each, so both take their place in the full grid
// of F/128 column tiles (the large blocks the first F1/128 of them).
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void gemm_q4k_swiglu_mix_kernel(
    const uint8_t* __restrict__ W, const int8_t* __restrict__ qx, const float* __restrict__ dxT, int64_t Mp,
    const uint16_t* __restrict__ dsp, int64_t M, int64_t F, int64_t K, uint16_t* __restrict__ h, int64_t F1) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[q4k_ring_bytes(128, 256)];
  const uint32_t gxb = static_cast<uint32_t>(F1 / 128), gyb = static_cast<uint32_t>((M + 127) / 128);
  const uint32_t L = blockIdx.x;
  if (L < gxb * gyb) {
    q4k_lds_body<2, 2, 2, 4, false, 2, 1, false, true, false, false, true>(
        W, qx, nullptr, dxT, Mp, dsp, M, 2 * F, K, nullptr, h, F, lds, L / gxb, L % gxb, 0);
  } else {
    const uint32_t L2 = L - gxb * gyb, gxs = static_cast<uint32_t>((F - F1 + 127) / 128);
    q4k_lds_body<1, 2, 2, 4, false, 2, 1, false, true, false, false, true>(
        W, qx, nullptr, dxT, Mp, dsp, M, 2 * F, K, nullptr, h, F, lds, L2 / gxs, gxb + L2 % gxs, 0);
  }
}

static void launch_swiglu_mix(const uint8_t* W, const QgWorkspace& ws, int64_t M, int64_t F, int64_t K,
                              uint16_t* h, int64_t F1, hipStream_t stream) {
  const int64_t blocks = (F1 / 128) * ((M + 127) / 128) + ((F - F1 + 127) / 128) * ((M + 63) / 64);
  gemm_q4k_swiglu_mix_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(512), 0, stream>>>(
      W, ws.q, ws.dxT, ws.Mp, ws.dsp, M, F, K, h, F1);
}

static void launch_mix(const uint8_t* W, const QgWorkspace& ws, int64_t M, int64_t N, int64_t K, float* y,
                       int64_t N1, hipStream_t stream) {
  const int64_t blocks = (N1 / 256) * ((M + 127) / 128) + ((N - N1 + 255) / 256) * ((M + 63) / 64);
  gemm_q4k_mix_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(512), 0, stream>>>(
      W, ws.q, ws.dx, ws.dxT, ws.Mp, ws.dsp, M, N, K, y, N1);
}

}  // namespace qg

namespace {

// The mixed-block launch (gemm_q4k_mix_kernel) where the 128x256 blocks of a
// problem would fill one round and part of another: N1 = the columns of
// exactly one round of them (256 / row tiles column tiles, a whole number),
// and the 64x256 blocks of the remaining columns at most one more round and at
// least half of one.  Returns N1, or 0 for the other kernels.
int64_t q4k_mix_columns(int64_t M, int64_t N, int64_t K) {
  constexpr int64_t kCUs = 256;
  if (M < 256 || K < 512) return 0;
  const int64_t gyb = (M + 127) / 128, gx = (N + 255) / 256;
  if (kCUs % gyb != 0) return 0;
  const int64_t c1 = kCUs / gyb;
  if (c1 >= gx) return 0;
  const int64_t small = (gx - c1) * ((M + 63) / 64);
  if (small > kCUs || 2 * small < kCUs) return 0;
  return c1 * 256;
}

// Kernel choice for a Q4_K problem (measured on the workloads' shapes):
// prompts of 512 rows or more with enough 128x256 tiles to cover every CU,
// and whose rounds of them take less time than the rounds of 64x128 blocks,
// take workgroups of 8 waves x 2x2 tiles; otherwise, with enough 64x128 blocks,
// workgroups of 8 waves x one tile at 4 waves per SIMD (two workgroups per
// CU).  Grids with fewer output blocks split K inside the workgroup: 64x128
// blocks with two K-groups (16 waves) when there are at least half as many
// blocks as CUs, else 32x64 blocks with four K-groups (8 waves) when those
// cover the CUs (both only where the rows fill most of the block).  Smaller
// grids take one 32x32 tile per wave with the K range split so that the chip
// gets about two waves per SIMD.
enum class Q4Pick { kLds128x256, kLds64x128, kLds64x128K2, kLds32x64K4, kSmall1, kSmall2, kSmall4, kSmall8 };

Q4Pick pick_q4k(int64_t M, int64_t N, int64_t K) {
  constexpr int64_t kCUs = 256;
  // about two waves per SIMD; one for decode-sized batches (their waves
  // apply a quarter of the epilogue: 1024 measured faster than 2048 at
  // M = 8 on 2560->9728, 9728->2560 and 4096->24576)
  const int64_t kTargetWaves = M <= 8 ? 1024 : 2048;
  const int64_t nsb = K / 256;
  const int64_t blocks64x128 = ((M + 63) / 64) * ((N + 127) / 128);
  // 128x256 blocks run one per CU and 64x128 blocks two, and a round of the
  // larger blocks does twice the work at about 1.19x the rate (2x2-tile waves
  // share their decoded weights and row scales): the larger blocks where
  // their rounds, times 2 / 1.19, are fewer than the 64x128 blocks' rounds.
  // Measured: 512x4096->32768 192 against 217 us, 512x2048->49152 159 against
  // 170, 896x4096->24576 280 against 304, 1024x4096->16384 201 against 224,
  // 1536x4096->24576 477 against 491-511, 1536x2560->9728 119 against 136; the
  // other way 640x2048->32768 149 against 140, 768x4096->24576 271 against
  // 246, 1024x2560->9728 114 against 88, 4096x9728->2560 452 against ~300-350.
  const int64_t blocks128x256 = ((M + 127) / 128) * ((N + 255) / 256);
  const int64_t rounds128 = (blocks128x256 + kCUs - 1) / kCUs;
  const int64_t rounds64 = (blocks64x128 + 2 * kCUs - 1) / (2 * kCUs);
  if (M >= 512 && blocks128x256 >= kCUs && 168 * rounds128 < 100 * rounds64) return Q4Pick::kLds128x256;
  if (blocks64x128 >= kCUs) return Q4Pick::kLds64x128;
  if (M >= 48 && blocks64x128 * 2 >= kCUs && nsb >= 4) return Q4Pick::kLds64x128K2;
  if (M >= 24 && ((M + 31) / 32) * ((N + 63) / 64) >= kCUs && nsb >= 8) return Q4Pick::kLds32x64K4;
  const int64_t tiles = ((M + 31) / 32) * ((N + 31) / 32);
  if (tiles >= kTargetWaves || nsb < 2) return Q4Pick::kSmall1;
  if (tiles * 2 >= kTargetWaves || nsb < 4) return Q4Pick::kSmall2;
  if (tiles * 4 >= kTargetWaves || nsb < 8) return Q4Pick::kSmall4;
  return Q4Pick::kSmall8;
}

}  // namespace

// Kernel names as a profiler lists them (A256 is the last template argument).
const char* qg_gemm_q4k_kernel_name(int64_t M, int64_t N, int64_t K, bool a256) {
  if (!a256 && q4k_mix_columns(M, N, K) > 0) return "gemm_q4k_mix_kernel";
  switch (pick_q4k(M, N, K)) {
    case Q4Pick::kLds128x256:
      return a256 ? "gemm_q4k_lds_kernel<1, 1, 2, 4, false, 2, 4, 1, true>"
                  : "gemm_q4k_lds_kernel<2, 2, 2, 4, false, 2, 2, 1, false>";
    case Q4Pick::kLds64x128:
      return a256 ? "gemm_q4k_lds_kernel<1, 1, 2, 4, false, 2, 4, 1, true>"
                  : "gemm_q4k_lds_kernel<1, 1, 2, 4, false, 2, 4, 1, false>";
    case Q4Pick::kLds64x128K2:
      return a256 ? "gemm_q4k_lds_kernel<1, 1, 2, 4, false, 2, 4, 2, true>"
                  : "gemm_q4k_lds_kernel<1, 1, 2, 4, false, 2, 4, 2, false>";
    case Q4Pick::kLds32x64K4:
      return a256 ? "gemm_q4k_lds_kernel<1, 1, 1, 2, false, 2, 2, 4, true>"
                  : "gemm_q4k_lds_kernel<1, 1, 1, 2, false, 2, 2, 4, false>";
    case Q4Pick::kSmall1: return M <= 8 ? "gemm_q4k_small_kernel<1, 4>" : "gemm_q4k_small_kernel<1, 16>";
    case Q4Pick::kSmall2: return M <= 8 ? "gemm_q4k_small_kernel<2, 4>" : "gemm_q4k_small_kernel<2, 16>";
    case Q4Pick::kSmall4: return M <= 8 ? "gemm_q4k_small_kernel<4, 4>" : "gemm_q4k_small_kernel<4, 16>";
    case Q4Pick::kSmall8: return M <= 8 ? "gemm_q4k_small_kernel<8, 4>" : "gemm_q4k_small_kernel<8, 16>";
  }
  return "?";
}

// a256: the per-256 workspace (every 32-value block of a super-block holds the
// super-block's scale).  The LDS kernels then combine sub-blocks in integers
// (for long prompts in 64x128 blocks: the 2x2-tile waves would need the
// integer sums of four tiles on top of their fp32 ones and spill; measured
// 725 against 514 TOPS at M = 8192); the small-grid kernel computes the same
// result with its per-block epilogue.
hipError_t qg_launch_gemm_q4k(const uint8_t* W, const QgWorkspace& ws, int64_t M, int64_t N,
                              int64_t K, float* y, hipStream_t stream, bool a256) {
  if (const int64_t N1 = a256 ? 0 : q4k_mix_columns(M, N, K); N1 > 0) {
    qg::launch_mix(W, ws, M, N, K, y, N1, stream);
    return hipGetLastError();
  }
  switch (pick_q4k(M, N, K)) {
    case Q4Pick::kLds128x256:
      if (a256) qg::launch_lds<1, 1, 2, 4, false, 2, 4, 1, true>(W, ws, M, N, K, y, stream);
      else qg::launch_lds<2, 2, 2, 4, false, 2>(W, ws, M, N, K, y, stream);
      break;
    case Q4Pick::kLds64x128:
      if (a256) qg::launch_lds<1, 1, 2, 4, false, 2, 4, 1, true>(W, ws, M, N, K, y, stream);
      else qg::launch_lds<1, 1, 2, 4, false, 2, 4>(W, ws, M, N, K, y, stream);
      break;
    case Q4Pick::kLds64x128K2:
      if (a256) qg::launch_lds<1, 1, 2, 4, false, 2, 4, 2, true>(W, ws, M, N, K, y, stream);
      else qg::launch_lds<1, 1, 2, 4, false, 2, 4, 2>(W, ws, M, N, K, y, stream);
      break;
    case Q4Pick::kLds32x64K4:
      if (a256) qg::launch_lds<1, 1, 1, 2, false, 2, 2, 4, true>(W, ws, M, N, K, y, stream);
      else qg::launch_lds<1, 1, 1, 2, false, 2, 2, 4>(W, ws, M, N, K, y, stream);
      break;
    case Q4Pick::kSmall1: qg::launch_small<1>(W, ws, M, N, K, y, stream); break;
    case Q4Pick::kSmall2: qg::launch_small<2>(W, ws, M, N, K, y, stream); break;
    case Q4Pick::kSmall4: qg::launch_small<4>(W, ws, M, N, K, y, stream); break;
    case Q4Pick::kSmall8: qg::launch_small<8>(W, ws, M, N, K, y, stream); break;
  }
  return hipGetLastError();
}

// SwiGLU-fused gate+up projection: the block shapes the plain GEMM takes for
// the 2F-column problem (a block covers half as many output columns, over the
// gate and the up rows of each); problems on the small-grid kernel are not
// fused.  Weight rows are addressed with 32-bit offsets from a block's first
// gate row, so (F + 128) rows must span less than 4 GiB.
bool qg_q4k_swiglu_fusable(int64_t M, int64_t F, int64_t K) {
  if (F < 1 || (F + 128) * (K / 256) * qg::kQ4Bytes >= (INT64_C(1) << 32)) return false;
  const Q4Pick p = pick_q4k(M, 2 * F, K);
  return p == Q4Pick::kLds128x256 || p == Q4Pick::kLds64x128 || p == Q4Pick::kLds64x128K2 ||
         p == Q4Pick::kLds32x64K4;
}

const char* qg_gemm_q4k_swiglu_kernel_name(int64_t M, int64_t F, int64_t K) {
  if (!qg_q4k_swiglu_fusable(M, F, K)) return nullptr;
  if (q4k_mix_columns(M, 2 * F, K) > 0) return "gemm_q4k_swiglu_mix_kernel";
  switch (pick_q4k(M, 2 * F, K)) {
    case Q4Pick::kLds128x256: return "gemm_q4k_swiglu_kernel<2, 2, 2, 4, 2, 2, 1>";
    case Q4Pick::kLds64x128: return "gemm_q4k_swiglu_kernel<1, 1, 2, 4, 2, 4, 1>";
    case Q4Pick::kLds64x128K2: return "gemm_q4k_swiglu_kernel<1, 1, 2, 4, 2, 4, 2>";
    case Q4Pick::kLds32x64K4: return "gemm_q4k_swiglu_kernel<1, 1, 1, 2, 2, 2, 4>";
    default: return nullptr;
  }
}

hipError_t qg_launch_gemm_q4k_swiglu(const uint8_t* W, const QgWorkspace& ws, int64_t M, int64_t F,
                                     int64_t K, uint16_t* h, hipStream_t stream) {
  if (!qg_q4k_swiglu_fusable(M, F, K)) return hipErrorInvalidValue;
  if (const int64_t N1 = q4k_mix_columns(M, 2 * F, K); N1 > 0) {
    qg::launch_swiglu_mix(W, ws, M, F, K, h, N1 / 2, stream);
    return hipGetLastError();
  }
  switch (pick_q4k(M, 2 * F, K)) {
    case Q4Pick::kLds128x256: qg::launch_swiglu<2, 2, 2, 4, 2, 2, 1>(W, ws, M, F, K, h, stream); break;
    case Q4Pick::kLds64x128: qg::launch_swiglu<1, 1, 2, 4, 2, 4, 1>(W, ws, M, F, K, h, stream); break;
    case Q4Pick::kLds64x128K2: qg::launch_swiglu<1, 1, 2, 4, 2, 4, 2>(W, ws, M, F, K, h, stream); break;
    case Q4Pick::kLds32x64K4: qg::launch_swiglu<1, 1, 1, 2, 2, 2, 4>(W, ws, M, F, K, h, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Q5_K: the Q4_K dispatch rule with the block shapes that fit its 176-byte
// blocks in LDS (two stages of 128x256 or of 64x128 with two K-groups would
// take 172 KB): 64x128 blocks for the two largest shapes (one per CU: 88 KB),
// 32x64 with three K-groups for the split-K ones.
const char* qg_gemm_q5k_kernel_name(int64_t M, int64_t N, int64_t K) {
  switch (pick_q4k(M, N, K)) {
    case Q4Pick::kLds128x256:
    case Q4Pick::kLds64x128: return "gemm_q5k_lds_kernel<1, 1, 2, 4, 2, 2, 1>";
    case Q4Pick::kLds64x128K2:
    case Q4Pick::kLds32x64K4: return "gemm_q5k_lds_kernel<1, 1, 1, 2, 2, 2, 3>";
    case Q4Pick::kSmall1: return M <= 8 ? "gemm_q5k_small_kernel<1, 4>" : "gemm_q5k_small_kernel<1, 16>";
    case Q4Pick::kSmall2: return M <= 8 ? "gemm_q5k_small_kernel<2, 4>" : "gemm_q5k_small_kernel<2, 16>";
    case Q4Pick::kSmall4: return M <= 8 ? "gemm_q5k_small_kernel<4, 4>" : "gemm_q5k_small_kernel<4, 16>";
    case Q4Pick::kSmall8: return M <= 8 ? "gemm_q5k_small_kernel<8, 4>" : "gemm_q5k_small_kernel<8, 16>";
  }
  return "?";
}

hipError_t qg_launch_gemm_q5k(const uint8_t* W, const QgWorkspace& ws, int64_t M, int64_t N,
                              int64_t K, float* y, hipStream_t stream) {
  switch (pick_q4k(M, N, K)) {
    case Q4Pick::kLds128x256:
    case Q4Pick::kLds64x128: qg::launch_q5k_lds<1, 1, 2, 4, 2, 2, 1>(W, ws, M, N, K, y, stream); break;
    case Q4Pick::kLds64x128K2:
    case Q4Pick::kLds32x64K4: qg::launch_q5k_lds<1, 1, 1, 2, 2, 2, 3>(W, ws, M, N, K, y, stream); break;
    case Q4Pick::kSmall1: qg::launch_small<1, true>(W, ws, M, N, K, y, stream); break;
    case Q4Pick::kSmall2: qg::launch_small<2, true>(W, ws, M, N, K, y, stream); break;
    case Q4Pick::kSmall4: qg::launch_small<4, true>(W, ws, M, N, K, y, stream); break;
    case Q4Pick::kSmall8: qg::launch_small<8, true>(W, ws, M, N, K, y, stream); break;
  }
  return hipGetLastError();
}

// Q8_0 (272 bytes per 256 values of a row): 64x128 blocks for the large
// grids (one per CU: two stages take 104 KB), otherwise 32x64 blocks with
// three K-groups (156 KB), or one where the row has fewer than three
// super-block lengths.
namespace {
enum class Q8Pick { kLds64x128, kLds32x64K3, kLds32x64 };
Q8Pick pick_q80(int64_t M, int64_t N, int64_t K) {
  switch (pick_q4k(M, N, K)) {
    case Q4Pick::kLds128x256:
    case Q4Pick::kLds64x128: return Q8Pick::kLds64x128;
    default: return K / 256 >= 3 ? Q8Pick::kLds32x64K3 : Q8Pick::kLds32x64;
  }
}
}  // namespace

const char* qg_gemm_q80_kernel_name(int64_t M, int64_t N, int64_t K) {
  switch (pick_q80(M, N, K)) {
    case Q8Pick::kLds64x128: return "gemm_q80_lds_kernel<1, 1, 2, 4, 2, 2, 1>";
    case Q8Pick::kLds32x64K3: return "gemm_q80_lds_kernel<1, 1, 1, 2, 2, 2, 3>";
    case Q8Pick::kLds32x64: return "gemm_q80_lds_kernel<1, 1, 1, 2, 2, 2, 1>";
  }
  return "?";
}

hipError_t qg_launch_gemm_q80(const uint8_t* W, const QgWorkspace& ws, int64_t M, int64_t N,
                              int64_t K, float* y, hipStream_t stream) {
  switch (pick_q80(M, N, K)) {
    case Q8Pick::kLds64x128: qg::launch_q80_lds<1, 1, 2, 4, 2, 2, 1>(W, ws, M, N, K, y, stream); break;
    case Q8Pick::kLds32x64K3: qg::launch_q80_lds<1, 1, 1, 2, 2, 2, 3>(W, ws, M, N, K, y, stream); break;
    case Q8Pick::kLds32x64: qg::launch_q80_lds<1, 1, 1, 2, 2, 2, 1>(W, ws, M, N, K, y, stream); break;
  }
  return hipGetLastError();
}

// SwiGLU-fused gate+up projection over Q5_K and Q8_0 weights: the block shapes
// of each format's plain GEMM for the 2F-column problem (Q5_K's small-grid
// problems are not fused); 32-bit weight offsets as for Q4_K.
bool qg_swiglu_fusable(int fmt, int64_t M, int64_t F, int64_t K) {
  if (fmt == QG_Q4_K) return qg_q4k_swiglu_fusable(M, F, K);
  const int64_t bb = fmt == QG_Q5_K ? qg::kQ5Bytes : 8 * qg::kQ8Bytes;
  if ((fmt != QG_Q5_K && fmt != QG_Q8_0) || F < 1 || (F + 128) * (K / 256) * bb >= (INT64_C(1) << 32))
    return false;
  if (fmt == QG_Q8_0) return true;
  const Q4Pick p = pick_q4k(M, 2 * F, K);
  return p == Q4Pick::kLds128x256 || p == Q4Pick::kLds64x128 || p == Q4Pick::kLds64x128K2 ||
         p == Q4Pick::kLds32x64K4;
}

const char* qg_gemm_swiglu_kernel_name(int fmt, int64_t M, int64_t F, int64_t K) {
  if (!qg_swiglu_fusable(fmt, M, F, K)) return nullptr;
  if (fmt == QG_Q4_K) return qg_gemm_q4k_swiglu_kernel_name(M, F, K);
  if (fmt == QG_Q5_K) {
    switch (pick_q4k(M, 2 * F, K)) {
      case Q4Pick::kLds128x256:
      case Q4Pick::kLds64x128: return "gemm_q5k_swiglu_kernel<1, 1, 2, 4, 2, 2, 1>";
      default: return "gemm_q5k_swiglu_kernel<1, 1, 1, 2, 2, 2, 3>";
    }
  }
  switch (pick_q80(M, 2 * F, K)) {
    case Q8Pick::kLds64x128: return "gemm_q80_swiglu_kernel<1, 1, 2, 4, 2, 2, 1>";
    case Q8Pick::kLds32x64K3: return "gemm_q80_swiglu_kernel<1, 1, 1, 2, 2, 2, 3>";
    default: return "gemm_q80_swiglu_kernel<1, 1, 1, 2, 2, 2, 1>";
  }
}

hipError_t qg_launch_gemm_swiglu(const uint8_t* W, int fmt, const QgWorkspace& ws, int64_t M, int64_t F,
                                 int64_t K, uint16_t* h, hipStream_t stream) {
  if (!qg_swiglu_fusable(fmt, M, F, K)) return hipErrorInvalidValue;
  if (fmt == QG_Q4_K) return qg_launch_gemm_q4k_swiglu(W, ws, M, F, K, h, stream);
  if (fmt == QG_Q5_K) {
    switch (pick_q4k(M, 2 * F, K)) {
      case Q4Pick::kLds128x256:
      case Q4Pick::kLds64x128:
        qg::launch_swiglu<1, 1, 2, 4, 2, 2, 1, QG_Q5_K>(W, ws, M, F, K, h, stream); break;
      default: qg::launch_swiglu<1, 1, 1, 2, 2, 2, 3, QG_Q5_K>(W, ws, M, F, K, h, stream); break;
    }
    return hipGetLastError();
  }
  switch (pick_q80(M, 2 * F, K)) {
    case Q8Pick::kLds64x128: qg::launch_swiglu<1, 1, 2, 4, 2, 2, 1, QG_Q8_0>(W, ws, M, F, K, h, stream); break;
    case Q8Pick::kLds32x64K3: qg::launch_swiglu<1, 1, 1, 2, 2, 2, 3, QG_Q8_0>(W, ws, M, F, K, h, stream); break;
    default: qg::launch_swiglu<1, 1, 1, 2, 2, 2, 1, QG_Q8_0>(W, ws, M, F, K, h, stream); break;
  }
  return hipGetLastError();
}
