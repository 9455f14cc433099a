// Skinny path for M <= 8 activation rows (decode-sized batches and the LM head
// on the last token only -- aprender issue #5305, sub-ticket #4313 "MMQ int8
// prefill matmul + LM head on the last token only").  Every weight byte is read
// once, so the kernel is bound by HBM bandwidth (the decode-GEMV yardstick of
// issue #5305's merged ticket #5221, "decode GEMV at 223-504 GB/s vs llama.cpp
// MMVQ 776-894", and the fraction-of-peak figures of issue #4220).  Same
// arithmetic as the tiled kernels: int8 codes times int8 activation codes
// summed per sub-block in int32 (v_dot4_i32_i8), scales and mins applied in
// fp32.
//
// Work split.  Four lanes share one 256-value super-block; each lane holds 64
// of its values, read with three 16-byte loads:
//   Q4_K  lane s (0..3): the 16-byte header (d, dmin, packed scales) and the
//         32 code bytes qs[32s .. 32s+31], i.e. sub-blocks 2s (low nibbles)
//         and 2s+1 (high nibbles).
//   Q5_K  the same (qs at byte 48) plus the 32 qh bytes, whose bits 2s and
//         2s+1 are the fifth bits of the lane's two sub-blocks: five loads.
//   Q8_0  a super-block's share of a row is eight 34-byte blocks (272 bytes);
//         lane s reads bytes 68s .. 68s+67 (blocks 2s and 2s+1, d and codes)
//         with four 16-byte loads and one dword.
//   Q6_K  lane s = 2*half + lh: ql[64half + 16lh ..+16], ql[64half + 32 +
//         16lh ..+16] and qh[32half + 16lh ..+16], i.e. the values
//         128half + 32c + 16lh + i (c = 0..3, i < 16), which are the 16-value
//         sub-blocks 8half + 2c + lh; plus one 8-byte load of the scales / d
//         region, the four lanes' pieces exchanged with quad DPP moves (a
//         separate 2-byte load of d measured ~5% slower).  Q6_K blocks are
//         210 bytes, so these loads are only 2-byte aligned (gfx950 serves
//         unaligned vector loads; realigning dword-aligned loads with
//         v_alignbyte measured no faster).
// Q6_K matrices whose steps start on 16-byte boundaries are instead loaded
// whole-line (see CO at the kernel) and the same fields read back from LDS.
// So a wavefront covers 16 super-blocks (4096 values) per step.  A row of nsb
// super-blocks takes ceil(nsb/16) steps; when nsb divides 16, one step covers
// R = 16/nsb whole rows.  Wavefronts take rows (or R-row groups) in turn, so
// the grid streams one narrow band of the matrix at a time; each wavefront has
// the loads of step t+1 in flight while step t is computed (two register
// buffers used in turn).
//
// Activations.  When a row takes a single step, every lane works on the same
// 64 activation values in every step, so it can keep their codes, block
// scales and the -32 correction of the Q6_K codes in registers (XREG: one or
// two activation rows, or short rows).  Otherwise the activation rows are
// staged in LDS once per workgroup (XLDS) or, when they do not fit, one
// 4096-value slice of K at a time (XSLICE): the workgroup stages slice t of
// every activation row, its wavefronts take the slice's step of each of
// their rows (up to kSlRows rows at a time, their partial sums kept per
// row), then the next slice.  Every lane accumulates its super-blocks in the
// same order in all three modes, so they give the same bits.
//
// Q6_K codes go to v_dot4_i32_i8 as the unsigned q6 in [0, 63] (below 128, so
// also valid signed bytes) and the offset is applied through the activation
// sum: sum (q6 - 32) x = sum q6 x - 32 sum x, with the dot chain started at
// -32 sum x.
#include <stdio.h>

#include "common.h"
#include "lds_stage.h"

namespace qg {

typedef uint32_t u32x4_a2 __attribute__((ext_vector_type(4), aligned(2)));

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot4(static_cast<int>(a), static_cast<int>(b), c, false);
}

__device__ __forceinline__ uint4 ld16_a2(const uint8_t* p) {
  const u32x4_a2 v = *reinterpret_cast<const u32x4_a2*>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Raw bytes one lane loads for one step.
struct SkRaw {
  uint4 a, b, c;    // Q4_K: header, qs lo 16, qs hi 16.  Q6_K: ql0, ql1, qh
  uint32_t s0, s1;  // Q6_K: 8 bytes of the scales / d region (see the load)
  uint4 e;          // Q6_K, coalesced loads: a, b, c, e are the step's chunks l, l+64, l+128, l+192
                    // Q5_K: qh[0..15]
  uint4 f;          // Q5_K: qh[16..31]
};

typedef uint32_t u32x2_a2 __attribute__((ext_vector_type(2), aligned(2)));

constexpr int kSkMaxLds = 64 * 1024;
enum { kXReg = 0, kXLds = 1, kXSlice = 2 };
constexpr int kSlRows = 2;  // XSLICE: rows a wavefront carries through the slices at a time
enum { kCoNone = 0, kCoReg = 1, kCoDma = 2 };

// sum over 16 int8 values
__device__ __forceinline__ int sum16(const uint4& x) {
  int s = dot4(0x01010101u, x.x, 0);
  s = dot4(0x01010101u, x.y, s);
  s = dot4(0x01010101u, x.z, s);
  return dot4(0x01010101u, x.w, s);
}

// Sum of v over each aligned group of G lanes (G = 4, 8, 16, 32, 64) with DPP
// moves; the sum ends in the group's last lane (for G <= 16 in all its lanes).
// Steps: quad swaps, half-row and row mirrors, then the row broadcasts of
// lane 15 and lane 31 into the following rows.
template <int G>
__device__ __forceinline__ float group_sum_last(float v) {
  static_assert(G == 4 || G == 8 || G == 16 || G == 32 || G == 64, "group size");
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  if (G >= 8)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
  if (G >= 16)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
  if (G >= 32)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false));
  if (G >= 64)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xC, 0xF, false));
  return v;
}

// FMT: QG_Q4_K / QG_Q5_K / QG_Q6_K / QG_Q8_0.  MR: activation rows.  R: rows per wavefront step
// (16/nsb when that divides, else 1).  XM: where the activations are read.
// TH: threads per workgroup (256, 512 or 1024; see skinny_threads).
// CO (Q6_K only): coalesced loads.  A step's sixteen super-blocks are 3360
// contiguous bytes; when every step starts 16-byte aligned and the matrix ends
// on a 16-byte boundary, lane l loads the step's aligned chunks l, l+64, l+128
// and l+192 (whole cache lines per load instead of 16-byte fields scattered at
// 2-byte alignment) into the wavefront's own 4 KB of LDS, and every lane reads
// its fields back from there.  kCoReg: the chunks go through registers (two
// register buffers, as the field loads); kCoDma: global_load_lds_dwordx4 puts
// them straight into two LDS buffers (no registers held; used for one or two
// activation rows, where it measured fastest).
template <int FMT, int MR, int R, int XM, int CO, int TH>
__global__ __launch_bounds__(TH) void skinny_kernel(
    const uint8_t* __restrict__ W, const int8_t* __restrict__ qx, const float* __restrict__ gdx,
    const float* __restrict__ gdS, int64_t N, int64_t K, float* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  static_assert(CO == kCoNone || FMT == QG_Q6_K, "coalesced loads are for Q6_K");
  constexpr bool KQ = FMT != QG_Q6_K;  // Q4_K, Q5_K, Q8_0: 64 values per lane, two per-32 blocks
  constexpr bool Q5 = FMT == QG_Q5_K, Q8 = FMT == QG_Q8_0;
  constexpr int NBUF = CO == kCoDma ? 2 : 1;
  __shared__ __attribute__((aligned(16))) uint8_t rowbuf[CO ? TH / 64 : 1][NBUF][CO ? 4096 : 16];
  constexpr int BB = FMT == QG_Q4_K ? kQ4Bytes : Q5 ? kQ5Bytes : Q8 ? 8 * kQ8Bytes : kQ6Bytes;
  constexpr int G = 64 / R;  // lanes per row within a step
  const int64_t nsb = K / 256, nb = K / 32;
  const int lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * (TH / 64) +
                       __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // activation rows: codes at xs + m * xk, scales at xd / xS + m * xnb, for
  // super-blocks from xj0 on (XSLICE: the staged slice)
  const int8_t* xs = qx;
  const float* xd = gdx;
  const float* xS = gdS;
  int64_t xk = K, xnb = nb, xj0 = 0;
  if constexpr (XM == kXLds) {
    int8_t* lq = reinterpret_cast<int8_t*>(smem);
    float* ld = reinterpret_cast<float*>(smem + MR * K);
    float* lS = ld + MR * nb;
    const int64_t nq = MR * K / 16, nd = MR * nb / 4;
    for (int64_t i = threadIdx.x; i < nq; i += TH)
      reinterpret_cast<uint4*>(lq)[i] = reinterpret_cast<const uint4*>(qx)[i];
    for (int64_t i = threadIdx.x; i < nd; i += TH) {
      reinterpret_cast<float4*>(ld)[i] = reinterpret_cast<const float4*>(gdx)[i];
      if (KQ) reinterpret_cast<float4*>(lS)[i] = reinterpret_cast<const float4*>(gdS)[i];
    }
    __syncthreads();
    xs = lq;
    xd = ld;
    xS = lS;
  }

  // wavefront w takes rows w*R + k*stride (+ 0..R-1), k = 0, 1, ...: at any
  // time the whole grid streams one narrow band of the weight matrix
  const int64_t stride = static_cast<int64_t>(gridDim.x) * (TH / 64) * R;
  const int64_t row_begin = wave * R;
  // (XSLICE: a wavefront without rows still stages slices and meets the barriers)
  if (XM != kXSlice && row_begin >= N) return;

  const int grp = lane >> 2, s = lane & 3;
  const int half = s >> 1, lh = s & 1;              // Q6_K lane roles
  const int ro = grp / (16 / R);                    // row of this lane within a step
  const int jb0 = R > 1 ? grp % (16 / R) : grp;     // super-block of this lane in a row's first step
  const int64_t ipr = R > 1 ? 1 : (nsb + 15) / 16;  // steps per row
  const int64_t nsteps = (N - row_begin + stride - 1) / stride * ipr;
  const int64_t row_bytes = nsb * BB;
  const int64_t last_chunk = N * row_bytes / 16 - 1;  // CO: the matrix is a whole number of chunks
  uint8_t* const lrow0 = rowbuf[CO ? threadIdx.x >> 6 : 0][0];
  uint8_t* const lrow1 = rowbuf[CO ? threadIdx.x >> 6 : 0][NBUF - 1];
  // lane offset inside a super-block of each of its loads
  constexpr uint32_t QS = Q5 ? 48u : 16u;  // first nibble byte (Q4_K, Q5_K)
  const uint32_t off_a = Q8 ? 68u * s : KQ ? 0u : static_cast<uint32_t>(64 * half + 16 * lh);
  const uint32_t off_b = Q8 ? 68u * s + 16u : KQ ? QS + 32u * s : static_cast<uint32_t>(64 * half + 32 + 16 * lh);
  const uint32_t off_c = Q8 ? 68u * s + 32u : KQ ? QS + 16u + 32u * s : static_cast<uint32_t>(128 + 32 * half + 16 * lh);

  // per-lane activation data for XREG (a lane's super-block never changes)
  constexpr int XR = XM == kXReg ? MR : 1;
  uint4 xr[XR][4];
  float xdr[XR][4];
  int xur[XR][4];
  if constexpr (XM == kXReg) {
    const int64_t jb = jb0 < nsb ? jb0 : nsb - 1;  // idle lanes (jb0 >= nsb) read valid data
#pragma unroll
    for (int m = 0; m < MR; m++) {
      if (KQ) {
        const uint4* xv = reinterpret_cast<const uint4*>(qx + m * K + 256 * jb + 64 * s);
#pragma unroll
        for (int c = 0; c < 4; c++) xr[m][c] = xv[c];
        const int64_t b0 = 8 * jb + 2 * s;
        xdr[m][0] = gdx[m * nb + b0];
        xdr[m][1] = gdx[m * nb + b0 + 1];
        xdr[m][2] = gdS[m * nb + b0];
        xdr[m][3] = gdS[m * nb + b0 + 1];
      } else {
        const int8_t* xp = qx + m * K + 256 * jb + 128 * half + 16 * lh;
#pragma unroll
        for (int c = 0; c < 4; c++) {
          xr[m][c] = *reinterpret_cast<const uint4*>(xp + 32 * c);
          xur[m][c] = -32 * sum16(xr[m][c]);
          xdr[m][c] = gdx[m * nb + 8 * jb + 4 * half + c];
        }
      }
    }
  }

  // Lanes past the row range or past the row's last super-block (partial last
  // steps) load a clamped, valid block and their contribution is dropped, so
  // the step code has no branches.
  auto load = [&](int64_t rs, int64_t it, SkRaw& r) {
    if constexpr (CO) {
      // chunk index of the step's first byte: row (row_begin + rs*stride),
      // super-block 16*it; the step's 210 chunks end at c_end, the lanes past
      // it (fourth load) re-read that chunk, and chunks past the matrix its last
      const int64_t cs = ((row_begin + rs * stride) * row_bytes + 16 * it * BB) / 16;
      const int64_t c_end = cs + 16 * BB / 16 - 1 < last_chunk ? cs + 16 * BB / 16 - 1 : last_chunk;
      const int64_t c0 = cs + lane;
      const uint4* wc = reinterpret_cast<const uint4*>(W);
      auto chunk = [&](int k) {
        const int64_t c = c0 + 64 * k;
        return wc + (c < c_end ? c : c_end);
      };
      if constexpr (CO == kCoDma) {
        // into the LDS buffer of this register set (its index rides in s0)
        uint8_t* lb = r.s0 ? lrow1 : lrow0;
#pragma unroll
        for (int k = 0; k < 4; k++) lds_dma16(chunk(k), lb + 1024 * k);
      } else {
        r.a = *chunk(0);
        r.b = *chunk(1);
        r.c = *chunk(2);
        r.e = *chunk(3);
      }
    } else {
      int64_t n = row_begin + rs * stride + ro, jb = jb0 + 16 * it;
      n = n < N ? n : N - 1;
      jb = jb < nsb ? jb : nsb - 1;
      const uint8_t* blk = W + n * row_bytes + jb * BB;
      if (Q8) {  // dword-aligned: 68 bytes from 68s
        r.a = ld16_a2(blk + off_a);
        r.b = ld16_a2(blk + off_b);
        r.c = ld16_a2(blk + off_c);
        r.e = ld16_a2(blk + off_c + 16);
        r.s0 = *reinterpret_cast<const uint32_t*>(blk + off_c + 32);
      } else if (KQ) {
        r.a = *reinterpret_cast<const uint4*>(blk + off_a);
        r.b = *reinterpret_cast<const uint4*>(blk + off_b);
        r.c = *reinterpret_cast<const uint4*>(blk + off_c);
        if (Q5) {
          r.e = *reinterpret_cast<const uint4*>(blk + 16);
          r.f = *reinterpret_cast<const uint4*>(blk + 32);
        }
      } else {
        r.a = ld16_a2(blk + off_a);
        r.b = ld16_a2(blk + off_b);
        r.c = ld16_a2(blk + off_c);
        // one 8-byte load per lane covers the 18 bytes of scales and d between
        // the four lanes of the block: s = 0, 1, 2 read bytes 192, 196, 200
        // (+8), s = 3 reads bytes 202..209 (scales 10..15 and d)
        const u32x2_a2 e = *reinterpret_cast<const u32x2_a2*>(blk + (s == 3 ? 202 : 192 + 4 * s));
        r.s0 = e.x;
        r.s1 = e.y;
      }
    }
  };

  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; m++) acc[m] = 0.0f;

  auto compute = [&](int64_t rs, int64_t it, const SkRaw raw) {
    const int64_t n = row_begin + rs * stride + ro, jbr = jb0 + 16 * it;
    const bool valid = n < N && jbr < nsb;
    const int64_t jb = jbr < nsb ? jbr : nsb - 1;
    uint4 fa, fb, fc;  // this lane's fields (see SkRaw)
    uint4 fe = {}, ff = {};  // Q5_K: the qh bytes
    uint32_t fs0, fs1;
    if constexpr (CO) {
      // through this wavefront's LDS row buffer: the step's chunks in, this
      // lane's fields (block grp of the step, 2-byte aligned) out
      const uint8_t* bp;
      if constexpr (CO == kCoDma) {
        // this step's four loads have landed once at most the next step's
        // four are outstanding (same-type loads complete in order; a pending
        // output store only makes the wait longer)
        asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        bp = (raw.s0 ? lrow1 : lrow0) + grp * BB;
      } else {
        *reinterpret_cast<uint4*>(lrow0 + 16 * lane) = raw.a;
        *reinterpret_cast<uint4*>(lrow0 + 16 * (lane + 64)) = raw.b;
        *reinterpret_cast<uint4*>(lrow0 + 16 * (lane + 128)) = raw.c;
        *reinterpret_cast<uint4*>(lrow0 + 16 * (lane + 192)) = raw.e;
        bp = lrow0 + grp * BB;
      }
      fa = ld16_a2(bp + off_a);
      fb = ld16_a2(bp + off_b);
      fc = ld16_a2(bp + off_c);
      const u32x2_a2 e = *reinterpret_cast<const u32x2_a2*>(bp + (s == 3 ? 202 : 192 + 4 * s));
      fs0 = e.x;
      fs1 = e.y;
    } else {
      fa = raw.a;
      fb = raw.b;
      fc = raw.c;
      fe = raw.e;
      ff = raw.f;
      fs0 = raw.s0;
      fs1 = raw.s1;
    }
    {
      if (KQ) {
        float dsc0, dsc1, dm0 = 0.0f, dm1 = 0.0f;
        uint32_t lo[8], hi[8];
        if constexpr (Q8) {
          // bytes 68s .. 68s+67: d of block 2s, its 32 codes (two bytes past a
          // dword: realigned), d of block 2s+1, its 32 codes (dword aligned)
          const uint32_t w[17] = {fa.x, fa.y, fa.z, fa.w, fb.x, fb.y, fb.z, fb.w, fc.x,
                                  fc.y, fc.z, fc.w, fe.x, fe.y, fe.z, fe.w, fs0};
          dsc0 = half_to_float(w[0] & 0xFFFFu);
          dsc1 = half_to_float(w[8] >> 16);
#pragma unroll
          for (int i = 0; i < 8; i++) {
            lo[i] = __builtin_amdgcn_alignbyte(w[i + 1], w[i], 2);
            hi[i] = w[9 + i];
          }
        } else {
        const float d = half_to_float(fa.x & 0xFFFFu), dmin = half_to_float(fa.x >> 16);
        const Q4Scales sc = unpack_q4_scales(fa.y, fa.z, fa.w);
        const uint32_t scw = s < 2 ? sc.sc_lo : sc.sc_hi, mw = s < 2 ? sc.m_lo : sc.m_hi;
        const int bi = 2 * (s & 1);
        dsc0 = d * static_cast<float>(byte_of(scw, bi));
        dsc1 = d * static_cast<float>(byte_of(scw, bi + 1));
        dm0 = dmin * static_cast<float>(byte_of(mw, bi));
        dm1 = dmin * static_cast<float>(byte_of(mw, bi + 1));
        const uint32_t w[8] = {fb.x, fb.y, fb.z, fb.w, fc.x, fc.y, fc.z, fc.w};
#pragma unroll
        for (int i = 0; i < 8; i++) {
          lo[i] = w[i] & 0x0F0F0F0Fu;
          hi[i] = (w[i] >> 4) & 0x0F0F0F0Fu;
        }
        }
        if (Q5) {  // bits 2s and 2s+1 of qh[l] are the fifth bits of values 64s + l and 64s + 32 + l
          const uint32_t qh[8] = {fe.x, fe.y, fe.z, fe.w, ff.x, ff.y, ff.z, ff.w};
#pragma unroll
          for (int i = 0; i < 8; i++) {
            lo[i] |= ((qh[i] >> (2 * s)) & 0x01010101u) << 4;
            hi[i] |= ((qh[i] >> (2 * s + 1)) & 0x01010101u) << 4;
          }
        }
        const int64_t b0 = 8 * jb + 2 * s;
#pragma unroll
        for (int m = 0; m < MR; m++) {
          uint4 x0, x1, x2, x3;
          float dx0, dx1, dS0, dS1;
          if constexpr (XM == kXReg) {
            x0 = xr[m][0]; x1 = xr[m][1]; x2 = xr[m][2]; x3 = xr[m][3];
            dx0 = xdr[m][0]; dx1 = xdr[m][1]; dS0 = xdr[m][2]; dS1 = xdr[m][3];
          } else {
            const uint4* xv = reinterpret_cast<const uint4*>(xs + m * xk + 256 * (jb - xj0) + 64 * s);
            x0 = xv[0]; x1 = xv[1]; x2 = xv[2]; x3 = xv[3];
            const float2 dxv = *reinterpret_cast<const float2*>(xd + m * xnb + b0 - 8 * xj0);
            const float2 dSv = *reinterpret_cast<const float2*>(xS + m * xnb + b0 - 8 * xj0);
            dx0 = dxv.x; dx1 = dxv.y; dS0 = dSv.x; dS1 = dSv.y;
          }
          int I0 = dot4(lo[0], x0.x, 0);
          I0 = dot4(lo[1], x0.y, I0); I0 = dot4(lo[2], x0.z, I0); I0 = dot4(lo[3], x0.w, I0);
          I0 = dot4(lo[4], x1.x, I0); I0 = dot4(lo[5], x1.y, I0); I0 = dot4(lo[6], x1.z, I0);
          I0 = dot4(lo[7], x1.w, I0);
          int I1 = dot4(hi[0], x2.x, 0);
          I1 = dot4(hi[1], x2.y, I1); I1 = dot4(hi[2], x2.z, I1); I1 = dot4(hi[3], x2.w, I1);
          I1 = dot4(hi[4], x3.x, I1); I1 = dot4(hi[5], x3.y, I1); I1 = dot4(hi[6], x3.z, I1);
          I1 = dot4(hi[7], x3.w, I1);
          float a = acc[m];
          a = __builtin_fmaf(static_cast<float>(I0), dsc0 * dx0, a);
          a = __builtin_fmaf(static_cast<float>(I1), dsc1 * dx1, a);
          if constexpr (!Q8) {
            a = __builtin_fmaf(-dm0, dS0, a);
            a = __builtin_fmaf(-dm1, dS1, a);
          }
          acc[m] = valid ? a : acc[m];
        }
      } else {
        // scales sc[8half .. 8half+7] as two dwords and d, from the quad's
        // loads: lane 1 takes sc[0..3] from lane 0, lane 3 sc[8..11] from
        // lane 2 and realigns sc[12..15] from its own bytes 202..209; d is
        // the top half of lane 3's second dword
        const uint32_t nb0 = static_cast<uint32_t>(
            __builtin_amdgcn_update_dpp(0, static_cast<int>(fs0), 0xA0, 0xF, 0xF, false));
        const uint32_t dq = static_cast<uint32_t>(
            __builtin_amdgcn_update_dpp(0, static_cast<int>(fs1), 0xFF, 0xF, 0xF, false));
        const float d = half_to_float(dq >> 16);
        const uint32_t s0 = (s & 1) ? nb0 : fs0;
        const uint32_t s1 = s == 1 ? fs0 : s == 3 ? __builtin_amdgcn_alignbyte(fs1, fs0, 2) : fs1;
        float dsc[4];
#pragma unroll
        for (int c = 0; c < 4; c++) {
          const uint32_t sw = c < 2 ? s0 : s1;
          dsc[c] = d * static_cast<float>(static_cast<int8_t>(byte_of(sw, (2 * c + lh) & 3)));
        }
        const uint32_t l0[4] = {fa.x, fa.y, fa.z, fa.w};
        const uint32_t l1[4] = {fb.x, fb.y, fb.z, fb.w};
        const uint32_t hh[4] = {fc.x, fc.y, fc.z, fc.w};
        uint32_t q[4][4];  // codes q6 in [0, 63], quarter c, dword i
#pragma unroll
        for (int i = 0; i < 4; i++) {
          q[0][i] = (l0[i] & 0x0F0F0F0Fu) | ((hh[i] << 4) & 0x30303030u);
          q[1][i] = (l1[i] & 0x0F0F0F0Fu) | ((hh[i] << 2) & 0x30303030u);
          q[2][i] = ((l0[i] >> 4) & 0x0F0F0F0Fu) | (hh[i] & 0x30303030u);
          q[3][i] = ((l1[i] >> 4) & 0x0F0F0F0Fu) | ((hh[i] >> 2) & 0x30303030u);
        }
        const int64_t b0 = 8 * jb + 4 * half;
#pragma unroll
        for (int m = 0; m < MR; m++) {
          float dxs[4];
          if constexpr (XM != kXReg) {
            const float4 dxv = *reinterpret_cast<const float4*>(xd + m * xnb + b0 - 8 * xj0);
            dxs[0] = dxv.x; dxs[1] = dxv.y; dxs[2] = dxv.z; dxs[3] = dxv.w;
          }
          float a = acc[m];
#pragma unroll
          for (int c = 0; c < 4; c++) {
            uint4 xv;
            int I;
            float dxc;
            if constexpr (XM == kXReg) {
              xv = xr[m][c];
              I = xur[m][c];
              dxc = xdr[m][c];
            } else {
              xv = *reinterpret_cast<const uint4*>(xs + m * xk + 256 * (jb - xj0) + 128 * half + 16 * lh + 32 * c);
              I = -32 * sum16(xv);
              dxc = dxs[c];
            }
            I = dot4(q[c][0], xv.x, I);
            I = dot4(q[c][1], xv.y, I);
            I = dot4(q[c][2], xv.z, I);
            I = dot4(q[c][3], xv.w, I);
            a = __builtin_fmaf(static_cast<float>(I), dsc[c] * dxc, a);
          }
          acc[m] = valid ? a : acc[m];
        }
      }
    }
    // end of a row (all its steps done): reduce over the row's lanes and store
    if (it == ipr - 1) {
#pragma unroll
      for (int m = 0; m < MR; m++) {
        const float v = group_sum_last<G>(acc[m]);
        acc[m] = 0.0f;
        if ((lane & (G - 1)) == G - 1 && n < N) y[m * N + n] = v;
      }
    }
  };

  if constexpr (XM == kXSlice) {
    static_assert(R == 1 && CO == kCoNone, "slices of rows of one step or more");
    int8_t* lq = reinterpret_cast<int8_t*>(smem);
    float* ld = reinterpret_cast<float*>(smem + MR * 4096);
    float* lS = ld + MR * 128;
    xs = lq;
    xd = ld;
    xS = lS;
    xk = 4096;
    xnb = 128;
    // this wavefront's rows, and the most rows any wavefront of the grid has
    // (every wavefront runs that many chunks, so all meet the same barriers)
    const int64_t my_rows = row_begin < N ? (N - row_begin + stride - 1) / stride : 0;
    const int64_t grid_rows = (N + stride - 1) / stride;
    for (int64_t c0 = 0; c0 < grid_rows; c0 += kSlRows) {
      const int64_t nr = my_rows - c0;  // rows of this chunk (<= 0: none)
      float accr[kSlRows][MR];
#pragma unroll
      for (int r = 0; r < kSlRows; r++)
#pragma unroll
        for (int m = 0; m < MR; m++) accr[r][m] = 0.0f;
      for (int64_t it = 0; it < ipr; it++) {
        SkRaw ra = {}, rb = {};
        __syncthreads();  // no wavefront reads the previous slice any more
        if (nr > 0) load(c0, it, ra);  // in flight while the slice is staged
        // slice it: super-blocks 16 it .. 16 it + 15 (fewer in the last) of
        // each activation row: codes [MR][4096], scales (and dS) [MR][128]
        const int64_t q0 = 4096 * it, qn = K - q0 < 4096 ? K - q0 : 4096;
        for (int i = threadIdx.x; i < MR * 256; i += TH) {
          const int m = i >> 8, c16 = i & 255;
          if (16 * c16 < qn)
            reinterpret_cast<uint4*>(lq + m * 4096)[c16] = reinterpret_cast<const uint4*>(qx + m * K + q0)[c16];
        }
        for (int i = threadIdx.x; i < MR * 32; i += TH) {
          const int m = i >> 5, c4 = i & 31;
          if (4 * c4 < qn / 32) {
            reinterpret_cast<float4*>(ld + m * 128)[c4] = reinterpret_cast<const float4*>(gdx + m * nb + q0 / 32)[c4];
            if (KQ)
              reinterpret_cast<float4*>(lS + m * 128)[c4] = reinterpret_cast<const float4*>(gdS + m * nb + q0 / 32)[c4];
          }
        }
        __syncthreads();
        xj0 = 16 * it;
        // the chunk's rows, the next one's loads issued before this one is computed
#pragma unroll
        for (int r = 0; r < kSlRows; r++) {
          if (r >= nr) break;
          if (r + 1 < nr && r + 1 < kSlRows) load(c0 + r + 1, it, (r & 1) ? ra : rb);
#pragma unroll
          for (int m = 0; m < MR; m++) acc[m] = accr[r][m];
          compute(c0 + r, it, (r & 1) ? rb : ra);  // stores the row after its last slice
#pragma unroll
          for (int m = 0; m < MR; m++) accr[r][m] = acc[m];
        }
      }
    }
    return;
  }

  // two register buffers in turn: the loads of step t+1 are issued before
  // step t is computed
  auto advance = [&](int64_t& rs, int64_t& it) {
    if (++it == ipr) {
      it = 0;
      ++rs;
    }
  };
  // The loads are issued unconditionally (past the last step they re-read a
  // clamped, valid block), so the compiler's wait before each step counts
  // exactly the next step's loads and leaves them in flight.
  SkRaw r0 = {}, r1 = {};
  if constexpr (CO == kCoDma) r1.s0 = 1;  // LDS buffer of each register set
  int64_t rs0 = 0, it0 = 0;
  load(rs0, it0, r0);
  for (int64_t t = 0; t < nsteps; t += 2) {
    int64_t rs1 = rs0, it1 = it0;
    advance(rs1, it1);
    load(rs1, it1, r1);
    compute(rs0, it0, r0);
    if (t + 1 >= nsteps) break;
    rs0 = rs1;
    it0 = it1;
    advance(rs0, it0);
    load(rs0, it0, r0);
    compute(rs1, it1, r1);
  }
}

// rows per wavefront step for K (16 / super-blocks per row when that divides)
inline int skinny_rows_per_step(int64_t K) {
  const int64_t nsb = K / 256;
  return (nsb == 1 || nsb == 2 || nsb == 4 || nsb == 8) ? static_cast<int>(16 / nsb) : 1;
}

inline int64_t skinny_lds_bytes(int fmt, int64_t M, int64_t K) {
  return fmt != QG_Q6_K ? M * K + 2 * M * (K / 32) * 4 : M * K + M * (K / 32) * 4;
}

// Rows of K <= 4096: registers for one or two activation rows, for short
// rows (K <= 2048, several rows per step) and when every wavefront takes many
// rows (N > 16384), which pays for loading 3-8 rows x 64 values per lane once
// (the M = 8 LM head: 179 us, against 217 us from LDS); otherwise LDS, where
// registers would hold those values for a row or two at one or two
// wavefronts per SIMD (up to 256 VGPRs: Q6_K 4096->2560 at M = 8 11.5 ->
// 8.6 us, Q4_K 2560->9728 at M = 4 11.3 -> 8.0 us).  Longer rows: LDS, or
// global memory (L2) when they do not fit.
inline int skinny_xmode(int fmt, int64_t M, int64_t N, int64_t K) {
  if (K <= 4096 && (M <= 2 || K <= 2048 || N > 16384)) return kXReg;
  if (skinny_lds_bytes(fmt, M, K) <= kSkMaxLds) return kXLds;
  return K <= 4096 ? kXReg : kXSlice;
}

// Launch shapes measured against the default of 256-thread workgroups (Q4_K
// and Q6_K matrices of one row per wavefront step, cold weights; every shape
// gives the same bits).  Where each workgroup stages long activation rows in
// LDS, fewer and larger workgroups stage them fewer times and still hold 16
// wavefronts per CU: one of 1024 threads per CU (12288->4096 Q6_K at M = 2 /
// 3 / 4: 13.7 -> 12.3, 17.4 -> 13.2, 18.9 -> 14.2 us; 9728->2560 Q4_K at
// M = 5 11.6 -> 10.6, M = 2-4 within 1%); two of 512 threads for rows of
// K <= 4096 over many weight rows (2560->9728 Q4_K at M = 3-6: 2-3%) and
// for 4096-value slices over a multiple of 4096 weight rows from six
// activation rows (12288->4096 Q6_K at M = 6 / 7 / 8: 22.5 -> 21.8, 24.8 ->
// 24.1, 27.2 -> 25.6 us; at M = 5 0.5-1.3% slower).
// The same kinds of shapes elsewhere (4096->2560 Q6_K from three activation
// rows, 3584->1024 Q4_K, 9728->2560 Q4_K in slices, 12288->4096 Q6_K at
// M = 1 and in slices at M = 5) measured no faster or slower and keep the
// default; so do Q5_K and Q8_0 outside the 512-thread plan for rows of
// K <= 4096 (the 1024-thread plan measured mixed on them).
enum class SkPlan { kDefault, k1024x1, k512x2, k512x1, k256x2 };

// Q6_K steps that start on 16-byte boundaries (several rows per step, or rows
// of a multiple of 8 super-blocks) in a matrix of whole 16-byte chunks: where
// the coalesced loads can run
inline bool skinny_aligned(int fmt, int64_t N, int64_t K) {
  const int64_t nsb = K / 256;
  return fmt == QG_Q6_K && (skinny_rows_per_step(K) > 1 || nsb % 8 == 0) && (N * nsb) % 8 == 0;
}

inline SkPlan skinny_plan(int fmt, int64_t M, int64_t N, int64_t K) {
  if (skinny_rows_per_step(K) != 1) return SkPlan::kDefault;
  const int xm = skinny_xmode(fmt, M, N, K);
  // (Q5_K and Q8_0 too: 2560->9728 at M = 3-8 2.4-5% faster)
  if (xm == kXLds && K <= 4096 && N >= 8192) return SkPlan::k512x2;
  if (fmt != QG_Q4_K && fmt != QG_Q6_K) return SkPlan::kDefault;
  if (xm == kXLds && K > 4096 && M >= 2 && N >= 2048) return SkPlan::k1024x1;
  if (xm == kXSlice && N % 4096 == 0 && M >= 6) return SkPlan::k512x2;
  // Q6_K rows with the activations in registers over at most 16384 weight
  // rows, one or two activation rows: field loads and two workgroups per CU,
  // not the coalesced loads (4096->2560 at M = 1 / 2: 5.09 -> 4.49, 5.87 ->
  // 4.88 us)
  if (fmt == QG_Q6_K && xm == kXReg && M <= 2 && N <= 16384) return SkPlan::k256x2;
  // Q6_K rows with the activations in registers over more than 16384 weight
  // rows (the LM head) from five activation rows, with the coalesced loads
  // through registers: one 512-thread workgroup per CU (4096->152064 at
  // M = 8 175.6 -> 164.6 and 177.1 -> 165.2 us, M = 5 / 6 1-2.5%, M = 7
  // within 1%)
  if (xm == kXReg && M >= 5 && N > 16384 && skinny_aligned(fmt, N, K)) return SkPlan::k512x1;
  return SkPlan::kDefault;
}

inline int skinny_threads(int fmt, int64_t M, int64_t N, int64_t K) {
  switch (skinny_plan(fmt, M, N, K)) {
    case SkPlan::k1024x1: return 1024;
    case SkPlan::k512x2:
    case SkPlan::k512x1: return 512;
    default: return 256;
  }
}

// Q6_K coalesced loads (CO) where the steps are aligned (skinny_aligned) and
// the activations sit in registers (with them in LDS or L2, measured slower):
// straight into LDS for up to two activation rows, through registers above
inline int skinny_coalesced(int fmt, int64_t M, int64_t N, int64_t K) {
  if (!skinny_aligned(fmt, N, K) || skinny_xmode(fmt, M, N, K) != kXReg ||
      skinny_plan(fmt, M, N, K) == SkPlan::k256x2)
    return kCoNone;
  return M <= 2 ? kCoDma : kCoReg;
}

// Workgroups of a skinny kernel that one CU holds at once (its registers and
// static LDS; the caller counts the activation rows in dynamic LDS), from the
// runtime's occupancy calculator, once per kernel.
template <int FMT, int MR, int R, int XM, int CO, int TH>
static int64_t skinny_resident() {
  static const int64_t n = [] {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, skinny_kernel<FMT, MR, R, XM, CO, TH>, TH, 0) !=
            hipSuccess || b < 1) {
      (void)hipGetLastError();  // unknown: no limit from it
      return int64_t{1} << 20;
    }
    return static_cast<int64_t>(b);
  }();
  return n;
}

template <int FMT, int MR, int R, int CO, int TH>
static hipError_t launch_skinny_rc(const uint8_t* W, const QgWorkspace& ws, int64_t N, int64_t K,
                                   float* y, hipStream_t stream) {
  // The same number of workgroups on every CU, all resident at once, and the
  // row groups dealt to the wavefronts in turn, so that no wavefront takes
  // more than one row group more than another: a CU with one workgroup more
  // than the rest sets the end of the launch (the LM head ran 104 us with 827
  // workgroups, 3 or 4 per CU, against 86 us with 768).  For 256-thread
  // workgroups: three per CU for the coalesced Q6_K loads (32 KB of LDS row
  // buffers each); two for rows of several steps with the activations staged
  // in LDS when that deals every wavefront the same number of rows
  // (12288->4096 Q6_K: two rows each, 11.8 -> 11.1 us; 9728->2560 Q4_K,
  // uneven at two, runs 6.4 us there and 5.9 at four); four otherwise (the LM
  // head 90 -> 86 us, 2560->9728 Q4_K 6.4 -> 5.7 us; one-step rows measured
  // slower at two); never more than the LDS holds at once; fewer workgroups
  // when there are fewer row groups than wavefronts, and never more than the
  // CU holds at once by its registers: the workgroups past that run as a
  // second, partial round (the LM head at M = 3 / 4, 130 and 154 VGPRs, three
  // 256-thread workgroups per CU: 124.9 -> 105.6 and 128.9 -> 112.8 us
  // against four).  Other workgroup sizes and counts per skinny_plan.
  constexpr int64_t kCUs = 256, kLdsPerCU = 160 * 1024, WPG = TH / 64;
  const int64_t row_groups = (N + R - 1) / R;
  const int xm = skinny_xmode(FMT, MR, N, K);
  const bool xlds = xm == kXLds;
  const int64_t xbytes = xm == kXLds ? skinny_lds_bytes(FMT, MR, K) : xm == kXSlice ? skinny_lds_bytes(FMT, MR, 4096) : 0;
  const int64_t lds = (CO == kCoNone ? 0 : WPG * (CO == kCoDma ? 2 : 1) * 4096) + xbytes;
  int64_t per_cu;
  switch (skinny_plan(FMT, MR, N, K)) {
    case SkPlan::k1024x1:
    case SkPlan::k512x1: per_cu = 1; break;
    case SkPlan::k512x2:
    case SkPlan::k256x2: per_cu = 2; break;
    default: per_cu = CO == kCoDma ? 3 : xlds && K > 4096 && row_groups % (WPG * kCUs * 2) == 0 ? 2 : 4;
  }
  if (lds > 0 && per_cu > kLdsPerCU / lds) per_cu = kLdsPerCU / lds > 0 ? kLdsPerCU / lds : 1;
  auto grid = [&](int64_t resident) {
    const int64_t pc = per_cu < resident ? per_cu : resident;
    return dim3(static_cast<unsigned>(row_groups < WPG * kCUs * pc ? (row_groups + WPG - 1) / WPG : kCUs * pc));
  };
  // (skinny_plan takes 1024 threads only with whole rows in LDS, 512 with
  // staged activations or, for Q6_K, with coalesced loads through registers;
  // other combinations are not built)
  switch (xm) {
    case kXReg:
      if constexpr (TH == 256 || (TH == 512 && CO == kCoReg))
        skinny_kernel<FMT, MR, R, kXReg, CO, TH><<<grid(skinny_resident<FMT, MR, R, kXReg, CO, TH>()), dim3(TH), 0,
                                                   stream>>>(W, ws.q, ws.dx, ws.dS, N, K, y);
      else
        return hipErrorInvalidValue;
      break;
    case kXLds:
      if constexpr (TH == 256 || CO == kCoNone)
        skinny_kernel<FMT, MR, R, kXLds, CO, TH>
            <<<grid(skinny_resident<FMT, MR, R, kXLds, CO, TH>()), dim3(TH),
               static_cast<size_t>(skinny_lds_bytes(FMT, MR, K)), stream>>>(W, ws.q, ws.dx, ws.dS, N, K, y);
      else
        return hipErrorInvalidValue;
      break;
    default:  // kXSlice: rows of K > 4096, one row per step, no coalesced loads
      if constexpr (R == 1 && CO == kCoNone && TH <= 512)
        skinny_kernel<FMT, MR, R, kXSlice, CO, TH><<<grid(skinny_resident<FMT, MR, R, kXSlice, CO, TH>()), dim3(TH),
                                                     static_cast<size_t>(xbytes), stream>>>(W, ws.q, ws.dx, ws.dS,
                                                                                              N, K, y);
      else
        return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int FMT, int MR, int R, int CO>
static hipError_t launch_skinny_co(const uint8_t* W, const QgWorkspace& ws, int64_t N, int64_t K,
                                   float* y, hipStream_t stream) {
  if constexpr (R == 1) {
    const int th = skinny_threads(FMT, MR, N, K);
    if constexpr (CO == kCoNone) {
      if constexpr (FMT == QG_Q4_K || FMT == QG_Q6_K)
        if (th == 1024) return launch_skinny_rc<FMT, MR, R, CO, 1024>(W, ws, N, K, y, stream);
      if (th == 512) return launch_skinny_rc<FMT, MR, R, CO, 512>(W, ws, N, K, y, stream);
    } else if constexpr (CO == kCoReg) {
      if (th == 512) return launch_skinny_rc<FMT, MR, R, CO, 512>(W, ws, N, K, y, stream);
    }
  }
  return launch_skinny_rc<FMT, MR, R, CO, 256>(W, ws, N, K, y, stream);
}

template <int FMT, int MR, int R>
static hipError_t launch_skinny_r(const uint8_t* W, const QgWorkspace& ws, int64_t N, int64_t K,
                                  float* y, hipStream_t stream) {
  if constexpr (FMT == QG_Q6_K) {
    switch (skinny_coalesced(FMT, MR, N, K)) {
      case kCoDma: return launch_skinny_co<FMT, MR, R, kCoDma>(W, ws, N, K, y, stream);
      case kCoReg: return launch_skinny_co<FMT, MR, R, kCoReg>(W, ws, N, K, y, stream);
      default: break;
    }
  }
  return launch_skinny_co<FMT, MR, R, kCoNone>(W, ws, N, K, y, stream);
}

template <int FMT, int MR>
static hipError_t launch_skinny(const uint8_t* W, const QgWorkspace& ws, int64_t N, int64_t K,
                                float* y, hipStream_t stream) {
  switch (K / 256) {
    case 1: return launch_skinny_r<FMT, MR, 16>(W, ws, N, K, y, stream);
    case 2: return launch_skinny_r<FMT, MR, 8>(W, ws, N, K, y, stream);
    case 4: return launch_skinny_r<FMT, MR, 4>(W, ws, N, K, y, stream);
    case 8: return launch_skinny_r<FMT, MR, 2>(W, ws, N, K, y, stream);
    default: return launch_skinny_r<FMT, MR, 1>(W, ws, N, K, y, stream);
  }
}

template <int FMT>
static hipError_t launch_skinny_fmt(const uint8_t* W, const QgWorkspace& ws, int64_t M, int64_t N,
                                    int64_t K, float* y, hipStream_t stream) {
  switch (M) {
    case 1: return launch_skinny<FMT, 1>(W, ws, N, K, y, stream);
    case 2: return launch_skinny<FMT, 2>(W, ws, N, K, y, stream);
    case 3: return launch_skinny<FMT, 3>(W, ws, N, K, y, stream);
    case 4: return launch_skinny<FMT, 4>(W, ws, N, K, y, stream);
    case 5: return launch_skinny<FMT, 5>(W, ws, N, K, y, stream);
    case 6: return launch_skinny<FMT, 6>(W, ws, N, K, y, stream);
    case 7: return launch_skinny<FMT, 7>(W, ws, N, K, y, stream);
    case 8: return launch_skinny<FMT, 8>(W, ws, N, K, y, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qg

const char* qg_gemm_skinny_kernel_name(int fmt, int64_t M, int64_t N, int64_t K) {
  thread_local char name[64];
  if (M < 1 || M > QG_SKINNY_MAX_M) return "?";
  snprintf(name, sizeof name, "skinny_kernel<%d, %d, %d, %d, %d, %d>", fmt, static_cast<int>(M),
           qg::skinny_rows_per_step(K), qg::skinny_xmode(fmt, M, N, K),
           qg::skinny_coalesced(fmt, M, N, K), qg::skinny_threads(fmt, M, N, K));
  return name;
}

hipError_t qg_launch_gemm_skinny(const uint8_t* W, int fmt, const QgWorkspace& ws, int64_t M,
                                 int64_t N, int64_t K, float* y, hipStream_t stream) {
  if (fmt == QG_Q4_K) return qg::launch_skinny_fmt<QG_Q4_K>(W, ws, M, N, K, y, stream);
  if (fmt == QG_Q5_K) return qg::launch_skinny_fmt<QG_Q5_K>(W, ws, M, N, K, y, stream);
  if (fmt == QG_Q8_0) return qg::launch_skinny_fmt<QG_Q8_0>(W, ws, M, N, K, y, stream);
  return qg::launch_skinny_fmt<QG_Q6_K>(W, ws, M, N, K, y, stream);
}
