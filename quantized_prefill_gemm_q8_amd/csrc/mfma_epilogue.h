// Shared pieces of the int8-MFMA GEMM kernels: the 32x32 accumulator layout,
// the weight-fragment decoders and the fp32 scale epilogue with a
// DPP-broadcast activation scale.
//
// v_mfma_i32_32x32x32_i8 and v_mfma_i32_32x32x16_i8 split their K between the
// two lane halves; A (activations) and B (weights) use the same assignment of
// k to (lane half, byte), so any consistent assignment of a sub-block's values
// to bytes gives the same dot product.
#pragma once

#include "common.h"

namespace qg {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Row (0..31) of a 32x32 MFMA output tile held in accumulator element r by a
// lane in half h of the wave.
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Row whose activation scale a lane supplies for the DPP broadcast: lane k of
// each 16-lane DPP row holds the scale of element k's output row.
__device__ __forceinline__ int dpp_scale_row(int lane) { return acc_row(lane & 15, lane >> 5); }

// acc[r] += dxr(broadcast from lane r of this DPP row) * u[r], r = 0..15, with
// u[r] = fl(I[r] * dsc) from the magic-biased accumulator D.  v_fmac_f32 with a
// DPP row_newbcast:r source hands lane r's dxr of each 16-lane row to all lanes
// of that row, so one VGPR per lane carries the sixteen row scales of a tile.
// Each group of eight opens with the two wait states a DPP read needs after a
// VALU write of its source, inside the same statement, so nothing the
// compiler schedules falls between the wait and the reads.
__device__ __forceinline__ void epilogue_scale(float (&acc)[16], const v16i& D, float dsc, float cc,
                                               float dxr) {
  float u[16];
#pragma unroll
  for (int r = 0; r < 16; r++) u[r] = __builtin_fmaf(bits_to_float(D[r]), dsc, cc);  // fl(I*dsc)
  asm("s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %8, %9 row_newbcast:0 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %1, %8, %10 row_newbcast:1 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %2, %8, %11 row_newbcast:2 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %3, %8, %12 row_newbcast:3 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %4, %8, %13 row_newbcast:4 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %5, %8, %14 row_newbcast:5 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %6, %8, %15 row_newbcast:6 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %7, %8, %16 row_newbcast:7 row_mask:0xf bank_mask:0xf bound_ctrl:1"
      : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]), "+v"(acc[5]), "+v"(acc[6]),
        "+v"(acc[7])
      : "v"(dxr), "v"(u[0]), "v"(u[1]), "v"(u[2]), "v"(u[3]), "v"(u[4]), "v"(u[5]), "v"(u[6]),
        "v"(u[7]));
  asm("s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %8, %9 row_newbcast:8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %1, %8, %10 row_newbcast:9 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %2, %8, %11 row_newbcast:10 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %3, %8, %12 row_newbcast:11 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %4, %8, %13 row_newbcast:12 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %5, %8, %14 row_newbcast:13 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %6, %8, %15 row_newbcast:14 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %7, %8, %16 row_newbcast:15 row_mask:0xf bank_mask:0xf bound_ctrl:1"
      : "+v"(acc[8]), "+v"(acc[9]), "+v"(acc[10]), "+v"(acc[11]), "+v"(acc[12]), "+v"(acc[13]), "+v"(acc[14]),
        "+v"(acc[15])
      : "v"(dxr), "v"(u[8]), "v"(u[9]), "v"(u[10]), "v"(u[11]), "v"(u[12]), "v"(u[13]), "v"(u[14]),
        "v"(u[15]));
}

// Q4_K: the 16 codes of sub-block j (j = 2c or 2c+1) for lane half h.  Bytes
// qs[32c + 16h .. +15] hold sub-block 2c in their low nibbles and 2c+1 in their
// high nibbles; raw holds those 16 bytes.
__device__ __forceinline__ v4i q4_codes(const uint4& raw, int high) {
  const int sh = 4 * high;
  return v4i{int((raw.x >> sh) & 0x0F0F0F0Fu), int((raw.y >> sh) & 0x0F0F0F0Fu),
             int((raw.z >> sh) & 0x0F0F0F0Fu), int((raw.w >> sh) & 0x0F0F0F0Fu)};
}

// Q5_K: the fifth code bit of a lane's 16 values of sub-block jb -- bit jb of
// each of its 16 qh bytes (qh[16h .. 16h + 15] for lane half h) -- moved to
// bit 4 of each byte, to be or-ed into the nibble codes of q4_codes.
__device__ __forceinline__ v4i q5_high(const uint4& qh, int jb) {
  return v4i{int(((qh.x >> jb) & 0x01010101u) << 4), int(((qh.y >> jb) & 0x01010101u) << 4),
             int(((qh.z >> jb) & 0x01010101u) << 4), int(((qh.w >> jb) & 0x01010101u) << 4)};
}

// Q8_0 (a 256-value slice of a weight row = eight 34-byte blocks: fp16 d, then
// 32 int8 codes; the slice starts 16-byte aligned): the 16 codes of block jb
// for lane half h, bytes 34*jb + 2 + 16h onwards -- dword aligned for odd jb,
// two bytes past a dword for even jb (then read from the dwords around them
// and realigned).  Reads dwords only.
__device__ __forceinline__ v4i q8_codes(const uint8_t* row, int jb, int h) {
  const int off = 34 * jb + 2 + 16 * h;
  const uint32_t* p = reinterpret_cast<const uint32_t*>(row + (off & ~3));
  if ((off & 3) == 0) return v4i{int(p[0]), int(p[1]), int(p[2]), int(p[3])};
  const uint32_t w0 = p[0], w1 = p[1], w2 = p[2], w3 = p[3], w4 = p[4];
  return v4i{int(__builtin_amdgcn_alignbyte(w1, w0, 2)), int(__builtin_amdgcn_alignbyte(w2, w1, 2)),
             int(__builtin_amdgcn_alignbyte(w3, w2, 2)), int(__builtin_amdgcn_alignbyte(w4, w3, 2))};
}
// Q8_0: the scale d of block jb of such a slice.
__device__ __forceinline__ float q8_scale(const uint8_t* row, int jb) {
  const uint32_t w = *reinterpret_cast<const uint32_t*>(row + ((34 * jb) & ~3));
  return half_to_float((jb & 1) ? (w >> 16) : (w & 0xFFFFu));
}

// Q6_K: 8 codes, as signed bytes q6 - 32, of 16-value sub-block s for lane half
// h: values v = 16s + 8h + i, i < 8.  With half = s/8, quarter c = (s%8)/2 and
// l0 = 16*(s%2) + 8h, the low nibbles are ql[64*half + 32*(c%2) + l0 + i] (low
// nibble for c < 2, high for c >= 2) and the top two bits are bits (2c, 2c+1)
// of qh[32*half + l0 + i].  blk is the block's first byte in global memory.
__device__ __forceinline__ long q6_codes(const uint8_t* blk, int s, int h) {
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

}  // namespace qg
