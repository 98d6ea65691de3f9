// LDS tile machinery shared by the bf16 MFMA attention kernels (forward and
// backward): tile geometry per head size, the 16-byte chunk swizzle, buffer
// DMA of 64-row tiles from HBM into LDS, and the operand offsets of the two
// ways a tile is read (rows as a 32x32x16 MFMA operand, or transposed on the
// way out of LDS).
#pragma once

#include "common.h"

namespace attn {

constexpr int BN = 64;  // rows (keys, or queries) per tile

typedef __attribute__((address_space(3))) void lds_void;
typedef short i16x4 __attribute__((ext_vector_type(4)));

// Tile geometry for head size D (64, 128 or 256).  A row is RB = 2*D bytes =
// NC 16-byte chunks; a tile of BN rows is NP pieces of 1 KB, RP rows each.  A
// 32x32x16 product over the head takes KS 16-wide slices; a product whose
// output runs along the head yields DB 32-wide blocks.
template <int D>
struct Geo {
  static constexpr int RB = 2 * D;
  static constexpr int NC = D / 8;
  static constexpr int TILE = BN * RB;
  static constexpr int NP = TILE / 1024;
  static constexpr int RP = 1024 / RB;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
};


// 16-byte chunk c of tile row r is stored at chunk position c ^ swz<D>(r).
// Both are GF(2)-linear in the row bits, chosen (by exhaustive check of
// every read instruction's lanes) so that the 16-byte K operand reads and
// the transposing V reads hit distinct banks: row bits 0..3 map to chunk
// bits 4, 10, 1, 8 for 256- and 512-byte rows, and to 2, 4, 1, 2 for 128-byte
// rows.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 64)
    return ((r & 1) << 1) ^ (((r >> 1) & 1) << 2) ^ ((r >> 2) & 1) ^ (((r >> 3) & 1) << 1);
  else
    return ((r & 1) << 2) ^ (((r >> 1) & 1) * 10) ^ ((r >> 2) & 1) ^ (r & 8);
}

__device__ __forceinline__ void wait_dma() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
}

// Copy keys [k0, k0+64) of one head (a buffer resource over the head) into a
// swizzled LDS tile.  The tile is NP pieces of 1 KB (RP rows); wave w issues
// pieces w, w + NW, ...  The whole offset is in the per-lane operand, which the
// buffer range check covers: rows past the end of the head read as zero.
struct HeadRef {
  __amdgpu_buffer_rsrc_t rs;
};
template <int D>
__device__ __forceinline__ HeadRef head_ref(const __bf16* head, int rows) {
  return HeadRef{__builtin_amdgcn_make_buffer_rsrc((void*)head, (short)0, rows * D * 2, 0x00020000)};
}
template <int D, int NW>
__device__ __forceinline__ void load_tile(HeadRef h, int k0, char* tile, int w, int lane) {
  // The buffer-resource builtin exists only for the GPU target.  The host
  // pass of a translation unit that instantiates one kernel twice (with and
  // without a key mask) would otherwise reject this body, so it only sees an
  // empty one; the host never runs device functions.
#if defined(__HIP_DEVICE_COMPILE__)
  using g = Geo<D>;
#pragma unroll
  for (int j = 0; j < (g::NP + NW - 1) / NW; ++j) {
    const int piece = w + j * NW;  // wave-uniform
    // with NP a multiple of NW every wave issues the same copies, with no
    // branch the compiler would have to count around
    if (g::NP % NW != 0 && piece >= g::NP) break;
    const int r = piece * g::RP + lane / g::NC;
    const int voff = r * g::RB + (((lane % g::NC) ^ swz<D>(r)) << 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(h.rs, (lds_void*)(tile + piece * 1024), 16,
                                             voff + k0 * g::RB, 0, 0, 0);
  }
#endif
}

__device__ __forceinline__ float xhalf_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Byte offsets inside a tile for lane (ln = lane % 32, hl = lane / 32).
// Row operand: 16 bytes of row ln (+32 per row block), chunk 2*ks + hl, i.e.
// the A (or B) operand of a 32x32x16 product over the head dimension.
template <int D>
__device__ __forceinline__ void row_operand_offsets(int ln, int hl, int (&off)[Geo<D>::KS]) {
  // the swizzle changes chunk bits 0..3 only: in 512-byte rows the upper 16
  // chunks sit at the lower 16's offsets + 256 (a constant the reads fold in)
  constexpr int H = D == 256 ? Geo<D>::KS / 2 : Geo<D>::KS;
#pragma unroll
  for (int ks = 0; ks < Geo<D>::KS; ++ks)
    off[ks] = ks < H ? ln * Geo<D>::RB + (((2 * ks + hl) ^ swz<D>(ln)) << 4) : off[ks - H] + 256;
}
// Transposed operand: two ds_read_b64_tr_b16 per 32-wide block db give the A
// operand of a product whose k index runs along the tile's rows (16 rows per
// k slice; the row order matches the 32x32 accumulator layout used as the B
// operand).
template <int D>
__device__ __forceinline__ void tr_operand_offsets(int lane, int (&off)[2][Geo<D>::DB]) {
  const int gq = lane >> 4, j = lane & 15;
  const int h = gq >> 1, dpart = gq & 1, ip = j >> 2, u = j & 3;
  constexpr int H = D == 256 ? Geo<D>::DB / 2 : Geo<D>::DB;  // as in row_operand_offsets
#pragma unroll
  for (int ih = 0; ih < 2; ++ih) {
    const int r = 8 * ih + 4 * h + ip;
#pragma unroll
    for (int db = 0; db < Geo<D>::DB; ++db)
      off[ih][db] = db < H ? r * Geo<D>::RB + (((4 * db + 2 * dpart + (u >> 1)) ^ swz<D>(r)) << 4) +
                                 (u & 1) * 8
                           : off[ih][db - H] + 256;
  }
}
// one transposed A operand (32 head dims of block db x 16 rows of slice kk)
template <int D>
__device__ __forceinline__ bf16x8 read_tr_operand(const char* tile, int kk, const int (&off)[2][Geo<D>::DB],
                                                  int db) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(tile + kk * 16 * Geo<D>::RB + off[0][db]));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(tile + kk * 16 * Geo<D>::RB + off[1][db]));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

}  // namespace attn
