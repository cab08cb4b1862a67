// LDS tile layout shared by the gfx950 attention kernels: 64-row bf16 tiles
// of a row-major [rows, D] matrix, moved HBM -> LDS by buffer loads that
// write LDS directly, stored with unpadded rows whose 16-byte chunks are
// XOR-swizzled by row.  The swizzle keeps both ways the kernels read a tile
// free of bank conflicts: rows as an MFMA A operand (8 consecutive dims of
// one row per lane, ds_read_b128), and columns through ds_read_b64_tr_b16
// (each 16-lane group gathers 4 rows x 4 dims and hands every lane one dim of
// the 4 rows), which yields the A operand of a product over the tile's rows.
#pragma once

#include "common.hpp"

namespace bea {

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_ptr;

// Chunk swizzle of row r.  D = 128 (16 chunks per row): 4 (r % 4) + (r / 4) % 4,
// so 16 consecutive rows and 4 consecutive rows x 4 chunk pairs each cover
// all 16 chunk positions.  D = 64 (8 chunks, two rows per 64 banks): the
// 3-bit reversal of (r / 2) % 8.
template <int D>
__device__ __forceinline__ uint32_t chunk_swz(uint32_t r) {
  if (D == 128) return ((r & 3u) << 2) | ((r >> 2) & 3u);
  const uint32_t x = (r >> 1) & 7u;
  return ((x & 1u) << 2) | (x & 2u) | ((x >> 2) & 1u);
}


// Per-lane LDS read addresses of the swizzled tiles.  The swizzle is an XOR
// on chunk bits, so every address is one base XOR an immediate.
//  * row read (A operand over dims), slice s: row col (+ 32 kb), chunk 2 s + half:
//      col * RB + 16 ((2 s + half) ^ swz(col)) = ka0 ^ (32 s).
//  * column read (A operand over rows), transposed read c of slice t for dim
//    block db: the lane addresses row 16 t + 8 c + 4 h + m and dims 32 db + 16 (G % 2) + 4 a .. +3,
//    with (G, a, m) = (lane / 16, lane % 4, (lane / 4) % 4) and h = G / 2:
//      D = 128: row*256 + 16 ((4 db + 2 g2 + a/2) ^ (4 m + (2 c ^ h))) + 8 (a & 1)
//             = 2048 c + (va0 ^ (64 db + 32 c)),  g2 = G % 2;
//      D = 64:  row*128 + 16 ((4 db + 2 g2 + a/2) ^ (4 (m/2) + 2 h + c)) + 8 (a & 1)
//             = 1024 c + (va0 ^ (64 db + 16 c)).
template <int D>
__device__ __forceinline__ void lds_read_bases(int lane, uint32_t& ka0, uint32_t& va0) {
  constexpr uint32_t RB = D * 2;
  const uint32_t col = (uint32_t)lane & 31u, half = (uint32_t)lane >> 5;
  ka0 = col * RB | ((half ^ chunk_swz<D>(col)) * 16u);
  const uint32_t G = (uint32_t)lane >> 4, a = (uint32_t)lane & 3u;
  const uint32_t mm = ((uint32_t)lane >> 2) & 3u, hh = G >> 1, g2 = G & 1u;
  const uint32_t z = D == 128 ? ((mm << 2) | ((2u * g2 + (a >> 1)) ^ hh))
                              : (((mm >> 1) << 2) | ((g2 ^ hh) << 1) | (a >> 1));
  va0 = (4u * hh + mm) * RB | (z * 16u) | ((a & 1u) * 8u);
}

// Global byte offset, within a 64-row tile, of the 16-byte chunk lane `lane`
// of wave `wave` (of 4) fetches in its first buffer load: the loads of one
// wave write whole rows (ROWS_PER_LOAD = 1024 / row bytes of them), row
// r = (4 x + wave) ROWS_PER_LOAD + lane / chunks for load x, and each lane
// fetches the logical chunk the swizzle places at its slot.
template <int D>
__device__ __forceinline__ uint32_t tile_lane_offset(int wave, int lane, uint32_t stride_b) {
  constexpr int CPR = D / 8;
  constexpr int ROWS_PER_LOAD = 1024 / (D * 2);
  const uint32_t row = (uint32_t)(wave * ROWS_PER_LOAD + lane / CPR);
  return row * stride_b + (((uint32_t)(lane % CPR)) ^ chunk_swz<D>(row)) * 16u;
}

// Rows [r0, r0 + 64) of a row-major bf16 matrix (row stride stride_b bytes,
// rows_left rows from r0 on exist; rows past them arrive as zeros) into the
// 64 x D LDS tile at dst, swizzled; this wave's share of the buffer loads.
// The caller waits for them (vmcnt) and publishes them with a barrier.
template <int D>
__device__ __forceinline__ void tile_dma(const uint16_t* base, long long r0, long long rows_left,
                                         uint32_t stride_b, unsigned char* dst, int wave,
                                         uint32_t lane_off) {
  constexpr int RB = D * 2;
  constexpr int ROWS_PER_LOAD = 1024 / RB;
  constexpr int LOADS = 64 / ROWS_PER_LOAD / 4;
  const long long bytes = max(0LL, min(rows_left * (long long)stride_b, 0x7fffffffLL));
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(base) + (size_t)r0 * (stride_b / 2), (short)0, (int)bytes,
      0x00020000);
#pragma unroll
  for (int x = 0; x < LOADS; ++x) {
    const int row0 = (x * 4 + wave) * ROWS_PER_LOAD;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)(dst + row0 * RB), 16, lane_off,
                                             (uint32_t)(x * 4 * ROWS_PER_LOAD) * stride_b, 0, 0);
  }
}

}  // namespace bea
