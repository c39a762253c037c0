// Device-side definitions shared by the gfx950 kernels of libsherry.
//
// Format (see include/sherry.h): 5-bit code c = 2*p + s per 4-weight block;
// tiles of 64 rows x 128 columns, 1280 bytes, row-tile-major.  Tile row
// r = 16t + i keeps its 32 codes as four 40-bit groups (group g = blocks
// 8g..8g+7); the group belongs to slot L = 16g + i, which holds its low 32
// bits as dword t of 16 bytes at 16L and its high 8 bits as byte t of the
// dword at 1024 + 4L.  A wave loading slot L per lane (16 + 4 bytes) thus
// holds in lane (i, g) block g's group of rows i, 16 + i, 32 + i, 48 + i:
// the operand layout of the matrix-core kernels, with no lane exchange.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sherry {

constexpr int kTileRows = 64;     // rows per format tile (one per wave lane)
constexpr int kTileK = 128;       // weights per row per tile (32 blocks)
constexpr int kTileBytes = 1280;  // 64 rows * 32 codes * 5 bits / 8
constexpr int kTileHiOff = 1024;  // byte offset of the groups' high bytes

// Tiles of an [N,K] matrix: padded to whole 64-row x 128-column tiles whose
// extra blocks hold code 0 and are never used by a product.
__host__ __device__ constexpr int row_tiles(int N) { return (N + kTileRows - 1) / kTileRows; }
__host__ __device__ constexpr int k_tiles(int K) { return (K + kTileK - 1) / kTileK; }

// Value (-1, 0 or +1) at position j of the block whose code is c.  The
// pattern index p = c >> 1 names the zero position z = p >> 2 and whether
// the 2nd / 3rd nonzero (in position order) flips sign relative to the 1st;
// the low bit of c negates the whole block.  [Sherry page §2.1]
__host__ __device__ constexpr int code_value(int c, int j) {
  const int p = c >> 1, z = p >> 2;
  if (j == z) return 0;
  const int rank = j < z ? j : j - 1;  // 0,1,2 = order among the nonzeros
  const int flip = rank == 0 ? 0 : (rank == 1 ? (p >> 1) & 1 : p & 1);
  const int v = flip ? -1 : 1;
  return (c & 1) ? -v : v;
}

// The block of code c as 4 int8 lanes of a dword (byte j = position j),
// without branches: the three nonzeros' bytes (0x01 or 0xFF) in order, then
// a zero byte inserted at position z.
__host__ __device__ constexpr uint32_t code_word(uint32_t c) {
  const uint32_t s = c & 1u, r2 = (c >> 1) & 1u, r1 = (c >> 2) & 1u, z = (c >> 3) & 3u;
  const uint32_t n1 = s, n2 = s ^ r1, n3 = s ^ r2;          // 1 = negative
  const uint32_t v3 = (0x010101u | (n1 * 0xFEu) | (n2 * 0xFE00u) | (n3 * 0xFE0000u));
  const uint32_t below = (1u << (8u * z)) - 1u;             // bytes before z
  return (v3 & below) | ((v3 << 8) & ~(below | (0xFFu << (8u * z))));
}

// The closed form above agrees with the definition for all 32 codes.
__host__ __device__ constexpr bool code_word_matches_definition() {
  for (int c = 0; c < 32; ++c) {
    uint32_t w = 0;
    for (int j = 0; j < 4; ++j) w |= (uint32_t)(uint8_t)(int8_t)code_value(c, j) << (8 * j);
    if (w != code_word((uint32_t)c)) return false;
  }
  return true;
}
static_assert(code_word_matches_definition(), "code_word disagrees with code_value");

// 2-bit baseline format (the plain ternary packing the Sherry page compares
// its 5-bit code against, §2.1): 0 -> 00, +1 -> 01, -1 -> 11; tiles of 64
// rows x 128 columns, 2048 bytes, row-tile-major; weights 0..63 of tile
// row r (bits 0..127) at tile byte 16*r, weights 64..127 at 1024 + 16*r.
constexpr int kTile2Bytes = 2048;
constexpr int kTile2HiOff = 1024;

// Four 2-bit weights (one byte b) as 4 int8 lanes of a dword.
__host__ __device__ constexpr uint32_t code2_word(uint32_t b) {
  uint32_t w = 0;
  for (int i = 0; i < 4; ++i) {
    const uint32_t c = (b >> (2 * i)) & 3u;
    const uint32_t v = c == 0 ? 0u : (c == 1 ? 0x01u : 0xFFu);   // 10 is never written
    w |= v << (8 * i);
  }
  return w;
}

// 4 x 4 transpose of 16-lane rows: out[t] row g = in[g] row t.
__device__ __forceinline__ void transpose4(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3,
                                           uint32_t (&out)[4]) {
  // swap the upper 32 lanes of the first operand with the lower 32 of the second
  const auto s02 = __builtin_amdgcn_permlane32_swap(r0, r2, false, false);
  const auto s13 = __builtin_amdgcn_permlane32_swap(r1, r3, false, false);
  // swap the odd 16-lane rows of the first operand with the even rows of the second
  const auto t01 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
  const auto t23 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
  out[0] = t01[0];
  out[1] = t01[1];
  out[2] = t23[0];
  out[3] = t23[1];
}

// From a wave's slot loads (lane L: the 16 bytes at 16L in w[0..3], the
// dword at 1024 + 4L in w[4]) to one tile row per lane: lane r = 16t + i
// gets row r's four code groups, the low 32 bits of group g in lo[g] and
// its high 8 bits in byte g of hb.  Group g of row r is dword t and byte t
// of slot 16g + i, so the transpose of the four dwords brings lane r its
// groups' low words, and the transpose of w[4] the four dwords holding
// their high bytes, whose byte t two byte permutes gather.
__device__ __forceinline__ void row_groups(const uint32_t (&w)[5], int lane, uint32_t (&lo)[4],
                                           uint32_t& hb) {
  uint32_t hw[4];
  transpose4(w[0], w[1], w[2], w[3], lo);
  transpose4(w[4], w[4], w[4], w[4], hw);
  // v_perm_b32 selector bytes: 0..3 pick bytes of the second operand, 4..7
  // of the first, 12 gives zero
  const uint32_t t = (uint32_t)(lane >> 4);
  const uint32_t s01 = t | ((4u + t) << 8) | 0x0C0C0000u;
  const uint32_t s23 = 0x00000C0Cu | (t << 16) | ((4u + t) << 24);
  hb = __builtin_amdgcn_perm(hw[1], hw[0], s01) | __builtin_amdgcn_perm(hw[3], hw[2], s23);
}

// Code jj (0..7) of a 40-bit group held as lo (bits 0..31) and the low
// byte of hi (bits 32..39).  Called with a compile-time jj, so the branches
// fold.
__device__ __forceinline__ uint32_t group_code(uint32_t lo, uint32_t hi, int jj) {
  if (jj <= 5) return (lo >> (5 * jj)) & 31u;
  if (jj == 6) return __builtin_amdgcn_alignbit(hi, lo, 30) & 31u;
  return (hi >> 3) & 31u;
}

// x as read from another lane of its 16-lane row by DPP control CTRL.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, x),
                                                               __builtin_bit_cast(int, x), CTRL, 0xF,
                                                               0xF, false));
}

// Maximum over the 64 lanes of a wave, the same value in every lane (all
// lanes active).  Within each 16-lane row by DPP permutes (swap neighbours,
// swap pairs, rotate by 4, rotate by 8), then over the four rows' values
// read from one lane each.  A shuffle (ds_bpermute) would cost an LDS round
// trip per step; these are VALU operations.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_move<0xB1>(v));    // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_move<0x4E>(v));    // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_move<0x124>(v));   // row_ror:4
  v = fmaxf(v, dpp_move<0x128>(v));   // row_ror:8
  const int u = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Workgroup barrier that orders only LDS accesses.  __syncthreads() also
// orders global memory, so it waits for every global load in flight; this
// one leaves prefetched loads outstanding across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Byte offset of format tile (rt, kt) for a matrix with K columns.
__device__ __forceinline__ size_t tile_offset(int rt, int kt, int KT) {
  return ((size_t)rt * (size_t)KT + (size_t)kt) * (size_t)kTileBytes;
}

}  // namespace sherry
