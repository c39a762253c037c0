// Sherry 3:4-sparse ternary matmul -- CPU ORACLE.
//
// TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
// statement of what the Sherry hot path computes.  Only the tests, the smoke
// check and the benchmark's CPU-baseline leg may load it.  It shares no code,
// header, table or constant with the GPU library, and neither side includes
// the other.
//
// Source: the page "Sherry框架：三元量化与3:4稀疏优化LLM推理"
// (pnsm.cn/news/1195499.html), cited below as [Sherry §n]:
//   §1.1  ternary weights {-1,0,+1}; exactly 3 of every 4 weights nonzero.
//   §2.1  offline compression: 5 bits per 4-weight block (4-bit pattern
//         index + 1 sign bit), 1.25 bit/weight.
//   §2.2  online inference: activations cut into 4-element segments, one
//         table of 16 pattern dot products per segment, lookup, sign,
//         integer add tree and a single float multiply.
//   §3.1  per block: min ||W - aT||^2 s.t. T in {-1,0,1}^4, ||T||_0 = 3,
//         solved by keeping the 3 largest |w| with their signs.
//
// Readings where the page is silent (each is also listed in the design notes):
//   * alpha is one scale per output row, the least-squares value for the
//     fixed T: alpha = <W,T>/<T,T> = (sum of kept |w|) / (3*K/4).  Summed in
//     double in ascending k, one double divide, rounded once to float.
//   * ties at the minimum |w|: the LOWEST index is dropped.
//   * a kept w that is +0.0 or -0.0 gets +1 (the test is w < 0).
//   * canonical pattern: first nonzero is +1.  sign bit s = 1 iff the block's
//     first nonzero is -1.  Pattern index p = 4*z + 2*r1 + r2 with z the zero
//     position and r1 (r2) = 1 iff the 2nd (3rd) nonzero's sign differs from
//     the 1st's.  The stored 5-bit code is c = 2*p + s.
//   * activations: per-token symmetric int8, s = max|x|/127 (float),
//     q = clamp(rint(x/s), -127, 127); an all-zero row gives q = 0, s = 1.
//   * output: y = ((float)acc * s_x[m]) * alpha[n], float, round-to-nearest.
//
// Packed layout (the library's format; the oracle writes and reads it bit by
// bit): W is [N,K] row-major, K % 4 == 0.  The matrix is padded to Np =
// N rounded up to 64 rows and Kp = K rounded up to 128 columns; tiles of 64
// rows x 128 columns (32 blocks per row) are stored row-tile-major,
// column-tile minor, 1280 bytes each.  Tile row r = 16t + i (t = 0..3,
// i = 0..15) has its 32 codes in four groups of 8: group g (blocks
// 8g..8g+7) is a 40-bit little-endian string, block 8g+jj at bits
// [5jj, 5jj+5).  The group belongs to slot L = 16g + i: its bits 0..31 are
// the 4 bytes at tile byte 16*L + 4*t, its bits 32..39 the byte at tile
// byte 1024 + 4*L + t.  Blocks past K and rows past N hold code 0 (they
// carry no weights; a product never uses them).  Total Np*Kp*5/32 bytes.
//
// Build: g++ -std=c++17 -O2 -fno-fast-math -ffp-contract=off -shared -fPIC
// (liboracle.so, single-threaded).  The same source built with -fopenmp
// (liboracle_omp.so) runs the int32 product over all host cores; nothing
// else differs.

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

// Canonical pattern p as 4 values in {-1,0,+1}; first nonzero is +1.
// [Sherry §2.1, §2.2: the 16 patterns of exactly-3-nonzero blocks up to sign]
void pattern_of(int p, int out[4]) {
  const int z = p >> 2;          // position of the zero
  const int r1 = (p >> 1) & 1;   // 2nd nonzero flips sign relative to 1st
  const int r2 = p & 1;          // 3rd nonzero flips sign relative to 1st
  int nth = 0;
  for (int j = 0; j < 4; ++j) {
    if (j == z) { out[j] = 0; continue; }
    int v = 1;
    if (nth == 1 && r1) v = -1;
    if (nth == 2 && r2) v = -1;
    out[j] = v;
    ++nth;
  }
}

// Full block for a 5-bit code c = 2p + s.
void block_of_code(int c, int out[4]) {
  pattern_of(c >> 1, out);
  if (c & 1)
    for (int j = 0; j < 4; ++j) out[j] = -out[j];
}

// Code of a block with exactly 3 nonzeros in {-1,+1}; -1 if not such a block.
int code_of_block(const int t[4]) {
  int z = -1, nz = 0;
  int sgn[3] = {0, 0, 0};
  for (int j = 0; j < 4; ++j) {
    if (t[j] == 0) {
      if (z >= 0) return -1;
      z = j;
    } else if (t[j] == 1 || t[j] == -1) {
      if (nz >= 3) return -1;
      sgn[nz++] = t[j];
    } else {
      return -1;
    }
  }
  if (z < 0 || nz != 3) return -1;
  const int s = sgn[0] < 0 ? 1 : 0;
  const int r1 = sgn[1] != sgn[0] ? 1 : 0;
  const int r2 = sgn[2] != sgn[0] ? 1 : 0;
  const int p = 4 * z + 2 * r1 + r2;
  return 2 * p + s;
}

int64_t pad_to(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Byte offset of the tile holding (row n, block b) and the row's slot in it.
void tile_slot(int64_t n, int64_t b, int64_t K, int64_t* tile_base, int64_t* r,
               int* j) {
  const int64_t KT = pad_to(K, 128) / 128;
  const int64_t rt = n / 64, kt = b / 32;
  *tile_base = (rt * KT + kt) * 1280;
  *r = n % 64;
  *j = (int)(b % 32);
}

// Byte address and bit position of bit k (0..4) of the code of block j
// (0..31) of tile row r.
void code_bit(int64_t tile_base, int64_t r, int j, int k, int64_t* byte, int* bit) {
  const int64_t t = r / 16, i = r % 16, g = j / 8;
  const int p = 5 * (j % 8) + k;            // bit within the 40-bit group
  const int64_t slot = 16 * g + i;
  if (p < 32) {
    *byte = tile_base + 16 * slot + 4 * t + p / 8;
    *bit = p % 8;
  } else {
    *byte = tile_base + 1024 + 4 * slot + t;
    *bit = p - 32;
  }
}

}  // namespace

extern "C" {

// Pattern p (0..15) as 4 int8 values.
int oracle_pattern(int p, int8_t* out4) {
  if (p < 0 || p > 15) return -1;
  int v[4];
  pattern_of(p, v);
  for (int j = 0; j < 4; ++j) out4[j] = (int8_t)v[j];
  return 0;
}

// Block for code c (0..31).
int oracle_decode_code(int c, int8_t* out4) {
  if (c < 0 || c > 31) return -1;
  int v[4];
  block_of_code(c, v);
  for (int j = 0; j < 4; ++j) out4[j] = (int8_t)v[j];
  return 0;
}

// Code for a block; -1 if the block is not exactly-3-nonzero ternary.
int oracle_encode_block(const int8_t* t4) {
  int v[4] = {t4[0], t4[1], t4[2], t4[3]};
  return code_of_block(v);
}

// [Sherry §3.1] keep the three largest |w| of each block with their signs;
// per-row least-squares alpha.  T is [N,K] int8 in {-1,0,1}.
int oracle_quantize(const float* W, int64_t N, int64_t K, int8_t* T,
                    float* alpha) {
  if (N <= 0 || K <= 0 || K % 4 != 0) return -1;
  for (int64_t n = 0; n < N; ++n) {
    const float* w = W + n * K;
    int8_t* t = T + n * K;
    double S = 0.0;
    for (int64_t k0 = 0; k0 < K; k0 += 4) {
      int z = 0;
      for (int j = 1; j < 4; ++j)
        if (std::fabs(w[k0 + j]) < std::fabs(w[k0 + z])) z = j;
      for (int j = 0; j < 4; ++j) {
        if (j == z) {
          t[k0 + j] = 0;
        } else {
          t[k0 + j] = w[k0 + j] < 0.0f ? (int8_t)-1 : (int8_t)1;
          S += (double)std::fabs(w[k0 + j]);
        }
      }
    }
    const double kept = (double)(3 * (K / 4));
    alpha[n] = (float)(S / kept);
  }
  return 0;
}

// Bytes of the packed layout for an [N,K] matrix (padding included).
int64_t oracle_packed_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || K % 4 != 0) return -1;
  return pad_to(N, 64) * pad_to(K, 128) * 5 / 32;
}

// Write T (exactly-3-nonzero ternary, [N,K]) in the packed layout.
int oracle_pack(const int8_t* T, int64_t N, int64_t K, uint8_t* packed) {
  if (N <= 0 || K <= 0 || K % 4 != 0) return -1;
  std::memset(packed, 0, (size_t)oracle_packed_bytes(N, K));
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t b = 0; b < K / 4; ++b) {
      int v[4];
      for (int j = 0; j < 4; ++j) v[j] = T[n * K + 4 * b + j];
      const int c = code_of_block(v);
      if (c < 0) return -2;
      int64_t base, r;
      int j;
      tile_slot(n, b, K, &base, &r, &j);
      for (int i = 0; i < 5; ++i) {
        if ((c >> i) & 1) {
          int64_t a;
          int within;
          code_bit(base, r, j, i, &a, &within);
          packed[a] |= (uint8_t)(1u << within);
        }
      }
    }
  }
  return 0;
}

// Read the packed layout back into dense T (the [N,K] part).
int oracle_unpack(const uint8_t* packed, int64_t N, int64_t K, int8_t* T) {
  if (N <= 0 || K <= 0 || K % 4 != 0) return -1;
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t b = 0; b < K / 4; ++b) {
      int64_t base, r;
      int j;
      tile_slot(n, b, K, &base, &r, &j);
      int c = 0;
      for (int i = 0; i < 5; ++i) {
        int64_t a;
        int within;
        code_bit(base, r, j, i, &a, &within);
        c |= ((packed[a] >> within) & 1) << i;
      }
      int v[4];
      block_of_code(c, v);
      for (int i = 0; i < 4; ++i) T[n * K + 4 * b + i] = (int8_t)v[i];
    }
  }
  return 0;
}

// The 2-bit baseline format (the "2-bit ternary packing" the Sherry page
// compares its 5-bit code against, [Sherry §2.1]): every weight of a
// ternary T in 2 bits, 0 -> 00, +1 -> 01, -1 -> 11, no sparsity assumed.
// Tiles of 64 rows x 128 columns, 2048 bytes, in the same row-tile-major
// order as the 5-bit format.  A row's 128 weights form a 256-bit
// little-endian string, weight j at bits [2j, 2j+2); bits 0..127 of tile
// row r sit at tile byte 16*r, bits 128..255 at tile byte 1024 + 16*r.
// Padded like the 5-bit format (to 64 rows and 128 columns; padding is 00).
int64_t oracle_packed2_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || K % 4 != 0) return -1;
  return pad_to(N, 64) * pad_to(K, 128) / 4;
}

int oracle_pack2(const int8_t* T, int64_t N, int64_t K, uint8_t* packed) {
  if (N <= 0 || K <= 0 || K % 4 != 0) return -1;
  std::memset(packed, 0, (size_t)oracle_packed2_bytes(N, K));
  const int64_t KT = pad_to(K, 128) / 128;
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t k = 0; k < K; ++k) {
      const int v = T[n * K + k];
      int code;
      if (v == 0) code = 0;
      else if (v == 1) code = 1;
      else if (v == -1) code = 3;
      else return -2;
      const int64_t tile = ((n / 64) * KT + k / 128) * 2048;
      const int64_t r = n % 64, j = k % 128;
      const int64_t bit = 2 * j;
      const int64_t byte = tile + (bit < 128 ? 16 * r + bit / 8 : 1024 + 16 * r + (bit - 128) / 8);
      packed[byte] |= (uint8_t)(code << (bit % 8));
    }
  }
  return 0;
}

int oracle_unpack2(const uint8_t* packed, int64_t N, int64_t K, int8_t* T) {
  if (N <= 0 || K <= 0 || K % 4 != 0) return -1;
  const int64_t KT = pad_to(K, 128) / 128;
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t k = 0; k < K; ++k) {
      const int64_t tile = ((n / 64) * KT + k / 128) * 2048;
      const int64_t r = n % 64, j = k % 128;
      const int64_t bit = 2 * j;
      const int64_t byte = tile + (bit < 128 ? 16 * r + bit / 8 : 1024 + 16 * r + (bit - 128) / 8);
      const int code = (packed[byte] >> (bit % 8)) & 3;
      if (code == 2) return -2;
      T[n * K + k] = (int8_t)(code == 0 ? 0 : (code == 1 ? 1 : -1));
    }
  }
  return 0;
}

// Per-token symmetric int8 quantization of activations x [M,K].
int oracle_act_quant(const float* x, int64_t M, int64_t K, int8_t* q,
                     float* s) {
  if (M <= 0 || K <= 0) return -1;
  for (int64_t m = 0; m < M; ++m) {
    const float* xr = x + m * K;
    float amax = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
      const float a = std::fabs(xr[k]);
      if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
      s[m] = 1.0f;
      for (int64_t k = 0; k < K; ++k) q[m * K + k] = 0;
      continue;
    }
    const float sc = amax / 127.0f;
    s[m] = sc;
    for (int64_t k = 0; k < K; ++k) {
      float r = std::rint(xr[k] / sc);
      if (r > 127.0f) r = 127.0f;
      if (r < -127.0f) r = -127.0f;
      q[m * K + k] = (int8_t)r;
    }
  }
  return 0;
}

// [Sherry §2.2] L[m][seg][p] = sum_j P_p[j] * q[m, 4*seg + j], 16 per segment.
int oracle_lut(const int8_t* q, int64_t M, int64_t K, int32_t* L) {
  if (M <= 0 || K <= 0 || K % 4 != 0) return -1;
  const int64_t S = K / 4;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t seg = 0; seg < S; ++seg)
      for (int p = 0; p < 16; ++p) {
        int P[4];
        pattern_of(p, P);
        int32_t acc = 0;
        for (int j = 0; j < 4; ++j) acc += P[j] * (int32_t)q[m * K + 4 * seg + j];
        L[(m * S + seg) * 16 + p] = acc;
      }
  return 0;
}

// acc[m,n] = sum_k q[m,k] * T[n,k]: the dense int8 x unpacked-ternary product.
// Returns -2 if any result would not fit int32.  Every output is its own
// plain sum; the outputs are independent, so the build with OpenMP
// (liboracle_omp.so, the same source) only spreads the weight rows over
// threads and returns identical values.
int oracle_gemm_i32(const int8_t* q, const int8_t* T, int64_t M, int64_t N,
                    int64_t K, int32_t* acc) {
  if (M <= 0 || N <= 0 || K <= 0) return -1;
  int overflow = 0;
#pragma omp parallel for schedule(static) reduction(| : overflow)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t m = 0; m < M; ++m) {
      int64_t a = 0;
      const int8_t* qr = q + m * K;
      const int8_t* tr = T + n * K;
      for (int64_t k = 0; k < K; ++k) a += (int64_t)qr[k] * (int64_t)tr[k];
      if (a > INT32_MAX || a < INT32_MIN) overflow = 1;
      else acc[m * N + n] = (int32_t)a;
    }
  return overflow ? -2 : 0;
}

// Threads the product above runs on: 1 in the plain build, the OpenMP
// team size in the OpenMP build.
int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

// [Sherry §2.2, step 4] y = ((float)acc * s_x[m]) * alpha[n].
int oracle_epilogue(const int32_t* acc, const float* s_x, const float* alpha,
                    int64_t M, int64_t N, float* y) {
  if (M <= 0 || N <= 0) return -1;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      const float a = (float)acc[m * N + n];
      const float t = a * s_x[m];
      y[m * N + n] = t * alpha[n];
    }
  return 0;
}

}  // extern "C"
