// Kernel 1 (offline compression) and the activation quantizer.
//
// [Sherry page §3.1] each 4-weight block keeps its three largest |w| with
// their signs; [§2.1] the result is stored as a 5-bit code (4-bit pattern
// index + sign bit).  The per-row scale is the least-squares value for the
// chosen T: (sum of kept |w|) / (number of kept weights).
#include "sherry_device.h"
#include "sherry_launch.h"

namespace sherry {
namespace {

// Code of one block of four weights: drop the first smallest |w|, keep the
// signs of the rest (w < 0 -> -1, else +1).
__device__ __forceinline__ uint32_t encode_block(float w0, float w1, float w2, float w3) {
  const float a0 = fabsf(w0), a1 = fabsf(w1), a2 = fabsf(w2), a3 = fabsf(w3);
  int z = 0;
  float amin = a0;
  if (a1 < amin) { z = 1; amin = a1; }
  if (a2 < amin) { z = 2; amin = a2; }
  if (a3 < amin) { z = 3; }
  const uint32_t n0 = w0 < 0.0f, n1 = w1 < 0.0f, n2 = w2 < 0.0f, n3 = w3 < 0.0f;
  // signs of the three kept weights in position order
  uint32_t f, g, h;
  switch (z) {
    case 0: f = n1; g = n2; h = n3; break;
    case 1: f = n0; g = n2; h = n3; break;
    case 2: f = n0; g = n1; h = n3; break;
    default: f = n0; g = n1; h = n2; break;
  }
  const uint32_t p = 4u * (uint32_t)z + 2u * (g ^ f) + (h ^ f);
  return 2u * p + f;
}

// One wave per format tile.  Lane L = 16g + i encodes the 8 blocks
// 8g..8g+7 of the tile rows 16t + i (t = 0..3) and writes each 40-bit group:
// its low 32 bits as dword t of the lane's 16 bytes, its high 8 bits as byte
// t of the lane's 4 bytes (both stores coalesced across the wave).  Rows past
// N and blocks past K (padding) get code 0 and read nothing.
__global__ __launch_bounds__(64) void pack_codes_kernel(const float* __restrict__ W,
                                                        uint8_t* __restrict__ packed,
                                                        int N, int K) {
  const int KT = k_tiles(K);
  const int rt = blockIdx.x / KT, kt = blockIdx.x % KT;
  const int lane = threadIdx.x;
  const int i = lane & 15, g = lane >> 4;
  const int kb = min(32, (K - kt * kTileK) / 4);   // real blocks of the tile's rows
  uint32_t lo[4], hi = 0;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int n = rt * kTileRows + 16 * t + i;
    const int nb = n < N ? kb : 0;
    const float4* src = reinterpret_cast<const float4*>(W + (size_t)min(n, N - 1) * K + (size_t)kt * kTileK);
    uint64_t v = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int b = 8 * g + j;
      if (b >= nb) continue;
      const float4 x = src[b];
      v |= (uint64_t)encode_block(x.x, x.y, x.z, x.w) << (5 * j);
    }
    lo[t] = (uint32_t)v;
    hi |= (uint32_t)(v >> 32) << (8 * t);
  }
  uint8_t* tile = packed + tile_offset(rt, kt, KT);
  *reinterpret_cast<uint4*>(tile + 16 * lane) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  *reinterpret_cast<uint32_t*>(tile + kTileHiOff + 4 * lane) = hi;
}

// The same ternarization written in the 2-bit baseline format: one wave per
// 64 x 128 tile, lane r = tile row r; weights 0..63 of the row as one
// 16-byte store, weights 64..127 as another (both coalesced).
__global__ __launch_bounds__(64) void pack2_codes_kernel(const float* __restrict__ W,
                                                         uint8_t* __restrict__ packed,
                                                         int N, int K) {
  const int KT = k_tiles(K);
  const int rt = blockIdx.x / KT, kt = blockIdx.x % KT;
  const int lane = threadIdx.x;
  const int n = rt * kTileRows + lane;
  const int nb = n < N ? min(32, (K - kt * kTileK) / 4) : 0;   // real blocks (padding: 00)
  const float4* src = reinterpret_cast<const float4*>(W + (size_t)min(n, N - 1) * K + (size_t)kt * kTileK);
  uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int b = 0; b < 32; ++b) {
    if (b >= nb) continue;
    const float4 v = src[b];
    // the block's values from its 5-bit code, then 2 bits per weight
    const uint32_t cw = code_word(encode_block(v.x, v.y, v.z, v.w));
    uint32_t bits = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t byte = (cw >> (8 * j)) & 0xFFu;
      bits |= (byte == 0 ? 0u : (byte == 1 ? 1u : 3u)) << (2 * j);
    }
    w[b >> 2] |= bits << (8 * (b & 3));
  }
  uint8_t* tile = packed + ((size_t)rt * KT + kt) * kTile2Bytes;
  *reinterpret_cast<uint4*>(tile + 16 * lane) = make_uint4(w[0], w[1], w[2], w[3]);
  *reinterpret_cast<uint4*>(tile + kTile2HiOff + 16 * lane) = make_uint4(w[4], w[5], w[6], w[7]);
}

// One thread per row: alpha[n] = sum of kept |w| in ascending k, in double,
// divided once by the kept count and rounded once to float.
__global__ __launch_bounds__(256) void pack_alpha_kernel(const float* __restrict__ W,
                                                         float* __restrict__ alpha, int N,
                                                         int K) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  const float4* src = reinterpret_cast<const float4*>(W + (size_t)n * K);
  double S = 0.0;
  for (int b = 0; b < K / 4; ++b) {
    const float4 v = src[b];
    const float a[4] = {fabsf(v.x), fabsf(v.y), fabsf(v.z), fabsf(v.w)};
    int z = 0;
    if (a[1] < a[z]) z = 1;
    if (a[2] < a[z]) z = 2;
    if (a[3] < a[z]) z = 3;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j != z) S += (double)a[j];
  }
  alpha[n] = (float)(S / (double)(3 * (K / 4)));
}

// One workgroup per token: s = max|x| / 127, q = clamp(rint(x / s), +-127).
// Every thread issues all of its loads before the first use, so a token costs
// one memory round trip; the values stay in registers for the second pass.
// J = float4 slots per thread (J * 1024 >= K); J = 0 is the looping form for
// rows longer than the register path holds.
__device__ __forceinline__ char4 quant4(const float4 v, float s) {
  char4 o;
  o.x = (signed char)fminf(fmaxf(rintf(v.x / s), -127.0f), 127.0f);
  o.y = (signed char)fminf(fmaxf(rintf(v.y / s), -127.0f), 127.0f);
  o.z = (signed char)fminf(fmaxf(rintf(v.z / s), -127.0f), 127.0f);
  o.w = (signed char)fminf(fmaxf(rintf(v.w / s), -127.0f), 127.0f);
  return o;
}

__device__ __forceinline__ float amax4(const float4 v) {
  return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

__device__ __forceinline__ float block_amax(float amax, float* red) {
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

template <int J>
__global__ __launch_bounds__(256) void quantize_act_kernel(const float* __restrict__ x,
                                                           int8_t* __restrict__ q,
                                                           float* __restrict__ s_x, int K) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  const float4* xr = reinterpret_cast<const float4*>(x + (size_t)m * K);
  char4* qr = reinterpret_cast<char4*>(q + (size_t)m * K);
  const int K4 = K / 4;
  float amax = 0.0f;
  if constexpr (J > 0) {
    float4 v[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int i = threadIdx.x + 256 * j;
      v[j] = i < K4 ? xr[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
#pragma unroll
    for (int j = 0; j < J; ++j) amax = fmaxf(amax, amax4(v[j]));
    amax = block_amax(amax, red);
    const bool zero = !(amax > 0.0f);
    const float s = zero ? 1.0f : amax / 127.0f;
    if (threadIdx.x == 0) s_x[m] = s;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int i = threadIdx.x + 256 * j;
      if (i < K4) qr[i] = zero ? make_char4(0, 0, 0, 0) : quant4(v[j], s);
    }
  } else {
    for (int i = threadIdx.x; i < K4; i += 256) amax = fmaxf(amax, amax4(xr[i]));
    amax = block_amax(amax, red);
    const bool zero = !(amax > 0.0f);
    const float s = zero ? 1.0f : amax / 127.0f;
    if (threadIdx.x == 0) s_x[m] = s;
    for (int i = threadIdx.x; i < K4; i += 256)
      qr[i] = zero ? make_char4(0, 0, 0, 0) : quant4(xr[i], s);
  }
}

}  // namespace

hipError_t launch_quantize_pack(const float* W, int N, int K, uint8_t* packed, float* alpha,
                                hipStream_t stream) {
  const int tiles = row_tiles(N) * k_tiles(K);
  hipLaunchKernelGGL(pack_codes_kernel, dim3(tiles), dim3(64), 0, stream, W, packed, N, K);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pack_alpha_kernel, dim3((N + 255) / 256), dim3(256), 0, stream, W, alpha,
                     N, K);
  return hipGetLastError();
}

hipError_t launch_quantize_pack2(const float* W, int N, int K, uint8_t* packed, float* alpha,
                                 hipStream_t stream) {
  const int tiles = row_tiles(N) * k_tiles(K);
  hipLaunchKernelGGL(pack2_codes_kernel, dim3(tiles), dim3(64), 0, stream, W, packed, N, K);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pack_alpha_kernel, dim3((N + 255) / 256), dim3(256), 0, stream, W, alpha,
                     N, K);
  return hipGetLastError();
}

hipError_t launch_quantize_act(const float* x, int M, int K, int8_t* q, float* s_x,
                               hipStream_t stream) {
  const int slots = (K / 4 + 255) / 256;
  const dim3 grid(M), block(256);
  if (slots <= 1) hipLaunchKernelGGL(quantize_act_kernel<1>, grid, block, 0, stream, x, q, s_x, K);
  else if (slots <= 2) hipLaunchKernelGGL(quantize_act_kernel<2>, grid, block, 0, stream, x, q, s_x, K);
  else if (slots <= 4) hipLaunchKernelGGL(quantize_act_kernel<4>, grid, block, 0, stream, x, q, s_x, K);
  else if (slots <= 8) hipLaunchKernelGGL(quantize_act_kernel<8>, grid, block, 0, stream, x, q, s_x, K);
  else if (slots <= 12) hipLaunchKernelGGL(quantize_act_kernel<12>, grid, block, 0, stream, x, q, s_x, K);
  else if (slots <= 16) hipLaunchKernelGGL(quantize_act_kernel<16>, grid, block, 0, stream, x, q, s_x, K);
  else hipLaunchKernelGGL(quantize_act_kernel<0>, grid, block, 0, stream, x, q, s_x, K);
  return hipGetLastError();
}

}  // namespace sherry
