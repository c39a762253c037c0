// Kernel 4: large-M (prefill) product.  The 5-bit codes are decoded to int8
// {-1,0,+1} and contracted with the int8 activations on the gfx950 matrix
// cores (v_mfma_i32_16x16x64_i8, int32 accumulation), followed by the same
// float rescale as the lookup path: y = ((float)acc * s_x[m]) * alpha[n].
// Decoding inside the int8 GEMM's prologue follows the fused
// decode-then-int8-GEMM structure the OdysseyLLM FastGEMM review describes
// for W4A8 (xllm-io page, FastGEMM section).
//
// Workgroup tile: BM = 64 activation rows x BN = 448 weight rows, k-steps of
// one format k-tile (128 inputs); 4 waves, one per SIMD.  The waves split the
// weight rows (112 each = 7 MFMA column blocks) and share the activation
// tile, so each wave owns 64 x 112 outputs (4 x 7 blocks of 16 x 16):
//  * activations: 64 x 128 int8 per k-step, loaded once per workgroup into a
//    double-buffered, chunk-major LDS tile (see a_slot), read as MFMA A
//    operands (16 bytes per lane) without bank conflicts;
//  * weights: each wave decodes exactly the B operands it consumes.  Lane l
//    of a 16-column block holds weight row l%16; lane group g = l/16 takes
//    codes 8g..8g+7 of the k-tile (inputs 32g..32g+31: the first half in
//    MFMA sub-step 0, the second in sub-step 1).  The A operands use the
//    same input order, which a dot product does not see.  Those 40 code bits
//    always lie in two dwords of the row's 160-bit string, so a lane loads
//    2 dwords per row; a 1024-entry LDS table maps a 10-bit code pair to its
//    8 int8 weights, so 4 codes cost two 8-byte lookups and four VALU ops.
//    No decoded weight is written to LDS or decoded twice in a workgroup;
//  * codes and activations come through buffer descriptors (32-bit lane
//    offsets, scalar k-step offset) two k-steps ahead into two register
//    stages used in turn; the barrier orders LDS only, so the prefetched
//    loads stay in flight across it.
// Tiles are numbered so that the 8 XCDs (workgroups are dealt round-robin)
// each own a slab of weight rows, which then stays in that XCD's L2 for all
// activation tiles.
#include "sherry_device.h"
#include "sherry_launch.h"

namespace sherry {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int kBM = 64, kBN = 448, kWN = kBN / 4, kNT = kWN / 16;  // 7 column blocks / wave
constexpr int kMT = kBM / 16;                                      // 4 row blocks / wave
constexpr int kBK = kTileK;                                        // 128
constexpr int kChunks = kBK / 16;                                  // 16-byte input chunks
constexpr int kAStage = kBM * kBK;                                 // 8 KB per k-step
constexpr int kOutLd = kBN + 4;          // floats per row of the epilogue tile (+16 B pad)
constexpr int kLdsMain = 2 * kAStage + 8192;     // activation stages + pair table
constexpr int kLdsOut = 16 * kOutLd * 4;         // epilogue tile
constexpr int kLdsBytes = kLdsMain > kLdsOut ? kLdsMain : kLdsOut;

// Activation tile in LDS, chunk-major: the 16-byte chunk c of row r sits at
// slot c * 64 + (r ^ c).  A wave's fragment read (16 consecutive rows, one
// chunk) covers 256 contiguous bytes, and a row-contiguous write (8 lanes,
// one row, chunks 0..7) hits 8 different bank groups.
__device__ __forceinline__ int a_slot(int r, int c) { return (c * kBM + (r ^ c)) * 16; }

// One MFMA sub-step: decode 4 codes per row into B operands (two 10-bit
// code pairs, one 8-byte table entry each), then 4 x 7 MFMAs.
__device__ __forceinline__ void mg_mfma(v4i (&acc)[kMT][kNT], const uint32_t (&f)[kNT],
                                        const int8_t* as, int l16, int c, const uint8_t* dec2) {
  v4i bop[kNT];
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
    const uint32_t v = f[t];
    const uint2 e0 = *reinterpret_cast<const uint2*>(dec2 + ((v << 3) & 0x1FF8u));
    const uint2 e1 = *reinterpret_cast<const uint2*>(dec2 + ((v >> 7) & 0x1FF8u));
    bop[t] = v4i{(int)e0.x, (int)e0.y, (int)e1.x, (int)e1.y};
  }
#pragma unroll
  for (int i = 0; i < kMT; ++i) {
    const v4i aop = *reinterpret_cast<const v4i*>(as + a_slot(16 * i + l16, c));
#pragma unroll
    for (int t = 0; t < kNT; ++t)
      acc[i][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop, bop[t], acc[i][t], 0, 0, 0);
  }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, size_t bytes) {
  const int n = bytes > 0x7FFFFFFFull ? 0x7FFFFFFF : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

__global__ __launch_bounds__(256) void mfma_gemm_kernel(GemmArgs a, int n_tiles) {
  // one LDS block: two activation stages, then the pair table; after the
  // main loop the epilogue tile reuses all of it
  // (32-bit words: every view below is a character type or 32-bit lanes)
  __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsBytes / 4];
  int8_t (*As)[kAStage] = reinterpret_cast<int8_t (*)[kAStage]>(lds);
  uint2* dec2 = reinterpret_cast<uint2*>(lds + 2 * kAStage / 4);

  const int M = a.M, N = a.N, K = a.K, KT = K / kTileK;
  // tile id -> (m tile, n tile): consecutive ids of one XCD share n tiles
  const int id = blockIdx.x;
  const int mt_count = (M + kBM - 1) / kBM;
  const int xcd = id & 7, slot = id >> 3;
  const int per_xcd = (n_tiles + 7) / 8;            // n tiles owned by one XCD
  const int owned = slot / mt_count;
  const int mt_idx = slot - owned * mt_count;
  const int nt_idx = xcd * per_xcd + owned;
  if (nt_idx >= n_tiles || mt_idx >= mt_count) return;  // padding ids
  const int m0 = mt_idx * kBM, n0 = nt_idx * kBN;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;

  // decode table: code pair (c0 | c1 << 5) -> the 8 int8 weights of both
  for (int i = tid; i < 1024; i += 256) dec2[i] = make_uint2(code_word(i & 31), code_word(i >> 5));

  // Buffer descriptors: the workgroup's first code tile row and first
  // activation row.  Per-lane offsets are 32-bit, the k-step is a scalar
  // offset, so a load costs no VALU work.
  const size_t pk_base = tile_offset(n0 / kTileRows, 0, KT);
  const size_t pk_total = (size_t)N * (size_t)K * 5 / 32;
  const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(a.packed + pk_base, pk_total - pk_base);
  const __amdgpu_buffer_rsrc_t ra =
      buffer_rsrc(a.x + (size_t)m0 * K, (size_t)(M - m0) * (size_t)K);

  // this lane's weight rows (one per 16-column block)
  int rows[kNT];
  bool rv[kNT];
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
    rows[t] = n0 + wave * kWN + 16 * t + l16;
    rv[t] = (n0 + wave * kWN + 16 * t) < N;  // N % 64 == 0: blocks are all-or-none
  }
  // The lane's two code dwords of a row: dword g and dword g+1 of the
  // 160-bit string (dword 4 lives in the tile's 4-byte part).  Rows past N
  // (whole 16-row blocks) read row N-1: their products land in columns that
  // are never stored, so no load needs a branch.
  const uint32_t sh = 8u * (uint32_t)g;  // bit 40g mod 32
  int lo_v[kNT], hi_v[kNT];
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
    const int row = rv[t] ? rows[t] : N - 1;
    const int tb = (row / kTileRows - n0 / kTileRows) * KT * kTileBytes;
    const int r = row % kTileRows;
    lo_v[t] = tb + 16 * r + 4 * g;
    hi_v[t] = tb + (g < 3 ? 16 * r + 4 * (g + 1) : kTileHiOff + 4 * r);
  }
  // activations: 64 rows x 128 bytes per k-step, two 16-byte chunks per
  // thread (8 lanes per row: coalesced); rows past M read row M-1 (they feed
  // only unstored output rows)
  int a_v[2], a_lds[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = tid + 256 * i, row = idx >> 3, c = idx & 7;
    a_v[i] = min(row, M - 1 - m0) * K + c * 16;
    a_lds[i] = a_slot(row, c);
  }

  v4i acc[kMT][kNT];
#pragma unroll
  for (int i = 0; i < kMT; ++i)
#pragma unroll
    for (int t = 0; t < kNT; ++t) acc[i][t] = v4i{0, 0, 0, 0};

  // Codes and activations of k-step kt for this lane.
  auto load = [&](int kt_, uint32_t* lo, uint32_t* hi, v4u& v0, v4u& v1) {
    const int ks = kt_ * kTileBytes, ka = kt_ * kBK;
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
      lo[t] = __builtin_amdgcn_raw_buffer_load_b32(rc, lo_v[t], ks, 0);
      hi[t] = __builtin_amdgcn_raw_buffer_load_b32(rc, hi_v[t], ks, 0);
    }
    v0 = __builtin_amdgcn_raw_buffer_load_b128(ra, a_v[0], ka, 0);
    v1 = __builtin_amdgcn_raw_buffer_load_b128(ra, a_v[1], ka, 0);
  };
  // One k-step from one register stage; the stage is refilled with the
  // loads for k-step kt+2 before the MFMAs.  The scheduling barriers keep
  // the refill loads inside their own step, so every step finds exactly one
  // newer stage in flight and waits only for its own.
  auto step = [&](int kt_, uint32_t* lo, uint32_t* hi, v4u& v0, v4u& v1) {
    int8_t* as = &As[kt_ & 1][0];
    *reinterpret_cast<v4u*>(as + a_lds[0]) = v0;
    *reinterpret_cast<v4u*>(as + a_lds[1]) = v1;
    // codes 8g..8g+3 (sub-step 0) and 8g+4..8g+7 (sub-step 1), 20 bits each
    uint32_t f0[kNT], f1[kNT];
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
      const uint32_t x0 = __builtin_amdgcn_alignbit(hi[t], lo[t], sh);
      f0[t] = x0;
      f1[t] = __builtin_amdgcn_alignbit(hi[t] >> sh, x0, 20);
    }
    load(min(kt_ + 2, KT - 1), lo, hi, v0, v1);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();  // this k-step's activations are in LDS
    mg_mfma(acc, f0, as, l16, 2 * g, reinterpret_cast<const uint8_t*>(dec2));
    mg_mfma(acc, f1, as, l16, 2 * g + 1, reinterpret_cast<const uint8_t*>(dec2));
    __builtin_amdgcn_sched_barrier(0);
  };

  // two register stages, ping-pong: no register copies between k-steps
  uint32_t lo0[kNT], hi0[kNT], lo1[kNT], hi1[kNT];
  v4u a00, a01, a10, a11;
  load(0, lo0, hi0, a00, a01);
  __builtin_amdgcn_sched_barrier(0);  // stage 0's loads strictly before stage 1's
  load(min(1, KT - 1), lo1, hi1, a10, a11);
  __builtin_amdgcn_sched_barrier(0);
  lds_barrier();  // decode table

  int kt = 0;
  for (; kt + 2 <= KT; kt += 2) {
    step(kt, lo0, hi0, a00, a01);
    step(kt + 1, lo1, hi1, a10, a11);
  }
  if (kt < KT) step(kt, lo0, hi0, a00, a01);

  // Epilogue, one 16-row block at a time: every wave writes its 16 x 112
  // results (y = ((float)acc * s_x[m]) * alpha[n], or the raw int32) into a
  // row-major LDS tile of 16 x 448, then the workgroup stores whole rows,
  // 16 bytes per lane, so each store instruction writes full 128-byte lines.
  // Lane (l16, g) of a 16 x 16 MFMA block holds column l16, rows 4g..4g+3.
  uint32_t* ot = lds;   // [16][kOutLd] result words
  const bool want_y = a.y != nullptr;
  float al[kNT];
#pragma unroll
  for (int t = 0; t < kNT; ++t) al[t] = want_y && rv[t] ? a.alpha[rows[t]] : 0.0f;
#pragma unroll
  for (int i = 0; i < kMT; ++i) {
    __syncthreads();  // previous use of the LDS area is finished
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ml = 4 * g + r;                 // row within the block
      const int m = min(m0 + 16 * i + ml, M - 1);
      const float sx = want_y ? a.s_x[m] : 0.0f;
#pragma unroll
      for (int t = 0; t < kNT; ++t) {
        const int col = wave * kWN + 16 * t + l16;
        uint32_t v;
        if (want_y) {
          const float tv = (float)acc[i][t][r] * sx;
          v = __builtin_bit_cast(uint32_t, tv * al[t]);
        } else {
          v = (uint32_t)acc[i][t][r];
        }
        ot[ml * kOutLd + col] = v;
      }
    }
    __syncthreads();
    // 16 rows x 112 float4 per block
    for (int e = tid; e < 16 * (kBN / 4); e += 256) {
      const int ml = e / (kBN / 4), c4 = e - ml * (kBN / 4);
      const int m = m0 + 16 * i + ml, n = n0 + 4 * c4;
      if (m < M && n < N) {
        const v4u v = *reinterpret_cast<const v4u*>(&ot[ml * kOutLd + 4 * c4]);
        void* dst = want_y ? static_cast<void*>(a.y + (size_t)m * N + n)
                           : static_cast<void*>(a.acc + (size_t)m * N + n);
        *reinterpret_cast<v4u*>(dst) = v;
      }
    }
  }
}

}  // namespace

int mfma_gemm_grid(int M, int N) {
  const int mt = (M + kBM - 1) / kBM, nt = (N + kBN - 1) / kBN;
  const int per_xcd = (nt + 7) / 8;
  return 8 * per_xcd * mt;
}

hipError_t launch_mfma_gemm(const GemmPlan& p, const GemmArgs& a, hipStream_t stream) {
  const int nt = (a.N + kBN - 1) / kBN;
  hipLaunchKernelGGL(mfma_gemm_kernel, dim3(p.grid), dim3(256), 0, stream, a, nt);
  return hipGetLastError();
}

}  // namespace sherry
