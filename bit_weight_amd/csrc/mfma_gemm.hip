// Kernel 4: large-M (prefill) product.  The 5-bit codes are decoded to int8
// {-1,0,+1} and contracted with the int8 activations on the gfx950 matrix
// cores (v_mfma_i32_16x16x64_i8, int32 accumulation), followed by the same
// float rescale as the lookup path: y = ((float)acc * s_x[m]) * alpha[n].
// Decoding inside the int8 GEMM's prologue follows the fused
// decode-then-int8-GEMM structure the OdysseyLLM FastGEMM review describes
// for W4A8 (xllm-io page, FastGEMM section).
//
// Workgroup tile: BM = 128 activation rows x BN = 256 weight rows (4 format
// row tiles), k-steps of one format k-tile (128 inputs); 4 waves, one per
// SIMD.  Wave w owns row tile w, i.e. 64 weight rows = 4 MFMA column blocks,
// against all 128 activation rows = 8 MFMA row blocks (8 x 4 accumulators).
// A decoded weight operand therefore feeds 8 MFMAs and an activation
// fragment 4, which keeps the LDS work per k-tile (pair-table lookups plus
// activation fragments) well below the matrix-core time.
//  * activations: 128 x 128 int8 per k-step, loaded once per workgroup into a
//    double-buffered, chunk-major LDS tile (see a_slot), read as MFMA A
//    operands (16 bytes per lane) without bank conflicts;
//  * weights: each wave decodes exactly the B operands it consumes.  It loads
//    its row tile's 1280-byte k-tile coalesced (lane r = tile row r, 16 + 4
//    bytes) and moves dwords g and g+1 of rows 16t..16t+15 to lane group g of
//    column block t with two 4 x 4 transposes of 16-lane rows
//    (v_permlane32_swap, then v_permlane16_swap).  Lane l of a block then
//    holds weight row l%16 and, for lane group g = l/16, codes 8g..8g+7 of
//    the k-tile (inputs 32g..32g+31: the first half in MFMA sub-step 0, the
//    second in sub-step 1); the A operands use the same input order, which a
//    dot product does not see.  A 1024-entry LDS table maps a 10-bit code
//    pair to its 8 int8 weights, so 4 codes cost two 8-byte lookups;
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

constexpr int kBM = 128, kBN = 256;             // workgroup tile
constexpr int kMT = kBM / 16;                   // 8 row blocks per wave
constexpr int kNT = kTileRows / 16;             // 4 column blocks per wave (one row tile)
constexpr int kBK = kTileK;                     // 128
constexpr int kAStage = kBM * kBK;              // 16 KB per k-step
constexpr int kAPerThread = kAStage / 16 / 256; // 16-byte chunks each thread stages (4)
constexpr int kThreads = 512;                   // 4 row tiles x 2 k-tile parities
constexpr int kOutLd = kBN + 4;                 // words per row of the epilogue tile (+16 B)
constexpr int kLdsMain = 4 * kAStage + 8192;    // 2 buffers x 2 parities + pair table
constexpr int kLdsOut = 16 * kOutLd * 4;        // epilogue tile (16 rows)
constexpr int kLdsBytes = kLdsMain > kLdsOut ? kLdsMain : kLdsOut;

// Activation tile in LDS, chunk-major: the 16-byte chunk c of row r sits at
// slot c * kBM + (r ^ c).  A wave's fragment read (16 consecutive rows, one
// chunk) covers 256 contiguous bytes, and a row-contiguous write (8 lanes,
// one row, chunks 0..7) hits 8 different bank groups.
__device__ __forceinline__ int a_slot(int r, int c) { return (c * kBM + (r ^ c)) * 16; }

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

// Decode of one MFMA sub-step: 4 codes per row into B operands (two 10-bit
// code pairs, one 8-byte table entry each).
__device__ __forceinline__ void mg_decode(v4i (&bop)[kNT], const uint32_t (&f)[kNT],
                                          const uint8_t* dec2) {
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
    const uint32_t v = f[t];
    const uint2 e0 = *reinterpret_cast<const uint2*>(dec2 + ((v << 3) & 0x1FF8u));
    const uint2 e1 = *reinterpret_cast<const uint2*>(dec2 + ((v >> 7) & 0x1FF8u));
    bop[t] = v4i{(int)e0.x, (int)e0.y, (int)e1.x, (int)e1.y};
  }
}

// The 8 x 4 MFMAs of one sub-step (A chunk c of the k-step tile at `as`).
// The A fragments of the next two row blocks are requested before the
// MFMAs of the current two, so the LDS latency hides behind 8 MFMAs.
__device__ __forceinline__ void mg_mfma(v4i (&acc)[kMT][kNT], const v4i (&bop)[kNT],
                                        const int8_t* as, int l16, int c) {
  auto frag = [&](int i) { return *reinterpret_cast<const v4i*>(as + a_slot(16 * i + l16, c)); };
  v4i a0 = frag(0), a1 = frag(1);
#pragma unroll
  for (int i = 0; i < kMT; i += 2) {
    v4i n0 = a0, n1 = a1;
    if (i + 2 < kMT) {
      n0 = frag(i + 2);
      n1 = frag(i + 3);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < kNT; ++t)
      acc[i][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, bop[t], acc[i][t], 0, 0, 0);
#pragma unroll
    for (int t = 0; t < kNT; ++t)
      acc[i + 1][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, bop[t], acc[i + 1][t], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    a0 = n0;
    a1 = n1;
  }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, size_t bytes) {
  const int n = bytes > 0x7FFFFFFFull ? 0x7FFFFFFF : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

__global__ __launch_bounds__(kThreads) void mfma_gemm_kernel(GemmArgs a, int n_tiles) {
  // one LDS block: the activation buffers [buffer][parity], then the pair
  // table; after the main loop the epilogue tile reuses all of it
  // (32-bit words: every view below is a character type or 32-bit lanes)
  __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsBytes / 4];
  int8_t (*As)[kAStage] = reinterpret_cast<int8_t (*)[kAStage]>(lds);
  uint2* dec2 = reinterpret_cast<uint2*>(lds + 4 * kAStage / 4);

  const int M = a.M, N = a.N, K = a.K, KT = K / kTileK, RT = N / kTileRows;
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
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave = wv & 3, kh = wv >> 2;            // row tile, k-tile parity
  const int l16 = lane & 15, g = lane >> 4;

  // decode table: code pair (c0 | c1 << 5) -> the 8 int8 weights of both
  for (int i = tid; i < 1024; i += kThreads)
    dec2[i] = make_uint2(code_word(i & 31), code_word(i >> 5));

  // This wave's row tile (N % 64 == 0, so a row tile is all valid or all
  // past N; one past N streams the last tile and stores nothing).
  const int rt_raw = n0 / kTileRows + wave;
  const bool n_live = rt_raw < RT;
  const int rt = n_live ? rt_raw : RT - 1;
  const __amdgpu_buffer_rsrc_t rc =
      buffer_rsrc(a.packed + tile_offset(rt, 0, KT), (size_t)KT * kTileBytes);
  const __amdgpu_buffer_rsrc_t ra =
      buffer_rsrc(a.x + (size_t)m0 * K, (size_t)(M - m0) * (size_t)K);
  const uint32_t sh = 8u * (uint32_t)g;  // bit 40g mod 32

  // activations: each parity's 256 threads stage its k-tile, 128 rows x 128
  // bytes, four 16-byte chunks per thread (8 lanes per row: coalesced); rows
  // past M read row M-1 (they feed only unstored output rows)
  int a_v[kAPerThread], a_lds[kAPerThread];
#pragma unroll
  for (int i = 0; i < kAPerThread; ++i) {
    const int idx = (tid & 255) + 256 * i, row = idx >> 3, c = idx & 7;
    a_v[i] = min(row, M - 1 - m0) * K + c * 16;
    a_lds[i] = a_slot(row, c);
  }

  v4i acc[kMT][kNT];
#pragma unroll
  for (int i = 0; i < kMT; ++i)
#pragma unroll
    for (int t = 0; t < kNT; ++t) acc[i][t] = v4i{0, 0, 0, 0};

  // Codes (coalesced, lane = tile row) and activations of this wave's
  // k-tile of pair j (2j + kh, clamped: a prefetch past the end re-reads the
  // last k-tile).
  const int KJ = (KT + 1) / 2;
  auto load = [&](int j, v4u& w, uint32_t& h, v4u (&av)[kAPerThread]) {
    const int kt_ = min(2 * j + kh, KT - 1);
    const int ks = kt_ * kTileBytes, ka = kt_ * kBK;
    w = __builtin_amdgcn_raw_buffer_load_b128(rc, 16 * lane, ks, 0);
    h = __builtin_amdgcn_raw_buffer_load_b32(rc, kTileHiOff + 4 * lane, ks, 0);
#pragma unroll
    for (int i = 0; i < kAPerThread; ++i)
      av[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, a_v[i], ka, 0);
  };
  const uint8_t* d2 = reinterpret_cast<const uint8_t*>(dec2);
  // One k-step from one register stage; the stage is refilled with the
  // loads for k-step kt+2 before the MFMAs.  The scheduling barriers keep
  // the refill loads inside their own step, so every step finds exactly one
  // newer stage in flight and waits only for its own.
  auto step = [&](int j, v4u& w, uint32_t& h, v4u (&av)[kAPerThread]) {
    int8_t* as = &As[(j & 1) * 2 + kh][0];
    const bool live = 2 * j + kh < KT;     // odd KT: the last pair has one k-tile
#pragma unroll
    for (int i = 0; i < kAPerThread; ++i) *reinterpret_cast<v4u*>(as + a_lds[i]) = av[i];
    // lane (l16, g) of block t <- dwords g (lo) and g+1 (hi) of row 16t+l16
    uint32_t lo[kNT], hi[kNT];
    transpose4(w.x, w.y, w.z, w.w, lo);
    transpose4(w.y, w.z, w.w, h, hi);
    // codes 8g..8g+3 (sub-step 0) and 8g+4..8g+7 (sub-step 1), 20 bits each
    uint32_t f0[kNT], f1[kNT];
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
      const uint32_t x0 = __builtin_amdgcn_alignbit(hi[t], lo[t], sh);
      f0[t] = x0;
      f1[t] = __builtin_amdgcn_alignbit(hi[t] >> sh, x0, 20);
    }
    load(min(j + 2, KJ - 1), w, h, av);
    __builtin_amdgcn_sched_barrier(0);
    v4i bop[kNT];
    mg_decode(bop, f0, d2);      // the table is fixed: no wait for the barrier
    lds_barrier();               // this pair's activations are in LDS
    if (live) {
      mg_mfma(acc, bop, as, l16, 2 * g);
      mg_decode(bop, f1, d2);
      mg_mfma(acc, bop, as, l16, 2 * g + 1);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // two register stages, ping-pong: no register copies between k-steps
  v4u w0, w1, av0[kAPerThread], av1[kAPerThread];
  uint32_t h0, h1;
  load(0, w0, h0, av0);
  __builtin_amdgcn_sched_barrier(0);  // stage 0's loads strictly before stage 1's
  load(min(1, KJ - 1), w1, h1, av1);
  __builtin_amdgcn_sched_barrier(0);
  lds_barrier();  // decode table

  int j = 0;
  for (; j + 2 <= KJ; j += 2) {
    step(j, w0, h0, av0);
    step(j + 1, w1, h1, av1);
  }
  if (j < KJ) step(j, w0, h0, av0);

  // Epilogue, one 16-row block at a time: every wave writes its 16 x 64
  // results (y = ((float)acc * s_x[m]) * alpha[n], or the raw int32) into a
  // row-major LDS tile of 16 x 256, then the workgroup stores whole rows,
  // 16 bytes per lane, so each store instruction writes full 128-byte lines.
  // Lane (l16, g) of a 16 x 16 MFMA block holds column l16, rows 4g..4g+3.
  uint32_t* ot = lds;   // [16][kOutLd] result words
  const bool want_y = a.y != nullptr;
  float al[kNT];
#pragma unroll
  for (int t = 0; t < kNT; ++t)
    al[t] = want_y && n_live ? a.alpha[rt * kTileRows + 16 * t + l16] : 0.0f;
#pragma unroll
  for (int i = 0; i < kMT; ++i) {
    __syncthreads();  // previous use of the LDS area is finished
    // the odd-parity waves hand their int32 sums to the even ones
    if (kh == 1) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < kNT; ++t)
          ot[(4 * g + r) * kOutLd + wave * kTileRows + 16 * t + l16] = (uint32_t)acc[i][t][r];
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < kNT; ++t)
          acc[i][t][r] += (int)ot[(4 * g + r) * kOutLd + wave * kTileRows + 16 * t + l16];
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ml = 4 * g + r;                 // row within the block
      const int m = min(m0 + 16 * i + ml, M - 1);
      const float sx = want_y ? a.s_x[m] : 0.0f;
#pragma unroll
      for (int t = 0; t < kNT; ++t) {
        const int col = wave * kTileRows + 16 * t + l16;
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
    }
    __syncthreads();
    // 16 rows x 64 float4 per block
    for (int e = tid; e < 16 * (kBN / 4); e += kThreads) {
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
  hipLaunchKernelGGL(mfma_gemm_kernel, dim3(p.grid), dim3(kThreads), 0, stream, a, nt);
  return hipGetLastError();
}

}  // namespace sherry
