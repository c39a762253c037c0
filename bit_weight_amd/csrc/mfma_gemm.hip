// Kernel 4: large-M (prefill) product.  The 5-bit codes are decoded to int8
// {-1,0,+1} and contracted with the int8 activations on the gfx950 matrix
// cores (v_mfma_i32_16x16x64_i8, int32 accumulation), followed by the same
// float rescale as the lookup path: y = ((float)acc * s_x[m]) * alpha[n].
// Decoding inside the int8 GEMM's prologue follows the fused
// decode-then-int8-GEMM structure the OdysseyLLM FastGEMM review describes
// for W4A8 (xllm-io page, FastGEMM section).
//
// Workgroup tile: BM = 128 activation rows x BN = 256 weight rows (4 format
// row tiles), k-steps of one format k-tile (128 inputs); 8 waves, two per
// SIMD: wave (kh, w) takes the k-tiles of phase kh (2j + kh) of row tile w,
// i.e. 64 weight rows = 4 MFMA column blocks, against all 128 activation
// rows = 8 MFMA row blocks (8 x 4 accumulators); the two phases' sums are
// added in the epilogue.  On a small grid the 8 waves split instead into 2
// row tiles x KP = 4 k-phases (BN = 128, k-tiles 4j + kh): twice the
// workgroups, each a quarter of K per wave; BM = 64 halves the tile again.
// A decoded weight operand therefore feeds 8 MFMAs and an activation
// fragment 4, which keeps the LDS work per k-tile (pair-table lookups plus
// activation fragments) well below the matrix-core time.
//  * activations: 128 x 128 int8 per k-step, copied once per workgroup
//    straight from global memory into LDS by buffer loads with LDS return
//    (no registers on the way), 8 lanes per 128-byte row so every load reads
//    whole lines; rows sit in a row-major tile whose 16-byte chunks are
//    XOR-swizzled (see a_off) so the MFMA A reads (16 rows, one chunk) hit 16
//    different bank groups.  Three buffers per phase: the copy for k-step
//    j+2 starts right after the barrier of step j, once every wave is done
//    with the buffer it overwrites, and has two steps to land (two buffers
//    and one step with BM = 128 and 4 phases, whose 12 x 16 KB would not
//    fit LDS; with BM = 64 four buffers and one barrier per two steps);
//  * weights: each wave decodes exactly the B operands it consumes.  It loads
//    its row tile's 1280-byte k-tile coalesced (lane l = slot l, 16 + 4
//    bytes), which by the format's design already holds, for column block t,
//    weight row 16t + l%16 and, for lane group g = l/16, codes 8g..8g+7 of
//    the k-tile (inputs 32g..32g+31: the first half in MFMA sub-step 0, the
//    second in sub-step 1): dword t and byte t of the slot's last dword.  The
//    A operands use the same input order, which a dot product does not see.
//    A 1024-entry LDS table maps a 10-bit code pair to its 8 int8 weights,
//    so 4 codes cost two 8-byte lookups;
//  * codes come through a buffer descriptor into two register stages used
//    in turn; a k-step's codes are decoded (table lookups) between the
//    MFMAs of the step before it, so the LDS lookups overlap matrix-core
//    work, and the 64 MFMAs of a step run back to back with the A reads two
//    row blocks ahead.  The barrier waits for exactly the activation copy of
//    its own step (a counted vmcnt), so the newer loads stay in flight
//    across it.
// Tiles are numbered so that the 8 XCDs (workgroups are dealt round-robin)
// each own a slab of weight rows, which then stays in that XCD's L2 for all
// activation tiles.
#include "sherry_device.h"
#include "sherry_launch.h"

namespace sherry {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int kNT = kTileRows / 16;             // 4 column blocks per wave (one row tile)
constexpr int kBK = kTileK;                     // 128
constexpr int kThreads = 512;                   // 8 waves: row tiles x k-phases

// The sizes that follow from the tile height BM (128 or 64 activation rows)
// and the number of k-phases KP (2 or 4).
template <int BM, int KP>
struct Tiling {
  static_assert(KP == 2 || KP == 4, "k-phases: 2 or 4");
  // 64-row tiles: one barrier per two k-steps, four activation buffers per
  // k-phase, the copies for steps j+2 and j+3 issued in step j (measured at
  // K=4096: M=128, N=14336 14.5 -> 13.6 us; M=320, N=11008 20.9 -> 20.5;
  // no faster with 128-row tiles).  Else a barrier per k-step with three
  // buffers (the copy for step j+2 issued in step j), or two with 128-row
  // tiles and 4 phases, whose 4 x 3 x 16 KB would not fit LDS (the copy for
  // step j+1 issued in step j).
  static constexpr bool kPair = BM == 64;
  static constexpr int kABufs = kPair ? 4 : (BM == 128 && KP == 4 ? 2 : 3);
  static constexpr int kRT = kThreads / 64 / KP;       // row tiles per workgroup (4 or 2)
  static constexpr int kBN = kRT * kTileRows;          // workgroup tile width (256 or 128 weight rows)
  // Words per row of the epilogue tiles.  One sums write (an accumulator
  // register of every lane) puts rows r, r+4, r+8, r+12 of an MFMA block in
  // lanes 0-15, 16-31, 32-47, 48-63; a pitch of 4 (mod 16) words spaces
  // those rows 16 banks apart, so no two lanes of a write share a bank.  (At
  // kBN + 16 the four rows were 1088 words, a multiple of 64, apart: measured
  // with the padded pitch, M=512, N=14336, K=4096 31.4 -> 31.1 us; M=256
  // 20.5 -> 19.9; M=128 13.7 -> 13.5.)
  static constexpr int kOutLd = kBN + 4;
  static constexpr int kLdsOut = KP * 32 * kOutLd * 4; // epilogue tiles (32 rows, every phase)
  static constexpr int kMT = BM / 16;                  // row blocks per wave (8 or 4)
  static constexpr int kAStage = BM * kBK;             // activation bytes per k-step
  static constexpr int kRowsPerWave = BM / kRT;        // rows each wave of a phase copies
  static constexpr int kACopies = kRowsPerWave / 8;    // 1 KB copies (8 rows) per wave per k-step
  static constexpr int kLdsMain = KP * kABufs * kAStage;  // activation buffers x phases
  static constexpr int kLdsBytes = kLdsMain > kLdsOut ? kLdsMain : kLdsOut;
  // vector-memory ops a wave issues between a k-step's activation copy and
  // that step's barrier: with three buffers the codes three steps ahead of
  // it (2), the next step's copy, and the codes four steps ahead (2); with
  // two, the codes two steps ahead of it (2); with a barrier per two steps
  // (the copy of steps j, j+1 issued at step j-2), the codes of steps j+1
  // and j+2 (2 + 2)
  static constexpr int kNewerLoads = kPair ? 4 : (kABufs == 3 ? 2 + kACopies + 2 : 2);
};

// Activation tile in LDS, row-major with 128-byte rows: the 16-byte chunk c
// of row r sits at chunk position c ^ ((r >> 1) & 7).  A fragment read (16
// consecutive rows, one chunk) then spreads over all 16 bank groups of a
// 256-byte bank period, and 8 lanes copying one row fill one row.
__device__ __forceinline__ int a_off(int r, int c) { return (r * 8 + (c ^ ((r >> 1) & 7))) * 16; }

// s_waitcnt operand: vmcnt(vm), lgkmcnt(0), expcnt not waited.
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 15) | ((vm >> 4) << 14) | 0x70; }

// B operands of one column block and sub-step: 4 codes (20 bits of v) as
// two code pairs, one 8-byte table entry each.
__device__ __forceinline__ v4i mg_decode4(uint32_t v, const uint8_t* dec2) {
  const uint2 e0 = *reinterpret_cast<const uint2*>(dec2 + ((v << 3) & 0x1FF8u));
  const uint2 e1 = *reinterpret_cast<const uint2*>(dec2 + ((v >> 7) & 0x1FF8u));
  return v4i{(int)e0.x, (int)e0.y, (int)e1.x, (int)e1.y};
}

// The 2 x MT x 4 MFMAs of one k-step (sub-steps s = 0, 1 read A chunk 2g+s
// of the tile at `as`, with B operands b0 / b1), and the table lookups that
// decode the next k-step's codes (f0 / f1) into n0 / n1: those of sub-step
// 0 spread over the groups of 8 MFMAs of sub-step 1 (b0 is dead by then, so
// n0 can take its registers), those of sub-step 1 after the MFMAs.  The A
// fragments of the next two row blocks are requested before the MFMAs of
// the current two, so the LDS latency hides behind 8 MFMAs.
template <bool kLive, int kMT>
__device__ __forceinline__ void mg_mfma(v4i (&acc)[kMT][kNT], const v4i (&b0)[kNT],
                                        const v4i (&b1)[kNT], const int8_t* as, int l16, int g,
                                        const uint32_t (&f0)[kNT], const uint32_t (&f1)[kNT],
                                        v4i (&n0)[kNT], v4i (&n1)[kNT], const uint8_t* dec2) {
  auto frag = [&](int u) {   // u = kMT s + row block
    return *reinterpret_cast<const v4i*>(as + a_off(16 * (u % kMT) + l16, 2 * g + u / kMT));
  };
  constexpr int kDecPerGroup = kNT / (kMT / 2);   // sub-step-0 lookups per group of sub-step 1
  v4i a0{0, 0, 0, 0}, a1{0, 0, 0, 0};
  if constexpr (kLive) {
    a0 = frag(0);
    a1 = frag(1);
  }
#pragma unroll
  for (int u = 0; u < 2 * kMT; u += 2) {
    v4i p0 = a0, p1 = a1;
    if (kLive && u + 2 < 2 * kMT) {
      p0 = frag(u + 2);
      p1 = frag(u + 3);
    }
    if (u >= kMT) {
#pragma unroll
      for (int d = 0; d < kDecPerGroup; ++d) {
        const int t = ((u - kMT) >> 1) * kDecPerGroup + d;
        n0[t] = mg_decode4(f0[t], dec2);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kLive) {
      const int i = u % kMT;
#pragma unroll
      for (int c = 0; c < kNT; ++c)
        acc[i][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, u < kMT ? b0[c] : b1[c], acc[i][c], 0, 0, 0);
#pragma unroll
      for (int c = 0; c < kNT; ++c)
        acc[i + 1][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, u < kMT ? b0[c] : b1[c], acc[i + 1][c], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    a0 = p0;
    a1 = p1;
  }
#pragma unroll
  for (int t = 0; t < kNT; ++t) n1[t] = mg_decode4(f1[t], dec2);
}

// 16 bytes per lane from the buffer at byte `voffset` straight into LDS at
// dst + 16 * lane (a buffer load with LDS return).  A plain function, not a
// lambda inside the kernel template: there the host pass rejects the LDS
// address-space cast and silently drops the kernel's host-side stub.
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t r, int8_t* dst, int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voffset, 0, 0,
                                           0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, size_t bytes) {
  const int n = bytes > 0x7FFFFFFFull ? 0x7FFFFFFF : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

template <int BM, int KP>
__global__ __launch_bounds__(kThreads) void mfma_gemm_kernel(const uint8_t* packed, const int8_t* x,
                                                             const float* xf, int M, int N, int K,
                                                             int n_tiles, int /*unused*/, const float* s_x,
                                                             const float* alpha, float* y, int32_t* acc_out,
                                                             int32_t* partials) {
  const GemmArgs a = product_args(packed, x, xf, M, N, K, s_x, alpha, y, acc_out, partials);
  using T = Tiling<BM, KP>;
  constexpr int kBM = BM, kMT = T::kMT, kAStage = T::kAStage, kACopies = T::kACopies;
  constexpr int kLdsBytes = T::kLdsBytes, kNewerLoads = T::kNewerLoads;
  constexpr int kRT = T::kRT, kBN = T::kBN, kOutLd = T::kOutLd, kABufs = T::kABufs;
  constexpr bool kPair = T::kPair;
  // the activation buffers [buffer][phase]; after the main loop the
  // epilogue tile reuses them
  // (32-bit words: every view below is a character type or 32-bit lanes)
  __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsBytes / 4];
  // the pair table in an array of its own: the compiler then sees that its
  // lookups cannot read what an activation copy in flight is writing.  Its
  // alignment places it first in LDS, below 64 KB, so a lookup's table base
  // folds into the instruction's offset field instead of costing a VALU OR
  // per lookup (measured at M=512, K=4096, N=14336: 32.7 -> 31.9 us)
  __shared__ __attribute__((aligned(1024))) uint2 dec2[1024];
  __shared__ float sxs[kBM];   // s_x of this tile's rows (epilogue)
  // arrivals at the step barrier of each k-tile parity (128-row tiles)
  __shared__ unsigned parity_arrivals[KP];

  const int KT = k_tiles(K), RT = row_tiles(N);
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
  const int wave = wv % kRT, kh = wv / kRT;        // row tile, k-phase
  const int l16 = lane & 15, g = lane >> 4;

  if (tid < KP) parity_arrivals[tid] = 0u;   // published by the prologue's barrier
  // decode table: code pair (c0 | c1 << 5) -> the 8 int8 weights of both
  for (int i = tid; i < 1024; i += kThreads)
    dec2[i] = make_uint2(code_word(i & 31), code_word(i >> 5));

  // This wave's row tile.  One wholly past N (N not a multiple of 256)
  // streams the last row tile again and stores nothing.  In a ragged last
  // row tile (N % 64 != 0) the padding rows decode code 0, the block
  // (0,+1,+1,+1), and form sums of their own: only the n < N mask of the
  // epilogue's stores keeps them out of the output.
  const int rt_raw = n0 / kTileRows + wave;
  const bool n_live = rt_raw < RT;
  const int rt = n_live ? rt_raw : RT - 1;
  const __amdgpu_buffer_rsrc_t rc =
      buffer_rsrc(a.packed + tile_offset(rt, 0, KT), (size_t)KT * kTileBytes);
  const __amdgpu_buffer_rsrc_t ra =
      buffer_rsrc(a.x + (size_t)m0 * K, (size_t)(M - m0) * (size_t)K);

  // activations: the kRT waves of a phase copy its k-tile, BM rows x 128
  // bytes; copy jj of wave `wave` fills rows (BM/kRT) wave + 8 jj .. +7, lane
  // L taking chunk (L & 7) ^ swizzle of row L >> 3 (its LDS position is
  // fixed at 16 L).  Rows past M read row M-1 (they feed only unstored rows).
  int a_v[kACopies];
#pragma unroll
  for (int jj = 0; jj < kACopies; ++jj) {
    const int row = T::kRowsPerWave * wave + 8 * jj + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    a_v[jj] = min(row, M - 1 - m0) * K + c * 16;
  }
  // first input of a copy's chunk in its k-step: the swizzle (row >> 1) & 7
  // of row (BM/kRT) wave + 8 jj + (lane >> 3) is 4 (jj & 1) + (lane >> 4)
  // (BM/kRT is a multiple of 16)
  static_assert(T::kRowsPerWave % 16 == 0, "rows per wave: a multiple of 16");
  int a_k[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) a_k[p] = 16 * ((lane & 7) ^ (4 * p + (lane >> 4)));
  // an offset the descriptor's range check rejects (the copy writes zeros)
  const int a_oob = (size_t)(M - m0) * (size_t)K > 0x7FFFFFFFull ? 0x7FFFFFFF : (M - m0) * K;
  auto a_buf = [&](int b) { return reinterpret_cast<int8_t*>(lds) + (b * KP + kh) * kAStage; };

  v4i acc[kMT][kNT];
#pragma unroll
  for (int i = 0; i < kMT; ++i)
#pragma unroll
    for (int t = 0; t < kNT; ++t) acc[i][t] = v4i{0, 0, 0, 0};

  // this wave's k-tile of step j (KP j + kh, clamped: a prefetch past the
  // end re-reads the last k-tile)
  const int KJ = (KT + KP - 1) / KP;
  auto ktile = [&](int j) { return min(KP * j + kh, KT - 1); };
  // codes, coalesced (lane = tile row)
  auto load_codes = [&](int j, v4u& w, uint32_t& h) {
    const int ks = ktile(j) * kTileBytes;
    w = __builtin_amdgcn_raw_buffer_load_b128(rc, 16 * lane, ks, 0);
    h = __builtin_amdgcn_raw_buffer_load_b32(rc, kTileHiOff + 4 * lane, ks, 0);
  };
  // this wave's share of the activation tile of step j into buffer b
  auto copy_a = [&](int j, int b) {
    const int ka = ktile(j) * kBK;
    int8_t* dst = a_buf(b) + T::kRowsPerWave * wave * kBK;
    // (the k-step offset is added to the lane offset, not passed as the
    // scalar offset, so the descriptor's range check sees the whole offset;
    // chunks past K, in a ragged last k-tile whose codes are padding, take
    // an out-of-range offset and land as zeros)
#pragma unroll
    for (int jj = 0; jj < kACopies; ++jj)
      copy16_to_lds(ra, dst + 8 * jj * kBK, ka + a_k[jj & 1] < K ? a_v[jj] + ka : a_oob);
  };
  const uint8_t* d2 = reinterpret_cast<const uint8_t*>(dec2);
  // the 20-bit code groups of one register stage: lane (l16, g) of block t
  // holds codes 8g..8g+3 of row 16t+l16 (sub-step 0) in the low 20 bits of
  // dword t, and codes 8g+4..8g+7 (sub-step 1) in its top 12 bits and byte t
  // of h.  The empty asm statements make the compiler form both halves here,
  // in registers of their own: left to itself it reads f0 out of the stage
  // registers and forms f1 late, so the code load into the stage that
  // follows gets fresh registers and the loop's back edge copies them back
  // after waiting for every load (measured at N=14336, K=4096: M=128 22.9
  // against 20.5 us with them).
  auto split = [&](const v4u& w, uint32_t h, uint32_t (&f0)[kNT], uint32_t (&f1)[kNT]) {
    const uint32_t wt[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
      f0[t] = wt[t];
      f1[t] = __builtin_amdgcn_alignbit(h >> (8 * t), wt[t], 20);
      asm volatile("" : "+v"(f0[t]), "+v"(f1[t]));
    }
  };
  // Step j (activation buffer b = j % kABufs): its B operands bc0 / bc1 were
  // decoded during step j-1; the register stage (wn, hn) holds the codes of
  // step j+1, decoded during this step's MFMAs into bn0 / bn1 and then
  // refilled with the codes of step j+3.
  // The step barrier.  With 128-row tiles it joins only the kRT waves of
  // this wave's k-phase, which share that phase's activation buffers and
  // nothing else until the epilogue: an LDS arrival count per phase, so the
  // phases' waves (two to a SIMD) need not leave each step together
  // (measured at N=14336, K=4096: M=512 31.7 -> 30.6 us, M=1024 66.6 ->
  // 60.6; with 64-row tiles it was 2 % slower, so those keep s_barrier).
  // The arrival and the polls are LDS instructions in asm: as built-ins the
  // compiler cannot tell them from the activation copies in flight and waits
  // for those first.  The poll is bounded (~0.3 s), so a wave always leaves.
  auto parity_barrier = [&](int j) {   // j: the barrier's index
    const uint32_t pa = (uint32_t)(size_t)((__attribute__((address_space(3))) unsigned*)&parity_arrivals[kh]);
    if (lane == 0) asm volatile("ds_add_u32 %0, %1" ::"v"(pa), "v"(1u) : "memory");
    const unsigned target = (unsigned)kRT * (unsigned)(j + 1);
    for (int spin = 0; spin < (1 << 22); ++spin) {
      unsigned c;
      asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(c) : "v"(pa) : "memory");
      if (__builtin_amdgcn_readfirstlane(c) >= target) break;
      __builtin_amdgcn_s_sleep(1);
    }
  };
  // `even`: j is even (a constant at every call), so with a barrier per two
  // steps the odd steps fold to the decode and the MFMAs.
  auto step = [&](int j, int b, bool even, v4u& wn, uint32_t& hn, const v4i (&bc0)[kNT],
                  const v4i (&bc1)[kNT], v4i (&bn0)[kNT], v4i (&bn1)[kNT]) {
    // every wave's copy of step j (and j+1) has landed and its earlier LDS
    // reads are done; then the buffer of step j-1 is free for the copy of
    // step j+2 (those of j-2, j-1 for j+2, j+3)
    if (!kPair || even) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kNewerLoads));
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (BM == 128)
        parity_barrier(j);
      else
        __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kPair) {
        copy_a(min(j + 2, KJ - 1), (b + 2) & 3);
        copy_a(min(j + 3, KJ - 1), (b + 3) & 3);
      } else if constexpr (kABufs == 3) {
        copy_a(min(j + 2, KJ - 1), b == 0 ? 2 : b - 1);
      } else {
        copy_a(min(j + 1, KJ - 1), b ^ 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    uint32_t f0[kNT], f1[kNT];
    split(wn, hn, f0, f1);
    load_codes(min(j + 3, KJ - 1), wn, hn);
    __builtin_amdgcn_sched_barrier(0);
    if (KP * j + kh < KT)    // KT not a multiple of KP: the last step is short
      mg_mfma<true, kMT>(acc, bc0, bc1, a_buf(b), l16, g, f0, f1, bn0, bn1, d2);
    else
      mg_mfma<false, kMT>(acc, bc0, bc1, a_buf(b), l16, g, f0, f1, bn0, bn1, d2);
  };

  // Two register stages of codes and two sets of B operands, ping-pong.
  // Issue order (the barrier's vmcnt counts on it): codes 0, copy 0,
  // codes 1, copy 1 (three buffers only), codes 2, then per step j:
  // barrier, copy j+2 (j+1 with two buffers), codes j+3.  With a barrier
  // per two steps: codes 0, copy 0, copy 1, codes 1, codes 2, then per
  // even step j: barrier, copies j+2 and j+3, codes j+3; per odd step:
  // codes j+3.
  v4u w0, w1;
  uint32_t h0, h1;
  v4i bA0[kNT], bA1[kNT], bB0[kNT], bB1[kNT];
  load_codes(0, w0, h0);
  __builtin_amdgcn_sched_barrier(0);
  copy_a(0, 0);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (kPair) {
    copy_a(min(1, KJ - 1), 1);
    __builtin_amdgcn_sched_barrier(0);
  }
  load_codes(min(1, KJ - 1), w1, h1);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (!kPair && kABufs == 3) copy_a(min(1, KJ - 1), 1);
  __builtin_amdgcn_sched_barrier(0);
  // decode table written (LDS only: the copies stay in flight)
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  __builtin_amdgcn_sched_barrier(0);
  {
    uint32_t f0[kNT], f1[kNT];
    split(w0, h0, f0, f1);
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
      bA0[t] = mg_decode4(f0[t], d2);
      bA1[t] = mg_decode4(f1[t], d2);
    }
    load_codes(min(2, KJ - 1), w0, h0);
    __builtin_amdgcn_sched_barrier(0);
  }

  int j = 0, b = 0;
  for (; j + 2 <= KJ; j += 2) {
    step(j, b, true, w1, h1, bA0, bA1, bB0, bB1);
    b = b + 1 == kABufs ? 0 : b + 1;
    step(j + 1, b, false, w0, h0, bB0, bB1, bA0, bA1);
    b = b + 1 == kABufs ? 0 : b + 1;
  }
  if (j < KJ) step(j, b, true, w1, h1, bA0, bA1, bB0, bB1);
  // the clamped copies past the end may still be landing in LDS, which the
  // epilogue reuses
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));

  // Epilogue, 32 rows (two row blocks) at a time: every wave writes its raw
  // int32 sums into its phase's row-major LDS tile, then each thread adds
  // the KP phases for 4 consecutive columns of one row and stores
  // y = ((float)acc * s_x[m]) * alpha[n] (or the int32 sum), 16 bytes per
  // lane, so each store instruction writes whole 128-byte lines, marked
  // non-temporal (the output is not read again here: measured 7 % faster at
  // M=512, N=14336, K=4096, where the 29 MB of fp32 output bound it).  Lane
  // (l16, g) of a 16 x 16 MFMA block holds column l16, rows 4g..4g+3.  The
  // scales are read once, before the first barrier.
  const bool want_y = a.y != nullptr;
  const int c4 = tid & (kBN / 4 - 1);          // this thread's 4 columns
  const int n = n0 + 4 * c4;
  float4 al4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (want_y && n < N) al4 = make_float4(a.alpha[n], a.alpha[n + 1], a.alpha[n + 2], a.alpha[n + 3]);
  if (want_y && tid < kBM) sxs[tid] = a.s_x[min(m0 + tid, M - 1)];
  // The scale loads complete here, before the first output store.  The
  // memory counter counts stores as well as loads, so a wait for alpha
  // placed after a store also waits for that store; left to itself the
  // compiler puts such a wait before every row's scaling, and the tile's
  // 16 rows of stores then leave one round trip at a time.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
  int* ot = reinterpret_cast<int*>(lds);       // [phase][32][kOutLd] sums
  int* mine = ot + kh * 32 * kOutLd;
#pragma unroll
  for (int qq = 0; qq < kMT / 2; ++qq) {
    __syncthreads();  // the previous use of the LDS area is finished
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < kNT; ++t)
          mine[(16 * ii + 4 * g + r) * kOutLd + wave * kTileRows + 16 * t + l16] = acc[2 * qq + ii][t][r];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 32 * (kBN / 4) / kThreads; ++k) {
      const int ml = tid / (kBN / 4) + (kThreads / (kBN / 4)) * k;   // row within the 32
      const int m = m0 + 32 * qq + ml;
      v4i sum = *reinterpret_cast<const v4i*>(&ot[ml * kOutLd + 4 * c4]);
#pragma unroll
      for (int ph = 1; ph < KP; ++ph) sum += *reinterpret_cast<const v4i*>(&ot[(ph * 32 + ml) * kOutLd + 4 * c4]);
      if (m < M && n < N) {
        if (want_y) {
          const float sx = sxs[32 * qq + ml];
          const float4 v = make_float4(((float)sum.x * sx) * al4.x, ((float)sum.y * sx) * al4.y,
                                       ((float)sum.z * sx) * al4.z, ((float)sum.w * sx) * al4.w);
          __builtin_nontemporal_store(__builtin_bit_cast(v4u, v), reinterpret_cast<v4u*>(a.y + (size_t)m * N + n));
        } else {
          __builtin_nontemporal_store(sum, reinterpret_cast<v4i*>(a.acc + (size_t)m * N + n));
        }
      }
    }
  }
}

template <int BM, int KP>
hipError_t launch_tiles(const GemmPlan& p, const GemmArgs& a, hipStream_t stream) {
  const int nt = (a.N + Tiling<BM, KP>::kBN - 1) / Tiling<BM, KP>::kBN;
  launch_product_kernel(mfma_gemm_kernel<BM, KP>, dim3(p.grid), dim3(kThreads), 0, stream, a, nt, 0);
  return hipGetLastError();
}

}  // namespace

// Static LDS per workgroup: activation buffers (or epilogue tiles), the pair
// table, the tile's s_x and, with 128-row tiles, the phase counters.
int mfma_gemm_lds_bytes(int bm, int kp) {
  const int main_bytes = bm == 128 ? (kp == 4 ? Tiling<128, 4>::kLdsBytes : Tiling<128, 2>::kLdsBytes)
                         : kp == 4 ? Tiling<64, 4>::kLdsBytes
                                   : Tiling<64, 2>::kLdsBytes;
  return main_bytes + 1024 * 8 + bm * 4 + (bm == 128 ? 4 * kp : 0);
}

int mfma_gemm_threads() { return kThreads; }

int mfma_gemm_grid(int M, int N, int bm, int kp) {
  const int bn = kThreads / 64 / kp * kTileRows;
  const int mt = (M + bm - 1) / bm, nt = (N + bn - 1) / bn;
  const int per_xcd = (nt + 7) / 8;
  return 8 * per_xcd * mt;
}

// plan.rw carries the tile height in units of 64 activation rows (1 or 2),
// plan.ch the k-phases (2 or 4).
hipError_t launch_mfma_gemm(const GemmPlan& p, const GemmArgs& a, hipStream_t stream) {
  if (p.rw == 1 && p.ch == 4) return launch_tiles<64, 4>(p, a, stream);
  if (p.rw == 1 && p.ch == 2) return launch_tiles<64, 2>(p, a, stream);
  if (p.rw == 2 && p.ch == 4) return launch_tiles<128, 4>(p, a, stream);
  if (p.rw == 2 && p.ch == 2) return launch_tiles<128, 2>(p, a, stream);
  return hipErrorInvalidValue;
}

}  // namespace sherry
