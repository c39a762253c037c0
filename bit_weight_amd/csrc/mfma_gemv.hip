// Small-M (decode and short chunks, M <= 64 per launch) product on the matrix cores:
// the 5-bit codes are decoded to int8 {-1,0,+1} in registers and contracted
// with the int8 activations by v_mfma_i32_16x16x64_i8, the M tokens padded
// to whole blocks of the instruction's 16 rows (one decoded operand feeds
// the instruction of every block).  y = ((float)acc * s_x[m]) * alpha[n] as in every
// path.  [Sherry page §2.2] computes the same integer sums through
// per-segment tables of pattern dot products; on gfx950 a decoded code pair
// feeds 8 multiply-adds per token of a matrix-core instruction for one LDS
// lookup and two VALU ops, where a table lookup costs one LDS read and about
// three VALU ops per block and token pair, so this form streams the codes at
// a higher rate.
//
// Mapping (wave64):
//  * A workgroup owns one format row tile (64 weight rows = 4 MFMA column
//    blocks of 16) and one K-split; its KW waves (4, 8 or 16) take the
//    split's k-tiles (128 inputs each) in turn, so many waves stream one row
//    tile and the whole grid keeps enough bytes in flight to cover HBM
//    latency.  The waves add their sums through LDS at the end; K-splits
//    across workgroups add theirs with the one-round-trip 64-bit atomic
//    count used by the lookup-table GEMV.
//  * B operand: lane l of a column block holds weight row l % 16; lane group
//    g = l / 16 takes codes 8g..8g+7 of the k-tile (the first four in MFMA
//    sub-step 0, the rest in sub-step 1).  The format stores exactly those
//    40 bits of the four column blocks' rows in slot l of the tile (16 + 4
//    bytes), so a wave loads its tile coalesced, lane l = slot l, and holds
//    every operand in place: block t's group is dword t plus byte t of the
//    slot's last dword.  (Stored row by row, the groups took two 4 x 4 lane
//    transposes per k-tile; measured without them: M=8, K=8192, N=28672
//    11.07 -> 10.8 us, M=1, K=4096, N=11008 4.72 -> 4.43.)  A 1024-entry
//    LDS table maps a 10-bit code pair to its 8 int8 weights.
//  * A operand: lane (l % 16, g) holds token 16b + l % 16 of block b, inputs 32g + 16s .. +15
//    of the k-tile in sub-step s (the same input order as B, which the dot
//    product does not see).  Loaded straight from global memory through a
//    buffer descriptor whose range ends at token M, so the padding tokens
//    read as zero without a branch.
//  * Fused form (FQ): the activations arrive as fp32.  Every workgroup reads
//    its tokens' whole rows once for the per-token scale s = max|x| / 127
//    (the same arithmetic as the stand-alone quantizer, so q and s are
//    bit-identical to it), quantizes the k-tiles of its K-split into LDS and
//    reads the A operands from there; this saves the quantizer's launch and
//    its round trip through memory on the decode path.
//  * Codes and activations are prefetched into register stages used in
//    turn: four (three or two with several token blocks) in the looped
//    form, so each wave keeps ~5 KB of its codes in flight (HBM streaming
//    needs bytes in flight x latency to cover the bandwidth); two in the
//    straight-line form, whose grids are large enough that the loads of
//    all waves saturate HBM anyway: there every wave must issue its first
//    stages before it decodes anything, and at launch the memory system
//    accepts them only as fast as it serves them (per-wave clock stamps at
//    M=8, K=8192, N=28672: ~2.3 us median from entry to the first decode
//    with four stages).
#include "sherry_device.h"
#include "sherry_launch.h"

namespace sherry {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int kBlk = kTileRows / 16;   // MFMA column blocks per wave
constexpr int kSL = 8;                 // most k-tiles per wave of the straight-line form
constexpr int kRedLd = kTileRows + 4;  // words per token row of the epilogue tile

__device__ __forceinline__ __amdgpu_buffer_rsrc_t gemv_rsrc(const void* base, size_t bytes) {
  const int n = bytes > 0x7FFFFFFFull ? 0x7FFFFFFF : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

// B operand of one sub-step: 4 codes (20 bits of v) as two code pairs.
__device__ __forceinline__ v4i decode4(uint32_t v, const uint8_t* dec2) {
  const uint2 e0 = *reinterpret_cast<const uint2*>(dec2 + ((v << 3) & 0x1FF8u));
  const uint2 e1 = *reinterpret_cast<const uint2*>(dec2 + ((v >> 7) & 0x1FF8u));
  return v4i{(int)e0.x, (int)e0.y, (int)e1.x, (int)e1.y};
}

// B operand of one sub-step in the 2-bit baseline format: 16 weights (one
// dword of 2-bit codes) as four byte-indexed lookups of 4 int8 weights.
__device__ __forceinline__ v4i decode16(uint32_t v, const uint32_t* tbl) {
  return v4i{(int)tbl[v & 255u], (int)tbl[(v >> 8) & 255u], (int)tbl[(v >> 16) & 255u],
             (int)tbl[v >> 24]};
}

__device__ __forceinline__ float amax4(const float4 v) {
  return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

// Activations of 16-token blocks are loaded four lanes per row (lane
// 4r + g: token r, inputs 32g..32g+31), so each group of four lanes reads
// one 128-byte line, and moved to the MFMA layout (lane 16g + r) by LDS
// crossbar permutes; token-per-lane loads put four lines under every four
// lanes.  Measured at N=14336, K=4096: M=16 7.9 -> 7.8 us, M=32 10.2 -> 8.9,
// M=64 16.6 -> 12.6; for 8-token blocks the permutes cost more than they
// save (M=8, K=8192, N=28672: 14.0 -> 15.6 us), so those keep the direct form.
constexpr bool quad_x(int MT, int MB) { return MT == 16 && MB >= 1; }

// KW waves share one row tile; MT = the token count of one MFMA token block
// rounded up to a power of two (1..16); MB = token blocks of 16 (MB > 1 only
// with MT = 16: up to 64 tokens, each decoded code feeding MB instructions);
// FQ = fused activation quantization (MT <= 4); FMT = code format: 0 = the
// 5-bit Sherry code, 1 = the 2-bit baseline packing (its tile row is 8
// dwords: lane group g takes dwords 2g and 2g+1, the same inputs
// 32g..32g+31, through the same two transposes).  ST = register stages.
// FS = fused form: float4 loads per thread covering the tokens' rows
// (>= M*K / (4 * 64 * KW); the launch picks the smallest power of two).
// SX = staged int8 activations: the split's x copied to LDS once, as in the
// fused form, instead of loaded per k-tile (the launch uses it at M = 1).
template <int KW, int MT, int MB, bool FQ, int FMT, int ST, int FS = 1, bool SX = false, bool SL = false>
__global__ __launch_bounds__(64 * KW) void mfma_gemv_kernel(const uint8_t* packed, const int8_t* x,
                                                            const float* xf, int M, int N, int K, int splits,
                                                            int kt_per_split, const float* s_x,
                                                            const float* alpha, float* y, int32_t* acc_out,
                                                            int32_t* partials) {
  const GemmArgs a = product_args(packed, x, xf, M, N, K, s_x, alpha, y, acc_out, partials);
  static_assert(MB == 1 || (MT == 16 && !FQ), "several token blocks are whole blocks of 16");
  static_assert(!SX || (!FQ && MB == 1 && MT <= 4), "staged int8 activations: at most 4 tokens");
  constexpr bool LX = FQ || SX;   // A operands read from the split's activations in LDS
  constexpr bool XQ = !FQ && quad_x(MT, MB);
  constexpr int kStages = ST;
  constexpr int NT = 64 * KW;
  constexpr int TB = FMT == 0 ? kTileBytes : kTile2Bytes;   // bytes per format tile
  __shared__ __attribute__((aligned(16))) uint32_t tbl2[FMT == 1 ? 256 : 1];
  constexpr int QS = LX ? kFuseMaxSpan * kTileK : 16;   // int8 activations per token in LDS
  __shared__ __attribute__((aligned(16))) uint2 dec2[1024];
  __shared__ __attribute__((aligned(16))) int red[KW * MT * kRedLd];   // [wave][token][row]
  // [token][k in split] int8, held as 32-bit words: written and read only as
  // 32-bit lanes, so no access reinterprets another type's storage
  __shared__ __attribute__((aligned(16))) uint32_t qs[LX ? MT * QS / 4 : 4];
  __shared__ float sred[FQ ? KW * MT + MT : 1];                          // partial maxima, scales

  const int KT = k_tiles(K);
  const int rt = blockIdx.x / splits;
  const int s = blockIdx.x - rt * splits;
  const int tid = threadIdx.x, lane = tid & 63;
  const int q = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar offsets
  const int l16 = lane & 15, g = lane >> 4;

  const int kt_begin = s * kt_per_split;
  const int kt_end = min(KT, kt_begin + kt_per_split);
  const int span = kt_end - kt_begin;
  const int nk = span > q ? (span - q + KW - 1) / KW : 0;

  // buffer descriptors: this row tile's codes, and the M tokens of x
  const size_t tb = (size_t)rt * KT * TB;
  const __amdgpu_buffer_rsrc_t rc = gemv_rsrc(a.packed + tb, (size_t)KT * TB);
  const __amdgpu_buffer_rsrc_t rx = gemv_rsrc(a.x, (size_t)M * (size_t)K);
  // an offset the descriptor's range check rejects (the load returns zeros)
  const int x_oob = (size_t)M * (size_t)K > 0x7FFFFFFFull ? 0x7FFFFFFF : M * K;
  // first input of the 16-byte chunks this lane loads (lane group g, or in
  // the four-lanes-per-row load layout g' = lane & 3)
  const int x_k = 32 * (XQ ? (lane & 3) : g);
  // lane offset of the activations (>= M*K for the padding tokens; the
  // k-tile offset is added to it, not passed as the scalar offset, so the
  // descriptor's range check sees the whole offset)
  const int x_v = XQ ? (lane >> 2) * K + 32 * (lane & 3) : l16 * K + 32 * g;
  const int xq_src = 4 * (4 * l16 + g);       // permute address: lane 16g + r <- lane 4r + g

  // i-th k-tile of this wave (clamped: the prefetch past the end re-reads
  // the last tile, whose values are never used)
  // (unconditional, so no branch merges the stage registers: a wave without
  // k-tiles reads a valid tile of its row tile and never uses it)
  auto load = [&](int i, v4u& w, v4u& h, v4u (&x0)[MB], v4u (&x1)[MB]) {
    const int kt = min(kt_begin + q + KW * max(min(i, nk - 1), 0), KT - 1);
    const int ks = kt * TB, ka = kt * kTileK;
    w = __builtin_amdgcn_raw_buffer_load_b128(rc, 16 * lane, ks, 0);
    if constexpr (FMT == 0) {
      h = v4u{__builtin_amdgcn_raw_buffer_load_b32(rc, kTileHiOff + 4 * lane, ks, 0), 0u, 0u, 0u};
    } else {
      h = __builtin_amdgcn_raw_buffer_load_b128(rc, kTile2HiOff + 16 * lane, ks, 0);
    }
    // chunks past K (a ragged last k-tile, whose codes are padding) load as
    // zeros: the offset is chosen before the load, so nothing waits for it
    const bool in0 = ka + x_k < K, in1 = ka + x_k + 16 < K;
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      if constexpr (!LX) {
        x0[b] = __builtin_amdgcn_raw_buffer_load_b128(rx, in0 ? x_v + 16 * b * K + ka : x_oob, 0, 0);
        x1[b] = __builtin_amdgcn_raw_buffer_load_b128(rx, in1 ? x_v + 16 * b * K + ka + 16 : x_oob, 0, 0);
      } else {
        x0[b] = v4u{0u, 0u, 0u, 0u};
        x1[b] = v4u{0u, 0u, 0u, 0u};
      }
    }
  };

  v4i acc[MB][kBlk];
#pragma unroll
  for (int b = 0; b < MB; ++b)
#pragma unroll
    for (int t = 0; t < kBlk; ++t) acc[b][t] = v4i{0, 0, 0, 0};

  // Fused form: the tokens' fp32 rows (M*K <= kFuseMaxMK floats) in one
  // burst of loads, issued before the codes so that waiting for them does
  // not wait for the code loads behind them.  Thread tid holds float4 F =
  // tid + NT*j of the [M,K] block (zero past its end, through the buffer
  // descriptor's range).
  v4u xv[FS];
  if constexpr (FQ) {
    const __amdgpu_buffer_rsrc_t rxf = gemv_rsrc(a.xf, (size_t)M * (size_t)K * 4);
#pragma unroll
    for (int j = 0; j < FS; ++j) xv[j] = __builtin_amdgcn_raw_buffer_load_b128(rxf, 16 * (tid + NT * j), 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  // Staged form (SX, int8 x, M <= 4): the split's activations as 16-byte
  // chunks, chunk c = tid + NT*j of [token][k in split] (span*8 per token),
  // loaded once, coalesced and ahead of the codes, and put in LDS below;
  // chunks past K or past the last token read as zeros
  constexpr int XCH = SX ? (MT * kFuseMaxSpan * 8 + NT - 1) / NT : 1;
  const int per_tok = span * 8;
  auto chunk_token = [&](int c) { return (c >= per_tok) + (c >= 2 * per_tok) + (c >= 3 * per_tok); };
  v4u xs[XCH];
  if constexpr (SX) {
#pragma unroll
    for (int j = 0; j < XCH; ++j) {
      const int c = tid + NT * j;
      const int m = chunk_token(c);
      const int jj = c - m * per_tok;   // chunk within the token's split (>= per_tok: none)
      const int k = kt_begin * kTileK + 16 * jj;
      xs[j] = __builtin_amdgcn_raw_buffer_load_b128(rx, m < M && jj < per_tok && k < K ? m * K + k : x_oob,
                                                    0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // kStages register stages, filled kStages k-tiles ahead and used in turn.
  // The scheduling barriers keep every refill inside its own step, so a step
  // waits only for its own stage while the newer ones stay in flight.
  v4u cw[kStages];
  v4u ch[kStages];
  v4u xa[kStages][MB], xb[kStages][MB];
#pragma unroll
  for (int st = 0; st < kStages; ++st) {
    load(st, cw[st], ch[st], xa[st], xb[st]);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (FMT == 0) {
    for (int i = tid; i < 1024; i += 64 * KW) dec2[i] = make_uint2(code_word(i & 31), code_word(i >> 5));
  } else {
    for (int i = tid; i < 256; i += 64 * KW) tbl2[i] = code2_word(i);
  }
  if constexpr (FQ) {
    // per-token scale over the whole row (every workgroup reads its tokens'
    // rows): the token of float4 F is the number of row ends at or below it
    const int K4 = K / 4;
    auto token_of = [&](int F) { return (F >= K4) + (F >= 2 * K4) + (F >= 3 * K4); };
    float am[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) am[m] = 0.0f;
#pragma unroll
    for (int j = 0; j < FS; ++j) {
      const int m = token_of(tid + NT * j);
      const float v = amax4(__builtin_bit_cast(float4, xv[j]));
#pragma unroll
      for (int mm = 0; mm < MT; ++mm)
        if (m == mm) am[mm] = fmaxf(am[mm], v);
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      am[m] = wave_max(am[m]);
      if (lane == 0) sred[q * MT + m] = am[m];
    }
    __syncthreads();
    if (tid < MT) {
      float v = 0.0f;
#pragma unroll
      for (int qq = 0; qq < KW; ++qq) v = fmaxf(v, sred[qq * MT + tid]);
      sred[KW * MT + tid] = v > 0.0f ? v / 127.0f : 1.0f;   // s = max|x| / 127; a zero row -> 1
    }
    __syncthreads();
    // quantize this split's k-tiles of every token into LDS, from the
    // registers: q = clamp(rint(x / s))
    const int e0 = kt_begin * (kTileK / 4), e1 = e0 + span * (kTileK / 4);
#pragma unroll
    for (int j = 0; j < FS; ++j) {
      const int F = tid + NT * j;
      const int m = token_of(F);
      const int e = F - m * K4;
      if (m < M && e >= e0 && e < e1) {
        const float sm = sred[KW * MT + m];
        const float4 v = __builtin_bit_cast(float4, xv[j]);
        const uint32_t b0 = (uint8_t)(int8_t)fminf(fmaxf(rintf(v.x / sm), -127.0f), 127.0f);
        const uint32_t b1 = (uint8_t)(int8_t)fminf(fmaxf(rintf(v.y / sm), -127.0f), 127.0f);
        const uint32_t b2 = (uint8_t)(int8_t)fminf(fmaxf(rintf(v.z / sm), -127.0f), 127.0f);
        const uint32_t b3 = (uint8_t)(int8_t)fminf(fmaxf(rintf(v.w / sm), -127.0f), 127.0f);
        qs[(m * QS) / 4 + (e - e0)] = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
      }
    }
    // a ragged last k-tile: inputs past K read as zero
    for (int e = max(e0, K4) + tid; e < e1; e += NT)
#pragma unroll
      for (int m = 0; m < MT; ++m)
        if (m < M) qs[(m * QS) / 4 + (e - e0)] = 0u;
  }
  if constexpr (SX) {
#pragma unroll
    for (int j = 0; j < XCH; ++j) {
      const int c = tid + NT * j;
      const int m = chunk_token(c);
      const int jj = c - m * per_tok;
      if (m < M && jj < per_tok) *reinterpret_cast<v4u*>(&qs[(m * QS) / 4 + 4 * jj]) = xs[j];
    }
  }
  lds_barrier();
  const uint8_t* d2 = reinterpret_cast<const uint8_t*>(dec2);

  auto step = [&](int i, bool refill, v4u& w, v4u& h, v4u (&x0)[MB], v4u (&x1)[MB]) {
    uint32_t f0[kBlk], f1[kBlk];
    if constexpr (FMT == 0) {
      // block t: this lane's 40-bit group is dword t (codes 8g..8g+3 in its
      // low 20 bits) and byte t of h (with the dword's top 12 bits, codes
      // 8g+4..8g+7)
      const uint32_t wt[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int t = 0; t < kBlk; ++t) {
        f0[t] = wt[t];
        f1[t] = __builtin_amdgcn_alignbit(h.x >> (8 * t), wt[t], 20);
      }
    } else {
      // lane (l16, g) of block t <- dwords 2g (sub-step 0) and 2g+1 (sub-step 1)
      transpose4(w.x, w.z, h.x, h.z, f0);
      transpose4(w.y, w.w, h.y, h.w, f1);
    }
    v4i a0[MB], a1[MB];
    if constexpr (LX) {
      // token l16 (zero past M), inputs 32g + 16s of this wave's i-th k-tile
      const uint32_t* src = &qs[(min(l16, M - 1) * QS + (q + KW * i) * kTileK + 32 * g) / 4];
      const v4i v0 = __builtin_bit_cast(v4i, *reinterpret_cast<const v4u*>(src));
      const v4i v1 = __builtin_bit_cast(v4i, *reinterpret_cast<const v4u*>(src + 4));
      const v4i z{0, 0, 0, 0};
      a0[0] = l16 < M ? v0 : z;
      a1[0] = l16 < M ? v1 : z;
    } else {
#pragma unroll
      for (int b = 0; b < MB; ++b) {
        a0[b] = __builtin_bit_cast(v4i, x0[b]);
        a1[b] = __builtin_bit_cast(v4i, x1[b]);
        if constexpr (XQ) {
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            a0[b][d] = __builtin_amdgcn_ds_bpermute(xq_src, a0[b][d]);
            a1[b][d] = __builtin_amdgcn_ds_bpermute(xq_src, a1[b][d]);
          }
        }
      }
    }
    if (refill) load(i + kStages, w, h, x0, x1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < kBlk; ++t) {
      const v4i bw = FMT == 0 ? decode4(f0[t], d2) : decode16(f0[t], tbl2);
#pragma unroll
      for (int b = 0; b < MB; ++b) acc[b][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0[b], bw, acc[b][t], 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < kBlk; ++t) {
      const v4i bw = FMT == 0 ? decode4(f1[t], d2) : decode16(f1[t], tbl2);
#pragma unroll
      for (int b = 0; b < MB; ++b) acc[b][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1[b], bw, acc[b][t], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  if constexpr (SL) {
    // at most kSL k-tiles per wave: straight-line steps, so no loop carries
    // the in-flight stage registers around a back edge (there the compiler
    // copies them into place, waiting for every load).  Past the wave's
    // last k-tile only the arithmetic is skipped; the refills are issued
    // regardless (re-reading its last tile), so no branch merges the stage
    // registers.
#pragma unroll
    for (int i = 0; i < kSL; ++i) {
      const int st = i % kStages;
      if (i < nk) step(i, false, cw[st], ch[st], xa[st], xb[st]);
      if (i + kStages < kSL) load(i + kStages, cw[st], ch[st], xa[st], xb[st]);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    int i = 0;
    for (; i + kStages <= nk; i += kStages) {
#pragma unroll
      for (int st = 0; st < kStages; ++st) step(i + st, true, cw[st], ch[st], xa[st], xb[st]);
    }
#pragma unroll
    for (int st = 0; st < kStages - 1; ++st)
      if (i + st < nk) step(i + st, true, cw[st], ch[st], xa[st], xb[st]);
  }

  // Epilogue, one token block at a time.  Every wave writes its sums to LDS
  // as [token][row]; then each lane owns one weight row and a fixed set of
  // tokens, so the K-split atomics of a lane are issued back to back (the
  // token test between them is wave-uniform) and cost one memory round trip.
  // Padding rows (past N) and padding tokens (past M) issue no atomic: as
  // no-op atomics on one valid cell, the 60 padding lanes of a ragged last
  // row tile would all hit one address, and the L2 serializes those (measured
  // at M=5, K=8192: N=4100 took 23.7 us against 6.3 at N=4096).
  constexpr int TPW = MT >= KW ? MT / KW : 1;        // tokens per wave and block
  const int n = rt * kTileRows + lane;
  const bool n_ok = n < N;                            // rows past N: padding, never stored
  const float al = a.y && n_ok ? a.alpha[n] : 0.0f;
  // the scales of this wave's tokens, loaded with alpha before any atomic
  // or store (the memory counter counts stores too: a scale loaded after a
  // store would make the next store wait for that one)
  float sxm[MB][TPW];
#pragma unroll
  for (int b = 0; b < MB; ++b)
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int m = 16 * b + q * TPW + i;
      sxm[b][i] = !FQ && a.y && q * TPW < MT && m < M ? a.s_x[m] : 0.0f;
    }
#pragma unroll
  for (int b = 0; b < MB; ++b) {
    if (b > 0) __syncthreads();   // the previous block's sums are read
#pragma unroll
    for (int t = 0; t < kBlk; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (4 * g + j < MT) red[(q * MT + 4 * g + j) * kRedLd + 16 * t + l16] = acc[b][t][j];
    __syncthreads();
    if (q * TPW >= MT) continue;
    int total[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int m = q * TPW + i;
      int v = 0;
#pragma unroll
      for (int qq = 0; qq < KW; ++qq) v += red[(qq * MT + m) * kRedLd + lane];
      total[i] = v;
    }
    bool last[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) last[i] = true;
    if (splits > 1) {
      unsigned long long* cells = reinterpret_cast<unsigned long long*>(a.partials);
      unsigned long long now[TPW];
#pragma unroll
      for (int i = 0; i < TPW; ++i) now[i] = 0ull;
      if (n_ok) {
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
          const int m = 16 * b + q * TPW + i;
          if (m < M)
            now[i] = __hip_atomic_fetch_add(cells + (size_t)m * N + n,
                                            (1ull << 32) + (unsigned long long)(long long)total[i],
                                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int m = 16 * b + q * TPW + i;
        now[i] += (1ull << 32) + (unsigned long long)(long long)total[i];
        total[i] = (int)(uint32_t)now[i];
        // the high word minus the borrow of a negative low word = arrivals
        last[i] = (((long long)now[i] - (long long)total[i]) >> 32) == (long long)splits;
        if (m < M && n_ok && last[i])
          __hip_atomic_store(cells + (size_t)m * N + n, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    // every output formed before the first store (the empty asm keeps each
    // product out of the store branches): the wait for alpha then comes
    // once, not between stores
    float yv[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int m = min(16 * b + q * TPW + i, MT - 1);
      yv[i] = ((float)total[i] * (FQ ? sred[KW * MT + m] : sxm[b][i])) * al;
      asm volatile("" : "+v"(yv[i]));
    }
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int m = 16 * b + q * TPW + i;
      if (m >= M || !n_ok || !last[i]) continue;
      if (a.y) {
        a.y[(size_t)m * N + n] = yv[i];
      } else {
        a.acc[(size_t)m * N + n] = total[i];
      }
    }
  }
}

template <int KW, int MT, int FS>
hipError_t launch_fused_fs(const GemmPlan& p, const GemmArgs& a, hipStream_t stream, int need) {
  if constexpr (FS < kFuseMaxMK / 4 / (64 * KW)) {
    if (need > FS) return launch_fused_fs<KW, MT, 2 * FS>(p, a, stream, need);
  }
  if (need > FS) return hipErrorInvalidValue;
  launch_product_kernel(mfma_gemv_kernel<KW, MT, 1, true, 0, 4, FS>, dim3(p.grid), dim3(64 * KW), 0, stream, a, p.splits, p.kt_per_split);
  return hipGetLastError();
}

template <int KW, bool FQ, int FMT>
hipError_t launch_kw(const GemmPlan& p, const GemmArgs& a, hipStream_t stream) {
  const dim3 grid(p.grid), block(64 * KW);
  if constexpr (FQ) {
    // fused form: float4 loads per thread for the tokens' rows
    const int need = (a.M * (a.K / 4) + 64 * KW - 1) / (64 * KW);
    if (a.M <= 1) return launch_fused_fs<KW, 1, 1>(p, a, stream, need);
    if (a.M <= 2) return launch_fused_fs<KW, 2, 1>(p, a, stream, need);
    if (a.M <= 4) return launch_fused_fs<KW, 4, 1>(p, a, stream, need);
    return hipErrorInvalidValue;
  } else {
    // one token: its split's int8 x staged in LDS (measured 2-4 % faster at
    // M=1; at M=4 the chunk loads, sized for the longest split, cost more
    // than the per-step loads they replace)
    // straight-line steps for one token block and 4 to 8 k-tiles per wave
    // (measured at M=8, K=8192, N=28672: 13.4 -> 12.2 us; with fewer k-tiles
    // the loop never takes its back edge, and with several token blocks it
    // was 2 % slower), with two register stages (against four, measured on
    // MI355X: M=8, K=8192, N=28672 12.5 -> 11.9 us; M=16, K=4096, N=14336
    // 6.8 -> 6.1; M=1, K=4096, N=11008 4.99 -> 4.73; no shape slower), also
    // under a K-split (the long-K plans split K to reach this form; N=8192,
    // K=28672, 4 splits of 7 k-tiles per wave: M=1 11.4 -> 10.2 us, M=4
    // 11.7 -> 10.8, M=8 11.8 -> 11.4)
    const int nkw = (p.kt_per_split + KW - 1) / KW;
    const bool sl4 = nkw >= 4 && nkw <= kSL;
#define SHERRY_GEMV(MT_, MB_, ST_, SX_, SL_) \
  launch_product_kernel(mfma_gemv_kernel<KW, MT_, MB_, false, FMT, ST_, 1, SX_, SL_>, grid, block, 0, stream, a, p.splits, p.kt_per_split)
    if (a.M <= 1 && p.kt_per_split <= kFuseMaxSpan) {
      if (sl4) SHERRY_GEMV(1, 1, 2, true, true); else SHERRY_GEMV(1, 1, 4, true, false);
    } else if (a.M <= 1) {
      if (sl4) SHERRY_GEMV(1, 1, 2, false, true); else SHERRY_GEMV(1, 1, 4, false, false);
    } else if (a.M <= 2) {
      if (sl4) SHERRY_GEMV(2, 1, 2, false, true); else SHERRY_GEMV(2, 1, 4, false, false);
    } else if (a.M <= 4) {
      if (sl4) SHERRY_GEMV(4, 1, 2, false, true); else SHERRY_GEMV(4, 1, 4, false, false);
    } else if (a.M <= 8) {
      if (sl4) SHERRY_GEMV(8, 1, 2, false, true); else SHERRY_GEMV(8, 1, 4, false, false);
    } else if (a.M <= 16) {
      if (sl4) SHERRY_GEMV(16, 1, 2, false, true); else SHERRY_GEMV(16, 1, 4, false, false);
    } else if constexpr (FMT == 0 && KW <= 8) {   // 16 waves leave too few registers for two blocks
      if (a.M <= 32) {
        SHERRY_GEMV(16, 2, 3, false, false);
      } else if (a.M <= kGemvMaxM) {
        SHERRY_GEMV(16, 4, 2, false, false);
      } else {
        return hipErrorInvalidValue;
      }
    } else {
      return hipErrorInvalidValue;
    }
#undef SHERRY_GEMV
    return hipGetLastError();
  }
}

template <bool FQ, int FMT>
hipError_t launch_fq(const GemmPlan& p, const GemmArgs& a, hipStream_t stream) {
  switch (p.rw) {
    case 4: return launch_kw<4, FQ, FMT>(p, a, stream);
    case 8: return launch_kw<8, FQ, FMT>(p, a, stream);
    case 16: return launch_kw<16, FQ, FMT>(p, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// The fused form takes up to kFuseMaxM tokens whose rows (M*K fp32) every
// workgroup reads once, and K-splits of at most kFuseMaxSpan k-tiles.
bool mfma_gemv_fusable(const GemmPlan& p, int M, int K) {
  return p.path == 2 && M <= kFuseMaxM && (long long)M * K <= kFuseMaxMK &&
         p.kt_per_split <= kFuseMaxSpan;
}

// plan.rw carries the waves per row tile for this path (4, 8 or 16).
hipError_t launch_mfma_gemv(const GemmPlan& p, const GemmArgs& a, hipStream_t stream) {
  return a.xf ? launch_fq<true, 0>(p, a, stream) : launch_fq<false, 0>(p, a, stream);
}

hipError_t launch_mfma_gemv2(const GemmPlan& p, const GemmArgs& a, hipStream_t stream) {
  if (a.xf) return hipErrorInvalidValue;
  return launch_fq<false, 1>(p, a, stream);
}

}  // namespace sherry
