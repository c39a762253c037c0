// Kernels 2 + 3: per-segment lookup tables in LDS and the small-M LUT-GEMV.
//
// [Sherry page §2.2] the activations are cut into 4-element segments; for
// every segment a table of the 16 canonical pattern dot products is built;
// each weight block is then one table lookup, its sign is applied and the
// results are summed in integers, with one float rescale at the end.
//
// Mapping on gfx950 (wave64):
//  * A workgroup has RW x KW waves (4, or 8 as 4 x 2): RW format row tiles
//    (64 output rows each, one row per lane) times KW waves that share a row
//    tile and take turns over its k-tiles.  It covers the k-tiles of one K-split in stages of CH
//    k-tiles (128 inputs each); the tables of one stage live in LDS.
//  * Each lane streams one slot of the tile, 16 + 4 bytes per k-tile, both
//    loads coalesced across the wave; the next stage's codes are requested
//    before the current stage's lookups.  Two 4 x 4 lane transposes then
//    give each lane its own row's 32 codes (the format stores them in four
//    slots, as the matrix-core kernels consume them).
//  * Table layout: dword [segment][token pair][code], 32 codes per table
//    (128 bytes).  Entry 2p holds the pattern-p dot products of two tokens as
//    two int16 halves; entry 2p+1 holds their negations, so the code's sign
//    bit is applied by the table half it selects.  All lanes of a wave read
//    the same 128-byte table at a time, so a lookup is bank-conflict free.
//    One thread builds the four patterns that share a zero position with
//    packed 16-bit adds: (a+b)+-c and (a-b)+-c.
//  * Lookups accumulate two tokens per v_pk_add_u16 in int16 halves, widened
//    into int32 after every k-tile (32 codes, |sum| <= 32*384 < 2^15).
//  * Waves sharing a row tile add their sums through LDS.  K-splits of one
//    row group then add theirs into a zero-filled 64-bit accumulator per
//    output with one returning atomic, 2^32 + partial: the high word counts
//    arrivals, the low word is the exact int32 sum.  The split that brings
//    the count to `splits` writes the output and stores the zero back, so
//    the reduction costs one memory round trip and no cache maintenance.
//  * Fused form (FQ, sherry_linear with M <= 4): the activations arrive as
//    fp32.  Every workgroup first reads its tokens' whole rows for the
//    per-token scale s = max|x| / 127, and the table builder quantizes the
//    4 inputs of its segment as it reads them, q = clamp(rint(x / s), +-127),
//    with the stand-alone quantizer's arithmetic, so q, the tables and y are
//    bit-identical to quantizing first; the quantizer's launch and the round
//    trip of q through memory are saved.
#include "sherry_device.h"
#include "sherry_launch.h"

namespace sherry {
namespace {

typedef short short2_t __attribute__((ext_vector_type(2)));

// Four fp32 activations quantized with scale s into the 4 int8 lanes of a
// dword (byte j = input j).
__device__ __forceinline__ int quant_word(const float* x, float s) {
  const float4 v = *reinterpret_cast<const float4*>(x);
  const uint32_t b0 = (uint8_t)(int8_t)fminf(fmaxf(rintf(v.x / s), -127.0f), 127.0f);
  const uint32_t b1 = (uint8_t)(int8_t)fminf(fmaxf(rintf(v.y / s), -127.0f), 127.0f);
  const uint32_t b2 = (uint8_t)(int8_t)fminf(fmaxf(rintf(v.z / s), -127.0f), 127.0f);
  const uint32_t b3 = (uint8_t)(int8_t)fminf(fmaxf(rintf(v.w / s), -127.0f), 127.0f);
  return (int)(b0 | (b1 << 8) | (b2 << 16) | (b3 << 24));
}

__device__ __forceinline__ float amax4(const float4 v) {
  return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

__device__ __forceinline__ short2_t pair_of(int x0, int x1, int j) {
  // int8 activation j of two tokens' segment words, widened to int16 halves
  return short2_t{(short)(int8_t)(x0 >> (8 * j)), (short)(int8_t)(x1 >> (8 * j))};
}

template <int MP, int CH, int RW, int KW, bool FQ>
__global__ __launch_bounds__(64 * RW * KW) void lut_gemv_kernel(const uint8_t* packed, const int8_t* x,
                                                                 const float* xf, int M, int N, int K,
                                                                 int splits, int kt_per_split,
                                                                 const float* s_x, const float* alpha,
                                                                 float* y, int32_t* acc_out,
                                                                 int32_t* partials) {
  const GemmArgs a = product_args(packed, x, xf, M, N, K, s_x, alpha, y, acc_out, partials);
  constexpr int NT = 64 * RW * KW;
  constexpr int CPW = (CH + KW - 1) / KW;        // k-tiles per wave per stage
  extern __shared__ uint32_t lut[];               // tables (dynamic LDS)
  __shared__ float fq_red[FQ ? RW * KW * 2 * MP : 1];   // fused form: partial maxima
  __shared__ float fq_s[FQ ? 2 * MP : 1];               //   and the per-token scales

  const int KT = k_tiles(K), RT = row_tiles(N);
  const int g = blockIdx.x / splits;
  const int s = blockIdx.x - g * splits;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = wave % RW, q = wave / RW;
  const int rt = g * RW + r;
  const bool active = rt < RT;
  const int kt_begin = s * kt_per_split;
  const int kt_end = min(KT, kt_begin + kt_per_split);
  const int nst = (kt_end - kt_begin + CH - 1) / CH;

  auto load_stage = [&](int st, uint32_t (&w)[CPW][5]) {
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int c = q + KW * i;
      const int kt = kt_begin + st * CH + c;
      if (active && c < CH && kt < kt_end) {
        const uint8_t* tb = a.packed + tile_offset(rt, kt, KT);
        const uint4 lo = *reinterpret_cast<const uint4*>(tb + 16 * lane);
        w[i][0] = lo.x; w[i][1] = lo.y; w[i][2] = lo.z; w[i][3] = lo.w;
        w[i][4] = *reinterpret_cast<const uint32_t*>(tb + kTileHiOff + 4 * lane);
      } else {
#pragma unroll
        for (int d = 0; d < 5; ++d) w[i][d] = 0;
      }
    }
  };

  uint32_t cur[CPW][5];
  load_stage(0, cur);

  if constexpr (FQ) {
    // per-token scale over the whole row (every workgroup reads its tokens'
    // rows), s = max|x| / 127, an all-zero row -> 1
    const int K4 = K / 4;
#pragma unroll
    for (int m = 0; m < 2 * MP; ++m) {
      float am = 0.0f;
      if (m < M) {
        const float4* xr = reinterpret_cast<const float4*>(a.xf + (size_t)m * K);
#pragma unroll 4
        for (int e = threadIdx.x; e < K4; e += NT) am = fmaxf(am, amax4(xr[e]));
      }
      am = wave_max(am);
      if (lane == 0) fq_red[wave * 2 * MP + m] = am;
    }
    __syncthreads();
    if (threadIdx.x < 2 * MP) {
      float v = 0.0f;
      for (int w = 0; w < RW * KW; ++w) v = fmaxf(v, fq_red[w * 2 * MP + threadIdx.x]);
      fq_s[threadIdx.x] = !(v > 0.0f) ? 1.0f : v / 127.0f;
    }
    __syncthreads();
  }

  // Table-build items per thread and stage: item = (segment, pair, zero
  // position z).  A thread's activation words for a stage's items (two
  // tokens' 4 inputs each) are loaded together, a stage ahead, so the build
  // waits for at most one memory round trip instead of one per item.
  constexpr int kItems = (CH * 32 * MP * 4 + NT - 1) / NT;
  auto load_x = [&](int st, int (&x0)[kItems], int (&x1)[kItems]) {
    const int kt_s = kt_begin + st * CH;
    const int items = min(CH, kt_end - kt_s) * 32 * MP * 4;
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const int it = threadIdx.x + NT * i;
      const int rest = it >> 2;       // segment * MP + pair
      const int pair = rest % MP;
      const int seg = rest / MP;
      const int k = kt_s * kTileK + 4 * seg;
      const int m0 = 2 * pair, m1 = 2 * pair + 1;
      // segments past K (padding of a ragged last k-tile) get zero tables
      x0[i] = 0;
      x1[i] = 0;
      if (it < items) {
        if constexpr (FQ) {
          if (m0 < M && k < K) x0[i] = quant_word(a.xf + (size_t)m0 * K + k, fq_s[m0]);
          if (m1 < M && k < K) x1[i] = quant_word(a.xf + (size_t)m1 * K + k, fq_s[m1]);
        } else {
          if (m0 < M && k < K) x0[i] = *reinterpret_cast<const int*>(a.x + (size_t)m0 * K + k);
          if (m1 < M && k < K) x1[i] = *reinterpret_cast<const int*>(a.x + (size_t)m1 * K + k);
        }
      }
    }
  };
  int xw0[kItems], xw1[kItems];
  load_x(0, xw0, xw1);

  int acc[2 * MP];
#pragma unroll
  for (int m = 0; m < 2 * MP; ++m) acc[m] = 0;

  for (int st = 0; st < nst; ++st) {
    const int kt_s = kt_begin + st * CH;
    const int nch = min(CH, kt_end - kt_s);
    // barriers on LDS only: __syncthreads() would also wait for the loads
    // of the next stage's activations and codes in flight
    if (st > 0) lds_barrier();    // previous stage's lookups are done

    // tables of this stage, from the activation words loaded for it
    {
      const int items = nch * 32 * MP * 4;
#pragma unroll
      for (int i = 0; i < kItems; ++i) {
        const int it = threadIdx.x + NT * i;
        if (it >= items) continue;
        const int z = it & 3;
        const int rest = it >> 2;       // segment * MP + pair
        const int x0 = xw0[i], x1 = xw1[i];
        // the three kept positions in order: ja < jb < jc, none equal to z
        const int ja = z == 0 ? 1 : 0;
        const int jb = z <= 1 ? 2 : 1;
        const int jc = z <= 2 ? 3 : 2;
        const short2_t ya = pair_of(x0, x1, ja), yb = pair_of(x0, x1, jb),
                       yc = pair_of(x0, x1, jc);
        const short2_t t = ya + yb, u = ya - yb;
        const short2_t zero{0, 0};
        // pattern 4z + 2*r1 + r2 -> codes 2p (positive) and 2p+1 (negated)
        const short2_t p0 = t + yc, p1 = t - yc, p2 = u + yc, p3 = u - yc;
        uint4* dst = reinterpret_cast<uint4*>(&lut[rest * 32 + 8 * z]);
        dst[0] = make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, zero - p0),
                            __builtin_bit_cast(uint32_t, p1), __builtin_bit_cast(uint32_t, zero - p1));
        dst[1] = make_uint4(__builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, zero - p2),
                            __builtin_bit_cast(uint32_t, p3), __builtin_bit_cast(uint32_t, zero - p3));
      }
    }
    if (st + 1 < nst) load_x(st + 1, xw0, xw1);
    lds_barrier();

    uint32_t nxt[CPW][5];
    if (st + 1 < nst) load_stage(st + 1, nxt);

    if (active) {
#pragma unroll
      for (int i = 0; i < CPW; ++i) {
        const int c = q + KW * i;
        if (c < nch) {
          short2_t h[MP];
#pragma unroll
          for (int pp = 0; pp < MP; ++pp) h[pp] = short2_t{0, 0};
          const uint32_t* lc = lut + c * (32 * MP * 32);
          uint32_t glo[4], ghb;   // this lane's row: its four code groups
          row_groups(cur[i], lane, glo, ghb);
#pragma unroll
          for (int j = 0; j < 32; ++j) {
            const uint32_t code = group_code(glo[j >> 3], ghb >> (8 * (j >> 3)), j & 7);
#pragma unroll
            for (int pp = 0; pp < MP; ++pp)
              h[pp] += __builtin_bit_cast(short2_t, lc[(j * MP + pp) * 32 + code]);
          }
#pragma unroll
          for (int pp = 0; pp < MP; ++pp) {
            acc[2 * pp] += (int)h[pp].x;
            acc[2 * pp + 1] += (int)h[pp].y;
          }
        }
      }
    }
    if (st + 1 < nst) {
#pragma unroll
      for (int i = 0; i < CPW; ++i)
#pragma unroll
        for (int d = 0; d < 5; ++d) cur[i][d] = nxt[i][d];
    }
  }

  // waves that share a row tile: add through LDS into the q == 0 wave
  if constexpr (KW > 1) {
    __syncthreads();  // tables no longer needed
    int* red = reinterpret_cast<int*>(lut);   // [KW-1][2MP][RW*64]
    if (q > 0) {
#pragma unroll
      for (int m = 0; m < 2 * MP; ++m)
        red[((q - 1) * 2 * MP + m) * (RW * 64) + r * 64 + lane] = acc[m];
    }
    __syncthreads();
    if (q > 0) return;
#pragma unroll
    for (int qq = 1; qq < KW; ++qq)
#pragma unroll
      for (int m = 0; m < 2 * MP; ++m)
        acc[m] += red[((qq - 1) * 2 * MP + m) * (RW * 64) + r * 64 + lane];
  }

  if (!active) return;
  const int n = rt * kTileRows + lane;
  if (n >= N) return;                           // rows past N: padding, never stored
  const float al = a.y ? a.alpha[n] : 0.0f;
  // The tokens' scales are loaded here, with alpha, before any atomic or
  // store: the memory counter counts stores too, so a scale loaded after
  // one token's store would make the next store wait for it, and the lane's
  // M stores would leave one round trip apart.
  float sxm[2 * MP];
#pragma unroll
  for (int m = 0; m < 2 * MP; ++m) sxm[m] = !FQ && a.y && m < M ? a.s_x[m] : 0.0f;
  // every token's atomic is issued before any result is used: one memory
  // round trip per lane whatever M is
  int total[2 * MP];
  bool last[2 * MP];
#pragma unroll
  for (int m = 0; m < 2 * MP; ++m) {
    total[m] = acc[m];
    last[m] = true;
  }
  if (splits > 1) {
    unsigned long long now[2 * MP];
#pragma unroll
    for (int m = 0; m < 2 * MP; ++m) {
      now[m] = 0;
      if (m < M) {
        unsigned long long* cell = reinterpret_cast<unsigned long long*>(a.partials) + (size_t)m * N + n;
        const unsigned long long inc = (1ull << 32) + (unsigned long long)(long long)acc[m];
        now[m] = __hip_atomic_fetch_add(cell, inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    // (no result is touched before the last atomic is issued)
#pragma unroll
    for (int m = 0; m < 2 * MP; ++m) {
      now[m] += (1ull << 32) + (unsigned long long)(long long)acc[m];
      total[m] = (int)(uint32_t)now[m];
      const long long count = ((long long)now[m] - (long long)total[m]) >> 32;
      last[m] = count == splits;
      if (m < M && last[m])
        __hip_atomic_store(reinterpret_cast<unsigned long long*>(a.partials) + (size_t)m * N + n, 0ull,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // every output is formed before the first store (the empty asm keeps
  // each product out of the store branches), so the one wait for alpha
  // comes before any store rather than between them
  float yv[2 * MP];
#pragma unroll
  for (int m = 0; m < 2 * MP; ++m) {
    yv[m] = ((float)total[m] * (FQ ? fq_s[m] : sxm[m])) * al;
    asm volatile("" : "+v"(yv[m]));
  }
#pragma unroll
  for (int m = 0; m < 2 * MP; ++m) {
    if (m >= M || !last[m]) continue;
    if (a.y) {
      a.y[(size_t)m * N + n] = yv[m];
    } else {
      a.acc[(size_t)m * N + n] = total[m];
    }
  }
}

template <int MP, int CH, int RW, int KW, bool FQ>
hipError_t launch_cfg(const GemmPlan& p, const GemmArgs& a, hipStream_t stream) {
  // the tables of a stage can take all of the first 64 KB of LDS, which
  // with the kernel's static arrays needs the larger dynamic limit
  if (p.lds_bytes + 1024 > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(lut_gemv_kernel<MP, CH, RW, KW, FQ>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, p.lds_bytes + 1024);
    if (e != hipSuccess) return e;
  }
  launch_product_kernel(lut_gemv_kernel<MP, CH, RW, KW, FQ>, dim3(p.grid), dim3(64 * RW * KW), p.lds_bytes,
                     stream, a, p.splits, p.kt_per_split);
  return hipGetLastError();
}

template <int MP, int CH, bool FQ>
hipError_t launch_ch(const GemmPlan& p, const GemmArgs& a, hipStream_t stream) {
  switch (p.rw) {
    case 4: return launch_cfg<MP, CH, 4, 1, FQ>(p, a, stream);
    case 2: return launch_cfg<MP, CH, 2, 2, FQ>(p, a, stream);
    case 1: return launch_cfg<MP, CH, 1, 4, FQ>(p, a, stream);
    // 8 waves: 4 row tiles x 2 waves that take turns over a stage's k-tiles
    case 8: if constexpr (CH >= 2) return launch_cfg<MP, CH, 4, 2, FQ>(p, a, stream); break;
    default: return hipErrorInvalidValue;
  }
}

template <int MP, bool FQ>
hipError_t launch_mp(const GemmPlan& p, const GemmArgs& a, hipStream_t stream) {
  switch (p.ch) {
    case 1: return launch_ch<MP, 1, FQ>(p, a, stream);
    case 2: return launch_ch<MP, 2, FQ>(p, a, stream);
    case 4: if constexpr (MP <= 4) return launch_ch<MP, 4, FQ>(p, a, stream); break;
    case 8: if constexpr (MP <= 2) return launch_ch<MP, 8, FQ>(p, a, stream); break;
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace

// The fused form takes up to kFuseMaxM tokens whose rows (M*K fp32) every
// workgroup reads once.
bool lut_gemv_fusable(const GemmPlan& p, int M, int K) {
  return p.path == 0 && M <= kFuseMaxM && (long long)M * K <= kFuseMaxMK;
}

hipError_t launch_lut_gemv(const GemmPlan& p, const GemmArgs& a, hipStream_t stream) {
  if (a.xf) {
    switch ((a.M + 1) / 2) {
      case 1: return launch_mp<1, true>(p, a, stream);
      case 2: return launch_mp<2, true>(p, a, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch ((a.M + 1) / 2) {
    case 1: return launch_mp<1, false>(p, a, stream);
    case 2: return launch_mp<2, false>(p, a, stream);
    case 3: return launch_mp<3, false>(p, a, stream);
    case 4: return launch_mp<4, false>(p, a, stream);
    case 5: return launch_mp<5, false>(p, a, stream);
    case 6: return launch_mp<6, false>(p, a, stream);
    case 7: return launch_mp<7, false>(p, a, stream);
    case 8: return launch_mp<8, false>(p, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sherry
