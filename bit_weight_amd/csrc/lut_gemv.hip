// Kernels 2 + 3: per-segment lookup tables in LDS and the small-M LUT-GEMV.
//
// [Sherry page §2.2] the activations are cut into 4-element segments; for
// every segment a table of the 16 canonical pattern dot products is built;
// each weight block is then one table lookup, its sign is applied and the
// results are summed in integers, with one float rescale at the end.
//
// Mapping on gfx950 (wave64):
//  * A workgroup owns 4 format row tiles (256 output rows, one row per lane)
//    and a contiguous range of `cpl` format k-tiles (128 inputs each).
//  * Each lane first issues its code loads (16 + 4 bytes per k-tile, both
//    coalesced across the wave), then the workgroup builds the tables for
//    its k-range while those loads are in flight.
//  * Table layout: dword [segment][token pair][code], 32 codes per table
//    (128 bytes).  Entry 2p holds the pattern-p dot products of two tokens as
//    two int16 halves; entry 2p+1 holds their negations, so the code's sign
//    bit is applied by the table half it selects.  All lanes of a wave read
//    the same 128-byte table at a time, so the read is bank-conflict free.
//  * Lookups accumulate two tokens per v_pk_add_u16 in int16 halves, which
//    are widened into int32 after every k-tile (32 codes, |sum| <= 32*384).
//  * K-splits of one row group publish int32 partial sums; the last
//    workgroup to arrive (an agent-scope counter) adds them in split order
//    and writes the output, then resets the counter for the next call.
#include "sherry_device.h"
#include "sherry_launch.h"

namespace sherry {
namespace {

typedef short short2_t __attribute__((ext_vector_type(2)));

template <int MP, int CPL>
__global__ __launch_bounds__(kGemvRows) void lut_gemv_kernel(GemmArgs a, int splits) {
  // [32*CPL segments][MP pairs][32 codes], then one flag dword.  Nothing
  // else lives in LDS, so the tables start at address 0 and every lookup's
  // segment offset folds into the ds_read immediate.
  extern __shared__ uint32_t lut[];
  constexpr int kLutDwords = 32 * CPL * MP * 32;
  int& is_last = *reinterpret_cast<int*>(&lut[kLutDwords]);

  const int M = a.M, N = a.N, K = a.K;
  const int KT = K / kTileK;
  const int g = blockIdx.x / splits;
  const int s = blockIdx.x - g * splits;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rt = g * kGemvWaves + wave;
  const bool active = rt < N / kTileRows;
  const int kt0 = s * CPL;
  const int nch = min(CPL, KT - kt0);

  // 1. stream this lane's codes (issued first; consumed after the table build)
  uint32_t w[CPL][5];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    if (active && c < nch) {
      const uint8_t* tb = a.packed + tile_offset(rt, kt0 + c, KT);
      const uint4 lo = *reinterpret_cast<const uint4*>(tb + 16 * lane);
      w[c][0] = lo.x; w[c][1] = lo.y; w[c][2] = lo.z; w[c][3] = lo.w;
      w[c][4] = *reinterpret_cast<const uint32_t*>(tb + kTileHiOff + 4 * lane);
    } else {
#pragma unroll
      for (int d = 0; d < 5; ++d) w[c][d] = 0;
    }
  }

  // 2. tables: item = (segment, pair, pattern p), p fastest
  {
    const int p = threadIdx.x & 15;
    const uint32_t pw = code_word(2 * p);
    const int items = 32 * nch * MP * 16;
    const int kbase = kt0 * kTileK;
    for (int it = threadIdx.x; it < items; it += kGemvRows) {
      const int rest = it >> 4;  // segment * MP + pair
      const int pair = rest % MP;
      const int seg = rest / MP;
      const int k = kbase + 4 * seg;
      const int m0 = 2 * pair, m1 = 2 * pair + 1;
      const int x0 = m0 < M ? *reinterpret_cast<const int*>(a.x + (size_t)m0 * K + k) : 0;
      const int x1 = m1 < M ? *reinterpret_cast<const int*>(a.x + (size_t)m1 * K + k) : 0;
      const int L0 = __builtin_amdgcn_sdot4((int)pw, x0, 0, false);
      const int L1 = __builtin_amdgcn_sdot4((int)pw, x1, 0, false);
      const uint32_t pos = ((uint32_t)L0 & 0xFFFFu) | ((uint32_t)L1 << 16);
      const uint32_t neg = ((uint32_t)(-L0) & 0xFFFFu) | ((uint32_t)(-L1) << 16);
      *reinterpret_cast<uint2*>(&lut[rest * 32 + 2 * p]) = make_uint2(pos, neg);
    }
  }
  __syncthreads();

  // 3. lookups
  int acc[2 * MP];
#pragma unroll
  for (int m = 0; m < 2 * MP; ++m) acc[m] = 0;
  if (active) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      if (c < nch) {
        short2_t h[MP];
#pragma unroll
        for (int i = 0; i < MP; ++i) h[i] = short2_t{0, 0};
        const uint32_t* lc = lut + c * 32 * MP * 32;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          const uint32_t code = code_at(w[c], j);
#pragma unroll
          for (int i = 0; i < MP; ++i) {
            const uint32_t v = lc[(j * MP + i) * 32 + code];
            h[i] += __builtin_bit_cast(short2_t, v);
          }
        }
#pragma unroll
        for (int i = 0; i < MP; ++i) {
          acc[2 * i] += (int)h[i].x;
          acc[2 * i + 1] += (int)h[i].y;
        }
      }
    }
  }

  const int n = rt * kTileRows + lane;
  if (splits > 1) {
    // 4. publish this split's partial sums; the last arrival reduces
    int32_t* part = a.partials + ((size_t)g * splits + s) * (size_t)M * kGemvRows;
    if (active) {
#pragma unroll
      for (int m = 0; m < 2 * MP; ++m)
        if (m < M) part[(size_t)m * kGemvRows + threadIdx.x] = acc[m];
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t old = __hip_atomic_fetch_add(&a.counters[g], 1u, __ATOMIC_ACQ_REL,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      is_last = (old == (uint32_t)(splits - 1));
    }
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    if (active) {
      const int32_t* base = a.partials + (size_t)g * splits * (size_t)M * kGemvRows;
#pragma unroll
      for (int m = 0; m < 2 * MP; ++m) {
        if (m < M) {
          int t = 0;
          for (int s2 = 0; s2 < splits; ++s2)
            t += base[((size_t)s2 * M + m) * kGemvRows + threadIdx.x];
          acc[m] = t;
        }
      }
    }
    if (threadIdx.x == 0)
      __hip_atomic_store(&a.counters[g], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // 5. epilogue: y = ((float)acc * s_x[m]) * alpha[n]
  if (!active) return;
  if (a.y) {
    const float al = a.alpha[n];
#pragma unroll
    for (int m = 0; m < 2 * MP; ++m)
      if (m < M) {
        const float t = (float)acc[m] * a.s_x[m];
        a.y[(size_t)m * N + n] = t * al;
      }
  } else {
#pragma unroll
    for (int m = 0; m < 2 * MP; ++m)
      if (m < M) a.acc[(size_t)m * N + n] = acc[m];
  }
}

template <int MP, int CPL>
hipError_t launch_mp_cpl(const GemmPlan& p, const GemmArgs& a, hipStream_t stream) {
  const size_t lds = ((size_t)32 * CPL * MP * 32 + 4) * sizeof(uint32_t);
  hipLaunchKernelGGL((lut_gemv_kernel<MP, CPL>), dim3(p.grid), dim3(kGemvRows), lds, stream, a,
                     p.splits);
  return hipGetLastError();
}

template <int MP>
hipError_t launch_mp(const GemmPlan& p, const GemmArgs& a, hipStream_t stream) {
  switch (p.cpl) {
    case 1: return launch_mp_cpl<MP, 1>(p, a, stream);
    case 2: return launch_mp_cpl<MP, 2>(p, a, stream);
    case 4: if constexpr (MP <= 2) return launch_mp_cpl<MP, 4>(p, a, stream); break;
    case 8: if constexpr (MP <= 1) return launch_mp_cpl<MP, 8>(p, a, stream); break;
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_lut_gemv(const GemmPlan& p, const GemmArgs& a, hipStream_t stream) {
  switch ((a.M + 1) / 2) {
    case 1: return launch_mp<1>(p, a, stream);
    case 2: return launch_mp<2>(p, a, stream);
    case 3: return launch_mp<3>(p, a, stream);
    case 4: return launch_mp<4>(p, a, stream);
    case 5: return launch_mp<5>(p, a, stream);
    case 6: return launch_mp<6>(p, a, stream);
    case 7: return launch_mp<7>(p, a, stream);
    case 8: return launch_mp<8>(p, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sherry
