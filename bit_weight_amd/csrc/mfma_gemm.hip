// Kernel 4: large-M (prefill) product.  The 5-bit codes are decoded to int8
// {-1,0,+1} tiles in LDS and contracted with int8 activations on the gfx950
// matrix cores (v_mfma_i32_32x32x32_i8), int32 accumulation, then the same
// float rescale as the lookup path: y = ((float)acc * s_x[m]) * alpha[n].
// Decoding ahead of an int8 contraction follows the fused decode-then-int8-GEMM
// structure the OdysseyLLM FastGEMM review describes for W4A8 (xllm-io page,
// FastGEMM section); here the decode is a 32-entry table of int8x4 words.
//
// Workgroup tile BM x BN over a k-step of one format k-tile (128 inputs);
// 4 waves in a 2 x 2 grid, each owning (BM/2) x (BN/2) outputs as 32x32
// MFMA blocks.  LDS rows are padded by 16 bytes so that 8 consecutive lanes
// reading 16 bytes each from consecutive rows touch all 32 banks once.
#include "sherry_device.h"
#include "sherry_launch.h"

namespace sherry {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kBK = 128;
constexpr int kLd = kBK + 16;

template <int BM, int BN>
__global__ __launch_bounds__(256) void mfma_gemm_kernel(GemmArgs a) {
  constexpr int TM = BM / 2 / 32, TN = BN / 2 / 32;  // MFMA blocks per wave
  __shared__ __attribute__((aligned(16))) int8_t As[BM * kLd];
  __shared__ __attribute__((aligned(16))) int8_t Bs[BN * kLd];
  __shared__ uint32_t dec[32];

  const int M = a.M, N = a.N, K = a.K, KT = K / kTileK;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;

  if (tid < 32) dec[tid] = code_word(tid);

  v16i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v16i{};

  // B decode assignment: BN rows x 2 halves of 16 codes; half is wave-uniform
  constexpr int BROWS_PER_PASS = 256 / 2;
  static_assert(BN % BROWS_PER_PASS == 0 || BN == 64, "BN");

  for (int kt = 0; kt < KT; ++kt) {
    // activations: BM rows x 128 bytes, 16 bytes per load
    constexpr int AV = BM * 8 / 256;
    uint4 areg[AV];
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const int idx = tid + 256 * i, row = idx >> 3, c16 = idx & 7;
      const int m = m0 + row;
      areg[i] = m < M ? *reinterpret_cast<const uint4*>(a.x + (size_t)m * K + (size_t)kt * kBK + c16 * 16)
                      : make_uint4(0, 0, 0, 0);
    }
    // codes: 16 codes (half a row's k-tile) per thread and pass
    constexpr int BP = (BN * 2 + 255) / 256;
    uint32_t w[BP][5];
#pragma unroll
    for (int pz = 0; pz < BP; ++pz) {
      const int slot = tid + 256 * pz;
      const int row = slot % BN;
      const int n = n0 + row;
      if (slot < BN * 2 && n < N) {
        const uint8_t* tb = a.packed + tile_offset(n / kTileRows, kt, KT);
        const int r = n % kTileRows;
        const uint4 lo = *reinterpret_cast<const uint4*>(tb + 16 * r);
        w[pz][0] = lo.x; w[pz][1] = lo.y; w[pz][2] = lo.z; w[pz][3] = lo.w;
        w[pz][4] = *reinterpret_cast<const uint32_t*>(tb + kTileHiOff + 4 * r);
      } else {
#pragma unroll
        for (int d = 0; d < 5; ++d) w[pz][d] = 0;
      }
    }
    __syncthreads();  // previous k-step's fragment reads are done
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const int idx = tid + 256 * i, row = idx >> 3, c16 = idx & 7;
      *reinterpret_cast<uint4*>(&As[row * kLd + c16 * 16]) = areg[i];
    }
#pragma unroll
    for (int pz = 0; pz < BP; ++pz) {
      const int slot = tid + 256 * pz;
      if (slot < BN * 2) {
        const int row = slot % BN, half = slot / BN;
        const int n = n0 + row;
        uint32_t o[16];
        if (half == 0) {
#pragma unroll
          for (int j = 0; j < 16; ++j) o[j] = n < N ? dec[code_at(w[pz], j)] : 0u;
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) o[j] = n < N ? dec[code_at(w[pz], 16 + j)] : 0u;
        }
        int8_t* dst = &Bs[row * kLd + half * 64];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<uint4*>(dst + 16 * q) =
              make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kBK / 32; ++kk) {
      v4i af[TM], bf[TN];
      const int kb = kk * 32 + (lane >> 5) * 16;
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const v4i*>(&As[(wm * (BM / 2) + i * 32 + (lane & 31)) * kLd + kb]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bf[j] = *reinterpret_cast<const v4i*>(&Bs[(wn * (BN / 2) + j * 32 + (lane & 31)) * kLd + kb]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  }

  // epilogue: lane holds column (lane % 32) and 16 rows of each 32x32 block
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = n0 + wn * (BN / 2) + j * 32 + (lane & 31);
      if (n >= N) continue;
      const float al = a.y ? a.alpha[n] : 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * (BM / 2) + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m >= M) continue;
        if (a.y) {
          const float t = (float)acc[i][j][r] * a.s_x[m];
          a.y[(size_t)m * N + n] = t * al;
        } else {
          a.acc[(size_t)m * N + n] = acc[i][j][r];
        }
      }
    }
}

}  // namespace

hipError_t launch_mfma_gemm(const GemmPlan& p, const GemmArgs& a, hipStream_t stream) {
  constexpr int BM = 128, BN = 128;
  dim3 grid((a.N + BN - 1) / BN, (a.M + BM - 1) / BM);
  hipLaunchKernelGGL((mfma_gemm_kernel<BM, BN>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sherry
