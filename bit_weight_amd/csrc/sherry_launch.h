// Internal launch interface between the C ABI (sherry_abi.hip) and the
// kernel translation units.  Shapes are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sherry {

// Launch plan of the product for one shape (host-side, pure).
struct GemmPlan {
  int path;          // 0 = lookup-table GEMV, 1 = decode + int8 MFMA GEMM,
                     // 2 = decode + int8 MFMA GEMV (M <= 64)
  int grid;          // workgroups
  int block;         // threads per workgroup
  int splits;        // K-splits per row group (GEMV)
  int kt_per_split;  // format k-tiles per K-split (GEMV)
  int rw;            // LUT GEMV: row tiles per workgroup; matrix-core GEMV: waves per
                     // row tile; prefill GEMM: tile height in units of 64 activation rows
  int ch;            // LUT GEMV: k-tiles per LDS table stage; prefill GEMM: k-phases (2 or 4)
  int groups;        // output row groups (GEMV)
  int lds_bytes;     // dynamic LDS per workgroup
  size_t ws_bytes;   // workspace bytes required
  int chunk;         // tokens per launch (0 = all M in one launch)
};

constexpr int kLutMaxM = 16;          // M <= 16 takes a GEMV path
constexpr int kGemvMaxM = 64;         // 16 < M <= 64: the matrix-core GEMV, unless path 1 is forced
constexpr int kChunkMaxM = 128;       // 64 < M <= 128: the prefill GEMM, or the GEMV in
constexpr int kChunkMaxGrid = 64;     //   launches of 64 tokens where the prefill grid is at
                                      //   most 64 workgroups (chunk_max_m)
constexpr int kGemvWaves = 4;         // waves per GEMV workgroup
constexpr int kCUs = 256;             // MI355X compute units: one round of one workgroup each
constexpr int kDefaultSmallMPath = 2;  // M <= 16: 0 = lookup tables, 2 = matrix-core GEMV
constexpr int kFuseMaxM = 4;           // fused quantization: at most 4 tokens,
constexpr int kFuseMaxMK = 16384;      //   M*K elements read per workgroup for the scales,
constexpr int kFuseMaxSpan = 32;       //   and k-tiles per K-split held in LDS as int8

// Tuning override of the GEMV plan (path -1 / others 0 = built-in choice),
// see sherry.h.
void set_plan_override(int path, int rw, int ch, int splits);

GemmPlan plan_gemm(int M, int N, int K);

struct GemmArgs {
  const int8_t* x;     // int8 activations [M,K], or
  const float* xf;     // fp32 activations quantized in the kernel (fused form; x unused)
  const float* s_x;
  const uint8_t* packed;
  const float* alpha;
  float* y;            // fp32 output, or
  int32_t* acc;        // int32 output (exactly one of y / acc is non-null)
  int M, N, K;
  int32_t* partials;   // workspace: zero-filled 64-bit accumulators [M,N] for K-splits
};

// The product kernels take their arguments as pointers and scalars, not as
// a GemmArgs struct, with the ones their first instructions need in front:
// packed, x, xf, M, N, K, two plan integers (the GEMVs: splits and k-tiles
// per split; the prefill GEMM: n tiles and 0), then s_x, alpha, y, acc,
// partials.  The build has the leading ones preloaded into SGPRs at
// dispatch (gfx950 kernel-argument preload), which removes a memory round
// trip from the start of every launch; a struct argument cannot be
// preloaded.
template <typename Kernel>
inline void launch_product_kernel(Kernel kernel, dim3 grid, dim3 block, size_t lds_bytes,
                                  hipStream_t stream, const GemmArgs& a, int plan0, int plan1) {
  hipLaunchKernelGGL(kernel, grid, block, lds_bytes, stream, a.packed, a.x, a.xf, a.M, a.N, a.K, plan0,
                     plan1, a.s_x, a.alpha, a.y, a.acc, a.partials);
}

// The GemmArgs a product kernel rebuilds from its arguments.
__device__ __forceinline__ GemmArgs product_args(const uint8_t* packed, const int8_t* x, const float* xf,
                                                 int M, int N, int K, const float* s_x, const float* alpha,
                                                 float* y, int32_t* acc, int32_t* partials) {
  GemmArgs a{};
  a.packed = packed;
  a.x = x;
  a.xf = xf;
  a.M = M;
  a.N = N;
  a.K = K;
  a.s_x = s_x;
  a.alpha = alpha;
  a.y = y;
  a.acc = acc;
  a.partials = partials;
  return a;
}

hipError_t launch_quantize_pack(const float* W, int N, int K, uint8_t* packed, float* alpha,
                                hipStream_t stream);
hipError_t launch_quantize_pack2(const float* W, int N, int K, uint8_t* packed, float* alpha,
                                 hipStream_t stream);
hipError_t launch_quantize_act(const float* x, int M, int K, int8_t* q, float* s_x,
                               hipStream_t stream);
hipError_t launch_lut_gemv(const GemmPlan& plan, const GemmArgs& args, hipStream_t stream);
hipError_t launch_mfma_gemv(const GemmPlan& plan, const GemmArgs& args, hipStream_t stream);
bool mfma_gemv_fusable(const GemmPlan& plan, int M, int K);
bool lut_gemv_fusable(const GemmPlan& plan, int M, int K);
// The same GEMV on the 2-bit baseline format (packed = kTile2Bytes tiles).
hipError_t launch_mfma_gemv2(const GemmPlan& plan, const GemmArgs& args, hipStream_t stream);
// The prefill GEMM's grid and LDS for tiles of bm (64 or 128) activation rows.
int mfma_gemm_grid(int M, int N, int bm, int kp);
int mfma_gemm_lds_bytes(int bm, int kp);
int mfma_gemm_threads();
hipError_t launch_mfma_gemm(const GemmPlan& plan, const GemmArgs& args, hipStream_t stream);
// The product (x int8) on the plan's path, in launches of plan.chunk tokens
// when the plan asks for it.  On a failed launch, *partial (if given) tells
// whether earlier launches of the same call were already enqueued.
hipError_t launch_product(const GemmPlan& plan, const GemmArgs& args, hipStream_t stream,
                          bool* partial = nullptr);

}  // namespace sherry
