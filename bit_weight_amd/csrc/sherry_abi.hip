// C ABI of libsherry: host-side validation, launch planning and dispatch.
// Every argument error is detected here before any HIP call.
#include <atomic>
#include <mutex>
#include <string.h>

#include "../../include/sherry.h"
#include "sherry_device.h"
#include "sherry_launch.h"

namespace sherry {

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 20;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Per-device check that the current device is a gfx950, cached.
constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
int g_dev_ok[kMaxDevices];

sherry_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return SHERRY_ERR_HIP;
  if (dev >= kMaxDevices) return SHERRY_ERR_DEVICE;
  std::call_once(g_dev_once[dev], [dev] {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      g_dev_ok[dev] = -1;
      return;
    }
    g_dev_ok[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
  });
  if (g_dev_ok[dev] < 0) return SHERRY_ERR_HIP;
  return g_dev_ok[dev] == 1 ? SHERRY_OK : SHERRY_ERR_DEVICE;
}

// K % 16: whole 4-weight blocks, and int8 activation rows 16-byte aligned
// for the kernels' 16-byte loads; N % 4: the prefill epilogue's 16-byte
// stores stay inside a row.  Other multiples of the 64 x 128 tiles are
// padding of the packed format.
bool shape_ok(int64_t M, int64_t N, int64_t K) {
  return M >= 1 && N >= 1 && K >= 1 && M <= kMaxDim && N <= kMaxDim && K <= kMaxDim &&
         K % 16 == 0 && N % 4 == 0;
}

}  // namespace

namespace {
std::atomic<int> g_ovr_path{-1}, g_ovr_rw{0}, g_ovr_ch{0}, g_ovr_splits{0};

// Small-M path: decode + int8 MFMA GEMV.  One row tile per workgroup and
// KW waves taking turns over its k-tiles.  With >= 128 row tiles, 8 waves
// per row tile and no K-split already keep >= 1024 waves streaming; smaller
// N uses 4 waves per row tile and splits K until there are >= 1024 waves and
// each wave has at most ~3 k-tiles (measured on MI355X at the LLaMA shapes).
GemmPlan mfma_gemv_plan_of(int M, int N, int K, int kw, int splits);

GemmPlan plan_mfma_gemv(int M, int N, int K) {
  const int KT = k_tiles(K), RT = row_tiles(N);
  const int ovr_kw = g_ovr_rw.load();
  int kw = ovr_kw == 4 || ovr_kw == 8 || ovr_kw == 16 ? ovr_kw : (RT >= 128 ? 8 : 4);
  if (M > 16 && kw > 8) kw = 8;   // several token blocks: at most 8 waves
  int splits = 1;
  if (g_ovr_splits.load() > 0) {
    splits = g_ovr_splits.load();
  } else if (RT < 128) {
    const int by_waves = (1024 + RT * kw - 1) / (RT * kw);
    const int by_depth = (KT + 3 * kw - 1) / (3 * kw);
    splits = by_waves > by_depth ? by_waves : by_depth;
    const int max_splits = KT / kw > 0 ? KT / kw : 1;   // >= one k-tile per wave
    if (splits > max_splits) splits = max_splits;
  }
  return mfma_gemv_plan_of(M, N, K, kw, splits);
}

// The matrix-core GEMV's plan for kw waves per row tile and (at most)
// `splits` K-splits.
GemmPlan mfma_gemv_plan_of(int M, int N, int K, int kw, int splits) {
  GemmPlan p{};
  const int KT = k_tiles(K), RT = row_tiles(N);
  if (splits > KT) splits = KT;
  if (splits < 1) splits = 1;
  const int kt_per_split = (KT + splits - 1) / splits;
  splits = (KT + kt_per_split - 1) / kt_per_split;
  int mt = 1;
  while (mt < M && mt < 16) mt *= 2;
  p.path = 2;
  p.groups = RT;
  p.rw = kw;            // waves per row tile on this path
  p.ch = 1;
  p.splits = splits;
  p.kt_per_split = kt_per_split;
  p.grid = RT * splits;
  p.block = 64 * kw;
  p.lds_bytes = 1024 * 8 + kw * mt * (kTileRows + 4) * 4;   // static: pair table + reduction
  p.ws_bytes = splits > 1 ? (size_t)M * N * sizeof(unsigned long long) : 0;
  return p;
}
}  // namespace

void set_plan_override(int path, int rw, int ch, int splits) {
  g_ovr_path = path;
  g_ovr_rw = rw;
  g_ovr_ch = ch;
  g_ovr_splits = splits;
}

hipError_t launch_product(const GemmPlan& plan, const GemmArgs& args, hipStream_t stream) {
  auto one = [&](const GemmArgs& a) {
    return plan.path == 0   ? launch_lut_gemv(plan, a, stream)
           : plan.path == 2 ? launch_mfma_gemv(plan, a, stream)
                            : launch_mfma_gemm(plan, a, stream);
  };
  if (plan.chunk <= 0 || args.M <= plan.chunk) return one(args);
  // launches of plan.chunk tokens in stream order; each leaves the split-K
  // workspace zero for the next
  for (int m0 = 0; m0 < args.M; m0 += plan.chunk) {
    GemmArgs c = args;
    c.M = args.M - m0 < plan.chunk ? args.M - m0 : plan.chunk;
    c.x = args.x + (size_t)m0 * args.K;
    if (args.s_x) c.s_x = args.s_x + m0;
    if (args.y) c.y = args.y + (size_t)m0 * args.N;
    if (args.acc) c.acc = args.acc + (size_t)m0 * args.N;
    const hipError_t e = one(c);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

namespace {
// Prefill GEMM: one workgroup per 128 x 256 output tile, no K-split.
// Tiles of 64 activation rows when that grid fits the GPU in one round
// (<= 256 workgroups), else 128: per workgroup the 128-row tile costs half
// the decode per multiply-add, but below ~256 tokens it leaves CUs idle
// (M=129..256 at N=14336: 112 tiles of 128 rows).  A forced prefill path
// with rw = 1 or 2 in the override picks the height.
GemmPlan plan_prefill(int M, int N, int K) {
  GemmPlan p{};
  const long long nt = (N + 255) / 256;
  int bm = ((M + 63) / 64) * nt <= 256 ? 64 : 128;
  const int ovr_rw = g_ovr_rw.load();
  if (g_ovr_path.load() == 1 && (ovr_rw == 1 || ovr_rw == 2)) bm = 64 * ovr_rw;
  p.path = 1;
  p.rw = bm / 64;
  p.grid = mfma_gemm_grid(M, N, bm);
  p.block = mfma_gemm_threads();
  p.splits = 1;
  p.kt_per_split = k_tiles(K);
  p.lds_bytes = mfma_gemm_lds_bytes(bm);
  p.ws_bytes = 0;
  return p;
}
}  // namespace

// M <= 16: the built-in small-M path (or the override's); 16 < M <= 64: the
// matrix-core GEMV unless the prefill kernel is forced; 64 < M <= 128: the
// same GEMV in launches of 64 tokens (each streams the weights again), except
// above 96 tokens when the prefill's 64-row tiles number >= 96, i.e. for
// wide N (measured at N=14336, K=4096: two GEMV launches take 19.7 us at
// M=96 and 22.2-22.9 us at M=104-128, the 112 prefill tiles 21.2 us; at
// N=4096 the prefill would have 32 tiles); M > 128: prefill.
GemmPlan plan_gemm(int M, int N, int K) {
  GemmPlan p{};
  const int ovr = g_ovr_path.load();
  if (M > kChunkMaxM || (M > kLutMaxM && ovr == 1)) return plan_prefill(M, N, K);
  if (M > kGemvMaxM) {
    const long long prefill_tiles = (long long)((M + 63) / 64) * ((N + 255) / 256);
    if (ovr < 0 && M > kChunkPrefillM && prefill_tiles >= kPrefillMinTiles) return plan_prefill(M, N, K);
    GemmPlan c = plan_mfma_gemv(kGemvMaxM, N, K);
    c.chunk = kGemvMaxM;
    return c;
  }
  if (M > kLutMaxM) return plan_mfma_gemv(M, N, K);
  const int path = ovr >= 0 ? ovr : kDefaultSmallMPath;
  if (path == 1) return plan_prefill(M, N, K);
  if (path == 2) return plan_mfma_gemv(M, N, K);
  const int MP = (M + 1) / 2;
  const int KT = k_tiles(K);
  const int RT = row_tiles(N);
  int ch_max = 1;                       // one stage of tables stays <= 32 KB
  while (ch_max < 8 && (ch_max * 2) * MP <= 8) ch_max *= 2;

  int rw = g_ovr_rw.load() > 0 ? g_ovr_rw.load() : 4;
  if (rw != 1 && rw != 2 && rw != 4) rw = 4;
  const int G = (RT + rw - 1) / rw;
  constexpr int kTargetWorkgroups = 512;
  int splits = g_ovr_splits.load() > 0 ? g_ovr_splits.load() : (kTargetWorkgroups + G - 1) / G;
  if (splits > KT) splits = KT;
  if (splits < 1) splits = 1;
  const int kt_per_split = (KT + splits - 1) / splits;
  splits = (KT + kt_per_split - 1) / kt_per_split;
  int ch = 1;
  const int ch_cap = g_ovr_ch.load() > 0 ? g_ovr_ch.load() : ch_max;
  while (ch * 2 <= ch_cap && ch * 2 <= ch_max && ch * 2 <= kt_per_split) ch *= 2;

  const int kw = kGemvWaves / rw;
  const int lut_bytes = ch * 32 * MP * 32 * 4;
  const int red_bytes = (kw - 1) * 2 * MP * rw * 64 * 4;
  p.path = 0;
  p.groups = G;
  p.rw = rw;
  p.ch = ch;
  p.splits = splits;
  p.kt_per_split = kt_per_split;
  p.grid = G * splits;
  p.block = 64 * kGemvWaves;
  p.lds_bytes = lut_bytes > red_bytes ? lut_bytes : red_bytes;
  p.ws_bytes = splits > 1 ? (size_t)M * N * sizeof(unsigned long long) : 0;
  return p;
}

}  // namespace sherry

using namespace sherry;

namespace {

sherry_status run_gemm(const int8_t* x, const float* s_x, const void* packed, const float* alpha,
                       float* y, int32_t* acc, int64_t M, int64_t N, int64_t K, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (!x || !packed || (y && (!s_x || !alpha)) || (!y && !acc)) return SHERRY_ERR_NULL;
  if (!shape_ok(M, N, K)) return SHERRY_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(packed, 16) || (y && !aligned(y, 4)) || (acc && !aligned(acc, 4)) ||
      (s_x && !aligned(s_x, 4)) || (alpha && !aligned(alpha, 4)))
    return SHERRY_ERR_ALIGN;
  const GemmPlan plan = plan_gemm((int)M, (int)N, (int)K);
  if (plan.ws_bytes > 0) {
    if (!workspace) return SHERRY_ERR_WORKSPACE;
    if (workspace_bytes < plan.ws_bytes) return SHERRY_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return SHERRY_ERR_ALIGN;
  }
  const sherry_status d = check_device();
  if (d != SHERRY_OK) return d;
  GemmArgs args{};
  args.x = x;
  args.s_x = s_x;
  args.packed = static_cast<const uint8_t*>(packed);
  args.alpha = alpha;
  args.y = y;
  args.acc = y ? nullptr : acc;
  args.M = (int)M;
  args.N = (int)N;
  args.K = (int)K;
  if (plan.ws_bytes > 0) args.partials = static_cast<int32_t*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = launch_product(plan, args, s);
  return e == hipSuccess ? SHERRY_OK : SHERRY_ERR_HIP;
}

size_t round256(size_t n) { return (n + 255) / 256 * 256; }

// Scratch of sherry_linear: q [M,K] and s_x [M] when the quantization is
// not fused into the product (any content; not kept zero).
// sherry_linear's plan: the product's, except on the matrix-core GEMV with a
// K-split when the quantization is fused.  Every fused workgroup reads its
// tokens' whole fp32 rows for the scales, so that form takes twice the waves
// per row tile and, from 8 K-splits on, half the splits (measured on MI355X:
// M=1, K=11008, N=4096 8.2 -> 7.2 us; M=4, K=N=4096 8.1 -> 7.8 us).  It keeps
// a K-split, so the workspace it needs is the product's.
GemmPlan plan_linear(int M, int N, int K, bool* fused_out) {
  const GemmPlan plan = plan_gemm(M, N, K);
  bool fused = mfma_gemv_fusable(plan, M, K) || lut_gemv_fusable(plan, M, K);
  GemmPlan out = plan;
  if (fused && plan.path == 2 && plan.splits > 1 && g_ovr_rw.load() == 0 && g_ovr_splits.load() == 0) {
    const int kw = plan.rw * 2 > 16 ? 16 : plan.rw * 2;
    const int splits = plan.splits >= 8 ? plan.splits / 2 : plan.splits;
    const GemmPlan f = mfma_gemv_plan_of(M, N, K, kw, splits);
    if (f.splits > 1 && mfma_gemv_fusable(f, M, K)) out = f;
  }
  if (fused_out) *fused_out = fused;
  return out;
}

size_t linear_scratch(int M, int N, int K, GemmPlan* plan_out, bool* fused_out) {
  bool fused = false;
  const GemmPlan plan = plan_linear(M, N, K, &fused);
  if (plan_out) *plan_out = plan;
  if (fused_out) *fused_out = fused;
  return fused ? 0 : round256((size_t)M * K) + round256((size_t)M * 4);
}

}  // namespace

extern "C" {

const char* sherry_status_string(int status) {
  switch (status) {
    case SHERRY_OK: return "SHERRY_OK";
    case SHERRY_ERR_NULL: return "SHERRY_ERR_NULL: a required pointer is NULL";
    case SHERRY_ERR_SHAPE: return "SHERRY_ERR_SHAPE: need 1<=M,N,K<=2^20, K%16==0, N%4==0";
    case SHERRY_ERR_ALIGN: return "SHERRY_ERR_ALIGN: pointer alignment requirement not met";
    case SHERRY_ERR_WORKSPACE: return "SHERRY_ERR_WORKSPACE: workspace missing or too small";
    case SHERRY_ERR_HIP: return "SHERRY_ERR_HIP: a HIP call or kernel launch failed";
    case SHERRY_ERR_DEVICE: return "SHERRY_ERR_DEVICE: current device is not gfx950";
    default: return "SHERRY_ERR_UNKNOWN";
  }
}

size_t sherry_packed_bytes(int64_t N, int64_t K) {
  if (!shape_ok(1, N, K)) return 0;
  return (size_t)row_tiles((int)N) * (size_t)k_tiles((int)K) * kTileBytes;
}

size_t sherry_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (!shape_ok(M, N, K)) return 0;
  return plan_gemm((int)M, (int)N, (int)K).ws_bytes;
}

sherry_status sherry_gemm_plan(int64_t M, int64_t N, int64_t K, int* path, int* grid, int* block,
                               int* splits, int* lds_bytes) {
  if (!shape_ok(M, N, K)) return SHERRY_ERR_SHAPE;
  const GemmPlan p = plan_gemm((int)M, (int)N, (int)K);
  if (path) *path = p.path;
  if (grid) *grid = p.grid;
  if (block) *block = p.block;
  if (splits) *splits = p.splits;
  if (lds_bytes) *lds_bytes = p.lds_bytes;
  return SHERRY_OK;
}

sherry_status sherry_linear_plan(int64_t M, int64_t N, int64_t K, int* path, int* grid, int* block,
                                 int* splits, int* lds_bytes, int* fused) {
  if (!shape_ok(M, N, K)) return SHERRY_ERR_SHAPE;
  bool f = false;
  const GemmPlan p = plan_linear((int)M, (int)N, (int)K, &f);
  if (path) *path = p.path;
  if (grid) *grid = p.grid;
  if (block) *block = p.block;
  if (splits) *splits = p.splits;
  if (lds_bytes) *lds_bytes = p.lds_bytes;
  if (fused) *fused = f ? 1 : 0;
  return SHERRY_OK;
}

sherry_status sherry_gemm_plan_override(int path, int rw, int ch, int splits) {
  if (path < -1 || path > 2 || rw < 0 || ch < 0 || splits < 0 ||
      (rw && rw != 1 && rw != 2 && rw != 4 && rw != 8 && rw != 16) ||
      (ch && ch != 1 && ch != 2 && ch != 4 && ch != 8))
    return SHERRY_ERR_SHAPE;
  set_plan_override(path, rw, ch, splits);
  return SHERRY_OK;
}

sherry_status sherry_quantize_pack(const float* W, int64_t N, int64_t K, void* packed, float* alpha,
                                   void* stream) {
  if (!W || !packed || !alpha) return SHERRY_ERR_NULL;
  if (!shape_ok(1, N, K)) return SHERRY_ERR_SHAPE;
  if (!aligned(W, 16) || !aligned(packed, 16) || !aligned(alpha, 4)) return SHERRY_ERR_ALIGN;
  const sherry_status d = check_device();
  if (d != SHERRY_OK) return d;
  const hipError_t e = launch_quantize_pack(W, (int)N, (int)K, static_cast<uint8_t*>(packed), alpha,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SHERRY_OK : SHERRY_ERR_HIP;
}

sherry_status sherry_quantize_act(const float* x, int64_t M, int64_t K, int8_t* q, float* s_x,
                                  void* stream) {
  if (!x || !q || !s_x) return SHERRY_ERR_NULL;
  if (M < 1 || K < 4 || M > kMaxDim || K > kMaxDim || K % 4 != 0) return SHERRY_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(q, 4) || !aligned(s_x, 4)) return SHERRY_ERR_ALIGN;
  const sherry_status d = check_device();
  if (d != SHERRY_OK) return d;
  const hipError_t e = launch_quantize_act(x, (int)M, (int)K, q, s_x, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SHERRY_OK : SHERRY_ERR_HIP;
}

sherry_status sherry_gemm(const int8_t* x, const float* s_x, const void* packed, const float* alpha,
                          float* y, int64_t M, int64_t N, int64_t K, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!y) return SHERRY_ERR_NULL;
  return run_gemm(x, s_x, packed, alpha, y, nullptr, M, N, K, workspace, workspace_bytes, stream);
}

sherry_status sherry_gemm_i32(const int8_t* x, const void* packed, int32_t* acc, int64_t M, int64_t N,
                              int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  if (!acc) return SHERRY_ERR_NULL;
  return run_gemm(x, nullptr, packed, nullptr, nullptr, acc, M, N, K, workspace, workspace_bytes,
                  stream);
}

size_t sherry_packed2_bytes(int64_t N, int64_t K) {
  if (!shape_ok(1, N, K)) return 0;
  return (size_t)row_tiles((int)N) * (size_t)k_tiles((int)K) * kTile2Bytes;
}

sherry_status sherry_quantize_pack2(const float* W, int64_t N, int64_t K, void* packed, float* alpha,
                                    void* stream) {
  if (!W || !packed || !alpha) return SHERRY_ERR_NULL;
  if (!shape_ok(1, N, K)) return SHERRY_ERR_SHAPE;
  if (!aligned(W, 16) || !aligned(packed, 16) || !aligned(alpha, 4)) return SHERRY_ERR_ALIGN;
  const sherry_status d = check_device();
  if (d != SHERRY_OK) return d;
  const hipError_t e = launch_quantize_pack2(W, (int)N, (int)K, static_cast<uint8_t*>(packed), alpha,
                                             static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SHERRY_OK : SHERRY_ERR_HIP;
}

size_t sherry_gemm2_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (!shape_ok(M, N, K) || M > kLutMaxM) return 0;
  return plan_mfma_gemv((int)M, (int)N, (int)K).ws_bytes;
}

sherry_status sherry_gemm2(const int8_t* x, const float* s_x, const void* packed, const float* alpha,
                           float* y, int64_t M, int64_t N, int64_t K, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (!x || !s_x || !packed || !alpha || !y) return SHERRY_ERR_NULL;
  if (!shape_ok(M, N, K) || M > kLutMaxM) return SHERRY_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(y, 4) || !aligned(s_x, 4) ||
      !aligned(alpha, 4))
    return SHERRY_ERR_ALIGN;
  const GemmPlan plan = plan_mfma_gemv((int)M, (int)N, (int)K);
  if (plan.ws_bytes > 0) {
    if (!workspace || workspace_bytes < plan.ws_bytes) return SHERRY_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return SHERRY_ERR_ALIGN;
  }
  const sherry_status d = check_device();
  if (d != SHERRY_OK) return d;
  GemmArgs args{};
  args.x = x;
  args.s_x = s_x;
  args.packed = static_cast<const uint8_t*>(packed);
  args.alpha = alpha;
  args.y = y;
  args.M = (int)M;
  args.N = (int)N;
  args.K = (int)K;
  if (plan.ws_bytes > 0) args.partials = static_cast<int32_t*>(workspace);
  const hipError_t e = launch_mfma_gemv2(plan, args, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SHERRY_OK : SHERRY_ERR_HIP;
}

size_t sherry_linear_scratch_bytes(int64_t M, int64_t N, int64_t K) {
  if (!shape_ok(M, N, K)) return 0;
  return linear_scratch((int)M, (int)N, (int)K, nullptr, nullptr);
}

sherry_status sherry_linear(const float* x, const void* packed, const float* alpha, float* y,
                            int64_t M, int64_t N, int64_t K, void* workspace,
                            size_t workspace_bytes, void* scratch, size_t scratch_bytes,
                            void* stream) {
  if (!x || !packed || !alpha || !y) return SHERRY_ERR_NULL;
  if (!shape_ok(M, N, K)) return SHERRY_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(alpha, 4) || !aligned(y, 4))
    return SHERRY_ERR_ALIGN;
  GemmPlan plan;
  bool fused = false;
  const size_t need_scratch = linear_scratch((int)M, (int)N, (int)K, &plan, &fused);
  if (plan.ws_bytes > 0) {
    if (!workspace || workspace_bytes < plan.ws_bytes) return SHERRY_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return SHERRY_ERR_ALIGN;
  }
  if (need_scratch > 0) {
    if (!scratch || scratch_bytes < need_scratch) return SHERRY_ERR_WORKSPACE;
    if (!aligned(scratch, 256)) return SHERRY_ERR_ALIGN;
  }
  const sherry_status d = check_device();
  if (d != SHERRY_OK) return d;
  hipStream_t st = static_cast<hipStream_t>(stream);
  GemmArgs args{};
  args.packed = static_cast<const uint8_t*>(packed);
  args.alpha = alpha;
  args.y = y;
  args.M = (int)M;
  args.N = (int)N;
  args.K = (int)K;
  if (plan.ws_bytes > 0) args.partials = static_cast<int32_t*>(workspace);
  hipError_t e;
  if (fused) {
    args.xf = x;
    e = plan.path == 0 ? launch_lut_gemv(plan, args, st) : launch_mfma_gemv(plan, args, st);
  } else {
    int8_t* q = static_cast<int8_t*>(scratch);
    float* s_x = reinterpret_cast<float*>(q + round256((size_t)M * K));
    e = launch_quantize_act(x, (int)M, (int)K, q, s_x, st);
    if (e == hipSuccess) {
      args.x = q;
      args.s_x = s_x;
      e = launch_product(plan, args, st);
    }
  }
  return e == hipSuccess ? SHERRY_OK : SHERRY_ERR_HIP;
}

}  // extern "C"
