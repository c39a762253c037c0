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
// per row tile and no K-split already keep >= 1024 waves streaming.  With
// fewer, up to 8 tokens use 4 waves per row tile and split K until there are
// >= 1024 waves and each wave has at most ~3 k-tiles; above 8 tokens (whole
// blocks of 16) the 64-bit cells of every split cost more than idle CUs
// save, so 8 waves per row tile and K-splits only to bring a wave to ~3
// k-tiles (measured on MI355X, kernel us, earlier rule -> this one:
// M=16 at N=K=4096 6.40 -> 5.86, M=64 there 13.9 -> 11.1, M=16 at N=4096,
// K=11008 9.16 -> 7.35; at M <= 8 the earlier rule was the best measured).
GemmPlan mfma_gemv_plan_of(int M, int N, int K, int kw, int splits);

GemmPlan plan_mfma_gemv(int M, int N, int K) {
  const int KT = k_tiles(K), RT = row_tiles(N);
  const int ovr_kw = g_ovr_rw.load();
  const bool ovr_has_kw = ovr_kw == 4 || ovr_kw == 8 || ovr_kw == 16;
  int kw = ovr_has_kw ? ovr_kw : (RT >= 128 || M > 8 ? 8 : 4);
  if (M > 16 && kw > 8) kw = 8;   // several token blocks: at most 8 waves
  int splits = 1;
  if (g_ovr_splits.load() > 0) {
    splits = g_ovr_splits.load();
  } else if (RT >= 128) {
    // long K, one token block: split until a wave has at most 8 k-tiles (the
    // straight-line form's limit), 16 above 8 tokens, where each split's
    // cells cost more (measured at N=8192, K=28672: M=1 16.6 -> 11.6 us,
    // M=8 17.1 -> 12.6, M=16 20.3 -> 14.7; at K <= 8192 no split stays the
    // best), unless the row tiles fill at most half the CUs: there the
    // splits' extra workgroups are worth their cells (N=8192 above 8 tokens,
    // 8 against 16 k-tiles per wave: M=10, K=14336 11.6 -> 8.6 us; M=16,
    // K=28672 13.9 -> 13.6; at N=14336, 224 row tiles, M=16, K=16384 a
    // split made it 13.3 -> 14.4).
    if (M <= 16) {
      const int per_split = kw * (M > 8 && 2 * RT > kCUs ? 16 : 8);
      splits = (KT + per_split - 1) / per_split;
    } else if (2 * RT <= kCUs && KT > 8 * kw) {
      // several token blocks at long K on row tiles that fill at most half
      // the CUs: split K so the grid fills one round (N=8192: M=32, K=28672
      // 25.4 -> 18.4 us; M=64, K=14336 23.0 -> 19.6; M=48, K=11008 18.4 ->
      // 15.9; four splits, two rounds, were slower than none, and at
      // N=14336, 224 row tiles, two splits made M=32, K=16384 17.0 -> 24.8)
      splits = kCUs / RT;
    }
  } else if (M > 8) {
    // KT / (3 kw), rounded, but no more workgroups than one round of CUs: a
    // second, partial round costs a whole wave of launches (measured at
    // N=4096, K=14336: 5 splits, 320 workgroups, M=17 13.9 us, M=64 25.0;
    // 4 splits 9.2 and 15.8)
    splits = (2 * KT + 3 * kw) / (6 * kw);
    if (splits * RT > kCUs) splits = kCUs / RT;
    if (splits < 1) splits = 1;
  } else {
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

hipError_t launch_product(const GemmPlan& plan, const GemmArgs& args, hipStream_t stream,
                          bool* partial) {
  if (partial) *partial = false;
  auto one = [&](const GemmArgs& a) {
    return plan.path == 0   ? launch_lut_gemv(plan, a, stream)
           : plan.path == 2 ? launch_mfma_gemv(plan, a, stream)
                            : launch_mfma_gemm(plan, a, stream);
  };
  if (plan.chunk <= 0 || args.M <= plan.chunk) return one(args);
  // launches of plan.chunk tokens in stream order; each leaves the split-K
  // workspace zero for the next.  A launch that fails to enqueue runs
  // nothing, so the workspace stays zero, but the tokens of the launches
  // before it are written and the later ones are not: *partial says so.
  for (int m0 = 0; m0 < args.M; m0 += plan.chunk) {
    GemmArgs c = args;
    c.M = args.M - m0 < plan.chunk ? args.M - m0 : plan.chunk;
    c.x = args.x + (size_t)m0 * args.K;
    if (args.s_x) c.s_x = args.s_x + m0;
    if (args.y) c.y = args.y + (size_t)m0 * args.N;
    if (args.acc) c.acc = args.acc + (size_t)m0 * args.N;
    const hipError_t e = one(c);
    if (e != hipSuccess) {
      if (partial) *partial = m0 > 0;
      return e;
    }
  }
  return hipSuccess;
}

namespace {
// Prefill GEMM: one workgroup per output tile (64 or 128 tokens x 128 or
// 256 weight rows), no K-split across workgroups.  A tile of 128 tokens
// costs half the decode per multiply-add, a tile of 128 weight rows splits
// each wave's K loop in four instead of two; the smaller tiles pay when the
// larger leave CUs idle (M=129..256 at N=14336: 112 tiles of 128 x 256).
// A forced prefill path with rw = 1 or 2 in the override picks the height,
// with ch = 2 or 4 the k-phases.
GemmPlan plan_prefill(int M, int N, int K) {
  GemmPlan p{};
  // Tiles in order of preference, the first whose grid fits the GPU in one
  // round (at most 256 tiles): 64 tokens x 128 weight rows with each
  // workgroup's K split over 4 wave phases; 128 x 128 with 4 phases; 64 x
  // 256 with 2 phases; else 128 x 256 with 2.  Splitting K four ways halves
  // each wave's loop on twice the workgroups (measured at K=4096, M=128:
  // N=14336 20.6 -> 14.5 us, N=4096 20.4 -> 14.2; at M=136, N=4096,
  // K=14336 56.3 -> 36.3), and 128-token tiles halve the decode per
  // multiply-add (M=129..256, N=14336, K=4096: 64 x 256 tiles 20.4 us,
  // 128 x 128 tiles 18.6).
  const long long mt64 = (M + 63) / 64, mt128 = (M + 127) / 128;
  const long long nt128 = (N + 127) / 128, nt256 = (N + 255) / 256;
  int bm = 128, kp = 2;
  if (mt64 * nt128 <= kCUs) bm = 64, kp = 4;
  else if (mt128 * nt128 <= kCUs) bm = 128, kp = 4;
  else if (mt64 * nt256 <= kCUs) bm = 64, kp = 2;
  const int ovr_rw = g_ovr_rw.load();
  const bool forced = g_ovr_path.load() == 1;
  if (forced && (ovr_rw == 1 || ovr_rw == 2)) {
    bm = 64 * ovr_rw;
    kp = (bm == 64 ? mt64 : mt128) * nt128 <= kCUs ? 4 : 2;
  }
  const int ovr_ch = g_ovr_ch.load();
  if (forced && (ovr_ch == 2 || ovr_ch == 4)) kp = ovr_ch;
  p.path = 1;
  p.rw = bm / 64;
  p.ch = kp;
  p.grid = mfma_gemm_grid(M, N, bm, kp);
  p.block = mfma_gemm_threads();
  p.splits = 1;
  p.kt_per_split = k_tiles(K);
  p.lds_bytes = mfma_gemm_lds_bytes(bm, kp);
  p.ws_bytes = 0;
  return p;
}
}  // namespace

// M <= 16: the built-in small-M path (or the override's); 16 < M <= 64: the
// matrix-core GEMV unless the prefill kernel is forced; 64 < M <= 128: the
// prefill kernel, except on a prefill grid of at most 64 workgroups whose
// waves take long shares of K (chunk_max_m), where the same GEMV in
// launches of 64 tokens (each streaming the weights again) is faster; wider
// grids keep the prefill (N=14336, K=4096 M=65 15.6 against 13.1 us;
// N=5504, K=8192 M=72 21.3 against 20.9);
// M > 128: prefill.
// 64 < M <= 128 on a prefill grid of at most 64 workgroups (N <= 4096):
// the most tokens for which the GEMV in launches of 64 tokens beats the
// prefill, by the prefill's k-tiles per wave (one round, so its time grows
// with them).  From sweeps of M = 65..128 step 8 (us, GEMV launches against
// the prefill's 64 x 128 tiles): N=4096, K=14336 (28 k-tiles per wave)
// 19.9 / 32.4 at M=65, 29.8 / 33.1 at M=128; K=11008 (22) 23.5 / 26.5 at
// M=96, 26.6 / 26.7 at M=104; K=8192 (16) 19.3 / 20.7 at M=80, 21.5 / 20.7
// at M=88; N=1024, K=8192 (16) 18.1 / 20.6 at M=80; K=4096 (8) 15.1 / 12.9
// at M=65.
int chunk_max_m(int kt_per_wave) {
  if (kt_per_wave <= 12) return kGemvMaxM;
  if (kt_per_wave <= 18) return 80;
  if (kt_per_wave <= 24) return 96;
  return kChunkMaxM;
}

GemmPlan plan_gemm(int M, int N, int K) {
  GemmPlan p{};
  const int ovr = g_ovr_path.load();
  if (M > kChunkMaxM || (M > kLutMaxM && ovr == 1)) return plan_prefill(M, N, K);
  if (M > kGemvMaxM) {
    const GemmPlan pf = plan_prefill(M, N, K);
    const int kt_per_wave = (k_tiles(K) + pf.ch - 1) / pf.ch;
    if (ovr < 0 && (pf.grid > kChunkMaxGrid || M > chunk_max_m(kt_per_wave))) return pf;
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

  // Built-in plan from sweeps of row tiles per workgroup x table stage x
  // K-splits on MI355X (M = 1..16 at N = 4096..28672, K = 4096..11008):
  // row tiles per workgroup (rw = 1, 2 or 4 row tiles of 4 / rw waves
  // each, or rw = 8: 4 row tiles of 2 waves): up to 4 tokens 1, or 2 from
  // 128 row tiles, and 4 from 448 row tiles; above 4 tokens 8.  K-splits of
  // 2 k-tiles for 1-2 tokens, 4 for 3-4 tokens; above 4 tokens 2 below 128
  // row tiles, 8 from 448, else 4; at most 16 splits: more workgroups keep
  // more lookups in flight, and the 64-bit cell atomics of the splits cost
  // less than idle CUs.  Table stages of one k-tile with 4 row tiles of one
  // wave, two with two waves (one k-tile each), else the largest stage that
  // fits.  Measured against the earlier rule (1 or 4 row tiles, stages as
  // large as fit, 2-k-tile splits above 8 tokens), us: M=8 at N=28672,
  // K=8192 39.3 -> 34.0; M=6 there 40.1 -> 26.7; M=16 there 70.0 -> 60.0;
  // M=1 there 17.3 -> 14.3; M=8 at N=K=4096 12.9 -> 9.9; M=12 at N=14336,
  // K=4096 27.0 -> 22.0; M=1 at N=14336, K=4096 7.3 -> 6.2; M=4 at N=11008
  // 10.8 -> 9.4.  The 8-wave form against 4 row tiles of one wave (2 to 4
  // row tiles above 4 tokens before), us: M=8 at N=28672, K=8192 33.8 ->
  // 29.2; M=16 at N=K=4096 17.3 -> 16.6; M=12 there 13.7 -> 11.6; M=8
  // there 10.1 -> 9.3; M=16 at N=14336 28.3 -> 27.4, at K=11008 29.2 ->
  // 27.3; at M=4 it was slower (6.0 against 6.3).
  const int rw_def = M > 4 ? 8 : RT >= 448 ? 4 : RT >= 128 ? 2 : 1;
  int rw = g_ovr_rw.load() > 0 ? g_ovr_rw.load() : rw_def;
  if (rw != 1 && rw != 2 && rw != 4 && rw != 8) rw = 4;
  const int kt_per_split_def = M <= 2 ? 2 : M <= 4 ? 4 : RT < 128 ? 2 : RT < 448 ? 4 : 8;
  int splits = g_ovr_splits.load() > 0 ? g_ovr_splits.load() : KT / kt_per_split_def;
  if (splits > 16 && g_ovr_splits.load() <= 0) splits = 16;
  if (splits > KT) splits = KT;
  if (splits < 1) splits = 1;
  const int kt_per_split = (KT + splits - 1) / splits;
  splits = (KT + kt_per_split - 1) / kt_per_split;
  if (rw == 8 && kt_per_split < 2) rw = 4;   // two waves need a stage of two k-tiles
  const int rtw = rw == 8 ? 4 : rw;          // row tiles per workgroup
  const int kw = rw == 8 ? 2 : kGemvWaves / rw;   // waves per row tile
  const int G = (RT + rtw - 1) / rtw;
  int ch = rw == 8 ? 2 : 1;
  const int ch_cap = g_ovr_ch.load() > 0 ? g_ovr_ch.load() : (rw == 4 || rw == 8 ? ch : ch_max);
  while (ch * 2 <= ch_cap && ch * 2 <= ch_max && ch * 2 <= kt_per_split) ch *= 2;

  const int lut_bytes = ch * 32 * MP * 32 * 4;
  const int red_bytes = (kw - 1) * 2 * MP * rtw * 64 * 4;
  p.path = 0;
  p.groups = G;
  p.rw = rw;
  p.ch = ch;
  p.splits = splits;
  p.kt_per_split = kt_per_split;
  p.grid = G * splits;
  p.block = 64 * rtw * kw;
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
  if (!aligned(x, 16) || !aligned(packed, 16) || (y && !aligned(y, 16)) || (acc && !aligned(acc, 16)) ||
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
  bool partial = false;
  const hipError_t e = launch_product(plan, args, s, &partial);
  return e == hipSuccess ? SHERRY_OK : (partial ? SHERRY_ERR_PARTIAL : SHERRY_ERR_HIP);
}

size_t round256(size_t n) { return (n + 255) / 256 * 256; }

}  // namespace

// ---------------------------------------------------------------------------
// Static split-K scratch of sherry_gemm_noalloc, for callers that cannot
// allocate device memory.  Each GPU the library runs on holds its own copy
// of this array until the process ends.  In host code `scratch` names a
// host-side stand-in, not the device array: the device address comes from
// hipGetSymbolAddress, once per device with that device current, and only
// that address is ever passed to a kernel.
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;
static __device__ __align__(256) unsigned long long scratch[kNoAllocScratchBytes / sizeof(unsigned long long)];

namespace {

// Zero-fills n16 16-byte chunks (a kernel, not hipMemsetAsync, so that a
// call under graph capture records a kernel node).
__global__ void zero_fill_kernel(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

struct NoAllocScratch {
  std::mutex mu;
  bool resolved = false;
  hipError_t err = hipSuccess;
  void* ptr = nullptr;     // device address of this device's `scratch`
  bool cleared = false;    // a clear has run eagerly (outside graph capture)
};
NoAllocScratch g_noalloc[kMaxDevices];

// The current device's scratch address.  The first call on a device resolves
// it, and until one call has run outside graph capture every call first
// enqueues a zero fill of the whole array on its own stream (the product's
// split-K cells must start at zero; every completed product leaves its
// cells zero again, so later calls need no clear).
sherry_status noalloc_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return SHERRY_ERR_HIP;
  if (dev >= kMaxDevices) return SHERRY_ERR_DEVICE;
  NoAllocScratch& st = g_noalloc[dev];
  std::lock_guard<std::mutex> lock(st.mu);
  if (!st.resolved) {
    void* p = nullptr;
    st.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    st.ptr = st.err == hipSuccess ? p : nullptr;
    st.resolved = true;
  }
  if (st.err != hipSuccess || !st.ptr) return SHERRY_ERR_HIP;
  if (!st.cleared) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess) return SHERRY_ERR_HIP;
    hipLaunchKernelGGL(zero_fill_kernel, dim3(512), dim3(256), 0, stream, static_cast<uint4*>(st.ptr),
                       kNoAllocScratchBytes / 16);
    if (hipGetLastError() != hipSuccess) return SHERRY_ERR_HIP;
    if (cap == hipStreamCaptureStatusNone) st.cleared = true;
  }
  *out = st.ptr;
  return SHERRY_OK;
}

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
    case SHERRY_ERR_PARTIAL:
      return "SHERRY_ERR_PARTIAL: a launch failed after earlier launches of the call were enqueued; "
             "the output is incomplete, the workspace is left zero";
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

sherry_status sherry_gemm_noalloc(const int8_t* x, const float* s_x, const void* packed,
                                  const float* alpha, float* y, int64_t M, int64_t N, int64_t K,
                                  void* stream) {
  if (!x || !s_x || !packed || !alpha || !y) return SHERRY_ERR_NULL;
  if (!shape_ok(M, N, K)) return SHERRY_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(y, 16) || !aligned(s_x, 4) ||
      !aligned(alpha, 4))
    return SHERRY_ERR_ALIGN;
  const GemmPlan plan = plan_gemm((int)M, (int)N, (int)K);
  if (plan.ws_bytes > kNoAllocScratchBytes) return SHERRY_ERR_WORKSPACE;
  const sherry_status d = check_device();
  if (d != SHERRY_OK) return d;
  hipStream_t s = static_cast<hipStream_t>(stream);
  GemmArgs args{};
  args.x = x;
  args.s_x = s_x;
  args.packed = static_cast<const uint8_t*>(packed);
  args.alpha = alpha;
  args.y = y;
  args.M = (int)M;
  args.N = (int)N;
  args.K = (int)K;
  if (plan.ws_bytes > 0) {
    void* cells = nullptr;
    const sherry_status st = noalloc_scratch(s, &cells);
    if (st != SHERRY_OK) return st;
    args.partials = static_cast<int32_t*>(cells);
  }
  bool partial = false;
  const hipError_t e = launch_product(plan, args, s, &partial);
  return e == hipSuccess ? SHERRY_OK : (partial ? SHERRY_ERR_PARTIAL : SHERRY_ERR_HIP);
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
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(y, 16) || !aligned(s_x, 4) ||
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
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(alpha, 4) || !aligned(y, 16))
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
  bool partial = false;
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
      e = launch_product(plan, args, st, &partial);
      partial = true;   // the quantizer's launch was enqueued before it
    }
  }
  return e == hipSuccess ? SHERRY_OK : (partial ? SHERRY_ERR_PARTIAL : SHERRY_ERR_HIP);
}

}  // extern "C"
