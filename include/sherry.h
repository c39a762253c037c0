/*
 * sherry.h -- C ABI of the Sherry 3:4-sparse ternary matmul library for
 * AMD MI355X (gfx950).
 *
 * Method: the page "Sherry框架：三元量化与3:4稀疏优化LLM推理"
 * (pnsm.cn/news/1195499.html).  Weights are ternary {-1,0,+1} with exactly
 * three nonzeros in every block of four consecutive weights of a row
 * (§1.1).  A block is stored in 5 bits: a 4-bit index into the 16 canonical
 * patterns plus one sign bit, 1.25 bit/weight (§2.1).  Inference cuts the
 * int8 activations into 4-element segments, builds one table of the 16
 * pattern dot products per segment, looks each weight block up, applies its
 * sign, sums in integers and rescales once in float (§2.2).  The ternary
 * block is the solution of min ||W - a*T||^2 with ||T||_0 = 3: keep the three
 * largest |w| with their signs (§3.1).
 *
 * Conventions shared by every entry point
 *   - W is [N,K] row-major fp32 (N outputs, K inputs); x and y are [M,K] and
 *     [M,N] row-major.  y[m,n] = sum_k x[m,k] * W[n,k] in the quantized
 *     domain: y = ((float)acc[m,n] * s_x[m]) * alpha[n],
 *     acc[m,n] = sum_k q[m,k] * T[n,k] exactly in int32.
 *   - Every pointer argument is a DEVICE pointer unless stated otherwise.
 *     The caller allocates and frees every buffer; the library allocates no
 *     device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work on `stream` and returns; results are
 *     visible after the caller synchronizes the stream.
 *   - Argument errors are found on the host before any HIP call; such a call
 *     enqueues nothing and returns a negative status.  A failed launch
 *     returns SHERRY_ERR_HIP, or SHERRY_ERR_PARTIAL when launches of the
 *     same call were enqueued before it.  A fault inside a kernel is
 *     reported by the caller's next synchronizing HIP call, not by this
 *     library.
 *   - Shapes supported: K % 16 == 0, N % 4 == 0, 1 <= M,N,K <= 2^20
 *     (whole 4-weight blocks, 16-byte aligned int8 activation rows and
 *     whole 16-byte output stores).
 *   - Code 5-bit layout ("packed"): code c = 2*p + s per block; p = 4*z +
 *     2*r1 + r2 where z is the zero position and r1 (r2) says the 2nd (3rd)
 *     nonzero's sign differs from the 1st's; s = 1 iff the 1st nonzero is -1.
 *     Rows are grouped in tiles of 64 rows x 128 columns (1280 bytes),
 *     row-tile-major and column-tile-minor.  Tile row r = 16t + i
 *     (t = 0..3, i = 0..15) keeps its 32 codes as four groups of 8: group g
 *     (blocks 8g..8g+7) is a 40-bit little-endian string with block 8g+jj at
 *     bits [5jj, 5jj+5).  It belongs to slot L = 16g + i: group bits 0..31
 *     are the 4 bytes at tile byte 16*L + 4*t, bits 32..39 the byte at tile
 *     byte 1024 + 4*L + t.  (Slot L is what lane L of a 64-wide wave loads;
 *     it holds that lane's matrix-core operands.)  The matrix is padded to
 *     whole tiles (N up to a
 *     multiple of 64, K up to a multiple of 128); padding blocks hold code 0
 *     and no product uses them.  Total sherry_packed_bytes(N,K) =
 *     ceil(N/64) * ceil(K/128) * 1280 bytes (N*K*5/32 when no padding).
 */
#ifndef SHERRY_H
#define SHERRY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SHERRY_OK = 0,
  SHERRY_ERR_NULL = -1,      /* a required pointer is NULL */
  SHERRY_ERR_SHAPE = -2,     /* M, N or K out of range or not a multiple */
  SHERRY_ERR_ALIGN = -3,     /* a pointer is not aligned as required */
  SHERRY_ERR_WORKSPACE = -4, /* workspace missing or smaller than required */
  SHERRY_ERR_HIP = -5,       /* a HIP runtime call or launch failed */
  SHERRY_ERR_DEVICE = -6,    /* the current device is not a gfx950 GPU */
  SHERRY_ERR_PARTIAL = -7    /* a launch failed after earlier launches of the
                                same call were enqueued (sherry_linear's
                                quantizer, or the 64-token launches of
                                64 < M <= 128): those complete, so the output
                                is partly written; a launch that fails runs
                                nothing and every launch that runs leaves the
                                split-K workspace zero, so the workspace needs
                                no re-zeroing */
} sherry_status;

/* Human-readable name of a status code (static string; never NULL). */
const char* sherry_status_string(int status);

/* Bytes of the packed 5-bit weight format for an [N,K] matrix: N*K*5/32.
 * Host-only, pure; returns 0 for an unsupported shape. */
size_t sherry_packed_bytes(int64_t N, int64_t K);

/* Bytes of scratch that sherry_gemm / sherry_gemm_i32 need for this shape
 * (0 when the chosen kernel needs none).  Host-only, pure.
 * The workspace holds one 64-bit accumulator per output when the product is
 * split along K.  It must be zero-filled once before its first use; every
 * completed call leaves it zero-filled again, so one buffer of the largest
 * size needed can serve any sequence of calls on one stream.  Calls that run
 * concurrently must not share a workspace. */
size_t sherry_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* Offline compression (kernel 1), §3.1 and §2.1.
 *   W      [N,K] fp32, finite values, 16-byte aligned (read only).
 *   packed sherry_packed_bytes(N,K) bytes, 16-byte aligned (written).
 *   alpha  [N] fp32 (written): alpha[n] = (sum of the kept |W[n,k]|,
 *          accumulated in double in ascending k) / (3*K/4), rounded once.
 * Per block the smallest |w| is dropped (the lowest index on ties) and the
 * other three keep their signs (w < 0 -> -1, otherwise +1, so -0.0 -> +1). */
sherry_status sherry_quantize_pack(const float* W, int64_t N, int64_t K,
                                   void* packed, float* alpha, void* stream);

/* Per-token symmetric int8 quantization of activations (the input stage of
 * the product; the page's lookup works on int8 segments, §2.2).
 *   x    [M,K] fp32, finite, 16-byte aligned.  K % 4 == 0 is enough here.
 *   q    [M,K] int8 (written), 4-byte aligned.
 *   s_x  [M] fp32 (written): s = max_k |x[m,k]| / 127 (float division);
 *        q = clamp(rint(x / s), -127, 127) rounding half to even.
 *        An all-zero row gives s = 1 and q = 0. */
sherry_status sherry_quantize_act(const float* x, int64_t M, int64_t K,
                                  int8_t* q, float* s_x, void* stream);

/* The product, §2.2: y[m,n] = ((float)acc[m,n] * s_x[m]) * alpha[n] with
 * acc[m,n] = sum_k x[m,k] * T[n,k] in int32 (exact; any int8 value of x is
 * accepted, -128 included).
 *   x        [M,K] int8, 16-byte aligned.
 *   s_x      [M] fp32.            alpha  [N] fp32 (from sherry_quantize_pack).
 *   packed   packed weights, 16-byte aligned.
 *   y        [M,N] fp32 (written), 16-byte aligned (with N % 4 == 0 every
 *            row then starts on a 16-byte boundary; the prefill GEMM stores
 *            16 bytes per lane).
 *   workspace / workspace_bytes: scratch of at least
 *            sherry_workspace_bytes(M,N,K) bytes, 256-byte aligned, zero
 *            filled before first use (may be NULL when that size is 0).
 * Every path decodes the codes or looks them up; which one runs depends on
 * M (sherry_gemm_plan reports it), and every path returns identical results:
 *   M <= 16: the matrix-core GEMV (codes decoded to int8 {-1,0,+1}, tokens
 *            padded to 16, one 64-row weight tile per workgroup), or the
 *            lookup-table GEMV (per-segment tables of the 16 pattern dot
 *            products and their negations in LDS, one lookup per weight
 *            block and token pair);
 *   16 < M <= 64: the matrix-core GEMV with the tokens in two or four
 *            blocks of 16;
 *   64 < M <= 128: the prefill GEMM below, except when its grid is at
 *            most 64 workgroups and its waves take long shares of K (more
 *            than 12 k-tiles each up to M = 80, more than 18 up to 96,
 *            more than 24 up to 128): then that GEMV in launches of 64
 *            tokens on the same stream (sherry_workspace_bytes covers one
 *            launch);
 *   M > 128: the prefill GEMM on the int8 matrix cores, in the first
 *            workgroup tile whose grid fits the GPU in one round (at most
 *            256 tiles): 64 tokens x 128 weight rows, 128 x 128, 64 x 256,
 *            else 128 x 256; tiles 128 rows wide split each workgroup's K
 *            over 4 wave phases, 256 rows wide over 2. */
sherry_status sherry_gemm(const int8_t* x, const float* s_x, const void* packed,
                          const float* alpha, float* y, int64_t M, int64_t N,
                          int64_t K, void* workspace, size_t workspace_bytes,
                          void* stream);

/* The same product as sherry_gemm for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): no workspace argument.  When the plan splits K, the
 * split-K cells live in a static device array of the library, 8 MiB per
 * GPU (held until the process ends), so shapes whose
 * sherry_workspace_bytes(M,N,K) exceeds 8 MiB (8388608) are rejected with
 * SHERRY_ERR_WORKSPACE before anything is enqueued.  The call allocates
 * nothing and calls no allocating routine.
 *   Arguments, alignment, shapes and results: as sherry_gemm (identical y).
 *   The first call on a device resolves the array's device address; until
 *   one call has run outside graph capture, each call first enqueues a
 *   zero fill of the array (one extra small kernel) on its stream.  Every
 *   completed call leaves the array zero again.
 *   Every call on one GPU shares that GPU's array: calls that can overlap
 *   on one GPU (different streams, or different threads without ordering)
 *   race and may return wrong sums; serialize them on one stream. */
sherry_status sherry_gemm_noalloc(const int8_t* x, const float* s_x, const void* packed,
                                  const float* alpha, float* y, int64_t M, int64_t N,
                                  int64_t K, void* stream);

/* Same product, stopping at the int32 accumulators: acc [M,N] int32
 * (written, 16-byte aligned).  Same kernels and workspace rules. */
sherry_status sherry_gemm_i32(const int8_t* x, const void* packed, int32_t* acc,
                              int64_t M, int64_t N, int64_t K, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Bytes of scratch (beyond the workspace) that sherry_linear needs for this
 * shape: q [M,K] and s_x [M] when the quantization is not fused into the
 * product, else 0.  Host-only, pure; 0 for an unsupported shape. */
size_t sherry_linear_scratch_bytes(int64_t M, int64_t N, int64_t K);

/* The whole decode step from fp32 activations: per-token int8 quantization
 * (as sherry_quantize_act) followed by the product (as sherry_gemm), with
 * identical results: y is bit-identical to calling the two.  Small token
 * counts (M <= 4, M*K <= 16384) on the matrix-core GEMV path quantize inside
 * the product kernel (one launch, no round trip of q through memory);
 * otherwise q and s_x are first written to `scratch`.
 *   x        [M,K] fp32, finite, 16-byte aligned.
 *   packed, alpha, y, M, N, K: as sherry_gemm.
 *   workspace / workspace_bytes: as sherry_gemm (sherry_workspace_bytes,
 *            zero filled before first use, left zero by every call).
 *   scratch / scratch_bytes: at least sherry_linear_scratch_bytes(M,N,K)
 *            bytes, 256-byte aligned, any content (may be NULL when 0);
 *            must not overlap the workspace. */
sherry_status sherry_linear(const float* x, const void* packed, const float* alpha,
                            float* y, int64_t M, int64_t N, int64_t K,
                            void* workspace, size_t workspace_bytes,
                            void* scratch, size_t scratch_bytes, void* stream);

/* --- 2-bit baseline -------------------------------------------------------
 * The plain ternary packing the Sherry page measures its 5-bit code against
 * (§2.1: the 5-bit code cuts bit-operation overhead relative to 2-bit
 * packing): the SAME ternary weights and alpha as sherry_quantize_pack,
 * written 2 bits per weight (0 -> 00, +1 -> 01, -1 -> 11), so every product
 * is identical to sherry_gemm's and only the format (2 vs 1.25 bit/weight)
 * and its decode differ.  Layout: tiles of 64 rows x 128 columns (2048
 * bytes), row-tile-major; weight j of tile row r at bits [2j, 2j+2) of the
 * row's 256-bit little-endian string, bits 0..127 at tile byte 16*r and bits
 * 128..255 at tile byte 1024 + 16*r.  Same shape rules as the 5-bit format. */

/* ceil(N/64) * ceil(K/128) * 2048 (N*K/4 when no padding; padding is 00);
 * host-only, pure; 0 for an unsupported shape. */
size_t sherry_packed2_bytes(int64_t N, int64_t K);

/* As sherry_quantize_pack, output in the 2-bit format (packed: 16-byte
 * aligned, sherry_packed2_bytes(N,K) bytes). */
sherry_status sherry_quantize_pack2(const float* W, int64_t N, int64_t K,
                                    void* packed, float* alpha, void* stream);

/* Scratch bytes of sherry_gemm2 (same zero-fill rule as
 * sherry_workspace_bytes); 0 when M > 16 or the shape is unsupported. */
size_t sherry_gemm2_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* The product on the 2-bit format, decode shapes only (1 <= M <= 16, else
 * SHERRY_ERR_SHAPE): the matrix-core GEMV with the codes decoded through a
 * 256-entry table (one lookup per 4 weights).  Arguments as sherry_gemm. */
sherry_status sherry_gemm2(const int8_t* x, const float* s_x, const void* packed,
                           const float* alpha, float* y, int64_t M, int64_t N,
                           int64_t K, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Launch plan sherry_gemm uses for a shape (host-only, pure; for
 * diagnostics and benchmarks).  Any output pointer may be NULL.
 *   path: 0 = lookup-table GEMV (per-segment tables in LDS, §2.2; M <= 16),
 *         1 = decode + int8 matrix-core GEMM (M > 64, except where path 2
 *             runs in launches of 64 tokens),
 *         2 = decode + int8 matrix-core GEMV (M <= 128; grid is per launch
 *             of at most 64 tokens).
 *   grid: workgroups per launch; block: threads per workgroup;
 *   splits: K-splits per output row group (1 = none);
 *   lds_bytes: LDS per workgroup. */
sherry_status sherry_gemm_plan(int64_t M, int64_t N, int64_t K, int* path,
                               int* grid, int* block, int* splits,
                               int* lds_bytes);

/* Launch plan of sherry_linear's product for a shape, with the same outputs
 * as sherry_gemm_plan, plus fused = 1 when the quantization runs inside the
 * product kernel (one launch), else 0 (sherry_quantize_act first, then the
 * product on the plan above).  The fused form on path 2 with a K-split takes
 * twice the waves per row tile of sherry_gemm's plan and, from 8 K-splits on,
 * half the splits: its workgroups each read their tokens' whole fp32 rows
 * for the scales, so fewer, wider workgroups cost less.  Host-only, pure;
 * follows sherry_gemm_plan_override (with rw or splits set, the fused form
 * keeps that plan). */
sherry_status sherry_linear_plan(int64_t M, int64_t N, int64_t K, int* path,
                                 int* grid, int* block, int* splits,
                                 int* lds_bytes, int* fused);

/* Tuning knob for benchmark sweeps and tests (host-only).  Replaces the
 * built-in launch plan for shapes with M <= 128 for every later call in this
 * process (M > 128 always uses path 1):
 *   path   -1 = built-in choice, or 0, 1, 2 as in sherry_gemm_plan; for
 *          16 < M <= 128, 1 gives the prefill GEMM and 0 or 2 the GEMV.
 *   rw     path 0: row tiles per workgroup, 1, 2 or 4 (the workgroup's 4
 *          waves are rw row tiles x 4/rw waves sharing one), or 8: 4 row
 *          tiles x 2 waves (512 threads; needs K-splits of at least 2
 *          k-tiles, else 4 is taken);
 *          path 2: waves per workgroup sharing its one row tile, 4, 8 or
 *          16 (at most 8 when M > 16);
 *          path 1 (forced): 1 or 2 = tiles of 64 or 128 tokens;
 *          0 (or a value the path does not take) = built-in choice.
 *   ch     path 0: k-tiles (128 inputs) per LDS table stage: 1, 2, 4
 *          or 8, capped so one stage stays within 32 KB (with rw = 8 at
 *          least 2, one per wave, up to 64 KB);
 *          path 1 (forced): 2 or 4 k-phases (4: tiles 128 weight rows
 *          wide, each workgroup's K split four ways);
 *          0 = built-in.
 *   splits K-splits per output row group; 0 = built-in choice.
 * Results do not depend on the plan.  sherry_workspace_bytes reflects the
 * override, so query it after setting one.  Not thread-safe with respect to
 * concurrent calls.  Returns SHERRY_ERR_SHAPE for an invalid value. */
sherry_status sherry_gemm_plan_override(int path, int rw, int ch, int splits);

/* --- Diagnostics (not part of the product) -------------------------------
 * Ceilings for the benchmark, measured in the same process as the product:
 * the plain streaming-read rate of a device buffer, the cost of an empty
 * launch and the rate of the decode step alone. */

/* Reads `bytes` (a multiple of 16) of device memory at `src` (16-byte
 * aligned) with 16-byte loads: grid x block threads (block a multiple of 64,
 * at most 1024), each keeping `unroll` (1, 2, 4 or 8) loads in flight, the
 * grid walking the buffer front to back.  Nothing is written unless the XOR
 * of all the data equals one fixed constant; then one dword goes to `sink`
 * (device, 4-byte aligned).  Asynchronous on `stream`. */
sherry_status sherry_probe_read(const void* src, size_t bytes, void* sink, int grid, int block,
                                int unroll, void* stream);

/* Enqueues an empty kernel (one workgroup of 64 threads) on `stream`. */
sherry_status sherry_probe_empty(void* stream);

/* The decode step of the matrix-core kernels with nothing else in the loop:
 * grid x block threads (block a multiple of 64, at most 1024; iters and
 * grid in [1, 2^20]) each look up sherry_probe_decode_codes(iters, 1, 1)
 * codes as code pairs in a 1024-entry table of 8-byte entries in LDS
 * (two 8-byte lookups per 4 codes, the product's decode).  The looked-up
 * values are folded and written to `sink` (device, 4-byte aligned) only if
 * they equal one fixed constant.  Asynchronous on `stream`. */
sherry_status sherry_probe_decode(int iters, void* sink, int grid, int block, void* stream);

/* Codes one sherry_probe_decode launch looks up (0 for non-positive
 * arguments).  Host-only. */
int64_t sherry_probe_decode_codes(int iters, int grid, int block);

#ifdef __cplusplus
}
#endif

#endif /* SHERRY_H */
