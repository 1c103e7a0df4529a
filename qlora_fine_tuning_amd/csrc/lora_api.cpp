// C ABI of the fused LoRA / QLoRA layer: argument validation (before any HIP call), workspace
// layout, and dispatch to the gfx950 kernels.  Declarations and conventions: include/lora.h.
#include "lora.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "launch.hpp"

namespace {

using namespace lora;

thread_local const char* g_last_hip_error = "hipSuccess";

constexpr int64_t kMaxElems = (int64_t)1 << 31;
// Longest row (N or K): the kernels address a 256-row tile with 32-bit byte offsets.
constexpr int64_t kMaxRow = (int64_t)1 << 20;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

lora_status check_dims(int64_t M, int64_t N, int64_t K, int32_t R) {
  if (M < 0 || N <= 0 || K <= 0 || N % 64 != 0 || K % 64 != 0) return LORA_ERR_SHAPE;
  if (M >= kMaxElems || N > kMaxRow || K > kMaxRow) return LORA_ERR_SHAPE;
  if (M * K >= kMaxElems || M * N >= kMaxElems || N * K >= kMaxElems) return LORA_ERR_SHAPE;
  if (R < 8 || R > 64 || R % 8 != 0) return LORA_ERR_RANK;
  return LORA_OK;
}

// every pointer non-null and 16-byte aligned
template <typename... P>
lora_status check_ptrs(P... ps) {
  const void* arr[] = {static_cast<const void*>(ps)...};
  for (const void* p : arr)
    if (p == nullptr) return LORA_ERR_NULL;
  for (const void* p : arr)
    if (!aligned16(p)) return LORA_ERR_ALIGN;
  return LORA_OK;
}

lora_status from_hip(hipError_t e) {
  if (e == hipSuccess) return LORA_OK;
  g_last_hip_error = hipGetErrorName(e);
  return LORA_ERR_HIP;
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Tokens per split of the dA/dB partial pass: 256 on the fp32 path; the bf16 / int4 path
// doubles it while the grid keeps at least 512 workgroups, the number resident at once (two per
// CU): longer-lived workgroups, fewer partials to write and add.
int64_t dadb_split_rows(int64_t M, int64_t N, int64_t K, bool mfma) {
  int64_t rows = kSplitRows;
  if (!mfma) return rows;
  const int64_t tiles = (K + kDadbCols - 1) / kDadbCols + (N + kDadbCols - 1) / kDadbCols;
  while (rows < 2048 && tiles * ((M + 2 * rows - 1) / (2 * rows)) >= 512) rows *= 2;
  return rows;
}
int64_t splits_for(int64_t M, int64_t N, int64_t K, bool mfma) {
  const int64_t rows = dadb_split_rows(M, N, K, mfma);
  return (M + rows - 1) / rows;
}

// Backward workspace: G [M][R] fp32 | partA [splits][R][K] fp32 | partB [splits][R][N] fp32,
// then, for an MFMA (bf16 / int4) input gradient whose N is split, its per-tile arrival
// counters and split partials, and for an MFMA input gradient of rank above 32, the scratch of
// its G pass (B transposed, per-share partials).
struct BwdLayout {
  size_t g, pa, pb, ctr, dxp, pan, total;
};
BwdLayout bwd_layout(int64_t M, int64_t N, int64_t K, int32_t R, bool mfma) {
  const int64_t s = splits_for(M, N, K, mfma);
  BwdLayout l;
  l.g = 0;
  l.pa = align256((size_t)M * R * sizeof(float));
  l.pb = l.pa + align256((size_t)s * R * K * sizeof(float));
  l.ctr = l.pb + align256((size_t)s * R * N * sizeof(float));
  l.dxp = l.ctr;
  l.total = l.ctr;
  const size_t part = mfma ? dx_part_bytes(M, N, K, R) : 0;
  if (part > 0) {
    l.dxp = l.ctr + align256((size_t)dx_tiles(M, K) * sizeof(uint32_t));
    l.total = l.dxp + align256(part);
  }
  l.pan = l.total;
  if (mfma && R > 32) l.total = l.pan + align256(panel_workspace_bytes(M, N, R));
  return l;
}

bool use_gemv(int64_t M, int64_t K) { return M >= 1 && M <= 8 && K % 1024 == 0; }

// The two halves of the backward; sizes and pointers validated by the callers.
lora_status bwd_dx_common(bool int4, lora_dtype dt, int64_t M, int64_t N, int64_t K, int32_t R,
                          float scale, const void* dY, const void* W, const void* Ws, const void* A,
                          const void* B, void* dX, void* ws, size_t ws_bytes, void* stream, bool fp4 = false) {
  const BwdLayout lay = bwd_layout(M, N, K, R, dt != LORA_F32);
  if (ws == nullptr || ws_bytes < lay.total) return LORA_ERR_WORKSPACE;
  if (!aligned16(ws)) return LORA_ERR_ALIGN;
  if (M == 0) return LORA_OK;
  char* base = static_cast<char*>(ws);
  float* G = reinterpret_cast<float*>(base + lay.g);
  DxArgs a{dY, W, Ws, A, B, dX, G, M, N, K, R, scale, reinterpret_cast<uint32_t*>(base + lay.ctr),
           reinterpret_cast<float*>(base + lay.dxp)};
  a.fp4 = fp4;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dt == LORA_F32) return from_hip(launch_dx_f32(a, s));
  if (R > 32) {  // the rank-64 input-gradient kernel reads G from this pass
    const hipError_t e = launch_panel_g(static_cast<const uint16_t*>(dY), static_cast<const uint16_t*>(B), G,
                                        base + lay.pan, M, N, R, s);
    if (e != hipSuccess) return from_hip(e);
  }
  return from_hip(launch_dx_mfma(a, int4, s));
}

lora_status bwd_dadb_common(lora_dtype dt, int64_t M, int64_t N, int64_t K, int32_t R, float scale,
                            const void* dY, const void* X, const float* XA, float* dA, float* dB,
                            void* ws, size_t ws_bytes, void* stream) {
  const BwdLayout lay = bwd_layout(M, N, K, R, dt != LORA_F32);
  if (ws == nullptr || ws_bytes < lay.total) return LORA_ERR_WORKSPACE;
  if (!aligned16(ws)) return LORA_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  DadbArgs d{X, dY, reinterpret_cast<const float*>(base + lay.g), XA,
             reinterpret_cast<float*>(base + lay.pa), reinterpret_cast<float*>(base + lay.pb),
             dA, dB, M, N, K, R, scale, (int)splits_for(M, N, K, dt != LORA_F32),
             (int)dadb_split_rows(M, N, K, dt != LORA_F32)};
  if (M > 0) {
    const hipError_t e = (dt == LORA_F32) ? launch_dadb_partials_f32(d, s) : launch_dadb_partials_bf16(d, s);
    if (e != hipSuccess) return from_hip(e);
  }
  return from_hip(launch_dadb_reduce(d, s));
}

// SwiGLU pair: the rank is that of each adapter (R), the stacked GEMM runs at 2N and 2R.
lora_status check_swiglu(int64_t M, int64_t N, int64_t K, int32_t R) {
  if (N <= 0 || N % 64 != 0 || N > kMaxRow / 2) return LORA_ERR_SHAPE;
  if (R < 8 || R > 32 || R % 8 != 0) return LORA_ERR_RANK;
  return check_dims(M, 2 * N, K, 2 * R);
}
// forward workspace: As [2R][K] bf16 | Bs [2N][2R] bf16
struct SwigluLayout {
  size_t as, bs, dgu, das, dbs, inner, total;
};
SwigluLayout swiglu_layout(int64_t M, int64_t N, int64_t K, int32_t R, bool bwd) {
  SwigluLayout l;
  l.as = 0;
  l.bs = align256((size_t)2 * R * K * 2);
  l.dgu = l.bs + align256((size_t)4 * N * R * 2);
  l.total = l.dgu;
  l.das = l.dbs = l.inner = l.total;
  if (!bwd) return l;
  // backward: then [dG | dU] (M x 2N bf16), the stacked dA (2R x K) and dB (2N x 2R) fp32, and
  // the stacked problem's backward workspace
  l.das = l.dgu + align256((size_t)M * 2 * N * 2);
  l.dbs = l.das + align256((size_t)2 * R * K * 4);
  l.inner = l.dbs + align256((size_t)4 * N * R * 4);
  l.total = l.inner + bwd_layout(M, 2 * N, K, 2 * R, true).total;
  return l;
}

// fmt: 0 bf16 weight; 64 int4 codes + fp16 scales (Ws); 32 MXFP4 codes + E8M0 bytes (Ws)
lora_status swiglu_fwd_impl(int fmt, int64_t M, int64_t N, int64_t K, int32_t R, float scale, const void* X,
                            const void* Wgu, const void* Ws, const void* Ag, const void* Au, const void* Bg, const void* Bu,
                            void* H, void* GU, float* XA, void* ws, size_t ws_bytes, void* stream) {
  lora_status st = check_swiglu(M, N, K, R);
  if (st != LORA_OK) return st;
  if (!std::isfinite(scale)) return LORA_ERR_VALUE;
  st = check_ptrs(Wgu, Ag, Au, Bg, Bu);
  if (st != LORA_OK) return st;
  if (M == 0) return LORA_OK;  // empty batch: X, H, GU and XA may be NULL
  st = check_ptrs(X, H, GU);
  if (st != LORA_OK) return st;
  if (XA != nullptr && !aligned16(XA)) return LORA_ERR_ALIGN;
  const SwigluLayout lay = swiglu_layout(M, N, K, R, false);
  if (ws == nullptr || ws_bytes < lay.total) return LORA_ERR_WORKSPACE;
  if (!aligned16(ws)) return LORA_ERR_ALIGN;
  char* base = static_cast<char*>(ws);
  uint16_t* As = reinterpret_cast<uint16_t*>(base + lay.as);
  uint16_t* Bs = reinterpret_cast<uint16_t*>(base + lay.bs);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_swiglu_stack(static_cast<const uint16_t*>(Ag), static_cast<const uint16_t*>(Au),
                                     static_cast<const uint16_t*>(Bg), static_cast<const uint16_t*>(Bu), As, Bs,
                                     N, K, R, s);
  if (e != hipSuccess) return from_hip(e);
  // [G | U] = X [Wg; Wu]^T + scale (X [Ag; Au]^T) [Bg 0; 0 Bu]^T: one GEMM over both
  // projections, whose epilogue also forms H = silu(G) U from the fp32 accumulators
  FwdArgs a{X, Wgu, Ws, As, Bs, GU, XA, M, 2 * N, K, 2 * R, scale, H};
  a.fp4 = fmt == 32;
  return from_hip(launch_fwd_mfma(a, fmt != 0, s));
}

lora_status swiglu_bwd_impl(int fmt, int64_t M, int64_t N, int64_t K, int32_t R, float scale, const void* dH,
                            const void* X, const void* Wgu, const void* Ws, const void* Ag, const void* Au, const void* Bg,
                            const void* Bu, const void* GU, const float* XA, void* dX, float* dAg, float* dAu,
                            float* dBg, float* dBu, void* ws, size_t ws_bytes, void* stream) {
  lora_status st = check_swiglu(M, N, K, R);
  if (st != LORA_OK) return st;
  if (!std::isfinite(scale)) return LORA_ERR_VALUE;
  st = check_ptrs(Wgu, Ag, Au, Bg, Bu, dAg, dAu, dBg, dBu);
  if (st != LORA_OK) return st;
  if (M > 0 && (st = check_ptrs(dH, X, GU, XA, dX)) != LORA_OK) return st;
  const SwigluLayout lay = swiglu_layout(M, N, K, R, true);
  if (ws == nullptr || ws_bytes < lay.total) return LORA_ERR_WORKSPACE;
  if (!aligned16(ws)) return LORA_ERR_ALIGN;
  char* base = static_cast<char*>(ws);
  uint16_t* As = reinterpret_cast<uint16_t*>(base + lay.as);
  uint16_t* Bs = reinterpret_cast<uint16_t*>(base + lay.bs);
  uint16_t* dGU = reinterpret_cast<uint16_t*>(base + lay.dgu);
  float* dAs = reinterpret_cast<float*>(base + lay.das);
  float* dBs = reinterpret_cast<float*>(base + lay.dbs);
  void* inner = base + lay.inner;
  const size_t inner_bytes = ws_bytes - lay.inner;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_swiglu_stack(static_cast<const uint16_t*>(Ag), static_cast<const uint16_t*>(Au),
                                     static_cast<const uint16_t*>(Bg), static_cast<const uint16_t*>(Bu), As, Bs,
                                     N, K, R, s);
  if (e != hipSuccess) return from_hip(e);
  e = launch_swiglu_bwd(static_cast<const uint16_t*>(dH), static_cast<const uint16_t*>(GU), dGU, M, N, s);
  if (e != hipSuccess) return from_hip(e);
  // the LoRA backward of the stacked GEMM with [dG | dU] as its upstream gradient
  st = bwd_dx_common(fmt != 0, LORA_BF16, M, 2 * N, K, 2 * R, scale, dGU, Wgu, Ws, As, Bs, dX, inner,
                     inner_bytes, stream, fmt == 32);
  if (st != LORA_OK) return st;
  st = bwd_dadb_common(LORA_BF16, M, 2 * N, K, 2 * R, scale, dGU, X, XA, dAs, dBs, inner, inner_bytes, stream);
  if (st != LORA_OK) return st;
  return from_hip(launch_swiglu_unstack(dAs, dBs, dAg, dAu, dBg, dBu, N, K, R, s));
}

}  // namespace

extern "C" {

const char* lora_status_str(int32_t code) {
  if (code < LORA_OK || code > LORA_ERR_HIP) return "unknown lora_status";
  switch (static_cast<lora_status>(code)) {
    case LORA_OK: return "LORA_OK";
    case LORA_ERR_NULL: return "LORA_ERR_NULL: a required pointer is NULL";
    case LORA_ERR_SHAPE: return "LORA_ERR_SHAPE: M < 0, N or K not a positive multiple of 64, or a tensor too large";
    case LORA_ERR_RANK: return "LORA_ERR_RANK: R must be a multiple of 8 in [8, 64]";
    case LORA_ERR_ALIGN: return "LORA_ERR_ALIGN: a pointer is not 16-byte aligned";
    case LORA_ERR_DTYPE: return "LORA_ERR_DTYPE: unknown element type";
    case LORA_ERR_WORKSPACE: return "LORA_ERR_WORKSPACE: workspace missing or too small";
    case LORA_ERR_GROUP: return "LORA_ERR_GROUP: int4 group size must be 64";
    case LORA_ERR_VALUE: return "LORA_ERR_VALUE: scale must be finite";
    case LORA_ERR_HIP: return "LORA_ERR_HIP: a HIP launch failed";
  }
  return "unknown lora_status";
}

const char* lora_last_hip_error(void) { return g_last_hip_error; }

lora_status lora_fwd(int32_t dt, int64_t M, int64_t N, int64_t K, int32_t R, float scale,
                     const void* X, const void* W, const void* A, const void* B, void* Y, float* XA,
                     void* stream) {
  if (dt != LORA_F32 && dt != LORA_BF16) return LORA_ERR_DTYPE;
  lora_status st = check_dims(M, N, K, R);
  if (st != LORA_OK) return st;
  if (!std::isfinite(scale)) return LORA_ERR_VALUE;
  st = check_ptrs(W, A, B);
  if (st != LORA_OK) return st;
  if (M == 0) return LORA_OK;  // empty batch: X, Y and XA may be NULL
  st = check_ptrs(X, Y);
  if (st != LORA_OK) return st;
  if (XA != nullptr && !aligned16(XA)) return LORA_ERR_ALIGN;
  FwdArgs a{X, W, nullptr, A, B, Y, XA, M, N, K, R, scale};
  hipStream_t s = static_cast<hipStream_t>(stream);
  return from_hip(dt == LORA_F32 ? launch_fwd_f32(a, s) : launch_fwd_mfma(a, false, s));
}

size_t lora_bwd_workspace_bytes(int32_t dt, int64_t M, int64_t N, int64_t K, int32_t R) {
  if (dt != LORA_F32 && dt != LORA_BF16) return 0;
  if (check_dims(M, N, K, R) != LORA_OK) return 0;
  return bwd_layout(M, N, K, R, dt != LORA_F32).total;
}

lora_status lora_bwd(int32_t dt, int64_t M, int64_t N, int64_t K, int32_t R, float scale,
                     const void* dY, const void* X, const void* W, const void* A, const void* B,
                     const float* XA, void* dX, float* dA, float* dB, void* ws, size_t ws_bytes,
                     void* stream) {
  if (dt != LORA_F32 && dt != LORA_BF16) return LORA_ERR_DTYPE;
  lora_status st = check_dims(M, N, K, R);
  if (st != LORA_OK) return st;
  if (!std::isfinite(scale)) return LORA_ERR_VALUE;
  st = check_ptrs(W, A, B, dA, dB);
  if (st != LORA_OK) return st;
  if (M > 0 && (st = check_ptrs(dY, X, XA, dX)) != LORA_OK) return st;
  st = bwd_dx_common(false, static_cast<lora_dtype>(dt), M, N, K, R, scale, dY, W, nullptr, A, B, dX, ws, ws_bytes,
                     stream);
  if (st != LORA_OK) return st;
  return bwd_dadb_common(static_cast<lora_dtype>(dt), M, N, K, R, scale, dY, X, XA, dA, dB, ws, ws_bytes, stream);
}

lora_status lora_bwd_dx(int32_t dt, int64_t M, int64_t N, int64_t K, int32_t R, float scale,
                        const void* dY, const void* W, const void* A, const void* B, void* dX,
                        void* ws, size_t ws_bytes, void* stream) {
  if (dt != LORA_F32 && dt != LORA_BF16) return LORA_ERR_DTYPE;
  lora_status st = check_dims(M, N, K, R);
  if (st != LORA_OK) return st;
  if (!std::isfinite(scale)) return LORA_ERR_VALUE;
  st = check_ptrs(W, A, B);
  if (st != LORA_OK) return st;
  if (M > 0 && (st = check_ptrs(dY, dX)) != LORA_OK) return st;
  return bwd_dx_common(false, static_cast<lora_dtype>(dt), M, N, K, R, scale, dY, W, nullptr, A, B, dX, ws, ws_bytes,
                       stream);
}

lora_status lora_bwd_dadb(int32_t dt, int64_t M, int64_t N, int64_t K, int32_t R, float scale,
                          const void* dY, const void* X, const float* XA, float* dA, float* dB,
                          void* ws, size_t ws_bytes, void* stream) {
  if (dt != LORA_F32 && dt != LORA_BF16) return LORA_ERR_DTYPE;
  lora_status st = check_dims(M, N, K, R);
  if (st != LORA_OK) return st;
  if (!std::isfinite(scale)) return LORA_ERR_VALUE;
  st = check_ptrs(dA, dB);
  if (st != LORA_OK) return st;
  if (M > 0 && (st = check_ptrs(dY, X, XA)) != LORA_OK) return st;
  return bwd_dadb_common(static_cast<lora_dtype>(dt), M, N, K, R, scale, dY, X, XA, dA, dB, ws, ws_bytes, stream);
}

lora_status qlora_quantize(int64_t N, int64_t K, int32_t group, const float* W, uint8_t* Wq,
                           void* Ws, void* stream) {
  if (group != 64 && group != 32) return LORA_ERR_GROUP;
  if (N <= 0 || K <= 0 || K % 64 != 0 || N >= kMaxElems || K >= kMaxElems || N * K >= kMaxElems)
    return LORA_ERR_SHAPE;
  lora_status st = check_ptrs(W, Wq, Ws);
  if (st != LORA_OK) return st;
  if (group == 32)
    return from_hip(launch_quantize_mxfp4(N, K, W, Wq, static_cast<uint8_t*>(Ws), static_cast<hipStream_t>(stream)));
  return from_hip(launch_quantize_int4(N, K, W, Wq, static_cast<uint16_t*>(Ws),
                                       static_cast<hipStream_t>(stream)));
}

lora_status qlora_dequant(int64_t N, int64_t K, int32_t group, const uint8_t* Wq, const void* Ws,
                          void* W_bf16, void* stream) {
  if (group != 64 && group != 32) return LORA_ERR_GROUP;
  if (N <= 0 || K <= 0 || K % 64 != 0 || N >= kMaxElems || K >= kMaxElems || N * K >= kMaxElems)
    return LORA_ERR_SHAPE;
  lora_status st = check_ptrs(Wq, Ws, W_bf16);
  if (st != LORA_OK) return st;
  if (group == 32)
    return from_hip(launch_dequant_mxfp4(N, K, Wq, static_cast<const uint8_t*>(Ws), static_cast<uint16_t*>(W_bf16),
                                         static_cast<hipStream_t>(stream)));
  return from_hip(launch_dequant_int4(N, K, Wq, static_cast<const uint16_t*>(Ws),
                                      static_cast<uint16_t*>(W_bf16), static_cast<hipStream_t>(stream)));
}

size_t qlora_fwd_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t R) {
  if (check_dims(M, N, K, R) != LORA_OK) return 0;
  if (!use_gemv(M, K)) return 0;
  return gemv_workspace_bytes(M, N, K, R);
}

lora_status qlora_fwd(int64_t M, int64_t N, int64_t K, int32_t R, float scale, int32_t group,
                      const void* X, const uint8_t* Wq, const void* Ws, const void* A, const void* B,
                      void* Y, float* XA, void* ws, size_t ws_bytes, void* stream) {
  if (group != 64 && group != 32) return LORA_ERR_GROUP;
  lora_status st = check_dims(M, N, K, R);
  if (st != LORA_OK) return st;
  if (!std::isfinite(scale)) return LORA_ERR_VALUE;
  st = check_ptrs(Wq, Ws, A, B);
  if (st != LORA_OK) return st;
  if (M == 0) return LORA_OK;  // empty batch: X, Y and XA may be NULL
  st = check_ptrs(X, Y);
  if (st != LORA_OK) return st;
  if (XA != nullptr && !aligned16(XA)) return LORA_ERR_ALIGN;
  const size_t need = qlora_fwd_workspace_bytes(M, N, K, R);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return LORA_ERR_WORKSPACE;
  if (need > 0 && !aligned16(ws)) return LORA_ERR_ALIGN;
  FwdArgs a{X, Wq, Ws, A, B, Y, XA, M, N, K, R, scale};
  a.fp4 = group == 32;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (use_gemv(M, K)) return from_hip(a.fp4 ? launch_gemv_mxfp4(a, ws, s) : launch_gemv_int4(a, ws, s));
  return from_hip(launch_fwd_mfma(a, true, s));
}

size_t qlora_bwd_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t R) {
  if (check_dims(M, N, K, R) != LORA_OK) return 0;
  return bwd_layout(M, N, K, R, true).total;
}

lora_status qlora_bwd(int64_t M, int64_t N, int64_t K, int32_t R, float scale, int32_t group,
                      const void* dY, const void* X, const uint8_t* Wq, const void* Ws, const void* A,
                      const void* B, const float* XA, void* dX, float* dA, float* dB, void* ws,
                      size_t ws_bytes, void* stream) {
  if (group != 64 && group != 32) return LORA_ERR_GROUP;
  lora_status st = check_dims(M, N, K, R);
  if (st != LORA_OK) return st;
  if (!std::isfinite(scale)) return LORA_ERR_VALUE;
  st = check_ptrs(Wq, Ws, A, B, dA, dB);
  if (st != LORA_OK) return st;
  if (M > 0 && (st = check_ptrs(dY, X, XA, dX)) != LORA_OK) return st;
  st = bwd_dx_common(true, LORA_BF16, M, N, K, R, scale, dY, Wq, Ws, A, B, dX, ws, ws_bytes, stream, group == 32);
  if (st != LORA_OK) return st;
  return bwd_dadb_common(LORA_BF16, M, N, K, R, scale, dY, X, XA, dA, dB, ws, ws_bytes, stream);
}

lora_status qlora_bwd_dx(int64_t M, int64_t N, int64_t K, int32_t R, float scale, int32_t group,
                         const void* dY, const uint8_t* Wq, const void* Ws, const void* A,
                         const void* B, void* dX, void* ws, size_t ws_bytes, void* stream) {
  if (group != 64 && group != 32) return LORA_ERR_GROUP;
  lora_status st = check_dims(M, N, K, R);
  if (st != LORA_OK) return st;
  if (!std::isfinite(scale)) return LORA_ERR_VALUE;
  st = check_ptrs(Wq, Ws, A, B);
  if (st != LORA_OK) return st;
  if (M > 0 && (st = check_ptrs(dY, dX)) != LORA_OK) return st;
  return bwd_dx_common(true, LORA_BF16, M, N, K, R, scale, dY, Wq, Ws, A, B, dX, ws, ws_bytes, stream, group == 32);
}

size_t lora_swiglu_fwd_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t R) {
  if (check_swiglu(M, N, K, R) != LORA_OK) return 0;
  return swiglu_layout(M, N, K, R, false).total;
}

lora_status lora_swiglu_fwd(int64_t M, int64_t N, int64_t K, int32_t R, float scale, const void* X,
                            const void* Wgu, const void* Ag, const void* Au, const void* Bg, const void* Bu,
                            void* H, void* GU, float* XA, void* ws, size_t ws_bytes, void* stream) {
  return swiglu_fwd_impl(0, M, N, K, R, scale, X, Wgu, nullptr, Ag, Au, Bg, Bu, H, GU, XA, ws, ws_bytes, stream);
}

lora_status qlora_swiglu_fwd(int64_t M, int64_t N, int64_t K, int32_t R, float scale, int32_t group, const void* X,
                             const uint8_t* Wguq, const void* Wgus, const void* Ag, const void* Au, const void* Bg,
                             const void* Bu, void* H, void* GU, float* XA, void* ws, size_t ws_bytes, void* stream) {
  if (group != 64 && group != 32) return LORA_ERR_GROUP;
  if (Wgus == nullptr) return LORA_ERR_NULL;
  return swiglu_fwd_impl(group, M, N, K, R, scale, X, Wguq, Wgus, Ag, Au, Bg, Bu, H, GU, XA, ws, ws_bytes, stream);
}

size_t lora_swiglu_bwd_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t R) {
  if (check_swiglu(M, N, K, R) != LORA_OK) return 0;
  return swiglu_layout(M, N, K, R, true).total;
}

lora_status lora_swiglu_bwd(int64_t M, int64_t N, int64_t K, int32_t R, float scale, const void* dH,
                            const void* X, const void* Wgu, const void* Ag, const void* Au, const void* Bg,
                            const void* Bu, const void* GU, const float* XA, void* dX, float* dAg, float* dAu,
                            float* dBg, float* dBu, void* ws, size_t ws_bytes, void* stream) {
  return swiglu_bwd_impl(0, M, N, K, R, scale, dH, X, Wgu, nullptr, Ag, Au, Bg, Bu, GU, XA, dX, dAg, dAu, dBg, dBu,
                         ws, ws_bytes, stream);
}

lora_status qlora_swiglu_bwd(int64_t M, int64_t N, int64_t K, int32_t R, float scale, int32_t group, const void* dH,
                             const void* X, const uint8_t* Wguq, const void* Wgus, const void* Ag, const void* Au,
                             const void* Bg, const void* Bu, const void* GU, const float* XA, void* dX, float* dAg,
                             float* dAu, float* dBg, float* dBu, void* ws, size_t ws_bytes, void* stream) {
  if (group != 64 && group != 32) return LORA_ERR_GROUP;
  if (Wgus == nullptr) return LORA_ERR_NULL;
  return swiglu_bwd_impl(group, M, N, K, R, scale, dH, X, Wguq, Wgus, Ag, Au, Bg, Bu, GU, XA, dX, dAg, dAu, dBg, dBu,
                         ws, ws_bytes, stream);
}

}  // extern "C"

// ---- RMSNorm ahead of a projection ----

namespace {

lora_status check_norm(int64_t M, int64_t K) {
  if (M < 0 || M >= kMaxElems || K < 64 || K % 64 != 0 || K > kNormMaxK) return LORA_ERR_SHAPE;
  if (M * K >= kMaxElems) return LORA_ERR_SHAPE;
  return LORA_OK;
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

}  // namespace

extern "C" {

lora_status lora_rmsnorm_fwd(int64_t M, int64_t K, float eps, const void* X, const void* g, void* Y, float* r,
                             void* stream) {
  lora_status st = check_norm(M, K);
  if (st != LORA_OK) return st;
  if (!std::isfinite(eps) || eps < 0.f) return LORA_ERR_VALUE;
  st = check_ptrs(g);
  if (st != LORA_OK) return st;
  if (M == 0) return LORA_OK;  // empty batch: X, Y and r may be NULL
  st = check_ptrs(X, Y);
  if (st != LORA_OK) return st;
  if (r == nullptr) return LORA_ERR_NULL;
  if (!aligned4(r)) return LORA_ERR_ALIGN;
  return from_hip(launch_rmsnorm_fwd(static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(g),
                                     static_cast<uint16_t*>(Y), r, M, K, eps, static_cast<hipStream_t>(stream)));
}

size_t lora_rmsnorm_bwd_workspace_bytes(int64_t M, int64_t K) {
  if (check_norm(M, K) != LORA_OK) return 0;
  return rmsnorm_bwd_part_floats(M, K) * 4;
}

lora_status lora_rmsnorm_bwd(int64_t M, int64_t K, const void* dY, const void* X, const void* g, const float* r,
                             void* dX, float* dg, void* ws, size_t ws_bytes, void* stream) {
  lora_status st = check_norm(M, K);
  if (st != LORA_OK) return st;
  st = check_ptrs(g);
  if (st != LORA_OK) return st;
  if (dg != nullptr) {  // dg comes from per-workgroup partials in the workspace
    if (!aligned4(dg)) return LORA_ERR_ALIGN;
    if (M > 0 && (ws == nullptr || ws_bytes < lora_rmsnorm_bwd_workspace_bytes(M, K))) return LORA_ERR_WORKSPACE;
    if (ws != nullptr && !aligned16(ws)) return LORA_ERR_ALIGN;
  }
  if (M > 0) {  // empty batch: dY, X, r and dX may be NULL
    st = check_ptrs(dY, X, dX);
    if (st != LORA_OK) return st;
    if (r == nullptr) return LORA_ERR_NULL;
    if (!aligned4(r)) return LORA_ERR_ALIGN;
  }
  return from_hip(launch_rmsnorm_bwd(static_cast<const uint16_t*>(dY), static_cast<const uint16_t*>(X),
                                     static_cast<const uint16_t*>(g), r, static_cast<uint16_t*>(dX), dg,
                                     static_cast<float*>(ws), M, K, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---- MXFP4 weights and their decode product ----

extern "C" {

lora_status mxfp4_quantize(int64_t N, int64_t K, const float* W, uint8_t* Wq, uint8_t* We, void* stream) {
  if (N <= 0 || K <= 0 || K % 64 != 0 || N >= kMaxElems || K >= kMaxElems || N * K >= kMaxElems)
    return LORA_ERR_SHAPE;
  lora_status st = check_ptrs(W, Wq, We);
  if (st != LORA_OK) return st;
  return from_hip(launch_quantize_mxfp4(N, K, W, Wq, We, static_cast<hipStream_t>(stream)));
}

lora_status mxfp4_dequant(int64_t N, int64_t K, const uint8_t* Wq, const uint8_t* We, void* W_bf16, void* stream) {
  if (N <= 0 || K <= 0 || K % 64 != 0 || N >= kMaxElems || K >= kMaxElems || N * K >= kMaxElems)
    return LORA_ERR_SHAPE;
  lora_status st = check_ptrs(Wq, We, W_bf16);
  if (st != LORA_OK) return st;
  return from_hip(launch_dequant_mxfp4(N, K, Wq, We, static_cast<uint16_t*>(W_bf16),
                                       static_cast<hipStream_t>(stream)));
}

size_t mxfp4_decode_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t R) {
  if (check_dims(M, N, K, R) != LORA_OK || !use_gemv(M, K)) return 0;
  return gemv_workspace_bytes(M, N, K, R);
}

lora_status qlora_decode_status(void* ws, size_t ws_bytes, uint32_t* status, int32_t clear, void* stream) {
  if (ws == nullptr || status == nullptr) return LORA_ERR_NULL;
  if (!aligned16(ws)) return LORA_ERR_ALIGN;
  if (ws_bytes < kDecodeHeaderBytes) return LORA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* ctl = static_cast<uint32_t*>(ws);
  hipError_t e = hipMemcpyAsync(status, ctl + kDecodeStatusWord, 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess && clear) e = hipMemsetAsync(ws, 0, ws_bytes, s);  // the whole workspace
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return from_hip(e);
}

lora_status qlora_decode_set_hold(void* ws, size_t ws_bytes, int32_t hold, void* stream) {
  if (ws == nullptr) return LORA_ERR_NULL;
  if (!aligned16(ws)) return LORA_ERR_ALIGN;
  if (ws_bytes < kDecodeHeaderBytes) return LORA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint32_t v = hold != 0 ? 1u : 0u;
  hipError_t e = hipMemcpyAsync(static_cast<uint32_t*>(ws) + kDecodeHoldWord, &v, 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return from_hip(e);
}

lora_status mxfp4_decode_fwd(int64_t M, int64_t N, int64_t K, int32_t R, float scale, const void* X, const uint8_t* Wq,
                             const uint8_t* We, const void* A, const void* B, void* Y, float* XA, void* ws,
                             size_t ws_bytes, void* stream) {
  lora_status st = check_dims(M, N, K, R);
  if (st != LORA_OK) return st;
  if (M < 1 || M > 8 || K % 1024 != 0) return LORA_ERR_SHAPE;  // the decode shapes only
  if (!std::isfinite(scale)) return LORA_ERR_VALUE;
  st = check_ptrs(X, Wq, We, A, B, Y);
  if (st != LORA_OK) return st;
  if (XA != nullptr && !aligned16(XA)) return LORA_ERR_ALIGN;
  const size_t need = mxfp4_decode_workspace_bytes(M, N, K, R);
  if (ws == nullptr || ws_bytes < need) return LORA_ERR_WORKSPACE;
  if (!aligned16(ws)) return LORA_ERR_ALIGN;
  const FwdArgs a{X, Wq, We, A, B, Y, XA, M, N, K, R, scale};
  return from_hip(launch_gemv_mxfp4(a, ws, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---- Cross-entropy over an LM head, in chunks of tokens ----

namespace {

// The default chunk keeps its fp32 logits (4 bytes per token and vocabulary word) within this
// budget, in whole multiples of 256 tokens and never fewer than 256.
constexpr size_t kCeLogitsBudget = (size_t)512 << 20;
constexpr int64_t kCeChunkUnit = 256;
constexpr int32_t kCeRank = 8;  // the rank the shape checks take (the LM head has no adapter)

int64_t ce_default_chunk(int64_t V) {
  if (V <= 0) return kCeChunkUnit;
  const int64_t c = (int64_t)(kCeLogitsBudget / ((size_t)V * 4)) / kCeChunkUnit * kCeChunkUnit;
  return c < kCeChunkUnit ? kCeChunkUnit : c;
}

int64_t ce_chunk(int64_t M, int64_t V, int64_t chunk) {
  const int64_t c = chunk > 0 ? chunk : ce_default_chunk(V);
  return M < c ? (M > 0 ? M : 1) : c;
}

lora_status check_ce(int64_t M, int64_t V, int64_t K, int64_t chunk) {
  if (M < 0 || M >= kMaxElems || chunk < 0) return LORA_ERR_SHAPE;
  const int64_t C = ce_chunk(M, V, chunk);
  return check_dims(C, V, K, kCeRank);  // V and K multiples of 64; the chunk's C x V below 2^31
}

// Per chunk: the (max, sum of exp) pairs, label logits and lse of its rows; with the gradient also
// the chunk's fp32 logits as a high and a low 16-bit plane (the gradient of the logits is written
// over the high plane), and the input-gradient kernel's split counters and partials.
struct CeLayout {
  size_t stats, lab, lse, hi, lo, ctr, part, total;
};
// input-gradient scratch of a chunk of m tokens: per-tile arrival counters, split partials
size_t ce_dx_ctr_bytes(int64_t m, int64_t K) { return align256((size_t)dx_tiles(m, K) * 4); }
size_t ce_dx_part_bytes(int64_t m, int64_t V, int64_t K) { return align256(dx_part_bytes(m, V, K, 16)); }
CeLayout ce_layout(int64_t M, int64_t V, int64_t K, int64_t chunk, bool grad) {
  const int64_t C = ce_chunk(M, V, chunk);
  const int64_t P = 2 * ((V + 255) / 256);  // partials per row: one per wave's 128 columns
  CeLayout l{};
  l.stats = 0;
  l.lab = l.stats + align256((size_t)P * C * 8);
  l.lse = l.lab + align256((size_t)C * 4);
  l.total = l.lse + align256((size_t)C * 4);
  if (grad) {
    l.hi = l.total;
    l.lo = l.hi + align256((size_t)C * V * 2);
    l.ctr = l.lo + align256((size_t)C * V * 2);
    // the input-gradient scratch of a full chunk and of the last, shorter one (whose split of V
    // may differ)
    const int64_t tail = M % C;
    size_t ctr = ce_dx_ctr_bytes(C, K), part = ce_dx_part_bytes(C, V, K);
    if (tail > 0) {
      ctr = std::max(ctr, ce_dx_ctr_bytes(tail, K));
      part = std::max(part, ce_dx_part_bytes(tail, V, K));
    }
    l.part = l.ctr + ctr;
    l.total = l.part + part;
  }
  return l;
}

}  // namespace

extern "C" {

int64_t lora_ce_default_chunk(int64_t V) { return ce_default_chunk(V); }

size_t lora_ce_workspace_bytes(int64_t M, int64_t V, int64_t K, int64_t chunk, int32_t grad) {
  if (check_ce(M, V, K, chunk) != LORA_OK) return 0;
  return ce_layout(M, V, K, chunk, grad != 0).total;
}

lora_status lora_ce(int64_t M, int64_t V, int64_t K, int64_t chunk, float grad_scale, const void* X, const void* W,
                    const int32_t* labels, float* loss, float* loss_total, void* dX, void* ws, size_t ws_bytes,
                    void* stream) {
  lora_status st = check_ce(M, V, K, chunk);
  if (st != LORA_OK) return st;
  if (!std::isfinite(grad_scale)) return LORA_ERR_VALUE;
  st = check_ptrs(W);
  if (st != LORA_OK) return st;
  if (M > 0 && (st = check_ptrs(X, labels, loss)) != LORA_OK) return st;
  if (dX != nullptr && !aligned16(dX)) return LORA_ERR_ALIGN;
  if (loss_total != nullptr && !aligned16(loss_total)) return LORA_ERR_ALIGN;
  const bool grad = dX != nullptr;
  const CeLayout lay = ce_layout(M, V, K, chunk, grad);
  if (M > 0 && (ws == nullptr || ws_bytes < lay.total)) return LORA_ERR_WORKSPACE;
  if (ws != nullptr && !aligned16(ws)) return LORA_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  const int64_t C = ce_chunk(M, V, chunk);
  const int P = (int)(2 * ((V + 255) / 256));
  float* stats = reinterpret_cast<float*>(base + lay.stats);
  float* lab = reinterpret_cast<float*>(base + lay.lab);
  float* lse = reinterpret_cast<float*>(base + lay.lse);
  uint16_t* hi = grad ? reinterpret_cast<uint16_t*>(base + lay.hi) : nullptr;
  uint16_t* lo = grad ? reinterpret_cast<uint16_t*>(base + lay.lo) : nullptr;
  hipError_t e = hipSuccess;
  if (M > 0) {
    // a label outside [0, V) is never found: its slot keeps NaN and so does its loss (every
    // reduction puts NaN back for the next chunk)
    e = launch_fill_u32(lab, (size_t)C * 4, 0x7fc00000u, s);
    if (e != hipSuccess) return from_hip(e);
  }
  for (int64_t c0 = 0; c0 < M; c0 += C) {
    const int64_t Mc = (M - c0 < C) ? M - c0 : C;
    FwdArgs a{static_cast<const uint16_t*>(X) + c0 * K, W, nullptr, nullptr, nullptr, nullptr, nullptr, Mc, V, K,
              kCeRank, grad_scale};
    a.ce.labels = labels + c0;
    a.ce.stats = stats;
    a.ce.lab_logit = lab;
    a.ce.hi = hi;
    a.ce.lo = lo;
    e = launch_ce_logits(a, s);
    if (e != hipSuccess) return from_hip(e);
    e = launch_ce_reduce(stats, lab, lse, loss + c0, P, Mc, s);
    if (e != hipSuccess) return from_hip(e);
    if (!grad) continue;
    // dlogits = grad_scale (softmax - onehot) over the high plane, then dX = dlogits W
    e = launch_ce_grad(hi, lo, lse, labels + c0, Mc, V, grad_scale, s);
    if (e != hipSuccess) return from_hip(e);
    DxArgs d{hi, W, nullptr, nullptr, nullptr, static_cast<uint16_t*>(dX) + c0 * K, nullptr, Mc, V, K, kCeRank, 0.f,
             reinterpret_cast<uint32_t*>(base + lay.ctr), reinterpret_cast<float*>(base + lay.part)};
    e = launch_dx_noadapter(d, s);
    if (e != hipSuccess) return from_hip(e);
  }
  if (loss_total != nullptr) return from_hip(launch_ce_sum(loss, loss_total, M, grad_scale, s));
  return LORA_OK;
}

lora_status lora_ce_scale_grad(int64_t M, int64_t K, const float* g, const void* dX, void* out, void* stream) {
  if (M < 0 || K <= 0 || K % 8 != 0 || M >= kMaxElems || K >= kMaxElems || M * K >= kMaxElems) return LORA_ERR_SHAPE;
  if (g == nullptr) return LORA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(g) & 3u) != 0) return LORA_ERR_ALIGN;
  if (M == 0) return LORA_OK;
  const lora_status st = check_ptrs(dX, out);
  if (st != LORA_OK) return st;
  return from_hip(launch_scale_bf16(static_cast<const uint16_t*>(dX), static_cast<uint16_t*>(out), M * K, g,
                                    static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---- RoPE ----

extern "C" {

lora_status lora_rope(int64_t M, int32_t H, int32_t Hk, int32_t D, int32_t rot, float base, int32_t inverse,
                      const int32_t* positions, void* Q, void* K, void* stream) {
  if (M < 0 || M >= kMaxElems || H < 1 || Hk < 0 || D < 16 || D % 8 != 0 || D > 2 * kRopeMaxPairs) return LORA_ERR_SHAPE;
  if (rot < 16 || rot % 16 != 0 || rot > D) return LORA_ERR_SHAPE;
  if (M * (int64_t)(H + Hk) * D >= kMaxElems) return LORA_ERR_SHAPE;
  if (!std::isfinite(base) || base <= 1.f) return LORA_ERR_VALUE;
  if (M == 0) return LORA_OK;  // empty batch: every pointer may be NULL
  lora_status st = check_ptrs(Q);
  if (st != LORA_OK) return st;
  if (positions == nullptr) return LORA_ERR_NULL;
  if (Hk > 0 && (st = check_ptrs(K)) != LORA_OK) return st;
  return from_hip(launch_rope(static_cast<uint16_t*>(Q), static_cast<uint16_t*>(K), positions, M, H, Hk, D, rot,
                              base, inverse != 0, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---- Diagnostics ----

extern "C" {

lora_status lora_probe_sclk(uint64_t* out, uint32_t ticks, void* stream) {
  if (out == nullptr) return LORA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(out) & 7u) != 0) return LORA_ERR_ALIGN;
  if (ticks < 1 || ticks > 100000000u) return LORA_ERR_VALUE;
  return from_hip(launch_sclk_probe(reinterpret_cast<unsigned long long*>(out), ticks,
                                    static_cast<hipStream_t>(stream)));
}

lora_status lora_probe_mfma(uint64_t* out, int32_t blocks, uint32_t iters, void* stream) {
  if (out == nullptr) return LORA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(out) & 7u) != 0) return LORA_ERR_ALIGN;
  if (blocks < 1 || blocks > 65536 || iters < 1 || iters > 1000000u) return LORA_ERR_VALUE;
  return from_hip(launch_mfma_rate(reinterpret_cast<unsigned long long*>(out), blocks, iters,
                                   static_cast<hipStream_t>(stream)));
}

lora_status lora_probe_mfma_issue(uint64_t* out, int32_t blocks, uint32_t iters, int32_t mode, void* stream) {
  if (out == nullptr) return LORA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(out) & 7u) != 0) return LORA_ERR_ALIGN;
  if (blocks < 1 || blocks > 65536 || iters < 1 || iters > 1000000u || mode < 0 || mode > 7) return LORA_ERR_VALUE;
  return from_hip(launch_mfma_issue(reinterpret_cast<unsigned long long*>(out), blocks, iters, mode,
                                    static_cast<hipStream_t>(stream)));
}

lora_status lora_probe_hbm_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (buf == nullptr || sink == nullptr) return LORA_ERR_NULL;
  if (!aligned16(buf) || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0) return LORA_ERR_ALIGN;
  if (bytes == 0 || bytes % 16 != 0) return LORA_ERR_VALUE;
  return from_hip(launch_hbm_read(buf, bytes, sink, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---- The decode product without a caller workspace ----
//
// For callers that cannot allocate (code under graph capture, tight serving loops): the decode
// path's workspace lives in a file-scope device array, one copy per device, whose address is
// taken once per device with hipGetSymbolAddress (in host code the array's name is only a
// stand-in).  Every call clears the array's control words with a small fill kernel before the
// decode kernel, so nothing a previous call left there (even one whose bounded wait gave up) is
// read.  Calls that overlap in time on one device share the array and race.

namespace {

constexpr size_t kDecodeScratchBytes = (size_t)2 << 20;
constexpr int kMaxDevices = 64;

}  // namespace

__device__ __align__(256) uint8_t lora_decode_scratch[kDecodeScratchBytes];

namespace {

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// this device's copy of the array (resolved on the first call on the device, that device current)
lora_status decode_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return from_hip(e);
  if (dev < 0 || dev >= kMaxDevices) return LORA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(lora_decode_scratch));
    if (e != hipSuccess) return from_hip(e);
    if (p == nullptr) return LORA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LORA_OK;
}

}  // namespace

extern "C" {

lora_status qlora_decode_fwd_noalloc(int64_t M, int64_t N, int64_t K, int32_t R, float scale, int32_t group,
                                     const void* X, const uint8_t* Wq, const void* Ws, const void* A,
                                     const void* B, void* Y, float* XA, void* stream) {
  if (group != 64 && group != 32) return LORA_ERR_GROUP;
  lora_status st = check_dims(M, N, K, R);
  if (st != LORA_OK) return st;
  if (!use_gemv(M, K)) return LORA_ERR_SHAPE;  // the decode shapes only
  if (!std::isfinite(scale)) return LORA_ERR_VALUE;
  st = check_ptrs(X, Wq, Ws, A, B, Y);
  if (st != LORA_OK) return st;
  if (XA != nullptr && !aligned16(XA)) return LORA_ERR_ALIGN;
  if (gemv_workspace_bytes(M, N, K, R) > kDecodeScratchBytes) return LORA_ERR_WORKSPACE;
  void* ws = nullptr;
  st = decode_scratch(&ws);
  if (st != LORA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_fill_u32(ws, gemv_control_bytes(N), 0u, s);
  if (e != hipSuccess) return from_hip(e);
  FwdArgs a{X, Wq, Ws, A, B, Y, XA, M, N, K, R, scale};
  a.fp4 = group == 32;
  return from_hip(a.fp4 ? launch_gemv_mxfp4(a, ws, s) : launch_gemv_int4(a, ws, s));
}

}  // extern "C"
