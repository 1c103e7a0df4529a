// Host-side launchers of the gfx950 kernels (argument structs shared by the C ABI layer).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lora {

// Rows of tokens reduced by one split of the token-dimension (split-K) dA / dB sums on the fp32
// path, and the shortest split of the bf16 / int4 path (which may double it).
constexpr int64_t kSplitRows = 256;
constexpr int64_t kDadbCols = 256;  // columns (k or n) per workgroup of the dA / dB partial pass

// epilogues of the forward GEMM
constexpr int kEpiLora = 0, kEpiSwiglu = 1, kEpiCeStats = 2;

// cross-entropy epilogues over an LM head's logits
struct CeArgs {
  const int32_t* labels = nullptr;  // [M] in [0, N)
  float* stats = nullptr;           // [M][2 tiles_n] (max, sum of exp) per wave's 128 columns
  float* lab_logit = nullptr;       // [M] the label's logit
  uint16_t* hi = nullptr;           // [M][N] high 16 bits of the fp32 logits, or null
  uint16_t* lo = nullptr;           // [M][N] their low 16 bits
};

struct FwdArgs {
  const void* X;
  const void* W;   // bf16 [N][K], fp32 [N][K], or packed int4 [N][K/2]
  const void* Ws;  // fp16 scales [N][K/64] (int4 only)
  const void* A;
  const void* B;
  void* Y;
  float* XA;       // may be null
  int64_t M, N, K;
  int R;
  float scale;
  void* H = nullptr;  // SwiGLU pair (bf16 W = [Wg; Wu], N = 2 Nh): H = silu(G) U, M x Nh
  CeArgs ce = {};
  bool fp4 = false;   // 4-bit W is MXFP4 (E8M0 exponents in Ws) rather than int4 with fp16 scales
};

struct DxArgs {
  const void* dY;
  const void* W;
  const void* Ws;
  const void* A;
  const void* B;
  void* dX;
  float* G;        // [M][R] fp32: dY B, written for the dA reduction
  int64_t M, N, K;
  int R;
  float scale;
  uint32_t* ctr;   // split-N path (bf16 / int4): dx_tiles() arrival counters,
  float* part;     // and dx_part_bytes() bytes of split partials
  bool fp4 = false;  // 4-bit W is MXFP4 rather than int4
};

struct DadbArgs {
  const void* X;    // [M][K]
  const void* dY;   // [M][N]
  const float* G;   // [M][R]
  const float* XA;  // [M][R]
  float* partA;     // [splits][R][K]
  float* partB;     // [splits][R][N]
  float* dA;        // [R][K]
  float* dB;        // [N][R]
  int64_t M, N, K;
  int R;
  float scale;
  int splits;
  int split_rows;  // tokens per split (the last split may be shorter)
};

// diagnostics (diag.hip): shader clock, matrix-core rate, streaming-read rate
hipError_t launch_sclk_probe(unsigned long long* out, unsigned int ticks, hipStream_t s);
hipError_t launch_mfma_rate(unsigned long long* out, int blocks, unsigned int iters, hipStream_t s);
hipError_t launch_mfma_issue(unsigned long long* out, int blocks, unsigned int iters, int mode, hipStream_t s);
hipError_t launch_hbm_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s);

// compute units of the current device (the persistent MFMA kernels launch one workgroup per CU)
int device_cus();

// bf16 / int4 MFMA paths
hipError_t launch_fwd_mfma(const FwdArgs& a, bool int4, hipStream_t s);
hipError_t launch_ce_logits(const FwdArgs& a, hipStream_t s);
// cross-entropy reductions (ce.hip): lse and loss per row from the stats, their fixed-order sum,
// and a 32-bit fill
// (the reduction also sets the label-logit slots back to NaN for the next chunk)
hipError_t launch_ce_reduce(const float* stats, float* lab_logit, float* lse, float* loss, int P, int64_t M,
                            hipStream_t s);
// out[0] = scale x the fixed-order sum of loss
hipError_t launch_ce_sum(const float* loss, float* out, int64_t M, float scale, hipStream_t s);
// dlogits = bf16(scale (exp(logits - lse) - onehot(label))) from the stored fp32 logits (16-bit
// planes hi and lo), written over hi
hipError_t launch_ce_grad(uint16_t* hi, const uint16_t* lo, const float* lse, const int32_t* labels, int64_t M,
                          int64_t V, float scale, hipStream_t s);
// out = bf16(in x g[0]) over n bf16 values (g: one fp32 in device memory)
hipError_t launch_scale_bf16(const uint16_t* in, uint16_t* out, int64_t n, const float* g, hipStream_t s);
hipError_t launch_fill_u32(void* p, size_t bytes, uint32_t v, hipStream_t s);
hipError_t launch_dx_mfma(const DxArgs& a, bool int4, hipStream_t s);
// dX = dY W with no adapter (the LM head's gradient; bf16, rank-16 tiling of the split partials)
hipError_t launch_dx_noadapter(const DxArgs& a, hipStream_t s);
// ranks 33..64: G = dY B as a pass of its own (written to G), ahead of the input-gradient kernel,
// which then reads G in its epilogue; `ws` holds panel_workspace_bytes() bytes
int panel_shares(int64_t M, int64_t C);
size_t panel_workspace_bytes(int64_t M, int64_t N, int R);
hipError_t launch_panel_g(const uint16_t* dY, const uint16_t* B, float* G, void* ws, int64_t M, int64_t N,
                          int R, hipStream_t s);
// ranks 33..64 of a forward that keeps XA: XA = X A^T as a pass of its own, its partials in
// `scratch` (the forward's Y, overwritten afterwards)
hipError_t launch_panel_xa(const uint16_t* X, const uint16_t* A, float* XA, void* scratch, size_t scratch_bytes,
                           int64_t M, int64_t K, int R, hipStream_t s);
// Bytes of one split partial of the input-gradient kernel: its 256 x 256 fp32 tile in MFMA
// fragment order (4 waves x 64 blocks x 1 KB) and, for ranks up to 32, its G panel.
constexpr size_t dx_slot_bytes(int rp) {
  return (size_t)4 * 64 * 64 * 16 + (rp <= 32 ? (size_t)4 * (rp / 16) * 4 * 64 * 16 : 0);
}
// input-gradient grid: output tiles, N ranges per tile, bytes of split partials (0 if unsplit)
int dx_tiles(int64_t M, int64_t K);
int dx_splits(int64_t M, int64_t N, int64_t K, int R);
int dx_split_hi(int64_t M, int64_t N, int64_t K, int R);
size_t dx_part_bytes(int64_t M, int64_t N, int64_t K, int R);
hipError_t launch_dadb_partials_bf16(const DadbArgs& a, hipStream_t s);
// RMSNorm ahead of a projection: forward (Y, reciprocal RMS r) and backward (dX, optional dg
// from per-workgroup partials and their slice sums in `part`, rmsnorm_bwd_part_floats() fp32)
constexpr int kNormCUs = 256;         // MI355X compute units: the persistent grids' unit
constexpr int64_t kNormMaxK = 16384;  // the forward holds a row in registers: 32 chunks per lane
int rmsnorm_bwd_grid(int64_t M, int64_t K, bool dg);
size_t rmsnorm_bwd_part_floats(int64_t M, int64_t K);
hipError_t launch_rmsnorm_fwd(const uint16_t* X, const uint16_t* g, uint16_t* Y, float* r, int64_t M, int64_t K,
                              float eps, hipStream_t s);
hipError_t launch_rmsnorm_bwd(const uint16_t* dY, const uint16_t* X, const uint16_t* g, const float* r, uint16_t* dX,
                              float* dg, float* part, int64_t M, int64_t K, hipStream_t s);

// RoPE in place on Q (M x H x D) and K (M x Hk x D), bf16; rot/2 <= kRopeMaxPairs
constexpr int kRopeMaxPairs = 512;
hipError_t launch_rope(uint16_t* Q, uint16_t* K, const int32_t* pos, int64_t M, int H, int Hk, int D, int rot,
                       float base, bool inverse, hipStream_t s);

// SwiGLU gate/up pair over the stacked weight [Wg; Wu]: stacked adapters, activation, upstream
// gradient of the stacked GEMM, and the split of the stacked adapter gradients
hipError_t launch_swiglu_stack(const uint16_t* Ag, const uint16_t* Au, const uint16_t* Bg, const uint16_t* Bu,
                               uint16_t* As, uint16_t* Bs, int64_t N, int64_t K, int R, hipStream_t s);
hipError_t launch_swiglu_bwd(const uint16_t* dH, const uint16_t* GU, uint16_t* dGU, int64_t M, int64_t N,
                             hipStream_t s);
hipError_t launch_swiglu_unstack(const float* dAs, const float* dBs, float* dAg, float* dAu, float* dBg,
                                 float* dBu, int64_t N, int64_t K, int R, hipStream_t s);
// fp32 paths
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s);
hipError_t launch_dx_f32(const DxArgs& a, hipStream_t s);
hipError_t launch_dadb_partials_f32(const DadbArgs& a, hipStream_t s);
// fixed-order reduction of the partials into dA and dB (any element type)
hipError_t launch_dadb_reduce(const DadbArgs& a, hipStream_t s);
// int4 utilities and the small-M matrix-vector path
hipError_t launch_quantize_int4(int64_t N, int64_t K, const float* W, uint8_t* Wq, uint16_t* Ws,
                                hipStream_t s);
hipError_t launch_dequant_int4(int64_t N, int64_t K, const uint8_t* Wq, const uint16_t* Ws,
                               uint16_t* Wout, hipStream_t s);
// decode path (M <= 8): `ws` holds gemv_workspace_bytes() bytes: a 16-byte header (status word,
// hold word) and then the per-tile arrival counters, ready tokens and the adapter counter, all zero
// before the first call and left zero by every call that completes normally
hipError_t launch_gemv_int4(const FwdArgs& a, void* ws, hipStream_t s);
constexpr int kDecodeStatusWord = 0, kDecodeHoldWord = 1;
constexpr size_t kDecodeHeaderBytes = 16;
// MXFP4 weights: codes (N x K/2 bytes, int4 nibble layout) and E8M0 block exponents (N x K/32
// bytes); the decode product takes them in a.W and a.Ws
hipError_t launch_quantize_mxfp4(int64_t N, int64_t K, const float* W, uint8_t* Wq, uint8_t* We, hipStream_t s);
hipError_t launch_dequant_mxfp4(int64_t N, int64_t K, const uint8_t* Wq, const uint8_t* We, uint16_t* Wout,
                                hipStream_t s);
hipError_t launch_gemv_mxfp4(const FwdArgs& a, void* ws, hipStream_t s);
size_t gemv_workspace_bytes(int64_t M, int64_t N, int64_t K, int R);
// leading bytes of that workspace holding the header and control words (zero between calls)
size_t gemv_control_bytes(int64_t N);

}  // namespace lora
