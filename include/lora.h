/*
 * lora.h - C ABI of the MI355X (gfx950) fused LoRA / QLoRA linear layer.
 *
 * The layer (tutorial ch. 5 "加速原理：Triton kernel 与 fused LoRA", §5.3, LoRA equation;
 * tutorial ch. 1 "项目背景与定位", §1.2, Delta W = (alpha/r) B A), written for row-major
 * batches of tokens:
 *
 *     XA = X A^T                       (M x R, the rank-R panel, saved for backward)
 *     Y  = X W^T + scale * XA B^T      (M x N)
 *
 * and its backward with W frozen (§5.3, the paragraph on the fused backward; gradients
 * derived by hand for the loss convention dL/dY = dY):
 *
 *     G  = dY B                        (M x R)
 *     dX = dY W + scale * G A          (M x K)
 *     dA = scale * G^T X               (R x K)
 *     dB = scale * dY^T XA             (N x R)
 *
 * QLoRA ("探微索隐：Unsloth 如何加速 LLM 推理？（以 Qwen 27B 为例）", §二.3): W is held as
 * symmetric int4 codes in -7..7, two per byte (even k in the low nibble, 4-bit two's
 * complement), in groups of 64 consecutive k that share one fp16 scale (absmax / 7).  The
 * kernels read the packed bytes and unpack them in registers:
 *     W~[n][k] = bf16_rne( q[n][k] * scale16[n][k/64] )
 * and use W~ in the formulas above.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Shapes: X M x K, W N x K (out x in), A R x K, B N x R, Y and dY M x N, dX M x K,
 *    XA and G M x R, dA R x K, dB N x R.  All tensors are dense row-major with no strides.
 *  - Sizes: M >= 0 (M == 0 is a valid empty batch); N and K positive multiples of 64;
 *    N and K at most 2^20; R a multiple of 8 in [8, 64]; every tensor below 2^31 elements.
 *  - Pointers are device pointers owned by the caller, 16-byte aligned, and outputs must
 *    not alias inputs.  The library allocates and frees nothing and keeps no state
 *    between calls; scratch memory comes from the caller's workspace.
 *  - `stream` is a hipStream_t (NULL for the null stream).  Work is enqueued on it and
 *    the call returns without synchronising; faults during execution surface at the
 *    caller's next synchronisation.
 *  - Arguments are validated before any HIP call; an invalid call returns an error code
 *    and leaves every output untouched.  A failed launch returns LORA_ERR_HIP.
 *  - `scale` is alpha / r, computed by the caller.
 *  - Outputs are overwritten, never accumulated into.
 *  - Results are deterministic: every reduction adds its terms in a fixed order (no
 *    floating-point atomics), so two identical calls give bitwise identical outputs.
 */
#ifndef LORA_MI355X_H
#define LORA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lora_status {
  LORA_OK = 0,
  LORA_ERR_NULL = 1,      /* a required pointer is NULL */
  LORA_ERR_SHAPE = 2,     /* M < 0, N or K not a positive multiple of 64, or a tensor too large */
  LORA_ERR_RANK = 3,      /* R not a multiple of 8 in [8, 64] */
  LORA_ERR_ALIGN = 4,     /* a pointer is not 16-byte aligned */
  LORA_ERR_DTYPE = 5,     /* unknown element type */
  LORA_ERR_WORKSPACE = 6, /* workspace NULL or smaller than the matching *_workspace_bytes() */
  LORA_ERR_GROUP = 7,     /* 4-bit group other than 64 (int4) or 32 (MXFP4) */
  LORA_ERR_VALUE = 8,     /* scale not finite, or eps not finite and >= 0 */
  LORA_ERR_HIP = 9        /* a HIP launch failed; lora_last_hip_error() names it */
} lora_status;

/* Element type of X, W, A, B, Y, dY and dX.  dA, dB, XA and G are always fp32.  The entry points
 * take it as an int32_t `dt` holding one of these values (any other value is LORA_ERR_DTYPE). */
typedef enum lora_dtype { LORA_F32 = 0, LORA_BF16 = 1 } lora_dtype;

/* Forward: Y = X W^T + scale (X A^T) B^T  (tutorial ch. 5, §5.3: one kernel per output tile
 * that adds the low-rank term in its epilogue, so no intermediate reaches HBM).
 *   X  [M][K], W [N][K], A [R][K], B [N][R]  of type `dt`     (inputs)
 *   Y  [M][N] of type `dt`                                     (output)
 *   XA [M][R] fp32, unscaled X A^T, or NULL to skip saving it   (output)
 * For R > 32 (bf16) with XA given, X A^T is computed by a pass of its own ahead of the main
 * kernel, which parks its partial sums in Y before overwriting Y; with XA NULL the main
 * kernel computes it (correct, but slower at that rank). */
lora_status lora_fwd(int32_t dt, int64_t M, int64_t N, int64_t K, int32_t R, float scale,
                     const void* X, const void* W, const void* A, const void* B,
                     void* Y, float* XA, void* stream);

/* Bytes of device workspace lora_bwd needs for these sizes: G; the partial sums of dA and dB,
 * one per split of the tokens (256 tokens per split for fp32; for bf16, 256 doubled while the
 * partial pass keeps at least 512 workgroups, one per 256 columns of K + N per split, and at
 * most 2048); for bf16, the input gradient's split partials (when its output has few tiles);
 * and, for R > 32, the scratch of its G = dY B pass.  The workspace needs no initialisation:
 * calls clear what they use. */
size_t lora_bwd_workspace_bytes(int32_t dt, int64_t M, int64_t N, int64_t K, int32_t R);

/* Backward with W frozen (tutorial ch. 5, §5.3, fused backward; hand-derived gradients):
 *   dX = dY W + scale (dY B) A,  dA = scale (dY B)^T X,  dB = scale dY^T XA.
 *   dY [M][N], X [M][K], W [N][K], A [R][K], B [N][R] of type `dt`   (inputs)
 *   XA [M][R] fp32 as saved by lora_fwd                             (input)
 *   dX [M][K] of type `dt`; dA [R][K] fp32; dB [N][R] fp32           (outputs)
 *   ws: device workspace of at least lora_bwd_workspace_bytes() bytes. */
lora_status lora_bwd(int32_t dt, int64_t M, int64_t N, int64_t K, int32_t R, float scale,
                     const void* dY, const void* X, const void* W, const void* A, const void* B,
                     const float* XA, void* dX, float* dA, float* dB,
                     void* ws, size_t ws_bytes, void* stream);

/* The backward in two halves (lora_bwd = lora_bwd_dx then lora_bwd_dadb on the same workspace):
 * the input gradient, which the previous layer waits for, and the adapter gradients, which can
 * be deferred (e.g. overlapped with the previous layer's input gradient).
 *   lora_bwd_dx:   dX = dY W + scale (dY B) A; also writes G = dY B (fp32 M x R) into `ws`.
 *   lora_bwd_dadb: dA = scale G^T X, dB = scale dY^T XA, reading G from `ws` as left there by
 *                  lora_bwd_dx (or qlora_bwd_dx) with the same sizes.
 * Same argument meanings and workspace size as lora_bwd.  lora_bwd_dadb takes dt = LORA_BF16 for
 * the QLoRA path (its activations are bf16). */
lora_status lora_bwd_dx(int32_t dt, int64_t M, int64_t N, int64_t K, int32_t R, float scale,
                        const void* dY, const void* W, const void* A, const void* B, void* dX,
                        void* ws, size_t ws_bytes, void* stream);
lora_status lora_bwd_dadb(int32_t dt, int64_t M, int64_t N, int64_t K, int32_t R, float scale,
                          const void* dY, const void* X, const float* XA, float* dA, float* dB,
                          void* ws, size_t ws_bytes, void* stream);

/* int4 quantise + pack of an fp32 weight ("探微索隐 ...", §二.3 names the 4-bit store and its
 * scaling coefficient; the exact format is given at the top of this header).
 *   W  [N][K] fp32                        (input)
 *   Wq [N][K/2] bytes, Ws [N][K/group] fp16 (outputs)
 * group must be 64.  Codes are decided exactly (ties to even on the exact quotient).
 * group = 32 selects the MXFP4 format instead (see mxfp4_quantize: E2M1 codes in the same nibble
 * layout, Ws = N x K/32 E8M0 exponent bytes) in qlora_quantize, qlora_dequant, qlora_fwd,
 * qlora_bwd and qlora_bwd_dx: QLoRA training and inference with FP4 weights, unpacked in
 * registers by the gfx950 scaled FP4 conversion. */
lora_status qlora_quantize(int64_t N, int64_t K, int32_t group, const float* W,
                           uint8_t* Wq, void* Ws, void* stream);

/* The dequantised weight W~ [N][K] as bf16 (the unpack routine the QLoRA kernels use). */
lora_status qlora_dequant(int64_t N, int64_t K, int32_t group, const uint8_t* Wq, const void* Ws,
                          void* W_bf16, void* stream);

/* Bytes of device workspace qlora_fwd needs: 0 unless 1 <= M <= 8 and K % 1024 == 0.  For that
 * (decode) path: a 16-byte header (a status word and a test hold word), the per-tile arrival
 * counters and ready tokens and an adapter counter (u32, 2 N/64 + 1 of them), then the fp32 partial
 * sums.  The header and the counters must be zero before the first call that uses the workspace
 * (allocate it zeroed, or clear it with qlora_decode_status); every call that completes normally
 * leaves them zero, so a workspace serves later calls of any M without clearing.  Two calls that
 * overlap in time must not share a workspace. */
size_t qlora_fwd_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t R);

/* QLoRA forward: Y = X W~^T + scale (X A^T) B^T with W~ unpacked in registers.  For M <= 8
 * and K a multiple of 1024 it runs as one HBM-bandwidth-bound matrix-vector kernel (per generated
 * token every weight byte is streamed once: "探微索隐 ...", §一, the memory wall of decoding): its
 * first workgroups compute X A^T and announce it to the tile workgroups, which wait for it a bounded
 * time (about a second); partial sums are added in a fixed order, so results do not depend on
 * timing.  If a wait gives up (e.g. when other work keeps the announcing workgroups off the
 * device), the tile's Y is written as NaN and the workspace's status word is set; from then on every
 * call on that workspace writes NaN until qlora_decode_status clears it.
 *   X [M][K], A [R][K], B [N][R] bf16; Wq [N][K/2]; Ws [N][K/64] fp16   (inputs)
 *   Y [M][N] bf16; XA [M][R] fp32 or NULL                               (outputs)
 *   ws: at least qlora_fwd_workspace_bytes() bytes (may be NULL when that is 0). */
lora_status qlora_fwd(int64_t M, int64_t N, int64_t K, int32_t R, float scale, int32_t group,
                      const void* X, const uint8_t* Wq, const void* Ws,
                      const void* A, const void* B, void* Y, float* XA,
                      void* ws, size_t ws_bytes, void* stream);

/* Status of a decode workspace (the M <= 8 path of qlora_fwd and mxfp4_decode_fwd): waits for the
 * stream, writes the status word to *status (0: every call completed normally; 1: a bounded wait
 * gave up, and that call's outputs and those of every later call were written as NaN) and, with
 * clear != 0, zeroes the whole workspace (ws_bytes) so it can be used again.  Synchronises
 * `stream`; not for use inside graph capture.  Errors: LORA_ERR_NULL, LORA_ERR_ALIGN,
 * LORA_ERR_WORKSPACE (fewer than 16 bytes), LORA_ERR_HIP. */
lora_status qlora_decode_status(void* ws, size_t ws_bytes, uint32_t* status, int32_t clear, void* stream);

/* Test hook for the decode path's failure handling: with hold != 0, calls on this workspace do not
 * announce X A^T to the tile workgroups, so their bounded waits give up (after about a second) and
 * the call reports it as above.  Synchronises `stream`. */
lora_status qlora_decode_set_hold(void* ws, size_t ws_bytes, int32_t hold, void* stream);

/* The decode path of qlora_fwd (1 <= M <= 8, K a multiple of 1024; group 64: int4, group 32:
 * MXFP4) for callers that cannot allocate: code under graph capture, tight serving loops,
 * harnesses that forbid allocation.  It takes no workspace: its scratch is a static device array
 * of 2 MiB per device (kept until the process ends), which the call clears (control words only, by
 * a small kernel) before the decode kernel runs; it calls no allocating routine.  Same arguments
 * and results as qlora_fwd otherwise (Y bitwise equal to qlora_fwd's for the same inputs).  Shapes
 * whose decode workspace (qlora_fwd_workspace_bytes) exceeds 2 MiB return LORA_ERR_WORKSPACE (at
 * M = 8 and rank 64 that is N above about 63000); non-decode shapes return LORA_ERR_SHAPE.  Calls on one device
 * share the array: two calls that overlap in time (e.g. on two streams) race.  A call whose bounded
 * wait gave up writes NaN (no status word is kept here; the next call starts clean). */
lora_status qlora_decode_fwd_noalloc(int64_t M, int64_t N, int64_t K, int32_t R, float scale, int32_t group,
                                     const void* X, const uint8_t* Wq, const void* Ws, const void* A,
                                     const void* B, void* Y, float* XA, void* stream);

/* Bytes of device workspace qlora_bwd needs. */
size_t qlora_bwd_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t R);

/* QLoRA backward: as lora_bwd with W := W~ unpacked in registers.  All of dY, X, A, B and
 * dX are bf16; dA, dB fp32. */
lora_status qlora_bwd(int64_t M, int64_t N, int64_t K, int32_t R, float scale, int32_t group,
                      const void* dY, const void* X, const uint8_t* Wq, const void* Ws,
                      const void* A, const void* B, const float* XA,
                      void* dX, float* dA, float* dB,
                      void* ws, size_t ws_bytes, void* stream);

/* qlora_bwd's input-gradient half (W := W~ unpacked in registers); pair with lora_bwd_dadb. */
lora_status qlora_bwd_dx(int64_t M, int64_t N, int64_t K, int32_t R, float scale, int32_t group,
                         const void* dY, const uint8_t* Wq, const void* Ws, const void* A,
                         const void* B, void* dX, void* ws, size_t ws_bytes, void* stream);

/* ---- SwiGLU gate/up pair with LoRA on both projections ----------------------------------
 * Tutorial ch. 5 §5.6 ("fused SwiGLU": SwiGLU(x) = (W_g x ⊙ sigmoid(W_g x)) ⊙ W_u x, the gate's
 * SiLU and the product with the up projection; the output projection W_d is a plain lora_fwd
 * layer) with §5.3's LoRA update on the gate and on the up projection:
 *   G = X Wg^T + scale (X Ag^T) Bg^T,  U = X Wu^T + scale (X Au^T) Bu^T,  H = silu(G) ⊙ U,
 *   silu(g) = g sigmoid(g).
 * bf16 tensors, row-major, 16-byte aligned: X (M x K); Wgu (2N x K): the frozen gate and up
 * weights stacked by rows, [Wg; Wu]; Ag, Au (R x K); Bg, Bu (N x R); R a multiple of 8 in
 * [8, 32]; N, K multiples of 64.  The two projections run as one LoRA GEMM over Wgu (each X
 * tile read once for both) at rank 2R with the adapters stacked as [Ag; Au] and
 * [Bg 0; 0 Bu], which the call assembles in its workspace.
 * Errors as for lora_fwd / lora_bwd; the workspace needs no initialisation. */

/* Bytes of device workspace lora_swiglu_fwd needs (the stacked adapters). */
size_t lora_swiglu_fwd_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t R);

/* Forward.  Outputs: H (M x N bf16); GU (M x 2N bf16) = [G | U], G in columns 0..N-1 and U in
 * N..2N-1, kept for the backward; XA (M x 2R fp32) = [X Ag^T | X Au^T], unscaled, kept for the
 * backward (may be NULL for inference).  H is formed in the GEMM's epilogue from the fp32 G and
 * U (sigmoid from the hardware exp2 and reciprocal) and rounded to bf16 once, as are G and U.
 * M = 0 is an empty batch. */
lora_status lora_swiglu_fwd(int64_t M, int64_t N, int64_t K, int32_t R, float scale,
                            const void* X, const void* Wgu, const void* Ag, const void* Au,
                            const void* Bg, const void* Bu, void* H, void* GU, float* XA,
                            void* ws, size_t ws_bytes, void* stream);

/* Bytes of device workspace lora_swiglu_bwd needs. */
size_t lora_swiglu_bwd_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t R);

/* Backward with Wg, Wu frozen (hand-derived from L = <dH, H>): from the saved GU,
 *   dU = dH ⊙ silu(G),  dG = dH ⊙ U ⊙ silu'(G),  silu'(g) = sigmoid(g) (1 + g (1 - sigmoid(g))),
 * then the LoRA backward of each projection: dX = dG Wg + dU Wu + scale ((dG Bg) Ag + (dU Bu) Au),
 * dAg = scale (dG Bg)^T X, dAu likewise, dBg = scale dG^T (X Ag^T), dBu likewise.  dH, X, GU
 * and dX bf16; XA (M x 2R fp32) from the forward; dAg, dAu (R x K) and dBg, dBu (N x R) fp32,
 * overwritten. */
lora_status lora_swiglu_bwd(int64_t M, int64_t N, int64_t K, int32_t R, float scale,
                            const void* dH, const void* X, const void* Wgu, const void* Ag,
                            const void* Au, const void* Bg, const void* Bu, const void* GU,
                            const float* XA, void* dX, float* dAg, float* dAu, float* dBg,
                            float* dBu, void* ws, size_t ws_bytes, void* stream);

/* The SwiGLU pair with the frozen stacked weight [Wg; Wu] in 4 bits (QLoRA): group 64, int4 codes
 * with fp16 scales (Wgus: 2N x K/64); group 32, MXFP4 codes with E8M0 bytes (Wgus: 2N x K/32);
 * Wguq: 2N x K/2 bytes, as qlora_quantize writes for the 2N x K fp32 stacked weight.  Otherwise
 * as lora_swiglu_fwd / lora_swiglu_bwd, with the same workspace sizes; the codes are unpacked in
 * registers on their way to the matrix cores.  Errors: also LORA_ERR_GROUP. */
lora_status qlora_swiglu_fwd(int64_t M, int64_t N, int64_t K, int32_t R, float scale,
                             int32_t group, const void* X, const uint8_t* Wguq, const void* Wgus,
                             const void* Ag, const void* Au, const void* Bg, const void* Bu, void* H,
                             void* GU, float* XA, void* ws, size_t ws_bytes, void* stream);
lora_status qlora_swiglu_bwd(int64_t M, int64_t N, int64_t K, int32_t R, float scale,
                             int32_t group, const void* dH, const void* X, const uint8_t* Wguq,
                             const void* Wgus, const void* Ag, const void* Au, const void* Bg,
                             const void* Bu, const void* GU, const float* XA, void* dX, float* dAg,
                             float* dAu, float* dBg, float* dBu, void* ws, size_t ws_bytes,
                             void* stream);

/* ---- RMSNorm ahead of a projection ------------------------------------------------------
 * Tutorial ch. 5 §5.4 (fused RMSNorm: the mean square of each row, eps, the root and the
 * per-feature scale g in one kernel that reads and writes the hidden state once):
 *   r[m] = 1 / sqrt((1/K) sum_k X[m][k]^2 + eps),   Y[m][k] = X[m][k] r[m] g[k].
 * Y is the X of the following lora_fwd / qlora_fwd / lora_swiglu_fwd, and of their backward
 * (dA needs it), so the caller keeps it.  X, Y (M x K) and g (K) bf16, r (M) fp32; K a multiple
 * of 64 in [64, 16384]; M >= 0; eps finite and >= 0 (with eps = 0 an all-zero row gives
 * non-finite output, as the formula does).  Sums and products in fp32, Y rounded to bf16 once.
 * X, Y, g 16-byte aligned; r 4-byte aligned.  Errors: LORA_ERR_SHAPE, LORA_ERR_VALUE (eps),
 * LORA_ERR_NULL, LORA_ERR_ALIGN, LORA_ERR_HIP.  M = 0 is an empty batch (X, Y, r may be NULL). */
lora_status lora_rmsnorm_fwd(int64_t M, int64_t K, float eps, const void* X, const void* g,
                             void* Y, float* r, void* stream);

/* Bytes of device workspace lora_rmsnorm_bwd needs when it computes dg (the per-workgroup dg
 * partials); none is needed without dg. */
size_t lora_rmsnorm_bwd_workspace_bytes(int64_t M, int64_t K);

/* Backward, hand-derived from L = <dY, Y> with xh = X r (r from the forward):
 *   dX[m][j] = r[m] (g[j] dY[m][j] - xh[m][j] c[m]),  c[m] = (1/K) sum_k g[k] dY[m][k] xh[m][k],
 *   dg[k]    = sum_m dY[m][k] xh[m][k].
 * dY, X, dX (M x K) and g bf16; r (M) fp32 as the forward wrote it; dg (K) fp32, overwritten, or
 * NULL when g is frozen (the LoRA / QLoRA case; then ws may be NULL).  With dg the workspace
 * holds lora_rmsnorm_bwd_workspace_bytes(M, K) bytes (16-byte aligned, no initialisation) and
 * the partials are added in a fixed order.  M = 0 gives dg = 0. */
lora_status lora_rmsnorm_bwd(int64_t M, int64_t K, const void* dY, const void* X, const void* g,
                             const float* r, void* dX, float* dg, void* ws, size_t ws_bytes,
                             void* stream);

/* ---- MXFP4 weights (decode) ---------------------------------------------------------------
 * "探微索隐：Unsloth 如何加速 LLM 推理？（以 Qwen 27B 为例）", §二.3 names FP4 beside INT4 for the
 * 4-bit weights streamed in decode.  The format is the OCP Microscaling FP4: 32 consecutive k of a
 * row share a scale 2^(E-127) stored as one byte E (E8M0); each element is a 4-bit E2M1 code (sign
 * bit 3, exponent bits 2..1 with bias 1, mantissa bit 0; exponent 0 is subnormal: m/2), two per
 * byte with even k in the low nibble.
 *   Wq: N x K/2 bytes of codes;  We: N x K/32 bytes of E;  W~[n][k] = e2m1(code) * 2^(E - 127)
 * (exact in bf16).  Bytes per weight: 0.5 + 1/32, as for the int4 format. */

/* Quantise an fp32 weight (N x K, K a multiple of 64, finite values): per block of 32,
 * se = floor(log2(absmax)) - 2 clamped to [-125, 125] (0 for a zero block), E = se + 127; each
 * |w| / 2^se is rounded to the nearest E2M1 magnitude {0, 1/2, 1, 3/2, 2, 3, 4, 6}, ties to the
 * one with mantissa bit 0 and values past 6 to 6, decided exactly; the sign bit is set for w < 0.
 * W, Wq, We 16-byte aligned.  Errors: LORA_ERR_SHAPE, LORA_ERR_NULL, LORA_ERR_ALIGN, LORA_ERR_HIP. */
lora_status mxfp4_quantize(int64_t N, int64_t K, const float* W, uint8_t* Wq, uint8_t* We,
                           void* stream);

/* W~ (N x K bf16) from the codes and exponents; E is read as 2^(E - 127) for E in 1..254. */
lora_status mxfp4_dequant(int64_t N, int64_t K, const uint8_t* Wq, const uint8_t* We, void* W_bf16,
                          void* stream);

/* Bytes of device workspace mxfp4_decode_fwd needs (0 outside its shapes); the same layout and
 * rules as qlora_fwd's decode path (control block zero before the first call, left zero by every
 * call that completes normally, status and clearing through qlora_decode_status). */
size_t mxfp4_decode_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t R);

/* Decode forward with the MXFP4 weight: Y = X W~^T + scale (X A^T) B^T for 1 <= M <= 8 tokens and
 * K a multiple of 1024 (other shapes: LORA_ERR_SHAPE), in the one-kernel decode product of
 * qlora_fwd with the E2M1 codes unpacked by the gfx950 scaled conversion.  X (M x K), A, B, Y
 * bf16; XA (M x R fp32, unscaled) may be NULL. */
lora_status mxfp4_decode_fwd(int64_t M, int64_t N, int64_t K, int32_t R, float scale,
                             const void* X, const uint8_t* Wq, const uint8_t* We, const void* A,
                             const void* B, void* Y, float* XA, void* ws, size_t ws_bytes,
                             void* stream);

/* ---- Cross-entropy over an LM head, in chunks of tokens ----------------------------------
 * Tutorial ch. 5 §5.7 (chunked cross-entropy: the logits of the whole batch are never formed;
 * each chunk of tokens computes its logits, its losses and its gradient, then drops the logits,
 * and the losses are summed).  For hidden states X (M x K bf16), the frozen LM head W (V x K bf16)
 * and labels (M int32 in [0, V)):
 *   loss[m]    = logsumexp_v (X W^T)[m][v] - (X W^T)[m][label[m]],
 *   loss_total = grad_scale * sum_m loss[m]                          (the objective),
 *   dX         = grad_scale (softmax(X W^T) - onehot(label)) W      (its gradient, M x K bf16),
 * so grad_scale = 1/M gives the mean loss and its gradient.  Per chunk of `chunk` tokens the
 * logits are formed once on the matrix cores; the pass keeps, per row and 128 columns, the maximum
 * and the sum of exp (fp32, from the accumulators) and the label's logit, and a fixed-order
 * reduction gives the log-sum-exp and the loss.  With dX the same pass also stores the chunk's
 * fp32 logits in the workspace (as a high and a low 16-bit plane, chunk x V x 4 bytes in all), an
 * elementwise pass writes the bf16 gradient of the logits over the high plane, and the
 * input-gradient kernel multiplies that by W.  chunk = 0 takes lora_ce_default_chunk(V): the
 * largest multiple of 256 tokens whose fp32 logits fit in 512 MiB (at least 256; 1024 at
 * V = 128000), so the workspace stays near that bound whatever M is.  V and K multiples of 64;
 * chunk x V below 2^31.  loss (M fp32) is written; loss_total (one fp32, the fixed-order sum of
 * loss times grad_scale) and dX may be NULL.  A label outside [0, V) gives loss NaN.  Errors as
 * for lora_fwd. */

/* The chunk lora_ce takes when its `chunk` is 0. */
int64_t lora_ce_default_chunk(int64_t V);

/* Bytes of device workspace lora_ce needs (grad: dX requested), no initialisation required. */
size_t lora_ce_workspace_bytes(int64_t M, int64_t V, int64_t K, int64_t chunk, int32_t grad);

lora_status lora_ce(int64_t M, int64_t V, int64_t K, int64_t chunk, float grad_scale,
                    const void* X, const void* W, const int32_t* labels, float* loss,
                    float* loss_total, void* dX, void* ws, size_t ws_bytes, void* stream);

/* The chain rule's last step for lora_ce's dX when the objective arrives with an upstream
 * gradient g (one fp32 in device memory, read by the kernel, so the host never waits for it):
 * out = bf16(dX * g[0]) over M x K bf16 values (out may equal dX).  K a multiple of 8; dX and out
 * 16-byte aligned, g 4-byte aligned.  Errors: LORA_ERR_SHAPE, LORA_ERR_NULL, LORA_ERR_ALIGN,
 * LORA_ERR_HIP. */
lora_status lora_ce_scale_grad(int64_t M, int64_t K, const float* g, const void* dX, void* out, void* stream);

/* ---- RoPE on the attention projections' outputs ------------------------------------------
 * Tutorial ch. 5 §5.5 (fused RoPE: each coordinate pair of q and k multiplied by a 2 x 2 rotation,
 * in one kernel and in place).  For token t at position positions[t] (int32; packed sequences
 * simply restart their positions), head h and j < rot/2, with theta = pos * base^(-2j/rot):
 *   (x_j, x_{j+rot/2}) <- (x_j cos theta - x_{j+rot/2} sin theta, x_{j+rot/2} cos theta + x_j sin theta)
 * (the listing's pairing); coordinates rot .. D-1 are left as they are.  inverse != 0 rotates by
 * -theta: the gradient with respect to the input, applied to dQ and dK.  Q (M x H x D) and K
 * (M x Hk x D) bf16, rotated in place (K may be NULL when Hk = 0; Q and K must not overlap,
 * since an overlapped element would be rotated twice); D a multiple of 8 in
 * [16, 1024]; rot a multiple of 16 in [16, D]; base finite and > 1.  Angles, sines and cosines
 * in fp32 (the angle's rounding is below 1e-3 rad for positions up to 2^14), results rounded to
 * bf16 once.  Errors: LORA_ERR_SHAPE, LORA_ERR_VALUE (base), LORA_ERR_NULL, LORA_ERR_ALIGN,
 * LORA_ERR_HIP. */
lora_status lora_rope(int64_t M, int32_t H, int32_t Hk, int32_t D, int32_t rot, float base,
                      int32_t inverse, const int32_t* positions, void* Q, void* K, void* stream);

/* ---- Diagnostics -----------------------------------------------------------------------
 * The shader clock as a kernel sees it (measurement support, not part of the layer): one wave
 * reads the shader-cycle counter and the 100 MHz real-time counter, spins until `ticks`
 * real-time ticks (10 ns each, 1..10^8) have passed, and writes the two deltas to out[0]
 * (shader cycles) and out[1] (real-time ticks); out[0] / out[1] * 100 is the average shader
 * clock in MHz over the spin.  out: device memory of two uint64, 8-byte aligned.  Errors:
 * LORA_ERR_NULL, LORA_ERR_ALIGN, LORA_ERR_VALUE (ticks), LORA_ERR_HIP. */
lora_status lora_probe_sclk(uint64_t* out, uint32_t ticks, void* stream);

/* The matrix-core ceiling under the chip's own power and clock limits (measurement support):
 * `blocks` workgroups of four waves (one per SIMD) each issue `iters` blocks of 64 independent
 * bf16 16x16x32 MFMAs with nothing in between.  Wave w writes out[3w] (shader cycles),
 * out[3w + 1] (100 MHz real-time ticks) and out[3w + 2] (a value that keeps its results live);
 * 64 x iters x 16384 FLOP per wave over its real time is the rate a bf16 GEMM cannot beat on
 * this chip.  out: device memory of 12 x blocks uint64, 8-byte aligned; blocks in [1, 65536],
 * iters in [1, 10^6].  Errors: LORA_ERR_NULL, LORA_ERR_ALIGN, LORA_ERR_VALUE, LORA_ERR_HIP. */
lora_status lora_probe_mfma(uint64_t* out, int32_t blocks, uint32_t iters, void* stream);

/* What other instructions between the MFMAs cost the matrix core (measurement support): the
 * lora_probe_mfma stream (mode 0) with, per mode, 2, 4 or 6 s_nop after every MFMA (1-3); 20
 * VALU operations after one MFMA in every 8 (4) or the same 20 spread two or three after each
 * MFMA (5); operands read from LDS, two 16-byte reads per lane per 8 MFMAs, used 64 MFMAs later
 * (6); one LDS DMA of 16 bytes per lane per 8 MFMAs (7).  Blocks of 64 MFMAs count in pairs:
 * each wave issues 128 x iters MFMAs.  Same out layout, sizes and errors as lora_probe_mfma;
 * mode in [0, 7] (else LORA_ERR_VALUE).  Mode 7 reads `out` itself as its copy source (before
 * the results are written), so out must not be read by anything else meanwhile. */
lora_status lora_probe_mfma_issue(uint64_t* out, int32_t blocks, uint32_t iters, int32_t mode, void* stream);

/* The streaming-read ceiling (measurement support): reads `bytes` of device memory at `buf`
 * once, 1 KB contiguous per wave load instruction, and writes nothing in practice (`sink`, one
 * device uint32, is written only if the folded words equal a fixed constant; a zero-filled buffer
 * folds to 0).  Time it with events over buffers larger than the 256 MB last-level cache.  buf
 * 16-byte aligned, bytes a positive multiple of 16.  Errors: LORA_ERR_NULL, LORA_ERR_ALIGN,
 * LORA_ERR_VALUE, LORA_ERR_HIP. */
lora_status lora_probe_hbm_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* Human-readable name of a status code, a lora_status value held in an int32_t (static storage;
 * "unknown lora_status" for any other value). */
const char* lora_status_str(int32_t s);

/* Name of the HIP error behind the last LORA_ERR_HIP on the calling thread (static storage). */
const char* lora_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LORA_MI355X_H */
