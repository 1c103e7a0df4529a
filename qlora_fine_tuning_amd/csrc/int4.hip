// int4 weight format utilities and the small-M (decode) QLoRA forward.
//
// "探微索隐：Unsloth 如何加速 LLM 推理？（以 Qwen 27B 为例）": §一 explains why decoding is
// bound by HBM bandwidth (each generated token streams every weight once for a
// matrix-vector product) and §二.3 keeps those weights as 4-bit codes that are turned back
// into bf16 values by a scaling coefficient in registers.  The format: symmetric codes in
// -7..7, two per byte (even k in the low nibble, 4-bit two's complement), one fp16 scale
// (absmax / 7) per 64 consecutive k of a row.
#include "common.hpp"
#include "launch.hpp"

namespace lora {

// ---- quantise + pack: one thread per (row, group of 64) --------------------------------
// s = fp16_rne(a / 7) with a = max|w|: the fp32 quotient is correctly rounded, and it cannot
// land on an fp16 rounding midpoint unless a / 7 is one exactly, so one more rounding to
// fp16 equals a single rounding of the exact quotient.  q = rint(w / s): likewise the
// correctly rounded fp32 quotient of an fp32 w by an fp16 s cannot land on a half-integer
// unless the exact quotient is one, so the code (ties to even) is the exact decision.
__global__ void __launch_bounds__(256)
quantize_int4_kernel(const float* __restrict__ W, uint8_t* __restrict__ Wq,
                     uint16_t* __restrict__ Ws, int64_t groups, int K) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= groups) return;
  const int gpr = K / 64;
  const int64_t row = g / gpr, gi = g - row * gpr;
  const float* src = W + row * K + gi * 64;
  float v[64];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const f32x4 t = *reinterpret_cast<const f32x4*>(src + 4 * i);
    v[4 * i] = t[0];
    v[4 * i + 1] = t[1];
    v[4 * i + 2] = t[2];
    v[4 * i + 3] = t[3];
  }
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 64; ++i) a = fmaxf(a, fabsf(v[i]));
  const _Float16 s16 = (_Float16)__fdiv_rn(a, 7.0f);
  const float s = (float)s16;
  uint32_t words[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    uint32_t wv = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int q = 0;
      if (s != 0.f) q = (int)fminf(fmaxf(rintf(__fdiv_rn(v[8 * d + i], s)), -7.f), 7.f);
      wv |= ((uint32_t)q & 0xfu) << (4 * i);
    }
    words[d] = wv;
  }
  uint8_t* dst = Wq + row * (K / 2) + gi * 32;
  st16(dst, (u32x4){words[0], words[1], words[2], words[3]});
  st16(dst + 16, (u32x4){words[4], words[5], words[6], words[7]});
  Ws[g] = __builtin_bit_cast(uint16_t, s16);
}

// ---- dequantise (the same unpack routine as the matrix kernels): one thread per 32 codes ----
__global__ void __launch_bounds__(256)
dequant_int4_kernel(const uint8_t* __restrict__ Wq, const uint16_t* __restrict__ Ws,
                    uint16_t* __restrict__ Wout, int64_t chunks, int K) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= chunks) return;
  const int cpr = K / 32;
  const int64_t row = c / cpr, kc = c - row * cpr;
  const u32x4 w = ld16(Wq + row * (K / 2) + kc * 16);
  const I4Mix sc = i4mix(half_bits_to_f32(Ws[row * (K / 64) + kc / 2]));
  uint16_t* dst = Wout + row * K + kc * 32;
#pragma unroll
  for (int d = 0; d < 4; ++d) st16(dst + 8 * d, dequant8_mix(w[d], sc));
}

// ---- MXFP4 (the FP4 of §二.3, read as the OCP Microscaling FP4 block format) -------------
// 32 consecutive k share a power-of-two scale 2^(E - 127) (one byte, E8M0); each element is an
// E2M1 code (sign bit 3, exponent bits 2..1 with bias 1, mantissa bit 0) in the same nibble
// layout as the int4 codes.  Block exponent se = floor(log2(absmax)) - 2, clamped to [-125, 125]
// so that every nonzero value and scale stay normal; a block of zeros takes se = 0.

// quantise + pack: one thread per (row, block of 32).  x = |w| 2^-se is exact wherever it can
// reach a rounding threshold (>= 0.25), so the code is the exact decision: nearest E2M1
// magnitude, ties to mantissa bit 0, past 6 to 6, written as counts of thresholds passed.
__global__ void __launch_bounds__(256)
quantize_mxfp4_kernel(const float* __restrict__ W, uint8_t* __restrict__ Wq, uint8_t* __restrict__ We,
                      int64_t blocks, int K) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= blocks) return;
  const int bpr = K / 32;
  const int64_t row = b / bpr, bi = b - row * bpr;
  const float* src = W + row * K + bi * 32;
  float v[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const f32x4 t = *reinterpret_cast<const f32x4*>(src + 4 * i);
    v[4 * i] = t[0];
    v[4 * i + 1] = t[1];
    v[4 * i + 2] = t[2];
    v[4 * i + 3] = t[3];
  }
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) a = fmaxf(a, fabsf(v[i]));
  // floor(log2 a) from the exponent field (a subnormal a clamps to -125 either way)
  const int ex = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;
  const int se = a == 0.f ? 0 : min(max(ex - 2, -125), 125);
  const float inv = __uint_as_float((uint32_t)(127 - se) << 23);  // 2^-se, normal
  uint32_t words[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t wv = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float w = v[8 * d + i], x = fabsf(w) * inv;
      uint32_t c = (uint32_t)(x > 0.25f) + (uint32_t)(x >= 0.75f) + (uint32_t)(x > 1.25f) + (uint32_t)(x >= 1.75f) +
                   (uint32_t)(x > 2.5f) + (uint32_t)(x >= 3.5f) + (uint32_t)(x > 5.f);
      c |= w < 0.f ? 8u : 0u;
      wv |= c << (4 * i);
    }
    words[d] = wv;
  }
  st16(Wq + row * (K / 2) + bi * 16, (u32x4){words[0], words[1], words[2], words[3]});
  We[b] = (uint8_t)(se + 127);
}

// dequantise: one thread per block of 32 codes
__global__ void __launch_bounds__(256)
dequant_mxfp4_kernel(const uint8_t* __restrict__ Wq, const uint8_t* __restrict__ We, uint16_t* __restrict__ Wout,
                     int64_t blocks, int K) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= blocks) return;
  const int bpr = K / 32;
  const int64_t row = b / bpr, bi = b - row * bpr;
  const u32x4 w = ld16(Wq + row * (K / 2) + bi * 16);
  const float sc = e8m0_to_f32(We[b]);
  uint16_t* dst = Wout + row * K + bi * 32;
#pragma unroll
  for (int d = 0; d < 4; ++d) st16(dst + 8 * d, dequant8_fp4(w[d], sc));
}

// ---- decode matrix-vector product, M <= 8 --------------------------------------------
// One kernel per call, bound by the bandwidth of streaming the packed weight once.
//
// Grid (one dimension): NXA adapter workgroups first, then T x S tile workgroups, sized so
// that all of them are resident at once (two per CU).
//  * Adapter workgroup x computes (X A^T) over k in [1024 x, 1024 x + 1024) for all R rows;
//    the last of them to finish (arrival counter) adds the NXA partials in order into
//    XA_f (workspace), writes the caller's XA, and sets every tile's ready token.
//  * Tile workgroup (tile, split) streams weight rows [64 tile, +64) over its share of K in
//    512-k steps through a three-stage LDS ring: per step and wave, four buffer_load ... lds
//    instructions of 4 rows x 256 contiguous bytes (16-byte pieces XOR-swizzled by row, so
//    the MFMA-layout reads are free of bank conflicts), two more for the step's slice of X
//    (shared by the four waves), one dword of scales and one read of the tile's ready token.
//    Two steps are in flight while one is computed; one barrier per step.  A lane reads four pieces (128 codes of its row),
//    unpacks them in registers and feeds 16 bf16 MFMAs whose 16 token columns hold the M
//    tokens.
//  * With several splits each tile workgroup publishes its fp32 partial; the last one of a
//    tile to finish (arrival counter) adds the partials in split order.  The workgroup that
//    completes a tile adds scale * XA_f B^T for its 64 rows once the tile's token is set
//    (normally seen during the loop), writes Y, and clears the token and the counter.
// Every control word is thus cleared by the one workgroup that used it last, and no word is
// shared by more than one tile.  Tile workgroups wait only for the adapter workgroups, which
// come first in the grid (dispatched first) and wait for nothing, and the wait is bounded.  If
// the token never arrives, the tile writes NaN and sets the sticky status word at the head of
// the workspace (a token set later would otherwise pass a stale X A^T to the next call); while
// the status word is set, every call on the workspace writes NaN at once, until the caller reads
// and clears it (qlora_decode_status).
// Cross-workgroup data (partials, XA_f, counters) crosses XCDs, whose L2 caches are not
// coherent with each other; it is written and read with device-scope relaxed atomic
// accesses, and every writer waits for its stores (vmcnt) before moving a counter.
constexpr int kDecRows = 64;      // weight rows per tile workgroup (16 per wave)
constexpr int kDecStep = 512;     // k per pipeline step
constexpr int kDecXK = 1024;      // k per adapter workgroup
constexpr int kDecStage = 4096;   // LDS bytes of one wave's step (16 rows x 256 B)
constexpr int kDecXRow = 1040;    // LDS bytes per token of a step's X slice (+16: distinct banks)
constexpr int kDecSlots = 512;    // resident workgroups (two per CU)
constexpr uint32_t kDecSpin = 1u << 22;  // bound on the ready-token wait (about a second)

// buffer_load ... lds as inline asm (see the tile loop): M0 holds the wave's LDS destination,
// the hardware adds 16 (or 4) bytes per lane.  M0 is not declared clobbered: the compiler
// treats it as reserved, and on gfx950 nothing else in these kernels reads it (LDS
// instructions do not use M0).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void dma16_asm(rsrc_t r, const void* lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds_addr(lds)), "v"(voff), "s"(r)
               : "memory");
}
__device__ __forceinline__ void dma4_dev_asm(rsrc_t r, const void* lds, uint32_t voff) {  // sc1: device scope
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen sc1 lds" ::"s"(lds_addr(lds)), "v"(voff), "s"(r)
               : "memory");
}
__device__ __forceinline__ void dma16_dev_asm(rsrc_t r, const void* lds, uint32_t voff) {  // sc1
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen sc1 lds" ::"s"(lds_addr(lds)), "v"(voff), "s"(r)
               : "memory");
}
__device__ __forceinline__ void dma4_asm(rsrc_t r, const void* lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(lds_addr(lds)), "v"(voff), "s"(r)
               : "memory");
}

struct DecodeArgs {
  const uint16_t* X;
  const uint8_t* Wq;
  const uint16_t* Ws;
  const uint16_t* A;
  const uint16_t* B;
  uint16_t* Y;
  float* XA;
  uint32_t* hdr;   // [0] status (nonzero: a wait gave up), [1] hold (test hook: no tokens published)
  uint32_t* ctl;   // [T] split arrival counters, [T] ready tokens, adapter arrival counter
  float* part;     // [S][T][M][64] tile partials
  float* pxa;      // [NXA][M][RP] adapter partials
  float* xaf;      // [M][RP] X A^T
  int M, N, K, R, S, NXA, NST;  // NST: 512-k steps per tile workgroup
  float scale;
};

__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// X A^T over one 1024-k slice: wave w takes k in [256 w, 256 w + 256) of the slice.
template <int RP>
__device__ void decode_adapter(const DecodeArgs& a, int xw, float* sred, int* sflag) {
  constexpr int NA = RP / 16;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int M = a.M, K = a.K;
  const int t = min(r16, M - 1);
  const int kw = xw * kDecXK + 256 * w;
  const uint32_t hold = __hip_atomic_load(a.hdr + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  f32x4 acc[NA];
#pragma unroll
  for (int ib = 0; ib < NA; ++ib) acc[ib] = fzero4();
  const rsrc_t rA = make_rsrc(a.A, (uint32_t)((size_t)a.R * K * 2));
#pragma unroll
  for (int j = 0; j < 8; ++j) {  // MFMA j: k = kw + 32 j + 8 g4 .. +7
    const int k = kw + 32 * j + 8 * g4;
    const u32x4 xf = ld16(a.X + (size_t)t * K + k);
#pragma unroll
    for (int ib = 0; ib < NA; ++ib)  // rows >= R read past the buffer end: zeros
      acc[ib] = mfma16(bload16(rA, (uint32_t)(((ib * 16 + r16) * K + k) * 2), 0u), xf, acc[ib]);
  }
  // acc[ib][v]: adapter row ib*16 + 4 g4 + v, token r16; add the four waves in order
#pragma unroll
  for (int ib = 0; ib < NA; ++ib)
#pragma unroll
    for (int v = 0; v < 4; ++v) sred[(w * RP + ib * 16 + 4 * g4 + v) * 16 + r16] = acc[ib][v];
  __syncthreads();
  for (int e = tid; e < M * a.R; e += 256) {
    const int tt = e / a.R, i = e - tt * a.R;
    const float s = ((sred[(0 * RP + i) * 16 + tt] + sred[(1 * RP + i) * 16 + tt]) + sred[(2 * RP + i) * 16 + tt]) +
                    sred[(3 * RP + i) * 16 + tt];
    st_dev(a.pxa + ((size_t)xw * M + tt) * RP + i, s);
  }
  wait_stores();
  __syncthreads();
  const int T = a.N / kDecRows;
  uint32_t* ctl = a.ctl;
  if (tid == 0)
    *sflag = __hip_atomic_fetch_add(ctl + 2 * T, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(a.NXA - 1);
  __syncthreads();
  if (!*sflag) return;
  for (int e = tid; e < M * a.R; e += 256) {
    const int tt = e / a.R, i = e - tt * a.R;
    // the partials in order, eight loads in flight at a time
    float s = 0.f;
    int x = 0;
    for (; x + 8 <= a.NXA; x += 8) {
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = ld_dev(a.pxa + ((size_t)(x + q) * M + tt) * RP + i);
#pragma unroll
      for (int q = 0; q < 8; ++q) s += v[q];
    }
    for (; x < a.NXA; ++x) s += ld_dev(a.pxa + ((size_t)x * M + tt) * RP + i);
    st_dev(a.xaf + tt * RP + i, s);
    if (a.XA != nullptr) a.XA[e] = s;
  }
  wait_stores();
  __syncthreads();
  if (hold == 0u)
    for (int t = tid; t < T; t += 256) __hip_atomic_store(ctl + T + t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (tid == 0) __hip_atomic_store(ctl + 2 * T, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// FP4: the weight is MXFP4 (a.Ws then holds the E8M0 bytes: 16 per row and 512-k step, the same
// bytes per step as the int4 scales, so the staging is shared)
template <int RP, bool FP4>
__global__ void __launch_bounds__(256) decode_int4_kernel(DecodeArgs a) {
  __shared__ __align__(16) uint8_t sW0[4 * kDecStage];
  __shared__ __align__(16) uint8_t sW1[4 * kDecStage];
  __shared__ __align__(16) uint8_t sW2[4 * kDecStage];
  __shared__ __align__(16) uint8_t sX0[8 * kDecXRow];
  __shared__ __align__(16) uint8_t sX1[8 * kDecXRow];
  __shared__ __align__(16) uint8_t sX2[8 * kDecXRow];
  __shared__ __align__(16) uint32_t sS0[4 * 64];
  __shared__ __align__(16) uint32_t sS1[4 * 64];
  __shared__ __align__(16) uint32_t sS2[4 * 64];
  __shared__ __align__(16) uint32_t sTok[4 * 64];  // each wave's latest read of the ready token
  __shared__ __align__(16) float sXaf[2 * 256];     // XA_f [M][RP] as last read by waves 0 and 1
  __shared__ __align__(16) uint32_t sJunk[4 * 64];  // destination of the empty loads
  __shared__ int sflag;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;
  const int bid = blockIdx.x;
  if (bid < a.NXA) {
    decode_adapter<RP>(a, bid, reinterpret_cast<float*>(sW0), &sflag);
    return;
  }
  const int T = a.N / kDecRows;
  const int tile = (bid - a.NXA) / a.S, ks = (bid - a.NXA) - tile * a.S;
  const int M = a.M, K = a.K, Kb = K / 2, NST = a.NST;
  const int st0 = ks * NST;                   // first 512-k step of this workgroup
  const int wrow = tile * kDecRows + 16 * w;  // first row of this wave

  const rsrc_t rX = make_rsrc(a.X, (uint32_t)((size_t)M * K * 2));
  const rsrc_t rW = make_rsrc(a.Wq, (uint32_t)((size_t)a.N * Kb));
  const rsrc_t rS = make_rsrc(a.Ws, (uint32_t)((size_t)a.N * (K / 64) * 2));
  const int rq = lane >> 4, slot = lane & 15;  // W DMA lane: row 4 q + rq of the wave, LDS slot
  const uint32_t vW0 = (uint32_t)((wrow + rq) * Kb + st0 * 256);
  const uint32_t vX0 = (uint32_t)(st0 * kDecStep * 2 + lane * 16);
  const uint32_t vS0 = (uint32_t)(((wrow + (lane >> 2)) * (K / 64) + st0 * 8) * 2 + (lane & 3) * 4);
  const rsrc_t rC = make_rsrc(a.ctl, (uint32_t)((2 * T + 1) * 4));
  const uint32_t vTok = (uint32_t)((T + tile) * 4);
  const rsrc_t rF = make_rsrc(a.xaf, (uint32_t)(M * RP * 4));
  // rows n .. n+3 of B for the final low-rank term, loaded now while the weights stream
  // (ranks up to 16; larger ranks load them at the end)
  const int nl = 16 * w + 4 * g4;
  const int n = tile * kDecRows + nl;
  u32x4 bpre[4][2];
  if (RP == 16) {
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int c = 0; c < 2; ++c) bpre[v][c] = (8 * c < a.R) ? ld16(a.B + (size_t)(n + v) * a.R + 8 * c) : zero4();
  }
  uint32_t seen = 0, fresh = 0;  // fresh: an XA_f read was issued after the token was seen
  // Step st of this workgroup into stage (sW, sX, sS): per wave 2 + 4 + 2 + 1 loads straight
  // to LDS, the first two device-coherent reads of the tile's ready token and of XA_f.  Steps >= NST read past every buffer's end (zeros, no memory traffic) so that every
  // wave always has the same number of loads in flight.  The loads are issued as inline asm,
  // outside the compiler's wait-count tracking, and waited for explicitly: the compiler
  // would otherwise wait for every LDS load in flight before the first LDS read, which
  // empties the pipeline.
  auto issue = [&](uint8_t* sW, uint8_t* sX, uint32_t* sS, int st) {
    const uint32_t oob = st < NST ? 0u : 0x40000000u;
    dma4_dev_asm(rC, sTok + w * 64, vTok);
    // XA_f (1 KB for each of waves 0 and 1, device-coherent), read once, at the first step after
    // the wave has seen the token; every other step issues an empty load in its place (the
    // condition is taken wave-uniform so that exactly one load is issued either way)
    if (w < 2 && __builtin_amdgcn_readfirstlane(seen && !fresh))
      dma16_dev_asm(rF, sXaf + w * 256, (uint32_t)(w * 1024 + lane * 16));
    else
      dma4_asm(rF, sJunk + w * 64, 0x40000000u);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 4 * q + rq;
      dma16_asm(rW, sW + w * kDecStage + q * 1024, vW0 + oob + (uint32_t)(4 * q * Kb + st * 256 + 16 * (slot ^ r)));
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // tokens 2 w and 2 w + 1 (tokens >= M: zeros)
      const int tt = 2 * w + h;
      const uint32_t toob = tt < M ? 0u : 0x40000000u;
      dma16_asm(rX, sX + tt * kDecXRow, vX0 + oob + toob + (uint32_t)(tt * K * 2 + st * kDecStep * 2));
    }
    dma4_asm(rS, sS + w * 64, vS0 + oob + (uint32_t)(st * 16));
  };

  const int t = min(r16, M - 1);
  // the status word, read now and used at the end: a workspace whose status is set gives NaN
  const uint32_t status0 = tid == 0 ? __hip_atomic_load(a.hdr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
  f32x4 acc[2] = {fzero4(), fzero4()};
  // one step: MFMA (piece i, dword j) covers k = 512 st + 32 (4 g4 + i) + 8 j .. +7
  auto compute = [&](const uint8_t* sW, const uint8_t* sX, const uint32_t* sS) {
    const uint8_t* stage = sW + w * kDecStage + r16 * 256;
    const uint8_t* xl = sX + t * kDecXRow + 256 * g4;
    // int4: the fp16 scales of groups 2 g4, 2 g4 + 1; FP4: the E8M0 bytes of blocks 4 g4 .. +3,
    // block 4 g4 + i being piece i
    const uint32_t sc = sS[w * 64 + r16 * 4 + g4];
    if constexpr (FP4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 wv = *reinterpret_cast<const u32x4*>(stage + 16 * ((4 * g4 + i) ^ r16));
        const float bs = e8m0_to_f32((sc >> (8 * i)) & 0xffu);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 xf = *reinterpret_cast<const u32x4*>(xl + 64 * i + 16 * j);
          acc[j & 1] = mfma16(dequant8_fp4(wv[j], bs), xf, acc[j & 1]);
        }
      }
    } else {
      const I4Mix m0 = i4mix(half_bits_to_f32((uint16_t)(sc & 0xffffu)));
      const I4Mix m1 = i4mix(half_bits_to_f32((uint16_t)(sc >> 16)));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 wv = *reinterpret_cast<const u32x4*>(stage + 16 * ((4 * g4 + i) ^ r16));
        const I4Mix& mx = (i < 2) ? m0 : m1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 xf = *reinterpret_cast<const u32x4*>(xl + 64 * i + 16 * j);
          acc[j & 1] = mfma16(dequant8_mix(wv[j], mx), xf, acc[j & 1]);
        }
      }
    }
  };
  // wait for this wave's loads of the current step (the next step's nine stay in flight)
  // and its LDS reads, then a barrier: every wave's loads of the step have landed and every
  // wave is done with the stage that is refilled next
  auto step_sync = []() { asm volatile("s_waitcnt vmcnt(9) lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

  sTok[w * 64 + lane] = 0u;  // read before the first token load lands (same wave: ordered)
  issue(sW0, sX0, sS0, 0);
  issue(sW1, sX1, sS1, 1);
  for (int st = 0; st < NST; st += 3) {
    step_sync();
    seen |= sTok[w * 64];
    issue(sW2, sX2, sS2, st + 2);
    fresh = seen;
    compute(sW0, sX0, sS0);
    if (st + 1 < NST) {
      step_sync();
      seen |= sTok[w * 64];
      issue(sW0, sX0, sS0, st + 3);
      fresh = seen;
      compute(sW1, sX1, sS1);
    }
    if (st + 2 < NST) {
      step_sync();
      seen |= sTok[w * 64];
      issue(sW1, sX1, sS1, st + 4);
      fresh = seen;
      compute(sW2, sX2, sS2);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the ring's last (empty) loads
  if (tid == 0) sflag = 0;
  __syncthreads();
  seen |= sTok[w * 64];
  if (w < 2 && lane == 0 && fresh) atomicOr(&sflag, 1 << w);  // LDS atomic
  __syncthreads();
  const bool xaf_local = sflag == 3;  // both halves of XA_f in LDS are current

  // acc: rows wrow + 4 g4 + v, token r16
  f32x4 p = acc[0] + acc[1];
  uint32_t* ctl = a.ctl;
  if (a.S > 1) {
    if (r16 < M) {
      float* dst = a.part + (((size_t)ks * T + tile) * M + r16) * kDecRows + nl;
#pragma unroll
      for (int v = 0; v < 4; ++v) st_dev(dst + v, p[v]);
    }
    wait_stores();
    __syncthreads();
    if (tid == 0)
      sflag = __hip_atomic_fetch_add(ctl + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(a.S - 1);
    __syncthreads();
    if (!sflag) return;
    if (r16 < M) {  // the split partials in order, two splits' loads in flight at a time
      p = fzero4();
      int s = 0;
      for (; s + 2 <= a.S; s += 2) {
        const float* s0 = a.part + (((size_t)s * T + tile) * M + r16) * kDecRows + nl;
        const float* s1 = a.part + (((size_t)(s + 1) * T + tile) * M + r16) * kDecRows + nl;
        float v0[4], v1[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) v0[v] = ld_dev(s0 + v), v1[v] = ld_dev(s1 + v);
#pragma unroll
        for (int v = 0; v < 4; ++v) p[v] = (p[v] + v0[v]) + v1[v];
      }
      if (s < a.S) {
        const float* src = a.part + (((size_t)s * T + tile) * M + r16) * kDecRows + nl;
#pragma unroll
        for (int v = 0; v < 4; ++v) p[v] += ld_dev(src + v);
      }
    }
  }

  // ---- this workgroup finishes the tile: wait for X A^T, add the low-rank term, write Y ----
  __syncthreads();
  if (tid == 0) {
    const bool poisoned = status0 != 0u;
    uint32_t n = 0;
    if (!seen && !poisoned)
      while (__hip_atomic_load(ctl + T + tile, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u && n < kDecSpin) {
        __builtin_amdgcn_s_sleep(8);
        ++n;
      }
    if (n >= kDecSpin) __hip_atomic_fetch_or(a.hdr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sflag = (n < kDecSpin) && !poisoned;
  }
  __syncthreads();
  const bool ready = sflag;
  float* sxa = sXaf;  // [M][RP]
  if (!xaf_local) {
    for (int e = tid; e < M * RP; e += 256) sxa[e] = ready ? ld_dev(a.xaf + e) : 0.f;
    __syncthreads();
  }
  if (r16 < M) {
    float lora[4] = {0.f, 0.f, 0.f, 0.f};
    for (int i0 = 0; i0 < a.R; i0 += 8) {
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(sxa + r16 * RP + i0);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(sxa + r16 * RP + i0 + 4);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const u32x4 bb = (RP == 16) ? ((i0 == 0) ? bpre[v][0] : bpre[v][1]) : ld16(a.B + (size_t)(n + v) * a.R + i0);
        float s = lora[v];
        s = fmaf(x0[0], bf16_lo(bb[0]), s); s = fmaf(x0[1], bf16_hi(bb[0]), s);
        s = fmaf(x0[2], bf16_lo(bb[1]), s); s = fmaf(x0[3], bf16_hi(bb[1]), s);
        s = fmaf(x1[0], bf16_lo(bb[2]), s); s = fmaf(x1[1], bf16_hi(bb[2]), s);
        s = fmaf(x1[2], bf16_lo(bb[3]), s); s = fmaf(x1[3], bf16_hi(bb[3]), s);
        lora[v] = s;
      }
    }
    f32x4 y;
#pragma unroll
    for (int v = 0; v < 4; ++v) y[v] = ready ? p[v] + a.scale * lora[v] : __builtin_nanf("");
    *reinterpret_cast<u32x2*>(a.Y + (size_t)r16 * a.N + n) = (u32x2){pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3])};
  }
  // clear this tile's token and counter for the next call
  if (tid == 0) {
    if (ready) __hip_atomic_store(ctl + T + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (a.S > 1) __hip_atomic_store(ctl + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---- host launchers ----
hipError_t launch_quantize_int4(int64_t N, int64_t K, const float* W, uint8_t* Wq, uint16_t* Ws,
                                hipStream_t s) {
  const int64_t groups = N * (K / 64);
  hipLaunchKernelGGL(quantize_int4_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, s,
                     W, Wq, Ws, groups, (int)K);
  return hipGetLastError();
}

hipError_t launch_quantize_mxfp4(int64_t N, int64_t K, const float* W, uint8_t* Wq, uint8_t* We, hipStream_t s) {
  const int64_t blocks = N * (K / 32);
  hipLaunchKernelGGL(quantize_mxfp4_kernel, dim3((unsigned)((blocks + 255) / 256)), dim3(256), 0, s, W, Wq, We,
                     blocks, (int)K);
  return hipGetLastError();
}

hipError_t launch_dequant_mxfp4(int64_t N, int64_t K, const uint8_t* Wq, const uint8_t* We, uint16_t* Wout,
                                hipStream_t s) {
  const int64_t blocks = N * (K / 32);
  hipLaunchKernelGGL(dequant_mxfp4_kernel, dim3((unsigned)((blocks + 255) / 256)), dim3(256), 0, s, Wq, We, Wout,
                     blocks, (int)K);
  return hipGetLastError();
}

hipError_t launch_dequant_int4(int64_t N, int64_t K, const uint8_t* Wq, const uint16_t* Ws,
                               uint16_t* Wout, hipStream_t s) {
  const int64_t chunks = N * (K / 32);
  hipLaunchKernelGGL(dequant_int4_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s,
                     Wq, Ws, Wout, chunks, (int)K);
  return hipGetLastError();
}

static int decode_rp(int R) { return R <= 16 ? 16 : (R <= 32 ? 32 : 64); }
static size_t a256(size_t b) { return (b + 255) & ~(size_t)255; }

// Decode grid: K splits S (a divisor of the 512-k step count) as many as keep every tile
// workgroup and the K / 1024 adapter workgroups resident at once.
static int decode_splits(int64_t N, int64_t K) {
  const int64_t T = N / kDecRows, nst = K / kDecStep, nxa = K / kDecXK;
  int S = 1;
  for (int64_t d = 1; d <= nst; ++d)
    if (nst % d == 0 && T * d + nxa <= kDecSlots) S = (int)d;
  return S;
}

struct DecodeLayout {
  size_t hdr, ctl, part, pxa, xaf, total;
};
static DecodeLayout decode_layout(int64_t M, int64_t N, int64_t K, int R) {
  const size_t T = (size_t)(N / kDecRows), S = (size_t)decode_splits(N, K), RP = (size_t)decode_rp(R);
  const size_t NXA = (size_t)(K / kDecXK);
  DecodeLayout l;
  l.hdr = 0;
  l.ctl = 16;
  l.part = a256(16 + (2 * T + 1) * 4);
  l.pxa = l.part + a256(S * T * (size_t)M * kDecRows * 4);
  l.xaf = l.pxa + a256(NXA * (size_t)M * RP * 4);
  l.total = l.xaf + a256((size_t)M * RP * 4);
  return l;
}

size_t gemv_workspace_bytes(int64_t M, int64_t N, int64_t K, int R) { return decode_layout(M, N, K, R).total; }
size_t gemv_control_bytes(int64_t N) { return a256(16 + (2 * (size_t)(N / kDecRows) + 1) * 4); }

template <bool FP4>
static hipError_t launch_gemv(const FwdArgs& f, void* ws, hipStream_t s) {
  const DecodeLayout l = decode_layout(f.M, f.N, f.K, f.R);
  char* base = static_cast<char*>(ws);
  DecodeArgs a;
  a.X = static_cast<const uint16_t*>(f.X);
  a.Wq = static_cast<const uint8_t*>(f.W);
  a.Ws = static_cast<const uint16_t*>(f.Ws);
  a.A = static_cast<const uint16_t*>(f.A);
  a.B = static_cast<const uint16_t*>(f.B);
  a.Y = static_cast<uint16_t*>(f.Y);
  a.XA = f.XA;
  a.hdr = reinterpret_cast<uint32_t*>(base + l.hdr);
  a.ctl = reinterpret_cast<uint32_t*>(base + l.ctl);
  a.part = reinterpret_cast<float*>(base + l.part);
  a.pxa = reinterpret_cast<float*>(base + l.pxa);
  a.xaf = reinterpret_cast<float*>(base + l.xaf);
  a.M = (int)f.M;
  a.N = (int)f.N;
  a.K = (int)f.K;
  a.R = f.R;
  a.S = decode_splits(f.N, f.K);
  a.NXA = (int)(f.K / kDecXK);
  a.NST = (int)(f.K / kDecStep) / a.S;
  a.scale = f.scale;
  const dim3 grid((unsigned)(a.NXA + (f.N / kDecRows) * a.S));
  const int RP = decode_rp(f.R);
  if (RP == 16)
    hipLaunchKernelGGL((decode_int4_kernel<16, FP4>), grid, dim3(256), 0, s, a);
  else if (RP == 32)
    hipLaunchKernelGGL((decode_int4_kernel<32, FP4>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_int4_kernel<64, FP4>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemv_int4(const FwdArgs& f, void* ws, hipStream_t s) { return launch_gemv<false>(f, ws, s); }
hipError_t launch_gemv_mxfp4(const FwdArgs& f, void* ws, hipStream_t s) { return launch_gemv<true>(f, ws, s); }

}  // namespace lora
