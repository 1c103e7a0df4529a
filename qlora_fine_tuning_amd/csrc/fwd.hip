// Fused LoRA / QLoRA forward on gfx950 bf16 MFMA.
//
//   Y = X W^T + scale * (X A^T) B^T,   XA = X A^T saved (unscaled, fp32)
//
// tutorial ch. 5 "加速原理：Triton kernel 与 fused LoRA", §5.3: one program per output tile
// accumulates the base product and the low-rank product and stores Y once, so no
// intermediate reaches HBM.  Here one workgroup owns a 256 x 256 tile of Y:
//  * the K loop stages X, W and A tiles (64 wide) through two LDS buffers.  X, A and bf16 W
//    go HBM -> LDS with buffer_load ... lds (no registers on the way), issued one step ahead
//    and spread between the MFMAs of the step's second half;
//  * each wave accumulates a 128 x 128 block of Y^T on 16x16x32 bf16 MFMA (the W tile is
//    the row operand, so each lane ends up holding 4 consecutive outputs of one Y row);
//  * the same LDS X fragments feed the rank-R panel X A^T (each of the two waves that
//    share a 128-row X slice computes half of it: 6.25% extra MFMA work at R = 16);
//  * the epilogue puts scale * XA through LDS, splits it into bf16 hi + lo parts and adds
//    B (hi + lo)^T into the fp32 accumulators with one more MFMA per 16 ranks, then
//    rounds Y to bf16 once.
// SwiGLU pair (tutorial ch. 5 §5.6): with W = [Wg; Wu] (2 Nh x K) the 256 W rows of a tile
// are 128 gate rows and the 128 up rows of the same outputs, so the two waves that share an X
// slice hold G and U of the same 128 x 128 block; they trade fp32 halves through LDS, and
// H = silu(G) U leaves the epilogue with G and U (bf16, for the backward).
// QLoRA ("探微索隐：Unsloth 如何加速 LLM 推理？（以 Qwen 27B 为例）", §二.3): the W tile
// arrives as packed int4 codes plus one fp16 scale per 64 k; each thread unpacks its
// codes in registers to bf16_rne(q * s) on the way into LDS.
#include "common.hpp"
#include "launch.hpp"

namespace lora {

// sigmoid from the hardware exp2 and reciprocal (about 1 ulp of fp32 each, far below the bf16
// rounding of H); the correctly rounded expf and division cost ~35 VALU operations per element,
// which the epilogue cannot hide behind matrix work
__device__ __forceinline__ float silu_sigmoid(float g) { return __builtin_amdgcn_rcpf(1.f + __expf(-g)); }

// A 128 x 64 block of Y (rows m, columns n: accumulator rows i < 4 of acc[i * 8 + j]) to bf16,
// staged through 16 KB of LDS so that each row leaves as full 16-byte chunks; 8 chunks per row,
// swizzled by the row's low 3 bits.
__device__ __forceinline__ void store_half_bf16(const f32x4* acc, uint16_t* stage, uint16_t* out, size_t ld,
                                                int rows_valid, int cols_valid, int lane) {
  const int l16 = lane & 15, g4 = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = 2 * i + (g4 >> 1);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const f32x4 v = acc[i * 8 + j];
      const u32x2 o = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
      *reinterpret_cast<u32x2*>(stage + (j * 16 + l16) * 64 + ((c ^ (l16 & 7)) << 3) + (g4 & 1) * 4) = o;
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes have landed
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    const int row = p * 8 + (lane >> 3), c = lane & 7;
    const u32x4 v = ld16(stage + row * 64 + ((c ^ (row & 7)) << 3));
    if (row < rows_valid && c * 8 < cols_valid) st16(out + (size_t)row * ld + c * 8, v);
  }
}

// PANEL: the panel X A^T is accumulated here from the X fragments of the main loop.  Without
// it (when the caller keeps XA: rank 64, and the rank-32 SwiGLU pair) XA has been computed by a
// pass of its own and is read in the epilogue: the rank-64 panel's accumulators and A fragments
// make the main loop spill, and the SwiGLU pair's many column tiles per row of X would each
// recompute the rank-32 panel.
// EPI (bf16 W only when not kEpiLora): kEpiSwiglu, N = 2 Nh stacked rows, Y = [G | U] (M x 2 Nh)
// and H (M x Nh) out; kEpiCeStats, the logits X W^T of an LM head (no adapter): per-row (max, sum
// of exp) of each wave's 128 columns into `stats`, the label's logit, and the fp32 logits
// themselves, split into high and low 16-bit planes, when `hi` is set (the gradient pass then
// reads them).
// FP4 (with INT4): the 4-bit weight is MXFP4, E2M1 codes in the same nibble layout and one E8M0
// exponent byte per 32 k (the two bytes of a 64-k step sit where the int4 fp16 scale would).
// Persistent (one resident workgroup per CU looping over tiles): the rank-16 instances with the
// LoRA or LM-head epilogue, and the rank-32 SwiGLU pair without the panel.  The others keep one
// tile per workgroup: with the tile loop around them the compiler fails or spills.
constexpr bool fwd_persistent(int rp, int epi, bool int4, bool panel) {
  return (rp <= 16 && epi != kEpiSwiglu) || (rp == 32 && epi == kEpiSwiglu && !panel);
}

template <int RP, bool INT4, bool PANEL, int EPI, bool FP4 = false>
__global__ void __launch_bounds__(kThreads)
fwd_mfma_kernel(const uint16_t* __restrict__ X, const void* __restrict__ Wp,
                const uint16_t* __restrict__ Wscale, const uint16_t* __restrict__ A,
                const uint16_t* __restrict__ Bm, uint16_t* __restrict__ Y,
                float* __restrict__ XA, uint16_t* __restrict__ H, CeArgs ce, int M, int N, int K, int R,
                float scale) {
  constexpr bool SWIGLU = EPI == kEpiSwiglu, CE = EPI >= kEpiCeStats, LORA = !CE;
  constexpr bool PERSIST = fwd_persistent(RP, EPI, INT4, PANEL);
  static_assert(!(CE && INT4), "the LM head takes a bf16 weight");
  static_assert(!(CE && PANEL), "the LM head has no adapter");
  constexpr int TT = kTile * kStep;  // elements of one 256 x 64 operand tile
  constexpr int AROWS = RP < 32 ? 32 : RP;  // adapter rows in LDS: each wave copies 8k of them
  constexpr int AT = AROWS * kStep;
  // Separate arrays per buffer: the compiler can then see that loads into one buffer never
  // alias reads of the other and keeps the copy engine and the MFMA loop overlapped.
  __shared__ __attribute__((aligned(1024))) uint16_t sX0[TT], sX1[TT], sW0[TT], sW1[TT];
  __shared__ __attribute__((aligned(1024))) uint16_t sA0[AT], sA1[AT];


  const int tiles_m = (M + kTile - 1) / kTile, tiles_n = (N + kTile - 1) / kTile;
  // Persistent instances: one workgroup per CU walks the tiles the non-persistent launch would
  // give the workgroups blockIdx, blockIdx + gridDim, ... (the grid a multiple of the 8 XCDs, so
  // all of them run on this workgroup's XCD and keep its L2 footprint); in the grouped order those
  // tiles lie in one row of tiles, so the rank panel X A^T computed on the first of them is reused
  // by the rest.  (Only the rank-16 instances other than the SwiGLU pair, and the LM head, loop
  // over tiles; the others keep one tile per workgroup: with the tile loop around them the
  // compiler fails or spills inside the main loop.)
  const int tiles = tiles_m * tiles_n;
  constexpr int NB = PANEL ? RP / 16 : 1;  // panel rank blocks held in registers
  f32x4 pacc_keep[NB][4];  // the panel kept across tiles (persistent instances)
  int panel_tm = -1;
  auto tile = [&](int vb) {
  f32x4 pacc_own[NB][4];  // one tile per workgroup: the panel lives with the tile
  auto& pacc = PERSIST ? pacc_keep : pacc_own;
  // The lane's values are derived afresh on every tile (through an opaque copy of the thread id):
  // hoisted out of the tile loop, the addresses computed from them would stay live across the
  // main loop, which has no registers to spare, and be spilled.
  int tid = (int)threadIdx.x;
  if constexpr (PERSIST) asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave >> 1, wm = wave & 1;  // this wave's 128-row half of n and of m
  const int l16 = lane & 15, g4 = lane >> 4;
  int tm, tn;
  grouped_tile(xcd_remap(vb, tiles), tiles_m, tiles_n, 8, tm, tn);
  const int m0 = tm * kTile, n0 = tn * kTile;
  const bool new_panel = PANEL && (!PERSIST || tm != panel_tm);
  panel_tm = tm;
  const int nk = K / kStep;
  const uint32_t rowb = (uint32_t)K * 2;  // bytes per row of X, W (bf16) and A

  const rsrc_t rX = make_rsrc(X + (size_t)m0 * K, (uint32_t)min(M - m0, kTile) * rowb);
  const rsrc_t rA = make_rsrc(A, (uint32_t)R * rowb);
  // SwiGLU: output columns ng .. ng+127 of H; tile rows 0-127 are those gate rows of W (rW),
  // rows 128-255 the up rows (rWu, Nh rows further on)
  const int nh = SWIGLU ? N / 2 : N, ng = SWIGLU ? tn * (kTile / 2) : n0;
  rsrc_t rW, rWu;
  if constexpr (SWIGLU && !INT4) {
    const uint32_t bytes = (uint32_t)min(nh - ng, kTile / 2) * rowb;
    rW = make_rsrc(static_cast<const uint16_t*>(Wp) + (size_t)ng * K, bytes);
    rWu = make_rsrc(static_cast<const uint16_t*>(Wp) + (size_t)(nh + ng) * K, bytes);
  } else if constexpr (!INT4) {
    rW = make_rsrc(static_cast<const uint16_t*>(Wp) + (size_t)n0 * K, (uint32_t)min(N - n0, kTile) * rowb);
  }

  // Lane offsets of the 16-byte LDS-DMA chunks: instruction i of wave w fills rows
  // (4i + w) * 8 .. +7 of a 256-row tile; lane l goes to physical chunk l & 7 of row
  // (l >> 3) there, which holds logical chunk (l & 7) ^ swz(row).
  // With swzf the slot does not depend on i, so one lane offset serves all 8 instructions.
  const uint32_t tile_voff = [&]() {
    const int r = wave * 8 + (lane >> 3);
    return (uint32_t)r * rowb + (uint32_t)((lane & 7) ^ swzf(r)) * 16u;
  }();
  // Offset of instruction i's rows: in the lane offset (one VGPR per i, kept across the loop) at
  // bf16 ranks 16 and 32, so a copy needs no scalar add before it; the others (short of VGPRs, or
  // measured slower: the 4-bit rank-16 forward) add it to the scalar offset.
  constexpr bool VROW = RP <= 32 && !INT4;
  auto voff_i = [&](int i) { return VROW ? tile_voff + (uint32_t)i * 32u * rowb : tile_voff; };
  auto soff_i = [&](int k0, int i) { return (uint32_t)k0 * 2u + (VROW ? 0u : (uint32_t)i * 32u * rowb); };
  auto dma_tile = [&](const rsrc_t& rs, uint16_t* dst, int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      dma16(rs, dst + (4 * i + wave) * 512, voff_i(i), soff_i(k0, i));
  };
  // instruction i of the W tile (rows (4i + w) * 8 ..): SwiGLU takes i < 4 from the gate rows
  // and i >= 4 from the up rows
  auto dma_w_part = [&](uint16_t* dst, int k0, int i) {
    if constexpr (SWIGLU)
      dma16(i < 4 ? rW : rWu, dst + (4 * i + wave) * 512, tile_voff,
            (uint32_t)k0 * 2u + (uint32_t)(i & 3) * 32u * rowb);
    else
      dma16(rW, dst + (4 * i + wave) * 512, voff_i(i), soff_i(k0, i));
  };
  auto dma_a = [&](uint16_t* dst, int k0) {
#pragma unroll
    for (int q0 = 0; q0 < AROWS / 8; q0 += 4) {  // rows q*8 .. q*8+7; rows >= R read as zero
      const int q = q0 + wave;
      const int r = q * 8 + (lane >> 3);
      const int c = (lane & 7) ^ swzf(r);
      dma16(rA, dst + q * 512, (uint32_t)r * rowb + (uint32_t)c * 16u, (uint32_t)k0 * 2u);
    }
  };

  // int4 W: one row per thread pair, thread (tid & 1) takes 32 of the row's 64 codes.  The
  // codes and raw fp16 scales of a step stay in registers (two sets, alternating by step) from
  // their load, two steps ahead, to their unpacking into LDS.
  struct W4 {
    u32x4 q[2];
    uint32_t s[2];  // fp16 bits; converted when used, so the load is not waited for early
  };
  W4 w4a, w4b;
  // Two sets, loaded two steps ahead; the rank-64 instance with the panel in the kernel (the
  // fallback for callers that do not keep XA) uses one set loaded one step ahead (its two-set
  // form crashes the compiler).
  constexpr bool AHEAD = INT4 && (RP <= 32 || !PANEL);
  // 4-bit W: codes and scales (fp16 per 64 k, or E8M0 bytes per 32 k: the same bytes per row);
  // SwiGLU takes tile rows 0-127 from the gate rows (rWq, rWs) and 128-255 from the up rows
  rsrc_t rWq, rWs, rWqU, rWsU;
  if constexpr (INT4) {
    const uint8_t* W8 = static_cast<const uint8_t*>(Wp);
    if constexpr (SWIGLU) {
      const uint32_t nrows = (uint32_t)min(nh - ng, kTile / 2);
      rWq = make_rsrc(W8 + (size_t)ng * (K / 2), nrows * (uint32_t)(K / 2));
      rWqU = make_rsrc(W8 + (size_t)(nh + ng) * (K / 2), nrows * (uint32_t)(K / 2));
      rWs = make_rsrc(Wscale + (size_t)ng * (K / 64), nrows * (uint32_t)(K / 64) * 2u);
      rWsU = make_rsrc(Wscale + (size_t)(nh + ng) * (K / 64), nrows * (uint32_t)(K / 64) * 2u);
    } else {
      const int nrows = min(N - n0, kTile);
      rWq = make_rsrc(W8 + (size_t)n0 * (K / 2), (uint32_t)nrows * (uint32_t)(K / 2));
      rWs = make_rsrc(Wscale + (size_t)n0 * (K / 64), (uint32_t)nrows * (uint32_t)(K / 64) * 2u);
    }
  }
  auto load_w4 = [&](W4& v, int kn) {
    const uint32_t k0 = (uint32_t)min(kn, nk - 1) * kStep;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t r = (uint32_t)((SWIGLU ? 0 : q * 128) + (tid >> 1));
      const rsrc_t& cq = (SWIGLU && q == 1) ? rWqU : rWq;
      const rsrc_t& cs = (SWIGLU && q == 1) ? rWsU : rWs;
      v.q[q] = bload16(cq, r * (uint32_t)(K / 2) + (uint32_t)(tid & 1) * 16u, k0 / 2u);
      v.s[q] = __builtin_amdgcn_raw_buffer_load_b16(cs, (int)(r * (uint32_t)(K / 64) * 2u), (int)(k0 / 32u), 0);
    }
  };
  // part p = 4 q + d: packed dword d (codes k = 8d .. 8d+7 of this half) of row q * 128 + ...
  auto store_w4_part = [&](const W4& v, uint16_t* w, int p) {
    const int q = p >> 2, d = p & 3;
    const int r = q * 128 + (tid >> 1);
    if constexpr (FP4)  // this thread's 32 codes are one block: its exponent byte is (tid & 1)
      st16(w + lds_offf(r, (tid & 1) * 4 + d),
           dequant8_fp4(v.q[q][d], e8m0_to_f32((v.s[q] >> (8 * (tid & 1))) & 0xffu)));
    else
      st16(w + lds_offf(r, (tid & 1) * 4 + d),
           dequant8_mix(v.q[q][d], i4mix(half_bits_to_f32((uint16_t)v.s[q]))));
  };
  auto store_w4 = [&](const W4& v, uint16_t* w) {
#pragma unroll
    for (int p = 0; p < 8; ++p) store_w4_part(v, w, p);
  };
  // The int4 store_w4_part of part p in stages, stage st after MFMA st of row p (the unpack of
  // step kt+1 spread over the first half of step kt; t: the part's working values).  The scale
  // terms are written per use and computed once (at the first part of each half) by the
  // compiler.  Used at rank 16 with int4 codes: measured on the QLoRA FFN forward, 0.97 -> 0.94
  // ms.  (The MXFP4 unpack, four conversions per part, gained nothing staged; the input
  // gradient's unpack neither; at ranks 32 and 64 the compiler crashes: AMDGPU Rewrite
  // AGPR-Copy-MFMA.)
  constexpr bool STAGED = INT4 && !FP4 && RP <= 16;
  auto store_w4_stage = [&](const W4& v, uint16_t* w, int p, int st, I4Stage& t) {
    const int q = p >> 2, d = p & 3;
    const int r = q * 128 + (tid >> 1);
    dequant8_mix_stage(st, v.q[q][d], i4mix(half_bits_to_f32((uint16_t)v.s[q])), t);
    if (st == 7) st16(w + lds_offf(r, (tid & 1) * 4 + d), dequant8_mix_last(t));
  };

  f32x4 acc[64];  // acc[i * 8 + j]: Y^T rows (W) block i, columns (X) block j
#pragma unroll
  for (int i = 0; i < 64; ++i) acc[i] = fzero4();
  mfma_acc_ready(acc);
  if (new_panel)
#pragma unroll
    for (int c = 0; c < NB; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) pacc[c][j] = fzero4();

  // adapter rows R .. AROWS-1 stay zero in both buffers
  if constexpr (PANEL)
    for (int e = R * kStep + tid * 8; e < AT; e += kThreads * 8) {
      st16(sA0 + e, zero4());
      st16(sA1 + e, zero4());
    }

  // MFMA operands of one 32-wide half step: 8 W fragments (rows of Y^T), 8 X fragments
  // (columns of Y^T), RP/16 adapter fragments.
  struct Frag {
    u32x4 w[8], x[8], a[NB];
  };
  // Reads the fragments of half step `kk` into `nx` while running the MFMAs of `cu`.  The
  // reads are spread between the MFMA rows so that LDS latency hides behind matrix work.
  // copy(d), d = 0..15, issues part d of the next step's copies after MFMAs 1 and 5 of row i
  // (d = 2 i, 2 i + 1): spread out, the copies never hold up the wave's MFMA issue the way a
  // burst of 17 copies right after the barrier does.
  auto phase = [&](const Frag& cu, Frag& nx, const uint16_t* x, const uint16_t* w,
                   const uint16_t* a, int kk, bool pan, auto&& copy) {
    const int ch = kk * 4 + g4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // every row of the next phase uses all eight X fragments: they go out in rows 0-3.  In
      // those rows the bf16 instances read the row's W fragment after the first MFMA, so no gap
      // between MFMAs holds more than three other instructions (a fourth costs the matrix core
      // four cycles).
      if (i < 4) {
        nx.x[2 * i] = ld16(x + lds_offf(wm * 128 + 2 * i * 16 + l16, ch));
        nx.x[2 * i + 1] = ld16(x + lds_offf(wm * 128 + (2 * i + 1) * 16 + l16, ch));
      }
      if (INT4 || i >= 4) nx.w[i] = ld16(w + lds_offf(wn * 128 + i * 16 + l16, ch));
      __builtin_amdgcn_sched_barrier(0);
      using Hook = std::decay_t<decltype(copy)>;
      [[maybe_unused]] typename std::conditional_t<IsEveryMfma<Hook>::value, Hook, EveryMfma<int, NoCopy>>::State hs{};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        mfma16_acc(acc[i * 8 + j], cu.w[i], cu.x[j]);
        if (!INT4 && i < 4 && j == 0) {
          __builtin_amdgcn_sched_barrier(0);
          nx.w[i] = ld16(w + lds_offf(wn * 128 + i * 16 + l16, ch));
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (IsEveryMfma<Hook>::value) {
          __builtin_amdgcn_sched_barrier(0);
          copy.f(i * 8 + j, hs);
          __builtin_amdgcn_sched_barrier(0);
        } else if constexpr (!std::is_same_v<std::decay_t<decltype(copy)>, NoCopy>) {
          if (j == 1 || j == 5) {
            __builtin_amdgcn_sched_barrier(0);
            copy(2 * i + (j == 5));
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (PANEL) if (pan) {  // a wave-uniform branch: only the first tile of a row
#pragma unroll
      for (int c = 0; c < RP / 16; ++c) nx.a[c] = ld16(a + lds_offf(c * 16 + l16, ch));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 xp = wn ? cu.x[4 + j] : cu.x[j];  // this wave's half of the panel rows
#pragma unroll
        for (int c = 0; c < RP / 16; ++c) pacc[c][j] = mfma16(cu.a[c], xp, pacc[c][j]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto read_frags = [&](Frag& f, const uint16_t* x, const uint16_t* w, const uint16_t* a, int kk, bool pan) {
    const int ch = kk * 4 + g4;
#pragma unroll
    for (int i = 0; i < 8; ++i) f.x[i] = ld16(x + lds_offf(wm * 128 + i * 16 + l16, ch));
#pragma unroll
    for (int i = 0; i < 8; ++i) f.w[i] = ld16(w + lds_offf(wn * 128 + i * 16 + l16, ch));
    if constexpr (PANEL)
      if (pan)
#pragma unroll
        for (int c = 0; c < RP / 16; ++c) f.a[c] = ld16(a + lds_offf(c * 16 + l16, ch));
  };
  // wait for the copies of the next step: for int4 W, the four register loads issued after
  // them (two steps ahead) stay in flight
  auto wait_all = [&]() {
    if constexpr (INT4) __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
    else wait_vmem();
    __syncthreads();
  };
  // Copies of step kn (clamped to the last step: a repeated copy of the last step into the
  // idle buffer is harmless and keeps the loop free of branches).
  auto prefetch = [&](int kn, uint16_t* xn, uint16_t* wnx, uint16_t* an, bool pan) {
    const int k1 = min(kn, nk - 1) * kStep;
    dma_tile(rX, xn, k1);
    if constexpr (!INT4)
#pragma unroll
      for (int i = 0; i < 8; ++i) dma_w_part(wnx, k1, i);
    if constexpr (PANEL)
      if (pan) dma_a(an, k1);
  };
  // The same copies in 16 parts for phase(): the adapter rows first, then X rows 8d.. (d < 8),
  // W rows (bf16) or the int4 register loads.
  auto prefetch_part = [&](int d, int kn, uint16_t* xn, uint16_t* wnx, uint16_t* an, bool pan) {
    const int k1 = min(kn, nk - 1) * kStep;
    if constexpr (PANEL)
      if (pan && d == 0) dma_a(an, k1);
    if (d < 8) {
      dma16(rX, xn + (4 * d + wave) * 512, voff_i(d), soff_i(k1, d));
    } else if constexpr (!INT4) {
      dma_w_part(wnx, k1, d - 8);
    }
  };
  const NoCopy nocopy;

  // Pipeline (buffers b = kt & 1): on entry to step kt the kk = 0 fragments of step kt are in
  // registers and the copies of step kt+1 are in flight into buffer 1-b.
  //   read kk = 1 fragments of step kt  ||  MFMAs of kk = 0
  //   wait for the step kt+1 copies; barrier (everyone is done reading buffer b)
  //   start the copies of step kt+2 into buffer b
  //   read kk = 0 fragments of step kt+1  ||  MFMAs of kk = 1
  // The main loop, with (pan) or without the rank panel's MFMAs and adapter copies
  const bool pan = PERSIST ? new_panel : PANEL;  // one tile per workgroup: always
  {
  Frag f0, f1;
  prefetch(0, sX0, sW0, sA0, pan);
  if constexpr (INT4) {
    load_w4(w4a, 0);
    if constexpr (AHEAD) load_w4(w4b, 1);
    store_w4(w4a, sW0);
  }
  wait_vmem();
  __syncthreads();
  read_frags(f0, sX0, sW0, sA0, 0, pan);
  prefetch(1, sX1, sW1, sA1, pan);
  if constexpr (INT4) load_w4(w4a, AHEAD ? 2 : 1);

  // One K step on fixed buffers (c = this step's, o = the other): the buffer identities are
  // compile-time, so the compiler can see that the copies into c never alias the reads of o.
  // w4n: the register set holding step kt+1's int4 W (stored during the first half) and then
  // receiving step kt+3's (loaded during the second half)
  auto step = [&](int kt, W4& w4n, uint16_t* xc, uint16_t* wc, uint16_t* ac, uint16_t* xo,
                  uint16_t* wo, uint16_t* ao) {
    if constexpr (INT4)  // the unpacked W of step kt+1, spread between the MFMAs
      if constexpr (STAGED)
        phase(f0, f1, xc, wc, ac, 1, pan, every_mfma<I4Stage>([&](int e, I4Stage& t) { store_w4_stage(w4n, wo, e >> 3, e & 7, t); }));
      else
        phase(f0, f1, xc, wc, ac, 1, pan, [&](int d) { if (d % 2 == 0) store_w4_part(w4n, wo, d / 2); });
    else
      phase(f0, f1, xc, wc, ac, 1, pan, nocopy);
    wait_all();
    phase(f1, f0, xo, wo, ao, 0, pan, [&](int d) {
      prefetch_part(d, kt + 2, xc, wc, ac, pan);
      if constexpr (INT4) { if (d == 15) load_w4(w4n, kt + (AHEAD ? 3 : 2)); }  // after every copy
    });
  };
  int kt = 0;
  W4& w4odd = AHEAD ? w4b : w4a;  // the set of odd steps
  for (; kt + 2 <= nk; kt += 2) {
    step(kt, w4odd, sX0, sW0, sA0, sX1, sW1, sA1);
    step(kt + 1, w4a, sX1, sW1, sA1, sX0, sW0, sA0);
  }
  if (kt < nk) step(kt, w4odd, sX0, sW0, sA0, sX1, sW1, sA1);
  }

  // B fragments of the low-rank epilogue, loaded now so their latency overlaps the panel work
  // (ranks up to 32; the rank-64 instances load them later, prefetching there crashes the
  // compiler)
  constexpr int BPRE = RP <= 32 ? RP / 16 : 1;
  u32x4 fbm[BPRE][8];
  auto load_bfrag = [&](u32x4 (&f)[8], int c) {
    const int rk = c * 16 + (g4 & 1) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // SwiGLU: B rows of the gate (wn = 0) or up (wn = 1) block of the stacked B
      const int n = (SWIGLU ? ng : n0 + wn * 128) + i * 16 + l16;
      const size_t row = (SWIGLU && wn) ? (size_t)(nh + n) : (size_t)n;
      f[i] = (n < nh && rk < R) ? ld16(Bm + row * R + rk) : zero4();
    }
  };
  if constexpr (RP <= 32 && LORA) {
#pragma unroll
    for (int c = 0; c < RP / 16; ++c) load_bfrag(fbm[c], c);
  }
  wait_vmem();
  __syncthreads();
  mfma_drain(acc);

  // ---- epilogue: XA panel -> LDS (and HBM once per row tile), then the rank-R update ----
  // panel rows are spread over the four freed tile buffers, 64 rows each
  constexpr int XS = RP + 4;  // fp32 row stride of the panel in LDS
  static_assert(64 * XS * 4 <= TT * 2, "panel slice must fit a tile buffer");
  auto xa_rows = [&](int q) -> float* {
    return reinterpret_cast<float*>(q == 0 ? sX0 : (q == 1 ? sX1 : (q == 2 ? sW0 : sW1)));
  };
  if constexpr (PANEL) {
#pragma unroll
    for (int c = 0; c < RP / 16; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ml = wm * 128 + (wn * 4 + j) * 16 + l16;
        const int rk = c * 16 + g4 * 4;
        *reinterpret_cast<f32x4*>(xa_rows(ml >> 6) + (ml & 63) * XS + rk) = pacc[c][j];
        if (XA != nullptr && tn == 0 && m0 + ml < M && rk < R)
          *reinterpret_cast<f32x4*>(XA + (size_t)(m0 + ml) * R + rk) = pacc[c][j];
      }
  } else if constexpr (LORA) {  // XA from its own pass (ranks >= R and tokens >= M as zeros)
    for (int e = tid; e < kTile * (RP / 4); e += kThreads) {
      const int ml = e / (RP / 4), rk = (e % (RP / 4)) * 4;
      const f32x4 v = (m0 + ml < M && rk < R) ? *reinterpret_cast<const f32x4*>(XA + (size_t)(m0 + ml) * R + rk) : fzero4();
      *reinterpret_cast<f32x4*>(xa_rows(ml >> 6) + (ml & 63) * XS + rk) = v;
    }
  }
  __syncthreads();

#pragma unroll
  for (int c = 0; c < (LORA ? RP / 16 : 0); ++c) {
    const int rk = c * 16 + (g4 & 1) * 8;
    if constexpr (RP > 32) load_bfrag(fbm[0], c);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int ml = wm * 128 + j * 16 + l16;
      const float* src = xa_rows(ml >> 6) + (ml & 63) * XS + rk;
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(src);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(src + 4);
      const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      u32x4 fx;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float h0, lo0, h1, lo1;
        split_bf16(scale * v[2 * e], h0, lo0);
        split_bf16(scale * v[2 * e + 1], h1, lo1);
        fx[e] = (g4 < 2) ? pack_bf16(h0, h1) : pack_bf16(lo0, lo1);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i * 8 + j] = mfma16(fbm[RP <= 32 ? c : 0][i], fx, acc[i * 8 + j]);
    }
  }

  // ---- store Y (bf16, one rounding), staged through this wave's freed tile buffer ----
  __syncthreads();  // every wave is done with the panel rows in LDS
  auto buf = [&](int w) { return w == 0 ? sX0 : (w == 1 ? sX1 : (w == 2 ? sW0 : sW1)); };
  uint16_t* const stage = buf(wave);
  const int mw = m0 + wm * 128;
  if constexpr (EPI == kEpiCeStats) {
    // each lane holds rows mw + 16 j + l16 and columns nb + 16 i + 4 g4 + e of the logits
    const int nb = n0 + wn * 128;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int m = mw + j * 16 + l16;
      const int lab = m < M ? ce.labels[m] : -1;
      float mx = -__builtin_inff(), lv = 0.f;
      bool found = false;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int n = nb + i * 16 + g4 * 4 + e;
          const float v = acc[i * 8 + j][e];
          if (n < N) mx = fmaxf(mx, v);
          if (n == lab) { lv = v; found = true; }
        }
      float sm = 0.f;
      if (mx != -__builtin_inff())
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (nb + i * 16 + g4 * 4 + e < N) sm += __expf(acc[i * 8 + j][e] - mx);
      // the four lanes of the row (l16 + 16 g4): partners combine the same two operands
#pragma unroll
      for (int o = 16; o <= 32; o <<= 1) {
        const float m2 = __shfl_xor(mx, o, 64), s2 = __shfl_xor(sm, o, 64);
        const float mn = fmaxf(mx, m2);
        if (mn != -__builtin_inff()) sm = sm * __expf(mx - mn) + s2 * __expf(m2 - mn);
        mx = mn;
      }
      if (g4 == 0 && m < M)
        *reinterpret_cast<float2*>(ce.stats + 2 * ((size_t)m * (2 * tiles_n) + tn * 2 + wn)) = make_float2(mx, sm);
      if (found) ce.lab_logit[m] = lv;  // the one lane in the grid holding the label's column
    }
    // the fp32 logits, staged through this wave's freed tile buffer in two 128 x 64 halves so that
    // each row leaves in whole segments; 16-byte chunk c of row r sits at slot c ^ (r & 15).  A
    // logit's 32 bits leave as two 16-bit halves, the high half into one plane and the low half
    // into another (128-byte row segments each): the gradient pass then writes the bf16 gradient
    // over the high plane in place, a dense M x N matrix, and no third buffer is needed.
    if (ce.hi != nullptr) {
      float* const st = reinterpret_cast<float*>(stage);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int r = j * 16 + l16, c = i * 4 + g4;
            *reinterpret_cast<f32x4*>(st + r * 64 + ((c ^ (r & 15)) << 2)) = acc[(4 * h + i) * 8 + j];
          }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes have landed
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int p = 0; p < 32; ++p) {
          const int r = p * 4 + (lane >> 4), c = lane & 15;
          const f32x4 v = *reinterpret_cast<const f32x4*>(st + r * 64 + ((c ^ (r & 15)) << 2));
          const int n = nb + h * 64 + c * 4;
          if (mw + r < M && n < N) {
            const size_t o = (size_t)(mw + r) * N + n;
            uint32_t b[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) b[e] = __float_as_uint(v[e]);
            *reinterpret_cast<uint2*>(ce.hi + o) =
                make_uint2((b[0] >> 16) | (b[1] & 0xffff0000u), (b[2] >> 16) | (b[3] & 0xffff0000u));
            *reinterpret_cast<uint2*>(ce.lo + o) =
                make_uint2((b[0] & 0xffffu) | (b[1] << 16), (b[2] & 0xffffu) | (b[3] << 16));
          }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // the reads are done before the next half is written
        __builtin_amdgcn_wave_barrier();
      }
    }
  } else if constexpr (!SWIGLU) {
    const int nw = n0 + wn * 128;
    store_block_bf16(acc, stage, Y + (size_t)mw * N + nw, (size_t)N, M - mw, N - nw, lane);
  } else {
    // G (gate waves) or U (up waves) of outputs ng .. ng+127 into [G | U]
    store_block_bf16(acc, stage, Y + (size_t)mw * N + (wn ? nh : 0) + ng, (size_t)N, M - mw, nh - ng, lane);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the staging reads are done
    // The gate wave finishes H for accumulator rows i < 4 (outputs ng .. ng+63), the up wave
    // for i >= 4; each hands the other half of its fp32 accumulators to its partner
    // (wave ^ 2, the same X slice) through its own buffer, lane-linear.
    float* const mine = reinterpret_cast<float*>(stage);
    const float* const theirs = reinterpret_cast<const float*>(buf(wave ^ 2));
    // (the branches on wn are wave-uniform; the barriers stay outside them)
    auto give = [&](auto keep_c) {
      constexpr int GIVE = 4 - decltype(keep_c)::value;
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          *reinterpret_cast<f32x4*>(mine + ((q * 8 + j) * 64 + lane) * 4) = acc[(GIVE + q) * 8 + j];
    };
    auto combine = [&](auto keep_c) {
      constexpr int KEEP = decltype(keep_c)::value;
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const f32x4 o = *reinterpret_cast<const f32x4*>(theirs + ((q * 8 + j) * 64 + lane) * 4);
          f32x4& a = acc[(KEEP + q) * 8 + j];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float g = KEEP == 0 ? a[e] : o[e], u = KEEP == 0 ? o[e] : a[e];
            a[e] = g * silu_sigmoid(g) * u;
          }
        }
    };
    auto put = [&](auto keep_c) {
      constexpr int KEEP = decltype(keep_c)::value;
      store_half_bf16(acc + KEEP * 8, stage, H + (size_t)mw * nh + ng + KEEP * 16, (size_t)nh, M - mw,
                      nh - ng - KEEP * 16, lane);
    };
    const std::integral_constant<int, 0> gate_half;
    const std::integral_constant<int, 4> up_half;
    if (wn) give(up_half); else give(gate_half);
    __syncthreads();
    if (wn) combine(up_half); else combine(gate_half);
    __syncthreads();  // the partner is done reading this wave's buffer
    if (wn) put(up_half); else put(gate_half);
  }
  };
  if constexpr (PERSIST) {
    for (int vb = blockIdx.x; vb < tiles; vb += gridDim.x) {
      tile(vb);
      __syncthreads();  // the next tile's copies reuse every wave's LDS
    }
  } else {
    tile(blockIdx.x);
  }
}

template <int RP, bool INT4, bool PANEL, int EPI = kEpiLora, bool FP4 = false>
static hipError_t launch_fwd_rp(const FwdArgs& a, hipStream_t s) {
  // SwiGLU: N = 2 Nh stacked rows, one tile per 128 outputs of H: ceil(2 Nh / 256) of them
  const int tiles = (int)(((a.M + kTile - 1) / kTile) * ((a.N + kTile - 1) / kTile));
  // persistent instances: one resident workgroup per CU, each looping over its run of tiles
  const int cus = device_cus() & ~7;  // a multiple of the 8 XCDs
  const int grid = (fwd_persistent(RP, EPI, INT4, PANEL) && cus > 0 && tiles > cus) ? cus : tiles;
  hipLaunchKernelGGL((fwd_mfma_kernel<RP, INT4, PANEL, EPI, FP4>), dim3(grid), dim3(kThreads), 0, s,
                     (const uint16_t*)a.X, a.W, (const uint16_t*)a.Ws, (const uint16_t*)a.A,
                     (const uint16_t*)a.B, (uint16_t*)a.Y, a.XA, (uint16_t*)a.H, a.ce, (int)a.M, (int)a.N,
                     (int)a.K, (int)a.R, a.scale);
  return hipGetLastError();
}

// logits of an LM head (X W^T, bf16 W, no adapter) with the cross-entropy epilogue: per-row
// statistics (a.ce.stats, a.ce.lab_logit) and, if a.ce.hi is set, the fp32 logits as 16-bit planes
hipError_t launch_ce_logits(const FwdArgs& a, hipStream_t s) { return launch_fwd_rp<16, false, false, kEpiCeStats>(a, s); }

hipError_t launch_fwd_mfma(const FwdArgs& a, bool int4, hipStream_t s) {
  const int rp = a.R <= 16 ? 16 : (a.R <= 32 ? 32 : 64);
  const bool swiglu = a.H != nullptr;
  if (swiglu && rp >= 32 && a.XA != nullptr) {
    // the SwiGLU pair at ranks 32 and 64: the panel by its own pass into XA (partials in Y, which
    // the kernel then overwrites), then the kernel without the panel (persistent at rank 32)
    const hipError_t e = launch_panel_xa(static_cast<const uint16_t*>(a.X), static_cast<const uint16_t*>(a.A),
                                         a.XA, a.Y, (size_t)a.M * a.N * 2, a.M, a.K, a.R, s);
    if (e != hipSuccess) return e;
    if (rp == 32) {
      if (!int4) return launch_fwd_rp<32, false, false, kEpiSwiglu>(a, s);
      return a.fp4 ? launch_fwd_rp<32, true, false, kEpiSwiglu, true>(a, s)
                   : launch_fwd_rp<32, true, false, kEpiSwiglu, false>(a, s);
    }
    if (!int4) return launch_fwd_rp<64, false, false, kEpiSwiglu>(a, s);
    return a.fp4 ? launch_fwd_rp<64, true, false, kEpiSwiglu, true>(a, s)
                 : launch_fwd_rp<64, true, false, kEpiSwiglu, false>(a, s);
  }
  if (swiglu && int4) {  // the SwiGLU pair over a stacked 4-bit weight
    if (a.fp4) {
      if (rp == 16) return launch_fwd_rp<16, true, true, kEpiSwiglu, true>(a, s);
      if (rp == 32) return launch_fwd_rp<32, true, true, kEpiSwiglu, true>(a, s);
      return launch_fwd_rp<64, true, true, kEpiSwiglu, true>(a, s);
    }
    if (rp == 16) return launch_fwd_rp<16, true, true, kEpiSwiglu>(a, s);
    if (rp == 32) return launch_fwd_rp<32, true, true, kEpiSwiglu>(a, s);
    return launch_fwd_rp<64, true, true, kEpiSwiglu>(a, s);
  }
  if (rp == 64 && a.XA != nullptr) {
    // the panel as a pass of its own into XA (its partials in Y, which the kernel then
    // overwrites), then the kernel without the panel
    const hipError_t e = launch_panel_xa(static_cast<const uint16_t*>(a.X), static_cast<const uint16_t*>(a.A),
                                         a.XA, a.Y, (size_t)a.M * a.N * 2, a.M, a.K, a.R, s);
    if (e != hipSuccess) return e;
    if (int4 && a.fp4) return launch_fwd_rp<64, true, false, kEpiLora, true>(a, s);
    return int4 ? launch_fwd_rp<64, true, false>(a, s) : launch_fwd_rp<64, false, false>(a, s);
  }
  if (swiglu) {
    if (rp == 16) return launch_fwd_rp<16, false, true, kEpiSwiglu>(a, s);
    if (rp == 32) return launch_fwd_rp<32, false, true, kEpiSwiglu>(a, s);
    return launch_fwd_rp<64, false, true, kEpiSwiglu>(a, s);
  }
  if (int4 && a.fp4) {
    if (rp == 16) return launch_fwd_rp<16, true, true, kEpiLora, true>(a, s);
    if (rp == 32) return launch_fwd_rp<32, true, true, kEpiLora, true>(a, s);
    return launch_fwd_rp<64, true, true, kEpiLora, true>(a, s);
  }
  if (int4) {
    if (rp == 16) return launch_fwd_rp<16, true, true>(a, s);
    if (rp == 32) return launch_fwd_rp<32, true, true>(a, s);
    return launch_fwd_rp<64, true, true>(a, s);
  }
  if (rp == 16) return launch_fwd_rp<16, false, true>(a, s);
  if (rp == 32) return launch_fwd_rp<32, false, true>(a, s);
  return launch_fwd_rp<64, false, true>(a, s);
}

}  // namespace lora
