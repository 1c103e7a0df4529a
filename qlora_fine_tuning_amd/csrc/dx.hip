// Fused LoRA / QLoRA input gradient on gfx950 bf16 MFMA.
//
//   G  = dY B                       (M x R, fp32, kept for the dA reduction)
//   dX = dY W + scale * G A         (M x K)
//
// tutorial ch. 5 "加速原理：Triton kernel 与 fused LoRA", §5.3 (the backward is fused as
// well); the gradient is derived by hand from Y = X W^T + scale X A^T B^T.  One workgroup
// owns a 256 (tokens) x 256 (k) tile of dX and loops over N, 64 at a time:
//  * dY tiles and W tiles go HBM -> LDS with buffer_load ... lds, both in their own row-major
//    order (coalesced), one step ahead in two buffers;
//  * the contraction index n runs along dY rows but down W columns: the W operand is read
//    with ds_read_b64_tr_b16, which hands each lane 4 consecutive rows of one column, so no
//    transposed copy of W is ever made;
//  * each wave accumulates a 128 (k) x 128 (m) block of dX^T in AGPRs; the rank-R panel
//    G = dY B comes from the same LDS dY fragments, with B^T read the same transposing way;
//  * the epilogue adds A^T (scale G)^T with a bf16 hi + lo split of scale * G, then rounds
//    dX once.
// When the output has too few tiles to fill the chip for a long N loop (the QLoRA FFN input
// gradient: 320 tiles, 432 steps), N is cut into S equal ranges and the grid holds S units per
// tile.  Every unit stores its fp32 partial of the tile (and of its G panel) and moves the
// tile's arrival counter; the last unit to arrive adds the S partials in split order (its own
// from registers) and runs the epilogue, so the sum does not depend on arrival order.  When S
// units per tile leave the last round of a persistent launch part empty, the first `split_hi`
// tiles take S + 1 shorter units instead, chosen so that these fill whole rounds: every CU then
// runs the same steps (the QLoRA FFN: 256 tiles x 3 units of 144 steps in three rounds, then
// 64 tiles x 4 units of 108 steps in a fourth, 540 steps per CU against 576 with 3 units each).
// QLoRA: W arrives as packed int4 codes plus fp16 group scales ("探微索隐：Unsloth 如何加速
// LLM 推理？（以 Qwen 27B 为例）", §二.3); threads unpack them in registers into the same
// row-major LDS tile.
#include "common.hpp"
#include "launch.hpp"

namespace lora {

// W tile in LDS: 4 blocks of 64 columns, each 64 rows (n) x 128 bytes; 16-byte chunk c of row
// r sits in slot c ^ wsw(r).  A transposing read covers 4 consecutive rows x 32 bytes; wsw
// separates rows r, r+2 (bit 1) and the row groups of neighbouring 16-lane groups (bit 3),
// so those reads hit distinct banks; bit 2 of the row (the same for the 4 rows of a read)
// spreads the int4 path's 16-byte stores of 16 consecutive rows over 16 distinct bank groups.
__device__ __forceinline__ int wsw(int r) {
  return (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2) | ((r >> 2) & 1);
}

// Split partials cross XCDs, whose L2 caches are not coherent with each other: they are
// written and read with device-scope (sc1) accesses, and every writer waits for its stores
// before it moves the tile's counter.
constexpr int kCpolSc1 = 16;  // cache-policy operand of the buffer intrinsics: sc1
__device__ __forceinline__ void st_part(rsrc_t r, uint32_t voff, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, 0, kCpolSc1);
}
__device__ __forceinline__ f32x4 ld_part(rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, kCpolSc1);
}

// The instances of rank 16, and the bf16 ones of rank 32, loop over units (one resident workgroup
// per CU); the others keep one unit per workgroup: with the loop around them the compiler fails
// or spills in the main loop.
constexpr bool dx_persistent(int rp, bool int4) { return rp <= 16 || (rp == 32 && !int4); }

// FP4 (with INT4): the 4-bit weight is MXFP4 (E2M1 codes, one E8M0 byte per 32 k; a thread's 64
// codes are two blocks, whose two bytes sit where the int4 fp16 scale would).
// NOADP: no adapter at all (dX = dY W, the gradient of an LM head's logits): no panel, no B or A
// copies and no low-rank epilogue; A, B and G are not read or written.
template <int RP, bool INT4, bool FP4 = false, bool NOADP = false>
__global__ void __launch_bounds__(kThreads)
dx_mfma_kernel(const uint16_t* __restrict__ dY, const void* __restrict__ Wp,
               const uint16_t* __restrict__ Wscale, const uint16_t* __restrict__ A,
               const uint16_t* __restrict__ Bm, uint16_t* __restrict__ dX,
               float* __restrict__ G, int M, int N, int K, int R, float scale, int splits,
               int split_hi_arg, float* __restrict__ part, uint32_t* __restrict__ ctr) {
  // The accumulators stay in AGPRs through inline-asm MFMAs (this file is built with the
  // panel MFMAs in VGPR form).  That is only sound while the compiler never has to move an
  // accumulator inside the loop (it cannot see an asm MFMA's result latency); the builtin
  // path (ASM = false) is kept for instances where it would have to.
  constexpr bool ASM = true;
  // Ranks up to 32 compute the panel G = dY B here, from the dY fragments of the main loop.
  // The rank-64 instances read G, computed by a pass of its own, in the epilogue: the panel's
  // 16 accumulator blocks and B fragments do not fit next to the main tile's, and with them
  // the compiler spills and moves accumulators.
  constexpr bool PANEL = RP <= 32 && !NOADP;
  constexpr bool PERSIST = dx_persistent(RP, INT4);
  constexpr int NB = PANEL ? RP / 16 : 1;  // panel rank blocks held in registers
  constexpr int TT = kTile * kStep;  // 16384 elements: dY tile 256 x 64, W tile 64 x 256
  constexpr int BT = kStep * RP;     // B tile: 64 rows (n) x RP ranks
  constexpr int BQ = (BT / 8 + kThreads - 1) / kThreads;  // 16-byte chunks per thread
  constexpr int BTA = BQ * kThreads * 8;  // every thread stores BQ chunks; the tail is padding
  __shared__ __attribute__((aligned(1024))) uint16_t sD0[TT], sD1[TT], sW0[TT], sW1[TT];
  __shared__ __attribute__((aligned(1024))) uint16_t sB0[BTA], sB1[BTA];

  const int tiles_m = (M + kTile - 1) / kTile, tiles_k = (K + kTile - 1) / kTile;
  const int tiles = tiles_m * tiles_k;
  // (the MXFP4 instance of rank 16 keeps equal splits: with the mixed ones the compiler spills
  // inside its main loop)
  const int split_hi = (FP4 && RP == 16) ? 0 : split_hi_arg;
  const int units = tiles * splits + split_hi;
  // Persistent: one workgroup per CU walks the units the non-persistent launch would give the
  // workgroups blockIdx, blockIdx + gridDim, ... (the grid a multiple of the 8 XCDs, so all run on
  // this workgroup's XCD); those lie in one row of tiles and one split, so the rank panel
  // G = dY B computed on the first of them is reused by the rest.
  f32x4 pacc[NB][4];
  int panel_tm = -1, panel_sp = -1;
  auto unit_body = [&](int vb) {
  int tid = (int)threadIdx.x;
  // (the lane's values are derived afresh for every unit: hoisted out of the unit loop, the
  // addresses computed from them would stay live across the main loop and be spilled)
  if constexpr (PERSIST) asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wk = wave >> 1, wm = wave & 1;
  const int l16 = lane & 15, g4 = lane >> 4;
  // unit -> (split, tile, splits of the tile), split-major: units running together share operand
  // panels in L2.  With split_hi > 0 each XCD's range of units (units / 8 of them) holds first
  // its share of the S-way tiles' units, in the rounds before, then its share of the (S+1)-way
  // tiles' units, which make up the last round.
  const int unit = xcd_remap(vb, units);
  int sp, tile, nsplit;
  if (split_hi == 0) {
    sp = unit / tiles;
    tile = unit - sp * tiles;
    nsplit = splits;
  } else {
    const int q = units >> 3, nlo = tiles - split_hi, lx = (nlo * splits) >> 3;
    const int x = unit / q, local = unit - x * q;
    if (local < lx) {
      const int l = x * lx + local;
      sp = l / nlo;
      tile = split_hi + (l - sp * nlo);
      nsplit = splits;
    } else {
      const int h = x * (q - lx) + (local - lx);
      sp = h / split_hi;
      tile = h - sp * split_hi;
      nsplit = splits + 1;
    }
  }
  int tm, tk;
  grouped_tile(tile, tiles_m, tiles_k, 8, tm, tk);
  // (the panel covers this unit's N range: the key is the row of tiles, the split and whether the
  // tile is one of the (S+1)-way ones)
  const int pkey = sp + (tile < split_hi ? 64 : 0);
  const bool new_panel = PANEL && (!PERSIST || tm != panel_tm || pkey != panel_sp);
  panel_tm = tm;
  panel_sp = pkey;
  const int m0 = tm * kTile, k0 = tk * kTile;
  const int ntot = N / kStep;
  const int sbeg = sp * ntot / nsplit;  // this unit's N steps: [sbeg, sbeg + nsteps)
  const int nsteps = (sp + 1) * ntot / nsplit - sbeg;
  const int nbase = sbeg * kStep;
  const uint32_t rowD = (uint32_t)N * 2, rowW = (uint32_t)K * 2;

  // ---- copies into LDS ----
  const rsrc_t rD = make_rsrc(dY + (size_t)m0 * N, (uint32_t)min(M - m0, kTile) * rowD);
  const uint32_t voffD = [&]() {
    const int r = wave * 8 + (lane >> 3);
    return (uint32_t)r * rowD + (uint32_t)((lane & 7) ^ swzf(r)) * 16u;
  }();
  // Offset of instruction i's rows: in the lane offset (one VGPR per i, kept across the loop) at
  // rank 16 and bf16 rank 32, so a copy needs no scalar add before it; the others (short of
  // VGPRs) add it to the scalar offset.
  constexpr bool VROW = RP == 16 || (RP == 32 && !INT4);
  auto voffd_i = [&](int i) { return VROW ? voffD + (uint32_t)i * 32u * rowD : voffD; };
  auto soffd_i = [&](int n0, int i) { return (uint32_t)n0 * 2u + (VROW ? 0u : (uint32_t)i * 32u * rowD); };
  auto dma_d = [&](uint16_t* dst, int n0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) dma16(rD, dst + (4 * i + wave) * 512, voffd_i(i), soffd_i(n0, i));
  };
  // W (bf16): instruction i of wave w fills block i >> 1, rows ((i & 1) * 4 + w) * 8 .. +7
  rsrc_t rW;
  if constexpr (!INT4)
    rW = make_rsrc(static_cast<const uint16_t*>(Wp) + k0, (uint32_t)((size_t)N * K - k0) * 2u);
  const uint32_t voffW = [&]() {
    const int r = wave * 8 + (lane >> 3);  // row within the 64-row tile, less (i & 1) * 32
    return (uint32_t)r * rowW + (uint32_t)((lane & 7) ^ wsw(r)) * 16u;
  }();
  auto voffw_i = [&](int i) {
    return voffW + (VROW ? (uint32_t)(i & 1) * 32u * rowW + (uint32_t)(i >> 1) * 128u : 0u);
  };
  auto soffw_i = [&](int n0, int i) {
    return (uint32_t)n0 * rowW + (VROW ? 0u : (uint32_t)(i & 1) * 32u * rowW + (uint32_t)(i >> 1) * 128u);
  };
  auto dma_w = [&](uint16_t* dst, int n0) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      dma16(rW, dst + (i >> 1) * 4096 + ((i & 1) * 4 + wave) * 512, voffw_i(i), soffw_i(n0, i));
  };
  // W (int4): each thread unpacks one row's 64 codes of one 64-column block (one scale group).
  // A step's codes and raw fp16 scale stay in registers from their load to their unpacking
  // into LDS: two sets alternating by step, loaded two steps ahead.
  struct W4 {
    u32x4 q[2];
    uint32_t s;  // fp16 bits; converted when used, so the load is not waited for early
  };
  W4 w4a, w4b;
  constexpr bool AHEAD = INT4;  // two register sets, two steps ahead
  rsrc_t rWq, rWs;
  if constexpr (INT4) {
    rWq = make_rsrc(static_cast<const uint8_t*>(Wp) + k0 / 2, (uint32_t)((size_t)N * (K / 2) - k0 / 2));
    rWs = make_rsrc(Wscale + k0 / 64, (uint32_t)((size_t)N * (K / 64) - k0 / 64) * 2u);
  }
  // lanes 16 b .. 16 b + 15 of wave w: rows 16 w .. 16 w + 15 of 64-column block b, lane l of
  // the 16 on row 2 (l & 7) + (l >> 3): a 16-byte LDS store serves 8 lanes per cycle, and rows
  // of one parity take 8 distinct wsw slots, so each 8 lanes fill the 8 distinct 16-byte bank
  // groups.  (Rows in lane order paired equal slots, r and r + 1: 2-way conflicts on every
  // store.  With the four blocks of a row on four consecutive lanes, 8 KB apart, the stores
  // conflicted 4-way.)  A load instruction still reads 16 rows x 128 contiguous bytes.
  // (rank 32 keeps rows in lane order: with the reordered rows its main loop spills)
  const int qrow = RP == 32 ? (tid & 15) + 16 * (tid >> 6) : ((tid << 1) & 14) | ((tid >> 3) & 1) | ((tid >> 2) & 48);
  const int qblk = (tid >> 4) & 3;
  auto load_w4 = [&](W4& v, int stn) {
    const uint32_t r = (uint32_t)(nbase + min(stn, nsteps - 1) * kStep + qrow);
    const uint32_t vo = r * (uint32_t)(K / 2) + (uint32_t)qblk * 32u;
    v.q[0] = bload16(rWq, vo, 0);
    v.q[1] = bload16(rWq, vo + 16u, 0);
    v.s = __builtin_amdgcn_raw_buffer_load_b16(rWs, (int)((r * (uint32_t)(K / 64) + (uint32_t)qblk) * 2u), 0, 0);
  };
  auto store_w4_part = [&](const W4& v, uint16_t* w, int d) {  // packed dword d of the 64 codes
    uint16_t* row = w + qblk * 4096 + qrow * 64;
    if constexpr (FP4)  // dwords 0-3 are block 0, 4-7 block 1
      st16(row + ((d ^ wsw(qrow)) << 3), dequant8_fp4(v.q[d >> 2][d & 3], e8m0_to_f32((v.s >> (8 * (d >> 2))) & 0xffu)));
    else
      st16(row + ((d ^ wsw(qrow)) << 3), dequant8_mix(v.q[d >> 2][d & 3], i4mix(half_bits_to_f32((uint16_t)v.s))));
  };
  auto store_w4 = [&](const W4& v, uint16_t* w) {
#pragma unroll
    for (int d = 0; d < 8; ++d) store_w4_part(v, w, d);
  };
  // B: 64 rows x RP ranks (ranks >= R are zero: their chunks read past the end of the buffer,
  // which returns zeros).  bf16 rank 16 copies it straight into LDS, 16-byte chunk c = 64 w + lane
  // by waves w < 2: row c / 2, ranks 8 (c % 2) ..  The others go through registers, branch-free
  // (chunks past the tile read a valid row and land in the padding; no select after the load, so
  // nothing waits for it before the LDS store): with the direct copy the rank-32 instances spill
  // in the main loop, and the MXFP4 one ran slower.
  constexpr bool BDMA = RP == 16 && !INT4;
  u32x4 rb[BQ];
  const rsrc_t rB = make_rsrc(Bm, (uint32_t)N * (uint32_t)R * 2u);
  auto dma_b = [&](uint16_t* b, int n0) {
    const int c = wave * 64 + lane, row = (c >> 1) & 63, rk = (c & 1) * 8;
    const uint32_t vo = rk < R ? ((uint32_t)row * (uint32_t)R + (uint32_t)rk) * 2u : 0x80000000u;
    if (wave < 2) dma16(rB, b + wave * 512, vo, (uint32_t)n0 * (uint32_t)R * 2u);
  };
  auto load_b = [&](int n0) {
#pragma unroll
    for (int q = 0; q < BQ; ++q) {
      const int c = q * kThreads + tid, row = (c / (RP / 8)) & 63, rk = (c % (RP / 8)) * 8;
      const uint32_t vo = rk < R ? ((uint32_t)(n0 + row) * (uint32_t)R + (uint32_t)rk) * 2u : 0x80000000u;
      rb[q] = bload16(rB, vo, 0);
    }
  };
  auto store_b = [&](uint16_t* b) {
#pragma unroll
    for (int q = 0; q < BQ; ++q) st16(b + (q * kThreads + tid) * 8, rb[q]);
  };

  f32x4 acc[64];  // acc[i * 8 + j]: dX^T rows (k) block i, columns (m) block j
#pragma unroll
  for (int i = 0; i < 64; ++i) acc[i] = fzero4();
  if (new_panel)
#pragma unroll
    for (int c = 0; c < NB; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) pacc[c][j] = fzero4();
  // with (pan) or without the panel's MFMAs and B copies: only the first unit of a row and split
  const bool pan = PERSIST ? new_panel : PANEL;
  if constexpr (ASM) mfma_acc_ready(acc);

  // transposing-read addresses: lane (l16, g4) reads rows 4 (l16 >> 2) + .. of its 16-lane
  // group (and the 4 rows after them), columns 4 (l16 & 3) ..; per 16-column block q of a
  // 64-column W block the chunk is 2q + ((l16 & 3) >> 1), swizzled by wsw of a row whose bits
  // 1..3 are fixed per lane (bit 2 flips for the second read).
  const int trow = g4 * 8 + (l16 >> 2);  // + kk * 32 (+ 4)
  // chunk 2q + x (x = (l16 & 3) >> 1) sits in slot (2q + x) ^ wsw(trow) = 2 (q ^ t2) + x, since
  // bit 0 of wsw(trow) is 0 (bit 2 of trow is 0): offset wbase + 16 (q ^ t2), q known at
  // compile time.  The rows 4 further on have bit 0 of the slot flipped: + woff4d.
  const int t2 = wsw(trow) >> 1;
  const int wbase = trow * 64 + (((l16 & 3) >> 1) << 3) + (l16 & 1) * 4;
  const int woff4d = 4 * 64 + ((((l16 & 3) >> 1) & 1) ? -8 : 8);
  auto woff = [&](int q) { return wbase + ((q ^ t2) << 4); };
  const int boff = trow * RP + (l16 & 3) * 4;

  struct Frag {
    u32x4 w[8], d[8], b[NB];
  };
  auto wfrag = [&](const uint16_t* w, int kk, int i) -> u32x4 {
    const int kb = wk * 8 + i;  // 16-column block within the 256-column tile
    const uint16_t* p = w + (kb >> 2) * 4096 + kk * 32 * 64;
    const int o = woff(kb & 3);
    return join(ld_tr(p + o), ld_tr(p + o + woff4d));
  };
  auto bfrag = [&](const uint16_t* b, int kk, int c) -> u32x4 {
    const uint16_t* p = b + kk * 32 * RP + boff + c * 16;
    return join(ld_tr(p), ld_tr(p + 4 * RP));
  };
  // copy(q), q = 0..15: part q of the next step's copies, issued after MFMAs 1 and 5 of row i
  // (see the forward kernel)
  auto phase = [&](const Frag& cu, Frag& nx, const uint16_t* d, const uint16_t* w,
                   const uint16_t* b, int kk, auto&& copy) {
    const int ch = kk * 4 + g4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // every row of the next phase uses all eight dY fragments: they go out in rows 0-3.  In
      // those rows the bf16 instances read the row's W fragment (two transposing reads) after
      // the first MFMA, so no gap between MFMAs holds more than three other instructions (a
      // fourth costs the matrix core four cycles); the 4-bit ones spill with that order.
      if (i < 4) {
        nx.d[2 * i] = ld16(d + lds_offf(wm * 128 + 2 * i * 16 + l16, ch));
        nx.d[2 * i + 1] = ld16(d + lds_offf(wm * 128 + (2 * i + 1) * 16 + l16, ch));
      }
      if (INT4 || i >= 4) nx.w[i] = wfrag(w, kk, i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if constexpr (ASM) mfma16_acc(acc[i * 8 + j], cu.w[i], cu.d[j]);
        else acc[i * 8 + j] = mfma16(cu.w[i], cu.d[j], acc[i * 8 + j]);
        if (!INT4 && i < 4 && j == 0) {
          __builtin_amdgcn_sched_barrier(0);
          nx.w[i] = wfrag(w, kk, i);
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (!std::is_same_v<std::decay_t<decltype(copy)>, NoCopy>) {
          if (j == 1 || j == 5) {
            __builtin_amdgcn_sched_barrier(0);
            copy(2 * i + (j == 5));
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (PANEL) if (pan) {  // wave-uniform
#pragma unroll
      for (int c = 0; c < RP / 16; ++c) nx.b[c] = bfrag(b, kk, c);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 dp = wk ? cu.d[4 + j] : cu.d[j];
#pragma unroll
        for (int c = 0; c < RP / 16; ++c) pacc[c][j] = mfma16(cu.b[c], dp, pacc[c][j]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto read_frags = [&](Frag& f, const uint16_t* d, const uint16_t* w, const uint16_t* b, int kk) {
    const int ch = kk * 4 + g4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      f.w[i] = wfrag(w, kk, i);
      f.d[i] = ld16(d + lds_offf(wm * 128 + i * 16 + l16, ch));
    }
    if constexpr (PANEL)
      if (pan)
#pragma unroll
        for (int c = 0; c < RP / 16; ++c) f.b[c] = bfrag(b, kk, c);
  };
  // wait for the copies of the next step: for int4 W, the three register loads issued after
  // them stay in flight
  auto wait_all = [&]() {
    if constexpr (INT4) __builtin_amdgcn_s_waitcnt(0x0F73);  // vmcnt(3)
    else wait_vmem();
    __syncthreads();
  };
  auto prefetch = [&](int st, uint16_t* dn, uint16_t* wn, uint16_t* bn) {
    const int n0 = nbase + min(st, nsteps - 1) * kStep;
    dma_d(dn, n0);
    if constexpr (!INT4) dma_w(wn, n0);
    if constexpr (PANEL && BDMA) {
      if (pan) dma_b(bn, n0);
    } else if constexpr (PANEL) {
      if (pan) load_b(n0);
    }
    (void)bn;
  };
  // the same copies in 16 parts for phase(): the B rows first (a register load, waited for
  // at the next barrier, so it gets the longest time), then dY rows 8q.. (q < 8), W rows (bf16)
  // or the int4 register loads
  auto prefetch_part = [&](int q, int st, uint16_t* dn, uint16_t* wn, uint16_t* bn) {
    const int n0 = nbase + min(st, nsteps - 1) * kStep;
    if constexpr (PANEL && BDMA) {
      if (pan && q == 0) dma_b(bn, n0);
    } else if constexpr (PANEL) {
      if (pan && q == 0) load_b(n0);
    }
    (void)bn;
    if (q < 8) {
      dma16(rD, dn + (4 * q + wave) * 512, voffd_i(q), soffd_i(n0, q));
    } else if constexpr (!INT4) {
      const int i = q - 8;
      dma16(rW, wn + (i >> 1) * 4096 + ((i & 1) * 4 + wave) * 512, voffw_i(i), soffw_i(n0, i));
    }
  };
  const NoCopy nocopy;
  auto finish = [&](uint16_t* wn, uint16_t* bn) {  // register-staged parts of a prefetch (bf16)
    (void)wn;
    if constexpr (PANEL && !BDMA) {
      if (pan) store_b(bn);
    } else {
      (void)bn;
    }
  };
  auto finish_b = [&](uint16_t* bn) {
    if constexpr (PANEL && !BDMA) {
      if (pan) store_b(bn);
    } else {
      (void)bn;
    }
  };

  // Same pipeline as the forward kernel (see there), over N steps of 64.
  Frag f0, f1;
  prefetch(0, sD0, sW0, sB0);
  if constexpr (INT4) {
    load_w4(w4a, 0);
    if constexpr (AHEAD) load_w4(w4b, 1);
    store_w4(w4a, sW0);
  }
  finish(sW0, sB0);
  wait_vmem();
  __syncthreads();
  read_frags(f0, sD0, sW0, sB0, 0);
  prefetch(1, sD1, sW1, sB1);
  if constexpr (INT4) load_w4(w4a, AHEAD ? 2 : 1);

  // one N step on fixed buffers (c = this step's, o = the other; see the forward kernel)
  // w4n: the register set holding step st+1's int4 W (stored during the first half) and then
  // receiving the next load (issued after the copies of step st+2)
  auto step = [&](int st, W4& w4n, uint16_t* dc, uint16_t* wc, uint16_t* bc, uint16_t* dn,
                  uint16_t* wn, uint16_t* bn) {
    if constexpr (INT4) {  // the unpacked W of step st+1, spread between the MFMAs
      phase(f0, f1, dc, wc, bc, 1, [&](int d) { if (d % 2 == 0) store_w4_part(w4n, wn, d / 2); });
      finish_b(bn);
    } else {
      phase(f0, f1, dc, wc, bc, 1, nocopy);
      finish(wn, bn);  // the register-staged parts of step st+1
    }
    wait_all();
    phase(f1, f0, dn, wn, bn, 0, [&](int q) {
      prefetch_part(q, st + 2, dc, wc, bc);
      if constexpr (INT4)
        if (q == 15) load_w4(w4n, st + 3);  // after every copy
    });
  };
  int st = 0;
  W4& w4odd = AHEAD ? w4b : w4a;  // the set of odd steps
  // LDS reads drained at the loop edge (after the panel MFMAs that follow the last of them):
  // a known state at the loop head, where the compiler would otherwise wait for the reads it
  // has just issued
  __builtin_amdgcn_s_waitcnt(kLgkm0);
  for (; st + 2 <= nsteps; st += 2) {
    step(st, w4odd, sD0, sW0, sB0, sD1, sW1, sB1);
    step(st + 1, w4a, sD1, sW1, sB1, sD0, sW0, sB0);
    __builtin_amdgcn_s_waitcnt(kLgkm0);
  }
  if (st < nsteps) step(st, w4odd, sD0, sW0, sB0, sD1, sW1, sB1);
  // the A tile of the low-rank epilogue, loaded now so its latency overlaps the panel work
  // (rank 16, and the one-unit instances of rank 32; the others load it later: prefetching there
  // crashes the compiler)
  constexpr bool APRE = !NOADP && (RP <= 16 || (RP == 32 && !PERSIST));
  constexpr int AQ = APRE ? (RP * 32 + kThreads - 1) / kThreads : 1;
  u32x4 av[AQ];
  if constexpr (APRE) {
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
      const int c = q * kThreads + tid, rank = c >> 5, kc = c & 31;
      av[q] = (c < RP * 32 && rank < R && k0 + kc * 8 < K) ? ld16(A + (size_t)rank * K + k0 + kc * 8) : zero4();
    }
  }
  wait_vmem();
  __syncthreads();
  if constexpr (ASM) mfma_drain(acc);

  // ---- split N: store this unit's partial; the last unit of the tile adds them all ----
  // (the split count again from the tile, rather than kept live across the main loop)
  const int ns = splits + (tile < split_hi ? 1 : 0);
  if (ns > 1) {
    // partial slot: [wave][acc block][lane] f32x4, then (with a panel) the G panel [wave][block][lane]
    constexpr uint32_t kAccBytes = 4 * 64 * 64 * 16, kPanBytes = PANEL ? 4 * (RP / 16) * 4 * 64 * 16 : 0;
    constexpr uint32_t kSlot = kAccBytes + kPanBytes;
    static_assert(kSlot <= dx_slot_bytes(RP), "the host sizes the partials with dx_slot_bytes");
    const rsrc_t rP = make_rsrc(part + (size_t)tile * (splits + (split_hi > 0)) * (kSlot / 4), (uint32_t)ns * kSlot);
    const uint32_t wa = ((uint32_t)wave * 64 * 64 + lane) * 16u;
    const uint32_t wp = kAccBytes + ((uint32_t)wave * (RP / 16) * 4 * 64 + lane) * 16u;
    const uint32_t own = (uint32_t)sp * kSlot;
#pragma unroll
    for (int i = 0; i < 64; ++i) st_part(rP, own + wa + i * 1024u, acc[i]);
    if constexpr (PANEL)
#pragma unroll
      for (int c = 0; c < RP / 16; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) st_part(rP, own + wp + (c * 4 + j) * 1024u, pacc[c][j]);
    wait_vmem();
    __shared__ int s_last;
    __syncthreads();
    if (tid == 0)
      s_last = __hip_atomic_fetch_add(ctr + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               (uint32_t)(ns - 1);
    __syncthreads();
    if (!s_last) return;
    // fixed order: ((p0 + p1) + p2) + ..., p_sp from registers; 16 blocks of loads in flight
#pragma unroll
    for (int c0 = 0; c0 < 64; c0 += 16) {
      f32x4 tot[16];
      for (int q = 0; q < ns; ++q) {
        f32x4 v[16];
        if (q == sp) {
#pragma unroll
          for (int i = 0; i < 16; ++i) v[i] = acc[c0 + i];
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) v[i] = ld_part(rP, (uint32_t)q * kSlot + wa + (c0 + i) * 1024u);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) tot[i] = q == 0 ? v[i] : tot[i] + v[i];
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[c0 + i] = tot[i];
    }
    if constexpr (PANEL)
#pragma unroll
    for (int c = 0; c < RP / 16; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 t = fzero4();
        for (int q = 0; q < ns; ++q) {
          const f32x4 v = q == sp ? pacc[c][j] : ld_part(rP, (uint32_t)q * kSlot + wp + (c * 4 + j) * 1024u);
          t = q == 0 ? v : t + v;
        }
        pacc[c][j] = t;
      }
    if (tid == 0) __hip_atomic_store(ctr + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    panel_tm = -1;  // pacc now holds the sum over the splits, not this unit's share
  }

  if constexpr (!NOADP) {
  // ---- epilogue: G panel -> LDS (and HBM once per row tile); A tile -> LDS ----
  // The four freed tile buffers each take 64 rows of G (fp32, stride GS) followed by RP/4
  // rows of the A tile (bf16, stride AS; the 32-byte pad staggers the banks of the 4 rows a
  // transposing read touches).
  constexpr int GS = RP + 4;
  constexpr int AS = kTile + 16;
  constexpr int AR = RP / 4;                // A rows per buffer
  constexpr int GBYTES = 64 * GS * 4;
  static_assert(GBYTES + AR * AS * 2 <= TT * 2, "epilogue tiles must fit a freed buffer");
  auto buf = [&](int q) -> char* {
    return reinterpret_cast<char*>(q == 0 ? sD0 : (q == 1 ? sD1 : (q == 2 ? sW0 : sW1)));
  };
  auto grow = [&](int ml) -> float* { return reinterpret_cast<float*>(buf(ml >> 6)) + (ml & 63) * GS; };
  auto arow_ptr = [&](int r) -> uint16_t* {
    return reinterpret_cast<uint16_t*>(buf(r / AR) + GBYTES) + (r % AR) * AS;
  };
  if constexpr (PANEL) {
#pragma unroll
    for (int c = 0; c < RP / 16; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ml = wm * 128 + (wk * 4 + j) * 16 + l16;
        const int rk = c * 16 + g4 * 4;
        *reinterpret_cast<f32x4*>(grow(ml) + rk) = pacc[c][j];
        if (tk == 0 && m0 + ml < M && rk < R)
          *reinterpret_cast<f32x4*>(G + (size_t)(m0 + ml) * R + rk) = pacc[c][j];
      }
  } else {  // G from the panel pass (ranks >= R and tokens >= M as zeros)
    for (int e = tid; e < kTile * (RP / 4); e += kThreads) {
      const int ml = e / (RP / 4), rk = (e % (RP / 4)) * 4;
      const f32x4 v = (m0 + ml < M && rk < R) ? *reinterpret_cast<const f32x4*>(G + (size_t)(m0 + ml) * R + rk) : fzero4();
      *reinterpret_cast<f32x4*>(grow(ml) + rk) = v;
    }
  }
  if constexpr (APRE) {
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
      const int c = q * kThreads + tid, rank = c >> 5, kc = c & 31;
      if (c < RP * 32) st16(arow_ptr(rank) + kc * 8, av[q]);
    }
  } else {
    for (int c = tid; c < RP * 32; c += kThreads) {
      const int rank = c >> 5, kc = c & 31;
      const u32x4 v = (rank < R && k0 + kc * 8 < K) ? ld16(A + (size_t)rank * K + k0 + kc * 8) : zero4();
      st16(arow_ptr(rank) + kc * 8, v);
    }
  }
  __syncthreads();

#pragma unroll
  for (int c = 0; c < RP / 16; ++c) {
    const int rk = c * 16 + (g4 & 1) * 8;
    // A^T operand: lane (l16, g4) gets A[rk .. rk+7][k] for column k = l16 of its block
    const int arow = c * 16 + (g4 & 1) * 8 + (l16 >> 2);
    const uint16_t* a0 = arow_ptr(arow) + (l16 & 3) * 4;
    const uint16_t* a1 = arow_ptr(arow + 4) + (l16 & 3) * 4;
    u32x4 fat[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) fat[i] = join(ld_tr(a0 + wk * 128 + i * 16), ld_tr(a1 + wk * 128 + i * 16));
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float* src = grow(wm * 128 + j * 16 + l16) + rk;
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(src);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(src + 4);
      const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      u32x4 fg;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float h0, lo0, h1, lo1;
        split_bf16(scale * v[2 * e], h0, lo0);
        split_bf16(scale * v[2 * e + 1], h1, lo1);
        fg[e] = (g4 < 2) ? pack_bf16(h0, h1) : pack_bf16(lo0, lo1);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i * 8 + j] = mfma16(fat[i], fg, acc[i * 8 + j]);
    }
  }

  }

  // ---- store dX (one rounding), staged through this wave's freed tile buffer ----
  __syncthreads();  // every wave is done with G and A in LDS
  uint16_t* const stage = wave == 0 ? sD0 : (wave == 1 ? sD1 : (wave == 2 ? sW0 : sW1));
  const int mw = m0 + wm * 128, kw = k0 + wk * 128;
  store_block_bf16(acc, stage, dX + (size_t)mw * K + kw, (size_t)K, M - mw, K - kw, lane);
  };
  if constexpr (PERSIST) {
    for (int vb = blockIdx.x; vb < units; vb += gridDim.x) {
      unit_body(vb);
      __syncthreads();  // the next unit's copies reuse every wave's LDS
    }
  } else {
    unit_body(blockIdx.x);
  }
}

__global__ void zero_u32_kernel(uint32_t* p, int n) {  // the split arrival counters
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

template <int RP, bool INT4, bool FP4 = false, bool NOADP = false>
static hipError_t launch_dx_rp(const DxArgs& a, hipStream_t s) {
  const int tiles = dx_tiles(a.M, a.K);
  const int splits = dx_splits(a.M, a.N, a.K, a.R);
  const int split_hi = (FP4 && RP == 16) ? 0 : dx_split_hi(a.M, a.N, a.K, a.R);
  if (splits > 1) {
    hipLaunchKernelGGL(zero_u32_kernel, dim3((tiles + 255) / 256), dim3(256), 0, s, a.ctr, tiles);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int units = tiles * splits + split_hi, cus = device_cus() & ~7;  // a multiple of the 8 XCDs
  const int grid = (dx_persistent(RP, INT4) && cus > 0 && units > cus) ? cus : units;
  hipLaunchKernelGGL((dx_mfma_kernel<RP, INT4, FP4, NOADP>), dim3(grid), dim3(kThreads), 0, s,
                     (const uint16_t*)a.dY, a.W, (const uint16_t*)a.Ws, (const uint16_t*)a.A,
                     (const uint16_t*)a.B, (uint16_t*)a.dX, a.G, (int)a.M, (int)a.N, (int)a.K,
                     (int)a.R, a.scale, splits, split_hi, a.part, a.ctr);
  return hipGetLastError();
}

hipError_t launch_dx_mfma(const DxArgs& a, bool int4, hipStream_t s) {
  const int rp = a.R <= 16 ? 16 : (a.R <= 32 ? 32 : 64);
  if (int4 && a.fp4) {
    if (rp == 16) return launch_dx_rp<16, true, true>(a, s);
    if (rp == 32) return launch_dx_rp<32, true, true>(a, s);
    return launch_dx_rp<64, true, true>(a, s);
  }
  if (int4) {
    if (rp == 16) return launch_dx_rp<16, true>(a, s);
    if (rp == 32) return launch_dx_rp<32, true>(a, s);
    return launch_dx_rp<64, true>(a, s);
  }
  if (rp == 16) return launch_dx_rp<16, false>(a, s);
  if (rp == 32) return launch_dx_rp<32, false>(a, s);
  return launch_dx_rp<64, false>(a, s);
}

// dX = dY W alone (bf16, no adapter): the LM head's input gradient.  a.A, a.B and a.G are unused;
// a.ctr and a.part as for the rank-16 instance.
hipError_t launch_dx_noadapter(const DxArgs& a, hipStream_t s) { return launch_dx_rp<16, false, false, true>(a, s); }

}  // namespace lora
