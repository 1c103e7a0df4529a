// Fused LoRA / QLoRA input gradient on gfx950 bf16 MFMA.
//
//   G  = dY B                       (M x R, fp32, kept for the dA reduction)
//   dX = dY W + scale * G A         (M x K)
//
// tutorial ch. 5 "加速原理：Triton kernel 与 fused LoRA", §5.3 (the backward is fused as
// well); the gradient is derived by hand from Y = X W^T + scale X A^T B^T.  One workgroup
// owns a 256 (tokens) x 256 (k) tile of dX and loops over N, 64 at a time:
//  * dY tiles go to LDS as they are (n contiguous); W tiles are read n-major from HBM and
//    transposed 8 x 8 in registers on the way into LDS, so both MFMA operands are read
//    with 16-byte LDS loads along the contraction index n;
//  * the rank-R panel G = dY B is accumulated from the same LDS dY fragments;
//  * the epilogue adds A^T (scale G)^T with a bf16 hi + lo split of scale * G, then
//    rounds dX once.
// QLoRA: W arrives as packed int4 codes plus fp16 group scales ("探微索隐：Unsloth 如何加速
// LLM 推理？（以 Qwen 27B 为例）", §二.3); each thread unpacks an 8 (n) x 8 (k) block of
// codes directly into the transposed order, so no separate transpose is needed.
#include "common.hpp"
#include "launch.hpp"

namespace lora {

template <int RP, bool INT4>
__global__ void __launch_bounds__(kThreads)
dx_mfma_kernel(const uint16_t* __restrict__ dY, const void* __restrict__ Wp,
               const uint16_t* __restrict__ Wscale, const uint16_t* __restrict__ A,
               const uint16_t* __restrict__ Bm, uint16_t* __restrict__ dX,
               float* __restrict__ G, int M, int N, int K, int R, float scale) {
  constexpr int TT = kTile * kStep;
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * TT + 2 * RP * kStep];
  uint16_t* const sDY = smem;           // [2][256 rows m][64 n]
  uint16_t* const sWT = smem + 2 * TT;  // [2][256 rows k][64 n]
  uint16_t* const sBT = smem + 4 * TT;  // [2][RP rows][64 n]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wk = wave >> 1, wm = wave & 1;
  const int l16 = lane & 15, g4 = lane >> 4;

  const int tiles_m = (M + kTile - 1) / kTile, tiles_k = (K + kTile - 1) / kTile;
  int tm, tk;
  grouped_tile(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_k, 8, tm, tk);
  const int m0 = tm * kTile, k0 = tk * kTile;
  const int nsteps = N / kStep;

  // this thread's 8 x 8 block of the W tile: rows n = nb*8 .. +7, columns k = kb*8 .. +7
  const int nb = tid >> 5, kb = tid & 31;
  const bool kin = k0 + kb * 8 < K;
  // this thread's slice of the B tile: row n = tid >> 2, ranks bq .. bq + RP/4 - 1
  constexpr int BQ = RP / 4;
  const int bn = tid >> 2, bq = (tid & 3) * BQ;

  u32x4 rdy[8], rw[8];
  uint32_t rq[8];
  float rs[8];
  uint16_t rb[BQ];

  auto gload = [&](int st) {
    const int n0 = st * kStep;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = i * kThreads + tid, r = c >> 3, ch = c & 7;
      rdy[i] = (m0 + r < M) ? ld16(dY + (size_t)(m0 + r) * N + n0 + ch * 8) : zero4();
    }
    if constexpr (!INT4) {
      const uint16_t* W = static_cast<const uint16_t*>(Wp);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        rw[j] = kin ? ld16(W + (size_t)(n0 + nb * 8 + j) * K + k0 + kb * 8) : zero4();
    } else {
      const uint8_t* Wq = static_cast<const uint8_t*>(Wp);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const size_t n = (size_t)(n0 + nb * 8 + j);
        if (kin) {
          rq[j] = *reinterpret_cast<const uint32_t*>(Wq + n * (K / 2) + (k0 + kb * 8) / 2);
          rs[j] = half_bits_to_f32(Wscale[n * (K / 64) + (k0 + kb * 8) / 64]);
        } else {
          rq[j] = 0u;
          rs[j] = 0.f;
        }
      }
    }
#pragma unroll
    for (int h = 0; h < BQ; h += 4) {
      const bool in = bq + h < R;
      const u32x2 v = in ? *reinterpret_cast<const u32x2*>(Bm + (size_t)(n0 + bn) * R + bq + h)
                         : (u32x2){0u, 0u};
      rb[h + 0] = (uint16_t)(v[0] & 0xffffu);
      rb[h + 1] = (uint16_t)(v[0] >> 16);
      rb[h + 2] = (uint16_t)(v[1] & 0xffffu);
      rb[h + 3] = (uint16_t)(v[1] >> 16);
    }
  };

  auto sstore = [&](int buf) {
    uint16_t* dy = sDY + buf * TT;
    uint16_t* wt = sWT + buf * TT;
    uint16_t* bt = sBT + buf * RP * kStep;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = i * kThreads + tid, r = c >> 3, ch = c & 7;
      st16(dy + lds_off(r, ch), rdy[i]);
    }
    if constexpr (!INT4) {
      u32x4 cols[8];
      transpose8x8(rw, cols);
#pragma unroll
      for (int e = 0; e < 8; ++e) st16(wt + lds_off(kb * 8 + e, nb), cols[e]);
    } else {
      I4Word wd[8];
      I4Scale sc[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        wd[j] = i4word(rq[j]);
        sc[j] = i4scale(rs[j]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {  // column k = kb*8 + e, rows n = nb*8 + 2d, +1
        u32x4 o;
#pragma unroll
        for (int d = 0; d < 4; ++d)
          o[d] = pack_bf16(dq1(wd[2 * d], e, sc[2 * d]), dq1(wd[2 * d + 1], e, sc[2 * d + 1]));
        st16(wt + lds_off(kb * 8 + e, nb), o);
      }
    }
#pragma unroll
    for (int h = 0; h < BQ; ++h) bt[lds_off(bq + h, bn >> 3) + (bn & 7)] = rb[h];
  };

  f32x4 acc[8][8];
  f32x4 pacc[RP / 16][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = fzero4();
#pragma unroll
  for (int c = 0; c < RP / 16; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) pacc[c][j] = fzero4();

  gload(0);
  sstore(0);
  __syncthreads();

  for (int st = 0; st < nsteps; ++st) {
    const int cur = st & 1;
    if (st + 1 < nsteps) gload(st + 1);
    const uint16_t* dy = sDY + cur * TT;
    const uint16_t* wt = sWT + cur * TT;
    const uint16_t* bt = sBT + cur * RP * kStep;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ch = kk * 4 + g4;
      u32x4 fa[8], fb[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) fa[i] = ld16(wt + lds_off(wk * 128 + i * 16 + l16, ch));
#pragma unroll
      for (int j = 0; j < 8; ++j) fb[j] = ld16(dy + lds_off(wm * 128 + j * 16 + l16, ch));
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = mfma16(fa[i], fb[j], acc[i][j]);
#pragma unroll
      for (int c = 0; c < RP / 16; ++c) {
        const u32x4 pb = ld16(bt + lds_off(c * 16 + l16, ch));
        if (wk == 0) {
#pragma unroll
          for (int j = 0; j < 4; ++j) pacc[c][j] = mfma16(pb, fb[j], pacc[c][j]);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) pacc[c][j] = mfma16(pb, fb[4 + j], pacc[c][j]);
        }
      }
    }
    if (st + 1 < nsteps) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: G panel -> LDS (and HBM once per row tile); A^T tile -> LDS ----
  constexpr int GS = RP + 4;  // fp32 row stride of G in LDS
  constexpr int AS = RP + 8;  // bf16 row stride of A^T in LDS
  float* const sG = reinterpret_cast<float*>(smem);
  uint16_t* const sAT = reinterpret_cast<uint16_t*>(sG + kTile * GS);
#pragma unroll
  for (int c = 0; c < RP / 16; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ml = wm * 128 + (wk * 4 + j) * 16 + l16;
      const int rk = c * 16 + g4 * 4;
      *reinterpret_cast<f32x4*>(sG + ml * GS + rk) = pacc[c][j];
      if (tk == 0 && m0 + ml < M && rk < R)
        *reinterpret_cast<f32x4*>(G + (size_t)(m0 + ml) * R + rk) = pacc[c][j];
    }
  for (int c = tid; c < RP * 32; c += kThreads) {
    const int rank = c >> 5, kc = c & 31;
    const u32x4 v = (rank < R && k0 + kc * 8 < K) ? ld16(A + (size_t)rank * K + k0 + kc * 8) : zero4();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sAT[(kc * 8 + 2 * e) * AS + rank] = (uint16_t)(v[e] & 0xffffu);
      sAT[(kc * 8 + 2 * e + 1) * AS + rank] = (uint16_t)(v[e] >> 16);
    }
  }
  __syncthreads();

#pragma unroll
  for (int c = 0; c < RP / 16; ++c) {
    const int rk = c * 16 + (g4 & 1) * 8;
    u32x4 fat[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) fat[i] = ld16(sAT + (wk * 128 + i * 16 + l16) * AS + rk);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float* src = sG + (wm * 128 + j * 16 + l16) * GS + rk;
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
      for (int i = 0; i < 8; ++i) acc[i][j] = mfma16(fat[i], fg, acc[i][j]);
    }
  }

  // ---- store dX (one rounding): lane holds dX[m][k .. k+3] ----
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int k = k0 + wk * 128 + i * 16 + g4 * 4;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int m = m0 + wm * 128 + j * 16 + l16;
      if (m < M && k < K) {
        const u32x2 o = {pack_bf16(acc[i][j][0], acc[i][j][1]), pack_bf16(acc[i][j][2], acc[i][j][3])};
        *reinterpret_cast<u32x2*>(dX + (size_t)m * K + k) = o;
      }
    }
  }
}

template <int RP, bool INT4>
static hipError_t launch_dx_rp(const DxArgs& a, hipStream_t s) {
  const int tiles = (int)(((a.M + kTile - 1) / kTile) * ((a.K + kTile - 1) / kTile));
  hipLaunchKernelGGL((dx_mfma_kernel<RP, INT4>), dim3(tiles), dim3(kThreads), 0, s,
                     (const uint16_t*)a.dY, a.W, (const uint16_t*)a.Ws, (const uint16_t*)a.A,
                     (const uint16_t*)a.B, (uint16_t*)a.dX, a.G, (int)a.M, (int)a.N, (int)a.K,
                     (int)a.R, a.scale);
  return hipGetLastError();
}

hipError_t launch_dx_mfma(const DxArgs& a, bool int4, hipStream_t s) {
  const int rp = a.R <= 16 ? 16 : (a.R <= 32 ? 32 : 64);
  if (int4) {
    if (rp == 16) return launch_dx_rp<16, true>(a, s);
    if (rp == 32) return launch_dx_rp<32, true>(a, s);
    return launch_dx_rp<64, true>(a, s);
  }
  if (rp == 16) return launch_dx_rp<16, false>(a, s);
  if (rp == 32) return launch_dx_rp<32, false>(a, s);
  return launch_dx_rp<64, false>(a, s);
}

}  // namespace lora
