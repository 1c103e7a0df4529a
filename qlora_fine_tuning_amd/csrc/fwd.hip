// Fused LoRA / QLoRA forward on gfx950 bf16 MFMA.
//
//   Y = X W^T + scale * (X A^T) B^T,   XA = X A^T saved (unscaled, fp32)
//
// tutorial ch. 5 "加速原理：Triton kernel 与 fused LoRA", §5.3: one program per output tile
// accumulates the base product and the low-rank product and stores Y once, so no
// intermediate reaches HBM.  Here one workgroup owns a 256 x 256 tile of Y:
//  * the K loop stages X, W and A tiles (64 wide) through double-buffered LDS;
//  * each wave accumulates a 128 x 128 block of Y^T on 16x16x32 bf16 MFMA (the W tile is
//    the row operand, so each lane ends up holding 4 consecutive outputs of one Y row);
//  * the same LDS X fragments feed the rank-R panel X A^T (each of the two waves that
//    share a 128-row X slice computes half of it: 6.25% extra MFMA work at R = 16);
//  * the epilogue puts scale * XA through LDS, splits it into bf16 hi + lo parts and adds
//    B (hi + lo)^T into the fp32 accumulators with one more MFMA per 16 ranks, then
//    rounds Y to bf16 once.
// QLoRA ("探微索隐：Unsloth 如何加速 LLM 推理？（以 Qwen 27B 为例）", §二.3): the W tile
// arrives as packed int4 codes plus one fp16 scale per 64 k; each thread unpacks its
// codes in registers to bf16_rne(q * s) on the way into LDS.
#include "common.hpp"
#include "launch.hpp"

namespace lora {

template <int RP, bool INT4>
__global__ void __launch_bounds__(kThreads)
fwd_mfma_kernel(const uint16_t* __restrict__ X, const void* __restrict__ Wp,
                const uint16_t* __restrict__ Wscale, const uint16_t* __restrict__ A,
                const uint16_t* __restrict__ Bm, uint16_t* __restrict__ Y,
                float* __restrict__ XA, int M, int N, int K, int R, float scale) {
  constexpr int TT = kTile * kStep;  // elements of one 256 x 64 operand tile
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * TT + 2 * RP * kStep];
  uint16_t* const sX = smem;           // [2][256 rows m][64 k]
  uint16_t* const sW = smem + 2 * TT;  // [2][256 rows n][64 k]
  uint16_t* const sA = smem + 4 * TT;  // [2][RP rows][64 k]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave >> 1, wm = wave & 1;  // this wave's 128-row half of n and of m
  const int l16 = lane & 15, g4 = lane >> 4;

  const int tiles_m = (M + kTile - 1) / kTile, tiles_n = (N + kTile - 1) / kTile;
  int tm, tn;
  grouped_tile(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, 8, tm, tn);
  const int m0 = tm * kTile, n0 = tn * kTile;
  const int nk = K / kStep;

  constexpr int AQ = (RP * 8 + kThreads - 1) / kThreads;  // 16-byte chunks of the A tile per thread
  u32x4 rx[8], rw[8], ra[AQ];
  float rs[2] = {0.f, 0.f};

  auto gload = [&](int kt) {
    const int k0 = kt * kStep;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = i * kThreads + tid, r = c >> 3, ch = c & 7;
      rx[i] = (m0 + r < M) ? ld16(X + (size_t)(m0 + r) * K + k0 + ch * 8) : zero4();
    }
    if constexpr (!INT4) {
      const uint16_t* W = static_cast<const uint16_t*>(Wp);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = i * kThreads + tid, r = c >> 3, ch = c & 7;
        rw[i] = (n0 + r < N) ? ld16(W + (size_t)(n0 + r) * K + k0 + ch * 8) : zero4();
      }
    } else {
      // one row per thread pair: thread (tid & 1) takes 32 of the row's 64 codes
      const uint8_t* Wq = static_cast<const uint8_t*>(Wp);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int n = n0 + q * 128 + (tid >> 1);
        if (n < N) {
          rw[q] = ld16(Wq + (size_t)n * (K / 2) + k0 / 2 + (tid & 1) * 16);
          rs[q] = half_bits_to_f32(Wscale[(size_t)n * (K / 64) + k0 / 64]);
        } else {
          rw[q] = zero4();
          rs[q] = 0.f;
        }
      }
    }
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
      const int c = q * kThreads + tid, r = c >> 3, ch = c & 7;
      ra[q] = (c < RP * 8 && r < R) ? ld16(A + (size_t)r * K + k0 + ch * 8) : zero4();
    }
  };

  auto sstore = [&](int buf) {
    uint16_t* x = sX + buf * TT;
    uint16_t* w = sW + buf * TT;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = i * kThreads + tid, r = c >> 3, ch = c & 7;
      st16(x + lds_off(r, ch), rx[i]);
    }
    if constexpr (!INT4) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = i * kThreads + tid, r = c >> 3, ch = c & 7;
        st16(w + lds_off(r, ch), rw[i]);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int r = q * 128 + (tid >> 1);
        const I4Scale sc = i4scale(rs[q]);
#pragma unroll
        for (int d = 0; d < 4; ++d)  // packed dword d = codes k = 8d .. 8d+7 of this half
          st16(w + lds_off(r, (tid & 1) * 4 + d), dequant8(rw[q][d], sc));
      }
    }
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
      const int c = q * kThreads + tid;
      if (c < RP * 8) st16(sA + buf * RP * kStep + lds_off(c >> 3, c & 7), ra[q]);
    }
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

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint16_t* x = sX + cur * TT;
    const uint16_t* w = sW + cur * TT;
    const uint16_t* a = sA + cur * RP * kStep;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ch = kk * 4 + g4;
      u32x4 fa[8], fb[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) fa[i] = ld16(w + lds_off(wn * 128 + i * 16 + l16, ch));
#pragma unroll
      for (int j = 0; j < 8; ++j) fb[j] = ld16(x + lds_off(wm * 128 + j * 16 + l16, ch));
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = mfma16(fa[i], fb[j], acc[i][j]);
#pragma unroll
      for (int c = 0; c < RP / 16; ++c) {
        const u32x4 pa = ld16(a + lds_off(c * 16 + l16, ch));
        if (wn == 0) {
#pragma unroll
          for (int j = 0; j < 4; ++j) pacc[c][j] = mfma16(pa, fb[j], pacc[c][j]);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) pacc[c][j] = mfma16(pa, fb[4 + j], pacc[c][j]);
        }
      }
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: XA panel -> LDS (and HBM once per row tile), then the rank-R update ----
  constexpr int XS = RP + 4;  // fp32 row stride of the panel in LDS
  float* const sXA = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int c = 0; c < RP / 16; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ml = wm * 128 + (wn * 4 + j) * 16 + l16;
      const int rk = c * 16 + g4 * 4;
      *reinterpret_cast<f32x4*>(sXA + ml * XS + rk) = pacc[c][j];
      if (XA != nullptr && tn == 0 && m0 + ml < M && rk < R)
        *reinterpret_cast<f32x4*>(XA + (size_t)(m0 + ml) * R + rk) = pacc[c][j];
    }
  __syncthreads();

#pragma unroll
  for (int c = 0; c < RP / 16; ++c) {
    const int rk = c * 16 + (g4 & 1) * 8;
    u32x4 fbm[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int n = n0 + wn * 128 + i * 16 + l16;
      fbm[i] = (n < N && rk < R) ? ld16(Bm + (size_t)n * R + rk) : zero4();
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float* src = sXA + (wm * 128 + j * 16 + l16) * XS + rk;
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
      for (int i = 0; i < 8; ++i) acc[i][j] = mfma16(fbm[i], fx, acc[i][j]);
    }
  }

  // ---- store Y (bf16, one rounding): lane holds Y[m][n .. n+3] ----
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int n = n0 + wn * 128 + i * 16 + g4 * 4;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int m = m0 + wm * 128 + j * 16 + l16;
      if (m < M && n < N) {
        const u32x2 o = {pack_bf16(acc[i][j][0], acc[i][j][1]), pack_bf16(acc[i][j][2], acc[i][j][3])};
        *reinterpret_cast<u32x2*>(Y + (size_t)m * N + n) = o;
      }
    }
  }
}

template <int RP, bool INT4>
static hipError_t launch_fwd_rp(const FwdArgs& a, hipStream_t s) {
  const int tiles = (int)(((a.M + kTile - 1) / kTile) * ((a.N + kTile - 1) / kTile));
  hipLaunchKernelGGL((fwd_mfma_kernel<RP, INT4>), dim3(tiles), dim3(kThreads), 0, s,
                     (const uint16_t*)a.X, a.W, (const uint16_t*)a.Ws, (const uint16_t*)a.A,
                     (const uint16_t*)a.B, (uint16_t*)a.Y, a.XA, (int)a.M, (int)a.N, (int)a.K,
                     (int)a.R, a.scale);
  return hipGetLastError();
}

hipError_t launch_fwd_mfma(const FwdArgs& a, bool int4, hipStream_t s) {
  const int rp = a.R <= 16 ? 16 : (a.R <= 32 ? 32 : 64);
  if (int4) {
    if (rp == 16) return launch_fwd_rp<16, true>(a, s);
    if (rp == 32) return launch_fwd_rp<32, true>(a, s);
    return launch_fwd_rp<64, true>(a, s);
  }
  if (rp == 16) return launch_fwd_rp<16, false>(a, s);
  if (rp == 32) return launch_fwd_rp<32, false>(a, s);
  return launch_fwd_rp<64, false>(a, s);
}

}  // namespace lora
