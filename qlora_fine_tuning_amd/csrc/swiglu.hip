// SwiGLU gate/up pair with LoRA on both projections (tutorial ch. 5 §5.6 "fused SwiGLU": the
// gate's SiLU and the elementwise product with the up projection; §5.3's LoRA update on each
// projection; the backward derived by hand from L = <dH, H>).
//
// The two projections run as ONE LoRA GEMM over the stacked frozen weight [Wg; Wu] (2N x K),
// so each X tile is read once for both.  The adapters are stacked to match: A as [Ag; Au]
// (2R x K), B block-diagonally as [Bg 0; 0 Bu] (2N x 2R), so the rank-2R update gives the
// gate columns Bg (X Ag^T) and the up columns Bu (X Au^T) and nothing across.  The forward
// GEMM's epilogue (fwd.hip) pairs gate and up rows in each tile and writes H = silu(G) U next
// to [G | U] (bf16, kept for the backward).  The kernels here:
//  * swiglu_stack_kernel: assembles the stacked A and B (small, per call: A and B are trained);
//  * swiglu_bwd_kernel: [dG | dU] = [dH * U * silu'(G) | dH * silu(G)], the upstream gradient of
//    the stacked GEMM, whose LoRA backward (at 2N, 2R) gives dX and the stacked adapter
//    gradients;
//  * swiglu_unstack_kernel: splits those into dAg, dAu and the diagonal blocks dBg, dBu.
// silu(g) = g * sigmoid(g), silu'(g) = sigmoid(g) (1 + g (1 - sigmoid(g))), in fp32; each output
// is rounded to bf16 once.
#include "common.hpp"
#include "launch.hpp"

namespace lora {

// hardware exp2 and reciprocal (about 1 ulp of fp32 each; every output is rounded to bf16)
__device__ __forceinline__ float sigmoid_f(float g) { return __builtin_amdgcn_rcpf(1.f + __expf(-g)); }
__device__ __forceinline__ float bf16_at(const u32x4& v, int i) {
  const uint32_t w = v[i >> 1];
  return (i & 1) ? bf16_hi(w) : bf16_lo(w);
}

// As = [Ag; Au] (2R x K), Bs = [Bg 0; 0 Bu] (2N x 2R); one 16-byte chunk per thread (K and R are
// multiples of 8, so no chunk of Bs straddles the two rank blocks)
__global__ void __launch_bounds__(256)
swiglu_stack_kernel(const uint16_t* __restrict__ Ag, const uint16_t* __restrict__ Au,
                    const uint16_t* __restrict__ Bg, const uint16_t* __restrict__ Bu,
                    uint16_t* __restrict__ As, uint16_t* __restrict__ Bs, int64_t N, int64_t K, int R) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t na = (int64_t)2 * R * K / 8, nb = (int64_t)4 * N * R / 8;
  if (t < na) {
    const int64_t e = t * 8, r = e / K, k = e - r * K;
    st16(As + e, ld16(r < R ? Ag + r * K + k : Au + (r - R) * K + k));
  } else if (t < na + nb) {
    const int64_t e = (t - na) * 8, n = e / (2 * R), j = e - n * (2 * R);
    u32x4 v = zero4();
    if (n < N && j < R) v = ld16(Bg + n * R + j);
    else if (n >= N && j >= R) v = ld16(Bu + (n - N) * R + (j - R));
    st16(Bs + e, v);
  }
}

// dGU[m][n] = dH U silu'(G), dGU[m][N + n] = dH silu(G); 8 columns per thread
__global__ void __launch_bounds__(256)
swiglu_bwd_kernel(const uint16_t* __restrict__ dH, const uint16_t* __restrict__ GU,
                  uint16_t* __restrict__ dGU, int64_t M, int64_t N) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t cpr = N / 8;
  if (t >= M * cpr) return;
  const int64_t m = t / cpr, n = (t - m * cpr) * 8;
  const u32x4 d = ld16(dH + m * N + n);
  const u32x4 g = ld16(GU + m * 2 * N + n), u = ld16(GU + m * 2 * N + N + n);
  u32x4 dg, du;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    float vg[2], vu[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = 2 * p + h;
      const float gi = bf16_at(g, i), si = sigmoid_f(gi), di = bf16_at(d, i);
      vu[h] = di * gi * si;
      vg[h] = di * bf16_at(u, i) * (si * (1.f + gi * (1.f - si)));
    }
    dg[p] = pack_bf16(vg[0], vg[1]);
    du[p] = pack_bf16(vu[0], vu[1]);
  }
  st16(dGU + m * 2 * N + n, dg);
  st16(dGU + m * 2 * N + N + n, du);
}

// dAg = dAs[0:R], dAu = dAs[R:2R] (R x K each); dBg[n][r] = dBs[n][r], dBu[n][r] = dBs[N+n][R+r]
__global__ void __launch_bounds__(256)
swiglu_unstack_kernel(const float* __restrict__ dAs, const float* __restrict__ dBs, float* __restrict__ dAg,
                      float* __restrict__ dAu, float* __restrict__ dBg, float* __restrict__ dBu, int64_t N,
                      int64_t K, int R) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rk = (int64_t)R * K, nr = N * R;
  if (t < rk) {
    dAg[t] = dAs[t];
  } else if (t < 2 * rk) {
    dAu[t - rk] = dAs[t];
  } else if (t < 2 * rk + nr) {
    const int64_t e = t - 2 * rk, n = e / R, r = e - n * R;
    dBg[e] = dBs[n * 2 * R + r];
  } else if (t < 2 * rk + 2 * nr) {
    const int64_t e = t - 2 * rk - nr, n = e / R, r = e - n * R;
    dBu[e] = dBs[(N + n) * 2 * R + R + r];
  }
}

static unsigned blocks_for(int64_t threads) { return (unsigned)((threads + 255) / 256); }

hipError_t launch_swiglu_stack(const uint16_t* Ag, const uint16_t* Au, const uint16_t* Bg, const uint16_t* Bu,
                               uint16_t* As, uint16_t* Bs, int64_t N, int64_t K, int R, hipStream_t s) {
  const int64_t n = (int64_t)2 * R * K / 8 + (int64_t)4 * N * R / 8;
  hipLaunchKernelGGL(swiglu_stack_kernel, dim3(blocks_for(n)), dim3(256), 0, s, Ag, Au, Bg, Bu, As, Bs, N, K, R);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const uint16_t* dH, const uint16_t* GU, uint16_t* dGU, int64_t M, int64_t N,
                             hipStream_t s) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3(blocks_for(M * (N / 8))), dim3(256), 0, s, dH, GU, dGU, M, N);
  return hipGetLastError();
}

hipError_t launch_swiglu_unstack(const float* dAs, const float* dBs, float* dAg, float* dAu, float* dBg,
                                 float* dBu, int64_t N, int64_t K, int R, hipStream_t s) {
  const int64_t n = (int64_t)2 * R * K + (int64_t)2 * N * R;
  hipLaunchKernelGGL(swiglu_unstack_kernel, dim3(blocks_for(n)), dim3(256), 0, s, dAs, dBs, dAg, dAu, dBg, dBu,
                     N, K, R);
  return hipGetLastError();
}

}  // namespace lora
