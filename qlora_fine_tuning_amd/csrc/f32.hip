// fp32 LoRA layer (forward, input gradient, adapter-gradient partials), vector ALU.
//
// Same structure as the bf16 MFMA path (tutorial ch. 5 "加速原理：Triton kernel 与 fused
// LoRA", §5.3): each workgroup owns a 64 x 64 output tile, accumulates the rank-R panel from
// the same LDS tiles as the main product, and adds the low-rank term in its epilogue before
// one store.  Every product and sum is fp32.
#include "common.hpp"
#include "launch.hpp"

namespace lora {

constexpr int kF = 64;   // output tile edge
constexpr int kFk = 16;  // contraction step

// Y = X W^T + scale (X A^T) B^T;  thread (tx, ty) owns outputs m = ty + 16 i, n = tx + 16 j.
template <int RP>
__global__ void __launch_bounds__(256)
fwd_f32_kernel(const float* __restrict__ X, const float* __restrict__ W, const float* __restrict__ A,
               const float* __restrict__ B, float* __restrict__ Y, float* __restrict__ XA,
               int M, int N, int K, int R, float scale) {
  __shared__ float sX[kF][kFk + 1], sW[kF][kFk + 1], sA[RP][kFk + 1];
  __shared__ float sXA[kF][RP + 1], sB[kF][RP + 1];
  const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
  const int m0 = blockIdx.y * kF, n0 = blockIdx.x * kF;
  const int pm = t >> 2, pr = t & 3;  // panel row and rank phase: ranks pr + 4 q
  float acc[4][4] = {};
  float pacc[RP / 4] = {};
  for (int k0 = 0; k0 < K; k0 += kFk) {
    {
      const int r = t >> 2, c = (t & 3) * 4;
      const f32x4 xv = (m0 + r < M) ? *reinterpret_cast<const f32x4*>(X + (size_t)(m0 + r) * K + k0 + c)
                                    : fzero4();
      const f32x4 wv = *reinterpret_cast<const f32x4*>(W + (size_t)(n0 + r) * K + k0 + c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sX[r][c + e] = xv[e];
        sW[r][c + e] = wv[e];
      }
    }
    for (int e = t; e < RP * kFk; e += 256) {
      const int r = e / kFk, c = e % kFk;
      sA[r][c] = (r < R) ? A[(size_t)r * K + k0 + c] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kFk; ++kk) {
      float xv[4], wv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) xv[i] = sX[ty + 16 * i][kk];
#pragma unroll
      for (int j = 0; j < 4; ++j) wv[j] = sW[tx + 16 * j][kk];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(xv[i], wv[j], acc[i][j]);
      const float xp = sX[pm][kk];
#pragma unroll
      for (int q = 0; q < RP / 4; ++q) pacc[q] = fmaf(xp, sA[pr + 4 * q][kk], pacc[q]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int q = 0; q < RP / 4; ++q) {
    const int rank = pr + 4 * q;
    sXA[pm][rank] = pacc[q];
    if (XA != nullptr && blockIdx.x == 0 && m0 + pm < M && rank < R) XA[(size_t)(m0 + pm) * R + rank] = pacc[q];
  }
  for (int e = t; e < kF * RP; e += 256) {
    const int r = e / RP, c = e % RP;
    sB[r][c] = (c < R) ? B[(size_t)(n0 + r) * R + c] : 0.f;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = ty + 16 * i;
    if (m0 + m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = tx + 16 * j;
      float l = 0.f;
      for (int r = 0; r < RP; ++r) l = fmaf(sXA[m][r], sB[n][r], l);
      Y[(size_t)(m0 + m) * N + n0 + n] = acc[i][j] + l * scale;
    }
  }
}

// G = dY B;  dX = dY W + scale G A;  thread (tx, ty) owns outputs m = ty + 16 i, k = tx + 16 j.
template <int RP>
__global__ void __launch_bounds__(256)
dx_f32_kernel(const float* __restrict__ dY, const float* __restrict__ W, const float* __restrict__ A,
              const float* __restrict__ B, float* __restrict__ dX, float* __restrict__ G,
              int M, int N, int K, int R, float scale) {
  __shared__ float sDY[kF][kFk + 1], sW[kFk][kF + 1], sB[kFk][RP + 1];
  __shared__ float sG[kF][RP + 1], sA[RP][kF + 1];
  const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
  const int m0 = blockIdx.y * kF, k0 = blockIdx.x * kF;
  const int pm = t >> 2, pr = t & 3;
  float acc[4][4] = {};
  float pacc[RP / 4] = {};
  for (int n0 = 0; n0 < N; n0 += kFk) {
    {
      const int r = t >> 2, c = (t & 3) * 4;
      const f32x4 v = (m0 + r < M) ? *reinterpret_cast<const f32x4*>(dY + (size_t)(m0 + r) * N + n0 + c)
                                   : fzero4();
#pragma unroll
      for (int e = 0; e < 4; ++e) sDY[r][c + e] = v[e];
      const int rw = t >> 4, cw = (t & 15) * 4;
      const f32x4 w = *reinterpret_cast<const f32x4*>(W + (size_t)(n0 + rw) * K + k0 + cw);
#pragma unroll
      for (int e = 0; e < 4; ++e) sW[rw][cw + e] = w[e];
    }
    for (int e = t; e < kFk * RP; e += 256) {
      const int r = e / RP, c = e % RP;
      sB[r][c] = (c < R) ? B[(size_t)(n0 + r) * R + c] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int nn = 0; nn < kFk; ++nn) {
      float dv[4], wv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) dv[i] = sDY[ty + 16 * i][nn];
#pragma unroll
      for (int j = 0; j < 4; ++j) wv[j] = sW[nn][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(dv[i], wv[j], acc[i][j]);
      const float dp = sDY[pm][nn];
#pragma unroll
      for (int q = 0; q < RP / 4; ++q) pacc[q] = fmaf(dp, sB[nn][pr + 4 * q], pacc[q]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int q = 0; q < RP / 4; ++q) {
    const int rank = pr + 4 * q;
    sG[pm][rank] = pacc[q];
    if (blockIdx.x == 0 && m0 + pm < M && rank < R) G[(size_t)(m0 + pm) * R + rank] = pacc[q];
  }
  for (int e = t; e < RP * kF; e += 256) {
    const int r = e / kF, c = e % kF;
    sA[r][c] = (r < R) ? A[(size_t)r * K + k0 + c] : 0.f;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = ty + 16 * i;
    if (m0 + m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = tx + 16 * j;
      float l = 0.f;
      for (int r = 0; r < RP; ++r) l = fmaf(sG[m][r], sA[r][k], l);
      dX[(size_t)(m0 + m) * K + k0 + k] = acc[i][j] + scale * l;
    }
  }
}

// Partial sums over one 256-token split: part[s][rank][c] = sum_m Q[m][c] P[m][rank],
// (Q, P) = (X, G) for dA and (dY, XA) for dB.  Thread: column c = t & 63, ranks t >> 6 + 4 q.
template <int RP>
__global__ void __launch_bounds__(256)
dadb_partial_f32_kernel(const float* __restrict__ X, const float* __restrict__ dY,
                        const float* __restrict__ G, const float* __restrict__ XA,
                        float* __restrict__ partA, float* __restrict__ partB,
                        int M, int N, int K, int R, int tilesA) {
  const bool jobA = (int)blockIdx.x < tilesA;
  const float* const Q = jobA ? X : dY;
  const float* const P = jobA ? G : XA;
  float* const part = jobA ? partA : partB;
  const int C = jobA ? K : N;
  const int c = (jobA ? (int)blockIdx.x : (int)blockIdx.x - tilesA) * kF + (threadIdx.x & 63);
  const int rg = threadIdx.x >> 6;
  const int mbeg = (int)blockIdx.y * (int)kSplitRows, mend = min(M, mbeg + (int)kSplitRows);
  float acc[RP / 4] = {};
  for (int m = mbeg; m < mend; ++m) {
    const float qv = Q[(size_t)m * C + c];
#pragma unroll
    for (int q = 0; q < RP / 4; ++q) {
      const int rank = rg + 4 * q;
      if (rank < R) acc[q] = fmaf(qv, P[(size_t)m * R + rank], acc[q]);
    }
  }
#pragma unroll
  for (int q = 0; q < RP / 4; ++q) {
    const int rank = rg + 4 * q;
    if (rank < R) part[((size_t)blockIdx.y * R + rank) * C + c] = acc[q];
  }
}

template <int RP>
static hipError_t fwd_f32_rp(const FwdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((fwd_f32_kernel<RP>), dim3((unsigned)(a.N / kF), (unsigned)((a.M + kF - 1) / kF)),
                     dim3(256), 0, s, (const float*)a.X, (const float*)a.W, (const float*)a.A,
                     (const float*)a.B, (float*)a.Y, a.XA, (int)a.M, (int)a.N, (int)a.K, a.R, a.scale);
  return hipGetLastError();
}
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s) {
  if (a.R <= 16) return fwd_f32_rp<16>(a, s);
  if (a.R <= 32) return fwd_f32_rp<32>(a, s);
  return fwd_f32_rp<64>(a, s);
}

template <int RP>
static hipError_t dx_f32_rp(const DxArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((dx_f32_kernel<RP>), dim3((unsigned)(a.K / kF), (unsigned)((a.M + kF - 1) / kF)),
                     dim3(256), 0, s, (const float*)a.dY, (const float*)a.W, (const float*)a.A,
                     (const float*)a.B, (float*)a.dX, a.G, (int)a.M, (int)a.N, (int)a.K, a.R, a.scale);
  return hipGetLastError();
}
hipError_t launch_dx_f32(const DxArgs& a, hipStream_t s) {
  if (a.R <= 16) return dx_f32_rp<16>(a, s);
  if (a.R <= 32) return dx_f32_rp<32>(a, s);
  return dx_f32_rp<64>(a, s);
}

template <int RP>
static hipError_t partials_f32_rp(const DadbArgs& a, hipStream_t s) {
  const int tilesA = (int)(a.K / kF), tilesB = (int)(a.N / kF);
  hipLaunchKernelGGL((dadb_partial_f32_kernel<RP>), dim3(tilesA + tilesB, a.splits), dim3(256), 0, s,
                     (const float*)a.X, (const float*)a.dY, a.G, a.XA, a.partA, a.partB, (int)a.M,
                     (int)a.N, (int)a.K, a.R, tilesA);
  return hipGetLastError();
}
hipError_t launch_dadb_partials_f32(const DadbArgs& a, hipStream_t s) {
  if (a.splits == 0) return hipSuccess;
  if (a.R <= 16) return partials_f32_rp<16>(a, s);
  if (a.R <= 32) return partials_f32_rp<32>(a, s);
  return partials_f32_rp<64>(a, s);
}

}  // namespace lora
