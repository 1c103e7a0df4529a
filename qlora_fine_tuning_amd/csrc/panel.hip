// The rank-R panel of the input gradient as a pass of its own, for ranks above 32:
//
//   G = dY B        (M x R, fp32)
//
// tutorial ch. 5 "加速原理：Triton kernel 与 fused LoRA", §5.3 (the LoRA backward; gradients
// derived by hand).  Up to rank 32 the input-gradient kernel computes G from the dY tiles it
// already holds; at rank 64 the panel's accumulators and operands no longer fit next to the
// main tile's, so G comes from here and the main kernel reads it in its epilogue.  The same
// kernels form the forward's XA = X A^T where the forward kernel goes without its panel (rank
// 64, and the rank-32 SwiGLU pair, whose many column tiles per row would each recompute it).
//
//  * bt_transpose_kernel: B (N x R, rank-contiguous) -> Bt (R x N), so that both MFMA operands
//    of the panel are contiguous along the contraction index n;
//  * panel_kernel: one workgroup per (128 tokens, share of N); each wave owns 32 tokens and the
//    ranks in 16-wide blocks (2 up to rank 32, else 4) and streams its dY rows and the Bt rows
//    straight from memory (no LDS: dY is read once, Bt is small and stays in L2), writing an
//    fp32 partial.  Two token blocks per wave halve the Bt loads per MFMA, and the next 128
//    columns' loads are in flight while the current ones are multiplied: at rank 64 the pass
//    takes ~10 us less at the attention shape than with 16 tokens per wave and no lookahead;
//  * panel_reduce_kernel: adds the partials in share order into G.
// The sums run in a fixed order: results are bitwise reproducible.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace lora {

constexpr int kPanelTB = 2;      // 16-token blocks per wave
constexpr int kPanelRows = 64 * kPanelTB;  // tokens per workgroup
constexpr int kPanelRanks = 64;  // ranks covered (R in 33..64; ranks >= R read as zero)

// Bt[r][n] = B[n][r]: a 64 x R block of B per workgroup through LDS.
__global__ void __launch_bounds__(256)
bt_transpose_kernel(const uint16_t* __restrict__ B, uint16_t* __restrict__ Bt, int N, int R) {
  __shared__ uint16_t tile[64][kPanelRanks + 2];
  const int n0 = blockIdx.x * 64, tid = threadIdx.x;
  for (int e = tid; e < 64 * R; e += 256) {
    const int n = e / R, r = e - n * R;
    tile[n][r] = B[(size_t)(n0 + n) * R + r];
  }
  __syncthreads();
  for (int e = tid; e < 64 * R; e += 256) {
    const int r = e >> 6, n = e & 63;
    Bt[(size_t)r * N + n0 + n] = tile[n][r];
  }
}

// out[s][m][r] = sum over c in share s of Q[m][c] * S[r][c]  (Q: M x C, S: R x C, bf16), rows
// of ldo floats: 64 for partials, or R when one share writes the panel itself (ranks < R only).
// Each wave owns TB blocks of 16 tokens and RB blocks of 16 ranks (RB = 2 up to rank 32): one
// 32-wide step loads TB token and RB rank fragments for TB x RB MFMAs, and the loads of the next
// four steps are in flight while the current four are multiplied.
template <int RB>
__global__ void __launch_bounds__(256)
panel_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ S, float* __restrict__ part,
             int M, int C, int R, int share, int ldo) {
  constexpr int TB = kPanelTB;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const int m0 = blockIdx.x * kPanelRows + wave * 16 * TB;
  const int cs = blockIdx.y;
  const int c0 = cs * share, c1 = min(C, c0 + share);
  const rsrc_t rQ = make_rsrc(Q + (size_t)m0 * C, (uint32_t)max(0, min(16 * TB, M - m0)) * (uint32_t)C * 2u);
  const rsrc_t rS = make_rsrc(S, (uint32_t)R * (uint32_t)C * 2u);
  const uint32_t qoff = ((uint32_t)l16 * (uint32_t)C + (uint32_t)(8 * g4)) * 2u;
  const uint32_t qrow16 = 16u * (uint32_t)C * 2u;  // 16 token rows
  f32x4 acc[RB][TB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[rb][t] = fzero4();
  struct Frags {
    u32x4 a[4][TB], s[4][RB];
  };
  auto load = [&](Frags& f, int c) {  // four 32-wide steps from column c
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int t = 0; t < TB; ++t) f.a[u][t] = bload16(rQ, qoff + (uint32_t)t * qrow16 + (uint32_t)(c + 32 * u) * 2u, 0);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        f.s[u][rb] = bload16(rS, ((uint32_t)(rb * 16 + l16) * (uint32_t)C + (uint32_t)(c + 32 * u + 8 * g4)) * 2u, 0);
    }
  };
  auto mma = [&](const Frags& f) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int t = 0; t < TB; ++t) acc[rb][t] = mfma16(f.s[u][rb], f.a[u][t], acc[rb][t]);
  };
  int c = c0;
  if (c + 128 <= c1) {
    Frags f0, f1;
    load(f0, c);
    for (; c + 256 <= c1; c += 256) {  // two 128-wide blocks per iteration, one in flight
      load(f1, c + 128);
      mma(f0);
      if (c + 384 <= c1) load(f0, c + 256);
      mma(f1);
    }
    if (c + 128 <= c1) {  // one block left, already loaded into f0
      mma(f0);
      c += 128;
    }
  }
  for (; c < c1; c += 32) {
    u32x4 a[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) a[t] = bload16(rQ, qoff + (uint32_t)t * qrow16 + (uint32_t)c * 2u, 0);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const u32x4 sv = bload16(rS, ((uint32_t)(rb * 16 + l16) * (uint32_t)C + (uint32_t)(c + 8 * g4)) * 2u, 0);
#pragma unroll
      for (int t = 0; t < TB; ++t) acc[rb][t] = mfma16(sv, a[t], acc[rb][t]);
    }
  }
  // acc[rb][t]: ranks rb*16 + 4 g4 .. +3 of token m0 + 16 t + l16
#pragma unroll
  for (int t = 0; t < TB; ++t) {
    const int m = m0 + 16 * t + l16;
    if (m < M) {
      float* dst = part + ((size_t)cs * M + m) * ldo;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        if (rb * 16 + 4 * g4 < ldo) *reinterpret_cast<f32x4*>(dst + rb * 16 + 4 * g4) = acc[rb][t];
    }
  }
}

// G[m][r] = sum_s part[s][m][r], s in order.
__global__ void __launch_bounds__(256)
panel_reduce_kernel(const float* __restrict__ part, float* __restrict__ G, int M, int R, int shares) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (int64_t)M * R) return;
  const int64_t m = e / R, r = e - m * R;
  const float* src = part + m * kPanelRanks + r;
  float s = 0.f;
  int q = 0;
  for (; q + 4 <= shares; q += 4) {
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = src[(int64_t)(q + u) * M * kPanelRanks];
#pragma unroll
    for (int u = 0; u < 4; ++u) s += v[u];
  }
  for (; q < shares; ++q) s += src[(int64_t)q * M * kPanelRanks];
  G[e] = s;
}

// Shares of N per 64-token block: enough workgroups to cover the chip twice, at least 256 wide.
int panel_shares(int64_t M, int64_t C) {
  const int64_t blocks = (M + kPanelRows - 1) / kPanelRows;
  int64_t s = std::max<int64_t>(1, (512 + blocks - 1) / blocks);
  s = std::min<int64_t>(s, std::max<int64_t>(1, C / 256));
  return (int)s;
}
static int64_t panel_share_len(int64_t C, int shares) { return ((C + shares - 1) / shares + 63) / 64 * 64; }

size_t panel_workspace_bytes(int64_t M, int64_t N, int R) {
  const int s = panel_shares(M, N);
  const size_t bt = ((size_t)R * N * 2 + 255) & ~(size_t)255;
  return bt + (size_t)s * M * kPanelRanks * 4;
}

hipError_t launch_panel_g(const uint16_t* dY, const uint16_t* B, float* G, void* ws, int64_t M, int64_t N,
                          int R, hipStream_t s) {
  const int shares = panel_shares(M, N);
  const int64_t len = panel_share_len(N, shares);
  const int used = (int)((N + len - 1) / len);
  uint16_t* Bt = static_cast<uint16_t*>(ws);
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + (((size_t)R * N * 2 + 255) & ~(size_t)255));
  hipLaunchKernelGGL(bt_transpose_kernel, dim3((unsigned)(N / 64)), dim3(256), 0, s, B, Bt, (int)N, R);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((M + kPanelRows - 1) / kPanelRows), (unsigned)used);
  if (R <= 32)
    hipLaunchKernelGGL(panel_kernel<2>, grid, dim3(256), 0, s, dY, Bt, part, (int)M, (int)N, R, (int)len, kPanelRanks);
  else
    hipLaunchKernelGGL(panel_kernel<4>, grid, dim3(256), 0, s, dY, Bt, part, (int)M, (int)N, R, (int)len, kPanelRanks);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t total = M * R;
  hipLaunchKernelGGL(panel_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part, G,
                     (int)M, R, used);
  return hipGetLastError();
}

// XA = X A^T (A is R x K, already contiguous along k).  The per-share partials go to `scratch`
// (scratch_bytes of it); with room for fewer than two shares, one share writes XA directly.
hipError_t launch_panel_xa(const uint16_t* X, const uint16_t* A, float* XA, void* scratch, size_t scratch_bytes,
                           int64_t M, int64_t K, int R, hipStream_t s) {
  int shares = panel_shares(M, K);
  const int64_t cap = (int64_t)(scratch_bytes / ((size_t)M * kPanelRanks * 4));
  if (cap < 2) shares = 1;
  shares = (int)std::min<int64_t>(shares, std::max<int64_t>(cap, 1));
  const int64_t len = panel_share_len(K, shares);
  const int used = (int)((K + len - 1) / len);
  const dim3 grid((unsigned)((M + kPanelRows - 1) / kPanelRows), (unsigned)used);
  auto run = [&](float* out, int ldo) {
    if (R <= 32)
      hipLaunchKernelGGL(panel_kernel<2>, grid, dim3(256), 0, s, X, A, out, (int)M, (int)K, R, (int)len, ldo);
    else
      hipLaunchKernelGGL(panel_kernel<4>, grid, dim3(256), 0, s, X, A, out, (int)M, (int)K, R, (int)len, ldo);
  };
  if (used == 1) {
    run(XA, R);
    return hipGetLastError();
  }
  float* part = static_cast<float*>(scratch);
  run(part, kPanelRanks);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t total = M * R;
  hipLaunchKernelGGL(panel_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part, XA,
                     (int)M, R, used);
  return hipGetLastError();
}

}  // namespace lora
