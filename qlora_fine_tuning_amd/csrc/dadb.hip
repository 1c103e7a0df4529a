// Adapter gradients as token-dimension split-K sums (tutorial ch. 5 "加速原理：Triton kernel
// 与 fused LoRA", §5.3, fused backward; hand-derived):
//
//   dA = scale * G^T X     (R x K),   G = dY B
//   dB = scale * dY^T XA   (N x R),   XA = X A^T (saved by the forward)
//
// Both are sums over tokens m of an outer product of a bf16 activation row (X or dY) with an
// fp32 rank-R row (G or XA).  Pass 1 gives every (256-column tile, 256-token split) pair to
// one workgroup, which writes its fp32 partial sum; pass 2 adds the partials of each
// element in split order.  No atomics, so results are bitwise reproducible.
//
// Pass 1 runs on bf16 MFMA.  The contraction index is the token m, along which the
// row-major activations are strided, so each thread transposes an 8 x 8 block in
// registers on the way into LDS.  The fp32 panel enters the MFMA as bf16 hi + lo parts
// (two MFMAs into one accumulator), keeping its fp32 accuracy.
#include "common.hpp"
#include "launch.hpp"

namespace lora {

static_assert(kDadbCols == kTile, "the host sizes the partial pass's grid with the tile width");

template <int RP>
__global__ void __launch_bounds__(kThreads)
dadb_partial_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ dY,
                    const float* __restrict__ G, const float* __restrict__ XA,
                    float* __restrict__ partA, float* __restrict__ partB,
                    int M, int N, int K, int R, int tilesA, int split_rows) {
  constexpr int TT = kTile * kStep;
  constexpr int PT = RP * kStep;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * TT + 4 * PT];
  uint16_t* const sQT = smem;              // [2][256 rows c][64 m]
  uint16_t* const sPh = smem + 2 * TT;     // [2][RP rows][64 m]  hi parts
  uint16_t* const sPl = sPh + 2 * PT;      // [2][RP rows][64 m]  lo parts

  const bool jobA = (int)blockIdx.x < tilesA;
  const uint16_t* const Q = jobA ? X : dY;
  const float* const P = jobA ? G : XA;
  float* const part = jobA ? partA : partB;
  const int C = jobA ? K : N;
  const int c0 = (jobA ? (int)blockIdx.x : (int)blockIdx.x - tilesA) * kTile;
  const int mbeg = (int)blockIdx.y * split_rows;
  const int mend = min(M, mbeg + split_rows);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;

  const int mb = tid >> 5, cb = tid & 31;  // 8 x 8 block: rows m = mb*8.., columns c = cb*8..
  const bool cin = c0 + cb * 8 < C;
  constexpr int BQ = RP / 4;
  const int pm = tid >> 2, pq = (tid & 3) * BQ;  // panel row m = pm, ranks pq .. pq+BQ-1

  u32x4 rq[8];
  float rp[BQ];

  auto gload = [&](int m0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int m = m0 + mb * 8 + j;
      rq[j] = (cin && m < mend) ? ld16(Q + (size_t)m * C + c0 + cb * 8) : zero4();
    }
    const int m = m0 + pm;
#pragma unroll
    for (int h = 0; h < BQ; h += 4) {
      const f32x4 v = (m < mend && pq + h < R) ? *reinterpret_cast<const f32x4*>(P + (size_t)m * R + pq + h)
                                               : fzero4();
      rp[h] = v[0];
      rp[h + 1] = v[1];
      rp[h + 2] = v[2];
      rp[h + 3] = v[3];
    }
  };
  auto sstore = [&](int buf) {
    uint16_t* qt = sQT + buf * TT;
    u32x4 cols[8];
    transpose8x8(rq, cols);
#pragma unroll
    for (int e = 0; e < 8; ++e) st16(qt + lds_off(cb * 8 + e, mb), cols[e]);
    uint16_t* ph = sPh + buf * PT;
    uint16_t* pl = sPl + buf * PT;
#pragma unroll
    for (int h = 0; h < BQ; ++h) {
      float hi, lo;
      split_bf16(rp[h], hi, lo);
      const int off = lds_off(pq + h, pm >> 3) + (pm & 7);
      ph[off] = (uint16_t)(__float_as_uint(hi) >> 16);
      pl[off] = (uint16_t)(pack_bf16(lo, 0.f) & 0xffffu);
    }
  };

  f32x4 acc[4][RP / 16];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < RP / 16; ++c) acc[i][c] = fzero4();

  const int nst = (mend - mbeg + kStep - 1) / kStep;
  if (nst > 0) {
    gload(mbeg);
    sstore(0);
  }
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int cur = st & 1;
    if (st + 1 < nst) gload(mbeg + (st + 1) * kStep);
    const uint16_t* qt = sQT + cur * TT;
    const uint16_t* ph = sPh + cur * PT;
    const uint16_t* pl = sPl + cur * PT;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ch = kk * 4 + g4;
      u32x4 fa[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = ld16(qt + lds_off(wave * 64 + i * 16 + l16, ch));
#pragma unroll
      for (int c = 0; c < RP / 16; ++c) {
        const u32x4 bh = ld16(ph + lds_off(c * 16 + l16, ch));
        const u32x4 bl = ld16(pl + lds_off(c * 16 + l16, ch));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[i][c] = mfma16(fa[i], bh, acc[i][c]);
          acc[i][c] = mfma16(fa[i], bl, acc[i][c]);
        }
      }
    }
    if (st + 1 < nst) sstore(cur ^ 1);
    __syncthreads();
  }

  // lane holds partial[c .. c+3][rank]; the partial is stored rank-major: part[split][rank][c]
  float* const out = part + (size_t)blockIdx.y * R * C;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = c0 + wave * 64 + i * 16 + g4 * 4;
#pragma unroll
    for (int cr = 0; cr < RP / 16; ++cr) {
      const int rank = cr * 16 + l16;
      if (rank < R && c < C) *reinterpret_cast<f32x4*>(out + (size_t)rank * C + c) = acc[i][cr];
    }
  }
}

// dA[rank][k] = scale * sum_s partA[s][rank][k];  dB[n][rank] = scale * sum_s partB[s][rank][n].
// One output per thread, consecutive threads on consecutive k (dA) or n (dB), so every split's
// loads are coalesced (dB is stored transposed, a small scattered write); the splits are added
// in split order, eight loads in flight at a time.
__global__ void __launch_bounds__(256)
dadb_reduce_kernel(const float* __restrict__ partA, const float* __restrict__ partB,
                   float* __restrict__ dA, float* __restrict__ dB, int N, int K, int R,
                   int splits, float scale) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nA = (int64_t)R * K, nB = (int64_t)R * N;
  const bool isA = t < nA;
  if (!isA && t >= nA + nB) return;
  const int64_t e = isA ? t : t - nA;       // A: rank * K + k;  B: rank * N + n
  const float* src = (isA ? partA : partB) + e;
  const int64_t stride = isA ? nA : nB;
  float s = 0.f;
  int sp = 0;
  for (; sp + 8 <= splits; sp += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[(int64_t)(sp + u) * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; sp < splits; ++sp) s += src[(int64_t)sp * stride];
  if (isA) {
    dA[e] = scale * s;
  } else {
    const int64_t r = e / N, n = e - r * N;
    dB[n * R + r] = scale * s;
  }
}

template <int RP>
static hipError_t launch_partials_rp(const DadbArgs& a, hipStream_t s) {
  const int tilesA = (int)((a.K + kTile - 1) / kTile);
  const int tilesB = (int)((a.N + kTile - 1) / kTile);
  hipLaunchKernelGGL((dadb_partial_kernel<RP>), dim3(tilesA + tilesB, a.splits), dim3(kThreads), 0, s,
                     (const uint16_t*)a.X, (const uint16_t*)a.dY, a.G, a.XA, a.partA, a.partB,
                     (int)a.M, (int)a.N, (int)a.K, a.R, tilesA, a.split_rows);
  return hipGetLastError();
}

hipError_t launch_dadb_partials_bf16(const DadbArgs& a, hipStream_t s) {
  if (a.splits == 0) return hipSuccess;
  if (a.R <= 16) return launch_partials_rp<16>(a, s);
  if (a.R <= 32) return launch_partials_rp<32>(a, s);
  return launch_partials_rp<64>(a, s);
}

hipError_t launch_dadb_reduce(const DadbArgs& a, hipStream_t s) {
  const int64_t total = (int64_t)a.R * (a.K + a.N);  // one output per thread
  const int blocks = (int)((total + 255) / 256);
  hipLaunchKernelGGL(dadb_reduce_kernel, dim3(blocks), dim3(256), 0, s, a.partA, a.partB, a.dA, a.dB,
                     (int)a.N, (int)a.K, a.R, a.splits, a.scale);
  return hipGetLastError();
}

}  // namespace lora
