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
  const I4Scale sc = i4scale(half_bits_to_f32(Ws[row * (K / 64) + kc / 2]));
  uint16_t* dst = Wout + row * K + kc * 32;
#pragma unroll
  for (int d = 0; d < 4; ++d) st16(dst + 8 * d, dequant8(w[d], sc));
}

// ---- decode matrix-vector product, M <= 8 --------------------------------------------
// Rows 0..N-1 of the partial-sum space are the int4 weight rows, rows N..N+RP-1 the adapter
// rows A (bf16), so X A^T is reduced by the same machinery as X W~^T.
// Grid: (row groups of 16*RBW rows, K splits).  Four waves split their workgroup's K range
// round-robin over 256-wide k blocks.  Per block a lane streams 32 contiguous bytes (64 codes,
// one scale group) of one row and feeds 8 bf16 MFMAs with the 16 tokens padded from M, so the
// dequantised values are consumed straight from registers.  The four waves' partial sums are
// added in LDS in wave order; splits are added in split order by the epilogue kernel.
constexpr int kGemvRows = 16;

template <int RBW>
__global__ void __launch_bounds__(256)
gemv_int4_kernel(const uint16_t* __restrict__ X, const uint8_t* __restrict__ Wq,
                 const uint16_t* __restrict__ Ws, const uint16_t* __restrict__ A,
                 float* __restrict__ part, int M, int N, int K, int R, int RP, int wgroups,
                 int kb_per_split) {
  __shared__ float sP[4][RBW * kGemvRows][8];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const int rg = blockIdx.x, ks = blockIdx.y;
  const bool adapter = rg >= wgroups;
  const int row0 = (adapter ? rg - wgroups : rg) * RBW * kGemvRows;
  const int NR = N + RP;
  const int kblocks = K / 256;
  const int kb0 = ks * kb_per_split, kb1 = min(kblocks, kb0 + kb_per_split);

  f32x4 acc[RBW];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) acc[rb] = fzero4();

  const bool xrow = l16 < M;
  for (int kb = kb0 + wave; kb < kb1; kb += 4) {
    const int kbase = kb * 256 + g4 * 64;
    u32x4 xf[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) xf[j] = xrow ? ld16(X + (size_t)l16 * K + kbase + j * 8) : zero4();
    if (!adapter) {
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) {
        const size_t row = (size_t)(row0 + rb * kGemvRows + l16);
        const uint8_t* p = Wq + row * (K / 2) + kbase / 2;
        const u32x4 w0 = ld16(p), w1 = ld16(p + 16);
        const I4Scale sc = i4scale(half_bits_to_f32(Ws[row * (K / 64) + kbase / 64]));
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[rb] = mfma16(dequant8(w0[j], sc), xf[j], acc[rb]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[rb] = mfma16(dequant8(w1[j], sc), xf[4 + j], acc[rb]);
      }
    } else {
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) {
        const int r = row0 + rb * kGemvRows + l16;
        const bool in = r < R;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const u32x4 af = in ? ld16(A + (size_t)r * K + kbase + j * 8) : zero4();
          acc[rb] = mfma16(af, xf[j], acc[rb]);
        }
      }
    }
  }

  // acc[rb][v] = partial sum for row rb*16 + 4*g4 + v and token l16
  if (l16 < 8) {
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) sP[wave][rb * kGemvRows + g4 * 4 + v][l16] = acc[rb][v];
  }
  __syncthreads();
  for (int e = tid; e < RBW * kGemvRows * 8; e += 256) {
    const int row = e >> 3, m = e & 7;
    const float s = ((sP[0][row][m] + sP[1][row][m]) + sP[2][row][m]) + sP[3][row][m];
    const int prow = adapter ? N + row0 + row : row0 + row;
    if ((adapter && row0 + row < RP) || (!adapter && prow < N))
      part[((size_t)ks * NR + prow) * 8 + m] = s;
  }
}

// Y[m][n] = bf16( sum_ks part[ks][n][m] + scale * sum_i XA[m][i] B[n][i] ),
// XA[m][i] = sum_ks part[ks][N + i][m].
__global__ void __launch_bounds__(256)
gemv_epilogue_kernel(const float* __restrict__ part, const uint16_t* __restrict__ Bm,
                     uint16_t* __restrict__ Y, float* __restrict__ XA, int M, int N, int R,
                     int RP, int ksplit, float scale) {
  __shared__ float sxa[8][64];
  const int tid = threadIdx.x;
  const int NR = N + RP;
  for (int e = tid; e < 8 * 64; e += 256) {
    const int m = e >> 6, i = e & 63;
    float s = 0.f;
    if (m < M && i < R)
      for (int ks = 0; ks < ksplit; ++ks) s += part[((size_t)ks * NR + N + i) * 8 + m];
    sxa[m][i] = s;
    if (XA != nullptr && blockIdx.x == 0 && m < M && i < R) XA[m * R + i] = s;
  }
  __syncthreads();
  const int n = blockIdx.x * 256 + tid;
  if (n >= N) return;
  float acc[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) acc[m] = 0.f;
  for (int ks = 0; ks < ksplit; ++ks) {
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(part + ((size_t)ks * NR + n) * 8);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(part + ((size_t)ks * NR + n) * 8 + 4);
    acc[0] += a0[0]; acc[1] += a0[1]; acc[2] += a0[2]; acc[3] += a0[3];
    acc[4] += a1[0]; acc[5] += a1[1]; acc[6] += a1[2]; acc[7] += a1[3];
  }
  float lora[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) lora[m] = 0.f;
  for (int i0 = 0; i0 < R; i0 += 8) {
    const u32x4 b = ld16(Bm + (size_t)n * R + i0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float b0 = bf16_lo(b[e]), b1 = bf16_hi(b[e]);
#pragma unroll
      for (int m = 0; m < 8; ++m) lora[m] += sxa[m][i0 + 2 * e] * b0 + sxa[m][i0 + 2 * e + 1] * b1;
    }
  }
  for (int m = 0; m < M; ++m) {
    const uint32_t o = pack_bf16(acc[m] + scale * lora[m], 0.f);
    Y[(size_t)m * N + n] = (uint16_t)(o & 0xffffu);
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

hipError_t launch_dequant_int4(int64_t N, int64_t K, const uint8_t* Wq, const uint16_t* Ws,
                               uint16_t* Wout, hipStream_t s) {
  const int64_t chunks = N * (K / 32);
  hipLaunchKernelGGL(dequant_int4_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s,
                     Wq, Ws, Wout, chunks, (int)K);
  return hipGetLastError();
}

// K splits of the decode product: the smallest divisor of the k-block count that gives at
// least 512 workgroups (two per CU), so that every CU keeps enough bytes in flight.
static int gemv_split(int64_t N, int64_t K) {
  const int kblocks = (int)(K / 256);
  const int64_t groups = N / (4 * kGemvRows);
  for (int d = 1; d <= kblocks; ++d)
    if (kblocks % d == 0 && groups * d >= 512) return d;
  return kblocks;
}

size_t gemv_workspace_floats(int64_t N, int64_t K, int R) {
  const int RP = R <= 16 ? 16 : (R <= 32 ? 32 : 64);
  return (size_t)gemv_split(N, K) * (size_t)(N + RP) * 8;
}

hipError_t launch_gemv_int4(const FwdArgs& a, float* part, hipStream_t s) {
  const int RP = a.R <= 16 ? 16 : (a.R <= 32 ? 32 : 64);
  const int ksplit = gemv_split(a.N, a.K);
  const int kblocks = (int)(a.K / 256);
  const int kbps = kblocks / ksplit;
  constexpr int RBW = 4;
  const int wgroups = (int)(a.N / (RBW * kGemvRows));
  const int agroups = (RP + RBW * kGemvRows - 1) / (RBW * kGemvRows);
  hipLaunchKernelGGL((gemv_int4_kernel<RBW>), dim3(wgroups + agroups, ksplit), dim3(256), 0, s,
                     (const uint16_t*)a.X, (const uint8_t*)a.W, (const uint16_t*)a.Ws,
                     (const uint16_t*)a.A, part, (int)a.M, (int)a.N, (int)a.K, a.R, RP, wgroups, kbps);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gemv_epilogue_kernel, dim3((unsigned)((a.N + 255) / 256)), dim3(256), 0, s,
                     (const float*)part, (const uint16_t*)a.B, (uint16_t*)a.Y, a.XA, (int)a.M, (int)a.N,
                     a.R, RP, ksplit, a.scale);
  return hipGetLastError();
}

}  // namespace lora
