// RMSNorm ahead of a LoRA projection (tutorial ch. 5 §5.4, fused RMSNorm: each row of the
// hidden state divided by the root of its mean square plus eps and scaled per feature by g, in
// one kernel that reads and writes the hidden state once).  The backward is derived by hand
// from L = <dY, Y>: with xh = x r,
//   dx_j = r (g_j dy_j - xh_j c),  c = (1/K) sum_k g_k dy_k xh_k,    dg_k = sum_m dy_mk xh_mk.
// Both directions are bound by HBM bandwidth: bf16 rows move as 16-byte chunks, consecutive
// lanes on consecutive chunks, every element of a row read once and written once.
//  * rmsnorm_fwd_kernel: one row per wave, held in registers between the sum of squares (a
//    butterfly over the wave, so every lane holds the same total) and the scaled store; the
//    reciprocal RMS r goes out for the backward.
//  * rmsnorm_bwd_kernel: one row per workgroup of 256 threads, so each thread keeps the same
//    columns from row to row: g stays in registers, and with DG the thread's dy * xh sums do
//    too, giving one dg partial per workgroup with no reduction across waves.  The row's dot
//    product is summed over the wave, then over the four waves through LDS in wave order.
//  * rmsnorm_dg_reduce_kernel: sums the workgroup partials in a fixed order.
#include "common.hpp"
#include "launch.hpp"

namespace lora {

constexpr int kNormThreads = 256;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;  // the same in every lane: each stage adds the same two operands in both partners
}

// Both kernels are persistent over rows (a grid of about two workgroups per CU, each wave or
// workgroup taking every stride-th row) and double-buffered: the next row's loads are issued
// before the current row is finished, so each wave keeps two rows of reads in flight.  Loads past
// the row's end (lanes without a chunk) or past the last row reread a valid chunk instead of
// being predicated, so no select waits on a prefetch; those values are discarded at use.

// CH: 16-byte chunks per lane (a row has K / 8 chunks; lane l takes chunks l, l + 64, ...); DB:
// double-buffered (the widest rows, 32 chunks per lane, hold one row at a time)
template <int CH, bool DB>
__global__ void __launch_bounds__(kNormThreads)
rmsnorm_fwd_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ g, uint16_t* __restrict__ Y,
                   float* __restrict__ r, int M, int K, float eps) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nch = K / 8, stride = gridDim.x * 4;
  auto load = [&](u32x4 (&x)[CH], int row) {
    const uint16_t* xr = X + (size_t)min(row, M - 1) * K;
#pragma unroll
    for (int c = 0; c < CH; ++c) x[c] = ld16(xr + min(c * 64 + lane, nch - 1) * 8);
  };
  auto finish = [&](u32x4 (&x)[CH], int row) {
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const bool in = c * 64 + lane < nch;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = in ? bf16_lo(x[c][e]) : 0.f, hi = in ? bf16_hi(x[c][e]) : 0.f;
        ss = fmaf(lo, lo, ss);
        ss = fmaf(hi, hi, ss);
      }
    }
    // only the packed row stays live across the reduction: the floats are unpacked again for
    // the store (one instruction each) instead of occupying 2 VGPRs per chunk element
#pragma unroll
    for (int c = 0; c < CH; ++c) asm volatile("" : "+v"(x[c]));
    ss = wave_sum(ss);
    const float rr = 1.f / sqrtf(ss / (float)K + eps);
    uint16_t* yr = Y + (size_t)row * K;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int ci = c * 64 + lane;
      if (ci < nch) {
        const u32x4 gv = ld16(g + ci * 8);
        u32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          y[e] = pack_bf16(bf16_lo(x[c][e]) * rr * bf16_lo(gv[e]), bf16_hi(x[c][e]) * rr * bf16_hi(gv[e]));
        st16(yr + ci * 8, y);
      }
    }
    if (lane == 0) r[row] = rr;
  };
  int row = blockIdx.x * 4 + wave;
  u32x4 xa[CH];
  if (row < M) load(xa, row);
  if constexpr (DB) {
    u32x4 xb[CH];
    for (; row < M; row += 2 * stride) {
      const bool more = row + stride < M;
      if (more) load(xb, row + stride);
      finish(xa, row);
      if (!more) break;
      if (row + 2 * stride < M) load(xa, row + 2 * stride);
      finish(xb, row + stride);
    }
  } else {
    for (; row < M; row += stride) {
      finish(xa, row);
      if (row + stride < M) load(xa, row + stride);
    }
  }
}

// CW: 16-byte chunks per thread (thread t takes chunks t, t + 256, ...); DG: accumulate the
// workgroup's dg partial into part[blockIdx.x][K]
template <int CW, bool DG>
__global__ void __launch_bounds__(kNormThreads)
rmsnorm_bwd_kernel(const uint16_t* __restrict__ dY, const uint16_t* __restrict__ X, const uint16_t* __restrict__ g,
                   const float* __restrict__ r, uint16_t* __restrict__ dX, float* __restrict__ part, int M, int K) {
  __shared__ float sdot[2][4];  // two slots: a row's slot is rewritten only two rows later
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = K / 8;
  u32x4 gv[CW];
#pragma unroll
  for (int c = 0; c < CW; ++c) gv[c] = ld16(g + min(c * kNormThreads + tid, nch - 1) * 8);
  float dga[DG ? CW : 1][8];
#pragma unroll
  for (int c = 0; c < (DG ? CW : 1); ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) dga[c][e] = 0.f;

  struct Row {
    u32x4 dy[CW], x[CW];
  };
  auto load = [&](Row& b, int row) {
    const size_t off = (size_t)min(row, M - 1) * K;
#pragma unroll
    for (int c = 0; c < CW; ++c) {
      const int ci = min(c * kNormThreads + tid, nch - 1);
      b.dy[c] = ld16(dY + off + ci * 8);
      b.x[c] = ld16(X + off + ci * 8);
    }
  };
  int slot = 0;
  auto finish = [&](Row& b, int row) {
    // g is unpacked afresh for each row rather than held as floats across the loop
#pragma unroll
    for (int c = 0; c < CW; ++c) asm volatile("" : "+v"(gv[c]));
    const float rr = r[row];
    float dot = 0.f;
#pragma unroll
    for (int c = 0; c < CW; ++c) {
      const bool in = c * kNormThreads + tid < nch;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pl = bf16_lo(gv[c][e]) * bf16_lo(b.dy[c][e]), ph = bf16_hi(gv[c][e]) * bf16_hi(b.dy[c][e]);
        dot = fmaf(in ? pl : 0.f, bf16_lo(b.x[c][e]) * rr, dot);
        dot = fmaf(in ? ph : 0.f, bf16_hi(b.x[c][e]) * rr, dot);
      }
    }
#pragma unroll
    for (int c = 0; c < CW; ++c) asm volatile("" : "+v"(b.dy[c]), "+v"(b.x[c]), "+v"(gv[c]));
    dot = wave_sum(dot);
    if (lane == 0) sdot[slot][wave] = dot;
    __syncthreads();
    const float cc = (((sdot[slot][0] + sdot[slot][1]) + sdot[slot][2]) + sdot[slot][3]) / (float)K;
    slot ^= 1;
    uint16_t* dxr = dX + (size_t)row * K;
#pragma unroll
    for (int c = 0; c < CW; ++c) {
      const int ci = c * kNormThreads + tid;
      if (ci < nch) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float xl = bf16_lo(b.x[c][e]) * rr, xh = bf16_hi(b.x[c][e]) * rr;
          const float dl = bf16_lo(b.dy[c][e]), dh = bf16_hi(b.dy[c][e]);
          v[2 * e] = rr * (bf16_lo(gv[c][e]) * dl - xl * cc);
          v[2 * e + 1] = rr * (bf16_hi(gv[c][e]) * dh - xh * cc);
          if constexpr (DG) {
            dga[c][2 * e] = fmaf(dl, xl, dga[c][2 * e]);
            dga[c][2 * e + 1] = fmaf(dh, xh, dga[c][2 * e + 1]);
          }
        }
        const u32x4 o = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]),
                         pack_bf16(v[6], v[7])};
        st16(dxr + ci * 8, o);
      }
    }
  };
  Row ba, bb;
  int row = blockIdx.x;  // < M: the grid never exceeds M
  load(ba, row);
  for (; row < M; row += 2 * gridDim.x) {
    const bool more = row + (int)gridDim.x < M;
    if (more) load(bb, row + gridDim.x);
    finish(ba, row);
    if (!more) break;
    if (row + 2 * (int)gridDim.x < M) load(ba, row + 2 * gridDim.x);
    finish(bb, row + gridDim.x);
  }
  if constexpr (DG) {
    float* pr = part + (size_t)blockIdx.x * K;
#pragma unroll
    for (int c = 0; c < CW; ++c) {
      const int ci = c * kNormThreads + tid;
      if (ci < nch) {
        *reinterpret_cast<f32x4*>(pr + ci * 8) = (f32x4){dga[c][0], dga[c][1], dga[c][2], dga[c][3]};
        *reinterpret_cast<f32x4*>(pr + ci * 8 + 4) = (f32x4){dga[c][4], dga[c][5], dga[c][6], dga[c][7]};
      }
    }
  }
}

// dg from the P workgroup partials in a fixed order, in two levels: slice s of kDgSlice partials
// (in order) for 256 columns per workgroup into part2[s][K], then the slices in order.
constexpr int kDgSlice = 32;

__global__ void __launch_bounds__(kNormThreads)
rmsnorm_dg_slices_kernel(const float* __restrict__ part, float* __restrict__ part2, int P, int K) {
  const int k = blockIdx.x * kNormThreads + threadIdx.x;
  const int p0 = blockIdx.y * kDgSlice, n = min(kDgSlice, P - p0);
  if (k >= K) return;
  float v[kDgSlice];
#pragma unroll
  for (int i = 0; i < kDgSlice; ++i) v[i] = i < n ? part[(size_t)(p0 + i) * K + k] : 0.f;
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < kDgSlice; ++i) acc += v[i];
  part2[(size_t)blockIdx.y * K + k] = acc;
}

// at most kDgMaxSlices slices (512 partials): all loads issued at once, then added in order
constexpr int kDgMaxSlices = 16;

__global__ void __launch_bounds__(kNormThreads)
rmsnorm_dg_final_kernel(const float* __restrict__ part2, float* __restrict__ dg, int S, int K) {
  const int k = blockIdx.x * kNormThreads + threadIdx.x;
  if (k >= K) return;
  float v[kDgMaxSlices];
#pragma unroll
  for (int s = 0; s < kDgMaxSlices; ++s) v[s] = s < S ? part2[(size_t)s * K + k] : 0.f;
  float acc = 0.f;
#pragma unroll
  for (int s = 0; s < kDgMaxSlices; ++s) acc += v[s];
  dg[k] = acc;
}

// Persistent grids: the workgroups resident at once on 256 CUs (per CU: 4 where a wave needs at
// most 128 VGPRs, 2 up to 256, else 1), never more than there are rows to share out.
template <int CH>
static hipError_t launch_fwd_ch(const uint16_t* X, const uint16_t* g, uint16_t* Y, float* r, int64_t M, int64_t K,
                                float eps, hipStream_t s) {
  constexpr bool DB = CH <= 16;
  const int64_t cap = (int64_t)kNormCUs * (CH <= 8 ? 4 : (CH <= 16 ? 2 : 1));
  const int64_t groups = (M + 3) / 4;
  const unsigned grid = (unsigned)(groups < cap ? groups : cap);
  hipLaunchKernelGGL((rmsnorm_fwd_kernel<CH, DB>), dim3(grid), dim3(kNormThreads), 0, s, X, g, Y, r, (int)M,
                     (int)K, eps);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_fwd(const uint16_t* X, const uint16_t* g, uint16_t* Y, float* r, int64_t M, int64_t K,
                              float eps, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int64_t ch = (K / 8 + 63) / 64;  // chunks per lane
  if (ch <= 1) return launch_fwd_ch<1>(X, g, Y, r, M, K, eps, s);
  if (ch <= 2) return launch_fwd_ch<2>(X, g, Y, r, M, K, eps, s);
  if (ch <= 4) return launch_fwd_ch<4>(X, g, Y, r, M, K, eps, s);
  if (ch <= 8) return launch_fwd_ch<8>(X, g, Y, r, M, K, eps, s);
  if (ch <= 12) return launch_fwd_ch<12>(X, g, Y, r, M, K, eps, s);
  if (ch <= 16) return launch_fwd_ch<16>(X, g, Y, r, M, K, eps, s);
  return launch_fwd_ch<32>(X, g, Y, r, M, K, eps, s);
}

// chunks per thread of the backward (one row per workgroup)
static int64_t bwd_chunks(int64_t K) { return (K / 8 + kNormThreads - 1) / kNormThreads; }

// With dg the grid is also the number of partials: half the resident count keeps their traffic
// small (8 MB at K = 4096).
int rmsnorm_bwd_grid(int64_t M, int64_t K, bool dg) {
  const bool wide = bwd_chunks(K) > 4;
  const int64_t cap = (int64_t)kNormCUs * (dg ? (wide ? 1 : 2) : (wide ? 2 : 4));
  return (int)(M < cap ? M : cap);
}
static_assert(kNormCUs * 2 <= kDgSlice * kDgMaxSlices, "dg partials beyond the final kernel's slices");

size_t rmsnorm_bwd_part_floats(int64_t M, int64_t K) {
  const int64_t P = rmsnorm_bwd_grid(M, K, true);
  return (size_t)(P + (P + kDgSlice - 1) / kDgSlice) * (size_t)K;
}

// dg = sum of the P partials: slices of kDgSlice into part2 (after the partials), then the slices
static hipError_t launch_dg_reduce(const float* part, float* dg, int P, int64_t K, hipStream_t s) {
  const int S = (P + kDgSlice - 1) / kDgSlice;
  float* part2 = const_cast<float*>(part) + (size_t)P * K;
  const unsigned cols = (unsigned)((K + kNormThreads - 1) / kNormThreads);
  if (S > 0) {
    hipLaunchKernelGGL(rmsnorm_dg_slices_kernel, dim3(cols, (unsigned)S), dim3(kNormThreads), 0, s, part, part2, P,
                       (int)K);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(rmsnorm_dg_final_kernel, dim3(cols), dim3(kNormThreads), 0, s, part2, dg, S, (int)K);
  return hipGetLastError();
}

template <int CW>
static hipError_t launch_bwd_cw(const uint16_t* dY, const uint16_t* X, const uint16_t* g, const float* r,
                                uint16_t* dX, float* dg, float* part, int64_t M, int64_t K, hipStream_t s) {
  const int grid = rmsnorm_bwd_grid(M, K, dg != nullptr);
  if (dg == nullptr) {
    hipLaunchKernelGGL((rmsnorm_bwd_kernel<CW, false>), dim3(grid), dim3(kNormThreads), 0, s, dY, X, g, r, dX,
                       nullptr, (int)M, (int)K);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((rmsnorm_bwd_kernel<CW, true>), dim3(grid), dim3(kNormThreads), 0, s, dY, X, g, r, dX, part,
                     (int)M, (int)K);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_dg_reduce(part, dg, grid, K, s);
}

hipError_t launch_rmsnorm_bwd(const uint16_t* dY, const uint16_t* X, const uint16_t* g, const float* r, uint16_t* dX,
                              float* dg, float* part, int64_t M, int64_t K, hipStream_t s) {
  if (M == 0) {  // an empty sum: dg = 0 (no partials are read)
    if (dg == nullptr) return hipSuccess;
    hipLaunchKernelGGL(rmsnorm_dg_final_kernel, dim3((unsigned)((K + kNormThreads - 1) / kNormThreads)),
                       dim3(kNormThreads), 0, s, part, dg, 0, (int)K);
    return hipGetLastError();
  }
  const int64_t cw = bwd_chunks(K);
  if (cw <= 1) return launch_bwd_cw<1>(dY, X, g, r, dX, dg, part, M, K, s);
  if (cw <= 2) return launch_bwd_cw<2>(dY, X, g, r, dX, dg, part, M, K, s);
  if (cw <= 3) return launch_bwd_cw<3>(dY, X, g, r, dX, dg, part, M, K, s);
  if (cw <= 4) return launch_bwd_cw<4>(dY, X, g, r, dX, dg, part, M, K, s);
  return launch_bwd_cw<8>(dY, X, g, r, dX, dg, part, M, K, s);
}

}  // namespace lora
