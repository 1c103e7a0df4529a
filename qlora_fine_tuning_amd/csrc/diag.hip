// Diagnostics for the measurement harness (not part of the layer).
//
//  * sclk_probe_kernel: the shader clock seen by a kernel.  One wave reads the shader-cycle
//    counter and the constant 100 MHz real-time counter, spins until the real-time counter has
//    advanced by `ticks` (10 ns each), and reads both again; the ratio of the deltas is the
//    average shader clock over the spin.  The spin ends on the real-time counter alone.
//  * mfma_rate_kernel: the matrix-core ceiling under the chip's own power limit.  Every wave
//    (one per SIMD: 256 threads per workgroup, all registers of the SIMD) issues `iters` blocks
//    of 64 independent v_mfma_f32_16x16x32_bf16 into 64 accumulators held in AGPRs, with no
//    other instruction in between, and records its shader cycles and real-time ticks.  The
//    MFMA rate it reaches bounds every bf16 GEMM on the same chip.
//  * mfma_issue_kernel<MODE>: the same MFMA stream (blocks of 64 in pairs) with other
//    instructions between the MFMAs, to measure what each kind costs the matrix core (MODE 0:
//    none).  A wave
//    issues one instruction per four cycles; a 16x16x32 MFMA occupies the matrix core for about
//    16, so about three other instructions fit behind each MFMA for free:
//      1, 2, 3: 2, 4, 6 s_nop after every MFMA;
//      4: 20 VALU operations (four independent fma chains) after one MFMA in every 8;
//      5: the same 20 spread, 3 after each of MFMAs 0-3 of a row of 8, 2 after each of 4-7;
//      6: the MFMAs' operands read from LDS, 2 reads of 16 bytes per lane per 8 MFMAs, each
//         used one block of 64 MFMAs later (so its latency is hidden);
//      7: one LDS DMA (buffer_load ... lds, 16 bytes per lane) per 8 MFMAs, to one of four
//         LDS destinations (M0 rewritten per copy), read from `out` itself through a buffer
//         resource of its size (reads past it return zeros; the copied words are never used).
//  * hbm_read_kernel: the streaming-read ceiling.  Each wave reads 1 KB contiguous per load
//    instruction (16 bytes per lane), four loads in flight per thread, grid-stride over the
//    buffer; the words are folded into a value that is stored only if it equals a fixed
//    constant (a zero-filled buffer folds to 0), so the loads cannot be removed and, in
//    practice, nothing is written.
#include "common.hpp"
#include "launch.hpp"

namespace lora {

__global__ void __launch_bounds__(64) sclk_probe_kernel(unsigned long long* out, unsigned int ticks) {
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  unsigned long long r1 = r0;
  while (r1 - r0 < ticks) r1 = __builtin_amdgcn_s_memrealtime();
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) {
    out[0] = c1 - c0;
    out[1] = r1 - r0;
  }
}

hipError_t launch_sclk_probe(unsigned long long* out, unsigned int ticks, hipStream_t s) {
  hipLaunchKernelGGL(sclk_probe_kernel, dim3(1), dim3(64), 0, s, out, ticks);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) mfma_rate_kernel(unsigned long long* out, unsigned int iters) {
  const int tid = threadIdx.x, lane = tid & 63;
  // operands: arbitrary finite bf16 patterns (small exponents), different per lane
  u32x4 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t x = 0x3f003f00u ^ ((uint32_t)(lane * 8 + i) * 0x00070007u & 0x007f007fu);
    a[i] = (u32x4){x, x ^ 0x00010001u, x ^ 0x00020002u, x ^ 0x00030003u};
    b[i] = (u32x4){x ^ 0x00040004u, x ^ 0x00050005u, x ^ 0x00060006u, x ^ 0x00070007u};
  }
  f32x4 acc[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) acc[i] = fzero4();
  mfma_acc_ready(acc);
  const unsigned long long c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (unsigned int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) mfma16_acc(acc[i * 8 + j], a[i], b[j]);
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  mfma_drain(acc);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 64; ++i) s += acc[i][0];
  if (lane == 0) {
    const size_t w = (size_t)blockIdx.x * 4 + (tid >> 6);
    out[3 * w + 0] = c1 - c0;
    out[3 * w + 1] = r1 - r0;
    out[3 * w + 2] = (unsigned long long)__float_as_uint(s);  // keeps the accumulators live
  }
}

hipError_t launch_mfma_rate(unsigned long long* out, int blocks, unsigned int iters, hipStream_t s) {
  hipLaunchKernelGGL(mfma_rate_kernel, dim3((unsigned)blocks), dim3(256), 0, s, out, iters);
  return hipGetLastError();
}

template <int MODE>
__global__ void __launch_bounds__(256) mfma_issue_kernel(unsigned long long* out, unsigned int iters,
                                                         uint32_t out_bytes) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[4096];  // 16 KB: read source, DMA target
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // operands: arbitrary finite bf16 patterns (small exponents), different per lane
  u32x4 a[2][8], b[2][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t x = 0x3f003f00u ^ ((uint32_t)(lane * 8 + i) * 0x00070007u & 0x007f007fu);
    a[0][i] = (u32x4){x, x ^ 0x00010001u, x ^ 0x00020002u, x ^ 0x00030003u};
    b[0][i] = (u32x4){x ^ 0x00040004u, x ^ 0x00050005u, x ^ 0x00060006u, x ^ 0x00070007u};
    a[1][i] = a[0][i];
    b[1][i] = b[0][i];
  }
  if constexpr (MODE == 6) {  // the LDS holds the same patterns: word w of row r of slot q
    for (int e = tid; e < 4096; e += 256) lds[e] = 0x3f003f00u ^ ((uint32_t)e * 0x00070007u & 0x007f007fu);
    __syncthreads();
  }
  const rsrc_t rs = make_rsrc(out, out_bytes);
  float vf[4] = {(float)lane, (float)wave, 1.f, 2.f};
  f32x4 acc[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) acc[i] = fzero4();
  mfma_acc_ready(acc);
  const unsigned long long c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (unsigned int it = 0; it < iters; ++it) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int cur = MODE == 6 ? blk : 0, nxt = 1 - cur;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (MODE == 6) {  // the next block's operands (16 reads per block, 1 KB each per wave)
          a[nxt][i] = ld16(&lds[((wave * 16 + i) & 15) * 256 + lane * 4]);
          b[nxt][i] = ld16(&lds[((wave * 16 + 8 + i) & 15) * 256 + lane * 4]);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          mfma16_acc(acc[i * 8 + j], a[cur][i], b[cur][j]);
          if constexpr (MODE == 1) asm volatile("s_nop 0\n\ts_nop 0");
          if constexpr (MODE == 2) asm volatile("s_nop 0\n\ts_nop 0\n\ts_nop 0\n\ts_nop 0");
          if constexpr (MODE == 3) asm volatile("s_nop 0\n\ts_nop 0\n\ts_nop 0\n\ts_nop 0\n\ts_nop 0\n\ts_nop 0");
          if constexpr (MODE == 4 || MODE == 5) {
            const int n = MODE == 4 ? (j == 1 ? 20 : 0) : (j < 4 ? 3 : 2);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q < n; ++q) vf[q & 3] = fmaf(vf[q & 3], 1.0001f, 0.5f);
            __builtin_amdgcn_sched_barrier(0);
          }
          if constexpr (MODE == 7) {
            if (j == 1) {
              __builtin_amdgcn_sched_barrier(0);
              dma16(rs, &lds[(wave * 4 + (i & 3)) * 256], (uint32_t)lane * 16u, 0u);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
      }
    }
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  mfma_drain(acc);
  if constexpr (MODE == 7) wait_vmem();
  float s = vf[0] + vf[1] + vf[2] + vf[3];
#pragma unroll
  for (int i = 0; i < 64; ++i) s += acc[i][0];
#pragma unroll
  for (int i = 0; i < 8; ++i) s += __uint_as_float(a[1][i][0] ^ b[1][i][1]);
  __syncthreads();  // every wave's copies into LDS and reads of `out` are done before the writes
  if (lane == 0) {
    const size_t w = (size_t)blockIdx.x * 4 + (tid >> 6);
    out[3 * w + 0] = c1 - c0;
    out[3 * w + 1] = r1 - r0;
    out[3 * w + 2] = (unsigned long long)__float_as_uint(s);  // keeps every result live
  }
}

hipError_t launch_mfma_issue(unsigned long long* out, int blocks, unsigned int iters, int mode, hipStream_t s) {
  const dim3 g((unsigned)blocks), t(256);
  const uint32_t bytes = (uint32_t)blocks * 4u * 3u * 8u;
  switch (mode) {
    case 0: hipLaunchKernelGGL(mfma_issue_kernel<0>, g, t, 0, s, out, iters, bytes); break;
    case 1: hipLaunchKernelGGL(mfma_issue_kernel<1>, g, t, 0, s, out, iters, bytes); break;
    case 2: hipLaunchKernelGGL(mfma_issue_kernel<2>, g, t, 0, s, out, iters, bytes); break;
    case 3: hipLaunchKernelGGL(mfma_issue_kernel<3>, g, t, 0, s, out, iters, bytes); break;
    case 4: hipLaunchKernelGGL(mfma_issue_kernel<4>, g, t, 0, s, out, iters, bytes); break;
    case 5: hipLaunchKernelGGL(mfma_issue_kernel<5>, g, t, 0, s, out, iters, bytes); break;
    case 6: hipLaunchKernelGGL(mfma_issue_kernel<6>, g, t, 0, s, out, iters, bytes); break;
    case 7: hipLaunchKernelGGL(mfma_issue_kernel<7>, g, t, 0, s, out, iters, bytes); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

constexpr uint32_t kReadMagic = 0x9e3779b9u;

__global__ void __launch_bounds__(256)
hbm_read_kernel(const u32x4* __restrict__ p, size_t n16, uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  uint32_t acc = 0;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 v0 = p[i], v1 = p[i + stride], v2 = p[i + 2 * stride], v3 = p[i + 3 * stride];
    acc ^= (v0[0] + v1[1]) ^ (v2[2] + v3[3]) ^ (v0[3] - v3[0]) ^ (v1[2] - v2[1]);
  }
  for (; i < n16; i += stride) acc ^= p[i][0] ^ p[i][2];
  if (acc == kReadMagic) sink[0] = acc;
}

hipError_t launch_hbm_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s) {
  const size_t n16 = bytes / 16;
  hipLaunchKernelGGL(hbm_read_kernel, dim3(2048), dim3(256), 0, s, static_cast<const u32x4*>(buf), n16, sink);
  return hipGetLastError();
}

}  // namespace lora
