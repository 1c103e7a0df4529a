// RoPE on the projections' outputs (tutorial ch. 5 §5.5, fused RoPE: every coordinate pair of q and
// k rotated in one kernel, in place, with no sliced copies or concatenation).  Pairs (x_j, x_{j+rot/2})
// for j < rot/2, the angle pos * base^(-2j/rot); coordinates rot .. D-1 pass through untouched.
// The backward is the same kernel with the angle negated (the rotation's transpose).
//
// One workgroup per token: the token's rot/2 (cos, sin) pairs are computed once into LDS (fp32,
// sincosf with full range reduction: angles reach ~1e4 rad), then every Q and K head of the token is
// rotated in 16-byte chunk pairs (8 pairs per thread and item), each value rounded to bf16 once.
// Bound by HBM: every rotated element is read and written once.
#include "common.hpp"
#include "launch.hpp"

namespace lora {

__global__ void __launch_bounds__(256)
rope_kernel(uint16_t* __restrict__ Q, uint16_t* __restrict__ Kt, const int32_t* __restrict__ pos, int H, int Hk, int D,
            int rot, float base, float sign) {
  __shared__ float2 sc[kRopeMaxPairs];
  const int t = blockIdx.x, tid = threadIdx.x;
  const int h2 = rot / 2;
  const float p = (float)pos[t];
  for (int j = tid; j < h2; j += 256) {
    const float inv = powf(base, -2.f * (float)j / (float)rot);
    float sn, cs;
    sincosf(p * inv, &sn, &cs);
    sc[j] = make_float2(cs, sign * sn);
  }
  __syncthreads();
  const int cph = h2 / 8;  // chunk pairs per head
  const int items = (H + Hk) * cph;
  for (int it = tid; it < items; it += 256) {
    const int head = it / cph, c = it - head * cph;
    uint16_t* row = head < H ? Q + ((size_t)t * H + head) * D : Kt + ((size_t)t * Hk + (head - H)) * D;
    const u32x4 a = ld16(row + c * 8), b = ld16(row + h2 + c * 8);
    u32x4 ra, rb;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float2 s0 = sc[c * 8 + 2 * e], s1 = sc[c * 8 + 2 * e + 1];
      const float a0 = bf16_lo(a[e]), a1 = bf16_hi(a[e]), b0 = bf16_lo(b[e]), b1 = bf16_hi(b[e]);
      ra[e] = pack_bf16(a0 * s0.x - b0 * s0.y, a1 * s1.x - b1 * s1.y);
      rb[e] = pack_bf16(b0 * s0.x + a0 * s0.y, b1 * s1.x + a1 * s1.y);
    }
    st16(row + c * 8, ra);
    st16(row + h2 + c * 8, rb);
  }
}

hipError_t launch_rope(uint16_t* Q, uint16_t* K, const int32_t* pos, int64_t M, int H, int Hk, int D, int rot,
                       float base, bool inverse, hipStream_t s) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_kernel, dim3((unsigned)M), dim3(256), 0, s, Q, K, pos, H, Hk, D, rot, base,
                     inverse ? -1.f : 1.f);
  return hipGetLastError();
}

}  // namespace lora
