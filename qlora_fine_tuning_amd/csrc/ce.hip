// Cross-entropy over an LM head, after the logits' epilogue (tutorial ch. 5 §5.7, chunked
// cross-entropy: per chunk of tokens the logits, the loss and the gradient, the logits dropped).
// The forward GEMM's statistics epilogue leaves, for each row and each wave's 128 columns, the
// maximum and the sum of exp(logit - maximum), and the label's logit.  Here:
//  * ce_reduce_kernel: the row's log-sum-exp from those partials, combined in a fixed order
//    (16 rows per workgroup, 16 threads per row each taking a sixteenth of the partials in order,
//    the sixteenths then in order), and loss = lse - logit[label];
//  * ce_grad_kernel: the gradient of the logits, scale (softmax - onehot) in bf16, from the fp32
//    logits the statistics pass stored and the row's log-sum-exp (bound by HBM: 4 bytes read and
//    2 written per logit, 8 logits per thread);
//  * ce_sum_kernel: the sum of the per-row losses in a fixed order (one workgroup);
//  * fill_kernel: fills a buffer with a 32-bit pattern (no memset node, so the call stays
//    capturable).
#include "common.hpp"
#include "launch.hpp"

namespace lora {

__device__ __forceinline__ void lse_merge(float& mx, float& sm, float m2, float s2) {
  if (s2 == 0.f) return;  // an empty partial (columns past the vocabulary)
  const float mn = fmaxf(mx, m2);
  sm = sm * expf(mx - mn) + s2 * expf(m2 - mn);  // exp(-inf) = 0 for the empty start
  mx = mn;
}

__global__ void __launch_bounds__(256)
ce_reduce_kernel(const float* __restrict__ stats, const float* __restrict__ lab_logit, float* __restrict__ lse,
                 float* __restrict__ loss, int P, int M) {
  __shared__ float smx[16][16], ssm[16][16];
  const int r = threadIdx.x & 15, sl = threadIdx.x >> 4;  // row in the workgroup, slice of partials
  const int m = blockIdx.x * 16 + r;
  const int q = (P + 15) / 16, p0 = sl * q, p1 = min(P, p0 + q);
  float mx = -__builtin_inff(), sm = 0.f;
  if (m < M)
    for (int p = p0; p < p1; ++p) {
      const float2 v = *reinterpret_cast<const float2*>(stats + 2 * ((size_t)p * M + m));
      lse_merge(mx, sm, v.x, v.y);
    }
  smx[sl][r] = mx;
  ssm[sl][r] = sm;
  __syncthreads();
  if (sl == 0 && m < M) {
    for (int w = 1; w < 16; ++w) lse_merge(mx, sm, smx[w][r], ssm[w][r]);
    const float l = mx + logf(sm);
    lse[m] = l;
    loss[m] = l - lab_logit[m];
  }
}

__global__ void __launch_bounds__(256)
ce_grad_kernel(const float* __restrict__ logits, const float* __restrict__ lse, const int32_t* __restrict__ labels,
               uint16_t* __restrict__ dl, int64_t M, int64_t V, float scale) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t cpr = V / 8;
  if (t >= M * cpr) return;
  const int64_t m = t / cpr, v0 = (t - m * cpr) * 8;
  const float* src = logits + m * V + v0;
  const f32x4 a = *reinterpret_cast<const f32x4*>(src), b = *reinterpret_cast<const f32x4*>(src + 4);
  const float ls = lse[m];
  const int64_t lab = labels[m] - v0;  // the label's position in this thread's 8 columns, if any
  float p[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p[e] = __expf((e < 4 ? a[e] : b[e - 4]) - ls);
    if (e == lab) p[e] -= 1.f;
    p[e] *= scale;
  }
  st16(dl + m * V + v0, (u32x4){pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]),
                                pack_bf16(p[6], p[7])});
}

__global__ void __launch_bounds__(256) ce_sum_kernel(const float* __restrict__ loss, float* __restrict__ out, int M) {
  __shared__ float s[256];
  float acc = 0.f;
  for (int i = threadIdx.x; i < M; i += 256) acc += loss[i];
  s[threadIdx.x] = acc;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {  // fixed pairing: t + h into t
    if ((int)threadIdx.x < h) s[threadIdx.x] += s[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = s[0];
}

__global__ void __launch_bounds__(256) fill_kernel(uint32_t* __restrict__ p, size_t words, uint32_t v) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (size_t)gridDim.x * 256) p[i] = v;
}

hipError_t launch_ce_reduce(const float* stats, const float* lab_logit, float* lse, float* loss, int P, int64_t M,
                            hipStream_t s) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(ce_reduce_kernel, dim3((unsigned)((M + 15) / 16)), dim3(256), 0, s, stats, lab_logit, lse, loss,
                     P, (int)M);
  return hipGetLastError();
}

hipError_t launch_ce_grad(const float* logits, const float* lse, const int32_t* labels, uint16_t* dl, int64_t M,
                          int64_t V, float scale, hipStream_t s) {
  const int64_t threads = M * (V / 8);
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(ce_grad_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, logits, lse, labels,
                     dl, M, V, scale);
  return hipGetLastError();
}

hipError_t launch_ce_sum(const float* loss, float* out, int64_t M, hipStream_t s) {
  hipLaunchKernelGGL(ce_sum_kernel, dim3(1), dim3(256), 0, s, loss, out, (int)M);
  return hipGetLastError();
}

hipError_t launch_fill_u32(void* p, size_t bytes, uint32_t v, hipStream_t s) {  // bytes: a multiple of 4
  const size_t words = bytes / 4;
  if (words == 0) return hipSuccess;
  const size_t blocks = (words + 255) / 256;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, s,
                     static_cast<uint32_t*>(p), words, v);
  return hipGetLastError();
}

}  // namespace lora
