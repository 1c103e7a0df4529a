// Cross-entropy over an LM head, after the logits' epilogue (tutorial ch. 5 §5.7, chunked
// cross-entropy: per chunk of tokens the logits, the loss and the gradient, the logits dropped).
// The forward GEMM's statistics epilogue leaves, for each row and each wave's 128 columns, the
// maximum and the sum of exp(logit - maximum), and the label's logit.  Here:
//  * ce_reduce_kernel: the row's log-sum-exp from those partials, combined in a fixed order, and
//    loss = lse - logit[label];
//  * ce_grad_kernel: the gradient of the logits, scale (softmax - onehot) in bf16, from the fp32
//    logits the statistics pass stored (as high and low 16-bit planes) and the row's log-sum-exp,
//    written over the high plane (bound by HBM: 4 bytes read and 2 written per logit);
//  * ce_sum_kernel: the sum of the per-row losses in a fixed order (one workgroup), times the
//    caller's scale (1/M for the mean);
//  * scale_bf16_kernel: a bf16 gradient times an upstream scalar held in device memory;
//  * fill_kernel: fills a buffer with a 32-bit pattern (no memset node, so the call stays
//    capturable).
#include "common.hpp"
#include "launch.hpp"

namespace lora {

// One wave per row (4 rows per workgroup).  A row's P partials are contiguous; lane `sl` takes
// partials sl, sl + 64, sl + 128, ... (each load instruction reads 512 contiguous bytes), in
// batches of 64 x kCeSlice with all of a batch's loads in flight: the batch's maximum, then the
// sum of s exp(m - maximum) in order, folded into the lane's running pair.  The 64 lanes' pairs
// are then folded by a butterfly whose two partners compute the same commutative expression, so
// every lane, and every run, ends with the same bits.  The wave also puts NaN back into the row's
// label-logit slot, so the next chunk finds it there unless its statistics pass writes the label's
// logit.  An empty partial (columns past V) holds sum 0; any other holds a sum of at least 1.
constexpr int kCeSlice = 16;
__device__ __forceinline__ void lse_fold(float& mx, float& sm, float m2, float s2) {
  if (s2 == 0.f) return;
  if (sm == 0.f) {
    mx = m2;
    sm = s2;
    return;
  }
  const float mn = fmaxf(mx, m2);
  sm = sm * expf(mx - mn) + s2 * expf(m2 - mn);
  mx = mn;
}

__global__ void __launch_bounds__(256)
ce_reduce_kernel(const float* __restrict__ stats, float* __restrict__ lab_logit, float* __restrict__ lse,
                 float* __restrict__ loss, int P, int M) {
  const int sl = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  const float* row = stats + 2 * (size_t)m * P;
  float mx = -__builtin_inff(), sm = 0.f;
  for (int b = 0; b < P; b += 64 * kCeSlice) {
    float2 v[kCeSlice];
#pragma unroll
    for (int u = 0; u < kCeSlice; ++u) {
      const int p = b + sl + 64 * u;
      v[u] = p < P ? *reinterpret_cast<const float2*>(row + 2 * p) : make_float2(-__builtin_inff(), 0.f);
    }
    float bm = -__builtin_inff();
#pragma unroll
    for (int u = 0; u < kCeSlice; ++u)
      if (v[u].y != 0.f) bm = fmaxf(bm, v[u].x);
    float bs = 0.f;
#pragma unroll
    for (int u = 0; u < kCeSlice; ++u)
      if (v[u].y != 0.f) bs += v[u].y * expf(v[u].x - bm);
    lse_fold(mx, sm, bm, bs);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float m2 = __shfl_xor(mx, o, 64), s2 = __shfl_xor(sm, o, 64);
    if (s2 != 0.f && sm != 0.f) {
      const float mn = fmaxf(mx, m2);
      sm = sm * expf(mx - mn) + s2 * expf(m2 - mn);
      mx = mn;
    } else if (s2 != 0.f) {
      mx = m2;
      sm = s2;
    }
  }
  if (sl == 0) {
    const float l = mx + logf(sm);
    lse[m] = l;
    loss[m] = l - lab_logit[m];
    lab_logit[m] = __builtin_nanf("");
  }
}

// One thread per 8 consecutive logits of a row: their two 16-bit planes in, the bf16 gradient out
// over the high plane (the same 16 bytes the thread read, so the pass runs in place).
__global__ void __launch_bounds__(256)
ce_grad_kernel(uint16_t* __restrict__ hi, const uint16_t* __restrict__ lo, const float* __restrict__ lse,
               const int32_t* __restrict__ labels, int64_t M, int64_t V, float scale) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t cpr = V / 8;
  if (t >= M * cpr) return;
  const int64_t m = t / cpr, v0 = (t - m * cpr) * 8;
  const size_t o = (size_t)m * V + v0;
  const u32x4 h = *reinterpret_cast<const u32x4*>(hi + o), l = *reinterpret_cast<const u32x4*>(lo + o);
  const float ls = lse[m];
  const int64_t lab = labels[m] - v0;  // the label's position in this thread's 8 columns, if any
  float p[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    p[2 * e] = __uint_as_float((h[e] << 16) | (l[e] & 0xffffu));
    p[2 * e + 1] = __uint_as_float((h[e] & 0xffff0000u) | (l[e] >> 16));
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p[e] = __expf(p[e] - ls);
    if (e == lab) p[e] -= 1.f;
    p[e] *= scale;
  }
  st16(hi + o, (u32x4){pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7])});
}

__global__ void __launch_bounds__(256)
ce_sum_kernel(const float* __restrict__ loss, float* __restrict__ out, int M, float scale) {
  __shared__ float s[256];
  float acc = 0.f;
  for (int i = threadIdx.x; i < M; i += 256) acc += loss[i];
  s[threadIdx.x] = acc;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {  // fixed pairing: t + h into t
    if ((int)threadIdx.x < h) s[threadIdx.x] += s[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = s[0] * scale;
}

// out = bf16(in x g[0]), 8 values per thread per step (n a multiple of 8)
__global__ void __launch_bounds__(256)
scale_bf16_kernel(const uint16_t* __restrict__ in, uint16_t* __restrict__ out, int64_t n8, const float* __restrict__ g) {
  const float f = g[0];
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(in + 8 * i);
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = pack_bf16(__uint_as_float(v[e] << 16) * f, __uint_as_float(v[e] & 0xffff0000u) * f);
    st16(out + 8 * i, w);
  }
}

__global__ void __launch_bounds__(256) fill_kernel(uint32_t* __restrict__ p, size_t words, uint32_t v) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (size_t)gridDim.x * 256) p[i] = v;
}

hipError_t launch_ce_reduce(const float* stats, float* lab_logit, float* lse, float* loss, int P, int64_t M,
                            hipStream_t s) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(ce_reduce_kernel, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, s, stats, lab_logit, lse, loss, P,
                     (int)M);
  return hipGetLastError();
}

hipError_t launch_ce_grad(uint16_t* hi, const uint16_t* lo, const float* lse, const int32_t* labels, int64_t M,
                          int64_t V, float scale, hipStream_t s) {
  const int64_t threads = M * (V / 8);
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(ce_grad_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, hi, lo, lse, labels,
                     M, V, scale);
  return hipGetLastError();
}

hipError_t launch_ce_sum(const float* loss, float* out, int64_t M, float scale, hipStream_t s) {
  hipLaunchKernelGGL(ce_sum_kernel, dim3(1), dim3(256), 0, s, loss, out, (int)M, scale);
  return hipGetLastError();
}

hipError_t launch_scale_bf16(const uint16_t* in, uint16_t* out, int64_t n, const float* g, hipStream_t s) {
  const int64_t n8 = n / 8;
  if (n8 == 0) return hipSuccess;
  const int64_t blocks = (n8 + 255) / 256;
  hipLaunchKernelGGL(scale_bf16_kernel, dim3((unsigned)(blocks < 2048 ? blocks : 2048)), dim3(256), 0, s, in, out, n8,
                     g);
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
