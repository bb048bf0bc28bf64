// Unpermute + routing-weighted reduce, fused with the shared-expert add and
// the residual add (page "Struct MoeLayer", `forward_prefill`: unpermute and
// weighted reduce, then the shared-expert blend; page
// "metrale_model_arch/nemotron_moe.rs", module doc: weighted sum, plus the
// shared expert, added to hidden).
//
// The routed rows y are in expert-sorted order (row inv[t*k + j] holds slot j
// of token t), or, from the decode-sized arm, in route order (inv == null:
// row t*k + j). Slots are summed in slot order (no atomics), so the result is
// deterministic. Each thread owns 4 consecutive columns; the k slot indices
// and weights are loaded first so that the k row loads issue together.
#include "kernels.h"

template <typename T> struct vec4;
template <> struct vec4<float> {
  static __device__ __forceinline__ floatx4 ld(const float* p) { return *(const floatx4*)p; }
  static __device__ __forceinline__ void st(float* p, floatx4 v) { *(floatx4*)p = v; }
};
template <> struct vec4<bf16> {
  static __device__ __forceinline__ floatx4 ld(const bf16* p) {
    const bf16x4 i = *(const bf16x4*)p;
    return floatx4{(float)i[0], (float)i[1], (float)i[2], (float)i[3]};
  }
  static __device__ __forceinline__ void st(bf16* p, floatx4 v) {
    bf16x4 o;
    o[0] = (bf16)v[0]; o[1] = (bf16)v[1]; o[2] = (bf16)v[2]; o[3] = (bf16)v[3];
    *(bf16x4*)p = o;
  }
};

template <typename T, bool LATENT>
__global__ void __launch_bounds__(256) unpermute_reduce_kernel(
    const T* __restrict__ y, const int* __restrict__ inv, const float* __restrict__ w, int n,
    int k, int D, const T* __restrict__ residual, const T* __restrict__ sh, T* __restrict__ out) {
  const int t = blockIdx.x;
  const int d = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (t >= n || d >= D) return;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  int p[MOE_MAX_TOPK_REDUCE];
  float wt[MOE_MAX_TOPK_REDUCE];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK_REDUCE; ++j)
    if (j < k) {
      p[j] = inv ? inv[t * k + j] : t * k + j;
      wt[j] = w[t * k + j];
    }
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK_REDUCE; ++j)
    if (j < k) acc += wt[j] * vec4<T>::ld(y + (size_t)p[j] * D + d);
  const size_t o = (size_t)t * D + d;
  if (!LATENT) {
    acc = vec4<T>::ld(residual + o) + acc;
    if (sh) acc += vec4<T>::ld(sh + o);
  }
  vec4<T>::st(out + o, acc);
}

// bf16: one workgroup per token, 8 columns (16 bytes) per thread; the k slot
// indices and weights are the same for the whole workgroup. Same summation
// order as above (slots in order, then residual, then shared).
// KMAX: the slot arrays' size (8 covers top-k <= 8 with half the registers
// of the general 16: more resident waves, measured 45.2 -> 39.4 us at 4096
// tokens, 15.9 -> 14.5 us at 1024).
template <bool LATENT, int KMAX>
__global__ void __launch_bounds__(1024) unpermute_reduce_bf16_kernel(
    const bf16* __restrict__ y, const int* __restrict__ inv, const float* __restrict__ w, int k,
    int D, const bf16* __restrict__ residual, const bf16* __restrict__ sh, bf16* __restrict__ out) {
  const int t = blockIdx.x;
  const int d = threadIdx.x * 8;
  if (d >= D) return;
  const size_t o = (size_t)t * D + d;
  // residual and shared rows do not depend on the slot indices: issued first
  bf16x8 r = {}, a = {};
  if (!LATENT) {
    r = *(const bf16x8*)(residual + o);
    if (sh) a = *(const bf16x8*)(sh + o);
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int p[KMAX];
  float wt[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    if (j < k) {
      p[j] = inv ? inv[t * k + j] : t * k + j;
      wt[j] = w[t * k + j];
    }
  bf16x8 v[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    if (j < k) v[j] = *(const bf16x8*)(y + (size_t)p[j] * D + d);
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    if (j < k)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] += wt[j] * (float)v[j][q];
  if (!LATENT) {
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = (float)r[q] + acc[q];
    if (sh) {
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] += (float)a[q];
    }
  }
  bf16x8 ob;
#pragma unroll
  for (int q = 0; q < 8; ++q) ob[q] = (bf16)acc[q];
  *(bf16x8*)(out + o) = ob;
}

hipError_t launch_unpermute_reduce(int dt, bool latent, const void* y, const int* inv,
                                   const float* w, int n, int k, int D, const void* residual,
                                   const void* sh, void* out, hipStream_t s) {
  if (k > MOE_MAX_TOPK_REDUCE) return hipErrorInvalidValue;
  if (dt == MOE_DT_BF16 && D % 8 == 0 && D / 8 <= 1024) {
    const dim3 block(((D / 8) + 63) / 64 * 64);
#define RED_LAUNCH(L, KM)                                                                       \
  hipLaunchKernelGGL((unpermute_reduce_bf16_kernel<L, KM>), dim3(n), block, 0, s, (const bf16*)y, \
                     inv, w, k, D, (const bf16*)residual, (const bf16*)sh, (bf16*)out)
    if (k <= 8) {
      if (latent) RED_LAUNCH(true, 8); else RED_LAUNCH(false, 8);
    } else {
      if (latent) RED_LAUNCH(true, MOE_MAX_TOPK_REDUCE); else RED_LAUNCH(false, MOE_MAX_TOPK_REDUCE);
    }
#undef RED_LAUNCH
    return hipGetLastError();
  }
  dim3 grid(n, (D / 4 + 255) / 256);
  if (dt == MOE_DT_BF16) {
    if (latent)
      hipLaunchKernelGGL((unpermute_reduce_kernel<bf16, true>), grid, dim3(256), 0, s,
                         (const bf16*)y, inv, w, n, k, D, (const bf16*)residual, (const bf16*)sh,
                         (bf16*)out);
    else
      hipLaunchKernelGGL((unpermute_reduce_kernel<bf16, false>), grid, dim3(256), 0, s,
                         (const bf16*)y, inv, w, n, k, D, (const bf16*)residual, (const bf16*)sh,
                         (bf16*)out);
  } else {
    if (latent)
      hipLaunchKernelGGL((unpermute_reduce_kernel<float, true>), grid, dim3(256), 0, s,
                         (const float*)y, inv, w, n, k, D, (const float*)residual,
                         (const float*)sh, (float*)out);
    else
      hipLaunchKernelGGL((unpermute_reduce_kernel<float, false>), grid, dim3(256), 0, s,
                         (const float*)y, inv, w, n, k, D, (const float*)residual,
                         (const float*)sh, (float*)out);
  }
  return hipGetLastError();
}
