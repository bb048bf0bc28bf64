// Unpermute + routing-weighted reduce, fused with the shared-expert add and
// the residual add (page "Struct MoeLayer", `forward_prefill`: unpermute and
// weighted reduce, then the shared-expert blend; page
// "metrale_model_arch/nemotron_moe.rs", module doc: weighted sum, plus the
// shared expert, added to hidden).
//
// The routed rows y are in expert-sorted order; row inv[t*k + j] holds slot j
// of token t. Slots are summed in slot order (no atomics), so the result is
// deterministic. Each thread owns 4 consecutive columns: 16-byte loads of y.
#include "kernels.h"

template <typename TO, bool LATENT>
__global__ void __launch_bounds__(256) unpermute_reduce_kernel(
    const float* __restrict__ y, const int* __restrict__ inv, const float* __restrict__ w, int n,
    int k, int D, const TO* __restrict__ residual, const float* __restrict__ sh,
    TO* __restrict__ out) {
  const int t = blockIdx.x;
  const int d = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (t >= n || d >= D) return;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const int p = inv[t * k + j];
    const float wt = w[t * k + j];
    const floatx4 v = *(const floatx4*)(y + (size_t)p * D + d);
    acc += wt * v;
  }
  const size_t o = (size_t)t * D + d;
  if (!LATENT) {
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = io<TO>::ld(residual + o + q) + acc[q];
    if (sh) acc += *(const floatx4*)(sh + o);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) io<TO>::st(out + o + q, acc[q]);
}

hipError_t launch_unpermute_reduce(int out_dt, bool latent, const float* y, const int* inv,
                                   const float* w, int n, int k, int D, const void* residual,
                                   const float* sh, void* out, hipStream_t s) {
  dim3 grid(n, (D / 4 + 255) / 256);
  if (out_dt == MOE_DT_BF16) {
    if (latent)
      hipLaunchKernelGGL((unpermute_reduce_kernel<bf16, true>), grid, dim3(256), 0, s, y, inv, w, n,
                         k, D, (const bf16*)residual, sh, (bf16*)out);
    else
      hipLaunchKernelGGL((unpermute_reduce_kernel<bf16, false>), grid, dim3(256), 0, s, y, inv, w,
                         n, k, D, (const bf16*)residual, sh, (bf16*)out);
  } else {
    if (latent)
      hipLaunchKernelGGL((unpermute_reduce_kernel<float, true>), grid, dim3(256), 0, s, y, inv, w,
                         n, k, D, (const float*)residual, sh, (float*)out);
    else
      hipLaunchKernelGGL((unpermute_reduce_kernel<float, false>), grid, dim3(256), 0, s, y, inv, w,
                         n, k, D, (const float*)residual, sh, (float*)out);
  }
  return hipGetLastError();
}
