// Weight fragment sources of the MFMA kernels (GEMM, GEMV, and the fused
// one-token down projection): bf16 weights pre-tiled to the MFMA lane order,
// or NVFP4 weights decoded in registers to exact bf16.
#pragma once

#include "common.h"
#include "kernels.h"

// Weight loads. A weight byte read once per forward (GEMV arm; grouped GEMMs
// whose experts fit one row tile) streams past the caches with non-temporal
// loads. Where the same weights are read once per row tile (dense GEMMs,
// experts with several row tiles) plain loads let the L2 serve the repeats
// (measured: the non-temporal hint cost 24% at 8192 tokens and 8% on the
// latent layer).
template <bool NT, typename T>
__device__ __forceinline__ T ld_w(const T* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// Eight E2M1 codes (nibble i = element i) times an fp32 block scale -> bf16.
// e2m1 * e4m3 has at most 6 significant bits, so every product is exact in bf16.
// gfx950 converts two E2M1 codes (byte j: low nibble first) to fp32 per
// instruction. Its scale operand acts as a power of two only, so it is 1 here
// and the E4M3 block scale multiplies in fp32.
__device__ __forceinline__ bf16x8 dequant8(uint32_t q, float sc) {
  const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 0);
  const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 1);
  const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 2);
  const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 3);
  bf16x8 o;
  o[0] = (bf16)(p0[0] * sc); o[1] = (bf16)(p0[1] * sc);
  o[2] = (bf16)(p1[0] * sc); o[3] = (bf16)(p1[1] * sc);
  o[4] = (bf16)(p2[0] * sc); o[5] = (bf16)(p2[1] * sc);
  o[6] = (bf16)(p3[0] * sc); o[7] = (bf16)(p3[1] * sc);
  return o;
}

// Weight fragment sources of the MFMA kernel. A fragment is what one wave
// consumes per 64-wide k-step for its FT 16-row tiles.
//  * bf16: pre-tiled [N/16][K/32][64 lanes][8]: lane l holds row l%16, k
//    8*(l/16)..+7 of a 16x32 block (1 KiB per block, one contiguous read);
//    or k-major [K/64][N/16][2][64][8] (b_kmajor: a workgroup's tiles of one
//    k-step form one contiguous run).
//  * NVFP4: pre-tiled packed nibbles [N/16][K/64][64 lanes][8 bytes] (dword s
//    holds the lane's 8 codes of k-chunk s) and block scales
//    [N/16][K/64][16 rows][4 bytes] (the row's four 16-element blocks of the
//    step); scale2 of the group multiplies the accumulator in the epilogue.
template <int WQ, int FT, bool NT> struct WSrc;

// Dead tiles (features past N, possible in the last feature tile) keep the
// loads unconditional but point every lane at two fixed 1 KiB blocks at the
// start of the group with a zero step: cached lines instead of a re-read of
// live weights. The two 32-wide halves of a step are 512 elements apart in
// both tile orders.
template <int FT, bool NT> struct WSrc<0, FT, NT> {
  struct Frag { bf16x8 v[FT][2]; };
  // Wave-uniform group base and per-tile offsets and steps (elements; scalar
  // registers), one per-lane offset shared by the tiles.
  const bf16* wg;
  int off[FT];
  int step[FT];  // elements per 64-wide k-step (0 for a dead tile)
  int loff;
  __device__ __forceinline__ void init(const GemmArgs& a, int g, int nf0, int lane) {
    wg = (const bf16*)a.B + (size_t)g * a.b_gstride;
    const int KC = a.K / 32;
    nf0 = __builtin_amdgcn_readfirstlane(nf0);
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      const int rt = (nf0 >> 4) + ft;
      const bool live = rt * 16 < a.N;
      if (a.b_kmajor) {  // [K/64][N/16][2][64][8]
        off[ft] = live ? rt * 2 * 64 * 8 : 0;
        step[ft] = live ? (a.N / 16) * 1024 : 0;
      } else {  // [N/16][K/32][64][8]
        off[ft] = live ? rt * KC * 64 * 8 : 0;
        step[ft] = live ? 1024 : 0;
      }
    }
    loff = lane * 8;
  }
  __device__ __forceinline__ void load(Frag& f, int ks) const {
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
#pragma unroll
      for (int s = 0; s < 2; ++s)
        f.v[ft][s] = ld_w<NT>((const bf16x8*)(wg + (off[ft] + ks * step[ft] + s * 512) + loff));
  }
  __device__ __forceinline__ bf16x8 get(const Frag& f, int ft, int s, int) const { return f.v[ft][s]; }
};

template <int FT, bool NT> struct WSrc<1, FT, NT> {
  struct Frag { u32x2 q[FT]; uint32_t sc[FT]; };
  // Wave-uniform group bases and per-tile offsets (scalar registers; callers
  // pass a wave-uniform nf0), one per-lane offset: each load is a scalar base
  // + vector offset address (the 48-feature tiles had spilled with a 64-bit
  // pointer pair per feature tile).
  const u32x2* qg;
  const uint32_t* sg;
  int qoff[FT], soff[FT], qstep[FT], sstep[FT];
  int lq, ls;
  __device__ __forceinline__ void init(const GemmArgs& a, int g, int nf0, int lane) {
    qg = (const u32x2*)((const uint8_t*)a.B + (size_t)g * a.b_gstride);
    sg = (const uint32_t*)(a.b_scales + (size_t)g * a.bs_gstride);
    const int KS = a.K / 64;
    nf0 = __builtin_amdgcn_readfirstlane(nf0);
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      const int rt = (nf0 >> 4) + ft;
      const bool live = rt * 16 < a.N;
      qoff[ft] = live ? rt * KS * 64 : 0;
      soff[ft] = live ? rt * KS * 16 : 0;
      qstep[ft] = live ? 64 : 0;
      sstep[ft] = live ? 16 : 0;
    }
    lq = lane;
    ls = lane & 15;
  }
  __device__ __forceinline__ void load(Frag& f, int ks) const {
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      f.q[ft] = ld_w<NT>(qg + (qoff[ft] + ks * qstep[ft]) + lq);
      f.sc[ft] = sg[(soff[ft] + ks * sstep[ft]) + ls];
    }
  }
  __device__ __forceinline__ bf16x8 get(const Frag& f, int ft, int s, int lane) const {
    // k-chunk s of lane group g = lane/16 lies in block 2s + g/2 of the step:
    // byte 2s of the scale word shifted by 8 * (g/2), decoded by gfx950's
    // E4M3 (OCP) -> fp32 conversion (exact for all 256 codes).
    const uint32_t sh = f.sc[ft] >> ((lane >> 5) * 8);
    const float sc = s == 0 ? __builtin_amdgcn_cvt_f32_fp8((int)sh, 0)
                            : __builtin_amdgcn_cvt_f32_fp8((int)sh, 2);
    return dequant8(f.q[ft][s], sc);
  }
};

