// GEMM kernels of the MoE layer on gfx950.
//
// Every projection of the layer is C[p][n] = sum_k A[arow(p)][k] * W[g][n][k]
// followed by an epilogue: the grouped expert GEMMs (page "Struct MoeLayer",
// `forward_prefill`: grouped up GEMM, activation, grouped down GEMM; each
// expert's weights read once per prefill instead of once per token), the
// shared expert and the fc1/fc2 latent projections (page
// "metrale_model_arch/nemotron_moe.rs", `prefill`: dense GEMMs over all
// tokens). relu^2 is fused into the up-projection epilogue (same page, module
// doc: routed up, relu^2, down).
//
// bf16 MFMA kernel (gemm_mfma_kernel):
//   * MFMA v_mfma_f32_16x16x32_bf16 with the WEIGHTS as the A operand (16
//     output features) and the ACTIVATIONS as the B operand (16 tokens), so a
//     lane's four results are four consecutive output features of one row.
//   * Weights are re-tiled once at layer creation into the MFMA lane order:
//     [N/16][K/32][64 lanes][8], lane l holding feature l%16 and k-elements
//     8*(l/16)..+7 of its 16x32 block. A wave's weight fetch for one MFMA is
//     then one contiguous 1 KiB read, and each weight byte is fetched by
//     exactly one wave (waves own disjoint features).
//   * A workgroup (NW = 4 or 8 waves) covers NW*WF features x BMT rows. The
//     BMT x 64 activation slice of each k-step is gathered (rows by the route
//     permutation) with 16-byte loads, staged through LDS (double buffered,
//     XOR-swizzled 16-byte chunks so the MFMA operand reads are conflict-free)
//     and shared by the waves.
//   * Weights for step k+1 are in flight while step k computes; the output
//     tile leaves through LDS as whole rows.
//   * Persistent grid, XCD-aware tile order (see gemm_mfma_kernel).
//   * NVFP4 weights (4-bit E2M1 + E4M3 per 16 along K + fp32 scale2 per
//     matrix; page "metrale_model_arch/nemotron_moe.rs", `ExpertPtrTable`) are
//     re-tiled the same way and dequantized in registers to exact bf16 before
//     the MFMA; scale2 multiplies the accumulator in the epilogue.
//
// Decode-sized GEMV (gemv_kernel): one workgroup per (row tile of <= 16 rows,
// 16 features); see below.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "kernels.h"
#include "wsrc.h"

// ---------------------------------------------------------------------------
// Tile decode shared by both kernels.
// ---------------------------------------------------------------------------
struct TileInfo {
  int g, row0, rows;
};

__device__ __forceinline__ bool decode_tile(const GemmArgs& a, int tile, int bmt, TileInfo& ti) {
  if (a.tiles) {
    if (tile >= *a.num_tiles) return false;
    const int2 t = a.tiles[tile];
    ti.g = t.x;
    const int lo = a.offsets[t.x], hi = a.offsets[t.x + 1];
    ti.row0 = lo + t.y;
    ti.rows = min(bmt, hi - ti.row0);
  } else {
    ti.g = 0;
    ti.row0 = tile * bmt;
    ti.rows = min(bmt, a.M - ti.row0);
  }
  return ti.rows > 0;
}

__device__ __forceinline__ int a_row_of(const GemmArgs& a, int p) {
  return a.a_rows ? a.a_rows[p] / a.a_div : p;
}

// ---------------------------------------------------------------------------
// fp32 SIMT GEMM: 64x64 output tile, 256 threads with 4x4 outputs each, BK=16.
// Used by fp32 layers (no fp32 MFMA shape is faster than this at their sizes).
// ---------------------------------------------------------------------------
template <int EPI>
__global__ void __launch_bounds__(256) gemm_simt_f32_kernel(GemmArgs a) {
  __shared__ float As[16][65];
  __shared__ float Bs[16][65];
  TileInfo ti;
  if (!decode_tile(a, blockIdx.y, 64, ti)) return;
  const int n0 = blockIdx.x * 64;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const float* A = (const float*)a.A;
  const float* B = (const float*)a.B + (size_t)ti.g * a.b_gstride;

  // Loader: row (tid>>2) of the tile, k-quad (tid&3).
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  const int arow = a_row_of(a, ti.row0 + min(lr, ti.rows - 1));
  const float* asrc = A + (size_t)arow * a.lda + lk;
  const int bn = min(n0 + lr, a.N - 1);
  const float* bsrc = B + (size_t)bn * a.K + lk;

  float acc[4][4] = {};
  for (int k0 = 0; k0 < a.K; k0 += 16) {
    float4 av = *(const float4*)(asrc + k0);
    float4 bv = *(const float4*)(bsrc + k0);
    As[lk + 0][lr] = av.x; As[lk + 1][lr] = av.y; As[lk + 2][lr] = av.z; As[lk + 3][lr] = av.w;
    Bs[lk + 0][lr] = bv.x; Bs[lk + 1][lr] = bv.y; Bs[lk + 2][lr] = bv.z; Bs[lk + 3][lr] = bv.w;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float ar[4], br[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { ar[i] = As[kk][ty * 4 + i]; br[i] = Bs[kk][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += ar[i] * br[j];
    }
    __syncthreads();
  }
  float* C = (float*)a.C;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ty * 4 + i;
    if (r >= ti.rows) continue;
    const int p = ti.row0 + r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= a.N) continue;
      float v = acc[i][j];
      if (EPI == EPI_RELU2) v = relu2(v);
      if (EPI == EPI_ADD_RES) {
        v += ((const float*)a.res)[(size_t)p * a.ldc + n];
        if (a.add) v += ((const float*)a.add)[(size_t)p * a.ldc + n];
      }
      C[(size_t)p * a.ldc + n] = v;
    }
  }
}

hipError_t launch_gemm_simt_f32(const GemmArgs& a, int epi, int grid_y, hipStream_t s) {
  dim3 grid((a.N + 63) / 64, grid_y);
  switch (epi) {
    case EPI_RELU2: hipLaunchKernelGGL(gemm_simt_f32_kernel<EPI_RELU2>, grid, dim3(256), 0, s, a); break;
    case EPI_STORE: hipLaunchKernelGGL(gemm_simt_f32_kernel<EPI_STORE>, grid, dim3(256), 0, s, a); break;
    case EPI_ADD_RES: hipLaunchKernelGGL(gemm_simt_f32_kernel<EPI_ADD_RES>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// bf16 MFMA GEMM.
// ---------------------------------------------------------------------------
template <typename TC> struct store4;
template <> struct store4<float> {
  static __device__ __forceinline__ void st(float* p, floatx4 v) { *(floatx4*)p = v; }
  static __device__ __forceinline__ floatx4 ld(const float* p) { return *(const floatx4*)p; }
};
template <> struct store4<bf16> {
  static __device__ __forceinline__ void st(bf16* p, floatx4 v) {
    bf16x4 o;
    o[0] = (bf16)v[0]; o[1] = (bf16)v[1]; o[2] = (bf16)v[2]; o[3] = (bf16)v[3];
    *(bf16x4*)p = o;
  }
  static __device__ __forceinline__ floatx4 ld(const bf16* p) {
    bf16x4 i = *(const bf16x4*)p;
    floatx4 v;
    v[0] = (float)i[0]; v[1] = (float)i[1]; v[2] = (float)i[2]; v[3] = (float)i[3];
    return v;
  }
};

// ---------------------------------------------------------------------------
// Persistent MFMA GEMM (grouped or dense), WQ = 0 bf16 weights, 1 NVFP4.
// ---------------------------------------------------------------------------
// Pipeline depth S: the loads of step k+S-1 are issued at the start of step
// k, and a gathered activation slice waits one more step in registers before
// it goes to LDS.
// Measured on the layer's shapes: three stages pay on 128 x 256 and 128 x 192
// tiles (7-9% on the bf16 grouped GEMMs from 4096 tokens up, 2% on the latent
// layer, 1% on NVFP4 weights at 4096 tokens) and on DEEP launches (dense, at
// most one 128 x 128 tile per CU, so one resident workgroup per CU and the
// register budget of a whole SIMD: 8-10% on the shared expert at 1024
// tokens); two elsewhere (three cost 2-5% on 64-row tiles, and spill at two
// 128 x 128 workgroups per CU).
// The 7-wave tiles (48 features per wave) keep two stages: with three their
// activation loads (three 16-byte chunks per thread) spill.
constexpr int mfma_stages(int bmt, int nw, bool deep) {
  return deep || (bmt == 128 && (nw == 6 || nw == 8)) ? 3 : 2;
}
// Workgroups per CU the register budget is sized for.
constexpr int mfma_min_blocks(int bmt, int nw, bool deep) {
  return (bmt >= 128 && nw == 4 && !deep) ? 2 : 1;
}

// LDS of one workgroup: the activation stages, or the staged output tile.
constexpr int mfma_lds_elems(int stages, int bmt, int cw) {
  return stages * bmt * 64 > bmt * (cw + 8) ? stages * bmt * 64 : bmt * (cw + 8);
}

// One output tile: BMT rows x (NW waves x WF) features, of which the first
// TL 16-row blocks hold live rows (ti.rows <= 16 * TL): the MFMAs and their
// operand reads skip the padding blocks.
template <int WF, int BMT, int NW, int EPI, typename TC, int WQ, bool GROUPED, bool NT,
          bool DEEP, int TL>
__device__ __forceinline__ void mfma_tile(const GemmArgs& a, const TileInfo& ti, int ftile,
                                          bf16* __restrict__ xs) {
  constexpr int S = mfma_stages(BMT, NW, DEEP);
  constexpr int FT = WF / 16;      // 16-feature tiles per wave
  constexpr int TT = BMT / 16;     // 16-row tiles per workgroup
  constexpr int BK = 64;           // k per step (two MFMA k-chunks of 32)
  constexpr int NTHR = NW * 64;    // threads
  constexpr int CHUNKS = BMT * 8;  // 16-byte chunks of one activation slice
  constexpr int LPASS = (CHUNKS + NTHR - 1) / NTHR;
  using Src = WSrc<WQ, FT, NT>;
  using Frag = typename Src::Frag;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nsteps = a.K / BK;

  // Activation loader: chunk c = (tid + threads*i) % CHUNKS -> row c/8,
  // 16-byte chunk c%8 (small tiles: several threads load the same chunk, so
  // every load is unconditional and the k-loop has no branches).
  const bf16* asrc[LPASS];
  int lds_off[LPASS];
#pragma unroll
  for (int i = 0; i < LPASS; ++i) {
    const int c = (tid + NTHR * i) % CHUNKS;
    const int row = c >> 3, ch = c & 7;
    const int r = min(row, ti.rows - 1);
    const int arow = GROUPED ? a_row_of(a, ti.row0 + r) : ti.row0 + r;
    asrc[i] = (const bf16*)a.A + (size_t)arow * a.lda + ch * 8;
    lds_off[i] = row * BK + ((ch ^ (row & 7)) << 3);
  }

  const int nf0 = ftile * (NW * WF) + wave * WF;  // first feature of this wave
  Src src;
  src.init(a, ti.g, nf0, lane);

  floatx4 acc[FT][TT];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[ft][tt] = floatx4{0.f, 0.f, 0.f, 0.f};

  // S-stage pipeline. At the start of step k the weights and the activation
  // slice of step k+S-1 are loaded into register set (k+S-1)%S. After the
  // MFMAs of step k, the slice of step k+1 (loaded at step k+2-S) goes from
  // its registers into LDS slot (k+1)%S. With S >= 3 a gathered slice is thus
  // written to LDS one step after its load was issued, and its latency hides
  // under two steps of MFMAs instead of one; with S = 2 the slice is loaded
  // and stored in the same step. The ring index is a compile-time constant:
  // the k-loop is unrolled by S.
  Frag w[S];
  bf16x8 areg[S][LPASS];
#pragma unroll
  for (int p = 0; p < S - 1; ++p) {
    const int kp = min(p, nsteps - 1);
    src.load(w[p], kp);
#pragma unroll
    for (int i = 0; i < LPASS; ++i) areg[p][i] = *(const bf16x8*)(asrc[i] + kp * BK);
  }
#pragma unroll
  for (int i = 0; i < LPASS; ++i) *(bf16x8*)(&xs[lds_off[i]]) = areg[0][i];
  __syncthreads();

  const int brow = lane & 15, bch = lane >> 4;
  auto compute = [&](int cur, const Frag& wc) {
    if constexpr (TL > 8 || (FT >= 3 && TL > 4)) {
      // More than 8 live 16-row blocks, or waves of three or more feature
      // tiles: the weight fragments of a half-step are decoded once, and the
      // activation fragments are read in two batches (registers: with all
      // eight at once the 48-feature tiles spilled, NVFP4 48 B/lane, bf16
      // 170-210 B/lane).
      constexpr int CH = (TL + 1) / 2;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8 wf[FT];
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) wf[ft] = src.get(wc, ft, s, lane);
#pragma unroll
        for (int c0 = 0; c0 < TL; c0 += CH) {
          bf16x8 xf[CH];
#pragma unroll
          for (int i = 0; i < CH; ++i) {
            const int row = (c0 + i) * 16 + brow;
            const int ch = s * 4 + bch;
            if (c0 + i < TL)
              xf[i] = *(const bf16x8*)(&xs[cur * BMT * 64 + row * BK + ((ch ^ (row & 7)) << 3)]);
          }
#pragma unroll
          for (int ft = 0; ft < FT; ++ft)
#pragma unroll
            for (int i = 0; i < CH; ++i)
              if (c0 + i < TL)
                acc[ft][c0 + i] =
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[ft], xf[i], acc[ft][c0 + i], 0, 0, 0);
        }
      }
      return;
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 xf[TL];
#pragma unroll
      for (int tt = 0; tt < TL; ++tt) {
        const int row = tt * 16 + brow;
        const int ch = s * 4 + bch;
        xf[tt] = *(const bf16x8*)(&xs[cur * BMT * 64 + row * BK + ((ch ^ (row & 7)) << 3)]);
      }
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) {
        const bf16x8 wf = src.get(wc, ft, s, lane);
#pragma unroll
        for (int tt = 0; tt < TL; ++tt)
          acc[ft][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, xf[tt], acc[ft][tt], 0, 0, 0);
      }
    }
  };
  // Step k (ring slot u = k % S). PREF: whether step k+S-1 exists; STAGE:
  // whether step k+1 exists (the steady state does both; only the last steps
  // of an item skip them).
  auto step = [&](int k, auto u_c, bool pref, bool stage) {
    constexpr int u = decltype(u_c)::value;
    constexpr int un = (u + S - 1) % S;  // ring slot of step k+S-1
    constexpr int u1 = (u + 1) % S;      // ring slot of step k+1
    const int kn = k + S - 1;
    if (pref) {
#pragma unroll
      for (int i = 0; i < LPASS; ++i) areg[un][i] = *(const bf16x8*)(asrc[i] + kn * BK);
      src.load(w[un], kn);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the MFMAs
    compute(u, w[u]);
    if (stage) {
#pragma unroll
      for (int i = 0; i < LPASS; ++i) *(bf16x8*)(&xs[u1 * BMT * 64 + lds_off[i]]) = areg[u1][i];
    }
    __syncthreads();
  };
  auto group = [&](int k0, bool tail) {
    [&]<int... U>(std::integer_sequence<int, U...>) {
      ((tail ? (k0 + U < nsteps ? step(k0 + U, std::integral_constant<int, U>{},
                                       k0 + U + S - 1 < nsteps, k0 + U + 1 < nsteps)
                                : void())
             : step(k0 + U, std::integral_constant<int, U>{}, true, true)),
       ...);
    }(std::make_integer_sequence<int, S>{});
  };
  int k0 = 0;
  for (; k0 + 2 * S - 1 <= nsteps; k0 += S) group(k0, false);  // no bounds checks
  for (; k0 < nsteps; k0 += S) group(k0, true);                // at most two groups

  // Epilogue: lane holds features nf0 + 16*ft + 4*(lane/16) + 0..3 of row 16*tt + lane%16.
  const float s2 = WQ == 1 ? a.b_scale2[ti.g] : 1.0f;
  TC* C = (TC*)a.C;
  if constexpr (EPI != EPI_ADD_RES) {
    // The bf16 tile goes through LDS (row stride CW + 8) and leaves as whole
    // rows: each 16-byte store sits in a contiguous run of CW * 2 bytes per
    // row instead of the accumulator layout's 32-byte pieces (measured 2-6%
    // faster where the outputs are large). fc2's residual add stages fp32
    // instead (below), so that it rounds once.
    constexpr int CW = NW * WF, SP = CW + 8;
    __syncthreads();  // every wave is done with the activation stages
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        floatx4 v = acc[ft][tt];
        if (WQ == 1) v *= s2;
        const int c = wave * WF + ft * 16 + 4 * (lane >> 4);
        if (EPI == EPI_RELU2 && (GROUPED || a.relu_n == 0 || ftile * CW + c < a.relu_n)) {
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = relu2(v[q]);
        }
        bf16x4 o;
        o[0] = (bf16)v[0]; o[1] = (bf16)v[1]; o[2] = (bf16)v[2]; o[3] = (bf16)v[3];
        const int r = tt * 16 + (lane & 15);
        *(bf16x4*)(&xs[r * SP + c]) = o;
      }
    __syncthreads();
    // Grouped outputs (h, y: tens of MB) are stored non-temporally: plain
    // stores mixed into the weight stream cost 6% more at the bench size.
    const int n0 = ftile * CW;
    for (int q = tid; q < BMT * (CW / 8); q += NTHR) {
      const int r = q / (CW / 8), c = (q % (CW / 8)) * 8;
      if (r < ti.rows && n0 + c < a.N) {
        bf16x8* dst = (bf16x8*)((bf16*)C + (size_t)(ti.row0 + r) * a.ldc + n0 + c);
        const bf16x8 v = *(const bf16x8*)(&xs[r * SP + c]);
        if constexpr (GROUPED) __builtin_nontemporal_store(v, dst);
        else *dst = v;
      }
    }
  } else {
    // fc2: acc + residual + shared, rounded to bf16 once. The fp32 tile goes
    // through LDS in passes of HR rows (row stride CW + 4 floats) and leaves as
    // whole rows, so residual, shared and output move as 16-byte row chunks
    // (the accumulator layout gives each lane 8-byte pieces of 32-byte runs).
    static_assert(std::is_same<TC, bf16>::value, "the MFMA kernels store bf16");
    constexpr int CW = NW * WF, SPF = CW + 4;
    constexpr int CAP = mfma_lds_elems(S, BMT, CW) * 2 / (SPF * 4);  // fp32 rows that fit
    constexpr int HR = CAP >= BMT ? BMT : CAP >= BMT / 2 ? BMT / 2 : CAP >= BMT / 4 ? BMT / 4 : BMT / 8;
    static_assert(HR >= 8 && BMT % HR == 0 && HR * SPF * 4 <= mfma_lds_elems(S, BMT, CW) * 2,
                  "fp32 staging does not fit");
    float* xf = reinterpret_cast<float*>(xs);
    const int n0 = ftile * CW;
    __syncthreads();  // every wave is done with the activation stages
    for (int h0 = 0; h0 < BMT; h0 += HR) {
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          const int r = tt * 16 + (lane & 15) - h0;
          if (r < 0 || r >= HR) continue;
          floatx4 v = acc[ft][tt];
          if (WQ == 1) v *= s2;
          const int c = wave * WF + ft * 16 + 4 * (lane >> 4);
          *(floatx4*)(&xf[r * SPF + c]) = v;
        }
      __syncthreads();
      for (int q = tid; q < HR * (CW / 8); q += NTHR) {
        const int r = q / (CW / 8), c = (q % (CW / 8)) * 8;
        if (h0 + r < ti.rows && n0 + c < a.N) {
          const floatx4 v0 = *(const floatx4*)(&xf[r * SPF + c]);
          const floatx4 v1 = *(const floatx4*)(&xf[r * SPF + c + 4]);
          const size_t o = (size_t)(ti.row0 + h0 + r) * a.ldc + n0 + c;
          const bf16x8 rv = *(const bf16x8*)((const bf16*)a.res + o);
          float sum[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
          for (int i = 0; i < 8; ++i) sum[i] += (float)rv[i];
          if (a.add) {
            const bf16x8 av = *(const bf16x8*)((const bf16*)a.add + o);
#pragma unroll
            for (int i = 0; i < 8; ++i) sum[i] += (float)av[i];
          }
          bf16x8 ob;
#pragma unroll
          for (int i = 0; i < 8; ++i) ob[i] = (bf16)sum[i];
          *(bf16x8*)((bf16*)C + o) = ob;
        }
      }
      __syncthreads();
    }
  }
  __syncthreads();  // LDS is reused by the next item
}

template <int WF, int BMT, int NW, int EPI, typename TC, int WQ, bool GROUPED, bool NT,
          bool DEEP>
__global__ void __launch_bounds__(NW * 64, mfma_min_blocks(BMT, NW, DEEP))
    gemm_mfma_kernel(GemmArgs a, int nft, int slots, int wg_per_xcd, int rows_major) {
  __shared__ __attribute__((aligned(16)))
  bf16 xs[mfma_lds_elems(mfma_stages(BMT, NW, DEEP), BMT, NW * WF)];
  const int xcd = blockIdx.x & 7;
  const int live = GROUPED ? min(*a.num_tiles, slots) : slots;
  const int outer = rows_major ? live : nft;    // the axis split over the XCDs
  const int inner = rows_major ? nft : live;    // walked whole by each XCD
  const int chunk = (outer + 7) / 8;
  const int o0 = xcd * chunk;
  const int items = max(0, min(chunk, outer - o0)) * inner;
  const int nrows = max(0, min(chunk, outer - o0));
  // Grouped launches with a.sched take their items dynamically: after its
  // first item (blockIdx.x >> 3) a workgroup takes the next unclaimed item
  // of its XCD from a.sched[xcd] (claimed at the start of the current item,
  // so the atomic's latency hides under it), which evens out items of
  // different lengths (partial feature tiles, experts of different row
  // counts). The last workgroup of each XCD to finish re-arms both counters
  // for the next launch (a.sched[8 + xcd] counts finished workgroups).
  const bool dyn = GROUPED && a.sched != nullptr;
  __shared__ int s_next[2];  // alternating: one barrier per item suffices
  int item = blockIdx.x >> 3;
  for (int it = 0; item < items; ++it) {
    unsigned claimed = 0;
    if (dyn && threadIdx.x == 0) claimed = atomicAdd(&a.sched[xcd], 1u);
    int slot, ftile;
    if (rows_major) {
      // groups of RG row tiles; inside a group the RG row tiles of one feature
      // tile are adjacent items (they read the same weight slice together)
      constexpr int RG = 4;
      const int g = item / (RG * inner), rem = item - g * RG * inner;
      const int rg = min(RG, nrows - g * RG);
      slot = o0 + g * RG + rem % rg;
      ftile = rem / rg;
    } else {
      slot = item % inner;
      ftile = o0 + item / inner;
    }
    TileInfo ti;
    bool live_tile = true;
    if (GROUPED) {
      live_tile = decode_tile(a, slot, BMT, ti);  // uniform
    } else {
      ti.g = 0;
      ti.row0 = slot * BMT;
      ti.rows = min(BMT, a.M - ti.row0);
    }
    if (live_tile) {
      // Live 16-row blocks, rounded up to a quarter of the tile: a grouped
      // tile is sized for the larger experts (at 1024 tokens over 128 experts
      // 57% of the 16-row blocks of the 128-row tiles are padding).
      // The last body covers the whole tile when TT is not a multiple of Q.
      constexpr int TT = BMT / 16, Q = TT >= 4 ? TT / 4 : 1, NQ = (TT + Q - 1) / Q;
      const int ttl = (ti.rows + 15) >> 4;
      [&]<int... P>(std::integer_sequence<int, P...>) {
        ((ttl <= (P + 1) * Q || P + 1 == NQ
              ? (mfma_tile<WF, BMT, NW, EPI, TC, WQ, GROUPED, NT, DEEP,
                           std::min((P + 1) * Q, TT)>(a, ti, ftile, xs),
                 true)
              : false) ||
         ...);
      }(std::make_integer_sequence<int, NQ>{});
    }
    if (dyn) {
      if (threadIdx.x == 0) s_next[it & 1] = wg_per_xcd + (int)claimed;
      __syncthreads();
      item = s_next[it & 1];
    } else {
      item += wg_per_xcd;
    }
  }
  if (dyn && threadIdx.x == 0) {
    if (atomicAdd(&a.sched[8 + xcd], 1u) == (unsigned)wg_per_xcd - 1) {
      atomicExch(&a.sched[xcd], 0u);
      atomicExch(&a.sched[8 + xcd], 0u);
    }
  }
}

template <int WF, int BMT, int NW, int EPI, typename TC, int WQ, bool GROUPED, bool NT,
          bool DEEP>
static hipError_t launch_persistent(const GemmArgs& a, int slots, hipStream_t s) {
  static int occ = 0;  // resident workgroups per CU (queried once per process)
  if (occ == 0) {
    int o = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &o, (const void*)gemm_mfma_kernel<WF, BMT, NW, EPI, TC, WQ, GROUPED, NT, DEEP>, NW * 64,
            0) !=
            hipSuccess ||
        o < 1)
      o = 1;
    occ = o;
  }
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n < 8)
      n = 256;
    cus = n;
  }
  const int nft = (a.N + NW * WF - 1) / (NW * WF);
  // Dense: split the larger operand over the XCDs' L2s.
  const double wbytes = (double)a.N * a.K * (WQ ? 0.5625 : 2.0);
  const double abytes = (double)a.M * a.K * 2.0;
  const int rows_major = GROUPED || abytes > wbytes;
  const int outer = rows_major ? slots : nft, inner = rows_major ? nft : slots;
  const int max_items_per_xcd = ((outer + 7) / 8) * inner;
  const int wg_per_xcd = std::max(1, std::min(max_items_per_xcd, (cus / 8) * occ));
  hipLaunchKernelGGL((gemm_mfma_kernel<WF, BMT, NW, EPI, TC, WQ, GROUPED, NT, DEEP>),
                     dim3(8 * wg_per_xcd), dim3(NW * 64), 0, s, a, nft, slots, wg_per_xcd,
                     rows_major);
  return hipGetLastError();
}

template <int WF, int BMT, int NW, int WQ, bool G, bool NT, bool DEEP = false>
static hipError_t launch_mfma_shape(const GemmArgs& a, int epi, int slots, hipStream_t s) {
  switch (epi) {
    case EPI_RELU2:
      return launch_persistent<WF, BMT, NW, EPI_RELU2, bf16, WQ, G, NT, DEEP>(a, slots, s);
    case EPI_STORE:
      return launch_persistent<WF, BMT, NW, EPI_STORE, bf16, WQ, G, NT, DEEP>(a, slots, s);
    case EPI_ADD_RES:  // only the dense fc2 adds residual + shared
      if constexpr (G) return hipErrorInvalidValue;
      else return launch_persistent<WF, BMT, NW, EPI_ADD_RES, bf16, WQ, false, NT, DEEP>(a, slots, s);
    default: return hipErrorInvalidValue;
  }
}

// 128-row tiles take 8 waves (128 x 256 outputs per workgroup: a quarter
// less L1 traffic per MFMA) when that still gives every CU two tiles or more
// (dense launches: see dense8 below); smaller launches keep 4 waves so that
// more CUs get work, and dense bf16 ones with at most one 4-wave tile per CU
// take the DEEP variant.
template <int WQ, bool G, bool NT>
static hipError_t launch_mfma_wq(const GemmArgs& a, MfmaCfg cfg, int epi, int slots,
                                 hipStream_t s) {
  if (cfg.wf == 32 && cfg.bmt == 128) {
    static int cus = 0;
    if (cus == 0) {
      int dev = 0, n = 0;
      if (hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        n = 256;
      cus = n;
    }
    const long long items8 = (long long)slots * ((a.N + 255) / 256);
    const long long items4 = (long long)slots * ((a.N + 127) / 128);
    // Dense launches take 8 waves from one tile per CU, unless the last
    // 256-wide feature tile is partial and there are under 1.5 tiles per CU
    // (measured: 10-15% faster for the latent shared expert and for 3712-wide
    // up projections at 4096 tokens, 8-16% slower for 2688-wide down ones).
    const bool dense8 = !G && items8 >= (long long)cus &&
                        (a.N % 256 == 0 || 2 * items8 >= 3LL * cus);
    // Weight-streaming grouped bf16 launches (each expert one row tile) take
    // the feature width that needs the least time per XCD, with one
    // workgroup per CU for each: rounds of items x (features per item + a
    // fixed 128-feature equivalent per item), a fit to the two projections at
    // 1024 and 2048 tokens. 336 features (7 waves of 48) only where they
    // divide N: the 2688-wide down projection goes from 6 rounds of 256 (last
    // feature tile half dead) to 7 of 192 (238 -> 224 us) and to 4 of 336
    // (220 -> 210 us; 2048 tokens 237 -> 215 us); the 1856-wide up
    // projection keeps 4 rounds of 256 (5 of 192 measured 218 -> 225 us, 5 of
    // 384 210 -> 221 us). Where the MFMAs bound the launch, the uneven waves
    // per SIMD cost 10-20%, so NVFP4 weights and multi-tile experts keep 8
    // waves.
    if constexpr (G && NT && WQ == 0)
      if (cfg.est_tiles > 0 && items8 >= 2LL * cus) {
        const long long t = (cfg.est_tiles + 7) / 8, w = std::max(1, cus / 8);
        auto cost = [&](long long width) {
          return (t * ((a.N + width - 1) / width) + w - 1) / w * (width + 128);
        };
        const long long c192 = cost(192), c256 = cost(256);
        if (a.N % 336 == 0 && cost(336) < std::min(c192, c256))
          return launch_mfma_shape<48, 128, 7, WQ, G, NT>(a, epi, slots, s);
        if (c192 < c256) return launch_mfma_shape<32, 128, 6, WQ, G, NT>(a, epi, slots, s);
      }
    // Grouped NVFP4 launches of two tiles per CU or more take 48 features per
    // wave (8 waves, 128 x 384 outputs): each activation fragment read from
    // LDS feeds three MFMAs instead of two, and the weights (4.5 bits each,
    // decoded in registers) cost few registers. 2688 = 7 x 384; 1856 in 4.8
    // tiles. Measured 1024 / 2048 / 4096 / 8192 tokens: 0.401 / 0.509 /
    // 0.878 / 1.567 -> 0.382 / 0.486 / 0.820 / 1.450 ms. So do grouped bf16
    // launches over experts of several row tiles (the MFMAs, not the weight
    // stream, bound them) where 384-wide tiles pad N no more than 256-wide
    // ones (1856 and 2688 yes, 1024 no): direct layer at 4096 / 8192 / 16384
    // tokens 0.943 / 1.661 / 3.009 -> 0.892 / 1.575 / 2.838 ms; the latent
    // down projection (1024 wide) had lost 8% on them.
    if constexpr (G && (WQ == 1 || !NT))
      if (items8 >= 2LL * cus &&
          (WQ == 1 || (a.N + 383) / 384 * 384 <= (a.N + 255) / 256 * 256))
        return launch_mfma_shape<48, 128, 8, WQ, G, NT>(a, epi, slots, s);
    // Dense launches take the 48-feature waves where their 1.5x longer items
    // need fewer item-time rounds (224 items in one round instead of 352 in
    // two: shared down at 4096 tokens, NVFP4 102 -> 77 us, bf16 94 -> 78 us;
    // bf16 shared up at 16384 tokens 5 rounds instead of 8, 332 -> 312 us).
    if constexpr (!G) {
      const long long items48 = (long long)slots * ((a.N + 383) / 384);
      const long long r32 = (items8 + cus - 1) / cus, r48 = (items48 + cus - 1) / cus;
      if (items8 >= cus && 3 * r48 < 2 * r32)
        return launch_mfma_shape<48, 128, 8, WQ, G, NT>(a, epi, slots, s);
    }
    if (items8 >= 2LL * cus || dense8)
      return launch_mfma_shape<32, 128, 8, WQ, G, NT>(a, epi, slots, s);
    // A dense bf16 launch with at most one tile per CU runs one workgroup per
    // CU with a deeper pipeline.
    if constexpr (WQ == 0 && !G)
      if (items4 <= cus) return launch_mfma_shape<32, 128, 4, WQ, G, NT, true>(a, epi, slots, s);
    return launch_mfma_shape<32, 128, 4, WQ, G, NT>(a, epi, slots, s);
  }
#define SHAPE(W, M) \
  if (cfg.wf == W && cfg.bmt == M) return launch_mfma_shape<W, M, 4, WQ, G, NT>(a, epi, slots, s);
  SHAPE(16, 16) SHAPE(32, 32) SHAPE(32, 64)
#undef SHAPE
  // 192-row tiles (8 waves, 192 x 256 outputs): grouped launches whose
  // experts hold up to 192 rows each take one tile per expert.
  if constexpr (G)
    if (cfg.wf == 32 && cfg.bmt == 192) return launch_mfma_shape<32, 192, 8, WQ, G, NT>(a, epi, slots, s);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_mfma(const GemmArgs& a, MfmaCfg cfg, int epi, bool tc_bf16, bool nvfp4,
                            int slots, bool stream_weights, hipStream_t s) {
  if (!tc_bf16) return hipErrorInvalidValue;  // bf16 layers keep every intermediate in bf16
  if (a.tiles) {  // grouped
    if (stream_weights)
      return nvfp4 ? launch_mfma_wq<1, true, true>(a, cfg, epi, slots, s)
                   : launch_mfma_wq<0, true, true>(a, cfg, epi, slots, s);
    return nvfp4 ? launch_mfma_wq<1, true, false>(a, cfg, epi, slots, s)
                 : launch_mfma_wq<0, true, false>(a, cfg, epi, slots, s);
  }
  // dense: every row tile re-reads the matrix, so its loads stay cached
  return nvfp4 ? launch_mfma_wq<1, false, false>(a, cfg, epi, slots, s)
               : launch_mfma_wq<0, false, false>(a, cfg, epi, slots, s);
}

// ---------------------------------------------------------------------------
// Decode-sized GEMV arm (at most 16 rows per row tile).
// One launch covers up to two segments: the routed experts (grouped, tile
// list) and the shared expert (dense), so small batches need no side stream.
// Item = (segment, row tile, 16-feature tile); one workgroup per item; the 4
// waves take the item's k-steps in interleaved groups of GU and each issues
// the loads of a whole group at a time (weights and the <= 16 activation rows
// straight from memory into MFMA registers), so many loads are in flight per
// CU even for one token.
// The partial sums meet in LDS and are added in wave order (deterministic).
// ---------------------------------------------------------------------------
struct GemvArgs {
  GemmArgs seg[2];
  int nseg;
  int nft[2];    // 16-feature tiles per segment
  int slots[2];  // row-tile slots per segment (grouped: tile-list capacity)
};

template <int EPI, typename TC, int WQ>
__global__ void __launch_bounds__(256) gemv_kernel(GemvArgs g) {
  constexpr int GU = 4;  // k-steps per load group (6 and 8 measured no faster)
  using Src = WSrc<WQ, 1, true>;
  using Frag = typename Src::Frag;
  __shared__ floatx4 part[3][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // Segment 1 (dense, every item live, the longer K at these shapes) takes
  // the first block indices so that its items start first.
  int item = blockIdx.x;
  int sg = 0;
  if (g.nseg > 1) {
    const int n1 = g.slots[1] * g.nft[1];
    if (item < n1) sg = 1;
    else item -= n1;
  }
  const GemmArgs& a = g.seg[sg];
  const int slot = item / g.nft[sg];
  const int ftile = item - slot * g.nft[sg];
  TileInfo ti;
  if (!decode_tile(a, slot, 16, ti)) return;  // uniform: the whole workgroup leaves

  const int nsteps = a.K / 64;
  const int nf0 = ftile * 16;
  Src src;
  src.init(a, ti.g, nf0, lane);
  const int r = min(lane & 15, ti.rows - 1);
  const bf16* xp = (const bf16*)a.A + (size_t)a_row_of(a, ti.row0 + r) * a.lda + (lane >> 4) * 8;
  // output row (route order when c_rows is set), loaded before the k-loop
  const int crow = a.c_rows ? a.c_rows[ti.row0 + r] : ti.row0 + r;

  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  // Load groups of GU k-steps dealt round-robin to the 4 waves: at any time
  // the workgroup reads one contiguous run of its 16-feature tile (measured
  // 1% faster at 1-16 tokens than 4 separate quarter-K streams).
  for (int kb = wave * GU; kb < nsteps; kb += 4 * GU) {
    Frag w[GU];
    bf16x8 x[GU][2];
#pragma unroll
    for (int u = 0; u < GU; ++u) {
      const int ks = min(kb + u, nsteps - 1);  // past the end: a valid step, not used
      src.load(w[u], ks);
      x[u][0] = *(const bf16x8*)(xp + ks * 64);
      x[u][1] = *(const bf16x8*)(xp + ks * 64 + 32);
    }
    __builtin_amdgcn_sched_barrier(0);  // all GU steps' loads issue before any MFMA
#pragma unroll
    for (int u = 0; u < GU; ++u) {
      if (kb + u >= nsteps) break;
#pragma unroll
      for (int s = 0; s < 2; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(src.get(w[u], 0, s, lane), x[u][s], acc, 0,
                                                      0, 0);
    }
  }
  if (wave > 0) part[wave - 1][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  acc += part[0][lane];
  acc += part[1][lane];
  acc += part[2][lane];
  const int n = nf0 + 4 * (lane >> 4);
  const int row = lane & 15;
  const int p = crow;  // row == r for every lane that stores
  if (n < a.N && row < ti.rows) {
    if (WQ == 1) acc *= a.b_scale2[ti.g];
    if (EPI == EPI_RELU2) {
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = relu2(acc[q]);
    }
    if (EPI == EPI_ADD_RES) {
      acc += store4<TC>::ld((const TC*)a.res + (size_t)p * a.ldc + n);
      if (a.add) acc += store4<TC>::ld((const TC*)a.add + (size_t)p * a.ldc + n);
    }
    store4<TC>::st((TC*)a.C + (size_t)p * a.ldc + n, acc);
  }
}

hipError_t launch_gemv(const GemmArgs* segs, const int* slots, int nseg, int epi, bool nvfp4,
                       hipStream_t s) {
  GemvArgs g{};
  g.nseg = nseg;
  int total = 0;
  for (int i = 0; i < nseg; ++i) {
    g.seg[i] = segs[i];
    g.nft[i] = (segs[i].N + 15) / 16;
    g.slots[i] = slots[i];
    total += g.nft[i] * slots[i];
  }
  if (total == 0) return hipSuccess;
  dim3 grid(total);
#define GEMV_LAUNCH(E, Q)                                                                      \
  hipLaunchKernelGGL((gemv_kernel<E, bf16, Q>), grid, dim3(256), 0, s, g)
  if (nvfp4) {
    switch (epi) {
      case EPI_RELU2: GEMV_LAUNCH(EPI_RELU2, 1); break;
      case EPI_STORE: GEMV_LAUNCH(EPI_STORE, 1); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (epi) {
      case EPI_RELU2: GEMV_LAUNCH(EPI_RELU2, 0); break;
      case EPI_STORE: GEMV_LAUNCH(EPI_STORE, 0); break;
      case EPI_ADD_RES: GEMV_LAUNCH(EPI_ADD_RES, 0); break;
      default: return hipErrorInvalidValue;
    }
  }
#undef GEMV_LAUNCH
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Decode-sized down projection fused with the weighted reduce (direct
// layers): out[t] = residual[t] + sum over routes (t, j) of w[t*k+j] *
// (h[route] . W_down[expert]) + shared_down(g_sh[t]) (page "Struct MoeLayer",
// `forward_prefill`: down GEMM, unpermute, weighted reduce, shared expert
// added; page "metrale_model_arch/nemotron_moe.rs", module doc: routed
// weighted sum plus the shared expert, added to hidden).
// One workgroup per 16 output features. Its waves take whole items: the
// routed 16-row tiles of the decode tile list (one expert each) and the
// shared expert's k-range splits, dealt round-robin. Each wave adds the
// routing-weighted results of its items into its own [token][feature] LDS
// partial (a tile holds distinct tokens, so the lanes of a wave never
// collide); the partials are summed in wave order and added to the residual
// once, in fp32, so the result is deterministic and the routed outputs never
// leave the CU.
// ---------------------------------------------------------------------------
template <int WQ>
__global__ void __launch_bounds__(GEMV_REDUCE_WAVES * 64) gemv_down_reduce_kernel(GemvReduceArgs g) {
  constexpr int NWV = GEMV_REDUCE_WAVES;
  constexpr int RING = 6;  // k-steps in flight per wave
  using Src = WSrc<WQ, 1, true>;
  using Frag = typename Src::Frag;
  __shared__ floatx4 part[NWV][16][4];  // [wave][token][4-feature group]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 16;
  const int r = lane & 15, fg = lane >> 4;
  part[wave][r][fg] = floatx4{0.f, 0.f, 0.f, 0.f};
  const GemmArgs& ra = g.routed;
  const int nt = *ra.num_tiles;
  const int items = nt + g.shared_splits;
  for (int it = wave; it < items; it += NWV) {
    const bool routed = it < nt;
    // the item's operand fields, selected per field (a reference to either
    // kernel argument would place them in scratch memory)
    GemmArgs a;
    a.A = routed ? ra.A : g.shared.A;
    a.lda = routed ? ra.lda : g.shared.lda;
    a.B = routed ? ra.B : g.shared.B;
    a.b_gstride = routed ? ra.b_gstride : g.shared.b_gstride;
    a.b_scales = routed ? ra.b_scales : g.shared.b_scales;
    a.bs_gstride = routed ? ra.bs_gstride : g.shared.bs_gstride;
    a.b_scale2 = routed ? ra.b_scale2 : g.shared.b_scale2;
    a.N = routed ? ra.N : g.shared.N;
    a.K = routed ? ra.K : g.shared.K;
    a.b_kmajor = routed ? ra.b_kmajor : g.shared.b_kmajor;
    int grp, row0, rows, k0, k1;
    if (routed) {
      TileInfo ti;
      if (!decode_tile(ra, it, 16, ti)) continue;  // uniform per wave
      grp = ti.g; row0 = ti.row0; rows = ti.rows;
      k0 = 0; k1 = a.K / 64;
    } else {
      const int sp = it - nt, ks = a.K / 64;
      grp = 0; row0 = 0; rows = g.n;
      k0 = (int)((long long)ks * sp / g.shared_splits);
      k1 = (int)((long long)ks * (sp + 1) / g.shared_splits);
    }
    Src src;
    src.init(a, grp, n0, lane);
    const bf16* xp =
        (const bf16*)a.A + (size_t)(row0 + min(r, rows - 1)) * a.lda + fg * 8;
    // Rolling ring of RING k-steps per wave: the loads of step ks + RING are
    // issued as soon as step ks has been consumed, so a wave (one workgroup
    // per CU here) keeps RING steps in flight through the whole k-range.
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    Frag wv[RING];
    bf16x8 x[RING][2];
    auto load = [&](int slot_ks, Frag& f, bf16x8* xs2) __attribute__((always_inline)) {
      const int ks = min(slot_ks, k1 - 1);  // past the range: a valid step, not used
      src.load(f, ks);
      xs2[0] = *(const bf16x8*)(xp + ks * 64);
      xs2[1] = *(const bf16x8*)(xp + ks * 64 + 32);
    };
#pragma unroll
    for (int u = 0; u < RING; ++u) load(k0 + u, wv[u], x[u]);
    for (int kb = k0; kb < k1; kb += RING) {
#pragma unroll
      for (int u = 0; u < RING; ++u) {
        if (kb + u < k1) {
#pragma unroll
          for (int s = 0; s < 2; ++s)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(src.get(wv[u], 0, s, lane), x[u][s],
                                                          acc, 0, 0, 0);
          if (kb + u + RING < k1) load(kb + u + RING, wv[u], x[u]);
        }
      }
    }
    // lane: features n0 + 4*fg .. +3 of tile row r
    if (r < rows) {
      if (WQ == 1) acc *= a.b_scale2[grp];
      int t = r;
      if (routed) {
        const int rid = g.perm[row0 + r];
        t = rid / g.k;
        acc *= g.w[rid];
      }
      part[wave][t][fg] += acc;
    }
  }
  __syncthreads();
  if (wave != 0 || r >= g.n) return;
  floatx4 sum = part[0][r][fg];
#pragma unroll
  for (int w = 1; w < NWV; ++w) sum += part[w][r][fg];
  const size_t o = (size_t)r * g.ldo + n0 + 4 * fg;
  sum = store4<bf16>::ld(g.residual + o) + sum;
  store4<bf16>::st(g.out + o, sum);
}

hipError_t launch_gemv_down_reduce(const GemvReduceArgs& g, int D, bool nvfp4, hipStream_t s) {
  if (D % 16 != 0 || g.n < 1 || g.n > 16) return hipErrorInvalidValue;
  const dim3 grid(D / 16), block(GEMV_REDUCE_WAVES * 64);
  if (nvfp4)
    hipLaunchKernelGGL(gemv_down_reduce_kernel<1>, grid, block, 0, s, g);
  else
    hipLaunchKernelGGL(gemv_down_reduce_kernel<0>, grid, block, 0, s, g);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Re-tile [G][N][K] row-major bf16 into the MFMA A-operand lane order:
// feature-major [G][N/16][K/32][64][8] or k-major [G][K/64][N/16][2][64][8].
// One thread per 16-byte destination chunk.
// ---------------------------------------------------------------------------
__global__ void retile_bf16_kernel(const bf16* __restrict__ src, bf16* __restrict__ dst, int G,
                                   int N, int K, int kmajor) {
  const size_t chunks = (size_t)G * N * K / 8;
  const int KC = K / 32, NT = N / 16, KS = K / 64;
  for (size_t c = blockIdx.x * (size_t)blockDim.x + threadIdx.x; c < chunks;
       c += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(c & 63);
    size_t blk = c >> 6;
    int kc, rt;
    size_t g;
    if (kmajor) {  // (g, ks, rt, s)
      const int s = (int)(blk & 1);
      blk >>= 1;
      rt = (int)(blk % NT);
      blk /= NT;
      kc = (int)(blk % KS) * 2 + s;
      g = blk / KS;
    } else {  // (g, rt, kc)
      kc = (int)(blk % KC);
      blk /= KC;
      rt = (int)(blk % NT);
      g = blk / NT;
    }
    const int row = rt * 16 + (lane & 15);
    const int k = kc * 32 + 8 * (lane >> 4);
    *(bf16x8*)(dst + c * 8) = *(const bf16x8*)(src + (g * N + row) * (size_t)K + k);
  }
}

hipError_t launch_retile_bf16(const bf16* src, bf16* dst, int G, int N, int K, bool kmajor,
                              hipStream_t s) {
  const size_t chunks = (size_t)G * N * K / 8;
  const int blocks = (int)std::min<size_t>((chunks + 255) / 256, 65536);
  hipLaunchKernelGGL(retile_bf16_kernel, dim3(blocks), dim3(256), 0, s, src, dst, G, N, K,
                     kmajor ? 1 : 0);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Re-tile NVFP4 [G][N][K/2] packed bytes and [G][N][K/16] E4M3 scales into the
// lane order of the MFMA kernel: packed -> [G][N/16][K/64][64 lanes][8 bytes]
// (lane l: row l%16; bytes 4*(l/16)..+3 and 16 + 4*(l/16)..+3 of the row's
// 32-byte k-step), scales -> [G][N/16][K/64][16 rows][4 bytes].
// ---------------------------------------------------------------------------
__global__ void retile_nvfp4_kernel(const uint8_t* __restrict__ qsrc,
                                    const uint8_t* __restrict__ ssrc, uint8_t* __restrict__ qdst,
                                    uint8_t* __restrict__ sdst, int G, int N, int K) {
  const int KS = K / 64, NT = N / 16;
  const size_t lanes = (size_t)G * NT * KS * 64;
  for (size_t c = blockIdx.x * (size_t)blockDim.x + threadIdx.x; c < lanes;
       c += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(c & 63);
    size_t blk = c >> 6;  // (g, rt, ks)
    const int ks = (int)(blk % KS);
    blk /= KS;
    const int rt = (int)(blk % NT);
    const size_t g = blk / NT;
    const int row = rt * 16 + (lane & 15);
    const uint8_t* rq = qsrc + (g * N + row) * (size_t)(K / 2) + ks * 32 + 4 * (lane >> 4);
    const uint32_t lo = *(const uint32_t*)rq;
    const uint32_t hi = *(const uint32_t*)(rq + 16);
    *(u32x2*)(qdst + c * 8) = u32x2{lo, hi};
    if (lane < 16) {
      const uint8_t* rs = ssrc + (g * N + rt * 16 + lane) * (size_t)(K / 16) + ks * 4;
      *(uint32_t*)(sdst + ((blk * KS + ks) * 16 + lane) * 4) = *(const uint32_t*)rs;
    }
  }
}

hipError_t launch_retile_nvfp4(const uint8_t* qsrc, const uint8_t* ssrc, uint8_t* qdst,
                               uint8_t* sdst, int G, int N, int K, hipStream_t s) {
  const size_t lanes = (size_t)G * (N / 16) * (K / 64) * 64;
  const int blocks = (int)std::min<size_t>((lanes + 255) / 256, 65536);
  hipLaunchKernelGGL(retile_nvfp4_kernel, dim3(blocks), dim3(256), 0, s, qsrc, ssrc, qdst, sdst, G,
                     N, K);
  return hipGetLastError();
}
