// Routing front end of the MoE layer on gfx950:
//   norm_gate_lds_kernel   bf16: RMSNorm (+ residual save) fused with the gate
//                          projection on MFMA, token rows staged in LDS
//   norm_gate_mfma_kernel  bf16, H too large for the LDS staging
//   norm_gate_kernel       fp32 layers (SIMT)
//   topk_sigmoid_kernel    wave64 sigmoid top-k with renormalized weights
//   route_sort_kernel      per-expert histogram, prefix sum and stable scatter,
//                          plus the (expert, row-block) tile list of the
//                          grouped GEMMs (one workgroup; route_hist_kernel +
//                          route_scatter_kernel when R exceeds one chunk)
//   route_small_kernel     decode-sized batches: all of the above in one launch
//
// Sources: page "metrale_model_arch/nemotron_moe.rs" (module doc: forward
// order RMS norm -> gate -> sigmoid top-k; `prefill`: rms_norm_residual,
// gate GEMM, scratch carve-out of ids and weights); page "Struct MoeLayer"
// (`forward_prefill`: sort-by-expert before the grouped GEMMs; `forward`:
// routing stays on the device; `fp32_routing_active`: router input at full
// precision).
#include "kernels.h"

// ---------------------------------------------------------------------------
// Fused RMSNorm + gate.
// Block = 256 threads (4 waves) handles TM tokens and experts
// [blockIdx.y * epb, min(E, (blockIdx.y + 1) * epb)).
//   1. sum of squares of each token row (one wave per token, TM <= 4 here)
//   2. normed rows in fp32 -> LDS; blockIdx.y == 0 also writes `normed` in the
//      activation dtype and `residual = hidden`
//   3. logits[t][e] = sum_i W_g[e][i] * n_f32[t][i]: lanes split the hidden
//      dimension in 8-element chunks, waves take experts in turn, and each
//      expert's partial sums end in a wave reduction.
// The gate reads the fp32 normed values, never the rounded copy, so the top-k
// decision sees full-precision logits.
// ---------------------------------------------------------------------------
template <typename TA, int TM>
__global__ void __launch_bounds__(256) norm_gate_kernel(const TA* __restrict__ hidden,
                                                        const TA* __restrict__ gamma,
                                                        const TA* __restrict__ wgate,
                                                        TA* __restrict__ normed,
                                                        TA* __restrict__ residual,
                                                        float* __restrict__ logits, int n,
                                                        int H, int E, int epb, float eps) {
  extern __shared__ float nsh[];  // [TM][H] fp32 normed rows
  __shared__ float rinv[TM];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * TM;
  const int tcount = min(TM, n - t0);

  // 1. inverse RMS per token
  for (int t = wave; t < TM; t += 4) {
    float ss = 0.f;
    if (t < tcount) {
      const TA* x = hidden + (size_t)(t0 + t) * H;
      for (int i = lane; i < H; i += 64) {
        float v = io<TA>::ld(x + i);
        ss += v * v;
      }
    }
    ss = wave_sum(ss);
    if (lane == 0) rinv[t] = 1.0f / sqrtf(ss / (float)H + eps);
  }
  __syncthreads();

  // 2. normed rows
  const bool writer = blockIdx.y == 0;
  for (int idx = threadIdx.x; idx < TM * H; idx += 256) {
    int t = idx / H, i = idx - t * H;
    float v = 0.f;
    if (t < tcount) {
      size_t g = (size_t)(t0 + t) * H + i;
      float x = io<TA>::ld(hidden + g);
      v = x * rinv[t] * io<TA>::ld(gamma + i);
      if (writer) {
        io<TA>::st(residual + g, x);
        io<TA>::st(normed + g, v);
      }
    }
    nsh[idx] = v;
  }
  __syncthreads();

  // 3. gate logits
  const int e_begin = blockIdx.y * epb;
  const int e_end = min(E, e_begin + epb);
  for (int e = e_begin + wave; e < e_end; e += 4) {
    float acc[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) acc[t] = 0.f;
    const TA* wrow = wgate + (size_t)e * H;
    for (int i0 = lane * 8; i0 < H; i0 += 512) {
      float wv[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) wv[q] = io<TA>::ld(wrow + i0 + q);
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        const float* nr = nsh + t * H + i0;
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[t] += wv[q] * nr[q];
      }
    }
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      float s = wave_sum(acc[t]);
      if (lane == 0 && t < tcount) logits[(size_t)(t0 + t) * E + e] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// Fused RMSNorm + gate for bf16 layers, on MFMA.
// Block = 4 waves, 16 tokens x experts [blockIdx.y * epb, +epb) (epb % 16 == 0).
//   1. inverse RMS of the 16 rows (each wave 4 rows)
//   2. the 32-wide k-steps of the hidden dimension are dealt round-robin to the
//      waves; a lane builds the MFMA B operand (token lane%16, k-elements
//      8*(lane/16)..+7) from hidden * rinv * gamma in fp32, writes normed
//      (bf16) and residual once (blockIdx.y == 0), and splits the fp32 value
//      into hi = bf16(n) and lo = bf16(n - hi). Two MFMAs per expert tile,
//      W_g x hi + W_g x lo, give logits with ~16 mantissa bits of n: the top-k
//      decision sees (nearly) the fp32 normed vector, not its bf16 rounding.
//   3. the four waves' partial sums meet in LDS and are added in wave order.
// Output lane layout: experts 4*(lane/16)+0..3 of token lane%16 (16-byte store).
// ---------------------------------------------------------------------------
template <int ET>  // expert tiles of 16 per block
__global__ void __launch_bounds__(256) norm_gate_mfma_kernel(const bf16* __restrict__ hidden,
                                                             const bf16* __restrict__ gamma,
                                                             const bf16* __restrict__ wgate,
                                                             bf16* __restrict__ normed,
                                                             bf16* __restrict__ residual,
                                                             float* __restrict__ logits, int n,
                                                             int H, int E, float eps) {
  __shared__ float rinv[16];
  __shared__ floatx4 red[4][ET][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 16;
  const int e0 = blockIdx.y * ET * 16;

  // 1. inverse RMS (each wave: rows wave*4 .. +3; the 16-byte loads of all
  //    four rows are issued together, 4 chunks per row at a time).
  {
    float ss[4] = {0.f, 0.f, 0.f, 0.f};
    for (int i0 = lane * 8; i0 < H; i0 += 512 * 4) {
      bf16x8 v[4][4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = wave * 4 + r;
        const bf16* x = hidden + (size_t)min(t0 + t, n - 1) * H;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + u * 512;
          v[r][u] = i < H ? *(const bf16x8*)(x + i) : bf16x8{};
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const float f = (float)v[r][u][q];
            ss[r] += f * f;
          }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float tot = wave_sum(ss[r]);
      if (lane == 0) rinv[wave * 4 + r] = 1.0f / sqrtf(tot / (float)H + eps);
    }
  }
  __syncthreads();

  // 2. k-steps of 32, dealt round-robin to the waves
  const int tok = lane & 15, kg = lane >> 4;
  const bool tvalid = t0 + tok < n;
  const float rv = rinv[tok];
  const bool writer = blockIdx.y == 0;
  const bf16* wbase[ET];
#pragma unroll
  for (int et = 0; et < ET; ++et) {
    const int e = min(e0 + et * 16 + tok, E - 1);  // rows past E: valid memory, never stored
    wbase[et] = wgate + (size_t)e * H + kg * 8;
  }
  floatx4 acc[ET];
#pragma unroll
  for (int et = 0; et < ET; ++et) acc[et] = floatx4{0.f, 0.f, 0.f, 0.f};
  const size_t row = (size_t)(t0 + tok) * H + kg * 8;
  // U k-steps per round: their loads are issued before any of them is used.
  constexpr int U = ET >= 8 ? 2 : 16 / ET > 8 ? 8 : 16 / ET;
  for (int kb = wave * 32; kb < H; kb += 128 * U) {
    bf16x8 wf[U][ET], xv[U], gv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k0 = min(kb + u * 128, H - 32);  // past the end: a valid step, not used
#pragma unroll
      for (int et = 0; et < ET; ++et) wf[u][et] = *(const bf16x8*)(wbase[et] + k0);
      xv[u] = tvalid ? *(const bf16x8*)(hidden + row + k0) : bf16x8{};
      gv[u] = *(const bf16x8*)(gamma + k0 + kg * 8);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k0 = kb + u * 128;
      if (k0 >= H) break;
      bf16x8 hi, lo, nb;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float v = (float)xv[u][q] * rv * (float)gv[u][q];
        hi[q] = (bf16)v;
        lo[q] = (bf16)(v - (float)hi[q]);
        nb[q] = hi[q];
      }
      if (writer && tvalid) {
        *(bf16x8*)(residual + row + k0) = xv[u];
        *(bf16x8*)(normed + row + k0) = nb;
      }
#pragma unroll
      for (int et = 0; et < ET; ++et) {
        acc[et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[u][et], hi, acc[et], 0, 0, 0);
        acc[et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[u][et], lo, acc[et], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int et = 0; et < ET; ++et) red[wave][et][lane] = acc[et];
  __syncthreads();

  // 3. cross-wave sum (wave w finishes tiles w, w+4, ...), fixed order
  for (int et = wave; et < ET; et += 4) {
    floatx4 v = red[0][et][lane];
    v += red[1][et][lane];
    v += red[2][et][lane];
    v += red[3][et][lane];
    const int e = e0 + et * 16 + 4 * kg;
    if (tvalid && e < E) {
      float* dst = logits + (size_t)(t0 + tok) * E + e;
      if (e + 3 < E && (E & 3) == 0) {
        *(floatx4*)dst = v;
      } else {
        for (int q = 0; q < 4 && e + q < E; ++q) dst[q] = v[q];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Sigmoid top-k. One wave64 per token; lane l holds experts l, l+64, ...
// Selection key = (fp32 bits of the score) << 32 | (0xFFFFFFFF - e): scores
// lie in [0, 1], so their bit patterns order like the values, and among equal
// scores the lower expert index has the larger key. k rounds of a wave-wide
// 64-bit max reduction pick the experts in slot order (score desc, index asc).
// ---------------------------------------------------------------------------
template <int EPL>
__device__ __forceinline__ void topk_token(const float* __restrict__ lrow, int E, int k,
                                           float scale, int* __restrict__ ids_row,
                                           float* __restrict__ w_row, int lane) {
  uint64_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    int e = lane + 64 * i;
    key[i] = 0;
    if (e < E) {
      float l = lrow[e];
      float s = 1.0f / (1.0f + expf(-l));
      key[i] = ((uint64_t)__float_as_uint(s) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
    }
  }
  int my_e = 0;
  float my_s = 0.f, sum = 0.f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const int e = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFu));
    const float s = __uint_as_float((uint32_t)(best >> 32));
    sum += s;
    if (lane == j) { my_e = e; my_s = s; }
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane + 64 * i == e) key[i] = 0;
  }
  if (lane < k) {
    float wv = sum > 0.f ? my_s / sum : 1.0f / (float)k;
    ids_row[lane] = my_e;
    w_row[lane] = wv * scale;
  }
}

template <int EPL>
__global__ void __launch_bounds__(256) topk_sigmoid_kernel(const float* __restrict__ logits,
                                                           int n, int E, int k, float scale,
                                                           int* __restrict__ ids,
                                                           float* __restrict__ wout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= n) return;
  topk_token<EPL>(logits + (size_t)t * E, E, k, scale, ids + (size_t)t * k, wout + (size_t)t * k,
                  lane);
}

// ---------------------------------------------------------------------------
// Stable route sort in one workgroup of 1024 threads (16 waves).
//   phase 1: per-expert histogram (LDS atomics: counts do not depend on order)
//   phase 2: exclusive prefix sum -> offsets; tile list of ceil(count/bm)
//            (expert, first local row) pairs per expert
//   phase 3: routes in chunks of 1024, in order. Inside a wave, the lanes
//            holding the same expert are found with one ballot per id bit;
//            a lane's rank is the number of such lanes below it. Waves add the
//            counts of lower waves in the same chunk, and the chunk adds the
//            running base of its expert. So positions ascend with the route id
//            within an expert: the order is stable and deterministic.
// Ids outside [0, E) are skipped (they get no position).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, WAVE);
    if (lane >= o) v += u;
  }
  return v;
}

struct SortLds {
  int cnt[MOE_MAX_E];
  int base[MOE_MAX_E];
  int wcnt[16][MOE_MAX_E];
  int wsum[2][16];
};

// The whole one-workgroup sort (1024 threads; every thread must call it).
__device__ void sort_block(const int* __restrict__ ids, int R, int E, int* __restrict__ counts,
                           int* __restrict__ offsets, int* __restrict__ perm,
                           int* __restrict__ inv, int bm, int2* __restrict__ tiles,
                           int* __restrict__ num_tiles, SortLds& L) {
  constexpr int RPT = 16;  // routes per thread loaded per batch (one load latency)
  int* cnt = L.cnt;
  int* base = L.base;
  auto& wcnt = L.wcnt;
  auto& wsum = L.wsum;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  for (int e = tid; e < MOE_MAX_E; e += 1024) {
    cnt[e] = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) wcnt[w][e] = 0;
  }
  __syncthreads();
  // 1. histogram
  for (int b0 = 0; b0 < R; b0 += 1024 * RPT) {
    int ev[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = b0 + i * 1024 + tid;
      ev[i] = r < R ? ids[r] : -1;
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      if (ev[i] >= 0 && ev[i] < E) atomicAdd(&cnt[ev[i]], 1);
  }
  __syncthreads();

  // 2. exclusive scans over experts of counts and tile counts (E <= 512:
  //    threads 0..511, 8 waves; wave-level shuffles, then the wave totals).
  const int c = tid < E ? cnt[tid] : 0;
  const int tc = (tid < E && bm > 0) ? (c + bm - 1) / bm : 0;
  const int ic = wave_incl_scan(c, lane), itc = wave_incl_scan(tc, lane);
  if (lane == 63) {
    wsum[0][wave] = ic;
    wsum[1][wave] = itc;
  }
  __syncthreads();
  int pc = 0, ptc = 0;
  for (int w = 0; w < wave; ++w) {
    pc += wsum[0][w];
    ptc += wsum[1][w];
  }
  if (tid < E) {
    const int excl = pc + ic - c;
    const int texcl = ptc + itc - tc;
    base[tid] = excl;
    counts[tid] = c;
    offsets[tid] = excl;
    if (tid == E - 1) {
      offsets[E] = excl + c;
      if (num_tiles) *num_tiles = texcl + tc;
    }
    if (tiles)
      for (int i = 0; i < tc; ++i) tiles[texcl + i] = make_int2(tid, i * bm);
  }
  __syncthreads();

  // 3. stable scatter, chunks of 1024 routes in order
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int b0 = 0; b0 < R; b0 += 1024 * RPT) {
    int ev[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = b0 + i * 1024 + tid;
      ev[i] = r < R ? ids[r] : -1;
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int c0 = b0 + i * 1024;
      if (c0 >= R) break;  // uniform across the block
      const int r = c0 + tid;
      const bool valid = ev[i] >= 0 && ev[i] < E;
      const int e = valid ? ev[i] : -1;
      uint64_t mask = __ballot(valid);
#pragma unroll
      for (int b = 0; b < 10; ++b) {  // 10 bits cover E <= 1024
        const bool bit = valid && ((e >> b) & 1);
        const uint64_t bal = __ballot(bit);
        mask &= bit ? bal : ~bal;
      }
      const int rank = __popcll(mask & below);
      if (valid && rank == 0) wcnt[wave][e] = __popcll(mask);
      __syncthreads();
      if (valid) {
        int pre = 0;
        for (int w = 0; w < wave; ++w) pre += wcnt[w][e];
        const int pos = base[e] + pre + rank;
        perm[pos] = r;
        inv[r] = pos;
      }
      __syncthreads();
      for (int ee = tid; ee < E; ee += 1024) {
        int sum = 0;
#pragma unroll
        for (int w = 0; w < 16; ++w) {
          sum += wcnt[w][ee];
          wcnt[w][ee] = 0;
        }
        base[ee] += sum;
      }
      __syncthreads();
    }
  }
}

__global__ void __launch_bounds__(1024) route_sort_kernel(const int* __restrict__ ids, int R,
                                                          int E, int* __restrict__ counts,
                                                          int* __restrict__ offsets,
                                                          int* __restrict__ perm,
                                                          int* __restrict__ inv, int bm,
                                                          int2* __restrict__ tiles,
                                                          int* __restrict__ num_tiles) {
  __shared__ SortLds lds;
  sort_block(ids, R, E, counts, offsets, perm, inv, bm, tiles, num_tiles, lds);
}

// ---------------------------------------------------------------------------
// Multi-block stable route sort for large R (two launches).
//   route_hist_kernel: block b counts the experts of routes [b*CH, (b+1)*CH)
//                      -> bcnt[b][E]
//   route_scatter_kernel: block b adds up bcnt over all blocks (totals and the
//                      part of lower blocks), scans over experts, and scatters
//                      its own chunk in order with the same ballot ranking as
//                      route_sort_kernel. Block 0 also writes counts, offsets
//                      and the tile list. Same result as the one-block kernel.
// ---------------------------------------------------------------------------
constexpr int SORT_CH = 2048;  // routes per block (2 per thread)

__global__ void __launch_bounds__(1024) route_hist_kernel(const int* __restrict__ ids, int R, int E,
                                                          int* __restrict__ bcnt) {
  __shared__ int cnt[MOE_MAX_E];
  const int tid = threadIdx.x;
  for (int e = tid; e < MOE_MAX_E; e += 1024) cnt[e] = 0;
  __syncthreads();
  const int r0 = blockIdx.x * SORT_CH;
  int ev[SORT_CH / 1024];
#pragma unroll
  for (int i = 0; i < SORT_CH / 1024; ++i) {
    const int r = r0 + i * 1024 + tid;
    ev[i] = r < R ? ids[r] : -1;
  }
#pragma unroll
  for (int i = 0; i < SORT_CH / 1024; ++i)
    if (ev[i] >= 0 && ev[i] < E) atomicAdd(&cnt[ev[i]], 1);
  __syncthreads();
  for (int e = tid; e < E; e += 1024) bcnt[(size_t)blockIdx.x * E + e] = cnt[e];
}

__global__ void __launch_bounds__(1024) route_scatter_kernel(
    const int* __restrict__ ids, int R, int E, const int* __restrict__ bcnt,
    int* __restrict__ counts, int* __restrict__ offsets, int* __restrict__ perm,
    int* __restrict__ inv, int bm, int2* __restrict__ tiles, int* __restrict__ num_tiles) {
  __shared__ int base[MOE_MAX_E];
  __shared__ int wcnt[16][MOE_MAX_E];
  __shared__ int wsum[2][16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nb = gridDim.x, b = blockIdx.x;
  for (int e = tid; e < MOE_MAX_E; e += 1024)
#pragma unroll
    for (int w = 0; w < 16; ++w) wcnt[w][e] = 0;
  // Totals and lower-block parts per expert (E <= 512 < 1024 threads).
  int c = 0, lower = 0;
  if (tid < E) {
    for (int bb = 0; bb < nb; ++bb) {
      const int v = bcnt[(size_t)bb * E + tid];
      c += v;
      if (bb < b) lower += v;
    }
  }
  const int tc = (tid < E && bm > 0) ? (c + bm - 1) / bm : 0;
  const int ic = wave_incl_scan(c, lane), itc = wave_incl_scan(tc, lane);
  if (lane == 63) {
    wsum[0][wave] = ic;
    wsum[1][wave] = itc;
  }
  __syncthreads();
  int pc = 0, ptc = 0;
  for (int w = 0; w < wave; ++w) {
    pc += wsum[0][w];
    ptc += wsum[1][w];
  }
  if (tid < E) {
    const int excl = pc + ic - c;
    base[tid] = excl + lower;
    if (b == 0) {
      const int texcl = ptc + itc - tc;
      counts[tid] = c;
      offsets[tid] = excl;
      if (tid == E - 1) {
        offsets[E] = excl + c;
        if (num_tiles) *num_tiles = texcl + tc;
      }
      if (tiles)
        for (int i = 0; i < tc; ++i) tiles[texcl + i] = make_int2(tid, i * bm);
    }
  }
  __syncthreads();

  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int r0 = b * SORT_CH;
  int ev[SORT_CH / 1024];
#pragma unroll
  for (int i = 0; i < SORT_CH / 1024; ++i) {
    const int r = r0 + i * 1024 + tid;
    ev[i] = r < R ? ids[r] : -1;
  }
#pragma unroll
  for (int i = 0; i < SORT_CH / 1024; ++i) {
    const int c0 = r0 + i * 1024;
    if (c0 >= R) break;  // uniform across the block
    const int r = c0 + tid;
    const bool valid = ev[i] >= 0 && ev[i] < E;
    const int e = valid ? ev[i] : -1;
    uint64_t mask = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 10; ++bit) {
      const bool on = valid && ((e >> bit) & 1);
      const uint64_t bal = __ballot(on);
      mask &= on ? bal : ~bal;
    }
    const int rank = __popcll(mask & below);
    if (valid && rank == 0) wcnt[wave][e] = __popcll(mask);
    __syncthreads();
    if (valid) {
      int pre = 0;
      for (int w = 0; w < wave; ++w) pre += wcnt[w][e];
      const int pos = base[e] + pre + rank;
      perm[pos] = r;
      inv[r] = pos;
    }
    __syncthreads();
    for (int ee = tid; ee < E; ee += 1024) {
      int sum = 0;
#pragma unroll
      for (int w = 0; w < 16; ++w) {
        sum += wcnt[w][ee];
        wcnt[w][ee] = 0;
      }
      base[ee] += sum;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// RMSNorm + gate for bf16 layers with the token rows staged in LDS.
// Block = 8 waves, 16 tokens x ET expert tiles of 16.
//   0. Each wave issues the loads of its first batch of gate fragments at
//      entry: they do not depend on the rows, so their latency overlaps the
//      row loads.
//   1. The 16 hidden rows are read once with contiguous 16-byte loads into
//      LDS (row stride H + 8 elements: the 16 rows of an MFMA operand read
//      fall in distinct banks); each wave issues the loads of both its rows
//      before it uses any, and sums the squares of its rows. gamma is staged
//      as well.
//   2. Wave w takes the k-steps j = w, w + 8, ... of every expert tile of the
//      block. The B operand is built once per step from LDS: y = x * gamma,
//      exact in fp32 (two 8-bit mantissas), split into hi = bf16(y) and
//      lo = bf16(y - hi), so the dot products see y to ~16 bits; each expert
//      tile then takes two MFMAs with its A operand (gate rows from the
//      pre-tiled gate matrix [E16/16][H/32][64 lanes][8], one contiguous 1 KiB
//      per wave load), loaded in batches of NG_F fragments, the next batch in
//      flight while one computes.
//   3. The 8 partial sums of a tile meet in LDS (over the staged rows, which
//      are dead by then) and are added in wave order, then scaled by the row's
//      fp32 inverse RMS: logit = rinv * (W_g . y), the gate of the fp32 normed
//      row.
//   The residual copy and normed = bf16(n) are written by all blocks of a
//   token group, each taking one contiguous range of 16-byte column chunks.
// ---------------------------------------------------------------------------
constexpr size_t NG_LDS_MAX = 160 * 1024;
constexpr int NG_F = 16;  // gate fragments per load batch
constexpr int NG_NB = 8;  // 16-byte chunks per lane and row in one load round

// LDS of one block: 16 rows of H + 8 (later the 8 x ET partial-sum tiles),
// gamma, 16 inverse RMS.
inline size_t norm_gate_lds_bytes(int H, int et) {
  const size_t rows = (size_t)16 * (H + 8) * 2, red = (size_t)8 * et * 64 * 16;
  return std::max(rows, red) + (size_t)H * 2 + 16 * 4;
}

template <int ET>
__global__ void __launch_bounds__(512) norm_gate_lds_kernel(const bf16* __restrict__ hidden,
                                                            const bf16* __restrict__ gamma,
                                                            const bf16* __restrict__ wgate_t,
                                                            bf16* __restrict__ normed,
                                                            bf16* __restrict__ residual,
                                                            float* __restrict__ logits, int n,
                                                            int H, int E, float eps) {
  extern __shared__ __attribute__((aligned(16))) unsigned char ng_smem[];
  constexpr int U = NG_F / ET;  // k-steps per batch
  const int HP = H + 8;
  const size_t rows_bytes = std::max((size_t)16 * HP * 2, (size_t)8 * ET * 64 * 16);
  bf16* xs = (bf16*)ng_smem;                          // [16][HP]
  floatx4* red = (floatx4*)ng_smem;                   // [8][ET][64], after the rows
  bf16* gs = (bf16*)(ng_smem + rows_bytes);           // [H]
  float* rinv = (float*)(gs + H);                     // [16]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * 16;
  // this block's share of the 16-byte column chunks for the residual and normed copies
  const int nch = H >> 3;
  const int c_lo = blockIdx.y * nch / gridDim.y, c_hi = (blockIdx.y + 1) * nch / gridDim.y;

  // 0. first batch of gate fragments: k-steps wave, wave + 8, ... of tiles
  // blockIdx.y * ET + 0 .. ET-1
  const int nsteps = H / 32;
  const bf16* wt = wgate_t + ((size_t)blockIdx.y * ET * nsteps * 64 + lane) * 8;
  auto load_batch = [&](bf16x8 (&wf)[U][ET], int j0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = min(j0 + u * 8, nsteps - 1);  // past the end: a valid step, not used
#pragma unroll
      for (int et = 0; et < ET; ++et)
        wf[u][et] = *(const bf16x8*)(wt + ((size_t)et * nsteps + j) * 512);
    }
  };
  bf16x8 wa[U][ET], wb[U][ET];
  load_batch(wa, wave);

  // 1. gamma and rows -> LDS (wave w: rows 2w, 2w+1), residual copy, sums of squares
  for (int i = tid * 8; i < H; i += 512 * 8) *(bf16x8*)(gs + i) = *(const bf16x8*)(gamma + i);
  {
    const int r0 = wave * 2;
    const bool valid0 = t0 + r0 < n, valid1 = t0 + r0 + 1 < n;
    const bf16* x0 = hidden + (size_t)min(t0 + r0, n - 1) * H;
    const bf16* x1 = hidden + (size_t)min(t0 + r0 + 1, n - 1) * H;
    float ss0 = 0.f, ss1 = 0.f;
    for (int i0 = lane * 8; i0 < H; i0 += 512 * NG_NB) {
      bf16x8 v0[NG_NB], v1[NG_NB];
#pragma unroll
      for (int u = 0; u < NG_NB; ++u) {
        const int i = i0 + u * 512;
        v0[u] = i < H ? *(const bf16x8*)(x0 + i) : bf16x8{};
        v1[u] = i < H ? *(const bf16x8*)(x1 + i) : bf16x8{};
      }
#pragma unroll
      for (int u = 0; u < NG_NB; ++u) {
        const int i = i0 + u * 512;
        if (i < H) {
          *(bf16x8*)(xs + r0 * HP + i) = v0[u];
          *(bf16x8*)(xs + (r0 + 1) * HP + i) = v1[u];
          if ((i >> 3) >= c_lo && (i >> 3) < c_hi) {
            if (valid0) *(bf16x8*)(residual + (size_t)(t0 + r0) * H + i) = v0[u];
            if (valid1) *(bf16x8*)(residual + (size_t)(t0 + r0 + 1) * H + i) = v1[u];
          }
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const float f0 = (float)v0[u][q], f1 = (float)v1[u][q];
            ss0 += f0 * f0;
            ss1 += f1 * f1;
          }
        }
      }
    }
    ss0 = wave_sum(ss0);
    ss1 = wave_sum(ss1);
    if (lane == 0) {
      rinv[r0] = 1.0f / sqrtf(ss0 / (float)H + eps);
      rinv[r0 + 1] = 1.0f / sqrtf(ss1 / (float)H + eps);
    }
  }
  __syncthreads();

  // 2. gate: every expert tile of the block from one split of each k-step
  const int tok = lane & 15, kg = lane >> 4;
  const float rv = rinv[tok];
  const bf16* xrow = xs + tok * HP + kg * 8;
  const bf16* grow = gs + kg * 8;
  floatx4 acc[ET];
#pragma unroll
  for (int et = 0; et < ET; ++et) acc[et] = floatx4{0.f, 0.f, 0.f, 0.f};
  auto compute_batch = [&](const bf16x8 (&wf)[U][ET], int j0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * 8;
      if (j >= nsteps) break;
      const bf16x8 xv = *(const bf16x8*)(xrow + j * 32);
      const bf16x8 gv = *(const bf16x8*)(grow + j * 32);
      bf16x8 hi, lo;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float v = (float)xv[q] * (float)gv[q];  // exact: 8-bit x 8-bit mantissas
        hi[q] = (bf16)v;
        lo[q] = (bf16)(v - (float)hi[q]);
      }
#pragma unroll
      for (int et = 0; et < ET; ++et) {
        acc[et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[u][et], hi, acc[et], 0, 0, 0);
        acc[et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[u][et], lo, acc[et], 0, 0, 0);
      }
    }
  };
  constexpr int BS = 8 * U;  // k-steps between consecutive batches of a wave
  for (int j0 = wave; j0 < nsteps; j0 += 2 * BS) {
    if (j0 + BS < nsteps) load_batch(wb, j0 + BS);
    compute_batch(wa, j0);
    if (j0 + BS >= nsteps) break;
    if (j0 + 2 * BS < nsteps) load_batch(wa, j0 + 2 * BS);
    compute_batch(wb, j0 + BS);
  }

  // normed rows: wave w rows 2w, 2w+1, this block's column chunks, from LDS
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int r = wave * 2 + rr;
    if (t0 + r >= n) continue;
    const float rr_inv = rinv[r];
    for (int i = lane * 8; i < H; i += 512) {
      if ((i >> 3) < c_lo || (i >> 3) >= c_hi) continue;
      const bf16x8 xv = *(const bf16x8*)(xs + r * HP + i);
      const bf16x8 gv = *(const bf16x8*)(gs + i);
      bf16x8 o;
#pragma unroll
      for (int q = 0; q < 8; ++q) o[q] = (bf16)((float)xv[q] * rr_inv * (float)gv[q]);
      *(bf16x8*)(normed + (size_t)(t0 + r) * H + i) = o;
    }
  }
  __syncthreads();  // every wave is done with the staged rows
#pragma unroll
  for (int et = 0; et < ET; ++et) red[(wave * ET + et) * 64 + lane] = acc[et];
  __syncthreads();

  // 3. tile et: the 8 waves' partial sums in wave order
  if (wave < ET) {
    floatx4 v = red[wave * 64 + lane];
#pragma unroll
    for (int w = 1; w < 8; ++w) v += red[(w * ET + wave) * 64 + lane];
    v *= rv;  // the row's inverse RMS, in fp32
    const int e = (blockIdx.y * ET + wave) * 16 + 4 * kg;
    if (t0 + tok < n && e < E) {
      float* dst = logits + (size_t)(t0 + tok) * E + e;
      if (e + 3 < E && (E & 3) == 0) {
        *(floatx4*)dst = v;
      } else {
        for (int q = 0; q < 4 && e + q < E; ++q) dst[q] = v[q];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Decode-sized routing front end in one launch (N <= 16 tokens, bf16).
// The gate projection is split over expert tiles of 16 and slices of the
// hidden dimension: block (et, hs) of ET x HS (about 64 blocks, 8 waves each)
// computes the partial dot products W_g[e] . (x_t * gamma) of its 16 experts
// over its slice of k-steps for all tokens (x * gamma exact in fp32, split
// into bf16 hi + lo for the MFMA, as in the batched kernel), summed over its
// waves in wave order, and stores them to `part`. Every block also computes
// the inverse RMS of every token with the same routine (so every block holds
// bit-identical values); the blocks of expert tile 0 write their slice of
// `normed` and `residual`. The last block to finish (release fence, counter,
// acquire fence) adds the partials over the slices in slice order, scales
// them by the inverse RMS into the fp32 logits, runs the top-k of every
// token and a stable sort sized for at most 16 x 16 routes, then re-arms the
// counter. Device-scope fences write back / invalidate the L2 of the issuing
// XCD, so only the wave that stored the partials fences.
// ---------------------------------------------------------------------------
constexpr int RS_THREADS = 512;   // 8 waves per block
constexpr int RS_MAX_BLOCKS = 64; // ET * HS bound (sizes the partial buffer)
constexpr int RS_MAX_R = 16 * MOE_MAX_TOPK_REDUCE;

int route_small_part_floats() { return RS_MAX_BLOCKS * 16 * 16; }  // hs_n * ET <= RS_MAX_BLOCKS

// Stable sort of R <= RS_MAX_R routes (ids in LDS) by expert, one block of
// RS_THREADS >= E threads: LDS histogram, exclusive scans of counts and row
// tiles over the experts, then each route's rank among the lower routes of
// its expert (positions ascend with the route id).
__device__ void sort_small(const int* __restrict__ sids, int R, int E, int* __restrict__ counts,
                           int* __restrict__ offsets, int* __restrict__ perm, int* __restrict__ inv,
                           int bm, int2* __restrict__ tiles, int* __restrict__ num_tiles,
                           int* __restrict__ cnt, int* __restrict__ base, int (*wsum)[8]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < E) cnt[tid] = 0;
  __syncthreads();
  for (int r = tid; r < R; r += RS_THREADS) atomicAdd(&cnt[sids[r]], 1);
  __syncthreads();
  const int c = tid < E ? cnt[tid] : 0;
  const int tc = tid < E ? (c + bm - 1) / bm : 0;
  const int ic = wave_incl_scan(c, lane), itc = wave_incl_scan(tc, lane);
  if (lane == 63) {
    wsum[0][wave] = ic;
    wsum[1][wave] = itc;
  }
  __syncthreads();
  int pc = 0, ptc = 0;
  for (int w = 0; w < wave; ++w) {
    pc += wsum[0][w];
    ptc += wsum[1][w];
  }
  if (tid < E) {
    const int excl = pc + ic - c, texcl = ptc + itc - tc;
    base[tid] = excl;
    counts[tid] = c;
    offsets[tid] = excl;
    if (tid == E - 1) {
      offsets[E] = excl + c;
      *num_tiles = texcl + tc;
    }
    for (int i = 0; i < tc; ++i) tiles[texcl + i] = make_int2(tid, i * bm);
  }
  __syncthreads();
  for (int r = tid; r < R; r += RS_THREADS) {
    const int e = sids[r];
    int rank = 0;
    for (int q = 0; q < r; ++q) rank += sids[q] == e;
    const int pos = base[e] + rank;
    perm[pos] = r;
    inv[r] = pos;
  }
}

template <int EPL>
__global__ void __launch_bounds__(RS_THREADS) route_small_kernel(
    const bf16* __restrict__ hidden, const bf16* __restrict__ gamma, const bf16* __restrict__ wgate,
    bf16* __restrict__ normed, bf16* __restrict__ residual, float* __restrict__ logits, int n,
    int H, int E, float eps, int k, float scale, int* __restrict__ ids, float* __restrict__ wts,
    int* __restrict__ counts, int* __restrict__ offsets, int* __restrict__ perm,
    int* __restrict__ inv, int bm, int2* __restrict__ tiles, int* __restrict__ num_tiles,
    float* __restrict__ part, int hs_n, unsigned* __restrict__ done) {
  __shared__ float rinv[16];
  __shared__ floatx4 red[8][64];
  __shared__ float lg[16 * MOE_MAX_E];
  __shared__ int sids[RS_MAX_R];
  __shared__ int scnt[MOE_MAX_E], sbase[MOE_MAX_E];
  __shared__ int wsum[2][8];
  __shared__ int is_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ET = gridDim.x / hs_n;
  const int et = blockIdx.x % ET, hs = blockIdx.x / ET;
  const int E16 = ET * 16;
  const int nsteps = H / 32;
  const int j0 = hs * nsteps / hs_n, j1 = (hs + 1) * nsteps / hs_n;  // this block's k-steps
  const int e0 = et * 16;
  float* pdot = part;  // [hs][16 tokens][E16]

  // Gate operands: lane holds token tok and k-elements 8*kg..+7 of a 32-wide
  // k-step; wave w takes k-steps j0 + w, j0 + w + 8, ... of the slice, in
  // batches of U whose loads issue together. The first batch is issued
  // before the RMS rows below, so the two load rounds overlap.
  const int tok = lane & 15, kg = lane >> 4;
  const bool tvalid = tok < n;
  const bf16* wrow = wgate + (size_t)min(e0 + tok, E - 1) * H + kg * 8;  // rows past E: never stored
  const size_t row = (size_t)tok * H + kg * 8;
  constexpr int U = 4;  // k-steps per load batch
  bf16x8 wf[U], xv[U], gv[U];
  auto load_batch = [&](int jb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k0 = min(jb + u * 8, j1 - 1) * 32;  // past the slice: a valid step, not used
      wf[u] = *(const bf16x8*)(wrow + k0);
      xv[u] = tvalid ? *(const bf16x8*)(hidden + row + k0) : bf16x8{};
      gv[u] = *(const bf16x8*)(gamma + k0 + kg * 8);
    }
  };
  const int jfirst = j0 + wave;
  if (jfirst < j1) load_batch(jfirst);

  // 1. inverse RMS of tokens wave and wave + 8 (the same code in every block,
  //    so every block holds bit-identical values): both rows' loads in one
  //    round per 2048 elements, each lane summing its chunks in order.
  if (wave < n) {
    const bf16* x0 = hidden + (size_t)wave * H;
    const bf16* x1 = hidden + (size_t)min(wave + 8, n - 1) * H;
    float s0 = 0.f, s1 = 0.f;
    for (int i0 = lane * 8; i0 < H; i0 += 512 * 4) {
      bf16x8 v0[4], v1[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * 512;
        v0[u] = i < H ? *(const bf16x8*)(x0 + i) : bf16x8{};
        v1[u] = i < H ? *(const bf16x8*)(x1 + i) : bf16x8{};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float f0 = (float)v0[u][q], f1 = (float)v1[u][q];
          s0 += f0 * f0;
          s1 += f1 * f1;
        }
    }
    s0 = wave_sum(s0);
    s1 = wave_sum(s1);
    if (lane == 0) {
      rinv[wave] = 1.0f / sqrtf(s0 / (float)H + eps);
      if (wave + 8 < n) rinv[wave + 8] = 1.0f / sqrtf(s1 / (float)H + eps);
    }
  }

  // 2. partial gate dot products W_g . (x * gamma) over the wave's k-steps
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int jb = jfirst; jb < j1; jb += 8 * U) {
    if (jb != jfirst) load_batch(jb);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (jb + u * 8 >= j1) break;
      bf16x8 hi, lo;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float v = (float)xv[u][q] * (float)gv[u][q];  // exact: 8-bit x 8-bit mantissas
        hi[q] = (bf16)v;
        lo[q] = (bf16)(v - (float)hi[q]);
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[u], hi, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[u], lo, acc, 0, 0, 0);
    }
  }
  red[wave][lane] = acc;
  __syncthreads();  // also orders rinv

  // residual and normed for this block's slice (expert tile 0 only)
  if (et == 0) {
    for (int c = j0 * 4 + (tid & 63); c < j1 * 4; c += 64) {  // 8-element chunks of the slice
      for (int t = tid >> 6; t < n; t += 8) {
        const size_t o = (size_t)t * H + c * 8;
        const bf16x8 xv = *(const bf16x8*)(hidden + o);
        const bf16x8 gv = *(const bf16x8*)(gamma + c * 8);
        bf16x8 nb;
#pragma unroll
        for (int q = 0; q < 8; ++q) nb[q] = (bf16)((float)xv[q] * rinv[t] * (float)gv[q]);
        *(bf16x8*)(residual + o) = xv;
        *(bf16x8*)(normed + o) = nb;
      }
    }
  }
  if (wave == 0) {
    floatx4 v = red[0][lane];
#pragma unroll
    for (int w = 1; w < 8; ++w) v += red[w][lane];
    *(floatx4*)(pdot + ((size_t)hs * 16 + tok) * E16 + e0 + 4 * kg) = v;
    // 3. the last block finishes routing (only this wave stored partials)
    __threadfence();
    int last = 0;
    if (lane == 0) last = atomicAdd(done, 1u) == gridDim.x - 1;
    last = __shfl(last, 0);
    if (last) __threadfence();
    if (lane == 0) is_last = last;
  }
  __syncthreads();
  if (!is_last) return;

  // logits = rinv * (sum of the partials in slice order), fp32; a thread
  // takes 4 consecutive experts of one token, its slices' loads in flight
  // together (8 at a time)
  for (int g = tid; g < n * (E16 / 4); g += RS_THREADS) {
    const int t = g / (E16 / 4), e = (g - t * (E16 / 4)) * 4;
    const floatx4* src = (const floatx4*)(pdot + (size_t)t * E16 + e);
    const size_t hstride = (size_t)16 * E16 / 4;
    floatx4 sum = {0.f, 0.f, 0.f, 0.f};
    for (int h0 = 0; h0 < hs_n; h0 += 8) {
      floatx4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = h0 + u < hs_n ? src[(h0 + u) * hstride] : floatx4{};
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (h0 + u < hs_n) sum += v[u];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (e + q < E) {
        const float l = rinv[t] * sum[q];
        lg[t * MOE_MAX_E + e + q] = l;
        logits[(size_t)t * E + e + q] = l;
      }
  }
  __syncthreads();
  // top-k: wave w takes tokens w and w + 8
  for (int t = wave; t < n; t += 8)
    topk_token<EPL>(lg + t * MOE_MAX_E, E, k, scale, sids + t * k, wts + (size_t)t * k, lane);
  __syncthreads();
  const int R = n * k;
  for (int r = tid; r < R; r += RS_THREADS) ids[r] = sids[r];
  sort_small(sids, R, E, counts, offsets, perm, inv, bm, tiles, num_tiles, scnt, sbase, wsum);
  if (tid == 0) *done = 0u;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <int TM>
static void norm_gate_tm(int act_dt, const void* hidden, const void* gamma, const void* wgate,
                         void* normed, void* residual, float* logits, int n, int H, int E,
                         float eps, hipStream_t s) {
  const int bx = (n + TM - 1) / TM;
  int ysplit = 1;
  // Small batches: spread the experts over more workgroups (at least 4 per block).
  while (bx * ysplit < 256 && E / (ysplit * 2) >= 4) ysplit *= 2;
  const int epb = (E + ysplit - 1) / ysplit;
  const size_t lds = (size_t)TM * H * sizeof(float);
  dim3 grid(bx, ysplit);
  if (act_dt == MOE_DT_BF16) {
    hipLaunchKernelGGL((norm_gate_kernel<bf16, TM>), grid, dim3(256), lds, s,
                       (const bf16*)hidden, (const bf16*)gamma, (const bf16*)wgate,
                       (bf16*)normed, (bf16*)residual, logits, n, H, E, epb, eps);
  } else {
    hipLaunchKernelGGL((norm_gate_kernel<float, TM>), grid, dim3(256), lds, s,
                       (const float*)hidden, (const float*)gamma, (const float*)wgate,
                       (float*)normed, (float*)residual, logits, n, H, E, epb, eps);
  }
}

hipError_t launch_norm_gate(int act_dt, const void* hidden, const void* gamma, const void* wgate,
                            const void* wgate_t, void* normed, void* residual, float* logits,
                            int n, int H, int E, float eps, hipStream_t s) {
  // Expert tiles per block: fewer as the token groups shrink, so that the
  // grid keeps >= 256 blocks where the tiles allow.
  const int bx = (n + 15) / 16, tiles = (E + 15) / 16;
  int et = 8;
  while (et > 1 && (tiles % et != 0 || bx * (tiles / et) < 256)) et /= 2;
  const size_t lds = norm_gate_lds_bytes(H, et);
  if (act_dt == MOE_DT_BF16 && wgate_t && lds <= NG_LDS_MAX) {
    static bool attr_set = false;  // the dynamic LDS exceeds the 64 KiB default
    if (!attr_set) {
      hipError_t e = hipSuccess;
      const void* fns[4] = {(const void*)norm_gate_lds_kernel<1>, (const void*)norm_gate_lds_kernel<2>,
                            (const void*)norm_gate_lds_kernel<4>, (const void*)norm_gate_lds_kernel<8>};
      for (const void* f : fns)
        if (e == hipSuccess)
          e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)NG_LDS_MAX);
      if (e != hipSuccess) return e;
      attr_set = true;
    }
    dim3 grid(bx, tiles / et);
    switch (et) {
#define NGL_CASE(X)                                                                          \
  case X:                                                                                    \
    hipLaunchKernelGGL((norm_gate_lds_kernel<X>), grid, dim3(512), lds, s, (const bf16*)hidden, \
                       (const bf16*)gamma, (const bf16*)wgate_t, (bf16*)normed,              \
                       (bf16*)residual, logits, n, H, E, eps);                               \
    break;
      NGL_CASE(1) NGL_CASE(2) NGL_CASE(4) NGL_CASE(8)
#undef NGL_CASE
    }
    return hipGetLastError();
  }
  if (act_dt == MOE_DT_BF16) {
    // 16 tokens per block; split the expert tiles over blockIdx.y until the
    // grid has >= 512 blocks (at least one 16-expert tile per block).
    const int bx = (n + 15) / 16;
    const int tiles = (E + 15) / 16;
    int et = tiles;
    while (et > 1 && bx * ((tiles + et - 1) / et) < 256) et = (et + 1) / 2;
    et = et >= 8 ? 8 : et >= 4 ? 4 : et >= 2 ? 2 : 1;
    dim3 grid(bx, (tiles + et - 1) / et);
    switch (et) {
#define NG_CASE(X)                                                                           \
  case X:                                                                                    \
    hipLaunchKernelGGL((norm_gate_mfma_kernel<X>), grid, dim3(256), 0, s, (const bf16*)hidden, \
                       (const bf16*)gamma, (const bf16*)wgate, (bf16*)normed, (bf16*)residual, \
                       logits, n, H, E, eps);                                                \
    break;
      NG_CASE(1) NG_CASE(2) NG_CASE(4) NG_CASE(8)
#undef NG_CASE
    }
    return hipGetLastError();
  }
  // fp32 layers: SIMT kernel; TM fp32 rows of H stay in LDS (<= 60 KiB).
  if (H * 4 * 4 <= 60 * 1024)
    norm_gate_tm<4>(act_dt, hidden, gamma, wgate, normed, residual, logits, n, H, E, eps, s);
  else if (H * 2 * 4 <= 60 * 1024)
    norm_gate_tm<2>(act_dt, hidden, gamma, wgate, normed, residual, logits, n, H, E, eps, s);
  else
    norm_gate_tm<1>(act_dt, hidden, gamma, wgate, normed, residual, logits, n, H, E, eps, s);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int n, int E, int k, float scale, int* ids, float* w,
                       hipStream_t s) {
  dim3 grid((n + 3) / 4);
  const int epl = (E + 63) / 64;
  switch (epl) {
#define TOPK_CASE(X)                                                                         \
  case X:                                                                                    \
    hipLaunchKernelGGL((topk_sigmoid_kernel<X>), grid, dim3(256), 0, s, logits, n, E, k, scale, \
                       ids, w);                                                              \
    break;
    TOPK_CASE(1) TOPK_CASE(2) TOPK_CASE(3) TOPK_CASE(4) TOPK_CASE(5) TOPK_CASE(6) TOPK_CASE(7)
    TOPK_CASE(8)
#undef TOPK_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_route_sort(const int* ids, int R, int E, int* counts, int* offsets, int* perm,
                             int* inv, int bm, int2* tiles, int* num_tiles, int* bcnt,
                             hipStream_t s) {
  const int nb = (R + SORT_CH - 1) / SORT_CH;
  if (bcnt == nullptr || nb <= 1) {
    hipLaunchKernelGGL(route_sort_kernel, dim3(1), dim3(1024), 0, s, ids, R, E, counts, offsets,
                       perm, inv, bm, tiles, num_tiles);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(route_hist_kernel, dim3(nb), dim3(1024), 0, s, ids, R, E, bcnt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_scatter_kernel, dim3(nb), dim3(1024), 0, s, ids, R, E, bcnt, counts,
                     offsets, perm, inv, bm, tiles, num_tiles);
  return hipGetLastError();
}

int route_sort_blocks(int R) { return (R + SORT_CH - 1) / SORT_CH; }

hipError_t launch_route_small(const void* hidden, const void* gamma, const void* wgate,
                              void* normed, void* residual, float* logits, int n, int H, int E,
                              float eps, int k, float scale, int* ids, float* w, int* counts,
                              int* offsets, int* perm, int* inv, int bm, int2* tiles,
                              int* num_tiles, float* part, unsigned* done, hipStream_t s) {
  if (n < 1 || n > 16 || E > MOE_MAX_E || n * k > RS_MAX_R || bm < 1) return hipErrorInvalidValue;
  const int ET = (E + 15) / 16, nsteps = H / 32;
  const int hs_n = std::max(1, std::min(nsteps, RS_MAX_BLOCKS / ET));
  dim3 grid(ET * hs_n);
  switch ((E + 63) / 64) {
#define RS_CASE(X)                                                                            \
  case X:                                                                                     \
    hipLaunchKernelGGL((route_small_kernel<X>), grid, dim3(RS_THREADS), 0, s, (const bf16*)hidden, \
                       (const bf16*)gamma, (const bf16*)wgate, (bf16*)normed, (bf16*)residual, \
                       logits, n, H, E, eps, k, scale, ids, w, counts, offsets, perm, inv, bm,  \
                       tiles, num_tiles, part, hs_n, done);                                   \
    break;
    RS_CASE(1) RS_CASE(2) RS_CASE(3) RS_CASE(4) RS_CASE(5) RS_CASE(6) RS_CASE(7) RS_CASE(8)
#undef RS_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
