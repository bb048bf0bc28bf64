// Internal kernel launch interface of the MoE layer library (not part of the C ABI).
#pragma once

#include "common.h"
#include "../../include/moe_layer.h"

#define MOE_MAX_E 512
#define MOE_MAX_TOPK_REDUCE 16  // = MOE_MAX_TOP_K

// Epilogues of the GEMM kernels.
enum {
  EPI_RELU2 = 0,    // C = relu(acc)^2
  EPI_STORE = 1,    // C = acc
  EPI_ADD_RES = 2   // C = acc + res + add   (res, add in C's dtype; add may be null)
};

// One GEMM launch: C[p][n] = sum_k A[arow(p)][k] * B[g][n][k], then the epilogue.
//   dense   (tiles == null): rows p in [0, M), group g = 0
//   grouped (tiles != null): tile i covers rows offsets[g] + r0 ...
//            min(offsets[g] + r0 + bm, offsets[g+1]) where (g, r0) = tiles[i];
//            only i < *num_tiles are live
//   arow(p) = a_rows ? a_rows[p] / a_div : p   (gather of permuted activations)
struct GemmArgs {
  const void* A;
  int lda;
  const int* a_rows;
  int a_div;
  const void* B;            // bf16/f32: [G][N][K] (MFMA path: pre-tiled, see gemm.hip)
  long long b_gstride;      // elements (bytes for NVFP4) between groups
  const uint8_t* b_scales;  // NVFP4 block scales (pre-tiled)
  long long bs_gstride;     // bytes between groups
  const float* b_scale2;    // NVFP4 per-group scale2
  void* C;
  int ldc;
  int M, N, K;
  const int2* tiles;
  const int* num_tiles;
  const int* offsets;
  int bm;
  const void* res;
  const void* add;  // EPI_ADD_RES second addend, C's dtype (may be null)
  int b_kmajor;     // bf16 weights in the k-major tile order (see launch_retile_bf16)
  const int* c_rows;  // GEMV arm: output row of row p is c_rows[p] (null: p)
  // Grouped MFMA launches: 16 zeroed counters (per-XCD next item, per-XCD
  // finished workgroups; left at zero by the launch) for dynamic item
  // scheduling, or null for the static schedule. Launches sharing one array
  // must not overlap.
  unsigned* sched;
  // Dense EPI_RELU2 launches: relu^2 only on output columns < relu_n (0: all
  // columns; a multiple of 4 otherwise).
  int relu_n;
};

// RMSNorm + residual + gate logits. wgate_t (bf16 layers, may be null) is the
// gate matrix re-tiled by launch_retile_bf16 with E padded to a multiple of 16
// (zero rows); it selects the LDS-staged kernel when 16 rows of H fit in LDS.
hipError_t launch_norm_gate(int act_dt, const void* hidden, const void* gamma, const void* wgate,
                            const void* wgate_t, void* normed, void* residual, float* logits,
                            int n, int H, int E, float eps, hipStream_t s);
hipError_t launch_topk(const float* logits, int n, int E, int k, float scale, int* ids, float* w,
                       hipStream_t s);
// Stable route sort. With a `bcnt` scratch of route_sort_blocks(R) * E ints
// and R above one block's chunk, two multi-block launches; else one workgroup.
hipError_t launch_route_sort(const int* ids, int R, int E, int* counts, int* offsets, int* perm,
                             int* inv, int bm, int2* tiles, int* num_tiles, int* bcnt,
                             hipStream_t s);
int route_sort_blocks(int R);

// Static device scratch (csrc/scratch.hip) of the allocation-free entry
// points: MOE_STATIC_SCRATCH_INTS ints per device, its device address
// resolved once per device. Used for the per-block expert counts of the
// multi-block route sort (route_sort_blocks(R) * E ints).
#define MOE_STATIC_SCRATCH_INTS (MOE_STATIC_SCRATCH_BYTES / 4)
hipError_t static_scratch(int** out);

// Decode-sized routing in one launch (bf16, n <= 16): norm + residual + gate
// split over expert tiles and hidden slices, then (last block) the logits,
// top-k and the stable sort. `part` is a workspace of route_small_part_floats()
// floats; `done` is a zeroed device counter that the kernel leaves at zero.
hipError_t launch_route_small(const void* hidden, const void* gamma, const void* wgate,
                              void* normed, void* residual, float* logits, int n, int H, int E,
                              float eps, int k, float scale, int* ids, float* w, int* counts,
                              int* offsets, int* perm, int* inv, int bm, int2* tiles,
                              int* num_tiles, float* part, unsigned* done, hipStream_t s);
int route_small_part_floats();

// fp32 SIMT GEMM (64x64 tiles, bm must be 64 in grouped mode); C fp32.
hipError_t launch_gemm_simt_f32(const GemmArgs& a, int epi, int grid_y, hipStream_t s);

// bf16 MFMA GEMM. cfg selects the tile shape; C is bf16 (tc_bf16 must be true).
struct MfmaCfg {
  int wf;   // features per wave (16, 32)
  int bmt;  // rows (tokens / routes) per workgroup tile (16, 32, 64, 128)
  int est_tiles = 0;  // grouped launches: expected live row tiles (0 = unknown)
};
// `slots` = row tiles (grouped: tile-list capacity, live count read on device).
// stream_weights (grouped launches only): non-temporal weight loads, for
// experts that take one row tile each (every weight byte read once).
hipError_t launch_gemm_mfma(const GemmArgs& a, MfmaCfg cfg, int epi, bool tc_bf16, bool nvfp4,
                            int slots, bool stream_weights, hipStream_t s);

// Decode-sized GEMV arm (row tiles of <= 16 rows, bf16 activations and
// output): nseg (1 or 2) segments in one launch, each with `slots` row tiles;
// grouped segments set `tiles`.
// Decode-sized down projection fused with the weighted reduce, residual
// and shared-expert add (direct layers, n <= 16): routed.A = h in decode
// tile-list order (tiles of <= 16 rows), routed.B the down weights; shared.A
// = shared up output [n][S], shared.B its down weights (shared_splits = 0:
// no shared expert). perm maps a tile-list row to its route t*k + j, w the
// route weights. out may alias neither residual nor the inputs.
constexpr int GEMV_REDUCE_WAVES = 8;
struct GemvReduceArgs {
  GemmArgs routed;
  GemmArgs shared;
  int shared_splits;  // k-range splits of the shared expert (0: none)
  const int* perm;
  const float* w;
  int k, n;
  const bf16* residual;
  bf16* out;
  int ldo;
};
hipError_t launch_gemv_down_reduce(const GemvReduceArgs& g, int D, bool nvfp4, hipStream_t s);
hipError_t launch_gemv(const GemmArgs* segs, const int* slots, int nseg, int epi, bool nvfp4,
                       hipStream_t s);

// Re-tile bf16 [G][N][K] row-major weights into the MFMA lane order.
// Re-tile bf16 [G][N][K] into the MFMA lane order of 16-feature x 32-k blocks
// (lane l: row l%16, k 8*(l/16)..+7). Feature-major: [G][N/16][K/32][64][8],
// each 16-feature tile contiguous along K. k-major: [G][K/64][N/16][2][64][8],
// all tiles of one 64-wide k-step contiguous.
hipError_t launch_retile_bf16(const bf16* src, bf16* dst, int G, int N, int K, bool kmajor,
                              hipStream_t s);

// Re-tile NVFP4 [G][N][K/2] packed + [G][N][K/16] scales into the MFMA lane order.
hipError_t launch_retile_nvfp4(const uint8_t* qsrc, const uint8_t* ssrc, uint8_t* qdst,
                               uint8_t* sdst, int G, int N, int K, hipStream_t s);

// Unpermute + weighted reduce (+ shared + residual in direct mode). y, residual,
// sh and out are in the activation dtype `dt`; sums run in fp32.
//   direct: out[t] = residual[t] + sum_j w[t][j] * y[inv[t*k+j]] + sh[t]
//   latent: out[t] = sum_j w[t][j] * y[inv[t*k+j]]      (res, sh unused)
// inv == null: y is in route order (row t*k + j).
hipError_t launch_unpermute_reduce(int dt, bool latent, const void* y, const int* inv,
                                   const float* w, int n, int k, int D, const void* residual,
                                   const void* sh, void* out, hipStream_t s);

hipError_t launch_nvfp4_quantize(const float* w, int G, int rows, int cols, uint8_t* packed,
                                 uint8_t* scales, float* scale2, hipStream_t s);
