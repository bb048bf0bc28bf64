// Host runtime of the MoE FFN layer: the C ABI declared in include/moe_layer.h.
//
// moe_layer_create (page "metrale_model_arch/nemotron_moe.rs",
// `NemotronMoeLayer::new`: the config checks and the weight hand-off) copies
// the weights into layer-owned HBM, re-tiling every bf16 projection into the
// MFMA lane order, and allocates a workspace for max_tokens so that a forward
// never allocates. moe_layer_forward (same page, `prefill`) enqueues:
//
//   norm_gate      RMSNorm + residual save + gate logits
//   shared up/down relu^2 FFN of the shared expert (needs only normed;
//                  side stream, see below)
//   fc1            latent projection (LatentMoE only)
//   topk           sigmoid top-k + weights
//   sort           histogram / prefix sum / stable scatter / tile list
//   grouped up     gathered rows x up_e, relu^2 epilogue -> h (bf16)
//   grouped down   h x down_e -> y (expert-sorted rows)
//   reduce         direct: hidden = residual + sum_j w*y + shared
//                  latent: o = sum_j w*y; fc2 GEMM with the residual and
//                  shared added in its epilogue -> hidden
//
// The shared expert runs on a side stream forked by an event after norm_gate
// and joined before the grouped GEMMs: it overlaps fc1, top-k and the sort,
// which leave CUs free, but not the grouped GEMMs, whose persistent grids fill
// the chip (a concurrent launch there only starves the other). Token counts up
// to 16 take the GEMV arm (forward_small), all on the caller's stream. Nothing
// reads back to the host.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

#define HIP_TRY(expr)                                                                   \
  do {                                                                                  \
    hipError_t _e = (expr);                                                             \
    if (_e != hipSuccess)                                                               \
      return fail(MOE_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(_e));          \
  } while (0)

size_t dt_size(int dt) { return dt == MOE_DT_F32 ? 4 : 2; }

}  // namespace

// Counter of the decode-sized routing kernel.
// Zeroed counters: [0] the decode-sized routing's, [1, 17) and [17, 33) the
// grouped up / down launches' item schedulers (each left at zero).
constexpr size_t kSyncWords = 33;

struct moe_layer {
  moe_layer_config_t cfg{};
  int device = 0;
  bool mfma = false;  // bf16 activations: MFMA kernels; fp32: SIMT kernels
  // Weights (layer-owned).
  void* gamma = nullptr;
  void* gate = nullptr;
  void* gate_t = nullptr;  // bf16: gate re-tiled to MFMA lane order, E padded to 16
  void* fc1 = nullptr;
  void* fc2 = nullptr;
  void* up = nullptr;
  void* down = nullptr;
  void* sh_up = nullptr;
  void* sh_down = nullptr;
  // NVFP4 experts: re-tiled block scales and per-matrix scale2 (the packed
  // nibbles live in up/down/sh_up/sh_down).
  bool nvfp4 = false;
  void *up_s = nullptr, *down_s = nullptr, *sh_up_s = nullptr, *sh_down_s = nullptr;
  float *up_s2 = nullptr, *down_s2 = nullptr, *sh_up_s2 = nullptr, *sh_down_s2 = nullptr;
  // Workspace (max_tokens rows).
  void* normed = nullptr;
  float* logits = nullptr;
  int* ids = nullptr;
  float* w = nullptr;
  int* counts = nullptr;
  int* offsets = nullptr;
  int* perm = nullptr;
  int* inv = nullptr;
  int2* tiles = nullptr;
  int* num_tiles = nullptr;
  int* bcnt = nullptr;    // per-block expert counts of the multi-block sort
  unsigned* sync = nullptr;  // zeroed counters (routing, grouped schedulers; left at zero)
  float* rs_part = nullptr;  // partial gate dot products of the decode-sized routing
  // bf16 latent layers with a shared expert: the shared up projection and fc1
  // share one pre-tiled weight matrix ([S + Lt][H]: sh_up, then fc1) and the
  // batched forward computes both in one launch into gz = [N][S + Lt]
  // (relu^2 on the first S columns only).
  bool merged_up = false;
  void* gz = nullptr;
  hipStream_t side = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  void* g_sh = nullptr;   // shared-expert activation [N][S]
  void* sh = nullptr;     // shared-expert output [N][H]
  void* z = nullptr;      // latent input [N][L]
  void* h = nullptr;      // routed activation [R][I]
  void* y = nullptr;      // routed output [R][D], expert-sorted rows
  void* o = nullptr;      // latent routed sum [N][L]
  std::vector<void*> allocs;
  int last_n = 0;
  // Stage timing: events[(fwd * MOE_NUM_STAGES + stage) * 2 + {0,1}].
  bool timing = false;
  uint32_t timing_mask = 0;
  int timing_cap = 0, timing_count = 0;
  std::vector<hipEvent_t> tev;
  std::vector<uint8_t> trec;  // [fwd * MOE_NUM_STAGES + stage] recorded

  int D() const { return cfg.latent_size > 0 ? cfg.latent_size : cfg.hidden_size; }
};

namespace {

int dalloc(moe_layer* L, void** p, size_t bytes) {
  *p = nullptr;
  if (bytes == 0) return MOE_OK;
  hipError_t e = hipMalloc(p, bytes);
  if (e != hipSuccess) {
    *p = nullptr;
    (void)hipGetLastError();
    return fail(MOE_ERR_OOM, "hipMalloc(%zu bytes) failed: %s", bytes, hipGetErrorString(e));
  }
  L->allocs.push_back(*p);
  return MOE_OK;
}

// Free one allocation made by dalloc (set-up temporaries).
int dfree(moe_layer* L, void* p) {
  for (size_t i = 0; i < L->allocs.size(); ++i)
    if (L->allocs[i] == p) {
      L->allocs.erase(L->allocs.begin() + i);
      HIP_TRY(hipFree(p));
      return MOE_OK;
    }
  return MOE_OK;
}

void free_layer(moe_layer* L) {
  if (!L) return;
  if (L->ev_fork) (void)hipEventDestroy(L->ev_fork);
  if (L->ev_join) (void)hipEventDestroy(L->ev_join);
  if (L->side) (void)hipStreamDestroy(L->side);
  for (void* p : L->allocs) (void)hipFree(p);
  for (hipEvent_t e : L->tev) (void)hipEventDestroy(e);
  delete L;
}

// Event pair around one stage of the current forward (no-op unless timing).
struct StageScope {
  moe_layer* L;
  int stage;
  hipStream_t s;
  bool on;
  StageScope(moe_layer* L_, int stage_, hipStream_t s_) : L(L_), stage(stage_), s(s_) {
    on = L->timing && (L->timing_mask >> stage & 1u) && L->timing_count < L->timing_cap;
    if (on) (void)hipEventRecord(L->tev[((size_t)L->timing_count * MOE_NUM_STAGES + stage) * 2], s);
  }
  ~StageScope() {
    if (!on) return;
    const size_t i = (size_t)L->timing_count * MOE_NUM_STAGES + stage;
    (void)hipEventRecord(L->tev[i * 2 + 1], s);
    L->trec[i] = 1;
  }
};

int check_config(const moe_layer_config_t& c) {
  if (c.num_experts < 1 || c.num_experts > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_INVALID_CONFIG, "num_experts=%d must be in 1..%d", c.num_experts,
                MOE_MAX_EXPERTS);
  if (c.top_k < 1 || c.top_k > c.num_experts || c.top_k > MOE_MAX_TOP_K)
    return fail(MOE_ERR_INVALID_CONFIG,
                "top_k=%d must be in 1..=%d and at most %d (routing bound)", c.top_k,
                c.num_experts, MOE_MAX_TOP_K);
  if (c.max_tokens < 1) return fail(MOE_ERR_INVALID_CONFIG, "max_tokens=%d < 1", c.max_tokens);
  // Routes r = t * top_k + j are 32-bit indices on the device (with headroom
  // for the tile list and the sort's chunk arithmetic).
  if ((long long)c.max_tokens * c.top_k > (1LL << 30))
    return fail(MOE_ERR_INVALID_CONFIG, "max_tokens * top_k = %lld exceeds 2^30 routes",
                (long long)c.max_tokens * c.top_k);
  const bool f32 = c.act_dtype == MOE_DT_F32;
  if (f32 && c.expert_dtype != MOE_DT_F32)
    return fail(MOE_ERR_INVALID_CONFIG, "fp32 activations need fp32 experts");
  if (c.act_dtype == MOE_DT_BF16 && c.expert_dtype != MOE_DT_BF16 &&
      c.expert_dtype != MOE_DT_NVFP4)
    return fail(MOE_ERR_INVALID_CONFIG, "bf16 activations need bf16 or NVFP4 experts");
  if (c.act_dtype != MOE_DT_F32 && c.act_dtype != MOE_DT_BF16)
    return fail(MOE_ERR_INVALID_CONFIG, "act_dtype=%d unsupported", c.act_dtype);
  const int q = f32 ? 16 : 64;
  const int dims[4] = {c.hidden_size, c.moe_inter, c.shared_inter, c.latent_size};
  const char* names[4] = {"hidden_size", "moe_inter", "shared_inter", "latent_size"};
  for (int i = 0; i < 4; ++i) {
    const bool optional = i >= 2;
    if (dims[i] < 0 || (!optional && dims[i] == 0) || dims[i] % q != 0)
      return fail(MOE_ERR_INVALID_CONFIG, "%s=%d must be a %smultiple of %d", names[i], dims[i],
                  optional ? "non-negative " : "positive ", q);
  }
  if (c.hidden_size > 8192)
    return fail(MOE_ERR_INVALID_CONFIG, "hidden_size=%d exceeds 8192", c.hidden_size);
  if (!(c.rms_eps >= 0.f)) return fail(MOE_ERR_INVALID_CONFIG, "rms_eps must be >= 0");
  return MOE_OK;
}

// Copy a weight matrix stack [G][N][K] into layer memory: bf16 is re-tiled for
// the MFMA kernels, fp32 is copied as is.
int upload_proj(moe_layer* L, void** dst, const void* src, int G, int N, int K, bool retile,
                hipStream_t s, const char* name, bool kmajor = false) {
  if (!src) return fail(MOE_ERR_INVALID_ARG, "weight '%s' is NULL", name);
  const size_t elems = (size_t)G * N * K;
  const size_t bytes = elems * (L->mfma ? 2 : 4);
  int rc = dalloc(L, dst, bytes);
  if (rc) return rc;
  if (retile) {
    HIP_TRY(launch_retile_bf16((const bf16*)src, (bf16*)*dst, G, N, K, kmajor, s));
  } else {
    HIP_TRY(hipMemcpyAsync(*dst, src, bytes, hipMemcpyDeviceToDevice, s));
  }
  return MOE_OK;
}

// Copy an NVFP4 stack [G][N][K] (packed, scales, scale2) into layer memory,
// re-tiled for the MFMA kernel.
int upload_nvfp4(moe_layer* L, void** q, void** sc, float** s2, const moe_nvfp4_t& src, int G,
                 int N, int K, hipStream_t s, const char* name) {
  if (!src.packed || !src.scales || !src.scale2)
    return fail(MOE_ERR_INVALID_ARG, "NVFP4 weight '%s' has a NULL pointer", name);
  int rc = dalloc(L, q, (size_t)G * N * K / 2);
  if (!rc) rc = dalloc(L, sc, (size_t)G * N * K / 16);
  if (!rc) rc = dalloc(L, (void**)s2, (size_t)G * 4);
  if (rc) return rc;
  HIP_TRY(launch_retile_nvfp4((const uint8_t*)src.packed, (const uint8_t*)src.scales,
                              (uint8_t*)*q, (uint8_t*)*sc, G, N, K, s));
  HIP_TRY(hipMemcpyAsync(*s2, src.scale2, (size_t)G * 4, hipMemcpyDeviceToDevice, s));
  return MOE_OK;
}

// Grouped launches: the row-tile height follows the mean rows per expert, so
// that most experts take one tile and few rows are padding. From 41 rows per
// expert on, 128-row tiles where there are 64 experts or more: at 48 (1024
// tokens, 128 experts, top-6) a fifth of the experts exceed 64 rows, and a
// second 64-row tile streams that expert's weights again and unbalances the
// XCDs' tile ranges; one 128-row tile per expert measured 7% faster on the up
// GEMM (the padding rows cost only MFMA time, which the weight stream leaves
// idle). With fewer experts (one GPU's expert shard: 16) the 128-row grid is
// too small to fill the chip and 64-row tiles stay 3% faster.
MfmaCfg grouped_cfg(int rows_per_group, int experts) {
  // From 97 to 168 rows per expert, one 192-row tile per expert reads (and,
  // for NVFP4, decodes) each weight slice once, where 128-row tiles gave many
  // experts a second, partial tile that fetched it again. Measured (bf16):
  // 2560 / 3072 / 3584 tokens over 128 experts, top-6, 0.819 / 0.925 / 0.978
  // -> 0.733 / 0.798 / 0.919 ms per layer; the latent layer at 2048 tokens,
  // top-8 (128 rows per expert), 0.625 -> 0.581 ms; NVFP4 at 3072 tokens
  // grouped up 339 -> 247 us. At 96 rows per expert and below, and at 192
  // (half the experts then take a second 192-row tile, and the 192-row tile
  // fits a 2-stage ring where the 128-row one has 3), 128-row tiles are
  // faster: 2048 tokens 0.629 vs 0.665 ms, 4096 tokens 0.988 vs 1.085 ms.
  if (rows_per_group > 96 && rows_per_group <= 168) return {32, 192};
  if (rows_per_group <= 16) return {16, 16};
  if (rows_per_group <= 32) return {32, 32};
  if (rows_per_group <= 40 || (rows_per_group <= 80 && experts < 64)) return {32, 64};
  return {32, 128};
}

// Dense launches (shared expert, fc1, fc2): 128-row tiles above 64 tokens
// (64-row tiles measured slower on every dense shape here but fc1).
MfmaCfg dense_cfg(int n) {
  if (n <= 16) return {16, 16};
  if (n <= 32) return {32, 32};
  if (n <= 64) return {32, 64};
  return {32, 128};
}

// One GEMM launch. `nvfp4` marks the expert projections of an NVFP4 layer;
// the caller fills the NVFP4 fields of `a`.
int gemm(moe_layer* L, const GemmArgs& a, int epi, bool out_bf16, MfmaCfg cfg, int slots,
         hipStream_t s, const char* what, bool nvfp4 = false, bool stream_weights = false) {
  hipError_t e = L->mfma ? launch_gemm_mfma(a, cfg, epi, out_bf16, nvfp4, slots, stream_weights, s)
                         : launch_gemm_simt_f32(a, epi, slots, s);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

// Set the weight operand of an expert projection (bf16/fp32 or NVFP4).
void set_weights(const moe_layer* L, GemmArgs& a, const void* w, const void* sc, const float* s2,
                 int N, int K) {
  a.B = w;
  if (L->nvfp4) {
    a.b_gstride = (long long)N * K / 2;
    a.b_scales = (const uint8_t*)sc;
    a.bs_gstride = (long long)N * K / 16;
    a.b_scale2 = s2;
  } else {
    a.b_gstride = (long long)N * K;
    // The down projections are stored k-major (all 16-feature tiles of a k-step
    // contiguous): measured 2% faster on the down GEMMs, but 6% slower on the
    // latent up GEMM and 1% on the decode up GEMV, which keep feature-major.
    a.b_kmajor = L->mfma && (w == L->down || w == L->sh_down);
  }
}

// Decode-sized arm (bf16/NVFP4 layers, N <= MOE_GEMV_MAX_N): one stream; the
// shared expert rides as a second segment of the grouped GEMV launches.
constexpr int MOE_GEMV_MAX_N = 16;

int forward_small(moe_layer* L, void* hidden, void* residual, int n, hipStream_t s) {
  const moe_layer_config_t& c = L->cfg;
  const int H = c.hidden_size, E = c.num_experts, k = c.top_k, I = c.moe_inter,
            S = c.shared_inter, Lt = c.latent_size, D = L->D();
  const int R = n * k;
  const int dslots = (n + 15) / 16;
  const int bm = 16;
  {
    // norm + gate + top-k + sort in one launch (timed as the norm_gate stage)
    StageScope sc(L, MOE_STAGE_NORM_GATE, s);
    HIP_TRY(launch_route_small(hidden, L->gamma, L->gate, L->normed, residual, L->logits, n, H,
                               E, c.rms_eps, k, c.routed_scaling_factor, L->ids, L->w,
                               L->counts, L->offsets, L->perm, L->inv, bm, L->tiles,
                               L->num_tiles, L->rs_part, L->sync, s));
  }
  const void* zin = L->normed;
  if (Lt > 0) {
    StageScope sc(L, MOE_STAGE_FC1, s);
    GemmArgs a{};
    a.A = L->normed; a.lda = H; a.B = L->fc1; a.C = L->z; a.ldc = Lt;
    a.M = n; a.N = Lt; a.K = H;
    HIP_TRY(launch_gemv(&a, &dslots, 1, EPI_STORE, false, s));
    zin = L->z;
  }
  const int tiles_cap = (R + bm - 1) / bm + std::min(E, R);
  const int slots[2] = {tiles_cap, dslots};
  const int nseg = S > 0 ? 2 : 1;
  {
    StageScope sc(L, MOE_STAGE_GROUPED_UP, s);
    GemmArgs g[2] = {};
    g[0].A = zin; g[0].lda = D; g[0].a_rows = L->perm; g[0].a_div = k;
    set_weights(L, g[0], L->up, L->up_s, L->up_s2, I, D);
    g[0].C = L->h; g[0].ldc = I; g[0].N = I; g[0].K = D;
    g[0].tiles = L->tiles; g[0].num_tiles = L->num_tiles; g[0].offsets = L->offsets; g[0].bm = bm;
    if (S > 0) {
      g[1].A = L->normed; g[1].lda = H; g[1].C = L->g_sh; g[1].ldc = S;
      g[1].M = n; g[1].N = S; g[1].K = H;
      set_weights(L, g[1], L->sh_up, L->sh_up_s, L->sh_up_s2, S, H);
    }
    HIP_TRY(launch_gemv(g, slots, nseg, EPI_RELU2, L->nvfp4, s));
  }
  if (Lt == 0 && n == 1) {
    // One token: down projection, weighted reduce, shared expert and
    // residual in one launch (the routed outputs stay in LDS). Its grid is
    // one workgroup per 16 output features (168 at hidden 2688), so it only
    // pays while the work per output tile is small: decode Zipf workload
    // 46.7 -> 45.3 us at 1 token, 2-8% slower than GEMV + reduce from 2.
    StageScope sc(L, MOE_STAGE_GROUPED_DOWN, s);
    GemvReduceArgs gr{};
    gr.routed.A = L->h; gr.routed.lda = I;
    set_weights(L, gr.routed, L->down, L->down_s, L->down_s2, D, I);
    gr.routed.N = D; gr.routed.K = I;
    gr.routed.tiles = L->tiles; gr.routed.num_tiles = L->num_tiles;
    gr.routed.offsets = L->offsets; gr.routed.bm = bm;
    if (S > 0) {
      gr.shared.A = L->g_sh; gr.shared.lda = S;
      set_weights(L, gr.shared, L->sh_down, L->sh_down_s, L->sh_down_s2, H, S);
      gr.shared.M = n; gr.shared.N = H; gr.shared.K = S;
      // k-range splits about as long as one routed item (I deep)
      gr.shared_splits = std::max(1, (S + I - 1) / I);
    }
    gr.perm = L->perm; gr.w = L->w; gr.k = k; gr.n = n;
    gr.residual = (const bf16*)residual; gr.out = (bf16*)hidden; gr.ldo = H;
    HIP_TRY(launch_gemv_down_reduce(gr, D, L->nvfp4, s));
  } else {
    {
      StageScope sc(L, MOE_STAGE_GROUPED_DOWN, s);
      GemmArgs g[2] = {};
      g[0].A = L->h; g[0].lda = I;
      set_weights(L, g[0], L->down, L->down_s, L->down_s2, D, I);
      g[0].C = L->y; g[0].ldc = D; g[0].N = D; g[0].K = I;
      g[0].tiles = L->tiles; g[0].num_tiles = L->num_tiles; g[0].offsets = L->offsets; g[0].bm = bm;
      g[0].c_rows = L->perm;  // y in route order: the reduce needs no index load
      if (S > 0) {
        g[1].A = L->g_sh; g[1].lda = S; g[1].C = L->sh; g[1].ldc = H;
        g[1].M = n; g[1].N = H; g[1].K = S;
        set_weights(L, g[1], L->sh_down, L->sh_down_s, L->sh_down_s2, H, S);
      }
      HIP_TRY(launch_gemv(g, slots, nseg, EPI_STORE, L->nvfp4, s));
    }
    if (Lt == 0) {
      StageScope sc(L, MOE_STAGE_REDUCE, s);
      HIP_TRY(launch_unpermute_reduce(c.act_dtype, false, L->y, nullptr, L->w, n, k, D, residual,
                                      S > 0 ? L->sh : nullptr, hidden, s));
    } else {
      {
        StageScope sc(L, MOE_STAGE_REDUCE, s);
        HIP_TRY(launch_unpermute_reduce(c.act_dtype, true, L->y, nullptr, L->w, n, k, D, nullptr,
                                        nullptr, L->o, s));
      }
      StageScope sc(L, MOE_STAGE_FC2, s);
      GemmArgs a{};
      a.A = L->o; a.lda = Lt; a.B = L->fc2; a.C = hidden; a.ldc = H;
      a.M = n; a.N = H; a.K = Lt;
      a.res = residual; a.add = S > 0 ? L->sh : nullptr;
      HIP_TRY(launch_gemv(&a, &dslots, 1, EPI_ADD_RES, false, s));
    }
  }
  L->last_n = n;
  if (L->timing && L->timing_count < L->timing_cap) L->timing_count++;
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_last_error.c_str(); }

int moe_layer_create(const moe_layer_config_t* cfg, const moe_layer_weights_t* wts, void* stream,
                     moe_layer_t** out) {
  if (out) *out = nullptr;
  if (!cfg || !wts || !out) return fail(MOE_ERR_INVALID_ARG, "NULL argument to moe_layer_create");
  int rc = check_config(*cfg);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  moe_layer* L = new moe_layer();
  L->cfg = *cfg;
  L->mfma = cfg->act_dtype == MOE_DT_BF16;
  const moe_layer_config_t& c = L->cfg;
  const int H = c.hidden_size, E = c.num_experts, k = c.top_k, I = c.moe_inter,
            S = c.shared_inter, Lt = c.latent_size, D = L->D(), N = c.max_tokens;
  const size_t R = (size_t)N * k;
  const size_t as = dt_size(c.act_dtype);

#define TRY(x)            \
  do {                    \
    int _r = (x);         \
    if (_r) {             \
      free_layer(L);      \
      return _r;          \
    }                     \
  } while (0)
#define TRYH(x)                                                                        \
  do {                                                                                 \
    hipError_t _e = (x);                                                               \
    if (_e != hipSuccess) {                                                            \
      free_layer(L);                                                                   \
      return fail(MOE_ERR_HIP, "%s failed: %s", #x, hipGetErrorString(_e));            \
    }                                                                                  \
  } while (0)

  L->nvfp4 = c.expert_dtype == MOE_DT_NVFP4;
  if (!wts->norm_gamma || !wts->gate ||
      (!L->nvfp4 && (!wts->up || !wts->down || (S > 0 && (!wts->shared_up || !wts->shared_down)))) ||
      (L->nvfp4 && (!wts->up_q.packed || !wts->down_q.packed ||
                    (S > 0 && (!wts->shared_up_q.packed || !wts->shared_down_q.packed))))) {
    free_layer(L);
    return fail(MOE_ERR_INVALID_ARG, "a required weight (gamma, gate, up, down, shared) is NULL");
  }
  if (Lt > 0 && (!wts->fc1 || !wts->fc2)) {
    free_layer(L);
    return fail(MOE_ERR_INVALID_ARG, "latent layers need fc1 and fc2");
  }
  TRYH(hipGetDevice(&L->device));
  // Weights.
  TRY(dalloc(L, &L->gamma, H * as));
  TRYH(hipMemcpyAsync(L->gamma, wts->norm_gamma, H * as, hipMemcpyDeviceToDevice, s));
  TRY(dalloc(L, &L->gate, (size_t)E * H * as));
  TRYH(hipMemcpyAsync(L->gate, wts->gate, (size_t)E * H * as, hipMemcpyDeviceToDevice, s));
  if (L->mfma) {
    const size_t e16 = (size_t)(E + 15) / 16 * 16;
    void* padded = nullptr;
    TRY(dalloc(L, &padded, e16 * H * 2));
    TRYH(hipMemsetAsync(padded, 0, e16 * H * 2, s));
    TRYH(hipMemcpyAsync(padded, wts->gate, (size_t)E * H * 2, hipMemcpyDeviceToDevice, s));
    TRY(dalloc(L, &L->gate_t, e16 * H * 2));
    TRYH(launch_retile_bf16((const bf16*)padded, (bf16*)L->gate_t, 1, (int)e16, H, false, s));
    TRYH(hipStreamSynchronize(s));
    TRY(dfree(L, padded));
  }
  L->merged_up = L->mfma && !L->nvfp4 && S > 0 && Lt > 0;
  if (L->merged_up) {
    if (!wts->fc1) return fail(MOE_ERR_INVALID_ARG, "weight 'fc1' is NULL");
    if (!wts->shared_up) return fail(MOE_ERR_INVALID_ARG, "weight 'shared_up' is NULL");
    TRY(dalloc(L, &L->sh_up, (size_t)(S + Lt) * H * 2));
    TRYH(launch_retile_bf16((const bf16*)wts->shared_up, (bf16*)L->sh_up, 1, S, H, false, s));
    L->fc1 = (bf16*)L->sh_up + (size_t)S * H;  // its tiles follow the shared up's
    TRYH(launch_retile_bf16((const bf16*)wts->fc1, (bf16*)L->fc1, 1, Lt, H, false, s));
    TRY(upload_proj(L, &L->fc2, wts->fc2, 1, H, Lt, L->mfma, s, "fc2"));
  } else if (Lt > 0) {
    TRY(upload_proj(L, &L->fc1, wts->fc1, 1, Lt, H, L->mfma, s, "fc1"));
    TRY(upload_proj(L, &L->fc2, wts->fc2, 1, H, Lt, L->mfma, s, "fc2"));
  }
  if (L->nvfp4) {
    TRY(upload_nvfp4(L, &L->up, &L->up_s, &L->up_s2, wts->up_q, E, I, D, s, "up"));
    TRY(upload_nvfp4(L, &L->down, &L->down_s, &L->down_s2, wts->down_q, E, D, I, s, "down"));
    if (S > 0) {
      TRY(upload_nvfp4(L, &L->sh_up, &L->sh_up_s, &L->sh_up_s2, wts->shared_up_q, 1, S, H, s,
                       "shared_up"));
      TRY(upload_nvfp4(L, &L->sh_down, &L->sh_down_s, &L->sh_down_s2, wts->shared_down_q, 1, H,
                       S, s, "shared_down"));
    }
  } else {
    TRY(upload_proj(L, &L->up, wts->up, E, I, D, L->mfma, s, "up"));
    TRY(upload_proj(L, &L->down, wts->down, E, D, I, L->mfma, s, "down", true));
    if (S > 0) {
      if (!L->merged_up)
        TRY(upload_proj(L, &L->sh_up, wts->shared_up, 1, S, H, L->mfma, s, "shared_up"));
      TRY(upload_proj(L, &L->sh_down, wts->shared_down, 1, H, S, L->mfma, s, "shared_down", true));
    }
  }
  // Workspace.
  const size_t tiles_cap = R + (size_t)E + 1;  // >= sum_e ceil(c_e / bm) for any bm >= 1
  TRY(dalloc(L, &L->normed, (size_t)N * H * as));
  TRY(dalloc(L, (void**)&L->logits, (size_t)N * E * 4));
  TRY(dalloc(L, (void**)&L->ids, R * 4));
  TRY(dalloc(L, (void**)&L->w, R * 4));
  TRY(dalloc(L, (void**)&L->counts, (size_t)E * 4));
  TRY(dalloc(L, (void**)&L->offsets, (size_t)(E + 1) * 4));
  TRY(dalloc(L, (void**)&L->perm, R * 4));
  TRY(dalloc(L, (void**)&L->inv, R * 4));
  TRY(dalloc(L, (void**)&L->tiles, tiles_cap * sizeof(int2)));
  TRY(dalloc(L, (void**)&L->num_tiles, 16));
  TRY(dalloc(L, (void**)&L->bcnt, (size_t)route_sort_blocks((int)R) * E * 4));
  TRY(dalloc(L, (void**)&L->sync, kSyncWords * 4));
  if (L->mfma) TRY(dalloc(L, (void**)&L->rs_part, (size_t)route_small_part_floats() * 4));
  if (L->mfma) {  // the shared expert's stream (default priority) and its events
    TRYH(hipStreamCreateWithFlags(&L->side, hipStreamNonBlocking));
    TRYH(hipEventCreateWithFlags(&L->ev_fork, hipEventDisableTiming));
    TRYH(hipEventCreateWithFlags(&L->ev_join, hipEventDisableTiming));
  }
  TRYH(hipMemsetAsync(L->sync, 0, kSyncWords * 4, s));
  if (S > 0) {
    TRY(dalloc(L, &L->g_sh, (size_t)N * S * as));
    TRY(dalloc(L, &L->sh, (size_t)N * H * as));
  }
  if (Lt > 0) {
    TRY(dalloc(L, &L->z, (size_t)N * Lt * as));
    TRY(dalloc(L, &L->o, (size_t)N * Lt * as));
  }
  if (L->merged_up) TRY(dalloc(L, &L->gz, (size_t)std::min(N, 1024) * (S + Lt) * as));
  TRY(dalloc(L, &L->h, R * I * as));
  TRY(dalloc(L, &L->y, R * D * as));

  // The norm+gate kernel keeps TM=4 fp32 rows of hidden in LDS.
  TRYH(hipStreamSynchronize(s));
#undef TRY
#undef TRYH
  *out = L;
  return MOE_OK;
}

void moe_layer_destroy(moe_layer_t* L) {
  if (!L) return;
  (void)hipDeviceSynchronize();
  free_layer(L);
}

int moe_layer_forward(moe_layer_t* L, void* hidden, void* residual, int32_t n, void* stream) {
  if (!L || !hidden || !residual) return fail(MOE_ERR_INVALID_ARG, "NULL argument to forward");
  if (n < 0) return fail(MOE_ERR_INVALID_ARG, "num_tokens=%d < 0", n);
  const moe_layer_config_t& c = L->cfg;
  if (n > c.max_tokens)
    return fail(MOE_ERR_TOO_MANY_TOKENS, "num_tokens=%d > max_tokens=%d", n, c.max_tokens);
  if (n == 0) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  if (L->mfma && n <= MOE_GEMV_MAX_N) return forward_small(L, hidden, residual, n, s);
  const int H = c.hidden_size, E = c.num_experts, k = c.top_k, I = c.moe_inter,
            S = c.shared_inter, Lt = c.latent_size, D = L->D();
  const int R = n * k;
  const bool bf = L->mfma;
  const MfmaCfg dc = dense_cfg(n);
  const int dbmt = bf ? dc.bmt : 64;
  const int dgrid = (n + dbmt - 1) / dbmt;

  // 1. RMSNorm + residual + gate logits.
  {
    StageScope sc(L, MOE_STAGE_NORM_GATE, s);
    HIP_TRY(launch_norm_gate(c.act_dtype, hidden, L->gamma, L->gate, L->gate_t, L->normed,
                             residual, L->logits, n, H, E, c.rms_eps, s));
  }

  // 2. Shared expert (needs only the normed rows).
  // MFMA layers: on the side stream, beside fc1, top-k and the sort (small or
  // latency-bound launches that leave CUs free), joined before the grouped
  // GEMMs, whose persistent grids would otherwise starve it.
  const bool side = S > 0 && bf;
  hipStream_t ss = side ? L->side : s;
  if (side) {
    HIP_TRY(hipEventRecord(L->ev_fork, s));
    HIP_TRY(hipStreamWaitEvent(L->side, L->ev_fork, 0));
  }
  // Merged up (bf16 latent layers, up to 1024 tokens): the shared up
  // projection and fc1 as one launch over [S + Lt] output columns, whose
  // items still fit one round there (latent layer at 1024 tokens 0.453 ->
  // 0.428 ms: fc1 no longer runs beside the shared expert); at 2048 tokens
  // both forms take two rounds (0.580 vs 0.581 ms) and at 4096 the separate
  // launches were 1% faster.
  const int gzw = S + Lt;
  const bool merge = L->merged_up && n <= 1024;
  if (S > 0) {
    {
      StageScope sc(L, MOE_STAGE_SHARED_UP, ss);
      GemmArgs a{};
      a.A = L->normed; a.lda = H; a.C = L->g_sh; a.ldc = S;
      a.M = n; a.N = S; a.K = H;
      set_weights(L, a, L->sh_up, L->sh_up_s, L->sh_up_s2, S, H);
      if (merge) {
        a.C = L->gz; a.ldc = gzw; a.N = gzw; a.relu_n = S;
      }
      int rc = gemm(L, a, EPI_RELU2, bf, dc, dgrid, ss, merge ? "shared up + fc1" : "shared up",
                    L->nvfp4);
      if (rc) return rc;
    }
    {
      StageScope sc(L, MOE_STAGE_SHARED_DOWN, ss);
      GemmArgs b{};
      b.A = merge ? L->gz : L->g_sh; b.lda = merge ? gzw : S;
      b.C = L->sh; b.ldc = H;
      b.M = n; b.N = H; b.K = S;
      set_weights(L, b, L->sh_down, L->sh_down_s, L->sh_down_s2, H, S);
      int rc = gemm(L, b, EPI_STORE, bf, dc, dgrid, ss, "shared down", L->nvfp4);
      if (rc) return rc;
    }
  }
  if (side) HIP_TRY(hipEventRecord(L->ev_join, L->side));

  // 3. Latent input.
  const void* zin = L->normed;
  int zld = D;
  if (merge) {
    zin = (const bf16*)L->gz + S;  // written by the merged up launch (side stream)
    zld = gzw;
  } else if (Lt > 0) {
    StageScope sc(L, MOE_STAGE_FC1, s);
    GemmArgs a{};
    a.A = L->normed; a.lda = H; a.B = L->fc1; a.C = L->z; a.ldc = Lt;
    a.M = n; a.N = Lt; a.K = H;
    int rc = gemm(L, a, EPI_STORE, bf, dc, dgrid, s, "fc1");
    if (rc) return rc;
    zin = L->z;
  }

  // 4. Routing.
  {
    StageScope sc(L, MOE_STAGE_TOPK, s);
    HIP_TRY(launch_topk(L->logits, n, E, k, c.routed_scaling_factor, L->ids, L->w, s));
  }
  MfmaCfg gc = grouped_cfg((R + E - 1) / E, E);
  const int bm = bf ? gc.bmt : 64;
  {
    StageScope sc(L, MOE_STAGE_SORT, s);
    HIP_TRY(launch_route_sort(L->ids, R, E, L->counts, L->offsets, L->perm, L->inv, bm,
                              L->tiles, L->num_tiles, L->bcnt, s));
  }
  const int tiles_cap = (R + bm - 1) / bm + std::min(E, R);
  // Experts expected to fit one row tile: each weight byte is read once.
  const bool one_tile = (long long)((R + E - 1) / E) * 4 <= (long long)bm * 3;
  if (one_tile) gc.est_tiles = std::min(E, R);

  if (side) HIP_TRY(hipStreamWaitEvent(s, L->ev_join, 0));

  // 5. Grouped expert GEMMs.
  {
    StageScope sc(L, MOE_STAGE_GROUPED_UP, s);
    GemmArgs a{};
    a.A = zin; a.lda = zld; a.a_rows = L->perm; a.a_div = k;
    set_weights(L, a, L->up, L->up_s, L->up_s2, I, D);
    a.C = L->h; a.ldc = I; a.N = I; a.K = D;
    a.tiles = L->tiles; a.num_tiles = L->num_tiles; a.offsets = L->offsets; a.bm = bm;
    // Dynamic item order where experts take several row tiles (items of
    // unequal length): 4096 tokens 0.981 -> 0.972 ms (bf16), 0.905 -> 0.890
    // ms (NVFP4). With one tile per expert the static order was faster
    // (1024 tokens 0.531 vs 0.544 ms, 2048 tokens 0.623 vs 0.637 ms).
    a.sched = one_tile ? nullptr : L->sync + 1;
    int rc = gemm(L, a, EPI_RELU2, bf, gc, tiles_cap, s, "grouped up", L->nvfp4, one_tile);
    if (rc) return rc;
  }
  {
    StageScope sc(L, MOE_STAGE_GROUPED_DOWN, s);
    GemmArgs b{};
    b.A = L->h; b.lda = I;
    set_weights(L, b, L->down, L->down_s, L->down_s2, D, I);
    b.C = L->y; b.ldc = D; b.N = D; b.K = I;
    b.tiles = L->tiles; b.num_tiles = L->num_tiles; b.offsets = L->offsets; b.bm = bm;
    b.sched = one_tile ? nullptr : L->sync + 17;
    int rc = gemm(L, b, EPI_STORE, bf, gc, tiles_cap, s, "grouped down", L->nvfp4, one_tile);
    if (rc) return rc;
  }

  // 6. Reduce, residual.
  if (Lt == 0) {
    StageScope sc(L, MOE_STAGE_REDUCE, s);
    HIP_TRY(launch_unpermute_reduce(c.act_dtype, false, L->y, L->inv, L->w, n, k, D, residual,
                                    S > 0 ? L->sh : nullptr, hidden, s));
  } else {
    {
      StageScope sc(L, MOE_STAGE_REDUCE, s);
      HIP_TRY(launch_unpermute_reduce(c.act_dtype, true, L->y, L->inv, L->w, n, k, D, nullptr,
                                      nullptr, L->o, s));
    }
    StageScope sc(L, MOE_STAGE_FC2, s);
    GemmArgs a{};
    a.A = L->o; a.lda = Lt; a.B = L->fc2; a.C = hidden; a.ldc = H;
    a.M = n; a.N = H; a.K = Lt;
    a.res = residual; a.add = S > 0 ? L->sh : nullptr;
    int rc = gemm(L, a, EPI_ADD_RES, bf, dc, dgrid, s, "fc2");
    if (rc) return rc;
  }
  L->last_n = n;
  if (L->timing && L->timing_count < L->timing_cap) L->timing_count++;
  return MOE_OK;
}

int moe_layer_timing_begin(moe_layer_t* L, uint32_t mask, int32_t max_forwards) {
  if (!L || max_forwards < 1 || max_forwards > 4096)
    return fail(MOE_ERR_INVALID_ARG, "timing_begin needs a layer and 1..4096 forwards");
  const size_t need = (size_t)max_forwards * MOE_NUM_STAGES * 2;
  while (L->tev.size() < need) {
    hipEvent_t e;
    HIP_TRY(hipEventCreate(&e));
    L->tev.push_back(e);
  }
  L->trec.assign((size_t)max_forwards * MOE_NUM_STAGES, 0);
  L->timing_mask = mask;
  L->timing_cap = max_forwards;
  L->timing_count = 0;
  L->timing = true;
  return MOE_OK;
}

int moe_layer_timing_end(moe_layer_t* L, float* total_ms, int32_t* launches) {
  if (!L || !total_ms || !launches) return fail(MOE_ERR_INVALID_ARG, "bad timing_end arguments");
  L->timing = false;
  for (int st = 0; st < MOE_NUM_STAGES; ++st) {
    total_ms[st] = 0.f;
    launches[st] = 0;
  }
  for (int f = 0; f < L->timing_count; ++f)
    for (int st = 0; st < MOE_NUM_STAGES; ++st) {
      const size_t i = (size_t)f * MOE_NUM_STAGES + st;
      if (!L->trec[i]) continue;
      HIP_TRY(hipEventSynchronize(L->tev[i * 2 + 1]));
      float ms = 0.f;
      HIP_TRY(hipEventElapsedTime(&ms, L->tev[i * 2], L->tev[i * 2 + 1]));
      total_ms[st] += ms;
      launches[st] += 1;
    }
  L->timing_count = 0;
  return MOE_OK;
}

int moe_layer_debug_read(moe_layer_t* L, int32_t which, void* dst, int64_t bytes, void* stream) {
  if (!L || !dst || bytes < 0) return fail(MOE_ERR_INVALID_ARG, "bad debug_read arguments");
  const moe_layer_config_t& c = L->cfg;
  const int64_t n = L->last_n, R = n * c.top_k;
  const void* src = nullptr;
  int64_t avail = 0;
  switch (which) {
    case MOE_DBG_NORMED: src = L->normed; avail = n * c.hidden_size * (int64_t)dt_size(c.act_dtype); break;
    case MOE_DBG_LOGITS: src = L->logits; avail = n * c.num_experts * 4; break;
    case MOE_DBG_IDS: src = L->ids; avail = R * 4; break;
    case MOE_DBG_WEIGHTS: src = L->w; avail = R * 4; break;
    case MOE_DBG_COUNTS: src = L->counts; avail = (int64_t)c.num_experts * 4; break;
    case MOE_DBG_OFFSETS: src = L->offsets; avail = (int64_t)(c.num_experts + 1) * 4; break;
    case MOE_DBG_PERM: src = L->perm; avail = R * 4; break;
    case MOE_DBG_INV: src = L->inv; avail = R * 4; break;
    default: return fail(MOE_ERR_INVALID_ARG, "unknown debug buffer %d", which);
  }
  if (n == 0) return fail(MOE_ERR_INVALID_ARG, "debug_read before any forward of this layer");
  if (bytes > avail)
    return fail(MOE_ERR_INVALID_ARG, "debug_read of %lld bytes exceeds the %lld written",
                (long long)bytes, (long long)avail);
  HIP_TRY(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, (hipStream_t)stream));
  return MOE_OK;
}

int moe_topk_sigmoid(const float* logits, int32_t n, int32_t E, int32_t k, float scale,
                     int32_t* ids, float* w, void* stream) {
  if (n < 0 || (n > 0 && (!logits || !ids || !w)))
    return fail(MOE_ERR_INVALID_ARG, "bad moe_topk_sigmoid arguments");
  if (E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > E || k > MOE_MAX_TOP_K)
    return fail(MOE_ERR_INVALID_CONFIG, "E=%d, k=%d outside the routing bounds", E, k);
  if (n == 0) return MOE_OK;
  HIP_TRY(launch_topk(logits, n, E, k, scale, ids, w, (hipStream_t)stream));
  return MOE_OK;
}

int moe_route_sort(const int32_t* ids, int32_t n, int32_t k, int32_t E, int32_t* counts,
                   int32_t* offsets, int32_t* perm, int32_t* inv, void* stream) {
  if (n < 0 || k < 1 || !counts || !offsets || (n > 0 && (!ids || !perm || !inv)))
    return fail(MOE_ERR_INVALID_ARG, "bad moe_route_sort arguments");
  if (E < 1 || E > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_INVALID_CONFIG, "E=%d outside 1..%d", E, MOE_MAX_EXPERTS);
  HIP_TRY(launch_route_sort(ids, n * k, E, counts, offsets, perm, inv, 0, nullptr, nullptr,
                            nullptr, (hipStream_t)stream));
  return MOE_OK;
}

int moe_route_sort_static(const int32_t* ids, int32_t n, int32_t k, int32_t E, int32_t* counts,
                          int32_t* offsets, int32_t* perm, int32_t* inv, void* stream) {
  // Size checks first: nothing below runs for a call the static scratch
  // cannot hold.
  if (n < 0 || k < 1) return fail(MOE_ERR_INVALID_ARG, "bad moe_route_sort_static arguments");
  if (E < 1 || E > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_INVALID_CONFIG, "E=%d outside 1..%d", E, MOE_MAX_EXPERTS);
  const long long R = (long long)n * k;
  if (R > (1LL << 30))
    return fail(MOE_ERR_INVALID_ARG, "n*k = %lld routes exceeds 2^30", R);
  const long long need = (long long)route_sort_blocks((int)R) * E;
  if (need > MOE_STATIC_SCRATCH_INTS)
    return fail(MOE_ERR_INVALID_ARG,
                "n*k = %lld routes with E=%d need %lld scratch ints, over the static "
                "scratch of %d (ceil(n*k/2048)*E must be <= %d)",
                R, E, need, MOE_STATIC_SCRATCH_INTS, MOE_STATIC_SCRATCH_INTS);
  if (!counts || !offsets || (n > 0 && (!ids || !perm || !inv)))
    return fail(MOE_ERR_INVALID_ARG, "bad moe_route_sort_static arguments");
  int* bcnt = nullptr;
  HIP_TRY(static_scratch(&bcnt));
  HIP_TRY(launch_route_sort(ids, (int)R, E, counts, offsets, perm, inv, 0, nullptr, nullptr, bcnt,
                            (hipStream_t)stream));
  return MOE_OK;
}

int moe_nvfp4_quantize(const float* w, int32_t G, int32_t rows, int32_t cols, uint8_t* packed,
                       uint8_t* scales, float* scale2, void* stream) {
  if (G < 0 || rows < 0 || cols < 0 || cols % 16 != 0)
    return fail(MOE_ERR_INVALID_ARG, "bad shape (cols must be a multiple of 16)");
  if ((size_t)G * rows * cols == 0) return MOE_OK;
  if (!w || !packed || !scales || !scale2) return fail(MOE_ERR_INVALID_ARG, "NULL pointer");
  HIP_TRY(launch_nvfp4_quantize(w, G, rows, cols, packed, scales, scale2, (hipStream_t)stream));
  return MOE_OK;
}

}  // extern "C"
