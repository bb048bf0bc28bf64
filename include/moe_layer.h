/*
 * moe_layer.h — C ABI of the MI355X (gfx950) Nemotron-H MoE FFN layer.
 *
 * The layer computes, for each of N token rows of `hidden` [N, H]
 * (page "metrale_model_arch/nemotron_moe.rs", module doc and
 * `NemotronMoeLayer::prefill`; page "Struct MoeLayer", `forward_prefill`):
 *
 *   residual_t = hidden_t                                   (pre-norm save)
 *   n_t        = hidden_t / sqrt(mean(hidden_t^2) + eps) * gamma
 *   s_t        = sigmoid(W_gate n_t)                         (fp32)
 *   ids_t      = the top_k experts by (s desc, index asc)
 *   w_tj       = s_t[ids_tj] / sum_j s_t[ids_tj] * routed_scaling_factor
 *   z_t        = fc1 n_t if latent_size > 0 else n_t
 *   routed_t   = sum_j w_tj * down_e relu(up_e z_t)^2,   e = ids_tj
 *   routed_t   = fc2 routed_t if latent_size > 0
 *   shared_t   = shared_down relu(shared_up n_t)^2       (0 if shared_inter == 0)
 *   hidden_t  <- residual_t + routed_t + shared_t
 *
 * Routing never reads back to the host: the top-k, the per-expert histogram,
 * its prefix sum and the scatter of routes run on the device (module doc of
 * the nemotron_moe.rs page; "Struct MoeLayer", `forward`).
 *
 * Conventions for every entry point:
 *   - Tensor arguments are DEVICE pointers (HBM of the current HIP device),
 *     row-major, densely packed. Matrices are [out][in] (the layout of the
 *     pages' packed `[N, K/2]` expert tables).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued on it and the call returns without synchronizing,
 *     except moe_layer_create, which synchronizes its stream before returning.
 *   - Return value: MOE_OK (0) or a negative MOE_ERR_* code. Every argument
 *     check runs on the host before any launch; on error nothing is enqueued
 *     and moe_last_error() returns a message (thread-local, valid until the
 *     next call on the same thread).
 */
#ifndef MOE_LAYER_H
#define MOE_LAYER_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,     /* NULL pointer, negative size, bad enum */
  MOE_ERR_INVALID_CONFIG = -2,  /* config refused (see moe_layer_create) */
  MOE_ERR_TOO_MANY_TOKENS = -3, /* num_tokens > max_tokens of the layer */
  MOE_ERR_OOM = -4,             /* device allocation failed in create */
  MOE_ERR_HIP = -5              /* a HIP runtime call or launch failed */
};

/* Storage types. NVFP4 = 4-bit E2M1 values, one E4M3 scale per 16 values
 * along K, one fp32 scale2 per matrix (page "metrale_model_arch/
 * nemotron_moe.rs", `ExpertPtrTable`: packed table, scale table, scale2). */
enum { MOE_DT_F32 = 0, MOE_DT_BF16 = 1, MOE_DT_NVFP4 = 2 };

/* Routing bounds of this library (the pages' constructor checks top_k and
 * num_experts against routing-kernel bounds whose values they do not print). */
#define MOE_MAX_EXPERTS 512
#define MOE_MAX_TOP_K 16

/* Layer shape (page "metrale_model_arch/nemotron_moe.rs": hidden_size,
 * num_experts, top_k, moe_inter, shared_expert_intermediate_size,
 * moe_latent_size, rms_norm_eps, routed_scaling_factor). */
typedef struct {
  int32_t hidden_size;    /* H */
  int32_t num_experts;    /* E, 1..MOE_MAX_EXPERTS */
  int32_t top_k;          /* k, 1..min(E, MOE_MAX_TOP_K) */
  int32_t moe_inter;      /* I, routed expert intermediate size */
  int32_t shared_inter;   /* S, shared expert intermediate size; 0 = none */
  int32_t latent_size;    /* L; 0 = direct (experts act on H), > 0 = LatentMoE */
  int32_t max_tokens;     /* largest N a forward may pass; sizes the workspace */
  float rms_eps;          /* RMSNorm epsilon (1e-5 in the shipped workloads) */
  float routed_scaling_factor; /* multiplies the routed sum (1.0 typical) */
  int32_t act_dtype;      /* MOE_DT_F32 | MOE_DT_BF16: hidden, residual, gamma,
                             gate, fc1, fc2 */
  int32_t expert_dtype;   /* MOE_DT_F32 | MOE_DT_BF16 | MOE_DT_NVFP4: routed and
                             shared experts. F32 requires act F32; BF16 and
                             NVFP4 require act BF16. */
} moe_layer_config_t;

/* One NVFP4 matrix stack [G][rows][K]: packed u8 [G][rows][K/2] (element k in
 * byte k/2, low nibble when k is even), E4M3 scales u8 [G][rows][K/16],
 * scale2 fp32 [G]. Value = e2m1(q) * e4m3(s) * scale2[g]. */
typedef struct {
  const void* packed;
  const void* scales;
  const float* scale2;
} moe_nvfp4_t;

/* Weights (page "metrale_model_arch/nemotron_moe.rs": NemotronMoeWeights,
 * input_norm). D = latent_size if latent else hidden_size.
 *   norm_gamma [H], gate [E][H]                     act dtype
 *   fc1 [L][H], fc2 [H][L] (latent only, else NULL)  act dtype
 *   up [E][I][D], down [E][D][I]                     expert dtype (F32/BF16)
 *   shared_up [S][H], shared_down [H][S]             expert dtype (F32/BF16)
 *   up_q, down_q, shared_up_q, shared_down_q         NVFP4 only (G = E for
 *                                                    up/down, G = 1 shared)
 * Unused pointers must be NULL. */
typedef struct {
  const void* norm_gamma;
  const void* gate;
  const void* fc1;
  const void* fc2;
  const void* up;
  const void* down;
  const void* shared_up;
  const void* shared_down;
  moe_nvfp4_t up_q, down_q, shared_up_q, shared_down_q;
} moe_layer_weights_t;

typedef struct moe_layer moe_layer_t;

/* Build a layer (page "metrale_model_arch/nemotron_moe.rs",
 * `NemotronMoeLayer::new`). The weights are copied (and repacked) into
 * layer-owned device memory; the caller may free its buffers once this
 * returns. A workspace for max_tokens is allocated here, so forward never
 * allocates. Synchronizes `stream`.
 * Errors: MOE_ERR_INVALID_ARG (NULL cfg/weights/out, missing weight),
 * MOE_ERR_INVALID_CONFIG (top_k outside 1..E, E > MOE_MAX_EXPERTS, top_k >
 * MOE_MAX_TOP_K, H/I/S/L not multiples of 64 (of 16 for f32 layers),
 * H > 8192, unsupported dtype pair, max_tokens < 1, max_tokens * top_k >
 * 2^30 routes), MOE_ERR_OOM, MOE_ERR_HIP.
 * On error *out is set to NULL. */
int moe_layer_create(const moe_layer_config_t* cfg, const moe_layer_weights_t* weights,
                     void* stream, moe_layer_t** out);

/* Forward over num_tokens rows (page "metrale_model_arch/nemotron_moe.rs",
 * `NemotronMoeLayer::prefill`; page "Struct NemotronMoeLayer", `decode`:
 * hidden is modified in place). hidden [N][H] in/out and residual [N][H]
 * out, act dtype, caller-owned. The input value of residual is ignored.
 * Asynchronous on `stream`: no host synchronization, no allocation, no
 * device-to-host copy. One forward at a time per layer (the workspace is
 * shared). num_tokens == 0 returns MOE_OK with nothing enqueued.
 * Small N (<= 16) runs the weight-streaming GEMV arm; larger N the sorted
 * grouped-GEMM arm, whose shared-expert launches go to a layer-owned stream
 * forked from and joined back to `stream` by events within the call, so all
 * of the forward's work is ordered after earlier work on `stream` and before
 * later work on it, and the call captures whole into a HIP graph.
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_TOO_MANY_TOKENS, MOE_ERR_HIP. */
int moe_layer_forward(moe_layer_t* layer, void* hidden, void* residual, int32_t num_tokens,
                      void* stream);

/* Free a layer and its device memory (NULL is a no-op). Synchronizes the
 * device work the layer enqueued. */
void moe_layer_destroy(moe_layer_t* layer);

/* Message for the last non-OK return on this thread ("" if none). */
const char* moe_last_error(void);

/* ---- Stage entry points (each one step of the forward, for stage-level
 * parity checks). ---- */

/* Sigmoid top-k with renormalized weights (page "metrale_model_arch/
 * nemotron_moe.rs": the batched sigmoid top-k routing kernel).
 * logits fp32 [n][E] -> ids int32 [n][k] (slot order: score desc, index asc),
 * w fp32 [n][k] = s / sum(s) * scale. One wavefront per token. */
int moe_topk_sigmoid(const float* logits, int32_t n, int32_t E, int32_t k, float scale,
                     int32_t* ids, float* w, void* stream);

/* Stable sort of routes r = t*k + j by expert ids[t][j] (page "Struct
 * MoeLayer", `forward_prefill`: sort step). ids int32 [n][k], values in
 * [0, E). Outputs: counts int32 [E], offsets int32 [E+1] (exclusive prefix
 * sum), perm int32 [n*k] (route at each sorted position, ascending r within
 * an expert), inv int32 [n*k] (sorted position of each route). */
int moe_route_sort(const int32_t* ids, int32_t n, int32_t k, int32_t E, int32_t* counts,
                   int32_t* offsets, int32_t* perm, int32_t* inv, void* stream);

/* Allocation-free form of moe_route_sort, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops and harnesses
 * that forbid allocation). Same arguments and bit-identical outputs as
 * moe_route_sort; runs the multi-block form of the sort (the one the layer's
 * forward uses at large route counts: a per-block expert histogram, then a
 * stable ballot-ranked scatter per block), whose per-block counts live in a
 * static device array of MOE_STATIC_SCRATCH_BYTES (1 MiB) that each GPU the
 * library runs on keeps until the process ends. Nothing is allocated and
 * nothing in that array needs clearing (every call writes the counts it
 * reads). Limit: ceil(n*k / 2048) * E <= 262144 (for example n*k up to 4M
 * routes at E = 128, 1M at E = 512); larger calls return
 * MOE_ERR_INVALID_ARG before anything is enqueued. Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (other
 * streams, other threads) race and must be serialized by the caller. */
#define MOE_STATIC_SCRATCH_BYTES (1 << 20)
int moe_route_sort_static(const int32_t* ids, int32_t n, int32_t k, int32_t E, int32_t* counts,
                          int32_t* offsets, int32_t* perm, int32_t* inv, void* stream);

/* Two-level NVFP4 quantizer for weights, into the storage format of page
 * "metrale_model_arch/nemotron_moe.rs" (`ExpertPtrTable`: packed table, block
 * scale table, scale2). The pages print no weight quantizer; this recipe is
 * the library's reading of the format (the page's own quantize kernel turns
 * bf16 activations into NVFP4 for the 4-bit x 4-bit GEMMs).
 * w fp32 [G][rows][cols] (cols % 16 == 0) -> packed u8 [G][rows][cols/2],
 * scales u8 [G][rows][cols/16], scale2 fp32 [G], per matrix g:
 *   scale2 = amax|W_g| / 2688, s_b = E4M3_rne(amax_b / (6 * scale2)),
 *   q = E2M1_rne(w / (e4m3(s_b) * scale2)) saturating at 6, ties to even,
 * all in fp32; a zero magnitude has its sign bit clear. */
int moe_nvfp4_quantize(const float* w, int32_t groups, int32_t rows, int32_t cols,
                       uint8_t* packed, uint8_t* scales, float* scale2, void* stream);

/* Internal buffers of the last forward, copied device-to-device into dst
 * (stream-ordered after that forward). `which`: */
enum {
  MOE_DBG_NORMED = 0,   /* act dtype [N][H] */
  MOE_DBG_LOGITS = 1,   /* fp32 [N][E] */
  MOE_DBG_IDS = 2,      /* int32 [N][k] */
  MOE_DBG_WEIGHTS = 3,  /* fp32 [N][k] */
  MOE_DBG_COUNTS = 4,   /* int32 [E] */
  MOE_DBG_OFFSETS = 5,  /* int32 [E+1] */
  MOE_DBG_PERM = 6,     /* int32 [N*k] */
  MOE_DBG_INV = 7       /* int32 [N*k] */
};
/* Copies the first `bytes` bytes of buffer `which` (MOE_ERR_INVALID_ARG if
 * bytes exceeds what the last forward wrote). */
int moe_layer_debug_read(moe_layer_t* layer, int32_t which, void* dst, int64_t bytes,
                         void* stream);

/* ---- Stage timing (tracing). When enabled, each forward records a HIP
 * event pair around every selected stage, on the stream that stage runs on
 * (the side stream for the shared expert). Not for use under graph capture. */
enum {
  MOE_STAGE_NORM_GATE = 0,    /* RMSNorm + residual + gate logits */
  MOE_STAGE_SHARED_UP = 1,    /* shared expert up GEMM + relu^2 */
  MOE_STAGE_SHARED_DOWN = 2,  /* shared expert down GEMM */
  MOE_STAGE_FC1 = 3,          /* latent fc1 GEMM */
  MOE_STAGE_TOPK = 4,         /* sigmoid top-k */
  MOE_STAGE_SORT = 5,         /* histogram / prefix sum / scatter */
  MOE_STAGE_GROUPED_UP = 6,   /* grouped up GEMM + relu^2 */
  MOE_STAGE_GROUPED_DOWN = 7, /* grouped down GEMM */
  MOE_STAGE_REDUCE = 8,       /* unpermute + weighted reduce (+ shared + residual) */
  MOE_STAGE_FC2 = 9,          /* latent fc2 GEMM (+ shared + residual) */
  MOE_NUM_STAGES = 10
};
/* Start recording the stages whose bit (1 << stage) is set in stage_mask for
 * the next max_forwards forwards (1..4096; later forwards are not recorded).
 * Allocates the events; call outside any timed or captured region. */
int moe_layer_timing_begin(moe_layer_t* layer, uint32_t stage_mask, int32_t max_forwards);
/* Stop recording, wait for the recorded events, and write per stage the sum
 * of the recorded durations in milliseconds (total_ms[MOE_NUM_STAGES]) and
 * how many launches were recorded (launches[MOE_NUM_STAGES]). */
int moe_layer_timing_end(moe_layer_t* layer, float* total_ms, int32_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* MOE_LAYER_H */
