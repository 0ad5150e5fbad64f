/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE token-dispatch library, libmoe.so.
 *
 * One Mixture-of-Experts layer on one GPU: five steps in four calls, and one call for all:
 *   moe_route        router GEMM, softmax over all experts, top-k, optional renormalisation
 *   moe_permute      stable sort of the (token, slot) rows by expert: counts, offsets,
 *                    perm, inv_perm, plus the launch plan of the grouped FFN
 *   moe_grouped_ffn  all experts in one pass: gate/up with SwiGLU fused, then down
 *   moe_combine      weighted sum of each token's expert rows in a fixed order
 *   moe_forward      the whole layer (optionally RMSNorm first, residual last)
 *
 * What is computed follows the pages this library is built from: a router sends each
 * token to k of E experts (dispatch README, intro; switchyard page, opening paragraph:
 * OLMoE routes each token to 8 of its 64 experts); rows are sorted by expert with a prefix
 * scan and no atomics (switchyard §02 "Route and sort"); each expert is a SwiGLU block and
 * all experts run in one launch (switchyard §02 "One launch for all experts"); the combine
 * is atomic-free and its result does not depend on where experts ran (switchyard page,
 * hero statistics: expert-parallel output equal to one GPU bit for bit; §02 "Kernels and
 * dispatch").  Shared experts follow the DeepSeek-MoE layout (dispatch README, "Stack");
 * int8 weight-only experts follow dispatch's per-channel format (dispatch README, "What has
 * been measured", phase 5a).
 *
 * Conventions (every function):
 *  - Array arguments are DEVICE pointers allocated and owned by the caller.  The library
 *    never allocates, frees or keeps a pointer past the call, and reads nothing back to
 *    the host.  Descriptors (moe_layer_desc_t, moe_expert_weights_t) are HOST memory,
 *    read during the call only.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream); the call
 *    returns without synchronising.
 *  - Arguments are checked before anything is enqueued.  On error nothing is enqueued and
 *    a negative moe_status_t is returned; moe_last_error() gives a thread-local message.
 *    A kernel launch failure reported by the runtime returns MOE_ERR_DEVICE; a fault
 *    during execution surfaces at the caller's next synchronisation.
 *  - T == 0 is a valid no-op.
 *  - Results are deterministic: identical inputs give bit-identical outputs on every run
 *    (no floating-point atomics anywhere).
 *  - The library keeps no state between calls (apart from the static scratch array of
 *    moe_forward_noalloc); calls that run concurrently need distinct outputs and workspaces.
 *  - Every pointer must be 16-byte aligned.
 *
 * Matrices are row-major [out, in] with `in` contiguous (the layout of a PyTorch Linear
 * weight).  Experts 0..E-1 are routed, E..E+S-1 are the always-on shared experts.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = -1,     /* a null required pointer, misalignment, or a size out of range */
  MOE_ERR_UNSUPPORTED = -2, /* a valid request this library does not implement (see limits) */
  MOE_ERR_WORKSPACE = -3,   /* ws_bytes / plan_bytes smaller than moe_workspace_bytes() */
  MOE_ERR_DEVICE = -4       /* the HIP runtime refused a launch */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_I8 = 2 } moe_dtype_t;

/* Which call a workspace is sized for (moe_workspace_bytes). */
typedef enum { MOE_WS_PERMUTE = 0, MOE_WS_GROUPED_FFN = 1, MOE_WS_FORWARD = 2 } moe_ws_kind_t;

typedef struct {
  int32_t d_model;     /* d: hidden size, multiple of 16, <= 16384                       */
  int32_t n_experts;   /* E: routed experts, 1..256                                       */
  int32_t top_k;       /* k: experts per token, 1..min(E, 16)                             */
  int32_t d_ff;        /* I: intermediate size of every expert, multiple of 16, <= 16384  */
  int32_t n_shared;    /* S: always-on shared experts (gate weight 1.0), 0..8             */
  int32_t renormalize; /* 1: divide the k gate weights by their sum                      */
  int32_t act_dtype;   /* moe_dtype_t of x, router weight, h, rows and y: F32 or BF16     */
  int32_t w_dtype;     /* moe_dtype_t of expert weights: equal to act_dtype, or I8 with
                          act_dtype BF16 (int8 weight-only)                                */
  int32_t pre_norm;    /* moe_forward only: 1 = RMSNorm(x) (no scale) before the layer    */
  float norm_eps;      /* epsilon of that RMSNorm                                          */
  float capacity_factor; /* 0: dropless.  > 0: each routed expert keeps its first
                          C = ceil(capacity_factor * T * k / E) rows (switchyard §03 "Load
                          balance": a capacity limit drops what an expert has no room for);
                          see moe_permute                                                  */
} moe_layer_desc_t;

typedef struct {
  const void* w_gate;  /* [E+S, I, d]  w_dtype                                            */
  const void* w_up;    /* [E+S, I, d]  w_dtype                                            */
  const void* w_down;  /* [E+S, d, I]  w_dtype                                            */
  const float* s_gate; /* [E+S, I] fp32 scale per output channel; MOE_I8 only, else NULL  */
  const float* s_up;   /* [E+S, I]                                                        */
  const float* s_down; /* [E+S, d]                                                        */
} moe_expert_weights_t;

/* Bytes of device workspace a call needs for up to `max_tokens` tokens:
 *   MOE_WS_PERMUTE      the `plan` buffer written by moe_permute and read by moe_grouped_ffn
 *   MOE_WS_GROUPED_FFN  the `ws` of moe_grouped_ffn (holds h, the SwiGLU intermediate)
 *   MOE_WS_FORWARD      the `ws` of moe_forward (everything the layer needs in between)
 * Returns 0 if the descriptor is invalid. */
size_t moe_workspace_bytes(const moe_layer_desc_t* desc, int32_t max_tokens, int32_t which);

/* Step 1 -- router and top-k gating (dispatch README, "Why this project": top-k gating
 * ahead of the expert kernel; switchyard §02 "Route and sort": one wavefront per token).
 *   logits[t,e] = sum_c x[t,c] * w_router[e,c] + router_bias[e]   (fp32 accumulation)
 *   ids[t,:]    = the k largest logits, largest first; equal logits go to the lower id;
 *                 NaN ranks below every number
 *   w[t,j]      = softmax over all E logits of expert ids[t,j]; divided by the sum of the
 *                 k weights when desc->renormalize
 * x [T,d] act_dtype; w_router [E,d] act_dtype; router_bias [E] fp32 or NULL.
 * logits_in [T,E] fp32 or NULL: when given, the GEMM is skipped and these logits are used
 *   as they are (x, w_router and router_bias are then ignored and may be NULL).
 * logits_out [T,E] fp32: receives the logits; required when logits_in is NULL, may be NULL
 *   otherwise.
 * topk_ids [T,k] int32, topk_w [T,k] fp32: outputs.
 * desc->pre_norm must be 0 (MOE_ERR_UNSUPPORTED otherwise): the RMSNorm prologue is
 * moe_forward's; the step calls take x as given. */
int32_t moe_route(const moe_layer_desc_t* desc, int32_t T, const void* x, const void* w_router,
                  const float* router_bias, const float* logits_in, float* logits_out,
                  int32_t* topk_ids, float* topk_w, void* stream);

/* Step 2 -- sort of the T*k rows by expert with a prefix scan and no atomics (switchyard
 * §02 "Route and sort").  Row f = t*k + j is (token t, slot j).
 *   counts[e]   number of rows routed to expert e                      [E]      int32
 *   offsets[g]  start of group g's rows; offsets[E] = T*k; shared expert s owns rows
 *               T*k + s*T .. T*k + (s+1)*T - 1 in token order           [E+S+1]  int32
 *   perm[r]     flat index f of sorted row r; rows of one expert keep ascending f
 *   inv_perm[f] sorted position of flat row f, or -1 if the row was dropped  [T*k] int32
 *   plan        device buffer of plan_bytes >= moe_workspace_bytes(desc, T, MOE_WS_PERMUTE);
 *               receives the touched-expert list and tile list that moe_grouped_ffn reads.
 * With desc->capacity_factor > 0, expert e keeps the first C of its rows (the lowest flat
 * indices, i.e. the head of its sorted segment) and the others are dropped: their inv_perm
 * is -1, moe_grouped_ffn leaves them unwritten and moe_combine skips them.  counts,
 * offsets and perm still describe every row.  Shared experts never drop.
 * topk_ids must hold values in [0, E); other values give unspecified (but in-bounds)
 * results. */
int32_t moe_permute(const moe_layer_desc_t* desc, int32_t T, const int32_t* topk_ids,
                    int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                    void* plan, size_t plan_bytes, void* stream);

/* Steps 3-4 -- grouped expert FFN over the sorted rows, every expert in one launch per
 * matrix (switchyard §02 "One launch for all experts": SwiGLU fused into the epilogue; a
 * weight-streaming grouped GEMV at decode sizes).  For sorted row r of group g and token t:
 *   h[r]    = silu(W_gate[g] x[t]) * (W_up[g] x[t])       silu(z) = z / (1 + exp(-z))
 *   rows[r] = W_down[g] h[r]
 * with int8 weights: W[g][n,:] = q[g][n,:] * s[g][n] (per output channel), the scale being
 * applied to the fp32 accumulator.  Accumulation is fp32; h is rounded to act_dtype.
 * x [T,d]; offsets, perm as written by moe_permute; plan as written by that same
 * moe_permute call; rows [T*k + S*T, d] act_dtype (output: the rows of dropped slots are
 * left unwritten); ws >= moe_workspace_bytes(desc, T, MOE_WS_GROUPED_FFN).
 * desc->pre_norm must be 0 (MOE_ERR_UNSUPPORTED otherwise), as for moe_route. */
int32_t moe_grouped_ffn(const moe_layer_desc_t* desc, int32_t T, const void* x,
                        const moe_expert_weights_t* weights, const int32_t* offsets,
                        const int32_t* perm, const void* plan, void* rows, void* ws,
                        size_t ws_bytes, void* stream);

/* Step 5 -- deterministic combine (switchyard page, hero statistics and §02 "Kernels and
 * dispatch": an atomic-free result that does not depend on where the experts ran):
 *   y[t] = sum_{j<k} topk_w[t,j] * rows[inv_perm[t*k+j]] + sum_{s<S} rows[T*k+s*T+t]
 *          + residual[t]
 * summed in fp32 in exactly that order, rounded once to act_dtype.
 * rows [T*k+S*T, d]; inv_perm [T*k] (a slot with inv_perm < 0 was dropped by the
 * capacity limit and adds nothing); topk_w [T,k] fp32; residual [T,d] or NULL (may be the
 * same buffer as y); y [T,d] act_dtype. */
int32_t moe_combine(const moe_layer_desc_t* desc, int32_t T, const void* rows,
                    const int32_t* inv_perm, const float* topk_w, const void* residual,
                    void* y, void* stream);

/* The whole layer: [RMSNorm] -> route -> permute -> grouped FFN -> combine (the layer as the
 * switchyard page draws it: tokens, router top-k, experts, combine, §02 "Kernels and
 * dispatch"; the RMSNorm prologue and residual serve a stack of such layers, one per
 * transformer block).
 *   y = residual + MoE(pre_norm ? x / sqrt(mean(x^2) + eps) : x)
 * The normalised input is rounded to act_dtype and fed to both router and experts.
 * x [T,d]; residual [T,d] or NULL (may alias x or y); y [T,d] (may alias x).
 * topk_ids_out [T,k] / topk_w_out [T,k]: optional copies of the routing (NULL to skip).
 * ws >= moe_workspace_bytes(desc, T, MOE_WS_FORWARD).
 * At decode sizes on the MOE_FFN_GEMV family, when every row's activations fit in one
 * workgroup's LDS (up to 9 tokens on an OLMoE-shaped layer, 6 on a DeepSeek-MoE-shaped one),
 * the down projection and the combine run as one launch; y is bit-identical to the separate
 * steps either way. */
int32_t moe_forward(const moe_layer_desc_t* desc, int32_t T, const void* x, const void* w_router,
                    const float* router_bias, const moe_expert_weights_t* weights,
                    const void* residual, void* y, int32_t* topk_ids_out, float* topk_w_out,
                    void* ws, size_t ws_bytes, void* stream);

/* moe_forward without a caller workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, serving loops that forbid allocation): the workspace is a
 * static scratch array inside the library's device code, 128 MiB, one copy per GPU, held
 * from the library's first use on that GPU until the process ends.  Arguments, results and
 * determinism are those of moe_forward (same kernels, bit-identical outputs); the call
 * allocates and frees nothing.  A layer and T whose moe_workspace_bytes(desc, T,
 * MOE_WS_FORWARD) exceeds 128 MiB is refused with MOE_ERR_WORKSPACE (about 2,700 tokens for
 * an OLMoE-shaped layer, 2,400 for a DeepSeek-MoE-shaped one).  Every call on one GPU uses
 * that GPU's one scratch array: calls that overlap in time on the same GPU (different
 * streams, or threads) race and give undefined results; serialise them.  The device is the
 * one `stream` belongs to. */
int32_t moe_forward_noalloc(const moe_layer_desc_t* desc, int32_t T, const void* x,
                            const void* w_router, const float* router_bias,
                            const moe_expert_weights_t* weights, const void* residual, void* y,
                            int32_t* topk_ids_out, float* topk_w_out, void* stream);

/* Kernels of the path, for moe_time_next_launch. */
typedef enum {
  MOE_KERNEL_RMSNORM = 0,  /* pre-norm of moe_forward                    */
  MOE_KERNEL_ROUTER = 1,   /* router GEMM                                */
  MOE_KERNEL_TOPK = 2,     /* softmax + top-k                            */
  MOE_KERNEL_PERMUTE = 3,  /* sort by expert + launch plan               */
  MOE_KERNEL_GATE_UP = 4,  /* grouped gate/up with the SwiGLU epilogue   */
  MOE_KERNEL_DOWN = 5,     /* grouped down projection                    */
  MOE_KERNEL_COMBINE = 6,  /* weighted combine                           */
  MOE_KERNEL_COUNT = 7
} moe_kernel_t;

/* One-shot timing hook for measuring a single kernel inside a call: the next launch of
 * `kernel` made by this thread (through any entry point) records start_event and stop_event
 * on that launch's stream, and the hook is then cleared.  A step that is one launch hands
 * the events to the launch itself (hipExtLaunchKernel), so they hold the kernel's own start
 * and end, the window a profiler's kernel trace reports; the multi-workgroup sort (chunk
 * histograms, past 64 chunks their scan, then the sort: two or three launches) is bracketed
 * by hipEventRecord before the first and after the last.  Where moe_forward runs the down projection and the combine as
 * one launch, MOE_KERNEL_DOWN holds that launch's own window and MOE_KERNEL_COMBINE brackets
 * the same launch.  The events (hipEvent_t) are created and owned by the caller;
 * NULL events disarm the hook.  Returns MOE_ERR_INVALID for an unknown kernel. */
int32_t moe_time_next_launch(int32_t kernel, void* start_event, void* stop_event);

/* Which kernel family moe_grouped_ffn (and moe_forward) launches for T tokens of this layer
 * (switchyard §02 "One launch for all experts": a weight-streaming grouped GEMV at decode
 * sizes, a grouped GEMM beyond; here a third family sits between them):
 *   MOE_FFN_GEMV       weight-streaming GEMV with VALU dot products (groups of a few rows)
 *   MOE_FFN_GEMV_MFMA  the same weight streaming with matrix-core math (groups of up to a few
 *                      dozen rows; bf16 activations, d and I multiples of 64)
 *   MOE_FFN_GEMM       grouped matrix-core GEMM fed by an LDS ring (larger groups)
 * All three compute the same function with fp32 accumulation; their results may differ in the
 * last bits.  Host-only: touches no GPU.  Returns the family, or a negative moe_status_t for
 * an invalid descriptor or T outside 1 .. the supported maximum. */
typedef enum { MOE_FFN_GEMV = 0, MOE_FFN_GEMV_MFMA = 1, MOE_FFN_GEMM = 2 } moe_ffn_kernel_t;
int32_t moe_ffn_kernel(const moe_layer_desc_t* desc, int32_t T);

/* Name of a status code, and the detail of this thread's last failure ("" if none). */
const char* moe_status_str(int32_t status);
const char* moe_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int32_t moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
