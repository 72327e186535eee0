/*
 * moe_api.h -- C ABI of the MI355X (gfx950) LatentMoE layer forward.
 *
 * The layer (the "Nemotron 3 Ultra 架构 QA" page, CH5 Q5.1-Q5.8 with the
 * activation of Q2.6; the Nemotron-3 Ultra architecture walkthrough on
 * 2kiu.com, section "LatentMoE 层"):
 *
 *   l   = x . W_r^T                 fp32 router logits over the uncompressed x   (QA Q5.2)
 *   s   = sigmoid(l)                independent per expert                       (QA Q5.2)
 *   c   = s + e_score_correction_bias, top-K experts by c                        (QA Q5.2, Q5.3)
 *   g   = routed_scaling * s[chosen] / sum(s[chosen])                            (walkthrough; QA Q5.8)
 *   z   = x . W_fc1^T               fc1_latent_proj, H -> L                       (QA Q5.1)
 *   y_e = W_down[e] . relu(W_up[e] . z)^2, non-gated expert MLP, L -> I -> L      (QA Q2.6, Q5.5, Q5.6)
 *   y_lat = sum_k g_k * y_{e_k}     gate applied to each expert output, summed    (QA Q5.5 point 3)
 *   out = y_lat . W_fc2^T + W_sd . relu(W_su . x)^2                               (QA Q5.1, Q5.7)
 *
 * Conventions for every entry point:
 *  - Pointers marked "device" point to GPU memory on the current HIP device;
 *    the caller allocates, owns and frees every buffer, including the
 *    workspace. The library never allocates device memory and keeps no state
 *    between calls.
 *  - bf16 tensors are passed as uint16_t bit patterns (IEEE binary32 upper
 *    halves). All matrices are row-major; every weight is [out, in] (the
 *    reduction index is contiguous).
 *  - Calls are asynchronous on `stream` (0 = the null stream): no host
 *    synchronisation, no host<->device copy. The return code reports argument
 *    validation and launch errors; faults inside kernels surface at the
 *    caller's next synchronisation.
 *  - Nothing throws across the ABI. Results are deterministic: a call with the
 *    same inputs gives bit-identical outputs (no floating-point atomics).
 *  - A token's K experts are reported in ascending expert index; equal choice
 *    scores are resolved toward the lower expert index.
 */
#ifndef MOE_API_H
#define MOE_API_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Sizes of one forward. T tokens, H hidden, L latent (moe_latent_size), E routed
 * experts, I expert intermediate, K experts per token, Is shared-expert
 * intermediate; routed_scaling multiplies the renormalised gates (5.0 in the
 * stated model, QA Q5.8). Host struct.
 *
 * n_group / topk_group: group-limited selection. The walkthrough section
 * "路由与共享专家" takes the top-K within groups and QA Q9.2 has the layer
 * inherit DeepseekV3MoE's routing; no page gives the group count, so the
 * default (0 or 1 for both) is the plain top-K over all E experts. With
 * n_group > 1 the E experts form n_group equal contiguous groups, a group's
 * score is the sum of its two highest choice scores (its one score for
 * one-expert groups), the topk_group best groups (equal scores: the lower
 * group) admit their experts, and the top-K is taken among those. Requires
 * E % n_group == 0, 1 <= topk_group <= n_group, K <= topk_group * E / n_group
 * (else MOE_ERR_INVALID) and n_group <= 64 (else MOE_ERR_UNSUPPORTED). */
typedef struct moe_dims {
  int32_t T, H, L, E, I, K, Is;
  float routed_scaling;
  int32_t n_group, topk_group;
} moe_dims;

/* Weights, all device pointers, all [out, in] row-major.
 *   w_router  [E, H]    fp32   router weight (QA Q5.2 reads it as fp32)
 *   corr_bias [E]       fp32   e_score_correction_bias (QA Q5.3, kept in fp32)
 *   w_fc1     [L, H]    bf16   fc1_latent_proj
 *   w_up      [E, I, L] bf16   expert up projections (QA Q5.6 3-D layout)
 *   w_down    [E, L, I] bf16   expert down projections
 *   w_fc2     [H, L]    bf16   fc2_latent_proj
 *   w_sh_up   [Is, H]   bf16   shared expert up
 *   w_sh_down [H, Is]   bf16   shared expert down
 * Every weight and activation pointer must be 16-byte aligned (the kernels
 * move 16 bytes per lane); moe_forward rejects others with MOE_ERR_INVALID. */
typedef struct moe_weights {
  const float* w_router;
  const float* corr_bias;
  const uint16_t* w_fc1;
  const uint16_t* w_up;
  const uint16_t* w_down;
  const uint16_t* w_fc2;
  const uint16_t* w_sh_up;
  const uint16_t* w_sh_down;
} moe_weights;

enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID = -1,      /* null pointer, non-positive size, K > E, bad C, bad groups */
  MOE_ERR_UNSUPPORTED = -2,  /* H, L, I or Is not a multiple of 64; E > 1024; K > 64;
                                T*K >= 2^31; 2*T*L >= 2^32 */
  MOE_ERR_WORKSPACE = -3,    /* workspace null, too small or not 256-byte aligned */
  MOE_ERR_HIP = -4,          /* a HIP launch failed */
  MOE_ERR_TOO_LARGE = -5     /* moe_forward_noalloc: the forward needs more than its static scratch */
};

/* Byte offsets, inside the moe_forward workspace, of the intermediate tensors
 * it leaves behind (valid after the stream reaches the end of the call):
 *   idx [T,K] int32, gate [T,K] fp32, gap [T] fp32, offsets [E+1] int32,
 *   row_token [T*K] int32, slot_row [T*K] int32 (index t*K+k),
 *   z [T,L] bf16, h [T*K,I] bf16, y [T*K,L] bf16, y_lat [T,L] bf16, hs [T,Is] bf16.
 * Returns MOE_OK or MOE_ERR_INVALID. */
typedef struct moe_ws_layout {
  size_t idx, gate, gap, offsets, row_token, slot_row, z, h, y, y_lat, hs, total;
} moe_ws_layout;

/* Router: fp32 logits, sigmoid, bias-adjusted top-K, renormalised and scaled gates.
 * (QA Q5.2, Q5.3, Q5.8; walkthrough "路由与共享专家"). Reads T, H, E, K,
 * routed_scaling, n_group and topk_group of dims (the other fields are ignored).
 *   x         device [T,H] bf16
 *   w_router  device [E,H] fp32;  corr_bias device [E] fp32
 *   topk_idx  device [T,K] int32 out: chosen experts, ascending per token
 *   topk_gate device [T,K] fp32 out: routed_scaling * s / sum(s) over the chosen
 *   topk_gap  device [T]   fp32 out, may be NULL: c_(K) - c_(K+1), the margin
 *             between the last chosen and the first unchosen admitted choice
 *             score in descending order (+inf when every admitted expert is
 *             chosen); with groups, the smaller of that and the margin between
 *             the last admitted and the first refused group score
 *   ws        device workspace of at least moe_route_workspace_bytes(dims) bytes,
 *             256-byte aligned
 * The logits are accumulated in fp32 from exact bf16 x fp32 products (the fp32
 * weight is split exactly into three bf16 parts: by a pass over the weight for
 * the tiled product, in registers for forwards of at most 64 tokens; from 4096
 * tokens the tiled product sums the two halves of H separately and adds them,
 * and with at most 128 experts it also sums each weight part separately); only
 * the summation order differs from an exact fp32 dot product. */
size_t moe_route_workspace_bytes(const moe_dims* dims);
int moe_route(const moe_dims* dims, const uint16_t* x, const float* w_router,
              const float* corr_bias, int32_t* topk_idx, float* topk_gate, float* topk_gap,
              void* ws, size_t ws_bytes, hipStream_t stream);

/* Permutation: group the T*K (token, slot) pairs by expert, tokens ascending within
 * an expert -- the rows a loop over the hit experts gathers (QA Q5.6) -- and
 * gather rows of `src` into that order. Reads T, E, K of dims (the other
 * fields are ignored). Entries of topk_idx outside [0,E) are skipped and their
 * slot_row is set to -1: the valid rows are then [0, off[E]) and, past them,
 * row_token is left unwritten and dst holds zero rows.
 *   topk_idx       device [T,K] int32, values in [0,E), distinct within a token
 *   src            device [T,C] bf16 (may be NULL together with dst: maps only)
 *   C              row length of src/dst in elements, a multiple of 8
 *   dst            device [T*K, C] bf16 out: dst[r] = src[row_token[r]] for r < off[E], else 0
 *   expert_offsets device [E+1] int32 out: rows of expert e are [off[e], off[e+1])
 *   row_token      device [T*K] int32 out: token of permuted row r
 *   slot_row       device [T*K] int32 out: permuted row of slot (t,k), index t*K+k
 *   ws             device workspace, >= moe_permute_workspace_bytes(dims), 256-aligned
 * Bit-exact and deterministic (no order-dependent atomics). */
size_t moe_permute_workspace_bytes(const moe_dims* dims);
int moe_permute(const moe_dims* dims, const int32_t* topk_idx, const uint16_t* src, int32_t C,
                uint16_t* dst, int32_t* expert_offsets, int32_t* row_token, int32_t* slot_row,
                void* ws, size_t ws_bytes, hipStream_t stream);

/* Whole layer forward (QA Q5.1): route -> permute -> fc1 -> experts (up, relu^2,
 * down) -> gate-weighted combine -> fc2 + shared expert.
 *   x   device [T,H] bf16;  out device [T,H] bf16 (fp32 accumulation, one rounding)
 *   ws  device workspace, >= moe_workspace_bytes(dims) bytes, 256-byte aligned;
 *       it keeps the intermediates listed in moe_ws_layout.
 * Intermediate roundings to bf16: z, h, y, y_lat, hs (the tensors the layer
 * stores in bf16); every sum is fp32.
 * Every kernel of the call runs on `stream`, in order; the library creates no
 * stream or event. Calls from several host threads are independent as long as
 * they use different workspaces and outputs. */
size_t moe_workspace_bytes(const moe_dims* dims);
int moe_workspace_layout(const moe_dims* dims, moe_ws_layout* layout);
int moe_forward(const moe_dims* dims, const moe_weights* w, const uint16_t* x, uint16_t* out,
                void* ws, size_t ws_bytes, hipStream_t stream);

/* Phases of moe_forward, in launch order. */
enum moe_phase {
  MOE_PHASE_ROUTER_SPLIT = 0,  /* fp32 router weight -> three bf16 parts */
  MOE_PHASE_ROUTER_GEMM,       /* router logits */
  MOE_PHASE_TOPK,              /* sigmoid, biased top-K, gates */
  MOE_PHASE_PERMUTE,           /* masks, scans, scatter */
  MOE_PHASE_FC1_SHARED_UP,     /* z = fc1(x) and hs = relu^2(sh_up(x)), one launch */
  MOE_PHASE_EXPERT_UP,         /* h = relu^2(up_e(z)) over the permuted rows */
  MOE_PHASE_EXPERT_DOWN,       /* y = down_e(h) */
  MOE_PHASE_COMBINE,           /* y_lat = sum_k g_k y */
  MOE_PHASE_FC2_SHARED_DOWN,   /* out = fc2(y_lat) + sh_down(hs), one launch */
  MOE_N_PHASES
};

/* moe_forward with timing markers, for measurement: before phase i it records
 * events[i] on `stream`, and after the last phase events[MOE_N_PHASES]
 * (hipEventRecord; the caller creates and owns the events). n_events must be at
 * least MOE_N_PHASES + 1, else MOE_ERR_INVALID. Same results as moe_forward. */
int moe_forward_profiled(const moe_dims* dims, const moe_weights* w, const uint16_t* x, uint16_t* out,
                         void* ws, size_t ws_bytes, hipStream_t stream, hipEvent_t* events, int n_events);

/* MX expert weights (OCP Microscaling formats: one E8M0 power-of-two scale per
 * 32 consecutive elements of a row). The released model stores its experts
 * block-scaled in 4 bits (the QA page on the experts' NVFP4 storage); these are
 * the block-scaled formats gfx950 decodes natively, for the weight-bound
 * few-token (decode) forward:
 *   format 0 (MXFP8): FP8 E4M3fn elements, one byte each (about 1/2 of bf16);
 *   format 1 (MXFP4): FP4 E2M1 elements, two per byte, element 2i in the low
 *                     nibble of byte i (about 1/4 of bf16).
 *   w_up        device [E, I, L]  or [E, I, L/2] (MXFP4) uint8 codes
 *   w_up_scale  device [E, I, L/32] uint8 E8M0 codes (scale 2^(code - 127))
 *   w_down      device [E, L, I]  or [E, L, I/2] (MXFP4) uint8 codes
 *   w_down_scale device [E, L, I/32] uint8 E8M0 codes
 * A weight's value is element(code) * 2^(scale code - 127). The code tensors
 * must be 16-byte aligned. */
typedef struct moe_experts_mx {
  const uint8_t* w_up;
  const uint8_t* w_up_scale;
  const uint8_t* w_down;
  const uint8_t* w_down_scale;
  int32_t format;          /* 0 = MXFP8 (E4M3), 1 = MXFP4 (E2M1) */
} moe_experts_mx;

/* Quantise bf16 weights src [rows, cols] (device, row-major; cols a multiple of
 * 32) to MXFP8: codes [rows, cols] and scales [rows, cols/32] (device, caller
 * owned). Per block of 32: e = floor(log2(max|v|)) - 8 clamped to [-127, 127]
 * (an all-zero block: e = -127), scale code e + 127; each element is
 * v * 2^-e rounded to the nearest E4M3 value, ties to even, saturating at 448.
 * Expert tensors [E, out, in] quantise as rows = E * out, cols = in.
 * MOE_ERR_INVALID for null pointers, src or codes not 16-byte aligned, rows <= 0
 * or cols not a positive multiple of 32. Asynchronous on `stream`. */
int moe_quantize_mxfp8(const uint16_t* src, int64_t rows, int32_t cols, uint8_t* codes, uint8_t* scales,
                       hipStream_t stream);

/* MXFP4 quantisation of bf16 weights src [rows, cols] (device, row-major; cols
 * a multiple of 32) into packed codes [rows, cols/2] (element 2i in the low
 * nibble of byte i) and scales [rows, cols/32] (device, caller owned). Per
 * block of 32: e = floor(log2(max|v|)) - 2 clamped to [-127, 127] (an all-zero
 * block: e = -127), scale code e + 127; each element is v * 2^-e rounded to the
 * nearest E2M1 value (0, 0.5, 1, 1.5, 2, 3, 4, 6 and negatives), ties to the
 * code with mantissa bit 0, saturating at 6. Errors as moe_quantize_mxfp8. */
int moe_quantize_mxfp4(const uint16_t* src, int64_t rows, int32_t cols, uint8_t* codes, uint8_t* scales,
                       hipStream_t stream);

/* moe_forward with the routed experts' weights in an MX format (`mx`; w->w_up
 * and w->w_down are not read and may be NULL). Same workspace as moe_forward. The
 * expert products decode each weight to its exact bf16 value in registers and
 * run the bf16 path, so the results are those of moe_forward on the
 * dequantised weights. Few-token forwards only: T > 64 returns
 * MOE_ERR_UNSUPPORTED (the tiled expert products read bf16 weights); a format
 * other than 0 or 1 returns MOE_ERR_INVALID. */
int moe_forward_mx(const moe_dims* dims, const moe_weights* w, const moe_experts_mx* mx, const uint16_t* x,
                   uint16_t* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_forward_mx with the timing markers of moe_forward_profiled. */
int moe_forward_mx_profiled(const moe_dims* dims, const moe_weights* w, const moe_experts_mx* mx,
                            const uint16_t* x, uint16_t* out, void* ws, size_t ws_bytes, hipStream_t stream,
                            hipEvent_t* events, int n_events);

/* ---- the layer's neighbours: pre-norm, residual, bias update ------------ */

/* Pre-norm RMSNorm (the QA page, CH2 Q2.8): per row t of x,
 *   y[t] = bf16( gamma * bf16( x[t] * rsqrt(mean_k x[t,k]^2 + eps) ) )
 * x, y device [T, H] bf16; gamma device [H] bf16 (the learned weight). The
 * page upcasts to fp32; here the mean, the scale and both products are
 * float64 and each rounding is one round-to-nearest-even to bf16, so every
 * output is the unique value of the definition (torch's fp32 execution of the
 * page's code can differ on rare elements by one bf16 step). x, gamma and y
 * must be 16-byte aligned; y may equal x. MOE_ERR_INVALID for null or
 * misaligned pointers, T <= 0, H not a positive multiple of 8, or eps
 * negative / not finite. Asynchronous on `stream`. */
int moe_rmsnorm(const uint16_t* x, const uint16_t* gamma, int64_t T, int32_t H, float eps, uint16_t* y,
                hipStream_t stream);

/* Workspace of moe_block_forward: moe_workspace_bytes plus the normed rows
 * (T * H bf16). 0 for invalid dims. */
size_t moe_block_workspace_bytes(const moe_dims* dims);

/* The MoE block (the QA page, CH2 Q2.1 point 3: each mixer sits inside
 * Pre-Norm + Residual; the block sketch of the 2kiu.com hybrid Mamba/MoE
 * walkthrough: residual = x, x = norm(x), x = residual + MoE(x)):
 *   out = bf16( x + moe_forward(moe_rmsnorm(x, gamma, eps)) )
 * The norm writes the normed rows into the workspace (after the layer's own
 * scratch; its moe_ws_layout offsets are unchanged) and the residual add runs
 * in the epilogue of the final product: fc2 + shared down are rounded to bf16,
 * added to x in fp32 and rounded once more. mx: NULL for the bf16 experts of
 * `w`, else MX experts as for moe_forward_mx (T <= 64). out may equal x
 * (every element of x is read before the same element of out is written).
 * Errors as moe_forward, plus MOE_ERR_INVALID for a null or misaligned gamma
 * or x, or a bad eps; MOE_ERR_WORKSPACE below moe_block_workspace_bytes. */
int moe_block_forward(const moe_dims* dims, const moe_weights* w, const moe_experts_mx* mx, const uint16_t* gamma,
                      float eps, const uint16_t* x, uint16_t* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* Auxiliary-loss-free load balancing (the QA page, CH5 Q5.3): with load_i the
 * slots routed to expert i (offsets[i+1] - offsets[i]) and the mean load
 * offsets[E] / E,
 *   corr_bias[i] <- corr_bias[i] - eta * (load_i - mean load)
 * evaluated in float64 without fused multiply-adds and rounded once to fp32.
 * offsets device [E+1] int32: the expert offsets of moe_permute, or those a
 * forward left in its workspace (moe_ws_layout.offsets). corr_bias device [E]
 * fp32, updated in place. MOE_ERR_INVALID for null pointers, E <= 0 or a
 * non-finite eta. Asynchronous on `stream`. */
int moe_bias_update(const int32_t* offsets, int32_t E, float eta, float* corr_bias, hipStream_t stream);

/* ---- allocation-free forward ------------------------------------------ */

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation: moe_forward
 * with its workspace taken from a scratch array of the library's own instead of
 * the caller's. The array is a static device array of MOE_NOALLOC_SCRATCH_BYTES
 * (128 MiB); each GPU the library is loaded on holds its own copy until the
 * process ends. The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); its first call on a device looks the array's
 * address up once (hipGetSymbolAddress) and keeps it for that device.
 *   dims, w, x, out, stream: as for moe_forward (same results, bit for bit).
 * Returns MOE_ERR_TOO_LARGE, before any HIP call, when moe_workspace_bytes(dims)
 * exceeds MOE_NOALLOC_SCRATCH_BYTES (the Ultra-shape layer fits up to 64 tokens
 * at a time; larger batches take moe_forward with a caller workspace), the
 * errors of moe_forward otherwise, and MOE_ERR_HIP if the array's address
 * cannot be looked up. Every call on one GPU uses that GPU's one array, which
 * keeps the last call's intermediates: calls that overlap in time on one GPU
 * (two streams, two host threads) race and must be ordered by the caller.
 * Nothing in the array needs to start at zero. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int moe_forward_noalloc(const moe_dims* dims, const moe_weights* w, const uint16_t* x, uint16_t* out,
                        hipStream_t stream);

/* Human-readable text of a status code (static storage). */
const char* moe_status_string(int status);

/* Library ABI version (major*100 + minor). */
int moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_API_H */
