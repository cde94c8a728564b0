/*
 * q4moe — affine 4-bit mixture-of-experts feed-forward on AMD MI355X (gfx950).
 *
 * Weight format (lily README, introduction and "Requirements": MLX affine
 * 4-bit weights, group size 64).  A Q4 matrix of n rows and k columns is
 *   codes  uint32 [n][k/8]   eight 4-bit codes per word; column j of a row is
 *                             in word j/8 at bits [4*(j%8), 4*(j%8)+4)
 *   scales bf16   [n][k/64]  one scale per 64 consecutive columns of a row
 *   biases bf16   [n][k/64]  one bias per 64 consecutive columns of a row
 * and stands for w[r][j] = scale[r][j/64] * code[r][j] + bias[r][j/64].
 * All arrays are row-major and contiguous.  Stacked matrices (count > 1) are
 * laid out [count][n][...].  Activations are bfloat16 bit patterns.
 *
 * Conventions for every entry point:
 *  - Pointers named in the argument lists are DEVICE pointers owned by the
 *    caller, except the descriptor structs, which are host memory read during
 *    the call only.  The library allocates nothing and keeps no state between
 *    calls; scratch comes from the caller's workspace (size from
 *    q4moe_workspace_bytes, 256-byte aligned).
 *  - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream) and
 *    the call returns without synchronising.  Inputs must stay unmodified and
 *    the workspace untouched until the stream reaches the end of the call.
 *  - Arguments are validated on the host before any HIP call.  Invalid shapes,
 *    null pointers or misaligned buffers return Q4MOE_EINVAL (or
 *    Q4MOE_EUNSUPPORTED for valid shapes outside what the kernels handle) and
 *    enqueue nothing.  A HIP launch error returns Q4MOE_EHIP.  There is no
 *    fallback path.  No C++ exception crosses this interface.
 *  - Alignment: codes, activations and outputs 16-byte aligned; scale and bias
 *    arrays 2-byte aligned; workspaces 256-byte aligned.
 */
#ifndef Q4MOE_H
#define Q4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t q4moe_bf16;   /* raw bfloat16 bits */
typedef void* q4moe_stream;    /* hipStream_t */

enum {
  Q4MOE_OK = 0,
  Q4MOE_EINVAL = 1,        /* null pointer, bad shape, misaligned buffer */
  Q4MOE_EUNSUPPORTED = 2,  /* valid but outside the kernels' limits */
  Q4MOE_EWORKSPACE = 3,    /* workspace missing or smaller than required */
  Q4MOE_EHIP = 4           /* a HIP runtime or launch error */
};

/* Output forms.  Q4MOE_OUT_BF16_RESIDUAL is accepted by moe_ffn_decode only: it
 * writes bf16(x + y), the next layer's input on a residual stream. */
enum { Q4MOE_OUT_F32 = 0, Q4MOE_OUT_BF16 = 1, Q4MOE_OUT_BF16_RESIDUAL = 2 };

/* Operation ids for q4moe_workspace_bytes. */
enum {
  Q4MOE_OP_GEMV = 0,
  Q4MOE_OP_GEMM = 1,
  Q4MOE_OP_ROUTE = 2,
  Q4MOE_OP_PERMUTE = 3,
  Q4MOE_OP_FFN_DECODE = 4,
  Q4MOE_OP_FFN_PREFILL = 5,
  Q4MOE_OP_LMHEAD = 6,
  Q4MOE_OP_FFN_DECODE_BATCH = 7
};

/* An affine matrix of 4-bit codes (the default), or of 8-bit codes (the
 * checkpoint's 8-bit exceptions: "lily-qwen3.8-flash-next" README, "The model";
 * "2026-09-02: Lily vs MLX 0.32.2", "Hardware and software"), or `count` stacked
 * matrices of the same shape.  8-bit codes: uint32 [count][n][k/4], code j of a
 * row in byte j%4 of word j/4 (least significant first), same groups and
 * w = scale*q + bias.  q4_gemv and lmhead_argmax take 8-bit matrices, the layer
 * calls an 8-bit router (router_q8) and an 8-bit shared expert, and
 * moe_route_topk_q8 an 8-bit router; the other calls return Q4MOE_EUNSUPPORTED
 * for them.
 *
 * codes_gm (optional, 4-bit only): the same codes group-major, as written by
 * q4moe_pack_group_major: uint32 [count][k/64][n][8], the 32 code bytes of group
 * g of row r at word ((e*k/64 + g)*n + r)*8, so that a group's bytes of consecutive
 * rows are contiguous.  q4_gemm and moe_ffn_prefill read it for their grouped GEMMs
 * (the products, their order and the results are those of the `codes` form) when
 * every 4-bit matrix they multiply carries it; every other call reads `codes`.  It is
 * a layout of the prefill's own, next to the MLX layout that decode streams row by
 * row. */
typedef struct {
  const uint32_t* codes;
  const q4moe_bf16* scales;
  const q4moe_bf16* biases;
  int64_t count;  /* >= 1 */
  int64_t n;      /* rows per matrix */
  int64_t k;      /* columns, a multiple of 64 */
  int32_t bits;   /* code width: 4 (0 also means 4) or 8 */
  int32_t reserved;  /* 0 */
  const uint32_t* codes_gm;  /* null, or the group-major copy of codes (16-byte aligned) */
} q4moe_matrix;

/*
 * One MoE feed-forward layer.  Routed expert e has gate and up matrices of
 * `inter` rows by `hidden` columns and a down matrix of `hidden` rows by
 * `inter` columns (gate/up/down stacked with count = n_experts).  The shared
 * expert, when sh_gate.codes is non-null, has the same shapes with count 1
 * and is added with weight 1, or with weight sigmoid(sh_gate_w . x) when the
 * layer carries a shared-expert gate vector (Qwen-family MoE layers do).  The router is bf16 [n_experts][hidden], or, when
 * router_q8.codes is non-null, the 8-bit affine matrix router_q8 (count 1,
 * n_experts x hidden, bits 8: the benchmark checkpoint's affine Q8 router-gate
 * exceptions, "2026-09-02: Lily vs MLX 0.32.2", "Hardware and software"), and
 * `router` may be null.  moe_ffn_decode, moe_ffn_decode_batch and moe_ffn_prefill
 * all take an 8-bit router (the standalone router: moe_route_topk_q8).  The
 * shared expert's three matrices may be 8-bit together (the q4-xl conversion
 * keeps it at 8 bits: "lily-qwen3.8-flash-next" README, "The model"); the layer
 * calls take that form (a mix of 4- and 8-bit shared matrices is
 * Q4MOE_EUNSUPPORTED).  Routed experts are 4-bit.
 */
typedef struct {
  int32_t hidden;
  int32_t inter;
  int32_t n_experts;
  int32_t top_k;
  const q4moe_bf16* router;
  q4moe_matrix gate, up, down;
  q4moe_matrix sh_gate, sh_up, sh_down;
  q4moe_matrix router_q8;  /* codes null: the bf16 router is used */
  const q4moe_bf16* sh_gate_w;  /* null, or bf16 [hidden]: the shared expert is weighted by
                                   sigmoid(sh_gate_w . x) in every layer call */
} q4moe_layer;

/*
 * y = W x, one bf16 vector x[k] against every row of W (count*n rows), fp32
 * accumulation, y written as fp32 or bf16 [count*n].  The decode form of the
 * 4-bit weight stream (lily-qwen3.8-flash-next README, "How the speed was
 * achieved": decode reads every weight once and is bandwidth-bound).
 */
int q4_gemv(const q4moe_matrix* W, const q4moe_bf16* x, void* y, int out_dtype,
            q4moe_stream stream);

/*
 * Y[m][r] = sum_j X[m][j] W[r][j] for bf16 rows X[m][k], Y [m][count*n] fp32 or
 * bf16.  The prefill form, run on fp16 matrix cores (lily-qwen3.8-flash-next
 * README, "How the speed was achieved": prefill GEMMs on the tensor units):
 * each row of X is scaled by an exact power of two into fp16 (exact for bf16
 * values within 2^-23 of the row's largest), each scale*q is rounded once to
 * fp16 (at most 2^-12 relative), the bias term is exact up to fp32 summation,
 * and accumulation is fp32.  Scales must be below 64 in magnitude.  Needs
 * Q4MOE_OP_GEMM workspace (m).
 */
int q4_gemm(const q4moe_matrix* W, const q4moe_bf16* X, int64_t m, void* Y, int out_dtype,
            void* workspace, size_t workspace_bytes, q4moe_stream stream);

/*
 * Router of the mixture-of-experts layer (lily README, introduction: the
 * checkpoint is a 35B-A3B model, about 3B of its 35B parameters active per
 * token, which is a router picking a few experts per token; the pages give no
 * rule, and softmax -> top-k -> renormalise is the plain reading):
 * logits[t][e] = router[e] . X[t] (fp32 accumulation), softmax over
 * all n_experts, the top_k largest kept in descending order (equal logits:
 * lower expert id first), their probabilities renormalised to sum to 1.
 * Writes ids int32 [T][top_k] and weights fp32 [T][top_k].  1 <= top_k <= 32,
 * top_k <= n_experts <= 1024, hidden a multiple of 64.  Needs
 * Q4MOE_OP_ROUTE workspace (T).
 */
int moe_route_topk(const q4moe_bf16* router, int32_t n_experts, int32_t hidden,
                   const q4moe_bf16* X, int64_t T, int32_t top_k, int32_t* ids, float* weights,
                   void* workspace, size_t workspace_bytes, q4moe_stream stream);

/*
 * moe_route_topk with the benchmark checkpoint's affine-Q8 router gate
 * ("2026-09-02: Lily vs MLX 0.32.2", "Hardware and software": the Q4 checkpoint
 * keeps its router gates at 8 bits): router_q8 is an 8-bit matrix (bits 8,
 * count 1) of n = n_experts rows by k = hidden columns, its logits
 * logits[t][e] = sum_j (scale*q + bias)[e][j] X[t][j] in fp32, the rest as
 * moe_route_topk.  The same workspace (Q4MOE_OP_ROUTE with n_experts).
 */
int moe_route_topk_q8(const q4moe_matrix* router_q8, const q4moe_bf16* X, int64_t T, int32_t top_k,
                      int32_t* ids, float* weights, void* workspace, size_t workspace_bytes,
                      q4moe_stream stream);

/*
 * Stable counting sort of the T*top_k rows r = t*top_k + slot by expert id
 * (token-to-expert grouping for the prefill expert GEMM; lily-qwen3.8-flash-next
 * README, "How the speed was achieved").  Writes offsets int32 [n_experts+1]
 * (offsets[e]..offsets[e+1] is expert e's segment), sorted_rows int32 [T*top_k]
 * (rows of each segment in increasing r) and inv_rows int32 [T*top_k] with
 * inv_rows[sorted_rows[p]] = p.  ids must lie in [0, n_experts); an
 * out-of-range id is skipped by the kernels and leaves the outputs
 * inconsistent.  Needs Q4MOE_OP_PERMUTE workspace (T*top_k).
 */
int moe_permute(const int32_t* ids, int64_t T, int32_t top_k, int32_t n_experts,
                int32_t* offsets, int32_t* sorted_rows, int32_t* inv_rows,
                void* workspace, size_t workspace_bytes, q4moe_stream stream);

/*
 * One token through the MoE layer (batch-1 greedy decode step):
 *   y = sum_i w_i down_{e_i}(silu(gate_{e_i} x) * up_{e_i} x) + shared(x)
 * with (e_i, w_i) from the router as in moe_route_topk.  x bf16 [hidden]; y fp32
 * or bf16 [hidden], or with Q4MOE_OUT_BF16_RESIDUAL the bf16 rounding (nearest,
 * ties to even) of x + y computed in fp32, which is the next layer's input when
 * layers are chained through a residual stream (lily-qwen3.8-flash-next, "How
 * the speed was achieved": a decode step runs every layer on the GPU, so the
 * host is off the critical path); y must not overlap x (Q4MOE_EINVAL).  ids_out
 * int32 [top_k] and w_out fp32 [top_k] may be null.  Intermediates stay fp32.  Runs as one launch of one workgroup per compute
 * unit; values passed between workgroups carry a per-launch tag kept in the
 * workspace, so the Q4MOE_OP_FFN_DECODE workspace must be zero-filled before
 * its first use and must stay with one device; each call leaves it ready for
 * the next.  Calls that share a workspace must not overlap.  Every wait inside
 * the kernel is bounded (about a quarter second): if one ever gives up, the
 * result is wrong and the 32-bit word at byte offset 2048 of the workspace is
 * incremented (it stays 0 in correct use).
 */
int moe_ffn_decode(const q4moe_layer* layer, const q4moe_bf16* x, void* y, int out_dtype,
                   int32_t* ids_out, float* w_out, void* workspace, size_t workspace_bytes,
                   q4moe_stream stream);

/*
 * moe_ffn_decode for callers that cannot allocate: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same arguments, result
 * and kernels, without a workspace: the call uses a fixed scratch array of 1 MiB
 * inside the library (one per device, held until the process ends; zero at load,
 * and every call leaves it ready for the next).  The call allocates nothing.
 * Layers whose Q4MOE_OP_FFN_DECODE workspace would exceed 1 MiB return
 * Q4MOE_EUNSUPPORTED (no layer that moe_ffn_decode takes needs that much).  All calls on one device share the array: calls that
 * overlap on one device (on different streams without ordering) race and give
 * wrong results.  Its abandoned-wait counter is internal (use moe_ffn_decode to
 * read one).
 */
int moe_ffn_decode_noalloc(const q4moe_layer* layer, const q4moe_bf16* x, void* y, int out_dtype,
                           int32_t* ids_out, float* w_out, q4moe_stream stream);

/*
 * B tokens, one per request, through the MoE layer in one decode step
 * (lily-qwen3.8-flash-next, "Running it": up to four requests by default
 * decode together), 1 <= B <= 8: row b of Y equals moe_ffn_decode on X[b] up
 * to rounding (intermediates stay fp32).  X bf16 [B][hidden]; Y fp32 or bf16
 * [B][hidden]; ids_out int32 [B][top_k] and w_out fp32 [B][top_k] may be null.
 * Each expert chosen by any of the tokens is read once for all of them.  Runs
 * as two launches: one of one workgroup per compute unit (router, every
 * token's top-k, the step's expert plan, gate/up with SwiGLU), whose
 * workgroups pass the router logits to each other as tagged words as
 * moe_ffn_decode does, then the down projection with the weighted sum.  B = 1
 * runs moe_ffn_decode's single launch when it applies (y not overlapping x,
 * and a workspace as large as Q4MOE_OP_FFN_DECODE needs: the
 * Q4MOE_OP_FFN_DECODE_BATCH size for one row includes it).  The
 * Q4MOE_OP_FFN_DECODE_BATCH workspace (B) must be zero-filled before its
 * first use and stay with one device; each call leaves it ready for the next,
 * and calls that share a workspace must not overlap.  Waits are bounded as in
 * moe_ffn_decode (the same counter at byte offset 2048).  Q4MOE_EUNSUPPORTED:
 * shapes whose staged vectors exceed 64 KB of LDS (B * hidden * 21 / 8 bytes
 * of inputs, or (top_k + 1) * inter * 37 / 8 bytes of SwiGLU outputs for one
 * token), or a device on which one front workgroup per compute unit cannot be
 * resident at once.
 */
int moe_ffn_decode_batch(const q4moe_layer* layer, const q4moe_bf16* X, int64_t B, void* Y,
                         int out_dtype, int32_t* ids_out, float* w_out, void* workspace,
                         size_t workspace_bytes, q4moe_stream stream);

/*
 * T tokens through the MoE layer (a prefill chunk, 2,048 tokens in the
 * "Measurement contract" of "2026-09-02: Lily vs MLX 0.32.2"): route, permute
 * by expert, grouped fp16-MFMA GEMMs (as q4_gemm) for gate/up with SwiGLU and
 * for down with the routing weight, then combine back in token order.  Row t
 * of Y equals moe_ffn_decode on X[t] up to rounding; the SwiGLU output is
 * computed in fp32 and rounded once to fp16 (after an exact power-of-two row
 * scaling; a value that lands below fp16's normal range there, under 2^-22 of
 * its row's largest, may round twice) before the down GEMM, and each expert's
 * weighted output is rounded
 * once to fp16 precision (11 significant bits, kept in range by a power of two
 * per four columns) before the combine adds them in fp32.  The GEMMs read the experts' group-major
 * codes when every 4-bit expert matrix of the layer (routed and shared) carries
 * them (q4moe_matrix.codes_gm; the results are the same bits either way).
 * Y fp32 or bf16 [T][hidden].  Needs Q4MOE_OP_FFN_PREFILL workspace (T).
 */
int moe_ffn_prefill(const q4moe_layer* layer, const q4moe_bf16* X, int64_t T, void* Y,
                    int out_dtype, void* workspace, size_t workspace_bytes, q4moe_stream stream);

/*
 * Greedy LM head: logits[b][r] = W[r] . X[b] in fp32 for b < B (1 <= B <= 8),
 * ids[b] = the lowest index of the largest logit (Lily decodes greedily: lily
 * README, introduction).  max_logit fp32 [B] may be null.  Needs
 * Q4MOE_OP_LMHEAD workspace (B), zero-filled before its first use: the call
 * keeps an arrival count of its workgroups and one running 64-bit maximum per
 * batch row there (the last workgroup to arrive reads them) and leaves both at
 * zero again, so calls that share a workspace must not overlap.
 */
int lmhead_argmax(const q4moe_matrix* W, const q4moe_bf16* X, int64_t B, int32_t* ids,
                  float* max_logit, void* workspace, size_t workspace_bytes, q4moe_stream stream);

/*
 * Write the group-major copy of a 4-bit matrix's codes (see q4moe_matrix) to dst:
 * uint32 [count][k/64][n][8] (count*n*k/8 words, 16-byte aligned, device memory the
 * caller owns; it must not overlap W->codes).  A layout step for prefill, done once per
 * matrix (when weights are loaded), not per call.  W must be 4-bit (8-bit:
 * Q4MOE_EUNSUPPORTED); W->codes_gm is ignored.  Asynchronous on `stream`.
 */
int q4moe_pack_group_major(const q4moe_matrix* W, uint32_t* dst, q4moe_stream stream);

/*
 * Workspace bytes for an operation.  `layer` is read for the FFN and ROUTE
 * ops (ROUTE uses layer->n_experts), `W` for GEMM and LMHEAD; `rows` is T, m
 * or B.  Returns 0 when no workspace is needed or the arguments are invalid.
 */
size_t q4moe_workspace_bytes(int op, const q4moe_layer* layer, const q4moe_matrix* W, int64_t rows);

/* Static text for a status code. */
const char* q4moe_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* Q4MOE_H */
