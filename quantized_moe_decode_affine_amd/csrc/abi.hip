// C ABI of libq4moe: argument validation (host only, before any HIP call)
// and dispatch to the kernel launchers.  Declarations and the contract of
// every entry point are in include/q4moe.h.
#include "../../include/q4moe.h"
#include "kernels.h"

#include <algorithm>
#include <new>

namespace q4moe {

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cached[dev] = cus;
  }
  return cached[dev];
}

}  // namespace q4moe

namespace {

using q4moe::Q4Mat;

constexpr int64_t kMaxRows32 = 0x7FFFFFFF;
constexpr int kMaxGemvK = 16384;
constexpr size_t kMaxDynLds = 64 * 1024;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool matrix_ok(const q4moe_matrix* W) {
  if (!W || !W->codes || !W->scales || !W->biases) return false;
  if (W->bits != 0 && W->bits != 4 && W->bits != 8) return false;
  if (W->count < 1 || W->n < 1 || W->k < 64 || W->k % 64) return false;
  if (!aligned(W->codes, 16) || !aligned(W->scales, 2) || !aligned(W->biases, 2)) return false;
  if (W->codes_gm && (W->bits == 8 || !aligned(W->codes_gm, 16))) return false;
  return true;
}

bool matrix_shape(const q4moe_matrix& W, int64_t count, int64_t n, int64_t k) {
  return matrix_ok(&W) && W.count == count && W.n == n && W.k == k;
}

Q4Mat to_mat(const q4moe_matrix& W) { return Q4Mat{W.codes, W.scales, W.biases, W.codes_gm}; }

bool is_q8(const q4moe_matrix& W) { return W.bits == 8; }

bool out_ok(const void* y, int out_dtype) {
  return y && aligned(y, 16) && (out_dtype == Q4MOE_OUT_F32 || out_dtype == Q4MOE_OUT_BF16);
}

// Validates a layer; on success fills `d`.
int layer_check(const q4moe_layer* L, q4moe::DecodeLayer* d) {
  if (!L) return Q4MOE_EINVAL;
  const bool rq8 = L->router_q8.codes != nullptr;
  if (!rq8 && (!L->router || !aligned(L->router, 16))) return Q4MOE_EINVAL;
  if (L->hidden < 64 || L->hidden % 64 || L->inter < 64 || L->inter % 64) return Q4MOE_EINVAL;
  if (L->n_experts < 1 || L->top_k < 1 || L->top_k > L->n_experts) return Q4MOE_EINVAL;
  if (L->n_experts > 1024 || L->top_k > 32 || L->hidden > kMaxGemvK) return Q4MOE_EUNSUPPORTED;
  const int64_t E = L->n_experts, H = L->hidden, I = L->inter;
  if (!matrix_shape(L->gate, E, I, H) || !matrix_shape(L->up, E, I, H) || !matrix_shape(L->down, E, H, I))
    return Q4MOE_EINVAL;
  const bool shared = L->sh_gate.codes != nullptr;
  if (shared && (!matrix_shape(L->sh_gate, 1, I, H) || !matrix_shape(L->sh_up, 1, I, H) ||
                 !matrix_shape(L->sh_down, 1, H, I)))
    return Q4MOE_EINVAL;
  for (const q4moe_matrix* m : {&L->gate, &L->up, &L->down})
    if (is_q8(*m)) return Q4MOE_EUNSUPPORTED;  // routed experts: 4-bit codes only
  // the shared expert: all three matrices 4-bit, or all three 8-bit (batch-1 decode only)
  const bool sh_q8 = shared && is_q8(L->sh_gate);
  if (shared && (is_q8(L->sh_up) != sh_q8 || is_q8(L->sh_down) != sh_q8)) return Q4MOE_EUNSUPPORTED;
  if (rq8 && (!matrix_shape(L->router_q8, 1, E, H) || !is_q8(L->router_q8))) return Q4MOE_EINVAL;
  d->hidden = L->hidden;
  d->inter = L->inter;
  d->n_experts = L->n_experts;
  d->top_k = L->top_k;
  d->has_shared = shared ? 1 : 0;
  d->router = L->router;
  d->gate = to_mat(L->gate);
  d->up = to_mat(L->up);
  d->down = to_mat(L->down);
  if (shared) {
    d->sh_gate = to_mat(L->sh_gate);
    d->sh_up = to_mat(L->sh_up);
    d->sh_down = to_mat(L->sh_down);
  } else {
    d->sh_gate = d->sh_up = d->sh_down = Q4Mat{nullptr, nullptr, nullptr};
  }
  d->router_q8 = rq8 ? to_mat(L->router_q8) : Q4Mat{nullptr, nullptr, nullptr};
  if (L->sh_gate_w && (!shared || !aligned(L->sh_gate_w, 16))) return Q4MOE_EINVAL;
  d->sh_gate_w = L->sh_gate_w;
  d->sh_q8 = sh_q8 ? 1 : 0;
  return Q4MOE_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? Q4MOE_OK : Q4MOE_EHIP; }

size_t lmhead_ws(int64_t rows, int64_t k, int64_t B) {
  (void)rows;
  (void)k;
  return 256 + (size_t)B * 8;  // arrival counter, then one 64-bit running maximum per batch row
}

}  // namespace

extern "C" {

const char* q4moe_strerror(int status) {
  switch (status) {
    case Q4MOE_OK: return "ok";
    case Q4MOE_EINVAL: return "invalid argument (null pointer, bad shape or misaligned buffer)";
    case Q4MOE_EUNSUPPORTED: return "shape outside the kernels' supported limits";
    case Q4MOE_EWORKSPACE: return "workspace missing or too small";
    case Q4MOE_EHIP: return "HIP runtime or launch error";
    default: return "unknown status";
  }
}

size_t q4moe_workspace_bytes(int op, const q4moe_layer* layer, const q4moe_matrix* W, int64_t rows) {
  if (rows < 0) return 0;
  switch (op) {
    case Q4MOE_OP_GEMV: return 0;
    case Q4MOE_OP_GEMM:
      if (!W || W->k < 64 || W->k % 64) return 0;
      return q4moe::gemm_workspace_bytes(rows, (int)W->k);
    case Q4MOE_OP_ROUTE:
      if (!layer || layer->n_experts < 1) return 0;
      return q4moe::route_workspace_bytes(rows, layer->n_experts);
    case Q4MOE_OP_PERMUTE:
      if (!layer || layer->n_experts < 1 || layer->top_k < 1) return 0;
      return q4moe::permute_workspace_bytes(rows * layer->top_k, layer->n_experts);
    case Q4MOE_OP_FFN_DECODE: {
      q4moe::DecodeLayer d;
      if (layer_check(layer, &d) != Q4MOE_OK) return 0;
      return q4moe::decode_workspace_bytes(d.hidden, d.inter, d.n_experts, d.top_k);
    }
    case Q4MOE_OP_FFN_PREFILL: {
      q4moe::DecodeLayer d;
      if (layer_check(layer, &d) != Q4MOE_OK) return 0;
      return q4moe::prefill_workspace_bytes(rows, d.hidden, d.inter, d.n_experts, d.top_k, d.has_shared);
    }
    case Q4MOE_OP_FFN_DECODE_BATCH: {
      q4moe::DecodeLayer d;
      if (layer_check(layer, &d) != Q4MOE_OK || rows < 1 || rows > q4moe::kMaxBatch) return 0;
      const size_t nb = q4moe::decode_batch_workspace_bytes(d.n_experts, d.top_k, d.inter, (int)rows);
      // one row runs the batch-1 layer kernel when it applies: room for its workspace too
      return rows == 1 ? std::max(nb, q4moe::decode_workspace_bytes(d.hidden, d.inter, d.n_experts, d.top_k)) : nb;
    }
    case Q4MOE_OP_LMHEAD:
      if (!W) return 0;
      return lmhead_ws(W->count * W->n, W->k, rows);
    default: return 0;
  }
}

int q4_gemv(const q4moe_matrix* W, const q4moe_bf16* x, void* y, int out_dtype, q4moe_stream stream) {
  try {
    if (!matrix_ok(W) || !x || !aligned(x, 16) || !out_ok(y, out_dtype)) return Q4MOE_EINVAL;
    if (W->k > kMaxGemvK) return Q4MOE_EUNSUPPORTED;
    const int64_t rows = W->count * W->n;
    if (is_q8(*W)) {
      if (q4moe::q8_gemv_lds_bytes((int)W->k, 1) > kMaxDynLds) return Q4MOE_EUNSUPPORTED;
      return hip_status(q4moe::run_q8_gemv(W->codes, W->scales, W->biases, rows, (int)W->k, x, y,
                                           out_dtype == Q4MOE_OUT_BF16, (hipStream_t)stream));
    }
    return hip_status(q4moe::run_q4_gemv(W->codes, W->scales, W->biases, rows, (int)W->k, x, y,
                                         out_dtype == Q4MOE_OUT_BF16, (hipStream_t)stream));
  } catch (...) {
    return Q4MOE_EHIP;
  }
}

int q4_gemm(const q4moe_matrix* W, const q4moe_bf16* X, int64_t m, void* Y, int out_dtype, void* workspace,
            size_t workspace_bytes, q4moe_stream stream) {
  try {
    if (!matrix_ok(W) || !X || !aligned(X, 16) || m < 0 || !out_ok(Y, out_dtype)) return Q4MOE_EINVAL;
    const int64_t n = W->count * W->n;
    if (n > kMaxRows32 || m > kMaxRows32 || is_q8(*W)) return Q4MOE_EUNSUPPORTED;
    if (m == 0) return Q4MOE_OK;
    const size_t need = q4moe::gemm_workspace_bytes(m, (int)W->k);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return Q4MOE_EWORKSPACE;
    Q4Mat w = to_mat(*W);
    if (W->count != 1) w.codes_gm = nullptr;  // the group-major form is per matrix; a stack is read row-major
    return hip_status(q4moe::run_q4_gemm(w, n, (int)W->k, X, m, Y, out_dtype == Q4MOE_OUT_BF16, workspace,
                                         (hipStream_t)stream));
  } catch (...) {
    return Q4MOE_EHIP;
  }
}

int moe_route_topk(const q4moe_bf16* router, int32_t n_experts, int32_t hidden, const q4moe_bf16* X, int64_t T,
                   int32_t top_k, int32_t* ids, float* weights, void* workspace, size_t workspace_bytes,
                   q4moe_stream stream) {
  try {
    if (!router || !aligned(router, 16) || !X || !aligned(X, 16) || !ids || !weights || T < 0) return Q4MOE_EINVAL;
    if (hidden < 64 || hidden % 64 || n_experts < 1 || top_k < 1 || top_k > n_experts) return Q4MOE_EINVAL;
    if (n_experts > 1024 || top_k > 32 || T * top_k > kMaxRows32) return Q4MOE_EUNSUPPORTED;
    if (T == 0) return Q4MOE_OK;
    if (!workspace || workspace_bytes < q4moe::route_workspace_bytes(T, n_experts) || !aligned(workspace, 256))
      return Q4MOE_EWORKSPACE;
    return hip_status(q4moe::run_route_topk(router, n_experts, hidden, X, T, top_k, ids, weights, workspace,
                                            (hipStream_t)stream));
  } catch (...) {
    return Q4MOE_EHIP;
  }
}

int moe_route_topk_q8(const q4moe_matrix* router_q8, const q4moe_bf16* X, int64_t T, int32_t top_k, int32_t* ids,
                      float* weights, void* workspace, size_t workspace_bytes, q4moe_stream stream) {
  try {
    if (!matrix_ok(router_q8) || !is_q8(*router_q8) || router_q8->count != 1) return Q4MOE_EINVAL;
    if (!X || !aligned(X, 16) || !ids || !weights || T < 0) return Q4MOE_EINVAL;
    const int64_t E = router_q8->n, H = router_q8->k;
    if (top_k < 1 || top_k > E) return Q4MOE_EINVAL;
    if (E > 1024 || top_k > 32 || H > kMaxGemvK || T * top_k > kMaxRows32) return Q4MOE_EUNSUPPORTED;
    if (T == 0) return Q4MOE_OK;
    if (!workspace || workspace_bytes < q4moe::route_workspace_bytes(T, (int)E) || !aligned(workspace, 256))
      return Q4MOE_EWORKSPACE;
    const Q4Mat m = to_mat(*router_q8);
    return hip_status(q4moe::run_route_topk(nullptr, (int)E, (int)H, X, T, top_k, ids, weights, workspace,
                                            (hipStream_t)stream, &m));
  } catch (...) {
    return Q4MOE_EHIP;
  }
}

int moe_permute(const int32_t* ids, int64_t T, int32_t top_k, int32_t n_experts, int32_t* offsets,
                int32_t* sorted_rows, int32_t* inv_rows, void* workspace, size_t workspace_bytes,
                q4moe_stream stream) {
  try {
    if (!ids || !offsets || !sorted_rows || !inv_rows || T < 0 || top_k < 1 || n_experts < 1) return Q4MOE_EINVAL;
    if (n_experts > 1024 || T * top_k > kMaxRows32) return Q4MOE_EUNSUPPORTED;
    const int64_t rows = T * top_k;
    if (!workspace || workspace_bytes < q4moe::permute_workspace_bytes(rows, n_experts) || !aligned(workspace, 256))
      return Q4MOE_EWORKSPACE;
    return hip_status(q4moe::run_permute(ids, rows, n_experts, offsets, sorted_rows, inv_rows, workspace, nullptr,
                                         (hipStream_t)stream));
  } catch (...) {
    return Q4MOE_EHIP;
  }
}

int moe_ffn_decode(const q4moe_layer* layer, const q4moe_bf16* x, void* y, int out_dtype, int32_t* ids_out,
                   float* w_out, void* workspace, size_t workspace_bytes, q4moe_stream stream) {
  try {
    q4moe::DecodeLayer d;
    const int st = layer_check(layer, &d);
    if (st != Q4MOE_OK) return st;
    const bool residual = out_dtype == Q4MOE_OUT_BF16_RESIDUAL;
    if (!x || !aligned(x, 16) || !(residual ? y && aligned(y, 16) : out_ok(y, out_dtype))) return Q4MOE_EINVAL;
    {  // y must not overlap x: the kernel still reads x while other workgroups write y
      const uintptr_t xb = reinterpret_cast<uintptr_t>(x), yb = reinterpret_cast<uintptr_t>(y);
      const uintptr_t xe = xb + (uintptr_t)d.hidden * 2, ye = yb + (uintptr_t)d.hidden * (out_dtype == Q4MOE_OUT_F32 ? 4 : 2);
      if (xb < ye && yb < xe) return Q4MOE_EINVAL;
    }
    if (q4moe::decode_lds_bytes(d) > kMaxDynLds) return Q4MOE_EUNSUPPORTED;
    const size_t need = q4moe::decode_workspace_bytes(d.hidden, d.inter, d.n_experts, d.top_k);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return Q4MOE_EWORKSPACE;
    // all workgroups must be resident together (they wait on each other's words)
    if (!q4moe::decode_fits(d)) return Q4MOE_EUNSUPPORTED;
    const int mode = residual ? q4moe::kOutBf16Residual : out_dtype == Q4MOE_OUT_BF16 ? q4moe::kOutBf16 : q4moe::kOutF32;
    return hip_status(q4moe::run_moe_ffn_decode(d, x, y, mode, ids_out, w_out, workspace, (hipStream_t)stream));
  } catch (...) {
    return Q4MOE_EHIP;
  }
}

int moe_ffn_decode_noalloc(const q4moe_layer* layer, const q4moe_bf16* x, void* y, int out_dtype, int32_t* ids_out,
                           float* w_out, q4moe_stream stream) {
  try {
    q4moe::DecodeLayer d;
    const int st = layer_check(layer, &d);
    if (st != Q4MOE_OK) return st;
    const bool residual = out_dtype == Q4MOE_OUT_BF16_RESIDUAL;
    if (!x || !aligned(x, 16) || !(residual ? y && aligned(y, 16) : out_ok(y, out_dtype))) return Q4MOE_EINVAL;
    {  // y must not overlap x
      const uintptr_t xb = reinterpret_cast<uintptr_t>(x), yb = reinterpret_cast<uintptr_t>(y);
      const uintptr_t xe = xb + (uintptr_t)d.hidden * 2, ye = yb + (uintptr_t)d.hidden * (out_dtype == Q4MOE_OUT_F32 ? 4 : 2);
      if (xb < ye && yb < xe) return Q4MOE_EINVAL;
    }
    if (q4moe::decode_lds_bytes(d) > kMaxDynLds) return Q4MOE_EUNSUPPORTED;
    // the layer's workspace must fit the fixed scratch array
    if (q4moe::decode_workspace_bytes(d.hidden, d.inter, d.n_experts, d.top_k) > q4moe::kNoAllocScratchBytes)
      return Q4MOE_EUNSUPPORTED;
    if (!q4moe::decode_fits(d)) return Q4MOE_EUNSUPPORTED;
    void* scratch = nullptr;
    if (q4moe::noalloc_scratch(&scratch) != hipSuccess) return Q4MOE_EHIP;
    const int mode = residual ? q4moe::kOutBf16Residual : out_dtype == Q4MOE_OUT_BF16 ? q4moe::kOutBf16 : q4moe::kOutF32;
    return hip_status(q4moe::run_moe_ffn_decode(d, x, y, mode, ids_out, w_out, scratch, (hipStream_t)stream));
  } catch (...) {
    return Q4MOE_EHIP;
  }
}

int moe_ffn_decode_batch(const q4moe_layer* layer, const q4moe_bf16* X, int64_t B, void* Y, int out_dtype,
                         int32_t* ids_out, float* w_out, void* workspace, size_t workspace_bytes,
                         q4moe_stream stream) {
  try {
    q4moe::DecodeLayer d;
    const int st = layer_check(layer, &d);
    if (st != Q4MOE_OK) return st;
    if (!X || !aligned(X, 16) || B < 1 || !out_ok(Y, out_dtype)) return Q4MOE_EINVAL;
    if (B > q4moe::kMaxBatch || !q4moe::decode_batch_supported(d, (int)B, kMaxDynLds)) return Q4MOE_EUNSUPPORTED;
    const size_t need = q4moe::decode_batch_workspace_bytes(d.n_experts, d.top_k, d.inter, (int)B);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return Q4MOE_EWORKSPACE;
    if (B == 1) {  // one token: the batch-1 layer kernel when it applies (one launch instead of two)
      const uintptr_t xb = reinterpret_cast<uintptr_t>(X), yb = reinterpret_cast<uintptr_t>(Y);
      const uintptr_t xe = xb + (uintptr_t)d.hidden * 2, ye = yb + (uintptr_t)d.hidden * (out_dtype == Q4MOE_OUT_F32 ? 4 : 2);
      if (!(xb < ye && yb < xe) && q4moe::decode_lds_bytes(d) <= kMaxDynLds &&
          workspace_bytes >= q4moe::decode_workspace_bytes(d.hidden, d.inter, d.n_experts, d.top_k) &&
          q4moe::decode_fits(d))
        return hip_status(q4moe::run_moe_ffn_decode(d, X, Y, out_dtype == Q4MOE_OUT_BF16 ? q4moe::kOutBf16 : q4moe::kOutF32,
                                                    ids_out, w_out, workspace, (hipStream_t)stream));
    }
    // the front launch's workgroups wait on each other: all must be resident together
    if (!q4moe::decode_batch_fits(d, (int)B)) return Q4MOE_EUNSUPPORTED;
    return hip_status(q4moe::run_moe_ffn_decode_batch(d, X, (int)B, Y, out_dtype == Q4MOE_OUT_BF16, ids_out, w_out,
                                                      workspace, kMaxDynLds, (hipStream_t)stream));
  } catch (...) {
    return Q4MOE_EHIP;
  }
}

int moe_ffn_prefill(const q4moe_layer* layer, const q4moe_bf16* X, int64_t T, void* Y, int out_dtype,
                    void* workspace, size_t workspace_bytes, q4moe_stream stream) {
  try {
    q4moe::DecodeLayer d;
    const int st = layer_check(layer, &d);
    if (st != Q4MOE_OK) return st;
    if (!X || !aligned(X, 16) || T < 0 || !out_ok(Y, out_dtype)) return Q4MOE_EINVAL;
    if (T * (d.top_k + 1) > kMaxRows32) return Q4MOE_EUNSUPPORTED;
    if (T == 0) return Q4MOE_OK;
    const size_t need =
        q4moe::prefill_workspace_bytes(T, d.hidden, d.inter, d.n_experts, d.top_k, d.has_shared);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return Q4MOE_EWORKSPACE;
    return hip_status(
        q4moe::run_moe_ffn_prefill(d, X, T, Y, out_dtype == Q4MOE_OUT_BF16, workspace, (hipStream_t)stream));
  } catch (...) {
    return Q4MOE_EHIP;
  }
}

int lmhead_argmax(const q4moe_matrix* W, const q4moe_bf16* X, int64_t B, int32_t* ids, float* max_logit,
                  void* workspace, size_t workspace_bytes, q4moe_stream stream) {
  try {
    if (!matrix_ok(W) || !X || !aligned(X, 16) || !ids || B < 1) return Q4MOE_EINVAL;
    const int64_t rows = W->count * W->n;
    if (B > 8 || rows > kMaxRows32 || B * W->k > kMaxGemvK) return Q4MOE_EUNSUPPORTED;
    if (is_q8(*W) && B == 1 && q4moe::q8_gemv_lds_bytes((int)W->k, 1) > kMaxDynLds)  // B >= 2: the MFMA head
      return Q4MOE_EUNSUPPORTED;
    const size_t need = lmhead_ws(rows, W->k, B);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return Q4MOE_EWORKSPACE;
    char* w = static_cast<char*>(workspace);
    unsigned* done = reinterpret_cast<unsigned*>(w);
    unsigned long long* keys = reinterpret_cast<unsigned long long*>(w + 256);
    if (is_q8(*W))
      return hip_status(q4moe::run_lmhead_argmax_q8(W->codes, W->scales, W->biases, rows, (int)W->k, X, (int)B,
                                                    ids, max_logit, keys, done, (hipStream_t)stream));
    return hip_status(q4moe::run_lmhead_argmax(W->codes, W->scales, W->biases, rows, (int)W->k, X, (int)B, ids,
                                               max_logit, keys, done, (hipStream_t)stream));
  } catch (...) {
    return Q4MOE_EHIP;
  }
}

int q4moe_pack_group_major(const q4moe_matrix* W, uint32_t* dst, q4moe_stream stream) {
  try {
    if (!W || !dst || !aligned(dst, 16)) return Q4MOE_EINVAL;
    q4moe_matrix m = *W;
    m.codes_gm = nullptr;  // not read here
    if (!matrix_ok(&m)) return Q4MOE_EINVAL;
    if (is_q8(m)) return Q4MOE_EUNSUPPORTED;
    const uintptr_t bytes = (uintptr_t)(m.count * m.n * (m.k / 8)) * 4;
    const uintptr_t a = reinterpret_cast<uintptr_t>(m.codes), b = reinterpret_cast<uintptr_t>(dst);
    if (a < b + bytes && b < a + bytes) return Q4MOE_EINVAL;  // overlapping copies
    return hip_status(q4moe::run_pack_group_major(m.codes, m.count, m.n, (int)m.k, dst, (hipStream_t)stream));
  } catch (...) {
    return Q4MOE_EHIP;
  }
}

}  // extern "C"
