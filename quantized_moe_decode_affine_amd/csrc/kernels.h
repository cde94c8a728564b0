// Internal launchers behind the C ABI (abi.cpp validates every argument
// before calling any of these).  All launch on the given stream and return
// the HIP status of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace q4moe {

// Number of compute units of the current device (cached per device).
int device_cu_count();

// ---- GEMV family (gemv.hip)
size_t gemv_lds_bytes(int k, int B);
// The GEMV family launches at most this many workgroups (one resident round).
constexpr int kMaxGemvBlocks = 2048;
hipError_t run_q4_gemv(const uint32_t* codes, const uint16_t* scales, const uint16_t* biases, int64_t rows,
                       int k, const uint16_t* x, void* y, int out_bf16, hipStream_t stream);
hipError_t run_lmhead_argmax(const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                             int64_t rows, int k, const uint16_t* X, int B, int32_t* ids, float* max_logit,
                             unsigned long long* keys, unsigned* done, hipStream_t stream);

// The same for 8-bit codes (4 per word): B = 1 runs the GEMV form (LDS per call from
// q8_gemv_lds_bytes), B = 2..8 the matrix-core LM head (LDS per call from gemv_lds_bytes).
size_t q8_gemv_lds_bytes(int k, int B);
hipError_t run_q8_gemv(const uint32_t* codes, const uint16_t* scales, const uint16_t* biases, int64_t rows,
                       int k, const uint16_t* x, void* y, int out_bf16, hipStream_t stream);
hipError_t run_lmhead_argmax_q8(const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                                int64_t rows, int k, const uint16_t* X, int B, int32_t* ids, float* max_logit,
                                unsigned long long* keys, unsigned* done, hipStream_t stream);

// ---- Q4 matrices as seen by the kernels
struct Q4Mat {
  const uint32_t* codes;   // [count][n][k/8]
  const uint16_t* scales;  // [count][n][k/64]
  const uint16_t* biases;
  const uint32_t* codes_gm = nullptr;  // null, or the codes group-major: [count][k/64][n][8]
};

// ---- decode MoE layer (decode.hip)
struct DecodeLayer {
  int hidden, inter, n_experts, top_k, has_shared;
  const uint16_t* router;                // [E][H]
  Q4Mat gate, up, down;                  // routed, stacked by expert
  Q4Mat sh_gate, sh_up, sh_down;         // shared (count 1) when has_shared
  Q4Mat router_q8;                       // 8-bit router [E][H/4] words, or codes null (bf16 router)
  const uint16_t* sh_gate_w;             // null, or bf16 [H]: shared expert weighted by sigmoid(w . x)
  int sh_q8;                             // shared expert in 8-bit codes ([.][H/4] or [.][I/4] words)
};
size_t decode_workspace_bytes(int hidden, int inter, int n_experts, int top_k);
size_t decode_lds_bytes(const DecodeLayer& L);
// True when one decode workgroup fits on every CU at once (its waits need them all resident).
bool decode_fits(const DecodeLayer& L);
// Output forms of the decode layer: fp32, bf16, or bf16(x + y) (the next layer's input).
enum { kOutF32 = 0, kOutBf16 = 1, kOutBf16Residual = 2 };
hipError_t run_moe_ffn_decode(const DecodeLayer& L, const uint16_t* x, void* y, int out_mode, int32_t* ids_out,
                              float* w_out, void* ws, hipStream_t stream);
// The no-allocation decode form's scratch: a file-scope device array of this many
// bytes; *out receives its address on the current device (taken once per device).
constexpr size_t kNoAllocScratchBytes = size_t(1) << 20;  // more than any layer the decode kernel takes needs (its LDS bounds the slots x intermediate)
constexpr int kMaxDevices = 64;
hipError_t noalloc_scratch(void** out);

// ---- batched decode, 1..kMaxBatch tokens (decode_batch.hip)
constexpr int kMaxBatch = 8;
size_t decode_batch_workspace_bytes(int n_experts, int top_k, int inter, int B);
bool decode_batch_supported(const DecodeLayer& L, int B, size_t max_lds);
// True when one front workgroup of the batched step fits on every CU at once.
bool decode_batch_fits(const DecodeLayer& L, int B);
hipError_t run_moe_ffn_decode_batch(const DecodeLayer& L, const uint16_t* X, int B, void* y, int out_bf16,
                                    int32_t* ids_out, float* w_out, void* ws, size_t max_lds, hipStream_t stream);

// ---- routing and permutation (route.hip)
size_t route_workspace_bytes(int64_t T, int n_experts);
// router_q8 (optional): an 8-bit affine router used in place of the bf16 one.
hipError_t run_route_topk(const uint16_t* router, int E, int H, const uint16_t* X, int64_t T, int k,
                          int32_t* ids, float* weights, void* ws, hipStream_t stream,
                          const Q4Mat* router_q8 = nullptr);
size_t permute_workspace_bytes(int64_t rows, int n_experts);

// Optional output of run_permute for the grouped GEMM: the sorted positions cut
// into tiles of tile_rows rows (never crossing a segment), then extra_rows more
// positions (the shared expert's rows, after the routed ones) cut the same way.
struct GroupTiles {
  int tile_rows;
  int max_tiles;          // table length: at least rows / tile_rows + n_experts + extra tiles
  int64_t extra_rows;
  int topk;               // row r = t * topk + slot belongs to token t
  const float* weights;   // routing weight of each row r (may be null: weight 1)
  int4* table;            // [max_tiles] {segment (expert; -1 extra; -2 unused), first position, rows, 0}
  int32_t* row_src;       // [rows] token of each sorted position
  float* row_w;           // [rows] routing weight of each sorted position
};
int group_max_tiles(int64_t rows, int n_experts, int64_t extra_rows, int tile_rows);

// fp16 preparation of bf16 rows for the grouped GEMM (power-of-two exponents, pair-order
// fp16 copy, two-part group sums), run by extra workgroups of the sort's rank launch.
struct PrepRowsJob {
  const uint16_t* A;  // bf16 [rows][K]
  int64_t rows;
  int K, Gp;
  uint16_t* out;      // fp16 [rows][K]
  uint16_t* sums;     // fp16 [rows][2][Gp]
  int32_t* exps;      // [rows]
};

// Stable counting sort of `rows` ids by expert (tiles may be null); prep (optional)
// prepares rows beside the rank step, in the same launch.
hipError_t run_permute(const int32_t* ids, int64_t rows, int n_experts, int32_t* offsets, int32_t* sorted_rows,
                       int32_t* inv_rows, void* ws, const GroupTiles* tiles, hipStream_t stream,
                       const PrepRowsJob* prep = nullptr);

// ---- grouped MFMA GEMM and the prefill layer (gemm.hip)
size_t gemm_workspace_bytes(int64_t m, int k);
hipError_t run_q4_gemm(const Q4Mat& W, int64_t n, int k, const uint16_t* X, int64_t m, void* Y, int out_bf16,
                       void* ws, hipStream_t stream);
// Group-major copy of a stack of 4-bit matrices' codes (Q4Mat::codes_gm layout).
hipError_t run_pack_group_major(const uint32_t* codes, int64_t count, int64_t n, int k, uint32_t* dst,
                                hipStream_t stream);
size_t prefill_workspace_bytes(int64_t T, int hidden, int inter, int n_experts, int top_k, int has_shared);
hipError_t run_moe_ffn_prefill(const DecodeLayer& L, const uint16_t* X, int64_t T, void* Y, int out_bf16,
                               void* ws, hipStream_t stream);

}  // namespace q4moe
