// Grouped affine-Q4 GEMM on fp16 matrix cores, and the prefill MoE layer
// built on it (lily-qwen3.8-flash-next README, "How the speed was achieved":
// prefill is compute-bound and runs the expert GEMM over token-to-expert
// groups; "2026-09-02: Lily vs MLX 0.32.2", "Measurement contract": prompts go
// through in 2,048-token chunks).
//
// Dequantization on MFMA without a per-group fold.  With w = s*q + b,
//   y[m][n] = sum_j x[m][j] (s[n][g] q[n][j]) + sum_g b[n][g] rowsum_g(x)[m].
// The B operand of the main product is s*q in fp16, made by one packed FMA per
// code pair: (1024 + q) is an fp16 whose mantissa holds q (bits 0x6400 | q), and
// fma(1024 + q, s, -1024 s) = s*q rounded once (s*q has at most 12 significant
// bits, so the rounding is at most 2^-12 relative and often absent); a nibble that
// sits in bits 4-7 is used in place as 64 + q (bits 0x5400 | q << 4) with -64 s.  The
// accumulators then run over the whole K range with no VALU work between the
// matrix instructions.  The bias term is a small product over the group index
// (biases in fp16 are exact; the row sums are split into two fp16 parts) fed to
// the same MFMA after the main loop.
//
// Rows enter as fp16 after an exact power-of-two scaling per row (prep_rows_kernel):
// the row's largest magnitude lands in [256, 512), so every value stays in fp16's
// range, bf16 inputs convert exactly (8 significant bits fit in 11) unless they are
// below 2^-23 of the row's largest, and a row's 64-wide group sums stay below 2^15.
// The epilogue multiplies the power back in.  The SwiGLU activations are written
// as fp16 with a power of two per four columns (each value rounded to 11
// significant bits) and get the per-row treatment before the down GEMM; that
// rescaling is exact unless a value falls below fp16's normal range, so each
// activation is rounded once, as if converted from fp32 directly.
//
// Tiling: a workgroup (4 waves) owns up to 96 rows of one group (expert) and 256
// output columns (or 128 gate + 128 up columns for the SwiGLU epilogue); each
// wave computes up to 3 x 2 MFMA 32x32 blocks.  The row tile is staged through
// LDS (already in the nibble-pair order) with three groups of look-ahead (four
// stages: two workgroups fill a CU's 160 KB of LDS); each lane loads its own 16
// code bytes per group for its column.  Workgroups of the same row tile are placed
// on the same XCD so the row tile stays in that XCD's L2.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "preprows.h"

namespace q4moe {

namespace {

constexpr int BM = 96;           // rows per tile (3 MFMA row blocks; experts hold ~40-90 rows)
constexpr int MB = BM / 32;
constexpr int BN = 256;          // output columns per tile (store/scale)
constexpr int kXcd = 8;

enum Epi { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_SCALE = 2 };

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

struct GemmParams {
  const uint16_t* A;          // fp16 rows [*][K] (pair order), scaled by 2^-row_exp
  const uint16_t* xs;         // fp16 [*][2][Gp] row group-sum parts, same row indexing as A
  const int32_t* row_exp;     // [*] power of two taken out of each A row
  const int4* tiles;          // per tile {segment (expert; -1 extra; -2 none), first position, rows, 0};
                              // null: tile t covers positions t*BM.. of the extra segment
  int n_tiles;                // table length (the grid may hold a few more tiles)
  const int32_t* row_src;     // gather mode: A row (token) of each routed position; positions >= P read row pos - P
  const float* route_w;       // scale epilogue: routing weight of each routed position
  const float* extra_w;       // scale epilogue: weight of each extra-segment row (shared-expert gate), or null (1)
  int gather;
  int64_t P;                  // positions of the routed segments
  int K, G, Gp;
  int bs_vec;                 // 1: every bias row may be read 8 groups (16 bytes) at a time
  int N;                      // output columns (store/scale) or intermediate width (swiglu)
  Q4Mat W, W2;                // routed experts (W2 = up for swiglu), stacked
  int64_t w_codes_stride, w_groups_stride;
  Q4Mat X, X2;                // the extra segment's matrix (shared expert / single matrix)
  int64_t extra_rows;         // positions of the extra segment (uniform tiling when tiles is null)
  int n_slices;
  int epi;
  void* out;                  // swiglu: fp32 activations; store/scale: fp32 or bf16
  int out_bf16;
  int64_t ldo;
  int vec_out;                // N and ldo multiples of 4, out aligned to 4 elements: 4-column stores
  int b_gm;                   // the 4-bit matrices' codes are read from their group-major copies
  // store/scale with vec_out: when set, out holds fp16 values scaled by 2^-e, with one e
  // per four consecutive columns of a row in out_exp[row][ldo/4] (the four values' largest
  // magnitude lands in [2^14, 2^15))
  int8_t* out_exp;
  // K-split extra segment (SwiGLU launch): its tiles leave the table's grid region and
  // take an appended region from main_blocks on, in which each (tile, slice) is ksplit
  // workgroups over consecutive K group ranges, each writing its raw gate and up sums
  // (times 2^row_exp) to part[ks][extra row][2N]; the activation preparation adds them.
  int ksplit;                 // 1: off
  int extra_tiles;            // ceil(extra_rows / BM)
  int64_t main_blocks;        // workgroups of the table region
  float* part;
#ifdef Q4MOE_GEMM_STAMPS
  int stamp_slot;             // which of the four stamp records this launch fills
#endif
};

// Workgroup stamps, in a diagnostic build only (-DQ4MOE_GEMM_STAMPS, built into the
// diagnostic library by build.py --stamps): thread 0 of every workgroup records the
// 100 MHz s_memrealtime counter at entry, once its tile's row indices are known, after
// the main loop, after the bias term and at the end, then the hardware ids it ran on
// (XCC id << 32 | HW_ID) and its work item (tile | slice << 20 | active row blocks << 28;
// all ones for a workgroup without a tile; bit 32 marks a K-split workgroup, bits 33..
// its K range), into record stamp_slot of the array.
#ifdef Q4MOE_GEMM_STAMPS
constexpr int kGemmStampBlocks = 4096;
__device__ unsigned long long g_gemm_stamps[4][kGemmStampBlocks][8];
__device__ __forceinline__ void gemm_stamps_write(const GemmParams& p, const unsigned long long (&t)[5],
                                                  unsigned long long item) {
  if (threadIdx.x != 0 || blockIdx.x >= kGemmStampBlocks) return;
  unsigned long long* r = g_gemm_stamps[p.stamp_slot & 3][blockIdx.x];
  const unsigned long long hw = (unsigned)__builtin_amdgcn_s_getreg((31 << 11) | 4);     // HW_ID
  const unsigned long long xcc = (unsigned)__builtin_amdgcn_s_getreg((31 << 11) | 20);   // XCC_ID
  for (int i = 0; i < 5; ++i) r[i] = t[i];
  r[5] = xcc << 32 | hw;
  r[6] = item;
  r[7] = 0;
}
#define Q4MOE_GSTAMP(i) (gst[i] = __builtin_amdgcn_s_memrealtime())
#else
#define Q4MOE_GSTAMP(i) \
  do {                  \
  } while (0)
#endif

__device__ __forceinline__ f16x8_t as_f16x8(uint4 v) { return __builtin_bit_cast(f16x8_t, v); }

// Global-address-space view of a pointer: a generic (flat) load could touch
// LDS, so it would have to wait for every LDS DMA still in flight.
typedef const uint16_t __attribute__((address_space(1)))* gu16_ptr;
__device__ __forceinline__ uint32_t ld_global_u16(const uint16_t* ptr) { return *(gu16_ptr)ptr; }

// Two fp16 1024.0 in a VGPR (an and-or takes at most one literal).
__device__ __forceinline__ uint32_t magic_pair_f16_reg() {
  uint32_t m;
  asm("v_mov_b32 %0, 0x64006400" : "=v"(m));
  return m;
}

// Two fp16 64.0 in a VGPR, and the mask of bits 4-7 of each half in an SGPR.
__device__ __forceinline__ uint32_t magic64_pair_f16_reg() {
  uint32_t m;
  asm("v_mov_b32 %0, 0x54005400" : "=v"(m));
  return m;
}
__device__ __forceinline__ uint32_t nibble_hi_mask_reg() {
  uint32_t m;
  asm("s_mov_b32 %0, 0x00f000f0" : "=s"(m));
  return m;
}

__device__ __forceinline__ uint32_t pair_fma(uint32_t p, f16x2_t s2, f16x2_t m2) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(f16x2_t, p), s2, m2));
}

// The 8 codes of one word as the B operand of one MFMA K-step (pair order), s*q each
// rounded once.  A pair (q_j, q_{j+4}) is nibble j of each 16-bit half.  Nibbles 0 and
// 2 (of w and of w >> 8) go into the low mantissa bits of 1024: (word & 0x000F000F) |
// 0x64006400 is (1024 + q_j, 1024 + q_{j+4}) exactly, and one packed FMA with (s, s)
// and (-1024 s, -1024 s) leaves s*q.  Nibbles 1 and 3 stay where they are, in mantissa
// bits 4-7 of 64: 0x5400 | q << 4 is 64 + q exactly, taken with -64 s (no shift needed).
__device__ __forceinline__ uint4 codes_to_operand(uint32_t w, f16x2_t s2, f16x2_t m2, f16x2_t m2_64) {
  const uint32_t w8 = w >> 8;
  return make_uint4(pair_fma((w & nibble_mask_reg()) | magic_pair_f16_reg(), s2, m2),
                    pair_fma((w & nibble_hi_mask_reg()) | magic64_pair_f16_reg(), s2, m2_64),
                    pair_fma((w8 & nibble_mask_reg()) | magic_pair_f16_reg(), s2, m2),
                    pair_fma((w8 & nibble_hi_mask_reg()) | magic64_pair_f16_reg(), s2, m2_64));
}

// The same for 8-bit codes: the 8 codes of a block are bytes 0..3 of w0 and of w1, and
// the pair (q_j, q_{j+4}) is byte j of each, placed by one v_perm into the low bytes of
// an fp16 pair; 1024 + q is exact in fp16 for q <= 255, and s*q (at most 16
// significant bits) is rounded once, as for 4-bit codes.
__device__ __forceinline__ uint32_t scaled_pair8(uint32_t w0, uint32_t w1, uint32_t sel, f16x2_t s2, f16x2_t m2) {
  const uint32_t p = __builtin_amdgcn_perm(w1, w0, sel) | magic_pair_f16_reg();
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(f16x2_t, p), s2, m2));
}

// selector of byte j of the low source and byte j of the high source, zero bytes between
constexpr uint32_t perm_pair_sel(int j) { return (uint32_t)j | (0x0Cu << 8) | ((4u + j) << 16) | (0x0Cu << 24); }

__device__ __forceinline__ uint4 codes8_to_operand(uint32_t w0, uint32_t w1, f16x2_t s2, f16x2_t m2) {
  return make_uint4(scaled_pair8(w0, w1, perm_pair_sel(0), s2, m2), scaled_pair8(w0, w1, perm_pair_sel(1), s2, m2),
                    scaled_pair8(w0, w1, perm_pair_sel(2), s2, m2), scaled_pair8(w0, w1, perm_pair_sel(3), s2, m2));
}

// bf16 bits -> fp16 (exact for magnitudes in fp16's normal range).
__device__ __forceinline__ _Float16 bf16_bits_to_f16(uint32_t bits) { return (_Float16)bf16_bits_to_f32(bits); }


// Pipeline depth (K groups in flight) and per-stage vector-memory ops per thread:
// MB A-tile LDS loads, 2 (4-bit) or 4 (8-bit) B-code LDS loads, 2 scale loads.
// The main loop waits for a group with up to kStages - 2 later groups still in flight.
constexpr int kStages = 4;  // the stage arrays below are written out for exactly 4
template <int kBits> constexpr int ops_per_stage() { return MB + 2 * (kBits / 4) + 2; }
constexpr int A_STAGE_BYTES = BM * 128;           // BM rows x one 64-column group of fp16
// 4 waves x 2 column blocks x 64 lanes x 16 bytes (4-bit codes) or 32 bytes (8-bit codes)
template <int kBits> constexpr int b_stage_bytes() { return 4 * 2 * 64 * 16 * (kBits / 4); }

// Which tiles of the table a launch takes: all, the routed experts' only, or the extra
// segment's (shared expert) only.
enum TileSel { TILES_ALL = 0, TILES_ROUTED = 1, TILES_EXTRA = 2 };

// Swizzled slot of (row r, 16-byte word w) in an A stage.  A 128-bit LDS read
// serves 16 lanes (16 rows here) per cycle from 64 four-byte banks, i.e. two
// 128-byte rows per bank sweep: rows of equal parity share a bank half, so the
// words are XOR-rotated by row bits 1-3, which differ among the 8 rows of each
// parity in any 16 consecutive rows.
__device__ __forceinline__ int a_swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int a_slot(int r, int w) { return r * 8 + (w ^ a_swz(r)); }

// kBits: the code width of the weights this launch reads (8: the extra segment only).
template <int kBits, int kSel>
__device__ __forceinline__ void grouped_gemm_body(const GemmParams& p) {
  constexpr int B_STAGE_BYTES = b_stage_bytes<kBits>();
  constexpr int kOpsPerStage = ops_per_stage<kBits>();
  constexpr int kBW = kBits / 4;  // 16-byte code words per lane, column block and group
  // One LDS array per pipeline stage: distinct variables let the compiler see
  // that reading one stage does not depend on the DMA still filling another,
  // so it does not wait for every outstanding load before each LDS read.
  // (The compiler tracks only a few distinct DMA targets, so A and B of a stage share one array.)
  __shared__ __align__(16) uint8_t s_st0[A_STAGE_BYTES + B_STAGE_BYTES], s_st1[A_STAGE_BYTES + B_STAGE_BYTES],
      s_st2[A_STAGE_BYTES + B_STAGE_BYTES], s_st3[A_STAGE_BYTES + B_STAGE_BYTES];
  auto stage_a = [&](int st) -> uint8_t* { return st == 0 ? s_st0 : st == 1 ? s_st1 : st == 2 ? s_st2 : s_st3; };
  auto stage_b = [&](int st) -> uint8_t* { return stage_a(st) + A_STAGE_BYTES; };
  // Two small arrays live in stage memory that is idle while they are used: the tile
  // rows' source rows in stage 3 (read before the main loop, which fills stage 3 only
  // after its first barrier), the rows' epilogue factors in stage 0 (after the main loop).
  static_assert(kStages == 4, "s_src sits in the stage the prologue leaves empty");
  int32_t* const s_src = reinterpret_cast<int32_t*>(s_st3);
  float* const s_wgt = reinterpret_cast<float*>(s_st0);  // routing weight (scale epilogue) times 2^row_exp

#ifdef Q4MOE_GEMM_STAMPS
  unsigned long long gst[5] = {0, 0, 0, 0, 0};
  Q4MOE_GSTAMP(0);
#endif
  // ---- tile of this workgroup (XCD-aware: all slices of a tile share an XCD)
  const bool split_region = (int64_t)blockIdx.x >= p.main_blocks;  // (only with ksplit > 1)
  const int bid = split_region ? (int)(blockIdx.x - p.main_blocks) : (int)blockIdx.x;
  const int xcd = bid % kXcd;
  const int q = bid / kXcd;
  const int slice = q % p.n_slices;
  const int q2 = q / p.n_slices;
  const int ks = split_region ? q2 % p.ksplit : 0;
  const int tile = (split_region ? q2 / p.ksplit : q2) * kXcd + xcd;
  int seg, rows;
  int64_t row0;
#ifdef Q4MOE_GEMM_STAMPS
  if (tile >= (split_region ? p.extra_tiles : p.n_tiles)) {
    gst[4] = __builtin_amdgcn_s_memrealtime();
    gemm_stamps_write(p, gst, ~0ull);
    return;
  }
#else
  if (tile >= (split_region ? p.extra_tiles : p.n_tiles)) return;
#endif
  if (split_region) {  // extra tile `tile`: positions P + tile*BM ..
    row0 = p.P + (int64_t)tile * BM;
    seg = -1;
    rows = (int)min<int64_t>(BM, p.extra_rows - (int64_t)tile * BM);
  } else if (p.tiles) {
    // (uniform: so that the weight pointers chosen by seg below come from scalar loads,
    // and the prologue has no vector loads for the main loop's first wait to drain)
    const int4 ti = p.tiles[tile];
    seg = __builtin_amdgcn_readfirstlane(ti.x);
    row0 = __builtin_amdgcn_readfirstlane(ti.y);
    rows = __builtin_amdgcn_readfirstlane(ti.z);
  } else {
    row0 = (int64_t)tile * BM;
    seg = row0 < p.extra_rows ? -1 : -2;
    rows = (int)min<int64_t>(BM, p.extra_rows - row0);
  }
  // this workgroup's K groups
  const int nks = split_region ? p.ksplit : 1;
  const int g_lo = ks * p.G / nks, g_hi = (ks + 1) * p.G / nks;
  if (seg == -2 || (kSel == TILES_ROUTED && seg < 0) || (kSel == TILES_EXTRA && seg >= 0) ||
      (seg == -1 && p.ksplit > 1 && !split_region)) {
#ifdef Q4MOE_GEMM_STAMPS
    gst[4] = __builtin_amdgcn_s_memrealtime();
    gemm_stamps_write(p, gst, ~0ull);
#endif
    return;
  }

  // ---- source row of each tile row (padding rows repeat the last real row; their
  // outputs are dropped).  Thread r < BM also loads its row's routing weight and
  // exponent, which only the epilogue needs: those loads stay in flight meanwhile.
  static_assert(BM <= 256, "one tile row per thread");
  float row_wgt = 1.0f;
  int row_e = 0;
  if (threadIdx.x < BM) {
    const int r = threadIdx.x;
    const int64_t pos = row0 + min(r, rows - 1);
    const bool routed = pos < p.P;
    const int32_t src = p.gather ? (routed ? p.row_src[pos] : (int32_t)(pos - p.P)) : (int32_t)pos;
    s_src[r] = src;
    if (p.epi == EPI_SCALE) row_wgt = routed ? p.route_w[pos] : (p.extra_w ? p.extra_w[pos - p.P] : 1.0f);
    row_e = p.row_exp[src];
  }

  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int ln = lane & 31, lh = lane >> 5;
  const bool swiglu = __builtin_amdgcn_readfirstlane(p.epi) == EPI_SWIGLU;

  // ---- weight rows (B columns) of this lane: nb = 0, 1
  const Q4Mat M0 = seg >= 0 ? p.W : p.X;  // (by value: selected in scalar registers)
  const Q4Mat M1 = seg >= 0 ? (swiglu ? p.W2 : p.W) : (swiglu ? p.X2 : p.X);
  const int64_t oc = seg >= 0 ? seg * p.w_codes_stride : 0;
  const int64_t og = seg >= 0 ? seg * p.w_groups_stride : 0;
  // Group-major codes: one K group of 32 consecutive rows is 1 KB of contiguous bytes,
  // so each B load instruction reads whole cache lines instead of 32 rows' 32-byte pieces.
  const bool gm = kBits == 4 && p.b_gm;
  const int64_t bstep = gm ? (int64_t)p.N * 2 : 2 * kBW;  // per K group, in 16-byte words
  int col[2];
  const uint4* bcodes[2];
  const uint16_t* bscale[2];
  const uint16_t* bbias[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    col[nb] = swiglu ? slice * 128 + wave * 32 + ln : slice * BN + wave * 64 + nb * 32 + ln;
    const int64_t wrow = min(col[nb], p.N - 1);
    const Q4Mat Mx = nb == 0 ? M0 : M1;
    // this lane's half of a group: 32 codes = 16 bytes (4-bit) or 32 bytes (8-bit)
    bcodes[nb] = gm ? reinterpret_cast<const uint4*>(Mx.codes_gm + oc) + wrow * 2 + lh
                    : reinterpret_cast<const uint4*>(Mx.codes + oc + wrow * (p.K * kBits / 32)) + kBW * lh;
    bscale[nb] = Mx.scales + og + wrow * p.G;
    bbias[nb] = Mx.biases + og + wrow * p.G;
  }
  __syncthreads();  // s_src ready
  Q4MOE_GSTAMP(1);

  // ---- A-tile loads of this thread: MB instructions, rows (wave*MB+i)*8 + lane/8, swizzled word
  const uint16_t* a_ptr[MB];
  int a_word[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int r = (wave * MB + i) * 8 + (lane >> 3);
    a_word[i] = (lane & 7) ^ a_swz(r);
    a_ptr[i] = p.A + (int64_t)s_src[r] * p.K + a_word[i] * 8;
  }
  // source rows of this lane's bias-term rows (s_src is overwritten by the main loop)
  int src_mb[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    src_mb[mb] = s_src[mb * 32 + ln];
    asm volatile("" : "+v"(src_mb[mb]));  // read here, before the loads that refill stage 3
  }

  // Issue all loads of K group g_lo + g into stage `st`.  Past the last group the last group
  // is loaded again (an L2 hit into a stage no step reads): every step then issues the
  // same loads and waits for the same count, with no branch for the compiler's own
  // wait placement to merge (after such a branch it waits for every load in flight).
  auto issue = [&](int g, int st, uint32_t (&sc)[2]) {
    g = min(g_lo + g, g_hi - 1);
#pragma unroll
    for (int i = 0; i < MB; ++i)
      __builtin_amdgcn_global_load_lds(a_ptr[i] + g * 64, stage_a(st) + (wave * MB + i) * 1024, 16, 0, 0);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int h = 0; h < kBW; ++h)
        __builtin_amdgcn_global_load_lds(bcodes[nb] + g * bstep + h, stage_b(st) + ((wave * 2 + nb) * kBW + h) * 1024,
                                         16, 0, 0);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) sc[nb] = ld_global_u16(bscale[nb] + g);
  };

  const int mblocks = (rows + 31) >> 5;  // active 32-row blocks (wave-uniform)
  const f32x16_t zero16 = {};
  f32x16_t acc[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = zero16;

  // Raw bf16 scale bits of the groups in flight, converted where they are used
  // (a conversion next to the load would make the wave wait for it there).
  uint32_t sc[kStages][2];


  // The main loop is specialised on the number of active row blocks so that a
  // group's body has no branches: every wait the compiler adds then sits at a
  // use of the data, not at a join right after the look-ahead loads.
  auto main_loop = [&](auto nmb_c) __attribute__((always_inline)) {
    constexpr int NMB = decltype(nmb_c)::value;
    // The first groups' loads, issued after the branch on NMB: issued before it, their
    // scale words are widened there at once, which waits for every load.  (The marker,
    // different in each specialisation, keeps the compiler from hoisting them back.)
    asm volatile("; grouped GEMM main loop, %0 row blocks" ::"n"(NMB));
#pragma unroll
    for (int st = 0; st < kStages - 1; ++st) issue(st, st, sc[st]);
    // One K group from stage ST (a compile-time stage, so each LDS access names one array).
    auto step = [&](int g, auto st_c) __attribute__((always_inline)) {
      constexpr int st = decltype(st_c)::value;
      constexpr int sn = (st + kStages - 1) % kStages;
      // keep each group's instructions (notably the scale conversions) inside its own step
      __builtin_amdgcn_sched_barrier(0);
      // Group g has landed for this wave and this wave's reads of the stage about
      // to be refilled are done; the barrier extends both to every wave.  (A
      // workgroup fence here would also wait for the look-ahead DMA.)  The loads of
      // groups g+1 and g+2, issued after group g's, may still be in flight.
      __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(kOpsPerStage * (kStages - 2)));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // The look-ahead group goes out first: every wave has finished reading the
      // stage it refills (the barrier above), and loads issued here have two whole
      // steps to land (left to the scheduler they sink below the MFMAs).
      issue(g + kStages - 1, sn, sc[sn]);
      __builtin_amdgcn_sched_barrier(0);

      const uint8_t* sa = stage_a(st);
      const uint8_t* sb = stage_b(st) + wave * 2 * kBW * 1024 + lane * 16;
      // This wave's B codes first, then A fragments double-buffered over row
      // blocks: block 0's reads are in flight during the B conversion, block
      // mb+1's during block mb's MFMAs.
      uint4 af[2][4];
      auto read_a = [&](int mb, uint4 (&dst)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
          dst[s4] = *reinterpret_cast<const uint4*>(sa + a_slot(mb * 32 + ln, 4 * lh + s4) * 16);
      };
      uint4 rb[2][kBW];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int h = 0; h < kBW; ++h) rb[nb][h] = *reinterpret_cast<const uint4*>(sb + (nb * kBW + h) * 1024);
      read_a(0, af[0]);
      f16x2_t s2[2], m2[2], m64[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        // the fp16 scale and its exact multiples -1024 s and -64 s
        const _Float16 sh = (_Float16)bf16_bits_to_f32(sc[st][nb]);
        const _Float16 mh = sh * (_Float16)-1024.0f, m6 = sh * (_Float16)-64.0f;
        s2[nb] = f16x2_t{sh, sh};
        m2[nb] = f16x2_t{mh, mh};
        m64[nb] = f16x2_t{m6, m6};
      }
      uint4 bop[2][4];  // this group's B operands, converted once, used by every row block
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        if constexpr (kBits == 4) {
          const uint4 r = rb[nb][0];
          bop[nb][0] = codes_to_operand(r.x, s2[nb], m2[nb], m64[nb]);
          bop[nb][1] = codes_to_operand(r.y, s2[nb], m2[nb], m64[nb]);
          bop[nb][2] = codes_to_operand(r.z, s2[nb], m2[nb], m64[nb]);
          bop[nb][3] = codes_to_operand(r.w, s2[nb], m2[nb], m64[nb]);
        } else {  // 8 codes per word pair
          bop[nb][0] = codes8_to_operand(rb[nb][0].x, rb[nb][0].y, s2[nb], m2[nb]);
          bop[nb][1] = codes8_to_operand(rb[nb][0].z, rb[nb][0].w, s2[nb], m2[nb]);
          bop[nb][2] = codes8_to_operand(rb[nb][1].x, rb[nb][1].y, s2[nb], m2[nb]);
          bop[nb][3] = codes8_to_operand(rb[nb][1].z, rb[nb][1].w, s2[nb], m2[nb]);
        }
      }
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        if (mb + 1 < NMB) read_a(mb + 1, af[(mb + 1) & 1]);
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          acc[mb][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(af[mb & 1][s4]), as_f16x8(bop[0][s4]),
                                                              acc[mb][0], 0, 0, 0);
          acc[mb][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(af[mb & 1][s4]), as_f16x8(bop[1][s4]),
                                                              acc[mb][1], 0, 0, 0);
        }
      }
    };
    int g0 = 0;
    const int ng = g_hi - g_lo;
    for (; g0 + kStages <= ng; g0 += kStages) {
      step(g0, std::integral_constant<int, 0>{});
      step(g0 + 1, std::integral_constant<int, 1>{});
      step(g0 + 2, std::integral_constant<int, 2>{});
      step(g0 + 3, std::integral_constant<int, 3>{});
    }
    // the last G mod 4 groups
    if (g0 < ng) step(g0, std::integral_constant<int, 0>{});
    if (g0 + 1 < ng) step(g0 + 1, std::integral_constant<int, 1>{});
    if (g0 + 2 < ng) step(g0 + 2, std::integral_constant<int, 2>{});
  };
  if (mblocks == 1)
    main_loop(std::integral_constant<int, 1>{});
  else if (mblocks == 2)
    main_loop(std::integral_constant<int, 2>{});
  else
    main_loop(std::integral_constant<int, 3>{});
  // the repeated last-group loads of the final steps are still in flight (into stages)
  __builtin_amdgcn_s_waitcnt(0);
  Q4MOE_GSTAMP(2);
  // ---- bias term: sum_g bias[n][g] * rowsum_g[m], on MFMA (fp16 biases exact, row sums in two parts).
  // Each 16-group slice takes one round of loads (the 8 groups' biases of this lane's column,
  // 16 bytes where aligned, and the rows' group-sum parts), issued one slice ahead.
  struct CorrLoads {
    uint4 bias[2];   // [nb]: 8 groups' bf16 biases
    uint4 xa[MB][2]; // [mb][part]: 8 groups' fp16 row-sum parts
  };
  auto corr_load = [&](int t, CorrLoads& L) __attribute__((always_inline)) {
    const int gbase = t * 16 + 8 * lh;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      if (p.bs_vec) {
        const bool any = gbase < p.G;  // with G % 8 == 0 a slice half is all real groups or all padding
        L.bias[nb] = any ? *reinterpret_cast<const uint4*>(bbias[nb] + gbase) : make_uint4(0, 0, 0, 0);
      } else {
        uint32_t bv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int g = min(gbase + j, p.G - 1);  // padding groups: loaded clamped, zeroed
          bv[j] = gbase + j < p.G ? ld_global_u16(bbias[nb] + g) : 0u;
        }
        L.bias[nb] = make_uint4(bv[0] | bv[1] << 16, bv[2] | bv[3] << 16, bv[4] | bv[5] << 16, bv[6] | bv[7] << 16);
      }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (mb >= mblocks) continue;
      const uint16_t* xr = p.xs + (int64_t)src_mb[mb] * 2 * p.Gp + gbase;
#pragma unroll
      for (int part_i = 0; part_i < 2; ++part_i) L.xa[mb][part_i] = *reinterpret_cast<const uint4*>(xr + part_i * p.Gp);
    }
  };
  auto corr_apply = [&](const CorrLoads& L) __attribute__((always_inline)) {
    uint4 bc[2];  // [nb]: the 8 groups' biases as fp16
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const uint32_t bw[4] = {L.bias[nb].x, L.bias[nb].y, L.bias[nb].z, L.bias[nb].w};
      uint32_t hv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f16x2_t h2 = {bf16_bits_to_f16(bw[j] & 0xFFFFu), bf16_bits_to_f16(bw[j] >> 16)};
        hv[j] = __builtin_bit_cast(uint32_t, h2);
      }
      bc[nb] = make_uint4(hv[0], hv[1], hv[2], hv[3]);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (mb >= mblocks) continue;
#pragma unroll
      for (int part_i = 0; part_i < 2; ++part_i)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(L.xa[mb][part_i]), as_f16x8(bc[nb]),
                                                               acc[mb][nb], 0, 0, 0);
    }
  };

  if (ks == 0) {  // (a K-split tile's bias term, over all groups, goes with its first range)
    const int nt = (p.Gp + 15) / 16;
    CorrLoads cur, nxt;
    corr_load(0, cur);
    for (int t = 0; t < nt; ++t) {
      if (t + 1 < nt) corr_load(t + 1, nxt);
      corr_apply(cur);
      cur = nxt;
    }
  }

  Q4MOE_GSTAMP(3);
  __syncthreads();  // every wave is past its last read of stage 0 (s_wgt below)
  // The factor is formed only here: computed where its loads are issued, it would make
  // the prologue wait for them before its barrier.
  asm volatile("" : "+v"(row_wgt), "+v"(row_e));
  if (threadIdx.x < BM) s_wgt[threadIdx.x] = ldexpf(row_wgt, row_e);  // exact: a power of two
  __syncthreads();

  // ---- epilogue.  D layout: column = lane % 32, row = 8*(i/4) + 4*(lane/32) + i%4.
  if (split_region) {
    // raw gate and up sums of this K range (exact power-of-two factor), 32 consecutive
    // columns per store instruction
    float* part = p.part + (int64_t)ks * p.extra_rows * 2 * p.N;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (mb >= mblocks) continue;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = mb * 32 + 8 * (i >> 2) + 4 * lh + (i & 3);
        if (r >= rows || col[0] >= p.N) continue;
        const float f = s_wgt[r];
        float* o = part + (row0 - p.P + r) * 2 * p.N + col[0];
        o[0] = f * acc[mb][0][i];
        o[p.N] = f * acc[mb][1][i];
      }
    }
  } else if (p.vec_out) {
    // Through LDS, 16 tile rows at a time (registers i = 8h .. 8h+7 of row block mb), in
    // stages 1 and 2 alternately, so that each thread stores whole 4-column chunks and a
    // wave's stores cover contiguous row segments: 4 (SwiGLU: 2) 16-byte stores per thread
    // and half block instead of one 4-byte store per lane and register.  The barriers are
    // LDS-only, so the stores of one half stay in flight while the next is staged.
    const int ncol = swiglu ? 128 : BN;  // columns of this workgroup's tile
    const int ostr = ncol + 8;           // row stride (floats): rows r and r + 4 fall 32 banks apart
    const int cpr = ncol >> 2;           // 4-column chunks per row
    const int colw = swiglu ? slice * 128 : slice * BN;
    static_assert(16 * (BN + 8) * 4 <= A_STAGE_BYTES + b_stage_bytes<4>(), "a half block fits one stage");
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (mb >= mblocks) break;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float* so = reinterpret_cast<float*>(h ? s_st2 : s_st1);
        const int rbase = mb * 32 + 16 * h;
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) {
          const int i = 8 * h + ii;
          const int rr = 8 * (ii >> 2) + 4 * lh + (ii & 3);
          const float f = s_wgt[rbase + rr];
          if (swiglu) {
            so[rr * ostr + wave * 32 + ln] = silu(f * acc[mb][0][i]) * (f * acc[mb][1][i]);
          } else {
            so[rr * ostr + wave * 64 + ln] = f * acc[mb][0][i];
            so[rr * ostr + wave * 64 + 32 + ln] = f * acc[mb][1][i];
          }
        }
        lds_sync();

        for (int c = threadIdx.x; c < 16 * cpr; c += 256) {
          const int rr = c / cpr, q = c - rr * cpr;
          const int r = rbase + rr, cc = colw + 4 * q;
          if (r < rows && cc < p.N) {
            const float4 v = *reinterpret_cast<const float4*>(so + rr * ostr + 4 * q);
            const int64_t o = (row0 + r) * p.ldo + cc;
            if (p.out_exp) {
              const float mx = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
              int e = 0;
              if (mx > 0.0f && mx <= 3.0e38f) {
                int ex;
                frexpf(mx, &ex);  // mx in [2^(ex-1), 2^ex)
                e = max(ex - 15, -127);
              }
              const f16x2_t lo = {(_Float16)ldexpf(v.x, -e), (_Float16)ldexpf(v.y, -e)};
              const f16x2_t hi = {(_Float16)ldexpf(v.z, -e), (_Float16)ldexpf(v.w, -e)};
              *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + o) =
                  make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
              p.out_exp[o >> 2] = (int8_t)e;
            } else if (p.out_bf16) {
              const uint2 w = make_uint2(f32_to_bf16_bits(v.x) | (f32_to_bf16_bits(v.y) << 16),
                                         f32_to_bf16_bits(v.z) | (f32_to_bf16_bits(v.w) << 16));
              *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + o) = w;
            } else {
              *reinterpret_cast<float4*>(static_cast<float*>(p.out) + o) = v;
            }
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (mb >= mblocks) continue;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = mb * 32 + 8 * (i >> 2) + 4 * lh + (i & 3);
        if (r >= rows) continue;
        const int64_t pos = row0 + r;
        const float f = s_wgt[r];
        if (swiglu) {
          if (col[0] < p.N) {
            const float a = silu(f * acc[mb][0][i]) * (f * acc[mb][1][i]);
            reinterpret_cast<float*>(p.out)[pos * p.ldo + col[0]] = a;
          }
        } else {
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            if (col[nb] >= p.N) continue;
            const float v = f * acc[mb][nb][i];
            if (p.out_bf16)
              reinterpret_cast<uint16_t*>(p.out)[pos * p.ldo + col[nb]] = (uint16_t)f32_to_bf16_bits(v);
            else
              reinterpret_cast<float*>(p.out)[pos * p.ldo + col[nb]] = v;
          }
        }
      }
    }
  }
#ifdef Q4MOE_GEMM_STAMPS
  gst[4] = __builtin_amdgcn_s_memrealtime();
  gemm_stamps_write(p, gst, (unsigned long long)tile | (unsigned long long)slice << 20 |
                                (unsigned long long)mblocks << 28 | (unsigned long long)split_region << 32 |
                                (unsigned long long)ks << 33);
#endif
}

__global__ __launch_bounds__(256, 2) void grouped_q4_gemm_kernel(GemmParams p) { grouped_gemm_body<4, TILES_ALL>(p); }
__global__ __launch_bounds__(256, 2) void grouped_q4_gemm_routed_kernel(GemmParams p) {
  grouped_gemm_body<4, TILES_ROUTED>(p);
}
// the extra segment with 8-bit codes: its doubled code stages take one workgroup per CU
__global__ __launch_bounds__(256, 1) void grouped_q8_gemm_extra_kernel(GemmParams p) {
  grouped_gemm_body<8, TILES_EXTRA>(p);
}

using prep::SplitRows;

template <typename In>
__global__ void prep_rows_kernel(const In* __restrict__ A, int64_t rows, int K, int Gp, uint16_t* __restrict__ out,
                                 uint16_t* __restrict__ sums, int32_t* __restrict__ exps, SplitRows sp,
                                 const int8_t* __restrict__ in_exp) {
  prep::prep_rows_body<In>(A, rows, K, Gp, out, sums, exps, sp, blockIdx.x, gridDim.x, in_exp);
}

// The shared expert's weight per token, sigmoid(w . X[t]) (the shared-expert gate), one wave
// per token.
__global__ void shared_gate_kernel(const uint16_t* __restrict__ w, const uint16_t* __restrict__ X, int64_t T, int H,
                                   float* __restrict__ gate) {
  const int lane = lane_id();
  const int64_t wstride = (int64_t)gridDim.x * (blockDim.x / kWave);
  for (int64_t t = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave; t < T; t += wstride) {
    const uint4* a = reinterpret_cast<const uint4*>(w);
    const uint4* b = reinterpret_cast<const uint4*>(X + t * H);
    float d0 = 0.f, d1 = 0.f;
    for (int c = lane; c < (H >> 3); c += kWave) {
      const uint4 u = a[c], v = b[c];
      d0 = dot2_bf16(u.x, v.x, d0);
      d1 = dot2_bf16(u.y, v.y, d1);
      d0 = dot2_bf16(u.z, v.z, d0);
      d1 = dot2_bf16(u.w, v.w, d1);
    }
    const float d = group_sum_rt(d0 + d1, 6);
    if (lane == 0) gate[t] = 1.0f / (1.0f + __expf(-d));
  }
}

// Y[t] = Ys[P + t] (shared expert, weight already applied) + sum_slot Ys[inv[t*k + slot]], fixed slot order.
// Eight columns 8c.. of per-position row r: fp16 values times their powers of two (one
// per four columns).
__device__ __forceinline__ void load_scaled8(const uint16_t* Ys, const int8_t* Ye, int64_t r, int c, int H,
                                             float (&v)[8]) {
  const uint4 w = reinterpret_cast<const uint4*>(Ys + r * H)[c];
  const uint32_t e2 = reinterpret_cast<const uint16_t*>(Ye + r * (H >> 2))[c];  // columns 0-3, 4-7
  const int e0 = (int8_t)(e2 & 0xFFu), e1 = (int8_t)(e2 >> 8);
  const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f16x2_t h = __builtin_bit_cast(f16x2_t, ww[j]);
    const int e = j < 2 ? e0 : e1;
    v[2 * j] = ldexpf((float)h.x, e);
    v[2 * j + 1] = ldexpf((float)h.y, e);
  }
}

// Each thread takes 8 columns of one token (16-byte loads of every row it adds).
__global__ void combine_kernel(const uint16_t* __restrict__ Ys, const int8_t* __restrict__ Ye,
                               const int32_t* __restrict__ inv, int64_t T, int k, int H, int has_shared, int64_t P,
                               void* __restrict__ Y, int out_bf16) {
  const int H8 = H >> 3;
  const int64_t total = T * H8;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / H8;
    const int c = (int)(i - t * H8);
    float acc[8] = {};
    if (has_shared) load_scaled8(Ys, Ye, P + t, c, H, acc);
    for (int j = 0; j < k; ++j) {
      float v[8];
      load_scaled8(Ys, Ye, inv[t * k + j], c, H, v);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] += v[q];
    }
    if (out_bf16) {
      uint4 o;
      o.x = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
      o.y = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
      o.z = f32_to_bf16_bits(acc[4]) | (f32_to_bf16_bits(acc[5]) << 16);
      o.w = f32_to_bf16_bits(acc[6]) | (f32_to_bf16_bits(acc[7]) << 16);
      reinterpret_cast<uint4*>(static_cast<uint16_t*>(Y) + t * H)[c] = o;
    } else {
      float4* y = reinterpret_cast<float4*>(static_cast<float*>(Y) + t * H) + 2 * c;
      y[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      y[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

int grid_for(int64_t n, int block) {
  int64_t b = (n + block - 1) / block;
  if (b > 65536) b = 65536;
  return (int)(b < 1 ? 1 : b);
}

int pad16(int g) { return (g + 15) & ~15; }

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// extra_q8: the extra segment (shared expert) holds 8-bit codes; it then takes a launch
// of its own after the routed tiles'.
hipError_t launch_grouped(GemmParams& p, int64_t max_tiles, hipStream_t stream, bool extra_q8 = false) {
  // (the SwiGLU epilogue writes a quarter of the bytes per tile and measured no faster
  // staged in fp32; it is staged for the scaled fp16 form, which needs 4 columns per thread)
  p.vec_out = (p.epi != EPI_SWIGLU || p.out_exp) && p.N % 4 == 0 && p.ldo % 4 == 0 &&
              (reinterpret_cast<uintptr_t>(p.out) & (p.out_bf16 ? 7u : 15u)) == 0;
  if (p.out_exp && !p.vec_out) return hipErrorInvalidValue;  // the scaled fp16 form is a vec_out epilogue
#ifdef Q4MOE_GEMM_STAMPS
  static int stamp_launches = 0;
  p.stamp_slot = stamp_launches++ & 3;
#endif
  p.bs_vec = p.G % 8 == 0;
  for (const Q4Mat* m : {&p.W, &p.W2, &p.X, &p.X2})
    if (m->scales && (!aligned16(m->scales) || !aligned16(m->biases))) p.bs_vec = 0;
  p.n_tiles = (int)max_tiles;
  const int64_t tiles_rounded = (max_tiles + kXcd - 1) / kXcd * kXcd;
  if (p.ksplit < 1) p.ksplit = 1;
  p.main_blocks = tiles_rounded * p.n_slices;
  p.extra_tiles = (int)((p.extra_rows + BM - 1) / BM);
  const int64_t blocks =
      p.main_blocks + (p.ksplit > 1 ? (int64_t)(p.extra_tiles + kXcd - 1) / kXcd * kXcd * p.n_slices * p.ksplit : 0);
  if (!extra_q8) {
    hipLaunchKernelGGL(grouped_q4_gemm_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL(grouped_q4_gemm_routed_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    hipLaunchKernelGGL(grouped_q8_gemm_extra_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

// fp16 pair-order copy, row exponents and group-sum parts of `rows` rows of length K.
template <typename In>
hipError_t launch_prep_rows(const In* A, int64_t rows, int K, uint16_t* out, uint16_t* sums, int32_t* exps,
                            hipStream_t stream, SplitRows sp = SplitRows{nullptr, INT64_MAX, 0, 1},
                            const int8_t* in_exp = nullptr) {
  if (rows == 0) return hipSuccess;
  const int Gp = pad16(K >> 6);
  const int64_t blocks = std::min<int64_t>((rows + 3) / 4, 8192);
  hipLaunchKernelGGL(prep_rows_kernel<In>, dim3((unsigned)blocks), dim3(256), 0, stream, A, rows, K, Gp, out, sums,
                     exps, sp, in_exp);
  return hipGetLastError();
}

}  // namespace

namespace {
// Group-major copy of 4-bit codes: 16-byte word i of dst is half (i & 1) of group g of
// row r of matrix e, with i >> 1 = (e*G + g)*n + r; the source row holds G*2 such words.
__global__ void pack_group_major_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t count,
                                        int64_t n, int64_t G) {
  const int64_t total = count * G * n * 2;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t rn = i >> 1;
    const int64_t r = rn % n, eg = rn / n;
    const int64_t g = eg % G, e = eg / G;
    dst[i] = src[(e * n + r) * (G * 2) + g * 2 + (i & 1)];
  }
}
}  // namespace

hipError_t run_pack_group_major(const uint32_t* codes, int64_t count, int64_t n, int k, uint32_t* dst,
                                hipStream_t stream) {
  const int64_t words = count * n * (k / 64) * 2;
  if (words == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((words + 255) / 256, 8192);
  hipLaunchKernelGGL(pack_group_major_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const uint4*>(codes), reinterpret_cast<uint4*>(dst), count, n,
                     (int64_t)(k / 64));
  return hipGetLastError();
}

// q4_gemm workspace: row-sum parts [m][2][Gp] fp16, row exponents [m], fp16 rows [m][k].
size_t gemm_workspace_bytes(int64_t m, int k) {
  return align256((size_t)m * 2 * pad16(k / 64) * 2) + align256((size_t)m * 4) + align256((size_t)m * k * 2);
}

hipError_t run_q4_gemm(const Q4Mat& W, int64_t n, int k, const uint16_t* X, int64_t m, void* Y, int out_bf16,
                       void* ws, hipStream_t stream) {
  char* c = static_cast<char*>(ws);
  uint16_t* xs = reinterpret_cast<uint16_t*>(c);
  c += align256((size_t)m * 2 * pad16(k / 64) * 2);
  int32_t* xe = reinterpret_cast<int32_t*>(c);
  c += align256((size_t)m * 4);
  uint16_t* xp = reinterpret_cast<uint16_t*>(c);
  hipError_t e = launch_prep_rows(X, m, k, xp, xs, xe, stream);
  if (e != hipSuccess) return e;
  GemmParams p{};
  p.A = xp;
  p.xs = xs;
  p.row_exp = xe;
  p.gather = 0;
  p.P = 0;
  p.K = k;
  p.G = k / 64;
  p.Gp = pad16(p.G);
  p.N = (int)n;
  p.X = W;
  p.X2 = W;
  p.b_gm = W.codes_gm != nullptr;
  p.extra_rows = m;
  p.n_slices = (int)((n + BN - 1) / BN);
  p.epi = EPI_STORE;
  p.out = Y;
  p.out_bf16 = out_bf16;
  p.ldo = n;
  return launch_grouped(p, (m + BM - 1) / BM, stream);
}

namespace {
// The shared expert's gate/up tiles (all T rows, the last of the launch) are split in K
// this many ways, so that the launch's last partial round of workgroups is short.
#ifndef Q4MOE_SHARED_KSPLIT
#define Q4MOE_SHARED_KSPLIT 2
#endif
constexpr int kSharedKSplit = Q4MOE_SHARED_KSPLIT;

struct PrefillWs {
  float* logits;
  int32_t* ids;
  float* weights;
  int32_t* offsets;
  int32_t* sorted_rows;
  int32_t* inv;
  int4* tiles;
  int32_t* row_src;
  float* row_w;
  void* perm_ws;
  uint16_t* xs_x;   // [T][2][Gp(H)] fp16 group-sum parts of the rows
  int32_t* xe_x;    // [T] row exponents
  uint16_t* xp;     // [T][H] fp16 rows (pair order)
  uint16_t* act16;  // [R][I] SwiGLU outputs: fp16 scaled by 2^-act_e
  int8_t* act_e;    // [R][I/4] the powers of two of act16, one per four columns
  uint16_t* act;    // [R][I] fp16 activations (pair order)
  uint16_t* xs_act; // [R][2][Gp(I)]
  int32_t* xe_act;  // [R]
  uint16_t* ys;     // [R][H] per-position outputs, weighted: fp16 scaled by 2^-ye
  int8_t* ye;       // [R][H/4] the powers of two of ys, one per four columns
  float* sh_gate;   // [T] shared-expert weight per token (with a shared-expert gate)
  float* part;      // [kSharedKSplit][T][2I] K-split gate and up sums of the 4-bit shared expert
  size_t total;
};

PrefillWs carve(void* base, int64_t T, int H, int I, int E, int k, int has_shared) {
  PrefillWs w{};
  char* c = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) { char* r = c ? c + off : nullptr; off += align256(bytes); return r; };
  const int64_t P = T * k, R = P + (has_shared ? T : 0);
  const int max_tiles = group_max_tiles(P, E, has_shared ? T : 0, BM);
  w.logits = reinterpret_cast<float*>(take(route_workspace_bytes(T, E)));
  w.ids = reinterpret_cast<int32_t*>(take(P * 4));
  w.weights = reinterpret_cast<float*>(take(P * 4));
  w.offsets = reinterpret_cast<int32_t*>(take((E + 1) * 4));
  w.sorted_rows = reinterpret_cast<int32_t*>(take(P * 4));
  w.inv = reinterpret_cast<int32_t*>(take(P * 4));
  w.tiles = reinterpret_cast<int4*>(take((size_t)max_tiles * 16));
  w.row_src = reinterpret_cast<int32_t*>(take(P * 4));
  w.row_w = reinterpret_cast<float*>(take(P * 4));
  w.perm_ws = take(permute_workspace_bytes(P, E));
  w.xs_x = reinterpret_cast<uint16_t*>(take((size_t)T * 2 * pad16(H / 64) * 2));
  w.xe_x = reinterpret_cast<int32_t*>(take((size_t)T * 4));
  w.xp = reinterpret_cast<uint16_t*>(take((size_t)T * H * 2));
  w.act16 = reinterpret_cast<uint16_t*>(take((size_t)R * I * 2));
  w.act_e = reinterpret_cast<int8_t*>(take((size_t)R * (I / 4)));
  w.act = reinterpret_cast<uint16_t*>(take((size_t)R * I * 2));
  w.xs_act = reinterpret_cast<uint16_t*>(take((size_t)R * 2 * pad16(I / 64) * 2));
  w.xe_act = reinterpret_cast<int32_t*>(take((size_t)R * 4));
  w.ys = reinterpret_cast<uint16_t*>(take((size_t)R * H * 2));
  w.ye = reinterpret_cast<int8_t*>(take((size_t)R * (H / 4)));
  w.sh_gate = reinterpret_cast<float*>(take((size_t)T * 4));
  w.part = reinterpret_cast<float*>(take(has_shared ? (size_t)kSharedKSplit * T * 2 * I * 4 : 0));
  w.total = off;
  return w;
}
}  // namespace

size_t prefill_workspace_bytes(int64_t T, int hidden, int inter, int n_experts, int top_k, int has_shared) {
  return carve(nullptr, T, hidden, inter, n_experts, top_k, has_shared).total;
}

hipError_t run_moe_ffn_prefill(const DecodeLayer& L, const uint16_t* X, int64_t T, void* Y, int out_bf16, void* ws,
                               hipStream_t stream) {
  const int H = L.hidden, I = L.inter, E = L.n_experts, k = L.top_k;
  PrefillWs w = carve(ws, T, H, I, E, k, L.has_shared);
  const int64_t P = T * k;
  const int64_t extra = L.has_shared ? T : 0;
  const int max_tiles = group_max_tiles(P, E, extra, BM);
  hipError_t e = run_route_topk(L.router, E, H, X, T, k, w.ids, w.weights, w.logits, stream, &L.router_q8);
  if (e != hipSuccess) return e;
  GroupTiles gt{};
  gt.tile_rows = BM;
  gt.max_tiles = max_tiles;
  gt.extra_rows = extra;
  gt.topk = k;
  gt.weights = w.weights;
  gt.table = w.tiles;
  gt.row_src = w.row_src;
  gt.row_w = w.row_w;
  // the token rows' fp16 preparation runs in the rank launch of the sort, beside its few workgroups
  const PrepRowsJob prep{X, T, H, pad16(H / 64), w.xp, w.xs_x, w.xe_x};
  e = run_permute(w.ids, P, E, w.offsets, w.sorted_rows, w.inv, w.perm_ws, &gt, stream, &prep);
  if (e != hipSuccess) return e;

  // gate/up with SwiGLU -> act16/act_e (fp16 with a power of two per four columns,
  // sorted positions; shared rows appended)
  GemmParams p{};
  p.A = w.xp;
  p.xs = w.xs_x;
  p.row_exp = w.xe_x;
  p.tiles = w.tiles;
  p.row_src = w.row_src;
  p.route_w = w.row_w;
  p.gather = 1;
  p.P = P;
  p.K = H;
  p.G = H / 64;
  p.Gp = pad16(p.G);
  p.N = I;
  p.W = L.gate;
  p.W2 = L.up;
  p.w_codes_stride = (int64_t)I * (H / 8);
  p.w_groups_stride = (int64_t)I * (H / 64);
  p.X = L.sh_gate;
  p.X2 = L.sh_up;
  p.extra_rows = extra;
  p.n_slices = (I + 127) / 128;
  p.epi = EPI_SWIGLU;
  p.out = w.act16;
  p.out_exp = w.act_e;
  p.out_bf16 = 0;
  p.ldo = I;
  const bool sh_q8 = L.has_shared && L.sh_q8;
  // the 4-bit shared expert's tiles split in K (the 8-bit one runs in a launch of its own)
  const int ksplit = L.has_shared && !sh_q8 ? std::min(kSharedKSplit, p.G) : 1;
  p.ksplit = ksplit;
  p.part = w.part;
  // group-major codes when every 4-bit matrix of the launch has them (an 8-bit shared
  // expert runs in a launch of its own that reads its row-major codes)
  auto gm = [](const Q4Mat& a, const Q4Mat& b) { return a.codes_gm && b.codes_gm; };
  p.b_gm = gm(L.gate, L.up) && (!L.has_shared || sh_q8 || gm(L.sh_gate, L.sh_up));
  e = launch_grouped(p, max_tiles, stream, sh_q8);
  if (e != hipSuccess) return e;

  const int64_t R = P + extra;
  const SplitRows sp = ksplit > 1 ? SplitRows{w.part, P, T * 2 * I, ksplit} : SplitRows{nullptr, INT64_MAX, 0, 1};
  e = launch_prep_rows(reinterpret_cast<const prep::f16x_t*>(w.act16), R, I, w.act, w.xs_act, w.xe_act, stream, sp,
                       w.act_e);
  if (e != hipSuccess) return e;

  // down with the routing weight -> ys (fp32, sorted positions)
  GemmParams d = p;
  d.ksplit = 1;
  d.part = nullptr;
  d.A = w.act;
  d.xs = w.xs_act;
  d.row_exp = w.xe_act;
  d.gather = 0;
  d.K = I;
  d.G = I / 64;
  d.Gp = pad16(d.G);
  d.N = H;
  d.W = L.down;
  d.W2 = L.down;
  d.w_codes_stride = (int64_t)H * (I / 8);
  d.w_groups_stride = (int64_t)H * (I / 64);
  d.X = L.sh_down;
  d.X2 = L.sh_down;
  d.b_gm = gm(L.down, L.down) && (!L.has_shared || sh_q8 || gm(L.sh_down, L.sh_down));
  d.n_slices = (H + BN - 1) / BN;
  d.epi = EPI_SCALE;
  d.out = w.ys;
  d.out_exp = w.ye;
  d.out_bf16 = 0;
  d.ldo = H;
  if (L.has_shared && L.sh_gate_w) {
    const int64_t blocks = std::min<int64_t>((T + 3) / 4, 4096);
    hipLaunchKernelGGL(shared_gate_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, L.sh_gate_w, X, T, H,
                       w.sh_gate);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    d.extra_w = w.sh_gate;
  }
  e = launch_grouped(d, max_tiles, stream, sh_q8);
  if (e != hipSuccess) return e;

  hipLaunchKernelGGL(combine_kernel, dim3(grid_for(T * (H / 8), 256)), dim3(256), 0, stream, w.ys, w.ye, w.inv, T,
                     k, H, L.has_shared, P, Y, out_bf16);
  return hipGetLastError();
}

}  // namespace q4moe

#ifdef Q4MOE_GEMM_STAMPS
// Diagnostic build only: copy the grouped-GEMM workgroup stamps ([4][4096][8] uint64,
// records filled in launch order modulo 4, layout as described above) to host memory.
extern "C" int q4moe_gemm_stamps(void* host, size_t bytes) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(q4moe::g_gemm_stamps), bytes);
}
#endif
