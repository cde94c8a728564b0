// Grouped affine-Q4 GEMM on bf16 matrix cores, and the prefill MoE layer
// built on it (lily-qwen3.8-flash-next README, "How the speed was achieved":
// prefill is compute-bound and runs the expert GEMM over token-to-expert
// groups; "2026-09-02: Lily vs MLX 0.32.2", "Measurement contract": prompts go
// through in 2,048-token chunks).
//
// Exact dequantization on MFMA: the B operand holds the codes as bfloat16
// (128 + q) (common.h), so one 64-column group yields
//   P'[m][n] = sum_j x[m][j] (128 + q[n][j])        (exact products, fp32 sum)
// and the output accumulates scale[n][g] * P'[m][n] per group (one VALU FMA
// per element per group).  The remaining term
//   sum_g (bias - 128*scale)[n][g] * rowsum_g(x)[m]
// is itself a small product over the group index; both factors are split
// exactly into bfloat16 parts (3 for the fp32 row sums, 2 for the offset
// bias, which needs at most 16 significant bits) and fed to the same MFMA
// after the main loop.  No weight is rounded.
//
// Tiling: a workgroup (4 waves) owns 128 rows of one group (expert) and 256
// output columns (or 128 gate + 128 up columns for the SwiGLU epilogue); each
// wave computes 4 x 2 MFMA 32x32 blocks.  The row tile is staged through LDS
// (permuted into the nibble-pair order) with one group of look-ahead; each
// lane loads its own 16 code bytes per group for its column.  Workgroups of
// the same row tile are placed on the same XCD so the row tile stays in that
// XCD's L2.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace q4moe {

namespace {

constexpr int BM = 96;           // rows per tile (3 MFMA row blocks; experts hold ~40-90 rows)
constexpr int MB = BM / 32;
constexpr int BN = 256;          // output columns per tile (store/scale)
constexpr int kXcd = 8;

enum Epi { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_SCALE = 2 };

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

struct GemmParams {
  const uint16_t* A;          // bf16 rows [*][K]
  const uint16_t* xs;         // bf16 [*][3][Gp] row group-sum parts, same row indexing as A
  const int4* tiles;          // per tile {segment (expert; -1 extra; -2 none), first position, rows, 0};
                              // null: tile t covers positions t*BM.. of the extra segment
  int n_tiles;                // table length (the grid may hold a few more tiles)
  const int32_t* row_src;     // gather mode: A row (token) of each routed position; positions >= P read row pos - P
  const float* route_w;       // scale epilogue: routing weight of each routed position
  int gather;
  int64_t P;                  // positions of the routed segments
  int K, G, Gp;
  int bs_vec;                 // 1: every scale/bias row may be read 8 groups (16 bytes) at a time
  int N;                      // output columns (store/scale) or intermediate width (swiglu)
  Q4Mat W, W2;                // routed experts (W2 = up for swiglu), stacked
  int64_t w_codes_stride, w_groups_stride;
  Q4Mat X, X2;                // the extra segment's matrix (shared expert / single matrix)
  int64_t extra_rows;         // positions of the extra segment (uniform tiling when tiles is null)
  int n_slices;
  int epi;
  void* out;
  int out_bf16;
  int64_t ldo;
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// Global-address-space view of a pointer: a generic (flat) load could touch
// LDS, so it would have to wait for every LDS DMA still in flight.
typedef const uint16_t __attribute__((address_space(1)))* gu16_ptr;
__device__ __forceinline__ uint32_t ld_global_u16(const uint16_t* ptr) { return *(gu16_ptr)ptr; }

__device__ __forceinline__ uint4 codes_to_operand(uint32_t w) {
  return make_uint4(nib_pair(w, 0), nib_pair(w, 4), nib_pair(w, 8), nib_pair(w, 12));
}

// s_waitcnt immediate for "at most n vector-memory ops outstanding" (gfx9 encoding,
// expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
// The same with lgkmcnt(0) (all of this wave's LDS reads done).
constexpr int vmcnt_lgkm0_imm(int n) { return vmcnt_imm(n) & ~(0xF << 8); }

// Pipeline depth (K groups in flight) and per-stage vector-memory ops per thread:
// MB A-tile LDS loads, 2 B-code LDS loads, 2 scale loads.
constexpr int kStages = 3;  // the stage arrays below are written out for exactly 3
constexpr int kOpsPerStage = MB + 4;
constexpr int A_STAGE_BYTES = BM * 128;           // BM rows x one 64-column group of bf16
constexpr int B_STAGE_BYTES = 4 * 2 * 64 * 16;    // 4 waves x 2 column blocks x 64 lanes x 16 bytes

// Swizzled slot of (row r, 16-byte word w) in an A stage: the words of a row
// are XOR-rotated by the row's low bits so that 8 consecutive rows reading the
// same word hit 8 different LDS bank groups.
__device__ __forceinline__ int a_slot(int r, int w) { return r * 8 + (w ^ (r & 7)); }

__global__ __launch_bounds__(256, 2) void grouped_q4_gemm_kernel(GemmParams p) {
  // One LDS array per pipeline stage: distinct variables let the compiler see
  // that reading one stage does not depend on the DMA still filling another,
  // so it does not wait for every outstanding load before each LDS read.
  // (The compiler tracks only a few distinct DMA targets, so A and B of a stage share one array.)
  __shared__ __align__(16) uint8_t s_st0[A_STAGE_BYTES + B_STAGE_BYTES], s_st1[A_STAGE_BYTES + B_STAGE_BYTES],
      s_st2[A_STAGE_BYTES + B_STAGE_BYTES];
  auto stage_a = [&](int st) -> uint8_t* { return st == 0 ? s_st0 : st == 1 ? s_st1 : s_st2; };
  auto stage_b = [&](int st) -> uint8_t* { return stage_a(st) + A_STAGE_BYTES; };
  __shared__ int32_t s_src[BM];
  __shared__ float s_wgt[BM];  // routing weight of each tile row (scale epilogue)

  // ---- tile of this workgroup (XCD-aware: all slices of a tile share an XCD)
  const int bid = blockIdx.x;
  const int xcd = bid % kXcd;
  const int q = bid / kXcd;
  const int slice = q % p.n_slices;
  const int tile = (q / p.n_slices) * kXcd + xcd;
  int seg, rows;
  int64_t row0;
  if (tile >= p.n_tiles) return;
  if (p.tiles) {
    const int4 ti = p.tiles[tile];
    seg = ti.x;
    row0 = ti.y;
    rows = ti.z;
  } else {
    row0 = (int64_t)tile * BM;
    seg = row0 < p.extra_rows ? -1 : -2;
    rows = (int)min<int64_t>(BM, p.extra_rows - row0);
  }
  if (seg == -2) return;

  // ---- source row and routing weight of each tile row (padding rows repeat the
  // last real row; their outputs are dropped)
  for (int r = threadIdx.x; r < BM; r += blockDim.x) {
    const int64_t pos = row0 + min(r, rows - 1);
    const bool routed = pos < p.P;
    s_src[r] = p.gather ? (routed ? p.row_src[pos] : (int32_t)(pos - p.P)) : (int32_t)pos;
    s_wgt[r] = p.epi == EPI_SCALE && routed ? p.route_w[pos] : 1.0f;
  }

  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int ln = lane & 31, lh = lane >> 5;
  const bool swiglu = p.epi == EPI_SWIGLU;

  // ---- weight rows (B columns) of this lane: nb = 0, 1
  const Q4Mat& M0 = seg >= 0 ? p.W : p.X;
  const Q4Mat& M1 = seg >= 0 ? (swiglu ? p.W2 : p.W) : (swiglu ? p.X2 : p.X);
  const int64_t oc = seg >= 0 ? seg * p.w_codes_stride : 0;
  const int64_t og = seg >= 0 ? seg * p.w_groups_stride : 0;
  int col[2];
  const uint4* bcodes[2];
  const uint16_t* bscale[2];
  const uint16_t* bbias[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    col[nb] = swiglu ? slice * 128 + wave * 32 + ln : slice * BN + wave * 64 + nb * 32 + ln;
    const int64_t wrow = min(col[nb], p.N - 1);
    const Q4Mat& Mx = nb == 0 ? M0 : M1;
    bcodes[nb] = reinterpret_cast<const uint4*>(Mx.codes + oc + wrow * (p.K >> 3)) + lh;
    bscale[nb] = Mx.scales + og + wrow * p.G;
    bbias[nb] = Mx.biases + og + wrow * p.G;
  }
  __syncthreads();  // s_src ready

  // ---- A-tile loads of this thread: MB instructions, rows (wave*MB+i)*8 + lane/8, swizzled word
  const uint16_t* a_ptr[MB];
  int a_word[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int r = (wave * MB + i) * 8 + (lane >> 3);
    a_word[i] = (lane & 7) ^ (r & 7);
    a_ptr[i] = p.A + (int64_t)s_src[r] * p.K + a_word[i] * 8;
  }

  // Issue all loads of K group g into stage `st` (groups past the end repeat the last one).
  auto issue = [&](int g, int st, uint32_t (&sc)[2]) {
    g = min(g, p.G - 1);
#pragma unroll
    for (int i = 0; i < MB; ++i)
      __builtin_amdgcn_global_load_lds(a_ptr[i] + g * 64, stage_a(st) + (wave * MB + i) * 1024, 16, 0, 0);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      __builtin_amdgcn_global_load_lds(bcodes[nb] + 2 * g, stage_b(st) + (wave * 2 + nb) * 1024, 16, 0, 0);
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
#pragma unroll
  for (int st = 0; st < kStages - 1; ++st) issue(st, st, sc[st]);

  // The main loop is specialised on the number of active row blocks so that a
  // group's body has no branches: every wait the compiler adds then sits at a
  // use of the data, not at a join right after the look-ahead loads.
  auto main_loop = [&](auto nmb_c) __attribute__((always_inline)) {
    constexpr int NMB = decltype(nmb_c)::value;
    // One K group from stage ST (a compile-time stage, so each LDS access names one array).
    auto step = [&](int g, auto st_c) __attribute__((always_inline)) {
      constexpr int st = decltype(st_c)::value;
      constexpr int sn = (st + kStages - 1) % kStages;
      // keep each group's instructions (notably the scale conversions) inside its own step
      __builtin_amdgcn_sched_barrier(0);
      // Group g has landed for this wave and this wave's reads of the stage about
      // to be refilled are done; the barrier extends both to every wave.  (A
      // workgroup fence here would also wait for the look-ahead DMA.)
      __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(kOpsPerStage * (kStages - 2)));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);

      const uint8_t* sa = stage_a(st);
      const uint8_t* sb = stage_b(st) + wave * 2 * 1024 + lane * 16;
      // This wave's B codes first, then A fragments double-buffered over row
      // blocks: block 0's reads are in flight during the B conversion, block
      // mb+1's during block mb's MFMAs.
      uint4 af[2][4];
      auto read_a = [&](int mb, uint4 (&dst)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
          dst[s4] = *reinterpret_cast<const uint4*>(sa + a_slot(mb * 32 + ln, 4 * lh + s4) * 16);
      };
      const uint4 rb0 = *reinterpret_cast<const uint4*>(sb);
      const uint4 rb1 = *reinterpret_cast<const uint4*>(sb + 1024);
      read_a(0, af[0]);
      issue(g + kStages - 1, sn, sc[sn]);  // the look-ahead group, after this step's LDS reads
      bf16x8_t bop[2][4];  // this group's B operands, converted once, used by every row block
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        bop[0][s4] = as_bf16x8(codes_to_operand(s4 == 0 ? rb0.x : s4 == 1 ? rb0.y : s4 == 2 ? rb0.z : rb0.w));
        bop[1][s4] = as_bf16x8(codes_to_operand(s4 == 0 ? rb1.x : s4 == 1 ? rb1.y : s4 == 2 ? rb1.z : rb1.w));
      }
      const float scale0 = bf16_bits_to_f32(sc[st][0]), scale1 = bf16_bits_to_f32(sc[st][1]);
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        if (mb + 1 < NMB) read_a(mb + 1, af[(mb + 1) & 1]);
        // two independent chains (one per column block) over the group's 4 K-steps, then the fold
        f32x16_t p0 = zero16, p1 = zero16;
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          p0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af[mb & 1][s4]), bop[0][s4], p0, 0, 0, 0);
          p1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af[mb & 1][s4]), bop[1][s4], p1, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          acc[mb][0][i] = fmaf(scale0, p0[i], acc[mb][0][i]);
          acc[mb][1][i] = fmaf(scale1, p1[i], acc[mb][1][i]);
        }
      }
    };
    static_assert(kStages == 3, "the steps below are written out for three stages");
    int g0 = 0;
    for (; g0 + kStages <= p.G; g0 += kStages) {
      step(g0, std::integral_constant<int, 0>{});
      step(g0 + 1, std::integral_constant<int, 1>{});
      step(g0 + 2, std::integral_constant<int, 2>{});
    }
    // the last G mod 3 groups
    if (g0 < p.G) step(g0, std::integral_constant<int, 0>{});
    if (g0 + 1 < p.G) step(g0 + 1, std::integral_constant<int, 1>{});
  };
  if (mblocks == 1)
    main_loop(std::integral_constant<int, 1>{});
  else if (mblocks == 2)
    main_loop(std::integral_constant<int, 2>{});
  else
    main_loop(std::integral_constant<int, 3>{});
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // drain the trailing (unused) loads before LDS is released

  // ---- offset/bias term: sum_g (bias - 128 scale)[n][g] * rowsum_g[m], on MFMA with exact bf16 parts.
  // Each 16-group slice takes one round of loads (the 8 groups' biases and scales of this lane's
  // column, 16 bytes each where aligned, and the rows' group-sum parts), issued one slice ahead.
  struct CorrLoads {
    uint4 bias[2], scale[2];  // [nb]: 8 groups' bf16 values
    uint4 xa[MB][3];          // [mb][part]: 8 groups' bf16 row-sum parts
  };
  auto corr_load = [&](int t, CorrLoads& L) __attribute__((always_inline)) {
    const int gbase = t * 16 + 8 * lh;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      if (p.bs_vec) {
        const bool any = gbase < p.G;  // with G % 8 == 0 a slice half is all real groups or all padding
        L.bias[nb] = any ? *reinterpret_cast<const uint4*>(bbias[nb] + gbase) : make_uint4(0, 0, 0, 0);
        L.scale[nb] = any ? *reinterpret_cast<const uint4*>(bscale[nb] + gbase) : make_uint4(0, 0, 0, 0);
      } else {
        uint32_t bv[8], sv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int g = min(gbase + j, p.G - 1);  // padding groups: loaded clamped, zeroed
          bv[j] = gbase + j < p.G ? ld_global_u16(bbias[nb] + g) : 0u;
          sv[j] = gbase + j < p.G ? ld_global_u16(bscale[nb] + g) : 0u;
        }
        L.bias[nb] = make_uint4(bv[0] | bv[1] << 16, bv[2] | bv[3] << 16, bv[4] | bv[5] << 16, bv[6] | bv[7] << 16);
        L.scale[nb] = make_uint4(sv[0] | sv[1] << 16, sv[2] | sv[3] << 16, sv[4] | sv[5] << 16, sv[6] | sv[7] << 16);
      }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (mb >= mblocks) continue;
      const uint16_t* xr = p.xs + (int64_t)s_src[mb * 32 + ln] * 3 * p.Gp + gbase;
#pragma unroll
      for (int part_i = 0; part_i < 3; ++part_i) L.xa[mb][part_i] = *reinterpret_cast<const uint4*>(xr + part_i * p.Gp);
    }
  };
  auto corr_apply = [&](const CorrLoads& L) __attribute__((always_inline)) {
    uint4 bc[2][2];  // [nb][hi/lo]
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const uint32_t bw[4] = {L.bias[nb].x, L.bias[nb].y, L.bias[nb].z, L.bias[nb].w};
      const uint32_t sw[4] = {L.scale[nb].x, L.scale[nb].y, L.scale[nb].z, L.scale[nb].w};
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t bj = (bw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu, sj = (sw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
        const float c = bf16_bits_to_f32(bj) - 128.0f * bf16_bits_to_f32(sj);  // padding groups: 0 - 0
        hi[j] = f32_to_bf16_bits(c);
        lo[j] = f32_to_bf16_bits(c - bf16_bits_to_f32(hi[j]));
      }
      bc[nb][0] = make_uint4(hi[0] | hi[1] << 16, hi[2] | hi[3] << 16, hi[4] | hi[5] << 16, hi[6] | hi[7] << 16);
      bc[nb][1] = make_uint4(lo[0] | lo[1] << 16, lo[2] | lo[3] << 16, lo[4] | lo[5] << 16, lo[6] | lo[7] << 16);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (mb >= mblocks) continue;
#pragma unroll
      for (int part_i = 0; part_i < 3; ++part_i)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int hl = 0; hl < 2; ++hl)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(L.xa[mb][part_i]), as_bf16x8(bc[nb][hl]),
                                                                 acc[mb][nb], 0, 0, 0);
    }
  };
  {
    const int nt = (p.Gp + 15) / 16;
    CorrLoads cur, nxt;
    corr_load(0, cur);
    for (int t = 0; t < nt; ++t) {
      if (t + 1 < nt) corr_load(t + 1, nxt);
      corr_apply(cur);
      cur = nxt;
    }
  }

  // ---- epilogue.  D layout: column = lane % 32, row = 8*(i/4) + 4*(lane/32) + i%4.
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    if (mb >= mblocks) continue;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = mb * 32 + 8 * (i >> 2) + 4 * lh + (i & 3);
      if (r >= rows) continue;
      const int64_t pos = row0 + r;
      if (swiglu) {
        if (col[0] < p.N) {
          // activations are written in the permuted 8-column order the next GEMM's A operand uses
          const int c = col[0], j = c & 7;
          const int pc = (c & ~7) | (j < 4 ? 2 * j : 2 * (j - 4) + 1);
          const float a = silu(acc[mb][0][i]) * acc[mb][1][i];
          reinterpret_cast<uint16_t*>(p.out)[pos * p.ldo + pc] = (uint16_t)f32_to_bf16_bits(a);
        }
      } else {
        const float wgt = s_wgt[r];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          if (col[nb] >= p.N) continue;
          const float v = wgt * acc[mb][nb][i];
          if (p.out_bf16)
            reinterpret_cast<uint16_t*>(p.out)[pos * p.ldo + col[nb]] = (uint16_t)f32_to_bf16_bits(v);
          else
            reinterpret_cast<float*>(p.out)[pos * p.ldo + col[nb]] = v;
        }
      }
    }
  }
}

// Per-row, per-64-column-group sums of a bf16 matrix, split exactly into three
// bfloat16 parts: sums[r][part][g] (groups padded with zeros to Gp).  When `ap`
// is given, also writes the rows with each 8-column block permuted into the
// (x0,x4),(x1,x5),(x2,x6),(x3,x7) pair order the MFMA A operand uses.
__global__ void prep_rows_kernel(const uint16_t* __restrict__ A, int64_t rows, int K, int Gp,
                                 uint16_t* __restrict__ sums, uint16_t* __restrict__ ap) {
  const int G = K >> 6;
  const int64_t total = rows * Gp;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / Gp;
    const int g = (int)(i - r * Gp);
    float s = 0.f;
    if (g < G) {
      const uint4* src = reinterpret_cast<const uint4*>(A + r * K + g * 64);
      uint4* dst = ap ? reinterpret_cast<uint4*>(ap + r * K + g * 64) : nullptr;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint4 v = src[j];
        s += (bf16_bits_to_f32(v.x & 0xFFFFu) + bf16_bits_to_f32(v.x >> 16)) +
             (bf16_bits_to_f32(v.y & 0xFFFFu) + bf16_bits_to_f32(v.y >> 16)) +
             (bf16_bits_to_f32(v.z & 0xFFFFu) + bf16_bits_to_f32(v.z >> 16)) +
             (bf16_bits_to_f32(v.w & 0xFFFFu) + bf16_bits_to_f32(v.w >> 16));
        if (dst) dst[j] = permute_block(v);
      }
    }
    const uint32_t h = f32_to_bf16_bits(s);
    const float r1 = s - bf16_bits_to_f32(h);
    const uint32_t m = f32_to_bf16_bits(r1);
    const uint32_t l = f32_to_bf16_bits(r1 - bf16_bits_to_f32(m));
    uint16_t* o = sums + r * 3 * Gp + g;
    o[0] = (uint16_t)h;
    o[Gp] = (uint16_t)m;
    o[2 * Gp] = (uint16_t)l;
  }
}

// Y[t] = Ys[P + t] (shared expert, weight already 1) + sum_slot Ys[inv[t*k + slot]], fixed slot order.
__global__ void combine_kernel(const float* __restrict__ Ys, const int32_t* __restrict__ inv, int64_t T, int k,
                               int H, int has_shared, int64_t P, void* __restrict__ Y, int out_bf16) {
  const int H4 = H >> 2;
  const int64_t total = T * H4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / H4;
    const int c = (int)(i - t * H4);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (has_shared) acc = reinterpret_cast<const float4*>(Ys + (P + t) * H)[c];
    for (int j = 0; j < k; ++j) {
      const float4 v = reinterpret_cast<const float4*>(Ys + (int64_t)inv[t * k + j] * H)[c];
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    if (out_bf16) {
      uint2 o;
      o.x = f32_to_bf16_bits(acc.x) | (f32_to_bf16_bits(acc.y) << 16);
      o.y = f32_to_bf16_bits(acc.z) | (f32_to_bf16_bits(acc.w) << 16);
      reinterpret_cast<uint2*>(static_cast<uint16_t*>(Y) + t * H)[c] = o;
    } else {
      reinterpret_cast<float4*>(static_cast<float*>(Y) + t * H)[c] = acc;
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

hipError_t launch_grouped(GemmParams& p, int64_t max_tiles, hipStream_t stream) {
  p.bs_vec = p.G % 8 == 0;
  for (const Q4Mat* m : {&p.W, &p.W2, &p.X, &p.X2})
    if (m->scales && (!aligned16(m->scales) || !aligned16(m->biases))) p.bs_vec = 0;
  p.n_tiles = (int)max_tiles;
  const int64_t tiles_rounded = (max_tiles + kXcd - 1) / kXcd * kXcd;
  const int64_t blocks = tiles_rounded * p.n_slices;
  hipLaunchKernelGGL(grouped_q4_gemm_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

// Row sums (and, with ap, the permuted copy) of `rows` bf16 rows of length K.
hipError_t launch_prep_rows(const uint16_t* A, int64_t rows, int K, uint16_t* sums, uint16_t* ap,
                            hipStream_t stream) {
  const int Gp = pad16(K >> 6);
  hipLaunchKernelGGL(prep_rows_kernel, dim3(grid_for(rows * Gp, 256)), dim3(256), 0, stream, A, rows, K, Gp, sums,
                     ap);
  return hipGetLastError();
}

}  // namespace

size_t gemm_workspace_bytes(int64_t m, int k) {
  return align256((size_t)m * 3 * pad16(k / 64) * 2) + align256((size_t)m * k * 2);
}

hipError_t run_q4_gemm(const Q4Mat& W, int64_t n, int k, const uint16_t* X, int64_t m, void* Y, int out_bf16,
                       void* ws, hipStream_t stream) {
  uint16_t* xs = static_cast<uint16_t*>(ws);
  uint16_t* xp = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + align256((size_t)m * 3 * pad16(k / 64) * 2));
  hipError_t e = launch_prep_rows(X, m, k, xs, xp, stream);
  if (e != hipSuccess) return e;
  GemmParams p{};
  p.A = xp;
  p.xs = xs;
  p.gather = 0;
  p.P = 0;
  p.K = k;
  p.G = k / 64;
  p.Gp = pad16(p.G);
  p.N = (int)n;
  p.X = W;
  p.X2 = W;
  p.extra_rows = m;
  p.n_slices = (int)((n + BN - 1) / BN);
  p.epi = EPI_STORE;
  p.out = Y;
  p.out_bf16 = out_bf16;
  p.ldo = n;
  return launch_grouped(p, (m + BM - 1) / BM, stream);
}

namespace {
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
  uint16_t* xs_x;
  uint16_t* xp;
  uint16_t* act;
  uint16_t* xs_act;
  float* ys;
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
  w.xs_x = reinterpret_cast<uint16_t*>(take((size_t)T * 3 * pad16(H / 64) * 2));
  w.xp = reinterpret_cast<uint16_t*>(take((size_t)T * H * 2));
  w.act = reinterpret_cast<uint16_t*>(take((size_t)R * I * 2));
  w.xs_act = reinterpret_cast<uint16_t*>(take((size_t)R * 3 * pad16(I / 64) * 2));
  w.ys = reinterpret_cast<float*>(take((size_t)R * H * 4));
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
  hipError_t e = run_route_topk(L.router, E, H, X, T, k, w.ids, w.weights, w.logits, stream);
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
  e = run_permute(w.ids, P, E, w.offsets, w.sorted_rows, w.inv, w.perm_ws, &gt, stream);
  if (e != hipSuccess) return e;
  e = launch_prep_rows(X, T, H, w.xs_x, w.xp, stream);
  if (e != hipSuccess) return e;

  // gate/up with SwiGLU -> act (bf16, sorted positions; shared rows appended)
  GemmParams p{};
  p.A = w.xp;
  p.xs = w.xs_x;
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
  p.out = w.act;
  p.out_bf16 = 1;
  p.ldo = I;
  e = launch_grouped(p, max_tiles, stream);
  if (e != hipSuccess) return e;

  const int64_t R = P + extra;
  e = launch_prep_rows(w.act, R, I, w.xs_act, nullptr, stream);
  if (e != hipSuccess) return e;

  // down with the routing weight -> ys (fp32, sorted positions)
  GemmParams d = p;
  d.A = w.act;
  d.xs = w.xs_act;
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
  d.n_slices = (H + BN - 1) / BN;
  d.epi = EPI_SCALE;
  d.out = w.ys;
  d.out_bf16 = 0;
  d.ldo = H;
  e = launch_grouped(d, max_tiles, stream);
  if (e != hipSuccess) return e;

  hipLaunchKernelGGL(combine_kernel, dim3(grid_for(T * (H / 4), 256)), dim3(256), 0, stream, w.ys, w.inv, T, k, H,
                     L.has_shared, P, Y, out_bf16);
  return hipGetLastError();
}

}  // namespace q4moe
