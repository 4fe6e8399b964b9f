// Internal interface between the C ABI layer (moe_api.cpp) and the gfx950
// kernels.  Every launch_* function only enqueues on the given stream and
// returns the launch status; shape checks happen in moe_api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kMaxExperts = 64;

// ---- device helpers ------------------------------------------------------

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 bits, round to nearest even, NaN kept quiet.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---- packed weight layout -------------------------------------------------
//
// A projection W[e][K][N] (K = reduction dim, N = output dim) is stored as
// 1 KiB blocks, one per (expert, 16-column tile nb, K unit u, stream g):
//   block index ((e * NB + nb) * U + u) * G + g,   NB = N / 16
// Inside a block, lane l (0..63) owns 16 contiguous bytes holding column
// n = nb*16 + (l & 15):
//   bf16 (U = K/32): element j (0..7) is k = u*32 + 8*(l >> 4) + j
//   int8 (U = K/64): byte j (0..15) is  k = u*64 + 32*(j >> 3) + 8*(l >> 4) + (j & 7)
//   int4 (U = K/128): value j (0..31) is k = u*128 + 32*(j >> 3) + 8*(l >> 4) + (j & 7),
//                    holding q + 8 in dword j >> 3 at bit 8*(j & 3) + 4*((j >> 2) & 1)
//   fp8 (as int8, one E4M3 code per byte)
//   MXFP4 (as int4, U = K/128): value j's E2M1 code in dword j >> 3 at bit
//                    8*((j & 7) >> 1) + 4*(j & 1); and per (expert, tile, unit,
//                    stream) a block of 16 scale dwords, dword c holding the E8M0
//                    exponents of column nb*16 + c for the unit's four 32-k steps
//                    (byte h: step h)
// which is the B-operand order of v_mfma_f32_16x16x32_bf16.  A wave loading
// one unit reads 1 KiB of contiguous memory: eight full 128-byte lines.
// G = 2 interleaves the SwiGLU gate (g = 0) and up (g = 1) matrices so one
// stream of a column tile carries both.

constexpr int kUnitBytes = 1024;

// qb: weight kind, 0 (bf16), 8 (int8), 9 (fp8), 4 (int4) or 5 (MXFP4).
inline size_t packed_bytes(int E, int K, int N, int G, int qb) {
  const size_t units = (size_t)K / (qb >= 8 ? 64 : (qb >= 4 ? 128 : 32));
  return (size_t)E * (size_t)(N / 16) * units * (size_t)G * kUnitBytes;
}
// Bytes of an MXFP4 projection's packed block scales.
inline size_t packed_mx_scale_bytes(int E, int K, int N, int G) {
  return (size_t)E * (size_t)(N / 16) * (size_t)(K / 128) * (size_t)G * 64;
}

hipError_t launch_pack_bf16(const uint16_t* src, void* dst, int E, int K, int N, int G, int g, hipStream_t s);
// Packed MXFP4 weights (and their packed block scales) of E experts -> the
// packed bf16 layout, exactly; experts without rows skipped when offsets
// ([E+1], device) is given.  dst holds packed_bytes(E, K, N, G, 0).
hipError_t launch_expand_fp4(const void* w, const uint32_t* scales, void* dst, const int32_t* offsets, int E, int K,
                             int N, int G, hipStream_t s);
hipError_t launch_pack_i8(const int8_t* src, void* dst, int E, int K, int N, int G, int g, hipStream_t s);
// int4 values held one per int8 (in [-8, 7]), packed two per byte.
hipError_t launch_pack_i4(const int8_t* src, void* dst, int E, int K, int N, int G, int g, hipStream_t s);
// MXFP4: E2M1 codes one per byte [E][K][N] into the packed nibble layout, and
// E8M0 exponents [E][K/32][N] into the packed scale blocks.
hipError_t launch_pack_fp4(const uint8_t* src, void* dst, int E, int K, int N, int G, int g, hipStream_t s);
hipError_t launch_pack_mx_scales(const uint8_t* src, void* dst, int E, int K, int N, int G, int g, hipStream_t s);

// ---- routing ---------------------------------------------------------------

// Neighbouring ops done by the routing pass (DeepSpeed-Inference summary,
// section 4: the layer norm before the intermediate GeMM; the residual add).
struct RouteFuse {
  int norm;              // 0: none; 1: layer norm; 2: RMS norm of each x row
  const float* gamma;    // [m]
  const float* beta;     // [m] or null (layer norm only)
  float eps;
  void* xn;              // with a norm: the normalised rows [T][m] in x's dtype (routed and returned)
  const void* residual;  // or null: the accumulator starts from it instead of zero ([T][ym])
  int res_bf16;          // residual dtype: bf16 (1) or fp32 (0)
  int quant;             // 8-bit activations: 0 none, 1 E4M3, 2 int8 (bf16 rows only)
  uint16_t* xq;          // with quant: the (normalised) rows quantised, as bf16 values [T][m], or null
  uint8_t* xc;           // with quant: their codes [T][m], or null
  float* xs;             // with quant: each row's scale [T]
};

// yacc (optional): fp32 [T][ym] accumulator that the routing pass zeroes (or
// fills with fuse->residual).  With fuse->norm the routing uses, and writes to
// fuse->xn, the normalised rows: inside the staged router, else by a row-norm
// kernel first.  With fuse->quant the experts' input rows (normalised ones
// with a norm) are also quantised to 8 bits, per row, as launch_quant_rows
// does: inside the staged router from its LDS copy of the rows, else by that
// kernel after the routing.
hipError_t launch_route_topk(const void* x, bool x_bf16, const float* wg, const float* bias, int T, int m, int E,
                             int k, bool logits_in, float* logits, int32_t* idx, float* w, float* yacc, int ym,
                             hipStream_t s, const RouteFuse* fuse = nullptr);

hipError_t launch_dispatch(const int32_t* idx, int n, int E, int32_t* counts, int32_t* offsets, int32_t* perm,
                           int32_t* inv_perm, hipStream_t s);

// ---- expert FFN, skinny (decode-sized) path ----------------------------------

enum SkinnyEpilogue {
  EPI_UP_SWIGLU = 0,  // H = bf16(SiLU(g) * u), two streams
  EPI_UP_RELU = 1,    // H = bf16(max(g, 0)),  one stream
  EPI_DOWN_ACC = 2,   // y_acc[t] += w * o  (fp32 atomics)
  EPI_DOWN_ROWS = 3,  // y_perm[r] = o     (fp32 rows)
};

struct SkinnyArgs {
  const void* w;           // packed weights of this projection
  const float* scale0;     // int8/int4/fp8: per-column scales of stream 0 [E][N]
  const float* scale1;     // int8/int4/fp8: per-column scales of stream 1 [E][N]
  const uint32_t* mx;      // MXFP4: the projection's packed block scales
  const uint16_t* act;     // bf16 activations: x [T][K] (gather) or H [T*k][K]
  const int32_t* perm;     // [T*k] dispatch permutation (input unless topk_idx is set)
  const int32_t* offsets;  // [E+1] dispatch offsets (input unless topk_idx is set)
  const int32_t* topk_idx; // [T*k] or null: derive the dispatch in the prologue
  int32_t* d_counts;       // with topk_idx: dispatch outputs published by logical block 0
  int32_t* d_offsets;
  int32_t* d_perm;
  int32_t* d_inv;
  const float* topk_w;     // [T*k] (EPI_DOWN_ACC)
  uint16_t* h_out;         // [T*k][N] bf16 (up epilogues)
  float* f_out;            // y_acc [T][N] or y_perm [T*k][N]
  int K, N, E, topk, T;
  int gather;              // 1: activation row = perm[r] / topk, 0: row r
  int W;                   // upper bound on (expert, row-chunk) pairs
  int ksplit;              // reduction slices per work item (EPI_DOWN_ACC only)
  int max_rows;            // > 0: experts with more rows are skipped (another kernel serves them)
  int min_rows;            // > 0: experts with at most this many rows are skipped
  int packed;              // 1: act is in the packed row layout (moe_index.hpp), no gather
  int h_packed;            // 1: the up epilogue writes H in the packed row layout
  size_t slice_stride;     // EPI_DOWN_ROWS with ksplit > 1: elements between the slices' rows
  int shared_act;          // 1: each workgroup copies a unit's activation fragments once into LDS
                           //    for all its waves (packed rows, columns split over the waves)
};

// Largest T*k for which the decode FFN (or the row packing before it) derives
// the dispatch itself.
constexpr int kFusedDispatchMax = 4096;

// Rows per work item for a given M-tile count (16 rows per tile).
inline int skinny_rows(int mt) { return 16 * mt; }

// mt: 16-row M tiles per work item (1, 2, 4; 12 for bf16 weights with shared
// activations, ct <= 2 and one column tile for SwiGLU); ct: 16-column tiles
// per wave sharing each activation load (1, 2, 4); qb: weight bits (0 bf16,
// 8 int8, 4 int4; the integer kinds take at most two M tiles).
// splitk: the four waves of a workgroup split the reduction (partials summed
// through LDS); otherwise each wave owns its column tiles over the whole range.
hipError_t launch_ffn_skinny(const SkinnyArgs& a, int epi, int qb, int mt, int ct, bool splitk, hipStream_t s);

// A projection split by expert size in one launch: `narrow` (four M tiles)
// for the experts it admits and `wide` (twelve M tiles) for the others, both
// with one column tile per wave for SwiGLU and two otherwise; bf16 weights,
// packed rows, shared activations, no split K.
hipError_t launch_ffn_skinny_split(const SkinnyArgs& narrow, const SkinnyArgs& wide, int epi, hipStream_t s);

// ---- expert FFN, grouped GEMM (prefill-sized) path ----------------------------

// Grouped GEMM over packed operands.  Activations and the hidden rows it
// writes are in the packed row layout of moe_index.hpp (16-row x 32-k
// fragments, each expert starting on a 16-row boundary).
struct GemmArgs {
  const void* w;           // packed weights of this projection (bf16, int8, fp8, int4 or MXFP4)
  const float* scale0;     // int8/int4/fp8 weights: per-column scales [E][N] (gate, or the only stream)
  const float* scale1;     // int8/int4/fp8 SwiGLU weights: the up stream's scales [E][N]
  const uint32_t* mx;      // MXFP4: the projection's packed block scales
  const uint16_t* act;     // packed bf16 activations [packed rows][K]
  const int32_t* offsets;  // [E+1] dispatch offsets
  uint16_t* h_out;         // packed H [packed rows][N] (up epilogues)
  float* f_out;            // y_perm [T*k][N] in dispatch order (EPI_DOWN_ROWS)
  int cg;                  // column blocks per group of the work order (>= 1)
  int skip_empty;          // 1: skip the products of row fragments past the last real row
  int K, N, E;
  int W;                   // upper bound on (expert, 256-row block) pairs
};

// K a multiple of 64 (and of the weight unit: 64 k for int8, 128 for int4),
// N a multiple of 64; qb: weight bits (0 bf16, 8 int8, 4 int4).  epi:
// EPI_UP_SWIGLU, EPI_UP_RELU or EPI_DOWN_ROWS.
hipError_t launch_ffn_gemm(const GemmArgs& a, int epi, int qb, hipStream_t s);
// Rows per row block (work item) of the grouped GEMM for weight bits qb.
int gemm_rows_per_block(int qb);

// Gathers x rows in dispatch order into the packed row layout.
struct PackArgs {
  const uint16_t* x;       // [T][K] bf16
  const int32_t* perm;     // [T*k] (input unless topk_idx is set)
  const int32_t* offsets;  // [E+1] (input unless topk_idx is set)
  uint16_t* out;           // [packed_rows_alloc(T*k, E)][K] packed
  const int32_t* topk_idx; // [T*k] or null: derive the dispatch here (T*k <= kFusedDispatchMax)
  int32_t* d_counts;       // with topk_idx: dispatch outputs published by workgroup 0
  int32_t* d_offsets;
  int32_t* d_perm;
  int32_t* d_inv;
  int T, K, E, topk;
  int rows;                // > 0: bound on the dispatched rows to pack (else T*topk)
};
hipError_t launch_pack_rows(const PackArgs& a, hipStream_t s);

// ---- fp8 x fp8 grouped GEMM (fp8 weights and fp8 activations) ------------------

// Gathers E4M3 code rows in dispatch order into packed 1 KiB units of 16 rows
// x 64 k (the packed fp8 weights' byte order, rows for columns), each expert
// starting on a 16-row boundary; padding rows are zero.  row_scale receives
// each packed row's token scale (0 for padding rows).
struct PackA8Args {
  const uint8_t* codes;    // [T][K] E4M3 (or int8) codes
  const float* scale;      // [T] per-token power-of-two scales
  const int32_t* perm;     // [T*k]
  const int32_t* offsets;  // [E+1]
  uint8_t* out;            // [packed_rows_alloc(T*k, E)][K] packed units
  float* row_scale;        // [packed_rows_alloc(T*k, E)]
  int T, K, E, topk;
  int rows;                // > 0: bound on the dispatched rows to pack (else T*topk)
};
hipError_t launch_pack_rows_a8(const PackA8Args& a, hipStream_t s);

// The up projection on the fp8 (or, int8 true, the int8) matrix cores:
// packed E4M3 (int8) activation units (act, with row_scale per packed row)
// times packed fp8 (int8) weights (w with scale0/scale1 per column); epi
// EPI_UP_SWIGLU or EPI_UP_RELU; H out as for launch_ffn_gemm.  K a multiple
// of 64, N a multiple of 64.
hipError_t launch_ffn_gemm_a8(const GemmArgs& a, const float* row_scale, int epi, bool int8, hipStream_t s);

// ---- expert FFN, fp32 path ----------------------------------------------------

struct F32Args {
  const float* w1;   // [E][K][N]
  const float* w3;   // [E][K][N] or null (ReLU)
  const float* act;  // x [T][K] (gather) or H [T*k][K]
  const int32_t* perm;
  const int32_t* offsets;
  const float* topk_w;
  float* out;        // H [T*k][N], y_acc [T][N] or y_perm [T*k][N]
  int K, N, E, topk, gather, W;
  int epi;           // EPI_UP_SWIGLU / EPI_UP_RELU / EPI_DOWN_ACC / EPI_DOWN_ROWS
};

hipError_t launch_ffn_f32(const F32Args& a, hipStream_t s);

// ---- combine / elementwise ------------------------------------------------------

// y[t] = sum_j w[t,j] * sum_q y_perm[q][inv[t,j]]: the unweighted expert rows,
// each the sum of `slices` partial rows slice_stride elements apart.
// residual (optional): [T][m] in y's dtype, added to each sum last.
hipError_t launch_combine(const float* y_perm, const int32_t* inv_perm, const float* topk_w, int T, int m, int k,
                          int slices, size_t slice_stride, void* y, bool y_bf16, hipStream_t s,
                          const void* residual = nullptr);
hipError_t launch_fill_zero(float* p, size_t n, hipStream_t s);
// fp8 / int8 activations: each row of x (T rows of m bf16) quantised to E4M3
// (or int8) with a per-row power-of-two scale; xq (if not null) receives the
// quantised values as bf16 (exact), xc (if not null) the codes, xs the
// scales.  m is a multiple of 64.
hipError_t launch_quant_rows(const uint16_t* x, int T, int m, bool int8, uint16_t* xq, uint8_t* xc, float* xs,
                             hipStream_t s);
hipError_t launch_f32_to_bf16(const float* src, uint16_t* dst, size_t n, hipStream_t s);

}  // namespace moe
