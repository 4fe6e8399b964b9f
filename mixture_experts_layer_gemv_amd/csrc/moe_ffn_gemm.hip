// Expert FFN for prefill-sized batches: a grouped GEMM on the matrix cores.
//
// When every expert holds hundreds of rows the FFN is compute-bound (the
// FFN's intensity grows with the batch until the kernel's compute peak is the
// roof: MoE-Lightning note, FFN roofline against batch size), so each weight
// byte is read from HBM about once and reused from LDS and L2.
//
// A workgroup computes a 256-row block of one expert against a 256-column
// block (128 hidden columns of gate and up for SwiGLU) with 2 x 4 waves, two
// per SIMD; each wave owns a 128 x 64 tile: 8 x 4 fragments of
// v_mfma_f32_16x16x32_bf16, 128 fp32 accumulators per lane.
//
// Both operands are packed in HBM as 1 KiB fragments in MFMA operand order
// (lane l's 16 bytes at byte 16 l): the weights once at load time, the
// activations by k_pack_rows (the rows gathered through the dispatch
// permutation, for the up projection) or by the up projection's epilogue
// (the hidden rows, for the down projection).  Gathering rows in place
// instead (16 rows x 64 bytes per copy, rows a multiple of 4 KiB apart)
// halves the copy rate.  Fragments stream through a 4-stage LDS ring of
// 32 KiB stages (32 k each), copied global -> LDS
// with global_load_lds_dwordx4 (lane l of a copy lands at base + 16 l): each
// copy is one contiguous 1 KiB read, and each wave reads a fragment with one
// conflict-free 16-byte ds_read per lane.  The two waves of each SIMD take
// turns: one multiplies the stage it holds in registers while the other reads
// its next stage and issues copies (ping-pong, two barriers per step); three
// to four stages of copies stay in flight.
// Workgroups run expert by expert, in groups of A.cg (2) column blocks x all
// of the expert's row blocks, on one XCD at a time: the ~32 resident
// workgroups (about two groups) then read ~8 activation tiles and ~4 weight
// tiles per stage, the rest hits in L2.  The grid is the host's upper bound
// on the items (the host never reads the expert counts).  The up
// projections deal each XCD an equal share of the real items, counted from
// the offsets (xcd_item), then padding: cut into eight equal parts of the
// grid instead, the padding at the end of the work order fell on the last
// XCD, which then idled for the last ~40 % of the Mixtral prefill up
// projection's ~30 rounds (3 % slower).  The down projection, ~4 rounds,
// keeps the equal parts of the grid (xcd_logical): dealing its real items
// evenly measured ~1 % slower.
//
// Measured on the Mixtral-shaped prefill layer (T = 8192), the up
// projection keeps the matrix pipe busy ~80 % of its active cycles, at
// ~1.67 GHz: with copies, LDS reads and products all running, the clock
// drops from 2.4 GHz, and a variant that only copies took three quarters of
// the kernel's time.
#include <type_traits>

#include "moe_convert.hpp"
#include "moe_dispatch_block.hpp"
#include "moe_index.hpp"
#include "moe_lds.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
// SiLU with the hardware exponential and reciprocal (a few ulp of fp32,
// far inside the bf16 rounding of H).
__device__ __forceinline__ float silu_fast(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Tile shape of one weight kind.  A stage holds one 16-byte weight unit of
// K (32 k for bf16, 64 for int8, 128 for int4: the packed weight layout's
// unit) for the workgroup's 256 weight columns, and the matching activation
// fragments of its BM rows.  int4 takes 128-row blocks so that a stage stays
// at 48 KiB (three fit the LDS): its weights are a quarter of bf16's bytes,
// so the halved weight reuse costs less than a shallower ring would.
template <int QB>
struct GemmShape {
  static constexpr int AH = q_ah(QB);            // 32-k activation fragments per row fragment and stage
  static constexpr int BM = q_bits(QB) == 4 ? 128 : 256;  // rows per workgroup
  static constexpr int MF = BM / 32;             // row fragments per wave (two wave rows)
  static constexpr int NAF = BM / 16 * AH;       // activation fragments per stage
  static constexpr int NBF = 16;                 // weight fragments per stage
  static constexpr int STAGE_KB = NAF + NBF;     // KiB per stage
  // ring depth: 4 stages of 32 KiB for bf16 (measured ahead of 5, which
  // fills the LDS, and of 3: 3.24 against 3.32 and 3.38 ms for the Mixtral
  // prefill up projection); 3 of 48 KiB for int8 and int4
  static constexpr int STAGES = QB == 0 ? 4 : 160 / STAGE_KB;
  static constexpr int CPA = NAF / 8;            // activation copies per wave and stage
  static constexpr int CPB = NBF / 8;            // weight copies per wave and stage
  static constexpr int CPS = CPA + CPB;          // copies per wave and stage
};

constexpr int kWR = 2;       // wave rows
constexpr int kWC = 4;       // wave columns
constexpr int kWaves = kWR * kWC;
constexpr int kNF = 4;       // column fragments per wave (64 weight columns)
constexpr int kFrag = 1024;  // bytes of one 64-lane x 16-byte fragment

// acc += a * b on the matrix cores, accumulating in place.  Written as
// inline assembly because the compiler otherwise gives each product a fresh
// destination and copies the accumulators around the loop, which doubles
// their register footprint.  An accumulator is reused only 16 or more
// products later, so consecutive products carry no dependence.
__device__ __forceinline__ void mfma_acc(floatx4_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

// The same for a product whose weight operand a vector instruction has just
// written (the integer kinds' conversion): a matrix instruction reading a
// register that a vector ALU instruction wrote needs two wait states, which
// the compiler does not insert for inline assembly.
__device__ __forceinline__ void mfma_acc_fresh(floatx4_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

// Ties an accumulator to the surrounding statements in its register file.
__device__ __forceinline__ void acc_tie(floatx4_t& acc) {
  asm volatile("" : "+v"(acc));
}

// The compiler cannot see that the assembly above is a matrix instruction,
// so the required gaps between ordinary vector instructions and products
// that touch the same registers are inserted here: before the first product
// (the accumulators were just zeroed) and after the last (the epilogue reads
// them; a 16x16x32 product needs fewer than 32 wait states).  The empty
// statements tie every accumulator to the gap so no access moves across it.
template <int MF, int NF>
__device__ __forceinline__ void mfma_fence_in(floatx4_t (&acc)[MF][NF], floatx4_t& accx) {
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j) acc_tie(acc[i][j]);
  acc_tie(accx);
  asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
}
template <int MF, int NF>
__device__ __forceinline__ void mfma_fence_out(floatx4_t (&acc)[MF][NF], floatx4_t& accx) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j) acc_tie(acc[i][j]);
  acc_tie(accx);
}

// H's zero row block (row block zrb of the packed H, N columns), 32-column
// fragments f0 .. f0 + nf - 1, written by the first row block of the first
// expert served, so that the down projection can read it in place of the
// row fragments past an expert's last row.
__device__ __forceinline__ void zero_h_block(uint16_t* h, int zrb, int N, int f0, int nf, int lane) {
  for (int f = 0; f < nf; ++f)
    reinterpret_cast<u32x4_t*>(h)[((long long)zrb * (N >> 5) + f0 + f) * 64 + lane] = u32x4_t{0u, 0u, 0u, 0u};
}

// One expert projection tile: BM rows x 256 weight columns over the whole
// reduction.  QB: weight bits (0 bf16, 8 int8, 4 int4); integer weights are
// converted exactly to bf16 after their LDS read (the decode kernels'
// conversions; fp8 takes int8's tile with the E4M3 conversion) and their
// per-column scale is applied in the epilogue; int4's
// storage offset (each weight enters as q + 136) is removed with the rows'
// activation sums, which the four waves of a wave row share out (one row
// fragment each, one extra product per activation fragment).
// SKIP: row fragments past the row block's last real row skip their
// products (the fragment reads still run, so the steady state keeps no branch
// around a load); for layers whose experts hold few rows.
template <int EPI, bool SKIP, int QB>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_ffn_gemm(
    const GemmArgs A) {
  using S = GemmShape<QB>;
  constexpr int G = EPI == EPI_UP_SWIGLU ? 2 : 1;
  constexpr int TPW = kNF / G;  // column tiles per wave
  constexpr int MF = S::MF, AH = S::AH, NAF = S::NAF, CPA = S::CPA, CPB = S::CPB, CPS = S::CPS;
  constexpr int STAGES = S::STAGES;
  constexpr int STAGE_BYTES = S::STAGE_KB * kFrag;
  static_assert(QB != 4 || MF == kWC, "int4 row sums: one row fragment per wave of a wave row");
  static_assert(CPS * (STAGES - 1) <= 63, "vmcnt holds at most 63");
  // stage layout: NAF activation fragments (row fragment rf, 32-k part h at
  // rf * AH + h), then 16 weight fragments (kWC wave columns x kNF fragments)
  __shared__ __attribute__((aligned(1024))) unsigned char ring[STAGES][STAGE_BYTES];
  __shared__ float rowsum_s[QB == 4 ? S::BM : 1];
  const int* const offs_s = A.offsets;  // uniform: scalar loads

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // wave row (BM/2 rows) and wave column; each wave row is one group of four
  // waves, one per SIMD (the ping-pong below)
  const int wm = wave / kWC;
  const int wn = wave % kWC;
  const int NB = A.N / 16;
  const int NBL = (NB + kWC * TPW - 1) / (kWC * TPW);  // column blocks

  int e, mb, nblock;
  const int L = EPI == EPI_DOWN_ROWS ? xcd_logical(blockIdx.x, gridDim.x)
                                     : xcd_item(blockIdx.x, gemm_items(offs_s, A.E, S::BM, NBL), 0);
  if (L < 0 || !gemm_item(offs_s, A.E, S::BM, NBL, A.cg, L, &e, &mb, &nblock)) return;
  const int tile_base = nblock * kWC * TPW;
  const int row0 = offs_s[e] + mb * S::BM;  // first dispatched row
  const int nrows = min(S::BM, offs_s[e + 1] - row0);
  const int prow0 = padded_offset(offs_s, e) + mb * S::BM;  // its packed row
  const int nfrag = (nrows + 15) >> 4;  // packed fragments holding real rows
  // this wave's row fragments that hold real rows (uniform)
  const int nf_w = __builtin_amdgcn_readfirstlane(min(max(nfrag - wm * MF, 0), MF));
  const int zrb = padded_offset(offs_s, A.E) >> 4;  // the zero row block

  // This wave copies activation fragments CPA w .. CPA w + CPA-1 and weight
  // fragments CPB w .. CPB w + CPB-1 of every stage.  Sources are a uniform
  // base that advances one weight unit per stage plus a constant 32-bit byte
  // offset per lane (the packed activations and one projection's packed
  // weights are each under 4 GiB; checked on the host).  Activation
  // fragments past the expert's last row read the zero row block after the
  // last expert's rows instead (their rows are never stored): the matrix
  // cores draw less power on zero operands, which lets the clock rise.
  const int U = A.K / (32 * AH);  // stages (weight units along K)
  const char* const abase = reinterpret_cast<const char*>(A.act);
  const char* const bbase = static_cast<const char*>(A.w);
  uint32_t aoff[CPA], boff[CPB];
#pragma unroll
  for (int j = 0; j < CPA; ++j) {
    const int f = CPA * wave + j;  // activation fragment f: row fragment f / AH, 32-k part f % AH
    const int rb = f / AH < nfrag ? (prow0 >> 4) + f / AH : zrb;
    aoff[j] = (uint32_t)(gemm_a_offset(rb, A.K, lane) + (f % AH) * kFrag);
  }
#pragma unroll
  for (int j = 0; j < CPB; ++j) boff[j] = (uint32_t)gemm_b_offset(e, NB, U, G, tile_base, kNF, CPB * wave + j, lane);

  // LDS byte addresses of this wave's first activation and weight slots
  const uint32_t ring_lds = lds_address(ring);
  const uint32_t a_lds = ring_lds + (uint32_t)(CPA * wave) * kFrag;
  const uint32_t b_lds = ring_lds + (uint32_t)(NAF + CPB * wave) * kFrag;

#define MOE_ISSUE(step)                                                                          \
  do {                                                                                           \
    const char* ab_ = abase + (size_t)(step) * (AH * kFrag);                                     \
    const char* bb_ = bbase + (size_t)(step) * G * kFrag;                                        \
    const uint32_t st_ = (uint32_t)((step) % STAGES) * STAGE_BYTES;                              \
    _Pragma("unroll") for (int j = 0; j < CPA; ++j) copy_frag(ab_, aoff[j], a_lds + st_ + j * kFrag); \
    _Pragma("unroll") for (int j = 0; j < CPB; ++j) copy_frag(bb_, boff[j], b_lds + st_ + j * kFrag); \
  } while (0)

  floatx4_t acc[MF][kNF];
  floatx4_t accx = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};  // int4: activation sums of row fragment wn
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < kNF; ++j) acc[i][j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
  mfma_fence_in(acc, accx);

  // The fragments of one stage, held in registers.  int8 weights stay raw
  // until their products (converted one fragment half at a time, which keeps
  // the 256-row tile's registers under the two-waves-per-SIMD budget); the
  // other kinds are converted when read.
  constexpr bool kLateCvt = QB == 8 || QB == 9;
  struct {
    bf16x8_t a[MF][AH], b[kNF][kLateCvt ? 1 : AH];
    u32x4_t braw[kLateCvt ? kNF : 1];
  } f;
#define MOE_LOAD_B(F, step)                                                                      \
  do {                                                                                           \
    const u32x4_t* st_ = reinterpret_cast<const u32x4_t*>(ring[(step) % STAGES]);                \
    _Pragma("unroll") for (int j = 0; j < kNF; ++j) {                                            \
      const u32x4_t w_ = st_[(NAF + wn * kNF + j) * 64 + lane];                                  \
      if constexpr (kLateCvt) {                                                                  \
        F.braw[j] = w_;                                                                          \
      } else if constexpr (QB == 4) {                                                            \
        _Pragma("unroll") for (int h = 0; h < AH; ++h) F.b[j][h] = u4x8_to_bf16_biased(w_[h]);   \
      } else {                                                                                   \
        F.b[j][0] = as_bf16x8(w_);                                                               \
      }                                                                                          \
    }                                                                                            \
  } while (0)
#define MOE_LOAD_A(F, step)                                                                      \
  do {                                                                                           \
    const u32x4_t* st_ = reinterpret_cast<const u32x4_t*>(ring[(step) % STAGES]);                \
    _Pragma("unroll") for (int i = 0; i < MF; ++i) _Pragma("unroll") for (int h = 0; h < AH; ++h) \
        F.a[i][h] = as_bf16x8(st_[((wm * MF + i) * AH + h) * 64 + lane]);                        \
  } while (0)
#define MOE_MMA(F)                                                                               \
  if constexpr (QB == 8) {                                                                       \
    /* int8: the four weight fragments converted before their products */                       \
    _Pragma("unroll") for (int h = 0; h < AH; ++h) {                                             \
      bf16x8_t bw_[kNF];                                                                         \
      _Pragma("unroll") for (int j = 0; j < kNF; ++j)                                            \
        bw_[j] = h == 0 ? i8x8_to_bf16(F.braw[j][0], F.braw[j][1])                               \
                        : i8x8_to_bf16(F.braw[j][2], F.braw[j][3]);                              \
      _Pragma("unroll") for (int i = 0; i < MF; ++i) {                                           \
        _Pragma("unroll") for (int j = 0; j < kNF; ++j) {                                        \
          if (!SKIP || i < nf_w) {                                                               \
            if (i == 0)                                                                          \
              mfma_acc_fresh(acc[i][j], F.a[i][h], bw_[j]);                                      \
            else                                                                                 \
              mfma_acc(acc[i][j], F.a[i][h], bw_[j]);                                            \
          }                                                                                      \
        }                                                                                        \
      }                                                                                          \
    }                                                                                            \
  } else if constexpr (kLateCvt) {                                                               \
    /* fp8: each weight fragment converted just before its products */                          \
    _Pragma("unroll") for (int h = 0; h < AH; ++h) {                                             \
      _Pragma("unroll") for (int j = 0; j < kNF; ++j) {                                          \
        const bf16x8_t bw_ = QB == 9 ? (h == 0 ? fp8x8_to_bf16(F.braw[j][0], F.braw[j][1])       \
                                               : fp8x8_to_bf16(F.braw[j][2], F.braw[j][3]))      \
                                     : (h == 0 ? i8x8_to_bf16(F.braw[j][0], F.braw[j][1])        \
                                               : i8x8_to_bf16(F.braw[j][2], F.braw[j][3]));      \
        _Pragma("unroll") for (int i = 0; i < MF; ++i) {                                         \
          if (!SKIP || i < nf_w) {                                                               \
            if (i == 0)                                                                          \
              mfma_acc_fresh(acc[i][j], F.a[i][h], bw_);                                         \
            else                                                                                 \
              mfma_acc(acc[i][j], F.a[i][h], bw_);                                               \
          }                                                                                      \
        }                                                                                        \
      }                                                                                          \
    }                                                                                            \
  } else {                                                                                       \
    _Pragma("unroll") for (int h = 0; h < AH; ++h) {                                             \
      _Pragma("unroll") for (int i = 0; i < MF; ++i) {                                           \
        if (!SKIP || i < nf_w) {                                                                 \
          _Pragma("unroll") for (int j = 0; j < kNF; ++j) {                                      \
            if (QB != 0 && i == 0)                                                               \
              mfma_acc_fresh(acc[i][j], F.a[i][h], F.b[j][h]);                                   \
            else                                                                                 \
              mfma_acc(acc[i][j], F.a[i][h], F.b[j][h]);                                         \
          }                                                                                      \
        }                                                                                        \
        if constexpr (QB == 4) {                                                                 \
          if (i == wn) mfma_acc_fresh(accx, F.a[i][h], ones);                                    \
        }                                                                                        \
      }                                                                                          \
    }                                                                                            \
  }

  const bf16x8_t ones = as_bf16x8(u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
  (void)ones;
  const int nsteps = U;  // >= 1
  {
    // Ping-pong.  Waves 0-3 (group 0, the first BM/2 rows) and 4-7 (group 1)
    // put one wave of each group on every SIMD.  Two barriers per step:
    // between B1(s) and B2(s) group 0 multiplies stage s while group 1 reads
    // stage s and issues its copies of stage s + STAGES - 1; between B2(s)
    // and B1(s+1) group 1 multiplies stage s while group 0 reads stage s+1
    // and issues its copies of stage s + STAGES.  So the matrix cores always
    // have one wave's products while the other wave waits for LDS and the
    // barrier.  Both groups run the same loop body [barrier, multiply,
    // barrier, read the next stage, copy]; group 1 enters it one barrier
    // later and group 0 passes one extra barrier at the end, so the counts
    // match.  A slot is refilled only after the barrier that follows both
    // groups' reads of it (each barrier waits for the wave's own LDS reads).
    // Before the barrier ahead of a wave's read of stage s, every wave has
    // waited until its own copies of s have landed (copies complete in issue
    // order): a group's copies are issued up to stage s + STAGES - 2 at that
    // point, so at most STAGES - 2 later stages stay outstanding; group 0's
    // wait before B1(s) (STAGES - 1 stages, its copies being one stage
    // further) only keeps the loop body the same.
    const bool g0 = wave < kWC;
#define MOE_ISSUE_CLAMPED(step) MOE_ISSUE((step) < nsteps ? (step) : nsteps - 1)
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s) MOE_ISSUE_CLAMPED(s);
    if (g0) {
      MOE_ISSUE_CLAMPED(STAGES - 1);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(CPS * (STAGES - 1)));
      ring_barrier();  // B0
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(CPS * (STAGES - 2)));
      ring_barrier();  // B0
      ring_barrier();  // B1(0)
    }
    MOE_LOAD_B(f, 0);
    MOE_LOAD_A(f, 0);
    if (!g0) MOE_ISSUE_CLAMPED(STAGES - 1);
    for (int ks = 0; ks < nsteps; ++ks) {
      if (g0)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(CPS * (STAGES - 1)));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(CPS * (STAGES - 2)));
      ring_barrier();  // group 0: B1(ks); group 1: B2(ks)
      // bf16 and int4 weights: the products at normal wave priority and the
      // next stage's activation fragments read before its weight fragments
      // (Mixtral prefill, bf16: up 2.84 -> 2.73 ms, down 1.55 -> 1.50 ms;
      // int4: up 2.5 % faster); int8 and fp8 read weights first (int8: 3-4 %
      // slower with activations first, fp8 unchanged), fp8 at normal
      // priority (1-1.5 % faster), int8 at the raised one
      if constexpr (QB == 0 || QB == 4 || QB == 9) {
        MOE_MMA(f);
      } else {
        asm volatile("s_setprio 1");
        MOE_MMA(f);
        asm volatile("s_setprio 0");
      }
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(CPS * (STAGES - 2)));
      ring_barrier();  // group 0: B2(ks); group 1: B1(ks+1)
      if constexpr (QB == 0 || QB == 4) {
        MOE_LOAD_A(f, ks + 1);
        MOE_LOAD_B(f, ks + 1);
      } else {
        MOE_LOAD_B(f, ks + 1);
        MOE_LOAD_A(f, ks + 1);
      }
      MOE_ISSUE_CLAMPED(ks + STAGES);
    }
    if (g0) ring_barrier();
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
#undef MOE_ISSUE_CLAMPED
  }
  mfma_fence_out(acc, accx);
#undef MOE_LOAD_A
#undef MOE_LOAD_B
#undef MOE_MMA
#undef MOE_ISSUE

  // int4: the activation sums of every row of the block, each computed by
  // one wave of its wave row, shared through LDS.  Lane l of accx holds rows
  // wn*16 + 4*(l>>4) + q of this wave row (every column the same).
  if constexpr (QB == 4) {
    if ((lane & 15) == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) rowsum_s[wm * MF * 16 + wn * 16 + 4 * (lane >> 4) + q] = accx[q];
    }
    __syncthreads();
  }

  // Epilogue.  Lane l of fragment (i, j) holds rows i*16 + 4*(l>>4) + q,
  // q = 0..3, of column (l & 15) of the fragment's tile.  The results go
  // through LDS (the ring is free once every wave is past its last read and
  // copy; each wave then uses a region of its own) so that every global
  // store writes 16 contiguous bytes per lane: a lane's four rows of one
  // column would otherwise take one narrow store each, and those stores
  // measured at ~10 % of the kernel (the CU's matrix cores idle meanwhile).
  const int nb0 = tile_base + wn * TPW;  // the wave's first column tile
  const bool live = nb0 < NB;            // NB is a multiple of 4: all of the wave's tiles or none
  __syncthreads();
  if constexpr (EPI == EPI_UP_SWIGLU || EPI == EPI_UP_RELU) {
    // H in the packed layout: the wave's TPW tiles are KF whole 32-column
    // fragments of each of its MF row fragments; staged in that layout, then
    // copied out fragment by fragment (fragments past the expert's last row
    // are not written: they belong to the next expert).
    constexpr int KF = TPW / 2;
    uint16_t* st = reinterpret_cast<uint16_t*>(&ring[0][0]) + wave * (MF * KF * 512);
    if (live) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int col = (nb0 + t) * 16 + (lane & 15);
        float sc0 = 1.0f, sc1 = 1.0f;
        if constexpr (QB != 0) {
          sc0 = A.scale0[(size_t)e * A.N + col];
          if constexpr (G == 2) sc1 = A.scale1[(size_t)e * A.N + col];
        }
        const int c = 16 * (t & 1) + (lane & 15);  // column inside the 32-column fragment
#pragma unroll
        for (int i = 0; i < MF; ++i) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = 4 * (lane >> 4) + q;
            float v0 = acc[i][t * G][q], v1 = acc[i][t * G + G - 1][q];
            if constexpr (QB == 4) {
              const float bias = kI4Bias * rowsum_s[wm * 16 * MF + i * 16 + r];
              v0 -= bias;
              v1 -= bias;
            }
            v0 *= sc0;
            v1 *= sc1;
            const float h = EPI == EPI_UP_SWIGLU ? silu_fast(v0) * v1 : (v0 > 0.0f ? v0 : 0.0f);
            st[(i * KF + (t >> 1)) * 512 + (r + 16 * (c >> 3)) * 8 + (c & 7)] = f32_to_bf16(h);
          }
        }
      }
      const long long fr0 = (long long)((prow0 + wm * 16 * MF) >> 4) * (A.N >> 5) + (nb0 >> 1);
      if (mb == 0 && offs_s[e] == 0 && wm == 0) zero_h_block(A.h_out, zrb, A.N, nb0 >> 1, KF, lane);
#pragma unroll
      for (int i = 0; i < MF; ++i) {
        if (wm * 16 * MF + 16 * i >= nrows) break;
#pragma unroll
        for (int kf = 0; kf < KF; ++kf) {
          const u32x4_t v = reinterpret_cast<const u32x4_t*>(st + (i * KF + kf) * 512)[lane];
          reinterpret_cast<u32x4_t*>(A.h_out)[(fr0 + (long long)i * (A.N >> 5) + kf) * 64 + lane] = v;
        }
      }
    }
  } else {
    // fp32 rows [row][N]: two row fragments (32 rows x the wave's 64 columns)
    // at a time, rows padded to RS floats against bank conflicts, then four
    // rows of 16 lanes x 16 bytes per store.
    static_assert(TPW == 4 && MF % 2 == 0, "down tile: 64 columns per wave, row fragments in pairs");
    constexpr int RS = 64 + 16;
    float* st = reinterpret_cast<float*>(&ring[0][0]) + wave * (32 * RS);
    if (live) {
      const int c0 = nb0 * 16;
      float sc[TPW];
#pragma unroll
      for (int t = 0; t < TPW; ++t) sc[t] = QB != 0 ? A.scale0[(size_t)e * A.N + c0 + 16 * t + (lane & 15)] : 1.0f;
#pragma unroll
      for (int pp = 0; pp < MF / 2; ++pp) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
          const int i = 2 * pp + ii;
#pragma unroll
          for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int r = 16 * ii + 4 * (lane >> 4) + q;
              float v0 = acc[i][t][q];
              if constexpr (QB == 4) v0 -= kI4Bias * rowsum_s[wm * 16 * MF + 16 * i + 4 * (lane >> 4) + q];
              st[r * RS + 16 * t + (lane & 15)] = v0 * sc[t];
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = 4 * j + (lane >> 4);
          const float4 v = *reinterpret_cast<const float4*>(st + r * RS + 4 * (lane & 15));
          const int row = wm * 16 * MF + 32 * pp + r;
          if (row < nrows) *reinterpret_cast<float4*>(A.f_out + (size_t)(row0 + row) * A.N + c0 + 4 * (lane & 15)) = v;
        }
      }
    }
  }
}

// Gathers the rows of x that the dispatch permutation lists into the packed
// fragment layout, expert by expert, each expert starting on a 16-row
// boundary; padding rows are zero.  One wave writes one 1 KiB fragment
// (lane l: 16 bytes of row l % 16 at k = 8 (l / 16)), fragments in packed
// order, so the writes are contiguous.
__global__ __launch_bounds__(256) void k_pack_rows(const PackArgs A) {
  __shared__ int offs_s[kMaxExperts + 1];
  __shared__ int poffs_s[kMaxExperts + 1];
  __shared__ DispatchLds<4> DL;
  __shared__ int row_a[32];  // with the dispatch derived here: assignment of each packed row of the block
  const int tid = threadIdx.x, lane = tid & 63;
  // first packed row of the block's first fragment; its four fragments span
  // at most two 16-row blocks (K/32 >= 2)
  const long long prow_base = (long long)blockIdx.x * 4 / (A.K / 32) * 16;
  if (A.topk_idx) {
    // The dispatch of the (small) batch, derived in every workgroup as in
    // the dispatch kernel; workgroup 0 publishes it for the FFN kernels.
    const int n = A.T * A.topk;
    block_histogram<4>(A.topk_idx, n, A.E, DL);
    if (tid <= A.E) offs_s[tid] = DL.offs[tid];
    if (tid < 32) row_a[tid] = -1;
    __syncthreads();
    if (tid <= A.E) poffs_s[tid] = padded_offset(offs_s, tid);
    __syncthreads();
    const bool publish = blockIdx.x == 0;
    block_stable_positions<4>(A.topk_idx, n, A.E, DL, [&](int a, int ea, int pos) {
      if (publish) {
        A.d_perm[pos] = a;
        A.d_inv[a] = pos;
      }
      const long long r = poffs_s[ea] + (pos - offs_s[ea]) - prow_base;
      if (r >= 0 && r < 32) row_a[r] = a;
    });
    if (publish) {
      if (tid < A.E) A.d_counts[tid] = DL.cnt[tid];
      if (tid <= A.E) A.d_offsets[tid] = DL.offs[tid];
    }
    __syncthreads();
  } else {
    if (tid <= A.E) offs_s[tid] = A.offsets[tid];
    __syncthreads();
    if (tid <= A.E) poffs_s[tid] = padded_offset(offs_s, tid);
    __syncthreads();
  }
  const int U = A.K / 32;
  const long long frag = (long long)blockIdx.x * 4 + (tid >> 6);
  const long long rb = frag / U;
  const int u = (int)(frag - rb * U);
  const long long prow = rb * 16 + (lane & 15);
  const int pe = poffs_s[A.E];
  if (prow >= pe + 16) return;  // past the last expert's padded rows and the zero row block
  int e = 0;
  if (prow < pe)
    while (poffs_s[e + 1] <= prow) ++e;
  const int local = (int)(prow - poffs_s[e]);
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (prow < pe && local < offs_s[e + 1] - offs_s[e]) {
    const int a = A.topk_idx ? row_a[prow - prow_base] : A.perm[offs_s[e] + local];
    const int token = a / A.topk;
    v = *reinterpret_cast<const u32x4_t*>(A.x + (size_t)token * A.K + u * 32 + 8 * (lane >> 4));
  }
  reinterpret_cast<u32x4_t*>(A.out)[frag * 64 + lane] = v;
}

// The same gather with the dispatch given (offsets, perm) and K / 32 a
// multiple of 4: a wave writes four consecutive fragments of one 16-row block,
// so each lane looks its row's assignment up once and issues the four loads
// of its row (64 contiguous bytes apart) together.
__global__ __launch_bounds__(256) void k_pack_rows4(const PackArgs A) {
  __shared__ int offs_s[kMaxExperts + 1];
  __shared__ int poffs_s[kMaxExperts + 1];
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid <= A.E) offs_s[tid] = A.offsets[tid];
  __syncthreads();
  if (tid <= A.E) poffs_s[tid] = padded_offset(offs_s, tid);
  __syncthreads();
  const int U = A.K / 32;
  const long long frag0 = ((long long)blockIdx.x * 4 + (tid >> 6)) * 4;
  const long long rb = frag0 / U;
  const int u0 = (int)(frag0 - rb * U);
  const long long prow = rb * 16 + (lane & 15);
  const int pe = poffs_s[A.E];
  if (prow >= pe + 16) return;  // past the last expert's padded rows and the zero row block
  int e = 0;
  if (prow < pe)
    while (poffs_s[e + 1] <= prow) ++e;
  const int local = (int)(prow - poffs_s[e]);
  u32x4_t v[4] = {};
  if (prow < pe && local < offs_s[e + 1] - offs_s[e]) {
    const int token = A.perm[offs_s[e] + local] / A.topk;
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(A.x + (size_t)token * A.K + u0 * 32 + 8 * (lane >> 4));
#pragma unroll
    for (int f = 0; f < 4; ++f) v[f] = src[4 * f];
  }
#pragma unroll
  for (int f = 0; f < 4; ++f) reinterpret_cast<u32x4_t*>(A.out)[(frag0 + f) * 64 + lane] = v[f];
}

// ---- fp8 x fp8 and int8 x int8: the up projection of 8-bit-activation layers ------
//
// With the activations quantised to E4M3 per token (one power-of-two scale
// each) and the weights in E4M3 with per-column scales, the first projection
// multiplies codes on the fp8 matrix cores (v_mfma_f32_32x32x64_f8f6f4) and
// applies the row scale and the column scale to the fp32 sums in the
// epilogue.  The tile, ring and ping-pong schedule are the bf16 kernel's; a
// stage now holds 64 k of 256 rows and 256 weight columns in the same 32 KiB
// (16 activation units + 16 weight units of 1 KiB), so a byte moved into LDS
// carries twice the products, and the fp8 products run at twice the bf16
// rate.  Both operands use the packed fp8 weights' unit layout (16 rows or
// columns x 64 k; lane l = r + 16 q holds k = 8 q + (0..7) and 32 + 8 q +
// (0..7)); a 32 x 64 product operand is two units, lane l = r + 32 g reading
// the 16 bytes of unit lanes 2 g and 2 g + 1, so that A and B pair the same k
// in every position.  Without scale operands (the per-token scale is a power
// of two applied in the epilogue), only that pairing matters.  int8 layers
// (the INT8 GeMM with both operands quantised) take the same units and
// operands, with the stage's 64 k as two v_mfma_i32_32x32x32_i8 products
// (exact int32 sums, converted in the epilogue).

// Gathers E4M3 code rows into packed units (one wave per unit).
__global__ __launch_bounds__(256) void k_pack_rows_a8(const PackA8Args A) {
  __shared__ int offs_s[kMaxExperts + 1];
  __shared__ int poffs_s[kMaxExperts + 1];
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid <= A.E) offs_s[tid] = A.offsets[tid];
  __syncthreads();
  if (tid <= A.E) poffs_s[tid] = padded_offset(offs_s, tid);
  __syncthreads();
  const int U = A.K / 64;
  const long long unit = (long long)blockIdx.x * 4 + (tid >> 6);
  const long long rb = unit / U;
  const int u = (int)(unit - rb * U);
  const long long prow = rb * 16 + (lane & 15);
  const int pe = poffs_s[A.E];
  if (prow >= pe + 16) return;  // past the last expert's padded rows and the zero row block
  int e = 0;
  if (prow < pe)
    while (poffs_s[e + 1] <= prow) ++e;
  const int local = (int)(prow - poffs_s[e]);
  const int q = lane >> 4;
  uint2 lo = make_uint2(0u, 0u), hi = make_uint2(0u, 0u);
  float rs = 0.0f;
  if (prow < pe && local < offs_s[e + 1] - offs_s[e]) {
    const int token = A.perm[offs_s[e] + local] / A.topk;
    const uint8_t* row = A.codes + (size_t)token * A.K + u * 64 + 8 * q;
    lo = *reinterpret_cast<const uint2*>(row);
    hi = *reinterpret_cast<const uint2*>(row + 32);
    rs = A.scale[token];
  }
  reinterpret_cast<uint4*>(A.out)[unit * 64 + lane] = make_uint4(lo.x, lo.y, hi.x, hi.y);
  if (u == 0 && q == 0) A.row_scale[prow] = rs;
}

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x16_t __attribute__((ext_vector_type(16)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

// acc += a * b (32 x 32 x 64, E4M3 operands), accumulating in place.  The
// leading s_nop covers a vector instruction that assembled an operand
// register just before (two wait states before a matrix instruction reads
// it).
__device__ __forceinline__ void mfma_f8(floatx16_t& acc, const i32x8_t& a, const i32x8_t& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

// The int8 form: the 64 k of a stage as two 32 x 32 x 32 products (the
// operand's bytes 0-15, then 16-31), exact int32 sums.
__device__ __forceinline__ void mfma_i8(i32x16_t& acc, const i32x8_t& a, const i32x8_t& b) {
  const i32x4_t a0 = {a[0], a[1], a[2], a[3]}, a1 = {a[4], a[5], a[6], a[7]};
  const i32x4_t b0 = {b[0], b[1], b[2], b[3]}, b1 = {b[4], b[5], b[6], b[7]};
  asm volatile("s_nop 1\n\tv_mfma_i32_32x32x32_i8 %0, %1, %2, %0" : "+v"(acc) : "v"(a0), "v"(b0));
  asm volatile("s_nop 1\n\tv_mfma_i32_32x32x32_i8 %0, %1, %2, %0" : "+v"(acc) : "v"(a1), "v"(b1));
}

template <int EPI, bool I8>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_ffn_gemm_a8(
    const GemmArgs A, const float* __restrict__ row_scale) {
  using acc_t = std::conditional_t<I8, i32x16_t, floatx16_t>;
  constexpr int G = EPI == EPI_UP_SWIGLU ? 2 : 1;
  constexpr int TPW = kNF / G;  // column tiles per wave
  constexpr int BM = 256, NAF = 16, NBF = 16, STAGES = 4, CPA = 2, CPB = 2, CPS = CPA + CPB;
  constexpr int STAGE_BYTES = (NAF + NBF) * kFrag;
  constexpr int RB = 4;  // 32-row blocks per wave (128 rows)
  static_assert(CPS * (STAGES - 1) <= 63, "vmcnt holds at most 63");
  __shared__ __attribute__((aligned(1024))) unsigned char ring[STAGES][STAGE_BYTES];
  const int* const offs_s = A.offsets;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kWC;
  const int wn = wave % kWC;
  const int NB = A.N / 16;
  const int NBL = (NB + kWC * TPW - 1) / (kWC * TPW);

  int e, mb, nblock;
  const int L = xcd_item(blockIdx.x, gemm_items(offs_s, A.E, BM, NBL), 0);  // an up projection: real items dealt evenly
  if (L < 0 || !gemm_item(offs_s, A.E, BM, NBL, A.cg, L, &e, &mb, &nblock)) return;
  const int tile_base = nblock * kWC * TPW;
  const int row0 = offs_s[e] + mb * BM;
  const int nrows = min(BM, offs_s[e + 1] - row0);
  const int prow0 = padded_offset(offs_s, e) + mb * BM;
  const int nfrag = (nrows + 15) >> 4;  // packed units holding real rows
  const int zrb = padded_offset(offs_s, A.E) >> 4;  // the zero row block

  // copies: activation units 2 w, 2 w + 1 and weight units 2 w, 2 w + 1 of
  // every stage (units past the expert's last row read the zero row block)
  const int U = A.K / 64;
  const char* const abase = reinterpret_cast<const char*>(A.act);
  const char* const bbase = static_cast<const char*>(A.w);
  uint32_t aoff[CPA], boff[CPB];
#pragma unroll
  for (int j = 0; j < CPA; ++j) {
    const int f = CPA * wave + j;
    const int rb = f < nfrag ? (prow0 >> 4) + f : zrb;
    aoff[j] = (uint32_t)((unsigned long long)rb * (unsigned)U * 1024ull + 16ull * lane);
  }
#pragma unroll
  for (int j = 0; j < CPB; ++j) boff[j] = (uint32_t)gemm_b_offset(e, NB, U, G, tile_base, kNF, CPB * wave + j, lane);
  const uint32_t ring_lds = lds_address(ring);
  const uint32_t a_lds = ring_lds + (uint32_t)(CPA * wave) * kFrag;
  const uint32_t b_lds = ring_lds + (uint32_t)(NAF + CPB * wave) * kFrag;

#define MOE_ISSUE(step)                                                                            \
  do {                                                                                             \
    const char* ab_ = abase + (size_t)(step) * kFrag;                                              \
    const char* bb_ = bbase + (size_t)(step) * G * kFrag;                                          \
    const uint32_t st_ = (uint32_t)((step) % STAGES) * STAGE_BYTES;                                \
    _Pragma("unroll") for (int j = 0; j < CPA; ++j) copy_frag(ab_, aoff[j], a_lds + st_ + j * kFrag); \
    _Pragma("unroll") for (int j = 0; j < CPB; ++j) copy_frag(bb_, boff[j], b_lds + st_ + j * kFrag); \
  } while (0)

  acc_t acc[RB][2];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][c][v] = 0;
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int c = 0; c < 2; ++c) asm volatile("" : "+v"(acc[i][c]));
  asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");

  // operand reads: lane l = r + 32 g of a 32 x 64 operand takes unit lanes
  // (r % 16) + 16 (2 g) and + 16 (2 g + 1) of unit r / 16 of the pair
  const int ul = (lane & 15) + 32 * (lane >> 5);  // first unit lane (its second is + 16)
  const int uh = (lane >> 4) & 1;                 // which unit of the pair
  struct {
    i32x8_t a[RB], b[2];
  } f;
  auto rd = [&](const u32x4_t* st, int unit, i32x8_t& dst) {
    const u32x4_t lo = st[unit * 64 + ul], hi = st[unit * 64 + ul + 16];
    dst = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
#define MOE_LOAD(F, step)                                                                          \
  do {                                                                                             \
    const u32x4_t* st_ = reinterpret_cast<const u32x4_t*>(ring[(step) % STAGES]);                  \
    _Pragma("unroll") for (int i = 0; i < RB; ++i) rd(st_, wm * 8 + 2 * i + uh, F.a[i]);             \
    _Pragma("unroll") for (int c = 0; c < 2; ++c)                                                  \
        rd(st_, NAF + wn * kNF + (G == 2 ? 2 * uh + c : 2 * c + uh), F.b[c]);                      \
  } while (0)
#define MOE_MMA(F)                                                                                 \
  _Pragma("unroll") for (int i = 0; i < RB; ++i) _Pragma("unroll") for (int c = 0; c < 2; ++c) {   \
    if constexpr (I8)                                                                              \
      mfma_i8(acc[i][c], F.a[i], F.b[c]);                                                          \
    else                                                                                           \
      mfma_f8(acc[i][c], F.a[i], F.b[c]);                                                          \
  }

  const int nsteps = U;
  {
    // the bf16 kernel's ping-pong (see k_ffn_gemm)
    const bool g0 = wave < kWC;
#define MOE_ISSUE_CLAMPED(step) MOE_ISSUE((step) < nsteps ? (step) : nsteps - 1)
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s) MOE_ISSUE_CLAMPED(s);
    if (g0) {
      MOE_ISSUE_CLAMPED(STAGES - 1);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(CPS * (STAGES - 1)));
      ring_barrier();
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(CPS * (STAGES - 2)));
      ring_barrier();
      ring_barrier();
    }
    MOE_LOAD(f, 0);
    if (!g0) MOE_ISSUE_CLAMPED(STAGES - 1);
    for (int ks = 0; ks < nsteps; ++ks) {
      if (g0)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(CPS * (STAGES - 1)));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(CPS * (STAGES - 2)));
      ring_barrier();
      asm volatile("s_setprio 1");
      MOE_MMA(f);
      asm volatile("s_setprio 0");
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(CPS * (STAGES - 2)));
      ring_barrier();
      MOE_LOAD(f, ks + 1);
      MOE_ISSUE_CLAMPED(ks + STAGES);
    }
    if (g0) ring_barrier();
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
#undef MOE_ISSUE_CLAMPED
  }
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int c = 0; c < 2; ++c) asm volatile("" : "+v"(acc[i][c]));
#undef MOE_LOAD
#undef MOE_MMA
#undef MOE_ISSUE

  // Epilogue.  Element v of acc[i][c] in lane l: row 32 i + 8 (v / 4) +
  // 4 (l / 32) + v % 4 of the wave's rows, column l % 32 of operand block c
  // (SwiGLU: gate c = 0 and up c = 1 of the same 32 hidden columns; ReLU:
  // 32 columns each).  H is staged in LDS in the packed layout (KF 32-column
  // fragments per 16-row fragment) and copied out 16 bytes per lane, as in
  // the bf16 kernel.
  constexpr int KF = TPW / 2;
  const int nb0 = tile_base + wn * TPW;
  const bool live = nb0 < NB;  // NB is a multiple of 4: all of the wave's tiles or none
  __syncthreads();
  uint16_t* st = reinterpret_cast<uint16_t*>(&ring[0][0]) + wave * (8 * KF * 512);
  if (live) {
    const int c32 = lane & 31;
#pragma unroll
    for (int c = 0; c < KF; ++c) {
      const int col = (nb0 + 2 * c) * 16 + c32;
      const float sc0 = A.scale0[(size_t)e * A.N + col];
      const float sc1 = G == 2 ? A.scale1[(size_t)e * A.N + col] : 1.0f;
#pragma unroll
      for (int i = 0; i < RB; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int R = 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);  // row of the wave's 128
          const int row = wm * 128 + R;
          const float rs = row < nrows ? row_scale[prow0 + row] : 0.0f;
          float h;
          if constexpr (EPI == EPI_UP_SWIGLU) {
            const float g = (float)acc[i][0][v] * sc0 * rs, up = (float)acc[i][1][v] * sc1 * rs;
            h = silu_fast(g) * up;
          } else {
            const float g = (float)acc[i][c][v] * sc0 * rs;
            h = g > 0.0f ? g : 0.0f;
          }
          st[((R >> 4) * KF + c) * 512 + ((R & 15) + 16 * (c32 >> 3)) * 8 + (c32 & 7)] = f32_to_bf16(h);
        }
      }
    }
    const long long fr0 = (long long)((prow0 + wm * 128) >> 4) * (A.N >> 5) + (nb0 >> 1);
    if (mb == 0 && offs_s[e] == 0 && wm == 0) zero_h_block(A.h_out, zrb, A.N, nb0 >> 1, KF, lane);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (wm * 128 + 16 * i >= nrows) break;
#pragma unroll
      for (int kf = 0; kf < KF; ++kf) {
        const u32x4_t v = reinterpret_cast<const u32x4_t*>(st + (i * KF + kf) * 512)[lane];
        reinterpret_cast<u32x4_t*>(A.h_out)[(fr0 + (long long)i * (A.N >> 5) + kf) * 64 + lane] = v;
      }
    }
  }
}

}  // namespace

template <int QB>
hipError_t launch_gemm_qb(const GemmArgs& a, int epi, hipStream_t s) {
  using S = GemmShape<QB>;
  const int G = epi == EPI_UP_SWIGLU ? 2 : 1;
  const int tiles_per_block = kWC * (kNF / G);
  const int NB = a.N / 16;
  const long long nbl = (NB + tiles_per_block - 1) / tiles_per_block;
  const long long work = nbl * a.W;  // a.W bounds the number of row blocks
  if (work <= 0) return hipSuccess;  // no expert is served
  if (work > 0x7FFFFFF0LL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((work + 7) / 8 * 8));
#define MOE_LAUNCH(SK)                                                                                    \
  switch (epi) {                                                                                          \
    case EPI_UP_SWIGLU: k_ffn_gemm<EPI_UP_SWIGLU, SK, QB><<<grid, kWaves * 64, 0, s>>>(a); break;           \
    case EPI_UP_RELU: k_ffn_gemm<EPI_UP_RELU, SK, QB><<<grid, kWaves * 64, 0, s>>>(a); break;               \
    case EPI_DOWN_ROWS: k_ffn_gemm<EPI_DOWN_ROWS, SK, QB><<<grid, kWaves * 64, 0, s>>>(a); break;           \
    default: return hipErrorInvalidValue;                                                                 \
  }
  if (a.skip_empty) {
    MOE_LAUNCH(true)
  } else {
    MOE_LAUNCH(false)
  }
#undef MOE_LAUNCH
  (void)S::BM;
  return hipGetLastError();
}

hipError_t launch_ffn_gemm(const GemmArgs& a, int epi, int qb, hipStream_t s) {
  const int uk = 32 * q_ah(qb);
  if (a.K % 64 || a.N % 64 || a.K <= 0 || a.N <= 0 || a.K % uk || a.cg < 1) return hipErrorInvalidValue;
  if (qb != 0 && (!a.scale0 || (epi == EPI_UP_SWIGLU && !a.scale1))) return hipErrorInvalidValue;
  switch (qb) {
    case 0: return launch_gemm_qb<0>(a, epi, s);
    case 8: return launch_gemm_qb<8>(a, epi, s);
    case 9: return launch_gemm_qb<9>(a, epi, s);
    case 4: return launch_gemm_qb<4>(a, epi, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_pack_rows(const PackArgs& a, hipStream_t s) {
  const long long n = a.rows > 0 ? a.rows : (long long)a.T * a.topk;
  const long long frags = packed_rows_alloc(n, a.E) / 16 * (a.K / 32);
  if (frags <= 0) return hipSuccess;
  if (!a.topk_idx && (a.K / 32) % 4 == 0) {
    const long long blocks = (frags / 4 + 3) / 4;  // one wave per four fragments
    k_pack_rows4<<<dim3((unsigned)blocks), 256, 0, s>>>(a);
  } else {
    const long long blocks = (frags + 3) / 4;  // one wave per fragment
    k_pack_rows<<<dim3((unsigned)blocks), 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_pack_rows_a8(const PackA8Args& a, hipStream_t s) {
  if (a.K % 64 || a.K <= 0) return hipErrorInvalidValue;
  const long long n = a.rows > 0 ? a.rows : (long long)a.T * a.topk;
  const long long units = packed_rows_alloc(n, a.E) / 16 * (a.K / 64);
  const long long blocks = (units + 3) / 4;  // one wave per unit
  if (blocks <= 0) return hipSuccess;
  k_pack_rows_a8<<<dim3((unsigned)blocks), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_ffn_gemm_a8(const GemmArgs& a, const float* row_scale, int epi, bool int8, hipStream_t s) {
  if (a.K % 64 || a.N % 64 || a.K <= 0 || a.N <= 0 || a.cg < 1 || !a.scale0 || !row_scale) return hipErrorInvalidValue;
  if (epi == EPI_UP_SWIGLU && !a.scale1) return hipErrorInvalidValue;
  const int G = epi == EPI_UP_SWIGLU ? 2 : 1;
  const int tiles_per_block = kWC * (kNF / G);
  const long long nbl = (a.N / 16 + tiles_per_block - 1) / tiles_per_block;
  const long long work = nbl * a.W;
  if (work <= 0) return hipSuccess;
  if (work > 0x7FFFFFF0LL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((work + 7) / 8 * 8));
#define MOE_A8(EP, I8_)                                                       \
  k_ffn_gemm_a8<EP, I8_><<<grid, kWaves * 64, 0, s>>>(a, row_scale);          \
  break;
  switch (epi * 2 + (int8 ? 1 : 0)) {
    case EPI_UP_SWIGLU * 2: MOE_A8(EPI_UP_SWIGLU, false)
    case EPI_UP_SWIGLU * 2 + 1: MOE_A8(EPI_UP_SWIGLU, true)
    case EPI_UP_RELU * 2: MOE_A8(EPI_UP_RELU, false)
    case EPI_UP_RELU * 2 + 1: MOE_A8(EPI_UP_RELU, true)
    default: return hipErrorInvalidValue;
  }
#undef MOE_A8
  return hipGetLastError();
}

int gemm_rows_per_block(int qb) { return q_bits(qb) == 4 ? GemmShape<4>::BM : (qb == 0 ? GemmShape<0>::BM : GemmShape<8>::BM); }

}  // namespace moe
