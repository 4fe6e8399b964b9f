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
// halves the copy rate.  Fragments stream through a 5-stage LDS ring of
// 32 KiB stages (32 k each; all 160 KiB of a CU's LDS), copied global -> LDS
// with global_load_lds_dwordx4 (lane l of a copy lands at base + 16 l): each
// copy is one contiguous 1 KiB read, and each wave reads a fragment with one
// conflict-free 16-byte ds_read per lane.  The two waves of each SIMD take
// turns: one multiplies the stage it holds in registers while the other reads
// its next stage and issues copies (ping-pong, two barriers per step); four
// to five stages of copies stay in flight.
// Workgroups run expert by expert, in groups of A.cg (4) column blocks x all
// of the expert's row blocks, on one XCD at a time: the ~32 resident
// workgroups then read ~8 activation tiles and ~4 weight tiles per stage,
// the rest hits in L2.
//
// Measured on the Mixtral-shaped prefill layer (T = 8192), the kernel runs
// the matrix cores about half the time: the global -> LDS copies alone take
// three quarters of its time, and with copies, LDS reads and products all
// running the clock drops from ~2.4 to ~2.0 GHz.
#include "moe_dispatch_block.hpp"
#include "moe_index.hpp"
#include "moe_lds.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

constexpr int kBM = 256;     // rows per workgroup
constexpr int kWR = 2;       // wave rows
constexpr int kWC = 4;       // wave columns
constexpr int kWaves = kWR * kWC;
constexpr int kMF = 8;       // row fragments per wave (128 rows)
constexpr int kNF = 4;       // column fragments per wave
constexpr int kCPW = 16 / kWaves;  // A (and B) fragments each wave copies per stage
constexpr int kCPS = 2 * kCPW;     // copies per wave per stage
constexpr int kStages = 5;   // LDS ring depth: 5 x 32 KiB, all of a CU's LDS
constexpr int kFrag = 1024;  // bytes of one 64-lane x 16-byte fragment

// acc += a * b on the matrix cores, accumulating in place.  Written as
// inline assembly because the compiler otherwise gives each product a fresh
// destination and copies the accumulators around the loop, which doubles
// their register footprint.  The accumulator is reused only 32 products
// later, so consecutive products carry no dependence.
__device__ __forceinline__ void mfma_acc(floatx4_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
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
__device__ __forceinline__ void mfma_fence_in(floatx4_t (&acc)[MF][NF]) {
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j) acc_tie(acc[i][j]);
  asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
}
template <int MF, int NF>
__device__ __forceinline__ void mfma_fence_out(floatx4_t (&acc)[MF][NF]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j) acc_tie(acc[i][j]);
}

// SKIP: row fragments past the row block's last real row skip their
// products (the fragment reads still run, so the steady state keeps no branch
// around a load); for layers whose experts hold few rows.
template <int EPI, bool SKIP>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_ffn_gemm(
    const GemmArgs A) {
  constexpr int G = EPI == EPI_UP_SWIGLU ? 2 : 1;
  constexpr int TPW = kNF / G;  // column tiles per wave
  // stage layout: 16 A fragments (256 rows x 32 k), then 16 B fragments
  // (kWC wave columns x kNF fragments)
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kStages][32 * kFrag];
  const int* const offs_s = A.offsets;  // uniform: scalar loads

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // wave row (128 rows) and wave column; each wave row is one group of four
  // waves, one per SIMD (the ping-pong below)
  const int wm = wave / kWC;
  const int wn = wave % kWC;
  const int NB = A.N / 16;
  const int NBL = (NB + kWC * TPW - 1) / (kWC * TPW);  // column blocks

  int e, mb, nblock;
  if (!gemm_item(offs_s, A.E, kBM, NBL, A.cg, xcd_logical(blockIdx.x, gridDim.x), &e, &mb, &nblock)) return;
  const int tile_base = nblock * kWC * TPW;
  const int row0 = offs_s[e] + mb * kBM;  // first dispatched row
  const int nrows = min(kBM, offs_s[e + 1] - row0);
  const int prow0 = padded_offset(offs_s, e) + mb * kBM;  // its packed row
  const int nfrag = (nrows + 15) >> 4;  // packed fragments holding real rows
  // this wave's row fragments that hold real rows (uniform)
  const int nf_w = __builtin_amdgcn_readfirstlane(min(max(nfrag - wm * kMF, 0), kMF));

  // This wave copies A fragments and B fragments kCPW w .. kCPW w + kCPW-1 of
  // every stage.  Sources are a uniform base that advances one 32-k unit per stage
  // plus a constant 32-bit byte offset per lane (the packed activations and
  // one projection's packed weights are each under 4 GiB; checked on the
  // host).  A fragments past the expert's last row re-read its last
  // fragment; their rows are never stored.
  const int U = A.K / 32;
  const char* const abase = reinterpret_cast<const char*>(A.act);
  const char* const bbase = static_cast<const char*>(A.w);
  uint32_t aoff[kCPW], boff[kCPW];
#pragma unroll
  for (int j = 0; j < kCPW; ++j) {
    const int f = kCPW * wave + j;  // A fragment f: rows f*16 .. +15; B fragment f
    aoff[j] = (uint32_t)gemm_a_offset((prow0 >> 4) + min(f, nfrag - 1), A.K, lane);
    boff[j] = (uint32_t)gemm_b_offset(e, NB, U, G, tile_base, kNF, f, lane);
  }

  // LDS byte address of the ring and of this wave's first fragment slot
  const uint32_t ring_lds = lds_address(ring);
  const uint32_t wave_lds = ring_lds + (uint32_t)(kCPW * wave) * kFrag;

#define MOE_ISSUE(step)                                                                          \
  do {                                                                                           \
    const char* ab_ = abase + (size_t)(step) * kFrag;                                            \
    const char* bb_ = bbase + (size_t)(step) * G * kFrag;                                        \
    const uint32_t st_ = wave_lds + (uint32_t)((step) % kStages) * (32 * kFrag);                 \
    _Pragma("unroll") for (int j = 0; j < kCPW; ++j) {                                           \
      copy_frag(ab_, aoff[j], st_ + j * kFrag);                                                  \
      copy_frag(bb_, boff[j], st_ + (16 + j) * kFrag);                                           \
    }                                                                                            \
  } while (0)

  floatx4_t acc[kMF][kNF];
#pragma unroll
  for (int i = 0; i < kMF; ++i)
#pragma unroll
    for (int j = 0; j < kNF; ++j) acc[i][j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
  mfma_fence_in(acc);

  // The fragments of one stage, held in registers.
  struct {
    bf16x8_t a[kMF], b[kNF];
  } f;
#define MOE_LOAD_B(F, step)                                                                      \
  do {                                                                                           \
    const u32x4_t* st_ = reinterpret_cast<const u32x4_t*>(ring[(step) % kStages]);               \
    _Pragma("unroll") for (int j = 0; j < kNF; ++j) F.b[j] = as_bf16x8(st_[(16 + wn * kNF + j) * 64 + lane]); \
  } while (0)
#define MOE_LOAD_A(F, step, i0, i1)                                                              \
  do {                                                                                           \
    const u32x4_t* st_ = reinterpret_cast<const u32x4_t*>(ring[(step) % kStages]);               \
    _Pragma("unroll") for (int i = (i0); i < (i1); ++i) F.a[i] = as_bf16x8(st_[(wm * kMF + i) * 64 + lane]); \
  } while (0)
#define MOE_MMA(F)                                                                               \
  _Pragma("unroll") for (int i = 0; i < kMF; ++i) {                                              \
    if (!SKIP || i < nf_w) {                                                                     \
      _Pragma("unroll") for (int j = 0; j < kNF; ++j) mfma_acc(acc[i][j], F.a[i], F.b[j]);       \
    }                                                                                            \
  }

  const int nsteps = U;  // even, >= 2 (K is a multiple of 64)
  {
    // Ping-pong.  Waves 0-3 (group 0, rows 0-127) and 4-7 (group 1, rows
    // 128-255) put one wave of each group on every SIMD.  Two barriers per
    // step: between B1(s) and B2(s) group 0 multiplies stage s while group 1
    // reads stage s and issues its copies of stage s+4; between B2(s) and
    // B1(s+1) group 1 multiplies stage s while group 0 reads stage s+1 and
    // issues its copies of stage s+5.  So the matrix cores always have one
    // wave's products while the other wave waits for LDS and the barrier.
    // Both groups run the same loop body [barrier, multiply, barrier, read
    // the next stage, copy]; group 1 enters it one barrier later and group 0
    // passes one extra barrier at the end, so the counts match.
    // A slot is refilled only after the barrier that follows both groups'
    // reads of it.  Before the barrier ahead of a stage's first read (B2(s-1)
    // for stage s) every wave's copies of it have landed: group 0 then has
    // stages up to s+3 issued, group 1 up to s+3, so at most 12 copies may
    // stay outstanding; group 0's wait before B1(s) (16) and group 1's before
    // B1(s+1) (12) only keep the loop body the same.
    const bool g0 = wave < kWC;
#define MOE_ISSUE_CLAMPED(step) MOE_ISSUE((step) < nsteps ? (step) : nsteps - 1)
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s) MOE_ISSUE_CLAMPED(s);
    if (g0) {
      MOE_ISSUE_CLAMPED(kStages - 1);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kCPS * (kStages - 1)));
      ring_barrier();  // B0
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kCPS * (kStages - 2)));
      ring_barrier();  // B0
      ring_barrier();  // B1(0)
    }
    MOE_LOAD_B(f, 0);
    MOE_LOAD_A(f, 0, 0, kMF);
    if (!g0) MOE_ISSUE_CLAMPED(kStages - 1);
    for (int ks = 0; ks < nsteps; ++ks) {
      if (g0)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kCPS * (kStages - 1)));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kCPS * (kStages - 2)));
      ring_barrier();  // group 0: B1(ks); group 1: B2(ks)
      asm volatile("s_setprio 1");
      MOE_MMA(f);
      asm volatile("s_setprio 0");
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kCPS * (kStages - 2)));
      ring_barrier();  // group 0: B2(ks); group 1: B1(ks+1)
      MOE_LOAD_B(f, ks + 1);
      MOE_LOAD_A(f, ks + 1, 0, kMF);
      MOE_ISSUE_CLAMPED(ks + kStages);
    }
    if (g0) ring_barrier();
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
#undef MOE_ISSUE_CLAMPED
  }
  mfma_fence_out(acc);
#undef MOE_LOAD_A
#undef MOE_LOAD_B
#undef MOE_MMA
#undef MOE_ISSUE

  // Epilogue.  Lane l of fragment (i, j) holds rows i*16 + 4*(l>>4) + q,
  // q = 0..3, of column (l & 15) of the fragment's tile.
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int nb = tile_base + wn * TPW + t;
    if (nb >= NB) continue;
    const int col = nb * 16 + (lane & 15);
#pragma unroll
    for (int i = 0; i < kMF; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = wm * 16 * kMF + i * 16 + 4 * (lane >> 4) + q;
        if (row >= nrows) continue;
        if constexpr (EPI == EPI_UP_SWIGLU) {
          const float gv = acc[i][t * 2][q], uv = acc[i][t * 2 + 1][q];
          A.h_out[packed_index(prow0 + row, col, A.N)] = f32_to_bf16(silu(gv) * uv);
        } else if constexpr (EPI == EPI_UP_RELU) {
          const float gv = acc[i][t][q];
          A.h_out[packed_index(prow0 + row, col, A.N)] = f32_to_bf16(gv > 0.0f ? gv : 0.0f);
        } else {
          A.f_out[(size_t)(row0 + row) * A.N + col] = acc[i][t][q];
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
  if (prow >= poffs_s[A.E]) return;  // past the last expert's padded rows
  int e = 0;
  while (poffs_s[e + 1] <= prow) ++e;
  const int local = (int)(prow - poffs_s[e]);
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (local < offs_s[e + 1] - offs_s[e]) {
    const int a = A.topk_idx ? row_a[prow - prow_base] : A.perm[offs_s[e] + local];
    const int token = a / A.topk;
    v = *reinterpret_cast<const u32x4_t*>(A.x + (size_t)token * A.K + u * 32 + 8 * (lane >> 4));
  }
  reinterpret_cast<u32x4_t*>(A.out)[frag * 64 + lane] = v;
}

}  // namespace

hipError_t launch_ffn_gemm(const GemmArgs& a, int epi, hipStream_t s) {
  if (a.K % 64 || a.N % 64 || a.K <= 0 || a.N <= 0 || a.cg < 1 || epi == EPI_DOWN_ACC)
    return hipErrorInvalidValue;  // an even step count, whole tiles
  const int G = epi == EPI_UP_SWIGLU ? 2 : 1;
  const int tiles_per_block = kWC * (kNF / G);
  const int NB = a.N / 16;
  const long long nbl = (NB + tiles_per_block - 1) / tiles_per_block;
  const long long work = nbl * a.W;  // a.W bounds the number of row blocks
  if (work <= 0) return hipSuccess;  // no expert is served
  const dim3 grid((unsigned)((work + 7) / 8 * 8));
#define MOE_LAUNCH(SK)                                                                               \
  switch (epi) {                                                                                     \
    case EPI_UP_SWIGLU: k_ffn_gemm<EPI_UP_SWIGLU, SK><<<grid, kWaves * 64, 0, s>>>(a); break;           \
    case EPI_UP_RELU: k_ffn_gemm<EPI_UP_RELU, SK><<<grid, kWaves * 64, 0, s>>>(a); break;               \
    case EPI_DOWN_ROWS: k_ffn_gemm<EPI_DOWN_ROWS, SK><<<grid, kWaves * 64, 0, s>>>(a); break;           \
    default: return hipErrorInvalidValue;                                                            \
  }
  if (a.skip_empty) {
    MOE_LAUNCH(true)
  } else {
    MOE_LAUNCH(false)
  }
#undef MOE_LAUNCH
  return hipGetLastError();
}

hipError_t launch_pack_rows(const PackArgs& a, hipStream_t s) {
  const long long frags = packed_rows_max((long long)a.T * a.topk, a.E) / 16 * (a.K / 32);
  const long long blocks = (frags + 3) / 4;  // one wave per fragment
  if (blocks <= 0) return hipSuccess;
  k_pack_rows<<<dim3((unsigned)blocks), 256, 0, s>>>(a);
  return hipGetLastError();
}

int gemm_rows_per_block() { return kBM; }

}  // namespace moe
