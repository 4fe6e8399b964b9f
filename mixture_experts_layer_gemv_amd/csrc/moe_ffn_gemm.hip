// Expert FFN for prefill-sized batches: a grouped GEMM on the matrix cores.
//
// When every expert holds hundreds of rows the FFN is compute-bound (the
// FFN's intensity grows with the batch until the kernel's compute peak is the
// roof: MoE-Lightning note, FFN roofline against batch size), so each weight
// byte is read from HBM about once and reused from LDS and L2.
//
// A workgroup computes a 256-row block of one expert against a block of
// column tiles with 2 x 4 waves (two per SIMD); each wave owns a 128 x 64
// tile (8 x 4 fragments of v_mfma_f32_16x16x32_bf16, 128 fp32 accumulators
// per lane).
// Both operands stream through a 4-stage LDS ring, 32 k per stage:
//  - the 256 activation rows (gathered through the dispatch permutation) are
//    copied global -> LDS with global_load_lds_dwordx4 straight into MFMA
//    A-operand order (lane l of a copy lands at base + 16 l), so every wave
//    reads a fragment with one conflict-free 16-byte ds_read per lane;
//  - the weight fragments are already packed in B-operand order in HBM, so a
//    copy of 1 KiB per fragment lands them in LDS ready to read;
//  - copies run three stages ahead of the MFMAs; a stage is consumed after a
//    vmcnt wait for its own copies and one barrier.
// No staging registers are needed for either operand.  Workgroups are ordered
// so the row blocks of one (expert, column block) run together on one XCD:
// its weight panel comes from HBM once and the other row blocks hit in L2.
#include "moe_index.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

constexpr int kBM = 256;     // rows per workgroup
constexpr int kWaves = 8;    // 2 wave rows x 4 wave columns
constexpr int kMF = 8;       // row fragments per wave (128 rows)
constexpr int kNF = 4;       // column fragments per wave
constexpr int kStages = 4;   // LDS ring depth (copies run kStages-1 steps ahead)
constexpr int kFrag = 1024;  // bytes of one 64-lane x 16-byte fragment

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left unconstrained).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Workgroup barrier without the release/acquire fences of __syncthreads():
// those would wait for every outstanding copy (vmcnt(0)) and collapse the
// ring; the stage being consumed is waited for explicitly with vmcnt_imm.
// The wave's own LDS reads finish first (lgkmcnt(0)), so a stage it read is
// free once every wave has passed; the memory clobber keeps LDS accesses on
// their side of the barrier.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// global -> LDS copy of one fragment: lane l moves the 16 bytes at
// sbase + voff (a uniform base and its own 32-bit offset) into LDS byte
// address lds + 16 l.  Issued as inline assembly so the compiler does not
// add its own conservative wait for the copy before unrelated LDS reads; the
// ring's explicit vmcnt waits and barriers order the accesses instead.
__device__ __forceinline__ void copy_frag(const void* sbase, uint32_t voff, uint32_t lds) {
  // m0 is set right here; nothing else in these kernels keeps a value in m0
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds) : "memory");
}

template <int EPI>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_ffn_gemm(
    const GemmArgs A) {
  constexpr int G = EPI == EPI_UP_SWIGLU ? 2 : 1;
  constexpr int TPW = kNF / G;  // column tiles per wave
  // stage layout: 16 A fragments (256 rows x 32 k), then 16 B fragments
  // (4 wave columns x 4 fragments)
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kStages][32 * kFrag];
  __shared__ int rows_s[kBM];
  __shared__ int offs_s[kMaxExperts + 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;  // wave row (128 rows), wave column
  const GemmWork gw = gemm_work(xcd_logical(blockIdx.x, gridDim.x), A.W);
  const int nblock = gw.nblock, mpair = gw.mpair;
  const int NB = A.N / 16;

  if (tid <= A.E) offs_s[tid] = A.offsets[tid];
  __syncthreads();
  int e, mb, npairs;
  if (!skinny_pair(offs_s, A.E, kBM, mpair, &e, &mb, &npairs)) return;
  const int tile_base = nblock * 4 * TPW;
  if (tile_base >= NB) return;
  const int row0 = offs_s[e] + mb * kBM;
  const int nrows = min(kBM, offs_s[e + 1] - row0);
  if (tid < kBM) {
    const int r = tid < nrows ? tid : 0;
    rows_s[tid] = A.gather ? A.perm[row0 + r] / A.topk : row0 + r;
  }
  __syncthreads();

  // This wave copies A fragments 2w, 2w+1 and B fragments 2w, 2w+1 of every
  // stage.  Sources are a uniform base that advances one 32-k unit per stage
  // plus a constant 32-bit byte offset per lane (activations and one
  // projection's packed weights are each well under 4 GiB; checked on the
  // host).
  const int U = A.K / 32;
  const char* const abase = reinterpret_cast<const char*>(A.act);
  const char* const bbase = static_cast<const char*>(A.w);
  uint32_t aoff[2], boff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int f = 2 * wave + j;  // A fragment f: rows f*16 .. +15; B fragment f
    aoff[j] = (uint32_t)gemm_a_offset(rows_s[f * 16 + (lane & 15)], A.K, lane);
    boff[j] = (uint32_t)gemm_b_offset(e, NB, U, G, tile_base, kNF, f, lane);
  }

  // LDS byte address of the ring and of this wave's first fragment slot
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)ring;
  const uint32_t wave_lds = ring_lds + (uint32_t)(2 * wave) * kFrag;

#define MOE_ISSUE(step)                                                                          \
  do {                                                                                           \
    const char* ab_ = abase + (size_t)(step) * 64;                                               \
    const char* bb_ = bbase + (size_t)(step) * G * kFrag;                                        \
    const uint32_t st_ = wave_lds + (uint32_t)((step) % kStages) * (32 * kFrag);                 \
    _Pragma("unroll") for (int j = 0; j < 2; ++j) {                                              \
      copy_frag(ab_, aoff[j], st_ + j * kFrag);                                                  \
      copy_frag(bb_, boff[j], st_ + (16 + j) * kFrag);                                           \
    }                                                                                            \
  } while (0)

  floatx4_t acc[kMF][kNF];
#pragma unroll
  for (int i = 0; i < kMF; ++i)
#pragma unroll
    for (int j = 0; j < kNF; ++j) acc[i][j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

#define MOE_COMPUTE(step)                                                                        \
  do {                                                                                           \
    const u32x4_t* st_ = reinterpret_cast<const u32x4_t*>(ring[(step) % kStages]);               \
    bf16x8_t af[kMF], bfr[kNF];                                                                  \
    _Pragma("unroll") for (int i = 0; i < kMF; ++i) af[i] = as_bf16x8(st_[(wm * kMF + i) * 64 + lane]); \
    _Pragma("unroll") for (int j = 0; j < kNF; ++j) bfr[j] = as_bf16x8(st_[(16 + wn * kNF + j) * 64 + lane]); \
    _Pragma("unroll") for (int i = 0; i < kMF; ++i) _Pragma("unroll") for (int j = 0; j < kNF; ++j) \
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);  \
  } while (0)

  // Each wave issues 4 copies per stage, kStages-1 stages ahead.  Before
  // consuming a stage a wave waits until only the copies of later stages are
  // outstanding (copies complete in order), then one barrier makes every
  // wave's copies of that stage visible and frees the stage consumed last.
  const int nsteps = U;
  if (nsteps >= kStages - 1) {
    MOE_ISSUE(0);
    MOE_ISSUE(1);
    MOE_ISSUE(2);
    int ks = 0;
    for (; ks + kStages - 1 < nsteps; ++ks) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(8));
      ring_barrier();
      MOE_ISSUE(ks + kStages - 1);
      MOE_COMPUTE(ks);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(8));
    ring_barrier();
    MOE_COMPUTE(ks);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(4));
    ring_barrier();
    MOE_COMPUTE(ks + 1);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    ring_barrier();
    MOE_COMPUTE(ks + 2);
  } else {
    for (int ks = 0; ks < nsteps; ++ks) {
      MOE_ISSUE(ks);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      ring_barrier();
      MOE_COMPUTE(ks);
      ring_barrier();
    }
  }
#undef MOE_ISSUE
#undef MOE_COMPUTE

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
        const int r = row0 + row;
        if constexpr (EPI == EPI_UP_SWIGLU) {
          const float gv = acc[i][t * 2][q], uv = acc[i][t * 2 + 1][q];
          A.h_out[(size_t)r * A.N + col] = f32_to_bf16(silu(gv) * uv);
        } else if constexpr (EPI == EPI_UP_RELU) {
          const float gv = acc[i][t][q];
          A.h_out[(size_t)r * A.N + col] = f32_to_bf16(gv > 0.0f ? gv : 0.0f);
        } else if constexpr (EPI == EPI_DOWN_ACC) {
          const int a = A.perm[r];
          unsafeAtomicAdd(A.f_out + (size_t)(a / A.topk) * A.N + col, A.topk_w[a] * acc[i][t][q]);
        } else {
          A.f_out[(size_t)r * A.N + col] = acc[i][t][q];
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_ffn_gemm(const GemmArgs& a, int epi, hipStream_t s) {
  const int G = epi == EPI_UP_SWIGLU ? 2 : 1;
  const int tiles_per_block = 4 * (kNF / G);
  const int NB = a.N / 16;
  const long long nbl = (NB + tiles_per_block - 1) / tiles_per_block;
  const long long work = nbl * a.W;
  const dim3 grid((unsigned)((work + 7) / 8 * 8));
  switch (epi) {
    case EPI_UP_SWIGLU: k_ffn_gemm<EPI_UP_SWIGLU><<<grid, kWaves * 64, 0, s>>>(a); break;
    case EPI_UP_RELU: k_ffn_gemm<EPI_UP_RELU><<<grid, kWaves * 64, 0, s>>>(a); break;
    case EPI_DOWN_ACC: k_ffn_gemm<EPI_DOWN_ACC><<<grid, kWaves * 64, 0, s>>>(a); break;
    default: k_ffn_gemm<EPI_DOWN_ROWS><<<grid, kWaves * 64, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

int gemm_rows_per_block() { return kBM; }

}  // namespace moe
