// C ABI of the MoE-layer forward pass (declared in include/moe_gemv.h):
// argument validation, the packed weight store, workspace carving and the
// launch sequence.  Nothing here computes; every step of the layer runs in
// the gfx950 kernels.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <algorithm>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "moe_gemv.h"
#include "moe_index.hpp"
#include "moe_kernels.hpp"

// The plan inputs of a layer: its shape, dtypes and tuning.  Every launch
// choice and the workspace layout are functions of this, T and k (and the
// device's compute-unit count), never of the process environment.
struct LayerCfg {
  int m = 0, p = 0, E = 0, kind = 0, w_dtype = 0;
  moe_tuning tune{};
};

// Host-resident experts (moe_weights_offload): the packed weights of every
// expert in pinned host memory, a few device slots caching experts, the copy
// stream that fills them, and the host-side bookkeeping of one forward.
struct Offload {
  int slots = 0;
  size_t up_stride = 0, dn_stride = 0;  // bytes of one expert's packed gate(+up) and down weights
  char* host = nullptr;                 // pinned: expert e's up at e * (up + dn stride), its down right after
  char* dev = nullptr;                  // slots x (up + dn stride)
  std::vector<int> slot_expert;         // expert held by each slot (-1: none)
  std::vector<long long> slot_used;     // last forward that used each slot (LRU)
  std::vector<hipEvent_t> ev_ready;     // per slot: its copy has landed
  std::vector<hipEvent_t> ev_done;      // per slot: the last FFN that read it has finished
  hipStream_t copy = nullptr;
  hipEvent_t ev_host = nullptr;         // the offsets copied back to the host
  hipEvent_t ev_table = nullptr;        // the per-expert offset table copied to the device
  int32_t* h_offs = nullptr;            // pinned [E+1]
  int32_t* h_table = nullptr;           // pinned [E][2]: each expert's row range
  int32_t* d_table = nullptr;           // device copy of h_table
  long long forwards = 0, hits = 0, misses = 0, bytes = 0;
  std::mutex mu;                        // one streamed forward at a time per handle
};

struct moe_weights {
  LayerCfg c;
  Offload* off = nullptr;  // non-null: experts live in host memory (moe_weights_offload)
  void* buf = nullptr;
  size_t bytes = 0;
  void* up = nullptr;    // packed gate(+up) [E][p/16][U][G] (bf16/int), or fp32 w1 [E][m][p]
  void* up3 = nullptr;   // fp32 SwiGLU only: w3 [E][m][p]
  void* down = nullptr;  // packed down [E][m/16][U][1] (bf16/int), or fp32 w2 [E][p][m]
  float* s_gate = nullptr;         // int8 / int4 / fp8: per-channel scales
  float* s_up = nullptr;
  float* s_down = nullptr;
  uint32_t* mx_up = nullptr;       // MXFP4: packed block scales of the gate(+up) projection
  uint32_t* mx_down = nullptr;     // and of the down projection
};

namespace {

thread_local std::string g_err;

moe_status fail(moe_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

moe_status ok() {
  g_err.clear();
  return MOE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t align256(size_t n) { return (n + 255) & ~size_t(255); }
hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

#define MOE_TRY_HIP(expr)                                                                       \
  do {                                                                                          \
    hipError_t e_ = (expr);                                                                     \
    if (e_ != hipSuccess) return fail(MOE_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

// ---- kernel timing (measurement aid) ------------------------------------------

struct Prof {
  std::mutex mu;
  bool on = false;
  int max = 0, n = 0;
  std::vector<hipEvent_t> ev;
  std::vector<const char*> name;
  std::map<std::string, std::pair<double, int>> total;
};
Prof g_prof;

template <class F>
hipError_t run(const char* name, hipStream_t s, F&& launch) {
  if (g_prof.on && g_prof.n < g_prof.max) {
    const int i = g_prof.n++;
    g_prof.name[i] = name;
    (void)hipEventRecord(g_prof.ev[2 * i], s);
    const hipError_t e = launch();
    (void)hipEventRecord(g_prof.ev[2 * i + 1], s);
    return e;
  }
  return launch();
}


// ---- shape / dtype rules ---------------------------------------------------------

moe_status check_shape(int T, int m, int p, int E, int k) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T=%d must be >= 0", T);
  if (m <= 0 || p <= 0) return fail(MOE_ERR_INVALID_ARG, "m=%d and p=%d must be positive", m, p);
  if (E < 1) return fail(MOE_ERR_INVALID_ARG, "E=%d must be >= 1", E);
  if (k < 1 || k > E) return fail(MOE_ERR_INVALID_ARG, "k=%d must be in [1, E=%d]", k, E);
  if (E > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "E=%d exceeds %d", E, MOE_MAX_EXPERTS);
  if (m % 64 || p % 64) return fail(MOE_ERR_UNSUPPORTED, "m=%d and p=%d must be multiples of 64", m, p);
  if ((long long)T * k > 0x7FFFFFFFLL) return fail(MOE_ERR_UNSUPPORTED, "T*k exceeds 2^31-1");
  return MOE_OK;
}

bool valid_dtype(int d) { return d >= MOE_F32 && d <= MOE_I8A8; }

// Quantised weights (int8, int4, fp8 or MXFP4, each with its scales).
bool quantised(int d) {
  return d == MOE_I8 || d == MOE_I8A8 || d == MOE_I4 || d == MOE_FP8 || d == MOE_FP8A8 || d == MOE_MXFP4;
}

// 8-bit activations: the experts read each token's row quantised to E4M3
// (MOE_FP8A8) or int8 (MOE_I8A8).
bool act8(const LayerCfg& c) { return c.w_dtype == MOE_FP8A8 || c.w_dtype == MOE_I8A8; }
bool act_int8(const LayerCfg& c) { return c.w_dtype == MOE_I8A8; }

// Weight-kind code of the kernels' variants: 0 bf16, 8 int8, 9 fp8, 4 int4,
// 5 MXFP4 (the tens of bits of a weight, and which of its kinds).
int weight_code(int d) {
  switch (d) {
    case MOE_I8:
    case MOE_I8A8: return 8;
    case MOE_FP8:
    case MOE_FP8A8: return 9;
    case MOE_I4: return 4;
    case MOE_MXFP4: return 5;
    default: return 0;
  }
}
int weight_bits(const LayerCfg& c) { return weight_code(c.w_dtype); }
// Narrow (4-bit) weights.
bool nibbles(int d) { return d == MOE_I4 || d == MOE_MXFP4; }

moe_status check_layer(int m, int p, int E, int kind, int w_dtype) {
  if (moe_status rc = check_shape(1, m, p, E, 1)) return rc;
  if (kind != MOE_MLP_RELU && kind != MOE_SWIGLU) return fail(MOE_ERR_INVALID_ARG, "unknown expert kind %d", kind);
  if (!valid_dtype(w_dtype)) return fail(MOE_ERR_UNSUPPORTED, "weight dtype %d unsupported", w_dtype);
  if (nibbles(w_dtype) && (m % 128 || p % 128))
    return fail(MOE_ERR_UNSUPPORTED, "4-bit weights need m=%d and p=%d to be multiples of 128", m, p);
  return MOE_OK;
}

moe_status check_tuning(const moe_tuning& t) {
  auto tri = [](int v) { return v == 0 || v == 1 || v == -1; };
  auto tiles = [](int v) { return v == 0 || v == 1 || v == 2 || v == 4; };
  if (t.ffn_path < MOE_PATH_AUTO || t.ffn_path > MOE_PATH_GEMM)
    return fail(MOE_ERR_INVALID_ARG, "ffn_path %d", t.ffn_path);
  if (!tiles(t.skinny_mt) || !tiles(t.up_ct) || !tiles(t.down_ct))
    return fail(MOE_ERR_INVALID_ARG, "skinny_mt, up_ct and down_ct must be 0, 1, 2 or 4");
  if (!tri(t.skinny_pack) || !tri(t.skinny_splitk) || !tri(t.skinny_shared) || !tri(t.skinny_wide) ||
      !tri(t.skinny_wide_down) || !tri(t.down_rows) || !tri(t.gemm_skip) || !tri(t.route_quant))
    return fail(MOE_ERR_INVALID_ARG, "a switch of the tuning is not 0, 1 or -1");
  if (t.down_ksplit < 0 || t.down_ksplit > 1024) return fail(MOE_ERR_INVALID_ARG, "down_ksplit %d", t.down_ksplit);
  if (t.gemm_cg < 0 || t.gemm_cg > 1024) return fail(MOE_ERR_INVALID_ARG, "gemm_cg %d", t.gemm_cg);
  return MOE_OK;
}

moe_status check_combo(int x_dtype, int w_dtype) {
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "x dtype %d unsupported", x_dtype);
  if (w_dtype == MOE_F32 && x_dtype != MOE_F32)
    return fail(MOE_ERR_UNSUPPORTED, "fp32 weights need fp32 activations");
  if (w_dtype != MOE_F32 && x_dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "bf16/int8/int4/fp8/MXFP4 weights need bf16 activations");
  return MOE_OK;
}

// Which kernels serve the expert FFN.
//  - GEMM: layers whose experts average at least kGemmMinRows rows run the
//    grouped MFMA GEMM on every expert (bf16, int8 or int4 weights).
//  - SKINNY: decode-sized layers.
//  - F32: fp32 layers.
// (A hybrid of the two, hot experts on the GEMM on a second stream and the
// rest on the decode kernels, measured slower than the decode kernels alone on
// the skewed Phi-3.5-shaped layer and is not offered.)
enum class Path { F32, SKINNY, GEMM };
constexpr int kGemmMinRows = 128;
// Grouped GEMM work order: column blocks per group (each group takes all of
// its expert's row blocks; the ~32 workgroups resident on an XCD share the
// group's tiles in L2).  Measured on the Mixtral prefill layers: 2 ahead of
// 3-8 by 0.7-2 % for 256-row blocks (bf16, int8; fp8 equal); 8 for int4's
// 128-row blocks, whose activation tile per stage is twice its weight tile
// (4.3 % ahead of 2, 1 % of 4).
int gemm_cg_default(int qb) { return qb == 4 ? 8 : 2; }

// 0 ("automatic") or the tuning's value.
int tuned(int v, int dflt) { return v != 0 ? v : dflt; }
bool tuned_on(int v, bool dflt) { return v == 0 ? dflt : v > 0; }

// The weight kind the grouped GEMM multiplies: MXFP4 layers expand their
// weights exactly to packed bf16 in the workspace first (each E2M1 value
// times its E8M0 block scale is a bf16 value) and run the bf16 kernel, whose
// ring has no room to stage block scales beside each weight stage.
int gemm_qb(const LayerCfg& c) { return c.w_dtype == MOE_MXFP4 ? 0 : weight_bits(c); }

// The GEMM addresses packed activations and one projection's packed weights
// with 32-bit byte offsets from a uniform base.
bool gemm_fits(const LayerCfg& c, int T, int k) {
  if (c.w_dtype == MOE_F32) return false;
  const unsigned long long lim = 1ull << 32;
  const int qb = gemm_qb(c);
  const unsigned long long G = c.kind == MOE_SWIGLU ? 2 : 1;
  const unsigned long long up_w = moe::packed_bytes(c.E, c.m, c.p, (int)G, qb);
  const unsigned long long dn_w = moe::packed_bytes(c.E, c.p, c.m, 1, qb);
  const unsigned long long rows = (unsigned long long)moe::packed_rows_alloc((long long)T * k, c.E);
  return up_w < lim && dn_w < lim && rows * c.m * 2 < lim && rows * c.p * 2 < lim;
}

Path ffn_path(const LayerCfg& c, int T, int k) {
  if (c.w_dtype == MOE_F32) return Path::F32;
  const bool fits = gemm_fits(c, T, k);
  if (c.tune.ffn_path == MOE_PATH_GEMM) return fits ? Path::GEMM : Path::SKINNY;
  if (c.tune.ffn_path == MOE_PATH_SKINNY || !fits) return Path::SKINNY;
  const long long n = (long long)T * k;
  return n >= (long long)kGemmMinRows * c.E ? Path::GEMM : Path::SKINNY;
}

// M tiles (16 rows each) per work item of the skinny kernels, from the mean
// rows per expert.
int skinny_mt(const LayerCfg& c, int T, int k) {
  const long long avg = ((long long)T * k + c.E - 1) / c.E;
  const int mt = tuned(c.tune.skinny_mt, avg <= 12 ? 1 : (avg <= 24 ? 2 : 4));
  if (quantised(c.w_dtype)) return mt <= 1 ? 1 : 2;  // the integer kernels stop at two M tiles
  return mt <= 1 ? 1 : (mt == 2 ? 2 : 4);
}

// With four M tiles per work item the skinny kernels read their activations
// as packed 1 KiB fragments (x gathered by k_pack_rows, H written packed by
// the up projection): one contiguous load per tile and K unit instead of 16
// half-line rows, which measured as the dominant cost of the skewed layer
// (-11 % there).  With one or two bf16 tiles the extra packing launch costs
// more than it saves, so rows are gathered directly.  At decode sizes the
// dispatch is derived by the first kernel either way: the packing, or the up
// projection's prologue.
bool skinny_packed(const LayerCfg& c, int T, int k) {
  if (c.w_dtype == MOE_F32) return false;
  // int8 (int4) weights span 64 (128) k per unit, so two M tiles already
  // read four (eight) activation fragments per unit: packed and shared
  // measured ahead there
  const bool dflt = skinny_mt(c, T, k) >= (quantised(c.w_dtype) ? 2 : 4);
  return tuned_on(c.tune.skinny_pack, dflt);
}

// Waves split the reduction unless the activations are packed (measured).
bool skinny_splitk(const LayerCfg& c, int T, int k) { return tuned_on(c.tune.skinny_splitk, !skinny_packed(c, T, k)); }

// Packed rows with the columns split over the waves: every wave of a
// workgroup reads the same activation fragments, so they are copied into
// LDS once per workgroup.
bool skinny_shared(const LayerCfg& c, int T, int k) {
  return skinny_packed(c, T, k) && !skinny_splitk(c, T, k) && tuned_on(c.tune.skinny_shared, true);
}

// Decode layers write the down projection's unweighted rows (one set per
// reduction slice) and finish with the combine kernel, instead of adding
// weighted rows into an fp32 accumulator with atomics: on the skewed layer
// one more slice of atomics cost 20 us, about 10^11 adds/s, while the rows
// and the combine move a few MB.
bool skinny_rows_combine(const LayerCfg& c) { return tuned_on(c.tune.down_rows, true); }

// Reduction slices per down-projection work item.  Splitting adds partial
// rows (or atomics); measured on the decode layers (512 to 1536 work items)
// one slice is as fast or faster, so only very small launches split.
int down_ksplit(const LayerCfg& c, long long items) {
  if (c.tune.down_ksplit > 0) return c.tune.down_ksplit;
  if (items >= 512) return 1;
  if (items >= 256) return 2;
  return 4;
}

// Column tiles per wave: enough to amortise each activation load over
// several weight streams when the activation side is wide (several M tiles,
// or int8 weights whose 16-byte unit spans 64 k).  The down projection (one
// stream per tile) takes 4 (2 with four M tiles, for registers); measured on
// the decode layers.
int skinny_ct(int mt, int qb, int g, int forced) {
  if (forced > 0) return forced >= 4 ? 4 : (forced >= 2 ? 2 : 1);
  const int aw = mt * (qb >= 8 ? 2 : (qb >= 4 ? 4 : 1));
  if (aw <= 1 && g > 1) return 1;
  if (mt >= 4) return 2;
  return 4;
}

// Compute units of the current device (cached per device).
int device_cus() {
  static std::mutex mu;
  static std::map<int, int> cus;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 256;
  }
  std::lock_guard<std::mutex> lk(mu);
  auto it = cus.find(dev);
  if (it != cus.end()) return it->second;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    n = 256;
  }
  cus[dev] = n;
  return n;
}

// The int8 down projection with shared activations (two M tiles, two waves
// per SIMD, so two resident workgroups per CU): two column tiles per wave and
// the fewest reduction slices (1, 2, 4) whose workgroups fill one round of
// the resident slots, counted from the expected number of (expert, chunk)
// pairs.  Measured on the int8 decode layer: 92 us against 99 us for four
// tiles and four slices, 124 us for one slice.
void int8_down_shape(const LayerCfg& c, int T, int k, int R, int* ct, int* ks) {
  const long long n = (long long)T * k;
  const long long pairs = std::min<long long>(c.E, n) + std::max<long long>(0, n - (long long)c.E * R) / R;
  *ct = 2;
  const long long blocks1 = (long long)moe::skinny_groups(c.m, *ct) * pairs;
  const long long slots = 2LL * device_cus();
  *ks = blocks1 * 10 >= slots * 9 ? 1 : (blocks1 * 2 * 10 >= slots * 9 ? 2 : 4);
  *ks = std::max(1, std::min(*ks, c.p / 64));
}

// Launch shape of the skinny down projection inside the layer: column tiles
// per wave and reduction slices.  Shared by the workspace layout (the
// unweighted rows are kept per slice) and the launch.
struct DownShape {
  int ct, ks;
};
DownShape skinny_down_shape(const LayerCfg& c, int T, int k) {
  const int mt = skinny_mt(c, T, k);
  const int qb = weight_bits(c);
  const bool splitk = skinny_splitk(c, T, k);
  const int R = moe::skinny_rows(mt);
  const int Wp = c.E + (int)((long long)T * k / R);
  DownShape d{skinny_ct(mt, qb, 1, c.tune.down_ct), 1};
  d.ks = down_ksplit(c, (long long)(splitk ? c.m / 16 / d.ct : moe::skinny_groups(c.m, d.ct)) * Wp);
  if (qb != 0 && skinny_shared(c, T, k) && c.tune.down_ct <= 0 && c.tune.down_ksplit <= 0)
    int8_down_shape(c, T, k, R, &d.ct, &d.ks);
  d.ks = std::max(1, std::min(d.ks, c.p / 64));
  return d;
}

// Workspace carving, in the order listed.
struct Ws {
  size_t logits, idx, w, counts, offsets, perm, inv, xn, xq, xs, h, yacc, yperm, xp, rs, wdq, total;
};

Ws ws_layout(const LayerCfg& c, int T, int k) {
  Ws L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t n = (size_t)T * k;
  const bool f32 = c.w_dtype == MOE_F32;
  L.logits = take((size_t)T * c.E * 4);
  L.idx = take(n * 4);
  L.w = take(n * 4);
  L.counts = take((size_t)c.E * 4);
  L.offsets = take((size_t)(c.E + 1) * 4);
  L.perm = take(n * 4);
  L.inv = take(n * 4);
  // the normalised input rows of the fused forward (x's dtype)
  L.xn = take((size_t)T * c.m * (f32 ? 4 : 2));
  // fp8 activations: the quantised rows (bf16 values) and the per-token scales
  L.xq = act8(c) ? take((size_t)T * c.m * 2) : off;
  L.xs = act8(c) ? take((size_t)T * 4) : off;
  const Path path = ffn_path(c, T, k);
  const bool gemm = path == Path::GEMM;
  const bool spack = path == Path::SKINNY && skinny_packed(c, T, k);
  // the grouped GEMM and the packed skinny kernels keep H and the gathered x
  // in the packed row layout
  const size_t prows = (size_t)moe::packed_rows_alloc((long long)n, c.E);
  L.h = take((gemm || spack ? prows : n) * (size_t)c.p * (f32 ? 4 : 2));
  L.yacc = take((size_t)T * c.m * 4);
  const size_t row_sets =
      gemm ? 1 : (path == Path::SKINNY && skinny_rows_combine(c) ? (size_t)skinny_down_shape(c, T, k).ks : 0);
  L.yperm = row_sets ? take(row_sets * n * (size_t)c.m * 4) : off;
  L.xp = gemm || spack ? take(prows * (size_t)c.m * 2) : off;
  // fp8 activations on the grouped GEMM: each packed row's token scale
  L.rs = gemm && act8(c) ? take(prows * 4) : off;
  // MXFP4 on the grouped GEMM: one projection's weights expanded to packed bf16
  const int G = c.kind == MOE_SWIGLU ? 2 : 1;
  L.wdq = gemm && c.w_dtype == MOE_MXFP4
              ? take(std::max(moe::packed_bytes(c.E, c.m, c.p, G, 0), moe::packed_bytes(c.E, c.p, c.m, 1, 0)))
              : off;
  L.total = off;
  return L;
}

// Inputs and outputs of the two FFN projections.
struct FfnIo {
  const void* x;
  int T, k;
  const int32_t* topk_idx;  // non-null: the first FFN kernel derives the dispatch
  int32_t *counts, *offsets, *perm, *inv;
  const float* topk_w;
  void* h;                  // hidden activations [T*k][p] (packed rows on the GEMM path)
  void* xp;                 // packed paths: x rows gathered into the packed row layout
  const float* xs = nullptr;  // fp8 activations: each token's scale (x is then the quantised rows)
  const uint8_t* xc = nullptr;  // fp8 activations on the grouped GEMM: the rows' E4M3 codes [T][m]
  float* rs = nullptr;          // and each packed row's scale
  float* down_out;          // y_acc [T][m] (combine) or y_perm [T*k][m]
  bool combine;             // inside the layer: the weighted combine follows
  float* yperm;             // with combine on the grouped-GEMM path, or the skinny path with
                            // rows: unweighted rows [slices][T*k][m]
  int* slices;              // set to the number of row slices written to yperm
  long long rows = -1;      // >= 0: the dispatched rows this call serves (one expert's, when
                            // streaming experts); sizes the launch grids tightly
  void* wdq = nullptr;      // MXFP4 on the grouped GEMM: room for one projection's weights in bf16
};

// The dispatched rows an FFN call serves: all T*k, or the caller's bound.
long long ffn_rows(const FfnIo& io) { return io.rows >= 0 ? io.rows : (long long)io.T * io.k; }

// 8-bit activations: where the FFN's quantised input rows go in the
// workspace: as bf16 values for the decode kernels, as E4M3 (int8) codes for
// the grouped GEMM, whose first projection multiplies codes on the fp8 (int8)
// matrix cores; and each token's scale.
struct QuantOut {
  uint16_t* xq;  // bf16 values (decode kernels) or null
  uint8_t* xc;   // codes (grouped GEMM) or null
  float* xs;
};
QuantOut quant_out(const LayerCfg& c, const FfnIo& io, char* ws, const Ws& L) {
  const bool gemm = ffn_path(c, io.T, io.k) == Path::GEMM;
  return QuantOut{gemm ? nullptr : reinterpret_cast<uint16_t*>(ws + L.xq),
                  gemm ? reinterpret_cast<uint8_t*>(ws + L.xq) : nullptr, reinterpret_cast<float*>(ws + L.xs)};
}

// Quantises the FFN's input rows (per token, into the workspace; already
// done when in_route, by the routing pass) and points io at them, with the
// packed rows' scales to come on the grouped GEMM.
moe_status quant_input(const LayerCfg& c, FfnIo& io, char* ws, const Ws& L, hipStream_t s, bool in_route = false) {
  if (!act8(c)) return MOE_OK;
  const bool gemm = ffn_path(c, io.T, io.k) == Path::GEMM;
  const QuantOut q = quant_out(c, io, ws, L);
  uint16_t* xq = q.xq;
  uint8_t* xc = q.xc;
  float* xs = q.xs;
  const uint16_t* x = static_cast<const uint16_t*>(io.x);
  if (!in_route)
    MOE_TRY_HIP(run("quant_rows", s, [&] { return moe::launch_quant_rows(x, io.T, c.m, act_int8(c), xq, xc, xs, s); }));
  if (gemm) {
    io.xc = xc;
    io.rs = reinterpret_cast<float*>(ws + L.rs);
  } else {
    io.x = xq;
  }
  io.xs = xs;
  return MOE_OK;
}

// Gathers x rows into the packed row layout.
moe_status run_pack(const LayerCfg& c, const FfnIo& io, hipStream_t s) {
  moe::PackArgs pk{};
  pk.x = static_cast<const uint16_t*>(io.x);
  pk.perm = io.perm;
  pk.offsets = io.offsets;
  pk.out = static_cast<uint16_t*>(io.xp);
  pk.T = io.T;
  pk.rows = io.rows >= 0 ? (int)io.rows : -1;
  pk.K = c.m;
  pk.E = c.E;
  pk.topk = io.k;
  if (io.topk_idx) {  // the dispatch is derived while packing
    pk.topk_idx = io.topk_idx;
    pk.d_counts = io.counts;
    pk.d_offsets = io.offsets;
    pk.d_perm = io.perm;
    pk.d_inv = io.inv;
  }
  MOE_TRY_HIP(run("pack_rows", s, [&] { return moe::launch_pack_rows(pk, s); }));
  return MOE_OK;
}

// Grouped GEMM over every expert: packed x -> packed H -> unweighted rows in
// dispatch order (y_rows).
moe_status run_gemm(const moe_weights* W, const FfnIo& io, float* y_rows, hipStream_t s) {
  const LayerCfg& c = W->c;
  const long long n = ffn_rows(io);
  const int qb = gemm_qb(c);
  const int bm = moe::gemm_rows_per_block(qb);
  const bool mx = c.w_dtype == MOE_MXFP4;
  if (mx && !io.wdq) return fail(MOE_ERR_WORKSPACE, "MXFP4 grouped GEMM without its weight buffer (internal)");
  const int G = c.kind == MOE_SWIGLU ? 2 : 1;
  moe::GemmArgs g{};
  g.offsets = io.offsets;
  g.E = c.E;
  // row blocks: at most n/bm full ones plus one partial per expert
  g.W = (int)(n / bm + std::min<long long>(c.E, n));
  if (g.W <= 0) return MOE_OK;  // no rows
  g.cg = tuned(c.tune.gemm_cg, gemm_cg_default(qb));
  // experts averaging under one full row block: skip the products of empty
  // row fragments
  g.skip_empty = tuned_on(c.tune.gemm_skip, n < (long long)bm * c.E);
  // up: packed x -> packed H
  g.w = W->up;
  g.scale0 = W->s_gate;
  g.scale1 = W->s_up;
  if (mx) {
    MOE_TRY_HIP(run("expand_w", s, [&] {
      return moe::launch_expand_fp4(W->up, W->mx_up, io.wdq, io.offsets, c.E, c.m, c.p, G, s);
    }));
    g.w = io.wdq;
  }
  g.act = static_cast<const uint16_t*>(io.xp);
  g.h_out = static_cast<uint16_t*>(io.h);
  g.K = c.m;
  g.N = c.p;
  const int up_epi = c.kind == MOE_SWIGLU ? moe::EPI_UP_SWIGLU : moe::EPI_UP_RELU;
  if (io.xc) {
    // fp8 activations: the codes' packed units and row scales, then the
    // up projection on the fp8 matrix cores
    moe::PackA8Args pk{};
    pk.codes = io.xc;
    pk.scale = io.xs;
    pk.perm = io.perm;
    pk.offsets = io.offsets;
    pk.out = static_cast<uint8_t*>(io.xp);
    pk.row_scale = io.rs;
    pk.T = io.T;
    pk.K = c.m;
    pk.E = c.E;
    pk.topk = io.k;
    pk.rows = io.rows >= 0 ? (int)io.rows : -1;
    MOE_TRY_HIP(run("pack_rows", s, [&] { return moe::launch_pack_rows_a8(pk, s); }));
    g.act = reinterpret_cast<const uint16_t*>(io.xp);
    MOE_TRY_HIP(run("gemm_up", s, [&] { return moe::launch_ffn_gemm_a8(g, io.rs, up_epi, act_int8(c), s); }));
  } else {
    MOE_TRY_HIP(run("gemm_up", s, [&] { return moe::launch_ffn_gemm(g, up_epi, qb, s); }));
  }
  // down: packed H -> rows in dispatch order
  g.w = W->down;
  if (mx) {  // the up projection has read the buffer by now (stream order)
    MOE_TRY_HIP(run("expand_w", s, [&] {
      return moe::launch_expand_fp4(W->down, W->mx_down, io.wdq, io.offsets, c.E, c.p, c.m, 1, s);
    }));
    g.w = io.wdq;
  }
  g.scale0 = W->s_down;
  g.scale1 = nullptr;
  g.act = static_cast<const uint16_t*>(io.h);
  g.h_out = nullptr;
  g.f_out = y_rows;
  g.K = c.p;
  g.N = c.m;
  MOE_TRY_HIP(run("gemm_down", s, [&] { return moe::launch_ffn_gemm(g, moe::EPI_DOWN_ROWS, qb, s); }));
  return MOE_OK;
}

// Skinny decode kernels over every expert.
moe_status run_skinny(const moe_weights* W, const FfnIo& io, hipStream_t s) {
  const LayerCfg& c = W->c;
  const int m = c.m, p = c.p, E = c.E, T = io.T, k = io.k;
  const bool swiglu = c.kind == MOE_SWIGLU;
  const int qb = weight_bits(c);
  const bool i8 = qb != 0;  // integer weights (int8 or int4)
  const int mt = skinny_mt(c, T, k);
  const bool packed = skinny_packed(c, T, k);
  const bool splitk = skinny_splitk(c, T, k);
  if (packed)
    if (moe_status rc = run_pack(c, io, s)) return rc;
  const int R = moe::skinny_rows(mt);
  moe::SkinnyArgs a{};
  a.perm = io.perm;
  a.offsets = io.offsets;
  a.topk = k;
  a.T = T;
  a.E = E;
  const long long nrows = ffn_rows(io);
  a.W = (int)std::max<long long>(1, std::min<long long>(E + nrows / R, nrows));
  a.topk_w = io.topk_w;
  a.ksplit = 1;
  if ((long long)(p / 16) * a.W * 4 >= 0x7FFFFFF0LL || (long long)(m / 16) * a.W * 4 >= 0x7FFFFFF0LL)
    return fail(MOE_ERR_UNSUPPORTED, "too many work items for one launch (T*k=%lld)", (long long)T * k);
  // up: gate (+up) projection with the activation epilogue, x -> H
  a.w = W->up;
  a.scale0 = W->s_gate;
  a.scale1 = W->s_up;
  a.mx = W->mx_up;
  a.act = static_cast<const uint16_t*>(packed ? io.xp : io.x);
  a.h_out = static_cast<uint16_t*>(io.h);
  a.K = m;
  a.N = p;
  a.gather = packed ? 0 : 1;
  a.packed = packed;
  a.h_packed = packed;
  a.shared_act = skinny_shared(c, T, k);
  // the dispatch is derived in this kernel's prologue (gathered rows) or was
  // derived by the row packing
  if (io.topk_idx && !packed) {
    a.topk_idx = io.topk_idx;
    a.d_counts = io.counts;
    a.d_offsets = io.offsets;
    a.d_perm = io.perm;
    a.d_inv = io.inv;
  }
  // Experts holding more than one chunk of four M tiles (the hot experts of a
  // skewed routing) would have their weights streamed once per 64-row chunk.
  // With shared activations both projections serve them with twelve-tile
  // work items instead (192-row chunks), in the same launch as the four-tile
  // items of the other experts.  For the down projection the split launch
  // runs at two waves per SIMD where the four-tile kernel alone runs at four;
  // with only the activation fragments that hold real rows copied, the split
  // still measured ahead on the skewed layer (167 against 173 us).
  const int up_epi = swiglu ? moe::EPI_UP_SWIGLU : moe::EPI_UP_RELU;
  const int up_ct = skinny_ct(mt, qb, swiglu ? 2 : 1, c.tune.up_ct);
  const bool wide =
      mt == 4 && up_ct == 2 && a.shared_act && !i8 && !a.topk_idx && tuned_on(c.tune.skinny_wide, true);
  constexpr int kWideMt = 12;
  moe::SkinnyArgs aw{};
  if (wide) {
    a.max_rows = R;
    aw = a;
    aw.max_rows = 0;
    aw.min_rows = R;
    // chunks: at most n/192 full ones plus one partial per expert above R rows
    const long long n = nrows;
    aw.W = (int)(n / moe::skinny_rows(kWideMt) + n / (R + 1) + 1);
  }
  MOE_TRY_HIP(run("ffn_up", s, [&]() -> hipError_t {
    return wide ? moe::launch_ffn_skinny_split(a, aw, up_epi, s)
                : moe::launch_ffn_skinny(a, up_epi, qb, mt, up_ct, splitk, s);
  }));
  // down: H -> unweighted rows (or the weighted combine)
  a.topk_idx = nullptr;
  a.d_counts = a.d_offsets = a.d_perm = a.d_inv = nullptr;
  a.w = W->down;
  a.scale0 = W->s_down;
  a.scale1 = nullptr;
  a.mx = W->mx_down;
  a.act = static_cast<const uint16_t*>(io.h);
  a.h_out = nullptr;
  a.f_out = io.down_out;
  a.K = p;
  a.N = m;
  a.gather = 0;
  a.packed = packed;
  a.h_packed = 0;
  const DownShape ds = skinny_down_shape(c, T, k);
  // inside the layer: unweighted rows per reduction slice for the combine,
  // or weighted rows added into y_acc; alone: unweighted rows, one slice
  const bool rows = io.combine && io.yperm && skinny_rows_combine(c);
  if (io.combine) a.ksplit = ds.ks;
  if (rows) {
    a.f_out = io.yperm;
    a.slice_stride = (size_t)T * k * m;
  }
  if (io.slices) *io.slices = rows ? a.ksplit : 1;
  const int dn_epi = io.combine && !rows ? moe::EPI_DOWN_ACC : moe::EPI_DOWN_ROWS;
  const bool wide_dn = wide && a.ksplit == 1 && ds.ct == 2 && tuned_on(c.tune.skinny_wide_down, true);
  if (wide && !wide_dn) a.max_rows = 0;  // the four-tile launch serves every expert
  if (wide_dn) {
    const int W_wide = aw.W;
    aw = a;
    aw.W = W_wide;
    aw.max_rows = 0;
    aw.min_rows = R;
  }
  MOE_TRY_HIP(run("ffn_down", s, [&]() -> hipError_t {
    return wide_dn ? moe::launch_ffn_skinny_split(a, aw, dn_epi, s)
                   : moe::launch_ffn_skinny(a, dn_epi, qb, mt, ds.ct, splitk, s);
  }));
  return MOE_OK;
}

moe_status run_ffn(const moe_weights* W, const FfnIo& io, hipStream_t s) {
  const LayerCfg& c = W->c;
  const int m = c.m, p = c.p, E = c.E, T = io.T, k = io.k;
  const bool swiglu = c.kind == MOE_SWIGLU;
  switch (ffn_path(c, T, k)) {
    case Path::F32: {
      moe::F32Args a{};
      a.perm = io.perm;
      a.offsets = io.offsets;
      a.topk = k;
      a.E = E;
      a.W = E + (int)((long long)T * k / 16);
      a.topk_w = io.topk_w;
      // up: x [T][m] -> H [T*k][p]
      a.w1 = static_cast<const float*>(W->up);
      a.w3 = swiglu ? static_cast<const float*>(W->up3) : nullptr;
      a.act = static_cast<const float*>(io.x);
      a.out = static_cast<float*>(io.h);
      a.K = m;
      a.N = p;
      a.gather = 1;
      a.epi = swiglu ? moe::EPI_UP_SWIGLU : moe::EPI_UP_RELU;
      MOE_TRY_HIP(run("ffn_f32_up", s, [&] { return moe::launch_ffn_f32(a, s); }));
      // down: H -> y
      a.w1 = static_cast<const float*>(W->down);
      a.w3 = nullptr;
      a.act = static_cast<const float*>(io.h);
      a.out = io.down_out;
      a.K = p;
      a.N = m;
      a.gather = 0;
      a.epi = io.combine ? moe::EPI_DOWN_ACC : moe::EPI_DOWN_ROWS;
      MOE_TRY_HIP(run("ffn_f32_down", s, [&] { return moe::launch_ffn_f32(a, s); }));
      return MOE_OK;
    }
    case Path::GEMM:
      if (!io.xc)  // (fp8 activations pack their codes in run_gemm)
        if (moe_status rc = run_pack(c, io, s)) return rc;
      // with the combine following: unweighted rows into y_perm
      return run_gemm(W, io, io.combine ? io.yperm : io.down_out, s);
    default:
      return run_skinny(W, io, s);
  }
}

// ---- host-resident experts --------------------------------------------------
//
// The pages' expert prefetch (HARMOEny article, section 3.2: compute one
// expert while the next one is fetched, so the transfer hides behind the
// compute once an expert holds enough tokens; GPU-cache article, sections 2
// and 3.2: a device cache of experts, and weight copies on a second stream)
// on one GPU.  After routing, the expert row counts come back to the host
// (one synchronisation); the touched experts are then run one at a time,
// those already in a slot first, then the misses by decreasing rows, each
// miss copied into a slot on the copy stream while the experts before it
// compute.  A slot is refilled only after the FFN that read it finished.
//
// Each expert runs the ordinary kernels on a one-expert view of the layer:
// its weights at its slot, its scales, its row range (a [2] offsets array),
// and the launch choices of the whole layer pinned in the view's tuning, so
// every row is computed exactly as by the resident forward.

// The whole layer's launch choices for (T, k), pinned so that a one-expert
// view makes the same ones.
moe_tuning pinned_tuning(const LayerCfg& c, int T, int k) {
  moe_tuning t = c.tune;
  const Path path = ffn_path(c, T, k);
  t.ffn_path = path == Path::GEMM ? MOE_PATH_GEMM : MOE_PATH_SKINNY;
  const int qb = weight_bits(c);
  if (path == Path::GEMM) {
    const long long n = (long long)T * k;
    t.gemm_skip = tuned_on(c.tune.gemm_skip, n < (long long)moe::gemm_rows_per_block(gemm_qb(c)) * c.E) ? 1 : -1;
    t.gemm_cg = tuned(c.tune.gemm_cg, gemm_cg_default(gemm_qb(c)));
  } else {
    const int mt = skinny_mt(c, T, k);
    t.skinny_mt = mt;
    t.skinny_pack = skinny_packed(c, T, k) ? 1 : -1;
    t.skinny_splitk = skinny_splitk(c, T, k) ? 1 : -1;
    t.skinny_shared = skinny_shared(c, T, k) ? 1 : -1;
    t.up_ct = skinny_ct(mt, qb, c.kind == MOE_SWIGLU ? 2 : 1, c.tune.up_ct);
    const DownShape ds = skinny_down_shape(c, T, k);
    t.down_ct = ds.ct;
    t.down_ksplit = ds.ks;
    t.down_rows = skinny_rows_combine(c) ? 1 : -1;
  }
  return t;
}

moe_status run_ffn_streamed(const moe_weights* W, const FfnIo& io, hipStream_t s) {
  Offload& O = *W->off;
  const LayerCfg& c = W->c;
  const int E = c.E, m = c.m, p = c.p;
  std::lock_guard<std::mutex> lk(O.mu);
  // the previous forward's table copy has finished reading h_table
  MOE_TRY_HIP(hipEventSynchronize(O.ev_table));
  MOE_TRY_HIP(hipMemcpyAsync(O.h_offs, io.offsets, (size_t)(E + 1) * 4, hipMemcpyDeviceToHost, s));
  MOE_TRY_HIP(hipEventRecord(O.ev_host, s));
  MOE_TRY_HIP(hipEventSynchronize(O.ev_host));
  const long long fwd = ++O.forwards;

  // touched experts: those in a slot first, then the others by decreasing rows
  std::vector<int> resident, missing;
  std::vector<int> slot_of_expert(E, -1);
  for (int sl = 0; sl < O.slots; ++sl)
    if (O.slot_expert[sl] >= 0) slot_of_expert[O.slot_expert[sl]] = sl;
  for (int e = 0; e < E; ++e) {
    const int rows = O.h_offs[e + 1] - O.h_offs[e];
    if (rows < 0 || O.h_offs[e + 1] > io.T * io.k) return fail(MOE_ERR_INVALID_ARG, "offsets are not a dispatch");
    O.h_table[2 * e] = O.h_offs[e];
    O.h_table[2 * e + 1] = O.h_offs[e + 1];
    if (rows == 0) continue;
    (slot_of_expert[e] >= 0 ? resident : missing).push_back(e);
  }
  std::stable_sort(missing.begin(), missing.end(), [&](int a, int b) {
    return O.h_offs[a + 1] - O.h_offs[a] > O.h_offs[b + 1] - O.h_offs[b];
  });
  std::vector<int> order = resident;
  order.insert(order.end(), missing.begin(), missing.end());
  MOE_TRY_HIP(hipMemcpyAsync(O.d_table, O.h_table, (size_t)E * 2 * 4, hipMemcpyHostToDevice, s));
  MOE_TRY_HIP(hipEventRecord(O.ev_table, s));

  // slots free for misses: those holding no touched expert, least recently used first
  std::vector<int> reusable;
  for (int sl = 0; sl < O.slots; ++sl) {
    const int e = O.slot_expert[sl];
    if (e < 0 || O.h_offs[e + 1] == O.h_offs[e]) reusable.push_back(sl);
  }
  std::stable_sort(reusable.begin(), reusable.end(), [&](int a, int b) { return O.slot_used[a] < O.slot_used[b]; });
  size_t reuse_head = 0;

  // the one-expert view's launch choices (of the whole layer)
  moe_weights V;
  V.c = c;
  V.c.E = 1;
  V.c.tune = pinned_tuning(c, io.T, io.k);
  const size_t up_dw = W->mx_up ? moe::packed_mx_scale_bytes(1, m, p, c.kind == MOE_SWIGLU ? 2 : 1) / 4 : 0;
  const size_t dn_dw = W->mx_down ? moe::packed_mx_scale_bytes(1, p, m, 1) / 4 : 0;

  const int n = (int)order.size();
  std::vector<int> slot_at(n, -1);
  int next = 0;  // next order position whose slot is not yet arranged
  for (int i = 0; i < n; ++i) {
    // arrange slots (and issue copies) as far ahead as free slots allow
    while (next < n) {
      const int e = order[next];
      if (slot_of_expert[e] >= 0) {
        slot_at[next++] = slot_of_expert[e];
        ++O.hits;
        continue;
      }
      if (reuse_head >= reusable.size()) break;
      const int sl = reusable[reuse_head++];
      if (O.slot_expert[sl] >= 0) slot_of_expert[O.slot_expert[sl]] = -1;
      O.slot_expert[sl] = e;
      slot_of_expert[e] = sl;
      char* dst = O.dev + (size_t)sl * (O.up_stride + O.dn_stride);
      const char* src = O.host + (size_t)e * (O.up_stride + O.dn_stride);
      MOE_TRY_HIP(hipStreamWaitEvent(O.copy, O.ev_done[sl], 0));
      MOE_TRY_HIP(hipMemcpyAsync(dst, src, O.up_stride + O.dn_stride, hipMemcpyHostToDevice, O.copy));
      MOE_TRY_HIP(hipEventRecord(O.ev_ready[sl], O.copy));
      O.bytes += (long long)(O.up_stride + O.dn_stride);
      ++O.misses;
      slot_at[next++] = sl;
    }
    if (slot_at[i] < 0) return fail(MOE_ERR_HIP, "no expert slot free (internal)");
    const int e = order[i], sl = slot_at[i];
    char* base = O.dev + (size_t)sl * (O.up_stride + O.dn_stride);
    V.up = base;
    V.down = base + O.up_stride;
    V.s_gate = W->s_gate ? W->s_gate + (size_t)e * p : nullptr;
    V.s_up = W->s_up ? W->s_up + (size_t)e * p : nullptr;
    V.s_down = W->s_down ? W->s_down + (size_t)e * m : nullptr;
    V.mx_up = W->mx_up ? W->mx_up + (size_t)e * up_dw : nullptr;
    V.mx_down = W->mx_down ? W->mx_down + (size_t)e * dn_dw : nullptr;
    FfnIo ie = io;
    ie.offsets = O.d_table + 2 * e;
    ie.topk_idx = nullptr;
    ie.rows = O.h_offs[e + 1] - O.h_offs[e];  // exact grids: the work spreads over every XCD
    MOE_TRY_HIP(hipStreamWaitEvent(s, O.ev_ready[sl], 0));
    if (moe_status rc = run_ffn(&V, ie, s)) return rc;
    MOE_TRY_HIP(hipEventRecord(O.ev_done[sl], s));
    O.slot_used[sl] = fwd;
    reusable.push_back(sl);  // refillable once this expert's FFN is done
  }
  return MOE_OK;
}

moe_status check_weights_match(const moe_weights* w, int m, int p, int E) {
  if (!w) return fail(MOE_ERR_INVALID_ARG, "weights handle is NULL");
  if (w->c.m != m || w->c.p != p || w->c.E != E)
    return fail(MOE_ERR_INVALID_ARG, "shape (m=%d,p=%d,E=%d) does not match the weights (m=%d,p=%d,E=%d)", m, p, E,
                w->c.m, w->c.p, w->c.E);
  return MOE_OK;
}

// The workspace a call received, checked against the layout it needs.
moe_status check_workspace(const Ws& L, const void* workspace, size_t ws_bytes) {
  if (!workspace || ws_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total, workspace ? ws_bytes : 0);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(MOE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_err.c_str(); }

int moe_abi_version(void) { return 2; }

moe_status moe_weights_create(int m, int p, int E, int kind, int w_dtype, const void* w1, const void* w_up,
                              const void* w2, const void* s1, const void* s_up, const void* s2, void* stream,
                              moe_weights** out) {
  if (!out) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (moe_status rc = check_layer(m, p, E, kind, w_dtype)) return rc;
  const bool swiglu = kind == MOE_SWIGLU;
  if (!w1 || !w2 || (swiglu && !w_up)) return fail(MOE_ERR_INVALID_ARG, "required weight pointer is NULL");
  if (!swiglu && w_up) return fail(MOE_ERR_INVALID_ARG, "w_up must be NULL for the ReLU MLP");
  const bool i8 = quantised(w_dtype);
  const bool mx = w_dtype == MOE_MXFP4;
  const int qb = weight_code(w_dtype);
  if (i8 && (!s1 || !s2 || (swiglu && !s_up))) return fail(MOE_ERR_INVALID_ARG, "quantised weights need their scales");
  if (!i8 && (s1 || s2 || s_up)) return fail(MOE_ERR_INVALID_ARG, "scales are only for quantised weights");
  if (!aligned16(w1) || !aligned16(w2) || (w_up && !aligned16(w_up)) || (s1 && !aligned16(s1)) ||
      (s2 && !aligned16(s2)) || (s_up && !aligned16(s_up)))
    return fail(MOE_ERR_INVALID_ARG, "weight pointers must be 16-byte aligned");

  const hipStream_t s = as_stream(stream);
  const int G = swiglu ? 2 : 1;
  size_t up_b, up3_b = 0, dn_b, sc_b = 0;
  if (w_dtype == MOE_F32) {
    up_b = (size_t)E * m * p * 4;
    up3_b = swiglu ? up_b : 0;
    dn_b = (size_t)E * p * m * 4;
  } else {
    up_b = moe::packed_bytes(E, m, p, G, qb);
    dn_b = moe::packed_bytes(E, p, m, 1, qb);
    if (mx)
      sc_b = align256(moe::packed_mx_scale_bytes(E, m, p, G)) + align256(moe::packed_mx_scale_bytes(E, p, m, 1));
    else if (i8)
      sc_b = align256((size_t)E * p * 4) * (swiglu ? 2 : 1) + align256((size_t)E * m * 4);
  }
  const size_t total = align256(up_b) + align256(up3_b) + align256(dn_b) + sc_b;
  moe_weights* W = new (std::nothrow) moe_weights;
  if (!W) return fail(MOE_ERR_OOM, "host allocation failed");
  W->c.m = m;
  W->c.p = p;
  W->c.E = E;
  W->c.kind = kind;
  W->c.w_dtype = w_dtype;
  W->bytes = total;
  if (hipMalloc(&W->buf, total) != hipSuccess) {
    delete W;
    (void)hipGetLastError();
    return fail(MOE_ERR_OOM, "hipMalloc of %zu bytes for the packed weights failed", total);
  }
  char* base = static_cast<char*>(W->buf);
  size_t off = 0;
  auto carve = [&](size_t b) {
    void* q = b ? base + off : nullptr;
    off += align256(b);
    return q;
  };
  W->up = carve(up_b);
  W->up3 = carve(up3_b);
  W->down = carve(dn_b);
  hipError_t e = hipSuccess;
  if (w_dtype == MOE_F32) {
    e = hipMemcpyAsync(W->up, w1, up_b, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess && swiglu) e = hipMemcpyAsync(W->up3, w_up, up3_b, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess) e = hipMemcpyAsync(W->down, w2, dn_b, hipMemcpyDeviceToDevice, s);
  } else if (mx) {
    W->mx_up = static_cast<uint32_t*>(carve(moe::packed_mx_scale_bytes(E, m, p, G)));
    W->mx_down = static_cast<uint32_t*>(carve(moe::packed_mx_scale_bytes(E, p, m, 1)));
    const uint8_t* const c1 = static_cast<const uint8_t*>(w1);
    e = moe::launch_pack_fp4(c1, W->up, E, m, p, G, 0, s);
    if (e == hipSuccess && swiglu) e = moe::launch_pack_fp4(static_cast<const uint8_t*>(w_up), W->up, E, m, p, G, 1, s);
    if (e == hipSuccess) e = moe::launch_pack_fp4(static_cast<const uint8_t*>(w2), W->down, E, p, m, 1, 0, s);
    if (e == hipSuccess) e = moe::launch_pack_mx_scales(static_cast<const uint8_t*>(s1), W->mx_up, E, m, p, G, 0, s);
    if (e == hipSuccess && swiglu)
      e = moe::launch_pack_mx_scales(static_cast<const uint8_t*>(s_up), W->mx_up, E, m, p, G, 1, s);
    if (e == hipSuccess) e = moe::launch_pack_mx_scales(static_cast<const uint8_t*>(s2), W->mx_down, E, p, m, 1, 0, s);
  } else if (i8) {
    W->s_gate = static_cast<float*>(carve((size_t)E * p * 4));
    if (swiglu) W->s_up = static_cast<float*>(carve((size_t)E * p * 4));
    W->s_down = static_cast<float*>(carve((size_t)E * m * 4));
    auto pack = qb == 4 ? moe::launch_pack_i4 : moe::launch_pack_i8;  // (fp8 codes move as bytes, like int8)
    e = pack(static_cast<const int8_t*>(w1), W->up, E, m, p, G, 0, s);
    if (e == hipSuccess && swiglu) e = pack(static_cast<const int8_t*>(w_up), W->up, E, m, p, G, 1, s);
    if (e == hipSuccess) e = pack(static_cast<const int8_t*>(w2), W->down, E, p, m, 1, 0, s);
    if (e == hipSuccess) e = hipMemcpyAsync(W->s_gate, s1, (size_t)E * p * 4, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess && swiglu) e = hipMemcpyAsync(W->s_up, s_up, (size_t)E * p * 4, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess) e = hipMemcpyAsync(W->s_down, s2, (size_t)E * m * 4, hipMemcpyDeviceToDevice, s);
  } else {
    e = moe::launch_pack_bf16(static_cast<const uint16_t*>(w1), W->up, E, m, p, G, 0, s);
    if (e == hipSuccess && swiglu) e = moe::launch_pack_bf16(static_cast<const uint16_t*>(w_up), W->up, E, m, p, G, 1, s);
    if (e == hipSuccess) e = moe::launch_pack_bf16(static_cast<const uint16_t*>(w2), W->down, E, p, m, 1, 0, s);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    (void)hipFree(W->buf);
    delete W;
    return fail(MOE_ERR_HIP, "packing the weights failed: %s", hipGetErrorString(e));
  }
  *out = W;
  return ok();
}

void free_offload(Offload* O) {
  if (!O) return;
  if (O->copy) (void)hipStreamSynchronize(O->copy);
  for (hipEvent_t e : O->ev_ready) if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : O->ev_done) if (e) (void)hipEventDestroy(e);
  if (O->ev_host) (void)hipEventDestroy(O->ev_host);
  if (O->ev_table) (void)hipEventDestroy(O->ev_table);
  if (O->copy) (void)hipStreamDestroy(O->copy);
  if (O->host) (void)hipHostFree(O->host);
  if (O->h_offs) (void)hipHostFree(O->h_offs);
  if (O->h_table) (void)hipHostFree(O->h_table);
  if (O->dev) (void)hipFree(O->dev);
  if (O->d_table) (void)hipFree(O->d_table);
  delete O;
}

moe_status moe_weights_destroy(moe_weights* w) {
  if (!w) return ok();
  (void)hipDeviceSynchronize();
  free_offload(w->off);
  const hipError_t e = w->buf ? hipFree(w->buf) : hipSuccess;
  delete w;
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipFree failed: %s", hipGetErrorString(e));
  return ok();
}

moe_status moe_weights_offload(moe_weights* w, int slots, void* stream) {
  if (!w) return fail(MOE_ERR_INVALID_ARG, "weights handle is NULL");
  if (w->off) return fail(MOE_ERR_INVALID_ARG, "the experts are already host-resident");
  if (slots < 1 || slots > w->c.E) return fail(MOE_ERR_INVALID_ARG, "slots=%d must be in [1, E=%d]", slots, w->c.E);
  if (w->c.w_dtype == MOE_F32) return fail(MOE_ERR_UNSUPPORTED, "fp32 weights stay device-resident");
  const LayerCfg& c = w->c;
  const int G = c.kind == MOE_SWIGLU ? 2 : 1, qb = weight_bits(c);
  Offload* O = new (std::nothrow) Offload;
  if (!O) return fail(MOE_ERR_OOM, "host allocation failed");
  O->slots = slots;
  O->up_stride = moe::packed_bytes(1, c.m, c.p, G, qb);
  O->dn_stride = moe::packed_bytes(1, c.p, c.m, 1, qb);
  const size_t per = O->up_stride + O->dn_stride;
  const hipStream_t s = as_stream(stream);
  hipError_t e = hipHostMalloc(reinterpret_cast<void**>(&O->host), per * (size_t)c.E, hipHostMallocDefault);
  if (e == hipSuccess) e = hipHostMalloc(reinterpret_cast<void**>(&O->h_offs), (size_t)(c.E + 1) * 4, hipHostMallocDefault);
  if (e == hipSuccess) e = hipHostMalloc(reinterpret_cast<void**>(&O->h_table), (size_t)c.E * 2 * 4, hipHostMallocDefault);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    free_offload(O);
    return fail(MOE_ERR_OOM, "pinned host allocation of %zu bytes failed", per * (size_t)c.E);
  }
  e = hipMalloc(reinterpret_cast<void**>(&O->dev), per * (size_t)slots);
  if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&O->d_table), (size_t)c.E * 2 * 4);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    free_offload(O);
    return fail(MOE_ERR_OOM, "device allocation of %zu bytes for %d expert slots failed", per * (size_t)slots, slots);
  }
  // the packed experts, expert by expert, to the host
  for (int x = 0; x < c.E && e == hipSuccess; ++x) {
    char* h = O->host + (size_t)x * per;
    e = hipMemcpyAsync(h, static_cast<char*>(w->up) + (size_t)x * O->up_stride, O->up_stride, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess)
      e = hipMemcpyAsync(h + O->up_stride, static_cast<char*>(w->down) + (size_t)x * O->dn_stride, O->dn_stride,
                         hipMemcpyDeviceToHost, s);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  // the scales move to an allocation of their own; the packed weights' device copy is freed
  void* sbuf = nullptr;
  char* old_up = static_cast<char*>(w->up);
  const size_t packed_end = (size_t)(static_cast<char*>(w->down) - old_up) + align256((size_t)c.E * O->dn_stride);
  const size_t sc_bytes = w->bytes - packed_end;
  if (e == hipSuccess && sc_bytes > 0) e = hipMalloc(&sbuf, sc_bytes);
  if (e == hipSuccess && sc_bytes > 0) e = hipMemcpyAsync(sbuf, old_up + packed_end, sc_bytes, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  O->slot_expert.assign(slots, -1);
  O->slot_used.assign(slots, 0);
  O->ev_ready.assign(slots, nullptr);
  O->ev_done.assign(slots, nullptr);
  for (int i = 0; i < slots && e == hipSuccess; ++i) {
    e = hipEventCreateWithFlags(&O->ev_ready[i], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&O->ev_done[i], hipEventDisableTiming);
  }
  if (e == hipSuccess) e = hipEventCreateWithFlags(&O->ev_host, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&O->ev_table, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventRecord(O->ev_table, s);  // (so the first forward's wait on it returns)
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&O->copy, hipStreamNonBlocking);  // default priority
  if (e != hipSuccess) {
    (void)hipGetLastError();
    if (sbuf) (void)hipFree(sbuf);
    free_offload(O);
    return fail(MOE_ERR_HIP, "moving the experts to host memory failed: %s", hipGetErrorString(e));
  }
  // rebase the scale pointers into the new allocation, free the old one
  auto rebase = [&](auto* ptr) -> decltype(ptr) {
    if (!ptr) return nullptr;
    return reinterpret_cast<decltype(ptr)>(static_cast<char*>(sbuf) +
                                           (reinterpret_cast<char*>(ptr) - (old_up + packed_end)));
  };
  w->s_gate = rebase(w->s_gate);
  w->s_up = rebase(w->s_up);
  w->s_down = rebase(w->s_down);
  w->mx_up = rebase(w->mx_up);
  w->mx_down = rebase(w->mx_down);
  (void)hipFree(w->buf);
  w->buf = sbuf;
  w->bytes = sc_bytes;
  w->up = w->down = w->up3 = nullptr;
  w->off = O;
  return ok();
}

moe_status moe_weights_offload_stats(const moe_weights* w, long long* hits, long long* misses, long long* bytes) {
  if (!w || !w->off || !hits || !misses || !bytes) return fail(MOE_ERR_INVALID_ARG, "no host-resident experts");
  std::lock_guard<std::mutex> lk(w->off->mu);
  *hits = w->off->hits;
  *misses = w->off->misses;
  *bytes = w->off->bytes;
  return ok();
}

moe_status moe_weights_set_tuning(moe_weights* w, const moe_tuning* t) {
  if (!w) return fail(MOE_ERR_INVALID_ARG, "weights handle is NULL");
  const moe_tuning v = t ? *t : moe_tuning{};
  if (moe_status rc = check_tuning(v)) return rc;
  w->c.tune = v;
  return ok();
}

moe_status moe_weights_get_tuning(const moe_weights* w, moe_tuning* t) {
  if (!w || !t) return fail(MOE_ERR_INVALID_ARG, "NULL argument");
  *t = w->c.tune;
  return ok();
}

moe_status moe_workspace_size(const moe_weights* w, int T, int k, size_t* bytes) {
  if (!w || !bytes) return fail(MOE_ERR_INVALID_ARG, "NULL argument");
  if (moe_status rc = check_shape(T, w->c.m, w->c.p, w->c.E, k)) return rc;
  *bytes = ws_layout(w->c, T, k).total;
  return ok();
}

moe_status moe_workspace_size_for(int m, int p, int E, int kind, int w_dtype, const moe_tuning* t, int T, int k,
                                  size_t* bytes) {
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  if (moe_status rc = check_layer(m, p, E, kind, w_dtype)) return rc;
  if (moe_status rc = check_shape(T, m, p, E, k)) return rc;
  LayerCfg c;
  c.m = m;
  c.p = p;
  c.E = E;
  c.kind = kind;
  c.w_dtype = w_dtype;
  c.tune = t ? *t : moe_tuning{};
  if (moe_status rc = check_tuning(c.tune)) return rc;
  *bytes = ws_layout(c, T, k).total;
  return ok();
}

moe_status moe_route_topk(const void* x, int x_dtype, const float* w_router, const float* b_router, int T, int m,
                          int E, int k, unsigned flags, float* logits, int32_t* topk_idx, float* topk_w,
                          void* stream) {
  if (moe_status rc = check_shape(T, m, 64, E, k)) return rc;
  const bool lin = (flags & MOE_ROUTE_LOGITS_IN) != 0;
  if (flags & ~MOE_ROUTE_LOGITS_IN) return fail(MOE_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if (!lin && x_dtype != MOE_F32 && x_dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "x dtype %d", x_dtype);
  if (T == 0) return ok();
  if (!topk_idx || !topk_w) return fail(MOE_ERR_INVALID_ARG, "topk_idx/topk_w are NULL");
  if (lin && !logits) return fail(MOE_ERR_INVALID_ARG, "MOE_ROUTE_LOGITS_IN needs logits");
  if (!lin && (!x || !w_router)) return fail(MOE_ERR_INVALID_ARG, "x/w_router are NULL");
  if (!lin && (!aligned16(x))) return fail(MOE_ERR_INVALID_ARG, "x must be 16-byte aligned");
  const hipStream_t s = as_stream(stream);
  MOE_TRY_HIP(run("route_topk", s, [&] {
    return moe::launch_route_topk(x, x_dtype == MOE_BF16, w_router, b_router, T, m, E, k, lin, logits, topk_idx,
                                  topk_w, nullptr, 0, s);
  }));
  return ok();
}

moe_status moe_dispatch(const int32_t* topk_idx, int T, int E, int k, int32_t* counts, int32_t* offsets,
                        int32_t* perm, int32_t* inv_perm, void* stream) {
  if (moe_status rc = check_shape(T, 64, 64, E, k)) return rc;
  if (!counts || !offsets) return fail(MOE_ERR_INVALID_ARG, "counts/offsets are NULL");
  if (T > 0 && (!topk_idx || !perm || !inv_perm)) return fail(MOE_ERR_INVALID_ARG, "NULL argument");
  const hipStream_t s = as_stream(stream);
  MOE_TRY_HIP(run("dispatch", s, [&] {
    return moe::launch_dispatch(topk_idx, T * k, E, counts, offsets, perm, inv_perm, s);
  }));
  return ok();
}

moe_status moe_expert_ffn(const moe_weights* w, const void* x, int x_dtype, int T, int m, int p, int E, int k,
                          const int32_t* perm, const int32_t* offsets, float* y_perm, void* workspace,
                          size_t ws_bytes, void* stream) {
  if (moe_status rc = check_weights_match(w, m, p, E)) return rc;
  if (moe_status rc = check_shape(T, m, p, E, k)) return rc;
  if (moe_status rc = check_combo(x_dtype, w->c.w_dtype)) return rc;
  if (T == 0) return ok();
  if (!x || !perm || !offsets || !y_perm) return fail(MOE_ERR_INVALID_ARG, "NULL argument");
  if (!aligned16(x) || !aligned16(y_perm)) return fail(MOE_ERR_INVALID_ARG, "x/y_perm must be 16-byte aligned");
  const Ws L = ws_layout(w->c, T, k);
  if (moe_status rc = check_workspace(L, workspace, ws_bytes)) return rc;
  char* ws = static_cast<char*>(workspace);
  FfnIo io{};
  io.x = x;
  io.T = T;
  io.k = k;
  io.perm = const_cast<int32_t*>(perm);
  io.offsets = const_cast<int32_t*>(offsets);
  io.h = ws + L.h;
  io.xp = ws + L.xp;
  io.down_out = y_perm;
  io.combine = false;
  io.wdq = ws + L.wdq;
  if (moe_status rc = quant_input(w->c, io, ws, L, as_stream(stream))) return rc;
  if (moe_status rc = w->off ? run_ffn_streamed(w, io, as_stream(stream)) : run_ffn(w, io, as_stream(stream)))
    return rc;
  return ok();
}

moe_status moe_combine(const float* y_perm, const int32_t* inv_perm, const float* topk_w, int T, int m, int k,
                       void* y, int y_dtype, void* stream) {
  if (T < 0 || m <= 0 || k < 1) return fail(MOE_ERR_INVALID_ARG, "bad sizes T=%d m=%d k=%d", T, m, k);
  if (m % 64) return fail(MOE_ERR_UNSUPPORTED, "m=%d must be a multiple of 64", m);
  if (y_dtype != MOE_F32 && y_dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "y dtype %d", y_dtype);
  if (k > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "k=%d too large", k);
  if (T == 0) return ok();
  if (!y_perm || !inv_perm || !topk_w || !y) return fail(MOE_ERR_INVALID_ARG, "NULL argument");
  if (!aligned16(y_perm) || !aligned16(y)) return fail(MOE_ERR_INVALID_ARG, "y_perm/y must be 16-byte aligned");
  const hipStream_t s = as_stream(stream);
  MOE_TRY_HIP(run("combine", s, [&] {
    return moe::launch_combine(y_perm, inv_perm, topk_w, T, m, k, 1, 0, y, y_dtype == MOE_BF16, s);
  }));
  return ok();
}

// (shared by the two quantisation entry points)
static moe_status quantize_rows(const void* x, int T, int m, bool int8, void* xq, float* scale, void* stream) {
  if (T < 0 || m <= 0) return fail(MOE_ERR_INVALID_ARG, "bad sizes T=%d m=%d", T, m);
  if (m % 64) return fail(MOE_ERR_UNSUPPORTED, "m=%d must be a multiple of 64", m);
  if (T == 0) return ok();
  if (!x || !xq || !scale) return fail(MOE_ERR_INVALID_ARG, "NULL argument");
  if (!aligned16(x) || !aligned16(xq)) return fail(MOE_ERR_INVALID_ARG, "x/xq must be 16-byte aligned");
  const hipStream_t s = as_stream(stream);
  MOE_TRY_HIP(run("quant_rows", s, [&] {
    return moe::launch_quant_rows(static_cast<const uint16_t*>(x), T, m, int8, static_cast<uint16_t*>(xq), nullptr,
                                  scale, s);
  }));
  return ok();
}

moe_status moe_quantize_rows_e4m3(const void* x, int T, int m, void* xq, float* scale, void* stream) {
  return quantize_rows(x, T, m, false, xq, scale, stream);
}

moe_status moe_quantize_rows_i8(const void* x, int T, int m, void* xq, float* scale, void* stream) {
  return quantize_rows(x, T, m, true, xq, scale, stream);
}

}  // extern "C"

namespace {

// The neighbouring ops of the fused forward (none by default).
struct Fusion {
  int norm = MOE_NORM_NONE;
  const float* gamma = nullptr;
  const float* beta = nullptr;
  float eps = 0.0f;
  const void* residual = nullptr;
  void* x_norm = nullptr;
};

// Arguments of one layer forward after validation of everything but the
// workspace.
moe_status check_forward(const moe_weights* w, const float* w_router, const void* x, int x_dtype, int T, int m, int p,
                         int E, int k, const void* y, int y_dtype) {
  if (moe_status rc = check_weights_match(w, m, p, E)) return rc;
  if (moe_status rc = check_shape(T, m, p, E, k)) return rc;
  if (moe_status rc = check_combo(x_dtype, w->c.w_dtype)) return rc;
  if (y_dtype != MOE_F32 && y_dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "y dtype %d", y_dtype);
  if (T == 0) return MOE_OK;
  if (!w_router || !x || !y) return fail(MOE_ERR_INVALID_ARG, "NULL argument");
  if (!aligned16(x) || !aligned16(y)) return fail(MOE_ERR_INVALID_ARG, "x/y must be 16-byte aligned");
  return MOE_OK;
}

// The launches of one layer forward into a checked workspace `ws` laid out
// as L.  T > 0.
moe_status enqueue_forward(const moe_weights* w, const float* w_router, const float* b_router, const void* x,
                           int x_dtype, int T, int k, void* y, int y_dtype, char* ws, const Ws& L,
                           int32_t* dbg_topk_idx, float* dbg_topk_w, float* dbg_logits, int32_t* dbg_counts,
                           int32_t* dbg_offsets, int32_t* dbg_perm, hipStream_t s, const Fusion& f) {
  const LayerCfg& c = w->c;
  const int m = c.m, E = c.E;
  float* logits = dbg_logits ? dbg_logits : reinterpret_cast<float*>(ws + L.logits);
  int32_t* idx = dbg_topk_idx ? dbg_topk_idx : reinterpret_cast<int32_t*>(ws + L.idx);
  float* tw = dbg_topk_w ? dbg_topk_w : reinterpret_cast<float*>(ws + L.w);
  int32_t* counts = dbg_counts ? dbg_counts : reinterpret_cast<int32_t*>(ws + L.counts);
  int32_t* offsets = dbg_offsets ? dbg_offsets : reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* perm = dbg_perm ? dbg_perm : reinterpret_cast<int32_t*>(ws + L.perm);
  int32_t* inv = reinterpret_cast<int32_t*>(ws + L.inv);
  const bool y_bf16 = y_dtype == MOE_BF16;
  float* yacc = y_bf16 ? reinterpret_cast<float*>(ws + L.yacc) : static_cast<float*>(y);
  const size_t ny = (size_t)T * m;
  const Path path = ffn_path(c, T, k);
  const bool gemm = path == Path::GEMM;
  // at decode sizes the dispatch is derived by the first FFN kernel: the up
  // projection's prologue, or the row packing before it
  const bool fused = !w->off && path == Path::SKINNY && (long long)T * k <= moe::kFusedDispatchMax;
  // unweighted expert rows and the combine kernel (the grouped GEMM, and the
  // skinny kernels unless tuned otherwise), or weighted rows added into y_acc
  // (zeroed by the router) and a final conversion
  const bool rows = gemm || (path == Path::SKINNY && skinny_rows_combine(c));

  // the neighbouring ops: the input rows' norm in the routing pass (the
  // experts then read the normalised rows), the residual added by the combine
  // or, on the accumulator paths, used as the accumulator's starting value
  void* xn = f.norm ? (f.x_norm ? f.x_norm : static_cast<void*>(ws + L.xn)) : nullptr;
  moe::RouteFuse rf{f.norm, f.gamma, f.beta, f.eps, xn, f.residual, y_bf16 ? 1 : 0, 0, nullptr, nullptr, nullptr};
  // 8-bit activations: the routing pass quantises the experts' input rows
  // (from its LDS copy of them), unless tuned off
  const bool q_in_route = act8(c) && tuned_on(c.tune.route_quant, true);
  if (q_in_route) {
    FfnIo shape{};
    shape.T = T;
    shape.k = k;
    const QuantOut q = quant_out(c, shape, ws, L);
    rf.quant = act_int8(c) ? 2 : 1;
    rf.xq = q.xq;
    rf.xc = q.xc;
    rf.xs = q.xs;
  }
  MOE_TRY_HIP(run("route_topk", s, [&] {
    return moe::launch_route_topk(x, x_dtype == MOE_BF16, w_router, b_router, T, m, E, k, false, logits, idx, tw,
                                  rows ? nullptr : yacc, m, s, &rf);
  }));
  if (!fused)
    MOE_TRY_HIP(run("dispatch", s, [&] { return moe::launch_dispatch(idx, T * k, E, counts, offsets, perm, inv, s); }));
  FfnIo io{};
  io.x = f.norm ? xn : x;
  io.T = T;
  io.k = k;
  io.topk_idx = fused ? idx : nullptr;
  io.counts = counts;
  io.offsets = offsets;
  io.perm = perm;
  io.inv = inv;
  io.topk_w = tw;
  io.h = ws + L.h;
  io.xp = ws + L.xp;
  io.down_out = yacc;
  io.combine = true;
  io.yperm = rows ? reinterpret_cast<float*>(ws + L.yperm) : nullptr;
  io.wdq = ws + L.wdq;
  int slices = 1;
  io.slices = &slices;
  if (moe_status rc = quant_input(c, io, ws, L, s, q_in_route)) return rc;
  if (moe_status rc = w->off ? run_ffn_streamed(w, io, s) : run_ffn(w, io, s)) return rc;
  if (rows) {
    MOE_TRY_HIP(run("combine", s, [&] {
      return moe::launch_combine(io.yperm, inv, tw, T, m, k, slices, (size_t)T * k * m, y, y_bf16, s, f.residual);
    }));
    return MOE_OK;
  }
  if (y_bf16)
    MOE_TRY_HIP(run("finalize", s, [&] { return moe::launch_f32_to_bf16(yacc, static_cast<uint16_t*>(y), ny, s); }));
  return MOE_OK;
}

moe_status layer_forward(const moe_weights* w, const float* w_router, const float* b_router, const void* x,
                         int x_dtype, int T, int m, int p, int E, int k, void* y, int y_dtype, void* workspace,
                         size_t ws_bytes, int32_t* dbg_topk_idx, float* dbg_topk_w, float* dbg_logits,
                         int32_t* dbg_counts, int32_t* dbg_offsets, int32_t* dbg_perm, void* stream,
                         const Fusion& f) {
  if (moe_status rc = check_forward(w, w_router, x, x_dtype, T, m, p, E, k, y, y_dtype)) return rc;
  if (T == 0) return ok();
  const Ws L = ws_layout(w->c, T, k);
  if (moe_status rc = check_workspace(L, workspace, ws_bytes)) return rc;
  if (moe_status rc = enqueue_forward(w, w_router, b_router, x, x_dtype, T, k, y, y_dtype,
                                      static_cast<char*>(workspace), L, dbg_topk_idx, dbg_topk_w, dbg_logits,
                                      dbg_counts, dbg_offsets, dbg_perm, as_stream(stream), f))
    return rc;
  return ok();
}

}  // namespace

extern "C" {

moe_status moe_layer_forward(const moe_weights* w, const float* w_router, const float* b_router, const void* x,
                             int x_dtype, int T, int m, int p, int E, int k, void* y, int y_dtype, void* workspace,
                             size_t ws_bytes, int32_t* dbg_topk_idx, float* dbg_topk_w, float* dbg_logits,
                             int32_t* dbg_counts, int32_t* dbg_offsets, int32_t* dbg_perm, void* stream) {
  return layer_forward(w, w_router, b_router, x, x_dtype, T, m, p, E, k, y, y_dtype, workspace, ws_bytes,
                       dbg_topk_idx, dbg_topk_w, dbg_logits, dbg_counts, dbg_offsets, dbg_perm, stream, Fusion{});
}

moe_status moe_layer_forward_fused(const moe_weights* w, const float* w_router, const float* b_router, const void* x,
                                   int x_dtype, int norm, const float* gamma, const float* beta, float eps,
                                   const void* residual, int T, int m, int p, int E, int k, void* y, int y_dtype,
                                   void* workspace, size_t ws_bytes, void* x_norm, int32_t* dbg_topk_idx,
                                   float* dbg_topk_w, float* dbg_logits, void* stream) {
  if (norm != MOE_NORM_NONE && norm != MOE_NORM_LAYER && norm != MOE_NORM_RMS)
    return fail(MOE_ERR_INVALID_ARG, "norm kind %d", norm);
  if (norm == MOE_NORM_NONE && (gamma || beta || x_norm))
    return fail(MOE_ERR_INVALID_ARG, "gamma, beta and x_norm need a norm");
  if (norm == MOE_NORM_RMS && beta) return fail(MOE_ERR_INVALID_ARG, "the RMS norm takes no beta");
  if (!(eps >= 0.0f) || eps > 1.0f) return fail(MOE_ERR_INVALID_ARG, "eps=%g must be in [0, 1]", (double)eps);
  if (T > 0 && norm != MOE_NORM_NONE && !gamma) return fail(MOE_ERR_INVALID_ARG, "gamma is NULL");
  if (residual && !aligned16(residual)) return fail(MOE_ERR_INVALID_ARG, "residual must be 16-byte aligned");
  if (x_norm && !aligned16(x_norm)) return fail(MOE_ERR_INVALID_ARG, "x_norm must be 16-byte aligned");
  if ((gamma && !aligned16(gamma)) || (beta && !aligned16(beta)))
    return fail(MOE_ERR_INVALID_ARG, "gamma/beta must be 16-byte aligned");
  Fusion f;
  f.norm = norm;
  f.gamma = gamma;
  f.beta = beta;
  f.eps = eps;
  f.residual = residual;
  f.x_norm = x_norm;
  return layer_forward(w, w_router, b_router, x, x_dtype, T, m, p, E, k, y, y_dtype, workspace, ws_bytes,
                       dbg_topk_idx, dbg_topk_w, dbg_logits, nullptr, nullptr, nullptr, stream, f);
}

}  // extern "C"

// ---- the allocation-free forward ----------------------------------------------
//
// Callers that cannot allocate device memory (code under graph capture, tight
// serving loops, harnesses that forbid it) get a forward whose workspace is
// this file-scope device array: each GPU the library runs on holds its own
// copy until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device memory; the device address comes from
// hipGetSymbolAddress, once per device with that device current, and only
// that address is passed to kernels.
namespace {

constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;  // device -> address of its scratch

// The current device's scratch address, looked up on its first use.
moe_status scratch_address(void** out) {
  int dev = 0;
  MOE_TRY_HIP(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it != g_scratch_ptr.end()) {
    *out = it->second;
    return MOE_OK;
  }
  void* ptr = nullptr;
  MOE_TRY_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
  if (!ptr || (reinterpret_cast<uintptr_t>(ptr) & 255u))
    return fail(MOE_ERR_HIP, "scratch array of device %d has no usable address", dev);
  g_scratch_ptr[dev] = ptr;
  *out = ptr;
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_layer_forward_noalloc(const moe_weights* w, const float* w_router, const float* b_router,
                                     const void* x, int x_dtype, int T, int m, int p, int E, int k, void* y,
                                     int y_dtype, void* stream) {
  if (moe_status rc = check_forward(w, w_router, x, x_dtype, T, m, p, E, k, y, y_dtype)) return rc;
  if (w->off) return fail(MOE_ERR_UNSUPPORTED, "host-resident experts need moe_layer_forward");
  if (T == 0) return ok();
  const Ws L = ws_layout(w->c, T, k);
  if (L.total > kScratchBytes)
    return fail(MOE_ERR_UNSUPPORTED, "T=%d needs %zu bytes of workspace, above the %zu-byte scratch of the "
                "allocation-free forward (use moe_layer_forward with a workspace)", T, L.total, kScratchBytes);
  void* ws = nullptr;
  if (moe_status rc = scratch_address(&ws)) return rc;
  // Every kernel writes each workspace region before reading it (the routing
  // pass zeroes the accumulator where one is used), so no region needs
  // clearing from the host.
  if (moe_status rc = enqueue_forward(w, w_router, b_router, x, x_dtype, T, k, y, y_dtype, static_cast<char*>(ws), L,
                                      nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, as_stream(stream),
                                      Fusion{}))
    return rc;
  return ok();
}

}  // extern "C"

struct moe_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;  // null for a forward with no launches (T = 0)
};

extern "C" {

moe_status moe_layer_graph_create(const moe_weights* w, const float* w_router, const float* b_router, const void* x,
                                  int x_dtype, int T, int m, int p, int E, int k, void* y, int y_dtype,
                                  void* workspace, size_t ws_bytes, moe_graph** out) {
  if (!out) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    if (g_prof.on) return fail(MOE_ERR_INVALID_ARG, "cannot capture while moe_profile_begin is active");
  }
  if (w && w->off) return fail(MOE_ERR_UNSUPPORTED, "a forward over host-resident experts synchronises the host and "
                                                    "cannot be captured");
  hipStream_t cs = nullptr;
  MOE_TRY_HIP(hipStreamCreateWithFlags(&cs, hipStreamNonBlocking));
  hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    (void)hipStreamDestroy(cs);
    return fail(MOE_ERR_HIP, "hipStreamBeginCapture: %s", hipGetErrorString(e));
  }
  const moe_status rc = moe_layer_forward(w, w_router, b_router, x, x_dtype, T, m, p, E, k, y, y_dtype, workspace,
                                          ws_bytes, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, cs);
  const std::string err = rc ? g_err : std::string();
  hipGraph_t graph = nullptr;
  e = hipStreamEndCapture(cs, &graph);  // ends the capture even after a failed forward
  (void)hipStreamDestroy(cs);
  if (rc) {
    if (graph) (void)hipGraphDestroy(graph);
    g_err = err;
    return rc;
  }
  if (e != hipSuccess || !graph) return fail(MOE_ERR_HIP, "hipStreamEndCapture: %s", hipGetErrorString(e));
  size_t nodes = 0;
  e = hipGraphGetNodes(graph, nullptr, &nodes);
  hipGraphExec_t exec = nullptr;
  if (e == hipSuccess && nodes > 0) e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(graph);
    return fail(MOE_ERR_HIP, "graph instantiation: %s", hipGetErrorString(e));
  }
  moe_graph* g = new (std::nothrow) moe_graph{graph, exec};
  if (!g) {
    if (exec) (void)hipGraphExecDestroy(exec);
    (void)hipGraphDestroy(graph);
    return fail(MOE_ERR_OOM, "graph handle allocation failed");
  }
  *out = g;
  return ok();
}

moe_status moe_graph_launch(const moe_graph* g, void* stream) {
  if (!g) return fail(MOE_ERR_INVALID_ARG, "graph is NULL");
  if (!g->exec) return ok();
  MOE_TRY_HIP(hipGraphLaunch(g->exec, as_stream(stream)));
  return ok();
}

moe_status moe_graph_destroy(moe_graph* g) {
  if (!g) return ok();
  hipError_t e = hipSuccess;
  if (g->exec) e = hipGraphExecDestroy(g->exec);
  const hipError_t e2 = hipGraphDestroy(g->graph);
  delete g;
  if (e != hipSuccess || e2 != hipSuccess)
    return fail(MOE_ERR_HIP, "graph destruction: %s", hipGetErrorString(e != hipSuccess ? e : e2));
  return ok();
}

moe_status moe_profile_begin(int max_launches) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (max_launches < 1 || max_launches > (1 << 20)) return fail(MOE_ERR_INVALID_ARG, "max_launches out of range");
  for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
  g_prof.ev.assign(2 * (size_t)max_launches, nullptr);
  for (auto& e : g_prof.ev) MOE_TRY_HIP(hipEventCreate(&e));
  g_prof.name.assign(max_launches, nullptr);
  g_prof.total.clear();
  g_prof.max = max_launches;
  g_prof.n = 0;
  g_prof.on = true;
  return ok();
}

moe_status moe_profile_end(void) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (!g_prof.on) return fail(MOE_ERR_INVALID_ARG, "profiling was not started");
  g_prof.on = false;
  for (int i = 0; i < g_prof.n; ++i) {
    MOE_TRY_HIP(hipEventSynchronize(g_prof.ev[2 * i + 1]));
    float ms = 0.0f;
    MOE_TRY_HIP(hipEventElapsedTime(&ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]));
    auto& t = g_prof.total[g_prof.name[i]];
    t.first += ms;
    t.second += 1;
  }
  for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
  g_prof.ev.clear();
  g_prof.n = 0;
  return ok();
}

moe_status moe_profile_query(const char* kernel, double* total_ms, int* launches) {
  if (!kernel || !total_ms || !launches) return fail(MOE_ERR_INVALID_ARG, "NULL argument");
  std::lock_guard<std::mutex> lk(g_prof.mu);
  auto it = g_prof.total.find(kernel);
  *total_ms = it == g_prof.total.end() ? 0.0 : it->second.first;
  *launches = it == g_prof.total.end() ? 0 : it->second.second;
  return ok();
}

}  // extern "C"
