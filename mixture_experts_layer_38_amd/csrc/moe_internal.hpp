// Internal declarations shared by the kernel translation units and the C ABI.
// Device helpers here are written for gfx950 (CDNA4): 64-lane wavefronts,
// MFMA builtins, raw 16-bit bf16 storage.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kWave = 64;
constexpr int kMaxExperts = 512;
constexpr int kMaxTopK = 16;
constexpr int kMaxGroups = 64;

// Tile geometry of the grouped bf16 MFMA GEMMs (prefill path).
constexpr int kGB_BM = 256;   // rows (tokens) per tile
constexpr int kG1_BNH = 128;  // hidden columns per gate/up tile (128 gate + 128 up rows of W)
constexpr int kG2_BN = 256;   // output columns per down tile
constexpr int kGB_BK = 64;    // K step
// Grouped GEMMs on e4m3 activations and weights (fp8 matrix cores).
constexpr int kF8_BM1 = 128;  // rows (tokens) per gate/up tile
constexpr int kF8_BM2 = 256;  // rows (h rows) per down tile
constexpr int kF8_BK = 128;   // K step = one scale block (elements = bytes)
constexpr int kActBlock = 128;  // activation quantisation block (1 x 128)
constexpr int kDispatchChunk = 128;  // (token, slot) entries per wave in the stable permutation
// fp32 layers: rows per work item of the grouped fp32 GEMMs (gate/up items
// cover 32 hidden units, down items 64 output columns)
constexpr int kF32_BM = 64;
// Weight-streaming path (small token counts): token rows and columns per workgroup item.
constexpr int kST_BM = 16;
constexpr int kST_N1 = 32;    // hidden columns per gate/up item (32 gate + 32 up rows)
constexpr int kST_N2 = 64;    // output columns per down item
constexpr int kST_KC = 128;   // K chunk (one fp8 scale block)

// ---------------------------------------------------------------------------
// scalar helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// round-to-nearest-even float32 -> bfloat16 (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// SiLU(z) = z / (1 + 2^(-z*log2(e))), on the hardware exp2 and reciprocal.
__device__ __forceinline__ float silu_fast(float z) {
  float e = __builtin_amdgcn_exp2f(-z * 1.4426950408889634f);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// float32 -> OCP e4m3 code (1 sign, 4 exponent bits with bias 7, 3 mantissa
// bits; largest finite 448), rounded to nearest even; magnitudes past 448
// saturate to 448; the sign bit is the float32 sign bit. Normal range: round
// the float32 significand to 3 bits at bit 20 and rebias the exponent; below
// 2^-6 the codes are the multiples of 2^-9, rounded by v_rndne_f32.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x3C800000u) {  // |v| >= 2^-6
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    code = (r >> 20) - (120u << 3);
    code = code > 0x7Eu ? 0x7Eu : code;
  } else {
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  }
  return ((u >> 24) & 0x80u) | code;
}

// scale of one 1 x 128 activation block: largest magnitude / 448 (IEEE
// division), 1 for an all-zero block
__device__ __forceinline__ float e4m3_block_scale(float amax) { return amax > 0.f ? amax / 448.0f : 1.0f; }

__device__ __forceinline__ uint32_t ordered_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave reductions without LDS traffic: four DPP steps (quad permutes 1,0,3,2
// and 2,3,0,1, half-row mirror, row mirror) make every 16-lane row uniform,
// then the four row values are read into scalar registers and combined in a
// fixed order; every lane gets the result.
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t lane_u32(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

template <int kCtrl>
__device__ __forceinline__ uint64_t dpp_max_u64(uint64_t v) {
  const uint64_t w = ((uint64_t)dpp_u32<kCtrl>((uint32_t)(v >> 32)) << 32) | dpp_u32<kCtrl>((uint32_t)v);
  return w > v ? w : v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_u64<0xB1>(v);
  v = dpp_max_u64<0x4E>(v);
  v = dpp_max_u64<0x141>(v);
  v = dpp_max_u64<0x140>(v);
  uint64_t r = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint64_t w = ((uint64_t)lane_u32((uint32_t)(v >> 32), 16 * q) << 32) | lane_u32((uint32_t)v, 16 * q);
    r = w > r ? w : r;
  }
  return r;
}

__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, __uint_as_float(dpp_u32<0xB1>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<0x4E>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<0x141>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<0x140>(__float_as_uint(v))));
  const float a = __uint_as_float(lane_u32(__float_as_uint(v), 0)), b = __uint_as_float(lane_u32(__float_as_uint(v), 16));
  const float c = __uint_as_float(lane_u32(__float_as_uint(v), 32)), d = __uint_as_float(lane_u32(__float_as_uint(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

__device__ __forceinline__ float wave_sum_f32(float v) {
  v += __uint_as_float(dpp_u32<0xB1>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x4E>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x141>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x140>(__float_as_uint(v)));
  const float a = __uint_as_float(lane_u32(__float_as_uint(v), 0)), b = __uint_as_float(lane_u32(__float_as_uint(v), 16));
  const float c = __uint_as_float(lane_u32(__float_as_uint(v), 32)), d = __uint_as_float(lane_u32(__float_as_uint(v), 48));
  return (a + b) + (c + d);
}

// Bounds checks of the debug build (compiled with MOE_DEBUG): an index read
// from memory that lies outside [0, n) is recorded -- the first violation's
// site code and value, in a word of device memory that moe_debug_status reads
// and clears -- and replaced by 0, so the access that follows stays inside
// its buffer. Device code is not linked across translation units, so each
// unit holds its own word and its own reader. Release builds compile the
// checks away.
#ifdef MOE_DEBUG
static __device__ unsigned long long moe_debug_word;
__device__ __forceinline__ int dcheck(int v, int n, int site) {
  if ((unsigned)v >= (unsigned)n) {
    atomicCAS(&moe_debug_word, 0ull, ((unsigned long long)(unsigned)site << 32) | (unsigned)v);
    return 0;
  }
  return v;
}
#define MOE_DEBUG_READER(name)                                                              \
  hipError_t name(unsigned long long* w) {                                                  \
    hipError_t e = hipMemcpyFromSymbol(w, HIP_SYMBOL(moe_debug_word), sizeof(*w), 0,        \
                                       hipMemcpyDeviceToHost);                              \
    if (e != hipSuccess) return e;                                                          \
    const unsigned long long z = 0;                                                         \
    return hipMemcpyToSymbol(HIP_SYMBOL(moe_debug_word), &z, sizeof(z), 0, hipMemcpyHostToDevice); \
  }
#else
__device__ __forceinline__ int dcheck(int v, int, int) { return v; }
#define MOE_DEBUG_READER(name)
#endif
// debug check sites (the code moe_debug_status reports)
enum DebugSite {
  kSiteGroupedTok = 1,     // gathered token row of a grouped GEMM tile
  kSiteGroupedRows = 2,    // a tile's first row inside its problem
  kSiteF8Tok = 3,          // gathered token row, e4m3-activation GEMM
  kSiteStreamTok = 4,      // gathered token row, streaming GEMM
  kSiteF32Tok = 5,         // gathered token row, fp32 GEMM
  kSiteCombineRow = 6,     // slot -> row of the combine
  kSiteBwdExpert = 7,      // expert index read by the router backward
  kSiteBwdRow = 8,         // slot -> row in the backward
  kSiteDispatchRow = 9,    // row a dispatch entry is placed at
};

// problem p in [0, E]: routed expert p (< E) or the shared expert (== E).
// Largest p with pre[p] <= i, for a non-decreasing pre[0..E+1].
__device__ __forceinline__ int find_problem(const int32_t* pre, int E, int i) {
  int lo = 0, hi = E;  // answer in [0, E]
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= i) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------------------
// kernel launchers (one translation unit each)
// ---------------------------------------------------------------------------

struct RouterArgs {
  const void* x;
  const float* gate_w;
  const float* bias;
  float* logits;
  int32_t* idx;
  float* gate;
  int32_t* counts;
  int T, D, E, G, kg, K;
  int act_bf16;
  int score_fn;
  int norm;
  float rsf;
  int num_cus;
  int splits;           // set by launch_router
  size_t logit_rows;    // rows of E floats the partial-logit planes may use (splits * T of them)
  uint16_t* w_split;    // [3][E][D] bf16 planes of gate_w (bf16 activations), or null
  int hist;             // 1: also count the selections into counts (else the dispatch does)
  float* score_sum;     // [E] column sums of the scores over the T tokens, or null
  float* score_part;    // [score_part_rows(T)][E] partial sums (when score_sum is set)
};
// rows of partial score sums launch_router needs for T tokens
int score_part_rows(int T);
// from this many tokens on, bf16 activations take the bf16x3 logits kernel
constexpr int kRouterX3MinTokens = 512;
// Up to this many (token, slot) entries the dispatch runs in one workgroup
// and derives the expert counts itself (the router's histogram is skipped).
constexpr int kSmallDispatch = 1024;
inline bool small_dispatch(int n) { return n > 0 && n <= kSmallDispatch; }
// number of partial-logit planes launch_router uses for T tokens
int router_splits(int T, int D, int E, int num_cus);
hipError_t launch_router(const RouterArgs& a, hipStream_t s);

struct DispatchArgs {
  const int32_t* idx;     // [T*K]
  const float* gate;      // [T*K] or null
  int32_t* counts;        // [E] (input: histogram)
  int32_t* counts_out;    // [E] user copy or null
  int32_t* offsets;       // [E+1]
  int32_t* chunk_base;    // [E][ceil(T*K/128)] first row of each chunk's entries of each expert
  int32_t* row_token;     // [T*K]
  float* row_gate;        // [T*K] or null
  int32_t* slot_row;      // [T*K]
  int32_t* pre1;          // [E+2] item prefix, gate/up GEMM
  int32_t* pre2;          // [E+2] item prefix, down GEMM
  int T, K, E;
  int shared_rows;        // rows of the shared problem (T, or 0 without shared expert)
  int bm1, bm2;           // rows per item, gate/up and down GEMMs
  int n1_routed, n1_shared;  // column items per row block, gate/up GEMM
  int n2_routed, n2_shared;  // column items per row block, down GEMM
};
hipError_t launch_histogram(const int32_t* idx, int32_t* counts, int n, int E, hipStream_t s);
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s);

struct ExpertGemmArgs {
  // geometry
  const int32_t* offsets;   // [E+1]
  const int32_t* row_token; // [T*K]
  const float* row_gate;    // [T*K]
  const int32_t* pre;       // [E+2] item prefix of this GEMM
  int E, T, D, H, Hs;
  int x_rows;               // rows of x (tokens of the call)
  int max_items;            // grid upper bound (items)
  // operands
  const void* a;            // GEMM1: x [T][D]; GEMM2: h routed [T*K][H]
  const void* a_shared;     // GEMM2: h shared [T][Hs]
  const void* w;            // routed weights (gate_up or down)
  const void* w_shared;
  const float* w_scale;     // fp8 only
  const float* w_shared_scale;
  void* c;                  // GEMM1: h routed; GEMM2: y routed
  void* c_shared;           // GEMM1: h shared; GEMM2: y shared
  // e4m3 activations only: 1x128 block scales of the A rows and of h
  const float* a_scale;         // GEMM1: x scales [x_rows][D/128]; GEMM2: h routed scales [T*K][H/128]
  const float* a_shared_scale;  // GEMM2: h shared scales [T][Hs/128]
  float* c_scale;               // GEMM1: h routed scales
  float* c_shared_scale;        // GEMM1: h shared scales
  // backward recompute (gate/up mode 2): c, c_shared receive [a | u] rows,
  // c2, c2_shared receive g * h rows; training forward (mode 3): c, c_shared
  // receive h, c2, c2_shared [a | u] and c3, c3_shared g * h
  void* c2;
  void* c2_shared;
  void* c3;
  void* c3_shared;
};
// grouped (prefill) GEMMs; fp8: e4m3 weights with 128x128 block scales
hipError_t launch_grouped_gateup(const ExpertGemmArgs& a, int fp8, hipStream_t s);
hipError_t launch_grouped_down(const ExpertGemmArgs& a, int fp8, hipStream_t s);
// gate/up GEMM that writes the pre-activations [a | u] and g * h (bf16) for the backward pass
hipError_t launch_grouped_recompute(const ExpertGemmArgs& a, hipStream_t s);
// the gate/up GEMM of a training forward (bf16): h, [a | u] and g * h
hipError_t launch_grouped_gateup_train(const ExpertGemmArgs& a, hipStream_t s);
// grouped GEMMs on e4m3 activations (1x128 block scales) and e4m3 weights
// (128x128 block scales), fp8 MFMA; the gate/up GEMM writes h as e4m3 + scales
hipError_t launch_grouped_gateup_f8(const ExpertGemmArgs& a, hipStream_t s);
hipError_t launch_grouped_down_f8(const ExpertGemmArgs& a, hipStream_t s);
// x bf16 [rows][cols] -> e4m3 codes [rows][cols] + scales [rows][cols/128]
hipError_t launch_quant_e4m3(const uint16_t* x, int rows, int cols, uint8_t* q, float* scale, hipStream_t s);
hipError_t launch_stream_gateup(const ExpertGemmArgs& a, int fp8, int max_items, int num_cus, hipStream_t s);
hipError_t launch_stream_down(const ExpertGemmArgs& a, int fp8, int max_items, int num_cus, hipStream_t s);
hipError_t launch_simple_gateup_f32(const ExpertGemmArgs& a, int TK, hipStream_t s);
hipError_t launch_simple_down_f32(const ExpertGemmArgs& a, int TK, hipStream_t s);

struct CombineArgs {
  const void* x;            // residual source, act dtype
  const void* y_routed;     // [T*K][D]
  const void* y_shared;     // [T][D] or null
  const int32_t* slot_row;  // [T*K]
  void* out;
  int T, D, K;
  int act_bf16, y_bf16, out_bf16;
  int add_residual;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);

// backward pass (after the router, the dispatch and the gate/up recompute)
struct BwdArgs {
  int E, T, D, H, Hs, K;
  int Ep;          // E rounded up to a multiple of 64 (dlogit rows, gate_w rows)
  int splits;      // K splits of the d gate_w product
  int score_fn, norm;
  float rsf;
  int add_residual;
  // routing and dispatch of the forward
  const int32_t* offsets;   // [E+1]
  const int32_t* row_token; // [T*K]
  const float* row_gate;    // [T*K]
  const int32_t* slot_row;  // [T*K]
  const int32_t* idx;       // [T*K]
  const float* logits;      // [T][E]
  const int32_t* pre;       // set per launch
  int32_t* pre_h;           // [E+2] tile prefix of the dH product
  int32_t* pre_x;           // [E+2] tile prefix of the dX product
  // inputs
  const uint16_t* x;        // [T][D] bf16
  const float* dout_f32;    // [T][D]
  const float* gate_w;      // [E][D] fp32
  const uint16_t* w_gu;     // [E][2H][D]
  const uint16_t* w_down;   // [E][D][H]
  const uint16_t* w_gu_shared;
  const uint16_t* w_down_shared;
  // workspace
  uint16_t* dout;           // [T][D] bf16 copy of d_out
  uint16_t* gw_bf16;        // [Ep][D]
  const uint16_t* au;       // [T*K][2H] recomputed [a | u]
  const uint16_t* au_shared;
  const uint16_t* gh;       // [T*K][H] g * h
  const uint16_t* gh_shared;
  uint16_t* dau;            // [T*K][2H] [dA | dU]
  uint16_t* dau_shared;
  float* part;              // [T*K][H/128] partial dL/dg
  float* part_shared;       // [T][Hs/128]
  uint16_t* dxr;            // [T*K][D]
  uint16_t* dxs;            // [T][D]
  uint16_t* dlogit;         // [T][Ep]
  float* dx_router;         // [T][D]
  float* gw_planes;         // [splits][E][D]
  // outputs (fp32)
  float* dx;                // [T][D]
  float* d_gate_w;          // [E][D]
  float* dw_gu;             // [E][2H][D]
  float* dw_down;           // [E][D][H]
  float* dw_gu_shared;      // [2Hs][D]
  float* dw_down_shared;    // [D][Hs]
};
hipError_t launch_layer_backward(const BwdArgs& a, hipStream_t s);

#ifdef MOE_DEBUG
// readers of each translation unit's debug word (value, then cleared)
hipError_t debug_read_dispatch(unsigned long long* w);
hipError_t debug_read_grouped(unsigned long long* w);
hipError_t debug_read_f8(unsigned long long* w);
hipError_t debug_read_stream(unsigned long long* w);
hipError_t debug_read_f32(unsigned long long* w);
hipError_t debug_read_bwd(unsigned long long* w);
#endif

// one workgroup: bias update (bias != null) and/or load statistics (stats != null)
hipError_t launch_balance(const int32_t* counts, int E, float gamma, float* bias, float* stats, hipStream_t s);
// one workgroup: load and importance statistics, expert- and device-level
hipError_t launch_balance_stats(const int32_t* counts, const float* score_sum, int E, int n_devices, float* stats,
                                hipStream_t s);
// dst[0..n) = 0 (a fill kernel, so that the call can sit in a captured graph)
hipError_t launch_zero_f32(float* dst, size_t n, hipStream_t s);

}  // namespace moe
