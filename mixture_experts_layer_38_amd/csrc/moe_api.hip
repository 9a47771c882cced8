// C ABI: parameter validation, workspace, and the launch sequence of the
// layer forward on one stream (router -> dispatch -> gate/up GEMM -> down GEMM
// -> combine). Nothing here waits for the device.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>

#include "moe_internal.hpp"

struct moe_cfg {
  moe_params p;
  int device;
  int num_cus;
  size_t ws_bytes;
  char* ws;
  float* logits;
  uint16_t* w_split;
  int32_t* idx;
  float* gate;
  int32_t* counts;
  int32_t* offsets;
  int32_t* chunk_base;
  int32_t* pre1;
  int32_t* pre2;
  int32_t* row_token;
  float* row_gate;
  int32_t* slot_row;
  void* h_routed;
  void* h_shared;
  void* y_routed;
  void* y_shared;
  // e4m3 activations: x codes and scales, h scales (h codes use h_routed / h_shared)
  uint8_t* xq;
  float* xs;
  float* hs_routed;
  float* hs_shared;
  // backward workspace (g*h uses h_routed / h_shared, the dx rows y_routed / y_shared)
  int Ep, bwd_splits;
  uint16_t* dout_bf;
  uint16_t* gw_bf;
  uint16_t* au;
  uint16_t* au_shared;
  uint16_t* gh;          // g * h rows (routed), read by dW_down
  uint16_t* gh_shared;
  int saved_T;           // tokens of the last training forward whose [a | u], g * h are in au, gh; -1: none
  uint16_t* dau;
  uint16_t* dau_shared;
  float* part;
  float* part_shared;
  uint16_t* dlogit;
  float* dx_router;
  float* gw_planes;
  int32_t* pre_h;
  int32_t* pre_x;
  size_t logit_rows;  // rows of the partial-logit planes region ([logit_rows][E] fp32)
  float* score_part;  // [score_part_rows(max_tokens)][E] partial score column sums
  float* score_sum;   // caller's [E] buffer for the score column sums, or null
  int last_hip_error;
  // stage timing
  bool timing;
  int timed_calls;
  hipEvent_t* events;  // [MOE_TIMING_CALLS][MOE_NUM_STAGES + 1]
};

namespace {

using namespace moe;

moe_status validate(const moe_params* p) {
  if (!p) return MOE_ERR_INVALID_ARG;
  if (p->dim <= 0 || p->n_routed <= 0 || p->hidden <= 0 || p->shared_hidden < 0) return MOE_ERR_INVALID_ARG;
  if (p->n_routed > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (p->top_k <= 0 || p->top_k > kMaxTopK) return MOE_ERR_INVALID_ARG;
  if (p->n_group <= 0 || p->n_group > kMaxGroups || p->n_routed % p->n_group != 0) return MOE_ERR_INVALID_ARG;
  if (p->topk_group <= 0 || p->topk_group > p->n_group) return MOE_ERR_INVALID_ARG;
  if ((long)p->top_k > (long)p->topk_group * (p->n_routed / p->n_group)) return MOE_ERR_INVALID_ARG;
  if (p->score_fn != MOE_SCORE_SOFTMAX && p->score_fn != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (p->act_dtype != MOE_F32 && p->act_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (p->weight_dtype < MOE_F32 || p->weight_dtype > MOE_FP8_E4M3) return MOE_ERR_INVALID_ARG;
  if (p->out_dtype != MOE_F32 && p->out_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (p->max_tokens < 0) return MOE_ERR_INVALID_ARG;
  if (p->path < MOE_PATH_AUTO || p->path > MOE_PATH_STREAM) return MOE_ERR_INVALID_ARG;
  if (p->act_quant != MOE_ACT_QUANT_NONE && p->act_quant != MOE_ACT_QUANT_E4M3_1X128) return MOE_ERR_INVALID_ARG;
  if (p->backward != 0 && p->backward != 1) return MOE_ERR_INVALID_ARG;
  if (!(p->routed_scaling_factor == p->routed_scaling_factor)) return MOE_ERR_INVALID_ARG;  // NaN
  // dtype combinations the library runs
  const bool f32 = p->act_dtype == MOE_F32 && p->weight_dtype == MOE_F32;
  const bool bf = p->act_dtype == MOE_BF16 && p->weight_dtype == MOE_BF16;
  const bool fp8 = p->act_dtype == MOE_BF16 && p->weight_dtype == MOE_FP8_E4M3;
  if (!(f32 || bf || fp8)) return MOE_ERR_UNSUPPORTED;
  // e4m3 activations: fp8 weights, bf16 x, grouped kernels only
  if (p->act_quant == MOE_ACT_QUANT_E4M3_1X128 && (!fp8 || p->path == MOE_PATH_STREAM)) return MOE_ERR_UNSUPPORTED;
  // the backward pass: bf16 activations and weights
  if (p->backward && (!bf || p->act_quant != MOE_ACT_QUANT_NONE)) return MOE_ERR_UNSUPPORTED;
  if (p->dim % 32 != 0) return MOE_ERR_UNSUPPORTED;
  if (!f32 && (p->dim % 128 || p->hidden % 128 || p->shared_hidden % 128)) return MOE_ERR_UNSUPPORTED;
  // the grouped GEMMs address x rows, an expert's h rows and one expert's
  // weights with 32-bit byte offsets
  const uint64_t hmax = (uint64_t)std::max(p->hidden, p->shared_hidden);
  if (!f32 && ((uint64_t)p->max_tokens * p->dim * 2 > 0xFFFFFFFFull ||
               (uint64_t)p->max_tokens * hmax * 2 > 0xFFFFFFFFull ||
               (uint64_t)2 * hmax * p->dim * 2 > 0xFFFFFFFFull))
    return MOE_ERR_UNSUPPORTED;
  // backward: the shared expert's [dA | dU] rows (T x 2*Hs bf16) are addressed the same way
  if (p->backward && (uint64_t)p->max_tokens * 2 * hmax * 2 > 0xFFFFFFFFull) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

enum class Path { kF32, kGrouped, kGroupedF8, kStream };

Path choose_path(const moe_params& p, int T) {
  if (p.weight_dtype == MOE_F32) return Path::kF32;
  if (p.act_quant == MOE_ACT_QUANT_E4M3_1X128) return Path::kGroupedF8;
  if (p.path == MOE_PATH_GROUPED) return Path::kGrouped;
  if (p.path == MOE_PATH_STREAM) return Path::kStream;
  return T > 256 ? Path::kGrouped : Path::kStream;
}

moe_status hip_fail(moe_cfg* c, hipError_t e) {
  c->last_hip_error = (int)e;
  return MOE_ERR_HIP;
}

bool on_cfg_device(const moe_cfg* c) {
  int d = -1;
  return hipGetDevice(&d) == hipSuccess && d == c->device;
}

// the dispatch tables (item prefixes) for the chosen GEMM path
void fill_dispatch_geometry(const moe_params& p, Path path, int T, DispatchArgs* d) {
  d->shared_rows = p.shared_hidden > 0 ? T : 0;
  if (path == Path::kGrouped) {
    d->bm1 = d->bm2 = kGB_BM;
    d->n1_routed = p.hidden / kG1_BNH;
    d->n1_shared = p.shared_hidden / kG1_BNH;
    d->n2_routed = d->n2_shared = (p.dim + kG2_BN - 1) / kG2_BN;
  } else if (path == Path::kGroupedF8) {
    d->bm1 = kF8_BM1;
    d->bm2 = kF8_BM2;
    d->n1_routed = p.hidden / kG1_BNH;
    d->n1_shared = p.shared_hidden / kG1_BNH;
    d->n2_routed = d->n2_shared = (p.dim + kG2_BN - 1) / kG2_BN;
  } else if (path == Path::kStream) {
    d->bm1 = d->bm2 = kST_BM;
    d->n1_routed = p.hidden / kST_N1;
    d->n1_shared = p.shared_hidden / kST_N1;
    d->n2_routed = d->n2_shared = p.dim / kST_N2;
  } else {
    d->bm1 = d->bm2 = kF32_BM;
    d->n1_routed = (p.hidden + 31) / 32;
    d->n1_shared = (p.shared_hidden + 31) / 32;
    d->n2_routed = d->n2_shared = (p.dim + 63) / 64;
  }
}

// records the boundary event `stage` (0 .. MOE_NUM_STAGES) of the current timed call
void mark(moe_cfg* c, int stage, hipStream_t s) {
  if (!c->timing || c->timed_calls >= MOE_TIMING_CALLS) return;
  (void)hipEventRecord(c->events[c->timed_calls * (MOE_NUM_STAGES + 1) + stage], s);
  if (stage == MOE_NUM_STAGES) c->timed_calls++;
}

void destroy_events(moe_cfg* c) {
  if (!c->events) return;
  for (int i = 0; i < MOE_TIMING_CALLS * (MOE_NUM_STAGES + 1); ++i) (void)hipEventDestroy(c->events[i]);
  free(c->events);
  c->events = nullptr;
}

__global__ void zero_counts_kernel(int32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

hipError_t zero_f32(float* p, size_t n, hipStream_t s) { return launch_zero_f32(p, n, s); }

// Workspace layout for c->p (max_tokens tokens) on a part with c->num_cus
// CUs: returns its size in bytes and, when base is given, points the cfg's
// buffers into it.
size_t layout_workspace(moe_cfg* c, char* base) {
  const moe_params* p = &c->p;
  const size_t Tm = (size_t)p->max_tokens, E = p->n_routed, K = p->top_k, D = p->dim;
  const size_t H = p->hidden, Hs = p->shared_hidden;
  const size_t act = (p->weight_dtype == MOE_F32) ? 4 : 2;  // h and y element size
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + std::max<size_t>(bytes, 1)); return o; };
  // partial-logit planes: the router uses at most 64 * CUs / T + 1 planes of
  // T rows (checked again before each launch)
  const size_t lg = (size_t)64 * c->num_cus + Tm;
  const size_t o_logits = take(lg * E * 4), o_idx = take(Tm * K * 4), o_gate = take(Tm * K * 4);
  const size_t o_spart = take((size_t)score_part_rows((int)Tm) * E * 4);
  // the bf16x3 router planes of gate_w are used from kRouterX3MinTokens tokens on
  const bool wsplit = p->act_dtype == MOE_BF16 && Tm >= (size_t)kRouterX3MinTokens;
  const size_t o_wsplit = wsplit ? take(3 * E * D * 2) : 0;
  const size_t o_counts = take(E * 4), o_offsets = take((E + 1) * 4), o_chunk = take(((Tm * K + kDispatchChunk - 1) / kDispatchChunk + 1) * E * 4);
  const size_t o_pre1 = take((E + 2) * 4), o_pre2 = take((E + 2) * 4);
  const size_t o_rt = take(Tm * K * 4), o_rg = take(Tm * K * 4), o_sr = take(Tm * K * 4);
  const size_t o_hr = take(Tm * K * H * act), o_hs = take(Tm * Hs * act);
  const size_t o_yr = take(Tm * K * D * act), o_ys = take(Tm * D * act);
  const bool aq = p->act_quant == MOE_ACT_QUANT_E4M3_1X128;
  const size_t o_xq = aq ? take(Tm * D) : 0, o_xs = aq ? take(Tm * (D / 128) * 4) : 0;
  const size_t o_hsr = aq ? take(Tm * K * (H / 128) * 4) : 0, o_hss = aq ? take(Tm * (Hs / 128) * 4) : 0;
  const bool bw = p->backward != 0;
  const size_t Ep = (E + 63) / 64 * 64;
  // d gate_w: K (tokens) split so that about one 256 x 256 tile per CU runs
  const int rw_tiles = (int)((Ep + 255) / 256) * (int)((D + 255) / 256);
  const int splits = bw ? std::max(1, std::min(32, (c->num_cus + rw_tiles - 1) / std::max(rw_tiles, 1))) : 0;
  const size_t o_dout = bw ? take(Tm * D * 2) : 0, o_gw = bw ? take(Ep * D * 2) : 0;
  const size_t o_au = bw ? take(Tm * K * 2 * H * 2) : 0, o_aus = bw ? take(Tm * 2 * Hs * 2) : 0;
  const size_t o_gh = bw ? take(Tm * K * H * 2) : 0, o_ghs = bw ? take(Tm * Hs * 2) : 0;
  const size_t o_dau = bw ? take(Tm * K * 2 * H * 2) : 0, o_daus = bw ? take(Tm * 2 * Hs * 2) : 0;
  const size_t o_part = bw ? take(Tm * K * (H / 128) * 4) : 0, o_parts = bw ? take(Tm * (Hs / 128) * 4) : 0;
  const size_t o_dlog = bw ? take(Tm * Ep * 2) : 0, o_dxr = bw ? take(Tm * D * 4) : 0;
  const size_t o_planes = bw ? take((size_t)splits * E * D * 4) : 0;
  const size_t o_preh = bw ? take((E + 2) * 4) : 0, o_prex = bw ? take((E + 2) * 4) : 0;
  if (!base) return off;
  c->logit_rows = lg;
  c->logits = (float*)(base + o_logits);
  c->score_part = (float*)(base + o_spart);
  c->w_split = wsplit ? (uint16_t*)(base + o_wsplit) : nullptr;
  c->idx = (int32_t*)(base + o_idx);
  c->gate = (float*)(base + o_gate);
  c->counts = (int32_t*)(base + o_counts);
  c->offsets = (int32_t*)(base + o_offsets);
  c->chunk_base = (int32_t*)(base + o_chunk);
  c->pre1 = (int32_t*)(base + o_pre1);
  c->pre2 = (int32_t*)(base + o_pre2);
  c->row_token = (int32_t*)(base + o_rt);
  c->row_gate = (float*)(base + o_rg);
  c->slot_row = (int32_t*)(base + o_sr);
  c->h_routed = base + o_hr;
  c->h_shared = base + o_hs;
  c->y_routed = base + o_yr;
  c->y_shared = base + o_ys;
  if (bw) {
    c->Ep = (int)Ep;
    c->bwd_splits = splits;
    c->dout_bf = (uint16_t*)(base + o_dout);
    c->gw_bf = (uint16_t*)(base + o_gw);
    c->au = (uint16_t*)(base + o_au);
    c->au_shared = (uint16_t*)(base + o_aus);
    c->gh = (uint16_t*)(base + o_gh);
    c->gh_shared = (uint16_t*)(base + o_ghs);
    c->dau = (uint16_t*)(base + o_dau);
    c->dau_shared = (uint16_t*)(base + o_daus);
    c->part = (float*)(base + o_part);
    c->part_shared = (float*)(base + o_parts);
    c->dlogit = (uint16_t*)(base + o_dlog);
    c->dx_router = (float*)(base + o_dxr);
    c->gw_planes = (float*)(base + o_planes);
    c->pre_h = (int32_t*)(base + o_preh);
    c->pre_x = (int32_t*)(base + o_prex);
  }
  if (aq) {
    c->xq = (uint8_t*)(base + o_xq);
    c->xs = (float*)(base + o_xs);
    c->hs_routed = (float*)(base + o_hsr);
    c->hs_shared = (float*)(base + o_hss);
  }
  return off;
}

// The no-allocation forward's workspace: one array per GPU, loaded with the
// code object and held until the process ends. Host code never passes its
// name to a kernel (on the host it is only a stand-in); the device address
// comes from hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxScratchDevices = 64;
static __device__ __align__(256) char scratch[kScratchBytes];
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxScratchDevices];
int g_scratch_cus[kMaxScratchDevices];

// the current device's scratch address and CU count (set up on its first use)
moe_status scratch_of_current_device(int* dev, char** ptr, int* cus) {
  if (hipGetDevice(dev) != hipSuccess) return MOE_ERR_HIP;
  if (*dev < 0 || *dev >= kMaxScratchDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[*dev]) {
    void* p = nullptr;
    int n = 0;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_ERR_HIP;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, *dev) != hipSuccess || n <= 0)
      return MOE_ERR_HIP;
    g_scratch_cus[*dev] = n;
    g_scratch_ptr[*dev] = static_cast<char*>(p);
  }
  *ptr = g_scratch_ptr[*dev];
  *cus = g_scratch_cus[*dev];
  return MOE_OK;
}

// The layer forward on the cfg's workspace (arguments checked by the caller
// for T and the device; the rest here).
moe_status forward_impl(moe_cfg* c, const void* x, int T, const float* gate_w, const float* sel_bias,
                             const moe_weights* expert_w, const moe_weights* shared_w, void* out,
                             int32_t* expert_counts, void* stream, bool train = false) {
  const moe_params& p = c->p;
  hipStream_t s = (hipStream_t)stream;
  if (T == 0) {
    if (expert_counts) {
      hipLaunchKernelGGL(zero_counts_kernel, dim3(1), dim3(256), 0, s, expert_counts, p.n_routed);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return hip_fail(c, e);
    }
    if (c->score_sum) {
      hipError_t e = zero_f32(c->score_sum, p.n_routed, s);
      if (e != hipSuccess) return hip_fail(c, e);
    }
    return MOE_OK;
  }
  if (!x || !gate_w || !out || !expert_w || !expert_w->gate_up || !expert_w->down) return MOE_ERR_INVALID_ARG;
  const bool fp8 = p.weight_dtype == MOE_FP8_E4M3;
  if (fp8 && (!expert_w->gate_up_scale || !expert_w->down_scale)) return MOE_ERR_INVALID_ARG;
  const bool has_shared = p.shared_hidden > 0;
  if (has_shared) {
    if (!shared_w || !shared_w->gate_up || !shared_w->down) return MOE_ERR_INVALID_ARG;
    if (fp8 && (!shared_w->gate_up_scale || !shared_w->down_scale)) return MOE_ERR_INVALID_ARG;
  }

  // a training forward takes the grouped path: its gate/up GEMM also leaves
  // [a | u] and g * h for the backward pass
  const Path path = train ? Path::kGrouped : choose_path(p, T);
  hipError_t e;

  // 1. router
  mark(c, 0, s);
  RouterArgs r{};
  r.x = x; r.gate_w = gate_w; r.bias = sel_bias; r.logits = c->logits;
  r.idx = c->idx; r.gate = c->gate; r.counts = c->counts;
  r.T = T; r.D = p.dim; r.E = p.n_routed; r.G = p.n_group; r.kg = p.topk_group; r.K = p.top_k;
  r.act_bf16 = p.act_dtype == MOE_BF16; r.score_fn = p.score_fn; r.norm = p.norm_topk;
  r.rsf = p.routed_scaling_factor;
  r.num_cus = c->num_cus;
  r.w_split = c->w_split;
  r.logit_rows = c->logit_rows;
  r.score_sum = c->score_sum;
  r.score_part = c->score_part;
  r.hist = !small_dispatch(T * p.top_k);  // the one-workgroup dispatch counts the entries itself
  if ((e = launch_router(r, s)) != hipSuccess) return hip_fail(c, e);
  mark(c, 1, s);

  // 2. dispatch
  DispatchArgs d{};
  d.idx = c->idx; d.gate = c->gate; d.counts = c->counts; d.counts_out = expert_counts;
  d.offsets = c->offsets; d.chunk_base = c->chunk_base; d.row_token = c->row_token; d.row_gate = c->row_gate;
  d.slot_row = c->slot_row; d.pre1 = c->pre1; d.pre2 = c->pre2;
  d.T = T; d.K = p.top_k; d.E = p.n_routed;
  fill_dispatch_geometry(p, path, T, &d);
  if ((e = launch_dispatch(d, s)) != hipSuccess) return hip_fail(c, e);
  mark(c, 2, s);

  // 3./4. expert GEMMs
  const int TK = T * p.top_k;
  ExpertGemmArgs g{};
  g.offsets = c->offsets; g.row_token = c->row_token; g.row_gate = c->row_gate;
  g.E = p.n_routed; g.T = has_shared ? T : 0; g.D = p.dim; g.H = p.hidden; g.Hs = p.shared_hidden;
  g.x_rows = T;
  ExpertGemmArgs g1 = g, g2 = g;
  g1.pre = c->pre1;
  g1.a = x; g1.w = expert_w->gate_up; g1.w_scale = expert_w->gate_up_scale;
  g1.w_shared = has_shared ? shared_w->gate_up : nullptr;
  g1.w_shared_scale = has_shared ? shared_w->gate_up_scale : nullptr;
  g1.c = c->h_routed; g1.c_shared = c->h_shared;
  g2.pre = c->pre2;
  g2.a = c->h_routed; g2.a_shared = c->h_shared; g2.w = expert_w->down; g2.w_scale = expert_w->down_scale;
  g2.w_shared = has_shared ? shared_w->down : nullptr;
  g2.w_shared_scale = has_shared ? shared_w->down_scale : nullptr;
  g2.c = c->y_routed; g2.c_shared = c->y_shared;

  // upper bounds on the item counts the dispatch can produce
  auto row_blocks = [&](int bm) { return (long)(TK + bm - 1) / bm + p.n_routed; };
  auto row_blocks_s = [&](int bm) { return has_shared ? (long)(T + bm - 1) / bm : 0L; };
  g1.max_items = (int)(row_blocks(d.bm1) * d.n1_routed + row_blocks_s(d.bm1) * d.n1_shared);
  g2.max_items = (int)(row_blocks(d.bm2) * d.n2_routed + row_blocks_s(d.bm2) * d.n2_shared);
  if (path == Path::kF32) {
    if ((e = launch_simple_gateup_f32(g1, TK, s)) != hipSuccess) return hip_fail(c, e);
    mark(c, 3, s);
    if ((e = launch_simple_down_f32(g2, TK, s)) != hipSuccess) return hip_fail(c, e);
  } else {
    if (path == Path::kGrouped && train) {
      g1.c2 = c->au; g1.c2_shared = c->au_shared; g1.c3 = c->gh; g1.c3_shared = c->gh_shared;
      if ((e = launch_grouped_gateup_train(g1, s)) != hipSuccess) return hip_fail(c, e);
      mark(c, 3, s);
      if ((e = launch_grouped_down(g2, fp8, s)) != hipSuccess) return hip_fail(c, e);
    } else if (path == Path::kGrouped) {
      if ((e = launch_grouped_gateup(g1, fp8, s)) != hipSuccess) return hip_fail(c, e);
      mark(c, 3, s);
      if ((e = launch_grouped_down(g2, fp8, s)) != hipSuccess) return hip_fail(c, e);
    } else if (path == Path::kGroupedF8) {
      // token rows to e4m3 (counted in the gate/up stage), then both GEMMs on
      // codes + block scales; the gate/up GEMM writes h as codes + scales
      if ((e = launch_quant_e4m3(static_cast<const uint16_t*>(x), T, p.dim, c->xq, c->xs, s)) != hipSuccess)
        return hip_fail(c, e);
      g1.a = c->xq; g1.a_scale = c->xs;
      g1.c_scale = c->hs_routed; g1.c_shared_scale = c->hs_shared;
      g2.a_scale = c->hs_routed; g2.a_shared_scale = c->hs_shared;
      if ((e = launch_grouped_gateup_f8(g1, s)) != hipSuccess) return hip_fail(c, e);
      mark(c, 3, s);
      if ((e = launch_grouped_down_f8(g2, s)) != hipSuccess) return hip_fail(c, e);
    } else {
      // persistent workgroups: as many as fit on the CUs at once
      if ((e = launch_stream_gateup(g1, fp8, g1.max_items, c->num_cus, s)) != hipSuccess) return hip_fail(c, e);
      mark(c, 3, s);
      if ((e = launch_stream_down(g2, fp8, g2.max_items, c->num_cus, s)) != hipSuccess) return hip_fail(c, e);
    }
  }

  // 5. combine
  mark(c, 4, s);
  CombineArgs cb{};
  cb.x = x; cb.y_routed = c->y_routed; cb.y_shared = has_shared ? c->y_shared : nullptr;
  cb.slot_row = c->slot_row; cb.out = out; cb.T = T; cb.D = p.dim; cb.K = p.top_k;
  cb.act_bf16 = p.act_dtype == MOE_BF16; cb.y_bf16 = p.weight_dtype != MOE_F32;
  cb.out_bf16 = p.out_dtype == MOE_BF16; cb.add_residual = p.add_residual;
  if ((e = launch_combine(cb, s)) != hipSuccess) return hip_fail(c, e);
  mark(c, 5, s);
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MOE_ERR_OOM: return "out of device memory";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_SCRATCH: return "input needs more than the no-allocation scratch holds";
  }
  return "unknown status";
}

moe_status moe_cfg_create(const moe_params* p, moe_cfg** out) {
  if (!out) return MOE_ERR_INVALID_ARG;
  *out = nullptr;
  moe_status st = validate(p);
  if (st != MOE_OK) return st;
  moe_cfg* c = new (std::nothrow) moe_cfg;
  if (!c) return MOE_ERR_OOM;
  memset(c, 0, sizeof(*c));
  c->p = *p;
  c->saved_T = -1;
  if (hipGetDevice(&c->device) != hipSuccess) { delete c; return MOE_ERR_HIP; }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, c->device) != hipSuccess) { delete c; return MOE_ERR_HIP; }
  c->num_cus = prop.multiProcessorCount;
  c->ws_bytes = layout_workspace(c, nullptr);
  if (hipMalloc((void**)&c->ws, c->ws_bytes) != hipSuccess) {
    (void)hipGetLastError();
    delete c;
    return MOE_ERR_OOM;
  }
  layout_workspace(c, c->ws);
  *out = c;
  return MOE_OK;
}

moe_status moe_cfg_destroy(moe_cfg* cfg) {
  if (!cfg) return MOE_OK;
  int prev = -1;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(cfg->device);
  (void)hipDeviceSynchronize();
  destroy_events(cfg);
  hipError_t e = hipFree(cfg->ws);
  if (prev >= 0) (void)hipSetDevice(prev);
  delete cfg;
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

size_t moe_cfg_workspace_bytes(const moe_cfg* cfg) { return cfg ? cfg->ws_bytes : 0; }

int moe_cfg_last_hip_error(const moe_cfg* cfg) { return cfg ? cfg->last_hip_error : 0; }

moe_status moe_cfg_set_stage_timing(moe_cfg* c, int enable) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (enable && !c->events) {
    const int n = MOE_TIMING_CALLS * (MOE_NUM_STAGES + 1);
    c->events = (hipEvent_t*)calloc(n, sizeof(hipEvent_t));
    if (!c->events) return MOE_ERR_OOM;
    for (int i = 0; i < n; ++i) {
      hipError_t e = hipEventCreate(&c->events[i]);
      if (e != hipSuccess) {
        for (int j = 0; j < i; ++j) (void)hipEventDestroy(c->events[j]);
        free(c->events);
        c->events = nullptr;
        return hip_fail(c, e);
      }
    }
  }
  c->timing = enable != 0 && c->events != nullptr;
  c->timed_calls = 0;
  return MOE_OK;
}

moe_status moe_cfg_stage_times(moe_cfg* c, double* ms, int* calls) {
  if (!c || !ms) return MOE_ERR_INVALID_ARG;
  for (int k = 0; k < MOE_NUM_STAGES; ++k) ms[k] = 0.0;
  const int n = c->timed_calls;
  if (calls) *calls = n;
  if (n == 0) return MOE_OK;
  hipError_t e = hipEventSynchronize(c->events[(n - 1) * (MOE_NUM_STAGES + 1) + MOE_NUM_STAGES]);
  if (e != hipSuccess) return hip_fail(c, e);
  for (int i = 0; i < n; ++i) {
    for (int k = 0; k < MOE_NUM_STAGES; ++k) {
      float t = 0.f;
      e = hipEventElapsedTime(&t, c->events[i * (MOE_NUM_STAGES + 1) + k], c->events[i * (MOE_NUM_STAGES + 1) + k + 1]);
      if (e != hipSuccess) return hip_fail(c, e);
      ms[k] += t;
    }
  }
  c->timed_calls = 0;
  return MOE_OK;
}

moe_status moe_router_forward(moe_cfg* c, const void* x, int T, const float* gate_w, const float* sel_bias,
                              int32_t* topk_idx, float* topk_gate, int32_t* expert_counts, void* stream) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (T < 0 || T > c->p.max_tokens) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!x || !gate_w || !topk_idx || !topk_gate)) return MOE_ERR_INVALID_ARG;
  if (!on_cfg_device(c)) return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  int32_t* counts = expert_counts ? expert_counts : c->counts;
  if (T == 0) {
    hipLaunchKernelGGL(zero_counts_kernel, dim3(1), dim3(256), 0, s, counts, c->p.n_routed);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && c->score_sum) e = zero_f32(c->score_sum, c->p.n_routed, s);
    return e == hipSuccess ? MOE_OK : hip_fail(c, e);
  }
  RouterArgs r{};
  r.x = x; r.gate_w = gate_w; r.bias = sel_bias; r.logits = c->logits;
  r.idx = topk_idx; r.gate = topk_gate; r.counts = counts;
  r.T = T; r.D = c->p.dim; r.E = c->p.n_routed; r.G = c->p.n_group; r.kg = c->p.topk_group; r.K = c->p.top_k;
  r.act_bf16 = c->p.act_dtype == MOE_BF16; r.score_fn = c->p.score_fn; r.norm = c->p.norm_topk;
  r.rsf = c->p.routed_scaling_factor;
  r.num_cus = c->num_cus;
  r.w_split = c->w_split;
  r.logit_rows = c->logit_rows;
  r.score_sum = c->score_sum;
  r.score_part = c->score_part;
  r.hist = 1;
  hipError_t e = launch_router(r, s);
  return e == hipSuccess ? MOE_OK : hip_fail(c, e);
}

moe_status moe_quantize_e4m3_1x128(const void* x, int rows, int cols, uint8_t* codes, float* scales,
                                   void* stream) {
  if (rows < 0 || cols <= 0 || cols % kActBlock != 0) return MOE_ERR_INVALID_ARG;
  if ((uint64_t)rows * (uint64_t)cols > (1ull << 34)) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (!x || !codes || !scales) return MOE_ERR_INVALID_ARG;
  return launch_quant_e4m3(static_cast<const uint16_t*>(x), rows, cols, codes, scales, (hipStream_t)stream) ==
                 hipSuccess
             ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_bias_update(const int32_t* expert_counts, int E, float gamma, float* sel_bias, void* stream) {
  if (!expert_counts || !sel_bias || E < 1 || E > kMaxExperts) return MOE_ERR_INVALID_ARG;
  if (!(gamma == gamma) || gamma > 3.4e38f || gamma < -3.4e38f) return MOE_ERR_INVALID_ARG;  // NaN, inf
  return launch_balance(expert_counts, E, gamma, sel_bias, nullptr, (hipStream_t)stream) == hipSuccess
             ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_load_stats(const int32_t* expert_counts, int E, float* stats, void* stream) {
  if (!expert_counts || !stats || E < 1 || E > kMaxExperts) return MOE_ERR_INVALID_ARG;
  return launch_balance(expert_counts, E, 0.f, nullptr, stats, (hipStream_t)stream) == hipSuccess
             ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_debug_status(int* site, int* value) {
  if (!site || !value) return MOE_ERR_INVALID_ARG;
  *site = 0;
  *value = 0;
#ifdef MOE_DEBUG
  if (hipDeviceSynchronize() != hipSuccess) return MOE_ERR_HIP;
  hipError_t (*readers[])(unsigned long long*) = {debug_read_dispatch, debug_read_grouped, debug_read_f8,
                                                   debug_read_stream, debug_read_f32, debug_read_bwd};
  for (auto rd : readers) {
    unsigned long long w = 0;
    if (rd(&w) != hipSuccess) return MOE_ERR_HIP;
    if (w != 0 && *site == 0) {
      *site = (int)(w >> 32);
      *value = (int)(uint32_t)w;
    }
  }
  return MOE_OK;
#else
  return MOE_ERR_UNSUPPORTED;
#endif
}

moe_status moe_cfg_set_score_sums(moe_cfg* c, float* score_sum) {
  if (!c) return MOE_ERR_INVALID_ARG;
  c->score_sum = score_sum;
  return MOE_OK;
}

moe_status moe_balance_stats(const int32_t* expert_counts, const float* score_sum, int E, int n_devices,
                             float* stats, void* stream) {
  if (!expert_counts || !score_sum || !stats || E < 1 || E > kMaxExperts) return MOE_ERR_INVALID_ARG;
  if (n_devices < 1 || n_devices > E || E % n_devices != 0) return MOE_ERR_INVALID_ARG;
  return launch_balance_stats(expert_counts, score_sum, E, n_devices, stats, (hipStream_t)stream) == hipSuccess
             ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_dispatch_forward(moe_cfg* c, const int32_t* topk_idx, int T, int32_t* offsets,
                                int32_t* row_token, int32_t* slot_row, void* stream) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (T < 0 || T > c->p.max_tokens) return MOE_ERR_INVALID_ARG;
  if (!offsets || (T > 0 && (!topk_idx || !row_token || !slot_row))) return MOE_ERR_INVALID_ARG;
  if (!on_cfg_device(c)) return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (!small_dispatch(T * c->p.top_k)) {  // the one-workgroup dispatch counts the entries itself
    e = launch_histogram(topk_idx, c->counts, T * c->p.top_k, c->p.n_routed, s);
    if (e != hipSuccess) return hip_fail(c, e);
  }
  DispatchArgs d{};
  d.idx = topk_idx; d.gate = nullptr; d.counts = c->counts; d.counts_out = nullptr;
  d.offsets = offsets; d.chunk_base = c->chunk_base; d.row_token = row_token; d.row_gate = nullptr;
  d.slot_row = slot_row; d.pre1 = c->pre1; d.pre2 = c->pre2;
  d.T = T; d.K = c->p.top_k; d.E = c->p.n_routed;
  fill_dispatch_geometry(c->p, choose_path(c->p, T), T, &d);
  e = launch_dispatch(d, s);
  return e == hipSuccess ? MOE_OK : hip_fail(c, e);
}

moe_status moe_layer_forward(moe_cfg* c, const void* x, int T, const float* gate_w, const float* sel_bias,
                             const moe_weights* expert_w, const moe_weights* shared_w, void* out,
                             int32_t* expert_counts, void* stream) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (T < 0 || T > c->p.max_tokens) return MOE_ERR_INVALID_ARG;
  if (!on_cfg_device(c)) return MOE_ERR_INVALID_ARG;
  return forward_impl(c, x, T, gate_w, sel_bias, expert_w, shared_w, out, expert_counts, stream);
}

moe_status moe_layer_forward_train(moe_cfg* c, const void* x, int T, const float* gate_w, const float* sel_bias,
                                   const moe_weights* expert_w, const moe_weights* shared_w, void* out,
                                   int32_t* expert_counts, void* stream) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (!c->p.backward) return MOE_ERR_UNSUPPORTED;
  if (T < 0 || T > c->p.max_tokens) return MOE_ERR_INVALID_ARG;
  if (!on_cfg_device(c)) return MOE_ERR_INVALID_ARG;
  c->saved_T = -1;
  const moe_status st = forward_impl(c, x, T, gate_w, sel_bias, expert_w, shared_w, out, expert_counts, stream, true);
  if (st == MOE_OK) c->saved_T = T;
  return st;
}

moe_status moe_layer_forward_noalloc(const moe_params* params, const void* x, int T, const float* gate_w,
                                     const float* sel_bias, const moe_weights* expert_w,
                                     const moe_weights* shared_w, void* out, int32_t* expert_counts,
                                     void* stream) {
  if (!params || T < 0) return MOE_ERR_INVALID_ARG;
  // a cfg on the stack: the layer as given, sized for exactly T tokens, no
  // backward workspace, its buffers in this device's scratch array
  moe_cfg c;
  memset(&c, 0, sizeof(c));
  c.p = *params;
  c.p.max_tokens = T;
  c.p.backward = 0;
  moe_status st = validate(&c.p);
  if (st != MOE_OK) return st;
  char* base = nullptr;
  if ((st = scratch_of_current_device(&c.device, &base, &c.num_cus)) != MOE_OK) return st;
  c.ws_bytes = layout_workspace(&c, nullptr);
  if (c.ws_bytes > kScratchBytes) return MOE_ERR_SCRATCH;
  c.ws = base;
  layout_workspace(&c, base);
  return forward_impl(&c, x, T, gate_w, sel_bias, expert_w, shared_w, out, expert_counts, stream);
}

// recompute: the gate/up products are recomputed (moe_layer_backward), else
// read from the last training forward (moe_layer_backward_saved)
static moe_status backward_impl(moe_cfg* c, const void* x, int T, const float* gate_w, const float* sel_bias,
                         const moe_weights* expert_w, const moe_weights* shared_w, const float* d_out, float* dx,
                         float* d_gate_w, const moe_weight_grads* d_expert_w, const moe_weight_grads* d_shared_w,
                         void* stream, bool recompute) {
  if (!c) return MOE_ERR_INVALID_ARG;
  const moe_params& p = c->p;
  if (!p.backward) return MOE_ERR_UNSUPPORTED;
  if (T < 0 || T > p.max_tokens) return MOE_ERR_INVALID_ARG;
  if (!recompute && c->saved_T != T) return MOE_ERR_INVALID_ARG;
  if (!on_cfg_device(c)) return MOE_ERR_INVALID_ARG;
  const bool has_shared = p.shared_hidden > 0;
  if (!gate_w || !d_gate_w || !expert_w || !expert_w->gate_up || !expert_w->down || !d_expert_w ||
      !d_expert_w->gate_up || !d_expert_w->down)
    return MOE_ERR_INVALID_ARG;
  if (has_shared && (!shared_w || !shared_w->gate_up || !shared_w->down || !d_shared_w || !d_shared_w->gate_up ||
                     !d_shared_w->down))
    return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!x || !d_out || !dx)) return MOE_ERR_INVALID_ARG;
  // d_out and dx are read and written 16 bytes at a time
  if (((uintptr_t)d_out | (uintptr_t)dx) & 15) return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  const size_t E = p.n_routed, D = p.dim, H = p.hidden, Hs = p.shared_hidden;
  hipError_t e;
  if (T == 0) {
    if ((e = zero_f32(d_gate_w, E * D, s)) != hipSuccess) return hip_fail(c, e);
    if ((e = zero_f32(d_expert_w->gate_up, E * 2 * H * D, s)) != hipSuccess) return hip_fail(c, e);
    if ((e = zero_f32(d_expert_w->down, E * D * H, s)) != hipSuccess) return hip_fail(c, e);
    if (has_shared) {
      if ((e = zero_f32(d_shared_w->gate_up, 2 * Hs * D, s)) != hipSuccess) return hip_fail(c, e);
      if ((e = zero_f32(d_shared_w->down, D * Hs, s)) != hipSuccess) return hip_fail(c, e);
    }
    return MOE_OK;
  }

  // routing and dispatch exactly as the forward (grouped geometry for the recompute)
  RouterArgs r{};
  r.x = x; r.gate_w = gate_w; r.bias = sel_bias; r.logits = c->logits;
  r.idx = c->idx; r.gate = c->gate; r.counts = c->counts;
  r.T = T; r.D = p.dim; r.E = p.n_routed; r.G = p.n_group; r.kg = p.topk_group; r.K = p.top_k;
  r.act_bf16 = 1; r.score_fn = p.score_fn; r.norm = p.norm_topk;
  r.rsf = p.routed_scaling_factor;
  r.num_cus = c->num_cus;
  r.w_split = c->w_split;
  r.logit_rows = c->logit_rows;
  r.hist = !small_dispatch(T * p.top_k);  // the one-workgroup dispatch counts the entries itself
  if ((e = launch_router(r, s)) != hipSuccess) return hip_fail(c, e);
  DispatchArgs d{};
  d.idx = c->idx; d.gate = c->gate; d.counts = c->counts; d.counts_out = nullptr;
  d.offsets = c->offsets; d.chunk_base = c->chunk_base; d.row_token = c->row_token; d.row_gate = c->row_gate;
  d.slot_row = c->slot_row; d.pre1 = c->pre1; d.pre2 = c->pre2;
  d.T = T; d.K = p.top_k; d.E = p.n_routed;
  fill_dispatch_geometry(p, Path::kGrouped, T, &d);
  if ((e = launch_dispatch(d, s)) != hipSuccess) return hip_fail(c, e);

  // gate/up recompute: [a | u] and g * h (a training forward left them otherwise)
  if (recompute) {
    c->saved_T = -1;  // au and gh now hold this call's values
    const int TK = T * p.top_k;
    ExpertGemmArgs g{};
    g.offsets = c->offsets; g.row_token = c->row_token; g.row_gate = c->row_gate; g.pre = c->pre1;
    g.E = p.n_routed; g.T = has_shared ? T : 0; g.D = p.dim; g.H = p.hidden; g.Hs = p.shared_hidden;
    g.x_rows = T;
    g.a = x; g.w = expert_w->gate_up; g.w_shared = has_shared ? shared_w->gate_up : nullptr;
    g.c = c->au; g.c_shared = c->au_shared; g.c2 = c->gh; g.c2_shared = c->gh_shared;
    const long mblk = (long)(TK + d.bm1 - 1) / d.bm1 + p.n_routed;
    const long mblk_s = has_shared ? (T + d.bm1 - 1) / d.bm1 : 0;
    g.max_items = (int)(mblk * d.n1_routed + mblk_s * d.n1_shared);
    if ((e = launch_grouped_recompute(g, s)) != hipSuccess) return hip_fail(c, e);
  }

  BwdArgs b{};
  b.E = p.n_routed; b.T = T; b.D = p.dim; b.H = p.hidden; b.Hs = p.shared_hidden; b.K = p.top_k;
  b.Ep = c->Ep; b.splits = c->bwd_splits;
  b.score_fn = p.score_fn; b.norm = p.norm_topk; b.rsf = p.routed_scaling_factor; b.add_residual = p.add_residual;
  b.offsets = c->offsets; b.row_token = c->row_token; b.row_gate = c->row_gate; b.slot_row = c->slot_row;
  b.idx = c->idx; b.logits = c->logits; b.pre_h = c->pre_h; b.pre_x = c->pre_x;
  b.x = static_cast<const uint16_t*>(x); b.dout_f32 = d_out; b.gate_w = gate_w;
  b.w_gu = static_cast<const uint16_t*>(expert_w->gate_up);
  b.w_down = static_cast<const uint16_t*>(expert_w->down);
  b.w_gu_shared = has_shared ? static_cast<const uint16_t*>(shared_w->gate_up) : nullptr;
  b.w_down_shared = has_shared ? static_cast<const uint16_t*>(shared_w->down) : nullptr;
  b.dout = c->dout_bf; b.gw_bf16 = c->gw_bf;
  b.au = c->au; b.au_shared = c->au_shared;
  b.gh = c->gh; b.gh_shared = c->gh_shared;
  b.dau = c->dau; b.dau_shared = c->dau_shared; b.part = c->part; b.part_shared = c->part_shared;
  b.dxr = static_cast<uint16_t*>(c->y_routed); b.dxs = static_cast<uint16_t*>(c->y_shared);
  b.dlogit = c->dlogit; b.dx_router = c->dx_router; b.gw_planes = c->gw_planes;
  b.dx = dx; b.d_gate_w = d_gate_w; b.dw_gu = d_expert_w->gate_up; b.dw_down = d_expert_w->down;
  b.dw_gu_shared = has_shared ? d_shared_w->gate_up : nullptr;
  b.dw_down_shared = has_shared ? d_shared_w->down : nullptr;
  if ((e = launch_layer_backward(b, s)) != hipSuccess) return hip_fail(c, e);
  return MOE_OK;
}

moe_status moe_layer_backward(moe_cfg* c, const void* x, int T, const float* gate_w, const float* sel_bias,
                              const moe_weights* expert_w, const moe_weights* shared_w, const float* d_out,
                              float* dx, float* d_gate_w, const moe_weight_grads* d_expert_w,
                              const moe_weight_grads* d_shared_w, void* stream) {
  return backward_impl(c, x, T, gate_w, sel_bias, expert_w, shared_w, d_out, dx, d_gate_w, d_expert_w, d_shared_w,
                       stream, true);
}

moe_status moe_layer_backward_saved(moe_cfg* c, const void* x, int T, const float* gate_w, const float* sel_bias,
                                    const moe_weights* expert_w, const moe_weights* shared_w, const float* d_out,
                                    float* dx, float* d_gate_w, const moe_weight_grads* d_expert_w,
                                    const moe_weight_grads* d_shared_w, void* stream) {
  return backward_impl(c, x, T, gate_w, sel_bias, expert_w, shared_w, d_out, dx, d_gate_w, d_expert_w, d_shared_w,
                       stream, false);
}

}  // extern "C"
