// Weight-streaming expert GEMMs for small token counts (decode), bf16 or fp8
// (OCP e4m3 with one fp32 scale per 128x128 block) weights, bf16 activations.
//
// With a few tokens per expert the layer is bound by reading each touched
// expert's weights once from HBM. A workgroup owns a sequence of work items:
// one item is up to 16 token rows of one problem (routed expert or the shared
// expert) against 64 of its weight rows over the whole K extent. Each of the
// four waves streams its own 16 weight rows straight from HBM into MFMA
// operands; the activation rows are shared by the four waves through a small
// LDS ring. An expert with more than 16 rows in the call gets one item per 16
// rows. Inside a problem the items go column-major (the row blocks of one
// weight slice are consecutive), and the item list is cut into one
// contiguous stretch per XCD (workgroup b runs on XCD b % 8): the XCD's
// workgroups walk their stretch in rounds of consecutive items, so the items
// that read one weight slice run side by side on one XCD and share its lines
// through that L2, and a row block's activations (the down GEMM's h rows,
// read by every item of the block) are fetched into one L2, not eight.
//
// v_mfma_f32_16x16x32_bf16: lane l supplies A[token l%16][8 k] and
// B[8 k][weight row l%16] for k-group l/16. Within a 128-wide K chunk, lane
// group q reads the 32 consecutive k at 32q and feeds k 32q+8j..+7 to MFMA j;
// A and B use the same assignment, so each dot product is unchanged.
// fp8 weights are widened to bf16 exactly (every e4m3 value is a bf16 value);
// the 128-wide chunk is accumulated unscaled, then multiplied by its block
// scale and added to the fp32 accumulator.
//
// Gate/up items: wave w takes 8 W_gate rows and the matching 8 W_up rows, so
// the SwiGLU epilogue (h = SiLU(gate) * up, DeepSeek-V2 walkthrough page MoE
// code and the SwiGLU expert of the architecture article, section 3.3) needs
// only a lane swap. Down items write g * (h W_down^T) for 16 output columns
// per wave.
//
// Latency: chunks are handled in groups of four. The weights and the
// activations of group g+1 -- of this item, or the first group of the
// workgroup's next item -- are requested before group g is multiplied; the
// activations go through registers into the other half of the LDS ring, with
// one barrier per group. The activations are requested before the weights,
// so the end-of-group wait for them leaves the weights in flight until the
// next group multiplies them, by which time the group after that is already
// requested. The problem tables (item prefix, expert row offsets)
// are cached in LDS, so finding an item's problem costs no global round trips.
#include <algorithm>
#include <type_traits>

#include "moe_internal.hpp"

namespace moe {

// 2 e4m3 codes (bytes 0-1 or 2-3 of w) -> 2 packed bf16, exact (unit scale).
// The packed result is kept as one 32-bit word and never split into lanes of
// a vector type.
template <bool kHigh>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHigh));
}

__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  const uint4 u = make_uint4(fp8x2_to_bf16x2<false>(lo), fp8x2_to_bf16x2<true>(lo),
                             fp8x2_to_bf16x2<false>(hi), fp8x2_to_bf16x2<true>(hi));
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

namespace {

constexpr int kU = 4;               // chunks per group
constexpr int kXcds = 8;            // XCDs of the part; workgroup b runs on XCD b % 8
constexpr int kALd = kST_KC + 8;    // LDS row length of an activation chunk (bf16), padded
constexpr int kASlot = 16 * kALd;   // one chunk of 16 activation rows

// One work item, as seen by one thread.
struct Item {
  const char* wptr;      // this lane's weight row at its k-group offset
  const float* sptr;     // this lane's block-scale row (fp8)
  const uint16_t* aptr;  // this thread's activation row (row tid/16, piece tid%16)
  bool aval;             // that row is a valid row of the item
  int nrows;             // valid rows (<= 16)
  int nch;               // 128-wide K chunks
  uint16_t* out;         // output row 0 of the item, at this wave's first column
  const float* gate;     // gates from row 0 (routed down items), else null
  int ldo;               // output row length
};

template <bool kFp8, int kMode>
__device__ __forceinline__ Item setup_item(const ExpertGemmArgs& a, const int32_t* s_pre, const int32_t* s_off,
                                           int item) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rr = lane & 15, q = lane >> 4;
  Item it;
  const int p = find_problem(s_pre, a.E, item);
  const bool routed = p < a.E;
  const int rows = routed ? s_off[p + 1] - s_off[p] : a.T;
  const int row_base = routed ? s_off[p] : 0;
  const int Hp = routed ? a.H : a.Hs;
  const int local = item - s_pre[p];
  // column-major: consecutive items are the row blocks of one weight slice
  const int nmb = (rows + kST_BM - 1) / kST_BM;  // >= 1: p owns this item
  const int nb = local / nmb;
  const int m0 = (local % nmb) * kST_BM;
  it.nrows = min(rows - m0, kST_BM);
  const int K = (kMode == 0) ? a.D : Hp;
  it.nch = K / kST_KC;
  // this wave's weight rows: gate/up -> 8 gate + 8 up rows; down -> 16 rows
  const int wcol = (kMode == 0) ? nb * kST_N1 + 8 * wave : nb * kST_N2 + 16 * wave;
  const int wrows = (kMode == 0) ? 2 * Hp : a.D;
  const int wrow = (kMode == 0) ? (rr < 8 ? wcol + rr : Hp + wcol + rr - 8) : wcol + rr;
  const size_t welt = kFp8 ? 1 : 2;
  const char* wbase = static_cast<const char*>(routed ? a.w : a.w_shared) +
                      (routed ? (size_t)p * wrows * K * welt : 0);
  it.wptr = wbase + (size_t)wrow * K * welt + (size_t)32 * q * welt;
  it.sptr = nullptr;
  if (kFp8) {
    const int kb = K / kST_KC;
    it.sptr = (routed ? a.w_scale + (size_t)p * (wrows / kST_KC) * kb : a.w_shared_scale) +
              (size_t)(wrow / kST_KC) * kb;
  }
  // activations: thread tid loads row tid/16, 8 elements at (tid%16)*8 of each chunk
  const int arow = tid >> 4;
  it.aval = arow < it.nrows;
  const int mm = m0 + (it.aval ? arow : 0);  // in-bounds row for masked threads
  if (kMode == 0) {
    const int tok = routed ? dcheck(a.row_token[row_base + mm], a.x_rows, kSiteStreamTok) : mm;
    it.aptr = static_cast<const uint16_t*>(a.a) + (size_t)tok * a.D + (tid & 15) * 8;
  } else {
    it.aptr = routed ? static_cast<const uint16_t*>(a.a) + (size_t)(row_base + mm) * a.H + (tid & 15) * 8
                     : static_cast<const uint16_t*>(a.a_shared) + (size_t)mm * a.Hs + (tid & 15) * 8;
  }
  if (kMode == 0) {
    it.ldo = Hp;
    it.out = (routed ? static_cast<uint16_t*>(a.c) + (size_t)(row_base + m0) * a.H
                     : static_cast<uint16_t*>(a.c_shared) + (size_t)m0 * a.Hs) + wcol;
    it.gate = nullptr;
  } else {
    it.ldo = a.D;
    it.out = (routed ? static_cast<uint16_t*>(a.c) + (size_t)(row_base + m0) * a.D
                     : static_cast<uint16_t*>(a.c_shared) + (size_t)m0 * a.D) + wcol;
    it.gate = routed ? a.row_gate + row_base + m0 : nullptr;
  }
  return it;
}

}  // namespace

template <bool kFp8, int kMode>  // kMode 0: gate/up + SwiGLU, 1: down + gate scale
__global__ __launch_bounds__(256) void stream_gemm_kernel(ExpertGemmArgs a) {
  __shared__ int32_t s_pre[kMaxExperts + 2];
  __shared__ int32_t s_off[kMaxExperts + 1];
  __shared__ __attribute__((aligned(16))) uint16_t s_act[2 * kU * kASlot];  // two groups of chunks
  for (int i = threadIdx.x; i < a.E + 2; i += 256) s_pre[i] = a.pre[i];
  for (int i = threadIdx.x; i < a.E + 1; i += 256) s_off[i] = a.offsets[i];
  __syncthreads();

  const int tid = threadIdx.x, lane = tid & 63;
  const int rr = lane & 15, q = lane >> 4;
  const int total = s_pre[a.E + 1];
  // XCD x (workgroups x, x + nx, ...) owns items [beg, end), one nx-th of
  // the list; its gx workgroups take them in rounds of gx consecutive items
  // (a grid that is not a multiple of the XCD count walks one stretch)
  const int nx = (gridDim.x % kXcds == 0) ? kXcds : 1;
  const int gx = (int)gridDim.x / nx;
  const int chunk = (total + nx - 1) / nx;
  const int beg = min(total, ((int)blockIdx.x % nx) * chunk);
  const int end = min(total, beg + chunk);
  int item = beg + (int)blockIdx.x / nx;
  if (item >= end) return;  // uniform over the workgroup

  constexpr int kWv = kFp8 ? 2 : 4;  // 16-byte weight loads per lane per chunk
  constexpr size_t welt = kFp8 ? 1 : 2;
  uint4 wv[2][kU][kWv];
  float sc[2][kU];
  uint4 pa[kU];  // this thread's activation pieces of the next group

  // The activation pieces are requested first and the weights last: loads
  // retire in issue order for the wait counter, so the wait for the
  // activations at the end of a group leaves the weights in flight, and the
  // following group's request goes out before they are waited for.
  auto load_group = [&](const Item& it, int g, uint4 (&w)[kU][kWv], float (&s)[kU]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = min(g * kU + u, it.nch - 1);  // past the end: a valid chunk, unused
      const uint4 v = *reinterpret_cast<const uint4*>(it.aptr + (size_t)c * kST_KC);
      pa[u] = it.aval ? v : make_uint4(0, 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = min(g * kU + u, it.nch - 1);
#pragma unroll
      for (int j = 0; j < kWv; ++j)
        w[u][j] = *reinterpret_cast<const uint4*>(it.wptr + (size_t)c * kST_KC * welt + 16 * j);
      s[u] = kFp8 ? it.sptr[c] : 1.0f;
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // activation pieces -> LDS ring half `set`
  auto store_act = [&](int set) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kU; ++u)
      *reinterpret_cast<uint4*>(&s_act[(set * kU + u) * kASlot + (tid >> 4) * kALd + (tid & 15) * 8]) = pa[u];
  };

  // Issue priority falls in four steps as this workgroup works through its
  // items: the workgroups sharing a CU hold equal item counts, and with equal
  // priority the oldest waves win the issue slots, so the first workgroup
  // on a CU would finish long before the last and leave the CU short of
  // requests in flight; a workgroup that is ahead now yields to those behind.
  const int my_items = (end - 1 - item) / gx + 1;
  int done = 0;
  auto set_priority = [&]() __attribute__((always_inline)) {
    switch (3 - min(3, (4 * done) / my_items)) {
      case 3: __builtin_amdgcn_s_setprio(3); break;
      case 2: __builtin_amdgcn_s_setprio(2); break;
      case 1: __builtin_amdgcn_s_setprio(1); break;
      default: __builtin_amdgcn_s_setprio(0); break;
    }
  };
  set_priority();
  Item cur = setup_item<kFp8, kMode>(a, s_pre, s_off, item);
  load_group(cur, 0, wv[0], sc[0]);
  store_act(0);
  __syncthreads();
  int aset = 0;  // ring half holding the current group's activations

  while (true) {
    const int ngr = (cur.nch + kU - 1) / kU;
    const int next_item = item + gx;
    const bool has_next = next_item < end;  // uniform over the workgroup
    Item nxt = cur;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};

    auto chunk = [&](const uint4 (&w)[kWv], float scale, const uint16_t* sa) __attribute__((always_inline)) {
      bf16x8 b[4], av[4];
      const uint16_t* ap = sa + rr * kALd + 32 * q;
#pragma unroll
      for (int j = 0; j < 4; ++j) av[j] = *reinterpret_cast<const bf16x8*>(ap + 8 * j);
      if (kFp8) {
        b[0] = fp8x8_to_bf16(w[0].x, w[0].y);
        b[1] = fp8x8_to_bf16(w[0].z, w[0].w);
        b[2] = fp8x8_to_bf16(w[1].x, w[1].y);
        b[3] = fp8x8_to_bf16(w[1].z, w[1].w);
        f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[j], b[j], t, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(t[i], scale, acc[i]);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = as_bf16x8(w[j]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[j], b[j], acc, 0, 0, 0);
      }
    };
    // group g from register slot GS: first request the following group (or
    // the next item's first group) into the other slot, then multiply, then
    // park the requested activations in the other ring half
    auto group = [&](int g, auto gs_c) __attribute__((always_inline)) {
      constexpr int GS = decltype(gs_c)::value;
      // one unconditional request (a branch around the loads would make the
      // waits after it drain them): the next group of this item, else the
      // next item's first group, else this group again (unused)
      const bool in_item = g + 1 < ngr;
      if (!in_item && has_next) nxt = setup_item<kFp8, kMode>(a, s_pre, s_off, next_item);
      const bool req = in_item || has_next;
      // activations first, then each chunk's weights just before a chunk of
      // this group is multiplied (requests spread between the MFMAs)
      const Item& src = in_item ? cur : nxt;
      const int gl = in_item ? g + 1 : (has_next ? 0 : g);
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int c = min(gl * kU + u, src.nch - 1);
        const uint4 v = *reinterpret_cast<const uint4*>(src.aptr + (size_t)c * kST_KC);
        pa[u] = src.aval ? v : make_uint4(0, 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        {
          const int c = min(gl * kU + u, src.nch - 1);
#pragma unroll
          for (int j = 0; j < kWv; ++j)
            wv[GS ^ 1][u][j] = *reinterpret_cast<const uint4*>(src.wptr + (size_t)c * kST_KC * welt + 16 * j);
          sc[GS ^ 1][u] = kFp8 ? src.sptr[c] : 1.0f;
        }
        if (g * kU + u < cur.nch) chunk(wv[GS][u], sc[GS][u], &s_act[(aset * kU + u) * kASlot]);
      }
      if (req) store_act(aset ^ 1);
      __syncthreads();
      aset ^= 1;
    };
    int g = 0;
    for (; g + 1 < ngr; g += 2) {
      group(g, std::integral_constant<int, 0>{});
      group(g + 1, std::integral_constant<int, 1>{});
    }
    if (g < ngr) {
      group(g, std::integral_constant<int, 0>{});
      // the next item's first group landed in register slot 1: move it to slot 0
#pragma unroll
      for (int u = 0; u < kU; ++u) {
#pragma unroll
        for (int j = 0; j < kWv; ++j) wv[0][u][j] = wv[1][u][j];
        sc[0][u] = sc[1][u];
      }
    }

    // epilogue: element i of lane l is token row 4*(l/16)+i, weight row l%16
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * q + i;
      const float v = acc[i];
      if (kMode == 0) {
        const float up = __shfl_xor(v, 8, kWave);
        if (rr < 8 && m < cur.nrows) cur.out[(size_t)m * cur.ldo + rr] = f32_to_bf16(silu_fast(v) * up);
      } else if (m < cur.nrows) {
        const float gv = cur.gate ? cur.gate[m] : 1.0f;
        cur.out[(size_t)m * cur.ldo + rr] = f32_to_bf16(gv * v);
      }
    }
    if (!has_next) break;
    item = next_item;
    cur = nxt;
    ++done;
    set_priority();
  }
}

// Workgroups of one kernel that fit on a CU at once (registers and LDS
// decide: the e4m3 kernels fit three, the bf16 ones two); the grid is that
// many per CU, capped at the item count and rounded down to a multiple of
// the XCD count, so every workgroup is resident from the start and none
// picks up its first item late.
template <bool kFp8, int kMode>
static int resident_per_cu() {
  static int n = 0;  // the same on every gfx950 device; a racing first call computes the same value
  if (n == 0) {
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, stream_gemm_kernel<kFp8, kMode>, 256, 0) != hipSuccess ||
        v < 1)
      v = 1;
    n = v;
  }
  return n;
}

template <bool kFp8, int kMode>
static hipError_t launch_stream(const ExpertGemmArgs& a, int max_items, int num_cus, hipStream_t s) {
  int blocks = std::min(max_items, resident_per_cu<kFp8, kMode>() * num_cus);
  if (blocks > kXcds) blocks -= blocks % kXcds;  // whole rounds of XCDs: one item stretch per XCD
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((stream_gemm_kernel<kFp8, kMode>), dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_stream_gateup(const ExpertGemmArgs& a, int fp8, int max_items, int num_cus, hipStream_t s) {
  return fp8 ? launch_stream<true, 0>(a, max_items, num_cus, s) : launch_stream<false, 0>(a, max_items, num_cus, s);
}

hipError_t launch_stream_down(const ExpertGemmArgs& a, int fp8, int max_items, int num_cus, hipStream_t s) {
  return fp8 ? launch_stream<true, 1>(a, max_items, num_cus, s) : launch_stream<false, 1>(a, max_items, num_cus, s);
}

MOE_DEBUG_READER(debug_read_stream)

}  // namespace moe
