// fp32 expert FFNs and the combine.
//
// The fp32 layer (fp32 activations and weights): grouped LDS-tiled GEMMs in
// fp32 FMAs, one launch per GEMM over every problem (routed expert e, or the
// shared expert), work items from the dispatch's item prefix like the bf16
// path. A work item is 64 rows (expert-contiguous rows, i.e. (token, expert)
// pairs, or tokens of the shared expert) x 64 weight rows: for gate/up, 32
// W_gate rows and the matching 32 W_up rows, so h = SiLU(gate) * up is formed
// in registers; for down, 64 output columns, times the row's gate. K steps of
// 32 staged through LDS with coalesced loads (consecutive threads read
// consecutive elements of a row), the next step's loads in flight while the
// current one is multiplied; each thread accumulates 4 rows x 4 columns in k
// order.
//
// The combine is the gate-weighted sum of the page-1 MoE forward plus the
// shared expert and the residual; it runs for every dtype.
#include "moe_internal.hpp"

namespace moe {

__device__ __forceinline__ float silu_precise(float z) { return z / (1.0f + expf(-z)); }

namespace {
constexpr int kF32_BK = 32, kF32_LD = kF32_BK + 1;
}

// kMode 0: gate/up + SwiGLU -> h; 1: down x gate -> y
template <int kMode>
__global__ __launch_bounds__(256) void grouped_f32_kernel(ExpertGemmArgs a) {
  __shared__ float sA[kF32_BM * kF32_LD];
  __shared__ float sB[64 * kF32_LD];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int tile = blockIdx.x;
  if (tile >= a.pre[a.E + 1]) return;
  const int p = find_problem(a.pre, a.E, tile);
  const bool routed = p < a.E;
  const int rows = routed ? a.offsets[p + 1] - a.offsets[p] : a.T;
  const int row_base = routed ? a.offsets[p] : 0;
  const int Hp = routed ? a.H : a.Hs;
  const int ncols = kMode == 0 ? (Hp + 31) / 32 : (a.D + 63) / 64;
  const int local = tile - a.pre[p];
  const int m0 = (local / ncols) * kF32_BM, nt = local % ncols;
  const int vrows = min(kF32_BM, rows - m0);
  const int K = kMode == 0 ? a.D : Hp;
  // A rows: gathered token rows of x (gate/up) or this problem's h rows (down)
  const float* arow[8];
  // B rows: W_gate / W_up rows nt*32 + c (gate/up) or W_down rows nt*64 + c (down)
  const float* W = kMode == 0
      ? (routed ? static_cast<const float*>(a.w) + (size_t)p * 2 * Hp * a.D : static_cast<const float*>(a.w_shared))
      : (routed ? static_cast<const float*>(a.w) + (size_t)p * a.D * Hp : static_cast<const float*>(a.w_shared));
  const float* brow[8];
  bool bval[8], aval[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int r = (tid >> 5) + 8 * q;  // row of the 64-row tile this thread stages
    aval[q] = r < vrows;
    const int rr = aval[q] ? m0 + r : m0;
    if (kMode == 0) {
      const int tok = routed ? dcheck(a.row_token[row_base + rr], a.x_rows, kSiteF32Tok) : rr;
      arow[q] = static_cast<const float*>(a.a) + (size_t)tok * a.D;
      const int c = nt * 32 + (r & 31);
      bval[q] = c < Hp;
      brow[q] = W + (size_t)((r < 32 ? 0 : Hp) + (bval[q] ? c : 0)) * a.D;
    } else {
      arow[q] = routed ? static_cast<const float*>(a.a) + (size_t)(row_base + rr) * Hp
                       : static_cast<const float*>(a.a_shared) + (size_t)rr * Hp;
      const int c = nt * 64 + r;
      bval[q] = c < a.D;
      brow[q] = W + (size_t)(bval[q] ? c : 0) * Hp;
    }
  }
  const int kc = tid & 31;  // the thread's element of each staged 32-wide row piece
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  // the next K slice is loaded into registers while the current one is
  // multiplied from LDS
  float va[8], vb[8];
  auto load_slice = [&](int k0) __attribute__((always_inline)) {
    const int k = k0 + kc;
    const bool kin = k < K;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      va[q] = (aval[q] && kin) ? arow[q][k] : 0.f;
      vb[q] = (bval[q] && kin) ? brow[q][k] : 0.f;
    }
  };
  load_slice(0);
  for (int k0 = 0; k0 < K; k0 += kF32_BK) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int r = (tid >> 5) + 8 * q;
      sA[r * kF32_LD + kc] = va[q];
      sB[r * kF32_LD + kc] = vb[q];
    }
    __syncthreads();
    if (k0 + kF32_BK < K) load_slice(k0 + kF32_BK);
#pragma unroll 8
    for (int kk = 0; kk < kF32_BK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = sA[(ty + 16 * i) * kF32_LD + kk];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = sB[(tx + 16 * j) * kF32_LD + kk];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ty + 16 * i;
    if (r >= vrows) continue;
    if (kMode == 0) {
      float* h = routed ? static_cast<float*>(a.c) + (size_t)(row_base + m0 + r) * Hp
                        : static_cast<float*>(a.c_shared) + (size_t)(m0 + r) * Hp;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = nt * 32 + tx + 16 * j;  // columns j (gate) and j + 2 (up) of the tile
        if (c < Hp) h[c] = silu_precise(acc[i][j]) * acc[i][j + 2];
      }
    } else {
      const float g = routed ? a.row_gate[row_base + m0 + r] : 1.0f;
      float* y = routed ? static_cast<float*>(a.c) + (size_t)(row_base + m0 + r) * a.D
                        : static_cast<float*>(a.c_shared) + (size_t)(m0 + r) * a.D;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = nt * 64 + tx + 16 * j;
        if (c < a.D) y[c] = g * acc[i][j];
      }
    }
  }
}

hipError_t launch_simple_gateup_f32(const ExpertGemmArgs& a, int TK, hipStream_t s) {
  (void)TK;
  if (a.max_items <= 0) return hipSuccess;
  hipLaunchKernelGGL(grouped_f32_kernel<0>, dim3(a.max_items), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_simple_down_f32(const ExpertGemmArgs& a, int TK, hipStream_t s) {
  (void)TK;
  if (a.max_items <= 0) return hipSuccess;
  hipLaunchKernelGGL(grouped_f32_kernel<1>, dim3(a.max_items), dim3(256), 0, s, a);
  return hipGetLastError();
}

// out[t] = [x[t]] + S[t] + sum_{k<K} Y[slot_row[t*K+k]], fp32, k in order.
// One workgroup per token, 8 consecutive columns per thread and step.
namespace {
// 8 consecutive values of one row, as loaded (bf16: one 16-byte piece;
// fp32: two)
template <bool kBf16>
struct Raw8 {
  uint4 u[kBf16 ? 1 : 2];
};
template <bool kBf16>
__device__ __forceinline__ Raw8<kBf16> load8(const void* base, size_t row, int D, int d0) {
  Raw8<kBf16> r;
  if (kBf16) {
    r.u[0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + row * D + d0);
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + row * D + d0);
    r.u[0] = p[0];
    r.u[1] = p[1];
  }
  return r;
}
// acc += v, or += -0.0 (which leaves every value, signed zeros included,
// unchanged) when !use: the load was issued regardless, so no wait sits
// behind a branch
template <bool kBf16>
__device__ __forceinline__ void add8(float (&acc)[8], const Raw8<kBf16>& v, bool use) {
  if (kBf16) {
    const uint32_t m = use ? 0xFFFFFFFFu : 0x80008000u, z = use ? 0u : 0x80008000u;
    const uint32_t w[4] = {(v.u[0].x & m) | z, (v.u[0].y & m) | z, (v.u[0].z & m) | z, (v.u[0].w & m) | z};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += __uint_as_float(w[i] << 16);
      acc[2 * i + 1] += __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const uint32_t w[8] = {v.u[0].x, v.u[0].y, v.u[0].z, v.u[0].w, v.u[1].x, v.u[1].y, v.u[1].z, v.u[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += __uint_as_float(use ? w[i] : 0x80000000u);
  }
}
}  // namespace

template <bool kYBf16, bool kXBf16, bool kOutBf16>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int t = blockIdx.x;
  int rows[kMaxTopK];
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k)
    rows[k] = (k < a.K) ? dcheck(a.slot_row[(size_t)t * a.K + k], a.T * a.K, kSiteCombineRow) : 0;
  const bool has_shared = a.y_shared != nullptr;
  // a source that is absent reads a valid row instead (never added)
  const void* sbase = has_shared ? a.y_shared : a.y_routed;
  const size_t srow = has_shared ? (size_t)t : (size_t)rows[0];
  // blockIdx.y: this workgroup's share of the row (several per token when tokens are few)
  for (int d0 = (blockIdx.y * blockDim.x + threadIdx.x) * 8; d0 < a.D; d0 += gridDim.y * blockDim.x * 8) {
    // every load of this step first (the residual if it is added, the shared
    // row, up to 8 routed rows), then the adds in the fixed order
    Raw8<kXBf16> xv{};
    if (a.add_residual) xv = load8<kXBf16>(a.x, (size_t)t, a.D, d0);
    const Raw8<kYBf16> sv = load8<kYBf16>(sbase, srow, a.D, d0);
    Raw8<kYBf16> v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = load8<kYBf16>(a.y_routed, (size_t)rows[k], a.D, d0);
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    if (a.add_residual) add8<kXBf16>(acc, xv, true);
    add8<kYBf16>(acc, sv, has_shared);
#pragma unroll
    for (int k = 0; k < 8; ++k) add8<kYBf16>(acc, v[k], k < a.K);
    if (a.K > 8) {
#pragma unroll
      for (int k = 8; k < kMaxTopK; ++k) v[k - 8] = load8<kYBf16>(a.y_routed, (size_t)rows[k], a.D, d0);
#pragma unroll
      for (int k = 8; k < kMaxTopK; ++k) add8<kYBf16>(acc, v[k - 8], k < a.K);
    }
    if (kOutBf16) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = (uint32_t)f32_to_bf16(acc[2 * i]) | ((uint32_t)f32_to_bf16(acc[2 * i + 1]) << 16);
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + (size_t)t * a.D + d0) =
          make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      // the output is written once and not read back here: streaming stores
      f32x4* p = reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + (size_t)t * a.D + d0);
      __builtin_nontemporal_store(f32x4{acc[0], acc[1], acc[2], acc[3]}, p);
      __builtin_nontemporal_store(f32x4{acc[4], acc[5], acc[6], acc[7]}, p + 1);
    }
  }
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int code = (a.y_bf16 ? 4 : 0) | (a.act_bf16 ? 2 : 0) | (a.out_bf16 ? 1 : 0);
  // threads per token: the 8-column chunks of a row spread evenly over at
  // most 256 threads (D = 7168: 224 threads x 4 chunks); with fewer tokens
  // than CUs, a row is split over several workgroups so that every thread
  // takes one chunk and the row loads of all tokens are in flight at once
  const int chunks = (a.D + 7) / 8, iters = (chunks + 255) / 256;
  const int split = (a.T < 256) ? iters : 1;
  dim3 g(a.T, split), b((chunks + iters - 1) / iters);
  switch (code) {
    case 0: hipLaunchKernelGGL((combine_kernel<false, false, false>), g, b, 0, s, a); break;
    case 1: hipLaunchKernelGGL((combine_kernel<false, false, true>), g, b, 0, s, a); break;
    case 2: hipLaunchKernelGGL((combine_kernel<false, true, false>), g, b, 0, s, a); break;
    case 3: hipLaunchKernelGGL((combine_kernel<false, true, true>), g, b, 0, s, a); break;
    case 4: hipLaunchKernelGGL((combine_kernel<true, false, false>), g, b, 0, s, a); break;
    case 5: hipLaunchKernelGGL((combine_kernel<true, false, true>), g, b, 0, s, a); break;
    case 6: hipLaunchKernelGGL((combine_kernel<true, true, false>), g, b, 0, s, a); break;
    default: hipLaunchKernelGGL((combine_kernel<true, true, true>), g, b, 0, s, a); break;
  }
  return hipGetLastError();
}

MOE_DEBUG_READER(debug_read_f32)

}  // namespace moe
