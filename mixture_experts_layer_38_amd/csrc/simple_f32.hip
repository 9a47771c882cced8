// fp32 expert FFNs and the combine.
//
// The fp32 layer (fp32 activations and weights) is tiny in every workload it
// serves, so its expert GEMMs are plain per-output dot products in fp32, one
// thread per output element; each row of the expert-contiguous buffer is one
// (token, expert) pair, or one token of the shared expert.
//
// The combine is the gate-weighted sum of the page-1 MoE forward plus the
// shared expert and the residual; it runs for every dtype.
#include "moe_internal.hpp"

namespace moe {

__device__ __forceinline__ float silu_precise(float z) { return z / (1.0f + expf(-z)); }

__global__ __launch_bounds__(64) void gateup_f32_kernel(ExpertGemmArgs a, int TK) {
  const int r = blockIdx.y;
  const bool routed = r < TK;
  const int p = routed ? find_problem(a.offsets, a.E - 1, r) : a.E;
  const int Hp = routed ? a.H : a.Hs;
  const int j = blockIdx.x * 64 + threadIdx.x;
  if (j >= Hp) return;
  const int tok = routed ? a.row_token[r] : r - TK;
  const float* x = static_cast<const float*>(a.a) + (size_t)tok * a.D;
  const float* W = routed ? static_cast<const float*>(a.w) + (size_t)p * 2 * Hp * a.D
                          : static_cast<const float*>(a.w_shared);
  const float* wg = W + (size_t)j * a.D;
  const float* wu = W + (size_t)(Hp + j) * a.D;
  float g = 0.f, u = 0.f;
  for (int d = 0; d < a.D; ++d) {
    g = fmaf(x[d], wg[d], g);
    u = fmaf(x[d], wu[d], u);
  }
  float* h = routed ? static_cast<float*>(a.c) + (size_t)r * Hp
                    : static_cast<float*>(a.c_shared) + (size_t)(r - TK) * Hp;
  h[j] = silu_precise(g) * u;
}

__global__ __launch_bounds__(64) void down_f32_kernel(ExpertGemmArgs a, int TK) {
  const int r = blockIdx.y;
  const bool routed = r < TK;
  const int p = routed ? find_problem(a.offsets, a.E - 1, r) : a.E;
  const int Hp = routed ? a.H : a.Hs;
  const int n = blockIdx.x * 64 + threadIdx.x;
  if (n >= a.D) return;
  const float* h = routed ? static_cast<const float*>(a.a) + (size_t)r * Hp
                          : static_cast<const float*>(a.a_shared) + (size_t)(r - TK) * Hp;
  const float* W = routed ? static_cast<const float*>(a.w) + (size_t)p * a.D * Hp
                          : static_cast<const float*>(a.w_shared);
  const float* wd = W + (size_t)n * Hp;
  float acc = 0.f;
  for (int j = 0; j < Hp; ++j) acc = fmaf(h[j], wd[j], acc);
  if (routed)
    static_cast<float*>(a.c)[(size_t)r * a.D + n] = a.row_gate[r] * acc;
  else
    static_cast<float*>(a.c_shared)[(size_t)(r - TK) * a.D + n] = acc;
}

hipError_t launch_simple_gateup_f32(const ExpertGemmArgs& a, int TK, hipStream_t s) {
  const int rows = TK + (a.Hs > 0 ? a.T : 0);
  if (rows == 0) return hipSuccess;
  const int hmax = a.H > a.Hs ? a.H : a.Hs;
  hipLaunchKernelGGL(gateup_f32_kernel, dim3((hmax + 63) / 64, rows), dim3(64), 0, s, a, TK);
  return hipGetLastError();
}

hipError_t launch_simple_down_f32(const ExpertGemmArgs& a, int TK, hipStream_t s) {
  const int rows = TK + (a.Hs > 0 ? a.T : 0);
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(down_f32_kernel, dim3((a.D + 63) / 64, rows), dim3(64), 0, s, a, TK);
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
  for (int k = 0; k < kMaxTopK; ++k) rows[k] = (k < a.K) ? a.slot_row[(size_t)t * a.K + k] : 0;
  const bool has_shared = a.y_shared != nullptr;
  // a source that is absent reads a valid row instead (never added)
  const void* sbase = has_shared ? a.y_shared : a.y_routed;
  const size_t srow = has_shared ? (size_t)t : (size_t)rows[0];
  for (int d0 = threadIdx.x * 8; d0 < a.D; d0 += blockDim.x * 8) {
    // every load of this step first (the residual, the shared row, up to 8
    // routed rows), then the adds in the fixed order
    const Raw8<kXBf16> xv = load8<kXBf16>(a.x, (size_t)t, a.D, d0);
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
      float4* p = reinterpret_cast<float4*>(static_cast<float*>(a.out) + (size_t)t * a.D + d0);
      p[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      p[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int code = (a.y_bf16 ? 4 : 0) | (a.act_bf16 ? 2 : 0) | (a.out_bf16 ? 1 : 0);
  // threads per token: the 8-column chunks of a row spread evenly over at
  // most 256 threads (D = 7168: 224 threads x 4 chunks)
  const int chunks = (a.D + 7) / 8, iters = (chunks + 255) / 256;
  dim3 g(a.T), b((chunks + iters - 1) / iters);
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

}  // namespace moe
