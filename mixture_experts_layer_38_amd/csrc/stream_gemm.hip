// Weight-streaming expert GEMMs for small token counts (decode), bf16 or fp8
// (OCP e4m3 with one fp32 scale per 128x128 block) weights, bf16 activations.
//
// With a few tokens per expert the layer is bound by reading each touched
// expert's weights once from HBM. Each wave owns one work item -- 16 weight
// rows of one problem (routed expert or the shared expert) over the whole K
// extent, for up to 64 token rows -- and streams those rows straight from HBM
// into MFMA operands without LDS: the weights are used by exactly one wave, and
// the activation rows (at most 64 per item) stay in L2.
//
// v_mfma_f32_16x16x32_bf16: lane l supplies A[token l%16][8 k] and
// B[8 k][weight row l%16] for k-group l/16. Within a 128-wide K chunk, lane
// group q reads the 32 consecutive k at 32q and feeds k 32q+8j..+7 to MFMA j;
// A and B use the same assignment, so each dot product is unchanged.
// fp8 weights are widened to bf16 exactly (every e4m3 value is a bf16 value);
// the 128-wide chunk is accumulated unscaled, then multiplied by its block
// scale and added to the fp32 accumulator.
//
// Gate/up items pair 8 W_gate rows with the matching 8 W_up rows, so the SwiGLU
// epilogue (h = SiLU(gate) * up, DeepSeek-V2 walkthrough page MoE code and the
// SwiGLU expert of the architecture article, section 3.3) needs only a lane
// swap. Down items write g * (h W_down^T) for 16 output columns.
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

template <bool kFp8, int kMode>  // kMode 0: gate/up + SwiGLU, 1: down + gate scale
__global__ __launch_bounds__(256) void stream_gemm_kernel(ExpertGemmArgs a) {
  const int lane = threadIdx.x & 63;
  const int rr = lane & 15, q = lane >> 4;
  const int total = a.pre[a.E + 1];
  const int n_waves = gridDim.x * 4;
  for (int item = blockIdx.x * 4 + (threadIdx.x >> 6); item < total; item += n_waves) {
    const int p = find_problem(a.pre, a.E, item);
    const bool routed = p < a.E;
    const int rows = routed ? a.offsets[p + 1] - a.offsets[p] : a.T;
    const int row_base = routed ? a.offsets[p] : 0;
    const int Hp = routed ? a.H : a.Hs;
    const int ncols = (kMode == 0) ? Hp / kST_N1 : a.D / kST_N2;
    const int local = item - a.pre[p];
    const int m0 = (local / ncols) * kST_BM;
    const int nb = local % ncols;
    const int nrows = min(rows - m0, kST_BM);
    const int K = (kMode == 0) ? a.D : Hp;
    const int wrows = (kMode == 0) ? 2 * Hp : a.D;

    // this lane's weight row
    const int wrow = (kMode == 0) ? (rr < 8 ? nb * kST_N1 + rr : Hp + nb * kST_N1 + rr - 8)
                                  : nb * kST_N2 + rr;
    const size_t welt = kFp8 ? 1 : 2;
    const char* wbase = static_cast<const char*>(routed ? a.w : a.w_shared) +
                        (routed ? (size_t)p * wrows * K * welt : 0);
    const char* wptr = wbase + (size_t)wrow * K * welt + (size_t)32 * q * welt;
    const float* sptr = nullptr;
    if (kFp8) {
      const int kb = K / kST_KC;
      sptr = (routed ? a.w_scale + (size_t)p * (wrows / kST_KC) * kb : a.w_shared_scale) +
             (size_t)(wrow / kST_KC) * kb;
    }
    // activation rows for up to four 16-row blocks
    const uint16_t* aptr[4];
    bool aval[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = m0 + 16 * mb + rr;
      aval[mb] = (16 * mb + rr) < nrows;
      const int mm = aval[mb] ? m : m0;  // in-bounds row for masked lanes
      if (kMode == 0) {
        const int tok = routed ? a.row_token[row_base + mm] : mm;
        aptr[mb] = static_cast<const uint16_t*>(a.a) + (size_t)tok * a.D + 32 * q;
      } else {
        aptr[mb] = routed ? static_cast<const uint16_t*>(a.a) + (size_t)(row_base + mm) * a.H + 32 * q
                          : static_cast<const uint16_t*>(a.a_shared) + (size_t)mm * a.Hs + 32 * q;
      }
    }
    const int nmb = (nrows + 15) >> 4;

    f32x4 acc[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

    constexpr int kWv = kFp8 ? 2 : 4;  // 16-byte weight loads per lane per chunk
    auto chunk = [&](int kc, const uint4* wv) {
      bf16x8 b[4];
      if (kFp8) {
        b[0] = fp8x8_to_bf16(wv[0].x, wv[0].y);
        b[1] = fp8x8_to_bf16(wv[0].z, wv[0].w);
        b[2] = fp8x8_to_bf16(wv[1].x, wv[1].y);
        b[3] = fp8x8_to_bf16(wv[1].z, wv[1].w);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = as_bf16x8(wv[j]);
      }
      const float scale = kFp8 ? sptr[kc / kST_KC] : 1.0f;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        if (mb < nmb) {
          const uint4* ap = reinterpret_cast<const uint4*>(aptr[mb] + kc);
          uint4 av[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) av[j] = aval[mb] ? ap[j] : make_uint4(0, 0, 0, 0);
          if (kFp8) {
            f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j)
              t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[j]), b[j], t, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mb][i] = fmaf(t[i], scale, acc[mb][i]);
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[j]), b[j], acc[mb], 0, 0, 0);
          }
        }
      }
    };
    // four chunks per step: all their weight loads are issued before any use,
    // so each wave keeps 4 chunks of its rows in flight
    constexpr int kU = 4;
    int kc = 0;
    for (; kc + kU * kST_KC <= K; kc += kU * kST_KC) {
      uint4 wv[kU][kWv];
#pragma unroll
      for (int u = 0; u < kU; ++u)
#pragma unroll
        for (int j = 0; j < kWv; ++j)
          wv[u][j] = *reinterpret_cast<const uint4*>(wptr + (size_t)(kc + u * kST_KC) * welt + 16 * j);
#pragma unroll
      for (int u = 0; u < kU; ++u) chunk(kc + u * kST_KC, wv[u]);
    }
    for (; kc < K; kc += kST_KC) {
      uint4 wv[kWv];
#pragma unroll
      for (int j = 0; j < kWv; ++j) wv[j] = *reinterpret_cast<const uint4*>(wptr + (size_t)kc * welt + 16 * j);
      chunk(kc, wv);
    }

    // epilogue: element i of lane l is token row 4*(l/16)+i, weight row l%16
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * mb + 4 * q + i;  // row within this pass
        const float v = acc[mb][i];
        if (kMode == 0) {
          const float up = __shfl_xor(v, 8, kWave);
          if (rr < 8 && m < nrows) {
            const float h = silu_fast(v) * up;
            uint16_t* hp = routed ? static_cast<uint16_t*>(a.c) + (size_t)(row_base + m0 + m) * a.H
                                  : static_cast<uint16_t*>(a.c_shared) + (size_t)(m0 + m) * a.Hs;
            hp[nb * kST_N1 + rr] = f32_to_bf16(h);
          }
        } else if (m < nrows) {
          if (routed) {
            const float g = a.row_gate[row_base + m0 + m];
            static_cast<uint16_t*>(a.c)[(size_t)(row_base + m0 + m) * a.D + nb * kST_N2 + rr] = f32_to_bf16(g * v);
          } else {
            static_cast<uint16_t*>(a.c_shared)[(size_t)(m0 + m) * a.D + nb * kST_N2 + rr] = f32_to_bf16(v);
          }
        }
      }
    }
  }
}

hipError_t launch_stream_gateup(const ExpertGemmArgs& a, int fp8, int n_waves, hipStream_t s) {
  const int blocks = (n_waves + 3) / 4;
  if (fp8)
    hipLaunchKernelGGL((stream_gemm_kernel<true, 0>), dim3(blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((stream_gemm_kernel<false, 0>), dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_stream_down(const ExpertGemmArgs& a, int fp8, int n_waves, hipStream_t s) {
  const int blocks = (n_waves + 3) / 4;
  if (fp8)
    hipLaunchKernelGGL((stream_gemm_kernel<true, 1>), dim3(blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((stream_gemm_kernel<false, 1>), dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
