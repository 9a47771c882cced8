// Grouped bf16 MFMA GEMMs of the routed experts and the shared expert
// (prefill-sized token counts).
//
// One launch covers every problem: routed expert e (its rows are the
// expert-contiguous rows offsets[e] .. offsets[e+1]-1 built by the dispatch)
// and the shared expert (all T tokens, gate 1). Work items are 256-row x
// N-column output tiles; the dispatch writes their per-problem prefix, and a
// block finds its problem by binary search, so the host never learns the
// per-expert row counts.
//
// Gate/up GEMM (fine-grained SwiGLU expert, DeepSeek-V2 walkthrough page MoE
// code; architecture article section 3.3): a tile loads 64 W_gate rows and the
// matching 64 W_up rows, so the SwiGLU h = SiLU(x W_gate^T) * (x W_up^T) is
// formed in registers and only h (bf16) is written. Token rows are gathered
// from x through the dispatch's row -> token map.
// Down GEMM: Y[row] = g_row * (h[row] W_down^T), bf16, 128 output columns per
// tile; the combine sums the K rows of each token in a fixed order.
//
// Tile 256 x 128 (gate/up: 256 rows x (64 gate + 64 up) columns), K step 64,
// 4 waves as 2 x 2, each wave 128 x 64 on v_mfma_f32_32x32x16_bf16. Global
// tiles are staged through LDS (rows padded to 144 bytes so that the 16-byte
// fragment reads of 16 consecutive rows hit distinct banks); the next K step
// is loaded into registers while the current one is multiplied.
// Blocks are mapped so that consecutive tiles (which share weight columns or
// token rows) land on the same XCD and its L2.
#include "moe_internal.hpp"

namespace moe {

namespace {
constexpr int BM = kGB_BM, BK = kGB_BK, LDSW = BK + 8;
}

template <int kMode>  // 0: gate/up + SwiGLU, 1: down + gate scale
__global__ __launch_bounds__(256) void grouped_gemm_bf16_kernel(ExpertGemmArgs a) {
  constexpr int BN = 128;
  __shared__ __attribute__((aligned(16))) uint16_t sA[BM * LDSW];
  __shared__ __attribute__((aligned(16))) uint16_t sB[BN * LDSW];

  const int total = a.pre[a.E + 1];
  const int chunk = (total + 7) >> 3;
  const int bid = blockIdx.x;
  const int slot = bid >> 3;
  if (slot >= chunk) return;
  const int tile = (bid & 7) * chunk + slot;
  if (tile >= total) return;

  const int p = find_problem(a.pre, a.E, tile);
  const bool routed = p < a.E;
  const int rows = routed ? a.offsets[p + 1] - a.offsets[p] : a.T;
  const int row_base = routed ? a.offsets[p] : 0;
  const int Hp = routed ? a.H : a.Hs;
  const int ntn = (kMode == 0) ? Hp / kG1_BNH : a.D / kG2_BN;
  const int local = tile - a.pre[p];
  const int m0 = (local / ntn) * BM;
  const int nt = local % ntn;
  const int K = (kMode == 0) ? a.D : Hp;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int c8 = tid & 7, r0 = tid >> 3;

  // global source rows of this thread's 8 A chunks and 4 B chunks
  const uint16_t* ap[8];
  bool av[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int m = m0 + r0 + 32 * j;
    av[j] = m < rows;
    const int mm = av[j] ? m : m0;
    if (kMode == 0) {
      const int tok = routed ? a.row_token[row_base + mm] : mm;
      ap[j] = static_cast<const uint16_t*>(a.a) + (size_t)tok * a.D + c8 * 8;
    } else {
      ap[j] = routed ? static_cast<const uint16_t*>(a.a) + (size_t)(row_base + mm) * a.H + c8 * 8
                     : static_cast<const uint16_t*>(a.a_shared) + (size_t)mm * a.Hs + c8 * 8;
    }
  }
  const uint16_t* wbase = routed ? static_cast<const uint16_t*>(a.w) +
                                       (size_t)p * ((kMode == 0) ? 2 * Hp : a.D) * K
                                 : static_cast<const uint16_t*>(a.w_shared);
  const uint16_t* bp[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int b = r0 + 32 * j;
    const int wrow = (kMode == 0) ? (b < 64 ? nt * 64 + b : Hp + nt * 64 + b - 64) : nt * BN + b;
    bp[j] = wbase + (size_t)wrow * K + c8 * 8;
  }

  uint4 ra[8], rb[4];
  auto load = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      ra[j] = av[j] ? *reinterpret_cast<const uint4*>(ap[j] + k0) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) rb[j] = *reinterpret_cast<const uint4*>(bp[j] + k0);
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][c][e] = 0.f;

  // B-tile rows of this wave's two 32-column blocks
  const int bb0 = (kMode == 0) ? 32 * wn : 64 * wn;
  const int bb1 = (kMode == 0) ? 64 + 32 * wn : 64 * wn + 32;
  const int lr = lane & 31, lk = (lane >> 5) * 8;

  load(0);
  for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<uint4*>(&sA[(r0 + 32 * j) * LDSW + c8 * 8]) = ra[j];
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<uint4*>(&sB[(r0 + 32 * j) * LDSW + c8 * 8]) = rb[j];
    __syncthreads();
    if (k0 + BK < K) load(k0 + BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 fa[4], fb[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[i] = *reinterpret_cast<const bf16x8*>(&sA[(wm * 128 + 32 * i + lr) * LDSW + kk + lk]);
      fb[0] = *reinterpret_cast<const bf16x8*>(&sB[(bb0 + lr) * LDSW + kk + lk]);
      fb[1] = *reinterpret_cast<const bf16x8*>(&sB[(bb1 + lr) * LDSW + kk + lk]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          acc[i][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[c], acc[i][c], 0, 0, 0);
    }
    __syncthreads();
  }

  // D layout of the 32x32 MFMA: element e of lane l is row 8*(e/4) + 4*(l/32) + e%4,
  // column l%32.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = m0 + wm * 128 + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      if (m >= rows) continue;
      if (kMode == 0) {
        const float h = silu_fast(acc[i][0][e]) * acc[i][1][e];
        uint16_t* hp = routed ? static_cast<uint16_t*>(a.c) + (size_t)(row_base + m) * a.H
                              : static_cast<uint16_t*>(a.c_shared) + (size_t)m * a.Hs;
        hp[nt * 64 + 32 * wn + lr] = f32_to_bf16(h);
      } else {
        const float g = routed ? a.row_gate[row_base + m] : 1.0f;
        uint16_t* yp = routed ? static_cast<uint16_t*>(a.c) + (size_t)(row_base + m) * a.D
                              : static_cast<uint16_t*>(a.c_shared) + (size_t)m * a.D;
        yp[nt * BN + 64 * wn + lr] = f32_to_bf16(g * acc[i][0][e]);
        yp[nt * BN + 64 * wn + 32 + lr] = f32_to_bf16(g * acc[i][1][e]);
      }
    }
  }
}

hipError_t launch_grouped_gateup_bf16(const ExpertGemmArgs& a, hipStream_t s) {
  const int blocks = ((a.max_items + 7) / 8) * 8;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(grouped_gemm_bf16_kernel<0>, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_grouped_down_bf16(const ExpertGemmArgs& a, hipStream_t s) {
  const int blocks = ((a.max_items + 7) / 8) * 8;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(grouped_gemm_bf16_kernel<1>, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
