// Router: fp32 logits (fp32 MFMA, or bf16 MFMA on exact bf16x3 weight splits
// for bf16 activations), then per-token scoring and group-limited top-K
// selection in wavefront registers.
//
// Follows the MoEGate forward of the DeepSeek-V2 walkthrough page (fp32 linear
// map, softmax, greedy or group-limited greedy top-K) and the selection-only
// bias of the DeepSeek-V3 basics page (section 1.2): the bias shifts the scores
// used to choose groups and experts; gates come from the unbiased scores.
#include <type_traits>

#include "moe_internal.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// logits[t][e] = sum_d x[t][d] * gate_w[e][d], fp32 accumulation.
// Tile: 64 tokens x 64 experts per workgroup, 4 waves of 16 tokens x 64 experts.
// v_mfma_f32_16x16x4_f32: lane l supplies A[row l%16][k l/16] and
// B[k l/16][col l%16]. Each lane reads 4 consecutive k from LDS and feeds them
// to 4 successive MFMAs (a consistent permutation of k in A and B leaves the
// dot products unchanged).
// ---------------------------------------------------------------------------
// For few tokens the reduction over D is split across blockIdx.z (kc columns
// each); every split writes its own partial logits plane, and the selection
// kernel adds the planes in a fixed order, so the result does not depend on
// scheduling.
template <bool kBf16X>
__global__ __launch_bounds__(256) void router_logits_kernel(const void* __restrict__ xv,
                                                            const float* __restrict__ w,
                                                            float* __restrict__ logits, int T,
                                                            int D, int E, int kc) {
  constexpr int BT = 64, BE = 64, BK = 32, LD = BK + 4;
  __shared__ __attribute__((aligned(16))) float sA[BT * LD];
  __shared__ __attribute__((aligned(16))) float sB[BE * LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * BT, e0 = blockIdx.y * BE;
  const int kbeg = blockIdx.z * kc, kend = min(D, kbeg + kc);
  logits += (size_t)blockIdx.z * T * E;

  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int lr = tid >> 2, lc = (tid & 3) * 8;  // loader: row, 8 columns
  const int rr = lane & 15, q = lane >> 4;
  const int lt = t0 + lr, le = e0 + lr;  // this thread's loader token and expert
  // The loads of kPre K steps are issued together, then the steps are
  // multiplied one after another: a split of a few steps (the small-batch
  // case) waits for memory once, not once per step.
  constexpr int kPre = 4;
  for (int kb = kbeg; kb < kend; kb += kPre * BK) {
    uint4 ra[kPre][2], rb[kPre][2];  // raw x (bf16: ra[u][0] only) and gate_w pieces
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
      const int k0 = kb + u * BK;
      ra[u][0] = ra[u][1] = rb[u][0] = rb[u][1] = make_uint4(0, 0, 0, 0);
      if (k0 < kend) {
        if (lt < T) {
          if (kBf16X) {
            ra[u][0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(xv) + (size_t)lt * D + k0 + lc);
          } else {
            const uint4* src = reinterpret_cast<const uint4*>(static_cast<const float*>(xv) + (size_t)lt * D + k0 + lc);
            ra[u][0] = src[0];
            ra[u][1] = src[1];
          }
        }
        if (le < E) {
          const uint4* src = reinterpret_cast<const uint4*>(w + (size_t)le * D + k0 + lc);
          rb[u][0] = src[0];
          rb[u][1] = src[1];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
      if (kb + u * BK >= kend) break;  // uniform over the workgroup
      float va[8];
      if (kBf16X) {
        const uint32_t p[4] = {ra[u][0].x, ra[u][0].y, ra[u][0].z, ra[u][0].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          va[2 * i] = __uint_as_float(p[i] << 16);
          va[2 * i + 1] = __uint_as_float(p[i] & 0xFFFF0000u);
        }
      } else {
        const uint32_t p[8] = {ra[u][0].x, ra[u][0].y, ra[u][0].z, ra[u][0].w,
                               ra[u][1].x, ra[u][1].y, ra[u][1].z, ra[u][1].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) va[i] = __uint_as_float(p[i]);
      }
      float4* da = reinterpret_cast<float4*>(&sA[lr * LD + lc]);
      da[0] = make_float4(va[0], va[1], va[2], va[3]);
      da[1] = make_float4(va[4], va[5], va[6], va[7]);
      uint4* db = reinterpret_cast<uint4*>(&sB[lr * LD + lc]);
      db[0] = rb[u][0];
      db[1] = rb[u][1];
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < BK; kk += 16) {
        const float4 a = *reinterpret_cast<const float4*>(&sA[(16 * wave + rr) * LD + kk + 4 * q]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float4 b = *reinterpret_cast<const float4*>(&sB[(16 * j + rr) * LD + kk + 4 * q]);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, acc[j], 0, 0, 0);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, acc[j], 0, 0, 0);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, acc[j], 0, 0, 0);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, acc[j], 0, 0, 0);
        }
      }
      __syncthreads();
    }
  }
  // D layout of the 16x16 MFMA: element i of lane l is row 4*(l/16)+i, column l%16
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = e0 + 16 * j + rr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 16 * wave + 4 * q + i;
      if (t < T && e < E) logits[(size_t)t * E + e] = acc[j][i];
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 activations: the same fp32 logits on bf16 MFMA.
// Each fp32 gate weight is split exactly into three bf16 terms,
// w = hi + mid + lo: hi is w with its significand cut to 8 bits, mid the
// remainder cut likewise, lo what is left (at most 8 significant bits, so
// exactly a bf16). A product of two bf16 values is exact in fp32, so
// x.w = x.hi + x.mid + x.lo is an fp32-accumulated dot product of exact
// products, on the bf16 matrix cores (3x the work, 16x the fp32 MFMA rate).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void split_gate_w_kernel(const float* __restrict__ w,
                                                           uint16_t* __restrict__ out, size_t n4) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;  // four weights per thread
  if (i >= n4) return;
  const float4 v = reinterpret_cast<const float4*>(w)[i];
  const float f[4] = {v.x, v.y, v.z, v.w};
  uint32_t h[4], m[4], l[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t hb = __float_as_uint(f[j]) & 0xFFFF0000u;
    const float r = f[j] - __uint_as_float(hb);  // exact
    const uint32_t mb = __float_as_uint(r) & 0xFFFF0000u;
    const float q = r - __uint_as_float(mb);     // exact, at most 8 significant bits
    h[j] = hb >> 16;
    m[j] = mb >> 16;
    l[j] = __float_as_uint(q) >> 16;
  }
  const size_t n = n4 * 4;
  uint2* o = reinterpret_cast<uint2*>(out);
  o[i] = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
  o[n / 4 + i] = make_uint2(m[0] | (m[1] << 16), m[2] | (m[3] << 16));
  o[n / 2 + i] = make_uint2(l[0] | (l[1] << 16), l[2] | (l[3] << 16));
}

// Tile: 128 tokens x 128 experts per workgroup, K step 64, LDS double-buffered.
// Wave w owns experts 32w..32w+31 of the tile for all 128 tokens (4 row blocks
// of v_mfma_f32_32x32x16_bf16), so each activation fragment read from LDS feeds
// the three weight planes. Lane l supplies row l%32 and k 8*(l/32)..+7 of each
// 16-wide K slice; output element i of lane l is row 8*(i/4)+4*(l/32)+i%4,
// column l%32. blockIdx.y selects a K split (own logits plane, as above).
constexpr int kX3_BT = 128, kX3_BE = 128, kX3_BK = 64, kX3_LD = kX3_BK + 8;

__global__ __launch_bounds__(256) void router_logits_x3_kernel(const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ wsplit,
                                                               float* __restrict__ logits, int T, int D,
                                                               int E, int kc, int n_et, int n_tiles) {
  constexpr int kTile = kX3_BT * kX3_LD;
  __shared__ __attribute__((aligned(16))) uint16_t sm[2][4][kTile];  // [buffer][x, hi, mid, lo]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x;
  // blocks b and b+8 run on the same XCD; give them the two expert tiles of one token tile
  const int pos = (b / 16) * 16 + (b % 8) * 2 + (b / 8) % 2;
  if (pos >= n_tiles) return;
  const int t0 = (pos / n_et) * kX3_BT, e0 = (pos % n_et) * kX3_BE;
  const int kbeg = blockIdx.y * kc, kend = min(D, kbeg + kc);
  const int nsteps = (kend - kbeg) / kX3_BK;
  logits += (size_t)blockIdx.y * T * E;

  // loader: row lr + 32*i, 8 columns at lc (4 rows of x and of each plane per thread)
  const int lr = tid >> 3, lc = (tid & 7) * 8;
  const uint16_t* gx = x + (size_t)min(t0 + lr, T - 1) * D + lc;
  const uint16_t* gw = wsplit + (size_t)min(e0 + lr, E - 1) * D + lc;
  size_t ox[4], ow[4];  // element offsets of the thread's rows (clamped into the operands)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ox[i] = (size_t)(min(t0 + lr + 32 * i, T - 1) - min(t0 + lr, T - 1)) * D;
    ow[i] = (size_t)(min(e0 + lr + 32 * i, E - 1) - min(e0 + lr, E - 1)) * D;
  }
  const size_t plane = (size_t)E * D;
  // Operands two K steps ahead through two register slots (slot k & 1 holds
  // step k; one wave per SIMD, so the accumulators can live in AGPRs and the
  // registers hold both slots); a step's 16 requests are spread over its
  // four substeps, between the MFMAs, and the fragments are double-buffered.
  typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;  // a value type: no aggregate copies
  u32x4 px[2][4], pw[2][12];
  auto store_tile = [&](int bf, int s) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(&sm[bf][0][(lr + 32 * i) * kX3_LD + lc]) = px[s][i];
#pragma unroll
    for (int j = 0; j < 12; ++j)
      *reinterpret_cast<u32x4*>(&sm[bf][1 + (j >> 2)][(lr + 32 * (j & 3)) * kX3_LD + lc]) = pw[s][j];
  };

  f32x16 acc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[m][i] = 0.f;

  const int fr = lane & 31, fk = 8 * (lane >> 5);
  bf16x8 bw[2][3], ax[2][4];
  auto read_frags = [&](int buf, int ks, int fs) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < 3; ++p)
      bw[fs][p] = *reinterpret_cast<const bf16x8*>(&sm[buf][1 + p][(32 * wave + fr) * kX3_LD + 16 * ks + fk]);
#pragma unroll
    for (int m = 0; m < 4; ++m)
      ax[fs][m] = *reinterpret_cast<const bf16x8*>(&sm[buf][0][(32 * m + fr) * kX3_LD + 16 * ks + fk]);
  };
  if (nsteps > 0) {
    const int k1 = kbeg + min(1, nsteps - 1) * kX3_BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) px[0][i] = *reinterpret_cast<const u32x4*>(gx + ox[i] + kbeg);
#pragma unroll
    for (int j = 0; j < 12; ++j) pw[0][j] = *reinterpret_cast<const u32x4*>(gw + (j >> 2) * plane + ow[j & 3] + kbeg);
#pragma unroll
    for (int i = 0; i < 4; ++i) px[1][i] = *reinterpret_cast<const u32x4*>(gx + ox[i] + k1);
#pragma unroll
    for (int j = 0; j < 12; ++j) pw[1][j] = *reinterpret_cast<const u32x4*>(gw + (j >> 2) * plane + ow[j & 3] + k1);
    store_tile(0, 0);
  }
  __syncthreads();
  if (nsteps > 0) read_frags(0, 0, 0);
  // one 16-wide substep: its share of the requests for step st + 2 (x rows in
  // substep 0, a third of the weight planes in each of 1 - 3), the next
  // substep's fragments, the MFMAs (indices are compile-time constants
  // throughout, so the operand slots stay in registers)
  auto substep = [&](auto ks_c, auto s_c, int buf, int kn) __attribute__((always_inline)) {
    constexpr int KS = decltype(ks_c)::value, S = decltype(s_c)::value;
    if constexpr (KS == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) px[S][i] = *reinterpret_cast<const u32x4*>(gx + ox[i] + kn);
    } else {
#pragma unroll
      for (int j = 4 * (KS - 1); j < 4 * KS; ++j)
        pw[S][j] = *reinterpret_cast<const u32x4*>(gw + (j >> 2) * plane + ow[j & 3] + kn);
    }
    if constexpr (KS < 3) read_frags(buf, KS + 1, (KS + 1) & 1);
#pragma unroll
    for (int p = 2; p >= 0; --p)  // smallest terms first
#pragma unroll
      for (int m = 0; m < 4; ++m)
        acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ax[KS & 1][m], bw[KS & 1][p], acc[m], 0, 0, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      if constexpr (KS < 3) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto step = [&](int st, auto s_c) __attribute__((always_inline)) {
    constexpr int S = decltype(s_c)::value;  // = st & 1: slot of step st, refilled with step st + 2
    const int buf = st & 1;
    // branch-free: the last steps reload the last K slice and write the idle buffer
    const int kn = kbeg + min(st + 2, nsteps - 1) * kX3_BK;
    substep(std::integral_constant<int, 0>{}, s_c, buf, kn);
    substep(std::integral_constant<int, 1>{}, s_c, buf, kn);
    substep(std::integral_constant<int, 2>{}, s_c, buf, kn);
    substep(std::integral_constant<int, 3>{}, s_c, buf, kn);
    store_tile(buf ^ 1, S ^ 1);
    __syncthreads();
    read_frags(buf ^ 1, 0, 0);
  };
  int st = 0;
  for (; st + 1 < nsteps; st += 2) {
    step(st, std::integral_constant<int, 0>{});
    step(st + 1, std::integral_constant<int, 1>{});
  }
  if (st < nsteps) step(st, std::integral_constant<int, 0>{});
  const int e = e0 + 32 * wave + fr;
  if (e < E) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = t0 + 32 * m + 8 * (i / 4) + 4 * (lane >> 5) + i % 4;
        if (t < T) logits[(size_t)t * E + e] = acc[m][i];
      }
  }
}

// ---------------------------------------------------------------------------
// Per-token scoring and selection; one wave per token, expert e = lane + 64*j.
// ---------------------------------------------------------------------------
// kVPL values per lane: experts lane, lane+64, ... (E <= 64*kVPL)
// Token t's selection by one wave: `lin` holds its E logits (global memory
// or LDS); its scores replace its logits in the global row `lrow` when their
// column sums are wanted.
template <int kVPL>
__device__ __forceinline__ void select_token(const RouterArgs& a, int t, const float* lin, float* lrow, int lane) {
  const int E = a.E;
  float s[kVPL], z[kVPL];
  float lmax = -INFINITY;
#pragma unroll
  for (int j = 0; j < kVPL; ++j) {
    const int e = lane + kWave * j;
    s[j] = (e < E) ? lin[e] : -INFINITY;
    lmax = fmaxf(lmax, s[j]);
  }
  if (a.score_fn == MOE_SCORE_SOFTMAX) {
    lmax = wave_max_f32(lmax);
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < kVPL; ++j) {
      const int e = lane + kWave * j;
      s[j] = (e < E) ? expf(s[j] - lmax) : 0.f;
      sum += s[j];
    }
    sum = wave_sum_f32(sum);
    const float inv = 1.0f / sum;
#pragma unroll
    for (int j = 0; j < kVPL; ++j) s[j] *= inv;
  } else {
#pragma unroll
    for (int j = 0; j < kVPL; ++j) s[j] = 1.0f / (1.0f + expf(-s[j]));
  }
#pragma unroll
  for (int j = 0; j < kVPL; ++j) {
    const int e = lane + kWave * j;
    z[j] = s[j] + ((a.bias != nullptr && e < E) ? a.bias[e] : 0.f);
  }
  // the scores replace the token's logits when their column sums are wanted
  if (a.score_sum != nullptr) {
#pragma unroll
    for (int j = 0; j < kVPL; ++j)
      if (lane + kWave * j < E) lrow[lane + kWave * j] = s[j];
  }

  // allowed[j]: expert lane+64j may be chosen
  uint32_t allowed = 0;
#pragma unroll
  for (int j = 0; j < kVPL; ++j)
    if (lane + kWave * j < E) allowed |= 1u << j;

  if (a.G > 1) {
    const int gs = E / a.G;
    int grp[kVPL];  // group of expert lane + 64j (G for lanes past E)
#pragma unroll
    for (int j = 0; j < kVPL; ++j) {
      const int e = lane + kWave * j;
      grp[j] = (e < E) ? e / gs : a.G;
    }
    // group maxima: lane g ends up holding max z over group g
    float gmax = -INFINITY;
    for (int g = 0; g < a.G; ++g) {
      float m = -INFINITY;
#pragma unroll
      for (int j = 0; j < kVPL; ++j)
        if (grp[j] == g) m = fmaxf(m, z[j]);
      m = wave_max_f32(m);
      if (lane == g) gmax = m;
    }
    // keep the kg best groups (ties: lower group index)
    uint64_t kept = 0;
    uint64_t key = (lane < a.G) ? (((uint64_t)ordered_key(gmax) << 32) | (uint32_t)(~lane)) : 0;
    for (int r = 0; r < a.kg; ++r) {
      const uint64_t best = wave_max_u64(key);
      const int g = (int)(~(uint32_t)best) & (kMaxGroups - 1);
      kept |= 1ull << g;
      if (lane == g) key = 0;
    }
#pragma unroll
    for (int j = 0; j < kVPL; ++j)
      if (grp[j] < a.G && !((kept >> grp[j]) & 1ull)) allowed &= ~(1u << j);
  }

  int my_e = -1;
  float my_s = 0.f, sum_sel = 0.f;
  for (int k = 0; k < a.K; ++k) {
    uint64_t key = 0;
#pragma unroll
    for (int j = 0; j < kVPL; ++j) {
      if ((allowed >> j) & 1u) {
        const int e = lane + kWave * j;
        const uint64_t kk = ((uint64_t)ordered_key(z[j]) << 32) | (uint32_t)(~e);
        key = kk > key ? kk : key;
      }
    }
    const uint64_t best = wave_max_u64(key);
    int e = (int)(~(uint32_t)best);
    e = (e < 0 || e >= E) ? 0 : e;  // unreachable: K <= candidate experts
    const int jw = e >> 6;
    float mine = 0.f;
#pragma unroll
    for (int j = 0; j < kVPL; ++j)
      if (j == jw) mine = s[j];
    const float se = __uint_as_float(lane_u32(__float_as_uint(mine), e & 63));
    if ((e & 63) == lane) allowed &= ~(1u << jw);
    sum_sel += se;
    if (lane == k) { my_e = e; my_s = se; }
  }
  if (lane < a.K) {
    float g = my_s;
    if (a.norm) g = g / sum_sel;
    g *= a.rsf;
    a.idx[(size_t)t * a.K + lane] = my_e;
    a.gate[(size_t)t * a.K + lane] = g;
  }
}

template <int kVPL>
__global__ __launch_bounds__(256) void router_select_kernel(RouterArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= a.T) return;
  float* lrow = a.logits + (size_t)t * a.E;
  select_token<kVPL>(a, t, lrow, lrow, lane);
}

// Several partial-logit planes: the token's planes are added in plane order
// (plane 0, then 1, 2, ...; the loads of 32 planes are issued at a time),
// the sums go to LDS and to plane 0, and one wave selects from LDS.
// kTPW = 1 (at most one token per CU): one token per workgroup, its E sums
// spread over the 256 threads, wave 0 selects. kTPW = 4: a token per wave,
// lane l adds the planes of experts l, l+64, ... and the wave selects; each
// lane reads back only the sums it wrote, so no barrier is needed.
template <int kVPL, int kTPW>
__global__ __launch_bounds__(256) void router_reduce_select_kernel(RouterArgs a) {
  __shared__ float sl[kTPW][kVPL * kWave];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = (kTPW == 1) ? (int)blockIdx.x : (int)blockIdx.x * 4 + wave;
  if (t >= a.T) return;  // kTPW = 4 only: whole waves
  const size_t n = (size_t)a.T * a.E;
  float* lrow = a.logits + (size_t)t * a.E;
  const int e_first = (kTPW == 1) ? (int)threadIdx.x : lane;
  const int e_step = (kTPW == 1) ? 256 : kWave;
  float* srow = sl[kTPW == 1 ? 0 : wave];
  for (int e = e_first; e < a.E; e += e_step) {
    float v = lrow[e];
    for (int sp = 1; sp < a.splits; sp += 32) {
      float tv[32];
#pragma unroll
      for (int u = 0; u < 32; ++u) tv[u] = (sp + u < a.splits) ? lrow[(size_t)(sp + u) * n + e] : 0.f;
#pragma unroll
      for (int u = 0; u < 32; ++u)
        if (sp + u < a.splits) v += tv[u];
    }
    srow[e] = v;
    if (a.score_sum == nullptr) lrow[e] = v;  // else the scores go there
  }
  if (kTPW == 1) {
    __syncthreads();
    if (wave != 0) return;
  }
  select_token<kVPL>(a, t, srow, lrow, lane);
}

// Column sums of the scores (the importance statistic of the load-balance
// code in the DeepSeekMoE + MLA notes, page 3): part[c][e] = sum of s[t][e]
// over the kScoreChunk tokens of chunk c, in token order (each of the four
// waves sums a quarter of the chunk, the quarters are added in order); then
// score_sum[e] = sum over the chunks in order, in double.
constexpr int kScoreChunk = 256;

__global__ __launch_bounds__(256) void score_part_kernel(const float* __restrict__ scores, int T, int E,
                                                         float* __restrict__ part) {
  __shared__ float q[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  const int t0 = blockIdx.y * kScoreChunk + wave * (kScoreChunk / 4);
  const int t1 = min(T, t0 + kScoreChunk / 4);
  float acc = 0.f;
  if (e < E)
    for (int t = t0; t < t1; ++t) acc += scores[(size_t)t * E + e];
  q[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && e < E) part[(size_t)blockIdx.y * E + e] = ((q[0][lane] + q[1][lane]) + q[2][lane]) + q[3][lane];
}

__global__ __launch_bounds__(512) void score_sum_kernel(const float* __restrict__ part, int chunks, int E,
                                                        float* __restrict__ score_sum) {
  const int e = threadIdx.x;
  if (e >= E) return;
  double acc = 0.0;
  for (int c = 0; c < chunks; ++c) acc += (double)part[(size_t)c * E + e];
  score_sum[e] = (float)acc;
}

int score_part_rows(int T) { return (T + kScoreChunk - 1) / kScoreChunk; }

// Width (a multiple of 32) of each K split of the fp32 kernel: about one
// workgroup per CU. kc >= D / sp, so there are at most sp planes, and
// sp <= ceil(num_cus / tiles) <= 64 * num_cus / T + 1 (tiles >= T / 64).
static int router_kc(int T, int D, int E, int num_cus) {
  const int tiles = ((T + 63) / 64) * ((E + 63) / 64);
  int sp = (num_cus + tiles - 1) / tiles;
  sp = sp < 1 ? 1 : (sp > D / 32 ? D / 32 : sp);
  return ((D + sp - 1) / sp + 31) / 32 * 32;
}

int router_splits(int T, int D, int E, int num_cus) {
  const int kc = router_kc(T, D, E, num_cus);
  return (D + kc - 1) / kc;
}

// Width (a multiple of kX3_BK) of each K split of the bf16x3 kernel: about
// one workgroup per CU, at most sp <= 32 * num_cus / T + 1 planes.
static int router_x3_kc(int T, int D, int E, int num_cus) {
  const int tiles = ((T + kX3_BT - 1) / kX3_BT) * ((E + kX3_BE - 1) / kX3_BE);
  int sp = (num_cus + tiles - 1) / tiles;
  const int cap = 32 * num_cus / T + 1;
  sp = sp > cap ? cap : sp;
  sp = sp > D / kX3_BK ? D / kX3_BK : sp;
  sp = sp < 1 ? 1 : sp;
  return ((D + sp - 1) / sp + kX3_BK - 1) / kX3_BK * kX3_BK;
}

hipError_t launch_router(const RouterArgs& a0, hipStream_t s) {
  RouterArgs a = a0;
  hipError_t err;
  if (a.act_bf16 && a.w_split && a.T >= kRouterX3MinTokens) {
    const int kc = router_x3_kc(a.T, a.D, a.E, a.num_cus);
    a.splits = (a.D + kc - 1) / kc;
    if ((size_t)a.splits * a.T > a.logit_rows) return hipErrorInvalidValue;
    const size_t n4 = (size_t)a.E * a.D / 4;
    hipLaunchKernelGGL(split_gate_w_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, a.gate_w,
                       a.w_split, n4);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const int n_et = (a.E + kX3_BE - 1) / kX3_BE;
    const int n_tiles = ((a.T + kX3_BT - 1) / kX3_BT) * n_et;
    dim3 g((n_tiles + 15) / 16 * 16, a.splits);
    hipLaunchKernelGGL(router_logits_x3_kernel, g, dim3(256), 0, s, static_cast<const uint16_t*>(a.x),
                       a.w_split, a.logits, a.T, a.D, a.E, kc, n_et, n_tiles);
  } else {
    const int kc = router_kc(a.T, a.D, a.E, a.num_cus);
    a.splits = (a.D + kc - 1) / kc;
    if ((size_t)a.splits * a.T > a.logit_rows) return hipErrorInvalidValue;
    dim3 g1((a.T + 63) / 64, (a.E + 63) / 64, a.splits);
    if (a.act_bf16)
      hipLaunchKernelGGL(router_logits_kernel<true>, g1, dim3(256), 0, s, a.x, a.gate_w, a.logits,
                         a.T, a.D, a.E, kc);
    else
      hipLaunchKernelGGL(router_logits_kernel<false>, g1, dim3(256), 0, s, a.x, a.gate_w, a.logits,
                         a.T, a.D, a.E, kc);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (a.splits > 1 && a.T <= a.num_cus) {  // add the planes and select: one token per workgroup
    const dim3 g((unsigned)a.T);
    if (a.E <= 2 * kWave)
      hipLaunchKernelGGL((router_reduce_select_kernel<2, 1>), g, dim3(256), 0, s, a);
    else if (a.E <= 4 * kWave)
      hipLaunchKernelGGL((router_reduce_select_kernel<4, 1>), g, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((router_reduce_select_kernel<kMaxExperts / kWave, 1>), g, dim3(256), 0, s, a);
  } else if (a.splits > 1) {  // ... one token per wave
    const dim3 g((unsigned)((a.T + 3) / 4));
    if (a.E <= 2 * kWave)
      hipLaunchKernelGGL((router_reduce_select_kernel<2, 4>), g, dim3(256), 0, s, a);
    else if (a.E <= 4 * kWave)
      hipLaunchKernelGGL((router_reduce_select_kernel<4, 4>), g, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((router_reduce_select_kernel<kMaxExperts / kWave, 4>), g, dim3(256), 0, s, a);
  } else {
    const dim3 g((unsigned)((a.T + 3) / 4));
    if (a.E <= 2 * kWave)
      hipLaunchKernelGGL(router_select_kernel<2>, g, dim3(256), 0, s, a);
    else if (a.E <= 4 * kWave)
      hipLaunchKernelGGL(router_select_kernel<4>, g, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(router_select_kernel<kMaxExperts / kWave>, g, dim3(256), 0, s, a);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (a.score_sum != nullptr) {
    const int chunks = score_part_rows(a.T);
    hipLaunchKernelGGL(score_part_kernel, dim3((a.E + 63) / 64, chunks), dim3(256), 0, s, a.logits, a.T, a.E,
                       a.score_part);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(score_sum_kernel, dim3(1), dim3(512), 0, s, a.score_part, chunks, a.E, a.score_sum);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return a.hist ? launch_histogram(a.idx, a.counts, a.T * a.K, a.E, s) : hipSuccess;
}

}  // namespace moe
