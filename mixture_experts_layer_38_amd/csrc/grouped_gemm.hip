// Grouped bf16 MFMA GEMMs of the routed experts and the shared expert
// (prefill-sized token counts), with bf16 weights or e4m3 weights (one fp32
// scale per 128x128 block, the block-wise quantisation of the architecture
// article, section 4): e4m3 weights are widened exactly to fp32, multiplied
// by their block scale and rounded to bf16 as they are written to LDS.
//
// One launch covers every problem: routed expert e (its rows are the
// expert-contiguous rows offsets[e] .. offsets[e+1]-1 built by the dispatch)
// and the shared expert (all T tokens, gate 1). Work items are 256-row x
// 256-column output tiles; the dispatch writes their per-problem prefix, and a
// block finds its problem by binary search, so the host never learns the
// per-expert row counts.
//
// Gate/up GEMM (fine-grained SwiGLU expert, DeepSeek-V2 walkthrough page MoE
// code; architecture article section 3.3): a tile loads 128 W_gate rows and the
// matching 128 W_up rows, so h = SiLU(x W_gate^T) * (x W_up^T) is formed in
// registers and only h (bf16) is written. Token rows are gathered from x
// through the dispatch's row -> token map.
// Down GEMM: Y[row] = g_row * (h[row] W_down^T), bf16, 256 output columns per
// tile; the combine sums the K rows of each token in a fixed order.
//
// Tile 256 x 256, K step 64, 8 waves (two per SIMD) as 2 x 4, each wave
// 128 x 64 as 4 x 2 blocks of v_mfma_f32_32x32x16_bf16 (128 fp32 accumulators
// per lane); two waves per SIMD keep both the matrix pipe and the LDS busy
// while the other waits. A wave's four 32-row blocks are interleaved with the
// other row-wave's (blocks wm, wm+2, wm+4, wm+6), so a ragged tile splits its
// valid rows evenly; the tile body is instantiated per count of valid row
// blocks (and of 64-row groups of token rows to load), so blocks with no
// valid row cost no MFMA, groups with no valid row no load or LDS write, and
// the K loop stays branch-free.
// Both operands are staged through two LDS buffers (rows padded to 144 bytes so
// that the 16-byte fragment reads of consecutive rows hit distinct banks): the
// weight rows of the next K step, and the token rows of the step after it
// (two register slots), are loaded into registers while the current step is
// multiplied, and the next step is written to the other buffer; one barrier
// per K step. The loads are spread between the MFMAs of the first three
// substeps (weights first) rather than issued together: a wave whose
// request cannot enter a full memory queue stalls, and with it the MFMAs
// behind it in program order.
// Blocks are mapped so that runs of consecutive tiles land on one XCD and its
// L2, with runs spread round-robin over the XCDs. Tiles are ordered
// column-tile major, and an expert's rows are split evenly (in 32-row blocks)
// over its two or three row tiles: the row tiles that read one weight slice
// run side by side at the same pace, so the second and third reads of each
// weight line hit that L2 (this halves the bytes fetched past L2). The shared
// expert (every token, dozens of row tiles) goes in groups of four row tiles,
// column-tile major inside a group: a run then covers 4 row tiles x 8 weight
// slices, which share both operands through L2.
#include <type_traits>

#include "moe_internal.hpp"

namespace moe {

namespace {
constexpr int BM = kGB_BM, BN = 256, BK = kGB_BK, LDW = BK + 8;
constexpr int kRows = BM + BN;  // LDS rows per buffer: A then B
constexpr int kRun = 32;        // consecutive tiles per XCD run
constexpr int kNC = 2;          // 32-column blocks per wave
constexpr int kLd = 8;          // 16-byte global loads per thread per K step

struct Tile {
  const uint16_t* a_rows;  // GEMM1: x; GEMM2: h of this problem (row 0 = row_base)
  const int32_t* tok;      // GEMM1 routed: row -> token map at row_base; null = identity
  const void* w;           // weights of this problem (bf16, or e4m3 codes)
  const float* ws;         // e4m3: the problem's 128x128 block scales, [rows/128][K/128]
  int kbn;                 // e4m3: K/128
  uint16_t* c;             // output rows of this problem (row 0 = row_base)
  uint16_t* c2;            // recompute mode: g * h rows; training mode: [a | u] rows
  uint16_t* c3;            // training mode: g * h rows
  const float* gate;       // GEMM2 routed: gates at row_base; null = 1
  uint32_t a_bytes;        // extent of a_rows (buffer range)
  uint32_t w_bytes;        // extent of w
  int lda;                 // row length of a_rows
  int ldc;                 // row length of c
  int K;                   // reduction length
  int Hp;                  // hidden of this problem
  int D;
  int m0, vrows, nt;
};
}  // namespace

template <int kMode, int NRB, int NLA, bool kW8>
__device__ __forceinline__ void tile_body(const Tile& t, uint16_t (*smem)[kRows * LDW], float* s_gate) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: no VGPR held across the K loop
  const int wm = wave >> 2, wn = wave & 3;
  const int c8 = tid & 7, r0 = tid >> 3;

  // loader: 8 chunks of 16 bytes per thread per K step, rows r0 + 64*j of
  // the 512 LDS rows (j < 4: A rows, j >= 4: B rows), read as buffer loads:
  // a 32-bit byte offset per row in a VGPR, the K position in a scalar offset.
  // Rows past the tile's valid rows (and columns past D) read a valid row
  // instead: their results are never stored, so every load is unconditional.
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(t.a_rows), (short)0, t.a_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(t.w), (short)0, t.w_bytes, 0x00020000);
  uint32_t voff[kLd / 2];
#pragma unroll
  for (int j = 0; j < kLd / 2; ++j) {
    const int m = r0 + 64 * j;
    const int mm = t.m0 + (m < t.vrows ? m : 0);
    const int row = (kMode != 1 && t.tok != nullptr) ? dcheck(t.tok[mm], (int)(t.a_bytes / (2u * t.lda)), kSiteGroupedTok) : mm;
    voff[j] = ((uint32_t)row * (uint32_t)t.lda + c8 * 8) * 2u;
  }
  // Weight (B) rows: one VGPR offset for the thread's first row, the other
  // rows' distance (uniform) in the scalar offset. bf16: rows r0 + 64*j
  // (gate/up: W_gate rows nt*128 + r0 + {0, 64}, then the same W_up rows;
  // down rows past D read row nt*256 + r0 instead). e4m3: thread tid takes B
  // row tid/2, bytes 32*(tid%2) .. +31 of the 64-byte K slice (two loads),
  // and the block scale of that row.
  uint32_t vb;
  uint32_t bd[kLd / 2];
  const float* wsrow = nullptr;
  if (kW8) {
    const int b = tid >> 1;
    int wrow = (kMode != 1) ? (b < 128 ? t.nt * 128 + b : t.Hp + t.nt * 128 + b - 128) : t.nt * BN + b;
    if (kMode == 1 && wrow >= t.D) wrow = 0;
    vb = (uint32_t)wrow * (uint32_t)t.K + 32u * (tid & 1);
    wsrow = t.ws + (size_t)(wrow >> 7) * t.kbn;
#pragma unroll
    for (int j = 0; j < kLd / 2; ++j) bd[j] = 16u * j;
  } else {
    const int wrow = (kMode != 1) ? t.nt * 128 + r0 : t.nt * BN + r0;
    vb = ((uint32_t)wrow * (uint32_t)t.K + c8 * 8) * 2u;
#pragma unroll
    for (int j = 0; j < kLd / 2; ++j) {
      int dr = (kMode != 1) ? (j & 1) * 64 + (j >> 1) * t.Hp : 64 * j;
      if (kMode == 1 && t.nt * BN + 64 * j >= t.D) dr = 0;
      bd[j] = (uint32_t)dr * (uint32_t)t.K * 2u;
    }
  }
  auto gload = [&](int j, int k0) __attribute__((always_inline)) {
    return j < kLd / 2
               ? __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra, voff[j], k0 * 2, 0))
               : __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                               rb, vb, (kW8 ? k0 : k0 * 2) + bd[j - kLd / 2], 0));
  };
  constexpr int kLdB = kW8 ? 2 : kLd / 2;  // 16-byte weight loads per thread per K step

  f32x16 acc[NRB > 0 ? NRB : 1][kNC];
#pragma unroll
  for (int i = 0; i < NRB; ++i)
#pragma unroll
    for (int c = 0; c < kNC; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][c][e] = 0.f;

  // LDS B rows of this wave's two 32-column blocks (gate/up: one W_gate block
  // and the matching W_up block)
  int bcol[kNC];
#pragma unroll
  for (int c = 0; c < kNC; ++c) bcol[c] = (kMode != 1) ? 128 * c + 32 * wn : 64 * wn + 32 * c;
  const int lr = lane & 31, lk = (lane >> 5) * 8;

  // down GEMM and recompute: the tile's gates into LDS for the epilogue
  if (kMode != 0 && tid < BM) s_gate[tid] = (t.gate != nullptr && tid < t.vrows) ? t.gate[t.m0 + tid] : 1.0f;

  // A rows (gathered token rows) are loaded two K steps ahead through two
  // register slots; B rows (weights) one step ahead
  const int nk = t.K / BK;
  uint4 pa[2][kLd / 2], pb[kLdB];
  float pbs = 1.0f;  // e4m3: block scale of the staged weight slice
#pragma unroll
  for (int j = 0; j < NLA; ++j) pa[0][j] = gload(j, 0);
#pragma unroll
  for (int j = 0; j < kLdB; ++j) pb[j] = gload(kLd / 2 + j, 0);
  if (kW8) pbs = wsrow[0];
#pragma unroll
  for (int j = 0; j < NLA; ++j) pa[1][j] = gload(j, (nk > 1 ? 1 : 0) * BK);

  // Fragments are double-buffered across the four 16-wide substeps of a K
  // step: the LDS reads of substep kk+1 are issued before the MFMAs of
  // substep kk, so their latency hides behind those MFMAs.
  constexpr int NA = NRB > 0 ? NRB : 1;
  bf16x8 fb[2][kNC], fa[2][NA];
  auto read_frags = [&](const uint16_t* sbuf, int kk, int slot) __attribute__((always_inline)) {
    const uint16_t* sA = sbuf;
    const uint16_t* sB = sbuf + BM * LDW;
#pragma unroll
    for (int c = 0; c < kNC; ++c)
      fb[slot][c] = *reinterpret_cast<const bf16x8*>(&sB[(bcol[c] + lr) * LDW + kk + lk]);
#pragma unroll
    for (int i = 0; i < NRB; ++i)
      fa[slot][i] = *reinterpret_cast<const bf16x8*>(&sA[(32 * (wm + 2 * i) + lr) * LDW + kk + lk]);
  };
  auto mfmas = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NRB; ++i)
#pragma unroll
      for (int c = 0; c < kNC; ++c)
        acc[i][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][i], fb[slot][c], acc[i][c], 0, 0, 0);
  };

  // The next K step's tile is written to the other LDS buffer interleaved
  // with the MFMAs of the last substep: its weight rows, loaded at the top of
  // this step, get three quarters of a step to land, its token rows, loaded a
  // step earlier, one and three quarters; the LDS writes overlap the matrix
  // work.
  auto store_a = [&](int buf, const uint4 (&v)[kLd / 2]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NLA; ++j) *reinterpret_cast<uint4*>(&smem[buf][(r0 + 64 * j) * LDW + c8 * 8]) = v[j];
  };
  auto store_b = [&](int buf) __attribute__((always_inline)) {
    if (kW8) {
      // 32 e4m3 codes -> exact fp32 -> times the block scale -> bf16 (RNE)
      uint16_t* dst = &smem[buf][(BM + (tid >> 1)) * LDW + 32 * (tid & 1)];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t w[4] = {pb[j].x, pb[j].y, pb[j].z, pb[j].w};
        uint32_t o[8];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[d], 1.0f, false);
          const f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[d], 1.0f, true);
          const bf16x2 a = {(__bf16)(lo.x * pbs), (__bf16)(lo.y * pbs)};
          const bf16x2 b = {(__bf16)(hi.x * pbs), (__bf16)(hi.y * pbs)};
          o[2 * d] = __builtin_bit_cast(uint32_t, a);
          o[2 * d + 1] = __builtin_bit_cast(uint32_t, b);
        }
        *reinterpret_cast<uint4*>(dst + 16 * j) = make_uint4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<uint4*>(dst + 16 * j + 8) = make_uint4(o[4], o[5], o[6], o[7]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < kLd / 2; ++j)
        *reinterpret_cast<uint4*>(&smem[buf][(r0 + 64 * (kLd / 2 + j)) * LDW + c8 * 8]) = pb[j];
    }
  };
#pragma unroll
  for (int j = 0; j < NLA; ++j) *reinterpret_cast<uint4*>(&smem[0][(r0 + 64 * j) * LDW + c8 * 8]) = pa[0][j];
  store_b(0);
  __syncthreads();
  // instruction counts per substep, for the interleave below
  constexpr int nr = kNC + NRB, nm = kNC * NRB, nw = kLd / 2;
  constexpr int p1 = nr < nm ? nr : nm;              // (MFMA, LDS read) pairs
  constexpr int nwr = NLA + kLd / 2;                 // LDS writes of the last substep (A, then B)
  constexpr int p4 = nwr < nm ? nwr : nm;            // last substep: (MFMA, LDS write) pairs

  read_frags(smem[0], 0, 0);
  auto kstep = [&](int kt, auto s_c) __attribute__((always_inline)) {
    constexpr int S = decltype(s_c)::value;  // register slot of A(kt), refilled with A(kt+2)
    const int cur = kt & 1;
    // The last step reloads its own K slice and writes the idle buffer, so
    // the step body has no branch (and the scheduler sees one region).
    const int knext = (kt + 1 < nk ? kt + 1 : kt) * BK;
    const int knext2 = (kt + 2 < nk ? kt + 2 : nk - 1) * BK;
    // Weight rows of the next step (spread over substep 0), token rows of
    // the step after it (spread over substep 1): loads complete in issue
    // order for the wait counter, so waiting for the weights at the end of
    // this step leaves the token rows in flight; spreading the requests keeps
    // the matrix instructions behind them from waiting on a full queue.
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s == 0) {
#pragma unroll
        for (int j = 0; j < kLdB; ++j) pb[j] = gload(kLd / 2 + j, knext);
        if (kW8) pbs = wsrow[knext >> 7];
      } else {
#pragma unroll
        for (int j = 0; j < (NLA < kLd / 4 ? NLA : kLd / 4); ++j) pa[S][j] = gload(j, knext2);
      }
      read_frags(smem[cur], 16 * (s + 1), (s + 1) & 1);
      mfmas(s & 1);
      constexpr int nv = (kLdB > kLd / 2 ? kLdB : kLd / 2);
#pragma unroll
      for (int q = 0; q < p1; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (q < nv) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x020, nv > p1 ? nv - p1 : 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, nr - p1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, nm - p1, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // substep 2: last fragments, the second half of the token rows
#pragma unroll
    for (int j = kLd / 4; j < NLA; ++j) pa[S][j] = gload(j, knext2);
    read_frags(smem[cur], 48, 1);
    mfmas(0);
#pragma unroll
    for (int q = 0; q < p1; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (q < kLd / 4) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, nr - p1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, nm - p1, 0);
    __builtin_amdgcn_sched_barrier(0);
    // substep 3: the whole next tile into the idle buffer
    store_a(cur ^ 1, pa[S ^ 1]);
    store_b(cur ^ 1);
    mfmas(1);
#pragma unroll
    for (int q = 0; q < p4; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x200, nwr - p4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, nm - p4, 0);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    read_frags(smem[cur ^ 1], 0, 0);
  };
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    kstep(kt, std::integral_constant<int, 0>{});
    kstep(kt + 1, std::integral_constant<int, 1>{});
  }
  if (kt < nk) kstep(kt, std::integral_constant<int, 0>{});

  // D layout of the 32x32 MFMA: element e of lane l is row 8*(e/4) + 4*(l/32) + e%4,
  // column l%32.
  // A 256 x 128 bf16 tile whose element (m, 32*wn + lr) is val(i, e) in this
  // lane is staged through LDS (rows of 136 elements), then written as full
  // 16-byte pieces of its rows (256 contiguous bytes each) to dst (row 0 = the
  // tile's first row, row length ldc). Rows e, e+1 (e even) of a lane are
  // adjacent rows of one column; an even lane swaps its row-(e+1) value for
  // its odd neighbour's row-e value (DPP quad permute 1,0,3,2), so each lane
  // writes two adjacent columns of one row as one 32-bit word.
  auto store_tile128 = [&](auto val, uint16_t* dst, int ldc) __attribute__((always_inline)) {
    constexpr int kLdh = 128 + 8;
    uint16_t* so = &smem[0][0];
    const bool odd = lane & 1;
    __syncthreads();  // the staging area is free (K loop or previous tile done)
#pragma unroll
    for (int i = 0; i < NRB; ++i) {
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const int m = 32 * (wm + 2 * i) + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const uint32_t b0 = f32_to_bf16(val(i, e, m)), b1 = f32_to_bf16(val(i, e + 1, m + 1));
        const uint32_t r = (uint32_t)__builtin_amdgcn_mov_dpp((int)(odd ? b0 : b1), 0xB1, 0xF, 0xF, false);
        const uint32_t w = odd ? (r | (b1 << 16)) : (b0 | (r << 16));
        *reinterpret_cast<uint32_t*>(&so[(m + (odd ? 1 : 0)) * kLdh + ((32 * wn + lr) & ~1)]) = w;
      }
    }
    __syncthreads();
    const int q = tid & 15;  // 16-byte piece of a row
#pragma unroll 4
    for (int r = tid >> 4; r < t.vrows; r += 32)
      *reinterpret_cast<uint4*>(dst + (size_t)(t.m0 + r) * ldc + 8 * q) =
          *reinterpret_cast<const uint4*>(&so[r * kLdh + 8 * q]);
  };
  if (kMode == 0) {
    // h tile (256 x 128)
    store_tile128([&](int i, int e, int) { return silu_fast(acc[i][0][e]) * acc[i][1][e]; },
                  t.c + t.nt * 128, t.ldc);
  } else if (kMode == 2) {
    // recompute for the backward pass: the pre-activations a = x W_gate^T and
    // u = x W_up^T (one bf16 row of 2*Hp: a then u) and g * SiLU(a) * u
    store_tile128([&](int i, int e, int) { return acc[i][0][e]; }, t.c + t.nt * 128, t.ldc);
    store_tile128([&](int i, int e, int) { return acc[i][1][e]; }, t.c + t.Hp + t.nt * 128, t.ldc);
    store_tile128([&](int i, int e, int m) { return s_gate[m] * silu_fast(acc[i][0][e]) * acc[i][1][e]; },
                  t.c2 + t.nt * 128, t.Hp);
  } else if (kMode == 3) {
    // forward of a training step: h as in mode 0, and from the same
    // accumulators what the backward pass would recompute (mode 2)
    store_tile128([&](int i, int e, int) { return silu_fast(acc[i][0][e]) * acc[i][1][e]; },
                  t.c + t.nt * 128, t.Hp);
    store_tile128([&](int i, int e, int) { return acc[i][0][e]; }, t.c2 + t.nt * 128, 2 * t.Hp);
    store_tile128([&](int i, int e, int) { return acc[i][1][e]; }, t.c2 + t.Hp + t.nt * 128, 2 * t.Hp);
    store_tile128([&](int i, int e, int m) { return s_gate[m] * silu_fast(acc[i][0][e]) * acc[i][1][e]; },
                  t.c3 + t.nt * 128, t.Hp);
  } else {
    // y tile (256 x 256): staged through LDS, then written as full 16-byte
    // pieces of each row (the tile's rows are 512 contiguous bytes of y).
    // Rows e, e+1 (e even) of a lane are adjacent rows of one column; an
    // even lane swaps its row-(e+1) value for its odd neighbour's row-e
    // value (DPP quad permute 1,0,3,2), so each lane writes two adjacent
    // columns of one row as one 32-bit word.
    constexpr int kLdo = BN + 8;  // staging row, elements (528 bytes)
    uint16_t* so = &smem[0][0];
    const bool odd = lane & 1;
    __syncthreads();  // the last fragment reads of the K loop are done
#pragma unroll
    for (int i = 0; i < NRB; ++i) {
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const int m = 32 * (wm + 2 * i) + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);  // row of element e
        const float g0 = s_gate[m], g1 = s_gate[m + 1];
#pragma unroll
        for (int c = 0; c < kNC; ++c) {
          const uint32_t b0 = f32_to_bf16(g0 * acc[i][c][e]), b1 = f32_to_bf16(g1 * acc[i][c][e + 1]);
          const uint32_t r = (uint32_t)__builtin_amdgcn_mov_dpp((int)(odd ? b0 : b1), 0xB1, 0xF, 0xF, false);
          const int col = 64 * wn + 32 * c + lr;
          const uint32_t w = odd ? (r | (b1 << 16)) : (b0 | (r << 16));
          *reinterpret_cast<uint32_t*>(&so[(m + (odd ? 1 : 0)) * kLdo + (col & ~1)]) = w;
        }
      }
    }
    __syncthreads();
    const int q = tid & 31;  // 16-byte piece of a row
    const int col = t.nt * BN + 8 * q;
    if (col < t.D) {  // D % 128 == 0: a piece is wholly inside or outside
#pragma unroll 4
      for (int r = tid >> 5; r < t.vrows; r += 16)
        *reinterpret_cast<uint4*>(t.c + (size_t)(t.m0 + r) * t.ldc + col) =
            *reinterpret_cast<const uint4*>(&so[r * kLdo + 8 * q]);
    }
  }
}

// kMode 0: gate/up + SwiGLU, 1: down + gate scale, 2: gate/up pre-activations
// and g * h for the backward pass, 3: mode 0's h together with mode 2's
// outputs (the forward of a training step); kW8: e4m3 weights with
// 128x128 block scales, widened to bf16 (times the scale) as they are staged
template <int kMode, bool kW8>
__global__ __launch_bounds__(512) void grouped_gemm_bf16_kernel(ExpertGemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2][kRows * LDW];
  __shared__ int32_t s_pre[kMaxExperts + 2];
  __shared__ int32_t s_off[kMaxExperts + 1];
  __shared__ float s_gate[BM];

  // Tiles come in runs of kRun consecutive tiles; run r goes to XCD r % 8,
  // so every XCD gets a mix of experts and of the shared expert's tiles while
  // a run's blocks share that XCD's L2. Blocks are handed to the XCDs
  // round-robin (block b runs on XCD b % 8).
  const int total = a.pre[a.E + 1];
  const int bid = blockIdx.x;
  const int slot = bid >> 3;
  const int tile = ((slot / kRun) * 8 + (bid & 7)) * kRun + slot % kRun;
  if (tile >= total) return;

  // problem tables into LDS: one round trip, then the search stays on chip
  for (int i = threadIdx.x; i < a.E + 2; i += blockDim.x) s_pre[i] = a.pre[i];
  for (int i = threadIdx.x; i < a.E + 1; i += blockDim.x) s_off[i] = a.offsets[i];
  __syncthreads();
  // workgroup-uniform values, made scalar: read from LDS they would sit in
  // VGPRs, and so would every pointer built from them
  const int p = __builtin_amdgcn_readfirstlane(find_problem(s_pre, a.E, tile));
  const bool routed = p < a.E;
  const int rows = __builtin_amdgcn_readfirstlane(routed ? s_off[p + 1] - s_off[p] : a.T);
  const int row_base = __builtin_amdgcn_readfirstlane(routed ? s_off[p] : 0);
  constexpr size_t kWB = kW8 ? 1 : 2;  // bytes per weight
  Tile t;
  t.Hp = routed ? a.H : a.Hs;
  t.D = a.D;
  const int local = __builtin_amdgcn_readfirstlane(tile - s_pre[p]);
  // an expert's rows are split evenly (in 32-row blocks) over its row tiles,
  // so the tiles that share a weight slice run at the same pace
  const int nmt = (rows + BM - 1) / BM;
  const int rpt = ((rows + nmt - 1) / nmt + 31) & ~31;
  if (routed) {
    t.m0 = (local % nmt) * rpt;  // column-tile major: the row tiles of one weight slice run together
    t.nt = local / nmt;
  } else {
    // the shared expert (every token: many row tiles): groups of 4 row tiles,
    // column-tile major inside a group, so a run of consecutive tiles covers
    // a few row tiles x a few weight slices and both operands stay in L2
    const int ncols = (s_pre[p + 1] - s_pre[p]) / nmt;
    const int g0 = (local / (4 * ncols)) * 4;
    const int gsz = min(4, nmt - g0);
    const int idx = local - g0 * ncols;
    t.m0 = (g0 + idx % gsz) * rpt;
    t.nt = idx / gsz;
  }
  t.K = (kMode != 1) ? a.D : t.Hp;
  t.m0 = dcheck(t.m0, rows, kSiteGroupedRows);
  t.vrows = min(rows - t.m0, rpt);
  if (kMode != 1) {
    t.a_rows = static_cast<const uint16_t*>(a.a);
    t.lda = a.D;
    t.tok = routed ? a.row_token + row_base : nullptr;
    t.w = routed ? static_cast<const char*>(a.w) + (size_t)p * 2 * t.Hp * a.D * kWB
                 : static_cast<const char*>(a.w_shared);
    t.kbn = a.D / 128;
    t.ws = kW8 ? (routed ? a.w_scale + (size_t)p * (2 * t.Hp / 128) * t.kbn : a.w_shared_scale) : nullptr;
    t.c3 = nullptr;
    if (kMode == 2) {
      t.c = routed ? static_cast<uint16_t*>(a.c) + (size_t)row_base * 2 * a.H : static_cast<uint16_t*>(a.c_shared);
      t.c2 = routed ? static_cast<uint16_t*>(a.c2) + (size_t)row_base * a.H : static_cast<uint16_t*>(a.c2_shared);
      t.ldc = 2 * t.Hp;
      t.gate = routed ? a.row_gate + row_base : nullptr;
    } else if (kMode == 3) {
      t.c = routed ? static_cast<uint16_t*>(a.c) + (size_t)row_base * a.H : static_cast<uint16_t*>(a.c_shared);
      t.c2 = routed ? static_cast<uint16_t*>(a.c2) + (size_t)row_base * 2 * a.H : static_cast<uint16_t*>(a.c2_shared);
      t.c3 = routed ? static_cast<uint16_t*>(a.c3) + (size_t)row_base * a.H : static_cast<uint16_t*>(a.c3_shared);
      t.ldc = t.Hp;
      t.gate = routed ? a.row_gate + row_base : nullptr;
    } else {
      t.c = routed ? static_cast<uint16_t*>(a.c) + (size_t)row_base * a.H : static_cast<uint16_t*>(a.c_shared);
      t.c2 = nullptr;
      t.ldc = t.Hp;
      t.gate = nullptr;
    }
    t.a_bytes = (uint32_t)((size_t)a.x_rows * a.D * 2);
    t.w_bytes = (uint32_t)((size_t)2 * t.Hp * a.D * kWB);
  } else {
    t.a_rows = routed ? static_cast<const uint16_t*>(a.a) + (size_t)row_base * a.H
                      : static_cast<const uint16_t*>(a.a_shared);
    t.lda = t.Hp;
    t.tok = nullptr;
    t.w = routed ? static_cast<const char*>(a.w) + (size_t)p * a.D * t.Hp * kWB
                 : static_cast<const char*>(a.w_shared);
    t.kbn = t.Hp / 128;
    t.ws = kW8 ? (routed ? a.w_scale + (size_t)p * (a.D / 128) * t.kbn : a.w_shared_scale) : nullptr;
    t.c = routed ? static_cast<uint16_t*>(a.c) + (size_t)row_base * a.D : static_cast<uint16_t*>(a.c_shared);
    t.c2 = nullptr;
    t.ldc = a.D;
    t.gate = routed ? a.row_gate + row_base : nullptr;
    t.a_bytes = (uint32_t)((size_t)rows * t.Hp * 2);
    t.w_bytes = (uint32_t)((size_t)a.D * t.Hp * kWB);
  }

  // valid 32-row blocks of this wave: wm + 2*i for i < nrb; the tile's
  // token rows are loaded in nla groups of 64 (rows past the last group are
  // neither loaded nor written to LDS: no fragment read reaches them). The
  // first row-wave has nrb == nla, the second nla or nla - 1.
  const int wm = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) >> 2;
  int nrb = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) nrb += (32 * (wm + 2 * i) < t.vrows) ? 1 : 0;
  const int nla = min(4, max(1, (t.vrows + 63) / 64));
  switch (nrb * 8 + nla) {
    case 4 * 8 + 4: tile_body<kMode, 4, 4, kW8>(t, smem, s_gate); break;
    case 3 * 8 + 4: tile_body<kMode, 3, 4, kW8>(t, smem, s_gate); break;
    case 3 * 8 + 3: tile_body<kMode, 3, 3, kW8>(t, smem, s_gate); break;
    case 2 * 8 + 3: tile_body<kMode, 2, 3, kW8>(t, smem, s_gate); break;
    case 2 * 8 + 2: tile_body<kMode, 2, 2, kW8>(t, smem, s_gate); break;
    case 1 * 8 + 2: tile_body<kMode, 1, 2, kW8>(t, smem, s_gate); break;
    case 1 * 8 + 1: tile_body<kMode, 1, 1, kW8>(t, smem, s_gate); break;
    default: tile_body<kMode, 0, 1, kW8>(t, smem, s_gate); break;
  }
}

// blocks covering every tile index below max_items under the run mapping
int grouped_blocks(int max_items, int run) {
  const int runs = (max_items + run - 1) / run;
  return ((runs + 7) / 8) * 8 * run;
}

hipError_t launch_grouped_gateup(const ExpertGemmArgs& a, int fp8, hipStream_t s) {
  const int blocks = grouped_blocks(a.max_items, kRun);
  if (blocks == 0) return hipSuccess;
  if (fp8)
    hipLaunchKernelGGL((grouped_gemm_bf16_kernel<0, true>), dim3(blocks), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL((grouped_gemm_bf16_kernel<0, false>), dim3(blocks), dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_grouped_recompute(const ExpertGemmArgs& a, hipStream_t s) {
  const int blocks = grouped_blocks(a.max_items, kRun);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_gemm_bf16_kernel<2, false>), dim3(blocks), dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_grouped_gateup_train(const ExpertGemmArgs& a, hipStream_t s) {
  const int blocks = grouped_blocks(a.max_items, kRun);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_gemm_bf16_kernel<3, false>), dim3(blocks), dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_grouped_down(const ExpertGemmArgs& a, int fp8, hipStream_t s) {
  const int blocks = grouped_blocks(a.max_items, kRun);
  if (blocks == 0) return hipSuccess;
  if (fp8)
    hipLaunchKernelGGL((grouped_gemm_bf16_kernel<1, true>), dim3(blocks), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL((grouped_gemm_bf16_kernel<1, false>), dim3(blocks), dim3(512), 0, s, a);
  return hipGetLastError();
}

MOE_DEBUG_READER(debug_read_grouped)

}  // namespace moe
