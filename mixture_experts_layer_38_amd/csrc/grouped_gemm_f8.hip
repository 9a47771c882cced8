// Grouped GEMMs of the routed experts and the shared expert with both inputs
// in e4m3 (the fp8 GEMMs of the architecture article, section 4.2: fp8
// inputs, fp32 accumulation, block-wise quantisation): token rows and h carry
// one fp32 scale per 1 x 128 block of a row, weights one per 128 x 128 block.
//
// One K step is 128 elements, i.e. one scale block of both operands. Per step
// and 16 x 16 output block, one v_mfma_scale_f32_16x16x128_f8f6f4 (unit
// hardware scale: the fp32 block scales are not powers of two) forms the
// block's partial sum of code products, which is added to the fp32
// accumulator times (row scale x weight scale) -- the per-block promotion
// that the block scales require. A lane's four accumulator rows are
// consecutive, so its row scales are one 16-byte LDS read per row block.
//
// Gate/up GEMM: a tile loads 128 W_gate rows and the matching 128 W_up rows,
// h = SiLU(gate) * up is formed in fp32 and, per 1 x 128 block of each row
// (the tile's 128 h columns are exactly one block), quantised to e4m3 in the
// epilogue: h leaves the kernel as codes + scales, ready for the down GEMM.
// Token rows are gathered (codes and their scales) through the dispatch's
// row -> token map. Down GEMM: Y[row] = g_row * (h[row] W_down^T), bf16.
//
// Both GEMMs: 8 waves (two per SIMD) as 2 x 4, each wave owns 64 columns
// (4 blocks of 16) and the row blocks wm + 2i of the tile, interleaved with
// the other row-wave's; the tile body is instantiated per count of valid row
// blocks. Operands are staged through two LDS buffers (rows padded to 144
// bytes), the next K step's operands are loaded into registers while the
// current one is multiplied and written to the idle buffer behind its MFMAs;
// one barrier per step. Tile order and the even split of an expert's rows
// over its row tiles follow the bf16 grouped GEMMs (runs of 32 tiles per XCD,
// column-tile major).
//
// The two GEMMs differ in tile height. Gate/up tiles are 128 x 256 (4 row
// blocks per wave): all fragments of a step are held in registers, the token
// rows are loaded two steps ahead, and the second pair of column blocks is
// read behind the first pair's MFMAs. Down tiles are 256 x 256 (8 row blocks
// per wave), which halves the weight bytes streamed per output: the four
// column fragments are held for the step while the row fragments (and their
// scales) stream through two register slots one row block ahead; the row
// block count is rounded up to an even number (a block past the valid rows
// multiplies a copy of a valid row and is never stored). The gate/up GEMM
// keeps the shorter tile: its extra scale work per MFMA (two weight scales)
// and its h-quantisation epilogue leave no registers for the taller one.
#include <type_traits>

#include "moe_internal.hpp"

namespace moe {

namespace {
constexpr int BM1 = kF8_BM1, BM2 = kF8_BM2;  // tile rows: gate/up, down
constexpr int BN = 256, BK = kF8_BK, LDB = BK + 16;  // LDS row stride in bytes
// bytes of one LDS operand buffer: A rows then B rows
constexpr int buf_bytes(int bm) { return (bm + BN) * LDB; }
constexpr int kBuf1 = buf_bytes(BM1), kBuf2 = buf_bytes(BM2);
constexpr int kRun = 32;
constexpr int kLdB = 4;        // 16-byte weight loads per thread per K step
constexpr int kHLd = BK + 4;   // gate/up epilogue: fp32 h staging row (floats)
constexpr int kYLd = BN + 8;   // down epilogue: bf16 y staging row (elements)
static_assert(BM1 * kHLd * 4 <= 2 * kBuf1, "h staging fits the operand buffers");
static_assert(BM2 * kYLd * 2 <= 2 * kBuf2, "y staging fits the operand buffers");

typedef __attribute__((ext_vector_type(8))) int i32x8;

struct TileF8 {
  const uint8_t* a_rows;  // GEMM1: x codes; GEMM2: h codes of this problem (row 0 = row_base)
  const int32_t* tok;     // GEMM1 routed: row -> token map at row_base; null = identity
  const float* a_scale;   // scales of a_rows' rows, [.][a_sld]
  int a_sld;              // K / 128
  const uint8_t* w;       // e4m3 weights of this problem
  const float* ws;        // their 128x128 block scales, [rows/128][K/128]
  void* c;                // GEMM1: h codes (row 0 = row_base); GEMM2: y bf16
  float* c_scale;         // GEMM1: h scales, [.][c_sld]
  int c_sld;              // Hp / 128
  const float* gate;      // GEMM2 routed: gates at row_base; null = 1
  uint32_t a_bytes, w_bytes;
  int lda, ldc, K, Hp, D;
  int m0, vrows, nt;
};

// 32 bytes of one LDS row as two 16-byte reads (rows are 16-byte aligned)
__device__ __forceinline__ i32x8 lds_frag(const uint8_t* p) {
  const uint4 lo = *reinterpret_cast<const uint4*>(p), hi = *reinterpret_cast<const uint4*>(p + 16);
  return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

__device__ __forceinline__ f32x4 mfma_f8(const i32x8& a, const i32x8& b, const f32x4& c) {
  // format 0 = e4m3 for both operands; E8M0 scale 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// source row of the tile's A row m (m < BM): rows past the valid ones read
// the tile's first row instead (loaded, never stored), so every load is
// unconditional; gate/up routed rows go through the row -> token map
__device__ __forceinline__ int a_source_row(const TileF8& t, int m) {
  const int mm = t.m0 + (m < t.vrows ? m : 0);
  return t.tok != nullptr ? dcheck(t.tok[mm], (int)(t.a_bytes / (uint32_t)t.lda), kSiteF8Tok) : mm;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}
}  // namespace

// Gate/up + SwiGLU + h quantisation, 128-row tiles: the tile's 128 hidden
// columns are W_gate rows nt*128 .. +127 and the same W_up rows.
template <int NRB>
__device__ __forceinline__ void gateup_body_f8(const TileF8& t, uint8_t (*smem)[kBuf1], float (*s_asc)[512]) {
  constexpr int BM = BM1, kLdA = 2;  // A rows r0 and r0 + 64
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int c16 = tid & 7, r0 = tid >> 3;

  // loader: 16-byte pieces; A rows r0 and r0 + 64 (128 bytes = one K step
  // each), B rows r0 + 64*j
  const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(t.a_rows, t.a_bytes);
  const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(t.w, t.w_bytes);
  uint32_t voa[kLdA];
#pragma unroll
  for (int j = 0; j < kLdA; ++j) voa[j] = (uint32_t)a_source_row(t, r0 + 64 * j) * (uint32_t)t.lda + c16 * 16;
  // B rows r0 + 64*j: one VGPR offset for row r0, the other rows' distance
  // (uniform) in the scalar offset: W_gate rows nt*128 + r0 + {0, 64}, then
  // the same W_up rows
  const uint32_t vob = (uint32_t)(t.nt * 128 + r0) * (uint32_t)t.K + c16 * 16;
  uint32_t bd[kLdB];
#pragma unroll
  for (int j = 0; j < kLdB; ++j) bd[j] = (uint32_t)((j & 1) * 64 + (j >> 1) * t.Hp) * (uint32_t)t.K;
  // row scales: thread tid stages the scale of A row tid % 128 (threads
  // past 128 write a copy that is never read, so the K loop has no branch)
  const float* asrow = t.a_scale + (size_t)a_source_row(t, tid & (BM - 1)) * t.a_sld;
  // weight scales: one 128-row block of W_gate and one of W_up (read
  // through vector loads one K step ahead: a scalar load in the loop would
  // make every LDS wait after it wait for the scalar load too)
  const uint32_t wso[2] = {(uint32_t)(t.nt * t.a_sld) * 4u, (uint32_t)((t.Hp / 128 + t.nt) * t.a_sld) * 4u};
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(t.ws, (uint32_t)(2 * t.Hp / 128 * t.a_sld) * 4u);
  auto load_ws = [&](int c, int kb) __attribute__((always_inline)) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, 0u, wso[c] + 4u * kb, 0));
  };

  auto gload_a = [&](int j, int k0) __attribute__((always_inline)) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra, voa[j], k0, 0));
  };
  auto gload_b = [&](int j, int k0) __attribute__((always_inline)) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rb, vob, k0 + bd[j], 0));
  };

  // 16 x 16 output blocks: row block i (rows 16*(wm + 2i) ..), column block
  // c: c < 2 the wave's two W_gate blocks, c >= 2 the matching W_up blocks
  constexpr int NA = NRB > 0 ? NRB : 1;
  f32x4 acc[NA][4];
#pragma unroll
  for (int i = 0; i < NA; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[i][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  int bcol[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) bcol[c] = 128 * (c >> 1) + 32 * wn + 16 * (c & 1);
  const int lr = lane & 15, lk = (lane >> 4) * 32;

  const int nk = t.K / BK;
  uint4 pa[2][kLdA], pb[kLdB];
  float pas[2];
#pragma unroll
  for (int j = 0; j < kLdA; ++j) pa[0][j] = gload_a(j, 0);
  pas[0] = asrow[0];
#pragma unroll
  for (int j = 0; j < kLdB; ++j) pb[j] = gload_b(j, 0);
  float swc[2] = {load_ws(0, 0), load_ws(1, 0)};  // weight scales of the step being multiplied
  {
    const int k1 = nk > 1 ? 1 : 0;
#pragma unroll
    for (int j = 0; j < kLdA; ++j) pa[1][j] = gload_a(j, k1 * BK);
    pas[1] = asrow[k1];
  }

  auto store_a = [&](int buf, const uint4 (&va)[kLdA], float vas) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kLdA; ++j) *reinterpret_cast<uint4*>(&smem[buf][(r0 + 64 * j) * LDB + c16 * 16]) = va[j];
    s_asc[buf][tid] = vas;
  };
  auto store_b = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kLdB; ++j)
      *reinterpret_cast<uint4*>(&smem[buf][(BM + r0 + 64 * j) * LDB + c16 * 16]) = pb[j];
  };
  store_a(0, pa[0], pas[0]);
  store_b(0);
  __syncthreads();

  // fragments: lane l holds row (or column) l % 16, K bytes 32*(l/16) .. +31
  i32x8 fa[NA], fb[4];
  f32x4 sa[NA];
  auto read_a = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NRB; ++i) {
      fa[i] = lds_frag(&smem[buf][(16 * (wm + 2 * i) + lr) * LDB + lk]);
      // scales of this lane's rows 16*(wm + 2i) + 4*(l/16) + 0..3
      sa[i] = *reinterpret_cast<const f32x4*>(&s_asc[buf][16 * (wm + 2 * i) + 4 * (lane >> 4)]);
    }
  };
  auto read_b = [&](int buf, int c) __attribute__((always_inline)) {
    fb[c] = lds_frag(&smem[buf][(BM + bcol[c] + lr) * LDB + lk]);
  };
  auto block = [&](int i, int c, float sw) __attribute__((always_inline)) {
    const f32x4 p = mfma_f8(fa[i], fb[c], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[i][c][e] = __builtin_fmaf(p[e], sa[i][e] * sw, acc[i][c][e]);
  };
  read_a(0);
  read_b(0, 0);
  read_b(0, 1);

  auto kstep = [&](int kt, auto s_c) __attribute__((always_inline)) {
    constexpr int S = decltype(s_c)::value;  // register slot of A(kt), refilled with A(kt+2)
    const int cur = kt & 1;
    const int knext = kt + 1 < nk ? kt + 1 : kt;
    const int knext2 = kt + 2 < nk ? kt + 2 : nk - 1;
    // weights (and their scales) of the next step first, token rows of the
    // step after it last: loads complete in issue order for the wait
    // counter, so waiting for the weights leaves the token rows in flight
#pragma unroll
    for (int j = 0; j < kLdB; ++j) pb[j] = gload_b(j, knext * BK);
    const float sw0 = swc[0], sw1 = swc[1];
    swc[0] = load_ws(0, knext);
    swc[1] = load_ws(1, knext);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kLdA; ++j) pa[S][j] = gload_a(j, knext2 * BK);
    pas[S] = asrow[knext2];
    __builtin_amdgcn_sched_barrier(0);
    // columns 2, 3 are read while columns 0, 1 are multiplied
    read_b(cur, 2);
    read_b(cur, 3);
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < NRB; ++i) block(i, c, sw0);
    __builtin_amdgcn_sched_barrier(0);
    // the next step's operands go to the idle buffer while columns 2, 3 are
    // multiplied (the last step rewrites its own slice: no branch)
    store_a(cur ^ 1, pa[S ^ 1], pas[S ^ 1]);
    store_b(cur ^ 1);
#pragma unroll
    for (int c = 2; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < NRB; ++i) block(i, c, sw1);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    read_a(cur ^ 1);
    read_b(cur ^ 1, 0);
    read_b(cur ^ 1, 1);
  };
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    kstep(kt, std::integral_constant<int, 0>{});
    kstep(kt + 1, std::integral_constant<int, 1>{});
  }
  if (kt < nk) kstep(kt, std::integral_constant<int, 0>{});
  __syncthreads();  // the fragment reads issued after the last step are done

  // D layout of the 16x16 MFMA: element j of lane l is row 4*(l/16) + j,
  // column l%16.
  {
    // h tile (128 x 128 fp32) into LDS, then each row's block is quantised:
    // four lanes per row, 32 columns each
    float* sh = reinterpret_cast<float*>(&smem[0][0]);
#pragma unroll
    for (int i = 0; i < NRB; ++i)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = 16 * (wm + 2 * i) + 4 * (lane >> 4) + e;
          sh[m * kHLd + 32 * wn + 16 * c + lr] = silu_fast(acc[i][c][e]) * acc[i][c + 2][e];
        }
    __syncthreads();
    const int r = tid >> 2, q = tid & 3;
    if (r < t.vrows) {  // the four lanes of a row are in or out together
      float v[32];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const f32x4 x4 = *reinterpret_cast<const f32x4*>(&sh[r * kHLd + 32 * q + 4 * j]);
        v[4 * j] = x4.x; v[4 * j + 1] = x4.y; v[4 * j + 2] = x4.z; v[4 * j + 3] = x4.w;
      }
      float amax = 0.f;
#pragma unroll
      for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
      amax = fmaxf(amax, __uint_as_float(dpp_u32<0xB1>(__float_as_uint(amax))));
      amax = fmaxf(amax, __uint_as_float(dpp_u32<0x4E>(__float_as_uint(amax))));
      const float s = e4m3_block_scale(amax);
      uint32_t w[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        w[j] = e4m3_code(v[4 * j] / s) | (e4m3_code(v[4 * j + 1] / s) << 8) | (e4m3_code(v[4 * j + 2] / s) << 16) |
               (e4m3_code(v[4 * j + 3] / s) << 24);
      uint8_t* dst = static_cast<uint8_t*>(t.c) + (size_t)(t.m0 + r) * t.ldc + t.nt * 128 + 32 * q;
      *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
      *reinterpret_cast<uint4*>(dst + 16) = make_uint4(w[4], w[5], w[6], w[7]);
      if (q == 0) t.c_scale[(size_t)(t.m0 + r) * t.c_sld + t.nt] = s;
    }
  }
}

// Down + gate scale, 256-row tiles: Y[row] = g_row * (h[row] W_down^T), the
// tile's 256 columns W_down rows nt*256 .. +255. NRB is even.
template <int NRB>
__device__ __forceinline__ void down_body_f8(const TileF8& t, uint8_t (*smem)[kBuf2], float (*s_asc)[512],
                                             float* s_gate) {
  static_assert(NRB % 2 == 0, "row blocks stream through two register slots");
  constexpr int BM = BM2, kLdA = 4;  // A rows r0 + 64*j
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int c16 = tid & 7, r0 = tid >> 3;

  // loader: 16-byte pieces of rows r0 + 64*j (128 bytes = one K step each)
  const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(t.a_rows, t.a_bytes);
  const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(t.w, t.w_bytes);
  uint32_t voa[kLdA];
#pragma unroll
  for (int j = 0; j < kLdA; ++j) voa[j] = (uint32_t)a_source_row(t, r0 + 64 * j) * (uint32_t)t.lda + c16 * 16;
  // B rows nt*256 + r0 + 64*j: one VGPR offset for row r0, the other rows'
  // distance (uniform) in the scalar offset; rows past D read row nt*256 + r0
  const uint32_t vob = (uint32_t)(t.nt * BN + r0) * (uint32_t)t.K + c16 * 16;
  uint32_t bd[kLdB];
#pragma unroll
  for (int j = 0; j < kLdB; ++j) bd[j] = (t.nt * BN + 64 * j >= t.D) ? 0u : (uint32_t)(64 * j) * (uint32_t)t.K;
  // row scales: thread tid stages the scale of A row tid % 256 (threads
  // past 256 write a copy that is never read, so the K loop has no branch)
  const float* asrow = t.a_scale + (size_t)a_source_row(t, tid & (BM - 1)) * t.a_sld;
  // weight scale: the 128-row block of W_down holding this wave's 64
  // columns (vector loads one K step ahead)
  int cb = (t.nt * BN + 64 * wn) >> 7;
  if (cb * 128 >= t.D) cb = 0;
  const uint32_t wso = (uint32_t)(cb * t.a_sld) * 4u;
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(t.ws, (uint32_t)(t.D / 128 * t.a_sld) * 4u);
  auto load_ws = [&](int kb) __attribute__((always_inline)) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, 0u, wso + 4u * kb, 0));
  };
  auto gload_a = [&](int j, int k0) __attribute__((always_inline)) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra, voa[j], k0, 0));
  };
  auto gload_b = [&](int j, int k0) __attribute__((always_inline)) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rb, vob, k0 + bd[j], 0));
  };

  // 16 x 16 output blocks: row block i (rows 16*(wm + 2i) ..), column block
  // c (columns 64*wn + 16c ..)
  constexpr int NA = NRB > 0 ? NRB : 1;
  f32x4 acc[NA][4];
#pragma unroll
  for (int i = 0; i < NA; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[i][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  int bcol[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) bcol[c] = 64 * wn + 16 * c;
  const int lr = lane & 15, lk = (lane >> 4) * 32;

  if (tid < BM) s_gate[tid] = (t.gate != nullptr && tid < t.vrows) ? t.gate[t.m0 + tid] : 1.0f;

  const int nk = t.K / BK;
  uint4 pa[kLdA], pb[kLdB];
  float pas;
#pragma unroll
  for (int j = 0; j < kLdA; ++j) pa[j] = gload_a(j, 0);
  pas = asrow[0];
#pragma unroll
  for (int j = 0; j < kLdB; ++j) pb[j] = gload_b(j, 0);
  float swc = load_ws(0);  // weight scale of the step being multiplied

  auto store_a = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kLdA; ++j) *reinterpret_cast<uint4*>(&smem[buf][(r0 + 64 * j) * LDB + c16 * 16]) = pa[j];
    s_asc[buf][tid] = pas;
  };
  auto store_b = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kLdB; ++j)
      *reinterpret_cast<uint4*>(&smem[buf][(BM + r0 + 64 * j) * LDB + c16 * 16]) = pb[j];
  };
  store_a(0);
  store_b(0);
  __syncthreads();

  // fragments: lane l holds row (or column) l % 16, K bytes 32*(l/16) .. +31;
  // the four B fragments are held for the whole step, the A fragments (and
  // the four row scales of each) stream through two slots, one row block
  // ahead of its MFMAs
  i32x8 fa[2], fb[4];
  f32x4 sa[2];
  auto read_a = [&](int buf, int i, int slot) __attribute__((always_inline)) {
    fa[slot] = lds_frag(&smem[buf][(16 * (wm + 2 * i) + lr) * LDB + lk]);
    // scales of this lane's rows 16*(wm + 2i) + 4*(l/16) + 0..3
    sa[slot] = *reinterpret_cast<const f32x4*>(&s_asc[buf][16 * (wm + 2 * i) + 4 * (lane >> 4)]);
  };
  auto read_b = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 4; ++c) fb[c] = lds_frag(&smem[buf][(BM + bcol[c] + lr) * LDB + lk]);
  };
  // row block i: four MFMAs on slot `slot`, each partial sum added to the
  // accumulators times (row scale x weight scale)
  auto block = [&](int i, int slot, float sw) __attribute__((always_inline)) {
    f32x4 s0;
#pragma unroll
    for (int e = 0; e < 4; ++e) s0[e] = sa[slot][e] * sw;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4 p = mfma_f8(fa[slot], fb[c], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][c][e] = __builtin_fmaf(p[e], s0[e], acc[i][c][e]);
    }
  };
  read_b(0);
  if (NRB > 0) read_a(0, 0, 0);

  auto kstep = [&](int kt) __attribute__((always_inline)) {
    const int cur = kt & 1;
    const int knext = kt + 1 < nk ? kt + 1 : kt;  // the last step reloads its own slice: no branch
    // weights (and their scales) first, token rows after: loads complete in
    // issue order for the wait counter
#pragma unroll
    for (int j = 0; j < kLdB; ++j) pb[j] = gload_b(j, knext * BK);
    const float sw = swc;
    swc = load_ws(knext);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kLdA; ++j) pa[j] = gload_a(j, knext * BK);
    pas = asrow[knext];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NRB; ++i) {
      if (i + 1 < NRB) read_a(cur, i + 1, (i + 1) & 1);
      // the next step's tile goes to the idle buffer behind the second half
      // of this step's row blocks
      if (i == (NRB > 2 ? NRB - 2 : NRB / 2)) {
        store_a(cur ^ 1);
        store_b(cur ^ 1);
      }
      block(i, i & 1, sw);
    }
    if (NRB == 0) {
      store_a(cur ^ 1);
      store_b(cur ^ 1);
    }
    __syncthreads();
    read_b(cur ^ 1);
    if (NRB > 0) read_a(cur ^ 1, 0, 0);
  };
  for (int kt = 0; kt < nk; ++kt) kstep(kt);
  __syncthreads();  // the fragment reads issued after the last step are done

  // D layout of the 16x16 MFMA: element j of lane l is row 4*(l/16) + j,
  // column l%16.
  {
    // y tile (256 x 256 bf16) staged through LDS, then written as 16-byte
    // pieces of each row. Rows e, e+1 (e even) of a lane are adjacent rows of
    // one column; an even lane swaps its row-(e+1) value for its odd
    // neighbour's row-e value (DPP quad permute 1,0,3,2), so each lane writes
    // two adjacent columns of one row as one 32-bit word.
    uint16_t* so = reinterpret_cast<uint16_t*>(&smem[0][0]);
    const bool odd = lane & 1;
#pragma unroll
    for (int i = 0; i < NRB; ++i) {
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const int m = 16 * (wm + 2 * i) + 4 * (lane >> 4) + e;
        const float g0 = s_gate[m], g1 = s_gate[m + 1];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t b0 = f32_to_bf16(g0 * acc[i][c][e]), b1 = f32_to_bf16(g1 * acc[i][c][e + 1]);
          const uint32_t rr = (uint32_t)__builtin_amdgcn_mov_dpp((int)(odd ? b0 : b1), 0xB1, 0xF, 0xF, false);
          const int col = 64 * wn + 16 * c + lr;
          const uint32_t w = odd ? (rr | (b1 << 16)) : (b0 | (rr << 16));
          *reinterpret_cast<uint32_t*>(&so[(m + (odd ? 1 : 0)) * kYLd + (col & ~1)]) = w;
        }
      }
    }
    __syncthreads();
    const int q = tid & 31;  // 16-byte piece of a row
    const int col = t.nt * BN + 8 * q;
    if (col < t.D) {  // D % 128 == 0: a piece is wholly inside or outside
      uint16_t* cy = static_cast<uint16_t*>(t.c);
#pragma unroll 4
      for (int r = tid >> 5; r < t.vrows; r += 16)
        *reinterpret_cast<uint4*>(cy + (size_t)(t.m0 + r) * t.ldc + col) =
            *reinterpret_cast<const uint4*>(&so[r * kYLd + 8 * q]);
    }
  }
}

// kMode 0: gate/up + SwiGLU + h quantisation, 1: down + gate scale
template <int kMode>
__global__ __launch_bounds__(512) void grouped_gemm_f8_kernel(ExpertGemmArgs a) {
  constexpr int BM = kMode == 0 ? BM1 : BM2;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2][buf_bytes(BM)];
  __shared__ __attribute__((aligned(16))) float s_asc[2][512];  // row scales (entries 0..BM-1 used)
  __shared__ int32_t s_pre[kMaxExperts + 2];
  __shared__ int32_t s_off[kMaxExperts + 1];
  __shared__ float s_gate[BM];

  // runs of kRun consecutive tiles, run r on XCD r % 8 (block b runs on XCD b % 8)
  const int total = a.pre[a.E + 1];
  const int bid = blockIdx.x;
  const int slot = bid >> 3;
  const int tile = ((slot / kRun) * 8 + (bid & 7)) * kRun + slot % kRun;
  if (tile >= total) return;

  for (int i = threadIdx.x; i < a.E + 2; i += blockDim.x) s_pre[i] = a.pre[i];
  for (int i = threadIdx.x; i < a.E + 1; i += blockDim.x) s_off[i] = a.offsets[i];
  __syncthreads();
  // workgroup-uniform values (scalar registers)
  const int p = __builtin_amdgcn_readfirstlane(find_problem(s_pre, a.E, tile));
  const bool routed = p < a.E;
  const int rows = __builtin_amdgcn_readfirstlane(routed ? s_off[p + 1] - s_off[p] : a.T);
  const int row_base = __builtin_amdgcn_readfirstlane(routed ? s_off[p] : 0);
  const int local = __builtin_amdgcn_readfirstlane(tile - s_pre[p]);
  TileF8 t;
  t.Hp = routed ? a.H : a.Hs;
  t.D = a.D;
  const int nmt = (rows + BM - 1) / BM;
  const int rpt = ((rows + nmt - 1) / nmt + 31) & ~31;
  t.m0 = (local % nmt) * rpt;
  t.nt = local / nmt;
  t.K = (kMode == 0) ? a.D : t.Hp;
  t.vrows = min(rows - t.m0, rpt);
  t.a_sld = t.K / 128;
  if (kMode == 0) {
    t.a_rows = static_cast<const uint8_t*>(a.a);
    t.lda = a.D;
    t.tok = routed ? a.row_token + row_base : nullptr;
    t.a_scale = a.a_scale;  // x scales, indexed by token
    t.w = routed ? static_cast<const uint8_t*>(a.w) + (size_t)p * 2 * t.Hp * a.D
                 : static_cast<const uint8_t*>(a.w_shared);
    t.ws = routed ? a.w_scale + (size_t)p * (2 * t.Hp / 128) * t.a_sld : a.w_shared_scale;
    t.c = routed ? static_cast<void*>(static_cast<uint8_t*>(a.c) + (size_t)row_base * a.H) : a.c_shared;
    t.c_scale = routed ? a.c_scale + (size_t)row_base * (a.H / 128) : a.c_shared_scale;
    t.c_sld = t.Hp / 128;
    t.ldc = t.Hp;
    t.gate = nullptr;
    t.a_bytes = (uint32_t)((size_t)a.x_rows * a.D);
    t.w_bytes = (uint32_t)((size_t)2 * t.Hp * a.D);
  } else {
    t.a_rows = routed ? static_cast<const uint8_t*>(a.a) + (size_t)row_base * a.H
                      : static_cast<const uint8_t*>(a.a_shared);
    t.lda = t.Hp;
    t.tok = nullptr;
    t.a_scale = routed ? a.a_scale + (size_t)row_base * (a.H / 128) : a.a_shared_scale;
    t.w = routed ? static_cast<const uint8_t*>(a.w) + (size_t)p * a.D * t.Hp
                 : static_cast<const uint8_t*>(a.w_shared);
    t.ws = routed ? a.w_scale + (size_t)p * (a.D / 128) * t.a_sld : a.w_shared_scale;
    t.c = routed ? static_cast<void*>(static_cast<uint16_t*>(a.c) + (size_t)row_base * a.D) : a.c_shared;
    t.c_scale = nullptr;
    t.c_sld = 0;
    t.ldc = a.D;
    t.gate = routed ? a.row_gate + row_base : nullptr;
    t.a_bytes = (uint32_t)((size_t)rows * t.Hp);
    t.w_bytes = (uint32_t)((size_t)a.D * t.Hp);
  }

  // valid 16-row blocks of this wave: wm + 2*i for i < nrb
  const int wm = (threadIdx.x >> 6) >> 2;
  int nrb = 0;
#pragma unroll
  for (int i = 0; i < BM / 32; ++i) nrb += (16 * (wm + 2 * i) < t.vrows) ? 1 : 0;
  if constexpr (kMode == 0) {
    switch (nrb) {
      case 4: gateup_body_f8<4>(t, smem, s_asc); break;
      case 3: gateup_body_f8<3>(t, smem, s_asc); break;
      case 2: gateup_body_f8<2>(t, smem, s_asc); break;
      case 1: gateup_body_f8<1>(t, smem, s_asc); break;
      default: gateup_body_f8<0>(t, smem, s_asc); break;
    }
  } else {
    // rounded up to an even count: five instantiations, not nine
    switch ((nrb + 1) & ~1) {
      case 8: down_body_f8<8>(t, smem, s_asc, s_gate); break;
      case 6: down_body_f8<6>(t, smem, s_asc, s_gate); break;
      case 4: down_body_f8<4>(t, smem, s_asc, s_gate); break;
      case 2: down_body_f8<2>(t, smem, s_asc, s_gate); break;
      default: down_body_f8<0>(t, smem, s_asc, s_gate); break;
    }
  }
}

namespace {
int grouped_blocks_f8(int max_items) {
  const int runs = (max_items + kRun - 1) / kRun;
  return ((runs + 7) / 8) * 8 * kRun;
}
}  // namespace

hipError_t launch_grouped_gateup_f8(const ExpertGemmArgs& a, hipStream_t s) {
  const int blocks = grouped_blocks_f8(a.max_items);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_gemm_f8_kernel<0>), dim3(blocks), dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_grouped_down_f8(const ExpertGemmArgs& a, hipStream_t s) {
  const int blocks = grouped_blocks_f8(a.max_items);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_gemm_f8_kernel<1>), dim3(blocks), dim3(512), 0, s, a);
  return hipGetLastError();
}

MOE_DEBUG_READER(debug_read_f8)

}  // namespace moe
