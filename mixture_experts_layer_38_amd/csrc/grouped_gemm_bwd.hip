// Backward pass of the layer (the back-propagation step of the training data
// flow in the "Transformer block" article): gradients of L = <d_out, out> with
// respect to x, gate_w and the routed and shared expert weights, with the
// expert choice held fixed and the gradient reaching the router through the
// gate values.
//
// Every product is one grouped bf16 MFMA GEMM C[m][n] = sum_k A[m][k] B[n][k]
// (fp32 accumulation) over 256 x 256 tiles, K step 64, 8 waves (two per SIMD)
// of 128 x 64 (4 x 2 blocks of v_mfma_f32_32x32x16_bf16), operands staged
// through two LDS buffers. The right operand is always stored k-major
// (B[n][k] = stored[k][n]: the weights read "the other way" than the
// forward, or activations summed over rows for the weight gradients) and
// keeps that layout in LDS: a thread loads 4 k-rows x 8 consecutive n (four
// 16-byte loads) and writes them as they are; the MFMA fragments (8
// consecutive k of one column) are then read with gfx950's transposing LDS
// read, two per fragment. The left operand is either natural (k contiguous,
// [row][k] in LDS, 16-byte chunks) or k-major and staged the same way as
// the right one. k-major operands past the valid K (an expert's ragged row
// count) are zero-filled, so the weight gradients of experts with few rows
// come out exact.
//
//   kDgradH   dH   = dOut[tok] W_down          (rows x H; epilogue: SwiGLU
//                                                backward -> [dA | dU], and
//                                                the partial sums of dL/dg)
//   kDgradX   dXr  = [dA | dU] [W_gate; W_up]  (rows x D, bf16)
//   kWgradD   dW_down = dOut[tok]^T (g h)      (D x H per expert, fp32)
//   kWgradGU  dW_gu   = [dA | dU]^T x[tok]     (2H x D per expert, fp32)
//   kRouterW  d gate_w = dlogit^T x            (E x D, split over T, fp32 planes)
//   kRouterX  dx_r     = dlogit gate_w         (T x D, fp32)
#include <type_traits>

#include <algorithm>
#include <type_traits>

#include "moe_internal.hpp"

namespace moe {

namespace {
constexpr int BM = 256, BN = 256, BK = 64, LDK = BK + 8;  // LDS row: 72 bf16 (144 bytes)
constexpr int kRowsL = BM + BN;
constexpr int kThreads = 512;
// The four expert GEMMs hand tiles out in runs of kRunB consecutive tile
// indices per XCD (block b runs on XCD b % 8; run r goes to XCD r % 8), so
// the tiles that share operand slices share that XCD's L2.
constexpr int kRunB = 32;
__device__ __forceinline__ int run_tile(int bid) {
  const int slot = bid >> 3;
  return ((slot / kRunB) * 8 + (bid & 7)) * kRunB + slot % kRunB;
}

enum : int { kDgradH = 0, kDgradX = 1, kWgradD = 2, kWgradGU = 3, kRouterW = 4, kRouterX = 5 };

struct BwdTile {
  const uint16_t* a;   // A storage (natural: rows m; k-major: rows k)
  const int32_t* amap; // row map of A's storage rows (null = identity)
  uint32_t a_bytes;
  int lda;
  const uint16_t* b;   // B storage, k-major (rows k)
  const int32_t* bmap;
  uint32_t b_bytes;
  int ldb;
  int M, N, K;         // valid extents
  int m0, n0, k0, k1;  // tile origin; K range [k0, k1)
  void* c;             // output (row m0 / col n0 not applied)
  int ldc;
  // kDgradH epilogue
  const uint16_t* au;  // [a | u] rows
  const float* gate;   // row gates (null = 1)
  float* part;         // partial dL/dg sums, [rows][npart]
  int npart, Hp;
};

__device__ __forceinline__ uint4 bload(const __amdgpu_buffer_rsrc_t& r, uint32_t voff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

__host__ __device__ constexpr int cdiv(int x, int y) { return (x + y - 1) / y; }

// Tile fields are the same in every lane; saying so keeps the buffer
// descriptors built from them in scalar registers (a descriptor the compiler
// cannot prove uniform costs a loop over its distinct values at every load).
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ uint32_t uniform_u32(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef short v4s8 __attribute__((ext_vector_type(8)));

// LDS layout: row r holds its 64 k values as eight 16-byte chunks, chunk c at
// position c ^ ((r >> 4) & 7) (rows padded to 144 bytes). With this swizzle
// the fragment reads (16 rows x one chunk per 16 lanes) and the transposed
// 8-byte stores (rows 8 apart, 4 k each) both fall on distinct banks.
__device__ __forceinline__ int lds_at(int r, int k) { return r * LDK + ((((k >> 3) ^ (r >> 4)) & 7) << 3) + (k & 7); }

// k-major operands (stored with k-rows in memory) keep that layout in LDS:
// row k holds the tile's 256 m (or n) values, rows 576 bytes apart (16 banks
// of offset per row). An MFMA fragment (8 consecutive k of one column) is
// read with two transposing reads (ds_read_b64_tr_b16): in each group of 16
// lanes, lane s names 4 values of row k0 + s/4 at column c0 + 4(s%4), and
// receives column c0 + s at rows k0 .. k0 + 3.
constexpr int KLD = BM + 32;
static_assert(BK * KLD == BM * LDK, "a k-major operand fills the same LDS as a natural one");
typedef short v4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8 lds_frag_tr(const uint16_t* base, int c0, int kk, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int k0 = kk + 8 * (g >> 1), col = c0 + 16 * (g & 1) + 4 * (s & 3);
  const uint16_t* p0 = base + (k0 + (s >> 2)) * KLD + col;
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4s __attribute__((address_space(3)))*)p0);
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4s __attribute__((address_space(3)))*)(p0 + 4 * KLD));
  const v4s8 u = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, u);
}
}  // namespace

// The tiles of one workgroup, in order: the first is t; with kPersist, next(tn)
// supplies the following ones (false when none is left). The loader state
// (buffer resources, row maps, offsets) belongs to the tile being loaded,
// which during a tile's last K step is already the next tile: that step
// requests the next tile's first slice instead of nothing, so the first
// loads of a tile overlap the previous tile's last MFMAs and epilogue.
template <int kMode, bool kAT, bool kPersist, int NRB, class Next>
__device__ __forceinline__ void bwd_tiles(BwdTile t, Next&& next, uint16_t (*smem)[kRowsL * LDK], float* s_red) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  // natural loader: rows r0 + 64j, 16-byte chunk c8 of the 64-wide K step
  const int c8 = tid & 7, r0 = tid >> 3;
  // k-major loader: k rows 4*kg .. +3 of the step, columns 8*mg .. +7 of the tile
  const int kg = tid >> 5, mg = tid & 31;

  // loader state of the tile being loaded
  __amdgpu_buffer_rsrc_t ra, rb, rma, rmb;
  bool has_amap, has_bmap;
  uint32_t aoff[4], acol, bcol;
  int lk0, lk1, llda, lldb;
  auto init_loader = [&](const BwdTile& L) __attribute__((always_inline)) {
    ra = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(const_cast<uint16_t*>(L.a)), (short)0, uniform_u32(L.a_bytes),
                                           0x00020000);
    rb = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(const_cast<uint16_t*>(L.b)), (short)0, uniform_u32(L.b_bytes),
                                           0x00020000);
    if (!kAT) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int m = L.m0 + r0 + 64 * j;
        m = m < L.M ? m : L.M - 1;
        const int row = L.amap ? L.amap[m] : m;
        aoff[j] = ((uint32_t)row * (uint32_t)L.lda + c8 * 8) * 2u;
      }
    }
    // k-major operands: byte offset of column 8*mg (rows added per step)
    acol = (uint32_t)(L.m0 + 8 * mg) * 2u;
    bcol = (uint32_t)(L.n0 + 8 * mg) * 2u;
    // The row maps are read through buffer resources, an absent map through
    // one of zero length (its reads return 0 and are replaced by the
    // identity), so the reads are unconditional: a branch around them would
    // split the step's scheduling region.
    has_amap = L.amap != nullptr;
    has_bmap = L.bmap != nullptr;
    rma = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(const_cast<int32_t*>(has_amap ? L.amap : reinterpret_cast<const int32_t*>(L.a))), (short)0,
        uniform_u32(has_amap ? (uint32_t)L.k1 * 4u : 0u), 0x00020000);
    rmb = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(const_cast<int32_t*>(has_bmap ? L.bmap : reinterpret_cast<const int32_t*>(L.b))), (short)0,
        uniform_u32(has_bmap ? (uint32_t)L.k1 * 4u : 0u), 0x00020000);
    lk0 = (int)uniform_u32((uint32_t)L.k0);
    lk1 = (int)uniform_u32((uint32_t)L.k1);
    llda = (int)uniform_u32((uint32_t)L.lda);
    lldb = (int)uniform_u32((uint32_t)L.ldb);
  };

  uint4 sa_[4], sb_[4];
  // storage rows of this thread's 4 k-rows of a step (through the row map
  // for gathered operands), found one step before their data is requested so
  // the map read and the row read are not a chain of two loads in one step
  struct KRows {
    int row[4];
    int ok;  // bit q: k-row q is inside [k0, k1) (else zero-filled)
  };
  auto krows = [&](const __amdgpu_buffer_rsrc_t& rm, bool has_map, int k0) __attribute__((always_inline)) {
    KRows r;
    r.ok = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k = k0 + 4 * kg + q;
      const bool ok = k < lk1;
      const int kk = ok ? k : lk0;
      const int v = (int)__builtin_amdgcn_raw_buffer_load_b32(rm, (uint32_t)kk * 4u, 0, 0);
      r.row[q] = has_map ? v : kk;
      r.ok |= (ok ? 1 : 0) << q;
    }
    return r;
  };
  // k-rows past the end are zero-filled when the data is written to LDS, not
  // when it arrives, so nothing waits for a load before the step's MFMAs
  auto load_kmajor = [&](const __amdgpu_buffer_rsrc_t& r, const KRows& kr, int ld, uint32_t col,
                         uint4 (&v)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = bload(r, (uint32_t)kr.row[q] * (uint32_t)ld * 2u + col);
  };
  KRows kra, krb;  // rows of the next load
  int oka = 0, okb = 0;  // valid k-rows of the loaded data
  auto load_a = [&](int k0) __attribute__((always_inline)) {
    if (kAT) {
      load_kmajor(ra, kra, llda, acol, sa_);
      oka = kra.ok;
      kra = krows(rma, has_amap, k0 + BK);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) sa_[j] = bload(ra, aoff[j] + (uint32_t)k0 * 2u);
    }
  };
  auto load_b = [&](int k0) __attribute__((always_inline)) {
    load_kmajor(rb, krb, lldb, bcol, sb_);
    okb = krb.ok;
    krb = krows(rmb, has_bmap, k0 + BK);
  };
  // 4 k-rows x 8 columns -> rows 4kg + q of the k-major LDS layout
  auto store_kmajor = [&](uint16_t* base, const uint4 (&vin)[4], int ok) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<uint4*>(&base[(4 * kg + q) * KLD + 8 * mg]) = ((ok >> q) & 1) ? vin[q] : make_uint4(0u, 0u, 0u, 0u);
  };
  auto store = [&](int buf) __attribute__((always_inline)) {
    if (kAT) {
      store_kmajor(&smem[buf][0], sa_, oka);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<uint4*>(&smem[buf][lds_at(r0 + 64 * j, c8 * 8)]) = sa_[j];
    }
    store_kmajor(&smem[buf][BM * LDK], sb_, okb);
  };

  // this wave's valid 32-row blocks (rows 128 wm + 32 i, i < NRB): blocks
  // past a ragged tile's last row cost no MFMA
  constexpr int NA = NRB > 0 ? NRB : 1;
  f32x16 acc[NA][2];
  const int lr = lane & 31, lk = (lane >> 5) * 8;
  // Fragments are double-buffered across the four 16-wide substeps: the LDS
  // reads of substep s+1 are issued before the MFMAs of substep s.
  bf16x8 fa[2][4], fb[2][2];
  auto read_frags = [&](const uint16_t* sbuf, int kk, int slot) __attribute__((always_inline)) {
    const uint16_t* sA = sbuf;
    const uint16_t* sB = sbuf + BM * LDK;
#pragma unroll
    for (int i = 0; i < NRB; ++i)
      fa[slot][i] = kAT ? lds_frag_tr(sA, 128 * wm + 32 * i, kk, lane)
                        : *reinterpret_cast<const bf16x8*>(&sA[lds_at(128 * wm + 32 * i + lr, kk + lk)]);
#pragma unroll
    for (int c = 0; c < 2; ++c) fb[slot][c] = lds_frag_tr(sB, 64 * wn + 32 * c, kk, lane);
  };
  // the rows of a tile's first step (then one step ahead, inside load_a/load_b)
  auto first_rows = [&]() __attribute__((always_inline)) {
    if (kAT) kra = krows(rma, has_amap, lk0);
    krb = krows(rmb, has_bmap, lk0);
  };

  // first tile: its first step (a tile without rows loads row 0, zero-filled)
  init_loader(t);
  first_rows();
  load_a(t.k0);
  load_b(t.k0);
  store(0);
  __syncthreads();
  read_frags(smem[0], 0, 0);
  int b0 = 0;  // LDS buffer holding the current tile's first step
  while (true) {
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][c][e] = 0.f;
    const int nk = (t.k1 - t.k0 + BK - 1) / BK;
    BwdTile tn = t;  // the next tile, found just before the last step (no registers held across the loop)
    bool more = false;
    // one K step: the next step's operands are requested (A's between the
    // MFMAs of substep 0, B's between those of substep 1: a request that
    // cannot enter a full memory queue stalls the wave, and the MFMAs behind
    // it with it) and written to the idle buffer after the MFMAs. The last
    // step requests the next tile's first step (persistent); the last step
    // of a workgroup's only tile requests and stages nothing (decided at
    // compile time: no branch around the loads; the epilogue that follows
    // starts with a barrier of its own).
    auto kstep = [&](int kt, auto last_c) __attribute__((always_inline)) {
      constexpr bool kLast = decltype(last_c)::value;
      constexpr bool kIdle = kLast && !kPersist;
      const int cur = (b0 + kt) & 1;
      int kn = t.k0 + (kt + 1) * BK;
      if constexpr (kLast) {
        if constexpr (kPersist) {
          init_loader(tn);
          first_rows();
          kn = tn.k0;
        }
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (s == 0 && !kIdle) load_a(kn);
        if (s == 1 && !kIdle) load_b(kn);
        if (s < 3) read_frags(smem[cur], 16 * (s + 1), (s + 1) & 1);
        if (s == 3 && !kIdle) store(cur ^ 1);  // the next step's operands, behind this substep's MFMAs
#pragma unroll
        for (int i = 0; i < NRB; ++i)
#pragma unroll
          for (int c = 0; c < 2; ++c)
            acc[i][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s & 1][i], fb[s & 1][c], acc[i][c], 0, 0, 0);
        if (s == 3) {
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
          }
        }
        if (s < 2) {
          // (MFMA, LDS read, global load) x 6, then (MFMA, global load) x 2
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (q < 6) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          }
        } else if (s == 2) {
#pragma unroll
          for (int q = 0; q < 6; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (!kIdle) {
        __syncthreads();
        read_frags(smem[cur ^ 1], 0, 0);
      }
    };
    for (int kt = 0; kt + 1 < nk; ++kt) kstep(kt, std::false_type{});
    if constexpr (kPersist) more = next(tn);
    if (nk > 0) {
      kstep(nk - 1, std::true_type{});
    } else if (kPersist) {
      // a tile without rows (zero gradient): the next tile's first step now
      init_loader(tn);
      first_rows();
      load_a(tn.k0);
      load_b(tn.k0);
      store(b0 ^ 1);
      __syncthreads();
      read_frags(smem[b0 ^ 1], 0, 0);
    }
    b0 = (b0 + (nk > 0 ? nk : 1)) & 1;

  // D layout of the 32x32 MFMA: element e of lane l is row 8*(e/4) + 4*(l/32) + e%4,
  // column l%32.
  if (kMode == kDgradH) {
    // dH = g * acc; [dA | dU] = dH * u * SiLU'(a) | dH * SiLU(a); the row's
    // partial dL/dg = sum over this tile's columns of acc * SiLU(a) * u.
    // One half of the tile's rows (those of one row-wave) at a time: its a
    // and u rows and gates are staged in LDS with 16-byte loads (LDS row r:
    // the tile's 256 a values, then its 256 u values), the half's waves
    // replace a and u by dA and dU there, and the rows leave as 16-byte
    // pieces (element-wise global accesses here would make every element
    // wait for its own loads).
    constexpr int kLdh = 2 * BN + 8;  // LDS row: a, then u (bf16)
    constexpr int kHalf = BM / 2;
    static_assert(kHalf * kLdh * 2 + kHalf * 4 + 8 * BM * 4 <= 2 * kRowsL * LDK * 2,
                  "a, u, gates and the row sums fit the operand buffers");
    uint16_t* sAU = &smem[0][0];
    float* sG = reinterpret_cast<float*>(sAU + kHalf * kLdh);
    float* sR = sG + kHalf;  // [8][BM] row partial sums (column wave, lane half)
    // a thread moves 16-byte piece pc = tid % 64 of rows tid / 64 + 8j: one
    // VGPR offset (its column; pieces past N get an offset past the buffer,
    // which reads 0 and writes nothing), the row in the scalar offset; a
    // wave's 64 lanes cover one row, so the row test is uniform
    const int pc = tid & 63, rw = tid >> 6;
    const uint32_t vcol = (t.n0 + 8 * (pc & 31) < t.N)
                              ? (uint32_t)((pc >= 32 ? t.Hp : 0) + t.n0 + 8 * (pc & 31)) * 2u
                              : 0x80000000u;
    const __amdgpu_buffer_rsrc_t rau = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(const_cast<uint16_t*>(t.au)), (short)0, uniform_u32((uint32_t)((size_t)t.M * 2 * t.Hp * 2)),
        0x00020000);
    const __amdgpu_buffer_rsrc_t rdau = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(static_cast<uint16_t*>(t.c)), (short)0, uniform_u32((uint32_t)((size_t)t.M * t.ldc * 2)),
        0x00020000);
    __syncthreads();  // every wave is past its last fragment reads
#pragma unroll 1
    for (int h = 0; h < 2; ++h) {
      const int mh = t.m0 + kHalf * h;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        uint4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int m = mh + rw + 8 * (8 * b + j);
          v[j] = make_uint4(0u, 0u, 0u, 0u);
          if (m < t.M)
            v[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rau, vcol, (uint32_t)m * (uint32_t)(2 * t.Hp) * 2u, 0));
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
          *reinterpret_cast<uint4*>(sAU + (rw + 8 * (8 * b + j)) * kLdh + 8 * pc) = v[j];
      }
      if (tid < kHalf) sG[tid] = (t.gate != nullptr && mh + tid < t.M) ? t.gate[mh + tid] : 1.0f;
      __syncthreads();
      if (wm == h) {
        // this lane's rows 32i + 8(e/4) + 4(l/32) + e%4 of the half, columns
        // 64wn + 32c + l%32; offsets from two per-lane bases (rows below and
        // from 64), so every access has an immediate offset
        const int lim = t.M - mh - 4 * (lane >> 5);  // row offsets ro < lim are valid rows
        uint16_t* lb0 = sAU + (4 * (lane >> 5)) * kLdh + 64 * wn + lr;
        uint16_t* lb1 = lb0 + 64 * kLdh;
        const float* gb = sG + 4 * (lane >> 5);
        float* rb = sR + (wn * 2 + ((lane >> 4) & 1)) * BM + kHalf * h + 4 * (lane >> 5);
        const bool col_ok[2] = {t.n0 + 64 * wn + lr < t.N, t.n0 + 64 * wn + 32 + lr < t.N};
#pragma unroll
        for (int i = 0; i < NRB; ++i)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int ro = 32 * i + 8 * (e >> 2) + (e & 3);  // row offset from the lane's base row
            uint16_t* ep = (i < 2 ? lb0 : lb1) + (32 * (i & 1) + 8 * (e >> 2) + (e & 3)) * kLdh;
            float sum = 0.f;
            if (ro < lim) {
              const float g = gb[ro];
#pragma unroll
              for (int c = 0; c < 2; ++c) {
                if (!col_ok[c]) continue;
                const float av = bf16f(ep[32 * c]);
                const float uv = bf16f(ep[BN + 32 * c]);
                const float sg = 1.0f / (1.0f + __expf(-av));
                const float sl = av * sg;
                const float dh = g * acc[i][c][e];
                ep[32 * c] = (uint16_t)f32_to_bf16(dh * uv * sg * (1.0f + av * (1.0f - sg)));
                ep[BN + 32 * c] = (uint16_t)f32_to_bf16(dh * sl);
                sum += acc[i][c][e] * sl * uv;
              }
            }
            // sum over the 32 lanes of a row group: 16-lane rows by DPP, then
            // the two rows and the four column waves through LDS, in a fixed
            // order
            float v = sum;
            v += __uint_as_float(dpp_u32<0xB1>(__float_as_uint(v)));
            v += __uint_as_float(dpp_u32<0x4E>(__float_as_uint(v)));
            v += __uint_as_float(dpp_u32<0x141>(__float_as_uint(v)));
            v += __uint_as_float(dpp_u32<0x140>(__float_as_uint(v)));
            if ((lane & 15) == 0) rb[ro] = v;
          }
      }
      __syncthreads();
      // dA and dU rows of this half, 16-byte pieces
#pragma unroll 4
      for (int j = 0; j < 16; ++j) {
        const int m = mh + rw + 8 * j;
        if (m < t.M)
          __builtin_amdgcn_raw_buffer_store_b128(
              __builtin_bit_cast(v4u, *reinterpret_cast<const uint4*>(sAU + (rw + 8 * j) * kLdh + 8 * pc)), rdau,
              vcol, (uint32_t)m * (uint32_t)t.ldc * 2u, 0);
      }
      __syncthreads();
    }
    if (tid < BM && t.m0 + tid < t.M) {
      float v = 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) v += sR[q * BM + tid];
      t.part[(size_t)(t.m0 + tid) * t.npart + t.n0 / BN] = v;
    }
  } else if (kMode == kDgradX) {
    // bf16 tile staged through LDS (rows of 264 elements over both buffers),
    // then written as full 16-byte pieces of each 512-byte row. Rows e, e+1
    // (e even) of a lane are adjacent rows of one column; an even lane swaps
    // its row-(e+1) value for its odd neighbour's row-e value (DPP quad
    // permute 1,0,3,2), so each lane writes two adjacent columns of one row
    // as one 32-bit word.
    constexpr int kLdo = BN + 8;
    static_assert(BM * kLdo <= 2 * kRowsL * LDK, "staging tile fits the two LDS buffers");
    uint16_t* so = &smem[0][0];
    const bool odd = lane & 1;
    __syncthreads();  // every wave is past its last fragment reads
#pragma unroll
    for (int i = 0; i < NRB; ++i)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          const int r = 128 * wm + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          const uint32_t b0 = f32_to_bf16(acc[i][c][e]), b1 = f32_to_bf16(acc[i][c][e + 1]);
          const uint32_t x = (uint32_t)__builtin_amdgcn_mov_dpp((int)(odd ? b0 : b1), 0xB1, 0xF, 0xF, false);
          const uint32_t w = odd ? (x | (b1 << 16)) : (b0 | (x << 16));
          const int col = 64 * wn + 32 * c + lr;
          *reinterpret_cast<uint32_t*>(&so[(r + (odd ? 1 : 0)) * kLdo + (col & ~1)]) = w;
        }
    __syncthreads();
    const int q = tid & 31;  // 16-byte piece of a row
    const int n = t.n0 + 8 * q;
    if (n < t.N) {  // N % 128 == 0: a piece is wholly inside or outside
#pragma unroll 4
      for (int r = tid >> 5; r < BM; r += 16) {
        if (t.m0 + r >= t.M) break;
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(t.c) + (size_t)(t.m0 + r) * t.ldc + n) =
            *reinterpret_cast<const uint4*>(&so[r * kLdo + 8 * q]);
      }
    }
  } else {
    // fp32 weight gradient: each wave stages one 32 x 64 block at a time in
    // its own part of the LDS buffer its last K step was read from (the next
    // tile's first step is in buffer b0), reads it back as 16-byte row
    // pieces and writes those (N % 128 == 0: a piece is wholly inside or
    // outside). The block's values leave in a quarter of the store
    // instructions that one 4-byte store per value takes. Only the wave's own
    // lanes share its part, so wavefront fences order the writes and the
    // reads; the barrier after the loop keeps the next tile's first writes to
    // this buffer behind every wave's last reads.
    constexpr int kLdw = 64 + 4;  // staged row: 64 fp32, 4 of padding
    static_assert(8 * 32 * kLdw * 4 <= kRowsL * LDK * 2, "eight 32 x 64 fp32 blocks fit one operand buffer");
    if constexpr (!kPersist) __syncthreads();  // every wave is past its last fragment reads
    float* sw = reinterpret_cast<float*>(&smem[b0 ^ 1][0]) + wave * (32 * kLdw);
    // the lane index taken afresh here, made opaque so that nothing derived
    // from it is hoisted to live across the K loop
    int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    asm volatile("" : "+v"(ln));
    const int pr = ln >> 4, pq = ln & 15;  // read-back: rows pr + 4j, 16-byte piece pq
    const int n = t.n0 + 64 * wn + 4 * pq;
    float* swl = sw + (4 * (ln >> 5)) * kLdw + (ln & 31);  // this lane's first staged value
#pragma unroll
    for (int i = 0; i < NRB; ++i) {
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) swl[(8 * (e >> 2) + (e & 3)) * kLdw + 32 * c] = acc[i][c][e];
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = pr + 4 * j;
        const int m = t.m0 + 128 * wm + 32 * i + r;
        const f32x4 v = *reinterpret_cast<const f32x4*>(&sw[r * kLdw + 4 * pq]);
        if (m < t.M && n < t.N)
          __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(static_cast<float*>(t.c) + (size_t)m * t.ldc + n));
        // at most four pieces in registers; after the last, the next block's writes follow these reads
        if (j == 3 || j == 7) __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      }
    }
    __syncthreads();
  }
    if (!more) break;
    t = tn;
  }
}

// One launch per product; tiles enumerate (problem, m tile, n tile) as the
// mode's geometry says.
template <int kMode>
__global__ __launch_bounds__(kThreads) void grouped_gemm_bwd_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2][kRowsL * LDK];
  float* s_red = reinterpret_cast<float*>(&smem[0][0]);  // epilogue only (8 x BM), after the K loop
  auto no_next = [](BwdTile&) { return false; };
  const int tile = (kMode <= kWgradGU) ? run_tile(blockIdx.x) : (int)blockIdx.x;
  BwdTile t;
  t.au = nullptr; t.gate = nullptr; t.part = nullptr; t.npart = 0; t.Hp = 0;
  t.amap = nullptr; t.bmap = nullptr;
  if (kMode == kDgradH || kMode == kDgradX) {
    // grouped over problems with ragged rows: tile prefix per problem
    if (tile >= a.pre[a.E + 1]) return;
    const int p = __builtin_amdgcn_readfirstlane(find_problem(a.pre, a.E, tile));
    const bool routed = p < a.E;
    const int rows = routed ? a.offsets[p + 1] - a.offsets[p] : a.T;
    const int rb = routed ? a.offsets[p] : 0;
    const int Hp = routed ? a.H : a.Hs;
    const int local = tile - a.pre[p];
    const int nmt = (rows + BM - 1) / BM;
    t.m0 = (local % nmt) * BM;
    t.n0 = (local / nmt) * BN;
    t.M = rows;
    t.k0 = 0;
    if (kMode == kDgradH) {
      // A = dOut rows (bf16), gathered; B[n = h][k = d] = W_down[d][h]
      t.a = a.dout;
      t.amap = routed ? a.row_token + rb : nullptr;
      t.a_bytes = (uint32_t)((size_t)a.T * a.D * 2);
      t.lda = a.D;
      t.b = routed ? a.w_down + (size_t)p * a.D * a.H : a.w_down_shared;
      t.b_bytes = (uint32_t)((size_t)a.D * Hp * 2);
      t.ldb = Hp;
      t.N = Hp;
      t.K = a.D;
      t.k1 = a.D;
      t.c = routed ? static_cast<void*>(a.dau + (size_t)rb * 2 * a.H) : static_cast<void*>(a.dau_shared);
      t.ldc = 2 * Hp;
      t.au = routed ? a.au + (size_t)rb * 2 * a.H : a.au_shared;
      t.gate = routed ? a.row_gate + rb : nullptr;
      t.part = routed ? a.part + (size_t)rb * cdiv(a.H, BN) : a.part_shared;
      t.npart = cdiv(Hp, BN);
      t.Hp = Hp;
    } else {
      // A = [dA | dU] rows; B[n = d][k = j] = W_gu[j][d]
      t.a = routed ? a.dau + (size_t)rb * 2 * a.H : a.dau_shared;
      t.a_bytes = (uint32_t)((size_t)rows * 2 * Hp * 2);
      t.lda = 2 * Hp;
      t.b = routed ? a.w_gu + (size_t)p * 2 * a.H * a.D : a.w_gu_shared;
      t.b_bytes = (uint32_t)((size_t)2 * Hp * a.D * 2);
      t.ldb = a.D;
      t.N = a.D;
      t.K = 2 * Hp;
      t.k1 = 2 * Hp;
      t.c = routed ? static_cast<void*>(a.dxr + (size_t)rb * a.D) : static_cast<void*>(a.dxs);
      t.ldc = a.D;
    }
    // valid 32-row blocks of this wave (rows 128 wm + 32 i)
    const int wm = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) >> 2;
    const int vr = min(BM, t.M - t.m0) - 128 * wm;
    switch (vr <= 0 ? 0 : min(4, (vr + 31) / 32)) {
      case 4: bwd_tiles<kMode, false, false, 4>(t, no_next, smem, s_red); break;
      case 3: bwd_tiles<kMode, false, false, 3>(t, no_next, smem, s_red); break;
      case 2: bwd_tiles<kMode, false, false, 2>(t, no_next, smem, s_red); break;
      case 1: bwd_tiles<kMode, false, false, 1>(t, no_next, smem, s_red); break;
      default: bwd_tiles<kMode, false, false, 0>(t, no_next, smem, s_red); break;
    }
  } else if (kMode == kWgradD || kMode == kWgradGU) {
    // every problem (experts, then the shared expert) gets its full weight
    // gradient; experts without rows get zeros
    const int Mr = kMode == kWgradD ? a.D : 2 * a.H, Nr = kMode == kWgradD ? a.H : a.D;
    const int Ms = kMode == kWgradD ? a.D : 2 * a.Hs, Ns = kMode == kWgradD ? a.Hs : a.D;
    const int per_r = cdiv(Mr, BM) * cdiv(Nr, BN), per_s = cdiv(Ms, BM) * cdiv(Ns, BN);
    const int total = a.E * per_r + (a.Hs > 0 ? per_s : 0);
    const BwdTile base = t;
    auto make = [&](int tile, BwdTile& t) -> bool {
      if (tile >= total) return false;
      t = base;
      const bool routed = tile < a.E * per_r;
      const int p = routed ? tile / per_r : a.E;
      const int local = routed ? tile % per_r : tile - a.E * per_r;
      const int M = routed ? Mr : Ms, N = routed ? Nr : Ns, Hp = routed ? a.H : a.Hs;
      const int rows = routed ? a.offsets[p + 1] - a.offsets[p] : a.T;
      const int rb = routed ? a.offsets[p] : 0;
      // groups of four m-tiles, column-major inside a group: a run of 32
      // consecutive tiles covers 4 m-slices x 8 n-slices of the operands
      const int nmt = cdiv(M, BM), nnt = cdiv(N, BN);
      const int g0 = (local / (4 * nnt)) * 4, gsz = min(4, nmt - g0);
      const int idx = local - g0 * nnt;
      t.m0 = (g0 + idx % gsz) * BM;
      t.n0 = (idx / gsz) * BN;
      t.M = M;
      t.N = N;
      t.K = rows;
      t.k0 = 0;
      t.k1 = rows;
      if (kMode == kWgradD) {
        // A[m = d][k = r] = dOut[tok(r)][d]; B[n = h][k = r] = (g h)[r][h]
        t.a = a.dout;
        t.amap = routed ? a.row_token + rb : nullptr;
        t.a_bytes = (uint32_t)((size_t)a.T * a.D * 2);
        t.lda = a.D;
        t.b = routed ? a.gh + (size_t)rb * a.H : a.gh_shared;
        t.b_bytes = (uint32_t)((size_t)(rows > 0 ? rows : 1) * Hp * 2);
        t.ldb = Hp;
        t.c = routed ? static_cast<void*>(a.dw_down + (size_t)p * a.D * a.H)
                     : static_cast<void*>(a.dw_down_shared);
        t.ldc = Hp;
      } else {
        // A[m = j][k = r] = [dA | dU][r][j]; B[n = d][k = r] = x[tok(r)][d]
        t.a = routed ? a.dau + (size_t)rb * 2 * a.H : a.dau_shared;
        t.a_bytes = (uint32_t)((size_t)(rows > 0 ? rows : 1) * 2 * Hp * 2);
        t.lda = 2 * Hp;
        t.b = a.x;
        t.bmap = routed ? a.row_token + rb : nullptr;
        t.b_bytes = (uint32_t)((size_t)a.T * a.D * 2);
        t.ldb = a.D;
        t.c = routed ? static_cast<void*>(a.dw_gu + (size_t)p * 2 * a.H * a.D)
                     : static_cast<void*>(a.dw_gu_shared);
        t.ldc = a.D;
      }
      return true;
    };
    // A persistent grid (a multiple of 8 workgroups, about one per CU): block b
    // takes the run-mapped tiles of blocks b, b + G, b + 2G, ... (increasing,
    // so the first one past the end ends the sequence). Short-K tiles (an
    // expert's tokens) are many, and the next tile's first loads then overlap
    // this tile's last MFMAs and its epilogue.
    int kseq = 0;
    if (!make(run_tile(blockIdx.x), t)) return;
    auto next = [&](BwdTile& tn) -> bool {
      ++kseq;
      return make(run_tile(blockIdx.x + kseq * gridDim.x), tn);
    };
    bwd_tiles<kMode, true, true, 4>(t, next, smem, s_red);
  } else if (kMode == kRouterW) {
    // d gate_w planes: A[m = e][k = t] = dlogit[t][e]; B[n = d][k = t] = x[t][d]; K split over planes
    const int nmt = cdiv(a.Ep, BM), nnt = cdiv(a.D, BN);
    const int per = nmt * nnt;
    if (tile >= per * a.splits) return;
    const int z = tile / per, local = tile % per;
    const int kc = ((a.T + a.splits - 1) / a.splits + BK - 1) / BK * BK;
    t.m0 = (local / nnt) * BM;
    t.n0 = (local % nnt) * BN;
    t.M = a.E;
    t.N = a.D;
    t.K = a.T;
    t.k0 = min(z * kc, a.T);
    t.k1 = min(t.k0 + kc, a.T);
    t.a = a.dlogit;
    t.a_bytes = (uint32_t)((size_t)a.T * a.Ep * 2);
    t.lda = a.Ep;
    t.b = a.x;
    t.b_bytes = (uint32_t)((size_t)a.T * a.D * 2);
    t.ldb = a.D;
    t.c = a.gw_planes + (size_t)z * a.E * a.D;
    t.ldc = a.D;
    bwd_tiles<kMode, true, false, 4>(t, no_next, smem, s_red);
  } else {
    // dx_r = dlogit gate_w: A = dlogit rows (K = Ep, zero-padded); B[n = d][k = e] = gate_w[e][d]
    const int nnt = cdiv(a.D, BN);
    if (tile >= cdiv(a.T, BM) * nnt) return;
    t.m0 = (tile / nnt) * BM;
    t.n0 = (tile % nnt) * BN;
    t.M = a.T;
    t.N = a.D;
    t.K = a.Ep;
    t.k0 = 0;
    t.k1 = a.Ep;
    t.a = a.dlogit;
    t.a_bytes = (uint32_t)((size_t)a.T * a.Ep * 2);
    t.lda = a.Ep;
    t.b = a.gw_bf16;
    t.b_bytes = (uint32_t)((size_t)a.Ep * a.D * 2);
    t.ldb = a.D;
    t.c = a.dx_router;
    t.ldc = a.D;
    bwd_tiles<kMode, false, false, 4>(t, no_next, smem, s_red);
  }
}

namespace {

// fp32 -> bf16 (RNE), rows of `cols` values into rows of `ldd` (zero padding)
// dst[r][c] = bf16(src[r][c]) for r < srows, c < cols; 0 elsewhere in the
// rows x ldd destination. 8 consecutive values per thread (cols and ldd are
// multiples of 8): two 16-byte loads, one 16-byte store.
__global__ __launch_bounds__(256) void to_bf16_kernel(const float* __restrict__ src, int rows, int cols, int srows,
                                                     uint16_t* __restrict__ dst, int ldd) {
  const int cpr = ldd / 8;  // 8-value pieces per destination row
  const int n = rows * cpr;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    const int r = i / cpr, c = (i - r * cpr) * 8;
    uint4 o = make_uint4(0u, 0u, 0u, 0u);
    if (r < srows && c < cols) {
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(src + (size_t)r * cols + c);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(src + (size_t)r * cols + c + 4);
      o.x = (uint32_t)f32_to_bf16(v0.x) | ((uint32_t)f32_to_bf16(v0.y) << 16);
      o.y = (uint32_t)f32_to_bf16(v0.z) | ((uint32_t)f32_to_bf16(v0.w) << 16);
      o.z = (uint32_t)f32_to_bf16(v1.x) | ((uint32_t)f32_to_bf16(v1.y) << 16);
      o.w = (uint32_t)f32_to_bf16(v1.z) | ((uint32_t)f32_to_bf16(v1.w) << 16);
    }
    *reinterpret_cast<uint4*>(dst + (size_t)r * ldd + c) = o;
  }
}

// pre[p] = tiles of problems < p: ceil(rows_p / 128) row tiles x n_p column
// tiles (one thread per problem, E + 1 <= 1024, block scan through LDS)
__global__ __launch_bounds__(1024) void tile_prefix_kernel(const int32_t* __restrict__ offsets, int E,
                                                           int shared_rows, int n_routed, int n_shared,
                                                           int32_t* __restrict__ pre) {
  __shared__ int wsum[16];
  const int p = threadIdx.x, lane = p & 63, w = p >> 6;
  int v = 0;
  if (p <= E) {
    const int rows = p < E ? offsets[p + 1] - offsets[p] : shared_rows;
    v = ((rows + BM - 1) / BM) * (p < E ? n_routed : n_shared);
  }
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int base = 0, all = 0;
  for (int q = 0; q < 16; ++q) {
    if (q < w) base += wsum[q];
    all += wsum[q];
  }
  if (p <= E) pre[p] = base + incl - v;
  if (p == 0) pre[E + 1] = all;
}

// router backward, one wave per token: dL/dg from the partial sums, through
// the renormalisation and rsf to the selected scores, through the score
// function to dlogit (bf16, row padded with zeros to Ep)
__global__ __launch_bounds__(256) void router_bwd_kernel(const float* __restrict__ logits,
                                                         const int32_t* __restrict__ idx,
                                                         const int32_t* __restrict__ slot_row,
                                                         const float* __restrict__ part, int npart, int T, int E,
                                                         int Ep, int K, int score_fn, int norm, float rsf,
                                                         uint16_t* __restrict__ dlogit) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  const float* l = logits + (size_t)t * E;
  // scores (fp32, as the forward)
  float mx = -3.4e38f;
  if (score_fn == MOE_SCORE_SOFTMAX) {
    for (int e = lane; e < E; e += 64) mx = fmaxf(mx, l[e]);
    mx = wave_max_f32(mx);
  }
  float den = 0.f;
  if (score_fn == MOE_SCORE_SOFTMAX) {
    for (int e = lane; e < E; e += 64) den += __expf(l[e] - mx);
    den = wave_sum_f32(den);
  }
  auto score = [&](int e) {
    return score_fn == MOE_SCORE_SOFTMAX ? __expf(l[e] - mx) / den : 1.0f / (1.0f + __expf(-l[e]));
  };
  // selected scores and dL/dg (lane k < K holds slot k)
  float ss = 0.f, dg = 0.f;
  int ek = -1;
  if (lane < K) {
    ek = dcheck(idx[(size_t)t * K + lane], E, kSiteBwdExpert);
    ss = score(ek);
    const float* pr = part + (size_t)dcheck(slot_row[(size_t)t * K + lane], T * K, kSiteBwdRow) * npart;
    for (int j = 0; j < npart; ++j) dg += pr[j];
  }
  float ds = rsf * dg;
  if (norm) {
    const float S = wave_sum_f32(ss);
    const float sdg = wave_sum_f32(ss * dg);
    ds = rsf * (dg / S - sdg / (S * S));
  }
  // sum_j s_j ds_j over the selected (softmax)
  const float sds = wave_sum_f32(lane < K ? ss * ds : 0.f);
  for (int e = lane; e < Ep; e += 64) {
    float v = 0.f;
    if (e < E) {
      // ds at e: from the lane that holds e, if selected
      float dse = 0.f;
      for (int k = 0; k < K; ++k) {
        const int ei = __shfl(ek, k);
        const float dsk = __shfl(ds, k);
        if (ei == e) dse = dsk;
      }
      const float se = score(e);
      v = score_fn == MOE_SCORE_SOFTMAX ? se * (dse - sds) : dse * se * (1.0f - se);
    }
    dlogit[(size_t)t * Ep + e] = f32_to_bf16(v);
  }
}

// dx[t] = [d_out[t]] + dX_shared[t] + sum_k dX_rows[slot(t,k)] + dx_router[t]
// 8 consecutive columns per thread (D % 128 == 0): every load of a step (the
// residual, the shared row, up to 8 slot rows, the router part) is issued
// before the first add, and the adds run in that fixed order; an absent
// source reads a valid row and adds -0.0 (which changes no value, signed
// zeros included), so no branch sits around a load.
__device__ __forceinline__ void add_bf16x8(float (&acc)[8], const uint4 s4, bool use) {
  const uint32_t m = use ? 0xFFFFFFFFu : 0x80008000u, z = use ? 0u : 0x80008000u;
  const uint32_t w[4] = {(s4.x & m) | z, (s4.y & m) | z, (s4.z & m) | z, (s4.w & m) | z};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc[2 * q] += __uint_as_float(w[q] << 16);
    acc[2 * q + 1] += __uint_as_float(w[q] & 0xFFFF0000u);
  }
}

__global__ __launch_bounds__(256) void dx_combine_kernel(const float* __restrict__ dout,
                                                         const uint16_t* __restrict__ dxr,
                                                         const uint16_t* __restrict__ dxs,
                                                         const float* __restrict__ dx_router,
                                                         const int32_t* __restrict__ slot_row, int T, int D, int K,
                                                         int add_residual, float* __restrict__ dx) {
  const int t = blockIdx.x;
  int rows[kMaxTopK];
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) rows[k] = dcheck(slot_row[(size_t)t * K + (k < K ? k : 0)], T * K, kSiteBwdRow);
  const bool has_shared = dxs != nullptr;
  const uint16_t* sbase = has_shared ? dxs + (size_t)t * D : dxr + (size_t)rows[0] * D;
  for (int d = 8 * threadIdx.x; d < D; d += 8 * blockDim.x) {
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(dout + (size_t)t * D + d);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(dout + (size_t)t * D + d + 4);
    const uint4 sv = *reinterpret_cast<const uint4*>(sbase + d);
    uint4 rk[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) rk[k] = *reinterpret_cast<const uint4*>(dxr + (size_t)rows[k] * D + d);
    const f32x4 r0 = *reinterpret_cast<const f32x4*>(dx_router + (size_t)t * D + d);
    const f32x4 r1 = *reinterpret_cast<const f32x4*>(dx_router + (size_t)t * D + d + 4);
    float acc[8];
    if (add_residual) {
      acc[0] = a0.x; acc[1] = a0.y; acc[2] = a0.z; acc[3] = a0.w;
      acc[4] = a1.x; acc[5] = a1.y; acc[6] = a1.z; acc[7] = a1.w;
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = 0.f;
    }
    add_bf16x8(acc, sv, has_shared);
#pragma unroll
    for (int k = 0; k < 8; ++k) add_bf16x8(acc, rk[k], k < K);
    if (K > 8) {
#pragma unroll
      for (int k = 8; k < kMaxTopK; ++k) rk[k - 8] = *reinterpret_cast<const uint4*>(dxr + (size_t)rows[k] * D + d);
#pragma unroll
      for (int k = 8; k < kMaxTopK; ++k) add_bf16x8(acc, rk[k - 8], k < K);
    }
    acc[0] += r0.x; acc[1] += r0.y; acc[2] += r0.z; acc[3] += r0.w;
    acc[4] += r1.x; acc[5] += r1.y; acc[6] += r1.z; acc[7] += r1.w;
    *reinterpret_cast<f32x4*>(dx + (size_t)t * D + d) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4*>(dx + (size_t)t * D + d + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
  }
}

// out[i] = sum over planes in order
__global__ __launch_bounds__(256) void planes_sum_kernel(const float* __restrict__ planes, size_t n, int splits,
                                                         float* __restrict__ out) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    float v = 0.f;
    for (int z = 0; z < splits; ++z) v += planes[(size_t)z * n + i];
    out[i] = v;
  }
}

int grid_for(size_t n) { return (int)std::min<size_t>((n + 255) / 256, 8192); }
// blocks covering every tile index below n under the run mapping
int run_grid(int n) { return cdiv(cdiv(n, kRunB), 8) * 8 * kRunB; }

}  // namespace

hipError_t launch_layer_backward(const BwdArgs& a, hipStream_t s) {
  hipError_t e;
  // dOut and gate_w to bf16 (gate_w rows padded with zeros to Ep)
  hipLaunchKernelGGL(to_bf16_kernel, dim3(grid_for((size_t)a.T * a.D / 8)), dim3(256), 0, s, a.dout_f32, a.T, a.D,
                     a.T, a.dout, a.D);
  hipLaunchKernelGGL(to_bf16_kernel, dim3(grid_for((size_t)a.Ep * a.D / 8)), dim3(256), 0, s, a.gate_w, a.Ep, a.D,
                     a.E, a.gw_bf16, a.D);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // tile prefixes of the two row-grouped products
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, s, a.offsets, a.E, a.Hs > 0 ? a.T : 0,
                     cdiv(a.H, BN), cdiv(a.Hs, BN), a.pre_h);
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, s, a.offsets, a.E, a.Hs > 0 ? a.T : 0,
                     cdiv(a.D, BN), cdiv(a.D, BN), a.pre_x);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const long mblk = (long)(a.T * a.K + BM - 1) / BM + a.E, mblk_s = a.Hs > 0 ? (a.T + BM - 1) / BM : 0;
  BwdArgs b = a;
  b.pre = a.pre_h;
  const int tiles_h = (int)(mblk * cdiv(a.H, BN) + mblk_s * cdiv(a.Hs, BN));
  hipLaunchKernelGGL(grouped_gemm_bwd_kernel<kDgradH>, dim3(run_grid(tiles_h)), dim3(kThreads), 0, s, b);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // router backward needs every dL/dg partial
  hipLaunchKernelGGL(router_bwd_kernel, dim3((a.T + 3) / 4), dim3(256), 0, s, a.logits, a.idx, a.slot_row, a.part,
                     cdiv(a.H, BN), a.T, a.E, a.Ep, a.K, a.score_fn, a.norm, a.rsf, a.dlogit);
  b.pre = a.pre_x;
  const int tiles_x = (int)(mblk * cdiv(a.D, BN) + mblk_s * cdiv(a.D, BN));
  hipLaunchKernelGGL(grouped_gemm_bwd_kernel<kDgradX>, dim3(run_grid(tiles_x)), dim3(kThreads), 0, s, b);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int tiles_wd = a.E * cdiv(a.D, BM) * cdiv(a.H, BN) + (a.Hs > 0 ? cdiv(a.D, BM) * cdiv(a.Hs, BN) : 0);
  // the weight gradients: a persistent grid of about one workgroup per CU (a
  // multiple of 8, the XCD count)
  int dev = 0, cus = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  const int persist = std::max(8, (cus / 8) * 8);
  hipLaunchKernelGGL(grouped_gemm_bwd_kernel<kWgradD>, dim3(std::min(run_grid(tiles_wd), persist)), dim3(kThreads), 0,
                     s, a);
  const int tiles_wgu =
      a.E * cdiv(2 * a.H, BM) * cdiv(a.D, BN) + (a.Hs > 0 ? cdiv(2 * a.Hs, BM) * cdiv(a.D, BN) : 0);
  hipLaunchKernelGGL(grouped_gemm_bwd_kernel<kWgradGU>, dim3(std::min(run_grid(tiles_wgu), persist)), dim3(kThreads), 0,
                     s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int tiles_rw = cdiv(a.Ep, BM) * cdiv(a.D, BN) * a.splits;
  hipLaunchKernelGGL(grouped_gemm_bwd_kernel<kRouterW>, dim3(tiles_rw), dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL(planes_sum_kernel, dim3(grid_for((size_t)a.E * a.D)), dim3(256), 0, s, a.gw_planes,
                     (size_t)a.E * a.D, a.splits, a.d_gate_w);
  const int tiles_rx = cdiv(a.T, BM) * cdiv(a.D, BN);
  hipLaunchKernelGGL(grouped_gemm_bwd_kernel<kRouterX>, dim3(tiles_rx), dim3(kThreads), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // threads per token: the 8-column pieces of a row spread evenly over at
  // most 256 threads (D = 7168: 224 threads x 4 pieces)
  const int pieces = a.D / 8, iters = (pieces + 255) / 256;
  hipLaunchKernelGGL(dx_combine_kernel, dim3(a.T), dim3((pieces + iters - 1) / iters), 0, s, a.dout_f32, a.dxr, a.Hs > 0 ? a.dxs : nullptr,
                     a.dx_router, a.slot_row, a.T, a.D, a.K, a.add_residual, a.dx);
  return hipGetLastError();
}

MOE_DEBUG_READER(debug_read_bwd)

}  // namespace moe
