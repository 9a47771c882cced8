// Dispatch: per-expert histogram, prefix scan into expert-contiguous row
// offsets (plus the work-item tables of the expert GEMMs), and the permutation
// of (token, slot) pairs into those rows.
//
// This replaces the repeat_interleave + per-expert boolean-mask gather of the
// MoE forward on the DeepSeek-V2 walkthrough page: every token is kept (no
// capacity limit, no dropping, as the DeepSeek-V3 basics page, section 1.2,
// states for training and inference).
#include "moe_internal.hpp"

namespace moe {

__global__ __launch_bounds__(256) void histogram_kernel(const int32_t* __restrict__ idx,
                                                        int32_t* __restrict__ counts, int n, int E) {
  __shared__ int32_t h[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
  __syncthreads();
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) {
    const int e = idx[i];
    if (e >= 0 && e < E) atomicAdd(&h[e], 1);  // out-of-range entries are skipped
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256)
    if (h[e]) atomicAdd(&counts[e], h[e]);
}

__global__ void zero_i32_kernel(int32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

hipError_t launch_histogram(const int32_t* idx, int32_t* counts, int n, int E, hipStream_t s) {
  hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(256), 0, s, counts, E);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || n == 0) return err;
  // at least 4096 entries per block: one LDS histogram each, then at most E
  // global atomics per block
  int blocks = (n + 4095) / 4096;
  if (blocks > 128) blocks = 128;
  hipLaunchKernelGGL(histogram_kernel, dim3(blocks), dim3(256), 0, s, idx, counts, n, E);
  return hipGetLastError();
}

// Exclusive scan over the 1024 threads of a block; returns the prefix, and the
// block total through *total.
__device__ int block_exclusive_scan(int v, int* total) {
  __shared__ int wsum[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(incl, o, 64);
    if (lane >= o) incl += n;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int base = 0, all = 0;
  for (int w = 0; w < 16; ++w) {
    if (w < wave) base += wsum[w];
    all += wsum[w];
  }
  __syncthreads();
  *total = all;
  return base + incl - v;
}

__global__ __launch_bounds__(1024) void dispatch_scan_kernel(DispatchArgs a) {
  const int p = threadIdx.x;  // problem: routed expert p < E, shared expert p == E
  const int rows = (p < a.E) ? a.counts[p] : (p == a.E ? a.shared_rows : 0);
  const int cnt = (p < a.E) ? rows : 0;
  const int mb1 = (rows + a.bm1 - 1) / a.bm1, mb2 = (rows + a.bm2 - 1) / a.bm2;
  const int it1 = (p <= a.E) ? mb1 * (p < a.E ? a.n1_routed : a.n1_shared) : 0;
  const int it2 = (p <= a.E) ? mb2 * (p < a.E ? a.n2_routed : a.n2_shared) : 0;
  int tot0, tot1, tot2;
  const int off = block_exclusive_scan(cnt, &tot0);
  const int o1 = block_exclusive_scan(it1, &tot1);
  const int o2 = block_exclusive_scan(it2, &tot2);
  if (p < a.E) {
    a.offsets[p] = off;
    if (a.counts_out) a.counts_out[p] = cnt;
  }
  if (p == a.E) a.offsets[p] = tot0;
  if (p <= a.E) {
    a.pre1[p] = o1;
    a.pre2[p] = o2;
  }
  if (p == a.E + 1) {
    a.pre1[p] = tot1;
    a.pre2[p] = tot2;
  }
}

// The permutation is stable: the row of entry (t, k) with expert e is
// offsets[e] + #{(t', k') before (t, k) with expert e}, i.e. an expert's rows
// hold its tokens in ascending order (the scope's definition of the step), so
// every sum over an expert's rows (the weight gradients of the backward pass)
// runs in one order on every call. Entries are split into chunks of
// kPermChunk (128), one wave each: (A) each chunk's expert histogram, (B)
// per expert (one wave, shuffle scan), the first row of each chunk (offsets
// plus the earlier chunks' counts), (C) each wave walks its chunk in order,
// 64 entries at a time,
// ranking equal experts among the lanes with ballots.
constexpr int kPermChunk = kDispatchChunk;

__global__ __launch_bounds__(256) void dispatch_chunk_count_kernel(DispatchArgs a) {
  __shared__ int32_t cnt[4][kMaxExperts];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = a.T * a.K;
  const int nchunks = (n + kPermChunk - 1) / kPermChunk;
  const int chunk = blockIdx.x * 4 + w;
  for (int e = lane; e < a.E; e += 64) cnt[w][e] = 0;
  __syncthreads();
  if (chunk < nchunks) {
    const int i1 = min(n, (chunk + 1) * kPermChunk);
    for (int i = chunk * kPermChunk + lane; i < i1; i += 64) {
      const int e = a.idx[i];
      if (e >= 0 && e < a.E) atomicAdd(&cnt[w][e], 1);  // out-of-range entries are skipped, as in the histogram
    }
  }
  __syncthreads();
  if (chunk < nchunks)
    for (int e = lane; e < a.E; e += 64) a.chunk_base[(size_t)e * nchunks + chunk] = cnt[w][e];
}

// one wave per expert: exclusive scan of its chunk counts (contiguous), plus
// the expert's first row
__global__ __launch_bounds__(256) void dispatch_chunk_scan_kernel(DispatchArgs a) {
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (e >= a.E) return;
  const int nchunks = (a.T * a.K + kPermChunk - 1) / kPermChunk;
  int32_t* base = a.chunk_base + (size_t)e * nchunks;
  int carry = a.offsets[e];
  for (int c0 = 0; c0 < nchunks; c0 += 64) {
    const int c = c0 + lane;
    const int v = c < nchunks ? base[c] : 0;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o, 64);
      if (lane >= o) incl += u;
    }
    if (c < nchunks) base[c] = carry + incl - v;
    carry += __shfl(incl, 63);
  }
}

__global__ __launch_bounds__(256) void dispatch_permute_kernel(DispatchArgs a) {
  __shared__ int32_t run[4][kMaxExperts];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = a.T * a.K;
  const int nchunks = (n + kPermChunk - 1) / kPermChunk;
  const int chunk = blockIdx.x * 4 + w;
  if (chunk < nchunks)
    for (int e = lane; e < a.E; e += 64) run[w][e] = a.chunk_base[(size_t)e * nchunks + chunk];
  __syncthreads();
  if (chunk >= nchunks) return;  // no barrier below: waves of a block work alone from here
  const int i1 = min(n, (chunk + 1) * kPermChunk);
  for (int g0 = chunk * kPermChunk; g0 < i1; g0 += 64) {
    const int i = g0 + lane;
    int e = i < i1 ? a.idx[i] : -1;
    if (e >= a.E) e = -1;
    // lanes holding the same expert, one distinct expert per round
    uint64_t todo = __ballot(e >= 0), mine = 0;
    while (todo) {
      const int v = __shfl(e, __ffsll((unsigned long long)todo) - 1);
      const uint64_t m = __ballot(e == v);
      if (e == v) mine = m;
      todo &= ~m;
    }
    const int base = e >= 0 ? run[w][e] : 0;
    if (e >= 0) {
      const int r = dcheck(base + __popcll(mine & ((1ull << lane) - 1ull)), a.T * a.K, kSiteDispatchRow);
      a.row_token[r] = i / a.K;
      if (a.row_gate) a.row_gate[r] = a.gate[i];
      a.slot_row[i] = r;
      // the highest lane of the expert's group moves the expert's next row on
      if ((mine >> lane) == 1ull) run[w][e] = base + __popcll(mine);
    }
  }
}

// Up to kSmallDispatch (1024) entries (decode-sized batches): the expert
// counts, the scan and the stable permutation in one workgroup, the 64-entry
// chunks being its 16 waves and the per-chunk counts living in LDS -- one
// launch instead of six (counts zeroed, histogram, scan, chunk counts, chunk
// scan, placement). The counts are written to a.counts for later readers.
static_assert(kSmallDispatch == 16 * 64, "one 64-entry chunk per wave of a 1024-thread block");

__global__ __launch_bounds__(1024) void dispatch_small_kernel(DispatchArgs a) {
  __shared__ int32_t cnt[16][kMaxExperts];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  // per-wave (chunk) expert counts
  for (int e = lane; e < a.E; e += 64) cnt[w][e] = 0;
  __syncthreads();
  const int n = a.T * a.K;
  const int i = tid;
  int e = i < n ? a.idx[i] : -1;
  if (e >= a.E) e = -1;  // out-of-range entries are skipped, as in the histogram
  if (e >= 0) atomicAdd(&cnt[w][e], 1);
  __syncthreads();
  // offsets and item prefixes, as dispatch_scan_kernel, on the counts summed
  // over the chunks
  const int p = tid;
  int ecount = 0;
  if (p < a.E) {
    for (int c = 0; c < 16; ++c) ecount += cnt[c][p];
    a.counts[p] = ecount;
  }
  const int rows = (p < a.E) ? ecount : (p == a.E ? a.shared_rows : 0);
  const int c0 = (p < a.E) ? rows : 0;
  const int mb1 = (rows + a.bm1 - 1) / a.bm1, mb2 = (rows + a.bm2 - 1) / a.bm2;
  const int it1 = (p <= a.E) ? mb1 * (p < a.E ? a.n1_routed : a.n1_shared) : 0;
  const int it2 = (p <= a.E) ? mb2 * (p < a.E ? a.n2_routed : a.n2_shared) : 0;
  int tot0, tot1, tot2;
  const int off = block_exclusive_scan(c0, &tot0);
  const int o1 = block_exclusive_scan(it1, &tot1);
  const int o2 = block_exclusive_scan(it2, &tot2);
  if (p < a.E) {
    a.offsets[p] = off;
    if (a.counts_out) a.counts_out[p] = c0;
  }
  if (p == a.E) a.offsets[p] = tot0;
  if (p <= a.E) {
    a.pre1[p] = o1;
    a.pre2[p] = o2;
  }
  if (p == a.E + 1) {
    a.pre1[p] = tot1;
    a.pre2[p] = tot2;
  }
  // per expert: the first row of each chunk's entries
  if (p < a.E) {
    int acc = off;
    for (int c = 0; c < 16; ++c) {
      const int v = cnt[c][p];
      cnt[c][p] = acc;
      acc += v;
    }
  }
  __syncthreads();
  // each wave ranks equal experts among its lanes (lane order = entry order)
  uint64_t todo = __ballot(e >= 0), mine = 0;
  while (todo) {
    const int v = __shfl(e, __ffsll((unsigned long long)todo) - 1);
    const uint64_t m = __ballot(e == v);
    if (e == v) mine = m;
    todo &= ~m;
  }
  if (e >= 0) {
    const int r = dcheck(cnt[w][e] + __popcll(mine & ((1ull << lane) - 1ull)), a.T * a.K, kSiteDispatchRow);
    a.row_token[r] = i / a.K;
    if (a.row_gate) a.row_gate[r] = a.gate[i];
    a.slot_row[i] = r;
  }
}

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s) {
  const int n = a.T * a.K;
  if (small_dispatch(n)) {
    hipLaunchKernelGGL(dispatch_small_kernel, dim3(1), dim3(1024), 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(1024), 0, s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (n == 0) return hipSuccess;
  const int nchunks = (n + kPermChunk - 1) / kPermChunk;
  const int blocks = (nchunks + 3) / 4;
  hipLaunchKernelGGL(dispatch_chunk_count_kernel, dim3(blocks), dim3(256), 0, s, a);
  hipLaunchKernelGGL(dispatch_chunk_scan_kernel, dim3((a.E + 3) / 4), dim3(256), 0, s, a);
  hipLaunchKernelGGL(dispatch_permute_kernel, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

MOE_DEBUG_READER(debug_read_dispatch)

}  // namespace moe
