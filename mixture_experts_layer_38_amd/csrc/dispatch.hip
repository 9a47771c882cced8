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
  const int mblocks = (rows + a.bm - 1) / a.bm;
  const int it1 = (p <= a.E) ? mblocks * (p < a.E ? a.n1_routed : a.n1_shared) : 0;
  const int it2 = (p <= a.E) ? mblocks * (p < a.E ? a.n2_routed : a.n2_shared) : 0;
  int tot0, tot1, tot2;
  const int off = block_exclusive_scan(cnt, &tot0);
  const int o1 = block_exclusive_scan(it1, &tot1);
  const int o2 = block_exclusive_scan(it2, &tot2);
  if (p < a.E) {
    a.offsets[p] = off;
    a.cursor[p] = off;
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

// Each block takes a chunk of kPermChunk (token, slot) entries: an LDS
// histogram of the chunk, one global atomic per expert to reserve the chunk's
// rows, then LDS atomics hand out rows inside each reservation. Row order
// within an expert is arbitrary (no result depends on it: every row is
// computed on its own and the combine adds a token's rows in slot order).
constexpr int kPermChunk = 2048;

__global__ __launch_bounds__(256) void dispatch_permute_kernel(DispatchArgs a) {
  __shared__ int32_t cnt[kMaxExperts];
  __shared__ int32_t base[kMaxExperts];
  const int n = a.T * a.K;
  const int i0 = blockIdx.x * kPermChunk, i1 = min(n, i0 + kPermChunk);
  for (int e = threadIdx.x; e < a.E; e += 256) cnt[e] = 0;
  __syncthreads();
  for (int i = i0 + threadIdx.x; i < i1; i += 256) {
    const int e = a.idx[i];
    if (e >= 0 && e < a.E) atomicAdd(&cnt[e], 1);  // out-of-range entries are skipped, as in the histogram
  }
  __syncthreads();
  for (int e = threadIdx.x; e < a.E; e += 256) {
    const int c = cnt[e];
    base[e] = c ? atomicAdd(&a.cursor[e], c) : 0;
    cnt[e] = 0;
  }
  __syncthreads();
  for (int i = i0 + threadIdx.x; i < i1; i += 256) {
    const int e = a.idx[i];
    if (e < 0 || e >= a.E) continue;
    const int r = base[e] + atomicAdd(&cnt[e], 1);
    a.row_token[r] = i / a.K;
    if (a.row_gate) a.row_gate[r] = a.gate[i];
    a.slot_row[i] = r;
  }
}

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(1024), 0, s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int n = a.T * a.K;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(dispatch_permute_kernel, dim3((n + kPermChunk - 1) / kPermChunk), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
