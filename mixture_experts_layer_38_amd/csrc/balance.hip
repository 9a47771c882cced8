// Load balance between steps: the auxiliary-loss-free bias update of the
// DeepSeek-V3 basics page (section 1.2) and the load and importance
// statistics of the load-balance code in the DeepSeekMoE + MLA notes (page 3).
//
// One workgroup of 512 threads, one expert per thread (E <= 512). Whether an
// expert is over- or underloaded is decided in integers (counts_e * E against
// sum(counts)), so the update has no rounding-dependent ties; the statistics
// are reduced in double, in a fixed order.
#include "moe_internal.hpp"

namespace moe {

__global__ __launch_bounds__(512) void balance_kernel(const int32_t* __restrict__ counts, int E, float gamma,
                                                      float* __restrict__ bias, float* __restrict__ stats) {
  __shared__ long long s_tot[512];
  __shared__ double s_a[512];
  __shared__ int s_max[512];
  const int e = threadIdx.x;
  const long long c = (e < E) ? (long long)counts[e] : 0;
  s_tot[e] = c;
  s_max[e] = (int)c;
  __syncthreads();
  for (int o = 256; o > 0; o >>= 1) {
    if (e < o) {
      s_tot[e] += s_tot[e + o];
      s_max[e] = max(s_max[e], s_max[e + o]);
    }
    __syncthreads();
  }
  const long long total = s_tot[0];
  if (bias != nullptr && e < E) {
    if (c * E > total) bias[e] = bias[e] - gamma;       // overloaded
    else if (c * E < total) bias[e] = bias[e] + gamma;  // underloaded
  }
  if (stats == nullptr) return;
  if (total == 0) {
    if (e < 3) stats[e] = 0.f;
    return;
  }
  // load_e = c_e / total; mean of load is 1/E
  const double load = (double)c / (double)total, inv_e = 1.0 / E;
  s_a[e] = (e < E) ? (load - inv_e) * (load - inv_e) : 0.0;
  __syncthreads();
  for (int o = 256; o > 0; o >>= 1) {
    if (e < o) s_a[e] += s_a[e + o];
    __syncthreads();
  }
  if (e == 0) {
    const double ss = s_a[0];
    stats[0] = (float)(E > 1 ? sqrt(ss / (E - 1)) : 0.0);   // std of load (n-1 denominator)
    stats[1] = (float)(ss / E);                              // mean (load - 1/E)^2
    stats[2] = (float)((double)s_max[0] * E / (double)total - 1.0);  // max / mean - 1
  }
}

// Sum over the block's 512 threads in a fixed tree order (every thread gets it).
__device__ double block_sum_512(double v, double* sh) {
  const int i = threadIdx.x;
  __syncthreads();
  sh[i] = v;
  __syncthreads();
  for (int o = 256; o > 0; o >>= 1) {
    if (i < o) sh[i] += sh[i + o];
    __syncthreads();
  }
  return sh[0];
}

// Mean and n-1 standard deviation of x over n entries (x valid on threads < n),
// and the balance-loss term mean((x - 1/n)^2).
__device__ void spread_stats(double x, int n, double* sh, float* std_out, float* loss_out) {
  const bool in = threadIdx.x < n;
  const double mean = block_sum_512(in ? x : 0.0, sh) / n;
  const double dev = in ? (x - mean) * (x - mean) : 0.0;
  const double tgt = in ? (x - 1.0 / n) * (x - 1.0 / n) : 0.0;
  const double ss = block_sum_512(dev, sh);
  const double st = block_sum_512(tgt, sh);
  if (threadIdx.x == 0) {
    *std_out = (float)(n > 1 ? sqrt(ss / (n - 1)) : 0.0);
    *loss_out = (float)(st / n);
  }
}

// The statistics of the load-balance code in the DeepSeekMoE + MLA notes
// (page 3): load_e = c_e / sum(c), importance_e = S_e / sum(S) with S_e the
// column sum of the scores; per device (devices own contiguous runs of
// E / n_devices experts) the sums of both, renormalised. stats: [0] load std,
// [1] load loss, [2] max violation, [3] importance std, [4] importance loss,
// [5] device load std, [6] device load loss, [7] device importance std,
// [8] device importance loss. A quantity whose total is 0 has every
// statistic 0.
__global__ __launch_bounds__(512) void balance_stats_kernel(const int32_t* __restrict__ counts,
                                                            const float* __restrict__ score_sum, int E,
                                                            int n_devices, float* __restrict__ stats) {
  __shared__ double sh[512];
  __shared__ double s_load[512], s_imp[512];
  __shared__ int s_max[512];
  const int e = threadIdx.x;
  const bool in = e < E;
  const double c = in ? (double)counts[e] : 0.0;
  const double sc = in ? (double)score_sum[e] : 0.0;
  s_max[e] = in ? counts[e] : 0;
  __syncthreads();
  for (int o = 256; o > 0; o >>= 1) {
    if (e < o) s_max[e] = max(s_max[e], s_max[e + o]);
    __syncthreads();
  }
  const int cmax = s_max[0];
  const double total = block_sum_512(c, sh);      // integers below 2^53: exact
  const double imp_total = block_sum_512(sc, sh);
  const double load = total > 0 ? c / total : 0.0;
  const double imp = imp_total > 0 ? sc / imp_total : 0.0;
  s_load[e] = load;
  s_imp[e] = imp;
  float lstd, lloss, istd, iloss;
  spread_stats(load, E, sh, &lstd, &lloss);
  spread_stats(imp, E, sh, &istd, &iloss);
  // device sums, each over its experts in order, then renormalised
  const int per = E / n_devices;
  double dl = 0.0, di = 0.0;
  if (e < n_devices)
    for (int j = e * per; j < (e + 1) * per; ++j) {
      dl += s_load[j];
      di += s_imp[j];
    }
  const double dl_tot = block_sum_512(e < n_devices ? dl : 0.0, sh);
  const double di_tot = block_sum_512(e < n_devices ? di : 0.0, sh);
  float dlstd, dlloss, distd, diloss;
  spread_stats(dl_tot > 0 ? dl / dl_tot : 0.0, n_devices, sh, &dlstd, &dlloss);
  spread_stats(di_tot > 0 ? di / di_tot : 0.0, n_devices, sh, &distd, &diloss);
  if (e == 0) {
    const bool lz = total == 0, iz = imp_total == 0;
    stats[0] = lz ? 0.f : lstd;
    stats[1] = lz ? 0.f : lloss;
    stats[2] = lz ? 0.f : (float)((double)cmax * E / total - 1.0);
    stats[3] = iz ? 0.f : istd;
    stats[4] = iz ? 0.f : iloss;
    stats[5] = lz ? 0.f : dlstd;
    stats[6] = lz ? 0.f : dlloss;
    stats[7] = iz ? 0.f : distd;
    stats[8] = iz ? 0.f : diloss;
  }
}

hipError_t launch_balance_stats(const int32_t* counts, const float* score_sum, int E, int n_devices, float* stats,
                                hipStream_t s) {
  hipLaunchKernelGGL(balance_stats_kernel, dim3(1), dim3(512), 0, s, counts, score_sum, E, n_devices, stats);
  return hipGetLastError();
}

__global__ void zero_f32_kernel(float* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

hipError_t launch_zero_f32(float* p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)(blocks < 16384 ? blocks : 16384)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_balance(const int32_t* counts, int E, float gamma, float* bias, float* stats, hipStream_t s) {
  hipLaunchKernelGGL(balance_kernel, dim3(1), dim3(512), 0, s, counts, E, gamma, bias, stats);
  return hipGetLastError();
}

}  // namespace moe
