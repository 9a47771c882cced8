// Load balance between steps: the auxiliary-loss-free bias update of the
// DeepSeek-V3 basics page (section 1.2) and the load statistics of the
// load-balance code in the DeepSeekMoE + MLA notes (page 3).
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

hipError_t launch_balance(const int32_t* counts, int E, float gamma, float* bias, float* stats, hipStream_t s) {
  hipLaunchKernelGGL(balance_kernel, dim3(1), dim3(512), 0, s, counts, E, gamma, bias, stats);
  return hipGetLastError();
}

}  // namespace moe
