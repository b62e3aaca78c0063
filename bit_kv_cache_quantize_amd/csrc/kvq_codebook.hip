// Sensitivity-weighted NUQ codebook builder ("KVQuant reading notes" 3.3, Algorithm 2):
// 2^b centres fitted to normalised activations a_i in [-1, 1] with weights F_i by weighted
// k-means. Centres start evenly spaced over [-1, 1]; an iteration assigns every activation
// to its nearest centre (ties to the smaller index, the NUQ lookup's rule) and moves each
// centre to the weighted mean of its members (a centre without members stays). It stops
// when no assignment changes, or after max_iters updates.
//
// Each iteration is two launches on the caller's stream, with no host round trip:
//   assign_kernel: one workgroup per contiguous range of samples; per sample the nearest
//     centre (fp64 distances), a count of changed assignments, and per centre the sums of
//     F a and F over the range (thread sums in sample order, then a fixed reduction tree);
//   update_kernel: one workgroup; per centre the range sums added in range order, the new
//     centre, the fp32 codebook; no changes (after the first iteration) sets the converged
//     flag, which turns every later launch into a no-op.
// Every sum has a fixed order, so the result is reproducible; centres and sums are fp64.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kCbThreads = 256;

// Fixed-order sum over the workgroup (one value per thread): each wave by lane swaps with
// decreasing distance, then the waves in order through LDS.
__device__ __forceinline__ double block_sum(double v, double* lds) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) lds[w] = v;
  __syncthreads();
  double s = 0.0;
  for (int i = 0; i < kCbThreads / 64; ++i) s += lds[i];
  return s;
}

template <int K>
__global__ __launch_bounds__(kCbThreads) void assign_kernel(CodebookArgs a) {
  __shared__ double s_red[kCbThreads / 64];
  __shared__ int s_cnt;
  const CodebookState* st = a.state;
  if (st->converged) return;   // uniform across the grid
  double c[K];
#pragma unroll
  for (int j = 0; j < K; ++j) c[j] = st->centres[j];
  const int64_t lo = (int64_t)blockIdx.x * a.per_range;
  const int64_t hi = lo + a.per_range < a.n ? lo + a.per_range : a.n;
  double sw[K], swa[K];
#pragma unroll
  for (int j = 0; j < K; ++j) { sw[j] = 0.0; swa[j] = 0.0; }
  int changed = 0;
  const bool first = st->iter == 0;
  for (int64_t i = lo + threadIdx.x; i < hi; i += kCbThreads) {
    const double x = (double)a.act[i];
    const double wt = a.weight ? (double)a.weight[i] : 1.0;
    int best = 0;
    double bd = fabs(x - c[0]);
#pragma unroll
    for (int j = 1; j < K; ++j) {
      const double d = fabs(x - c[j]);
      if (d < bd) { bd = d; best = j; }   // strict: ties keep the smaller index
    }
    const uint8_t old = a.assign[i];
    if (first || old != (uint8_t)best) ++changed;
    a.assign[i] = (uint8_t)best;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const bool m = j == best;
      sw[j] += m ? wt : 0.0;
      swa[j] += m ? wt * x : 0.0;
    }
  }
  // changed assignments (integer: any order)
  if (threadIdx.x == 0) s_cnt = 0;
  __syncthreads();
  atomicAdd(&s_cnt, changed);
  double* part = a.partials + (size_t)blockIdx.x * (2 * K);
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const double t_w = block_sum(sw[j], s_red);
    const double t_wa = block_sum(swa[j], s_red);
    if (threadIdx.x == 0) { part[2 * j] = t_w; part[2 * j + 1] = t_wa; }
  }
  __syncthreads();
  if (threadIdx.x == 0) a.changes[blockIdx.x] = s_cnt;
}

template <int K>
__global__ __launch_bounds__(64) void update_kernel(CodebookArgs a) {
  CodebookState* st = a.state;
  if (st->converged) return;
  const int j = threadIdx.x;
  __shared__ int s_total;
  if (j == 0) {
    int64_t tot = 0;
    for (int r = 0; r < a.n_ranges; ++r) tot += a.changes[r];
    s_total = tot > 0 ? 1 : 0;
  }
  __syncthreads();
  const bool stop = st->iter > 0 && s_total == 0;   // no assignment changed: converged
  if (j < K && !stop) {
    double w = 0.0, wa = 0.0;
    for (int r = 0; r < a.n_ranges; ++r) {
      w += a.partials[(size_t)r * (2 * K) + 2 * j];
      wa += a.partials[(size_t)r * (2 * K) + 2 * j + 1];
    }
    if (w > 0.0) st->centres[j] = wa / w;
  }
  __syncthreads();
  if (j < K) a.out[j] = (float)st->centres[j];
  if (j == 0) {
    if (stop) st->converged = 1;
    else st->iter += 1;
    if (a.iters_out) *a.iters_out = st->iter;
  }
}

__global__ void init_kernel(CodebookArgs a, int k) {
  CodebookState* st = a.state;
  const int j = threadIdx.x;
  if (j < k) {
    st->centres[j] = -1.0 + 2.0 * (double)j / (double)(k - 1);
    a.out[j] = (float)st->centres[j];
  }
  if (j == 0) {
    st->converged = 0;
    st->iter = 0;
    if (a.iters_out) *a.iters_out = 0;
  }
}

template <int K>
hipError_t run(const CodebookArgs& a, int max_iters, hipStream_t s) {
  hipLaunchKernelGGL(init_kernel, dim3(1), dim3(64), 0, s, a, K);
  for (int it = 0; it < max_iters; ++it) {
    hipLaunchKernelGGL((assign_kernel<K>), dim3(a.n_ranges), dim3(kCbThreads), 0, s, a);
    hipLaunchKernelGGL((update_kernel<K>), dim3(1), dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_codebook_build(int bits, const CodebookArgs& a, int max_iters, hipStream_t s) {
  switch (bits) {
    case 2: return run<4>(a, max_iters, s);
    case 3: return run<8>(a, max_iters, s);
    case 4: return run<16>(a, max_iters, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
