// Device implementation of the seeded input generator described in
// synth/__init__.py (SplitMix64 counter-based words, 16-bit fields indexing
// normal / log-normal quantile tables, single IEEE fp32 operations, fp16 RNE).
// It holds no quantization or attention arithmetic.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t word(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * kGamma); }

__device__ __forceinline__ uint32_t field16(uint64_t key, uint64_t sample) {
  return (uint32_t)(word(key, sample >> 2) >> (16 * (sample & 3))) & 0xFFFFu;
}

// one thread = 4 consecutive channels of one token (one generator word per tensor)
__global__ void fill_kv_kernel(__half* k, __half* v, int Hkv, long long t0, int n_tok, const uint64_t* keys_k,
                               const uint64_t* keys_v, const uint64_t* keys_g, const float* mu, const float* sd,
                               const float* nt, const float* lg) {
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long per_unit = (long long)n_tok * 32;
  const int unit = blockIdx.y;                  // b * Hkv + h
  if (gid >= per_unit) return;
  const int h = unit % Hkv;
  const long long tl = gid >> 5;                // token within this call
  const int c0 = (int)(gid & 31) * 4;
  const long long t = t0 + tl;                  // absolute position
  const uint64_t wk = word(keys_k[unit], (uint64_t)(t * 32 + (c0 >> 2)));
  const uint64_t wv = word(keys_v[unit], (uint64_t)(t * 32 + (c0 >> 2)));
  const float g = lg[field16(keys_g[unit], (uint64_t)t)];
  __half ko[4], vo[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int c = c0 + r;
    const float zk = nt[(wk >> (16 * r)) & 0xFFFF];
    const float zv = nt[(wv >> (16 * r)) & 0xFFFF];
    ko[r] = __float2half_rn(__fadd_rn(mu[h * 128 + c], __fmul_rn(sd[h * 128 + c], zk)));
    vo[r] = __float2half_rn(__fmul_rn(zv, g));
  }
  const size_t off = ((size_t)unit * n_tok + (size_t)tl) * 128 + c0;
  *reinterpret_cast<uint2*>(k + off) = *reinterpret_cast<const uint2*>(ko);
  *reinterpret_cast<uint2*>(v + off) = *reinterpret_cast<const uint2*>(vo);
}

__global__ void fill_q_kernel(__half* q, const uint64_t* keys_q, const float* nt) {
  const int head = blockIdx.x, c = threadIdx.x;
  q[(size_t)head * 128 + c] = __float2half_rn(nt[field16(keys_q[head], (uint64_t)c)]);
}

}  // namespace

extern "C" {

// k, v: fp16 [B][Hkv][n_tok][128] for absolute positions t0 .. t0+n_tok-1.
// keys_*: uint64 [B][Hkv] stream keys; mu, sd: f32 [Hkv][128]; nt, lg: f32 [65536].
int kvqsynth_fill_kv(void* k, void* v, int B, int Hkv, long long t0, int n_tok, const void* keys_k,
                     const void* keys_v, const void* keys_g, const void* mu, const void* sd, const void* nt,
                     const void* lg, void* stream) {
  if (n_tok <= 0) return 0;
  const long long per_unit = (long long)n_tok * 32;
  dim3 grid((unsigned)((per_unit + 255) / 256), (unsigned)(B * Hkv));
  hipLaunchKernelGGL(fill_kv_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<__half*>(k), static_cast<__half*>(v), Hkv, t0, n_tok,
                     static_cast<const uint64_t*>(keys_k), static_cast<const uint64_t*>(keys_v),
                     static_cast<const uint64_t*>(keys_g), static_cast<const float*>(mu),
                     static_cast<const float*>(sd), static_cast<const float*>(nt), static_cast<const float*>(lg));
  return (int)hipGetLastError();
}

// q: fp16 [n_heads_total][128]; keys_q: uint64 [n_heads_total]
int kvqsynth_fill_q(void* q, int n_heads_total, const void* keys_q, const void* nt, void* stream) {
  hipLaunchKernelGGL(fill_q_kernel, dim3(n_heads_total), dim3(128), 0, static_cast<hipStream_t>(stream),
                     static_cast<__half*>(q), static_cast<const uint64_t*>(keys_q), static_cast<const float*>(nt));
  return (int)hipGetLastError();
}

}
