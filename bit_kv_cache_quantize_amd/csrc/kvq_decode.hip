// Split-K decode attention reading the packed cache directly.
//
// What is computed ("KVQuant reading notes", Algorithm 1 attention part and 3.7;
// "reproducing TurboQuant" 4.2 and 5.2; "KVarN" method step 5): for every query
// head h of a kv head, softmax(scale * q_h . RoPE(k_hat_n, n)) weighted sum of
// v_hat_n over all cached tokens, where k_hat / v_hat are dequantized in
// registers from the block records (RTN q*s+m, NUQ C[q]*h+z, SYM (u-8)*s, KVarN
// times s1), outlier positions take their fp16 value, and the fp16 tail is
// read as is.
//
// Work decomposition (one workgroup = one split of one (sequence, kv head)):
//   * 4 waves; wave w streams the 64-token halves of parity w&1 of the blocks
//     blo + (w>>1), +2, ... with its own online-softmax state, so the main loop
//     has no barrier. Each lane therefore keeps one token offset j = 64*(w&1)+lane
//     for the whole kernel (its RoPE offset angles live in registers).
//   * q.K: lane = token, full 128-channel row (one coalesced 32/48/64-byte row
//     per lane). Per-block channel constants (query folded with the channel
//     scale, RoPE base rotation) are computed per lane for the channel pair
//     (2*lane, 2*lane+1) and broadcast with v_readlane into scalar registers.
//   * P.V: lane = channel pair, 64 tokens of a channel-major half-row (tokens in
//     the transposed 4-token-group order of the record); the probabilities are
//     broadcast with v_readlane.
//   * the four wave states are merged in LDS; KVarN returns to the original
//     domain with one Hadamard rotation of the merged output; the split's
//     partial (m, l, o) goes to the workspace and a small second kernel merges
//     the splits (log-sum-exp rule); with a single split the workgroup writes
//     the output itself. (Merging inside the kernel through a completion
//     counter needs an agent-scope release per workgroup, i.e. an L2
//     write-back per workgroup, which costs far more than a second launch.)
#include "kvq_decode_common.h"

namespace kvq {
namespace {

using namespace dec;

template <int MODE, int BITS, int G, bool ROPE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void decode_kernel(DecodeArgs a) {
  extern __shared__ __align__(16) uint8_t s_dyn[];
  __shared__ float s_q[G * 128];
  __shared__ float s_lut[32];
  __shared__ float s_theta[64];
  __shared__ float s_p[4][G * 64];
  __shared__ float s_m[4][G], s_l[4][G];
  __shared__ float s_o[4][G * 128];

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  for (int i = tid; i < G * 128; i += kThreads)
    s_q[i] = __half2float(a.q[((size_t)b * a.Hq + (size_t)kvh * G) * 128 + i]);
  if (MODE == NUQ && tid < 32) s_lut[tid] = a.cb[(kvh * 2 + (tid >> 4)) * kCbStride + (tid & 15)];
  if (ROPE && tid < 64) s_theta[tid] = a.rope_off[128 * 64 * 2 + tid];
  __syncthreads();

  Decoder<MODE, BITS, G, ROPE> d(a, lane, w, s_lut, s_p[w], s_q, s_theta, s_dyn + (size_t)w * a.wave_lds);
  float rc[64], rs[64];
  if constexpr (ROPE) {
    const float2* off = reinterpret_cast<const float2*>(a.rope_off) + d.j;   // pair-major: [i][j]
#pragma unroll
    for (int i = 0; i < 64; ++i) { const float2 v = off[i * 128]; rc[i] = v.x; rs[i] = v.y; }
  }

  const int blo = split * a.blocks_per_split;
  const int bhi = min(seq_nblk(a, blockIdx.z), blo + a.blocks_per_split);
  d.run(blo, bhi, rc, rs);
  if (split == a.splits - 1 && 64 * d.par < seq_tail(a, blockIdx.z) && w < 2) d.tail_half(rc, rs);

  // ---- merge the four wave states
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float l = wave_sum(d.l_run[h]);
    if constexpr (MODE == RTN || MODE == NUQ) {
      const float pmw = wave_sum(d.pm[h]);
      d.acc0[h] += pmw;
      d.acc1[h] += pmw;
    }
    if (lane == 0) { s_m[w][h] = d.m_run[h]; s_l[w][h] = l; }
    s_o[w][h * 128 + 2 * lane] = d.acc0[h];
    s_o[w][h * 128 + 2 * lane + 1] = d.acc1[h];
  }
  __syncthreads();
  for (int i = tid; i < G * 128; i += kThreads) {
    const int h = i >> 7;
    float M = fmaxf(fmaxf(s_m[0][h], s_m[1][h]), fmaxf(s_m[2][h], s_m[3][h]));
    float o = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float sw = s_m[ww][h] == -INFINITY ? 0.f : exp2f(s_m[ww][h] - M);
      o = fmaf(sw, s_o[ww][i], o);
    }
    s_o[0][i] = o;
  }
  __syncthreads();
  if constexpr (MODE == KVARN) {
    // merged output is in the rotated domain: one orthonormal Hadamard rotation back
    for (int s = 0; s < 7; ++s) {
      const int hs = 1 << s;
      for (int id = tid; id < G * 64; id += kThreads) {
        const int h = id >> 6, k = id & 63;
        const int i = h * 128 + (((k >> s) << (s + 1)) | (k & (hs - 1)));
        const float x = s_o[0][i], y = s_o[0][i + hs];
        s_o[0][i] = x + y;
        s_o[0][i + hs] = x - y;
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < G * 128; i += kThreads) {
    const int h = i >> 7, c = i & 127;
    const size_t row = (size_t)b * a.Hq + (size_t)kvh * G + h;
    float o = s_o[0][i];
    if constexpr (MODE == KVARN) o *= kInvSqrt128;
    const float M = fmaxf(fmaxf(s_m[0][h], s_m[1][h]), fmaxf(s_m[2][h], s_m[3][h]));
    float L = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww)
      if (s_m[ww][h] != -INFINITY) L = fmaf(exp2f(s_m[ww][h] - M), s_l[ww][h], L);
    if (a.part_slots == 1) {
      a.out[row * kD + c] = o / L;          // one split: this workgroup saw every token
    } else {
      float* part = a.part + (row * a.part_slots + split) * kPartStride;
      part[2 + c] = o;
      if (c == 0) { part[0] = M; part[1] = L; }
    }
  }
}

// Merge the split partials of one (sequence, query head) with the log-sum-exp rule.
// Up to S splits: every partial is loaded up front (indices past the split count read the last
// partial again and are not used), so all loads are in flight together, one memory round trip;
// the merge then runs in split order.
template <int S>
__global__ __launch_bounds__(128) void combine_kernel(const float* part_all, float* out, int Hq, int splits) {
  const int hq = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
  const size_t row = (size_t)b * Hq + hq;
  const float* part = part_all + row * splits * kPartStride;
  float m[S], l[S], o[S];
#pragma unroll
  for (int sp = 0; sp < S; ++sp) {
    const float* p = part + min(sp, splits - 1) * kPartStride;
    m[sp] = p[0];
    l[sp] = p[1];
    o[sp] = p[2 + c];
  }
  // branch-free, so that no load is deferred into a conditional: a repeated last partial does not
  // change the maximum, and it enters the sums with weight 0 (an exact no-op)
  float M = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < S; ++sp) M = fmaxf(M, m[sp]);
  float L = 0.f, acc = 0.f;
#pragma unroll
  for (int sp = 0; sp < S; ++sp) {
    const float wgt = (sp >= splits || m[sp] == -INFINITY) ? 0.f : exp2f(m[sp] - M);
    L = fmaf(wgt, l[sp], L);
    acc = fmaf(wgt, o[sp], acc);
  }
  out[row * kD + c] = acc / L;
}

// The same merge for any split count: the (m, l) pairs of all splits are staged in LDS first,
// so the loads of the per-channel partials are independent and stay in flight together.
__global__ __launch_bounds__(128) void combine_kernel_lds(const float* part_all, float* out, int Hq, int splits) {
  // up to kMaxSplits splits plus the partials of the fp16 part (at most kMaxSplits + 1 in all)
  __shared__ float s_w[kMaxSplits + 1];
  __shared__ float s_l[kMaxSplits + 1];
  const int hq = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
  const size_t row = (size_t)b * Hq + hq;
  const float* part = part_all + row * splits * kPartStride;
  if (c < splits) {
    s_w[c] = part[c * kPartStride];
    s_l[c] = part[c * kPartStride + 1];
  }
  __syncthreads();
  float M = -INFINITY;
  for (int sp = 0; sp < splits; ++sp) M = fmaxf(M, s_w[sp]);
  float L = 0.f, o = 0.f;
#pragma unroll 8
  for (int sp = 0; sp < splits; ++sp) {
    const float m = s_w[sp];
    const float wgt = m == -INFINITY ? 0.f : exp2f(m - M);
    L = fmaf(wgt, s_l[sp], L);
    o = fmaf(wgt, part[sp * kPartStride + 2 + c], o);
  }
  out[row * kD + c] = o / L;
}


template <int MODE, int BITS, int G, bool ROPE>
hipError_t launch_d(const DecodeArgs& a, int batch, hipStream_t s) {
  hipLaunchKernelGGL((decode_kernel<MODE, BITS, G, ROPE>), dim3(a.splits, a.Hkv, batch), dim3(kThreads),
                     (size_t)4 * a.wave_lds, s, a);
  return hipGetLastError();
}

template <int MODE, int BITS, bool ROPE>
hipError_t launch_g(int group, const DecodeArgs& a, int batch, hipStream_t s) {
  switch (group) {
    case 1: return launch_d<MODE, BITS, 1, ROPE>(a, batch, s);
    case 2: return launch_d<MODE, BITS, 2, ROPE>(a, batch, s);
    case 4: return launch_d<MODE, BITS, 4, ROPE>(a, batch, s);
    case 8: return launch_d<MODE, BITS, 8, ROPE>(a, batch, s);
    default: return hipErrorInvalidValue;
  }
}

template <int MODE, int BITS>
hipError_t launch_r(int group, int rope, const DecodeArgs& a, int batch, hipStream_t s) {
  if constexpr (MODE == KVARN) {
    if (rope) return hipErrorInvalidValue;
    return launch_g<MODE, BITS, false>(group, a, batch, s);
  } else {
    return rope ? launch_g<MODE, BITS, true>(group, a, batch, s)
                : launch_g<MODE, BITS, false>(group, a, batch, s);
  }
}

}  // namespace

hipError_t launch_decode(int mode, int bits, int group, int rope, const DecodeArgs& a, int batch,
                         hipStream_t s) {
  switch (mode * 8 + bits) {
    case RTN * 8 + 2: return launch_r<RTN, 2>(group, rope, a, batch, s);
    case RTN * 8 + 3: return launch_r<RTN, 3>(group, rope, a, batch, s);
    case RTN * 8 + 4: return launch_r<RTN, 4>(group, rope, a, batch, s);
    case RTN * 8 + 8: return launch_r<RTN, 8>(group, rope, a, batch, s);
    case NUQ * 8 + 2: return launch_r<NUQ, 2>(group, rope, a, batch, s);
    case NUQ * 8 + 3: return launch_r<NUQ, 3>(group, rope, a, batch, s);
    case NUQ * 8 + 4: return launch_r<NUQ, 4>(group, rope, a, batch, s);
    case KVARN * 8 + 2: return launch_r<KVARN, 2>(group, rope, a, batch, s);
    case KVARN * 8 + 3: return launch_r<KVARN, 3>(group, rope, a, batch, s);
    case KVARN * 8 + 4: return launch_r<KVARN, 4>(group, rope, a, batch, s);
    case KVARN * 8 + 8: return launch_r<KVARN, 8>(group, rope, a, batch, s);
    case SYM * 8 + 4: return launch_r<SYM, 4>(group, rope, a, batch, s);
    case SYM * 8 + 8: return launch_r<SYM, 8>(group, rope, a, batch, s);
    case ASYM * 8 + 4: return launch_r<ASYM, 4>(group, rope, a, batch, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_combine(const float* part, float* out, int Hq, int splits, int batch, hipStream_t s) {
  const dim3 grid(Hq, batch), block(128);
  if (splits <= 4) hipLaunchKernelGGL(combine_kernel<4>, grid, block, 0, s, part, out, Hq, splits);
  else if (splits <= 8) hipLaunchKernelGGL(combine_kernel<8>, grid, block, 0, s, part, out, Hq, splits);
  else if (splits <= 16) hipLaunchKernelGGL(combine_kernel<16>, grid, block, 0, s, part, out, Hq, splits);
  else if (splits <= 32) hipLaunchKernelGGL(combine_kernel<32>, grid, block, 0, s, part, out, Hq, splits);
  else hipLaunchKernelGGL(combine_kernel_lds, grid, block, 0, s, part, out, Hq, splits);
  return hipGetLastError();
}

}  // namespace kvq
