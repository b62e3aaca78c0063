// Decode attention over the fp16 part of a cache that keeps attention-sink tokens or a
// window of recent tokens in fp16 ("KVQuant reading notes" 3.5: the first token in fp16;
// 4.2: KIVI's full-precision window of recent tokens): the sink rows and the body tokens not
// yet quantized, for the G query heads of one (sequence, kv head). The result is one more
// split partial (m, l, o), merged with the quantized blocks' partials by the log-sum-exp
// combine, or the output itself when nothing is quantized.
//
// One workgroup of four waves per (sequence, kv head). Wave w takes 64-token chunks
// w, w + 4, ...: lane = token for the scores (the key row rotated by its absolute position
// when keys are stored before RoPE: cos / sin of the position angle by angle addition from
// the block-base and in-block tables) and for loading the token's value row into LDS, online
// softmax per head, then lane = channel pair for P.V over the staged rows. The four wave
// states merge in LDS.
#include "kvq_decode_common.h"

namespace kvq {
namespace {

using namespace dec;

constexpr int kF16Threads = 256;

template <int G, bool ROPE>
__global__ __launch_bounds__(kF16Threads) void decode_fp16_kernel(DecodeArgs a) {
  __shared__ __align__(16) float s_q[G * 128];
  __shared__ float s_p[4][G][64];
  __shared__ float s_m[4][G], s_l[4][G];
  __shared__ __align__(16) float s_o[4][G][128];
  // each wave's chunk of value rows (fp16), rows padded by 16 bytes so that the 64 lanes'
  // row writes spread over the banks
  __shared__ __align__(16) uint4 s_v[4][64][17];

  const int kvh = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int i = tid; i < G * 128; i += kF16Threads)
    s_q[i] = __half2float(a.q[((size_t)b * a.Hq + (size_t)kvh * G) * 128 + i]) * a.scale_log2;
  __syncthreads();

  const int sink = a.tail_rows - a.ring_rows;   // rows reserved for sink tokens
  const int n_tok = a.sink_n + a.fp16_n;
  const __half* tk = a.tail + (size_t)(b * a.Hkv + kvh) * (size_t)(2 * a.tail_rows * kD);
  const __half* tv = tk + (size_t)a.tail_rows * kD;
  // fp16 row of token t of the list (sink tokens first, then body tokens fp16_u0 ...)
  auto row_of = [&](int t) -> int {
    return t < a.sink_n ? t : sink + (a.fp16_u0 + (t - a.sink_n)) % a.ring_rows;
  };

  float m_run[G], l_run[G], o0[G], o1[G];
#pragma unroll
  for (int h = 0; h < G; ++h) { m_run[h] = -INFINITY; l_run[h] = 0.f; o0[h] = 0.f; o1[h] = 0.f; }

  for (int c0 = 64 * w; c0 < n_tok; c0 += 256) {
    const int t = c0 + lane;
    const bool valid = t < n_tok;
    float sc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) sc[h] = 0.f;
    if (valid) {
      const int row = row_of(t);
      const uint4* vrow = reinterpret_cast<const uint4*>(tv + (size_t)row * kD);
#pragma unroll
      for (int c8 = 0; c8 < 16; ++c8) s_v[w][lane][c8] = vrow[c8];
      const uint4* krow = reinterpret_cast<const uint4*>(tk + (size_t)row * kD);
      // position angle = block base + in-block offset (sink tokens: offset only)
      const float2* base = nullptr;
      const float2* off = reinterpret_cast<const float2*>(a.rope_off);
      int j = t;
      if (ROPE && t >= a.sink_n) {
        const int u = a.fp16_u0 + (t - a.sink_n);
        base = reinterpret_cast<const float2*>(a.rope_base) + (size_t)(u >> 7) * 64;
        j = u & 127;
      }
#pragma unroll 2
      for (int c8 = 0; c8 < 16; ++c8) {
        const uint4 kv = krow[c8];
        const uint32_t kd[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int i = 4 * c8 + k;   // channel pair
          float2 kk = __half22float2(__builtin_bit_cast(__half2, kd[k]));
          if constexpr (ROPE) {
            float2 cs = off[(size_t)i * 128 + j];
            if (base) {
              const float2 bs = base[i];
              cs = make_float2(fmaf(bs.x, cs.x, -bs.y * cs.y), fmaf(bs.y, cs.x, bs.x * cs.y));
            }
            kk = make_float2(fmaf(kk.x, cs.x, -kk.y * cs.y), fmaf(kk.x, cs.y, kk.y * cs.x));
          }
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float2 qq = *reinterpret_cast<const float2*>(s_q + h * 128 + 2 * i);
            sc[h] = fmaf(kk.x, qq.x, fmaf(kk.y, qq.y, sc[h]));
          }
        }
      }
    }
    const int nv = min(64, n_tok - c0);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float sl = valid ? sc[h] : -INFINITY;
      const float mnew = fmaxf(m_run[h], wave_max(sl));
      const float alpha = exp2f(m_run[h] - mnew);
      const float p = valid ? exp2f(sl - mnew) : 0.f;
      l_run[h] = fmaf(l_run[h], alpha, wave_sum(p));
      o0[h] *= alpha;
      o1[h] *= alpha;
      m_run[h] = mnew;
      s_p[w][h][lane] = p;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int tt = 0; tt < nv; ++tt) {
      const float2 vv = __half22float2(reinterpret_cast<const __half2*>(&s_v[w][tt][0])[lane]);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pv = s_p[w][h][tt];
        o0[h] = fmaf(pv, vv.x, o0[h]);
        o1[h] = fmaf(pv, vv.y, o1[h]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (lane == 0) { s_m[w][h] = m_run[h]; s_l[w][h] = l_run[h]; }
    s_o[w][h][2 * lane] = o0[h];
    s_o[w][h][2 * lane + 1] = o1[h];
  }
  __syncthreads();
  for (int i = tid; i < G * 128; i += kF16Threads) {
    const int h = i >> 7, c = i & 127;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, s_m[ww][h]);
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      if (s_m[ww][h] == -INFINITY) continue;
      const float sw = exp2f(s_m[ww][h] - M);
      o = fmaf(sw, s_o[ww][h][c], o);
      L = fmaf(sw, s_l[ww][h], L);
    }
    const size_t row = (size_t)b * a.Hq + (size_t)kvh * G + h;
    if (a.side_slot < 0) {
      a.out[row * kD + c] = o / L;
    } else {
      float* part = a.part + (row * a.part_slots + a.side_slot) * kPartStride;
      part[2 + c] = o;
      if (c == 0) { part[0] = M; part[1] = L; }
    }
  }
}

template <int G>
hipError_t launch_g(int rope, const DecodeArgs& a, int batch, hipStream_t s) {
  if (rope) hipLaunchKernelGGL((decode_fp16_kernel<G, true>), dim3(a.Hkv, batch), dim3(kF16Threads), 0, s, a);
  else hipLaunchKernelGGL((decode_fp16_kernel<G, false>), dim3(a.Hkv, batch), dim3(kF16Threads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_fp16(int group, int rope, const DecodeArgs& a, int batch, hipStream_t s) {
  switch (group) {
    case 1: return launch_g<1>(rope, a, batch, s);
    case 2: return launch_g<2>(rope, a, batch, s);
    case 4: return launch_g<4>(rope, a, batch, s);
    case 8: return launch_g<8>(rope, a, batch, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
