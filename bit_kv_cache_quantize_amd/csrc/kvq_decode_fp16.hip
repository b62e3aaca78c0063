// Decode attention over the fp16 part of a cache that keeps attention-sink tokens or a
// window of recent tokens in fp16 ("KVQuant reading notes" 3.5: the first token in fp16;
// 4.2: KIVI's full-precision window of recent tokens): the sink rows and the body tokens not
// yet quantized, for the G query heads of one (sequence, kv head). The result is one more
// split partial (m, l, o), merged with the quantized blocks' partials by the log-sum-exp
// combine, or the output itself when nothing is quantized.
//
// One workgroup of four waves per chunk of the fp16 part of a (sequence, kv head): the host
// cuts the part into chunks of whole 16-token groups, one partial each, as many as the free
// partial slots allow. Wave w takes the chunk's 16-token groups w, w + 4, ...; four lanes
// share a token, each with 16 of its 64 channel pairs, and issue all of their loads for the
// group at once (key and value quarter rows, and for keys stored before RoPE the in-block and
// block-base angles of their pairs), so that a group costs one memory round trip. The key
// quarter is rotated by the token's absolute position (angle addition of the two tables), its
// partial scores are summed over the token's four lanes, the online softmax runs per head,
// and the value quarters staged in LDS feed P.V with lane = channel pair. The four wave
// states merge in LDS into the chunk's partial.
#include "kvq_decode_common.h"

namespace kvq {
namespace {

using namespace dec;

constexpr int kGroup = 16;   // tokens per wave and step
// waves per workgroup (512 threads leave each wave the registers for all of its loads)
template <int G> constexpr int fp16_waves() { return 4; }   // waves per workgroup

template <int G, bool ROPE>
__global__ __launch_bounds__(64 * fp16_waves<G>()) __attribute__((amdgpu_waves_per_eu(G >= 8 ? 1 : 2, 2))) void decode_fp16_kernel(DecodeArgs a) {
  constexpr int NW = fp16_waves<G>(), NT = 64 * NW;
  __shared__ __align__(16) float s_q[G * 128];
  __shared__ float s_p[NW][G][kGroup];
  __shared__ float s_m[NW][G], s_l[NW][G];
  __shared__ __align__(16) float s_o[NW][G][128];
  // each wave's group of value rows (fp16), rows padded by 16 bytes against bank conflicts
  __shared__ __align__(16) uint4 s_v[NW][kGroup][17];

  const int kvh = blockIdx.x, b = blockIdx.y, z = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tk = lane >> 2, qq = lane & 3;   // token of the group, quarter of its channels
  for (int i = tid; i < G * 128; i += NT)
    s_q[i] = __half2float(a.q[((size_t)b * a.Hq + (size_t)kvh * G) * 128 + i]) * a.scale_log2;
  __syncthreads();

  const int sink = a.tail_rows - a.ring_rows;   // rows reserved for sink tokens
  const int n_tok = a.sink_n + a.fp16_n;
  const __half* tk_rows = a.tail + (size_t)(b * a.Hkv + kvh) * (size_t)(2 * a.tail_rows * kD);
  const __half* tv_rows = tk_rows + (size_t)a.tail_rows * kD;
  // fp16 row of token t of the list (sink tokens first, then body tokens fp16_u0 ...)
  auto row_of = [&](int t) -> int {
    return t < a.sink_n ? t : sink + (a.fp16_u0 + (t - a.sink_n)) % a.ring_rows;
  };

  float m_run[G], l_run[G], o0[G], o1[G];
#pragma unroll
  for (int h = 0; h < G; ++h) { m_run[h] = -INFINITY; l_run[h] = 0.f; o0[h] = 0.f; o1[h] = 0.f; }

  const int t0 = z * a.side_chunk, t1 = min(n_tok, t0 + a.side_chunk);   // this chunk's tokens
  for (int c0 = t0 + kGroup * w; c0 < t1; c0 += NW * kGroup) {
    const int t = c0 + tk;
    const bool valid = t < t1;
    const int tc = min(t, t1 - 1);   // lanes past the end load the chunk's last token (masked below)
    const int row = row_of(tc);
    // ---- every load of the group first (the value quarter first: it is stored to LDS first)
    uint4 kq[4], vq[4];
    const uint4* krow = reinterpret_cast<const uint4*>(tk_rows + (size_t)row * kD) + 4 * qq;
    const uint4* vrow = reinterpret_cast<const uint4*>(tv_rows + (size_t)row * kD) + 4 * qq;
#pragma unroll
    for (int k = 0; k < 4; ++k) vq[k] = vrow[k];
#pragma unroll
    for (int k = 0; k < 4; ++k) kq[k] = krow[k];
    float2 cs[16], bs[16];
    bool body = false;
    if constexpr (ROPE) {
      // position angle = block base + in-block offset (sink tokens: the offset only)
      body = tc >= a.sink_n;
      const int u = a.fp16_u0 + (tc - a.sink_n);
      const int j = body ? (u & 127) : tc;
      const float2* off = reinterpret_cast<const float2*>(a.rope_off) + (size_t)(16 * qq) * 128 + j;
      const float2* base = reinterpret_cast<const float2*>(a.rope_base) + (size_t)(body ? u >> 7 : 0) * 64 + 16 * qq;
#pragma unroll
      for (int p = 0; p < 16; ++p) { cs[p] = off[(size_t)p * 128]; bs[p] = base[p]; }
    }
    __builtin_amdgcn_sched_barrier(0);   // all of the group's loads in flight before the first use
    // ---- the value quarter into LDS, the partial scores of this quarter
#pragma unroll
    for (int k = 0; k < 4; ++k) s_v[w][tk][4 * qq + k] = vq[k];
    float sc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) sc[h] = 0.f;
    // with 8 heads the query reads stay inside the loop (hoisted out of it, the 256 values per
    // lane would exceed the registers): an opaque zero offset
    int qz = 0;
    if constexpr (G >= 8) asm volatile("" : "+v"(qz));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t kd[4] = {kq[k].x, kq[k].y, kq[k].z, kq[k].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int p = 4 * k + e, i = 16 * qq + p;   // channel pair
        float2 kk = __half22float2(__builtin_bit_cast(__half2, kd[e]));
        if constexpr (ROPE) {
          float2 c = cs[p];
          if (body) c = make_float2(fmaf(bs[p].x, c.x, -bs[p].y * c.y), fmaf(bs[p].y, c.x, bs[p].x * c.y));
          kk = make_float2(fmaf(kk.x, c.x, -kk.y * c.y), fmaf(kk.x, c.y, kk.y * c.x));
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float2 qv = *reinterpret_cast<const float2*>(s_q + qz + h * 128 + 2 * i);
          sc[h] = fmaf(kk.x, qv.x, fmaf(kk.y, qv.y, sc[h]));
        }
      }
    }
    // ---- the token's score (sum over its four lanes), online softmax per head
    const int nv = min(kGroup, t1 - c0);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float v = sc[h];
      v += dpp_f<0xB1>(v);   // quad_perm(1, 0, 3, 2)
      v += dpp_f<0x4E>(v);   // quad_perm(2, 3, 0, 1)
      const float sl = valid ? v : -INFINITY;
      const float mnew = fmaxf(m_run[h], wave_max(sl));
      const float alpha = exp2f(m_run[h] - mnew);
      const float p = valid ? exp2f(sl - mnew) : 0.f;
      l_run[h] = fmaf(l_run[h], alpha, wave_sum(qq == 0 ? p : 0.f));
      o0[h] *= alpha;
      o1[h] *= alpha;
      m_run[h] = mnew;
      if (qq == 0) s_p[w][h][tk] = p;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ---- P.V over the group's staged rows, lane = channel pair
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
  for (int i = tid; i < G * 128; i += NT) {
    const int h = i >> 7, c = i & 127;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, s_m[ww][h]);
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      if (s_m[ww][h] == -INFINITY) continue;
      const float sw = exp2f(s_m[ww][h] - M);
      o = fmaf(sw, s_o[ww][h][c], o);
      L = fmaf(sw, s_l[ww][h], L);
    }
    const size_t row = (size_t)b * a.Hq + (size_t)kvh * G + h;
    if (a.side_slot < 0) {
      a.out[row * kD + c] = o / L;
    } else {
      float* part = a.part + (row * a.part_slots + a.side_slot + z) * kPartStride;
      part[2 + c] = o;
      if (c == 0) { part[0] = M; part[1] = L; }
    }
  }
}

template <int G>
hipError_t launch_g(int rope, const DecodeArgs& a, int batch, int n_side, hipStream_t s) {
  const dim3 grid(a.Hkv, batch, n_side), block(64 * fp16_waves<G>());
  if (rope) hipLaunchKernelGGL((decode_fp16_kernel<G, true>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((decode_fp16_kernel<G, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_fp16(int group, int rope, const DecodeArgs& a, int batch, int n_side, hipStream_t s) {
  static_assert(kSideChunk == kGroup * 4, "one group per wave and chunk");
  switch (group) {
    case 1: return launch_g<1>(rope, a, batch, n_side, s);
    case 2: return launch_g<2>(rope, a, batch, n_side, s);
    case 4: return launch_g<4>(rope, a, batch, n_side, s);
    case 8: return launch_g<8>(rope, a, batch, n_side, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
