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
//   * P.V: lane = channel pair, 64 tokens of a channel-major half-row; the
//     probabilities are broadcast with v_readlane.
//   * the four wave states are merged in LDS; KVarN returns to the original
//     domain with one Hadamard rotation of the merged output; the split's
//     partial (m, l, o) goes to the workspace, and the last split of a
//     (sequence, kv head) to finish merges all of them (log-sum-exp rule) and
//     writes the output, so one decode call is one kernel launch.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr float kInvSqrt128 = 0.08838834764831845f;

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

// Orthonormal 128-point Hadamard transform of a vector held as channel pairs
// (2*lane, 2*lane+1) across the 64 lanes of a wave.
__device__ __forceinline__ void fwht_wave(float& x, float& y, int lane) {
  float a = x + y, b = x - y;        // channel bit 0 inside the lane
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {  // channel bits 1..6 = lane bits 0..5
    const float pa = __shfl_xor(a, m), pb = __shfl_xor(b, m);
    const bool hi = (lane & m) != 0;
    a = hi ? pa - a : a + pa;
    b = hi ? pb - b : b + pb;
  }
  x = a * kInvSqrt128;
  y = b * kInvSqrt128;
}

// code of element i of a packed row of n codes held in registers w[]
template <int BITS, int N>
__device__ __forceinline__ uint32_t code_at(const uint32_t* w, int i) {
  if constexpr (BITS == 4) {
    return (w[i >> 3] >> (4 * (i & 7))) & 15u;
  } else if constexpr (BITS == 2) {
    return (w[i >> 4] >> (2 * (i & 15))) & 3u;
  } else {
    const uint32_t lo = (w[i >> 4] >> (2 * (i & 15))) & 3u;
    const uint32_t hi = (w[N / 16 + (i >> 5)] >> (i & 31)) & 1u;
    return lo | (hi << 2);
  }
}

// code of element i of a packed row in memory (used for the sparse outlier fix-ups)
template <int BITS, int N>
__device__ __forceinline__ uint32_t code_mem(const uint8_t* row, int i) {
  if constexpr (BITS == 4) {
    return (row[i >> 1] >> (4 * (i & 1))) & 15u;
  } else if constexpr (BITS == 2) {
    return (row[i >> 2] >> (2 * (i & 3))) & 3u;
  } else {
    const uint32_t lo = (row[i >> 2] >> (2 * (i & 3))) & 3u;
    const uint32_t hi = (row[N / 4 + (i >> 3)] >> (i & 7)) & 1u;
    return lo | (hi << 2);
  }
}

template <int NBYTES>
__device__ __forceinline__ void load_row(uint32_t* w, const uint8_t* p) {
  static_assert(NBYTES % 8 == 0, "row bytes");
  if constexpr (NBYTES % 16 == 0) {
#pragma unroll
    for (int k = 0; k < NBYTES / 16; ++k) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[k];
      w[4 * k] = v.x; w[4 * k + 1] = v.y; w[4 * k + 2] = v.z; w[4 * k + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < NBYTES / 8; ++k) {
      const uint2 v = reinterpret_cast<const uint2*>(p)[k];
      w[2 * k] = v.x; w[2 * k + 1] = v.y;
    }
  }
}

template <int MODE, int BITS, int G, bool ROPE>
struct Decoder {
  static constexpr int R = 16 * BITS;      // bytes per 128 codes
  static constexpr int RH = R / 2;         // bytes per 64 codes

  const DecodeArgs& a;
  const int lane, w, par, j;
  const float* lut;                        // NUQ: [0,16) keys, [16,32) values
  float* pbuf;                             // this wave's probabilities [G][64]
  const float* qs;                         // query, original domain [G][128]
  float qx[G], qy[G];                      // query pair (2*lane, 2*lane+1), rotated for KVarN
  float m_run[G], l_run[G], pm[G], acc0[G], acc1[G];

  __device__ Decoder(const DecodeArgs& args, int lane_, int w_, const float* lut_, float* pbuf_,
                     const float* qs_)
      : a(args), lane(lane_), w(w_), par(w_ & 1), j(64 * (w_ & 1) + lane_), lut(lut_), pbuf(pbuf_),
        qs(qs_) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      qx[h] = qs[h * 128 + 2 * lane];
      qy[h] = qs[h * 128 + 2 * lane + 1];
      if constexpr (MODE == KVARN) fwht_wave(qx[h], qy[h], lane);
      m_run[h] = -INFINITY; l_run[h] = 0.f; pm[h] = 0.f; acc0[h] = 0.f; acc1[h] = 0.f;
    }
  }

  __device__ __forceinline__ float kval(uint32_t code) const {
    if constexpr (MODE == NUQ) return lut[code];
    else return (float)code;
  }
  __device__ __forceinline__ float vval(uint32_t code) const {
    if constexpr (MODE == NUQ) return lut[16 + code];
    else return (float)code;
  }

  // per-channel key statistics of channel c as (S, M): x = val(code) * S + M
  __device__ __forceinline__ void kstat(const uint8_t* rec, int c, float& S, float& M) const {
    if constexpr (MODE == SYM) {
      S = __half2float(reinterpret_cast<const __half*>(rec + a.lay.ks)[c]);
      M = -8.f * S;
    } else if constexpr (MODE == NUQ) {
      M = reinterpret_cast<const float*>(rec + a.lay.ks)[c];
      S = reinterpret_cast<const float*>(rec + a.lay.ks)[128 + c];
    } else {
      S = reinterpret_cast<const float*>(rec + a.lay.ks)[c];
      M = reinterpret_cast<const float*>(rec + a.lay.ks)[128 + c];
    }
  }

  // Online-softmax update with this lane's log2-domain scores sl[h]; returns p[h].
  __device__ __forceinline__ void softmax_step(float* sl, float* p) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mnew = fmaxf(m_run[h], wave_max(sl[h]));
      const float alpha = exp2f(m_run[h] - mnew);
      p[h] = exp2f(sl[h] - mnew);
      m_run[h] = mnew;
      l_run[h] = l_run[h] * alpha + p[h];
      pm[h] *= alpha;
      acc0[h] *= alpha;
      acc1[h] *= alpha;
    }
  }

  // One 64-token half (parity par) of block blk.
  __device__ void half_block(int blk, const float (&rc)[64], const float (&rs)[64]) {
    const uint8_t* rec = a.rec + ((size_t)(blockIdx.z * a.Hkv + blockIdx.y) * a.max_blocks + blk) *
                                     (size_t)a.lay.rec_bytes;
    // ---- q . K for token j
    uint32_t kw[R / 4];
    load_row<R>(kw, rec + a.lay.kc + (size_t)j * R);
    float Sx, Sy, Mx, My;
    kstat(rec, 2 * lane, Sx, Mx);
    kstat(rec, 2 * lane + 1, Sy, My);
    float sc[G];
    if constexpr (!ROPE) {
      float QSx[G], QSy[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        QSx[h] = qx[h] * Sx;
        QSy[h] = qy[h] * Sy;
        sc[h] = wave_sum(fmaf(qx[h], Mx, qy[h] * My));   // sum_c q_c * M_c
      }
#pragma unroll
      for (int i = 0; i < 64; ++i) {
        const float vx = kval(code_at<BITS, 128>(kw, 2 * i));
        const float vy = kval(code_at<BITS, 128>(kw, 2 * i + 1));
#pragma unroll
        for (int h = 0; h < G; ++h) {
          sc[h] = fmaf(vx, readlane_f(QSx[h], i), sc[h]);
          sc[h] = fmaf(vy, readlane_f(QSy[h], i), sc[h]);
        }
      }
    } else {
      // rotate the query pair back by the block base angle n0*theta_i (angle addition)
      const float2 cs0 = reinterpret_cast<const float2*>(a.rope_base)[(size_t)blk * 64 + lane];
      float P1[G], P2[G], P3[G], P4[G], P5[G], P6[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float al = fmaf(qx[h], cs0.x, qy[h] * cs0.y);
        const float be = fmaf(qy[h], cs0.x, -qx[h] * cs0.y);
        P1[h] = al * Sx; P2[h] = be * Sy; P3[h] = fmaf(al, Mx, be * My);
        P4[h] = be * Sx; P5[h] = -al * Sy; P6[h] = fmaf(be, Mx, -al * My);
        sc[h] = 0.f;
      }
#pragma unroll
      for (int i = 0; i < 64; ++i) {
        const float vx = kval(code_at<BITS, 128>(kw, 2 * i));
        const float vy = kval(code_at<BITS, 128>(kw, 2 * i + 1));
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float U = fmaf(vx, readlane_f(P1[h], i), fmaf(vy, readlane_f(P2[h], i), readlane_f(P3[h], i)));
          const float W = fmaf(vx, readlane_f(P4[h], i), fmaf(vy, readlane_f(P5[h], i), readlane_f(P6[h], i)));
          sc[h] = fmaf(rc[i], U, fmaf(rs[i], W, sc[h]));
        }
      }
    }
    if constexpr (MODE != KVARN) {
      if (a.k_out > 0) {
        // key outliers of row j (CSR): replace the dense value by the fp16 one
        const uint16_t* ptr = reinterpret_cast<const uint16_t*>(rec + a.lay.ko_ptr);
        const uint8_t* idx = rec + a.lay.ko_idx;
        const __half* val = reinterpret_cast<const __half*>(rec + a.lay.ko_val);
        const int e1 = ptr[j + 1];
        for (int e = ptr[j]; e < e1; ++e) {
          const int c = idx[e];
          float S, M;
          kstat(rec, c, S, M);
          const float dense = fmaf(kval(code_mem<BITS, 128>(rec + a.lay.kc + (size_t)j * R, c)), S, M);
          const float delta = __half2float(val[e]) - dense;
#pragma unroll
          for (int h = 0; h < G; ++h) {
            float coef;
            if constexpr (ROPE) {
              const int i = c >> 1;
              const float2 cs0 = reinterpret_cast<const float2*>(a.rope_base)[(size_t)blk * 64 + i];
              const float2 csj = reinterpret_cast<const float2*>(a.rope_off)[j * 64 + i];
              const float cp = cs0.x * csj.x - cs0.y * csj.y;
              const float sp = cs0.y * csj.x + cs0.x * csj.y;
              const float qa = qs[h * 128 + 2 * i], qb = qs[h * 128 + 2 * i + 1];
              coef = (c & 1) ? qb * cp - qa * sp : qa * cp + qb * sp;
            } else {
              coef = qs[h * 128 + c];
            }
            sc[h] = fmaf(delta, coef, sc[h]);
          }
        }
      }
    }
    float sl[G], p[G];
    float s1t = 1.f;
    if constexpr (MODE == KVARN) s1t = reinterpret_cast<const float*>(rec + a.lay.k1)[j];
#pragma unroll
    for (int h = 0; h < G; ++h) sl[h] = sc[h] * s1t * a.scale_log2;
    softmax_step(sl, p);

    // ---- P . V over the 64 tokens of this half, channel pair (2*lane, 2*lane+1)
    float pp[G], pmb[G];
    if constexpr (MODE == SYM) {
#pragma unroll
      for (int h = 0; h < G; ++h) { pp[h] = p[h]; pmb[h] = wave_sum(p[h]); }
    } else {
      float S_t, M_t;
      if constexpr (MODE == NUQ) {
        M_t = reinterpret_cast<const float*>(rec + a.lay.vs)[j];
        S_t = reinterpret_cast<const float*>(rec + a.lay.vs)[128 + j];
      } else {
        S_t = reinterpret_cast<const float*>(rec + a.lay.vs)[j];
        M_t = reinterpret_cast<const float*>(rec + a.lay.vs)[128 + j];
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        pp[h] = p[h] * S_t;
        if constexpr (MODE == KVARN) pmb[h] = wave_sum(p[h] * M_t);
        else pm[h] = fmaf(p[h], M_t, pm[h]);
      }
    }
    if (a.k_out > 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) pbuf[h * 64 + lane] = p[h];
    }
    uint32_t vw[R / 4];
    const uint8_t* vbase = rec + a.lay.vc + (size_t)par * (128 * RH);
    load_row<R>(vw, vbase + (size_t)lane * R);          // rows 2*lane and 2*lane+1
    float o0[G], o1[G];
#pragma unroll
    for (int h = 0; h < G; ++h) { o0[h] = 0.f; o1[h] = 0.f; }
#pragma unroll
    for (int t = 0; t < 64; ++t) {
      const float v0 = vval(code_at<BITS, 64>(vw, t));
      const float v1 = vval(code_at<BITS, 64>(vw + R / 8, t));
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pv = readlane_f(pp[h], t);
        o0[h] = fmaf(pv, v0, o0[h]);
        o1[h] = fmaf(pv, v1, o1[h]);
      }
    }
    if constexpr (MODE == KVARN) {
      const float2 s1c = reinterpret_cast<const float2*>(rec + a.lay.v1)[lane];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        acc0[h] = fmaf(s1c.x, o0[h] + pmb[h], acc0[h]);
        acc1[h] = fmaf(s1c.y, o1[h] + pmb[h], acc1[h]);
      }
    } else if constexpr (MODE == SYM) {
      const __half2 sc2 = reinterpret_cast<const __half2*>(rec + a.lay.vs)[lane];
      const float s0 = __low2float(sc2), s1 = __high2float(sc2);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        acc0[h] = fmaf(s0, fmaf(-8.f, pmb[h], o0[h]), acc0[h]);
        acc1[h] = fmaf(s1, fmaf(-8.f, pmb[h], o1[h]), acc1[h]);
      }
    } else {
#pragma unroll
      for (int h = 0; h < G; ++h) { acc0[h] += o0[h]; acc1[h] += o1[h]; }
    }
    if constexpr (MODE != KVARN) {
      if (a.k_out > 0) {
        // value outliers of channels 2*lane, 2*lane+1 (CSC) that fall in this half
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const uint16_t* ptr = reinterpret_cast<const uint16_t*>(rec + a.lay.vo_ptr);
        const uint8_t* idx = rec + a.lay.vo_idx;
        const __half* val = reinterpret_cast<const __half*>(rec + a.lay.vo_val);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int c = 2 * lane + k;
          const int e1 = ptr[c + 1];
          for (int e = ptr[c]; e < e1; ++e) {
            const int t = idx[e] - 64 * par;
            if (t < 0 || t >= 64) continue;
            const uint32_t code = code_mem<BITS, 64>(vbase + (size_t)c * RH, t);
            float dense;
            if constexpr (MODE == SYM) {
              const float S = __half2float(reinterpret_cast<const __half*>(rec + a.lay.vs)[c]);
              dense = ((float)code - 8.f) * S;
            } else if constexpr (MODE == NUQ) {
              const float Z = reinterpret_cast<const float*>(rec + a.lay.vs)[64 * par + t];
              const float H = reinterpret_cast<const float*>(rec + a.lay.vs)[128 + 64 * par + t];
              dense = fmaf(vval(code), H, Z);
            } else {
              const float S = reinterpret_cast<const float*>(rec + a.lay.vs)[64 * par + t];
              const float M = reinterpret_cast<const float*>(rec + a.lay.vs)[128 + 64 * par + t];
              dense = fmaf(vval(code), S, M);
            }
            const float delta = __half2float(val[e]) - dense;
#pragma unroll
            for (int h = 0; h < G; ++h) {
              if (k == 0) acc0[h] = fmaf(pbuf[h * 64 + t], delta, acc0[h]);
              else acc1[h] = fmaf(pbuf[h * 64 + t], delta, acc1[h]);
            }
          }
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
  }

  // Tokens 64*par .. 64*par+63 of the fp16 tail (n_valid of them), position 128*nblk + j.
  __device__ void tail_half(const float (&rc)[64], const float (&rs)[64]) {
    const int n_valid = min(64, a.tail_n - 64 * par);
    const __half* tk = a.tail + (size_t)(blockIdx.z * a.Hkv + blockIdx.y) * (2 * kT * kD);
    const __half* tv = tk + kT * kD;
    const bool valid = lane < n_valid;
    float sc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) sc[h] = 0.f;
    // query in the original domain
    float ox[G], oy[G];
#pragma unroll
    for (int h = 0; h < G; ++h) { ox[h] = qs[h * 128 + 2 * lane]; oy[h] = qs[h * 128 + 2 * lane + 1]; }
    const __half2* krow = reinterpret_cast<const __half2*>(tk + (size_t)j * kD);
    if constexpr (!ROPE) {
#pragma unroll 8
      for (int i = 0; i < 64; ++i) {
        const float2 kk = valid ? __half22float2(krow[i]) : make_float2(0.f, 0.f);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          sc[h] = fmaf(kk.x, readlane_f(ox[h], i), sc[h]);
          sc[h] = fmaf(kk.y, readlane_f(oy[h], i), sc[h]);
        }
      }
    } else {
      const float2 cs0 = reinterpret_cast<const float2*>(a.rope_base)[(size_t)a.nblk * 64 + lane];
      float AL[G], BE[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        AL[h] = fmaf(ox[h], cs0.x, oy[h] * cs0.y);
        BE[h] = fmaf(oy[h], cs0.x, -ox[h] * cs0.y);
      }
#pragma unroll
      for (int i = 0; i < 64; ++i) {
        const float2 kk = valid ? __half22float2(krow[i]) : make_float2(0.f, 0.f);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float al = readlane_f(AL[h], i), be = readlane_f(BE[h], i);
          const float U = fmaf(kk.x, al, kk.y * be);
          const float W = fmaf(kk.x, be, -kk.y * al);
          sc[h] = fmaf(rc[i], U, fmaf(rs[i], W, sc[h]));
        }
      }
    }
    float sl[G], p[G];
#pragma unroll
    for (int h = 0; h < G; ++h) sl[h] = valid ? sc[h] * a.scale_log2 : -INFINITY;
    softmax_step(sl, p);
    float o0[G], o1[G];
#pragma unroll
    for (int h = 0; h < G; ++h) { o0[h] = 0.f; o1[h] = 0.f; }
    const __half2* vcol = reinterpret_cast<const __half2*>(tv + (size_t)(64 * par) * kD) + lane;
    for (int t = 0; t < n_valid; ++t) {
      const float2 vv = __half22float2(vcol[(size_t)t * (kD / 2)]);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pv = readlane_f(p[h], t);
        o0[h] = fmaf(pv, vv.x, o0[h]);
        o1[h] = fmaf(pv, vv.y, o1[h]);
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if constexpr (MODE == KVARN) fwht_wave(o0[h], o1[h], lane);   // into the rotated domain
      acc0[h] += o0[h];
      acc1[h] += o1[h];
    }
  }
};

template <int MODE, int BITS, int G, bool ROPE>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  __shared__ float s_q[G * 128];
  __shared__ float s_lut[32];
  __shared__ float s_p[4][G * 64];
  __shared__ float s_m[4][G], s_l[4][G];
  __shared__ float s_o[4][G * 128];

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  for (int i = tid; i < G * 128; i += kThreads)
    s_q[i] = __half2float(a.q[((size_t)b * a.Hq + (size_t)kvh * G) * 128 + i]);
  if (MODE == NUQ && tid < 32) s_lut[tid] = a.cb[(kvh * 2 + (tid >> 4)) * 16 + (tid & 15)];
  __syncthreads();

  Decoder<MODE, BITS, G, ROPE> d(a, lane, w, s_lut, s_p[w], s_q);
  float rc[64], rs[64];
  if constexpr (ROPE) {
    const float2* off = reinterpret_cast<const float2*>(a.rope_off) + (size_t)d.j * 64;
#pragma unroll
    for (int i = 0; i < 64; ++i) { const float2 v = off[i]; rc[i] = v.x; rs[i] = v.y; }
  }

  const int blo = split * a.blocks_per_split;
  const int bhi = min(a.nblk, blo + a.blocks_per_split);
  for (int blk = blo + (w >> 1); blk < bhi; blk += 2) d.half_block(blk, rc, rs);
  if (split == a.splits - 1 && 64 * d.par < a.tail_n && w < 2) d.tail_half(rc, rs);

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
    float* part = a.part + (((size_t)b * a.Hq + (size_t)kvh * G + h) * a.splits + split) * kPartStride;
    float o = s_o[0][i];
    if constexpr (MODE == KVARN) o *= kInvSqrt128;
    part[2 + c] = o;
    if (c == 0) {
      const float M = fmaxf(fmaxf(s_m[0][h], s_m[1][h]), fmaxf(s_m[2][h], s_m[3][h]));
      float L = 0.f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww)
        if (s_m[ww][h] != -INFINITY) L = fmaf(exp2f(s_m[ww][h] - M), s_l[ww][h], L);
      part[0] = M;
      part[1] = L;
    }
  }

  // ---- the last split of this (sequence, kv head) to finish merges all splits
  // (log-sum-exp rule) and writes the output; it then clears the counter.
  __shared__ int s_last;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  const size_t unit = (size_t)b * a.Hkv + kvh;
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(a.counters + unit, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (unsigned)(a.splits - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  for (int i = tid; i < G * 128; i += kThreads) {
    const int h = i >> 7, c = i & 127;
    const size_t row = (size_t)b * a.Hq + (size_t)kvh * G + h;
    const float* part = a.part + row * a.splits * kPartStride;
    float M = -INFINITY;
    for (int sp = 0; sp < a.splits; ++sp) M = fmaxf(M, part[sp * kPartStride]);
    float L = 0.f, o = 0.f;
    for (int sp = 0; sp < a.splits; ++sp) {
      const float m = part[sp * kPartStride];
      if (m == -INFINITY) continue;
      const float wgt = exp2f(m - M);
      L = fmaf(wgt, part[sp * kPartStride + 1], L);
      o = fmaf(wgt, part[sp * kPartStride + 2 + c], o);
    }
    a.out[row * kD + c] = o / L;
  }
  if (tid == 0) __hip_atomic_store(a.counters + unit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void zero_kernel(unsigned* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

template <int MODE, int BITS, int G, bool ROPE>
hipError_t launch_d(const DecodeArgs& a, int batch, hipStream_t s) {
  hipLaunchKernelGGL((decode_kernel<MODE, BITS, G, ROPE>), dim3(a.splits, a.Hkv, batch), dim3(kThreads),
                     0, s, a);
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
    case NUQ * 8 + 2: return launch_r<NUQ, 2>(group, rope, a, batch, s);
    case NUQ * 8 + 3: return launch_r<NUQ, 3>(group, rope, a, batch, s);
    case NUQ * 8 + 4: return launch_r<NUQ, 4>(group, rope, a, batch, s);
    case KVARN * 8 + 2: return launch_r<KVARN, 2>(group, rope, a, batch, s);
    case KVARN * 8 + 3: return launch_r<KVARN, 3>(group, rope, a, batch, s);
    case KVARN * 8 + 4: return launch_r<KVARN, 4>(group, rope, a, batch, s);
    case SYM * 8 + 4: return launch_r<SYM, 4>(group, rope, a, batch, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_zero(unsigned* p, size_t n, hipStream_t s) {
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace kvq
