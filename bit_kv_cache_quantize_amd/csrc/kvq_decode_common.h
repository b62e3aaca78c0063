// Device helpers shared by the decode kernels (VALU and matrix-core paths):
// wave reductions, the orthonormal Hadamard transform of a wave-held vector,
// packed-code extraction and the VALU half-block decoder (also used for the
// fp16 tail by the matrix-core kernel).
#pragma once
#include "kvq_internal.h"

namespace kvq {
namespace dec {


constexpr int kThreads = 256;
constexpr float kInvSqrt128 = 0.08838834764831845f;

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Wave reductions: data-parallel-primitive moves combine the lanes of each 16-lane row
// (swap neighbours, swap pairs, mirror within 8, mirror within 16), then the four row
// results are read as scalars. Every lane returns the same value.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);    // quad_perm(1, 0, 3, 2)
  v += dpp_f<0x4E>(v);    // quad_perm(2, 3, 0, 1)
  v += dpp_f<0x141>(v);   // row_half_mirror
  v += dpp_f<0x140>(v);   // row_mirror
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}

// Maximum of non-NaN values on their integer images: flipping the magnitude bits of
// negative values makes signed integer order equal float order, and the integer max fuses
// with the lane moves (one instruction per step; a float max would first quiet its inputs).
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}

// The integer image (an involution: it also maps an image back to its float's bits).
__device__ __forceinline__ int ord_image(int b) { return b ^ ((b >> 31) & 0x7FFFFFFF); }

// Maximum over the wave as an integer image (a scalar: callers can keep running maxima in
// this form and compare them on the scalar unit).
__device__ __forceinline__ int wave_max_ord(float x) {
  int v = ord_image(__float_as_int(x));
  v = max(v, dpp_i<0xB1>(v));
  v = max(v, dpp_i<0x4E>(v));
  v = max(v, dpp_i<0x141>(v));
  v = max(v, dpp_i<0x140>(v));
  return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

__device__ __forceinline__ float wave_max(float x) { return __int_as_float(ord_image(wave_max_ord(x))); }

// Bit pattern of the maximum of non-negative values (the integer order of their bit
// patterns is their order; a negative value is never above a non-negative one). The result
// is a scalar: callers derive powers of two from its exponent field with scalar operations.
__device__ __forceinline__ int wave_max_bits_nonneg(float x) {
  int v = __float_as_int(x);
  v = max(v, dpp_i<0xB1>(v));
  v = max(v, dpp_i<0x4E>(v));
  v = max(v, dpp_i<0x141>(v));
  v = max(v, dpp_i<0x140>(v));
  return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
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
  if constexpr (BITS == 8) {
    return (w[i >> 2] >> (8 * (i & 3))) & 255u;
  } else if constexpr (BITS == 4) {
    return (w[i >> 3] >> (4 * (i & 7))) & 15u;
  } else if constexpr (BITS == 2) {
    return (w[i >> 4] >> (2 * (i & 15))) & 3u;
  } else {
    const uint32_t lo = (w[i >> 4] >> (2 * (i & 15))) & 3u;
    const uint32_t hi = (w[N / 16 + (i >> 5)] >> (i & 31)) & 1u;
    return lo | (hi << 2);
  }
}

// A packed code row into registers. Code rows are read once per decode: non-temporal loads.
template <int NBYTES>
__device__ __forceinline__ void load_row(uint32_t* w, const uint8_t* p) {
  typedef uint32_t v4 __attribute__((ext_vector_type(4)));
  typedef uint32_t v2 __attribute__((ext_vector_type(2)));
  static_assert(NBYTES % 8 == 0, "row bytes");
  if constexpr (NBYTES % 16 == 0) {
#pragma unroll
    for (int k = 0; k < NBYTES / 16; ++k) {
      const v4 v = __builtin_nontemporal_load(reinterpret_cast<const v4*>(p) + k);
      w[4 * k] = v.x; w[4 * k + 1] = v.y; w[4 * k + 2] = v.z; w[4 * k + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < NBYTES / 8; ++k) {
      const v2 v = __builtin_nontemporal_load(reinterpret_cast<const v2*>(p) + k);
      w[2 * k] = v.x; w[2 * k + 1] = v.y;
    }
  }
}

// Token (relative to its half) stored at position p of a value half-row: the 4x4
// grid of 4-token groups is transposed (an involution), so that the 16 tokens a
// matrix-core lane contracts over are adjacent.
__host__ __device__ constexpr int half_row_token(int p) { return 16 * ((p >> 2) & 3) + 4 * (p >> 4) + (p & 3); }

// code of element i (runtime) of a packed row held in registers: selects the word
// without dynamic register indexing (sparse outlier fix-ups only)
template <int BITS, int N>
__device__ __forceinline__ uint32_t code_sel(const uint32_t* w, int i) {
  constexpr int NW = N * BITS / 32;
  if constexpr (BITS == 3) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int k = 0; k < N / 16; ++k) lo = (k == (i >> 4)) ? w[k] : lo;
#pragma unroll
    for (int k = 0; k < N / 32; ++k) hi = (k == (i >> 5)) ? w[N / 16 + k] : hi;
    return ((lo >> (2 * (i & 15))) & 3u) | (((hi >> (i & 31)) & 1u) << 2);
  } else {
    constexpr int PER = 32 / BITS;
    uint32_t x = 0;
#pragma unroll
    for (int k = 0; k < NW; ++k) x = (k == i / PER) ? w[k] : x;
    return (x >> (BITS * (i % PER))) & ((1u << BITS) - 1u);
  }
}

// Per-wave LDS staging used by the sparse outlier fix-ups of one half block.
struct OutlierLds {
  uint8_t* blob;   // the record's outlier segments, from ko_val to the end of vo_idx
  float* kS;       // [128] key scale (S) per channel
  float* kM;       // [128] key offset (M) per channel
  float* vS;       // [64] value scale per token of this half
  float* vM;       // [64]
  float2* rb;      // [64] RoPE base (cos, sin) of the block
};

template <int MODE, int BITS, int G, bool ROPE>
struct Decoder {
  static constexpr int R = 16 * BITS;      // bytes per 128 codes
  static constexpr float kSymOff = (float)(1 << (BITS - 1));   // symmetric codes: u = q + 8 (int8: q + 128)
  static constexpr int RH = R / 2;         // bytes per 64 codes
  static constexpr int NOB = 3;            // prefetched 16-byte chunks of the outlier blob per lane

  // Everything one half block needs, loaded one half block ahead.
  struct Buf {
    uint32_t kw[R / 4];     // key row of token j
    uint32_t vw[R / 4];     // value half-rows of channels 2*lane, 2*lane+1
    float2 ks, km;          // key (S, M) of channels 2*lane, 2*lane+1
    float2 tst;             // value (S, M) of token j; SYM / ASYM: value scales of channels 2*lane, 2*lane+1
    float2 tz;              // ASYM: value zero points of channels 2*lane, 2*lane+1
    float s1t;              // KVarN s1 of token j
    float2 s1c;             // KVarN s1 of channels 2*lane, 2*lane+1
    float2 rb;              // RoPE (cos, sin) of the block base for pair lane
  };

  const DecodeArgs& a;
  const int lane, w, par, j;
  const float* lut;                        // NUQ: [0,16) keys, [16,32) values
  float* pbuf;                             // this wave's probabilities [G][64]
  const float* qs;                         // query, original domain [G][128]
  const float* theta;                      // RoPE theta_i [64] (LDS)
  OutlierLds ol;
  int ob_bytes, ob_chunks;
  float qx[G], qy[G];                      // query pair (2*lane, 2*lane+1), rotated for KVarN
  float m_run[G], l_run[G], pm[G], acc0[G], acc1[G];

  __device__ Decoder(const DecodeArgs& args, int lane_, int w_, const float* lut_, float* pbuf_,
                     const float* qs_, const float* theta_, uint8_t* wlds)
      : a(args), lane(lane_), w(w_), par(w_ & 1), j(64 * (w_ & 1) + lane_), lut(lut_), pbuf(pbuf_),
        qs(qs_), theta(theta_) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      qx[h] = qs[h * 128 + 2 * lane];
      qy[h] = qs[h * 128 + 2 * lane + 1];
      if constexpr (MODE == KVARN) fwht_wave(qx[h], qy[h], lane);
      m_run[h] = -INFINITY; l_run[h] = 0.f; pm[h] = 0.f; acc0[h] = 0.f; acc1[h] = 0.f;
    }
    ob_bytes = 0;
    ob_chunks = 0;
    if (a.k_out > 0) {
      ob_bytes = (int)(a.lay.vo_idx + 128u * a.k_out - a.lay.ko_val);
      ob_chunks = (ob_bytes + 15) / 16;
      const int blob = (ob_bytes + 15) & ~15;
      ol.blob = wlds;
      ol.kS = reinterpret_cast<float*>(wlds + blob);
      ol.kM = ol.kS + 128;
      ol.vS = ol.kM + 128;
      ol.vM = ol.vS + 64;
      ol.rb = reinterpret_cast<float2*>(ol.vM + 64);
    }
  }

  __device__ __forceinline__ const uint8_t* record(int blk) const {
    return a.rec + record_offset(a, blockIdx.z, blockIdx.y, blk);
  }

  __device__ __forceinline__ float kval(uint32_t code) const {
    if constexpr (MODE == NUQ) return lut[code];
    else return (float)code;
  }
  __device__ __forceinline__ float vval(uint32_t code) const {
    if constexpr (MODE == NUQ) return lut[16 + code];
    else return (float)code;
  }

  // Issue every load of one half block (no use of the results here).
  __device__ __forceinline__ void fetch(Buf& B, int blk) const {
    const uint8_t* rec = record(blk);
    load_row<R>(B.kw, rec + a.lay.kc + (size_t)j * R);
    load_row<R>(B.vw, rec + a.lay.vc + (size_t)par * (128 * RH) + (size_t)lane * R);   // rows 2*lane, 2*lane+1
    if constexpr (MODE == SYM) {
      const __half2 k2 = reinterpret_cast<const __half2*>(rec + a.lay.ks)[lane];
      B.ks = __half22float2(k2);
      B.km = make_float2(-kSymOff * B.ks.x, -kSymOff * B.ks.y);
      B.tst = __half22float2(reinterpret_cast<const __half2*>(rec + a.lay.vs)[lane]);
    } else if constexpr (MODE == ASYM) {   // x = (u - 8) s + zero = u s + (zero - 8 s)
      B.ks = __half22float2(reinterpret_cast<const __half2*>(rec + a.lay.ks)[lane]);
      const float2 kz = __half22float2(reinterpret_cast<const __half2*>(rec + a.lay.ks + 256)[lane]);
      B.km = make_float2(fmaf(-kSymOff, B.ks.x, kz.x), fmaf(-kSymOff, B.ks.y, kz.y));
      B.tst = __half22float2(reinterpret_cast<const __half2*>(rec + a.lay.vs)[lane]);
      B.tz = __half22float2(reinterpret_cast<const __half2*>(rec + a.lay.vs + 256)[lane]);
    } else if constexpr (MODE == NUQ) {
      B.km = reinterpret_cast<const float2*>(rec + a.lay.ks)[lane];          // z
      B.ks = reinterpret_cast<const float2*>(rec + a.lay.ks + 512)[lane];    // h
      B.tst.x = reinterpret_cast<const float*>(rec + a.lay.vs)[128 + j];     // h of token j
      B.tst.y = reinterpret_cast<const float*>(rec + a.lay.vs)[j];           // z of token j
    } else {
      B.ks = reinterpret_cast<const float2*>(rec + a.lay.ks)[lane];
      B.km = reinterpret_cast<const float2*>(rec + a.lay.ks + 512)[lane];
      B.tst.x = reinterpret_cast<const float*>(rec + a.lay.vs)[j];
      B.tst.y = reinterpret_cast<const float*>(rec + a.lay.vs)[128 + j];
    }
    if constexpr (MODE == KVARN) {
      B.s1t = reinterpret_cast<const float*>(rec + a.lay.k1)[j];
      B.s1c = reinterpret_cast<const float2*>(rec + a.lay.v1)[lane];
    }
    if constexpr (ROPE) B.rb = reinterpret_cast<const float2*>(a.rope_base)[(size_t)blk * 64 + lane];
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

  __device__ __forceinline__ void wave_sync() const {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // Stage the outlier lists and the statistics the fix-ups read into this wave's LDS.
  // o0..o2: blob chunks lane, lane+64, lane+128 (indices clamped to the blob), loaded
  // at the start of the half block so that their latency hides behind the q.K loop.
  __device__ __forceinline__ void stage_outliers(const Buf& B, const uint8_t* rec, const uint4& o0,
                                                 const uint4& o1, const uint4& o2) {
    if (ob_chunks <= NOB * 64) {
      uint4* dst = reinterpret_cast<uint4*>(ol.blob);
      if (lane < ob_chunks) dst[lane] = o0;
      if (lane + 64 < ob_chunks) dst[lane + 64] = o1;
      if (lane + 128 < ob_chunks) dst[lane + 128] = o2;
    } else {
      const uint4* src = reinterpret_cast<const uint4*>(rec + a.lay.ko_val);
      uint4* dst = reinterpret_cast<uint4*>(ol.blob);
      for (int k = lane; k < ob_chunks; k += 64) dst[k] = src[k];
      // many outliers per vector (rare): end this path with nothing in flight, so that the
      // counter waits after the join stay exact on the common path
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    }
    ol.kS[2 * lane] = B.ks.x; ol.kS[2 * lane + 1] = B.ks.y;
    ol.kM[2 * lane] = B.km.x; ol.kM[2 * lane + 1] = B.km.y;
    if constexpr (MODE != SYM && MODE != ASYM) { ol.vS[lane] = B.tst.x; ol.vM[lane] = B.tst.y; }
    if constexpr (ROPE) ol.rb[lane] = B.rb;
    wave_sync();
  }

  // One 64-token half (parity par) of block blk whose loads are in B.
  __device__ __forceinline__ void process(const Buf& B, int blk, const float (&rc)[64], const float (&rs)[64]) {
    const uint8_t* rec = record(blk);
    const bool outl = MODE != KVARN && a.k_out > 0;
    // issued unconditionally (without outliers from the record's first chunk, read anyway):
    // a load under a branch would make the counter waits after it drain every load in flight
    const uint4* src = reinterpret_cast<const uint4*>(rec + (outl ? a.lay.ko_val : a.lay.kc));
    const int last = outl ? ob_chunks - 1 : 0;
    const uint4 ob0 = src[min(lane, last)], ob1 = src[min(lane + 64, last)], ob2 = src[min(lane + 128, last)];

    // ---- q . K for token j
    float sc[G];
    if constexpr (!ROPE) {
      float QSx[G], QSy[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        QSx[h] = qx[h] * B.ks.x;
        QSy[h] = qy[h] * B.ks.y;
        sc[h] = wave_sum(fmaf(qx[h], B.km.x, qy[h] * B.km.y));   // sum_c q_c * M_c
      }
#pragma unroll
      for (int i0 = 0; i0 < 64; i0 += 8) {
        float vx[8], vy[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          vx[i] = kval(code_at<BITS, 128>(B.kw, 2 * (i0 + i)));
          vy[i] = kval(code_at<BITS, 128>(B.kw, 2 * (i0 + i) + 1));
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int h = 0; h < G; ++h) {
            sc[h] = fmaf(vx[i], readlane_f(QSx[h], i0 + i), sc[h]);
            sc[h] = fmaf(vy[i], readlane_f(QSy[h], i0 + i), sc[h]);
          }
      }
    } else {
      // the query pair rotated back by the block base angle n0*theta_i, folded with the
      // channel statistics: U = P1 vx + P2 vy + P3, W = P4 vx + P5 vy + P6,
      // score += cos(j theta_i) U + sin(j theta_i) W
      float P1[G], P2[G], P3[G], P4[G], P5[G], P6[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float al = fmaf(qx[h], B.rb.x, qy[h] * B.rb.y);
        const float be = fmaf(qy[h], B.rb.x, -qx[h] * B.rb.y);
        P1[h] = al * B.ks.x; P2[h] = be * B.ks.y; P3[h] = fmaf(al, B.km.x, be * B.km.y);
        P4[h] = be * B.ks.x; P5[h] = -al * B.ks.y; P6[h] = fmaf(be, B.km.x, -al * B.km.y);
        sc[h] = 0.f;
      }
#pragma unroll
      for (int i0 = 0; i0 < 64; i0 += 8) {
        float vx[8], vy[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          vx[i] = kval(code_at<BITS, 128>(B.kw, 2 * (i0 + i)));
          vy[i] = kval(code_at<BITS, 128>(B.kw, 2 * (i0 + i) + 1));
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const int ii = i0 + i;
            const float U = fmaf(vx[i], readlane_f(P1[h], ii), fmaf(vy[i], readlane_f(P2[h], ii), readlane_f(P3[h], ii)));
            const float W = fmaf(vx[i], readlane_f(P4[h], ii), fmaf(vy[i], readlane_f(P5[h], ii), readlane_f(P6[h], ii)));
            sc[h] = fmaf(rc[ii], U, fmaf(rs[ii], W, sc[h]));
          }
      }
    }
    if constexpr (MODE != KVARN) {
      if (outl) {
        stage_outliers(B, rec, ob0, ob1, ob2);
        // key outliers of row j (CSR): the fp16 value replaces the dense one
        const uint16_t* ptr = reinterpret_cast<const uint16_t*>(ol.blob + (a.lay.ko_ptr - a.lay.ko_val));
        const uint8_t* idx = ol.blob + (a.lay.ko_idx - a.lay.ko_val);
        const __half* val = reinterpret_cast<const __half*>(ol.blob);
        const int e1 = ptr[j + 1];
        for (int e = ptr[j]; e < e1; ++e) {
          const int c = idx[e];
          const float dense = fmaf(kval(code_sel<BITS, 128>(B.kw, c)), ol.kS[c], ol.kM[c]);
          const float delta = __half2float(val[e]) - dense;
          float cp = 1.f, sp = 0.f;
          if constexpr (ROPE) {
            const int i = c >> 1;
            float sj, cj;
            sincosf((float)j * theta[i], &sj, &cj);
            const float2 b0 = ol.rb[i];
            cp = b0.x * cj - b0.y * sj;
            sp = b0.y * cj + b0.x * sj;
          }
#pragma unroll
          for (int h = 0; h < G; ++h) {
            float coef;
            if constexpr (ROPE) {
              const int i = c >> 1;
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
    const float s1t = MODE == KVARN ? B.s1t : 1.f;
#pragma unroll
    for (int h = 0; h < G; ++h) sl[h] = sc[h] * s1t * a.scale_log2;
    softmax_step(sl, p);

    // ---- P . V over the 64 tokens of this half, channel pair (2*lane, 2*lane+1)
    float pp[G], pmb[G];
    if constexpr (MODE == SYM || MODE == ASYM) {
#pragma unroll
      for (int h = 0; h < G; ++h) { pp[h] = p[h]; pmb[h] = wave_sum(p[h]); }
    } else {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        pp[h] = p[h] * B.tst.x;
        if constexpr (MODE == KVARN) pmb[h] = wave_sum(p[h] * B.tst.y);
        else pm[h] = fmaf(p[h], B.tst.y, pm[h]);
      }
    }
    if (outl) {
#pragma unroll
      for (int h = 0; h < G; ++h) pbuf[h * 64 + lane] = p[h];
    }
    float o0[G], o1[G];
#pragma unroll
    for (int h = 0; h < G; ++h) { o0[h] = 0.f; o1[h] = 0.f; }
#pragma unroll
    for (int t0 = 0; t0 < 64; t0 += 8) {
      float v0[8], v1[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        v0[t] = vval(code_at<BITS, 64>(B.vw, t0 + t));
        v1[t] = vval(code_at<BITS, 64>(B.vw + R / 8, t0 + t));
      }
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float pv = readlane_f(pp[h], half_row_token(t0 + t));
          o0[h] = fmaf(pv, v0[t], o0[h]);
          o1[h] = fmaf(pv, v1[t], o1[h]);
        }
    }
    if constexpr (MODE == KVARN) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        acc0[h] = fmaf(B.s1c.x, o0[h] + pmb[h], acc0[h]);
        acc1[h] = fmaf(B.s1c.y, o1[h] + pmb[h], acc1[h]);
      }
    } else if constexpr (MODE == SYM) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        acc0[h] = fmaf(B.tst.x, fmaf(-kSymOff, pmb[h], o0[h]), acc0[h]);
        acc1[h] = fmaf(B.tst.y, fmaf(-kSymOff, pmb[h], o1[h]), acc1[h]);
      }
    } else if constexpr (MODE == ASYM) {   // s_c (sum p (u - 8)) + zero_c sum p
#pragma unroll
      for (int h = 0; h < G; ++h) {
        acc0[h] = fmaf(B.tz.x, pmb[h], fmaf(B.tst.x, fmaf(-kSymOff, pmb[h], o0[h]), acc0[h]));
        acc1[h] = fmaf(B.tz.y, pmb[h], fmaf(B.tst.y, fmaf(-kSymOff, pmb[h], o1[h]), acc1[h]));
      }
    } else {
#pragma unroll
      for (int h = 0; h < G; ++h) { acc0[h] += o0[h]; acc1[h] += o1[h]; }
    }
    if constexpr (MODE != KVARN) {
      if (outl) {
        // value outliers of channels 2*lane, 2*lane+1 (CSC) that fall in this half
        wave_sync();
        const uint16_t* ptr = reinterpret_cast<const uint16_t*>(ol.blob + (a.lay.vo_ptr - a.lay.ko_val));
        const uint8_t* idx = ol.blob + (a.lay.vo_idx - a.lay.ko_val);
        const __half* val = reinterpret_cast<const __half*>(ol.blob + (a.lay.vo_val - a.lay.ko_val));
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int c = 2 * lane + k;
          const int e1 = ptr[c + 1];
          for (int e = ptr[c]; e < e1; ++e) {
            const int t = idx[e] - 64 * par;
            if (t < 0 || t >= 64) continue;
            const uint32_t code = code_sel<BITS, 64>(B.vw + k * (R / 8), half_row_token(t));
            float dense;
            if constexpr (MODE == SYM) dense = ((float)code - kSymOff) * (k ? B.tst.y : B.tst.x);
            else if constexpr (MODE == ASYM)
              dense = fmaf((float)code - kSymOff, k ? B.tst.y : B.tst.x, k ? B.tz.y : B.tz.x);
            else dense = fmaf(vval(code), ol.vS[t], ol.vM[t]);
            const float delta = __half2float(val[e]) - dense;
#pragma unroll
            for (int h = 0; h < G; ++h) {
              if (k == 0) acc0[h] = fmaf(pbuf[h * 64 + t], delta, acc0[h]);
              else acc1[h] = fmaf(pbuf[h * 64 + t], delta, acc1[h]);
            }
          }
        }
        wave_sync();
      }
    }
  }

  // Tokens 64*par .. 64*par+63 of the fp16 tail (n_valid of them), position 128*nblk + j.
  __device__ __forceinline__ void tail_half(const float (&rc)[64], const float (&rs)[64]) {
    const int n_valid = min(64, seq_tail(a, blockIdx.z) - 64 * par);
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
#pragma unroll
      for (int i = 0; i < 64; ++i) {
        const float2 kk = valid ? __half22float2(krow[i]) : make_float2(0.f, 0.f);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          sc[h] = fmaf(kk.x, readlane_f(ox[h], i), sc[h]);
          sc[h] = fmaf(kk.y, readlane_f(oy[h], i), sc[h]);
        }
      }
    } else {
      const float2 cs0 = reinterpret_cast<const float2*>(a.rope_base)[(size_t)seq_nblk(a, blockIdx.z) * 64 + lane];
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

  // All half blocks of this wave, one half block of loads in flight ahead of the math. The
  // next block is fetched unconditionally (past the split's end: its last block again), so
  // that the wait before a block covers its own loads only: a load under a branch makes the
  // counter wait at the join drain every load in flight, the prefetch included.
  __device__ __forceinline__ void run(int blo, int bhi, const float (&rc)[64], const float (&rs)[64]) {
    Buf A, Bb;
    int blk = blo + (w >> 1);
    if (blk >= bhi) return;
    const int last = bhi - 1;
    fetch(A, blk);
    while (true) {
      fetch(Bb, min(blk + 2, last));
      process(A, blk, rc, rs);
      blk += 2;
      if (blk >= bhi) break;
      fetch(A, min(blk + 2, last));
      process(Bb, blk, rc, rs);
      blk += 2;
      if (blk >= bhi) break;
    }
  }
};

}  // namespace dec
}  // namespace kvq
