// Quantization-error diagnostic ("KVarN" summary, core method): per cached token, the error
// of its key and value vectors split into a norm part E_M = (||x|| - ||x_hat||)^2 and a
// direction part E_D = 2 ||x|| ||x_hat|| (1 - cos angle), E_M + E_D = ||x - x_hat||^2. x is
// the caller's original fp16 vector, x_hat the cache's own record dequantized in fp64 in the
// original domain: RTN q s + m, NUQ C[q] h + z, symmetric int4 (q - 8) s, outlier positions
// replaced by their fp16 values, KVarN (q s + m) s1 rotated back by the orthonormal Hadamard
// transform.
//
// One workgroup of 512 threads per (block, sequence, kv head); the record is staged in LDS.
// Thread (t, qd) holds channels 32 qd .. 32 qd + 31 of token t in registers; the four
// threads of a token (lanes 4t .. 4t + 3 of a wave) exchange values for the last two
// Hadamard stages and add their per-token sums. The
// dense values are dequantized everywhere; each outlier entry then corrects the sums by the
// difference between its fp16 value and the dense value stored at its position.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kDiagThreads = 512;
constexpr int kQ = 4;                  // threads per token
constexpr int kC = kD / kQ;            // channels per thread

template <int MODE, int BITS>
struct DiagBlock {
  static constexpr int R = 16 * BITS;   // bytes per 128 codes
  const DiagArgs& a;
  const uint8_t* rec;                   // the record in LDS
  const float* cb;                      // codebooks of this kv head (NUQ): keys then values

  // Code of token t, channel c: keys token-major, values channel-major in two token halves
  // with the 4x4 grid of 4-token groups transposed within a half-row (include/kvq.h).
  __device__ __forceinline__ uint32_t code_at(int tensor, int t, int c) const {
    const uint8_t* row;
    int p;   // position of the code in its row
    if (tensor == 0) {
      row = rec + a.lay.kc + t * R;
      p = c;
    } else {
      const int u = t & 63;
      row = rec + a.lay.vc + ((t >> 6) * 128 + c) * (R / 2);
      p = 16 * ((u >> 2) & 3) + 4 * (u >> 4) + (u & 3);
    }
    const int n = tensor == 0 ? 128 : 64;   // codes in the row
    if constexpr (BITS == 8) return row[p];
    if constexpr (BITS == 4) return (row[p >> 1] >> (4 * (p & 1))) & 15u;
    if constexpr (BITS == 2) return (row[p >> 2] >> (2 * (p & 3))) & 3u;
    const uint32_t lo = (row[p >> 2] >> (2 * (p & 3))) & 3u;
    const uint32_t hi = (row[n / 4 + (p >> 3)] >> (p & 7)) & 1u;
    return lo | (hi << 2);
  }

  __device__ __forceinline__ float f32_at(uint32_t off) const { return *reinterpret_cast<const float*>(rec + off); }

  // Dense dequantized value (fp64) of token t, channel c; KVarN: in the rotated domain.
  __device__ __forceinline__ double dequant(int tensor, int t, int c, uint32_t q) const {
    const uint32_t st = tensor == 0 ? a.lay.ks : a.lay.vs;
    const int vi = tensor == 0 ? c : t;   // statistics index: key channel, value token
    if constexpr (MODE == SYM) {
      const __half s = reinterpret_cast<const __half*>(rec + st)[c];   // per channel for both
      return ((double)q - (double)(1 << (BITS - 1))) * (double)__half2float(s);
    } else if constexpr (MODE == ASYM) {   // per channel for both: (u - 8) s + zero
      const __half s = reinterpret_cast<const __half*>(rec + st)[c];
      const __half z = reinterpret_cast<const __half*>(rec + st + 256)[c];
      return ((double)q - 8.0) * (double)__half2float(s) + (double)__half2float(z);
    } else if constexpr (MODE == NUQ) {
      const double z = f32_at(st + 4 * vi), h = f32_at(st + 512 + 4 * vi);
      return (double)cb[tensor * kCbStride + q] * h + z;
    } else {
      const double s = f32_at(st + 4 * vi), m = f32_at(st + 512 + 4 * vi);
      double x = (double)q * s + m;
      if constexpr (MODE == KVARN)
        x *= tensor == 0 ? (double)f32_at(a.lay.k1 + 4 * t) : (double)f32_at(a.lay.v1 + 4 * c);
      return x;
    }
  }
};

template <int MODE, int BITS>
__global__ __launch_bounds__(kDiagThreads) void diag_kernel(DiagArgs a) {
  extern __shared__ __align__(16) uint8_t s_rec[];
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, t = tid >> 2, qd = tid & 3;
  const size_t unit = (size_t)b * a.Hkv + h;
  const uint8_t* rec = a.rec + (unit * a.max_blocks + (size_t)(a.block0 + j)) * a.lay.rec_bytes;
  for (uint32_t i = tid; i < a.lay.rec_bytes / 16; i += kDiagThreads)
    reinterpret_cast<uint4*>(s_rec)[i] = reinterpret_cast<const uint4*>(rec)[i];
  __syncthreads();
  const DiagBlock<MODE, BITS> D{a, s_rec, a.cb + (size_t)h * 2 * kCbStride};
  const size_t row = unit * (size_t)a.n_blocks * kT + (size_t)j * kT + t;   // token row of the inputs
  for (int tensor = 0; tensor < 2; ++tensor) {
    double xh[kC];
#pragma unroll
    for (int e = 0; e < kC; ++e) {
      const int c = kC * qd + e;
      xh[e] = D.dequant(tensor, t, c, D.code_at(tensor, t, c));
    }
    if constexpr (MODE == KVARN) {
      // back to the original domain: y = H x / sqrt(128) over the token's 128 channels
      // (natural-order butterflies: channel bits 0..4 within the thread, 5..6 across the
      // token's threads)
#pragma unroll
      for (int hs = 1; hs < kC; hs <<= 1)
#pragma unroll
        for (int e = 0; e < kC; ++e)
          if (!(e & hs)) {
            const double p = xh[e], q = xh[e | hs];
            xh[e] = p + q;
            xh[e | hs] = p - q;
          }
#pragma unroll
      for (int m = 1; m < kQ; m <<= 1) {
        const bool upper = (qd & m) != 0;
#pragma unroll
        for (int e = 0; e < kC; ++e) {
          const double p = __shfl_xor(xh[e], m);
          xh[e] = upper ? p - xh[e] : xh[e] + p;
        }
      }
#pragma unroll
      for (int e = 0; e < kC; ++e) xh[e] *= 0.08838834764831845;   // 1 / sqrt(128)
    }
    const __half* x = (tensor ? a.v_in : a.k_in) + row * kD + kC * qd;
    double nx = 0.0, nh = 0.0, dot = 0.0;
#pragma unroll
    for (int e = 0; e < kC; e += 8) {
      const uint4 raw = *reinterpret_cast<const uint4*>(x + e);
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float2 f = __half22float2(__builtin_bit_cast(__half2, w[k]));
        const double x0 = f.x, x1 = f.y, h0 = xh[e + 2 * k], h1 = xh[e + 2 * k + 1];
        nx += x0 * x0 + x1 * x1;
        nh += h0 * h0 + h1 * h1;
        dot += x0 * h0 + x1 * h1;
      }
    }
    if constexpr (MODE != KVARN) {
      if (a.k_out > 0) {
        // outlier entries of this token in this half: replace the dense value in the sums
        const uint8_t* base = s_rec;
        auto fix = [&](int c, const __half v) {
          const double dense = D.dequant(tensor, t, c, D.code_at(tensor, t, c));
          const double o = (double)__half2float(v), xc = (double)__half2float(x[c - kC * qd]);
          nh += o * o - dense * dense;
          dot += xc * (o - dense);
        };
        if (tensor == 0) {   // keys: CSR by token
          const uint16_t* ptr = reinterpret_cast<const uint16_t*>(base + a.lay.ko_ptr);
          const uint8_t* idx = base + a.lay.ko_idx;
          const __half* val = reinterpret_cast<const __half*>(base + a.lay.ko_val);
          for (int e = ptr[t]; e < ptr[t + 1]; ++e)
            if (idx[e] / kC == qd) fix(idx[e], val[e]);
        } else {             // values: CSC by channel
          const uint16_t* ptr = reinterpret_cast<const uint16_t*>(base + a.lay.vo_ptr);
          const uint8_t* idx = base + a.lay.vo_idx;
          const __half* val = reinterpret_cast<const __half*>(base + a.lay.vo_val);
          for (int c = kC * qd; c < kC * qd + kC; ++c)
            for (int e = ptr[c]; e < ptr[c + 1]; ++e)
              if (idx[e] == t) fix(c, val[e]);
        }
      }
    }
#pragma unroll
    for (int m = 1; m < kQ; m <<= 1) {
      nx += __shfl_xor(nx, m);
      nh += __shfl_xor(nh, m);
      dot += __shfl_xor(dot, m);
    }
    if (qd == 0) {
      const double a_ = sqrt(nx), b_ = sqrt(nh);
      double* o = a.out + row * 4 + 2 * tensor;
      o[0] = (a_ - b_) * (a_ - b_);
      o[1] = 2.0 * (a_ * b_ - dot);
    }
  }
}

template <int MODE, int BITS>
hipError_t launch_d(const DiagArgs& a, int batch, hipStream_t s) {
  hipLaunchKernelGGL((diag_kernel<MODE, BITS>), dim3(a.n_blocks, a.Hkv, batch), dim3(kDiagThreads),
                     (size_t)a.lay.rec_bytes, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_diag(int mode, int bits, const DiagArgs& a, int batch, hipStream_t s) {
  switch (mode * 8 + bits) {
    case RTN * 8 + 2: return launch_d<RTN, 2>(a, batch, s);
    case RTN * 8 + 3: return launch_d<RTN, 3>(a, batch, s);
    case RTN * 8 + 4: return launch_d<RTN, 4>(a, batch, s);
    case RTN * 8 + 8: return launch_d<RTN, 8>(a, batch, s);
    case NUQ * 8 + 2: return launch_d<NUQ, 2>(a, batch, s);
    case NUQ * 8 + 3: return launch_d<NUQ, 3>(a, batch, s);
    case NUQ * 8 + 4: return launch_d<NUQ, 4>(a, batch, s);
    case KVARN * 8 + 2: return launch_d<KVARN, 2>(a, batch, s);
    case KVARN * 8 + 3: return launch_d<KVARN, 3>(a, batch, s);
    case KVARN * 8 + 4: return launch_d<KVARN, 4>(a, batch, s);
    case KVARN * 8 + 8: return launch_d<KVARN, 8>(a, batch, s);
    case SYM * 8 + 4: return launch_d<SYM, 4>(a, batch, s);
    case SYM * 8 + 8: return launch_d<SYM, 8>(a, batch, s);
    case ASYM * 8 + 4: return launch_d<ASYM, 4>(a, batch, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
