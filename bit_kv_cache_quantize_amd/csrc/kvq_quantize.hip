// Quantize-on-append: one workgroup turns one completed 128-token block of one
// (sequence, kv head) into its packed record.
//
// Steps per tensor (keys, then values), following the pages:
//   - stage the 128 x 128 fp16 block (fp16 tail rows + new rows) in LDS as fp32;
//   - KVarN only: 128-point Hadamard rotation of every token across channels and
//     Sinkhorn-style variance normalisation in the log-std domain, giving s1
//     ("KVarN" summary, core method and method steps);
//   - per vector (a key channel over the block's tokens, a value token over its
//     channels; symmetric int4 groups values per channel too): top-k |x| outliers
//     kept in fp16 ("KVQuant reading notes" 3.4), min/max over the rest, then
//     RTN (notes 1.2, 3.1), codebook argmin (notes 1.2, 3.3) or symmetric int4
//     with an fp16 scale ("reproducing TurboQuant" 4.2);
//   - pack codes (key rows token-major, value rows channel-major in two token
//     halves, each half-row in a 4x4-group transposed token order), write
//     statistics, s1 and the CSR / CSC outlier lists.
// Every quantization decision uses IEEE fp32 operations written out with
// explicit rounding intrinsics (no contraction), rintf (round half even) and
// fp16 round-to-nearest-even, so that codes and scales are reproducible.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kPitch = 129;          // LDS row pitch of the fp32 tile (bank spread)
constexpr int kThreads = 256;

struct QuantSmem {
  float x[kT * kPitch];              // element (t, c) at x[t * kPitch + c]
  uint8_t q[kT * kD];                // code of (t, c) at q[t * kD + c]
  uint8_t olist[kD * kMaxOut];       // outlier element indices per vector
  float ra[kT], cb[kD];              // VarN: exp(-r_t), exp(-c_ch)
  float rl[kT], cl[kD];              // VarN: log scales
  int cnt[kT + 1];
  float lut[16];
};

__device__ __forceinline__ int xidx(int va, int v, int e) {
  // va == 0: vector = channel v, element = token e; va == 1: vector = token v, element = channel e
  return va == 0 ? e * kPitch + v : v * kPitch + e;
}

__device__ __forceinline__ uint64_t mag_key(float x, int e) {
  // larger key = larger |x|, then smaller element index
  return ((uint64_t)(__float_as_uint(x) & 0x7fffffffu) << 8) | (uint64_t)(255 - e);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = __shfl_xor((uint32_t)v, m), hi = __shfl_xor((uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}

// Pack dword w of a row of n codes, code i given by get(i).
template <int BITS, typename Get>
__device__ __forceinline__ uint32_t pack_dword(int n, int w, Get get) {
  uint32_t r = 0;
  if constexpr (BITS == 4) {
#pragma unroll
    for (int i = 0; i < 8; ++i) r |= (uint32_t)get(8 * w + i) << (4 * i);
  } else if constexpr (BITS == 2) {
#pragma unroll
    for (int i = 0; i < 16; ++i) r |= (uint32_t)get(16 * w + i) << (2 * i);
  } else {
    const int ncrumb = n / 16;       // dwords of the 2-bit plane
    if (w < ncrumb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) r |= (uint32_t)(get(16 * w + i) & 3) << (2 * i);
    } else {
      const int wb = w - ncrumb;
#pragma unroll
      for (int i = 0; i < 32; ++i) r |= (uint32_t)((get(32 * wb + i) >> 2) & 1) << i;
    }
  }
  return r;
}

// Rotate every token row of the tile by the orthonormal Sylvester Hadamard matrix.
__device__ void fwht_rows(QuantSmem& sm, int tid) {
  for (int s = 0; s < 7; ++s) {
    const int hs = 1 << s;
    for (int id = tid; id < kT * 64; id += kThreads) {
      const int t = id >> 6, k = id & 63;
      const int i = ((k >> s) << (s + 1)) | (k & (hs - 1));
      float* row = sm.x + t * kPitch;
      const float a = row[i], b = row[i + hs];
      row[i] = __fadd_rn(a, b);
      row[i + hs] = __fsub_rn(a, b);
    }
    __syncthreads();
  }
  const float inv = 0.08838834764831845f;   // 1 / sqrt(128)
  for (int id = tid; id < kT * kD; id += kThreads) {
    float& x = sm.x[(id >> 7) * kPitch + (id & 127)];
    x = __fmul_rn(x, inv);
  }
  __syncthreads();
}

// Population std over 128 elements of the scaled tile, two threads per vector.
// va == 0: per channel v over tokens; va == 1: per token v over channels.
__device__ float varn_std(const QuantSmem& sm, int va, int v, int hf) {
  float sum = 0.f;
  for (int i = 0; i < 64; ++i) {
    const int e = hf * 64 + i;
    const int t = va == 0 ? e : v, c = va == 0 ? v : e;
    sum = __fadd_rn(sum, __fmul_rn(__fmul_rn(sm.x[t * kPitch + c], sm.ra[t]), sm.cb[c]));
  }
  sum = __fadd_rn(sum, __shfl_xor(sum, 1));
  const float mean = __fdiv_rn(sum, 128.f);
  float ss = 0.f;
  for (int i = 0; i < 64; ++i) {
    const int e = hf * 64 + i;
    const int t = va == 0 ? e : v, c = va == 0 ? v : e;
    const float d = __fsub_rn(__fmul_rn(__fmul_rn(sm.x[t * kPitch + c], sm.ra[t]), sm.cb[c]), mean);
    ss = __fadd_rn(ss, __fmul_rn(d, d));
  }
  ss = __fadd_rn(ss, __shfl_xor(ss, 1));
  return __fsqrt_rn(__fdiv_rn(ss, 128.f));
}

// Variance normalisation (channel step, then token step, per iteration) in the
// log-std domain; leaves rl (per token) and cl (per channel) log scales in LDS.
__device__ void varn(QuantSmem& sm, int tid, int iters) {
  if (tid < 128) { sm.rl[tid] = 0.f; sm.cl[tid] = 0.f; }
  __syncthreads();
  const int v = tid >> 1, hf = tid & 1;
  for (int it = 0; it < iters; ++it) {
    if (tid < 128) { sm.ra[tid] = expf(-sm.rl[tid]); sm.cb[tid] = expf(-sm.cl[tid]); }
    __syncthreads();
    float sd = varn_std(sm, 0, v, hf);
    __syncthreads();
    if (hf == 0 && sd > 0.f) sm.cl[v] = __fadd_rn(sm.cl[v], logf(sd));
    __syncthreads();
    if (tid < 128) sm.cb[tid] = expf(-sm.cl[tid]);
    __syncthreads();
    sd = varn_std(sm, 1, v, hf);
    __syncthreads();
    if (hf == 0 && sd > 0.f) sm.rl[v] = __fadd_rn(sm.rl[v], logf(sd));
    __syncthreads();
  }
}

template <int MODE, int BITS>
__global__ __launch_bounds__(kThreads) void quantize_kernel(QuantArgs a) {
  __shared__ QuantSmem sm;
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const size_t unit = (size_t)b * a.Hkv + h;
  uint8_t* rec = a.rec + (unit * a.max_blocks + (size_t)(a.blk0 + j)) * a.lay.rec_bytes;
  constexpr int R = 16 * BITS;                 // bytes per 128 codes
  constexpr int QMAX = (1 << BITS) - 1;
  const int k_out = a.k_out;

  for (int tensor = 0; tensor < 2; ++tensor) {
    const __half* in = (tensor ? a.v_in : a.k_in) + unit * (size_t)a.n_new * kD;
    const __half* tl = a.tail + unit * (2 * kT * kD) + (size_t)tensor * kT * kD;
    // --- stage the block: rows < t0 of block 0 come from the fp16 tail
    for (int id = tid; id < kT * 16; id += kThreads) {
      const int row = id >> 4, ch = (id & 15) * 8;
      const __half* src = (j == 0 && row < a.t0) ? tl + row * kD + ch
                                                 : in + (size_t)(j * kT + row - a.t0) * kD + ch;
      const uint4 w = *reinterpret_cast<const uint4*>(src);
      const __half* hv = reinterpret_cast<const __half*>(&w);
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.x[row * kPitch + ch + e] = __half2float(hv[e]);
    }
    if (tid < 16 && MODE == NUQ) sm.lut[tid] = a.cb[(h * 2 + tensor) * 16 + tid];
    __syncthreads();

    // vector axis: keys per channel; values per token, except symmetric int4
    const int va = (tensor == 0 || MODE == SYM) ? 0 : 1;

    if constexpr (MODE == KVARN) {
      fwht_rows(sm, tid);
      varn(sm, tid, a.varn_iters);
      // s1: keys per token, values per channel; divide the tile by it
      if (tid < 128) {
        const float s1 = expf(tensor == 0 ? sm.rl[tid] : sm.cl[tid]);
        sm.ra[tid] = s1;
        float* dst = reinterpret_cast<float*>(rec + (tensor == 0 ? a.lay.k1 : a.lay.v1));
        dst[tid] = s1;
      }
      __syncthreads();
      for (int id = tid; id < kT * kD; id += kThreads) {
        const int t = id >> 7, c = id & 127;
        float& x = sm.x[t * kPitch + c];
        x = __fdiv_rn(x, sm.ra[tensor == 0 ? t : c]);
      }
      __syncthreads();
    }

    // --- per vector: outliers, statistics, codes (two threads per vector)
    const int v = tid >> 1, hf = tid & 1;
    uint64_t thr = ~0ull;
    if (MODE != KVARN && k_out > 0) {
      uint64_t prev = ~0ull;
      for (int p = 0; p < k_out; ++p) {
        uint64_t best = 0;
        for (int i = 0; i < 64; ++i) {
          const int e = hf * 64 + i;
          const uint64_t key = mag_key(sm.x[xidx(va, v, e)], e);
          if (key < prev && key > best) best = key;
        }
        const uint64_t o = shfl_xor_u64(best, 1);
        best = o > best ? o : best;
        if (hf == 0) sm.olist[v * kMaxOut + p] = (uint8_t)(255 - (int)(best & 255));
        prev = best;
      }
      thr = prev;
    }
    float lo = INFINITY, hi = -INFINITY, amax = 0.f;
    for (int i = 0; i < 64; ++i) {
      const int e = hf * 64 + i;
      const float x = sm.x[xidx(va, v, e)];
      const bool outl = (MODE != KVARN && k_out > 0) && mag_key(x, e) >= thr;
      if (!outl) { lo = fminf(lo, x); hi = fmaxf(hi, x); amax = fmaxf(amax, fabsf(x)); }
    }
    lo = fminf(lo, __shfl_xor(lo, 1));
    hi = fmaxf(hi, __shfl_xor(hi, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 1));

    float sa, sb;           // RTN/KVARN: s, m; NUQ: z, h; SYM: s (fp16-rounded), unused
    if constexpr (MODE == NUQ) {
      sa = __fmul_rn(__fadd_rn(hi, lo), 0.5f);
      sb = __fmul_rn(__fsub_rn(hi, lo), 0.5f);
    } else if constexpr (MODE == SYM) {
      sa = __half2float(__float2half_rn(__fdiv_rn(amax, 7.0f)));
      sb = 0.f;
    } else {
      sa = __fdiv_rn(__fsub_rn(hi, lo), (float)QMAX);
      sb = lo;
    }
    for (int i = 0; i < 64; ++i) {
      const int e = hf * 64 + i;
      const float x = sm.x[xidx(va, v, e)];
      int code;
      if constexpr (MODE == NUQ) {
        float u = sb == 0.f ? 0.f : __fdiv_rn(__fsub_rn(x, sa), sb);
        u = fminf(fmaxf(u, -1.f), 1.f);
        float best = INFINITY;
        code = 0;
#pragma unroll
        for (int c = 0; c <= QMAX; ++c) {
          const float d = fabsf(__fsub_rn(u, sm.lut[c]));
          if (d < best) { best = d; code = c; }
        }
      } else if constexpr (MODE == SYM) {
        const float r = sa == 0.f ? 0.f : rintf(__fdiv_rn(x, sa));
        code = (int)fminf(fmaxf(r, -8.f), 7.f) + 8;
      } else {
        const float r = sa == 0.f ? 0.f : rintf(__fdiv_rn(__fsub_rn(x, sb), sa));
        code = (int)fminf(fmaxf(r, 0.f), (float)QMAX);
      }
      const int t = va == 0 ? e : v, c = va == 0 ? v : e;
      sm.q[t * kD + c] = (uint8_t)code;
    }
    // statistics of vector v
    if (hf == 0) {
      uint8_t* st = rec + (tensor == 0 ? a.lay.ks : a.lay.vs);
      if constexpr (MODE == SYM) {
        reinterpret_cast<__half*>(st)[v] = __float2half_rn(sa);
      } else if constexpr (MODE == NUQ) {
        reinterpret_cast<float*>(st)[v] = sa;          // z
        reinterpret_cast<float*>(st)[128 + v] = sb;    // h
      } else {
        reinterpret_cast<float*>(st)[v] = sa;          // s
        reinterpret_cast<float*>(st)[128 + v] = sb;    // m
      }
    }
    __syncthreads();

    // --- pack codes
    if (tensor == 0) {
      // key rows, token-major: row t = channels 0..127
      constexpr int DW = R / 4;
      uint32_t* dst = reinterpret_cast<uint32_t*>(rec + a.lay.kc);
      for (int id = tid; id < kT * DW; id += kThreads) {
        const int t = id / DW, w = id % DW;
        dst[id] = pack_dword<BITS>(128, w, [&](int i) { return sm.q[t * kD + i]; });
      }
    } else {
      // value rows, channel-major in two token halves: row (half, c) = tokens 64*half + i
      constexpr int DW = R / 8;
      uint32_t* dst = reinterpret_cast<uint32_t*>(rec + a.lay.vc);
      for (int id = tid; id < 2 * kD * DW; id += kThreads) {
        const int row = id / DW, w = id % DW;
        const int half = row >> 7, c = row & 127;
        // position i of a half-row holds token 16*((i>>2)&3) + 4*(i>>4) + (i&3) of the half
        dst[id] = pack_dword<BITS>(64, w, [&](int i) {
          return sm.q[(64 * half + 16 * ((i >> 2) & 3) + 4 * (i >> 4) + (i & 3)) * kD + c];
        });
      }
    }

    // --- outliers: keys CSR by token, values CSC by channel, sorted by (row, column)
    if (MODE != KVARN && k_out > 0) {
      // storage row r and column u: keys (r = token, u = channel), values (r = channel, u = token)
      auto member = [&](int r, int u) -> bool {
        const int t = tensor == 0 ? r : u, c = tensor == 0 ? u : r;
        const int vv = va == 0 ? c : t, ee = va == 0 ? t : c;
        for (int p = 0; p < k_out; ++p)
          if (sm.olist[vv * kMaxOut + p] == ee) return true;
        return false;
      };
      if (tid < 128) {
        int n = 0;
        for (int u = 0; u < 128; ++u) n += member(tid, u) ? 1 : 0;
        sm.cnt[tid + 1] = n;
      }
      __syncthreads();
      if (tid == 0) {
        sm.cnt[0] = 0;
        for (int r = 0; r < 128; ++r) sm.cnt[r + 1] += sm.cnt[r];
      }
      __syncthreads();
      uint8_t* base = rec;
      __half* val = reinterpret_cast<__half*>(base + (tensor == 0 ? a.lay.ko_val : a.lay.vo_val));
      uint16_t* ptr = reinterpret_cast<uint16_t*>(base + (tensor == 0 ? a.lay.ko_ptr : a.lay.vo_ptr));
      uint8_t* idx = base + (tensor == 0 ? a.lay.ko_idx : a.lay.vo_idx);
      if (tid <= 128) ptr[tid] = (uint16_t)sm.cnt[tid];
      if (tid < 128) {
        int pos = sm.cnt[tid];
        for (int u = 0; u < 128; ++u) {
          if (member(tid, u)) {
            const int t = tensor == 0 ? tid : u, c = tensor == 0 ? u : tid;
            val[pos] = __float2half_rn(sm.x[t * kPitch + c]);   // exact: the tile holds widened fp16
            idx[pos] = (uint8_t)u;
            ++pos;
          }
        }
      }
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kThreads) void tail_kernel(TailArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  const size_t unit = (size_t)b * a.Hkv + h;
  for (int tensor = 0; tensor < 2; ++tensor) {
    const __half* in = (tensor ? a.v_in : a.k_in) + unit * (size_t)a.n_new * kD;
    __half* tl = a.tail + unit * (2 * kT * kD) + (size_t)tensor * kT * kD;
    for (int id = threadIdx.x; id < a.count * 16; id += kThreads) {
      const int row = id >> 4, ch = (id & 15) * 8;
      *reinterpret_cast<uint4*>(tl + (size_t)(a.dst0 + row) * kD + ch) =
          *reinterpret_cast<const uint4*>(in + (size_t)(a.src0 + row) * kD + ch);
    }
  }
}

template <int MODE, int BITS>
hipError_t launch_q(const QuantArgs& a, int n_blocks, int batch, hipStream_t s) {
  hipLaunchKernelGGL((quantize_kernel<MODE, BITS>), dim3(n_blocks, a.Hkv, batch), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(int mode, int bits, const QuantArgs& a, int n_blocks, int batch,
                           hipStream_t s) {
  switch (mode * 8 + bits) {
    case RTN * 8 + 2: return launch_q<RTN, 2>(a, n_blocks, batch, s);
    case RTN * 8 + 3: return launch_q<RTN, 3>(a, n_blocks, batch, s);
    case RTN * 8 + 4: return launch_q<RTN, 4>(a, n_blocks, batch, s);
    case NUQ * 8 + 2: return launch_q<NUQ, 2>(a, n_blocks, batch, s);
    case NUQ * 8 + 3: return launch_q<NUQ, 3>(a, n_blocks, batch, s);
    case NUQ * 8 + 4: return launch_q<NUQ, 4>(a, n_blocks, batch, s);
    case KVARN * 8 + 2: return launch_q<KVARN, 2>(a, n_blocks, batch, s);
    case KVARN * 8 + 3: return launch_q<KVARN, 3>(a, n_blocks, batch, s);
    case KVARN * 8 + 4: return launch_q<KVARN, 4>(a, n_blocks, batch, s);
    case SYM * 8 + 4: return launch_q<SYM, 4>(a, n_blocks, batch, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_tail(const TailArgs& a, int batch, hipStream_t s) {
  hipLaunchKernelGGL(tail_kernel, dim3(a.Hkv, batch), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvq
