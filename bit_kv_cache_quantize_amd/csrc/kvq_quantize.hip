// Quantize-on-append: one workgroup turns one tensor (the keys or the values) of
// one completed 128-token block of one (sequence, kv head) into its part of the
// packed record.
//
// Steps per tensor, following the pages:
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
// Every quantization decision uses IEEE fp32 operations (no contraction:
// the library is built with -ffp-contract=off and correctly rounded division),
// rintf (round half even) and fp16 round-to-nearest-even, so that codes and
// scales are reproducible. The one exception is KVarN's variance normalisation
// (hardware exp2 / log2), whose scales are specified to a relative tolerance.
//
// The 128 x 128 tile stays in registers: wave w holds tokens 32w .. 32w+31 and
// lane (r = lane >> 4, g = lane & 15) holds tokens t_i = 32w + 4i + r (i = 0..7)
// at channels 8g .. 8g+7, as fp16 pairs widened on use (KVarN: fp32). Each 16-byte
// load covers 8 channels of one token, so a wave reads four consecutive 256-byte
// rows per instruction.
//   per-channel reductions: the lane's 8 tokens, the four r lanes (xor 16, 32),
//     then the four waves through LDS (all threads combine the four partials in
//     the same order, so every holder of a channel gets the same value);
//   per-token reductions: the lane's 8 channels, then the 16 g lanes (xor 1..8).
// The kernel is bound by vector-ALU issue: cross-lane moves use the LDS permute
// unit unless a row move fuses into its use, and a vector's statistics (their
// divisions) are derived once, in an owner lane, and permuted to the others.
// Key codes are packed straight from registers (a lane holds 8 consecutive
// channels of a token row); value codes go through an LDS tile for the
// channel-major layout. Outlier lists are built with a per-row bitmask in LDS:
// the row pointer is a prefix sum of row popcounts and an entry's slot is the
// row pointer plus the popcount of the bits below its column.
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
constexpr float kInvSqrt128 = 0.08838834764831845f;

struct Smem {
  uint8_t vq[kT * kD];            // value codes, (t, c) at t * 128 + c
  uint32_t red[2][4][kD];         // per-channel cross-wave partials, two alternating buffers
  float rlo[4][kD], rhi[4][kD];   // per-channel min / max partials
  uint32_t omask[kD][4];          // outlier bitmask per storage row
  uint32_t okey[kD][kMaxOut];     // selection keys of each vector's outliers
  uint16_t optr[kD + 1];          // storage row pointers
  float2 nlut[kNuqLutStride];     // NUQ code table of this (kv head, tensor)
};

// Key of the top-k |x| selection: larger magnitude first, then lower element index e
// (magnitude bits from bit 8 up, 127 - e in bits 1..7, the sign in bit 0, which never
// decides since (magnitude, index) is unique); a key gives back its element's position
// within the vector and, for fp16 tiles, the element's exact fp16 bits.
__device__ __forceinline__ uint32_t mag_key(float x, int e) {
  // fp32 form (KVarN tiles, which never select outliers): magnitude bits above bit 13
  const uint32_t u = __float_as_uint(x);
  return (((u & 0x7fffffffu) >> 13) << 8) | ((uint32_t)(127 - e) << 1) | (u >> 31);
}
__device__ __forceinline__ uint32_t key_index(uint32_t key) { return 127u - ((key >> 1) & 127u); }
__device__ __forceinline__ uint16_t key_bits(uint32_t key) { return (uint16_t)(((key & 1u) << 15) | ((key >> 8) & 0x7fffu)); }

// The block tile of one lane: 8 tokens x 8 channels. Non-KVarN modes keep the fp16
// input bits (two channels per register) and widen on use, which halves the live
// registers; KVarN keeps fp32, since it rotates and rescales the tile.
template <bool F32> struct Tile;
// (127 - element index) << 1 of four elements, one byte each: the index part of their keys.
__device__ __forceinline__ uint32_t key_idx4(int e0, int step) {
  uint32_t w = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) w |= (uint32_t)((127 - (e0 + k * step)) << 1) << (8 * k);
  return w;
}

template <> struct Tile<true> {
  float v[8][8];
  __device__ __forceinline__ uint32_t key4(int i, int e, uint32_t iw, int k) const {
    return mag_key(v[i][e], 127 - (int)((iw >> (8 * k)) & 0xffu) / 2);
  }
  __device__ __forceinline__ float f(int i, int e) const { return v[i][e]; }
  __device__ __forceinline__ float d(int i, int e, float off) const { return __fsub_rn(v[i][e], off); }
  __device__ __forceinline__ uint32_t key(int i, int e, int idx) const { return mag_key(v[i][e], idx); }
};
template <> struct Tile<false> {
  uint32_t v[8][4];
  __device__ __forceinline__ uint32_t bits(int i, int e) const { return (e & 1) ? v[i][e >> 1] >> 16 : v[i][e >> 1] & 0xffffu; }
  __device__ __forceinline__ float f(int i, int e) const { return __half2float(__ushort_as_half((unsigned short)bits(i, e))); }
  // x - off rounded once to fp32, read straight from the fp16 half (one mixed-precision fma:
  // x * 1 is exact, so this is the IEEE subtraction)
  __device__ __forceinline__ float d(int i, int e, float off) const {
    float r;
    if (e & 1)
      asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(v[i][e >> 1]), "v"(off));
    else
      asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(v[i][e >> 1]), "v"(off));
    return r;
  }
  __device__ __forceinline__ uint32_t key(int i, int e, int idx) const {
    const uint32_t h = (e & 1) ? v[i][e >> 1] >> 16 : v[i][e >> 1] & 0xffffu;
    return ((h & 0x7fffu) << 8) | ((uint32_t)(127 - idx) << 1) | (h >> 15);
  }
  // The same key from a byte permutation: byte 0 = index byte k of iw, bytes 1-2 = the
  // element's fp16 bits (its sign lands in bit 23), byte 3 = 0; then the sign moves to bit 0.
  __device__ __forceinline__ uint32_t key4(int i, int e, uint32_t iw, int k) const {
    const uint32_t sel = (uint32_t)k | ((4u + 2u * (e & 1)) << 8) | ((5u + 2u * (e & 1)) << 16) | (0x0cu << 24);
    const uint32_t t = __builtin_amdgcn_perm(v[i][e >> 1], iw, sel);
    return (t & 0x007fffffu) | (t >> 23);
  }
};

struct MaxU { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; } };
struct MinF { __device__ float operator()(float a, float b) const { return fminf(a, b); } };
struct MaxF { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };

// The value of another lane by a data-parallel move within each row of 16 lanes.
template <int CTRL, typename T>
__device__ __forceinline__ T dpp_mov(T v) {
  static_assert(sizeof(T) == 4, "32-bit values");
  return __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// Lane l ^ m's value through the LDS permute unit (no vector-ALU instruction: this kernel is
// bound by vector-ALU issue, so cross-row moves go there unless a move fuses into its use).
template <typename T>
__device__ __forceinline__ T shfl_x(T v, int m) {
  if constexpr (sizeof(T) == 4 && !__is_same(T, float)) return (T)__shfl_xor((int)v, m);
  else return __shfl_xor(v, m);
}

// v[e] = this lane's partial for channel 8g + e. Returns the channel totals over
// all 128 tokens in v (identical in every lane holding the channel).
template <typename T, typename Op>
__device__ __forceinline__ void chan_reduce(T (&v)[8], T* buf, int w, int r, int g, Op op) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    v[e] = op(v[e], shfl_x(v[e], 16));
    v[e] = op(v[e], shfl_x(v[e], 32));
  }
  if (r == 0) {
    uint4* dst = reinterpret_cast<uint4*>(buf + w * kD + 8 * g);
    dst[0] = make_uint4(__builtin_bit_cast(uint32_t, v[0]), __builtin_bit_cast(uint32_t, v[1]),
                        __builtin_bit_cast(uint32_t, v[2]), __builtin_bit_cast(uint32_t, v[3]));
    dst[1] = make_uint4(__builtin_bit_cast(uint32_t, v[4]), __builtin_bit_cast(uint32_t, v[5]),
                        __builtin_bit_cast(uint32_t, v[6]), __builtin_bit_cast(uint32_t, v[7]));
  }
  __syncthreads();
  T p[4][8];
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) {
    const uint4* src = reinterpret_cast<const uint4*>(buf + ww * kD + 8 * g);
    const uint4 lo = src[0], hi = src[1];
    p[ww][0] = __builtin_bit_cast(T, lo.x); p[ww][1] = __builtin_bit_cast(T, lo.y);
    p[ww][2] = __builtin_bit_cast(T, lo.z); p[ww][3] = __builtin_bit_cast(T, lo.w);
    p[ww][4] = __builtin_bit_cast(T, hi.x); p[ww][5] = __builtin_bit_cast(T, hi.y);
    p[ww][6] = __builtin_bit_cast(T, hi.z); p[ww][7] = __builtin_bit_cast(T, hi.w);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = op(op(op(p[0][e], p[1][e]), p[2][e]), p[3][e]);
}

// op (minimum or maximum: exact in any order) over the 16 g lanes of a token, identical in
// all of them. Unsigned maxima take data-parallel row moves, which fuse into the maximum
// (one instruction per step); float operands go through the permute unit (a row move would
// stay a separate vector instruction in front of the IEEE minimum / maximum).
template <typename T, typename Op>
__device__ __forceinline__ T tok_reduce(T v, Op op) {
  if constexpr (__is_same(T, uint32_t)) {
    v = op(v, dpp_mov<0xB1>(v));    // quad_perm(1, 0, 3, 2)
    v = op(v, dpp_mov<0x4E>(v));    // quad_perm(2, 3, 0, 1)
    v = op(v, dpp_mov<0x141>(v));   // row_half_mirror: the other quad of the half row
    v = op(v, dpp_mov<0x140>(v));   // row_mirror: the other half of the row
  } else {
    v = op(v, shfl_x(v, 1));
    v = op(v, shfl_x(v, 2));
    v = op(v, shfl_x(v, 4));
    v = op(v, shfl_x(v, 8));
  }
  return v;
}

// Orthonormal Sylvester Hadamard rotation of every token row (8 channels per lane,
// channel bits 3..6 = g bits 0..3).
__device__ __forceinline__ void fwht_rows(float (&x)[8][8], int g) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int hs = 1; hs < 8; hs <<= 1)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (!(e & hs)) {
          const float p = x[i][e], q = x[i][e | hs];
          x[i][e] = __fadd_rn(p, q);
          x[i][e | hs] = __fsub_rn(p, q);
        }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
      const bool hi = (g & m) != 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __shfl_xor(x[i][e], m);
        x[i][e] = hi ? __fsub_rn(p, x[i][e]) : __fadd_rn(x[i][e], p);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) x[i][e] = __fmul_rn(x[i][e], kInvSqrt128);
  }
}

// Makes the tile look modified to the optimiser, so that values derived from it are
// recomputed where they are used instead of being kept live.
template <typename T, int N>
__device__ __forceinline__ void opaque(T (&x)[8][N]) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < N; ++e) asm volatile("" : "+v"(x[i][e]));
}

// Mean and centred sum of squares (m2) of a group of elements.
struct Mom { float mean, m2; };

// Two groups of n elements each merged into one of 2n (the pairwise update of Chan, Golub and
// LeVeque: m2 = m2_a + m2_b + (n / 2) (mean_b - mean_a)^2). The result does not depend on the
// order of the operands, bit for bit (the sums commute, the difference only changes sign), so
// partner lanes that each pass (own, other) end with identical statistics.
__device__ __forceinline__ Mom merge(Mom a, Mom b, float half_n) {
  const float d = __fsub_rn(b.mean, a.mean);
  return {__fmul_rn(__fadd_rn(a.mean, b.mean), 0.5f), __fmaf_rn(__fmul_rn(d, d), half_n, __fadd_rn(a.m2, b.m2))};
}

// Moments of eight values (two passes: the mean, then the squared deviations from it).
__device__ __forceinline__ Mom mom8(const float (&t)[8]) {
  const float sum = __fadd_rn(__fadd_rn(__fadd_rn(t[0], t[1]), __fadd_rn(t[2], t[3])),
                              __fadd_rn(__fadd_rn(t[4], t[5]), __fadd_rn(t[6], t[7])));
  const float mean = __fmul_rn(sum, 0.125f);
  float m2 = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float d = __fsub_rn(t[k], mean);
    m2 = __fmaf_rn(d, d, m2);
  }
  return {mean, m2};
}

template <int CTRL>
__device__ __forceinline__ Mom merge_dpp(Mom m, float half_n) {
  return merge(m, Mom{dpp_mov<CTRL>(m.mean), dpp_mov<CTRL>(m.m2)}, half_n);
}
// Partner rows by lane swaps: rows r and r ^ 1 (X16) or r ^ 2 (X32) of the wave; each swap
// returns the (lower, upper) pair in every lane.
template <bool X32>
__device__ __forceinline__ Mom merge_rows(Mom m, float half_n) {
  const uint32_t a = __float_as_uint(m.mean), b = __float_as_uint(m.m2);
  if constexpr (X32) {
    const auto pa = __builtin_amdgcn_permlane32_swap(a, a, false, false);
    const auto pb = __builtin_amdgcn_permlane32_swap(b, b, false, false);
    return merge(Mom{__uint_as_float(pa[0]), __uint_as_float(pb[0])}, Mom{__uint_as_float(pa[1]), __uint_as_float(pb[1])}, half_n);
  } else {
    const auto pa = __builtin_amdgcn_permlane16_swap(a, a, false, false);
    const auto pb = __builtin_amdgcn_permlane16_swap(b, b, false, false);
    return merge(Mom{__uint_as_float(pa[0]), __uint_as_float(pb[0])}, Mom{__uint_as_float(pa[1]), __uint_as_float(pb[1])}, half_n);
  }
}

// log2 of the population standard deviation of 128 elements from their m2; a zero spread
// keeps the previous log-scale.
__device__ __forceinline__ float log2_std(float m2, float prev) {
  return m2 > 0.f ? __fmaf_rn(__builtin_amdgcn_logf(m2), 0.5f, -3.5f) : prev;
}

// Variance normalisation in the log2 domain: per iteration a channel step, then a token step.
// A step adds the log of the standard deviation of the currently scaled tile to its log-scale;
// since scaling a channel by exp(-c) scales its deviation by the same factor, the channel
// log-scale after its step is the log deviation of the tile scaled by the token factors
// alone (and the token log-scale, after its step, that of the tile scaled by the channel
// factors alone), which is what is computed here, without the accumulated increments. Each
// statistic is one merged (mean, m2) reduction: 8 elements per lane, then lane merges
// (rows of 16 lanes by data-parallel moves, the four rows of a wave by lane swaps, the four
// waves through LDS). Returns the log2-scales of this lane's tokens (rl) and channels (cl).
// exp2 and log2 are the hardware approximations (about one ulp): the KVarN scales are
// reproduced to a relative tolerance, not bit for bit.
__device__ __forceinline__ void varn(const float (&x)[8][8], float (&rl)[8], float (&cl)[8], int iters, Smem& sm,
                                     int w, int r, int g) {
#pragma unroll
  for (int k = 0; k < 8; ++k) { rl[k] = 0.f; cl[k] = 0.f; }
  for (int it = 0; it < iters; ++it) {
    // channel step: per channel, the deviation over tokens of x * exp2(-rl)
    float er[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) er[i] = __builtin_amdgcn_exp2f(-rl[i]);
    Mom cm[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float t[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) t[i] = __fmul_rn(x[i][e], er[i]);
      cm[e] = merge_rows<true>(merge_rows<false>(mom8(t), 4.f), 8.f);
    }
    // cross-wave: two alternating buffers (the channel and token steps in between keep a
    // wave from rewriting a buffer another wave may still read)
    float* bm = (it & 1) ? &sm.rlo[0][0] : reinterpret_cast<float*>(&sm.red[0][0][0]);
    float* bq = (it & 1) ? &sm.rhi[0][0] : reinterpret_cast<float*>(&sm.red[1][0][0]);
    if (r == 0) {
      float4* dm = reinterpret_cast<float4*>(bm + w * kD + 8 * g);
      float4* dq = reinterpret_cast<float4*>(bq + w * kD + 8 * g);
      dm[0] = make_float4(cm[0].mean, cm[1].mean, cm[2].mean, cm[3].mean);
      dm[1] = make_float4(cm[4].mean, cm[5].mean, cm[6].mean, cm[7].mean);
      dq[0] = make_float4(cm[0].m2, cm[1].m2, cm[2].m2, cm[3].m2);
      dq[1] = make_float4(cm[4].m2, cm[5].m2, cm[6].m2, cm[7].m2);
    }
    __syncthreads();
    Mom pw[4][8];
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float4* sm4 = reinterpret_cast<const float4*>(bm + ww * kD + 8 * g);
      const float4* sq4 = reinterpret_cast<const float4*>(bq + ww * kD + 8 * g);
      const float4 m0 = sm4[0], m1 = sm4[1], q0 = sq4[0], q1 = sq4[1];
      pw[ww][0] = {m0.x, q0.x}; pw[ww][1] = {m0.y, q0.y}; pw[ww][2] = {m0.z, q0.z}; pw[ww][3] = {m0.w, q0.w};
      pw[ww][4] = {m1.x, q1.x}; pw[ww][5] = {m1.y, q1.y}; pw[ww][6] = {m1.z, q1.z}; pw[ww][7] = {m1.w, q1.w};
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const Mom m = merge(merge(pw[0][e], pw[1][e], 16.f), merge(pw[2][e], pw[3][e], 16.f), 32.f);
      cl[e] = log2_std(m.m2, cl[e]);
    }
    // token step: per token, the deviation over channels of x * exp2(-cl)
    float ec[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ec[e] = __builtin_amdgcn_exp2f(-cl[e]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float u[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) u[e] = __fmul_rn(x[i][e], ec[e]);
      Mom m = mom8(u);
      m = merge_dpp<0xB1>(m, 4.f);    // quad_perm(1, 0, 3, 2)
      m = merge_dpp<0x4E>(m, 8.f);    // quad_perm(2, 3, 0, 1)
      m = merge_dpp<0x141>(m, 16.f);  // row_half_mirror
      m = merge_dpp<0x140>(m, 32.f);  // row_mirror
      rl[i] = log2_std(m.m2, rl[i]);
    }
  }
  __syncthreads();   // the last step's buffer is free for the later phases
}

// The two planes of eight 3-bit codes given as the nibbles of v (code e in bits 4e..4e+2, bit
// 4e+3 clear): lo2 = the low two bits of code e at bit 2e (bits 0..15 valid), hi1 = bit 2 of code
// e at bit e (bits 0..7 valid); the bits above are left unspecified. Each step keeps every
// other field in place and moves its neighbour down next to it, (a & m) | (b & ~m) being one
// bit-field insert (written out: the compiler otherwise rewrites the chain into more
// instructions from the known-zero bits of the codes).
template <uint32_t M>
__device__ __forceinline__ uint32_t bsel(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "s"(M), "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ void planes3(uint32_t v, uint32_t& lo2, uint32_t& hi1) {
  const uint32_t v2 = v >> 2;                    // also: bit 2 of code e at bit 4e
  uint32_t y = bsel<0x03030303u>(v, v2);          // byte k, bits 0..3: codes 2k, 2k+1
  y = bsel<0x000F000Fu>(y, y >> 4);               // half-word m, bits 0..7: codes 4m .. 4m+3
  lo2 = bsel<0x000000FFu>(y, y >> 8);             // bits 0..15: codes 0 .. 7
  uint32_t z = bsel<0x01010101u>(v2, v2 >> 3);    // byte k, bits 0..1
  z = bsel<0x00030003u>(z, z >> 6);               // half-word m, bits 0..3
  hi1 = bsel<0x0000000Fu>(z, z >> 12);            // bits 0..7
}

// RN(d / s) from r = RN(1 / s): q0 = RN(d r), the exact residual e = d - q0 s (one fma),
// then RN(q0 + e r). With a correctly rounded reciprocal this correction step returns the
// correctly rounded quotient (Markstein's theorem; no overflow or underflow occurs for
// these operands), i.e. the same value as an IEEE division, in three instructions.
__device__ __forceinline__ float div_rn(float d, float s, float r) {
  const float q0 = __fmul_rn(d, r);
  const float e = __fmaf_rn(-q0, s, d);
  return __fmaf_rn(e, r, q0);
}

// NUQ code = number of decision thresholds tau_j <= u (tau ascending, 2^b - 1 of them; the
// host derives them from the codebook so that this equals the first-index argmin of the
// fp32 distances |u - C_j|). One compare and one carry-add per threshold, no branches.
template <int BITS>
__device__ __forceinline__ uint32_t nuq_search(float u, const float* tau) {
  uint32_t code = 0;
#pragma unroll
  for (int t = 0; t < (1 << BITS) - 1; ++t) code += u >= tau[t] ? 1u : 0u;
  return code;
}

// Statistics of one vector: (sa, sb) = RTN/KVarN (s, m), NUQ (z, h), symmetric int4 (s, -),
// rc = RN(1 / divisor) for the element divisions, 0 for a zero divisor (every quotient of a
// finite element then comes out 0, the zero-divisor rule, with no per-element test), and
// off = what an element's difference is taken from (m, z, or 0).
struct VecStats { float sa, sb, rc, off; };

template <int MODE, int BITS>
__device__ __forceinline__ VecStats stats_of(float lo, float hi, float amax) {
  VecStats v;
  if constexpr (MODE == NUQ) {
    v.sa = __fmul_rn(__fadd_rn(hi, lo), 0.5f);   // z
    v.sb = __fmul_rn(__fsub_rn(hi, lo), 0.5f);   // h
    v.rc = v.sb == 0.f ? 0.f : __fdiv_rn(1.f, v.sb);
    v.off = v.sa;
  } else if constexpr (MODE == ASYM) {
    // s = fp16((max - min) / 15), zero = fp16(min + 8 s): min maps to -8, max to 7
    v.sa = __half2float(__float2half_rn(__fdiv_rn(__fsub_rn(hi, lo), 15.0f)));
    v.sb = __half2float(__float2half_rn(__fadd_rn(lo, __fmul_rn(8.0f, v.sa))));
    v.rc = v.sa == 0.f ? 0.f : __fdiv_rn(1.f, v.sa);
    v.off = v.sb;
  } else if constexpr (MODE == SYM) {
    v.sa = __half2float(__float2half_rn(__fdiv_rn(amax, (float)((1 << (BITS - 1)) - 1))));   // absmax / 7 (int8: 127)
    v.sb = 0.f;
    v.rc = v.sa == 0.f ? 0.f : __fdiv_rn(1.f, v.sa);
    v.off = 0.f;
  } else {
    v.sa = __fdiv_rn(__fsub_rn(hi, lo), (float)((1 << BITS) - 1));   // s
    v.sb = lo;                                                       // m
    v.rc = v.sa == 0.f ? 0.f : __fdiv_rn(1.f, v.sa);
    v.off = lo;
  }
  return v;
}

// Lane addr / 4's copy of v, through the LDS permute unit (no vector-ALU instruction).
__device__ __forceinline__ float bperm(int addr, float v) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(v)));
}
// The statistics of another lane's vector (off follows from the others).
template <int MODE>
__device__ __forceinline__ VecStats bperm_stats(int addr, const VecStats& v) {
  VecStats o;
  o.sa = bperm(addr, v.sa);
  o.sb = bperm(addr, v.sb);
  o.rc = bperm(addr, v.rc);
  o.off = MODE == NUQ ? o.sa : (MODE == SYM ? 0.f : o.sb);
  return o;
}
// x[k] for a lane-dependent k in 0..7: three levels of per-lane selects on the bits of k, each a
// byte permute whose selector takes all four bytes of one operand (0x03020100: the second,
// 0x07060504: the first). Written this way because the compiler turns plain selects here into
// an indexed load from a private-memory copy of x.
__device__ __forceinline__ float sel8(const float (&x)[8], int k) {
  const uint32_t s0 = (k & 1) ? 0x07060504u : 0x03020100u, s1 = (k & 2) ? 0x07060504u : 0x03020100u,
                 s2 = (k & 4) ? 0x07060504u : 0x03020100u;
  auto pick = [](uint32_t s, float a, float b) {   // b where the selector takes the first operand
    return __uint_as_float(__builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), s));
  };
  const float a0 = pick(s0, x[0], x[1]), a1 = pick(s0, x[2], x[3]);
  const float a2 = pick(s0, x[4], x[5]), a3 = pick(s0, x[6], x[7]);
  return pick(s2, pick(s1, a0, a1), pick(s1, a2, a3));
}

// Code of one element from d = x - off: RTN/KVarN clamp(rint((x - m) / s)), NUQ argmin over
// the codebook of clamp((x - z) / h, -1, 1), symmetric int4 clamp(rint(x / s), -8, 7) + 8; a
// zero divisor gives code 0 (symmetric: 8) through rc = 0. An outlier position is a NaN: its
// quotient clamps to the lowest code (0).
template <int MODE, int BITS, bool LUT = false>
__device__ __forceinline__ uint32_t code_of(float d, const VecStats& v, const float* tau, const float2* lut = nullptr) {
  constexpr int QMAX = (1 << BITS) - 1;
  if constexpr (MODE == NUQ) {
    const float q = div_rn(d, v.sb, v.rc);
    const float u = fminf(fmaxf(q, -1.f), 1.f);
    if constexpr (LUT) {
      // bucket of u (one fma, truncation of a value in [0, 1024]), then at most one compare;
      // the entry's count is stored as integer bits
      const float2 e = lut[(int)__fmaf_rn(u, 0.5f * kNuqBuckets, 0.5f * kNuqBuckets)];
      return __float_as_uint(e.x) + (u >= e.y ? 1u : 0u);
    }
    return nuq_search<BITS>(u, tau);
  } else if constexpr (MODE == SYM || MODE == ASYM) {
    const float q = rintf(div_rn(d, v.sa, v.rc));
    constexpr int H = 1 << (BITS - 1);   // offset binary: u = q + 8 (int8: q + 128)
    return (uint32_t)((int)fminf(fmaxf(q, (float)-H), (float)(H - 1)) + H);
  } else {
    const float q = rintf(div_rn(d, v.sa, v.rc));
    return (uint32_t)fminf(fmaxf(q, 0.f), (float)QMAX);
  }
}

// One tensor (TENSOR 0: keys, 1: values) of block j of (sequence b, kv head h). KO: outliers
// per vector, 0 (none), 1 (one), 2 (two or more: a.k_out).
template <int MODE, int BITS, int TENSOR, int KO, bool LUT>
__device__ __forceinline__ void quantize_tensor(const QuantArgs& a, Smem& sm, int j, int h, int b) {
  constexpr int tensor = TENSOR;
  const int tid = threadIdx.x, lane = tid & 63, r = lane >> 4, g = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const size_t unit = (size_t)b * a.Hkv + h;
  // paged caches: the sequence's own length places the block and its input rows
  const int len_b = a.pg.table ? a.pg.len[b] : 0;
  const int blk0 = a.pg.table ? len_b >> 7 : a.blk0;
  const int u_old = a.pg.table ? len_b : a.u_old;
  const int in_row0 = a.pg.table ? -len_b : a.in_row0;
  uint8_t* rec = a.rec + (a.pg.table ? ((size_t)page_of(a.pg, b, blk0 + j) * a.Hkv + h)
                                     : (unit * a.max_blocks + (size_t)(blk0 + j))) * a.lay.rec_bytes;
  constexpr int R = 16 * BITS;                                  // bytes per 128 codes
  const int k_out = KO == 0 ? 0 : (KO == 1 ? 1 : a.k_out);
  constexpr bool per_chan = TENSOR == 0 || MODE == SYM || MODE == ASYM;   // vector = a channel over the block's tokens
  int ph = 0;                                                   // alternating cross-wave buffer

  if (k_out > 0)
    for (int i = tid; i < kD * 4; i += kThreads) (&sm.omask[0][0])[i] = 0u;

  // ---- load the block: body tokens appended before this call come from the fp16 ring
  Tile<MODE == KVARN> X;
  {
    const __half* in = (tensor ? a.v_in : a.k_in) + unit * (size_t)a.n_new * kD;
    const __half* tl = a.tail + unit * (size_t)(2 * a.tail_rows * kD) + (size_t)tensor * a.tail_rows * kD;
    const int u0 = (blk0 + j) * kT;   // body token of the block's first row
    uint4 raw[8];
    if (u0 >= u_old) {
      // (uniform) every row from the new input: a buffer resource over the block's 128 rows,
      // the lane's offset in a register and each row's offset in the scalar offset operand
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<__half*>(in + ((size_t)u0 + in_row0) * kD), (short)0, kT * kD * 2, 0x00020000);
      const uint32_t lo = (uint32_t)(((32 * w + r) * kD + 8 * g) * 2);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, lo, 4 * i * kD * 2, 0);
        raw[i] = make_uint4(v.x, v.y, v.z, v.w);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int u = u0 + 32 * w + 4 * i + r;
        const __half* src = u < u_old ? tl + (size_t)(a.sink + u % a.ring_rows) * kD
                                      : in + ((size_t)u + in_row0) * kD;
        raw[i] = *reinterpret_cast<const uint4*>(src + 8 * g);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t wd[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if constexpr (MODE == KVARN) {
          const float2 f = __half22float2(__builtin_bit_cast(__half2, wd[k]));
          X.v[i][2 * k] = f.x;
          X.v[i][2 * k + 1] = f.y;
        } else {
          X.v[i][k] = wd[k];
        }
      }
    }
  }
  float tau[16];   // NUQ decision thresholds (uniform: scalar registers)
  if constexpr (MODE == NUQ) {
#pragma unroll
    for (int c = 0; c < 16; ++c) tau[c] = a.cb[(h * 2 + tensor) * kCbStride + 16 + c];
  }
  if constexpr (LUT) {   // the code table into LDS (read after the statistics' barriers)
    const float2* src = a.nuq_lut + (size_t)(h * 2 + tensor) * kNuqLutStride;
    for (int k = tid; k <= kNuqBuckets; k += kThreads) sm.nlut[k] = src[k];
  }

  // ---- KVarN: rotate, normalise, divide by s1
  if constexpr (MODE == KVARN) {
    float (&x)[8][8] = X.v;
    fwht_rows(x, g);
    float rl[8], cl[8];
    varn(x, rl, cl, a.varn_iters, sm, w, r, g);
    float* s1dst = reinterpret_cast<float*>(rec + (tensor == 0 ? a.lay.k1 : a.lay.v1));
    if (tensor == 0) {   // keys: s1 per token
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float s1 = exp2f(rl[i]), r1 = __fdiv_rn(1.f, s1);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[i][e] = div_rn(x[i][e], s1, r1);
        if (g == 0) s1dst[32 * w + 4 * i + r] = s1;
      }
    } else {             // values: s1 per channel
      float s1[8], r1[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) { s1[e] = exp2f(cl[e]); r1[e] = __fdiv_rn(1.f, s1[e]); }
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[i][e] = div_rn(x[i][e], s1[e], r1[e]);
      if (w == 0 && r == 0) {
        reinterpret_cast<float4*>(s1dst + 8 * g)[0] = make_float4(s1[0], s1[1], s1[2], s1[3]);
        reinterpret_cast<float4*>(s1dst + 8 * g)[1] = make_float4(s1[4], s1[5], s1[6], s1[7]);
      }
    }
  }

  // ---- outlier selection: per vector the k_out largest keys, one max-reduction per round
  // (rounds after the first skip the keys already taken); thr = the last one taken
  // thr[e] for channel 8g+e when per_chan, thr[i] for token t_i otherwise
  uint32_t thr[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) thr[k] = 0xffffffffu;
  // index bytes of this lane's elements: per channel the token 32w + 4i + r (i = 0..7), per
  // token the channel 8g + e (e = 0..7)
  const uint32_t kiw[2] = {per_chan ? key_idx4(32 * w + r, 4) : key_idx4(8 * g, 1),
                           per_chan ? key_idx4(32 * w + 16 + r, 4) : key_idx4(8 * g + 4, 1)};
  for (int p = 0; p < k_out; ++p) {
    opaque(X.v);   // keeps the per-element keys from being hoisted out of the loop (64 more live registers)
    uint32_t best[8];
    if constexpr (per_chan) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t key = X.key4(i, e, kiw[i >> 2], i & 3);
          m = (KO == 1 || key < thr[e]) ? (key > m ? key : m) : m;
        }
        best[e] = m;
      }
      chan_reduce(best, &sm.red[ph][0][0], w, r, g, MaxU());
      ph ^= 1;
      if (w == 0 && r == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sm.okey[8 * g + e][p] = best[e];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t m = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t key = X.key4(i, e, kiw[e >> 2], e & 3);
          m = (KO == 1 || key < thr[i]) ? (key > m ? key : m) : m;
        }
        best[i] = tok_reduce(m, MaxU());
      }
      if (g == 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) sm.okey[32 * w + 4 * i + r][p] = best[i];
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) thr[k] = best[k];
  }
  // this lane's outliers. One per vector: its element index, compared directly (d = index
  // minus this lane's first element). Several: bit 8(i & 3) + e of om[i >> 2].
  int d1[8];
  uint32_t om[2] = {0u, 0u};
  if constexpr (KO == 1) {
#pragma unroll
    for (int k = 0; k < 8; ++k) d1[k] = (int)key_index(thr[k]) - (per_chan ? 32 * w + r : 8 * g);
  } else if constexpr (KO == 2) {
    opaque(X.v);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool o = per_chan ? X.key4(i, e, kiw[i >> 2], i & 3) >= thr[e] : X.key4(i, e, kiw[e >> 2], e & 3) >= thr[i];
        om[i >> 2] |= o ? (1u << (8 * (i & 3) + e)) : 0u;
      }
  }
  auto is_out = [&](int i, int e) -> bool {
    if constexpr (KO == 0) return false;
    else if constexpr (KO == 1) return per_chan ? d1[e] == 4 * i : d1[i] == e;
    else return (om[i >> 2] >> (8 * (i & 3) + e)) & 1u;
  };
  if constexpr (KO > 0) {
    // Outlier positions become NaN in the tile: minimum and maximum skip a NaN, so the
    // statistics are those of the non-outliers, and the code of a NaN comes out as 0 (the
    // code stored at an outlier position; its fp16 value replaces it at decode).
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int h = 0; h < 4; ++h)
        X.v[i][h] |= (is_out(i, 2 * h) ? 0x7fffu : 0u) | (is_out(i, 2 * h + 1) ? 0x7fff0000u : 0u);
  }

  // ---- statistics over the non-outliers
  if constexpr (MODE != KVARN) opaque(X.v);   // widen again where used (keeps 32, not 64, tile registers)
  VecStats vs[8];   // per channel e when per_chan, per token i otherwise
  if constexpr (per_chan) {
    float lo[8], hi[8];
    if constexpr (MODE != KVARN) {
      // on the fp16 tile, two channels per packed min / max (exact: the elements are fp16;
      // a NaN, an outlier, is skipped as by fminf / fmaxf)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        h2 mn = __builtin_bit_cast(h2, X.v[0][k]);
        h2 mx = MODE == SYM ? __builtin_elementwise_abs(mn) : mn;
#pragma unroll
        for (int i = 1; i < 8; ++i) {
          const h2 x = __builtin_bit_cast(h2, X.v[i][k]);
          mn = __builtin_elementwise_min(mn, x);
          mx = __builtin_elementwise_max(mx, MODE == SYM ? __builtin_elementwise_abs(x) : x);
        }
        lo[2 * k] = (float)mn[0];
        lo[2 * k + 1] = (float)mn[1];
        hi[2 * k] = MODE == SYM ? fmaxf(0.f, (float)mx[0]) : (float)mx[0];
        hi[2 * k + 1] = MODE == SYM ? fmaxf(0.f, (float)mx[1]) : (float)mx[1];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        lo[e] = INFINITY;
        hi[e] = -INFINITY;
#pragma unroll
        for (int i = 0; i < 8; ++i) {   // an outlier is a NaN here: skipped
          const float x = X.f(i, e);
          lo[e] = fminf(lo[e], x);
          hi[e] = fmaxf(hi[e], x);
        }
      }
    }
    // both reductions share one barrier
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      lo[e] = fminf(lo[e], __shfl_xor(lo[e], 16));
      lo[e] = fminf(lo[e], __shfl_xor(lo[e], 32));
      hi[e] = fmaxf(hi[e], __shfl_xor(hi[e], 16));
      hi[e] = fmaxf(hi[e], __shfl_xor(hi[e], 32));
    }
    if (r == 0) {
      float4* dl = reinterpret_cast<float4*>(&sm.rlo[w][8 * g]);
      float4* dh = reinterpret_cast<float4*>(&sm.rhi[w][8 * g]);
      dl[0] = make_float4(lo[0], lo[1], lo[2], lo[3]); dl[1] = make_float4(lo[4], lo[5], lo[6], lo[7]);
      dh[0] = make_float4(hi[0], hi[1], hi[2], hi[3]); dh[1] = make_float4(hi[4], hi[5], hi[6], hi[7]);
    }
    __syncthreads();
    // the statistics (their divisions are the costly part) of channels 8g + 2r and 8g + 2r + 1
    // are derived in row r of the wave; the other rows' come by lane permutes
    VecStats own[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int c = 8 * g + 2 * r + k;
      const float l = fminf(fminf(fminf(sm.rlo[0][c], sm.rlo[1][c]), sm.rlo[2][c]), sm.rlo[3][c]);
      const float u = fmaxf(fmaxf(fmaxf(sm.rhi[0][c], sm.rhi[1][c]), sm.rhi[2][c]), sm.rhi[3][c]);
      own[k] = stats_of<MODE, BITS>(l, u, u);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) vs[e] = bperm_stats<MODE>(4 * g + 64 * (e >> 1), own[e & 1]);
  } else {
    float lot[8], hit[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float lo = INFINITY, hi = -INFINITY;
      if constexpr (MODE != KVARN) {   // packed fp16 min / max over the token's 8 channels
        const h2 a0 = __builtin_bit_cast(h2, X.v[i][0]), a1 = __builtin_bit_cast(h2, X.v[i][1]);
        const h2 a2 = __builtin_bit_cast(h2, X.v[i][2]), a3 = __builtin_bit_cast(h2, X.v[i][3]);
        const h2 mn = __builtin_elementwise_min(__builtin_elementwise_min(a0, a1), __builtin_elementwise_min(a2, a3));
        const h2 mx = __builtin_elementwise_max(__builtin_elementwise_max(a0, a1), __builtin_elementwise_max(a2, a3));
        lo = fminf(lo, fminf((float)mn[0], (float)mn[1]));
        hi = fmaxf(hi, fmaxf((float)mx[0], (float)mx[1]));
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {   // an outlier is a NaN here: skipped
          const float x = X.f(i, e);
          lo = fminf(lo, x);
          hi = fmaxf(hi, x);
        }
      }
      lot[i] = tok_reduce(lo, MinF());
      hit[i] = tok_reduce(hi, MaxF());
    }
    // the statistics of token t_i are derived in lanes g = i, 8 + i of the row; the other
    // lanes take them by lane permutes
    const VecStats own = stats_of<MODE, BITS>(sel8(lot, g & 7), sel8(hit, g & 7), sel8(hit, g & 7));
#pragma unroll
    for (int i = 0; i < 8; ++i) vs[i] = bperm_stats<MODE>(64 * r + 4 * i, own);
  }

  // ---- statistics out
  {
    uint8_t* st = rec + (tensor == 0 ? a.lay.ks : a.lay.vs);
    if constexpr (per_chan) {
      if (w == 0 && r == 0) {
        if constexpr (MODE == SYM) {
          uint32_t hw[4];
#pragma unroll
          for (int k = 0; k < 4; ++k)
            hw[k] = __builtin_bit_cast(uint32_t, __halves2half2(__float2half_rn(vs[2 * k].sa), __float2half_rn(vs[2 * k + 1].sa)));
          *reinterpret_cast<uint4*>(st + 16 * g) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        } else if constexpr (MODE == ASYM) {   // fp16 scales, then fp16 zero points
          uint32_t hs[4], hz[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            hs[k] = __builtin_bit_cast(uint32_t, __halves2half2(__float2half_rn(vs[2 * k].sa), __float2half_rn(vs[2 * k + 1].sa)));
            hz[k] = __builtin_bit_cast(uint32_t, __halves2half2(__float2half_rn(vs[2 * k].sb), __float2half_rn(vs[2 * k + 1].sb)));
          }
          *reinterpret_cast<uint4*>(st + 16 * g) = make_uint4(hs[0], hs[1], hs[2], hs[3]);
          *reinterpret_cast<uint4*>(st + 256 + 16 * g) = make_uint4(hz[0], hz[1], hz[2], hz[3]);
        } else {
          float4* ds = reinterpret_cast<float4*>(st) + 2 * g;
          float4* dm = reinterpret_cast<float4*>(st + 512) + 2 * g;
          ds[0] = make_float4(vs[0].sa, vs[1].sa, vs[2].sa, vs[3].sa); ds[1] = make_float4(vs[4].sa, vs[5].sa, vs[6].sa, vs[7].sa);
          dm[0] = make_float4(vs[0].sb, vs[1].sb, vs[2].sb, vs[3].sb); dm[1] = make_float4(vs[4].sb, vs[5].sb, vs[6].sb, vs[7].sb);
        }
      }
    } else if (g == 0) {
      float* ds = reinterpret_cast<float*>(st);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int t = 32 * w + 4 * i + r;
        ds[t] = vs[i].sa;
        ds[128 + t] = vs[i].sb;
      }
    }
  }

  // ---- codes (an outlier position, a NaN in the tile, gets code 0)
  if constexpr (MODE != KVARN) opaque(X.v);
  if constexpr (TENSOR == 0) {
    // key rows, token-major: this lane's 8 codes of row t_i go straight to memory
    uint8_t* kc = rec + a.lay.kc;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = 32 * w + 4 * i + r;
      uint32_t c[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) c[e] = code_of<MODE, BITS, LUT>(X.d(i, e, vs[e].off), vs[e], tau, sm.nlut);
      uint8_t* row = kc + (size_t)t * R;
      if constexpr (BITS == 8) {
        *reinterpret_cast<uint2*>(row + 8 * g) =
            make_uint2(c[0] | c[1] << 8 | c[2] << 16 | c[3] << 24, c[4] | c[5] << 8 | c[6] << 16 | c[7] << 24);
      } else if constexpr (BITS == 4) {
        uint32_t v = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) v |= c[e] << (4 * e);
        *reinterpret_cast<uint32_t*>(row + 4 * g) = v;
      } else if constexpr (BITS == 2) {
        uint32_t v = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) v |= c[e] << (2 * e);
        *reinterpret_cast<uint16_t*>(row + 2 * g) = (uint16_t)v;
      } else {
        uint32_t v = 0, lo2, hi1;
#pragma unroll
        for (int e = 0; e < 8; ++e) v |= c[e] << (4 * e);
        planes3(v, lo2, hi1);
        *reinterpret_cast<uint16_t*>(row + 2 * g) = (uint16_t)lo2;
        row[32 + g] = (uint8_t)hi1;
      }
    }
  } else {
    // value codes: LDS tile, then one thread per channel-major half-row
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = 32 * w + 4 * i + r;
      uint32_t c[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        c[e] = code_of<MODE, BITS, LUT>(X.d(i, e, (per_chan ? vs[e] : vs[i]).off), per_chan ? vs[e] : vs[i], tau, sm.nlut);
      *reinterpret_cast<uint2*>(&sm.vq[t * kD + 8 * g]) =
          make_uint2(c[0] | c[1] << 8 | c[2] << 16 | c[3] << 24, c[4] | c[5] << 8 | c[6] << 16 | c[7] << 24);
    }
    __syncthreads();
    {
      constexpr int RH = R / 2;
      const int half = tid >> 7, c = tid & 127;
      // position p of the half-row holds token 16*((p>>2)&3) + 4*(p>>4) + (p&3) of the half
      auto code = [&](int p) -> uint32_t {
        return sm.vq[(64 * half + 16 * ((p >> 2) & 3) + 4 * (p >> 4) + (p & 3)) * kD + c];
      };
      uint8_t* dst = rec + a.lay.vc + (size_t)(half * 128 + c) * RH;
      if constexpr (BITS == 8) {
        uint32_t wd[16];
#pragma unroll
        for (int k = 0; k < 16; ++k)
          wd[k] = code(4 * k) | code(4 * k + 1) << 8 | code(4 * k + 2) << 16 | code(4 * k + 3) << 24;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          reinterpret_cast<uint4*>(dst)[k] = make_uint4(wd[4 * k], wd[4 * k + 1], wd[4 * k + 2], wd[4 * k + 3]);
      } else if constexpr (BITS == 4) {
        uint32_t wd[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          uint32_t v = 0;
#pragma unroll
          for (int e = 0; e < 8; ++e) v |= code(8 * k + e) << (4 * e);
          wd[k] = v;
        }
        reinterpret_cast<uint4*>(dst)[0] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
        reinterpret_cast<uint4*>(dst)[1] = make_uint4(wd[4], wd[5], wd[6], wd[7]);
      } else if constexpr (BITS == 2) {
        uint32_t wd[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint32_t v = 0;
#pragma unroll
          for (int e = 0; e < 16; ++e) v |= code(16 * k + e) << (2 * e);
          wd[k] = v;
        }
        *reinterpret_cast<uint4*>(dst) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
      } else {
        uint32_t lo2[4], hi1[2] = {0u, 0u};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint32_t l[2], h[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            uint32_t v = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) v |= code(16 * k + 8 * hh + e) << (4 * e);
            planes3(v, l[hh], h[hh]);
          }
          lo2[k] = (l[0] & 0xFFFFu) | (l[1] << 16);
          hi1[k >> 1] |= ((h[0] & 0xFFu) | ((h[1] & 0xFFu) << 8)) << (16 * (k & 1));
        }
        *reinterpret_cast<uint4*>(dst) = make_uint4(lo2[0], lo2[1], lo2[2], lo2[3]);
        *reinterpret_cast<uint2*>(dst + 16) = make_uint2(hi1[0], hi1[1]);
      }
    }
  }

  // ---- outliers: keys CSR by token (row t, column c), values CSC by channel (row c,
  // column t); entries sorted by (row, column), fp16 value bits kept exactly. The keys of
  // every vector's outliers were recorded during the selection; each encodes its element.
  if (KO != 0) {
    __syncthreads();                                   // okey complete, omask cleared
    const int n_ent = 128 * k_out;
    auto place = [&](int n, int& row, int& col, uint32_t& key) {
      const int v = n & 127, p = n >> 7;
      key = sm.okey[v][p];
      const int e = (int)key_index(key);
      const int t = per_chan ? e : v, c = per_chan ? v : e;
      row = tensor == 0 ? t : c;
      col = tensor == 0 ? c : t;
    };
    for (int n = tid; n < n_ent; n += kThreads) {
      int row, col;
      uint32_t key;
      place(n, row, col, key);
      atomicOr(&sm.omask[row][col >> 5], 1u << (col & 31));
    }
    __syncthreads();
    if (w == 0) {
      const int n0 = __popc(sm.omask[2 * lane][0]) + __popc(sm.omask[2 * lane][1]) + __popc(sm.omask[2 * lane][2]) +
                     __popc(sm.omask[2 * lane][3]);
      const int n1 = __popc(sm.omask[2 * lane + 1][0]) + __popc(sm.omask[2 * lane + 1][1]) +
                     __popc(sm.omask[2 * lane + 1][2]) + __popc(sm.omask[2 * lane + 1][3]);
      int incl = n0 + n1;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d);
        if (lane >= d) incl += y;
      }
      const int excl = incl - n0 - n1;
      sm.optr[2 * lane] = (uint16_t)excl;
      sm.optr[2 * lane + 1] = (uint16_t)(excl + n0);
      if (lane == 63) sm.optr[128] = (uint16_t)incl;
    }
    __syncthreads();
    uint16_t* val = reinterpret_cast<uint16_t*>(rec + (tensor == 0 ? a.lay.ko_val : a.lay.vo_val));
    uint16_t* ptr = reinterpret_cast<uint16_t*>(rec + (tensor == 0 ? a.lay.ko_ptr : a.lay.vo_ptr));
    uint8_t* idx = rec + (tensor == 0 ? a.lay.ko_idx : a.lay.vo_idx);
    if (tid <= 128) ptr[tid] = sm.optr[tid];
    for (int n = tid; n < n_ent; n += kThreads) {
      int row, col;
      uint32_t key;
      place(n, row, col, key);
      int pos = sm.optr[row];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t m = sm.omask[row][d];
        const int lim = col - 32 * d;   // bits of word d below col
        pos += lim >= 32 ? __popc(m) : (lim > 0 ? __popc(m & ((1u << lim) - 1u)) : 0);
      }
      val[pos] = key_bits(key);   // the element's fp16 input bits, exactly
      idx[pos] = (uint8_t)col;
    }
  }
}

// NUQ with 3 or 4 bits codes through the table of its codebook when the table is usable
// (entry 0's count is -1 otherwise, and the thresholds are counted).
template <int MODE, int BITS, int TENSOR, int KO>
__device__ __forceinline__ void run_tensor(const QuantArgs& a, Smem& sm, int j, int h, int b) {
  if constexpr (MODE == NUQ && BITS >= 3) {
    if (__float_as_uint(a.nuq_lut[(size_t)(h * 2 + TENSOR) * kNuqLutStride].x) != 0xFFFFFFFFu) {
      quantize_tensor<MODE, BITS, TENSOR, KO, true>(a, sm, j, h, b);
      return;
    }
  }
  quantize_tensor<MODE, BITS, TENSOR, KO, false>(a, sm, j, h, b);
}

template <int MODE, int BITS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(MODE == KVARN ? 2 : 4))) void quantize_kernel(QuantArgs a) {
  __shared__ Smem sm;
  const int j = blockIdx.x >> 1, h = blockIdx.y, b = blockIdx.z;
  // paged caches: the grid covers the largest number of blocks any sequence completes
  if (a.pg.table && j >= ((a.pg.len[b] + a.pg.n_new[b]) >> 7) - (a.pg.len[b] >> 7)) return;
  if (MODE == KVARN || a.k_out == 0) {
    if (blockIdx.x & 1) run_tensor<MODE, BITS, 1, 0>(a, sm, j, h, b);
    else run_tensor<MODE, BITS, 0, 0>(a, sm, j, h, b);
  } else if constexpr (MODE != KVARN) {
    if (a.k_out == 1) {
      if (blockIdx.x & 1) run_tensor<MODE, BITS, 1, 1>(a, sm, j, h, b);
      else run_tensor<MODE, BITS, 0, 1>(a, sm, j, h, b);
    } else {
      if (blockIdx.x & 1) run_tensor<MODE, BITS, 1, 2>(a, sm, j, h, b);
      else run_tensor<MODE, BITS, 0, 2>(a, sm, j, h, b);
    }
  }
}

// New fp16 rows into the (layer, sequence, kv head)'s fp16 region: sink tokens to their
// rows, body tokens to their ring slots.
__global__ __launch_bounds__(kThreads) void tail_kernel(TailArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  const size_t unit = (size_t)b * a.Hkv + h;
  int n_sink = a.n_sink, ring_src0 = a.ring_src0, ring_count = a.ring_count, ring_u0 = a.ring_u0;
  if (a.pg.table) {   // paged: the new tokens after the sequence's last complete block
    const int len = a.pg.len[b], end = len + a.pg.n_new[b];
    n_sink = 0;
    ring_u0 = max(len, end & ~(kT - 1));
    ring_count = end - ring_u0;
    ring_src0 = ring_u0 - len;
  }
  const int n_rows = n_sink + ring_count;
  // workgroup z copies rows 16z .. 16z + 15 of the list (one 16-byte piece per thread and
  // tensor: a single memory round trip)
  const int r0 = 16 * (int)blockIdx.z, r1 = min(n_rows, r0 + 16);
  if (r0 >= r1) return;
  for (int tensor = 0; tensor < 2; ++tensor) {
    const __half* in = (tensor ? a.v_in : a.k_in) + unit * (size_t)a.n_new * kD;
    __half* tl = a.tail + unit * (size_t)(2 * a.tail_rows * kD) + (size_t)tensor * a.tail_rows * kD;
    for (int id = r0 * 16 + threadIdx.x; id < r1 * 16; id += kThreads) {
      const int i = id >> 4, ch = (id & 15) * 8;
      int src, dst;
      if (i < n_sink) {
        src = i;
        dst = a.sink_row0 + i;
      } else {
        src = ring_src0 + (i - n_sink);
        dst = a.sink + (ring_u0 + (i - n_sink)) % a.ring_rows;
      }
      *reinterpret_cast<uint4*>(tl + (size_t)dst * kD + ch) = *reinterpret_cast<const uint4*>(in + (size_t)src * kD + ch);
    }
  }
}

template <int MODE, int BITS>
hipError_t launch_q(const QuantArgs& a, int n_blocks, int batch, hipStream_t s) {
  // x: (block, tensor) pairs, tensor = the low bit
  hipLaunchKernelGGL((quantize_kernel<MODE, BITS>), dim3(2 * n_blocks, a.Hkv, batch), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(int mode, int bits, const QuantArgs& a, int n_blocks, int batch,
                           hipStream_t s) {
  switch (mode * 8 + bits) {
    case RTN * 8 + 2: return launch_q<RTN, 2>(a, n_blocks, batch, s);
    case RTN * 8 + 3: return launch_q<RTN, 3>(a, n_blocks, batch, s);
    case RTN * 8 + 4: return launch_q<RTN, 4>(a, n_blocks, batch, s);
    case RTN * 8 + 8: return launch_q<RTN, 8>(a, n_blocks, batch, s);
    case NUQ * 8 + 2: return launch_q<NUQ, 2>(a, n_blocks, batch, s);
    case NUQ * 8 + 3: return launch_q<NUQ, 3>(a, n_blocks, batch, s);
    case NUQ * 8 + 4: return launch_q<NUQ, 4>(a, n_blocks, batch, s);
    case KVARN * 8 + 2: return launch_q<KVARN, 2>(a, n_blocks, batch, s);
    case KVARN * 8 + 3: return launch_q<KVARN, 3>(a, n_blocks, batch, s);
    case KVARN * 8 + 4: return launch_q<KVARN, 4>(a, n_blocks, batch, s);
    case KVARN * 8 + 8: return launch_q<KVARN, 8>(a, n_blocks, batch, s);
    case SYM * 8 + 4: return launch_q<SYM, 4>(a, n_blocks, batch, s);
    case SYM * 8 + 8: return launch_q<SYM, 8>(a, n_blocks, batch, s);
    case ASYM * 8 + 4: return launch_q<ASYM, 4>(a, n_blocks, batch, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_tail(const TailArgs& a, int batch, hipStream_t s) {
  // one workgroup per 16 rows of the largest list (sink rows and ring slots: tail_rows)
  hipLaunchKernelGGL(tail_kernel, dim3(a.Hkv, batch, (a.tail_rows + 15) / 16), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvq
