// Split-K decode attention on the matrix cores (v_mfma_f32_16x16x32_f16), for
// caches without pre-RoPE keys, without outliers and at 2 or 4 bits (uniform
// RTN, KVarN and symmetric int4). Other configurations use the VALU kernel.
//
// Same computation as the VALU kernel ("KVQuant reading notes" Algorithm 1
// attention part; "KVarN" method step 5; "reproducing TurboQuant" 4.2): for the
// query heads of one kv head, softmax(scale * q . k_hat) weighted sum of v_hat
// over all cached tokens, dequantized from the packed codes on the fly.
//
// Work decomposition: workgroup = one split of one (sequence, kv head), four
// waves. At 2 bits wave w streams whole blocks w, w + 4, ... (both 64-token halves:
// the block's Q' operand, statistics and softmax update are made once); at 4 bits
// the waves of a pair share blocks, wave w taking half w & 1 of blocks w / 2,
// w / 2 + 2, ... (two halves' record buffers would not fit in registers). The next
// block's loads are issued, unconditionally, before the current one is processed,
// through a buffer resource over the split's records (past the split's end they
// read nothing); the first block's loads are issued before the query is staged.
// Per wave and 64-token half block:
//   * scores S^T = K_codes (64 tokens x 128 channels) . Q' (128 x 16): the
//     codes enter the matrix core as exact fp16 integers (one bit-field select
//     into the exponent of 1024 and one packed fma per code pair); Q' = q * s_c
//     per block (the per-channel key scale) as an fp16 high part in columns
//     0..7 and the low part (the rounding error, rounded) in columns 8..15, so
//     one product covers both and a row move adds them; the zero point enters as
//     a per-head bias sum_c q_c m_c.
//   * P.V as O = V_codes^T (128 channels x 64 tokens) . P' (64 x 16): P' is the
//     probability times the per-token value scale, taken straight from the
//     score registers (the value half-rows store tokens in the order that makes
//     this possible), split into the same high / low columns; per-channel
//     scales (KVarN s1, int4 scales) multiply the per-block product before it
//     is accumulated; the two columns of a head are added once at the end.
//   * the online softmax runs per head on the 16 scores per half each lane holds
//     (the accumulators are rescaled only when some running maximum moved); the
//     fp16 tail is handled by a vector-unit pass over its rows.
//   * fp16 has a narrow exponent range, so the fp32 operands are brought near 1 by a
//     power of two before the split (exact, and undone after the product): Q' per head
//     by its largest |q_c s_c|, P' per block by its largest value scale S_t. Data
//     of any magnitude in the fp16 input range, and KVarN blocks whose two scales
//     trade magnitude (s_RTN tiny and s1 huge, or the reverse), keep full precision.
#include "kvq_decode_common.h"

namespace kvq {
namespace {

// 1 / x for x a power of two (normal), exactly: 2^(1 - e) with x = 0.5 * 2^e.
__device__ __forceinline__ float recip_pow2(float x) {
  return __builtin_amdgcn_ldexpf(1.f, 1 - __builtin_amdgcn_frexp_expf(x));
}

using namespace dec;

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));
typedef uint32_t u2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack2(float a, float b) {   // two fp32 -> fp16 pair, RNE
  h2 v;
  v[0] = (_Float16)a;
  v[1] = (_Float16)b;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ h8 make8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const u4v v = {a, b, c, d};
  return __builtin_bit_cast(h8, v);
}

// Sum / maximum over the four rows of the wave (lanes l, l ^ 16, l ^ 32, l ^ 48) by lane swaps
// on the vector unit; each swap returns the (even row, odd row) or (low half, high half) pair in
// every lane, so all four lanes end with the same bits.
__device__ __forceinline__ float rows_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float rows_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float s = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// (x & mask) | 0x64006400 in one v_bfi_b32 (the exponent bits of 1024 lie outside every mask
// used here); written out because the compiler otherwise emits an and and an or. The result
// only feeds vector instructions (fix), never a matrix-core operand directly.
__device__ __forceinline__ uint32_t with_exp(uint32_t x, uint32_t mask) {
  uint32_t r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(mask), "v"(x), "s"(0x64006400u));
  return r;
}

// A pair (1024 + K*c0, 1024 + K*c1) from with_exp (K = 1, 4, 16 or 64: a code field at bit
// 0, 2, 4 or 6 of each 16-bit half), mapped to the exact small integers c - OFF by one fma:
// (1024 + K*c) / K is exact in fp16 and so is the fused subtraction.
template <int K, int OFF>
__device__ __forceinline__ uint32_t fix(uint32_t magic_pair) {
  constexpr _Float16 inv = (_Float16)(1.0f / K), off = (_Float16)(-(1024 / K + OFF));
  const h2 d = __builtin_elementwise_fma(__builtin_bit_cast(h2, magic_pair), h2{inv, inv}, h2{off, off});
  return __builtin_bit_cast(uint32_t, d);
}

// Slot i (0..7) of an MFMA operand built from one packed word of codes: 4-bit words give
// pairs (e, e+4) of their 8 codes; 2-bit words give pairs (e, e+8) of their 16 codes, the
// low (h = 0) or high (h = 1) four pairs per operand.
__host__ __device__ constexpr int slot4(int i) { return (i & 1) ? (i >> 1) + 4 : (i >> 1); }
__host__ __device__ constexpr int slot2(int h, int i) { return (i & 1) ? (i >> 1) + 4 * h + 8 : (i >> 1) + 4 * h; }

// Eight codes of operand k-step ks, as fp16 integers minus OFF. The code fields of the low
// byte of each 16-bit half are masked in place; one shift by 8 brings the high bytes down.
template <int BITS, int OFF>
__device__ __forceinline__ h8 codes8(const uint32_t* w, int ks) {
  if constexpr (BITS == 4) {
    const uint32_t x = w[ks], y = x >> 8;
    return make8(fix<1, OFF>(with_exp(x, 0x000F000Fu)), fix<16, OFF>(with_exp(x, 0x00F000F0u)),
                 fix<1, OFF>(with_exp(y, 0x000F000Fu)), fix<16, OFF>(with_exp(y, 0x00F000F0u)));
  } else {
    const uint32_t x = (ks & 1) ? w[ks >> 1] >> 8 : w[ks >> 1];
    return make8(fix<1, OFF>(with_exp(x, 0x00030003u)), fix<4, OFF>(with_exp(x, 0x000C000Cu)),
                 fix<16, OFF>(with_exp(x, 0x00300030u)), fix<64, OFF>(with_exp(x, 0x00C000C0u)));
  }
}

// Channel (0..31, within a lane's 32-channel key chunk) of slot i of score k-step ks.
template <int BITS>
__host__ __device__ constexpr int kchan(int ks, int i) {
  return BITS == 4 ? 8 * ks + slot4(i) : 16 * (ks >> 1) + slot2(ks & 1, i);
}
// Position (0..15, within a lane's 16-position value chunk) of slot i of P.V k-step ks.
template <int BITS>
__host__ __device__ constexpr int vpos(int ks, int i) {
  return BITS == 4 ? 8 * ks + slot4(i) : slot2(ks, i);
}

// Matrix-core column n (0..15) of both products: n < 8 carries the fp16 high part of head n,
// n >= 8 the low part (the fp32 operand minus its fp16 rounding, rounded) of head n - 8, so
// one product gives both parts and the row move "row_ror:8" (lane n <-> n ^ 8) adds them.
template <int MODE, int BITS, int G>
struct MfmaDecoder {
  static_assert(G <= 8, "the high and low parts of the heads share the 16 columns");
  static constexpr int R = 16 * BITS;        // bytes per 128 codes
  static constexpr int RH = R / 2;           // bytes per 64 codes
  static constexpr int KW = R / 16;          // dwords of a lane's 32-channel key chunk
  static constexpr int VW = RH / 16;         // dwords of a lane's 16-position value chunk
  static constexpr int OFFK = MODE == SYM ? 8 : 0;          // key codes enter as c - OFFK
  static constexpr int OFFV = MODE == SYM ? 8 : (1 << (BITS - 1));   // value codes: c - OFFV (centred)
  static constexpr int META = MODE == SYM ? 512 : (MODE == KVARN ? 3072 : 2048);   // ks, vs (, k1, v1) bytes
  static constexpr int NMETA = (META + 1023) / 1024;                              // 16-byte chunks per lane
  static constexpr bool QF16 = MODE == SYM;   // query and key scales are fp16: operand by packed fp16 math
  // 64-token halves a wave processes per block. 2 bits: whole blocks, so that the block's
  // Q' operand, statistics and softmax update are made once per block, not once per half;
  // 4 bits: the record buffers would not fit twice in registers, so a wave takes one half
  // of every other block (the two waves of a pair share the blocks).
  static constexpr int NH = BITS == 2 ? 2 : 1;

  struct Buf {
    uint32_t kw[4 * NH][KW];  // key chunks of tokens 16*tt + n of the wave's halves, channels 32*q .. 32*q+31
    uint32_t vw[NH][8][VW];   // per half: value chunks of channels 16*ct + n, positions 16*q .. 16*q+15
    uint4 meta[NMETA];        // block statistics (staged in LDS)
  };

  const DecodeArgs& a;
  const int lane, w, par, n, q;
  const uint32_t lo_mask;     // all ones on the low-part columns (n >= 8)
  __amdgpu_buffer_rsrc_t rs;  // this (sequence, kv head)'s records
  uint32_t koff, voff;        // this lane's key / value chunk offsets in a record
  uint8_t* meta;              // this wave's LDS copy of the block statistics
  uint32_t qh[QF16 ? 16 : 1]; // fp16 query pairs of head n & 7 in operand slot order (0 if n & 7 >= G)
  float qv[QF16 ? 1 : 32];    // fp32 query of head n & 7, channels 32*q .. 32*q+31
  f4 acc[8];                  // O[16*ct + 4*q + e][column n]
  float m_run, l_run, pm;     // head n & 7 (l_run, pm: this lane's share)
  float vsc;                  // RTN, KVarN: the power of two acc is currently scaled by (wave-uniform)

  __device__ MfmaDecoder(const DecodeArgs& args, int lane_, int w_, uint8_t* meta_)
      : a(args), lane(lane_), w(w_), par(w_ & 1), n(lane_ & 15), q(lane_ >> 4),
        lo_mask((lane_ & 8) ? 0xFFFFFFFFu : 0u), meta(meta_) {
    koff = a.lay.kc + (uint32_t)(((NH == 1 ? 64 * par : 0) + n) * R + q * (R / 4));
    voff = a.lay.vc + (uint32_t)((NH == 1 ? par * (128 * RH) : 0) + n * RH + q * (RH / 4));
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) acc[ct] = f4{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;
    l_run = 0.f;
    pm = 0.f;
    vsc = 1.f;
  }

  // The query of head n & 7 (qs: [G][128] in LDS, KVarN: rotated), once per workgroup.
  __device__ __forceinline__ void set_query(const float* qs) {
    const int h = n & 7;
    const float* qrow = qs + (h < G ? h : 0) * 128 + 32 * q;
    if constexpr (QF16) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          qh[4 * ks + s] = h < G ? pack2(qrow[kchan<BITS>(ks, 2 * s)], qrow[kchan<BITS>(ks, 2 * s + 1)]) : 0u;
    } else {
#pragma unroll
      for (int c = 0; c < 32; ++c) qv[c] = h < G ? qrow[c] : 0.f;
    }
  }

  // First token of half h of the wave's block (2 bits: both halves; 4 bits: its own half).
  __device__ __forceinline__ int tb(int h) const { return 64 * (NH == 1 ? par : h); }

  // 2^-e for the exponent e of a non-negative finite x (x * 2^-e in [0.5, 1)); 1 for x = 0.
  static __device__ __forceinline__ float pow2_normaliser(float x) {
    return x > 0.f ? __builtin_amdgcn_ldexpf(1.f, -__builtin_amdgcn_frexp_expf(x)) : 1.f;
  }

  // Record loads go through a buffer resource over this split's records: the lane offset is
  // a 32-bit register (fixed per lane plus the block's offset in the split), the per-load
  // displacement an immediate (no per-lane 64-bit address math). The range check of the
  // resource covers lane offset and displacement, so a fetch past the split's last block
  // returns zeros without touching memory.
  // The codes are read once: non-temporal loads (cache-policy bit "nt"); the statistics,
  // read by both waves of a block, keep the default policy.
  static constexpr int kNT = 2;
  // Paged caches: the resource spans the layer's page pool, a block's offset comes from the
  // block table, and a block past the split's end gets the pool's size (reads nothing).
  int blo_ = 0, nb_ = 0;
  uint32_t pool_bytes_ = 0;
  __device__ __forceinline__ uint32_t block_off(int rel) const {
    if (a.pg.table)
      return rel < nb_ ? (uint32_t)record_offset(a, blockIdx.z, blockIdx.y, blo_ + rel) : pool_bytes_;
    return (uint32_t)rel * a.lay.rec_bytes;
  }
  __device__ __forceinline__ void fetch(Buf& B, int rel) const {   // rel: block index in the split
    const uint32_t boff = block_off(rel);
    constexpr int soff = 0;
#pragma unroll
    for (int tt = 0; tt < 4 * NH; ++tt) {
      if constexpr (KW == 4) {
        const u4v v = __builtin_amdgcn_raw_buffer_load_b128(rs, boff + koff + 16 * tt * R, soff, kNT);
        B.kw[tt][0] = v.x; B.kw[tt][1] = v.y; B.kw[tt][2] = v.z; B.kw[tt][3] = v.w;
      } else {
        const u2v v = __builtin_amdgcn_raw_buffer_load_b64(rs, boff + koff + 16 * tt * R, soff, kNT);
        B.kw[tt][0] = v.x; B.kw[tt][1] = v.y;
      }
    }
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const uint32_t o = boff + voff + (uint32_t)h * (128 * RH) + 16 * ct * RH;
        if constexpr (VW == 2) {
          const u2v v = __builtin_amdgcn_raw_buffer_load_b64(rs, o, soff, kNT);
          B.vw[h][ct][0] = v.x; B.vw[h][ct][1] = v.y;
        } else {
          B.vw[h][ct][0] = __builtin_amdgcn_raw_buffer_load_b32(rs, o, soff, kNT);
        }
      }
#pragma unroll
    for (int k = 0; k < NMETA; ++k) {
      const u4v v = __builtin_amdgcn_raw_buffer_load_b128(
          rs, boff + a.lay.ks + 16u * (uint32_t)min(lane + 64 * k, META / 16 - 1), soff, 0);
      B.meta[k] = uint4{v.x, v.y, v.z, v.w};
    }
  }

  __device__ __forceinline__ void wave_sync() const {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // fp32 x -> the fp16 part of this lane's column: x rounded (high columns) or x minus that
  // rounding, rounded (low columns); two values per call.
  __device__ __forceinline__ uint32_t part2(float xa, float xb) const {
    const uint32_t c = pack2(xa, xb) & lo_mask;
    // x - c in one mixed-precision fma per value (fp32 x, fp16 c from the low / high half),
    // rounded once to fp16 into the low / high half; exact before the rounding since c is x
    // rounded to fp16, or 0
    // The result is a matrix-core operand. The compiler's hazard tracking does not see into
    // assembler statements, and a vector write needs two wait states before a matrix-core
    // read of the same register: the statement ends with them (s_nop 1).
    uint32_t r;
    asm("v_fma_mixlo_f16 %0, %1, 1.0, -%2 op_sel_hi:[0,0,1]" : "=v"(r) : "v"(xa), "v"(c));
    asm("v_fma_mixhi_f16 %0, %1, 1.0, -%2 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\ts_nop 1" : "+v"(r) : "v"(xb), "v"(c));
    return r;
  }

  __device__ __forceinline__ void process(const Buf& B) {
    // ---- stage the block statistics: [ks | vs | k1 | v1] as in the record; fp16 key
    // scales (lanes 0..15, channels 8*lane .. 8*lane+7) go in the slot-pair order (c, c+4)
#pragma unroll
    for (int k = 0; k < NMETA; ++k) {
      uint4 m = B.meta[k];
      if constexpr (QF16) {
        if (k == 0 && lane < 16)
          m = uint4{(m.x & 0xFFFFu) | (m.z << 16), (m.x >> 16) | (m.z & 0xFFFF0000u),
                    (m.y & 0xFFFFu) | (m.w << 16), (m.y >> 16) | (m.w & 0xFFFF0000u)};
      }
      if (lane + 64 * k < META / 16) reinterpret_cast<uint4*>(meta)[lane + 64 * k] = m;
    }
    wave_sync();
    const float* kS = reinterpret_cast<const float*>(meta);                 // RTN / KVARN
    const float* kM = kS + 128;
    const uint8_t* vbase = meta + (MODE == SYM ? 256 : 1024);
    const float* vS = reinterpret_cast<const float*>(vbase);
    const float* vM = vS + 128;
    const __half* vS16 = reinterpret_cast<const __half*>(vbase);
    const float* k1 = reinterpret_cast<const float*>(meta + 2048);
    const float* v1 = k1 + 128;

    // ---- Q' = q * s_c for this lane's column and channels, in operand slot order; bias
    // sum_c q_c m_c
    uint32_t qo[4][4];
    float bias = 0.f;
    float kscale = 1.f;         // Q' of this head was multiplied by kscale (a power of two)
    if constexpr (QF16) {
      // fp16 q times fp16 s: the high part is the product rounded once, the low part the
      // fused q*s - high rounded once
      const uint4* sp = reinterpret_cast<const uint4*>(meta) + 4 * q;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint4 s4 = sp[ks];
        const uint32_t sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const h2 qq = __builtin_bit_cast(h2, qh[4 * ks + s]), ss = __builtin_bit_cast(h2, sv[s]);
          const h2 c = __builtin_bit_cast(h2, __builtin_bit_cast(uint32_t, qq * ss) & lo_mask);
          qo[ks][s] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(qq, ss, -c));
        }
      }
    } else {
      // this lane's 32 channels of scale and offset in 16-byte reads, then used in slot order
      const int c0 = 32 * q;
      float ksv[32], kmv[32];
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const float4 s4 = *reinterpret_cast<const float4*>(kS + c0 + 4 * v);
        const float4 m4 = *reinterpret_cast<const float4*>(kM + c0 + 4 * v);
        ksv[4 * v] = s4.x; ksv[4 * v + 1] = s4.y; ksv[4 * v + 2] = s4.z; ksv[4 * v + 3] = s4.w;
        kmv[4 * v] = m4.x; kmv[4 * v + 1] = m4.y; kmv[4 * v + 2] = m4.z; kmv[4 * v + 3] = m4.w;
      }
      float qs[32], qmax = 0.f;
#pragma unroll
      for (int c = 0; c < 32; ++c) {
        qs[c] = qv[c] * ksv[c];
        qmax = fmaxf(qmax, fabsf(qs[c]));
      }
      kscale = pow2_normaliser(rows_max(qmax));   // per head: its 128 channels
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int ca = kchan<BITS>(ks, 2 * s), cb = kchan<BITS>(ks, 2 * s + 1);
          qo[ks][s] = part2(qs[ca] * kscale, qs[cb] * kscale);
          bias = fmaf(qv[ca], kmv[ca], fmaf(qv[cb], kmv[cb], bias));
        }
      bias = rows_sum(bias);
    }
    const h8 qb[4] = {make8(qo[0][0], qo[0][1], qo[0][2], qo[0][3]), make8(qo[1][0], qo[1][1], qo[1][2], qo[1][3]),
                      make8(qo[2][0], qo[2][1], qo[2][2], qo[2][3]), make8(qo[3][0], qo[3][1], qo[3][2], qo[3][3])};

    // ---- raw scores for tokens tb(h) + 16*tt + 4*q + e of each half h, head n & 7 (KVarN:
    // already in the log2 domain; otherwise the log2 scale is applied inside the exponent)
    constexpr bool PRESCALED = MODE == KVARN;
    const float kunscale = recip_pow2(kscale);   // exact: a power of two
    // KVarN: the log2 scale folded into the fma's constants (the per-token s1 multiplies after)
    const float ku = PRESCALED ? kunscale * a.scale_log2 : kunscale;
    const float kb = PRESCALED ? bias * a.scale_log2 : bias;
    float sc[NH][4][4];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        f4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          d = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes8<BITS, OFFK>(B.kw[4 * h + tt], ks), qb[ks], d, 0, 0, 0);
        float s1[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (MODE == KVARN) {
          const float4 t = *reinterpret_cast<const float4*>(k1 + tb(h) + 16 * tt + 4 * q);
          s1[0] = t.x; s1[1] = t.y; s1[2] = t.z; s1[3] = t.w;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float full = d[e] + dpp_f<0x128>(d[e]);   // high + low column
          if constexpr (MODE == KVARN) sc[h][tt][e] = fmaf(full, ku, kb) * s1[e];
          else if constexpr (MODE == RTN) sc[h][tt][e] = fmaf(full, kunscale, bias);
          else sc[h][tt][e] = full;
        }
      }

    // ---- online softmax for head n & 7 (16 scores per half and lane, 4 lanes per head and part)
    const float sl = PRESCALED ? 1.f : a.scale_log2;
    float mx = sc[0][0][0];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sc[h][tt][e]);
    mx = rows_max(mx);
    const float mnew = fmaxf(m_run, mx * sl);
    const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
    m_run = mnew;
    // p' = p * S_t (value scale per token; 1 for int4). The value codes enter centred, so
    // the part of sum_t p_t v_t that does not depend on the code is sum_t p_t (M_t + OFFV * S_t).
    float p[NH][4][4], lsum = 0.f, msum = 0.f;
    float S_t[NH][4][4], M_t[NH][4][4];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        if constexpr (MODE != SYM) {
          const float4 ts = *reinterpret_cast<const float4*>(vS + tb(h) + 16 * tt + 4 * q);
          const float4 tm = *reinterpret_cast<const float4*>(vM + tb(h) + 16 * tt + 4 * q);
          S_t[h][tt][0] = ts.x; S_t[h][tt][1] = ts.y; S_t[h][tt][2] = ts.z; S_t[h][tt][3] = ts.w;
          M_t[h][tt][0] = tm.x; M_t[h][tt][1] = tm.y; M_t[h][tt][2] = tm.z; M_t[h][tt][3] = tm.w;
        }
      }
    // P' = p S_t vscale, vscale a power of two putting the largest S_t of the wave's tokens
    // in [0.5, 1) (wave-uniform: every row holds all the tokens' scales after the row maximum)
    float vscale = 1.f;
    if constexpr (MODE != SYM) {
      float smax = 0.f;
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int e = 0; e < 4; ++e) smax = fmaxf(smax, S_t[h][tt][e]);
      vscale = pow2_normaliser(rows_max(smax));
    }
    // pv = p * vscale straight from the exponent (vscale = 2^ev); the sums are taken back to
    // p's units after the loop (powers of two: exact)
    const float vunscale = recip_pow2(vscale);   // exact: a power of two
    const float eshift = MODE == SYM ? -mnew : (float)(__builtin_amdgcn_frexp_expf(vscale) - 1) - mnew;
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(sc[h][tt][e], sl, eshift));
          lsum += pv;
          if constexpr (MODE != SYM) msum = fmaf(pv, fmaf((float)OFFV, S_t[h][tt][e], M_t[h][tt][e]), msum);
          p[h][tt][e] = MODE == SYM ? pv : pv * S_t[h][tt][e];
        }
      }
    if constexpr (MODE != SYM) lsum *= vunscale;
    l_run = fmaf(l_run, alpha, lsum);
    // RTN and KVarN: acc holds its sums in units of the current vscale; a new vscale rescales
    // it (exactly, a power of two) together with the softmax correction
    constexpr bool VSC = MODE == RTN || MODE == KVARN;
    const float arescale = VSC ? alpha * (vscale * recip_pow2(vsc)) : alpha;   // powers of two: exact
    if (__builtin_amdgcn_ballot_w64(arescale != 1.f)) {   // a running maximum or the value scale moved
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) acc[ct] *= arescale;
    }
    if constexpr (VSC) vsc = vscale;
    float g = 0.f;                     // KVarN: code-independent part, added before the channel s1
    if constexpr (MODE == RTN) {
      pm = fmaf(pm, alpha, msum * vunscale);
    } else if constexpr (MODE == KVARN) {
      g = rows_sum(msum);              // in units of vscale, as the accumulators
      g = lo_mask ? 0.f : g;           // once per head: on the high column
    }

    // ---- P' operand per half, this lane's part, slots in the order of the value chunks
    h8 b0[NH], b1[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      uint32_t po[2][4];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int pa = vpos<BITS>(ks, 2 * s), pbp = vpos<BITS>(ks, 2 * s + 1);
          po[ks][s] = part2(p[h][(pa >> 2) & 3][pa & 3], p[h][(pbp >> 2) & 3][pbp & 3]);
        }
      b0[h] = make8(po[0][0], po[0][1], po[0][2], po[0][3]);
      b1[h] = make8(po[1][0], po[1][1], po[1][2], po[1][3]);
    }

    // ---- O += V^T P' per 16-channel tile (every half of the wave's block, then the channel
    // scales)
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      f4 t = MODE == RTN ? acc[ct] : f4{g, g, g, g};   // KVarN: the code-independent part enters here
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        t = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes8<BITS, OFFV>(B.vw[h][ct], 0), b0[h], t, 0, 0, 0);
        t = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes8<BITS, OFFV>(B.vw[h][ct], 1), b1[h], t, 0, 0, 0);
      }
      if constexpr (MODE == RTN) {
        acc[ct] = t;
      } else if constexpr (MODE == KVARN) {
        const float4 v = *reinterpret_cast<const float4*>(v1 + 16 * ct + 4 * q);
        const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[ct][e] = fmaf(f[e], t[e], acc[ct][e]);
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(vS16 + 16 * ct + 4 * q);
        const h2 lo = __builtin_bit_cast(h2, v.x), hi = __builtin_bit_cast(h2, v.y);
        acc[ct][0] = fmaf((float)lo[0], t[0], acc[ct][0]);
        acc[ct][1] = fmaf((float)lo[1], t[1], acc[ct][1]);
        acc[ct][2] = fmaf((float)hi[0], t[2], acc[ct][2]);
        acc[ct][3] = fmaf((float)hi[1], t[3], acc[ct][3]);
      }
    }
    wave_sync();   // the statistics area is rewritten by the next block
  }

  // The split's records (blocks blo .. bhi-1) and the first block's loads, issued before the
  // query is ready (the kernel's set-up then overlaps them). Unconditional: a wave without
  // blocks reads past the resource's range, which returns zeros without a memory access.
  Buf A, Bb;
  int rel;
  __device__ __forceinline__ void begin(int blo, int bhi) {
    blo_ = blo;
    nb_ = max(bhi - blo, 0);
    if (a.pg.table) {
      pool_bytes_ = (uint32_t)a.pg.n_pages * (uint32_t)a.Hkv * a.lay.rec_bytes;
      rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.rec), (short)0, (int)pool_bytes_, 0x00020000);
    } else {
      const uint8_t* base = a.rec + record_offset(a, blockIdx.z, blockIdx.y, blo);
      rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, (int)(nb_ * a.lay.rec_bytes),
                                             0x00020000);
    }
    // this wave's blocks (relative to blo): 2 bits rel = w, w + 4, ...; 4 bits rel = w / 2,
    // w / 2 + 2, ... (its half of each)
    rel = NH == 2 ? w : w >> 1;
    fetch(A, rel);
  }

  __device__ __forceinline__ void run() {
    constexpr int step = NH == 2 ? 4 : 2;
    const int nb = nb_;
    if (rel >= nb) return;
    // the next block is fetched unconditionally (past the end it reads nothing), so the wait
    // before a block's first use covers that block's loads only; a fetch under a branch would
    // make the counter wait drain the prefetch as well
    while (true) {
      fetch(Bb, rel + step);
      process(A);
      rel += step;
      if (rel >= nb) break;
      fetch(A, rel + step);
      process(Bb);
      rel += step;
      if (rel >= nb) break;
    }
  }
};

// Tokens 64*w .. 64*w+63 of the fp16 tail (w = 0, 1) for the G heads: lane = token for the
// scores, lane = channel pair for P.V; the query and the probabilities are read from LDS
// as broadcasts. Writes (m, l, o) of this half into m_out[G], l_out[G], o_out[G][128]
// (KVarN: o in the rotated domain, like the block accumulators).
template <int MODE, int G>
__device__ __forceinline__ void tail_half_lds(const DecodeArgs& a, int w, int lane, bool active, const float* qs,
                                              float* pbuf, float* m_out, float* l_out, float* o_out) {
  const int n_valid = active ? min(64, seq_tail(a, blockIdx.z) - 64 * w) : 0;
  const __half* tk = a.tail + (size_t)(blockIdx.z * a.Hkv + blockIdx.y) * (2 * kT * kD);
  const __half* tv = tk + kT * kD;
  float sc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) sc[h] = 0.f;
  if (lane < n_valid) {
    const uint4* krow = reinterpret_cast<const uint4*>(tk + (size_t)(64 * w + lane) * kD);
#pragma unroll 2
    for (int c8 = 0; c8 < 16; ++c8) {
      const uint4 kv = krow[c8];
      const float2 k0 = __half22float2(__builtin_bit_cast(__half2, kv.x));
      const float2 k1 = __half22float2(__builtin_bit_cast(__half2, kv.y));
      const float2 k2 = __half22float2(__builtin_bit_cast(__half2, kv.z));
      const float2 k3 = __half22float2(__builtin_bit_cast(__half2, kv.w));
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float4 qa = *reinterpret_cast<const float4*>(qs + h * 128 + 8 * c8);
        const float4 qb = *reinterpret_cast<const float4*>(qs + h * 128 + 8 * c8 + 4);
        float t = sc[h];
        t = fmaf(k0.x, qa.x, t); t = fmaf(k0.y, qa.y, t); t = fmaf(k1.x, qa.z, t); t = fmaf(k1.y, qa.w, t);
        t = fmaf(k2.x, qb.x, t); t = fmaf(k2.y, qb.y, t); t = fmaf(k3.x, qb.z, t); t = fmaf(k3.y, qb.w, t);
        sc[h] = t;
      }
    }
  }
  if (n_valid == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (lane == 0) { m_out[h] = -INFINITY; l_out[h] = 0.f; }
      o_out[h * 128 + 2 * lane] = 0.f;
      o_out[h * 128 + 2 * lane + 1] = 0.f;
    }
    return;
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float sl = lane < n_valid ? sc[h] * a.scale_log2 : -INFINITY;
    const float m = wave_max(sl);
    const float p = lane < n_valid ? exp2f(sl - m) : 0.f;
    const float l = wave_sum(p);
    pbuf[h * 64 + lane] = p;
    if (lane == 0) { m_out[h] = m; l_out[h] = l; }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float o0[G], o1[G];
#pragma unroll
  for (int h = 0; h < G; ++h) { o0[h] = 0.f; o1[h] = 0.f; }
  const __half2* vcol = reinterpret_cast<const __half2*>(tv + (size_t)(64 * w) * kD) + lane;
  for (int t = 0; t < n_valid; ++t) {
    const float2 vv = __half22float2(vcol[(size_t)t * (kD / 2)]);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float pv = pbuf[h * 64 + t];
      o0[h] = fmaf(pv, vv.x, o0[h]);
      o1[h] = fmaf(pv, vv.y, o1[h]);
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if constexpr (MODE == KVARN) fwht_wave(o0[h], o1[h], lane);
    o_out[h * 128 + 2 * lane] = o0[h];
    o_out[h * 128 + 2 * lane + 1] = o1[h];
  }
}

template <int MODE, int BITS, int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void decode_mfma_kernel(DecodeArgs a) {
  __shared__ float s_q[G * 128];                 // query, original domain
  __shared__ float s_qr[G * 128];                // query for the blocks (KVarN: rotated)
  __shared__ __align__(16) uint8_t s_meta[4][3072];
  __shared__ float s_m[6][G], s_l[6][G];
  __shared__ float s_o[6][G * 128];

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  // the query's loads, then the first block's (their latencies overlap), then the query
  // into LDS: the compiler's wait for the query registers leaves the block's loads in flight
  constexpr int NQ = (G * 128 + kThreads - 1) / kThreads;
  const uint16_t* qsrc = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)b * a.Hq + (size_t)kvh * G) * 128;
  uint32_t qreg[NQ];   // fp16 bits (threads past the end reread the last element)
#pragma unroll
  for (int k = 0; k < NQ; ++k) qreg[k] = qsrc[min(tid + k * kThreads, G * 128 - 1)];
  MfmaDecoder<MODE, BITS, G> d(a, lane, w, s_meta[w]);
  const int blo = split * a.blocks_per_split;
  const int bhi = min(seq_nblk(a, b), blo + a.blocks_per_split);
  d.begin(blo, bhi);
  __builtin_amdgcn_sched_barrier(0);   // the query's first use stays behind the block's loads
#pragma unroll
  for (int k = 0; k < NQ; ++k) {
    const int i = tid + k * kThreads;
    if (i < G * 128) {
      const float v = __half2float(__ushort_as_half((unsigned short)qreg[k]));
      s_q[i] = v;
      s_qr[i] = v;
    }
  }
  __syncthreads();
  if constexpr (MODE == KVARN) {
    // rotate each head's query into the Hadamard domain of the keys (one wave per head)
    for (int h = w; h < G; h += 4) {
      float x = s_q[h * 128 + 2 * lane], y = s_q[h * 128 + 2 * lane + 1];
      fwht_wave(x, y, lane);
      s_qr[h * 128 + 2 * lane] = x;
      s_qr[h * 128 + 2 * lane + 1] = y;
    }
    __syncthreads();
  }

  d.set_query(s_qr);
  d.run();

  // ---- this wave's matrix-core state
  const int n = lane & 15, q = lane >> 4;
  float l = d.l_run;
  l = rows_sum(l);
  float pmw = d.pm;
  pmw = rows_sum(pmw);
  float o[8][4];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct)
#pragma unroll
    for (int e = 0; e < 4; ++e) o[ct][e] = d.acc[ct][e] + dpp_f<0x128>(d.acc[ct][e]);   // high + low column
  if constexpr (MODE == RTN || MODE == KVARN) {
    const float un = recip_pow2(d.vsc);   // the accumulators' value scale, a power of two (exact)
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) o[ct][e] *= un;
  }
  if (n < G) {
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) s_o[w][n * 128 + 16 * ct + 4 * q + e] = o[ct][e] + pmw;
    if (q == 0) { s_m[w][n] = d.m_run; s_l[w][n] = l; }
  }
  // ---- the fp16 tail (waves 0 and 1; it belongs to the last split)
  if (w < 2) {
    const bool active = split == a.splits - 1 && 64 * w < seq_tail(a, b);
    tail_half_lds<MODE, G>(a, w, lane, active, s_q, reinterpret_cast<float*>(s_meta[w]), s_m[4 + w], s_l[4 + w],
                           s_o[4 + w]);
  }
  __syncthreads();
  for (int i = tid; i < G * 128; i += kThreads) {
    const int h = i >> 7;
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < 6; ++s) M = fmaxf(M, s_m[s][h]);
    float o = 0.f;
#pragma unroll
    for (int s = 0; s < 6; ++s)
      if (s_m[s][h] != -INFINITY) o = fmaf(exp2f(s_m[s][h] - M), s_o[s][i], o);
    s_o[0][i] = o;
  }
  __syncthreads();
  if constexpr (MODE == KVARN) {
    // back from the Hadamard domain: one wave per head, the 128-point transform in registers
    // (the same butterflies in the same order as the query's, then the 1/sqrt(128) scale)
    for (int h = w; h < G; h += 4) {
      float x = s_o[0][h * 128 + 2 * lane], y = s_o[0][h * 128 + 2 * lane + 1];
      fwht_wave(x, y, lane);
      s_o[0][h * 128 + 2 * lane] = x;
      s_o[0][h * 128 + 2 * lane + 1] = y;
    }
    __syncthreads();
  }
  for (int i = tid; i < G * 128; i += kThreads) {
    const int h = i >> 7, c = i & 127;
    const size_t row = (size_t)b * a.Hq + (size_t)kvh * G + h;
    const float o = s_o[0][i];
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < 6; ++s) M = fmaxf(M, s_m[s][h]);
    float L = 0.f;
#pragma unroll
    for (int s = 0; s < 6; ++s)
      if (s_m[s][h] != -INFINITY) L = fmaf(exp2f(s_m[s][h] - M), s_l[s][h], L);
    if (a.part_slots == 1) {
      a.out[row * kD + c] = o / L;
    } else {
      float* part = a.part + (row * a.part_slots + split) * kPartStride;
      part[2 + c] = o;
      if (c == 0) { part[0] = M; part[1] = L; }
    }
  }
}

template <int MODE, int BITS, int G>
hipError_t launch_m(const DecodeArgs& a, int batch, hipStream_t s) {
  hipLaunchKernelGGL((decode_mfma_kernel<MODE, BITS, G>), dim3(a.splits, a.Hkv, batch), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int MODE, int BITS>
hipError_t launch_mg(int group, const DecodeArgs& a, int batch, hipStream_t s) {
  switch (group) {
    case 1: return launch_m<MODE, BITS, 1>(a, batch, s);
    case 2: return launch_m<MODE, BITS, 2>(a, batch, s);
    case 4: return launch_m<MODE, BITS, 4>(a, batch, s);
    case 8: return launch_m<MODE, BITS, 8>(a, batch, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool mfma_supported(int mode, int bits, int rope, int k_out) {
  return !rope && k_out == 0 && (bits == 2 || bits == 4) && (mode == RTN || mode == KVARN || mode == SYM);
}

hipError_t launch_decode_mfma(int mode, int bits, int group, const DecodeArgs& a, int batch, hipStream_t s) {
  switch (mode * 8 + bits) {
    case RTN * 8 + 2: return launch_mg<RTN, 2>(group, a, batch, s);
    case RTN * 8 + 4: return launch_mg<RTN, 4>(group, a, batch, s);
    case KVARN * 8 + 2: return launch_mg<KVARN, 2>(group, a, batch, s);
    case KVARN * 8 + 4: return launch_mg<KVARN, 4>(group, a, batch, s);
    case SYM * 8 + 4: return launch_mg<SYM, 4>(group, a, batch, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
