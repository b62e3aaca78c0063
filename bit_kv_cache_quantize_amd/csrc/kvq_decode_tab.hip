// Split-K decode attention for caches with pre-RoPE keys and one query head per kv
// head (the LLaMA-7B shapes), 2- or 3-bit RTN or NUQ codes, with or without outliers.
//
// Same computation as the other decode kernels ("KVQuant reading notes", Algorithm 1
// attention part, 1.3 and 3.2 for RoPE, 3.4 for the outliers): softmax(scale * q .
// RoPE(k_hat_n, n)) weighted sum of v_hat_n over every cached token.
//
// What differs is how a key reaches its score. Rotate the query back by the block's base
// angle n0 * theta_i (pair i = channels 2i, 2i+1) and fold in the pair's dequantization;
// the pair's contribution to the score of in-block token j is then
//     cos(j theta_i) * U_i(a, b) + sin(j theta_i) * W_i(a, b),
//     U_i = al_i k_x(a) + be_i k_y(b),   W_i = be_i k_x(a) - al_i k_y(b),
// where (a, b) are the pair's two codes and (al_i, be_i) the rotated query pair. U and W
// depend only on the block and the two codes, so the two waves that share a block
// tabulate them in LDS for every code combination (16 entries per pair at 2 bits, 64 at
// 3 bits), indexed by the pair's bits as they lie in the packed row. A token then costs,
// per channel pair, the index extraction, one 8-byte LDS read and two fma; cos(j theta_i)
// and sin(j theta_i) are per-lane registers (each lane keeps one in-block offset j).
//
// Values: lane = channel pair of a 64-token half-row. The codes of two adjacent tokens
// index a constant LDS table of their code values (RTN codes, NUQ codebook entries), and
// their weights p_t * S_t (S_t the token's value scale) are broadcast from LDS; the
// code-independent part sum_t p_t M_t is added once per head.
//
// Outliers replace the dense value: each CSR (keys) / CSC (values) entry adds
// (fp16 value - dense value) times the entry's weight. A token's lane walks its own CSR
// row (its key entries, in channel order) after the table part of its score; a channel's
// lane walks its own CSC column (value entries, in token order). Every sum therefore has
// a fixed order: two runs give bitwise equal results.
//
// Work decomposition: one workgroup of two waves = one split of one (sequence, kv head);
// wave h takes the 64-token half h of every block of the split. Two barriers per block
// (tables built, tables consumed) synchronize only these two waves. Each load of the next
// block is issued as soon as the registers it refills are dead, so it is in flight during
// the rest of the current block.
#include "kvq_decode_common.h"

namespace kvq {
namespace {

// 1 / x for x a power of two (normal), exactly: 2^(1 - e) with x = 0.5 * 2^e.
__device__ __forceinline__ float recip_pow2(float x) {
  return __builtin_amdgcn_ldexpf(1.f, 1 - __builtin_amdgcn_frexp_expf(x));
}

using namespace dec;

constexpr float kInv2Pi = 0.15915494309189535f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// BIG: the outlier segments of a block exceed one 16-byte chunk per thread; the extra chunks
// are loaded in a loop (kept out of the common instantiation: a load loop under a branch
// makes the counter wait at its join drain the key and value prefetches).
// MC: matrix cores allowed (false: the 2-bit RTN values use the LDS table of code pairs too,
// the configuration a caller selects to compare the two).
template <int MODE, int BITS, bool BIG, bool MC>
struct TabDecoder {
  static constexpr int R = 16 * BITS;                 // key row bytes
  static constexpr int RH = R / 2;                    // value half-row bytes
  static constexpr int PT = BITS == 3 ? 64 : 16;      // table entries per channel pair
  // Pair tables: entry idx of pair i at byte 8 * (PS * i + idx), (U, W) as 8 bytes, with
  // idx = a | b << 2 at 2 bits (x code a, y code b) and n | h << 4 at 3 bits (n: the pair's
  // nibble of the crumb plane, the two low bits of a and of b; h: its crumb of the bit plane,
  // bit 2 of a and of b). The tables are PT + 2 entries apart: the 16-byte pad staggers the
  // LDS bank groups of consecutive pairs, so that the lanes of a build step (one pair each)
  // do not all write the same banks. The lookups keep their immediate offsets (no extra
  // instruction). (A 3-bit table spans 512 bytes, two entries per 8-byte bank: random
  // lookups conflict; U and W as separate 256-byte arrays of 4-byte entries measured more
  // conflicts, not fewer.)
  static constexpr int PS = PT + 2;
  static constexpr int KWD = R / 4;                   // dwords of a key row
  // 2-bit RTN values go through the matrix cores (codes are small integers, exact in
  // fp16); NUQ codebook values and 3-bit codes use the LDS table of code pairs.
  static constexpr bool MV = MC && MODE == RTN && BITS == 2;

  // Loads of the next block, each issued as soon as the registers it refills are dead.
  struct Meta {           // issued after the table build
    float4 kst;           // (scale_x, scale_y, offset_x, offset_y) of pair ib
    float2 rb;            // (cos, sin) of the block base angle for pair ib
    u32x4 ob;             // outlier segment chunk j (j = thread of the workgroup)
  };
  struct Keys {           // issued after the scores
    uint32_t kw[KWD];     // key row of token j
  };
  struct Vals {           // issued after the values
    uint32_t vw[KWD];     // value half-rows of channels ch0, ch1
    float2 tst;           // value (S, M) of token j
  };

  struct Shared {
    float2* tab;          // the pair tables [64][PS]
    float2* qb;           // rotated query pairs [64] (al, be)
    float* kd0;           // dense key value of code 0 per channel [128] (outlier corrections)
    const float2* vlut;   // value code pairs [PT]
    float* pS;            // this wave's p * S per token of the half [64]
    float* p;             // this wave's p per token [64]
    float* M;             // this wave's value offset M per token [64]
    uint8_t* blob;        // outlier staging
    const float* trev;    // theta_i / (2 pi) [64]
    const float* cbk;     // key codebook [16] (NUQ)
    const float* cbv;     // value codebook [16] (NUQ)
    _Float16* wt;         // matrix-core values: this wave's weights p*S as fp16 high and low
                          // parts in operand order [2][16 steps][4 slots]
    const _Float16* zero; // 64 zero fp16 (operand rows 2 and 3)
    float* Sv;            // this wave's value scale S per token [64] (outlier corrections)
    float* pref;          // this wave's prefix sums of the value-outlier corrections [128k + 1]
    float4* kent;         // 2 bits: this wave's key-outlier entries, folded (see key_outliers) [128k]
  };

  const DecodeArgs& a;
  const Shared S;
  const int lane, par, j, ib, hb;
  int ob_bytes, ob_chunks;
  int m_ord;              // running maximum of the scores, as its integer image (ord_image)
  float l_run, pm, acc0, acc1;
  f4 dacc[2];             // matrix-core accumulators of the two channel groups
  float vsc;              // the power of two dacc is scaled by (wave-uniform)
  float wpre;             // power of two undoing the code scale of this token's operand slot
  float qx_, qy_;         // the query pair ib (scale folded), read once

  __device__ TabDecoder(const DecodeArgs& args, const Shared& sh, int lane_, int w_)
      : a(args), S(sh), lane(lane_), par(w_), j(64 * w_ + lane_), ib((64 * w_ + lane_) >> 1), hb(lane_ & 1) {
    m_ord = ord_image(__float_as_int(-INFINITY));
    const __half2 q2 = reinterpret_cast<const __half2*>(a.q + ((size_t)blockIdx.z * a.Hq + blockIdx.y) * 128)[ib];
    qx_ = __low2float(q2) * a.scale_log2;
    qy_ = __high2float(q2) * a.scale_log2;
    if constexpr (MV) {
      dacc[0] = f4{0.f, 0.f, 0.f, 0.f};
      dacc[1] = f4{0.f, 0.f, 0.f, 0.f};
      vsc = 1.f;
      wpre = __builtin_amdgcn_ldexpf(1.f, 19 - 2 * code_slot(half_row_token(lane_) & 7));
    }
    l_run = 0.f;
    pm = 0.f;
    acc0 = 0.f;
    acc1 = 0.f;
    ob_bytes = 0;
    ob_chunks = 0;
    if (a.k_out > 0) {
      ob_bytes = (int)(a.lay.vo_idx + 128u * a.k_out - a.lay.ko_val);
      ob_chunks = (ob_bytes + 15) / 16;
    }
  }

  // The two value channels of this lane: pairs (2*lane, 2*lane+1) for the table path; for
  // the matrix-core path the lane's column in each of the two 64-channel groups.
  __device__ __forceinline__ int ch0() const { return MV ? lane : 2 * lane; }
  __device__ __forceinline__ int ch1() const { return MV ? 64 + lane : 2 * lane + 1; }

  __device__ __forceinline__ const uint8_t* record(int blk) const {
    return a.rec + record_offset(a, blockIdx.z, blockIdx.y, blk);
  }

  // Record loads go through a buffer resource over this split's records (blocks blo ..
  // bhi-1): 32-bit lane offsets, and the resource's range check turns a load of the block
  // after the split's last into zeros that touch no memory. Every load of the next block is
  // therefore issued unconditionally: a load under a branch makes the memory-counter waits
  // after the join drain every load in flight.
  // Paged caches: the resource spans the layer's page pool and each block's offset comes
  // from the block table; a block past the split's end gets the pool's size as offset.
  __amdgpu_buffer_rsrc_t rsb;
  int blo_, bhi_;
  uint32_t pool_bytes_;
  __device__ __forceinline__ void bind(int blo, int bhi) {
    blo_ = blo;
    bhi_ = bhi;
    if (a.pg.table) {
      pool_bytes_ = (uint32_t)a.pg.n_pages * (uint32_t)a.Hkv * a.lay.rec_bytes;
      rsb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.rec), (short)0, (int)pool_bytes_, 0x00020000);
    } else {
      rsb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(record(blo)), (short)0,
                                              (int)(max(bhi - blo, 0) * a.lay.rec_bytes), 0x00020000);
    }
  }
  __device__ __forceinline__ uint32_t boff(int blk) const {
    if (a.pg.table)
      return blk < bhi_ ? (uint32_t)record_offset(a, blockIdx.z, blockIdx.y, blk) : pool_bytes_;
    return (uint32_t)(blk - blo_) * a.lay.rec_bytes;
  }
  static constexpr int kNT = 2;   // cache policy "nt": the code rows are read once
  // loads of one block: fetch_meta (4), fetch_keys, fetch_vals (2 + the code rows)
  static constexpr int row_loads(int nbytes) { return nbytes % 16 == 0 ? nbytes / 16 : nbytes / 8; }
  static constexpr int kBlockLoads = 4 + row_loads(R) + 2 + (MV ? 2 * row_loads(RH) : row_loads(R));

  template <int NBYTES>
  __device__ __forceinline__ void load_row_b(uint32_t* w, uint32_t off) const {
    static_assert(NBYTES % 8 == 0, "row bytes");
    if constexpr (NBYTES % 16 == 0) {
#pragma unroll
      for (int k = 0; k < NBYTES / 16; ++k) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsb, off + 16 * k, 0, kNT);
        w[4 * k] = v.x; w[4 * k + 1] = v.y; w[4 * k + 2] = v.z; w[4 * k + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int k = 0; k < NBYTES / 8; ++k) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rsb, off + 8 * k, 0, kNT);
        w[2 * k] = v.x; w[2 * k + 1] = v.y;
      }
    }
  }

  __device__ __forceinline__ float ldf(uint32_t off) const {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsb, off, 0, 0));
  }

  __device__ __forceinline__ void fetch_meta(Meta& Mt, int blk) const {
    const uint32_t o = boff(blk);
    // each pair is converted to float as a whole: with the two halves bit-cast one at a
    // time, this compiler narrows the 8-byte load to 4 bytes and uses them for both halves
    const float2 s2 = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rsb, o + a.lay.ks + 8u * ib, 0, 0));
    const float2 m2 =
        __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rsb, o + a.lay.ks + 512u + 8u * ib, 0, 0));
    if constexpr (MODE == NUQ) Mt.kst = make_float4(m2.x, m2.y, s2.x, s2.y);   // (h, h, z, z)   RTN s, m / NUQ z, h
    else Mt.kst = make_float4(s2.x, s2.y, m2.x, m2.y);                          // (s, s, m, m)
    Mt.rb = reinterpret_cast<const float2*>(a.rope_base)[(size_t)blk * 64 + ib];   // rows 0 .. nblk exist
    // without outliers the offset lies past the range: zeros, no memory access
    const uint32_t oo = a.k_out > 0 ? o + a.lay.ko_val + 16u * (uint32_t)min(j, ob_chunks - 1) : 0xFFFFFFF0u;
    Mt.ob = __builtin_amdgcn_raw_buffer_load_b128(rsb, oo, 0, 0);
  }

  __device__ __forceinline__ void fetch_keys(Keys& K, int blk) const {
    load_row_b<R>(K.kw, boff(blk) + a.lay.kc + (uint32_t)j * R);
  }

  // The statistics are loaded before the code rows: they are staged at the top of the next
  // block, and the in-order load counter then leaves the rows in flight.
  __device__ __forceinline__ void fetch_vals(Vals& V, int blk) const {
    const uint32_t o = boff(blk);
    if constexpr (MODE == NUQ) {
      V.tst.x = ldf(o + a.lay.vs + 4u * (128 + j));   // h
      V.tst.y = ldf(o + a.lay.vs + 4u * j);           // z
    } else {
      V.tst.x = ldf(o + a.lay.vs + 4u * j);
      V.tst.y = ldf(o + a.lay.vs + 4u * (128 + j));
    }
    if constexpr (MV) {
      load_row_b<RH>(V.vw, o + a.lay.vc + (uint32_t)(par * 128 + ch0()) * RH);
      load_row_b<RH>(V.vw + KWD / 2, o + a.lay.vc + (uint32_t)(par * 128 + ch1()) * RH);
    } else {
      load_row_b<R>(V.vw, o + a.lay.vc + (uint32_t)par * (128 * RH) + (uint32_t)lane * R);
    }
  }

  __device__ __forceinline__ float kcode(int c, uint32_t code) const {
    if constexpr (MODE == NUQ) return S.cbk[code];
    else return (float)code;
  }

  // Half of pair ib's table (the other lane of the pair writes the rest), the pair's rotated
  // query and its channel statistics. Lane hb writes the entries whose y code has its top
  // bit (bit 1 at 2 bits, bit 2 at 3 bits) equal to hb, so that the two lanes' stores land
  // in different banks.
  __device__ __forceinline__ void build(const Meta& B) const {
    const float qx = qx_, qy = qy_;
    const float al = fmaf(qx, B.rb.x, qy * B.rb.y);
    const float be = fmaf(qy, B.rb.x, -qx * B.rb.y);
    if (hb == 0) S.qb[ib] = make_float2(al, be);
    if (a.k_out > 0) S.kd0[2 * ib + hb] = hb ? fmaf(kcode(1, 0u), B.kst.y, B.kst.w) : fmaf(kcode(0, 0u), B.kst.x, B.kst.z);
    constexpr int NA = 1 << BITS;          // codes of the x channel
    constexpr int NB = BITS == 3 ? 4 : 2;  // codes of the y channel covered by this lane
    // U(a, b) = al kx(a) + be ky(b), W(a, b) = be kx(a) - al ky(b): one fma per value
    float kx[NA], Ay[NB], By[NB];
#pragma unroll
    for (int c = 0; c < NA; ++c) kx[c] = fmaf(kcode(0, c), B.kst.x, B.kst.z);
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      const int y = NB * hb + c;
      const float ky = fmaf(kcode(1, y), B.kst.y, B.kst.w);
      Ay[c] = be * ky;
      By[c] = -al * ky;
    }
    uint8_t* tab = reinterpret_cast<uint8_t*>(S.tab) + ib * PS * 8;
    // the lane's entries idx = hb * PT/2 + ee; the bits that name the lane's half do not
    // enter ca (x code) or cbl (index of the y code in this lane's range)
    auto entry = [&](int ee) {
      int ca, cbl;
      if constexpr (BITS == 3) {   // idx = lo2(a) | lo2(b) << 2 | hi(a) << 4 | hi(b) << 5
        ca = (ee & 3) | (((ee >> 4) & 1) << 2);
        cbl = (ee >> 2) & 3;
      } else {                     // idx = a | b << 2
        ca = ee & 3;
        cbl = (ee >> 2) & 1;
      }
      return make_float2(fmaf(al, kx[ca], Ay[cbl]), fmaf(be, kx[ca], By[cbl]));
    };
#pragma unroll
    for (int e = 0; e < PT / 2; e += 2) {
      const float2 v0 = entry(e), v1 = entry(e + 1);
      *reinterpret_cast<float4*>(tab + 8 * (hb * (PT / 2) + e)) = make_float4(v0.x, v0.y, v1.x, v1.y);
    }
  }

  // Table index of pair i of a packed row held in w[].
  __device__ __forceinline__ uint32_t pair_index(const uint32_t* wd, int i, int nrow) const {
    // nrow: codes in the row (128 keys, 64 values)
    const uint32_t nib = __builtin_amdgcn_ubfe(wd[i >> 3], 4 * (i & 7), 4);
    if constexpr (BITS == 3) {
      const uint32_t hi = __builtin_amdgcn_ubfe(wd[nrow / 16 + (i >> 4)], 2 * (i & 15), 2);
      return nib | (hi << 4);
    } else {
      return nib;
    }
  }

  // A 3-bit row (NC dwords of the crumb plane: pair i's two low-bit crumbs are nibble i;
  // NC / 2 dwords of the bit plane: pair i's two high bits are crumb i) spread once so that
  // the table offset 8 * (n | h << 4) of any pair costs a byte permute and a shift:
  //   ev[d], od[d]: the even / odd nibbles of crumb dword d, times 16, one per byte;
  //   hm[e][m]:     crumb m of every byte of bit-plane dword e, in bits 0-1 of that byte.
  // Pair i's nibble is byte ((i & 7) >> 1) of ev / od[i >> 3], its crumb is byte
  // ((i & 15) >> 2) of hm[i >> 4][i & 3]; the permute puts them in bytes 0 and 1 (zeros in
  // bytes 2 and 3): 16 n + 256 h, twice the offset. (Offsets without the shift, 8 n + 256 h,
  // put both high bits above the LDS bank bits and measured slower: more bank conflicts.)
  // The empty asm keeps the compiler from folding the shared shifts back into per-pair
  // operations.
  template <int NC>
  struct Spread3 {
    uint32_t ev[NC], od[NC], hm[NC / 2][4];
    __device__ __forceinline__ void make(const uint32_t* w) {
#pragma unroll
      for (int d = 0; d < NC; ++d) {
        ev[d] = (w[d] << 4) & 0xF0F0F0F0u;
        od[d] = w[d] & 0xF0F0F0F0u;
        asm volatile("" : "+v"(ev[d]), "+v"(od[d]));
      }
#pragma unroll
      for (int e = 0; e < NC / 2; ++e) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          hm[e][m] = (w[NC + e] >> (2 * m)) & 0x03030303u;
          asm volatile("" : "+v"(hm[e][m]));
        }
      }
    }
    __device__ __forceinline__ uint32_t off(int i) const {
      const uint32_t E = (i & 1) ? od[i >> 3] : ev[i >> 3];
      const uint32_t sel = 0x0C0C0000u | ((4u + ((i & 15) >> 2)) << 8) | (uint32_t)((i & 7) >> 1);
      return __builtin_amdgcn_perm(hm[i >> 4][i & 3], E, sel) >> 1;
    }
  };

  __device__ __forceinline__ void wave_sync() const {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  __device__ __forceinline__ float m_run() const { return __int_as_float(ord_image(m_ord)); }

  // Online-softmax update with this lane's log2-domain score; returns p.
  // The exponent arguments are <= 0 (differences to the running maximum): the hardware
  // exp2 is used directly (results below 2^-126 are flushed to zero; they are below the
  // rounding of any sum they enter). The running sums are rescaled only when the (wave-
  // uniform) maximum moved: otherwise the factor is exactly 1.
  __device__ __forceinline__ float softmax_step(float sl) {
    // the maximum on integer images: scalar operations (scores are never NaN)
    const int mi = max(m_ord, wave_max_ord(sl));
    const float mnew = __int_as_float(ord_image(mi));
    const float p = __builtin_amdgcn_exp2f(sl - mnew);
    if (mi != m_ord) {
      const float alpha = __builtin_amdgcn_exp2f(m_run() - mnew);
      l_run = fmaf(l_run, alpha, p);
      pm *= alpha;
      acc0 *= alpha;
      acc1 *= alpha;
      if constexpr (MV) {
        dacc[0] *= alpha;
        dacc[1] *= alpha;
      }
      m_ord = mi;
    } else {
      l_run += p;
    }
    return p;
  }

  // Outlier segments of block blk into the LDS staging (before the barrier that precedes
  // their use): the chunk held in registers, the rest (many outliers per vector) loaded here.
  __device__ __forceinline__ void stage_blob(const Meta& Mt, int blk) const {
    u32x4* dst = reinterpret_cast<u32x4*>(S.blob);
    dst[min(j, ob_chunks - 1)] = Mt.ob;   // lanes past the end rewrite the last chunk (same value)
    if constexpr (BIG) {
      for (int k = j + 128; k < ob_chunks; k += 128)
        dst[k] = __builtin_amdgcn_raw_buffer_load_b128(rsb, boff(blk) + a.lay.ko_val + 16u * k, 0, 0);
    }
  }

  // Score of token j over the whole row (table, rotated query, statistics and outlier
  // staging of the block complete).
  __device__ __forceinline__ float scores(const Keys& B, const float (&rc)[64], const float (&rs)[64]) const {

    // ---- scores: two fma per channel pair on the tabulated (U, W). Software-pipelined in
    // chunks of CH pairs: the table reads of chunk c+1 are issued before the fma of chunk c
    // (scheduling barriers keep that order), so 2*CH LDS reads are in flight at a time.
    constexpr int CH = 8;
    float sc0 = 0.f, sc1 = 0.f;
    float2 uw[2][CH];
    // 2 bits: the byte offsets (index * 8) of all pairs come from two masked shifts per
    // code dword, even nibbles in one word and odd nibbles in the other, one byte each;
    // a pair's offset is then a single byte extraction. The empty asm keeps the compiler
    // from folding the shared shifts back into two operations per pair.
    // 3 bits: the same for both planes (Spread3), a pair's offset is a byte permute and a
    // shift.
    uint32_t ev[8], od[8];
    Spread3<8> sp;
    if constexpr (BITS == 2) {
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        ev[d] = (B.kw[d] << 3) & 0x78787878u;
        od[d] = (B.kw[d] >> 1) & 0x78787878u;
        asm volatile("" : "+v"(ev[d]), "+v"(od[d]));
      }
    } else {
      sp.make(B.kw);
    }
    auto kread = [&](int c, float2 (&dst)[CH]) {
#pragma unroll
      for (int k = 0; k < CH; ++k) {
        const int i = c * CH + k;
        const uint8_t* t = reinterpret_cast<const uint8_t*>(S.tab) + (size_t)i * PS * 8;
        if constexpr (BITS == 2) {
          const uint32_t w = (i & 1) ? od[i >> 3] : ev[i >> 3];
          dst[k] = *reinterpret_cast<const float2*>(t + __builtin_amdgcn_ubfe(w, 8 * ((i & 7) >> 1), 8));
        } else {
          dst[k] = *reinterpret_cast<const float2*>(t + sp.off(i));
        }
      }
    };
    kread(0, uw[0]);
#pragma unroll
    for (int c = 0; c < 64 / CH; ++c) {
      if (c + 1 < 64 / CH) kread(c + 1, uw[(c + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < CH; ++k) {
        sc0 = fmaf(rc[c * CH + k], uw[c & 1][k].x, sc0);
        sc1 = fmaf(rs[c * CH + k], uw[c & 1][k].y, sc1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    float sc = sc0 + sc1;

    // key outliers: this token's CSR row, in channel order. Entry (j, c) adds
    // (fp16 value - dense value of code 0) times the query coefficient of channel c at
    // in-block offset j: cos(j theta_i) al + sin(j theta_i) be (x channel) or
    // cos(j theta_i) be - sin(j theta_i) al (y channel) of pair i = c / 2.
    if (a.k_out > 0) sc += key_outliers();
    return sc;
  }

  // The key-outlier correction of token j. A row holds as many entries as the token has
  // outlier channels, so the wave runs its loop as often as its longest row. 2 bits: first
  // every entry of this half's rows is folded once, spread over the lanes in CSR order, into
  // (x qa, x qb, theta_i / 2 pi) with x = fp16 value - dense value and (qa, qb) = (al, be)
  // or (be, -al); a row step is then one 16-byte read, the angle and two fma.
  __device__ __forceinline__ float key_outliers() const {
    const uint16_t* kptr = reinterpret_cast<const uint16_t*>(S.blob + (a.lay.ko_ptr - a.lay.ko_val));
    const uint8_t* kidx = S.blob + (a.lay.ko_idx - a.lay.ko_val);
    const __half* kval = reinterpret_cast<const __half*>(S.blob);
    float corr = 0.f;
    if constexpr (BITS == 2) {
      const int E0 = kptr[64 * par], E1 = kptr[64 * par + 64];
      for (int e = E0 + lane; e < E1; e += 64) {
        const int c = kidx[e], i = c >> 1;
        const float2 q2 = S.qb[i];
        const float x = __half2float(kval[e]) - S.kd0[c];
        S.kent[e - E0] = (c & 1) ? make_float4(x * q2.y, -(x * q2.x), S.trev[i], 0.f)
                                 : make_float4(x * q2.x, x * q2.y, S.trev[i], 0.f);
      }
      wave_sync();
      const int e1 = kptr[j + 1] - E0;
      for (int e = kptr[j] - E0; e < e1; ++e) {
        const float4 t = S.kent[e];
        const float ang = (float)j * t.z;
        corr = fmaf(__builtin_amdgcn_cosf(ang), t.x, fmaf(__builtin_amdgcn_sinf(ang), t.y, corr));
      }
    } else {
      const int e1 = kptr[j + 1];
      for (int e = kptr[j]; e < e1; ++e) {
        const int c = kidx[e], i = c >> 1;
        const float ang = (float)j * S.trev[i];
        const float cj = __builtin_amdgcn_cosf(ang), sj = __builtin_amdgcn_sinf(ang);
        const float2 q2 = S.qb[i];
        const float coef = (c & 1) ? fmaf(cj, q2.y, -sj * q2.x) : fmaf(cj, q2.x, sj * q2.y);
        corr = fmaf(__half2float(kval[e]) - S.kd0[c], coef, corr);
      }
    }
    return corr;
  }

  // Values of this half (channels ch0, ch1) weighted by the probabilities of its
  // tokens; p is this lane's (token j's) probability.
  __device__ __forceinline__ void values(const Vals& V, float p) {
    pm = fmaf(p, V.tst.y, pm);                 // sum_t p_t M_t (code-independent part)
    const float ps = p * V.tst.x;
    S.pS[lane] = ps;
    S.p[lane] = p;
    S.M[lane] = V.tst.y;
    if (a.k_out > 0) S.Sv[lane] = V.tst.x;
    if constexpr (MV) {
      // the weight as fp16 high and low parts, at the operand slot of token j's position,
      // after a power of two that puts the half block's largest value scale in [0.5, 1) and
      // the slot's power of two (at most 2^15: within fp16's range; both exact and undone at
      // the end); the accumulators follow the current power of two
      // (value scales are >= 0; vs = 2^-e for the largest one m * 2^e, m in [0.5, 1): for a
      // normal maximum of biased exponent E, the float of biased exponent 253 - E)
      const int sb = wave_max_bits_nonneg(V.tst.x);
      const int E = (sb >> 23) & 0xFF;
      float vs;
      if (sb <= 0) vs = 1.f;
      else if (E >= 1 && E <= 252) vs = __int_as_float((253 - E) << 23);
      else vs = __builtin_amdgcn_ldexpf(1.f, -__builtin_amdgcn_frexp_expf(__int_as_float(sb)));
      if (vs != vsc) {
        const float f = vs * recip_pow2(vsc);   // powers of two: exact
        dacc[0] *= f;
        dacc[1] *= f;
        vsc = vs;
      }
      const float psv = ps * vs * wpre;
      const _Float16 hi = (_Float16)psv;
      const _Float16 lo = (_Float16)(psv - (float)hi);
      const int pos = half_row_token(lane);   // the position map is its own inverse
      S.wt[mv_slot(pos)] = hi;
      S.wt[64 + mv_slot(pos)] = lo;
    }
    wave_sync();
    if constexpr (MV) {
      // Values on the matrix cores (4x4x4 blocks): block b, column i = channel 64 g + 4 b + i;
      // operand rows 0 and 1 = the weights' high and low fp16 parts, rows 2 and 3 zero; 16
      // steps of 4 positions cover the half-row. A code enters as the fp16 subnormal
      // code * 2^(2 s - 24) (code_pair_f16: the code bits left in place at slot s) and its
      // weight was multiplied by 2^(19 - 2 s): every product is weight * code * 2^-5,
      // exactly, with no constant part to subtract.
      const int i = lane & 3;
      const _Float16* arow = i == 0 ? S.wt : (i == 1 ? S.wt + 64 : S.zero);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t x[2][3];   // per group: the code dword shifted left by 4, as is, right by 6
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const uint32_t d = V.vw[4 * g + q];
          x[g][0] = d << 4;
          x[g][1] = d;
          x[g][2] = d >> 6;
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int st = 4 * q + t;
          const h4 A = *reinterpret_cast<const h4*>(arow + 4 * st);
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const h4 B = __builtin_bit_cast(h4, u32x2{code_pair_f16(x[g], 2 * t), code_pair_f16(x[g], 2 * t + 1)});
            dacc[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(A, B, dacc[g], 0, 0, 0);
          }
        }
      }
    } else {
      // ---- P.V over the 64 tokens of this half, channels 2*lane and 2*lane+1
      // (pipelined like the scores: reads of chunk c+1 before the fma of chunk c)
      constexpr int CV = 2;
      float o0 = 0.f, o1 = 0.f;
      float2 vb[2][CV][3];
      // 3 bits: the two half-rows spread once (Spread3). The weights of the two token pairs
      // of a chunk (tokens t .. t + 3 of the half-row order) come in one 16-byte read.
      static_assert(CV == 2, "one weight read per two token pairs");
      Spread3<4> s0, s1;
      if constexpr (BITS == 3) {
        s0.make(V.vw);
        s1.make(V.vw + KWD / 2);
      }
      const uint8_t* vl = reinterpret_cast<const uint8_t*>(S.vlut);
      auto vread = [&](int c, float2 (&dst)[CV][3]) {
        const float4 w4 = *reinterpret_cast<const float4*>(S.pS + half_row_token(2 * CV * c));
        dst[0][0] = make_float2(w4.x, w4.y);
        dst[1][0] = make_float2(w4.z, w4.w);
#pragma unroll
        for (int k = 0; k < CV; ++k) {
          const int pp = c * CV + k;   // positions 2pp, 2pp+1: tokens half_row_token(2pp) + 0, 1
          if constexpr (BITS == 3) {
            dst[k][1] = *reinterpret_cast<const float2*>(vl + s0.off(pp));
            dst[k][2] = *reinterpret_cast<const float2*>(vl + s1.off(pp));
          } else {
            dst[k][1] = *reinterpret_cast<const float2*>(vl + 8u * pair_index(V.vw, pp, 64));
            dst[k][2] = *reinterpret_cast<const float2*>(vl + 8u * pair_index(V.vw + KWD / 2, pp, 64));
          }
        }
      };
      vread(0, vb[0]);
#pragma unroll
      for (int c = 0; c < 32 / CV; ++c) {
        if (c + 1 < 32 / CV) vread(c + 1, vb[(c + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < CV; ++k) {
          const float2 ps = vb[c & 1][k][0], v0 = vb[c & 1][k][1], v1 = vb[c & 1][k][2];
          o0 = fmaf(ps.x, v0.x, fmaf(ps.y, v0.y, o0));
          o1 = fmaf(ps.x, v1.x, fmaf(ps.y, v1.y, o1));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      acc0 += o0;
      acc1 += o1;
    }
    // ---- value outliers: entry e of the CSC list (token t, fp16 value x) adds
    // p_t (x - dense value of code 0) to its channel, for the tokens of this half. The
    // entries are spread over the lanes (2k per lane, in list order), their corrections
    // summed into a prefix array; a channel's correction is the difference of the prefix
    // at its two column pointers. No loop depends on a column's length, and every sum has
    // a fixed order.
    if (a.k_out > 0) {
      value_prefix();
      const uint16_t* vptr = reinterpret_cast<const uint16_t*>(S.blob + (a.lay.vo_ptr - a.lay.ko_val));
      acc0 += S.pref[vptr[ch0() + 1]] - S.pref[vptr[ch0()]];
      acc1 += S.pref[vptr[ch1() + 1]] - S.pref[vptr[ch1()]];
      wave_sync();   // the prefix array is rewritten by the next block
    }
  }

  // Exclusive prefix sums of the value-outlier corrections of this half into S.pref[0 .. E]
  // (E = 128 k entries; S.pref[E] = the total).
  __device__ __forceinline__ void value_prefix() const {
    const uint8_t* vidx = S.blob + (a.lay.vo_idx - a.lay.ko_val);
    const __half* vval = reinterpret_cast<const __half*>(S.blob + (a.lay.vo_val - a.lay.ko_val));
    const float v0 = MODE == NUQ ? S.cbv[0] : 0.f;
    // correction of an entry at token t of the block (0 unless t lies in this half)
    auto corr = [&](int tok, __half x) {
      const int t = tok - 64 * par;
      const bool mine = t >= 0 && t < 64;
      const int tt = mine ? t : 0;
      const float c = S.p[tt] * (__half2float(x) - fmaf(v0, S.Sv[tt], S.M[tt]));
      return mine ? c : 0.f;
    };
    const int per = 2 * a.k_out;   // entries per lane
    const int e0 = lane * per;
    if (per == 2) {
      // one outlier per vector: the lane's two entries come in one read each for the
      // token indices and the values, and stay in registers
      const uint32_t ti = *reinterpret_cast<const uint16_t*>(vidx + e0);
      const __half2 xv = *reinterpret_cast<const __half2*>(vval + e0);
      const float c0 = corr((int)(ti & 0xFF), __low2half(xv));
      const float c1 = corr((int)(ti >> 8), __high2half(xv));
      const float tot = c0 + c1;
      const float run = wave_scan(tot) - tot;
      *reinterpret_cast<float2*>(S.pref + e0) = make_float2(run, run + c0);
      if (lane == 63) S.pref[128] = run + tot;
    } else {
      float tot = 0.f;
      for (int i = 0; i < per; ++i) {
        const int e = e0 + i;
        const float c = corr((int)vidx[e], vval[e]);
        S.pref[e] = c;
        tot += c;
      }
      float run = wave_scan(tot) - tot;
      for (int i = 0; i < per; ++i) {
        const int e = e0 + i;
        const float c = S.pref[e];
        S.pref[e] = run;
        run += c;
      }
      if (lane == 63) S.pref[64 * per] = run;
    }
    wave_sync();
  }

  // Inclusive prefix sum over the 64 lanes (shifts within 16-lane rows, then the row totals
  // broadcast to the following rows).
  static __device__ __forceinline__ float wave_scan(float x) {
    int v = __float_as_int(x);
    v = __float_as_int(__int_as_float(v) + __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false)));
    v = __float_as_int(__int_as_float(v) + __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false)));
    v = __float_as_int(__int_as_float(v) + __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false)));
    v = __float_as_int(__int_as_float(v) + __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false)));
    v = __float_as_int(__int_as_float(v) + __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false)));
    v = __float_as_int(__int_as_float(v) + __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false)));
    return __int_as_float(v);
  }

  // Operand slot (4 * step + k) of half-row position pos in the matrix-core value product:
  // step s takes positions 16q + m + {0, 8, 1, 9} (q = s / 4, m = 2 (s % 4)), the order in
  // which two conversions of one code dword produce them.
  static __device__ __forceinline__ int mv_slot(int pos) {
    return 16 * (pos >> 4) + 4 * ((pos & 7) >> 1) + 2 * (pos & 1) + ((pos >> 3) & 1);
  }

  // Slot s (bits 2s, 2s + 1 of each 16-bit half) at which the code of position p of a
  // 16-code dword (and of p + 8) is read: positions 0, 1 from the dword shifted left by 4,
  // 2 .. 4 from the dword itself, 5 .. 7 from the dword shifted right by 6.
  static constexpr __host__ __device__ int code_slot(int p) { return p < 2 ? p + 2 : (p < 5 ? p : p - 3); }

  // Positions p and p + 8 of a 16-code dword as two fp16 subnormals code * 2^(2 s - 24)
  // (exact; s = code_slot(p)): only the code bits at slot s are kept, one and per pair.
  // x: the dword shifted left by 4, as is, right by 6.
  static __device__ __forceinline__ uint32_t code_pair_f16(const uint32_t (&x)[3], int p) {
    const int s = code_slot(p);
    const uint32_t src = x[p < 2 ? 0 : (p < 5 ? 1 : 2)];
    return src & (s == 2 ? 0x00300030u : (s == 3 ? 0x00C000C0u : 0x03000300u));
  }

  // Tokens 64*par .. 64*par+63 of the fp16 tail (position 128*nblk + j), waves 0 and 1.
  // Runs once per (sequence, kv head): the per-offset angles come from the table in memory
  // (the main loop's registers for them are dead here).
  __device__ __forceinline__ void tail_half(const float2* qt) {
    const int n_valid = min(64, seq_tail(a, blockIdx.z) - 64 * par);
    const __half* tk = a.tail + (size_t)(blockIdx.z * a.Hkv + blockIdx.y) * (2 * kT * kD);
    const __half* tv = tk + kT * kD;
    const bool valid = lane < n_valid;
    float sc = 0.f;
    const uint4* krow = reinterpret_cast<const uint4*>(tk + (size_t)j * kD);
    const float2* off = reinterpret_cast<const float2*>(a.rope_off) + j;   // pair-major: [i][j]
#pragma unroll 1
    for (int i0 = 0; i0 < 64; i0 += 4) {
      const uint4 kv = valid ? krow[i0 / 4] : make_uint4(0u, 0u, 0u, 0u);
      const uint32_t kd[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int i = i0 + k;
        const float2 kk = __half22float2(__builtin_bit_cast(__half2, kd[k]));
        const float2 q2 = qt[i];
        const float2 cs = off[(size_t)i * 128];
        const float U = fmaf(kk.x, q2.x, kk.y * q2.y);
        const float W = fmaf(kk.x, q2.y, -kk.y * q2.x);
        sc = fmaf(cs.x, U, fmaf(cs.y, W, sc));
      }
    }
    const float p = softmax_step(valid ? sc : -INFINITY);
    S.p[lane] = p;
    wave_sync();
    float o0 = 0.f, o1 = 0.f;
    if constexpr (MV) {
      const __half* vrow = tv + (size_t)(64 * par) * kD;
      for (int t = 0; t < n_valid; ++t) {
        const float pv = S.p[t];
        o0 = fmaf(pv, __half2float(vrow[(size_t)t * kD + ch0()]), o0);
        o1 = fmaf(pv, __half2float(vrow[(size_t)t * kD + ch1()]), o1);
      }
    } else {
      const __half2* vcol = reinterpret_cast<const __half2*>(tv + (size_t)(64 * par) * kD) + lane;
      for (int t = 0; t < n_valid; ++t) {
        const float2 vv = __half22float2(vcol[(size_t)t * (kD / 2)]);
        const float pv = S.p[t];
        o0 = fmaf(pv, vv.x, o0);
        o1 = fmaf(pv, vv.y, o1);
      }
    }
    acc0 += o0;
    acc1 += o1;
    wave_sync();
  }
};

constexpr int kTabThreads = 128;

template <int MODE, int BITS, bool BIG, bool MC>
__global__ __launch_bounds__(kTabThreads) __attribute__((amdgpu_waves_per_eu(2))) void decode_tab_kernel(DecodeArgs a) {
  using Dec = TabDecoder<MODE, BITS, BIG, MC>;
  constexpr int PT = Dec::PT;
  extern __shared__ __align__(16) uint8_t s_dyn[];
  __shared__ __align__(16) float2 s_tab[64 * Dec::PS];
  __shared__ __align__(16) float2 s_vlut[PT];
  __shared__ __align__(16) float2 s_qb[64];
  __shared__ __align__(16) float s_kd0[128];
  __shared__ float s_trev[64];
  __shared__ float s_cb[32];
  // [wave][p * S, p][token]
  __shared__ __align__(16) float s_pps[2][2][64];
  __shared__ __align__(16) float s_M[2][64];
  __shared__ __align__(16) _Float16 s_wt[Dec::MV ? 2 : 1][Dec::MV ? 128 : 8];
  __shared__ __align__(16) _Float16 s_zero[Dec::MV ? 64 : 8];
  __shared__ __align__(16) float s_S[2][64];
  __shared__ float s_m[2], s_l[2];

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  if (tid < 64) s_trev[tid] = a.rope_off[128 * 64 * 2 + tid] * kInv2Pi;
  if (MODE == NUQ && tid < 32) s_cb[tid] = a.cb[(kvh * 2 + (tid >> 4)) * kCbStride + (tid & 15)];
  if (Dec::MV && tid < 64) s_zero[tid] = (_Float16)0.f;
  __syncthreads();
  if (tid < PT) {
    // code values of two adjacent value tokens, in the same index order as the key tables
    int ca, cb2;
    if constexpr (BITS == 3) {
      ca = (tid & 3) | (((tid >> 4) & 1) << 2);
      cb2 = ((tid >> 2) & 3) | (((tid >> 5) & 1) << 2);
    } else {
      ca = tid & 3;
      cb2 = (tid >> 2) & 3;
    }
    s_vlut[tid] = MODE == NUQ ? make_float2(s_cb[16 + ca], s_cb[16 + cb2]) : make_float2((float)ca, (float)cb2);
  }

  typename Dec::Shared sh;
  sh.tab = s_tab;
  sh.qb = s_qb;
  sh.kd0 = s_kd0;
  sh.vlut = s_vlut;
  sh.pS = s_pps[w][0];
  sh.p = s_pps[w][1];
  sh.M = s_M[w];
  sh.blob = s_dyn;
  sh.trev = s_trev;
  sh.cbk = s_cb;
  sh.cbv = s_cb + 16;
  sh.wt = s_wt[Dec::MV ? w : 0];
  sh.zero = s_zero;
  sh.Sv = s_S[w];
  {
    // dynamic LDS: the outlier segments, then one prefix array per wave
    const int blob16 = a.k_out > 0 ? ((int)(a.lay.vo_idx + 128u * a.k_out - a.lay.ko_val) + 15) & ~15 : 0;
    const int pref16 = ((128 * a.k_out + 1) * 4 + 15) & ~15;
    sh.pref = reinterpret_cast<float*>(s_dyn + blob16 + w * pref16);
    // 2 bits: then one array of folded key-outlier entries per wave
    sh.kent = reinterpret_cast<float4*>(s_dyn + blob16 + 2 * pref16 + w * (128 * 16 * a.k_out));
  }
  Dec d(a, sh, lane, w);

  float rc[64], rs[64];
  {
    const float2* off = reinterpret_cast<const float2*>(a.rope_off) + d.j;   // pair-major: [i][j]
#pragma unroll
    for (int i = 0; i < 64; ++i) { const float2 v = off[i * 128]; rc[i] = v.x; rs[i] = v.y; }
  }
  __builtin_amdgcn_sched_barrier(0);   // the angle loads are issued before the block's

  const int blo = split * a.blocks_per_split;
  const int bhi = min(seq_nblk(a, b), blo + a.blocks_per_split);
  d.bind(blo, bhi);
  typename Dec::Meta Mt;
  typename Dec::Keys Kc;
  typename Dec::Vals V;
  // unconditional: an empty split's loads lie past the range (rope_base row blo <= nblk)
  d.fetch_meta(Mt, blo);
  d.fetch_keys(Kc, blo);
  d.fetch_vals(V, blo);
  // Wait for the angle loads (the memory counter counts in order) but not for the first
  // block's: the two latencies overlap, and the main loop starts with only the block loads
  // in flight, the same state as at the end of every iteration, so that the memory-counter
  // waits inside the loop count exactly those loads.
  static_assert(Dec::kBlockLoads < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | Dec::kBlockLoads);   // vmcnt(kBlockLoads)
  __syncthreads();   // the value table is complete
  for (int blk = blo; blk < bhi; ++blk) {
    // the loads of the next block are unconditional (past the split's end they read
    // nothing), so that no branch makes the memory-counter waits conservative
    const int nxt = blk + 1;
    if (a.k_out > 0) d.stage_blob(Mt, blk);
    d.build(Mt);
    d.fetch_meta(Mt, nxt);
    __syncthreads();   // tables, rotated query, statistics and outlier staging complete
    const float sc = d.scores(Kc, rc, rs);
    d.fetch_keys(Kc, nxt);
    const float p = d.softmax_step(sc);
    d.values(V, p);
    d.fetch_vals(V, nxt);
    __syncthreads();   // every read of the tables and of the staging done
  }

  // ---- the fp16 tail (it belongs to the last split)
  if (split == a.splits - 1 && seq_tail(a, b) > 0) {
    float2* qt = s_qb;
    if (d.hb == 0) {
      // query pair ib rotated back by the tail block's base angle
      const float2 rb = reinterpret_cast<const float2*>(a.rope_base)[(size_t)seq_nblk(a, b) * 64 + d.ib];
      const float qx = d.qx_, qy = d.qy_;
      qt[d.ib] = make_float2(fmaf(qx, rb.x, qy * rb.y), fmaf(qy, rb.x, -qx * rb.y));
    }
    __syncthreads();
    if (64 * d.par < seq_tail(a, b)) d.tail_half(qt);
  }

  // ---- merge the two wave states
  float* s_o = reinterpret_cast<float*>(&s_tab[0]);   // [2][128], the tables are no longer read
  __syncthreads();
  {
    const float l = wave_sum(d.l_run);
    const float pmw = wave_sum(d.pm);
    if (lane == 0) { s_m[w] = d.m_run(); s_l[w] = l; }
    float o0 = d.acc0 + pmw, o1 = d.acc1 + pmw;
    if constexpr (Dec::MV) {
      const float un = 32.f * recip_pow2(d.vsc);   // 2^5 undoes the operand scaling; powers of two: exact
      o0 += (d.dacc[0][0] + d.dacc[0][1]) * un;
      o1 += (d.dacc[1][0] + d.dacc[1][1]) * un;
    }
    s_o[w * 128 + d.ch0()] = o0;
    s_o[w * 128 + d.ch1()] = o1;
  }
  __syncthreads();
  {
    const int c = tid;
    const float M = fmaxf(s_m[0], s_m[1]);
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int ww = 0; ww < 2; ++ww) {
      if (s_m[ww] == -INFINITY) continue;
      const float sw = exp2f(s_m[ww] - M);
      o = fmaf(sw, s_o[ww * 128 + c], o);
      L = fmaf(sw, s_l[ww], L);
    }
    const size_t row = (size_t)b * a.Hq + kvh;
    if (a.part_slots == 1) {
      a.out[row * kD + c] = o / L;
    } else {
      float* part = a.part + (row * a.part_slots + split) * kPartStride;
      part[2 + c] = o;
      if (c == 0) { part[0] = M; part[1] = L; }
    }
  }
}

template <int MODE, int BITS, bool MC = true>
hipError_t launch_t(const DecodeArgs& a, int batch, hipStream_t s) {
  const bool big = a.k_out > 0 && (a.lay.vo_idx + 128u * a.k_out - a.lay.ko_val + 15u) / 16u > (unsigned)kTabThreads;
  if (big)
    hipLaunchKernelGGL((decode_tab_kernel<MODE, BITS, true, MC>), dim3(a.splits, a.Hkv, batch), dim3(kTabThreads),
                       (size_t)a.wave_lds, s, a);   // outlier staging
  else
    hipLaunchKernelGGL((decode_tab_kernel<MODE, BITS, false, MC>), dim3(a.splits, a.Hkv, batch), dim3(kTabThreads),
                       (size_t)a.wave_lds, s, a);
  return hipGetLastError();
}

}  // namespace

bool tab_supported(int mode, int bits, int group, int rope) {
  return rope && group == 1 && (bits == 2 || bits == 3) && (mode == RTN || mode == NUQ);
}

hipError_t launch_decode_tab(int mode, int bits, bool matrix_cores, const DecodeArgs& a, int batch, hipStream_t s) {
  switch (mode * 8 + bits) {
    case RTN * 8 + 2: return matrix_cores ? launch_t<RTN, 2>(a, batch, s) : launch_t<RTN, 2, false>(a, batch, s);
    case RTN * 8 + 3: return launch_t<RTN, 3>(a, batch, s);
    case NUQ * 8 + 2: return launch_t<NUQ, 2>(a, batch, s);
    case NUQ * 8 + 3: return launch_t<NUQ, 3>(a, batch, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
