// Internal declarations shared by the host API and the HIP kernels of libkvq.
// Layout of a block record and the argument blocks the launches take.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int kT = 128;          // tokens per quantization block
constexpr int kD = 128;          // head dimension
constexpr int kMaxOut = 8;       // outliers per vector
constexpr int kPartStride = 2 + kD;  // one split partial: m, l, o[128]
constexpr int kMaxSplits = 64;       // decode splits per (sequence, kv head)
constexpr int kSideChunk = 64;       // fp16-part tokens per workgroup (four waves of 16 tokens)
// Device codebook slot per (layer, kv head, K/V): entries C[0..15], then the NUQ decision
// thresholds tau[0..14] (see kvq_api.hip).
constexpr int kCbStride = 32;
// NUQ code table: u in [-1, 1] falls in bucket floor((u + 1) * 512) of 1024 (1024: u = 1);
// an entry holds (number of decision thresholds below every u that can land in the bucket,
// the one threshold that may still split it, or +inf). Entry 0 with count -1: the codebook
// has two thresholds too close for the table and the kernel counts thresholds instead.
constexpr int kNuqBuckets = 1024;
constexpr int kNuqLutStride = 1032;   // entries per (layer, kv head, K/V) slot (1025 used)

enum Mode { RTN = 0, NUQ = 1, KVARN = 2, SYM = 3, ASYM = 4 };

// Byte offsets of the segments of one block record (all 16-byte aligned).
struct RecordLayout {
  uint32_t kc, vc, ks, vs, k1, v1;
  uint32_t ko_val, ko_ptr, ko_idx, vo_val, vo_ptr, vo_idx;
  uint32_t rec_bytes;   // padded to 256
  uint32_t payload;     // sum of segment sizes
};

RecordLayout make_layout(int mode, int bits, int k_out);

// Paged caches: each layer's records live in a pool of pages, page p holding one 128-token
// block of every kv head ([n_pages][Hkv] records); a caller-owned device table maps block j
// of sequence b to its page. Sequences hold their own token counts (ragged batches).
constexpr int kMaxPagedBatch = 64;
struct PagedSeq {
  const int32_t* table;       // [batch][table_stride] page of each block (device), or null
  int table_stride, n_pages;
  int len[kMaxPagedBatch];    // tokens of each sequence before this call (append) / held (decode)
  int n_new[kMaxPagedBatch];  // tokens this call appends to each sequence (append)
};

// Page of block blk of sequence b, clamped into the pool: a bad table entry gives wrong
// results, never an access outside the pool.
// The table is read through the constant address space: the index is uniform across the
// workgroup, so the read is one scalar load (a vector load would make the next wait on the
// vector memory counter drain every record prefetch in flight).
__device__ __forceinline__ int page_of(const PagedSeq& p, int b, int blk) {
  typedef const __attribute__((address_space(4))) int32_t* ConstI32;
  const int v = ((ConstI32)p.table)[(size_t)b * p.table_stride + blk];
  return v < 0 ? 0 : (v >= p.n_pages ? p.n_pages - 1 : v);
}

// fp16 rows of one (layer, sequence, kv head): K [tail_rows][128] then V [tail_rows][128];
// rows 0 .. sink-1 hold the attention-sink tokens, row sink + (u mod ring_rows) holds body
// token u (the tokens after the sink, numbered from 0) while it is not quantized.
struct QuantArgs {
  RecordLayout lay;
  int k_out, varn_iters;
  const __half* k_in;    // [B][Hkv][n_new][128]
  const __half* v_in;
  int n_new, blk0;       // blk0: body block of the launch's first block
  int u_old;             // body tokens appended before this call: u < u_old are in the ring
  int in_row0;           // input row of body token u (u >= u_old) is u + in_row0
  int sink, ring_rows, tail_rows;
  int Hkv, max_blocks;
  uint8_t* rec;          // records of the layer, [B][Hkv][max_blocks] (paged: the page pool)
  const __half* tail;    // fp16 rows of the layer, [B][Hkv][2][tail_rows][128]
  const float* cb;       // codebooks of the layer, [Hkv][2][kCbStride]
  const float2* nuq_lut; // NUQ code tables of the layer, [Hkv][2][kNuqLutStride] (NUQ only)
  PagedSeq pg;           // paged caches: blk0, u_old and in_row0 follow from pg.len[b]
};

// Staging of new fp16 rows: input rows [0, n_sink) to tail rows sink_row0 + i (sink
// tokens), input rows [ring_src0, ring_src0 + ring_count) to body tokens ring_u0 + i.
struct TailArgs {
  const __half* k_in;
  const __half* v_in;
  int n_new, Hkv;
  int n_sink, sink_row0;
  int ring_src0, ring_count, ring_u0;
  int sink, ring_rows, tail_rows;
  __half* tail;
  PagedSeq pg;           // paged caches: the ranges follow from pg.len[b] and pg.n_new[b]
};

struct DecodeArgs {
  RecordLayout lay;
  int k_out;
  const uint8_t* rec;
  const __half* tail;
  const float* cb;
  const float* rope_base;   // [max_blocks + 1][64][2]: cos, sin of (sink + 128 * block) * theta_i
  const float* rope_off;    // [64][128][2]: cos, sin of j * theta_i (pair-major); then theta_i[64]
  const __half* q;          // [B][Hq][128]
  float* part;              // [B][Hq][splits][2 + 128]
  float* out;               // [B][Hq][128]
  int Hkv, Hq, max_blocks;
  int nblk, tail_n, splits, blocks_per_split;
  int part_slots;           // split partials per (sequence, query head); 1: write out directly
  float scale_log2;         // softmax scale * log2(e)
  int wave_lds;             // dynamic LDS bytes per wave for outlier staging (0 without outliers)
  // fp16 part outside the blocks (sink tokens and the body tokens not yet quantized),
  // decoded by its own kernel when a sink or a window is configured (tail_n is then 0):
  // side_chunk tokens per workgroup, the partial of workgroup z in slot side_slot + z
  // (side_slot < 0: one workgroup writes the output itself)
  int sink_n, fp16_u0, fp16_n, ring_rows, tail_rows, side_slot, side_chunk;
  PagedSeq pg;              // paged caches: per-sequence lengths and the block table
};

// Full blocks and fp16 tail tokens of sequence b.
__device__ __forceinline__ int seq_nblk(const DecodeArgs& a, int b) { return a.pg.table ? a.pg.len[b] >> 7 : a.nblk; }
__device__ __forceinline__ int seq_tail(const DecodeArgs& a, int b) { return a.pg.table ? a.pg.len[b] & 127 : a.tail_n; }
// Byte offset of the record of block blk of (sequence b, kv head h) from a.rec.
__device__ __forceinline__ size_t record_offset(const DecodeArgs& a, int b, int h, int blk) {
  if (a.pg.table) return ((size_t)page_of(a.pg, b, blk) * a.Hkv + h) * a.lay.rec_bytes;
  return (((size_t)b * a.Hkv + h) * a.max_blocks + blk) * a.lay.rec_bytes;
}

// Error diagnostic over quantized blocks block0 .. block0 + n_blocks - 1 of every (sequence,
// kv head): inputs [B][Hkv][n_blocks * 128][128] fp16, out [B][Hkv][n_blocks * 128][4] fp64.
struct DiagArgs {
  RecordLayout lay;
  int k_out;
  const uint8_t* rec;       // records of the layer
  const float* cb;          // codebooks of the layer, [Hkv][2][kCbStride]
  const __half* k_in;
  const __half* v_in;
  int block0, n_blocks, Hkv, max_blocks;
  double* out;
};

// Weighted k-means codebook builder state (device memory, in the caller's workspace).
struct CodebookState {
  double centres[16];
  int converged;            // set once an iteration changes no assignment
  int iter;                 // update steps taken
};
struct CodebookArgs {
  const float* act;         // [n] normalised activations in [-1, 1]
  const float* weight;      // [n] weights, or null for unit weights
  int64_t n, per_range;     // samples; samples per assign workgroup
  int n_ranges;             // assign workgroups
  uint8_t* assign;          // [n] current centre of every sample
  double* partials;         // [n_ranges][2 K]: sum F, sum F a per centre
  int* changes;             // [n_ranges] changed assignments
  CodebookState* state;
  float* out;               // [K] the codebook
  int32_t* iters_out;       // update steps (or null)
};
constexpr int kCodebookMaxRanges = 1024;
hipError_t launch_codebook_build(int bits, const CodebookArgs& a, int max_iters, hipStream_t s);

hipError_t launch_quantize(int mode, int bits, const QuantArgs& a, int n_blocks, int batch,
                           hipStream_t s);
hipError_t launch_tail(const TailArgs& a, int batch, hipStream_t s);
hipError_t launch_decode(int mode, int bits, int group, int rope, const DecodeArgs& a, int batch,
                         hipStream_t s);
// Matrix-core decode: caches without pre-RoPE keys and outliers, 2 or 4 bits, RTN / KVarN / int4.
bool mfma_supported(int mode, int bits, int rope, int k_out);
hipError_t launch_decode_mfma(int mode, int bits, int group, const DecodeArgs& a, int batch, hipStream_t s);
// Table decode: pre-RoPE keys, one query head per kv head, 2 or 3 bits, RTN / NUQ.
bool tab_supported(int mode, int bits, int group, int rope);
hipError_t launch_decode_tab(int mode, int bits, bool matrix_cores, const DecodeArgs& a, int batch, hipStream_t s);
hipError_t launch_combine(const float* part, float* out, int Hq, int splits, int batch, hipStream_t s);
// fp16 sink and window tokens of every (sequence, kv head): partial slot side_slot (or out).
hipError_t launch_decode_fp16(int group, int rope, const DecodeArgs& a, int batch, int n_side, hipStream_t s);
hipError_t launch_diag(int mode, int bits, const DiagArgs& a, int batch, hipStream_t s);

}  // namespace kvq
