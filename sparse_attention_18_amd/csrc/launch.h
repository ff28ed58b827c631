// Internal launch interface between the C-ABI layer (abi.cpp) and the
// kernel translation units.  Every launcher takes validated arguments and
// enqueues on `stream`; it returns the hipGetLastError() of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

// Sequence layout shared by all stages (device arrays + host-validated bounds).
struct SeqLayout {
  const int32_t *q_offsets;
  const int32_t *kv_offsets;
  const int32_t *q_pos0;
  int32_t batch;
  int64_t total_q, total_kv, max_q_len, max_kv_len;
};

// Paged key / KV caches: key position s of sequence b is row
// table[b * max_blocks + s / block_size] * block_size + s % block_size.
struct PagedKV {
  const int32_t *table;   // nullptr: rows are packed, kv_offsets[b] + s
  int32_t block_shift;    // log2(block_size), block_size a power of two >= 64
  int32_t max_blocks;     // row stride of the table
  int32_t num_blocks;     // num_blocks << block_shift < 2^31
};

// Fused decode top-k: per (row, 1024-key chunk) slot the decode indexer
// leaves a table of the chunk's nonzero score bins, its length, and the
// chunk's keys grouped by bin (instead of the scores); the select kernel
// reads them.  Rows of at most kFuseMaxLen keys (the select's position
// bitmaps live in LDS).
constexpr int kFuseChunk = 1024;       // keys per chunk (one decode indexer workgroup)
constexpr int kFuseBins = 4096;        // top 12 bits of the order-preserving key
constexpr int kFuseTabCap = kFuseChunk;   // a chunk has at most this many nonzero bins
constexpr int64_t kFuseMaxLen = 1 << 18;
struct FuseArgs {
  uint32_t *tab;    // [rows * nchunk][kFuseTabCap]; nullptr: no fused selection
  uint32_t *nz;     // [rows * nchunk]: table entries (nonzero bins) of the chunk
  uint32_t *list;   // [rows * nchunk][kFuseChunk]
  int32_t nchunk;   // slots per row: ceil(max_kv_len / kFuseChunk)
};

struct IndexerArgs {
  SeqLayout seq;
  PagedKV pg;
  const uint8_t *q_fp8;
  const float *q_scale;
  const float *w;
  const uint8_t *k_fp8;
  const float *k_scale;
  float *scores;
  int64_t ld;
  int32_t idx_heads, idx_dim;
  FuseArgs fuse;    // decode kernel only: also leave the fused top-k's data
};

struct TopkArgs {
  SeqLayout seq;
  const float *scores;
  int64_t ld;
  int32_t *idx;
  int32_t k;
  void *workspace;
  size_t workspace_bytes;
  int32_t seg_len, nseg;   // few-rows path: scores per segment, segments per row (set by the launcher)
  FuseArgs fuse;           // launch_topk_fused: what the decode indexer left
};

struct AttnArgs {
  SeqLayout seq;
  PagedKV pg;
  const uint16_t *q;
  const uint16_t *kv;
  const int32_t *idx;
  uint16_t *out;
  float *lse;
  int32_t heads, d_latent, d_rope, k;
  float scale;
  void *workspace;
  size_t workspace_bytes;
  int32_t nsplit;    // workgroups per token (set by the launcher)
};

// Prefill-mode attention: per-head keys (a 128-wide part and a 64-wide
// rotary part shared by the heads) and per-head 128-wide values, the
// selected positions applied as a mask over dense key tiles.
struct MhaArgs {
  SeqLayout seq;
  const uint16_t *q;        // [total_q, heads, 192]
  const uint16_t *k_nope;   // [total_kv, heads, 128]
  const uint16_t *k_rope;   // [total_kv, 64]
  const uint16_t *v;        // [total_kv, heads, 128]
  const int32_t *idx;       // [total_q, k]
  uint16_t *out;            // [total_q, heads, 128]
  float *lse;               // [total_q, heads] or nullptr
  int32_t heads, k;
  float scale;
  void *workspace;
  size_t workspace_bytes;
};
constexpr int64_t kMhaMaxKvLen = 131072;   // a row's mask is built in LDS

// Indexer alignment loss: idx == nullptr selects the dense warm-up form (all
// causal keys); grad rows are ld_grad apart (dense: by key position; sparse:
// by entry of idx).
struct AlignArgs {
  SeqLayout seq;
  const uint16_t *q;
  const uint16_t *kv;
  const float *lse;
  const float *scores;
  int64_t ld_scores;
  const int32_t *idx;
  float *loss;
  float *grad;
  int64_t ld_grad;
  int32_t heads, d_latent, d_rope, k;
  float scale;
};

// Indexer backward: grad rows are ld_grad apart (sparse: by entry of idx;
// dense, idx == nullptr: by key position); dq and dw are written, dk is
// added to.
struct IndexerBwdArgs {
  SeqLayout seq;
  const uint8_t *q_fp8;
  const float *q_scale;
  const float *w;
  const uint8_t *k_fp8;
  const float *k_scale;
  const int32_t *idx;
  const float *grad;
  int64_t ld_grad;
  float *dq;
  float *dw;
  float *dk;
  int32_t idx_heads, idx_dim, k;
  // Optional (nullptr: dk by atomics).  Sparse form on the MFMA shape: dk in
  // two passes through at least indexer_bwd_workspace_bytes() bytes.
  void *workspace;
  size_t workspace_bytes;
  // Set by the launcher from the workspace.
  float *contrib;
  int32_t *skey;
  int32_t *bnd;
  int32_t kpad, nbr;
};

hipError_t launch_indexer(const IndexerArgs &a, hipStream_t stream);
hipError_t launch_indexer_backward(const IndexerBwdArgs &a, hipStream_t stream);
hipError_t launch_align_loss(const AlignArgs &a, hipStream_t stream);
hipError_t launch_topk(const TopkArgs &a, hipStream_t stream);
hipError_t launch_sparse_attn(const AttnArgs &a, hipStream_t stream);
hipError_t launch_mha_prefill(const MhaArgs &a, hipStream_t stream);
size_t mha_workspace_bytes(const SeqLayout &seq);
// Top-k from the fused data of a decode indexer launch (a.fuse set, a.scores
// the same launch's scores for the exact fallback).
hipError_t launch_topk_fused(const TopkArgs &a, hipStream_t stream);
// Whether the fused decode selection serves a problem, and its workspace.
bool fuse_eligible(const SeqLayout &seq);
size_t fuse_workspace_bytes(const SeqLayout &seq);
size_t sparse_attn_workspace_bytes(const AttnArgs &a);
size_t topk_workspace_bytes(const TopkArgs &a);
size_t indexer_bwd_workspace_bytes(const IndexerBwdArgs &a);

// The indexer scores rows with its decode kernel (keys streamed per row, no
// key tiles shared by queries) when every sequence has at most two query rows.
inline bool decode_indexer(const SeqLayout &seq) { return seq.max_q_len <= 2; }

// Sequence metadata for one sequence, clamped to the host-validated bounds so
// that inconsistent device offsets can never produce an out-of-bounds access.
struct SeqInfo {
  int64_t q0, q1;    // packed query rows [q0, q1)
  int64_t kv0;       // first packed key row
  int64_t kvlen;     // keys of this sequence (<= max_kv_len)
  int64_t pos0;      // position of row q0
};

__device__ __forceinline__ SeqInfo clamp_seq(const SeqLayout &L, int64_t q0, int64_t q1, int64_t k0,
                                             int64_t k1, int64_t p0) {
  SeqInfo s;
  q0 = q0 < 0 ? 0 : (q0 > L.total_q ? L.total_q : q0);
  q1 = q1 < q0 ? q0 : (q1 > L.total_q ? L.total_q : q1);
  k0 = k0 < 0 ? 0 : (k0 > L.total_kv ? L.total_kv : k0);
  k1 = k1 < k0 ? k0 : (k1 > L.total_kv ? L.total_kv : k1);
  int64_t kvlen = k1 - k0;
  if (kvlen > L.max_kv_len) kvlen = L.max_kv_len;
  p0 = p0 < 0 ? 0 : p0;
  s.q0 = q0;
  s.q1 = q1;
  s.kv0 = k0;
  s.kvlen = kvlen;
  s.pos0 = p0;
  return s;
}

__device__ __forceinline__ SeqInfo load_seq(const SeqLayout &L, int b) {
  return clamp_seq(L, L.q_offsets[b], L.q_offsets[b + 1], L.kv_offsets[b], L.kv_offsets[b + 1], L.q_pos0[b]);
}

// Position of packed query row r in sequence s, clamped into [0, kvlen-1]
// (-1 when the sequence has no keys).
__device__ __forceinline__ int64_t row_pos(const SeqInfo &s, int64_t r) {
  int64_t p = s.pos0 + (r - s.q0);
  return p > s.kvlen - 1 ? s.kvlen - 1 : p;
}

// Sequence owning packed query row r: the last b with q_offsets[b] <= r
// (offsets are non-decreasing, so that is the count of such b, minus one).
// r must be uniform across the wave and every lane active: each lane loads
// offsets lane, lane + 64, lane + 128 and lane + 192 at once and ballots count
// them, which costs one memory round trip per 256 sequences instead of the
// log2(batch) dependent loads of a binary search.
__device__ __forceinline__ int find_seq(const SeqLayout &L, int64_t r) {
  const int lane = __lane_id();
  int cnt = 0;
  for (int base = 0; base < L.batch; base += 256) {
    bool le[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = base + 64 * u + lane;
      le[u] = i < L.batch && (int64_t)L.q_offsets[i] <= r;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) cnt += __popcll(__ballot(le[u]));
  }
  return cnt > 0 ? cnt - 1 : 0;
}

// find_seq in two halves, so that the offset loads can go out early and
// other loads behind them: find_seq_issue loads this lane's four candidate
// offsets among the first 256 sequences (addresses clamped, so the loads are
// unconditional); find_seq_done counts them like find_seq (searching on for
// batches beyond 256).  Same requirements as find_seq.
__device__ __forceinline__ void find_seq_issue(const SeqLayout &L, int (&o)[4]) {
  const int lane = __lane_id();
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = 64 * u + lane;
    o[u] = L.q_offsets[i < L.batch ? i : L.batch - 1];
  }
}

__device__ __forceinline__ int find_seq_done(const SeqLayout &L, int64_t r, const int (&o)[4]) {
  const int lane = __lane_id();
  int cnt = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) cnt += __popcll(__ballot(64 * u + lane < L.batch && (int64_t)o[u] <= r));
  for (int base = 256; base < L.batch; base += 256) {
    bool le[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = base + 64 * u + lane;
      le[u] = i < L.batch && (int64_t)L.q_offsets[i] <= r;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) cnt += __popcll(__ballot(le[u]));
  }
  return cnt > 0 ? cnt - 1 : 0;
}

// Cache row of key position pos (0 <= pos < s.kvlen) of sequence b.  With a
// block table, the block index and the table entry are clamped in bounds.
template <bool kPaged>
__device__ __forceinline__ int64_t kv_row(const PagedKV &pg, const SeqInfo &s, int b, int64_t pos) {
  if (!kPaged) return s.kv0 + pos;
  const int p32 = (int)pos;   // positions fit int32 (validated on the host)
  int blk = p32 >> pg.block_shift;
  blk = blk < 0 ? 0 : (blk >= pg.max_blocks ? pg.max_blocks - 1 : blk);
  int phys = pg.table[b * pg.max_blocks + blk];
  phys = phys < 0 ? 0 : (phys >= pg.num_blocks ? pg.num_blocks - 1 : phys);
  int slot = p32 - (blk << pg.block_shift);
  const int bmask = (1 << pg.block_shift) - 1;
  slot = slot < 0 ? 0 : (slot > bmask ? bmask : slot);
  return (int64_t)((phys << pg.block_shift) + slot);
}

// Sequence of packed query row r and its metadata.  Decode batches hold one
// query row per sequence (row r is sequence r); that layout is checked on
// loads issued together with the general search, so there the metadata
// arrives in one memory round trip instead of two.  r must be uniform across
// the wave and every lane active.
__device__ __forceinline__ int row_seq(const SeqLayout &L, int64_t r, SeqInfo &s) {
  const int rr = (int)(r < L.batch ? r : L.batch - 1);
  const int64_t q0 = L.q_offsets[rr], q1 = L.q_offsets[rr + 1];
  const int64_t k0 = L.kv_offsets[rr], k1 = L.kv_offsets[rr + 1], p0 = L.q_pos0[rr];
  if (r < L.batch && q0 == r && q1 == r + 1) {
    s = clamp_seq(L, q0, q1, k0, k1, p0);
    return rr;
  }
  const int b = find_seq(L, r);
  s = load_seq(L, b);
  return b;
}

// row_seq with the search offsets already loaded by find_seq_issue.
__device__ __forceinline__ int row_seq_issued(const SeqLayout &L, int64_t r, const int (&o)[4], SeqInfo &s) {
  const int rr = (int)(r < L.batch ? r : L.batch - 1);
  const int64_t q0 = L.q_offsets[rr], q1 = L.q_offsets[rr + 1];
  const int64_t k0 = L.kv_offsets[rr], k1 = L.kv_offsets[rr + 1], p0 = L.q_pos0[rr];
  if (r < L.batch && q0 == r && q1 == r + 1) {
    s = clamp_seq(L, q0, q1, k0, k1, p0);
    return rr;
  }
  const int b = find_seq_done(L, r, o);
  s = load_seq(L, b);
  return b;
}

}  // namespace dsa
