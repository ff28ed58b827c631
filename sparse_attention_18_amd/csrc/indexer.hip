// Lightning indexer for gfx950: FP8 e4m3fn MFMA scoring of causal
// (query, key) pairs with the ReLU and w-weighted head sum fused into the
// MFMA epilogue, so no per-head score is ever written.
//
// The method (ivugangingo.com article on DeepSeek-V3.2, "Sparse attention with
// almost linear long-context costs"; r.nikiv.dev summary, "How DSA Works"):
// a few low-precision heads score every (query, key) pair.  The formula this
// library fixes, since the pages give none:
//     score(t,s) = q_scale[t] * k_scale[s] * sum_j w[t,j] * ReLU(q8[t,j] . k8[s])
// (the per-token scales are positive, so they move outside the ReLU).
//
// Mapping onto v_mfma_f32_16x16x128_f8f6f4: M = 16 indexer heads of one
// query, N = 16 keys, K = the 128-wide head dimension (zero padded for
// d_I < 128).  Each lane then owns 4 heads x 1 key of every MFMA result, so
// the head sum is mostly in-lane; the remaining sum over the four 16-lane
// rows is a permlane reduce-scatter that leaves lane l holding key l of a
// 64-key block -- one coalesced 256-byte store per query and block.
//
// The prefill epilogue uses ReLU(x) = (x + |x|) / 2:
//     sum_j w_j ReLU(x_j) = sum_j (w_j/2) |x_j|  +  Qe . k,   Qe = sum_j (w_j/2) q_j
// so each (head, key) result costs one fused multiply-add with an |.| source
// modifier instead of a max and a multiply-add.  The linear term Qe . k is
// one more dot product per (query, key); it rides on one extra MFMA per
// 16-key block whose A rows are Qe split into three e4m3fn pieces
// (p1 + p2 + p3 = Qe * 2^e, exact up to about 2^-12 of max|Qe|).
#include "common.h"
#include "launch.h"

namespace dsa {
namespace {

constexpr int kWaves = 4;          // waves per workgroup
constexpr int kKeyTile = 64;       // keys per LDS tile in the prefill kernel
constexpr int kRowBytes = 128;     // one key row in LDS (d_I padded to 128)
constexpr int64_t kL2Bytes = 4 << 20;   // L2 per XCD

// LDS position of 16-byte chunk j of key n inside a key tile.  Chunk slots
// are XOR-swizzled by (n >> 1) & 7 so the 16 lanes of a row reading the same
// chunk of 16 consecutive keys hit 16 distinct 16-byte bank groups.
__device__ __forceinline__ int ktile_offset(int n, int j) {
  return n * kRowBytes + 16 * (j ^ ((n >> 1) & 7));
}

// The A operand (16 heads x 128 dims of one query, this lane's 32-byte
// K-chunk) and the fp32 weights of the 4 heads this lane accumulates.
template <int HB>
struct QueryRegs {
  v8i a[HB];
  float w[HB][4];
};

template <int HB>
__device__ __forceinline__ void load_query(QueryRegs<HB> &q, const IndexerArgs &p, int64_t row,
                                           bool valid, int g, int c, float wfac) {
  // Branch-free: every address is clamped in bounds, invalid parts are zeroed
  // by selects, so the prologue stays one basic block.
  const int H = p.idx_heads, d = p.idx_dim;
  const float qs = valid ? p.q_scale[row] * wfac : 0.0f;
  const bool dim_ok = 32 * g < d;
  const int dim_off = dim_ok ? 32 * g : 0;
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int head = hb * 16 + c;
    const bool ok = valid && head < H && dim_ok;
    const v4i *src =
        reinterpret_cast<const v4i *>(p.q_fp8 + (row * H + (head < H ? head : H - 1)) * d + dim_off);
    const v4i lo = src[0], hi = src[1];
    q.a[hb] = ok ? v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}
                 : v8i{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h2 = hb * 16 + 4 * g + i;
      const float wv = p.w[row * H + (h2 < H ? h2 : H - 1)];
      q.w[hb][i] = (valid && h2 < H) ? wv * qs : 0.0f;
    }
  }
}

// Per-lane head sum over this lane's 4*HB heads for one 16-key block, starting
// from `s`: sum_j w_j * ReLU(dot_j) (kAbs = false) or sum_j w_j * |dot_j|
// (kAbs = true, the weights then already carry the factor 1/2).  The HB MFMAs
// are independent, so they issue back to back before the epilogue uses them.
template <int HB, bool kAbs>
__device__ __forceinline__ float score_block(const QueryRegs<HB> &q, const v8i &b, float s) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  v4f d[HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) d[hb] = mfma_16x16x128_fp8(q.a[hb], b, zero);
#pragma unroll
  for (int hb = 0; hb < HB; ++hb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      s = fmaf(q.w[hb][i], kAbs ? fabsf(d[hb][i]) : fmaxf(d[hb][i], 0.f), s);
  return s;
}

constexpr int kLinPieces = 3;  // e4m3fn pieces carrying Qe

// Builds the linear-term operand of this wave's QW queries in LDS:
//   Qe[d] = sum_j (q_scale * w_j / 2) * q8[j][d]        (fp32)
//   x = Qe * 2^e with max|x| in [128, 256);  x = p1 + p2 + p3 + tiny rest,
// each p an e4m3fn vector (the residual after each piece is exact in fp32).
// `dst` receives the pieces as rows [qi][piece][128 bytes] and `inv` the
// factor 2^-e per query.  Half-wave h handles query 2r+h in round r; each lane
// owns 4 consecutive dims.
template <int QW>
__device__ __forceinline__ void build_linear_pieces(const IndexerArgs &p, const int64_t (&grow)[QW],
                                                    const bool (&valid)[QW], int lane,
                                                    uint8_t *dst, float *inv) {
  const int H = p.idx_heads, d = p.idx_dim;
  const int half = lane >> 5, dl = 4 * (lane & 31);
  const bool dim_ok = dl < d;
#pragma unroll
  for (int r = 0; r < (QW + 1) / 2; ++r) {
    const bool has_pair = 2 * r + 1 < QW;
    const int qi = 2 * r + half;
    const bool live = half == 0 || has_pair;
    const int64_t row = (half && has_pair) ? grow[has_pair ? 2 * r + 1 : 2 * r] : grow[2 * r];
    const bool ok = live && ((half && has_pair) ? valid[has_pair ? 2 * r + 1 : 2 * r] : valid[2 * r]);
    const uint8_t *qrow = p.q_fp8 + row * H * d + (dim_ok ? dl : 0);
    const float *wrow = p.w + row * H;
    float e0 = 0.f, e1 = 0.f, e2 = 0.f, e3 = 0.f;
#pragma unroll 64
    for (int j = 0; j < H; ++j) {
      const uint32_t x = *reinterpret_cast<const uint32_t *>(qrow + (int64_t)j * d);
      const float wj = wrow[j];
      const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(x, 1.0f, false);
      const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(x, 1.0f, true);
      e0 = fmaf(wj, lo[0], e0);
      e1 = fmaf(wj, lo[1], e1);
      e2 = fmaf(wj, hi[0], e2);
      e3 = fmaf(wj, hi[1], e3);
    }
    const float f = (ok && dim_ok) ? 0.5f * p.q_scale[row] : 0.f;
    e0 *= f; e1 *= f; e2 *= f; e3 *= f;
    float m = fmaxf(fmaxf(fabsf(e0), fabsf(e1)), fmaxf(fabsf(e2), fabsf(e3)));
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    // m = f * 2^ex with f in [0.5, 1): scaling by 2^(8 - ex) puts max|x| in [128, 256).
    const int sh = m > 0.f ? 8 - __builtin_amdgcn_frexp_expf(m) : 0;
    float x[4] = {ldexpf(e0, sh), ldexpf(e1, sh), ldexpf(e2, sh), ldexpf(e3, sh)};
#pragma unroll
    for (int pc = 0; pc < kLinPieces; ++pc) {
      typedef short v2s __attribute__((ext_vector_type(2)));
      v2s pk = {0, 0};
      pk = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(pk, x[0], x[1], 1.0f, false);
      pk = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(pk, x[2], x[3], 1.0f, true);
      const uint32_t bits = (uint32_t)(uint16_t)pk[0] | ((uint32_t)(uint16_t)pk[1] << 16);
      const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(bits, 1.0f, false);
      const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(bits, 1.0f, true);
      x[0] -= lo[0]; x[1] -= lo[1]; x[2] -= hi[0]; x[3] -= hi[1];
      if (live) *reinterpret_cast<uint32_t *>(dst + (qi * kLinPieces + pc) * 128 + dl) = bits;
    }
    if (live && (lane & 31) == 0) inv[qi] = ldexpf(1.0f, -sh);
  }
}

// Combine the four 16-lane rows' partial sums of four 16-key blocks: lane l
// ends with the full score of key l of the 64-key group.
__device__ __forceinline__ float reduce_four_blocks(float p0, float p1, float p2, float p3) {
  const float x02 = reduce_scatter32(p0, p2);
  const float x13 = reduce_scatter32(p1, p3);
  return reduce_scatter16(x02, x13);
}

// Prefill: grid (key split, query tile, sequence).  Each wave keeps QW query
// rows resident (A operands + weights); the workgroup streams its key range
// through double-buffered LDS tiles shared by all waves.  With kPaged the
// keys come from block-table caches; a 64-key tile never crosses a block
// (tiles start at multiples of 64, blocks hold a multiple of 64 rows).
template <int HB, int QW, bool kPaged>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void indexer_prefill_kernel(IndexerArgs p, int key_split, int xcd_splits) {
  constexpr int QT = kWaves * QW;
  __shared__ __attribute__((aligned(16))) uint8_t ktile[2][kKeyTile * kRowBytes];
  __shared__ __attribute__((aligned(16))) uint8_t linq[kWaves][QW * kLinPieces * 128];
  __shared__ float lininv[kWaves][QW];

  const int sb = (int)__builtin_amdgcn_workgroup_id_z();
  const SeqInfo s = load_seq(p.seq, sb);
  const int64_t qlen = s.q1 - s.q0;
  // Without XCD-bound splits the query tiles go out last first: the causal
  // triangle makes them the longest, and the short ones then fill the tail.
  const int wy = (int)__builtin_amdgcn_workgroup_id_y();
  const int qtile = __builtin_amdgcn_readfirstlane(xcd_splits ? wy : (int)gridDim.y - 1 - wy);
  const int64_t row_begin = (int64_t)qtile * QT;
  if (row_begin >= qlen || s.kvlen <= 0) return;
  const int64_t rows_here = qlen - row_begin < QT ? qlen - row_begin : QT;
  const int64_t last_pos = row_pos(s, s.q0 + row_begin + rows_here - 1);
  // Positions inside one sequence fit in int32 (the offsets are int32).
  // With xcd_splits, workgroup x runs on XCD x % 8 (dispatch is round-robin
  // over the eight XCDs, and the split count is a multiple of 8), so each XCD
  // keeps a fixed set of key splits in its L2.  The splits go to the XCDs in snake order
  // (x, 15 - x, 16 + x, 31 - x, ...): under the causal triangle later splits
  // have less work, and the pairs even it out across the XCDs.
  const int sx = (int)__builtin_amdgcn_workgroup_id_x(), sxcd = sx & 7, sj = sx >> 3;
  const int key_begin = (!xcd_splits ? sx : ((sj & 1) ? 8 * sj + 7 - sxcd : 8 * sj + sxcd)) * key_split;
  if (key_begin > last_pos) return;
  const int key_end = key_begin + key_split < last_pos + 1 ? key_begin + key_split : (int)last_pos + 1;
  const int kvlen = (int)s.kvlen;

  // The wave index is uniform; reading it through readfirstlane keeps every
  // per-query quantity below in scalar registers.
  const int tid = (int)__builtin_amdgcn_workitem_id_x(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;

  // Rows past the end of the tile get zero weights (and are never stored),
  // so no per-query branch splits the tile loop.
  QueryRegs<HB> q[QW];
  int64_t grow[QW];
  int pos[QW];
  bool valid[QW];
#pragma unroll
  for (int qi = 0; qi < QW; ++qi) {
    const int64_t r = row_begin + wave * QW + qi;
    valid[qi] = r < qlen;
    grow[qi] = s.q0 + (valid[qi] ? r : 0);
    pos[qi] = valid[qi] ? (int)row_pos(s, grow[qi]) : -1;
  }
  // The linear operand first, while no query operand occupies registers: all
  // of its loads can then be in flight at once.
  build_linear_pieces<QW>(p, grow, valid, lane, linq[wave], lininv[wave]);
#pragma unroll
  for (int qi = 0; qi < QW; ++qi) load_query<HB>(q[qi], p, grow[qi], valid[qi], g, c, 0.5f);

  // Each thread stages two 16-byte chunks of a 64-key tile (512 chunks).
  const int d = p.idx_dim;
  v4i stage[2];
  const uint8_t *kbase = p.k_fp8 + s.kv0 * d;
  auto fetch = [&](int t0) {
    // paged: the tile's first row (a tile stays inside one block; a tile
    // past the keys reads tile 0, whose values are then zeroed)
    const int64_t rb = kPaged ? kv_row<true>(p.pg, s, sb, t0 < kvlen ? t0 : 0) : 0;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int chunk = tid + 256 * e, n = chunk >> 3, j = chunk & 7;
      const int key = t0 + n;
      const bool ok = key < kvlen && 16 * j < d;
      const uint8_t *src = kPaged ? p.k_fp8 + (rb + n) * d
                                  : kbase + (int64_t)(key < kvlen ? key : 0) * d;
      const v4i x = *reinterpret_cast<const v4i *>(src + (16 * j < d ? 16 * j : 0));
      stage[e] = ok ? x : v4i{0, 0, 0, 0};
    }
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int chunk = tid + 256 * e, n = chunk >> 3, j = chunk & 7;
      *reinterpret_cast<v4i *>(&ktile[buf][ktile_offset(n, j)]) = stage[e];
    }
  };

  fetch(key_begin);
  commit(0);
  __syncthreads();

  // Linear-term A operand: row m = 4*qi + piece (qi < QW, piece < 3), K-chunk
  // g = dims 32g..32g+31.  The MFMA then leaves query g's three pieces in
  // elements 0..2 of the 16-lane row g, so `lin_fac[qi]` is 2^-e of query qi
  // in row qi and zero elsewhere: the reduce-scatter adds the term once.
  v8i lin_a = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  {
    const int pq = c >> 2, pc = c & 3;
    if (pq < QW && pc < kLinPieces) {
      const uint8_t *src = &linq[wave][(pq * kLinPieces + pc) * 128 + 32 * g];
      const v4i lo = *reinterpret_cast<const v4i *>(src);
      const v4i hi = *reinterpret_cast<const v4i *>(src + 16);
      lin_a = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  }
  float lin_fac[QW];
#pragma unroll
  for (int qi = 0; qi < QW; ++qi) lin_fac[qi] = g == qi ? lininv[wave][qi] : 0.f;

  int buf = 0;
  const float *kscale = p.k_scale + s.kv0;
  float *srow[QW];
#pragma unroll
  for (int qi = 0; qi < QW; ++qi) srow[qi] = p.scores + grow[qi] * p.ld;
  for (int t0 = key_begin; t0 < key_end; t0 += kKeyTile) {
    // The next tile's loads are clamped in bounds, so they are issued
    // unconditionally; the stores come last.  Both keep the whole tile body
    // one basic block, which lets the MFMAs and the epilogue interleave.
    const bool has_next = t0 + kKeyTile < key_end;
    fetch(t0 + kKeyTile);
    const int my_key = t0 + lane;
    const float ks = kPaged ? p.k_scale[kv_row<true>(p.pg, s, sb, t0) + lane]   // t0 < kvlen
                            : kscale[my_key < kvlen ? my_key : 0];

    float part[QW][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int n = kb * 16 + c;
      const v4i lo = *reinterpret_cast<const v4i *>(&ktile[buf][ktile_offset(n, 2 * g)]);
      const v4i hi = *reinterpret_cast<const v4i *>(&ktile[buf][ktile_offset(n, 2 * g + 1)]);
      const v8i bop = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const v4f e = mfma_16x16x128_fp8(lin_a, bop, v4f{0.f, 0.f, 0.f, 0.f});
      const float lin = e[0] + e[1] + e[2];
#pragma unroll
      for (int qi = 0; qi < QW; ++qi)
        part[qi][kb] = score_block<HB, true>(q[qi], bop, lin_fac[qi] * lin);
    }
    float v[QW];
#pragma unroll
    for (int qi = 0; qi < QW; ++qi)
      v[qi] = reduce_four_blocks(part[qi][0], part[qi][1], part[qi][2], part[qi][3]) * ks;
#pragma unroll
    for (int qi = 0; qi < QW; ++qi)
      if (my_key < key_end && my_key <= pos[qi]) srow[qi][my_key] = v[qi];
    if (has_next) {
      commit(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }
}

// ---- Selection data for the fused top-k (decode).  Each 1024-key chunk of
// a row bins its scores by the top 12 bits of their order-preserving keys
// (sign, exponent and three mantissa bits: 4096 bins, an eighth of an octave
// wide) and leaves, for the row's select kernel (topk.hip):
//  * a table of its nonzero bins in descending order, one word each:
//      bin << 20 | (first list slot of the bin) << 10 | (count - 1)
//    (a chunk has at most 1024 keys, so at most 1024 entries), and its length;
//  * its keys grouped by bin in that order, one word each:
//      (low 20 bits of the order key) << 10 | position within the chunk.
// The bins of the chunk's largest keys come first, so the select reads only
// the prefix of each list down to the bin that holds the row's k-th key; the
// lists replace the scores, which this path does not store.
__device__ __forceinline__ uint32_t fuse_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;                 // -0.0 ranks as +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// LDS operations of one wave complete in issue order; waiting for them all
// makes this wave's LDS writes visible to its next reads of other addresses.
__device__ __forceinline__ void lds_drain() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Run by one wave (the chunk's last to finish its keys) over the nloc
// (>= 1) scores in `sc`, using `hist` (kFuseBins words of LDS) as scratch;
// the other waves of the workgroup may already have exited.
__device__ __forceinline__ void bin_chunk(float *sc, uint32_t *hist, int nloc, int lane, uint32_t *tab,
                                          uint32_t *nz, uint32_t *list) {
  constexpr int kKeys = kFuseChunk / 64, kBins = kFuseBins / 64;   // per lane: 16 keys, 64 bins
#pragma unroll
  for (int u = 0; u < kBins / 4; ++u)
    *reinterpret_cast<v4i *>(&hist[4 * lane + 256 * u]) = v4i{0, 0, 0, 0};
  uint32_t key[kKeys];
#pragma unroll
  for (int u = 0; u < kKeys / 4; ++u) {
    const v4f sv = *reinterpret_cast<const v4f *>(sc + 4 * lane + 256 * u);
#pragma unroll
    for (int j = 0; j < 4; ++j) key[4 * u + j] = fuse_order_key(sv[j]);
  }
  lds_drain();
#pragma unroll
  for (int u = 0; u < kKeys; ++u)
    if (4 * lane + 256 * (u >> 2) + (u & 3) < nloc) atomicAdd(&hist[key[u] >> 20], 1u);
  lds_drain();
  // Lane l owns bins 4095 - 64l .. 4032 - 64l (descending); a wave scan of
  // (nonzero bins << 16 | keys) gives its first table entry and list slot.
  uint32_t cnt[kBins], tot = 0, nzb = 0;
#pragma unroll
  for (int u = 0; u < kBins / 4; ++u) {
    const v4i c4 = *reinterpret_cast<const v4i *>(&hist[kFuseBins - 4 - kBins * lane - 4 * u]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      cnt[4 * u + j] = (uint32_t)c4[3 - j];
      tot += cnt[4 * u + j];
      nzb += cnt[4 * u + j] != 0u;
    }
  }
  const uint32_t packed = (nzb << 16) | tot;
  const uint32_t inc = wave_scan<0>(packed);
  const uint32_t all = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
  uint32_t slot = (inc - packed) & 0xFFFFu, entry = (inc - packed) >> 16;
#pragma unroll
  for (int i = 0; i < kBins; ++i) {
    if (cnt[i] != 0u) {
      const uint32_t bin = (uint32_t)(kFuseBins - 1 - kBins * lane - i);
      tab[entry++] = bin << 20 | slot << 10 | (cnt[i] - 1u);
      hist[bin] = slot;                          // the bin's next free slot
      slot += cnt[i];
    }
  }
  if (lane == 0) *nz = all >> 16;
  lds_drain();
  // Scatter into LDS (over the scores, all read above), then one coalesced copy.
  uint32_t *lst = reinterpret_cast<uint32_t *>(sc);
#pragma unroll
  for (int u = 0; u < kKeys; ++u) {
    const int li = 4 * lane + 256 * (u >> 2) + (u & 3);
    if (li < nloc) lst[atomicAdd(&hist[key[u] >> 20], 1u)] = (key[u] & 0xFFFFFu) << 10 | (uint32_t)li;
  }
  lds_drain();
#pragma unroll
  for (int u = 0; u < kKeys / 4; ++u)
    if (4 * lane + 256 * u < nloc)
      *reinterpret_cast<v4i *>(list + 4 * lane + 256 * u) = *reinterpret_cast<const v4i *>(lst + 4 * lane + 256 * u);
}

// Decode (few query rows per sequence): grid (key chunk, query row).  Keys
// are used by one query only, so each wave streams its own 256-key slice
// straight from HBM into MFMA B operands; nothing goes through LDS.
constexpr int kDecodeChunk = 1024;  // keys per workgroup (4 waves x 256)
static_assert(kDecodeChunk == kFuseChunk, "a fused chunk is one decode workgroup's keys");

template <int HB, bool kPaged, bool kFuse>
__global__ __launch_bounds__(256) void indexer_decode_kernel(IndexerArgs p) {
  const int64_t row = __builtin_amdgcn_workgroup_id_y();
  SeqInfo s;
  const int b = row_seq(p.seq, row, s);
  if (row < s.q0 || row >= s.q1 || s.kvlen <= 0) return;
  const int64_t pos = row_pos(s, row);
  const int tid = (int)__builtin_amdgcn_workitem_id_x(), lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int64_t chunk_begin = (int64_t)__builtin_amdgcn_workgroup_id_x() * kDecodeChunk;
  if (chunk_begin > pos) return;
  const int64_t wave_begin = chunk_begin + wave * (kDecodeChunk / kWaves);
  // A wave past the row's last key has no work (with kFuse it still joins the
  // workgroup's barriers below).
  if (!kFuse && wave_begin > pos) return;
  __shared__ uint32_t s_done;                    // waves that have finished their keys
  if (kFuse) {
    if (tid == 0) s_done = 0u;
    __syncthreads();
  }
  const int64_t wave_end = wave_begin + kDecodeChunk / kWaves < pos + 1
                               ? wave_begin + kDecodeChunk / kWaves : pos + 1;

  QueryRegs<HB> q;
  load_query<HB>(q, p, row, true, g, c, 1.0f);
  const int d = p.idx_dim;

  // Keys and key scales are read through buffer descriptors spanning this
  // wave's slice: loads past it return zeros, so every load is issued
  // unconditionally.  The whole offset goes in the vector offset (the scalar
  // offset is not part of the range check).  With no branch around them the
  // compiler counts them, and the wait before a step's MFMAs covers only that
  // step's loads; the next step's stay in flight.  Dims at or past d_I get an
  // offset past the range (zeros too).  The scores go to LDS and are written
  // out after the last load: a store between the loads would hold up the
  // waits on them, which share one in-order counter.
  __shared__ __attribute__((aligned(16))) float s_sc[kWaves][kDecodeChunk / kWaves];
  const int nk = wave_begin > pos ? 0 : __builtin_amdgcn_readfirstlane((int)(wave_end - wave_begin));   // 0..256 keys
  auto rsrc = [&](const void *base, int bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    const uint64_t u = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a) |
                       ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)) << 32);
    return __builtin_amdgcn_make_buffer_rsrc((void *)(uintptr_t)u, (short)0, bytes, 0x00020000);
  };
  const __amdgpu_buffer_rsrc_t krs = rsrc(p.k_fp8 + (kPaged ? 0 : (s.kv0 + wave_begin) * d), kPaged ? 0 : nk * d);
  const __amdgpu_buffer_rsrc_t srs = rsrc(p.k_scale + (kPaged ? 0 : s.kv0 + wave_begin), kPaged ? 0 : nk * 4);
  const int koff = 32 * g < d ? c * d + 32 * g : 0x40000000;
  auto load_step = [&](int st, v8i (&kr)[4], float &ks) {
    if (kPaged) {
      // one block per 64-key step: descriptors over that step's rows
      const int cnt = nk - 64 * st < 0 ? 0 : (nk - 64 * st > 64 ? 64 : nk - 64 * st);
      const int64_t at = wave_begin + 64 * st;
      const int64_t rb = kv_row<true>(p.pg, s, b, at < s.kvlen ? at : 0);
      const __amdgpu_buffer_rsrc_t kst = rsrc(p.k_fp8 + rb * d, cnt * d);
      const __amdgpu_buffer_rsrc_t sst = rsrc(p.k_scale + rb, cnt * 4);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int vo = koff + kb * 16 * d;
        const v4i lo = __builtin_amdgcn_raw_buffer_load_b128(kst, vo, 0, 0);
        const v4i hi = __builtin_amdgcn_raw_buffer_load_b128(kst, vo + 16, 0, 0);
        kr[kb] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      ks = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sst, lane * 4, 0, 0));
      return;
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int vo = koff + (st * 64 + kb * 16) * d;
      const v4i lo = __builtin_amdgcn_raw_buffer_load_b128(krs, vo, 0, 0);
      const v4i hi = __builtin_amdgcn_raw_buffer_load_b128(krs, vo + 16, 0, 0);
      kr[kb] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    ks = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srs, lane * 4 + st * 256, 0, 0));
  };
  auto score_step = [&](int st, const v8i (&kr)[4], float ks) {
    float part[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) part[kb] = score_block<HB, false>(q, kr[kb], 0.f);
    s_sc[wave][st * 64 + lane] = reduce_four_blocks(part[0], part[1], part[2], part[3]) * ks;
  };
  // Two register sets take turns (no copy of a set whose loads are still in
  // flight, which would wait for them); loads past the slice read zeros.
  const int nsteps = (nk + 63) / 64;   // 0 for an idle wave
  v8i ka[4], kb2[4];
  float ksa, ksb;
  // (The scheduling barriers keep each set's loads ahead of the other set's
  // MFMAs.)
  if (nsteps > 0) load_step(0, ka, ksa);
  for (int st = 0; st < nsteps; st += 2) {
    load_step(st + 1, kb2, ksb);
    __builtin_amdgcn_sched_barrier(0);
    score_step(st, ka, ksa);
    if (st + 1 < nsteps) {
      load_step(st + 2, ka, ksa);
      __builtin_amdgcn_sched_barrier(0);
      score_step(st + 1, kb2, ksb);
    }
  }
  if constexpr (kFuse) {
    // The last wave to finish bins the whole chunk; the others leave.
    __shared__ __attribute__((aligned(16))) uint32_t s_hist[kFuseBins];
    lds_drain();
    uint32_t done = 0u;
    if (lane == 0) done = atomicAdd(&s_done, 1u);
    if (__builtin_amdgcn_readfirstlane(done) != kWaves - 1) return;
    lds_drain();
    const int nloc = (int)(pos + 1 - chunk_begin < kDecodeChunk ? pos + 1 - chunk_begin : kDecodeChunk);
    const int64_t slot = row * p.fuse.nchunk + (int64_t)__builtin_amdgcn_workgroup_id_x();
    bin_chunk(&s_sc[0][0], s_hist, nloc, lane, p.fuse.tab + slot * kFuseTabCap, p.fuse.nz + slot,
              p.fuse.list + slot * kDecodeChunk);
  } else {
    float *srow = p.scores + row * p.ld;
    for (int64_t t0 = wave_begin; t0 < wave_end; t0 += 64) {
      const int64_t my_key = t0 + lane;
      if (my_key < wave_end) srow[my_key] = s_sc[wave][t0 - wave_begin + lane];
    }
  }
}

template <int HB, int QW>
hipError_t launch_prefill(const IndexerArgs &a, hipStream_t stream) {
  constexpr int QT = kWaves * QW;
  const int64_t qtiles = (a.seq.max_q_len + QT - 1) / QT;
  const int64_t kv = a.seq.max_kv_len;
  // Work estimate: the longest sequence's queries sit at its last max_q_len
  // positions; busy_blocks(sp) counts the workgroups with causal keys.
  const double first_pos = (double)(kv - a.seq.max_q_len);
  auto busy_blocks = [&](int64_t sp) {
    const double t = (double)qtiles;
    return ((t * first_pos + QT * t * (t + 1) / 2) / sp + t / 2) * a.seq.batch;
  };
  auto split_of = [&](int64_t m) { return ((kv + m - 1) / m + 63) / 64 * 64; };
  int64_t nsplit, split;
  int xcd_splits;
  if (kv * a.idx_dim <= (int64_t)kL2Bytes) {
    // The longest sequence's keys fit one XCD's L2, so every XCD can hold all
    // of them: as few splits as leave 1024 or more workgroups with keys (the
    // queries are loaded, and their linear operand built, once per split).
    nsplit = 1;
    while (nsplit < 8 && busy_blocks(split_of(nsplit)) < 1024) nsplit *= 2;
    split = split_of(nsplit);
    xcd_splits = 0;
  } else {
    // Key splits: 8m of them, m >= 2, of equal length (a multiple of 64), so
    // that every XCD gets the same share of the keys.  m is the smallest that
    // leaves about 6K workgroups with work (several rounds of the 256 CUs x
    // 2-3 resident workgroups, so the causal tail evens out), with splits of
    // at least 256 keys; fewer, longer splits load the queries and build
    // their linear operand less often.
    int64_t m = 2;
    while (split_of(8 * (m + 1)) >= 256 && busy_blocks(split_of(8 * m)) < 6144) ++m;
    nsplit = 8 * m;
    split = split_of(nsplit);
    xcd_splits = 1;
  }
  dim3 grid((unsigned)nsplit, (unsigned)qtiles, (unsigned)a.seq.batch);
  if (a.pg.table != nullptr)
    hipLaunchKernelGGL((indexer_prefill_kernel<HB, QW, true>), grid, dim3(256), 0, stream, a, (int)split,
                       xcd_splits);
  else
    hipLaunchKernelGGL((indexer_prefill_kernel<HB, QW, false>), grid, dim3(256), 0, stream, a, (int)split,
                       xcd_splits);
  return hipGetLastError();
}

template <int HB>
hipError_t launch_decode(const IndexerArgs &a, hipStream_t stream) {
  dim3 grid((unsigned)((a.seq.max_kv_len + kDecodeChunk - 1) / kDecodeChunk), (unsigned)a.seq.total_q);
  const bool paged = a.pg.table != nullptr, fuse = a.fuse.tab != nullptr;
  if (paged && fuse)
    hipLaunchKernelGGL((indexer_decode_kernel<HB, true, true>), grid, dim3(256), 0, stream, a);
  else if (paged)
    hipLaunchKernelGGL((indexer_decode_kernel<HB, true, false>), grid, dim3(256), 0, stream, a);
  else if (fuse)
    hipLaunchKernelGGL((indexer_decode_kernel<HB, false, true>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((indexer_decode_kernel<HB, false, false>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int HB>
hipError_t dispatch(const IndexerArgs &a, hipStream_t stream) {
  // A handful of query rows per sequence: stream keys per row.
  if (decode_indexer(a.seq)) return launch_decode<HB>(a, stream);
  return launch_prefill<HB, (HB >= 8 ? 1 : (HB >= 2 ? 2 : 4))>(a, stream);
}

}  // namespace

hipError_t launch_indexer(const IndexerArgs &a, hipStream_t stream) {
  if (a.seq.total_q == 0 || a.seq.total_kv == 0) return hipSuccess;
  const int hb = (a.idx_heads + 15) / 16;
  if (hb <= 1) return dispatch<1>(a, stream);
  if (hb <= 2) return dispatch<2>(a, stream);
  if (hb <= 4) return dispatch<4>(a, stream);
  return dispatch<8>(a, stream);
}

}  // namespace dsa
