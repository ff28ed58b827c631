// Prefill-mode sparse attention on gfx950: per-head keys and values.
//
// The threadnavigator.com thread on DeepSeek-V3.2 (first tweet) notes that
// the model keeps separate attention modes for disaggregated prefill and
// decode.  Read as MLA's two forms of one attention: decode runs the absorbed
// form (sparse_attn.hip: one shared 576-wide row per key, gathered once for
// all heads); prefill runs the per-head form computed here, where head h of
// query row r has a 192-wide query (128 + 64 rotary), key position s has a
// per-head key (k_nope[s, h] (128) followed by the rotary key k_rope[s] (64)
// that all heads share) and a per-head value v[s, h] (128):
//   logit[h, s] = scale * (q[r, h, :128] . k_nope[s, h] + q[r, h, 128:] . k_rope[s])
//   out[r, h]   = sum_{s in sel(r)} softmax_s(logit[h, :]) * v[s, h]
// with sel(r) the distinct selected positions of row r inside its sequence
// (ivugangingo.com article, "Sparse attention with almost linear long-context
// costs": attention runs over the selected set only).
//
// Shape of the computation.  With per-head keys a query's selection cannot
// share one gather across heads, and neighbouring queries of a prefill chunk
// select mostly the same keys; so this form runs over dense 64-key tiles of
// the sequence, per (head, 256 query rows), and applies the selection as a
// bit mask.  Tiles no row of the block selected are skipped.  Per tile and
// head the work is 256 x 64 x (192 + 128) MACs on bf16 MFMA: this form is
// compute-bound where the absorbed form is bound by its gathers.
//
// Launches (all on the caller's stream):
//   1. mha_plan_kernel: query blocks of up to 256 rows of one sequence;
//   2. mha_mask_kernel: per query row, the bit mask of its selected
//      positions, one 64-bit word per key tile, stored block-major
//      (mask[block][tile][row in block]) so that a block's words for one tile
//      are 2 KB contiguous;
//   3. mha_tiles_kernel: per block, the ascending list of tiles any of its
//      rows selected;
//   4. mha_prefill_kernel: one workgroup of 8 waves per (head, block), each
//      wave 32 query rows.  Per listed tile: S^T = K . Q^T (12 bf16 MFMA
//      k-steps over 192 dims, two 32-key halves), the mask, an online
//      softmax in a lazily moved exponent frame, then O^T += V^T . P^T
//      (P straight from the S^T registers, V^T through transposing LDS
//      reads).  Tiles (K nope, K rope, V, mask words) arrive by LDS-DMA in a
//      three-stage ring, one tile ahead of the compute; the two waves of a
//      SIMD run their phases in opposite order.
#include "common.h"
#include "kv_gather.h"
#include "launch.h"

namespace dsa {
namespace {

constexpr int kMN = 128;              // per-head key part decompressed from the latent
constexpr int kMR = 64;               // rotary key part, shared by the heads
constexpr int kMQ = kMN + kMR;        // query / key width per head
constexpr int kMV = 128;              // value width per head
constexpr int kMKB = 64;              // keys per tile
constexpr int kMQB = 256;             // query rows per block (8 waves x 32)
constexpr int kMWaves = 8;
constexpr int kMStages = 3;
constexpr int kMMaxTiles = (int)(kMhaMaxKvLen / kMKB);
// A stage: 1 KB blocks of K nope (64 rows x 16 chunks of 16 B), K rope
// (64 x 8), V (64 x 16) and the block's 256 mask words.  Row data sits in
// blocks of 16 rows x 4 chunks: chunk c of row r at block
// (r / 16) * (C / 4) + c / 4, slot (r % 16) * 4 + ((c % 4) ^ ((r / 4) % 4)),
// so that 16 rows read at one chunk hit 16 distinct bank groups.
constexpr int kBNope = 0, kBRope = 16, kBV = 24, kBMask = 40, kBStage = 42;
constexpr int kMStageBytes = kBStage * 1024;
constexpr float kMSlack = 8.f;        // log2 headroom of the exponent frame
static_assert(kMStages * kMStageBytes <= 160 * 1024 - 1024, "LDS budget");

__device__ __forceinline__ v8bf lds_v8bf(const DSA_LDS uint8_t *ptr) {
  const v4i x = *reinterpret_cast<const DSA_LDS v4i *>(ptr);
  return as_v8bf(x);
}

struct MhaWs {
  int4 *info;          // [nblk]: sequence (-1: unused), first row, rows
  int32_t *prefix;     // [batch]: first block of each sequence
  int32_t *count;      // [nblk]: listed tiles
  int32_t *list;       // [nblk][W]: tile indices
  uint64_t *mask;      // [nblk][W][256]
  int32_t nblk, W;
  SeqLayout seq;
};

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

struct MhaLayout {
  int64_t nblk, W, info, prefix, count, list, mask, total;
};

MhaLayout mha_layout(const SeqLayout &seq) {
  MhaLayout L;
  L.nblk = (seq.total_q + kMQB - 1) / kMQB + seq.batch;
  L.W = seq.max_kv_len > 0 ? (seq.max_kv_len + kMKB - 1) / kMKB : 1;
  L.info = 0;
  L.prefix = round_up(L.info + L.nblk * 16, 256);
  L.count = round_up(L.prefix + (int64_t)seq.batch * 4, 256);
  L.list = round_up(L.count + L.nblk * 4, 256);
  L.mask = round_up(L.list + L.nblk * L.W * 4, 256);
  L.total = round_up(L.mask + L.nblk * L.W * kMQB * 8, 256);
  return L;
}

// Exclusive prefix of one value per thread over a workgroup of T threads;
// *total receives the sum.  s_w holds T / 64 partials.
template <int T>
__device__ __forceinline__ int block_excl(int v, int *s_w, int *total) {
  const int tid = __builtin_amdgcn_workitem_id_x(), lane = tid & 63, wv = tid >> 6;
  const int inc = (int)wave_scan<0>((uint32_t)v);
  if (lane == 63) s_w[wv] = inc;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < T / 64; ++i) {
    const int x = s_w[i];
    before += i < wv ? x : 0;
    all += x;
  }
  __syncthreads();
  *total = all;
  return before + inc - v;
}

// ---- 1. query blocks ----------------------------------------------------
__global__ __launch_bounds__(1024) void mha_plan_kernel(SeqLayout seq, MhaWs w) {
  __shared__ int s_w[16];
  const int tid = __builtin_amdgcn_workitem_id_x();
  int carry = 0;
  for (int base = 0; base < seq.batch; base += 1024) {
    const int b = base + tid;
    SeqInfo s{};
    int nb = 0;
    if (b < seq.batch) {
      s = load_seq(seq, b);
      nb = (int)((s.q1 - s.q0 + kMQB - 1) / kMQB);
    }
    int chunk;
    const int first = carry + block_excl<1024>(nb, s_w, &chunk);
    if (b < seq.batch) {
      w.prefix[b] = first;
      for (int lb = 0; lb < nb && first + lb < w.nblk; ++lb) {
        const int64_t r0 = s.q0 + (int64_t)lb * kMQB;
        const int64_t n = s.q1 - r0;
        w.info[first + lb] = make_int4(b, (int)r0, (int)(n < kMQB ? n : kMQB), 0);
      }
    }
    carry += chunk;
  }
  for (int e = carry + tid; e < w.nblk; e += 1024) w.info[e] = make_int4(-1, 0, 0, 0);
}

// ---- 2. row masks -------------------------------------------------------
__global__ __launch_bounds__(256) void mha_mask_kernel(MhaArgs p, MhaWs w) {
  __shared__ uint32_t bm[2 * kMMaxTiles];
  const int tid = __builtin_amdgcn_workitem_id_x();
  const int64_t r = __builtin_amdgcn_workgroup_id_x();
  SeqInfo s;
  const int b = row_seq(p.seq, r, s);
  const int W = w.W;
  for (int i = tid; i < 2 * W; i += 256) bm[i] = 0u;
  __syncthreads();
  const int32_t *row = p.idx + r * p.k;
  for (int i = tid; i < p.k; i += 256) {
    const int v = row[i];
    if (v >= 0 && v < s.kvlen) atomicOr(&bm[v >> 5], 1u << (v & 31));
  }
  __syncthreads();
  if (r < s.q0 || r >= s.q1) return;            // inconsistent offsets: row owned by no block
  const int rel = (int)(r - s.q0);
  const int blk = w.prefix[b] + rel / kMQB;
  if (blk < 0 || blk >= w.nblk) return;
  uint64_t *dst = w.mask + (int64_t)blk * W * kMQB + rel % kMQB;
  for (int t = tid; t < W; t += 256)
    dst[(int64_t)t * kMQB] = (uint64_t)bm[2 * t] | ((uint64_t)bm[2 * t + 1] << 32);
}

// ---- 3. per-block tile lists -------------------------------------------
__global__ __launch_bounds__(512) void mha_tiles_kernel(MhaWs w) {
  __shared__ uint8_t flag[kMMaxTiles];
  __shared__ int s_w[8];
  const int tid = __builtin_amdgcn_workitem_id_x(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int blk = __builtin_amdgcn_workgroup_id_x();
  const int4 info = w.info[blk];
  if (info.x < 0) {
    if (tid == 0) w.count[blk] = 0;
    return;
  }
  const int W = w.W, nrows = info.z;
  // only tiles inside the block's own sequence (so every key row a listed
  // tile loads is in bounds, whatever the offsets)
  const SeqInfo s = load_seq(w.seq, info.x);
  const int wt = (int)((s.kvlen + kMKB - 1) / kMKB < W ? (s.kvlen + kMKB - 1) / kMKB : W);
  const uint64_t *m = w.mask + (int64_t)blk * W * kMQB;
  for (int t = wave; t < wt; t += kMWaves) {
    uint64_t x = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int rr = 4 * lane + e;
      if (rr < nrows) x |= m[(int64_t)t * kMQB + rr];
    }
    const uint32_t any = wave_reduce<1>((uint32_t)x | (uint32_t)(x >> 32));
    if (lane == 0) flag[t] = any != 0u;
  }
  __syncthreads();
  int cnt = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int t = 4 * tid + e;
    cnt += t < wt ? flag[t] : 0;
  }
  int total;
  int at = block_excl<512>(cnt, s_w, &total);
  int32_t *lst = w.list + (int64_t)blk * W;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int t = 4 * tid + e;
    if (t < wt && flag[t]) lst[at++] = t;
  }
  if (tid == 0) w.count[blk] = total;
}

// ---- 4. attention -------------------------------------------------------
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mha_prefill_kernel(MhaArgs p, MhaWs w) {
  __shared__ __attribute__((aligned(1024))) uint8_t tiles[kMStages * kMStageBytes];

  const int tid = __builtin_amdgcn_workitem_id_x(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = lane >> 5, j = lane & 31, jl = lane & 15, half = (lane >> 4) & 1;

  // Work item (head, block).  Workgroup ids go round-robin over the 8 XCDs;
  // each XCD takes a contiguous range of items, so the blocks of one head
  // run together on one XCD and share its L2 for that head's keys and values.
  // Within a head the longest blocks (latest rows) go first.
  const int wg = __builtin_amdgcn_workgroup_id_x();
  const int64_t items = (int64_t)p.heads * w.nblk;
  const int64_t per_xcd = (items + 7) / 8;
  const int64_t local = wg >> 3;
  const int64_t item = (int64_t)(wg & 7) * per_xcd + local;
  if (local >= per_xcd || item >= items) return;
  const int h = (int)(item / w.nblk);
  const int blk = w.nblk - 1 - (int)(item % w.nblk);
  const int4 info = w.info[blk];
  if (info.x < 0) return;
  const SeqInfo s = load_seq(p.seq, info.x);
  const int nrows = info.z;
  const int ntiles = w.count[blk];
  const int32_t *tl = w.list + (int64_t)blk * w.W;

  const int my = 32 * wave + j;                  // row inside the block
  const bool row_ok = my < nrows;
  const int64_t row = info.y + (row_ok ? my : nrows - 1);
  const int H = p.heads;

  // Q^T operands: k-step ks = dims 16ks..16ks+15; lane (G, j) holds query
  // row j's dims 16ks + 8G .. +7.
  v8bf qb[kMQ / 16];
  {
    const uint16_t *qrow = p.q + (row * H + h) * (int64_t)kMQ + 8 * G;
#pragma unroll
    for (int ks = 0; ks < kMQ / 16; ++ks) qb[ks] = as_v8bf(*reinterpret_cast<const v4i *>(qrow + 16 * ks));
  }

  // ---- tile loads: 42 LDS-DMA blocks per tile, block q by wave q % 8.
  // Row-data block: slot i holds row 16 rb + i / 4, chunk 4 cq + ((i % 4) ^ (i / 16)).
  const int ri = lane >> 2, lc = (lane & 3) ^ (lane >> 4);
  const int64_t kv0 = s.kv0;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(DSA_LDS uint8_t *)tiles;
  auto issue = [&](int tile, int stage) {
    // listed tiles start inside the sequence: 1 <= rows_valid <= 64
    const int rows_valid = (int)(s.kvlen - (int64_t)tile * kMKB < kMKB ? s.kvlen - (int64_t)tile * kMKB : kMKB);
    const int64_t key0 = kv0 + (int64_t)tile * kMKB;
    const uint32_t lds_stage = lds0 + stage * kMStageBytes;
#pragma unroll
    for (int n = 0; n < 6; ++n) {
      const int q = wave + kMWaves * n;
      if (q >= kBStage) break;
      const uint32_t lds = lds_stage + q * 1024;
      if (q < kBMask) {
        const bool rope = q >= kBRope && q < kBV;
        const int qq = rope ? q - kBRope : (q < kBRope ? q - kBNope : q - kBV);
        const int cpr = rope ? 2 : 4;                  // chunk quads per row
        const int rb = qq / cpr, cq = qq % cpr;
        int r = 16 * rb + ri;
        r = r < rows_valid ? r : rows_valid - 1;
        const uint8_t *base;
        uint32_t stride;
        if (rope) {
          base = reinterpret_cast<const uint8_t *>(p.k_rope + key0 * kMR);
          stride = kMR * 2;
        } else {
          const uint16_t *t = q < kBRope ? p.k_nope : p.v;
          base = reinterpret_cast<const uint8_t *>(t + (key0 * H + h) * (int64_t)kMN);
          stride = (uint32_t)H * kMN * 2;
        }
        const uint32_t voff = (uint32_t)r * stride + (uint32_t)(4 * cq + lc) * 16;
        lds_dma16_x1(voff, sbase(base), lds);
      } else {
        const uint64_t *mb = w.mask + ((int64_t)blk * w.W + tile) * kMQB + (q - kBMask) * 128;
        lds_dma16_x1((uint32_t)lane * 16, sbase(mb), lds);
      }
    }
  };

  // ---- per-lane LDS offsets
  // S^T A operand, key half kh, k-step ks: row 32 kh + j, chunk 2 ks' + G
  // (ks' = ks, or ks - 8 in the rope region).
  const int sw = (j >> 2) & 3;
  const int k_lane = (j & 15) * 64;
  auto k_off = [&](int kh, int ks) {
    if (ks < kMN / 16) {
      const int b1k = kBNope + (2 * kh + (j >> 4)) * 4 + (ks >> 1);
      return b1k * 1024 + k_lane + (((2 * (ks & 1) + G) ^ sw) * 16);
    }
    const int kr = ks - kMN / 16;
    const int b1k = kBRope + (2 * kh + (j >> 4)) * 2 + (kr >> 1);
    return b1k * 1024 + k_lane + (((2 * (kr & 1) + G) ^ sw) * 16);
  };
  // V^T A operand through ds_read_b64_tr_b16: a 16-lane group reads rows
  // r0 + jl / 4 at dims 32 u + 16 half + 4 (jl % 4) .. +3 and receives, per
  // lane jl, dim 32 u + 16 half + jl of rows r0 .. r0 + 3.  Keys of k-step
  // (kh, hf), element e: 32 kh + 16 hf + 4 G + e (e < 4), + 8 for e >= 4 --
  // the order in which the S^T registers hold them.
  const int a4 = jl >> 2, b4 = jl & 3;
  const int v_lo = (4 * G + a4) * 64 + (((2 * half + (b4 >> 1)) ^ G) * 16) + 8 * (b4 & 1);
  const int v_hi = (8 + 4 * G + a4) * 64 + (((2 * half + (b4 >> 1)) ^ (2 + G)) * 16) + 8 * (b4 & 1);
  auto load_vt = [&](const DSA_LDS uint8_t *tb, int kh, int hf, int u) {
    const int b1k = kBV + (2 * kh + hf) * 4 + u;
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DSA_LDS v4s *)(tb + b1k * 1024 + v_lo));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DSA_LDS v4s *)(tb + b1k * 1024 + v_hi));
    const v2i lo2 = __builtin_bit_cast(v2i, lo), hi2 = __builtin_bit_cast(v2i, hi);
    return as_v8bf(v4i{lo2[0], lo2[1], hi2[0], hi2[1]});
  };

  v16f o[kMV / 32];
#pragma unroll
  for (int u = 0; u < kMV / 32; ++u) o[u] = v16f{};
  float l_part = 0.f;
  float m_used = -1e30f;                         // exponent frame (log2 units); no key yet
  const float c2 = p.scale * kLog2e;

  // Phase 1 of a tile: S^T, mask, frame, P (bf16, registers).
  auto qk_softmax = [&](const DSA_LDS uint8_t *tb, v8bf (&pk)[2][2]) {
    // S^T: two 32-key halves, 12 dependent k-steps each, interleaved
    // (step i: half i % 2, k-step i / 2); A operands read kLA steps ahead.
    constexpr int kSteps = 2 * (kMQ / 16), kLA = 4;
    v16f sc[2] = {v16f{}, v16f{}};
    v8bf a[kLA];
#pragma unroll
    for (int i = 0; i < kLA; ++i) a[i] = lds_v8bf(tb + k_off(i & 1, i >> 1));
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
      sc[i & 1] = mfma_32x32x16_bf16(a[i % kLA], qb[i >> 1], sc[i & 1]);
      if (i + kLA < kSteps)
        a[i % kLA] = lds_v8bf(tb + k_off((i + kLA) & 1, (i + kLA) >> 1));
      __builtin_amdgcn_sched_barrier(0);
    }
    const uint64_t mw = row_ok ? *reinterpret_cast<const DSA_LDS uint64_t *>(tb + kBMask * 1024 + my * 8) : 0ull;

    // mask, tile maximum, frame
    // element r of half kh is key 32 kh + 8 (r / 4) + 4 G + r % 4: bit
    // 8 (r / 4) + r % 4 of the half's word shifted by 4 G
    float mt = -INFINITY;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const uint32_t mh = (uint32_t)(mw >> (32 * kh + 4 * G));
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = (mh & (1u << (8 * (r >> 2) + (r & 3)))) ? sc[kh][r] : -INFINITY;
        sc[kh][r] = x;
        mt = fmaxf(mt, x);
      }
    }
    mt = max_across_halves(mt) * c2;
    if (mt > m_used + kMSlack) {
      const float alpha = __builtin_amdgcn_exp2f(m_used - mt);
      l_part *= alpha;
#pragma unroll
      for (int u = 0; u < kMV / 32; ++u) o[u] *= alpha;
      m_used = mt;
    }
    // P = 2^(logit * c2 - frame); masked logits give 0
    float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pe = __builtin_amdgcn_exp2f(fmaf(sc[kh][r], c2, -m_used));
        if (r & 1) ls1 += pe;
        else ls0 += pe;
        pk[kh][r >> 3][r & 7] = (__bf16)pe;
      }
    l_part += ls0 + ls1;
  };
  // Phase 2: O^T[dims][rows] += V^T . P^T, 16 independent MFMAs (step i:
  // k-step (kh, hf) = (i / 8, (i / 4) % 2), dims block u = i % 4), V^T read
  // two steps ahead.
  auto pv = [&](const DSA_LDS uint8_t *tb, const v8bf (&pk)[2][2]) {
    constexpr int kPV = 16, kVA = 2;
    v8bf va[kVA];
#pragma unroll
    for (int i = 0; i < kVA; ++i) va[i] = load_vt(tb, i >> 3, (i >> 2) & 1, i & 3);
#pragma unroll
    for (int i = 0; i < kPV; ++i) {
      o[i & 3] = mfma_32x32x16_bf16(va[i % kVA], pk[i >> 3][(i >> 2) & 1], o[i & 3]);
      if (i + kVA < kPV) va[i % kVA] = load_vt(tb, (i + kVA) >> 3, ((i + kVA) >> 2) & 1, (i + kVA) & 3);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The two waves of a SIMD (w and w + 4) run the phases in opposite order:
  // waves 0-3 do S^T, softmax, P.V of tile t; waves 4-7 start step t with
  // the P.V of tile t - 1 (its P kept in registers, its frame still the
  // one P was made in) and keep tile t's P for the next step.  One wave's
  // softmax then runs while the other issues MFMAs.  Tile t + 1 is loaded
  // during step t into stage (t + 1) % 3, which step t - 1's P.V (deferred
  // or not) no longer reads once the step's barrier has passed.  A deferred
  // wave issues those loads after its P.V (which reads stage (t - 1) % 3),
  // so its MFMAs start right at the barrier.
  const bool defer = wave >= kMWaves / 2;
  v8bf pk[2][2];                  // P of the tile whose P.V is pending
  if (ntiles > 0) issue(tl[0], 0);
  // stage bases as scalars (LDS byte addresses), so that every operand read
  // is one scalar base + the lane's offset + an immediate
  auto stage_ptr = [&](int st) {
    return (const DSA_LDS uint8_t *)tiles + __builtin_amdgcn_readfirstlane(st * kMStageBytes);
  };
  int st_cur = 0, st_prev = kMStages - 1;
  for (int t = 0; t < ntiles; ++t) {
    wait_vmcnt<0>();              // this wave's blocks of tile t have landed
    __syncthreads();              // tile t visible; stage (t + 1) % 3 free
    const int st_next = st_cur == kMStages - 1 ? 0 : st_cur + 1;
    if (defer && t > 0) pv(stage_ptr(st_prev), pk);
    if (t + 1 < ntiles) issue(tl[t + 1], st_next);
    qk_softmax(stage_ptr(st_cur), pk);
    if (!defer) pv(stage_ptr(st_cur), pk);
    st_prev = st_cur;
    st_cur = st_next;
  }
  if (defer && ntiles > 0) pv(stage_ptr(st_prev), pk);

  // ---- epilogue: lane (G, j) holds row j's dims 32 u + 8 (e / 4) + 4 G + e % 4
  const float l_tot = sum_across_halves(l_part);
  if (!row_ok) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  uint16_t *orow = p.out + (row * H + h) * (int64_t)kMV + 4 * G;
#pragma unroll
  for (int u = 0; u < kMV / 32; ++u)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const uint32_t lo = pack_bf16x2(o[u][4 * q4] * inv, o[u][4 * q4 + 1] * inv);
      const uint32_t hi = pack_bf16x2(o[u][4 * q4 + 2] * inv, o[u][4 * q4 + 3] * inv);
      *reinterpret_cast<v2i *>(orow + 32 * u + 8 * q4) = v2i{(int)lo, (int)hi};
    }
  if (p.lse != nullptr && G == 0)
    p.lse[row * H + h] = l_tot > 0.f ? (m_used + log2f(l_tot)) * kLn2 : -INFINITY;
}

}  // namespace

size_t mha_workspace_bytes(const SeqLayout &seq) { return (size_t)mha_layout(seq).total; }

hipError_t launch_mha_prefill(const MhaArgs &a, hipStream_t stream) {
  if (a.seq.total_q == 0) return hipSuccess;
  const MhaLayout L = mha_layout(a.seq);
  uint8_t *base = static_cast<uint8_t *>(a.workspace);
  MhaWs w;
  w.info = reinterpret_cast<int4 *>(base + L.info);
  w.prefix = reinterpret_cast<int32_t *>(base + L.prefix);
  w.count = reinterpret_cast<int32_t *>(base + L.count);
  w.list = reinterpret_cast<int32_t *>(base + L.list);
  w.mask = reinterpret_cast<uint64_t *>(base + L.mask);
  w.nblk = (int32_t)L.nblk;
  w.W = (int32_t)L.W;
  w.seq = a.seq;
  mha_plan_kernel<<<1, 1024, 0, stream>>>(a.seq, w);
  mha_mask_kernel<<<(unsigned)a.seq.total_q, 256, 0, stream>>>(a, w);
  mha_tiles_kernel<<<(unsigned)L.nblk, 512, 0, stream>>>(w);
  const int64_t items = (int64_t)a.heads * L.nblk;
  const int64_t per_xcd = (items + 7) / 8;
  mha_prefill_kernel<<<(unsigned)(8 * per_xcd), kMWaves * 64, 0, stream>>>(a, w);
  return hipGetLastError();
}

}  // namespace dsa
