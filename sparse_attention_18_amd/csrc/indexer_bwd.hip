// Backward of the lightning indexer (training) for gfx950.
//
// The method (ivugangingo.com article on DeepSeek-V3.2, section "DeepSeek
// sparse attention pre-training continues"): the indexer is the part the
// alignment loss trains.  Given that loss's gradient g[t, s] on the scores,
// the chain rule through
//     score(t, s) = sum_j w[t, j] * ReLU(z[t, j, s]),   z = q~[t, j] . k~[s]
// (q~ = q_scale * q8 and k~ = k_scale * k8 dequantised; the ReLU's derivative
// at 0 taken as 0) gives, over the token's keys (its selected set, or every
// causal key in the dense warm-up form):
//     dw[t, j]   = sum_s g[t, s] * ReLU(z[t, j, s])
//     dq~[t, j]  = sum_s E[j, s] * k8[s],      E[j, s] = g[t, s] * w[t, j] * k_scale[s] * [z > 0]
//     dk~[s]    += (q_scale[t] / k_scale[s]) * sum_j E[j, s] * q8[t, j]
//
// MFMA path (H_I = 64, d_I = 128): one workgroup of 8 waves per token; keys
// in 64-key tiles, staged through LDS in three buffers.
//  * z on v_mfma_f32_16x16x128_f8f6f4 straight from the FP8 bytes, so the
//    ReLU mask is decided on the fp32 dot product of the exact e4m3 values.
//  * E is formed in fp32 and split into two bf16 terms (hi + lo carries it to
//    about 2^-17); e4m3 values are exact in bf16.  dq~ = E . K8 and the
//    tile's dk~ block = E^T . Q8 run on v_mfma_f32_16x16x32_bf16 (a hi and a
//    lo product each) with fp32 accumulation; dq stays in registers across
//    the tiles.
//  * dq contracts over keys and dk over heads, so E goes to LDS twice
//    (head-major and key-major), each key tile is transposed once into bf16
//    (dims x keys), and Q8's transpose is built once per token.
//  * A key is selected by many queries, so dk rows of different tokens
//    collide.  Without a workspace each tile's block is added to dk with
//    fp32 atomics; these are resolved beyond the L2 (about one 4-byte write
//    to HBM per atomic), which makes them the kernel's bound.  With one
//    (sparse form), dk is formed in two passes: the token kernel stores each
//    (token, key) contribution, 128 floats, at the key's rank in the token's
//    ascending key list, along with that list and, per 64-key block of the
//    sequence, where the block's keys start in it; then one workgroup per
//    64-key block gathers the contributions to its keys from every token of
//    the sequence, sums them per key in registers and adds the sums to dk
//    (about one atomic per dk element and 4096 tokens instead of one per
//    token that selected the key).
#include <climits>

#include "common.h"
#include "launch.h"

namespace dsa {
namespace {

constexpr int kBT = 256;        // threads per workgroup (fp32 path)
constexpr int kBKeys = 64;      // keys per tile
constexpr int kBMaxK = 4096;

// Byte offset of 16-byte chunk j (of 8) of row n in a tile of 128-byte fp8
// rows; chunks are XOR-swizzled by (n >> 1) & 7 as in the forward indexer.
__device__ __forceinline__ int f8_off(int n, int j) { return n * 128 + 16 * (j ^ ((n >> 1) & 7)); }

// Byte offset of bf16 element c of row r in an array of 64-element (128-byte)
// rows; the 16-byte chunks of row r are XOR-swizzled by (r ^ (r >> 3)) & 7,
// so 16 lanes reading the same chunk of 16 consecutive rows, and the
// transpose writing rows 8 apart, spread over the banks.
__device__ __forceinline__ int b16_off(int r, int c) {
  return r * 128 + ((((c >> 3) ^ r ^ (r >> 3)) & 7) << 4) + (c & 7) * 2;
}

// bf16 bits of a float that is exactly representable (an e4m3 value).
__device__ __forceinline__ uint32_t top16(float f) { return __float_as_uint(f) >> 16; }

// Transpose a [64 rows][128 dims] fp8 tile (f8_off layout) into bf16
// [128 dims][64 rows] (b16_off layout).  Thread: rows 4rg..4rg+3, dims
// 8dg..8dg+7; four 8-byte reads, eight 8-byte writes.
__device__ __forceinline__ void transpose_f8_bf16(const DSA_LDS uint8_t *src, DSA_LDS uint8_t *dst, int tid) {
  const int rg = tid & 15, dg = tid >> 4;
  float f[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const v2i x = *reinterpret_cast<const DSA_LDS v2i *>(src + f8_off(4 * rg + i, dg >> 1) + 8 * (dg & 1));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((uint32_t)x[h], 1.0f, false);
      const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((uint32_t)x[h], 1.0f, true);
      f[i][4 * h + 0] = lo[0];
      f[i][4 * h + 1] = lo[1];
      f[i][4 * h + 2] = hi[0];
      f[i][4 * h + 3] = hi[1];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t a = top16(f[0][e]) | (top16(f[1][e]) << 16);
    const uint32_t b = top16(f[2][e]) | (top16(f[3][e]) << 16);
    *reinterpret_cast<DSA_LDS v2i *>(dst + b16_off(8 * dg + e, 4 * rg)) = v2i{(int)a, (int)b};
  }
}

__device__ __forceinline__ v8bf lds_v8bf(const DSA_LDS uint8_t *p) {
  return __builtin_bit_cast(v8bf, *reinterpret_cast<const DSA_LDS v4i *>(p));
}

// Eight waves, two per SIMD, so that one wave's MFMAs can run while the
// other waits on LDS, on its key loads or (atomic form) on its dk atomics,
// which share the in-order vector-memory counter with those loads.  Wave w:
// z and E for keys 16(w%4).. and head blocks 2(w/4), 2(w/4)+1; dq for heads
// 16(w%4).. and dims 64(w/4)..; the dk block for keys 16(w%4).. and dims
// 64(w/4)..
constexpr int kBW = 8;              // waves per workgroup (MFMA path)
constexpr int kBT8 = kBW * 64;

constexpr int kRKB = 64;   // keys per block of the two-pass dk reduction

// Ascending sort of the token's compacted (position, entry) pairs in LDS,
// bitonic over the next power of two >= m (<= kBMaxK) with INT_MAX padding.
// Called by every thread of the workgroup.
__device__ void sort_keys(int *key, uint16_t *val, int m, int tid) {
  int n2 = 1;
  while (n2 < m) n2 <<= 1;
  for (int i = m + tid; i < n2; i += kBT8) {
    key[i] = INT_MAX;
    val[i] = 0;
  }
  __syncthreads();
  for (int size = 2; size <= n2; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < n2 / 2; i += kBT8) {
        const int lo = 2 * i - (i & (stride - 1)), hi = lo + stride;
        const bool up = (lo & size) == 0;
        const int a = key[lo], b = key[hi];
        if ((a > b) == up) {
          key[lo] = b;
          key[hi] = a;
          const uint16_t t = val[lo];
          val[lo] = val[hi];
          val[hi] = t;
        }
      }
      __syncthreads();
    }
}

// kStore (sparse form only): the two-pass dk; see the file comment.
template <bool kDense, bool kStore>
__global__ __launch_bounds__(kBT8) void indexer_bwd_kernel(IndexerBwdArgs p) {
  static_assert(!(kDense && kStore), "the stored contributions are for the sparse form");
  constexpr int H = 64, D = 128;
  __shared__ __attribute__((aligned(16))) uint8_t ktile[3][kBKeys * 128];
  __shared__ __attribute__((aligned(16))) uint8_t kT[D * 128];          // bf16 [dims][64]
  __shared__ __attribute__((aligned(16))) uint8_t eh[2][H * 128];       // bf16 [heads][keys]: hi, lo
  __shared__ __attribute__((aligned(16))) uint8_t et[2][kBKeys * 128];  // bf16 [keys][heads]: hi, lo
  __shared__ float tks[3][kBKeys], tg[3][kBKeys];
  __shared__ int tpos[3][kBKeys];
  __shared__ int idxl[kDense ? 1 : kBMaxK];
  __shared__ uint16_t slotl[kDense ? 1 : kBMaxK];
  __shared__ int s_scan[kBW];
  __shared__ float sdw[4][H];

  const int64_t t = __builtin_amdgcn_workgroup_id_x();
  const int tid = __builtin_amdgcn_workitem_id_x(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int w4 = wave & 3, wh = wave >> 2;   // key / head-or-dim quarter and half of this wave
  const int r16 = lane & 15, g4 = lane >> 4;
  const int k = p.k;

  SeqInfo s;
  row_seq(p.seq, t, s);
  const bool row_ok = t >= s.q0 && t < s.q1;
  const float qsc = p.q_scale[t];
  const float *grow = p.grad + t * p.ld_grad;

  // z operands (A of 16x16x128) for head blocks hb = 2*wh + i: head
  // hb*16 + r16, dims 32*g4 .. +31; w of the lane's result heads hb*16 + 4*g4 + j.
  v8i qa[2];
  float wv[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int hb = 2 * wh + i;
    const v4i *src = reinterpret_cast<const v4i *>(p.q_fp8 + (t * H + hb * 16 + r16) * (int64_t)D + 32 * g4);
    const v4i lo = src[0], hi = src[1];
    qa[i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
    for (int j = 0; j < 4; ++j) wv[i][j] = p.w[t * H + hb * 16 + 4 * g4 + j];
  }

  // Key set: m keys; sparse, compacted with their entry slots.
  int m;
  if constexpr (!kDense) {
    constexpr int per = kBMaxK / kBT8;
    const int32_t *irow = p.idx + t * k;
    const int i0 = tid * per;
    int vals[per];
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < per; ++e) {
      const int i = i0 + e;
      int v = -1;
      if (row_ok && i < k) v = irow[i];
      vals[e] = (v >= 0 && v < s.kvlen) ? v : -1;
      cnt += vals[e] >= 0;
    }
    const int inc = (int)wave_scan<0>((uint32_t)cnt);
    if (lane == 63) s_scan[wave] = inc;
    __syncthreads();
    int base = inc - cnt;
    m = 0;
#pragma unroll
    for (int w2 = 0; w2 < kBW; ++w2) {
      const int x = s_scan[w2];
      base += w2 < wave ? x : 0;
      m += x;
    }
#pragma unroll
    for (int e = 0; e < per; ++e)
      if (vals[e] >= 0) {
        idxl[base] = vals[e];
        slotl[base] = (uint16_t)(i0 + e);
        ++base;
      }
    __syncthreads();
    if constexpr (kStore) {
      // Contributions go to the key's rank in the ascending list: the
      // top-k's lists already are; others are sorted here.
      int unsorted = 0;
      for (int c = tid; c + 1 < m; c += kBT8) unsorted |= idxl[c] > idxl[c + 1];
      if (__syncthreads_or(unsorted)) sort_keys(idxl, slotl, m, tid);
      int32_t *krow = p.skey + t * p.kpad;
      for (int c = tid; c < m; c += kBT8) krow[c] = idxl[c];
      // bnd[t][jl]: how many of the token's keys lie below the start of the
      // sequence's 64-key block jl (blocks of packed key rows, counted from
      // the one holding the sequence's first key), for jl = 0 .. nb.
      const int64_t jlo = s.kv0 / kRKB;
      const int nb = s.kvlen > 0 ? (int)((s.kv0 + s.kvlen - 1) / kRKB - jlo + 1) : 0;
      int32_t *brow = p.bnd + t * p.nbr;
      for (int jl = tid; jl <= nb; jl += kBT8) {
        const int64_t thr = (jlo + jl) * kRKB - s.kv0;
        int lo = 0, hi = m;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (idxl[mid] < thr) lo = mid + 1;
          else hi = mid;
        }
        brow[jl] = lo;
      }
    }
  } else {
    m = row_ok ? (int)(row_pos(s, t) + 1) : 0;
  }

  // Tile staging: each thread carries one 16-byte chunk of the 64 key rows;
  // threads 0..63 also the key's scale, gradient and position.  Keys past m
  // get zero bytes and a zero gradient (their loads read key m - 1, so every
  // load is issued unconditionally).  Two register sets take turns: the
  // loads for tile i + 2 go out at the start of tile i, into the set tile i
  // came from, and reach LDS at the end of tile i + 1 -- two tiles of work
  // in between, since a gathered row takes longer than one tile to arrive.
  const uint8_t *kseq = p.k_fp8 + s.kv0 * D;
  struct Stage {
    v4i k;
    float ks, g;
    int pos;
  };
  auto fetch = [&](Stage &st, int t0) {
    {
      const int n = tid >> 3, j = tid & 7;
      const int c = t0 + n;
      const int cc = c < m ? c : m - 1;
      const int pos = kDense ? cc : idxl[cc];
      const v4i x = *reinterpret_cast<const v4i *>(kseq + (int64_t)pos * D + 16 * j);
      st.k = c < m ? x : v4i{0, 0, 0, 0};
    }
    const int c = t0 + (tid & (kBKeys - 1));
    const int cc = c < m ? c : m - 1;
    st.pos = kDense ? cc : idxl[cc];
    st.ks = p.k_scale[s.kv0 + st.pos];
    const float gv = grow[kDense ? cc : (int)slotl[cc]];
    st.g = c < m ? gv : 0.f;
  };
  auto commit = [&](const Stage &st, int buf) {
    *reinterpret_cast<v4i *>(&ktile[buf][f8_off(tid >> 3, tid & 7)]) = st.k;
    if (tid < kBKeys) {
      tks[buf][tid] = st.ks;
      tg[buf][tid] = st.g;
      tpos[buf][tid] = st.pos;
    }
  };

  float dw[2][4];
  v4f dq[4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) dw[i][j] = 0.f;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) dq[nb] = v4f{0.f, 0.f, 0.f, 0.f};

  Stage sa, sb;
  if (m > 0) {
    fetch(sa, 0);
    fetch(sb, kBKeys);
    // Q8 transposed to bf16 [dims][heads] (through ktile[2] and kT), then
    // read once as the dk products' B operands: dim 64*wh + nb*16 + r16,
    // heads 32*ks + 8*g4 .. +7.
    *reinterpret_cast<v4i *>(&ktile[2][f8_off(tid >> 3, tid & 7)]) =
        *reinterpret_cast<const v4i *>(p.q_fp8 + (t * H + (tid >> 3)) * (int64_t)D + 16 * (tid & 7));
    commit(sa, 0);
    __syncthreads();
    if (tid < 256) transpose_f8_bf16((const DSA_LDS uint8_t *)ktile[2], (DSA_LDS uint8_t *)kT, tid);
    __syncthreads();
  }
  v8bf qb[4][2];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      qb[nb][ks] = m > 0 ? lds_v8bf((const DSA_LDS uint8_t *)kT + b16_off(64 * wh + nb * 16 + r16, 32 * ks + 8 * g4))
                         : v8bf{};
  __syncthreads();

  const int key_l = 16 * w4 + r16;   // this lane's tile key in the z layout
  float *dkseq = p.dk + s.kv0 * D;
  // One tile: loads for tile + 2 into `ld`, compute from LDS buffer `buf`,
  // then `cm` (tile + 1's data) into the next buffer.
  auto tile_step = [&](int t0, int buf, Stage &ld, const Stage &cm) {
    fetch(ld, t0 + 2 * kBKeys);
    const DSA_LDS uint8_t *kt = (const DSA_LDS uint8_t *)ktile[buf];
    // z for key key_l (B: its dims 32*g4 .. +31) and the wave's two head blocks
    v4f z[2];
    {
      const v4i lo = *reinterpret_cast<const DSA_LDS v4i *>(kt + f8_off(key_l, 2 * g4));
      const v4i hi = *reinterpret_cast<const DSA_LDS v4i *>(kt + f8_off(key_l, 2 * g4 + 1));
      const v8i bop = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
      for (int i = 0; i < 2; ++i) z[i] = mfma_16x16x128_fp8(qa[i], bop, v4f{0.f, 0.f, 0.f, 0.f});
    }
    const float gk = tg[buf][key_l] * tks[buf][key_l];   // g * k_scale of the lane's key
    const float cw = gk * qsc;
    // The mask is decided on the e4m3 dot product, which has the sign of z
    // only when both scales are positive; with a zero scale z is 0 and the
    // ReLU's derivative there is 0.
    const bool sc_pos = qsc > 0.f && tks[buf][key_l] > 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int hb = 2 * wh + i;
      uint32_t hiw[4], low[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float zr = z[i][j];
        dw[i][j] = fmaf(fmaxf(zr, 0.f), cw, dw[i][j]);
        const float e = (zr > 0.f && sc_pos) ? wv[i][j] * gk : 0.f;
        // hi = e rounded to bf16 (round to nearest even), lo = the remainder
        const __bf16 eh16 = (__bf16)e;
        const __bf16 el16 = (__bf16)(e - (float)eh16);
        hiw[j] = __builtin_bit_cast(uint16_t, eh16);
        low[j] = __builtin_bit_cast(uint16_t, el16);
        const int head = hb * 16 + 4 * g4 + j;
        *reinterpret_cast<uint16_t *>(&eh[0][b16_off(head, key_l)]) = (uint16_t)hiw[j];
        *reinterpret_cast<uint16_t *>(&eh[1][b16_off(head, key_l)]) = (uint16_t)low[j];
      }
      const int c0 = hb * 16 + 4 * g4;
      *reinterpret_cast<v2i *>(&et[0][b16_off(key_l, c0)]) =
          v2i{(int)(hiw[0] | (hiw[1] << 16)), (int)(hiw[2] | (hiw[3] << 16))};
      *reinterpret_cast<v2i *>(&et[1][b16_off(key_l, c0)]) =
          v2i{(int)(low[0] | (low[1] << 16)), (int)(low[2] | (low[3] << 16))};
    }
    if (tid < 256) transpose_f8_bf16(kt, (DSA_LDS uint8_t *)kT, tid);
    __syncthreads();

    // dq[heads 16*w4 + ...][dims 64*wh + ...] += E . K8   (K = the tile's keys)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const v8bf ahi = lds_v8bf((const DSA_LDS uint8_t *)eh[0] + b16_off(16 * w4 + r16, 32 * ks + 8 * g4));
      const v8bf alo = lds_v8bf((const DSA_LDS uint8_t *)eh[1] + b16_off(16 * w4 + r16, 32 * ks + 8 * g4));
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const v8bf b = lds_v8bf((const DSA_LDS uint8_t *)kT + b16_off(64 * wh + nb * 16 + r16, 32 * ks + 8 * g4));
        dq[nb] = mfma_16x16x32_bf16(ahi, b, dq[nb]);
        dq[nb] = mfma_16x16x32_bf16(alo, b, dq[nb]);
      }
    }
    // dk block[keys 16*w4 + ...][dims 64*wh + ...] = E^T . Q8   (K = heads)
    v4f dkb[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) dkb[nb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const v8bf ahi = lds_v8bf((const DSA_LDS uint8_t *)et[0] + b16_off(16 * w4 + r16, 32 * ks + 8 * g4));
      const v8bf alo = lds_v8bf((const DSA_LDS uint8_t *)et[1] + b16_off(16 * w4 + r16, 32 * ks + 8 * g4));
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        dkb[nb] = mfma_16x16x32_bf16(ahi, qb[nb][ks], dkb[nb]);
        dkb[nb] = mfma_16x16x32_bf16(alo, qb[nb][ks], dkb[nb]);
      }
    }
    // element j: key 16*w4 + 4*g4 + j, dim 64*wh + nb*16 + r16
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = 16 * w4 + 4 * g4 + j;
      // E already carries k_scale; a zero scale has E = 0 and a zero factor
      const float kscl = tks[buf][key];
      const float f = kscl > 0.f ? qsc / kscl : 0.f;
      if constexpr (kStore) {
        // the key's rank t0 + key < kpad (a multiple of 64 >= k); ranks past
        // m get zeros, which the reduction never reads
        float *crow = p.contrib + (t * p.kpad + t0 + key) * D + 64 * wh + r16;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) __builtin_nontemporal_store(dkb[nb][j] * f, crow + nb * 16);
      } else {
        // keys past m have E = 0: they add zeros to key m - 1's row, which
        // keeps the atomics (vector-memory ops) out of a branch
        float *drow = dkseq + (int64_t)tpos[buf][key] * D + 64 * wh + r16;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) unsafeAtomicAdd(drow + nb * 16, dkb[nb][j] * f);
      }
    }
    commit(cm, buf == 2 ? 0 : buf + 1);
    __syncthreads();
  };
  for (int t0 = 0, buf = 0; t0 < m; t0 += 2 * kBKeys) {
    tile_step(t0, buf, sa, sb);
    buf = buf == 2 ? 0 : buf + 1;
    if (t0 + kBKeys < m) {
      tile_step(t0 + kBKeys, buf, sb, sa);
      buf = buf == 2 ? 0 : buf + 1;
    }
  }

  // dw: sum over the 16 lanes of a row group (keys), then over the four waves
  // that share the head blocks.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v = dw[i][j];
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) v += __shfl_xor(v, off);
      if (r16 == 0) sdw[w4][(2 * wh + i) * 16 + 4 * g4 + j] = v;
    }
  __syncthreads();
  if (!row_ok) return;
  if (tid < H) p.dw[t * H + tid] = (sdw[0][tid] + sdw[1][tid]) + (sdw[2][tid] + sdw[3][tid]);
  // dq: element j of block nb is head 16*w4 + 4*g4 + j, dim 64*wh + nb*16 + r16
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float *qrow = p.dq + (t * H + 16 * w4 + 4 * g4 + j) * (int64_t)D + 64 * wh + r16;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) qrow[nb * 16] = dq[nb][j];
  }
}

// Second pass of the two-pass dk: one workgroup per block of 64 packed key
// rows.  For every sequence whose keys overlap the block, its tokens are
// taken 4096 at a time: each token's run of ranks [bnd[jl], bnd[jl + 1]) in
// its ascending key list is exactly its keys in the block, so an exclusive
// scan of the run lengths numbers the window's (token, key) pairs.  Pairs
// are then handled kRCap at a time: every token writes its index over its
// run (pair -> token), every pair's key and contribution offset are found
// once, and a counting sort by key lays the offsets out key by key.  The
// sorted pairs are split evenly over the 16 half-waves (key popularity
// varies, so a split by key would leave most of them waiting for one); each
// walks its slice, kRU pairs in flight, summing a run of one key's pairs in
// registers and adding the run's 128 sums to the key's dk row when the key
// changes -- an fp32 atomic, since a key's run can straddle two slices, but
// about one per key and batch instead of one per (token, key) pair.  With
// few blocks (an early chunk of a long prefill) each block's tokens are
// split over nsplit workgroups, so that the grid still fills the chip.
// Workgroup ids are laid out so that consecutive blocks run on one XCD and
// share the bnd lines in its L2.
constexpr int kRWin = 4096;            // tokens per scan window
constexpr int kRCap = 4096;            // pairs per batch
constexpr int kRT = 512;
constexpr int kRHW = kRT / 32;         // half-waves
constexpr int kRU = 8;
static_assert(kRCap % kRT == 0, "whole pair slots per thread");

__global__ __launch_bounds__(kRT) void dk_reduce_kernel(IndexerBwdArgs p, int nblk, int nsplit, int per) {
  constexpr int D = 128, PER = kRCap / kRT;
  __shared__ int s_lo[kRWin], s_ex[kRWin + 1];
  __shared__ uint16_t s_row[kRCap];
  __shared__ int s_soff[kRCap];          // (token - w0) * kpad + rank, sorted by key
  __shared__ int s_bin[kRKB + 1], s_cur[kRKB];
  __shared__ int s_wsum[kRT / 64];
  __shared__ int s_b0;
  const int wid = __builtin_amdgcn_workgroup_id_x();
  const int lin = (wid & 7) * per + (wid >> 3);
  const int j = lin / nsplit, split = lin - j * nsplit;
  if (j >= nblk) return;
  const int tid = __builtin_amdgcn_workitem_id_x(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hw = tid >> 5, l32 = tid & 31;
  const int64_t G0 = (int64_t)j * kRKB;
  const int64_t G1 = G0 + kRKB < p.seq.total_kv ? G0 + kRKB : p.seq.total_kv;
  // first sequence whose keys end after G0 (key offsets are non-decreasing)
  if (wave == 0) {
    int cnt = 0;
    for (int base = 0; base < p.seq.batch; base += 64) {
      const int b = base + lane;
      const bool le = b < p.seq.batch && (int64_t)p.seq.kv_offsets[b + 1] <= G0;
      cnt += __popcll(__ballot(le));
    }
    if (lane == 0) s_b0 = cnt;
  }
  __syncthreads();
  for (int b = s_b0; b < p.seq.batch; ++b) {
    const SeqInfo s = load_seq(p.seq, b);
    if (s.kv0 >= G1) break;
    if (s.kvlen == 0 || s.kv0 + s.kvlen <= G0) continue;
    const int jl = (int)(j - s.kv0 / kRKB);   // 0 <= jl < the sequence's block count
    // this workgroup's share of the sequence's tokens
    const int64_t nq = s.q1 - s.q0;
    const int64_t qa = s.q0 + nq * split / nsplit, qb = s.q0 + nq * (split + 1) / nsplit;
    for (int64_t w0 = qa; w0 < qb; w0 += kRWin) {
      const int nrow = (int)(qb - w0 < kRWin ? qb - w0 : kRWin);
      // thread: tokens 8*tid .. +7 of the window; runs clamped into [0, kpad]
      int lo8[8], len8[8], sum = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 8 * tid + e;
        int lo = 0, hi = 0;
        if (i < nrow) {
          const int32_t *br = p.bnd + (w0 + i) * p.nbr + jl;
          lo = br[0];
          hi = br[1];
          lo = lo < 0 ? 0 : (lo > p.kpad ? p.kpad : lo);
          hi = hi < lo ? lo : (hi > p.kpad ? p.kpad : hi);
        }
        lo8[e] = lo;
        len8[e] = hi - lo;
        sum += hi - lo;
      }
      const int inc = (int)wave_scan<0>((uint32_t)sum);
      if (lane == 63) s_wsum[wave] = inc;
      __syncthreads();
      int before = inc - sum, P = 0;
#pragma unroll
      for (int w2 = 0; w2 < kRT / 64; ++w2) {
        const int x = s_wsum[w2];
        before += w2 < wave ? x : 0;
        P += x;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 8 * tid + e;
        if (i < nrow) {
          s_lo[i] = lo8[e];
          s_ex[i] = before;
        }
        before += len8[e];
      }
      if (tid == 0) s_ex[nrow] = P;
      __syncthreads();
      const int64_t cbase = w0 * p.kpad;
      for (int P0 = 0; P0 < P; P0 += kRCap) {
        const int np = P - P0 < kRCap ? P - P0 : kRCap;
        // pair -> token over this batch
        for (int e = 0; e < 8; ++e) {
          const int i = 8 * tid + e;
          if (i >= nrow) break;
          const int a = s_ex[i], b2 = s_ex[i + 1];
          const int x0 = a > P0 ? a : P0;
          const int x1 = b2 < P0 + np ? b2 : P0 + np;
          for (int x = x0; x < x1; ++x) s_row[x - P0] = (uint16_t)i;
        }
        if (tid < kRKB) s_bin[tid] = 0;
        __syncthreads();
        // each pair's contribution offset and key (an index into the block;
        // -1: not in it), then the key histogram
        int off8[PER], key8[PER];
#pragma unroll
        for (int r = 0; r < PER; ++r) {
          const int x = tid + kRT * r;
          key8[r] = -1;
          off8[r] = 0;
          if (x < np) {
            const int i = s_row[x];
            off8[r] = i * p.kpad + s_lo[i] + (P0 + x - s_ex[i]);
            const int64_t l = s.kv0 + p.skey[cbase + off8[r]] - G0;
            key8[r] = (l >= 0 && l < kRKB) ? (int)l : -1;
          }
        }
#pragma unroll
        for (int r = 0; r < PER; ++r)
          if (key8[r] >= 0) __hip_atomic_fetch_add(&s_bin[key8[r]], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __syncthreads();
        if (wave == 0) {
          const int c = lane < kRKB ? s_bin[lane] : 0;
          const int incl = (int)wave_scan<0>((uint32_t)c);
          if (lane < kRKB) {
            s_bin[lane] = incl - c;
            s_cur[lane] = incl - c;
          }
          if (lane == kRKB - 1) s_bin[kRKB] = incl;
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < PER; ++r)
          if (key8[r] >= 0) {
            const int at = __hip_atomic_fetch_add(&s_cur[key8[r]], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            s_soff[at] = off8[r];
          }
        __syncthreads();
        // this half-wave's slice [x0, x1) of the sorted pairs; key of slot x:
        // the last key with s_bin[key] <= x
        const int T = s_bin[kRKB];
        const int x0 = T * hw / kRHW, x1 = T * (hw + 1) / kRHW;
        if (x0 < x1) {
          int key = 0;
#pragma unroll
          for (int st = kRKB / 2; st >= 1; st >>= 1)
            if (s_bin[key + st] <= x0) key += st;
          int next = s_bin[key + 1];
          float run[4] = {0.f, 0.f, 0.f, 0.f};
          auto flush = [&]() {
            float *dst = p.dk + (G0 + key) * D + l32;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              unsafeAtomicAdd(dst + 32 * q, run[q]);
              run[q] = 0.f;
            }
          };
          for (int base = x0; base < x1; base += kRU) {
            float v[kRU][4];
#pragma unroll
            for (int u = 0; u < kRU; ++u) {
              const int xi = base + u < x1 ? base + u : x1 - 1;
              const float *src = p.contrib + (cbase + s_soff[xi]) * D + l32;
#pragma unroll
              for (int q = 0; q < 4; ++q) v[u][q] = __builtin_nontemporal_load(src + 32 * q);
            }
#pragma unroll
            for (int u = 0; u < kRU; ++u) {
              const int xi = base + u;
              if (xi < x1) {
                if (xi >= next) {   // a new key (keys with no pairs are skipped)
                  flush();
                  do {
                    ++key;
                    next = s_bin[key + 1];
                  } while (xi >= next);
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) run[q] += v[u][q];
              }
            }
          }
          flush();
        }
        __syncthreads();   // s_row, s_bin and s_soff are rewritten by the next batch
      }
      __syncthreads();     // the next window rewrites s_lo, s_ex and s_wsum
    }
  }
}

// Generic path: any H_I <= 128 and d_I <= 128; one workgroup per token,
// fp32 arithmetic on the dequantised values, keys in chunks of 32.
constexpr int kSBKeys = 32;
constexpr int kSBMaxQ = 64;     // dq entries per thread: H_I * d_I <= 128 * 128 = 64 * 256

template <bool kDense>
__global__ __launch_bounds__(kBT) void small_indexer_bwd_kernel(IndexerBwdArgs p) {
  __shared__ float qd[128 * 128];           // q~ [H][d]
  __shared__ float kc[kSBKeys][128];        // k~ of the chunk's keys
  __shared__ float ec[128][kSBKeys];        // E = g * w * [z > 0]
  __shared__ float rc[128][kSBKeys];        // g * ReLU(z)
  __shared__ float gc[kSBKeys];
  __shared__ int pc[kSBKeys];
  __shared__ int rows[kDense ? 1 : kBMaxK];
  __shared__ int nvalid;
  const int64_t t = blockIdx.x;
  SeqInfo s;
  row_seq(p.seq, t, s);
  if (t < s.q0 || t >= s.q1) return;
  const int H = p.idx_heads, D = p.idx_dim, k = p.k, tid = threadIdx.x;
  const float qsc = p.q_scale[t];
  const float *grow = p.grad + t * p.ld_grad;
  for (int i = tid; i < H * D; i += kBT) {
    const uint32_t byte = p.q_fp8[t * H * (int64_t)D + i];
    qd[i] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(byte, 1.0f, false)[0] * qsc;
  }
  // key list: dense, positions 0..pos; sparse, the valid entries in slot order
  int n;
  if (kDense) {
    n = (int)(row_pos(s, t) + 1);
  } else {
    if (tid == 0) {
      int c = 0;
      for (int i = 0; i < k; ++i) {
        const int v = p.idx[t * k + i];
        if (v >= 0 && v < s.kvlen) rows[c++] = i;   // the slot; its position is idx[slot]
      }
      nvalid = c;
    }
    __syncthreads();
    n = nvalid;
  }
  float dqa[kSBMaxQ];
#pragma unroll
  for (int i = 0; i < kSBMaxQ; ++i) dqa[i] = 0.f;
  float dwa = 0.f;
  for (int c0 = 0; c0 < n; c0 += kSBKeys) {
    __syncthreads();
    if (tid < kSBKeys) {
      const int c = c0 + tid;
      int pos = 0;
      float g = 0.f;
      if (c < n) {
        const int slot = kDense ? c : rows[c];
        pos = kDense ? c : p.idx[t * k + slot];
        g = grow[slot];
      }
      pc[tid] = pos;
      gc[tid] = g;
    }
    __syncthreads();
    for (int i = tid; i < kSBKeys * D; i += kBT) {
      const int c = i / D, d = i % D;
      const uint32_t byte = p.k_fp8[(s.kv0 + pc[c]) * (int64_t)D + d];
      kc[c][d] = c0 + c < n ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(byte, 1.0f, false)[0] *
                                  p.k_scale[s.kv0 + pc[c]]
                            : 0.f;
    }
    __syncthreads();
    for (int i = tid; i < H * kSBKeys; i += kBT) {
      const int j = i / kSBKeys, c = i % kSBKeys;
      float z = 0.f;
      for (int d = 0; d < D; ++d) z = fmaf(qd[j * D + d], kc[c][d], z);
      ec[j][c] = z > 0.f ? gc[c] * p.w[t * H + j] : 0.f;
      rc[j][c] = gc[c] * fmaxf(z, 0.f);
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kSBMaxQ; ++q) {
      const int i = tid + kBT * q;
      if (i < H * D) {
        const int j = i / D, d = i % D;
        float a = dqa[q];
        for (int c = 0; c < kSBKeys; ++c) a = fmaf(ec[j][c], kc[c][d], a);
        dqa[q] = a;
      }
    }
    for (int i = tid; i < kSBKeys * D; i += kBT) {
      const int c = i / D, d = i % D;
      if (c0 + c >= n) continue;
      float a = 0.f;
      for (int j = 0; j < H; ++j) a = fmaf(ec[j][c], qd[j * D + d], a);
      unsafeAtomicAdd(p.dk + (s.kv0 + pc[c]) * (int64_t)D + d, a);
    }
    if (tid < H)
      for (int c = 0; c < kSBKeys; ++c) dwa += rc[tid][c];
  }
#pragma unroll
  for (int q = 0; q < kSBMaxQ; ++q) {
    const int i = tid + kBT * q;
    if (i < H * D) p.dq[t * H * (int64_t)D + i] = dqa[q];
  }
  if (tid < H) p.dw[t * H + tid] = dwa;
}

}  // namespace

namespace {

// Two-pass workspace: contributions [total_q][kpad][128] f32 | ascending key
// lists [total_q][kpad] i32 | block starts [total_q][nbr] i32.
struct BwdWs {
  size_t contrib, skey, bnd, total;
  int32_t kpad, nbr;
};

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

BwdWs bwd_ws(const IndexerBwdArgs &a) {
  BwdWs w;
  w.kpad = (a.k + kBKeys - 1) / kBKeys * kBKeys;
  w.nbr = (int32_t)((a.seq.max_kv_len + kRKB - 1) / kRKB + 2);
  const size_t rows = (size_t)a.seq.total_q;
  w.contrib = round256(rows * (size_t)w.kpad * 128 * sizeof(float));
  w.skey = round256(rows * (size_t)w.kpad * sizeof(int32_t));
  w.bnd = round256(rows * (size_t)w.nbr * sizeof(int32_t));
  w.total = w.contrib + w.skey + w.bnd;
  return w;
}

}  // namespace

size_t indexer_bwd_workspace_bytes(const IndexerBwdArgs &a) {
  if (a.seq.total_q == 0 || a.idx_heads != 64 || a.idx_dim != 128) return 0;
  return bwd_ws(a).total;
}

hipError_t launch_indexer_backward(const IndexerBwdArgs &a0, hipStream_t stream) {
  if (a0.seq.total_q == 0) return hipSuccess;
  IndexerBwdArgs a = a0;
  const dim3 grid((unsigned)a.seq.total_q), block(kBT);
  const bool dense = a.idx == nullptr;
  if (a.idx_heads == 64 && a.idx_dim == 128) {
    if (dense) {
      hipLaunchKernelGGL((indexer_bwd_kernel<true, false>), grid, dim3(kBT8), 0, stream, a);
    } else if (a.workspace != nullptr) {
      const BwdWs w = bwd_ws(a);
      uint8_t *base = static_cast<uint8_t *>(a.workspace);
      a.contrib = reinterpret_cast<float *>(base);
      a.skey = reinterpret_cast<int32_t *>(base + w.contrib);
      a.bnd = reinterpret_cast<int32_t *>(base + w.contrib + w.skey);
      a.kpad = w.kpad;
      a.nbr = w.nbr;
      hipLaunchKernelGGL((indexer_bwd_kernel<false, true>), grid, dim3(kBT8), 0, stream, a);
      if (a.seq.total_kv > 0) {
        // at least about 2048 workgroups (two per CU, four rounds) when the
        // blocks alone are fewer
        const int nblk = (int)((a.seq.total_kv + kRKB - 1) / kRKB);
        int nsplit = (2048 + nblk - 1) / nblk;
        nsplit = nsplit > 64 ? 64 : nsplit;
        const int per = (int)(((int64_t)nblk * nsplit + 7) / 8);
        hipLaunchKernelGGL(dk_reduce_kernel, dim3(8 * (unsigned)per), dim3(kRT), 0, stream, a, nblk, nsplit, per);
      }
    } else {
      hipLaunchKernelGGL((indexer_bwd_kernel<false, false>), grid, dim3(kBT8), 0, stream, a);
    }
  } else {
    if (dense) hipLaunchKernelGGL(small_indexer_bwd_kernel<true>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(small_indexer_bwd_kernel<false>, grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace dsa
