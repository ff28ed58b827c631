// Indexer alignment loss (training) for gfx950.
//
// The method (ivugangingo.com article on DeepSeek-V3.2, section "DeepSeek
// sparse attention pre-training continues"): the lightning indexer is trained
// with a Kullback-Leibler loss towards the main attention's distribution --
// over all causal keys while dense attention is still in use (the warm-up),
// over the selected keys once the selector is on.  The pages give no formula;
// this library computes, for query token t with key set K_t:
//   target   p_s = (1/H) sum_h exp(logit[h, s] - lse[h])            s in K_t
//   indexer  q_s = exp(I[t, s]) / sum_{s' in K_t} exp(I[t, s'])
//   loss[t]  = sum_s p_s (ln p_s - ln q_s),   d loss[t] / d I[t, s] = q_s - p_s
// with logit = scale * q_h . kv_s as in the sparse attention and lse[h] that
// attention's log-sum-exp over the same K_t: each head's softmax then sums to
// one, and 1/H is the L1 normalisation of their sum.  Only the indexer side
// is differentiated.
//
// MFMA path (D = 576, H = 32 * NW): one workgroup of NW waves per token.
//  * Key rows come into LDS 32 at a time in the sparse attention's tile
//    layout and LDS-DMA gather, two tiles ahead of use (three buffers): this
//    pass has half the attention's arithmetic per row, so each tile needs
//    longer in flight.  A tile's 32 indexer scores come by LDS-DMA as well
//    (each lane loads the aligned group of four holding its score), so no
//    register load is outstanding across a step and the vector-memory waits
//    only ever cover the tile due next.
//  * S = Q . K^T on v_mfma_f32_32x32x16_bf16: M = the wave's 32 heads (Q
//    resident in registers), N = the 32 keys, K = 576 in two independent
//    accumulation chains.  A lane holds one key and 16 heads, so the head sum
//    is in-lane plus one exchange between the wave's halves; the waves'
//    partial sums meet in LDS.
//  * One wave (round-robin over tiles) finishes a tile during the next step:
//    p, q, the gradient entries and its share of the loss.
#include "common.h"
#include "kv_gather.h"
#include "launch.h"

namespace dsa {
namespace {

constexpr int kAStages = 3;      // key tiles: one in use, two in flight
constexpr int kSStages = 4;      // score groups: also the tile being finished
constexpr int kAMaxK = 4096;

// Merge the pair (m2, s2) into (m, s), where s = sum of exp2(x - m) over a set.
__device__ __forceinline__ void merge_ms(float &m, float &s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  s = M == -INFINITY ? 0.f
                     : s * __builtin_amdgcn_exp2f(m - M) + s2 * __builtin_amdgcn_exp2f(m2 - M);
  m = M;
}

// Block-wide merge of every thread's (m, s); all threads get the result.  The
// caller synchronises before `red` is written again.
template <int NW>
__device__ __forceinline__ void block_merge_ms(float &m, float &s, float2 *red, int lane, int wave) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
    merge_ms(m, s, m2, s2);
  }
  if (lane == 0) red[wave] = make_float2(m, s);
  __syncthreads();
  m = red[0].x;
  s = red[0].y;
#pragma unroll
  for (int w = 1; w < NW; ++w) merge_ms(m, s, red[w].x, red[w].y);
}

template <int NW>
__device__ __forceinline__ float block_sum(float v, float *red, int lane, int wave) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) r += red[w];
  return r;
}

template <int NW, bool kDense>
__global__ __launch_bounds__(NW * 64) void align_loss_kernel(AlignArgs p) {
  constexpr int H = NW * 32;
  constexpr int T = NW * 64;
  constexpr int KS = kD / 16;                 // 36 MFMA k-steps
  constexpr int kRB = 4 / NW;                 // 8-row blocks of a tile per wave
  constexpr int kWindows = 3 * kRB;
  constexpr int kOps = 9 * kRB + 1;           // DMA instructions per wave and tile
  static_assert(kOps < 64, "vmcnt range");
  __shared__ __attribute__((aligned(16))) uint8_t kvbuf[kAStages][kTileBytes];
  __shared__ __attribute__((aligned(16))) float ivb[kSStages][NW][64 * 4];
  __shared__ int idxl[kDense ? 1 : kAMaxK];
  __shared__ uint16_t slotl[kDense ? 1 : kAMaxK];
  __shared__ float psum[2][NW][32];
  __shared__ float2 s_ms[NW];
  __shared__ int s_scan[NW];
  __shared__ float s_loss[NW];

  const int64_t t = __builtin_amdgcn_workgroup_id_x();
  const int tid = __builtin_amdgcn_workitem_id_x(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = lane >> 5, c32 = lane & 31;
  const int k = p.k;

  // A operands: lane (G, c32) holds head 32*wave + c32, dims 16kk + 8G .. +7.
  v8bf qa[KS];
  {
    const uint16_t *qrow = p.q + (t * H + wave * 32 + c32) * (int64_t)kD + 8 * G;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) qa[kk] = as_v8bf(*reinterpret_cast<const v4i *>(qrow + 16 * kk));
  }
  // lse (log2 units) of the heads of this lane's S elements: element jj is
  // head 8(jj/4) + 4G + jj%4 of the wave.
  float lse2[16];
  {
    const float *lrow = p.lse + t * H + wave * 32 + 4 * G;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const v4f x = *reinterpret_cast<const v4f *>(lrow + 8 * j);
#pragma unroll
      for (int i = 0; i < 4; ++i) lse2[4 * j + i] = x[i] * kLog2e;
    }
  }

  SeqInfo s;
  row_seq(p.seq, t, s);
  const bool row_ok = t >= s.q0 && t < s.q1;
  const float *srow = p.scores + t * p.ld_scores;
  float *grow = p.grad + t * p.ld_grad;

  // The key set (m keys; sparse: compacted, with their entry slots) and the
  // indexer softmax statistics over it, in log2 units.
  int m;
  float im = -INFINITY, is = 0.f;
  if constexpr (!kDense) {
    constexpr int per = kAMaxK / T;
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
#pragma unroll
    for (int e = 0; e < per; ++e) {
      const int i = i0 + e;
      if (row_ok && i < k && vals[e] < 0) grow[i] = 0.f;   // skipped entries
      if (vals[e] >= 0) merge_ms(im, is, srow[vals[e]] * kLog2e, 1.f);
    }
    const int inc = (int)wave_scan<0>((uint32_t)cnt);
    if (lane == 63) s_scan[wave] = inc;
    __syncthreads();
    int base = inc - cnt;
    m = 0;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) {
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
  } else {
    m = row_ok ? (int)(row_pos(s, t) + 1) : 0;
#pragma unroll 8
    for (int i = tid; i < m; i += T) merge_ms(im, is, srow[i] * kLog2e, 1.f);
  }
  block_merge_ms<NW>(im, is, s_ms, lane, wave);   // its barrier also publishes idxl
  const float lse_i = im + log2f(is);             // log2 of the indexer's normaliser
  const int ntiles = (m + kBN - 1) / kBN;
  wait_vmcnt<0>();   // register loads complete before any LDS-DMA is in flight

  auto key_pos = [&](int r) { return kDense ? r : idxl[r]; };
  // Gather of tile tl: this wave's row blocks wave + NW*q (as in the sparse
  // attention, rows past m repeat the last key), plus the tile's scores.
  // Sequence rows are addressed with 32-bit byte offsets (the host bounds
  // max_kv_len * 1152 below 2^32).
  const uint8_t *kvseq = reinterpret_cast<const uint8_t *>(p.kv + s.kv0 * (int64_t)kD);
  auto gather_setup = [&](int tl, uint32_t (&voff)[kRB]) {
#pragma unroll
    for (int q = 0; q < kRB; ++q) {
      const int row = 8 * (wave + NW * q) + (lane >> 3);
      const int r = tl * kBN + row;
      voff[q] = (uint32_t)key_pos(r < m ? r : m - 1) * (uint32_t)(kD * 2) +
                16 * ((lane & 7) ^ ((row >> 1) & 7));
    }
    // scores: lane l takes the 16-byte group holding key c32's score; rows
    // hold a multiple of four scores and start 16-byte aligned, so the group
    // lies inside the row.
    const int r = tl * kBN + c32;
    const uint32_t soff = (uint32_t)(key_pos(r < m ? r : m - 1) & ~3) * 4u;
    lds_dma16_x1(soff, sbase(srow),
                 __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(DSA_LDS float *)ivb[tl % kSStages][wave]));
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(DSA_LDS uint8_t *)kvbuf[tl % kAStages]);
  };
  auto gather_window = [&](const uint32_t (&voff)[kRB], uint32_t base, int w) {
    const int q = w / 3, win = w % 3;
    const uint32_t lb = __builtin_amdgcn_readfirstlane(base + ((wave + NW * q) * kGroups + 4 * win) * kBlock);
    const uint8_t *g = kvseq + 128 * 4 * win;      // chunk group 4*win
    if (win < 2)
      lds_dma16_x4(voff[q], sbase(g), sbase(g + 128 - 1024), sbase(g + 256 - 2048), sbase(g + 384 - 3072), lb);
    else
      lds_dma16_x1(voff[q], sbase(g), lb);
  };

  const float sl2 = p.scale * kLog2e;
  float loss2 = 0.f;   // this lane's share of the loss, log2 units
  if (ntiles > 0) {
#pragma unroll
    for (int tl = 0; tl < 2; ++tl)
      if (tl < ntiles) {
        uint32_t vo[kRB];
        const uint32_t gb = gather_setup(tl, vo);
#pragma unroll
        for (int w = 0; w < kWindows; ++w) gather_window(vo, gb, w);
      }
    // Step tt: tile tt's S (gathering tile tt + 2 along the way), after
    // finishing tile tt - 1.  Tiles tt and tt + 1 were issued earlier, so
    // only tile tt + 1's loads may still be in flight at the top.
    for (int tt = 0; tt <= ntiles; ++tt) {
      if (tt + 1 < ntiles) wait_vmcnt<kOps>();
      else wait_vmcnt<0>();
      __syncthreads();
      if (tt > 0) {
        const int tf = tt - 1;
        if (wave == tf % NW && lane < 32) {
          const int c = tf * kBN + lane;
          if (c < m) {
            float ps = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) ps += psum[tf & 1][w2][lane];
            ps *= 1.f / H;
            const int pos = key_pos(c);
            const float iv = ivb[tf % kSStages][wave][4 * lane + (pos & 3)];
            const float d2 = fmaf(iv, kLog2e, -lse_i);   // log2 q
            if (ps > 0.f) loss2 += ps * (log2f(ps) - d2);
            grow[kDense ? c : slotl[c]] = __builtin_amdgcn_exp2f(d2) - ps;
          }
        }
      }
      if (tt < ntiles) {
        const bool g2 = tt + 2 < ntiles;
        uint32_t vo[kRB];
        uint32_t gb = 0;
        if (g2) gb = gather_setup(tt + 2, vo);
        const DSA_LDS uint8_t *tb = (const DSA_LDS uint8_t *)kvbuf[tt % kAStages];
        v16f s0 = {}, s1 = {};
        // B operands read LA k-steps ahead: the scheduling barrier below keeps
        // each step's instructions in place, so a read issued right before its
        // MFMA would expose the LDS latency at every step
        constexpr int LA = 4;
        v4i bq[LA];
#pragma unroll
        for (int kk = 0; kk < LA; ++kk)
          bq[kk] = *reinterpret_cast<const DSA_LDS v4i *>(tb + tile_off(c32, 2 * kk + G));
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          const v4i b = bq[kk % LA];
          if (kk + LA < KS)
            bq[kk % LA] = *reinterpret_cast<const DSA_LDS v4i *>(tb + tile_off(c32, 2 * (kk + LA) + G));
          if (kk & 1) s1 = mfma_32x32x16_bf16(qa[kk], as_v8bf(b), s1);
          else s0 = mfma_32x32x16_bf16(qa[kk], as_v8bf(b), s0);
          if (g2)
#pragma unroll
            for (int w = 0; w < kWindows; ++w)
              if (kk == w * KS / kWindows) gather_window(vo, gb, w);
          __builtin_amdgcn_sched_barrier(0);
        }
        // head sum for key c32: raw v_exp_f32 (arguments below -126 give 0,
        // a probability under 2^-126 next to the head's total of 1)
        float ph[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jj = 0; jj < 16; ++jj)
          ph[jj & 3] += __builtin_amdgcn_exp2f(fmaf(s0[jj] + s1[jj], sl2, -lse2[jj]));
        const float part = sum_across_halves((ph[0] + ph[1]) + (ph[2] + ph[3]));
        if (G == 0) psum[tt & 1][wave][c32] = part;
      }
    }
  }
  const float tot = block_sum<NW>(loss2, s_loss, lane, wave);
  if (tid == 0 && row_ok) p.loss[t] = tot * kLn2;
}

// Small-shape path: any H <= 128 and D <= 1024; one workgroup per token,
// plain fp32 dot products.
constexpr int kSmallT = 256;

template <bool kDense>
__global__ __launch_bounds__(kSmallT) void small_align_loss_kernel(AlignArgs p) {
  __shared__ int rows[kDense ? 1 : kAMaxK];
  __shared__ float2 s_ms[kSmallT / 64];
  __shared__ float s_loss[kSmallT / 64];
  const int64_t t = blockIdx.x;
  SeqInfo s;
  row_seq(p.seq, t, s);
  if (t < s.q0 || t >= s.q1) return;
  const int H = p.heads, D = p.d_latent + p.d_rope, k = p.k;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float *srow = p.scores + t * p.ld_scores;
  float *grow = p.grad + t * p.ld_grad;
  // entries to visit: dense, positions 0..pos; sparse, the k slots
  const int n = kDense ? (int)(row_pos(s, t) + 1) : k;
  float im = -INFINITY, is = 0.f;
  for (int i = tid; i < n; i += kSmallT) {
    int pos = i;
    if (!kDense) {
      const int v = p.idx[t * k + i];
      pos = (v >= 0 && v < s.kvlen) ? v : -1;
      rows[i] = pos;
    }
    if (pos >= 0) merge_ms(im, is, srow[pos] * kLog2e, 1.f);
  }
  block_merge_ms<kSmallT / 64>(im, is, s_ms, lane, wave);
  const float lse_i = im + log2f(is);
  const uint16_t *qt = p.q + t * H * (int64_t)D;
  const float *lt = p.lse + t * H;
  float loss2 = 0.f;
  for (int i = tid; i < n; i += kSmallT) {
    const int pos = kDense ? i : rows[i];
    if (pos < 0) {
      grow[i] = 0.f;
      continue;
    }
    const uint16_t *kr = p.kv + (s.kv0 + pos) * (int64_t)D;
    float ps = 0.f;
    for (int h = 0; h < H; ++h) {
      float acc = 0.f;
      for (int d = 0; d < D; ++d) acc = fmaf(bf16_bits_to_f32(qt[h * D + d]), bf16_bits_to_f32(kr[d]), acc);
      ps += expf(acc * p.scale - lt[h]);
    }
    ps /= (float)H;
    const float d2 = fmaf(srow[pos], kLog2e, -lse_i);
    if (ps > 0.f) loss2 += ps * (log2f(ps) - d2);
    grow[i] = exp2f(d2) - ps;
  }
  const float tot = block_sum<kSmallT / 64>(loss2, s_loss, lane, wave);
  if (tid == 0) p.loss[t] = tot * kLn2;
}

bool mfma_align_shape(const AlignArgs &a) {
  return a.d_latent == kDL && a.d_rope == kD - kDL &&
         (a.heads == 32 || a.heads == 64 || a.heads == 128);
}

template <int NW>
void launch_mfma(const AlignArgs &a, hipStream_t stream) {
  const dim3 grid((unsigned)a.seq.total_q), block(NW * 64);
  if (a.idx == nullptr) hipLaunchKernelGGL((align_loss_kernel<NW, true>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((align_loss_kernel<NW, false>), grid, block, 0, stream, a);
}

}  // namespace

hipError_t launch_align_loss(const AlignArgs &a, hipStream_t stream) {
  if (a.seq.total_q == 0) return hipSuccess;
  if (mfma_align_shape(a)) {
    switch (a.heads / 32) {
      case 1: launch_mfma<1>(a, stream); break;
      case 2: launch_mfma<2>(a, stream); break;
      default: launch_mfma<4>(a, stream); break;
    }
  } else {
    const dim3 grid((unsigned)a.seq.total_q);
    if (a.idx == nullptr) hipLaunchKernelGGL(small_align_loss_kernel<true>, grid, dim3(kSmallT), 0, stream, a);
    else hipLaunchKernelGGL(small_align_loss_kernel<false>, grid, dim3(kSmallT), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace dsa
