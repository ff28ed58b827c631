// Sparse MQA/MLA attention over the selected KV rows, for gfx950.
//
// The method (ivugangingo.com article on DeepSeek-V3.2, "Sparse attention with
// almost linear long-context costs"): after the selector keeps the top-k key
// positions of a query, the main attention path runs MQA and MLA over that
// sparse set only.  Here every head of a token shares one latent KV row per
// key: the key is the whole row (latent + rope, D wide), the value its latent
// part.  logit = scale * q_h . kv_s; out_h = softmax-weighted sum of the
// latent parts; lse_h = log of the softmax denominator.
//
// MFMA path (d_latent = 512, d_rope = 64, H = 32 * NW heads), one workgroup
// of NW waves per query token:
//  * the token's valid indices are compacted once into LDS; its selected
//    rows are then gathered 32 at a time straight into LDS with LDS-DMA loads
//    (global_load_lds, 16-byte chunks), three tiles in flight; every head of
//    the token shares this one gather.  A tile is a sequence of 1 KB blocks,
//    row-block major: block (r / 8) * 9 + c / 8 holds chunks 8(c/8)..+7 of
//    rows 8(r/8)..+7, and 16-byte chunk c of row r sits in it at slot
//    (r % 8) * 8 + ((c % 8) ^ ((r >> 1) & 7)).  One DMA load fills one block,
//    so a wave's loads need one row index per tile and immediate offsets; a
//    wave's 9 blocks of a row block are consecutive, so one M0 value serves
//    four loads (the instruction offset moves the LDS destination and the
//    global source alike).  MFMA operand reads of 16 consecutive rows hit 16
//    distinct bank groups;
//  * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16: wave w takes heads
//    32w..32w+31 (N), Q^T resident in registers, the 32 keys of the tile as
//    M and the 576 dims as K;
//  * softmax in the S^T layout: a lane holds one head, so the running max and
//    sum need one cross-half exchange per tile.  The exponent frame is fixed
//    at the first tile's max and never rescaled; a later tile exceeding it by
//    more than 2^32 flags the token, which is then recomputed in the frame of
//    its true maximum (exact, and only reachable with extreme logits);
//  * P^T (bf16) goes through LDS, so that O^T = V^T . P^T can be split by
//    latent dims instead of heads: wave w owns dims (512/NW)w .. and all H
//    heads.  V^T comes from the row-major tile through ds_read_b64_tr_b16,
//    whose rate is well below ds_read_b128 -- with the dims split each V
//    element is read through it once per workgroup rather than once per wave.
//
// Few tokens (decode): the token's compacted index list is cut into nsplit
// contiguous ranges, one workgroup each, so that the batch fills the chip.
// Each range's workgroup writes its unnormalised O (fp16 with a power-of-two
// scale per head and wave), its exponent frame and its softmax denominator
// per head to the workspace; a small combine kernel then
// rescales the ranges to their common maximum frame (the usual merge of
// partial softmax sums) and writes out and lse.
#include <type_traits>

#include "common.h"
#include "kv_gather.h"
#include "launch.h"

namespace dsa {
namespace {

constexpr int kStages = 3;
constexpr int kMaxK = 4096;
constexpr float kFrameSlack = 32.f;          // log2 headroom above the frame max
constexpr int kMaxSplits = 4;                // workgroups per token in the split path
constexpr int kMaxWaves = 4;                 // scales per (split, token, head) in the split path
// S^T links before the first gather window of a step: kLeadPrefill with one
// workgroup per token, 0 in the split (few-token) path, whose gathers come
// from a cache far larger than the MALL and want every cycle of lead time
constexpr int kLeadPrefill = 10;

// Two floats to fp16 bits (round to nearest even), packed low | high.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}

// S^T accumulation MFMAs, pinned to VGPRs.  The P.V accumulators fill all
// 256 AGPRs; left to itself the compiler puts this accumulator in AGPRs too
// and spills part of O.  The chain's dependent MFMAs are interlocked by the
// hardware; the chain ends in qk_mfma_last_drain, which waits for the result.
__device__ __forceinline__ void qk_mfma_first(v16f &acc, const v4i &a, const v8bf &b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk_mfma(v16f &acc, const v4i &a, const v8bf &b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
// The last link of the chain, with the wait for its result, in one asm
// statement: the compiler takes an asm's result as ready and its sources as
// free once it issues, so an instruction placed between a separate last link
// and its wait could read sums still in flight (a copy of the accumulator)
// or overwrite C, which the matrix core reads late in the instruction.  The
// output is not tied to the accumulator, so that no copy is needed after it.
__device__ __forceinline__ v16f qk_mfma_last_drain(const v16f &acc, const v4i &a, const v8bf &b) {
  v16f r;
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3\n\ts_nop 15\n\ts_nop 15"
               : "=&v"(r) : "v"(a), "v"(b), "v"(acc) : "memory");
  return r;
}

template <int NW, bool kPaged, int kGatherLead>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_sparse_attn_kernel(AttnArgs p) {
  constexpr int H = NW * 32;
  constexpr int T = NW * 64;                 // threads
  constexpr int DW = kDL / NW;               // latent dims per wave in P.V
  constexpr int MB = DW / 32;                // 32-dim M blocks per wave
  static_assert(DW * NW == kDL && MB * 32 == DW, "latent dims must split evenly over waves");
  static_assert(kTileInsts % NW == 0, "tile loads must split evenly over waves");
  __shared__ __attribute__((aligned(16))) uint8_t kvbuf[kStages][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t pbuf[2][NW * 2 * 1024];
  __shared__ int idxl[kMaxK];
  __shared__ float lsum[H];
  __shared__ int s_scan[NW];
  __shared__ int s_flag;

  // Raw ids: this kernel is large enough that the ockl wrappers behind
  // blockIdx/threadIdx are not reliably inlined.
  // Workgroup id = split * total_q + token: when total_q is a multiple of 8
  // the splits of a token share an XCD (ids go round-robin over the 8 XCDs),
  // so its Q rows are read once into that XCD's L2.
  const int64_t wg = __builtin_amdgcn_workgroup_id_x();
  const int split = (int)(wg / p.seq.total_q);
  const int64_t t = wg - (int64_t)split * p.seq.total_q;
  // The wave index is uniform: readfirstlane keeps everything derived from
  // it (LDS block bases, M0 values) in scalar registers.
  const int tid = __builtin_amdgcn_workitem_id_x(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = lane >> 5, c32 = lane & 31, jl = lane & 15, half = (lane >> 4) & 1;
  const int k = p.k;

  // Loads go out in this order: the row's index entries, the sequence
  // search's offsets, then the Q^T operands.  The vector memory counter
  // completes in issue order, so the wait for the first two groups leaves the
  // Q^T loads in flight through the sequence lookup, the compaction and the
  // first tile's gather.  All of them are unconditional (clamped addresses),
  // so the compiler counts them exactly.
  constexpr int per = kMaxK / T;             // entries per thread (k <= kMaxK)
  int raw[per];
  {
    const int32_t *idx_row = p.idx + t * k;  // row t < total_q: in bounds
    const int i0 = tid * per;
#pragma unroll
    for (int e = 0; e < per; ++e) raw[e] = idx_row[i0 + e < k ? i0 + e : k - 1];
  }
  int soff[4];
  find_seq_issue(p.seq, soff);
  __builtin_amdgcn_sched_barrier(0);
  // Q^T operands of this wave's heads: k-step kk = dims 16kk..16kk+15, lane
  // (G, c32) holds head 32*wave + c32, dims 16kk + 8G .. +7.
  const int head = wave * 32 + c32;
  v8bf qb[kD / 16];
  {
    const uint16_t *qrow = p.q + (t * H + head) * (int64_t)kD + 8 * G;
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk)
      qb[kk] = as_v8bf(*reinterpret_cast<const v4i *>(qrow + 16 * kk));
  }
  __builtin_amdgcn_sched_barrier(0);

  SeqInfo s;
  const int b = row_seq_issued(p.seq, t, soff, s);
  const bool row_ok = t >= s.q0 && t < s.q1;

  // Compact the row's valid indices (in order) into idxl; m = their count.
  int m;
  {
    const int i0 = tid * per;
    int vals[per];
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < per; ++e) {
      const int v = (row_ok && i0 + e < k) ? raw[e] : -1;
      vals[e] = (v >= 0 && v < s.kvlen) ? v : -1;
      cnt += vals[e] >= 0;
    }
    if (kPaged) {
      // positions become cache rows here, once per token (rows < 2^31)
#pragma unroll
      for (int e = 0; e < per; ++e)
        if (vals[e] >= 0) vals[e] = (int)kv_row<true>(p.pg, s, b, vals[e]);
    }
    const int inc = (int)wave_scan<0>((uint32_t)cnt);
    if (lane == 63) s_scan[wave] = inc;
    if (tid == 0) s_flag = 0;
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
      if (vals[e] >= 0) idxl[base++] = vals[e];
    __syncthreads();
  }
  // This workgroup's range of the compacted list: whole tiles, split evenly.
  const int chunk = (((m + p.nsplit - 1) / p.nsplit) + kBN - 1) / kBN * kBN;
  const int r_begin = split * chunk < m ? split * chunk : m;
  const int r_end = r_begin + chunk < m ? r_begin + chunk : m;
  const int nrows = r_end - r_begin;
  const int ntiles = (nrows + kBN - 1) / kBN;
  const int *idxr = idxl + r_begin;

  // Gather of tile `tl` into its stage buffer; rows past m repeat a valid
  // row.  This wave owns row blocks rb = wave + NW*q (q < kRB); the load of
  // chunk group cg of row block rb fills block rb*9 + cg: lane (row 8rb +
  // lane/8, slot lane%8) receives logical chunk 8cg + ((lane%8) ^ f(row)).
  // A row block's 9 loads go out as three windows (groups 0-3, 4-7, 8), one
  // M0 value each.
  constexpr int kRB = 4 / NW;
  constexpr int kWindows = 3 * kRB;
  // Uniform sequence base; a row's byte offset fits in 32 bits (the host
  // bounds max_kv_len * 1152 below 2^32 for this path).  Paged caches: each
  // lane's row address is a full 64-bit value (GOff).
  using GOff = typename std::conditional<kPaged, uint64_t, uint32_t>::type;
  const uint8_t *kvseq = reinterpret_cast<const uint8_t *>(p.kv + (kPaged ? 0 : s.kv0 * (int64_t)kD));
  auto gather_setup = [&](int tl, GOff (&voff)[kRB]) {
#pragma unroll
    for (int q = 0; q < kRB; ++q) {
      const int row = 8 * (wave + NW * q) + (lane >> 3);
      const int r = tl * kBN + row;
      const int gi = idxr[r < nrows ? r : 0];
      const uint32_t in_row = 16 * ((lane & 7) ^ ((row >> 1) & 7));
      if constexpr (kPaged)
        voff[q] = (uint64_t)(uintptr_t)kvseq + (uint64_t)(uint32_t)gi * (uint64_t)(kD * 2) + in_row;
      else
        voff[q] = (uint32_t)gi * (uint32_t)(kD * 2) + in_row;
    }
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(DSA_LDS uint8_t *)kvbuf[tl % kStages]);
  };
  // Window w: row block wave + NW*(w/3), chunk groups 4*(w%3) .. (+3, or 8).
  auto gather_window = [&](const GOff (&voff)[kRB], uint32_t base, int w) {
    const int q = w / 3, win = w % 3;
    const uint32_t lb = __builtin_amdgcn_readfirstlane(base + ((wave + NW * q) * kGroups + 4 * win) * kBlock);
    if constexpr (kPaged) {
      const uint64_t a = voff[q] + 128 * 4 * win;   // chunk group 4*win
      if (win < 2)
        lds_dma16v_x4(a, a + 128 - 1024, a + 256 - 2048, a + 384 - 3072, lb);
      else
        lds_dma16v_x1(a, lb);
    } else {
      const uint8_t *g = kvseq + 128 * 4 * win;      // chunk group 4*win
      if (win < 2)
        lds_dma16_x4(voff[q], sbase(g), sbase(g + 128 - 1024), sbase(g + 256 - 2048), sbase(g + 384 - 3072), lb);
      else
        lds_dma16_x1(voff[q], sbase(g), lb);
    }
  };

  const float sl2 = p.scale * kLog2e;
  float m_used = -INFINITY;   // exponent frame of this lane's head (log2 units)
  float m_seen = -INFINITY;   // true running max of this lane's head
  float l_part = 0.f;
  v16f o[MB][NW];

  // Per-lane in-tile byte offsets.  QK operand for k-step kk: row c32,
  // logical chunk 2kk + G -> group kk/4 (added as an immediate) and in-group
  // slot (2(kk%4) + G) ^ f(c32).  V^T operand for (hf, u): rows r0 = 16hf +
  // 4G + jl/4 and r0 + 8, dims wave*DW + 32u + 16*half + 4*(jl%4), i.e. group
  // wave*DW/64 + u/2, in-group index 4(u%2) + 2*half + (jl/2)%2, byte 8*(jl%2).
  const int fq = (c32 >> 1) & 7;
  auto qk_off = [&](int kk) {
    return (c32 >> 3) * kRowBlockBytes + ((c32 & 7) * 8 + ((2 * (kk & 3) + G) ^ fq)) * 16 + kBlock * (kk >> 2);
  };
  auto v_off = [&](int hf, int u, int which) {
    const int r = 16 * hf + 4 * G + (jl >> 2) + 8 * which;
    const int in = (4 * (u & 1) + 2 * half + ((jl >> 1) & 1)) ^ ((r >> 1) & 7);
    return (r >> 3) * kRowBlockBytes + (wave * DW / 64 + (u >> 1)) * kBlock + ((r & 7) * 8 + in) * 16 +
           (jl & 1) * 8;
  };
  auto load_v = [&](const DSA_LDS uint8_t *tb, int hf, int u) {
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DSA_LDS v4s *)(tb + v_off(hf, u, 0)));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DSA_LDS v4s *)(tb + v_off(hf, u, 1)));
    const v2i lo2 = __builtin_bit_cast(v2i, lo), hi2 = __builtin_bit_cast(v2i, hi);
    return as_v8bf(v4i{lo2[0], lo2[1], hi2[0], hi2[1]});
  };
  auto load_p = [&](const DSA_LDS uint8_t *pb, int hf, int nb) {
    return *reinterpret_cast<const DSA_LDS v8bf *>(pb + ((nb * 2 + hf) * 64 + lane) * 16);
  };

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int u = 0; u < MB; ++u)
#pragma unroll
      for (int nb = 0; nb < NW; ++nb) o[u][nb] = v16f{};
    l_part = 0.f;
    bool overflow = false;

    // ---- one pipeline step: S^T of tile `tq` interleaved with
    // O^T[dims of this wave][all heads] += V^T . P^T of the previous tile
    // (tile buffer tbp, P^T buffer pbp).  The two are independent, so
    // alternating their MFMAs hides the dependent-issue latency of the S^T
    // accumulation chain.  The next tile's gather (when `gnext`) goes out in
    // a few windows along the way.
    auto step_phase = [&](int tq, const DSA_LDS uint8_t *tbp, const DSA_LDS uint8_t *pbp, bool gnext) {
      constexpr int KS = kD / 16, LA = 3, NPV = 2 * MB * NW;
      static_assert(NPV <= KS, "P.V MFMAs ride along the S^T chain");
      // Window w of the next tile's gather goes out after link
      // w * KS / kWindows + kGatherLead of the chain (the last link at the
      // latest).  Right after the step's barrier its LDS writes land among
      // the step's first operand reads: on the last 128K chunk a lead of 10
      // of the 36 links was the fastest (1-3 % per launch); the decode
      // split path, gathering from HBM, is 2 % faster without a lead.
      auto gather_link = [](int w) {
        const int at = w * KS / kWindows + kGatherLead;
        return at < KS ? at : KS - 1;
      };
      const DSA_LDS uint8_t *tbq = (const DSA_LDS uint8_t *)kvbuf[tq % kStages];
      GOff src[kRB];
      uint32_t gbase = 0;
      if (gnext) gbase = gather_setup(tq + 1, src);
      v16f sc;
      v4i a[LA];
#pragma unroll
      for (int kk = 0; kk < LA; ++kk) a[kk] = *reinterpret_cast<const DSA_LDS v4i *>(tbq + qk_off(kk));
      // P.V MFMA i: group g = i / NW = hf * MB + u, head block nb = i % NW.
      v8bf pbn[NW], av[2];
#pragma unroll
      for (int nb = 0; nb < NW; ++nb) pbn[nb] = load_p(pbp, 0, nb);
      av[0] = load_v(tbp, 0, 0);
#pragma unroll
      for (int i = 0; i < KS; ++i) {
        if (i == 0) qk_mfma_first(sc, a[0], qb[0]);
        else if (i + 1 < KS) qk_mfma(sc, a[i % LA], qb[i]);
        else sc = qk_mfma_last_drain(sc, a[i % LA], qb[i]);
        if (i + LA < KS) a[i % LA] = *reinterpret_cast<const DSA_LDS v4i *>(tbq + qk_off(i + LA));
        if (i < NPV) {
          const int g = i / NW, nb = i % NW, hf = g / MB, u = g % MB;
          if (nb == 0 && g + 1 < 2 * MB) av[(g + 1) & 1] = load_v(tbp, (g + 1) / MB, (g + 1) % MB);
          o[u][nb] = mfma_32x32x16_bf16(av[g & 1], pbn[nb], o[u][nb]);
          // last use of this head block's P^T for hf = 0: fetch the hf = 1 one
          if (hf == 0 && u == MB - 1) pbn[nb] = load_p(pbp, 1, nb);
        }
        if (gnext)
#pragma unroll
          for (int w = 0; w < kWindows; ++w)
            if (i == gather_link(w)) gather_window(src, gbase, w);
        __builtin_amdgcn_sched_barrier(0);
      }
      return sc;
    };

    // ---- softmax of tile tq: scale + mask + max, frame update, exp2 + sum
    // + bf16, publish P^T into pbuf[tq & 1].
    // The logits stay unscaled until the exponent: scale * log2(e) > 0, so
    // the maximum of the raw values times it is the scaled maximum, and the
    // scaling rides on the FMA that forms the exponent's argument.
    auto sm_scale = [&](v16f &sc, int tq, int j0, int j1, float &mt) {
      const int valid_rows = nrows - tq * kBN;   // >= 1
      const bool partial = valid_rows < kBN; // only the last tile can be partial
      if (partial) {
        const int vr = valid_rows - 4 * G;      // element jj is row 8(jj/4) + 4G + jj%4
#pragma unroll
        for (int jj = j0; jj < j1; ++jj)
          if (8 * (jj >> 2) + (jj & 3) >= vr) sc[jj] = -INFINITY;
      }
#pragma unroll
      for (int jj = j0; jj < j1; ++jj) mt = fmaxf(mt, sc[jj]);
    };
    auto sm_frame = [&](float mt) {
      mt = max_across_halves(mt) * sl2;
      m_seen = fmaxf(m_seen, mt);
      if (m_used == -INFINITY) m_used = mt;          // first tile
      overflow |= mt > m_used + kFrameSlack;
    };
    auto sm_exp = [&](const v16f &sc, v8bf (&pb)[2], int j0, int j1) {
      float ls[4] = {0.f, 0.f, 0.f, 0.f};   // four short sum chains instead of one long one
#pragma unroll
      for (int jj = j0; jj < j1; ++jj) {
        // raw v_exp_f32: arguments below -126 flush to 0, which a softmax
        // weight that small is anyway next to the frame maximum's 1.0
        const float pe = __builtin_amdgcn_exp2f(fmaf(sc[jj], sl2, -m_used));
        ls[jj & 3] += pe;
        pb[jj >> 3][jj & 7] = (__bf16)pe;
      }
      l_part += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    };
    auto sm_store = [&](const v8bf (&pb)[2], int tq) {
      uint8_t *pw = pbuf[tq & 1];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        *reinterpret_cast<v8bf *>(pw + ((wave * 2 + hf) * 64 + lane) * 16) = pb[hf];
    };

    // Pipeline: tile t's rows are gathered during step t-1; step t runs S^T
    // of tile t together with P.V of tile t-1, then tile t's softmax.
    // Three tile buffers: t-1 (P.V), t (S^T), t+1 (in flight); two P buffers.
    // One barrier per step publishes tile t and P(t-1) and frees the buffers
    // step t+1 overwrites.  The first step's P.V multiplies a zero P^T (P
    // buffer 1, cleared below) with tile 0's rows; the last step's S^T is
    // discarded -- one code path for every step.
    {
      uint8_t *pz = pbuf[1] + tid * (sizeof(pbuf[1]) / T);
#pragma unroll
      for (int e = 0; e < (int)(sizeof(pbuf[1]) / T / 16); ++e)
        reinterpret_cast<v4i *>(pz)[e] = v4i{0, 0, 0, 0};
    }
    if (ntiles > 0) {
      {
        GOff src[kRB];
        const uint32_t gbase = gather_setup(0, src);
#pragma unroll
        for (int w = 0; w < kWindows; ++w) gather_window(src, gbase, w);
      }
      for (int t = 0; t <= ntiles; ++t) {
        // This wave's share of tile t landed (nothing is in flight at the last
        // step).  Unconditional, so that the compiler also knows no vector
        // memory op of its own is pending inside the loop.
        wait_vmcnt<0>();
        __syncthreads();                  // tile t and P(t-1) visible; buffer (t+1)%3 free
        const int tp = t > 0 ? t - 1 : 0;
        const DSA_LDS uint8_t *tbp = (const DSA_LDS uint8_t *)kvbuf[tp % kStages];
        const DSA_LDS uint8_t *pbp = (const DSA_LDS uint8_t *)pbuf[t > 0 ? (tp & 1) : 1];
        v16f sc = step_phase(t, tbp, pbp, t + 1 < ntiles);
        if (t < ntiles) {
          float mt = -INFINITY;
          v8bf pb[2];
          sm_scale(sc, t, 0, 16, mt);
          sm_frame(mt);
          sm_exp(sc, pb, 0, 16);
          sm_store(pb, t);
        }
      }
    }
    // A frame overflow anywhere: redo the token in the frame of its true max.
    if (__ballot(overflow) != 0ull && lane == 0) atomicOr(&s_flag, 1);
    __syncthreads();
    const bool again = s_flag != 0;
    __syncthreads();
    if (!again) break;
    m_used = m_seen;
    if (tid == 0) s_flag = 0;
  }

  const float l_tot = sum_across_halves(l_part);
  if (p.nsplit > 1) {
    // ---- partial epilogue: the frame and denominator per head, and the
    // unnormalised O^T in fp16 (round to nearest) after a power-of-two scale
    // per (head, wave) that brings the wave's DW dims of the head into
    // [-1, 1]: 2^-11 relative per element, and no overflow for any finite O.
    if (!row_ok) return;
    const int64_t slot = (int64_t)split * p.seq.total_q + t;
    const int64_t nslot = (int64_t)p.nsplit * p.seq.total_q;
    uint16_t *wo = reinterpret_cast<uint16_t *>(p.workspace) + slot * H * (int64_t)kDL;
    float2 *wml = reinterpret_cast<float2 *>(reinterpret_cast<uint16_t *>(p.workspace) + nslot * H * kDL);
    float *wsc = reinterpret_cast<float *>(wml + nslot * H);
    if (G == 0) wml[slot * H + head] = make_float2(m_used, l_tot);
#pragma unroll
    for (int nb = 0; nb < NW; ++nb) {
      float mx = 0.f;
#pragma unroll
      for (int u = 0; u < MB; ++u)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, fabsf(o[u][nb][j]));
      mx = max_across_halves(mx);   // the head's other half of the wave's dims
      // mx = f 2^e with f in [0.5, 1); e is clamped so both 2^e and 2^-e are
      // normal floats (a head whose values are all below 2^-100 keeps zeros)
      int e = mx > 0.f ? __builtin_amdgcn_frexp_expf(mx) : 0;
      e = e < -100 ? -100 : e;
      const float inv = ldexpf(1.f, -e);
      if (G == 0) wsc[(slot * H + nb * 32 + c32) * kMaxWaves + wave] = ldexpf(1.f, e);
      uint16_t *ohead = wo + (nb * 32 + c32) * (int64_t)kDL + wave * DW + 4 * G;
#pragma unroll
      for (int u = 0; u < MB; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t w0 = pack_f16x2(o[u][nb][4 * i] * inv, o[u][nb][4 * i + 1] * inv);
          const uint32_t w1 = pack_f16x2(o[u][nb][4 * i + 2] * inv, o[u][nb][4 * i + 3] * inv);
          *reinterpret_cast<v2i *>(ohead + 32 * u + 8 * i) = v2i{(int)w0, (int)w1};
        }
    }
    return;
  }

  // ---- epilogue: denominators through LDS, normalise, store bf16
  if (G == 0) lsum[head] = l_tot;
  if (p.lse != nullptr && G == 0 && row_ok)
    p.lse[t * H + head] = l_tot > 0.f ? (m_used + log2f(l_tot)) * kLn2 : -INFINITY;
  __syncthreads();
  if (!row_ok) return;
  uint16_t *orow = p.out + t * H * (int64_t)kDL;
#pragma unroll
  for (int nb = 0; nb < NW; ++nb) {
    const float lt = lsum[nb * 32 + c32];
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    uint16_t *ohead = orow + (nb * 32 + c32) * (int64_t)kDL + wave * DW + 4 * G;
#pragma unroll
    for (int u = 0; u < MB; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w0 = pack_bf16x2(o[u][nb][4 * i + 0] * inv, o[u][nb][4 * i + 1] * inv);
        const uint32_t w1 = pack_bf16x2(o[u][nb][4 * i + 2] * inv, o[u][nb][4 * i + 3] * inv);
        *reinterpret_cast<v2i *>(ohead + 32 * u + 8 * i) = v2i{(int)w0, (int)w1};
      }
  }
}

// Merge of the nsplit partial results of a token (MFMA path, nsplit > 1):
// with frames m_s (log2 units), denominators l_s and unnormalised O_s,
//   M = max_s m_s,  e_s = 2^(m_s - M),  out = sum_s e_s O_s / sum_s e_s l_s,
//   lse = (M + log2 sum_s e_s l_s) * ln 2.
// One workgroup of 128 threads per (token, head); thread i owns dims 4i..4i+3.
__global__ __launch_bounds__(128) void combine_splits_kernel(AttnArgs p, int heads) {
  const int64_t th = __builtin_amdgcn_workgroup_id_x();     // token * heads + head
  const int tid = (int)__builtin_amdgcn_workitem_id_x();
  const int64_t t = th / heads;
  SeqInfo s;
  const int b = row_seq(p.seq, t, s);
  if (t < s.q0 || t >= s.q1) return;
  const int S = p.nsplit;   // 2..kMaxSplits
  const int64_t per_split = p.seq.total_q * heads;
  const uint16_t *wo = reinterpret_cast<const uint16_t *>(p.workspace);
  const float2 *wml = reinterpret_cast<const float2 *>(wo + (int64_t)S * per_split * kDL);
  const float *wsc = reinterpret_cast<const float *>(wml + (int64_t)S * per_split);
  const int wv = 4 * tid / (kDL / (heads / 32));   // the wave that held these dims
  // Every split's loads are issued before any is used (clamped to the last
  // split past S, whose weight is then zero).
  float2 ml[kMaxSplits];
  float sc[kMaxSplits];
  v2i x[kMaxSplits];
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp) {
    const int64_t at = (int64_t)(sp < S ? sp : S - 1) * per_split + th;
    ml[sp] = wml[at];
    sc[sp] = wsc[at * kMaxWaves + wv];
    x[sp] = *reinterpret_cast<const v2i *>(wo + at * kDL + 4 * tid);
  }
  float M = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp) M = fmaxf(M, ml[sp].x);
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int sp = 0; sp < kMaxSplits; ++sp) {
      const float e = (sp < S && ml[sp].x != -INFINITY) ? __builtin_amdgcn_exp2f(ml[sp].x - M) : 0.f;
      L = fmaf(e, ml[sp].y, L);
      const float f = e * sc[sp];
      const v4f v = {(float)__builtin_bit_cast(_Float16, (uint16_t)((uint32_t)x[sp][0] & 0xFFFFu)),
                     (float)__builtin_bit_cast(_Float16, (uint16_t)((uint32_t)x[sp][0] >> 16)),
                     (float)__builtin_bit_cast(_Float16, (uint16_t)((uint32_t)x[sp][1] & 0xFFFFu)),
                     (float)__builtin_bit_cast(_Float16, (uint16_t)((uint32_t)x[sp][1] >> 16))};
      acc = acc + f * v;
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const uint32_t w0 = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  const uint32_t w1 = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<v2i *>(p.out + th * kDL + 4 * tid) = v2i{(int)w0, (int)w1};
  if (tid == 0 && p.lse != nullptr) p.lse[th] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

// Small-shape path: any H <= 128 and D <= 1024.  One workgroup per token;
// plain fp32 dot products, one head at a time.
constexpr int kSmallThreads = 256;
constexpr int kSmallMaxD = 1024;
constexpr int kSmallMaxK = 4096;

template <bool kPaged>
__global__ __launch_bounds__(kSmallThreads) void small_sparse_attn_kernel(AttnArgs p) {
  __shared__ float qs[kSmallMaxD];
  __shared__ float prob[kSmallMaxK];
  __shared__ int rows[kSmallMaxK];
  __shared__ float red[kSmallThreads / 64];
  const int64_t t = blockIdx.x;
  SeqInfo s;
  const int b = row_seq(p.seq, t, s);
  if (t < s.q0 || t >= s.q1) return;
  const int H = p.heads, D = p.d_latent + p.d_rope, DL = p.d_latent, k = p.k;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < k; i += kSmallThreads) {
    const int v = p.idx[t * k + i];
    // cache row (packed: relative to the sequence's first row)
    rows[i] = (v >= 0 && v < s.kvlen) ? (kPaged ? (int)kv_row<true>(p.pg, s, b, v) : v) : -1;
  }
  auto block_reduce = [&](float v, bool is_max) {
    for (int d = 32; d >= 1; d >>= 1) {
      const float o = __shfl_xor(v, d, 64);
      v = is_max ? fmaxf(v, o) : v + o;
    }
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < kSmallThreads / 64; ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
    return r;
  };
  for (int h = 0; h < H; ++h) {
    __syncthreads();
    for (int d = tid; d < D; d += kSmallThreads) qs[d] = bf16_bits_to_f32(p.q[(t * H + h) * D + d]);
    __syncthreads();
    float mx = -INFINITY;
    for (int i = tid; i < k; i += kSmallThreads) {
      float x = -INFINITY;
      if (rows[i] >= 0) {
        const uint16_t *kr = p.kv + ((kPaged ? 0 : s.kv0) + rows[i]) * (int64_t)D;
        float acc = 0.f;
        for (int d = 0; d < D; ++d) acc = fmaf(qs[d], bf16_bits_to_f32(kr[d]), acc);
        x = acc * p.scale;
      }
      prob[i] = x;
      mx = fmaxf(mx, x);
    }
    mx = block_reduce(mx, true);
    float sum = 0.f;
    for (int i = tid; i < k; i += kSmallThreads) {
      const float e = rows[i] >= 0 ? expf(prob[i] - mx) : 0.f;
      prob[i] = e;
      sum += e;
    }
    sum = block_reduce(sum, false);
    const float inv = sum > 0.f ? 1.f / sum : 0.f;
    if (tid == 0 && p.lse != nullptr) p.lse[t * H + h] = sum > 0.f ? mx + logf(sum) : -INFINITY;
    for (int d = tid; d < DL; d += kSmallThreads) {
      float acc = 0.f;
      for (int i = 0; i < k; ++i)
        if (rows[i] >= 0) acc = fmaf(prob[i], bf16_bits_to_f32(p.kv[((kPaged ? 0 : s.kv0) + rows[i]) * (int64_t)D + d]), acc);
      p.out[(t * H + h) * DL + d] = (uint16_t)f32_to_bf16_bits(acc * inv);
    }
  }
}

bool mfma_shape(const AttnArgs &a) {
  // The latent dims split evenly over NW waves only for NW in {1, 2, 4}.
  return a.d_latent == kDL && a.d_rope == kD - kDL &&
         (a.heads == 32 || a.heads == 64 || a.heads == 128);
}

// Workgroups per token: enough that a small batch still covers the 256 CUs
// (at most kMaxSplits).
int attn_splits(const AttnArgs &a) {
  if (!mfma_shape(a) || a.seq.total_q == 0) return 1;
  const int64_t s = 256 / a.seq.total_q;
  return s >= kMaxSplits ? kMaxSplits : (s >= 2 ? 2 : 1);
}

template <int NW>
void launch_mla(const AttnArgs &a, bool paged, bool split, dim3 grid, hipStream_t stream) {
  const dim3 block(NW * 64);
  if (paged) {
    if (split) hipLaunchKernelGGL((mla_sparse_attn_kernel<NW, true, 0>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((mla_sparse_attn_kernel<NW, true, kLeadPrefill>), grid, block, 0, stream, a);
  } else {
    if (split) hipLaunchKernelGGL((mla_sparse_attn_kernel<NW, false, 0>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((mla_sparse_attn_kernel<NW, false, kLeadPrefill>), grid, block, 0, stream, a);
  }
}

}  // namespace

size_t sparse_attn_workspace_bytes(const AttnArgs &a) {
  const int S = attn_splits(a);
  if (S == 1) return 0;
  // per (split, token, head): 512 fp16 values, frame and denominator, and
  // kMaxWaves scales
  return (size_t)S * a.seq.total_q * a.heads * (kDL * sizeof(uint16_t) + (2 + kMaxWaves) * sizeof(float));
}

hipError_t launch_sparse_attn(const AttnArgs &args, hipStream_t stream) {
  if (args.seq.total_q == 0) return hipSuccess;
  AttnArgs a = args;
  a.nsplit = attn_splits(a);
  if (a.nsplit > 1 && (a.workspace == nullptr || a.workspace_bytes < sparse_attn_workspace_bytes(a)))
    return hipErrorInvalidValue;   // the ABI layer checks the size first
  const dim3 grid((unsigned)(a.seq.total_q * a.nsplit));
  const bool paged = a.pg.table != nullptr;
  if (mfma_shape(a)) {
    const bool split = a.nsplit > 1;
    switch (a.heads / 32) {
      case 1:
        launch_mla<1>(a, paged, split, grid, stream);
        break;
      case 2:
        launch_mla<2>(a, paged, split, grid, stream);
        break;
      default:
        launch_mla<4>(a, paged, split, grid, stream);
        break;
    }
    if (a.nsplit > 1)
      hipLaunchKernelGGL(combine_splits_kernel, dim3((unsigned)(a.seq.total_q * a.heads)), dim3(128), 0,
                         stream, a, (int)a.heads);
  } else {
    if (paged) hipLaunchKernelGGL(small_sparse_attn_kernel<true>, grid, dim3(kSmallThreads), 0, stream, a);
    else hipLaunchKernelGGL(small_sparse_attn_kernel<false>, grid, dim3(kSmallThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace dsa
