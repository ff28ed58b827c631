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
//  * the token's selected rows are gathered 32 at a time straight into LDS
//    with global_load_lds (16-byte chunks); every head of the token shares
//    this one gather.  Row pitch 1152 B with the chunk index XOR-swizzled by
//    (row >> 1) & 7 keeps the MFMA operand reads free of bank conflicts;
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
#include "common.h"
#include "launch.h"

namespace dsa {
namespace {

constexpr int kD = 576;                      // latent + rope
constexpr int kDL = 512;                     // latent (value) width
constexpr int kBN = 32;                      // keys per tile
constexpr int kChunks = kD * 2 / 16;         // 72 chunks of 16 B per row
constexpr int kPitch = kChunks * 16;         // 1152 B
constexpr int kTileBytes = kBN * kPitch;     // 36864 B
constexpr int kTileInsts = kBN * kChunks / 64;  // 36 wave-wide 1 KB loads per tile
constexpr int kStages = 2;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kFrameSlack = 32.f;          // log2 headroom above the frame max
static_assert(kBN * kChunks % 64 == 0, "tile must be whole 1 KB loads");

__device__ __forceinline__ v8bf as_v8bf(const v4i &x) { return __builtin_bit_cast(v8bf, x); }

// Physical 16-byte slot of logical chunk c in tile row r (self-inverse).
__device__ __forceinline__ int swz(int r, int c) { return (c & ~7) | ((c ^ (r >> 1)) & 7); }

template <int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_sparse_attn_kernel(AttnArgs p) {
  constexpr int H = NW * 32;
  constexpr int DW = kDL / NW;               // latent dims per wave in P.V
  constexpr int MB = DW / 32;                // 32-dim M blocks per wave
  static_assert(DW * NW == kDL && MB * 32 == DW, "latent dims must split evenly over waves");
  __shared__ __attribute__((aligned(16))) uint8_t kvbuf[kStages][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t pbuf[NW * 2 * 1024];
  __shared__ float lsum[H];
  __shared__ int s_ntiles, s_flag;

  const int64_t t = blockIdx.x;
  const int b = find_seq(p.seq, t);
  const SeqInfo s = load_seq(p.seq, b);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = lane >> 5, c32 = lane & 31, jl = lane & 15, half = (lane >> 4) & 1;
  const int k = p.k;
  const int32_t *idx_row = p.idx + t * k;
  const bool row_ok = t >= s.q0 && t < s.q1;

  // Tiles to visit: up to the last valid index of the row.
  if (tid == 0) {
    s_ntiles = 0;
    s_flag = 0;
  }
  __syncthreads();
  {
    int last = -1;
    if (row_ok)
      for (int i = tid; i < k; i += NW * 64) {
        const int v = idx_row[i];
        if (v >= 0 && v < s.kvlen) last = i;
      }
    for (int d = 32; d >= 1; d >>= 1) last = max(last, __shfl_xor(last, d, 64));
    if (lane == 0) atomicMax(&s_ntiles, (last + kBN) / kBN);
  }
  __syncthreads();
  const int ntiles = s_ntiles;

  // Q^T operands of this wave's heads: k-step kk = dims 16kk..16kk+15, lane
  // (G, c32) holds head 32*wave + c32, dims 16kk + 8G .. +7.
  const int head = wave * 32 + c32;
  v8bf qb[kD / 16];
  {
    const uint16_t *qrow = p.q + (t * H + head) * (int64_t)kD + 8 * G;
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk)   // row t < total_q: always in bounds
      qb[kk] = as_v8bf(*reinterpret_cast<const v4i *>(qrow + 16 * kk));
  }
  const float sl2 = p.scale * kLog2e;

  // Gather tile `tl` (row indices held by lanes 0..31 in `my_idx`).
  auto gather = [&](int buf, int my_idx, uint32_t vmask) {
    uint8_t *base = kvbuf[buf];
    for (int i = wave; i < kTileInsts; i += NW) {
      const int pch = i * 64 + lane, row = pch / kChunks, slot = pch - row * kChunks;
      const int gi = __shfl(my_idx, row, 64);
      const int64_t grow = s.kv0 + (((vmask >> row) & 1u) ? gi : 0);
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void *>(p.kv + grow * kD + 8 * swz(row, slot)),
          (DSA_LDS void *)(base + i * 1024), 16, 0, 0);
    }
  };
  auto fetch_raw = [&](int tl) {
    const int i = tl * kBN + lane;
    return (lane < kBN && tl < ntiles && i < k) ? idx_row[i] : -1;
  };
  auto validate = [&](int raw, uint32_t &vmask) {
    const bool valid = raw >= 0 && raw < s.kvlen;
    vmask = (uint32_t)__ballot(valid);
    return valid ? raw : 0;
  };

  float m_used = -INFINITY;   // exponent frame of this lane's head (log2 units)
  float m_seen = -INFINITY;   // true running max of this lane's head
  float l_part = 0.f;
  v16f o[MB][NW];

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int u = 0; u < MB; ++u)
#pragma unroll
      for (int nb = 0; nb < NW; ++nb) o[u][nb] = v16f{};
    l_part = 0.f;
    bool overflow = false;

    uint32_t vm_cur = 0;
    int raw = -1;
    if (ntiles > 0) {
      raw = fetch_raw(0);
      const int id0 = validate(raw, vm_cur);
      gather(0, id0, vm_cur);
      raw = fetch_raw(1);
    }
    for (int tl = 0; tl < ntiles; ++tl) {
      const int buf = tl & 1;
      __builtin_amdgcn_s_waitcnt(0);  // this wave's gathers for tile tl + the index prefetch
      __syncthreads();                // all gathers landed; P and buffer buf^1 free again
      const uint32_t vmask = vm_cur;
      if (tl + 1 < ntiles) {
        const int id = validate(raw, vm_cur);
        gather(buf ^ 1, id, vm_cur);
      }
      raw = fetch_raw(tl + 2);
      const uint8_t *tile = kvbuf[buf];

      // ---- S^T (32 keys x this wave's 32 heads)
      v16f sc = {};
      {
        const uint8_t *arow = tile + c32 * kPitch;
#pragma unroll
        for (int kk = 0; kk < kD / 16; ++kk) {
          const v4i a = *reinterpret_cast<const v4i *>(arow + 16 * swz(c32, 2 * kk + G));
          sc = mfma_32x32x16_bf16(as_v8bf(a), qb[kk], sc);
        }
      }
      // ---- softmax: lane holds keys 8(j/4) + 4G + j%4 of head `head`
      float mt = -INFINITY;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = 8 * (j >> 2) + 4 * G + (j & 3);
        float x = sc[j] * sl2;
        if (!((vmask >> key) & 1u)) x = -INFINITY;
        sc[j] = x;
        mt = fmaxf(mt, x);
      }
      mt = max_across_halves(mt);
      m_seen = fmaxf(m_seen, mt);
      if (m_used == -INFINITY) m_used = mt;          // first tile with a valid key
      overflow |= mt > m_used + kFrameSlack;
      const float mf = m_used == -INFINITY ? 0.f : m_used;
      v8bf pb[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pe = exp2f(sc[8 * hf + e] - mf);
          l_part += pe;
          pb[hf][e] = (__bf16)pe;
        }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        *reinterpret_cast<v8bf *>(pbuf + ((wave * 2 + hf) * 64 + lane) * 16) = pb[hf];
      __syncthreads();  // P of every head published

      // ---- O^T[dims of this wave][all heads] += V^T . P^T
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        v8bf av[MB];
        const int r0 = 16 * hf + 4 * G + (jl >> 2), r1 = r0 + 8;
#pragma unroll
        for (int u = 0; u < MB; ++u) {
          const int d0 = wave * DW + 32 * u + 16 * half + 4 * (jl & 3);
          const int c = d0 >> 3, off = (d0 & 7) * 2;
          const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (DSA_LDS v4s *)(tile + r0 * kPitch + 16 * swz(r0, c) + off));
          const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (DSA_LDS v4s *)(tile + r1 * kPitch + 16 * swz(r1, c) + off));
          const v2i lo2 = __builtin_bit_cast(v2i, lo), hi2 = __builtin_bit_cast(v2i, hi);
          av[u] = as_v8bf(v4i{lo2[0], lo2[1], hi2[0], hi2[1]});
        }
#pragma unroll
        for (int nb = 0; nb < NW; ++nb) {
          const v8bf pbn = *reinterpret_cast<const v8bf *>(pbuf + ((nb * 2 + hf) * 64 + lane) * 16);
#pragma unroll
          for (int u = 0; u < MB; ++u) o[u][nb] = mfma_32x32x16_bf16(av[u], pbn, o[u][nb]);
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

  // ---- epilogue: denominators through LDS, normalise, store bf16
  const float l_tot = sum_across_halves(l_part);
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

// Small-shape path: any H <= 128 and D <= 1024.  One workgroup per token;
// plain fp32 dot products, one head at a time.
constexpr int kSmallThreads = 256;
constexpr int kSmallMaxD = 1024;
constexpr int kSmallMaxK = 4096;

__global__ __launch_bounds__(kSmallThreads) void small_sparse_attn_kernel(AttnArgs p) {
  __shared__ float qs[kSmallMaxD];
  __shared__ float prob[kSmallMaxK];
  __shared__ int rows[kSmallMaxK];
  __shared__ float red[kSmallThreads / 64];
  const int64_t t = blockIdx.x;
  const int b = find_seq(p.seq, t);
  const SeqInfo s = load_seq(p.seq, b);
  if (t < s.q0 || t >= s.q1) return;
  const int H = p.heads, D = p.d_latent + p.d_rope, DL = p.d_latent, k = p.k;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < k; i += kSmallThreads) {
    const int v = p.idx[t * k + i];
    rows[i] = (v >= 0 && v < s.kvlen) ? v : -1;
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
        const uint16_t *kr = p.kv + (s.kv0 + rows[i]) * (int64_t)D;
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
        if (rows[i] >= 0) acc = fmaf(prob[i], bf16_bits_to_f32(p.kv[(s.kv0 + rows[i]) * (int64_t)D + d]), acc);
      p.out[(t * H + h) * DL + d] = (uint16_t)f32_to_bf16_bits(acc * inv);
    }
  }
}

}  // namespace

size_t sparse_attn_workspace_bytes(const AttnArgs &) { return 0; }

hipError_t launch_sparse_attn(const AttnArgs &a, hipStream_t stream) {
  if (a.seq.total_q == 0) return hipSuccess;
  const dim3 grid((unsigned)a.seq.total_q);
  // The latent dims split evenly over NW waves only for NW in {1, 2, 4}.
  const bool mfma = a.d_latent == kDL && a.d_rope == kD - kDL &&
                    (a.heads == 32 || a.heads == 64 || a.heads == 128);
  if (mfma) {
    switch (a.heads / 32) {
      case 1: hipLaunchKernelGGL(mla_sparse_attn_kernel<1>, grid, dim3(64), 0, stream, a); break;
      case 2: hipLaunchKernelGGL(mla_sparse_attn_kernel<2>, grid, dim3(128), 0, stream, a); break;
      default: hipLaunchKernelGGL(mla_sparse_attn_kernel<4>, grid, dim3(256), 0, stream, a); break;
    }
  } else {
    hipLaunchKernelGGL(small_sparse_attn_kernel, grid, dim3(kSmallThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace dsa
