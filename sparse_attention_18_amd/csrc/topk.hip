// Fine-grained top-k selector for gfx950.
//
// The method (ivugangingo.com article on DeepSeek-V3.2, "Sparse attention with
// almost linear long-context costs"; r.nikiv.dev summary, "How DSA Works"):
// per query keep the k key positions with the largest indexer scores (k = 2048
// on the pages).  This library lists them in ascending position, breaks ties
// at the k-th value toward the lower position (-0.0 == +0.0) and pads with -1
// when a row has fewer than k causal candidates.
//
// One 512-thread workgroup per query row (two fit a CU); the row (n = pos+1 fp32 scores) is
// read once from HBM in the common case:
//  1. n <= k: every position is selected.
//  2. Otherwise, a lower bound T_lo on the k-th largest order key comes from
//     2048 sampled scores (exact select over the sample): the sample rank is
//     the expected count above the k-th key plus three standard deviations,
//     so the candidates number about k plus a margin.  For rows that fit the
//     candidate buffer (n <= kCap) T_lo is the minimum key, i.e. all.
//  3. One streaming pass (eight 16-byte loads in flight per thread) appends
//     every (key, position) with key >= T_lo to an LDS candidate buffer: one
//     prefix scan and one LDS atomic per wave and step; order not kept.
//  4. Exact radix select over the candidates gives the k-th key T and the
//     number of candidates above it.  Because T >= T_lo, every score equal to
//     T and every score above it is a candidate.
//  5. Two LDS bitmaps over positions mark "above T" and "equal to T"; popcount
//     prefix scans over the bitmap words take the lowest-position equal keys
//     that are needed and emit the selection in ascending position.
// If the sample was unlucky (fewer than k or more than kCap candidates) or the
// row is longer than the bitmap, an exact fallback selects with radix passes
// over the row in global memory and emits it with chunked prefix scans.
#include "common.h"
#include "launch.h"

namespace dsa {
namespace {

constexpr int kThreads = 512;
constexpr int kWavesPerBlock = kThreads / 64;
constexpr int kCap = 5632;               // candidate buffer entries (key + position); two
                                         // workgroups' LDS fit one CU
constexpr int kMaxBitmapN = 131072;      // longest row handled with LDS bitmaps
constexpr int kBitmapWords = kMaxBitmapN / 32;
constexpr int kSamples = 2048;           // 64 runs of 32 consecutive scores
constexpr int kSampleRuns = 64;

struct TopkShared {
  uint32_t keys[kCap];
  uint32_t pos[kCap];
  uint32_t sel[kBitmapWords];
  uint32_t eq[kBitmapWords];
  uint32_t hist[256];
  uint32_t scan[kWavesPerBlock];
  uint32_t bcast[4];
  uint32_t count;
};

// Monotone map fp32 -> uint32 (larger float -> larger key); -0.0 maps like +0.0.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  return v;
}

// Exclusive scan over the workgroup in thread order; also returns the total.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, TopkShared &sh, uint32_t &total) {
  const int tid = (int)__builtin_amdgcn_workitem_id_x(), lane = tid & 63, wave = tid >> 6;
  const uint32_t inc = wave_inclusive_scan(v, lane);
  if (lane == 63) sh.scan[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    uint32_t x = lane < kWavesPerBlock ? sh.scan[lane] : 0u;
    const uint32_t xi = wave_inclusive_scan(x, lane);
    if (lane < kWavesPerBlock) sh.scan[lane] = xi - x;
    if (lane == kWavesPerBlock - 1) sh.bcast[3] = xi;
  }
  __syncthreads();
  const uint32_t r = sh.scan[wave] + inc - v;
  total = sh.bcast[3];
  __syncthreads();
  return r;
}

__device__ __forceinline__ uint32_t block_or(uint32_t v, TopkShared &sh, bool is_and) {
  const int tid = (int)__builtin_amdgcn_workitem_id_x(), lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const uint32_t t = __shfl_xor(v, d, 64);
    v = is_and ? (v & t) : (v | t);
  }
  if (lane == 0) sh.scan[wave] = v;
  __syncthreads();
  uint32_t r = sh.scan[0];
  for (int i = 1; i < kWavesPerBlock; ++i) r = is_and ? (r & sh.scan[i]) : (r | sh.scan[i]);
  __syncthreads();
  return r;
}

// Exact select: the kth-largest (1-based) key among `count` keys read through
// `get(i)`, and how many keys are strictly larger.  Radix passes of up to 8
// bits, most significant first, after skipping the bits every key shares.
template <typename Get>
__device__ void radix_select(Get get, int64_t count, uint32_t kth, TopkShared &sh, uint32_t &thr,
                             uint32_t &n_above) {
  const int tid = (int)__builtin_amdgcn_workitem_id_x(), lane = tid & 63;
  uint32_t vor = 0u, vand = 0xFFFFFFFFu;
  for (int64_t i = tid; i < count; i += kThreads) {
    const uint32_t k = get(i);
    vor |= k;
    vand &= k;
  }
  vor = block_or(vor, sh, false);
  vand = block_or(vand, sh, true);
  const uint32_t diff = vor ^ vand;
  n_above = 0;
  if (diff == 0u) {            // all keys equal
    thr = vor;
    return;
  }
  int shift = 32 - __builtin_clz(diff);          // bits [shift, 32) are shared
  uint32_t prefix = shift == 32 ? 0u : (vor >> shift) << shift;
  uint32_t mask = shift == 32 ? 0u : ~((1u << shift) - 1u);
  uint32_t kk = kth;
  while (shift > 0) {
    const int nb = shift < 8 ? shift : 8;
    shift -= nb;
    const uint32_t dmask = (1u << nb) - 1u;
    for (int i = tid; i < 256; i += kThreads) sh.hist[i] = 0u;
    __syncthreads();
    for (int64_t i = tid; i < count; i += kThreads) {
      const uint32_t k = get(i);
      if ((k & mask) == prefix) atomicAdd(&sh.hist[(k >> shift) & dmask], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane L owns bins 255-4L .. 252-4L (highest bins first)
      uint32_t c[4], s = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = sh.hist[255 - 4 * lane - i];
        s += c[i];
      }
      const uint32_t inc = wave_inclusive_scan(s, lane);
      const uint32_t exc = inc - s;
      const bool hit = exc < kk && inc >= kk;
      if (hit) {
        uint32_t cum = exc;
        int bin = 0;
        uint32_t above = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (cum + c[i] >= kk) {
            bin = 255 - 4 * lane - i;
            above = cum;
            break;
          }
          cum += c[i];
        }
        sh.bcast[0] = (uint32_t)bin;
        sh.bcast[1] = above;
      }
    }
    __syncthreads();
    const uint32_t bin = sh.bcast[0], above = sh.bcast[1];
    __syncthreads();
    kk -= above;
    n_above += above;
    prefix |= bin << shift;
    mask |= dmask << shift;
  }
  thr = prefix;
}

// Emit rows with n <= k: positions 0..n-1, then -1.
__device__ void emit_all(int32_t *out, int64_t n, int k) {
  for (int i = (int)__builtin_amdgcn_workitem_id_x(); i < k; i += kThreads) out[i] = i < n ? i : -1;
}

// Exact fallback over the row in global memory.
__device__ void select_from_global(const float *row, int64_t n, int k, int32_t *out, TopkShared &sh) {
  uint32_t thr, n_above;
  radix_select([&](int64_t i) { return order_key(row[i]); }, n, (uint32_t)k, sh, thr, n_above);
  const uint32_t need_eq = (uint32_t)k - n_above;
  uint32_t eq_seen = 0, written = 0;
  constexpr int V = 4;
  for (int64_t base = 0; base < n; base += (int64_t)kThreads * V) {
    uint32_t key[V];
    uint32_t n_eq = 0;
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const int64_t i = base + (int64_t)__builtin_amdgcn_workitem_id_x() * V + e;
      key[e] = i < n ? order_key(row[i]) : 0u;
      n_eq += (i < n && key[e] == thr) ? 1u : 0u;
    }
    uint32_t eq_total;
    uint32_t eq_before = eq_seen + block_exclusive_scan(n_eq, sh, eq_total);
    bool take[V];
    uint32_t n_take = 0;
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const int64_t i = base + (int64_t)__builtin_amdgcn_workitem_id_x() * V + e;
      bool t = false;
      if (i < n) {
        if (key[e] > thr) t = true;
        else if (key[e] == thr) { t = eq_before < need_eq; ++eq_before; }
      }
      take[e] = t;
      n_take += t ? 1u : 0u;
    }
    uint32_t tk_total;
    uint32_t at = written + block_exclusive_scan(n_take, sh, tk_total);
#pragma unroll
    for (int e = 0; e < V; ++e)
      if (take[e]) out[at++] = (int32_t)(base + (int64_t)__builtin_amdgcn_workitem_id_x() * V + e);
    eq_seen += eq_total;
    written += tk_total;
  }
}

__global__ __launch_bounds__(kThreads)
void topk_kernel(TopkArgs p) {
  __shared__ TopkShared sh;
  const int64_t row = __builtin_amdgcn_workgroup_id_x();
  const int b = find_seq(p.seq, row);
  const SeqInfo s = load_seq(p.seq, b);
  int32_t *out = p.idx + row * p.k;
  if (row < s.q0 || row >= s.q1 || s.kvlen <= 0) {
    emit_all(out, 0, p.k);
    return;
  }
  const int64_t n = row_pos(s, row) + 1;
  const int k = p.k;
  if (n <= k) {
    emit_all(out, n, k);
    return;
  }
  const float *rowp = p.scores + row * p.ld;
  if (n > kMaxBitmapN) {
    select_from_global(rowp, n, k, out, sh);
    return;
  }
  const int tid = (int)__builtin_amdgcn_workitem_id_x(), lane = tid & 63;

  // 2. lower bound on the k-th key from a sample (all keys if the row fits)
  uint32_t t_lo = 0u;
  if (n > kCap) {
    const int64_t span = n - 32;
    for (int i = tid; i < kSamples; i += kThreads) {
      const int run = i >> 5, off = i & 31;
      const int64_t start = span * run / (kSampleRuns - 1);
      sh.keys[i] = order_key(rowp[start + off]);
    }
    __syncthreads();
    const double expect = (double)kSamples * (double)k / (double)n;
    int64_t j = (int64_t)(expect + 3.0 * sqrt(expect) + 4.0);
    if (j > kSamples) j = kSamples;
    uint32_t n_above_s;
    radix_select([&](int64_t i) { return sh.keys[i]; }, kSamples, (uint32_t)j, sh, t_lo, n_above_s);
  }
  if (tid == 0) sh.count = 0u;
  __syncthreads();

  // 3. candidate filter: one pass over the row; per step each thread loads
  // 8 float4 (32 scores, 8 contiguous 16 KB blocks across the workgroup).
  constexpr int kVec = 8;
  for (int64_t base = 0; base < n; base += (int64_t)kThreads * 4 * kVec) {
    float4 v[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      const int64_t i0 = base + ((int64_t)e * kThreads + tid) * 4;
      if (i0 + 3 < n) {
        v[e] = *reinterpret_cast<const float4 *>(rowp + i0);
      } else {
        v[e].x = i0 + 0 < n ? rowp[i0 + 0] : 0.f;
        v[e].y = i0 + 1 < n ? rowp[i0 + 1] : 0.f;
        v[e].z = i0 + 2 < n ? rowp[i0 + 2] : 0.f;
        v[e].w = i0 + 3 < n ? rowp[i0 + 3] : 0.f;
      }
    }
    uint32_t pass_bits = 0u;
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      const int64_t i0 = base + ((int64_t)e * kThreads + tid) * 4;
      const float f[4] = {v[e].x, v[e].y, v[e].z, v[e].w};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (i0 + c < n && order_key(f[c]) >= t_lo) pass_bits |= 1u << (4 * e + c);
    }
    const uint32_t cnt = (uint32_t)__popc(pass_bits);
    const uint32_t inc = wave_inclusive_scan(cnt, lane);
    uint32_t wbase = 0;
    if (lane == 63 && inc > 0) wbase = atomicAdd(&sh.count, inc);
    wbase = __shfl(wbase, 63, 64);
    uint32_t at = wbase + inc - cnt;
    // static loop over the 32 slots (a runtime index into v[] would move it
    // out of registers)
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      const float f[4] = {v[e].x, v[e].y, v[e].z, v[e].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if ((pass_bits >> (4 * e + c)) & 1u) {
          if (at < (uint32_t)kCap) {
            sh.keys[at] = order_key(f[c]);
            sh.pos[at] = (uint32_t)(base + ((int64_t)e * kThreads + tid) * 4 + c);
          }
          ++at;
        }
      }
    }
  }
  __syncthreads();
  const uint32_t cand = sh.count;
  __syncthreads();
  if (cand > (uint32_t)kCap || cand < (uint32_t)k) {
    select_from_global(rowp, n, k, out, sh);
    return;
  }

  // 4. exact k-th key among the candidates
  uint32_t thr, n_above;
  radix_select([&](int64_t i) { return sh.keys[i]; }, cand, (uint32_t)k, sh, thr, n_above);
  const uint32_t need_eq = (uint32_t)k - n_above;

  // 5. bitmaps over positions, then ordered emission
  const int words = (int)((n + 31) / 32);
  for (int i = tid; i < words; i += kThreads) {
    sh.sel[i] = 0u;
    sh.eq[i] = 0u;
  }
  __syncthreads();
  for (uint32_t i = tid; i < cand; i += kThreads) {
    const uint32_t key = sh.keys[i], ps = sh.pos[i];
    if (key > thr) atomicOr(&sh.sel[ps >> 5], 1u << (ps & 31));
    else if (key == thr) atomicOr(&sh.eq[ps >> 5], 1u << (ps & 31));
  }
  __syncthreads();
  // each thread owns a contiguous run of words, so thread order = position order
  const int wpt = (words + kThreads - 1) / kThreads;
  const int w0 = tid * wpt, w1 = w0 + wpt < words ? w0 + wpt : words;
  uint32_t my_eq = 0;
  for (int w = w0; w < w1; ++w) my_eq += (uint32_t)__popc(sh.eq[w]);
  uint32_t tot;
  uint32_t eq_before = block_exclusive_scan(my_eq, sh, tot);
  uint32_t my_sel = 0;
  for (int w = w0; w < w1; ++w) {
    uint32_t e = sh.eq[w];
    const uint32_t pc = (uint32_t)__popc(e);
    uint32_t take = need_eq > eq_before ? need_eq - eq_before : 0u;
    if (take > pc) take = pc;
    uint32_t kept = 0u;
    for (uint32_t t = 0; t < take; ++t) {
      kept |= e & (0u - e);   // lowest set bit
      e &= e - 1u;
    }
    eq_before += pc;
    const uint32_t fin = sh.sel[w] | kept;
    sh.sel[w] = fin;
    my_sel += (uint32_t)__popc(fin);
  }
  uint32_t at = block_exclusive_scan(my_sel, sh, tot);
  for (int w = w0; w < w1; ++w) {
    uint32_t f = sh.sel[w];
    while (f) {
      const int bit = __builtin_ctz(f);
      f &= f - 1u;
      out[at++] = w * 32 + bit;
    }
  }
}

}  // namespace

size_t topk_workspace_bytes(const TopkArgs &) { return 0; }

hipError_t launch_topk(const TopkArgs &a, hipStream_t stream) {
  if (a.seq.total_q == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)a.seq.total_q), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsa
