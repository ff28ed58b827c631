// Fine-grained top-k selector for gfx950.
//
// The method (ivugangingo.com article on DeepSeek-V3.2, "Sparse attention with
// almost linear long-context costs"; r.nikiv.dev summary, "How DSA Works"):
// per query keep the k key positions with the largest indexer scores (k = 2048
// on the pages).  This library lists them in ascending position, breaks ties
// at the k-th value toward the lower position (-0.0 == +0.0) and pads with -1
// when a row has fewer than k causal candidates.
//
// One 512-thread workgroup per query row (three fit a CU, so one row's select
// and emission overlap other rows' streaming); the row (n = pos+1 fp32
// scores) is read once from HBM in the common case:
//  1. n <= k: every position is selected.
//  2. Otherwise, a lower bound T_lo on the k-th largest order key comes from
//     2048 sampled scores (a 16-bit radix select over the sample; the lower
//     edge of the bin holding the sample's rank-j key): the sample rank is
//     the expected count above the k-th key plus three standard deviations,
//     so the candidates number about k plus a margin.  For rows that fit the
//     candidate buffer (n <= kCap) T_lo is the minimum key, i.e. all.
//  3. One streaming pass (two steps of four 16-byte loads per thread in
//     flight) writes every (key, position) with key >= T_lo to an LDS
//     candidate buffer in position order: per step, ballots give each
//     passing score its rank inside its wave, and one exchange of the wave
//     totals through LDS gives the rank inside the workgroup.
//  4. Exact radix select over the candidates gives the k-th key T and the
//     number of candidates above it.  Because T >= T_lo, every score equal to
//     T and every score above it is a candidate.
//  5. The candidates are in ascending position, so two prefix scans (ties
//     seen before each thread's run, then selected before it) emit the
//     selection in ascending position, taking the lowest-position ties.
// If the sample was unlucky (fewer than k or more than kCap candidates), an
// exact fallback selects with radix passes over the row in global memory and
// emits it with chunked prefix scans.
#include "common.h"
#include "launch.h"

namespace dsa {
namespace {

constexpr int kThreads = 512;
constexpr int kWavesPerBlock = kThreads / 64;
constexpr int kCap = 5632;               // candidate buffer entries (key + position); three
                                         // workgroups' LDS fit one CU
constexpr int kSamples = 2048;           // 64 runs of 32 consecutive scores
constexpr int kSampleRuns = 64;
constexpr int kVec = 4;                  // float4 loads per thread and filter step

struct TopkShared {
  uint32_t keys[kCap];
  uint32_t pos[kCap];
  uint32_t hist[256];
  uint32_t scan[kWavesPerBlock];
  uint32_t bcast[4];
  uint32_t wtot[2][kWavesPerBlock][kVec];  // per step parity: passing scores per wave and slot
};

// Monotone map fp32 -> uint32 (larger float -> larger key); -0.0 maps like +0.0.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of order_key for keys of finite scores.
__device__ __forceinline__ float key_to_float(uint32_t key) {
  const uint32_t u = (key & 0x80000000u) ? (key ^ 0x80000000u) : ~key;
  return __uint_as_float(u);
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
// With max_passes < 4 it stops early and returns the lower edge of the radix
// bin that holds the kth-largest key: a lower bound on that key (n_above is
// then the count above the bin).
template <typename Get>
__device__ void radix_select(Get get, int64_t count, uint32_t kth, TopkShared &sh, uint32_t &thr,
                             uint32_t &n_above, int max_passes = 4) {
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
  for (int pass = 0; shift > 0 && pass < max_passes; ++pass) {
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
  const int tid = (int)__builtin_amdgcn_workitem_id_x(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // The first two filter steps do not depend on the sample bound: their loads
  // go out first, so that their latency overlaps the sample phase.
  constexpr int kStep = kThreads * 4 * kVec;
  const int nn = (int)n;
  const int n_full = nn / kStep;
  auto load_step = [&](int base, float4 (&v)[kVec]) {
#pragma unroll
    for (int e = 0; e < kVec; ++e) v[e] = *reinterpret_cast<const float4 *>(rowp + base + (e * kThreads + tid) * 4);
  };
  float4 va[kVec], vb[kVec];
  if (n_full > 0) load_step(0, va);
  if (n_full > 1) load_step(kStep, vb);

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
    // two radix passes (16 bits below the shared prefix) are enough: the
    // bin's lower edge is a valid lower bound, and a bin that narrow adds
    // few scores
    radix_select([&](int64_t i) { return sh.keys[i]; }, kSamples, (uint32_t)j, sh, t_lo, n_above_s, 2);
  }
  __syncthreads();

  // 3. candidate filter in position order.  Slot (e, c) of thread tid holds
  // position base + (e * kThreads + tid) * 4 + c, so position order is slot
  // e, then wave, then lane, then c: a passing score's rank is the passing
  // scores of earlier slots e' < e (all waves), of earlier waves in slot e,
  // of lower lanes in this wave and slot (ballot + mbcnt), and of c' < c.
  // A score passes when it is >= the sample bound, compared as floats (the
  // bound is a key of a finite score, so float order and key order agree;
  // -0 and +0 both compare equal to a zero bound, as their keys do).
  const float f_lo = t_lo == 0u ? -INFINITY : key_to_float(t_lo);   // key 0: every score passes
  uint32_t done = 0;   // candidates of the steps before (uniform)
  auto filter_step = [&](int base, const float4 (&v)[kVec], bool partial, int par) {
    uint32_t lane_before[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      const int i0 = base + (e * kThreads + tid) * 4;
      const float f[4] = {v[e].x, v[e].y, v[e].z, v[e].w};
      uint32_t tot = 0, below = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint64_t m = __ballot((!partial || i0 + c < nn) && f[c] >= f_lo);
        tot += (uint32_t)__popcll(m);
        below += __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      }
      lane_before[e] = below;
      if (lane == 0) sh.wtot[par][wave][e] = tot;
    }
    __syncthreads();
    uint32_t run = done;
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      uint32_t tot = 0, before = 0;
#pragma unroll
      for (int w = 0; w < kWavesPerBlock; ++w) {
        const uint32_t x = sh.wtot[par][w][e];
        tot += x;
        before += w < wave ? x : 0u;
      }
      uint32_t at = run + before + lane_before[e];
      run += tot;
      const int i0 = base + (e * kThreads + tid) * 4;
      const float f[4] = {v[e].x, v[e].y, v[e].z, v[e].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if ((!partial || i0 + c < nn) && f[c] >= f_lo) {
          if (at < (uint32_t)kCap) {
            sh.keys[at] = order_key(f[c]);
            sh.pos[at] = (uint32_t)(i0 + c);
          }
          ++at;
        }
      }
    }
    done = run;
  };
  {
    // steps st and st+1 are in flight when step st is filtered
    for (int st = 0; st < n_full; st += 2) {
      filter_step(st * kStep, va, false, 0);
      if (st + 2 < n_full) load_step((st + 2) * kStep, va);
      if (st + 1 < n_full) {
        filter_step((st + 1) * kStep, vb, false, 1);
        if (st + 3 < n_full) load_step((st + 3) * kStep, vb);
      }
    }
    const int tail = n_full * kStep;
    if (tail < nn) {
#pragma unroll
      for (int e = 0; e < kVec; ++e) {
        const int i0 = tail + (e * kThreads + tid) * 4;
        float4 x;
        x.x = i0 + 0 < nn ? rowp[i0 + 0] : 0.f;
        x.y = i0 + 1 < nn ? rowp[i0 + 1] : 0.f;
        x.z = i0 + 2 < nn ? rowp[i0 + 2] : 0.f;
        x.w = i0 + 3 < nn ? rowp[i0 + 3] : 0.f;
        va[e] = x;
      }
      filter_step(tail, va, true, n_full & 1);
    }
  }
  __syncthreads();
  const uint32_t cand = done;
  if (cand > (uint32_t)kCap || cand < (uint32_t)k) {
    select_from_global(rowp, n, k, out, sh);
    return;
  }

  // 4. exact k-th key among the candidates
  uint32_t thr, n_above;
  radix_select([&](int64_t i) { return sh.keys[i]; }, cand, (uint32_t)k, sh, thr, n_above);
  const uint32_t need_eq = (uint32_t)k - n_above;

  // 5. ordered emission: each thread owns a contiguous run of candidates
  // (ascending positions); ties are taken lowest position first.
  const uint32_t per = (cand + kThreads - 1) / kThreads;
  const uint32_t c0 = (uint32_t)tid * per < cand ? (uint32_t)tid * per : cand;
  const uint32_t c1 = c0 + per < cand ? c0 + per : cand;
  uint32_t n_sel = 0, n_eq = 0;
  for (uint32_t i = c0; i < c1; ++i) {
    const uint32_t key = sh.keys[i];
    n_sel += key > thr ? 1u : 0u;
    n_eq += key == thr ? 1u : 0u;
  }
  uint32_t tot;
  const uint32_t eq_before = block_exclusive_scan(n_eq, sh, tot);
  uint32_t take = need_eq > eq_before ? need_eq - eq_before : 0u;
  if (take > n_eq) take = n_eq;
  uint32_t at = block_exclusive_scan(n_sel + take, sh, tot);
  for (uint32_t i = c0; i < c1; ++i) {
    const uint32_t key = sh.keys[i];
    bool keep = key > thr;
    if (key == thr && take > 0u) {
      keep = true;
      --take;
    }
    if (keep) out[at++] = (int32_t)sh.pos[i];
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
