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
//     4096 sampled scores (a 16-bit radix select over the sample; the lower
//     edge of the bin holding the sample's rank-j key): the sample rank is
//     the expected count above the k-th key plus 4.5 standard deviations, so
//     the candidates number about k plus a margin.  For rows that fit the
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
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace dsa {
namespace {

constexpr int kThreads = 512;
constexpr int kWavesPerBlock = kThreads / 64;
constexpr int kCap = 5632;               // candidate buffer entries (key + position); three
                                         // workgroups' LDS fit one CU
constexpr int kSamples = 4096;           // 128 runs of 32 consecutive scores
constexpr int kSampleRuns = 128;
constexpr int kVec = 4;                  // float4 loads per thread and filter step
constexpr int kMaxSegs = 32;             // segments per row in the few-rows path
constexpr int kSplitRows = 512;          // batches up to this many rows use that path

struct TopkShared {
  union {
    struct {
      uint32_t keys[kCap];
      uint32_t pos[kCap];
    };
    uint32_t sample[kSamples];   // the sample phase only
  };
  uint32_t hist[256];
  uint32_t scan[kWavesPerBlock];
  uint32_t scan2[kWavesPerBlock];
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

// Exclusive scan over the workgroup in thread order; also returns the total.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, TopkShared &sh, uint32_t &total) {
  const int tid = (int)__builtin_amdgcn_workitem_id_x(), lane = tid & 63, wave = tid >> 6;
  const uint32_t inc = wave_scan<0>(v);
  if (lane == 63) sh.scan[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    uint32_t x = lane < kWavesPerBlock ? sh.scan[lane] : 0u;
    const uint32_t xi = wave_scan<0>(x);
    if (lane < kWavesPerBlock) sh.scan[lane] = xi - x;
    if (lane == kWavesPerBlock - 1) sh.bcast[3] = xi;
  }
  __syncthreads();
  const uint32_t r = sh.scan[wave] + inc - v;
  total = sh.bcast[3];
  __syncthreads();
  return r;
}

// Bitwise or and and of every thread's key over the workgroup.
__device__ __forceinline__ void block_or_and(uint32_t &vor, uint32_t &vand, TopkShared &sh) {
  const int tid = (int)__builtin_amdgcn_workitem_id_x(), lane = tid & 63, wave = tid >> 6;
  const uint32_t o = wave_reduce<1>(vor), a = wave_reduce<2>(vand);
  if (lane == 0) {
    sh.scan[wave] = o;
    sh.scan2[wave] = a;
  }
  __syncthreads();
  vor = sh.scan[0];
  vand = sh.scan2[0];
#pragma unroll
  for (int i = 1; i < kWavesPerBlock; ++i) {
    vor |= sh.scan[i];
    vand &= sh.scan2[i];
  }
  __syncthreads();
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
  block_or_and(vor, vand, sh);
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
      const uint32_t inc = wave_scan<0>(s);
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

// Lower bound on the k-th largest key of a row with n > kCap scores (uniform
// over the workgroup; 0 when every score passes).  A row of at most kSamples
// scores is read whole and the bound comes from its own k-th key.  A longer
// row is sampled: S = kSamples scores in 128 runs of 32 consecutive ones
// spread evenly over the row.  The bound is the sample's key of rank
// j = E + 4.5 sqrt(E) + 4, where E = S k / n is the expected number of
// sampled scores at or above the row's k-th key (sqrt(E) its Poisson
// deviation): the bound exceeds that key only if j or more sampled scores
// lie above it.  The bound sits near rank n j / S of the row, which is about
// the number of candidates the filter then keeps.
__device__ uint32_t sample_bound(const float *rowp, int64_t n, int k, TopkShared &sh) {
  static_assert(kSamples % kThreads == 0 && kSamples <= 2 * kCap, "sample layout");
  uint32_t t_lo = 0u;
  if (n > kCap) {
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const bool whole = n <= kSamples;
    const int count = whole ? (int)n : kSamples;
    const int64_t span = n - 32;
    constexpr int kPer = kSamples / kThreads;
    float v[kPer];   // all loads in flight before the first LDS store
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = tid + u * kThreads, run = i >> 5, off = i & 31;
      const int64_t at = whole ? (i < n ? i : n - 1) : span * run / (kSampleRuns - 1) + off;
      v[u] = rowp[at];
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (tid + u * kThreads < count) sh.sample[tid + u * kThreads] = order_key(v[u]);
    __syncthreads();
    int64_t j = k;
    if (!whole) {
      const double expect = (double)kSamples * (double)k / (double)n;
      j = (int64_t)(expect + 4.5 * sqrt(expect) + 4.0);
      if (j > kSamples) j = kSamples;
    }
    uint32_t n_above_s;
    // two radix passes (16 bits below the shared prefix) are enough: the
    // bin's lower edge is a valid lower bound, and a bin that narrow adds
    // few scores
    radix_select([&](int64_t i) { return sh.sample[i]; }, count, (uint32_t)j, sh, t_lo, n_above_s, 2);
  }
  __syncthreads();
  return t_lo;
}

constexpr int kStep = kThreads * 4 * kVec;   // scores per filter step

__device__ __forceinline__ void load_step(const float *rowp, int base, float4 (&v)[kVec]) {
  const int tid = (int)__builtin_amdgcn_workitem_id_x();
#pragma unroll
  for (int e = 0; e < kVec; ++e) v[e] = *reinterpret_cast<const float4 *>(rowp + base + (e * kThreads + tid) * 4);
}

// Candidate sinks: entry `at` of the position-ordered candidate list.
struct LdsSink {
  TopkShared *sh;
  __device__ void put(uint32_t at, uint32_t key, uint32_t pos) const {
    if (at < (uint32_t)kCap) {
      sh->keys[at] = key;
      sh->pos[at] = pos;
    }
  }
};
struct GlobalSink {
  uint2 *c;
  __device__ void put(uint32_t at, uint32_t key, uint32_t pos) const {
    if (at < (uint32_t)kCap) c[at] = make_uint2(key, pos);
  }
};

// Candidate filter over scores [lo, hi) of a row (lo a multiple of 4 floats
// from a 16-byte aligned row), in position order.  va / vb must already hold
// steps 0 and 1 of the range where those are full steps.  Slot (e, c) of
// thread tid holds position base + (e * kThreads + tid) * 4 + c, so position
// order is slot e, then wave, then lane, then c: a passing score's rank is
// the passing scores of earlier slots e' < e (all waves), of earlier waves in
// slot e, of lower lanes in this wave and slot (ballot + mbcnt), and of
// c' < c.  A score passes when it is >= f_lo.  Returns the number of passing
// scores (uniform; entries at or past kCap are counted but not stored).
template <class Sink>
__device__ uint32_t filter_range(const float *rowp, int lo, int hi, float f_lo, const Sink &sink,
                                 TopkShared &sh, float4 (&va)[kVec], float4 (&vb)[kVec]) {
  const int tid = (int)__builtin_amdgcn_workitem_id_x(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_full = (hi - lo) / kStep;
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
        const uint64_t m = __ballot((!partial || i0 + c < hi) && f[c] >= f_lo);
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
        if ((!partial || i0 + c < hi) && f[c] >= f_lo) {
          sink.put(at, order_key(f[c]), (uint32_t)(i0 + c));
          ++at;
        }
      }
    }
    done = run;
  };
  // steps st and st+1 are in flight when step st is filtered
  for (int st = 0; st < n_full; st += 2) {
    filter_step(lo + st * kStep, va, false, 0);
    if (st + 2 < n_full) load_step(rowp, lo + (st + 2) * kStep, va);
    if (st + 1 < n_full) {
      filter_step(lo + (st + 1) * kStep, vb, false, 1);
      if (st + 3 < n_full) load_step(rowp, lo + (st + 3) * kStep, vb);
    }
  }
  const int tail = lo + n_full * kStep;
  if (tail < hi) {
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      const int i0 = tail + (e * kThreads + tid) * 4;
      float4 x;
      x.x = i0 + 0 < hi ? rowp[i0 + 0] : 0.f;
      x.y = i0 + 1 < hi ? rowp[i0 + 1] : 0.f;
      x.z = i0 + 2 < hi ? rowp[i0 + 2] : 0.f;
      x.w = i0 + 3 < hi ? rowp[i0 + 3] : 0.f;
      va[e] = x;
    }
    filter_step(tail, va, true, n_full & 1);
  }
  __syncthreads();
  return done;
}

// Steps 4 and 5 over a position-ordered candidate list in LDS (k <= cand <= kCap).
__device__ void select_and_emit(uint32_t cand, int k, int32_t *out, TopkShared &sh) {
  const int tid = (int)__builtin_amdgcn_workitem_id_x();
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

// One workgroup per row (batches with enough rows to fill the chip).
__global__ __launch_bounds__(kThreads)
void topk_kernel(TopkArgs p) {
  __shared__ TopkShared sh;
  const int64_t row = __builtin_amdgcn_workgroup_id_x();
  SeqInfo s;
  const int b = row_seq(p.seq, row, s);
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
  const int nn = (int)n;

  // The first two filter steps do not depend on the sample bound: their loads
  // go out first, so that their latency overlaps the sample phase.
  float4 va[kVec], vb[kVec];
  if (nn / kStep > 0) load_step(rowp, 0, va);
  if (nn / kStep > 1) load_step(rowp, kStep, vb);
  const uint32_t t_lo = sample_bound(rowp, n, k, sh);
  // the bound is a key of a finite score, so float order and key order agree
  // (-0 and +0 both compare equal to a zero bound, as their keys do); key 0
  // lets every score pass
  const float f_lo = t_lo == 0u ? -INFINITY : key_to_float(t_lo);
  const uint32_t cand = filter_range(rowp, 0, nn, f_lo, LdsSink{&sh}, sh, va, vb);
  if (cand > (uint32_t)kCap || cand < (uint32_t)k) {
    select_from_global(rowp, n, k, out, sh);
    return;
  }
  select_and_emit(cand, k, out, sh);
}

// Few rows (decode): each row is cut into segments of seg_len scores, one
// workgroup each.  Every segment's workgroup derives the same sample bound
// from the whole row, filters its own segment and writes its candidates, in
// position order, to a fixed slot of the workspace together with their
// count; the segments' lists concatenated are exactly the list the
// one-workgroup filter builds.
__global__ __launch_bounds__(kThreads)
void topk_segment_kernel(TopkArgs p, uint32_t *counts, uint2 *cands) {
  __shared__ TopkShared sh;
  const int64_t row = __builtin_amdgcn_workgroup_id_y();
  const int seg = __builtin_amdgcn_workgroup_id_x();
  SeqInfo s;
  const int b = row_seq(p.seq, row, s);
  if (row < s.q0 || row >= s.q1 || s.kvlen <= 0) return;
  const int64_t n = row_pos(s, row) + 1;
  const int k = p.k;
  const int lo = seg * p.seg_len;
  if (n <= k || lo >= n) return;
  const int hi = n - lo > p.seg_len ? lo + p.seg_len : (int)n;
  const float *rowp = p.scores + row * p.ld;
  float4 va[kVec], vb[kVec];
  if ((hi - lo) / kStep > 0) load_step(rowp, lo, va);
  if ((hi - lo) / kStep > 1) load_step(rowp, lo + kStep, vb);
  const uint32_t t_lo = sample_bound(rowp, n, k, sh);
  const float f_lo = t_lo == 0u ? -INFINITY : key_to_float(t_lo);
  const size_t slot = (size_t)row * p.nseg + seg;
  const uint32_t cand = filter_range(rowp, lo, hi, f_lo, GlobalSink{cands + slot * kCap}, sh, va, vb);
  if (__builtin_amdgcn_workitem_id_x() == 0) counts[slot] = cand;
}

// Merge of a row's segment lists: one workgroup per row.
__global__ __launch_bounds__(kThreads)
void topk_merge_kernel(TopkArgs p, const uint32_t *counts, const uint2 *cands) {
  __shared__ TopkShared sh;
  const int64_t row = __builtin_amdgcn_workgroup_id_x();
  SeqInfo s;
  const int b = row_seq(p.seq, row, s);
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
  const int tid = (int)__builtin_amdgcn_workitem_id_x();
  const int nseg = (int)((n + p.seg_len - 1) / p.seg_len);
  const uint32_t *cnt = counts + (size_t)row * p.nseg;
  // segment offsets by an exclusive scan over the (at most kThreads) counts
  const uint32_t c = tid < nseg ? cnt[tid] : 0u;
  uint32_t total;
  const uint32_t off = block_exclusive_scan(c > (uint32_t)kCap ? (uint32_t)kCap + 1u : c, sh, total);
  if (total > (uint32_t)kCap || total < (uint32_t)k) {
    select_from_global(p.scores + row * p.ld, n, k, out, sh);
    return;
  }
  // copy the segment lists into LDS at their offsets: wave w copies
  // segments w, w + 8, ...  (nseg <= kMaxSegs, so hist holds both arrays)
  if (tid < nseg) {
    sh.hist[tid] = off;
    sh.hist[kMaxSegs + tid] = c;
  }
  __syncthreads();
  const int lane = tid & 63, wave = tid >> 6;
  const uint2 *src = cands + (size_t)row * p.nseg * kCap;
  for (int sgi = wave; sgi < nseg; sgi += kWavesPerBlock) {
    const uint32_t o = sh.hist[sgi], cs = sh.hist[kMaxSegs + sgi];
    for (uint32_t i0 = lane; i0 < cs; i0 += 64 * 8) {
      uint2 v[8];   // eight loads in flight before the LDS stores
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t i = i0 + 64 * u;
        if (i < cs) v[u] = src[(size_t)sgi * kCap + i];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t i = i0 + 64 * u;
        if (i < cs) {
          sh.keys[o + i] = v[u].x;
          sh.pos[o + i] = v[u].y;
        }
      }
    }
  }
  __syncthreads();
  select_and_emit(total, k, out, sh);
}

// ---- Fused decode selection.  The decode indexer (indexer.hip, bin_chunk)
// leaves, per 1024-key chunk of a row, the chunk's nonzero bins of the top 12
// order-key bits (descending, with each bin's count and first list slot) and
// its keys grouped by bin.  One workgroup per row then:
//  1. sums the chunks' bin counts into a 4096-bin row histogram and finds
//     the bin B1 holding the k-th largest key and the count A above it --
//     exactly, without a sample and without reading the scores;
//  2. reads from each chunk's list only the prefix down to B1: the A keys
//     above B1 (all selected; only their positions are kept) and the E keys
//     in B1;
//  3. selects the (k - A)-th largest among the E keys of B1 (radix passes
//     over their low 20 bits) as the threshold T;
//  4. marks the selected positions in an LDS bitmap over the row (ties at T
//     go through a second bitmap, of which the lowest positions are kept)
//     and writes the set bits in ascending order.
// The threads are dealt to the row's chunks (tpc per chunk), so every load's
// address is known without a search.  When more than kCap keys fall in B1
// they are read from the lists in global memory instead of LDS (exact, slower).
constexpr int kFuseMaxChunks = (int)(kFuseMaxLen / kFuseChunk);
constexpr int kFuseWords = (int)(kFuseMaxLen / 32);
constexpr int kFuseBatch = 8;        // loads in flight per thread
static_assert(kFuseMaxChunks <= kThreads / 2, "at least two threads per chunk");
static_assert(kFuseWords % kThreads == 0 && kFuseBins % kThreads == 0, "bitmap and histogram split");

struct FusedShared {
  union {
    uint32_t hist[kFuseBins];                     // step 1: row histogram
    struct {
      uint32_t sel[kFuseWords];                   // step 4: selected positions
      uint32_t eq[kFuseWords];                    //         positions whose key is T
    } bm;
  };
  uint32_t above[4096];                           // positions of the A keys above B1 (A < k)
  uint32_t na[kFuseMaxChunks], ne[kFuseMaxChunks];    // per chunk: keys above B1, keys in B1
  uint32_t offa[kFuseMaxChunks], offe[kFuseMaxChunks];
};

// The lowest `r` set bits of x.
__device__ __forceinline__ uint32_t lowest_set_bits(uint32_t x, uint32_t r) {
  uint32_t kept = 0u;
  for (uint32_t i = 0; i < r && x != 0u; ++i) {
    const uint32_t lsb = x & (0u - x);
    kept |= lsb;
    x ^= lsb;
  }
  return kept;
}

__global__ __launch_bounds__(kThreads)
void topk_fused_kernel(TopkArgs p) {
  __shared__ TopkShared sh;
  __shared__ FusedShared fs;
  const int64_t row = __builtin_amdgcn_workgroup_id_x();
  SeqInfo s;
  row_seq(p.seq, row, s);
  int32_t *out = p.idx + row * p.k;
  if (row < s.q0 || row >= s.q1 || s.kvlen <= 0) {
    emit_all(out, 0, p.k);
    return;
  }
  const int64_t n = row_pos(s, row) + 1;       // <= kFuseMaxLen (checked on the host)
  const int k = p.k;
  if (n <= k) {
    emit_all(out, n, k);
    return;
  }
  const int tid = (int)__builtin_amdgcn_workitem_id_x();
  const int W = (int)((n + kFuseChunk - 1) / kFuseChunk);   // 3..256 chunks
  int tpc = kThreads;                                       // threads per chunk
  while (tpc * W > kThreads) tpc >>= 1;
  const int cw = tid / tpc, sub = tid % tpc;                // this thread's chunk
  const bool has_chunk = cw < W;
  const int64_t slot = row * p.fuse.nchunk + (has_chunk ? cw : 0);
  const uint32_t *tab = p.fuse.tab + slot * kFuseTabCap;
  const uint32_t *lst = p.fuse.list + slot * kFuseChunk;
  auto bin_of = [](uint32_t v) { return v >> 20; };
  auto cnt_of = [](uint32_t v) { return (v & 1023u) + 1u; };

  // 1. row histogram.  Table entries sub, sub + tpc, ... of this thread's
  // chunk; the first kFuseBatch stay in registers for step 2.
  uint32_t z = has_chunk ? p.fuse.nz[slot] : 0u;
  z = z < (uint32_t)kFuseTabCap ? z : (uint32_t)kFuseTabCap;
  for (int i = tid; i < kFuseBins; i += kThreads) fs.hist[i] = 0u;
  uint32_t t0[kFuseBatch];
#pragma unroll
  for (int u = 0; u < kFuseBatch; ++u) {
    const uint32_t e = sub + u * tpc;
    t0[u] = tab[e < z ? e : 0u];
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kFuseBatch; ++u)
    if (sub + u * tpc < z) atomicAdd(&fs.hist[bin_of(t0[u])], cnt_of(t0[u]));
  for (uint32_t e0 = sub + kFuseBatch * tpc; e0 < z; e0 += kFuseBatch * tpc) {
    uint32_t v[kFuseBatch];
#pragma unroll
    for (int u = 0; u < kFuseBatch; ++u) {
      const uint32_t e = e0 + u * tpc;
      v[u] = tab[e < z ? e : 0u];
    }
#pragma unroll
    for (int u = 0; u < kFuseBatch; ++u)
      if (e0 + u * tpc < z) atomicAdd(&fs.hist[bin_of(v[u])], cnt_of(v[u]));
  }
  if (tid < W) {
    fs.na[tid] = 0u;
    fs.ne[tid] = 0u;
  }
  __syncthreads();
  {
    // thread t owns bins 4095 - 8t .. 4088 - 8t (descending)
    constexpr int kPer = kFuseBins / kThreads;
    uint32_t hc[kPer], hs = 0u;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      hc[i] = fs.hist[kFuseBins - 1 - kPer * tid - i];
      hs += hc[i];
    }
    uint32_t tot;
    uint32_t cum = block_exclusive_scan(hs, sh, tot);
    if (cum < (uint32_t)k && cum + hs >= (uint32_t)k) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        if (cum < (uint32_t)k && cum + hc[i] >= (uint32_t)k) {
          sh.bcast[0] = (uint32_t)(kFuseBins - 1 - kPer * tid - i);
          sh.bcast[1] = cum;
          sh.bcast[2] = hc[i];
        }
        cum += hc[i];
      }
    }
    __syncthreads();
  }
  const uint32_t B1 = sh.bcast[0], A = sh.bcast[1], E = sh.bcast[2];

  // 2. per chunk: keys above B1 (na) and in B1 (ne), where they go, and the
  // list prefixes themselves
  auto count_entry = [&](uint32_t v) {
    const uint32_t b = bin_of(v);
    if (b > B1) atomicAdd(&fs.na[cw], cnt_of(v));
    else if (b == B1) fs.ne[cw] = cnt_of(v);
  };
#pragma unroll
  for (int u = 0; u < kFuseBatch; ++u)
    if (sub + u * tpc < z) count_entry(t0[u]);
  for (uint32_t e0 = sub + kFuseBatch * tpc; e0 < z; e0 += kFuseBatch * tpc) {
    uint32_t v[kFuseBatch];
#pragma unroll
    for (int u = 0; u < kFuseBatch; ++u) {
      const uint32_t e = e0 + u * tpc;
      v[u] = tab[e < z ? e : 0u];
    }
#pragma unroll
    for (int u = 0; u < kFuseBatch; ++u)
      if (e0 + u * tpc < z) count_entry(v[u]);
  }
  __syncthreads();
  {
    // A < k <= 4096 fits 13 bits, E <= n <= 2^18 the 19 above them
    const uint32_t pk = tid < W ? (fs.ne[tid] << 13 | fs.na[tid]) : 0u;
    uint32_t ptot;
    const uint32_t pex = block_exclusive_scan(pk, sh, ptot);
    if (tid < W) {
      fs.offa[tid] = pex & 0x1FFFu;
      fs.offe[tid] = pex >> 13;
    }
    __syncthreads();
  }
  const bool e_in_lds = E <= (uint32_t)kCap;
  {
    const uint32_t na = has_chunk ? fs.na[cw] : 0u;
    const uint32_t take = has_chunk ? na + (e_in_lds ? fs.ne[cw] : 0u) : 0u;
    const uint32_t oa = has_chunk ? fs.offa[cw] : 0u, oe = has_chunk ? fs.offe[cw] : 0u;
    for (uint32_t e0 = sub; e0 < take; e0 += kFuseBatch * tpc) {
      uint32_t v[kFuseBatch];
#pragma unroll
      for (int u = 0; u < kFuseBatch; ++u) {
        const uint32_t e = e0 + u * tpc;
        v[u] = lst[e < take ? e : 0u];
      }
#pragma unroll
      for (int u = 0; u < kFuseBatch; ++u) {
        const uint32_t e = e0 + u * tpc;
        if (e < take) {
          const uint32_t q = (uint32_t)cw * kFuseChunk + (v[u] & 1023u);
          if (e < na) {
            fs.above[oa + e] = q;
          } else {
            sh.keys[oe + e - na] = B1 << 20 | v[u] >> 10;
            sh.pos[oe + e - na] = q;
          }
        }
      }
    }
  }
  __syncthreads();

  // The i-th key of B1 (in chunk order) and its position: from LDS, or from
  // the lists when there are too many of them for LDS.
  auto b1_entry = [&](uint32_t i, uint32_t &key, uint32_t &q) {
    if (e_in_lds) {
      key = sh.keys[i];
      q = sh.pos[i];
      return;
    }
    int lo = 0, hi = W - 1;                       // the last chunk whose offe is <= i
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (fs.offe[mid] <= i) lo = mid;
      else hi = mid - 1;
    }
    const uint32_t v = p.fuse.list[(row * p.fuse.nchunk + lo) * kFuseChunk + fs.na[lo] + (i - fs.offe[lo])];
    key = B1 << 20 | v >> 10;
    q = (uint32_t)lo * kFuseChunk + (v & 1023u);
  };

  // 3. threshold among the keys of B1
  uint32_t thr, n_above;
  radix_select([&](int64_t i) { uint32_t key, q; b1_entry((uint32_t)i, key, q); return key; }, E,
               (uint32_t)k - A, sh, thr, n_above);
  const uint32_t need_eq = (uint32_t)k - A - n_above;

  // 4. position bitmaps, ties limited to the lowest positions, emission.
  // Thread t owns words [t * wpt, t * wpt + wpt).
  const int nw = (int)((n + 31) >> 5);
  const int wpt = (nw + kThreads - 1) / kThreads;  // <= kFuseWords / kThreads
  for (int i = tid; i < nw; i += kThreads) {
    fs.bm.sel[i] = 0u;
    fs.bm.eq[i] = 0u;
  }
  __syncthreads();
  for (uint32_t i = tid; i < A; i += kThreads) {
    const uint32_t q = fs.above[i];
    atomicOr(&fs.bm.sel[q >> 5], 1u << (q & 31));
  }
  for (uint32_t i = tid; i < E; i += kThreads) {
    uint32_t key, q;
    b1_entry(i, key, q);
    if (key > thr) atomicOr(&fs.bm.sel[q >> 5], 1u << (q & 31));
    else if (key == thr) atomicOr(&fs.bm.eq[q >> 5], 1u << (q & 31));
  }
  __syncthreads();
  const int w0 = wpt * tid;
  uint32_t ec = 0u;
  for (int u = 0; u < wpt; ++u) ec += w0 + u < nw ? (uint32_t)__popc(fs.bm.eq[w0 + u]) : 0u;
  uint32_t etot;
  uint32_t eb = block_exclusive_scan(ec, sh, etot);
  uint32_t sc = 0u;
  for (int u = 0; u < wpt; ++u) {
    if (w0 + u < nw) {
      const uint32_t x = fs.bm.eq[w0 + u], c = (uint32_t)__popc(x);
      const uint32_t keep = need_eq > eb ? (need_eq - eb < c ? need_eq - eb : c) : 0u;
      uint32_t y = fs.bm.sel[w0 + u];
      if (keep) y |= keep == c ? x : lowest_set_bits(x, keep);
      fs.bm.sel[w0 + u] = y;
      sc += (uint32_t)__popc(y);
      eb += c;
    }
  }
  uint32_t stot;
  uint32_t at = block_exclusive_scan(sc, sh, stot);
  for (int u = 0; u < wpt; ++u) {
    if (w0 + u < nw) {
      uint32_t x = fs.bm.sel[w0 + u];
      while (x != 0u) {
        if (at < (uint32_t)k) out[at] = (int32_t)(32 * (w0 + u) + __builtin_ctz(x));
        ++at;
        x &= x - 1u;
      }
    }
  }
}
}  // namespace

namespace {

// Segment geometry of the few-rows path; false when the one-workgroup-per-row
// kernel serves the batch.
bool split_geometry(const TopkArgs &a, int32_t &seg_len, int32_t &nseg) {
  if (a.seq.total_q > kSplitRows || a.seq.max_kv_len < 4 * (int64_t)kStep) return false;
  // as many segments as fit one round of workgroups (three per CU on 256
  // CUs), at most kMaxSegs per row
  const int64_t steps = (a.seq.max_kv_len + kStep - 1) / kStep;
  const int64_t per_row = std::max<int64_t>(1, std::min<int64_t>(kMaxSegs, 768 / a.seq.total_q));
  const int64_t seg_steps = (steps + per_row - 1) / per_row;
  seg_len = (int32_t)(seg_steps * kStep);
  nseg = (int32_t)((a.seq.max_kv_len + seg_len - 1) / seg_len);
  return true;
}

size_t split_bytes(const TopkArgs &a, int32_t nseg) {
  const size_t slots = (size_t)a.seq.total_q * (size_t)nseg;
  return ((slots * sizeof(uint32_t) + 255) / 256) * 256 + slots * kCap * sizeof(uint2);
}

}  // namespace

size_t topk_workspace_bytes(const TopkArgs &a) {
  int32_t seg_len, nseg;
  return split_geometry(a, seg_len, nseg) ? split_bytes(a, nseg) : 0;
}

bool fuse_eligible(const SeqLayout &seq) {
  return decode_indexer(seq) && seq.total_q > 0 && seq.max_kv_len > 0 && seq.max_kv_len <= kFuseMaxLen;
}

size_t fuse_workspace_bytes(const SeqLayout &seq) {
  if (!fuse_eligible(seq)) return 0;
  const size_t slots = (size_t)seq.total_q * (size_t)((seq.max_kv_len + kFuseChunk - 1) / kFuseChunk);
  auto r256 = [](size_t x) { return (x + 255) / 256 * 256; };
  return r256(slots * kFuseTabCap * 4) + r256(slots * 4) + slots * kFuseChunk * 4;
}

hipError_t launch_topk_fused(const TopkArgs &a, hipStream_t stream) {
  if (a.seq.total_q == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_fused_kernel, dim3((unsigned)a.seq.total_q), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs &a, hipStream_t stream) {
  if (a.seq.total_q == 0) return hipSuccess;
  TopkArgs s = a;
  if (split_geometry(a, s.seg_len, s.nseg) && a.workspace != nullptr &&
      a.workspace_bytes >= split_bytes(a, s.nseg)) {
    const size_t slots = (size_t)a.seq.total_q * (size_t)s.nseg;
    uint32_t *counts = static_cast<uint32_t *>(a.workspace);
    uint2 *cands = reinterpret_cast<uint2 *>(static_cast<uint8_t *>(a.workspace) +
                                             ((slots * sizeof(uint32_t) + 255) / 256) * 256);
    hipLaunchKernelGGL(topk_segment_kernel, dim3((unsigned)s.nseg, (unsigned)a.seq.total_q),
                       dim3(kThreads), 0, stream, s, counts, cands);
    hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)a.seq.total_q), dim3(kThreads), 0, stream,
                       s, counts, cands);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)a.seq.total_q), dim3(kThreads), 0, stream, s);
  return hipGetLastError();
}

}  // namespace dsa
