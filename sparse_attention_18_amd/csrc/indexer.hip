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
#include "common.h"
#include "launch.h"

namespace dsa {
namespace {

constexpr int kWaves = 4;          // waves per workgroup
constexpr int kKeyTile = 64;       // keys per LDS tile in the prefill kernel
constexpr int kRowBytes = 128;     // one key row in LDS (d_I padded to 128)

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
                                           bool valid, int g, int c) {
  // Branch-free: every address is clamped in bounds, invalid parts are zeroed
  // by selects, so the prologue stays one basic block.
  const int H = p.idx_heads, d = p.idx_dim;
  const float qs = valid ? p.q_scale[row] : 0.0f;
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

// sum_j w_j * ReLU(dot_j) over this lane's 4*HB heads for one 16-key block.
// The HB MFMAs are independent, so they issue back to back before the
// epilogue consumes them.
template <int HB>
__device__ __forceinline__ float score_block(const QueryRegs<HB> &q, const v8i &b) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  v4f d[HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) d[hb] = mfma_16x16x128_fp8(q.a[hb], b, zero);
  float s = 0.f;
#pragma unroll
  for (int hb = 0; hb < HB; ++hb)
#pragma unroll
    for (int i = 0; i < 4; ++i) s = fmaf(q.w[hb][i], fmaxf(d[hb][i], 0.f), s);
  return s;
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
// through double-buffered LDS tiles shared by all waves.
template <int HB, int QW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void indexer_prefill_kernel(IndexerArgs p, int key_split) {
  constexpr int QT = kWaves * QW;
  __shared__ __attribute__((aligned(16))) uint8_t ktile[2][kKeyTile * kRowBytes];

  const SeqInfo s = load_seq(p.seq, blockIdx.z);
  const int64_t qlen = s.q1 - s.q0;
  const int64_t row_begin = (int64_t)blockIdx.y * QT;
  if (row_begin >= qlen || s.kvlen <= 0) return;
  const int64_t rows_here = qlen - row_begin < QT ? qlen - row_begin : QT;
  const int64_t last_pos = row_pos(s, s.q0 + row_begin + rows_here - 1);
  const int64_t key_begin = (int64_t)blockIdx.x * key_split;
  if (key_begin > last_pos) return;
  const int64_t key_end = key_begin + key_split < last_pos + 1 ? key_begin + key_split : last_pos + 1;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;

  // Rows past the end of the tile get zero weights (and are never stored),
  // so no per-query branch splits the tile loop.
  QueryRegs<HB> q[QW];
  int64_t pos[QW], grow[QW];
#pragma unroll
  for (int qi = 0; qi < QW; ++qi) {
    const int64_t r = row_begin + wave * QW + qi;
    const bool valid = r < qlen;
    grow[qi] = s.q0 + (valid ? r : 0);
    pos[qi] = valid ? row_pos(s, grow[qi]) : -1;
    load_query<HB>(q[qi], p, grow[qi], valid, g, c);
  }

  // Each thread stages two 16-byte chunks of a 64-key tile (512 chunks).
  const int d = p.idx_dim;
  v4i stage[2];
  auto fetch = [&](int64_t t0) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int chunk = tid + 256 * e, n = chunk >> 3, j = chunk & 7;
      const int64_t key = t0 + n;
      const bool ok = key < s.kvlen && 16 * j < d;
      const v4i x = *reinterpret_cast<const v4i *>(
          p.k_fp8 + (s.kv0 + (key < s.kvlen ? key : 0)) * d + (16 * j < d ? 16 * j : 0));
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
  int buf = 0;
  for (int64_t t0 = key_begin; t0 < key_end; t0 += kKeyTile) {
    const bool has_next = t0 + kKeyTile < key_end;
    if (has_next) fetch(t0 + kKeyTile);
    const int64_t my_key = t0 + lane;
    const float ks = p.k_scale[s.kv0 + (my_key < s.kvlen ? my_key : 0)];

    float part[QW][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int n = kb * 16 + c;
      const v4i lo = *reinterpret_cast<const v4i *>(&ktile[buf][ktile_offset(n, 2 * g)]);
      const v4i hi = *reinterpret_cast<const v4i *>(&ktile[buf][ktile_offset(n, 2 * g + 1)]);
      const v8i bop = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
      for (int qi = 0; qi < QW; ++qi) part[qi][kb] = score_block<HB>(q[qi], bop);
    }
#pragma unroll
    for (int qi = 0; qi < QW; ++qi) {
      const float v = reduce_four_blocks(part[qi][0], part[qi][1], part[qi][2], part[qi][3]);
      if (my_key < key_end && my_key <= pos[qi]) p.scores[grow[qi] * p.ld + my_key] = v * ks;
    }
    if (has_next) {
      commit(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }
}

// Decode (few query rows per sequence): grid (key chunk, query row).  Keys
// are used by one query only, so each wave streams its own 256-key slice
// straight from HBM into MFMA B operands; nothing goes through LDS.
constexpr int kDecodeChunk = 1024;  // keys per workgroup (4 waves x 256)

template <int HB>
__global__ __launch_bounds__(256) void indexer_decode_kernel(IndexerArgs p) {
  const int64_t row = blockIdx.y;
  const int b = find_seq(p.seq, row);
  const SeqInfo s = load_seq(p.seq, b);
  if (row < s.q0 || row >= s.q1 || s.kvlen <= 0) return;
  const int64_t pos = row_pos(s, row);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int64_t wave_begin = (int64_t)blockIdx.x * kDecodeChunk + wave * (kDecodeChunk / kWaves);
  if (wave_begin > pos) return;
  const int64_t wave_end = wave_begin + kDecodeChunk / kWaves < pos + 1
                               ? wave_begin + kDecodeChunk / kWaves : pos + 1;

  QueryRegs<HB> q;
  load_query<HB>(q, p, row, true, g, c);
  const int d = p.idx_dim;

  auto load_b = [&](int64_t t0, int kb) {
    const int64_t key = t0 + kb * 16 + c;
    v4i lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
    if (key < wave_end && 32 * g < d) {
      const v4i *src = reinterpret_cast<const v4i *>(p.k_fp8 + (s.kv0 + key) * d + 32 * g);
      lo = src[0];
      hi = src[1];
    }
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };

  v8i cur[4], nxt[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) cur[kb] = load_b(wave_begin, kb);
  for (int64_t t0 = wave_begin; t0 < wave_end; t0 += 64) {
    const bool has_next = t0 + 64 < wave_end;
    if (has_next) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) nxt[kb] = load_b(t0 + 64, kb);
    }
    const int64_t my_key = t0 + lane;
    const float ks = my_key < wave_end ? p.k_scale[s.kv0 + my_key] : 0.f;
    float part[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) part[kb] = score_block<HB>(q, cur[kb]);
    const float v = reduce_four_blocks(part[0], part[1], part[2], part[3]);
    if (my_key < wave_end) p.scores[row * p.ld + my_key] = v * ks;
    if (has_next) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) cur[kb] = nxt[kb];
    }
  }
}

template <int HB, int QW>
hipError_t launch_prefill(const IndexerArgs &a, hipStream_t stream) {
  constexpr int QT = kWaves * QW;
  const int64_t qtiles = (a.seq.max_q_len + QT - 1) / QT;
  // Key split: as long as possible (fewer Q re-loads) while keeping several
  // workgroups per CU; the split count is padded to a multiple of 8 so that a
  // split always lands on the same XCD (workgroups go round-robin over 8 XCDs).
  int64_t split = 2048;
  auto blocks = [&](int64_t sp) {
    const int64_t ns = ((a.seq.max_kv_len + sp - 1) / sp + 7) / 8 * 8;
    return ns * qtiles * a.seq.batch;
  };
  while (split > kKeyTile && blocks(split) < 4 * 256) split /= 2;
  const int64_t nsplit = ((a.seq.max_kv_len + split - 1) / split + 7) / 8 * 8;
  dim3 grid((unsigned)nsplit, (unsigned)qtiles, (unsigned)a.seq.batch);
  hipLaunchKernelGGL((indexer_prefill_kernel<HB, QW>), grid, dim3(256), 0, stream, a, (int)split);
  return hipGetLastError();
}

template <int HB>
hipError_t launch_decode(const IndexerArgs &a, hipStream_t stream) {
  dim3 grid((unsigned)((a.seq.max_kv_len + kDecodeChunk - 1) / kDecodeChunk), (unsigned)a.seq.total_q);
  hipLaunchKernelGGL((indexer_decode_kernel<HB>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int HB>
hipError_t dispatch(const IndexerArgs &a, hipStream_t stream) {
  // A handful of query rows per sequence: stream keys per row.
  if (a.seq.max_q_len <= 2) return launch_decode<HB>(a, stream);
  return launch_prefill<HB, (HB >= 4 ? 8 / HB : 4)>(a, stream);
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
