// C ABI of libdsa.so (declared in include/dsa.h): argument validation on the
// host, workspace carving and dispatch to the gfx950 kernels.  Nothing is
// enqueued unless every check passes.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dsa.h"
#include "launch.h"

namespace {

thread_local std::string g_error;

dsa_status fail(dsa_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

bool aligned16(const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }
bool aligned4(const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 3u) == 0; }

#define DSA_CHECK(cond, st, ...)              \
  do {                                        \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

// Checks shared by every entry point.
dsa_status check_problem(const dsa_problem *p) {
  DSA_CHECK(p != nullptr, DSA_ERR_INVALID_ARGUMENT, "problem is NULL");
  DSA_CHECK(p->batch >= 1, DSA_ERR_INVALID_ARGUMENT, "batch must be >= 1 (got %d)", p->batch);
  DSA_CHECK(p->total_q >= 0 && p->total_kv >= 0, DSA_ERR_INVALID_ARGUMENT,
            "total_q and total_kv must be >= 0");
  DSA_CHECK(p->total_q <= INT32_MAX && p->total_kv <= INT32_MAX, DSA_ERR_UNSUPPORTED,
            "total_q and total_kv must fit int32 row indices");
  DSA_CHECK(p->max_q_len >= 0 && p->max_q_len <= p->total_q, DSA_ERR_INVALID_ARGUMENT,
            "max_q_len must be in [0, total_q] (got %lld, total_q %lld)",
            (long long)p->max_q_len, (long long)p->total_q);
  DSA_CHECK(p->max_kv_len >= 0 && p->max_kv_len <= p->total_kv, DSA_ERR_INVALID_ARGUMENT,
            "max_kv_len must be in [0, total_kv] (got %lld, total_kv %lld)",
            (long long)p->max_kv_len, (long long)p->total_kv);
  DSA_CHECK(p->q_offsets && p->kv_offsets && p->q_pos0, DSA_ERR_INVALID_ARGUMENT,
            "q_offsets, kv_offsets and q_pos0 must be non-NULL device arrays");
  DSA_CHECK(aligned4(p->q_offsets) && aligned4(p->kv_offsets) && aligned4(p->q_pos0),
            DSA_ERR_INVALID_ARGUMENT, "offset arrays must be 4-byte aligned");
  DSA_CHECK(p->topk >= 1, DSA_ERR_INVALID_ARGUMENT, "topk must be >= 1 (got %d)", p->topk);
  DSA_CHECK(p->topk <= 4096, DSA_ERR_UNSUPPORTED, "topk must be <= 4096 (got %d)", p->topk);
  return DSA_OK;
}

dsa_status check_indexer_dims(const dsa_problem *p) {
  DSA_CHECK(p->idx_heads >= 1, DSA_ERR_INVALID_ARGUMENT, "idx_heads must be >= 1");
  DSA_CHECK(p->idx_heads <= 128, DSA_ERR_UNSUPPORTED, "idx_heads must be <= 128 (got %d)",
            p->idx_heads);
  DSA_CHECK(p->idx_dim == 32 || p->idx_dim == 64 || p->idx_dim == 128, DSA_ERR_UNSUPPORTED,
            "idx_dim must be 32, 64 or 128 (got %d)", p->idx_dim);
  return DSA_OK;
}

bool mfma_attn_shape(const dsa_problem *p) {
  return p->d_latent == 512 && p->d_rope == 64 &&
         (p->heads == 32 || p->heads == 64 || p->heads == 128);
}

dsa_status check_attn_dims(const dsa_problem *p, bool paged = false) {
  DSA_CHECK(p->heads >= 1, DSA_ERR_INVALID_ARGUMENT, "heads must be >= 1");
  DSA_CHECK(p->heads <= 128, DSA_ERR_UNSUPPORTED, "heads must be <= 128 (got %d)", p->heads);
  DSA_CHECK(p->d_latent >= 1 && p->d_rope >= 0, DSA_ERR_INVALID_ARGUMENT,
            "d_latent must be >= 1 and d_rope >= 0");
  DSA_CHECK(mfma_attn_shape(p) || p->d_latent + p->d_rope <= 1024, DSA_ERR_UNSUPPORTED,
            "d_latent + d_rope must be <= 1024 outside the (512, 64) MFMA shape");
  // The MFMA path addresses a sequence's rows with 32-bit byte offsets (the
  // paged path with 64-bit addresses).
  DSA_CHECK(paged || !mfma_attn_shape(p) || p->max_kv_len <= (int64_t)(UINT32_MAX / 1152u), DSA_ERR_UNSUPPORTED,
            "max_kv_len must be <= %u for the (512, 64) attention shape (got %lld)",
            (unsigned)(UINT32_MAX / 1152u), (long long)p->max_kv_len);
  DSA_CHECK(std::isfinite(p->softmax_scale) && p->softmax_scale > 0.f, DSA_ERR_INVALID_ARGUMENT,
            "softmax_scale must be finite and > 0");
  return DSA_OK;
}

dsa_status check_ld(const dsa_problem *p, int64_t ld) {
  DSA_CHECK(ld >= p->max_kv_len && ld >= 1, DSA_ERR_INVALID_ARGUMENT,
            "ld_scores (%lld) must be >= max_kv_len (%lld) and >= 1", (long long)ld,
            (long long)p->max_kv_len);
  DSA_CHECK(ld % 4 == 0, DSA_ERR_INVALID_ARGUMENT, "ld_scores must be a multiple of 4");
  DSA_CHECK(p->total_q == 0 || ld <= INT64_MAX / 4 / p->total_q, DSA_ERR_INVALID_ARGUMENT,
            "scores matrix size overflows");
  return DSA_OK;
}

// A paged-cache description consistent with the problem.
dsa_status check_paged(const dsa_problem *p, const dsa_paged_kv *pg) {
  DSA_CHECK(pg != nullptr, DSA_ERR_INVALID_ARGUMENT, "paged-cache description is NULL");
  DSA_CHECK(pg->block_table != nullptr && aligned4(pg->block_table), DSA_ERR_INVALID_ARGUMENT,
            "block_table must be a non-NULL, 4-byte aligned device array");
  DSA_CHECK(pg->block_size >= 64 && (pg->block_size & (pg->block_size - 1)) == 0, DSA_ERR_UNSUPPORTED,
            "block_size must be a power of two >= 64 (got %d)", pg->block_size);
  DSA_CHECK(pg->max_blocks >= 1, DSA_ERR_INVALID_ARGUMENT, "max_blocks must be >= 1");
  DSA_CHECK((int64_t)pg->max_blocks * pg->block_size >= p->max_kv_len, DSA_ERR_INVALID_ARGUMENT,
            "max_blocks * block_size (%lld) must cover max_kv_len (%lld)",
            (long long)pg->max_blocks * pg->block_size, (long long)p->max_kv_len);
  DSA_CHECK(pg->num_blocks >= 1, DSA_ERR_INVALID_ARGUMENT, "num_blocks must be >= 1");
  DSA_CHECK(p->max_kv_len <= INT32_MAX, DSA_ERR_UNSUPPORTED, "max_kv_len must fit int32");
  DSA_CHECK(pg->num_blocks <= INT32_MAX / pg->block_size, DSA_ERR_UNSUPPORTED,
            "num_blocks * block_size must be below 2^31");
  DSA_CHECK((int64_t)p->batch * pg->max_blocks <= INT32_MAX, DSA_ERR_UNSUPPORTED,
            "batch * max_blocks must fit int32");
  return DSA_OK;
}

dsa::PagedKV paged_of(const dsa_paged_kv *pg) {
  dsa::PagedKV k;
  k.table = pg ? pg->block_table : nullptr;
  k.block_shift = 0;
  if (pg) while ((1 << k.block_shift) < pg->block_size) ++k.block_shift;
  k.max_blocks = pg ? pg->max_blocks : 0;
  k.num_blocks = pg ? (int32_t)pg->num_blocks : 0;
  return k;
}

dsa_status check_ptr(const void *ptr, bool needed, const char *name) {
  if (!needed) return DSA_OK;
  DSA_CHECK(ptr != nullptr, DSA_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  DSA_CHECK(aligned16(ptr), DSA_ERR_INVALID_ARGUMENT, "%s must be 16-byte aligned", name);
  return DSA_OK;
}

#define DSA_TRY(expr)                    \
  do {                                   \
    dsa_status st_ = (expr);             \
    if (st_ != DSA_OK) return st_;       \
  } while (0)

dsa::SeqLayout layout_of(const dsa_problem *p) {
  dsa::SeqLayout L;
  L.q_offsets = p->q_offsets;
  L.kv_offsets = p->kv_offsets;
  L.q_pos0 = p->q_pos0;
  L.batch = p->batch;
  L.total_q = p->total_q;
  L.total_kv = p->total_kv;
  L.max_q_len = p->max_q_len;
  L.max_kv_len = p->max_kv_len;
  return L;
}

dsa_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return DSA_OK;
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#ifdef DSA_DEBUG
// Debug builds: the device arrays the kernels index with -- the sequence
// offsets and first positions, and a paged cache's block table -- are copied
// to the host (after synchronizing the stream) and checked before anything
// is launched.  Release builds cannot check them and only clamp every index
// derived from them inside the kernels.
dsa_status debug_check_layout(const dsa_problem *p, const dsa_paged_kv *pg, void *stream) {
  const int B = p->batch;
  std::vector<int32_t> qo(B + 1), ko(B + 1), p0(B);
  DSA_TRY(hip_status(hipStreamSynchronize(static_cast<hipStream_t>(stream)), "debug: stream synchronize"));
  DSA_TRY(hip_status(hipMemcpy(qo.data(), p->q_offsets, qo.size() * 4, hipMemcpyDeviceToHost),
                     "debug: copying q_offsets"));
  DSA_TRY(hip_status(hipMemcpy(ko.data(), p->kv_offsets, ko.size() * 4, hipMemcpyDeviceToHost),
                     "debug: copying kv_offsets"));
  DSA_TRY(hip_status(hipMemcpy(p0.data(), p->q_pos0, p0.size() * 4, hipMemcpyDeviceToHost),
                     "debug: copying q_pos0"));
  DSA_CHECK(qo[0] == 0 && qo[B] == p->total_q, DSA_ERR_INVALID_ARGUMENT,
            "debug: q_offsets must run from 0 to total_q (%lld), found %d .. %d",
            (long long)p->total_q, qo[0], qo[B]);
  DSA_CHECK(ko[0] == 0 && ko[B] == p->total_kv, DSA_ERR_INVALID_ARGUMENT,
            "debug: kv_offsets must run from 0 to total_kv (%lld), found %d .. %d",
            (long long)p->total_kv, ko[0], ko[B]);
  for (int b = 0; b < B; ++b) {
    const int64_t ql = (int64_t)qo[b + 1] - qo[b], kl = (int64_t)ko[b + 1] - ko[b];
    DSA_CHECK(ql >= 0 && ql <= p->max_q_len, DSA_ERR_INVALID_ARGUMENT,
              "debug: sequence %d has %lld query rows (max_q_len %lld)", b, (long long)ql,
              (long long)p->max_q_len);
    DSA_CHECK(kl >= 0 && kl <= p->max_kv_len, DSA_ERR_INVALID_ARGUMENT,
              "debug: sequence %d has %lld keys (max_kv_len %lld)", b, (long long)kl,
              (long long)p->max_kv_len);
    DSA_CHECK(p0[b] >= 0 && p0[b] + ql <= kl, DSA_ERR_INVALID_ARGUMENT,
              "debug: sequence %d: q_pos0 (%d) + query rows (%lld) exceeds its keys (%lld)", b, p0[b],
              (long long)ql, (long long)kl);
  }
  if (pg != nullptr) {
    std::vector<int32_t> tab((size_t)B * pg->max_blocks);
    DSA_TRY(hip_status(hipMemcpy(tab.data(), pg->block_table, tab.size() * 4, hipMemcpyDeviceToHost),
                       "debug: copying block_table"));
    for (int b = 0; b < B; ++b) {
      const int64_t used = ((int64_t)ko[b + 1] - ko[b] + pg->block_size - 1) / pg->block_size;
      for (int64_t j = 0; j < used; ++j) {
        const int32_t v = tab[(size_t)b * pg->max_blocks + j];
        DSA_CHECK(v >= 0 && v < pg->num_blocks, DSA_ERR_INVALID_ARGUMENT,
                  "debug: block_table[%d][%lld] = %d is outside [0, %lld)", b, (long long)j, v,
                  (long long)pg->num_blocks);
      }
    }
  }
  return DSA_OK;
}
#define DSA_DEBUG_CHECK(p, pg, stream) DSA_TRY(debug_check_layout((p), (pg), (stream)))
#else
#define DSA_DEBUG_CHECK(p, pg, stream) ((void)0)
#endif

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Leading dimension of the scores matrix dsa_forward keeps in its workspace.
int64_t forward_ld(const dsa_problem *p) {
  const int64_t n = p->max_kv_len < 1 ? 1 : p->max_kv_len;
  return (n + 63) / 64 * 64;
}

dsa::AttnArgs attn_args(const dsa_problem *p, const uint16_t *q, const uint16_t *kv,
                        const int32_t *idx, uint16_t *out, float *lse, void *ws, size_t wsb,
                        const dsa_paged_kv *pg = nullptr) {
  dsa::AttnArgs a;
  a.seq = layout_of(p);
  a.pg = paged_of(pg);
  a.q = q;
  a.kv = kv;
  a.idx = idx;
  a.out = out;
  a.lse = lse;
  a.heads = p->heads;
  a.d_latent = p->d_latent;
  a.d_rope = p->d_rope;
  a.k = p->topk;
  a.scale = p->softmax_scale;
  a.workspace = ws;
  a.workspace_bytes = wsb;
  a.nsplit = 1;
  return a;
}

dsa::TopkArgs topk_args(const dsa_problem *p, const float *scores, int64_t ld, int32_t *idx,
                        void *ws = nullptr, size_t wsb = 0) {
  dsa::TopkArgs a;
  a.seq = layout_of(p);
  a.scores = scores;
  a.ld = ld;
  a.idx = idx;
  a.k = p->topk;
  a.workspace = ws;
  a.workspace_bytes = wsb;
  a.seg_len = 0;
  a.nseg = 0;
  a.fuse = dsa::FuseArgs{};
  return a;
}

dsa::IndexerArgs indexer_args(const dsa_problem *p, const uint8_t *q_fp8, const float *q_scale,
                              const float *w, const uint8_t *k_fp8, const float *k_scale,
                              float *scores, int64_t ld, const dsa_paged_kv *pg = nullptr) {
  dsa::IndexerArgs a;
  a.seq = layout_of(p);
  a.pg = paged_of(pg);
  a.q_fp8 = q_fp8;
  a.q_scale = q_scale;
  a.w = w;
  a.k_fp8 = k_fp8;
  a.k_scale = k_scale;
  a.scores = scores;
  a.ld = ld;
  a.idx_heads = p->idx_heads;
  a.idx_dim = p->idx_dim;
  a.fuse = dsa::FuseArgs{};
  return a;
}

dsa_status check_indexer_ptrs(const dsa_problem *p, const uint8_t *q_fp8, const float *q_scale,
                              const float *w, const uint8_t *k_fp8, const float *k_scale) {
  const bool q = p->total_q > 0, k = p->total_kv > 0;
  DSA_TRY(check_ptr(q_fp8, q, "q_fp8"));
  DSA_TRY(check_ptr(q_scale, q, "q_scale"));
  DSA_TRY(check_ptr(w, q, "w"));
  DSA_TRY(check_ptr(k_fp8, k, "k_fp8"));
  DSA_TRY(check_ptr(k_scale, k, "k_scale"));
  return DSA_OK;
}

dsa_status check_attn_ptrs(const dsa_problem *p, const uint16_t *q, const uint16_t *kv,
                           uint16_t *out, float *lse) {
  const bool hq = p->total_q > 0;
  DSA_TRY(check_ptr(q, hq, "q"));
  DSA_TRY(check_ptr(kv, p->total_kv > 0, "kv"));
  DSA_TRY(check_ptr(out, hq, "out"));
  if (lse != nullptr) DSA_TRY(check_ptr(lse, hq, "lse"));
  return DSA_OK;
}

size_t ws_attn(const dsa_problem *p) {
  return dsa::sparse_attn_workspace_bytes(attn_args(p, nullptr, nullptr, nullptr, nullptr,
                                                    nullptr, nullptr, 0));
}
size_t ws_topk(const dsa_problem *p, int64_t ld) {
  return dsa::topk_workspace_bytes(topk_args(p, nullptr, ld, nullptr));
}
size_t ws_indexer_bwd(const dsa_problem *p) {
  dsa::IndexerBwdArgs a{};
  a.seq = layout_of(p);
  a.idx_heads = p->idx_heads;
  a.idx_dim = p->idx_dim;
  a.k = p->topk;
  return dsa::indexer_bwd_workspace_bytes(a);
}

// Layout of dsa_forward's workspace: scores | indices | top-k scratch | attention scratch.
// dsa_forward_fused selects from what the decode indexer leaves per 1024-key
// chunk instead of from scores: no scores region, and the top-k scratch holds
// the chunks' data.
struct ForwardWs {
  size_t scores, idx, topk, attn, total;
  bool fused;
};
ForwardWs forward_ws(const dsa_problem *p, bool fuse = false) {
  ForwardWs w;
  const int64_t ld = forward_ld(p);
  const dsa::SeqLayout L = layout_of(p);
  w.fused = fuse && dsa::fuse_eligible(L);
  w.scores = w.fused ? 0 : round_up((size_t)p->total_q * (size_t)ld * sizeof(float), 256);
  w.idx = round_up((size_t)p->total_q * (size_t)p->topk * sizeof(int32_t), 256);
  w.topk = round_up(w.fused ? dsa::fuse_workspace_bytes(L) : ws_topk(p, ld), 256);
  w.attn = round_up(ws_attn(p), 256);
  w.total = w.scores + w.idx + w.topk + w.attn;
  return w;
}

// The fused top-k's buffers inside the top-k scratch (fuse_workspace_bytes).
dsa::FuseArgs fuse_layout(const dsa_problem *p, void *base) {
  dsa::FuseArgs f;
  f.nchunk = (int32_t)((p->max_kv_len + dsa::kFuseChunk - 1) / dsa::kFuseChunk);
  const size_t slots = (size_t)p->total_q * (size_t)f.nchunk;
  uint8_t *b = static_cast<uint8_t *>(base);
  f.tab = reinterpret_cast<uint32_t *>(b);
  f.nz = reinterpret_cast<uint32_t *>(b + round_up(slots * dsa::kFuseTabCap * 4, 256));
  f.list = reinterpret_cast<uint32_t *>(b + round_up(slots * dsa::kFuseTabCap * 4, 256) +
                                        round_up(slots * 4, 256));
  return f;
}

}  // namespace

extern "C" {

const char *dsa_last_error(void) { return g_error.c_str(); }

#ifdef DSA_DEBUG
const char *dsa_version(void) { return "dsa 0.1.0 gfx950 debug"; }
#else
const char *dsa_version(void) { return "dsa 0.1.0 gfx950"; }
#endif

size_t dsa_workspace_bytes(const dsa_problem *p, int which) {
  if (check_problem(p) != DSA_OK) return (size_t)-1;
  switch (which) {
    case DSA_WS_TOPK: return ws_topk(p, forward_ld(p));
    case DSA_WS_ATTN: return ws_attn(p);
    case DSA_WS_FORWARD: return forward_ws(p).total;
    case DSA_WS_FORWARD_FUSED:
      if (!dsa::fuse_eligible(layout_of(p))) {
        fail(DSA_ERR_UNSUPPORTED, "dsa_forward_fused serves at most two query rows per sequence "
             "and rows of at most %lld keys", (long long)dsa::kFuseMaxLen);
        return (size_t)-1;
      }
      return forward_ws(p, true).total;
    case DSA_WS_INDEXER_BWD: return ws_indexer_bwd(p);
    case DSA_WS_ATTN_PREFILL:
      if (p->max_kv_len > dsa::kMhaMaxKvLen) {
        fail(DSA_ERR_UNSUPPORTED, "dsa_sparse_attn_prefill serves max_kv_len <= %lld",
             (long long)dsa::kMhaMaxKvLen);
        return (size_t)-1;
      }
      return dsa::mha_workspace_bytes(layout_of(p));
    default: fail(DSA_ERR_INVALID_ARGUMENT, "unknown workspace selector %d", which); return (size_t)-1;
  }
}

}  // extern "C"

namespace {

dsa_status indexer_impl(const dsa_problem *p, const dsa_paged_kv *pg, const uint8_t *q_fp8,
                        const float *q_scale, const float *w, const uint8_t *k_fp8,
                        const float *k_scale, float *scores, int64_t ld_scores, void *stream) {
  DSA_TRY(check_problem(p));
  if (pg != nullptr) DSA_TRY(check_paged(p, pg));
  DSA_TRY(check_indexer_dims(p));
  DSA_TRY(check_ld(p, ld_scores));
  DSA_TRY(check_indexer_ptrs(p, q_fp8, q_scale, w, k_fp8, k_scale));
  DSA_TRY(check_ptr(scores, p->total_q > 0, "scores"));
  DSA_DEBUG_CHECK(p, pg, stream);
  return hip_status(dsa::launch_indexer(indexer_args(p, q_fp8, q_scale, w, k_fp8, k_scale,
                                                     scores, ld_scores, pg),
                                        static_cast<hipStream_t>(stream)),
                    "indexer launch");
}

}  // namespace

extern "C" {

dsa_status dsa_indexer_scores(const dsa_problem *p, const uint8_t *q_fp8, const float *q_scale,
                              const float *w, const uint8_t *k_fp8, const float *k_scale,
                              float *scores, int64_t ld_scores, void *stream) {
  return indexer_impl(p, nullptr, q_fp8, q_scale, w, k_fp8, k_scale, scores, ld_scores, stream);
}

dsa_status dsa_indexer_scores_paged(const dsa_problem *p, const dsa_paged_kv *pg,
                                    const uint8_t *q_fp8, const float *q_scale, const float *w,
                                    const uint8_t *k_cache, const float *ks_cache, float *scores,
                                    int64_t ld_scores, void *stream) {
  if (pg == nullptr) return fail(DSA_ERR_INVALID_ARGUMENT, "paged-cache description is NULL");
  return indexer_impl(p, pg, q_fp8, q_scale, w, k_cache, ks_cache, scores, ld_scores, stream);
}

dsa_status dsa_topk(const dsa_problem *p, const float *scores, int64_t ld_scores,
                    int32_t *topk_idx, void *workspace, size_t workspace_bytes, void *stream) {
  DSA_TRY(check_problem(p));
  DSA_TRY(check_ld(p, ld_scores));
  DSA_TRY(check_ptr(scores, p->total_q > 0, "scores"));
  DSA_TRY(check_ptr(topk_idx, p->total_q > 0, "topk_idx"));
  const size_t need = ws_topk(p, ld_scores);
  DSA_CHECK(workspace_bytes >= need && (need == 0 || workspace != nullptr), DSA_ERR_WORKSPACE,
            "top-k workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  DSA_CHECK(need == 0 || aligned16(workspace), DSA_ERR_INVALID_ARGUMENT,
            "workspace must be 16-byte aligned");
  DSA_DEBUG_CHECK(p, nullptr, stream);
  return hip_status(dsa::launch_topk(topk_args(p, scores, ld_scores, topk_idx, workspace,
                                               workspace_bytes),
                                     static_cast<hipStream_t>(stream)),
                    "top-k launch");
}

}  // extern "C"

namespace {

dsa_status attn_impl(const dsa_problem *p, const dsa_paged_kv *pg, const uint16_t *q,
                     const uint16_t *kv, const int32_t *topk_idx, uint16_t *out, float *lse,
                     void *workspace, size_t workspace_bytes, void *stream) {
  DSA_TRY(check_problem(p));
  if (pg != nullptr) DSA_TRY(check_paged(p, pg));
  DSA_TRY(check_attn_dims(p, pg != nullptr));
  DSA_TRY(check_attn_ptrs(p, q, kv, out, lse));
  DSA_TRY(check_ptr(topk_idx, p->total_q > 0, "topk_idx"));
  const size_t need = ws_attn(p);
  DSA_CHECK(workspace_bytes >= need && (need == 0 || workspace != nullptr), DSA_ERR_WORKSPACE,
            "attention workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  DSA_CHECK(need == 0 || aligned16(workspace), DSA_ERR_INVALID_ARGUMENT,
            "workspace must be 16-byte aligned");
  DSA_DEBUG_CHECK(p, pg, stream);
  return hip_status(dsa::launch_sparse_attn(attn_args(p, q, kv, topk_idx, out, lse, workspace,
                                                      workspace_bytes, pg),
                                            static_cast<hipStream_t>(stream)),
                    "attention launch");
}

dsa_status prefill_attn_impl(const dsa_problem *p, const uint16_t *q, const uint16_t *k_nope,
                             const uint16_t *k_rope, const uint16_t *v, const int32_t *topk_idx,
                             uint16_t *out, float *lse, void *workspace, size_t workspace_bytes,
                             void *stream) {
  DSA_TRY(check_problem(p));
  DSA_CHECK(p->heads >= 1, DSA_ERR_INVALID_ARGUMENT, "heads must be >= 1");
  DSA_CHECK(p->heads <= 128, DSA_ERR_UNSUPPORTED, "heads must be <= 128 (got %d)", p->heads);
  DSA_CHECK(p->d_rope == 64, DSA_ERR_UNSUPPORTED,
            "the prefill form needs d_rope = 64 (per-head keys 128 + 64; got %d)", p->d_rope);
  DSA_CHECK(p->max_kv_len <= dsa::kMhaMaxKvLen, DSA_ERR_UNSUPPORTED,
            "the prefill form serves max_kv_len <= %lld (got %lld)", (long long)dsa::kMhaMaxKvLen,
            (long long)p->max_kv_len);
  DSA_CHECK(std::isfinite(p->softmax_scale) && p->softmax_scale > 0.f, DSA_ERR_INVALID_ARGUMENT,
            "softmax_scale must be finite and > 0");
  const bool hq = p->total_q > 0, hk = p->total_kv > 0;
  DSA_TRY(check_ptr(q, hq, "q"));
  DSA_TRY(check_ptr(k_nope, hk, "k_nope"));
  DSA_TRY(check_ptr(k_rope, hk, "k_rope"));
  DSA_TRY(check_ptr(v, hk, "v"));
  DSA_TRY(check_ptr(topk_idx, hq, "topk_idx"));
  DSA_TRY(check_ptr(out, hq, "out"));
  if (lse != nullptr) DSA_TRY(check_ptr(lse, hq, "lse"));
  const size_t need = dsa::mha_workspace_bytes(layout_of(p));
  DSA_CHECK(workspace_bytes >= need && workspace != nullptr, DSA_ERR_WORKSPACE,
            "prefill attention workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  DSA_CHECK(aligned16(workspace), DSA_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  DSA_DEBUG_CHECK(p, nullptr, stream);
  dsa::MhaArgs a;
  a.seq = layout_of(p);
  a.q = q;
  a.k_nope = k_nope;
  a.k_rope = k_rope;
  a.v = v;
  a.idx = topk_idx;
  a.out = out;
  a.lse = lse;
  a.heads = p->heads;
  a.k = p->topk;
  a.scale = p->softmax_scale;
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  return hip_status(dsa::launch_mha_prefill(a, static_cast<hipStream_t>(stream)),
                    "prefill attention launch");
}

dsa_status forward_impl(const dsa_problem *p, const dsa_paged_kv *pg, const uint8_t *q_fp8,
                        const float *q_scale, const float *w, const uint8_t *k_fp8,
                        const float *k_scale, const uint16_t *q, const uint16_t *kv, uint16_t *out,
                        float *lse, int32_t *topk_idx_out, void *workspace, size_t workspace_bytes,
                        void *stream, bool fuse = false) {
  DSA_TRY(check_problem(p));
  if (pg != nullptr) DSA_TRY(check_paged(p, pg));
  DSA_TRY(check_indexer_dims(p));
  DSA_TRY(check_attn_dims(p, pg != nullptr));
  DSA_CHECK(!fuse || dsa::fuse_eligible(layout_of(p)), DSA_ERR_UNSUPPORTED,
            "dsa_forward_fused serves at most two query rows per sequence and rows of at most "
            "%lld keys", (long long)dsa::kFuseMaxLen);
  DSA_TRY(check_indexer_ptrs(p, q_fp8, q_scale, w, k_fp8, k_scale));
  DSA_TRY(check_attn_ptrs(p, q, kv, out, lse));
  if (topk_idx_out != nullptr) DSA_TRY(check_ptr(topk_idx_out, p->total_q > 0, "topk_idx_out"));
  const ForwardWs ws = forward_ws(p, fuse);
  DSA_CHECK(workspace_bytes >= ws.total && workspace != nullptr, DSA_ERR_WORKSPACE,
            "forward workspace needs %zu bytes (got %zu)", ws.total, workspace_bytes);
  DSA_CHECK(aligned16(workspace), DSA_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  DSA_DEBUG_CHECK(p, pg, stream);
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t *base = static_cast<uint8_t *>(workspace);
  float *scores = reinterpret_cast<float *>(base);
  int32_t *idx = topk_idx_out != nullptr ? topk_idx_out
                                         : reinterpret_cast<int32_t *>(base + ws.scores);
  void *topk_ws = base + ws.scores + ws.idx;
  void *attn_ws = base + ws.scores + ws.idx + ws.topk;
  const int64_t ld = forward_ld(p);
  dsa::IndexerArgs ia = indexer_args(p, q_fp8, q_scale, w, k_fp8, k_scale, scores, ld, pg);
  dsa::TopkArgs ta = topk_args(p, scores, ld, idx, topk_ws, ws.topk);
  if (ws.fused) ia.fuse = ta.fuse = fuse_layout(p, topk_ws);
  DSA_TRY(hip_status(dsa::launch_indexer(ia, st), "indexer launch"));
  DSA_TRY(hip_status(ws.fused ? dsa::launch_topk_fused(ta, st) : dsa::launch_topk(ta, st),
                     "top-k launch"));
  return hip_status(dsa::launch_sparse_attn(attn_args(p, q, kv, idx, out, lse, attn_ws, ws.attn, pg),
                                            st),
                    "attention launch");
}

}  // namespace

extern "C" {

dsa_status dsa_sparse_attn(const dsa_problem *p, const uint16_t *q, const uint16_t *kv,
                           const int32_t *topk_idx, uint16_t *out, float *lse, void *workspace,
                           size_t workspace_bytes, void *stream) {
  return attn_impl(p, nullptr, q, kv, topk_idx, out, lse, workspace, workspace_bytes, stream);
}

dsa_status dsa_sparse_attn_prefill(const dsa_problem *p, const uint16_t *q, const uint16_t *k_nope,
                                   const uint16_t *k_rope, const uint16_t *v,
                                   const int32_t *topk_idx, uint16_t *out, float *lse,
                                   void *workspace, size_t workspace_bytes, void *stream) {
  return prefill_attn_impl(p, q, k_nope, k_rope, v, topk_idx, out, lse, workspace, workspace_bytes,
                           stream);
}

dsa_status dsa_sparse_attn_paged(const dsa_problem *p, const dsa_paged_kv *pg, const uint16_t *q,
                                 const uint16_t *kv_cache, const int32_t *topk_idx, uint16_t *out,
                                 float *lse, void *workspace, size_t workspace_bytes, void *stream) {
  if (pg == nullptr) return fail(DSA_ERR_INVALID_ARGUMENT, "paged-cache description is NULL");
  return attn_impl(p, pg, q, kv_cache, topk_idx, out, lse, workspace, workspace_bytes, stream);
}

dsa_status dsa_forward(const dsa_problem *p, const uint8_t *q_fp8, const float *q_scale,
                       const float *w, const uint8_t *k_fp8, const float *k_scale,
                       const uint16_t *q, const uint16_t *kv, uint16_t *out, float *lse,
                       int32_t *topk_idx_out, void *workspace, size_t workspace_bytes,
                       void *stream) {
  return forward_impl(p, nullptr, q_fp8, q_scale, w, k_fp8, k_scale, q, kv, out, lse, topk_idx_out,
                      workspace, workspace_bytes, stream);
}

dsa_status dsa_forward_paged(const dsa_problem *p, const dsa_paged_kv *pg, const uint8_t *q_fp8,
                             const float *q_scale, const float *w, const uint8_t *k_cache,
                             const float *ks_cache, const uint16_t *q, const uint16_t *kv_cache,
                             uint16_t *out, float *lse, int32_t *topk_idx_out, void *workspace,
                             size_t workspace_bytes, void *stream) {
  if (pg == nullptr) return fail(DSA_ERR_INVALID_ARGUMENT, "paged-cache description is NULL");
  return forward_impl(p, pg, q_fp8, q_scale, w, k_cache, ks_cache, q, kv_cache, out, lse,
                      topk_idx_out, workspace, workspace_bytes, stream);
}

dsa_status dsa_forward_fused(const dsa_problem *p, const dsa_paged_kv *pg, const uint8_t *q_fp8,
                             const float *q_scale, const float *w, const uint8_t *k_fp8,
                             const float *k_scale, const uint16_t *q, const uint16_t *kv,
                             uint16_t *out, float *lse, int32_t *topk_idx_out, void *workspace,
                             size_t workspace_bytes, void *stream) {
  return forward_impl(p, pg, q_fp8, q_scale, w, k_fp8, k_scale, q, kv, out, lse, topk_idx_out,
                      workspace, workspace_bytes, stream, true);
}

}  // extern "C"

namespace {

dsa_status align_impl(const dsa_problem *p, const uint16_t *q, const uint16_t *kv, const float *lse,
                      const float *scores, int64_t ld_scores, const int32_t *topk_idx, float *loss,
                      float *grad, int64_t ld_grad, void *stream) {
  DSA_TRY(check_problem(p));
  DSA_TRY(check_attn_dims(p));
  DSA_TRY(check_ld(p, ld_scores));
  const bool hq = p->total_q > 0;
  DSA_TRY(check_ptr(q, hq, "q"));
  DSA_TRY(check_ptr(kv, p->total_kv > 0, "kv"));
  DSA_TRY(check_ptr(lse, hq, "lse"));
  DSA_TRY(check_ptr(scores, hq, "scores"));
  DSA_TRY(check_ptr(loss, hq, "loss"));
  DSA_TRY(check_ptr(grad, hq, "grad"));
  if (topk_idx != nullptr) DSA_TRY(check_ptr(topk_idx, hq, "topk_idx"));
  // With no query rows nothing is read or written (an empty index array may
  // reach here as NULL, which would otherwise select the dense form's bound).
  const int64_t need = topk_idx != nullptr ? (int64_t)p->topk : p->max_kv_len;
  DSA_CHECK(!hq || (ld_grad >= need && ld_grad >= 1), DSA_ERR_INVALID_ARGUMENT,
            "ld_grad (%lld) must be >= %s (%lld) and >= 1", (long long)ld_grad,
            topk_idx != nullptr ? "topk" : "max_kv_len", (long long)need);
  DSA_CHECK(!hq || ld_grad <= INT64_MAX / 4 / p->total_q, DSA_ERR_INVALID_ARGUMENT,
            "grad matrix size overflows");
  DSA_DEBUG_CHECK(p, nullptr, stream);
  dsa::AlignArgs a;
  a.seq = layout_of(p);
  a.q = q;
  a.kv = kv;
  a.lse = lse;
  a.scores = scores;
  a.ld_scores = ld_scores;
  a.idx = topk_idx;
  a.loss = loss;
  a.grad = grad;
  a.ld_grad = ld_grad;
  a.heads = p->heads;
  a.d_latent = p->d_latent;
  a.d_rope = p->d_rope;
  a.k = p->topk;
  a.scale = p->softmax_scale;
  return hip_status(dsa::launch_align_loss(a, static_cast<hipStream_t>(stream)),
                    "alignment loss launch");
}

}  // namespace

extern "C" {

dsa_status dsa_indexer_align_loss(const dsa_problem *p, const uint16_t *q, const uint16_t *kv,
                                  const float *lse, const float *scores, int64_t ld_scores,
                                  const int32_t *topk_idx, float *loss, float *grad,
                                  int64_t ld_grad, void *stream) {
  return align_impl(p, q, kv, lse, scores, ld_scores, topk_idx, loss, grad, ld_grad, stream);
}

}  // extern "C"

namespace {

dsa_status indexer_bwd_impl(const dsa_problem *p, const uint8_t *q_fp8, const float *q_scale,
                            const float *w, const uint8_t *k_fp8, const float *k_scale,
                            const int32_t *topk_idx, const float *grad, int64_t ld_grad, float *dq,
                            float *dw, float *dk, void *workspace, size_t workspace_bytes,
                            void *stream) {
  DSA_TRY(check_problem(p));
  DSA_TRY(check_indexer_dims(p));
  DSA_TRY(check_indexer_ptrs(p, q_fp8, q_scale, w, k_fp8, k_scale));
  const bool hq = p->total_q > 0;
  DSA_TRY(check_ptr(grad, hq, "grad"));
  DSA_TRY(check_ptr(dq, hq, "dq"));
  DSA_TRY(check_ptr(dw, hq, "dw"));
  DSA_TRY(check_ptr(dk, p->total_kv > 0, "dk"));
  if (topk_idx != nullptr) DSA_TRY(check_ptr(topk_idx, hq, "topk_idx"));
  // With no query rows nothing is read or written (an empty index array may
  // reach here as NULL, which would otherwise select the dense form's bound).
  const int64_t need = topk_idx != nullptr ? (int64_t)p->topk : p->max_kv_len;
  DSA_CHECK(!hq || (ld_grad >= need && ld_grad >= 1), DSA_ERR_INVALID_ARGUMENT,
            "ld_grad (%lld) must be >= %s (%lld) and >= 1", (long long)ld_grad,
            topk_idx != nullptr ? "topk" : "max_kv_len", (long long)need);
  DSA_CHECK(!hq || ld_grad <= INT64_MAX / 4 / p->total_q, DSA_ERR_INVALID_ARGUMENT,
            "grad matrix size overflows");
  DSA_CHECK(p->max_kv_len <= INT32_MAX, DSA_ERR_UNSUPPORTED, "max_kv_len must fit int32");
  if (workspace != nullptr && topk_idx != nullptr) {
    const size_t need = ws_indexer_bwd(p);
    DSA_CHECK(workspace_bytes >= need, DSA_ERR_WORKSPACE,
              "indexer backward workspace needs %zu bytes (got %zu)", need, workspace_bytes);
    DSA_CHECK(aligned16(workspace), DSA_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
    DSA_CHECK(p->total_kv / 64 < INT32_MAX, DSA_ERR_UNSUPPORTED, "total_kv too large for the workspace path");
  }
  DSA_DEBUG_CHECK(p, nullptr, stream);
  dsa::IndexerBwdArgs a{};
  a.seq = layout_of(p);
  a.q_fp8 = q_fp8;
  a.q_scale = q_scale;
  a.w = w;
  a.k_fp8 = k_fp8;
  a.k_scale = k_scale;
  a.idx = topk_idx;
  a.grad = grad;
  a.ld_grad = ld_grad;
  a.dq = dq;
  a.dw = dw;
  a.dk = dk;
  a.idx_heads = p->idx_heads;
  a.idx_dim = p->idx_dim;
  a.k = p->topk;
  // the dense form and the fp32 path take no workspace
  a.workspace = topk_idx != nullptr ? workspace : nullptr;
  a.workspace_bytes = workspace_bytes;
  return hip_status(dsa::launch_indexer_backward(a, static_cast<hipStream_t>(stream)),
                    "indexer backward launch");
}

}  // namespace

extern "C" {

dsa_status dsa_indexer_backward(const dsa_problem *p, const uint8_t *q_fp8, const float *q_scale,
                                const float *w, const uint8_t *k_fp8, const float *k_scale,
                                const int32_t *topk_idx, const float *grad, int64_t ld_grad,
                                float *dq, float *dw, float *dk, void *workspace,
                                size_t workspace_bytes, void *stream) {
  return indexer_bwd_impl(p, q_fp8, q_scale, w, k_fp8, k_scale, topk_idx, grad, ld_grad, dq, dw,
                          dk, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// dsa_forward_noalloc: dsa_forward with its workspace in a fixed device array
// of this library, for callers that cannot allocate device memory.

namespace {

// One copy per GPU, made when the library's code object is loaded on that
// device and held until the process ends.  In host code this name is only a
// stand-in for the symbol: its device address comes from hipGetSymbolAddress
// (scratch_address below), and only that address is ever passed on.
static __device__ __align__(256) uint8_t scratch[DSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device (the first call on it) and kept.
dsa_status scratch_address(void **out) {
  int dev = -1;
  DSA_TRY(hip_status(hipGetDevice(&dev), "hipGetDevice"));
  DSA_CHECK(dev >= 0 && dev < kMaxDevices, DSA_ERR_UNSUPPORTED,
            "device %d is beyond the %d devices dsa_forward_noalloc tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *ptr = nullptr;
    DSA_TRY(hip_status(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"));
    DSA_CHECK(ptr != nullptr && aligned16(ptr), DSA_ERR_HIP, "scratch has no usable device address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

}  // namespace

extern "C" {

dsa_status dsa_forward_noalloc(const dsa_problem *p, const uint8_t *q_fp8, const float *q_scale,
                               const float *w, const uint8_t *k_fp8, const float *k_scale,
                               const uint16_t *q, const uint16_t *kv, uint16_t *out, float *lse,
                               int32_t *topk_idx_out, void *stream) {
  // Sizes first, so that an oversized problem is refused before any HIP call.
  DSA_TRY(check_problem(p));
  const size_t need = forward_ws(p).total;
  DSA_CHECK(need <= (size_t)DSA_NOALLOC_SCRATCH_BYTES, DSA_ERR_UNSUPPORTED,
            "dsa_forward_noalloc: this problem needs %zu bytes of workspace, more than the "
            "%zu-byte device scratch; use dsa_forward with a caller workspace",
            need, (size_t)DSA_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  DSA_TRY(scratch_address(&ws));
  return forward_impl(p, nullptr, q_fp8, q_scale, w, k_fp8, k_scale, q, kv, out, lse, topk_idx_out,
                      ws, (size_t)DSA_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
