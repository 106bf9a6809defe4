// C ABI of the dynamic sparse prefill attention library: argument checks on the
// host, workspace carving, and kernel dispatch on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/dsa.h"
#include "internal.h"

using namespace dsa;

namespace {

thread_local std::string g_err;

dsa_status fail(dsa_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
dsa_status fail(dsa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

dsa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return DSA_OK;
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Every workspace size carries 256 bytes of slack, so the carving can start at
// the first 256-byte boundary of whatever the caller passed.
void* ws_base(void* ws) { return ws ? (void*)(((uintptr_t)ws + 255) & ~(uintptr_t)255) : nullptr; }

// Q, K, V, O and the indexer's q_idx / k_idx rows are read and written with
// 16-byte vector accesses and LDS DMA.
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

dsa_status check_shape(const dsa_shape* s) {
  if (!s) return fail(DSA_ERR_INVALID_ARG, "shape is null");
  if (s->batch < 1 || s->heads < 1 || s->kv_heads < 1 || s->q_len < 1 || s->kv_len < 1)
    return fail(DSA_ERR_INVALID_ARG, "shape sizes must be >= 1");
  if (s->heads % s->kv_heads != 0) return fail(DSA_ERR_INVALID_ARG, "heads %% kv_heads != 0");
  if (s->head_dim != 128) return fail(DSA_ERR_UNSUPPORTED, "head_dim %d (only 128 is built)", s->head_dim);
  if (s->q_offset < 0 || (int64_t)s->q_len + s->q_offset != s->kv_len)
    return fail(DSA_ERR_INVALID_ARG, "need q_len + q_offset == kv_len");
  if (s->kv_len >= (1 << 30)) return fail(DSA_ERR_INVALID_ARG, "kv_len too large");
  if (s->heads > 256) return fail(DSA_ERR_UNSUPPORTED, "more than 256 heads");
  if ((int64_t)s->batch * s->heads > kMaxHeadTable)
    return fail(DSA_ERR_UNSUPPORTED, "batch * heads > %d", kMaxHeadTable);
  return DSA_OK;
}

dsa_status check_heads(const dsa_shape* s, const int32_t* heads, int32_t n, HeadList& out) {
  if (!heads) return fail(DSA_ERR_INVALID_ARG, "heads is null");
  if (n < 1 || n > s->heads) return fail(DSA_ERR_INVALID_ARG, "n_heads %d out of range", n);
  bool seen[256] = {};
  out.n = n;
  for (int i = 0; i < n; ++i) {
    if (heads[i] < 0 || heads[i] >= s->heads) return fail(DSA_ERR_INVALID_ARG, "head index %d out of range", heads[i]);
    if (seen[heads[i]]) return fail(DSA_ERR_INVALID_ARG, "head %d listed twice", heads[i]);
    seen[heads[i]] = true;
    out.h[i] = heads[i];
  }
  return DSA_OK;
}

struct WsCarver {
  char* base;
  size_t off = 0;
  explicit WsCarver(void* p) : base((char*)ws_base(p)) {}
  template <class T>
  T* take(size_t count) {
    T* p = base ? (T*)(base + off) : nullptr;
    off = align256(off + count * sizeof(T));
    return p;
  }
};

size_t ws_vs(const dsa_shape* s, int n_heads) {
  return align256(vs_workspace_floats(s->batch * n_heads, s->kv_len) * 4) + 256;
}

// Pooled Q and K; the block scores stay on chip (a strip of query blocks per
// workgroup) unless a row of them is too long for that, then they go through
// the workspace.
size_t ws_block(const dsa_shape* s, int n_heads, int block) {
  const size_t nqb = (s->q_len + block - 1) / block, nkb = (s->kv_len + block - 1) / block;
  WsCarver c(nullptr);
  c.take<uint16_t>((size_t)s->batch * s->heads * nqb * 128);
  c.take<uint16_t>((size_t)s->batch * s->kv_heads * nkb * 128);
  if (block_strip_rows((int)nkb, nullptr) < 1) c.take<float>((size_t)s->batch * n_heads * nqb * nkb);
  return c.off + 256;
}

// Pooled Q and K, the per-strip partial masses, and vbar / sbar.
size_t ws_vs_pooled(const dsa_shape* s, int n_heads, int block) {
  const size_t nqb = (s->q_len + block - 1) / block, nkb = (s->kv_len + block - 1) / block;
  WsCarver c(nullptr);
  c.take<uint16_t>((size_t)s->batch * s->heads * nqb * 128);
  c.take<uint16_t>((size_t)s->batch * s->kv_heads * nkb * 128);
  c.take<float>((size_t)s->batch * n_heads * pooled_vs_partial_floats((int)nqb, (int)nkb));
  c.take<float>((size_t)s->batch * n_heads * (2 * nkb));
  return c.off + 256;
}

size_t ws_attn(const dsa_shape* s) { return align256(attn_workspace_bytes(s->batch, s->heads, s->kv_len)) + 256; }
bool block_size_ok(int b) { return b == 16 || b == 32 || b == 64 || b == 128; }

// The indexer over a batch: one sequence after another on the caller's stream,
// each with its slice of every per-sequence array; they share the workspace,
// which stream order keeps from overlapping.
hipError_t launch_indexer_batches(const IndexerArgs& a, int B, void* ws, hipStream_t st) {
  for (int b = 0; b < B; ++b) {
    IndexerArgs x = a;
    const size_t rows = (size_t)b * a.Nq;
    x.q_idx += rows * a.Hi * 128;
    x.k_idx += (size_t)b * a.Nk * 128;
    x.w += rows * a.Hi;
    x.tok += rows * a.tok_cap;
    x.tok_count += rows;
    if (x.route) x.route += rows * a.route_heads;
    if (x.cand_idx) {
      x.cand_idx += rows * a.cand_cap;
      x.cand_count += rows;
    }
    const hipError_t e = launch_indexer(x, ws, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* dsa_status_string(dsa_status s) {
  switch (s) {
    case DSA_OK: return "ok";
    case DSA_ERR_INVALID_ARG: return "invalid argument";
    case DSA_ERR_UNSUPPORTED: return "unsupported";
    case DSA_ERR_WORKSPACE: return "workspace missing or too small";
    case DSA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* dsa_last_error(void) { return g_err.c_str(); }

dsa_status dsa_workspace_size(int32_t op, const dsa_shape* shape, const int32_t* params, int32_t n_params,
                              size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(DSA_ERR_INVALID_ARG, "bytes is null");
  dsa_status st = check_shape(shape);
  if (st) return st;
  auto need = [&](int n) { return n_params >= n && (n == 0 || params != nullptr); };
  switch (op) {
    case DSA_OP_VS:
      if (!need(2) || params[0] < 1 || params[0] > shape->heads) return fail(DSA_ERR_INVALID_ARG, "VS params");
      *bytes = ws_vs(shape, params[0]);
      return DSA_OK;
    case DSA_OP_BLOCK:
      if (!need(2) || params[0] < 1 || params[0] > shape->heads || !block_size_ok(params[1]))
        return fail(DSA_ERR_INVALID_ARG, "BLOCK params");
      *bytes = ws_block(shape, params[0], params[1]);
      return DSA_OK;
    case DSA_OP_TOKENS:
      if (!need(3) || params[0] < 1 || params[1] < 0 || params[1] > params[0] || params[2] < 1)
        return fail(DSA_ERR_INVALID_ARG, "TOKENS params");
      *bytes = align256(indexer_workspace_bytes(shape->q_len, shape->kv_len, params[0], params[1], 0)) + 256;
      return DSA_OK;
    case DSA_OP_TOKENS_HIER:
      if (!need(4) || params[0] < 1 || params[1] < 1 || params[1] > params[0] || params[3] < 1 ||
          params[2] < params[3] || params[2] > kMaxCandidates)
        return fail(DSA_ERR_INVALID_ARG, "TOKENS_HIER params");
      *bytes = align256(indexer_workspace_bytes(shape->q_len, shape->kv_len, params[0], params[1], params[2])) + 256;
      return DSA_OK;
    case DSA_OP_ATTN:
      *bytes = ws_attn(shape);
      return DSA_OK;
    case DSA_OP_VS_POOLED:
      if (!need(2) || params[0] < 1 || params[0] > shape->heads || !block_size_ok(params[1]))
        return fail(DSA_ERR_INVALID_ARG, "VS_POOLED params");
      *bytes = ws_vs_pooled(shape, params[0], params[1]);
      return DSA_OK;
    default:
      return fail(DSA_ERR_INVALID_ARG, "unknown op %d", op);
  }
}

dsa_status build_index_ashape(const dsa_shape* shape, const int32_t* heads, int32_t n_heads, int32_t sink,
                              int32_t local, dsa_vs_index out, void* stream) {
  g_err.clear();
  dsa_status st = check_shape(shape);
  if (st) return st;
  HeadList hl;
  if ((st = check_heads(shape, heads, n_heads, hl))) return st;
  if (sink < 0 || local < 1) return fail(DSA_ERR_INVALID_ARG, "need sink >= 0 and local >= 1");
  const int nc = std::min(sink, shape->kv_len), nd = std::min(local, shape->kv_len);
  if (!out.cols || !out.cols_count || !out.diags || !out.diags_count)
    return fail(DSA_ERR_INVALID_ARG, "index set pointers are null");
  if (out.cols_cap < nc || out.diags_cap < nd) return fail(DSA_ERR_INVALID_ARG, "index set capacity too small");
  return hip_status(launch_ashape_fill(shape->batch, shape->heads, hl, nc, nd, out.cols, out.cols_count, out.cols_cap,
                                       out.diags, out.diags_count, out.diags_cap, (hipStream_t)stream),
                    "build_index_ashape");
}

dsa_status build_index_vs(const dsa_shape* shape, const void* q, const void* k, const int32_t* heads, int32_t n_heads,
                          int32_t last_q, int32_t nv, int32_t ns, dsa_vs_index out, float* v_scores, float* s_scores,
                          void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  dsa_status st = check_shape(shape);
  if (st) return st;
  HeadList hl;
  if ((st = check_heads(shape, heads, n_heads, hl))) return st;
  if (!q || !k) return fail(DSA_ERR_INVALID_ARG, "q or k is null");
  if (!aligned16(q) || !aligned16(k)) return fail(DSA_ERR_INVALID_ARG, "q and k must be 16-byte aligned");
  if (last_q < 1 || last_q > 64 || last_q > shape->q_len) return fail(DSA_ERR_INVALID_ARG, "last_q out of range");
  if (nv < 0 || ns < 0 || nv > shape->kv_len || ns > shape->kv_len) return fail(DSA_ERR_INVALID_ARG, "budgets out of range");
  if (!out.cols || !out.cols_count || !out.diags || !out.diags_count)
    return fail(DSA_ERR_INVALID_ARG, "index set pointers are null");
  if (out.cols_cap < nv || out.diags_cap < ns) return fail(DSA_ERR_INVALID_ARG, "index set capacity too small");
  const size_t need = ws_vs(shape, n_heads);
  if (!ws || ws_bytes < need) return fail(DSA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);

  const size_t R = (size_t)shape->batch * n_heads, Nk = shape->kv_len;
  WsCarver c(ws);
  float* vbuf = c.take<float>(R * Nk);
  float* sbuf = c.take<float>(R * Nk);
  size_t n_ml, n_dg;
  vs_part_floats((int)R, (int)Nk, &n_ml, &n_dg);
  float* pml = c.take<float>(n_ml);
  float* pdg = c.take<float>(n_dg);
  VsScoreArgs a;
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.B = shape->batch; a.H = shape->heads; a.Hkv = shape->kv_heads;
  a.Nq = shape->q_len; a.Nk = shape->kv_len; a.last_q = last_q;
  a.heads = hl;
  a.v_out = v_scores ? v_scores : vbuf;
  a.s_out = s_scores ? s_scores : sbuf;
  a.part_ml = pml;
  a.part_diag = pdg;
  hipStream_t s = (hipStream_t)stream;
  if ((st = hip_status(launch_vs_scores(a, s), "build_index_vs: scores"))) return st;
  return hip_status(launch_vs_select(a.v_out, a.s_out, shape->batch, shape->kv_len, shape->heads, hl, nv, ns, out.cols,
                                     out.cols_count, out.cols_cap, out.diags, out.diags_count, out.diags_cap, s),
                    "build_index_vs: select");
}

dsa_status build_index_block(const dsa_shape* shape, const void* q, const void* k, const int32_t* heads,
                             int32_t n_heads, int32_t block, int32_t mode, int32_t topk, float log_alpha,
                             int32_t force_first, int32_t force_diag, dsa_block_index out, void* qbar, void* kbar,
                             float* scores, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  dsa_status st = check_shape(shape);
  if (st) return st;
  HeadList hl;
  if ((st = check_heads(shape, heads, n_heads, hl))) return st;
  if (!q || !k) return fail(DSA_ERR_INVALID_ARG, "q or k is null");
  if (!aligned16(q) || !aligned16(k)) return fail(DSA_ERR_INVALID_ARG, "q and k must be 16-byte aligned");
  if (!block_size_ok(block)) return fail(DSA_ERR_UNSUPPORTED, "block %d (16, 32, 64 or 128)", block);
  if (shape->q_offset % block != 0)
    return fail(DSA_ERR_UNSUPPORTED, "the block rule needs q_offset (%d) to be a multiple of the block (%d)",
                shape->q_offset, block);
  if (mode != DSA_SELECT_TOPK && mode != DSA_SELECT_THRESHOLD) return fail(DSA_ERR_INVALID_ARG, "mode %d", mode);
  if (mode == DSA_SELECT_TOPK && topk < 0) return fail(DSA_ERR_INVALID_ARG, "topk < 0");
  if (mode == DSA_SELECT_THRESHOLD && !(log_alpha <= 0.f)) return fail(DSA_ERR_INVALID_ARG, "log_alpha must be <= 0");
  if (out.block != block) return fail(DSA_ERR_INVALID_ARG, "out.block != block");
  if (!out.idx || !out.count) return fail(DSA_ERR_INVALID_ARG, "index set pointers are null");
  const int nqb = (shape->q_len + block - 1) / block, nkb = (shape->kv_len + block - 1) / block;
  const int qb0 = shape->q_offset / block;          // the chunk's first query block, absolute
  const int forced = (force_first ? 1 : 0) + (force_diag ? 1 : 0);
  // the last query block sees key blocks [0, qb0 + nqb)
  const int need_cap = mode == DSA_SELECT_TOPK ? std::min(qb0 + nqb, topk + forced) : qb0 + nqb;
  if (out.cap < need_cap) return fail(DSA_ERR_INVALID_ARG, "out.cap %d < %d", out.cap, need_cap);
  const size_t need = ws_block(shape, n_heads, block);
  if (!ws || ws_bytes < need) return fail(DSA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);

  const bool on_chip = block_strip_rows(nkb, nullptr) >= 1;
  WsCarver c(ws);
  uint16_t* qb = c.take<uint16_t>((size_t)shape->batch * shape->heads * nqb * 128);
  uint16_t* kb = c.take<uint16_t>((size_t)shape->batch * shape->kv_heads * nkb * 128);
  float* sc = on_chip ? nullptr : c.take<float>((size_t)shape->batch * n_heads * nqb * nkb);
  if (qbar) qb = (uint16_t*)qbar;
  if (kbar) kb = (uint16_t*)kbar;
  if (scores) sc = scores;
  HeadList kvl;
  kvl.n = 0;
  bool kvseen[256] = {};
  const int rep = shape->heads / shape->kv_heads;
  for (int i = 0; i < hl.n; ++i) {
    const int kvh = hl.h[i] / rep;
    if (!kvseen[kvh]) { kvseen[kvh] = true; kvl.h[kvl.n++] = kvh; }
  }
  hipStream_t s = (hipStream_t)stream;
  if ((st = hip_status(launch_pool((const uint16_t*)q, shape->batch, shape->heads, shape->q_len, hl, block, qb, s),
                       "build_index_block: pool q")))
    return st;
  if ((st = hip_status(launch_pool((const uint16_t*)k, shape->batch, shape->kv_heads, shape->kv_len, kvl, block, kb, s),
                       "build_index_block: pool k")))
    return st;
  const float scale = (float)(1.0 / std::sqrt(128.0));
  if (on_chip)
    return hip_status(launch_block_index(qb, kb, shape->batch, shape->heads, shape->kv_heads, nqb, nkb, qb0, hl, scale,
                                         mode, topk, log_alpha, force_first, force_diag, out.idx, out.count, out.cap,
                                         scores, s),
                      "build_index_block: scores + select");
  if ((st = hip_status(launch_block_scores(qb, kb, shape->batch, shape->heads, shape->kv_heads, nqb, nkb, qb0, hl, scale,
                                           sc, s),
                       "build_index_block: scores")))
    return st;
  return hip_status(launch_block_select(sc, shape->batch, shape->heads, nqb, nkb, qb0, hl, mode, topk, log_alpha,
                                        force_first, force_diag, out.idx, out.count, out.cap, s),
                    "build_index_block: select");
}

dsa_status build_index_vs_pooled(const dsa_shape* shape, const void* q, const void* k, const int32_t* heads,
                                 int32_t n_heads, int32_t block, int32_t nv_blocks, int32_t ns_blocks,
                                 dsa_vs_index out, float* v_scores, float* s_scores, void* ws, size_t ws_bytes,
                                 void* stream) {
  g_err.clear();
  dsa_status st = check_shape(shape);
  if (st) return st;
  HeadList hl;
  if ((st = check_heads(shape, heads, n_heads, hl))) return st;
  if (!q || !k) return fail(DSA_ERR_INVALID_ARG, "q or k is null");
  if (!aligned16(q) || !aligned16(k)) return fail(DSA_ERR_INVALID_ARG, "q and k must be 16-byte aligned");
  if (!block_size_ok(block)) return fail(DSA_ERR_UNSUPPORTED, "block %d (16, 32, 64 or 128)", block);
  if (shape->q_offset % block != 0)
    return fail(DSA_ERR_UNSUPPORTED, "pooled discovery needs q_offset (%d) to be a multiple of the block (%d)",
                shape->q_offset, block);
  if (nv_blocks < 0 || ns_blocks < 0 || nv_blocks > kMaxPooledBlocks || ns_blocks > kMaxPooledBlocks)
    return fail(DSA_ERR_UNSUPPORTED, "nv_blocks and ns_blocks must be in [0, %d]", kMaxPooledBlocks);
  const int nqb = (shape->q_len + block - 1) / block, nkb = (shape->kv_len + block - 1) / block;
  if (block_strip_rows(nkb, nullptr) < 1)
    return fail(DSA_ERR_UNSUPPORTED, "%d key blocks: a row of block scores does not fit on chip", nkb);
  if (!out.cols || !out.cols_count || !out.diags || !out.diags_count)
    return fail(DSA_ERR_INVALID_ARG, "index set pointers are null");
  const int64_t need_c = std::min<int64_t>(shape->kv_len, (int64_t)nv_blocks * block);
  const int64_t need_d = std::min<int64_t>(shape->kv_len, (int64_t)ns_blocks * (2 * block - 1));
  if (out.cols_cap < need_c || out.diags_cap < need_d)
    return fail(DSA_ERR_INVALID_ARG, "index set capacity too small (need %lld columns, %lld diagonals)",
                (long long)need_c, (long long)need_d);
  const size_t need = ws_vs_pooled(shape, n_heads, block);
  if (!ws || ws_bytes < need) return fail(DSA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);

  const size_t R = (size_t)shape->batch * n_heads;
  WsCarver c(ws);
  uint16_t* qb = c.take<uint16_t>((size_t)shape->batch * shape->heads * nqb * 128);
  uint16_t* kb = c.take<uint16_t>((size_t)shape->batch * shape->kv_heads * nkb * 128);
  const size_t pf = pooled_vs_partial_floats(nqb, nkb);
  float* part = c.take<float>(R * pf);
  float* masses = c.take<float>(R * (2 * nkb));
  const int nstrips = (int)(pf / (size_t)(2 * nkb));
  float* vpart = part;
  float* spart = part + R * (size_t)nstrips * nkb;
  float* vbar = v_scores ? v_scores : masses;
  float* sbar = s_scores ? s_scores : masses + R * nkb;
  HeadList kvl;
  kvl.n = 0;
  bool kvseen[256] = {};
  const int rep = shape->heads / shape->kv_heads;
  for (int i = 0; i < hl.n; ++i) {
    const int kvh = hl.h[i] / rep;
    if (!kvseen[kvh]) { kvseen[kvh] = true; kvl.h[kvl.n++] = kvh; }
  }
  hipStream_t s = (hipStream_t)stream;
  if ((st = hip_status(launch_pool((const uint16_t*)q, shape->batch, shape->heads, shape->q_len, hl, block, qb, s),
                       "build_index_vs_pooled: pool q")))
    return st;
  if ((st = hip_status(launch_pool((const uint16_t*)k, shape->batch, shape->kv_heads, shape->kv_len, kvl, block, kb, s),
                       "build_index_vs_pooled: pool k")))
    return st;
  return hip_status(launch_pooled_vs(qb, kb, shape->batch, shape->heads, shape->kv_heads, nqb, nkb,
                                     shape->q_offset / block, shape->kv_len,
                                     block, hl, (float)(1.0 / std::sqrt(128.0)), vpart, spart, vbar, sbar, nv_blocks,
                                     ns_blocks, out.cols, out.cols_count, out.cols_cap, out.diags, out.diags_count,
                                     out.diags_cap, s),
                    "build_index_vs_pooled");
}

dsa_status build_index_tokens(const dsa_shape* shape, const void* q_idx, const void* k_idx, const float* w,
                              int32_t n_idx_heads, int32_t route_heads, int32_t route_block, int32_t topk,
                              dsa_token_index out, int32_t* route, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  dsa_status st = check_shape(shape);
  if (st) return st;
  if (!q_idx || !k_idx || !w) return fail(DSA_ERR_INVALID_ARG, "q_idx, k_idx or w is null");
  if (!aligned16(q_idx) || !aligned16(k_idx)) return fail(DSA_ERR_INVALID_ARG, "q_idx and k_idx must be 16-byte aligned");
  if (n_idx_heads < 1 || n_idx_heads > 64) return fail(DSA_ERR_UNSUPPORTED, "n_idx_heads must be in [1, 64]");
  if (route_heads < 0 || route_heads > n_idx_heads) return fail(DSA_ERR_INVALID_ARG, "route_heads out of range");
  if (route_heads > 8) return fail(DSA_ERR_UNSUPPORTED, "route_heads > 8");
  if (route_heads > 0 && !block_size_ok(route_block))
    return fail(DSA_ERR_UNSUPPORTED, "route_block %d (16, 32, 64 or 128)", route_block);
  // score rows are written through 32-bit buffer offsets (four rows per wave)
  if (shape->kv_len > (1 << 27)) return fail(DSA_ERR_UNSUPPORTED, "the indexer takes kv_len <= 2^27");
  if (topk < 1) return fail(DSA_ERR_INVALID_ARG, "topk < 1");
  if (!out.idx || !out.count) return fail(DSA_ERR_INVALID_ARG, "index set pointers are null");
  if (out.cap < std::min(topk, shape->kv_len)) return fail(DSA_ERR_INVALID_ARG, "out.cap < topk");
  const size_t need = align256(indexer_workspace_bytes(shape->q_len, shape->kv_len, n_idx_heads, route_heads, 0)) + 256;
  if (!ws || ws_bytes < need) return fail(DSA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  IndexerArgs a;
  a.cand = 0;
  a.cand_idx = nullptr; a.cand_count = nullptr; a.cand_cap = 0;
  a.q_idx = (const uint16_t*)q_idx;
  a.k_idx = (const uint16_t*)k_idx;
  a.w = w;
  a.Nq = shape->q_len; a.Nk = shape->kv_len; a.Hi = n_idx_heads; a.q_offset = shape->q_offset;
  a.route_heads = route_heads; a.topk = topk; a.route_block = route_heads > 0 ? route_block : 64;
  a.tok = out.idx; a.tok_count = out.count; a.tok_cap = out.cap;
  a.route = route;
  return hip_status(launch_indexer_batches(a, shape->batch, ws_base(ws), (hipStream_t)stream), "build_index_tokens");
}

dsa_status build_index_tokens_hier(const dsa_shape* shape, const void* q_idx, const void* k_idx, const float* w,
                                   int32_t n_idx_heads, int32_t route_heads, int32_t route_block, int32_t cand,
                                   int32_t topk,
                                   dsa_token_index out, const dsa_token_index* cands, int32_t* route, void* ws,
                                   size_t ws_bytes, void* stream) {
  g_err.clear();
  dsa_status st = check_shape(shape);
  if (st) return st;
  if (!q_idx || !k_idx || !w) return fail(DSA_ERR_INVALID_ARG, "q_idx, k_idx or w is null");
  if (!aligned16(q_idx) || !aligned16(k_idx)) return fail(DSA_ERR_INVALID_ARG, "q_idx and k_idx must be 16-byte aligned");
  if (n_idx_heads < 1 || n_idx_heads > 64) return fail(DSA_ERR_UNSUPPORTED, "n_idx_heads must be in [1, 64]");
  if (route_heads < 1 || route_heads > n_idx_heads) return fail(DSA_ERR_INVALID_ARG, "route_heads out of range");
  if (route_heads > 8) return fail(DSA_ERR_UNSUPPORTED, "route_heads > 8");
  if (!block_size_ok(route_block)) return fail(DSA_ERR_UNSUPPORTED, "route_block %d (16, 32, 64 or 128)", route_block);
  if (shape->kv_len > (1 << 27)) return fail(DSA_ERR_UNSUPPORTED, "the indexer takes kv_len <= 2^27");
  if (topk < 1) return fail(DSA_ERR_INVALID_ARG, "topk < 1");
  if (topk > kMaxTokensPerQuery) return fail(DSA_ERR_UNSUPPORTED, "topk > %d", kMaxTokensPerQuery);
  if (cand < topk || cand > kMaxCandidates) return fail(DSA_ERR_INVALID_ARG, "cand must be in [topk, %d]", kMaxCandidates);
  if (!out.idx || !out.count) return fail(DSA_ERR_INVALID_ARG, "index set pointers are null");
  if (out.cap < std::min(topk, shape->kv_len)) return fail(DSA_ERR_INVALID_ARG, "out.cap < topk");
  if (cands && (!cands->idx || !cands->count || cands->cap < cand))
    return fail(DSA_ERR_INVALID_ARG, "cands: null pointers or cap < cand");
  const size_t need =
      align256(indexer_workspace_bytes(shape->q_len, shape->kv_len, n_idx_heads, route_heads, cand)) + 256;
  if (!ws || ws_bytes < need) return fail(DSA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  IndexerArgs a;
  a.q_idx = (const uint16_t*)q_idx;
  a.k_idx = (const uint16_t*)k_idx;
  a.w = w;
  a.Nq = shape->q_len; a.Nk = shape->kv_len; a.Hi = n_idx_heads; a.q_offset = shape->q_offset;
  a.route_heads = route_heads; a.topk = topk; a.route_block = route_block;
  a.tok = out.idx; a.tok_count = out.count; a.tok_cap = out.cap;
  a.route = route;
  a.cand = cand;
  a.cand_idx = cands ? cands->idx : nullptr;
  a.cand_count = cands ? cands->count : nullptr;
  a.cand_cap = cands ? cands->cap : cand;
  return hip_status(launch_indexer_batches(a, shape->batch, ws_base(ws), (hipStream_t)stream),
                    "build_index_tokens_hier");
}

}  // extern "C"

namespace {

// Argument checks and kernel arguments shared by both attention entry points.
dsa_status prepare_attn(const dsa_shape* shape, const void* q, const void* k, const void* v, const int32_t* head_kind,
                        const dsa_vs_index* vs, const dsa_block_index* blk, const dsa_token_index* tok,
                        int32_t out_dtype, void* o, float* lse, AttnArgs& a) {
  dsa_status st = check_shape(shape);
  if (st) return st;
  if (!q || !k || !v || !o) return fail(DSA_ERR_INVALID_ARG, "q, k, v or o is null");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(DSA_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  if (!head_kind) return fail(DSA_ERR_INVALID_ARG, "head_kind is null");
  if (out_dtype != DSA_OUT_BF16 && out_dtype != DSA_OUT_F32) return fail(DSA_ERR_INVALID_ARG, "out_dtype");
  std::memset(&a, 0, sizeof a);
  bool use[4] = {};
  for (int h = 0; h < shape->heads; ++h) {
    if (head_kind[h] < 0 || head_kind[h] > 3) return fail(DSA_ERR_INVALID_ARG, "head_kind[%d] = %d", h, head_kind[h]);
    use[head_kind[h]] = true;
    a.kind[h] = (int8_t)head_kind[h];
  }
  if (use[DSA_PATTERN_VS]) {
    if (!vs || !vs->cols || !vs->cols_count || !vs->diags || !vs->diags_count || vs->cols_cap < 0 || vs->diags_cap < 0)
      return fail(DSA_ERR_INVALID_ARG, "VS heads need a VS index set");
  }
  if (use[DSA_PATTERN_BLOCK]) {
    if (!blk || !blk->idx || !blk->count || blk->cap < 1) return fail(DSA_ERR_INVALID_ARG, "block heads need a block index set");
    if (!block_size_ok(blk->block)) return fail(DSA_ERR_UNSUPPORTED, "block size %d", blk->block);
    if (shape->q_offset % blk->block != 0)
      return fail(DSA_ERR_UNSUPPORTED, "block heads need q_offset (%d) to be a multiple of the block (%d)",
                  shape->q_offset, blk->block);
  }
  if (use[DSA_PATTERN_TOKEN]) {
    if (!tok || !tok->idx || !tok->count || tok->cap < 1) return fail(DSA_ERR_INVALID_ARG, "token heads need a token index set");
    if (tok->cap > kMaxTokensPerQuery) return fail(DSA_ERR_UNSUPPORTED, "more than %d tokens per query", kMaxTokensPerQuery);
  }
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.o = o; a.lse = lse; a.out_f32 = out_dtype == DSA_OUT_F32;
  a.B = shape->batch; a.H = shape->heads; a.Hkv = shape->kv_heads;
  a.Nq = shape->q_len; a.Nk = shape->kv_len; a.q_offset = shape->q_offset;
  if (use[DSA_PATTERN_VS]) {
    a.cols = vs->cols; a.cols_count = vs->cols_count; a.cols_cap = vs->cols_cap;
    a.diags = vs->diags; a.diags_count = vs->diags_count; a.diags_cap = vs->diags_cap;
  }
  if (use[DSA_PATTERN_BLOCK]) {
    a.bidx = blk->idx; a.bcount = blk->count; a.bcap = blk->cap; a.block = blk->block;
    a.nqb = (shape->q_len + blk->block - 1) / blk->block;
    a.qb0 = shape->q_offset / blk->block;
  }
  if (use[DSA_PATTERN_TOKEN]) {
    a.tidx = tok->idx; a.tcount = tok->count; a.tcap = tok->cap;
  }
  return DSA_OK;
}

}  // namespace

extern "C" {

dsa_status sparse_prefill_attn(const dsa_shape* shape, const void* q, const void* k, const void* v,
                               const int32_t* head_kind, const dsa_vs_index* vs, const dsa_block_index* blk,
                               const dsa_token_index* tok, int32_t out_dtype, void* o, float* lse, void* ws,
                               size_t ws_bytes, void* stream) {
  g_err.clear();
  AttnArgs a;
  dsa_status st = prepare_attn(shape, q, k, v, head_kind, vs, blk, tok, out_dtype, o, lse, a);
  if (st) return st;
  const size_t need = ws_attn(shape);
  if (!ws || ws_bytes < need) return fail(DSA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  return hip_status(launch_attention(a, ws_base(ws), (hipStream_t)stream), "sparse_prefill_attn");
}

dsa_status sparse_prefill_attn_noalloc(const dsa_shape* shape, const void* q, const void* k, const void* v,
                                       const int32_t* head_kind, const dsa_vs_index* vs, const dsa_block_index* blk,
                                       const dsa_token_index* tok, int32_t out_dtype, void* o, float* lse,
                                       void* stream) {
  g_err.clear();
  AttnArgs a;
  dsa_status st = prepare_attn(shape, q, k, v, head_kind, vs, blk, tok, out_dtype, o, lse, a);
  if (st) return st;
  const size_t need = attn_workspace_bytes(shape->batch, shape->heads, shape->kv_len);
  if (need > kStaticScratchBytes)
    return fail(DSA_ERR_UNSUPPORTED,
                "sparse_prefill_attn_noalloc: this shape needs %zu bytes of scratch, the static buffer holds %zu "
                "(use sparse_prefill_attn with a workspace)",
                need, kStaticScratchBytes);
  void* ws = nullptr;
  if ((st = hip_status(static_scratch(&ws), "sparse_prefill_attn_noalloc: scratch address"))) return st;
  return hip_status(launch_attention(a, ws, (hipStream_t)stream), "sparse_prefill_attn_noalloc");
}

}  // extern "C"
