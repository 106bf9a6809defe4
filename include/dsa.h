/*
 * dsa.h -- C ABI of the MI355X (gfx950) dynamic sparse prefill attention library.
 *
 * The library builds per-head sparse indices and runs causal flash attention
 * over only the selected entries, the prefill method of MInference ("MInference
 * 1.0" explainer, sections on the three sparse patterns and on inference-time
 * dynamic masks; the authors' abstract: per-head pattern chosen offline,
 * indices built online, sparse kernels over pattern + indices), with the block
 * rule of MoBA ("Optimizing Mixture of Block Attention", FlashMoBA section:
 * top-k over mean key blocks) and FlashPrefill ("FlashPrefill", section 2.1
 * block means, section 2.2 max-relative threshold, section 2.3 index-driven
 * jumps), and the indexer token top-k of DSA/MISA ("MISA", sections on the
 * problem and on how MISA works).
 *
 * Conventions shared by every entry point
 *  - Every function returns a dsa_status.  No exception crosses the ABI and
 *    the library never aborts the process.
 *  - Tensor arguments are device pointers owned by the caller.  The library
 *    does not allocate device memory, free it, or keep a pointer after the
 *    call returns.  Scratch memory comes from a caller-provided workspace
 *    whose size dsa_workspace_size() reports.  The size includes 256 bytes
 *    of slack, so the workspace pointer needs no particular alignment.
 *  - Q, K, V, O and the indexer's q_idx and k_idx must be 16-byte aligned
 *    (they are read and written with 16-byte accesses); a misaligned pointer
 *    returns DSA_ERR_INVALID_ARG.
 *  - Arguments are checked on the host before any HIP call.  Kernels are then
 *    enqueued on `stream` (a hipStream_t; NULL means the default stream) and
 *    the call returns without synchronising.  Errors during execution show up
 *    at the caller's next synchronisation.  A failed launch returns
 *    DSA_ERR_HIP.
 *  - Layouts are dense row-major.  Q is [B, H, Nq, d], K and V are
 *    [B, Hkv, Nk, d], all bf16.  Q head h reads KV head h / (H / Hkv).
 *    d must be 128.  Query row i sits at absolute position i + q_offset, and
 *    Nq + q_offset == Nk (a prefill chunk that ends at the last key).
 *  - Index lists are int32 in ascending order.  Ties in every top-k go to the
 *    lower index.
 *  - The calls keep no state between them and may run concurrently on
 *    different streams with disjoint outputs and workspaces.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t dsa_status;
enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1,   /* a null pointer, a size out of range, a bad enum */
  DSA_ERR_UNSUPPORTED = 2,   /* a valid request this build does not implement (e.g. d != 128) */
  DSA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than dsa_workspace_size() */
  DSA_ERR_HIP = 4            /* a HIP call or kernel launch failed */
};

/* Pattern kind of a head (the offline per-head assignment).  A-shape heads are
 * passed as DSA_PATTERN_VS with the closed-form sets of build_index_ashape(). */
enum {
  DSA_PATTERN_DENSE = 0,     /* all causal keys */
  DSA_PATTERN_VS = 1,        /* vertical columns + slash diagonals */
  DSA_PATTERN_BLOCK = 2,     /* selected key blocks per query block */
  DSA_PATTERN_TOKEN = 3      /* per-query token list, shared by all heads */
};

enum { DSA_SELECT_TOPK = 0, DSA_SELECT_THRESHOLD = 1 };
enum { DSA_OUT_BF16 = 0, DSA_OUT_F32 = 1 };
enum { DSA_OP_VS = 1, DSA_OP_BLOCK = 2, DSA_OP_TOKENS = 3, DSA_OP_ATTN = 4, DSA_OP_TOKENS_HIER = 5,
       DSA_OP_VS_POOLED = 6 };

typedef struct dsa_shape {
  int32_t batch;       /* B  >= 1 */
  int32_t heads;       /* H  >= 1 */
  int32_t kv_heads;    /* Hkv >= 1, H % Hkv == 0 */
  int32_t q_len;       /* Nq >= 1 */
  int32_t kv_len;      /* Nk >= 1, Nk < 2^30 */
  int32_t head_dim;    /* d == 128 */
  int32_t q_offset;    /* >= 0, Nq + q_offset == Nk */
} dsa_shape;

/* Vertical-Slash index set of every head (device memory, caller-owned).
 * cols[b][h][0 .. cols_count[b][h]) are key columns j, diags[b][h][0 ..
 * diags_count[b][h]) are offsets o = i - j; both ascending and < Nk.  The
 * head's mask is M(i) = { j <= p_i : j in cols or p_i - j in diags }. */
typedef struct dsa_vs_index {
  int32_t* cols;         /* [B, H, cols_cap] */
  int32_t* cols_count;   /* [B, H] */
  int32_t  cols_cap;
  int32_t* diags;        /* [B, H, diags_cap] */
  int32_t* diags_count;  /* [B, H] */
  int32_t  diags_cap;
} dsa_vs_index;

/* Block index set (device memory, caller-owned).  Row I holds the chunk's
 * query block I, absolute block Ia = q_offset / block + I (positions
 * [Ia*block, (Ia+1)*block)): idx[b][h][I][0 .. count[b][h][I]) are its selected
 * key blocks J <= Ia, ascending.  M(i) = { j <= p_i : j / block in Sel(p_i /
 * block) }.  Requires q_offset to be a multiple of block; nqb = ceil(Nq / block). */
typedef struct dsa_block_index {
  int32_t* idx;          /* [B, H, nqb, cap] */
  int32_t* count;        /* [B, H, nqb] */
  int32_t  cap;
  int32_t  block;        /* 16, 32, 64 or 128 */
} dsa_block_index;

/* Token index set (device memory, caller-owned), one list per query shared by
 * all heads: idx[b][i][0 .. count[b][i]) are keys j <= p_i, ascending.  The
 * attention ignores entries outside [0, p_i] (negative, or after the query's
 * own position): M(i) is causal whatever the list holds. */
typedef struct dsa_token_index {
  int32_t* idx;          /* [B, Nq, cap] */
  int32_t* count;        /* [B, Nq] */
  int32_t  cap;
} dsa_token_index;

/* Message text of a status (static storage). */
const char* dsa_status_string(dsa_status s);

/* Text of the last error raised on the calling thread ("" if none). */
const char* dsa_last_error(void);

/* Workspace bytes one call needs.  `params` per op:
 *   DSA_OP_VS:     {n_heads, last_q}
 *   DSA_OP_BLOCK:  {n_heads, block}
 *   DSA_OP_TOKENS: {n_idx_heads, route_heads, topk}
 *   DSA_OP_TOKENS_HIER: {n_idx_heads, route_heads, cand, topk}
 *   DSA_OP_ATTN:   {} (none)
 *   DSA_OP_VS_POOLED: {n_heads, block}
 * Writes the size to *bytes.  Sizes depend on shapes only, never on data. */
dsa_status dsa_workspace_size(int32_t op, const dsa_shape* shape, const int32_t* params,
                              int32_t n_params, size_t* bytes);

/* A-shape heads as Vertical-Slash sets ("MInference 1.0" explainer, three
 * sparse patterns / A-shape: sink tokens plus a local window, a static mask).
 * For each head in heads[0..n_heads) (host array of head indices) writes
 * cols = [0, min(sink, Nk)) and diags = [0, min(local, Nk)), so that
 * M(i) = { j <= p_i : j < sink or p_i - j < local }.  `out` must have
 * cols_cap >= min(sink, Nk) and diags_cap >= min(local, Nk).
 * sink >= 0, local >= 1. */
dsa_status build_index_ashape(const dsa_shape* shape, const int32_t* heads, int32_t n_heads,
                              int32_t sink, int32_t local, dsa_vs_index out, void* stream);

/* Vertical-Slash index build ("MInference 1.0" explainer, inference-time
 * dynamic masks: the last last_q queries are scored against all keys and the
 * important columns and diagonals kept).  For each listed head:
 *   p[r, j] = softmax_j (q_{Nq-last_q+r} . k_j / sqrt(d)) over causal j,
 *   v[j] = sum_r p[r, j],  s[o] = sum_r p[r, p_r - o],
 *   cols = top-nv of v over [0, Nk), diags = top-ns of s over [0, Nk).
 * q, k: device bf16 Q and K.  1 <= last_q <= min(64, Nq); 0 <= nv <= cols_cap,
 * 0 <= ns <= diags_cap, nv, ns <= Nk.  v_scores / s_scores (nullable, device
 * float [B, n_heads, Nk]) receive v and s, row b * n_heads + t holding listed
 * head heads[t] of batch b (listed order, not head number).  Workspace:
 * dsa_workspace_size(DSA_OP_VS, {n_heads, last_q}). */
dsa_status build_index_vs(const dsa_shape* shape, const void* q, const void* k,
                          const int32_t* heads, int32_t n_heads, int32_t last_q,
                          int32_t nv, int32_t ns, dsa_vs_index out,
                          float* v_scores, float* s_scores,
                          void* ws, size_t ws_bytes, void* stream);

/* Block index build ("MInference 1.0" explainer: Block-Sparse heads pool Q and
 * K per block and keep important blocks; "FlashPrefill" section 2.1 mean keys,
 * section 2.2 threshold; MoBA's FlashMoBA top-k over key-block means).
 *   Qbar_I, Kbar_J = exact block means rounded to bf16 (round to nearest even);
 *   query block I of a prefill chunk is absolute block Ia = q_offset / block + I
 *   (its rows are the chunk's rows I * block ..; q_offset = 0 for a whole prompt);
 *   S[I, J] = Qbar_I . Kbar_J / sqrt(d) for J <= Ia;
 *   mode DSA_SELECT_TOPK: top-`topk` of J in [0, Ia] minus forced blocks;
 *   mode DSA_SELECT_THRESHOLD: J with S[I, J] >= max_J' S[I, J'] + log_alpha;
 *   then the union with block 0 (force_first) and block Ia (force_diag).
 * Lists hold absolute key blocks, one list per query block of the chunk (nqb =
 * ceil(q_len / block) of them).  block in {16, 32, 64, 128}; q_offset must be a
 * multiple of block (DSA_ERR_UNSUPPORTED otherwise); out.cap >= the largest count
 * (top-k: min(qb0 + nqb, topk + forced); threshold: qb0 + nqb, with qb0 =
 * q_offset / block).  Nullable outputs for inspection:
 * qbar ([B, H, nqb, d] bf16, indexed by head number, rows of listed heads
 * written), kbar ([B, Hkv, nkb, d] bf16, rows of the listed heads' KV heads
 * written) and scores ([B, n_heads, nqb, nkb] float in listed order, -inf for
 * J > Ia).  Workspace:
 * dsa_workspace_size(DSA_OP_BLOCK, {n_heads, block}). */
dsa_status build_index_block(const dsa_shape* shape, const void* q, const void* k,
                             const int32_t* heads, int32_t n_heads, int32_t block,
                             int32_t mode, int32_t topk, float log_alpha,
                             int32_t force_first, int32_t force_diag,
                             dsa_block_index out, void* qbar, void* kbar, float* scores,
                             void* ws, size_t ws_bytes, void* stream);

/* Vertical-Slash sets discovered from pooled block scores ("FlashPrefill"
 * section 2.1: one search over blocks, keys represented by their block means,
 * finds the vertical, slash and block shapes at once; the page states no rule
 * for the first two, this is the one the library defines).  For each listed head:
 *   Qbar, Kbar, S[I, J] = Qbar_I . Kbar_J / sqrt(d) (J <= Ia) as in
 *   build_index_block (query block I of the chunk is absolute block Ia =
 *   q_offset / block + I); P[I, :] = softmax over J <= Ia of S[I, J];
 *   vbar[J] = sum_I P[I, J] (vertical mass of key block J),
 *   sbar[D] = sum_I P[I, Ia - D] (slash mass of block offset D, D < nkb);
 *   kept key blocks = top-nv_blocks of vbar, kept offsets = top-ns_blocks of
 *   sbar (ties to the lower index);
 *   cols = every key of a kept key block, diags = every token offset
 *   [max(0, D*block - (block-1)), min(Nk-1, D*block + (block-1))] of a kept D.
 * The result goes to `out` like build_index_vs (attention takes it as a
 * Vertical-Slash set).  block in {16, 32, 64, 128}; q_offset a multiple of block;
 * 0 <= nv_blocks, ns_blocks <= 1024; cols_cap >= min(Nk, nv_blocks * block),
 * diags_cap >= min(Nk, ns_blocks * (2 * block - 1)); at most 32768 key blocks.
 * v_scores ([B, n_heads, nkb]) and s_scores ([B, n_heads, nkb]), nullable
 * device floats, receive vbar and sbar in listed order.  Workspace:
 * dsa_workspace_size(DSA_OP_VS_POOLED, {n_heads, block}). */
dsa_status build_index_vs_pooled(const dsa_shape* shape, const void* q, const void* k,
                                 const int32_t* heads, int32_t n_heads, int32_t block,
                                 int32_t nv_blocks, int32_t ns_blocks, dsa_vs_index out,
                                 float* v_scores, float* s_scores,
                                 void* ws, size_t ws_bytes, void* stream);

/* Indexer token top-k ("MISA": the DSA indexer scores every key with 64 light
 * heads and keeps the best tokens; MISA's router looks at keys in large blocks
 * and lets only a few heads per query score tokens).
 *   score[i, j] = sum_{h in H(i)} w[i, h] * max(0, q_idx[i, h] . k_idx[j]), j <= p_i
 *   route_heads == 0: H(i) = all heads.  route_heads = r > 0: H(i) = the r heads
 *   of largest w[i,h] * max(0, max_J q_idx[i,h] . Kbar_J), Kbar_J the bf16 mean of
 *   indexer keys [RJ, RJ + R) over complete blocks RJ + R - 1 <= p_i, R =
 *   route_block in {16, 32, 64, 128} (read only when route_heads > 0).
 *   tokens = top-`topk` of score[i, :] (count min(topk, p_i + 1)).
 * q_idx: device bf16 [B, Nq, n_idx_heads, 128]; k_idx: device bf16 [B, Nk, 128];
 * w: device float [B, Nq, n_idx_heads]; out: [B, Nq, cap].  The sequences of a
 * batch run one after another on `stream` and share the workspace.  route
 * (nullable, device int32 [B, Nq, route_heads]) receives H(i) ascending.
 * out.cap >= topk.  Workspace:
 * dsa_workspace_size(DSA_OP_TOKENS, {n_idx_heads, route_heads, topk}). */
dsa_status build_index_tokens(const dsa_shape* shape, const void* q_idx, const void* k_idx,
                              const float* w, int32_t n_idx_heads, int32_t route_heads,
                              int32_t route_block, int32_t topk, dsa_token_index out, int32_t* route,
                              void* ws, size_t ws_bytes, void* stream);

/* Hierarchical indexer token top-k ("MISA", section on how MISA works, the
 * hierarchical variant: the router's few heads find a larger candidate list,
 * then every indexer head checks only those candidates).
 *   stage 1: H(i) = the route_heads routed heads and score_r[i, j] the routed
 *     score, both as in build_index_tokens; C(i) = top-`cand` keys j <= p_i by
 *     score_r (ties to the lower index);
 *   stage 2: score[i, j] = sum over every head h of w[i, h] * max(0, q_idx[i, h]
 *     . k_idx[j]) for j in C(i); tokens = top-`topk` of C(i) by it (ties to the
 *     lower index), ascending, min(topk, |C(i)|) keys.
 * Arguments as build_index_tokens, plus: route_heads in [1, 8]; topk <= 4096;
 * cand in [topk, 65536]; cands (nullable, device [B, Nq, cap], cap >= cand) receives C(i)
 * ascending, otherwise C(i) lives in the workspace.  Workspace:
 * dsa_workspace_size(DSA_OP_TOKENS_HIER, {n_idx_heads, route_heads, cand, topk}). */
dsa_status build_index_tokens_hier(const dsa_shape* shape, const void* q_idx, const void* k_idx,
                                   const float* w, int32_t n_idx_heads, int32_t route_heads,
                                   int32_t route_block, int32_t cand, int32_t topk, dsa_token_index out,
                                   const dsa_token_index* cands, int32_t* route,
                                   void* ws, size_t ws_bytes, void* stream);

/* Sparse prefill attention over each head's index set ("MInference 1.0"
 * explainer, GPU kernels: attention only at the indexed positions;
 * "FlashPrefill" section 2.3: the kernel walks compact index lists instead of
 * skipping masked tiles):
 *   O[b,h,i] = sum_{j in M_h(i)} softmax_j(q_i . k_j / sqrt(d)) v_j,
 *   LSE[b,h,i] = log sum_{j in M_h(i)} exp(q_i . k_j / sqrt(d)).
 * head_kind: HOST int32 [H] of DSA_PATTERN_*; the index struct of every kind
 * used must be non-null (vs / blk / tok).  Rows with an empty M(i) get O = 0
 * and LSE = -inf.  out_dtype DSA_OUT_BF16 or DSA_OUT_F32 selects O's type
 * ([B, H, Nq, d]); lse (nullable) is float [B, H, Nq].  Block sets of 16 or 32
 * ("Optimizing Mixture of Block Attention" explainer: small blocks) are walked
 * 32 keys at a time per 32 query rows.  Workspace:
 * dsa_workspace_size(DSA_OP_ATTN, {}). */
dsa_status sparse_prefill_attn(const dsa_shape* shape, const void* q, const void* k,
                               const void* v, const int32_t* head_kind,
                               const dsa_vs_index* vs, const dsa_block_index* blk,
                               const dsa_token_index* tok, int32_t out_dtype,
                               void* o, float* lse, void* ws, size_t ws_bytes, void* stream);

/* sparse_prefill_attn for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, arguments and results, with no workspace
 * argument.  Its scratch is a static device array of 32 MiB that the library
 * holds on every device it runs on until the process ends; shapes whose
 * scratch (about B * H * Nk / 2 bytes) exceeds it return DSA_ERR_UNSUPPORTED
 * and must use sparse_prefill_attn.  The call itself allocates nothing.  All
 * calls on one device share that array and the call clears what it needs
 * first: calls that overlap in time on one device (different streams, or
 * different threads) race and give undefined results. */
dsa_status sparse_prefill_attn_noalloc(const dsa_shape* shape, const void* q, const void* k,
                                       const void* v, const int32_t* head_kind,
                                       const dsa_vs_index* vs, const dsa_block_index* blk,
                                       const dsa_token_index* tok, int32_t out_dtype,
                                       void* o, float* lse, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H_ */
