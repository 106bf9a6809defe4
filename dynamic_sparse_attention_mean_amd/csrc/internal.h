// Internal launch interfaces between the C-ABI layer (api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

constexpr int kMaxHeadTable = 512;   // B*H entries a single attention launch can schedule
constexpr int kMaxQueues = 8;        // one work queue per XCD

struct HeadList {                    // small head lists travel as kernel arguments
  int32_t n;
  int32_t h[256];
};
struct TokenGroups {                 // token heads h0 .. h0 + cnt - 1 of one KV head, cnt <= 16
  int32_t n;
  int32_t h0[128];
  int32_t cnt[128];
};

// ----------------------------------------------------------------- pooling
// dst[b][head][I][:] = bf16(mean of src[b][head][I*block .. ][:]) for the listed
// heads (head indices into src's head axis).  src is [B, Hs, N, 128] bf16.
hipError_t launch_pool(const uint16_t* src, int B, int Hs, int N, const HeadList& heads,
                       int block, uint16_t* dst, hipStream_t st);

// ------------------------------------------------------------ block scores
// scores[b][h][I][J] = qbar[b][h][I] . kbar[b][kvh][J] * scale for J <= qb0 + I
// (fp32; query block I of a chunk is absolute block qb0 + I).
hipError_t launch_block_scores(const uint16_t* qbar, const uint16_t* kbar, int B, int H, int Hkv,
                               int nqb, int nkb, int qb0, const HeadList& heads, float scale, float* scores,
                               hipStream_t st);

// --------------------------------------------- fused block scores + select
// Scores of a strip of query blocks held on chip (LDS), then the selection of
// every row of the strip; `scores` (nullable, [B, n_heads, nqb, nkb]) receives
// an inspection copy.  block_strip_rows() gives the rows per strip for nkb key
// blocks (0: a row does not fit on chip; the two-kernel path below then runs).
constexpr int kBlockStripFloats = 32768;   // 128 KB of fp32 scores per workgroup
int block_strip_rows(int nkb, int* stride);
hipError_t launch_block_index(const uint16_t* qbar, const uint16_t* kbar, int B, int H, int Hkv, int nqb, int nkb,
                              int qb0, const HeadList& heads, float scale, int mode, int topk, float log_alpha,
                              int force_first, int force_diag, int32_t* idx, int32_t* count, int cap,
                              float* scores, hipStream_t st);

// Vertical and slash discovery from the pooled block scores: per listed head,
// the per-strip partials (vpart [B, n_heads, nstrips, nkb], spart [.., nkb];
// pooled_vs_partial_floats() per row of B * n_heads), the masses vbar
// [B, n_heads, nkb] and sbar [B, n_heads, nkb] (one per key block offset), the
// top nvb key blocks and nsb block offsets, expanded into the Vertical-Slash
// set ([B, H, cap] rows).  Query block I of a chunk is absolute block qb0 + I.
constexpr int kMaxPooledBlocks = 1024;     // kept key blocks / block offsets per head
size_t pooled_vs_partial_floats(int nqb, int nkb);
hipError_t launch_pooled_vs(const uint16_t* qbar, const uint16_t* kbar, int B, int H, int Hkv, int nqb, int nkb,
                            int qb0, int Nk, int block, const HeadList& heads, float scale, float* vpart, float* spart,
                            float* vbar, float* sbar, int nvb, int nsb, int32_t* cols, int32_t* cols_count,
                            int cols_cap, int32_t* diags, int32_t* diags_count, int diags_cap, hipStream_t st);

// ---------------------------------------------------------------- select
// Per listed head and query block I: block selection over scores row I
// (rows too long to keep on chip: the scores go through the workspace).
hipError_t launch_block_select(const float* scores, int B, int H, int nqb, int nkb, int qb0,
                               const HeadList& heads, int mode, int topk, float log_alpha,
                               int force_first, int force_diag, int32_t* idx, int32_t* count,
                               int cap, hipStream_t st);


// ------------------------------------------------------------ vertical-slash
struct VsScoreArgs {
  const uint16_t* q;      // [B, H, Nq, 128]
  const uint16_t* k;      // [B, Hkv, Nk, 128]
  int B, H, Hkv, Nq, Nk, last_q;
  HeadList heads;
  float* v_out;           // [B, n_heads, Nk] column sums
  float* s_out;           // [B, n_heads, Nk] diagonal sums
  float* part_ml;         // [B, n_heads, nchunks, 2, 64] per-chunk row max / sum
  float* part_diag;       // [B, n_heads, nchunks, chunk_keys + 64] per-chunk diagonal sums
  float* row_stats;       // [B, n_heads, 2, 64] each row's maximum and 1 / sum (after part_ml)
  int nchunks, chunk_keys; // set by launch_vs_scores
};
// Listed heads grouped by KV head for the scoring passes: group s holds the
// listed indices order[first[s] .. first[s] + cnt[s]) (at most 4, one KV head).
struct VsGroupTable {
  int32_t n;
  int16_t first[256];
  int16_t order[256];
  int8_t cnt[256];
};
size_t vs_workspace_floats(int n_rows, int Nk);   // n_rows = B * n_heads
void vs_part_floats(int n_rows, int Nk, size_t* ml, size_t* diag);   // the per-chunk partials within it
hipError_t launch_vs_scores(const VsScoreArgs& a, hipStream_t st);

// Top-nv of v and top-ns of s per listed head ([B, n_heads, Nk] rows) into the
// VS index set ([B, H, cap] rows).
hipError_t launch_vs_select(const float* v, const float* s, int B, int Nk, int H, const HeadList& heads, int nv,
                            int ns, int32_t* cols, int32_t* cols_count, int cols_cap, int32_t* diags,
                            int32_t* diags_count, int diags_cap, hipStream_t st);

// A-shape sets: cols = [0, sink), diags = [0, local) for each listed head.
hipError_t launch_ashape_fill(int B, int H, const HeadList& heads, int ncols, int ndiags,
                              int32_t* cols, int32_t* cols_count, int cols_cap,
                              int32_t* diags, int32_t* diags_count, int diags_cap, hipStream_t st);

// --------------------------------------------------------------- attention
struct AttnArgs {
  const uint16_t* q; const uint16_t* k; const uint16_t* v;
  void* o; float* lse; int out_f32;
  int B, H, Hkv, Nq, Nk, q_offset;
  int8_t kind[256];                  // per Q head
  // Vertical-Slash sets and their compiled form (workspace)
  const int32_t* cols; const int32_t* cols_count; int cols_cap;
  const int32_t* diags; const int32_t* diags_count; int diags_cap;
  uint32_t* sbits; uint32_t* vbits;  // diagonal bitmap (two leading pad words), column bitmap
  uint32_t* cbits;                   // bit c set iff c is a step centre (offsets of the sub-block steps)
  int32_t* clist;                    // the centres ascending: {c, diagonal bits of [c - 32, c + 31] (2 words), 0}
  int32_t* ccount; int32_t* cle;     // their number; #{centres <= 32 x + 31} for x in [0, ccap)
  int sw, vw, cw, ccap;              // words per head of each bitmap; clist capacity (entries)
  int32_t* win;                      // [B*H][2]: window length and sink of a head whose sets are
                                     // cols = [0, sink), diags = [0, window) (else window = -1)
  // Block sets
  const int32_t* bidx; const int32_t* bcount; int bcap, block, nqb;
  int qb0;                           // lists are per query block of the chunk; its first is absolute block qb0
  // Token sets
  const int32_t* tidx; const int32_t* tcount; int tcap;
  // Scheduling
  int32_t* counters;                 // [kMaxQueues] work-queue heads (zeroed by the launcher)
};
size_t attn_workspace_bytes(int B, int H, int Nk);
hipError_t launch_attention(AttnArgs& a, void* ws, hipStream_t st);
// The attention scratch of the entry point that allocates nothing: a static
// device array of kStaticScratchBytes; *ptr receives its address on the
// current device (looked up once per device).
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
hipError_t static_scratch(void** ptr);

// --------------------------------------------------------------- indexer
struct IndexerArgs {
  const uint16_t* q_idx;   // [Nq, Hi, 128]
  const uint16_t* k_idx;   // [Nk, 128]
  const float* w;          // [Nq, Hi]
  int Nq, Nk, Hi, q_offset, route_heads, topk;
  int route_block;         // keys per router block (16, 32, 64 or 128)
  int32_t* tok; int32_t* tok_count; int tok_cap;
  int32_t* route;          // nullable [Nq, route_heads]
  // hierarchical option (cand > 0): candidates per query, their list (nullable:
  // workspace) with capacity cand_cap and counts
  int cand;
  int32_t* cand_idx; int32_t* cand_count; int cand_cap;
};
size_t indexer_workspace_bytes(int Nq, int Nk, int Hi, int route_heads, int cand);
hipError_t launch_indexer(const IndexerArgs& a, void* ws, hipStream_t st);
constexpr int kMaxTokensPerQuery = 4096;
constexpr int kMaxCandidates = 65536;   // candidates per query of the hierarchical indexer
// Attention of the TOKEN heads over per-query token lists.
hipError_t launch_token_attention(const AttnArgs& a, hipStream_t st);

// zero n int32 words (used instead of hipMemsetAsync so the sequence stays
// capturable into a graph)
hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t st);

}  // namespace dsa
