// Vertical-Slash index build and A-shape sets.
//
// "MInference 1.0" explainer (inference-time dynamic masks): for a Vertical-Slash
// head the last last_q queries are scored against every key ("rough attention")
// and the important vertical columns and slash diagonals are kept; A-shape heads
// use a static sink + local-window mask (three sparse patterns / A-shape).
//
//   p[r, j] = softmax_j(q_r . k_j / sqrt(d)) over j <= p_r = Nk - L + r
//   v[j] = sum_r p[r, j]        s[o] = sum_r p[r, p_r - o]
//
// Two passes over K on v_mfma_f32_32x32x16_bf16, one workgroup per group of
// listed heads that share a KV head (and per chunk of keys): pass 1 finds each
// row's max and sum of exponentials; pass 2 forms the normalised p and reduces
// it along columns and diagonals.  Every reduction runs in a fixed order, so v
// and s are bitwise reproducible.
#include "common.h"
#include "internal.h"
#include "select.h"

#include <algorithm>
#include <atomic>

namespace dsa {
namespace {

// A chunk of keys (one workgroup per group of heads and chunk) holds a multiple
// of 32 keys, at most kVsChunkMax; the host picks the size that spreads the
// workgroups most evenly over the chip.  Pass 2 keeps a chunk's column sums and
// diagonal partials (chunk + 63 of them) in LDS.
constexpr int kVsChunkMin = 256;
constexpr int kVsChunkMax = 512;

struct Frag {
  bf16x8 q[8];
};

__device__ __forceinline__ void load_qfrag(const VsScoreArgs& a, int b, int h, int r, Frag& f) {
  const int hh = (threadIdx.x & 63) >> 5;
  const uint16_t* qp = a.q + ((size_t)(b * a.H + h) * a.Nq + (a.Nq - a.last_q + r)) * 128;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (r < a.last_q) x = *(const u32x4*)(qp + 16 * ks + 8 * hh);
    f.q[ks] = __builtin_bit_cast(bf16x8, x);
  }
}

constexpr float kScale2 = 1.4426950408889634f * 0.08838834764831845f;   // log2(e) / sqrt(128)

// ---------------------------------------------------------------------------
// The two passes per KV group: a workgroup takes up to GH listed heads that
// read the same KV head (two waves per head: query rows 0-31 and 32-63), so
// each 32-key block of K is brought into LDS once (DMA) for all of them.
// Per block a wave forms the scores of its 32 rows on v_mfma_f32_32x32x16_bf16
// with the K fragments read from LDS: pass 1 as S^T (a lane holds one row, so
// row maxima and sums stay in the lane), pass 2 as S (a lane holds one key
// column, so column sums stay in registers and diagonal sums take a lane
// rotation, as described at the kernel).
constexpr int GH = 4;                // heads per workgroup
constexpr int GT = 2 * GH * 64;      // threads: wave w serves head slot w / 2, rows 32 (w % 2) ..
constexpr int KB = 32;               // keys per block

typedef __attribute__((address_space(3))) char lds_char_vs_t;
__device__ __forceinline__ void vs_wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ int vs_swz(int r, int c) { return c ^ (r & 15); }
// DMA of K block kb (32 keys, 8 KB) into an LDS stage: lane l of wave w takes
// row 4 w + l / 16 and writes LDS chunk l % 16 of that row, which holds the
// row's 16-byte chunk (l % 16) ^ (row % 16); keys past the end are clamped.
__device__ __forceinline__ void vs_issue_block(const uint16_t* kp, int Nk, int kb, char* stage) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int r = 4 * w + (l >> 4);
  const int key = min(kb * KB + r, Nk - 1);
  const int c = vs_swz(r, l & 15);
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_char_vs_t*)stage + w * 1024);
  dma16(kp + (size_t)key * 128 + c * 8, lds);
}
// The compiler's wait for the Q fragment loads, placed here (after the first
// DMAs are issued) rather than at their first use inside a block loop, where
// it would drain the DMAs of later blocks in every iteration.
__device__ __forceinline__ void vs_take_q(const Frag& f) {
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) asm volatile("" :: "v"(f.q[ks]));
}

// S^T of one 32-key block against this wave's 32 query rows, K from LDS.
__device__ __forceinline__ f32x16 vs_block_scores(const char* stage, const Frag& f) {
  const int l = threadIdx.x & 63, qn = l & 31, hh = l >> 5;
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
  u32x4 kf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) kf[ks] = *(const u32x4*)(stage + qn * 256 + vs_swz(qn, 2 * ks + hh) * 16);
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[ks]), f.q[ks], acc, 0, 0, 0);
  return acc;
}

// S of one 32-key block for this wave's 32 query rows (queries as the A
// operand): lane l gets key l % 32 for rows 8 (v / 4) + 4 (l / 32) + v % 4.
__device__ __forceinline__ f32x16 vs_block_rows(const char* stage, const Frag& f) {
  const int l = threadIdx.x & 63, qn = l & 31, hh = l >> 5;
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
  u32x4 kf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) kf[ks] = *(const u32x4*)(stage + qn * 256 + vs_swz(qn, 2 * ks + hh) * 16);
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.q[ks], __builtin_bit_cast(bf16x8, kf[ks]), acc, 0, 0, 0);
  return acc;
}

struct VsGroupInfo {
  int ng, hi, h, kvh;                // heads in the group, this wave's listed index and head, KV head
  bool on;                           // this wave's head slot is used
};
__device__ __forceinline__ VsGroupInfo vs_group_info(const VsScoreArgs& a, const VsGroupTable& t) {
  VsGroupInfo gi;
  const int sg = blockIdx.x;
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 7);
  gi.ng = t.cnt[sg];
  gi.on = g < gi.ng;
  gi.hi = t.order[t.first[sg] + (gi.on ? g : 0)];
  gi.h = a.heads.h[gi.hi];
  gi.kvh = a.heads.h[t.order[t.first[sg]]] / (a.H / a.Hkv);
  return gi;
}

// Wait until at most n of this wave's DMAs are outstanding (n = 0 .. 4).
__device__ __forceinline__ void vs_wait_vm_upto(int n) {
  if (n >= 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else if (n == 3) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
  else if (n == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
  else if (n == 1) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

constexpr int P1ST = 6;              // pass 1 ring stages: blocks prefetched five ahead
constexpr int P2ST = 4;              // pass 2 ring stages: blocks prefetched three ahead

__global__ __launch_bounds__(GT) void vs_group_pass1_kernel(VsScoreArgs a, VsGroupTable t) {
  __shared__ __align__(1024) char s_k[P1ST][KB * 256];
  const int c = blockIdx.y, b = blockIdx.z;
  const VsGroupInfo gi = vs_group_info(a, t);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, hh = l >> 5, qn = l & 31;
  const int r = 32 * (w & 1) + qn;
  const int pr = a.Nk - a.last_q + r;
  Frag f;
  load_qfrag(a, b, gi.h, gi.on ? r : 64, f);           // rows >= last_q load zeros
  const uint16_t* kp = a.k + ((size_t)(b * a.Hkv + gi.kvh) * a.Nk) * 128;
  const int nblk = (a.Nk + KB - 1) / KB;
  const int cb = a.chunk_keys / KB;
  const int kb0 = c * cb, kb1 = min(nblk, kb0 + cb);
  float m = -INFINITY, s = 0.f;
  // the loop stores nothing, so DMAs are this wave's only vector memory
  // operations and complete in issue order: a partial count is safe
  for (int i = 0; i < P1ST - 1 && kb0 + i < kb1; ++i) vs_issue_block(kp, a.Nk, kb0 + i, s_k[i]);
  vs_take_q(f);
  for (int kb = kb0; kb < kb1; ++kb) {
    const int st = (kb - kb0) % P1ST;
    vs_wait_vm_upto(min(P1ST - 2, kb1 - 1 - kb));     // block kb landed (later ones may be in flight)
    __syncthreads();                                 // ... for every wave; all are done with kb - 1
    if (kb + P1ST - 1 < kb1) vs_issue_block(kp, a.Nk, kb + P1ST - 1, s_k[(st + P1ST - 1) % P1ST]);
    if (gi.on) {
      const f32x16 acc = vs_block_scores(s_k[st], f);
      float z[16];
      float mt = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = kb * KB + 8 * (v >> 2) + 4 * hh + (v & 3);
        const bool ok = key < a.Nk && key <= pr && r < a.last_q;
        z[v] = ok ? acc[v] * kScale2 : -INFINITY;
        mt = fmaxf(mt, z[v]);
      }
      if (mt > -INFINITY) {
        const float mn = fmaxf(m, mt);
        float add = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) add += __builtin_amdgcn_exp2f(z[v] - mn);
        s = s * __builtin_amdgcn_exp2f(m - mn) + add;
        m = mn;
      }
    }
  }
  // the row's two lanes (hh = 0, 1), combined in the same order on both
  const float m2 = __shfl_xor(m, 32, 64), s2 = __shfl_xor(s, 32, 64);
  const float mm = fmaxf(m, m2);
  const float ss = (mm == -INFINITY) ? 0.f
                   : (hh == 0 ? s * __builtin_amdgcn_exp2f(m - mm) + s2 * __builtin_amdgcn_exp2f(m2 - mm)
                              : s2 * __builtin_amdgcn_exp2f(m2 - mm) + s * __builtin_amdgcn_exp2f(m - mm));
  if (gi.on && hh == 0) {
    float* pm = a.part_ml + (((size_t)(b * a.heads.n + gi.hi) * a.nchunks + c) * 2) * 64;
    pm[r] = mm;
    pm[64 + r] = ss;
  }
}

// Each row's maximum and sum over all chunks of pass 1: sixteen threads per row
// merge contiguous runs of chunks (ascending), then one merges the sixteen
// results in order.  Writes the maximum and 1 / sum.
__global__ __launch_bounds__(1024) void vs_row_stats_kernel(VsScoreArgs a) {
  __shared__ float s_m[16][64], s_s[16][64];
  const int hi = blockIdx.x, b = blockIdx.y;
  const size_t row = (size_t)(b * a.heads.n + hi);
  const int r = threadIdx.x & 63, p = threadIdx.x >> 6;
  const int per = (a.nchunks + 15) / 16;
  const int c0 = min(a.nchunks, p * per), c1 = min(a.nchunks, c0 + per);
  const float* pm = a.part_ml + (row * a.nchunks) * 128;
  float m = -INFINITY, s = 0.f;
  for (int cb = c0; cb < c1; cb += 8) {
    float mc[8], sc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {               // eight chunks' loads in flight
      const bool ok = cb + j < c1;
      mc[j] = ok ? pm[(size_t)(cb + j) * 128 + r] : -INFINITY;
      sc[j] = ok ? pm[(size_t)(cb + j) * 128 + 64 + r] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float mn = fmaxf(m, mc[j]);
      if (mn != -INFINITY) s = s * __builtin_amdgcn_exp2f(m - mn) + sc[j] * __builtin_amdgcn_exp2f(mc[j] - mn);
      m = mn;
    }
  }
  s_m[p][r] = m;
  s_s[p][r] = s;
  __syncthreads();
  if (p == 0) {
    m = -INFINITY;
    s = 0.f;
    for (int q = 0; q < 16; ++q) {
      const float mq = s_m[q][r], sq = s_s[q][r];
      const float mn = fmaxf(m, mq);
      if (mn != -INFINITY) s = s * __builtin_amdgcn_exp2f(m - mn) + sq * __builtin_amdgcn_exp2f(mq - mn);
      m = mn;
    }
    a.row_stats[row * 128 + r] = m;
    a.row_stats[row * 128 + 64 + r] = s > 0.f ? 1.0f / s : 0.f;
  }
}

// Pass 2.  Per block a wave forms S (its 32 query rows by the block's 32 keys)
// with the query fragments as the A operand, so lane l holds key l % 32 of the
// block for sixteen rows.  Column sums are the lane's own sixteen weights plus
// those of lane l ^ 32 (the other sixteen rows).  Diagonal sums: for each of
// the sixteen rows rl, lane t takes the weight of key (rl - t) mod 32 from its
// half of the wave (ds_bpermute), which lies on diagonal rl - key = t when
// t <= rl and t - 32 otherwise; the two accumulators of lane t are offsets
// base + t and base + t - 32 of the block, and the second is the first one of
// the next block, so it is carried and added there.  Sums run in a fixed order
// (rows ascending within a half, then the halves, then block before carry,
// then rows 0-31 before 32-63).  The loop issues no global stores (a store
// shares the DMA's counter and would make the partial waits unsafe): each
// wave's column sums and diagonal partials collect in its own LDS rows and
// are written out once at the end.
__global__ __launch_bounds__(GT) __attribute__((amdgpu_waves_per_eu(4))) void vs_group_pass2_kernel(VsScoreArgs a, VsGroupTable t) {
  __shared__ __align__(1024) char s_k[P2ST][KB * 256];
  __shared__ float s_dw[2 * GH][kVsChunkMax + 64];
  __shared__ float s_cw[2 * GH][kVsChunkMax];
  __shared__ float s_mr[GH][64], s_il[GH][64];
  const int CK = a.chunk_keys, c = blockIdx.y, b = blockIdx.z;
  const VsGroupInfo gi = vs_group_info(a, t);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, hh = l >> 5, qn = l & 31;
  const int g = w >> 1;
  const int r = 32 * (w & 1) + qn;           // the query row this lane loads
  const size_t row = (size_t)(b * a.heads.n + gi.hi);

  // each row's final maximum and 1 / sum (vs_row_stats_kernel)
  if ((w & 1) == 0 && gi.on) {
    s_mr[g][l] = a.row_stats[row * 128 + l];
    s_il[g][l] = a.row_stats[row * 128 + 64 + l];
  }
  for (int i = tid; i < 2 * GH * (kVsChunkMax + 64); i += GT) (&s_dw[0][0])[i] = 0.f;
  Frag f;
  load_qfrag(a, b, gi.h, gi.on ? r : 64, f);
  const uint16_t* kp = a.k + ((size_t)(b * a.Hkv + gi.kvh) * a.Nk) * 128;
  const int nblk = (a.Nk + KB - 1) / KB;
  const int kb0 = c * (CK / KB), kb1 = min(nblk, kb0 + CK / KB);
  __syncthreads();                                        // row statistics visible; s_dw cleared
  // rows of this lane's sixteen weights: rl(v) = 8 (v / 4) + 4 hh + v % 4, so
  // the statistics of rows v = 4 j .. 4 j + 3 are four adjacent floats
  const float* smr = &s_mr[g][32 * (w & 1) + 4 * hh];
  const float* sil = &s_il[g][32 * (w & 1) + 4 * hh];
  const int p0 = a.Nk - a.last_q + 32 * (w & 1);          // position of the wave's row 0
  const int rows_on = a.last_q - 32 * (w & 1);            // rows rl < rows_on exist
  float* dw = s_dw[w];
  float* cw = s_cw[w];
  // slot of offset base(kb) + qn, base(kb) = p0 - 32 kb, with slot 0 at offset
  // Nk - last_q - (c + 1) CK + 1
  const int slot0 = 32 * (w & 1) + CK - 1 + qn;
  float carry = 0.f;
  // from here on the DMAs are the only vector memory operations in flight
  for (int i = 0; i < P2ST - 1 && kb0 + i < kb1; ++i) vs_issue_block(kp, a.Nk, kb0 + i, s_k[i]);
  vs_take_q(f);
  for (int kb = kb0; kb < kb1; ++kb) {
    const int st = (kb - kb0) % P2ST;
    vs_wait_vm_upto(min(P2ST - 2, kb1 - 1 - kb));         // block kb landed (later ones may be in flight)
    __syncthreads();                                     // ... for every wave; all are done with kb - 1
    if (kb + P2ST - 1 < kb1) vs_issue_block(kp, a.Nk, kb + P2ST - 1, s_k[(st + P2ST - 1) % P2ST]);
    if (gi.on) {
      const f32x16 acc = vs_block_rows(s_k[st], f);
      const int key = kb * KB + qn;
      float p[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // read here rather than kept in registers: a wave's statistics would
        // take 32 registers for the whole loop
        const f32x4 mr = *(const f32x4*)(smr + 8 * j), il = *(const f32x4*)(sil + 8 * j);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v = 4 * j + e, rl = 8 * j + 4 * hh + e;
          const bool ok = key < a.Nk && key <= p0 + rl && rl < rows_on;
          p[v] = ok ? __builtin_amdgcn_exp2f(acc[v] * kScale2 - mr[e]) * il[e] : 0.f;
        }
      }
      float cs = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) cs += p[v];
      float da = 0.f, db = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rl = 8 * (v >> 2) + 4 * hh + (v & 3);
        const int src = (((rl - qn) & 31) + 32 * hh) << 2;
        const float x = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, p[v])));
        const bool lo = qn <= rl;
        da += lo ? x : 0.f;
        db += lo ? 0.f : x;
      }
      const float cs2 = __shfl_xor(cs, 32, 64);
      const float da2 = __shfl_xor(da, 32, 64);
      const float db2 = __shfl_xor(db, 32, 64);
      if (hh == 0) {
        const int i = kb - kb0;
        cw[i * KB + qn] = cs + cs2;
        dw[slot0 - KB * i] = (da + da2) + carry;
        carry = db + db2;
      }
    }
  }
  // the last block's carried offsets (lane 0's is always zero: no key lies
  // 32 positions after its row within a block)
  if (gi.on && hh == 0 && qn > 0) dw[slot0 - KB * (kb1 - kb0)] = carry;
  __syncthreads();
  if (gi.on) {
    const int tl = tid & 127;
    float* vo = a.v_out + row * a.Nk;
    const int n = min(a.Nk, kb1 * KB) - kb0 * KB;
    for (int i = tl; i < n; i += 128) vo[kb0 * KB + i] = s_cw[2 * g][i] + s_cw[2 * g + 1][i];
    float* pd = a.part_diag + (row * a.nchunks + c) * (size_t)(CK + 64);
    for (int i = tl; i < CK + 64; i += 128) pd[i] = s_dw[2 * g][i] + s_dw[2 * g + 1][i];
  }
}

__global__ __launch_bounds__(256) void vs_diag_combine_kernel(VsScoreArgs a) {
  const int hi = blockIdx.y, b = blockIdx.z;
  const size_t row = (size_t)(b * a.heads.n + hi);
  const int CK = a.chunk_keys, span = CK + 64;
  const float* pd = a.part_diag + row * a.nchunks * span;
  float* so = a.s_out + row * a.Nk;
  for (int o = blockIdx.x * 256 + threadIdx.x; o < a.Nk; o += gridDim.x * 256) {
    // chunk c holds offsets [Nk - last_q - (c + 1) CK + 1, Nk - last_q - c CK + 63]:
    // at most two chunks, summed in ascending order
    int chi = (a.Nk - a.last_q + 63 - o) / CK;
    chi = min(chi, a.nchunks - 1);
    float s = 0.f;
    for (int cc = max(0, chi - 1); cc <= chi; ++cc) {
      const int o_min = a.Nk - a.last_q - (cc + 1) * CK + 1;
      const int idx = o - o_min;
      if (idx >= 0 && idx < CK + 63) s += pd[(size_t)cc * span + idx];
    }
    so[o] = s;
  }
}

// Top-nv of v and top-ns of s for each listed head (blockIdx.x: 0 = v, 1 = s).
__global__ __launch_bounds__(1024) void vs_select_kernel(const float* v, const float* s, int Nk, int H,
                                                         HeadList heads, int nv, int ns, int32_t* cols,
                                                         int32_t* cols_count, int cols_cap, int32_t* diags,
                                                         int32_t* diags_count, int diags_cap) {
  __shared__ Select3Smem<1024> sm;
  const int which = blockIdx.x, hi = blockIdx.y, b = blockIdx.z;
  const int h = heads.h[hi];
  const size_t row = (size_t)(b * heads.n + hi);
  const size_t bh = (size_t)b * H + h;
  const float* sc = (which == 0 ? v : s) + row * Nk;
  int32_t* out = which == 0 ? cols + bh * cols_cap : diags + bh * diags_cap;
  const int n = select_topk_3pass<1024>(sc, Nk, which == 0 ? nv : ns, out, sm);
  if (threadIdx.x == 0) (which == 0 ? cols_count : diags_count)[bh] = n;
}

__global__ void ashape_fill_kernel(int H, HeadList heads, int ncols, int ndiags, int32_t* cols,
                                   int32_t* cols_count, int cols_cap, int32_t* diags, int32_t* diags_count,
                                   int diags_cap) {
  const int hi = blockIdx.x, b = blockIdx.y;
  const size_t bh = (size_t)b * H + heads.h[hi];
  for (int i = threadIdx.x; i < ncols; i += blockDim.x) cols[bh * cols_cap + i] = i;
  for (int i = threadIdx.x; i < ndiags; i += blockDim.x) diags[bh * diags_cap + i] = i;
  if (threadIdx.x == 0) {
    cols_count[bh] = ncols;
    diags_count[bh] = ndiags;
  }
}

}  // namespace

// Per-chunk partials for n_rows listed heads, enough for any chunk size the
// launch may pick (the smallest gives the most chunks).
void vs_part_floats(int n_rows, int Nk, size_t* ml, size_t* diag) {
  size_t nch = 0, span = 0;
  for (int ck = kVsChunkMin; ck <= kVsChunkMax; ck += KB) {
    const size_t n = (size_t)(Nk + ck - 1) / ck;
    nch = std::max(nch, n);
    span = std::max(span, n * (size_t)(ck + 64));
  }
  *ml = (size_t)n_rows * (nch + 1) * 128;      // + each row's final statistics
  *diag = (size_t)n_rows * span;
}

size_t vs_workspace_floats(int n_rows, int Nk) {
  size_t ml, dg;
  vs_part_floats(n_rows, Nk, &ml, &dg);
  return (size_t)n_rows * 2 * (size_t)Nk + ml + dg;
}

// Workgroups of pass 2 that run at once on the current device.
// Per device, queried once (a racing second query stores the same value).
static int vs_slots() {
  static std::atomic<int> cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 512;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, vs_group_pass2_kernel, GT, 0) != hipSuccess || per <= 0)
      per = 1;
    n = cus * per;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// The chunk size (a multiple of 32 keys in [kVsChunkMin, kVsChunkMax]) that
// minimises rounds of workgroups x (keys per workgroup + a fixed start-up cost
// of about four blocks: the Q loads and the ring's first fill), the pass time
// when every workgroup streams its chunk at the same rate.  Ties go to the
// larger chunk.
static int vs_chunk_keys(int units_per_chunk_row, int Nk, int slots) {
  int best = kVsChunkMax;
  long long best_cost = -1;
  for (int ck = kVsChunkMax; ck >= kVsChunkMin; ck -= KB) {
    const long long wgs = (long long)units_per_chunk_row * ((Nk + ck - 1) / ck);
    const long long cost = ((wgs + slots - 1) / slots) * (ck + 4 * KB);
    if (best_cost < 0 || cost < best_cost) { best = ck; best_cost = cost; }
  }
  return best;
}

hipError_t launch_vs_scores(const VsScoreArgs& a0, hipStream_t st) {
  VsScoreArgs a = a0;
  // listed heads grouped by KV head (stable), split into groups of at most GH
  VsGroupTable t;
  t.n = 0;
  int pos = 0;
  const int rep = a.H / a.Hkv;
  bool done[256] = {};
  for (int i = 0; i < a.heads.n; ++i) {
    if (done[i]) continue;
    const int kvh = a.heads.h[i] / rep;
    for (int j = i; j < a.heads.n; ++j) {
      if (done[j] || a.heads.h[j] / rep != kvh) continue;
      if (t.n == 0 || t.cnt[t.n - 1] == GH || a.heads.h[t.order[t.first[t.n - 1]]] / rep != kvh) {
        t.first[t.n] = (int16_t)pos;
        t.cnt[t.n] = 0;
        ++t.n;
      }
      t.order[pos++] = (int16_t)j;
      ++t.cnt[t.n - 1];
      done[j] = true;
    }
  }
  a.chunk_keys = vs_chunk_keys(t.n * a.B, a.Nk, vs_slots());
  a.nchunks = (a.Nk + a.chunk_keys - 1) / a.chunk_keys;
  dim3 grid(t.n, a.nchunks, a.B);
  a.row_stats = a.part_ml + (size_t)a.B * a.heads.n * a.nchunks * 128;
  hipLaunchKernelGGL(vs_group_pass1_kernel, grid, dim3(GT), 0, st, a, t);
  hipLaunchKernelGGL(vs_row_stats_kernel, dim3(a.heads.n, a.B), dim3(1024), 0, st, a);
  hipLaunchKernelGGL(vs_group_pass2_kernel, grid, dim3(GT), 0, st, a, t);
  const int cb = std::min(64, (a.Nk + 255) / 256);
  hipLaunchKernelGGL(vs_diag_combine_kernel, dim3(cb, a.heads.n, a.B), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_vs_select(const float* v, const float* s, int B, int Nk, int H, const HeadList& heads, int nv,
                            int ns, int32_t* cols, int32_t* cols_count, int cols_cap, int32_t* diags,
                            int32_t* diags_count, int diags_cap, hipStream_t st) {
  hipLaunchKernelGGL(vs_select_kernel, dim3(2, heads.n, B), dim3(1024), 0, st, v, s, Nk, H, heads, nv, ns, cols,
                     cols_count, cols_cap, diags, diags_count, diags_cap);
  return hipGetLastError();
}

hipError_t launch_ashape_fill(int B, int H, const HeadList& heads, int ncols, int ndiags, int32_t* cols,
                              int32_t* cols_count, int cols_cap, int32_t* diags, int32_t* diags_count,
                              int diags_cap, hipStream_t st) {
  if (heads.n == 0) return hipSuccess;
  hipLaunchKernelGGL(ashape_fill_kernel, dim3(heads.n, B), dim3(256), 0, st, H, heads, ncols, ndiags, cols,
                     cols_count, cols_cap, diags, diags_count, diags_cap);
  return hipGetLastError();
}

}  // namespace dsa
