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

namespace dsa {
namespace {

constexpr int CH = 16;           // key tiles per chunk
constexpr int CK = CH * 64;      // keys per chunk
constexpr int DSPAN = CK + 64;   // diagonal partials per chunk (CK + 63 used)

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
// Per block a wave forms S^T for its 32 rows on v_mfma_f32_32x32x16_bf16 with
// the K fragments read from LDS.  Pass 2 stages each head's weights in LDS and
// reduces them along columns (four lanes per column, rows in a fixed order)
// and diagonals (one lane per diagonal, rows ascending).
constexpr int GH = 4;                // heads per workgroup
constexpr int GT = 2 * GH * 64;      // threads: wave w serves head slot w / 2, rows 32 (w % 2) ..
constexpr int KB = 32;               // keys per block
constexpr int CKB = CK / KB;         // blocks per chunk

typedef __attribute__((address_space(3))) void lds_void_vs_t;
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
  __builtin_amdgcn_global_load_lds(kp + (size_t)key * 128 + c * 8, (lds_void_vs_t*)(stage + w * 1024), 16, 0, 0);
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

// Wait until at most n of this wave's DMAs are outstanding (n = 0, 1, 2).
__device__ __forceinline__ void vs_wait_vm_upto(int n) {
  if (n >= 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
  else if (n == 1) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

constexpr int P1ST = 4;              // pass 1 ring stages: blocks prefetched three ahead

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
  const int kb0 = c * CKB, kb1 = min(nblk, kb0 + CKB);
  float m = -INFINITY, s = 0.f;
  // the loop stores nothing, so DMAs are this wave's only vector memory
  // operations and complete in issue order: a partial count is safe
  for (int i = 0; i < P1ST - 1 && kb0 + i < kb1; ++i) vs_issue_block(kp, a.Nk, kb0 + i, s_k[i]);
  for (int kb = kb0; kb < kb1; ++kb) {
    const int st = (kb - kb0) % P1ST;
    vs_wait_vm_upto(min(P1ST - 2, kb1 - 1 - kb));     // block kb landed (later ones may be in flight)
    __syncthreads();                                  // ... for every wave; all are done with kb - 1
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

__global__ __launch_bounds__(GT) void vs_group_pass2_kernel(VsScoreArgs a, VsGroupTable t) {
  __shared__ __align__(1024) char s_k[2][KB * 256];
  __shared__ float s_p[GH][64 * (KB + 1)];
  __shared__ float s_diag[GH][DSPAN];
  __shared__ float s_mr[GH][64], s_il[GH][64];
  const int c = blockIdx.y, b = blockIdx.z;
  const VsGroupInfo gi = vs_group_info(a, t);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, hh = l >> 5, qn = l & 31;
  const int g = w >> 1;
  const int r = 32 * (w & 1) + qn;
  const int pr = a.Nk - a.last_q + r;
  const size_t row = (size_t)(b * a.heads.n + gi.hi);

  // final row max and sum of each head, over all chunks in ascending order
  if ((w & 1) == 0 && gi.on) {
    const float* pm = a.part_ml + (row * a.nchunks) * 128;
    float m = -INFINITY, s = 0.f;
    for (int cc = 0; cc < a.nchunks; ++cc) {
      const float mc = pm[cc * 128 + l], sc = pm[cc * 128 + 64 + l];
      const float mn = fmaxf(m, mc);
      if (mn != -INFINITY) s = s * __builtin_amdgcn_exp2f(m - mn) + sc * __builtin_amdgcn_exp2f(mc - mn);
      m = mn;
    }
    s_mr[g][l] = m;
    s_il[g][l] = s > 0.f ? 1.0f / s : 0.f;
  }
  for (int i = tid; i < GH * DSPAN; i += GT) (&s_diag[0][0])[i] = 0.f;
  Frag f;
  load_qfrag(a, b, gi.h, gi.on ? r : 64, f);
  const uint16_t* kp = a.k + ((size_t)(b * a.Hkv + gi.kvh) * a.Nk) * 128;
  const int nblk = (a.Nk + KB - 1) / KB;
  const int kb0 = c * CKB, kb1 = min(nblk, kb0 + CKB);
  const int o_min = a.Nk - a.last_q - (c + 1) * CK + 1;   // offset of diagonal slot 0 of this chunk
  float* vo = a.v_out + row * a.Nk;
  float* sp = s_p[g];
  const int tl = tid & 127;                               // this thread's place among its head's 128
  vs_issue_block(kp, a.Nk, kb0, s_k[0]);
  __syncthreads();                                        // row statistics visible
  const float mr = s_mr[g][r & 63], il = s_il[g][r & 63];
  // A block's column sums are stored at the start of the next block, right
  // after its wait: stores and the DMA share one counter, so a store issued at
  // the end of a block would hold up the next block's wait for the DMA.
  float cs_pend = 0.f;
  int col_pend = -1;
  for (int kb = kb0; kb < kb1; ++kb) {
    const int st = (kb - kb0) & 1;
    vs_wait_vm();
    __syncthreads();                                      // block kb landed; the last block's sums are done
    if (col_pend >= 0) vo[col_pend] = cs_pend;
    col_pend = -1;
    if (kb + 1 < kb1) vs_issue_block(kp, a.Nk, kb + 1, s_k[st ^ 1]);
    if (gi.on) {
      const f32x16 acc = vs_block_scores(s_k[st], f);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int cc = 8 * (v >> 2) + 4 * hh + (v & 3);
        const int key = kb * KB + cc;
        const bool ok = key < a.Nk && key <= pr && r < a.last_q;
        sp[r * (KB + 1) + cc] = ok ? __builtin_amdgcn_exp2f(acc[v] * kScale2 - mr) * il : 0.f;
      }
    }
    __syncthreads();
    if (gi.on) {
      {
        // column sums: four lanes per column, 16 rows each, then (p0 + p1) + (p2 + p3)
        const int col = tl >> 2, part = tl & 3;
        float cs = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) cs += sp[(16 * part + i) * (KB + 1) + col];
        cs += __shfl_xor(cs, 1, 64);
        cs += __shfl_xor(cs, 2, 64);
        if (part == 0 && kb * KB + col < a.Nk) { cs_pend = cs; col_pend = kb * KB + col; }
      }
      if (tl < 95) {
        // diagonal dl = r - cc in [-31, 63]: the terms of keys cc = 0 .. 31 (rows
        // dl + cc, ascending); a fixed count lets eight reads be in flight at a
        // time.  Rows outside [0, 63] read row 0 (in bounds) and add nothing.
        const int dl = tl - 31;
        float ds = 0.f;
#pragma unroll 8
        for (int cc = 0; cc < KB; ++cc) {
          const int rr = dl + cc;
          const bool in = rr >= 0 && rr < 64;
          const float x = sp[(in ? rr : 0) * (KB + 1) + cc];
          ds += in ? x : 0.f;
        }
        s_diag[g][a.Nk - a.last_q - kb * KB + dl - o_min] += ds;
      }
    }
  }
  if (col_pend >= 0) vo[col_pend] = cs_pend;
  __syncthreads();
  if (gi.on) {
    float* pd = a.part_diag + (row * a.nchunks + c) * DSPAN;
    for (int i = tl; i < DSPAN; i += 128) pd[i] = s_diag[g][i];
  }
}

__global__ __launch_bounds__(256) void vs_diag_combine_kernel(VsScoreArgs a) {
  const int hi = blockIdx.y, b = blockIdx.z;
  const size_t row = (size_t)(b * a.heads.n + hi);
  const float* pd = a.part_diag + row * a.nchunks * DSPAN;
  float* so = a.s_out + row * a.Nk;
  for (int o = blockIdx.x * 256 + threadIdx.x; o < a.Nk; o += gridDim.x * 256) {
    int chi = (a.Nk - a.last_q + 63 - o) / CK;
    chi = min(chi, a.nchunks - 1);
    float s = 0.f;
    for (int cc = max(0, chi - 1); cc <= chi; ++cc) {
      const int o_min = a.Nk - a.last_q - (cc * CH + CH - 1) * 64 - 63;
      const int idx = o - o_min;
      if (idx >= 0 && idx < CK + 63) s += pd[(size_t)cc * DSPAN + idx];
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

size_t vs_workspace_floats(int n_rows, int Nk) {
  const int nchunks = ((Nk + 63) / 64 + CH - 1) / CH;
  return (size_t)n_rows * (2 * (size_t)Nk + (size_t)nchunks * 128 + (size_t)nchunks * DSPAN);
}

hipError_t launch_vs_scores(const VsScoreArgs& a0, hipStream_t st) {
  VsScoreArgs a = a0;
  a.chunk_tiles = CH;
  a.nchunks = ((a.Nk + 63) / 64 + CH - 1) / CH;
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
  dim3 grid(t.n, a.nchunks, a.B);
  hipLaunchKernelGGL(vs_group_pass1_kernel, grid, dim3(GT), 0, st, a, t);
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
