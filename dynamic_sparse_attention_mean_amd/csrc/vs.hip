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
// Two passes over K per head on v_mfma_f32_32x32x16_bf16: pass 1 finds each
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

// K fragments of keys kt*64 + 32 kb + (0..31) (zero beyond Nk).
struct KFrag {
  u32x4 x[8];
};
__device__ __forceinline__ void load_kfrag(const uint16_t* kp, int Nk, int kt, int kb, KFrag& k) {
  const int l = threadIdx.x & 63, hh = l >> 5;
  const int key = kt * 64 + 32 * kb + (l & 31);
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (key < Nk) x = *(const u32x4*)(kp + (size_t)key * 128 + 16 * ks + 8 * hh);
    k.x[ks] = x;
  }
}

// S^T block: those keys against this wave's 32 query rows.
__device__ __forceinline__ f32x16 score_block(const KFrag& k, const Frag& f) {
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, k.x[ks]), f.q[ks], acc, 0, 0, 0);
  return acc;
}

constexpr float kScale2 = 1.4426950408889634f * 0.08838834764831845f;   // log2(e) / sqrt(128)

__global__ __launch_bounds__(256) void vs_pass1_kernel(VsScoreArgs a) {
  __shared__ float s_m[2][64], s_l[2][64];
  const int hi = blockIdx.x, c = blockIdx.y, b = blockIdx.z;
  const int h = a.heads.h[hi];
  const int kvh = h / (a.H / a.Hkv);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, hh = l >> 5, qn = l & 31;
  const int kb = w & 1, qb = w >> 1;
  const int r = 32 * qb + qn;
  const int pr = a.Nk - a.last_q + r;
  Frag f;
  load_qfrag(a, b, h, r, f);
  const uint16_t* kp = a.k + ((size_t)(b * a.Hkv + kvh) * a.Nk) * 128;
  float m = -INFINITY, s = 0.f;
  const int kt_end = min((c + 1) * CH, (a.Nk + 63) / 64);
  KFrag kn;
  if (c * CH < kt_end) load_kfrag(kp, a.Nk, c * CH, kb, kn);
  for (int kt = c * CH; kt < kt_end; ++kt) {
    const KFrag kc = kn;
    if (kt + 1 < kt_end) load_kfrag(kp, a.Nk, kt + 1, kb, kn);   // one tile ahead
    const f32x16 acc = score_block(kc, f);
    float z[16];
    float mt = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = kt * 64 + 32 * kb + 8 * (v >> 2) + 4 * hh + (v & 3);
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
  // combine the two lanes of each query (hh = 0, 1), then the two key halves
  const float m2 = __shfl_xor(m, 32, 64), s2 = __shfl_xor(s, 32, 64);
  const float mm = fmaxf(m, m2);
  const float ss = (mm == -INFINITY) ? 0.f
                   : (hh == 0 ? s * __builtin_amdgcn_exp2f(m - mm) + s2 * __builtin_amdgcn_exp2f(m2 - mm)
                              : s2 * __builtin_amdgcn_exp2f(m2 - mm) + s * __builtin_amdgcn_exp2f(m - mm));
  if (hh == 0) { s_m[kb][r] = mm; s_l[kb][r] = ss; }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int rr = threadIdx.x;
    const float ma = s_m[0][rr], mb = s_m[1][rr];
    const float mm2 = fmaxf(ma, mb);
    const float ll = (mm2 == -INFINITY) ? 0.f
                     : s_l[0][rr] * __builtin_amdgcn_exp2f(ma - mm2) + s_l[1][rr] * __builtin_amdgcn_exp2f(mb - mm2);
    float* pm = a.part_ml + (((size_t)(b * a.heads.n + hi) * a.nchunks + c) * 2) * 64;
    pm[rr] = mm2;
    pm[64 + rr] = ll;
  }
}

__global__ __launch_bounds__(256) void vs_pass2_kernel(VsScoreArgs a) {
  __shared__ float s_p[64 * 65];
  __shared__ float s_diag[DSPAN];
  __shared__ float s_mr[64], s_il[64];
  const int hi = blockIdx.x, c = blockIdx.y, b = blockIdx.z;
  const int h = a.heads.h[hi];
  const int kvh = h / (a.H / a.Hkv);
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, hh = l >> 5, qn = l & 31;
  const int kb = w & 1, qb = w >> 1;
  const int r = 32 * qb + qn;
  const int pr = a.Nk - a.last_q + r;
  const size_t row = (size_t)(b * a.heads.n + hi);

  if (tid < 64) {
    // final row max and sum, combined over all chunks in ascending order
    const float* pm = a.part_ml + (row * a.nchunks) * 128;
    float m = -INFINITY, s = 0.f;
    for (int cc = 0; cc < a.nchunks; ++cc) {
      const float mc = pm[cc * 128 + tid], sc = pm[cc * 128 + 64 + tid];
      const float mn = fmaxf(m, mc);
      if (mn != -INFINITY) s = s * __builtin_amdgcn_exp2f(m - mn) + sc * __builtin_amdgcn_exp2f(mc - mn);
      m = mn;
    }
    s_mr[tid] = m;
    s_il[tid] = s > 0.f ? 1.0f / s : 0.f;
  }
  for (int i = tid; i < DSPAN; i += 256) s_diag[i] = 0.f;
  __syncthreads();

  Frag f;
  load_qfrag(a, b, h, r, f);
  const uint16_t* kp = a.k + ((size_t)(b * a.Hkv + kvh) * a.Nk) * 128;
  const float mr = s_mr[r & 63], il = s_il[r & 63];
  const int kt0 = c * CH;
  const int kt_end = min((c + 1) * CH, (a.Nk + 63) / 64);
  // offset of local diagonal slot 0 of this chunk
  const int o_min = a.Nk - a.last_q - (kt0 + CH - 1) * 64 - 63;
  float* vo = a.v_out + row * a.Nk;
  KFrag kn;
  if (kt0 < kt_end) load_kfrag(kp, a.Nk, kt0, kb, kn);
  for (int kt = kt0; kt < kt_end; ++kt) {
    const KFrag kc = kn;
    if (kt + 1 < kt_end) load_kfrag(kp, a.Nk, kt + 1, kb, kn);   // one tile ahead
    const f32x16 acc = score_block(kc, f);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int cc = 32 * kb + 8 * (v >> 2) + 4 * hh + (v & 3);
      const int key = kt * 64 + cc;
      const bool ok = key < a.Nk && key <= pr && r < a.last_q;
      s_p[r * 65 + cc] = ok ? __builtin_amdgcn_exp2f(acc[v] * kScale2 - mr) * il : 0.f;
    }
    __syncthreads();
    {
      // column sums: four lanes per column, 16 rows each, then (p0 + p1) + (p2 + p3)
      const int col = tid >> 2, part = tid & 3;
      float cs = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) cs += s_p[(16 * part + i) * 65 + col];
      cs += __shfl_xor(cs, 1, 64);
      cs += __shfl_xor(cs, 2, 64);
      if (part == 0 && kt * 64 + col < a.Nk) vo[kt * 64 + col] = cs;
    }
    // diagonal sums: two lanes per diagonal dl = r - c (lower and upper rows of
    // its range), then their sum; lanes 254 and 255 idle
    {
      const int dg = tid >> 1, part = tid & 1;
      const int dl = min(dg, 126) - 63;
      const int rlo = max(0, dl), rhi = min(63, 63 + dl);
      const int rmid = (rlo + rhi + 1) >> 1;
      float ds = 0.f;
      if (dg < 127) {
        const int r0 = part ? rmid : rlo, r1 = part ? rhi + 1 : rmid;
        for (int rr = r0; rr < r1; ++rr) ds += s_p[rr * 65 + (rr - dl)];
      }
      ds += __shfl_xor(ds, 1, 64);
      if (dg < 127 && part == 0) {
        const int o = a.Nk - a.last_q - kt * 64 + dl;
        s_diag[o - o_min] += ds;
      }
    }
    __syncthreads();
  }
  float* pd = a.part_diag + (row * a.nchunks + c) * DSPAN;
  for (int i = tid; i < DSPAN; i += 256) pd[i] = s_diag[i];
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
  dim3 grid(a.heads.n, a.nchunks, a.B);
  hipLaunchKernelGGL(vs_pass1_kernel, grid, dim3(256), 0, st, a);
  hipLaunchKernelGGL(vs_pass2_kernel, grid, dim3(256), 0, st, a);
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
