// Block rule: mean-pooled Q/K blocks, block scores, top-k or threshold selection.
//
// "MInference 1.0" explainer (inference-time dynamic masks): Block-Sparse heads
// average Q and K over blocks, score blocks and keep the important ones.
// "FlashPrefill" section 2.1: blocks represented by mean-pooled keys; section
// 2.2: keep blocks whose score clears a threshold relative to the row maximum.
// MoBA "FlashMoBA" section: top-k key blocks from their centroids.
#include "common.h"
#include "internal.h"
#include "select.h"

#include <algorithm>

namespace dsa {
namespace {

// One workgroup per (block, head, batch).  256 threads: c16 = tid & 15 owns
// 8 columns, rg = tid >> 4 owns rows rg, rg + 16, ...  The sum is taken in fp64
// (exact for bf16 inputs whose magnitudes span less than 2^45), divided once
// (correctly rounded), and rounded once to bf16 (nearest even).
__global__ __launch_bounds__(256) void pool_kernel(const uint16_t* __restrict__ src, int Hs, int N,
                                                   HeadList heads, int block, int nb,
                                                   uint16_t* __restrict__ dst) {
  __shared__ double red[16][129];
  const int I = blockIdx.x, hi = blockIdx.y, b = blockIdx.z;
  const int h = heads.h[hi];
  const uint16_t* base = src + ((size_t)(b * Hs + h) * N) * 128;
  const int r0 = I * block, r1 = min(N, r0 + block);
  const int tid = threadIdx.x, c16 = tid & 15, rg = tid >> 4;
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  for (int r = r0 + rg; r < r1; r += 16) {
    const u32x4 x = *(const u32x4*)(base + (size_t)r * 128 + c16 * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += (double)bf16_lo(x[e]);
      acc[2 * e + 1] += (double)bf16_hi(x[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rg][c16 * 8 + e] = acc[e];
  __syncthreads();
  if (tid < 128) {
    double s = 0.0;
    for (int g = 0; g < 16; ++g) s += red[g][tid];
    const double mean = s / (double)(r1 - r0);
    dst[((size_t)(b * Hs + h) * nb + I) * 128 + tid] = (uint16_t)f64_to_bf16_bits(mean);
  }
}

// Block scores S[I][J] = qbar_I . kbar_J * scale (J <= qb0 + I: row I is the
// chunk's query block I, absolute block qb0 + I), 64x64 tile per workgroup,
// four waves of 32x32 each, v_mfma_f32_32x32x16_bf16.
__global__ __launch_bounds__(256) void block_scores_kernel(const uint16_t* __restrict__ qbar,
                                                           const uint16_t* __restrict__ kbar, int H, int Hkv,
                                                           int nqb, int nkb, int qb0, HeadList heads, float scale,
                                                           float* __restrict__ scores) {
  const int J0 = blockIdx.x * 64, I0 = blockIdx.y * 64;
  const int hi = blockIdx.z % heads.n, b = blockIdx.z / heads.n;
  if (J0 > qb0 + I0 + 63) {
    // wholly above the diagonal: -inf (selection reads only J <= qb0 + I)
    float* sp = scores + ((size_t)(b * heads.n + hi) * nqb) * nkb;
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
      const int I = I0 + (e >> 6), J = J0 + (e & 63);
      if (I < nqb && J < nkb) sp[(size_t)I * nkb + J] = -INFINITY;
    }
    return;
  }
  const int h = heads.h[hi];
  const int kvh = h / (H / Hkv);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, hh = l >> 5;
  const int wi = w >> 1, wj = w & 1;
  const int qrow = I0 + 32 * wi + (l & 31);
  const int krow = J0 + 32 * wj + (l & 31);
  const uint16_t* qp = qbar + ((size_t)(b * H + h) * nqb) * 128;
  const uint16_t* kp = kbar + ((size_t)(b * Hkv + kvh) * nkb) * 128;
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    u32x4 xa = {0u, 0u, 0u, 0u}, xb = {0u, 0u, 0u, 0u};
    if (qrow < nqb) xa = *(const u32x4*)(qp + (size_t)qrow * 128 + 16 * ks + 8 * hh);
    if (krow < nkb) xb = *(const u32x4*)(kp + (size_t)krow * 128 + 16 * ks + 8 * hh);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xa), __builtin_bit_cast(bf16x8, xb),
                                                  acc, 0, 0, 0);
  }
  float* sp = scores + ((size_t)(b * heads.n + hi) * nqb) * nkb;
  const int J = J0 + 32 * wj + (l & 31);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int I = I0 + 32 * wi + 8 * (v >> 2) + 4 * hh + (v & 3);
    if (I < nqb && J < nkb) sp[(size_t)I * nkb + J] = (J <= qb0 + I) ? acc[v] * scale : -INFINITY;
  }
}

// One workgroup per (query block I of the chunk, listed head, batch); its
// absolute block is Ia = qb0 + I.
__global__ __launch_bounds__(256) void block_select_kernel(const float* __restrict__ scores, int H, int nqb,
                                                           int nkb, int qb0, HeadList heads, int mode, int topk,
                                                           float log_alpha, int force_first, int force_diag,
                                                           int32_t* __restrict__ idx, int32_t* __restrict__ count,
                                                           int cap) {
  __shared__ SelectSmem<256> sm;
  const int I = blockIdx.x, hi = blockIdx.y, b = blockIdx.z;
  const int Ia = qb0 + I;
  const int h = heads.h[hi];
  const float* row = scores + (((size_t)(b * heads.n + hi) * nqb) + I) * nkb;
  int32_t* out = idx + (((size_t)(b * H + h) * nqb) + I) * cap;
  int n;
  if (mode == 0) {
    // candidates [0, Ia] minus the forced blocks; those are the smallest (0) and
    // largest (Ia) indices, so the merged list is [0] + selected + [Ia].
    n = select_topk<256>(row, 0, Ia + 1, force_first ? 0 : -1, force_diag ? Ia : -1, topk,
                         out + (force_first ? 1 : 0), sm);
    if (threadIdx.x == 0) {
      int c = n;
      if (force_first) { out[0] = 0; ++c; }
      if (force_diag && !(force_first && Ia == 0)) { out[c] = Ia; ++c; }
      count[(size_t)(b * H + h) * nqb + I] = c;
    }
  } else {
    // threshold over all J <= Ia; forced blocks are added when not already kept
    n = select_threshold<256>(row, 0, Ia + 1, log_alpha, out, 0, sm, nullptr);
    if (threadIdx.x == 0) {
      int c = n;
      if (force_first && (c == 0 || out[0] != 0)) {
        for (int i = c; i > 0; --i) out[i] = out[i - 1];
        out[0] = 0;
        ++c;
      }
      if (force_diag && (c == 0 || out[c - 1] != Ia)) { out[c] = Ia; ++c; }
      count[(size_t)(b * H + h) * nqb + I] = c;
    }
  }
}

// ---------------------------------------------------------------------------
// Fused block scores + selection: the score matrix never leaves the chip
// (FlashMoBA's tiled top-k, "Optimizing Mixture of Block Attention", FlashMoBA
// section; "FlashPrefill" section 2.1, scoring fused with the block search).
//
// A workgroup of 16 waves owns a strip of R consecutive query blocks of one
// head (of a prefill chunk whose first query block is absolute block qb0).  It
// computes their scores S[I][J] (J < qb0 + I0 + R) on
// v_mfma_f32_16x16x32_bf16 into LDS (A = 16 pooled keys, B = the strip's
// pooled queries), then wave r selects row I0 + r from LDS: the radix top-k
// (four 8-bit digits of the order-preserving key, a per-wave histogram) or the
// threshold (one max-reduce), and one ordered compaction that also takes the
// forced blocks.  Rows of the strip have `stride` floats (a multiple of 16
// plus 4, so that consecutive rows start on different banks).
constexpr int FB_WAVES = 16;
constexpr int FB_THREADS = FB_WAVES * 64;

__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// S[r][J] = qbar_{I0 + r} . kbar_J * scale for r < rows, J < nk into the LDS
// strip s_sc (row r at r * stride).  B operand: strip row qr = l % 16, dims
// 32 kk + 8 kg .. + 7; A operand: 16 keys of a tile; the 16 waves take the
// tiles round robin.  Entries J > I0 + r of row r are computed too (and never
// read as scores).
__device__ __forceinline__ void strip_scores(const uint16_t* __restrict__ qp, const uint16_t* __restrict__ kp, int I0,
                                             int rows, int nk, float scale, int stride, float* s_sc) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int qr = l & 15, kg = l >> 4;
  bf16x8 qf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (qr < rows) x = *(const u32x4*)(qp + (size_t)(I0 + qr) * 128 + 32 * kk + 8 * kg);
    qf[kk] = __builtin_bit_cast(bf16x8, x);
  }
  const int ntile = (nk + 15) / 16;
  for (int t = w; t < ntile; t += FB_WAVES) {
    const int key = 16 * t + (l & 15);               // A operand row: this lane's key
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (key < nk) x = *(const u32x4*)(kp + (size_t)key * 128 + 32 * kk + 8 * kg);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x), qf[kk], acc, 0, 0, 0);
    }
    // acc[i] = S[row qr][key 16 t + 4 kg + i]
    if (qr < rows) *(f32x4*)&s_sc[qr * stride + 16 * t + 4 * kg] = acc * scale;
  }
}

__global__ __launch_bounds__(FB_THREADS) void block_index_kernel(
    const uint16_t* __restrict__ qbar, const uint16_t* __restrict__ kbar, int H, int Hkv, int nqb, int nkb,
    int qb0, HeadList heads, float scale, int R, int stride, int mode, int topk, float log_alpha, int force_first,
    int force_diag, int32_t* __restrict__ idx, int32_t* __restrict__ count, int cap, float* __restrict__ scores_out) {
  __shared__ __align__(16) float s_sc[kBlockStripFloats];
  __shared__ uint32_t s_hist[FB_WAVES][256];
  const int I0 = blockIdx.x * R;
  const int hi = blockIdx.y, b = blockIdx.z;
  const int h = heads.h[hi];
  const int kvh = h / (H / Hkv);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int rows = min(R, nqb - I0);
  const int nk = min(nkb, qb0 + I0 + rows);            // keys any row of the strip sees: J < nk
  const uint16_t* qp = qbar + ((size_t)(b * H + h) * nqb) * 128;
  const uint16_t* kp = kbar + ((size_t)(b * Hkv + kvh) * nkb) * 128;
  strip_scores(qp, kp, I0, rows, nk, scale, stride, s_sc);
  __syncthreads();

  if (scores_out) {
    // inspection copy of the strip: the full rows, -inf for J > qb0 + I
    for (int r = 0; r < rows; ++r) {
      float* dst = scores_out + (((size_t)(b * heads.n + hi) * nqb) + I0 + r) * nkb;
      for (int J = tid; J < nkb; J += FB_THREADS) dst[J] = J <= qb0 + I0 + r ? s_sc[r * stride + J] : -INFINITY;
    }
  }
  if (w >= rows) return;

  // ---- selection of row I (absolute query block Ia) by wave w
  const int I = I0 + w;
  const int Ia = qb0 + I;
  const float* sr = s_sc + w * stride;
  int32_t* out = idx + (((size_t)(b * H + h) * nqb) + I) * cap;
  const int ex0 = force_first ? 0 : -1;
  const int ex1 = force_diag ? Ia : -1;
  uint32_t T = 0u;
  int need_eq = 0;
  bool all = false, none = false;
  float cut = 0.f;
  if (mode == 0) {
    const int nex = (ex0 == 0 ? 1 : 0) + ((ex1 >= 0 && ex1 != ex0) ? 1 : 0);
    const int ncand = Ia + 1 - nex;
    none = topk <= 0 || ncand <= 0;
    all = !none && topk >= ncand;
    if (!none && !all) {
      uint32_t* hist = s_hist[w];
      uint32_t prefix = 0u, pmask = 0u;
      int kk = topk;
      for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) hist[l + 64 * i] = 0u;
        wave_lds_sync();
        for (int j = l; j <= Ia; j += 64) {
          if (j == ex0 || j == ex1) continue;
          const uint32_t key = f32_order_key(sr[j]);
          if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
        }
        wave_lds_sync();
        // lane l owns bins 255 - 4 l .. 252 - 4 l (digits in descending order)
        uint32_t c[4], sum = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) { c[i] = hist[255 - 4 * l - i]; sum += c[i]; }
        const uint32_t incl = wave_incl_scan(sum);
        const uint32_t excl = incl - sum;
        const bool hit = excl < (uint32_t)kk && incl >= (uint32_t)kk;
        uint32_t dig = 0u, before = excl;
        if (hit) {
          uint32_t run = excl;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (run + c[i] >= (uint32_t)kk) { dig = 255u - 4u * l - i; before = run; break; }
            run += c[i];
          }
        }
        const int src = __builtin_ctzll(__builtin_amdgcn_ballot_w64(hit));
        dig = __shfl(dig, src, 64);
        before = __shfl(before, src, 64);
        kk -= (int)before;
        prefix |= dig << shift;
        pmask |= 255u << shift;
        wave_lds_sync();
      }
      T = prefix;
      need_eq = kk;
    }
  } else {
    float mx = -INFINITY;
    for (int j = l; j <= Ia; j += 64) mx = fmaxf(mx, sr[j]);
    cut = wave_max(mx) + log_alpha;
  }
  // ordered compaction: forced blocks, then the selected ones (keys above T and
  // the lowest-indexed keys equal to T, or scores at or above the cut)
  int pos = 0, eqb = 0;
  for (int j0 = 0; j0 <= Ia; j0 += 64) {
    const int j = j0 + l;
    bool take = false, e = false;
    if (j <= Ia) {
      if (j == ex0 || j == ex1) {
        take = true;
      } else if (mode == 0) {
        if (all) {
          take = true;
        } else if (!none) {
          const uint32_t key = f32_order_key(sr[j]);
          take = key > T;
          e = key == T;
        }
      } else {
        take = sr[j] >= cut;
      }
    }
    const uint64_t be = __builtin_amdgcn_ballot_w64(e);
    take = take || (e && eqb + (int)ballot_rank(be) < need_eq);
    const uint64_t bt = __builtin_amdgcn_ballot_w64(take);
    const int at = pos + (int)ballot_rank(bt);
    if (take && at < cap) out[at] = j;
    pos += __popcll(bt);
    eqb += __popcll(be);
  }
  if (l == 0) count[(size_t)(b * H + h) * nqb + I] = min(pos, cap);
}

// ---------------------------------------------------------------------------
// Vertical and slash discovery from the pooled block scores ("FlashPrefill"
// section 2.1: one block search over mean-pooled keys finds the vertical,
// slash and block shapes together).  The rule: the block-level attention
// P[I, :] = softmax_{J <= I} S[I, J]; the vertical mass of key block J,
// vbar[J] = sum_I P[I, J]; the slash mass of block offset D, sbar[D] =
// sum_I P[I, I - D]; the top key blocks and offsets, expanded to every key of
// a kept block (columns) and every token offset of a kept block offset
// (diagonals D B - (B - 1) .. D B + (B - 1)).
//
// In a prefill chunk, query block I of the chunk is absolute block Ia = qb0 + I:
// its softmax runs over J <= Ia and its slash terms are the offsets Ia - J, so
// the slash masses have one entry per key block offset (nkb of them).
//
// pooled_vs_partial_kernel: a strip's scores on chip (strip_scores), each
// row's softmax in place (wave r owns row r), then the strip's column sums and
// block-diagonal sums, rows added in ascending order, to its slot of the
// partial arrays (every column and offset written, zeros where the strip has
// no term).  pooled_vs_combine_kernel adds the strips in ascending order:
// vbar and sbar are bitwise reproducible.
__global__ __launch_bounds__(FB_THREADS) void pooled_vs_partial_kernel(
    const uint16_t* __restrict__ qbar, const uint16_t* __restrict__ kbar, int H, int Hkv, int nqb, int nkb, int qb0,
    HeadList heads, float scale, int R, int stride, int nstrips, float* __restrict__ vpart, float* __restrict__ spart) {
  __shared__ __align__(16) float s_sc[kBlockStripFloats];
  const int I0 = blockIdx.x * R;
  const int hi = blockIdx.y, b = blockIdx.z;
  const int h = heads.h[hi];
  const int kvh = h / (H / Hkv);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int rows = min(R, nqb - I0);
  const int nk = min(nkb, qb0 + I0 + rows);
  strip_scores(qbar + ((size_t)(b * H + h) * nqb) * 128, kbar + ((size_t)(b * Hkv + kvh) * nkb) * 128, I0, rows,
               nk, scale, stride, s_sc);
  __syncthreads();
  if (w < rows) {
    // P[I, J] = exp(S - max) / sum over J <= Ia; entries J > Ia become 0
    const int I = qb0 + I0 + w;
    float* sr = s_sc + w * stride;
    constexpr float kLog2e = 1.4426950408889634f;
    float mx = -INFINITY;
    for (int j = l; j <= I; j += 64) mx = fmaxf(mx, sr[j]);
    mx = wave_max(mx);
    float sum = 0.f;
    for (int j = l; j <= I; j += 64) sum += __builtin_amdgcn_exp2f((sr[j] - mx) * kLog2e);
    const float il = 1.0f / wave_sum(sum);
    for (int j = l; j < nk; j += 64) sr[j] = j <= I ? __builtin_amdgcn_exp2f((sr[j] - mx) * kLog2e) * il : 0.f;
  }
  __syncthreads();
  const size_t slot = (size_t)(b * heads.n + hi) * nstrips + blockIdx.x;
  float* vp = vpart + slot * nkb;
  for (int J = tid; J < nkb; J += FB_THREADS) {
    float acc = 0.f;
    if (J < nk)
      for (int r = 0; r < rows; ++r) acc += s_sc[r * stride + J];
    vp[J] = acc;
  }
  float* sp = spart + slot * nkb;
  for (int D = tid; D < nkb; D += FB_THREADS) {
    float acc = 0.f;
    for (int r = 0; r < rows; ++r) {
      const int J = qb0 + I0 + r - D;
      if (J >= 0) acc += s_sc[r * stride + J];
    }
    sp[D] = acc;
  }
}

// vbar / sbar rows [B, n_heads, nkb] each: the strips' partials added in ascending order.
__global__ __launch_bounds__(256) void pooled_vs_combine_kernel(const float* __restrict__ vpart,
                                                                const float* __restrict__ spart, int nkb,
                                                                int n_heads, int nstrips, float* __restrict__ vbar,
                                                                float* __restrict__ sbar) {
  const int x = blockIdx.x * 256 + threadIdx.x;
  const int hi = blockIdx.y, b = blockIdx.z;
  const size_t row = (size_t)b * n_heads + hi;
  if (x < nkb) {
    float acc = 0.f;
    for (int t = 0; t < nstrips; ++t) acc += vpart[(row * nstrips + t) * nkb + x];
    vbar[row * nkb + x] = acc;
  } else if (x < 2 * nkb) {
    const int D = x - nkb;
    float acc = 0.f;
    for (int t = 0; t < nstrips; ++t) acc += spart[(row * nstrips + t) * nkb + D];
    sbar[row * nkb + D] = acc;
  }
}

// Top key blocks of vbar (blockIdx.x = 0) or top block offsets of sbar (1) for
// one listed head, expanded into the Vertical-Slash set of that head: the keys
// of the kept blocks, ascending (only the last key block can be partial, and it
// sorts last), or the union of the kept offsets' diagonal ranges, ascending
// (range i adds [max(lo_i, hi_(i-1) + 1), hi_i]: both ends ascend with D).
__global__ __launch_bounds__(1024) void pooled_vs_select_kernel(const float* __restrict__ vbar,
                                                                const float* __restrict__ sbar, int H,
                                                                int nkb, int Nk, int block, HeadList heads, int nvb,
                                                                int nsb, int32_t* cols, int32_t* cols_count,
                                                                int cols_cap, int32_t* diags, int32_t* diags_count,
                                                                int diags_cap) {
  __shared__ Select3Smem<1024> sm;
  __shared__ int32_t s_sel[kMaxPooledBlocks];
  __shared__ int32_t s_wave[16];
  const int which = blockIdx.x, hi = blockIdx.y, b = blockIdx.z;
  const int h = heads.h[hi];
  const size_t row = (size_t)b * heads.n + hi;
  const size_t bh = (size_t)b * H + h;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int m = which == 0 ? select_topk_3pass<1024>(vbar + row * nkb, nkb, nvb, s_sel, sm)
                           : select_topk_3pass<1024>(sbar + row * nkb, nkb, nsb, s_sel, sm);
  __syncthreads();
  if (which == 0) {
    int32_t* out = cols + bh * cols_cap;
    for (int e = tid; e < m * block; e += 1024) {
      const int key = s_sel[e / block] * block + e % block;
      if (key < Nk && e < cols_cap) out[e] = key;
    }
    if (tid == 0) cols_count[bh] = m == 0 ? 0 : min(cols_cap, (m - 1) * block + min(block, Nk - s_sel[m - 1] * block));
    return;
  }
  // new offsets of each kept block offset, then their exclusive prefix sums
  int c = 0;
  int lo = 0, hi_i = -1;
  if (tid < m) {
    const int D = s_sel[tid];
    lo = max(0, D * block - (block - 1));
    hi_i = min(Nk - 1, D * block + (block - 1));
    if (tid > 0) lo = max(lo, min(Nk - 1, s_sel[tid - 1] * block + (block - 1)) + 1);
    c = max(0, hi_i - lo + 1);
  }
  // block scan over the 1024 threads (m <= kMaxPooledBlocks = 1024)
  const uint32_t incl = wave_incl_scan((uint32_t)c);
  if (l == 63) s_wave[w] = (int)incl;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < w; ++i) base += s_wave[i];
  const int start = base + (int)incl - c;
  int32_t* out = diags + bh * diags_cap;
  for (int o = lo; o <= hi_i && tid < m; ++o)
    if (start + (o - lo) < diags_cap) out[start + (o - lo)] = o;
  if (tid == 1023) diags_count[bh] = min(diags_cap, base + (int)incl);
}

}  // namespace

int block_strip_rows(int nkb, int* stride) {
  const int st = ((nkb + 15) & ~15) + 4;
  if (stride) *stride = st;
  return std::min(16, kBlockStripFloats / st);
}

hipError_t launch_block_index(const uint16_t* qbar, const uint16_t* kbar, int B, int H, int Hkv, int nqb, int nkb,
                              int qb0, const HeadList& heads, float scale, int mode, int topk, float log_alpha,
                              int force_first, int force_diag, int32_t* idx, int32_t* count, int cap,
                              float* scores, hipStream_t st) {
  if (heads.n == 0) return hipSuccess;
  int stride = 0;
  const int R = block_strip_rows(nkb, &stride);
  if (R < 1) return hipErrorInvalidValue;
  dim3 grid((nqb + R - 1) / R, heads.n, B);
  hipLaunchKernelGGL(block_index_kernel, grid, dim3(FB_THREADS), 0, st, qbar, kbar, H, Hkv, nqb, nkb, qb0, heads,
                     scale, R,
                     stride, mode, topk, log_alpha, force_first, force_diag, idx, count, cap, scores);
  return hipGetLastError();
}

hipError_t launch_pooled_vs(const uint16_t* qbar, const uint16_t* kbar, int B, int H, int Hkv, int nqb, int nkb,
                            int qb0, int Nk, int block, const HeadList& heads, float scale, float* vpart, float* spart,
                            float* vbar, float* sbar, int nvb, int nsb, int32_t* cols, int32_t* cols_count,
                            int cols_cap, int32_t* diags, int32_t* diags_count, int diags_cap, hipStream_t st) {
  if (heads.n == 0) return hipSuccess;
  int stride = 0;
  const int R = block_strip_rows(nkb, &stride);
  if (R < 1 || nvb > kMaxPooledBlocks || nsb > kMaxPooledBlocks) return hipErrorInvalidValue;
  const int nstrips = (nqb + R - 1) / R;
  hipLaunchKernelGGL(pooled_vs_partial_kernel, dim3(nstrips, heads.n, B), dim3(FB_THREADS), 0, st, qbar, kbar, H, Hkv,
                     nqb, nkb, qb0, heads, scale, R, stride, nstrips, vpart, spart);
  hipLaunchKernelGGL(pooled_vs_combine_kernel, dim3((2 * nkb + 255) / 256, heads.n, B), dim3(256), 0, st, vpart,
                     spart, nkb, heads.n, nstrips, vbar, sbar);
  hipLaunchKernelGGL(pooled_vs_select_kernel, dim3(2, heads.n, B), dim3(1024), 0, st, vbar, sbar, H, nkb, Nk, block,
                     heads, nvb, nsb, cols, cols_count, cols_cap, diags, diags_count, diags_cap);
  return hipGetLastError();
}

size_t pooled_vs_partial_floats(int nqb, int nkb) {
  const int R = block_strip_rows(nkb, nullptr);
  const size_t nstrips = R >= 1 ? (size_t)(nqb + R - 1) / R : 0;
  return nstrips * (size_t)(2 * nkb);
}

hipError_t launch_pool(const uint16_t* src, int B, int Hs, int N, const HeadList& heads, int block, uint16_t* dst,
                       hipStream_t st) {
  const int nb = (N + block - 1) / block;
  if (heads.n == 0) return hipSuccess;
  hipLaunchKernelGGL(pool_kernel, dim3(nb, heads.n, B), dim3(256), 0, st, src, Hs, N, heads, block, nb, dst);
  return hipGetLastError();
}

hipError_t launch_block_scores(const uint16_t* qbar, const uint16_t* kbar, int B, int H, int Hkv, int nqb, int nkb,
                               int qb0, const HeadList& heads, float scale, float* scores, hipStream_t st) {
  if (heads.n == 0) return hipSuccess;
  dim3 grid((nkb + 63) / 64, (nqb + 63) / 64, heads.n * B);
  hipLaunchKernelGGL(block_scores_kernel, grid, dim3(256), 0, st, qbar, kbar, H, Hkv, nqb, nkb, qb0, heads, scale,
                     scores);
  return hipGetLastError();
}

hipError_t launch_block_select(const float* scores, int B, int H, int nqb, int nkb, int qb0, const HeadList& heads,
                               int mode, int topk, float log_alpha, int force_first, int force_diag, int32_t* idx,
                               int32_t* count, int cap, hipStream_t st) {
  if (heads.n == 0) return hipSuccess;
  hipLaunchKernelGGL(block_select_kernel, dim3(nqb, heads.n, B), dim3(256), 0, st, scores, H, nqb, nkb, qb0, heads,
                     mode,
                     topk, log_alpha, force_first, force_diag, idx, count, cap);
  return hipGetLastError();
}

}  // namespace dsa
