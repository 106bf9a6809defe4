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

// Block scores S[I][J] = qbar_I . kbar_J * scale (J <= I), 64x64 tile per
// workgroup, four waves of 32x32 each, v_mfma_f32_32x32x16_bf16.
__global__ __launch_bounds__(256) void block_scores_kernel(const uint16_t* __restrict__ qbar,
                                                           const uint16_t* __restrict__ kbar, int H, int Hkv,
                                                           int nqb, int nkb, HeadList heads, float scale,
                                                           float* __restrict__ scores) {
  const int J0 = blockIdx.x * 64, I0 = blockIdx.y * 64;
  if (J0 > I0 + 63) return;
  const int hi = blockIdx.z % heads.n, b = blockIdx.z / heads.n;
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
    if (I < nqb && J < nkb) sp[(size_t)I * nkb + J] = (J <= I) ? acc[v] * scale : -INFINITY;
  }
}

// One workgroup per (query block I, listed head, batch).
__global__ __launch_bounds__(256) void block_select_kernel(const float* __restrict__ scores, int H, int nqb,
                                                           int nkb, HeadList heads, int mode, int topk,
                                                           float log_alpha, int force_first, int force_diag,
                                                           int32_t* __restrict__ idx, int32_t* __restrict__ count,
                                                           int cap) {
  __shared__ SelectSmem<256> sm;
  const int I = blockIdx.x, hi = blockIdx.y, b = blockIdx.z;
  const int h = heads.h[hi];
  const float* row = scores + (((size_t)(b * heads.n + hi) * nqb) + I) * nkb;
  int32_t* out = idx + (((size_t)(b * H + h) * nqb) + I) * cap;
  int n;
  if (mode == 0) {
    // candidates [0, I] minus the forced blocks; those are the smallest (0) and
    // largest (I) indices, so the merged list is [0] + selected + [I].
    n = select_topk<256>(row, 0, I + 1, force_first ? 0 : -1, force_diag ? I : -1, topk,
                         out + (force_first ? 1 : 0), sm);
    if (threadIdx.x == 0) {
      int c = n;
      if (force_first) { out[0] = 0; ++c; }
      if (force_diag && !(force_first && I == 0)) { out[c] = I; ++c; }
      count[(size_t)(b * H + h) * nqb + I] = c;
    }
  } else {
    // threshold over all J <= I; forced blocks are added when not already kept
    n = select_threshold<256>(row, 0, I + 1, log_alpha, out, 0, sm, nullptr);
    if (threadIdx.x == 0) {
      int c = n;
      if (force_first && (c == 0 || out[0] != 0)) {
        for (int i = c; i > 0; --i) out[i] = out[i - 1];
        out[0] = 0;
        ++c;
      }
      if (force_diag && (c == 0 || out[c - 1] != I)) { out[c] = I; ++c; }
      count[(size_t)(b * H + h) * nqb + I] = c;
    }
  }
}

}  // namespace

hipError_t launch_pool(const uint16_t* src, int B, int Hs, int N, const HeadList& heads, int block, uint16_t* dst,
                       hipStream_t st) {
  const int nb = (N + block - 1) / block;
  if (heads.n == 0) return hipSuccess;
  hipLaunchKernelGGL(pool_kernel, dim3(nb, heads.n, B), dim3(256), 0, st, src, Hs, N, heads, block, nb, dst);
  return hipGetLastError();
}

hipError_t launch_block_scores(const uint16_t* qbar, const uint16_t* kbar, int B, int H, int Hkv, int nqb, int nkb,
                               const HeadList& heads, float scale, float* scores, hipStream_t st) {
  if (heads.n == 0) return hipSuccess;
  dim3 grid((nkb + 63) / 64, (nqb + 63) / 64, heads.n * B);
  hipLaunchKernelGGL(block_scores_kernel, grid, dim3(256), 0, st, qbar, kbar, H, Hkv, nqb, nkb, heads, scale, scores);
  return hipGetLastError();
}

hipError_t launch_block_select(const float* scores, int B, int H, int nqb, int nkb, const HeadList& heads, int mode,
                               int topk, float log_alpha, int force_first, int force_diag, int32_t* idx,
                               int32_t* count, int cap, hipStream_t st) {
  if (heads.n == 0) return hipSuccess;
  hipLaunchKernelGGL(block_select_kernel, dim3(nqb, heads.n, B), dim3(256), 0, st, scores, H, nqb, nkb, heads, mode,
                     topk, log_alpha, force_first, force_diag, idx, count, cap);
  return hipGetLastError();
}

}  // namespace dsa
