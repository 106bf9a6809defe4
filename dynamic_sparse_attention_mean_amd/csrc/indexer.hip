// Indexer token top-k (DSA) and its routed variant (MISA), plus attention over
// per-query token lists.
//
// "MISA" (gist.science 2605.07363), section on the problem: the DeepSeek sparse
// attention indexer scores every key with 64 light heads and keeps the best
// tokens, and the main attention reads only those.  Section on how MISA works:
// a router looks at the keys in large blocks, picks 8 of the 64 heads for each
// query, and only those heads score tokens.
//
//   score[i, j] = sum_{h in H(i)} w[i, h] * max(0, q_idx[i, h] . k_idx[j])   (j <= p_i)
//   router:  r[i, h] = w[i, h] * max(0, max_J q_idx[i, h] . Kbar_J), complete blocks J
//   tokens:  top-k of score[i, :], ties to the lower index, ascending
//
// Kernels (gfx950):
//   qk_heads_kernel<MODE>: (query, head) rows x keys on v_mfma_f32_32x32x16_bf16.
//     The rows of a wave are one query's 64 heads (dense indexer, router) or four
//     queries' routed heads (routed indexer); keys stream through a two-stage LDS
//     ring (DMA).  Epilogues: ReLU * w summed over heads (indexer) or a running
//     max over blocks (router).  The MFMA output layout puts 16 heads of one key
//     in a lane, so the head sum is 16 in-lane FMAs plus one lane swap.
//   router_select_kernel: top-r heads per query (rank counting over 64 values).
//   token_select_kernel: radix top-k per query row (select.h).
//   Hierarchical option (MISA section on how it works, the two-stage variant):
//     the routed scores pick `cand` candidates per query (token_select_kernel),
//     cand_score_kernel rescores them with every head (the query's 64 head rows
//     as the MFMA A operand, the gathered candidate keys as B, read straight
//     from global memory: each query has its own keys, so there is nothing to
//     share through LDS), and cand_select_kernel keeps the top-k of them.
//   token_attn_kernel: per (query, head) softmax over the gathered token list on
//     VALU; the grid is head-major so a head's K/V stays in the Infinity Cache.
//   token_attn_group_kernel: heads that share a KV head (8 or more per KV head,
//     MQA included) and the per-query token list: one wave gathers each token's
//     K and V row once for up to 16 such heads and runs both products on
//     v_mfma_f32_16x16x32_bf16.
#include "common.h"
#include "internal.h"
#include "select.h"

#include <algorithm>

namespace dsa {
namespace {

constexpr int KT = 64;            // keys per tile
constexpr int NW = 8;             // waves per workgroup
constexpr int NTI = NW * 64;      // threads per workgroup

enum { MODE_DENSE = 0, MODE_ROUTED = 1, MODE_ROUTER = 2 };

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;
typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4_t;

__device__ __forceinline__ void dma16(const void* g, lds_void_t* lds_base) {
  __builtin_amdgcn_global_load_lds(g, lds_base, 16, 0, 0);
}
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ int swz(int r, int c) { return c ^ (r & 15); }
// max(0, x) for every finite x in one instruction: the median of x, 0 and the
// largest finite float (v_med3_f32).  fmaxf(x, 0) costs two (a canonicalising
// max of x with itself first), and a median against +inf is folded back into it.
__device__ __forceinline__ float relu(float x) { return __builtin_amdgcn_fmed3f(x, 0.f, 3.40282347e38f); }

struct QkArgs {
  const uint16_t* q_idx;     // [Nq, Hi, 128]
  const uint16_t* keys;      // [nkeys, 128] (k_idx, or block means for the router)
  const float* w;            // [Nq, Hi]
  const int32_t* route;      // [Nq, R] routed heads (MODE_ROUTED)
  float* out;                // MODE_DENSE / ROUTED: scores [Nq, Nk]; MODE_ROUTER: r [Nq, Hi]
  int Nq, Nk, Hi, R, q_offset, nkeys, block;
};

// Queries of this workgroup: MODE_DENSE / ROUTER -> 8 (one per wave), MODE_ROUTED -> 32 (four per wave).
template <int MODE>
__global__ __launch_bounds__(NTI) void qk_heads_kernel(const QkArgs a) {
  __shared__ __align__(1024) char s_k[2][KT * 256];
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, qn = l & 31, hh = l >> 5;
  constexpr int QPW = MODE == MODE_ROUTED ? 4 : 1;     // queries per wave
  constexpr int NB = MODE == MODE_ROUTED ? 1 : 2;      // 32-row blocks per wave
  const int q0 = (blockIdx.x * NW + w) * QPW;          // first query of this wave

  // ---- A operand: the wave's (query, head) rows, kept in registers
  //   block hb, row m = l & 31 -> (query, head); lane holds d = 16 ks + 8 hh .. +7
  bf16x8 af[NB][8];
  float wv[NB][16];                                    // w of the 16 rows this lane's outputs cover
  bool rows_ok[NB];
#pragma unroll
  for (int hb = 0; hb < NB; ++hb) {
    int qq, head;
    if (MODE == MODE_ROUTED) {
      qq = q0 + (qn >> 3);
      const int slot = qn & 7;
      head = (qq < a.Nq && slot < a.R) ? a.route[(size_t)qq * a.R + slot] : -1;
    } else {
      qq = q0;
      head = 32 * hb + qn;
      if (head >= a.Hi) head = -1;
    }
    const bool ok = qq < a.Nq && head >= 0;
    rows_ok[hb] = ok;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (ok) x = *(const u32x4*)(a.q_idx + ((size_t)qq * a.Hi + head) * 128 + 16 * ks + 8 * hh);
      af[hb][ks] = __builtin_bit_cast(bf16x8, x);
    }
    // output rows of value v: m = 8 (v >> 2) + 4 hh + (v & 3)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = 8 * (v >> 2) + 4 * hh + (v & 3);
      int q2, h2;
      if (MODE == MODE_ROUTED) {
        q2 = q0 + (m >> 3);
        const int slot = m & 7;
        h2 = (q2 < a.Nq && slot < a.R) ? a.route[(size_t)q2 * a.R + slot] : -1;
      } else {
        q2 = q0;
        h2 = 32 * hb + m;
        if (h2 >= a.Hi) h2 = -1;
      }
      wv[hb][v] = (q2 < a.Nq && h2 >= 0) ? a.w[(size_t)q2 * a.Hi + h2] : 0.f;
    }
  }
  (void)rows_ok;

  // keys each query may see: j <= p_q (indexer) or complete blocks (router)
  int last_key;   // last key (tile row index into a.keys) any query of the workgroup needs
  {
    const int qmax = min(a.Nq - 1, (blockIdx.x * NW + NW) * QPW - 1);
    const int pmax = qmax + a.q_offset;
    last_key = MODE == MODE_ROUTER ? ((pmax + 1) / a.block - 1) : pmax;
    last_key = min(last_key, a.nkeys - 1);
  }
  const int ntiles = last_key >= 0 ? last_key / KT + 1 : 0;

  // this lane's limits: query of each output value
  float rmax[NB][16];
#pragma unroll
  for (int hb = 0; hb < NB; ++hb)
#pragma unroll
    for (int v = 0; v < 16; ++v) rmax[hb][v] = -INFINITY;

  // DMA of a 16 KB key tile: wave w, instruction j fills LDS block 8 j + w,
  // i.e. rows 4 (8 j + w) + lane / 16
  auto issue = [&](int tile, int stage) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int blk = 8 * j + w;
      const int r = 4 * blk + (l >> 4);
      const int key = min(tile * KT + r, a.nkeys - 1);
      const int c = swz(r, l & 15);
      dma16(a.keys + (size_t)key * 128 + c * 8, (lds_void_t*)(s_k[stage] + blk * 1024));
    }
  };
  // Score rows leave one tile late: the stores of tile t are issued right after
  // the DMA of tile t + 2, so the wait at the top of a tile (vmcnt(0); loads
  // and stores may complete out of order, so no partial count is safe) finds
  // both already given a whole tile of compute to finish.  Buffer stores: lanes
  // with nothing to write get an offset past the end, which the hardware drops.
  const int nrow = MODE == MODE_ROUTER ? 0 : max(0, min(QPW, a.Nq - q0));
  // bytes of this wave's score rows: at most 4 rows of 2^27 floats, 2^31 bytes, which
  // fits the descriptor's unsigned 32-bit record count (computed without signed overflow)
  const uint32_t obytes = (uint32_t)((size_t)nrow * (size_t)a.Nk * 4u);
  const __amdgpu_buffer_rsrc_t orow =
      __builtin_amdgcn_make_buffer_rsrc(a.out + (size_t)min(q0, a.Nq) * a.Nk, (short)0, (int)obytes, 0x00020000);
  float pend_v[2][QPW];
  uint32_t pend_o[2][QPW];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int j = 0; j < QPW; ++j) { pend_v[kb][j] = 0.f; pend_o[kb][j] = 0xFFFFFFFFu; }
  auto flush = [&]() {
    if (MODE == MODE_ROUTER) return;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < QPW; ++j)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(pend_v[kb][j]), orow, pend_o[kb][j], 0, 0);
  };
  if (ntiles > 0) issue(0, 0);
  for (int t = 0; t < ntiles; ++t) {
    const int stage = t & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // tile t landed (each wave waited for its own DMA) and every wave is done
    // reading the stage the next DMA overwrites.  A bare s_barrier: nothing in
    // global memory needs ordering here.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (t + 1 < ntiles) issue(t + 1, stage ^ 1);
    if (t > 0) flush();                                // scores of tile t - 1
    const char* sk = s_k[stage];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int row = 32 * kb + qn;
      u32x4 kf[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) kf[ks] = *(const u32x4*)(sk + row * 256 + swz(row, 2 * ks + hh) * 16);
      f32x16 c[NB];
#pragma unroll
      for (int hb = 0; hb < NB; ++hb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) c[hb][v] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
          c[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[hb][ks], __builtin_bit_cast(bf16x8, kf[ks]), c[hb], 0, 0, 0);
      }
      const int key = t * KT + 32 * kb + qn;           // key of this lane's output column
      if (MODE == MODE_ROUTER) {
        // complete block `key` (J) is visible to query q iff 64 J + 63 <= p_q
        const int p = q0 + a.q_offset;
        const bool vis = key <= last_key && (key + 1) * a.block - 1 <= p;
#pragma unroll
        for (int hb = 0; hb < NB; ++hb)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (vis) rmax[hb][v] = fmaxf(rmax[hb][v], c[hb][v]);
      } else {
        float s[QPW];
#pragma unroll
        for (int j = 0; j < QPW; ++j) s[j] = 0.f;
#pragma unroll
        for (int hb = 0; hb < NB; ++hb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int j = MODE == MODE_ROUTED ? (v >> 2) : 0;   // query of row 8 (v >> 2) + ...
            s[j] = __builtin_fmaf(wv[hb][v], relu(c[hb][v]), s[j]);
          }
#pragma unroll
        for (int j = 0; j < QPW; ++j) {
          const float tot = s[j] + __shfl_xor(s[j], 32, 64);
          const int qq = q0 + j;
          const bool wr = hh == (j & 1) && qq < a.Nq && key <= qq + a.q_offset && key < a.Nk;
          pend_v[kb][j] = tot;
          pend_o[kb][j] = wr ? (uint32_t)(j * a.Nk + key) * 4u : 0xFFFFFFFFu;
        }
      }
    }
  }
  if (ntiles > 0) flush();                             // scores of the last tile
  if (MODE == MODE_ROUTER) {
    // max over the lanes of each head (the 32 key columns), then r = w * max(0, .)
#pragma unroll
    for (int hb = 0; hb < NB; ++hb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float x = rmax[hb][v];
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
        rmax[hb][v] = x;
      }
    if (qn == 0 && q0 < a.Nq) {
#pragma unroll
      for (int hb = 0; hb < NB; ++hb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int h = 32 * hb + 8 * (v >> 2) + 4 * hh + (v & 3);
          if (h < a.Hi) {
            const float mx = rmax[hb][v];
            a.out[(size_t)q0 * a.Hi + h] = wv[hb][v] * (mx > 0.f ? mx : 0.f);
          }
        }
    }
  }
}

// Top-R heads per query by r (ties to the lower head), ascending head order.
__global__ void router_select_kernel(const float* r, int Nq, int Hi, int R, int32_t* route, int32_t* route_out) {
  const int q = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (q >= Nq) return;
  const float x = l < Hi ? r[(size_t)q * Hi + l] : -INFINITY;
  int rank = 0;
  for (int o = 0; o < Hi; ++o) {
    const float y = __shfl(x, o, 64);
    rank += (y > x) || (y == x && o < l);
  }
  const bool sel = l < Hi && rank < R;
  const uint64_t bal = __builtin_amdgcn_ballot_w64(sel);
  if (sel) {
    const uint32_t pos = ballot_rank(bal);
    route[(size_t)q * R + pos] = l;
    if (route_out) route_out[(size_t)q * R + pos] = l;
  }
}

// Top-k per query row over keys [0, p_q], ties to the lower index, written in
// ascending order (three passes over the row: select_topk_3pass).
constexpr int TS_THREADS = 1024;

__global__ __launch_bounds__(TS_THREADS) void token_select_kernel(const float* scores, int Nq, int Nk, int q_offset,
                                                                  int k, int32_t* tok, int32_t* cnt, int cap) {
  __shared__ Select3Smem<TS_THREADS> sm;
  const int q = blockIdx.x;
  const int n = min(q + q_offset + 1, Nk);
  const int m = select_topk_3pass<TS_THREADS>(scores + (size_t)q * Nk, n, k, tok + (size_t)q * cap, sm);
  if (threadIdx.x == 0) cnt[q] = m;
}

// ---------------------------------------------------------------- hierarchical option
constexpr int CS_WAVES = 4;       // queries (waves) per workgroup

// score[q, c] = sum_h w[q, h] max(0, q_idx[q, h] . k_idx[cand[q, c]]) for c < ccount[q].
// Candidate rows have stride ccap (the caller's list capacity), score rows
// stride ostride (the workspace's, which holds exactly `cand` per query).
// One wave per query: rows 32 hb + m of the A operand are heads, columns the
// 32 candidates of a block; the next block's keys are loaded while this one's
// MFMAs run.
__global__ __launch_bounds__(CS_WAVES * 64) void cand_score_kernel(const uint16_t* __restrict__ q_idx,
                                                                   const uint16_t* __restrict__ k_idx,
                                                                   const float* __restrict__ w,
                                                                   const int32_t* __restrict__ cand,
                                                                   const int32_t* __restrict__ ccount, int Nq, int Hi,
                                                                   int ccap, int ostride, float* __restrict__ out) {
  const int wv_ = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = blockIdx.x * CS_WAVES + wv_;
  if (q >= Nq) return;
  const int l = threadIdx.x & 63, qn = l & 31, hh = l >> 5;
  bf16x8 af[2][8];
  float wv[2][16];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int head = 32 * hb + qn;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (head < Hi) x = *(const u32x4*)(q_idx + ((size_t)q * Hi + head) * 128 + 16 * ks + 8 * hh);
      af[hb][ks] = __builtin_bit_cast(bf16x8, x);
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int h2 = 32 * hb + 8 * (v >> 2) + 4 * hh + (v & 3);
      wv[hb][v] = h2 < Hi ? w[(size_t)q * Hi + h2] : 0.f;
    }
  }
  const int n = __builtin_amdgcn_readfirstlane(ccount[q]);
  const int32_t* cq = cand + (size_t)q * ccap;
  float* oq = out + (size_t)q * ostride;
  const int nb = (n + 31) / 32;
  // this lane's key row of block b: candidate 32 b + qn (the first one past the end)
  auto load = [&](int b, u32x4 (&kf)[8]) {
    const int c = 32 * b + qn;
    const int key = cq[c < n ? c : 0];
    const uint16_t* row = k_idx + (size_t)key * 128 + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kf[ks] = *(const u32x4*)(row + 16 * ks);
  };
  u32x4 kc[8], kn[8];
  if (nb > 0) load(0, kc);
  for (int b = 0; b < nb; ++b) {
    if (b + 1 < nb) load(b + 1, kn);
    f32x16 c[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) c[hb][v] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        c[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[hb][ks], __builtin_bit_cast(bf16x8, kc[ks]), c[hb], 0, 0, 0);
    }
    float sacc = 0.f;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc = __builtin_fmaf(wv[hb][v], relu(c[hb][v]), sacc);
    const float tot = sacc + __shfl_xor(sacc, 32, 64);
    const int col = 32 * b + qn;
    if (hh == 0 && col < n) oq[col] = tot;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kc[ks] = kn[ks];
  }
}

// Top-k of a query's rescored candidates (ties to the lower position, which is
// the lower key: candidate lists ascend), mapped back to key indices.
__global__ __launch_bounds__(TS_THREADS) void cand_select_kernel(const float* scores, int sstride,
                                                                 const int32_t* cand, const int32_t* ccount, int ccap,
                                                                 int k, int32_t* tok, int32_t* cnt, int cap) {
  __shared__ Select3Smem<TS_THREADS> sm;
  __shared__ int32_t pos[kMaxTokensPerQuery];
  const int q = blockIdx.x;
  const int n = ccount[q];
  const int m = select_topk_3pass<TS_THREADS>(scores + (size_t)q * sstride, n, min(k, kMaxTokensPerQuery), pos, sm);
  __syncthreads();
  for (int r = threadIdx.x; r < m; r += TS_THREADS) tok[(size_t)q * cap + r] = cand[(size_t)q * ccap + pos[r]];
  if (threadIdx.x == 0) cnt[q] = m;
}

// ---------------------------------------------------------------- token attention
constexpr int TA_THREADS = 256;
constexpr int TA_MAXTOK = 4096;
constexpr int TA_U = 8;            // token rows each 16-lane group keeps in flight

// Sum over the 16 lanes of each DPP row; every lane of the row gets the total.
// quad_perm [1,0,3,2] and [2,3,0,1] sum each quad, row_half_mirror joins the
// two quads of each 8-lane half, row_mirror joins the two halves.
__device__ __forceinline__ float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
  return x;
}

// One workgroup per (head, query); heads outermost so a head's K/V stay cached.
// A 16-lane group owns one token row at a time (lane = 8 dims, 16 bytes of the
// row), the four groups of a wave take four tokens, and every group keeps
// TA_U rows in flight: the gathered K rows (scores) and V rows (output) stream
// with enough loads outstanding to cover the cache latency.
__global__ __launch_bounds__(TA_THREADS) void token_attn_kernel(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                                                int H, int Hkv, int Nq, int Nk, const int32_t* tidx,
                                                                const int32_t* tcount, int tcap, void* o, float* lse,
                                                                int out_f32, int B, HeadList th) {
  __shared__ float s_p[TA_MAXTOK];
  __shared__ int32_t s_t[TA_MAXTOK];
  __shared__ float s_red[4][4][128];
  __shared__ float s_ms[8];
  const int bid = blockIdx.x;
  const int h = th.h[bid / (Nq * B)];
  const int rem = bid % (Nq * B);
  const int b = rem / Nq, i = rem % Nq;
  const int kvh = h / (H / Hkv);
  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63;
  const int sub = l & 15, tg = l >> 4;
  const int n = min(min(tcount[(size_t)b * Nq + i], tcap), TA_MAXTOK);
  const int32_t* tl = tidx + ((size_t)b * Nq + i) * tcap;
  // keys after the query's position (j > p_i) are not part of M(i): dropped like out-of-range ones
  const int p_i = i + (Nk - Nq);
  for (int x = tid; x < n; x += TA_THREADS) {
    const int j = tl[x];
    s_t[x] = (j >= 0 && j <= p_i) ? j : -1;
  }
  __syncthreads();
  const uint16_t* qrow = q + (((size_t)b * H + h) * Nq + i) * 128;
  const uint16_t* kb = k + ((size_t)b * Hkv + kvh) * (size_t)Nk * 128;
  const uint16_t* vb = v + ((size_t)b * Hkv + kvh) * (size_t)Nk * 128;
  const u32x4 qx = *(const u32x4*)(qrow + sub * 8);
  // scores in log2 units: q . k * log2(e) / sqrt(128)
  const float scale2 = 1.4426950408889634f * 0.08838834764831845f;
  float qv[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) { qv[2 * e] = bf16_lo(qx[e]) * scale2; qv[2 * e + 1] = bf16_hi(qx[e]) * scale2; }

  // ---- scores: token x = x0 + 16 u + 4 wv + tg
  float mloc = -INFINITY;
  for (int x0 = 0; x0 < n; x0 += 16 * TA_U) {
    u32x4 kx[TA_U];
    int jj[TA_U];
#pragma unroll
    for (int u = 0; u < TA_U; ++u) {
      const int x = x0 + 16 * u + 4 * wv + tg;
      jj[u] = x < n ? s_t[x] : -1;
      u32x4 z = {0u, 0u, 0u, 0u};
      kx[u] = jj[u] >= 0 ? *(const u32x4*)(kb + (size_t)jj[u] * 128 + sub * 8) : z;
    }
#pragma unroll
    for (int u = 0; u < TA_U; ++u) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        d = __builtin_fmaf(qv[2 * e], bf16_lo(kx[u][e]), d);
        d = __builtin_fmaf(qv[2 * e + 1], bf16_hi(kx[u][e]), d);
      }
      d = row16_sum(d);
      const int x = x0 + 16 * u + 4 * wv + tg;
      const float sc = jj[u] >= 0 ? d : -INFINITY;
      if (x < n) {
        if (sub == 0) s_p[x] = sc;
        mloc = fmaxf(mloc, sc);
      }
    }
  }
  mloc = wave_max(mloc);
  if (l == 0) s_ms[wv] = mloc;
  __syncthreads();
  const float m = fmaxf(fmaxf(s_ms[0], s_ms[1]), fmaxf(s_ms[2], s_ms[3]));
  float lsum = 0.f;
  for (int x = tid; x < n; x += TA_THREADS) {
    const float p = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s_p[x] - m);
    s_p[x] = p;
    lsum += p;
  }
  lsum = wave_sum(lsum);
  if (l == 0) s_ms[4 + wv] = lsum;
  __syncthreads();

  // ---- output: lane accumulates dims 8 sub .. +7 over its group's tokens
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int x0 = 0; x0 < n; x0 += 16 * TA_U) {
    u32x4 vx[TA_U];
    float pp[TA_U];
#pragma unroll
    for (int u = 0; u < TA_U; ++u) {
      const int x = x0 + 16 * u + 4 * wv + tg;
      const int j = x < n ? s_t[x] : -1;
      pp[u] = j >= 0 ? s_p[x] : 0.f;
      u32x4 z = {0u, 0u, 0u, 0u};
      vx[u] = j >= 0 ? *(const u32x4*)(vb + (size_t)j * 128 + sub * 8) : z;
    }
#pragma unroll
    for (int u = 0; u < TA_U; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] = __builtin_fmaf(pp[u], bf16_lo(vx[u][e]), acc[2 * e]);
        acc[2 * e + 1] = __builtin_fmaf(pp[u], bf16_hi(vx[u][e]), acc[2 * e + 1]);
      }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) s_red[wv][tg][sub * 8 + e] = acc[e];
  __syncthreads();
  if (tid < 128) {
    const float ltot = s_ms[4] + s_ms[5] + s_ms[6] + s_ms[7];
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    float sum = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2)
#pragma unroll
      for (int g2 = 0; g2 < 4; ++g2) sum += s_red[w2][g2][tid];
    const float val = sum * inv;
    const size_t oi = (((size_t)b * H + h) * Nq + i) * 128 + tid;
    if (out_f32) ((float*)o)[oi] = val;
    else ((uint16_t*)o)[oi] = (uint16_t)f32_to_bf16_bits(val);
    if (tid == 0 && lse) lse[((size_t)b * H + h) * Nq + i] = ltot > 0.f ? (m + __log2f(ltot)) * 0.6931471805599453f : -INFINITY;
  }
}

// ---------------------------------------------------------------- token attention, shared K/V
// MISA's problem section: the main attention reads only the tokens the indexer
// kept, one list per query for all heads.  When many heads share one KV head,
// the K and V rows of a query's tokens serve every one of them: a wave takes
// (query, up to 16 heads of one KV head) and gathers each row once.
//   S^T = K Q^T   (keys x heads): A = 16 gathered K rows x 32 dims, straight
//                 from global memory; B = the heads' q (kept in registers).
//   O^T += V^T P^T (dims x heads): B = the lane's own bf16 weights; A = V^T,
//                 read with ds_read_b64_tr_b16 from the wave's LDS copy of the
//                 chunk's 32 V rows.  The keys along the K dimension are
//                 ordered so that the score layout of the first product is the
//                 weight layout of the second: lane (g, t) holds keys
//                 16 kb + 4 g + i (kb = 0, 1; i = 0..3) of head t in both.
constexpr int TG_WAVES = 4;
constexpr int TG_VSTRIDE = 288;      // bytes per staged V row: 256 + 32, so 8 rows of a transposing read hit 64 banks
constexpr int TG_MAXGROUPS = 128;

__global__ __launch_bounds__(TG_WAVES * 64) void token_attn_group_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int H, int Hkv,
    int Nq, int Nk, int B, const int32_t* __restrict__ tidx, const int32_t* __restrict__ tcount, int tcap, void* o,
    float* lse, int out_f32, TokenGroups tg) {
  __shared__ __align__(16) char s_v[TG_WAVES][32 * TG_VSTRIDE];
  const int wv_ = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = threadIdx.x & 63, t = l & 15, g = l >> 4;
  const int gi = blockIdx.y;
  const int h0 = tg.h0[gi], nh = tg.cnt[gi];
  const int row = blockIdx.x * TG_WAVES + wv_;          // b * Nq + i
  if (row >= B * Nq) return;
  const int b = row / Nq, i = row % Nq;
  const int kvh = h0 / (H / Hkv);
  const uint16_t* kb = k + ((size_t)b * Hkv + kvh) * (size_t)Nk * 128;
  const uint16_t* vb = v + ((size_t)b * Hkv + kvh) * (size_t)Nk * 128;
  const bool hok = t < nh;
  u32x4 qf[4];
#pragma unroll
  for (int ds = 0; ds < 4; ++ds) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (hok) x = *(const u32x4*)(q + (((size_t)b * H + h0 + t) * Nq + i) * 128 + 32 * ds + 8 * g);
    qf[ds] = x;
  }
  const int n = min(tcount[row], tcap);
  const int32_t* tl = tidx + (size_t)row * tcap;
  char* sv = s_v[wv_];
  const uint32_t svb = (uint32_t)(uintptr_t)(lds_char_t*)sv;
  const float scale2 = 1.4426950408889634f * 0.08838834764831845f;   // log2(e) / sqrt(128)

  // one chunk of 32 tokens: K fragments (A operand of the scores) for keys
  // 16 kb + t, and this lane's half of V row l / 2
  struct Chunk {
    u32x4 kf[2][4];
    u32x4 vx[8];
    bool kval[2];
  };
  // keys after the query's position (j > p_i) are not part of M(i): dropped like out-of-range ones
  const int p_i = i + (Nk - Nq);
  auto token = [&](int x, bool& ok) {
    int j = x < n ? tl[x] : -1;
    ok = j >= 0 && j <= p_i;
    return ok ? j : 0;
  };
  auto load = [&](int c0, Chunk& c) {
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk) {
      bool ok;
      const int j = token(c0 + 16 * kbk + t, ok);
      c.kval[kbk] = ok;
      const uint16_t* kr = kb + (size_t)j * 128 + 8 * g;
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) c.kf[kbk][ds] = *(const u32x4*)(kr + 32 * ds);
    }
    bool ok;
    const int j = token(c0 + (l >> 1), ok);
    const uint16_t* vr = vb + (size_t)j * 128 + 64 * (l & 1);
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) c.vx[cc] = *(const u32x4*)(vr + 8 * cc);
  };

  f32x4 acc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  Chunk cur, nxt;
  if (n > 0) load(0, cur);
  for (int c0 = 0; c0 < n; c0 += 32) {
    // stage this chunk's V rows (the wave's own LDS; its reads of the last
    // chunk were issued before these writes, and LDS runs a wave's accesses in order)
#pragma unroll
    for (int cc = 0; cc < 8; ++cc)
      *(lds_u32x4_t*)(uintptr_t)(svb + (l >> 1) * TG_VSTRIDE + 128 * (l & 1) + 16 * cc) = cur.vx[cc];
    if (c0 + 32 < n) load(c0 + 32, nxt);
    // ---- scores: S^T[16 kb + 4 g + i][t]
    f32x4 sc[2];
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk) {
      sc[kbk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < 4; ++ds)
        sc[kbk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.kf[kbk][ds]),
                                                           __builtin_bit_cast(bf16x8, qf[ds]), sc[kbk], 0, 0, 0);
    }
    // validity of the keys this lane's scores cover: key 16 kb + 4 g + i was
    // loaded by lane 4 g + i (group 0)
    float mx = -INFINITY;
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk) {
      const uint32_t okb = (uint32_t)__builtin_amdgcn_ballot_w64(cur.kval[kbk]) & 0xFFFFu;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const bool ok = (okb >> (4 * g + ii)) & 1u;
        sc[kbk][ii] = ok ? sc[kbk][ii] : -INFINITY;
        mx = fmaxf(mx, sc[kbk][ii]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * scale2;
    const bool grow = mx > m_run + 8.0f;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float mnew = grow ? mx : m_run;
      const float f = grow ? __builtin_amdgcn_exp2f(m_run - mnew) : 1.0f;   // m_run = -inf gives 0
      l_run *= f;
#pragma unroll
      for (int db = 0; db < 8; ++db) acc[db] *= f;
      m_run = mnew;
    }
    const float muse = (m_run == -INFINITY) ? 0.f : m_run;
    uint32_t pk[4];
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
      for (int ii = 0; ii < 4; ii += 2) {
        const uint32_t pb = pack_bf16x2(__builtin_amdgcn_exp2f(__builtin_fmaf(sc[kbk][ii], scale2, -muse)),
                                        __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kbk][ii + 1], scale2, -muse)));
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pb), ones, l_run, false);
        pk[2 * kbk + ii / 2] = pb;
      }
    const u32x4 bx = {pk[0], pk[1], pk[2], pk[3]};
    const bf16x8 pop = __builtin_bit_cast(bf16x8, bx);
    // ---- O^T += V^T P^T: rows 4 g + t / 4 (keys 0..15) and 16 + 4 g + t / 4,
    // four dims 16 db + 4 (t % 4) .. + 3 each
    const uint32_t va = svb + (4 * g + (t >> 2)) * TG_VSTRIDE + 8 * (t & 3);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const short4_t ya = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(uintptr_t)(va + 32 * db));
      const short4_t yb =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(uintptr_t)(va + 16 * TG_VSTRIDE + 32 * db));
      const short8_t ab = {ya[0], ya[1], ya[2], ya[3], yb[0], yb[1], yb[2], yb[3]};
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ab), pop, acc[db], 0, 0, 0);
    }
    cur = nxt;
  }
  // ---- epilogue: head t's sum over the four lane groups; O = acc / l
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (!hok) return;
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  const size_t obase = (((size_t)b * H + h0 + t) * Nq + i) * 128;
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    const int d = 16 * db + 4 * g;
    const f32x4 ov = acc[db] * inv;
    if (out_f32) {
      *(f32x4*)((float*)o + obase + d) = ov;
    } else {
      u32x2 bv = {pack_bf16x2(ov[0], ov[1]), pack_bf16x2(ov[2], ov[3])};
      *(u32x2*)((uint16_t*)o + obase + d) = bv;
    }
  }
  if (g == 0 && lse)
    lse[((size_t)b * H + h0 + t) * Nq + i] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
}

struct IdxLayout {
  size_t off_scores, off_kbar, off_r, off_route, off_cand, off_ccnt, off_resc, total;
};
IdxLayout idx_layout(int Nq, int Nk, int Hi, int R, int cand) {
  IdxLayout L;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t off = 0;
  L.off_scores = off; off = al(off + (size_t)Nq * Nk * 4);
  L.off_kbar = off; off = al(off + (size_t)((Nk + 15) / 16) * 128 * 2);   // router blocks of 16 keys or more
  L.off_r = off; off = al(off + (size_t)Nq * Hi * 4);
  L.off_route = off; off = al(off + (size_t)Nq * std::max(R, 1) * 4);
  L.off_cand = off; off = al(off + (size_t)Nq * cand * 4);
  L.off_ccnt = off; off = al(off + (size_t)(cand > 0 ? Nq : 0) * 4);
  L.off_resc = off; off = al(off + (size_t)Nq * cand * 4);
  L.total = off;
  return L;
}

}  // namespace

size_t indexer_workspace_bytes(int Nq, int Nk, int Hi, int route_heads, int cand) {
  return idx_layout(Nq, Nk, Hi, route_heads, cand).total;
}

hipError_t launch_indexer(const IndexerArgs& a, void* ws, hipStream_t st) {
  if (a.route_heads > 8 || (a.cand > 0 && a.route_heads < 1)) return hipErrorNotSupported;
  IdxLayout L = idx_layout(a.Nq, a.Nk, a.Hi, a.route_heads, a.cand);
  char* base = (char*)ws;
  float* scores = (float*)(base + L.off_scores);
  QkArgs q;
  q.q_idx = a.q_idx;
  q.w = a.w;
  q.Nq = a.Nq; q.Nk = a.Nk; q.Hi = a.Hi; q.q_offset = a.q_offset;
  q.block = a.route_block;
  if (a.route_heads > 0) {
    // router: block means of the indexer keys, head scores, top-R heads
    uint16_t* kbar = (uint16_t*)(base + L.off_kbar);
    float* r = (float*)(base + L.off_r);
    int32_t* route = (int32_t*)(base + L.off_route);
    HeadList one;
    one.n = 1;
    one.h[0] = 0;
    hipError_t e = launch_pool(a.k_idx, 1, 1, a.Nk, one, a.route_block, kbar, st);
    if (e != hipSuccess) return e;
    q.keys = kbar;
    q.nkeys = (a.Nk + a.route_block - 1) / a.route_block;
    q.out = r;
    q.route = nullptr;
    q.R = 0;
    hipLaunchKernelGGL(qk_heads_kernel<MODE_ROUTER>, dim3((a.Nq + NW - 1) / NW), dim3(NTI), 0, st, q);
    hipLaunchKernelGGL(router_select_kernel, dim3((a.Nq + 3) / 4), dim3(256), 0, st, r, a.Nq, a.Hi, a.route_heads,
                       route, a.route);
    q.keys = a.k_idx;
    q.nkeys = a.Nk;
    q.out = scores;
    q.route = route;
    q.R = a.route_heads;
    hipLaunchKernelGGL(qk_heads_kernel<MODE_ROUTED>, dim3((a.Nq + 4 * NW - 1) / (4 * NW)), dim3(NTI), 0, st, q);
  } else {
    q.keys = a.k_idx;
    q.nkeys = a.Nk;
    q.out = scores;
    q.route = nullptr;
    q.R = 0;
    hipLaunchKernelGGL(qk_heads_kernel<MODE_DENSE>, dim3((a.Nq + NW - 1) / NW), dim3(NTI), 0, st, q);
  }
  if (a.cand > 0) {
    // hierarchical: routed top-cand candidates, rescored by every head, top-k of them
    int32_t* cidx = a.cand_idx ? a.cand_idx : (int32_t*)(base + L.off_cand);
    int32_t* ccnt = a.cand_count ? a.cand_count : (int32_t*)(base + L.off_ccnt);
    const int ccap = a.cand_idx ? a.cand_cap : a.cand;
    float* resc = (float*)(base + L.off_resc);
    hipLaunchKernelGGL(token_select_kernel, dim3(a.Nq), dim3(TS_THREADS), 0, st, scores, a.Nq, a.Nk, a.q_offset, a.cand,
                       cidx, ccnt, ccap);
    hipLaunchKernelGGL(cand_score_kernel, dim3((a.Nq + CS_WAVES - 1) / CS_WAVES), dim3(CS_WAVES * 64), 0, st, a.q_idx,
                       a.k_idx, a.w, cidx, ccnt, a.Nq, a.Hi, ccap, a.cand, resc);
    hipLaunchKernelGGL(cand_select_kernel, dim3(a.Nq), dim3(TS_THREADS), 0, st, resc, a.cand, cidx, ccnt, ccap, a.topk,
                       a.tok, a.tok_count, a.tok_cap);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(token_select_kernel, dim3(a.Nq), dim3(TS_THREADS), 0, st, scores, a.Nq, a.Nk, a.q_offset, a.topk, a.tok,
                     a.tok_count, a.tok_cap);
  return hipGetLastError();
}

hipError_t launch_token_attention(const AttnArgs& a, hipStream_t st) {
  if (a.tcap > TA_MAXTOK) return hipErrorNotSupported;
  HeadList th;
  th.n = 0;
  for (int h = 0; h < a.H; ++h)
    if (a.kind[h] == 3) th.h[th.n++] = h;
  if (th.n == 0) return hipSuccess;
  const int rep = a.H / a.Hkv;
  if (rep >= 8) {
    // runs of consecutive token heads of one KV head, at most 16 per group
    TokenGroups tg;
    tg.n = 0;
    for (int x = 0; x < th.n && tg.n <= TG_MAXGROUPS; ++x) {
      const int h = th.h[x];
      const bool extend = tg.n > 0 && h == tg.h0[tg.n - 1] + tg.cnt[tg.n - 1] && h / rep == tg.h0[tg.n - 1] / rep &&
                          tg.cnt[tg.n - 1] < 16;
      if (extend) {
        ++tg.cnt[tg.n - 1];
      } else if (tg.n < TG_MAXGROUPS) {
        tg.h0[tg.n] = h;
        tg.cnt[tg.n] = 1;
        ++tg.n;
      } else {
        tg.n = TG_MAXGROUPS + 1;                         // too many groups: per-head kernel below
      }
    }
    if (tg.n <= TG_MAXGROUPS) {
      hipLaunchKernelGGL(token_attn_group_kernel, dim3((unsigned)((a.B * a.Nq + TG_WAVES - 1) / TG_WAVES), tg.n),
                         dim3(TG_WAVES * 64), 0, st, a.q, a.k, a.v, a.H, a.Hkv, a.Nq, a.Nk, a.B, a.tidx, a.tcount,
                         a.tcap, a.o, a.lse, a.out_f32, tg);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL(token_attn_kernel, dim3((unsigned)((size_t)th.n * a.B * a.Nq)), dim3(TA_THREADS), 0, st, a.q,
                     a.k, a.v, a.H, a.Hkv, a.Nq, a.Nk, a.tidx, a.tcount, a.tcap, a.o, a.lse, a.out_f32, a.B, th);
  return hipGetLastError();
}

}  // namespace dsa
