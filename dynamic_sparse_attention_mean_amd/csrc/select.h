// Sort-free selection inside one workgroup (gfx950, wave64).
//
// Top-k: radix select of the k-th largest order-preserving 32-bit key (four
// 8-bit digits, MSB first, histograms in LDS), then one compaction pass that
// keeps every key above it and the lowest-indexed keys equal to it, written in
// ascending index order.  Threshold: one max-reduce, then the same compaction
// with the cut max + log_alpha.  Both follow the selection rules of "FlashPrefill"
// section 2.2 (threshold relative to the row maximum, no sort) and the top-k of
// MoBA's FlashMoBA section, with ties to the lower index.
#pragma once
#include "common.h"

namespace dsa {

template <int NTH>
struct SelectSmem {
  uint32_t hist[256];
  uint32_t wv[NTH / 64][2];
  uint32_t scal[4];
  float fmax[NTH / 64];
};

// Candidates: j in [lo, hi) except ex0 and ex1 (-1 for none).
template <int NTH>
__device__ __forceinline__ bool sel_is_cand(int j, int ex0, int ex1) { return j != ex0 && j != ex1; }

// Writes the selected indices (ascending) to out[0..count) and returns count
// (uniform across the workgroup).  k <= 0 selects nothing.
template <int NTH>
__device__ int select_topk(const float* __restrict__ sc, int lo, int hi, int ex0, int ex1, int k,
                           int32_t* __restrict__ out, SelectSmem<NTH>& sm) {
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  constexpr int NW = NTH / 64;
  int nex = (ex0 >= lo && ex0 < hi) + (ex1 >= lo && ex1 < hi && ex1 != ex0);
  const int ncand = hi - lo - nex;
  if (k <= 0 || ncand <= 0) return 0;

  uint32_t T = 0u;         // keys > T all selected, == T lowest-index first
  int need_eq = 0;
  bool take_all = k >= ncand;
  if (!take_all) {
    uint32_t prefix = 0u, pmask = 0u;
    int kk = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += NTH) sm.hist[i] = 0u;
      __syncthreads();
      for (int j = lo + tid; j < hi; j += NTH) {
        if (!sel_is_cand<NTH>(j, ex0, ex1)) continue;
        const uint32_t key = f32_order_key(sc[j]);
        if ((key & pmask) == prefix) atomicAdd(&sm.hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (w == 0) {
        // lane l owns bins 255-4l .. 252-4l (descending digit order)
        uint32_t c[4];
        uint32_t s = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) { c[i] = sm.hist[255 - 4 * l - i]; s += c[i]; }
        const uint32_t incl = wave_incl_scan(s);
        const uint32_t excl = incl - s;
        // the lane where the cumulative count first reaches kk
        const bool hit = excl < (uint32_t)kk && incl >= (uint32_t)kk;
        if (hit) {
          uint32_t run = excl;
          for (int i = 0; i < 4; ++i) {
            if (run + c[i] >= (uint32_t)kk) {
              sm.scal[0] = 255u - 4u * l - i;
              sm.scal[1] = run;
              break;
            }
            run += c[i];
          }
        }
      }
      __syncthreads();
      const uint32_t dgt = sm.scal[0];
      kk -= (int)sm.scal[1];
      prefix |= dgt << shift;
      pmask |= 255u << shift;
      __syncthreads();
    }
    T = prefix;
    need_eq = kk;
  }

  // compaction: wave w owns the contiguous segment [s0, s1)
  const int n = hi - lo;
  const int seg = (n + NW - 1) / NW;
  const int s0 = lo + min(n, w * seg), s1 = lo + min(n, (w + 1) * seg);
  uint32_t gt = 0u, eq = 0u;
  for (int j0 = s0; j0 < s1; j0 += 64) {
    const int j = j0 + l;
    bool g = false, e = false;
    if (j < s1 && sel_is_cand<NTH>(j, ex0, ex1)) {
      if (take_all) g = true;
      else {
        const uint32_t key = f32_order_key(sc[j]);
        g = key > T;
        e = key == T;
      }
    }
    gt += __popcll(__builtin_amdgcn_ballot_w64(g));
    eq += __popcll(__builtin_amdgcn_ballot_w64(e));
  }
  if (l == 0) { sm.wv[w][0] = gt; sm.wv[w][1] = eq; }
  __syncthreads();
  uint32_t out_pos = 0u, eq_before = 0u;
  for (int i = 0; i < w; ++i) {
    const uint32_t g2 = sm.wv[i][0], e2 = sm.wv[i][1];
    const int rem = need_eq - (int)eq_before;
    out_pos += g2 + (uint32_t)max(0, min(rem, (int)e2));
    eq_before += e2;
  }
  for (int j0 = s0; j0 < s1; j0 += 64) {
    const int j = j0 + l;
    bool g = false, e = false;
    if (j < s1 && sel_is_cand<NTH>(j, ex0, ex1)) {
      if (take_all) g = true;
      else {
        const uint32_t key = f32_order_key(sc[j]);
        g = key > T;
        e = key == T;
      }
    }
    const uint64_t be = __builtin_amdgcn_ballot_w64(e);
    const bool take = g || (e && (int)(eq_before + ballot_rank(be)) < need_eq);
    const uint64_t bs = __builtin_amdgcn_ballot_w64(take);
    if (take) out[out_pos + ballot_rank(bs)] = j;
    out_pos += __popcll(bs);
    eq_before += __popcll(be);
  }
  __syncthreads();
  return take_all ? ncand : k;
}

// Threshold selection over all of [lo, hi): keep sc[j] >= max + log_alpha.
// Returns the count; writes ascending indices to out.  Also reports whether
// index `probe0` and `probe1` were kept (for merging forced entries).
template <int NTH>
__device__ int select_threshold(const float* __restrict__ sc, int lo, int hi, float log_alpha,
                                int32_t* __restrict__ out, int out_shift, SelectSmem<NTH>& sm,
                                float* cut_out) {
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  constexpr int NW = NTH / 64;
  if (hi <= lo) return 0;
  float mx = -INFINITY;
  for (int j = lo + tid; j < hi; j += NTH) mx = fmaxf(mx, sc[j]);
  mx = wave_max(mx);
  if (l == 0) sm.fmax[w] = mx;
  __syncthreads();
  mx = sm.fmax[0];
  for (int i = 1; i < NW; ++i) mx = fmaxf(mx, sm.fmax[i]);
  const float cut = mx + log_alpha;
  if (cut_out) *cut_out = cut;
  const int n = hi - lo;
  const int seg = (n + NW - 1) / NW;
  const int s0 = lo + min(n, w * seg), s1 = lo + min(n, (w + 1) * seg);
  uint32_t cnt = 0u;
  for (int j0 = s0; j0 < s1; j0 += 64) {
    const int j = j0 + l;
    const bool g = j < s1 && sc[j] >= cut;
    cnt += __popcll(__builtin_amdgcn_ballot_w64(g));
  }
  __syncthreads();
  if (l == 0) sm.wv[w][0] = cnt;
  __syncthreads();
  uint32_t pos = (uint32_t)out_shift;
  for (int i = 0; i < w; ++i) pos += sm.wv[i][0];
  uint32_t total = 0u;
  for (int i = 0; i < NW; ++i) total += sm.wv[i][0];
  for (int j0 = s0; j0 < s1; j0 += 64) {
    const int j = j0 + l;
    const bool g = j < s1 && sc[j] >= cut;
    const uint64_t b = __builtin_amdgcn_ballot_w64(g);
    if (g) out[pos + ballot_rank(b)] = j;
    pos += __popcll(b);
  }
  __syncthreads();
  return (int)total;
}


// Top-k over a long row in three passes (rows of 10^4 - 10^6 keys):
//   1. histogram of the top 12 bits of the order-preserving key (4096 bins);
//      the bin b holding the k-th largest key follows from a suffix scan;
//   2. the keys of bin b go to LDS (key, index) and each wave counts, over its
//      own contiguous segment, the keys above bin b;
//   3. an LDS radix select on the low 20 bits of the candidates gives the exact
//      k-th key T and how many keys equal to T are taken (lowest index first);
//      the last pass writes every key > T and those keys == T in index order.
// If bin b holds more candidates than LDS has room for, the row falls back to
// the digit-by-digit select_topk.  Candidates are [0, n); returns the count
// (uniform across the workgroup), writes ascending indices to out.  A row that
// starts on a 16-byte boundary is read four keys per lane (one dwordx4 load);
// pass 3 then orders a lane's four keys after the lanes before it with wave
// prefix sums.
constexpr int kSel3Cap = 6144;     // candidates of the threshold bin kept in LDS

// Keys j .. j + 3 of the row (those below `end`); a lane's four keys come
// from one 16-byte load when all four are in range.
__device__ __forceinline__ void sel_load4(const float* __restrict__ sc, int j, int end, uint32_t (&key)[4],
                                          bool (&ok)[4]) {
  if (j + 3 < end) {
    const f32x4 x = *(const f32x4*)(sc + j);
#pragma unroll
    for (int e = 0; e < 4; ++e) { key[e] = f32_order_key(x[e]); ok[e] = true; }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ok[e] = j + e < end;
      key[e] = ok[e] ? f32_order_key(sc[j + e]) : 0u;
    }
  }
}

// Loads per lane a wave keeps in flight in the streaming passes.
constexpr int kSelU = 4;

// The kSelU 256-key chunks of a wave from jg on: whole chunks (all below
// `end`) by one 16-byte load per lane, all issued before any is used; a
// partial chunk is read key by key in sel_keys.
__device__ __forceinline__ void sel_load_group(const float* __restrict__ sc, int jg, int end, int l,
                                               f32x4 (&raw)[kSelU]) {
#pragma unroll
  for (int u = 0; u < kSelU; ++u) {
    const int j0 = jg + 256 * u;
    raw[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (j0 + 256 <= end) raw[u] = *(const f32x4*)(sc + j0 + 4 * l);
  }
}

// Order keys of this lane's four keys j .. j + 3 of the chunk at j0.
__device__ __forceinline__ void sel_keys(const f32x4& raw, const float* __restrict__ sc, int j0, int j, int end,
                                         uint32_t (&key)[4], bool (&ok)[4]) {
  if (j0 + 256 <= end) {
#pragma unroll
    for (int e = 0; e < 4; ++e) { key[e] = f32_order_key(raw[e]); ok[e] = true; }
  } else {
    sel_load4(sc, j, end, key, ok);
  }
}

template <int NTH>
struct Select3Smem {
  union {
    struct {
      uint32_t hist[4096];
      uint32_t ckey[kSel3Cap];
      int32_t cidx[kSel3Cap];
      uint32_t wgt[NTH / 64], weq[NTH / 64];
      uint32_t scal[8];
    } t;
    SelectSmem<NTH> r;
  };
};

template <int NTH>
__device__ __forceinline__ int select_topk_3pass(const float* __restrict__ sc, int n, int k, int32_t* __restrict__ out,
                                 Select3Smem<NTH>& sm) {
  constexpr int NW = NTH / 64;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  if (k <= 0 || n <= 0) return 0;
  if (k >= n) {                                     // every candidate
    for (int j = tid; j < n; j += NTH) out[j] = j;
    return n;
  }
  const bool vec = ((uintptr_t)sc & 15u) == 0;
  // ---- pass 1: 12-bit histogram
  for (int i = tid; i < 4096; i += NTH) sm.t.hist[i] = 0u;
  __syncthreads();
  if (vec) {
    // kSelU loads per lane are issued before any is used: one load in flight
    // per lane leaves a pass bound by memory latency, not bandwidth
    const int n4 = n >> 2;
    int j4 = tid;
    for (; j4 + (kSelU - 1) * NTH < n4; j4 += kSelU * NTH) {
      f32x4 x[kSelU];
#pragma unroll
      for (int u = 0; u < kSelU; ++u) x[u] = *(const f32x4*)(sc + 4 * (j4 + u * NTH));
#pragma unroll
      for (int u = 0; u < kSelU; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) atomicAdd(&sm.t.hist[f32_order_key(x[u][e]) >> 20], 1u);
    }
    for (; j4 < n4; j4 += NTH) {
      const f32x4 x = *(const f32x4*)(sc + 4 * j4);
#pragma unroll
      for (int e = 0; e < 4; ++e) atomicAdd(&sm.t.hist[f32_order_key(x[e]) >> 20], 1u);
    }
    for (int j = 4 * n4 + tid; j < n; j += NTH) atomicAdd(&sm.t.hist[f32_order_key(sc[j]) >> 20], 1u);
  } else {
    for (int j = tid; j < n; j += NTH) atomicAdd(&sm.t.hist[f32_order_key(sc[j]) >> 20], 1u);
  }
  __syncthreads();
  if (w == 0) {
    // lane l owns bins 4095 - 64 l .. 4032 - 64 l (descending)
    uint32_t s = 0u;
    for (int i = 0; i < 64; ++i) s += sm.t.hist[4095 - 64 * l - i];
    const uint32_t incl = wave_incl_scan(s);
    const uint32_t excl = incl - s;
    if (excl < (uint32_t)k && incl >= (uint32_t)k) {
      uint32_t run = excl;
      for (int i = 0; i < 64; ++i) {
        const uint32_t c = sm.t.hist[4095 - 64 * l - i];
        if (run + c >= (uint32_t)k) {
          sm.t.scal[0] = 4095u - 64u * l - i;   // threshold bin
          sm.t.scal[1] = run;                   // keys above it
          sm.t.scal[2] = c;                     // keys in it
          break;
        }
        run += c;
      }
    }
  }
  __syncthreads();
  const uint32_t bin = sm.t.scal[0], above = sm.t.scal[1], inbin = sm.t.scal[2];
  if (inbin > (uint32_t)kSel3Cap) {
    __syncthreads();                                // the storage is reused below
    return select_topk<NTH>(sc, 0, n, -1, -1, k, out, sm.r);
  }
  // ---- pass 2: candidates of the threshold bin; keys above it per wave segment
  // (segments start on multiples of 4, so a segment's dwordx4 loads stay aligned)
  const int seg = vec ? (((n + NW - 1) / NW + 3) & ~3) : (n + NW - 1) / NW;
  const int s0 = min(n, w * seg), s1 = min(n, (w + 1) * seg);
  if (tid == 0) sm.t.scal[3] = 0u;
  __syncthreads();
  uint32_t gt = 0u;
  if (vec) {
    uint32_t gl = 0u;
    for (int jg = s0; jg < s1; jg += 256 * kSelU) {
      f32x4 raw[kSelU];
      sel_load_group(sc, jg, s1, l, raw);
#pragma unroll
      for (int u = 0; u < kSelU; ++u) {
        const int j0 = jg + 256 * u;
        if (j0 >= s1) break;
        const int j = j0 + 4 * l;
        uint32_t key[4];
        bool ok[4];
        sel_keys(raw[u], sc, j0, j, s1, key, ok);
        uint32_t nc = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          gl += (ok[e] && (key[e] >> 20) > bin) ? 1u : 0u;
          nc += (ok[e] && (key[e] >> 20) == bin) ? 1u : 0u;
        }
        const uint32_t incl = wave_incl_scan(nc);
        const uint32_t tot = __shfl(incl, 63, 64);
        if (tot) {
          uint32_t base = 0u;
          if (l == 0) base = atomicAdd(&sm.t.scal[3], tot);
          base = __shfl(base, 0, 64);
          uint32_t pos = base + incl - nc;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (ok[e] && (key[e] >> 20) == bin) {
              sm.t.ckey[pos] = key[e];
              sm.t.cidx[pos] = j + e;
              ++pos;
            }
        }
      }
    }
    gt = wave_sum_u32(gl);
  } else
  for (int j0 = s0; j0 < s1; j0 += 64) {
    const int j = j0 + l;
    uint32_t key = 0u;
    bool g = false, c = false;
    if (j < s1) {
      key = f32_order_key(sc[j]);
      g = (key >> 20) > bin;
      c = (key >> 20) == bin;
    }
    gt += __popcll(__builtin_amdgcn_ballot_w64(g));
    const uint64_t bc = __builtin_amdgcn_ballot_w64(c);
    if (bc) {
      uint32_t base = 0u;
      if (l == 0) base = atomicAdd(&sm.t.scal[3], (uint32_t)__popcll(bc));
      base = __shfl(base, 0, 64);
      if (c) {
        const uint32_t pos = base + ballot_rank(bc);
        sm.t.ckey[pos] = key;
        sm.t.cidx[pos] = j;
      }
    }
  }
  __syncthreads();
  // ---- exact threshold among the candidates: radix select on the low 20 bits
  const int nc = (int)inbin;
  uint32_t prefix = bin << 20, pmask = 0xFFF00000u;
  int need = k - (int)above;                        // 1 <= need <= nc
  for (int dg = 0; dg < 3; ++dg) {
    const int sh = dg == 0 ? 12 : (dg == 1 ? 4 : 0);   // digits: bits 19-12, 11-4, 3-0
    const uint32_t dmask = dg == 2 ? 15u : 255u;
    for (int i = tid; i < 256; i += NTH) sm.t.hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < nc; i += NTH) {
      const uint32_t key = sm.t.ckey[i];
      if ((key & pmask) == prefix) atomicAdd(&sm.t.hist[(key >> sh) & dmask], 1u);
    }
    __syncthreads();
    if (w == 0) {
      // lane l owns digits dmask - 4l .. dmask - 4l - 3 (descending); the lane
      // whose range holds the need-th key names the digit and the count above it
      uint32_t c[4];
      uint32_t s = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = (int)dmask - 4 * l - i;
        c[i] = d >= 0 ? sm.t.hist[d] : 0u;
        s += c[i];
      }
      const uint32_t incl = wave_incl_scan(s);
      const uint32_t excl = incl - s;
      if (excl < (uint32_t)need && incl >= (uint32_t)need) {
        uint32_t run = excl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (run + c[i] >= (uint32_t)need) {
            sm.t.scal[4] = (uint32_t)((int)dmask - 4 * l - i);
            sm.t.scal[5] = run;
            break;
          }
          run += c[i];
        }
      }
    }
    __syncthreads();
    prefix |= sm.t.scal[4] << sh;
    pmask |= dmask << sh;
    need -= (int)sm.t.scal[5];
    __syncthreads();
  }
  const uint32_t T = prefix;
  const int need_eq = need;
  // per-segment counts of candidates above T / equal to T
  if (l == 0) { sm.t.wgt[w] = gt; sm.t.weq[w] = 0u; }
  __syncthreads();
  for (int i = tid; i < nc; i += NTH) {
    const uint32_t key = sm.t.ckey[i];
    const int sgi = sm.t.cidx[i] / seg;
    if (key > T) atomicAdd(&sm.t.wgt[sgi], 1u);
    else if (key == T) atomicAdd(&sm.t.weq[sgi], 1u);
  }
  __syncthreads();
  uint32_t out_pos = 0u, eq_before = 0u;
  for (int i = 0; i < w; ++i) {
    const uint32_t g2 = sm.t.wgt[i], e2 = sm.t.weq[i];
    out_pos += g2 + (uint32_t)max(0, min(need_eq - (int)eq_before, (int)e2));
    eq_before += e2;
  }
  // ---- pass 3: write the selected keys of this wave's segment in index order
  if (vec) {
    for (int jg = s0; jg < s1; jg += 256 * kSelU) {
      f32x4 raw[kSelU];
      sel_load_group(sc, jg, s1, l, raw);
#pragma unroll
      for (int u = 0; u < kSelU; ++u) {
        const int j0 = jg + 256 * u;
        if (j0 >= s1) break;
        const int j = j0 + 4 * l;
        uint32_t key[4];
        bool ok[4];
        sel_keys(raw[u], sc, j0, j, s1, key, ok);
        uint32_t ne = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) ne += (ok[e] && key[e] == T) ? 1u : 0u;
        const uint32_t e_incl = wave_incl_scan(ne);
        const uint32_t e_tot = __shfl(e_incl, 63, 64);
        uint32_t erank = eq_before + e_incl - ne;      // keys == T before this lane's first
        bool take[4];
        uint32_t nt = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool g = ok[e] && key[e] > T;
          const bool q = ok[e] && key[e] == T;
          take[e] = g || (q && (int)erank < need_eq);
          erank += q ? 1u : 0u;
          nt += take[e] ? 1u : 0u;
        }
        const uint32_t t_incl = wave_incl_scan(nt);
        const uint32_t t_tot = __shfl(t_incl, 63, 64);
        uint32_t opos = out_pos + t_incl - nt;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (take[e]) out[opos++] = j + e;
        out_pos += t_tot;
        eq_before += e_tot;
      }
    }
  } else
  for (int j0 = s0; j0 < s1; j0 += 64) {
    const int j = j0 + l;
    bool g = false, e = false;
    if (j < s1) {
      const uint32_t key = f32_order_key(sc[j]);
      g = key > T;
      e = key == T;
    }
    const uint64_t be = __builtin_amdgcn_ballot_w64(e);
    const bool take = g || (e && (int)(eq_before + ballot_rank(be)) < need_eq);
    const uint64_t bs = __builtin_amdgcn_ballot_w64(take);
    if (take) out[out_pos + ballot_rank(bs)] = j;
    out_pos += __popcll(bs);
    eq_before += __popcll(be);
  }
  __syncthreads();
  return k;
}

}  // namespace dsa
