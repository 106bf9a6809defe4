// Sparse prefill attention over per-head index sets (gfx950).
//
// What it computes: for each head h and query row i,
//   O[i] = sum_{j in M_h(i)} softmax_j(q_i . k_j / sqrt(d)) v_j,  LSE[i] = log sum exp,
// with M_h(i) given by the head's pattern and index set ("MInference 1.0"
// explainer, GPU kernels section; authors' abstract: sparse kernels over
// pattern + indices).  Following "FlashPrefill" section 2.3, the kernel walks
// compact lists of key tiles (index-driven jumps) rather than testing every tile.
//
// Design (MI355X):
//  * one work item = (batch, head, 64-query tile); workgroup = 2 waves, each wave
//    owns 32 query rows and computes S^T = K Q^T and O^T += V^T P^T with
//    v_mfma_f32_32x32x16_bf16 (fp32 accumulate).  Using S^T makes the MFMA output
//    of P^T usable directly as the B operand of the PV product (no shuffle).
//  * K tiles (64 keys) are staged in LDS with a 16-byte XOR swizzle; V tiles are
//    stored transposed (V^T, 8-byte XOR swizzle) so the PV A operand is two
//    8-byte LDS reads.  Global loads of tile n+1 are issued before tile n is
//    computed (register prefetch, single LDS buffer).
//  * online softmax in fp32 (base 2), P rounded to bf16 for the PV MFMA, lazy
//    rescaling of the accumulator only when the running max grows by > 8 (log2).
//  * Vertical-Slash heads: a compile step turns the column/diagonal lists into
//    bitmaps and the set A of key-tile offsets a touched by a selected diagonal.
//    Query tile t visits key tiles t - a (slash strips) with an exact per-element
//    mask (diagonal bit | column bit) and skips each 32x32 sub-block whose mask is
//    empty; columns outside those tiles are gathered 64 at a time.  Every (i, j)
//    is visited exactly once, so the set semantics (no double counting) hold.
//  * persistent workgroups pull items from per-XCD queues (t descending, so the
//    long causal rows start first) and steal from other queues when theirs is
//    empty; heads are packed into queues by estimated cost.
#include "common.h"
#include "internal.h"

#include <algorithm>
#include <vector>

namespace dsa {
namespace {

constexpr int TQ = 64;       // query rows per work item
constexpr int TK = 64;       // keys per tile
constexpr int NT = 128;      // threads per workgroup
constexpr int GCAP = 1024;   // gathered columns staged per round

enum { M_NONE = 0, M_CAUSAL = 1, M_VS = 2, M_GATHER = 3, M_EMPTY = 4 };

struct Sched {
  int nq;                       // number of queues
  int T;                        // query tiles per head
  int qstart[kMaxQueues + 1];   // heads of queue g: heads[qstart[g] .. qstart[g+1])
  int16_t heads[kMaxHeadTable]; // b * H + h
};

struct BhList {
  int n;
  int16_t bh[kMaxHeadTable];
};

// ------------------------------------------------------------------ bitmaps
__device__ __forceinline__ bool test_bit(const uint32_t* bm, int i) { return (bm[i >> 5] >> (i & 31)) & 1u; }

// any / all bits set in [lo, hi] (inclusive, 0 <= lo <= hi) of an unpadded bitmap
__device__ bool range_any(const uint32_t* bm, int lo, int hi) {
  for (int wd = lo >> 5; wd <= (hi >> 5); ++wd) {
    uint32_t m = ~0u;
    if (wd == (lo >> 5)) m &= ~0u << (lo & 31);
    if (wd == (hi >> 5)) m &= ~0u >> (31 - (hi & 31));
    if (bm[wd] & m) return true;
  }
  return false;
}
__device__ bool range_all(const uint32_t* bm, int lo, int hi) {
  for (int wd = lo >> 5; wd <= (hi >> 5); ++wd) {
    uint32_t m = ~0u;
    if (wd == (lo >> 5)) m &= ~0u << (lo & 31);
    if (wd == (hi >> 5)) m &= ~0u >> (31 - (hi & 31));
    if ((bm[wd] & m) != m) return false;
  }
  return true;
}

// Set the bits of the listed columns (vbits) and diagonals (sbits, stored with
// one leading pad word so that windows starting at negative offsets read 0).
__global__ void vs_setbits_kernel(AttnArgs a, BhList L) {
  const int hi = blockIdx.y;
  if (hi >= L.n) return;
  const int bh = L.bh[hi];
  const int nc = min(a.cols_count[bh], a.cols_cap), nd = min(a.diags_count[bh], a.diags_cap);
  const int32_t* cols = a.cols + (size_t)bh * a.cols_cap;
  const int32_t* diags = a.diags + (size_t)bh * a.diags_cap;
  uint32_t* vb = a.vbits + (size_t)bh * a.vw;
  uint32_t* sb = a.sbits + (size_t)bh * a.sw;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < nc + nd; i += gridDim.x * blockDim.x) {
    if (i < nc) {
      int j = cols[i];
      if (j >= 0 && j < a.Nk) atomicOr(&vb[j >> 5], 1u << (j & 31));
    } else {
      int o = diags[i - nc];
      if (o >= 0 && o < a.Nk) atomicOr(&sb[(o >> 5) + 1], 1u << (o & 31));
    }
  }
}

// Tile offsets a in [0, TA): a is in A iff a selected diagonal crosses some pair
// (query tile t, key tile t - a), i.e. offsets [64a - 63, 64a + 63] hold a set
// bit; a >= 1 is "full" (no mask needed) iff all of them are set.
__global__ __launch_bounds__(256) void vs_tiles_kernel(AttnArgs a, BhList L, int TA) {
  const int bh = L.bh[blockIdx.x];
  const uint32_t* sb = a.sbits + (size_t)bh * a.sw + 1;     // unpadded view
  uint32_t* ab = a.abits + (size_t)bh * a.aw;
  uint32_t* fb = a.fbits + (size_t)bh * a.aw;
  int32_t* al = a.alist + (size_t)bh * a.acap;
  __shared__ int s_wave[4];
  __shared__ int s_base;
  if (threadIdx.x == 0) s_base = 0;
  __syncthreads();
  const int w = threadIdx.x >> 6;
  for (int a0 = 0; a0 < TA; a0 += 256) {
    const int t = a0 + threadIdx.x;
    bool inA = false, full = false;
    if (t < TA) {
      const int lo = max(0, 64 * t - 63), hi = min(a.Nk - 1, 64 * t + 63);
      if (lo <= hi) {
        inA = range_any(sb, lo, hi);
        full = (t >= 1) && inA && range_all(sb, lo, hi);
      }
      if (inA) atomicOr(&ab[t >> 5], 1u << (t & 31));
      if (full) atomicOr(&fb[t >> 5], 1u << (t & 31));
    }
    const uint64_t bal = __builtin_amdgcn_ballot_w64(inA);
    const uint32_t rank = ballot_rank(bal);
    if ((threadIdx.x & 63) == 0) s_wave[w] = __popcll(bal);
    __syncthreads();
    int off = s_base;
    for (int i = 0; i < w; ++i) off += s_wave[i];
    if (inA) al[off + rank] = t;
    __syncthreads();
    if (threadIdx.x == 0) s_base += s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.acount[bh] = s_base;
}

// ---------------------------------------------------------------- main kernel
struct TileRegs {
  u32x4 k[8];
  u32x4 v[8];
};

struct Entry {
  int mode;    // M_*
  int kt;      // key tile (tiles) or gather chunk (M_GATHER)
  int cnt;     // valid keys in a gather chunk
};

__device__ __forceinline__ void load_tile(const uint16_t* __restrict__ kb, const uint16_t* __restrict__ vb,
                                          int Nk, const Entry& e, const int32_t* s_cols, TileRegs& r) {
  const int tid = threadIdx.x;
  const int c16 = tid & 15;
  const int r0 = tid >> 4;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  if (e.mode == M_EMPTY) return;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int rr = r0 + 8 * i;
    int key;
    bool ok;
    if (e.mode == M_GATHER) {
      ok = rr < e.cnt;
      key = ok ? s_cols[e.kt * TK + rr] : 0;
    } else {
      key = e.kt * TK + rr;
      ok = key < Nk;
    }
    r.k[i] = ok ? *(const u32x4*)(kb + (size_t)key * 128 + c16 * 8) : zero;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int kq = r0 + 8 * i;
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const int rr = 4 * kq + e4;
      int key;
      bool ok;
      if (e.mode == M_GATHER) {
        ok = rr < e.cnt;
        key = ok ? s_cols[e.kt * TK + rr] : 0;
      } else {
        key = e.kt * TK + rr;
        ok = key < Nk;
      }
      r.v[4 * i + e4] = ok ? *(const u32x4*)(vb + (size_t)key * 128 + c16 * 8) : zero;
    }
  }
}

__device__ __forceinline__ void store_tile(const TileRegs& r, uint16_t* s_k, uint16_t* s_v) {
  const int tid = threadIdx.x;
  const int c16 = tid & 15;
  const int r0 = tid >> 4;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int rr = r0 + 8 * i;
    *(u32x4*)(s_k + rr * 128 + ((c16 ^ (rr & 15)) * 8)) = r.k[i];
  }
  // V^T: row d (128 of them) holds 64 keys; this thread owns d = 8*c16 .. +7 and
  // key quads kq = r0, r0 + 8.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int kq = r0 + 8 * i;
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      const int d = 8 * c16 + dd;
      const int wsel = dd >> 1;
      uint32_t x0 = r.v[4 * i + 0][wsel], x1 = r.v[4 * i + 1][wsel];
      uint32_t x2 = r.v[4 * i + 2][wsel], x3 = r.v[4 * i + 3][wsel];
      uint32_t lo, hi;
      if (dd & 1) {
        lo = (x0 >> 16) | (x1 & 0xffff0000u);
        hi = (x2 >> 16) | (x3 & 0xffff0000u);
      } else {
        lo = (x0 & 0xffffu) | (x1 << 16);
        hi = (x2 & 0xffffu) | (x3 << 16);
      }
      u32x2 pk = {lo, hi};
      *(u32x2*)(s_v + d * TK + ((kq ^ (d & 15)) * 4)) = pk;
    }
  }
}

struct ItemCtx {
  int b, h, kvh, kind, t, P0, nrows, tq, last_pos;
  const int32_t* alist;   // VS
  int nstrip;
  const uint32_t* fbits;
  const uint32_t* sbits;  // padded
  const uint32_t* vbits;
  const int32_t* blist;   // BLOCK
  int nblk, per;
  int ngather;            // staged this round
  int nent;
};

__device__ __forceinline__ Entry entry_of(const ItemCtx& c, int n) {
  Entry e;
  e.cnt = 0;
  if (c.kind == 1) {                       // VS
    if (n < c.nstrip) {
      const int a = c.alist[n];
      e.kt = c.tq - a;
      e.mode = (a >= 1 && test_bit(c.fbits, a)) ? M_NONE : M_VS;
    } else {
      const int ch = n - c.nstrip;
      e.kt = ch;
      e.cnt = min(TK, c.ngather - ch * TK);
      e.mode = M_GATHER;
    }
  } else if (c.kind == 2) {                // BLOCK
    const int J = c.blist[n / c.per];
    e.kt = J * c.per + n % c.per;
    if (J < 0 || e.kt * TK > c.last_pos) e.mode = M_EMPTY;
    else e.mode = (e.kt * TK + TK - 1 > c.P0) ? M_CAUSAL : M_NONE;
  } else {                                 // DENSE
    e.kt = n;
    e.mode = (e.kt * TK + TK - 1 > c.P0) ? M_CAUSAL : M_NONE;
  }
  return e;
}

__global__ __launch_bounds__(NT) void attn_kernel(const AttnArgs a, const Sched sc) {
  __shared__ __align__(16) uint16_t s_k[TK * 128];
  __shared__ __align__(16) uint16_t s_v[128 * TK];
  __shared__ int32_t s_cols[GCAP];
  __shared__ int s_misc[4];

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  const int qn = l & 31;
  const int hh = l >> 5;
  const float scale2 = 1.4426950408889634f * 0.08838834764831845f;  // log2(e) / sqrt(128)
  const int rep = a.H / a.Hkv;
  const int myq = blockIdx.x % sc.nq;

  for (int qi = 0; qi < sc.nq; ++qi) {
    const int g = (myq + qi) % sc.nq;
    const int nh = sc.qstart[g + 1] - sc.qstart[g];
    const int nitems = nh * sc.T;
    if (nh == 0) continue;
    while (true) {
      __syncthreads();
      if (tid == 0) s_misc[0] = atomicAdd(&a.counters[g], 1);
      __syncthreads();
      const int it = s_misc[0];
      if (it >= nitems) break;

      ItemCtx c;
      const int bh = sc.heads[sc.qstart[g] + it % nh];
      c.b = bh / a.H;
      c.h = bh % a.H;
      c.kvh = c.h / rep;
      c.kind = a.kind[c.h];
      c.t = sc.T - 1 - it / nh;
      const int r0 = c.t * TQ;
      c.nrows = min(TQ, a.Nq - r0);
      c.P0 = r0 + a.q_offset;
      c.last_pos = c.P0 + c.nrows - 1;
      c.tq = c.P0 / TK;
      c.nstrip = 0;
      c.ngather = 0;
      c.per = 1;
      c.nblk = 0;

      const uint16_t* kbp = a.k + ((size_t)(c.b * a.Hkv + c.kvh) * a.Nk) * 128;
      const uint16_t* vbp = a.v + ((size_t)(c.b * a.Hkv + c.kvh) * a.Nk) * 128;
      const uint16_t* qbp = a.q + ((size_t)bh * a.Nq) * 128;

      // Q as the B operand of S^T = K Q^T: lane holds Q[row][16 ks + 8 hh .. +7].
      const int qrow = r0 + 32 * w + qn;
      const int iq = c.P0 + 32 * w + qn;          // absolute position of the lane's row
      const bool row_ok = qrow < a.Nq;
      bf16x8 qf[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (row_ok) x = *(const u32x4*)(qbp + (size_t)qrow * 128 + 16 * ks + 8 * hh);
        qf[ks] = __builtin_bit_cast(bf16x8, x);
      }

      f32x16 acc[4];
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[db][v] = 0.f;
      float m_run = -INFINITY, l_run = 0.f;

      int gcursor = 0;
      int gcount = 0;
      if (c.kind == 1) {
        c.alist = a.alist + (size_t)bh * a.acap;
        c.fbits = a.fbits + (size_t)bh * a.aw;
        c.sbits = a.sbits + (size_t)bh * a.sw;
        c.vbits = a.vbits + (size_t)bh * a.vw;
        // strips: alist ascending, keep a <= tq
        const int na = a.acount[bh];
        int lo = 0, hi = na;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (c.alist[mid] <= c.tq) lo = mid + 1; else hi = mid;
        }
        c.nstrip = lo;
        gcount = min(a.cols_count[bh], a.cols_cap);
      } else if (c.kind == 2) {
        const int I = c.P0 / a.block;
        c.blist = a.bidx + ((size_t)bh * a.nqb + I) * a.bcap;
        c.nblk = min(a.bcount[(size_t)bh * a.nqb + I], a.bcap);
        c.per = a.block / TK;
      }

      for (int round = 0;; ++round) {
        if (c.kind == 1) {
          // stage the next columns of this item: j <= last_pos outside strip tiles
          const int32_t* cols = a.cols + (size_t)bh * a.cols_cap;
          const uint32_t* ab = a.abits + (size_t)bh * a.aw;
          int staged = 0;
          while (gcursor < gcount && staged <= GCAP - NT) {
            const int idx = gcursor + tid;
            bool keep = false;
            if (idx < gcount) {
              const int j = cols[idx];
              keep = (j >= 0) && (j <= c.last_pos) && !test_bit(ab, c.tq - (j >> 6));
            }
            const uint64_t bal = __builtin_amdgcn_ballot_w64(keep);
            __syncthreads();
            if (l == 0) s_misc[1 + w] = __popcll(bal);
            __syncthreads();
            const int off = staged + (w ? s_misc[1] : 0);
            if (keep) s_cols[off + ballot_rank(bal)] = cols[idx];
            staged += s_misc[1] + s_misc[2];
            gcursor += NT;
            // columns are ascending: stop once past the item's last row
            const int lastc = cols[min(gcursor, gcount) - 1];
            if (lastc > c.last_pos) gcursor = gcount;
          }
          __syncthreads();
          c.ngather = staged;
          c.nent = (round == 0 ? c.nstrip : 0) + (staged + TK - 1) / TK;
          if (round > 0) c.nstrip = 0;
        } else if (c.kind == 2) {
          c.nent = c.nblk * c.per;
        } else {
          c.nent = c.last_pos / TK + 1;
        }

        TileRegs regs;
        Entry cur, nxt;
        if (c.nent > 0) {
          cur = entry_of(c, 0);
          load_tile(kbp, vbp, a.Nk, cur, s_cols, regs);
        }
        for (int n = 0; n < c.nent; ++n) {
          __syncthreads();
          if (cur.mode != M_EMPTY) store_tile(regs, s_k, s_v);
          __syncthreads();
          if (n + 1 < c.nent) {
            nxt = entry_of(c, n + 1);
            load_tile(kbp, vbp, a.Nk, nxt, s_cols, regs);
          }
          if (cur.mode != M_EMPTY) {
            // ---- masks of the two 32-key halves for this lane's row
            uint32_t M[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
              uint32_t m = ~0u;
              if (cur.mode == M_GATHER) {
                m = 0u;
                const int sbase = cur.kt * TK + 32 * kb + 4 * hh;
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                  for (int ii = 0; ii < 4; ++ii) {
                    const int slot = 32 * kb + 4 * hh + 8 * j + ii;
                    if (slot < cur.cnt && s_cols[sbase + 8 * j + ii] <= iq) m |= 1u << (8 * j + ii);
                  }
              } else if (cur.mode != M_NONE && row_ok) {
                const int kbase = cur.kt * TK + 32 * kb + 4 * hh;
                const int otop = iq - kbase;
                const uint32_t cm = otop < 0 ? 0u : (otop >= 31 ? ~0u : ((2u << otop) - 1u));
                if (cur.mode == M_CAUSAL) {
                  m = cm;
                } else {
                  uint32_t W = 0u;
                  if (otop >= 0) {
                    const int olo = otop - 31;
                    const int wi = (olo >> 5) + 1;
                    const uint64_t two = (uint64_t)c.sbits[wi] | ((uint64_t)c.sbits[wi + 1] << 32);
                    W = (uint32_t)(two >> (olo & 31));
                  }
                  const uint32_t vw = c.vbits[(cur.kt * TK + 32 * kb) >> 5] >> (4 * hh);
                  m = (__builtin_bitreverse32(W) | vw) & cm;
                }
              }
              if (!row_ok) m = 0u;
              M[kb] = m;
            }
            bool act[2];
            act[0] = __builtin_amdgcn_ballot_w64(M[0] != 0u) != 0;
            act[1] = __builtin_amdgcn_ballot_w64(M[1] != 0u) != 0;

            // ---- S^T = K Q^T for the active halves
            f32x16 sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
              for (int v = 0; v < 16; ++v) sacc[kb][v] = 0.f;
              if (act[kb]) {
                const int row = 32 * kb + qn;
#pragma unroll
                for (int ks = 0; ks < 8; ++ks) {
                  const u32x4 x = *(const u32x4*)(s_k + row * 128 + (((2 * ks + hh) ^ (row & 15)) * 8));
                  sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x), qf[ks],
                                                                     sacc[kb], 0, 0, 0);
                }
              }
            }
            // ---- mask + online softmax (base 2)
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
              if (!act[kb]) continue;
#pragma unroll
              for (int v = 0; v < 16; ++v) {
                const int s = 8 * (v >> 2) + (v & 3);
                float x = sacc[kb][v] * scale2;
                if (!((M[kb] >> s) & 1u)) x = -INFINITY;
                sacc[kb][v] = x;
                mx = fmaxf(mx, x);
              }
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const bool grow = mx > m_run + 8.0f;
            if (__builtin_amdgcn_ballot_w64(grow) != 0) {
              const float mnew = grow ? mx : m_run;
              const float f = grow ? __builtin_amdgcn_exp2f(m_run - mnew) : 1.0f;   // m_run = -inf gives 0
              l_run *= f;
#pragma unroll
              for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[db][v] *= f;
              m_run = mnew;
            }
            const float muse = (m_run == -INFINITY) ? 0.f : m_run;
            uint32_t pk[2][8];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
              if (!act[kb]) continue;
#pragma unroll
              for (int v = 0; v < 16; v += 2) {
                const float p0 = __builtin_amdgcn_exp2f(sacc[kb][v] - muse);
                const float p1 = __builtin_amdgcn_exp2f(sacc[kb][v + 1] - muse);
                // normalise with the same bf16-rounded weights the PV product uses
                const uint32_t pb = pack_bf16x2(p0, p1);
                l_run += bf16_lo(pb) + bf16_hi(pb);
                pk[kb][v >> 1] = pb;
              }
            }
            // ---- O^T += V^T P^T; key step ks2 covers keys 16 ks2 .. +15
#pragma unroll
            for (int ks2 = 0; ks2 < 4; ++ks2) {
              const int kb = ks2 >> 1;
              if (!act[kb]) continue;
              const int o8 = (ks2 & 1) * 4;
              u32x4 bx = {pk[kb][o8], pk[kb][o8 + 1], pk[kb][o8 + 2], pk[kb][o8 + 3]};
              const bf16x8 bop = __builtin_bit_cast(bf16x8, bx);
              const int ch0 = 4 * ks2 + hh, ch1 = 4 * ks2 + 2 + hh;
#pragma unroll
              for (int db = 0; db < 4; ++db) {
                const int d = 32 * db + qn;
                const u32x2 y0 = *(const u32x2*)(s_v + d * TK + ((ch0 ^ (d & 15)) * 4));
                const u32x2 y1 = *(const u32x2*)(s_v + d * TK + ((ch1 ^ (d & 15)) * 4));
                u32x4 ax = {y0[0], y0[1], y1[0], y1[1]};
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ax), bop, acc[db], 0, 0, 0);
              }
            }
          }
          cur = nxt;
        }
        if (!(c.kind == 1 && gcursor < gcount)) break;
      }

      // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2
      const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
      const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
      if (row_ok) {
        const size_t obase = ((size_t)bh * a.Nq + qrow) * 128;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int d = 32 * db + 8 * j + 4 * hh;
            const float o0 = acc[db][4 * j] * inv, o1 = acc[db][4 * j + 1] * inv;
            const float o2 = acc[db][4 * j + 2] * inv, o3 = acc[db][4 * j + 3] * inv;
            if (a.out_f32) {
              f32x4 ov = {o0, o1, o2, o3};
              *(f32x4*)((float*)a.o + obase + d) = ov;
            } else {
              u32x2 ov = {pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
              *(u32x2*)((uint16_t*)a.o + obase + d) = ov;
            }
          }
        if (hh == 0 && a.lse) {
          a.lse[(size_t)bh * a.Nq + qrow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
        }
      }
    }
  }
}

__global__ void zero_u32_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

int cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
  }
  return n;
}

struct VsLayout {
  int sw, vw, aw, acap, TA;
  size_t off_s, off_v, off_a, off_f, off_al, off_ac, off_ctr, total_words;
};

VsLayout vs_layout(int B, int H, int Nk) {
  VsLayout L;
  L.sw = (Nk + 31) / 32 + 3;
  L.vw = (Nk + 31) / 32 + 2;
  L.TA = (Nk + TK - 1) / TK + 1;
  L.aw = (L.TA + 31) / 32 + 1;
  L.acap = L.TA;
  const size_t nbh = (size_t)B * H;
  size_t off = 0;
  L.off_ctr = off; off += 64;
  L.off_s = off; off += nbh * L.sw;
  L.off_v = off; off += nbh * L.vw;
  L.off_a = off; off += nbh * L.aw;
  L.off_f = off; off += nbh * L.aw;
  L.off_ac = off; off += nbh;
  L.total_words = off;          // region zeroed before every call
  L.off_al = off; off += nbh * L.acap;
  (void)off;
  return L;
}

}  // namespace

size_t attn_workspace_bytes(int B, int H, int Nk) {
  VsLayout L = vs_layout(B, H, Nk);
  return (L.off_al + (size_t)B * H * L.acap) * 4 + 256;
}

hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  int blocks = (int)std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(zero_u32_kernel, dim3(blocks), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

hipError_t launch_attention(AttnArgs& a, void* ws, hipStream_t st) {
  const int T = (a.Nq + TQ - 1) / TQ;
  VsLayout L = vs_layout(a.B, a.H, a.Nk);
  uint32_t* base = (uint32_t*)ws;
  a.counters = (int32_t*)(base + L.off_ctr);
  a.sbits = base + L.off_s;
  a.vbits = base + L.off_v;
  a.abits = base + L.off_a;
  a.fbits = base + L.off_f;
  a.acount = (int32_t*)(base + L.off_ac);
  a.alist = (int32_t*)(base + L.off_al);
  a.sw = L.sw; a.vw = L.vw; a.aw = L.aw; a.acap = L.acap;

  hipError_t e = launch_zero_u32(base, L.total_words, st);
  if (e != hipSuccess) return e;

  // Vertical-Slash compile
  BhList vs;
  vs.n = 0;
  for (int b = 0; b < a.B; ++b)
    for (int h = 0; h < a.H; ++h)
      if (a.kind[h] == 1) vs.bh[vs.n++] = (int16_t)(b * a.H + h);
  if (vs.n > 0) {
    hipLaunchKernelGGL(vs_setbits_kernel, dim3(8, vs.n), dim3(256), 0, st, a, vs);
    hipLaunchKernelGGL(vs_tiles_kernel, dim3(vs.n), dim3(256), 0, st, a, vs, L.TA);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }

  // Queue assignment: estimate each head's cost (key tiles over all its query
  // tiles), longest first into the least-loaded queue.
  struct HC { double cost; int bh; };
  std::vector<HC> heads;
  for (int b = 0; b < a.B; ++b)
    for (int h = 0; h < a.H; ++h) {
      const int kd = a.kind[h];
      if (kd < 0 || kd > 2) continue;
      double per;
      if (kd == 0) per = 0.5 * (a.Nk / (double)TK);
      else if (kd == 2) per = std::min<double>(a.bcap * (a.block / TK), 0.5 * a.Nk / TK);
      else per = std::min<double>(0.5 * a.Nk / TK, 2.0 * a.diags_cap / TK + 1 + a.cols_cap / (double)TK);
      heads.push_back({per * T, b * a.H + h});
    }
  if (heads.empty()) return hipSuccess;
  std::stable_sort(heads.begin(), heads.end(), [](const HC& x, const HC& y) { return x.cost > y.cost; });
  Sched sc;
  sc.T = T;
  sc.nq = std::min<int>(kMaxQueues, (int)heads.size());
  std::vector<std::vector<int>> qh(sc.nq);
  std::vector<double> load(sc.nq, 0.0);
  for (const HC& x : heads) {
    int best = 0;
    for (int g = 1; g < sc.nq; ++g) if (load[g] < load[best]) best = g;
    load[best] += x.cost;
    qh[best].push_back(x.bh);
  }
  int pos = 0;
  for (int g = 0; g < sc.nq; ++g) {
    sc.qstart[g] = pos;
    std::sort(qh[g].begin(), qh[g].end());
    for (int bh : qh[g]) sc.heads[pos++] = (int16_t)bh;
  }
  sc.qstart[sc.nq] = pos;

  const long items = (long)heads.size() * T;
  long grid = std::min<long>(items, (long)cu_count() * 4);
  grid = std::max<long>(sc.nq, (grid / sc.nq) * sc.nq);
  hipLaunchKernelGGL(attn_kernel, dim3((unsigned)grid), dim3(NT), 0, st, a, sc);
  return hipGetLastError();
}

}  // namespace dsa
