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
// two leading pad words so that windows starting at negative offsets read 0).
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
      if (o >= 0 && o < a.Nk) atomicOr(&sb[(o >> 5) + 2], 1u << (o & 31));
    }
  }
}

// Tile offsets a in [0, TA): a is in A iff a selected diagonal crosses some pair
// (query tile t, key tile t - a), i.e. offsets [64a - 63, 64a + 63] hold a set
// bit; a >= 1 is "full" (no mask needed) iff all of them are set.
__global__ __launch_bounds__(256) void vs_tiles_kernel(AttnArgs a, BhList L, int TA) {
  const int bh = L.bh[blockIdx.x];
  const uint32_t* sb = a.sbits + (size_t)bh * a.sw + 2;     // unpadded view
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
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

// 16 bytes per lane straight from global memory into LDS; lane l of the wave
// lands at lds_base + 16 l (lds_base is wave-uniform).
__device__ __forceinline__ void dma16(const void* g, lds_void_t* lds_base) {
  __builtin_amdgcn_global_load_lds(g, lds_base, 16, 0, 0);
}
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// LDS layouts (both [64 keys][256 bytes], 16-byte chunks XOR-swizzled by row):
//   K: chunk c of row r at c ^ (r & 15)      -> conflict-free ds_read_b128 of 16 rows
//   V: chunk c of row r at c ^ 4 (r & 3)     -> conflict-free ds_read_b64_tr_b16
__device__ __forceinline__ int swz_k(int r, int c) { return c ^ (r & 15); }
__device__ __forceinline__ int swz_v(int r, int c) { return c ^ ((r & 3) << 2); }

struct Entry {
  int mode;    // M_*
  int kt;      // key tile, or gather chunk for M_GATHER
  int cnt;     // valid keys of a gather chunk
};

struct ItemCtx {
  int b, h, kvh, kind, t, P0, nrows, tq, last_pos;
  const int32_t* alist;    // VS strips (tile offsets, ascending)
  int nstrip;
  const uint32_t* fbits;
  const uint32_t* sbits;   // padded by two leading words
  const uint32_t* vbits;
  const int32_t* blist;    // BLOCK
  int nblk, per;
  int ngather;             // staged this round
  int nent;
};

// raw source value of entry n: the tile offset (VS strip) or block id (BLOCK)
__device__ __forceinline__ int entry_raw(const ItemCtx& c, int n) {
  if (n >= c.nent) return 0;
  if (c.kind == 1) return n < c.nstrip ? c.alist[n] : 0;
  if (c.kind == 2) return c.blist[n / c.per];
  return 0;
}

__device__ __forceinline__ Entry entry_of(const ItemCtx& c, int n, int raw) {
  Entry e;
  e.cnt = 0;
  if (c.kind == 1) {
    if (n < c.nstrip) {
      e.kt = c.tq - raw;
      e.mode = (raw >= 1 && test_bit(c.fbits, raw)) ? M_NONE : M_VS;
    } else {
      const int ch = n - c.nstrip;
      e.kt = ch;
      e.cnt = min(TK, c.ngather - ch * TK);
      e.mode = M_GATHER;
    }
  } else if (c.kind == 2) {
    e.kt = raw * c.per + n % c.per;
    if (raw < 0 || e.kt * TK > c.last_pos) e.mode = M_EMPTY;
    else e.mode = (e.kt * TK + TK - 1 > c.P0) ? M_CAUSAL : M_NONE;
  } else {
    e.kt = n;
    e.mode = (e.kt * TK + TK - 1 > c.P0) ? M_CAUSAL : M_NONE;
  }
  return e;
}

// Issue the DMA of one 64-key tile of K or V (rows = keys) into LDS.
template <bool IS_V>
__device__ __forceinline__ void issue_tile(const uint16_t* __restrict__ base, int Nk, const Entry& e,
                                           const int32_t* s_cols, char* lds, int w, int lane) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int blk = 2 * j + w;                 // which 1 KB (4 rows) this wave-instruction fills
    const int r = blk * 4 + (lane >> 4);
    const int pc = lane & 15;
    const int c = IS_V ? swz_v(r, pc) : swz_k(r, pc);
    int key;
    if (e.mode == M_GATHER) key = s_cols[e.kt * TK + (r < e.cnt ? r : 0)];
    else key = min(e.kt * TK + r, Nk - 1);
    dma16(base + (size_t)key * 128 + c * 8, (lds_void_t*)(lds + blk * 1024));
  }
}

struct MaskWords {
  uint32_t s0, s1, s2;   // diagonal bits window (VS)
  uint32_t v0, v1;       // column bits of the key tile (VS)
};

__device__ __forceinline__ void issue_mask_loads(const ItemCtx& c, const Entry& e, int iq, bool row_ok, MaskWords& mw) {
  if (e.mode != M_VS) return;
  // offsets o = iq - key for keys kt*64 + 0..63: window [iq - 64 kt - 63, iq - 64 kt]
  const int lo = iq - e.kt * TK - 63;
  const int wi = row_ok ? (lo >> 5) + 2 : 0;   // lo >= -63 on real rows, so wi >= 0 (two pad words)
  mw.s0 = c.sbits[wi];
  mw.s1 = c.sbits[wi + 1];
  mw.s2 = c.sbits[wi + 2];
  mw.v0 = c.vbits[2 * e.kt];
  mw.v1 = c.vbits[2 * e.kt + 1];
}

__device__ __forceinline__ uint64_t causal_mask64(int top) {   // bits c <= top
  return top < 0 ? 0ull : (top >= 63 ? ~0ull : ((2ull << top) - 1ull));
}

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2))) void attn_kernel(const AttnArgs a, const Sched sc) {
  __shared__ __align__(1024) char s_k[TK * 256];
  __shared__ __align__(1024) char s_v[TK * 256];
  __shared__ int32_t s_cols[GCAP];
  __shared__ int s_misc[4];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
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

      const int qrow = r0 + 32 * w + qn;
      const int iq = c.P0 + 32 * w + qn;          // absolute position of this lane's row
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

      int gcursor = 0, gcount = 0;
      if (c.kind == 1) {
        c.alist = a.alist + (size_t)bh * a.acap;
        c.fbits = a.fbits + (size_t)bh * a.aw;
        c.sbits = a.sbits + (size_t)bh * a.sw;
        c.vbits = a.vbits + (size_t)bh * a.vw;
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
          // stage this item's columns: 0 <= j <= last_pos, outside the strip tiles
          const int32_t* cols = a.cols + (size_t)bh * a.cols_cap;
          const uint32_t* ab = a.abits + (size_t)bh * a.aw;
          int staged = 0;
          while (gcursor < gcount && staged <= GCAP - NT) {
            const int idx = gcursor + tid;
            bool keep = false;
            int j = 0;
            if (idx < gcount) {
              j = cols[idx];
              keep = (j >= 0) && (j <= c.last_pos) && !test_bit(ab, c.tq - (j >> 6));
            }
            const uint64_t bal = __builtin_amdgcn_ballot_w64(keep);
            __syncthreads();
            if (l == 0) s_misc[1 + w] = __popcll(bal);
            __syncthreads();
            const int off = staged + (w ? s_misc[1] : 0);
            if (keep) s_cols[off + ballot_rank(bal)] = j;
            staged += s_misc[1] + s_misc[2];
            gcursor += NT;
            const int lastc = cols[min(gcursor, gcount) - 1];
            if (lastc > c.last_pos) gcursor = gcount;
          }
          __syncthreads();
          c.ngather = staged;
          if (round > 0) c.nstrip = 0;
          c.nent = c.nstrip + (staged + TK - 1) / TK;
        } else if (c.kind == 2) {
          c.nent = c.nblk * c.per;
        } else {
          c.nent = c.last_pos / TK + 1;
        }

        Entry cur;
        MaskWords mw = {0u, 0u, 0u, 0u, 0u};
        int raw_next = 0;
        if (c.nent > 0) {
          cur = entry_of(c, 0, entry_raw(c, 0));
          raw_next = entry_raw(c, 1);
          if (cur.mode != M_EMPTY) issue_tile<false>(kbp, a.Nk, cur, s_cols, s_k, w, l);
          issue_mask_loads(c, cur, iq, row_ok, mw);
        }
        for (int n = 0; n < c.nent; ++n) {
          wait_vm();
          __syncthreads();                       // K_n visible; every wave is done with V_{n-1}
          const bool live = cur.mode != M_EMPTY;
          if (live) issue_tile<true>(vbp, a.Nk, cur, s_cols, s_v, w, l);

          // ---- this lane's 64-bit mask over the tile's keys (bit c <-> key kt*64 + c)
          uint64_t M = ~0ull;
          if (cur.mode == M_CAUSAL) {
            M = causal_mask64(iq - cur.kt * TK);
          } else if (cur.mode == M_VS) {
            const int lo = iq - cur.kt * TK - 63;
            const int sh = lo & 31;
            const uint64_t lo64 = ((uint64_t)mw.s1 << 32) | mw.s0;
            const uint64_t hi64 = (uint64_t)mw.s2;
            const uint64_t win = sh ? ((lo64 >> sh) | (hi64 << (64 - sh))) : lo64;   // bit b <-> offset lo + b
            const uint64_t rev = ((uint64_t)__builtin_bitreverse32((uint32_t)win) << 32) |
                                 __builtin_bitreverse32((uint32_t)(win >> 32));       // bit c <-> key c
            M = (rev | (((uint64_t)mw.v1 << 32) | mw.v0)) & causal_mask64(iq - cur.kt * TK);
          } else if (cur.mode == M_GATHER) {
            // columns are ascending: keys c < n_le are <= iq
            const int base = cur.kt * TK;
            int lo2 = 0, hi2 = cur.cnt;
            while (lo2 < hi2) {
              const int mid = (lo2 + hi2) >> 1;
              if (s_cols[base + mid] <= iq) lo2 = mid + 1; else hi2 = mid;
            }
            M = lo2 >= 64 ? ~0ull : ((1ull << lo2) - 1ull);
          }
          if (!row_ok) M = 0ull;
          const bool masked = cur.mode != M_NONE;
          bool act[2];
          act[0] = live && __builtin_amdgcn_ballot_w64((uint32_t)M != 0u) != 0;
          act[1] = live && __builtin_amdgcn_ballot_w64((uint32_t)(M >> 32) != 0u) != 0;

          // ---- S^T = K Q^T
          f32x16 sacc[2];
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int v = 0; v < 16; ++v) sacc[kb][v] = 0.f;
            if (act[kb]) {
              const int row = 32 * kb + qn;
#pragma unroll
              for (int ks = 0; ks < 8; ++ks) {
                const u32x4 x = *(const u32x4*)(s_k + row * 256 + swz_k(row, 2 * ks + hh) * 16);
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x), qf[ks], sacc[kb],
                                                                   0, 0, 0);
              }
            }
          }
          // ---- mask and online softmax (scores kept raw; scale folded into exp2)
          float mx = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            if (!act[kb]) continue;
            const uint32_t mk = (uint32_t)(M >> (32 * kb)) >> (4 * hh);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              float x = sacc[kb][v];
              if (masked && !((mk >> (8 * (v >> 2) + (v & 3))) & 1u)) x = -INFINITY;
              sacc[kb][v] = x;
              mx = fmaxf(mx, x);
            }
          }
          mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * scale2;
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
              const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][v], scale2, -muse));
              const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][v + 1], scale2, -muse));
              // normalise with the same bf16-rounded weights the PV product uses
              const uint32_t pb = pack_bf16x2(p0, p1);
              l_run += bf16_lo(pb) + bf16_hi(pb);
              pk[kb][v >> 1] = pb;
            }
          }

          wait_vm();
          __syncthreads();                       // V_n visible; every wave is done with K_n
          Entry nxt;
          nxt.mode = M_EMPTY;
          if (n + 1 < c.nent) {
            nxt = entry_of(c, n + 1, raw_next);
            raw_next = entry_raw(c, n + 2);
            if (nxt.mode != M_EMPTY) issue_tile<false>(kbp, a.Nk, nxt, s_cols, s_k, w, l);
            issue_mask_loads(c, nxt, iq, row_ok, mw);
          }

          // ---- O^T += V^T P^T, keys 16 ks2 .. +15 per step
#pragma unroll
          for (int ks2 = 0; ks2 < 4; ++ks2) {
            const int kb = ks2 >> 1;
            if (!act[kb]) continue;
            const int o8 = (ks2 & 1) * 4;
            u32x4 bx = {pk[kb][o8], pk[kb][o8 + 1], pk[kb][o8 + 2], pk[kb][o8 + 3]};
            const bf16x8 bop = __builtin_bit_cast(bf16x8, bx);
            const int G = l >> 4, s = l & 15;
            const int rowa = 16 * ks2 + 4 * (G >> 1) + (s >> 2);
            const int rowb = rowa + 8;
#pragma unroll
            for (int db = 0; db < 4; ++db) {
              const int cch = 4 * db + 2 * (G & 1) + ((s & 3) >> 1);
              const int half = (s & 1) * 8;
              lds_short4_t* pa = (lds_short4_t*)((__attribute__((address_space(3))) char*)s_v + rowa * 256 +
                                                 swz_v(rowa, cch) * 16 + half);
              lds_short4_t* pb2 = (lds_short4_t*)((__attribute__((address_space(3))) char*)s_v + rowb * 256 +
                                                  swz_v(rowb, cch) * 16 + half);
              const short4_t ya = __builtin_amdgcn_ds_read_tr16_b64_v4i16(pa);
              const short4_t yb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(pb2);
              typedef short short8_t __attribute__((ext_vector_type(8)));
              const short8_t ab = {ya[0], ya[1], ya[2], ya[3], yb[0], yb[1], yb[2], yb[3]};
              acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ab), bop, acc[db], 0, 0, 0);
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
  L.sw = (Nk + 31) / 32 + 5;
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
