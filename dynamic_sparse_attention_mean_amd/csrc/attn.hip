// Sparse prefill attention over per-head index sets (gfx950).
//
// What it computes: for each head h and query row i,
//   O[i] = sum_{j in M_h(i)} softmax_j(q_i . k_j / sqrt(d)) v_j,  LSE[i] = log sum exp,
// with M_h(i) given by the head's pattern and index set ("MInference 1.0"
// explainer, GPU kernels section; authors' abstract: sparse kernels over
// pattern + indices).  As "FlashPrefill" section 2.3 prescribes, the kernel
// walks compact lists of key tiles (index-driven jumps), never testing the
// tiles it does not need.
//
// Design (MI355X, gfx950):
//  * A work item is (batch, head, pair of adjacent 64-row query tiles): 128 rows,
//    one workgroup of 4 waves, each wave owning 32 rows.  The pair streams the
//    union of its two tiles' key-tile lists once, so every K/V tile brought into
//    LDS serves up to 128 rows; each wave applies its own exact mask and skips
//    32x32 sub-blocks with no selected entry.
//  * S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16 (fp32 accumulate):
//    the MFMA output of S^T is, after the softmax, exactly the B operand layout
//    of the PV product, so P never leaves registers.
//  * K and V tiles travel global -> LDS by DMA (global_load_lds_dwordx4) into a
//    two-stage ring: tile n+1 is in flight while tile n is computed, one barrier
//    per tile.  16-byte chunks are XOR-swizzled per row so the ds_read_b128 of K
//    and the transposing ds_read_b64_tr_b16 of V are bank-conflict free.
//  * Online softmax in fp32 (base 2, scale folded into the exponent), P rounded
//    to bf16 for the MFMA and summed in that same rounding (v_dot2_f32_bf16), the
//    accumulator rescaled lazily (only when the row max grows by > 8 in log2).
//  * Vertical-Slash heads run on a skewed schedule of 32x32 sub-blocks.  In the
//    sub-block of 32 rows starting at position R and 32 keys starting at R - 32e
//    every offset i - j lies in [32e - 31, 32e + 31], whatever R is; so a compile
//    step turns the diagonal list into the set D of such e that hold a selected
//    diagonal.  For each e in D (descending) wave w of the pair takes the 32 keys
//    starting at P0 + 32 (w - e): all four waves have a sub-block at every step,
//    and the block a wave uses is the one its neighbour used one step before, so
//    a step brings in one new 32-key block of K and V (a five-slot LDS ring).
//    Each sub-block carries the exact mask (diagonal bit | column bit, causal).
//    Columns a wave's sub-blocks do not cover are gathered 64 at a time and the
//    wave masks the ones it covered.  Every selected (i, j) is visited exactly
//    once.  A head whose sets are exactly a sink [0, S) of columns and the
//    diagonals [0, L) (the A-shape sets) is recognised by the compile step and
//    runs like a dense head over the 64-key tiles of the sink and the window,
//    with a closed-form mask on the edge tiles.
//  * Persistent workgroups pull items from per-XCD queues (longest rows first)
//    and steal from other queues when their own is empty.
#include "common.h"
#include "internal.h"

#include <algorithm>
#include <mutex>
#include <type_traits>
#include <vector>

namespace dsa {
namespace {

constexpr int TQ = 64;       // rows per query tile
constexpr int TK = 64;       // keys per key tile
constexpr int NT = 256;      // 4 waves: two query tiles x two 32-row halves
constexpr int GCAP = 2048;   // gathered columns staged per round

enum { M_NONE = 0, M_CAUSAL = 1, M_WIN = 2, M_GATHER = 3, M_SKIP = 4 };

// Entries of the schedule's head table: b * H + h, with two flag bits for the
// pairs of block heads (see launch_attention).
constexpr int kPairBit = 0x4000, kParityBit = 0x2000, kHeadMask = 0x1FFF;
static_assert(kMaxHeadTable <= kHeadMask + 1, "head index and flags overlap");

struct Sched {
  int nq;                       // number of queues
  int T2;                       // query-tile pairs per head
  int qstart[kMaxQueues + 1];   // heads of queue g: heads[qstart[g] .. qstart[g+1])
  int16_t heads[kMaxHeadTable]; // b * H + h
};

struct BhList {
  int n;
  int16_t bh[kMaxHeadTable];
};

// Reads of the small per-head tables held in the kernel arguments at a
// wave-uniform index, as whole dwords: gfx9 has no sub-dword scalar loads, so
// an int16 or int8 element read directly becomes a vector load.
static_assert(offsetof(Sched, heads) % 4 == 0 && offsetof(AttnArgs, kind) % 4 == 0, "dword-aligned tables");
typedef int32_t __attribute__((may_alias)) alias_i32_t;
__device__ __forceinline__ int arg_i16(const int16_t* t, int i) {
  const int32_t w = reinterpret_cast<const alias_i32_t*>(t)[i >> 1];
  return (i & 1) ? (w >> 16) : (int)(int16_t)(w & 0xFFFF);
}
__device__ __forceinline__ int arg_i8(const int8_t* t, int i) {
  const int32_t w = reinterpret_cast<const alias_i32_t*>(t)[i >> 2];
  return (int)(int8_t)(w >> (8 * (i & 3)));
}

// ------------------------------------------------------------------ bitmaps

// any bit set in [lo, hi] (inclusive, 0 <= lo <= hi) of an unpadded bitmap
__device__ bool range_any(const uint32_t* bm, int lo, int hi) {
  for (int wd = lo >> 5; wd <= (hi >> 5); ++wd) {
    uint32_t m = ~0u;
    if (wd == (lo >> 5)) m &= ~0u << (lo & 31);
    if (wd == (hi >> 5)) m &= ~0u >> (31 - (hi & 31));
    if (bm[wd] & m) return true;
  }
  return false;
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

// Step centres of a Vertical-Slash head.  A 32x32 sub-block whose rows start at
// position R and whose keys start at R - c holds the offsets i - j in
// [c - 31, c + 31], offset c on all 32 rows.  A set C of such centres, any two
// at least 32 apart, visits every (i, j) at most once in each wave's key
// blocks; it visits every row of offset o iff o is a centre or lies between
// two centres exactly 32 apart.  C is built greedily over the selected offsets
// in ascending order: an offset already covered is skipped, one within 32 of
// the last centre extends the run by a centre 32 further on, and any other
// offset starts a new run centred on itself.  So a band of W consecutive
// offsets costs 1 + ceil((W - 1) / 32) sub-blocks per wave, and a lone diagonal
// one.  An offset with no selected offset in the 63 before it always starts a
// run; each thread takes the run starts of one bitmap word and follows the
// greedy from there until the next such offset.
//
// Outputs per head: the centres ascending, each with the 64 diagonal bits of
// offsets [c - 32, c + 31] ({c, bits 0-31, bits 32-63, 0}); a bitmap of the
// centres; and the prefix counts #{c in C : c <= 32 x + 31}.  A head whose lists
// are exactly cols = [0, S) and diags = [0, L) (the A-shape sets: sink S, local
// window L) is marked as a window head: its mask is closed-form and runs on
// whole tiles.
// Diagonal bitmaps of up to this many words are staged in LDS by the compile
// step (the greedy's reads are then LDS reads); longer ones are read in place.
constexpr int kCentreLdsWords = 16384;

// 64 bits of a bitmap window w[0..4] (bit 0 of w[0] at position p0), from
// bit position lo on (p0 <= lo <= p0 + 95).
__device__ __forceinline__ uint64_t window64(const uint32_t (&w)[5], int p0, int lo) {
  const int rel = lo - p0, k = rel >> 5, sh = rel & 31;
  const uint64_t a = ((uint64_t)w[k + 1] << 32) | w[k];
  return sh == 0 ? a : (a >> sh) | ((uint64_t)w[k + 2] << (64 - sh));
}

// The greedy of one run start s over a head's unpadded diagonal bitmap
// (word(i): word i, zero outside the bitmap): calls f(c) for each centre, in
// order, until the next offset that starts a run of its own.  An offset within
// 32 of the last centre c never does (the last selected offset before it lies
// in [c - 31, c]); one further on does when none of the 63 offsets before it
// is selected.  Each step reads the five words around c at once.
template <typename Word, typename F>
__device__ void follow_run(const Word& word, int s, F&& f) {
  int c = s;
  f(c);
  while (true) {
    const int b = (c - 62) >> 5;                          // floor division
    uint32_t w[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) w[i] = word(b + i);
    const uint64_t nx = window64(w, 32 * b, c + 1) & (~0ull >> 1);   // offsets c + 1 .. c + 63
    if (nx == 0) break;
    const int o = c + 1 + __builtin_ctzll(nx);
    if (o <= c + 32) {
      c += 32;
    } else {
      if ((window64(w, 32 * b, o - 63) & (~0ull >> 1)) == 0) break;   // offsets o - 63 .. o - 1
      c = o;
    }
    f(c);
  }
}

// Workgroup barrier for LDS data only: unlike __syncthreads it does not wait
// for this wave's global stores (the compile step's outputs) to complete.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Exclusive prefix sum of v over a 256-thread workgroup (s: 4 ints of LDS).
__device__ __forceinline__ int block_excl_scan(int v, int* s) {
  const int w = threadIdx.x >> 6;
  const int incl = (int)wave_incl_scan((uint32_t)v);
  if ((threadIdx.x & 63) == 63) s[w] = incl;
  lds_barrier();
  int off = incl - v;
  for (int i = 0; i < w; ++i) off += s[i];
  lds_barrier();
  return off;
}

__global__ __launch_bounds__(256) void vs_centres_kernel(AttnArgs a, BhList L, int ND) {
  __shared__ uint32_t s_bits[kCentreLdsWords];
  __shared__ int32_t s_starts[kCentreLdsWords / 2 + 8];  // run starts of one chunk of words
  __shared__ uint8_t s_cb[kCentreLdsWords + 8];          // a centre in 32 positions x, when they fit
  const int bh = L.bh[blockIdx.x];
  const uint32_t* sb = a.sbits + (size_t)bh * a.sw + 2;     // unpadded view (two zero words before it)
  uint32_t* cb = a.cbits + (size_t)bh * a.cw;
  int32_t* cl = a.clist + (size_t)bh * a.ccap * 4;
  int32_t* cle = a.cle + (size_t)bh * a.ccap;
  __shared__ int s_scan[4];
  __shared__ int s_prefix;
  if (threadIdx.x == 0) s_prefix = 1;
  __syncthreads();
  {
    const int nc = min(a.cols_count[bh], a.cols_cap), nd = min(a.diags_count[bh], a.diags_cap);
    const int32_t* cols = a.cols + (size_t)bh * a.cols_cap;
    const int32_t* diags = a.diags + (size_t)bh * a.diags_cap;
    bool ok = true;
    for (int i = threadIdx.x; i < nc; i += 256) ok = ok && cols[i] == i;
    for (int i = threadIdx.x; i < nd; i += 256) ok = ok && diags[i] == i;
    if (!ok) s_prefix = 0;
    __syncthreads();
    if (threadIdx.x == 0) {
      a.win[2 * bh] = s_prefix ? nd : -1;
      a.win[2 * bh + 1] = nc;
    }
  }
  // a window head runs on whole tiles and never reads its centres
  if (s_prefix) return;
  const int nwords = (a.Nk + 31) / 32;
  const bool in_lds = nwords <= kCentreLdsWords;          // then ND <= kCentreLdsWords + 1
  if (in_lds) {
    for (int i = threadIdx.x; i < nwords; i += 256) s_bits[i] = sb[i];
    for (int i = threadIdx.x; i < ND; i += 256) s_cb[i] = 0;
  }
  __syncthreads();
  auto centres = [&](const auto& word) {
    int base = 0;                                      // centres written so far
    for (int c0 = 0; c0 < nwords; c0 += kCentreLdsWords) {
      const int c1 = min(nwords, c0 + kCentreLdsWords);
      // 1. the run starts of words [c0, c1), ascending: a word's lowest set bit
      // o with none of the 63 offsets before it selected (any later set bit of
      // a word has one less than 32 before it)
      int nst = 0;
      for (int x0 = c0; x0 < c1; x0 += 256) {
        const int x = x0 + threadIdx.x;
        bool st = false;
        int o = 0;
        if (x < c1) {
          const uint32_t m = word(x);
          if (m) {
            o = 32 * x + __builtin_ctz(m);
            const uint64_t prev = ((uint64_t)word(x - 1) << 32) | word(x - 2);   // offsets 32x - 64 .. 32x - 1
            st = (prev >> ((o & 31) + 1)) == 0;
          }
        }
        const uint64_t bal = __builtin_amdgcn_ballot_w64(st);
        const int wv = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) s_scan[wv] = __popcll(bal);
        lds_barrier();
        int pos = nst;
        for (int i = 0; i < wv; ++i) pos += s_scan[i];
        if (st) s_starts[pos + (int)ballot_rank(bal)] = o;
        nst += s_scan[0] + s_scan[1] + s_scan[2] + s_scan[3];
        lds_barrier();
      }
      // 2. one run start per thread: count its centres, place them, write them
      for (int r0 = 0; r0 < nst; r0 += 256) {
        const int i = r0 + threadIdx.x;
        const int st = i < nst ? s_starts[i] : -1;
        int cnt = 0;
        if (st >= 0) follow_run(word, st, [&](int) { ++cnt; });
        int off = base + block_excl_scan(cnt, s_scan);
        if (st >= 0) {
          follow_run(word, st, [&](int c) {
            // the 64 diagonal bits of offsets [c - 32, c + 31]
            const int wi = (c >> 5) - 1, sh = c & 31;
            const uint64_t lo = ((uint64_t)word(wi + 1) << 32) | word(wi);
            const uint64_t win = sh == 0 ? lo : (lo >> sh) | ((uint64_t)word(wi + 2) << (64 - sh));
            u32x4 e = {(uint32_t)c, (uint32_t)win, (uint32_t)(win >> 32), 0u};
            *(u32x4*)(cl + 4 * (size_t)off) = e;
            cb[c >> 5] = 1u << (c & 31);                    // one centre per word at most
            if (in_lds) s_cb[c >> 5] = 1;
            ++off;
          });
        }
        // the next round starts after the last centre of this one
        if (threadIdx.x == 255) s_scan[0] = off;
        lds_barrier();
        base = s_scan[0];
        lds_barrier();
      }
    }
    return base;
  };
  int total;
  if (in_lds) {
    total = centres([&](int i) -> uint32_t { return (i >= 0 && i < nwords) ? s_bits[i] : 0u; });
  } else {
    total = centres([&](int i) -> uint32_t { return (i >= 0 && i < nwords) ? sb[i] : 0u; });
    __syncthreads();                                    // the global centre bitmap is read back below
  }
  // prefix counts per 32 positions (at most one centre per 32 positions): each
  // thread counts the centres of its range, one scan, then fills it
  const int pc = (ND + 255) / 256;
  const int c_lo = threadIdx.x * pc, c_hi = min(ND, c_lo + pc);
  int n_own = 0;
  for (int x = c_lo; x < c_hi; ++x) n_own += (in_lds ? s_cb[x] != 0 : cb[x] != 0u) ? 1 : 0;
  int run = block_excl_scan(n_own, s_scan);
  for (int x = c_lo; x < c_hi; ++x) {
    run += (in_lds ? s_cb[x] != 0 : cb[x] != 0u) ? 1 : 0;
    cle[x] = run;
  }
  if (threadIdx.x == 0) a.ccount[bh] = total;
}

// ---------------------------------------------------------------- main kernel
typedef __attribute__((address_space(3))) void lds_void_t;
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;
typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4_t;

// Four DMAs of 1 KB (a full tile's share of one wave) with one M0 save/restore.
__device__ __forceinline__ void dma16x4(const char* g0, const char* g1, const char* g2, const char* g3, uint32_t l0,
                                        uint32_t l1, uint32_t l2, uint32_t l3) {
  uint32_t save;
  asm volatile("s_mov_b32 %0, m0\n\t"
               "s_mov_b32 m0, %5\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\t"
               "s_mov_b32 m0, %6\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, off\n\t"
               "s_mov_b32 m0, %7\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %3, off\n\t"
               "s_mov_b32 m0, %8\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %4, off\n\t"
               "s_mov_b32 m0, %0"
               : "=&s"(save)
               : "v"(g0), "v"(g1), "v"(g2), "v"(g3), "s"(l0), "s"(l1), "s"(l2), "s"(l3)
               : "memory");
}
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// LDS tiles are [64 keys][256 bytes] with 16-byte chunks XOR-swizzled by row:
//   K: chunk c of row r at c ^ (r & 15)      -> conflict-free ds_read_b128 of 16 rows
//   V: chunk c of row r at c ^ 4 (r & 3)     -> conflict-free ds_read_b64_tr_b16
__device__ __forceinline__ int swz_k(int r, int c) { return c ^ (r & 15); }
__device__ __forceinline__ int swz_v(int r, int c) { return c ^ ((r & 3) << 2); }

// Wave-uniform read of data the kernel never writes, through the constant
// address space so that it becomes a scalar load (lgkmcnt, not vmcnt): the
// K/V DMAs are then the only vector memory operations in the tile loop, and
// the vmcnt wait at the top of a step waits for nothing else.
typedef const __attribute__((address_space(4))) int32_t c_i32_t;
typedef const __attribute__((address_space(4))) uint32_t c_u32_t;
__device__ __forceinline__ int ldc(const int32_t* p, size_t i) { return ((c_i32_t*)p)[i]; }
__device__ __forceinline__ uint32_t ldc(const uint32_t* p, size_t i) { return ((c_u32_t*)p)[i]; }
typedef const __attribute__((address_space(4))) u32x4 c_u32x4_t;
// entry i of an array of 16-byte records, as one scalar load
__device__ __forceinline__ u32x4 ldc4(const int32_t* p, size_t i) { return ((c_u32x4_t*)p)[i]; }

// One entry of a pair's tile stream.
struct Entry {
  int kind;    // 0 key tile, 1 gather chunk, -1 none
  int kt;      // key tile index, or gather chunk index
  int cnt;     // valid keys of a gather chunk
  int flags;   // bit h: query tile h of the pair uses this entry
};

struct Item {
  int bh, kvh, kind, P0, last_pos, tq1;
  // WINDOW (kind 3): tiles [0, n0) then n1, n1 + 1, ...; sink wsink, window wlen
  int wsink, wlen;
  // BLOCK
  const int32_t* l0;       // list of query block I0 (or of the shared block)
  const int32_t* l1;       // list of query block I0 + 1 (block 64 only)
  int n0, n1, per;
  // stream
  int nent, ngather;
};

// Cursor over a pair's entries.  The list lookups an entry will need are
// issued by cursor_fetch() at the end of the step before (one step of
// prefetch), after that step's LDS reads: scalar loads share the LDS reads'
// wait counter.
struct Cursor {
  int n;                   // index of the next entry
  int raw;                 // prefetched value for entry n (shared block list)
  int i0, i1, x0, x1;      // two-list merge state (block 64): heads of both lists
  int x0n, x1n;            // prefetched successors of the heads
  bool fetch_raw, fetch0, fetch1;   // lookups cursor_fetch() still has to issue
};

__device__ __forceinline__ int list_at(const int32_t* L, int n, int i) { return i < n ? ldc(L, i) : 0x7fffffff; }

__device__ __forceinline__ void cursor_init(const Item& it, Cursor& c) {
  c.n = 0;
  c.raw = 0;
  c.fetch_raw = c.fetch0 = c.fetch1 = false;
  c.i0 = c.i1 = 0;
  c.x0 = c.x1 = c.x0n = c.x1n = 0x7fffffff;
  if (it.kind == 2 && it.per == 2) c.raw = it.n0 > 0 ? ldc(it.l0, 0) : 0;
  else if (it.kind == 2) {
    c.x0 = list_at(it.l0, it.n0, 0); c.x1 = list_at(it.l1, it.n1, 0);
    c.x0n = list_at(it.l0, it.n0, 1); c.x1n = list_at(it.l1, it.n1, 1);
  }
}

__device__ __forceinline__ bool cursor_has_next(const Item& it, const Cursor& c) {
  if (it.kind == 2 && it.per == 1) return min(c.x0, c.x1) != 0x7fffffff;
  return c.n < it.nent;
}

// Produce entry c.n and advance.  Valid only while cursor_has_next().
__device__ __forceinline__ Entry cursor_next(const Item& it, Cursor& c) {
  Entry e;
  e.cnt = 0;
  e.flags = 3;
  e.kind = 0;
  const int n = c.n++;
  if (it.kind == 1) {
    e.kind = 1;
    e.kt = n;
    e.cnt = min(TK, it.ngather - n * TK);
  } else if (it.kind == 2 && it.per == 2) {
    e.kt = c.raw * 2 + (n & 1);
    c.fetch_raw = (n & 1) != 0;            // entry n + 1 starts the next list element
  } else if (it.kind == 2) {
    const int x = min(c.x0, c.x1);
    e.kt = x;
    e.flags = (c.x0 == x ? 1 : 0) | (c.x1 == x ? 2 : 0);
    if (c.x0 == x) { ++c.i0; c.x0 = c.x0n; c.fetch0 = true; }
    if (c.x1 == x) { ++c.i1; c.x1 = c.x1n; c.fetch1 = true; }
  } else if (it.kind == 3) {
    e.kt = n < it.n0 ? n : it.n1 + (n - it.n0);
  } else {
    e.kt = n;
  }
  // out-of-range block ids or tiles beyond the pair's last row contribute nothing
  if (e.kind == 0 && (e.kt < 0 || e.kt * TK > it.last_pos)) e.flags = 0;
  return e;
}

// The list lookups the last cursor_next() left for later (see Cursor).
__device__ __forceinline__ void cursor_fetch(const Item& it, Cursor& c) {
  if (c.fetch_raw) c.raw = ((c.n >> 1) < it.n0) ? ldc(it.l0, c.n >> 1) : 0;
  if (c.fetch0) c.x0n = list_at(it.l0, it.n0, c.i0 + 1);
  if (c.fetch1) c.x1n = list_at(it.l1, it.n1, c.i1 + 1);
  c.fetch_raw = c.fetch0 = c.fetch1 = false;
}

// DMA of one 64-key tile of K or V into LDS.  Wave w fills the 1 KB blocks
// 4j + w, i.e. rows 16j + rl with rl = 4w + lane/16.  A full tile is a
// wave-uniform base plus this lane's constant offset; a partial tile or a
// gather chunk computes each row's key.
template <bool IS_V>
__device__ __forceinline__ void issue_tile(const uint16_t* __restrict__ base, int Nk, const Entry& e,
                                           const int32_t* s_cols, uint32_t lds, int w, int lane, uint32_t off) {
  if (e.flags == 0) return;
  if (e.kind == 0 && e.kt * TK + TK <= Nk) {
    const char* tb = (const char*)(base + (size_t)e.kt * TK * 128) + off;
    dma16x4(tb, tb + 4096, tb + 8192, tb + 12288, lds + w * 1024, lds + (4 + w) * 1024, lds + (8 + w) * 1024,
            lds + (12 + w) * 1024);
    return;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 16 * j + 4 * w + (lane >> 4);
    const int c = IS_V ? swz_v(r, lane & 15) : swz_k(r, lane & 15);
    int key;
    if (e.kind == 1) key = s_cols[e.kt * TK + (r < e.cnt ? r : 0)];
    else key = min(e.kt * TK + r, Nk - 1);
    dma16(base + (size_t)key * 128 + c * 8, lds + (4 * j + w) * 1024);
  }
}

__device__ __forceinline__ uint32_t causal_mask32(int top) {   // bits c <= top
  return top < 0 ? 0u : (top >= 31 ? ~0u : ((2u << top) - 1u));
}

#ifndef DSA_ATTN_WAVES_PER_SIMD
#define DSA_ATTN_WAVES_PER_SIMD 2
#endif
// Wave priority around MFMA groups (s_setprio): a wave that reaches its MFMAs
// issues them ahead of the other waves' softmax work on the same SIMD.  Off by
// default: without it dense 64-key tile steps run about 2 % faster and the
// mixed layer is unchanged.
#ifndef DSA_ATTN_SETPRIO
#define DSA_ATTN_SETPRIO 0
#endif
#if DSA_ATTN_SETPRIO
#define DSA_PRIO_HI() __builtin_amdgcn_s_setprio(1)
#define DSA_PRIO_LO() __builtin_amdgcn_s_setprio(0)
#else
#define DSA_PRIO_HI() ((void)0)
#define DSA_PRIO_LO() ((void)0)
#endif

// LDS arena of one workgroup.  The five-slot ring of 32-key K/V blocks used by
// the Vertical-Slash sub-block steps covers all of it; the two-stage ring of
// 64-key tiles, the gathered column list, its coverage bytes and a few shared
// counters are laid out inside it for the other phases.  80 KB: two workgroups
// fill the 160 KB of a CU.
constexpr int NSLOT = 5;
constexpr int SLOT = 2 * 32 * 256;                 // K [32 rows][256 B], then V
constexpr int LDS_BYTES = NSLOT * SLOT;
constexpr int OFF_COLS = 2 * 2 * TK * 256;         // after the 64-key ring [stage][K, V]
constexpr int OFF_COV = OFF_COLS + GCAP * 4;
constexpr int OFF_MISC = OFF_COV + GCAP;
static_assert(OFF_MISC + 8 * 4 <= LDS_BYTES, "LDS arena overflow");
// Small-block gather (blocks of 16 or 32): a two-stage ring of 32-key units
// (two slots), then a 16-bit mask per unit and the compacted unit list; the
// shared counters at OFF_MISC stay clear of both.
constexpr int kSmallUnits = 7168;                  // 32-key units per item (keys < 229376)
constexpr int OFF_UMASK = 2 * SLOT;
constexpr int OFF_ULIST = OFF_UMASK + kSmallUnits * 2;
static_assert(OFF_ULIST + kSmallUnits * 4 <= OFF_MISC, "small-block regions overlap the shared counters");
// Blocks of 16 gathered in pairs: behind the same two-slot ring, one mask byte
// per 16-key block and the compacted block list.
constexpr int kPairBlocks = 8192;                  // 16-key blocks per item (keys < 131072)
constexpr int OFF_BMASK = 2 * SLOT;
constexpr int OFF_BLIST = OFF_BMASK + kPairBlocks;
static_assert(OFF_BLIST + kPairBlocks * 4 <= OFF_MISC, "paired-block regions overlap the shared counters");

// Ring slot arithmetic on small non-negative values (unsigned: a multiply-high
// and a shift, not the signed remainder's fix-ups).
__device__ __forceinline__ int umod5(int x) { return (int)((uint32_t)x % (uint32_t)NSLOT); }
__device__ __forceinline__ int addmod5(int a, int b) { const int t = a + b; return t >= NSLOT ? t - NSLOT : t; }

template <bool SMALL>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(DSA_ATTN_WAVES_PER_SIMD))) void attn_kernel(
    const AttnArgs a, const Sched sc) {
  __shared__ __align__(1024) char s_lds[LDS_BYTES];
  int32_t* const s_cols = (int32_t*)(s_lds + OFF_COLS);
  uint8_t* const s_cov = (uint8_t*)(s_lds + OFF_COV);
  int* const s_misc = (int*)(s_lds + OFF_MISC);

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ih = w >> 1;               // which query tile of the pair
  const int wr = w & 1;                // which 32-row half of that tile
  const int l = tid & 63;
  const int qn = l & 31;
  const int hh = l >> 5;
  const float scale2 = 1.4426950408889634f * 0.08838834764831845f;  // log2(e) / sqrt(128)
  const int rep = a.H / a.Hkv;
  const int myq = blockIdx.x % sc.nq;
  const int rl = 4 * w + (l >> 4);
  const uint32_t off_k = rl * 256 + (((l & 15) ^ (rl & 15)) * 16);
  const uint32_t off_v = rl * 256 + (((l & 15) ^ ((rl & 3) << 2)) * 16);
  // lane-constant parts of the V fragment addresses
  const int G = l >> 4, si = l & 15;
  const int v_row0 = 4 * (G >> 1) + (si >> 2);           // + 16 s2 (+ 8)
  const int v_half = (si & 1) * 8;
  // LDS byte address of the arena (64-key ring: stage s, K (0) or V (1) at + (2 s + kv) * 16 KB)
  const uint32_t ring = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_char_t*)&s_lds[0]);
  // This lane's LDS addresses of its K fragments (row qn of a 32-key block, chunk 2 ks + hh) and V
  // fragments (row v_row0, the chunk of d block db), arena base included.  The swizzle makes them
  // lane-dependent; every other part of an address (ring stage, key half, 16-key step) is then an
  // immediate offset of the read.
  uint32_t kaddr[8], vaddr[4];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) kaddr[ks] = ring + qn * 256 + swz_k(qn, 2 * ks + hh) * 16;
#pragma unroll
  for (int db = 0; db < 4; ++db)
    vaddr[db] = ring + v_row0 * 256 + swz_v(v_row0, 4 * db + 2 * (G & 1) + ((si & 3) >> 1)) * 16 + v_half;

  for (int qi = 0; qi < sc.nq; ++qi) {
    const int g = (myq + qi) % sc.nq;
    const int nh = sc.qstart[g + 1] - sc.qstart[g];
    const int nitems = nh * sc.T2;
    if (nh == 0) continue;
    while (true) {
      __syncthreads();
      if (tid == 0) s_misc[0] = atomicAdd(&a.counters[g], 1);
      __syncthreads();
      // wave-uniform, so that the head and kind lookups below are scalar loads
      // from the kernel arguments rather than a chain of vector loads
      const int itn = __builtin_amdgcn_readfirstlane(s_misc[0]);
      if (itn >= nitems) break;

      Item it;
      const int he = arg_i16(sc.heads, sc.qstart[g] + itn % nh);
      const bool paired = (he & kPairBit) != 0;     // one query tile of heads bh0, bh0 + 1
      const int bh0 = he & kHeadMask;
      it.bh = bh0 + (paired ? ih : 0);               // this wave's head
      const int b = it.bh / a.H, h = it.bh % a.H;
      it.kvh = h / rep;
      it.kind = arg_i8(a.kind, h);
      const int p = sc.T2 - 1 - itn / nh;
      const int r0 = p * 2 * TQ + (paired && (he & kParityBit) ? TQ : 0);
      it.P0 = r0 + a.q_offset;
      it.last_pos = min(a.Nq, r0 + (paired ? TQ : 2 * TQ)) - 1 + a.q_offset;
      it.tq1 = it.P0 / TK + 1;
      it.ngather = 0;
      it.per = 1;
      it.n0 = it.n1 = 0;
      it.l0 = it.l1 = nullptr;

      const uint16_t* kbp = a.k + ((size_t)(b * a.Hkv + it.kvh) * a.Nk) * 128;
      const uint16_t* vbp = a.v + ((size_t)(b * a.Hkv + it.kvh) * a.Nk) * 128;
      const uint16_t* qbp = a.q + ((size_t)it.bh * a.Nq) * 128;

      const int qrow = r0 + (paired ? 0 : TQ * ih) + 32 * wr + qn;
      const int P0w = it.P0 + (paired ? 0 : TQ * ih); // first position of this wave's query tile
      const int R0w = P0w + 32 * wr;                   // position of this wave's first row
      const int iq = R0w + qn;                         // absolute position of this lane's row
      const bool row_ok = qrow < a.Nq;
      bf16x8 qf[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (row_ok) x = *(const u32x4*)(qbp + (size_t)qrow * 128 + 16 * ks + 8 * hh);
        qf[ks] = __builtin_bit_cast(bf16x8, x);
      }
      // The Q fragments are taken in right after an item's first K/V DMA is
      // issued (take_q below): the wait the compiler puts there covers the Q
      // loads and that DMA together.  Left to its first use inside a loop,
      // the wait would also drain the DMA of the next step.
      auto take_q = [&]() {
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) asm volatile("" :: "v"(qf[ks]));
      };
      f32x16 acc[4];
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[db][v] = 0.f;
      float m_run = -INFINITY, l_run = 0.f;

      // ---- pieces of the online softmax over 32-key sub-blocks
      // S^T = K Q^T for the 32 keys whose swizzled K rows start at kofs (the
      // eight K fragments are read first).
      auto qk32 = [&](uint32_t kofs, f32x16& sacc) {
#pragma unroll
        for (int v = 0; v < 16; ++v) sacc[v] = 0.f;
        u32x4 kf[8];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) kf[ks] = *(const lds_u32x4_t*)(uintptr_t)(kaddr[ks] + kofs);
        DSA_PRIO_HI();
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[ks]), qf[ks], sacc, 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        DSA_PRIO_LO();
      };
      // Scores of keys whose bit in M (bit c <-> key c of this lane's row) is
      // clear become -inf (bit select).
      auto mask32 = [&](f32x16& sacc, uint32_t M) {
        const uint32_t mk = M >> (4 * hh);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int pos = 8 * (v >> 2) + (v & 3);
          const uint32_t keep = (uint32_t)((int32_t)(mk << (31 - pos)) >> 31);   // all ones if kept
          sacc[v] = __uint_as_float((__float_as_uint(sacc[v]) & keep) | (0xff800000u & ~keep));
        }
      };
      // Row maximum of the raw scores in this lane (the row's other half is in lane l ^ 32).
      auto lane_max = [&](const f32x16& sacc) {
        float mx = fmaxf(fmaxf(sacc[0], sacc[1]), sacc[2]);
#pragma unroll
        for (int v = 3; v < 15; v += 2) mx = fmaxf(fmaxf(mx, sacc[v]), sacc[v + 1]);
        return fmaxf(mx, sacc[15]);
      };
      // Fold in a new scaled row maximum: rows rescale lazily, only when the
      // maximum grows by more than 8 (log2 units).  Returns the maximum the
      // weights are taken against.
      auto grow_to = [&](float mx) {
        {
          // rows live in lanes l and l ^ 32: swap halves and take the max
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
          mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * scale2;
        }
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
        return (m_run == -INFINITY) ? 0.f : m_run;
      };
      // bf16 weights exp2(s scale - muse) of one sub-block (the row sum takes
      // the same rounded values), then O^T += V^T P^T with the V rows at vofs
      // (two 16-key steps).
      auto pv32 = [&](const f32x16& sacc, float muse, uint32_t vofs, uint32_t halves = 3u) {
        const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
        uint32_t pk[8];
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[v], scale2, -muse));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[v + 1], scale2, -muse));
          const uint32_t pb = pack_bf16x2(p0, p1);
          l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pb), ones, l_run, false);
          pk[v >> 1] = pb;
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          // a 16-key half no lane of the wave kept has only zero weights: its
          // product adds nothing (halves: bit s2 set when some lane keeps one)
          if (!((halves >> s2) & 1u)) continue;
          u32x4 bx = {pk[4 * s2], pk[4 * s2 + 1], pk[4 * s2 + 2], pk[4 * s2 + 3]};
          const bf16x8 bop = __builtin_bit_cast(bf16x8, bx);
          // rows 16 s2 + v_row0 (a) and + 8 (b): the same swizzle as row v_row0
          short4_t ya[4], yb[4];
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            ya[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(uintptr_t)(vaddr[db] + vofs + 16 * s2 * 256));
            yb[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_short4_t*)(uintptr_t)(vaddr[db] + vofs + (16 * s2 + 8) * 256));
          }
          DSA_PRIO_HI();
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const short8_t ab = {ya[db][0], ya[db][1], ya[db][2], ya[db][3], yb[db][0], yb[db][1], yb[db][2], yb[db][3]};
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ab), bop, acc[db], 0, 0, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);
          __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);
          DSA_PRIO_LO();
        }
      };

      // One 32x32 sub-block: S^T over the 32 keys at kofs, the online softmax
      // under the mask M, O^T += V^T P^T with the V rows at vofs.
      // `sparse`: the mask is rarely full (Vertical-Slash), so it is applied
      // without first testing for a full mask.
      auto sub32 = [&](uint32_t kofs, uint32_t vofs, uint32_t M, bool sparse = false) {
        if (!row_ok) M = 0u;
        const uint64_t blo = __builtin_amdgcn_ballot_w64((M & 0xFFFFu) != 0u);
        const uint64_t bhi = __builtin_amdgcn_ballot_w64((M >> 16) != 0u);
        if ((blo | bhi) == 0) return;
        f32x16 sacc;
        qk32(kofs, sacc);
        if (sparse || __builtin_amdgcn_ballot_w64(M != ~0u) != 0) mask32(sacc, M);
        const uint32_t halves = (blo != 0 ? 1u : 0u) | (bhi != 0 ? 2u : 0u);
        const float muse = grow_to(lane_max(sacc));
        pv32(sacc, muse, vofs, halves);
      };

      // Two 32x32 sub-blocks of one 64-key tile (the second at + 32 rows): both
      // S^T products first, then one softmax over the 64 keys (one maximum, one
      // rescale decision), then both PV products.
      auto sub64 = [&](uint32_t kofs, uint32_t vofs, uint32_t M0, uint32_t M1) {
        if (!row_ok) { M0 = 0u; M1 = 0u; }
        const bool r0 = __builtin_amdgcn_ballot_w64(M0 != 0u) != 0;
        const bool r1 = __builtin_amdgcn_ballot_w64(M1 != 0u) != 0;
        if (!r0 && !r1) return;
        f32x16 sa0, sa1;
#pragma unroll
        for (int v = 0; v < 16; ++v) { sa0[v] = 0.f; sa1[v] = 0.f; }
        if (r0) qk32(kofs, sa0);
        if (r1) qk32(kofs + 8192, sa1);
        // an absent half has M = 0 in every lane: masked to -inf
        if (__builtin_amdgcn_ballot_w64(M0 != ~0u) != 0) mask32(sa0, M0);
        if (__builtin_amdgcn_ballot_w64(M1 != ~0u) != 0) mask32(sa1, M1);
        const float muse = grow_to(fmaxf(lane_max(sa0), lane_max(sa1)));
        if (r0) pv32(sa0, muse, vofs);
        if (r1) pv32(sa1, muse, vofs + 8192);
      };

      int gcursor = 0, gcount = 0;
      const uint32_t* cbits = nullptr;
      if (it.kind == 1 && ldc(a.win, 2 * (size_t)it.bh) >= 0) {
        // window head: key tiles of the sink [0, S) and of the window
        // [P0 - L + 1, last_pos], merged when they meet
        it.kind = 3;
        it.wlen = ldc(a.win, 2 * (size_t)it.bh);
        it.wsink = ldc(a.win, 2 * (size_t)it.bh + 1);
        const int tw0 = max(0, it.P0 - it.wlen + 1) / TK;
        const int tend = it.last_pos / TK + 1;
        const int ts = (min(it.wsink, it.last_pos + 1) + TK - 1) / TK;     // sink tiles [0, ts)
        if (it.wlen == 0) {
          it.n0 = ts;
          it.n1 = ts;
          it.nent = ts;
        } else if (ts >= tw0) {
          it.n0 = 0;
          it.n1 = 0;
          it.nent = tend;
        } else {
          it.n0 = ts;
          it.n1 = tw0;
          it.nent = ts + (tend - tw0);
        }
      } else if (it.kind == 1) {
        cbits = a.cbits + (size_t)it.bh * a.cw;
        gcount = min(ldc(a.cols_count, it.bh), a.cols_cap);
        // the arena is reused below: every wave has read the item number
        __syncthreads();

        // ---- Vertical-Slash sub-block steps over the head's step centres c,
        // descending (keys ascend): the step of centre c gives wave w the 32 keys
        // from P0 + 32 w - c, in ring slot sb + w (mod 5).  Within a run (the next
        // centre is c - 32) wave w next takes the block wave w + 1 used, so a step
        // brings in one new block, loaded one step ahead into the free slot
        // sb + 4.  The first step of a new run needs four new blocks: wave 0's
        // goes into the free slot during the step before, the other three into
        // the slots that step used, once every wave is done with them.
        const uint32_t* vbits = a.vbits + (size_t)it.bh * a.vw;
        const int32_t* cl = a.clist + (size_t)it.bh * a.ccap * 4;
        const int cmax = it.P0 + 127;            // wave 3's block still has a key >= 0
        int k = ldc(a.cle, (size_t)it.bh * a.ccap + min(cmax >> 5, a.ccap - 1)) - 1;
        if (k >= 0 && ldc(cl, 4 * (size_t)k) > cmax) --k;   // one centre at most per 32 positions
        auto issue_keys = [&](int k0, int slot) {
          const uint32_t lb = ring + (uint32_t)(slot * SLOT);
          if (k0 >= 0 && k0 + 32 <= a.Nk) {
            const char* kb = (const char*)(kbp + (size_t)k0 * 128);
            const char* vb = (const char*)(vbp + (size_t)k0 * 128);
            dma16x4(kb + off_k, kb + off_k + 4096, vb + off_v, vb + off_v + 4096, lb + w * 1024,
                    lb + (4 + w) * 1024, lb + 8192 + w * 1024, lb + 8192 + (4 + w) * 1024);
          } else {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const int r = 16 * j + rl;
              const int key = min(max(k0 + r, 0), a.Nk - 1);
              dma16(kbp + (size_t)key * 128 + swz_k(r, l & 15) * 8, lb + (4 * j + w) * 1024);
              dma16(vbp + (size_t)key * 128 + swz_v(r, l & 15) * 8, lb + 8192 + (4 * j + w) * 1024);
            }
          }
        };
        if (k >= 0) {
          const bool wave_on = R0w <= it.last_pos;
          // A step's entry {c, diagonal bits of offsets [c - 32, c + 31]} is
          // loaded two steps ahead and this wave's column words one step ahead
          // (scalar loads), so that their latency hides behind a step.
          struct ColWords {
            uint32_t c0, c1;
          };
          auto load_cols = [&](int c) {
            ColWords x = {0u, 0u};
            const int k0 = it.P0 + 32 * w - c;
            if (c >= 0 && wave_on && k0 + 31 >= 0) {
              // two adjacent words (the bitmap has a pad word past its last
              // one); c1 is used only when k0 >= 0
              const int cw = max(k0, 0) >> 5;
              x.c0 = ldc(vbits, cw);
              x.c1 = ldc(vbits, cw + 1);
            }
            return x;
          };
          const u32x4 none = {~0u, 0u, 0u, 0u};
          u32x4 ec = ldc4(cl, k);
          u32x4 en = k >= 1 ? ldc4(cl, k - 1) : none;
          int sb = 0;
          for (int i = 0; i <= 3; ++i) issue_keys(it.P0 + 32 * i - (int)ec[0], i);
          take_q();
          ColWords wc = load_cols((int)ec[0]);
          while (true) {
            const int cc = (int)ec[0], cn = (int)en[0];
            const int k0 = it.P0 + 32 * w - cc;
            const bool active = wave_on && k0 + 31 >= 0;
            const bool run = cn >= 0 && cn == cc - 32;
            wait_vm();
            __syncthreads();                     // this step's blocks landed; the previous step is done
            if (run) issue_keys(it.P0 + 128 - cc, addmod5(sb, 4));      // the one new block of a run
            else if (cn >= 0) issue_keys(it.P0 - cn, addmod5(sb, 4));   // wave 0's block of the next run
            if (active) {
              // lane row r sees offsets cc + r - j for keys j = 0..31: bits
              // 32 + r - j of the entry's window
              const uint64_t dwin = ((uint64_t)ec[2] << 32) | ec[1];
              uint32_t M = __builtin_bitreverse32((uint32_t)(dwin >> (1 + qn)));
              if (k0 >= 0) {
                M |= (uint32_t)((((uint64_t)wc.c1 << 32) | wc.c0) >> (k0 & 31));
              } else {
                M = (M | (wc.c0 << (-k0))) & (~0u << (-k0));
              }
              if (cc < 31) M &= causal_mask32(qn + cc);
              const int sl = addmod5(sb, w);
              sub32(sl * SLOT, sl * SLOT + 8192, M, true);
            }
            if (cn >= 0 && !run) {
              // Before a new run: its other three blocks go into the slots of
              // this step, once every wave is done with them.
              __syncthreads();
#pragma unroll
              for (int v = 1; v <= 3; ++v) issue_keys(it.P0 + 32 * v - cn, umod5(sb + 4 + v));
            }
            // The next step's words and the entry after it, issued once this
            // step's LDS reads are done: scalar loads and LDS reads share one
            // counter, so issued earlier, the step's first LDS wait would also
            // wait for them.  Here their latency overlaps the next step's DMA
            // wait and barrier.
            const ColWords wn = load_cols(cn);
            const u32x4 enn = k >= 2 ? ldc4(cl, k - 2) : none;
            if (--k < 0) break;
            sb = run ? addmod5(sb, 1) : addmod5(sb, 4);
            ec = en;
            en = enn;
            wc = wn;
          }
        }
        __syncthreads();                         // the slots are free for the gather phase
      } else if (SMALL && it.kind == 2 && a.block == 16 && it.last_pos / 16 < kPairBlocks) {
        // Blocks of 16, gathered per item in pairs: the item's eight query
        // blocks mark every 16-key block they selected (bit q for query block
        // q), the marked blocks are compacted into one ascending list, and
        // each two consecutive list entries, adjacent in key space or not, fill
        // one 32-key unit of the ring (keys 0-15 from the first, 16-31 from the
        // second).  Query blocks of an item mostly select the same blocks, so
        // a unit is mostly full for both query blocks of a wave, where a
        // 32-key unit of key space would often carry one selected half.
        __syncthreads();                         // every wave has read the item number; the arena is free
        const int nb = it.last_pos / 16 + 1;     // 16-key blocks the item's rows can see
        uint8_t* const bmask = (uint8_t*)(s_lds + OFF_BMASK);
        uint32_t* const bmask32 = (uint32_t*)bmask;
        uint32_t* const blist = (uint32_t*)(s_lds + OFF_BLIST);
        for (int i = tid; i < (nb + 3) / 4; i += NT) bmask32[i] = 0u;
        __syncthreads();
        {
          const int I0 = it.P0 / 16;
          for (int q = w; q < 8; q += 4) {
            const int I = I0 + q;                // absolute query block
            const int Ir = I - a.qb0;            // its row of the chunk's lists
            if (Ir >= a.nqb || I * 16 > it.last_pos) continue;
            const int32_t* li = a.bidx + ((size_t)it.bh * a.nqb + Ir) * a.bcap;
            const int n = min(ldc(a.bcount, (size_t)it.bh * a.nqb + Ir), a.bcap);
            for (int x = l; x < n; x += 64) {
              const int J = li[x];
              if (J < 0 || J >= nb) continue;   // out of range, or after the item's last row
              atomicOr(&bmask32[J >> 2], (1u << q) << (8 * (J & 3)));
            }
          }
        }
        __syncthreads();
        int nlist = 0;
        for (int j0 = 0; j0 < nb; j0 += NT) {
          const int J = j0 + tid;
          const uint32_t m = J < nb ? (uint32_t)bmask[J] : 0u;
          const uint64_t bal = __builtin_amdgcn_ballot_w64(m != 0u);
          if (l == 0) s_misc[1 + w] = __popcll(bal);
          __syncthreads();
          int off = nlist;
          for (int i = 0; i < w; ++i) off += s_misc[1 + i];
          if (m != 0u) blist[off + ballot_rank(bal)] = (uint32_t)J | (m << 16);
          nlist += s_misc[1] + s_misc[2] + s_misc[3] + s_misc[4];
          __syncthreads();
        }
        // one unit from two blocks: rows 16 j + rl of the slot from block Jj
        auto issue_pair = [&](int J0, int J1, uint32_t lb) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int r = 16 * j + rl;
            const int key = min(16 * (j ? J1 : J0) + rl, a.Nk - 1);
            dma16(kbp + (size_t)key * 128 + swz_k(r, l & 15) * 8, lb + (4 * j + w) * 1024);
            dma16(vbp + (size_t)key * 128 + swz_v(r, l & 15) * 8, lb + 8192 + (4 * j + w) * 1024);
          }
        };
        // entry 2 i + 1 of an odd list is absent: block 0, no query block
        auto entry = [&](int x) { return x < nlist ? blist[x] : 0u; };
        const int npair = (nlist + 1) / 2;
        if (npair > 0) issue_pair((int)(entry(0) & 0xFFFFu), (int)(entry(1) & 0xFFFFu), ring);
        take_q();
        const int qb = (32 * w + qn) / 16;       // this lane's query block within the item
        auto causal16 = [](int top) -> uint32_t {   // bits c <= top of 16
          return top < 0 ? 0u : top >= 15 ? 0xFFFFu : (2u << top) - 1u;
        };
        for (int i = 0; i < npair; ++i) {
          const uint32_t e0 = entry(2 * i), e1 = entry(2 * i + 1);
          wait_vm();
          __syncthreads();                       // unit i landed; every wave is done with unit i - 1
          if (i + 1 < npair)
            issue_pair((int)(entry(2 * i + 2) & 0xFFFFu), (int)(entry(2 * i + 3) & 0xFFFFu),
                       ring + (uint32_t)(((i + 1) & 1) * SLOT));
          const int J0 = (int)(e0 & 0xFFFFu), J1 = (int)(e1 & 0xFFFFu);
          uint32_t M = (((e0 >> (16 + qb)) & 1u) ? causal16(iq - 16 * J0) : 0u) |
                       ((((e1 >> (16 + qb)) & 1u) ? causal16(iq - 16 * J1) : 0u) << 16);
          const uint32_t st = (uint32_t)((i & 1) * SLOT);
          sub32(st, st + 8192, M);
        }
        it.kind = 4;                             // no tile steps for this item
      } else if (SMALL && it.kind == 2 && a.block < TK && it.last_pos / 32 < kSmallUnits) {
        // Blocks of 16 or 32, gathered per item: the item's query blocks (8 of
        // 16 rows or 4 of 32) mark the 16-key halves of every 32-key unit they
        // selected in a per-unit mask (16 bits: query block q, half h at bit
        // 2 q + h); the marked units are compacted into one ascending list and
        // streamed through a two-stage ring, each unit's K and V loaded once for
        // all four waves.  A wave computes a unit for the rows of its query
        // blocks that selected it (its mask bits, and causal), so the softmax of
        // every row is merged on chip across the units it uses.
        __syncthreads();                         // every wave has read the item number; the arena is free
        const int nu = it.last_pos / 32 + 1;     // 32-key units the item's rows can see
        uint16_t* const umask = (uint16_t*)(s_lds + OFF_UMASK);
        uint32_t* const ulist = (uint32_t*)(s_lds + OFF_ULIST);
        uint32_t* const umask32 = (uint32_t*)umask;
        for (int i = tid; i < (nu + 1) / 2; i += NT) umask32[i] = 0u;
        __syncthreads();
        {
          const int sh = a.block == 16 ? 1 : 0;  // list entry J lies in unit J >> sh
          const int nq_item = 2 * TQ / a.block;
          const int I0 = it.P0 / a.block;
          for (int q = w; q < nq_item; q += 4) {
            const int I = I0 + q;                // absolute query block
            const int Ir = I - a.qb0;            // its row of the chunk's lists
            if (Ir >= a.nqb || I * a.block > it.last_pos) continue;
            const int32_t* li = a.bidx + ((size_t)it.bh * a.nqb + Ir) * a.bcap;
            const int n = min(ldc(a.bcount, (size_t)it.bh * a.nqb + Ir), a.bcap);
            for (int x = l; x < n; x += 64) {
              const int J = li[x];
              const int u = J >> sh;
              if (J < 0 || u >= nu) continue;   // out of range, or after the item's last row
              const uint32_t bits = sh ? (1u << (2 * q + (J & 1))) : (3u << (2 * q));
              atomicOr(&umask32[u >> 1], bits << (16 * (u & 1)));
            }
          }
        }
        __syncthreads();
        int nlist = 0;
        for (int u0 = 0; u0 < nu; u0 += NT) {
          const int u = u0 + tid;
          const uint32_t m = u < nu ? (uint32_t)umask[u] : 0u;
          const uint64_t bal = __builtin_amdgcn_ballot_w64(m != 0u);
          if (l == 0) s_misc[1 + w] = __popcll(bal);
          __syncthreads();
          int off = nlist;
          for (int i = 0; i < w; ++i) off += s_misc[1 + i];
          if (m != 0u) ulist[off + ballot_rank(bal)] = (uint32_t)u | (m << 16);
          nlist += s_misc[1] + s_misc[2] + s_misc[3] + s_misc[4];
          __syncthreads();
        }
        auto issue_unit = [&](int u, uint32_t lb) {
          const int k0 = 32 * u;
          if (k0 + 32 <= a.Nk) {
            const char* kb = (const char*)(kbp + (size_t)k0 * 128);
            const char* vb = (const char*)(vbp + (size_t)k0 * 128);
            dma16x4(kb + off_k, kb + off_k + 4096, vb + off_v, vb + off_v + 4096, lb + w * 1024,
                    lb + (4 + w) * 1024, lb + 8192 + w * 1024, lb + 8192 + (4 + w) * 1024);
          } else {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const int r = 16 * j + rl;
              const int key = min(k0 + r, a.Nk - 1);
              dma16(kbp + (size_t)key * 128 + swz_k(r, l & 15) * 8, lb + (4 * j + w) * 1024);
              dma16(vbp + (size_t)key * 128 + swz_v(r, l & 15) * 8, lb + 8192 + (4 * j + w) * 1024);
            }
          }
        };
        if (nlist > 0) issue_unit((int)(ulist[0] & 0xFFFFu), ring);
        take_q();
        // this lane's query block within the item and the shift of its mask bits
        const int qsh = 2 * ((32 * w + qn) / a.block);
        for (int i = 0; i < nlist; ++i) {
          const uint32_t e = ulist[i];
          wait_vm();
          __syncthreads();                       // unit i landed; every wave is done with unit i - 1
          if (i + 1 < nlist) issue_unit((int)(ulist[i + 1] & 0xFFFFu), ring + (uint32_t)(((i + 1) & 1) * SLOT));
          const int u = (int)(e & 0xFFFFu);
          const uint32_t g = (e >> (16 + qsh)) & 3u;
          uint32_t M = ((g & 1u) ? 0x0000FFFFu : 0u) | ((g & 2u) ? 0xFFFF0000u : 0u);
          M &= causal_mask32(iq - 32 * u);
          const uint32_t st = (uint32_t)((i & 1) * SLOT);
          sub32(st, st + 8192, M);
        }
        it.kind = 4;                             // no tile steps for this item
      } else if (SMALL && it.kind == 2 && a.block < TK) {
        // Blocks of 16 or 32 on very long sequences (more 32-key units than the
        // gather masks hold): each wave walks the lists of its own 32 rows (one
        // list for block 32, two for block 16) 32 keys at a time through its own
        // 16 KB slot of the arena, with no workgroup barrier.
        __syncthreads();                         // every wave has read the item number
        const uint32_t wslot = (uint32_t)(w * SLOT);
        if (R0w <= it.last_pos) {
          const int Ir = R0w / a.block - a.qb0;  // the list row of the wave's first query block
          const int32_t* la = a.bidx + ((size_t)it.bh * a.nqb + Ir) * a.bcap;
          const int na = min(ldc(a.bcount, (size_t)it.bh * a.nqb + Ir), a.bcap);
          // rows 16-31: the next query block
          const bool two = a.block == 16 && Ir + 1 < a.nqb && R0w + 16 < a.Nq + a.q_offset;
          const int32_t* lb = two ? a.bidx + ((size_t)it.bh * a.nqb + Ir + 1) * a.bcap : la;
          const int nb = two ? min(ldc(a.bcount, (size_t)it.bh * a.nqb + Ir + 1), a.bcap) : 0;
          const int sh = a.block == 16 ? 1 : 0;   // list entry J lies in 32-key unit J >> sh
          constexpr int NONE = 0x7fffffff;
          int ia = 0, ib = 0;
          int ja = na > 0 ? ldc(la, 0) : NONE, jb = nb > 0 ? ldc(lb, 0) : NONE;
          const uint32_t lslot = ring + wslot;
          while (true) {
            const int u = min(ja == NONE ? NONE : (ja >> sh), jb == NONE ? NONE : (jb >> sh));
            if (u == NONE) break;
            // the 16-key halves of unit u that rows 0-15 (ga) and rows 16-31 (gb) use
            uint32_t ga = 0u, gb = 0u;
            while (ja != NONE && (ja >> sh) == u) {
              ga |= sh ? (1u << (ja & 1)) : 3u;
              ++ia;
              ja = ia < na ? ldc(la, ia) : NONE;
            }
            while (jb != NONE && (jb >> sh) == u) {
              gb |= 1u << (jb & 1);
              ++ib;
              jb = ib < nb ? ldc(lb, ib) : NONE;
            }
            if (!sh) gb = ga;                    // block 32: one list for all 32 rows
            if (u < 0) continue;                 // out-of-range block ids contribute nothing
            // K and V rows 32 u .. 32 u + 31 (clamped into the key range) into the
            // slot: instruction i fills rows 4 i .. 4 i + 3, lane l row 4 i + l / 16
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const int r = 4 * i + (l >> 4);
              const int key = min(max(32 * u + r, 0), a.Nk - 1);
              dma16(kbp + (size_t)key * 128 + swz_k(r, l & 15) * 8, lslot + i * 1024);
              dma16(vbp + (size_t)key * 128 + swz_v(r, l & 15) * 8, lslot + 8192 + i * 1024);
            }
            wait_vm();
            const uint32_t g = qn < 16 ? ga : gb;
            uint32_t M = ((g & 1u) ? 0x0000FFFFu : 0u) | ((g & 2u) ? 0xFFFF0000u : 0u);
            M &= causal_mask32(iq - 32 * u);
            sub32(wslot, wslot + 8192, M);
          }
        }
        it.kind = 4;                             // no tile steps for this item
      } else if (it.kind == 2) {
        it.per = a.block / TK;
        const int I0 = it.P0 / a.block - a.qb0;  // the list row of the item's first query block
        // A pair's second query tile of the last pair of tiles can lie past the
        // last query (an odd number of tiles): then the item has no rows and
        // reads no list (its query block would be past the heads' lists).
        const bool has_rows = r0 < a.Nq;
        it.l0 = a.bidx + ((size_t)bh0 * a.nqb + (has_rows ? I0 : 0)) * a.bcap;
        it.n0 = has_rows ? min(ldc(a.bcount, (size_t)bh0 * a.nqb + I0), a.bcap) : 0;
        it.l1 = it.l0;
        if (paired) {
          // the second head's list of the same query block
          it.l1 = a.bidx + ((size_t)(bh0 + 1) * a.nqb + (has_rows ? I0 : 0)) * a.bcap;
          it.n1 = has_rows ? min(ldc(a.bcount, (size_t)(bh0 + 1) * a.nqb + I0), a.bcap) : 0;
        } else if (it.per == 1 && I0 + 1 < a.nqb && r0 + TQ < a.Nq) {
          it.l1 = a.bidx + ((size_t)it.bh * a.nqb + I0 + 1) * a.bcap;
          it.n1 = min(ldc(a.bcount, (size_t)it.bh * a.nqb + I0 + 1), a.bcap);
        }
      }

      for (;;) {
        if (SMALL && it.kind == 4) break;
        if (it.kind == 1) {
          // stage this pair's columns j <= last_pos, except those every wave's
          // sub-blocks already cover; cov bit w marks a column wave w covered
          // (or one after all of wave w's rows)
          const int32_t* cols = a.cols + (size_t)it.bh * a.cols_cap;
          int staged = 0;
          while (gcursor < gcount && staged <= GCAP - NT) {
            const int idx = gcursor + tid;
            bool keep = false;
            int j = 0;
            uint32_t cov = 0xFu;
            if (idx < gcount) {
              j = cols[idx];
              if (j >= 0 && j <= it.last_pos) {
                cov = 0u;
#pragma unroll
                for (int w4 = 0; w4 < 4; ++w4) {
                  // wave w4's block holds key j at the steps of centres in [lo, lo + 31]
                  const int lo = it.P0 + 32 * w4 - j;
                  const bool c = lo + 31 < 0 || it.P0 + 32 * w4 > it.last_pos ||
                                 range_any(cbits, max(lo, 0), min(lo + 31, 32 * a.cw - 1));
                  cov |= (c ? 1u : 0u) << w4;
                }
                keep = cov != 0xFu;
              }
            }
            const uint64_t bal = __builtin_amdgcn_ballot_w64(keep);
            __syncthreads();
            if (l == 0) s_misc[1 + w] = __popcll(bal);
            __syncthreads();
            int off = staged;
            for (int i = 0; i < w; ++i) off += s_misc[1 + i];
            if (keep) {
              s_cols[off + ballot_rank(bal)] = j;
              s_cov[off + ballot_rank(bal)] = (uint8_t)cov;
            }
            staged += s_misc[1] + s_misc[2] + s_misc[3] + s_misc[4];
            gcursor += NT;
            const int lastc = cols[min(gcursor, gcount) - 1];
            if (lastc > it.last_pos) gcursor = gcount;
          }
          __syncthreads();
          it.ngather = staged;
          it.nent = (staged + TK - 1) / TK;
        } else if (it.kind == 2) {
          // per == 2: one shared list; per == 1: the cursor merges two lists and
          // stops when both are exhausted (nent is only an upper bound)
          it.nent = it.per == 2 ? 2 * it.n0 : it.n0 + it.n1;
        } else if (it.kind == 0) {
          it.nent = it.last_pos / TK + 1;
        }

        Cursor cc;
        cursor_init(it, cc);
        Entry cur;
        cur.kind = -1;
        cur.flags = 0;
        bool have = cursor_has_next(it, cc);
        if (have) {
          cur = cursor_next(it, cc);
          issue_tile<false>(kbp, a.Nk, cur, s_cols, ring, w, l, off_k);
          issue_tile<true>(vbp, a.Nk, cur, s_cols, ring + TK * 256, w, l, off_v);
          cursor_fetch(it, cc);
        }
        take_q();
        // One tile step on ring stage `stage` (a compile-time constant, so every
        // LDS address below is a lane-constant register plus an immediate).
        auto step = [&](auto stage_c) {
          constexpr int stage = decltype(stage_c)::value;
          // ---- this wave's view of the entry (key tiles wholly after its rows,
          // and waves with no row inside the chunk, skip)
          int mode;
          if (!((cur.flags >> ih) & 1) || (cur.kind == 0 && cur.kt * TK > P0w + TQ - 1) || R0w > it.last_pos)
            mode = M_SKIP;
          else if (cur.kind == 1) mode = M_GATHER;
          else if (it.kind == 3)
            // unmasked if every key is causal and inside the window or the sink for all the wave's rows
            mode = (cur.kt * TK + TK - 1 <= R0w && (R0w + 31 - cur.kt * TK <= it.wlen - 1 || cur.kt * TK + TK <= it.wsink))
                       ? M_NONE : M_WIN;
          else mode = (cur.kt * TK + TK - 1 > P0w) ? M_CAUSAL : M_NONE;
          wait_vm();
          __syncthreads();                       // tile n landed; every wave is done with tile n - 1
          Entry nxt;
          nxt.kind = -1;
          nxt.flags = 0;
          const bool have_n = cursor_has_next(it, cc);
          if (have_n) {
            nxt = cursor_next(it, cc);
            issue_tile<false>(kbp, a.Nk, nxt, s_cols, ring + (stage ^ 1) * 2 * TK * 256, w, l, off_k);
            issue_tile<true>(vbp, a.Nk, nxt, s_cols, ring + ((stage ^ 1) * 2 + 1) * TK * 256, w, l, off_v);
          }

          uint32_t Mk[2];
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            // ---- mask over keys 32 kb .. +31 (bit c <-> key kt*64 + 32 kb + c)
            const int ktop = iq - cur.kt * TK - 32 * kb;   // keys c <= ktop are causal
            uint32_t M = ~0u;
            if (mode == M_SKIP) {
              M = 0u;
            } else if (mode == M_CAUSAL) {
              M = causal_mask32(ktop);
            } else if (mode == M_WIN) {
              // keys c <= ktop, and c >= ktop - (L - 1) (window) or below the sink
              const int c0 = ktop - it.wlen + 1;
              const uint32_t inwin = c0 <= 0 ? ~0u : (c0 >= 32 ? 0u : (~0u << c0));
              const int cs = it.wsink - (cur.kt * TK + 32 * kb);
              const uint32_t insink = cs >= 32 ? ~0u : (cs <= 0 ? 0u : ((1u << cs) - 1u));
              M = causal_mask32(ktop) & (inwin | insink);
            } else if (mode == M_GATHER) {
              // staged columns ascend: the keys <= iq are a prefix of the chunk
              const int base = cur.kt * TK + 32 * kb;
              const int cnt = max(0, min(32, cur.cnt - 32 * kb));
              if (cnt == 32 && s_cols[base + 31] <= iq) {
                M = ~0u;
              } else {
                int lo = 0, hi = cnt;
                while (lo < hi) {
                  const int mid = (lo + hi) >> 1;
                  if (s_cols[base + mid] <= iq) lo = mid + 1; else hi = mid;
                }
                M = lo >= 32 ? ~0u : ((1u << lo) - 1u);
              }
              // columns this wave's sub-blocks already visited
              const bool ex = (s_cov[base + (l & 31)] >> w) & 1u;
              M &= ~(uint32_t)__builtin_amdgcn_ballot_w64(ex);
            }
            Mk[kb] = M;
          }
          sub64(stage * 2 * TK * 256, (stage * 2 + 1) * TK * 256, Mk[0], Mk[1]);
          cursor_fetch(it, cc);                  // after the step's LDS reads (see Cursor)
          cur = nxt;
          have = have_n;
        };
        while (have) {
          step(std::integral_constant<int, 0>{});
          if (!have) break;
          step(std::integral_constant<int, 1>{});
        }
        if (!(it.kind == 1 && gcursor < gcount)) break;
        __syncthreads();                         // the last tile's gathered columns are no longer read
      }

      // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2
      const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
      const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
      if (row_ok) {
        const size_t obase = ((size_t)it.bh * a.Nq + qrow) * 128;
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
          a.lse[(size_t)it.bh * a.Nq + qrow] =
              l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
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
  int sw, vw, cw, ND;
  size_t off_s, off_v, off_c, off_cc, off_ctr, off_cl, off_cle, off_win, total_words;
};

VsLayout vs_layout(int B, int H, int Nk) {
  VsLayout L;
  L.sw = (Nk + 31) / 32 + 5;
  L.vw = (Nk + 31) / 32 + 2;
  L.ND = (Nk + 30) / 32 + 1;     // centres lie in [0, Nk + 30]: at most one per 32 positions
  L.cw = L.ND;
  const size_t nbh = (size_t)B * H;
  size_t off = 0;
  L.off_ctr = off; off += 64;
  L.off_s = off; off += nbh * L.sw;
  L.off_v = off; off += nbh * L.vw;
  L.off_c = off; off += nbh * L.cw;
  L.off_cc = off; off += nbh;
  L.total_words = off;          // region zeroed before every call
  off = (off + 3) & ~size_t(3);  // 16-byte entries, read as one scalar load each
  L.off_cl = off; off += nbh * L.ND * 4;
  L.off_cle = off; off += nbh * L.ND;
  L.off_win = off; off += nbh * 2;
  (void)off;
  return L;
}

}  // namespace

// Scratch of the attention entry point that allocates nothing (for callers
// that cannot call hipMalloc): one copy of this array lives on every device the
// library runs on, until the process ends.  Host code never uses the array's
// name as an address: the per-device address comes from hipGetSymbolAddress,
// taken once per device with that device current.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

hipError_t static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

size_t attn_workspace_bytes(int B, int H, int Nk) {
  VsLayout L = vs_layout(B, H, Nk);
  return (L.off_win + (size_t)B * H * 2) * 4 + 256;
}

hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  int blocks = (int)std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(zero_u32_kernel, dim3(blocks), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

hipError_t launch_attention(AttnArgs& a, void* ws, hipStream_t st) {
  const int T = (a.Nq + TQ - 1) / TQ;
  const int T2 = (T + 1) / 2;
  VsLayout L = vs_layout(a.B, a.H, a.Nk);
  uint32_t* base = (uint32_t*)ws;
  a.counters = (int32_t*)(base + L.off_ctr);
  a.sbits = base + L.off_s;
  a.vbits = base + L.off_v;
  a.cbits = base + L.off_c;
  a.ccount = (int32_t*)(base + L.off_cc);
  a.clist = (int32_t*)(base + L.off_cl);
  a.cle = (int32_t*)(base + L.off_cle);
  a.win = (int32_t*)(base + L.off_win);
  a.sw = L.sw; a.vw = L.vw; a.cw = L.cw; a.ccap = L.ND;

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
    hipLaunchKernelGGL(vs_centres_kernel, dim3(vs.n), dim3(256), 0, st, a, vs, L.ND);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }

  // Queue assignment.  Each head's cost is estimated (key tiles over all its
  // query tiles); the Q heads that share a KV head go to the same queue, so
  // that the items running together on one XCD stream the same K/V tiles
  // through that XCD's L2.  Groups are placed longest first into the
  // least-loaded queue; within a queue, consecutive items are the group's
  // heads at the same query rows.
  // Block heads with 64-key blocks come in pairs of neighbouring heads of one
  // KV group where they can: an item of a pair is one query tile of both heads
  // (waves 0-1 the first head, 2-3 the second), which merges the two heads'
  // lists of the same query block, rather than two query tiles of one head.
  // Heads that share their K choose many of the same key blocks, so more of
  // the merged tiles serve all four waves.  A pair is listed twice, once per
  // parity of its query tiles, so that every entry still has T2 items.
  struct HC { double cost; int bh; int enc; };
  std::vector<HC> heads;
  const int rep_h = a.H / a.Hkv;
  for (int b = 0; b < a.B; ++b)
    for (int h = 0; h < a.H; ++h) {
      const int kd = a.kind[h];
      if (kd < 0 || kd > 2) continue;
      const bool pair = kd == 2 && a.block == TK && h + 1 < a.H && a.kind[h + 1] == 2 && h / rep_h == (h + 1) / rep_h;
      if (pair) {
        const double per = std::min<double>(a.bcap * (a.block / TK), 0.5 * a.Nk / TK);
        const int bh = b * a.H + h;
        heads.push_back({per * T, bh, bh | kPairBit});
        heads.push_back({per * T, bh, bh | kPairBit | kParityBit});
        ++h;
        continue;
      }
      double per;
      if (kd == 0) per = 0.5 * (a.Nk / (double)TK);
      else if (kd == 2 && a.block < TK) per = std::min<double>(a.bcap * (32.0 / a.block), 0.5 * a.Nk / TK);
      else if (kd == 2) per = std::min<double>(a.bcap * (a.block / TK), 0.5 * a.Nk / TK);
      else per = std::min<double>(0.5 * a.Nk / TK, 2.0 * a.diags_cap / TK + 1 + a.cols_cap / (double)TK);
      heads.push_back({per * T, b * a.H + h, b * a.H + h});
    }
  if ((e = launch_token_attention(a, st)) != hipSuccess) return e;
  if (heads.empty()) return hipSuccess;
  const int rep = a.H / a.Hkv;
  struct GC { double cost; int key; std::vector<int> bh; };
  std::vector<GC> groups;
  for (const HC& x : heads) {
    const int key = (x.bh / a.H) * a.Hkv + (x.bh % a.H) / rep;   // b * Hkv + kv head
    if (groups.empty() || groups.back().key != key) groups.push_back({0.0, key, {}});
    groups.back().cost += x.cost;
    groups.back().bh.push_back(x.enc);
  }
  std::stable_sort(groups.begin(), groups.end(), [](const GC& x, const GC& y) { return x.cost > y.cost; });
  Sched sc;
  sc.T2 = T2;
  sc.nq = std::min<int>(kMaxQueues, (int)groups.size());
  std::vector<std::vector<int>> qh(sc.nq);
  std::vector<double> load(sc.nq, 0.0);
  for (const GC& x : groups) {
    int best = 0;
    for (int g = 1; g < sc.nq; ++g) if (load[g] < load[best]) best = g;
    load[best] += x.cost;
    for (int bh : x.bh) qh[best].push_back(bh);
  }
  int pos = 0;
  for (int g = 0; g < sc.nq; ++g) {
    sc.qstart[g] = pos;
    std::sort(qh[g].begin(), qh[g].end());
    for (int bh : qh[g]) sc.heads[pos++] = (int16_t)bh;
  }
  sc.qstart[sc.nq] = pos;

  const long items = (long)heads.size() * T2;
  long grid = std::min<long>(items, (long)cu_count() * 2);
  grid = std::max<long>(sc.nq, (grid / sc.nq) * sc.nq);
  bool small = false;
  if (a.block > 0 && a.block < TK)
    for (int h = 0; h < a.H; ++h) small = small || a.kind[h] == 2;
  if (small) hipLaunchKernelGGL(attn_kernel<true>, dim3((unsigned)grid), dim3(NT), 0, st, a, sc);
  else hipLaunchKernelGGL(attn_kernel<false>, dim3((unsigned)grid), dim3(NT), 0, st, a, sc);
  return hipGetLastError();
}

}  // namespace dsa
