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
//  * Vertical-Slash heads: a compile step turns the column / diagonal lists into
//    bitmaps and the set A of key-tile offsets a crossed by a selected diagonal
//    (pairs use A u (A+1)).  Strip tiles carry an exact per-element mask
//    (diagonal bit | column bit, causal); columns outside all strip tiles are
//    gathered 64 at a time.  Every selected (i, j) is visited exactly once.
//  * Persistent workgroups pull items from per-XCD queues (longest rows first)
//    and steal from other queues when their own is empty.
#include "common.h"
#include "internal.h"

#include <algorithm>
#include <type_traits>
#include <vector>

namespace dsa {
namespace {

constexpr int TQ = 64;       // rows per query tile
constexpr int TK = 64;       // keys per key tile
constexpr int NT = 256;      // 4 waves: two query tiles x two 32-row halves
constexpr int GCAP = 2048;   // gathered columns staged per round

enum { M_NONE = 0, M_CAUSAL = 1, M_VS = 2, M_GATHER = 3, M_SKIP = 4 };

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

// Key-tile offsets a in [0, TA).  a is in A iff a selected diagonal crosses
// some pair (query tile t, key tile t - a), i.e. offsets [64a - 63, 64a + 63]
// hold a set bit; a >= 1 is "full" (no mask needed) iff all of them are set.
// A query-tile pair (t, t + 1) visits key tiles t + 1 - a for a in A2 = A u (A+1);
// A2 is written as an ascending list and as a bitmap.
__global__ __launch_bounds__(256) void vs_tiles_kernel(AttnArgs a, BhList L, int TA) {
  const int bh = L.bh[blockIdx.x];
  const uint32_t* sb = a.sbits + (size_t)bh * a.sw + 2;     // unpadded view
  uint32_t* fb = a.fbits + (size_t)bh * a.aw;
  uint32_t* a2b = a.a2bits + (size_t)bh * a.aw;
  int32_t* al = a.a2list + (size_t)bh * a.acap;
  int32_t* ale = a.a2le + (size_t)bh * a.acap;
  __shared__ int s_wave[4];
  __shared__ int s_base;
  if (threadIdx.x == 0) s_base = 0;
  __syncthreads();
  const int w = threadIdx.x >> 6;
  auto in_a = [&](int t) {
    if (t < 0 || t >= TA) return false;
    const int lo = max(0, 64 * t - 63), hi = min(a.Nk - 1, 64 * t + 63);
    return lo <= hi && range_any(sb, lo, hi);
  };
  for (int a0 = 0; a0 < TA; a0 += 256) {
    const int t = a0 + threadIdx.x;
    bool in2 = false;
    if (t < TA) {
      const bool inA = in_a(t);
      in2 = inA || in_a(t - 1);
      if (inA && t >= 1) {
        const int lo = 64 * t - 63, hi = min(a.Nk - 1, 64 * t + 63);
        if (lo <= hi && range_all(sb, lo, hi)) atomicOr(&fb[t >> 5], 1u << (t & 31));
      }
      if (in2) atomicOr(&a2b[t >> 5], 1u << (t & 31));
    }
    const uint64_t bal = __builtin_amdgcn_ballot_w64(in2);
    const uint32_t rank = ballot_rank(bal);
    if ((threadIdx.x & 63) == 0) s_wave[w] = __popcll(bal);
    __syncthreads();
    int off = s_base;
    for (int i = 0; i < w; ++i) off += s_wave[i];
    if (in2) al[off + rank] = t;
    if (t < TA) ale[t] = off + rank + (in2 ? 1 : 0);     // #{a in A2 : a <= t}
    __syncthreads();
    if (threadIdx.x == 0) s_base += s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.a2count[bh] = s_base;
}

// ---------------------------------------------------------------- main kernel
typedef __attribute__((address_space(3))) void lds_void_t;
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;
typedef __attribute__((address_space(3))) char lds_char_t;

// 16 bytes per lane straight from global memory into LDS; lane l of the wave
// lands at LDS byte address lds_addr + 16 l (lds_addr is wave-uniform).
// Issued from inline assembly on purpose: the compiler does not track these
// LDS writes, so it adds no wait of its own before the LDS reads of the other
// ring stage (its own wait would drain the DMA just issued for the next tile).
// The explicit vmcnt wait at the top of each step orders a tile's DMA before
// the reads of its stage; the "memory" clobber keeps the compiler from moving
// LDS accesses across the issue.  The instruction has no register results.
// M0 (the LDS base) is saved and restored around it, so the compiler's view of
// M0 never changes.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_addr) {
  uint32_t save;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\t"
               "s_mov_b32 m0, %0"
               : "=&s"(save) : "v"(g), "s"(lds_addr) : "memory");
}
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
__device__ __forceinline__ bool test_bit_c(const uint32_t* bm, int i) { return (ldc(bm, i >> 5) >> (i & 31)) & 1u; }

// One entry of a pair's tile stream.
struct Entry {
  int kind;    // 0 key tile, 1 gather chunk, -1 none
  int kt;      // key tile index, or gather chunk index
  int cnt;     // valid keys of a gather chunk
  int flags;   // bit h: query tile h of the pair uses this entry
  int full;    // VS strip tile: bit h set if every entry is selected for query tile h
};

struct Item {
  int bh, kvh, kind, P0, last_pos, tq1;
  // VS
  const int32_t* a2;       // strip tile offsets (relative to tq1), ascending
  const uint32_t* fb;      // "full" bits of tile offsets
  int nstrip;
  // BLOCK
  const int32_t* l0;       // list of query block I0 (or of the shared block)
  const int32_t* l1;       // list of query block I0 + 1 (block 64 only)
  int n0, n1, per;
  // stream
  int nent, ngather;
};

// Cursor over a pair's entries.  The global-memory lookups of entry n + 1 are
// issued while entry n is being processed (one step of prefetch).
struct Cursor {
  int n;                   // index of the next entry
  int raw;                 // prefetched value for entry n (VS strip / shared block list)
  int i0, i1, x0, x1;      // two-list merge state (block 64): heads of both lists
  int x0n, x1n;            // prefetched successors of the heads
};

__device__ __forceinline__ int list_at(const int32_t* L, int n, int i) { return i < n ? ldc(L, i) : 0x7fffffff; }

__device__ __forceinline__ void cursor_init(const Item& it, Cursor& c) {
  c.n = 0;
  c.raw = 0;
  c.i0 = c.i1 = 0;
  c.x0 = c.x1 = c.x0n = c.x1n = 0x7fffffff;
  if (it.kind == 1) c.raw = it.nstrip > 0 ? ldc(it.a2, 0) : 0;
  else if (it.kind == 2 && it.per == 2) c.raw = it.n0 > 0 ? ldc(it.l0, 0) : 0;
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
  e.full = 0;
  const int n = c.n++;
  if (it.kind == 1) {
    if (n < it.nstrip) {
      // tile offset of query tile h of the pair is raw - 1 + h; offsets >= 1 may be full
      const int r = c.raw;
      e.kt = it.tq1 - r;
      if (r >= 2 && test_bit_c(it.fb, r - 1)) e.full |= 1;
      if (r >= 1 && test_bit_c(it.fb, r)) e.full |= 2;
      c.raw = (n + 1 < it.nstrip) ? ldc(it.a2, n + 1) : 0;
    } else {
      e.kind = 1;
      e.kt = n - it.nstrip;
      e.cnt = min(TK, it.ngather - e.kt * TK);
    }
  } else if (it.kind == 2 && it.per == 2) {
    e.kt = c.raw * 2 + (n & 1);
    if (n & 1) c.raw = ((n >> 1) + 1 < it.n0) ? ldc(it.l0, (n >> 1) + 1) : 0;
  } else if (it.kind == 2) {
    const int x = min(c.x0, c.x1);
    e.kt = x;
    e.flags = (c.x0 == x ? 1 : 0) | (c.x1 == x ? 2 : 0);
    if (c.x0 == x) { ++c.i0; c.x0 = c.x0n; c.x0n = list_at(it.l0, it.n0, c.i0 + 1); }
    if (c.x1 == x) { ++c.i1; c.x1 = c.x1n; c.x1n = list_at(it.l1, it.n1, c.i1 + 1); }
  } else {
    e.kt = n;
  }
  // out-of-range block ids or tiles beyond the pair's last row contribute nothing
  if (e.kind == 0 && (e.kt < 0 || e.kt * TK > it.last_pos)) e.flags = 0;
  return e;
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
// issues them ahead of the other waves' softmax work on the same SIMD.
#ifndef DSA_ATTN_SETPRIO
#define DSA_ATTN_SETPRIO 1
#endif
#if DSA_ATTN_SETPRIO
#define DSA_PRIO_HI() __builtin_amdgcn_s_setprio(1)
#define DSA_PRIO_LO() __builtin_amdgcn_s_setprio(0)
#else
#define DSA_PRIO_HI() ((void)0)
#define DSA_PRIO_LO() ((void)0)
#endif

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(DSA_ATTN_WAVES_PER_SIMD))) void attn_kernel(
    const AttnArgs a, const Sched sc) {
  __shared__ __align__(1024) char s_kv[2][2][TK * 256];   // [stage][0 = K, 1 = V]
  __shared__ int32_t s_cols[GCAP];
  __shared__ int s_misc[8];

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
  const int v_row0 = 4 * (G >> 1) + (si >> 2);           // + 32 kb + 16 s2 (+ 8)
  const int v_half = (si & 1) * 8;
  // LDS byte address of the ring; stage s, K (0) or V (1) at + (2 s + kv) * 16 KB
  const uint32_t ring = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_char_t*)&s_kv[0][0][0]);

  for (int qi = 0; qi < sc.nq; ++qi) {
    const int g = (myq + qi) % sc.nq;
    const int nh = sc.qstart[g + 1] - sc.qstart[g];
    const int nitems = nh * sc.T2;
    if (nh == 0) continue;
    while (true) {
      __syncthreads();
      if (tid == 0) s_misc[0] = atomicAdd(&a.counters[g], 1);
      __syncthreads();
      const int itn = s_misc[0];
      if (itn >= nitems) break;

      Item it;
      it.bh = sc.heads[sc.qstart[g] + itn % nh];
      const int b = it.bh / a.H, h = it.bh % a.H;
      it.kvh = h / rep;
      it.kind = a.kind[h];
      const int p = sc.T2 - 1 - itn / nh;
      const int r0 = p * 2 * TQ;
      it.P0 = r0 + a.q_offset;
      it.last_pos = min(a.Nq, r0 + 2 * TQ) - 1 + a.q_offset;
      it.tq1 = it.P0 / TK + 1;
      it.nstrip = 0;
      it.ngather = 0;
      it.per = 1;
      it.n0 = it.n1 = 0;
      it.a2 = nullptr;
      it.fb = nullptr;
      it.l0 = it.l1 = nullptr;

      const uint16_t* kbp = a.k + ((size_t)(b * a.Hkv + it.kvh) * a.Nk) * 128;
      const uint16_t* vbp = a.v + ((size_t)(b * a.Hkv + it.kvh) * a.Nk) * 128;
      const uint16_t* qbp = a.q + ((size_t)it.bh * a.Nq) * 128;

      const int qrow = r0 + TQ * ih + 32 * wr + qn;
      const int P0w = it.P0 + TQ * ih;                // first position of this wave's query tile
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
      // Take the Q fragments in before the tile loop: otherwise the compiler
      // waits for these loads at their first use inside the loop, where the
      // wait would also drain the K/V DMA in flight.
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) asm volatile("" :: "v"(qf[ks]));
      f32x16 acc[4];
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[db][v] = 0.f;
      float m_run = -INFINITY, l_run = 0.f;

      const uint32_t* sbits = nullptr;
      const uint32_t* vbits = nullptr;
      int gcursor = 0, gcount = 0;
      if (it.kind == 1) {
        it.a2 = a.a2list + (size_t)it.bh * a.acap;
        it.fb = a.fbits + (size_t)it.bh * a.aw;
        sbits = a.sbits + (size_t)it.bh * a.sw;
        vbits = a.vbits + (size_t)it.bh * a.vw;
        it.nstrip = ldc(a.a2le, (size_t)it.bh * a.acap + it.tq1);
        gcount = min(ldc(a.cols_count, it.bh), a.cols_cap);
      } else if (it.kind == 2) {
        it.per = a.block / TK;
        const int I0 = it.P0 / a.block;
        it.l0 = a.bidx + ((size_t)it.bh * a.nqb + I0) * a.bcap;
        it.n0 = min(ldc(a.bcount, (size_t)it.bh * a.nqb + I0), a.bcap);
        it.l1 = it.l0;
        if (it.per == 1 && I0 + 1 < a.nqb && r0 + TQ < a.Nq) {
          it.l1 = a.bidx + ((size_t)it.bh * a.nqb + I0 + 1) * a.bcap;
          it.n1 = min(ldc(a.bcount, (size_t)it.bh * a.nqb + I0 + 1), a.bcap);
        }
      }

      for (int round = 0;; ++round) {
        if (it.kind == 1) {
          // stage this pair's columns: 0 <= j <= last_pos and outside every strip tile
          const int32_t* cols = a.cols + (size_t)it.bh * a.cols_cap;
          const uint32_t* a2b = a.a2bits + (size_t)it.bh * a.aw;
          int staged = 0;
          while (gcursor < gcount && staged <= GCAP - NT) {
            const int idx = gcursor + tid;
            bool keep = false;
            int j = 0;
            if (idx < gcount) {
              j = cols[idx];
              keep = (j >= 0) && (j <= it.last_pos) && !test_bit(a2b, it.tq1 - (j >> 6));
            }
            const uint64_t bal = __builtin_amdgcn_ballot_w64(keep);
            __syncthreads();
            if (l == 0) s_misc[1 + w] = __popcll(bal);
            __syncthreads();
            int off = staged;
            for (int i = 0; i < w; ++i) off += s_misc[1 + i];
            if (keep) s_cols[off + ballot_rank(bal)] = j;
            staged += s_misc[1] + s_misc[2] + s_misc[3] + s_misc[4];
            gcursor += NT;
            const int lastc = cols[min(gcursor, gcount) - 1];
            if (lastc > it.last_pos) gcursor = gcount;
          }
          __syncthreads();
          it.ngather = staged;
          if (round > 0) it.nstrip = 0;
          it.nent = it.nstrip + (staged + TK - 1) / TK;
        } else if (it.kind == 2) {
          // per == 2: one shared list; per == 1: the cursor merges two lists and
          // stops when both are exhausted (nent is only an upper bound)
          it.nent = it.per == 2 ? 2 * it.n0 : it.n0 + it.n1;
        } else {
          it.nent = it.last_pos / TK + 1;
        }

        Cursor cc;
        cursor_init(it, cc);
        Entry cur;
        cur.kind = -1;
        cur.flags = 0;
        cur.full = 0;
        bool have = cursor_has_next(it, cc);
        if (have) {
          cur = cursor_next(it, cc);
          issue_tile<false>(kbp, a.Nk, cur, s_cols, ring, w, l, off_k);
          issue_tile<true>(vbp, a.Nk, cur, s_cols, ring + TK * 256, w, l, off_v);
        }
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
          else if (it.kind == 1) mode = ((cur.full >> ih) & 1) ? M_NONE : M_VS;
          else mode = (cur.kt * TK + TK - 1 > P0w) ? M_CAUSAL : M_NONE;
          // diagonal-bitmap words covering this wave's windows and the tile's
          // column bits (scalar loads, issued before the wait)
          uint32_t W0 = 0u, W1 = 0u, W2 = 0u, W3 = 0u, mv0 = 0u, mv1 = 0u;
          int wbase = 0;
          if (mode == M_VS) {
            wbase = R0w - cur.kt * TK - 63;               // window start of this wave's row 0 (>= -63)
            const uint32_t* swp = sbits + ((wbase >> 5) + 2);
            W0 = ldc(swp, 0); W1 = ldc(swp, 1); W2 = ldc(swp, 2); W3 = ldc(swp, 3);
            mv0 = ldc(vbits, 2 * cur.kt); mv1 = ldc(vbits, 2 * cur.kt + 1);
          }
          wait_vm();
          __syncthreads();                       // tile n landed; every wave is done with tile n - 1
          Entry nxt;
          nxt.kind = -1;
          nxt.flags = 0;
          nxt.full = 0;
          const bool have_n = cursor_has_next(it, cc);
          if (have_n) {
            nxt = cursor_next(it, cc);
            issue_tile<false>(kbp, a.Nk, nxt, s_cols, ring + (stage ^ 1) * 2 * TK * 256, w, l, off_k);
            issue_tile<true>(vbp, a.Nk, nxt, s_cols, ring + ((stage ^ 1) * 2 + 1) * TK * 256, w, l, off_v);
          }
          const char* sk = s_kv[stage][0];
          const lds_char_t* sv = (const lds_char_t*)s_kv[stage][1];

          // 64-bit window of diagonal bits for this lane's row (bit b <-> offset lo + b)
          uint64_t swin = 0;
          if (mode == M_VS) {
            const int sh = (wbase & 31) + qn;            // 0 .. 62
            const uint64_t lo64 = ((uint64_t)W1 << 32) | W0;
            const uint64_t hi64 = ((uint64_t)W3 << 32) | W2;
            swin = sh ? ((lo64 >> sh) | (hi64 << (64 - sh))) : lo64;
          }

#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            // ---- mask over keys 32 kb .. +31 (bit c <-> key kt*64 + 32 kb + c)
            const int ktop = iq - cur.kt * TK - 32 * kb;   // keys c <= ktop are causal
            uint32_t M = ~0u;
            if (mode == M_SKIP) {
              M = 0u;
            } else if (mode == M_CAUSAL) {
              M = causal_mask32(ktop);
            } else if (mode == M_VS) {
              // key c of this half sits at window bit 63 - 32 kb - c
              const uint32_t part = kb == 0 ? (uint32_t)(swin >> 32) : (uint32_t)swin;
              M = (__builtin_bitreverse32(part) | (kb == 0 ? mv0 : mv1)) & causal_mask32(ktop);
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
            }
            if (!row_ok) M = 0u;
            if (__builtin_amdgcn_ballot_w64(M != 0u) == 0) continue;
            const bool masked = __builtin_amdgcn_ballot_w64(M != ~0u) != 0;

            // ---- S^T = K Q^T for these 32 keys (eight K fragments read first)
            f32x16 sacc;
#pragma unroll
            for (int v = 0; v < 16; ++v) sacc[v] = 0.f;
            const int row = 32 * kb + qn;
            u32x4 kf[8];
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) kf[ks] = *(const u32x4*)(sk + row * 256 + swz_k(row, 2 * ks + hh) * 16);
            DSA_PRIO_HI();
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
              sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[ks]), qf[ks], sacc, 0, 0, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
            DSA_PRIO_LO();

            // ---- mask (one wave-uniform branch), online softmax on raw scores
            // (the scale is folded into exp2)
            if (masked) {
              const uint32_t mk = M >> (4 * hh);
#pragma unroll
              for (int v = 0; v < 16; ++v) {
                const int pos = 8 * (v >> 2) + (v & 3);
                const uint32_t keep = (uint32_t)((int32_t)(mk << (31 - pos)) >> 31);   // all ones if kept
                sacc[v] = __uint_as_float((__float_as_uint(sacc[v]) & keep) | (0xff800000u & ~keep));
              }
            }
            float mx = fmaxf(fmaxf(sacc[0], sacc[1]), sacc[2]);
#pragma unroll
            for (int v = 3; v < 15; v += 2) mx = fmaxf(fmaxf(mx, sacc[v]), sacc[v + 1]);
            mx = fmaxf(mx, sacc[15]);
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
            const float muse = (m_run == -INFINITY) ? 0.f : m_run;
            const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
            uint32_t pk[8];
#pragma unroll
            for (int v = 0; v < 16; v += 2) {
              const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[v], scale2, -muse));
              const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[v + 1], scale2, -muse));
              const uint32_t pb = pack_bf16x2(p0, p1);
              // the row sum uses the same bf16-rounded weights as the PV product
              l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pb), ones, l_run, false);
              pk[v >> 1] = pb;
            }

            // ---- O^T += V^T P^T over these 32 keys (two 16-key steps)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
              u32x4 bx = {pk[4 * s2], pk[4 * s2 + 1], pk[4 * s2 + 2], pk[4 * s2 + 3]};
              const bf16x8 bop = __builtin_bit_cast(bf16x8, bx);
              const int rowa = 32 * kb + 16 * s2 + v_row0;
              const int rowb = rowa + 8;
              short4_t ya[4], yb[4];
#pragma unroll
              for (int db = 0; db < 4; ++db) {
                const int cch = 4 * db + 2 * (G & 1) + ((si & 3) >> 1);
                ya[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_short4_t*)(sv + rowa * 256 + swz_v(rowa, cch) * 16 + v_half));
                yb[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_short4_t*)(sv + rowb * 256 + swz_v(rowb, cch) * 16 + v_half));
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
          }
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
  int sw, vw, aw, acap, TA;
  size_t off_s, off_v, off_f, off_a2, off_ac, off_ctr, off_al, off_ale, total_words;
};

VsLayout vs_layout(int B, int H, int Nk) {
  VsLayout L;
  L.sw = (Nk + 31) / 32 + 5;
  L.vw = (Nk + 31) / 32 + 2;
  L.TA = (Nk + TK - 1) / TK + 2;
  L.aw = (L.TA + 31) / 32 + 1;
  L.acap = L.TA;
  const size_t nbh = (size_t)B * H;
  size_t off = 0;
  L.off_ctr = off; off += 64;
  L.off_s = off; off += nbh * L.sw;
  L.off_v = off; off += nbh * L.vw;
  L.off_f = off; off += nbh * L.aw;
  L.off_a2 = off; off += nbh * L.aw;
  L.off_ac = off; off += nbh;
  L.total_words = off;          // region zeroed before every call
  L.off_al = off; off += nbh * L.acap;
  L.off_ale = off; off += nbh * L.acap;
  (void)off;
  return L;
}

}  // namespace

size_t attn_workspace_bytes(int B, int H, int Nk) {
  VsLayout L = vs_layout(B, H, Nk);
  return (L.off_ale + (size_t)B * H * L.acap) * 4 + 256;
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
  a.fbits = base + L.off_f;
  a.a2bits = base + L.off_a2;
  a.a2count = (int32_t*)(base + L.off_ac);
  a.a2list = (int32_t*)(base + L.off_al);
  a.a2le = (int32_t*)(base + L.off_ale);
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

  // Queue assignment.  Each head's cost is estimated (key tiles over all its
  // query tiles); the Q heads that share a KV head go to the same queue, so
  // that the items running together on one XCD stream the same K/V tiles
  // through that XCD's L2.  Groups are placed longest first into the
  // least-loaded queue; within a queue, consecutive items are the group's
  // heads at the same query rows.
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
  if ((e = launch_token_attention(a, st)) != hipSuccess) return e;
  if (heads.empty()) return hipSuccess;
  const int rep = a.H / a.Hkv;
  struct GC { double cost; int key; std::vector<int> bh; };
  std::vector<GC> groups;
  for (const HC& x : heads) {
    const int key = (x.bh / a.H) * a.Hkv + (x.bh % a.H) / rep;   // b * Hkv + kv head
    if (groups.empty() || groups.back().key != key) groups.push_back({0.0, key, {}});
    groups.back().cost += x.cost;
    groups.back().bh.push_back(x.bh);
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
  hipLaunchKernelGGL(attn_kernel, dim3((unsigned)grid), dim3(NT), 0, st, a, sc);
  return hipGetLastError();
}

}  // namespace dsa
