// Tile scheduling shared by the tiled grouped-GEMM kernels (prefill path).
//
// A launch covers the expert-contiguous rows produced by the dispatch: expert
// e owns rows [offsets[e], offsets[e+1]).  Its row tiles of BM rows and its
// column tiles form one list, expert-major, then groups of NGROUP column
// tiles, then row tiles; every workgroup maps its index to a tile of that list
// on the device from `offsets`, so the host never reads the routing back.  The
// hardware hands workgroup i to XCD (i mod 8): each XCD walks a contiguous
// range of the list, so the ~32 tiles it runs at once share 8 row blocks and 4
// column blocks of one expert and their k-slices come from that XCD's L2.
// When an XCD's last wave of tiles would leave more than half of its compute
// units idle, the leftover tiles can be cut into k-pieces (partial sums in a
// workspace, summed by a second kernel in piece order).
#pragma once

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int BM = kPrefillBM;  // 256 rows
constexpr int BN = 256;         // LDS B-tile columns
constexpr int BK = 32;
#ifndef MOE_NGROUP
#define MOE_NGROUP 4
#endif
constexpr int NGROUP = MOE_NGROUP;  // column tiles per scheduling group

constexpr int kXcds = 8;          // the hardware hands workgroup i to XCD (i mod 8)
constexpr int kMaxTailSplit = 8;  // k-pieces per leftover tile

struct Tile {
  int e, m, nt, row0, rows;
  int k0, k1;  // k-steps [k0, k1) of this workgroup's share of the tile
  int slot;    // >= 0: a k-piece of a split tile, partial sums go to this slot
};

// Row tiles per expert, gathered by each wave in parallel: lane l holds
// experts 4l .. 4l+3 (n <= 256), `pre` counts the row tiles of the experts
// before 4l and `total` those of all experts.  Serial loops over the experts
// here cost several microseconds per workgroup at n = 64, on the critical path
// between one tile and the next on a CU.
static_assert(kMaxN <= 256, "expert_tiles covers 4 experts per lane");
struct ExpertTiles {
  int mt[4];
  int pre, total;
};

__device__ ExpertTiles expert_tiles(const int* __restrict__ offsets, int n) {
  const int lane = threadIdx.x & 63;
  ExpertTiles t;
  int s = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * lane + j;
    const int c = e < n ? offsets[e + 1] - offsets[e] : 0;
    t.mt[j] = (c + BM - 1) / BM;
    s += t.mt[j];
  }
  int incl = s;  // inclusive scan over the lanes
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  t.pre = incl - s;
  t.total = __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
  return t;
}

// Position L of the tile list -> expert, row tile, column tile.  The list is
// expert-major, then groups of NGROUP column tiles, then row tiles; expert e
// owns positions [NT * P(e), NT * P(e+1)) with P the running sum of row tiles.
__device__ bool tile_at(const int* __restrict__ offsets, const ExpertTiles& et, int NT, int L, Tile& tc) {
  int hit = -1, base = 0, mt = 0;
  int p = et.pre;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (et.mt[j] > 0 && L >= NT * p && L < NT * (p + et.mt[j])) {
      hit = j;
      base = p;
      mt = et.mt[j];
    }
    p += et.mt[j];
  }
  const unsigned long long owner = __ballot(hit >= 0);  // at most one lane
  if (owner == 0) return false;
  const int src = __ffsll(owner) - 1;
  const int e = __builtin_amdgcn_readfirstlane(4 * src + __shfl(hit, src));
  mt = __builtin_amdgcn_readfirstlane(__shfl(mt, src));
  L -= NT * __builtin_amdgcn_readfirstlane(__shfl(base, src));
  const int ng = NT / NGROUP;
  const int gsz = mt * NGROUP;
  const int grp = L / gsz;
  int m, nt;
  if (grp < ng) {
    const int rem = L - grp * gsz;
    m = rem / NGROUP;
    nt = grp * NGROUP + rem % NGROUP;
  } else {
    const int rem = L - ng * gsz;
    const int gt = NT - ng * NGROUP;
    m = rem / gt;
    nt = ng * NGROUP + rem % gt;
  }
  tc.e = e;
  tc.m = m;
  tc.nt = nt;
  tc.row0 = offsets[e] + m * BM;
  const int left = offsets[e + 1] - tc.row0;
  tc.rows = left < BM ? left : BM;
  return true;
}

// Work of one XCD: the contiguous tiles [beg, beg + cnt) of the list.  `q`
// tiles fill whole waves of the XCD's `cus` compute units; when the `r`
// leftover tiles would leave more than half of the last wave idle (and the
// kernel may split), each is cut into `s` k-pieces of `chunk` k-steps, so
// the last wave is r * s <= cus shorter workgroups.
struct XcdPlan {
  int beg, cnt, q, r, s, chunk;
};

// `gran`: k-steps (of BK) a piece is a multiple of (the kernel's unrolled k-loop).
__device__ XcdPlan xcd_plan(int total, int x, int cus, int nk, bool may_split, int gran) {
  XcdPlan t;
  const int per = (total + kXcds - 1) / kXcds;
  t.beg = x * per;
  t.cnt = max(0, min(per, total - t.beg));
  t.q = t.cnt / cus * cus;
  t.r = t.cnt - t.q;
  t.s = 1;
  t.chunk = nk;
  if (may_split && t.r > 0 && 2 * t.r <= cus) {
    const int s0 = min(min(cus / t.r, kMaxTailSplit), nk / gran);
    if (s0 >= 2) {
      t.chunk = gran * ((nk / gran + s0 - 1) / s0);  // whole unrolled k-loops
      t.s = (nk + t.chunk - 1) / t.chunk;
    }
  }
  return t;
}

// Positions in an XCD's share: q whole tiles, then r * s k-pieces when the
// leftover tiles are split, else all cnt tiles whole.
__device__ __forceinline__ int queue_len(const XcdPlan& t) { return t.s == 1 ? t.cnt : t.q + t.r * t.s; }

// Position `pos` of XCD x's share (plan t) -> tile or k-piece; false past its end.
__device__ bool queue_tile(const int* __restrict__ offsets, const ExpertTiles& et, int NT, int nk, int cus, int x,
                           const XcdPlan& t, int pos, Tile& tc) {
  tc.k0 = 0;
  tc.k1 = nk;
  tc.slot = -1;
  int L;
  if (t.s == 1) {
    if (pos >= t.cnt) return false;
    L = t.beg + pos;
  } else if (pos < t.q) {
    L = t.beg + pos;
  } else {
    const int u = pos - t.q;
    if (u >= t.r * t.s) return false;
    L = t.beg + t.q + u % t.r;
    const int piece = u / t.r;
    tc.k0 = piece * t.chunk;
    tc.k1 = min(nk, tc.k0 + t.chunk);
    tc.slot = x * cus + u;
  }
  return tile_at(offsets, et, NT, L, tc);
}

// Maps this workgroup to its tile (or k-piece of a tile); false if it has none.
// Every wave computes the same answer from offsets[0..n].
__device__ bool decode_tile(const int* __restrict__ offsets, int n, int NT, int nk, int cus,
                            bool may_split, int gran, Tile& tc) {
  const ExpertTiles et = expert_tiles(offsets, n);
  const int x = blockIdx.x % kXcds;
  const XcdPlan t = xcd_plan(et.total * NT, x, cus, nk, may_split, gran);
  return queue_tile(offsets, et, NT, nk, cus, x, t, blockIdx.x / kXcds, tc);
}

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | ((vm >> 4) << 14);
}
constexpr int WAITCNT_ALL = waitcnt_imm(0, 15);

// Direct global -> LDS load: lane l's 16 bytes land at M0 + 16 l.  Written in
// asm so that the compiler does not make every later LDS read wait for it; the
// kernels wait for these loads themselves (s_waitcnt vmcnt, counted by issue order).
__device__ __forceinline__ void load_lds16(const void* g, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(g), "{m0}"(lds_addr) : "memory");
}

// Grid: per XCD at most ceil(tiles / 8) tiles plus one extra wave of pieces.
inline unsigned prefill_grid(int64_t TK, int n, int NT, int cus) {
  const int64_t tiles_ub = ((TK + BM - 1) / BM + n) * (int64_t)NT;  // sum_e ceil(c_e/BM) bound
  const int64_t per = (tiles_ub + kXcds - 1) / kXcds;
  return (unsigned)((per + cus) * kXcds);
}

}  // namespace
}  // namespace moe
