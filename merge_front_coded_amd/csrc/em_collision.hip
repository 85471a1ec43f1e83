// Collision-bitmap variants of the keep step, with the temporary rank512 and
// rank2048 directories.
//
// Everett, "Collision bitmap and rank experiment":
//  * "Corrected record ordinals": for each B_j find lb_j = lower_bound(A, B_j)
//    and set bit C_{lb_j} by atomic OR when the keys match (matches can share a
//    bitmap word); the bitmap is cleared on the GPU first and bits past |A|
//    stay zero.  With R(i) = sum_{t<i} C_t, B_j lands at j + lb_j - R(lb_j)
//    and a surviving A_i at i + lower_bound(B, A_i) - R(i).
//  * "Temporary rank layouts": rank512 stores, per 512-bit block, the set
//    bits before the block (32 bits) and, for each of its 64-bit words after
//    the first, the set bits before that word inside the block (seven 9-bit
//    fields); a query reads the directory and one masked 64-bit word.  rank2048 gives each
//    2048-bit block one 8-byte entry: a 32-bit absolute prefix and the
//    populations before its second, third and fourth 512-bit runs, packed
//    (10, 11 and 11 bits); a query adds the popcounts of up to seven whole
//    64-bit words of its run and one masked word.  Both are built by count ->
//    global scan -> finish.
//  * "The three experimental paths", and the suggested modes collision512,
//    collision2048, collision512-tiled and collision512-compact:
//      - independent lower bounds (EM_COLLISION_512, EM_COLLISION_2048): each
//        surviving A_i searches B's keys for lower_bound(B, A_i);
//      - tiled (EM_COLLISION_512_TILED): A in tiles of 32 consecutive records,
//        one search per tile and a monotone cursor; B keeps independent
//        searches (it is the sparse side in the skewed workload);
//      - compact A then Merge Path (EM_COLLISION_512_COMPACT): the surviving
//        A references go to i - R(i) of a compact list, which is then merged
//        with B (disjoint key sets now) by merge-path partitions.
//
// The tiled A search and cursor run over the saved lower bounds lb_j, not
// over B's keys: for a surviving A_i, B_j < A_i exactly when lb_j <= i (a
// B_j with lb_j = i and an equal key would have collided and removed A_i), so
// lower_bound(B, A_i) = #{j : lb_j <= i}, and lb is non-decreasing in j.  The
// tiled A side therefore reads no key bytes at all.
#include "em_internal.h"

namespace em {

constexpr int kColBlock = 256;
constexpr uint32_t kTileA = 32;
constexpr uint32_t kSuperBits = 2048;  // rank2048 block; the bitmap is kept in whole ones

struct Rank512View {
  const uint32_t* bits;  // bitmap words (whole 2048-bit blocks + 16 pad words)
  const uint32_t* dir;   // 3 u32 per 512-bit block, nblk + 1 blocks
  // Exclusive rank: set bits at positions < p (p <= nbits).
  __device__ __forceinline__ uint32_t rank(uint32_t p) const {
    const uint32_t b = p >> 9;
    uint32_t r = dir[3 * b];
    const uint32_t q = (p >> 6) & 7u;
    if (q) {
      const uint64_t packed = dir[3 * b + 1] | (static_cast<uint64_t>(dir[3 * b + 2]) << 32);
      r += static_cast<uint32_t>((packed >> (9 * (q - 1))) & 511u);
    }
    const uint32_t m = p & 63u;
    if (m) {
      const uint32_t w = p >> 6;
      const uint64_t word = bits[2 * w] | (static_cast<uint64_t>(bits[2 * w + 1]) << 32);
      r += static_cast<uint32_t>(__builtin_popcountll(word & ((1ull << m) - 1)));
    }
    return r;
  }
};

// rank2048 entry: bits 0..31 the set bits before the block, bits 32..41 /
// 42..52 / 53..63 those inside it before its runs 1 / 2 / 3.  (The 32-bit
// absolute field would restart at each 2^32-bit epoch; positions here are
// below 2^25, so all of them are in the first epoch, whose base is 0.)
struct Rank2048View {
  const uint32_t* bits;
  const uint64_t* dir;  // nsb + 1 entries
  __device__ __forceinline__ uint32_t rank(uint32_t p) const {
    const uint64_t e = dir[p >> 11];
    uint32_t r = static_cast<uint32_t>(e);
    const uint32_t run = (p >> 9) & 3u;
    if (run == 1) r += static_cast<uint32_t>(e >> 32) & 0x3FFu;
    if (run == 2) r += static_cast<uint32_t>(e >> 42) & 0x7FFu;
    if (run == 3) r += static_cast<uint32_t>(e >> 53) & 0x7FFu;
    // whole 64-bit words of the run before p, then the masked word
    const uint64_t* w64 = reinterpret_cast<const uint64_t*>(bits);
    const uint32_t w0 = (p >> 9) << 3, w1 = p >> 6;
    for (uint32_t w = w0; w < w1; ++w) r += static_cast<uint32_t>(__builtin_popcountll(w64[w]));
    const uint32_t m = p & 63u;
    if (m) r += static_cast<uint32_t>(__builtin_popcountll(w64[w1] & ((1ull << m) - 1)));
    return r;
  }
};

// rank512 count: population of each 512-bit block; entry nblk is 0 so that
// the scan leaves the total there.
__global__ __launch_bounds__(kColBlock) void k_rank_count(const uint32_t* __restrict__ bits,
                                                          uint32_t nblk, uint32_t* __restrict__ cnt) {
  const uint32_t b = blockIdx.x * kColBlock + threadIdx.x;
  if (b > nblk) return;
  uint32_t c = 0;
  if (b < nblk) {
    const uint4* p = reinterpret_cast<const uint4*>(bits + 16 * b);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 t = p[q];
      c += __builtin_popcount(t.x) + __builtin_popcount(t.y) + __builtin_popcount(t.z) +
           __builtin_popcount(t.w);
    }
  }
  cnt[b] = c;
}

// rank512 finish: directory entry of every block from the scanned block prefixes.
__global__ __launch_bounds__(kColBlock) void k_rank_finish(const uint32_t* __restrict__ bits,
                                                           uint32_t nblk,
                                                           const uint32_t* __restrict__ prefix,
                                                           uint32_t* __restrict__ dir) {
  const uint32_t b = blockIdx.x * kColBlock + threadIdx.x;
  if (b > nblk) return;
  uint64_t packed = 0;
  if (b < nblk) {
    uint32_t run = 0;
    for (uint32_t q = 0; q < 7; ++q) {
      run += __builtin_popcount(bits[16 * b + 2 * q]) + __builtin_popcount(bits[16 * b + 2 * q + 1]);
      packed |= static_cast<uint64_t>(run) << (9 * q);
    }
  }
  dir[3 * b] = prefix[b];
  dir[3 * b + 1] = static_cast<uint32_t>(packed);
  dir[3 * b + 2] = static_cast<uint32_t>(packed >> 32);
}

// rank2048 count: population of each 2048-bit block (entry nsb is 0).
__global__ __launch_bounds__(kColBlock) void k_rank2048_count(const uint32_t* __restrict__ bits,
                                                              uint32_t nsb, uint32_t* __restrict__ cnt) {
  const uint32_t b = blockIdx.x * kColBlock + threadIdx.x;
  if (b > nsb) return;
  uint32_t c = 0;
  if (b < nsb) {
    const uint4* p = reinterpret_cast<const uint4*>(bits + 64 * b);
    for (int q = 0; q < 16; ++q) {
      const uint4 t = p[q];
      c += __builtin_popcount(t.x) + __builtin_popcount(t.y) + __builtin_popcount(t.z) +
           __builtin_popcount(t.w);
    }
  }
  cnt[b] = c;
}

// rank2048 finish: the block's absolute prefix and its runs' populations.
__global__ __launch_bounds__(kColBlock) void k_rank2048_finish(const uint32_t* __restrict__ bits,
                                                               uint32_t nsb,
                                                               const uint32_t* __restrict__ prefix,
                                                               uint64_t* __restrict__ dir) {
  const uint32_t b = blockIdx.x * kColBlock + threadIdx.x;
  if (b > nsb) return;
  uint64_t e = prefix[b];
  if (b < nsb) {
    uint32_t before = 0;
    for (uint32_t run = 0; run < 3; ++run) {
      for (uint32_t w = 0; w < 16; ++w) before += __builtin_popcount(bits[64 * b + 16 * run + w]);
      e |= static_cast<uint64_t>(before) << (run == 0 ? 32 : run == 1 ? 42 : 53);
    }
  }
  dir[b] = e;
}

// mark: lower bound of every B key in A, collision bit on an equal key.
// lower_bound(A, key) inside [lo, hi]
__device__ __forceinline__ uint32_t lower_bound_in(const em_side_t& A, const uint8_t* kbytes, KeyRef k, uint32_t lo,
                                                   uint32_t hi) {
  while (lo < hi) {
    const uint32_t mid = lo + ((hi - lo) >> 1);
    if (cmp_keys(A.keys, key_of(A, mid), kbytes, k) < 0)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

// B in groups of 64 consecutive records: a first kernel finds the lower
// bound of each group's first key in all of A (and A.n after the last
// group); each record then searches only between its group's bound and the
// next group's (B is sorted, so its lower bounds are monotone): about 7
// instead of 23 dependent key comparisons per record at 8M + 8M.  Used when
// B holds at least one record per 64 of A (else, edges == nullptr, every
// record searches all of A: with few B records a group's range stays wide
// and the first kernel's searches only add a serial step).
constexpr uint32_t kMarkGroup = 64;

__global__ __launch_bounds__(kColBlock) void k_mark_edges(em_side_t A, em_side_t B, uint32_t groups,
                                                          uint32_t* __restrict__ edges) {
  const uint32_t g = blockIdx.x * kColBlock + threadIdx.x;
  if (g > groups) return;
  edges[g] = g < groups ? lower_bound_in(A, B.keys, key_of(B, g * kMarkGroup), 0, A.n) : A.n;
}

__global__ __launch_bounds__(kColBlock) void k_mark(em_side_t A, em_side_t B, const uint32_t* __restrict__ edges,
                                                    uint32_t* __restrict__ bits, uint32_t* __restrict__ lb_out) {
  const uint32_t j = blockIdx.x * kColBlock + threadIdx.x;
  if (j >= B.n) return;
  const KeyRef kb = key_of(B, j);
  // (for unsorted inputs the bounds may be out of order: the result is then
  // the lower one, still inside A)
  const uint32_t lo = edges ? lower_bound_in(A, B.keys, kb, edges[j / kMarkGroup], edges[j / kMarkGroup + 1])
                            : lower_bound_in(A, B.keys, kb, 0, A.n);
  if (lo < A.n && cmp_keys(A.keys, key_of(A, lo), B.keys, kb) == 0)
    atomicOr(bits + (lo >> 5), 1u << (lo & 31u));
  lb_out[j] = lo;
}

template <class View>
__global__ __launch_bounds__(kColBlock) void k_scatter_B(uint32_t nA, uint32_t nB, View rv,
                                                         const uint32_t* __restrict__ lb,
                                                         uint32_t* __restrict__ final_refs,
                                                         uint32_t* __restrict__ ord_B) {
  const uint32_t j = blockIdx.x * kColBlock + threadIdx.x;
  if (j >= nB) return;
  const uint32_t i = lb[j];
  const uint32_t o = j + i - rv.rank(i);
  final_refs[o] = nA + j;
  if (ord_B) ord_B[j] = o;
}

// Independent lower bounds: each surviving A_i searches B's keys.
template <class View>
// (edges, when not null: the lower bounds in B of the first keys of A's
// groups of 64, as k_mark's, to narrow each search)
__global__ __launch_bounds__(kColBlock) void k_scatter_A_search(em_side_t A, em_side_t B, View rv,
                                                                const uint32_t* __restrict__ edges,
                                                                uint32_t* __restrict__ final_refs,
                                                                uint32_t* __restrict__ ord_A) {
  const uint32_t i = blockIdx.x * kColBlock + threadIdx.x;
  if (i >= A.n) return;
  if ((rv.bits[i >> 5] >> (i & 31u)) & 1u) {
    if (ord_A) ord_A[i] = EM_NONE;
    return;
  }
  const KeyRef ka = key_of(A, i);
  const uint32_t lo = edges ? lower_bound_in(B, A.keys, ka, edges[i / kMarkGroup], edges[i / kMarkGroup + 1])
                            : lower_bound_in(B, A.keys, ka, 0, B.n);
  const uint32_t o = i + lo - rv.rank(i);
  final_refs[o] = i;
  if (ord_A) ord_A[i] = o;
}

// A in tiles of 64 kTileA consecutive records, one tile per wave: one search
// in the saved lower bounds and one rank query per tile, then runs of 64
// records, a lane each, so that consecutive lanes write consecutive
// ordinals and references.  For a run starting at i0 (a multiple of 64), the
// B records whose lower bound lies in [i0, i0 + 64) are counted by position
// in an LDS histogram (their lower bounds are the next entries of the sorted
// array, read 64 at a time), whose prefix gives each lane #{j : lb_j <= i};
// its collisions before i are the run's start rank plus a popcount of the
// run's 64 bitmap bits below it.
__global__ __launch_bounds__(kColBlock) void k_scatter_A(uint32_t nA, uint32_t nB, Rank512View rv,
                                                         const uint32_t* __restrict__ lb,
                                                         uint32_t* __restrict__ final_refs,
                                                         uint32_t* __restrict__ ord_A) {
  __shared__ uint32_t hist[kColBlock / kWave][kWave];
  const uint32_t lane = threadIdx.x & (kWave - 1);
  uint32_t* h = hist[threadIdx.x / kWave];
  const uint64_t start = (static_cast<uint64_t>(blockIdx.x) * kColBlock + threadIdx.x) / kWave * (kWave * kTileA);
  if (start >= nA) return;  // (the whole wave; no workgroup barrier follows)
  const uint32_t i_start = static_cast<uint32_t>(start);
  // cb = #{j : lb_j < i_start}, then the rank at i_start (the same in every lane)
  uint32_t lo = 0, hi = nB;
  while (lo < hi) {
    const uint32_t mid = lo + ((hi - lo) >> 1);
    if (lb[mid] < i_start)
      lo = mid + 1;
    else
      hi = mid;
  }
  uint32_t cb = lo;
  uint32_t r0 = rv.rank(i_start);
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  for (uint32_t k = 0; k < kTileA; ++k) {
    const uint32_t i0 = i_start + kWave * k;
    if (i0 >= nA) break;
    h[lane] = 0;
    wave_sync();
    uint32_t cend = cb;
    while (true) {
      const uint32_t j = cend + lane;
      const uint32_t v = j < nB ? lb[j] : 0xFFFFFFFFu;
      const bool in = v >= i0 && v < i0 + kWave;  // (v >= i0 holds for sorted inputs: the j < cb are below i0)
      if (in) atomicAdd(&h[v - i0], 1u);
      const uint32_t n_in = static_cast<uint32_t>(__builtin_popcountll(__ballot(in)));  // a prefix of the lanes
      cend += n_in;
      if (n_in < kWave) break;
    }
    wave_sync();
    const uint32_t cur = cb + wave_inclusive_scan<uint32_t>(h[lane]);
    const uint64_t word = rv.bits[i0 >> 5] | (static_cast<uint64_t>(rv.bits[(i0 >> 5) + 1]) << 32);
    const uint32_t i = i0 + lane;
    if (i < nA) {
      if ((word >> lane) & 1u) {
        if (ord_A) ord_A[i] = EM_NONE;
      } else {
        const uint32_t r = r0 + static_cast<uint32_t>(__builtin_popcountll(word & ((1ull << lane) - 1)));
        const uint32_t o = i + cur - r;
        final_refs[o] = i;
        if (ord_A) ord_A[i] = o;
      }
    }
    r0 += static_cast<uint32_t>(__builtin_popcountll(word));
    cb = cend;
    wave_sync();  // (the histogram is cleared for the next run after every lane read it)
  }
}

// Compact A: surviving A_i goes to slot i - R(i) of cA (one bitmap word per
// thread; the rank is queried once per word).  A replaced A_i gets EM_NONE.
__global__ __launch_bounds__(kColBlock) void k_compact_A(uint32_t nA, Rank512View rv,
                                                         uint32_t* __restrict__ cA,
                                                         uint32_t* __restrict__ ord_A) {
  const uint32_t t = blockIdx.x * kColBlock + threadIdx.x;
  const uint32_t i0 = t * 32u;
  if (i0 >= nA) return;
  const uint32_t i1 = i0 + 32u < nA ? i0 + 32u : nA;
  uint32_t r = rv.rank(i0);
  const uint32_t cbits = rv.bits[i0 >> 5];
  for (uint32_t i = i0; i < i1; ++i) {
    if ((cbits >> (i - i0)) & 1u) {
      ++r;
      if (ord_A) ord_A[i] = EM_NONE;
    } else {
      cA[i - r] = i;
    }
  }
}

// Merge Path over the compact A list (A'_x = A[cA[x]]) and B, whose key sets
// are disjoint: a workgroup takes kMcItems consecutive outputs, finds the
// co-ranks of its two diagonals (threads 0 and 1), then each thread finds
// the co-rank of its own diagonal inside that range and merges kMcIPT
// outputs.  The co-rank of diagonal d is the number of A' among the first d
// outputs: the smallest x with A'_x > B_{d-1-x} (or x = min(d, |A'|)).
constexpr uint32_t kMcIPT = 4;
constexpr uint32_t kMcItems = kColBlock * kMcIPT;

__device__ __forceinline__ uint32_t corank_compact(const em_side_t& A, const em_side_t& B,
                                                   const uint32_t* cA, uint32_t d, uint32_t lo,
                                                   uint32_t hi) {
  while (lo < hi) {
    const uint32_t mid = lo + ((hi - lo) >> 1);  // mid < min(d, |A'|), d - 1 - mid < |B|
    if (cmp_keys(A.keys, key_of(A, cA[mid]), B.keys, key_of(B, d - 1 - mid)) <= 0)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(kColBlock) void k_merge_compact(em_side_t A, em_side_t B, Rank512View rv,
                                                             const uint32_t* __restrict__ cA,
                                                             uint32_t* __restrict__ final_refs,
                                                             uint32_t* __restrict__ ord_A,
                                                             uint32_t* __restrict__ ord_B) {
  __shared__ uint32_t s_i[2];
  const uint32_t nAc = A.n - rv.rank(A.n);
  const uint32_t N = nAc + B.n;
  const uint32_t d0 = blockIdx.x * kMcItems;
  if (d0 >= N) return;
  const uint32_t d1 = min(d0 + kMcItems, N);
  if (threadIdx.x < 2) {
    const uint32_t d = threadIdx.x ? d1 : d0;
    s_i[threadIdx.x] = corank_compact(A, B, cA, d, d > B.n ? d - B.n : 0u, min(d, nAc));
  }
  __syncthreads();
  const uint32_t i0 = s_i[0], i1 = s_i[1];
  const uint32_t j0 = d0 - i0, j1 = d1 - i1;
  const uint32_t dt = d0 + threadIdx.x * kMcIPT;
  if (dt >= d1) return;
  // this thread's diagonal: i in [max(i0, dt - j1), min(i1, dt - j0)]
  const uint32_t lo = max(i0, dt > j1 ? dt - j1 : 0u), hi = min(i1, dt - j0);
  uint32_t i = corank_compact(A, B, cA, dt, lo, hi < lo ? lo : hi);
  uint32_t j = dt - i;
  const uint32_t dend = min(dt + kMcIPT, d1);
  for (uint32_t d = dt; d < dend; ++d) {
    const bool takeA = j >= j1 || (i < i1 && cmp_keys(A.keys, key_of(A, cA[i]), B.keys, key_of(B, j)) <= 0);
    if (takeA) {
      const uint32_t r = cA[i++];
      final_refs[d] = r;
      if (ord_A) ord_A[r] = d;
    } else {
      final_refs[d] = A.n + j;
      if (ord_B) ord_B[j] = d;
      ++j;
    }
  }
}

template <class View>
__global__ void k_collision_total(uint32_t nA, uint32_t nB, View rv, uint32_t* d_S) {
  *d_S = nA + nB - rv.rank(nA);
}

// Copy a caller bitmap into whole blocks, clearing bits >= nbits.
__global__ __launch_bounds__(kColBlock) void k_copy_bits(const uint32_t* __restrict__ src, uint32_t nbits,
                                                         uint32_t* __restrict__ dst, uint32_t nwords) {
  const uint32_t w = blockIdx.x * kColBlock + threadIdx.x;
  if (w >= nwords) return;
  uint32_t v = 0;
  const uint32_t start = w * 32u;
  if (start < nbits) {
    v = src[w];
    const uint32_t valid = nbits - start;
    if (valid < 32) v &= (1u << valid) - 1u;
  }
  dst[w] = v;
}

template <class View>
__global__ __launch_bounds__(kColBlock) void k_rank_probe(View rv, const uint32_t* __restrict__ pos,
                                                          uint32_t npos, uint32_t nbits,
                                                          uint32_t* __restrict__ out) {
  const uint32_t t = blockIdx.x * kColBlock + threadIdx.x;
  if (t >= npos) return;
  const uint32_t p = pos[t];
  out[t] = p <= nbits ? rv.rank(p) : EM_NONE;
}

// ---- workspace layout shared by the collision path and the probes ----

struct RankLayout {
  uint32_t nblk;     // 512-bit blocks
  uint32_t nsb;      // 2048-bit blocks
  uint32_t* bits;    // 64 * nsb + 16 words
  uint32_t* dir;     // rank512: 3 * (nblk + 1)
  uint64_t* dir2048; // rank2048: nsb + 1
  uint32_t* cnt;     // nblk + 1
  uint32_t* prefix;  // nblk + 2
  uint8_t* scan_ws;
  size_t scan_bytes;
  size_t used;
};

static RankLayout rank_layout(void* ws, uint32_t nbits) {
  RankLayout L{};
  L.nblk = (nbits + 511u) / 512u;
  L.nsb = (nbits + kSuperBits - 1) / kSuperBits;
  WsCursor cur{static_cast<uint8_t*>(ws), 0};
  L.bits = cur.take<uint32_t>(64 * static_cast<size_t>(L.nsb) + 16);
  L.dir = cur.take<uint32_t>(3 * (static_cast<size_t>(L.nblk) + 1));
  L.dir2048 = cur.take<uint64_t>(static_cast<size_t>(L.nsb) + 1);
  L.cnt = cur.take<uint32_t>(static_cast<size_t>(L.nblk) + 1);
  L.prefix = cur.take<uint32_t>(static_cast<size_t>(L.nblk) + 2);
  L.scan_bytes = scan_ws(L.nblk + 1);
  L.scan_ws = cur.take<uint8_t>(L.scan_bytes);
  L.used = cur.used;
  return L;
}

size_t rank_ws(uint32_t nbits) { return align_up(rank_layout(nullptr, nbits).used, 256); }

// Collision workspace of one mode: the rank layout, the saved B lower bounds
// and (compact mode) the compact A list.
static size_t mark_edges_bytes(uint32_t nB) {
  return align_up((static_cast<size_t>(nB) / kMarkGroup + 2) * sizeof(uint32_t), 256);
}

static size_t collision_mode_ws(uint32_t nA, uint32_t nB, uint32_t mode) {
  size_t b = rank_ws(nA) + align_up(static_cast<size_t>(nB) * sizeof(uint32_t) + 4, 256) + mark_edges_bytes(nB) +
             mark_edges_bytes(nA);
  if (mode == EM_COLLISION_512_COMPACT) b += align_up(static_cast<size_t>(nA) * sizeof(uint32_t) + 4, 256);
  return b;
}

size_t collision_ws(uint32_t nA, uint32_t nB) { return collision_mode_ws(nA, nB, EM_COLLISION_512_COMPACT); }

static inline uint32_t blocks_for(uint64_t n) {
  return static_cast<uint32_t>((n + kColBlock - 1) / kColBlock);
}

// count -> scan -> finish over a bitmap already in L.bits
static int rank_build(RankLayout& L, bool r2048, hipStream_t st) {
  if (r2048) {
    hipLaunchKernelGGL(k_rank2048_count, dim3(blocks_for(L.nsb + 1)), dim3(kColBlock), 0, st, L.bits, L.nsb,
                       L.cnt);
    int rc = scan_launch<uint32_t>(L.cnt, L.nsb + 1, L.prefix, L.scan_ws, L.scan_bytes, st);
    if (rc) return rc;
    hipLaunchKernelGGL(k_rank2048_finish, dim3(blocks_for(L.nsb + 1)), dim3(kColBlock), 0, st, L.bits,
                       L.nsb, L.prefix, L.dir2048);
    return check_launch();
  }
  hipLaunchKernelGGL(k_rank_count, dim3(blocks_for(L.nblk + 1)), dim3(kColBlock), 0, st, L.bits, L.nblk,
                     L.cnt);
  int rc = scan_launch<uint32_t>(L.cnt, L.nblk + 1, L.prefix, L.scan_ws, L.scan_bytes, st);
  if (rc) return rc;
  hipLaunchKernelGGL(k_rank_finish, dim3(blocks_for(L.nblk + 1)), dim3(kColBlock), 0, st, L.bits,
                     L.nblk, L.prefix, L.dir);
  return check_launch();
}

static int collision_run(const em_side_t& A, const em_side_t& B, uint32_t mode, uint32_t* final_refs,
                         uint32_t* ord_A, uint32_t* ord_B, uint32_t* d_S, void* ws, hipStream_t st) {
  RankLayout L = rank_layout(ws, A.n);
  uint8_t* after = static_cast<uint8_t*>(ws) + align_up(L.used, 256);
  uint32_t* lb = reinterpret_cast<uint32_t*>(after);
  uint32_t* edges = reinterpret_cast<uint32_t*>(after + align_up(static_cast<size_t>(B.n) * 4 + 4, 256));
  uint32_t* edgesA = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(edges) + mark_edges_bytes(B.n));
  uint32_t* cA = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(edgesA) + mark_edges_bytes(A.n));
  // the A-side searches of B (modes 512 and 2048) narrowed the same way
  const uint32_t* a_edges = nullptr;
  if (A.n && B.n && (mode == EM_COLLISION_512 || mode == EM_COLLISION_2048) &&
      static_cast<uint64_t>(A.n) * kMarkGroup >= B.n) {
    const uint32_t groups = (A.n + kMarkGroup - 1) / kMarkGroup;
    hipLaunchKernelGGL(k_mark_edges, dim3(blocks_for(static_cast<uint64_t>(groups) + 1)), dim3(kColBlock), 0, st, B,
                       A, groups, edgesA);
    a_edges = edgesA;
  }
  clear_u32(L.bits, 64 * static_cast<size_t>(L.nsb) + 16, st);
  if (B.n) {
    const uint32_t groups = (B.n + kMarkGroup - 1) / kMarkGroup;
    const bool narrow = static_cast<uint64_t>(B.n) * kMarkGroup >= A.n;
    if (narrow)
      hipLaunchKernelGGL(k_mark_edges, dim3(blocks_for(static_cast<uint64_t>(groups) + 1)), dim3(kColBlock), 0, st,
                         A, B, groups, edges);
    hipLaunchKernelGGL(k_mark, dim3(blocks_for(B.n)), dim3(kColBlock), 0, st, A, B, narrow ? edges : nullptr, L.bits,
                       lb);
  }
  int rc = check_launch();
  if (rc) return rc;
  const bool r2048 = mode == EM_COLLISION_2048;
  rc = rank_build(L, r2048, st);
  if (rc) return rc;
  const Rank512View v512{L.bits, L.dir};
  const Rank2048View v2048{L.bits, L.dir2048};
  if (mode == EM_COLLISION_512_COMPACT) {
    if (A.n)
      hipLaunchKernelGGL(k_compact_A, dim3(blocks_for((A.n + 31) / 32)), dim3(kColBlock), 0, st, A.n, v512,
                         cA, ord_A);
    const uint64_t N = static_cast<uint64_t>(A.n) + B.n;  // a bound on the merged count
    if (N)
      hipLaunchKernelGGL(k_merge_compact, dim3(static_cast<uint32_t>((N + kMcItems - 1) / kMcItems)),
                         dim3(kColBlock), 0, st, A, B, v512, cA, final_refs, ord_A, ord_B);
    hipLaunchKernelGGL(k_collision_total<Rank512View>, dim3(1), dim3(1), 0, st, A.n, B.n, v512, d_S);
    return check_launch();
  }
  if (r2048) {
    if (B.n)
      hipLaunchKernelGGL(k_scatter_B<Rank2048View>, dim3(blocks_for(B.n)), dim3(kColBlock), 0, st, A.n, B.n,
                         v2048, lb, final_refs, ord_B);
    if (A.n)
      hipLaunchKernelGGL(k_scatter_A_search<Rank2048View>, dim3(blocks_for(A.n)), dim3(kColBlock), 0, st, A,
                         B, v2048, a_edges, final_refs, ord_A);
    hipLaunchKernelGGL(k_collision_total<Rank2048View>, dim3(1), dim3(1), 0, st, A.n, B.n, v2048, d_S);
    return check_launch();
  }
  if (B.n)
    hipLaunchKernelGGL(k_scatter_B<Rank512View>, dim3(blocks_for(B.n)), dim3(kColBlock), 0, st, A.n, B.n,
                       v512, lb, final_refs, ord_B);
  if (A.n) {
    if (mode == EM_COLLISION_512_TILED)
      hipLaunchKernelGGL(k_scatter_A,
                         dim3(blocks_for(static_cast<uint64_t>(kWave) *
                                         ((A.n + kWave * kTileA - 1) / (kWave * kTileA)))),
                         dim3(kColBlock), 0, st, A.n, B.n, v512, lb, final_refs, ord_A);
    else
      hipLaunchKernelGGL(k_scatter_A_search<Rank512View>, dim3(blocks_for(A.n)), dim3(kColBlock), 0, st, A,
                         B, v512, a_edges, final_refs, ord_A);
  }
  hipLaunchKernelGGL(k_collision_total<Rank512View>, dim3(1), dim3(1), 0, st, A.n, B.n, v512, d_S);
  return check_launch();
}

static int rank_probe(const uint32_t* bitmap, uint32_t nbits, const uint32_t* positions, uint32_t npos,
                      uint32_t* out, void* ws, size_t ws_bytes, void* stream, bool r2048) {
  if (!ws || (npos && (!positions || !out)) || (nbits && !bitmap)) return EM_EINVAL;
  if (reinterpret_cast<uintptr_t>(ws) & 255) return EM_EINVAL;
  if (nbits >= EM_MAX_RECORDS + (1u << 13)) return EM_ERANGE;
  if (ws_bytes < rank_ws(nbits)) return EM_ENOSPC;
  hipStream_t st = as_stream(stream);
  RankLayout L = rank_layout(ws, nbits);
  const uint32_t nwords = 64 * L.nsb + 16;
  hipLaunchKernelGGL(k_copy_bits, dim3(blocks_for(nwords)), dim3(kColBlock), 0, st, bitmap, nbits, L.bits,
                     nwords);
  int rc = check_launch();
  if (rc) return rc;
  rc = rank_build(L, r2048, st);
  if (rc) return rc;
  if (npos) {
    if (r2048)
      hipLaunchKernelGGL(k_rank_probe<Rank2048View>, dim3(blocks_for(npos)), dim3(kColBlock), 0, st,
                         Rank2048View{L.bits, L.dir2048}, positions, npos, nbits, out);
    else
      hipLaunchKernelGGL(k_rank_probe<Rank512View>, dim3(blocks_for(npos)), dim3(kColBlock), 0, st,
                         Rank512View{L.bits, L.dir}, positions, npos, nbits, out);
  }
  return check_launch();
}

}  // namespace em

using namespace em;

extern "C" size_t em_rank512_workspace_bytes(uint32_t nbits) { return rank_ws(nbits); }
extern "C" size_t em_rank2048_workspace_bytes(uint32_t nbits) { return rank_ws(nbits); }

extern "C" size_t em_collision_workspace_bytes(uint32_t nA, uint32_t nB, uint32_t mode) {
  return collision_mode_ws(nA, nB, mode);
}

extern "C" int em_collision_rank_mode(const em_side_t* A, const em_side_t* B, uint32_t mode,
                                      uint32_t* final_refs, uint32_t* ord_A, uint32_t* ord_B, uint32_t* d_S,
                                      void* ws, size_t ws_bytes, void* stream) {
  int rc = check_pair(A, B);
  if (rc) return rc;
  if (mode > EM_COLLISION_512_COMPACT) return EM_EINVAL;
  if (!final_refs || !d_S || !ws) return EM_EINVAL;
  if (reinterpret_cast<uintptr_t>(ws) & 255) return EM_EINVAL;
  if (ws_bytes < collision_mode_ws(A->n, B->n, mode)) return EM_ENOSPC;
  return collision_run(*A, *B, mode, final_refs, ord_A, ord_B, d_S, ws, as_stream(stream));
}

extern "C" int em_collision_rank(const em_side_t* A, const em_side_t* B, uint32_t* final_refs,
                                 uint32_t* ord_A, uint32_t* ord_B, uint32_t* d_S, void* ws,
                                 size_t ws_bytes, void* stream) {
  return em_collision_rank_mode(A, B, EM_COLLISION_512_TILED, final_refs, ord_A, ord_B, d_S, ws, ws_bytes,
                                stream);
}

extern "C" int em_rank512_probe(const uint32_t* bitmap, uint32_t nbits, const uint32_t* positions,
                                uint32_t npos, uint32_t* out, void* ws, size_t ws_bytes, void* stream) {
  return rank_probe(bitmap, nbits, positions, npos, out, ws, ws_bytes, stream, false);
}

extern "C" int em_rank2048_probe(const uint32_t* bitmap, uint32_t nbits, const uint32_t* positions,
                                 uint32_t npos, uint32_t* out, void* ws, size_t ws_bytes, void* stream) {
  return rank_probe(bitmap, nbits, positions, npos, out, ws, ws_bytes, stream, true);
}
