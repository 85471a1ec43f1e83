// Collision-bitmap variant of the keep step, with the temporary rank512
// directory.
//
// Everett, "Collision bitmap and rank experiment":
//  * "Corrected record ordinals": for each B_j find lb_j = lower_bound(A, B_j)
//    and set bit C_{lb_j} by atomic OR when the keys match (matches can share a
//    bitmap word); the bitmap is cleared on the GPU first and bits past |A|
//    stay zero.  With R(i) = sum_{t<i} C_t, B_j lands at j + lb_j - R(lb_j)
//    and a surviving A_i at i + lower_bound(B, A_i) - R(i).
//  * "Temporary rank layouts": each 512-bit block has a 32-bit absolute prefix
//    and seven 9-bit prefixes for its 64-bit pairs, built by count -> global
//    scan -> finish; a query reads the directory and one masked 64-bit word.
//  * "The three experimental paths": B keeps independent searches (it is the
//    sparse side in the skewed workload); A is handled by tiles of 32
//    consecutive records, one search per tile and a monotone cursor.
//
// The A tile's search and cursor run over the saved lower bounds lb_j, not
// over B's keys: for a surviving A_i, B_j < A_i exactly when lb_j <= i (a
// B_j with lb_j = i and an equal key would have collided and removed A_i), so
// lower_bound(B, A_i) = #{j : lb_j <= i}, and lb is non-decreasing in j.  The
// A side therefore reads no key bytes at all.
#include "em_internal.h"

namespace em {

constexpr int kColBlock = 256;
constexpr uint32_t kRankBlockBits = 512;
constexpr uint32_t kTileA = 32;

struct RankView {
  const uint32_t* bits;  // bitmap words (whole 512-bit blocks + 2 pad words)
  const uint32_t* dir;   // 3 u32 per block, nblk + 1 blocks
};

// Exclusive rank: set bits at positions < p (p <= nbits).
__device__ __forceinline__ uint32_t rank512(RankView rv, uint32_t p) {
  const uint32_t b = p >> 9;
  uint32_t r = rv.dir[3 * b];
  const uint32_t q = (p >> 6) & 7u;
  if (q) {
    const uint64_t packed = rv.dir[3 * b + 1] | (static_cast<uint64_t>(rv.dir[3 * b + 2]) << 32);
    r += static_cast<uint32_t>((packed >> (9 * (q - 1))) & 511u);
  }
  const uint32_t m = p & 63u;
  if (m) {
    const uint32_t w = p >> 6;
    const uint64_t word = rv.bits[2 * w] | (static_cast<uint64_t>(rv.bits[2 * w + 1]) << 32);
    r += static_cast<uint32_t>(__builtin_popcountll(word & ((1ull << m) - 1)));
  }
  return r;
}

// count: population of each 512-bit block; entry nblk is 0 so that the scan
// leaves the total there.
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

// finish: directory entry of every block from the scanned block prefixes.
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

// mark: lower bound of every B key in A, collision bit on an equal key.
__global__ __launch_bounds__(kColBlock) void k_mark(em_side_t A, em_side_t B, uint32_t* __restrict__ bits,
                                                    uint32_t* __restrict__ lb_out) {
  const uint32_t j = blockIdx.x * kColBlock + threadIdx.x;
  if (j >= B.n) return;
  const KeyRef kb = key_of(B, j);
  uint32_t lo = 0, hi = A.n;
  while (lo < hi) {
    const uint32_t mid = lo + ((hi - lo) >> 1);
    if (cmp_keys(A.keys, key_of(A, mid), B.keys, kb) < 0)
      lo = mid + 1;
    else
      hi = mid;
  }
  if (lo < A.n && cmp_keys(A.keys, key_of(A, lo), B.keys, kb) == 0)
    atomicOr(bits + (lo >> 5), 1u << (lo & 31u));
  lb_out[j] = lo;
}

__global__ __launch_bounds__(kColBlock) void k_scatter_B(uint32_t nA, uint32_t nB, RankView rv,
                                                         const uint32_t* __restrict__ lb,
                                                         uint32_t* __restrict__ final_refs,
                                                         uint32_t* __restrict__ ord_B) {
  const uint32_t j = blockIdx.x * kColBlock + threadIdx.x;
  if (j >= nB) return;
  const uint32_t i = lb[j];
  const uint32_t o = j + i - rank512(rv, i);
  final_refs[o] = nA + j;
  if (ord_B) ord_B[j] = o;
}

// A in tiles of kTileA consecutive records: one search in the saved lower
// bounds, then a monotone cursor; the rank is queried once per tile and then
// advanced by the tile's own collision bits.
__global__ __launch_bounds__(kColBlock) void k_scatter_A(uint32_t nA, uint32_t nB, RankView rv,
                                                         const uint32_t* __restrict__ lb,
                                                         uint32_t* __restrict__ final_refs,
                                                         uint32_t* __restrict__ ord_A) {
  const uint32_t t = blockIdx.x * kColBlock + threadIdx.x;
  const uint32_t i0 = t * kTileA;
  if (i0 >= nA) return;
  const uint32_t i1 = i0 + kTileA < nA ? i0 + kTileA : nA;
  // cur = #{j : lb_j <= i0}
  uint32_t lo = 0, hi = nB;
  while (lo < hi) {
    const uint32_t mid = lo + ((hi - lo) >> 1);
    if (lb[mid] <= i0)
      lo = mid + 1;
    else
      hi = mid;
  }
  uint32_t cur = lo;
  uint32_t r = rank512(rv, i0);
  const uint32_t cbits = rv.bits[i0 >> 5];  // kTileA == 32: the tile is one bitmap word
  for (uint32_t i = i0; i < i1; ++i) {
    const uint32_t c = (cbits >> (i - i0)) & 1u;
    if (c) {
      if (ord_A) ord_A[i] = EM_NONE;
    } else {
      while (cur < nB && lb[cur] <= i) ++cur;
      const uint32_t o = i + cur - r;
      final_refs[o] = i;
      if (ord_A) ord_A[i] = o;
    }
    r += c;
  }
}

__global__ void k_collision_total(uint32_t nA, uint32_t nB, RankView rv, uint32_t* d_S) {
  *d_S = nA + nB - rank512(rv, nA);
}

// Copy a caller bitmap into whole 512-bit blocks, clearing bits >= nbits.
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

__global__ __launch_bounds__(kColBlock) void k_rank_probe(RankView rv, const uint32_t* __restrict__ pos,
                                                          uint32_t npos, uint32_t nbits,
                                                          uint32_t* __restrict__ out) {
  const uint32_t t = blockIdx.x * kColBlock + threadIdx.x;
  if (t >= npos) return;
  const uint32_t p = pos[t];
  out[t] = p <= nbits ? rank512(rv, p) : EM_NONE;
}

// ---- workspace layout shared by the collision path and the probe ----

struct RankLayout {
  uint32_t nblk;
  uint32_t* bits;    // 16 * nblk + 16 words
  uint32_t* dir;     // 3 * (nblk + 1)
  uint32_t* cnt;     // nblk + 1
  uint32_t* prefix;  // nblk + 2
  uint8_t* scan_ws;
  size_t scan_bytes;
  size_t used;
};

static RankLayout rank_layout(void* ws, uint32_t nbits) {
  RankLayout L{};
  L.nblk = (nbits + kRankBlockBits - 1) / kRankBlockBits;
  WsCursor cur{static_cast<uint8_t*>(ws), 0};
  L.bits = cur.take<uint32_t>(16 * static_cast<size_t>(L.nblk) + 16);
  L.dir = cur.take<uint32_t>(3 * (static_cast<size_t>(L.nblk) + 1));
  L.cnt = cur.take<uint32_t>(static_cast<size_t>(L.nblk) + 1);
  L.prefix = cur.take<uint32_t>(static_cast<size_t>(L.nblk) + 2);
  L.scan_bytes = scan_ws(L.nblk + 1);
  L.scan_ws = cur.take<uint8_t>(L.scan_bytes);
  L.used = cur.used;
  return L;
}

size_t rank_ws(uint32_t nbits) { return align_up(rank_layout(nullptr, nbits).used, 256); }

size_t collision_ws(uint32_t nA, uint32_t nB) {
  return align_up(rank_ws(nA) + 256 + static_cast<size_t>(nB) * sizeof(uint32_t), 256);
}

static inline uint32_t blocks_for(uint64_t n) {
  return static_cast<uint32_t>((n + kColBlock - 1) / kColBlock);
}

// count -> scan -> finish over a bitmap already in L.bits
static int rank_build(RankLayout& L, hipStream_t st) {
  hipLaunchKernelGGL(k_rank_count, dim3(blocks_for(L.nblk + 1)), dim3(kColBlock), 0, st, L.bits, L.nblk,
                     L.cnt);
  int rc = scan_launch<uint32_t>(L.cnt, L.nblk + 1, L.prefix, L.scan_ws, L.scan_bytes, st);
  if (rc) return rc;
  hipLaunchKernelGGL(k_rank_finish, dim3(blocks_for(L.nblk + 1)), dim3(kColBlock), 0, st, L.bits,
                     L.nblk, L.prefix, L.dir);
  return check_launch();
}

}  // namespace em

using namespace em;

extern "C" size_t em_rank512_workspace_bytes(uint32_t nbits) { return rank_ws(nbits); }

extern "C" int em_collision_rank(const em_side_t* A, const em_side_t* B, uint32_t* final_refs,
                                 uint32_t* ord_A, uint32_t* ord_B, uint32_t* d_S, void* ws,
                                 size_t ws_bytes, void* stream) {
  int rc = check_pair(A, B);
  if (rc) return rc;
  if (!final_refs || !d_S || !ws) return EM_EINVAL;
  if (reinterpret_cast<uintptr_t>(ws) & 255) return EM_EINVAL;
  if (ws_bytes < collision_ws(A->n, B->n)) return EM_ENOSPC;
  hipStream_t st = as_stream(stream);
  RankLayout L = rank_layout(ws, A->n);
  uint32_t* lb = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + align_up(L.used, 256));
  clear_u32(L.bits, 16 * static_cast<size_t>(L.nblk) + 16, st);
  if (B->n)
    hipLaunchKernelGGL(k_mark, dim3(blocks_for(B->n)), dim3(kColBlock), 0, st, *A, *B, L.bits, lb);
  rc = check_launch();
  if (rc) return rc;
  rc = rank_build(L, st);
  if (rc) return rc;
  RankView rv{L.bits, L.dir};
  if (B->n)
    hipLaunchKernelGGL(k_scatter_B, dim3(blocks_for(B->n)), dim3(kColBlock), 0, st, A->n, B->n, rv, lb,
                       final_refs, ord_B);
  if (A->n)
    hipLaunchKernelGGL(k_scatter_A, dim3(blocks_for((A->n + kTileA - 1) / kTileA)), dim3(kColBlock), 0,
                       st, A->n, B->n, rv, lb, final_refs, ord_A);
  hipLaunchKernelGGL(k_collision_total, dim3(1), dim3(1), 0, st, A->n, B->n, rv, d_S);
  return check_launch();
}

extern "C" int em_rank512_probe(const uint32_t* bitmap, uint32_t nbits, const uint32_t* positions,
                                uint32_t npos, uint32_t* out, void* ws, size_t ws_bytes, void* stream) {
  if (!ws || (npos && (!positions || !out)) || (nbits && !bitmap)) return EM_EINVAL;
  if (reinterpret_cast<uintptr_t>(ws) & 255) return EM_EINVAL;
  if (nbits >= EM_MAX_RECORDS + (1u << 13)) return EM_ERANGE;
  if (ws_bytes < rank_ws(nbits)) return EM_ENOSPC;
  hipStream_t st = as_stream(stream);
  RankLayout L = rank_layout(ws, nbits);
  const uint32_t nwords = 16 * L.nblk + 16;
  hipLaunchKernelGGL(k_copy_bits, dim3(blocks_for(nwords)), dim3(kColBlock), 0, st, bitmap, nbits, L.bits,
                     nwords);
  int rc = check_launch();
  if (rc) return rc;
  rc = rank_build(L, st);
  if (rc) return rc;
  if (npos)
    hipLaunchKernelGGL(k_rank_probe, dim3(blocks_for(npos)), dim3(kColBlock), 0, st,
                       RankView{L.bits, L.dir}, positions, npos, nbits, out);
  return check_launch();
}
