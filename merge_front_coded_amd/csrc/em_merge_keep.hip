// Stable merge of each partition plus the keep-newer scan and compaction.
//
// Everett, "GPU construction experiment", merge paragraph: merge by diagonal
// partitions with ties going to the older side, then compare each output
// with its neighbour and keep only the final reference of a run of equal
// keys (the newer record, a newer tombstone included), an exclusive scan
// giving each kept reference its ordinal in the compacted order.  "CUDA merge path: merging sorted
// arrays in parallel": each worker starts from its own co-rank and takes
// exactly as many steps as its slice is long.
//
// gfx950 design (one 512-thread workgroup = one partition of `items_per_part`
// outputs):
//  * the partition's A and B key offsets and each key's first 8 bytes (the
//    prefix cache) go to LDS; the key bytes stay in HBM, so a partition needs
//    about 24 bytes of LDS per output and several partitions share a compute
//    unit, which hides the latency of their loads and look-backs;
//  * each thread finds its slice's co-rank inside the partition by a
//    fixed-step search on the prefix cache and merges IPT outputs
//    (merge_slice); the comparison that decides each step also tells whether
//    an A record equals its B neighbour, so the keep flag needs no second pass
//    (an equal pair split by the partition boundary is caught by comparing the
//    partition's last A with the next partition's first B);
//  * a block scan of keep flags gives partition-local ordinals, and a
//    decoupled look-back over partitions (dynamic tickets) gives the global
//    survivor base in the same pass;
//  * survivors, ord_A and ord_B are staged in LDS (over the dead prefix
//    cache) and written with consecutive lanes on consecutive words.
#include "em_tile.h"

namespace em {

constexpr int kMergeBlock = 512;

template <int IPT>
struct MergeShared {
  static constexpr int kTile = kMergeBlock * IPT;
  uint32_t a_off[kTile + 2];
  uint32_t b_off[kTile + 2];
  // prefix cache: each key's first 8 bytes, big-endian, zero padded; the
  // compaction arrays reuse it after the merge
  union {
    struct {
      uint64_t a_pfx[kTile + 2];
      uint64_t b_pfx[kTile + 2];
    } m;
    struct {
      uint32_t out[kTile];
      uint32_t ords[kTile];
    } c;
  } u;
  uint32_t scan[kMergeBlock / kWave + 1];
  uint32_t notes[kMergeBlock];  // the merge's list of pairs to check, kWave words per wave
  uint32_t tile, base;
};

template <int IPT>
__global__ __launch_bounds__(kMergeBlock) void k_merge_keep(
    em_side_t A, em_side_t B, const uint32_t* __restrict__ splits, uint32_t items, uint32_t P,
    uint32_t* __restrict__ final_refs, uint32_t* __restrict__ ord_A, uint32_t* __restrict__ ord_B,
    uint32_t* __restrict__ d_S, uint32_t* __restrict__ ticket, uint64_t* __restrict__ desc) {
  using Sh = MergeShared<IPT>;
  __shared__ Sh sh;
  const uint32_t tid = threadIdx.x;
  if (tid == 0) sh.tile = atomicAdd(ticket, 1u);
  __syncthreads();
  const uint32_t tile = sh.tile;
  const uint32_t N = A.n + B.n;
  const uint32_t d0 = tile * items;
  const uint32_t d1 = (d0 + items < N) ? d0 + items : N;
  uint32_t i0 = splits[tile], i1 = splits[tile + 1];
  // Splits from em_partition on sorted inputs always pass this check; any
  // other splits leave the partition empty rather than index outside it.
  const bool valid = i0 <= d0 && i1 <= d1 && i0 <= i1 && d0 - i0 <= d1 - i1 && i1 <= A.n &&
                     d1 - i1 <= B.n;
  if (!valid) {
    i0 = 0;
    i1 = 0;
  }
  const uint32_t j0 = valid ? d0 - i0 : 0, j1 = valid ? d1 - i1 : 0;
  const uint32_t nA_t = i1 - i0, nB_t = j1 - j0;
  const uint32_t len = valid ? d1 - d0 : 0;
  const bool has_next_b = valid && j1 < B.n;
  const uint32_t nb_off = nB_t + (has_next_b ? 2u : 1u);

  {
    // all offset loads first, then the LDS stores, so the loads overlap in
    // flight (a thread past the end loads the first offset again, so that no
    // load sits under a condition of its own)
    constexpr int kPer = IPT + 1;  // ceil((kTile + 2) / kMergeBlock)
    uint32_t va[kPer], vb[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const uint32_t x = tid + u * kMergeBlock;
      va[u] = A.key_off[i0 + (x <= nA_t ? x : 0u)];
      vb[u] = B.key_off[j0 + (x < nb_off ? x : 0u)];
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const uint32_t x = tid + u * kMergeBlock;
      if (x <= nA_t) sh.a_off[x] = va[u];
      if (x < nb_off) sh.b_off[x] = vb[u];
    }
  }
  __syncthreads();

  // ---- prefix cache (the keys themselves stay in HBM: comparisons the
  // prefixes leave open read them in place, and the small LDS footprint
  // keeps more partitions resident) ----
  fill_prefix_caches<kMergeBlock, IPT + 1>(PfxSide{sh.a_off, nA_t + 1, A.keys, sh.u.m.a_pfx},
                                           PfxSide{sh.b_off, nb_off, B.keys, sh.u.m.b_pfx}, 0u);
  __syncthreads();

  // ---- merge this thread's slice ----
  uint32_t refs[IPT];
  const uint32_t k = tid * IPT;
  const uint32_t kept = merge_slice<IPT>(sh.a_off, sh.b_off, sh.u.m.a_pfx, sh.u.m.b_pfx, A.keys, 0u, B.keys,
                                         0u, k, len, nA_t, nB_t, has_next_b, i0, A.n, j0, refs, sh.notes);

  // ---- keep scan inside the partition (its barriers end every read of the
  // prefix cache, which the compaction arrays then reuse) ----
  uint32_t total;
  uint32_t ord = block_exclusive_scan<uint32_t, kMergeBlock>(kept, sh.scan, total);
#pragma unroll
  for (int s = 0; s < IPT; ++s) {
    if (k + s >= len) continue;
    const uint32_t r = refs[s];
    const uint32_t ref = r & ~kDrop;
    const bool drop = (r & kDrop) != 0;
    if (ref < A.n) {
      sh.u.c.ords[ref - i0] = drop ? EM_NONE : ord;
    } else {
      sh.u.c.ords[nA_t + (ref - A.n - j0)] = ord;
    }
    if (!drop) sh.u.c.out[ord++] = ref;
  }

  // ---- survivor base of this partition (decoupled look-back) ----
  if (tid < kWave) {
    const uint64_t excl = lookback(desc, tile, total);
    if (tid == 0) {
      sh.base = static_cast<uint32_t>(excl);
      if (tile == P - 1) d_S[0] = static_cast<uint32_t>(excl) + total;
    }
  }
  __syncthreads();
  const uint32_t base = sh.base;

  for (uint32_t x = tid; x < total; x += kMergeBlock) final_refs[base + x] = sh.u.c.out[x];
  if (ord_A)
    for (uint32_t x = tid; x < nA_t; x += kMergeBlock) {
      const uint32_t o = sh.u.c.ords[x];
      ord_A[i0 + x] = o == EM_NONE ? EM_NONE : base + o;
    }
  if (ord_B)
    for (uint32_t y = tid; y < nB_t; y += kMergeBlock) ord_B[j0 + y] = base + sh.u.c.ords[nA_t + y];
}

__global__ void k_set_u32(uint32_t* p, uint32_t v) { *p = v; }

template <int IPT>
static void launch_merge(const em_side_t& A, const em_side_t& B, const uint32_t* splits, uint32_t items,
                         uint32_t P, uint32_t* final_refs, uint32_t* ord_A, uint32_t* ord_B,
                         uint32_t* d_S, uint32_t* ticket, uint64_t* desc, hipStream_t st) {
  hipLaunchKernelGGL(k_merge_keep<IPT>, dim3(P), dim3(kMergeBlock), 0, st, A, B, splits, items, P,
                     final_refs, ord_A, ord_B, d_S, ticket, desc);
}

size_t merge_keep_ws(uint32_t N, uint32_t items_per_part) {
  if (items_per_part == 0) return 0;
  const size_t P = (static_cast<size_t>(N) + items_per_part - 1) / items_per_part;
  return 256 + align_up(P * sizeof(uint64_t), 256);
}

}  // namespace em

using namespace em;

extern "C" int em_merge_keep(const em_side_t* A, const em_side_t* B, const uint32_t* splits,
                             uint32_t items_per_part, uint32_t* final_refs, uint32_t* ord_A,
                             uint32_t* ord_B, uint32_t* d_S, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_pair(A, B);
  if (rc) return rc;
  if (!splits || !final_refs || !d_S || !ws) return EM_EINVAL;
  if (items_per_part == 0 || items_per_part > EM_MAX_ITEMS_PER_PART) return EM_EINVAL;
  if (reinterpret_cast<uintptr_t>(ws) & 255) return EM_EINVAL;
  const uint32_t N = A->n + B->n;
  if (ws_bytes < merge_keep_ws(N, items_per_part)) return EM_ENOSPC;
  hipStream_t st = as_stream(stream);
  if (N == 0) {
    hipLaunchKernelGGL(k_set_u32, dim3(1), dim3(1), 0, st, d_S, 0u);
    return check_launch();
  }
  const uint32_t P = (N + items_per_part - 1) / items_per_part;
  WsCursor cur{static_cast<uint8_t*>(ws), 0};
  uint32_t* ticket = cur.take<uint32_t>(64);
  uint64_t* desc = cur.take<uint64_t>(P);
  clear_lookback(ticket, 1, desc, nullptr, P, st);
  const uint32_t ipt = (items_per_part + kMergeBlock - 1) / kMergeBlock;
  if (ipt <= 1)
    launch_merge<1>(*A, *B, splits, items_per_part, P, final_refs, ord_A, ord_B, d_S, ticket, desc, st);
  else if (ipt <= 2)
    launch_merge<2>(*A, *B, splits, items_per_part, P, final_refs, ord_A, ord_B, d_S, ticket, desc, st);
  else if (ipt <= 4)
    launch_merge<4>(*A, *B, splits, items_per_part, P, final_refs, ord_A, ord_B, d_S, ticket, desc, st);
  else
    launch_merge<8>(*A, *B, splits, items_per_part, P, final_refs, ord_A, ord_B, d_S, ticket, desc, st);
  return check_launch();
}
