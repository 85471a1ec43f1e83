// Stable merge of each partition plus the keep-newer scan and compaction.
//
// Everett, "GPU construction experiment", merge paragraph: merge by diagonal
// partitions, equal keys put the older input first, a neighbouring-key
// comparison and an exclusive scan keep the last reference of each equal-key
// run (so the newer record wins; a newer tombstone stays), and the compacted
// order fixes every survivor's ordinal.  "CUDA merge path: merging sorted
// arrays in parallel": each worker starts from its own co-rank and takes
// exactly as many steps as its slice is long.
//
// gfx950 design (one workgroup = one partition of `items_per_part` outputs):
//  * the partition's A and B key offsets are staged in LDS once;
//  * each thread finds its slice's co-rank inside the partition by bisection
//    on the staged offsets and merges IPT outputs; the comparison that decides
//    each step also tells whether an A record equals its B neighbour, so the
//    keep flag needs no second pass (an equal pair split by the partition
//    boundary is caught by comparing the partition's last A with the next
//    partition's first B);
//  * a block scan of keep flags gives partition-local ordinals, and a
//    decoupled look-back over partitions (dynamic tickets) gives the global
//    survivor base in the same pass;
//  * survivors, ord_A and ord_B are staged in LDS and written with
//    consecutive lanes on consecutive words.
#include "em_internal.h"

namespace em {

constexpr int kMergeBlock = 256;
constexpr uint32_t kDrop = 0x80000000u;  // refs are < 2^24, bit 31 marks a dropped A

template <int IPT>
struct MergeShared {
  static constexpr int kTile = kMergeBlock * IPT;
  uint32_t a_off[kTile + 2];
  uint32_t b_off[kTile + 2];
  uint32_t out[kTile];
  uint32_t ords[kTile];
  uint32_t scan[kMergeBlock / kWave + 1];
  uint32_t tile;
  uint32_t base;
};

template <int IPT>
__global__ __launch_bounds__(kMergeBlock) void k_merge_keep(
    em_side_t A, em_side_t B, const uint32_t* __restrict__ splits, uint32_t items, uint32_t P,
    uint32_t* __restrict__ final_refs, uint32_t* __restrict__ ord_A, uint32_t* __restrict__ ord_B,
    uint32_t* __restrict__ d_S, uint32_t* __restrict__ ticket, uint64_t* __restrict__ desc) {
  __shared__ MergeShared<IPT> sh;
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

  for (uint32_t x = tid; x <= nA_t; x += kMergeBlock) sh.a_off[x] = A.key_off[i0 + x];
  for (uint32_t x = tid; x < nb_off; x += kMergeBlock) sh.b_off[x] = B.key_off[j0 + x];
  __syncthreads();

  auto keyA = [&](uint32_t a) { return KeyRef{sh.a_off[a], sh.a_off[a + 1] - sh.a_off[a]}; };
  auto keyB = [&](uint32_t b) { return KeyRef{sh.b_off[b], sh.b_off[b + 1] - sh.b_off[b]}; };

  // ---- merge this thread's slice ----
  uint32_t refs[IPT];
  uint32_t kept = 0;
  const uint32_t k = tid * IPT;
  if (k < len) {
    uint32_t lo = k > nB_t ? k - nB_t : 0;
    uint32_t hi = k < nA_t ? k : nA_t;
    while (lo < hi) {
      const uint32_t mid = (lo + hi + 1) >> 1;
      const uint32_t j = k - mid;
      const bool too_big = j < nB_t && cmp_keys(A.keys, keyA(mid - 1), B.keys, keyB(j)) > 0;
      if (too_big)
        hi = mid - 1;
      else
        lo = mid;
    }
    uint32_t a = lo, b = k - lo;
#pragma unroll
    for (int s = 0; s < IPT; ++s) {
      refs[s] = kDrop;  // placeholder for "no item"
      if (k + s < len) {
        int c;
        if (a < nA_t && b < nB_t) {
          c = cmp_keys(A.keys, keyA(a), B.keys, keyB(b));
        } else if (a < nA_t) {
          // B exhausted inside the partition: only the partition's last A can
          // equal the next partition's first B.
          c = (a == nA_t - 1 && has_next_b && cmp_keys(A.keys, keyA(a), B.keys, keyB(nB_t)) == 0) ? 0
                                                                                                   : -1;
        } else {
          c = 1;
        }
        if (c <= 0) {
          refs[s] = (i0 + a) | (c == 0 ? kDrop : 0u);
          ++a;
        } else {
          refs[s] = A.n + j0 + b;
          ++b;
        }
        kept += c != 0;
      }
    }
  } else {
#pragma unroll
    for (int s = 0; s < IPT; ++s) refs[s] = kDrop;
  }

  // ---- keep scan inside the partition ----
  uint32_t total;
  uint32_t ord = block_exclusive_scan<uint32_t, kMergeBlock>(kept, sh.scan, total);
#pragma unroll
  for (int s = 0; s < IPT; ++s) {
    if (k + s >= len) continue;
    const uint32_t r = refs[s];
    const uint32_t ref = r & ~kDrop;
    const bool drop = (r & kDrop) != 0;
    if (ref < A.n) {
      sh.ords[ref - i0] = drop ? EM_NONE : ord;
    } else {
      sh.ords[nA_t + (ref - A.n - j0)] = ord;
    }
    if (!drop) sh.out[ord++] = ref;
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

  for (uint32_t x = tid; x < total; x += kMergeBlock) final_refs[base + x] = sh.out[x];
  if (ord_A)
    for (uint32_t x = tid; x < nA_t; x += kMergeBlock) {
      const uint32_t o = sh.ords[x];
      ord_A[i0 + x] = o == EM_NONE ? EM_NONE : base + o;
    }
  if (ord_B)
    for (uint32_t y = tid; y < nB_t; y += kMergeBlock) ord_B[j0 + y] = base + sh.ords[nA_t + y];
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
  clear_u32(ticket, 1, st);
  clear_u64(desc, P, st);
  const uint32_t ipt = (items_per_part + kMergeBlock - 1) / kMergeBlock;
  if (ipt <= 1)
    launch_merge<1>(*A, *B, splits, items_per_part, P, final_refs, ord_A, ord_B, d_S, ticket, desc, st);
  else if (ipt <= 2)
    launch_merge<2>(*A, *B, splits, items_per_part, P, final_refs, ord_A, ord_B, d_S, ticket, desc, st);
  else if (ipt <= 4)
    launch_merge<4>(*A, *B, splits, items_per_part, P, final_refs, ord_A, ord_B, d_S, ticket, desc, st);
  else if (ipt <= 8)
    launch_merge<8>(*A, *B, splits, items_per_part, P, final_refs, ord_A, ord_B, d_S, ticket, desc, st);
  else
    launch_merge<16>(*A, *B, splits, items_per_part, P, final_refs, ord_A, ord_B, d_S, ticket, desc, st);
  return check_launch();
}
