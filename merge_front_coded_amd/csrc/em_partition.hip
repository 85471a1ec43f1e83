// Merge-path partition: the co-rank of every partition diagonal.
//
// "CUDA merge path: merging sorted arrays in parallel", "The merge matrix, and
// the diagonal that cuts it": the merge's first d outputs consist of A[0..i)
// and B[0..d-i); i is found by bisection over [max(0, d-|B|), min(d, |A|)].  With
// ties going to A (Everett, "GPU construction experiment", the merge
// paragraph) a candidate i is too large exactly when A[i-1] > B[d-i]; that
// test is false up to the co-rank and true after it.
//
// gfx950 design: a group of 4 lanes per diagonal, sixteen diagonals per
// wave.  Each round the group tests 4 evenly spaced candidates at once and a
// ballot locates the crossing, so the range shrinks 4-fold per round (twelve
// rounds for 8M-record inputs, 48 key reads per diagonal).  The search is
// bound by its key reads rather than by its rounds: at 8M+8M (7,813
// diagonals), run alone in a loop so that the keys it reads stay cached,
// groups of 2, 4, 8, 16, 32 and 64 lanes took 42, 27, 31, 46, 73 and 114 us.
// Run after an emitter has swept the caches, 4 and 16 lanes both take 42 us:
// the cold key reads, twelve dependent rounds of them, set the time.
#include "em_tile.h"

namespace em {

constexpr int kPartBlock = 256;
constexpr uint32_t kGroup = 4;  // lanes per diagonal

__global__ __launch_bounds__(kPartBlock) void k_partition(em_side_t A, em_side_t B, uint32_t items,
                                                          uint32_t P, uint32_t* __restrict__ splits) {
  const uint32_t gtid = blockIdx.x * kPartBlock + threadIdx.x;
  const uint32_t diag = gtid / kGroup;
  const uint32_t t = gtid % kGroup;                   // lane in the group
  const uint32_t gshift = (lane_id() / kGroup) * kGroup;  // the group's bits in a wave ballot
  const uint32_t N = A.n + B.n;
  const bool live = diag <= P;
  const uint64_t d64 = static_cast<uint64_t>(diag) * items;
  const uint32_t d = live ? (d64 < N ? static_cast<uint32_t>(d64) : N) : 0;
  uint32_t lo = live ? (d > B.n ? d - B.n : 0) : 0;
  uint32_t hi = live ? (d < A.n ? d : A.n) : 0;
  // the co-rank lies in [lo, hi] and the "too large" test is false at lo
  lo = corank_group<kGroup>(A, B, d, lo, hi, t, gshift);
  if (live && t == 0) splits[diag] = lo;
}

}  // namespace em

using namespace em;

extern "C" int em_partition(const em_side_t* A, const em_side_t* B, uint32_t items_per_part,
                            uint32_t* splits, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  int rc = check_pair(A, B);
  if (rc) return rc;
  if (!splits || items_per_part == 0) return EM_EINVAL;
  const uint32_t N = A->n + B->n;
  const uint32_t P = (N + items_per_part - 1) / items_per_part;
  const uint32_t groups = P + 1;
  const uint32_t per_block = kPartBlock / kGroup;
  const uint32_t blocks = (groups + per_block - 1) / per_block;
  hipLaunchKernelGGL(k_partition, dim3(blocks), dim3(kPartBlock), 0, as_stream(stream), *A, *B,
                     items_per_part, P, splits);
  return check_launch();
}
