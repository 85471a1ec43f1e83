// Merge-path partition: the co-rank of every partition diagonal.
//
// "CUDA merge path: merging sorted arrays in parallel", "The merge matrix, and
// the diagonal that cuts it": the first d outputs of the merge are A[0..i) and
// B[0..d-i); i is found by bisection over [max(0, d-|B|), min(d, |A|)].  With
// ties going to A (Everett, "GPU construction experiment", the merge
// paragraph) a candidate i is too large exactly when A[i-1] > B[d-i]; that
// test is false up to the co-rank and true after it.
//
// gfx950 design: one wave64 per diagonal.  Each round the 64 lanes test 64
// evenly spaced candidates at once and a ballot locates the crossing, so the
// range shrinks 64-fold per round (about 4 rounds for 8M-record inputs)
// instead of taking ~23 dependent global-memory bisection steps per thread.
#include "em_internal.h"

namespace em {

constexpr int kPartBlock = 256;

__global__ __launch_bounds__(kPartBlock) void k_partition(em_side_t A, em_side_t B, uint32_t items,
                                                          uint32_t P, uint32_t* __restrict__ splits) {
  const uint32_t wave = (blockIdx.x * kPartBlock + threadIdx.x) / kWave;
  const uint32_t lane = lane_id();
  if (wave > P) return;  // uniform per wave
  const uint32_t N = A.n + B.n;
  const uint64_t d64 = static_cast<uint64_t>(wave) * items;
  const uint32_t d = d64 < N ? static_cast<uint32_t>(d64) : N;
  uint32_t lo = d > B.n ? d - B.n : 0;
  uint32_t hi = d < A.n ? d : A.n;
  // Invariant: the co-rank lies in [lo, hi] and the "too large" test is false at lo.
  while (lo < hi) {
    const uint32_t span = hi - lo;
    const uint32_t c = lo + static_cast<uint32_t>((static_cast<uint64_t>(lane + 1) * span) / kWave);
    bool too_big = false;
    if (c > 0 && d - c < B.n && c > lo) {
      too_big = cmp_keys(A.keys, key_of(A, c - 1), B.keys, key_of(B, d - c)) > 0;
    }
    const uint64_t mask = __ballot(too_big);
    // lanes [0, t) are false and lanes [t, 64) true (monotone predicate)
    const uint32_t t = mask ? static_cast<uint32_t>(__builtin_ctzll(mask)) : kWave;
    const uint32_t c_prev = t == 0 ? lo
                                   : lo + static_cast<uint32_t>((static_cast<uint64_t>(t) * span) / kWave);
    if (t == kWave) {
      lo = hi;
    } else {
      const uint32_t c_t = lo + static_cast<uint32_t>((static_cast<uint64_t>(t + 1) * span) / kWave);
      lo = c_prev;
      hi = c_t - 1;
    }
  }
  if (lane == 0) splits[wave] = lo;
}

}  // namespace em

using namespace em;

extern "C" int em_partition(const em_side_t* A, const em_side_t* B, uint32_t items_per_part,
                            uint32_t* splits, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  int rc = check_pair(A, B);
  if (rc) return rc;
  if (!splits || items_per_part == 0 || items_per_part > EM_MAX_ITEMS_PER_PART) return EM_EINVAL;
  const uint32_t N = A->n + B->n;
  const uint32_t P = (N + items_per_part - 1) / items_per_part;
  const uint32_t waves = P + 1;
  const uint32_t per_block = kPartBlock / kWave;
  const uint32_t blocks = (waves + per_block - 1) / per_block;
  hipLaunchKernelGGL(k_partition, dim3(blocks), dim3(kPartBlock), 0, as_stream(stream), *A, *B,
                     items_per_part, P, splits);
  return check_launch();
}
