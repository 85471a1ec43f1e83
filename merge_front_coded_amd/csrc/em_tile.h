// Device building blocks shared by the merge, front-coding and fused kernels:
// side selection by reference, the merge of one thread's slice of a
// partition (with the 8-byte prefix cache), and the MSB-first bit appender
// that writes records into an LDS window of output words.
#pragma once

#include "em_internal.h"

namespace em {

constexpr uint32_t kDrop = 0x80000000u;  // refs are < 2^24, bit 31 marks a dropped A

// The fields of the side a reference names, chosen by value selects (taking
// the address of a by-value kernel argument would force a private copy).
struct SideView {
  const uint8_t* keys;
  const uint32_t* key_off;
  const uint8_t* vals;
  const uint32_t* val_off;
  const uint8_t* tomb;
  bool isB;
};

__device__ __forceinline__ SideView pick(const em_side_t& A, const em_side_t& B, uint32_t ref,
                                         uint32_t& idx) {
  // A reference outside [0, |A|+|B|) can only come from contract-violating
  // inputs; it is clamped so that no access leaves the arrays.
  const uint32_t N = A.n + B.n;
  if (ref >= N) ref = N - 1;
  const bool b = ref >= A.n;
  idx = b ? ref - A.n : ref;
  return SideView{b ? B.keys : A.keys, b ? B.key_off : A.key_off, b ? B.vals : A.vals,
                  b ? B.val_off : A.val_off, b ? B.tomb : A.tomb, b};
}

__device__ __forceinline__ KeyRef key_of(const SideView& s, uint32_t r) {
  const uint32_t p = s.key_off[r];
  return KeyRef{p, s.key_off[r + 1] - p};
}

// The value's bit count in the record grammar; also its byte length (0 for a
// tombstone) and start.  All loads are issued before any is used.
__device__ __forceinline__ uint32_t value_bits(const SideView& s, uint32_t idx, uint32_t& vlen,
                                               bool& tomb, uint32_t* vpos = nullptr) {
  const uint32_t v0 = s.val_off[idx], v1 = s.val_off[idx + 1];
  // (a side without tombstone flags reads a byte it then ignores, so that the
  // load needs no branch)
  const uint8_t tv = *(s.tomb ? s.tomb + idx : reinterpret_cast<const uint8_t*>(s.val_off + idx));
  tomb = s.tomb != nullptr && tv != 0;
  vlen = tomb ? 0u : v1 - v0;
  if (vpos) *vpos = tomb ? 0u : v0;
  return tomb ? 1u : 1u + eg0_len(vlen) + 8u * vlen;
}

// Merges this thread's slice of the partition exactly.  Keys are read
// through (base, position - lo + at) per side: the LDS copy when staged, the
// arenas otherwise.  Returns the kept count; refs[] get the merged references
// with kDrop on a replaced A.
//
// Most comparisons are settled by the 8-byte prefixes and the lengths.  The
// rest (equal prefixes, both keys longer than 8 bytes: above all an A key and
// its replacing B key) need the suffixes.  A lane that meets one parks it;
// the other lanes keep stepping, and the parked comparisons of the whole wave
// are then done together, so a wave pays about one suffix comparison per
// lane instead of one per step at which any of its lanes ties.
template <int IPT>
__device__ __forceinline__ uint32_t merge_slice_exact(const uint32_t* a_off, const uint32_t* b_off,
                                                const uint64_t* a_pfx, const uint64_t* b_pfx,
                                                const uint8_t* abase, uint32_t a_adj,
                                                const uint8_t* bbase, uint32_t b_adj, uint32_t k,
                                                uint32_t len, uint32_t nA_t, uint32_t nB_t,
                                                bool has_next_b, uint32_t i0, uint32_t nA_all,
                                                uint32_t j0, uint32_t (&refs)[IPT], uint32_t cp = 0) {
  // Prefix first; zero padding plus the lengths keep proper-prefix order exact
  // (Everett, "GPU construction experiment", prefix-cache paragraph).  The
  // cached 8 bytes start cp bytes into every key, all keys sharing those cp.
  // Returns false when the suffixes must decide.
  auto quick = [&](uint32_t a, uint32_t b, int& c) -> bool {
    const uint64_t pa = a_pfx[a], pb = b_pfx[b];
    if (pa != pb) {
      c = pa < pb ? -1 : 1;
      return true;
    }
    const uint32_t la = a_off[a + 1] - a_off[a], lb = b_off[b + 1] - b_off[b];
    c = (la > lb) - (la < lb);
    return la <= cp + 8 || lb <= cp + 8;
  };
  auto suffix = [&](uint32_t a, uint32_t b) -> int {
    const uint32_t pa = a_off[a], pb = b_off[b];
    return cmp_keys(abase, KeyRef{pa - a_adj + cp + 8, a_off[a + 1] - pa - cp - 8}, bbase,
                    KeyRef{pb - b_adj + cp + 8, b_off[b + 1] - pb - cp - 8});
  };
#pragma unroll
  for (int s = 0; s < IPT; ++s) refs[s] = kDrop;
  if (k >= len) return 0;

  // co-rank of diagonal k inside the partition: the largest a with
  // A[a-1] <= B[k-a] (A first on equal keys)
  uint32_t lo = k > nB_t ? k - nB_t : 0;
  uint32_t hi = k < nA_t ? k : nA_t;
  for (;;) {
    bool park = false;
    uint32_t pmid = 0;
    while (lo < hi) {
      const uint32_t mid = (lo + hi + 1) >> 1;
      const uint32_t j = k - mid;
      int c = -1;
      if (j < nB_t && !quick(mid - 1, j, c)) {
        park = true;
        pmid = mid;
        break;
      }
      if (c > 0)
        hi = mid - 1;
      else
        lo = mid;
    }
    if (__ballot(park) == 0) break;
    if (park) {
      if (suffix(pmid - 1, k - pmid) > 0)
        hi = pmid - 1;
      else
        lo = pmid;
    }
  }

  // the thread's IPT outputs, recorded as bit masks (bit s: output s is an A,
  // and whether that A is replaced) so that parking needs no dynamic index
  // into refs[]
  const uint32_t a0 = lo, b0 = k - lo;
  const uint32_t n = len - k < static_cast<uint32_t>(IPT) ? len - k : static_cast<uint32_t>(IPT);
  uint32_t a = a0, b = b0, s = 0, amask = 0, dmask = 0;
  for (;;) {
    bool park = false, boundary = false;
    while (s < n) {
      int c;
      if (a < nA_t && b < nB_t) {
        if (!quick(a, b, c)) {
          park = true;
          break;
        }
      } else if (a < nA_t) {
        // B exhausted inside the partition: only the partition's last A can
        // equal the next partition's first B.
        c = -1;
        if (a == nA_t - 1 && has_next_b) {
          int e;
          if (!quick(a, nB_t, e)) {
            park = boundary = true;
            break;
          }
          if (e == 0) c = 0;
        }
      } else {
        c = 1;
      }
      if (c <= 0) {
        amask |= 1u << s;
        if (c == 0) dmask |= 1u << s;
        ++a;
      } else {
        ++b;
      }
      ++s;
    }
    if (__ballot(park) == 0) break;
    if (park) {
      int c = suffix(a, boundary ? nB_t : b);
      if (boundary) c = c == 0 ? 0 : -1;
      if (c <= 0) {
        amask |= 1u << s;
        if (c == 0) dmask |= 1u << s;
        ++a;
      } else {
        ++b;
      }
      ++s;
    }
  }
  a = a0;
  b = b0;
#pragma unroll
  for (int t = 0; t < IPT; ++t) {
    if (static_cast<uint32_t>(t) < n) {
      if ((amask >> t) & 1u) {
        refs[t] = (i0 + a) | (((dmask >> t) & 1u) ? kDrop : 0u);
        ++a;
      } else {
        refs[t] = nA_all + j0 + b;
        ++b;
      }
    }
  }
  return n - static_cast<uint32_t>(__builtin_popcount(dmask));
}

// The same merge with a fixed-step search and no suffix reads on the way.
// A comparison the prefixes and lengths leave open between two keys of equal
// length is taken as "equal" and the pair is noted; once the slice is merged
// every noted pair is compared in full (the whole wave at once).  If all of
// them are equal, every comparison the merge made was exact and so is its
// result; otherwise, or when a pair of different lengths is left open, `bad`
// is set and the caller redoes the partition with merge_slice_exact.
template <int IPT>
__device__ __forceinline__ uint32_t merge_slice_fast(const uint32_t* a_off, const uint32_t* b_off,
                                                     const uint64_t* a_pfx, const uint64_t* b_pfx,
                                                     const uint8_t* abase, uint32_t a_adj,
                                                     const uint8_t* bbase, uint32_t b_adj, uint32_t k,
                                                     uint32_t len, uint32_t nA_t, uint32_t nB_t,
                                                     bool has_next_b, uint32_t i0, uint32_t nA_all,
                                                     uint32_t j0, uint32_t (&refs)[IPT], bool& bad,
                                                     uint32_t* wave_list, uint32_t cp = 0) {
  constexpr int kNotes = 4;
  uint32_t note[kNotes];  // noted pairs, A index | B index << 16
#pragma unroll
  for (int q = 0; q < kNotes; ++q) note[q] = 0;
  uint32_t nnote = 0;
  bool open_pair = false;
  // c: -1, 0 or 1; a pair left open counts as 0 and is noted when `use`
  // (written with selects only: the search runs every step in every lane)
  auto cmp = [&](uint32_t a, uint32_t b, bool use) -> int {
    const uint64_t pa = a_pfx[a], pb = b_pfx[b];
    const uint32_t la = a_off[a + 1] - a_off[a], lb = b_off[b + 1] - b_off[b];
    const bool peq = pa == pb;
    const int cpfx = pa < pb ? -1 : 1;
    const int cl = (la > lb) - (la < lb);
    const bool open = use & peq & (la > cp + 8u) & (lb > cp + 8u);
    open_pair |= open & (la != lb);
    const uint32_t v = a | (b << 16);
#pragma unroll
    for (int q = 0; q < kNotes; ++q) note[q] = (open & (nnote == static_cast<uint32_t>(q))) ? v : note[q];
    nnote += open ? 1u : 0u;
    return open ? 0 : (peq ? cl : cpfx);
  };
#pragma unroll
  for (int s = 0; s < IPT; ++s) refs[s] = kDrop;
  bad = false;
  if (k >= len) return 0;

  // co-rank of diagonal k: the largest a in [lo, hi] with A[a-1] <= B[k-a],
  // by binary lifting over the same number of steps in every lane
  const uint32_t lo = k > nB_t ? k - nB_t : 0;
  const uint32_t hi = k < nA_t ? k : nA_t;
  uint32_t a = lo;
  for (uint32_t step = 1u << (31 - __builtin_clz(len)); step; step >>= 1) {
    const uint32_t m = a + step;
    const uint32_t j = k - m;
    const bool in = m <= hi;                  // then m <= k, so j did not wrap
    const bool probe = in && j < nB_t;        // B exhausted: A[m-1] is not too large
    const int c = cmp(probe ? m - 1 : 0u, probe ? j : 0u, probe);
    a = (in && !(probe && c > 0)) ? m : a;
  }

  uint32_t b = k - a;
  uint32_t kept = 0;
#pragma unroll
  for (int s = 0; s < IPT; ++s) {
    const bool live = k + s < len;
    const bool both = a < nA_t && b < nB_t;
    // B exhausted inside the partition: only the partition's last A can equal
    // the next partition's first B
    const bool edge = !both && a < nA_t && a + 1 == nA_t && has_next_b;
    const bool use = live && (both || edge);
    const int e = cmp(use ? a : 0u, both ? b : (use ? nB_t : 0u), use);
    const int c = both ? e : a < nA_t ? ((edge && e == 0) ? 0 : -1) : 1;
    if (live) {
      refs[s] = c <= 0 ? ((i0 + a) | (c == 0 ? kDrop : 0u)) : nA_all + j0 + b;
      kept += c != 0;
    }
    a += (live && c <= 0) ? 1u : 0u;
    b += (live && c > 0) ? 1u : 0u;
  }

  // Check the pairs taken as equal.  The wave's noted pairs are listed in
  // LDS (wave_list, kWave entries of this wave's own) and each lane takes
  // one, so that the key loads of up to 64 pairs are in flight together: one
  // memory round trip for the wave, instead of one per note of its busiest
  // lane.  A lane whose own notes already fail lists none.
  bool ok = !open_pair && nnote <= static_cast<uint32_t>(kNotes);
  if (__ballot(nnote != 0) != 0) {
    const uint32_t nn = ok ? nnote : 0u;  // < 8: three bits
    const uint64_t lt = (1ull << __lane_id()) - 1ull;
    uint32_t pre = 0, tot = 0;
#pragma unroll
    for (int bit = 0; bit < 3; ++bit) {
      const uint64_t m = __ballot((nn >> bit) & 1u);
      pre += static_cast<uint32_t>(__popcll(m & lt)) << bit;
      tot += static_cast<uint32_t>(__popcll(m)) << bit;
    }
    bool fail = false;
    for (uint32_t base = 0; base < tot; base += kWave) {  // (wave-uniform)
#pragma unroll
      for (int q = 0; q < kNotes; ++q) {
        const uint32_t at = pre + static_cast<uint32_t>(q);
        if (static_cast<uint32_t>(q) < nn && at >= base && at < base + kWave) wave_list[at - base] = note[q];
      }
      // (LDS accesses of one wave are performed in program order; the
      // fences keep the compiler from moving them across each other)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (base + __lane_id() < tot) {
        const uint32_t v = wave_list[__lane_id()];
        const uint32_t x = v & 0xFFFFu, y = v >> 16;
        const uint32_t px = a_off[x], py = b_off[y];
        // (a listed pair has equal lengths: a pair of different lengths set open_pair)
        fail |= cmp_keys(abase, KeyRef{px - a_adj + cp + 8, a_off[x + 1] - px - cp - 8}, bbase,
                         KeyRef{py - b_adj + cp + 8, b_off[y + 1] - py - cp - 8}) != 0;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    ok = ok && __ballot(fail) == 0;
  }
  bad = !ok;
  return kept;
}

// The merge of a workgroup's partition: every thread calls it (threads past
// the partition's end get kDrop refs and a zero count).  Exact whichever
// branch runs.  `notes` is LDS scratch of kWave words per wave of the
// workgroup.  try_fast (uniform): try the merge on the cached prefixes
// first; otherwise go straight to the exact one.  stat (nullable): when the
// first is tried, thread 0 adds 1 + (2^32 if it failed) to *stat.
template <int IPT>
__device__ __forceinline__ uint32_t merge_slice(const uint32_t* a_off, const uint32_t* b_off,
                                                const uint64_t* a_pfx, const uint64_t* b_pfx,
                                                const uint8_t* abase, uint32_t a_adj,
                                                const uint8_t* bbase, uint32_t b_adj, uint32_t k,
                                                uint32_t len, uint32_t nA_t, uint32_t nB_t,
                                                bool has_next_b, uint32_t i0, uint32_t nA_all,
                                                uint32_t j0, uint32_t (&refs)[IPT], uint32_t* notes,
                                                uint32_t cp = 0, bool try_fast = true,
                                                uint64_t* stat = nullptr) {
  bool redo = true;
  uint32_t kept = 0;
  if (try_fast) {
    bool bad;
    kept = merge_slice_fast<IPT>(a_off, b_off, a_pfx, b_pfx, abase, a_adj, bbase, b_adj, k, len, nA_t, nB_t,
                                 has_next_b, i0, nA_all, j0, refs, bad, notes + (threadIdx.x / kWave) * kWave, cp);
    redo = __syncthreads_or(bad) != 0;
    if (stat && threadIdx.x == 0)
      atomicAdd(reinterpret_cast<unsigned long long*>(stat), 1ull + (redo ? (1ull << 32) : 0ull));
  }
  if (redo)
    kept = merge_slice_exact<IPT>(a_off, b_off, a_pfx, b_pfx, abase, a_adj, bbase, b_adj, k, len, nA_t,
                                  nB_t, has_next_b, i0, nA_all, j0, refs, cp);
  return kept;
}

// Whether a partition tries the merge on cached prefixes before the exact
// one, and whether it records the outcome.  On inputs whose cached bytes tie
// between keys of different lengths in nearly every partition (long shared
// prefixes: paths, URLs), that merge almost always fails and its time is
// lost.  stat holds the partitions that tried it (low 32 bits) and those that
// failed (high 32 bits) so far in the launch.  The first kFastSample
// partitions (by ticket) and every kFastResample-th after them try it and
// record the outcome; the others read stat and skip it when at least 7/8 of
// the tries failed.  (Few recorded outcomes keep the atomic traffic on that
// one word small.)  Either way the merge is exact; only its time depends on
// the choice.
constexpr uint32_t kFastSample = 128, kFastResample = 32;

__device__ __forceinline__ bool fast_merge_records(uint32_t tile) {
  return tile < kFastSample || tile % kFastResample == 0;
}

__device__ __forceinline__ bool fast_merge_worth_trying(const uint64_t* stat, uint32_t tile) {
  if (fast_merge_records(tile)) return true;
  const uint64_t s = __hip_atomic_load(stat, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t tried = static_cast<uint32_t>(s), failed = static_cast<uint32_t>(s >> 32);
  return tried == 0 || static_cast<uint64_t>(failed) * 8u < static_cast<uint64_t>(tried) * 7u;
}

// Exact bit LCP of two keys that share their first cp bytes, from the 8
// cached bytes at cp when these settle it, else from the key bytes after them.
__device__ __forceinline__ uint32_t lcp_cached(uint64_t p, uint64_t q, uint32_t cp, const uint8_t* pb, KeyRef pk,
                                               const uint8_t* qb, KeyRef qk) {
  const uint32_t m = pk.len < qk.len ? pk.len : qk.len;  // >= cp
  if (p != q) {
    const uint32_t d = 8u * cp + static_cast<uint32_t>(__builtin_clzll(p ^ q));
    return d < 8u * m ? d : 8u * m;
  }
  if (m <= cp + 8) return 8u * m;
  return 8u * (cp + 8) + lcp_bits(pb, KeyRef{pk.pos + cp + 8, pk.len - cp - 8}, qb,
                                  KeyRef{qk.pos + cp + 8, qk.len - cp - 8});
}

// Key order of two keys that share their first cp bytes.
__device__ __forceinline__ int cmp_cached(uint64_t p, uint64_t q, uint32_t cp, const uint8_t* pb, KeyRef pk,
                                          const uint8_t* qb, KeyRef qk) {
  if (p != q) return p < q ? -1 : 1;
  if (pk.len <= cp + 8 || qk.len <= cp + 8) return (pk.len > qk.len) - (pk.len < qk.len);
  return cmp_keys(pb, KeyRef{pk.pos + cp + 8, pk.len - cp - 8}, qb, KeyRef{qk.pos + cp + 8, qk.len - cp - 8});
}

// Where the prefix cache of a partition should start (Everett, "GPU
// construction experiment", prefix-cache paragraph: the cached bytes follow
// the common prefix the compared keys are known to share).  Every cached key
// lies between the smallest and the largest of them, so all share the leading
// bytes that the first and last cached keys of each side and the two first
// keys share: the minimum of those three LCPs.  Returns 0 unless those keys
// agree in their first 8 cached bytes (a_pfx / b_pfx, loaded at offset 0),
// else that common prefix in whole bytes, measured from the key bytes.
// a_off / b_off hold the na + 1 / nb + 1 offsets of the cached keys.  Every
// thread calls it; `flag` is a word of LDS.
__device__ __forceinline__ uint32_t cache_offset(const uint32_t* a_off, uint32_t na, const uint32_t* b_off,
                                                 uint32_t nb, const uint64_t* a_pfx, const uint64_t* b_pfx,
                                                 const uint8_t* akeys, const uint8_t* bkeys, uint32_t* flag) {
  const uint32_t tid = threadIdx.x;
  if (tid == 0) {
    bool all8 = na + nb > 0;
    auto share8 = [](uint64_t p, uint32_t lp, uint64_t q, uint32_t lq) { return p == q && lp >= 8 && lq >= 8; };
    const uint32_t la0 = na ? a_off[1] - a_off[0] : 0, laz = na ? a_off[na] - a_off[na - 1] : 0;
    const uint32_t lb0 = nb ? b_off[1] - b_off[0] : 0, lbz = nb ? b_off[nb] - b_off[nb - 1] : 0;
    if (na) all8 = all8 && share8(a_pfx[0], la0, a_pfx[na - 1], laz);
    if (nb) all8 = all8 && share8(b_pfx[0], lb0, b_pfx[nb - 1], lbz);
    if (na && nb) all8 = all8 && share8(a_pfx[0], la0, b_pfx[0], lb0);
    *flag = all8 ? 0xFFFFFFFFu : 0u;
  }
  __syncthreads();
  if (__builtin_amdgcn_readfirstlane(*flag) == 0) return 0;  // (uniform)
  __syncthreads();
  if (tid < 3) {
    uint32_t l = 0xFFFFFFFFu;
    if (tid == 0 && na)
      l = lcp_bits(akeys, KeyRef{a_off[0], a_off[1] - a_off[0]}, akeys, KeyRef{a_off[na - 1], a_off[na] - a_off[na - 1]});
    else if (tid == 1 && nb)
      l = lcp_bits(bkeys, KeyRef{b_off[0], b_off[1] - b_off[0]}, bkeys, KeyRef{b_off[nb - 1], b_off[nb] - b_off[nb - 1]});
    else if (tid == 2 && na && nb)
      l = lcp_bits(akeys, KeyRef{a_off[0], a_off[1] - a_off[0]}, bkeys, KeyRef{b_off[0], b_off[1] - b_off[0]});
    atomicMin(flag, l >> 3);
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*flag);
}

// The prefix caches of both sides' keys whose offsets are in LDS: for each
// side, pfx[x] (x + 1 < n_off) is bytes [cp, cp + 8) of key x (bytes
// offs[x] .. offs[x+1] of its arena) as a big-endian word, zero past the
// key's end.  The thread takes x = threadIdx.x + u * kThreads for u < kPer.
// Every load of both sides is issued before any is waited for, whatever x
// is (a thread past the end reads its arena's first bytes and drops them):
// a load under a condition of its own was compiled into a branch with the
// wait for it inside, one memory round trip per load.
struct PfxSide {
  const uint32_t* offs;
  uint32_t n_off;
  const uint8_t* keys;
  uint64_t* pfx;
};

template <int kThreads, int kPer>
__device__ __forceinline__ void fill_prefix_caches(const PfxSide& a, const PfxSide& b, uint32_t cp) {
  // (at most five rounds of both sides in flight: ten 12-byte loads)
  constexpr int kBatch = 5;
#pragma unroll
  for (int u0 = 0; u0 < kPer; u0 += kBatch) {
    uint64_t v[2][kBatch];
    uint32_t nb[2][kBatch];
#pragma unroll
    for (int du = 0; du < kBatch && u0 + du < kPer; ++du) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const PfxSide& sd = q ? b : a;
        const uint32_t x = threadIdx.x + (u0 + du) * kThreads;
        const bool ok = x + 1 < sd.n_off;
        const uint32_t xs = ok ? x : 0u;  // (an index inside the offsets either way)
        const uint32_t p0 = sd.offs[xs], ln = sd.offs[xs + 1] - p0 - cp;
        nb[q][du] = ok ? (ln < 8u ? ln : 8u) : 0u;
        v[q][du] = load_be8(sd.keys, ok ? p0 + cp : 0u);
      }
    }
#pragma unroll
    for (int du = 0; du < kBatch && u0 + du < kPer; ++du) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const PfxSide& sd = q ? b : a;
        const uint32_t x = threadIdx.x + (u0 + du) * kThreads;
        if (x + 1 < sd.n_off) sd.pfx[x] = v[q][du] & be_mask(nb[q][du]);
      }
    }
  }
}

// Source bit positions are 32-bit for a source in LDS (a staged span) and
// 64-bit for an arena in global memory.

// 32 source bits starting at bit `bp` of a dword array (MSB-first stream order)
template <typename Pos>
__device__ __forceinline__ uint32_t bits32_at(const uint32_t* base, Pos bp) {
  const uint32_t* p = base + (bp >> 5);
  const uint32_t hi = __builtin_bswap32(p[0]), lo = __builtin_bswap32(p[1]);
  const uint32_t sh = static_cast<uint32_t>(bp & 31u);
  // v_alignbit takes its shift modulo 32, so offset 0 is the high dword itself
  return sh ? __builtin_amdgcn_alignbit(hi, lo, 32u - sh) : hi;
}

// Source bits [bp, bp + n) of a dword array placed at an output position
// that is f bits into output word o[0] (the caller writes o[0] itself, from
// the first 32 - f source bits):
// output word i >= 1 holds source bits [P, P + 32) with P = bp + 32 i - f,
// so every one of them is one funnel shift of two consecutive source dwords
// with a shift that is the same for the whole span.  Words 1 .. W-1 are
// stored; the bits of the partial word W (when f2 = (f + n) mod 32 > 0) are
// returned.  Reads of global memory reach at most one dword past the one
// holding the span's last bit; reads of LDS at most five.
template <typename Pos>
__device__ __forceinline__ uint32_t span_words(uint32_t* o, const uint32_t* base, Pos bp, uint32_t f,
                                               uint32_t W, uint32_t f2) {
  // P >= 1: bits of dwords (P - 1) / 32 and the next, shifted right by -P
  // mod 32 (a shift of 0 gives the second dword)
  const uint32_t* p = base + ((bp + 31u - f) >> 5);
  const uint32_t sh = (f - static_cast<uint32_t>(bp)) & 31u;
  o += 1;
  const uint32_t cnt = W - 1;  // words 1 .. W-1 go to o[0 .. cnt)
  uint32_t cur = __builtin_bswap32(p[0]);
  // (the loop's end is computed up front, so that its counter is not needed
  // after it)
  const uint32_t t = cnt & ~3u, rem = cnt & 3u;
  // the last source dword needed; indices past it re-read it
  const uint32_t last = t + rem + (f2 ? 1u : 0u);
  // source dwords 1 .. 4 past the current one (raw), loaded one round ahead
  // of their use, so that each round's loads overlap the previous round's
  // shifts and stores.  A source in LDS (32-bit positions: a staged span) is
  // read up to four dwords past `last`, which stays inside the workgroup's
  // LDS (the stage is followed by other arrays) and is never used; a source
  // in global memory re-reads `last` instead.
  auto ld = [&](uint32_t k) -> uint32_t {
    if constexpr (sizeof(Pos) == 4)
      return p[k];
    else
      return p[min(k, last)];
  };
  uint32_t n1 = p[min(1u, last)], n2 = p[min(2u, last)], n3 = p[min(3u, last)], n4 = p[min(4u, last)];
  for (uint32_t i = 0; i < t; i += 4) {
    const uint32_t m1 = ld(i + 5), m2 = ld(i + 6), m3 = ld(i + 7), m4 = ld(i + 8);
    const uint32_t b1 = __builtin_bswap32(n1), b2 = __builtin_bswap32(n2);
    const uint32_t b3 = __builtin_bswap32(n3), b4 = __builtin_bswap32(n4);
    o[i] = __builtin_amdgcn_alignbit(cur, b1, sh);
    o[i + 1] = __builtin_amdgcn_alignbit(b1, b2, sh);
    o[i + 2] = __builtin_amdgcn_alignbit(b2, b3, sh);
    o[i + 3] = __builtin_amdgcn_alignbit(b3, b4, sh);
    cur = b4;
    n1 = m1, n2 = m2, n3 = m3, n4 = m4;
  }
  // up to three more words, then the partial word (source dwords t+1 ..
  // t+rem, and one more when f2 > 0, already loaded)
  const uint32_t m1 = __builtin_bswap32(n1), m2 = __builtin_bswap32(n2);
  const uint32_t m3 = __builtin_bswap32(n3), m4 = __builtin_bswap32(n4);
  if (rem > 0) o[t] = __builtin_amdgcn_alignbit(cur, m1, sh);
  if (rem > 1) o[t + 1] = __builtin_amdgcn_alignbit(m1, m2, sh);
  if (rem > 2) o[t + 2] = __builtin_amdgcn_alignbit(m2, m3, sh);
  uint32_t acc = 0;
  if (f2) {
    const uint32_t x = rem == 0 ? cur : rem == 1 ? m1 : rem == 2 ? m2 : m3;
    const uint32_t y = rem == 0 ? m1 : rem == 1 ? m2 : rem == 2 ? m3 : m4;
    acc = __builtin_amdgcn_alignbit(x, y, sh) & ~(0xFFFFFFFFu >> f2);
  }
  return acc;
}

// Direct placement into a window that is zero wherever nothing has been
// written yet: the n low bits of v (1 <= n <= 64), MSB first, at bit p.
// Every word is ORed (other fields and records may share them).
__device__ __forceinline__ void or_bits64(uint32_t* out, uint32_t p, uint64_t v, uint32_t n) {
  const uint32_t f = p & 31u;
  uint32_t* o = out + (p >> 5);
  const uint64_t u = v << (64u - n);  // left-aligned
  const uint32_t hi = static_cast<uint32_t>(u >> 32), lo = static_cast<uint32_t>(u);
  atomicOr(o, hi >> f);
  if (f + n > 32u) atomicOr(o + 1, __builtin_amdgcn_alignbit(hi, lo, f));  // (a shift of 0 gives lo)
  if (f + n > 64u) atomicOr(o + 2, lo << (32u - f));                      // (f > 0 here)
}

// Direct placement of source bits [bp, bp + n) of a dword array at window bit
// p: the first and the last word, which neighbouring fields may share, are
// ORed, and every word between them is stored.
template <typename Pos>
__device__ __forceinline__ void or_span(uint32_t* out, uint32_t p, const uint32_t* base, Pos bp, uint32_t n) {
  if (n == 0) return;
  const uint32_t f = p & 31u;
  uint32_t* o = out + (p >> 5);
  const uint32_t x0 = bits32_at(base, bp);
  if (f + n <= 32u) {
    atomicOr(o, (n >= 32u ? x0 : x0 & ~(0xFFFFFFFFu >> n)) >> f);
    return;
  }
  if (f)
    atomicOr(o, x0 >> f);
  else
    o[0] = x0;  // the span covers the whole word
  const uint32_t W = (f + n) >> 5, f2 = (f + n) & 31u;
  const uint32_t acc = span_words(o, base, bp, f, W, f2);
  if (f2) atomicOr(o + W, acc);
}

// Co-rank of diagonal d (A records among the first d outputs of the stable
// merge, ties to A) inside [lo, hi], where the "too large" test A[i-1] > B[d-i]
// is false at lo.  Searched by a group of G lanes (G a power of two up to
// 64): t is the lane in the group, gshift the group's first lane in the
// wave.  Each round tests G evenly spaced candidates and a ballot finds the
// crossing, shrinking the range G-fold.
template <uint32_t G>
__device__ __forceinline__ uint32_t corank_group(const em_side_t& A, const em_side_t& B, uint32_t d, uint32_t lo,
                                                 uint32_t hi, uint32_t t, uint32_t gshift) {
  static_assert(G >= 2 && G <= 64 && (G & (G - 1)) == 0, "a power of two lanes, at most a wave");
  while (lo < hi) {
    const uint32_t span = hi - lo;
    const uint32_t c = lo + static_cast<uint32_t>((static_cast<uint64_t>(t + 1) * span) / G);
    bool too_big = false;
    if (c > 0 && d - c < B.n && c > lo) {
      too_big = cmp_keys(A.keys, key_of(A, c - 1), B.keys, key_of(B, d - c)) > 0;
    }
    const uint64_t gmask = G == 64 ? ~0ull : ((1ull << G) - 1);
    const uint64_t mask = (__ballot(too_big) >> gshift) & gmask;
    // lanes [0, f) of the group are false and lanes [f, G) true (monotone predicate)
    const uint32_t f = mask ? static_cast<uint32_t>(__builtin_ctzll(mask)) : G;
    const uint32_t c_prev = lo + static_cast<uint32_t>((static_cast<uint64_t>(f) * span) / G);
    if (f == G) {
      lo = hi;
    } else {
      const uint32_t c_f = lo + static_cast<uint32_t>((static_cast<uint64_t>(f + 1) * span) / G);
      lo = c_prev;
      hi = c_f - 1;
    }
  }
  return lo;
}

__device__ __forceinline__ uint32_t corank16(const em_side_t& A, const em_side_t& B, uint32_t d, uint32_t lo,
                                             uint32_t hi, uint32_t t, uint32_t gshift) {
  return corank_group<16>(A, B, d, lo, hi, t, gshift);
}

// Co-rank of diagonal d given coarse co-ranks around it: csplits[c] is the
// co-rank of diagonal c * coarse (em_partition's output for `coarse`
// outputs per partition, Pc partitions).  Read directly at a coarse
// boundary, searched by corank16 inside the coarse partition otherwise (a
// group of 16 lanes: t is the lane in the group, gshift its first lane).
__device__ __forceinline__ uint32_t fine_corank(const em_side_t& A, const em_side_t& B,
                                                const uint32_t* csplits, uint32_t coarse, uint32_t Pc,
                                                uint32_t d, uint32_t t, uint32_t gshift) {
  const uint32_t N = A.n + B.n;
  if (d >= N) return csplits[Pc];
  const uint32_t c = d / coarse;
  if (d == c * coarse) return csplits[c];
  const uint32_t Dc = c * coarse, Dn = min(Dc + coarse, N);
  const uint32_t Ic = csplits[c], In = csplits[c + 1];
  const uint32_t Jc = Dc - Ic, Jn = Dn - In;
  uint32_t lo = max(max(Ic, d > Jn ? d - Jn : 0u), d > B.n ? d - B.n : 0u);
  uint32_t hi = min(min(In, d - min(Jc, d)), min(d, A.n));
  if (hi < lo) hi = lo;  // only for coarse splits that do not come from em_partition
  return corank16(A, B, d, lo, hi, t, gshift);
}

}  // namespace em
