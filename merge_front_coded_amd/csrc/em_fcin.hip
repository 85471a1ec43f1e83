// Front-coded input: a payload (with its navigation or its record offsets)
// decoded back into key and value arenas, so that a compressed side can enter
// the merge.
//
// Everett, "GPU construction experiment":
//  * block parse: GPU select gives each block's physical offset (with the
//    common-value-width correction); one invocation parses a block's at most
//    fifteen records: its first control gives the absolute retained length,
//    later controls count back from the predecessor's key length, values are
//    skipped by their own grammar and their bit spans recorded;
//  * literal owners: with r_i record i's retained key length, bit p of key i
//    belongs to the literal of j = max{t <= i : r_t <= p}; a minimum tree over
//    the retained lengths answers that query in O(log n): from the record's
//    leaf, go up until some left sibling's minimum is <= p, then go down
//    into the right child whenever its minimum is <= p (else the left one);
//    leaves past the last record hold an infinite value.  A byte resolved from its highest bit backward can
//    combine several literal fragments;
//  * full-key materialization as a consumer of the same descriptors (the
//    paragraph that names it as the alternative to owner searches during
//    comparison): every key is written out whole, then the ordinary merge
//    runs on the arenas.
//
// Following the owners from the top bit of key i down, the fragments are
// contiguous: the owner j of bit r_i - 1 owns all of [r_j, r_i) (every record
// after j up to i retains more than r_i - 1 bits), then the owner of bit
// r_j - 1 takes over, and so on down to a record with r = 0.
#include <algorithm>

#include "em_internal.h"

namespace em {

constexpr int kFiBlock = 256;
constexpr uint32_t kFiRecs = 15;  // records per block (the W15 period)
constexpr uint32_t kFiInf = 0xFFFFFFFFu;
constexpr int kFpBlock = 256;
constexpr uint32_t kFpPer = 16;                  // rows of kFpBlock records per tile
constexpr uint32_t kFpTile = kFpBlock * kFpPer;  // records per workgroup
constexpr int kFpTilesBlock = 1024;
constexpr uint32_t kFpTilesPer = 4;  // tiles per thread of the tile scan: EM_MAX_RECORDS / kFpTile / 1024

enum : uint64_t {
  kFiErrRange = 1,    // a field reaches past T, or an EG0 code is malformed
  kFiErrPrefix = 2,   // an inherited prefix longer than the predecessor's key
  kFiErrBytes = 4,    // a key that is not whole bytes
  kFiErrBlock = 8,    // a block does not end where the next one starts
  kFiErrTotal = 16,   // an arena of 2^32 bytes or more
  kFiErrCap = 32,     // an output arena smaller than the decoded bytes
};

struct FiLayout {
  uint32_t S, nb, P2;
  uint64_t* starts;   // nb block start bits
  uint32_t* r;        // S retained key bits
  uint32_t* kbytes;   // S + 1 key bytes (scan input; entry S is 0)
  uint32_t* vbytes;   // S + 1 value bytes
  uint64_t* lit;      // S payload bit of each literal's first bit
  uint8_t* tflag;     // S tombstone flags
  uint64_t* koff;     // S + 2 key arena offsets (scan output)
  uint64_t* voff;     // S + 2 value arena offsets
  uint32_t* tree;     // 2 P2 minimum tree over r (heap order, leaves at P2)
  uint32_t* pse;      // S: the last earlier record with a smaller r (kFiInf: none)
  uint64_t* fp_agg;   // prefix cache: per tile of kFpTile records, its composed step (m, v)
  uint64_t* fp_x;     // prefix cache: per tile, the first 64 key bits of the record before it
  uint8_t* scan_ws;
  size_t scan_bytes;
  size_t used;
};

static FiLayout fi_layout(void* ws, uint32_t S) {
  FiLayout L{};
  L.S = S;
  L.nb = (S + kFiRecs - 1) / kFiRecs;
  L.P2 = 1;
  while (L.P2 < S) L.P2 <<= 1;
  WsCursor cur{static_cast<uint8_t*>(ws), 0};
  const size_t n = static_cast<size_t>(S) + 2;
  L.starts = cur.take<uint64_t>(L.nb + 1);
  L.r = cur.take<uint32_t>(n);
  L.kbytes = cur.take<uint32_t>(n);
  L.vbytes = cur.take<uint32_t>(n);
  L.lit = cur.take<uint64_t>(n);
  L.tflag = cur.take<uint8_t>(n);
  L.koff = cur.take<uint64_t>(n);
  L.voff = cur.take<uint64_t>(n);
  L.tree = cur.take<uint32_t>(2 * static_cast<size_t>(L.P2));
  L.pse = cur.take<uint32_t>(n);
  L.fp_agg = cur.take<uint64_t>(2 * (static_cast<size_t>(S) / kFpTile + 1));
  L.fp_x = cur.take<uint64_t>(static_cast<size_t>(S) / kFpTile + 1);
  L.scan_bytes = scan_ws(S + 1);
  L.scan_ws = cur.take<uint8_t>(L.scan_bytes);
  L.used = cur.used;
  return L;
}

static inline uint32_t fi_blocks(uint64_t n) { return static_cast<uint32_t>((n + kFiBlock - 1) / kFiBlock); }

// The payload as a bit stream: 32 bits starting at bit x (MSB first), zero
// past the stored words.
struct FiBits {
  const uint32_t* w;
  uint64_t nwords;
  __device__ __forceinline__ uint32_t word(uint64_t i) const {
    return i < nwords ? __builtin_bswap32(w[i]) : 0u;
  }
  // (the two words in one 8-byte load: multi-dword loads need only dword
  // alignment)
  __device__ __forceinline__ uint32_t at32(uint64_t x) const {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2), aligned(4)));
    const uint64_t i = x >> 5;
    const uint32_t s = static_cast<uint32_t>(x & 31u);
    uint32_t hi, lo;
    if (i + 1 < nwords) {
      const u32x2 q = *reinterpret_cast<const u32x2*>(w + i);
      hi = __builtin_bswap32(q.x);
      lo = __builtin_bswap32(q.y);
    } else {
      hi = word(i);
      lo = word(i + 1);
    }
    return s ? __builtin_amdgcn_alignbit(hi, lo, 32u - s) : hi;
  }
  // words i .. i+3 with one 16-byte load (multi-dword loads need only dword
  // alignment), word by word at the end of the payload
  __device__ __forceinline__ void word4(uint64_t i, uint32_t (&v)[4]) const {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4), aligned(4)));
    if (i + 3 < nwords) {
      const u32x4 q = *reinterpret_cast<const u32x4*>(w + i);
      v[0] = __builtin_bswap32(q.x);
      v[1] = __builtin_bswap32(q.y);
      v[2] = __builtin_bswap32(q.z);
      v[3] = __builtin_bswap32(q.w);
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] = word(i + t);
    }
  }
};

// The payload as a bit stream read through an LDS copy of words
// [w0, w0 + n) (raw, as stored), the rest from global memory: the same
// values as FiBits, for a workgroup that staged the span it reads.
struct FiWin {
  const uint32_t* lds;
  uint64_t w0;
  uint32_t n;
  FiBits g;
  __device__ __forceinline__ uint32_t word(uint64_t i) const {
    const uint64_t d = i - w0;
    return d < n ? __builtin_bswap32(lds[d]) : g.word(i);
  }
  __device__ __forceinline__ uint32_t at32(uint64_t x) const {
    const uint64_t i = x >> 5;
    const uint32_t s = static_cast<uint32_t>(x & 31u);
    const uint32_t hi = word(i), lo = word(i + 1);
    return s ? __builtin_amdgcn_alignbit(hi, lo, 32u - s) : hi;
  }
};

// Words [w0, w1) of the payload, from w0 rounded down to a multiple of four,
// clamped to the stored words and to kWords, into lds (16-byte aligned) by the
// workgroup of kThreads: 16-byte loads, all issued before the stores.
// Returns how many words lds holds (w0 is updated); the caller synchronises
// before reading them.
template <int kThreads, uint32_t kWords>
__device__ __forceinline__ uint32_t fi_stage(uint32_t* __restrict__ lds, const FiBits& g, uint64_t& w0, uint64_t w1) {
  static_assert(kWords % (4 * kThreads) == 0, "whole rounds of 16-byte loads");
  constexpr int kIters = kWords / (4 * kThreads);
  w0 &= ~static_cast<uint64_t>(3);
  w1 = min_u64(w1, g.nwords);
  const uint32_t n = w1 > w0 ? static_cast<uint32_t>(min_u64(w1 - w0, kWords)) : 0u;
  const uint32_t n4 = n / 4;
  const uint4* src = reinterpret_cast<const uint4*>(g.w + w0);
  if (n4) {  // (uniform)
    // Every load is issued whatever x is (a lane past the end loads group 0
    // again), and every loaded value is used once outside the stores'
    // conditions (an empty asm), so that the compiler keeps the loads
    // together: a load left to its store's branch was compiled with the wait
    // for it right behind it, one memory round trip per load.
    uint4 v[kIters];
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const uint32_t x = threadIdx.x + it * kThreads;
      v[it] = src[x < n4 ? x : 0u];
    }
#pragma unroll
    for (int it = 0; it < kIters; ++it) asm volatile("" ::"v"(v[it].x));
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const uint32_t x = threadIdx.x + it * kThreads;
      if (x < n4) reinterpret_cast<uint4*>(lds)[x] = v[it];
    }
  }
  for (uint32_t t = 4 * n4 + threadIdx.x; t < n; t += kThreads) lds[t] = g.w[w0 + t];
  return n;
}

// ---- block starts ----

// From record offsets: block k starts at off[15k].
__global__ __launch_bounds__(kFiBlock) void k_fi_starts_off(const uint64_t* __restrict__ off, uint32_t nb,
                                                            uint64_t* __restrict__ starts) {
  const uint32_t k = blockIdx.x * kFiBlock + threadIdx.x;
  if (k < nb) starts[k] = off[static_cast<uint64_t>(k) * kFiRecs];
}

// From the navigation sections: select entry k (a sparse group lists its
// high-bit positions; a dense one is walked from its sample), add the common
// width times the ordinal back.
__global__ __launch_bounds__(kFiBlock) void k_fi_starts_ef(const em_ef_info_t* __restrict__ info,
                                                           const uint64_t* __restrict__ lows,
                                                           const uint64_t* __restrict__ highs,
                                                           const uint64_t* __restrict__ samples,
                                                           const uint64_t* __restrict__ exceptions, uint32_t nb,
                                                           uint64_t* __restrict__ starts) {
  const uint32_t k = blockIdx.x * kFiBlock + threadIdx.x;
  if (k >= nb) return;
  const uint64_t L = info->L, w = info->width, G = info->groups, hw = info->high_words;
  const uint32_t g = k / 256, rk = k % 256;
  const uint64_t x0 = samples[2ull * g + 1];
  const uint64_t x1 = g + 1 < G ? samples[2ull * g + 3] : info->exceptions;
  uint64_t p;
  if (x1 > x0) {
    p = exceptions[x0 + rk];
  } else {
    // the rk-th set bit at or after the group's first one
    p = samples[2ull * g];
    uint64_t wi = p >> 6;
    uint64_t word = wi < hw ? highs[wi] & (~0ull << (p & 63)) : 0ull;
    uint32_t need = rk;
    while (true) {
      const uint32_t c = static_cast<uint32_t>(__builtin_popcountll(word));
      if (need < c || wi + 1 >= hw) break;
      need -= c;
      word = highs[++wi];
    }
    for (uint32_t t = 0; t < need; ++t) word &= word - 1;  // drop the lower set bits
    p = 64 * wi + (word ? static_cast<uint64_t>(__builtin_ctzll(word)) : 63ull);
  }
  uint64_t low = 0;
  if (L) {
    const uint64_t at = static_cast<uint64_t>(k) * L;
    low = lows[at >> 6] >> (at & 63);
    if ((at & 63) + L > 64) low |= lows[(at >> 6) + 1] << (64 - (at & 63));
    low &= (L == 64 ? ~0ull : (1ull << L) - 1);
  }
  const uint64_t e = ((p - k) << L) | low;
  starts[k] = e + static_cast<uint64_t>(k) * kFiRecs * w;
}

// ---- block parse: one lane per block of at most 15 records ----

// 64 bits of the payload from bit x on (MSB first, zero past the stored words)
__device__ __forceinline__ uint64_t fi_peek64(const FiWin& b, uint64_t x) {
  const uint64_t i = x >> 5;
  const uint32_t sft = static_cast<uint32_t>(x & 31u);
  const uint32_t a = b.word(i), c1 = b.word(i + 1), c2 = b.word(i + 2);
  const uint32_t hi = sft ? __builtin_amdgcn_alignbit(a, c1, 32u - sft) : a;
  const uint32_t lo = sft ? __builtin_amdgcn_alignbit(c1, c2, 32u - sft) : c1;
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// One order-0 Exp-Golomb code at the top of a 64-bit window: its value and
// length, or length 0 when the window does not hold it (a code here is at
// most 63 bits: its value is below 2^31).
__device__ __forceinline__ uint32_t fi_eg0_win(uint64_t win, uint32_t& len) {
  const uint32_t z = win ? static_cast<uint32_t>(__builtin_clzll(win)) : 64u;
  if (z > 31u) {
    len = 0;
    return 0;
  }
  len = 2 * z + 1;
  return static_cast<uint32_t>(win >> (64 - len)) - 1u;
}

// Parse: a one-wave workgroup takes G consecutive blocks (G chosen so that
// their span of the payload, which is contiguous, usually fits the LDS
// window), stages that span with coalesced loads and parses one block per
// lane from LDS (reads past the staged words go to global memory).  Each
// record costs two 64-bit windows (its two controls, then the value header);
// the outputs go through restrict pointers, so that no store holds back a
// later load.
constexpr uint32_t kFiParseWave = 64;
constexpr uint32_t kFiParseWords = 2048;  // 8 KB of payload

__global__ __launch_bounds__(kFiParseWave) void k_fi_parse(FiBits bits, uint64_t T, uint32_t S, uint32_t nb,
                                                           uint32_t G, const uint64_t* __restrict__ starts,
                                                           uint32_t* __restrict__ r_out,
                                                           uint32_t* __restrict__ kbytes,
                                                           uint32_t* __restrict__ vbytes, uint64_t* __restrict__ lit,
                                                           uint8_t* __restrict__ tflag,
                                                           uint64_t* __restrict__ err) {
  __shared__ __align__(16) uint32_t span[kFiParseWords];
  const uint32_t k0 = blockIdx.x * G;
  const uint32_t k1 = min(k0 + G, nb);
  const uint64_t p0 = starts[k0], p1 = k1 < nb ? starts[k1] : T;
  // (+3 words: a 64-bit window at the last value header reads three)
  uint64_t w0 = p0 >> 5;
  const uint32_t n = p1 >= p0 ? fi_stage<kFiParseWave, kFiParseWords>(span, bits, w0, (p1 >> 5) + 3) : 0u;
  __syncthreads();
  const FiWin win{span, w0, n, bits};
  const uint32_t k = k0 + threadIdx.x;
  if (threadIdx.x >= G || k >= k1) return;
  const uint32_t i0 = k * kFiRecs, i1 = min(i0 + kFiRecs, S);
  uint64_t pos = starts[k];
  const uint64_t end = k + 1 < nb ? starts[k + 1] : T;
  uint64_t e = pos > T ? static_cast<uint64_t>(kFiErrBlock) : 0;
  uint32_t kprev = 0;
  for (uint32_t i = i0; i < i1 && !e; ++i) {
    uint64_t w64 = fi_peek64(win, pos);
    uint32_t n1, n2 = 0;
    const uint32_t c = fi_eg0_win(w64, n1);
    uint32_t s = 0;
    if (n1) {
      if (n1 < 64) s = fi_eg0_win(w64 << n1, n2);
      if (n1 == 64 || n1 + n2 > 64 || n2 == 0) {  // (a rare long pair: read the second code afresh)
        w64 = fi_peek64(win, pos + n1);
        s = fi_eg0_win(w64, n2);
        if (!n2) e |= kFiErrRange;
      }
    } else {
      e |= kFiErrRange;
    }
    if (pos + n1 + n2 > T) e |= kFiErrRange;
    pos += n1 + n2;
    uint32_t l;
    if (i == i0) {  // i mod 15 = 0: c = 1 + l
      l = c - 1u;
      if (c == 0 || (i == 0 && l != 0)) e |= kFiErrPrefix;
    } else {
      l = kprev - c;
      if (c > kprev) e |= kFiErrPrefix;
    }
    const uint64_t kb = static_cast<uint64_t>(l) + s;
    if (kb & 7u) e |= kFiErrBytes;
    r_out[i] = l;
    kbytes[i] = static_cast<uint32_t>(kb >> 3);
    lit[i] = pos;
    pos += s;  // the literal
    // value header: presence bit, then EG0(byte length)
    const uint64_t vw = fi_peek64(win, pos);
    uint32_t vlen = 0, nv = 1;
    const bool present = (vw >> 63) != 0;
    if (present) {
      uint32_t n3;
      vlen = fi_eg0_win(vw << 1, n3);
      if (!n3) e |= kFiErrRange;
      nv += n3;
    }
    if (pos + nv > T) e |= kFiErrRange;
    pos += nv;
    vbytes[i] = vlen;
    tflag[i] = present ? 0 : 1;
    pos += 8ull * vlen;
    if (pos > T) e |= kFiErrRange;
    kprev = static_cast<uint32_t>(kb);
  }
  // the block must end where the next one starts (the last one at T)
  if (!e && pos != end) e |= kFiErrBlock;
  if (k == 0) {
    kbytes[S] = 0;
    vbytes[S] = 0;
  }
  if (e) atomicOr(reinterpret_cast<unsigned long long*>(err), static_cast<unsigned long long>(e));
}

// ---- minimum tree over the retained lengths ----

__global__ __launch_bounds__(kFiBlock) void k_fi_leaves(const uint32_t* __restrict__ r, uint32_t S, uint32_t P2,
                                                        uint32_t* __restrict__ tree) {
  const uint32_t i = blockIdx.x * kFiBlock + threadIdx.x;
  if (i < P2) tree[P2 + i] = i < S ? r[i] : kFiInf;
}

// Levels first, first / 2, ... of the tree, from their children: a
// workgroup takes cnt0 = min(256, first) consecutive nodes of level `first`
// and the subtree above them in LDS, down to one node (1 + log2 cnt0 levels
// per launch).
__global__ __launch_bounds__(kFiBlock) void k_fi_levels(uint32_t* __restrict__ tree, uint32_t first,
                                                        uint32_t cnt0) {
  __shared__ uint32_t buf[kFiBlock];
  const uint32_t t = threadIdx.x;
  uint32_t cnt = cnt0, f = first;
  uint32_t m = kFiInf;
  if (t < cnt) {
    const uint32_t v = f + blockIdx.x * cnt + t;
    m = min(tree[2 * v], tree[2 * v + 1]);
    tree[v] = m;
    buf[t] = m;
  }
  while (cnt > 1) {
    __syncthreads();
    cnt >>= 1;
    f >>= 1;
    if (t < cnt) m = min(buf[2 * t], buf[2 * t + 1]);
    __syncthreads();
    if (t < cnt) {
      buf[t] = m;
      tree[f + blockIdx.x * cnt + t] = m;
    }
  }
}

// The literal owner of bit p of key i, p < r_i: j = max{t <= i : r_t <= p}.
__device__ __forceinline__ uint32_t fi_owner(const uint32_t* __restrict__ tree, uint32_t P2, uint32_t i,
                                             uint32_t p) {
  uint32_t v = P2 + i;
  while (v > 1) {
    if ((v & 1u) && tree[v - 1] <= p) {  // a left sibling holds a record with r <= p
      v -= 1;
      while (v < P2) v = tree[2 * v + 1] <= p ? 2 * v + 1 : 2 * v;
      return v - P2;
    }
    v >>= 1;
  }
  return kFiInf;  // none (only for p outside every key; the parse rules this out)
}

// ---- materialization ----
// The owner chain of key i is a chain of "previous smaller" records: the
// owner of bit r_i - 1 is pse(i) = max{t < i : r_t < r_i} (every record after
// it up to i retains at least r_i bits), and the owner of the bit below
// fragment j's start is pse(j).  pse comes from one owner query per record.
// Block heads (records 15k) follow their chain to a record with r = 0 for
// their inherited bytes (the kernel before writes those); any other record
// follows it while it stays inside its block and takes the bits below from
// its block head's key (all records from the head on keep those bits).

__global__ __launch_bounds__(kFiBlock) void k_fi_pse(FiLayout L) {
  const uint32_t i = blockIdx.x * kFiBlock + threadIdx.x;
  if (i >= L.S) return;
  const uint32_t r = L.r[i];
  L.pse[i] = r ? fi_owner(L.tree, L.P2, i, r - 1) : kFiInf;
}

// nbytes bytes from payload bit x on.  Output dword m is bits
// [x + 32m, x + 32m + 32), one funnel shift of payload words i0 + m and
// i0 + m + 1 (i0 = x / 32), so each payload word is read once; sixteen bytes
// at a time, the four words of a group in one 16-byte load issued before the
// group's stores (a byte store may alias any load, so a load after it would
// wait for it), whole words where the destination is aligned.
template <class Bits>
__device__ __forceinline__ void fi_copy_bytes(const Bits& bits, uint64_t x, uint8_t* __restrict__ dst,
                                              uint32_t nbytes) {
  if (nbytes == 0) return;
  const uint64_t i0 = x >> 5;
  const uint32_t sh = static_cast<uint32_t>(x & 31u);
  uint32_t prev = bits.word(i0);
  uint32_t m = 0;
  for (; m + 16 <= nbytes; m += 16) {
    uint32_t nx[4], v[4];
    bits.word4(i0 + m / 4 + 1, nx);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t a = t ? nx[t - 1] : prev;
      v[t] = sh ? __builtin_amdgcn_alignbit(a, nx[t], 32u - sh) : a;
    }
    prev = nx[3];
    if ((reinterpret_cast<uintptr_t>(dst + m) & 3) == 0) {
#pragma unroll
      for (int t = 0; t < 4; ++t) *reinterpret_cast<uint32_t*>(dst + m + 4 * t) = __builtin_bswap32(v[t]);
    } else {
#pragma unroll
      for (int t = 0; t < 16; ++t) dst[m + t] = static_cast<uint8_t>(v[t >> 2] >> (24 - 8 * (t & 3)));
    }
  }
  for (; m < nbytes; m += 4) {
    const uint32_t nx = bits.word(i0 + m / 4 + 1);
    const uint32_t v = sh ? __builtin_amdgcn_alignbit(prev, nx, 32u - sh) : prev;
    prev = nx;
    const uint32_t n = nbytes - m < 4 ? nbytes - m : 4;
    for (uint32_t t = 0; t < n; ++t) dst[m + t] = static_cast<uint8_t>(v >> (24 - 8 * t));
  }
}

// Key i from the top byte down.  The current fragment (record j) covers key
// bits [lo, hi] with key bit q at payload bit base + q.  head = kFiInf: the
// chain runs to the end; else bits below a fragment whose pse is at or
// before `head` come from the head's key in the arena.
template <class Bits>
__device__ __forceinline__ void fi_key(const Bits& bits, const FiLayout& L, uint32_t i, uint32_t head,
                                       const uint8_t* __restrict__ head_key, uint8_t* __restrict__ key,
                                       uint32_t kb, uint64_t* __restrict__ err) {
  uint32_t j = i;
  uint32_t lo = L.r[i];
  uint64_t base = L.lit[i] - lo;
  bool from_head = false;  // bits below lo are the head key's
  // the bytes wholly inside the record's own literal: a straight copy
  const uint32_t own = (lo + 7) >> 3;
  if (own < kb) fi_copy_bytes(bits, base + 8ull * own, key + own, kb - own);
  for (uint32_t b = own < kb ? own : kb; b-- > 0;) {
    uint32_t byte = 0;
    uint32_t hi = 8 * b + 7;  // highest key bit of this byte still to fill
    while (true) {
      if (lo > hi && !from_head) {
        const uint32_t nj = L.pse[j];
        if (head != kFiInf && (nj == kFiInf || nj <= head)) {
          from_head = true;
        } else {
          if (nj == kFiInf || L.r[nj] > hi) {
            atomicOr(reinterpret_cast<unsigned long long*>(err), static_cast<unsigned long long>(kFiErrPrefix));
            return;
          }
          j = nj;
          lo = L.r[j];
          base = L.lit[j] - lo;
        }
      }
      if (from_head && lo > hi) {  // bits [8b, hi] from the head key
        byte |= head_key[b] & (0xFFu << (7u - (hi & 7u)));
        break;
      }
      const uint32_t rl = max(8 * b, lo);  // run [rl, hi] from the current fragment, 1..8 bits
      const uint32_t n = hi - rl + 1;
      const uint32_t v = bits.at32(base + rl) >> (32u - n);
      byte |= v << (7u - (hi & 7u));
      if (rl == 8 * b) break;
      hi = rl - 1;  // the rest of the byte lies below this fragment
    }
    key[b] = static_cast<uint8_t>(byte);
  }
}

// a block's first record may not inherit more than its predecessor's key;
// the arenas must hold the record
__device__ __forceinline__ bool fi_record_ok(const FiLayout& L, uint32_t i, uint64_t key_cap, uint64_t val_cap) {
  if (i > 0 && L.r[i] > 8u * L.kbytes[i - 1]) return false;
  return L.koff[i] + L.kbytes[i] <= key_cap && L.voff[i] + L.vbytes[i] <= val_cap;
}

// Payload bits [x, x + 8 n) to LDS bytes dst[0, n): single byte stores up
// to dst's first 4-byte boundary and after its last, whole dwords between
// them, each one funnel shift of two payload words with a shift that is the
// same for the whole run (as in fi_copy_bytes).
template <class Bits>
__device__ __forceinline__ void fi_copy_to_lds(const Bits& bits, uint64_t x, uint8_t* dst, uint32_t n) {
  if (n == 0) return;
  const uint32_t head = min((4u - (static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst)) & 3u)) & 3u, n);
  if (head) {
    const uint32_t v = bits.at32(x);
    for (uint32_t t = 0; t < head; ++t) dst[t] = static_cast<uint8_t>(v >> (24u - 8u * t));
  }
  const uint32_t nd = (n - head) >> 2;
  if (nd) {
    const uint64_t y = x + 8ull * head;
    const uint64_t i0 = y >> 5;
    const uint32_t sh = static_cast<uint32_t>(y & 31u);
    uint32_t* d = reinterpret_cast<uint32_t*>(dst + head);
    uint32_t prev = bits.word(i0);
    uint32_t k = 0;
    for (; k + 4 <= nd; k += 4) {
      uint32_t nx[4];
      bits.word4(i0 + k + 1, nx);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t a = t ? nx[t - 1] : prev;
        d[k + t] = __builtin_bswap32(sh ? __builtin_amdgcn_alignbit(a, nx[t], 32u - sh) : a);
      }
      prev = nx[3];
    }
    for (; k < nd; ++k) {
      const uint32_t nx = bits.word(i0 + k + 1);
      d[k] = __builtin_bswap32(sh ? __builtin_amdgcn_alignbit(prev, nx, 32u - sh) : prev);
      prev = nx;
    }
  }
  const uint32_t m = head + 4u * nd;
  if (m < n) {
    const uint32_t v = bits.at32(x + 8ull * m);
    for (uint32_t t = 0; m + t < n; ++t) dst[m + t] = static_cast<uint8_t>(v >> (24u - 8u * t));
  }
}

// LDS bytes src[0, n) to dst[0, n) (any alignments, no overlap): single bytes
// up to dst's first 4-byte boundary and after its last, whole dwords between
// them, each from the two aligned source dwords that hold its bytes (reads
// reach at most 3 bytes past src + n).
__device__ __forceinline__ void lds_copy_bytes(const uint8_t* src, uint8_t* dst, uint32_t n) {
  const uint32_t head = min((4u - (static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst)) & 3u)) & 3u, n);
  for (uint32_t t = 0; t < head; ++t) dst[t] = src[t];
  const uint32_t nd = (n - head) >> 2;
  if (nd) {
    const uint8_t* s = src + head;
    const uint32_t so = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(s)) & 3u;
    const uint32_t* sw = reinterpret_cast<const uint32_t*>(s - so);
    uint32_t* d = reinterpret_cast<uint32_t*>(dst + head);
    uint32_t lo = sw[0];
    for (uint32_t k = 0; k < nd; ++k) {
      const uint32_t hi = sw[k + 1];
      d[k] = so ? __builtin_amdgcn_alignbyte(hi, lo, so) : lo;  // (little-endian bytes s[4k ..])
      lo = hi;
    }
  }
  for (uint32_t t = head + 4u * nd; t < n; ++t) dst[t] = src[t];
}

// block heads' inherited bytes, one thread each: key bytes [0, ceil(r_i / 8)),
// the last of them complete (it also holds the literal's first bits).  The
// literal bytes after them are the records kernel's.
__device__ __forceinline__ uint32_t fi_head_bytes(const FiLayout& L, uint32_t i) {
  return min((L.r[i] + 7u) >> 3, L.kbytes[i]);
}

// Key bytes [0, nbytes) of record i down its whole owner chain (the same
// fragments as fi_key with no head), written as they complete from the top.
// A head's chain is long (about a dozen owners at 8M+8M, each covering a few
// bits) and every owner's fields are a cold load, so each step issues the
// current fragment's payload reads and the next owner's r, literal position
// and pse together: one memory round trip per owner instead of three.
template <class Bits>
__device__ __forceinline__ void fi_head_prefix(const Bits& bits, const FiLayout& L, uint32_t i,
                                               uint8_t* __restrict__ key, uint32_t nbytes,
                                               uint64_t* __restrict__ err) {
  if (nbytes == 0) return;
  uint32_t hi = 8u * nbytes;  // key bits [hi, 8 nbytes) are done (pending byte aside)
  uint32_t lo = min(L.r[i], hi);
  uint64_t base = L.lit[i] - L.r[i];  // key bit q of the current owner is payload bit base + q
  uint32_t np = L.pse[i];
  uint32_t pv = 0;  // key byte hi >> 3 as far as it is filled (when hi is not byte aligned)
  while (true) {
    // this fragment's partial bytes: the top one (completing the pending
    // byte) and the bottom one; whole bytes between them are copied below
    const uint32_t top_lo = max(lo, hi & ~7u);
    const bool has_top = (hi & 7u) && top_lo < hi;
    const uint32_t t_hi = has_top ? top_lo : hi;          // byte aligned, or lo
    const uint32_t w_lo = min((lo + 7u) & ~7u, t_hi);     // whole bytes [w_lo, t_hi)
    const bool has_bot = lo < w_lo;                        // bits [lo, w_lo) of byte lo >> 3
    const uint32_t vt = has_top ? bits.at32(base + top_lo) : 0u;
    const uint32_t vb = has_bot ? bits.at32(base + lo) : 0u;
    // the next owner, loaded alongside
    const bool more = lo > 0;
    uint32_t nr = 0, nnp = kFiInf;
    uint64_t nlit = 0;
    if (more && np != kFiInf) {
      nr = L.r[np];
      nlit = L.lit[np];
      nnp = L.pse[np];
    }
    if (has_top) {  // key bits [top_lo, hi) into the pending byte
      const uint32_t n = hi - top_lo;
      pv |= (vt >> (32u - n)) << (8u - (hi & 7u));
      if (top_lo == (hi & ~7u)) key[hi >> 3] = static_cast<uint8_t>(pv), pv = 0;
    }
    if (w_lo < t_hi) fi_copy_bytes(bits, base + w_lo, key + (w_lo >> 3), (t_hi - w_lo) >> 3);
    if (has_bot) {  // key bits [lo, w_lo): the low end of byte lo >> 3, pending
      const uint32_t n = w_lo - lo;
      pv = vb >> (32u - n);  // (w_lo is the byte's end)
    }
    if (!more) return;  // (lo = 0: nothing is pending)
    if (np == kFiInf || nr >= lo) {  // no earlier owner for the bits below
      atomicOr(reinterpret_cast<unsigned long long*>(err), static_cast<unsigned long long>(kFiErrPrefix));
      return;
    }
    hi = lo;
    lo = nr;
    base = nlit - nr;
    np = nnp;
  }
}

__global__ __launch_bounds__(kFiBlock) void k_fi_heads(FiBits bits, FiLayout L, uint8_t* __restrict__ keys,
                                                       uint64_t key_cap, uint64_t val_cap,
                                                       uint64_t* __restrict__ err) {
  const uint32_t k = blockIdx.x * kFiBlock + threadIdx.x;
  if (k >= L.nb) return;
  const uint32_t i = k * kFiRecs;
  if (!fi_record_ok(L, i, key_cap, val_cap)) return;  // (flagged by k_fi_records)
  fi_head_prefix(bits, L, i, keys + L.koff[i], fi_head_bytes(L, i), err);
}

// Key j's inherited bits [0, r_j) in the LDS window, from the keys of the
// earlier records of its block: once every literal (and each head's whole
// key) is in the window, walking t = j-1, j-2, ... down to the block head,
// key j's bits [r_t, hi) are key t's own literal bits whenever r_t < hi (hi:
// the bits still to fill, the smallest r met so far; every record between
// them inherited at least hi bits), and the head's key gives the rest.  The
// bytes are composed from the top down: whole bytes are copied, a byte split
// between two sources is assembled in a register.  r[] and kp[] hold the
// block's retained lengths and window offsets, indexed by thread; key j's
// own literal bits of its byte r_j / 8 are already there.  Reads of another
// key's partial byte keep only its literal bits, which its own thread does
// not change.
__device__ __forceinline__ void fi_prefix_lds(uint8_t* kwin, const uint32_t* r, const uint32_t* kp, uint32_t j,
                                              uint32_t head) {
  uint32_t hi = r[j];
  if (hi == 0) return;
  uint8_t* key = kwin + kp[j];
  uint32_t acc = (hi & 7u) ? key[hi >> 3] : 0u;  // the byte being assembled, (hi - 1) / 8
  for (uint32_t t = j - 1;; --t) {
    const bool at_head = t == head;
    const uint32_t lo = at_head ? 0u : r[t];
    if (lo < hi) {
      const uint8_t* src = kwin + kp[t];
      while (hi > lo) {
        if ((hi & 7u) == 0 && hi - lo >= 8) {  // whole bytes [ceil(lo / 8), hi / 8); acc is empty
          const uint32_t b0 = (lo + 7u) >> 3, b1 = hi >> 3;
          lds_copy_bytes(src + b0, key + b0, b1 - b0);
          hi = 8u * b0;
          continue;
        }
        const uint32_t b = (hi - 1u) >> 3, blo = max(lo, 8u * b);
        acc |= src[b] & (0xFFu >> (blo - 8u * b)) & (0xFFu << (8u * b + 8u - hi));
        hi = blo;
        if (blo == 8u * b) {
          key[b] = static_cast<uint8_t>(acc);
          acc = 0;
        }
      }
      if (hi == 0) return;
    }
    if (at_head) return;  // (only a chain that failed the prefix check ends here)
  }
}

// every record: offsets, tombstone flag, value bytes, and the key bytes not
// written before (all of a record's that is not a block head; a head's
// literal).  A workgroup takes rpb consecutive records
// (one a thread; rpb a multiple of 15, so whole blocks), whose key bytes and
// value bytes are two contiguous ranges.  When both fit the LDS window (each
// from the 16-byte boundary below its start), the records are written there
// and the workgroup copies the two ranges out with 16-byte stores, single
// bytes only in the groups it shares with its neighbours.  In the window a
// block head's inherited bytes are copied from the arena (the kernel before
// wrote them) and its literal from the payload; every other record writes its
// literal, and after one barrier takes its first r_i bits from the literals of
// the earlier records of its block and the head's key (fi_prefix_lds), all
// records at once.  (Copying each record's prefix from its predecessor's
// finished key took fourteen barrier rounds, each with one fifteenth of the
// threads busy.)  A workgroup whose ranges do not fit
// writes each record to the arenas directly: the heads' literals first, then,
// after a barrier, every other key by the owner chain, which may read a
// head's literal bytes.
constexpr uint32_t kFiWin = 24576;

// [b0, b1) of an arena from its window copy starting at base = b0 & ~15
__device__ __forceinline__ void fi_copy_out(uint8_t* __restrict__ arena, const uint8_t* __restrict__ w,
                                            uint64_t base, uint64_t b0, uint64_t b1) {
  const uint32_t groups = static_cast<uint32_t>((b1 - base + 15) >> 4);
  for (uint32_t g = threadIdx.x; g < groups; g += kFiBlock) {
    const uint64_t a = base + 16ull * g;
    if (a >= b0 && a + 16 <= b1) {
      // (non-temporal: 1% faster for the records kernel; the byte-profile
      // emitter's copy-out was slower so)
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(w + 16 * g), reinterpret_cast<u32x4*>(arena + a));
    } else {
      for (uint32_t t = 0; t < 16; ++t)
        if (a + t >= b0 && a + t < b1) arena[a + t] = w[16 * g + t];
    }
  }
}

__global__ __launch_bounds__(kFiBlock) void k_fi_records(FiBits bits, FiLayout L, uint32_t rpb,
                                                         uint8_t* __restrict__ keys, uint64_t key_cap,
                                                         uint32_t* __restrict__ key_off, uint8_t* __restrict__ vals,
                                                         uint64_t val_cap, uint32_t* __restrict__ val_off,
                                                         uint8_t* __restrict__ tomb, uint64_t* __restrict__ err) {
  __shared__ __align__(16) uint8_t win[kFiWin + 16];  // (+16: reads past a copied key's end)
  __shared__ uint32_t rr[kFiBlock], kp[kFiBlock];     // retained bits and window offset of each record
  if (L.S == 0) {  // (nothing was parsed or scanned)
    if (blockIdx.x == 0 && threadIdx.x == 0) key_off[0] = val_off[0] = 0;
    return;
  }
  const uint32_t r0 = blockIdx.x * rpb, r1 = min(r0 + rpb, L.S);

  const uint64_t kb0 = L.koff[r0], kb1 = L.koff[r1], vb0 = L.voff[r0], vb1 = L.voff[r1];
  const uint64_t kbase = kb0 & ~static_cast<uint64_t>(15), vbase = vb0 & ~static_cast<uint64_t>(15);
  const uint64_t kspan = (kb1 - kbase + 15) & ~static_cast<uint64_t>(15);
  const uint64_t vspan = (vb1 - vbase + 15) & ~static_cast<uint64_t>(15);
  const bool staged = kb0 <= kb1 && vb0 <= vb1 && kb1 <= key_cap && vb1 <= val_cap &&
                      kspan + vspan <= kFiWin;  // (uniform over the workgroup)
  uint8_t* kwin = win;
  uint8_t* vwin = win + (staged ? kspan : 0);
  const uint32_t i = r0 + threadIdx.x;
  bool ok = false;     // a staged record that takes its inherited prefix from the window
  bool chain = false;  // an unstaged record that takes its key by the owner chain
  if (threadIdx.x < rpb && i < r1) {
    const uint64_t ko = L.koff[i], vo = L.voff[i];
    key_off[i] = static_cast<uint32_t>(ko);
    val_off[i] = static_cast<uint32_t>(vo);
    tomb[i] = L.tflag[i];
    const uint32_t kb = L.kbytes[i], vb = L.vbytes[i];
    const uint32_t head = i - i % kFiRecs;
    // the value's first byte: after the literal (8 kb - r_i bits) and the
    // value header (the presence bit and, for a present value, EG0(length))
    const uint64_t vbit = L.lit[i] + (8ull * kb - L.r[i]) + (L.tflag[i] ? 1u : 1u + eg0_len(vb));
    if (!fi_record_ok(L, i, key_cap, val_cap)) {
      const bool prefix = i > 0 && L.r[i] > 8u * L.kbytes[i - 1];
      atomicOr(reinterpret_cast<unsigned long long*>(err),
               static_cast<unsigned long long>(prefix ? kFiErrPrefix : kFiErrCap));
    } else if (staged) {
      uint8_t* key = kwin + (ko - kbase);
      rr[threadIdx.x] = L.r[i];
      kp[threadIdx.x] = static_cast<uint32_t>(ko - kbase);
      if (i != head) {
        // the literal: key bits [r_i, 8 kb); a byte it shares with the
        // inherited prefix gets its low bits here, its high bits afterwards
        const uint32_t l = L.r[i], b = l >> 3, part = l & 7u;
        if (part && b < kb) {
          key[b] = static_cast<uint8_t>(bits.at32(L.lit[i]) >> (24u + part));
          fi_copy_to_lds(bits, L.lit[i] + (8u - part), key + b + 1, kb - b - 1);
        } else if (b < kb) {
          fi_copy_to_lds(bits, L.lit[i], key + b, kb - b);
        }
        ok = true;
      } else {
        const uint32_t own = fi_head_bytes(L, i);
        for (uint32_t t = 0; t < own; ++t) key[t] = keys[ko + t];
        if (own < kb) fi_copy_to_lds(bits, L.lit[i] + (8ull * own - L.r[i]), key + own, kb - own);
      }
      fi_copy_to_lds(bits, vbit, vwin + (vo - vbase), vb);
    } else {
      if (i == head) {
        const uint32_t own = fi_head_bytes(L, i);
        if (own < kb) fi_copy_bytes(bits, L.lit[i] + (8ull * own - L.r[i]), keys + ko + own, kb - own);
      } else {
        chain = true;
      }
      fi_copy_bytes(bits, vbit, vals + vo, vb);
    }
  }
  if (r1 == L.S && threadIdx.x == 0) {
    key_off[L.S] = static_cast<uint32_t>(L.koff[L.S]);
    val_off[L.S] = static_cast<uint32_t>(L.voff[L.S]);
  }
  if (!staged) {  // (uniform over the workgroup)
    __syncthreads();  // the heads' literals are in the arena
    if (chain) fi_key(bits, L, i, i - i % kFiRecs, keys + L.koff[i - i % kFiRecs], keys + L.koff[i], L.kbytes[i], err);
    return;
  }
  __syncthreads();  // every literal and every head's key is in the window
  if (ok) fi_prefix_lds(kwin, rr, kp, threadIdx.x, threadIdx.x - threadIdx.x % kFiRecs);  // (r0: a multiple of 15)
  __syncthreads();
  fi_copy_out(keys, kwin, kbase, kb0, kb1);
  fi_copy_out(vals, vwin, vbase, vb0, vb1);
}

// ---- the prefix cache filled from the literal owners ----
//
// Everett, "GPU construction experiment", the prefix-cache and literal-owner
// paragraphs: the merge caches eight key bytes per record, and bit p of key
// i is the literal bit of its owner j = max{t <= i : r_t <= p}.  For the
// first 64 bits this owner rule is a running composition: record i keeps the
// top min(r_i, 64) bits of record i-1's first 64 bits (every record from the
// owner of such a bit up to i inherited it) and writes its own literal bits
// [r_i, min(64, 8 k_i)) below them, zero past the key's end.  A step
// "keep the top m bits of x, then OR v" composes associatively
// ((m1, v1) then (m2, v2) = (min(m1, m2), (v1 & top(m2)) | v2)), so every
// record's 64 bits come from one scan over the records instead of a walk down
// each record's owner chain.

struct FpStep {
  uint32_t m;  // top bits kept
  uint64_t v;  // bits ORed after
};

__device__ __forceinline__ uint64_t fp_top(uint32_t m) {
  return m >= 64u ? ~0ull : (m == 0 ? 0ull : ~0ull << (64u - m));
}

// a, then b
__device__ __forceinline__ FpStep fp_then(FpStep a, FpStep b) {
  return FpStep{min(a.m, b.m), (a.v & fp_top(b.m)) | b.v};
}

__device__ __forceinline__ FpStep fp_record(const FiBits& bits, const FiLayout& L, uint32_t i) {
  const uint32_t r = L.r[i];
  const uint32_t e = min(64u, 8u * L.kbytes[i]);  // the key's bits inside the cache
  if (r >= e) return FpStep{min(r, 64u), 0ull};
  const uint64_t lit = L.lit[i];
  const uint64_t w = (static_cast<uint64_t>(bits.at32(lit)) << 32) | bits.at32(lit + 32);
  return FpStep{r, (w >> r) & fp_top(e) & ~fp_top(r)};  // literal bit k at key bit r + k
}

__device__ __forceinline__ FpStep fp_shfl_up(FpStep a, uint32_t d) {
  return FpStep{__shfl_up(a.m, d), (static_cast<uint64_t>(__shfl_up(static_cast<uint32_t>(a.v >> 32), d)) << 32) |
                                       __shfl_up(static_cast<uint32_t>(a.v), d)};
}

// Exclusive ordered scan of one step per thread over the workgroup (kThreads
// a multiple of kWave); `tot` receives the composition of all of them.
template <int kThreads>
__device__ __forceinline__ FpStep fp_block_exclusive(FpStep x, FpStep* sh, FpStep& tot) {
  constexpr int kW = kThreads / kWave;
  const uint32_t lane = __lane_id(), wave = threadIdx.x / kWave;
  FpStep inc = x;
#pragma unroll
  for (uint32_t d = 1; d < kWave; d <<= 1) {
    const FpStep o = fp_shfl_up(inc, d);
    if (lane >= d) inc = fp_then(o, inc);
  }
  FpStep exc = fp_shfl_up(inc, 1);
  if (lane == 0) exc = FpStep{64u, 0ull};
  if (lane == kWave - 1) sh[wave] = inc;
  __syncthreads();
  FpStep before{64u, 0ull}, all{64u, 0ull};  // the waves before this one; all waves
  for (int w = 0; w < kW; ++w) {
    if (static_cast<uint32_t>(w) < wave) before = fp_then(before, sh[w]);
    all = fp_then(all, sh[w]);
  }
  tot = all;
  __syncthreads();
  return fp_then(before, exc);
}

// A tile is kFpPer rows of kFpBlock consecutive records, one a thread, so
// that the field loads, the literal reads and the stores of a row are
// consecutive; the rows are composed in order.
__device__ __forceinline__ FpStep fp_row_record(const FiBits& bits, const FiLayout& L, uint32_t tile, uint32_t u) {
  const uint32_t i = tile * kFpTile + u * kFpBlock + threadIdx.x;
  return i < L.S ? fp_record(bits, L, i) : FpStep{64u, 0ull};
}

__global__ __launch_bounds__(kFpBlock) void k_fp_reduce(FiBits bits, FiLayout L) {
  __shared__ FpStep sh[kFpBlock / kWave];
  FpStep agg{64u, 0ull};
  for (uint32_t u = 0; u < kFpPer && blockIdx.x * kFpTile + u * kFpBlock < L.S; ++u) {
    FpStep tot;
    (void)fp_block_exclusive<kFpBlock>(fp_row_record(bits, L, blockIdx.x, u), sh, tot);
    agg = fp_then(agg, tot);
  }
  if (threadIdx.x == 0) {
    L.fp_agg[2 * blockIdx.x] = agg.m;
    L.fp_agg[2 * blockIdx.x + 1] = agg.v;
  }
}

// the first 64 key bits of the record before each tile (0 before the first)
__global__ __launch_bounds__(kFpTilesBlock) void k_fp_tiles(FiLayout L, uint32_t ntiles) {
  __shared__ FpStep sh[kFpTilesBlock / kWave];
  const uint32_t t0 = threadIdx.x * kFpTilesPer;
  FpStep a{64u, 0ull};
  for (uint32_t q = 0; q < kFpTilesPer && t0 + q < ntiles; ++q)
    a = fp_then(a, FpStep{static_cast<uint32_t>(L.fp_agg[2 * (t0 + q)]), L.fp_agg[2 * (t0 + q) + 1]});
  FpStep tot;
  FpStep before = fp_block_exclusive<kFpTilesBlock>(a, sh, tot);
  for (uint32_t q = 0; q < kFpTilesPer && t0 + q < ntiles; ++q) {
    L.fp_x[t0 + q] = before.v;  // (applied to the all-zero start)
    before = fp_then(before, FpStep{static_cast<uint32_t>(L.fp_agg[2 * (t0 + q)]), L.fp_agg[2 * (t0 + q) + 1]});
  }
}

__global__ __launch_bounds__(kFpBlock) void k_fp_apply(FiBits bits, FiLayout L, uint64_t* __restrict__ pfx) {
  __shared__ FpStep sh[kFpBlock / kWave];
  uint64_t x = L.fp_x[blockIdx.x];  // the first 64 bits of the record before the row
  for (uint32_t u = 0; u < kFpPer && blockIdx.x * kFpTile + u * kFpBlock < L.S; ++u) {
    const uint32_t i = blockIdx.x * kFpTile + u * kFpBlock + threadIdx.x;
    const FpStep st = fp_row_record(bits, L, blockIdx.x, u);
    FpStep tot;
    const FpStep inc = fp_then(fp_block_exclusive<kFpBlock>(st, sh, tot), st);
    if (i < L.S) pfx[i] = (x & fp_top(inc.m)) | inc.v;
    x = (x & fp_top(tot.m)) | tot.v;
  }
}

// totals and the size checks, after the scans
__global__ void k_fi_totals(FiLayout L, uint64_t* __restrict__ totals) {
  const uint64_t kt = L.koff[L.S], vt = L.voff[L.S];
  totals[0] = kt;
  totals[1] = vt;
  if (kt > 0xFFFFFFFFull || vt > 0xFFFFFFFFull) totals[2] |= kFiErrTotal;
}

__global__ void k_fi_clear(uint64_t* totals) {
  totals[0] = totals[1] = totals[2] = 0;
}

// ---- owner-search comparison of two compressed inputs' keys ----
//
// Everett, "GPU construction experiment", the literal-owner paragraph: a merge
// of compressed inputs may compare keys without expanding them, taking each
// key bit from its owner's literal; the page leaves the cost of that against
// materializing the keys to measurement.  Bit p of key i belongs to
// j = max{t <= i : r_t <= p}: the record's own literal holds bits [r_i, k_i),
// pse(i) (the last earlier record with a smaller r) holds [r_pse(i), r_i),
// and so on down the pse chain to a record with r = 0 (record 0 has r = 0,
// so the chain always ends).

// Key bits [x0, x0 + 256) of record i as eight most-significant-first words,
// zero at and past key bit kend, every bit taken from its owner's literal.
// False when the chain breaks, which a parse without error bits excludes.
template <class Bits>
__device__ __forceinline__ bool fi_window(const Bits& bits, const FiLayout& L, uint32_t i, uint32_t kend,
                                          uint32_t x0, uint32_t (&w)[8]) {
#pragma unroll
  for (int t = 0; t < 8; ++t) w[t] = 0;
  const uint32_t x1 = min(kend, x0 + 256u);
  uint32_t j = i, lo = L.r[i], hi = kend;  // record j's literal holds key bits [lo, hi)
  uint64_t base = L.lit[i] - lo;           // key bit q of that fragment: payload bit base + q
  while (true) {
    const uint32_t a = max(lo, x0), b = min(hi, x1);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t w0 = x0 + 32u * t;  // word t: key bits [w0, w0 + 32)
      const uint32_t qa = max(a, w0), qb = min(b, w0 + 32u);
      if (qa < qb) {
        const uint32_t n = qb - qa;  // 1 .. 32 bits, placed qa - w0 bits into the word
        const uint32_t v = bits.at32(base + qa);
        w[t] |= (n == 32u ? v : (v >> (32u - n)) << (32u - n)) >> (qa - w0);
      }
    }
    if (lo <= x0) return true;
    const uint32_t nj = L.pse[j];
    if (nj >= j) return false;  // (no earlier owner)
    const uint32_t nlo = L.r[nj];
    if (nlo >= lo) return false;
    hi = lo;
    j = nj;
    lo = nlo;
    base = L.lit[nj] - nlo;
  }
}

// Pair q: key ia[q] of input A against key jb[q] of input B, from byte
// `from` on (the bytes before it are taken as shared), in windows of 256
// bits; lcp[q] = their bit LCP, cmp[q] = the sign of A's key minus B's in
// unsigned bytewise order with a proper prefix first.  An index past its
// input, or a broken owner chain, gives lcp = kFiInf and cmp = 0.
constexpr int kFcBlock = 256;

__global__ __launch_bounds__(kFcBlock) void k_fi_compare(FiBits ba, FiLayout La, FiBits bb, FiLayout Lb, uint32_t n,
                                                         const uint32_t* __restrict__ ia,
                                                         const uint32_t* __restrict__ jb, uint32_t from,
                                                         uint32_t* __restrict__ lcp, int32_t* __restrict__ cmp) {
  const uint32_t q = blockIdx.x * kFcBlock + threadIdx.x;
  if (q >= n) return;
  const uint32_t i = ia[q], j = jb[q];
  uint32_t l = kFiInf;
  int32_t c = 0;
  if (i < La.S && j < Lb.S) {
    const uint32_t ka = 8u * La.kbytes[i], kb = 8u * Lb.kbytes[j], m = min(ka, kb);
    const uint32_t start = from < m / 8u ? 8u * from : m;
    bool done = false, broken = false;  // done: the first differing bit is known
    for (uint32_t x0 = start; x0 < m && !done; x0 += 256u) {
      uint32_t wa[8], wb[8];
      if (!fi_window(ba, La, i, ka, x0, wa) || !fi_window(bb, Lb, j, kb, x0, wb)) {
        broken = true;
        break;
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t d = wa[t] ^ wb[t];
        if (!done && d) {
          done = true;
          const uint32_t p = x0 + 32u * t + static_cast<uint32_t>(__builtin_clz(d));
          if (p < m) {  // (a difference at or past the shorter key's end is none)
            l = p;
            c = wa[t] > wb[t] ? 1 : -1;
          }
        }
      }
    }
    if (broken) {
      l = kFiInf;
      c = 0;
    } else if (l == kFiInf) {  // equal up to the shorter key's end
      l = m;
      c = ka < kb ? -1 : (ka > kb ? 1 : 0);
    }
  }
  if (lcp) lcp[q] = l;
  if (cmp) cmp[q] = c;
}

}  // namespace em

using namespace em;

extern "C" size_t em_fcin_workspace_bytes(uint32_t S) { return align_up(fi_layout(nullptr, S).used, 256); }

extern "C" int em_fcin_parse(const uint32_t* payload, uint64_t payload_words, uint64_t T, uint32_t S,
                             const uint64_t* off, const em_ef_info_t* nav_info, const uint64_t* nav_lows,
                             const uint64_t* nav_highs, const uint64_t* nav_samples,
                             const uint64_t* nav_exceptions, uint64_t* d_totals, void* ws, size_t ws_bytes,
                             void* stream) {
  if (!d_totals || !ws || (reinterpret_cast<uintptr_t>(ws) & 255)) return EM_EINVAL;
  if (S >= EM_MAX_RECORDS) return EM_ERANGE;
  if ((S == 0) != (T == 0)) return EM_EINVAL;
  if (S && !payload) return EM_EINVAL;
  if (payload_words < (T + 31) / 32) return EM_EINVAL;
  if (S && !off && !(nav_info && nav_highs && nav_samples && nav_lows && nav_exceptions)) return EM_EINVAL;
  if (ws_bytes < em_fcin_workspace_bytes(S)) return EM_ENOSPC;
  hipStream_t st = as_stream(stream);
  const FiLayout L = fi_layout(ws, S);
  hipLaunchKernelGGL(k_fi_clear, dim3(1), dim3(1), 0, st, d_totals);
  if (S == 0) return check_launch();
  const FiBits bits{payload, payload_words};
  if (off)
    hipLaunchKernelGGL(k_fi_starts_off, dim3(fi_blocks(L.nb)), dim3(kFiBlock), 0, st, off, L.nb, L.starts);
  else
    hipLaunchKernelGGL(k_fi_starts_ef, dim3(fi_blocks(L.nb)), dim3(kFiBlock), 0, st, nav_info, nav_lows, nav_highs,
                       nav_samples, nav_exceptions, L.nb, L.starts);
  // blocks per parse workgroup: the mean block filling three quarters of the staged span
  const uint64_t mean_block = std::max<uint64_t>(1, (T / 8 + L.nb - 1) / L.nb);
  const uint32_t G = static_cast<uint32_t>(
      std::max<uint64_t>(1, std::min<uint64_t>(kFiParseWave, (3 * 4 * kFiParseWords / 4) / mean_block)));
  hipLaunchKernelGGL(k_fi_parse, dim3((L.nb + G - 1) / G), dim3(kFiParseWave), 0, st, bits, T, S, L.nb, G, L.starts,
                     L.r, L.kbytes, L.vbytes, L.lit, L.tflag, d_totals + 2);
  int rc = check_launch();
  if (rc) return rc;
  rc = scan_launch<uint64_t>(L.kbytes, S + 1, L.koff, L.scan_ws, L.scan_bytes, st);
  if (rc) return rc;
  rc = scan_launch<uint64_t>(L.vbytes, S + 1, L.voff, L.scan_ws, L.scan_bytes, st);
  if (rc) return rc;
  hipLaunchKernelGGL(k_fi_totals, dim3(1), dim3(1), 0, st, L, d_totals);
  // the minimum tree over the retained lengths
  hipLaunchKernelGGL(k_fi_leaves, dim3(fi_blocks(L.P2)), dim3(kFiBlock), 0, st, L.r, S, L.P2, L.tree);
  for (uint32_t first = L.P2 / 2; first >= 1;) {
    const uint32_t cnt0 = first < static_cast<uint32_t>(kFiBlock) ? first : static_cast<uint32_t>(kFiBlock);
    hipLaunchKernelGGL(k_fi_levels, dim3(first / cnt0), dim3(kFiBlock), 0, st, L.tree, first, cnt0);
    uint32_t lev = 1;  // 1 + log2(cnt0) levels built
    for (uint32_t c = cnt0; c > 1; c >>= 1) ++lev;
    first >>= lev;
  }
  hipLaunchKernelGGL(k_fi_pse, dim3(fi_blocks(S)), dim3(kFiBlock), 0, st, L);
  return check_launch();
}

extern "C" int em_fcin_materialize(const uint32_t* payload, uint64_t payload_words, uint32_t S, uint8_t* keys,
                                   uint64_t key_cap, uint32_t* key_off, uint8_t* vals, uint64_t val_cap,
                                   uint32_t* val_off, uint8_t* tomb, uint64_t* d_totals, void* ws,
                                   size_t ws_bytes, void* stream) {
  if (!d_totals || !ws || (reinterpret_cast<uintptr_t>(ws) & 255)) return EM_EINVAL;
  if (S >= EM_MAX_RECORDS) return EM_ERANGE;
  if (!key_off || !val_off || (S && (!payload || !tomb))) return EM_EINVAL;
  if ((key_cap && !keys) || (val_cap && !vals)) return EM_EINVAL;
  if (ws_bytes < em_fcin_workspace_bytes(S)) return EM_ENOSPC;
  hipStream_t st = as_stream(stream);
  const FiLayout L = fi_layout(ws, S);
  const FiBits bits{payload, payload_words};
  if (S)
    hipLaunchKernelGGL(k_fi_heads, dim3(fi_blocks(L.nb)), dim3(kFiBlock), 0, st, bits, L, keys, key_cap, val_cap,
                       d_totals + 2);
  // records per workgroup: the mean record (from the arena capacities, at
  // least its size) filling two thirds of the window
  const uint64_t mean = S ? (key_cap + val_cap + S - 1) / S : 1;
  uint32_t rpb = static_cast<uint32_t>(
      std::max<uint64_t>(kFiRecs, std::min<uint64_t>(kFiBlock, (2 * kFiWin / 3) / std::max<uint64_t>(mean, 1))));
  rpb -= rpb % kFiRecs;  // whole blocks
  hipLaunchKernelGGL(k_fi_records, dim3(S ? (S + rpb - 1) / rpb : 1), dim3(kFiBlock), 0, st, bits, L, rpb, keys,
                     key_cap, key_off, vals, val_cap, val_off, tomb, d_totals + 2);
  return check_launch();
}

extern "C" int em_fcin_compare(const uint32_t* payload_a, uint64_t words_a, uint32_t S_a, const void* ws_a,
                               size_t ws_a_bytes, const uint32_t* payload_b, uint64_t words_b, uint32_t S_b,
                               const void* ws_b, size_t ws_b_bytes, uint32_t n, const uint32_t* ia,
                               const uint32_t* jb, uint32_t from_byte, uint32_t* lcp_bits, int32_t* cmp,
                               void* stream) {
  if (!ws_a || !ws_b || (reinterpret_cast<uintptr_t>(ws_a) & 255) || (reinterpret_cast<uintptr_t>(ws_b) & 255))
    return EM_EINVAL;
  if (S_a >= EM_MAX_RECORDS || S_b >= EM_MAX_RECORDS) return EM_ERANGE;
  if ((S_a && !payload_a) || (S_b && !payload_b)) return EM_EINVAL;
  if (n && (!ia || !jb || (!lcp_bits && !cmp))) return EM_EINVAL;
  if (ws_a_bytes < em_fcin_workspace_bytes(S_a) || ws_b_bytes < em_fcin_workspace_bytes(S_b)) return EM_ENOSPC;
  if (n == 0) return EM_OK;
  const FiLayout La = fi_layout(const_cast<void*>(ws_a), S_a), Lb = fi_layout(const_cast<void*>(ws_b), S_b);
  const FiBits ba{payload_a, words_a}, bb{payload_b, words_b};
  hipLaunchKernelGGL(k_fi_compare, dim3((n + kFcBlock - 1) / kFcBlock), dim3(kFcBlock), 0, as_stream(stream), ba,
                     La, bb, Lb, n, ia, jb, from_byte, lcp_bits, cmp);
  return check_launch();
}

extern "C" int em_fcin_prefix8(const uint32_t* payload, uint64_t payload_words, uint32_t S, uint64_t* pfx,
                               void* ws, size_t ws_bytes, void* stream) {
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255)) return EM_EINVAL;
  if (S >= EM_MAX_RECORDS) return EM_ERANGE;
  if (S && (!payload || !pfx)) return EM_EINVAL;
  if (ws_bytes < em_fcin_workspace_bytes(S)) return EM_ENOSPC;
  if (S == 0) return EM_OK;
  hipStream_t st = as_stream(stream);
  const FiLayout L = fi_layout(ws, S);
  const FiBits bits{payload, payload_words};
  const uint32_t ntiles = (S + kFpTile - 1) / kFpTile;  // <= kFpTilesBlock * kFpTilesPer
  hipLaunchKernelGGL(k_fp_reduce, dim3(ntiles), dim3(kFpBlock), 0, st, bits, L);
  hipLaunchKernelGGL(k_fp_tiles, dim3(1), dim3(kFpTilesBlock), 0, st, L, ntiles);
  hipLaunchKernelGGL(k_fp_apply, dim3(ntiles), dim3(kFpBlock), 0, st, bits, L, pfx);
  return check_launch();
}
