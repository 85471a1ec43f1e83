// The whole path in one pass: per partition of merged outputs, one
// workgroup finds the partition's co-ranks, merges with keep-newer, computes
// exact bit LCPs and record lengths, takes its survivor base and its bit base
// from two decoupled look-backs, and writes its own payload words.  A second,
// small kernel writes the words that partition boundaries cut.
//
// Everett, "GPU construction experiment": merge by diagonal partitions with
// ties to the older side; keep the last reference of each equal-key run; the
// compacted order fixes predecessors and ordinals (the global survivor index
// fixes the phase of the c_i rule); exact lengths are scanned into bit
// offsets by one global scan with no per-chunk reset (here: a scan inside
// each partition plus a look-back over the partitions' bit totals); every
// 32-bit output word has one writer, which stores it once; the prefix cache
// holds the eight key bytes after the common prefix the partition's keys
// share.
//
// One 256-thread workgroup per partition of `items` (<= 1024) outputs:
//  1. co-ranks of the partition's two diagonals, searched inside the coarse
//     partition that coarse_splits gives;
//  2. the partition's key offsets (with the two A keys and the B key before
//     it and the B key after it), value offsets and tombstone flags go to LDS
//     with coalesced loads: nothing per survivor is read from HBM later;
//  3. the prefix cache: each key's 8 bytes at offset cp, where cp is the
//     number of leading bytes all cached keys share (0 unless the first and
//     last keys of both sides agree in their first 8 bytes, then measured
//     exactly and the cache reloaded at cp);
//  4. merge and keep-newer (merge_slice), compaction; the survivor count goes
//     to the first look-back at once;
//  5. exact bit LCPs from the cache (key bytes beyond it read only when the
//     cached bytes tie), value lengths and flags from LDS; the survivor base
//     from the first look-back; controls, lengths, a block scan into
//     partition-local bit offsets, the partition's bit total published to
//     the second look-back;
//  6. emission in chunks of up to 256 survivors (one per thread): the
//     chunk's value bytes are staged in LDS by LDS-DMA (the bit base is
//     resolved while they are in flight); each thread ORs its record's
//     fields into an LDS window of output words (key suffixes read in place
//     with 16-byte loads: the merge has just brought those lines into the
//     cache); the complete words go out with 16-byte non-temporal stores; the
//     word the chunk shares with the next one is carried over in LDS, and the
//     partition's first and last partial words go to edge_lo / edge_hi.
#include "em_tile.h"

namespace em {

constexpr int kOpBlock = 256;
constexpr int kOpWaves = kOpBlock / kWave;
constexpr uint32_t kOpMaxItems = 4 * kOpBlock;  // outputs per partition, at most
// Five workgroups share a compute unit (under 32 KB of LDS each at 512
// outputs).  A chunk of survivors is sized per partition so that its bits
// fill about 90% of the window and its source spans about 85% of the stage;
// on the headline workload that is about 120 survivors (545 bits and 68
// source bytes each, the replaced records' bytes included).
constexpr uint32_t kOpWin = 2304;     // window words (9 KB)
constexpr uint32_t kOpStage = 13312;  // staged key and value bytes
constexpr uint32_t kOpMaxChunk = kOpBlock;  // survivors per chunk, at most

template <int IPT>
struct OpShared {
  static constexpr int kTile = kOpBlock * IPT;
  uint32_t a_off[kTile + 4];   // key offsets of A records aK0 .. i1 (aK0 = i0 - 2 when it exists)
  uint32_t b_off[kTile + 4];   // key offsets of B records bK0 .. j1 (+ the next B)
  uint32_t a_voff[kTile + 1];  // value offsets of A records i0 .. i1
  uint32_t b_voff[kTile + 1];  // value offsets of B records j0 .. j1
  uint8_t a_tomb[kTile];
  uint8_t b_tomb[kTile];
  union alignas(16) {
    struct {
      uint64_t a_pfx[kTile + 4];  // 8 bytes at offset cp of A keys aK0 .., big-endian, zero padded
      uint64_t b_pfx[kTile + 4];  // the same for B keys bK0 ..
    } m;
    struct {
      uint64_t spfx[kTile];  // survivors' cached bytes, compacted
      uint32_t surv[kTile];  // survivors' references, compacted
      uint32_t ords[kTile];  // per input record: survivor ordinal in the partition, or EM_NONE
    } c;
    struct {
      uint32_t win[kOpWin];        // output words (big-endian bit order)
      uint4 stage[kOpStage / 16];  // staged key and value spans of the chunk
    } e;
  } u;
  uint64_t scan64[IPT * kOpWaves + 1];
  uint64_t red[3 * kOpWaves];  // look-back reductions
  uint32_t scan32[kOpWaves + 1];
  uint32_t notes[kOpBlock];  // the merge's list of pairs to check, kWave words per wave
  uint32_t tile, i0, i1, g0, cp, carry;
  uint32_t span_lo[4], span_hi[4], stage_at[5];  // A keys, B keys, A values, B values
  uint64_t src_at[4];     // global address of each staged span's first byte, less stage_at
  uint64_t base;          // the partition's bit base
  uint64_t clo, chi;      // the chunk's local bit range
};

struct OpOut {
  uint32_t* d_S;
  uint64_t* d_T;
  uint32_t* payload;
  uint64_t* desc_b;     // bit-base look-back
  uint64_t* tile_bits;  // bit total of each partition
  uint32_t* edge_lo;    // each partition's bits in its first word, when that word is shared
  uint32_t* edge_hi;    // each partition's bits in its last word, when that word is shared
  uint32_t* final_refs;  // optional per-record outputs
  uint32_t* ord_A;
  uint32_t* ord_B;
  uint32_t* len_bits;
  uint32_t* lcp_bits;
  uint64_t* off;
};

// ---------------------------------------------------------------------------
// Window writers.  The window holds output words in big-endian bit order and
// starts zeroed; words that also hold bits of another field or record are
// ORed, words inside one copied span are stored.

// n (1..64) bits of v, right-aligned, at window bit p.
__device__ __forceinline__ void wput(uint32_t* win, uint32_t p, uint64_t v, uint32_t n) {
  const uint64_t x = v << (64u - n);
  const uint32_t hi = static_cast<uint32_t>(x >> 32), lo = static_cast<uint32_t>(x);
  const uint32_t s = p & 31u;
  uint32_t* o = win + (p >> 5);
  const uint32_t last = (s + n - 1u) >> 5;  // 0, 1 or 2
  atomicOr(o, hi >> s);
  if (last >= 1) atomicOr(o + 1, __builtin_amdgcn_alignbit(hi, lo, s));
  if (last >= 2) atomicOr(o + 2, __builtin_amdgcn_alignbit(lo, 0u, s));
}

typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));

// n >= 1 source bits [sb, sb + n) of a dword array (stream order: bit p is
// bit 7 - p mod 8 of byte p / 8) at window bit p.  Output word k >= 1 holds
// source bits [P1 + 32 (k-1), +32) with P1 = sb + 32 - f: one funnel shift of
// source dwords D + k - 1 and D + k, D = (P1 - 1) / 32, by (-P1) mod 32.
// Reads reach at most one dword past the one holding the last bit.
template <class Src>
__device__ __forceinline__ void wcopy(uint32_t* win, uint32_t p, Src src, uint32_t sb, uint32_t n) {
  const uint32_t f = p & 31u;
  uint32_t* o = win + (p >> 5);
  const uint32_t r0 = sb & 31u;
  const uint32_t a0 = __builtin_bswap32(src[sb >> 5]), a1 = __builtin_bswap32(src[(sb >> 5) + 1]);
  const uint32_t src32 = r0 ? __builtin_amdgcn_alignbit(a0, a1, 32u - r0) : a0;  // 32 bits from sb
  const uint32_t end = f + n;  // in the first word's coordinates
  uint32_t first = src32 >> f;
  if (end < 32u) first &= ~(0xFFFFFFFFu >> end);
  atomicOr(o, first);
  if (end <= 32u) return;
  const uint32_t K = (end - 1u) >> 5;  // last output word touched (>= 1)
  const uint32_t P1 = sb + 32u - f;
  const uint32_t D = (P1 - 1u) >> 5;
  const uint32_t sh = (0u - P1) & 31u;
  uint32_t cur = __builtin_bswap32(src[D]);
  uint32_t k = 1;
  for (; k + 4u <= K; k += 4) {  // four full words per round (all before K)
    const u32x4a4 q = *reinterpret_cast<const u32x4a4*>(&src[D + k]);
    const uint32_t n1 = __builtin_bswap32(q.x), n2 = __builtin_bswap32(q.y);
    const uint32_t n3 = __builtin_bswap32(q.z), n4 = __builtin_bswap32(q.w);
    o[k] = __builtin_amdgcn_alignbit(cur, n1, sh);
    o[k + 1] = __builtin_amdgcn_alignbit(n1, n2, sh);
    o[k + 2] = __builtin_amdgcn_alignbit(n2, n3, sh);
    o[k + 3] = __builtin_amdgcn_alignbit(n3, n4, sh);
    cur = n4;
  }
  const uint32_t tail = end & 31u;  // valid bits of word K (0: all 32)
  for (; k <= K; ++k) {
    const uint32_t nx = __builtin_bswap32(src[D + k]);
    const uint32_t v = __builtin_amdgcn_alignbit(cur, nx, sh);
    cur = nx;
    if (k < K || tail == 0)
      o[k] = v;
    else
      atomicOr(o + k, v & ~(0xFFFFFFFFu >> tail));
  }
}

// One record's fields: segment ends relative to the record start, the two
// immediates and the source bit positions of its key suffix and value bytes.
struct OpRec {
  uint32_t c, s;  // control and suffix bits k - l
  uint32_t b1, b2, b3, b4, b5;
  uint64_t vh;    // presence bit and EG0(value length) (b4 - b3 bits; 0 for a tombstone)
  uint32_t kbit, vbit;  // source bit positions, relative to the key and value bases
};

// The whole record at window bit p.
__device__ __forceinline__ void append_whole(uint32_t* win, uint32_t p, const OpRec& r, const uint32_t* kbase,
                                             const uint32_t* vbase) {
  if (r.b2 <= 64u) {
    wput(win, p, (static_cast<uint64_t>(r.c + 1u) << (r.b2 - r.b1)) | (static_cast<uint64_t>(r.s) + 1u), r.b2);
  } else {
    wput(win, p, static_cast<uint64_t>(r.c) + 1u, r.b1);
    wput(win, p + r.b1, static_cast<uint64_t>(r.s) + 1u, r.b2 - r.b1);
  }
  if (r.s) wcopy(win, p + r.b2, kbase, r.kbit, r.s);
  if (r.vh) wput(win, p + r.b3, r.vh, r.b4 - r.b3);  // a tombstone's 0 bit is already there
  if (r.b5 > r.b4) wcopy(win, p + r.b4, vbase, r.vbit, r.b5 - r.b4);
}

// The record's bits [from, to) (relative to its start) at window bit p.
__device__ __forceinline__ void append_clipped(uint32_t* win, uint32_t p, const OpRec& r, uint32_t from,
                                               uint32_t to, const uint32_t* kbase, const uint32_t* vbase) {
  auto imm = [&](uint64_t v, uint32_t a, uint32_t b) {  // field occupying [a, b)
    const uint32_t lo = max(a, from), hi = min(b, to);
    if (lo < hi)
      wput(win, p + (lo - from), (v >> (b - hi)) & (hi - lo == 64 ? ~0ull : ((1ull << (hi - lo)) - 1)), hi - lo);
  };
  auto span = [&](const uint32_t* base, uint32_t bp, uint32_t a, uint32_t b) {
    const uint32_t lo = max(a, from), hi = min(b, to);
    if (lo < hi) wcopy(win, p + (lo - from), base, bp + (lo - a), hi - lo);
  };
  imm(static_cast<uint64_t>(r.c) + 1u, 0, r.b1);
  imm(static_cast<uint64_t>(r.s) + 1u, r.b1, r.b2);
  span(kbase, r.kbit, r.b2, r.b3);
  if (r.vh) imm(r.vh, r.b3, r.b4);
  span(vbase, r.vbit, r.b4, r.b5);
}

// Exclusive prefix of the values of the tiles before `tile` by decoupled
// look-back, read by the whole workgroup: thread t reads the descriptor t
// places back, so one round covers kOpBlock predecessors (a tile in the
// middle of the grid has hundreds of predecessors in flight, whose
// descriptors still hold aggregates).  Every thread calls it; `red` is LDS
// scratch of 3 * kOpWaves words.  The caller publishes the inclusive value.
__device__ __forceinline__ uint64_t lookback_block(uint64_t* desc, uint32_t tile, uint64_t* red) {
  if (tile == 0) return 0;
  const uint32_t tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  uint64_t excl = 0;
  int64_t base = static_cast<int64_t>(tile) - 1;
  for (;;) {
    const int64_t idx = base - static_cast<int64_t>(tid);
    const uint64_t v = idx >= 0 ? desc_load(desc + idx) : kDescIncl;
    const uint64_t st = v >> 62;
    const uint64_t incl = __ballot(st == 2), nr = __ballot(st == 0);
    if (lane == 0) {
      red[w] = incl ? w * kWave + static_cast<uint32_t>(__builtin_ctzll(incl)) : kOpBlock;
      red[kOpWaves + w] = nr ? w * kWave + static_cast<uint32_t>(__builtin_ctzll(nr)) : kOpBlock;
    }
    __syncthreads();
    uint32_t F = kOpBlock, R = kOpBlock;  // first inclusive, first not yet published
#pragma unroll
    for (int q = 0; q < kOpWaves; ++q) {
      F = min(F, static_cast<uint32_t>(red[q]));
      R = min(R, static_cast<uint32_t>(red[kOpWaves + q]));
    }
    if (R < kOpBlock && R <= F) {  // (uniform) a value needed is not there yet
      __syncthreads();
      __builtin_amdgcn_s_sleep(1);
      continue;
    }
    uint64_t mine = tid <= F ? (v & kDescValue) : 0;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) mine += __shfl_xor(mine, d, kWave);
    if (lane == 0) red[2 * kOpWaves + w] = mine;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kOpWaves; ++q) excl += red[2 * kOpWaves + q];
    __syncthreads();
    if (F < kOpBlock) break;  // (uniform)
    base -= kOpBlock;
  }
  return excl;
}

template <int IPT>
__global__ __launch_bounds__(kOpBlock) __attribute__((amdgpu_waves_per_eu(4))) void k_onepass(
    em_side_t A, em_side_t B, const uint32_t* __restrict__ csplits, uint32_t coarse, uint32_t items, uint32_t P,
    OpOut out, uint32_t* __restrict__ ticket, uint64_t* __restrict__ desc_s) {
  using Sh = OpShared<IPT>;
  __shared__ Sh sh;
  const uint32_t tid = threadIdx.x;
  const uint32_t N = A.n + B.n;
  if (tid == 0) sh.tile = atomicAdd(ticket, 1u);
  __syncthreads();
  const uint32_t tile = __builtin_amdgcn_readfirstlane(sh.tile);  // (uniform: scalar registers)
  const uint32_t d0 = tile * items;
  const uint32_t d1 = min(d0 + items, N);

  // ---- 1. co-ranks of the partition's two diagonals (two 16-lane groups) ----
  if (tid < 32) {
    const uint32_t Pc = (N + coarse - 1) / coarse;
    const uint32_t d = tid < 16 ? d0 : d1;
    const uint32_t i = fine_corank(A, B, csplits, coarse, Pc, d, tid & 15u, tid & 16u);
    if ((tid & 15u) == 0) (tid < 16 ? sh.i0 : sh.i1) = i;
  }
  __syncthreads();
  uint32_t i0 = __builtin_amdgcn_readfirstlane(sh.i0), i1 = __builtin_amdgcn_readfirstlane(sh.i1);
  // Splits from em_partition on sorted inputs always pass this check; any
  // other splits leave the partition empty rather than index outside it.
  const bool valid = i0 <= d0 && i1 <= d1 && i0 <= i1 && d0 - i0 <= d1 - i1 && i1 <= A.n && d1 - i1 <= B.n;
  if (!valid) {
    i0 = 0;
    i1 = 0;
  }
  const uint32_t j0 = valid ? d0 - i0 : 0, j1 = valid ? d1 - i1 : 0;
  const uint32_t nA_t = i1 - i0, nB_t = j1 - j0;
  const uint32_t len = valid ? d1 - d0 : 0;
  const bool has_next_b = valid && j1 < B.n;
  const uint32_t aK0 = i0 >= 2 ? i0 - 2 : 0, a_first = i0 - aK0;
  const uint32_t bK0 = j0 >= 1 ? j0 - 1 : 0, b_first = j0 - bK0;
  const uint32_t na_off = i1 - aK0 + 1;
  const uint32_t nb_off = j1 + (has_next_b ? 1u : 0u) - bK0 + 1;

  // ---- 2. key offsets, value offsets, tombstone flags (all loads, then all
  // stores; a thread past the end reads a valid entry and drops it, so that
  // no load sits under a condition of its own) ----
  {
    constexpr int kPer = IPT + 1;  // ceil((kTile + 4) / kOpBlock)
    uint32_t ka[kPer], kb[kPer], va[kPer], vb[kPer];
    uint8_t ta[IPT], tb[IPT];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const uint32_t x = tid + u * kOpBlock;
      ka[u] = A.key_off[aK0 + (x < na_off ? x : 0u)];
      kb[u] = B.key_off[bK0 + (x < nb_off ? x : 0u)];
      va[u] = A.val_off[i0 + (x <= nA_t ? x : 0u)];
      vb[u] = B.val_off[j0 + (x <= nB_t ? x : 0u)];
    }
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
      const uint32_t x = tid + u * kOpBlock;
      const bool ha = x < nA_t && A.tomb, hb = x < nB_t && B.tomb;
      // (without a flag to read, the side's first value offset is read instead)
      ta[u] = *(ha ? A.tomb + i0 + x : reinterpret_cast<const uint8_t*>(A.val_off + i0));
      tb[u] = *(hb ? B.tomb + j0 + x : reinterpret_cast<const uint8_t*>(B.val_off + j0));
      if (!ha) ta[u] = 0;
      if (!hb) tb[u] = 0;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const uint32_t x = tid + u * kOpBlock;
      if (x < na_off) sh.a_off[x] = ka[u];
      if (x < nb_off) sh.b_off[x] = kb[u];
      if (x <= nA_t) sh.a_voff[x] = va[u];
      if (x <= nB_t) sh.b_voff[x] = vb[u];
    }
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
      const uint32_t x = tid + u * kOpBlock;
      if (x < nA_t) sh.a_tomb[x] = ta[u];
      if (x < nB_t) sh.b_tomb[x] = tb[u];
    }
  }
  __syncthreads();

  // ---- 3. prefix cache (offset 0, then at the common prefix when it is long) ----
  auto load_cache = [&](uint32_t cp) {
    constexpr int kPer = IPT + 1;
    fill_prefix_caches<kOpBlock, kPer>(PfxSide{sh.a_off, na_off, A.keys, sh.u.m.a_pfx},
                                       PfxSide{sh.b_off, nb_off, B.keys, sh.u.m.b_pfx}, cp);
  };
  load_cache(0);
  __syncthreads();
  const uint32_t cp = cache_offset(sh.a_off, na_off - 1, sh.b_off, nb_off - 1, sh.u.m.a_pfx, sh.u.m.b_pfx, A.keys,
                                   B.keys, &sh.cp);
  if (cp) {  // (uniform) the cached keys share cp >= 8 bytes: cache the 8 after them
    load_cache(cp);
    __syncthreads();
  }

  const uint32_t* ao = sh.a_off + a_first;  // A[i0 + x] is key [ao[x], ao[x+1])
  const uint32_t* bo = sh.b_off + b_first;  // B[j0 + y] is key [bo[y], bo[y+1])
  const uint64_t* apf = sh.u.m.a_pfx + a_first;
  const uint64_t* bpf = sh.u.m.b_pfx + b_first;

  // ---- 4. merge and keep-newer; publish the survivor count ----
  uint32_t refs[IPT];
  const uint32_t k = tid * IPT;
  const uint32_t kept = merge_slice<IPT>(ao, bo, apf, bpf, A.keys, 0u, B.keys, 0u, k, len, nA_t, nB_t, has_next_b,
                                         i0, A.n, j0, refs, sh.notes, cp);
  // cached bytes of this thread's outputs and of the keys before the
  // partition, read before the compaction arrays overwrite the cache
  uint64_t opfx[IPT];
#pragma unroll
  for (int s = 0; s < IPT; ++s) {
    const uint32_t ref = refs[s] & ~kDrop;
    opfx[s] = (k + s < len) ? (ref < A.n ? apf[ref - i0] : bpf[ref - A.n - j0]) : 0ull;
  }
  const uint64_t pa1 = a_first >= 1 ? sh.u.m.a_pfx[a_first - 1] : 0ull;
  const uint64_t pa2 = a_first >= 2 ? sh.u.m.a_pfx[a_first - 2] : 0ull;
  const uint64_t pb1 = b_first >= 1 ? sh.u.m.b_pfx[b_first - 1] : 0ull;
  uint32_t n_kept;
  uint32_t ord = block_exclusive_scan<uint32_t, kOpBlock>(kept, sh.scan32, n_kept);
  n_kept = __builtin_amdgcn_readfirstlane(n_kept);
  if (tid == 0) lookback_publish(desc_s, tile, n_kept);
#pragma unroll
  for (int s = 0; s < IPT; ++s) {
    if (k + s >= len) continue;
    const uint32_t r = refs[s];
    const uint32_t ref = r & ~kDrop;
    const bool drop = (r & kDrop) != 0;
    if (ref < A.n)
      sh.u.c.ords[ref - i0] = drop ? EM_NONE : ord;
    else
      sh.u.c.ords[nA_t + (ref - A.n - j0)] = ord;
    if (!drop) {
      sh.u.c.surv[ord] = ref;
      sh.u.c.spfx[ord] = opfx[s];
      ++ord;
    }
  }
  __syncthreads();

  // ---- 5. each survivor: key, value, predecessor, LCP ----
  auto key_at = [&](uint32_t ref) -> KeyRef {
    if (ref >= A.n) {
      const uint32_t y = ref - A.n - j0;
      return KeyRef{bo[y], bo[y + 1] - bo[y]};
    }
    const uint32_t x = ref - i0;
    return KeyRef{ao[x], ao[x + 1] - ao[x]};
  };
  uint32_t sref[IPT], l[IPT], klen[IPT], kprev[IPT];
#pragma unroll
  for (int u = 0; u < IPT; ++u) {
    const uint32_t x = tid + u * kOpBlock;
    sref[u] = klen[u] = l[u] = kprev[u] = 0;
    if (x >= n_kept) continue;
    const uint32_t ref = sh.u.c.surv[x];
    sref[u] = ref;
    const uint8_t* xb = ref >= A.n ? B.keys : A.keys;
    const KeyRef xk = key_at(ref);
    const uint64_t xp = sh.u.c.spfx[x];
    if (x > 0) {
      const uint32_t pref = sh.u.c.surv[x - 1];
      const KeyRef pk = key_at(pref);
      l[u] = lcp_cached(sh.u.c.spfx[x - 1], xp, cp, pref >= A.n ? B.keys : A.keys, pk, xb, xk);
      kprev[u] = 8u * pk.len;
    } else if (d0 > 0) {
      // The largest surviving key before the partition: A[i0-1] unless it is
      // the replaced copy of this very key (then A[i0-2]), or B[j0-1],
      // whichever is larger.
      bool hA = false, hB = false;
      KeyRef ka{0, 0}, kb{0, 0};
      uint64_t pa = 0, pbx = 0;
      if (a_first >= 1) {
        ka = KeyRef{sh.a_off[a_first - 1], sh.a_off[a_first] - sh.a_off[a_first - 1]};
        pa = pa1;
        hA = true;
        if (cmp_cached(pa, xp, cp, A.keys, ka, xb, xk) == 0) {
          hA = a_first >= 2;
          if (hA) {
            ka = KeyRef{sh.a_off[a_first - 2], sh.a_off[a_first - 1] - sh.a_off[a_first - 2]};
            pa = pa2;
          }
        }
      }
      if (b_first >= 1) {
        kb = KeyRef{sh.b_off[b_first - 1], sh.b_off[b_first] - sh.b_off[b_first - 1]};
        pbx = pb1;
        hB = true;
      }
      if (hA || hB) {
        const bool use_a = hA && (!hB || cmp_cached(pa, pbx, cp, A.keys, ka, B.keys, kb) > 0);
        const KeyRef pk = use_a ? ka : kb;
        l[u] = lcp_cached(use_a ? pa : pbx, xp, cp, use_a ? A.keys : B.keys, pk, xb, xk);
        kprev[u] = 8u * pk.len;
      }
    }
    klen[u] = xk.len;
  }
  // value length and presence of a survivor, from LDS
  auto val_at = [&](uint32_t ref, uint32_t& vpos, uint32_t& vlen) -> bool {  // true: tombstone
    const bool isB = ref >= A.n;
    const uint32_t x = isB ? ref - A.n - j0 : ref - i0;
    const uint32_t* vo = isB ? sh.b_voff : sh.a_voff;
    const bool t = (isB ? sh.b_tomb[x] : sh.a_tomb[x]) != 0;
    vpos = vo[x];
    vlen = t ? 0u : vo[x + 1] - vpos;
    return t;
  };

  // ---- 6. survivor base (first look-back) ----
  const uint32_t g0 = static_cast<uint32_t>(lookback_block(desc_s, tile, sh.red));
  if (tid == 0) desc_store(desc_s + tile, kDescIncl | (g0 + n_kept));

  // ---- 7. controls, exact lengths, partition-local bit offsets ----
  uint32_t cc[IPT], rlen[IPT];
#pragma unroll
  for (int u = 0; u < IPT; ++u) {
    const uint32_t x = tid + u * kOpBlock;
    cc[u] = rlen[u] = 0;
    if (x >= n_kept) continue;
    uint32_t vpos, vlen;
    const bool t = val_at(sref[u], vpos, vlen);
    const uint32_t kb = 8u * klen[u];
    cc[u] = ((g0 + x) % 15u == 0) ? 1u + l[u] : kprev[u] - l[u];
    rlen[u] = eg0_len(cc[u]) + eg0_len(kb - l[u]) + (kb - l[u]) + (t ? 1u : 1u + eg0_len(vlen) + 8u * vlen);
  }
  uint64_t tile_bits, sb[IPT], rl[IPT];
#pragma unroll
  for (int u = 0; u < IPT; ++u) rl[u] = rlen[u];
  block_exclusive_scan_rounds<uint64_t, kOpBlock, IPT>(rl, sh.scan64, sb, tile_bits);
  if (tid == 0) lookback_publish(out.desc_b, tile, tile_bits);

  // optional per-record outputs; the ordinals leave LDS before the window reuses it
#pragma unroll
  for (int u = 0; u < IPT; ++u) {
    const uint32_t x = tid + u * kOpBlock;
    if (x >= n_kept) continue;
    if (out.final_refs) out.final_refs[g0 + x] = sref[u];
    if (out.lcp_bits) out.lcp_bits[g0 + x] = l[u];
    if (out.len_bits) out.len_bits[g0 + x] = rlen[u];
  }
  if (out.ord_A)
    for (uint32_t x = tid; x < nA_t; x += kOpBlock) {
      const uint32_t o = sh.u.c.ords[x];
      out.ord_A[i0 + x] = o == EM_NONE ? EM_NONE : g0 + o;
    }
  if (out.ord_B)
    for (uint32_t y = tid; y < nB_t; y += kOpBlock) out.ord_B[j0 + y] = g0 + sh.u.c.ords[nA_t + y];
  if (tid == 0) {
    out.tile_bits[tile] = tile_bits;
    out.edge_lo[tile] = 0;
    out.edge_hi[tile] = 0;
    sh.carry = 0;
  }

  // ---- 8. emission, chunk by chunk ----
  // (readfirstlane returns an int: each half goes through uint32_t, so that a
  // low half of 2^31 or more does not sign-extend into the high one)
  auto uni64 = [](uint64_t v) {
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32)));
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v)));
    return (static_cast<uint64_t>(hi) << 32) | lo;
  };
  const uint64_t tbits = uni64(tile_bits);
  // Survivors per chunk: its bits should fill about 90% of the window and
  // its source spans (keys and values of every record between its first and
  // last survivor, replaced ones included) about 85% of the stage.
  uint32_t cs = kOpMaxChunk;
  if (n_kept) {
    const uint64_t src = static_cast<uint64_t>(ao[nA_t] - ao[0]) + (bo[nB_t] - bo[0]) +
                         (sh.a_voff[nA_t] - sh.a_voff[0]) + (sh.b_voff[nB_t] - sh.b_voff[0]);
    const uint64_t by_bits = (static_cast<uint64_t>(kOpWin) * 32u * 9u / 10u) * n_kept / (tbits ? tbits : 1);
    const uint64_t by_src = (static_cast<uint64_t>(kOpStage) * 85u / 100u) * n_kept / (src + 16u * len + 1u);
    const uint64_t c = min_u64(by_bits, by_src);
    cs = c < 1 ? 1u : (c > kOpMaxChunk ? kOpMaxChunk : static_cast<uint32_t>(c));
  }
  cs = __builtin_amdgcn_readfirstlane(cs);
  const uint32_t nch = (n_kept + cs - 1) / cs;
  uint32_t* const win = sh.u.e.win;
  const uint32_t* const stg = reinterpret_cast<const uint32_t*>(sh.u.e.stage);
  uint64_t Bt = 0;
  if (tid == 0) sh.carry = 0;
#pragma unroll 1
  for (uint32_t ch = 0; ch < nch; ++ch) {
    const uint32_t x0 = ch * cs, x1 = min(x0 + cs, n_kept);
    // this thread's survivor in the chunk, if any (at most one of its slots)
    bool act = false;
    uint32_t ref = 0, lc = 0, ctl = 0, rl = 0, slot = 0;
    uint64_t lo = 0;
#pragma unroll
    for (int v = 0; v < IPT; ++v) {
      const uint32_t xv = tid + v * kOpBlock;
      const bool in = xv >= x0 && xv < x1;
      act |= in;
      slot = in ? static_cast<uint32_t>(v) : slot;
      ref = in ? sref[v] : ref;
      lc = in ? l[v] : lc;
      ctl = in ? cc[v] : ctl;
      rl = in ? rlen[v] : rl;
      lo = in ? sb[v] : lo;
      if (in && xv == x0) sh.clo = sb[v];
      if (in && xv == x1 - 1) sh.chi = sb[v] + rlen[v];
    }
    const bool isB = ref >= A.n;
    uint32_t vpos = 0, vlen = 0;
    bool tomb = false;
    KeyRef xk{0, 0};
    if (act) {
      tomb = val_at(ref, vpos, vlen);
      xk = key_at(ref);
    }
    if (tid < 4) {
      sh.span_lo[tid] = 0xFFFFFFFFu;
      sh.span_hi[tid] = 0;
    }
    __syncthreads();  // (also: every read of the compaction arrays is done)
    const uint32_t ksl = xk.pos + (lc >> 3);  // first key byte the record emits
    {
      // Lanes holding the same slot v have survivors in lane order, and a
      // side's survivors are in arena order: per slot, the first and last
      // such lane bound each span.
      const bool ks = act && ksl < xk.pos + xk.len, vs = act && vlen != 0;
#pragma unroll
      for (int v = 0; v < IPT; ++v) {
        const bool in = slot == static_cast<uint32_t>(v);
        span_widen(in && ks && !isB, ksl, xk.pos + xk.len, &sh.span_lo[0], &sh.span_hi[0]);
        span_widen(in && ks && isB, ksl, xk.pos + xk.len, &sh.span_lo[1], &sh.span_hi[1]);
        span_widen(in && vs && !isB, vpos, vpos + vlen, &sh.span_lo[2], &sh.span_hi[2]);
        span_widen(in && vs && isB, vpos, vpos + vlen, &sh.span_lo[3], &sh.span_hi[3]);
      }
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t at = 0;
      for (int q = 0; q < 4; ++q) {
        sh.stage_at[q] = at;
        if (sh.span_lo[q] < sh.span_hi[q]) {
          const uint32_t slo = sh.span_lo[q] & ~15u;
          // reads reach at most one dword past the last byte's dword
          const uint32_t shi = (sh.span_hi[q] + 8u + 15u) & ~15u;
          sh.span_lo[q] = slo;
          sh.span_hi[q] = shi;
          const uint8_t* base = q == 0 ? A.keys : q == 1 ? B.keys : q == 2 ? A.vals : B.vals;
          sh.src_at[q] = reinterpret_cast<uint64_t>(base) + slo - at;
          at += shi - slo;
        } else {
          sh.span_lo[q] = 0;
          sh.span_hi[q] = 0;
          sh.src_at[q] = 0;  // (no staged byte maps to an empty span)
        }
      }
      sh.stage_at[4] = at;
    }
    __syncthreads();
    const uint32_t stage_total = __builtin_amdgcn_readfirstlane(sh.stage_at[4]);
    const bool staged = stage_total <= kOpStage;
    if (staged && stage_total > 0) {
      // global -> LDS without registers: each wave moves 64 consecutive
      // 16-byte chunks, lane i's chunk landing 16 i bytes after the wave's base
      const uint32_t total16 = stage_total / 16;
      const uint32_t at1 = sh.stage_at[1], at2 = sh.stage_at[2], at3 = sh.stage_at[3];
      const uint32_t lane = tid & (kWave - 1);
      for (uint32_t c0 = (tid / kWave) * kWave; c0 < total16; c0 += kOpBlock) {
        const uint32_t c = c0 + lane;
        if (c < total16) {
          const uint32_t byte = c * 16;
          const uint32_t q = (byte >= at1) + (byte >= at2) + (byte >= at3);
          lds_dma16(reinterpret_cast<const uint8_t*>(sh.src_at[q] + byte), sh.u.e.stage + c0);
        }
      }
    }
    if (ch == 0) {
      // the bit base, while the first chunk's sources are in flight
      Bt = lookback_block(out.desc_b, tile, sh.red);
      if (tid == 0) {
        desc_store(out.desc_b + tile, kDescIncl | (Bt + tbits));
        sh.base = Bt;
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    Bt = uni64(sh.base);
    const uint64_t clo = uni64(sh.clo), chi = uni64(sh.chi);
    if (ch == 0 && out.off) {
#pragma unroll
      for (int v = 0; v < IPT; ++v) {
        const uint32_t y = tid + v * kOpBlock;
        if (y < n_kept) out.off[g0 + y] = Bt + sb[v];
      }
    }

    // the record's fields
    OpRec r;
    const uint32_t kbits = 8u * xk.len;
    r.c = ctl;
    r.s = kbits - lc;
    r.b1 = eg0_len(r.c);
    r.b2 = r.b1 + eg0_len(r.s);
    r.b3 = r.b2 + r.s;
    const uint32_t ev = eg0_len(vlen);
    r.b4 = r.b3 + (tomb ? 1u : 1u + ev);
    r.b5 = rl;
    r.vh = tomb ? 0ull : ((1ull << ev) | (static_cast<uint64_t>(vlen) + 1ull));
    const uint32_t qk = isB ? 1u : 0u, qv = isB ? 3u : 2u;
    // staged: bit positions in the stage; in place: the arena pointer moves to
    // the dword holding the first byte, so that positions stay 32-bit
    r.kbit = staged ? 8u * (ksl - sh.span_lo[qk] + sh.stage_at[qk]) + (lc & 7u) : 8u * (ksl & 3u) + (lc & 7u);
    r.vbit = staged ? 8u * (vpos - sh.span_lo[qv] + sh.stage_at[qv]) : 8u * (vpos & 3u);
    const uint32_t* kg = reinterpret_cast<const uint32_t*>((isB ? B.keys : A.keys) + (ksl & ~3u));
    const uint32_t* vg = reinterpret_cast<const uint32_t*>((isB ? B.vals : A.vals) + (vpos & ~3u));

    // window slices over the chunk's bits [Bt + clo, Bt + chi); each slice
    // starts at a multiple of 128 bits, and a later slice repeats the bits of
    // the words before its predecessor's end that the predecessor left partial
    const uint64_t alo = Bt + clo, ahi = Bt + chi;
    const uint64_t first_full = (Bt + 31) >> 5;  // the partition's first word of its own
    uint64_t next_w = max_u64(first_full, alo >> 5);  // next word to store
    const uint64_t ro = Bt + lo, re = ro + rl;
    const bool whole = ((ahi - ((alo >> 7) << 7) + 31) >> 5) <= kOpWin;  // (uniform) one slice
    for (uint64_t s0 = (alo >> 7) << 7;;) {
      const uint64_t s1 = min_u64(s0 + 32ull * kOpWin, ahi);
      const uint64_t wbase = s0 >> 5;
      const uint32_t used4 = static_cast<uint32_t>(((s1 - s0 + 31) / 32 + 3) / 4);
      for (uint32_t i = tid; i < used4; i += kOpBlock) reinterpret_cast<uint4*>(win)[i] = uint4{0, 0, 0, 0};
      __syncthreads();
      // (ORed: other lanes may already be ORing their first bits into it)
      if (tid == 0 && s0 <= alo && ch > 0 && (alo & 31u)) atomicOr(&win[(alo >> 5) - wbase], sh.carry);
      if (act && ro < s1 && re > s0) {
        if (whole) {
          if (staged)
            append_whole(win, static_cast<uint32_t>(ro - s0), r, stg, stg);
          else
            append_whole(win, static_cast<uint32_t>(ro - s0), r, kg, vg);
        } else {
          const uint32_t from = ro >= s0 ? 0u : static_cast<uint32_t>(s0 - ro);
          const uint32_t to = re <= s1 ? rl : static_cast<uint32_t>(s1 - ro);
          const uint32_t p = static_cast<uint32_t>(ro + from - s0);
          if (staged)
            append_clipped(win, p, r, from, to, stg, stg);
          else
            append_clipped(win, p, r, from, to, kg, vg);
        }
      }
      __syncthreads();
      // complete words of this slice: 16-byte stores between a head and a tail
      auto wv = [&](uint64_t w) { return __builtin_bswap32(win[static_cast<uint32_t>(w - wbase)]); };
      const uint64_t o_lo = max_u64(next_w, wbase), o_hi = s1 >> 5;
      if (o_lo < o_hi) {
        // (indices relative to window word 0, payload word wbase, a multiple of four)
        uint32_t* const dst = out.payload + wbase;
        const uint32_t r_lo = static_cast<uint32_t>(o_lo - wbase), r_hi = static_cast<uint32_t>(o_hi - wbase);
        const uint32_t a_lo = min((r_lo + 3u) & ~3u, r_hi), a_hi = max(r_hi & ~3u, a_lo);
        for (uint32_t i = r_lo + tid; i < a_lo; i += kOpBlock) dst[i] = __builtin_bswap32(win[i]);
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        for (uint32_t i = a_lo + 4 * tid; i < a_hi; i += 4 * kOpBlock) {
          const uint4 v = reinterpret_cast<const uint4*>(win)[i / 4];
          const u32x4 q = {__builtin_bswap32(v.x), __builtin_bswap32(v.y), __builtin_bswap32(v.z),
                           __builtin_bswap32(v.w)};
          __builtin_nontemporal_store(q, reinterpret_cast<u32x4*>(dst + i));
        }
        for (uint32_t i = a_hi + tid; i < r_hi; i += kOpBlock) dst[i] = __builtin_bswap32(win[i]);
        next_w = o_hi;
      }
      if (tid == 0) {
        // the partition's first word, shared with the previous partition: its
        // bits are complete in the window of the last chunk starting in it
        // (earlier chunks' bits arrive there through the carry)
        if ((Bt & 31u) && s0 <= alo && (alo >> 5) == (Bt >> 5)) out.edge_lo[tile] = wv(Bt >> 5);
        if (s1 == ahi && (ahi & 31u)) {
          if (ch + 1 < nch)
            sh.carry = win[(ahi >> 5) - wbase];  // completed by the next chunk
          else
            out.edge_hi[tile] = wv(ahi >> 5);  // the partition's last word, shared with the next
        }
      }
      if (s1 == ahi) break;  // (uniform)
      __syncthreads();
      s0 = (s1 >> 7) << 7;
    }
    __syncthreads();
  }
  if (n_kept == 0) {  // (uniform) no survivors here: the bit base still passes through
    Bt = lookback_block(out.desc_b, tile, sh.red);
    if (tid == 0) desc_store(out.desc_b + tile, kDescIncl | Bt);
  }
  if (tid == 0 && tile == P - 1) {
    out.d_S[0] = g0 + n_kept;
    out.d_T[0] = Bt + tbits;
    if (out.off) out.off[g0 + n_kept] = Bt + tbits;
  }
}

// The words that a partition boundary, or the end of the payload, cuts.
// Thread q (1 <= q <= P; boundary P is T) takes the word W holding boundary q
// when it is the first boundary inside W: W is the last word of the previous
// partition with bits, f, and the first word of the partitions starting
// inside W; W = f's bits there | theirs (an empty partition contributes none).
__device__ __forceinline__ uint64_t op_start(const uint64_t* desc_b, const uint64_t* tile_bits, uint32_t r) {
  return (desc_b[r] & kDescValue) - tile_bits[r];
}

__global__ __launch_bounds__(256) void k_op_edges(const uint64_t* __restrict__ desc_b,
                                                  const uint64_t* __restrict__ tile_bits,
                                                  const uint32_t* __restrict__ edge_lo,
                                                  const uint32_t* __restrict__ edge_hi, uint32_t P,
                                                  uint32_t* __restrict__ payload) {
  const uint32_t q = blockIdx.x * 256 + threadIdx.x;
  if (q == 0 || q > P) return;
  if (q < P && tile_bits[q] == 0) return;  // (the next partition with bits, or T, has the same boundary)
  const uint64_t Bq = q < P ? op_start(desc_b, tile_bits, q) : (desc_b[P - 1] & kDescValue);
  if ((Bq & 31u) == 0) return;
  uint32_t f = q - 1;
  while (f > 0 && tile_bits[f] == 0) --f;
  if (tile_bits[f] == 0) return;  // (no bits before Bq; then Bq = 0)
  const uint64_t W = Bq >> 5;
  if (op_start(desc_b, tile_bits, f) > 32 * W) return;  // f starts inside W: its own boundary takes W
  uint32_t v = edge_hi[f];
  for (uint32_t r = q; r < P && op_start(desc_b, tile_bits, r) < 32 * (W + 1); ++r) v |= edge_lo[r];
  payload[W] = v;
}

// Workspace: the two look-backs' descriptors, partition bit totals, edge words.
struct OpLayout {
  uint32_t* ticket;
  uint64_t* desc_s;
  uint64_t* desc_b;
  uint64_t* tile_bits;
  uint32_t* edge_lo;
  uint32_t* edge_hi;
};

size_t op_ws_bytes(uint32_t N, uint32_t items) {
  const size_t P = items ? (static_cast<size_t>(N) + items - 1) / items : 0;
  const size_t p = P ? P : 1;
  return 256 + 3 * align_up(p * 8, 256) + 2 * align_up(p * 4, 256);
}

static OpLayout op_layout(void* ws, uint32_t N, uint32_t items) {
  const size_t P = items ? (static_cast<size_t>(N) + items - 1) / items : 0;
  const size_t p = P ? P : 1;
  WsCursor cur{static_cast<uint8_t*>(ws), 0};
  OpLayout L;
  L.ticket = cur.take<uint32_t>(64);
  L.desc_s = cur.take<uint64_t>(p);
  L.desc_b = cur.take<uint64_t>(p);
  L.tile_bits = cur.take<uint64_t>(p);
  L.edge_lo = cur.take<uint32_t>(p);
  L.edge_hi = cur.take<uint32_t>(p);
  return L;
}

template <int IPT>
static void launch_op(const em_side_t& A, const em_side_t& B, const uint32_t* csplits, uint32_t coarse,
                      uint32_t items, uint32_t P, const OpOut& o, const OpLayout& L, hipStream_t st) {
  hipLaunchKernelGGL((k_onepass<IPT>), dim3(P), dim3(kOpBlock), 0, st, A, B, csplits, coarse, items, P, o, L.ticket,
                     L.desc_s);
}

}  // namespace em

using namespace em;

extern "C" size_t em_onepass_workspace_bytes(uint32_t nA, uint32_t nB, uint32_t items_per_part) {
  const uint64_t N = static_cast<uint64_t>(nA) + nB;
  return op_ws_bytes(N >= EM_MAX_RECORDS ? EM_MAX_RECORDS : static_cast<uint32_t>(N),
                     items_per_part ? items_per_part : 1);
}

extern "C" int em_merge_fc_onepass(const em_side_t* A, const em_side_t* B, const uint32_t* coarse_splits,
                                   uint32_t coarse_items, uint32_t items_per_part, uint32_t* payload,
                                   uint64_t payload_words, uint32_t* d_S, uint64_t* d_T, uint32_t* final_refs,
                                   uint32_t* ord_A, uint32_t* ord_B, uint32_t* len_bits, uint32_t* lcp_bits,
                                   uint64_t* off, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_pair(A, B);
  if (rc) return rc;
  if (!ws || items_per_part == 0 || items_per_part > kOpMaxItems) return EM_EINVAL;
  if (reinterpret_cast<uintptr_t>(ws) & 255) return EM_EINVAL;
  if (ws_bytes < op_ws_bytes(A->n + B->n, items_per_part)) return EM_ENOSPC;
  if (!payload || !coarse_splits || !d_S || !d_T) return EM_EINVAL;
  if (reinterpret_cast<uintptr_t>(payload) & 15) return EM_EINVAL;
  if (coarse_items == 0 || coarse_items % items_per_part || coarse_items > EM_MAX_ITEMS_PER_PART * 256u)
    return EM_EINVAL;
  uint64_t bound = 0;
  rc = em_payload_bound_bits(A, B, &bound);
  if (rc) return rc;
  if (payload_words < (bound + 31) / 32) return EM_ENOSPC;
  hipStream_t st = as_stream(stream);
  const uint32_t N = A->n + B->n;
  if (N == 0) {
    clear_u32(d_S, 1, st);
    clear_u64(d_T, 1, st);
    if (off) clear_u64(off, 1, st);
    return check_launch();
  }
  const uint32_t P = (N + items_per_part - 1) / items_per_part;
  const OpLayout L = op_layout(ws, N, items_per_part);
  clear_lookback(L.ticket, 1, L.desc_s, L.desc_b, P, st);
  const OpOut o{d_S, d_T, payload, L.desc_b, L.tile_bits, L.edge_lo, L.edge_hi,
                final_refs, ord_A, ord_B, len_bits, lcp_bits, off};
  if (items_per_part <= static_cast<uint32_t>(kOpBlock))
    launch_op<1>(*A, *B, coarse_splits, coarse_items, items_per_part, P, o, L, st);
  else if (items_per_part <= 2u * kOpBlock)
    launch_op<2>(*A, *B, coarse_splits, coarse_items, items_per_part, P, o, L, st);
  else
    launch_op<4>(*A, *B, coarse_splits, coarse_items, items_per_part, P, o, L, st);
  hipLaunchKernelGGL(k_op_edges, dim3(P / 256 + 1), dim3(256), 0, st, L.desc_b, L.tile_bits, L.edge_lo, L.edge_hi,
                     P, payload);
  return check_launch();
}
