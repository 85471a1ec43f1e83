// Internal helpers of the gfx950 merge / front-coding library: key access,
// comparisons and bit LCP on byte arenas, wave64 primitives, the
// decoupled look-back used by the single-pass scans, and host-side launch
// plumbing.  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "em.h"

namespace em {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Byte-arena access.  Arena bases are 16-byte aligned and padded by
// EM_ARENA_PAD (32) readable bytes, so the aligned dwords around any byte
// position inside an arena, up to 20 bytes past it, are always readable.

// 8 bytes starting at byte `pos`, as a big-endian u64 (first byte most
// significant): numeric order of these words is bytewise order of the bytes.
__device__ __forceinline__ uint64_t load_be8(const uint8_t* base, uint32_t pos) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(base + (pos & ~3u));
  const uint32_t s = pos & 3u;
  const uint32_t w0 = w[0], w1 = w[1], w2 = w[2];
  const uint32_t lo = __builtin_amdgcn_alignbyte(w1, w0, s);
  const uint32_t hi = __builtin_amdgcn_alignbyte(w2, w1, s);
  return (static_cast<uint64_t>(__builtin_bswap32(lo)) << 32) | __builtin_bswap32(hi);
}

// Mask keeping the first `nbytes` (0..8) bytes of a big-endian word.
__device__ __forceinline__ uint64_t be_mask(uint32_t nbytes) {
  return nbytes >= 8 ? ~0ull : (nbytes == 0 ? 0ull : ~0ull << (8 * (8 - nbytes)));
}

struct KeyRef {
  uint32_t pos;  // byte offset in its arena
  uint32_t len;  // bytes
};

// 16 bytes starting at byte `pos` as two big-endian u64s (reads the five
// aligned dwords around them).
__device__ __forceinline__ void load_be16(const uint8_t* base, uint32_t pos, uint64_t& hi, uint64_t& lo) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(base + (pos & ~3u));
  const uint32_t s = pos & 3u;
  const uint32_t w0 = w[0], w1 = w[1], w2 = w[2], w3 = w[3], w4 = w[4];
  const uint32_t d0 = __builtin_amdgcn_alignbyte(w1, w0, s);
  const uint32_t d1 = __builtin_amdgcn_alignbyte(w2, w1, s);
  const uint32_t d2 = __builtin_amdgcn_alignbyte(w3, w2, s);
  const uint32_t d3 = __builtin_amdgcn_alignbyte(w4, w3, s);
  hi = (static_cast<uint64_t>(__builtin_bswap32(d0)) << 32) | __builtin_bswap32(d1);
  lo = (static_cast<uint64_t>(__builtin_bswap32(d2)) << 32) | __builtin_bswap32(d3);
}

// The next up-to-32 common bytes of two keys, as four big-endian u64s each,
// bytes past `r` (the common bytes left) zeroed.  Both halves are loaded
// before either is used, so one memory round trip covers 32 bytes.
struct Chunk32 {
  uint64_t v[4];
};
__device__ __forceinline__ void load_pair32(const uint8_t* ka, uint32_t pa, const uint8_t* kb, uint32_t pb,
                                            uint32_t r, Chunk32& a, Chunk32& b) {
  load_be16(ka, pa, a.v[0], a.v[1]);
  load_be16(kb, pb, b.v[0], b.v[1]);
  a.v[2] = a.v[3] = b.v[2] = b.v[3] = 0;
  if (r > 16) {
    load_be16(ka, pa + 16, a.v[2], a.v[3]);
    load_be16(kb, pb + 16, b.v[2], b.v[3]);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t rq = r > 8u * q ? r - 8u * q : 0u;
    const uint64_t m = be_mask(rq);
    a.v[q] &= m;
    b.v[q] &= m;
  }
}

// Unsigned bytewise comparison with a proper prefix first: <0, 0, >0.
__device__ __forceinline__ int cmp_keys(const uint8_t* ka, KeyRef a, const uint8_t* kb, KeyRef b) {
  const uint32_t m = a.len < b.len ? a.len : b.len;
  for (uint32_t t = 0; t < m; t += 32) {
    Chunk32 x, y;
    load_pair32(ka, a.pos + t, kb, b.pos + t, m - t, x, y);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (x.v[q] != y.v[q]) return x.v[q] < y.v[q] ? -1 : 1;
  }
  return (a.len > b.len) - (a.len < b.len);
}

// Exact bit LCP (MSB first within bytes), clamped to the shorter key.
__device__ __forceinline__ uint32_t lcp_bits(const uint8_t* ka, KeyRef a, const uint8_t* kb, KeyRef b) {
  const uint32_t m = a.len < b.len ? a.len : b.len;
  for (uint32_t t = 0; t < m; t += 32) {
    Chunk32 x, y;
    load_pair32(ka, a.pos + t, kb, b.pos + t, m - t, x, y);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint64_t d = x.v[q] ^ y.v[q];
      if (d) return 8 * t + 64u * q + static_cast<uint32_t>(__builtin_clzll(d));
    }
  }
  return 8 * m;
}

__device__ __forceinline__ KeyRef key_of(const em_side_t& s, uint32_t r) {
  const uint32_t p = s.key_off[r];
  return KeyRef{p, s.key_off[r + 1] - p};
}

// Unsigned 64-bit min and max.  HIP's own min/max, given two different
// 64-bit integer types (unsigned long and unsigned long long), resolve to
// their double overload: about twenty VALU instructions through f64, exact only
// below 2^53.
__host__ __device__ __forceinline__ uint64_t min_u64(uint64_t a, uint64_t b) { return a < b ? a : b; }
__host__ __device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// E(x) = 2 floor(log2(x+1)) + 1, the length of order-zero Exp-Golomb.
__device__ __forceinline__ uint32_t eg0_len(uint64_t x) {
  return 2u * (63u - static_cast<uint32_t>(__builtin_clzll(x + 1))) + 1u;
}

// The bounds of this wave's selected lanes' ranges [lo, hi), for ranges that
// increase with the lane (as in span_widen below): the first selected lane's
// lo and the last one's hi, wave-uniform; (~0, 0) when no lane is selected.
// Every active lane of the wave calls it.
__device__ __forceinline__ void wave_bounds(bool sel, uint32_t lo, uint32_t hi, uint32_t& blo, uint32_t& bhi) {
  const uint64_t m = __ballot(sel);
  blo = 0xFFFFFFFFu;
  bhi = 0;
  if (m) {
    blo = __builtin_amdgcn_readlane(lo, __builtin_ctzll(m));
    bhi = __builtin_amdgcn_readlane(hi, 63 - __builtin_clzll(m));
  }
}

// Widens a workgroup's byte span [*span_lo, *span_hi) (LDS) to cover the
// ranges [lo, hi) of this wave's selected lanes, for ranges that increase
// with the lane (a later selected lane's lo and hi are at least an earlier
// one's, as for the records of one side in merged order): the first
// selected lane holds the smallest lo and the last the largest hi, so the
// first selected lane updates both bounds.  (An LDS atomic from every lane on
// the same word is serialised by the LDS, one lane per cycle.)  Every active
// lane of the wave calls it.
__device__ __forceinline__ void span_widen(bool sel, uint32_t lo, uint32_t hi, uint32_t* span_lo,
                                           uint32_t* span_hi) {
  const uint64_t m = __ballot(sel);
  if (m) {
    const int first = __builtin_ctzll(m), last = 63 - __builtin_clzll(m);
    // (wave-uniform operands: the atomics then compile to one lane's LDS
    // atomic, not to a loop over the active lanes)
    const uint32_t vlo = __builtin_amdgcn_readlane(lo, first), vhi = __builtin_amdgcn_readlane(hi, last);
    if (__lane_id() == static_cast<uint32_t>(first)) {
      atomicMin(span_lo, vlo);
      atomicMax(span_hi, vhi);
    }
  }
}

// gfx950 global -> LDS load without registers: each active lane moves 16
// bytes from `src` (per lane) to `lds_wave_base` + 16 * lane, where
// `lds_wave_base` is the same for the whole wave.  The caller waits for the
// loads (s_waitcnt vmcnt) and synchronises before reading the LDS.
// The sources staged this way are read once, so the loads carry the
// non-temporal cache policy (cache-policy bit 1).  The emitter measured the
// same with either policy, within the run-to-run spread.
__device__ __forceinline__ void lds_dma16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint4*>(src), lds_wave_base, 16, 0, 2);
}

// ---------------------------------------------------------------------------
// Wave64 / block primitives.

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

template <class T>
__device__ __forceinline__ T wave_inclusive_scan(T v) {
  const uint32_t lane = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    T o = __shfl_up(v, d, kWave);
    if (lane >= static_cast<uint32_t>(d)) v += o;
  }
  return v;
}

// Exclusive scan across a block of NT threads.  `smem` holds NT/64 + 1 values.
// Returns the thread's exclusive prefix and writes the block total.
template <class T, int NT>
__device__ __forceinline__ T block_exclusive_scan(T v, T* smem, T& total) {
  constexpr int NW = NT / kWave;
  const uint32_t lane = lane_id();
  const uint32_t wid = threadIdx.x / kWave;
  T inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) smem[wid] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    T acc = 0;
    for (int w = 0; w < NW; ++w) {
      T t = smem[w];
      smem[w] = acc;
      acc += t;
    }
    smem[NW] = acc;
  }
  __syncthreads();
  total = smem[NW];
  T r = smem[wid] + inc - v;
  __syncthreads();
  return r;
}

// Exclusive scan of R values per thread where value u of thread t is element
// u * NT + t of the sequence (rounds of a strided layout), with two barriers.
// `smem` holds R * NT/64 + 1 values.
template <class T, int NT, int R>
__device__ __forceinline__ void block_exclusive_scan_rounds(const T (&v)[R], T* smem, T (&out)[R],
                                                            T& total) {
  constexpr int NW = NT / kWave;
  const uint32_t lane = lane_id();
  const uint32_t wid = threadIdx.x / kWave;
  T inc[R];
#pragma unroll
  for (int u = 0; u < R; ++u) {
    inc[u] = wave_inclusive_scan(v[u]);
    if (lane == kWave - 1) smem[u * NW + wid] = inc[u];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    T acc = 0;
    for (int w = 0; w < R * NW; ++w) {
      T t = smem[w];
      smem[w] = acc;
      acc += t;
    }
    smem[R * NW] = acc;
  }
  __syncthreads();
  total = smem[R * NW];
#pragma unroll
  for (int u = 0; u < R; ++u) out[u] = smem[u * NW + wid] + inc[u] - v[u];
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Decoupled look-back over per-tile descriptors (single-pass scan).  A
// descriptor packs a 2-bit status and a 62-bit value in one u64 so that one
// atomic access reads both.  Tiles take ids from an atomic ticket in launch
// order, so every tile waits only on tiles that already hold a ticket and are
// therefore resident or finished: the wait always ends.

constexpr uint64_t kDescAgg = 1ull << 62;
constexpr uint64_t kDescIncl = 2ull << 62;
constexpr uint64_t kDescValue = (1ull << 62) - 1;

// Relaxed agent-scope atomics: the status and the value travel in the same
// word and no other memory is handed between tiles, so no ordering is needed.
// (Acquire/release at agent scope would write back and invalidate the XCD's L2
// on every access, which also evicts the key bytes the merge relies on.)
__device__ __forceinline__ void desc_store(uint64_t* d, uint64_t v) {
  __hip_atomic_store(d, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t desc_load(const uint64_t* d) {
  return __hip_atomic_load(const_cast<uint64_t*>(d), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Publishes `aggregate` for `tile` (tile 0 publishes it as its inclusive
// value).  One lane suffices.  A tile publishes as early as it can and
// resolves as late as it can, so that its successors rarely wait.
__device__ __forceinline__ void lookback_publish(uint64_t* desc, uint32_t tile, uint64_t aggregate) {
  desc_store(desc + tile, (tile == 0 ? kDescIncl : kDescAgg) | aggregate);
}

// Called by all 64 lanes of ONE wave after lookback_publish: returns the
// exclusive prefix of all earlier tiles and publishes the inclusive value.
__device__ __forceinline__ uint64_t lookback_resolve(uint64_t* desc, uint32_t tile, uint64_t aggregate) {
  const uint32_t lane = lane_id();
  if (tile == 0) return 0;
  uint64_t excl = 0;
  int64_t base = static_cast<int64_t>(tile) - 1;
  while (true) {
    const int64_t idx = base - static_cast<int64_t>(lane);
    const uint64_t v = idx >= 0 ? desc_load(desc + idx) : kDescIncl;
    const uint64_t status = v >> 62;
    const uint64_t not_ready = __ballot(status == 0);
    const uint64_t incl = __ballot(status == 2);
    uint64_t upto;  // lanes whose values are summed this round
    if (incl) {
      const uint32_t f = static_cast<uint32_t>(__builtin_ctzll(incl));
      upto = f == 63 ? ~0ull : ((2ull << f) - 1);
    } else {
      upto = ~0ull;
    }
    if (not_ready & upto) {
      __builtin_amdgcn_s_sleep(1);
      continue;
    }
    uint64_t mine = ((upto >> lane) & 1ull) ? (v & kDescValue) : 0;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) mine += __shfl_xor(mine, d, kWave);
    excl += mine;
    if (incl) break;
    base -= kWave;
  }
  if (lane == 0) desc_store(desc + tile, kDescIncl | (excl + aggregate));
  return excl;
}

// Publish and resolve in one go (called by all 64 lanes of ONE wave).
__device__ __forceinline__ uint64_t lookback(uint64_t* desc, uint32_t tile, uint64_t aggregate) {
  if (lane_id() == 0) lookback_publish(desc, tile, aggregate);
  return lookback_resolve(desc, tile, aggregate);
}

// ---------------------------------------------------------------------------
// Host-side plumbing.

int set_hip_error(hipError_t e);  // records e, returns EM_EDEVICE
int check_launch();               // EM_OK or EM_EDEVICE after the last launch

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int check_side(const em_side_t* s);  // EM_OK / EM_EINVAL / EM_ERANGE
int check_pair(const em_side_t* A, const em_side_t* B);

// Workspace carving: sections are 256-byte aligned.
struct WsCursor {
  uint8_t* base;
  size_t used;
  template <class T>
  T* take(size_t count) {
    used = align_up(used, 256);
    T* p = reinterpret_cast<T*>(base + used);
    used += count * sizeof(T);
    return p;
  }
};

// Sizes of each call's workspace (bytes).
size_t merge_keep_ws(uint32_t N, uint32_t items_per_part);
size_t scan_ws(uint32_t S);
size_t collision_ws(uint32_t nA, uint32_t nB);
size_t rank_ws(uint32_t nbits);

// Zero `n` u64 words (a fill kernel rather than a memset so that the sequence
// stays valid inside a captured graph).
void clear_u64(uint64_t* p, size_t n, hipStream_t st);

// Single-pass exclusive scan of n u32 values into out[0..n] (out[n] = total),
// using workspace laid out as scan_ws(n) describes.
template <class OutT>
int scan_launch(const uint32_t* in, uint32_t n, OutT* out, void* ws, size_t ws_bytes, hipStream_t st);
void clear_u32(uint32_t* p, size_t n, hipStream_t st);
// A look-back's state in one launch: nt u32 ticket words and nd u64
// descriptors of d0 (and of d1 when it is not null).
void clear_lookback(uint32_t* ticket, size_t nt, uint64_t* d0, uint64_t* d1, size_t nd, hipStream_t st);

// A record offset in partition form: partition number (< 2^24) above this
// bit, the offset inside the partition's bits below it.
constexpr int kTiledShift = 40;

// Chunk ticket counters of the resident emitter: kEmitCtrs counters,
// kEmitCtrStride u32 apart (one 128-byte line each).  They must be zero
// before the first launch; each launch leaves them zero.
constexpr uint32_t kEmitCtrs = 8;
constexpr uint32_t kEmitCtrStride = 32;
constexpr uint32_t kEmitCtrWords = kEmitCtrs * kEmitCtrStride;

// The payload emitter reading S and T from device memory and record offsets
// as partition number << 40 | partition-local offset plus partition bit
// bases (em_fc.hip); off_out (nullable) receives the S+1 offsets; ctr holds
// kEmitCtrWords u32 of ticket counters.
int emit_launch_dev(const em_side_t& A, const em_side_t& B, const uint32_t* final_refs,
                    const uint32_t* lcp_bits, const uint64_t* toff, const uint64_t* tbase,
                    uint64_t* off_out, uint32_t* payload, const uint32_t* d_S, const uint64_t* d_T,
                    uint32_t* ctr, hipStream_t st);

}  // namespace em
