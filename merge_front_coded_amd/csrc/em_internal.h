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
// EM_ARENA_PAD readable bytes, so the aligned dwords around any byte position
// inside an arena (or up to 16 bytes past its end) are always readable.

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

// Unsigned bytewise comparison with a proper prefix first: <0, 0, >0.
__device__ __forceinline__ int cmp_keys(const uint8_t* ka, KeyRef a, const uint8_t* kb, KeyRef b) {
  const uint32_t m = a.len < b.len ? a.len : b.len;
  for (uint32_t t = 0; t < m; t += 8) {
    const uint64_t mask = be_mask(m - t);
    const uint64_t va = load_be8(ka, a.pos + t) & mask;
    const uint64_t vb = load_be8(kb, b.pos + t) & mask;
    if (va != vb) return va < vb ? -1 : 1;
  }
  return (a.len > b.len) - (a.len < b.len);
}

// Exact bit LCP (MSB first within bytes), clamped to the shorter key.
__device__ __forceinline__ uint32_t lcp_bits(const uint8_t* ka, KeyRef a, const uint8_t* kb, KeyRef b) {
  const uint32_t m = a.len < b.len ? a.len : b.len;
  for (uint32_t t = 0; t < m; t += 8) {
    const uint64_t mask = be_mask(m - t);
    const uint64_t x = (load_be8(ka, a.pos + t) ^ load_be8(kb, b.pos + t)) & mask;
    if (x) return 8 * t + static_cast<uint32_t>(__builtin_clzll(x));
  }
  return 8 * m;
}

__device__ __forceinline__ KeyRef key_of(const em_side_t& s, uint32_t r) {
  const uint32_t p = s.key_off[r];
  return KeyRef{p, s.key_off[r + 1] - p};
}

// E(x) = 2 floor(log2(x+1)) + 1, the length of order-zero Exp-Golomb.
__device__ __forceinline__ uint32_t eg0_len(uint64_t x) {
  return 2u * (63u - static_cast<uint32_t>(__builtin_clzll(x + 1))) + 1u;
}

// gfx950 global -> LDS load without registers: each active lane moves 16
// bytes from `src` (per lane) to `lds_wave_base` + 16 * lane, where
// `lds_wave_base` is the same for the whole wave.  The caller waits for the
// loads (s_waitcnt vmcnt) and synchronises before reading the LDS.
__device__ __forceinline__ void lds_dma16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint4*>(src), lds_wave_base, 16, 0, 0);
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

}  // namespace em
