// Byte-profile front coding of the survivors: LEB128 counts, byte literals,
// presence tags and a common value width.
//
// Everett, "Byte-profile GPU merge", "Pipeline": the GPU detects the common
// encoded value width, sizes and scans the output records and emits their
// byte FC payload (width seventeen: a tag byte for presence followed by
// sixteen bytes of value); the control rule is the bit profile's ("GPU construction
// experiment", the c_i equation) counted in bytes.
//
// Record layout (read as; the page names the parts only): LEB128(c_i),
// LEB128(k_i - l_i), key bytes l_i .. k_i - 1, then the value.  With l_i the
// byte LCP with the preceding survivor and k_i the key's byte length,
// c_i = 1 + l_i when i mod 15 = 0, else k_{i-1} - l_i.  Fixed framing (every
// present value L bytes long, or none present): width W = 1 + L, each value a
// tag byte (1 present, 0 tombstone) and L bytes (zeros for a tombstone).
// Otherwise (W = 0): tag 0 for a tombstone; tag 1, LEB128(length) and the
// bytes for a present value.  LEB128: seven bits per byte, low group first,
// high bit set while more follow.
#include <algorithm>

#include "em_tile.h"

namespace em {

constexpr int kBpBlock = 256;
constexpr uint32_t kBpWidthGrid = 1024;

__host__ __device__ inline uint32_t leb_bytes(uint32_t x) {
  return x < (1u << 7) ? 1u : x < (1u << 14) ? 2u : x < (1u << 21) ? 3u : x < (1u << 28) ? 4u : 5u;
}

struct BpWs {
  uint32_t* stat;  // [0] min and [1] max present value length, [2] present count
};

static BpWs bp_layout(void* ws) {
  WsCursor cur{static_cast<uint8_t*>(ws), 0};
  BpWs L{};
  L.stat = cur.take<uint32_t>(4);
  return L;
}

__global__ void k_bp_init(uint32_t* stat) {
  stat[0] = 0xFFFFFFFFu;
  stat[1] = 0;
  stat[2] = 0;
}

// min and max byte length of the present values, and how many are present
__global__ __launch_bounds__(kBpBlock) void k_bp_stats(em_side_t A, em_side_t B,
                                                       const uint32_t* __restrict__ final_refs, uint32_t S,
                                                       uint32_t* __restrict__ stat) {
  __shared__ uint32_t s0[kBpBlock / kWave], s1[kBpBlock / kWave], s2[kBpBlock / kWave];
  uint32_t lo = 0xFFFFFFFFu, hi = 0, cnt = 0;
  for (uint32_t i = blockIdx.x * kBpBlock + threadIdx.x; i < S; i += gridDim.x * kBpBlock) {
    uint32_t idx, vlen;
    bool tomb;
    const SideView s = pick(A, B, final_refs[i], idx);
    value_bits(s, idx, vlen, tomb);
    if (!tomb) {
      lo = min(lo, vlen);
      hi = max(hi, vlen);
      ++cnt;
    }
  }
  for (int d = kWave / 2; d > 0; d >>= 1) {
    lo = min(lo, static_cast<uint32_t>(__shfl_xor(static_cast<int>(lo), d)));
    hi = max(hi, static_cast<uint32_t>(__shfl_xor(static_cast<int>(hi), d)));
    cnt += static_cast<uint32_t>(__shfl_xor(static_cast<int>(cnt), d));
  }
  const uint32_t wv = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    s0[wv] = lo;
    s1[wv] = hi;
    s2[wv] = cnt;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (uint32_t t = 1; t < kBpBlock / kWave; ++t) {
      lo = min(lo, s0[t]);
      hi = max(hi, s1[t]);
      cnt += s2[t];
    }
    if (cnt) {
      atomicMin(stat, lo);
      atomicMax(stat + 1, hi);
      atomicAdd(stat + 2, cnt);
    }
  }
}

__global__ void k_bp_width(const uint32_t* __restrict__ stat, uint32_t S, uint32_t* __restrict__ d_width) {
  uint32_t w = 0;
  if (S) {
    if (stat[2] == 0)
      w = 1;  // no present value: the tag alone
    else if (stat[0] == stat[1])
      w = 1u + stat[0];
  }
  d_width[0] = w;
}

struct BpRec {
  uint32_t c, sfx, kpos, vlen, vpos, l;
  bool tomb, isB;
};

// Record i's fields: byte LCP from the bit LCP, c from the predecessor's key length.
__device__ __forceinline__ BpRec bp_record(const em_side_t& A, const em_side_t& B,
                                           const uint32_t* __restrict__ final_refs,
                                           const uint32_t* __restrict__ lcp_bits, uint32_t i) {
  uint32_t idx;
  const SideView s = pick(A, B, final_refs[i], idx);
  const KeyRef x = key_of(s, idx);
  uint32_t kprev = 0;
  if (i > 0) {
    uint32_t pidx;
    const SideView ps = pick(A, B, final_refs[i - 1], pidx);
    kprev = ps.key_off[pidx + 1] - ps.key_off[pidx];
  }
  BpRec r;
  r.l = min(lcp_bits[i] >> 3, x.len);  // (a stale array must not send reads past the key)
  r.c = (i % 15u == 0) ? 1u + r.l : kprev - r.l;
  r.sfx = x.len - r.l;
  r.kpos = x.pos + r.l;
  value_bits(s, idx, r.vlen, r.tomb, &r.vpos);
  r.isB = s.isB;
  return r;
}

__device__ __forceinline__ uint32_t bp_value_bytes(const BpRec& r, uint32_t W) {
  return W ? W : (r.tomb ? 1u : 1u + leb_bytes(r.vlen) + r.vlen);
}

__global__ __launch_bounds__(kBpBlock) void k_bp_lengths(em_side_t A, em_side_t B,
                                                         const uint32_t* __restrict__ final_refs,
                                                         const uint32_t* __restrict__ lcp_bits, uint32_t S,
                                                         const uint32_t* __restrict__ d_width,
                                                         uint32_t* __restrict__ len_bytes) {
  const uint32_t i = blockIdx.x * kBpBlock + threadIdx.x;
  if (i >= S) return;
  const BpRec r = bp_record(A, B, final_refs, lcp_bits, i);
  len_bytes[i] = leb_bytes(r.c) + leb_bytes(r.sfx) + r.sfx + bp_value_bytes(r, d_width[0]);
}

__device__ __forceinline__ uint64_t bp_put_leb(uint8_t* __restrict__ out, uint64_t at, uint32_t x) {
  do {
    const uint32_t b = x & 127u;
    x >>= 7;
    out[at++] = static_cast<uint8_t>(x ? (b | 128u) : b);
  } while (x);
  return at;
}

// n bytes from src to dst.  The destination is aligned first (single bytes
// up to a dword boundary), then written sixteen bytes at a time with dword
// stores, each output dword one funnel shift of two aligned source dwords
// (the loads of a group of five issued before its stores; arenas are padded,
// so the dword after the last byte is readable); the last 0..15 bytes as
// dwords and single bytes.  Records write disjoint bytes, so the single-byte
// stores at their ends never race with a neighbour's.
__device__ __forceinline__ void bp_copy(uint8_t* __restrict__ dst, const uint8_t* __restrict__ src, uint32_t n) {
  const uint32_t h = min(n, static_cast<uint32_t>(-reinterpret_cast<uintptr_t>(dst)) & 3u);
  for (uint32_t t = 0; t < h; ++t) dst[t] = src[t];
  dst += h;
  src += h;
  n -= h;
  const uint32_t* a = reinterpret_cast<const uint32_t*>(reinterpret_cast<uintptr_t>(src) & ~static_cast<uintptr_t>(3));
  const uint32_t sh = 8u * static_cast<uint32_t>(reinterpret_cast<uintptr_t>(src) & 3);
  uint32_t* d = reinterpret_cast<uint32_t*>(dst);
  uint32_t m = 0;  // dwords written
  for (; 4 * m + 16 <= n; m += 4) {
    uint32_t w[5];
#pragma unroll
    for (int t = 0; t < 5; ++t) w[t] = a[m + t];
#pragma unroll
    for (int t = 0; t < 4; ++t) d[m + t] = sh ? __builtin_amdgcn_alignbit(w[t + 1], w[t], sh) : w[t];
  }
  for (; 4 * m + 4 <= n; ++m) {
    const uint32_t w0 = a[m], w1 = a[m + 1];
    d[m] = sh ? __builtin_amdgcn_alignbit(w1, w0, sh) : w0;  // little-endian bytes
  }
  for (uint32_t t = 4 * m; t < n; ++t) dst[t] = src[t];
}

// n zero bytes: single bytes up to a dword boundary, dwords, single bytes
__device__ __forceinline__ void bp_zero(uint8_t* __restrict__ dst, uint32_t n) {
  const uint32_t h = min(n, static_cast<uint32_t>(-reinterpret_cast<uintptr_t>(dst)) & 3u);
  for (uint32_t t = 0; t < h; ++t) dst[t] = 0;
  uint32_t* d = reinterpret_cast<uint32_t*>(dst + h);
  uint32_t m = 0;
  for (; 4 * m + 4 <= n - h; ++m) d[m] = 0;
  for (uint32_t t = h + 4 * m; t < n; ++t) dst[t] = 0;
}

// Record i's bytes at dst[at ..), its key suffix from ksrc and its value from
// vsrc: dst a window in LDS or the payload itself, the sources staged in LDS
// or in place (each call site passes one combination, so that its loads and
// stores have one address space).
__device__ __forceinline__ void bp_write_record(uint8_t* __restrict__ dst, uint64_t at, const BpRec& r, uint32_t W,
                                                const uint8_t* __restrict__ ksrc,
                                                const uint8_t* __restrict__ vsrc) {
  at = bp_put_leb(dst, at, r.c);
  at = bp_put_leb(dst, at, r.sfx);
  bp_copy(dst + at, ksrc, r.sfx);
  at += r.sfx;
  dst[at++] = r.tomb ? 0 : 1;
  if (W) {
    if (r.tomb)
      bp_zero(dst + at, W - 1);
    else
      bp_copy(dst + at, vsrc, W - 1);
  } else if (!r.tomb) {
    at = bp_put_leb(dst, at, r.vlen);
    bp_copy(dst + at, vsrc, r.vlen);
  }
}

// A workgroup takes rpb consecutive records (one a thread), whose bytes
// [off[r0], off[r1]) are contiguous.  When they fit the LDS window (with the
// window starting at the 16-byte boundary below off[r0]), each thread writes
// its record there and the workgroup copies the window out with 16-byte
// stores, single bytes only in the two groups it shares with its neighbours;
// otherwise each thread writes its record to the payload directly.  The
// records' sources lie in four contiguous spans (A keys, B keys, A values, B
// values: the survivors of one side are increasing), which a windowed
// workgroup stages in LDS with 16-byte LDS-DMA loads when they fit, so that
// its threads copy from LDS instead of reading scattered global addresses.
constexpr uint32_t kBpWin = 12288;    // output bytes
constexpr uint32_t kBpStage = 12288;  // staged source bytes

struct BpShared {
  uint4 win[kBpWin / 16];
  uint4 stage[kBpStage / 16];
  uint32_t span_lo[4], span_hi[4];  // byte spans of the four sources
  uint4 wspan_lo[kBpBlock / kWave], wspan_hi[kBpBlock / kWave];  // each wave's bounds of the four
  uint32_t stage_at[5];             // LDS byte offset of each staged span, [4] = total
  uint64_t src_at[4];               // global address of each staged span's first byte, less stage_at
};

__global__ __launch_bounds__(kBpBlock) void k_bp_emit(em_side_t A, em_side_t B,
                                                      const uint32_t* __restrict__ final_refs,
                                                      const uint32_t* __restrict__ lcp_bits, uint32_t S,
                                                      uint32_t rpb, const uint64_t* __restrict__ off,
                                                      const uint32_t* __restrict__ d_width,
                                                      uint8_t* __restrict__ payload, uint64_t cap,
                                                      uint32_t* __restrict__ overflow) {
  __shared__ BpShared sh;
  const uint32_t tid = threadIdx.x;
  const uint32_t r0 = blockIdx.x * rpb;
  const uint32_t r1 = min(r0 + rpb, S);
  const uint64_t b0 = off[r0], b1 = off[r1];
  const uint64_t base = b0 & ~static_cast<uint64_t>(15);
  const bool staged = b0 <= b1 && b1 <= cap && b1 - base <= kBpWin;  // (uniform over the workgroup)
  const uint32_t W = d_width[0];
  const uint32_t i = r0 + tid;
  bool ok = false;
  BpRec r{};
  uint64_t at = 0;
  uint32_t vn = 0;  // value bytes copied from the source
  if (tid < rpb && i < r1) {
    r = bp_record(A, B, final_refs, lcp_bits, i);
    at = off[i];
    const uint64_t end = off[i + 1];
    // offsets or a width that do not belong to these records, or no room:
    // flag it and write nothing of the record (within the window, that
    // leaves its bytes unspecified)
    if (at > end || end > cap || end - at != leb_bytes(r.c) + leb_bytes(r.sfx) + r.sfx + bp_value_bytes(r, W) ||
        (W && !r.tomb && r.vlen != W - 1) || (staged && (at < b0 || end > b1))) {
      atomicOr(overflow, 1u);
    } else {
      ok = true;
      vn = r.tomb ? 0u : r.vlen;
    }
  }
  if (staged) {  // (uniform) a side's records are in arena order: see wave_bounds
    const bool ks = ok && r.sfx != 0, vs = ok && vn != 0;
    uint4 blo, bhi;  // (wave-uniform)
    wave_bounds(ks && !r.isB, r.kpos, r.kpos + r.sfx, blo.x, bhi.x);
    wave_bounds(ks && r.isB, r.kpos, r.kpos + r.sfx, blo.y, bhi.y);
    wave_bounds(vs && !r.isB, r.vpos, r.vpos + vn, blo.z, bhi.z);
    wave_bounds(vs && r.isB, r.vpos, r.vpos + vn, blo.w, bhi.w);
    if ((tid & (kWave - 1)) == 0) {
      sh.wspan_lo[tid / kWave] = blo;
      sh.wspan_hi[tid / kWave] = bhi;
    }
  }
  if (!staged) {  // (uniform)
    if (ok)
      bp_write_record(payload, at, r, W, (r.isB ? B.keys : A.keys) + r.kpos, (r.isB ? B.vals : A.vals) + r.vpos);
    return;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t slo[4], shi[4];
    for (int q = 0; q < 4; ++q) {
      slo[q] = 0xFFFFFFFFu;
      shi[q] = 0;
    }
    for (int w = 0; w < kBpBlock / kWave; ++w) {
      const uint4 a = sh.wspan_lo[w], b = sh.wspan_hi[w];
      slo[0] = min(slo[0], a.x), slo[1] = min(slo[1], a.y), slo[2] = min(slo[2], a.z), slo[3] = min(slo[3], a.w);
      shi[0] = max(shi[0], b.x), shi[1] = max(shi[1], b.y), shi[2] = max(shi[2], b.z), shi[3] = max(shi[3], b.w);
    }
    uint32_t s_at = 0;
    for (int q = 0; q < 4; ++q) {
      sh.stage_at[q] = s_at;
      if (slo[q] < shi[q]) {
        // the copy reads up to 4 bytes past a span's last byte
        const uint32_t lo = slo[q] & ~15u, hi = (shi[q] + 4u + 15u) & ~15u;
        sh.span_lo[q] = lo;
        sh.span_hi[q] = hi;
        const uint8_t* base = q == 0 ? A.keys : q == 1 ? B.keys : q == 2 ? A.vals : B.vals;
        sh.src_at[q] = reinterpret_cast<uint64_t>(base) + lo - s_at;
        s_at += hi - lo;
      } else {
        sh.span_lo[q] = sh.span_hi[q] = 0;
        sh.src_at[q] = 0;  // (no staged byte maps to an empty span)
      }
    }
    sh.stage_at[4] = s_at;
  }
  __syncthreads();
  const bool src_staged = sh.stage_at[4] <= kBpStage;  // (uniform)
  if (src_staged && sh.stage_at[4] > 0) {
    // global -> LDS without registers: each wave moves 64 consecutive
    // 16-byte chunks, lane i's chunk landing 16 i bytes after the wave's base
    const uint32_t total16 = sh.stage_at[4] / 16;
    const uint32_t at1 = sh.stage_at[1], at2 = sh.stage_at[2], at3 = sh.stage_at[3];
    const uint32_t lane = tid & (kWave - 1);
    for (uint32_t c0 = (tid / kWave) * kWave; c0 < total16; c0 += kBpBlock) {
      const uint32_t c = c0 + lane;
      if (c < total16) {
        const uint32_t byte = c * 16;
        const uint32_t q = (byte >= at1) + (byte >= at2) + (byte >= at3);
        lds_dma16(reinterpret_cast<const uint8_t*>(sh.src_at[q] + byte), sh.stage + c0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();
  uint8_t* win = reinterpret_cast<uint8_t*>(sh.win);
  if (ok) {
    if (src_staged) {
      const uint8_t* st = reinterpret_cast<const uint8_t*>(sh.stage);
      const uint32_t qk = r.isB ? 1u : 0u, qv = 2u + qk;
      // (an empty field's source is never read)
      const uint8_t* ks = st + (r.sfx ? sh.stage_at[qk] + (r.kpos - sh.span_lo[qk]) : 0u);
      const uint8_t* vs = st + (vn ? sh.stage_at[qv] + (r.vpos - sh.span_lo[qv]) : 0u);
      bp_write_record(win, at - base, r, W, ks, vs);
    } else {
      bp_write_record(win, at - base, r, W, (r.isB ? B.keys : A.keys) + r.kpos,
                      (r.isB ? B.vals : A.vals) + r.vpos);
    }
  }
  __syncthreads();
  // 16-byte groups of the window, counted from `base`: [g_lo, g_hi) lie
  // whole inside [b0, b1) and are stored at once; the (at most two) groups
  // outside that range, which the workgroup shares with its neighbours, go
  // byte by byte
  const uint32_t groups = static_cast<uint32_t>((b1 - base + 15) >> 4);
  const uint32_t g_lo = static_cast<uint32_t>((b0 - base + 15) >> 4), g_hi = static_cast<uint32_t>((b1 - base) >> 4);
  uint4* const dst = reinterpret_cast<uint4*>(payload + base);
  for (uint32_t g = g_lo + tid; g < g_hi; g += kBpBlock) dst[g] = sh.win[g];
  if (tid < 2) {
    const uint32_t g = tid == 0 ? 0u : g_hi;
    if (g < groups && (g < g_lo || g >= g_hi) && !(tid == 1 && g == 0)) {
      const uint64_t a = base + 16ull * g;
      for (uint32_t t = 0; t < 16; ++t)
        if (a + t >= b0 && a + t < b1) payload[a + t] = win[16 * g + t];
    }
  }
}

static inline uint32_t bp_blocks(uint64_t n) { return static_cast<uint32_t>((n + kBpBlock - 1) / kBpBlock); }

}  // namespace em

using namespace em;

extern "C" size_t em_bp_workspace_bytes(uint32_t S) {
  (void)S;
  return 256;
}

extern "C" int em_bp_lengths(const em_side_t* A, const em_side_t* B, const uint32_t* final_refs,
                             const uint32_t* lcp_bits, uint32_t S, uint32_t* len_bytes, uint32_t* d_width, void* ws,
                             size_t ws_bytes, void* stream) {
  int rc = check_pair(A, B);
  if (rc) return rc;
  if (S > A->n + B->n) return EM_EINVAL;
  if (!d_width || !ws || (reinterpret_cast<uintptr_t>(ws) & 255)) return EM_EINVAL;
  if (S && (!final_refs || !lcp_bits || !len_bytes)) return EM_EINVAL;
  if (ws_bytes < em_bp_workspace_bytes(S)) return EM_ENOSPC;
  hipStream_t st = as_stream(stream);
  const BpWs L = bp_layout(ws);
  hipLaunchKernelGGL(k_bp_init, dim3(1), dim3(1), 0, st, L.stat);
  if (S)
    hipLaunchKernelGGL(k_bp_stats, dim3(min(bp_blocks(S), kBpWidthGrid)), dim3(kBpBlock), 0, st, *A, *B, final_refs,
                       S, L.stat);
  hipLaunchKernelGGL(k_bp_width, dim3(1), dim3(1), 0, st, L.stat, S, d_width);
  if (S)
    hipLaunchKernelGGL(k_bp_lengths, dim3(bp_blocks(S)), dim3(kBpBlock), 0, st, *A, *B, final_refs, lcp_bits, S,
                       d_width, len_bytes);
  return check_launch();
}

extern "C" int em_bp_emit(const em_side_t* A, const em_side_t* B, const uint32_t* final_refs,
                          const uint32_t* lcp_bits, uint32_t S, const uint64_t* off, uint64_t T,
                          const uint32_t* d_width, uint8_t* payload, uint64_t payload_cap, uint32_t* d_overflow,
                          void* stream) {
  int rc = check_pair(A, B);
  if (rc) return rc;
  if (S > A->n + B->n) return EM_EINVAL;
  if ((S == 0) != (T == 0)) return EM_EINVAL;
  if (!d_width || !d_overflow) return EM_EINVAL;
  if (S && (!final_refs || !lcp_bits || !off || !payload)) return EM_EINVAL;
  if (payload_cap < T) return EM_ENOSPC;
  hipStream_t st = as_stream(stream);
  clear_u32(d_overflow, 1, st);
  if (S) {
    // records per workgroup: the mean record filling two thirds of the window
    const uint64_t mean = (T + S - 1) / S;
    const uint32_t rpb = static_cast<uint32_t>(
        std::max<uint64_t>(16, std::min<uint64_t>(kBpBlock, (2 * kBpWin / 3) / std::max<uint64_t>(mean, 1))));
    const uint32_t grid = (S + rpb - 1) / rpb;
    hipLaunchKernelGGL(k_bp_emit, dim3(grid), dim3(kBpBlock), 0, st, *A, *B, final_refs, lcp_bits, S, rpb, off,
                       d_width, payload, payload_cap, d_overflow);
  }
  return check_launch();
}
