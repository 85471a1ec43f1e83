// Front coding of the survivors: exact record lengths and the word-owned
// payload emitter.
//
// Everett, "GPU construction experiment":
//  * the control equation: c_i = 1 + l_i when i mod 15 = 0, else
//    k_{i-1} - l_i, with l_i the exact bit LCP with the preceding survivor
//    (l_0 = 0) and k_i the key length in bits;
//  * the record grammar: EG0(c_i), EG0(k_i - l_i), the remaining key bits and
//    the value (0 for a tombstone; 1, EG0(byte length) and the bytes
//    otherwise); E(x) = 2 floor(log2(x+1)) + 1; MSB-first bits; no padding;
//  * emission: one invocation owns each final 32-bit word, gathers its bits
//    and writes it once; unused final bits are zero; the key suffix is copied
//    from the selected record's own key (every distinct key survives, so the
//    merged predecessor shares at least the source predecessor's prefix).
#include "em_internal.h"

namespace em {

constexpr int kLenBlock = 256;

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

__device__ __forceinline__ uint32_t value_bits(const SideView& s, uint32_t idx, uint32_t& vlen,
                                               bool& tomb) {
  tomb = s.tomb != nullptr && s.tomb[idx] != 0;
  vlen = tomb ? 0u : s.val_off[idx + 1] - s.val_off[idx];
  return tomb ? 1u : 1u + eg0_len(vlen) + 8u * vlen;
}

__global__ __launch_bounds__(kLenBlock) void k_fc_lengths(em_side_t A, em_side_t B,
                                                          const uint32_t* __restrict__ final_refs,
                                                          uint32_t S, uint32_t* __restrict__ len_bits,
                                                          uint32_t* __restrict__ lcp_out) {
  const uint32_t i = blockIdx.x * kLenBlock + threadIdx.x;
  if (i >= S) return;
  uint32_t idx;
  const SideView s = pick(A, B, final_refs[i], idx);
  const KeyRef x = key_of(s, idx);
  const uint32_t k = 8u * x.len;
  uint32_t l = 0, kprev = 0;
  if (i > 0) {
    uint32_t pidx;
    const SideView ps = pick(A, B, final_refs[i - 1], pidx);
    const KeyRef p = key_of(ps, pidx);
    kprev = 8u * p.len;
    l = lcp_bits(ps.keys, p, s.keys, x);
  }
  const uint32_t c = (i % 15u == 0) ? 1u + l : kprev - l;
  uint32_t vlen;
  bool tomb;
  const uint32_t v = value_bits(s, idx, vlen, tomb);
  len_bits[i] = eg0_len(c) + eg0_len(k - l) + (k - l) + v;
  if (lcp_out) lcp_out[i] = l;
}

// ---------------------------------------------------------------------------
// Emitter.  A workgroup owns kEmitRecs consecutive records and every payload
// word whose first bit lies inside them; the last such word may continue into
// up to kEmitExtra following records (each record is at least 3 bits long:
// one bit for each EG0 field when its argument is 0, one value bit).
//
// The workgroup first turns its records into a table of bit segments in LDS,
// five per record: the EG0 control field(s) as immediate bits, the key suffix
// as a span of source bits, the presence bit and EG0(value length) as
// immediate bits, and the value bytes as a span of source bits.  A map from
// each owned word to the segment holding its first bit follows.  Each thread
// then assembles whole 32-bit words: a map read, and per segment piece either
// a shift of an immediate or two aligned dword loads and a funnel shift.

constexpr int kEmitBlock = 256;
constexpr uint32_t kEmitRecs = 256;
constexpr uint32_t kEmitExtra = 16;
constexpr uint32_t kEmitTable = kEmitRecs + kEmitExtra;
constexpr uint32_t kSegPerRec = 5;
constexpr uint32_t kEmitSegs = kEmitTable * kSegPerRec;
constexpr uint32_t kEmitMapWords = 8192;
constexpr uint32_t kRecPerThread = (kEmitTable + kEmitBlock - 1) / kEmitBlock;

// segment kinds: 0 immediate, 1 A keys, 2 B keys, 3 A values, 4 B values
struct EmitShared {
  uint64_t start[kEmitSegs];  // absolute first bit in the payload
  uint64_t data[kEmitSegs];   // immediate bits, or first source bit in its arena
  uint32_t len[kEmitSegs];    // bits
  uint32_t kind[kEmitSegs];
  uint16_t map[kEmitMapWords];
  uint32_t kbits[kEmitTable];
  uint32_t kprev0;
};

__device__ __forceinline__ uint32_t source_bits(const uint8_t* base, uint64_t bitpos, uint32_t n) {
  // n (1..32) bits of an arena's MSB-first bit stream starting at bitpos
  const uint32_t* w = reinterpret_cast<const uint32_t*>(base) + (bitpos >> 5);
  const uint64_t x = (static_cast<uint64_t>(__builtin_bswap32(w[0])) << 32) | __builtin_bswap32(w[1]);
  return static_cast<uint32_t>((x << (bitpos & 31)) >> (64 - n));
}

__global__ __launch_bounds__(kEmitBlock) void k_emit(em_side_t A, em_side_t B,
                                                     const uint32_t* __restrict__ final_refs,
                                                     const uint32_t* __restrict__ lcp_in, uint32_t S,
                                                     const uint64_t* __restrict__ off, uint64_t T,
                                                     uint32_t* __restrict__ payload) {
  __shared__ EmitShared sh;
  const uint32_t tid = threadIdx.x;
  const uint32_t R0 = blockIdx.x * kEmitRecs;
  const uint32_t nown = (S - R0) < kEmitRecs ? S - R0 : kEmitRecs;
  const uint32_t cnt = (S - R0) < kEmitTable ? S - R0 : kEmitTable;

  // phase 1: per-record fields (thread t takes records t and t + 256)
  uint32_t r_kpos[kRecPerThread], r_l[kRecPerThread], r_vpos[kRecPerThread], r_vlen[kRecPerThread];
  uint32_t r_info[kRecPerThread];
  uint64_t r_off[kRecPerThread];
#pragma unroll
  for (uint32_t u = 0; u < kRecPerThread; ++u) {
    const uint32_t j = tid + u * kEmitBlock;
    if (j >= cnt) continue;
    const uint32_t r = R0 + j;
    uint32_t idx;
    const SideView s = pick(A, B, final_refs[r], idx);
    const KeyRef x = key_of(s, idx);
    uint32_t l;
    if (lcp_in) {
      l = min(lcp_in[r], 8u * x.len);  // a stale array must not send reads past the key
    } else if (r == 0) {
      l = 0;
    } else {
      uint32_t pidx;
      const SideView ps = pick(A, B, final_refs[r - 1], pidx);
      l = lcp_bits(ps.keys, key_of(ps, pidx), s.keys, x);
    }
    uint32_t vlen;
    bool tomb;
    value_bits(s, idx, vlen, tomb);
    r_kpos[u] = x.pos;
    r_l[u] = l;
    r_vpos[u] = tomb ? 0u : s.val_off[idx];
    r_vlen[u] = vlen;
    r_info[u] = (s.isB ? 1u : 0u) | (tomb ? 2u : 0u);
    r_off[u] = off[r];
    sh.kbits[j] = 8u * x.len;
  }
  if (tid == 0) {
    uint32_t kp = 0;
    if (R0 > 0) {
      uint32_t pidx;
      const SideView ps = pick(A, B, final_refs[R0 - 1], pidx);
      kp = 8u * (ps.key_off[pidx + 1] - ps.key_off[pidx]);
    }
    sh.kprev0 = kp;
  }
  __syncthreads();

  // phase 2: controls and the segment table
#pragma unroll
  for (uint32_t u = 0; u < kRecPerThread; ++u) {
    const uint32_t j = tid + u * kEmitBlock;
    if (j >= cnt) continue;
    const uint32_t r = R0 + j;
    const uint32_t k = sh.kbits[j], l = r_l[u];
    const uint32_t kprev = j ? sh.kbits[j - 1] : sh.kprev0;
    const uint32_t c = (r % 15u == 0) ? 1u + l : kprev - l;
    const uint32_t e1 = eg0_len(c), e2 = eg0_len(k - l);
    const bool isB = r_info[u] & 1u, tomb = r_info[u] & 2u;
    const uint32_t base = j * kSegPerRec;
    uint64_t at = r_off[u];
    // EG0(c) EG0(k-l): one immediate when both fit in 64 bits
    uint32_t len0, len1;
    uint64_t d0, d1;
    if (e1 + e2 <= 64) {
      len0 = e1 + e2;
      d0 = (static_cast<uint64_t>(c + 1u) << e2) | (k - l + 1u);
      len1 = 0;
      d1 = 0;
    } else {
      len0 = e1;
      d0 = c + 1u;
      len1 = e2;
      d1 = k - l + 1u;
    }
    const uint32_t ev = eg0_len(r_vlen[u]);
    const uint32_t lens[kSegPerRec] = {len0, len1, k - l, tomb ? 1u : 1u + ev, 8u * r_vlen[u]};
    const uint64_t datas[kSegPerRec] = {
        d0, d1, 8ull * r_kpos[u] + l,
        tomb ? 0ull : ((1ull << ev) | (static_cast<uint64_t>(r_vlen[u]) + 1ull)), 8ull * r_vpos[u]};
    const uint32_t kinds[kSegPerRec] = {0u, 0u, isB ? 2u : 1u, 0u, isB ? 4u : 3u};
#pragma unroll
    for (uint32_t q = 0; q < kSegPerRec; ++q) {
      sh.start[base + q] = at;
      sh.len[base + q] = lens[q];
      sh.data[base + q] = datas[q];
      sh.kind[base + q] = kinds[q];
      at += lens[q];
    }
  }
  const uint32_t nseg = cnt * kSegPerRec;
  const uint32_t nown_seg = nown * kSegPerRec;
  __syncthreads();

  // phase 3: map each owned word to the segment holding its first bit
  const uint64_t w_end = (T + 31) >> 5;
  const uint64_t bit_lo = sh.start[0];
  const uint64_t bit_hi = nown < cnt ? sh.start[nown_seg] : sh.start[nseg - 1] + sh.len[nseg - 1];
  const uint64_t w_lo = (bit_lo + 31) >> 5;
  const uint64_t w_hi = min((bit_hi + 31) >> 5, w_end);
  const bool use_map = w_hi > w_lo && (w_hi - w_lo) <= kEmitMapWords;
  if (use_map) {
    for (uint32_t q = tid; q < nown_seg; q += kEmitBlock) {
      const uint32_t ln = sh.len[q];
      if (!ln) continue;
      const uint64_t st = sh.start[q];
      const uint64_t a = (st + 31) >> 5, b = min((st + ln + 31) >> 5, w_hi);
      for (uint64_t w = a; w < b; ++w) sh.map[w - w_lo] = static_cast<uint16_t>(q);
    }
  }
  __syncthreads();

  // phase 4: assemble and store every owned word once
  for (uint64_t w = w_lo + tid; w < w_hi; w += kEmitBlock) {
    uint64_t pos = w << 5;
    uint32_t si;
    if (use_map) {
      si = sh.map[w - w_lo];
    } else {
      uint32_t lo = 0, hi = nown_seg - 1;
      while (lo < hi) {
        const uint32_t mid = (lo + hi + 1) >> 1;
        if (sh.start[mid] <= pos)
          lo = mid;
        else
          hi = mid - 1;
      }
      si = lo;
    }
    uint64_t acc = 0;
    uint32_t need = 32;
    while (need) {
      if (pos >= T) {
        acc <<= need;
        break;
      }
      while (si + 1 < nseg && pos >= sh.start[si] + sh.len[si]) ++si;
      const uint64_t st = sh.start[si];
      const uint32_t ln = sh.len[si];
      if (pos >= st + ln) {  // cannot happen for offsets produced by em_scan
        acc <<= need;
        break;
      }
      const uint32_t rel = static_cast<uint32_t>(pos - st);
      const uint32_t n = min(need, ln - rel);
      const uint32_t kind = sh.kind[si];
      const uint64_t d = sh.data[si];
      uint32_t bits;
      if (kind == 0) {
        bits = static_cast<uint32_t>((d >> (ln - rel - n)) & ((1ull << n) - 1));
      } else {
        const uint8_t* base = kind == 1 ? A.keys : kind == 2 ? B.keys : kind == 3 ? A.vals : B.vals;
        bits = source_bits(base, d + rel, n);
      }
      acc = (acc << n) | bits;
      need -= n;
      pos += n;
    }
    payload[w] = __builtin_bswap32(static_cast<uint32_t>(acc));
  }
}

}  // namespace em

using namespace em;

extern "C" int em_fc_lengths(const em_side_t* A, const em_side_t* B, const uint32_t* final_refs,
                             uint32_t S, uint32_t* len_bits, uint32_t* lcp_bits, void* ws,
                             size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  int rc = check_pair(A, B);
  if (rc) return rc;
  if (S > A->n + B->n) return EM_EINVAL;
  if (S == 0) return EM_OK;
  if (!final_refs || !len_bits) return EM_EINVAL;
  const uint32_t blocks = (S + kLenBlock - 1) / kLenBlock;
  hipLaunchKernelGGL(k_fc_lengths, dim3(blocks), dim3(kLenBlock), 0, as_stream(stream), *A, *B,
                     final_refs, S, len_bits, lcp_bits);
  return check_launch();
}

extern "C" int em_emit(const em_side_t* A, const em_side_t* B, const uint32_t* final_refs,
                       const uint32_t* lcp_bits, uint32_t S, const uint64_t* off, uint64_t T,
                       uint32_t* payload, uint64_t payload_words, void* ws, size_t ws_bytes,
                       void* stream) {
  (void)ws;
  (void)ws_bytes;
  int rc = check_pair(A, B);
  if (rc) return rc;
  if (S > A->n + B->n) return EM_EINVAL;
  if ((S == 0) != (T == 0)) return EM_EINVAL;
  if (S == 0) return EM_OK;
  if (!final_refs || !off || !payload) return EM_EINVAL;
  if (payload_words < (T + 31) / 32) return EM_ENOSPC;
  const uint32_t blocks = (S + kEmitRecs - 1) / kEmitRecs;
  hipLaunchKernelGGL(k_emit, dim3(blocks), dim3(kEmitBlock), 0, as_stream(stream), *A, *B,
                     final_refs, lcp_bits, S, off, T, payload);
  return check_launch();
}
