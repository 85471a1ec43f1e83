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

constexpr int kEmitBlock = 256;
constexpr uint32_t kEmitRecs = 256;
constexpr uint32_t kEmitExtra = 16;
constexpr uint32_t kEmitTable = kEmitRecs + kEmitExtra;

struct EmitShared {
  uint64_t off[kEmitTable + 1];  // record start bits; off[cnt] = end of the last
  uint32_t c1[kEmitTable];       // c + 1 (the EG0 field value)
  uint32_t s1[kEmitTable];       // k - l + 1
  uint32_t kpos[kEmitTable];     // key byte offset in its arena
  uint32_t l[kEmitTable];        // first emitted key bit
  uint32_t klen[kEmitTable];     // k - l (bits); holds k until the controls are formed
  uint32_t vpos[kEmitTable];     // value byte offset
  uint32_t vlen[kEmitTable];     // value bytes (0 for a tombstone)
  uint32_t info[kEmitTable];     // E(c) | E(k-l) << 8 | E(vlen) << 16 | side B << 24 | tomb << 25
  uint32_t kprev0;
};

__device__ __forceinline__ uint32_t field_bits(uint64_t v, uint32_t e, uint32_t o, uint32_t n) {
  // n bits of the e-bit field v starting o bits after its most significant bit
  return static_cast<uint32_t>((v >> (e - o - n)) & ((1ull << n) - 1));
}

__device__ __forceinline__ uint32_t stream_bits(const uint8_t* base, uint32_t pos, uint32_t bit,
                                                uint32_t n) {
  // n (<= 32) bits of the byte string at `pos`, starting at bit `bit`
  const uint64_t w = load_be8(base, pos + (bit >> 3));
  return static_cast<uint32_t>((w << (bit & 7)) >> (64 - n));
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

  // phase 1: per-record fields that need no neighbour
  for (uint32_t j = tid; j < cnt; j += kEmitBlock) {
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
    sh.off[j] = off[r];
    sh.kpos[j] = x.pos;
    sh.l[j] = l;
    sh.klen[j] = 8u * x.len;
    sh.vpos[j] = tomb ? 0u : s.val_off[idx];
    sh.vlen[j] = vlen;
    sh.info[j] = (s.isB ? 1u << 24 : 0u) | (tomb ? 1u << 25 : 0u);
  }
  if (tid == 0) {
    sh.off[cnt] = off[R0 + cnt];
    uint32_t kp = 0;
    if (R0 > 0) {
      uint32_t pidx;
      const SideView ps = pick(A, B, final_refs[R0 - 1], pidx);
      kp = 8u * (ps.key_off[pidx + 1] - ps.key_off[pidx]);
    }
    sh.kprev0 = kp;
  }
  __syncthreads();
  // phase 2: the controls need the predecessor's key length
  uint32_t c_[2], k_[2];
  for (uint32_t j = tid, u = 0; j < cnt; j += kEmitBlock, ++u) {
    const uint32_t kprev = j ? sh.klen[j - 1] : sh.kprev0;
    const uint32_t r = R0 + j;
    c_[u] = (r % 15u == 0) ? 1u + sh.l[j] : kprev - sh.l[j];
    k_[u] = sh.klen[j];
  }
  __syncthreads();
  for (uint32_t j = tid, u = 0; j < cnt; j += kEmitBlock, ++u) {
    const uint32_t c = c_[u], k = k_[u], l = sh.l[j];
    sh.c1[j] = c + 1u;
    sh.s1[j] = k - l + 1u;
    sh.klen[j] = k - l;
    sh.info[j] |= eg0_len(c) | (eg0_len(k - l) << 8) | (eg0_len(sh.vlen[j]) << 16);
  }
  __syncthreads();

  // phase 3: every word whose first bit lies in this block's own records
  const uint64_t bit_lo = sh.off[0];
  const uint64_t bit_hi = sh.off[nown];
  const uint64_t w_lo = (bit_lo + 31) >> 5;
  const uint64_t w_end = (T + 31) >> 5;
  const uint64_t w_hi = min((bit_hi + 31) >> 5, w_end);
  for (uint64_t w = w_lo + tid; w < w_hi; w += kEmitBlock) {
    uint64_t pos = w << 5;
    // last own record starting at or before pos
    uint32_t lo = 0, hi = nown - 1;
    while (lo < hi) {
      const uint32_t mid = (lo + hi + 1) >> 1;
      if (sh.off[mid] <= pos)
        lo = mid;
      else
        hi = mid - 1;
    }
    uint32_t j = lo;
    uint64_t acc = 0;
    uint32_t need = 32;
    while (need) {
      if (pos >= T) {
        acc <<= need;
        break;
      }
      while (j + 1 < cnt && pos >= sh.off[j + 1]) ++j;
      const uint32_t info = sh.info[j];
      const uint32_t e1 = info & 0xFF, e2 = (info >> 8) & 0xFF, ev = (info >> 16) & 0xFF;
      const bool tomb = (info >> 25) & 1u;
      const uint32_t rel = static_cast<uint32_t>(pos - sh.off[j]);
      const uint32_t b1 = e1, b2 = b1 + e2, b3 = b2 + sh.klen[j];
      const uint32_t b4 = b3 + (tomb ? 1u : 1u + ev);
      uint32_t n, bits;
      if (rel < b1) {
        n = min(need, b1 - rel);
        bits = field_bits(sh.c1[j], e1, rel, n);
      } else if (rel < b2) {
        n = min(need, b2 - rel);
        bits = field_bits(sh.s1[j], e2, rel - b1, n);
      } else if (rel < b3) {
        n = min(need, b3 - rel);
        const uint8_t* keys = (info >> 24) & 1u ? B.keys : A.keys;
        bits = stream_bits(keys, sh.kpos[j], sh.l[j] + (rel - b2), n);
      } else if (rel < b4) {
        n = min(need, b4 - rel);
        // presence bit then EG0(vlen): the field value is 2^ev + vlen + 1 over 1 + ev bits
        const uint64_t vh = tomb ? 0ull : ((1ull << ev) | (static_cast<uint64_t>(sh.vlen[j]) + 1ull));
        bits = field_bits(vh, b4 - b3, rel - b3, n);
      } else {
        const uint32_t b5 = b4 + 8u * sh.vlen[j];
        if (rel >= b5) {  // cannot happen for offsets produced by em_scan
          acc <<= need;
          break;
        }
        n = min(need, b5 - rel);
        const uint8_t* vals = (info >> 24) & 1u ? B.vals : A.vals;
        bits = stream_bits(vals, sh.vpos[j], rel - b4, n);
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
