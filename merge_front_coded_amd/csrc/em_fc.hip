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
//  1. Per-record fields are loaded and turned into five bit segments per
//     record in LDS: the EG0 control field(s) as immediate bits, the key
//     suffix as a span of source bits, the presence bit and EG0(value length)
//     as immediate bits, and the value bytes as a span of source bits.
//  2. The records' source bytes lie in four contiguous arena spans (A keys,
//     B keys, A values, B values: survivors of one side are increasing).
//     They are staged into LDS with 16-byte loads when they fit; otherwise
//     this workgroup reads them from global memory.
//  3. Each thread assembles a contiguous run of output words, walking the
//     segments sequentially, into an LDS output window that is then stored
//     with consecutive lanes on consecutive words.  Every word is written once.

constexpr int kEmitBlock = 256;
constexpr uint32_t kEmitRecs = 128;
constexpr uint32_t kEmitExtra = 16;
constexpr uint32_t kEmitTable = kEmitRecs + kEmitExtra;
constexpr uint32_t kSegPerRec = 5;
constexpr uint32_t kEmitSegs = kEmitTable * kSegPerRec;
constexpr uint32_t kEmitWindow = 4096;     // output words assembled per round
constexpr uint32_t kEmitStage = 32 * 1024;  // bytes of staged source spans

// segment kinds: 0 immediate, 1 A keys, 2 B keys, 3 A values, 4 B values
struct EmitShared {
  uint64_t start[kEmitSegs];  // absolute first bit in the payload
  uint64_t data[kEmitSegs];   // immediate bits, or first source bit in its arena
  uint32_t len[kEmitSegs];    // bits
  uint32_t kind[kEmitSegs];
  uint32_t kbits[kEmitTable];
  uint32_t out[kEmitWindow];
  uint4 stage[kEmitStage / 16];
  uint32_t span_lo[4], span_hi[4];  // byte spans of the four sources (lo = ~0 when unused)
  uint32_t stage_at[5];             // LDS byte offset of each staged span, [4] = total
  uint32_t kprev0;
};

// 64 source bits starting at the dword holding bit `bitpos`, big-endian
__device__ __forceinline__ uint64_t window64(const uint32_t* w) {
  return (static_cast<uint64_t>(__builtin_bswap32(w[0])) << 32) | __builtin_bswap32(w[1]);
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
  if (tid < 4) {
    sh.span_lo[tid] = 0xFFFFFFFFu;
    sh.span_hi[tid] = 0;
  }
  __syncthreads();

  // ---- 1. per-record fields (one record per thread) ----
  const uint32_t j = tid;
  uint32_t r_kpos = 0, r_klen = 0, r_l = 0, r_vpos = 0, r_vlen = 0;
  bool r_isB = false, r_tomb = false;
  uint64_t r_off = 0;
  if (j < cnt) {
    const uint32_t r = R0 + j;
    uint32_t idx;
    const SideView s = pick(A, B, final_refs[r], idx);
    const KeyRef x = key_of(s, idx);
    if (lcp_in) {
      r_l = min(lcp_in[r], 8u * x.len);  // a stale array must not send reads past the key
    } else if (r > 0) {
      uint32_t pidx;
      const SideView ps = pick(A, B, final_refs[r - 1], pidx);
      r_l = lcp_bits(ps.keys, key_of(ps, pidx), s.keys, x);
    }
    uint32_t vlen;
    bool tomb;
    value_bits(s, idx, vlen, tomb);
    r_kpos = x.pos;
    r_klen = x.len;
    r_vpos = tomb ? 0u : s.val_off[idx];
    r_vlen = vlen;
    r_isB = s.isB;
    r_tomb = tomb;
    r_off = off[r];
    sh.kbits[j] = 8u * x.len;
    // source spans: the key bytes from the first emitted byte, the value bytes
    const uint32_t kk = r_isB ? 1u : 0u;
    const uint32_t klo = r_kpos + (r_l >> 3);
    if (klo < r_kpos + r_klen) {
      atomicMin(&sh.span_lo[kk], klo);
      atomicMax(&sh.span_hi[kk], r_kpos + r_klen);
    }
    if (r_vlen) {
      atomicMin(&sh.span_lo[2 + kk], r_vpos);
      atomicMax(&sh.span_hi[2 + kk], r_vpos + r_vlen);
    }
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

  // ---- segment table ----
  if (j < cnt) {
    const uint32_t r = R0 + j;
    const uint32_t k = 8u * r_klen, l = r_l;
    const uint32_t kprev = j ? sh.kbits[j - 1] : sh.kprev0;
    const uint32_t c = (r % 15u == 0) ? 1u + l : kprev - l;
    const uint32_t e1 = eg0_len(c), e2 = eg0_len(k - l);
    uint32_t len0, len1;
    uint64_t d0, d1;
    if (e1 + e2 <= 64) {  // EG0(c) EG0(k-l) as one immediate
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
    const uint32_t ev = eg0_len(r_vlen);
    const uint32_t lens[kSegPerRec] = {len0, len1, k - l, r_tomb ? 1u : 1u + ev, 8u * r_vlen};
    const uint64_t datas[kSegPerRec] = {
        d0, d1, 8ull * r_kpos + l,
        r_tomb ? 0ull : ((1ull << ev) | (static_cast<uint64_t>(r_vlen) + 1ull)), 8ull * r_vpos};
    const uint32_t kinds[kSegPerRec] = {0u, 0u, r_isB ? 2u : 1u, 0u, r_isB ? 4u : 3u};
    const uint32_t base = j * kSegPerRec;
    uint64_t at = r_off;
#pragma unroll
    for (uint32_t q = 0; q < kSegPerRec; ++q) {
      sh.start[base + q] = at;
      sh.len[base + q] = lens[q];
      sh.data[base + q] = datas[q];
      sh.kind[base + q] = kinds[q];
      at += lens[q];
    }
  }
  if (tid == 0) {
    uint32_t at = 0;
    for (int q = 0; q < 4; ++q) {
      sh.stage_at[q] = at;
      if (sh.span_lo[q] < sh.span_hi[q]) {
        const uint32_t lo = sh.span_lo[q] & ~15u;
        // a 64-bit window read at the last byte reaches at most 7 bytes past it
        const uint32_t hi = (sh.span_hi[q] + 8u + 15u) & ~15u;
        sh.span_lo[q] = lo;
        sh.span_hi[q] = hi;
        at += hi - lo;
      } else {
        sh.span_lo[q] = 0;
        sh.span_hi[q] = 0;
      }
    }
    sh.stage_at[4] = at;
  }
  __syncthreads();

  // ---- 2. stage the source spans ----
  const bool staged = sh.stage_at[4] <= kEmitStage;
  if (staged) {
    const uint32_t total16 = sh.stage_at[4] / 16;
    for (uint32_t c = tid; c < total16; c += kEmitBlock) {
      const uint32_t byte = c * 16;
      uint32_t q = 0;
      while (q < 3 && byte >= sh.stage_at[q + 1]) ++q;
      const uint8_t* base = q == 0 ? A.keys : q == 1 ? B.keys : q == 2 ? A.vals : B.vals;
      const uint32_t src = sh.span_lo[q] + (byte - sh.stage_at[q]);
      sh.stage[c] = *reinterpret_cast<const uint4*>(base + src);
    }
  }
  __syncthreads();

  // ---- 3. assemble the owned words ----
  const uint32_t nseg = cnt * kSegPerRec;
  const uint32_t nown_seg = nown * kSegPerRec;
  const uint64_t w_end = (T + 31) >> 5;
  const uint64_t bit_lo = sh.start[0];
  const uint64_t bit_hi = nown < cnt ? sh.start[nown_seg] : sh.start[nseg - 1] + sh.len[nseg - 1];
  const uint64_t w_lo = (bit_lo + 31) >> 5;
  const uint64_t w_hi = min((bit_hi + 31) >> 5, w_end);
  const uint32_t* stage32 = reinterpret_cast<const uint32_t*>(sh.stage);

  for (uint64_t win = w_lo; win < w_hi; win += kEmitWindow) {
    const uint32_t nw = static_cast<uint32_t>(min(static_cast<uint64_t>(kEmitWindow), w_hi - win));
    const uint32_t per = (nw + kEmitBlock - 1) / kEmitBlock;
    const uint32_t x0 = tid * per;
    const uint32_t x1 = min(x0 + per, nw);
    if (x0 < x1) {
      uint64_t pos = (win + x0) << 5;
      // segment holding `pos`: the last one starting at or before it
      uint32_t lo = 0, hi = nseg - 1;
      while (lo < hi) {
        const uint32_t mid = (lo + hi + 1) >> 1;
        if (sh.start[mid] <= pos)
          lo = mid;
        else
          hi = mid - 1;
      }
      uint32_t si = lo;
      for (uint32_t x = x0; x < x1; ++x) {
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
            const uint64_t bp = d + rel;  // absolute bit in the arena
            uint64_t wv;
            if (staged) {
              const uint32_t q = kind - 1;
              const uint64_t lb = bp - 8ull * sh.span_lo[q] + 8ull * sh.stage_at[q];
              wv = window64(stage32 + (lb >> 5));
            } else {
              const uint8_t* base = kind == 1 ? A.keys : kind == 2 ? B.keys : kind == 3 ? A.vals : B.vals;
              wv = window64(reinterpret_cast<const uint32_t*>(base) + (bp >> 5));
            }
            bits = static_cast<uint32_t>((wv << (bp & 31)) >> (64 - n));
          }
          acc = (acc << n) | bits;
          need -= n;
          pos += n;
        }
        sh.out[x] = __builtin_bswap32(static_cast<uint32_t>(acc));
      }
    }
    __syncthreads();
    for (uint32_t x = tid; x < nw; x += kEmitBlock) payload[win + x] = sh.out[x];
    __syncthreads();
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
