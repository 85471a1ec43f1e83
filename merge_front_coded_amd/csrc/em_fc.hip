// Front coding of the survivors: exact record lengths and the word-owned
// payload emitter.
//
// Everett, "GPU construction experiment":
//  * the control equation: c_i = 1 + l_i when i mod 15 = 0, else
//    k_{i-1} - l_i, where l_i counts the leading bits survivor i shares with
//    survivor i - 1 (l_0 = 0) and k_i is the key length in bits;
//  * the record grammar: EG0(c_i), EG0(k_i - l_i), key bits l_i .. k_i - 1,
//    then the value (0 for a tombstone; 1, EG0(byte length) and the bytes
//    otherwise); E(x) = 2 floor(log2(x+1)) + 1; most significant bit first;
//    records back to back;
//  * emission: every 32-bit output word has one writer, which collects its
//    bits and stores it once; the tail after the last record is zero; the key
//    suffix comes from the source record's own key (every distinct key survives, so the
//    merged predecessor shares at least the source predecessor's prefix).
#include "em_tile.h"

namespace em {

constexpr int kLenBlock = 256;

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
// Emitter.  A workgroup takes `rpb` consecutive records and owns every payload
// word whose first bit lies inside them; the last such word may continue into
// up to kEmitExtra following records (each record is at least 3 bits long:
// one bit for each EG0 field when its argument is 0, one value bit), which the
// workgroup also encodes.  Steps:
//  1. one thread per record loads its fields; the records' source bytes lie in
//     four contiguous arena spans (A keys, B keys, A values, B values, since
//     the survivors of one side are increasing), which are staged into LDS
//     with 16-byte loads when they fit (otherwise read from global memory);
//  2. each thread appends its record's bits -- EG0(c), EG0(k-l), the key
//     suffix, the presence bit and EG0(value length), the value bytes -- to an
//     LDS window of output words: words holding only its own bits are plain
//     stores, the two boundary words it shares with its neighbours are ORed;
//  3. the owned words are copied from the window to the payload with
//     consecutive lanes on consecutive words, each word written once.
// A window that would overflow LDS is processed in slices; each thread then
// clips its record to the slice.

constexpr int kEmitBlock = 256;
constexpr uint32_t kEmitExtra = 16;
constexpr uint32_t kEmitMaxRecs = kEmitBlock - kEmitExtra;  // owned records per workgroup, at most
// LDS per workgroup is kept small (about 25 KB) so that six workgroups share
// a compute unit: the emitter waits on three dependent global loads per
// workgroup (records, their offsets, the source spans), and more workgroups
// in flight hide them better than larger ones.
constexpr uint32_t kEmitWindow = 2560;      // output words per slice (10 KB)
constexpr uint32_t kEmitStage = 14 * 1024;  // staged source bytes

struct EmitShared {
  uint32_t out[kEmitWindow];
  uint4 stage[kEmitStage / 16];
  uint32_t kbits[kEmitBlock];
  uint32_t span_lo[4], span_hi[4];  // byte spans of the four sources
  uint4 wspan_lo[kEmitBlock / kWave], wspan_hi[kEmitBlock / kWave];  // each wave's bounds of the four
  uint32_t stage_at[5];             // LDS byte offset of each staged span, [4] = total
  uint64_t src_at[4];               // global address of each staged span's first byte, less stage_at
  uint32_t kprev0;
  uint32_t next;  // the workgroup's next chunk ticket
  uint64_t bit_lo, bit_hi, bit_ext;
};
// The span copy reads a staged source up to four dwords past the last dword
// a span needs; the array after the stage keeps such reads inside the
// workgroup's LDS.
static_assert(offsetof(EmitShared, kbits) == offsetof(EmitShared, stage) + sizeof(EmitShared::stage) &&
                  sizeof(EmitShared::kbits) >= 16,
              "the stage is followed by at least 16 bytes of the same allocation");

// One record's fields for the slice loop; segment ends are relative to the
// record start, kbit/vbit are the source bit positions of the key suffix and
// the value bytes.
struct EmitRecord {
  bool live;
  uint64_t off, end;
  uint32_t c, k, l;
  uint64_t vh;
  uint32_t b1, b2, b3, b4, b5;
  uint64_t kbit, vbit;
};

// Steps 2 and 3 for the workgroup: the records' bits go into the LDS window
// slice by slice, and each slice's owned words are copied out.  Thread 0
// publishes `ticket` in sh.next before the first copy-out (it waits for the
// ticket's atomic there, after the window is built).
template <typename Pos>  // source bit positions: uint32_t for staged sources (LDS), uint64_t otherwise
__device__ __forceinline__ void emit_slices(EmitShared& sh, const EmitRecord& r, const uint32_t* kbase,
                                            const uint32_t* vbase, uint64_t T, uint32_t* payload,
                                            uint32_t ticket) {
  const uint32_t tid = threadIdx.x;
  // first bit of window word 0: a multiple of 128 bits, so that four-word
  // groups of the payload are four-word groups of the window
  const uint64_t wb = (sh.bit_lo >> 7) << 7;
  const uint64_t w_lo = (sh.bit_lo + 31) >> 5;         // first owned word
  const uint64_t w_hi = min_u64((sh.bit_hi + 31) >> 5, (T + 31) >> 5);
  // bits past the last owned word are not needed
  const uint64_t ext = min_u64(sh.bit_ext, 32ull * w_hi);
  for (uint64_t s0 = wb; s0 < ext && (s0 >> 5) < w_hi; s0 += 32ull * kEmitWindow) {
    const uint64_t s1 = min_u64(s0 + 32ull * kEmitWindow, ext);
    if (s0 != wb) {  // (the window arrives zeroed for the first slice)
      const uint32_t used4 = static_cast<uint32_t>(((s1 - s0 + 31) / 32 + 3) / 4);
      for (uint32_t i = tid; i < used4; i += kEmitBlock) reinterpret_cast<uint4*>(sh.out)[i] = uint4{0, 0, 0, 0};
      __syncthreads();
    }
    if (r.live && r.off < s1 && r.end > s0) {
      // this record's bits inside [s0, s1), relative to the record start
      const uint32_t from = r.off >= s0 ? 0u : static_cast<uint32_t>(s0 - r.off);
      const uint32_t to = r.end <= s1 ? r.b5 : static_cast<uint32_t>(s1 - r.off);
      // Each field, clipped to the slice, goes straight to its own position
      // in the window: EG0(c) EG0(k-l) (one 64-bit field when they fit), the
      // key suffix, presence + EG0(value length), the value bytes.
      const uint32_t p0 = static_cast<uint32_t>(r.off + from - s0);  // window bit of record bit `from`
      auto imm = [&](uint64_t v, uint32_t a, uint32_t b) {  // field of b - a <= 64 bits at [a, b)
        const uint32_t lo = max(a, from), hi = min(b, to);
        if (lo < hi) {
          const uint64_t x = (v >> (b - hi)) & (hi - lo == 64u ? ~0ull : ((1ull << (hi - lo)) - 1ull));
          if (x) or_bits64(sh.out, p0 + (lo - from), x, hi - lo);
        }
      };
      auto span = [&](const uint32_t* base, uint64_t bp, uint32_t a, uint32_t b) {
        const uint32_t lo = max(a, from), hi = min(b, to);
        if (lo < hi) or_span<Pos>(sh.out, p0 + (lo - from), base, static_cast<Pos>(bp) + (lo - a), hi - lo);
      };
      if (r.b2 <= 64u) {
        imm((static_cast<uint64_t>(r.c) + 1u) << (r.b2 - r.b1) | (static_cast<uint64_t>(r.k - r.l) + 1u), 0, r.b2);
      } else {
        imm(static_cast<uint64_t>(r.c) + 1u, 0, r.b1);
        imm(static_cast<uint64_t>(r.k - r.l) + 1u, r.b1, r.b2);
      }
      span(kbase, r.kbit, r.b2, r.b3);
      imm(r.vh, r.b3, r.b4);
      span(vbase, r.vbit, r.b4, r.b5);
    }
    if (s0 == wb && tid == 0) sh.next = ticket;
    __syncthreads();
    // owned words of this slice: 16-byte stores between a scalar head and
    // tail; indices are relative to window word 0 (payload word s0 / 32, a
    // multiple of four)
    const uint64_t wbase = s0 >> 5;
    uint32_t* const dst = payload + wbase;
    const uint32_t o_lo = static_cast<uint32_t>(max_u64(w_lo, wbase) - wbase);
    const uint32_t o_hi = static_cast<uint32_t>(min_u64(w_hi, (s1 + 31) >> 5) - wbase);
    const uint32_t a_lo = min((o_lo + 3u) & ~3u, o_hi), a_hi = max(o_hi & ~3u, a_lo);
    for (uint32_t i = o_lo + tid; i < a_lo; i += kEmitBlock) dst[i] = __builtin_bswap32(sh.out[i]);
    // (non-temporal: the payload is written once and not read back here;
    // streaming it past the caches measured 2% faster than plain stores)
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    for (uint32_t i = a_lo + 4 * tid; i < a_hi; i += 4 * kEmitBlock) {
      const uint4 v = reinterpret_cast<const uint4*>(sh.out)[i / 4];
      const u32x4 q = {__builtin_bswap32(v.x), __builtin_bswap32(v.y), __builtin_bswap32(v.z), __builtin_bswap32(v.w)};
      __builtin_nontemporal_store(q, reinterpret_cast<u32x4*>(dst + i));
    }
    for (uint32_t i = a_hi + tid; i < o_hi; i += kEmitBlock) dst[i] = __builtin_bswap32(sh.out[i]);
    __syncthreads();
  }
  if (!(wb < ext && (wb >> 5) < w_hi)) {  // no slice (offsets that leave the chunk no bits)
    if (tid == 0) sh.next = ticket;
    __syncthreads();
  }
}

// Record offsets: off[r] directly (kTiled = false), or a partition number
// above bit kTiledShift plus a partition-local offset, to which the
// partition's bit base tbase[] is added (kTiled = true; off_out, when given,
// then receives the offsets of the owned records and T).

// The first loads of a thread's record: its reference, the offsets of its
// start and end, its LCP (and, for thread 0, the record before the chunk).
struct RecPre {
  uint32_t ref, lcp;
  uint64_t o0, o1;
  uint32_t pref;  // thread 0: the reference of the record before the chunk
};

template <bool kTiled, bool kLcp>
__device__ __forceinline__ RecPre load_rec_pre(const uint32_t* __restrict__ final_refs,
                                               const uint32_t* __restrict__ lcp_in,
                                               const uint64_t* __restrict__ off, uint32_t S, uint32_t R0,
                                               uint32_t rpb) {
  RecPre p{0, 0, 0, 0, 0};
  const uint32_t j = threadIdx.x;
  if (j == 0 && R0 > 0 && R0 < S) p.pref = final_refs[R0 - 1];
  const uint32_t cnt = (S - R0) < rpb + kEmitExtra ? S - R0 : rpb + kEmitExtra;
  if (R0 < S && j < cnt) {
    const uint32_t r = R0 + j;
    p.ref = final_refs[r];
    p.o0 = off[r];
    // partition-form offsets have no entry S: the last record reads entry
    // S-1 again (both loads are issued before either is waited for)
    const uint64_t o1 = off[kTiled && r + 1 == S ? r : r + 1];
    p.o1 = o1;
    p.lcp = kLcp ? lcp_in[r] : 0u;
  }
  return p;
}

// One workgroup's records [R0, R0 + rpb) (and up to kEmitExtra after them).
// kLcp: LCPs come from lcp_in (else they are recomputed from the keys).
template <bool kTiled, bool kLcp>
__device__ __forceinline__ void emit_chunk(EmitShared& sh, const em_side_t& A, const em_side_t& B,
                                           const uint32_t* __restrict__ final_refs,
                                           const uint32_t* __restrict__ lcp_in, uint32_t S,
                                           const uint64_t* __restrict__ off,
                                           const uint64_t* __restrict__ tbase,
                                           uint64_t* __restrict__ off_out, uint64_t T,
                                           uint32_t* __restrict__ payload, uint32_t R0, uint32_t rpb,
                                           const RecPre& pre, uint32_t* ctr) {
  const uint32_t tid = threadIdx.x;
  const uint32_t nown = (S - R0) < rpb ? S - R0 : rpb;
  const uint32_t cnt = (S - R0) < rpb + kEmitExtra ? S - R0 : rpb + kEmitExtra;
  // The window starts zeroed for the first slice (the previous chunk's last
  // barrier ended its reads of the window; several barriers follow before
  // the first bits are placed).
  for (uint32_t i = tid; i < kEmitWindow / 4; i += kEmitBlock) reinterpret_cast<uint4*>(sh.out)[i] = uint4{0, 0, 0, 0};

  // ---- 1. this thread's record ----
  const uint32_t j = tid;
  const bool active = j < cnt;
  uint32_t kpos = 0, klen = 0, l = 0, vpos = 0, vlen = 0;
  bool isB = false, tomb = false;
  uint64_t rec_off = 0, rec_end = 0;
  if (active) {
    const uint32_t r = R0 + j;
    const bool last = r + 1 == S;
    const uint32_t ref = pre.ref;
    // every load of this record's fields is issued before any is used
    uint64_t b0 = 0, b1 = 0;
    if (kTiled) {
      b0 = tbase[pre.o0 >> kTiledShift];
      b1 = tbase[pre.o1 >> kTiledShift];
    }
    uint32_t idx;
    const SideView s = pick(A, B, ref, idx);
    const KeyRef x = key_of(s, idx);
    bool t;
    value_bits(s, idx, vlen, t, &vpos);
    if (j == 0) {
      // the key length of the record before the chunk (for c of its first record)
      uint32_t kp = 0;
      if (R0 > 0) {
        uint32_t pidx;
        const SideView ps = pick(A, B, pre.pref, pidx);
        kp = 8u * (ps.key_off[pidx + 1] - ps.key_off[pidx]);
      }
      sh.kprev0 = kp;
    }
    if (kLcp) {
      l = min(pre.lcp, 8u * x.len);  // a stale array must not send reads past the key
    } else if (r > 0) {
      uint32_t pidx;
      const SideView ps = pick(A, B, final_refs[r - 1], pidx);
      l = lcp_bits(ps.keys, key_of(ps, pidx), s.keys, x);
    }
    constexpr uint64_t kLocal = (1ull << kTiledShift) - 1;
    rec_off = kTiled ? b0 + (pre.o0 & kLocal) : pre.o0;
    rec_end = kTiled ? (last ? T : b1 + (pre.o1 & kLocal)) : pre.o1;
    tomb = t;
    kpos = x.pos;
    klen = x.len;
    isB = s.isB;
    sh.kbits[j] = 8u * x.len;
    if (j == 0) sh.bit_lo = rec_off;
    if (j == nown - 1) sh.bit_hi = rec_end;
    if (j == cnt - 1) sh.bit_ext = rec_end;
    if (kTiled && off_out && j < nown) {
      off_out[r] = rec_off;
      if (r + 1 == S) off_out[S] = T;
    }
  }
  __syncthreads();
  // the source spans: the owned records', and those of the records after them
  // that start inside the last owned word (usually one); a side's records
  // are in arena order, so each span runs from its first record's bytes to
  // its last record's
  {
    const bool src = active && (j < nown || rec_off < 32ull * ((sh.bit_hi + 31) >> 5));
    const uint32_t klo = kpos + (l >> 3), khi = kpos + klen;
    const bool ks = src && klo < khi, vs = src && vlen != 0;
    uint4 blo, bhi;  // (wave-uniform)
    wave_bounds(ks && !isB, klo, khi, blo.x, bhi.x);
    wave_bounds(ks && isB, klo, khi, blo.y, bhi.y);
    wave_bounds(vs && !isB, vpos, vpos + vlen, blo.z, bhi.z);
    wave_bounds(vs && isB, vpos, vpos + vlen, blo.w, bhi.w);
    if ((tid & (kWave - 1)) == 0) {
      sh.wspan_lo[tid / kWave] = blo;
      sh.wspan_hi[tid / kWave] = bhi;
    }
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t slo[4], shi[4];
    for (int q = 0; q < 4; ++q) {
      slo[q] = 0xFFFFFFFFu;
      shi[q] = 0;
    }
    for (int w = 0; w < kEmitBlock / kWave; ++w) {
      const uint4 a = sh.wspan_lo[w], b = sh.wspan_hi[w];
      slo[0] = min(slo[0], a.x), slo[1] = min(slo[1], a.y), slo[2] = min(slo[2], a.z), slo[3] = min(slo[3], a.w);
      shi[0] = max(shi[0], b.x), shi[1] = max(shi[1], b.y), shi[2] = max(shi[2], b.z), shi[3] = max(shi[3], b.w);
    }
    uint32_t at = 0;
    for (int q = 0; q < 4; ++q) {
      sh.stage_at[q] = at;
      if (slo[q] < shi[q]) {
        const uint32_t lo = slo[q] & ~15u;
        // a 32-bit read at the last byte reaches at most 7 bytes past it
        const uint32_t hi = (shi[q] + 8u + 15u) & ~15u;
        sh.span_lo[q] = lo;
        sh.span_hi[q] = hi;
        const uint8_t* base = q == 0 ? A.keys : q == 1 ? B.keys : q == 2 ? A.vals : B.vals;
        sh.src_at[q] = reinterpret_cast<uint64_t>(base) + lo - at;
        at += hi - lo;
      } else {
        sh.span_lo[q] = 0;
        sh.span_hi[q] = 0;
        sh.src_at[q] = 0;  // (no staged byte maps to an empty span)
      }
    }
    sh.stage_at[4] = at;
  }
  // controls (need the predecessor's key length)
  uint32_t c = 0;
  if (active) {
    const uint32_t r = R0 + j;
    const uint32_t kprev = j ? sh.kbits[j - 1] : sh.kprev0;
    c = (r % 15u == 0) ? 1u + l : kprev - l;
  }
  __syncthreads();

  // ---- stage the source spans ----
  const bool staged = sh.stage_at[4] <= kEmitStage;
  if (staged && sh.stage_at[4] > 0) {
    // global -> LDS without registers: each wave moves 64 consecutive
    // 16-byte chunks, lane i's chunk landing 16 i bytes after the wave's base
    const uint32_t total16 = sh.stage_at[4] / 16;
    const uint32_t at1 = sh.stage_at[1], at2 = sh.stage_at[2], at3 = sh.stage_at[3];
    const uint32_t lane = tid & (kWave - 1);
    for (uint32_t c0 = (tid / kWave) * kWave; c0 < total16; c0 += kEmitBlock) {
      const uint32_t c = c0 + lane;
      if (c < total16) {
        const uint32_t byte = c * 16;
        const uint32_t q = (byte >= at1) + (byte >= at2) + (byte >= at3);
        lds_dma16(reinterpret_cast<const uint8_t*>(sh.src_at[q] + byte), sh.stage + c0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
  }
  // The next chunk's ticket: taken here, after the last global load of the
  // chunk, so that its round trip overlaps the LDS work below (a later wait
  // for a load would also wait for it).
  // (an increment-with-wrap at 2^32 - 1 is an add of one here; unlike an add,
  // the compiler does not rewrite it into a wave-combined form whose result
  // it must wait for at once)
  uint32_t ticket = 0;
  if (ctr && tid == 0) ticket = __builtin_amdgcn_atomic_inc32(ctr, 0xFFFFFFFFu, __ATOMIC_RELAXED, "agent");
  // source bit positions of this record's key suffix and value bytes
  const uint32_t k = 8u * klen;
  const uint32_t e1 = eg0_len(c), e2 = eg0_len(k - l), ev = eg0_len(vlen);
  const uint32_t vhl = tomb ? 1u : 1u + ev;
  const uint64_t vh = tomb ? 0ull : ((1ull << ev) | (static_cast<uint64_t>(vlen) + 1ull));
  // segment ends relative to the record start
  const uint32_t b1 = e1, b2 = b1 + e2, b3 = b2 + (k - l), b4 = b3 + vhl, b5 = b4 + 8u * vlen;
  EmitRecord rec{active && b5 == rec_end - rec_off, rec_off, rec_end, c, k, l, vh, b1, b2, b3, b4, b5, 0, 0};
  __syncthreads();
  // The two source kinds get separate code so that the staged one reads LDS
  // with LDS instructions (a pointer that may be either would be read with
  // flat loads).
  if (staged) {
    const uint32_t qk = isB ? 1u : 0u, qv = 2u + qk;
    // relative to the first emitted key byte, which lies inside the span
    rec.kbit = 8ull * (kpos + (l >> 3) - sh.span_lo[qk] + sh.stage_at[qk]) + (l & 7u);
    rec.vbit = 8ull * (vpos - sh.span_lo[qv] + sh.stage_at[qv]);
    const uint32_t* st = reinterpret_cast<const uint32_t*>(sh.stage);
    emit_slices<uint32_t>(sh, rec, st, st, T, payload, ticket);
  } else {
    rec.kbit = 8ull * kpos + l;
    rec.vbit = 8ull * vpos;
    emit_slices<uint64_t>(sh, rec, reinterpret_cast<const uint32_t*>(isB ? B.keys : A.keys),
                reinterpret_cast<const uint32_t*>(isB ? B.vals : A.vals), T, payload, ticket);
  }
}

// Records per workgroup: the expected output bits and staged source bytes of
// one workgroup fill about 90% of the window and the stage (a workgroup above
// that takes its window in slices or reads its sources in place).  Staged
// spans also hold the keys of replaced records and 16-byte margins, so the
// source estimate is all input bytes per survivor plus 4.
__host__ __device__ inline uint32_t emit_rpb(uint32_t S, uint64_t T, uint64_t src_bytes) {
  const double mean_bits = static_cast<double>(T) / S;
  const double mean_src = static_cast<double>(src_bytes) / S + 4.0;
  const double r1 = 0.9 * kEmitWindow * 32.0 / mean_bits;
  const double r2 = 0.9 * kEmitStage / mean_src;
  const double r = r1 < r2 ? r1 : r2;
  return r >= kEmitMaxRecs ? kEmitMaxRecs : (r < 16.0 ? 16u : static_cast<uint32_t>(r));
}

// One workgroup per `rpb` records (kDev = false: S, T and rpb come from the
// host), or a grid of workgroups that are all resident at once (kDev = true:
// S and T are read from device memory, where earlier kernels left them, and
// rpb follows from them).  A resident workgroup starts with chunk
// blockIdx.x and then takes chunks from one of kEmitCtrs ticket counters
// (workgroup b uses counter b mod kEmitCtrs, whose tickets name the chunks
// congruent to it beyond those the workgroups start with), so that
// workgroups that drew short chunks take more; spreading the tickets over
// several counters keeps any one address cool.  Counter x hands out exactly
// as many tickets as there are chunks congruent to x (one per chunk taken
// from it, one that ends the loop for each workgroup that ran a chunk), so
// the workgroup that draws the last one sets it back to zero for the next
// launch.  (Six waves per SIMD: the register budget this asks for is still
// faster than five.)
template <bool kDev, bool kTiled, bool kLcp>
__global__ __launch_bounds__(kEmitBlock) __attribute__((amdgpu_waves_per_eu(6))) void k_emit(em_side_t A, em_side_t B,
                                                     const uint32_t* __restrict__ final_refs,
                                                     const uint32_t* __restrict__ lcp_in, uint32_t S_arg,
                                                     const uint64_t* __restrict__ off,
                                                     const uint64_t* __restrict__ tbase,
                                                     uint64_t* __restrict__ off_out, uint64_t T_arg,
                                                     uint32_t* __restrict__ payload, uint32_t rpb_arg,
                                                     const uint32_t* __restrict__ d_S,
                                                     const uint64_t* __restrict__ d_T, uint64_t src_bytes,
                                                     uint32_t* __restrict__ ctr) {
  __shared__ EmitShared sh;
  const uint32_t S = kDev ? d_S[0] : S_arg;
  const uint64_t T = kDev ? d_T[0] : T_arg;
  if (S == 0) return;
  const uint32_t rpb = kDev ? emit_rpb(S, T, src_bytes) : rpb_arg;
  if (!kDev) {
    const uint32_t R0 = blockIdx.x * rpb;
    if (R0 >= S) return;
    const RecPre pre = load_rec_pre<kTiled, kLcp>(final_refs, lcp_in, off, S, R0, rpb);
    emit_chunk<kTiled, kLcp>(sh, A, B, final_refs, lcp_in, S, off, tbase, off_out, T, payload, R0, rpb, pre,
                             nullptr);
    return;
  }
  const uint32_t nchunks = (S - 1) / rpb + 1;
  const uint32_t G = gridDim.x, R = G < kEmitCtrs ? G : kEmitCtrs;
  const uint32_t x = blockIdx.x % R;
  const uint32_t nb = (G - x + R - 1) / R;                            // workgroups on counter x
  const uint32_t nx = x < nchunks ? (nchunks - 1 - x) / R + 1 : 0;  // chunks congruent to x
  uint32_t* const my_ctr = ctr + x * kEmitCtrStride;
  uint64_t chunk = blockIdx.x;  // 64 bits: a ticket near 2^32 must end the loop, not wrap
  while (chunk < nchunks) {
    const uint32_t R0 = static_cast<uint32_t>(chunk * rpb);  // < S
    const RecPre pre = load_rec_pre<kTiled, kLcp>(final_refs, lcp_in, off, S, R0, rpb);
    emit_chunk<kTiled, kLcp>(sh, A, B, final_refs, lcp_in, S, off, tbase, off_out, T, payload, R0, rpb, pre,
                             my_ctr);
    // (sh.next is rewritten only after the next chunk's first barriers)
    const uint32_t t = sh.next;
    chunk = static_cast<uint64_t>(R) * (static_cast<uint64_t>(t) + nb) + x;
    if (chunk >= nchunks && threadIdx.x == 0 && t == nx - 1)
      __hip_atomic_store(my_ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
  const uint64_t src = A->key_bytes + B->key_bytes + A->val_bytes + B->val_bytes;
  const uint32_t rpb = emit_rpb(S, T, src);
  const uint32_t blocks = (S + rpb - 1) / rpb;
  if (lcp_bits)
    hipLaunchKernelGGL((k_emit<false, false, true>), dim3(blocks), dim3(kEmitBlock), 0, as_stream(stream), *A,
                       *B, final_refs, lcp_bits, S, off, nullptr, nullptr, T, payload, rpb, nullptr, nullptr,
                       src, nullptr);
  else
    hipLaunchKernelGGL((k_emit<false, false, false>), dim3(blocks), dim3(kEmitBlock), 0, as_stream(stream),
                       *A, *B, final_refs, nullptr, S, off, nullptr, nullptr, T, payload, rpb, nullptr,
                       nullptr, src, nullptr);
  return check_launch();
}

namespace em {

// Workgroups of k_emit<true, true, true> that one device holds at once.
int emit_resident_grid(int dev, int* grid) {
  static int cache[64] = {0};
  if (dev < 0 || dev >= 64) return set_hip_error(hipErrorInvalidDevice);
  if (cache[dev] == 0) {
    int cus = 0, per = 0;
    hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return set_hip_error(e);
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k_emit<true, true, true>, kEmitBlock, 0);
    if (e != hipSuccess) return set_hip_error(e);
    cache[dev] = (cus > 0 ? cus : 1) * (per > 0 ? per : 1);
  }
  *grid = cache[dev];
  return EM_OK;
}

// The emitter after kernels that left S and T in device memory and record
// offsets as partition number + local offset (tbase: partition bit bases):
// exactly as many workgroups as the device holds at once (a workgroup that
// had to wait for another to finish would add its whole run to the tail).
int emit_launch_dev(const em_side_t& A, const em_side_t& B, const uint32_t* final_refs,
                    const uint32_t* lcp_bits, const uint64_t* toff, const uint64_t* tbase,
                    uint64_t* off_out, uint32_t* payload, const uint32_t* d_S, const uint64_t* d_T,
                    uint32_t* ctr, hipStream_t st) {
  int dev = 0, grid = 0;
  if (hipGetDevice(&dev) != hipSuccess) return set_hip_error(hipErrorInvalidDevice);
  const int rc = emit_resident_grid(dev, &grid);
  if (rc) return rc;
  const uint64_t src = A.key_bytes + B.key_bytes + A.val_bytes + B.val_bytes;
  hipLaunchKernelGGL((k_emit<true, true, true>), dim3(grid), dim3(kEmitBlock), 0, st, A, B, final_refs,
                     lcp_bits, 0u, toff, tbase, off_out, 0ull, payload, 0u, d_S, d_T, src, ctr);
  return check_launch();
}

}  // namespace em
