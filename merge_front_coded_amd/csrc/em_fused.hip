// The whole path in one pass: co-rank, stable merge, keep-newer, exact bit
// LCP and lengths, bit offsets and word-owned payload emission, one workgroup
// per partition of `items` merged outputs.
//
// Everett, "GPU construction experiment": merge by diagonal partitions with
// equal keys older first, keep the last reference of each equal-key run, the
// compacted order fixes predecessors and ordinals, exact lengths (c_i
// equation, record grammar) are scanned into bit offsets by one global scan
// with no per-chunk reset, and each output word is written once.  Two
// decoupled look-backs over partitions (dynamic tickets) give each partition
// its survivor base (which fixes the global W15 phase) and its bit base.
//
// Partition and word ownership.  A payload word belongs to the partition that
// holds its last bit (the final word to the last partition).  A partition's
// first word may therefore begin with bits of earlier partitions: every
// partition publishes the last 32 bits of the stream up to its end ("tail"),
// and the owner of that word reads its predecessor's tail.  All waits point
// to partitions with smaller tickets, so they always end.
//
// Staging.  The partition's key offsets (including the two A keys and the B
// key before it, for its first survivor's predecessor, and the B key after
// it, for an equal pair split by the boundary), value offsets, tombstones, key
// bytes and value bytes are loaded once; key and value bytes go
// global -> LDS by LDS-DMA when they fit, otherwise they are read in place.
// The partition's bit stream is built in an LDS window at local alignment and
// stored shifted to its global bit base, in slices when it is longer than the
// window.
#include <type_traits>

#include "em_tile.h"

namespace em {

constexpr int kFuseBlock = 256;
constexpr uint32_t kFuseTile = kFuseBlock;          // outputs per partition, at most
constexpr uint32_t kFuseKeyCap = 14 * 1024;          // staged key bytes (multiple of 1 KB)
constexpr uint32_t kFuseValCap = 12 * 1024;          // staged value bytes (multiple of 1 KB)
constexpr uint32_t kFuseWin = 4096;                  // output words per slice
constexpr uint64_t kTailReady = 1ull << 63;

struct FuseShared {
  uint32_t a_off[kFuseTile + 4];  // key offsets of A records aK0 .. i1 (aK0 = i0 - 2 when it exists)
  uint32_t b_off[kFuseTile + 4];  // key offsets of B records bK0 .. j1 (+ the next B)
  uint32_t a_voff[kFuseTile + 1];
  uint32_t b_voff[kFuseTile + 1];
  uint8_t a_tomb[kFuseTile];
  uint8_t b_tomb[kFuseTile];
  union {
    struct {
      uint64_t a_pfx[kFuseTile + 2];
      uint64_t b_pfx[kFuseTile + 2];
    } m;
    uint32_t win[kFuseWin + 2];
  } u;
  uint4 keys[kFuseKeyCap / 16];
  uint4 vals[kFuseValCap / 16];
  uint32_t surv[kFuseTile];
  uint32_t ords[kFuseTile];
  uint64_t scan64[kFuseBlock / kWave + 1];
  uint32_t scan32[kFuseBlock / kWave + 1];
  uint32_t tile, i0, i1, g0, carry;
  uint64_t b0;
  uint32_t prev_tail;
};

struct FuseOut {
  uint32_t* payload;
  uint32_t* d_S;
  uint64_t* d_T;
  // optional (nullable) per-record outputs, same meaning as the separate calls
  uint32_t* final_refs;
  uint32_t* ord_A;
  uint32_t* ord_B;
  uint32_t* len_bits;
  uint32_t* lcp_bits;
  uint64_t* off;
};

// co-rank of diagonal d given the coarse co-ranks around it
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

__global__ __launch_bounds__(kFuseBlock) void k_merge_fc(
    em_side_t A, em_side_t B, const uint32_t* __restrict__ csplits, uint32_t coarse, uint32_t items,
    uint32_t P, FuseOut out, uint32_t* __restrict__ ticket, uint64_t* __restrict__ desc_s,
    uint64_t* __restrict__ desc_b, uint64_t* __restrict__ tail) {
  __shared__ FuseShared sh;
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & (kWave - 1);
  const uint32_t N = A.n + B.n;
  if (tid == 0) sh.tile = atomicAdd(ticket, 1u);
  __syncthreads();
  const uint32_t tile = sh.tile;
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
  uint32_t i0 = sh.i0, i1 = sh.i1;
  const bool valid = i0 <= d0 && i1 <= d1 && i0 <= i1 && d0 - i0 <= d1 - i1 && i1 <= A.n &&
                     d1 - i1 <= B.n;
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

  // ---- 2. offsets, value offsets, tombstones (all loads, then all stores) ----
  {
    constexpr int kPer = 2;  // (kFuseTile + 4) / kFuseBlock rounded up
    uint32_t ka[kPer], kb[kPer], va[kPer], vb[kPer];
    uint8_t ta[kPer], tb[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const uint32_t x = tid + u * kFuseBlock;
      ka[u] = x < na_off ? A.key_off[aK0 + x] : 0u;
      kb[u] = x < nb_off ? B.key_off[bK0 + x] : 0u;
      va[u] = x <= nA_t ? A.val_off[i0 + x] : 0u;
      vb[u] = x <= nB_t ? B.val_off[j0 + x] : 0u;
      ta[u] = (x < nA_t && A.tomb) ? A.tomb[i0 + x] : 0;
      tb[u] = (x < nB_t && B.tomb) ? B.tomb[j0 + x] : 0;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const uint32_t x = tid + u * kFuseBlock;
      if (x < na_off) sh.a_off[x] = ka[u];
      if (x < nb_off) sh.b_off[x] = kb[u];
      if (x <= nA_t) sh.a_voff[x] = va[u];
      if (x <= nB_t) sh.b_voff[x] = vb[u];
      if (x < nA_t) sh.a_tomb[x] = ta[u];
      if (x < nB_t) sh.b_tomb[x] = tb[u];
    }
  }
  __syncthreads();

  // ---- 3. stage key and value bytes ----
  // Key spans get a 16-byte margin (comparisons read up to 11 bytes past a
  // key), value spans 8 bytes (a 64-bit window read at the last byte).
  const uint32_t a_lo = sh.a_off[0] & ~15u;
  const uint32_t a_bytes = ((sh.a_off[na_off - 1] + 16u + 15u) & ~15u) - a_lo;
  const uint32_t b_lo = sh.b_off[0] & ~15u;
  const uint32_t b_bytes = ((sh.b_off[nb_off - 1] + 16u + 15u) & ~15u) - b_lo;
  const uint32_t av_lo = sh.a_voff[0] & ~15u;
  const uint32_t av_bytes = ((sh.a_voff[nA_t] + 8u + 15u) & ~15u) - av_lo;
  const uint32_t bv_lo = sh.b_voff[0] & ~15u;
  const uint32_t bv_bytes = ((sh.b_voff[nB_t] + 8u + 15u) & ~15u) - bv_lo;
  const bool staged = a_bytes + b_bytes <= kFuseKeyCap && av_bytes + bv_bytes <= kFuseValCap;
  {
    const uint32_t nk16 = staged ? (a_bytes + b_bytes) / 16 : 0u, na16 = a_bytes / 16;
    const uint32_t nv16 = staged ? (av_bytes + bv_bytes) / 16 : 0u, nav16 = av_bytes / 16;
    for (uint32_t c0 = (tid / kWave) * kWave; c0 < nk16; c0 += kFuseBlock) {
      const uint32_t c = c0 + lane;
      if (c < nk16)
        lds_dma16(c < na16 ? A.keys + a_lo + 16u * c : B.keys + b_lo + 16u * (c - na16), sh.keys + c0);
    }
    for (uint32_t c0 = (tid / kWave) * kWave; c0 < nv16; c0 += kFuseBlock) {
      const uint32_t c = c0 + lane;
      if (c < nv16)
        lds_dma16(c < nav16 ? A.vals + av_lo + 16u * c : B.vals + bv_lo + 16u * (c - nav16), sh.vals + c0);
    }
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();
  // The rest of the partition's work is compiled twice, for the LDS copy and
  // for the arenas, so that the staged variant reads LDS with LDS
  // instructions (a pointer that may be either would be read with flat loads).
  auto rest = [&](auto staged_tag) __attribute__((always_inline)) {
    constexpr bool ST = decltype(staged_tag)::value;
    const uint8_t* kbA = ST ? reinterpret_cast<const uint8_t*>(sh.keys) : A.keys;
    const uint8_t* kbB = ST ? reinterpret_cast<const uint8_t*>(sh.keys) : B.keys;
    const uint32_t kadjA = ST ? a_lo : 0u, kadjB = ST ? b_lo - a_bytes : 0u;
    const uint8_t* vbA = ST ? reinterpret_cast<const uint8_t*>(sh.vals) : A.vals;
    const uint8_t* vbB = ST ? reinterpret_cast<const uint8_t*>(sh.vals) : B.vals;
    const uint32_t vadjA = ST ? av_lo : 0u, vadjB = ST ? bv_lo - av_bytes : 0u;

    // ---- 4. prefix cache of the partition's merge keys ----
    {
      const uint32_t* ao = sh.a_off + a_first;
      const uint32_t* bo = sh.b_off + b_first;
      const uint32_t nbk = nB_t + (has_next_b ? 1u : 0u);
      for (uint32_t x = tid; x < nA_t; x += kFuseBlock) {
        const uint32_t ln = ao[x + 1] - ao[x];
        sh.u.m.a_pfx[x] = load_be8(kbA, ao[x] - kadjA) & be_mask(ln < 8 ? ln : 8);
      }
      for (uint32_t y = tid; y < nbk; y += kFuseBlock) {
        const uint32_t ln = bo[y + 1] - bo[y];
        sh.u.m.b_pfx[y] = load_be8(kbB, bo[y] - kadjB) & be_mask(ln < 8 ? ln : 8);
      }
    }
    __syncthreads();

    // ---- 5. merge (one output per thread) and keep-newer ----
    uint32_t refs[1];
    const uint32_t kept = merge_slice<1>(sh.a_off + a_first, sh.b_off + b_first, sh.u.m.a_pfx, sh.u.m.b_pfx,
                                         kbA, kadjA, kbB, kadjB, tid, len, nA_t, nB_t, has_next_b, i0, A.n,
                                         j0, refs);
    uint32_t n_kept;
    const uint32_t ord = block_exclusive_scan<uint32_t, kFuseBlock>(kept, sh.scan32, n_kept);
    if (tid < len) {
      const uint32_t ref = refs[0] & ~kDrop;
      const bool drop = (refs[0] & kDrop) != 0;
      if (ref < A.n)
        sh.ords[ref - i0] = drop ? EM_NONE : ord;
      else
        sh.ords[nA_t + (ref - A.n - j0)] = ord;
      if (!drop) sh.surv[ord] = ref;
    }

    // ---- 6. publish the survivor count early; the base is resolved later ----
    if (tid == 0) lookback_publish(desc_s, tile, n_kept);
    __syncthreads();

    // ---- 7. this thread's survivor: key, value, predecessor, LCP ----
    const bool has = tid < n_kept;
    uint32_t kpos = 0, klen = 0, l = 0, kprev = 0, vpos = 0, vlen = 0;
    bool isB = false, tomb = false;
    if (has) {
      const uint32_t ref = sh.surv[tid];
      isB = ref >= A.n;
      uint32_t ko, kend;
      if (isB) {
        const uint32_t y = ref - A.n - j0;
        ko = sh.b_off[b_first + y] - kadjB;
        kend = sh.b_off[b_first + y + 1] - kadjB;
        tomb = sh.b_tomb[y] != 0;
        vlen = tomb ? 0u : sh.b_voff[y + 1] - sh.b_voff[y];
        vpos = sh.b_voff[y] - vadjB;
      } else {
        const uint32_t x = ref - i0;
        ko = sh.a_off[a_first + x] - kadjA;
        kend = sh.a_off[a_first + x + 1] - kadjA;
        tomb = sh.a_tomb[x] != 0;
        vlen = tomb ? 0u : sh.a_voff[x + 1] - sh.a_voff[x];
        vpos = sh.a_voff[x] - vadjA;
      }
      kpos = ko;
      klen = kend - ko;
      const uint8_t* xb = isB ? kbB : kbA;
      const KeyRef xk{ko, klen};
      // predecessor survivor's key
      bool have_p = false;
      const uint8_t* pb = nullptr;
      KeyRef pk{0, 0};
      if (tid > 0) {
        const uint32_t pref = sh.surv[tid - 1];
        have_p = true;
        if (pref >= A.n) {
          const uint32_t y = pref - A.n - j0;
          pb = kbB;
          pk = KeyRef{sh.b_off[b_first + y] - kadjB, sh.b_off[b_first + y + 1] - sh.b_off[b_first + y]};
        } else {
          const uint32_t x = pref - i0;
          pb = kbA;
          pk = KeyRef{sh.a_off[a_first + x] - kadjA, sh.a_off[a_first + x + 1] - sh.a_off[a_first + x]};
        }
      } else if (d0 > 0) {
        // The largest key before the partition: A[i0-1] unless it is the older
        // copy of this very key (then A[i0-2]), or B[j0-1], whichever is larger.
        // (With no survivor before the partition there is no such key.)
        bool hA = false, hB = false;
        KeyRef ka{0, 0}, kb{0, 0};
        if (a_first >= 1) {
          ka = KeyRef{sh.a_off[a_first - 1] - kadjA, sh.a_off[a_first] - sh.a_off[a_first - 1]};
          hA = true;
          if (cmp_keys(kbA, ka, xb, xk) == 0) {
            hA = a_first >= 2;
            if (hA) ka = KeyRef{sh.a_off[a_first - 2] - kadjA, sh.a_off[a_first - 1] - sh.a_off[a_first - 2]};
          }
        }
        if (b_first >= 1) {
          kb = KeyRef{sh.b_off[b_first - 1] - kadjB, sh.b_off[b_first] - sh.b_off[b_first - 1]};
          hB = true;
        }
        if (hA && hB) {
          const bool a_larger = cmp_keys(kbA, ka, kbB, kb) > 0;
          pb = a_larger ? kbA : kbB;
          pk = a_larger ? ka : kb;
          have_p = true;
        } else if (hA || hB) {
          pb = hA ? kbA : kbB;
          pk = hA ? ka : kb;
          have_p = true;
        }
      }
      if (have_p) {
        l = lcp_bits(pb, pk, xb, xk);
        kprev = 8u * pk.len;
      }
    }

    // ---- 8. survivor base (look-back 1), controls and exact lengths ----
    if (tid < kWave) {
      const uint64_t g = lookback_resolve(desc_s, tile, n_kept);
      if (tid == 0) sh.g0 = static_cast<uint32_t>(g);
    }
    __syncthreads();
    const uint32_t g0 = sh.g0;
    if (out.final_refs)
      for (uint32_t x = tid; x < n_kept; x += kFuseBlock) out.final_refs[g0 + x] = sh.surv[x];
    if (out.ord_A)
      for (uint32_t x = tid; x < nA_t; x += kFuseBlock) {
        const uint32_t o = sh.ords[x];
        out.ord_A[i0 + x] = o == EM_NONE ? EM_NONE : g0 + o;
      }
    if (out.ord_B)
      for (uint32_t y = tid; y < nB_t; y += kFuseBlock) out.ord_B[j0 + y] = g0 + sh.ords[nA_t + y];
    const uint32_t k = 8u * klen;
    const uint32_t c = ((g0 + tid) % 15u == 0) ? 1u + l : kprev - l;
    const uint32_t e1 = eg0_len(c), e2 = eg0_len(k - l), ev = eg0_len(vlen);
    const uint32_t rb1 = e1, rb2 = rb1 + e2, rb3 = rb2 + (k - l), rb4 = rb3 + (tomb ? 1u : 1u + ev);
    const uint32_t rb5 = rb4 + 8u * vlen;
    const uint64_t rlen = has ? rb5 : 0u;

    // ---- 9. local bit offsets; publish the bit total early ----
    uint64_t tile_bits;
    const uint64_t sb = block_exclusive_scan<uint64_t, kFuseBlock>(rlen, sh.scan64, tile_bits);
    if (tid == 0) lookback_publish(desc_b, tile, tile_bits);

    // ---- 10. emission: the local bit stream in window slices, stored shifted ----
    // A single-slice partition builds its whole stream and publishes its tail
    // before it resolves its bit base; a longer one resolves first.
    const uint64_t nloc = (tile_bits + 31) >> 5;  // local words
    const uint32_t nslices = nloc ? static_cast<uint32_t>((nloc + kFuseWin - 1) / kFuseWin) : 1u;
    const bool early = nslices == 1;
    if (!early) {
      if (tid < kWave) {
        const uint64_t b = lookback_resolve(desc_b, tile, tile_bits);
        if (tid == 0) sh.b0 = b;
      }
    }
    const bool last_tile = tile == P - 1;
    const uint64_t vh = tomb ? 0ull : ((1ull << ev) | (static_cast<uint64_t>(vlen) + 1ull));
    const uint32_t* kw = reinterpret_cast<const uint32_t*>(isB ? kbB : kbA);
    const uint32_t* vw = reinterpret_cast<const uint32_t*>(isB ? vbB : vbA);
    const uint64_t kbit = 8ull * kpos + l;
    const uint64_t vbit = 8ull * vpos;
    for (uint32_t sl = 0; sl < nslices; ++sl) {
      const uint64_t w0 = static_cast<uint64_t>(sl) * kFuseWin;  // first local word of the slice
      const uint64_t s0 = w0 << 5, s1 = min(s0 + 32ull * kFuseWin, tile_bits);
      const uint32_t nz =
          static_cast<uint32_t>(min(static_cast<uint64_t>(kFuseWin), nloc - min(nloc, w0))) + 2;
      for (uint32_t i = tid; i < nz; i += kFuseBlock) sh.u.win[i] = 0;
      __syncthreads();
      if (has && sb < s1 && sb + rlen > s0) {
        const uint32_t from = sb >= s0 ? 0u : static_cast<uint32_t>(s0 - sb);
        const uint32_t to = sb + rlen <= s1 ? rb5 : static_cast<uint32_t>(s1 - sb);
        BitAppender ap;
        ap.start(sh.u.win, static_cast<uint32_t>(sb + from - s0));
        auto imm = [&](uint64_t v, uint32_t a, uint32_t b) {  // field occupying [a, b)
          const uint32_t lo = max(a, from), hi = min(b, to);
          if (lo < hi)
            ap.put64((v >> (b - hi)) & (hi - lo == 64 ? ~0ull : ((1ull << (hi - lo)) - 1)), hi - lo);
        };
        auto span = [&](const uint32_t* base, uint64_t bp, uint32_t a, uint32_t b) {
          const uint32_t lo = max(a, from), hi = min(b, to);
          if (lo < hi) put_span(ap, base, bp + (lo - a), hi - lo);
        };
        imm(static_cast<uint64_t>(c) + 1u, 0, rb1);
        imm(static_cast<uint64_t>(k - l) + 1u, rb1, rb2);
        span(kw, kbit, rb2, rb3);
        imm(vh, rb3, rb4);
        span(vw, vbit, rb4, rb5);
        ap.finish();
      }
      __syncthreads();
      auto loc = [&](uint64_t w) -> uint32_t {  // local word w, for w in [w0 - 1, w0 + kFuseWin]
        if (w + 1 == 0) return sh.prev_tail;     // w = -1: the bits before the partition
        if (w < w0) return sh.carry;             // the previous slice's last word
        return sh.u.win[w - w0];
      };
      if (sl == nslices - 1 && tid == 0) {
        // publish this partition's tail: the last 32 bits of the stream up to its end
        uint32_t tv, tn;
        if (tile_bits >= 32) {
          const uint64_t e = tile_bits - 32, ew = e >> 5;
          const uint32_t r = static_cast<uint32_t>(e & 31u);
          tv = r ? __builtin_amdgcn_alignbit(loc(ew), loc(ew + 1), 32u - r) : loc(ew);
          tn = 32;
        } else {
          uint64_t pv = 0, pn = 0;
          if (tile > 0) {
            uint64_t t;
            while (!((t = desc_load(tail + tile - 1)) & kTailReady)) __builtin_amdgcn_s_sleep(1);
            pv = t & 0xFFFFFFFFu;
            pn = (t >> 32) & 63u;
          }
          const uint32_t tb = static_cast<uint32_t>(tile_bits);
          const uint64_t mine = tb ? (sh.u.win[0] >> (32u - tb)) : 0u;
          tv = static_cast<uint32_t>((pv << tb) | mine);
          tn = static_cast<uint32_t>(min(pn + tb, 32ull));
        }
        desc_store(tail + tile, kTailReady | (static_cast<uint64_t>(tn) << 32) | tv);
      }
      if (sl == 0) {
        if (early && tid < kWave) {
          const uint64_t b = lookback_resolve(desc_b, tile, tile_bits);
          if (tid == 0) sh.b0 = b;
        }
        if (tid == 0) {
          uint32_t pt = 0;
          if ((sh.b0 & 31u) && tile > 0) {  // this partition's first word starts with earlier bits
            uint64_t t;
            while (!((t = desc_load(tail + tile - 1)) & kTailReady)) __builtin_amdgcn_s_sleep(1);
            pt = static_cast<uint32_t>(t);
          }
          sh.prev_tail = pt;
        }
      }
      __syncthreads();
      // owned words (a word belongs to the partition holding its last bit)
      const uint64_t b0 = sh.b0;
      const uint32_t s_sh = static_cast<uint32_t>(b0 & 31u);
      const uint64_t q = b0 >> 5;
      const uint64_t b_end = b0 + tile_bits;
      const uint64_t g_hi = (b_end >> 5) + ((last_tile && (b_end & 31u)) ? 1u : 0u);
      const uint64_t ga = q + w0, gb = min(g_hi, q + w0 + kFuseWin);
      for (uint64_t g = ga + tid; g < gb; g += kFuseBlock) {
        const uint64_t li = g - q;  // local word holding the word's last bits
        const uint32_t lo_w = loc(li);
        const uint32_t hi_w = s_sh ? loc(li - 1) : 0u;
        out.payload[g] = __builtin_bswap32(s_sh ? __builtin_amdgcn_alignbit(hi_w, lo_w, s_sh) : lo_w);
      }
      __syncthreads();
      if (tid == 0) sh.carry = sh.u.win[kFuseWin - 1];
      __syncthreads();
    }
    const uint64_t b0 = sh.b0;
    if (has) {
      if (out.len_bits) out.len_bits[g0 + tid] = static_cast<uint32_t>(rlen);
      if (out.lcp_bits) out.lcp_bits[g0 + tid] = l;
      if (out.off) out.off[g0 + tid] = b0 + sb;
    }
    if (last_tile && tid == 0) {
      out.d_S[0] = g0 + n_kept;
      out.d_T[0] = b0 + tile_bits;
      if (out.off) out.off[g0 + n_kept] = b0 + tile_bits;
    }
  };
  if (staged)
    rest(std::true_type{});
  else
    rest(std::false_type{});
}

size_t fused_ws(uint32_t N, uint32_t items) {
  const size_t P = items ? (static_cast<size_t>(N) + items - 1) / items : 0;
  return 256 + 3 * align_up((P ? P : 1) * sizeof(uint64_t), 256);
}

}  // namespace em

using namespace em;

extern "C" size_t em_merge_fc_workspace_bytes(uint32_t nA, uint32_t nB, uint32_t items_per_part) {
  const uint64_t N = static_cast<uint64_t>(nA) + nB;
  return align_up(fused_ws(N >= EM_MAX_RECORDS ? EM_MAX_RECORDS : static_cast<uint32_t>(N),
                           items_per_part ? items_per_part : 1), 256);
}

extern "C" int em_merge_fc(const em_side_t* A, const em_side_t* B, const uint32_t* coarse_splits,
                           uint32_t coarse_items, uint32_t items_per_part, uint32_t* payload,
                           uint64_t payload_words, uint32_t* d_S, uint64_t* d_T, uint32_t* final_refs,
                           uint32_t* ord_A, uint32_t* ord_B, uint32_t* len_bits, uint32_t* lcp_bits,
                           uint64_t* off, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_pair(A, B);
  if (rc) return rc;
  if (!coarse_splits || !payload || !d_S || !d_T || !ws) return EM_EINVAL;
  if (items_per_part == 0 || items_per_part > kFuseTile) return EM_EINVAL;
  if (coarse_items == 0 || coarse_items % items_per_part || coarse_items > EM_MAX_ITEMS_PER_PART * 256u)
    return EM_EINVAL;
  if (reinterpret_cast<uintptr_t>(ws) & 255) return EM_EINVAL;
  if ((reinterpret_cast<uintptr_t>(payload) & 15)) return EM_EINVAL;
  const uint32_t N = A->n + B->n;
  if (ws_bytes < fused_ws(N, items_per_part)) return EM_ENOSPC;
  uint64_t bound = 0;
  rc = em_payload_bound_bits(A, B, &bound);
  if (rc) return rc;
  if (payload_words < (bound + 31) / 32) return EM_ENOSPC;
  hipStream_t st = as_stream(stream);
  if (N == 0) {
    clear_u32(d_S, 1, st);
    clear_u64(d_T, 1, st);
    if (off) clear_u64(off, 1, st);
    return check_launch();
  }
  const uint32_t P = (N + items_per_part - 1) / items_per_part;
  WsCursor cur{static_cast<uint8_t*>(ws), 0};
  uint32_t* ticket = cur.take<uint32_t>(64);
  uint64_t* desc_s = cur.take<uint64_t>(P);
  uint64_t* desc_b = cur.take<uint64_t>(P);
  uint64_t* tail = cur.take<uint64_t>(P);
  clear_u32(ticket, 1, st);
  clear_u64(desc_s, static_cast<size_t>(P), st);
  clear_u64(desc_b, static_cast<size_t>(P), st);
  clear_u64(tail, static_cast<size_t>(P), st);
  FuseOut o{payload, d_S, d_T, final_refs, ord_A, ord_B, len_bits, lcp_bits, off};
  hipLaunchKernelGGL(k_merge_fc, dim3(P), dim3(kFuseBlock), 0, st, *A, *B, coarse_splits, coarse_items,
                     items_per_part, P, o, ticket, desc_s, desc_b, tail);
  return check_launch();
}
