// The whole path in three kernels: (1) per partition, co-ranks, the stable
// merge with keep-newer, exact bit LCPs, record lengths and partition-local
// bit offsets; (2) one workgroup scans the partitions' bit totals; (3) the
// word-owned payload emitter, reading the survivor count and payload length
// the first two left in device memory.  (The single-pass form of the whole
// path is em_onepass.hip.)
//
// Everett, "GPU construction experiment": merge by diagonal partitions with
// ties to the older side; keep the last reference of each equal-key run; the
// compacted order fixes predecessors and ordinals; exact lengths (c_i
// equation, record grammar) are scanned into bit offsets by one global scan
// with no per-chunk reset (here: a scan inside each partition plus a scan of
// the partition totals); each output word is written once.
//
// Kernel 1, one 512-thread workgroup per partition of `items` outputs:
//  * co-ranks of the partition's two diagonals, searched inside the coarse
//    partition that coarse_splits gives (read directly when the coarse
//    partitions are the partitions);
//  * the partition's key offsets and 8 bytes of each key go to LDS,
//    including the two A keys and the B key before the partition (for its
//    first survivor's predecessor) and the B key after it (for an equal pair
//    split by the boundary): the first 8 bytes, or, when all those keys share
//    a common prefix of 8 bytes or more, the 8 bytes after it (the pages'
//    prefix cache); key bytes stay in HBM;
//  * merge and keep as in em_merge_keep (a partition goes straight to the
//    exact merge when most of the launch's sampled partitions failed the
//    merge on cached prefixes); the survivor count is published to
//    a decoupled look-back right away and resolved after the LCPs (the global
//    survivor index fixes the W15 phase of c_i);
//  * each survivor's exact bit LCP with its predecessor comes from the two
//    cached words when they differ or a key ends inside them, and from the
//    key bytes in HBM otherwise; value lengths and tombstone flags are read
//    while the LCPs run;
//  * lengths, a block scan into partition-local bit offsets, and the
//    partition's bit total.  A survivor's offset is stored with its
//    partition number; the emitter adds the partition's bit base.
#include "em_tile.h"

namespace em {

constexpr int kMlBlock = 512;
// The workspace's first words: the partition ticket, the emitter's ticket
// counters from kEmitCtrStride, and the merge statistics on a line of their
// own from kMlStatWord; all zero at the start of each launch.
constexpr uint32_t kMlStatWord = kEmitCtrStride + kEmitCtrWords;
constexpr uint32_t kMlTicketWords = kMlStatWord + kEmitCtrStride;
constexpr int kMlWaves = kMlBlock / kWave;
constexpr uint32_t kMlMaxItems = 4 * kMlBlock;  // outputs per partition, at most

template <int IPT>
struct MlShared {
  static constexpr int kTile = kMlBlock * IPT;
  uint32_t a_off[kTile + 4];  // key offsets of A records aK0 .. i1 (aK0 = i0 - 2 when it exists)
  uint32_t b_off[kTile + 4];  // key offsets of B records bK0 .. j1 (+ the next B)
  union alignas(16) {
    struct {
      uint64_t a_pfx[kTile + 4];  // first 8 bytes of A keys aK0 .., big-endian, zero padded
      uint64_t b_pfx[kTile + 4];  // the same for B keys bK0 ..
    } m;
    struct {
      uint64_t spfx[kTile];  // survivors' prefixes, compacted
      uint32_t surv[kTile];  // survivors' references, compacted
      uint32_t ords[kTile];  // per input record: survivor ordinal in the partition, or EM_NONE
    } c;
  } u;
  uint64_t scan64[IPT * kMlWaves + 1];
  uint32_t scan32[kMlWaves + 1];
  uint32_t notes[kMlBlock];  // the merge's list of pairs to check, kWave words per wave
  uint32_t tile, i0, i1, g0, cp;
  uint32_t try_fast;  // this partition tries the merge on cached prefixes first
};

struct MlOut {
  uint32_t* d_S;
  uint32_t* final_refs;
  uint32_t* lcp_bits;
  uint64_t* toff;       // partition << kTiledShift | partition-local bit offset
  uint64_t* tile_bits;  // bit total of each partition
  uint32_t* ord_A;      // optional
  uint32_t* ord_B;      // optional
  uint32_t* len_bits;   // optional
};

// (Six waves per SIMD: three 512-thread partitions per compute unit, which
// their LDS allows.)
template <int IPT>
__global__ __launch_bounds__(kMlBlock) __attribute__((amdgpu_waves_per_eu(6))) void k_merge_len(em_side_t A, em_side_t B,
                                                        const uint32_t* __restrict__ csplits,
                                                        uint32_t coarse, uint32_t items, uint32_t P,
                                                        MlOut out, uint32_t* __restrict__ ticket,
                                                        uint64_t* __restrict__ desc_s) {
  using Sh = MlShared<IPT>;
  __shared__ Sh sh;
  const uint32_t tid = threadIdx.x;
  const uint32_t N = A.n + B.n;
  // the launch's record of merges on cached prefixes tried and failed (a line of its own)
  uint64_t* const fast_stat = reinterpret_cast<uint64_t*>(ticket + kMlStatWord);
  if (tid == 0) {
    const uint32_t t = atomicAdd(ticket, 1u);
    sh.tile = t;
    sh.try_fast = fast_merge_worth_trying(fast_stat, t) ? 1u : 0u;
  }
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

  // ---- 2. key offsets (all loads, then all stores; a thread past the end
  // loads the first offset again, so that no load sits under a condition
  // of its own) ----
  {
    constexpr int kPer = IPT + 1;  // ceil((kTile + 4) / kMlBlock)
    uint32_t ka[kPer], kb[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const uint32_t x = tid + u * kMlBlock;
      ka[u] = A.key_off[aK0 + (x < na_off ? x : 0u)];
      kb[u] = B.key_off[bK0 + (x < nb_off ? x : 0u)];
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const uint32_t x = tid + u * kMlBlock;
      if (x < na_off) sh.a_off[x] = ka[u];
      if (x < nb_off) sh.b_off[x] = kb[u];
    }
  }
  __syncthreads();

  // ---- 3. prefix cache of every key whose offsets are in LDS: 8 bytes at
  // offset 0, or after the common prefix of all of them when that is at
  // least 8 bytes long (all loads, then all stores) ----
  auto load_cache = [&](uint32_t cp) {
    constexpr int kPer = IPT + 1;  // ceil((kTile + 3) / kMlBlock)
    fill_prefix_caches<kMlBlock, kPer>(PfxSide{sh.a_off, na_off, A.keys, sh.u.m.a_pfx},
                                       PfxSide{sh.b_off, nb_off, B.keys, sh.u.m.b_pfx}, cp);
  };
  load_cache(0);
  __syncthreads();
  const uint32_t cp = cache_offset(sh.a_off, na_off - 1, sh.b_off, nb_off - 1, sh.u.m.a_pfx, sh.u.m.b_pfx, A.keys,
                                   B.keys, &sh.cp);
  if (cp) {  // (uniform)
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
  const uint32_t kept = merge_slice<IPT>(ao, bo, apf, bpf, A.keys, 0u, B.keys, 0u, k, len, nA_t, nB_t,
                                         has_next_b, i0, A.n, j0, refs, sh.notes, cp,
                                         __builtin_amdgcn_readfirstlane(sh.try_fast) != 0,
                                         fast_merge_records(tile) ? fast_stat : nullptr);
  // prefixes of this thread's outputs, and (thread 0) of the keys before the
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
  uint32_t ord = block_exclusive_scan<uint32_t, kMlBlock>(kept, sh.scan32, n_kept);
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
  uint32_t klen[IPT], l[IPT], kprev[IPT], vlen[IPT], sref[IPT];
  bool tomb[IPT];
  // value lengths and tombstone flags from HBM, all issued before the LCPs
  uint32_t v0[IPT], v1[IPT];
  uint8_t tv[IPT];
#pragma unroll
  for (int u = 0; u < IPT; ++u) {
    const uint32_t x = tid + u * kMlBlock;
    const uint32_t ref = x < n_kept ? sh.u.c.surv[x] : 0u;
    sref[u] = ref;
    const bool isB = ref >= A.n;
    const uint32_t idx = isB ? ref - A.n : ref;
    const uint32_t* vo = isB ? B.val_off : A.val_off;
    const uint8_t* tb = isB ? B.tomb : A.tomb;
    // (read once: streamed past the caches, which keeps the partition's key
    // lines there longer for the checks and LCPs; measured 2% faster; the key
    // offsets were slower so)
    v0[u] = __builtin_nontemporal_load(vo + idx);
    v1[u] = __builtin_nontemporal_load(vo + idx + 1);
    // (a side without tombstone flags reads a byte it then ignores)
    tv[u] = *(tb ? tb + idx : reinterpret_cast<const uint8_t*>(vo + idx));
  }
#pragma unroll
  for (int u = 0; u < IPT; ++u) {
    const uint32_t x = tid + u * kMlBlock;
    klen[u] = l[u] = kprev[u] = vlen[u] = 0;
    tomb[u] = false;
    if (x >= n_kept) continue;
    const uint32_t ref = sref[u];
    const bool isB = ref >= A.n;
    const bool t = (isB ? B.tomb : A.tomb) != nullptr && tv[u] != 0;
    const uint8_t* xb = isB ? B.keys : A.keys;
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
    tomb[u] = t;
    vlen[u] = t ? 0u : v1[u] - v0[u];
  }

  // ---- 6. survivor base (look-back) ----
  if (tid < kWave) {
    const uint64_t g = lookback_resolve(desc_s, tile, n_kept);
    if (tid == 0) sh.g0 = static_cast<uint32_t>(g);
  }
  __syncthreads();
  const uint32_t g0 = __builtin_amdgcn_readfirstlane(sh.g0);

  // ---- 7. controls, exact lengths, partition-local bit offsets ----
  uint32_t rlen[IPT];
#pragma unroll
  for (int u = 0; u < IPT; ++u) {
    const uint32_t x = tid + u * kMlBlock;
    rlen[u] = 0;
    if (x >= n_kept) continue;
    const uint32_t kb = 8u * klen[u];
    const uint32_t c = ((g0 + x) % 15u == 0) ? 1u + l[u] : kprev[u] - l[u];
    rlen[u] = eg0_len(c) + eg0_len(kb - l[u]) + (kb - l[u]) +
              (tomb[u] ? 1u : 1u + eg0_len(vlen[u]) + 8u * vlen[u]);
  }
  // survivors tid, tid + 512, ...: one scan over the rounds
  uint64_t tile_bits, sb[IPT], rl[IPT];
#pragma unroll
  for (int u = 0; u < IPT; ++u) rl[u] = rlen[u];
  block_exclusive_scan_rounds<uint64_t, kMlBlock, IPT>(rl, sh.scan64, sb, tile_bits);

  // ---- 8. outputs ----
  const uint64_t tag = static_cast<uint64_t>(tile) << kTiledShift;
#pragma unroll
  for (int u = 0; u < IPT; ++u) {
    const uint32_t x = tid + u * kMlBlock;
    if (x >= n_kept) continue;
    __builtin_nontemporal_store(sref[u], out.final_refs + g0 + x);
    __builtin_nontemporal_store(l[u], out.lcp_bits + g0 + x);
    __builtin_nontemporal_store(tag | sb[u], out.toff + g0 + x);
    if (out.len_bits) out.len_bits[g0 + x] = rlen[u];
  }
  if (out.ord_A)
    for (uint32_t x = tid; x < nA_t; x += kMlBlock) {
      const uint32_t o = sh.u.c.ords[x];
      out.ord_A[i0 + x] = o == EM_NONE ? EM_NONE : g0 + o;
    }
  if (out.ord_B)
    for (uint32_t y = tid; y < nB_t; y += kMlBlock) out.ord_B[j0 + y] = g0 + sh.u.c.ords[nA_t + y];
  if (tid == 0) {
    out.tile_bits[tile] = tile_bits;
    if (tile == P - 1) out.d_S[0] = g0 + n_kept;
  }
}

// Exclusive scan of the partitions' bit totals into bit bases (one
// workgroup; P is at most 2^16), and T.  Up to 8192 partitions (8M+8M at
// 2048 outputs each is 7,813) a thread's values are loaded at once and kept
// in registers: the kernel is a chain of latencies, and a loop of dependent
// loads, read twice, took 11 us.
constexpr int kTsBlock = 1024;
constexpr uint32_t kTsRegs = 8;

__global__ __launch_bounds__(kTsBlock) void k_tile_scan(const uint64_t* __restrict__ tile_bits, uint32_t P,
                                                        uint64_t* __restrict__ tbase, uint64_t* __restrict__ d_T) {
  __shared__ uint64_t scan[kTsBlock / kWave + 1];
  const uint32_t tid = threadIdx.x;
  const uint32_t per = (P + kTsBlock - 1) / kTsBlock;
  const uint32_t lo = min(tid * per, P), hi = min(lo + per, P);
  uint64_t total;
  if (per <= kTsRegs) {  // (uniform)
    uint64_t v[kTsRegs];
    uint64_t sum = 0;
#pragma unroll
    for (uint32_t q = 0; q < kTsRegs; ++q) {
      v[q] = lo + q < hi ? tile_bits[lo + q] : 0ull;
      sum += v[q];
    }
    uint64_t acc = block_exclusive_scan<uint64_t, kTsBlock>(sum, scan, total);
#pragma unroll
    for (uint32_t q = 0; q < kTsRegs; ++q) {
      if (lo + q < hi) tbase[lo + q] = acc;
      acc += v[q];
    }
  } else {
    uint64_t sum = 0;
    for (uint32_t t = lo; t < hi; ++t) sum += tile_bits[t];
    uint64_t acc = block_exclusive_scan<uint64_t, kTsBlock>(sum, scan, total);
    for (uint32_t t = lo; t < hi; ++t) {
      const uint64_t v = tile_bits[t];
      tbase[t] = acc;
      acc += v;
    }
  }
  if (tid == 0) d_T[0] = total;
}

struct MlLayout {
  uint32_t* ticket;  // [0]: partition ticket of k_merge_len; from [kEmitCtrStride]: the emitter's
                     // counters; [kMlStatWord]: the merge statistics (u64)
  uint64_t* desc_s;
  uint64_t* tile_bits;
  uint64_t* tbase;
  uint32_t* refs;  // used when the caller passes no final_refs
  uint32_t* lcp;   // used when the caller passes no lcp_bits
  uint64_t* toff;
};

MlLayout ml_layout(void* ws, uint32_t N, uint32_t items) {
  const size_t P = items ? (static_cast<size_t>(N) + items - 1) / items : 0;
  WsCursor cur{static_cast<uint8_t*>(ws), 0};
  MlLayout L;
  L.ticket = cur.take<uint32_t>(kMlTicketWords);
  L.desc_s = cur.take<uint64_t>(P ? P : 1);
  L.tile_bits = cur.take<uint64_t>(P ? P : 1);
  L.tbase = cur.take<uint64_t>(P ? P : 1);
  L.refs = cur.take<uint32_t>(N ? N : 1);
  L.lcp = cur.take<uint32_t>(N ? N : 1);
  L.toff = cur.take<uint64_t>(N ? N : 1);
  return L;
}

size_t ml_ws_bytes(uint32_t N, uint32_t items) {
  const size_t P = items ? (static_cast<size_t>(N) + items - 1) / items : 0;
  const size_t p = P ? P : 1, n = N ? N : 1;
  return align_up(kMlTicketWords * 4, 256) + 3 * align_up(p * 8, 256) + 2 * align_up(n * 4, 256) +
         align_up(n * 8, 256);
}

template <int IPT>
static void launch_ml(const em_side_t& A, const em_side_t& B, const uint32_t* csplits, uint32_t coarse,
                      uint32_t items, uint32_t P, const MlOut& o, const MlLayout& L, hipStream_t st) {
  hipLaunchKernelGGL((k_merge_len<IPT>), dim3(P), dim3(kMlBlock), 0, st, A, B, csplits, coarse, items, P,
                     o, L.ticket, L.desc_s);
}

static void launch_ml_items(const em_side_t& A, const em_side_t& B, const uint32_t* csplits, uint32_t coarse,
                            uint32_t items, uint32_t P, const MlOut& o, const MlLayout& L, hipStream_t st) {
  if (items <= static_cast<uint32_t>(kMlBlock))
    launch_ml<1>(A, B, csplits, coarse, items, P, o, L, st);
  else if (items <= 2u * kMlBlock)
    launch_ml<2>(A, B, csplits, coarse, items, P, o, L, st);
  else
    launch_ml<4>(A, B, csplits, coarse, items, P, o, L, st);
}

}  // namespace em

using namespace em;

extern "C" size_t em_merge_fc_workspace_bytes(uint32_t nA, uint32_t nB, uint32_t items_per_part) {
  const uint64_t N = static_cast<uint64_t>(nA) + nB;
  return ml_ws_bytes(N >= EM_MAX_RECORDS ? EM_MAX_RECORDS : static_cast<uint32_t>(N),
                     items_per_part ? items_per_part : 1);
}

// Checks shared by the entry points below.
static int ml_check(const em_side_t* A, const em_side_t* B, uint32_t items_per_part, const void* ws,
                    size_t ws_bytes) {
  int rc = check_pair(A, B);
  if (rc) return rc;
  if (!ws || items_per_part == 0 || items_per_part > kMlMaxItems) return EM_EINVAL;
  if (reinterpret_cast<uintptr_t>(ws) & 255) return EM_EINVAL;
  if (ws_bytes < ml_ws_bytes(A->n + B->n, items_per_part)) return EM_ENOSPC;
  return EM_OK;
}

extern "C" int em_merge_lengths(const em_side_t* A, const em_side_t* B, const uint32_t* coarse_splits,
                                uint32_t coarse_items, uint32_t items_per_part, uint32_t* d_S, uint64_t* d_T,
                                uint32_t* final_refs, uint32_t* ord_A, uint32_t* ord_B, uint32_t* len_bits,
                                uint32_t* lcp_bits, void* ws, size_t ws_bytes, void* stream) {
  int rc = ml_check(A, B, items_per_part, ws, ws_bytes);
  if (rc) return rc;
  if (!coarse_splits || !d_S || !d_T) return EM_EINVAL;
  if (coarse_items == 0 || coarse_items % items_per_part || coarse_items > EM_MAX_ITEMS_PER_PART * 256u)
    return EM_EINVAL;
  hipStream_t st = as_stream(stream);
  const uint32_t N = A->n + B->n;
  if (N == 0) {
    clear_u32(d_S, 1, st);
    clear_u64(d_T, 1, st);
    return check_launch();
  }
  const uint32_t P = (N + items_per_part - 1) / items_per_part;
  const MlLayout L = ml_layout(ws, N, items_per_part);
  clear_lookback(L.ticket, kMlTicketWords, L.desc_s, nullptr, P, st);
  MlOut o{d_S, final_refs ? final_refs : L.refs, lcp_bits ? lcp_bits : L.lcp, L.toff, L.tile_bits,
          ord_A, ord_B, len_bits};
  launch_ml_items(*A, *B, coarse_splits, coarse_items, items_per_part, P, o, L, st);
  hipLaunchKernelGGL(k_tile_scan, dim3(1), dim3(kTsBlock), 0, st, L.tile_bits, P, L.tbase, d_T);
  return check_launch();
}

extern "C" int em_emit_merged(const em_side_t* A, const em_side_t* B, uint32_t items_per_part,
                              uint32_t* payload, uint64_t payload_words, const uint32_t* d_S,
                              const uint64_t* d_T, const uint32_t* final_refs, const uint32_t* lcp_bits,
                              uint64_t* off, void* ws, size_t ws_bytes, void* stream) {
  int rc = ml_check(A, B, items_per_part, ws, ws_bytes);
  if (rc) return rc;
  if (!payload || !d_S || !d_T) return EM_EINVAL;
  if (reinterpret_cast<uintptr_t>(payload) & 15) return EM_EINVAL;
  uint64_t bound = 0;
  rc = em_payload_bound_bits(A, B, &bound);
  if (rc) return rc;
  if (payload_words < (bound + 31) / 32) return EM_ENOSPC;
  hipStream_t st = as_stream(stream);
  const uint32_t N = A->n + B->n;
  if (N == 0) {
    if (off) clear_u64(off, 1, st);
    return check_launch();
  }
  const MlLayout L = ml_layout(ws, N, items_per_part);
  return emit_launch_dev(*A, *B, final_refs ? final_refs : L.refs, lcp_bits ? lcp_bits : L.lcp, L.toff,
                         L.tbase, off, payload, d_S, d_T, L.ticket + kEmitCtrStride, st);
}

extern "C" int em_merge_fc(const em_side_t* A, const em_side_t* B, const uint32_t* coarse_splits,
                           uint32_t coarse_items, uint32_t items_per_part, uint32_t* payload,
                           uint64_t payload_words, uint32_t* d_S, uint64_t* d_T, uint32_t* final_refs,
                           uint32_t* ord_A, uint32_t* ord_B, uint32_t* len_bits, uint32_t* lcp_bits,
                           uint64_t* off, void* ws, size_t ws_bytes, void* stream) {
  // every check of the second half first, so that an error leaves nothing enqueued
  int rc = ml_check(A, B, items_per_part, ws, ws_bytes);
  if (rc) return rc;
  if (!payload || !coarse_splits || !d_S || !d_T) return EM_EINVAL;
  if (reinterpret_cast<uintptr_t>(payload) & 15) return EM_EINVAL;
  uint64_t bound = 0;
  rc = em_payload_bound_bits(A, B, &bound);
  if (rc) return rc;
  if (payload_words < (bound + 31) / 32) return EM_ENOSPC;
  rc = em_merge_lengths(A, B, coarse_splits, coarse_items, items_per_part, d_S, d_T, final_refs, ord_A, ord_B,
                        len_bits, lcp_bits, ws, ws_bytes, stream);
  if (rc) return rc;
  return em_emit_merged(A, B, items_per_part, payload, payload_words, d_S, d_T, final_refs, lcp_bits, off, ws,
                        ws_bytes, stream);
}
