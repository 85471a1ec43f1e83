/*
 * em.h -- C ABI of the MI355X (gfx950) replacement merge into a front-coded
 * bit payload.
 *
 * Two strictly sorted, unique-key string record sets are merged: an older
 * side A and a newer side B.  On an equal key the newer record wins and a
 * newer tombstone stays a record.  The survivors are front coded into one
 * canonical MSB-first bit payload.  The calls, in order:
 *
 *   em_partition -> em_merge_keep (or em_collision_rank) -> em_fc_lengths
 *                -> em_scan -> em_emit
 *
 * Between them the host reads the survivor count S (after the merge) and the
 * payload length T in bits (after the scan), as the pages' host does.
 *
 * Conventions for every call:
 *  - All buffer pointers are DEVICE pointers unless a parameter says "host".
 *    The caller owns all memory; the library never allocates, frees or
 *    synchronises.  Work is enqueued on `stream` (a hipStream_t; NULL = the
 *    default stream) and completes asynchronously: inputs must stay alive and
 *    unchanged, and outputs must not be read, until the stream has reached the
 *    call's work.
 *  - `ws` is caller-owned device scratch of `ws_bytes` bytes, 256-byte
 *    aligned, at least em_workspace_bytes() for the same sizes.  Its contents
 *    on entry do not matter and are undefined on return.
 *  - Every call returns EM_OK or a negative EM_E* code.  On error nothing
 *    defined has been written and the outputs must not be used or published
 *    (Everett, "GPU construction experiment": a failed construction is not
 *    permission to publish).  Argument errors are detected before any work is
 *    enqueued.
 *  - Inputs are trusted, not admitted (Everett, "Byte-profile GPU merge",
 *    "Pipeline"): each side must be strictly increasing in unsigned bytewise
 *    order with a proper prefix first.  On input that breaks this the output
 *    is unspecified and memory safety is not guaranteed (some kernels clamp
 *    references and partition splits, but not every call is guarded); a
 *    caller with untrusted input must check its order first.
 *  - Caps (Everett, "GPU construction experiment", the host bound check, and
 *    "Byte-profile GPU merge", "Pipeline"): |A| + |B| < 2^24 records; each
 *    arena < 2^32 bytes (u32 offsets); key and value lengths < 2^27 bytes.
 *    Bit offsets and payload lengths are 64-bit, which lifts the pages'
 *    2 Gibit prototype cap.
 */
#ifndef EM_H
#define EM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EM_OK 0
#define EM_EINVAL (-1)  /* null, misaligned or inconsistent argument */
#define EM_ERANGE (-2)  /* a cap is exceeded */
#define EM_ENOSPC (-3)  /* workspace or output capacity too small */
#define EM_EDEVICE (-4) /* a HIP call failed; em_last_hip_error() has its code */

#define EM_NONE 0xFFFFFFFFu          /* ordinal of a replaced (dropped) A record */
#define EM_MAX_RECORDS (1u << 24)    /* |A| + |B| must be below this */
#define EM_MAX_FIELD_BYTES (1u << 27) /* key and value lengths must be below this */
#define EM_ARENA_PAD 32u             /* readable bytes required past each arena's end */
#define EM_MAX_ITEMS_PER_PART 4096u  /* largest merge tile (outputs per partition) */

/*
 * One input side.  Record r has key bytes keys[key_off[r] .. key_off[r+1])
 * and value bytes vals[val_off[r] .. val_off[r+1]).  tomb[r] != 0 marks a
 * tombstone (its value bytes are ignored); tomb may be NULL (no tombstones).
 * key_off and val_off have n+1 non-decreasing entries starting at 0.
 * keys and vals must be 16-byte aligned and readable for key_bytes +
 * EM_ARENA_PAD (resp. val_bytes + EM_ARENA_PAD) bytes; the pad's contents are
 * never used.  key_bytes and val_bytes are host copies of key_off[n] and
 * val_off[n].
 */
typedef struct {
  const uint8_t *keys;
  const uint32_t *key_off;
  const uint8_t *vals;
  const uint32_t *val_off;
  const uint8_t *tomb;
  uint32_t n;
  uint64_t key_bytes;
  uint64_t val_bytes;
} em_side_t;

/* Device scratch in bytes needed by every call below for these sizes
 * (host only, enqueues nothing).  items_per_part as for em_partition. */
size_t em_workspace_bytes(uint32_t nA, uint32_t nB, uint32_t items_per_part);

/*
 * Host only.  A conservative upper bound on T, the payload length in bits:
 * 8 * (all key and value arena bytes) + (|A| + |B|) * 184, since each record
 * spends at most 61 bits on each of EG0(c), EG0(k-l) and EG0(value length)
 * plus one presence bit under the caps (Everett, "GPU construction
 * experiment": the output is sized on the host from an upper bound before any scan).
 * Writes *bound (host pointer).  EM_EINVAL on NULL arguments, EM_ERANGE when a
 * cap is exceeded.
 */
int em_payload_bound_bits(const em_side_t *A, const em_side_t *B, uint64_t *bound);

/*
 * Merge-path partition ("CUDA merge path: merging sorted arrays in
 * parallel", "The merge matrix, and the diagonal that cuts it"; Everett,
 * "GPU construction experiment", the merge paragraph).  For p = 0..P with
 * P = ceil(N / items_per_part), N = |A| + |B|, writes splits[p] = the co-rank
 * of diagonal d_p = min(p * items_per_part, N): the number of A records among
 * the first d_p outputs of the stable merge in which equal keys put A first.
 * splits: P+1 u32.  items_per_part >= 1 (em_merge_keep needs at most
 * EM_MAX_ITEMS_PER_PART; em_merge_fc takes coarser splits).
 */
int em_partition(const em_side_t *A, const em_side_t *B, uint32_t items_per_part, uint32_t *splits,
                 void *ws, size_t ws_bytes, void *stream);

/*
 * Stable merge and keep-newer scan (Everett, "GPU construction experiment",
 * the merge paragraph and the paragraph on the compacted order).  Merges each
 * partition of em_partition's splits (same items_per_part), drops every A
 * record whose key equals the next merged record's key, and compacts the
 * survivors in merged order.  A reference names a record: A_i -> i,
 * B_j -> |A| + j.  Writes:
 *   final_refs[0..S)  survivors' references in output order (capacity N);
 *   ord_A[|A|]        output ordinal of A_i, or EM_NONE if replaced (nullable);
 *   ord_B[|B|]        output ordinal of B_j (nullable);
 *   d_S[0]            S, the survivor count (device u32).
 */
int em_merge_keep(const em_side_t *A, const em_side_t *B, const uint32_t *splits,
                  uint32_t items_per_part, uint32_t *final_refs, uint32_t *ord_A, uint32_t *ord_B,
                  uint32_t *d_S, void *ws, size_t ws_bytes, void *stream);

/*
 * Collision-bitmap variant of the keep step (Everett, "Collision bitmap and
 * rank experiment", "Corrected record ordinals", "Temporary rank layouts" and
 * "The three experimental paths").  Clears a bitmap over A, marks bit C_i by
 * atomic OR when lower_bound(A, B_j) = i holds an equal key, builds the
 * temporary rank512 directory (count, scan, finish), and places B_j at
 * j + lb_j - R(lb_j) and each surviving A_i at i + lb(B, A_i) - R(i), where
 * R is the exclusive collision rank; A is handled in tiles of 32 consecutive
 * records with one search and a monotone cursor.  Same outputs and meaning as
 * em_merge_keep (ord_A / ord_B nullable); needs no partition.
 */
int em_collision_rank(const em_side_t *A, const em_side_t *B, uint32_t *final_refs, uint32_t *ord_A,
                      uint32_t *ord_B, uint32_t *d_S, void *ws, size_t ws_bytes, void *stream);

/*
 * The collision variants side by side (same page: "The three experimental
 * paths" and the suggested modes collision512, collision2048,
 * collision512-tiled and collision512-compact).  Every mode marks collisions
 * and saves B's lower bounds as em_collision_rank does, and gives the same
 * outputs; they differ in the rank directory and in how A is placed:
 *   EM_COLLISION_512          rank512; each surviving A_i binary-searches B's
 *                             keys for lower_bound(B, A_i);
 *   EM_COLLISION_2048         the same with the rank2048 directory (one 8-byte
 *                             entry per 2048 bits: 32-bit absolute prefix and
 *                             the populations before its 512-bit runs 1..3);
 *   EM_COLLISION_512_TILED    rank512; A in tiles of 32 (em_collision_rank);
 *   EM_COLLISION_512_COMPACT  rank512; surviving A references are compacted
 *                             to i - R(i), then merged with B by Merge Path
 *                             (their key sets are disjoint).
 * ws: em_collision_workspace_bytes(|A|, |B|, mode), 256-byte aligned (the
 * compact mode adds 4|A| bytes).  An unknown mode is EM_EINVAL.
 */
#define EM_COLLISION_512 0u
#define EM_COLLISION_2048 1u
#define EM_COLLISION_512_TILED 2u
#define EM_COLLISION_512_COMPACT 3u
size_t em_collision_workspace_bytes(uint32_t nA, uint32_t nB, uint32_t mode);
int em_collision_rank_mode(const em_side_t *A, const em_side_t *B, uint32_t mode, uint32_t *final_refs,
                           uint32_t *ord_A, uint32_t *ord_B, uint32_t *d_S, void *ws, size_t ws_bytes,
                           void *stream);

/*
 * Exact record lengths (Everett, "GPU construction experiment": the c_i
 * control equation and the record grammar paragraph).  For survivor i with
 * key length k_i bits and exact bit LCP l_i with survivor i-1 (l_0 = 0,
 * clamped to the shorter key): c_i = 1 + l_i when i mod 15 = 0, else
 * k_{i-1} - l_i; v_i = 1 for a tombstone, else 1 + E(len) + 8 len;
 * len_bits[i] = E(c_i) + E(k_i - l_i) + (k_i - l_i) + v_i with
 * E(x) = 2 floor(log2(x+1)) + 1.  S is the host value read from d_S.
 * len_bits: S u32.  lcp_bits: S u32 receiving l_i (nullable; em_emit reuses it).
 */
int em_fc_lengths(const em_side_t *A, const em_side_t *B, const uint32_t *final_refs, uint32_t S,
                  uint32_t *len_bits, uint32_t *lcp_bits, void *ws, size_t ws_bytes, void *stream);

/*
 * Exclusive scan of record lengths into 64-bit bit offsets (Everett, "GPU
 * construction experiment": one global scan, no per-chunk reset).
 * off: S+1 u64; off[0] = 0, off[i+1] = off[i] + len_bits[i], off[S] = T.
 */
int em_scan(const uint32_t *len_bits, uint32_t S, uint64_t *off, void *ws, size_t ws_bytes,
            void *stream);

/*
 * em_scan for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same scan and result, with the look-back state in a fixed device array of
 * the library (33,024 bytes per device, held until the process ends) instead
 * of a workspace.  Allocates nothing.  S must be below EM_MAX_RECORDS
 * (EM_ERANGE otherwise).  Every call on one device shares that device's
 * array: calls that overlap on one device (other streams, other host
 * threads) race and must not be issued; calls in order on one stream are
 * fine (each clears the state it needs).
 */
int em_scan_noalloc(const uint32_t *len_bits, uint32_t S, uint64_t *off, void *stream);

/*
 * Word-owned payload emission (Everett, "GPU construction experiment": every
 * 32-bit output word has a single writer, which collects all of its bits and
 * stores it one time; bits run most significant first; records follow each
 * other with no gaps; the bits after the last record are zero; the key suffix
 * comes from the source record's own key).  Record i occupies bits [off[i], off[i+1]):
 * EG0(c_i) EG0(k_i - l_i) key bits [l_i, k_i) then 0 (tombstone) or
 * 1 EG0(value length) value bytes.  EG0(x) is floor(log2(x+1)) zero bits
 * followed by x+1 in binary.  Stream bit p is bit 7 - (p mod 8) of payload
 * byte p / 8, so each u32 word holds four consecutive stream bytes.
 * Writes exactly ceil(T / 32) words; payload_words is the capacity.
 * lcp_bits from em_fc_lengths (nullable: recomputed when NULL).  T is the host
 * value off[S].
 */
int em_emit(const em_side_t *A, const em_side_t *B, const uint32_t *final_refs,
            const uint32_t *lcp_bits, uint32_t S, const uint64_t *off, uint64_t T, uint32_t *payload,
            uint64_t payload_words, void *ws, size_t ws_bytes, void *stream);

/*
 * First half of the whole path (Everett, "GPU construction experiment": merge
 * by diagonal partitions, keep-newer, exact lengths, one global scan of bit
 * offsets).  One workgroup per partition of items_per_part (1..2048) merged
 * outputs finds its co-ranks inside the coarse partition given by
 * coarse_splits (em_partition's output for coarse_items, a multiple of
 * items_per_part; read directly when coarse_items == items_per_part),
 * merges, keeps the newer record, and computes LCPs, exact lengths and
 * partition-local bit offsets, taking its survivor base from a decoupled
 * look-back; one workgroup then scans the partitions' bit totals.  Writes
 * d_S[0] (u32) and d_T[0] (u64), the optional (nullable) per-record arrays
 * final_refs, ord_A, ord_B, len_bits, lcp_bits of the separate calls, and,
 * in the workspace, what em_emit_merged reads (record offsets in partition
 * form, partition bit bases; final_refs and lcp_bits when those are NULL).
 * The workspace (em_merge_fc_workspace_bytes, 256-byte aligned) is about 16
 * bytes per record.
 */
int em_merge_lengths(const em_side_t *A, const em_side_t *B, const uint32_t *coarse_splits,
                     uint32_t coarse_items, uint32_t items_per_part, uint32_t *d_S, uint64_t *d_T,
                     uint32_t *final_refs, uint32_t *ord_A, uint32_t *ord_B, uint32_t *len_bits,
                     uint32_t *lcp_bits, void *ws, size_t ws_bytes, void *stream);

/*
 * Second half: word-owned emission (as em_emit) after em_merge_lengths on the
 * same stream, with the same A, B, items_per_part, workspace, final_refs and
 * lcp_bits (NULL where em_merge_lengths got NULL).  Reads S and T from d_S and
 * d_T; a fixed grid of resident workgroups walks the records.  Writes
 * payload[ceil(T/32)] (payload_words is the capacity and must cover
 * em_payload_bound_bits; 16-byte aligned) and, when off is not NULL, the S+1
 * bit offsets of em_scan.  Nothing has to be read by the host in between.
 */
int em_emit_merged(const em_side_t *A, const em_side_t *B, uint32_t items_per_part, uint32_t *payload,
                   uint64_t payload_words, const uint32_t *d_S, const uint64_t *d_T,
                   const uint32_t *final_refs, const uint32_t *lcp_bits, uint64_t *off, void *ws,
                   size_t ws_bytes, void *stream);

/*
 * The whole path in one call: em_merge_lengths then em_emit_merged, with the
 * same arguments (every argument is checked before anything is enqueued).
 * Writes the payload, d_S, d_T and the optional (nullable) per-record arrays
 * final_refs, ord_A, ord_B, len_bits, lcp_bits, off of the separate calls.
 */
size_t em_merge_fc_workspace_bytes(uint32_t nA, uint32_t nB, uint32_t items_per_part);
int em_merge_fc(const em_side_t *A, const em_side_t *B, const uint32_t *coarse_splits,
                uint32_t coarse_items, uint32_t items_per_part, uint32_t *payload,
                uint64_t payload_words, uint32_t *d_S, uint64_t *d_T, uint32_t *final_refs,
                uint32_t *ord_A, uint32_t *ord_B, uint32_t *len_bits, uint32_t *lcp_bits,
                uint64_t *off, void *ws, size_t ws_bytes, void *stream);

/*
 * The whole path in one pass (Everett, "GPU construction experiment": the
 * same steps; each output word is written once; the prefix cache holds the
 * eight key bytes after the common prefix the compared keys share).  One
 * workgroup per partition of items_per_part (1..1024) merged outputs finds
 * the partition's co-ranks inside the coarse partition of coarse_splits
 * (em_partition's output for coarse_items, a multiple of items_per_part),
 * merges with keep-newer, computes LCPs and exact lengths, takes its survivor
 * base and its bit base from two decoupled look-backs over the partitions,
 * and writes its records' payload words itself; a small second kernel writes
 * the words that partition boundaries cut.  Results as em_merge_fc: the
 * payload (16-byte aligned, payload_words covering em_payload_bound_bits),
 * d_S, d_T and the optional (nullable) per-record arrays final_refs, ord_A,
 * ord_B, len_bits, lcp_bits, off.  ws: em_onepass_workspace_bytes(|A|, |B|,
 * items_per_part) bytes, 256-byte aligned (about 40 bytes per partition).
 */
size_t em_onepass_workspace_bytes(uint32_t nA, uint32_t nB, uint32_t items_per_part);
int em_merge_fc_onepass(const em_side_t *A, const em_side_t *B, const uint32_t *coarse_splits,
                        uint32_t coarse_items, uint32_t items_per_part, uint32_t *payload,
                        uint64_t payload_words, uint32_t *d_S, uint64_t *d_T, uint32_t *final_refs,
                        uint32_t *ord_A, uint32_t *ord_B, uint32_t *len_bits, uint32_t *lcp_bits,
                        uint64_t *off, void *ws, size_t ws_bytes, void *stream);

/*
 * Rank512 probe (Everett, "Collision bitmap and rank experiment",
 * "Validation and measurement plan": compare GPU rank queries against scalar
 * prefix counts).  Builds the same temporary rank512 directory that
 * em_collision_rank uses from `bitmap` (nbits bits; bit q is bit q mod 32 of
 * u32 word q / 32; bits >= nbits are ignored) and writes, for each of the
 * npos positions p <= nbits, out[t] = number of set bits below p.
 * nbits < 2^24 + 2^13.
 */
int em_rank512_probe(const uint32_t *bitmap, uint32_t nbits, const uint32_t *positions, uint32_t npos,
                     uint32_t *out, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes em_rank512_probe needs for nbits bits (host only). */
size_t em_rank512_workspace_bytes(uint32_t nbits);

/*
 * The same probe for the rank2048 directory of EM_COLLISION_2048 (same page,
 * "Temporary rank layouts": an 8-byte directory entry per 2048 bits with the
 * populations of its 512-bit runs; queries read up to eight bitmap words).
 * Arguments, limits and errors as em_rank512_probe; workspace
 * em_rank2048_workspace_bytes(nbits).
 */
int em_rank2048_probe(const uint32_t *bitmap, uint32_t nbits, const uint32_t *positions, uint32_t npos,
                      uint32_t *out, void *ws, size_t ws_bytes, void *stream);
size_t em_rank2048_workspace_bytes(uint32_t nbits);

/*
 * Output navigation (Everett, "GPU construction experiment": the KV03
 * paragraph and the output-EF paragraph).  The record offsets are sampled at
 * ordinals 0, 15, 30, ... and at EOF (n = em_ef_entry_count(S) =
 * ceil(S/15) + 1 entries; the last is T); when every survivor's encoded value
 * has the same width w (1 for a tombstone, else 1 + E(len) + 8 len), w times
 * the ordinal is subtracted.  The entries are Elias-Fano coded:
 *   L = floor(log2(floor((e_{n-1} + 1) / n))), 0 when that quotient is 0;
 *   lows[]:       entry k's low L bits at bit k L (bit b is bit b mod 64 of
 *                 u64 word b / 64);
 *   highs[]:      bit (e_k >> L) + k set, n + (e_{n-1} >> L) bits;
 *   samples[]:    per group of 256 entries the pair (position of its first
 *                 high bit, exception entries of the groups before it);
 *   exceptions[]: the high-bit position of every entry of each group whose
 *                 positions span at least 4096 bits, in order.
 * Unused bits of the last low and high words are zero; words past the
 * lengths in *info are not written.  info (device memory) receives n, L, w
 * and the section lengths (low_words, high_bits, high_words, groups,
 * exceptions).  Each output's capacity in u64 words comes from
 * em_ef_capacity(n) (at most n, ceil(3n/64), 2 ceil(n/256), n), and the
 * workspace from em_ef_workspace_bytes(n) (256-byte aligned).  Capacities too
 * small: EM_ENOSPC.
 *
 * em_ef_navigation: from the survivors (final_refs, S), their offsets
 * off[0..S] and T, after em_scan / em_emit (or em_emit_merged with off).
 * S = 0 needs T = 0 and gives the one entry 0.
 * em_ef_encode: from n explicit non-decreasing entries (width is recorded
 * in info only); n >= 1.
 */
typedef struct {
  uint64_t n, L, width, low_words, high_bits, high_words, groups, exceptions;
} em_ef_info_t;
uint32_t em_ef_entry_count(uint32_t S);
int em_ef_capacity(uint32_t n_entries, uint64_t *low_words, uint64_t *high_words, uint64_t *sample_words,
                   uint64_t *exception_words);
size_t em_ef_workspace_bytes(uint32_t n_entries);
int em_ef_navigation(const em_side_t *A, const em_side_t *B, const uint32_t *final_refs, uint32_t S,
                     const uint64_t *off, uint64_t T, uint64_t *lows, uint64_t low_cap, uint64_t *highs,
                     uint64_t high_cap, uint64_t *samples, uint64_t sample_cap, uint64_t *exceptions,
                     uint64_t exception_cap, em_ef_info_t *info, void *ws, size_t ws_bytes, void *stream);
int em_ef_encode(const uint64_t *entries, uint32_t n, uint64_t width, uint64_t *lows, uint64_t low_cap,
                 uint64_t *highs, uint64_t high_cap, uint64_t *samples, uint64_t sample_cap,
                 uint64_t *exceptions, uint64_t exception_cap, em_ef_info_t *info, void *ws, size_t ws_bytes,
                 void *stream);

/*
 * Front-coded input (Everett, "GPU construction experiment": the block-parse
 * paragraph, the literal-owner paragraph j = max{t <= i : r_t <= p} with its
 * minimum tree, and full-key materialization as a consumer of the parsed
 * descriptors).  Decodes a payload of S records and T bits -- as em_emit or
 * em_emit_merged wrote it -- back into the arenas of a side, so that it can
 * be merged again.  Two calls, because the arena sizes are known only after
 * the parse:
 *   em_fcin_parse: block starts from the record offsets off[0..S] when off
 *     is not NULL, else by select on the navigation sections of
 *     em_ef_navigation (nav_info and the four arrays, device memory); one
 *     thread parses each block of at most 15 records (retained length r_i,
 *     key bytes, literal position, value bytes, tombstone flag); the key and
 *     value arena offsets are scanned and a minimum tree over r_i is built.
 *     Writes d_totals[0] = key arena bytes, d_totals[1] = value arena bytes
 *     and d_totals[2] = error bits (0: none; 1: a field past T or a bad
 *     EG0 code, 2: an inherited prefix longer than the predecessor's key,
 *     4: a key that is not whole bytes, 8: a block not ending where the next
 *     starts, 16: an arena of 2^32 bytes or more, 32: an output arena too
 *     small).  d_totals is u64[3] in device memory.
 *   em_fcin_materialize: after the host read d_totals (no errors): writes
 *     keys (key_cap bytes), key_off[S+1], vals (val_cap bytes), val_off[S+1]
 *     and tomb[S]; every inherited key bit comes from its owner's literal.
 *     Arenas smaller than the totals set error bit 32 and leave the
 *     records that do not fit unwritten.
 * payload: u32 words in stream byte order, payload_words >= ceil(T/32).  The
 * same workspace (em_fcin_workspace_bytes(S), 256-byte aligned) must reach
 * both calls unchanged.
 */
size_t em_fcin_workspace_bytes(uint32_t S);
int em_fcin_parse(const uint32_t *payload, uint64_t payload_words, uint64_t T, uint32_t S, const uint64_t *off,
                  const em_ef_info_t *nav_info, const uint64_t *nav_lows, const uint64_t *nav_highs,
                  const uint64_t *nav_samples, const uint64_t *nav_exceptions, uint64_t *d_totals, void *ws,
                  size_t ws_bytes, void *stream);
int em_fcin_materialize(const uint32_t *payload, uint64_t payload_words, uint32_t S, uint8_t *keys,
                        uint64_t key_cap, uint32_t *key_off, uint8_t *vals, uint64_t val_cap, uint32_t *val_off,
                        uint8_t *tomb, uint64_t *d_totals, void *ws, size_t ws_bytes, void *stream);

/*
 * The prefix cache of a front-coded input filled from the literal owners,
 * with no key arena (Everett, "GPU construction experiment", the
 * prefix-cache paragraph -- eight key bytes cached per record -- and the
 * literal-owner paragraph: bit p of key i is the literal bit of
 * j = max{t <= i : r_t <= p}).  After em_fcin_parse on the same payload and
 * workspace (no error bits), writes pfx[i] = the first 8 bytes of key i as a
 * big-endian u64 (first key byte most significant), zero past the key's end,
 * for i in [0, S).  pfx: u64[S] in device memory.  Every value depends only on
 * the parse's outputs, so the call can run in place of, or besides,
 * em_fcin_materialize.  Errors: EM_EINVAL (NULL or misaligned workspace, NULL
 * payload or pfx with S > 0), EM_ERANGE (S >= EM_MAX_RECORDS), EM_ENOSPC
 * (ws_bytes below em_fcin_workspace_bytes(S)).
 */
int em_fcin_prefix8(const uint32_t *payload, uint64_t payload_words, uint32_t S, uint64_t *pfx, void *ws,
                    size_t ws_bytes, void *stream);

/*
 * Owner-search comparison of keys of two front-coded inputs, with no key
 * arena (Everett, "GPU construction experiment", the literal-owner paragraph:
 * bit p of key i is the literal bit of j = max{t <= i : r_t <= p}; a merge of
 * compressed inputs needs such comparisons past its prefix cache, and the
 * page leaves their cost against materialization to measurement).  After
 * em_fcin_parse on each payload (no error bits; input A: payload_a of S_a
 * records with workspace ws_a, input B likewise), for q in [0, n) compares
 * key ia[q] of A with key jb[q] of B from byte from_byte on -- the bytes
 * before it are taken as shared, as when a merge's cached bytes tie -- and
 * writes lcp_bits[q] = the exact bit LCP of the two keys (clamped to the
 * shorter one, counting the skipped bytes) and cmp[q] = -1, 0 or 1, the
 * sign of A's key against B's in unsigned bytewise order with a proper
 * prefix first.  Every key bit is read from its owner's literal in the
 * payload, down the pse chain the parse built.  ia, jb: u32[n]; lcp_bits:
 * u32[n], cmp: i32[n] (either may be NULL, not both), device memory.  An
 * index past its input gives lcp_bits = 0xFFFFFFFF and cmp = 0.  The
 * workspaces are only read.  Errors: EM_EINVAL (NULL or misaligned
 * workspace, NULL payload with records, NULL index arrays or both outputs
 * NULL with n > 0), EM_ERANGE (S_a or S_b >= EM_MAX_RECORDS), EM_ENOSPC (a
 * workspace below em_fcin_workspace_bytes of its S).
 */
int em_fcin_compare(const uint32_t *payload_a, uint64_t words_a, uint32_t S_a, const void *ws_a,
                    size_t ws_a_bytes, const uint32_t *payload_b, uint64_t words_b, uint32_t S_b,
                    const void *ws_b, size_t ws_b_bytes, uint32_t n, const uint32_t *ia, const uint32_t *jb,
                    uint32_t from_byte, uint32_t *lcp_bits, int32_t *cmp, void *stream);

/*
 * Byte-profile front coding (Everett, "Byte-profile GPU merge", "Pipeline":
 * byte LEB128 counts, byte FC literals, optional-value tags, a common encoded
 * value width -- width seventeen is a presence tag and sixteen payload
 * bytes; with the c_i rule of "GPU construction experiment" in bytes).
 * Record: LEB128(c_i), LEB128(k_i - l_i), key bytes l_i .. k_i-1, value;
 * l_i = byte LCP with the preceding survivor (= lcp_bits >> 3), k_i = key
 * bytes, c_i = 1 + l_i when i mod 15 = 0, else k_{i-1} - l_i.  Value: fixed
 * framing when every present value has one byte length L (or none is
 * present): width W = 1 + L, a tag byte (1 present, 0 tombstone) and L bytes
 * (zeros for a tombstone); else W = 0: tag 0, or tag 1, LEB128(length) and the
 * bytes.  LEB128 is unsigned, seven bits a byte, low group first.
 *   em_bp_lengths: d_width[0] (device u32) = W, and len_bytes[S] (u32);
 *     ws: em_bp_workspace_bytes(S), 256-byte aligned.
 *   em_scan over len_bytes gives the byte offsets off[S+1] and T = off[S].
 *   em_bp_emit: the payload bytes (payload_cap >= T); one thread per record.
 *     d_overflow (device u32) is set to 1 when an offset does not match its
 *     record, passes payload_cap, or a present value is not W - 1 bytes under
 *     fixed framing; the payload bytes are then unspecified (nothing is
 *     written at or past payload_cap).
 *   em_bp_navigation: the navigation sections of em_ef_navigation over the
 *     byte offsets, the width taken from d_width (entries off[15k] - 15k W and
 *     T - S W); arguments and capacities as em_ef_navigation.
 * final_refs and lcp_bits are those of the keep step and em_fc_lengths.
 */
size_t em_bp_workspace_bytes(uint32_t S);
int em_bp_lengths(const em_side_t *A, const em_side_t *B, const uint32_t *final_refs, const uint32_t *lcp_bits,
                  uint32_t S, uint32_t *len_bytes, uint32_t *d_width, void *ws, size_t ws_bytes, void *stream);
int em_bp_emit(const em_side_t *A, const em_side_t *B, const uint32_t *final_refs, const uint32_t *lcp_bits,
               uint32_t S, const uint64_t *off, uint64_t T, const uint32_t *d_width, uint8_t *payload,
               uint64_t payload_cap, uint32_t *d_overflow, void *stream);
int em_bp_navigation(const uint64_t *off, uint32_t S, uint64_t T, const uint32_t *d_width, uint64_t *lows,
                     uint64_t low_cap, uint64_t *highs, uint64_t high_cap, uint64_t *samples, uint64_t sample_cap,
                     uint64_t *exceptions, uint64_t exception_cap, em_ef_info_t *info, void *ws, size_t ws_bytes,
                     void *stream);

/* Text for an EM_* code (static string). */
const char *em_strerror(int code);

/* The hipError_t of the most recent EM_EDEVICE return on this thread (0 if none). */
int em_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EM_H */
