/*
 * CPU oracle for the replacement merge into a front-coded bit payload.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * helper with the GPU library.
 *
 * Every function is the plain definition from the pages, written for a reader
 * to check by eye: single thread, one record at a time, one bit at a time.
 * It is deliberately slow.
 *
 * Sources (page title, then the part of it followed):
 *  [MP]  "CUDA merge path: merging sorted arrays in parallel" (100 Days of GPU,
 *        day 36): the sequential loop at the top of the page and "The merge
 *        matrix, and the diagonal that cuts it" (co-rank of output index k).
 *  [DSA] "Chapter 14: Merge Sort and Sample Sort", section 14.1 "Parallel Merge
 *        of Two Sorted Arrays" (two-pointer baseline, co_rank definition).
 *  [GC]  Everett, "GPU construction experiment": the merge paragraph (stable
 *        merge, older first on equal keys, keep-newer scan, tombstones stay),
 *        the control equation for c_i, the record grammar paragraph (EG0
 *        fields, value framing, E(x) and the record length, MSB-first bits,
 *        no padding, word-owned payload with zero unused final bits) and the
 *        prefix-cache paragraph (proper-prefix order, LCP clamped to the
 *        shorter key); the KV03 and output-EF paragraphs for the output
 *        navigation (sampled offsets, common value width, Elias-Fano lows
 *        and highs, 256-entry groups, the 4096-bit sparse threshold); the
 *        block-parse paragraph for decoding a payload back into arenas.
 *  [CB]  Everett, "Collision bitmap and rank experiment": "Corrected record
 *        ordinals" (collision bits, exclusive rank R, ordinal formulas).
 *  [BP]  Everett, "Byte-profile GPU merge": "Pipeline" (byte LEB128 counts,
 *        byte FC literals, optional-value tags, common value width).
 *
 * Readings where the pages leave a step open (each one is listed with its
 * reason in the project's design notes):
 *  - key order is unsigned bytewise lexicographic with a proper prefix first,
 *    which equals MSB-first bitwise order;
 *  - k_i counts key bits (8 per byte); the selector bit the pages keep in the
 *    file dictionary is not part of the payload;
 *  - c_i is used exactly as printed, including c_0 = 1 + l_0 = 1;
 *  - i in "i mod 15" is the global output ordinal; the prefix is never reset;
 *  - EG0(x) is textbook order-0 Exp-Golomb: floor(log2(x+1)) zero bits, then
 *    x+1 in binary, most significant bit first;
 *  - field order: EG0(c), EG0(k-l), key bits l..k-1, value;
 *  - value: tombstone = one 0 bit; present = 1, EG0(byte length), the bytes;
 *  - stream bit p is bit 7-(p mod 8) of byte floor(p/8); the payload is that
 *    byte stream zero padded to a multiple of 4 bytes;
 *  - bit offsets are 64-bit.
 */
#include <stdint.h>
#include <string.h>

typedef struct {
  const uint8_t *keys;     /* key arena */
  const uint32_t *key_off; /* n+1 offsets: key r = keys[key_off[r] .. key_off[r+1]) */
  const uint8_t *vals;     /* value arena */
  const uint32_t *val_off; /* n+1 offsets */
  const uint8_t *tomb;     /* tomb[r] != 0: tombstone; may be NULL (no tombstones) */
  uint32_t n;
} or_side;

#define OR_NONE 0xFFFFFFFFu

static const uint8_t *key_ptr(const or_side *s, uint32_t r) { return s->keys + s->key_off[r]; }
static uint32_t key_len(const or_side *s, uint32_t r) { return s->key_off[r + 1] - s->key_off[r]; }
static int is_tomb(const or_side *s, uint32_t r) { return s->tomb != 0 && s->tomb[r] != 0; }

/* Unsigned bytewise comparison, a proper prefix first.  <0, 0, >0. */
int or_key_cmp(const or_side *X, uint32_t i, const or_side *Y, uint32_t j) {
  const uint8_t *a = key_ptr(X, i), *b = key_ptr(Y, j);
  uint32_t la = key_len(X, i), lb = key_len(Y, j);
  uint32_t m = la < lb ? la : lb;
  for (uint32_t t = 0; t < m; ++t)
    if (a[t] != b[t]) return a[t] < b[t] ? -1 : 1;
  if (la == lb) return 0;
  return la < lb ? -1 : 1;
}

/* A reference names one input record: A_i -> i, B_j -> |A| + j. */
static const or_side *ref_side(const or_side *A, const or_side *B, uint32_t ref, uint32_t *idx) {
  if (ref < A->n) {
    *idx = ref;
    return A;
  }
  *idx = ref - A->n;
  return B;
}

/*
 * [MP] sequential loop, [DSA] two-pointer baseline: take A's head while it is
 * <= B's head, so that ties go to the older side ([GC] merge paragraph).
 * refs has |A|+|B| entries.
 */
void or_merge(const or_side *A, const or_side *B, uint32_t *refs) {
  uint32_t i = 0, j = 0, k = 0;
  while (i < A->n || j < B->n) {
    if (j >= B->n || (i < A->n && or_key_cmp(A, i, B, j) <= 0))
      refs[k++] = i++;
    else
      refs[k++] = A->n + j++;
  }
}

/*
 * [MP] "The merge matrix, and the diagonal that cuts it": the co-rank of output
 * index d is the number of A elements among the first d merged outputs.
 */
uint32_t or_corank(const uint32_t *refs, uint32_t nA, uint32_t d) {
  uint32_t c = 0;
  for (uint32_t k = 0; k < d; ++k)
    if (refs[k] < nA) ++c;
  return c;
}

/*
 * [GC] merge paragraph: comparing each reference's key with the next one's,
 * only the final reference of a run of equal keys is kept, so that the newer
 * record wins (a tombstone is a record like any other).  The position of a kept reference in the compacted order is its
 * output ordinal.  ord_A / ord_B receive that ordinal, or OR_NONE for a
 * dropped record.  Returns the survivor count S.
 */
uint32_t or_keep(const or_side *A, const or_side *B, const uint32_t *refs, uint32_t N,
                 uint32_t *final_refs, uint32_t *ord_A, uint32_t *ord_B) {
  uint32_t S = 0;
  for (uint32_t r = 0; r < A->n; ++r) ord_A[r] = OR_NONE;
  for (uint32_t r = 0; r < B->n; ++r) ord_B[r] = OR_NONE;
  for (uint32_t t = 0; t < N; ++t) {
    uint32_t i0, i1;
    const or_side *s0 = ref_side(A, B, refs[t], &i0);
    int dropped = 0;
    if (t + 1 < N) {
      const or_side *s1 = ref_side(A, B, refs[t + 1], &i1);
      dropped = or_key_cmp(s0, i0, s1, i1) == 0;
    }
    if (dropped) continue;
    final_refs[S] = refs[t];
    if (s0 == A)
      ord_A[i0] = S;
    else
      ord_B[i0] = S;
    ++S;
  }
  return S;
}

/* ---- bit writer: stream bit p is bit 7-(p mod 8) of byte p/8 ---- */

typedef struct {
  uint8_t *buf;
  uint64_t cap_bits;
  uint64_t pos;
  int overflow;
} bitw;

static void put_bit(bitw *w, unsigned bit) {
  if (w->pos >= w->cap_bits) {
    w->overflow = 1;
    ++w->pos;
    return;
  }
  if (bit) w->buf[w->pos >> 3] |= (uint8_t)(0x80u >> (w->pos & 7));
  ++w->pos;
}

/* [GC] record grammar: order-zero Exp-Golomb.  floor(log2(x+1)) zeros, then
 * x+1 written in binary, most significant bit first. */
static void put_eg0(bitw *w, uint64_t x) {
  uint64_t y = x + 1;
  unsigned nbits = 0; /* number of binary digits of y */
  for (uint64_t t = y; t != 0; t >>= 1) ++nbits;
  for (unsigned z = 0; z + 1 < nbits; ++z) put_bit(w, 0);
  for (unsigned b = nbits; b-- > 0;) put_bit(w, (unsigned)((y >> b) & 1));
}

/* Bit b of a byte string, most significant bit of each byte first. */
static unsigned byte_bit(const uint8_t *s, uint64_t b) { return (s[b >> 3] >> (7 - (b & 7))) & 1u; }

/* [GC] prefix-cache paragraph: leading equal bits, clamped to the shorter key. */
static uint64_t bit_lcp(const uint8_t *p, uint64_t kp, const uint8_t *x, uint64_t kx) {
  uint64_t m = kp < kx ? kp : kx, b = 0;
  while (b < m && byte_bit(p, b) == byte_bit(x, b)) ++b;
  return b;
}

/* Exact bit LCP of key i of X and key j of Y (both lengths in bits). */
uint64_t or_key_lcp_bits(const or_side *X, uint32_t i, const or_side *Y, uint32_t j) {
  return bit_lcp(key_ptr(X, i), 8ull * key_len(X, i), key_ptr(Y, j), 8ull * key_len(Y, j));
}

/*
 * [GC] control equation and record grammar.  For survivor i with key bits k_i,
 * exact bit LCP l_i with the preceding survivor (l_0 = 0):
 *   c_i = 1 + l_i        when i mod 15 = 0
 *   c_i = k_{i-1} - l_i  otherwise;
 * record = EG0(c_i) EG0(k_i - l_i) key bits [l_i, k_i) value, where a
 * tombstone value is a single 0 and a present value is 1 EG0(byte length)
 * bytes.  Records follow each other with no padding.
 *
 * Writes len_bits[S], lcp_bits[S] (either may be NULL), off[S+1] (exclusive
 * bit offsets, off[S] = T) and the payload bytes (payload must be zeroed,
 * payload_cap_bytes long).  Returns T, or UINT64_MAX when the payload
 * capacity is too small.
 */
uint64_t or_encode(const or_side *A, const or_side *B, const uint32_t *final_refs, uint32_t S,
                   uint32_t *len_bits, uint32_t *lcp_bits, uint64_t *off, uint8_t *payload,
                   uint64_t payload_cap_bytes) {
  bitw w = {payload, payload_cap_bytes * 8, 0, 0};
  const uint8_t *prev = 0;
  uint64_t kprev = 0;
  for (uint32_t i = 0; i < S; ++i) {
    uint32_t r;
    const or_side *s = ref_side(A, B, final_refs[i], &r);
    const uint8_t *x = key_ptr(s, r);
    uint64_t k = 8ull * key_len(s, r);
    uint64_t l = i == 0 ? 0 : bit_lcp(prev, kprev, x, k);
    uint64_t c = (i % 15 == 0) ? 1 + l : kprev - l;
    off[i] = w.pos;
    put_eg0(&w, c);
    put_eg0(&w, k - l);
    for (uint64_t b = l; b < k; ++b) put_bit(&w, byte_bit(x, b));
    if (is_tomb(s, r)) {
      put_bit(&w, 0);
    } else {
      const uint8_t *v = s->vals + s->val_off[r];
      uint32_t vlen = s->val_off[r + 1] - s->val_off[r];
      put_bit(&w, 1);
      put_eg0(&w, vlen);
      for (uint64_t b = 0; b < 8ull * vlen; ++b) put_bit(&w, byte_bit(v, b));
    }
    if (len_bits) len_bits[i] = (uint32_t)(w.pos - off[i]);
    if (lcp_bits) lcp_bits[i] = (uint32_t)l;
    prev = x;
    kprev = k;
  }
  off[S] = w.pos;
  return w.overflow ? UINT64_MAX : w.pos;
}

/* Number of records any lower bound search returns: keys of Y strictly less
 * than key X_i.  Textbook binary search over the sorted side Y. */
static uint32_t lower_bound(const or_side *Y, const or_side *X, uint32_t i) {
  uint32_t lo = 0, hi = Y->n;
  while (lo < hi) {
    uint32_t mid = lo + (hi - lo) / 2;
    if (or_key_cmp(Y, mid, X, i) < 0)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

/*
 * [CB] "Corrected record ordinals".  For each B_j, lb_j = lower_bound(A, B_j)
 * and C[lb_j] = 1 exactly when the keys match.  R(i) = sum_{t<i} C_t for
 * i = 0..|A|.  A surviving A_i gets ordinal i + lower_bound(B, A_i) - R(i); B_j
 * gets j + lb_j - R(lb_j).  Writes the collision bits (one byte each), R
 * (|A|+1 entries), lb (|B|), the ordinals (OR_NONE for a replaced A) and the
 * final references placed at those ordinals.  Returns |A| + |B| - R(|A|).
 */
uint32_t or_collision(const or_side *A, const or_side *B, uint8_t *C, uint32_t *R, uint32_t *lbB,
                      uint32_t *ord_A, uint32_t *ord_B, uint32_t *final_refs) {
  for (uint32_t i = 0; i < A->n; ++i) C[i] = 0;
  for (uint32_t j = 0; j < B->n; ++j) {
    lbB[j] = lower_bound(A, B, j);
    if (lbB[j] < A->n && or_key_cmp(A, lbB[j], B, j) == 0) C[lbB[j]] = 1;
  }
  R[0] = 0;
  for (uint32_t i = 0; i < A->n; ++i) R[i + 1] = R[i] + C[i];
  for (uint32_t i = 0; i < A->n; ++i) {
    if (C[i]) {
      ord_A[i] = OR_NONE;
      continue;
    }
    ord_A[i] = i + lower_bound(B, A, i) - R[i];
    final_refs[ord_A[i]] = i;
  }
  for (uint32_t j = 0; j < B->n; ++j) {
    ord_B[j] = j + lbB[j] - R[lbB[j]];
    final_refs[ord_B[j]] = A->n + j;
  }
  return A->n + B->n - R[A->n];
}

/* [CB] "Temporary rank layouts": exclusive rank = number of set bits at
 * positions < p.  Bit q of the map is bit (q mod 32) of 32-bit word q/32. */
uint32_t or_rank(const uint32_t *words, uint32_t p) {
  uint32_t c = 0;
  for (uint32_t q = 0; q < p; ++q) c += (words[q >> 5] >> (q & 31)) & 1u;
  return c;
}

/*
 * [GC] Output navigation.  The KV03 paragraph: physical offsets are sampled
 * at ordinals 0, 15, 30, ... plus EOF, and when every encoded value has the
 * same width, that width times the sample's ordinal is subtracted from the
 * offset.  The output-EF paragraph: each entry comes from the record-offset
 * scan (the last from the payload extent); the entries are Elias-Fano coded
 * into packed lows and high bits; every group of 256 entries whose positions
 * in the high bits span at least 4096 bits is sparse, and a scan of the
 * sparse groups' sizes assigns them ranges of explicit exception positions;
 * each group has a sample pair.
 *
 * Readings (the section layouts are not printed on the pages):
 *  - value width of record i: 1 for a tombstone, else 1 + E(len) + 8 len;
 *    the common width w is that width when all S records share it, else 0
 *    (and 0 when S = 0);
 *  - entries: n = ceil(S/15) + 1; e_k = off[15k] - 15k w for 15k < S, and
 *    the last entry e_{n-1} = T - S w;
 *  - low width L = floor(log2(floor((e_{n-1} + 1) / n))), 0 when that
 *    quotient is 0;
 *  - lows: entry k's low L bits at bit k L of little-endian 64-bit words
 *    (bit b is bit b mod 64 of word b/64); unused bits zero;
 *  - high bits: bit (e_k >> L) + k set, n + (e_{n-1} >> L) bits long, same
 *    word order;
 *  - group g holds entries 256g .. min(256g + 256, n) - 1; its span is
 *    p_last - p_first + 1 with p_k = (e_k >> L) + k; sparse when >= 4096;
 *  - sample pair of group g: (p_first, number of exception entries of the
 *    groups before g);
 *  - exceptions: the p_k of every entry of a sparse group, in order.
 */
typedef struct {
  uint64_t n, L, width, low_words, high_bits, high_words, groups, exceptions;
} or_ef_info;

/* Encoded value width of survivor i (record grammar: 0 for a tombstone;
 * 1, EG0(byte length) and the bytes otherwise). */
static uint64_t eg0_bits(uint64_t x) {
  unsigned z = 0;
  while ((x + 1) >> (z + 1)) ++z; /* z = floor(log2(x + 1)) */
  return 2ull * z + 1;
}

uint64_t or_common_width(const or_side *A, const or_side *B, const uint32_t *final_refs, uint32_t S) {
  uint64_t w = 0;
  for (uint32_t i = 0; i < S; ++i) {
    uint32_t r;
    const or_side *s = ref_side(A, B, final_refs[i], &r);
    uint64_t v = 1;
    if (!is_tomb(s, r)) {
      uint64_t len = s->val_off[r + 1] - s->val_off[r];
      v = 1 + eg0_bits(len) + 8 * len;
    }
    if (i == 0)
      w = v;
    else if (v != w)
      return 0;
  }
  return w;
}

/* The n = ceil(S/15) + 1 navigation entries. */
void or_ef_entries(const uint64_t *off, uint32_t S, uint64_t T, uint64_t w, uint64_t *e) {
  uint64_t k = 0;
  for (uint64_t ord = 0; ord < S; ord += 15) e[k++] = off[ord] - ord * w;
  e[k] = T - (uint64_t)S * w;
}

static void set_bit64(uint64_t *words, uint64_t b) { words[b >> 6] |= 1ull << (b & 63); }

/* Elias-Fano sections of the non-decreasing entries e[0..n).  The output
 * arrays must be zeroed and large enough (at most n low words, ceil((3n + 1)
 * / 64) high words, 2 ceil(n / 256) sample words, n exception words). */
void or_ef_encode(const uint64_t *e, uint64_t n, uint64_t width, uint64_t *lows, uint64_t *highs,
                  uint64_t *samples, uint64_t *exc, or_ef_info *info) {
  const uint64_t last = e[n - 1];
  const uint64_t q = (last + 1) / n;
  uint64_t L = 0;
  while (q >> (L + 1)) ++L; /* floor(log2 q) for q >= 1; 0 for q = 0 */
  for (uint64_t k = 0; k < n; ++k) {
    for (uint64_t b = 0; b < L; ++b)
      if ((e[k] >> b) & 1) set_bit64(lows, k * L + b);
    set_bit64(highs, (e[k] >> L) + k);
  }
  const uint64_t high_bits = n + (last >> L);
  const uint64_t groups = (n + 255) / 256;
  uint64_t nexc = 0;
  for (uint64_t g = 0; g < groups; ++g) {
    const uint64_t k0 = 256 * g, k1 = (k0 + 256 < n ? k0 + 256 : n);
    const uint64_t p0 = (e[k0] >> L) + k0, p1 = (e[k1 - 1] >> L) + (k1 - 1);
    samples[2 * g] = p0;
    samples[2 * g + 1] = nexc;
    if (p1 - p0 + 1 >= 4096)
      for (uint64_t k = k0; k < k1; ++k) exc[nexc++] = (e[k] >> L) + k;
  }
  info->n = n;
  info->L = L;
  info->width = width;
  info->low_words = (n * L + 63) / 64;
  info->high_bits = high_bits;
  info->high_words = (high_bits + 63) / 64;
  info->groups = groups;
  info->exceptions = nexc;
}

/*
 * [GC] Compressed input: the block-parse paragraph (a block's first control
 * gives its absolute retained length, later controls count back from the
 * predecessor's key length; values are skipped by their own grammar) read
 * with the record grammar, one record after the other.  Each key is its
 * predecessor's first l_i bits followed by its own literal; this sequential
 * definition is what the literal-owner formula resolves in parallel.
 * Decodes S records of a payload of T bits into a key arena (key_off[S+1]),
 * a value arena (val_off[S+1]) and tombstone flags.  Returns 0, or -1 when
 * the payload is malformed (a field reaches past T, an inherited prefix is
 * longer than the predecessor's key, a key is not whole bytes, bits remain
 * after record S-1) or a capacity is too small.
 */
typedef struct {
  const uint8_t *p;
  uint64_t n, pos;
  int bad;
} bitr;

static unsigned get_bit(bitr *r) {
  if (r->pos >= r->n) {
    r->bad = 1;
    return 0;
  }
  unsigned b = (r->p[r->pos >> 3] >> (7 - (r->pos & 7))) & 1u;
  r->pos++;
  return b;
}

static uint64_t get_eg0(bitr *r) {
  unsigned z = 0;
  while (!r->bad && get_bit(r) == 0) {
    if (++z > 63) {
      r->bad = 1;
      return 0;
    }
  }
  uint64_t v = 1;
  for (unsigned t = 0; t < z && !r->bad; ++t) v = (v << 1) | get_bit(r);
  return v - 1;
}

int or_fc_decode(const uint8_t *payload, uint64_t T, uint32_t S, uint8_t *keys, uint64_t key_cap,
                 uint32_t *key_off, uint8_t *vals, uint64_t val_cap, uint32_t *val_off, uint8_t *tomb) {
  bitr r = {payload, T, 0, 0};
  uint64_t kprev = 0, kat = 0, vat = 0, prev_at = 0;
  for (uint32_t i = 0; i < S; ++i) {
    const uint64_t c = get_eg0(&r), s = get_eg0(&r);
    if (r.bad) return -1;
    uint64_t l;
    if (i % 15 == 0) {
      if (c == 0) return -1;
      l = c - 1;
    } else {
      if (c > kprev) return -1;
      l = kprev - c;
    }
    if (l > kprev) return -1; /* (l_0 must be 0: kprev is 0 before the first record) */
    const uint64_t k = l + s;
    if (k % 8 || kat + k / 8 > key_cap || kat + k / 8 > 0xFFFFFFFFull) return -1;
    key_off[i] = (uint32_t)kat;
    uint8_t *x = keys + kat;
    for (uint64_t b = 0; b < k / 8; ++b) x[b] = 0;
    for (uint64_t b = 0; b < k; ++b) {
      unsigned bit = b < l ? (keys[prev_at + (b >> 3)] >> (7 - (b & 7))) & 1u : get_bit(&r);
      x[b >> 3] |= (uint8_t)(bit << (7 - (b & 7)));
    }
    prev_at = kat;
    kat += k / 8;
    kprev = k;
    val_off[i] = (uint32_t)vat;
    if (get_bit(&r)) {
      tomb[i] = 0;
      const uint64_t len = get_eg0(&r);
      if (r.bad || vat + len > val_cap || vat + len > 0xFFFFFFFFull) return -1;
      for (uint64_t b = 0; b < len; ++b) {
        unsigned v = 0;
        for (int t = 0; t < 8; ++t) v = (v << 1) | get_bit(&r);
        vals[vat + b] = (uint8_t)v;
      }
      vat += len;
    } else {
      tomb[i] = 1;
    }
    if (r.bad) return -1;
  }
  key_off[S] = (uint32_t)kat;
  val_off[S] = (uint32_t)vat;
  return r.pos == T ? 0 : -1;
}

/*
 * [BP]  Everett, "Byte-profile GPU merge": the "Pipeline" steps (byte LEB128
 * counts, byte FC literals and optional-value tags; a common encoded value
 * width, width seventeen being a tag byte for presence followed by sixteen
 * bytes of value), with the control rule of [GC] counted in bytes.
 *
 * Readings (the page names the parts, not their bytes):
 *  - l_i is the byte LCP with the preceding survivor (l_0 = 0), k_i the key
 *    length in bytes; c_i = 1 + l_i when i mod 15 = 0, else k_{i-1} - l_i;
 *  - a record is LEB128(c_i), LEB128(k_i - l_i), key bytes l_i .. k_i-1, then
 *    its value; LEB128 is unsigned little-endian base 128 (low seven bits
 *    first, the high bit of a byte set when another byte follows);
 *  - fixed framing when every present survivor's value has the same byte
 *    length L (or no survivor is present): width W = 1 + L, each value a tag
 *    byte (1 present, 0 tombstone) and L bytes (zeros for a tombstone);
 *  - otherwise variable framing: a tombstone is the tag byte 0, a present
 *    value the tag byte 1, LEB128(byte length) and the bytes; width 0;
 *  - no padding; the payload is the byte stream.
 */
static unsigned leb_len(uint64_t x) {
  unsigned n = 1;
  while (x >= 128) {
    x >>= 7;
    ++n;
  }
  return n;
}

static uint64_t put_leb(uint8_t *out, uint64_t at, uint64_t cap, uint64_t x, int *over) {
  do {
    uint8_t b = (uint8_t)(x & 127);
    x >>= 7;
    if (x) b |= 128;
    if (at < cap)
      out[at] = b;
    else
      *over = 1;
    ++at;
  } while (x);
  return at;
}

static uint64_t byte_lcp(const uint8_t *p, uint64_t np, const uint8_t *x, uint64_t nx) {
  uint64_t m = np < nx ? np : nx, t = 0;
  while (t < m && p[t] == x[t]) ++t;
  return t;
}

/* The framing width: 1 + L when every present survivor's value is L bytes
 * (or none is present), else 0 (variable framing).  0 for S = 0. */
uint64_t or_bp_width(const or_side *A, const or_side *B, const uint32_t *final_refs, uint32_t S) {
  int seen = 0;
  uint64_t L = 0;
  for (uint32_t i = 0; i < S; ++i) {
    uint32_t r;
    const or_side *s = ref_side(A, B, final_refs[i], &r);
    if (is_tomb(s, r)) continue;
    uint64_t len = s->val_off[r + 1] - s->val_off[r];
    if (!seen) {
      L = len;
      seen = 1;
    } else if (len != L) {
      return 0;
    }
  }
  return S ? 1 + L : 0;
}

/* Byte-profile encoding of the survivors: len_bytes[S], lcp_bytes[S],
 * off[S+1] (byte offsets), payload (payload_cap bytes, zeroed by the
 * caller).  Returns the payload length, or UINT64_MAX when it does not fit. */
uint64_t or_bp_encode(const or_side *A, const or_side *B, const uint32_t *final_refs, uint32_t S,
                      uint64_t width, uint32_t *len_bytes, uint32_t *lcp_bytes, uint64_t *off,
                      uint8_t *payload, uint64_t payload_cap) {
  uint64_t at = 0, kprev = 0;
  const uint8_t *prev = 0;
  int over = 0;
  for (uint32_t i = 0; i < S; ++i) {
    uint32_t r;
    const or_side *s = ref_side(A, B, final_refs[i], &r);
    const uint8_t *x = key_ptr(s, r);
    const uint64_t k = key_len(s, r);
    const uint64_t l = i == 0 ? 0 : byte_lcp(prev, kprev, x, k);
    const uint64_t c = (i % 15 == 0) ? 1 + l : kprev - l;
    off[i] = at;
    at = put_leb(payload, at, payload_cap, c, &over);
    at = put_leb(payload, at, payload_cap, k - l, &over);
    for (uint64_t b = l; b < k; ++b) {
      if (at < payload_cap)
        payload[at] = x[b];
      else
        over = 1;
      ++at;
    }
    const int t = is_tomb(s, r);
    const uint8_t *v = s->vals + s->val_off[r];
    const uint64_t vlen = t ? 0 : s->val_off[r + 1] - s->val_off[r];
    if (at < payload_cap)
      payload[at] = t ? 0 : 1;
    else
      over = 1;
    ++at;
    if (width) {
      for (uint64_t b = 0; b + 1 < width; ++b) {
        if (at < payload_cap)
          payload[at] = t ? 0 : v[b];
        else
          over = 1;
        ++at;
      }
    } else if (!t) {
      at = put_leb(payload, at, payload_cap, vlen, &over);
      for (uint64_t b = 0; b < vlen; ++b) {
        if (at < payload_cap)
          payload[at] = v[b];
        else
          over = 1;
        ++at;
      }
    }
    len_bytes[i] = (uint32_t)(at - off[i]);
    lcp_bytes[i] = (uint32_t)l;
    prev = x;
    kprev = k;
  }
  off[S] = at;
  return over ? UINT64_MAX : at;
}
