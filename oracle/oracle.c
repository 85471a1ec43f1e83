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
 *        shorter key).
 *  [CB]  Everett, "Collision bitmap and rank experiment": "Corrected record
 *        ordinals" (collision bits, exclusive rank R, ordinal formulas).
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
 * <= B's head, so equal keys put the older input first ([GC] merge paragraph).
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
 * [GC] merge paragraph: a neighbouring-key comparison keeps the last
 * reference of each equal-key run, so the newer record wins; a tombstone stays
 * a record.  The position of a kept reference in the compacted order is its
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
