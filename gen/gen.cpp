// Seeded synthetic input generator for the merge / front-coding hot path.
//
// Produces two record sets, an older side A and a newer side B.  Each side is
// strictly increasing under unsigned bytewise order (a proper prefix sorts
// first) and therefore has unique keys; a chosen number of keys appear on both
// sides.  Records carry a value (an arbitrary byte string) or, on B, may be
// tombstones.  Output per side: a key byte arena with n+1 u32 offsets, a value
// byte arena with n+1 u32 offsets, and one tombstone byte per record.
//
// This module holds none of the merge or encoding arithmetic.  It only draws
// keys, sorts and de-duplicates the drawn pool, and assigns keys to the sides.
//
// Randomness: xoshiro256** (Blackman & Vigna, 2018), state seeded with
// splitmix64 from the caller's 64-bit seed.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <string>
#include <unordered_set>
#include <vector>

namespace {

struct Rng {
  uint64_t s[4];
  static uint64_t splitmix(uint64_t& x) {
    uint64_t z = (x += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  explicit Rng(uint64_t seed) {
    uint64_t x = seed;
    for (auto& w : s) w = splitmix(x);
  }
  static uint64_t rotl(uint64_t v, int k) { return (v << k) | (v >> (64 - k)); }
  uint64_t next() {
    const uint64_t r = rotl(s[1] * 5, 7) * 9;
    const uint64_t t = s[1] << 17;
    s[2] ^= s[0];
    s[3] ^= s[1];
    s[1] ^= s[2];
    s[0] ^= s[3];
    s[2] ^= t;
    s[3] = rotl(s[3], 45);
    return r;
  }
  // uniform integer in [0, n), n >= 1 (multiply-shift on 32 random bits)
  uint32_t below(uint32_t n) { return (uint32_t)(((next() >> 32) * (uint64_t)n) >> 32); }
  uint64_t below64(uint64_t n) {  // rejection-free enough for n << 2^64
    return (uint64_t)(((unsigned __int128)next() * n) >> 64);
  }
  uint32_t range(uint32_t lo, uint32_t hi) { return lo + below(hi - lo + 1); }  // inclusive
  double uniform() { return (double)(next() >> 11) * (1.0 / 9007199254740992.0); }
};

// Finite Zipf over ranks 1..n with exponent s; returns a 0-based rank.
struct Zipf {
  std::vector<double> cdf;
  Zipf(uint32_t n, double s) : cdf(n) {
    double acc = 0;
    for (uint32_t r = 0; r < n; ++r) {
      acc += 1.0 / std::pow((double)(r + 1), s);
      cdf[r] = acc;
    }
    for (auto& c : cdf) c /= acc;
  }
  uint32_t draw(Rng& g) const {
    double u = g.uniform();
    size_t r = std::upper_bound(cdf.begin(), cdf.end(), u) - cdf.begin();
    return (uint32_t)std::min(r, cdf.size() - 1);
  }
};

enum KeyKind { KEY_UNIFORM = 0, KEY_PATHS = 1, KEY_U128 = 2, KEY_URL = 3 };
enum ValKind { VAL_UNIFORM = 0, VAL_FIXED = 1, VAL_LOGUNIFORM = 2 };

}  // namespace

extern "C" {

typedef struct {
  int key_kind;
  uint32_t kmin, kmax;       // KEY_UNIFORM: length range (inclusive); KEY_URL: total length range
  const char* alphabet;      // KEY_UNIFORM symbols
  uint32_t nalpha;
  uint32_t seg_min, seg_max; // KEY_PATHS: segments per key
  uint32_t vocab;            // KEY_PATHS / KEY_URL: vocabulary size
  uint32_t sl_min, sl_max;   // vocabulary entry length range
  double zipf_s;             // vocabulary Zipf exponent
  uint32_t hosts;            // KEY_URL: number of hosts
  double host_zipf;          // KEY_URL: host Zipf exponent
  uint32_t hl_min, hl_max;   // KEY_URL: host label length range
  uint32_t digits;           // KEY_URL: decimal suffix length
  int val_kind;
  uint32_t vmin, vmax;       // VAL_UNIFORM range; VAL_FIXED uses vmin; VAL_LOGUNIFORM uses vmax
  uint64_t nA, nB, nX;       // side sizes and number of keys present on both sides
  double tombA, tombB;       // Bernoulli tombstone probability per record
  uint64_t seed;
} gen_params;

}  // extern "C"

namespace {

struct Pool {
  std::vector<uint8_t> bytes;
  std::vector<uint64_t> off;  // n+1
  size_t n() const { return off.size() - 1; }
  const uint8_t* key(size_t i) const { return bytes.data() + off[i]; }
  uint32_t len(size_t i) const { return (uint32_t)(off[i + 1] - off[i]); }
};

std::string random_word(Rng& g, uint32_t lo, uint32_t hi) {
  uint32_t L = g.range(lo, hi);
  std::string s(L, 'a');
  for (auto& c : s) c = (char)('a' + g.below(26));
  return s;
}

std::vector<std::string> vocabulary(Rng& g, uint32_t n, uint32_t lo, uint32_t hi) {
  std::unordered_set<std::string> seen;
  std::vector<std::string> v;
  v.reserve(n);
  while (v.size() < n) {
    std::string w = random_word(g, lo, hi);
    if (seen.insert(w).second) v.push_back(std::move(w));
  }
  return v;
}

void draw_keys(const gen_params& p, Rng& g, uint64_t count, Pool& out) {
  out.bytes.clear();
  out.off.assign(1, 0);
  out.off.reserve(count + 1);
  std::vector<std::string> vocab, hosts;
  Zipf* zv = nullptr;
  Zipf* zh = nullptr;
  if (p.key_kind == KEY_PATHS || p.key_kind == KEY_URL) {
    vocab = vocabulary(g, p.vocab, p.sl_min, p.sl_max);
    zv = new Zipf(p.vocab, p.zipf_s);
  }
  if (p.key_kind == KEY_URL) {
    hosts = vocabulary(g, p.hosts, p.hl_min, p.hl_max);
    zh = new Zipf(p.hosts, p.host_zipf);
  }
  std::string s;
  out.bytes.reserve((size_t)count * (p.key_kind == KEY_U128 ? 16 : (p.kmin + p.kmax) / 2 + 8));
  for (uint64_t i = 0; i < count; ++i) {
    switch (p.key_kind) {
      case KEY_UNIFORM: {
        uint32_t L = g.range(p.kmin, p.kmax);
        for (uint32_t t = 0; t < L; ++t) out.bytes.push_back((uint8_t)p.alphabet[g.below(p.nalpha)]);
        break;
      }
      case KEY_PATHS: {
        s.clear();
        uint32_t segs = g.range(p.seg_min, p.seg_max);
        for (uint32_t t = 0; t < segs; ++t) {
          if (t) s.push_back('/');
          s += vocab[zv->draw(g)];
        }
        out.bytes.insert(out.bytes.end(), s.begin(), s.end());
        break;
      }
      case KEY_U128: {
        uint64_t hi = g.next(), lo = g.next();
        for (int b = 7; b >= 0; --b) out.bytes.push_back((uint8_t)(hi >> (8 * b)));
        for (int b = 7; b >= 0; --b) out.bytes.push_back((uint8_t)(lo >> (8 * b)));
        break;
      }
      case KEY_URL: {
        uint32_t L = g.range(p.kmin, p.kmax);
        s = "https://";
        s += hosts[zh->draw(g)];
        s += ".example/";
        uint32_t body = L - p.digits;
        while (s.size() < body) {
          s += vocab[zv->draw(g)];
          s.push_back('/');
        }
        s.resize(body);
        for (uint32_t t = 0; t < p.digits; ++t) s.push_back((char)('0' + g.below(10)));
        out.bytes.insert(out.bytes.end(), s.begin(), s.end());
        break;
      }
    }
    out.off.push_back(out.bytes.size());
  }
  delete zv;
  delete zh;
}

// ---- sorting the drawn pool (input preparation, not part of the method) ----

struct Item {
  uint64_t pfx;  // 8 key bytes starting at the current depth, big-endian, zero padded
  uint32_t rem;  // min(bytes remaining from depth, 9): 9 means the key continues past the window
  uint32_t idx;
};

void fill_items(const Pool& pool, Item* it, size_t cnt, uint32_t depth) {
  for (size_t t = 0; t < cnt; ++t) {
    const uint8_t* k = pool.key(it[t].idx);
    uint32_t L = pool.len(it[t].idx);
    uint32_t r = L > depth ? L - depth : 0;
    uint64_t v = 0;
    for (uint32_t b = 0; b < 8; ++b) v = (v << 8) | (b < r ? k[depth + b] : 0);
    it[t].pfx = v;
    it[t].rem = r > 8 ? 9 : r;
  }
}

void sort_run(const Pool& pool, Item* it, size_t cnt, uint32_t depth) {
  if (cnt < 2) return;
  fill_items(pool, it, cnt, depth);
  std::sort(it, it + cnt, [](const Item& a, const Item& b) {
    if (a.pfx != b.pfx) return a.pfx < b.pfx;
    return a.rem < b.rem;
  });
  size_t s = 0;
  while (s < cnt) {
    size_t e = s + 1;
    while (e < cnt && it[e].pfx == it[s].pfx && it[e].rem == it[s].rem) ++e;
    if (e - s > 1 && it[s].rem == 9) sort_run(pool, it + s, e - s, depth + 8);
    s = e;
  }
}

bool same_key(const Pool& p, uint32_t a, uint32_t b) {
  return p.len(a) == p.len(b) && std::memcmp(p.key(a), p.key(b), p.len(a)) == 0;
}

// Sorted, de-duplicated pool indices.
std::vector<uint32_t> sorted_unique(const Pool& pool) {
  std::vector<Item> it(pool.n());
  for (size_t i = 0; i < it.size(); ++i) it[i].idx = (uint32_t)i;
  sort_run(pool, it.data(), it.size(), 0);
  std::vector<uint32_t> out;
  out.reserve(it.size());
  for (size_t i = 0; i < it.size(); ++i)
    if (out.empty() || !same_key(pool, out.back(), it[i].idx)) out.push_back(it[i].idx);
  return out;
}

template <class T>
void shuffle(Rng& g, std::vector<T>& v) {
  for (size_t i = v.size(); i > 1; --i) std::swap(v[i - 1], v[g.below64(i)]);
}

uint32_t draw_vlen(const gen_params& p, Rng& g) {
  switch (p.val_kind) {
    case VAL_FIXED: return p.vmin;
    case VAL_LOGUNIFORM: {
      double e = std::exp(g.uniform() * std::log((double)p.vmax + 1.0));
      uint32_t v = (uint32_t)std::floor(e);
      return v ? v - 1 : 0;
    }
    default: return g.range(p.vmin, p.vmax);
  }
}

// One output record: which pool key, tombstone flag and value length.
struct Rec {
  uint32_t key;
  uint32_t vlen;  // 0 for a tombstone
  uint8_t tomb;
};

struct Result {
  Pool pool;
  std::vector<Rec> side[2];
  uint64_t key_bytes[2] = {0, 0}, val_bytes[2] = {0, 0};
  uint64_t val_seed[2] = {0, 0};
  int err = 0;
};

}  // namespace

extern "C" {

// Plans both sides: draws and sorts the key pool, picks the keys of each side
// and every record's tombstone flag and value length.  Returns a handle
// (never NULL); gen_error() reports a non-zero code when the parameters are
// inconsistent or the key space cannot supply enough distinct keys.
void* gen_run(const gen_params* pp) {
  const gen_params& p = *pp;
  Result* res = new Result();
  if (p.nX > p.nA || p.nX > p.nB) {
    res->err = 1;
    return res;
  }
  Rng g(p.seed);
  const uint64_t U = p.nA + p.nB - p.nX;  // distinct keys needed
  std::vector<uint32_t> uniq;
  double factor = 1.02;
  for (int attempt = 0;; ++attempt) {
    uint64_t want = (uint64_t)std::ceil((double)U * factor) + 64;
    draw_keys(p, g, want, res->pool);
    uniq = sorted_unique(res->pool);
    if (uniq.size() >= U) break;
    if (attempt == 12) {
      res->err = 2;
      return res;
    }
    factor *= 1.3;
  }
  // Keep U of the distinct keys, chosen uniformly (order kept), by dropping
  // the surplus at random; then assign roles A only / B only / both.
  std::vector<uint8_t> keep(uniq.size(), 1);
  for (uint64_t dropped = 0, surplus = uniq.size() - U; dropped < surplus;) {
    uint64_t i = g.below64(uniq.size());
    if (keep[i]) {
      keep[i] = 0;
      ++dropped;
    }
  }
  std::vector<uint8_t> role;  // 0 = A only, 1 = B only, 2 = both
  role.reserve(U);
  role.insert(role.end(), p.nA - p.nX, 0);
  role.insert(role.end(), p.nB - p.nX, 1);
  role.insert(role.end(), p.nX, 2);
  shuffle(g, role);
  res->side[0].reserve(p.nA);
  res->side[1].reserve(p.nB);
  size_t r = 0;
  for (size_t i = 0; i < uniq.size(); ++i) {
    if (!keep[i]) continue;
    const uint8_t ro = role[r++];
    const uint32_t k = uniq[i];
    for (int sd = 0; sd < 2; ++sd) {
      if (ro == (sd == 0 ? 1 : 0)) continue;  // this key is not on side sd
      const bool t = g.uniform() < (sd == 0 ? p.tombA : p.tombB);
      const uint32_t vl = draw_vlen(p, g);
      res->side[sd].push_back(Rec{k, t ? 0u : vl, (uint8_t)(t ? 1 : 0)});
      res->key_bytes[sd] += res->pool.len(k);
      res->val_bytes[sd] += t ? 0u : vl;
    }
  }
  res->val_seed[0] = g.next();
  res->val_seed[1] = g.next();
  return res;
}

int gen_error(void* h) { return ((Result*)h)->err; }

void gen_sizes(void* h, int side, uint64_t* n, uint64_t* key_bytes, uint64_t* val_bytes) {
  const Result* res = (const Result*)h;
  *n = res->side[side].size();
  *key_bytes = res->key_bytes[side];
  *val_bytes = res->val_bytes[side];
}

// Writes one side straight into the caller's buffers (sizes from gen_sizes):
// keys gathered from the sorted pool, value bytes drawn from the side's own
// stream, n+1 offsets each, one tombstone byte per record.
void gen_copy(void* h, int side, uint8_t* keys, uint32_t* key_off, uint8_t* vals, uint32_t* val_off,
              uint8_t* tomb) {
  const Result* res = (const Result*)h;
  const Pool& pool = res->pool;
  const std::vector<Rec>& recs = res->side[side];
  Rng g(res->val_seed[side]);
  uint64_t kp = 0, vp = 0;
  key_off[0] = 0;
  val_off[0] = 0;
  for (size_t i = 0; i < recs.size(); ++i) {
    if (i + 8 < recs.size()) __builtin_prefetch(pool.bytes.data() + pool.off[recs[i + 8].key]);
    const Rec& rc = recs[i];
    const uint32_t L = pool.len(rc.key);
    std::memcpy(keys + kp, pool.key(rc.key), L);
    kp += L;
    key_off[i + 1] = (uint32_t)kp;
    tomb[i] = rc.tomb;
    uint32_t t = 0;
    for (; t + 8 <= rc.vlen; t += 8) {
      const uint64_t x = g.next();
      std::memcpy(vals + vp + t, &x, 8);
    }
    if (t < rc.vlen) {
      const uint64_t x = g.next();
      std::memcpy(vals + vp + t, &x, rc.vlen - t);
    }
    vp += rc.vlen;
    val_off[i + 1] = (uint32_t)vp;
  }
}

void gen_free(void* h) { delete (Result*)h; }

}  // extern "C"
