// Output navigation: the Elias-Fano sections over the payload's sampled
// record offsets.
//
// Everett, "GPU construction experiment":
//  * the KV03 paragraph: the sampled offsets are those of every fifteenth
//    record from the first, and the end of the payload; with one encoded
//    value width shared by all records, the sample's ordinal times that width
//    is taken off;
//  * the output-EF paragraph: the entries come from the record-offset scan
//    (the last from the payload length); a group of 256 entries is sparse
//    when its high positions spread over 4096 bits or more; a scan of the
//    sparse groups' counts assigns their exception ranges; word-owned kernels
//    write the packed lows, the high bits, the sample pairs and the sparse
//    positions, zero padded.
//
// Section layout (the pages do not print it; read as): n = ceil(S/15) + 1
// entries e_k; L = floor(log2(floor((e_{n-1} + 1) / n))) (0 when that is 0);
// lows: entry k's low L bits at bit k L of little-endian 64-bit words; high
// bits: bit p_k = (e_k >> L) + k set, n + (e_{n-1} >> L) bits; group g =
// entries 256g .. 256g + 255, sparse when p_last - p_first + 1 >= 4096;
// sample pair of g: (p_first, exception entries before g); exceptions: p_k of
// every entry of a sparse group.
#include "em_tile.h"

namespace em {

constexpr int kNavBlock = 256;
constexpr uint32_t kNavGroup = 256;
constexpr uint32_t kNavSparseSpan = 4096;

// Where the entries come from: the record offsets (every 15th, then T, less
// width x ordinal), or an explicit array.
struct EfSrc {
  const uint64_t* off;     // S + 1 offsets (nullptr: use direct)
  const uint64_t* direct;  // n entries
  uint64_t T;
  uint32_t S;
  __device__ __forceinline__ uint64_t entry(uint32_t k, uint64_t w) const {
    if (direct) return direct[k];
    const uint64_t ord = 15ull * k;
    return ord < S ? off[ord] - ord * w : T - static_cast<uint64_t>(S) * w;
  }
};

struct EfWs {
  uint32_t* vmin;     // [0] min and [1] max of the value widths
  uint32_t* cnt;      // groups + 1: exception entries of each group (last 0)
  uint32_t* exc_at;   // groups + 2: their exclusive prefix
  uint8_t* scan_ws;
  size_t scan_bytes;
  size_t used;
};

static EfWs ef_layout(void* ws, uint32_t groups) {
  EfWs L{};
  WsCursor cur{static_cast<uint8_t*>(ws), 0};
  L.vmin = cur.take<uint32_t>(2);
  L.cnt = cur.take<uint32_t>(static_cast<size_t>(groups) + 1);
  L.exc_at = cur.take<uint32_t>(static_cast<size_t>(groups) + 2);
  L.scan_bytes = scan_ws(groups + 1);
  L.scan_ws = cur.take<uint8_t>(L.scan_bytes);
  L.used = cur.used;
  return L;
}

static inline uint32_t ef_entries(uint32_t S) { return (S + 14) / 15 + 1; }
static inline uint32_t nav_blocks(uint64_t n) { return static_cast<uint32_t>((n + kNavBlock - 1) / kNavBlock); }

__global__ void k_ef_init(uint32_t* vmin) {
  vmin[0] = 0xFFFFFFFFu;
  vmin[1] = 0;
}

// Smallest and largest encoded value width over the survivors: a fixed grid
// strides over them and each workgroup adds one pair of atomics (one per
// workgroup of a grid over all survivors would queue tens of thousands on
// the same two words).
constexpr uint32_t kNavWidthGrid = 1024;

__global__ __launch_bounds__(kNavBlock) void k_ef_width(em_side_t A, em_side_t B,
                                                        const uint32_t* __restrict__ final_refs, uint32_t S,
                                                        uint32_t* __restrict__ vmin) {
  __shared__ uint32_t smin[kNavBlock / kWave], smax[kNavBlock / kWave];
  uint32_t lo = 0xFFFFFFFFu, hi = 0;
  for (uint32_t i = blockIdx.x * kNavBlock + threadIdx.x; i < S; i += gridDim.x * kNavBlock) {
    uint32_t idx, vlen;
    bool tomb;
    const SideView s = pick(A, B, final_refs[i], idx);
    const uint32_t v = value_bits(s, idx, vlen, tomb);
    lo = min(lo, v);
    hi = max(hi, v);
  }
  for (int d = kWave / 2; d > 0; d >>= 1) {
    lo = min(lo, static_cast<uint32_t>(__shfl_xor(static_cast<int>(lo), d)));
    hi = max(hi, static_cast<uint32_t>(__shfl_xor(static_cast<int>(hi), d)));
  }
  const uint32_t wv = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    smin[wv] = lo;
    smax[wv] = hi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (uint32_t t = 1; t < kNavBlock / kWave; ++t) {
      lo = min(lo, smin[t]);
      hi = max(hi, smax[t]);
    }
    atomicMin(vmin, lo);
    atomicMax(vmin + 1, hi);
  }
}

// The header: common width, n, L, section lengths.  width_in >= 0: that
// width; kWidthOnDevice: vmin[0] holds it; else the value widths' min and max
// in vmin decide.
constexpr int64_t kWidthOnDevice = -2;

__global__ void k_ef_header(EfSrc src, uint32_t n, int64_t width_in, const uint32_t* __restrict__ vmin,
                            em_ef_info_t* __restrict__ info) {
  uint64_t w = 0;
  if (width_in >= 0)
    w = static_cast<uint64_t>(width_in);
  else if (width_in == kWidthOnDevice)
    w = vmin[0];
  else if (src.S > 0 && vmin[0] == vmin[1])
    w = vmin[0];
  const uint64_t last = src.entry(n - 1, w);
  const uint64_t q = (last + 1) / n;
  const uint64_t L = q ? 63u - static_cast<uint32_t>(__builtin_clzll(q)) : 0u;
  const uint64_t hb = n + (last >> L);
  info->n = n;
  info->L = L;
  info->width = w;
  info->low_words = (static_cast<uint64_t>(n) * L + 63) / 64;
  info->high_bits = hb;
  info->high_words = (hb + 63) / 64;
  info->groups = (n + kNavGroup - 1) / kNavGroup;
}

// Lows: one thread per 64-bit word, gathering the fields that overlap it.
__global__ __launch_bounds__(kNavBlock) void k_ef_lows(EfSrc src, const em_ef_info_t* __restrict__ info,
                                                       uint64_t* __restrict__ lows) {
  const uint64_t wi = static_cast<uint64_t>(blockIdx.x) * kNavBlock + threadIdx.x;
  if (wi >= info->low_words) return;
  const uint64_t L = info->L, w = info->width, n = info->n;
  const uint64_t b0 = 64 * wi, b1 = b0 + 64;
  uint64_t word = 0;
  const uint64_t mask = L == 64 ? ~0ull : ((1ull << L) - 1);
  for (uint64_t k = b0 / L; k < n && k * L < b1; ++k) {
    const uint64_t v = src.entry(static_cast<uint32_t>(k), w) & mask;
    const uint64_t at = k * L;  // field bits [at, at + L)
    if (at >= b0)
      word |= v << (at - b0);
    else
      word |= v >> (b0 - at);
  }
  lows[wi] = word;
}

// High bits: one thread per 64-bit word; the entries whose positions fall in
// it are found by a binary search over the increasing p_k.
__global__ __launch_bounds__(kNavBlock) void k_ef_highs(EfSrc src, const em_ef_info_t* __restrict__ info,
                                                        uint64_t* __restrict__ highs) {
  const uint64_t wi = static_cast<uint64_t>(blockIdx.x) * kNavBlock + threadIdx.x;
  if (wi >= info->high_words) return;
  const uint64_t L = info->L, w = info->width;
  const uint32_t n = static_cast<uint32_t>(info->n);
  auto pos = [&](uint32_t k) { return (src.entry(k, w) >> L) + k; };
  const uint64_t b0 = 64 * wi, b1 = b0 + 64;
  uint32_t lo = 0, hi = n;  // first k with pos(k) >= b0
  while (lo < hi) {
    const uint32_t mid = lo + ((hi - lo) >> 1);
    if (pos(mid) < b0)
      lo = mid + 1;
    else
      hi = mid;
  }
  uint64_t word = 0;
  for (uint32_t k = lo; k < n; ++k) {
    const uint64_t p = pos(k);
    if (p >= b1) break;
    word |= 1ull << (p - b0);
  }
  highs[wi] = word;
}

// Groups: exception entries of each (its size when sparse, else 0).
__global__ __launch_bounds__(kNavBlock) void k_ef_groups(EfSrc src, const em_ef_info_t* __restrict__ info,
                                                         uint32_t* __restrict__ cnt) {
  const uint32_t g = blockIdx.x * kNavBlock + threadIdx.x;
  const uint32_t G = static_cast<uint32_t>(info->groups);
  if (g > G) return;
  uint32_t c = 0;
  if (g < G) {
    const uint64_t L = info->L, w = info->width;
    const uint32_t n = static_cast<uint32_t>(info->n);
    const uint32_t k0 = g * kNavGroup, k1 = min(k0 + kNavGroup, n);
    const uint64_t p0 = (src.entry(k0, w) >> L) + k0, p1 = (src.entry(k1 - 1, w) >> L) + (k1 - 1);
    c = p1 - p0 + 1 >= kNavSparseSpan ? k1 - k0 : 0u;
  }
  cnt[g] = c;
}

// Sample pairs (one thread per group) and exception positions (one thread
// per entry of a sparse group).
__global__ __launch_bounds__(kNavBlock) void k_ef_samples(EfSrc src, em_ef_info_t* __restrict__ info,
                                                          const uint32_t* __restrict__ exc_at,
                                                          uint64_t* __restrict__ samples) {
  const uint32_t g = blockIdx.x * kNavBlock + threadIdx.x;
  const uint32_t G = static_cast<uint32_t>(info->groups);
  if (g == 0) info->exceptions = exc_at[G];
  if (g >= G) return;
  const uint32_t k0 = g * kNavGroup;
  samples[2 * static_cast<uint64_t>(g)] = (src.entry(k0, info->width) >> info->L) + k0;
  samples[2 * static_cast<uint64_t>(g) + 1] = exc_at[g];
}

__global__ __launch_bounds__(kNavBlock) void k_ef_exceptions(EfSrc src, const em_ef_info_t* __restrict__ info,
                                                             const uint32_t* __restrict__ cnt,
                                                             const uint32_t* __restrict__ exc_at,
                                                             uint64_t* __restrict__ exceptions) {
  const uint32_t k = blockIdx.x * kNavBlock + threadIdx.x;
  if (k >= info->n) return;
  const uint32_t g = k / kNavGroup;
  if (cnt[g] == 0) return;
  exceptions[exc_at[g] + (k - g * kNavGroup)] = (src.entry(k, info->width) >> info->L) + k;
}

static int ef_run(const EfSrc& src, uint32_t n, int64_t width_in, const em_side_t* A, const em_side_t* B,
                  const uint32_t* final_refs, uint64_t* lows, uint64_t* highs, uint64_t* samples,
                  uint64_t* exceptions, em_ef_info_t* info, void* ws, hipStream_t st,
                  const uint32_t* width_dev = nullptr) {
  const uint32_t groups = (n + kNavGroup - 1) / kNavGroup;
  EfWs L = ef_layout(ws, groups);
  if (width_dev) {
    L.vmin = const_cast<uint32_t*>(width_dev);  // (read only)
    width_in = kWidthOnDevice;
  } else if (width_in < 0) {
    hipLaunchKernelGGL(k_ef_init, dim3(1), dim3(1), 0, st, L.vmin);
    if (src.S)
      hipLaunchKernelGGL(k_ef_width, dim3(min(nav_blocks(src.S), kNavWidthGrid)), dim3(kNavBlock), 0, st, *A, *B,
                         final_refs, src.S, L.vmin);
  }
  hipLaunchKernelGGL(k_ef_header, dim3(1), dim3(1), 0, st, src, n, width_in, L.vmin, info);
  // grids from the capacities (at most n low words and 3n high bits); the
  // kernels stop at the lengths the header computed
  hipLaunchKernelGGL(k_ef_lows, dim3(nav_blocks(n)), dim3(kNavBlock), 0, st, src, info, lows);
  hipLaunchKernelGGL(k_ef_highs, dim3(nav_blocks((3ull * n + 63) / 64)), dim3(kNavBlock), 0, st, src, info, highs);
  hipLaunchKernelGGL(k_ef_groups, dim3(nav_blocks(groups + 1)), dim3(kNavBlock), 0, st, src, info, L.cnt);
  int rc = check_launch();
  if (rc) return rc;
  rc = scan_launch<uint32_t>(L.cnt, groups + 1, L.exc_at, L.scan_ws, L.scan_bytes, st);
  if (rc) return rc;
  hipLaunchKernelGGL(k_ef_samples, dim3(nav_blocks(groups + 1)), dim3(kNavBlock), 0, st, src, info, L.exc_at,
                     samples);
  hipLaunchKernelGGL(k_ef_exceptions, dim3(nav_blocks(n)), dim3(kNavBlock), 0, st, src, info, L.cnt, L.exc_at,
                     exceptions);
  return check_launch();
}

static int ef_capacity(uint64_t n, uint64_t* low_words, uint64_t* high_words, uint64_t* sample_words,
                       uint64_t* exc_words) {
  if (!low_words || !high_words || !sample_words || !exc_words) return EM_EINVAL;
  *low_words = n;
  *high_words = (3 * n + 63) / 64;
  *sample_words = 2 * ((n + kNavGroup - 1) / kNavGroup);
  *exc_words = n;
  return EM_OK;
}

static int ef_check_out(uint64_t n, const uint64_t* lows, const uint64_t* highs, const uint64_t* samples,
                        const uint64_t* exceptions, const em_ef_info_t* info, const uint64_t* caps) {
  if (!lows || !highs || !samples || !exceptions || !info) return EM_EINVAL;
  uint64_t need[4];
  ef_capacity(n, need, need + 1, need + 2, need + 3);
  for (int t = 0; t < 4; ++t)
    if (caps[t] < need[t]) return EM_ENOSPC;
  return EM_OK;
}

}  // namespace em

using namespace em;

extern "C" int em_ef_capacity(uint32_t n_entries, uint64_t* low_words, uint64_t* high_words,
                              uint64_t* sample_words, uint64_t* exception_words) {
  if (n_entries == 0) return EM_EINVAL;
  return ef_capacity(n_entries, low_words, high_words, sample_words, exception_words);
}

extern "C" uint32_t em_ef_entry_count(uint32_t S) { return ef_entries(S); }

extern "C" size_t em_ef_workspace_bytes(uint32_t n_entries) {
  const uint32_t groups = (n_entries + kNavGroup - 1) / kNavGroup;
  return align_up(ef_layout(nullptr, groups).used, 256);
}

extern "C" int em_ef_navigation(const em_side_t* A, const em_side_t* B, const uint32_t* final_refs, uint32_t S,
                                const uint64_t* off, uint64_t T, uint64_t* lows, uint64_t low_cap,
                                uint64_t* highs, uint64_t high_cap, uint64_t* samples, uint64_t sample_cap,
                                uint64_t* exceptions, uint64_t exception_cap, em_ef_info_t* info, void* ws,
                                size_t ws_bytes, void* stream) {
  int rc = check_pair(A, B);
  if (rc) return rc;
  if (S > A->n + B->n) return EM_EINVAL;
  if ((S == 0) != (T == 0)) return EM_EINVAL;
  if (S && (!final_refs || !off)) return EM_EINVAL;
  const uint32_t n = ef_entries(S);
  const uint64_t caps[4] = {low_cap, high_cap, sample_cap, exception_cap};
  rc = ef_check_out(n, lows, highs, samples, exceptions, info, caps);
  if (rc) return rc;
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255)) return EM_EINVAL;
  if (ws_bytes < em_ef_workspace_bytes(n)) return EM_ENOSPC;
  const EfSrc src{off, nullptr, T, S};
  return ef_run(src, n, -1, A, B, final_refs, lows, highs, samples, exceptions, info, ws, as_stream(stream));
}

extern "C" int em_ef_encode(const uint64_t* entries, uint32_t n, uint64_t width, uint64_t* lows, uint64_t low_cap,
                            uint64_t* highs, uint64_t high_cap, uint64_t* samples, uint64_t sample_cap,
                            uint64_t* exceptions, uint64_t exception_cap, em_ef_info_t* info, void* ws,
                            size_t ws_bytes, void* stream) {
  if (n == 0 || !entries) return EM_EINVAL;
  if (n >= EM_MAX_RECORDS) return EM_ERANGE;
  if (width > 0x7FFFFFFFull) return EM_EINVAL;
  const uint64_t caps[4] = {low_cap, high_cap, sample_cap, exception_cap};
  int rc = ef_check_out(n, lows, highs, samples, exceptions, info, caps);
  if (rc) return rc;
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255)) return EM_EINVAL;
  if (ws_bytes < em_ef_workspace_bytes(n)) return EM_ENOSPC;
  const EfSrc src{nullptr, entries, 0, 0};
  return ef_run(src, n, static_cast<int64_t>(width), nullptr, nullptr, nullptr, lows, highs, samples, exceptions,
                info, ws, as_stream(stream));
}

extern "C" int em_bp_navigation(const uint64_t* off, uint32_t S, uint64_t T, const uint32_t* d_width,
                                uint64_t* lows, uint64_t low_cap, uint64_t* highs, uint64_t high_cap,
                                uint64_t* samples, uint64_t sample_cap, uint64_t* exceptions,
                                uint64_t exception_cap, em_ef_info_t* info, void* ws, size_t ws_bytes,
                                void* stream) {
  if (!d_width || (S && !off)) return EM_EINVAL;
  if (S >= EM_MAX_RECORDS) return EM_ERANGE;
  if ((S == 0) != (T == 0)) return EM_EINVAL;
  const uint32_t n = ef_entries(S);
  const uint64_t caps[4] = {low_cap, high_cap, sample_cap, exception_cap};
  int rc = ef_check_out(n, lows, highs, samples, exceptions, info, caps);
  if (rc) return rc;
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255)) return EM_EINVAL;
  if (ws_bytes < em_ef_workspace_bytes(n)) return EM_ENOSPC;
  const EfSrc src{off, nullptr, T, S};
  return ef_run(src, n, kWidthOnDevice, nullptr, nullptr, nullptr, lows, highs, samples, exceptions, info, ws,
                as_stream(stream), d_width);
}
