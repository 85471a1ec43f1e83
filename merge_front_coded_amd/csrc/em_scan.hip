// Exclusive scan of u32 values into u64 (bit offsets) or u32 (rank block
// prefixes) in one pass: each workgroup scans a tile of kScanTile values and
// obtains the sum of all earlier tiles by decoupled look-back.
//
// Everett, "GPU construction experiment": exact lengths are scanned into bit
// offsets by one global scan, with no independently encoded chunk resetting
// the prefix.  The offsets are 64-bit here because the payloads of the large
// workloads exceed 2^32 bits.
#include <mutex>

#include "em_internal.h"

namespace em {

constexpr int kScanBlock = 256;
constexpr int kScanIpt = 16;
constexpr uint32_t kScanTile = kScanBlock * kScanIpt;

// A tile moves between global memory and registers through LDS, so that
// both its loads and its stores are 16 bytes a lane on consecutive addresses
// (a thread's own sixteen consecutive values, loaded or stored directly, put
// 64 scattered addresses on every memory instruction).
template <class OutT>
__global__ __launch_bounds__(kScanBlock) void k_scan(const uint32_t* __restrict__ in, uint32_t n,
                                                     OutT* __restrict__ out, uint32_t* __restrict__ ticket,
                                                     uint64_t* __restrict__ desc, uint32_t ntiles) {
  __shared__ uint64_t wsum[kScanBlock / kWave + 1];
  __shared__ uint32_t s_tile;
  __shared__ uint64_t s_base;
  __shared__ uint4 stage[kScanTile * sizeof(OutT) / 16];
  const uint32_t tid = threadIdx.x;
  if (tid == 0) s_tile = atomicAdd(ticket, 1u);
  __syncthreads();
  const uint32_t tile = s_tile;
  const uint32_t base = tile * kScanTile;
  const uint32_t first = base + tid * kScanIpt;
  // (uniform; the 16-byte paths need 16-byte aligned arrays)
  const bool full = base + kScanTile <= n && (reinterpret_cast<uintptr_t>(in) & 15) == 0;
  const bool full_out = full && (reinterpret_cast<uintptr_t>(out) & 15) == 0;

  uint32_t v[kScanIpt];
  if (full) {
    // striped 16-byte loads into LDS, then each thread's own values
    const uint4* p = reinterpret_cast<const uint4*>(in + base);
#pragma unroll
    for (int q = 0; q < kScanIpt / 4; ++q) stage[q * kScanBlock + tid] = p[q * kScanBlock + tid];
    __syncthreads();
    const uint4* mine = stage + tid * (kScanIpt / 4);
#pragma unroll
    for (int q = 0; q < kScanIpt / 4; ++q) {
      const uint4 t = mine[q];
      v[4 * q] = t.x;
      v[4 * q + 1] = t.y;
      v[4 * q + 2] = t.z;
      v[4 * q + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int q = 0; q < kScanIpt; ++q) v[q] = first + q < n ? in[first + q] : 0u;
  }
  uint64_t local = 0;
#pragma unroll
  for (int q = 0; q < kScanIpt; ++q) local += v[q];

  uint64_t total;
  uint64_t excl = block_exclusive_scan<uint64_t, kScanBlock>(local, wsum, total);
  if (tid < kWave) {
    const uint64_t b = lookback(desc, tile, total);
    if (tid == 0) s_base = b;
  }
  __syncthreads();
  uint64_t run = s_base + excl;
  if (full_out) {
    // each thread's values into LDS, then striped 16-byte stores
    OutT* so = reinterpret_cast<OutT*>(stage) + tid * kScanIpt;
#pragma unroll
    for (int q = 0; q < kScanIpt; ++q) {
      so[q] = static_cast<OutT>(run);
      run += v[q];
    }
    __syncthreads();
    uint4* po = reinterpret_cast<uint4*>(out + base);
    constexpr int kChunks = kScanTile * sizeof(OutT) / 16 / kScanBlock;
#pragma unroll
    for (int q = 0; q < kChunks; ++q) po[q * kScanBlock + tid] = stage[q * kScanBlock + tid];
  } else {
#pragma unroll
    for (int q = 0; q < kScanIpt; ++q) {
      if (first + q < n) out[first + q] = static_cast<OutT>(run);
      run += v[q];
    }
  }
  if (tile == ntiles - 1 && tid == kScanBlock - 1) out[n] = static_cast<OutT>(s_base + total);
}

template <class OutT>
__global__ void k_set_value(OutT* p, OutT v) {
  *p = v;
}

size_t scan_ws(uint32_t n) {
  const size_t tiles = (static_cast<size_t>(n) + kScanTile - 1) / kScanTile;
  return 256 + align_up((tiles ? tiles : 1) * sizeof(uint64_t), 256);
}

template <class OutT>
int scan_launch(const uint32_t* in, uint32_t n, OutT* out, void* ws, size_t ws_bytes, hipStream_t st) {
  if (ws_bytes < scan_ws(n)) return EM_ENOSPC;
  if (n == 0) {
    hipLaunchKernelGGL(k_set_value<OutT>, dim3(1), dim3(1), 0, st, out, static_cast<OutT>(0));
    return check_launch();
  }
  const uint32_t ntiles = (n + kScanTile - 1) / kScanTile;
  WsCursor cur{static_cast<uint8_t*>(ws), 0};
  uint32_t* ticket = cur.take<uint32_t>(64);
  uint64_t* desc = cur.take<uint64_t>(ntiles);
  clear_lookback(ticket, 1, desc, nullptr, ntiles, st);
  hipLaunchKernelGGL(k_scan<OutT>, dim3(ntiles), dim3(kScanBlock), 0, st, in, n, out, ticket, desc,
                     ntiles);
  return check_launch();
}

template int scan_launch<uint32_t>(const uint32_t*, uint32_t, uint32_t*, void*, size_t, hipStream_t);
template int scan_launch<uint64_t>(const uint32_t*, uint32_t, uint64_t*, void*, size_t, hipStream_t);

}  // namespace em

using namespace em;

extern "C" int em_scan(const uint32_t* len_bits, uint32_t S, uint64_t* off, void* ws, size_t ws_bytes,
                       void* stream) {
  if (!off || !ws) return EM_EINVAL;
  if (S > 0 && !len_bits) return EM_EINVAL;
  if (S >= EM_MAX_RECORDS) return EM_ERANGE;
  if (reinterpret_cast<uintptr_t>(ws) & 255) return EM_EINVAL;
  if (S > 0 && (reinterpret_cast<uintptr_t>(len_bits) & 15)) return EM_EINVAL;
  return scan_launch<uint64_t>(len_bits, S, off, ws, ws_bytes, as_stream(stream));
}

// ---------------------------------------------------------------------------
// The same scan with its look-back state in a fixed device array instead of
// a caller workspace, for callers that cannot allocate.  The array holds the
// state for the largest S the ABI accepts (2^24 - 1 values: 4096 tiles).

namespace em {
constexpr size_t kScanScratchBytes = 256 + 4096 * sizeof(uint64_t);
}  // namespace em

// One copy per device, kept until the process ends.  Host code never uses
// this name as an address: the device address comes from
// hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[em::kScanScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first
// call on each device, with that device current).
int scan_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return em::set_hip_error(e);
  if (dev < 0 || dev >= kMaxDevices) return em::set_hip_error(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> guard(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return em::set_hip_error(e);
    if (!p) return em::set_hip_error(hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return EM_OK;
}
}  // namespace

extern "C" int em_scan_noalloc(const uint32_t* len_bits, uint32_t S, uint64_t* off, void* stream) {
  if (!off) return EM_EINVAL;
  if (S > 0 && !len_bits) return EM_EINVAL;
  if (S >= EM_MAX_RECORDS) return EM_ERANGE;
  if (S > 0 && (reinterpret_cast<uintptr_t>(len_bits) & 15)) return EM_EINVAL;
  if (scan_ws(S) > kScanScratchBytes) return EM_ERANGE;
  void* ws = nullptr;
  const int rc = scan_scratch(&ws);
  if (rc) return rc;
  return scan_launch<uint64_t>(len_bits, S, off, ws, kScanScratchBytes, as_stream(stream));
}
