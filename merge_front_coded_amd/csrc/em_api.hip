// Host-side parts of the C ABI shared by every call: argument checks, error
// codes, workspace sizing, the payload bound and the fill kernels.
#include "em_internal.h"

namespace em {

static thread_local int g_last_hip_error = 0;

int set_hip_error(hipError_t e) {
  g_last_hip_error = static_cast<int>(e);
  return EM_EDEVICE;
}

int check_launch() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? EM_OK : set_hip_error(e);
}

int check_side(const em_side_t* s) {
  if (!s) return EM_EINVAL;
  if (!s->key_off || !s->val_off || !s->keys || !s->vals) return EM_EINVAL;
  if ((reinterpret_cast<uintptr_t>(s->keys) & 15) || (reinterpret_cast<uintptr_t>(s->vals) & 15))
    return EM_EINVAL;
  if ((reinterpret_cast<uintptr_t>(s->key_off) & 3) || (reinterpret_cast<uintptr_t>(s->val_off) & 3))
    return EM_EINVAL;
  if (s->n >= EM_MAX_RECORDS) return EM_ERANGE;
  if (s->key_bytes > 0xFFFFFFFFull || s->val_bytes > 0xFFFFFFFFull) return EM_ERANGE;
  return EM_OK;
}

int check_pair(const em_side_t* A, const em_side_t* B) {
  int rc = check_side(A);
  if (rc) return rc;
  rc = check_side(B);
  if (rc) return rc;
  if (static_cast<uint64_t>(A->n) + B->n >= EM_MAX_RECORDS) return EM_ERANGE;
  return EM_OK;
}

__global__ void k_clear_u64(uint64_t* p, size_t n) {
  size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  for (; i < n; i += static_cast<size_t>(gridDim.x) * blockDim.x) p[i] = 0;
}

__global__ void k_clear_u32(uint32_t* p, size_t n) {
  size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  for (; i < n; i += static_cast<size_t>(gridDim.x) * blockDim.x) p[i] = 0;
}

__global__ void k_clear_lookback(uint32_t* t, size_t nt, uint64_t* d0, uint64_t* d1, size_t nd) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < nt || i < nd; i += stride) {
    if (i < nt) t[i] = 0;
    if (i < nd) {
      d0[i] = 0;
      if (d1) d1[i] = 0;
    }
  }
}

void clear_lookback(uint32_t* ticket, size_t nt, uint64_t* d0, uint64_t* d1, size_t nd, hipStream_t st) {
  const size_t n = nt > nd ? nt : nd;
  if (!n) return;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_clear_lookback, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, st, ticket, nt, d0, d1,
                     nd);
}

void clear_u64(uint64_t* p, size_t n, hipStream_t st) {
  if (!n) return;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_clear_u64, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, st, p, n);
}

void clear_u32(uint32_t* p, size_t n, hipStream_t st) {
  if (!n) return;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_clear_u32, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, st, p, n);
}

}  // namespace em

using namespace em;

extern "C" {

size_t em_workspace_bytes(uint32_t nA, uint32_t nB, uint32_t items_per_part) {
  const uint64_t N64 = static_cast<uint64_t>(nA) + nB;
  const uint32_t N = N64 >= EM_MAX_RECORDS ? EM_MAX_RECORDS : static_cast<uint32_t>(N64);
  size_t need = scan_ws(N);
  if (items_per_part >= 1) {
    size_t m = merge_keep_ws(N, items_per_part);
    if (m > need) need = m;
  }
  size_t c = collision_ws(nA, nB);
  if (c > need) need = c;
  return align_up(need, 256);
}

int em_payload_bound_bits(const em_side_t* A, const em_side_t* B, uint64_t* bound) {
  if (!A || !B || !bound) return EM_EINVAL;
  if (static_cast<uint64_t>(A->n) + B->n >= EM_MAX_RECORDS) return EM_ERANGE;
  if (A->key_bytes > 0xFFFFFFFFull || B->key_bytes > 0xFFFFFFFFull || A->val_bytes > 0xFFFFFFFFull ||
      B->val_bytes > 0xFFFFFFFFull)
    return EM_ERANGE;
  const uint64_t raw = A->key_bytes + B->key_bytes + A->val_bytes + B->val_bytes;
  *bound = 8 * raw + (static_cast<uint64_t>(A->n) + B->n) * 184u;
  return EM_OK;
}

const char* em_strerror(int code) {
  switch (code) {
    case EM_OK: return "success";
    case EM_EINVAL: return "invalid argument (null, misaligned or inconsistent)";
    case EM_ERANGE: return "a size cap is exceeded";
    case EM_ENOSPC: return "workspace or output capacity too small";
    case EM_EDEVICE: return "HIP runtime error (see em_last_hip_error)";
    default: return "unknown error code";
  }
}

int em_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
