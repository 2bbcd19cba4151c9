// Allocation-free form of the split shard pass: the partial results live in
// a file-scope device array instead of a caller workspace, for callers that
// cannot allocate device memory (code under graph capture, tight serving
// loops, harnesses that forbid hipMalloc).
//
// Each GPU the library runs on holds one copy of the array until the process
// ends.  Host code never passes the array's name to a kernel or a copy: it
// uses the device address hipGetSymbolAddress returns for the current device,
// looked up once per device.  Every call on a GPU reuses that GPU's array, so
// calls that overlap on one GPU (different streams, or a second host thread)
// race on it.  Nothing in it needs clearing: each call overwrites every
// partial row (out and lse) before the merge reads it.
#include <atomic>
#include <cstdint>

#include "ra_common.h"

namespace {

constexpr int64_t kScratchOutFloats = RA_NOALLOC_MAX_PARTIAL_FLOATS;
constexpr int64_t kScratchLseFloats = RA_NOALLOC_MAX_LSE_FLOATS;

__device__ __align__(256) float scratch[kScratchOutFloats + kScratchLseFloats];

constexpr int kMaxDevices = 64;
std::atomic<float*> g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch` (NULL with *err set on failure).
float* scratch_address(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  float* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  void* addr = nullptr;
  *err = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
  if (*err != hipSuccess || addr == nullptr) return nullptr;
  ptr = static_cast<float*>(addr);
  g_scratch_ptr[dev].store(ptr, std::memory_order_release);  // the same address if two threads race here
  return ptr;
}

}  // namespace

extern "C" ra_status ring_attn_shard_fwd_split_noalloc(const ra_attn_desc* desc, int32_t rank, const void* q,
                                                       int32_t n_blocks, const int32_t* block_owner,
                                                       const void* const* k_blocks, const void* const* v_blocks,
                                                       int32_t n_splits, void* out, float* lse, int64_t* stats,
                                                       void* stream) {
  if (!desc) return ra::set_error(RA_EINVAL, "desc is NULL");
  if (desc->seq_len < 1 || desc->n_shards < 1 || desc->batch < 1 || desc->h_q < 1 || n_splits < 1)
    return ring_attn_shard_fwd_split(desc, rank, q, n_blocks, block_owner, k_blocks, v_blocks, n_splits, nullptr,
                                     nullptr, out, lse, stats, stream);  // reports the argument error
  // Products saturate instead of wrapping, so no descriptor slips past the
  // size check by overflow.
  auto mul = [](int64_t a, int64_t b) {
    int64_t r;
    return __builtin_mul_overflow(a, b, &r) ? INT64_MAX : r;
  };
  const int64_t rows = mul(mul(desc->batch, desc->h_q), desc->seq_len / desc->n_shards);
  const int64_t lse_floats = mul(n_splits, rows);
  const int64_t out_floats = mul(lse_floats, desc->head_dim);
  if (out_floats > kScratchOutFloats || lse_floats > kScratchLseFloats)
    return ra::set_error(RA_EINVAL,
                         "n_splits * batch * h_q * S/c * head_dim = %lld floats exceeds the static scratch "
                         "(%lld floats for partial outputs, %lld for their lse); use ring_attn_shard_fwd_split "
                         "with a workspace",
                         (long long)out_floats, (long long)kScratchOutFloats, (long long)kScratchLseFloats);
  hipError_t e = hipSuccess;
  float* base = scratch_address(&e);
  if (!base) return ra::set_error(RA_EHIP, "scratch address lookup failed: %s", hipGetErrorString(e));
  return ring_attn_shard_fwd_split(desc, rank, q, n_blocks, block_owner, k_blocks, v_blocks, n_splits, base,
                                   base + kScratchOutFloats, out, lse, stats, stream);
}
