// Reference streaming kernels for the bandwidth ceiling the prologue is
// measured against.  Both move 16 bytes per lane, one vector per lane, in
// 64-lane (one-wave) blocks, with the same load and store policy as the
// prologue's q stream (non-temporal loads, "nt sc1" stores: 1.1-1.2% faster
// than "nt" stores for both kernels on MI355X, so the ceilings use them too):
//   stream_copy  dst[i] = src[i]                       (read n + write n bytes)
//   stream_rmw   buf[i] = buf[i] ^ mask, in place      (read n + write n bytes)
// The in-place form is the access pattern of the prologue's Q heads, which
// are read and written back at the same address, without the arithmetic.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "occupancy.hpp"
#include "prologue_launch.hpp"
#include "wave_ops.hpp"

namespace fp8kv {
namespace {

// One wave per block: measured on MI355X with cold caches, the in-place form
// moves 6.77 TB/s over 2 GiB and 8 GiB with 64-lane blocks, against 6.56-6.58
// with 128 or 256 lanes and 6.25-6.38 with 512 or 1024.
constexpr int kThreads = 64;

// The in-place RMW caps its launches from 128 MiB up at 25 blocks per CU
// (the uncapped launch holds 32).  Measured on MI355X, uncapped against
// capped: with cold caches 43.20 / 42.79, 82.49 / 81.19, 161.04 / 158.86,
// 634.4 / 620.7 and 2537 / 2473 us over 128 MiB, 256 MiB, 512 MiB, 2 GiB and
// 8 GiB (level at 64 MiB: 23.80 / 23.80); launched back to back over 2 GiB,
// 6.74-6.82 against 6.89-6.96 TB/s.  21 blocks per CU was level with no cap,
// 18 and fewer slower.  The copy is not capped: with cold caches the cap
// gained 1-2% from 128 MiB up, but launched back to back, as the copy
// ceiling of the benchmark is, it lost 2-3% (6.42-6.43 against 6.59-6.63
// TB/s over 512 MiB each way).
// (These were measured with "nt" stores; with "nt sc1" stores the capped
// RMW moved 6.97-6.99 TB/s back to back over 2 GiB.)
constexpr int kCapBlocksPerCu = 25;
constexpr int64_t kCapMinBytes = int64_t{128} << 20;

unsigned cap_lds(int64_t bytes) {
  return bytes >= kCapMinBytes ? static_cast<unsigned>(lds_for_blocks_per_cu(kCapBlocksPerCu))
                               : 0u;
}

__global__ void __launch_bounds__(kThreads) stream_copy_kernel(
    u32x4_t* __restrict__ dst, const u32x4_t* __restrict__ src, int64_t n16) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i < n16) store16_nt_sc1(dst + i, load16<true>(src + i));
}

__global__ void __launch_bounds__(kThreads) stream_rmw_kernel(
    u32x4_t* __restrict__ buf, int64_t n16, uint32_t mask) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i < n16) store16_nt_sc1(buf + i, load16<true>(buf + i) ^ mask);
}

int grid_for(int64_t n16, uint32_t* blocks) {
  const int64_t b = (n16 + kThreads - 1) / kThreads;
  if (b > 0x7FFFFFFF) return FP8KV_ERR_SHAPE;
  *blocks = static_cast<uint32_t>(b);
  return FP8KV_OK;
}

}  // namespace

int launch_stream_copy(void* dst, const void* src, int64_t n16, hipStream_t stream) {
  uint32_t blocks = 0;
  if (int st = grid_for(n16, &blocks)) return st;
  u32x4_t* d = static_cast<u32x4_t*>(dst);
  const u32x4_t* s = static_cast<const u32x4_t*>(src);
  void* args[] = {&d, &s, &n16};
  return hipLaunchKernel(reinterpret_cast<const void*>(&stream_copy_kernel),
                         dim3(blocks), dim3(kThreads), args, 0, stream) == hipSuccess
             ? FP8KV_OK
             : FP8KV_ERR_LAUNCH;
}

int launch_stream_rmw(void* buf, int64_t n16, uint32_t mask, hipStream_t stream) {
  uint32_t blocks = 0;
  if (int st = grid_for(n16, &blocks)) return st;
  u32x4_t* b = static_cast<u32x4_t*>(buf);
  void* args[] = {&b, &n16, &mask};
  return hipLaunchKernel(reinterpret_cast<const void*>(&stream_rmw_kernel),
                         dim3(blocks), dim3(kThreads), args, cap_lds(n16 * 16),
                         stream) == hipSuccess
             ? FP8KV_OK
             : FP8KV_ERR_LAUNCH;
}

}  // namespace fp8kv
