// Measurement probe, not part of the decode path: reads the cache rows a
// page table names (576 bytes each, as 36 chunks of 16 B) and does nothing
// with them but an XOR into one dword per thread.  Its rate on a workload's
// own rows is the practical HBM ceiling of the partial kernel's gather
// pattern (page size 1, rows scattered over the cache).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLoads = 8;  // 16-byte loads in flight per thread

__global__ void __launch_bounds__(256) probe_gather_kernel(const uint8_t* __restrict__ kv,
                                                           const int32_t* __restrict__ idx, uint32_t nchunks,
                                                           uint32_t* __restrict__ out) {
  const uint32_t G = gridDim.x * 256u;
  const uint32_t g = blockIdx.x * 256u + threadIdx.x;
  u32x4 acc = {0, 0, 0, 0};
  for (uint32_t base = g; base < nchunks; base += kLoads * G) {
    u32x4 v[kLoads];
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      const uint32_t i = base + k * G;
      v[k] = u32x4{0, 0, 0, 0};
      if (i < nchunks) {
        const uint32_t t = i / 36u, c = i - 36u * t;
        v[k] = *reinterpret_cast<const u32x4*>(kv + (int64_t)idx[t] * 576 + 16 * c);
      }
    }
#pragma unroll
    for (int k = 0; k < kLoads; ++k) acc ^= v[k];
  }
  out[g] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace

// kv [num_slots][576] u8 (16-byte aligned), idx [ntok] int32 inside
// [0, num_slots) (the caller's guarantee), out [grid * 256] u32.  Returns 0,
// 1 for bad sizes (ntok * 36 + kLoads * grid * 256 must stay below 2^31),
// 3 for a failed launch.
extern "C" int mla_probe_gather(const uint8_t* kv, const int32_t* idx, int64_t ntok, uint32_t* out, int32_t grid,
                                void* stream) {
  if (!kv || !idx || !out || ntok < 0 || grid < 1) return 1;
  if (ntok * 36 + (int64_t)kLoads * grid * 256 >= (1LL << 31)) return 1;
  hipLaunchKernelGGL(probe_gather_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, kv, idx,
                     (uint32_t)(ntok * 36), out);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}
