// Streaming-read probe: the HBM read ceiling that the decode kernels are
// compared against (the "measured read ceiling" denominator of the SM86
// kernel paragraph of the ro99/strata README).  Each workgroup streams its own
// contiguous share of the buffer with non-temporal 16-byte loads, eight in
// flight per lane; the data is folded into one word that is stored only if it
// equals a value the fill never produces, so no load can be removed.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace strata {

typedef uint32_t u32x4p __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) u32x4p g_u32x4p;

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;
constexpr int kProbeGrid = 2048;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4p* __restrict__ p,
                                                                   uint64_t per_wg, uint32_t* out) {
  const u32x4p* q = p + per_wg * blockIdx.x;
  u32x4p acc = {0u, 0u, 0u, 0u};
  for (uint64_t i = threadIdx.x; i + (kProbeUnroll - 1) * kProbeThreads < per_wg;
       i += kProbeUnroll * kProbeThreads) {
    u32x4p v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u)
      v[u] = __builtin_nontemporal_load((g_u32x4p*)(q + i + u * kProbeThreads));
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
  }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x5eed5eedu) out[0] = 1u;
}

// Bytes the probe reads from a buffer of `bytes` (whole unrolled passes only).
uint64_t read_probe_bytes(uint64_t bytes) {
  const uint64_t per = bytes / 16 / kProbeGrid;
  const uint64_t step = uint64_t(kProbeUnroll) * kProbeThreads;
  return (per / step) * step * 16 * kProbeGrid;
}

hipError_t launch_read_probe(const void* p, uint64_t bytes, uint32_t* out, hipStream_t s) {
  const uint64_t per = bytes / 16 / kProbeGrid;
  read_probe_kernel<<<kProbeGrid, kProbeThreads, 0, s>>>(static_cast<const u32x4p*>(p), per, out);
  return hipGetLastError();
}

}  // namespace strata
