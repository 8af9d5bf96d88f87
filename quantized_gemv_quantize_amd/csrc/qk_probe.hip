// qk_probe.hip - read-stream probe: the bandwidth one launch of a given size gets
// from HBM when it has nothing to do but read.
//
// The GEMV roofline divides algorithmic bytes by kernel time and compares with the
// vendor HBM peak; this kernel measures the ceiling a launch of the same size can
// reach on the machine (start-up and drain included), so the GEMV can also be
// reported as a fraction of that.  Each wavefront reads one 2048-byte group with
// two 16-byte loads per lane, all issued before any use (the load pattern of the
// fastest read-only kernels measured on gfx950 at 25-33 MB), and stores the XOR of
// the group's 32-bit words, so the loads cannot be elided and the result can be
// checked.
#include <hip/hip_ext.h>

#include "qk_device.h"
#include "qk_internal.h"

namespace qk {
namespace {

constexpr int kProbeThreads = 256;

__device__ __forceinline__ uint32_t xor_dpp(uint32_t v) {
  v ^= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xB1, 0xF, 0xF, false));
  v ^= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4E, 0xF, 0xF, false));
  v ^= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x141, 0xF, 0xF, false));
  v ^= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x140, 0xF, 0xF, false));
  // lanes 15, 31, 47, 63 now hold their row's XOR
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 15)) ^
         static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 31)) ^
         static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 47)) ^
         static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint4* __restrict__ src, int64_t n16,
                                                                   int64_t ngroups, uint32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t group = static_cast<int64_t>(blockIdx.x) * (kProbeThreads / 64) + wave_id();
  if (group >= ngroups) return;  // wave-uniform
  const int64_t i0 = group * 128 + lane, i1 = i0 + 64;
  uint4 a = make_uint4(0u, 0u, 0u, 0u), b = make_uint4(0u, 0u, 0u, 0u);
  if (i0 < n16) a = src[i0];
  if (i1 < n16) b = src[i1];
  const uint32_t v = xor_dpp(a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w);
  if (lane == 0) out[group] = v;
}

}  // namespace

hipError_t launch_read_probe(const uint8_t* src, int64_t bytes, uint32_t* out, hipStream_t s, hipEvent_t e0,
                             hipEvent_t e1) {
  const int64_t n16 = bytes / 16;
  const int64_t ngroups = (n16 + 127) / 128;
  unsigned grid = 0;
  if (!launch_grid((ngroups + kProbeThreads / 64 - 1) / (kProbeThreads / 64), kProbeThreads, &grid))
    return hipErrorInvalidConfiguration;
  const uint4* p = reinterpret_cast<const uint4*>(src);
  if (e0 != nullptr || e1 != nullptr) {
    hipExtLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(kProbeThreads), 0, s, e0, e1, 0, p, n16, ngroups, out);
  } else {
    read_probe_kernel<<<grid, kProbeThreads, 0, s>>>(p, n16, ngroups, out);
  }
  return hipGetLastError();
}

}  // namespace qk
