// qk_probe.hip - read-stream probe: the bandwidth one launch of a given size gets
// from HBM when it has nothing to do but read.
//
// The GEMV roofline divides algorithmic bytes by kernel time and compares with the
// vendor HBM peak; this kernel measures the ceiling a launch of the same size can
// reach on the machine (start-up and drain included), so the GEMV can also be
// reported as a fraction of that.  A wavefront reads one group of KB kilobytes
// (KB 16-byte loads per lane, all issued before any use) and stores the XOR of the
// group's 32-bit words, so the loads cannot be elided and the result can be checked.
// Load-pattern variants, all with the same result:
//   - group size: 1, 2 (the default: the pattern of the fastest read-only kernels
//     measured on gfx950 at 25-33 MB), 4, 8 or 16 KB per wavefront;
//   - grid: one wavefront per group, or a persistent grid of a given number of
//     4-wavefront workgroups whose wavefronts stride over the groups;
//   - plain or non-temporal (streaming) loads.
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

template <bool NT>
__device__ __forceinline__ uint4 load16(const uint4* p) {
  if constexpr (NT) {
    uint4 v;
    v.x = __builtin_nontemporal_load(&p->x);
    v.y = __builtin_nontemporal_load(&p->y);
    v.z = __builtin_nontemporal_load(&p->z);
    v.w = __builtin_nontemporal_load(&p->w);
    return v;
  } else {
    return *p;
  }
}

// KB 16-byte pieces per lane = KB kilobytes per wavefront and group.  Wavefront w of
// the grid reads groups w, w + nwaves, ... (one group each when the grid covers all
// groups).
template <int KB, bool NT>
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint4* __restrict__ src, int64_t n16,
                                                                   int64_t ngroups, uint32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * (kProbeThreads / 64);
  for (int64_t group = static_cast<int64_t>(blockIdx.x) * (kProbeThreads / 64) + wave_id(); group < ngroups;
       group += nwaves) {  // wave-uniform
    const int64_t i0 = group * (64 * KB) + lane;
    uint4 v[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int64_t i = i0 + 64 * k;
      v[k] = (i < n16) ? load16<NT>(src + i) : make_uint4(0u, 0u, 0u, 0u);
    }
    uint32_t x = 0;
#pragma unroll
    for (int k = 0; k < KB; ++k) x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    x = xor_dpp(x);
    if (lane == 0) out[group] = x;
  }
}

template <int KB, bool NT>
hipError_t launch_probe(const uint4* p, int64_t n16, uint32_t* out, int64_t grid_blocks, hipStream_t s,
                        hipEvent_t e0, hipEvent_t e1) {
  const int64_t ngroups = (n16 + 64 * KB - 1) / (64 * KB);
  const int64_t need = (ngroups + kProbeThreads / 64 - 1) / (kProbeThreads / 64);
  unsigned grid = 0;
  if (!launch_grid(grid_blocks > 0 ? std::min(grid_blocks, need) : need, kProbeThreads, &grid))
    return hipErrorInvalidConfiguration;
  auto k = read_probe_kernel<KB, NT>;
  if (e0 != nullptr || e1 != nullptr) {
    hipExtLaunchKernelGGL(k, dim3(grid), dim3(kProbeThreads), 0, s, e0, e1, 0, p, n16, ngroups, out);
  } else {
    k<<<grid, kProbeThreads, 0, s>>>(p, n16, ngroups, out);
  }
  return hipGetLastError();
}

template <bool NT>
hipError_t launch_probe_kb(int kb, const uint4* p, int64_t n16, uint32_t* out, int64_t grid_blocks,
                           hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  switch (kb) {
    case 1: return launch_probe<1, NT>(p, n16, out, grid_blocks, s, e0, e1);
    case 2: return launch_probe<2, NT>(p, n16, out, grid_blocks, s, e0, e1);
    case 4: return launch_probe<4, NT>(p, n16, out, grid_blocks, s, e0, e1);
    case 8: return launch_probe<8, NT>(p, n16, out, grid_blocks, s, e0, e1);
    case 16: return launch_probe<16, NT>(p, n16, out, grid_blocks, s, e0, e1);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool read_probe_kb_ok(int kb) { return kb == 1 || kb == 2 || kb == 4 || kb == 8 || kb == 16; }

hipError_t launch_read_probe(const uint8_t* src, int64_t bytes, uint32_t* out, int kb, int64_t grid_blocks,
                             int nontemporal, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const int64_t n16 = bytes / 16;
  const uint4* p = reinterpret_cast<const uint4*>(src);
  if (nontemporal) return launch_probe_kb<true>(kb, p, n16, out, grid_blocks, s, e0, e1);
  return launch_probe_kb<false>(kb, p, n16, out, grid_blocks, s, e0, e1);
}

}  // namespace qk
