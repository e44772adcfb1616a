// Which XCD (accelerated compute die) each work group of a launch runs on.
//
// The attention work lists place every (window, head) group's items on one
// XCD by assuming that work group b runs on XCD b mod 8 (the dispatcher hands
// work groups to the dies round-robin); this probe lets the host check that
// once per device: lane 0 of each work group stores the XCC_ID hardware
// register (gfx9.4+ hwreg 20, bits 3:0).

#include "wsp_internal.h"

namespace wsp {

namespace {

// s_getreg operand: hwreg XCC_ID (20), offset 0, 4 bits.
constexpr int kHwRegXccId = ((4 - 1) << 11) | (0 << 6) | 20;

__global__ __launch_bounds__(64) void xcd_probe_kernel(int32_t *__restrict__ xcc) {
    if (threadIdx.x == 0) xcc[blockIdx.x] = __builtin_amdgcn_s_getreg(kHwRegXccId) & 0xF;
}

}  // namespace

hipError_t launch_xcd_probe(int32_t *xcc, int n_blocks, hipStream_t s) {
    if (n_blocks <= 0) return hipSuccess;
    xcd_probe_kernel<<<dim3(unsigned(n_blocks)), dim3(64), 0, s>>>(xcc);
    return hipGetLastError();
}

}  // namespace wsp
