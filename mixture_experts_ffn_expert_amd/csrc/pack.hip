// pack.hip -- conversion of expert weights into the library's packed layout.
//
// The grouped expert GEMMs (gemm.hip) read weights as 1 KiB blocks of 16
// rows x 32 k in the lane order of one 16 x 32 MFMA operand, so that every
// weight load of a wavefront is one contiguous 1 KiB (the layout is described
// in gemm.hip). This kernel writes that layout once, when weights are loaded;
// it is not part of a layer step. One thread moves one 16-byte chunk.
#include "launch.h"

namespace moe {

__global__ __launch_bounds__(256) void pack_kernel(const uint16_t* __restrict__ w, int E, int R,
                                                   int kdim, int gateup, size_t per_expert,
                                                   uint16_t* __restrict__ out) {
  const size_t chunks_per_expert = per_expert / 16;
  const size_t total = (size_t)E * chunks_per_expert;
  const int nkb = packed_nkb(kdim);
  const int I = R / 2;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const size_t e = idx / chunks_per_expert;
    const size_t rem = idx - e * chunks_per_expert;
    const int blk = (int)(rem / 64);
    const int q = (int)(rem % 64);
    const int c = q >> 4, r = q & 15;
    int row, kb;
    bool ok;
    if (gateup) {
      const int f = blk & 1;
      kb = (blk >> 1) % nkb;
      const int cb = (blk >> 1) / nkb;
      const int col = cb * 16 + r;
      ok = col < I;
      row = (f ? I : 0) + col;
    } else {
      kb = blk % nkb;
      row = (blk / nkb) * 16 + r;
      ok = row < R;
    }
    const int k = kb * 32 + c * 8;
    ok = ok && k < kdim;  // kdim is a multiple of 8: a chunk is all in or all out
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (ok) v = *reinterpret_cast<const uint4*>(w + (e * R + row) * (size_t)kdim + k);
    *reinterpret_cast<uint4*>(out + idx * 8) = v;
  }
}

hipError_t launch_pack(const uint16_t* w, int E, int R, int kdim, int gateup, uint16_t* out,
                       hipStream_t s) {
  const size_t per_expert = packed_expert_bytes(R, kdim, gateup != 0);
  const size_t total = (size_t)E * per_expert / 16;
  const size_t want = (total + 255) / 256;
  const unsigned grid = (unsigned)(want < 8192 ? want : 8192);
  hipLaunchKernelGGL(pack_kernel, dim3(grid), dim3(256), 0, s, w, E, R, kdim, gateup, per_expert,
                     out);
  return hipGetLastError();
}

}  // namespace moe
