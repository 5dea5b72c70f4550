// One-time weight pre-pack into the grouped GEMM's MFMA fragment order.
//
// A row-major weight tensor W[E][R][K] (R rows of row_bytes bytes each) is
// cut into blocks of 16 rows x 64 bytes.  Each block becomes one
// contiguous 1 KiB chunk in which lane l's 16 bytes sit at offset 16*l:
// row (l % 16) of the block, bytes 16*(l / 16) .. +15 of the 64-byte step.
// Chunks are ordered (expert, 16-row block, step), so the K run of a
// 16-row block is contiguous.  The transform is a byte permutation, the
// same for bf16 and e4m3 weights; it runs once when the weights are loaded
// and is not part of a forward call.
#include "moe_common.h"

namespace moe {

__global__ void __launch_bounds__(256)
pack_weights_kernel(const u32x4* __restrict__ w, size_t n_pieces, int rows, int row_bytes,
                    u32x4* __restrict__ packed) {
  const int nsteps = row_bytes / 64;
  const size_t row_vecs = (size_t)row_bytes / 16;
  for (size_t piece = (size_t)blockIdx.x * blockDim.x + threadIdx.x; piece < n_pieces;
       piece += (size_t)gridDim.x * blockDim.x) {
    const size_t chunk = piece / 64;
    const int lane = (int)(piece % 64);
    const int step = (int)(chunk % nsteps);
    const size_t block = chunk / nsteps;              // expert * (rows / 16) + row block
    const size_t row = block * 16 + (lane & 15);      // row index over all experts
    packed[piece] = w[row * row_vecs + (size_t)step * 4 + (lane >> 4)];
  }
}

}  // namespace moe

namespace moe_host {

hipError_t launch_pack(const void* w, int E, int rows, int row_bytes, void* packed,
                       hipStream_t s) {
  const size_t n_pieces = (size_t)E * rows * row_bytes / 16;
  size_t blocks = (n_pieces + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(moe::pack_weights_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<const moe::u32x4*>(w), n_pieces, rows, row_bytes,
                     static_cast<moe::u32x4*>(packed));
  return hipGetLastError();
}

}  // namespace moe_host
