// quantize.hip -- step a1: f32 activations -> q8_K blocks.
//
// The CPU gemm_quant on the pages quantizes activation rows to int8 blocks
// before the packed dot, one block per thread-pool task (molayo article
// "PocketLLM: 단일 가속기에서 대규모 언어 모델 실행", status row "src/ -- C++
// engine").  Here one 64-lane wavefront owns one 256-value block: each lane
// holds four consecutive values (one 16-byte load, the wave reads 1 KiB
// contiguous), amax is a butterfly max over the wave, and the block is written
// as d | 256 int8 | 16 int16 group sums with dword stores.
//
// Arithmetic (must match the oracle bit for bit): d = amax / 127 with a
// correctly rounded f32 division; q = rint(x / d) (round half to even, correctly
// rounded division) clamped to [-127, 127]; a zero d gives an all-zero block.
#include "launch.h"
#include "quant_block.h"

namespace gemmq {

// Block `blk` of the M x K/256 blocks starts at value 256 blk of X (rows are
// contiguous), so no division by K/256 is needed.
__global__ __launch_bounds__(256) void quantize_q8K_kernel(const float* __restrict__ X,
                                                           uint8_t* __restrict__ Xq,
                                                           int64_t nblocks) {
  const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  if (blk >= nblocks) return;  // wave-uniform
  const float4 v = *reinterpret_cast<const float4*>(X + blk * kQK + 4 * lane);
  q8k_store(Xq + blk * kQ8KBytes, q8k_block(v), lane);
}

int launch_quantize_q8K(const float* X, uint8_t* Xq, int64_t M, int64_t K, hipStream_t st) {
  const int64_t nb = K / kQK;
  const int64_t nblocks = M * nb;
  const int64_t grid = (nblocks + 3) / 4;
  if (grid > 0x7fffffffLL) return -1;
  hipLaunchKernelGGL(quantize_q8K_kernel, dim3((uint32_t)grid), dim3(256), 0, st, X, Xq, nblocks);
  return 0;
}

}  // namespace gemmq
