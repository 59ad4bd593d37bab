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
#include "device.h"
#include "launch.h"

namespace gemmq {

__global__ __launch_bounds__(256) void quantize_q8K_kernel(const float* __restrict__ X,
                                                           uint8_t* __restrict__ Xq,
                                                           int64_t nblocks, int64_t nb,
                                                           int64_t K) {
  const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  if (blk >= nblocks) return;  // wave-uniform
  const int64_t m = blk / nb, b = blk - m * nb;
  const float4 v = *reinterpret_cast<const float4*>(X + m * K + b * kQK + 4 * lane);

  float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));

  const float d = a / 127.0f;
  int q0 = 0, q1 = 0, q2 = 0, q3 = 0;
  if (d != 0.0f) {
    q0 = (int)fminf(fmaxf(rintf(v.x / d), -127.0f), 127.0f);
    q1 = (int)fminf(fmaxf(rintf(v.y / d), -127.0f), 127.0f);
    q2 = (int)fminf(fmaxf(rintf(v.z / d), -127.0f), 127.0f);
    q3 = (int)fminf(fmaxf(rintf(v.w / d), -127.0f), 127.0f);
  }
  uint8_t* out = Xq + blk * kQ8KBytes;
  const uint32_t packed = (uint32_t)(q0 & 0xff) | ((uint32_t)(q1 & 0xff) << 8) |
                          ((uint32_t)(q2 & 0xff) << 16) | ((uint32_t)(q3 & 0xff) << 24);
  *reinterpret_cast<uint32_t*>(out + 4 + 4 * lane) = packed;

  // group g = 16 values = lanes 4g..4g+3
  int s = q0 + q1 + q2 + q3;
  s += __shfl_xor(s, 1, 64);
  s += __shfl_xor(s, 2, 64);
  const int s_next = __shfl_down(s, 4, 64);  // sum of group g+1 at lane 4g
  if ((lane & 7) == 0)
    *reinterpret_cast<uint32_t*>(out + 260 + 2 * (lane >> 2)) =
        (uint32_t)(s & 0xffff) | ((uint32_t)(s_next & 0xffff) << 16);
  if (lane == 0) *reinterpret_cast<float*>(out) = d;
}

int launch_quantize_q8K(const float* X, uint8_t* Xq, int64_t M, int64_t K, hipStream_t st) {
  const int64_t nb = K / kQK;
  const int64_t nblocks = M * nb;
  const int64_t grid = (nblocks + 3) / 4;
  if (grid > 0x7fffffffLL) return -1;
  hipLaunchKernelGGL(quantize_q8K_kernel, dim3((uint32_t)grid), dim3(256), 0, st, X, Xq, nblocks,
                     nb, K);
  return 0;
}

}  // namespace gemmq
