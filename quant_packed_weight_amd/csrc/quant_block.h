// quant_block.h -- one q8_K block quantized by one 64-lane wavefront.
//
// The CPU gemm_quant on the pages quantizes activations to int8 blocks, the
// llama.cpp way, before its packed dot (molayo article "PocketLLM: 단일
// 가속기에서 대규모 언어 모델 실행", status row "src/ -- C++ engine").  That
// q8_K block stores per 256 values an f32 scale d, the 256 int8 values and 16
// int16 sums of 16 consecutive values.  Lane l holds values
// 4l..4l+3.  Arithmetic (shared by the standalone quantizer and the fused
// GEMV, so both produce the same bytes): d = amax / 127 as a correctly rounded
// f32 division; q = rint(x / d) (correctly rounded division, round half to
// even) clamped to [-127, 127]; a zero d gives an all-zero block.

#pragma once
#include "device.h"

namespace gemmq {

// Exchange with lane ^ D inside the wave: DPP quad permutes for 1 and 2,
// ds_swizzle (xor mode, within 32-lane halves) for 4, 8 and 16, a bpermute for 32.
template <int D>
__device__ __forceinline__ int qb_xor(int v) {
  if constexpr (D == 1)
    return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
  else if constexpr (D == 2)
    return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
  else if constexpr (D == 4 || D == 8 || D == 16)
    return __builtin_amdgcn_ds_swizzle(v, 0x1F | (D << 10));
  else
    return __shfl_xor(v, D, 64);
}

template <int D>
__device__ __forceinline__ float qb_xor_f(float v) {
  return __builtin_bit_cast(float, qb_xor<D>(__builtin_bit_cast(int, v)));
}

// The lane's share of a quantized block.
struct Q8Lane {
  float d;          // the block's scale (all lanes)
  uint32_t packed;  // int8 values 4l..4l+3, little-endian
  uint32_t sums;    // lanes 8j: sums of groups 2j (low half) and 2j+1 (high half)
};

// Every lane of the wave must be active.
__device__ __forceinline__ Q8Lane q8k_block(float4 v) {
  float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  a = fmaxf(a, qb_xor_f<1>(a));
  a = fmaxf(a, qb_xor_f<2>(a));
  a = fmaxf(a, qb_xor_f<4>(a));
  a = fmaxf(a, qb_xor_f<8>(a));
  a = fmaxf(a, qb_xor_f<16>(a));
  a = fmaxf(a, qb_xor_f<32>(a));

  Q8Lane r;
  r.d = a / 127.0f;
  int q0 = 0, q1 = 0, q2 = 0, q3 = 0;
  if (r.d != 0.0f) {  // wave-uniform
    q0 = (int)fminf(fmaxf(rintf(v.x / r.d), -127.0f), 127.0f);
    q1 = (int)fminf(fmaxf(rintf(v.y / r.d), -127.0f), 127.0f);
    q2 = (int)fminf(fmaxf(rintf(v.z / r.d), -127.0f), 127.0f);
    q3 = (int)fminf(fmaxf(rintf(v.w / r.d), -127.0f), 127.0f);
  }
  r.packed = (uint32_t)(q0 & 0xff) | ((uint32_t)(q1 & 0xff) << 8) |
             ((uint32_t)(q2 & 0xff) << 16) | ((uint32_t)(q3 & 0xff) << 24);
  // group g = 16 values = lanes 4g..4g+3; after two xor steps every lane of the
  // group holds its sum, and lane 8j reads group 2j+1's from lane 8j+4
  int s = q0 + q1 + q2 + q3;
  s += qb_xor<1>(s);
  s += qb_xor<2>(s);
  const int s_next = qb_xor<4>(s);
  r.sums = (uint32_t)(s & 0xffff) | ((uint32_t)(s_next & 0xffff) << 16);
  return r;
}

// Stores the lane's share in the q8_K layout (d | 256 int8 | 16 int16) at `out`.
__device__ __forceinline__ void q8k_store(uint8_t* out, const Q8Lane& q, int lane) {
  *reinterpret_cast<uint32_t*>(out + 4 + 4 * lane) = q.packed;
  if ((lane & 7) == 0) *reinterpret_cast<uint32_t*>(out + 260 + 2 * (lane >> 2)) = q.sums;
  if (lane == 0) *reinterpret_cast<float*>(out) = q.d;
}

}  // namespace gemmq
