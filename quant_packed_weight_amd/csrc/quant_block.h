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

// DPP moves inside 16-lane rows (bound_ctrl: lanes without a source read 0).
template <int CTRL>
__device__ __forceinline__ int qb_dpp(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}
constexpr int kQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kRowRor4 = 0x124;  // rotate right by 4 within the row
constexpr int kRowRor8 = 0x128;
constexpr int kRowShl4 = 0x104;  // lane i reads lane i + 4 of its row

// The lane's share of a quantized block.
struct Q8Lane {
  float d;          // the block's scale (all lanes)
  uint32_t packed;  // int8 values 4l..4l+3, little-endian
  uint32_t sums;    // lanes 8j: sums of groups 2j (low half) and 2j+1 (high half)
};

// Every lane of the wave must be active.
__device__ __forceinline__ Q8Lane q8k_block(float4 v) {
  // amax as the largest |x| bit pattern (for non-negative finite floats the
  // integer order is the float order): DPP inside each 16-lane row, then the
  // four row maxima read back as scalars
  uint32_t a = __builtin_bit_cast(uint32_t, v.x) & 0x7fffffffu;
  a = max(a, __builtin_bit_cast(uint32_t, v.y) & 0x7fffffffu);
  a = max(a, __builtin_bit_cast(uint32_t, v.z) & 0x7fffffffu);
  a = max(a, __builtin_bit_cast(uint32_t, v.w) & 0x7fffffffu);
  a = max(a, (uint32_t)qb_dpp<kQuadXor1>((int)a));
  a = max(a, (uint32_t)qb_dpp<kQuadXor2>((int)a));
  a = max(a, (uint32_t)qb_dpp<kRowRor4>((int)a));
  a = max(a, (uint32_t)qb_dpp<kRowRor8>((int)a));
  const uint32_t r01 = max((uint32_t)__builtin_amdgcn_readlane((int)a, 0),
                           (uint32_t)__builtin_amdgcn_readlane((int)a, 16));
  const uint32_t r23 = max((uint32_t)__builtin_amdgcn_readlane((int)a, 32),
                           (uint32_t)__builtin_amdgcn_readlane((int)a, 48));
  const float amax = __builtin_bit_cast(float, max(r01, r23));

  Q8Lane r;
  r.d = amax / 127.0f;
  int q0 = 0, q1 = 0, q2 = 0, q3 = 0;
  if (r.d != 0.0f) {  // wave-uniform
    q0 = (int)fminf(fmaxf(rintf(v.x / r.d), -127.0f), 127.0f);
    q1 = (int)fminf(fmaxf(rintf(v.y / r.d), -127.0f), 127.0f);
    q2 = (int)fminf(fmaxf(rintf(v.z / r.d), -127.0f), 127.0f);
    q3 = (int)fminf(fmaxf(rintf(v.w / r.d), -127.0f), 127.0f);
  }
  r.packed = (uint32_t)(q0 & 0xff) | ((uint32_t)(q1 & 0xff) << 8) |
             ((uint32_t)(q2 & 0xff) << 16) | ((uint32_t)(q3 & 0xff) << 24);
  // group g = 16 values = lanes 4g..4g+3; after two quad steps every lane of
  // the group holds its sum, and lane 8j reads group 2j+1's from lane 8j+4
  int s = q0 + q1 + q2 + q3;
  s += qb_dpp<kQuadXor1>(s);
  s += qb_dpp<kQuadXor2>(s);
  const int s_next = qb_dpp<kRowShl4>(s);
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
