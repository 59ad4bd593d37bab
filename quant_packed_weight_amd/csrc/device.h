// device.h -- gfx950 device helpers shared by the libgemmq kernels: raw loads,
// binary16 conversion and the register-level super-block unpacker (step a2 of
// the packed linear layer: the weights are decoded inside the kernel and never
// widened in memory -- PocketLLM README, "What it runs").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gemmq {

constexpr int kQK = 256;
constexpr int kQ4KBytes = 144;
constexpr int kQ6KBytes = 210;
constexpr int kQ8KBytes = 292;

// 16-byte vector with only 4-byte alignment promised: gfx950 global loads accept
// dword-aligned addresses for dwordx4, so this still lowers to one load.
struct __attribute__((aligned(4))) u32x4 {
  uint32_t x, y, z, w;
};

__device__ __forceinline__ u32x4 ld16(const uint8_t* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ uint4 ld16a(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint32_t ld4(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
__device__ __forceinline__ uint2 ld8(const uint8_t* p) {
  struct __attribute__((aligned(4))) u2 { uint32_t x, y; };
  u2 v = *reinterpret_cast<const u2*>(p);
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint16_t ld2(const uint8_t* p) { return *reinterpret_cast<const uint16_t*>(p); }

// binary16 bits -> f32 (exact; f16 denormals are preserved by the kernel's
// float mode).
__device__ __forceinline__ float f16_to_f32(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xffffu));
}

// ---------------------------------------------------------------- q4_K scales
// The 12 scale bytes as three words h1 = s[0..3], h2 = s[4..7], h3 = s[8..11].
// Sub-blocks 0..3: scale = low 6 bits of s[j], min = low 6 bits of s[j+4].
// Sub-blocks 4..7: low 4 bits from s[j+4] (scale: low nibble, min: high nibble),
// top 2 bits from bits 6..7 of s[j-4] (scale) and of s[j] (min).
// All eight values of each kind come out packed one per byte.
struct Q4KScales {
  uint32_t sc_lo, sc_hi;  // scales of sub-blocks 0..3 and 4..7, one per byte
  uint32_t mn_lo, mn_hi;  // mins, same packing
};

__device__ __forceinline__ Q4KScales q4k_scales(uint32_t h1, uint32_t h2, uint32_t h3) {
  Q4KScales s;
  s.sc_lo = h1 & 0x3f3f3f3fu;
  s.mn_lo = h2 & 0x3f3f3f3fu;
  s.sc_hi = (h3 & 0x0f0f0f0fu) | ((h1 >> 2) & 0x30303030u);
  s.mn_hi = ((h3 >> 4) & 0x0f0f0f0fu) | ((h2 >> 2) & 0x30303030u);
  return s;
}

// Byte `j` (0..7) of a packed lo/hi pair.
__device__ __forceinline__ uint32_t byte_of(uint32_t lo, uint32_t hi, int j) {
  uint32_t w = j < 4 ? lo : hi;
  return (w >> (8 * (j & 3))) & 0xffu;
}

// q4_K quants: a word of qs bytes holds four low nibbles (the 4 weights of the
// first sub-block of its 64-weight group) and four high nibbles (the second).
__device__ __forceinline__ uint32_t lo_nib(uint32_t w) { return w & 0x0f0f0f0fu; }
__device__ __forceinline__ uint32_t hi_nib(uint32_t w) { return (w >> 4) & 0x0f0f0f0fu; }

// ---------------------------------------------------------------- q6_K quants
// Four 6-bit quants (0..63, one per byte) of quarter c of a 128-weight half:
// low 4 bits from a ql word (low nibbles for c < 2, high nibbles otherwise), top
// 2 bits from bits 2c..2c+1 of each byte of the matching qh word.
// The qh word is rotated right by 2c - 4 (mod 32), which puts bits 2c, 2c+1 of
// each byte at bits 4, 5 of the same byte; the other bits of the rotation are
// masked off, so one rotate and one and-or replace a shift, a mask and a
// shift-or.
__device__ __forceinline__ uint32_t q6k_quad(uint32_t qlw, uint32_t qhw, int c) {
  const uint32_t low = (c < 2 ? qlw : (qlw >> 4)) & 0x0f0f0f0fu;
  const uint32_t high = __builtin_amdgcn_alignbit(qhw, qhw, (uint32_t)(2 * c - 4) & 31u);
  return (high & 0x30303030u) | low;
}

// Loads n dwords starting at a 2-byte-aligned address: reads the dword-aligned
// span that covers them (n+1 dwords, never past `p + 4n + 2`) and shifts.
template <int n>
__device__ __forceinline__ void ld_dwords_a2(const uint8_t* p, uint32_t (&out)[n]) {
  // the pointer is stepped back rather than rebuilt from an integer, so that
  // the loads keep the global address space (not flat loads)
  const uint32_t sh = (uint32_t)(reinterpret_cast<uintptr_t>(p) & 3u);  // 0 or 2
  const uint32_t* base = reinterpret_cast<const uint32_t*>(p - sh);
  uint32_t raw[n + 1];
#pragma unroll
  for (int i = 0; i < n; ++i) raw[i] = base[i];
  // the last dword is only needed when the span is misaligned; when aligned it
  // would lie past the n dwords asked for, so it is not read then.
  raw[n] = sh ? base[n] : 0u;
#pragma unroll
  for (int i = 0; i < n; ++i) out[i] = __builtin_amdgcn_alignbyte(raw[i + 1], raw[i], sh);
}

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

__device__ __forceinline__ float wave_sum_xor(float v, int mask) {
  return v + __shfl_xor(v, mask, 64);
}

}  // namespace gemmq
