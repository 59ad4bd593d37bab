// decode.hip -- diagnostic export of step a2: packed weights -> f32 using the
// same unpacking helpers as the matmul kernels (device.h).  Not on the compute
// path; it exists so the unpacker can be checked bit for bit.
//
// q2_K, q4_K, q5_K: w = fma(d*sc, q, -(dmin*m)).  Both products are exact in
// f32 (at most 17 significant bits), so the fused multiply-add rounds the exact
// value d*sc*q - dmin*m once.  q3_K: (d*sc)*q and q6_K: (d*sc)*(q-32) are exact
// (at most 20 and 23 bits).
#include "device.h"
#include "launch.h"

namespace gemmq {

// one thread per 16 consecutive weights of a block
__global__ __launch_bounds__(256) void decode_q4K_kernel(const uint8_t* __restrict__ W,
                                                         float* __restrict__ out, int64_t nseg) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= nseg) return;
  const int64_t blk = t >> 4;
  const int seg = (int)(t & 15);  // weights 16seg .. 16seg+15
  const uint8_t* wb = W + blk * kQ4KBytes;
  const uint4 hd = ld16a(wb);
  const int j = seg >> 1;           // sub-block
  const int g = seg >> 2;           // 64-weight group
  const int r0 = 16 * (seg & 3);    // offset inside the group: 0, 16 -> low; 32, 48 -> high
  const uint4 qv = ld16a(wb + 16 + 32 * g + (r0 & 31));
  const Q4KScales s = q4k_scales(hd.y, hd.z, hd.w);
  const float d = f16_to_f32(hd.x), dmin = f16_to_f32(hd.x >> 16);
  const float d1 = d * (float)byte_of(s.sc_lo, s.sc_hi, j);
  const float m1 = dmin * (float)byte_of(s.mn_lo, s.mn_hi, j);
  const uint32_t words[4] = {qv.x, qv.y, qv.z, qv.w};
  float* o = out + blk * kQK + 16 * seg;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t q4 = r0 < 32 ? lo_nib(words[k]) : hi_nib(words[k]);
    float4 v;
    v.x = fmaf(d1, (float)(q4 & 0xffu), -m1);
    v.y = fmaf(d1, (float)((q4 >> 8) & 0xffu), -m1);
    v.z = fmaf(d1, (float)((q4 >> 16) & 0xffu), -m1);
    v.w = fmaf(d1, (float)(q4 >> 24), -m1);
    *reinterpret_cast<float4*>(o + 4 * k) = v;
  }
}

__global__ __launch_bounds__(256) void decode_q6K_kernel(const uint8_t* __restrict__ W,
                                                         float* __restrict__ out, int64_t nseg) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= nseg) return;
  const int64_t blk = t >> 4;
  const int seg = (int)(t & 15);          // sub-block = weights 16seg .. 16seg+15
  const int hh = seg >> 3, c = (seg & 7) >> 1, l0 = 16 * (seg & 1);
  const uint8_t* wb = W + blk * kQ6KBytes;
  uint32_t ql[4], qh[4];
  ld_dwords_a2<4>(wb + 64 * hh + 32 * (c & 1) + l0, ql);
  ld_dwords_a2<4>(wb + 128 + 32 * hh + l0, qh);
  const int sc = (int)(int8_t)(ld2(wb + 192 + (seg & ~1)) >> (8 * (seg & 1)));
  const float ds = f16_to_f32(ld2(wb + 208)) * (float)sc;
  float* o = out + blk * kQK + 16 * seg;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t q = q6k_quad(ql[k], qh[k], c);
    float4 v;
    v.x = ds * (float)((int)(q & 0xffu) - 32);
    v.y = ds * (float)((int)((q >> 8) & 0xffu) - 32);
    v.z = ds * (float)((int)((q >> 16) & 0xffu) - 32);
    v.w = ds * (float)((int)(q >> 24) - 32);
    *reinterpret_cast<float4*>(o + 4 * k) = v;
  }
}

// q2_K: thread = sub-block s (16 weights): quarter (s%8)/2 of half s/8, bytes
// 16(s%2).. of that half's 32 quant bytes; scale/min byte s.
__global__ __launch_bounds__(256) void decode_q2K_kernel(const uint8_t* __restrict__ W,
                                                         float* __restrict__ out, int64_t nseg) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= nseg) return;
  const int64_t blk = t >> 4;
  const int s = (int)(t & 15);
  const int h = s >> 3, qq = (s & 7) >> 1, l0 = 16 * (s & 1);
  const uint8_t* wb = W + blk * 84;
  const u32x4 qv = ld16(wb + 16 + 32 * h + l0);
  const uint32_t sm = (ld4(wb + 4 * (s >> 2)) >> (8 * (s & 3))) & 0xffu;
  const uint32_t dd = ld4(wb + 80);
  const float d1 = f16_to_f32(dd) * (float)(sm & 15u);
  const float m1 = f16_to_f32(dd >> 16) * (float)(sm >> 4);
  const uint32_t words[4] = {qv.x, qv.y, qv.z, qv.w};
  float* o = out + blk * kQK + 16 * s;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t q = (words[k] >> (2 * qq)) & 0x03030303u;
    float4 v;
    v.x = fmaf(d1, (float)(q & 0xffu), -m1);
    v.y = fmaf(d1, (float)((q >> 8) & 0xffu), -m1);
    v.z = fmaf(d1, (float)((q >> 16) & 0xffu), -m1);
    v.w = fmaf(d1, (float)(q >> 24), -m1);
    *reinterpret_cast<float4*>(o + 4 * k) = v;
  }
}

// q3_K: thread = sub-block s; the low parts as q2_K's quants, the mask bit
// 4(s/8) + (s%8)/2 of mask bytes 16(s%2)..; 110-byte blocks are 2-byte aligned
// and every read stays inside the block.
__global__ __launch_bounds__(256) void decode_q3K_kernel(const uint8_t* __restrict__ W,
                                                         float* __restrict__ out, int64_t nseg) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= nseg) return;
  const int64_t blk = t >> 4;
  const int s = (int)(t & 15);
  const int h = s >> 3, qq = (s & 7) >> 1, l0 = 16 * (s & 1);
  const uint8_t* wb = W + blk * 110;
  uint32_t qs[4], hm[4];
  ld_dwords_a2<4>(wb + 32 + 32 * h + l0, qs);
  ld_dwords_a2<4>(wb + l0, hm);
  // scale s = 4g + k: low nibble of byte 4(g&1) + k (high nibble when g >= 2),
  // top bits 2g..2g+1 of byte 8 + k
  const int g = s >> 2, k = s & 3;
  const int blo = 4 * (g & 1) + k, bhi = 8 + k;
  const uint32_t lo = (((uint32_t)ld2(wb + 96 + (blo & ~1)) >> (8 * (blo & 1))) >> (4 * (g >> 1))) & 15u;
  const uint32_t hi = (((uint32_t)ld2(wb + 96 + (bhi & ~1)) >> (8 * (bhi & 1))) >> (2 * g)) & 3u;
  const float ds = f16_to_f32(ld2(wb + 108)) * (float)((int)(lo | (hi << 4)) - 32);
  float* o = out + blk * kQK + 16 * s;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t u = ((qs[j] >> (2 * qq)) & 0x03030303u) |
                       (((hm[j] >> (4 * h + qq)) & 0x01010101u) << 2);  // q + 4
    float4 v;
    v.x = ds * (float)((int)(u & 0xffu) - 4);
    v.y = ds * (float)((int)((u >> 8) & 0xffu) - 4);
    v.z = ds * (float)((int)((u >> 16) & 0xffu) - 4);
    v.w = ds * (float)((int)(u >> 24) - 4);
    *reinterpret_cast<float4*>(o + 4 * j) = v;
  }
}

// q5_K: thread = 16 weights (seg) of sub-block seg/2, laid out as q4_K's plus
// high bit 2(seg/4) + (seg%4 >= 2) of high-bit bytes 16(seg%2)..
__global__ __launch_bounds__(256) void decode_q5K_kernel(const uint8_t* __restrict__ W,
                                                         float* __restrict__ out, int64_t nseg) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= nseg) return;
  const int64_t blk = t >> 4;
  const int seg = (int)(t & 15);
  const uint8_t* wb = W + blk * 176;
  const uint4 hd = ld16a(wb);
  const int j = seg >> 1, g = seg >> 2, r0 = 16 * (seg & 3);
  const uint4 qv = ld16a(wb + 48 + 32 * g + (r0 & 31));
  const uint4 hv = ld16a(wb + 16 + (r0 & 31));
  const Q4KScales sm = q4k_scales(hd.y, hd.z, hd.w);
  const float d1 = f16_to_f32(hd.x) * (float)byte_of(sm.sc_lo, sm.sc_hi, j);
  const float m1 = f16_to_f32(hd.x >> 16) * (float)byte_of(sm.mn_lo, sm.mn_hi, j);
  const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w}, hw[4] = {hv.x, hv.y, hv.z, hv.w};
  const int hb = 2 * g + (r0 >= 32 ? 1 : 0);
  float* o = out + blk * kQK + 16 * seg;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t q = (r0 < 32 ? lo_nib(qw[k]) : hi_nib(qw[k])) | (((hw[k] >> hb) & 0x01010101u) << 4);
    float4 v;
    v.x = fmaf(d1, (float)(q & 0xffu), -m1);
    v.y = fmaf(d1, (float)((q >> 8) & 0xffu), -m1);
    v.z = fmaf(d1, (float)((q >> 16) & 0xffu), -m1);
    v.w = fmaf(d1, (float)(q >> 24), -m1);
    *reinterpret_cast<float4*>(o + 4 * k) = v;
  }
}

int launch_decode(int fmt, const uint8_t* W, float* Wf, int64_t N, int64_t K, hipStream_t st) {
  const int64_t nseg = N * (K / kQK) * 16;
  const int64_t grid = (nseg + 255) / 256;
  if (grid > 0x7fffffffLL) return -1;
  const dim3 g((uint32_t)grid), b(256);
  switch (fmt) {
    case 10: hipLaunchKernelGGL(decode_q2K_kernel, g, b, 0, st, W, Wf, nseg); break;
    case 11: hipLaunchKernelGGL(decode_q3K_kernel, g, b, 0, st, W, Wf, nseg); break;
    case 12: hipLaunchKernelGGL(decode_q4K_kernel, g, b, 0, st, W, Wf, nseg); break;
    case 13: hipLaunchKernelGGL(decode_q5K_kernel, g, b, 0, st, W, Wf, nseg); break;
    default: hipLaunchKernelGGL(decode_q6K_kernel, g, b, 0, st, W, Wf, nseg);
  }
  return 0;
}

}  // namespace gemmq
