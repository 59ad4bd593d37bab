// decode.hip -- diagnostic export of step a2: packed weights -> f32 using the
// same unpacking helpers as the matmul kernels (device.h).  Not on the compute
// path; it exists so the unpacker can be checked bit for bit.
//
// q4_K: w = fma(d*sc, q, -(dmin*m)).  Both products are exact in f32 (at most
// 17 significant bits), so the fused multiply-add rounds the exact value
// d*sc*q - dmin*m once.  q6_K: (d*sc)*(q-32) is exact (at most 23 bits).
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

int launch_decode(int fmt, const uint8_t* W, float* Wf, int64_t N, int64_t K, hipStream_t st) {
  const int64_t nseg = N * (K / kQK) * 16;
  const int64_t grid = (nseg + 255) / 256;
  if (grid > 0x7fffffffLL) return -1;
  if (fmt == 12)
    hipLaunchKernelGGL(decode_q4K_kernel, dim3((uint32_t)grid), dim3(256), 0, st, W, Wf, nseg);
  else
    hipLaunchKernelGGL(decode_q6K_kernel, dim3((uint32_t)grid), dim3(256), 0, st, W, Wf, nseg);
  return 0;
}

}  // namespace gemmq
