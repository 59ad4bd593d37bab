// gemv.hip -- step a3: the decode-time packed GEMV, M = 1..8 activation rows.
//
// Decode time on the pages is the walk over the packed weights (molayo article
// "PocketLLM: 단일 가속기에서 대규모 언어 모델 실행", status row "src/ -- C++
// engine": the packed dot walks each weight row once per tile of activation
// rows).  On gfx950 that walk is an HBM stream, so the kernel is shaped for it:
//
//  * one 64-lane wavefront owns a tile of R weight rows; eight lanes share a
//    super-block, each taking one 16-byte chunk of its packed quants (q4_K) or
//    one 32-weight quarter (q6_K), so a wave reads eight consecutive blocks of a
//    row per step and the row's bytes stream in order;
//  * the lane's activation fragment for a block position is loaded once and
//    reused for all R rows of the tile;
//  * integer dot products run on v_dot4 (int8 x int8 -> int32); the sub-block
//    scale/min correction stays in integers and one f32 fold per block and lane
//    applies d_w, dmin and d_x;
//  * the 64 lane partials of each output are summed by a fixed xor butterfly.
//
// Every output's arithmetic (per-lane block order, butterfly shape) depends only
// on K, never on M or R, so row m of an M-row call equals a one-row call on that
// row bit for bit.
#include "device.h"
#include "launch.h"

namespace gemmq {

// ---------------------------------------------------------------- q4_K
// Lane (G = lane/8, c = lane%8) takes qs bytes 16c..16c+15 of blocks G, G+8, ...
// Those bytes hold, as low nibbles, weights 64g+16h+t of sub-block 2g and, as high
// nibbles, weights 64g+32+16h+t of sub-block 2g+1 (g = c/2, h = c%2, t < 16); the
// matching activation sums are groups 4g+h and 4g+2+h.
template <int MT, int R>
__global__ __launch_bounds__(256) void gemv_q4K_kernel(const uint8_t* __restrict__ W,
                                                       const uint8_t* __restrict__ Xq,
                                                       float* __restrict__ Y, int64_t N, int nb) {
  const int lane = lane_id();
  const int64_t n0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
  if (n0 >= N) return;  // wave-uniform
  const int G = lane >> 3, c = lane & 7, g = c >> 1, h = c & 1;
  const int xoff = 4 + 64 * g + 16 * h;
  const int bsoff = 260 + 8 * g;
  const int bshift = 16 * h;
  const bool upper = g >= 2;        // sub-blocks 4..7 use the second packed word
  const int sshift = 16 * (g & 1);  // byte position of sub-block 2g inside it

  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;

  for (int b = G; b < nb; b += 8) {
    float dx[MT];
    u32x4 xl[MT], xh[MT];
    int bs0[MT], bs1[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const uint8_t* xb = Xq + ((int64_t)m * nb + b) * kQ8KBytes;
      dx[m] = *reinterpret_cast<const float*>(xb);
      xl[m] = ld16(xb + xoff);
      xh[m] = ld16(xb + xoff + 32);
      const uint2 s = ld8(xb + bsoff);
      bs0[m] = (int)(int16_t)(s.x >> bshift);
      bs1[m] = (int)(int16_t)(s.y >> bshift);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      int64_t n = n0 + r;
      if (n >= N) n = N - 1;  // tail rows: read a valid row, never stored
      const uint8_t* wb = W + (n * nb + b) * kQ4KBytes;
      const uint4 hd = ld16a(wb);
      const uint4 qv = ld16a(wb + 16 + 16 * c);
      const float d = f16_to_f32(hd.x), dmin = f16_to_f32(hd.x >> 16);
      const Q4KScales s = q4k_scales(hd.y, hd.z, hd.w);
      const uint32_t scw = upper ? s.sc_hi : s.sc_lo;
      const uint32_t mnw = upper ? s.mn_hi : s.mn_lo;
      const int sc0 = (scw >> sshift) & 0xff, sc1 = (scw >> (sshift + 8)) & 0xff;
      const int mn0 = (mnw >> sshift) & 0xff, mn1 = (mnw >> (sshift + 8)) & 0xff;
      const uint32_t l0 = lo_nib(qv.x), l1 = lo_nib(qv.y), l2 = lo_nib(qv.z), l3 = lo_nib(qv.w);
      const uint32_t h0 = hi_nib(qv.x), h1 = hi_nib(qv.y), h2 = hi_nib(qv.z), h3 = hi_nib(qv.w);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        int dl = __builtin_amdgcn_sdot4((int)l0, (int)xl[m].x, 0, false);
        dl = __builtin_amdgcn_sdot4((int)l1, (int)xl[m].y, dl, false);
        dl = __builtin_amdgcn_sdot4((int)l2, (int)xl[m].z, dl, false);
        dl = __builtin_amdgcn_sdot4((int)l3, (int)xl[m].w, dl, false);
        int dh = __builtin_amdgcn_sdot4((int)h0, (int)xh[m].x, 0, false);
        dh = __builtin_amdgcn_sdot4((int)h1, (int)xh[m].y, dh, false);
        dh = __builtin_amdgcn_sdot4((int)h2, (int)xh[m].z, dh, false);
        dh = __builtin_amdgcn_sdot4((int)h3, (int)xh[m].w, dh, false);
        const int isc = sc0 * dl + sc1 * dh;
        const int imn = mn0 * bs0[m] + mn1 * bs1[m];
        float t = d * (float)isc;
        t = fmaf(-dmin, (float)imn, t);
        acc[r][m] = fmaf(dx[m], t, acc[r][m]);
      }
    }
  }

  float out = 0.0f;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float v = acc[r][m];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v = wave_sum_xor(v, off);
      if (lane == r * MT + m) out = v;
    }
  if (lane < R * MT) {
    const int r = lane / MT, m = lane - (lane / MT) * MT;
    const int64_t n = n0 + r;
    if (n < N) Y[(int64_t)m * N + n] = out;
  }
}

// ---------------------------------------------------------------- q6_K
// Lane (G = lane/8, c = lane%8) takes the 32-weight quarter q = c%4 of half
// hh = c/4 of blocks G, G+8, ...: weights 128hh + 32q + l, low bits from ql bytes
// 64hh + 32(q&1) + l, top bits from qh bytes 32hh + l, sub-blocks 8hh+2q and
// 8hh+2q+1.  Blocks are 210 bytes, so fields are only 2-byte aligned: they are
// read as dword-aligned spans and realigned in registers.
template <int MT, int R>
__global__ __launch_bounds__(256) void gemv_q6K_kernel(const uint8_t* __restrict__ W,
                                                       const uint8_t* __restrict__ Xq,
                                                       float* __restrict__ Y, int64_t N, int nb) {
  const int lane = lane_id();
  const int64_t n0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
  if (n0 >= N) return;
  const int G = lane >> 3, c = lane & 7, hh = c >> 2, q = c & 3;
  const int qloff = 64 * hh + 32 * (q & 1);
  const int qhoff = 128 + 32 * hh;
  const int scoff = 192 + 8 * hh + 2 * q;
  const int xoff = 4 + 128 * hh + 32 * q;
  const int bsoff = 260 + 2 * (8 * hh + 2 * q);

  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;

  for (int b = G; b < nb; b += 8) {
    float dx[MT];
    u32x4 xa[MT], xb2[MT];
    int bs0[MT], bs1[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const uint8_t* xb = Xq + ((int64_t)m * nb + b) * kQ8KBytes;
      dx[m] = *reinterpret_cast<const float*>(xb);
      xa[m] = ld16(xb + xoff);
      xb2[m] = ld16(xb + xoff + 16);
      const uint32_t s = ld4(xb + bsoff);
      bs0[m] = (int)(int16_t)(s & 0xffffu);
      bs1[m] = (int)(int16_t)(s >> 16);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      int64_t n = n0 + r;
      if (n >= N) n = N - 1;
      const uint8_t* wb = W + (n * nb + b) * kQ6KBytes;
      uint32_t ql[8], qh[8];
      ld_dwords_a2<8>(wb + qloff, ql);
      ld_dwords_a2<8>(wb + qhoff, qh);
      const uint32_t scp = ld2(wb + scoff);
      const int sc0 = (int)(int8_t)(scp & 0xffu), sc1 = (int)(int8_t)(scp >> 8);
      const float d = f16_to_f32(ld2(wb + 208));
      uint32_t qq[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) qq[k] = q6k_quad(ql[k], qh[k], q);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        int d0 = __builtin_amdgcn_sdot4((int)qq[0], (int)xa[m].x, 0, false);
        d0 = __builtin_amdgcn_sdot4((int)qq[1], (int)xa[m].y, d0, false);
        d0 = __builtin_amdgcn_sdot4((int)qq[2], (int)xa[m].z, d0, false);
        d0 = __builtin_amdgcn_sdot4((int)qq[3], (int)xa[m].w, d0, false);
        int d1 = __builtin_amdgcn_sdot4((int)qq[4], (int)xb2[m].x, 0, false);
        d1 = __builtin_amdgcn_sdot4((int)qq[5], (int)xb2[m].y, d1, false);
        d1 = __builtin_amdgcn_sdot4((int)qq[6], (int)xb2[m].z, d1, false);
        d1 = __builtin_amdgcn_sdot4((int)qq[7], (int)xb2[m].w, d1, false);
        const int isc = sc0 * (d0 - 32 * bs0[m]) + sc1 * (d1 - 32 * bs1[m]);
        acc[r][m] = fmaf(dx[m], d * (float)isc, acc[r][m]);
      }
    }
  }

  float out = 0.0f;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float v = acc[r][m];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v = wave_sum_xor(v, off);
      if (lane == r * MT + m) out = v;
    }
  if (lane < R * MT) {
    const int r = lane / MT, m = lane - (lane / MT) * MT;
    const int64_t n = n0 + r;
    if (n < N) Y[(int64_t)m * N + n] = out;
  }
}

// ---------------------------------------------------------------- launch
namespace {

// Rows per wave: as many as keep at least ~2048 waves in flight (8 per CU on
// 256 CUs), at most 32 accumulators per lane.
int pick_rows(int M, int64_t N) {
  int R = 8;
  while (R > 1 && (N / R < 2048 || R * M > 32)) R >>= 1;
  return R;
}

template <int MT, int R>
void launch_one(int fmt, const uint8_t* W, const uint8_t* Xq, float* Y, int64_t N, int nb,
                hipStream_t st) {
  const int64_t waves = (N + R - 1) / R;
  const dim3 grid((uint32_t)((waves + 3) / 4));
  if (fmt == 12)
    hipLaunchKernelGGL((gemv_q4K_kernel<MT, R>), grid, dim3(256), 0, st, W, Xq, Y, N, nb);
  else
    hipLaunchKernelGGL((gemv_q6K_kernel<MT, R>), grid, dim3(256), 0, st, W, Xq, Y, N, nb);
}

template <int MT>
void launch_m(int fmt, int R, const uint8_t* W, const uint8_t* Xq, float* Y, int64_t N, int nb,
              hipStream_t st) {
  switch (R) {
    case 8: if constexpr (MT * 8 <= 32) { launch_one<MT, 8>(fmt, W, Xq, Y, N, nb, st); return; }
      [[fallthrough]];
    case 4: if constexpr (MT * 4 <= 32) { launch_one<MT, 4>(fmt, W, Xq, Y, N, nb, st); return; }
      [[fallthrough]];
    case 2: launch_one<MT, 2>(fmt, W, Xq, Y, N, nb, st); return;
    default: launch_one<MT, 1>(fmt, W, Xq, Y, N, nb, st); return;
  }
}

}  // namespace

int launch_gemv(int fmt, const uint8_t* W, const uint8_t* Xq, float* Y, int M, int64_t N,
                int64_t K, hipStream_t st) {
  const int64_t nb = K / kQK;
  if (nb > 0x7fffffffLL) return -1;
  const int R = pick_rows(M, N);
  const int64_t waves = (N + R - 1) / R;
  if ((waves + 3) / 4 > 0x7fffffffLL) return -1;
  switch (M) {
    case 1: launch_m<1>(fmt, R, W, Xq, Y, N, (int)nb, st); break;
    case 2: launch_m<2>(fmt, R, W, Xq, Y, N, (int)nb, st); break;
    case 3: launch_m<3>(fmt, R, W, Xq, Y, N, (int)nb, st); break;
    case 4: launch_m<4>(fmt, R, W, Xq, Y, N, (int)nb, st); break;
    case 5: launch_m<5>(fmt, R, W, Xq, Y, N, (int)nb, st); break;
    case 6: launch_m<6>(fmt, R, W, Xq, Y, N, (int)nb, st); break;
    case 7: launch_m<7>(fmt, R, W, Xq, Y, N, (int)nb, st); break;
    case 8: launch_m<8>(fmt, R, W, Xq, Y, N, (int)nb, st); break;
    default: return -1;
  }
  return 0;
}

}  // namespace gemmq
