// gemm.hip -- step a4: the prefill packed GEMM on int8 MFMA (M >= 9).
//
// The pages' prefill GEMM walks each packed weight row once per tile of
// activation rows and applies the block scales on the way (molayo article
// "PocketLLM: 단일 가속기에서 대규모 언어 모델 실행", status row "src/ -- C++
// engine": row tile of 8 activation rows; q4_K 8-column panels).  On gfx950
// the dense contraction goes to v_mfma_i32_32x32x32_i8, and the design is set
// by keeping the vector ALU off the critical path:
//
//  * The sub-block scale is folded into the weight operand.  For q4_K,
//    sc = 8a + b with a, b in 0..7, so sc*q = 8(a*q) + b*q with both products
//    in 0..105: two int8 planes whose MFMA sums, combined as 8*A + B, give
//    I_sc = sum_j sc_j * dot_j for the whole 256-weight super-block in int32.
//    For q6_K, v = sc*(q-32) in -4064..4096 splits as 128*hi + lo with
//    lo = v & 127 and hi = v >> 7 in -32..32.
//  * The q4_K min term I_min = sum_j m_j * (bsum_2j + bsum_2j+1) is a K=16
//    contraction of the activation group sums with the mins; the int16 sums are
//    split into int8 planes (bsum = 128*bh + bl) and it runs as two more MFMAs.
//  * One f32 epilogue per super-block and output:
//    y += d_x * (d * I_sc - dmin * I_min)   (q6_K: y += d_x * d * I_sc).
//
// Work decomposition: a 256-thread workgroup computes a 128 (M) x 64 (N) tile.
// Per super-block it stages the activation tile (int8 values, d_x, sum planes)
// and the weight tile, unpacked once into the two int8 planes, in LDS; then each
// of the four waves runs a 64 x 32 sub-tile (two 32x32 MFMA tiles) from LDS.
// Every output's arithmetic depends only on its own row and column, so any
// subset of rows gives identical bits.
#include "device.h"
#include "launch.h"

namespace gemmq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 128;       // activation rows per workgroup
constexpr int kBN = 64;        // weight rows (output columns) per workgroup
constexpr int kRow = 256 + 16; // LDS row stride of an int8 K-row (padded)

// LDS map (bytes)
constexpr int kOffA = 0;                       // [kBM][kRow] activation int8
constexpr int kOffPa = kOffA + kBM * kRow;     // [kBN][kRow] weight plane A (hi)
constexpr int kOffPb = kOffPa + kBN * kRow;    // [kBN][kRow] weight plane B (lo)
constexpr int kOffBs = kOffPb + kBN * kRow;    // [kBM][32]   sum planes bl | bh
constexpr int kOffDx = kOffBs + kBM * 32;      // [kBM] f32   d_x
constexpr int kOffD = kOffDx + kBM * 4;        // [kBN] f32   d
constexpr int kOffDm = kOffD + kBN * 4;        // [kBN] f32   dmin
constexpr int kOffMn = kOffDm + kBN * 4;       // [kBN][8]    mins
constexpr int kLds = kOffMn + kBN * 8;

// bytes of w (each <= 15) times a (<= 7): per 16-bit half the product stays below
// 2^16 and no byte carries into the next.
__device__ __forceinline__ uint32_t mul_bytes(uint32_t w, uint32_t a) {
  const u16x2 v = __builtin_bit_cast(u16x2, w);
  const u16x2 s = {(unsigned short)a, (unsigned short)a};
  return __builtin_bit_cast(uint32_t, v * s);
}

__device__ __forceinline__ v16i mfma(v4i a, v4i b, v16i c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void st16(uint8_t* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  *reinterpret_cast<uint4*>(p) = make_uint4(a, b, c, d);
}

// ------------------------------------------------- staging: activation tile
// thread t: row t/2, half t%2 of the 256 int8 values; half 0 also d_x, half 1
// also the two int8 planes of the 16 group sums.
__device__ __forceinline__ void stage_x(uint8_t* lds, const uint8_t* __restrict__ Xq, int64_t m0,
                                        int64_t M, int nb, int b) {
  const int t = threadIdx.x;
  const int row = t >> 1, part = t & 1;
  const int64_t m = m0 + row;
  uint8_t* dstA = lds + kOffA + row * kRow + 128 * part;
  if (m < M) {
    const uint8_t* xb = Xq + (m * nb + b) * kQ8KBytes;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4 v = ld16(xb + 4 + 128 * part + 16 * i);
      st16(dstA + 16 * i, v.x, v.y, v.z, v.w);
    }
    if (part == 0) {
      reinterpret_cast<float*>(lds + kOffDx)[row] = *reinterpret_cast<const float*>(xb);
    } else {
      const u32x4 s0 = ld16(xb + 260), s1 = ld16(xb + 276);
      const uint32_t sw[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
      uint32_t bl[4], bh[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t u0 = sw[2 * k], u1 = sw[2 * k + 1];  // sums 4k..4k+3
        bl[k] = (u0 & 0x7fu) | (((u0 >> 16) & 0x7fu) << 8) | ((u1 & 0x7fu) << 16) |
                (((u1 >> 16) & 0x7fu) << 24);
        const uint32_t h0 = (uint32_t)((int)(int16_t)(u0 & 0xffffu) >> 7) & 0xffu;
        const uint32_t h1 = (uint32_t)((int)u0 >> 23) & 0xffu;
        const uint32_t h2 = (uint32_t)((int)(int16_t)(u1 & 0xffffu) >> 7) & 0xffu;
        const uint32_t h3 = (uint32_t)((int)u1 >> 23) & 0xffu;
        bh[k] = h0 | (h1 << 8) | (h2 << 16) | (h3 << 24);
      }
      uint8_t* dstB = lds + kOffBs + row * 32;
      st16(dstB, bl[0], bl[1], bl[2], bl[3]);
      st16(dstB + 16, bh[0], bh[1], bh[2], bh[3]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) st16(dstA + 16 * i, 0, 0, 0, 0);
    if (part == 0) {
      reinterpret_cast<float*>(lds + kOffDx)[row] = 0.0f;
    } else {
      st16(lds + kOffBs + row * 32, 0, 0, 0, 0);
      st16(lds + kOffBs + row * 32 + 16, 0, 0, 0, 0);
    }
  }
}

// ------------------------------------------------- staging: q4_K weight tile
// thread t: column t/4, 64-weight group g = t%4 (qs bytes 32g..32g+31, holding
// sub-block 2g in the low nibbles and 2g+1 in the high nibbles).
__device__ __forceinline__ void stage_w_q4K(uint8_t* lds, const uint8_t* __restrict__ W,
                                            int64_t n0, int64_t N, int nb, int b) {
  const int t = threadIdx.x;
  const int col = t >> 2, g = t & 3;
  const int64_t n = n0 + col;
  uint4 hd = make_uint4(0, 0, 0, 0), q0 = hd, q1 = hd;
  if (n < N) {
    const uint8_t* wb = W + (n * nb + b) * kQ4KBytes;
    hd = ld16a(wb);
    q0 = ld16a(wb + 16 + 32 * g);
    q1 = ld16a(wb + 32 + 32 * g);
  }
  const Q4KScales s = q4k_scales(hd.y, hd.z, hd.w);
  const uint32_t scw = g >= 2 ? s.sc_hi : s.sc_lo;
  const uint32_t mnw = g >= 2 ? s.mn_hi : s.mn_lo;
  const int sh = 16 * (g & 1);
  const uint32_t sc0 = (scw >> sh) & 0xffu, sc1 = (scw >> (sh + 8)) & 0xffu;
  const uint32_t mn0 = (mnw >> sh) & 0xffu, mn1 = (mnw >> (sh + 8)) & 0xffu;
  const uint32_t a0 = sc0 >> 3, b0 = sc0 & 7u, a1 = sc1 >> 3, b1 = sc1 & 7u;
  const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
  uint32_t pal[8], pah[8], pbl[8], pbh[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t lo = lo_nib(w[k]), hi = hi_nib(w[k]);
    pal[k] = mul_bytes(lo, a0);
    pbl[k] = mul_bytes(lo, b0);
    pah[k] = mul_bytes(hi, a1);
    pbh[k] = mul_bytes(hi, b1);
  }
  uint8_t* pa = lds + kOffPa + col * kRow + 64 * g;
  uint8_t* pb = lds + kOffPb + col * kRow + 64 * g;
  st16(pa, pal[0], pal[1], pal[2], pal[3]);
  st16(pa + 16, pal[4], pal[5], pal[6], pal[7]);
  st16(pa + 32, pah[0], pah[1], pah[2], pah[3]);
  st16(pa + 48, pah[4], pah[5], pah[6], pah[7]);
  st16(pb, pbl[0], pbl[1], pbl[2], pbl[3]);
  st16(pb + 16, pbl[4], pbl[5], pbl[6], pbl[7]);
  st16(pb + 32, pbh[0], pbh[1], pbh[2], pbh[3]);
  st16(pb + 48, pbh[4], pbh[5], pbh[6], pbh[7]);
  *reinterpret_cast<uint16_t*>(lds + kOffMn + col * 8 + 2 * g) = (uint16_t)(mn0 | (mn1 << 8));
  if (g == 0) {
    reinterpret_cast<float*>(lds + kOffD)[col] = f16_to_f32(hd.x);
    reinterpret_cast<float*>(lds + kOffDm)[col] = f16_to_f32(hd.x >> 16);
  }
}

// ------------------------------------------------- staging: q6_K weight tile
// thread t: column t/4, part p4 = t%4 -> half hh = p4/2, quarters q = p4%2 (low
// nibbles of ql bytes 64hh+32q..) and q+2 (their high nibbles).  Plane A gets
// hi = v >> 7, plane B gets lo = v & 127, v = sc * (quant - 32).
__device__ __forceinline__ uint32_t q6_pack_plane(uint32_t e, uint32_t o, bool hi) {
  // e holds bytes 0 and 2 as 16-bit lanes, o holds bytes 1 and 3
  uint32_t pe, po;
  if (hi) {
    pe = __builtin_bit_cast(uint32_t, __builtin_bit_cast(i16x2, e) >> (i16x2){7, 7});
    po = __builtin_bit_cast(uint32_t, __builtin_bit_cast(i16x2, o) >> (i16x2){7, 7});
  } else {
    pe = e & 0x007f007fu;
    po = o & 0x007f007fu;
  }
  return (pe & 0x00ff00ffu) | ((po & 0x00ff00ffu) << 8);
}

__device__ __forceinline__ void stage_w_q6K(uint8_t* lds, const uint8_t* __restrict__ W,
                                            int64_t n0, int64_t N, int nb, int b) {
  const int t = threadIdx.x;
  const int col = t >> 2, p4 = t & 3, hh = p4 >> 1, q = p4 & 1;
  const int64_t n = n0 + col;
  uint32_t ql[8], qh[8];
  uint32_t scA = 0, scB = 0, dbits = 0;
  if (n < N) {
    const uint8_t* wb = W + (n * nb + b) * kQ6KBytes;
    ld_dwords_a2<8>(wb + 64 * hh + 32 * q, ql);
    ld_dwords_a2<8>(wb + 128 + 32 * hh, qh);
    scA = ld2(wb + 192 + 8 * hh + 2 * q);      // sub-blocks 8hh+2q, +1 (quarter q)
    scB = ld2(wb + 192 + 8 * hh + 2 * q + 4);  // sub-blocks 8hh+2q+4, +5 (quarter q+2)
    dbits = ld2(wb + 208);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) ql[k] = qh[k] = 0;
  }
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const int quarter = q + 2 * which;
    const uint32_t scp = which ? scB : scA;
    uint32_t hiw[8], low[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t quad = q6k_quad(ql[k], qh[k], quarter);  // 4 quants 0..63
      const int s = (int)(int8_t)((k < 4 ? scp : (scp >> 8)) & 0xffu);
      const i16x2 sv = {(short)s, (short)s};
      const i16x2 off = {32, 32};
      const i16x2 e = (__builtin_bit_cast(i16x2, quad & 0x00ff00ffu) - off) * sv;
      const i16x2 o = (__builtin_bit_cast(i16x2, (quad >> 8) & 0x00ff00ffu) - off) * sv;
      const uint32_t eu = __builtin_bit_cast(uint32_t, e), ou = __builtin_bit_cast(uint32_t, o);
      hiw[k] = q6_pack_plane(eu, ou, true);
      low[k] = q6_pack_plane(eu, ou, false);
    }
    uint8_t* pa = lds + kOffPa + col * kRow + 128 * hh + 32 * quarter;
    uint8_t* pb = lds + kOffPb + col * kRow + 128 * hh + 32 * quarter;
    st16(pa, hiw[0], hiw[1], hiw[2], hiw[3]);
    st16(pa + 16, hiw[4], hiw[5], hiw[6], hiw[7]);
    st16(pb, low[0], low[1], low[2], low[3]);
    st16(pb + 16, low[4], low[5], low[6], low[7]);
  }
  if (p4 == 0) reinterpret_cast<float*>(lds + kOffD)[col] = f16_to_f32(dbits);
}

// ------------------------------------------------- the kernel
template <int FMT>
__global__ __launch_bounds__(256, 2) void gemm_kernel(const uint8_t* __restrict__ W,
                                                      const uint8_t* __restrict__ Xq,
                                                      float* __restrict__ Y, int64_t M, int64_t N,
                                                      int nb) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int64_t n0 = (int64_t)blockIdx.x * kBN;
  const int64_t m0 = (int64_t)blockIdx.y * kBM;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int i = lane & 31, hsel = lane >> 5;
  const int arow0 = wm * 64 + i;       // LDS row of M-tile 0 (M-tile 1: +32)
  const int bcol = wn * 32 + i;        // LDS column of this lane's B fragment

  float y[2][16];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) y[mt][r] = 0.0f;

  for (int b = 0; b < nb; ++b) {
    stage_x(lds, Xq, m0, M, nb, b);
    if constexpr (FMT == 12)
      stage_w_q4K(lds, W, n0, N, nb, b);
    else
      stage_w_q6K(lds, W, n0, N, nb, b);
    __syncthreads();

    v4i af[2][8];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int kc = 0; kc < 8; ++kc)
        af[mt][kc] = *reinterpret_cast<const v4i*>(lds + kOffA + (arow0 + 32 * mt) * kRow +
                                                   32 * kc + 16 * hsel);
    v16i acc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) acc[mt] = (v16i){0};
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      const v4i bf = *reinterpret_cast<const v4i*>(lds + kOffPa + bcol * kRow + 32 * kc + 16 * hsel);
      acc[0] = mfma(af[0][kc], bf, acc[0]);
      acc[1] = mfma(af[1][kc], bf, acc[1]);
    }
    constexpr int kPlane = FMT == 12 ? 8 : 128;  // weight of plane A
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) acc[mt] = acc[mt] * kPlane;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      const v4i bf = *reinterpret_cast<const v4i*>(lds + kOffPb + bcol * kRow + 32 * kc + 16 * hsel);
      acc[0] = mfma(af[0][kc], bf, acc[0]);
      acc[1] = mfma(af[1][kc], bf, acc[1]);
    }

    const float dcol = reinterpret_cast<const float*>(lds + kOffD)[bcol];
    if constexpr (FMT == 12) {
      const float mcol = reinterpret_cast<const float*>(lds + kOffDm)[bcol];
      // B fragments of the min term: bytes t = 0..15 carry m_{t/2}; the low
      // lane half pairs them with bl, the high half with bh.
      const uint2 mv = *reinterpret_cast<const uint2*>(lds + kOffMn + bcol * 8);
      const uint32_t e0 = __builtin_amdgcn_perm(mv.x, mv.x, 0x01010000u);
      const uint32_t e1 = __builtin_amdgcn_perm(mv.x, mv.x, 0x03030202u);
      const uint32_t e2 = __builtin_amdgcn_perm(mv.y, mv.y, 0x01010000u);
      const uint32_t e3 = __builtin_amdgcn_perm(mv.y, mv.y, 0x03030202u);
      const v4i mfrag = {(int)e0, (int)e1, (int)e2, (int)e3};
      const v4i zero = {0, 0, 0, 0};
      const v4i bml = hsel == 0 ? mfrag : zero;
      const v4i bmh = hsel == 1 ? mfrag : zero;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const v4i amin = *reinterpret_cast<const v4i*>(lds + kOffBs + (arow0 + 32 * mt) * 32 +
                                                       16 * hsel);
        v16i am = mfma(amin, bmh, (v16i){0});
        am = am * 128;
        am = mfma(amin, bml, am);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 dx = *reinterpret_cast<const float4*>(
              lds + kOffDx + 4 * (wm * 64 + 32 * mt + 8 * q4 + 4 * hsel));
          const float dxs[4] = {dx.x, dx.y, dx.z, dx.w};
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int r = 4 * q4 + s;
            float tt = dcol * (float)acc[mt][r];
            tt = fmaf(-mcol, (float)am[r], tt);
            y[mt][r] = fmaf(dxs[s], tt, y[mt][r]);
          }
        }
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 dx = *reinterpret_cast<const float4*>(
              lds + kOffDx + 4 * (wm * 64 + 32 * mt + 8 * q4 + 4 * hsel));
          const float dxs[4] = {dx.x, dx.y, dx.z, dx.w};
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int r = 4 * q4 + s;
            y[mt][r] = fmaf(dxs[s], dcol * (float)acc[mt][r], y[mt][r]);
          }
        }
    }
    __syncthreads();
  }

  // 32x32 accumulator layout: lane holds column lane%32; register r holds row
  // 8*(r/4) + 4*(lane/32) + r%4.
  const int64_t col = n0 + bcol;
  if (col < N) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 64 + 32 * mt + 8 * (r >> 2) + 4 * hsel + (r & 3);
        if (row < M) Y[row * N + col] = y[mt][r];
      }
  }
}

int launch_gemm(int fmt, const uint8_t* W, const uint8_t* Xq, float* Y, int64_t M, int64_t N,
                int64_t K, hipStream_t st) {
  const int64_t nb = K / kQK;
  const int64_t gx = (N + kBN - 1) / kBN, gy = (M + kBM - 1) / kBM;
  if (nb > 0x7fffffffLL || gx > 0x7fffffffLL || gy > 65535) return -1;
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute((const void*)gemm_kernel<12>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLds) != hipSuccess)
      return -1;
    if (hipFuncSetAttribute((const void*)gemm_kernel<14>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLds) != hipSuccess)
      return -1;
    attr_set = true;
  }
  const dim3 grid((uint32_t)gx, (uint32_t)gy);
  if (fmt == 12)
    hipLaunchKernelGGL(gemm_kernel<12>, grid, dim3(256), kLds, st, W, Xq, Y, M, N, (int)nb);
  else
    hipLaunchKernelGGL(gemm_kernel<14>, grid, dim3(256), kLds, st, W, Xq, Y, M, N, (int)nb);
  return 0;
}

}  // namespace gemmq
