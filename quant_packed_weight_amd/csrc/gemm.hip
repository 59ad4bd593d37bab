// gemm.hip -- step a4: the prefill packed GEMM on int8 MFMA (M >= 9).
//
// The pages' prefill GEMM walks each packed weight row once per tile of
// activation rows and applies the block scales on the way (molayo article
// "PocketLLM: 단일 가속기에서 대규모 언어 모델 실행", status row "src/ -- C++
// engine": row tile of 8 activation rows; q4_K 8-column panels).  On gfx950
// the dense contraction goes to v_mfma_i32_32x32x32_i8, and the design keeps
// the vector ALU and the memory latency off the critical path:
//
//  * The sub-block scale is folded into the weight operand.  For q4_K,
//    sc = 8a + b with a, b in 0..7, so sc*q = 8(a*q) + b*q with both products
//    in 0..105: two int8 planes whose MFMA sums, combined as 8*A + B, give
//    I_sc = sum_j sc_j * dot_j for a whole 256-weight super-block in int32.
//    For q6_K, v = sc*(q-32) in -4064..4096 splits as 128*hi + lo with
//    lo = v & 127 and hi = v >> 7 in -32..32; q5_K's v = sc*q (0..1953) splits
//    the same way; q2_K's v = sc*q (0..45) is one plane; q3_K's v = sc*q
//    (-124..128) is one plane as -v (-128..124) with d negated.
//  * The min term I_min = sum_g m_g * bsum_g (q4_K and q5_K: m_g the min of the
//    32-weight sub-block holding group g; q2_K: of the group itself) is a
//    K = 16 contraction of the activation group sums (|bsum| <= 2032) with the
//    mins (<= 63): both are exact in f16 and every partial sum is below 2^24,
//    so one v_mfma_f32_32x32x16_f16 gives it exactly, already in f32.
//  * One f32 epilogue per super-block and output:
//    y += d_x * (d * I_sc - dmin * I_min)   (q3_K, q6_K: y += d_x * d * I_sc).
//
// Kernels:
//  * q4_K: the two- and four-tile kernels in gemm_q4k.hip (launched from here).
//  * q6_K on grids of 2048 workgroups and more: the four-tile kernel in
//    gemm_q6k.hip (the same integer sums and epilogue, so the same bits).
//  * q2_K, q3_K, q5_K, q6_K (gemm_plane_kernel): a 256-thread workgroup
//    computes a 128 (M) x 64 (N) tile, each of its four waves a 64 x 32
//    sub-tile, or -- where the 128-row grid would have at most 256 workgroups,
//    one per CU -- a 64 x 64 tile of 32 x 32 wave sub-tiles, which doubles the
//    workgroups of small launches.  Per super-block the workgroup stages the
//    activation tile (int8 values, d_x, and for q2_K/q5_K the group sums) and
//    the weight tile -- unpacked once into its int8 planes (and mins) -- in
//    LDS; the global loads of super-block b+1 are issued before the MFMAs of
//    super-block b and held in registers; one 75 KB stage (56 KB for 64 rows)
//    lets two workgroups share a CU.
// In both, every output's arithmetic depends only on its own row and column,
// so any subset of rows gives identical bits.  The grid's first dimension is
// the concatenation of every grouped matrix's column tiles.
#include <atomic>

#include "device.h"
#include "gemm_common.h"
#include "launch.h"

namespace gemmq {

namespace {

using namespace gk;

constexpr int kBN = 64;  // weight rows (output columns) per workgroup

// LDS map of one stage (bytes): the weight side at fixed offsets, then the
// activation side for MT row tiles per wave (64 MT activation rows per
// workgroup).  Formats with a min term (q2_K, q5_K) also stage dmin, the weight
// mins and the activation group sums (f16 over the 16 groups of 16); the
// others leave those regions unused.
constexpr int kOffPa = 0;                    // [kBN][kRow] weight plane A (weight 128)
constexpr int kOffPb = kOffPa + kBN * kRow;  // [kBN][kRow] weight plane B
constexpr int kOffD = kOffPb + kBN * kRow;   // [kBN] f32 d
constexpr int kOffDm = kOffD + kBN * 4;      // [kBN] f32 dmin
constexpr int kOffMn = kOffDm + kBN * 4;     // [kBN][16] f16 mins (per group of 16)
constexpr int kOffX = kOffMn + kBN * 32;     // the activation side
template <int MT>
struct PlaneX {
  static constexpr int kBM = 64 * MT;                   // activation rows per workgroup
  static constexpr int kOffA = kOffX;                   // [kBM][kRow] activation int8
  static constexpr int kOffDx = kOffA + kBM * kRow;     // [kBM] f32 d_x
  static constexpr int kOffBs = kOffDx + kBM * 4;       // [kBM][16] f16 group sums
  static constexpr int kLds = kOffBs + kBM * 32;        // one stage
};
static_assert(2 * PlaneX<2>::kLds <= 160 * 1024, "two workgroups per CU");

// ------------------------------------------------- activation tile (plane kernel)
// thread t: row t/2, half t%2 of the 256 int8 values; half 0 also d_x.  With
// MIN (formats with a min term) also sums 8*half..8*half+7 (the other formats
// need none: q6_K's -32 offset and q3_K's -4 are inside the weight planes).
template <bool MIN>
struct XRegs {
  u32x4 q[8];
  uint32_t d;
  u32x4 s;  // MIN only
};

// Rows past M load a copy of row M-1: MFMA rows are independent and those
// outputs are never stored, so no branch is needed.
__device__ __forceinline__ const uint8_t* x_row(const uint8_t* __restrict__ Xq, int64_t m0,
                                                int64_t M, int nb) {
  const int64_t m = m0 + (threadIdx.x >> 1);
  return Xq + (m < M ? m : M - 1) * nb * kQ8KBytes;
}

template <bool MIN>
__device__ __forceinline__ void load_x(XRegs<MIN>& r, const uint8_t* xrow, int b) {
  const int part = threadIdx.x & 1;
  const uint8_t* xb = xrow + b * kQ8KBytes;
#pragma unroll
  for (int i = 0; i < 8; ++i) r.q[i] = ld16(xb + 4 + 128 * part + 16 * i);
  r.d = part == 0 ? ld4(xb) : 0u;
  if constexpr (MIN) r.s = ld16(xb + 260 + 16 * part);
}

template <int MT, bool MIN>
__device__ __forceinline__ void store_x(uint8_t* st, const XRegs<MIN>& r) {
  using X = PlaneX<MT>;
  const int t = threadIdx.x, row = t >> 1, part = t & 1;
  uint8_t* a = st + X::kOffA + row * kRow + 128 * part;
#pragma unroll
  for (int i = 0; i < 8; ++i) st16(a + 16 * i, r.q[i].x, r.q[i].y, r.q[i].z, r.q[i].w);
  if (part == 0) reinterpret_cast<uint32_t*>(st + X::kOffDx)[row] = r.d;
  if constexpr (MIN)
    st16(st + X::kOffBs + row * 32 + 16 * part, i16x2_to_h2(r.s.x), i16x2_to_h2(r.s.y),
         i16x2_to_h2(r.s.z), i16x2_to_h2(r.s.w));
}

// Columns past N load a copy of column N-1 (never stored).  SILU: N counts the
// interleaved gate (even) and up (odd) rows; the up matrix is Wu.
template <bool SILU, int BYTES>
__device__ __forceinline__ const uint8_t* w_row(const uint8_t* __restrict__ W,
                                                const uint8_t* __restrict__ Wu, int64_t n0,
                                                int64_t N, int nb) {
  int64_t n = n0 + (threadIdx.x >> 2);
  if constexpr (SILU) {
    if (n >= N) n = N - 2 + (n & 1);
    return ((n & 1) ? Wu : W) + (n >> 1) * nb * BYTES;
  } else {
    return W + (n < N ? n : N - 1) * nb * BYTES;
  }
}

// ------------------------------------------------- weight tiles of the plane kernel
// Per format: block bytes, int8 planes per weight, and whether a min term
// (-dmin * sum_g m_g * bsum_g) is added.
//   q6_K: v = sc*(q-32) in -4064..4096 -> plane A = v >> 7, plane B = v & 127.
//   q5_K: v = sc*q in 0..1953          -> plane A = v >> 7, plane B = v & 127.
//   q2_K: v = sc*q in 0..45            -> plane A = v.
//   q3_K: v = sc*q in -124..128        -> plane A = -v (in -128..124), d negated.
template <int FMT>
struct PlaneFmt;
template <>
struct PlaneFmt<10> {
  static constexpr int kBytes = 84, kPlanes = 1;
  static constexpr bool kMin = true;
};
template <>
struct PlaneFmt<11> {
  static constexpr int kBytes = 110, kPlanes = 1;
  static constexpr bool kMin = false;
};
template <>
struct PlaneFmt<13> {
  static constexpr int kBytes = 176, kPlanes = 2;
  static constexpr bool kMin = true;
};
template <>
struct PlaneFmt<14> {
  static constexpr int kBytes = 210, kPlanes = 2;
  static constexpr bool kMin = false;
};

// The repacked q3_K / q6_K layouts (type id + 256, repack.hip): the same
// planes from aligned loads.
template <>
struct PlaneFmt<256 + 11> : PlaneFmt<11> {};
template <>
struct PlaneFmt<256 + 14> : PlaneFmt<14> {};

// The raw bytes one thread holds for its (column, part) of a super-block.
//   q6_K: thread t: column t/4, part p4 = t%4 -> half hh = p4/2, quarters
//   q = p4%2 (low nibbles of ql bytes 64hh+32q..) and q+2 (their high nibbles).
//   q2_K, q3_K, q5_K: part c = t%4 -> weights 64c..64c+63.
template <int FMT>
struct WRegs;
template <>
struct WRegs<14> {
  uint32_t ql[8], qh[8];
  uint32_t sc, d;
};
template <>
struct WRegs<13> {
  uint32_t ql[8], qh[8];  // low nibbles of group c; all 32 high-bit bytes
  uint32_t h[4];          // d, dmin and the 12 scale bytes
};
template <>
struct WRegs<10> {
  uint32_t qs[8];  // the 32 quant bytes of half c/2
  uint32_t sc, dd;  // scale/min bytes 4c..4c+3; d and dmin
};
template <>
struct WRegs<11> {
  uint32_t qs[8], hm[8];  // low parts of half c/2; all 32 mask bytes
  uint32_t sc[3], d;      // the 12 scale bytes; d
};

// 32 bytes at a 2-byte-aligned address: the 36 bytes from p rounded down to a
// dword (so at most p + 35 is read; every caller stays inside its block),
// shifted into place.
__device__ __forceinline__ void ld32_a2(const uint8_t* p, uint32_t (&o)[8]) {
  // stepped back from p (not rebuilt from an integer): global, not flat, loads
  const uint32_t sh = (uint32_t)(reinterpret_cast<uintptr_t>(p) & 3u);
  const uint8_t* base = p - sh;
  const u32x4 x0 = ld16(base), x1 = ld16(base + 16);
  const uint32_t raw[9] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w, ld4(base + 32)};
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = __builtin_amdgcn_alignbyte(raw[i + 1], raw[i], sh);
}

__device__ __forceinline__ void load_w(WRegs<14>& r, const uint8_t* wrow, int b) {
  const int p4 = threadIdx.x & 3, hh = p4 >> 1, q = p4 & 1;
  const uint8_t* wb = wrow + b * kQ6KBytes;
  ld32_a2(wb + 64 * hh + 32 * q, r.ql);
  ld32_a2(wb + 128 + 32 * hh, r.qh);
  r.sc = (uint32_t)ld2(wb + 192 + 8 * hh + 2 * q) | ((uint32_t)ld2(wb + 196 + 8 * hh + 2 * q) << 16);
  r.d = ld2(wb + 208);
}

// v = s q + c (s = s2 / 2, c = c2 / 2) for the four bytes of q, split into
// the planes hi = v >> 7 and lo = v & 127, through the doubled product: bytes
// 0, 2 and 1, 3 of q go to 16-bit lanes, one v_pk_mad_u16 each makes
// 2v = 256 hi + 2 lo (|2v| < 2^15), whose lanes' high bytes are hi and low
// bytes 2 lo; both are gathered back in quant order.
__device__ __forceinline__ void planes_2v(uint32_t q, u16x2 s2, u16x2 c2, uint32_t& hi,
                                          uint32_t& lo) {
  const uint32_t e = __builtin_amdgcn_perm(0u, q, 0x0c020c00u);
  const uint32_t o = __builtin_amdgcn_perm(0u, q, 0x0c030c01u);
  const uint32_t we = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, e) * s2 + c2);
  const uint32_t wo = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, o) * s2 + c2);
  hi = __builtin_amdgcn_perm(wo, we, 0x07030501u);
  lo = (__builtin_amdgcn_perm(wo, we, 0x06020400u) >> 1) & 0x7f7f7f7fu;
}

__device__ __forceinline__ void store_w(uint8_t* st, const WRegs<14>& r) {
  const int t = threadIdx.x, col = t >> 2, p4 = t & 3, hh = p4 >> 1, q = p4 & 1;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const int quarter = q + 2 * which;
    const uint32_t scp = which ? (r.sc >> 16) : r.sc;
    uint32_t hiw[8], low[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t quad = q6k_quad(r.ql[k], r.qh[k], quarter);  // 4 quants 0..63
      const int s = (int)(int8_t)((k < 4 ? scp : (scp >> 8)) & 0xffu);
      // v = s (q - 32): 2v = 2s q - 64 s
      const u16x2 s2 = {(unsigned short)(2 * s), (unsigned short)(2 * s)};
      u16x2 c2 = {(unsigned short)(-64 * s), (unsigned short)(-64 * s)};
      asm volatile("" : "+v"(c2));  // keep the multiply-add (the optimizer would factor it)
      planes_2v(quad, s2, c2, hiw[k], low[k]);
    }
    uint8_t* pa = st + kOffPa + col * kRow + 128 * hh + 32 * quarter;
    uint8_t* pb = st + kOffPb + col * kRow + 128 * hh + 32 * quarter;
    st16(pa, hiw[0], hiw[1], hiw[2], hiw[3]);
    st16(pa + 16, hiw[4], hiw[5], hiw[6], hiw[7]);
    st16(pb, low[0], low[1], low[2], low[3]);
    st16(pb + 16, low[4], low[5], low[6], low[7]);
  }
  if (p4 == 0) reinterpret_cast<float*>(st + kOffD)[col] = f16_to_f32(r.d);
}

// q5_K (176-byte blocks, 16-byte aligned)
__device__ __forceinline__ void load_w(WRegs<13>& r, const uint8_t* wrow, int b) {
  const int c = threadIdx.x & 3;
  const uint8_t* wb = wrow + b * 176;
  const uint4 l0 = ld16a(wb + 48 + 32 * c), l1 = ld16a(wb + 64 + 32 * c);
  const uint4 h0 = ld16a(wb + 16), h1 = ld16a(wb + 32), hd = ld16a(wb);
  r.ql[0] = l0.x; r.ql[1] = l0.y; r.ql[2] = l0.z; r.ql[3] = l0.w;
  r.ql[4] = l1.x; r.ql[5] = l1.y; r.ql[6] = l1.z; r.ql[7] = l1.w;
  r.qh[0] = h0.x; r.qh[1] = h0.y; r.qh[2] = h0.z; r.qh[3] = h0.w;
  r.qh[4] = h1.x; r.qh[5] = h1.y; r.qh[6] = h1.z; r.qh[7] = h1.w;
  r.h[0] = hd.x; r.h[1] = hd.y; r.h[2] = hd.z; r.h[3] = hd.w;
}


__device__ __forceinline__ uint32_t h2_pair(uint32_t a, uint32_t b) {
  const h2 v = {(_Float16)(int)a, (_Float16)(int)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ void store_w(uint8_t* st, const WRegs<13>& r) {
  const int t = threadIdx.x, col = t >> 2, c = t & 3;
  const Q4KScales sm = q4k_scales(r.h[1], r.h[2], r.h[3]);
#pragma unroll
  for (int half = 0; half < 2; ++half) {  // sub-block 2c + half
    const uint32_t sc = byte_of(sm.sc_lo, sm.sc_hi, 2 * c + half);
    uint32_t hiw[8], low[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t nib = half ? hi_nib(r.ql[k]) : lo_nib(r.ql[k]);
      const uint32_t q = nib | (((r.qh[k] >> (2 * c + half)) & 0x01010101u) << 4);
      // v = sc q in 0..1953 (hi = v >> 7 <= 15)
      planes_2v(q, (u16x2){(unsigned short)(2 * sc), (unsigned short)(2 * sc)}, (u16x2){0, 0},
                hiw[k], low[k]);
    }
    uint8_t* pa = st + kOffPa + col * kRow + 64 * c + 32 * half;
    uint8_t* pb = st + kOffPb + col * kRow + 64 * c + 32 * half;
    st16(pa, hiw[0], hiw[1], hiw[2], hiw[3]);
    st16(pa + 16, hiw[4], hiw[5], hiw[6], hiw[7]);
    st16(pb, low[0], low[1], low[2], low[3]);
    st16(pb + 16, low[4], low[5], low[6], low[7]);
  }
  // the mins of sub-blocks 2c, 2c+1 cover group sums 4c..4c+3
  const uint32_t m0 = byte_of(sm.mn_lo, sm.mn_hi, 2 * c), m1 = byte_of(sm.mn_lo, sm.mn_hi, 2 * c + 1);
  const uint32_t p0 = h2_pair(m0, m0), p1 = h2_pair(m1, m1);
  *reinterpret_cast<uint2*>(st + kOffMn + col * 32 + 8 * c) = make_uint2(p0, p1);
  if (c == 0) {
    reinterpret_cast<float*>(st + kOffD)[col] = f16_to_f32(r.h[0]);
    reinterpret_cast<float*>(st + kOffDm)[col] = f16_to_f32(r.h[0] >> 16);
  }
}

// q2_K (84-byte blocks, 4-byte aligned)
__device__ __forceinline__ void load_w(WRegs<10>& r, const uint8_t* wrow, int b) {
  const int c = threadIdx.x & 3;
  const uint8_t* wb = wrow + b * 84;
  const u32x4 q0 = ld16(wb + 16 + 32 * (c >> 1)), q1 = ld16(wb + 32 + 32 * (c >> 1));
  r.qs[0] = q0.x; r.qs[1] = q0.y; r.qs[2] = q0.z; r.qs[3] = q0.w;
  r.qs[4] = q1.x; r.qs[5] = q1.y; r.qs[6] = q1.z; r.qs[7] = q1.w;
  r.sc = ld4(wb + 4 * c);
  r.dd = ld4(wb + 80);
}

__device__ __forceinline__ void store_w(uint8_t* st, const WRegs<10>& r) {
  const int t = threadIdx.x, col = t >> 2, c = t & 3;
  uint8_t* pa = st + kOffPa + col * kRow + 64 * c;
#pragma unroll
  for (int g = 0; g < 4; ++g) {  // sub-block 4c + g: quarter 2(c&1) + g/2, bytes 16(g&1)..
    const int sh = 2 * (2 * (c & 1) + (g >> 1));
    const uint32_t sc = (r.sc >> (8 * g)) & 15u;
    uint32_t v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = mul_bytes((r.qs[4 * (g & 1) + k] >> sh) & 0x03030303u, sc);
    st16(pa + 16 * g, v[0], v[1], v[2], v[3]);
  }
  const uint32_t m = (r.sc >> 4) & 0x0f0f0f0fu;  // the four mins, one per byte
  *reinterpret_cast<uint2*>(st + kOffMn + col * 32 + 8 * c) =
      make_uint2(h2_pair(m & 0xffu, (m >> 8) & 0xffu), h2_pair((m >> 16) & 0xffu, m >> 24));
  if (c == 0) {
    reinterpret_cast<float*>(st + kOffD)[col] = f16_to_f32(r.dd);
    reinterpret_cast<float*>(st + kOffDm)[col] = f16_to_f32(r.dd >> 16);
  }
}

template <>
struct WRegs<256 + 11> : WRegs<11> {};
template <>
struct WRegs<256 + 14> : WRegs<14> {};

// The repacked layouts: block bi of a matrix of NB blocks at m (16-byte aligned)
//   q6_K: ql[NB][128] | qh[NB][64] | sc[NB][16] | d[NB][2]
__device__ __forceinline__ void load_w_rp(WRegs<14>& r, const uint8_t* m, int64_t NB, int64_t bi) {
  const int p4 = threadIdx.x & 3, hh = p4 >> 1, q = p4 & 1;
  const uint8_t* lp = m + 128 * bi + 64 * hh + 32 * q;
  const uint8_t* hp = m + 128 * NB + 64 * bi + 32 * hh;
  const uint4 l0 = ld16a(lp), l1 = ld16a(lp + 16), h0 = ld16a(hp), h1 = ld16a(hp + 16);
  r.ql[0] = l0.x; r.ql[1] = l0.y; r.ql[2] = l0.z; r.ql[3] = l0.w;
  r.ql[4] = l1.x; r.ql[5] = l1.y; r.ql[6] = l1.z; r.ql[7] = l1.w;
  r.qh[0] = h0.x; r.qh[1] = h0.y; r.qh[2] = h0.z; r.qh[3] = h0.w;
  r.qh[4] = h1.x; r.qh[5] = h1.y; r.qh[6] = h1.z; r.qh[7] = h1.w;
  const uint8_t* sp = m + 192 * NB + 16 * bi + 8 * hh + 2 * q;
  r.sc = (uint32_t)ld2(sp) | ((uint32_t)ld2(sp + 4) << 16);
  r.d = ld2(m + 208 * NB + 2 * bi);
}

//   q3_K: hmask[NB][32] | qs[NB][64] | scales[NB][12] | d[NB][2]
__device__ __forceinline__ void load_w_rp(WRegs<11>& r, const uint8_t* m, int64_t NB, int64_t bi) {
  const int c = threadIdx.x & 3;
  const uint8_t* qp = m + 32 * NB + 64 * bi + 32 * (c >> 1);
  const uint4 h0 = ld16a(m + 32 * bi), h1 = ld16a(m + 32 * bi + 16);
  const uint4 q0 = ld16a(qp), q1 = ld16a(qp + 16);
  r.hm[0] = h0.x; r.hm[1] = h0.y; r.hm[2] = h0.z; r.hm[3] = h0.w;
  r.hm[4] = h1.x; r.hm[5] = h1.y; r.hm[6] = h1.z; r.hm[7] = h1.w;
  r.qs[0] = q0.x; r.qs[1] = q0.y; r.qs[2] = q0.z; r.qs[3] = q0.w;
  r.qs[4] = q1.x; r.qs[5] = q1.y; r.qs[6] = q1.z; r.qs[7] = q1.w;
  const uint8_t* sp = m + 96 * NB + 12 * bi;
  r.sc[0] = ld4(sp);
  r.sc[1] = ld4(sp + 4);
  r.sc[2] = ld4(sp + 8);
  r.d = ld2(m + 108 * NB + 2 * bi);
}

// q3_K (110-byte blocks, 2-byte aligned: every read stays inside the block)
__device__ __forceinline__ void load_w(WRegs<11>& r, const uint8_t* wrow, int b) {
  const int c = threadIdx.x & 3;
  const uint8_t* wb = wrow + b * 110;
  ld32_a2(wb, r.hm);
  ld32_a2(wb + 32 + 32 * (c >> 1), r.qs);
  ld_dwords_a2<3>(wb + 96, r.sc);
  r.d = ld2(wb + 108);
}

__device__ __forceinline__ void store_w(uint8_t* st, const WRegs<11>& r) {
  const int t = threadIdx.x, col = t >> 2, c = t & 3, h = c >> 1;
  uint8_t* pa = st + kOffPa + col * kRow + 64 * c;
  // scales 4c..4c+3: low nibbles from byte word c&1 (high nibbles when c >= 2),
  // top bits 2c..2c+1 of the bytes of word 2
  // (a select, not r.sc[c & 1]: a runtime index would put the array in scratch)
  const uint32_t lo4 = (((c & 1) ? r.sc[1] : r.sc[0]) >> (4 * (c >> 1))) & 0x0f0f0f0fu;
  const uint32_t hi2 = (r.sc[2] >> (2 * c)) & 0x03030303u;
  const uint32_t u6 = lo4 | (hi2 << 4);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int qq = 2 * (c & 1) + (g >> 1);
    const short s = (short)((int)((u6 >> (8 * g)) & 63u) - 32);
    const i16x2 s2 = {s, s}, four = {4, 4};
    uint32_t v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t low = (r.qs[4 * (g & 1) + k] >> (2 * qq)) & 0x03030303u;
      const uint32_t hb = (r.hm[4 * (g & 1) + k] >> (4 * h + qq)) & 0x01010101u;
      const uint32_t u = low | (hb << 2);  // q + 4 in 0..7
      // -sc * q = sc * (4 - (q + 4)), in -128..124
      const i16x2 e = (four - __builtin_bit_cast(i16x2, u & 0x00ff00ffu)) * s2;
      const i16x2 o = (four - __builtin_bit_cast(i16x2, (u >> 8) & 0x00ff00ffu)) * s2;
      v[k] = (__builtin_bit_cast(uint32_t, e) & 0x00ff00ffu) |
             ((__builtin_bit_cast(uint32_t, o) & 0x00ff00ffu) << 8);
    }
    st16(pa + 16 * g, v[0], v[1], v[2], v[3]);
  }
  if (c == 0) reinterpret_cast<float*>(st + kOffD)[col] = -f16_to_f32(r.d);
}

// ------------------------------------------------- one super-block from LDS
// 32x32 accumulator layout: lane holds column lane%32; register r holds row
// 8*(r/4) + 4*(lane/32) + r%4.
template <int FMT, int MT>
__device__ __forceinline__ void compute(const uint8_t* st, float (&y)[MT][16], int arow0, int bcol,
                                        int hsel) {
  using X = PlaneX<MT>;
  constexpr int PLANES = PlaneFmt<FMT>::kPlanes;
  constexpr bool MIN = PlaneFmt<FMT>::kMin;
  // acc = I_sc, exact in int32.  With two row tiles: plane A (hi) over the
  // super-block, then acc <<= 7, then plane B (lo) on top -- two independent
  // chains, one per tile.  With one: the planes go to two accumulators, one
  // activation fragment feeding both, combined as (A << 7) + B -- the same
  // integer, from two chains of eight instead of one of sixteen.
  v16i acc[MT];
  if constexpr (MT == 1 && PLANES == 2) {
    v16i accb;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      const int ko = 32 * kc + 16 * hsel;
      const v4i a = *reinterpret_cast<const v4i*>(st + X::kOffA + arow0 * kRow + ko);
      const v4i ba = *reinterpret_cast<const v4i*>(st + kOffPa + bcol * kRow + ko);
      const v4i bb = *reinterpret_cast<const v4i*>(st + kOffPb + bcol * kRow + ko);
      acc[0] = mfma_i8(a, ba, kc == 0 ? (v16i){0} : acc[0]);
      accb = mfma_i8(a, bb, kc == 0 ? (v16i){0} : accb);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[0][r] = (int)(((uint32_t)acc[0][r] << 7) + (uint32_t)accb[r]);
  } else {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = (v16i){0};
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      const int ko = 32 * kc + 16 * hsel;
      const v4i ba = *reinterpret_cast<const v4i*>(st + kOffPa + bcol * kRow + ko);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = mfma_i8(*reinterpret_cast<const v4i*>(st + X::kOffA + (arow0 + 32 * mt) * kRow + ko),
                          ba, acc[mt]);
    }
    if constexpr (PLANES == 2) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mt][r] = (int)((uint32_t)acc[mt][r] << 7);
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) {
        const int ko = 32 * kc + 16 * hsel;
        const v4i bb = *reinterpret_cast<const v4i*>(st + kOffPb + bcol * kRow + ko);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt] = mfma_i8(*reinterpret_cast<const v4i*>(st + X::kOffA + (arow0 + 32 * mt) * kRow + ko),
                            bb, acc[mt]);
      }
    }
  }
  // the min term: sum_g m_g * bsum_g over the 16 groups, exact in f32
  v16f accm[MT];
  float dmcol = 0.0f;
  if constexpr (MIN) {
    dmcol = reinterpret_cast<const float*>(st + kOffDm)[bcol];
    const v8h bm = *reinterpret_cast<const v8h*>(st + kOffMn + bcol * 32 + 16 * hsel);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      accm[mt] = mfma_f16(*reinterpret_cast<const v8h*>(st + X::kOffBs + (arow0 + 32 * mt) * 32 + 16 * hsel),
                          bm, (v16f){0.0f});
  }
  const float dcol = reinterpret_cast<const float*>(st + kOffD)[bcol];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 dx = *reinterpret_cast<const float4*>(
          st + X::kOffDx + 4 * (arow0 - (arow0 & 31) + 32 * mt + 8 * q4 + 4 * hsel));
      const float dxs[4] = {dx.x, dx.y, dx.z, dx.w};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int r = 4 * q4 + s;
        float t = dcol * (float)acc[mt][r];
        if constexpr (MIN) t = fmaf(-dmcol, accm[mt][r], t);
        y[mt][r] = fmaf(dxs[s], t, y[mt][r]);
      }
    }
}

// ------------------------------------------------- the plane kernel (q2_K, q3_K, q5_K, q6_K)
// MT row tiles per wave: 2 (128 activation rows per workgroup) or 1 (64
// rows, for launches whose 128-row grid leaves CUs idle); the tile height does
// not enter any output's arithmetic.
template <int FMT, bool SILU, int MT>
__global__ __launch_bounds__(256, 2) void gemm_plane_kernel(const GroupTiles gt,
                                                            const uint8_t* __restrict__ Xq,
                                                            int64_t M, int nb) {
  constexpr int kBM = PlaneX<MT>::kBM;
  constexpr bool MIN = PlaneFmt<FMT>::kMin;
  constexpr bool RP = FMT > 255;  // repacked layout
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const TileMatrix tm = tile_matrix(gt, blockIdx.x);
  const uint8_t* __restrict__ W = tm.W;
  float* __restrict__ Y = tm.Y;
  const int64_t N = tm.N;
  const uint32_t tile = tm.local;
  const int64_t n0 = (int64_t)tile * kBN;
  const int64_t m0 = (int64_t)blockIdx.y * kBM;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int i = lane & 31, hsel = lane >> 5;
  const int arow0 = wm * 32 * MT + i;  // LDS row of M-tile 0 (M-tile 1: +32)
  const int bcol = wn * 32 + i;   // LDS column of this lane's B fragment

  float y[MT][16];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) y[mt][r] = 0.0f;

  const uint8_t* xrow = x_row(Xq, m0, M, nb);
  const uint8_t* wrow = w_row<SILU, PlaneFmt<FMT>::kBytes>(W, gt.W[1], n0, N, nb);
  // repacked: this thread's matrix, the index of its row's first block, and
  // the blocks in that matrix
  const uint8_t* wmat = W;
  int64_t wblk = 0;
  if constexpr (RP) {
    int64_t n = n0 + (threadIdx.x >> 2);
    if constexpr (SILU) {
      if (n >= N) n = N - 2 + (n & 1);
      wmat = (n & 1) ? gt.W[1] : W;
      n >>= 1;
    } else if (n >= N) {
      n = N - 1;
    }
    wblk = n * nb;
  }
  const int64_t NB = (SILU ? N >> 1 : N) * nb;
  // D register sets of loads in flight: super-block b + D is loaded while b is
  // computed.  The 64-row form (small grids: at most two workgroups per CU,
  // often one) waits on memory latency at depth 1, and has the registers for a
  // second set.
  constexpr int D = MT == 1 ? 2 : 1;
  XRegs<MIN> xr[D];
  WRegs<FMT> wr[D];
  // the activation tile: two threads a row, so with MT = 1 waves 2 and 3 stage
  // none of it
  const bool xs = MT == 2 || threadIdx.x < 2 * kBM;
  auto load = [&](int j, int b) {
    if (xs) load_x(xr[j], xrow, b);
    if constexpr (RP)
      load_w_rp(wr[j], wmat, NB, wblk + b);
    else
      load_w(wr[j], wrow, b);
  };
#pragma unroll
  for (int j = 0; j < D; ++j)
    if (j < nb) load(j, j);
  for (int b0 = 0; b0 < nb; b0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int b = b0 + j;
      if (b < nb) {
        if (xs) store_x<MT>(lds, xr[j]);
        store_w(lds, wr[j]);
        __syncthreads();
        if (b + D < nb) load(j, b + D);  // in flight during the MFMAs below
        compute<FMT, MT>(lds, y, arow0, bcol, hsel);
        __syncthreads();
      }
    }
  }

  const int64_t col = n0 + bcol;
  if constexpr (SILU) {
    // lanes 2k / 2k+1 hold gate / up of output col / 2 for the same rows
    const int64_t n = col >> 1, Nout = N >> 1;
    const bool odd = (i & 1) != 0;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float g, u;
        silu_pair(y[mt][r], y[mt][r + 1], odd, g, u);
        const int rr = r + (odd ? 1 : 0);
        const int64_t row = m0 + wm * 32 * MT + 32 * mt + 8 * (rr >> 2) + 4 * hsel + (rr & 3);
        if (n < Nout && row < M) Y[row * Nout + n] = silu_mul_f32(g, u);
      }
  } else if (col < N) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 32 * MT + 32 * mt + 8 * (r >> 2) + 4 * hsel + (r & 3);
        if (row < M) Y[row * N + col] = y[mt][r];
      }
  }
}

}  // namespace

namespace {

// the dynamic LDS limit is a per-device attribute of each kernel
template <int FMT, bool SILU>
bool plane_lds() {
  return hipFuncSetAttribute((const void*)gemm_plane_kernel<FMT, SILU, 1>,
                             hipFuncAttributeMaxDynamicSharedMemorySize,
                             PlaneX<1>::kLds) == hipSuccess &&
         hipFuncSetAttribute((const void*)gemm_plane_kernel<FMT, SILU, 2>,
                             hipFuncAttributeMaxDynamicSharedMemorySize,
                             PlaneX<2>::kLds) == hipSuccess;
}

template <bool SILU>
bool set_lds_limits() {
  static std::atomic<int> attr_done[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  if (attr_done[dev].load(std::memory_order_acquire) == 0) {
    if (!plane_lds<14, SILU>() || !plane_lds<11, SILU>() || !plane_lds<256 + 11, SILU>() ||
        !plane_lds<256 + 14, SILU>() || !plane_lds<10, SILU>() || !plane_lds<13, SILU>() ||
        !q4k_prepare(SILU) || !q6k_prepare(SILU))
      return false;
    attr_done[dev].store(1, std::memory_order_release);
  }
  return true;
}

template <bool SILU, int MT>
int launch_plane(int fmt, const GroupTiles& gt, uint32_t gx, const uint8_t* Xq, int64_t M, int nb,
                 hipStream_t st) {
  const int64_t gy = (M + PlaneX<MT>::kBM - 1) / PlaneX<MT>::kBM;
  if (gy > 65535) return -1;
  const dim3 grid(gx, (uint32_t)gy), block(256);
  constexpr int lds = PlaneX<MT>::kLds;
  switch (fmt) {
    case 10:
      hipLaunchKernelGGL((gemm_plane_kernel<10, SILU, MT>), grid, block, lds, st, gt, Xq, M, nb);
      break;
    case 11:
      hipLaunchKernelGGL((gemm_plane_kernel<11, SILU, MT>), grid, block, lds, st, gt, Xq, M, nb);
      break;
    case 13:
      hipLaunchKernelGGL((gemm_plane_kernel<13, SILU, MT>), grid, block, lds, st, gt, Xq, M, nb);
      break;
    case 256 + 11:
      hipLaunchKernelGGL((gemm_plane_kernel<256 + 11, SILU, MT>), grid, block, lds, st, gt, Xq, M,
                         nb);
      break;
    case 256 + 14:
      hipLaunchKernelGGL((gemm_plane_kernel<256 + 14, SILU, MT>), grid, block, lds, st, gt, Xq, M,
                         nb);
      break;
    default:
      hipLaunchKernelGGL((gemm_plane_kernel<14, SILU, MT>), grid, block, lds, st, gt, Xq, M, nb);
  }
  return 0;
}

// the plane kernel's 64-row tiles up to this many 128-row workgroups
constexpr int64_t kPlaneSmallGrid = 256;

// q6_K: the four-tile kernel from this many workgroups (eight per CU; measured
// on the Qwen3-1.7B shapes: the 151936-row head at M = 512 561.7 against
// 702.8 us on the plane kernel, at M = 64 -- 1187 workgroups -- 188.6 against
// 182.6 us, down (2048 x 6144) at M = 2048 -- 256 workgroups -- 111.6 against
// 103.0 us)
constexpr int64_t kQ6FourTileWorkgroups = 2048;

template <bool SILU>
int launch_any(int fmt, const Group& grp, const uint8_t* Xq, int64_t M, int64_t K,
               hipStream_t st) {
  const int64_t nb = K / kQK;
  if (!gemm_fits(fmt, M, K)) return -1;
  if (!set_lds_limits<SILU>()) return -2;
  GroupTiles gt;
  if (fmt == 14 || fmt == 256 + 14) {
    // the four-tile q6_K kernel (128 x 128 workgroup tiles) where the launch
    // has enough of them to fill the chip; the plane kernel's 64-column tiles
    // below that.  Both give every output the same integer sum and the same
    // f32 epilogue in the same order, so the choice changes no bits.
    if (!(SILU ? make_pair_tiles(grp, 128, gt) : make_tiles(grp, 128, gt))) return -1;
    if ((int64_t)gt.start[kMaxGroup] * ((M + 127) / 128) >= kQ6FourTileWorkgroups)
      return launch_gemm_q6k(gt, fmt, SILU, Xq, M, K, st);
  }
  const int64_t bn = fmt == 12 ? 128 : kBN;
  if (!(SILU ? make_pair_tiles(grp, bn, gt) : make_tiles(grp, bn, gt))) return -1;
  if (fmt == 12) return launch_gemm_q4k(gt, SILU, Xq, M, K, st);
  const uint32_t gx = gt.start[kMaxGroup];
  if (gx == 0) return 0;
  // 64-row tiles where 128-row ones would leave CUs without a workgroup (at
  // most 256 of them; measured on q5_K and q6_K shapes of the Qwen3 layers at
  // M = 64..2048, e.g. 2048 x 6144 q6_K at M = 512 81.6 -> 65.4 us, at
  // M = 2048 -- 512 tiles of 128 rows -- 102.3 against 137.7 us)
  if ((int64_t)gx * ((M + 127) / 128) <= kPlaneSmallGrid)
    return launch_plane<SILU, 1>(fmt, gt, gx, Xq, M, (int)nb, st);
  return launch_plane<SILU, 2>(fmt, gt, gx, Xq, M, (int)nb, st);
}

}  // namespace

// One limit for every format: 65535 tiles of 64 activation rows, the grid's
// second dimension at the q4_K kernel's tile (the plane kernel's 128-row tiles
// would take twice as many).
bool gemm_fits(int fmt, int64_t M, int64_t K) {
  (void)fmt;
  return K / kQK <= 0x7fffffffLL && M <= 65535LL * 64;
}

int prepare_gemm(bool silu) {
  return (silu ? set_lds_limits<true>() : set_lds_limits<false>()) ? 0 : -2;
}

int launch_gemm(int fmt, const Group& grp, const uint8_t* Xq, int64_t M, int64_t K,
                hipStream_t st) {
  return launch_any<false>(fmt, grp, Xq, M, K, st);
}

int launch_gemm_silu(int fmt, const Group& grp, const uint8_t* Xq, int64_t M, int64_t K,
                     hipStream_t st) {
  if (grp.count != 2 || grp.N[0] != grp.N[1]) return -1;
  return launch_any<true>(fmt, grp, Xq, M, K, st);
}

}  // namespace gemmq
