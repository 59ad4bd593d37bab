// skinny.hip -- q4_K packed matmul on int8 MFMA for a few activation rows
// (batched decode, M <= 16; the automatic path takes it for 4 <= M <= 16).
//
// At these M the GEMV's dot products run once per activation row and turn the
// vector ALU into the bound, while the 64-row GEMM tile wastes most of its
// matrix work.  Here one v_mfma_i32_16x16x64_i8 serves all (up to 16) rows:
//
//  * workgroup = one 16-column tile (16 weight rows) of one matrix; its KS
//    waves split the row's super-blocks in contiguous parts (KS and the parts
//    depend on K only, so an output's summation order never depends on M);
//  * lane (n, c), n = lane % 16, c = lane / 16, holds weight column n and
//    K-quarter c of every 64-wide MFMA step: for the 64-weight group g of a
//    super-block that is 16 quant bytes at qs[32g + 16 (c & 1)], low nibbles
//    for c < 2, high nibbles for c >= 2 (sub-block 2g + c / 2), and activation
//    row n's int8 values 64g + 16c .. 64g + 16c + 15;
//  * the sub-block scale is folded into the weight operand as in the prefill
//    GEMM (sc = 8a + b, two int8 planes a*q and b*q, combined as 8A + B in
//    int32), the min term sum_g m_g * bsum_g is one v_mfma_f32_16x16x16_f16
//    (integers below 2^24 throughout, so exact), and the epilogue per
//    super-block is y += d_x * (d * I_sc - dmin * I_min) in f32;
//  * each wave loads one super-block at a time straight into registers (70
//    VGPRs, seven waves per SIMD: more waves in flight measured faster than
//    holding the next super-block's loads during the arithmetic);
//  * the waves' partial sums are added in LDS in wave order;
//  * SILU: gate and up rows interleaved in one tile, the product
//    silu(gate) * up written in place of the two outputs.
// Rows past M read as zero and columns past N re-read the last row; neither is
// stored.
#include "device.h"
#include "launch.h"

namespace gemmq {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// At most 8 waves per workgroup (measured on the Qwen3-8B layer at M = 4..16:
// 16 waves, one workgroup per CU, left the loads of one workgroup exposed; 4
// waves made the 48-super-block rows too long per wave).
constexpr int kMaxKS = 8;
// 16-column tiles per wave (two, sharing the activation loads, measured slower:
// 165 VGPRs, three waves per SIMD)
constexpr int kCT = 1;

// bytes of w (each <= 15) times a (<= 7), byte by byte (no carries)
__device__ __forceinline__ uint32_t mul_bytes(uint32_t w, uint32_t a) {
  const u16x2 v = __builtin_bit_cast(u16x2, w);
  const u16x2 s = {(unsigned short)a, (unsigned short)a};
  return __builtin_bit_cast(uint32_t, v * s);
}

// two int16 (packed in a dword) -> two f16 (exact: |value| <= 2032)
__device__ __forceinline__ uint32_t i16x2_to_h2(uint32_t w) {
  const h2 v = {(_Float16)(short)(w & 0xffffu), (_Float16)(short)(w >> 16)};
  return __builtin_bit_cast(uint32_t, v);
}

// What one lane reads for one super-block.
struct SkRegs {
  uint4 hd[kCT];    // its column's header: d, dmin | scales
  uint4 q[kCT][4];  // quant bytes of groups 0..3
  u32x4 xa[4];  // activation row n's values of groups 0..3, K-quarter c
  uint2 bs;     // activation row n's group sums 4c .. 4c+3
  uint32_t dx;  // activation row n's d
};

__device__ __forceinline__ void sk_load(SkRegs& r, const uint8_t* const (&wrow)[kCT],
                                        const uint8_t* xrow, int b, int c, bool xok) {
#pragma unroll
  for (int t = 0; t < kCT; ++t) {
    const uint8_t* wb = wrow[t] + (int64_t)b * kQ4KBytes;
    r.hd[t] = ld16a(wb);
#pragma unroll
    for (int g = 0; g < 4; ++g) r.q[t][g] = ld16a(wb + 16 + 32 * g + 16 * (c & 1));
  }
  const uint8_t* xb = xrow + (int64_t)b * kQ8KBytes;
  if (xok) {
#pragma unroll
    for (int g = 0; g < 4; ++g) r.xa[g] = ld16(xb + 4 + 64 * g + 16 * c);
    r.bs = ld8(xb + 260 + 8 * c);
    r.dx = ld4(xb);
  } else {  // rows past M: zero operands, nothing loaded
#pragma unroll
    for (int g = 0; g < 4; ++g) r.xa[g] = u32x4{0u, 0u, 0u, 0u};
    r.bs = make_uint2(0u, 0u);
    r.dx = 0u;
  }
}

__device__ __forceinline__ void sk_compute(const SkRegs& r, int lane, int c,
                                           float (&y)[kCT][4]) {
  const int hb = c >> 1;              // high nibbles (second sub-block of each group)
  const uint32_t sh = 4u * (uint32_t)hb;
  float dxs[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)  // output register i holds row 4c + i; its d_x sits in lane 4c + i
    dxs[i] = __builtin_bit_cast(float, __shfl((int)r.dx, 4 * c + i, 64));
  const uint32_t bh[2] = {i16x2_to_h2(r.bs.x), i16x2_to_h2(r.bs.y)};
  const v4h sfrag = __builtin_bit_cast(v4h, bh);
#pragma unroll
  for (int t = 0; t < kCT; ++t) {
    const Q4KScales s = q4k_scales(r.hd[t].y, r.hd[t].z, r.hd[t].w);
    v4i acca = (v4i){0, 0, 0, 0}, accb = (v4i){0, 0, 0, 0};
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      // scale of sub-block 2g + hb: byte 2(g & 1) + hb of sc_lo (g < 2) or sc_hi
      const uint32_t sc = ((g < 2 ? s.sc_lo : s.sc_hi) >> (8 * (2 * (g & 1) + hb))) & 0x3fu;
      const uint32_t a = sc >> 3, bb = sc & 7u;
      const uint32_t w4[4] = {r.q[t][g].x, r.q[t][g].y, r.q[t][g].z, r.q[t][g].w};
      v4i pa, pb;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t nib = (w4[k] >> sh) & 0x0f0f0f0fu;
        pa[k] = (int)mul_bytes(nib, a);
        pb[k] = (int)mul_bytes(nib, bb);
      }
      const v4i xa = {(int)r.xa[g].x, (int)r.xa[g].y, (int)r.xa[g].z, (int)r.xa[g].w};
      acca = __builtin_amdgcn_mfma_i32_16x16x64_i8(xa, pa, acca, 0, 0, 0);
      accb = __builtin_amdgcn_mfma_i32_16x16x64_i8(xa, pb, accb, 0, 0, 0);
    }
    // min term: lane (n, c) carries group sums 4c..4c+3 of row n against the mins
    // of sub-blocks 2c, 2c, 2c+1, 2c+1 of column n
    const uint32_t mw = (c < 2 ? s.mn_lo : s.mn_hi) >> (16 * (c & 1));
    const _Float16 m0 = (_Float16)(float)(mw & 0xffu), m1 = (_Float16)(float)((mw >> 8) & 0xffu);
    const v4h mfrag = {m0, m0, m1, m1};
    const v4f am = __builtin_amdgcn_mfma_f32_16x16x16f16(sfrag, mfrag,
                                                         (v4f){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    const float dcol = f16_to_f32(r.hd[t].x), mcol = f16_to_f32(r.hd[t].x >> 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int isc = (int)(((uint32_t)acca[i] << 3) + (uint32_t)accb[i]);
      float tt = dcol * (float)isc;
      tt = fmaf(-mcol, am[i], tt);
      y[t][i] = fmaf(dxs[i], tt, y[t][i]);
    }
  }
  (void)lane;
}

// y = silu(g) * u in f32, the same steps as the GEMV's and the GEMM's:
// e = exp(-g), g / (1 + e) correctly rounded, times u
__device__ __forceinline__ float silu_mul_f32(float g, float u) {
  return g / (1.0f + expf(-g)) * u;
}

// SILU: the tiles cover the gate/up pair as one virtual matrix of 2N rows, row
// 2p = gate row p (gt.W[0]) and row 2p+1 = up row p (gt.W[1]); lanes n and n^1
// hold one output column's gate and up, and the even lane writes
// silu(gate) * up to column p of the single output.
template <bool SILU>
__global__ __launch_bounds__(64 * kMaxKS) void skinny_q4k_kernel(const GroupTiles gt,
                                                                  const uint8_t* __restrict__ Xq,
                                                                  int M, int nb, int bpw) {
  __shared__ float red[kMaxKS][kCT][4][64];
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int ks = (int)(blockDim.x >> 6);
  const int lane = lane_id(), n = lane & 15, c = lane >> 4;
  const TileMatrix tm = tile_matrix(gt, blockIdx.x);
  const int64_t N = tm.N;  // SILU: 2 x the output columns
  int64_t col[kCT];
  const uint8_t* wrow[kCT];
#pragma unroll
  for (int t = 0; t < kCT; ++t) {
    col[t] = (int64_t)tm.local * (16 * kCT) + 16 * t + n;
    const int64_t colc = col[t] < N ? col[t] : N - 1;
    if constexpr (SILU)
      wrow[t] = ((colc & 1) ? gt.W[1] : tm.W) + (colc >> 1) * nb * kQ4KBytes;
    else
      wrow[t] = tm.W + colc * nb * kQ4KBytes;
  }
  const bool xok = n < M;
  const uint8_t* xrow = Xq + (int64_t)(xok ? n : M - 1) * nb * kQ8KBytes;
  const int b0 = wave * bpw, b1 = b0 + bpw < nb ? b0 + bpw : nb;

  float y[kCT][4];
#pragma unroll
  for (int t = 0; t < kCT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) y[t][i] = 0.f;
  for (int b = b0; b < b1; ++b) {
    SkRegs cur;
    sk_load(cur, wrow, xrow, b, c, xok);
    sk_compute(cur, lane, c, y);
  }
  if (ks > 1) {
#pragma unroll
    for (int t = 0; t < kCT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][t][i][lane] = y[t][i];
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int t = 0; t < kCT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = red[0][t][i][lane];
        for (int w = 1; w < ks; ++w) v += red[w][t][i][lane];
        y[t][i] = v;
      }
  }
#pragma unroll
  for (int t = 0; t < kCT; ++t) {
    if constexpr (SILU) {
      const int64_t Nout = N >> 1, p = col[t] >> 1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float up = __shfl_xor(y[t][i], 1, 64);  // every lane takes part
        const int row = 4 * c + i;
        if ((n & 1) == 0 && p < Nout && row < M)
          tm.Y[(int64_t)row * Nout + p] = silu_mul_f32(y[t][i], up);
      }
    } else if (col[t] < N) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * c + i;
        if (row < M) tm.Y[(int64_t)row * N + col[t]] = y[t][i];
      }
    }
  }
}

}  // namespace

// Waves per workgroup and super-blocks per wave for rows of nb super-blocks:
// at most 8 waves, each a contiguous part of ceil(nb / 8) super-blocks.
void skinny_split(int nb, int& ks, int& bpw) {
  bpw = (nb + kMaxKS - 1) / kMaxKS;
  ks = (nb + bpw - 1) / bpw;
}

bool skinny_fits(int fmt, int64_t M) { return fmt == 12 && M >= 1 && M <= 16; }

template <bool SILU>
int launch_skinny_any(int fmt, const Group& g, const uint8_t* Xq, int M, int64_t K,
                      hipStream_t st) {
  if (!skinny_fits(fmt, M)) return -1;
  const int64_t nb64 = K / kQK;
  if (nb64 < 1 || nb64 > 0x7fffffffLL) return -1;
  const int nb = (int)nb64;
  GroupTiles gt;
  if (!(SILU ? make_pair_tiles(g, 16 * kCT, gt) : make_tiles(g, 16 * kCT, gt))) return -1;
  const uint32_t tiles = gt.start[kMaxGroup];
  if (tiles == 0) return 0;
  int ks, bpw;
  skinny_split(nb, ks, bpw);
  hipLaunchKernelGGL(skinny_q4k_kernel<SILU>, dim3(tiles), dim3(64 * ks), 0, st, gt, Xq, M, nb,
                     bpw);
  return 0;
}

int launch_skinny(int fmt, const Group& g, const uint8_t* Xq, int M, int64_t K, hipStream_t st) {
  return launch_skinny_any<false>(fmt, g, Xq, M, K, st);
}

int launch_skinny_silu(int fmt, const Group& g, const uint8_t* Xq, int M, int64_t K,
                       hipStream_t st) {
  if (g.count != 2 || g.N[0] != g.N[1]) return -1;
  return launch_skinny_any<true>(fmt, g, Xq, M, K, st);
}

}  // namespace gemmq
