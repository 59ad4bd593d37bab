// skinny.hip -- q4_K packed matmul on int8 MFMA for a few activation rows
// (q6_K's counterpart is skinny_q6k.hip; the launchers here route it there)
// (batched decode and short prefills, M <= 64; the automatic path takes it for
// 3 <= M <= 16, and up to M = 64 for launches with few enough output columns).
//
// The pages' CPU kernel walks each packed weight row once per tile of 8
// activation rows (molayo article "PocketLLM: 단일 가속기에서 대규모 언어 모델
// 실행", status row "src/ -- C++ engine").  On gfx950, at these M the GEMV's dot
// products run once per activation row and turn the vector ALU into the bound,
// while the 64-row GEMM tile wastes most of its matrix work.  Here one
// v_mfma_i32_16x16x64_i8 serves 16 rows, and a wave holds one to four such row
// tiles (M <= 16, 32, 48, 64) on the same weight planes, so each weight byte is
// read and unpacked once for all the rows:
//
//  * workgroup = one 16-column tile (16 weight rows) of one matrix; its KS
//    waves split the row's super-blocks in contiguous parts (KS and the parts
//    depend on K only, so an output's summation order never depends on M);
//  * lane (n, c), n = lane % 16, c = lane / 16, holds weight column n and the
//    64-weight group c of the super-block: its 32 quant bytes qs[32c..32c+31]
//    (two 16-byte loads, no byte loaded twice in the wave) and activation row
//    n's int8 values 64c .. 64c + 63; MFMA step g takes the lane's weights
//    64c + 16g .. +15 (low nibbles of bytes 16 (g & 1) .. +15 for g < 2, high
//    nibbles for g >= 2; sub-block 2c + g / 2) against the same activations --
//    A and B in the same K order, so the instruction's own K layout does not
//    matter (one 16-byte quant load per MFMA step per lane instead, measured
//    8-12% slower: the wave's load count sets the pace);
//  * the sub-block scale is folded into the weight operand as in the prefill
//    GEMM (sc = 8a + b, two int8 planes a*q and b*q, combined as 8A + B in
//    int32), the min term sum_g m_g * bsum_g is one v_mfma_f32_16x16x16_f16
//    (integers below 2^24 throughout, so exact), and the epilogue per
//    super-block is y += d_x * (d * I_sc - dmin * I_min) in f32;
//  * each wave loads one super-block at a time straight into registers (68
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

// At most 8 waves per workgroup (measured on the Qwen3-8B layer: 16 waves, one
// workgroup per CU, left a workgroup's loads exposed; 4 waves were slower at
// M = 4..8 and 1-4% faster at M = 16..32).
constexpr int kMaxKS = 8;

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

// What one lane reads for one super-block: its weight column's bytes, and for
// each of the MT 16-row tiles, activation row 16 mt + n's bytes.
template <int MT>
struct SkRegs {
  uint4 hd;         // the column's header: d, dmin | scales
  uint4 q[2];       // quant bytes 32c .. 32c + 31 (group c)
  u32x4 xa[MT][4];  // activation values of groups 0..3, K-quarter c
  uint2 bs[MT];     // activation group sums 4c .. 4c+3
  uint32_t dx[MT];  // activation d
};

template <int MT>
__device__ __forceinline__ void sk_load(SkRegs<MT>& r, const uint8_t* wrow,
                                        const uint8_t* const (&xrow)[MT], int b, int c,
                                        const bool (&xok)[MT]) {
  const uint8_t* wb = wrow + (int64_t)b * kQ4KBytes;
  r.hd = ld16a(wb);
  r.q[0] = ld16a(wb + 16 + 32 * c);
  r.q[1] = ld16a(wb + 32 + 32 * c);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const uint8_t* xb = xrow[mt] + (int64_t)b * kQ8KBytes;
    if (xok[mt]) {
#pragma unroll
      for (int g = 0; g < 4; ++g) r.xa[mt][g] = ld16(xb + 4 + 64 * c + 16 * g);
      r.bs[mt] = ld8(xb + 260 + 8 * c);
      r.dx[mt] = ld4(xb);
    } else {  // rows past M: zero operands, nothing loaded
#pragma unroll
      for (int g = 0; g < 4; ++g) r.xa[mt][g] = u32x4{0u, 0u, 0u, 0u};
      r.bs[mt] = make_uint2(0u, 0u);
      r.dx[mt] = 0u;
    }
  }
}

// One super-block: the planes are unpacked once and serve every row tile.
template <int MT>
__device__ __forceinline__ void sk_compute(const SkRegs<MT>& r, int c, float (&y)[MT][4]) {
  const Q4KScales s = q4k_scales(r.hd.y, r.hd.z, r.hd.w);
  v4i acca[MT], accb[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acca[mt] = accb[mt] = (v4i){0, 0, 0, 0};
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    // step g, quarter c: weights 64c + 16g .. +15 = nibble half g >> 1 of quant
    // bytes 32c + 16 (g & 1) .. +15, sub-block 2c + (g >> 1)
    const int j = 2 * c + (g >> 1);
    const uint32_t sc = ((j < 4 ? s.sc_lo : s.sc_hi) >> (8 * (j & 3))) & 0x3fu;
    const uint4 qg = r.q[g & 1];
    const uint32_t shg = 4u * (uint32_t)(g >> 1);
    const uint32_t a = sc >> 3, bb = sc & 7u;
    const uint32_t w4[4] = {qg.x, qg.y, qg.z, qg.w};
    v4i pa, pb;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t nib = (w4[k] >> shg) & 0x0f0f0f0fu;
      pa[k] = (int)mul_bytes(nib, a);
      pb[k] = (int)mul_bytes(nib, bb);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const v4i xa = {(int)r.xa[mt][g].x, (int)r.xa[mt][g].y, (int)r.xa[mt][g].z,
                      (int)r.xa[mt][g].w};
      acca[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xa, pa, acca[mt], 0, 0, 0);
      accb[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xa, pb, accb[mt], 0, 0, 0);
    }
  }
  // min term: lane (n, c) carries group sums 4c..4c+3 of row n against the mins
  // of sub-blocks 2c, 2c, 2c+1, 2c+1 of column n
  const uint32_t mw = (c < 2 ? s.mn_lo : s.mn_hi) >> (16 * (c & 1));
  const _Float16 m0 = (_Float16)(float)(mw & 0xffu), m1 = (_Float16)(float)((mw >> 8) & 0xffu);
  const v4h mfrag = {m0, m0, m1, m1};
  const float dcol = f16_to_f32(r.hd.x), mcol = f16_to_f32(r.hd.x >> 16);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const uint32_t bh[2] = {i16x2_to_h2(r.bs[mt].x), i16x2_to_h2(r.bs[mt].y)};
    const v4h sfrag = __builtin_bit_cast(v4h, bh);
    const v4f am = __builtin_amdgcn_mfma_f32_16x16x16f16(sfrag, mfrag,
                                                         (v4f){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    // output register i holds row 16 mt + 4c + i; its d_x sits in lane 4c + i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float dx = __builtin_bit_cast(float, __shfl((int)r.dx[mt], 4 * c + i, 64));
      const int isc = (int)(((uint32_t)acca[mt][i] << 3) + (uint32_t)accb[mt][i]);
      float tt = dcol * (float)isc;
      tt = fmaf(-mcol, am[i], tt);
      y[mt][i] = fmaf(dx, tt, y[mt][i]);
    }
  }
}

// y = silu(g) * u in f32, the same steps as the GEMV's and the GEMM's:
// e = exp(-g), g / (1 + e) correctly rounded, times u
__device__ __forceinline__ float silu_mul_f32(float g, float u) {
  return g / (1.0f + expf(-g)) * u;
}

// SILU: the tiles cover the gate/up pair as one virtual matrix of 2N rows, row
// 2p = gate row p (gt.W[0]) and row 2p+1 = up row p (gt.W[1]); lanes n and n^1
// hold one output column's gate and up, and the even lane writes
// silu(gate) * up to column p of the single output.  MT: 16-row tiles of
// activation rows per wave (M <= 16 MT).
template <bool SILU, int MT>
__global__ __launch_bounds__(64 * kMaxKS) void skinny_q4k_kernel(const GroupTiles gt,
                                                                  const uint8_t* __restrict__ Xq,
                                                                  int M, int nb, int bpw) {
  __shared__ float red[kMaxKS][MT][4][64];
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int ks = (int)(blockDim.x >> 6);
  const int lane = lane_id(), n = lane & 15, c = lane >> 4;
  const TileMatrix tm = tile_matrix(gt, blockIdx.x);
  const int64_t N = tm.N;  // SILU: 2 x the output columns
  const int64_t col = (int64_t)tm.local * 16 + n;
  const int64_t colc = col < N ? col : N - 1;
  const uint8_t* wrow;
  if constexpr (SILU)
    wrow = ((colc & 1) ? gt.W[1] : tm.W) + (colc >> 1) * nb * kQ4KBytes;
  else
    wrow = tm.W + colc * nb * kQ4KBytes;
  bool xok[MT];
  const uint8_t* xrow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int row = 16 * mt + n;
    xok[mt] = row < M;
    xrow[mt] = Xq + (int64_t)(xok[mt] ? row : M - 1) * nb * kQ8KBytes;
  }
  const int b0 = wave * bpw, b1 = b0 + bpw < nb ? b0 + bpw : nb;

  float y[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) y[mt][i] = 0.f;
  for (int b = b0; b < b1; ++b) {
    SkRegs<MT> cur;
    sk_load<MT>(cur, wrow, xrow, b, c, xok);
    sk_compute<MT>(cur, c, y);
  }
  if (ks > 1) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][mt][i][lane] = y[mt][i];
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = red[0][mt][i][lane];
        for (int w = 1; w < ks; ++w) v += red[w][mt][i][lane];
        y[mt][i] = v;
      }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if constexpr (SILU) {
      const int64_t Nout = N >> 1, p = col >> 1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float up = __shfl_xor(y[mt][i], 1, 64);  // every lane takes part
        const int row = 16 * mt + 4 * c + i;
        if ((n & 1) == 0 && p < Nout && row < M)
          tm.Y[(int64_t)row * Nout + p] = silu_mul_f32(y[mt][i], up);
      }
    } else if (col < N) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * mt + 4 * c + i;
        if (row < M) tm.Y[(int64_t)row * N + col] = y[mt][i];
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

bool skinny_fits(int fmt, int64_t M) { return fmt == 12 && M >= 1 && M <= 64; }

template <bool SILU>
int launch_skinny_any(int fmt, const Group& g, const uint8_t* Xq, int M, int64_t K,
                      hipStream_t st) {
  if (!skinny_fits(fmt, M)) return -1;
  const int64_t nb64 = K / kQK;
  if (nb64 < 1 || nb64 > 0x7fffffffLL) return -1;
  const int nb = (int)nb64;
  GroupTiles gt;
  if (!(SILU ? make_pair_tiles(g, 16, gt) : make_tiles(g, 16, gt))) return -1;
  const uint32_t tiles = gt.start[kMaxGroup];
  if (tiles == 0) return 0;
  int ks, bpw;
  skinny_split(nb, ks, bpw);
  // 68-69 / 101-104 / 134-137 / 167-170 VGPRs for one to four row tiles, no scratch
  const dim3 grid(tiles), block(64 * ks);
  switch ((M + 15) / 16) {
    case 1: hipLaunchKernelGGL((skinny_q4k_kernel<SILU, 1>), grid, block, 0, st, gt, Xq, M, nb, bpw); break;
    case 2: hipLaunchKernelGGL((skinny_q4k_kernel<SILU, 2>), grid, block, 0, st, gt, Xq, M, nb, bpw); break;
    case 3: hipLaunchKernelGGL((skinny_q4k_kernel<SILU, 3>), grid, block, 0, st, gt, Xq, M, nb, bpw); break;
    default: hipLaunchKernelGGL((skinny_q4k_kernel<SILU, 4>), grid, block, 0, st, gt, Xq, M, nb, bpw); break;
  }
  return 0;
}

int launch_skinny(int fmt, const Group& g, const uint8_t* Xq, int M, int64_t K, hipStream_t st) {
  if (fmt == 14 || fmt == 256 + 14) return launch_skinny_q6k(fmt, g, Xq, M, K, st);
  return launch_skinny_any<false>(fmt, g, Xq, M, K, st);
}

int launch_skinny_silu(int fmt, const Group& g, const uint8_t* Xq, int M, int64_t K,
                       hipStream_t st) {
  if (fmt == 14 || fmt == 256 + 14) return launch_skinny_q6k_silu(fmt, g, Xq, M, K, st);
  if (g.count != 2 || g.N[0] != g.N[1]) return -1;
  return launch_skinny_any<true>(fmt, g, Xq, M, K, st);
}

}  // namespace gemmq
