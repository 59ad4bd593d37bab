// gemm_q6k.hip -- step a4 for q6_K: the prefill packed GEMM on int8 MFMA.
//
// The pages keep q6_K -- v, down and the output head of the q4_K_M mix -- on a
// path of its own (molayo article "PocketLLM: 단일 가속기에서 대규모 언어
// 모델 실행", status row "src/ -- C++ engine": q6_K and output.weight stay on
// the row path because their sums do not fit the q4_K panel kernel's int16).
// Here the q6_K GEMM takes the structure of the four-tile q4_K kernel
// (gemm_q4k.hip), with q6_K's own operand:
//
//  * A 32-wide MFMA step is two q6_K sub-blocks, and lane half h supplies the
//    16 weights of one of them (sub-block 2 kc + h of step kc), so each lane's
//    operand in a step has one scale.  The scale and the quants' offset 32 are
//    folded into the weight: v = sc * (q - 32) (q the 6-bit quant, sc signed
//    8-bit; |v| <= 4096) is made doubled in 16-bit lanes, 2v = 2 sc q - 64 sc
//    (one v_pk_mad_u16 per two weights), and since 2v = 256 hi + 2 lo with
//    hi = v >> 7 (-32..32) and lo = v & 127, one v_perm gathers the lanes'
//    high bytes as the hi plane and one more, a shift and a mask give the lo
//    plane: two int8 planes, two MFMA chains per tile, combined as
//    128 A_hi + A_lo = sum_j sc_j (dot_j - 32 bsum_j) exactly in int32.  No
//    min term is left: the epilogue per super-block and output is
//    y += d_x * (d * I).
//  * A wave takes 32 weight columns and four 32-row tiles (128 activation
//    rows), so one unpack of its columns serves four tiles; the unpack runs
//    beside the first tile's MFMAs, each later tile's MFMAs beside the
//    previous tile's epilogue.  The activation values and d_x stream through
//    two LDS stages (79 KB, two workgroups per CU) filled by direct
//    buffer->LDS loads; each lane loads its column's raw bytes straight into
//    registers one super-block ahead -- from the 210-byte blocks (2-byte
//    aligned: dword spans realigned with v_alignbyte) or from the repacked
//    layout's field arrays.
//  * No split over K, as in the plane kernel (gemm.hip): both kernels then
//    form every output with the same integer sums and the same f32 steps in
//    the same order, so the choice between them (by grid size) changes no
//    bits.
// Every output's arithmetic and summation order depend on its own row and
// column and on K, never on M: any subset of rows gives identical bits.
#include "device.h"
#include "gemm_common.h"
#include "launch.h"

namespace gemmq {

namespace {

using namespace gk;

constexpr int kT = 4;  // 32-row tiles per wave
using Map = TileStage<kT>;

constexpr int kLdsBytes = 2 * Map::kStage;  // two stages
static_assert(2 * kLdsBytes <= 160 * 1024, "two workgroups per CU");

typedef short i16x2 __attribute__((ext_vector_type(2)));

// The raw q6_K bytes lane (i, h) needs of one super-block of its weight row:
// ql bytes 64 hh + 32 q1 + 16 h .. +15 (hh, q1 in 0..1: the low nibbles give
// quarter q1 of half hh, the high nibbles quarter q1 + 2), qh bytes
// 32 hh + 16 h .. +15 (bits 2q, 2q+1 for quarter q), all 16 scales, and d.
struct Q6Raw {
  uint4 ql[2][2];
  uint4 qh[2];
  uint4 sc;
  uint32_t d;
};

// 16 bytes at a 2-byte-aligned address: five dwords from the address stepped
// back to a dword (up to p + 17 is read; every caller has that much of its
// block left), realigned.
__device__ __forceinline__ uint4 ld16_a2(const uint8_t* p) {
  const uint32_t sh = (uint32_t)(reinterpret_cast<uintptr_t>(p) & 3u);  // 0 or 2
  const uint8_t* b = p - sh;
  const u32x4 a = ld16(b);
  const uint32_t e = ld4(b + 16);
  return make_uint4(__builtin_amdgcn_alignbyte(a.y, a.x, sh), __builtin_amdgcn_alignbyte(a.z, a.y, sh),
                    __builtin_amdgcn_alignbyte(a.w, a.z, sh), __builtin_amdgcn_alignbyte(e, a.w, sh));
}

// RP: the repacked layout ql[NB][128] | qh[NB][64] | sc[NB][16] | d[NB][2]
// (every field 16-byte aligned); else 210-byte blocks.
template <bool RP>
__device__ __forceinline__ void q6_load_raw(Q6Raw& r, const uint8_t* mat, int64_t blk, int64_t NB,
                                            int h) {
  if constexpr (RP) {
    const uint8_t* lp = mat + 128 * blk + 16 * h;
    const uint8_t* hp = mat + 128 * NB + 64 * blk + 16 * h;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int q1 = 0; q1 < 2; ++q1) r.ql[hh][q1] = ld16a(lp + 64 * hh + 32 * q1);
      r.qh[hh] = ld16a(hp + 32 * hh);
    }
    r.sc = ld16a(mat + 192 * NB + 16 * blk);
    r.d = ld2(mat + 208 * NB + 2 * blk);
  } else {
    const uint8_t* wb = mat + blk * kQ6KBytes;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int q1 = 0; q1 < 2; ++q1) r.ql[hh][q1] = ld16_a2(wb + 64 * hh + 32 * q1 + 16 * h);
      r.qh[hh] = ld16_a2(wb + 128 + 32 * hh + 16 * h);
    }
    // scales (bytes 192..207) and d (208, 209): five dwords from byte 188
    // (block 4-byte aligned) or 190 (2 mod 4)
    const uint32_t sh = (uint32_t)(reinterpret_cast<uintptr_t>(wb) & 3u);
    const uint8_t* sb = wb + 188 + sh;
    const u32x4 a = ld16(sb);
    const uint32_t e = ld4(sb + 16);
    r.sc = sh ? make_uint4(__builtin_amdgcn_alignbyte(a.y, a.x, 2), __builtin_amdgcn_alignbyte(a.z, a.y, 2),
                           __builtin_amdgcn_alignbyte(a.w, a.z, 2), __builtin_amdgcn_alignbyte(e, a.w, 2))
              : make_uint4(a.y, a.z, a.w, e);
    r.d = ld2(wb + 208);
  }
}

__device__ __forceinline__ uint32_t u4(const uint4& v, int k) {
  return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}

// scale j of the column as a signed 16-bit value in both halves of a dword
__device__ __forceinline__ uint32_t sc_pair(const uint4& sc, int j) {
  const int s = __builtin_amdgcn_sbfe((int)u4(sc, j >> 2), 8 * (j & 3), 8);
  return __builtin_amdgcn_perm((uint32_t)s, (uint32_t)s, 0x05040100u);
}

// The two planes of MFMA step kc for lane half h: the 16 weights of sub-block
// 2 kc + h (quarter q = kc & 3 of half hh = kc >> 2, bytes 16 h .. 16 h + 15).
// scp: the scale in both 16-bit halves; v = sc q - 32 sc = sc (q - 32).
__device__ __forceinline__ void q6_planes(const Q6Raw& r, int kc, uint32_t scp, v4i& hi, v4i& lo) {
  const int hh = kc >> 2, q = kc & 3;
  const uint4 l = r.ql[hh][q & 1], qh = r.qh[hh];
  const u16x2 s1 = __builtin_bit_cast(u16x2, scp);
  const u16x2 s2 = s1 + s1;                  // 2 sc
  u16x2 c2 = s1 * (u16x2){0xffc0, 0xffc0};  // -64 sc (mod 2^16)
  // hidden from the optimizer, which would otherwise factor 2 sc q - 64 sc back
  // into (q - 32) 2 sc: one v_pk_mad_u16 per lane pair instead of a subtract
  // and a multiply
  asm volatile("" : "+v"(c2));
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t lw = q >= 2 ? u4(l, k) >> 4 : u4(l, k);
    const uint32_t hw = u4(qh, k);
    // bits 2q, 2q+1 of each qh byte to bits 4, 5
    const uint32_t hs = q == 0 ? hw << 4 : q == 1 ? hw << 2 : q == 2 ? hw : hw >> 2;
    const uint32_t qd = (hs & 0x30303030u) | (lw & 0x0f0f0f0fu);  // four quants, 0..63
    // bytes 0, 2 and 1, 3 into 16-bit lanes: 2v = 2 sc q - 64 sc, v = sc (q -
    // 32), |2v| <= 8192
    const uint32_t e0 = __builtin_amdgcn_perm(0u, qd, 0x0c020c00u);
    const uint32_t e1 = __builtin_amdgcn_perm(0u, qd, 0x0c030c01u);
    const u16x2 v0 = __builtin_bit_cast(u16x2, e0) * s2 + c2;
    const u16x2 v1 = __builtin_bit_cast(u16x2, e1) * s2 + c2;
    const uint32_t w0 = __builtin_bit_cast(uint32_t, v0), w1 = __builtin_bit_cast(uint32_t, v1);
    // 2v = 256 hi + 2 lo with hi = v >> 7 (arithmetic) and lo = v & 127: the
    // high byte of each 16-bit lane is hi, the low byte 2 lo; bytes gathered
    // back in quant order
    hi[k] = (int)__builtin_amdgcn_perm(w1, w0, 0x07030501u);
    lo[k] = (int)((__builtin_amdgcn_perm(w1, w0, 0x06020400u) >> 1) & 0x7f7f7f7fu);
  }
}

// One super-block for one wave from stage `st`: per tile and step one
// activation fragment feeds the hi- and the lo-plane MFMA; tile 0 builds the
// next step's planes beside its MFMAs, and each tile's epilogue follows its
// MFMAs.  dma(t, k) issues step k of tile t's share of the next stage's loads;
// next() loads the next super-block's raw weights once tile 0 has built the
// planes.
template <typename Dma, typename Next>
__device__ __forceinline__ void q6_compute(const uint8_t* st, const Q6Raw& raw, float (&y)[kT][16],
                                           int i, int h, Dma&& dma, Next&& next) {
  constexpr int kAhead = 1;  // activation fragments read this many steps ahead
  constexpr int kF = 8 * kT;
  const uint8_t* abase = st + Map::kOffQ + i * kRow + 16 * h;
  const uint8_t* dxp = st + Map::kOffDx + 16 * h;  // + 4 (32 t + 8 q4): d_x of 4 rows
  v4i af[kF];
  auto read_af = [&](int f) __attribute__((always_inline)) {
    af[f] = *reinterpret_cast<const v4i*>(abase + (32 * (f >> 3)) * kRow + 32 * (f & 7));
  };
#pragma unroll
  for (int f = 0; f < kAhead; ++f) read_af(f);

  const float dcol = f16_to_f32(raw.d);

  v4i ph[8], pl[8];
  q6_planes(raw, 0, sc_pair(raw.sc, h), ph[0], pl[0]);
  __builtin_amdgcn_sched_barrier(0);

#pragma unroll
  for (int t = 0; t < kT; ++t) {
    if (t == 0)
      __builtin_amdgcn_s_setprio(2);
    else
      __builtin_amdgcn_s_setprio(1);
    v16i aa, ab;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      dma(t, kc);
      aa = mfma_i8(af[8 * t + kc], ph[kc], kc == 0 ? (v16i){0} : aa);
      ab = mfma_i8(af[8 * t + kc], pl[kc], kc == 0 ? (v16i){0} : ab);
      if (8 * t + kc + kAhead < kF) read_af(8 * t + kc + kAhead);
      if (t == 0 && kc < 7)
        q6_planes(raw, kc + 1, sc_pair(raw.sc, 2 * (kc + 1) + h), ph[kc + 1], pl[kc + 1]);
      if (t == 0 && kc == 7) next();  // the raw bytes are dead once the planes are built
      __builtin_amdgcn_sched_barrier(0);
    }
    // I = sum_j sc_j (dot_j - 32 bsum_j) = 128 A_hi + A_lo, and the tile's
    // epilogue y += d_x * (d * I) at once (the other wave of the SIMD fills the
    // gaps: holding it into the next tile, as the q4_K kernel does, needs 32
    // registers that the q6_K raw bytes take)
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 dx = *reinterpret_cast<const float4*>(dxp + 4 * (32 * t + 8 * q4));
      const float dxs[4] = {dx.x, dx.y, dx.z, dx.w};
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int r = 4 * q4 + s4;
        const int I = (int)(((uint32_t)aa[r] << 7) + (uint32_t)ab[r]);
        y[t][r] = fmaf(dxs[s4], dcol * (float)I, y[t][r]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// FMT: 14 (q6_K) or 256 + 14 (repacked).  SILU: the tile's 128 weight rows are
// the interleaved pair rows: lane i of wave w takes gate row 16w + i/2 of the
// tile's 64 outputs for even i, the up row for odd i.
template <int FMT, bool SILU>
__global__ __launch_bounds__(256, 2) void gemm_q6k4_kernel(
    const GroupTiles gt, const uint8_t* __restrict__ Xq, int64_t M, int nb) {
  constexpr bool RP = FMT > 255;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int wave8 = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wave = wave8;
  const int lane = lane_id(), i = lane & 31, h = lane >> 5;
  // XCD-aware order (as the q4_K kernels): each XCD takes a contiguous block
  // of the (column tile, M-tile) order with the M-tiles fastest
  const uint32_t gy = gridDim.y, total = gridDim.x * gy;
  const uint32_t lin = blockIdx.x + gridDim.x * blockIdx.y;
  const uint32_t full = total & ~7u;
  const uint32_t ord = lin < full ? (lin & 7u) * (full >> 3) + (lin >> 3) : lin;
  const TileMatrix tm = tile_matrix(gt, ord / gy);
  float* __restrict__ Y = tm.Y;
  const int64_t N = tm.N;
  const uint32_t tile = tm.local;
  const int64_t n0 = (int64_t)tile * Map::kBN, m0 = (int64_t)(ord % gy) * Map::kBM;
  const uint32_t xstride = (uint32_t)nb * kQ8KBytes;
  const int64_t mrows = M - m0 < Map::kBM ? M - m0 : Map::kBM;
  const rsrc_t xr = make_rsrc(Xq + m0 * xstride, (uint32_t)(mrows * xstride));
  // this lane's weight row, clamped into the matrix (rows past N load a valid
  // row whose outputs are never stored): its matrix and first block index
  const int64_t Nout = SILU ? N >> 1 : N, o0 = SILU ? (int64_t)tile * (Map::kBN / 2) : n0;
  const uint8_t* mat;
  int64_t blk0;
  if constexpr (SILU) {
    const int64_t o = o0 + 16 * wave + (i >> 1);
    mat = (i & 1) ? gt.W[1] : tm.W;
    blk0 = (o < Nout ? o : Nout - 1) * (int64_t)nb;
  } else {
    const int64_t c = n0 + 32 * wave + i;
    mat = tm.W;
    blk0 = (c < N ? c : N - 1) * (int64_t)nb;
  }
  const int64_t NB = Nout * (int64_t)nb;  // repacked: blocks in the matrix
  const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>((lds_void_t*)lds);
  auto stage_off = [&](int slot) __attribute__((always_inline)) {
    return (uint32_t)(slot * Map::kStage);
  };

  // value rows as 16-byte loads of 64 padded 16-byte units each, offsets as
  // in the four-tile q4_K kernel: wave w issues loads j = w + 4 k; unit
  // U = 64 j + lane is unit U % 17 of row U / 17, and with U0 = 64 w + lane
  // load k is row U0 / 17 + 15 k + e, unit U0 % 17 + k - 17 e (e = 1 from
  // k = 17 - U0 % 17 on)
  constexpr int kVal = 17 * kT / 2;  // value loads per stage
  const uint32_t u0 = 64u * (uint32_t)wave + (uint32_t)lane;
  const uint32_t vx0 = (u0 / 17u) * xstride + 4u + 16u * (u0 % 17u);
  const uint32_t kwrap = 17u - u0 % 17u;
  const uint32_t vdx = (uint32_t)(64 * wave + lane) * xstride;  // waves 0, 1: d_x of 64 rows
  // the next stage's loads: value load k (k < 17 T / 8) and, from waves 0 and
  // 1, the d_x of 64 rows (k = 20)
  auto issue = [&](int b, int slot, int k) __attribute__((always_inline)) {
    const uint32_t st = lds0 + stage_off(slot);
    const uint32_t xb = (uint32_t)b * kQ8KBytes;
    if (k < (kVal + 3) / 4) {
      static_assert(Map::kOffQ == 0, "value rows at the stage base");
      const uint32_t v = (uint32_t)k < kwrap ? vx0 : vx0 + (xstride - 272u);
      const uint32_t dst = st + 1024u * (uint32_t)(wave + 4 * k);
      if (4 * k + 3 < kVal)
        dma16(xr, v, smad(15u * k, xstride, xb + 16u * k), dst);
      else
        dma16_if(wave + 4 * k < kVal, xr, v, smad(15u * k, xstride, xb + 16u * k), dst);
    } else if (k == 20) {
      dma4_if(2 * wave < kT, xr, vdx, xb, st + Map::kOffDx + 256 * wave);
    }
  };
  auto issue_all = [&](int b, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 21; ++k) issue(b, slot, k);
  };

  float y[kT][16];
#pragma unroll
  for (int t = 0; t < kT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) y[t][r] = 0.0f;

  auto blk = [&](int s) __attribute__((always_inline)) { return s < nb ? s : nb - 1; };
  Q6Raw raw, rawn;
  issue_all(blk(0), 0);
  q6_load_raw<RP>(raw, mat, blk0 + blk(0), NB, h);
  int slot = 0;
  for (int s = 0; s < nb; ++s) {
    wait_vm<0>();   // own loads of stage s and the raw weights landed
    lds_barrier();  // stage s complete everywhere; the other stage is free
    const int nxt = slot ^ 1;
    const int bn = blk(s + 1);
    q6_compute(lds + stage_off(slot), raw, y, i, h,
               [&](int t, int k) __attribute__((always_inline)) {
                 // value loads at steps 0, 2, 4 and 6 of all tiles but the
                 // last, d_x at step 5 of tile 0
                 if (t + 1 < kT && !(k & 1)) issue(bn, nxt, (k >> 1) + 4 * t);
                 if (t == 0 && k == 5) issue(bn, nxt, 20);
               },
               [&]() __attribute__((always_inline)) {
                 q6_load_raw<RP>(rawn, mat, blk0 + bn, NB, h);
               });
    raw = rawn;
    slot = nxt;
  }
  wait_vm<0>();  // no load into LDS outlives the workgroup

  if constexpr (SILU) {
    const int64_t n = o0 + 16 * wave + (i >> 1);
    const bool odd = (i & 1) != 0;
#pragma unroll
    for (int t = 0; t < kT; ++t)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float g, u;
        silu_pair(y[t][r], y[t][r + 1], odd, g, u);
        const int rr = r + (odd ? 1 : 0);
        const int64_t row = m0 + 32 * t + 8 * (rr >> 2) + 4 * h + (rr & 3);
        if (n < Nout && row < M) Y[row * Nout + n] = silu_mul_f32(g, u);
      }
  } else {
    const int64_t col = n0 + 32 * wave + i;
    if (col < N) {
      float* yp = Y + (m0 + 4 * h) * N + col;
#pragma unroll
      for (int t = 0; t < kT; ++t)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int64_t row = m0 + 32 * t + 8 * q4 + 4 * h;
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4)
            if (row + s4 < M) yp[s4 * N] = y[t][4 * q4 + s4];
          yp += 8 * N;
        }
    }
  }
}

template <int FMT, bool SILU>
bool q6_set_lds() {
  return hipFuncSetAttribute((const void*)gemm_q6k4_kernel<FMT, SILU>,
                             hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes) == hipSuccess;
}

template <int FMT, bool SILU>
void q6_launch(const GroupTiles& gt, uint32_t gx, int64_t gy, const uint8_t* Xq, int64_t M,
               int nb, hipStream_t st) {
  hipLaunchKernelGGL((gemm_q6k4_kernel<FMT, SILU>), dim3(gx, (uint32_t)gy), dim3(256), kLdsBytes,
                     st, gt, Xq, M, nb);
}

}  // namespace

bool q6k_prepare(bool silu) {
  if (silu) return q6_set_lds<14, true>() && q6_set_lds<256 + 14, true>();
  return q6_set_lds<14, false>() && q6_set_lds<256 + 14, false>();
}

int launch_gemm_q6k(const GroupTiles& gt, int fmt, bool silu, const uint8_t* Xq, int64_t M,
                    int64_t K, hipStream_t st) {
  const int nb = (int)(K / kQK);
  const uint32_t gx = gt.start[kMaxGroup];
  if (gx == 0) return 0;
  const int64_t gy = (M + Map::kBM - 1) / Map::kBM;
  if (gy > 65535) return -1;
  if (fmt == 14)
    silu ? q6_launch<14, true>(gt, gx, gy, Xq, M, nb, st)
         : q6_launch<14, false>(gt, gx, gy, Xq, M, nb, st);
  else
    silu ? q6_launch<256 + 14, true>(gt, gx, gy, Xq, M, nb, st)
         : q6_launch<256 + 14, false>(gt, gx, gy, Xq, M, nb, st);
  return 0;
}

}  // namespace gemmq
