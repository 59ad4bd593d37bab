// gemm_q4k.hip -- step a4 for q4_K: the prefill packed GEMM on int8 MFMA.
//
// The pages' prefill GEMM walks each packed weight row once per tile of
// activation rows and applies the block scales on the way (molayo article
// "PocketLLM: 단일 가속기에서 대규모 언어 모델 실행", status row "src/ -- C++
// engine": row tile of 8 activation rows; q4_K 8-column panels).  On gfx950 the
// dense contraction goes to v_mfma_i32_32x32x32_i8 (one 32-weight sub-block per
// instruction) and the kernel is organised around what the matrix core leaves
// to the vector ALU:
//
//  * The sub-block scale is folded into the weight operand: sc = 8a + b with
//    a, b in 0..7, so sc*q = 8(a*q) + b*q with both products in 0..105.  Per
//    32-row tile the a-plane and the b-plane chains over the super-block's
//    eight sub-blocks go to two int32 accumulators A and B (each activation
//    fragment feeds both), and 8 A + B = I_sc = sum_j sc_j * dot_j exactly.
//  * The min term I_min = sum_g m_g * bsum_g is one v_mfma_f32_32x32x16_f16
//    per tile (|bsum| <= 2032 and m <= 63 are exact in f16, every partial sum
//    is an integer below 2^24).
//  * One f32 epilogue per super-block and output:
//    y += d_x * (d * I_sc - dmin * I_min).
//  * What the vector ALU pays per output and super-block is the epilogue (five
//    instructions); what it pays per weight is the plane unpack.  A wave
//    therefore takes 32 weight columns and T row tiles (32 T activation rows)
//    so that one unpack of its columns serves T tiles, the epilogue of tile t
//    runs beside the matrix work of tile t+1 (the last tile's beside the next
//    super-block's first), and the unpack beside the first tile's a-plane
//    chain.
//
// Workgroup: four waves side by side on 128 weight columns, 32 T activation
// rows.  The activation values, group sums and d_x stream through two LDS
// stages filled by direct buffer->LDS loads of 1 KiB each (16 bytes a lane),
// issued a few at a time beside the matrix work; each wave loads its columns'
// raw q4_K blocks straight into registers one super-block ahead.  With T = 4 a workgroup holds 79 KB of LDS
// and two of them share a CU.  Long rows (32 super-blocks or more) split over
// two K-groups of four waves in one 512-thread workgroup; the second hands its
// partial sums to the first through LDS.  The split depends on K only and the
// row-tile count only changes which rows share a wave, so every output's
// arithmetic and summation order depend on its own row and column and on K,
// never on M or on the tile shape: any subset of rows gives identical bits.
#include "device.h"
#include "gemm_common.h"
#include "launch.h"

namespace gemmq {

namespace {

using namespace gk;

// ====================================================================
// Two row tiles per wave (64 activation rows per workgroup), for launches of
// fewer rows (use_four_tile below): the raw weight tile is staged in LDS too.
// ====================================================================
// The kernel streams both operands through a ring of LDS stages filled by
// direct buffer->LDS loads (no registers held for the prefetch, no copy loop):
//   workgroup = 4 waves, tile 64 (M) x 128 (N); wave w: all 64 rows, weight
//   columns 32w..32w+31, unpacking its own planes (shared by its two M-tiles);
//   stage = int8 values [64][272] | group sums [64][16] | d_x [64] |
//   raw q4_K blocks [128][144] (38 KB); two stages, so two workgroups share a
//   CU and one computes while the other waits;
//   the two planes go to two accumulators so every activation fragment is
//   read from LDS once, three MFMA steps ahead of its use.
// The next stage's loads are issued a sixteenth at a time, one part per
// compute chunk, so the load queue never stalls the wave for long.  They are
// issued from inline assembly: the compiler then neither sees them as LDS
// writes (it would drain every load before each LDS read) nor tracks them, and
// the kernel waits on vmcnt itself: a stage's loads are complete once fewer
// than one stage's worth of later loads is outstanding.
namespace q4s {
constexpr int kBM = 64;
constexpr int kBN = 128;
constexpr int kS = 2;                       // LDS stages
constexpr int kOffQ = 0;                    // [kBM][kRow] int8
constexpr int kOffBs = kBM * kRow;          // [kBM][16] int16 group sums
constexpr int kOffDx = kOffBs + kBM * 32;   // [kBM] f32 d_x
constexpr int kOffW = kOffDx + kBM * 4;     // [kBN][144] raw weight blocks
constexpr int kStage = kOffW + kBN * kQ4KBytes;
// SPLIT K-groups of four waves per workgroup: 1 (76 KB, two workgroups per CU)
// or 2 (152.6 KB, one workgroup of eight waves per CU, each group half of the
// super-blocks); both give two waves per SIMD when the grid fills the CUs, and
// the split keeps two per SIMD on grids of one workgroup per CU.  It is chosen
// from K alone (rows of 32 super-blocks or more), so an output's summation
// order never depends on M.
template <int SPLIT>
constexpr int lds_bytes() { return kS * SPLIT * kStage; }
// loads per stage issued by each wave: 4 value loads + 4 weight chunks (wave 0
// a fifth value load and the 64 d_x, waves 0 and 1 a fifth weight chunk and
// the group sums); waits count the smallest number, which can only wait for
// more than needed.
constexpr int kDma = 8;
constexpr int kWait = kDma * (kS - 2) < 63 ? kDma * (kS - 2) : 63;  // vmcnt field is 6 bits
}  // namespace q4s

// f32 epilogue of accumulator registers r0..r0+n-1 of one 32x32 tile:
// y += d_x * (d * I_sc - dmin * I_min), I_sc = 8 * A + B from the two plane
// accumulators; dx[r] is d_x of the register's row.
template <int n>
__device__ __forceinline__ void q4s_epilogue(const v16i& acca, const v16i& accb, const v16f& am,
                                             const float (&dx)[16], float dcol, float mcol,
                                             float (&y)[16], int r0) {
#pragma unroll
  for (int r = r0; r < r0 + n; ++r) {
    const int isc = (int)(((uint32_t)acca[r] << 3) + (uint32_t)accb[r]);
    float tt = dcol * (float)isc;
    tt = fmaf(-mcol, am[r], tt);
    y[r] = fmaf(dx[r], tt, y[r]);
  }
}

// d_x of the 16 rows a lane's accumulator registers hold in the tile whose
// first row in the stage is row0 - 4h: register r <-> row row0 + 8(r/4) + r%4.
__device__ __forceinline__ void q4s_load_dx(const uint8_t* st, int row0, float (&dx)[16]) {
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const float4 v = *reinterpret_cast<const float4*>(st + q4s::kOffDx + 4 * (row0 + 8 * q4));
    dx[4 * q4] = v.x;
    dx[4 * q4 + 1] = v.y;
    dx[4 * q4 + 2] = v.z;
    dx[4 * q4 + 3] = v.w;
  }
}

// the two weight planes of MFMA step kc from the lane's raw quant bytes
__device__ __forceinline__ void q4s_planes(const uint4 (&q)[4], const uint32_t (&aw)[2],
                                           const uint32_t (&bw)[2], int kc, v4i& pa, v4i& pb) {
  const uint4 raw = q[kc >> 1];
  const uint32_t r4[4] = {raw.x, raw.y, raw.z, raw.w};
  const uint32_t a = (aw[kc >> 2] >> (8 * (kc & 3))) & 0xffu;
  const uint32_t bb = (bw[kc >> 2] >> (8 * (kc & 3))) & 0xffu;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t nib = (kc & 1) ? hi_nib(r4[k]) : lo_nib(r4[k]);
    pa[k] = (int)mul_bytes(nib, a);
    pb[k] = (int)mul_bytes(nib, bb);
  }
}

// One super-block for one wave from stage `st`: lane (i, h) holds weight row
// i of the wave's 32 and K-half h of every 32-wide MFMA step (bytes 16h..16h+15
// of the sub-block).  The work is laid out in fenced chunks so that vector
// work sits beside independent matrix work: M-tile 0's MFMAs of step kc run
// beside the unpacking of step kc+1, M-tile 1's MFMAs beside tile 0's
// epilogue; tile 1's epilogue closes the super-block.  dma(p), p = 0..15, is
// called at the head of chunk p: it issues one part of the next stage's loads,
// so the load queue fills a little at a time instead of stalling the wave.
template <typename Dma>
__device__ __forceinline__ void q4s_compute(const uint8_t* st, int wrow, float (&y)[2][16], int i,
                                            int h, Dma&& dma) {
  using q4s::kOffBs;
  using q4s::kOffQ;
  const uint8_t* wb = st + q4s::kOffW + wrow * kQ4KBytes;
  const uint8_t* a0 = st + kOffQ + i * kRow + 16 * h;  // M-tile 0 fragments, step kc at +32 kc
  const uint8_t* a1 = a0 + 32 * kRow;                  // M-tile 1
  // activation fragments are read kAhead chunks before their MFMAs: fragment
  // f = 0..15 is M-tile f/8, step f%8
  constexpr int kAhead = 3;
  v4i af[16];
  auto read_af = [&](int f) {
    af[f] = *reinterpret_cast<const v4i*>((f < 8 ? a0 : a1) + 32 * (f & 7));
  };
  const uint4 hd = *reinterpret_cast<const uint4*>(wb);
  uint4 q[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) q[p] = *reinterpret_cast<const uint4*>(wb + 16 + 32 * p + 16 * h);
#pragma unroll
  for (int f = 0; f < kAhead; ++f) read_af(f);
  const Q4KScales s = q4k_scales(hd.y, hd.z, hd.w);
  const uint32_t aw[2] = {(s.sc_lo >> 3) & 0x07070707u, (s.sc_hi >> 3) & 0x07070707u};
  const uint32_t bw[2] = {s.sc_lo & 0x07070707u, s.sc_hi & 0x07070707u};
  v4i pa[8], pb[8];
  q4s_planes(q, aw, bw, 0, pa[0], pb[0]);
  __builtin_amdgcn_sched_barrier(0);

  // Wave priorities (s_setprio) by phase: of the two waves that share a SIMD
  // (one from each workgroup on the CU), the one whose matrix work is ahead
  // gets the issue slots first -- phase A 2, phase B 1, the epilogue-only
  // phase C 0 -- so MFMAs keep arriving while the other wave's vector work
  // fills the gaps (measured +6% at M = 512, bit-identical results).
  // phase A: M-tile 0, unpack one step ahead
  __builtin_amdgcn_s_setprio(2);
  v16i acca0 = (v16i){0}, accb0 = (v16i){0};
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) {
    dma(kc);
    acca0 = mfma_i8(af[kc], pa[kc], acca0);
    accb0 = mfma_i8(af[kc], pb[kc], accb0);
    read_af(kc + kAhead);
    if (kc < 7) q4s_planes(q, aw, bw, kc + 1, pa[kc + 1], pb[kc + 1]);
    __builtin_amdgcn_sched_barrier(0);
  }

  // min-term operands: lane half h carries group sums 8h..8h+7 against m_{(8h+t)/2}
  const uint32_t mw = h ? s.mn_hi : s.mn_lo;
  v8h mfrag;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const _Float16 m = (_Float16)(float)((mw >> (8 * k)) & 0xffu);
    mfrag[2 * k] = m;
    mfrag[2 * k + 1] = m;
  }
  v8h sfrag[2];  // group sums of row 32t+i, already f16 in the stage
#pragma unroll
  for (int t = 0; t < 2; ++t) sfrag[t] = stage_bsums(st + kOffBs, 32 * t + i, h);
  const float dcol = f16_to_f32(hd.x), mcol = f16_to_f32(hd.x >> 16);
  float dx[16];
  q4s_load_dx(st, 4 * h, dx);
  const v16f am0 = mfma_f16(sfrag[0], mfrag, (v16f){0});
  __builtin_amdgcn_sched_barrier(0);

  // phase B: M-tile 1 beside tile 0's epilogue, two registers per step
  __builtin_amdgcn_s_setprio(1);
  v16i acca1 = (v16i){0}, accb1 = (v16i){0};
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) {
    dma(8 + kc);
    acca1 = mfma_i8(af[8 + kc], pa[kc], acca1);
    accb1 = mfma_i8(af[8 + kc], pb[kc], accb1);
    if (8 + kc + kAhead < 16) read_af(8 + kc + kAhead);
    q4s_epilogue<2>(acca0, accb0, am0, dx, dcol, mcol, y[0], 2 * kc);
    __builtin_amdgcn_sched_barrier(0);
  }

  // phase C: tile 1's epilogue
  __builtin_amdgcn_s_setprio(0);
  q4s_load_dx(st, 32 + 4 * h, dx);
  const v16f am1 = mfma_f16(sfrag[1], mfrag, (v16f){0});
  q4s_epilogue<16>(acca1, accb1, am1, dx, dcol, mcol, y[1], 0);
}

// SILU: the tile's 128 weight rows are gate rows 64t..64t+63 then up rows
// 64t..64t+63 (two buffer descriptors; load groups 0..8 and 9..17 split exactly
// at row 64), and lane i of wave w unpacks gate row 16w + i/2 for even i, the up
// row for odd i, so each MFMA column pair holds (gate, up) of one output.
template <int SPLIT, bool SILU>
__global__ __launch_bounds__(256 * SPLIT, 3 - SPLIT) void gemm_q4k2_kernel(
    const GroupTiles gt, const uint8_t* __restrict__ Xq, int64_t M, int nb) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  // SPLIT groups of four waves: K-group kg takes super-blocks [kg nb0, ...);
  // in each group wave `wave` owns weight columns 32 wave .. 32 wave + 31
  const int wave8 = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int kg = SPLIT > 1 ? wave8 >> 2 : 0, wave = wave8 & 3;
  const int lane = lane_id(), i = lane & 31, h = lane >> 5;
  // XCD-aware order: workgroup L (x fastest) runs on XCD L % 8, each XCD with
  // its own L2.  Give XCD x a contiguous block of the (column tile, M-tile)
  // order with the M-tiles fastest, so the workgroups that read one weight
  // tile run together on one XCD and fetch it from HBM once.
  const uint32_t gy = gridDim.y, total = gridDim.x * gy;
  const uint32_t lin = blockIdx.x + gridDim.x * blockIdx.y;
  const uint32_t full = total & ~7u;
  const uint32_t ord = lin < full ? (lin & 7u) * (full >> 3) + (lin >> 3) : lin;
  const TileMatrix tm = tile_matrix(gt, ord / gy);
  const uint8_t* __restrict__ W = tm.W;
  float* __restrict__ Y = tm.Y;
  const int64_t N = tm.N;
  const uint32_t tile = tm.local;
  const int64_t n0 = (int64_t)tile * q4s::kBN, m0 = (int64_t)(ord % gy) * q4s::kBM;
  const uint32_t xstride = (uint32_t)nb * kQ8KBytes, wstride = (uint32_t)nb * kQ4KBytes;
  // the workgroup's activation rows and weight rows as two buffers: rows past
  // M or N read as zero (their outputs are never stored)
  const int64_t mrows = M - m0 < q4s::kBM ? M - m0 : q4s::kBM;
  const rsrc_t xr = make_rsrc(Xq + m0 * xstride, (uint32_t)(mrows * xstride));
  // SILU: outputs o0..o0+63 of Nout; wr covers the gate rows, wr2 the up rows
  const int64_t Nout = SILU ? N >> 1 : N, o0 = SILU ? (int64_t)tile * (q4s::kBN / 2) : n0;
  const int64_t orows = SILU ? (Nout - o0 < q4s::kBN / 2 ? Nout - o0 : q4s::kBN / 2)
                             : (N - n0 < q4s::kBN ? N - n0 : q4s::kBN);
  const rsrc_t wr = make_rsrc(W + o0 * wstride, (uint32_t)(orows * wstride));
  const rsrc_t wr2 = SILU ? make_rsrc(gt.W[1] + o0 * wstride, (uint32_t)(orows * wstride)) : wr;
  // this group's half of every stage
  const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>((lds_void_t*)lds) +
                        (uint32_t)kg * q4s::kStage;
  uint8_t* const ldsg = lds + kg * q4s::kStage;
  constexpr int kStride = SPLIT * q4s::kStage;  // bytes from one stage to the next

  // per-lane source offsets within one super-block column
  // value rows: the stage's 64 padded rows (17 16-byte units each) are 17
  // 16-byte loads of 64 units: unit U = 64 j + lane is unit U % 17 of row
  // U / 17 (unit 16, the padding, reads the first group sums: never used).
  // Wave w issues j = w + 4 k (k < 4) and wave 0 also j = 16.  The q8_K
  // values are only 4-byte aligned; the 16-byte loads do not need more.
  uint32_t vx[5];
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    const uint32_t U = 64u * (k < 4 ? (uint32_t)(wave + 4 * k) : 16u) + (uint32_t)lane;
    vx[k] = (U / 17u) * xstride + 4u + 16u * (U % 17u);
  }
  // group sums: 64 rows x 32 bytes, two 16-byte loads (waves 0, 1): lane l
  // takes row 32 w + l / 2, half l % 2
  const uint32_t vbs = (uint32_t)(32 * wave + (lane >> 1)) * xstride + 260 + 16 * (lane & 1);
  const uint32_t vdx = (uint32_t)lane * xstride;  // d_x of row lane
  // weight load u = wave + 4j (u < 18) covers 16-byte chunks 64u..64u+63 of
  // the 128 x 9-chunk tile, i.e. row c / 9, chunk c % 9 for c = 64u + lane
  uint32_t vw[5];
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    const uint32_t u = (uint32_t)(wave + 4 * j);
    const uint32_t c = 64u * u + (uint32_t)lane;
    const uint32_t row = c / 9u - (SILU && u >= 9u ? 64u : 0u);  // up rows from wr2's base
    vw[j] = row * wstride + 16u * (c % 9u);
  }

  // part p (0..15) of the loads of super-block b into stage `slot`: value
  // loads (0..4), the group sums (8), d_x (10), the weight chunks (11..15)
  auto issue = [&](int b, int slot, int p) {
    const uint32_t st = lds0 + (uint32_t)slot * kStride;
    const uint32_t xb = (uint32_t)b * kQ8KBytes, wb = (uint32_t)b * kQ4KBytes;
    if (p < 4) {
      dma16(xr, vx[p], xb, st + q4s::kOffQ + 1024u * (uint32_t)(wave + 4 * p));
    } else if (p == 4) {
      dma16_if(wave == 0, xr, vx[4], xb, st + q4s::kOffQ + 1024u * 16u);
    } else if (p == 8) {
      dma16_if(wave < 2, xr, vbs, xb, st + q4s::kOffBs + 1024u * (uint32_t)wave);
    } else if (p == 10) {
      dma4_if(wave == 0, xr, vdx, xb, st + q4s::kOffDx);
    } else if (p >= 11 && p < 15) {
      const int u = wave + 4 * (p - 11);
      dma16(SILU && u >= 9 ? wr2 : wr, vw[p - 11], wb, st + q4s::kOffW + 1024 * u);
    } else if (p == 15) {
      dma16_if(wave < 2, SILU ? wr2 : wr, vw[4], wb, st + q4s::kOffW + 1024 * (wave + 16));
    }  // parts 5..7 and 9 load nothing
  };
  float y[2][16];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) y[t][r] = 0.0f;
  // the LDS weight row this lane unpacks (its MFMA column)
  const int wrow_l = SILU ? ((i & 1) ? 64 : 0) + 16 * wave + (i >> 1) : 32 * wave + i;

  // Step s: group kg works on super-block b0 + s.  Every step issues one stage
  // of loads -- past the group's last block they re-read a valid block into a
  // stage nobody reads -- so the wait count is static.
  const int nb0 = SPLIT > 1 ? (nb + 1) >> 1 : nb;
  const int b0 = kg ? nb0 : 0, bend = kg ? nb : nb0;
  auto blk = [&](int s) { return b0 + s < nb ? b0 + s : nb - 1; };
#pragma unroll
  for (int s = 0; s < q4s::kS - 1; ++s)
#pragma unroll
    for (int p = 0; p < 16; ++p) issue(blk(s), s, p);
  int slot = 0;
  for (int s = 0; s < nb0; ++s) {
    wait_vm<q4s::kWait>();  // own loads of stage s landed
    if (wave < 2)  // the group sums this wave loaded, to f16
      bsums_to_f16(ldsg + slot * kStride + q4s::kOffBs + 1024 * wave, lane);
    lds_barrier();  // stage s complete everywhere; the stage of s-1 is free
    const int nxt = slot == 0 ? q4s::kS - 1 : slot - 1;
    const int bn = blk(s + q4s::kS - 1);
    if (b0 + s < bend)
      // the weight chunks (parts 11..15, the loads that go to HBM) first, so
      // their latency has the whole super-block to pass (measured: o_proj
      // 582 -> 633, down 742 -> 770 TOP/s at M = 512, cold weights)
      q4s_compute(ldsg + slot * kStride, wrow_l, y, i, h,
                  [&](int p) { issue(bn, nxt, (p + 11) & 15); });
    else  // the second group's idle last step (odd nb): only its loads
#pragma unroll
      for (int p = 0; p < 16; ++p) issue(bn, nxt, p);
    slot = slot + 1 == q4s::kS ? 0 : slot + 1;
  }
  wait_vm<0>();  // no load into LDS outlives the workgroup

  if constexpr (SPLIT > 1) {
    // the second K-group hands its partial sums to the first through LDS; the
    // first adds them (its own first) and stores
    lds_barrier();
    float* red = reinterpret_cast<float*>(lds) + wave * (32 * 64) + lane;
    if (kg == 1) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[(16 * t + r) * 64] = y[t][r];
    }
    lds_barrier();
    if (kg == 1) return;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) y[t][r] += red[(16 * t + r) * 64];
  }
  if constexpr (SILU) {
    // lanes 2k / 2k+1 hold gate / up of output o0 + 16 wave + k for the same rows
    const int64_t n = o0 + 16 * wave + (i >> 1);
    const bool odd = (i & 1) != 0;
#pragma unroll
    for (int t = 0; t < 2; ++t)
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
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + 32 * t + 8 * (r >> 2) + 4 * h + (r & 3);
          if (row < M) Y[row * N + col] = y[t][r];
        }
    }
  }
}


// ====================================================================
// Four row tiles per wave (128 activation rows per workgroup), for launches
// of 1024 activation rows and more, and of 576..1023 rows where their grid
// favours it (use_four_tile below): the raw weights go straight to registers.
// ====================================================================
template <int T, int SPLIT>
constexpr int q4_lds_bytes() {
  return 2 * SPLIT * TileStage<T>::kStage;
}
static_assert(2 * q4_lds_bytes<4, 1>() <= 160 * 1024, "two T = 4 workgroups per CU");
static_assert(q4_lds_bytes<4, 2>() <= 160 * 1024, "one split T = 4 workgroup per CU");

// The raw q4_K bytes lane (i, h) needs of one super-block of its weight row:
// the 16-byte header (d, dmin, scales) and quant bytes 16h..16h+15 of each of
// the four 32-byte groups (the K-half h of every 32-weight MFMA step).
struct Q4Raw {
  uint4 hd;
  uint4 q[4];
};

__device__ __forceinline__ void q4_load_raw(Q4Raw& r, const uint8_t* wb, int h) {
  r.hd = ld16a(wb);
#pragma unroll
  for (int p = 0; p < 4; ++p) r.q[p] = ld16a(wb + 16 + 32 * p + 16 * h);
}

// Per super-block scale words: byte j of a[j >> 2] is sc_j >> 3, of b[j >> 2]
// sc_j & 7.
struct Q4Fac {
  uint32_t a[2], b[2];
};

__device__ __forceinline__ Q4Fac q4_factors(const Q4KScales& s) {
  return Q4Fac{{(s.sc_lo >> 3) & 0x07070707u, (s.sc_hi >> 3) & 0x07070707u},
               {s.sc_lo & 0x07070707u, s.sc_hi & 0x07070707u}};
}

// byte j & 3 of w replicated into both 16-bit halves (zero high bytes)
__device__ __forceinline__ uint32_t rep_byte(uint32_t w, int j) {
  const uint32_t k = (uint32_t)(j & 3);
  return __builtin_amdgcn_perm(w, w, 0x0c000c00u | k | (k << 16));
}

// quant nibbles of MFMA step kc (sub-block kc): low nibbles of group kc/2 for
// even kc, high nibbles for odd kc
__device__ __forceinline__ v4i q4_nibs(const Q4Raw& r, int kc) {
  const uint4 raw = r.q[kc >> 1];
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  v4i n;
#pragma unroll
  for (int k = 0; k < 4; ++k) n[k] = (int)((kc & 1) ? hi_nib(w[k]) : lo_nib(w[k]));
  return n;
}

__device__ __forceinline__ v4i q4_plane(const v4i& nib, uint32_t f) {
  v4i p;
#pragma unroll
  for (int k = 0; k < 4; ++k) p[k] = (int)mul_bytes2((uint32_t)nib[k], f);
  return p;
}

// One super-block for one wave from stage `st`: lane (i, h) holds weight column
// i of the wave's 32 and K-half h of every 32-wide MFMA step.  Per tile and
// step one activation fragment feeds two independent MFMAs (the a-plane and
// the b-plane accumulator, combined as 8 A + B when the tile is done), beside
// half of the previous tile's epilogue; tile 0 builds the planes one step
// ahead instead, and the last tile's epilogue closes the super-block.  dma(t, k)
// is called at step k of tile t to issue that step's share of the next stage's
// loads; next() loads the next super-block's raw weights: with two tiles at
// the start (registers allow it), else at the start of the last tile.  Wave priorities by phase (s_setprio): the two waves that share a
// SIMD come from different workgroups and drift; the one whose matrix work is
// ahead gets the issue slots first -- tile 0 (MFMAs and unpack) 2, the other
// tiles (MFMAs and epilogues) 1, the epilogue-only close 0 -- so MFMAs keep
// arriving while the other wave's vector work fills the gaps.
template <int T, typename Dma, typename Next>
__device__ __forceinline__ void q4_compute(const uint8_t* st, const Q4Raw& raw, float (&y)[T][16],
                                           int i, int h, Dma&& dma, Next&& next) {
  using Map = TileStage<T>;
  constexpr int kAhead = 3;  // activation fragments read this many steps ahead
  constexpr int kF = 8 * T;
  const uint8_t* abase = st + Map::kOffQ + i * kRow + 16 * h;
  const uint8_t* dxp = st + Map::kOffDx + 16 * h;  // + 4 (32 t + 8 q4): d_x of 4 rows
  // fragment f: tile f / 8, step f % 8
  v4i af[kF];
  auto read_af = [&](int f) __attribute__((always_inline)) {
    af[f] = *reinterpret_cast<const v4i*>(abase + (32 * (f >> 3)) * kRow + 32 * (f & 7));
  };
#pragma unroll
  for (int f = 0; f < kAhead; ++f) read_af(f);

  const Q4KScales s = q4k_scales(raw.hd.y, raw.hd.z, raw.hd.w);
  const Q4Fac fac = q4_factors(s);
  // min-term operand: lane half h carries group sums 8h..8h+7 against
  // m_{(8h+t)/2}, i.e. the mins of sub-blocks 4h..4h+3, each twice
  const uint32_t mw = h ? s.mn_hi : s.mn_lo;
  v8h mfrag;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const _Float16 m = (_Float16)(float)((mw >> (8 * k)) & 0xffu);
    mfrag[2 * k] = m;
    mfrag[2 * k + 1] = m;
  }
  const float dcol = f16_to_f32(raw.hd.x), mcol = f16_to_f32(raw.hd.x >> 16);

  v4i pa[8], pb[8];
  {
    const v4i nib = q4_nibs(raw, 0);
    pa[0] = q4_plane(nib, rep_byte(fac.a[0], 0));
    pb[0] = q4_plane(nib, rep_byte(fac.b[0], 0));
  }
  v16i pacc;  // the previous tile's I_sc and I_min
  v16f pim;
  __builtin_amdgcn_sched_barrier(0);

#pragma unroll
  for (int t = 0; t < T; ++t) {
    if (t == 0)
      __builtin_amdgcn_s_setprio(2);
    else
      __builtin_amdgcn_s_setprio(1);
    v16i aa, ab;
    // d_x of the previous tile's rows: all four words up front where registers
    // allow (T = 2), else each two steps before its use
    float4 dxv[4];
    auto read_dx = [&](int q4) __attribute__((always_inline)) {
      dxv[q4] = *reinterpret_cast<const float4*>(dxp + 4 * (32 * (t - 1) + 8 * q4));
    };
    if (t > 0) {
#pragma unroll
      for (int q4 = 0; q4 < (T == 2 ? 4 : 1); ++q4) read_dx(q4);
    }
    v8h bsf;  // this tile's group sums, read mid-tile
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      dma(t, kc);
      if (T > 2 && t > 0 && (kc & 1) && kc < 7) read_dx((kc + 1) >> 1);
      if (kc == 4) bsf = stage_bsums(st + Map::kOffBs, 32 * t + i, h);
      aa = mfma_i8(af[8 * t + kc], pa[kc], kc == 0 ? (v16i){0} : aa);
      ab = mfma_i8(af[8 * t + kc], pb[kc], kc == 0 ? (v16i){0} : ab);
      if (8 * t + kc + kAhead < kF) read_af(8 * t + kc + kAhead);
      if (t == 0) {
        if (kc < 7) {
          const v4i nib = q4_nibs(raw, kc + 1);
          pa[kc + 1] = q4_plane(nib, rep_byte(fac.a[(kc + 1) >> 2], kc + 1));
          pb[kc + 1] = q4_plane(nib, rep_byte(fac.b[(kc + 1) >> 2], kc + 1));
        }
      } else {
        // two registers per step
        tile_epi<2>(pacc, pim, dxv[kc >> 1], dcol, mcol, y[t - 1], kc >> 1, 2 * (kc & 1));
      }
      if (t == (T > 2 ? T - 1 : 0) && kc == 0) next();
      __builtin_amdgcn_sched_barrier(0);
    }
    // I_sc = 8 A + B
#pragma unroll
    for (int r = 0; r < 16; ++r) pacc[r] = (int)(((uint32_t)aa[r] << 3) + (uint32_t)ab[r]);
    pim = mfma_f16(bsf, mfrag, (v16f){0});
    __builtin_amdgcn_sched_barrier(0);
  }
  // the last tile's epilogue
  __builtin_amdgcn_s_setprio(0);
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4)
    tile_epi<4>(pacc, pim,
              *reinterpret_cast<const float4*>(dxp + 4 * (32 * (T - 1) + 8 * q4)), dcol, mcol,
              y[T - 1], q4, 0);
}

// SILU: the tile's 128 weight rows are the interleaved pair rows 128 t ..: lane
// i of wave w takes gate row 16w + i/2 of the tile's 64 outputs for even i, the
// up row for odd i, so each MFMA column pair holds (gate, up) of one output.
template <int T, int SPLIT, bool SILU>
__global__ __launch_bounds__(256 * SPLIT, 3 - SPLIT) void gemm_q4k4_kernel(
    const GroupTiles gt, const uint8_t* __restrict__ Xq, int64_t M, int nb) {
  using Map = TileStage<T>;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  // SPLIT groups of four waves: K-group kg takes super-blocks [kg nb0, ...);
  // in each group wave `wave` owns weight columns 32 wave .. 32 wave + 31
  const int wave8 = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int kg = SPLIT > 1 ? wave8 >> 2 : 0, wave = wave8 & 3;
  const int lane = lane_id(), i = lane & 31, h = lane >> 5;
  // XCD-aware order: workgroup L (x fastest) runs on XCD L % 8, each XCD with
  // its own L2.  Give XCD x a contiguous block of the (column tile, M-tile)
  // order with the M-tiles fastest, so the workgroups that read one weight
  // tile run together on one XCD and fetch it from HBM once.
  const uint32_t gy = gridDim.y, total = gridDim.x * gy;
  const uint32_t lin = blockIdx.x + gridDim.x * blockIdx.y;
  const uint32_t full = total & ~7u;
  const uint32_t ord = lin < full ? (lin & 7u) * (full >> 3) + (lin >> 3) : lin;
  const TileMatrix tm = tile_matrix(gt, ord / gy);
  const uint8_t* __restrict__ W = tm.W;
  float* __restrict__ Y = tm.Y;
  const int64_t N = tm.N;
  const uint32_t tile = tm.local;
  const int64_t n0 = (int64_t)tile * Map::kBN, m0 = (int64_t)(ord % gy) * Map::kBM;
  const uint32_t xstride = (uint32_t)nb * kQ8KBytes;
  // the workgroup's activation rows as one buffer: rows past M read as zero
  // (their outputs are never stored)
  const int64_t mrows = M - m0 < Map::kBM ? M - m0 : Map::kBM;
  const rsrc_t xr = make_rsrc(Xq + m0 * xstride, (uint32_t)(mrows * xstride));
  // this lane's weight row (its MFMA column), clamped into the matrix: rows
  // past N load a valid row whose outputs are never stored
  const int64_t Nout = SILU ? N >> 1 : N, o0 = SILU ? (int64_t)tile * (Map::kBN / 2) : n0;
  const uint8_t* wrow;
  if constexpr (SILU) {
    const int64_t o = o0 + 16 * wave + (i >> 1);
    wrow = ((i & 1) ? gt.W[1] : W) + (o < Nout ? o : Nout - 1) * (int64_t)nb * kQ4KBytes;
  } else {
    const int64_t c = n0 + 32 * wave + i;
    wrow = W + (c < N ? c : N - 1) * (int64_t)nb * kQ4KBytes;
  }
  const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>((lds_void_t*)lds);
  auto stage_off = [&](int slot) __attribute__((always_inline)) { return (uint32_t)((slot * SPLIT + kg) * Map::kStage); };

  // per-lane source offsets within one super-block column
  // value rows: the stage's 32 T padded rows (17 16-byte units each) are
  // 17 T / 2 16-byte loads of 64 units: unit U = 64 j + lane is unit U % 17 of
  // row U / 17 (unit 16, the padding, reads the first group sums: never used).
  // Wave w issues j = w + 4 k, k = 0 .. 17 T / 8 - 1 (the last only where
  // j < 17 T / 2).  With U0 = 64 w + lane, load k takes U = U0 + 256 k, and
  // 256 = 15 * 17 + 1: row U0 / 17 + 15 k + e, unit U0 % 17 + k - 17 e, where
  // e = 1 once U0 % 17 + k reaches 17.  The lane keeps its offset for e = 0
  // and the first k with e = 1; the 15 k rows and 16 k bytes go into the
  // scalar offset.
  constexpr int kVal = 17 * T / 2;  // value loads per stage
  const uint32_t u0 = 64u * (uint32_t)wave + (uint32_t)lane;
  const uint32_t vx0 = (u0 / 17u) * xstride + 4u + 16u * (u0 % 17u);
  const uint32_t kwrap = 17u - u0 % 17u;
  // group sums: 32 T rows x 32 bytes, one 16-byte load per wave (waves < T):
  // lane l takes row 32 w + l / 2, half l % 2
  const uint32_t vbs = (uint32_t)(32 * wave + (lane >> 1)) * xstride + 260 + 16 * (lane & 1);
  const uint32_t vdx = (uint32_t)(64 * wave + lane) * xstride;  // waves < T/2: d_x of 64 rows
  // The next stage's loads: value load k (k < 17 T / 8), the group sums
  // (k = 16) and, from waves 0..T/2-1, the d_x of 64 rows (k = 20).
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
    } else if (k == 16) {
      if constexpr (T >= 4)
        dma16(xr, vbs, xb, st + Map::kOffBs + 1024u * (uint32_t)wave);
      else
        dma16_if(wave < T, xr, vbs, xb, st + Map::kOffBs + 1024u * (uint32_t)wave);
    } else if (k == 20) {
      dma4_if(2 * wave < T, xr, vdx, xb, st + Map::kOffDx + 256 * wave);
    }
  };
  auto issue_all = [&](int b, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 21; ++k) issue(b, slot, k);
  };

  float y[T][16];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) y[t][r] = 0.0f;

  // Step s: group kg works on super-block b0 + s.  Every step issues one stage
  // of loads -- past the group's last block they re-read a valid block into a
  // stage nobody reads -- and waits for all of them at the next step.
  const int nb0 = SPLIT > 1 ? (nb + 1) >> 1 : nb;
  const int b0 = kg ? nb0 : 0, bend = kg ? nb : nb0;
  auto blk = [&](int s) __attribute__((always_inline)) { return b0 + s < nb ? b0 + s : nb - 1; };
  Q4Raw raw, rawn;
  issue_all(blk(0), 0);
  q4_load_raw(raw, wrow + (int64_t)blk(0) * kQ4KBytes, h);
  int slot = 0;
  for (int s = 0; s < nb0; ++s) {
    wait_vm<0>();   // own loads of stage s and the raw weights landed
    if (wave < T)  // the group sums this wave loaded, to f16
      bsums_to_f16(lds + stage_off(slot) + Map::kOffBs + 1024 * wave, lane);
    lds_barrier();  // stage s complete everywhere; the other stage is free
    const int nxt = slot ^ 1;
    const int bn = blk(s + 1);
    const uint8_t* wnext = wrow + (int64_t)bn * kQ4KBytes;
    if (b0 + s < bend) {
      q4_compute<T>(lds + stage_off(slot), raw, y, i, h,
                    [&](int t, int k) __attribute__((always_inline)) {
                      // spread over all tiles but the last: value loads at
                      // steps 0, 2, 4 and 6, the group sums and d_x at step 7
                      if (t + 1 < T && !(k & 1)) issue(bn, nxt, (k >> 1) + 4 * t);
                      if (t == 0 && k == 7) issue(bn, nxt, 16);
                      if (t == 0 && k == 5) issue(bn, nxt, 20);
                    },
                    [&]() __attribute__((always_inline)) { q4_load_raw(rawn, wnext, h); });
    } else {  // the second group's idle last step (odd nb): only its loads
      issue_all(bn, nxt);
      q4_load_raw(rawn, wnext, h);
    }
    raw = rawn;
    slot = nxt;
  }
  wait_vm<0>();  // no load into LDS outlives the workgroup

  if constexpr (SPLIT > 1) {
    // the second K-group hands its partial sums to the first through LDS; the
    // first adds them (its own first) and stores
    lds_barrier();
    float* red = reinterpret_cast<float*>(lds) + wave * (16 * T * 64) + lane;
    if (kg == 1) {
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[(16 * t + r) * 64] = y[t][r];
    }
    lds_barrier();
    if (kg == 1) return;
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) y[t][r] += red[(16 * t + r) * 64];
  }
  if constexpr (SILU) {
    // lanes 2k / 2k+1 hold gate / up of output o0 + 16 wave + k for the same rows
    const int64_t n = o0 + 16 * wave + (i >> 1);
    const bool odd = (i & 1) != 0;
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float g, u;
        silu_pair(y[t][r], y[t][r + 1], odd, g, u);
        const int rr = r + (odd ? 1 : 0);
        const int64_t row = m0 + 32 * t + 8 * (rr >> 2) + 4 * h + (rr & 3);
        if (n < Nout && row < M) Y[row * Nout + n] = silu_mul_f32(g, u);
      }
  } else {
    // register r of tile t is row m0 + 32t + 8(r/4) + 4h + r%4: walk one
    // pointer down the rows; whole tiles inside M skip the row checks
    const int64_t col = n0 + 32 * wave + i;
    if (col < N) {
      float* yp = Y + (m0 + 4 * h) * N + col;
      if (m0 + Map::kBM <= M) {
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) yp[s4 * N] = y[t][4 * q4 + s4];
            yp += 8 * N;
          }
      } else {
#pragma unroll
        for (int t = 0; t < T; ++t)
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
}

template <int T, int SPLIT, bool SILU>
bool q4_set_lds() {
  return hipFuncSetAttribute((const void*)gemm_q4k4_kernel<T, SPLIT, SILU>,
                             hipFuncAttributeMaxDynamicSharedMemorySize,
                             q4_lds_bytes<T, SPLIT>()) == hipSuccess;
}

template <int SPLIT, bool SILU>
bool q2_set_lds() {
  return hipFuncSetAttribute((const void*)gemm_q4k2_kernel<SPLIT, SILU>,
                             hipFuncAttributeMaxDynamicSharedMemorySize,
                             q4s::lds_bytes<SPLIT>()) == hipSuccess;
}

template <int SPLIT, bool SILU>
void q4_launch4(const GroupTiles& gt, uint32_t gx, int64_t gy, const uint8_t* Xq, int64_t M,
                int nb, hipStream_t st) {
  constexpr int kLdsBytes = q4_lds_bytes<4, SPLIT>();
  hipLaunchKernelGGL((gemm_q4k4_kernel<4, SPLIT, SILU>), dim3(gx, (uint32_t)gy),
                     dim3(256 * SPLIT), kLdsBytes, st, gt, Xq, M, nb);
}

template <int SPLIT, bool SILU>
void q4_launch2(const GroupTiles& gt, uint32_t gx, int64_t gy, const uint8_t* Xq, int64_t M,
                int nb, hipStream_t st) {
  constexpr int kLdsBytes = q4s::lds_bytes<SPLIT>();
  hipLaunchKernelGGL((gemm_q4k2_kernel<SPLIT, SILU>), dim3(gx, (uint32_t)gy), dim3(256 * SPLIT),
                     kLdsBytes, st, gt, Xq, M, nb);
}

// From this many activation rows the four-tile kernel runs (measured on the
// Qwen3-8B layer: at M = 2048 it takes 866 us per pass against 977 us for the
// two-tile kernel; at M = 512 the two-tile kernel's 64-row tiles give the grid
// twice the workgroups and it takes 253 us against 307 us).  Both kernels give
// every output the same arithmetic in the same order, so the choice changes
// no bits.
// The two kernels give the same bits, so the choice between them is by time
// alone (measured per launch on the Qwen3-8B shapes, M = 512..2048, same
// process): the four-tile kernel from 1024 rows, never below 576, and in
// between when its grid, counted in rounds over the workgroups the CUs hold at
// once (two per CU, one for the split form), costs no more than the two-tile
// kernel's: rounds of 128 rows at ~1.3x the per-row rate (the split form
// ~1.2x) against rounds of 64 rows.
constexpr int64_t kQ4FourTileM = 1024;
constexpr int64_t kQ4TwoTileM = 576;
bool use_four_tile(int64_t tiles, int64_t M, bool split) {
  if (M >= kQ4FourTileM) return true;
  if (M < kQ4TwoTileM) return false;
  const int64_t slots = split ? 256 : 512;
  const int64_t r2 = (tiles * ((M + 63) / 64) + slots - 1) / slots;
  const int64_t r4 = (tiles * ((M + 127) / 128) + slots - 1) / slots;
  return r4 * 128 * 10 <= r2 * 64 * (split ? 12 : 13);
}

}  // namespace

bool q4k_prepare(bool silu) {
  if (silu)
    return q4_set_lds<4, 1, true>() && q4_set_lds<4, 2, true>() && q2_set_lds<1, true>() &&
           q2_set_lds<2, true>();
  return q4_set_lds<4, 1, false>() && q4_set_lds<4, 2, false>() && q2_set_lds<1, false>() &&
         q2_set_lds<2, false>();
}

// The tiles of `gt` (128 weight rows each) over M activation rows; the caller
// raised the LDS limits (q4k_prepare) and checked M against the grid.
int launch_gemm_q4k(const GroupTiles& gt, bool silu, const uint8_t* Xq, int64_t M, int64_t K,
                    hipStream_t st) {
  const int nb = (int)(K / kQK);
  const uint32_t gx = gt.start[kMaxGroup];
  if (gx == 0) return 0;
  // long rows run split over K (the choice depends on K only)
  const bool split = nb >= 32;
  if (use_four_tile(gx, M, split)) {
    const int64_t gy = (M + 127) / 128;
    if (gy > 65535) return -1;
    if (split)
      silu ? q4_launch4<2, true>(gt, gx, gy, Xq, M, nb, st)
           : q4_launch4<2, false>(gt, gx, gy, Xq, M, nb, st);
    else
      silu ? q4_launch4<1, true>(gt, gx, gy, Xq, M, nb, st)
           : q4_launch4<1, false>(gt, gx, gy, Xq, M, nb, st);
  } else {
    const int64_t gy = (M + q4s::kBM - 1) / q4s::kBM;
    if (split)
      silu ? q4_launch2<2, true>(gt, gx, gy, Xq, M, nb, st)
           : q4_launch2<2, false>(gt, gx, gy, Xq, M, nb, st);
    else
      silu ? q4_launch2<1, true>(gt, gx, gy, Xq, M, nb, st)
           : q4_launch2<1, false>(gt, gx, gy, Xq, M, nb, st);
  }
  return 0;
}

}  // namespace gemmq
