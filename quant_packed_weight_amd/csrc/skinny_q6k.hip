// skinny_q6k.hip -- q6_K packed matmul on int8 MFMA for a few activation rows
// (batched decode, M <= 16), the q6_K counterpart of skinny.hip.
//
// The pages keep q6_K -- the format of v, down and the output head in the
// q4_K_M mix -- on a row path of its own (molayo article "PocketLLM: 단일
// 가속기에서 대규모 언어 모델 실행", status row "src/ -- C++ engine": q6_K and
// output.weight stay on their own path because its sums overflow int16).  On
// gfx950 the decode GEMV's v_dot4 products run once per activation row, so at
// M = 8 the vector ALU and the per-row activation reads bound it (the LM head
// took 4-5x its M = 1 time).  Here a q6_K sub-block -- 16 weights sharing one
// int8 scale -- is exactly the K depth of one v_mfma_i32_32x32x16_i8, so the
// 6-bit quants enter the matrix core as they are (0..63 fits int8), each
// sub-block's product comes out whole and is scaled on its own:
//
//  * workgroup = one 32-column tile (32 weight rows) of one matrix; its KS
//    waves split the row's super-blocks in contiguous parts (KS and the parts
//    depend on K only, so an output's summation order never depends on M);
//  * lane (n, h), n = lane % 32, h = lane / 32, holds weight column n and, of
//    every sub-block j, the 8 weights 16 j + 8 h .. +7 (and activation row n's
//    values at the same positions): sub-block j = 8 hh + 2 q + jb of half hh,
//    quarter q takes the low (q < 2) or high nibbles of ql bytes
//    64 hh + 32 (q & 1) + 16 jb + 8 h .. +7 and bits 2q, 2q+1 of qh bytes
//    32 hh + 16 jb + 8 h .. +7 -- each lane reads its own 96 of the block's
//    192 quant bytes, no byte twice in the wave -- straight from memory, or
//    (plain layout, rows of more than 8 super-blocks) from a copy of the
//    wave's 32 blocks in LDS made with 16-byte loads, which costs the L1 a
//    fraction of the tag lookups;
//  * per sub-block one MFMA gives I_j = sum q x over its 16 weights for 32
//    rows x 32 columns; the lane's output registers sit in its own column, so
//    the scale is a per-lane integer: acc += sc_j * I_j (24-bit multiply-add,
//    |acc| < 2^28), only on the registers that hold rows below M (the
//    16-row form: 8 of the 16; M <= 8: 4);
//  * the offset 32 of the quants is taken out with the activation group sums:
//    sum_j sc_j (I_j - 32 bsum_j), the bsum part one v_mfma_f32_32x32x16_f16
//    over the 16 sub-blocks (sc and bsum exact in f16, every partial sum an
//    integer below 2^24, so exact);
//  * y += (d_x d) (acc - 32 corr) in f32 per super-block;
//  * the waves' partial sums are added in LDS in wave order;
//  * SILU: gate and up rows interleaved in one tile (columns 2p, 2p+1), the
//    product silu(gate) * up written in place of the two outputs.
// Rows past M read as zero and columns past N re-read the last row; neither is
// stored.  The plain block layout (210-byte blocks, 2-byte aligned) and the
// repacked one (field arrays, repack.hip) read the same bytes.
#include "device.h"
#include "launch.h"

namespace gemmq {

namespace {

typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

constexpr int kMaxKS = 8;

// 8 bytes at a 2-byte-aligned address p: three dwords from p rounded down to
// a dword (so up to p + 9 is read; every caller has at least 12 bytes of its
// block from there), shifted into place.  The pointer is stepped back, not
// rebuilt from an integer, so the loads stay global-memory loads.
__device__ __forceinline__ uint2 ld8_a2(const uint8_t* p) {
  const uint32_t sh = (uint32_t)(reinterpret_cast<uintptr_t>(p) & 3u);  // 0 or 2
  const uint32_t* b = reinterpret_cast<const uint32_t*>(p - sh);
  const uint32_t r0 = b[0], r1 = b[1], r2 = b[2];
  return make_uint2(__builtin_amdgcn_alignbyte(r1, r0, sh), __builtin_amdgcn_alignbyte(r2, r1, sh));
}

// two int16 (packed in a dword) -> two f16 (exact: |value| <= 2048)
__device__ __forceinline__ uint32_t i16x2_to_h2(uint32_t w) {
  const h2 v = {(_Float16)(short)(w & 0xffffu), (_Float16)(short)(w >> 16)};
  return __builtin_bit_cast(uint32_t, v);
}

// two int8 (bytes k, k+1 of w) -> two f16
__device__ __forceinline__ uint32_t i8x2_to_h2(uint32_t w, int k) {
  const h2 v = {(_Float16)(int)(int8_t)(w >> (8 * k)), (_Float16)(int)(int8_t)(w >> (8 * k + 8))};
  return __builtin_bit_cast(uint32_t, v);
}

// What one lane reads for one super-block.
struct Sk6W {
  uint2 ql[2][2][2];  // [hh][q & 1][jb]: ql bytes 64 hh + 32 (q&1) + 16 jb + 8 h .. +7
  uint2 qh[2][2];     // [hh][jb]: qh bytes 32 hh + 16 jb + 8 h .. +7
  uint32_t sc[4];     // the column's 16 int8 scales
  uint32_t d;         // f16 d (low half)
};

struct Sk6X {
  uint2 x[16];   // activation values 16 j + 8 h .. +7, j = 0..15
  uint4 bs;      // group sums 8 h .. 8 h + 7 (int16)
  uint32_t dx;   // d_x (f32 bits)
};

template <bool RP>
__device__ __forceinline__ void sk6_load_w(Sk6W& r, const uint8_t* mat, int64_t blk, int64_t NB,
                                           int h) {
  if constexpr (RP) {
    // ql[NB][128] | qh[NB][64] | sc[NB][16] | d[NB][2]
    const uint8_t* lp = mat + 128 * blk + 8 * h;
    const uint8_t* hp = mat + 128 * NB + 64 * blk + 8 * h;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int q1 = 0; q1 < 2; ++q1)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) r.ql[hh][q1][jb] = ld8(lp + 64 * hh + 32 * q1 + 16 * jb);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) r.qh[hh][jb] = ld8(hp + 32 * hh + 16 * jb);
    const uint4 s = ld16a(mat + 192 * NB + 16 * blk);
    r.sc[0] = s.x; r.sc[1] = s.y; r.sc[2] = s.z; r.sc[3] = s.w;
    r.d = ld2(mat + 208 * NB + 2 * blk);
  } else {
    const uint8_t* wb = mat + blk * kQ6KBytes;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int q1 = 0; q1 < 2; ++q1)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
          r.ql[hh][q1][jb] = ld8_a2(wb + 64 * hh + 32 * q1 + 16 * jb + 8 * h);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) r.qh[hh][jb] = ld8_a2(wb + 128 + 32 * hh + 16 * jb + 8 * h);
    // scales (bytes 192..207) and d (208, 209): five dwords from byte 188
    // (block 4-byte aligned) or 190 (2 mod 4), the last ending at byte 207 or 209
    const uint32_t sh = (uint32_t)(reinterpret_cast<uintptr_t>(wb) & 3u);
    const uint32_t* sb = reinterpret_cast<const uint32_t*>(wb + 188 + sh);
    const uint32_t r0 = sb[0], r1 = sb[1], r2 = sb[2], r3 = sb[3], r4 = sb[4];
    // the scales start 4 bytes (aligned block) or 2 bytes into the span
    r.sc[0] = sh ? __builtin_amdgcn_alignbyte(r1, r0, 2) : r1;
    r.sc[1] = sh ? __builtin_amdgcn_alignbyte(r2, r1, 2) : r2;
    r.sc[2] = sh ? __builtin_amdgcn_alignbyte(r3, r2, 2) : r3;
    r.sc[3] = sh ? __builtin_amdgcn_alignbyte(r4, r3, 2) : r4;
    r.d = ld2(wb + 208);
  }
}

// Weight staging (plain layout).  A lane of the MFMA layout wants 8-byte runs
// of its own column, so loading them straight from memory makes every 16-lane
// group of every load touch 16 rows' cache lines, one L1 tag lookup each:
// about 1300 lookups per wave and super-block, and at one lookup per clock that
// bounds the launch.  Instead each wave first copies its 32 columns' blocks
// into LDS -- each 16-lane group one column's 208 leading bytes with 16-byte
// loads, a few lines per group -- and then reads the runs from there.  Column
// c's slot starts at dword kSlot * c (an odd stride, so the lanes' dword reads
// fall in different banks); block byte i sits at slot byte s + i, s the
// block's start mod 4 (0 or 2); dword 52 holds the bytes that carry d.
constexpr int kSlot = 57;               // dwords per column slot
constexpr int kWaveStage = 32 * kSlot;  // dwords per wave

// A tile column's row: its matrix and its first block's index.
struct Sk6Src {
  const uint8_t* mat;
  int64_t blk;
};

// `blk(c)`: the first byte of tile column c's current block.
template <typename Blk>
__device__ __forceinline__ void sk6_stage(uint32_t* sw, const Blk& blk, int lane) {
  const int k = lane & 15;  // 16-byte piece k of the slot (k < 13)
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int c = 4 * r + (lane >> 4);
    if (k < 13) {
      // from the block's start rounded down to a dword: 208 bytes, all inside
      // this block or the one before it (s = 2 only past a matrix's first block)
      const uint8_t* wb = blk(c);
      const uint32_t sh = (uint32_t)(reinterpret_cast<uintptr_t>(wb) & 3u);
      const u32x4 v = ld16(wb - sh + 16 * k);
      uint32_t* d = sw + kSlot * c + 4 * k;
      d[0] = v.x;
      d[1] = v.y;
      d[2] = v.z;
      d[3] = v.w;
    }
  }
}

// The bytes that hold d of the block at wb, into column c's slot: s = 2, the
// dword ending at block byte 209; s = 0, bytes 208 and 209 alone (the dword
// from 208 would pass the block's end).
__device__ __forceinline__ void sk6_stage_d(uint32_t* sw, const uint8_t* wb, int c) {
  const uint32_t sh = (uint32_t)(reinterpret_cast<uintptr_t>(wb) & 3u);
  sw[kSlot * c + 52] = sh ? ld4(wb - sh + 208) : (uint32_t)ld2(wb + 208);
}

// The lane's runs from its column's slot sl (block start shift s, 0 or 2): the
// same values sk6_load_w reads from memory.
__device__ __forceinline__ void sk6_read_w(Sk6W& r, const uint32_t* sl, uint32_t s, int h) {
  auto run = [&](int o) -> uint2 {  // block bytes o .. o + 7, o a multiple of 8
    const uint32_t* p = sl + (o >> 2);
    const uint32_t r0 = p[0], r1 = p[1], r2 = p[2];
    return make_uint2(__builtin_amdgcn_alignbyte(r1, r0, s), __builtin_amdgcn_alignbyte(r2, r1, s));
  };
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int q1 = 0; q1 < 2; ++q1)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) r.ql[hh][q1][jb] = run(64 * hh + 32 * q1 + 16 * jb + 8 * h);
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) r.qh[hh][jb] = run(128 + 32 * hh + 16 * jb + 8 * h);
  // scales: block bytes 192..207; d: 208, 209
  uint32_t w[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) w[i] = sl[48 + i];
#pragma unroll
  for (int i = 0; i < 4; ++i) r.sc[i] = __builtin_amdgcn_alignbyte(w[i + 1], w[i], s);
  r.d = s ? w[4] >> 16 : w[4] & 0xffffu;
}

__device__ __forceinline__ void sk6_load_x(Sk6X& r, const uint8_t* xb, bool ok, int h) {
  if (ok) {
#pragma unroll
    for (int j = 0; j < 16; ++j) r.x[j] = ld8(xb + 4 + 16 * j + 8 * h);
    const u32x4 b = ld16(xb + 260 + 16 * h);
    r.bs = make_uint4(b.x, b.y, b.z, b.w);
    r.dx = ld4(xb);
  } else {  // rows past M: zero operands, nothing loaded
#pragma unroll
    for (int j = 0; j < 16; ++j) r.x[j] = make_uint2(0u, 0u);
    r.bs = make_uint4(0u, 0u, 0u, 0u);
    r.dx = 0u;
  }
}

// One super-block.  RL: output registers holding rows below M (4: M <= 8,
// 8: M <= 16); register i holds row 8 (i / 4) + 4 h + i % 4.
template <int RL>
__device__ __forceinline__ void sk6_compute(const Sk6W& w, const Sk6X& x, int h, float (&y)[RL]) {
  // the weight operands of the 16 sub-blocks, j = 8 hh + 2 q + jb
  long wop[16];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
    for (int q1 = 0; q1 < 2; ++q1) {
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        const uint2 l = w.ql[hh][q1][jb];
        const uint2 hb = w.qh[hh][jb];
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          const int q = q1 + 2 * q2;  // quarter: low nibbles for q < 2
          uint32_t t[2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const uint32_t lv = k ? l.y : l.x, hv = k ? hb.y : hb.x;
            // bits 2q, 2q+1 of each qh byte moved to bits 4, 5
            const uint32_t hs = q == 0 ? hv << 4 : q == 1 ? hv << 2 : q == 2 ? hv : hv >> 2;
            t[k] = (hs & 0x30303030u) | ((q2 ? lv >> 4 : lv) & 0x0f0f0f0fu);
          }
          wop[8 * hh + 2 * q + jb] = (long)(((uint64_t)t[1] << 32) | t[0]);
        }
      }
    }
  }
  // one MFMA per sub-block, the scaling of the previous one's product in its
  // shadow (two products live, so the matrix core never waits on the adds)
  int acc[RL];
#pragma unroll
  for (int i = 0; i < RL; ++i) acc[i] = 0;
  v16i I[2];
#pragma unroll
  for (int j = 0; j <= 16; ++j) {
    if (j < 16) {
      const long xop = (long)(((uint64_t)x.x[j].y << 32) | x.x[j].x);
      I[j & 1] = __builtin_amdgcn_mfma_i32_32x32x16_i8(xop, wop[j], (v16i){0}, 0, 0, 0);
    }
    if (j > 0) {
      const int jp = j - 1;
      const int sc = (int)(int8_t)(w.sc[jp >> 2] >> (8 * (jp & 3)));
#pragma unroll
      for (int i = 0; i < RL; ++i) acc[i] = __mul24(sc, I[jp & 1][i]) + acc[i];
    }
  }
  // sum_j sc_j bsum_j: A = the row's group sums 8h..8h+7, B = the column's
  // scales 8h..8h+7 (same K order on both sides)
  const uint32_t bh[4] = {i16x2_to_h2(x.bs.x), i16x2_to_h2(x.bs.y), i16x2_to_h2(x.bs.z),
                          i16x2_to_h2(x.bs.w)};
  const uint32_t s0 = h ? w.sc[2] : w.sc[0], s1 = h ? w.sc[3] : w.sc[1];
  const uint32_t sh[4] = {i8x2_to_h2(s0, 0), i8x2_to_h2(s0, 2), i8x2_to_h2(s1, 0),
                          i8x2_to_h2(s1, 2)};
  const v16f corr = __builtin_amdgcn_mfma_f32_32x32x16_f16(
      __builtin_bit_cast(v8h, bh), __builtin_bit_cast(v8h, sh), (v16f){0.f}, 0, 0, 0);
  const float d = f16_to_f32(w.d);
#pragma unroll
  for (int i = 0; i < RL; ++i) {
    // d_x of register i's row, from the lane that loaded it
    const int row = 8 * (i >> 2) + 4 * h + (i & 3);
    const float dx = __builtin_bit_cast(float, __shfl((int)x.dx, row, 64));
    const float t = fmaf(-32.0f, corr[i], (float)acc[i]);
    y[i] = fmaf(dx * d, t, y[i]);
  }
}

// y = silu(g) * u in f32, the same steps as the other kernels'
__device__ __forceinline__ float silu_mul_f32(float g, float u) {
  return g / (1.0f + expf(-g)) * u;
}

// FMT: 14 (q6_K) or 256 + 14 (its repacked layout).  SILU: the tiles cover the
// gate/up pair as one virtual matrix of 2N rows (row 2p gate row p of gt.W[0],
// row 2p+1 up row p of gt.W[1]); lanes n and n ^ 1 hold one output column's
// gate and up.
// STG: the staged weight loads (plain layout), the M <= 8 form held to four
// waves per SIMD (two workgroups per CU) as the direct form has.
template <int FMT, bool SILU, int RL, bool STG>
__global__ __launch_bounds__(64 * kMaxKS, STG ? (RL == 4 ? 4 : 2) : 1) void skinny_q6k_kernel(
    const GroupTiles gt, const uint8_t* __restrict__ Xq, int M, int nb, int bpw) {
  constexpr bool RP = FMT > 255;
  // per wave: (STG) its staged blocks, and after its last super-block its
  // partial sums for the reduction
  constexpr int kStride = STG ? kWaveStage : RL * 64;
  __shared__ uint32_t stage[kMaxKS * kStride];
  static_assert(RL * 64 <= kStride, "partial sums fit a wave's area");
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int ks = (int)(blockDim.x >> 6);
  const int lane = lane_id(), n = lane & 31, h = lane >> 5;
  const TileMatrix tm = tile_matrix(gt, blockIdx.x);
  const int64_t N = tm.N;  // SILU: 2 x the output columns
  const int64_t col = (int64_t)tm.local * 32 + n;
  const int64_t NB = (SILU ? N >> 1 : N) * nb;  // repacked: blocks in the matrix
  // the matrix and first block of tile column c (past N: the last column)
  auto column = [&](int c) -> Sk6Src {
    const int64_t cl = (int64_t)tm.local * 32 + c;
    const int64_t cc = cl < N ? cl : N - 1;
    if constexpr (SILU) return Sk6Src{(cc & 1) ? gt.W[1] : tm.W, (cc >> 1) * nb};
    else return Sk6Src{tm.W, cc * nb};
  };
  const Sk6Src own = column(n);
  const bool xok = n < M;
  const uint8_t* xrow = Xq + (int64_t)(xok ? n : M - 1) * nb * kQ8KBytes;
  const int b0 = wave * bpw, b1 = b0 + bpw < nb ? b0 + bpw : nb;
  uint32_t* sw = stage + wave * kStride;

  float y[RL];
#pragma unroll
  for (int i = 0; i < RL; ++i) y[i] = 0.f;
  for (int b = b0; b < b1; ++b) {
    if constexpr (STG) {
      static_assert(!RP, "the staged loads read the plain block layout");
      // the first byte of tile column c's block b
      auto blk = [&](int c) -> const uint8_t* {
        const Sk6Src t = column(c);
        return t.mat + (t.blk + b) * kQ6KBytes;
      };
      sk6_stage(sw, blk, lane);
      const uint8_t* mine = own.mat + (own.blk + b) * kQ6KBytes;
      if (h == 0) sk6_stage_d(sw, mine, n);
      Sk6X x;
      sk6_load_x(x, xrow + (int64_t)b * kQ8KBytes, xok, h);
      // the copies are read by other lanes of this wave only
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      Sk6W w;
      const uint32_t s = (uint32_t)(reinterpret_cast<uintptr_t>(mine) & 3u);
      sk6_read_w(w, sw + kSlot * n, s, h);
      sk6_compute<RL>(w, x, h, y);
      // every lane's reads of this block precede the next block's copies
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
    } else {
      Sk6W w;
      Sk6X x;
      sk6_load_w<RP>(w, own.mat, own.blk + b, NB, h);
      sk6_load_x(x, xrow + (int64_t)b * kQ8KBytes, xok, h);
      sk6_compute<RL>(w, x, h, y);
    }
  }
  if (ks > 1) {
    // the partial sums' bits in the wave's own area, added in wave order
#pragma unroll
    for (int i = 0; i < RL; ++i) sw[64 * i + lane] = __builtin_bit_cast(uint32_t, y[i]);
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int i = 0; i < RL; ++i) {
      float v = __builtin_bit_cast(float, stage[64 * i + lane]);
      for (int k = 1; k < ks; ++k) v += __builtin_bit_cast(float, stage[k * kStride + 64 * i + lane]);
      y[i] = v;
    }
  }
#pragma unroll
  for (int i = 0; i < RL; ++i) {
    const int row = 8 * (i >> 2) + 4 * h + (i & 3);
    if constexpr (SILU) {
      const int64_t Nout = N >> 1, p = col >> 1;
      const float up = __shfl_xor(y[i], 1, 64);  // every lane takes part
      if ((n & 1) == 0 && p < Nout && row < M) tm.Y[(int64_t)row * Nout + p] = silu_mul_f32(y[i], up);
    } else if (col < N && row < M) {
      tm.Y[(int64_t)row * N + col] = y[i];
    }
  }
}

template <int FMT, bool SILU>
void launch_rl(const GroupTiles& gt, const uint8_t* Xq, int M, int nb, int ks, int bpw,
               hipStream_t st) {
  const dim3 grid(gt.start[kMaxGroup]), block(64 * ks);
  // staged weight loads for the plain layout on rows of more than 8
  // super-blocks (several per wave); elsewhere the direct loads measured faster
  // (the same bits either way)
  if constexpr (FMT == 14) {
    if (nb > 8) {
      if (M <= 8)
        hipLaunchKernelGGL((skinny_q6k_kernel<FMT, SILU, 4, true>), grid, block, 0, st, gt, Xq, M, nb, bpw);
      else
        hipLaunchKernelGGL((skinny_q6k_kernel<FMT, SILU, 8, true>), grid, block, 0, st, gt, Xq, M, nb, bpw);
      return;
    }
  }
  if (M <= 8)
    hipLaunchKernelGGL((skinny_q6k_kernel<FMT, SILU, 4, false>), grid, block, 0, st, gt, Xq, M, nb, bpw);
  else
    hipLaunchKernelGGL((skinny_q6k_kernel<FMT, SILU, 8, false>), grid, block, 0, st, gt, Xq, M, nb, bpw);
}

}  // namespace

bool skinny_q6k_fits(int fmt, int64_t M) {
  return (fmt == 14 || fmt == 256 + 14) && M >= 1 && M <= 16;
}

template <bool SILU>
int launch_skinny_q6k_any(int fmt, const Group& g, const uint8_t* Xq, int M, int64_t K,
                          hipStream_t st) {
  if (!skinny_q6k_fits(fmt, M)) return -1;
  const int64_t nb64 = K / kQK;
  if (nb64 < 1 || nb64 > 0x7fffffffLL) return -1;
  const int nb = (int)nb64;
  GroupTiles gt;
  if (!(SILU ? make_pair_tiles(g, 32, gt) : make_tiles(g, 32, gt))) return -1;
  if (gt.start[kMaxGroup] == 0) return 0;
  // waves per workgroup and super-blocks per wave: at most 8 waves, each a
  // contiguous part of ceil(nb / 8) super-blocks (a function of K alone)
  const int bpw = (nb + kMaxKS - 1) / kMaxKS;
  const int ks = (nb + bpw - 1) / bpw;
  if (fmt == 14)
    launch_rl<14, SILU>(gt, Xq, M, nb, ks, bpw, st);
  else
    launch_rl<256 + 14, SILU>(gt, Xq, M, nb, ks, bpw, st);
  return 0;
}

int launch_skinny_q6k(int fmt, const Group& g, const uint8_t* Xq, int M, int64_t K,
                      hipStream_t st) {
  return launch_skinny_q6k_any<false>(fmt, g, Xq, M, K, st);
}

int launch_skinny_q6k_silu(int fmt, const Group& g, const uint8_t* Xq, int M, int64_t K,
                           hipStream_t st) {
  if (g.count != 2 || g.N[0] != g.N[1]) return -1;
  return launch_skinny_q6k_any<true>(fmt, g, Xq, M, K, st);
}

}  // namespace gemmq
