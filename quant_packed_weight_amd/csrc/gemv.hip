// gemv.hip -- step a3: the decode-time packed GEMV, M = 1..8 activation rows.
//
// Decode time on the pages is the walk over the packed weights (molayo article
// "PocketLLM: 단일 가속기에서 대규모 언어 모델 실행", status row "src/ -- C++
// engine": the packed dot walks each weight row once per tile of activation
// rows).  On gfx950 that walk is an HBM stream, and a plain one-shot read kernel
// (one wave per row slice, all loads issued at once) already reaches ~5.8 TB/s
// on a 28 MB matrix, so this kernel keeps exactly that access shape and spends
// as few vector instructions per weight byte as it can:
//
//  * One 64-lane wavefront owns P weight rows and issues every weight load of
//    them before any arithmetic.  Four lanes share a super-block: q4_K lane g
//    takes the 32 quant bytes of 64-weight group g (sub-blocks 2g and 2g+1),
//    q5_K the same plus the 32 high-bit bytes; q2_K and q3_K lane g takes
//    weights 64g..64g+63 (sub-blocks 4g..4g+3) from the 32 bytes of 2-bit
//    parts of half g/2 (q3_K also the 32 mask bytes); q6_K lane (half hh,
//    pair p) takes quarters p and p+2 of half hh.  A round
//    is 16 consecutive blocks of a row (or, for rows of 16/P blocks, P rows side
//    by side), so one load instruction of the wave covers 2.3 KiB (q4_K) of
//    contiguous weight bytes.
//  * Activation fragments are read straight from global memory: the q8_K rows
//    are small and stay cache-resident, and staging them in LDS (tried) costs a
//    barrier and a second round trip that the stream cannot hide.  A wave
//    whose row fills a round takes two rows (R = 2): each activation fragment
//    it loads serves both, which halves the cached activation traffic that
//    otherwise slows the weight stream (measured: 3.6 -> 4.0 TB/s over the
//    Qwen3-8B layer's launches).
//  * Integer dot products on v_dot4 (int8 x int8 -> int32); the scale and min
//    corrections use 24-bit multiplies and v_dot2 on the int16 group sums; one
//    f32 fold per block and lane applies d_w, dmin and d_x.
//  * The 64/P lane partials of each output are combined by a fixed xor tree.
//  * Rows longer than one round are split over up to four waves of one
//    workgroup (a round each, looping beyond 64 blocks): more, shorter waves
//    keep the stream as parallel as for short rows; the waves' partial sums
//    are added in LDS in wave order.
//  * The fused form (FUSED, through gemmq_linear_group at decode shapes) also
//    does the activation quantizer's work: a workgroup of eight row groups
//    loads its share of the f32 activations first, then its weights, quantizes
//    (the same q8k_block routine as the quantizer kernel) into LDS while the
//    weights are in flight, and computes from LDS after one barrier.  That
//    saves the quantizer launch; every workgroup repeats the quantization, so
//    it is only used for rows of at most 16 blocks and M <= 4, on launches
//    small enough that a quantizer launch of its own would cost more.
//  * The staged form (FUSED and STAGE) runs the same workgroups on q8_K blocks
//    already in memory, each wave copying its share into LDS (three loads a
//    block) instead of quantizing it: taken by large launches (rows x M x
//    K/256 from 2^18), where the plain form's per-lane activation reads from L2
//    and the fused form's repeated quantizing cost more, up to M = 8.
//
// Every output's arithmetic (per-lane block order, the xor tree and the wave
// order) depends only on K, never on M or N, and is the same in all forms, so
// row m of an M-row call equals a one-row call on that row bit for bit.
#include "device.h"
#include "launch.h"
#include "quant_block.h"

namespace gemmq {

namespace {


typedef short i16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int dot2(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot2(__builtin_bit_cast(i16x2, a), __builtin_bit_cast(i16x2, b), c,
                                false);
}
__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// 36 bytes from a dword-aligned address in three loads (two of 16 B).
__device__ __forceinline__ void ld36(const uint8_t* p, uint32_t (&o)[9]) {
  const u32x4 a = ld16(p), b = ld16(p + 16);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  o[8] = ld4(p + 32);
}

// 32 bytes at a 2-byte-aligned address: the 36 bytes from p rounded down to a
// dword (so at most p + 35 is read; every caller stays inside its block),
// shifted into place.  The address is rebuilt from an integer, so these are
// flat loads; the same loads kept global (p stepped back instead) measured 4%
// slower over the 151936 x 2048 q6_K head at M = 1 and no faster elsewhere.
__device__ __forceinline__ void ld32_a2(const uint8_t* p, uint32_t (&o)[8]) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  uint32_t raw[9];
  ld36(reinterpret_cast<const uint8_t*>(a & ~uintptr_t(3)), raw);
  const uint32_t sh = (uint32_t)(a & 3u);
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = __builtin_amdgcn_alignbyte(raw[i + 1], raw[i], sh);
}

// Exchange with lane ^ D: DPP quad permutes for 1 and 2, ds_swizzle (xor mode,
// inside 32-lane halves) for 4, 8 and 16, a bpermute for 32.
template <int D>
__device__ __forceinline__ float xor_lane(float v) {
  const int i = __builtin_bit_cast(int, v);
  int r;
  if constexpr (D == 1)
    r = __builtin_amdgcn_mov_dpp(i, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
  else if constexpr (D == 2)
    r = __builtin_amdgcn_mov_dpp(i, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
  else if constexpr (D == 4 || D == 8 || D == 16)
    r = __builtin_amdgcn_ds_swizzle(i, 0x1F | (D << 10));   // and 0x1F, or 0, xor D
  else
    r = __shfl_xor(i, D, 64);
  return __builtin_bit_cast(float, r);
}

// One step at xor distance D.  While a lane holds several values it keeps half
// and sends half (reduce-scatter); otherwise it adds its partner's value.  Each
// sum adds the partials of lanes l and l ^ D, so the f32 result of every output
// is the same whichever lane computes it and however many values there are.
template <int D, int V>
__device__ __forceinline__ void seg_step(float (&v)[V], int& cnt, int lane) {
  if (cnt > 1) {
    const bool up = (lane & D) != 0;
    const int h = cnt / 2;
#pragma unroll
    for (int j = 0; j < V / 2; ++j) {
      if (j < h) {
        const float send = up ? v[j] : v[j + h];
        const float keep = up ? v[j + h] : v[j];
        v[j] = keep + xor_lane<D>(send);
      }
    }
    cnt = h;
  } else {
    v[0] = v[0] + xor_lane<D>(v[0]);
  }
}

// Whether a wave compiled for MT activation rows computes row m of a call with
// M rows: rows up to MT/2 always (the MT-row form serves MT/2 < M <= MT), the
// others while m < M.  Skipped rows keep a zero partial that is never stored;
// the reduction over the MT-row layout is the same, so the bits of the real
// rows do not depend on the skip.  The eight-row form computes every row (the
// wave-uniform branches measured 10-60% slower there at any M, while the
// four-row form gained up to 30% at M = 3 and up to 14% at M = 4).
template <int MT>
__device__ __forceinline__ bool row_live(int m, int M) {
  return MT > 4 || m <= MT / 2 || m < M;
}

// Reduce-scatter over segments of SEG lanes (V <= SEG, a power of two): lane l
// ends with the total of value vidx<V, SEG>(l) in v[0].
template <int V, int SEG>
__device__ __forceinline__ void seg_reduce(float (&v)[V], int lane) {
  int cnt = V;
  if constexpr (SEG >= 64) seg_step<32>(v, cnt, lane);
  if constexpr (SEG >= 32) seg_step<16>(v, cnt, lane);
  if constexpr (SEG >= 16) seg_step<8>(v, cnt, lane);
  if constexpr (SEG >= 8) seg_step<4>(v, cnt, lane);
  if constexpr (SEG >= 4) seg_step<2>(v, cnt, lane);
  seg_step<1>(v, cnt, lane);
}

// Full butterfly of one value over a segment of SEG lanes (same pairs).
template <int SEG>
__device__ __forceinline__ float seg_all(float v) {
  if constexpr (SEG >= 64) v = v + xor_lane<32>(v);
  if constexpr (SEG >= 32) v = v + xor_lane<16>(v);
  if constexpr (SEG >= 16) v = v + xor_lane<8>(v);
  if constexpr (SEG >= 8) v = v + xor_lane<4>(v);
  if constexpr (SEG >= 4) v = v + xor_lane<2>(v);
  return v + xor_lane<1>(v);
}

template <int V, int SEG>
__device__ __forceinline__ int vidx(int lane) {
  int idx = 0, cnt = V;
#pragma unroll
  for (int d = SEG / 2; d >= 1; d >>= 1)
    if (cnt > 1) {
      cnt /= 2;
      if (lane & d) idx += cnt;
    }
  return idx;
}

template <int V, int SEG>
__device__ __forceinline__ bool holder(int lane) {
  int cnt = V;
  bool ok = true;
#pragma unroll
  for (int d = SEG / 2; d >= 1; d >>= 1) {
    if (cnt > 1)
      cnt /= 2;
    else if (lane & d)
      ok = false;
  }
  return ok;
}

// Activation fragment of block b, row m: two 32-byte runs of values at byte
// offsets qoff and qoff2, the dwords of group sums at soff and soff2 (offsets
// into the 32 bytes of sums), and d.
struct XFrag {
  u32x4 a0, a1, b0, b1;
  uint32_t s0, s1;
  float d;
};

__device__ __forceinline__ XFrag x_frag(const uint8_t* __restrict__ Xq, int nb, int m, int b,
                                        int qoff, int qoff2, int soff, int soff2) {
  XFrag f;
  const uint8_t* p = Xq + ((int64_t)m * nb + b) * kQ8KBytes;
  f.a0 = ld16(p + 4 + qoff);
  f.a1 = ld16(p + 4 + qoff + 16);
  f.b0 = ld16(p + 4 + qoff2);
  f.b1 = ld16(p + 4 + qoff2 + 16);
  f.s0 = ld4(p + 260 + soff);
  f.s1 = ld4(p + 260 + soff2);
  f.d = *reinterpret_cast<const float*>(p);
  return f;
}

// The fused form's LDS copy of the activations: block (m, b) at (m nb + b) kXL
// bytes holds the 256 values (16-byte aligned), the 16 sums at +256 and d at +288.
constexpr int kXL = 304;

__device__ __forceinline__ XFrag x_frag_lds(const uint8_t* xl, int nb, int m, int b, int qoff,
                                            int qoff2, int soff, int soff2) {
  const uint8_t* p = xl + (m * nb + b) * kXL;
  const uint4 a0 = *reinterpret_cast<const uint4*>(p + qoff);
  const uint4 a1 = *reinterpret_cast<const uint4*>(p + qoff + 16);
  const uint4 b0 = *reinterpret_cast<const uint4*>(p + qoff2);
  const uint4 b1 = *reinterpret_cast<const uint4*>(p + qoff2 + 16);
  XFrag f;
  f.a0 = {a0.x, a0.y, a0.z, a0.w};
  f.a1 = {a1.x, a1.y, a1.z, a1.w};
  f.b0 = {b0.x, b0.y, b0.z, b0.w};
  f.b1 = {b1.x, b1.y, b1.z, b1.w};
  f.s0 = *reinterpret_cast<const uint32_t*>(p + 256 + soff);
  f.s1 = *reinterpret_cast<const uint32_t*>(p + 256 + soff2);
  f.d = *reinterpret_cast<const float*>(p + 288);
  return f;
}

__device__ __forceinline__ int dot16(const uint32_t* w, const u32x4& x, int s) {
  s = dot4(w[0], x.x, s);
  s = dot4(w[1], x.y, s);
  s = dot4(w[2], x.z, s);
  return dot4(w[3], x.w, s);
}

// ---------------------------------------------------------------- kernel
// SiLU-gated product (SILU): y = silu(g) * u from the two outputs g, u of one
// row of the gate and the up matrix, in f32: e = exp(-g) (the device expf),
// s = g / (1 + e) correctly rounded, y = s * u.
__device__ __forceinline__ float silu_mul_f32(float g, float u) {
  return g / (1.0f + expf(-g)) * u;
}

// Blocks each wave of the fused form quantizes: the M nb <= MT nbmax blocks of
// the activation (nbmax = 16 / P when P rows of 16 / P blocks share a round,
// else rows of up to 16 blocks) spread over its RG waves, at most four.  Rows
// of 8 blocks at M = 1, for instance, need one block per wave, not two.
constexpr int fused_qb(int MT, int P, int RG) {
  const int n = (MT * (P > 1 ? 16 / P : 16) + RG - 1) / RG;
  return n < 4 ? n : 4;
}

// Blocks each wave of the staged form copies: the same count, up to eight (a
// copy is three loads, not a quantization), so that it also serves M = 5..8.
constexpr int stage_qb(int MT, int P, int RG) {
  const int n = (MT * (P > 1 ? 16 / P : 16) + RG - 1) / RG;
  return n < 8 ? n : 8;
}

// FMT: the GGUF type id (10 q2_K .. 14 q6_K), plus 256 for the repacked q3_K /
// q6_K layout (repack.hip).  MT activation rows computed (>= M).  IT rounds of 16
// blocks loaded together.  P rows per round.  KS waves share one row (P = 1):
// wave w takes rounds w, w + KS, ... and the KS partial sums meet in LDS, added
// in wave order.  R rows per wave (P = 1), computed side by side on the same
// activation fragments.  The grid is the concatenation of every grouped
// matrix's tiles (one tile = P R rows, one workgroup of KS waves).
// SILU: the group is one virtual matrix of 2N rows whose row 2n is gate row n
// (gt.W[0]) and row 2n+1 up row n (gt.W[1]); P R is even, so a wave's rows come
// in (gate, up) pairs computed exactly as in two plain calls, and the pair's
// outputs meet in LDS for y[m][n] = silu(g) * u (Y has N columns).
template <int FMT, int MT, int IT, int P, int KS, int R, int RG, bool FUSED, bool SILU,
          bool STAGE = false>
__global__ __launch_bounds__(64 * KS * RG) void gemv_kernel(const GroupTiles gt,
                                                            uint8_t* __restrict__ Xq,
                                                            const float* __restrict__ X, int nb,
                                                            int M) {
  constexpr bool RP = FMT > 255;  // the repacked layout of q3_K / q6_K
  constexpr int BF = FMT & 255;   // the block format
  constexpr int SEG = 64 / P;  // lanes that share a row
  constexpr int BPR = 16 / P;  // blocks of a row per round when P > 1
  constexpr int BB = BF == 10 ? 84 : BF == 11 ? 110 : BF == 12 ? kQ4KBytes : BF == 13 ? 176
                                                                                  : kQ6KBytes;
  constexpr int NW = KS * RG;  // waves of the workgroup
  const int lane = lane_id();
  const int G = lane >> 2, c = lane & 3;
  const int prow = P > 1 ? G / BPR : 0;
  const int bl0 = P > 1 ? G % BPR : G;
  static_assert(KS == 1 || P == 1, "split rows only when one row fills a round");
  static_assert(R == 1 || P == 1, "several rows per wave only when one row fills a round");
  static_assert(!FUSED || IT == 1, "the fused form takes one round per wave");
  static_assert(!SILU || (P * R) % 2 == 0, "gate/up rows come in pairs");
  constexpr int V = R * MT;  // outputs of a wave: value r * MT + m is row r, activation row m
  const int wv = NW > 1 ? __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) : 0;
  const int w = wv % KS, rg = wv / KS;  // K share and row group of this wave
  const TileMatrix tm = tile_matrix(gt, blockIdx.x);
  // take the activation pointers with the rest of the kernel arguments, so the
  // loads below do not wait for a second round of scalar loads
  asm volatile("" ::"s"(Xq), "s"(X));
  const uint8_t* __restrict__ W = tm.W;
  float* __restrict__ Y = tm.Y;
  const int64_t N = tm.N;
  const int64_t n0 = (int64_t)tm.local * (RG * P * R) + rg * (P * R);  // first row of this wave
  const uint8_t* wrow[R];  // the row's first block (block layout)
  const uint8_t* wmat[R];  // repacked: the row's matrix and its first block index
  int64_t wblk[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int64_t n = n0 + prow + r;
    if constexpr (SILU) {
      if (n >= N) n = N - 2 + (n & 1);  // tail pairs: a valid pair, never stored
      wmat[r] = (n & 1) ? gt.W[1] : W;
      wblk[r] = (n >> 1) * nb;
    } else {
      if (n >= N) n = N - 1;  // tail rows: a valid row, never stored
      wmat[r] = W;
      wblk[r] = n * nb;
    }
    wrow[r] = wmat[r] + wblk[r] * BB;
  }
  // repacked: blocks in the matrix (its field arrays are NB entries long)
  const int64_t NB = (SILU ? N >> 1 : N) * nb;

  // per-lane constants
  // q2_K, q3_K, q4_K, q5_K lane c: values 64c..64c+63, sums 4c..4c+3 (q4_K and
  //   q5_K: sub-blocks 2c, 2c+1; q2_K and q3_K: sub-blocks 4c..4c+3).
  // q6_K lane c = (hh, p) = (c/2, c%2): quarters p and p+2 of half hh, i.e. values
  //   128hh+32p.. and 128hh+32p+64.., sums 8hh+2p, +1 and 8hh+2p+4, +5.
  const int qoff = BF != 14 ? 64 * c : 128 * (c >> 1) + 32 * (c & 1);
  const int qoff2 = BF != 14 ? 64 * c + 32 : qoff + 64;
  const int soff = BF != 14 ? 8 * c : 2 * (8 * (c >> 1) + 2 * (c & 1));
  const int soff2 = soff + (BF != 14 ? 4 : 8);

  float acc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = 0.0f;

  // the fused form quantizes the activations into this workgroup's LDS, one
  // q8_K block per wave at a time, as [m][b] blocks of kXL bytes
  extern __shared__ __attribute__((aligned(16))) uint8_t xl[];
  auto xfrag = [&](int m, int b) {
    if constexpr (FUSED)
      return x_frag_lds(xl, nb, m, b, qoff, qoff2, soff, soff2);
    else
      return x_frag(Xq, nb, m, b, qoff, qoff2, soff, soff2);
  };

  // wq: q4_K quant bytes, q5_K low nibbles, q2_K/q3_K 2-bit bytes of half c/2,
  //     q6_K ql bytes; wh: q6_K qh bytes, q5_K high bits, q3_K mask (32 bytes each)
  // hd: q4_K/q5_K block header; q6_K [0] scale bytes, [1] d; q2_K [0] scale/min
  //     bytes 4c..4c+3, [1] d and dmin; q3_K [0..2] scale bytes, [3] d
  uint32_t wq[IT][R][8], wh[IT][R][8];
  uint32_t hd[IT][R][4];
  // ---- 1. every weight load of the IT rounds from block s0 on (lanes past the
  // row's end load its last block when `clamp`, else nothing)
  auto load_round = [&](int s0, bool clamp) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int i = 0; i < IT; ++i) {
        int b = s0 + bl0 + 16 * i;
        if (clamp) b = b < nb ? b : nb - 1;
        if (b < nb) {
          const uint8_t* wb = wrow[r] + b * BB;
          if constexpr (BF == 12 || BF == 13) {
            constexpr int QO = BF == 12 ? 16 : 48;  // quant (low nibble) bytes
            const uint4 h = ld16a(wb);
            const uint4 q0 = ld16a(wb + QO + 32 * c), q1 = ld16a(wb + QO + 16 + 32 * c);
            hd[i][r][0] = h.x; hd[i][r][1] = h.y; hd[i][r][2] = h.z; hd[i][r][3] = h.w;
            wq[i][r][0] = q0.x; wq[i][r][1] = q0.y; wq[i][r][2] = q0.z; wq[i][r][3] = q0.w;
            wq[i][r][4] = q1.x; wq[i][r][5] = q1.y; wq[i][r][6] = q1.z; wq[i][r][7] = q1.w;
            if constexpr (BF == 13) {
              const uint4 h0 = ld16a(wb + 16), h1 = ld16a(wb + 32);
              wh[i][r][0] = h0.x; wh[i][r][1] = h0.y; wh[i][r][2] = h0.z; wh[i][r][3] = h0.w;
              wh[i][r][4] = h1.x; wh[i][r][5] = h1.y; wh[i][r][6] = h1.z; wh[i][r][7] = h1.w;
            }
          } else if constexpr (BF == 10) {
            const u32x4 q0 = ld16(wb + 16 + 32 * (c >> 1)), q1 = ld16(wb + 32 + 32 * (c >> 1));
            wq[i][r][0] = q0.x; wq[i][r][1] = q0.y; wq[i][r][2] = q0.z; wq[i][r][3] = q0.w;
            wq[i][r][4] = q1.x; wq[i][r][5] = q1.y; wq[i][r][6] = q1.z; wq[i][r][7] = q1.w;
            hd[i][r][0] = ld4(wb + 4 * c);
            hd[i][r][1] = ld4(wb + 80);
          } else if constexpr (BF == 11 && RP) {
            // hmask[NB][32] | qs[NB][64] | scales[NB][12] | d[NB][2]
            const uint8_t* m = wmat[r];
            const int64_t bi = wblk[r] + b;
            const uint4 h0 = ld16a(m + 32 * bi), h1 = ld16a(m + 32 * bi + 16);
            const uint8_t* qp = m + 32 * NB + 64 * bi + 32 * (c >> 1);
            const uint4 q0 = ld16a(qp), q1 = ld16a(qp + 16);
            wh[i][r][0] = h0.x; wh[i][r][1] = h0.y; wh[i][r][2] = h0.z; wh[i][r][3] = h0.w;
            wh[i][r][4] = h1.x; wh[i][r][5] = h1.y; wh[i][r][6] = h1.z; wh[i][r][7] = h1.w;
            wq[i][r][0] = q0.x; wq[i][r][1] = q0.y; wq[i][r][2] = q0.z; wq[i][r][3] = q0.w;
            wq[i][r][4] = q1.x; wq[i][r][5] = q1.y; wq[i][r][6] = q1.z; wq[i][r][7] = q1.w;
            const uint8_t* sp = m + 96 * NB + 12 * bi;
            hd[i][r][0] = ld4(sp); hd[i][r][1] = ld4(sp + 4); hd[i][r][2] = ld4(sp + 8);
            hd[i][r][3] = ld2(m + 108 * NB + 2 * bi);
          } else if constexpr (BF == 11) {
            // 110-byte blocks are 2-byte aligned; every read stays in the block
            ld32_a2(wb, wh[i][r]);
            ld32_a2(wb + 32 + 32 * (c >> 1), wq[i][r]);
            uint32_t sb[3];
            ld_dwords_a2<3>(wb + 96, sb);
            hd[i][r][0] = sb[0]; hd[i][r][1] = sb[1]; hd[i][r][2] = sb[2];
            hd[i][r][3] = ld2(wb + 108);
          } else if constexpr (RP) {
            // q6_K repacked: ql[NB][128] | qh[NB][64] | sc[NB][16] | d[NB][2]
            const int hh = c >> 1, p = c & 1;
            const uint8_t* m = wmat[r];
            const int64_t bi = wblk[r] + b;
            const uint8_t* lp = m + 128 * bi + 64 * hh + 32 * p;
            const uint8_t* hp = m + 128 * NB + 64 * bi + 32 * hh;
            const uint4 l0 = ld16a(lp), l1 = ld16a(lp + 16), h0 = ld16a(hp), h1 = ld16a(hp + 16);
            wq[i][r][0] = l0.x; wq[i][r][1] = l0.y; wq[i][r][2] = l0.z; wq[i][r][3] = l0.w;
            wq[i][r][4] = l1.x; wq[i][r][5] = l1.y; wq[i][r][6] = l1.z; wq[i][r][7] = l1.w;
            wh[i][r][0] = h0.x; wh[i][r][1] = h0.y; wh[i][r][2] = h0.z; wh[i][r][3] = h0.w;
            wh[i][r][4] = h1.x; wh[i][r][5] = h1.y; wh[i][r][6] = h1.z; wh[i][r][7] = h1.w;
            const uint8_t* sp = m + 192 * NB + 16 * bi + 8 * hh + 2 * p;
            hd[i][r][0] = (uint32_t)ld2(sp) | ((uint32_t)ld2(sp + 4) << 16);
            hd[i][r][1] = ld2(m + 208 * NB + 2 * bi);
          } else {
            const int hh = c >> 1, p = c & 1;
            ld32_a2(wb + 64 * hh + 32 * p, wq[i][r]);
            ld32_a2(wb + 128 + 32 * hh, wh[i][r]);
            hd[i][r][0] = (uint32_t)ld2(wb + 192 + 8 * hh + 2 * p) |
                          ((uint32_t)ld2(wb + 196 + 8 * hh + 2 * p) << 16);
            hd[i][r][1] = ld2(wb + 208);
          }
        }
      }
    }
  };
  // ---- 2. arithmetic, block by block
  auto compute_round = [&](int s0) {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int b = s0 + bl0 + 16 * i;
      if (b >= nb) break;
      if constexpr (BF == 12 || BF == 13) {
        // scales and mins of sub-blocks 2c and 2c+1 as byte pairs (q5_K: the
        // same header; its quants add the high bits 2c and 2c+1 as bit 4)
        int sc0[R], sc1[R];
        uint32_t m0[R], m1[R], lo[R][8], hi[R][8];
        float d[R], dmin[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint32_t h1 = hd[i][r][1], h2 = hd[i][r][2], h3 = hd[i][r][3];
          const int s = 16 * (c & 1);
          uint32_t scp, mnp;
          if (c < 2) {
            scp = (h1 >> s) & 0x3f3fu;
            mnp = (h2 >> s) & 0x3f3fu;
          } else {
            scp = ((h3 >> s) & 0x0f0fu) | ((h1 >> (s + 2)) & 0x3030u);
            mnp = ((h3 >> (s + 4)) & 0x0f0fu) | ((h2 >> (s + 2)) & 0x3030u);
          }
          sc0[r] = (int)(scp & 0xffu);
          sc1[r] = (int)(scp >> 8);
          m0[r] = (mnp & 0xffu) * 0x10001u;
          m1[r] = (mnp >> 8) * 0x10001u;
          d[r] = f16_to_f32(hd[i][r][0]);
          dmin[r] = f16_to_f32(hd[i][r][0] >> 16);
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            lo[r][k] = lo_nib(wq[i][r][k]);
            hi[r][k] = hi_nib(wq[i][r][k]);
            if constexpr (BF == 13) {
              lo[r][k] |= ((wh[i][r][k] >> (2 * c)) & 0x01010101u) << 4;
              hi[r][k] |= ((wh[i][r][k] >> (2 * c + 1)) & 0x01010101u) << 4;
            }
          }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (!row_live<MT>(m, M)) break;  // wave-uniform: rows past M are not computed
          const XFrag x = xfrag(m < M ? m : M - 1, b);
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const int dl = dot16(lo[r] + 4, x.a1, dot16(lo[r], x.a0, 0));
            const int dh = dot16(hi[r] + 4, x.b1, dot16(hi[r], x.b0, 0));
            const int isc = __mul24(sc0[r], dl) + __mul24(sc1[r], dh);
            const int imn = dot2(x.s0, m0[r], dot2(x.s1, m1[r], 0));
            float t = d[r] * (float)isc;
            t = fmaf(-dmin[r], (float)imn, t);
            acc[r * MT + m] = fmaf(x.d, t, acc[r * MT + m]);
          }
        }
      } else if constexpr (BF == 10 || BF == 11) {
        // sub-blocks 4c + g, g = 0..3, against activation runs a0, a1, b0, b1:
        // quarter 2(c&1) + g/2 of half c/2, bytes 16(g&1)..16(g&1)+15 of it
        uint32_t qg[R][4][4];
        int sg[R][4];
        uint32_t mp0[R], mp1[R];  // q2_K: mins (4c, 4c+1), (4c+2, 4c+3) as int16 pairs
        float d[R], dmin[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int qq = 2 * (c & 1) + (g >> 1);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              uint32_t v = (wq[i][r][4 * (g & 1) + k] >> (2 * qq)) & 0x03030303u;
              if constexpr (BF == 11)  // q + 4 in 0..7: the mask bit adds 4
                v |= ((wh[i][r][4 * (g & 1) + k] >> (4 * (c >> 1) + qq)) & 0x01010101u) << 2;
              qg[r][g][k] = v;
            }
          }
          if constexpr (BF == 10) {
            const uint32_t w = hd[i][r][0];
#pragma unroll
            for (int g = 0; g < 4; ++g) sg[r][g] = (int)((w >> (8 * g)) & 15u);
            mp0[r] = ((w >> 4) & 0xfu) | ((w << 4) & 0xf0000u);
            mp1[r] = ((w >> 20) & 0xfu) | ((w >> 12) & 0xf0000u);
            d[r] = f16_to_f32(hd[i][r][1]);
            dmin[r] = f16_to_f32(hd[i][r][1] >> 16);
          } else {
            // scales 4c..4c+3: low nibbles from word c&1 (its high nibbles when
            // c >= 2), top bits 2c..2c+1 of the bytes of word 2; minus 32
            const uint32_t lo4 = (hd[i][r][c & 1] >> (4 * (c >> 1))) & 0x0f0f0f0fu;
            const uint32_t u6 = lo4 | (((hd[i][r][2] >> (2 * c)) & 0x03030303u) << 4);
#pragma unroll
            for (int g = 0; g < 4; ++g) sg[r][g] = (int)((u6 >> (8 * g)) & 63u) - 32;
            // the -4 offset against the group sums: -4 * sum_g sc_g * bsum_g
            mp0[r] = (uint32_t)(sg[r][0] & 0xffff) | ((uint32_t)sg[r][1] << 16);
            mp1[r] = (uint32_t)(sg[r][2] & 0xffff) | ((uint32_t)sg[r][3] << 16);
            d[r] = f16_to_f32(hd[i][r][3]);
            dmin[r] = 0.0f;
          }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (!row_live<MT>(m, M)) break;  // wave-uniform: rows past M are not computed
          const XFrag x = xfrag(m < M ? m : M - 1, b);
#pragma unroll
          for (int r = 0; r < R; ++r) {
            int isc = __mul24(sg[r][0], dot16(qg[r][0], x.a0, 0)) +
                      __mul24(sg[r][1], dot16(qg[r][1], x.a1, 0)) +
                      __mul24(sg[r][2], dot16(qg[r][2], x.b0, 0)) +
                      __mul24(sg[r][3], dot16(qg[r][3], x.b1, 0));
            const int isum = dot2(x.s0, mp0[r], dot2(x.s1, mp1[r], 0));
            float t;
            if constexpr (BF == 10) {
              t = d[r] * (float)isc;
              t = fmaf(-dmin[r], (float)isum, t);
            } else {
              t = d[r] * (float)(isc - 4 * isum);
            }
            acc[r * MT + m] = fmaf(x.d, t, acc[r * MT + m]);
          }
        }
      } else {
        const int p = c & 1;
        uint32_t qa[R][8], qb[R][8], spa[R], spb[R];
        int e0[R], e1[R], e2[R], e3[R];
        float d[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint32_t sp = hd[i][r][0];  // bytes 0,1: quarter p; bytes 2,3: quarter p+2
          d[r] = f16_to_f32(hd[i][r][1]);
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            qa[r][k] = q6k_quad(wq[i][r][k], wh[i][r][k], p);
            qb[r][k] = q6k_quad(wq[i][r][k], wh[i][r][k], p + 2);
          }
          e0[r] = (int)(int8_t)(sp & 0xffu);
          e1[r] = (int)(int8_t)((sp >> 8) & 0xffu);
          e2[r] = (int)(int8_t)((sp >> 16) & 0xffu);
          e3[r] = (int)(int8_t)(sp >> 24);
          spa[r] = (uint32_t)(e0[r] & 0xffff) | ((uint32_t)e1[r] << 16);
          spb[r] = (uint32_t)(e2[r] & 0xffff) | ((uint32_t)e3[r] << 16);
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (!row_live<MT>(m, M)) break;  // wave-uniform: rows past M are not computed
          const XFrag x = xfrag(m < M ? m : M - 1, b);
#pragma unroll
          for (int r = 0; r < R; ++r) {
            // sum_j sc_j * (dot_j - 32 * sum_j) over the lane's four 16-weight sub-blocks
            int isc = __mul24(e0[r], dot16(qa[r], x.a0, 0)) +
                      __mul24(e1[r], dot16(qa[r] + 4, x.a1, 0)) +
                      __mul24(e2[r], dot16(qb[r], x.b0, 0)) +
                      __mul24(e3[r], dot16(qb[r] + 4, x.b1, 0));
            isc -= 32 * dot2(x.s0, spa[r], dot2(x.s1, spb[r], 0));
            acc[r * MT + m] = fmaf(x.d, d[r] * (float)isc, acc[r * MT + m]);
          }
        }
      }
    }
  };

  if constexpr (FUSED) {
    // activation loads first, weight loads next, so quantizing waits only for
    // the former; every load is unconditional (clamped), so the wait counts
    // are exact
    // blocks quantized per wave, at most
    constexpr int QB = STAGE ? stage_qb(MT, P, NW) : fused_qb(MT, P, NW);
    const int nq = M * nb;
    const int s0 = 16 * w;
    if constexpr (!STAGE) {
      float4 xv[QB];
#pragma unroll
      for (int j = 0; j < QB; ++j) {
        int t = wv + NW * j;
        t = t < nq ? t : nq - 1;
        xv[j] = *reinterpret_cast<const float4*>(X + (int64_t)t * kQK + 4 * lane);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the two groups of loads in this order
      load_round(s0, true);
      __builtin_amdgcn_sched_barrier(0);
      // every wave quantizes QB blocks without branches (past the last block it
      // repeats it), so the blocks' reductions interleave; only real blocks are
      // stored
      Q8Lane q[QB];
#pragma unroll
      for (int j = 0; j < QB; ++j) q[j] = q8k_block(xv[j]);
#pragma unroll
      for (int j = 0; j < QB; ++j) {
        const int t = wv + NW * j;
        if (t < nq) {  // wave-uniform
          uint8_t* o = xl + t * kXL;
          *reinterpret_cast<uint32_t*>(o + 4 * lane) = q[j].packed;
          if ((lane & 7) == 0) *reinterpret_cast<uint32_t*>(o + 256 + 2 * (lane >> 2)) = q[j].sums;
          if (lane == 0) *reinterpret_cast<float*>(o + 288) = q[j].d;
          if (blockIdx.x == 0) q8k_store(Xq + (int64_t)t * kQ8KBytes, q[j], lane);
        }
      }
    } else {
      // the staged form: the q8_K blocks already at Xq, copied into the same
      // LDS layout (values, the 16 group sums, d)
      uint32_t cv[QB], cs[QB], cd[QB];
#pragma unroll
      for (int j = 0; j < QB; ++j) {
        int t = wv + NW * j;
        t = t < nq ? t : nq - 1;
        const uint8_t* xb = Xq + (int64_t)t * kQ8KBytes;
        cv[j] = ld4(xb + 4 + 4 * lane);
        cs[j] = ld4(xb + 260 + 4 * (lane & 7));
        cd[j] = ld4(xb);
      }
      __builtin_amdgcn_sched_barrier(0);
      load_round(s0, true);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < QB; ++j) {
        const int t = wv + NW * j;
        if (t < nq) {  // wave-uniform
          uint8_t* o = xl + t * kXL;
          *reinterpret_cast<uint32_t*>(o + 4 * lane) = cv[j];
          if (lane < 8) *reinterpret_cast<uint32_t*>(o + 256 + 4 * lane) = cs[j];
          if (lane == 0) *reinterpret_cast<uint32_t*>(o + 288) = cd[j];
        }
      }
    }
    __syncthreads();
    if (s0 < nb) compute_round(s0);
  } else {
    for (int s0 = 16 * IT * w; s0 < nb; s0 += 16 * IT * KS) {
      load_round(s0, false);
      compute_round(s0);
    }
  }

  // ---- 3. lane reduction and store
  const int64_t nn0 = n0 + prow;
  // SILU: the wave's finished values by (row slot prow R + r, m), then combined
  __shared__ float sv[SILU ? NW : 1][SILU ? P * R * MT : 1];
  auto put = [&](int64_t nn, int slot, int m, float v) {
    if constexpr (SILU)
      sv[wv][slot * MT + m] = v;
    else if (m < M && nn < N)
      Y[(int64_t)m * N + nn] = v;
  };
  if constexpr (KS > 1) {
    // lanes of the xor tree hold the wave's partial of value vidx; the KS
    // partials of each value are added in wave order by wave 0
    __shared__ float red[RG][KS][V];
    float v[V];
#pragma unroll
    for (int j = 0; j < V; ++j) v[j] = acc[j];
    seg_reduce<V, 64>(v, lane);
    const bool hold = holder<V, 64>(lane);
    const int j = vidx<V, 64>(lane);
    if (hold) red[rg][w][j] = v[0];
    __syncthreads();
    if (w == 0 && hold) {
      float t = red[rg][0][j];
#pragma unroll
      for (int k = 1; k < KS; ++k) t += red[rg][k][j];
      put(nn0 + j / MT, j / MT, j % MT, t);
    }
  } else if constexpr (V <= SEG) {
    float v[V];
#pragma unroll
    for (int j = 0; j < V; ++j) v[j] = acc[j];
    seg_reduce<V, SEG>(v, lane);
    if (holder<V, SEG>(lane)) {
      const int j = vidx<V, SEG>(lane);
      put(nn0 + j / MT, prow * R + j / MT, j % MT, v[0]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const float v = seg_all<SEG>(acc[j]);
      if ((lane & (SEG - 1)) == 0) put(nn0 + j / MT, prow * R + j / MT, j % MT, v);
    }
  }
  if constexpr (SILU) {
    // the slots were written by other lanes of this wave (for split rows by
    // wave 0 of the row group, which alone reads them): a wave's LDS accesses
    // complete in order, the fence keeps the compiler from reordering them
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (KS == 1 || w == 0) {
      constexpr int NO = (P * R / 2) * MT;  // (gate, up) pairs x activation rows
      static_assert(NO <= 64, "one output per lane");
      const int64_t Nout = N >> 1;
      if (lane < NO) {
        const int pr = lane / MT, m = lane % MT;
        const float g = sv[wv][(2 * pr) * MT + m], u = sv[wv][(2 * pr + 1) * MT + m];
        const int64_t n = (n0 >> 1) + pr;
        if (m < M && n < Nout) Y[(int64_t)m * Nout + n] = silu_mul_f32(g, u);
      }
    }
  }
}

// The fused form: rows of at most 16 blocks (one wave per row group, one round
// each), M <= 4 and M nb <= 32, in workgroups of kRG row groups whose waves
// quantize up to kQB blocks each.  Longer rows are not fused: every workgroup
// would quantize the whole longer activation (measured slower than the
// separate quantizer launch at K = 12288).
constexpr int kRG = 8;
constexpr int kQB = 4;

// X == nullptr: the plain form, reading the q8_K blocks at Xq.  Otherwise the
// fused form: every workgroup quantizes X into its LDS and workgroup 0 also
// writes the blocks to Xq.  SILU: grp holds the gate (0) and up (1) matrices
// of equal N and one output Y (see the kernel); their tiles cover the 2N
// interleaved rows (make_pair_tiles).
template <bool SILU>
bool group_tiles(const Group& grp, int64_t rows_per_tile, GroupTiles& gt) {
  return SILU ? make_pair_tiles(grp, rows_per_tile, gt) : make_tiles(grp, rows_per_tile, gt);
}

template <int FMT, int MT, bool SILU, int IT, int P, int KS, int R = 1>
int launch_cfg(const Group& grp, uint8_t* Xq, const float* X, int nb, int M, bool stage,
               hipStream_t st) {
  GroupTiles gt;
  // X: the fused form; stage (X null): the same workgroups staging the q8_K
  // blocks at Xq in LDS, where the shape allows it (else the plain form)
  if constexpr (IT == 1 && KS == 1 && MT <= 8) {
    constexpr int RG = kRG;
    if (X) {
      if constexpr (MT <= 4) {
        // the kernel quantizes up to fused_qb(MT, P, RG) blocks per wave
        constexpr int QB = fused_qb(MT, P, RG);
        if (M * nb > kQB * RG || M * nb > QB * RG) return -1;
        if (!group_tiles<SILU>(grp, RG * P * R, gt)) return -1;
        const uint32_t tiles = gt.start[kMaxGroup];
        if (tiles == 0) return 0;
        hipLaunchKernelGGL((gemv_kernel<FMT, MT, IT, P, KS, R, RG, true, SILU>), dim3(tiles),
                           dim3(64 * KS * RG), (size_t)M * nb * kXL, st, gt, Xq, X, nb, M);
        return 0;
      } else {
        return -1;
      }
    }
    // the staged form copies up to stage_qb(MT, P, RG) blocks per wave
    if (stage && M * nb <= stage_qb(MT, P, RG) * RG) {
      if (!group_tiles<SILU>(grp, RG * P * R, gt)) return -1;
      const uint32_t tiles = gt.start[kMaxGroup];
      if (tiles == 0) return 0;
      hipLaunchKernelGGL((gemv_kernel<FMT, MT, IT, P, KS, R, RG, true, SILU, true>), dim3(tiles),
                         dim3(64 * KS * RG), (size_t)M * nb * kXL, st, gt, Xq, X, nb, M);
      return 0;
    }
  } else {
    if (X) return -1;
  }
  if (!group_tiles<SILU>(grp, P * R, gt)) return -1;
  const uint32_t tiles = gt.start[kMaxGroup];
  if (tiles == 0) return 0;
  hipLaunchKernelGGL((gemv_kernel<FMT, MT, IT, P, KS, R, 1, false, SILU>), dim3(tiles),
                     dim3(64 * KS), 0, st, gt, Xq, (const float*)nullptr, nb, M);
  return 0;
}

// The lane mapping depends on K only: P rows side by side when a row has 16/P
// blocks; one round of 16 blocks per wave for rows of up to 16 blocks, and up
// to four waves per row beyond that (each looping over rounds for longer rows);
// two rows per wave whenever a row fills a round.
int split_waves(int nb) { return nb <= 16 ? 1 : nb <= 32 ? 2 : nb <= 48 ? 3 : nb <= 64 ? 4 : 0; }

template <int FMT, int MT, bool SILU>
int launch_mt(const Group& g, uint8_t* Xq, const float* X, int nb, int M, bool stage,
              hipStream_t st) {
  if (nb == 1) return launch_cfg<FMT, MT, SILU, 1, 16, 1>(g, Xq, X, nb, M, stage, st);
  if (nb == 2) return launch_cfg<FMT, MT, SILU, 1, 8, 1>(g, Xq, X, nb, M, stage, st);
  if (nb == 4) return launch_cfg<FMT, MT, SILU, 1, 4, 1>(g, Xq, X, nb, M, stage, st);
  if (nb == 8) return launch_cfg<FMT, MT, SILU, 1, 2, 1>(g, Xq, X, nb, M, stage, st);
  if (nb <= 16) return launch_cfg<FMT, MT, SILU, 1, 1, 1, 2>(g, Xq, X, nb, M, stage, st);
  if (nb <= 32) return launch_cfg<FMT, MT, SILU, 1, 1, 2, 2>(g, Xq, X, nb, M, stage, st);
  if (nb <= 48) return launch_cfg<FMT, MT, SILU, 1, 1, 3, 2>(g, Xq, X, nb, M, stage, st);
  if (nb <= 64) return launch_cfg<FMT, MT, SILU, 1, 1, 4, 2>(g, Xq, X, nb, M, stage, st);
  return launch_cfg<FMT, MT, SILU, 2, 1, 4, 2>(g, Xq, X, nb, M, stage, st);
}

template <int FMT, bool SILU>
int launch_fmt(const Group& g, uint8_t* Xq, const float* X, int M, int nb, bool stage,
               hipStream_t st) {
  switch (M) {
    case 1: return launch_mt<FMT, 1, SILU>(g, Xq, X, nb, M, stage, st);
    case 2: return launch_mt<FMT, 2, SILU>(g, Xq, X, nb, M, stage, st);
    case 3:
    case 4: return launch_mt<FMT, 4, SILU>(g, Xq, X, nb, M, stage, st);
    case 5:
    case 6:
    case 7:
    case 8:
      if (X) return -1;
      return launch_mt<FMT, 8, SILU>(g, Xq, X, nb, M, stage, st);
    default: return -1;
  }
}

template <bool SILU>
int launch_any(int fmt, const Group& g, uint8_t* Xq, const float* X, int M, int64_t K,
               bool stage, hipStream_t st) {
  const int64_t nb = K / kQK;
  if (nb > 0x7fffffffLL) return -1;
  switch (fmt) {
    case 10: return launch_fmt<10, SILU>(g, Xq, X, M, (int)nb, stage, st);
    case 11: return launch_fmt<11, SILU>(g, Xq, X, M, (int)nb, stage, st);
    case 12: return launch_fmt<12, SILU>(g, Xq, X, M, (int)nb, stage, st);
    case 13: return launch_fmt<13, SILU>(g, Xq, X, M, (int)nb, stage, st);
    case 14: return launch_fmt<14, SILU>(g, Xq, X, M, (int)nb, stage, st);
    case 256 + 11: return launch_fmt<256 + 11, SILU>(g, Xq, X, M, (int)nb, stage, st);
    case 256 + 14: return launch_fmt<256 + 14, SILU>(g, Xq, X, M, (int)nb, stage, st);
    default: return -1;
  }
}

}  // namespace

namespace {

// The staged form pays where the launch is large: its workgroups copy the q8_K
// blocks (a few loads) instead of reading activation fragments from L2 per
// lane (the plain form) or quantizing them again (the fused form).  Measured
// with rows x M x blocks-per-row as the size (one process, cold weights): with
// the q8_K blocks given, the staged form from 2^18 (Qwen3-8B gate/up at M = 1,
// 393216: 12.48 -> 11.49 us; the q6_K LM head 151936 x 2048 at M = 1 61.8 ->
// 43.7 us; q/k/v at M = 1, 98304, 5.11 against 5.37 us stays plain); from f32
// activations, a quantizer launch of its own and the staged form from 2^19
// (the head at M = 1 48.7 -> 46.6 us, at M = 2 68.4 -> 51.2 us, 8B gate/up at
// M = 2 19.8 -> 15.1 us; 8B gate/up at M = 1 stays fused, 12.5 against 13.2),
// and from 2^18 where each fused wave would quantize four blocks (Qwen3-1.7B
// gate/up at M = 3 / 4, 294912 / 393216: 9.2 / 9.9 -> 7.5 / 8.0 us; launches
// below 2^18 stay fused, e.g. its q+k at M = 4 5.1 against 6.8 us).
constexpr int64_t kStageWork = int64_t(1) << 18;
constexpr int64_t kSplitQuantizerWork = int64_t(1) << 19;

int64_t group_rows(const Group& g) {
  int64_t r = 0;
  for (int i = 0; i < g.count; ++i) r += g.N[i];
  return r;
}

bool stage_pays(int64_t rows, int64_t M, int64_t K) {
  return rows * M * (K / kQK) >= kStageWork;
}

}  // namespace

int launch_gemv(int fmt, const Group& g, const uint8_t* Xq, int M, int64_t K, hipStream_t st) {
  uint8_t* xq = const_cast<uint8_t*>(Xq);  // read only in the plain and staged forms
  return launch_any<false>(fmt, g, xq, nullptr, M, K, stage_pays(group_rows(g), M, K), st);
}

bool gemv_fusable(int64_t M, int64_t K) {
  const int64_t nb = K / kQK;
  if (M < 1 || M > 4 || nb < 1 || nb > 16) return false;
  return split_waves((int)nb) == 1 && M * nb <= (int64_t)kQB * kRG;
}

bool gemv_holds_activation(int64_t M, int64_t K, int64_t rows) {
  const int64_t nb = K / kQK;
  if (M < 1 || M > 4 || nb < 1 || nb > 16 || M * nb > stage_qb(4, 1, kRG) * kRG) return false;
  return stage_pays(rows, M, K);
}

bool gemv_fuse_quantizer(int64_t M, int64_t K, int64_t rows) {
  if (!gemv_fusable(M, K)) return false;
  // blocks each wave of the fused launch would quantize (the kernel the
  // launchers pick: MT rows computed, P rows side by side)
  const int64_t nb = K / kQK, work = rows * M * nb;
  const int MT = M <= 1 ? 1 : M <= 2 ? 2 : 4;
  const int P = nb == 1 ? 16 : nb == 2 ? 8 : nb == 4 ? 4 : nb == 8 ? 2 : 1;
  const int qb = fused_qb(MT, P, kRG);
  return work < kSplitQuantizerWork && !(qb >= 4 && work >= kStageWork);
}

int launch_gemv_fused(int fmt, const Group& g, const float* X, uint8_t* Xq, int M, int64_t K,
                      hipStream_t st) {
  if (!gemv_fusable(M, K)) return -1;
  return launch_any<false>(fmt, g, Xq, X, M, K, false, st);
}

int launch_gemv_silu(int fmt, const Group& g, const uint8_t* Xq, const float* X, uint8_t* Xq_out,
                     int M, int64_t K, hipStream_t st) {
  if (g.count != 2 || g.N[0] != g.N[1]) return -1;
  if (X) {
    if (!gemv_fusable(M, K)) return -1;
    return launch_any<true>(fmt, g, Xq_out, X, M, K, false, st);
  }
  return launch_any<true>(fmt, g, const_cast<uint8_t*>(Xq), nullptr, M, K,
                          stage_pays(group_rows(g), M, K), st);
}

}  // namespace gemmq
