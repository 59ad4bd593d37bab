// launch.h -- internal launchers behind the C ABI (abi.hip).  Each launcher
// assumes its arguments were validated by the ABI layer and returns 0, -1 when
// the problem does not fit the launch geometry, or -2 when the runtime refused
// a per-device kernel attribute the launch needs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gemmq {

// Up to kMaxGroup weight matrices of one format that read the same activations
// and run as one launch: matrix g has N[g] rows at W[g] and writes Y[g].
constexpr int kMaxGroup = 4;
struct Group {
  const uint8_t* W[kMaxGroup];
  float* Y[kMaxGroup];
  int64_t N[kMaxGroup];
  int count;
};

// Kernel-side view: the launch's first grid dimension is the concatenation of
// every matrix's tiles; tile t belongs to matrix g with start[g] <= t < start[g+1].
struct GroupTiles {
  const uint8_t* W[kMaxGroup];
  float* Y[kMaxGroup];
  int64_t N[kMaxGroup];
  uint32_t start[kMaxGroup + 1];
  int count;
};

// Fills `t` from `g` with ceil(N/rows_per_tile) tiles per matrix; false when the
// total does not fit a grid dimension.
inline bool make_tiles(const Group& g, int64_t rows_per_tile, GroupTiles& t) {
  int64_t s = 0;
  t.count = g.count;
  for (int i = 0; i < kMaxGroup; ++i) {
    const bool on = i < g.count;
    t.W[i] = on ? g.W[i] : nullptr;
    t.Y[i] = on ? g.Y[i] : nullptr;
    t.N[i] = on ? g.N[i] : 0;
    t.start[i] = (uint32_t)s;
    if (on) s += (g.N[i] + rows_per_tile - 1) / rows_per_tile;
    if (s > 0x7fffffffLL) return false;
  }
  t.start[kMaxGroup] = (uint32_t)s;
  return true;
}

// The SiLU-gated pair (gate g.W[0], up g.W[1], equal N, one output g.Y[0]) as one
// virtual matrix of 2N rows whose row 2n is gate row n and row 2n+1 up row n;
// the up pointer rides in t.W[1].
inline bool make_pair_tiles(const Group& g, int64_t rows_per_tile, GroupTiles& t) {
  Group v{};
  v.count = 1;
  v.W[0] = g.W[0];
  v.Y[0] = g.Y[0];
  v.N[0] = 2 * g.N[0];
  if (!make_tiles(v, rows_per_tile, t)) return false;
  t.W[1] = g.W[1];
  return true;
}
// The matrix that tile `tile` (wave-uniform) belongs to: its weights, output,
// rows, and the tile's index within it.  Every field is read at a fixed offset
// and chosen by selects, so the kernel arguments arrive in one round of scalar
// loads instead of a second, dependent one.
struct TileMatrix {
  const uint8_t* W;
  float* Y;
  int64_t N;
  uint32_t local;
};

__device__ __forceinline__ TileMatrix tile_matrix(const GroupTiles& t, uint32_t tile) {
  TileMatrix m{t.W[0], t.Y[0], t.N[0], tile};
#pragma unroll
  for (int i = 1; i < kMaxGroup; ++i) {
    const bool in = i < t.count && tile >= t.start[i];
    m.W = in ? t.W[i] : m.W;
    m.Y = in ? t.Y[i] : m.Y;
    m.N = in ? t.N[i] : m.N;
    m.local = in ? tile - t.start[i] : m.local;
  }
  return m;
}

int launch_quantize_q8K(const float* X, uint8_t* Xq, int64_t M, int64_t K, hipStream_t st);

// skinny_q6k.hip: the small-M q6_K MFMA kernel (q6_K and its repacked layout,
// M <= 16); 0, or -1 when the arguments do not fit it
int launch_skinny_q6k(int fmt, const Group& g, const uint8_t* Xq, int M, int64_t K,
                      hipStream_t st);
int launch_skinny_q6k_silu(int fmt, const Group& g, const uint8_t* Xq, int M, int64_t K,
                           hipStream_t st);

// The GEMV on q8_K blocks at Xq: the plain form, or the staged one on large
// launches (see gemv.hip).
int launch_gemv(int fmt, const Group& g, const uint8_t* Xq, int M, int64_t K, hipStream_t st);

int launch_gemm(int fmt, const Group& g, const uint8_t* Xq, int64_t M, int64_t K, hipStream_t st);
// Checked before anything is enqueued, so that a call is refused whole:
// whether M rows of K fit the GEMM's grid (a pure function of its arguments),
// and the per-device set-up of its kernels (raising their dynamic LDS limit:
// 0, or -2 when the runtime refuses).
bool gemm_fits(int fmt, int64_t M, int64_t K);
int prepare_gemm(bool silu);
// gemm_q4k.hip: the q4_K GEMM over the 128-row weight tiles of `gt` (its LDS
// limits raised once per device by q4k_prepare; 0 or -1 as the launchers).
bool q4k_prepare(bool silu);
int launch_gemm_q4k(const GroupTiles& gt, bool silu, const uint8_t* Xq, int64_t M, int64_t K,
                    hipStream_t st);
// gemm_q6k.hip: the q6_K GEMM (fmt 14 or its repacked layout) over the
// 128-row weight tiles of `gt`, limits raised once per device by q6k_prepare
bool q6k_prepare(bool silu);
int launch_gemm_q6k(const GroupTiles& gt, int fmt, bool silu, const uint8_t* Xq, int64_t M,
                    int64_t K, hipStream_t st);
// The fused decode form: quantize X (M x K f32) and run the GEMV in one launch,
// each workgroup quantizing into its own LDS; Xq receives the q8_K blocks.
// Taken when gemv_fusable(M, K): M <= 4 and M K / 256 small enough (see gemv.hip).
bool gemv_fusable(int64_t M, int64_t K);
// gemv_fusable and few enough rows (all matrices of the call) that quantizing in
// every workgroup costs less than a quantizer launch of its own.
bool gemv_fuse_quantizer(int64_t M, int64_t K, int64_t rows);
// M <= 4, rows of at most 16 blocks, and a launch large enough (rows: all
// matrices of the call) that the GEMV stages the activation in LDS.
bool gemv_holds_activation(int64_t M, int64_t K, int64_t rows);
int launch_gemv_fused(int fmt, const Group& g, const float* X, uint8_t* Xq, int M, int64_t K,
                      hipStream_t st);
// SiLU-gated product of a gate and an up matrix (g.W[0], g.W[1], equal N, output
// g.Y[0] of N columns): y = silu(gate x) * (up x).  X == nullptr reads Xq; else
// the fused form quantizes X (gemv_fusable) and writes Xq_out.
int launch_gemv_silu(int fmt, const Group& g, const uint8_t* Xq, const float* X, uint8_t* Xq_out,
                     int M, int64_t K, hipStream_t st);
int launch_gemm_silu(int fmt, const Group& g, const uint8_t* Xq, int64_t M, int64_t K,
                     hipStream_t st);

int launch_decode(int fmt, const uint8_t* W, float* Wf, int64_t N, int64_t K, hipStream_t st);
// q3_K (11) / q6_K (14) matrix -> its repacked layout (same size)
int launch_repack(int fmt, const uint8_t* W, uint8_t* out, int64_t N, int64_t K, hipStream_t st);

}  // namespace gemmq
