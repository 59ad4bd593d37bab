// gemm_common.h -- pieces the prefill GEMM kernels share (gemm.hip: the plane
// kernel for q2_K, q3_K, q5_K; gemm_q4k.hip: the q4_K kernels; gemm_q6k.hip:
// the q6_K kernel): matrix-core wrappers, the plane-byte multiply, buffer
// descriptors and direct buffer->LDS loads, the SiLU-gated output pair, and
// the four-tile kernels' activation stage and epilogue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gemmq {
namespace gk {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

constexpr int kRow = 256 + 16;  // LDS stride of one int8 K-row (padded against bank conflicts)

// bytes of w (each <= 15) times a (<= 7): per 16-bit half the product stays below
// 2^16 and no byte carries into the next.
__device__ __forceinline__ uint32_t mul_bytes(uint32_t w, uint32_t a) {
  const u16x2 v = __builtin_bit_cast(u16x2, w);
  const u16x2 s = {(unsigned short)a, (unsigned short)a};
  return __builtin_bit_cast(uint32_t, v * s);
}

// bytes of w times the factor already replicated into both 16-bit halves of f
__device__ __forceinline__ uint32_t mul_bytes2(uint32_t w, uint32_t f) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, w) * __builtin_bit_cast(u16x2, f));
}

__device__ __forceinline__ v16i mfma_i8(v4i a, v4i b, v16i c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v16f mfma_f16(v8h a, v8h b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void st16(uint8_t* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  *reinterpret_cast<uint4*>(p) = make_uint4(a, b, c, d);
}

// two int16 (packed in a dword) -> two f16 (exact: |value| <= 2048)
__device__ __forceinline__ uint32_t i16x2_to_h2(uint32_t w) {
  const h2 v = {(_Float16)(short)(w & 0xffffu), (_Float16)(short)(w >> 16)};
  return __builtin_bit_cast(uint32_t, v);
}

typedef int rsrc_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

// Raw buffer descriptor over [base, base + bytes): offsets at or past `bytes`
// read as zero.  Both arguments must be wave-uniform; the components are
// taken through readfirstlane so that the descriptor lives in scalar
// registers (the inline-asm loads below require it there, and under register
// pressure the compiler may otherwise compute it with vector instructions).
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return (rsrc_t){__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                  __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffffu)),
                  __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}

// 64 lanes x 16 bytes: lane l's 16 bytes from buffer byte voff(l) + soff (any
// 4-byte aligned source) to LDS byte lds + 16 l (lds wave-uniform, through M0).
// The s_nop covers the one wait state an M0 write needs before a load into
// LDS.  Issued from inline assembly: through the builtin the compiler treats
// such a load as an LDS write of unknown alias and drains every load before
// each LDS read, so the kernels count these loads themselves (wait_vm).
__device__ __forceinline__ void dma16(rsrc_t rs, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rs),
               "s"(soff), "{m0}"(lds)
               : "memory");
}

// 64 lanes x 4 bytes (lane l's dword to LDS byte lds + 4 l) or 16 bytes as
// dma16, taken only where the wave-uniform flag `take` is nonzero.  The branch
// is inside the asm: a branch the compiler sees splits the basic block,
// and work fenced beside the matrix instructions (sched_barrier acts within a
// block) is then sunk past it.
__device__ __forceinline__ void dma4_if(uint32_t take, rsrc_t rs, uint32_t voff, uint32_t soff,
                                        uint32_t lds) {
  const uint32_t t = __builtin_amdgcn_readfirstlane(take);
  asm volatile("s_cmp_eq_u32 %4, 0\n\ts_cbranch_scc1 1f\n\ts_nop 0\n\t"
               "buffer_load_dword %0, %1, %2 offen lds\n1:" ::"v"(voff),
               "s"(rs), "s"(soff), "{m0}"(lds), "s"(t)
               : "memory", "scc");
}

__device__ __forceinline__ void dma16_if(uint32_t take, rsrc_t rs, uint32_t voff, uint32_t soff,
                                         uint32_t lds) {
  const uint32_t t = __builtin_amdgcn_readfirstlane(take);
  asm volatile("s_cmp_eq_u32 %4, 0\n\ts_cbranch_scc1 1f\n\ts_nop 0\n\t"
               "buffer_load_dwordx4 %0, %1, %2 offen lds\n1:" ::"v"(voff),
               "s"(rs), "s"(soff), "{m0}"(lds), "s"(t)
               : "memory", "scc");
}

// a * b + c in scalar registers, computed where it is used: the kernels issue
// dozens of row loads per stage, and offsets the compiler hoisted out of the
// loop would each hold a scalar register for the whole kernel.
__device__ __forceinline__ uint32_t smad(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm volatile("s_mul_i32 %0, %1, %2\n\ts_add_u32 %0, %0, %3" : "=&s"(r) : "s"(a), "s"(b), "s"(c)
               : "scc");
  return r;
}

// s_waitcnt vmcnt(N), leaving the other counters alone.  Through the builtin,
// not inline asm: the compiler's own wait insertion then knows every vector
// load issued before this point is complete, and does not add a wait of its
// own (which would also wait for loads issued after this point) before the
// first use of a register loaded earlier.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// own LDS writes done, then the workgroup barrier; the memory clobber keeps the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// y = silu(g) * u (the same f32 steps as the GEMV's): e = exp(-g), g / (1 + e), * u
__device__ __forceinline__ float silu_mul_f32(float g, float u) {
  return g / (1.0f + expf(-g)) * u;
}

// the value of lane ^ 1 (quad permute [1,0,3,2]); every lane must be active
__device__ __forceinline__ float pair_partner(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF,
                                                            0xF, true));
}

// Lanes 2k (odd = false) and 2k+1 hold the gate and the up output of one column
// for two rows a, b.  One swap hands the even lane (gate_a, up_a) and the odd
// lane (gate_b, up_b), so each lane finishes one row of the pair.
__device__ __forceinline__ void silu_pair(float a, float b, bool odd, float& g, float& u) {
  const float got = pair_partner(odd ? a : b);  // even lanes get up_a, odd lanes gate_b
  g = odd ? got : a;
  u = odd ? b : got;
}


// ---- the four-tile kernels' activation stage (q4_K and q6_K, from 1024 rows)

// LDS map of one stage for T 32-row tiles (bytes): the int8 values, the int16
// group sums and d_x of the workgroup's 32 T activation rows
template <int T>
struct TileStage {
  static constexpr int kBM = 32 * T;                // activation rows per workgroup
  static constexpr int kBN = 128;                   // weight rows (output columns) per workgroup
  static constexpr int kOffQ = 0;                   // [kBM][kRow] int8 values
  static constexpr int kOffBs = kBM * kRow;         // [kBM][16] int16 group sums
  static constexpr int kOffDx = kOffBs + kBM * 32;  // [kBM] f32 d_x
  static constexpr int kStage = kOffDx + kBM * 4;
};

// The group sums one wave loaded into a stage (32 rows x 16 int16, its lane l
// at p + 16 l) rewritten in place as f16 (exact: |sum| <= 2032), by that wave
// between its wait for its own loads and the stage barrier: each row's sums
// are converted once per workgroup instead of once per wave that reads them.
__device__ __forceinline__ void bsums_to_f16(uint8_t* p, int lane) {
  uint4* q = reinterpret_cast<uint4*>(p + 16 * lane);
  const uint4 v = *q;
  *q = make_uint4(i16x2_to_h2(v.x), i16x2_to_h2(v.y), i16x2_to_h2(v.z), i16x2_to_h2(v.w));
}

// group sums of row `row` of the stage (converted by bsums_to_f16), groups
// 8h..8h+7
__device__ __forceinline__ v8h stage_bsums(const uint8_t* bsp, int row, int h) {
  return *reinterpret_cast<const v8h*>(bsp + row * 32 + 16 * h);
}

// The epilogue of one tile: y += d_x * (d * I - dm * C) for accumulator
// registers 4 q4 + s0 .. 4 q4 + s0 + n - 1, whose rows (8 q4 + 4h + s of the
// tile) have their d_x in one 16-byte LDS word.  q4_K: I = I_sc, C = I_min,
// dm = dmin; q6_K: I = sum sc q x, C = sum sc bsum, dm = 32 d.
template <int n>
__device__ __forceinline__ void tile_epi(const v16i& acc, const v16f& im, float4 dx, float d,
                                         float dm, float (&y)[16], int q4, int s0) {
  const float dxs[4] = {dx.x, dx.y, dx.z, dx.w};
#pragma unroll
  for (int s = s0; s < s0 + n; ++s) {
    const int r = 4 * q4 + s;
    float t = d * (float)acc[r];
    t = fmaf(-dm, im[r], t);
    y[r] = fmaf(dxs[s], t, y[r]);
  }
}

}  // namespace gk
}  // namespace gemmq
