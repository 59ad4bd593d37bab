// probe.hip -- measured ceilings for the matmul kernels: int8 MFMAs with no
// memory traffic or vector work, and the shader clock they run at; the same
// with a given amount of independent vector work beside every MFMA; and a
// plain read-only stream of device memory (the GEMV's bound).
//
// Every wave keeps kChains independent accumulator chains of
// v_mfma_i32_32x32x32_i8 on register operands, so the matrix cores never wait
// on a result; the achieved rate is the sustained dense int8 MFMA throughput of
// the GPU as it is clocked under that load, the denominator against which the
// GEMM's own rate is best read (the datasheet figure assumes the peak engine
// clock).  Wave 0 of workgroup 0 reads the shader-clock counter (s_memtime) and
// the constant 100 MHz counter (s_memrealtime) around its loop, so the host can
// derive the clock the loop ran at.
#include "launch.h"

namespace gemmq {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kChains = 4;

__global__ __launch_bounds__(256) void mfma_probe_kernel(int64_t iters, int32_t* __restrict__ out,
                                                         uint64_t* __restrict__ clk) {
  const int t = (int)threadIdx.x;
  v4i a = {t, 7 * t + 1, 13 * t + 2, 29 * t + 3};
  v4i b = {3 * t + 5, 11 * t + 7, 17 * t + 9, 23 * t + 11};
  asm volatile("" : "+v"(a), "+v"(b));  // operands the compiler cannot fold
  v16i c[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) c[k] = (v16i){0};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < kChains; ++k) c[k] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c[k], 0, 0, 0);
  }
  // the sum reads every accumulator, so it waits for the last MFMAs
  int32_t s = 0;
#pragma unroll
  for (int k = 0; k < kChains; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c[k][r];
  asm volatile("" ::"v"(s));
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  out[(int64_t)blockIdx.x * 256 + t] = s;
  if (blockIdx.x == 0 && t == 0) {
    clk[0] = t1 - t0;
    clk[1] = r1 - r0;
  }
}

// The same chains with V independent f32 FMAs after every MFMA (no operand
// comes from a matrix result), the order fixed by scheduling groups: one MFMA,
// then its V vector instructions.  The time per MFMA against V is what the
// GEMMs' budget needs: how much vector work one matrix instruction hides, and
// what a vector instruction costs past that.
template <int V>
__global__ __launch_bounds__(256) void mfma_valu_probe_kernel(int64_t iters,
                                                              int32_t* __restrict__ out,
                                                              uint64_t* __restrict__ clk) {
  const int t = (int)threadIdx.x;
  v4i a = {t, 7 * t + 1, 13 * t + 2, 29 * t + 3};
  v4i b = {3 * t + 5, 11 * t + 7, 17 * t + 9, 23 * t + 11};
  asm volatile("" : "+v"(a), "+v"(b));
  v16i c[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) c[k] = (v16i){0};
  float f[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    f[r] = (float)(t + r);
    asm volatile("" : "+v"(f[r]));
  }
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < kChains; ++k) {
      c[k] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c[k], 0, 0, 0);
#pragma unroll
      for (int v = 0; v < V; ++v) {
        float& x = f[(k * V + v) & 15];
        x = fmaf(x, 1.0000001f, 0.5f);
      }
    }
#pragma unroll
    for (int k = 0; k < kChains; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      if (V > 0) __builtin_amdgcn_sched_group_barrier(0x002, V, 0);  // then V VALU
    }
  }
  int32_t s = 0;
#pragma unroll
  for (int k = 0; k < kChains; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c[k][r];
#pragma unroll
  for (int r = 0; r < 16; ++r) asm volatile("" ::"v"(f[r]));  // the vector work stays live
  asm volatile("" ::"v"(s));
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  out[(int64_t)blockIdx.x * 256 + t] = s;
  if (blockIdx.x == 0 && t == 0) {
    clk[0] = t1 - t0;
    clk[1] = r1 - r0;
  }
}

// Read-only stream: 2048 waves (256 workgroups of eight), each reading one
// contiguous span of the buffer (a multiple of 8 KiB, the last one shorter) as
// a matmul wave reads its weight rows: every load instruction covers 1 KiB,
// eight of them are issued before any is used (loads past the span's end are
// switched off, so a buffer smaller than a round is still read in one).  Every
// wave stores the XOR of what it read, so no load can be dropped.  The time of
// the launch gives the sustained read rate of device memory with nothing else
// in the way, and on a buffer the size of one matmul's weights, the time a
// plain stream of those bytes takes.
constexpr int kReadWaves = 2048;
constexpr int kReadUnroll = 8;

__global__ __launch_bounds__(512) void read_probe_kernel(const uint4* __restrict__ src,
                                                         int64_t nvec, uint32_t* __restrict__ out) {
  constexpr int64_t kRound = 64 * kReadUnroll;  // 16-byte vectors per wave and round
  const int lane = (int)(threadIdx.x & 63);
  const int64_t wid = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t nw = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t span = ((nvec + nw - 1) / nw + kRound - 1) / kRound * kRound;
  const int64_t lo = wid * span, hi = lo + span < nvec ? lo + span : nvec;
  uint32_t a = 0;
  for (int64_t i = lo + lane; i < hi; i += kRound) {
    uint4 v[kReadUnroll];
#pragma unroll
    for (int k = 0; k < kReadUnroll; ++k)
      v[k] = i + 64 * k < hi ? src[i + 64 * k] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int k = 0; k < kReadUnroll; ++k) a ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  // fold the wave (xor over the lanes) and store one word per wave
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) a ^= (uint32_t)__shfl_xor((int)a, m, 64);
  if (lane == 0) out[wid] = a;
}

}  // namespace

int probe_mfma_chains() { return kChains; }

int probe_read_waves() { return kReadWaves; }

int launch_probe_read(const void* src, int64_t bytes, uint32_t* out, hipStream_t st) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(kReadWaves / 8), dim3(512), 0, st,
                     static_cast<const uint4*>(src), bytes / 16, out);
  return 0;
}

int launch_probe_mfma_valu(int64_t iters, int64_t blocks, int valu, int32_t* out, uint64_t* clk,
                           hipStream_t st) {
  const dim3 g((uint32_t)blocks), b(256);
  switch (valu) {
    case 0: hipLaunchKernelGGL(mfma_valu_probe_kernel<0>, g, b, 0, st, iters, out, clk); break;
    case 4: hipLaunchKernelGGL(mfma_valu_probe_kernel<4>, g, b, 0, st, iters, out, clk); break;
    case 8: hipLaunchKernelGGL(mfma_valu_probe_kernel<8>, g, b, 0, st, iters, out, clk); break;
    case 12: hipLaunchKernelGGL(mfma_valu_probe_kernel<12>, g, b, 0, st, iters, out, clk); break;
    case 16: hipLaunchKernelGGL(mfma_valu_probe_kernel<16>, g, b, 0, st, iters, out, clk); break;
    default: return -1;
  }
  return 0;
}

int launch_probe_mfma(int64_t iters, int64_t blocks, int32_t* out, uint64_t* clk,
                      hipStream_t st) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((uint32_t)blocks), dim3(256), 0, st, iters, out,
                     clk);
  return 0;
}

}  // namespace gemmq
