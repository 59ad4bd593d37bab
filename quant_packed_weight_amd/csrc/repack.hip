// repack.hip -- load-time repack of q3_K and q6_K matrices.
//
// Both formats have blocks whose size is not a multiple of 16 bytes (110 and
// 210), so inside a matrix their fields start on any even address and every
// kernel load of them has to read a dword-aligned span and realign it.  The
// repacked matrix holds the same bytes with each field stored for all blocks in
// block order (structure of arrays over the whole matrix, NB blocks):
//   q6_K: ql[NB][128] | qh[NB][64] | sc[NB][16] | d[NB][2]
//   q3_K: hmask[NB][32] | qs[NB][64] | scales[NB][12] | d[NB][2]
// so every field of 16 or more bytes per block starts 16-byte aligned (the
// scales of q3_K 4-byte aligned) and the kernels load them with aligned vector
// loads.  It plays the role the pages give the q4_K 8-column panels (molayo
// article "PocketLLM: 단일 가속기에서 대규모 언어 모델 실행", status row "src/ --
// C++ engine": a load-time layout for the packed kernels), with the same
// bytes per weight.
#include "device.h"
#include "launch.h"

namespace gemmq {

namespace {

// one thread per 2-byte unit of the source: every field is an even number of
// bytes at an even offset, so a unit never straddles two fields
template <int F0, int F1, int F2, int F3>
__global__ __launch_bounds__(256) void repack_kernel(const uint8_t* __restrict__ W,
                                                     uint8_t* __restrict__ out, int64_t nb) {
  constexpr int BB = F0 + F1 + F2 + F3, U = BB / 2;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= nb * U) return;
  const int64_t i = t / U;
  const int o = 2 * (int)(t - i * U);
  int64_t dst;
  if (o < F0)
    dst = i * F0 + o;
  else if (o < F0 + F1)
    dst = nb * F0 + i * F1 + (o - F0);
  else if (o < F0 + F1 + F2)
    dst = nb * (F0 + F1) + i * F2 + (o - F0 - F1);
  else
    dst = nb * (F0 + F1 + F2) + i * F3 + (o - F0 - F1 - F2);
  *reinterpret_cast<uint16_t*>(out + dst) = ld2(W + i * BB + o);
}

}  // namespace

int launch_repack(int fmt, const uint8_t* W, uint8_t* out, int64_t N, int64_t K, hipStream_t st) {
  const int64_t nb = N * (K / kQK);
  const int64_t units = nb * (fmt == 14 ? 105 : 55);
  const int64_t grid = (units + 255) / 256;
  if (grid > 0x7fffffffLL) return -1;
  if (grid == 0) return 0;
  if (fmt == 14)
    hipLaunchKernelGGL((repack_kernel<128, 64, 16, 2>), dim3((uint32_t)grid), dim3(256), 0, st, W,
                       out, nb);
  else
    hipLaunchKernelGGL((repack_kernel<32, 64, 12, 2>), dim3((uint32_t)grid), dim3(256), 0, st, W,
                       out, nb);
  return 0;
}

}  // namespace gemmq
