// launch.h -- internal launchers behind the C ABI (abi.hip).  Each launcher
// assumes its arguments were validated by the ABI layer and returns 0, or -1
// when the problem does not fit the launch geometry.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gemmq {

int launch_quantize_q8K(const float* X, uint8_t* Xq, int64_t M, int64_t K, hipStream_t st);

int launch_gemv(int fmt, const uint8_t* W, const uint8_t* Xq, float* Y, int M, int64_t N,
                int64_t K, hipStream_t st);

int launch_gemm(int fmt, const uint8_t* W, const uint8_t* Xq, float* Y, int64_t M, int64_t N,
                int64_t K, hipStream_t st);

int launch_decode(int fmt, const uint8_t* W, float* Wf, int64_t N, int64_t K, hipStream_t st);

}  // namespace gemmq
