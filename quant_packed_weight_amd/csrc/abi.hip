// abi.hip -- the C ABI of libgemmq (declared in include/gemmq.h).
//
// Every entry point validates its arguments before touching the device, so a
// bad call returns a named status and launches nothing (the pages refuse what
// they do not implement by name rather than guessing -- PocketLLM README,
// "Roadmap" and "Try it").  The library owns no memory and keeps no per-call
// state; the only process-wide state is per device: the architecture check
// and whether the GEMM kernels' LDS limit has been raised.
#include <atomic>
#include <cstring>

#include "gemmq.h"
#include "launch.h"

namespace gemmq {
// probe.hip: the int8 MFMA ceiling (independent accumulator chains per wave)
int probe_mfma_chains();
int launch_probe_mfma(int64_t iters, int64_t blocks, int32_t* out, uint64_t* clk, hipStream_t st);
// the same with `valu` (0, 4, 8, 12 or 16) f32 FMAs after every MFMA; -1 otherwise
int launch_probe_mfma_valu(int64_t iters, int64_t blocks, int valu, int32_t* out, uint64_t* clk,
                           hipStream_t st);
int probe_read_waves();
int launch_probe_read(const void* src, int64_t bytes, uint32_t* out, hipStream_t st);
// skinny.hip / skinny_q6k.hip: the small-M MFMA kernels (q4_K; q6_K and its
// repacked layout)
int launch_skinny(int fmt, const Group& g, const uint8_t* Xq, int M, int64_t K, hipStream_t st);
int launch_skinny_silu(int fmt, const Group& g, const uint8_t* Xq, int M, int64_t K,
                       hipStream_t st);
}  // namespace gemmq

namespace {

constexpr int kMaxDevices = 64;
// activation rows the small-M MFMA kernels take: q4_K up to 64, q6_K up to 16
// (automatic choice: from 3)
constexpr int64_t kSkinnyMinM = 3, kSkinnyMaxM = 64, kSkinnyQ6MaxM = 16;
// automatic choice past one 16-row tile: the small-M kernel while the launch's
// output columns times its 16-row tiles stay within this bound
constexpr int64_t kSkinnyColTiles = 20480;
// q6_K (either layout): the automatic choice takes the small-M kernel at
// 9 <= M <= 16, and at 3 <= M <= 8 from this many output columns (below them
// its 32-column workgroups are too few to fill the chip and the GEMV is faster:
// measured on the Qwen3-1.7B shapes, v 1024 and down 2048 columns against the
// 151936-column head) -- except at M <= 4 where the GEMV holds the activation in
// LDS (M K/256 <= 32; the head at M = 3 / 4: 58.3 / 59.2 us against 85.9 / 86.0).
// Plain q6_K on rows of more than 8 super-blocks, where the kernel stages its
// weight blocks in LDS, also from columns x super-blocks = kSkinnyQ6Work at
// M = 5..8 (where the GEMV runs its 8-row form): at M = 8 4096 x 4096 12.4
// against 14.8 us, Qwen3-8B down 4096 x 12288 27.7 against 34.3, 8192 x 4096
// 14.7 against 27.2; below it the GEMV stays ahead (1024 x 4096 10.4 against
// 10.8, 2048 x 6144 13.7 against 15.7).  At M = 3, 4 the same holds only on rows
// of more than 64 super-blocks (the GEMV's two-round form) from kSkinnyQ6LongWork:
// 5120 x 17408 37.4 against 60.7 us, 4096 x 20480 40.7 against 49.5, while
// 2048 x 17408 (139264) stays on the GEMV, 25.7 against 34.8.
constexpr int64_t kSkinnyQ6Cols = 16384;
constexpr int64_t kSkinnyQ6Work = int64_t(1) << 16;
constexpr int64_t kSkinnyQ6LongWork = int64_t(1) << 18;
std::atomic<int> g_arch_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

// the largest M the small-M kernel takes in this format (0: not available)
int64_t skinny_max_m(int fmt) {
  if (fmt == GEMMQ_Q4_K) return kSkinnyMaxM;
  if (fmt == GEMMQ_Q6_K || fmt == GEMMQ_Q6_K_R) return kSkinnyQ6MaxM;
  return 0;
}

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GEMMQ_E_DEVICE;
  if (dev >= kMaxDevices) return GEMMQ_E_DEVICE;
  int state = g_arch_ok[dev].load(std::memory_order_acquire);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GEMMQ_E_DEVICE;
    state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_ok[dev].store(state, std::memory_order_release);
  }
  return state == 1 ? GEMMQ_OK : GEMMQ_E_DEVICE;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int fmt_bytes(int fmt) {
  switch (fmt) {
    case GEMMQ_Q2_K: return GEMMQ_Q2_K_BYTES;
    case GEMMQ_Q3_K: return GEMMQ_Q3_K_BYTES;
    case GEMMQ_Q4_K: return GEMMQ_Q4_K_BYTES;
    case GEMMQ_Q5_K: return GEMMQ_Q5_K_BYTES;
    case GEMMQ_Q6_K: return GEMMQ_Q6_K_BYTES;
    case GEMMQ_Q3_K_R: return GEMMQ_Q3_K_BYTES;
    case GEMMQ_Q6_K_R: return GEMMQ_Q6_K_BYTES;
    default: return 0;
  }
}

// Weight base alignment: blocks of 144 and 176 bytes keep every block 16-byte
// aligned, and so do the repacked layouts' field arrays (the kernels load them
// with aligned 16-byte loads); the others only need dword alignment of the base.
uintptr_t fmt_align(int fmt) {
  return fmt == GEMMQ_Q4_K || fmt == GEMMQ_Q5_K || fmt == GEMMQ_Q3_K_R || fmt == GEMMQ_Q6_K_R ? 16
                                                                                                 : 4;
}

// Launcher outcome: -1 means the shape does not fit the kernel's launch
// geometry, -2 that the runtime refused a per-device kernel attribute; the
// callers check both before enqueuing anything (shape_matmul, prepare_matmul),
// so here they only guard the launchers' own checks.  The thread's pending HIP error is
// cleared just before each launch (see clear_pending), so an error read here
// belongs to our launch.
int launched(int rc) {
  if (rc == -1) return GEMMQ_E_SHAPE;
  if (rc != 0) return GEMMQ_E_LAUNCH;
  return hipGetLastError() == hipSuccess ? GEMMQ_OK : GEMMQ_E_LAUNCH;
}

void clear_pending() { (void)hipGetLastError(); }

// Bounds that keep every byte offset below 2^62 and every grid dimension legal.
constexpr int64_t kMaxK = (int64_t)1 << 24;
constexpr int64_t kMaxRows = (int64_t)1 << 31;

int check_weights(int fmt, const void* W, int64_t N, int64_t K) {
  if (fmt_bytes(fmt) == 0) return GEMMQ_E_UNSUPPORTED_FORMAT;
  if (N < 0) return GEMMQ_E_INVALID_ARG;
  if (K <= 0 || K % GEMMQ_QK != 0 || K > kMaxK || N > kMaxRows) return GEMMQ_E_SHAPE;
  if (N > 0 && !W) return GEMMQ_E_INVALID_ARG;
  if (W && !aligned(W, fmt_align(fmt))) return GEMMQ_E_ALIGNMENT;
  return GEMMQ_OK;
}

}  // namespace

extern "C" {

int gemmq_abi_version(void) { return GEMMQ_ABI_VERSION; }

const char* gemmq_status_str(int status) {
  switch (status) {
    case GEMMQ_OK: return "GEMMQ_OK";
    case GEMMQ_E_INVALID_ARG: return "GEMMQ_E_INVALID_ARG: null pointer, negative size or bad path";
    case GEMMQ_E_UNSUPPORTED_FORMAT:
      return "GEMMQ_E_UNSUPPORTED_FORMAT: the weight format must be q2_K (10), q3_K (11), q4_K "
             "(12), q5_K (13), q6_K (14) or a repacked q3_K / q6_K (267, 270; gemmq_decode and "
             "gemmq_repack take the plain ones only); the small-M path takes q4_K, q6_K and q6_K_R";
    case GEMMQ_E_SHAPE:
      return "GEMMQ_E_SHAPE: K must be a positive multiple of 256 up to 2^24, rows up to 2^31; "
             "the GEMV path takes M <= 8, the small-M path M <= 64 (q6_K: 16), the GEMM path M <= "
             "4194240";
    case GEMMQ_E_ALIGNMENT: return "GEMMQ_E_ALIGNMENT: a pointer breaks the documented alignment";
    case GEMMQ_E_DEVICE: return "GEMMQ_E_DEVICE: the current HIP device is not a gfx950";
    case GEMMQ_E_LAUNCH: return "GEMMQ_E_LAUNCH: the HIP runtime rejected a kernel launch";
    default: return "GEMMQ_E_UNKNOWN: not a libgemmq status";
  }
}

size_t gemmq_block_bytes(int fmt) { return (size_t)fmt_bytes(fmt); }

size_t gemmq_weight_bytes(int fmt, int64_t N, int64_t K) {
  const int bb = fmt_bytes(fmt);
  if (!bb || N < 0 || K < 0 || K % GEMMQ_QK != 0 || K > kMaxK || N > kMaxRows) return 0;
  return (size_t)N * (size_t)(K / GEMMQ_QK) * (size_t)bb;
}

size_t gemmq_q8K_bytes(int64_t M, int64_t K) {
  if (M < 0 || K < 0 || K % GEMMQ_QK != 0 || K > kMaxK || M > kMaxRows) return 0;
  return (size_t)M * (size_t)(K / GEMMQ_QK) * GEMMQ_Q8_K_BYTES;
}

int gemmq_quantize_q8K(const float* X, void* Xq, int64_t M, int64_t K, void* stream) {
  if (M < 0) return GEMMQ_E_INVALID_ARG;
  if (K <= 0 || K % GEMMQ_QK != 0 || K > kMaxK || M > kMaxRows) return GEMMQ_E_SHAPE;
  if (M == 0) return GEMMQ_OK;
  if (!X || !Xq) return GEMMQ_E_INVALID_ARG;
  if (!aligned(X, 16) || !aligned(Xq, 4)) return GEMMQ_E_ALIGNMENT;
  const int dv = check_device();
  if (dv != GEMMQ_OK) return dv;
  clear_pending();
  return launched(gemmq::launch_quantize_q8K(X, static_cast<uint8_t*>(Xq), M, K,
                                             static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Validation shared by the group entry points: fills `g` with the non-empty
// matrices in order and `rows` with their total; GEMMQ_OK or the error.
int check_group(int fmt, int count, const void* const* W, float* const* Y, const int64_t* N,
                int64_t M, int64_t K, int path, gemmq::Group& g, int64_t& rows) {
  if (count < 1 || count > gemmq::kMaxGroup || !W || !Y || !N) return GEMMQ_E_INVALID_ARG;
  g = gemmq::Group{};
  rows = 0;
  for (int i = 0; i < count; ++i) {
    const int rc = check_weights(fmt, W[i], N[i], K);
    if (rc != GEMMQ_OK) return rc;
    rows += N[i];
  }
  if (M < 0) return GEMMQ_E_INVALID_ARG;
  if (M > kMaxRows || rows > kMaxRows) return GEMMQ_E_SHAPE;
  if (path != GEMMQ_PATH_AUTO && path != GEMMQ_PATH_GEMV && path != GEMMQ_PATH_GEMM &&
      path != GEMMQ_PATH_SKINNY)
    return GEMMQ_E_INVALID_ARG;
  if (path == GEMMQ_PATH_GEMV && M > 8) return GEMMQ_E_SHAPE;
  if (path == GEMMQ_PATH_SKINNY && skinny_max_m(fmt) == 0) return GEMMQ_E_UNSUPPORTED_FORMAT;
  if (path == GEMMQ_PATH_SKINNY && M > skinny_max_m(fmt)) return GEMMQ_E_SHAPE;
  if (M == 0 || rows == 0) return GEMMQ_OK;
  for (int i = 0; i < count; ++i)
    if (N[i] > 0 && !Y[i]) return GEMMQ_E_INVALID_ARG;
  for (int i = 0; i < count; ++i)
    if (N[i] > 0 && !aligned(Y[i], 4)) return GEMMQ_E_ALIGNMENT;
  // empty matrices are dropped; the others keep their order
  for (int i = 0; i < count; ++i) {
    if (N[i] == 0) continue;
    g.W[g.count] = static_cast<const uint8_t*>(W[i]);
    g.Y[g.count] = Y[i];
    g.N[g.count] = N[i];
    ++g.count;
  }
  return GEMMQ_OK;
}

// The kernel family a launch of M activation rows and `cols` output columns (all
// matrices of the launch together) runs on.  The automatic choice follows the
// measured crossovers on the Qwen3-8B layer: the decode GEMV up to M = 8 (q4_K: up
// to M = 2); for q4_K at 3 <= M <= 64 the small-M MFMA kernel, always for one
// 16-row tile and for t > 1 tiles while cols * t <= kSkinnyColTiles (its time grows
// with cols * t, while the GEMM at these M runs one 64-row tile per column tile
// and costs about the same at any cols below a chip's worth of workgroups); the
// GEMM beyond -- except q4_K at M = 3, 4 on launches where the GEMV holds the
// activation in LDS (Qwen3-8B q/k/v at M = 3 9.8 against 11.0 us, gate/up 18.8
// against 21.8; down, 48 blocks a row, stays: 18.5 against 13.5).  q6_K (either
// layout) takes its small-M kernel at 9 <= M <= 16,
// and at 3 <= M <= 8 once the launch has kSkinnyQ6Cols columns, unless the GEMV
// can hold the activation in LDS (gemv_fusable); plain q6_K at 5 <= M <= 8 on
// rows of more than 8 super-blocks also from kSkinnyQ6Work columns x blocks, and
// at M = 3, 4 on rows of more than 64 from kSkinnyQ6LongWork.
int pick_path(int fmt, int path, int64_t M, int64_t K, int64_t cols) {
  if (path != GEMMQ_PATH_AUTO) return path;
  if (fmt == GEMMQ_Q4_K && M <= 4 && gemmq::gemv_holds_activation(M, K, cols))
    return GEMMQ_PATH_GEMV;
  if (fmt == GEMMQ_Q4_K && M >= kSkinnyMinM && M <= kSkinnyMaxM) {
    const int64_t t = (M + 15) / 16;
    if (t == 1 || cols * t <= kSkinnyColTiles) return GEMMQ_PATH_SKINNY;
  }
  if ((fmt == GEMMQ_Q6_K || fmt == GEMMQ_Q6_K_R) && M >= kSkinnyMinM && M <= kSkinnyQ6MaxM &&
      (M > 8 || (cols >= kSkinnyQ6Cols && !gemmq::gemv_fusable(M, K))))
    return GEMMQ_PATH_SKINNY;
  const int64_t nb = K / 256;
  if (fmt == GEMMQ_Q6_K && M >= 5 && M <= 8 && nb > 8 && cols * nb >= kSkinnyQ6Work)
    return GEMMQ_PATH_SKINNY;
  if (fmt == GEMMQ_Q6_K && M >= 3 && M <= 4 && nb > 64 && cols * nb >= kSkinnyQ6LongWork)
    return GEMMQ_PATH_SKINNY;
  return M <= 8 ? GEMMQ_PATH_GEMV : GEMMQ_PATH_GEMM;
}

// What a matmul launch on `path` could refuse is checked before anything is
// enqueued, so a group or linear call never leaves the quantizer's output
// written and then refuses its matmul.  Only the GEMM has limits of its own:
// its grid's M-tiles (a shape check, made with the argument checks) and the
// per-device dynamic LDS limit of its kernels (made once the device is known).
int shape_matmul(int fmt, int path, int64_t M, int64_t K) {
  return path != GEMMQ_PATH_GEMM || gemmq::gemm_fits(fmt, M, K) ? GEMMQ_OK : GEMMQ_E_SHAPE;
}

int prepare_matmul(int path, bool silu) {
  return path != GEMMQ_PATH_GEMM || gemmq::prepare_gemm(silu) == 0 ? GEMMQ_OK : GEMMQ_E_LAUNCH;
}

int launch_matmul(int fmt, int path, const gemmq::Group& g, const uint8_t* xq, int64_t M,
                  int64_t K, hipStream_t st) {
  if (path == GEMMQ_PATH_GEMV) return gemmq::launch_gemv(fmt, g, xq, (int)M, K, st);
  if (path == GEMMQ_PATH_SKINNY) return gemmq::launch_skinny(fmt, g, xq, (int)M, K, st);
  return gemmq::launch_gemm(fmt, g, xq, M, K, st);
}

}  // namespace

extern "C" {

int gemmq_gemm_group(int fmt, int count, const void* const* W, float* const* Y,
                     const int64_t* N, const void* Xq, int64_t M, int64_t K, int path,
                     void* stream) {
  gemmq::Group g;
  int64_t rows = 0;
  int rc = check_group(fmt, count, W, Y, N, M, K, path, g, rows);
  if (rc != GEMMQ_OK || M == 0 || rows == 0) return rc;
  if (!Xq) return GEMMQ_E_INVALID_ARG;
  if (!aligned(Xq, 4)) return GEMMQ_E_ALIGNMENT;
  const int p = pick_path(fmt, path, M, K, rows);
  rc = shape_matmul(fmt, p, M, K);
  if (rc != GEMMQ_OK) return rc;
  const int dv = check_device();
  if (dv != GEMMQ_OK) return dv;
  rc = prepare_matmul(p, false);
  if (rc != GEMMQ_OK) return rc;
  const uint8_t* xq = static_cast<const uint8_t*>(Xq);
  hipStream_t st = static_cast<hipStream_t>(stream);
  clear_pending();
  return launched(launch_matmul(fmt, p, g, xq, M, K, st));
}

int gemmq_linear_group(int fmt, int count, const void* const* W, float* const* Y,
                       const int64_t* N, const float* X, void* Xq, int64_t M, int64_t K,
                       int path, void* stream) {
  gemmq::Group g;
  int64_t rows = 0;
  int rc = check_group(fmt, count, W, Y, N, M, K, path, g, rows);
  if (rc != GEMMQ_OK || M == 0) return rc;
  if (!X || !Xq) return GEMMQ_E_INVALID_ARG;
  if (!aligned(X, 16) || !aligned(Xq, 4)) return GEMMQ_E_ALIGNMENT;
  const int p = pick_path(fmt, path, M, K, rows);
  if (rows > 0 && (rc = shape_matmul(fmt, p, M, K)) != GEMMQ_OK) return rc;
  const int dv = check_device();
  if (dv != GEMMQ_OK) return dv;
  if (rows > 0 && (rc = prepare_matmul(p, false)) != GEMMQ_OK) return rc;
  uint8_t* xq = static_cast<uint8_t*>(Xq);
  hipStream_t st = static_cast<hipStream_t>(stream);
  clear_pending();
  if (rows > 0 && p == GEMMQ_PATH_GEMV && gemmq::gemv_fuse_quantizer(M, K, rows))
    return launched(gemmq::launch_gemv_fused(fmt, g, X, xq, (int)M, K, st));
  rc = launched(gemmq::launch_quantize_q8K(X, xq, M, K, st));
  if (rc != GEMMQ_OK || rows == 0) return rc;
  return launched(launch_matmul(fmt, p, g, xq, M, K, st));
}

int gemmq_linear_silu_mul(int fmt, const void* Wg, const void* Wu, const float* X, void* Xq,
                          float* Y, int64_t M, int64_t N, int64_t K, int path, void* stream) {
  int rc = check_weights(fmt, Wg, N, K);
  if (rc == GEMMQ_OK) rc = check_weights(fmt, Wu, N, K);
  if (rc != GEMMQ_OK) return rc;
  if (M < 0) return GEMMQ_E_INVALID_ARG;
  if (M > kMaxRows || 2 * N > kMaxRows) return GEMMQ_E_SHAPE;
  if (path != GEMMQ_PATH_AUTO && path != GEMMQ_PATH_GEMV && path != GEMMQ_PATH_GEMM &&
      path != GEMMQ_PATH_SKINNY)
    return GEMMQ_E_INVALID_ARG;
  if (path == GEMMQ_PATH_GEMV && M > 8) return GEMMQ_E_SHAPE;
  if (path == GEMMQ_PATH_SKINNY && skinny_max_m(fmt) == 0) return GEMMQ_E_UNSUPPORTED_FORMAT;
  if (path == GEMMQ_PATH_SKINNY && M > skinny_max_m(fmt)) return GEMMQ_E_SHAPE;
  if (M == 0) return GEMMQ_OK;
  if (!X || !Xq || (N > 0 && !Y)) return GEMMQ_E_INVALID_ARG;
  if (!aligned(X, 16) || !aligned(Xq, 4) || (N > 0 && !aligned(Y, 4))) return GEMMQ_E_ALIGNMENT;
  const int p = pick_path(fmt, path, M, K, 2 * N);  // as gemmq_linear_group on {Wg, Wu}
  if (N > 0 && (rc = shape_matmul(fmt, p, M, K)) != GEMMQ_OK) return rc;
  const int dv = check_device();
  if (dv != GEMMQ_OK) return dv;
  if (N > 0 && (rc = prepare_matmul(p, true)) != GEMMQ_OK) return rc;
  gemmq::Group g{};
  g.count = 2;
  g.W[0] = static_cast<const uint8_t*>(Wg);
  g.W[1] = static_cast<const uint8_t*>(Wu);
  g.Y[0] = g.Y[1] = Y;
  g.N[0] = g.N[1] = N;
  uint8_t* xq = static_cast<uint8_t*>(Xq);
  hipStream_t st = static_cast<hipStream_t>(stream);
  clear_pending();
  if (N > 0 && p == GEMMQ_PATH_GEMV && gemmq::gemv_fuse_quantizer(M, K, 2 * N))
    return launched(gemmq::launch_gemv_silu(fmt, g, nullptr, X, xq, (int)M, K, st));
  rc = launched(gemmq::launch_quantize_q8K(X, xq, M, K, st));
  if (rc != GEMMQ_OK || N == 0) return rc;
  if (p == GEMMQ_PATH_GEMV)
    return launched(gemmq::launch_gemv_silu(fmt, g, xq, nullptr, nullptr, (int)M, K, st));
  if (p == GEMMQ_PATH_SKINNY)
    return launched(gemmq::launch_skinny_silu(fmt, g, xq, (int)M, K, st));
  return launched(gemmq::launch_gemm_silu(fmt, g, xq, M, K, st));
}

int gemmq_linear(int fmt, const void* W, const float* X, void* Xq, float* Y, int64_t M, int64_t N,
                 int64_t K, void* stream) {
  return gemmq_linear_group(fmt, 1, &W, &Y, &N, X, Xq, M, K, GEMMQ_PATH_AUTO, stream);
}

int gemmq_gemm_ex(int fmt, const void* W, const void* Xq, float* Y, int64_t M, int64_t N,
                  int64_t K, int path, void* stream) {
  return gemmq_gemm_group(fmt, 1, &W, &Y, &N, Xq, M, K, path, stream);
}

int gemmq_gemm(int fmt, const void* W, const void* Xq, float* Y, int64_t M, int64_t N, int64_t K,
               void* stream) {
  return gemmq_gemm_ex(fmt, W, Xq, Y, M, N, K, GEMMQ_PATH_AUTO, stream);
}

int gemmq_repack(int fmt, const void* W, void* Wr, int64_t N, int64_t K, void* stream) {
  if (fmt != GEMMQ_Q3_K && fmt != GEMMQ_Q6_K) return GEMMQ_E_UNSUPPORTED_FORMAT;
  const int rc = check_weights(fmt, W, N, K);
  if (rc != GEMMQ_OK) return rc;
  if (N == 0) return GEMMQ_OK;
  if (!Wr) return GEMMQ_E_INVALID_ARG;
  if (!aligned(Wr, 16)) return GEMMQ_E_ALIGNMENT;
  const uintptr_t a = reinterpret_cast<uintptr_t>(W), b = reinterpret_cast<uintptr_t>(Wr);
  const uintptr_t bytes = (uintptr_t)gemmq_weight_bytes(fmt, N, K);
  if (a < b + bytes && b < a + bytes) return GEMMQ_E_INVALID_ARG;  // out of place only
  const int dv = check_device();
  if (dv != GEMMQ_OK) return dv;
  clear_pending();
  return launched(gemmq::launch_repack(fmt, static_cast<const uint8_t*>(W),
                                       static_cast<uint8_t*>(Wr), N, K,
                                       static_cast<hipStream_t>(stream)));
}

int gemmq_decode(int fmt, const void* W, float* Wf, int64_t N, int64_t K, void* stream) {
  if (fmt == GEMMQ_Q3_K_R || fmt == GEMMQ_Q6_K_R) return GEMMQ_E_UNSUPPORTED_FORMAT;
  const int rc = check_weights(fmt, W, N, K);
  if (rc != GEMMQ_OK) return rc;
  if (N == 0) return GEMMQ_OK;
  if (!Wf) return GEMMQ_E_INVALID_ARG;
  if (!aligned(Wf, 16)) return GEMMQ_E_ALIGNMENT;
  const int dv = check_device();
  if (dv != GEMMQ_OK) return dv;
  clear_pending();
  return launched(gemmq::launch_decode(fmt, static_cast<const uint8_t*>(W), Wf, N, K,
                                       static_cast<hipStream_t>(stream)));
}

int gemmq_probe_mfma_i8(int64_t iters, int64_t blocks, int32_t* out, uint64_t* clocks,
                        void* stream) {
  // the iteration cap keeps a mistaken argument from occupying the GPU for
  // long (10^6 rounds of 2048 workgroups run for about a second)
  if (!out || !clocks || iters < 1 || iters > GEMMQ_PROBE_MAX_ITERS || blocks < 1 ||
      blocks > 65535)
    return GEMMQ_E_INVALID_ARG;
  if (!aligned(out, 4) || !aligned(clocks, 8)) return GEMMQ_E_ALIGNMENT;
  if (gemmq::probe_mfma_chains() != GEMMQ_PROBE_CHAINS) return GEMMQ_E_LAUNCH;
  const int dv = check_device();
  if (dv != GEMMQ_OK) return dv;
  clear_pending();
  return launched(
      gemmq::launch_probe_mfma(iters, blocks, out, clocks, static_cast<hipStream_t>(stream)));
}

int gemmq_probe_mfma_valu(int64_t iters, int64_t blocks, int32_t valu, int32_t* out,
                          uint64_t* clocks, void* stream) {
  if (!out || !clocks || iters < 1 || iters > GEMMQ_PROBE_MAX_ITERS || blocks < 1 ||
      blocks > 65535 || valu < 0 || valu > 16 || valu % 4 != 0)
    return GEMMQ_E_INVALID_ARG;
  if (!aligned(out, 4) || !aligned(clocks, 8)) return GEMMQ_E_ALIGNMENT;
  if (gemmq::probe_mfma_chains() != GEMMQ_PROBE_CHAINS) return GEMMQ_E_LAUNCH;
  const int dv = check_device();
  if (dv != GEMMQ_OK) return dv;
  clear_pending();
  return launched(gemmq::launch_probe_mfma_valu(iters, blocks, valu, out, clocks,
                                                static_cast<hipStream_t>(stream)));
}

int gemmq_probe_read(const void* src, int64_t bytes, uint32_t* out, void* stream) {
  if (!src || !out || bytes < 16 || bytes % 16 != 0 || bytes > ((int64_t)1 << 40))
    return GEMMQ_E_INVALID_ARG;
  if (!aligned(src, 16) || !aligned(out, 4)) return GEMMQ_E_ALIGNMENT;
  if (gemmq::probe_read_waves() != GEMMQ_PROBE_READ_WORDS) return GEMMQ_E_LAUNCH;
  const int dv = check_device();
  if (dv != GEMMQ_OK) return dv;
  clear_pending();
  return launched(gemmq::launch_probe_read(src, bytes, out, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
