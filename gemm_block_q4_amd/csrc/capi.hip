// C ABI of the Q4_K FFN library: argument validation, workspace layout and
// dispatch.  Validation follows the pages' launchers: a null weight pointer is
// rejected before any launch ("realizar -- q4k_gemv_cached_uses.rs",
// q4k_gemv_indexed_async), k must be a multiple of 256 (q4k_gemv_cached), and
// sizes are overflow-checked ("micro_moe.rs", elements / checked_mul).  No
// HIP call happens before every argument check has passed.
#include <hip/hip_runtime.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <set>
#include <utility>

#include "../../include/q4k.h"
#include "q4k_device.hpp"
#include "q4k_internal.hpp"

namespace q4k {

hipError_t lds_opt_in(const void* kern, size_t lds) {
  constexpr size_t kDefaultLds = 64 * 1024;
  constexpr size_t kLdsPerCu = 160 * 1024;
  if (lds <= kDefaultLds) return hipSuccess;
  if (lds > kLdsPerCu) return hipErrorInvalidValue;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::set<std::pair<const void*, int>> done;
  std::lock_guard<std::mutex> lock(mu);
  if (done.count({kern, dev})) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kLdsPerCu));
  if (e != hipSuccess) return e;
  done.insert({kern, dev});
  return hipSuccess;
}

}  // namespace q4k

using namespace q4k;

namespace {

constexpr size_t kAlign = 16;
constexpr size_t kWsAlign = 256;
constexpr size_t kQ6kBlockBytes = 210;  // block_q6_K
constexpr int kMaxDevices = 64;
// Decode path: the per-token sub-block sums and the per-row partials live in
// LDS, which bounds the reduction length.
constexpr int kDecodeMaxK = 32768;
// Prefill path: 64 tokens per workgroup row of the grid (grid.y <= 65535).
constexpr int kPrefillMaxM = 64 * 65535;
// k bound of the prefill kernels: a workgroup's 128 weight rows and 128
// activation rows then stay below 2^31 bytes (32-bit buffer offsets).
constexpr int kPrefillMaxK = 1 << 20;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool mul_ok(size_t a, size_t b, size_t* out) {
  if (a != 0 && b > SIZE_MAX / a) return false;
  *out = a * b;
  return true;
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// 0 unknown, 1 gfx950, 2 other; cached per device ordinal.
std::atomic<int> g_arch_ok[kMaxDevices];

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return Q4K_ERR_DEVICE;
  if (dev < 0 || dev >= kMaxDevices) return Q4K_ERR_DEVICE;
  int state = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return Q4K_ERR_DEVICE;
    state = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_ok[dev].store(state, std::memory_order_relaxed);
  }
  return state == 1 ? Q4K_OK : Q4K_ERR_DEVICE;
}

// Compute units of the current device (0 if unknown), cached per ordinal.
std::atomic<int> g_cus[kMaxDevices];

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int cus = g_cus[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      return 0;
    g_cus[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

int launch_status(hipError_t e) { return e == hipSuccess ? Q4K_OK : Q4K_ERR_LAUNCH; }

// Weight matrix [rows][cols] checks shared by every entry point.
int check_matrix(int rows, int cols, size_t* bytes) {
  if (rows < 1 || cols < Q4K_QK || cols % Q4K_QK != 0) return Q4K_ERR_SHAPE;
  size_t blocks;
  if (!mul_ok(static_cast<size_t>(rows), static_cast<size_t>(cols / Q4K_QK), &blocks)) return Q4K_ERR_OVERFLOW;
  if (blocks > static_cast<size_t>(INT32_MAX)) return Q4K_ERR_OVERFLOW;  // 32-bit block indices
  if (!mul_ok(blocks, Q4K_BLOCK_BYTES, bytes)) return Q4K_ERR_OVERFLOW;
  return Q4K_OK;
}

int check_elems(int m, int k) {
  size_t e;
  if (!mul_ok(static_cast<size_t>(m), static_cast<size_t>(k), &e)) return Q4K_ERR_OVERFLOW;
  if (e > static_cast<size_t>(INT32_MAX) * 4) return Q4K_ERR_OVERFLOW;  // grid of m*k/4 lanes fits
  return Q4K_OK;
}

// Workspace layout of ffn_swiglu_q4k.
struct FfnLayout {
  size_t total = 0;
  // decode dense (and MoE: h and the pair outputs of every (token, slot) pair)
  size_t h = 0, y_pair = 0;
  // prefill and decode_q8: Q8_1 of x and of h, and h itself (decode_q8; in
  // the prefill regime the span of h holds the k-split gate/up sums of the
  // fused pass's last row tiles, and the span qx .. qh the down pass's
  // k-split partial sums)
  size_t qx = 0, dx = 0, qh = 0, dh = 0;
  // MoE prefill: the pairs sorted by expert, the tile table and its count
  // (qh, dh: Q8_1(h) of the pairs in sorted order; y_pair: pair outputs)
  size_t list = 0, tiles = 0, count = 0;
  int max_tiles = 0;
};

// Token rows per tile of the grouped MoE prefill passes (the MMQ tile).
constexpr int kMoeTileRows = 128;

int resolve_regime(int regime, int m) {
  if (regime == Q4K_REGIME_AUTO) return m <= Q4K_DECODE_MAX_TOKENS ? Q4K_REGIME_DECODE : Q4K_REGIME_PREFILL;
  return regime;
}

bool ffn_layout(int m, int hidden, int inter, int top_k, int regime, FfnLayout* L) {
  if (m < 1 || hidden < Q4K_QK || inter < Q4K_QK || hidden % Q4K_QK || inter % Q4K_QK) return false;
  if (top_k < 0 || top_k > 64) return false;
  regime = resolve_regime(regime, m);
  if (regime != Q4K_REGIME_DECODE && regime != Q4K_REGIME_PREFILL && regime != Q4K_REGIME_DECODE_Q8)
    return false;
  if ((regime == Q4K_REGIME_DECODE || regime == Q4K_REGIME_DECODE_Q8) && m > Q4K_DECODE_MAX_TOKENS)
    return false;
  if (top_k > 0 && regime == Q4K_REGIME_DECODE_Q8) return false;
  const size_t M = static_cast<size_t>(m), H = static_cast<size_t>(hidden), I = static_cast<size_t>(inter);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = round_up(off + bytes, kWsAlign);
    return at;
  };
  if (top_k > 0 && regime == Q4K_REGIME_PREFILL) {
    const size_t pairs = M * static_cast<size_t>(top_k);
    if (pairs > static_cast<size_t>(INT32_MAX) || pairs * H > (SIZE_MAX / 8) || pairs * I > (SIZE_MAX / 8))
      return false;
    L->max_tiles = moe_route_max_tiles(static_cast<int>(pairs), kMoeRouteMaxExperts, kMoeTileRows);
    L->qx = take(M * H);
    L->dx = take(M * H / 32 * 4);
    L->list = take(pairs * 4);
    L->tiles = take(static_cast<size_t>(L->max_tiles) * 16);
    L->count = take(4);
    L->qh = take(pairs * I);
    L->dh = take(pairs * I / 32 * 4);
    L->y_pair = take(pairs * H * 4);
  } else if (top_k > 0) {
    const size_t pairs = M * static_cast<size_t>(top_k);
    L->h = take(pairs * I * 4);
    L->y_pair = take(pairs * H * 4);
  } else if (regime == Q4K_REGIME_DECODE) {
    L->h = take(M * I * 4);
  } else {
    if (M * H > (SIZE_MAX / 8) || M * I > (SIZE_MAX / 8)) return false;
    L->qx = take(M * H);
    L->dx = take(M * H / 32 * 4);
    L->h = take(M * I * 4);
    L->qh = take(M * I);
    L->dh = take(M * I / 32 * 4);
  }
  L->total = off;
  return true;
}

}  // namespace

extern "C" {

size_t q4k_weight_bytes(int rows, int cols) {
  if (rows < 0 || cols < 0 || cols % Q4K_QK != 0) return 0;
  size_t blocks, bytes;
  if (!mul_ok(static_cast<size_t>(rows), static_cast<size_t>(cols / Q4K_QK), &blocks)) return 0;
  if (!mul_ok(blocks, Q4K_BLOCK_BYTES, &bytes)) return 0;
  return bytes;
}

const char* q4k_status_string(int status) {
  switch (status) {
    case Q4K_OK: return "ok";
    case Q4K_ERR_NULL: return "a required pointer is NULL";
    case Q4K_ERR_SHAPE: return "a size is out of range or not a required multiple";
    case Q4K_ERR_ALIGN: return "a pointer is not aligned as required";
    case Q4K_ERR_OVERFLOW: return "a derived size overflows";
    case Q4K_ERR_WORKSPACE: return "workspace missing or too small";
    case Q4K_ERR_LAUNCH: return "the HIP runtime reported a launch error";
    case Q4K_ERR_DEVICE: return "the current device is not gfx950";
    case Q4K_ERR_SCRATCH: return "the call needs more scratch than the allocation-free entry point's fixed buffer holds";
    default: return "unknown status";
  }
}

int q4k_gemv(const void* w, const float* x, float* y, int m, int n, int k, void* stream) {
  if (!w || !x || !y) return Q4K_ERR_NULL;
  if (m < 1 || m > Q4K_DECODE_MAX_TOKENS) return Q4K_ERR_SHAPE;
  if (k > kDecodeMaxK) return Q4K_ERR_SHAPE;
  size_t wbytes;
  int st = check_matrix(n, k, &wbytes);
  if (st) return st;
  if ((st = check_elems(m, k)) || (st = check_elems(m, n))) return st;
  if (!aligned(w, kAlign) || !aligned(x, kAlign) || !aligned(y, 4)) return Q4K_ERR_ALIGN;
  if ((st = check_device())) return st;
  GemvArgs a{};
  a.w = static_cast<const uint8_t*>(w);
  a.mat_bytes = wbytes;
  a.x = x;
  a.ldx = k;
  a.y = y;
  a.ldy = n;
  a.n = n;
  a.k = k;
  a.m = m;
  return launch_status(launch_gemv(a, static_cast<hipStream_t>(stream)));
}

int q8_1_quantize(const void* x, int x_dtype, int m, int k, int8_t* qs, uint32_t* ds,
                  void* stream) {
  if (!x || !qs || !ds) return Q4K_ERR_NULL;
  if (x_dtype != Q4K_F32 && x_dtype != Q4K_BF16) return Q4K_ERR_SHAPE;
  if (m < 1 || k < Q4K_Q8_1_BLOCK || k % Q4K_Q8_1_BLOCK != 0) return Q4K_ERR_SHAPE;
  int st = check_elems(m, k);
  if (st) return st;
  if (!aligned(x, x_dtype == Q4K_F32 ? 16 : 8) || !aligned(qs, 4) || !aligned(ds, 4)) return Q4K_ERR_ALIGN;
  if ((st = check_device())) return st;
  return launch_status(launch_q8_1_quantize(x, x_dtype == Q4K_BF16, m, k, qs, ds,
                                            static_cast<hipStream_t>(stream)));
}

int q4k_quantize(const void* x, int x_dtype, int rows, int cols, void* w, void* stream) {
  if (!x || !w) return Q4K_ERR_NULL;
  if (x_dtype != Q4K_F32 && x_dtype != Q4K_BF16) return Q4K_ERR_SHAPE;
  if (rows < 1 || cols < Q4K_QK) return Q4K_ERR_SHAPE;
  size_t wbytes;
  int st = check_matrix(rows, cols, &wbytes);
  if (st) return st;
  if ((st = check_elems(rows, cols))) return st;
  if (!aligned(x, kAlign) || !aligned(w, kAlign)) return Q4K_ERR_ALIGN;  // 16-byte loads of x
  if ((st = check_device())) return st;
  return launch_status(launch_quantize_q4k(x, x_dtype == Q4K_BF16, rows, cols, static_cast<uint8_t*>(w),
                                           static_cast<hipStream_t>(stream)));
}

static int mmq_common(const void* w, const int8_t* qs, const uint32_t* ds, float* y, uint16_t* y_bf16,
                      int32_t* partials, int m, int n, int k, void* stream) {
  if (!w || !qs || (!partials && (!ds || (!y && !y_bf16)))) return Q4K_ERR_NULL;
  if (m < 1 || m > kPrefillMaxM || k > kPrefillMaxK) return Q4K_ERR_SHAPE;
  size_t wbytes;
  int st = check_matrix(n, k, &wbytes);
  if (st) return st;
  if ((st = check_elems(m, k)) || (st = check_elems(m, n))) return st;
  if (partials) {
    size_t e;
    if (!mul_ok(static_cast<size_t>(m) * static_cast<size_t>(n), static_cast<size_t>(k / 32), &e)) return Q4K_ERR_OVERFLOW;
  }
  if (!aligned(w, kAlign) || !aligned(qs, kAlign) || (ds && !aligned(ds, 4)) ||
      (y && !aligned(y, 4)) || (y_bf16 && !aligned(y_bf16, 2)) || (partials && !aligned(partials, 4)))
    return Q4K_ERR_ALIGN;
  if ((st = check_device())) return st;
  MmqArgs a{};
  a.w = static_cast<const uint8_t*>(w);
  a.qs = qs;
  a.ds = ds;
  a.y = y;
  a.y_bf16 = y_bf16;
  a.partials = partials;
  a.m = m;
  a.n = n;
  a.k = k;
  return launch_status(launch_mmq(a, static_cast<hipStream_t>(stream)));
}

int q4k_mmq(const void* w, const int8_t* qs, const uint32_t* ds, float* y, int m, int n, int k,
            void* stream) {
  return mmq_common(w, qs, ds, y, nullptr, nullptr, m, n, k, stream);
}

int q4k_mmq_bf16(const void* w, const int8_t* qs, const uint32_t* ds, uint16_t* y, int m, int n, int k,
                 void* stream) {
  if (!y) return Q4K_ERR_NULL;
  return mmq_common(w, qs, ds, nullptr, y, nullptr, m, n, k, stream);
}

int q4k_q8_gemv(const void* w, const int8_t* qs, const uint32_t* ds, float* y, int m, int n, int k,
                void* stream) {
  if (!w || !qs || !ds || !y) return Q4K_ERR_NULL;
  if (m < 1 || m > Q4K_DECODE_MAX_TOKENS || k > kDecodeMaxK) return Q4K_ERR_SHAPE;
  size_t wbytes;
  int st = check_matrix(n, k, &wbytes);
  if (st) return st;
  if ((st = check_elems(m, k)) || (st = check_elems(m, n))) return st;
  if (!aligned(w, kAlign) || !aligned(qs, kAlign) || !aligned(ds, 8) || !aligned(y, 4)) return Q4K_ERR_ALIGN;
  if ((st = check_device())) return st;
  return launch_status(launch_q8_gemv(static_cast<const uint8_t*>(w), qs, ds, y, m, n, k,
                                      static_cast<hipStream_t>(stream)));
}

size_t q6k_weight_bytes(int rows, int cols) {
  if (rows < 0 || cols < 0 || cols % Q4K_QK != 0) return 0;
  size_t blocks, bytes;
  if (!mul_ok(static_cast<size_t>(rows), static_cast<size_t>(cols / Q4K_QK), &blocks)) return 0;
  if (!mul_ok(blocks, kQ6kBlockBytes, &bytes)) return 0;
  return bytes;
}

int q6k_gemv(const void* w, const float* x, float* y, int n, int k, void* stream) {
  if (!w || !x || !y) return Q4K_ERR_NULL;
  if (n < 1 || k < Q4K_QK || k % Q4K_QK != 0 || k > kDecodeMaxK) return Q4K_ERR_SHAPE;
  size_t blocks, bytes;
  if (!mul_ok(static_cast<size_t>(n), static_cast<size_t>(k / Q4K_QK), &blocks) ||
      blocks > static_cast<size_t>(INT32_MAX) || !mul_ok(blocks, kQ6kBlockBytes, &bytes))
    return Q4K_ERR_OVERFLOW;
  if (!aligned(w, kAlign) || !aligned(x, kAlign) || !aligned(y, 4)) return Q4K_ERR_ALIGN;
  int st = check_device();
  if (st) return st;
  return launch_status(launch_q6k_gemv(static_cast<const uint8_t*>(w), x, y, n, k,
                                       static_cast<hipStream_t>(stream)));
}

int q4k_test_mmq_partials(const void* w, const int8_t* qs, int m, int n, int k,
                          int32_t* partials, void* stream) {
  if (!partials) return Q4K_ERR_NULL;
  return mmq_common(w, qs, nullptr, nullptr, nullptr, partials, m, n, k, stream);
}

int q4k_test_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink) return Q4K_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0) return Q4K_ERR_SHAPE;
  if (bytes / 16 / 256 >= 0x7FFFFFFFu) return Q4K_ERR_OVERFLOW;
  if (!aligned(buf, kAlign) || !aligned(sink, 4)) return Q4K_ERR_ALIGN;
  const int st = check_device();
  if (st) return st;
  return launch_status(launch_read_ceiling(buf, bytes, sink, static_cast<hipStream_t>(stream)));
}

int fp8_absmax_rows(const float* x, int rows, int cols, float* absmax, void* stream) {
  if (!x || !absmax) return Q4K_ERR_NULL;
  if (rows < 1 || cols < 1) return Q4K_ERR_SHAPE;
  size_t e;
  if (!mul_ok(static_cast<size_t>(rows), static_cast<size_t>(cols), &e)) return Q4K_ERR_OVERFLOW;
  if (!aligned(x, 4) || !aligned(absmax, 4)) return Q4K_ERR_ALIGN;
  const int st = check_device();
  if (st) return st;
  return launch_status(launch_fp8_absmax_rows(x, rows, cols, absmax, static_cast<hipStream_t>(stream)));
}

int fp8_quantize_rows(const float* x, int rows, int cols, const float* absmax, uint8_t* q, void* stream) {
  if (!x || !absmax || !q) return Q4K_ERR_NULL;
  if (rows < 1 || cols < 1) return Q4K_ERR_SHAPE;
  size_t e;
  if (!mul_ok(static_cast<size_t>(rows), static_cast<size_t>(cols), &e)) return Q4K_ERR_OVERFLOW;
  if ((e + 255) / 256 > 0x7FFFFFFFu) return Q4K_ERR_OVERFLOW;  // grid of one value per thread
  if (!aligned(x, 4) || !aligned(absmax, 4)) return Q4K_ERR_ALIGN;
  const int st = check_device();
  if (st) return st;
  return launch_status(launch_fp8_quantize_rows(x, rows, cols, absmax, q, static_cast<hipStream_t>(stream)));
}

int fp8_gemm_dequant(const uint8_t* a, const float* a_absmax, const uint8_t* w, const float* w_absmax, float* y,
                     int m, int n, int k, void* stream) {
  if (!a || !a_absmax || !w || !w_absmax || !y) return Q4K_ERR_NULL;
  if (m < 1 || m > kPrefillMaxM || n < 1 || k < 16 || k % 16 != 0 || k > kPrefillMaxK) return Q4K_ERR_SHAPE;
  if ((static_cast<size_t>(n) + 127) / 128 > 0x7FFFFFFFu) return Q4K_ERR_SHAPE;
  size_t e;
  if (!mul_ok(static_cast<size_t>(m), static_cast<size_t>(n), &e) ||
      !mul_ok(static_cast<size_t>(m), static_cast<size_t>(k), &e) ||
      !mul_ok(static_cast<size_t>(n), static_cast<size_t>(k), &e))
    return Q4K_ERR_OVERFLOW;
  if (!aligned(a, kAlign) || !aligned(w, kAlign) || !aligned(a_absmax, 4) || !aligned(w_absmax, 4) ||
      !aligned(y, 4))
    return Q4K_ERR_ALIGN;
  const int st = check_device();
  if (st) return st;
  return launch_status(launch_fp8_gemm(a, a_absmax, w, w_absmax, y, m, n, k, static_cast<hipStream_t>(stream)));
}

size_t ffn_swiglu_q4k_workspace_bytes(int m, int hidden, int inter, int top_k, int regime) {
  FfnLayout L;
  if (!ffn_layout(m, hidden, inter, top_k, regime, &L)) return 0;
  return L.total;
}

}  // extern "C"

namespace {

// Scratch memory of the allocation-free FFN entry point: one copy per device
// (the loader places it in each device's memory with the code object).  Host
// code never passes `scratch` itself to a kernel (on the host it names a
// stand-in, not the device copy); it resolves the device address once per
// device with hipGetSymbolAddress and passes that.
static __device__ __align__(256) uint8_t scratch[Q4K_NOALLOC_SCRATCH_BYTES];

std::atomic<void*> g_scratch[kMaxDevices];

// Device address of `scratch` on the current device (nullptr on error).
void* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

// ffn_swiglu_q4k with the caller's workspace, or (use_scratch) with the
// library's fixed scratch buffer of the current device.
int ffn_common(const void* w_gate, const void* w_up, const void* w_down, int n_experts,
               const void* x, int x_dtype, int m, int hidden, int inter, const int32_t* ids,
               const float* wts, int top_k, int regime, float* y, void* workspace,
               size_t workspace_bytes, bool use_scratch, void* stream) {
  if (!w_gate || !w_up || !w_down || !x || !y) return Q4K_ERR_NULL;
  if (x_dtype != Q4K_F32 && x_dtype != Q4K_BF16) return Q4K_ERR_SHAPE;
  if (m < 1 || n_experts < 1) return Q4K_ERR_SHAPE;
  const bool moe = ids != nullptr;
  if (moe) {
    if (!wts) return Q4K_ERR_NULL;
    if (top_k < 1 || top_k > 64 || top_k > n_experts) return Q4K_ERR_SHAPE;
  } else {
    if (n_experts != 1 || (top_k != 0 && top_k != 1)) return Q4K_ERR_SHAPE;
    top_k = 0;
  }
  if (regime < Q4K_REGIME_AUTO || regime > Q4K_REGIME_DECODE_Q8) return Q4K_ERR_SHAPE;
  const int reg = resolve_regime(regime, m);
  const bool decode = reg == Q4K_REGIME_DECODE || reg == Q4K_REGIME_DECODE_Q8;
  if (decode && m > Q4K_DECODE_MAX_TOKENS) return Q4K_ERR_SHAPE;
  if (moe && reg == Q4K_REGIME_DECODE_Q8) return Q4K_ERR_SHAPE;
  if (moe && reg == Q4K_REGIME_PREFILL) {
    // the routing kernel's per-expert counters live in LDS; the gate/up pass
    // addresses Q8_1(x) by token row with 32-bit offsets
    if (n_experts > kMoeRouteMaxExperts) return Q4K_ERR_SHAPE;
    if (static_cast<long long>(m) * top_k <= INT32_MAX &&
        moe_route_max_tiles(m * top_k, n_experts, kMoeTileRows) > 65535)  // grid rows of the passes
      return Q4K_ERR_SHAPE;
    if (static_cast<long long>(m) * hidden > (1ll << 31) ||
        static_cast<long long>(m) * top_k * inter > (1ll << 31) ||
        static_cast<long long>(m) * top_k > INT32_MAX)
      return Q4K_ERR_OVERFLOW;
  }
  if (decode && (hidden > kDecodeMaxK || inter > kDecodeMaxK)) return Q4K_ERR_SHAPE;
  if (reg == Q4K_REGIME_PREFILL && (m > kPrefillMaxM || hidden > kPrefillMaxK || inter > kPrefillMaxK))
    return Q4K_ERR_SHAPE;
  size_t gu_bytes, dn_bytes;
  int st = check_matrix(inter, hidden, &gu_bytes);
  if (st) return st;
  if ((st = check_matrix(hidden, inter, &dn_bytes))) return st;
  size_t bank;
  if (!mul_ok(gu_bytes, static_cast<size_t>(n_experts), &bank) ||
      !mul_ok(dn_bytes, static_cast<size_t>(n_experts), &bank))
    return Q4K_ERR_OVERFLOW;
  if ((st = check_elems(m, hidden)) || (st = check_elems(m, inter))) return st;
  if (moe && ((st = check_elems(m * top_k, hidden)) || (st = check_elems(m * top_k, inter)))) return st;
  FfnLayout L;
  if (!ffn_layout(m, hidden, inter, top_k, reg, &L)) return Q4K_ERR_SHAPE;
  if (use_scratch) {
    if (L.total > Q4K_NOALLOC_SCRATCH_BYTES) return Q4K_ERR_SCRATCH;
  } else if (!workspace || workspace_bytes < L.total) {
    return Q4K_ERR_WORKSPACE;
  }
  if (!aligned(w_gate, kAlign) || !aligned(w_up, kAlign) || !aligned(w_down, kAlign) ||
      !aligned(x, kAlign) || !aligned(y, 4) || (!use_scratch && !aligned(workspace, kAlign)) ||
      (ids && !aligned(ids, 4)) || (wts && !aligned(wts, 4)))
    return Q4K_ERR_ALIGN;
  if ((st = check_device())) return st;
  if (use_scratch) {
    workspace = scratch_ptr();
    if (!workspace) return Q4K_ERR_LAUNCH;
    workspace_bytes = Q4K_NOALLOC_SCRATCH_BYTES;
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* h = reinterpret_cast<float*>(ws + L.h);

  if (moe && reg == Q4K_REGIME_PREFILL) {
    // Grouped prefill ("micro_moe.rs": one group per (token, selection)
    // pair; "q4k_mmq.rs" prefill pipeline per group): x -> Q8_1 per token;
    // the pairs sorted by expert and cut into 128-row tiles; one grouped
    // gate/up MMQ over every (expert, row tile) that gathers its pairs'
    // token rows and writes Q8_1(silu(g)*u) in sorted order; one grouped
    // down MMQ over those rows that writes each pair's output row; the
    // slot-order weighted combine.
    const int pairs = m * top_k;
    int8_t* qx = reinterpret_cast<int8_t*>(ws + L.qx);
    uint32_t* dx = reinterpret_cast<uint32_t*>(ws + L.dx);
    int32_t* list = reinterpret_cast<int32_t*>(ws + L.list);
    int32_t* tiles = reinterpret_cast<int32_t*>(ws + L.tiles);
    int32_t* count = reinterpret_cast<int32_t*>(ws + L.count);
    int8_t* qh = reinterpret_cast<int8_t*>(ws + L.qh);
    uint32_t* dh = reinterpret_cast<uint32_t*>(ws + L.dh);
    float* y_pair = reinterpret_cast<float*>(ws + L.y_pair);
    const int grid_rows = moe_route_max_tiles(pairs, n_experts, kMoeTileRows);
    hipError_t e = launch_q8_1_quantize(x, x_dtype == Q4K_BF16, m, hidden, qx, dx, s);
    if (e != hipSuccess) return Q4K_ERR_LAUNCH;
    if ((e = launch_moe_route(ids, pairs, n_experts, kMoeTileRows, list, tiles, count, s)) != hipSuccess)
      return Q4K_ERR_LAUNCH;
    MmqArgs gu{};
    gu.w = static_cast<const uint8_t*>(w_gate);
    gu.w_up = static_cast<const uint8_t*>(w_up);
    gu.qs = qx;
    gu.ds = dx;
    gu.q_out = qh;
    gu.d_out = dh;
    gu.m = m;
    gu.n = inter;
    gu.k = hidden;
    gu.group_tiles = tiles;
    gu.group_count = count;
    gu.group_list = list;
    gu.group_mat_bytes = gu_bytes;
    gu.group_top_k = top_k;
    gu.group_grid_rows = grid_rows;
    if ((e = launch_mmq(gu, s)) != hipSuccess) return Q4K_ERR_LAUNCH;
    MmqArgs dn{};
    dn.w = static_cast<const uint8_t*>(w_down);
    dn.qs = qh;
    dn.ds = dh;
    dn.y = y_pair;
    dn.m = pairs;
    dn.n = hidden;
    dn.k = inter;
    dn.group_tiles = tiles;
    dn.group_count = count;
    dn.group_list = list;
    dn.group_mat_bytes = dn_bytes;
    dn.group_scatter = 1;
    dn.group_grid_rows = grid_rows;
    if ((e = launch_mmq(dn, s)) != hipSuccess) return Q4K_ERR_LAUNCH;
    return launch_status(launch_moe_combine(y_pair, wts, ids, m, top_k, n_experts, hidden, y, s));
  }

  if (moe) {
    // Gate/up: every (token, slot) pair is an independent pass over its
    // expert's rows on x row t (h row = pair).  Down: per token, its slots'
    // experts on the pairs' h rows, summed with the routing weights in slot
    // order.
    GemvArgs gu{};
    gu.w = static_cast<const uint8_t*>(w_gate);
    gu.w_up = static_cast<const uint8_t*>(w_up);
    gu.mat_bytes = gu_bytes;
    gu.x = x;
    gu.x_bf16 = x_dtype == Q4K_BF16;
    gu.ldx = hidden;
    gu.y = h;
    gu.ldy = inter;
    gu.n = inter;
    gu.k = hidden;
    gu.m = m;
    gu.ids = ids;
    gu.x_by_token = 1;
    gu.top_k = top_k;
    gu.n_experts = n_experts;
    gu.pairs = m * top_k;
    hipError_t e = launch_gemv(gu, s);
    if (e != hipSuccess) return Q4K_ERR_LAUNCH;
    float* y_pair = reinterpret_cast<float*>(ws + L.y_pair);
    GemvArgs dn = gu;
    dn.w = static_cast<const uint8_t*>(w_down);
    dn.w_up = nullptr;
    dn.mat_bytes = dn_bytes;
    dn.x = h;
    dn.x_bf16 = 0;
    dn.ldx = inter;
    dn.y = y;
    dn.ldy = hidden;
    dn.n = hidden;
    dn.k = inter;
    dn.x_by_token = 0;
    dn.wts = wts;
    // down with the combine folded in when the rows fit one wavefront, else
    // pair outputs and the combine kernel
    e = launch_moe_down(dn, s);
    if (e != hipErrorNotSupported) return launch_status(e);
    dn.y = y_pair;
    if ((e = launch_gemv(dn, s)) != hipSuccess) return Q4K_ERR_LAUNCH;
    return launch_status(launch_moe_combine(y_pair, wts, ids, m, top_k, n_experts, hidden, y, s));
  }

  if (reg == Q4K_REGIME_DECODE) {
    GemvArgs gu{};
    gu.w = static_cast<const uint8_t*>(w_gate);
    gu.w_up = static_cast<const uint8_t*>(w_up);
    gu.mat_bytes = gu_bytes;
    gu.x = x;
    gu.x_bf16 = x_dtype == Q4K_BF16;
    gu.ldx = hidden;
    gu.y = h;
    gu.ldy = inter;
    gu.n = inter;
    gu.k = hidden;
    gu.m = m;
    // 2..8 tokens: the down pass may split k in two halves that add into y,
    // which the gate/up pass zeroes; not when y overlaps x (an in-place call:
    // x must stay intact until the gate/up pass has read it)
    const size_t x_bytes = static_cast<size_t>(m) * hidden * (x_dtype == Q4K_BF16 ? 2 : 4);
    const size_t y_bytes = static_cast<size_t>(m) * hidden * 4;
    const uintptr_t xa = reinterpret_cast<uintptr_t>(x), ya = reinterpret_cast<uintptr_t>(y);
    const bool split = gemv_mfma_splits(m, hidden, inter) == 2 && (ya + y_bytes <= xa || xa + x_bytes <= ya);
    if (split) {
      gu.zero_out = y;
      gu.zero_n = m * hidden;
    }
    hipError_t e = launch_gemv(gu, s);
    if (e != hipSuccess) return Q4K_ERR_LAUNCH;
    GemvArgs dn{};
    dn.w = static_cast<const uint8_t*>(w_down);
    dn.mat_bytes = dn_bytes;
    dn.x = h;
    dn.ldx = inter;
    dn.y = y;
    dn.ldy = hidden;
    dn.n = hidden;
    dn.k = inter;
    dn.m = m;
    if (split) dn.splits = 2;
    return launch_status(launch_gemv(dn, s));
  }

  int8_t* qx = reinterpret_cast<int8_t*>(ws + L.qx);
  uint32_t* dx = reinterpret_cast<uint32_t*>(ws + L.dx);
  int8_t* qh = reinterpret_cast<int8_t*>(ws + L.qh);
  uint32_t* dh = reinterpret_cast<uint32_t*>(ws + L.dh);
  hipError_t e = launch_q8_1_quantize(x, x_dtype == Q4K_BF16, m, hidden, qx, dx, s);
  if (e != hipSuccess) return Q4K_ERR_LAUNCH;

  if (reg == Q4K_REGIME_DECODE_Q8) {
    // x -> Q8_1 -> gate/up integer-dot GEMV with silu*mul -> h -> Q8_1 ->
    // down integer-dot GEMV
    if ((e = launch_q8_gemv_gu(static_cast<const uint8_t*>(w_gate), static_cast<const uint8_t*>(w_up), qx,
                               dx, h, m, inter, hidden, s)) != hipSuccess)
      return Q4K_ERR_LAUNCH;
    if ((e = launch_q8_1_quantize(h, 0, m, inter, qh, dh, s)) != hipSuccess) return Q4K_ERR_LAUNCH;
    return launch_status(launch_q8_gemv(static_cast<const uint8_t*>(w_down), qh, dh, y, m, hidden, inter, s));
  }

  // Prefill: x -> Q8_1 -> MMQ gate/up with silu*mul and Q8_1(h) in its
  // epilogue -> MMQ down (h itself is never stored).
  MmqArgs gu{};
  gu.w = static_cast<const uint8_t*>(w_gate);
  gu.w_up = static_cast<const uint8_t*>(w_up);
  gu.qs = qx;
  gu.ds = dx;
  gu.y = h;
  gu.q_out = qh;
  gu.d_out = dh;
  gu.m = m;
  gu.n = inter;
  gu.k = hidden;
  // The fused pass runs (inter/64) x ceil(m/128) workgroups, one per compute
  // unit at a time.  When its last round would leave compute units idle
  // (512 tokens at 5120/17408: 1088 workgroups, 4.25 rounds on 256 CUs), the
  // last row tiles run first as a k-split pass that fills one round, whose
  // gate and up sums go to the span of h (not read by this FFN's passes
  // before the down pass overwrites it) and are added in split order by a
  // small kernel that applies silu * mul and writes their Q8_1(h); the other
  // row tiles then run as before.
  const int cus = device_cus();
  const int rt = inter / 64, tt = (m + 127) / 128;
  const long long gu_tiles = static_cast<long long>(rt) * tt;
  const int kb_all = hidden / Q4K_QK;
  int tail = 0, tsplit = 1;
  if (cus > 0 && gu_tiles > cus && gu_tiles % cus != 0) {
    tail = static_cast<int>((gu_tiles % cus + tt - 1) / tt);
    tsplit = std::min({4, kb_all, cus / (tail * tt), rt / (2 * tail)});
    // every split owns at least one block (e.g. 5 blocks: 3 splits, not 4)
    while (tsplit > 1 && (tsplit - 1) * ((kb_all + tsplit - 1) / tsplit) >= kb_all) --tsplit;
    if (tsplit < 2) tail = 0;
  }
  if (tail > 0) {
    float* parts = h;
    MmqArgs tp = gu;
    tp.y = nullptr;
    tp.q_out = nullptr;
    tp.d_out = nullptr;
    tp.gu_parts = parts;
    tp.row_tile0 = rt - tail;
    tp.row_tiles = tail;
    tp.splits = tsplit;
    tp.split_blocks = (kb_all + tsplit - 1) / tsplit;
    if ((e = launch_mmq(tp, s)) != hipSuccess) return Q4K_ERR_LAUNCH;
    if ((e = launch_mmq_gu_finish(parts, tsplit, m, tail * 64, (rt - tail) * 64, inter, qh, dh, s)) !=
        hipSuccess)
      return Q4K_ERR_LAUNCH;
    gu.row_tiles = rt - tail;
  }
  if ((e = launch_mmq(gu, s)) != hipSuccess) return Q4K_ERR_LAUNCH;
  MmqArgs dn{};
  dn.w = static_cast<const uint8_t*>(w_down);
  dn.qs = qh;
  dn.ds = dh;
  dn.y = y;
  dn.m = m;
  dn.n = hidden;
  dn.k = inter;
  // When the down pass has too few workgroups to fill the device, split its
  // k range; the partial sums go to the span of qx, dx and h, which the down
  // pass does not read, and are added in split order.
  const size_t plane = static_cast<size_t>(m) * static_cast<size_t>(hidden);
  const int max_splits = static_cast<int>(std::min<size_t>((L.qh - L.qx) / (plane * 4), 8));
  const int splits = cus > 0 && max_splits > 1 && aligned(y, 16)  // the reduction stores float4
                         ? mmq_choose_splits(m, hidden, inter, max_splits, cus)
                         : 1;
  if (splits == 1) return launch_status(launch_mmq(dn, s));
  float* parts = reinterpret_cast<float*>(ws + L.qx);
  dn.y = parts;
  dn.splits = splits;
  dn.split_blocks = (inter / Q4K_QK + splits - 1) / splits;
  dn.split_stride = plane;
  if ((e = launch_mmq(dn, s)) != hipSuccess) return Q4K_ERR_LAUNCH;
  return launch_status(launch_mmq_split_reduce(parts, splits, plane, plane, y, s));
}

}  // namespace

extern "C" {

int ffn_swiglu_q4k(const void* w_gate, const void* w_up, const void* w_down, int n_experts,
                   const void* x, int x_dtype, int m, int hidden, int inter, const int32_t* ids,
                   const float* wts, int top_k, int regime, float* y, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return ffn_common(w_gate, w_up, w_down, n_experts, x, x_dtype, m, hidden, inter, ids, wts, top_k,
                    regime, y, workspace, workspace_bytes, false, stream);
}

int ffn_swiglu_q4k_noalloc(const void* w_gate, const void* w_up, const void* w_down, int n_experts,
                           const void* x, int x_dtype, int m, int hidden, int inter,
                           const int32_t* ids, const float* wts, int top_k, int regime, float* y,
                           void* stream) {
  return ffn_common(w_gate, w_up, w_down, n_experts, x, x_dtype, m, hidden, inter, ids, wts, top_k,
                    regime, y, nullptr, 0, true, stream);
}

}  // extern "C"
