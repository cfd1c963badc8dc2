// C ABI of libqmv: argument validation, error reporting and dispatch.
//
// Unsupported or malformed requests are rejected on the host, before any
// launch, with a message naming the argument or the missing capability
// (aot-llm README: unsupported tensor types are rejected with a message
// naming the tensor; pytensor-ml issue 53, PR 18 acceptance rules: fail with
// the missing capability named, not at token 1).
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "qmv_internal.h"

namespace {

thread_local char g_last_error[256] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return QMV_OK;
}

const char* fmt_name(int fmt) {
  switch (fmt) {
    case QMV_Q8_0: return "Q8_0";
    case QMV_W4A16_G64: return "W4A16_G64";
    case QMV_Q4K: return "Q4K";
    case QMV_Q6K: return "Q6K";
    case QMV_Q4_0: return "Q4_0";
    case QMV_Q5_0: return "Q5_0";
    case QMV_Q5K: return "Q5K";
    case QMV_DENSE_BF16: return "DENSE_BF16";
    case QMV_I8_ROW: return "I8_ROW";
    default: return "?";
  }
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Per-device architecture check, cached after the first query.
constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(QMV_ERR_DEVICE, "hipGetDevice failed (no HIP device?)");
  if (dev < kMaxDevices) {
    const int st = g_dev_state[dev].load(std::memory_order_relaxed);
    if (st == 1) return QMV_OK;
    if (st == -1) return fail(QMV_ERR_DEVICE, "device %d is not gfx950", dev);
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
    return fail(QMV_ERR_DEVICE, "hipGetDeviceProperties(%d) failed", dev);
  const bool is950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_dev_state[dev].store(is950 ? 1 : -1, std::memory_order_relaxed);
  if (!is950) return fail(QMV_ERR_DEVICE, "device %d is %s, the library is built for gfx950", dev,
                          prop.gcnArchName);
  return QMV_OK;
}

int check_fmt(int fmt) {
  if (qmv::block_of(fmt) == 0) return fail(QMV_ERR_FORMAT, "unknown format %d", fmt);
  return QMV_OK;
}

// N, K, batch sanity and size limits shared by all entry points.
int check_shape(int fmt, int64_t N, int64_t K, int64_t batch, const char* batch_name) {
  const int blk = qmv::block_of(fmt);
  if (N < 1) return fail(QMV_ERR_SHAPE, "N=%lld must be >= 1", (long long)N);
  if (K < 1) return fail(QMV_ERR_SHAPE, "K=%lld must be >= 1", (long long)K);
  if (K % blk) return fail(QMV_ERR_SHAPE, "K=%lld is not a multiple of the %s block (%d)",
                           (long long)K, fmt_name(fmt), blk);
  if (batch < 1) return fail(QMV_ERR_SHAPE, "%s=%lld must be >= 1", batch_name, (long long)batch);
  // kernels index rows and K with 32-bit ints and planes with 64-bit offsets
  const int64_t lim = int64_t(1) << 31;
  if (N >= lim || K >= lim) return fail(QMV_ERR_OVERFLOW, "N or K too large for 32-bit indexing");
  if (N > (int64_t(1) << 62) / K) return fail(QMV_ERR_OVERFLOW, "N*K overflows");
  return QMV_OK;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(QMV_ERR_LAUNCH, "%s launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int qmv_abi_version(int* layout_version) {
  if (layout_version) *layout_version = QMV_LAYOUT_VERSION;
  return QMV_ABI_VERSION;
}

const char* qmv_status_string(int status) {
  switch (status) {
    case QMV_OK: return "ok";
    case QMV_ERR_NULL: return "null pointer";
    case QMV_ERR_FORMAT: return "unknown format";
    case QMV_ERR_UNSUPPORTED: return "unsupported";
    case QMV_ERR_SHAPE: return "bad shape";
    case QMV_ERR_ALIGN: return "misaligned pointer";
    case QMV_ERR_DTYPE: return "bad dtype";
    case QMV_ERR_OVERFLOW: return "size overflow";
    case QMV_ERR_DEVICE: return "device error";
    case QMV_ERR_LAUNCH: return "launch failed";
    default: return "unknown status";
  }
}

const char* qmv_last_error(void) { return g_last_error; }

int qmv_packed_bytes(int fmt, int64_t N, int64_t K, int64_t batch, size_t* out_bytes) {
  int st;
  if ((st = check_fmt(fmt))) return st;
  if ((st = check_shape(fmt, N, K, batch, "batch"))) return st;
  if (!out_bytes) return fail(QMV_ERR_NULL, "out_bytes is NULL");
  const qmv::Planes p = qmv::planes_of(fmt, N, K);
  if (batch > INT64_MAX / p.total) return fail(QMV_ERR_OVERFLOW, "batch * packed bytes overflows");
  *out_bytes = static_cast<size_t>(batch * p.total);
  return ok();
}

int qmv_pack(int fmt, int64_t N, int64_t K, int64_t batch, const qmv_logical* src, void* dst,
             void* stream) {
  int st;
  if ((st = check_fmt(fmt))) return st;
  if ((st = check_shape(fmt, N, K, batch, "batch"))) return st;
  if (batch > 65535) return fail(QMV_ERR_OVERFLOW, "batch=%lld exceeds 65535", (long long)batch);
  if (!src) return fail(QMV_ERR_NULL, "src is NULL");
  if (!dst) return fail(QMV_ERR_NULL, "dst is NULL");
  if (!src->q) return fail(QMV_ERR_NULL, "src->q is NULL");
  const int naux = qmv::aux_count(fmt);
  for (int i = 0; i < naux; ++i)
    if (!src->aux[i]) return fail(QMV_ERR_NULL, "src->aux[%d] is NULL (%s needs %d)", i, fmt_name(fmt), naux);
  if (!aligned(dst, 16)) return fail(QMV_ERR_ALIGN, "dst is not 16-byte aligned");
  // f16 arrays (and the bf16 weights) 2-byte aligned, I8_ROW's f32 scales 4-byte
  const uintptr_t aux_align = fmt == QMV_I8_ROW ? 4 : 2;
  for (int i = 0; i < naux; ++i)
    if (!aligned(src->aux[i], aux_align))
      return fail(QMV_ERR_ALIGN, "src->aux[%d] is not %d-byte aligned", i, int(aux_align));
  if (fmt == QMV_DENSE_BF16 && !aligned(src->q, 2)) return fail(QMV_ERR_ALIGN, "src->q is not 2-byte aligned");
  const qmv::Planes p = qmv::planes_of(fmt, N, K);
  if (batch > INT64_MAX / p.total) return fail(QMV_ERR_OVERFLOW, "batch * packed bytes overflows");
  if ((N * K * (fmt == QMV_DENSE_BF16 ? 2 : 1) + 255) / 256 >= (int64_t(1) << 31))
    return fail(QMV_ERR_OVERFLOW, "matrix too large for one pack launch");
  if ((st = check_device())) return st;
  return launched(qmv::launch_pack(fmt, N, K, batch, *src, static_cast<uint8_t*>(dst), as_stream(stream)),
                  "pack");
}

static int check_matvec_args(int fmt, int64_t N, int64_t K, int64_t batch, const void* W, const void* x,
                             int x_dtype, const void* y, int y_dtype, const char* who) {
  int st;
  if ((st = check_shape(fmt, N, K, batch, "batch"))) {
    if (*who) {  // name the item
      char msg[sizeof(g_last_error)];
      std::snprintf(msg, sizeof(msg), "%s", g_last_error);
      fail(st, "%s%s", who, msg);
    }
    return st;
  }
  if (!W) return fail(QMV_ERR_NULL, "%sW is NULL", who);
  if (!x) return fail(QMV_ERR_NULL, "%sx is NULL", who);
  if (!y) return fail(QMV_ERR_NULL, "%sy is NULL", who);
  if (x_dtype != QMV_F32 && x_dtype != QMV_F16 && x_dtype != QMV_BF16 && x_dtype != QMV_Q8X)
    return fail(QMV_ERR_DTYPE, "x_dtype=%d is not a qmv_dtype", x_dtype);
  if (y_dtype != QMV_F32 && y_dtype != QMV_F16 && y_dtype != QMV_BF16 && y_dtype != QMV_Q8X)
    return fail(QMV_ERR_DTYPE, "y_dtype=%d is not a qmv_dtype", y_dtype);
  if (x_dtype == QMV_BF16 || (x_dtype == QMV_F16 && fmt != QMV_W4A16_G64) ||
      (x_dtype == QMV_Q8X && fmt == QMV_DENSE_BF16))
    return fail(QMV_ERR_UNSUPPORTED, "%s%s matvec takes x as f32%s", who, fmt_name(fmt),
                fmt == QMV_W4A16_G64 ? ", f16 or Q8X" : fmt == QMV_DENSE_BF16 ? "" : " or Q8X");
  if (y_dtype != QMV_F32) return fail(QMV_ERR_UNSUPPORTED, "matvec writes y as f32 only");
  if (!aligned(W, 16)) return fail(QMV_ERR_ALIGN, "%sW is not 16-byte aligned", who);
  if (!aligned(x, 16)) return fail(QMV_ERR_ALIGN, "%sx is not 16-byte aligned", who);
  if (!aligned(y, 4)) return fail(QMV_ERR_ALIGN, "%sy is not 4-byte aligned", who);
  const int64_t lim = int64_t(1) << 31;
  if (N * 16 >= lim) return fail(QMV_ERR_OVERFLOW, "N=%lld too large for the row grid", (long long)N);
  return QMV_OK;
}

int qmv_matvec(int fmt, int64_t N, int64_t K, int64_t batch, const void* W, const void* x,
               int x_dtype, void* y, int y_dtype, void* stream) {
  int st;
  if ((st = check_fmt(fmt))) return st;
  if ((st = check_matvec_args(fmt, N, K, batch, W, x, x_dtype, y, y_dtype, ""))) return st;
  if ((st = check_device())) return st;
  return launched(qmv::launch_matvec(fmt, N, K, batch, static_cast<const uint8_t*>(W), x, x_dtype,
                                     static_cast<float*>(y), as_stream(stream)),
                  "matvec");
}

int qmv_matvec_ex(int fmt, int64_t N, int64_t K, int64_t batch, const void* W, const void* x, int x_dtype,
                  void* y, int y_dtype, const qmv_epilogue* ep, void* stream) {
  int st;
  if ((st = check_fmt(fmt))) return st;
  if ((st = check_matvec_args(fmt, N, K, batch, W, x, x_dtype, y, y_dtype, ""))) return st;
  const float* bias = ep ? ep->bias : nullptr;
  const float* res = ep ? ep->residual : nullptr;
  if (bias && !aligned(bias, 4)) return fail(QMV_ERR_ALIGN, "ep->bias is not 4-byte aligned");
  if (res && !aligned(res, 4)) return fail(QMV_ERR_ALIGN, "ep->residual is not 4-byte aligned");
  if ((st = check_device())) return st;
  return launched(qmv::launch_matvec_epi(fmt, N, K, batch, static_cast<const uint8_t*>(W), nullptr, x, x_dtype,
                                         static_cast<float*>(y), bias, res, as_stream(stream)),
                  "matvec_ex");
}

int qmv_matvec_swiglu(int fmt, int64_t N, int64_t K, int64_t batch, const void* W_gate, const void* W_up,
                      const void* x, int x_dtype, void* h, int h_dtype, void* stream) {
  int st;
  if ((st = check_fmt(fmt))) return st;
  if (!W_gate) return fail(QMV_ERR_NULL, "W_gate is NULL");
  if (!W_up) return fail(QMV_ERR_NULL, "W_up is NULL");
  if ((st = check_matvec_args(fmt, N, K, batch, W_gate, x, x_dtype, h, h_dtype, ""))) return st;
  if (!aligned(W_up, 16)) return fail(QMV_ERR_ALIGN, "W_up is not 16-byte aligned");
  if ((st = check_device())) return st;
  return launched(qmv::launch_matvec_epi(fmt, N, K, batch, static_cast<const uint8_t*>(W_gate),
                                         static_cast<const uint8_t*>(W_up), x, x_dtype, static_cast<float*>(h),
                                         nullptr, nullptr, as_stream(stream)),
                  "matvec_swiglu");
}

int qmv_matvec_grouped(int fmt, int64_t K, int64_t batch, int count, const qmv_matvec_item* items,
                       int x_dtype, int y_dtype, void* stream) {
  int st;
  if (fmt != 0 && (st = check_fmt(fmt))) return st;
  if (count < 1 || count > 4096) return fail(QMV_ERR_SHAPE, "count=%d must be in [1, 4096]", count);
  if (!items) return fail(QMV_ERR_NULL, "items is NULL");
  char who[32];
  for (int i = 0; i < count; ++i) {
    std::snprintf(who, sizeof(who), "items[%d].", i);
    const int f = items[i].fmt ? items[i].fmt : fmt;
    if (f == 0) return fail(QMV_ERR_FORMAT, "%sfmt is 0 and the call's fmt is 0", who);
    if (qmv::block_of(f) == 0) return fail(QMV_ERR_FORMAT, "%sfmt=%d is not a qmv_format", who, f);
    if ((st = check_matvec_args(f, items[i].N, K, batch, items[i].W, items[i].x, x_dtype, items[i].y,
                                y_dtype, who)))
      return st;
  }
  if ((st = check_device())) return st;
  hipStream_t s = as_stream(stream);
  {
    hipError_t e = hipSuccess;
    if (batch == 1 ? qmv::launch_matvec_grouped_b1(fmt, K, count, items, x_dtype, s, &e)
                   : qmv::launch_matvec_grouped_mfma(fmt, K, batch, count, items, x_dtype, s, &e))
      return launched(e, "grouped matvec");
  }
  for (int i = 0; i < count; ++i) {
    const int f = items[i].fmt ? items[i].fmt : fmt;
    const hipError_t e = qmv::launch_matvec(f, items[i].N, K, batch, static_cast<const uint8_t*>(items[i].W),
                                            items[i].x, x_dtype, static_cast<float*>(items[i].y), s);
    if (e != hipSuccess) return launched(e, "grouped matvec");
  }
  return ok();
}

int qmv_gemm(int fmt, int64_t N, int64_t K, int64_t M, const void* W, const void* X, int x_dtype,
             void* Y, int y_dtype, void* stream) {
  int st;
  if ((st = check_fmt(fmt))) return st;
  if ((st = check_shape(fmt, N, K, M, "M"))) return st;
  if (!W) return fail(QMV_ERR_NULL, "W is NULL");
  if (!X) return fail(QMV_ERR_NULL, "X is NULL");
  if (!Y) return fail(QMV_ERR_NULL, "Y is NULL");
  if (x_dtype != QMV_F32 && x_dtype != QMV_F16 && x_dtype != QMV_BF16)
    return fail(QMV_ERR_DTYPE, "x_dtype=%d is not a qmv_dtype", x_dtype);
  if (y_dtype != QMV_F32 && y_dtype != QMV_F16 && y_dtype != QMV_BF16)
    return fail(QMV_ERR_DTYPE, "y_dtype=%d is not a qmv_dtype", y_dtype);
  if (fmt != QMV_W4A16_G64)
    return fail(QMV_ERR_UNSUPPORTED, "gemm supports W4A16_G64 only (got %s)", fmt_name(fmt));
  if (x_dtype != QMV_BF16 || y_dtype != QMV_BF16)
    return fail(QMV_ERR_UNSUPPORTED, "gemm takes X and writes Y as bf16");
  if (!aligned(W, 16)) return fail(QMV_ERR_ALIGN, "W is not 16-byte aligned");
  if (!aligned(X, 16)) return fail(QMV_ERR_ALIGN, "X is not 16-byte aligned");
  if (!aligned(Y, 4)) return fail(QMV_ERR_ALIGN, "Y is not 4-byte aligned");
  if (M >= (int64_t(1) << 31)) return fail(QMV_ERR_OVERFLOW, "M too large");
  if ((st = check_device())) return st;
  return launched(qmv::launch_gemm(fmt, N, K, M, static_cast<const uint8_t*>(W),
                                   static_cast<const uint16_t*>(X), static_cast<uint16_t*>(Y),
                                   as_stream(stream)),
                  "gemm");
}

int qmv_q8x_bytes(int64_t K, int64_t batch, size_t* out_bytes) {
  if (K < 32 || K % 32) return fail(QMV_ERR_SHAPE, "K=%lld must be a positive multiple of 32", (long long)K);
  if (batch < 1) return fail(QMV_ERR_SHAPE, "batch=%lld must be >= 1", (long long)batch);
  if (!out_bytes) return fail(QMV_ERR_NULL, "out_bytes is NULL");
  if (K >= (int64_t(1) << 31) || batch > (int64_t(1) << 40) / qmv::q8x_record_bytes(K))
    return fail(QMV_ERR_OVERFLOW, "batch * K too large");
  *out_bytes = static_cast<size_t>(batch * qmv::q8x_record_bytes(K));
  return ok();
}

int qmv_quantize_x(int64_t K, int64_t batch, const float* x, void* xq, void* stream) {
  int st;
  size_t bytes = 0;
  if ((st = qmv_q8x_bytes(K, batch, &bytes))) return st;
  if (!x) return fail(QMV_ERR_NULL, "x is NULL");
  if (!xq) return fail(QMV_ERR_NULL, "xq is NULL");
  if (!aligned(x, 16)) return fail(QMV_ERR_ALIGN, "x is not 16-byte aligned");
  if (!aligned(xq, 16)) return fail(QMV_ERR_ALIGN, "xq is not 16-byte aligned");
  if (batch * (K / 32) >= (int64_t(1) << 31) * 256)
    return fail(QMV_ERR_OVERFLOW, "too many blocks for one launch");
  if ((st = check_device())) return st;
  return launched(qmv::launch_quantize_x(K, batch, x, static_cast<uint8_t*>(xq), as_stream(stream)),
                  "quantize_x");
}

int qmv_dequant(int fmt, int64_t N, int64_t K, const void* W, float* out, void* stream) {
  int st;
  if ((st = check_fmt(fmt))) return st;
  if ((st = check_shape(fmt, N, K, 1, "batch"))) return st;
  if (!W) return fail(QMV_ERR_NULL, "W is NULL");
  if (!out) return fail(QMV_ERR_NULL, "out is NULL");
  if (!aligned(W, 16)) return fail(QMV_ERR_ALIGN, "W is not 16-byte aligned");
  if (!aligned(out, 16)) return fail(QMV_ERR_ALIGN, "out is not 16-byte aligned");
  if ((N * (K / 32) + 255) / 256 >= (int64_t(1) << 31))
    return fail(QMV_ERR_OVERFLOW, "matrix too large for one dequant launch");
  if ((st = check_device())) return st;
  return launched(qmv::launch_dequant(fmt, N, K, static_cast<const uint8_t*>(W), out, as_stream(stream)),
                  "dequant");
}

}  // extern "C"
