// qmv_dequant: packed matrix -> dense f32 [N][K], bit-exact to the format
// definitions (the correctness baseline's packed-block -> dense conversion,
// pytensor-ml issue 53, PR 15 item F-41).  Not on the hot path.
//
// Each operation is a separate IEEE f32 operation in the normative order;
// floating-point contraction is disabled in this file so that no multiply
// and add fuse into one rounding.
#include "qmv_internal.h"

#pragma clang fp contract(off)

namespace qmv {
namespace {

constexpr int kThreads = 256;

// One thread per 32-weight unit of a row: writes out[n][32u .. 32u+31].
template <int FMT>
__global__ void dequant_units(const uint8_t* __restrict__ W, int64_t off1, int64_t off2,
                              int64_t off3, int64_t N, int64_t K, float* __restrict__ out) {
  const int64_t units = K / 32;
  const int64_t gid = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (gid >= N * units) return;
  const int64_t n = gid / units;
  const int64_t u = gid - n * units;
  float w[32];
  if constexpr (FMT == QMV_Q8_0) {
    const int8_t* qs = reinterpret_cast<const int8_t*>(W) + n * K + 32 * u;
    const uint16_t* sc = reinterpret_cast<const uint16_t*>(W + off1) + n * (K / 32) + u;
    const float s = f16_bits_to_f32(*sc);
    for (int i = 0; i < 32; ++i) w[i] = s * static_cast<float>(qs[i]);
  } else if constexpr (FMT == QMV_W4A16_G64) {
    const uint8_t* qs = W + n * (K / 2) + 16 * u;
    const uint32_t sz = reinterpret_cast<const uint32_t*>(W + off1)[n * (K / 64) + u / 2];
    const float s = f16_bits_to_f32(sz & 0xFFFFu), z = f16_bits_to_f32(sz >> 16);
    for (int i = 0; i < 16; ++i) {
      w[2 * i] = s * (static_cast<float>(qs[i] & 15u) - z);
      w[2 * i + 1] = s * (static_cast<float>(qs[i] >> 4) - z);
    }
  } else if constexpr (FMT == QMV_Q4K) {
    const uint8_t* qs = W + n * (K / 2) + 16 * u;
    const uint32_t* rec = reinterpret_cast<const uint32_t*>(W + off1) + 4 * (n * (K / 256) + u / 8);
    const float d = f16_bits_to_f32(rec[0] & 0xFFFFu), dmin = f16_bits_to_f32(rec[0] >> 16);
    const uint64_t lo = uint64_t(rec[1]) | (uint64_t(rec[2]) << 32);       // bits 0..63 of V
    const uint64_t hi = uint64_t(rec[2] >> 16) | (uint64_t(rec[3]) << 16);  // bits 48..95 of V
    const int j = static_cast<int>(u & 7);
    const float sc = static_cast<float>((lo >> (6 * j)) & 63u);
    const float m = static_cast<float>((hi >> (6 * j)) & 63u);
    const float ds = d * sc, dm = dmin * m;
    for (int i = 0; i < 16; ++i) {
      w[2 * i] = ds * static_cast<float>(qs[i] & 15u) - dm;
      w[2 * i + 1] = ds * static_cast<float>(qs[i] >> 4) - dm;
    }
  } else if constexpr (FMT == QMV_Q4_0 || FMT == QMV_Q5_0 || FMT == QMV_Q5K) {
    const uint8_t* qs = W + n * (K / 2) + 16 * u;
    uint32_t qh = 0;
    if constexpr (FMT != QMV_Q4_0) qh = reinterpret_cast<const uint32_t*>(W + off1)[n * (K / 32) + u];
    float ds, dm, off;
    if constexpr (FMT == QMV_Q5K) {
      const uint32_t* rec = reinterpret_cast<const uint32_t*>(W + off2) + 4 * (n * (K / 256) + u / 8);
      const float d = f16_bits_to_f32(rec[0] & 0xFFFFu), dmin = f16_bits_to_f32(rec[0] >> 16);
      const uint64_t lo = uint64_t(rec[1]) | (uint64_t(rec[2]) << 32);
      const uint64_t hi = uint64_t(rec[2] >> 16) | (uint64_t(rec[3]) << 16);
      const int j = static_cast<int>(u & 7);
      ds = d * static_cast<float>((lo >> (6 * j)) & 63u);
      dm = dmin * static_cast<float>((hi >> (6 * j)) & 63u);
      off = 0.0f;
    } else {
      const int64_t dpl = FMT == QMV_Q4_0 ? off1 : off2;
      ds = f16_bits_to_f32(reinterpret_cast<const uint16_t*>(W + dpl)[n * (K / 32) + u]);
      dm = 0.0f;
      off = FMT == QMV_Q4_0 ? 8.0f : 16.0f;
    }
    for (int k = 0; k < 32; ++k) {
      // fifth bit of weight k = 8i + 2c + e sits at bit 8c + 2i + e of qh
      const int i = k >> 3, c = (k & 7) >> 1, e = k & 1;
      const uint32_t lo4 = (k & 1) ? (qs[k >> 1] >> 4) : (qs[k >> 1] & 15u);
      const uint32_t q = lo4 | (((qh >> (8 * c + 2 * i + e)) & 1u) << 4);
      if constexpr (FMT == QMV_Q5K) w[k] = ds * static_cast<float>(q) - dm;
      else w[k] = ds * (static_cast<float>(q) - off);
    }
  } else if constexpr (FMT == QMV_DENSE_BF16) {
    const uint16_t* b = reinterpret_cast<const uint16_t*>(W) + n * K + 32 * u;
    for (int k = 0; k < 32; ++k) w[k] = bf16_bits_to_f32(b[k]);
  } else if constexpr (FMT == QMV_I8_ROW) {
    const int8_t* qs = reinterpret_cast<const int8_t*>(W) + n * K + 32 * u;
    const float sc = reinterpret_cast<const float*>(W + off1)[n];
    for (int k = 0; k < 32; ++k) w[k] = sc * static_cast<float>(qs[k]);
  } else {  // QMV_Q6K
    const uint8_t* ql = W + n * (K / 2) + 16 * u;
    const uint32_t* qh = reinterpret_cast<const uint32_t*>(W + off1) + n * (K / 16) + 2 * u;
    const int8_t* sv = reinterpret_cast<const int8_t*>(W + off2) + n * (K / 16) + 2 * u;
    const float d = f16_bits_to_f32(reinterpret_cast<const uint16_t*>(W + off3)[n * (K / 256) + u / 8]);
    for (int k = 0; k < 32; ++k) {
      // k within the unit: word t = k / 16 of qh; inside it kk = k % 16 = 8*(f>>1) + 2c + (f&1)
      const int t = k >> 4, kk = k & 15;
      const int c = (kk & 7) >> 1, f = ((kk >> 3) << 1) | (kk & 1);
      const uint32_t lo4 = (k & 1) ? (ql[k >> 1] >> 4) : (ql[k >> 1] & 15u);
      const uint32_t hi2 = (qh[t] >> (8 * c + 2 * f)) & 3u;
      const float q = static_cast<float>(lo4 | (hi2 << 4));
      const float ds = d * static_cast<float>(sv[t]);
      w[k] = ds * (q - 32.0f);
    }
  }
  float4* o = reinterpret_cast<float4*>(out + n * K + 32 * u);
  for (int i = 0; i < 8; ++i) o[i] = make_float4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
}

}  // namespace

hipError_t launch_dequant(int fmt, int64_t N, int64_t K, const uint8_t* W, float* out,
                          hipStream_t s) {
  const Planes p = planes_of(fmt, N, K);
  const int64_t items = N * (K / 32);
  const dim3 grid(static_cast<unsigned>((items + kThreads - 1) / kThreads));
  switch (fmt) {
    case QMV_Q8_0:
      hipLaunchKernelGGL(dequant_units<QMV_Q8_0>, grid, dim3(kThreads), 0, s, W, p.off[1], p.off[2],
                         p.off[3], N, K, out);
      break;
    case QMV_W4A16_G64:
      hipLaunchKernelGGL(dequant_units<QMV_W4A16_G64>, grid, dim3(kThreads), 0, s, W, p.off[1],
                         p.off[2], p.off[3], N, K, out);
      break;
    case QMV_Q4K:
      hipLaunchKernelGGL(dequant_units<QMV_Q4K>, grid, dim3(kThreads), 0, s, W, p.off[1], p.off[2],
                         p.off[3], N, K, out);
      break;
    case QMV_Q6K:
      hipLaunchKernelGGL(dequant_units<QMV_Q6K>, grid, dim3(kThreads), 0, s, W, p.off[1], p.off[2],
                         p.off[3], N, K, out);
      break;
    case QMV_Q4_0:
      hipLaunchKernelGGL(dequant_units<QMV_Q4_0>, grid, dim3(kThreads), 0, s, W, p.off[1], p.off[2],
                         p.off[3], N, K, out);
      break;
    case QMV_Q5_0:
      hipLaunchKernelGGL(dequant_units<QMV_Q5_0>, grid, dim3(kThreads), 0, s, W, p.off[1], p.off[2],
                         p.off[3], N, K, out);
      break;
    case QMV_Q5K:
      hipLaunchKernelGGL(dequant_units<QMV_Q5K>, grid, dim3(kThreads), 0, s, W, p.off[1], p.off[2],
                         p.off[3], N, K, out);
      break;
    case QMV_DENSE_BF16:
      hipLaunchKernelGGL(dequant_units<QMV_DENSE_BF16>, grid, dim3(kThreads), 0, s, W, p.off[1], p.off[2],
                         p.off[3], N, K, out);
      break;
    case QMV_I8_ROW:
      hipLaunchKernelGGL(dequant_units<QMV_I8_ROW>, grid, dim3(kThreads), 0, s, W, p.off[1], p.off[2],
                         p.off[3], N, K, out);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qmv
