// qmv_pack kernels: logical arrays -> packed layout v1.
//
// Integer bit placement only; values are unchanged.  Runs once per matrix,
// outside any decode loop (pytensor-ml issue 53, PR 17: a one-time repack,
// cached and metered; PR 18 acceptance rules: no dequantization or transpose
// inside the token loop).  One thread per output byte / word / record; the
// grid's y dimension walks the stacked matrices.
#include "qmv_internal.h"

namespace qmv {
namespace {

constexpr int kThreads = 256;

inline dim3 grid_for(int64_t items, int64_t batch) {
  int64_t blocks = (items + kThreads - 1) / kThreads;
  return dim3(static_cast<unsigned>(blocks), static_cast<unsigned>(batch));
}

// Byte-wise copy of a plane that keeps its logical layout (q8_0 qs / scale,
// q6k s / d).
__global__ void copy_bytes(const uint8_t* __restrict__ src, int64_t src_stride,
                           uint8_t* __restrict__ dst, int64_t dst_stride, int64_t n) {
  int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= n) return;
  dst[blockIdx.y * dst_stride + i] = src[blockIdx.y * src_stride + i];
}

// Nibble plane: byte j of a row = q[2j] & 15 | (q[2j+1] & 15) << 4.
// Over the flattened [N][K] array this is byte j = q[2j] | q[2j+1] << 4.
__global__ void pack_nibbles(const uint8_t* __restrict__ q, int64_t q_stride,
                             uint8_t* __restrict__ dst, int64_t dst_stride, int64_t nbytes) {
  int64_t j = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (j >= nbytes) return;
  const uint8_t* qb = q + blockIdx.y * q_stride;
  uint32_t lo = qb[2 * j] & 15u, hi = qb[2 * j + 1] & 15u;
  dst[blockIdx.y * dst_stride + j] = static_cast<uint8_t>(lo | (hi << 4));
}

// W4A16 scale/zero words: scale | zero << 16.
__global__ void pack_sz(const uint16_t* __restrict__ scale, const uint16_t* __restrict__ zero,
                        int64_t src_stride, uint32_t* __restrict__ dst, int64_t dst_stride,
                        int64_t nwords) {
  int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= nwords) return;
  int64_t s = blockIdx.y * src_stride + i;
  dst[blockIdx.y * dst_stride + i] = uint32_t(scale[s]) | (uint32_t(zero[s]) << 16);
}

// Q4K meta record per super-block: d, dmin, then 8 six-bit sc and 8 six-bit m
// in a 96-bit little-endian field (sc_j at bit 6j, m_j at bit 48 + 6j).
__global__ void pack_q4k_meta(const uint8_t* __restrict__ sc, const uint8_t* __restrict__ m,
                              const uint16_t* __restrict__ d, const uint16_t* __restrict__ dmin,
                              int64_t nsb, uint4* __restrict__ dst, int64_t dst_stride_rec) {
  int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (t >= nsb) return;
  int64_t base = blockIdx.y * nsb + t;
  const uint8_t* s8 = sc + base * 8;
  const uint8_t* m8 = m + base * 8;
  uint64_t lo48 = 0, hi48 = 0;
  for (int j = 0; j < 8; ++j) {
    lo48 |= uint64_t(s8[j] & 63u) << (6 * j);
    hi48 |= uint64_t(m8[j] & 63u) << (6 * j);
  }
  // 96-bit V = lo48 | hi48 << 48, split into three 32-bit words
  uint32_t w1 = static_cast<uint32_t>(lo48);
  uint32_t w2 = static_cast<uint32_t>(lo48 >> 32) | static_cast<uint32_t>(hi48 << 16);
  uint32_t w3 = static_cast<uint32_t>(hi48 >> 16);
  uint4 rec;
  rec.x = uint32_t(d[base]) | (uint32_t(dmin[base]) << 16);
  rec.y = w1;
  rec.z = w2;
  rec.w = w3;
  dst[blockIdx.y * dst_stride_rec + t] = rec;
}

// Q6K high-bit plane: word t covers 16 weights; bits 8c+2f..8c+2f+1 hold bits
// 4-5 of q[16t + 8*(f>>1) + 2c + (f&1)], so that after splitting a 32-bit word of
// the low-nibble plane into its even and odd nibbles, the matching 2-bit fields
// line up byte for byte.
__global__ void pack_q6k_qh(const uint8_t* __restrict__ q, int64_t q_stride,
                            uint32_t* __restrict__ dst, int64_t dst_stride, int64_t nwords) {
  int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (t >= nwords) return;
  const uint8_t* q16 = q + blockIdx.y * q_stride + 16 * t;
  uint32_t w = 0;
  for (int c = 0; c < 4; ++c)
    for (int f = 0; f < 4; ++f) {
      int k = 8 * (f >> 1) + 2 * c + (f & 1);
      w |= ((uint32_t(q16[k]) >> 4) & 3u) << (8 * c + 2 * f);
    }
  dst[blockIdx.y * dst_stride + t] = w;
}

// Q5_0 / Q5K fifth-bit plane: word t covers 32 weights; bit 8c + 2i + e holds
// bit 4 of q[32t + 8i + 2c + e], so that after splitting a 32-bit word of the
// low-nibble plane into its even and odd nibbles (e = 0 / 1), the fifth bits
// of word i are (qh >> (2i + e)) & 0x01010101, byte for byte.
__global__ void pack_q5_qh(const uint8_t* __restrict__ q, int64_t q_stride,
                           uint32_t* __restrict__ dst, int64_t dst_stride, int64_t nwords) {
  int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (t >= nwords) return;
  const uint8_t* q32 = q + blockIdx.y * q_stride + 32 * t;
  uint32_t w = 0;
  for (int i = 0; i < 4; ++i)
    for (int c = 0; c < 4; ++c)
      for (int e = 0; e < 2; ++e) w |= ((uint32_t(q32[8 * i + 2 * c + e]) >> 4) & 1u) << (8 * c + 2 * i + e);
  dst[blockIdx.y * dst_stride + t] = w;
}

}  // namespace

hipError_t launch_pack(int fmt, int64_t N, int64_t K, int64_t batch, const qmv_logical& src,
                       uint8_t* dst, hipStream_t s) {
  const Planes p = planes_of(fmt, N, K);
  const int64_t NK = N * K;
  const uint8_t* q = static_cast<const uint8_t*>(src.q);
  switch (fmt) {
    case QMV_Q8_0: {
      hipLaunchKernelGGL(copy_bytes, grid_for(NK, batch), dim3(kThreads), 0, s, q, NK,
                         dst + p.off[0], p.total, NK);
      const int64_t nb = N * (K / 32) * 2;
      hipLaunchKernelGGL(copy_bytes, grid_for(nb, batch), dim3(kThreads), 0, s,
                         static_cast<const uint8_t*>(src.aux[0]), nb, dst + p.off[1], p.total, nb);
      break;
    }
    case QMV_W4A16_G64: {
      hipLaunchKernelGGL(pack_nibbles, grid_for(NK / 2, batch), dim3(kThreads), 0, s, q, NK,
                         dst + p.off[0], p.total, NK / 2);
      const int64_t ng = N * (K / 64);
      // dst stride in 32-bit words: p.total is a multiple of 256, so this is exact
      hipLaunchKernelGGL(pack_sz, grid_for(ng, batch), dim3(kThreads), 0, s,
                         static_cast<const uint16_t*>(src.aux[0]),
                         static_cast<const uint16_t*>(src.aux[1]), ng,
                         reinterpret_cast<uint32_t*>(dst + p.off[1]), p.total / 4, ng);
      break;
    }
    case QMV_Q4K: {
      hipLaunchKernelGGL(pack_nibbles, grid_for(NK / 2, batch), dim3(kThreads), 0, s, q, NK,
                         dst + p.off[0], p.total, NK / 2);
      const int64_t nsb = N * (K / 256);
      hipLaunchKernelGGL(pack_q4k_meta, grid_for(nsb, batch), dim3(kThreads), 0, s,
                         static_cast<const uint8_t*>(src.aux[0]),
                         static_cast<const uint8_t*>(src.aux[1]),
                         static_cast<const uint16_t*>(src.aux[2]),
                         static_cast<const uint16_t*>(src.aux[3]), nsb,
                         reinterpret_cast<uint4*>(dst + p.off[1]), p.total / 16);
      break;
    }
    case QMV_Q6K: {
      hipLaunchKernelGGL(pack_nibbles, grid_for(NK / 2, batch), dim3(kThreads), 0, s, q, NK,
                         dst + p.off[0], p.total, NK / 2);
      hipLaunchKernelGGL(pack_q6k_qh, grid_for(NK / 16, batch), dim3(kThreads), 0, s, q, NK,
                         reinterpret_cast<uint32_t*>(dst + p.off[1]), p.total / 4, NK / 16);
      const int64_t ns = N * (K / 16);
      hipLaunchKernelGGL(copy_bytes, grid_for(ns, batch), dim3(kThreads), 0, s,
                         static_cast<const uint8_t*>(src.aux[0]), ns, dst + p.off[2], p.total, ns);
      const int64_t nd = N * (K / 256) * 2;
      hipLaunchKernelGGL(copy_bytes, grid_for(nd, batch), dim3(kThreads), 0, s,
                         static_cast<const uint8_t*>(src.aux[1]), nd, dst + p.off[3], p.total, nd);
      break;
    }
    case QMV_Q4_0:
    case QMV_Q5_0:
    case QMV_Q5K: {
      hipLaunchKernelGGL(pack_nibbles, grid_for(NK / 2, batch), dim3(kThreads), 0, s, q, NK,
                         dst + p.off[0], p.total, NK / 2);
      int plane = 1;
      if (fmt != QMV_Q4_0) {
        hipLaunchKernelGGL(pack_q5_qh, grid_for(NK / 32, batch), dim3(kThreads), 0, s, q, NK,
                           reinterpret_cast<uint32_t*>(dst + p.off[1]), p.total / 4, NK / 32);
        plane = 2;
      }
      if (fmt == QMV_Q5K) {
        const int64_t nsb = N * (K / 256);
        hipLaunchKernelGGL(pack_q4k_meta, grid_for(nsb, batch), dim3(kThreads), 0, s,
                           static_cast<const uint8_t*>(src.aux[0]),
                           static_cast<const uint8_t*>(src.aux[1]),
                           static_cast<const uint16_t*>(src.aux[2]),
                           static_cast<const uint16_t*>(src.aux[3]), nsb,
                           reinterpret_cast<uint4*>(dst + p.off[2]), p.total / 16);
      } else {
        const int64_t nd = N * (K / 32) * 2;
        hipLaunchKernelGGL(copy_bytes, grid_for(nd, batch), dim3(kThreads), 0, s,
                           static_cast<const uint8_t*>(src.aux[0]), nd, dst + p.off[plane], p.total, nd);
      }
      break;
    }
    case QMV_DENSE_BF16:
      hipLaunchKernelGGL(copy_bytes, grid_for(2 * NK, batch), dim3(kThreads), 0, s, q, 2 * NK,
                         dst + p.off[0], p.total, 2 * NK);
      break;
    case QMV_I8_ROW:
      hipLaunchKernelGGL(copy_bytes, grid_for(NK, batch), dim3(kThreads), 0, s, q, NK, dst + p.off[0], p.total, NK);
      hipLaunchKernelGGL(copy_bytes, grid_for(4 * N, batch), dim3(kThreads), 0, s,
                         static_cast<const uint8_t*>(src.aux[0]), 4 * N, dst + p.off[1], p.total, 4 * N);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qmv
