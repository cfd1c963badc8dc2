// Decode matvec y = W x straight from packed blocks, batch 1..8 per pass.
//
// The pages' GPU decode path multiplies f32 activations against weights that
// are dequantized on the fly, and its matrix-vector kernels are bound by their
// vector loads (aot-llm README, Metal backend notes); batched prompts decode
// each quantized block once and use it for several activations (aot-llm
// README, "Batched prompt processing" and the 1x4 micro-kernel notes).
//
// gfx950 mapping.  Rows are split across 64-lane wavefronts; inside a wave,
// LPR lanes (64, 32 or 16) share one row and each lane streams 16-byte units
// of the row's quant plane with one 128-bit load, so a wave-wide load reads
// 1 KiB of contiguous HBM (64/LPR consecutive rows back to back).  A unit is
// 32 weights: one Q4K sub-block, half a W4A16 group, two Q6K sub-blocks,
// one Q8_0 block (two loads).  Nibbles and 2-bit fields are unpacked in
// registers; block scales / mins are applied once per unit in f32, with the
// integer part factored out of the inner product:
//   Q8_0   s * sum q x
//   W4A16  s * (sum q x - z * sum x)
//   Q4K    (d sc) * sum q x - (dmin m) * sum x
//   Q6K    (d s_j) * (sum q x - 32 sum x)       per 16-weight sub-block
// With fp16 activations, W4A16 uses packed fp16 dot products: a nibble q
// becomes the exact fp16 value 1024 + q by OR-ing it into 0x6400, and the
// 1024 offset is folded into the zero term.  Each lane's partial sums for
// R rows x B vectors are then reduced across the LPR lanes of the row with a
// butterfly that halves the value count at every step, so the reduction costs
// about R*B + log2(LPR) cross-lane exchanges instead of R*B*log2(LPR).

#include "qmv_internal.h"

namespace qmv {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kThreads = 64 * kWavesPerBlock;

typedef __attribute__((ext_vector_type(2))) _Float16 half2_t;

__device__ __forceinline__ float byte_f32(uint32_t v, int c) {
  return static_cast<float>((v >> (8 * c)) & 0xFFu);  // v_cvt_f32_ubyteN
}

__device__ __forceinline__ float sbyte_f32(uint32_t v, int c) {
  return static_cast<float>(static_cast<int32_t>(v << (24 - 8 * c)) >> 24);
}

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// Reduce V values across groups of LPR lanes.  Afterwards lane l holds the
// group total of value index (l % LPR) / (LPR / V) in v[0].
template <int V, int LPR>
__device__ __forceinline__ void reduce_rows(float (&v)[V], int lane) {
  static_assert((V & (V - 1)) == 0 && V <= LPR, "V must be a power of two <= LPR");
  int dist = LPR / 2;
#pragma unroll
  for (int C = V; C > 1; C >>= 1, dist >>= 1) {
    const bool upper = (lane & dist) != 0;
#pragma unroll
    for (int i = 0; i < C / 2; ++i) {
      const float lo = v[i], hi = v[i + C / 2];
      const float send = upper ? lo : hi;
      const float keep = upper ? hi : lo;
      v[i] = keep + shfl_xor_f(send, dist);
    }
  }
#pragma unroll
  for (; dist >= 1; dist >>= 1) v[0] += shfl_xor_f(v[0], dist);
}

template <int N_>
struct Pow2Ceil {
  static constexpr int value = N_ <= 1 ? 1 : N_ <= 2 ? 2 : N_ <= 4 ? 4 : N_ <= 8 ? 8 : 16;
};

// FMT: format; XF16: activations are fp16 (else f32); LPR: lanes per row;
// B: vectors per pass; R: rows per lane group.
// PAIR: SwiGLU, y = silu(W x) * (W2 x) (W2 the up matrix, same format and
// shape); otherwise bias [N] and res [nb][N] (null: none) are added in the
// epilogue: y = res + (W x + bias).
// XQ8: x is a QMV_Q8X buffer (8-bit codes and an f32 scale per 32 activations):
// every 32-weight unit is one or two integer dot products (v_dot4_i32_i8,
// exact in int32) scaled back in f32.
template <int FMT, bool XF16, int LPR, int B, int R, bool PAIR = false, bool XQ8 = false>
__global__ __launch_bounds__(kThreads) void matvec_kernel(
    const uint8_t* __restrict__ W, int64_t off1, int64_t off2, int64_t off3,
    const void* __restrict__ xv, float* __restrict__ y, int N, int K, int nb,
    const uint8_t* __restrict__ W2, const float* __restrict__ bias, const float* res) {
  constexpr int RPW = 64 / LPR;  // rows side by side in one wave
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPR;
  const int l = lane % LPR;
  const int wave = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int base = wave * (R * RPW);
  if (base >= N) return;  // whole wave leaves together; no block-level barrier follows
  const int U = K >> 5;   // 32-weight units per row

  int row[R];
#pragma unroll
  for (int r = 0; r < R; ++r) row[r] = min(base + r * RPW + sub, N - 1);

  float acc[R][B];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;

  [[maybe_unused]] const int64_t xrec = (K + K / 8 + 15) / 16 * 16;  // bytes per Q8X vector
  auto units = [&](const uint8_t* __restrict__ W, float (&acc)[R][B]) {
#pragma unroll 2
    for (int u = l; u < U; u += LPR) {
      if constexpr (XQ8) {
        constexpr bool I8 = FMT == QMV_Q8_0 || FMT == QMV_I8_ROW;
        uint4 q[R][2];
        float sA[R], mA[R], sB[R];
        uint2 qh6[R];
        uint32_t qh5[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int64_t rw = row[r];
          if constexpr (I8) {
            const uint4* p = reinterpret_cast<const uint4*>(W + rw * K) + 2 * u;
            q[r][0] = p[0];
            q[r][1] = p[1];
            sA[r] = FMT == QMV_Q8_0 ? f16_bits_to_f32(reinterpret_cast<const uint16_t*>(W + off1)[rw * (K >> 5) + u])
                                    : reinterpret_cast<const float*>(W + off1)[rw];
          } else {
            q[r][0] = reinterpret_cast<const uint4*>(W + rw * (K >> 1))[u];
            if constexpr (FMT == QMV_Q5_0 || FMT == QMV_Q5K)
              qh5[r] = reinterpret_cast<const uint32_t*>(W + off1)[rw * (K >> 5) + u];
            if constexpr (FMT == QMV_W4A16_G64) {
              const uint32_t sz = reinterpret_cast<const uint32_t*>(W + off1)[rw * (K >> 6) + (u >> 1)];
              sA[r] = f16_bits_to_f32(sz & 0xFFFFu);
              mA[r] = f16_bits_to_f32(sz >> 16);
            } else if constexpr (FMT == QMV_Q4_0 || FMT == QMV_Q5_0) {
              const int64_t dpl = FMT == QMV_Q4_0 ? off1 : off2;
              sA[r] = f16_bits_to_f32(reinterpret_cast<const uint16_t*>(W + dpl)[rw * (K >> 5) + u]);
            } else if constexpr (FMT == QMV_Q4K || FMT == QMV_Q5K) {
              const uint4 rec = reinterpret_cast<const uint4*>(W + (FMT == QMV_Q4K ? off1 : off2))[rw * (K >> 8) + (u >> 3)];
              const int j = u & 7;
              const uint64_t lo = uint64_t(rec.y) | (uint64_t(rec.z) << 32);
              const uint64_t hi = uint64_t(rec.z >> 16) | (uint64_t(rec.w) << 16);
              sA[r] = f16_bits_to_f32(rec.x & 0xFFFFu) * static_cast<float>(static_cast<uint32_t>(lo >> (6 * j)) & 63u);
              mA[r] = f16_bits_to_f32(rec.x >> 16) * static_cast<float>(static_cast<uint32_t>(hi >> (6 * j)) & 63u);
            } else if constexpr (FMT == QMV_Q6K) {
              qh6[r] = reinterpret_cast<const uint2*>(W + off1)[rw * (K >> 5) + u];
              const uint32_t s2 = reinterpret_cast<const uint16_t*>(W + off2)[rw * (K >> 5) + u];
              const float d = f16_bits_to_f32(reinterpret_cast<const uint16_t*>(W + off3)[rw * (K >> 8) + (u >> 3)]);
              sA[r] = d * static_cast<float>(static_cast<int8_t>(s2 & 0xFFu));
              sB[r] = d * static_cast<float>(static_cast<int8_t>(s2 >> 8));
            }
          }
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const int bb = min(b, nb - 1);
          const uint8_t* xr = static_cast<const uint8_t*>(xv) + int64_t(bb) * xrec;
          const uint4 x0 = reinterpret_cast<const uint4*>(xr)[2 * u], x1 = reinterpret_cast<const uint4*>(xr)[2 * u + 1];
          const float dx = reinterpret_cast<const float*>(xr + K)[u];
          const int xw[8] = {int(x0.x), int(x0.y), int(x0.z), int(x0.w), int(x1.x), int(x1.y), int(x1.z), int(x1.w)};
          int sxA = 0, sxB = 0;  // code sums (Q6K: the two 16-weight halves)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if (FMT == QMV_Q6K && j >= 4) sxB = __builtin_amdgcn_sdot4(xw[j], 0x01010101, sxB, false);
            else sxA = __builtin_amdgcn_sdot4(xw[j], 0x01010101, sxA, false);
          }
#pragma unroll
          for (int r = 0; r < R; ++r) {
            if constexpr (I8) {
              const int ww[8] = {int(q[r][0].x), int(q[r][0].y), int(q[r][0].z), int(q[r][0].w),
                                 int(q[r][1].x), int(q[r][1].y), int(q[r][1].z), int(q[r][1].w)};
              int dot = 0;
#pragma unroll
              for (int j = 0; j < 8; ++j) dot = __builtin_amdgcn_sdot4(ww[j], xw[j], dot, false);
              acc[r][b] = fmaf(sA[r] * dx, static_cast<float>(dot), acc[r][b]);
            } else {
              int dA = 0, dB = 0;
              const uint32_t wq[4] = {q[r][0].x, q[r][0].y, q[r][0].z, q[r][0].w};
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                uint32_t ev = wq[i] & 0x0F0F0F0Fu, od = (wq[i] >> 4) & 0x0F0F0F0Fu;
                if constexpr (FMT == QMV_Q6K) {
                  const uint32_t h = (i >> 1) ? qh6[r].y : qh6[r].x;
                  const int f = (i & 1) * 2;
                  ev |= ((h >> (2 * f)) & 0x03030303u) << 4;
                  od |= ((h >> (2 * f + 2)) & 0x03030303u) << 4;
                } else if constexpr (FMT == QMV_Q5_0 || FMT == QMV_Q5K) {
                  ev |= ((qh5[r] >> (2 * i)) & 0x01010101u) << 4;
                  od |= ((qh5[r] >> (2 * i + 1)) & 0x01010101u) << 4;
                }
                // activation codes in the same even / odd split of k = 8i .. 8i + 7
                const int xe = int(__builtin_amdgcn_perm(uint32_t(xw[2 * i + 1]), uint32_t(xw[2 * i]), 0x06040200u));
                const int xo = int(__builtin_amdgcn_perm(uint32_t(xw[2 * i + 1]), uint32_t(xw[2 * i]), 0x07050301u));
                int& d = (FMT == QMV_Q6K && i >= 2) ? dB : dA;
                d = __builtin_amdgcn_sdot4(int(ev), xe, d, false);
                d = __builtin_amdgcn_sdot4(int(od), xo, d, false);
              }
              float c;
              if constexpr (FMT == QMV_W4A16_G64) c = sA[r] * fmaf(-mA[r], static_cast<float>(sxA), static_cast<float>(dA));
              else if constexpr (FMT == QMV_Q4_0) c = sA[r] * static_cast<float>(dA - 8 * sxA);
              else if constexpr (FMT == QMV_Q5_0) c = sA[r] * static_cast<float>(dA - 16 * sxA);
              else if constexpr (FMT == QMV_Q4K || FMT == QMV_Q5K)
                c = fmaf(sA[r], static_cast<float>(dA), -mA[r] * static_cast<float>(sxA));
              else c = fmaf(sA[r], static_cast<float>(dA - 32 * sxA), sB[r] * static_cast<float>(dB - 32 * sxB));
              acc[r][b] = fmaf(dx, c, acc[r][b]);
            }
          }
        }
      } else if constexpr (FMT == QMV_Q8_0 || FMT == QMV_I8_ROW) {

        uint4 q[R][2];
        float s[R];
  #pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint4* p = reinterpret_cast<const uint4*>(W + int64_t(row[r]) * K) + 2 * u;
          q[r][0] = p[0];
          q[r][1] = p[1];
          if constexpr (FMT == QMV_Q8_0)
            s[r] = f16_bits_to_f32(reinterpret_cast<const uint16_t*>(W + off1)[int64_t(row[r]) * (K >> 5) + u]);
          else
            s[r] = reinterpret_cast<const float*>(W + off1)[row[r]];
        }
  #pragma unroll
        for (int b = 0; b < B; ++b) {
          const int bb = min(b, nb - 1);
          const float4* xp = reinterpret_cast<const float4*>(static_cast<const float*>(xv) + int64_t(bb) * K) + 8 * u;
          float qx[R];
  #pragma unroll
          for (int r = 0; r < R; ++r) qx[r] = 0.0f;
  #pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float4 xx = xp[i];
            const float xa[4] = {xx.x, xx.y, xx.z, xx.w};
  #pragma unroll
            for (int r = 0; r < R; ++r) {
              const uint4 qq = q[r][i >> 2];
              const uint32_t wd = (i & 3) == 0 ? qq.x : (i & 3) == 1 ? qq.y : (i & 3) == 2 ? qq.z : qq.w;
  #pragma unroll
              for (int c = 0; c < 4; ++c) qx[r] = fmaf(sbyte_f32(wd, c), xa[c], qx[r]);
            }
          }
  #pragma unroll
          for (int r = 0; r < R; ++r) acc[r][b] = fmaf(s[r], qx[r], acc[r][b]);
        }
      } else if constexpr (FMT == QMV_DENSE_BF16) {
        uint4 q[R][4];
  #pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint4* p = reinterpret_cast<const uint4*>(W + (int64_t(row[r]) * K + 32 * u) * 2);
  #pragma unroll
          for (int i = 0; i < 4; ++i) q[r][i] = p[i];
        }
  #pragma unroll
        for (int b = 0; b < B; ++b) {
          const int bb = min(b, nb - 1);
          const float4* xp = reinterpret_cast<const float4*>(static_cast<const float*>(xv) + int64_t(bb) * K) + 8 * u;
  #pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float4 xx = xp[i];  // x[4i .. 4i + 3]: weights 4i .. 4i + 3 are words 2 (i % 2), +1 of q[i / 2]
  #pragma unroll
            for (int r = 0; r < R; ++r) {
              const uint4 qq = q[r][i >> 1];
              const uint32_t w0 = (i & 1) ? qq.z : qq.x, w1 = (i & 1) ? qq.w : qq.y;
              float t = acc[r][b];
              t = fmaf(__builtin_bit_cast(float, w0 << 16), xx.x, t);
              t = fmaf(__builtin_bit_cast(float, w0 & 0xFFFF0000u), xx.y, t);
              t = fmaf(__builtin_bit_cast(float, w1 << 16), xx.z, t);
              t = fmaf(__builtin_bit_cast(float, w1 & 0xFFFF0000u), xx.w, t);
              acc[r][b] = t;
            }
          }
        }
      } else if constexpr (FMT == QMV_W4A16_G64 && XF16) {
        uint4 q[R];
        uint32_t sz[R];
  #pragma unroll
        for (int r = 0; r < R; ++r) {
          q[r] = reinterpret_cast<const uint4*>(W + int64_t(row[r]) * (K >> 1))[u];
          sz[r] = reinterpret_cast<const uint32_t*>(W + off1)[int64_t(row[r]) * (K >> 6) + (u >> 1)];
        }
  #pragma unroll
        for (int b = 0; b < B; ++b) {
          const int bb = min(b, nb - 1);
          const uint4* xp = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(xv) + int64_t(bb) * K) + 4 * u;
          float qx[R], sx = 0.0f;
  #pragma unroll
          for (int r = 0; r < R; ++r) qx[r] = 0.0f;
          const half2_t one2 = as_h2(0x3C003C00u);
  #pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint4 xx = xp[i];  // x[8i .. 8i+7] as fp16 pairs (01)(23)(45)(67)
            // pairs matching the nibble split below: (x0,x4) (x1,x5) (x2,x6) (x3,x7)
            const half2_t p04 = as_h2(__builtin_amdgcn_perm(xx.z, xx.x, 0x05040100u));
            const half2_t p15 = as_h2(__builtin_amdgcn_perm(xx.z, xx.x, 0x07060302u));
            const half2_t p26 = as_h2(__builtin_amdgcn_perm(xx.w, xx.y, 0x05040100u));
            const half2_t p37 = as_h2(__builtin_amdgcn_perm(xx.w, xx.y, 0x07060302u));
            sx = __builtin_amdgcn_fdot2(p04, one2, sx, false);
            sx = __builtin_amdgcn_fdot2(p15, one2, sx, false);
            sx = __builtin_amdgcn_fdot2(p26, one2, sx, false);
            sx = __builtin_amdgcn_fdot2(p37, one2, sx, false);
  #pragma unroll
            for (int r = 0; r < R; ++r) {
              const uint32_t wd = i == 0 ? q[r].x : i == 1 ? q[r].y : i == 2 ? q[r].z : q[r].w;
              // word wd holds k = 8i..8i+7 as nibbles: byte c = q[2c] | q[2c+1] << 4;
              // (wd >> 4j) & 0x000F000F picks k = j (low half) and k = j + 4 (high half)
              const half2_t h0 = as_h2((wd & 0x000F000Fu) | 0x64006400u);
              const half2_t h1 = as_h2(((wd >> 4) & 0x000F000Fu) | 0x64006400u);
              const half2_t h2 = as_h2(((wd >> 8) & 0x000F000Fu) | 0x64006400u);
              const half2_t h3 = as_h2(((wd >> 12) & 0x000F000Fu) | 0x64006400u);
              qx[r] = __builtin_amdgcn_fdot2(h0, p04, qx[r], false);
              qx[r] = __builtin_amdgcn_fdot2(h1, p15, qx[r], false);
              qx[r] = __builtin_amdgcn_fdot2(h2, p26, qx[r], false);
              qx[r] = __builtin_amdgcn_fdot2(h3, p37, qx[r], false);
            }
          }
  #pragma unroll
          for (int r = 0; r < R; ++r) {
            const float s = f16_bits_to_f32(sz[r] & 0xFFFFu);
            const float zo = 1024.0f + f16_bits_to_f32(sz[r] >> 16);  // exact
            acc[r][b] = fmaf(s, fmaf(-zo, sx, qx[r]), acc[r][b]);
          }
        }
      } else {
        // 4-bit and 6-bit formats with f32 (or fp16-converted) activations
        uint4 q[R];
        float sA[R], mA[R];          // per-unit multiplier of sum q x, and of sum x
        float sB[R];                 // Q6K: second sub-block's multiplier
        uint2 qh[R];
        uint32_t qh5[R];             // Q5_0 / Q5K fifth bits of the unit
  #pragma unroll
        for (int r = 0; r < R; ++r) {
          q[r] = reinterpret_cast<const uint4*>(W + int64_t(row[r]) * (K >> 1))[u];
          if constexpr (FMT == QMV_Q5_0 || FMT == QMV_Q5K)
            qh5[r] = reinterpret_cast<const uint32_t*>(W + off1)[int64_t(row[r]) * (K >> 5) + u];
          if constexpr (FMT == QMV_Q4_0 || FMT == QMV_Q5_0) {
            const int64_t dpl = FMT == QMV_Q4_0 ? off1 : off2;
            sA[r] = f16_bits_to_f32(reinterpret_cast<const uint16_t*>(W + dpl)[int64_t(row[r]) * (K >> 5) + u]);
            mA[r] = FMT == QMV_Q4_0 ? 8.0f : 16.0f;
          } else if constexpr (FMT == QMV_W4A16_G64) {
            const uint32_t sz = reinterpret_cast<const uint32_t*>(W + off1)[int64_t(row[r]) * (K >> 6) + (u >> 1)];
            sA[r] = f16_bits_to_f32(sz & 0xFFFFu);
            mA[r] = f16_bits_to_f32(sz >> 16);
          } else if constexpr (FMT == QMV_Q4K || FMT == QMV_Q5K) {
            const uint4 rec = reinterpret_cast<const uint4*>(W + (FMT == QMV_Q4K ? off1 : off2))[int64_t(row[r]) * (K >> 8) + (u >> 3)];
            const int j = u & 7;
            const uint64_t lo = uint64_t(rec.y) | (uint64_t(rec.z) << 32);
            const uint64_t hi = uint64_t(rec.z >> 16) | (uint64_t(rec.w) << 16);
            const float sc = static_cast<float>(static_cast<uint32_t>(lo >> (6 * j)) & 63u);
            const float m = static_cast<float>(static_cast<uint32_t>(hi >> (6 * j)) & 63u);
            sA[r] = f16_bits_to_f32(rec.x & 0xFFFFu) * sc;
            mA[r] = f16_bits_to_f32(rec.x >> 16) * m;
          } else {  // Q6K
            qh[r] = reinterpret_cast<const uint2*>(W + off1)[int64_t(row[r]) * (K >> 5) + u];
            const uint32_t s2 = reinterpret_cast<const uint16_t*>(W + off2)[int64_t(row[r]) * (K >> 5) + u];
            const float d = f16_bits_to_f32(reinterpret_cast<const uint16_t*>(W + off3)[int64_t(row[r]) * (K >> 8) + (u >> 3)]);
            sA[r] = d * static_cast<float>(static_cast<int8_t>(s2 & 0xFFu));
            sB[r] = d * static_cast<float>(static_cast<int8_t>(s2 >> 8));
          }
        }
  #pragma unroll
        for (int b = 0; b < B; ++b) {
          const int bb = min(b, nb - 1);
          float qx[R][2], sx[2] = {0.0f, 0.0f};
  #pragma unroll
          for (int r = 0; r < R; ++r) qx[r][0] = qx[r][1] = 0.0f;
  #pragma unroll
          for (int i = 0; i < 4; ++i) {
            float xa[8];
            if constexpr (XF16) {
              const uint4 xx = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(xv) + int64_t(bb) * K)[4 * u + i];
              const uint32_t xw[4] = {xx.x, xx.y, xx.z, xx.w};
  #pragma unroll
              for (int c = 0; c < 4; ++c) {
                xa[2 * c] = f16_bits_to_f32(xw[c] & 0xFFFFu);
                xa[2 * c + 1] = f16_bits_to_f32(xw[c] >> 16);
              }
            } else {
              const float4* xp = reinterpret_cast<const float4*>(static_cast<const float*>(xv) + int64_t(bb) * K) + 8 * u + 2 * i;
              const float4 x0 = xp[0], x1 = xp[1];
              xa[0] = x0.x; xa[1] = x0.y; xa[2] = x0.z; xa[3] = x0.w;
              xa[4] = x1.x; xa[5] = x1.y; xa[6] = x1.z; xa[7] = x1.w;
            }
            const int part = (FMT == QMV_Q6K) ? (i >> 1) : 0;
            sx[part] += ((xa[0] + xa[1]) + (xa[2] + xa[3])) + ((xa[4] + xa[5]) + (xa[6] + xa[7]));
  #pragma unroll
            for (int r = 0; r < R; ++r) {
              const uint32_t wd = i == 0 ? q[r].x : i == 1 ? q[r].y : i == 2 ? q[r].z : q[r].w;
              uint32_t ev = wd & 0x0F0F0F0Fu;         // byte c: q[8i + 2c]
              uint32_t od = (wd >> 4) & 0x0F0F0F0Fu;  // byte c: q[8i + 2c + 1]
              if constexpr (FMT == QMV_Q6K) {
                const uint32_t h = (i >> 1) ? qh[r].y : qh[r].x;
                const int f = (i & 1) * 2;
                ev |= ((h >> (2 * f)) & 0x03030303u) << 4;
                od |= ((h >> (2 * f + 2)) & 0x03030303u) << 4;
              } else if constexpr (FMT == QMV_Q5_0 || FMT == QMV_Q5K) {
                ev |= ((qh5[r] >> (2 * i)) & 0x01010101u) << 4;
                od |= ((qh5[r] >> (2 * i + 1)) & 0x01010101u) << 4;
              }
              float t = qx[r][part];
  #pragma unroll
              for (int c = 0; c < 4; ++c) {
                t = fmaf(byte_f32(ev, c), xa[2 * c], t);
                t = fmaf(byte_f32(od, c), xa[2 * c + 1], t);
              }
              qx[r][part] = t;
            }
          }
  #pragma unroll
          for (int r = 0; r < R; ++r) {
            if constexpr (FMT == QMV_W4A16_G64 || FMT == QMV_Q4_0 || FMT == QMV_Q5_0) {
              acc[r][b] = fmaf(sA[r], fmaf(-mA[r], sx[0], qx[r][0]), acc[r][b]);
            } else if constexpr (FMT == QMV_Q4K || FMT == QMV_Q5K) {
              acc[r][b] = fmaf(sA[r], qx[r][0], acc[r][b]);
              acc[r][b] = fmaf(-mA[r], sx[0], acc[r][b]);
            } else {  // Q6K
              acc[r][b] = fmaf(sA[r], fmaf(-32.0f, sx[0], qx[r][0]), acc[r][b]);
              acc[r][b] = fmaf(sB[r], fmaf(-32.0f, sx[1], qx[r][1]), acc[r][b]);
            }
          }
        }
      }
    }
  };
  units(W, acc);
  constexpr int NM = PAIR ? 2 : 1;
  [[maybe_unused]] float acc2[R][B];
  if constexpr (PAIR) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int b = 0; b < B; ++b) acc2[r][b] = 0.0f;
    units(W2, acc2);
  }

  // cross-lane reduction of the R*B (x2 with PAIR) partial sums of each row group
  constexpr int RB = R * B;
  constexpr int V = Pow2Ceil<RB * NM>::value;
  float v[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    if constexpr (PAIR) v[i] = i < RB ? acc[i / B][i % B] : i < 2 * RB ? acc2[(i - RB) / B][(i - RB) % B] : 0.0f;
    else v[i] = (i < RB) ? acc[i / B][i % B] : 0.0f;
  }
  reduce_rows<V, LPR>(v, lane);
  constexpr int span = LPR / V;
  // the up total of value idx sits RB spans further in the same row group
  const float up = PAIR ? __shfl(v[0], min(lane + RB * span, 63), 64) : 0.0f;
  if ((l % span) == 0) {
    const int idx = l / span;
    if (idx < RB) {
      const int r = idx / B, b = idx % B;
      const int rr = base + r * RPW + sub;
      if (rr < N && b < nb) {
        float out;
        if constexpr (PAIR) {
          out = silu_mul(v[0], up);
        } else {
          out = v[0];
          if (bias) out += bias[rr];
          if (res) out = res[int64_t(b) * N + rr] + out;
        }
        y[int64_t(b) * N + rr] = out;
      }
    }
  }
}

struct EpiArgs {
  const uint8_t* W2;
  const float* bias;
  const float* res;
};

template <int FMT, bool XF16, int LPR, int B, int R, bool XQ8>
hipError_t go(const uint8_t* W, const Planes& p, const void* x, float* y, int N, int K, int nb,
              const EpiArgs& e, hipStream_t s) {
  constexpr int rows_per_wave = R * (64 / LPR);
  const int waves = (N + rows_per_wave - 1) / rows_per_wave;
  const int blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
  if (e.W2)
    hipLaunchKernelGGL((matvec_kernel<FMT, XF16, LPR, B, R, true, XQ8>), dim3(blocks), dim3(kThreads), 0, s, W,
                       p.off[1], p.off[2], p.off[3], x, y, N, K, nb, e.W2, nullptr, nullptr);
  else
    hipLaunchKernelGGL((matvec_kernel<FMT, XF16, LPR, B, R, false, XQ8>), dim3(blocks), dim3(kThreads), 0, s, W,
                       p.off[1], p.off[2], p.off[3], x, y, N, K, nb, nullptr, e.bias, e.res);
  return hipGetLastError();
}

template <int FMT, bool XF16, int LPR, bool XQ8>
hipError_t pick_br(const uint8_t* W, const Planes& p, const void* x, float* y, int N, int K,
                   int nb, const EpiArgs& e, hipStream_t s) {
  // Two rows per lane group once there are enough rows to keep ~8 waves per CU.
  const bool two = (int64_t(N) * LPR) / 64 >= 8 * 256 * 2;
  if (nb <= 1) return two ? go<FMT, XF16, LPR, 1, 2, XQ8>(W, p, x, y, N, K, nb, e, s)
                          : go<FMT, XF16, LPR, 1, 1, XQ8>(W, p, x, y, N, K, nb, e, s);
  if (nb <= 2) return two ? go<FMT, XF16, LPR, 2, 2, XQ8>(W, p, x, y, N, K, nb, e, s)
                          : go<FMT, XF16, LPR, 2, 1, XQ8>(W, p, x, y, N, K, nb, e, s);
  if (nb <= 4) return two ? go<FMT, XF16, LPR, 4, 2, XQ8>(W, p, x, y, N, K, nb, e, s)
                          : go<FMT, XF16, LPR, 4, 1, XQ8>(W, p, x, y, N, K, nb, e, s);
  return go<FMT, XF16, LPR, 8, 1, XQ8>(W, p, x, y, N, K, nb, e, s);
}

template <int FMT, bool XF16, bool XQ8 = false>
hipError_t pick_lpr(const uint8_t* W, const Planes& p, const void* x, float* y, int N, int K,
                    int nb, const EpiArgs& e, hipStream_t s) {
  // Lanes per row: a whole wave per row once a row has >= 64 units (a ragged
  // last pass costs less than the parallelism lost by packing more rows into
  // a wave); shorter rows share the wave so every lane still has a unit.
  const int U = K / 32;
  if (U >= 64) return pick_br<FMT, XF16, 64, XQ8>(W, p, x, y, N, K, nb, e, s);
  if (U > 16) return pick_br<FMT, XF16, 32, XQ8>(W, p, x, y, N, K, nb, e, s);
  return pick_br<FMT, XF16, 16, XQ8>(W, p, x, y, N, K, nb, e, s);
}

}  // namespace

namespace {
// A/B comparison only: QMV_MATVEC_MFMA=0 sends batch >= 2 to the FMA kernel,
// =2 also sends batch 1 to the matrix-core kernel.
int mfma_mode() {
  static const int v = [] {
    return ab_switch("QMV_MATVEC_MFMA", 1);
  }();
  return v;
}
bool use_mfma() { return mfma_mode() != 0; }
}  // namespace

hipError_t launch_matvec(int fmt, int64_t N, int64_t K, int64_t batch, const uint8_t* W,
                         const void* x, int x_dtype, float* y, hipStream_t s) {
  return launch_matvec_epi(fmt, N, K, batch, W, nullptr, x, x_dtype, y, nullptr, nullptr, s);
}

// With a fused epilogue (W2: SwiGLU; else bias / res, null: none).  Batch 1
// runs on the streaming kernel, 2..8 vectors per pass on the matrix-core
// kernel for its formats (Q8_0, W4A16, Q4K, Q6K) and f32 / f16 activations,
// otherwise on the FMA kernel.
hipError_t launch_matvec_epi(int fmt, int64_t N, int64_t K, int64_t batch, const uint8_t* W, const uint8_t* W2,
                             const void* x, int x_dtype, float* y, const float* bias, const float* res,
                             hipStream_t s) {
  const Planes p = planes_of(fmt, N, K);
  const bool f16 = (x_dtype == QMV_F16);
  const bool q8 = (x_dtype == QMV_Q8X);
  const int64_t xstride = q8 ? q8x_record_bytes(K) : K * (f16 ? 2 : 4);  // bytes per vector
  const bool plain = !W2 && !bias && !res;
  if (batch == 1) {
    hipError_t e = hipSuccess;
    if (plain && mfma_mode() == 2 && launch_matvec_mfma(fmt, N, K, 1, W, x, x_dtype, y, s, &e)) return e;
    if (launch_matvec_b1_epi(fmt, N, K, W, W2, x, x_dtype, y, bias, res, s, &e)) return e;
  }
  for (int64_t b0 = 0; b0 < batch; b0 += 8) {
    const int nb = static_cast<int>(batch - b0 < 8 ? batch - b0 : 8);
    const void* xb = static_cast<const uint8_t*>(x) + b0 * xstride;
    float* yb = y + b0 * N;
    const EpiArgs ea{W2, bias, res ? res + b0 * N : nullptr};
    hipError_t e = hipSuccess;
    if (nb >= 2 && use_mfma() &&
        launch_matvec_mfma_epi(fmt, N, K, nb, W, W2, xb, x_dtype, yb, bias, ea.res, s, &e)) {
      if (e != hipSuccess) return e;
      continue;
    }
    // a last chunk of one vector (batch 9, 17, ...) on the streaming kernel
    if (nb == 1 && launch_matvec_b1_epi(fmt, N, K, W, W2, xb, x_dtype, yb, bias, ea.res, s, &e)) {
      if (e != hipSuccess) return e;
      continue;
    }
    if (q8) {
      switch (fmt) {
        case QMV_Q8_0: e = pick_lpr<QMV_Q8_0, false, true>(W, p, xb, yb, int(N), int(K), nb, ea, s); break;
        case QMV_W4A16_G64: e = pick_lpr<QMV_W4A16_G64, false, true>(W, p, xb, yb, int(N), int(K), nb, ea, s); break;
        case QMV_Q4K: e = pick_lpr<QMV_Q4K, false, true>(W, p, xb, yb, int(N), int(K), nb, ea, s); break;
        case QMV_Q6K: e = pick_lpr<QMV_Q6K, false, true>(W, p, xb, yb, int(N), int(K), nb, ea, s); break;
        case QMV_Q4_0: e = pick_lpr<QMV_Q4_0, false, true>(W, p, xb, yb, int(N), int(K), nb, ea, s); break;
        case QMV_Q5_0: e = pick_lpr<QMV_Q5_0, false, true>(W, p, xb, yb, int(N), int(K), nb, ea, s); break;
        case QMV_Q5K: e = pick_lpr<QMV_Q5K, false, true>(W, p, xb, yb, int(N), int(K), nb, ea, s); break;
        case QMV_I8_ROW: e = pick_lpr<QMV_I8_ROW, false, true>(W, p, xb, yb, int(N), int(K), nb, ea, s); break;
        default: return hipErrorInvalidValue;
      }
      if (e != hipSuccess) return e;
      continue;
    }
    switch (fmt) {
      case QMV_Q8_0: e = pick_lpr<QMV_Q8_0, false>(W, p, xb, yb, int(N), int(K), nb, ea, s); break;
      case QMV_W4A16_G64:
        e = f16 ? pick_lpr<QMV_W4A16_G64, true>(W, p, xb, yb, int(N), int(K), nb, ea, s)
                : pick_lpr<QMV_W4A16_G64, false>(W, p, xb, yb, int(N), int(K), nb, ea, s);
        break;
      case QMV_Q4K: e = pick_lpr<QMV_Q4K, false>(W, p, xb, yb, int(N), int(K), nb, ea, s); break;
      case QMV_Q6K: e = pick_lpr<QMV_Q6K, false>(W, p, xb, yb, int(N), int(K), nb, ea, s); break;
      case QMV_Q4_0: e = pick_lpr<QMV_Q4_0, false>(W, p, xb, yb, int(N), int(K), nb, ea, s); break;
      case QMV_Q5_0: e = pick_lpr<QMV_Q5_0, false>(W, p, xb, yb, int(N), int(K), nb, ea, s); break;
      case QMV_Q5K: e = pick_lpr<QMV_Q5K, false>(W, p, xb, yb, int(N), int(K), nb, ea, s); break;
      case QMV_DENSE_BF16: e = pick_lpr<QMV_DENSE_BF16, false>(W, p, xb, yb, int(N), int(K), nb, ea, s); break;
      case QMV_I8_ROW: e = pick_lpr<QMV_I8_ROW, false>(W, p, xb, yb, int(N), int(K), nb, ea, s); break;
      default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace qmv
